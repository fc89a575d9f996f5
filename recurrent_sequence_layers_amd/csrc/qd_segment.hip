// Segmented schedule of the chunk forward for long sequences over few heads.
//
// The recurrence acts on the state from the right (Q-Delta reading notes §2.4):
//   S_t = S_{t-1} A_t + beta_t v_t k_t^T,   A_t = alpha_t (I - beta_t x_t k_t^T),
// so over a run of tokens the exit state is affine in the entry state:
//   S_out = S_in M + G,   M = A_1 ... A_n,   G = S_out when S_in = 0.
// M itself is the exit state of the same recurrence started from S_in = I with v = 0,
// and G is the exit state started from 0 with the real v.  Both therefore come from
// the ordinary chunk kernel, run over the sequence cut into P segments that are laid
// side by side as P batch entries ([B][T][H][d] is [B*P][T/P][H][d] in memory):
//
//   1. M_p: chunk kernel on every segment, v = 0, S0 = I (d_k x d_k), no output;
//   2. G_p: chunk kernel on every segment, real v, S0 = 0, no output;
//   3. S_in[0] = S0, S_in[p+1] = S_in[p] M_p + G_p (fp32, below); S_T = S_in[P-1] M + G;
//   4. the chunk kernel on every segment from its S_in, writing o.
//
// Each pass has P times the parallelism of the single-pass schedule, for three passes
// of work.  It pays when the single pass leaves most compute units idle.
//
// For a single sequence (B = 1), the first segment's entry state is
// the caller's S0, so that segment needs neither map: it is walked once, with its output,
// in the same launch as steps 1 and 2 over the other P - 1 segments, on compute units of
// its own.  Its exit state starts step 3, and step 4 covers the other segments.  It is
// made longer than the others so that its walk ends with their two state-only walks.
#include "qd_device.h"
#include "qd_internal.h"

#include <atomic>

namespace qd {
namespace {

// M[s][i][j] = (i == j) for every segment-head s
__global__ __launch_bounds__(256) void identity_fill_kernel(float *M, int dk, size_t n) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const int e = static_cast<int>(i % (static_cast<size_t>(dk) * dk));
    M[i] = (e / dk == e % dk) ? 1.f : 0.f;
}

// Entry states of the segments and the exit state of the sequence, for rows
// [R * blockIdx.y, R * blockIdx.y + R) of S for (batch, head) blockIdx.x:
//   S <- S0 (or 0); for p: S_in[b P + p] = S; S <- S M[b P + p] + G[b P + p];  S_T = S.
// The whole of M[b P + p] sits in LDS for step p while the next segment's map is already
// on its way into registers, so each step waits on one barrier, not on a global load;
// each thread owns DK / 32 columns of one row and sums over the rows of M in order.
template <int DK>
__global__ __launch_bounds__(256) void segment_propagate_kernel(const float *S0, const float *M, const float *G,
                                                                float *Sin, float *S_T, int P, int H, int dv) {
    constexpr int R = 8, CPT = DK / 32, NV = DK * DK / 4 / 256;
    __shared__ __attribute__((aligned(16))) float Ss[R][DK];
    __shared__ __attribute__((aligned(16))) float Ms[DK][DK];
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int r0 = R * blockIdx.y;
    const int t = threadIdx.x, row = t / 32, c0 = (t % 32) * CPT;
    const size_t off0 = ((static_cast<size_t>(bh)) * dv + r0 + row) * DK + c0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) Ss[row][c0 + c] = S0 ? S0[off0 + c] : 0.f;
    auto seg = [&](int p) { return static_cast<size_t>(b * P + p) * H + h; };
    f32x4 mv[NV];                                  // the next map, in flight
    auto load_map = [&](int p) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(M + seg(p) * DK * DK);
#pragma unroll
        for (int j = 0; j < NV; ++j) mv[j] = src[t + 256 * j];
    };
    load_map(0);
    for (int p = 0; p < P; ++p) {
        const size_t off = (seg(p) * dv + r0 + row) * DK + c0;
        float acc[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = G[off + c];
        __syncthreads();                           // S of this step written; the previous map consumed
#pragma unroll
        for (int j = 0; j < NV; ++j) reinterpret_cast<f32x4 *>(&Ms[0][0])[t + 256 * j] = mv[j];
        if (p + 1 < P) load_map(p + 1);
#pragma unroll
        for (int c = 0; c < CPT; ++c) Sin[off + c] = Ss[row][c0 + c];
        __syncthreads();
#pragma unroll 8
        for (int i = 0; i < DK; ++i) {
            const float sv = Ss[row][i];
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[c] += sv * Ms[i][c0 + c];
        }
        __syncthreads();                           // every thread has read S
#pragma unroll
        for (int c = 0; c < CPT; ++c) Ss[row][c0 + c] = acc[c];
    }
    __syncthreads();
    if (S_T) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) S_T[off0 + c] = Ss[row][c0 + c];
    }
}

}  // namespace

int device_cu_count() {
    // the library's one host-side cache: the compute-unit count of each device, read
    // once per device (an attribute that cannot change while the process runs)
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int n = cached[dev].load(std::memory_order_relaxed);
        if (n > 0) return n;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) return 0;
    if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

int chunk_fwd_segments(int dtype, int B, int T, int H, int dk, int dv, int C) {
    // the state-only passes use the bf16 eight-wave kernel (null v and o)
    if (dtype != 1 || (C != 32 && C != 64) || B <= 0 || H <= 0 || T <= 0) return 1;
    const long long units = static_cast<long long>(B) * H * (dv > dk ? dv : dk) / 64;
    const int cus = device_cu_count();
    int P = 1;
    while (P < 16 && units * 2 * P <= cus && T % (2 * P * C) == 0 && T / (2 * P * C) >= 8) P *= 2;
    return P;
}

size_t chunk_fwd_segment_workspace(int B, int T, int H, int dk, int dv, int P) {
    (void)T;
    if (P <= 1) return 0;
    const size_t nseg = static_cast<size_t>(B) * P * H;
    return nseg * (static_cast<size_t>(dk) * dk + 2 * static_cast<size_t>(dv) * dk) * sizeof(float);
}

// The single-sequence schedule: the first segment (L0 chunks) walked with its output beside
// the maps of the other P - 1 segments (L chunks each), then the propagation from its exit
// state and the other segments' outputs.  Workspace: Mseg, Gseg and Sin of the P - 1
// segments and the first segment's exit state, within chunk_fwd_segment_workspace(P).
static hipError_t launch_segmented_overlapped(int dk, int C, const ChunkArgs &a, int P, void *ws,
                                              hipStream_t stream) {
    const int H = a.H, dv = a.dv, Q = P - 1;
    const int NC = a.T / C;
    const int u0 = H * a.n_dvt;                         // workgroups of one output walk over a segment
    const int um = H * (dk / 64);                       // ... of one transition-map walk
    const int cus = device_cu_count();
    const int spare = cus - u0 > 0 ? cus - u0 : 1;
    // rounds of the state-only walks on the units the first segment leaves free; a chunk
    // step of the state-only instance takes about 7/8 of an output step (raw inputs walk
    // the output instance throughout)
    const int rounds = (Q * (um + u0) + spare - 1) / spare;
    const double ratio = a.raw ? 1.0 : 0.875;
    int L = static_cast<int>(NC / (Q + ratio * rounds) + 0.5);
    if (L > (NC - 1) / Q) L = (NC - 1) / Q;
    if (L < 1) L = 1;
    const int L0 = NC - Q * L;
    const size_t nseg = static_cast<size_t>(Q) * H;
    float *const Mseg = static_cast<float *>(ws);                       // [Q][H][d_k][d_k]
    float *const Gseg = Mseg + nseg * dk * dk;                          // [Q][H][d_v][d_k]
    float *const Sin = Gseg + nseg * dv * dk;                           // [Q][H][d_v][d_k]
    float *const S1 = Sin + nseg * dv * dk;                             // [H][d_v][d_k]
    const size_t nM = nseg * dk * dk;
    hipLaunchKernelGGL(identity_fill_kernel, dim3(static_cast<unsigned>((nM + 255) / 256)), dim3(256), 0, stream,
                       Mseg, dk, nM);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    // the first segment: its own entry state, its output, its exit state into S1
    ChunkArgs a0 = a;
    a0.T = L0 * C;
    a0.S_T = S1;
    // the other segments as Q batch entries of L C tokens, from token L0 C on
    const size_t tok = static_cast<size_t>(L0) * C * H;
    ChunkArgs seg = a;
    seg.B = Q;
    seg.T = L * C;
    seg.q = static_cast<const uint16_t *>(a.q) + tok * dk;
    seg.k = static_cast<const uint16_t *>(a.k) + tok * dk;
    seg.v = static_cast<const uint16_t *>(a.v) + tok * dv;
    seg.alpha = a.alpha ? a.alpha + tok : nullptr;
    seg.beta = a.beta + tok;
    seg.lam = a.lam ? a.lam + tok : nullptr;
    seg.o = a.o ? static_cast<uint16_t *>(a.o) + tok * dv : nullptr;
    ChunkArgs m = seg;                                  // 1. maps: v = 0, S0 = I, no output
    m.v = nullptr; m.o = nullptr; m.S0 = Mseg; m.S_T = Mseg; m.dv = dk; m.n_dvt = dk / 64;
    ChunkArgs g = seg;                                  // 2. exit states from zero, no output
    g.o = nullptr; g.S0 = nullptr; g.S_T = Gseg;
    if ((err = launch_chunk_fwd_pipe_overlap(dk, C, a0, m, g, stream)) != hipSuccess) return err;
    // 3. entry states of the other segments from the first one's exit state
    const dim3 pg(static_cast<unsigned>(H), static_cast<unsigned>(dv / 8));
    if (dk == 128)
        hipLaunchKernelGGL((segment_propagate_kernel<128>), pg, dim3(256), 0, stream, S1, Mseg, Gseg, Sin, a.S_T, Q, H, dv);
    else
        hipLaunchKernelGGL((segment_propagate_kernel<64>), pg, dim3(256), 0, stream, S1, Mseg, Gseg, Sin, a.S_T, Q, H, dv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // 4. the other segments' outputs
    ChunkArgs f = seg;
    f.S0 = Sin; f.S_T = nullptr;
    return launch_chunk_fwd(1, dk, C, f, stream);
}

hipError_t launch_chunk_fwd_segmented(int dtype, int dk, int C, const ChunkArgs &a, int P, void *ws,
                                      hipStream_t stream) {
    if (a.B == 1 && dtype == 1 && a.o != nullptr && a.v != nullptr && a.T % C == 0 && a.T / C >= 2 * P)
        return launch_segmented_overlapped(dk, C, a, P, ws, stream);
    const size_t nseg = static_cast<size_t>(a.B) * P * a.H;
    float *const Mseg = static_cast<float *>(ws);                       // [B P][H][d_k][d_k]
    float *const Gseg = Mseg + nseg * dk * dk;                          // [B P][H][d_v][d_k]
    float *const Sin = Gseg + nseg * a.dv * dk;                         // [B P][H][d_v][d_k]
    const size_t nM = nseg * dk * dk;
    hipLaunchKernelGGL(identity_fill_kernel, dim3(static_cast<unsigned>((nM + 255) / 256)), dim3(256), 0, stream,
                       Mseg, dk, nM);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    ChunkArgs seg = a;
    seg.B = a.B * P;
    seg.T = a.T / P;
    // 1. transition maps: v = 0, S0 = I, state updated in place, no output
    ChunkArgs m = seg;
    m.v = nullptr; m.o = nullptr; m.S0 = Mseg; m.S_T = Mseg; m.dv = dk; m.n_dvt = dk / 64;
    if ((err = launch_chunk_fwd(dtype, dk, C, m, stream)) != hipSuccess) return err;
    // 2. exit states from zero entry states, no output
    ChunkArgs g = seg;
    g.o = nullptr; g.S0 = nullptr; g.S_T = Gseg;
    if ((err = launch_chunk_fwd(dtype, dk, C, g, stream)) != hipSuccess) return err;
    // 3. entry states of the segments and the exit state of the sequence
    const dim3 pg(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>(a.dv / 8));
    if (dk == 128)
        hipLaunchKernelGGL((segment_propagate_kernel<128>), pg, dim3(256), 0, stream, a.S0, Mseg, Gseg, Sin, a.S_T, P,
                           a.H, a.dv);
    else
        hipLaunchKernelGGL((segment_propagate_kernel<64>), pg, dim3(256), 0, stream, a.S0, Mseg, Gseg, Sin, a.S_T, P,
                           a.H, a.dv);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // 4. the outputs, every segment from its entry state
    ChunkArgs f = seg;
    f.S0 = Sin; f.S_T = nullptr;
    return launch_chunk_fwd(dtype, dk, C, f, stream);
}

}  // namespace qd
