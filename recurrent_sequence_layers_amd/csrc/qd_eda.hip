// Erase-then-Delta (page "Erase-then-Delta Attention" explainer, core method, the
// two-step pseudo-code) for gfx950, in this library's d_v x d_k state convention (the
// page's K x V memory transposed).  Per token, with a unit erase direction e:
//
//   S <- S - (S e) e^T ;   S <- S + (v - S k) k^T ;   o = S q
//
// The erase is itself a delta-rule step with key e, value 0 and beta = 1, so the layer
// is DeltaNet (beta = 1) over the interleaved sequence e_1, k_1, e_2, k_2, ... with zero
// values at the erase tokens, read out at the k tokens.  The chunked forward runs exactly
// that.  In bf16 at C = 32, 64 the eight-wave chunk kernel's EDA instance reads the
// interleaved sequence in place (qd_chunk_fwd_pipe.hip).  The other instances build it:
// an interleave kernel writes the 2T-token sequence into the caller's workspace, the
// chunk forward (its alpha = 1, lambda = 0 instance) runs over it, and a gather kernel
// keeps the outputs of the k tokens.  The decode step is its own kernel: from one read of
// a state row, S e, S k and S q give the erased row's products through e.k and e.q.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 8;

__device__ __forceinline__ float group8_sum(float x) {
    x += __shfl_xor(x, 1, kLanesPerRow);
    x += __shfl_xor(x, 2, kLanesPerRow);
    x += __shfl_xor(x, 4, kLanesPerRow);
    return x;
}

// 16-byte vectors: token-head row r of q, k, e, v to rows 2r, 2r+1 of the interleaved
// arrays (row-major [B][T][H] -> [B][2T][H] with r = (b T + t) H + h), beta2 = 1.
__global__ __launch_bounds__(kThreads) void eda_interleave_kernel(const uint4 *q, const uint4 *k, const uint4 *e,
                                                                   const uint4 *v, uint4 *q2, uint4 *k2, uint4 *v2,
                                                                   float *beta2, int T, int H, int vk, int vv,
                                                                   size_t rows) {
    const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    const size_t nk = rows * vk, nv = rows * vv;
    if (i < nk) {
        const size_t r = i / vk, c = i % vk;
        const size_t bt = r / H, h = r % H, b = bt / T, t = bt % T;
        const size_t r0 = ((b * 2 * T + 2 * t) * H + h), r1 = r0 + H;    // erase token, then the k token
        q2[r0 * vk + c] = q[i];
        q2[r1 * vk + c] = q[i];
        k2[r0 * vk + c] = e[i];
        k2[r1 * vk + c] = k[i];
    }
    if (i < nv) {
        const size_t r = i / vv, c = i % vv;
        const size_t bt = r / H, h = r % H, b = bt / T, t = bt % T;
        const size_t r0 = ((b * 2 * T + 2 * t) * H + h), r1 = r0 + H;
        v2[r0 * vv + c] = make_uint4(0, 0, 0, 0);
        v2[r1 * vv + c] = v[i];
    }
    if (i < 2 * rows) beta2[i] = 1.f;
}

// o row r <- o2 row of its k token
__global__ __launch_bounds__(kThreads) void eda_gather_kernel(const uint4 *o2, uint4 *o, int T, int H, int vv,
                                                               size_t rows) {
    const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= rows * vv) return;
    const size_t r = i / vv, c = i % vv;
    const size_t bt = r / H, h = r % H, b = bt / T, t = bt % T;
    o[i] = o2[((b * 2 * T + 2 * t + 1) * H + h) * vv + c];
}

template <class P, int DK, int DV>
__global__ __launch_bounds__(kThreads) void eda_step_kernel(const EdaStepArgs args) {
    using R = typename P::R;
    constexpr int NG = DK / (4 * kLanesPerRow);
    constexpr int ROWS_PER_PASS = kWave / kLanesPerRow;
    constexpr int ROWS_PER_WAVE = DV / 4;
    constexpr int NPASS = ROWS_PER_WAVE / ROWS_PER_PASS;
    static_assert(NPASS >= 1 && NG >= 1, "unsupported step shape");

    const int nh = blockIdx.x;
    const int lane = lane_id(), wave = wave_id();
    const int sub = lane % kLanesPerRow, grp = lane / kLanesPerRow;
    const R *gq = static_cast<const R *>(args.q) + static_cast<size_t>(nh) * DK;
    const R *gk = static_cast<const R *>(args.k) + static_cast<size_t>(nh) * DK;
    const R *ge = static_cast<const R *>(args.e) + static_cast<size_t>(nh) * DK;
    const R *gv = static_cast<const R *>(args.v) + static_cast<size_t>(nh) * DV;
    R *go = static_cast<R *>(args.o) + static_cast<size_t>(nh) * DV;
    float *S = args.S + static_cast<size_t>(nh) * DV * DK;

    f32x4 s[NPASS][NG];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = wave * ROWS_PER_WAVE + p * ROWS_PER_PASS + grp;
#pragma unroll
        for (int m = 0; m < NG; ++m)
            s[p][m] = *reinterpret_cast<const f32x4 *>(S + static_cast<size_t>(row) * DK + 4 * (m * kLanesPerRow + sub));
    }
    f32x4 kk[NG], qq[NG], ee[NG];
    float ek = 0.f, eq = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NG; ++m) {
        const int c = 4 * (m * kLanesPerRow + sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kk[m][i] = P::to_f32(gk[c + i]);
            qq[m][i] = P::to_f32(gq[c + i]);
            ee[m][i] = P::to_f32(ge[c + i]);
            ek += ee[m][i] * kk[m][i];
            eq += ee[m][i] * qq[m][i];
            kq += kk[m][i] * qq[m][i];
        }
    }
    ek = group8_sum(ek);
    eq = group8_sum(eq);
    kq = group8_sum(kq);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = wave * ROWS_PER_WAVE + p * ROWS_PER_PASS + grp;
        float se = 0.f, sk = 0.f, sq = 0.f;
#pragma unroll
        for (int m = 0; m < NG; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                se += s[p][m][i] * ee[m][i];
                sk += s[p][m][i] * kk[m][i];
                sq += s[p][m][i] * qq[m][i];
            }
        se = group8_sum(se);
        sk = group8_sum(sk);
        sq = group8_sum(sq);
        const float err = P::to_f32(gv[row]) - (sk - se * ek);   // v - (erased S) k
#pragma unroll
        for (int m = 0; m < NG; ++m)
            *reinterpret_cast<f32x4 *>(S + static_cast<size_t>(row) * DK + 4 * (m * kLanesPerRow + sub)) =
                s[p][m] - se * ee[m] + err * kk[m];
        if (sub == 0) go[row] = P::from_f32(sq - se * eq + err * kq);
    }
}

template <class P, int DK, int DV>
hipError_t launch_eda_step_typed(const EdaStepArgs &a, hipStream_t stream) {
    if (a.N * a.H == 0) return hipSuccess;
    hipLaunchKernelGGL((eda_step_kernel<P, DK, DV>), dim3(a.N * a.H), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <class P>
hipError_t launch_eda_step_p(int dk, int dv, const EdaStepArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_eda_step_typed<P, 128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_eda_step_typed<P, 128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_eda_step_typed<P, 64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_eda_step_typed<P, 64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

// bf16 at C = 32, 64 reads the interleaved sequence in place (no workspace); the other
// instances build it in the workspace
static bool eda_in_place(int dtype, int C) { return dtype == 1 && (C == 32 || C == 64); }

size_t eda_chunk_workspace(int dtype, int B, int T, int H, int dk, int dv, int C) {
    if (eda_in_place(dtype, C)) return 0;
    const size_t es = dtype == 1 ? 2 : 4;
    const size_t rows2 = 2 * static_cast<size_t>(B) * T * H;
    // q2, k2 [B][2T][H][d_k]; v2, o2 [B][2T][H][d_v]; beta2 [B][2T][H]
    return rows2 * (2 * dk + 2 * dv) * es + ((rows2 * 4 + 15) / 16) * 16;
}

hipError_t launch_eda_chunk(int dtype, int dk, int C, const EdaChunkArgs &a, void *ws, hipStream_t stream) {
    if (eda_in_place(dtype, C)) {
        ChunkArgs f;
        f.q = a.q; f.k = a.k; f.v = a.v; f.e = a.e;
        f.alpha = nullptr; f.beta = nullptr; f.lam = nullptr;
        f.S0 = a.S0; f.o = a.o; f.S_T = a.S_T;
        f.B = a.B; f.T = a.T; f.H = a.H; f.dv = a.dv; f.n_dvt = a.dv / 64;
        return launch_chunk_fwd_pipe_eda(dk, C, f, stream);
    }
    const size_t es = dtype == 1 ? 2 : 4;
    const size_t rows = static_cast<size_t>(a.B) * a.T * a.H, rows2 = 2 * rows;
    unsigned char *p = static_cast<unsigned char *>(ws);
    void *q2 = p;
    void *k2 = p + rows2 * dk * es;
    void *v2 = p + 2 * rows2 * dk * es;
    void *o2 = p + (2 * dk + a.dv) * rows2 * es;
    float *beta2 = reinterpret_cast<float *>(p + (2 * dk + 2 * a.dv) * rows2 * es);
    const int vk = static_cast<int>(dk * es / 16), vv = static_cast<int>(a.dv * es / 16);
    if (rows > 0) {
        const size_t n = rows * (vk > vv ? vk : vv) > 2 * rows ? rows * (vk > vv ? vk : vv) : 2 * rows;
        hipLaunchKernelGGL(eda_interleave_kernel, dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, static_cast<const uint4 *>(a.q), static_cast<const uint4 *>(a.k),
                           static_cast<const uint4 *>(a.e), static_cast<const uint4 *>(a.v), static_cast<uint4 *>(q2),
                           static_cast<uint4 *>(k2), static_cast<uint4 *>(v2), beta2, a.T, a.H, vk, vv, rows);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    ChunkArgs f;
    f.q = q2; f.k = k2; f.v = v2;
    f.alpha = nullptr; f.beta = beta2; f.lam = nullptr;
    f.S0 = a.S0; f.o = o2; f.S_T = a.S_T;
    f.B = a.B; f.T = 2 * a.T; f.H = a.H; f.dv = a.dv; f.n_dvt = a.dv / 64;
    hipError_t err = launch_chunk_fwd(dtype, dk, C, f, stream);
    if (err != hipSuccess || rows == 0) return err;
    hipLaunchKernelGGL(eda_gather_kernel, dim3(static_cast<unsigned>((rows * vv + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, static_cast<const uint4 *>(o2), static_cast<uint4 *>(a.o), a.T,
                       a.H, vv, rows);
    return hipGetLastError();
}

hipError_t launch_eda_step(int dtype, int dk, int dv, const EdaStepArgs &a, hipStream_t stream) {
    return dtype == 1 ? launch_eda_step_p<Bf16>(dk, dv, a, stream) : launch_eda_step_p<F32>(dk, dv, a, stream);
}

}  // namespace qd
