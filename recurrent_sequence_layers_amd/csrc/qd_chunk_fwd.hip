// Fused chunkwise Q-Delta layer forward for gfx950.
//
// One workgroup owns one (batch, head, 64-wide value-column tile) and walks the
// sequence chunk by chunk, keeping its slice of the state S^T (d_k x 64, fp32) in
// MFMA accumulator registers for the whole sequence.  Every chunk is read from HBM
// once (q, k, the v tile, the gates) and its output tile is written once; all
// chunk intermediates live in LDS.  Per chunk (Q-Delta reading notes §2.6, the
// chunkwise WY/UT form with entry state):
//
//   g     = cumsum(log alpha)                       (log-space decays, all factors <= 1)
//   QK^T, KK^T on MFMA;  X K^T = K K^T + diag(lambda) Q K^T
//   L     = strictly-lower(diag(beta) X K^T)
//   T     = (I + L)^-1      16x16 diagonal blocks by forward substitution, then
//                           block doubling on MFMA (UT transform, notes Eq. 27)
//   M1    = (H o T) diag(beta),   M2 = -D_g T diag(beta),   A = H o (Q K^T)
//   U~    = M1 V                                    ((I + L_g)^-1 B V, using
//                                                   (I + L_g)^-1 = H o (I + L)^-1)
//   Z     = U~ + M2 (K S^T + diag(lambda) Q S^T)    (= U~ - D_g W S^T)
//   O     = D_g Q S^T + A Z
//   S^T  <- exp(g_last) S^T + K^T diag(exp(g_last - g)) Z
//
// Waves: four per workgroup; in the state-dependent part wave w owns value columns
// [16w, 16w + 16) of the tile, so S^T, K S^T, Q S^T, Z and O for those columns stay
// in its registers and feed one another as MFMA operands without LDS round trips.
// Every LDS matrix is row-major; operands needed transposed (K^T, V, blocks of T)
// are read with the gfx950 LDS transpose read.  The next chunk's raw inputs are
// loaded into registers while the current chunk computes (addresses are clamped to
// the last valid row, so the loads carry no branches; rows past the end are zeroed
// when they are written to LDS).  A short last chunk is padded with alpha = 1,
// beta = 0, q = k = v = 0, which leaves the state and the valid outputs unchanged.
#include "qd_chunk_common.h"
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kDVT = 64;  // value columns per workgroup

template <class P, int DK, int CH>
struct ChunkLayout {
    using R = typename P::R;
    static constexpr int PAD = 16 / P::kBytes;   // 16 bytes of row padding
    static constexpr int PK = DK + PAD;          // pitch of Q, K rows (d_k wide)
    static constexpr int PC = CH + PAD;          // pitch of chunk-wide rows
    static constexpr int PV = kDVT + PAD;        // pitch of V rows and of the output staging
    static constexpr int NQ = CH * PK;
    static constexpr int NV = CH * PV;
    static constexpr int NCC = CH * PC;
    static constexpr int NT = (CH * PV > NCC) ? CH * PV : NCC;  // T buffer doubles as O staging
    // element offsets (16-byte aligned: every row pitch is a multiple of 16 bytes)
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + NQ;
    static constexpr int oV = oK + NQ;
    static constexpr int oL = oV + NV;      // L, later M1
    static constexpr int oM2 = oL + NCC;
    static constexpr int oT = oM2 + NCC;    // T, later O staging
    static constexpr int oA = oT + NT;      // A = H o QK^T
    static constexpr int nR = oA + NCC;
    static constexpr int gate_bytes = 5 * CH * 4;
    static constexpr int bytes = nR * P::kBytes + gate_bytes;
    static_assert((PK * P::kBytes) % 16 == 0 && (PC * P::kBytes) % 16 == 0 && (PV * P::kBytes) % 16 == 0,
                  "row pitches must keep 16-byte alignment");
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
};

template <class P, int DK, int CH, bool HAS_A, bool HAS_L>
__global__ __launch_bounds__(kThreads, 1) void chunk_fwd_kernel(const ChunkArgs args) {
    using R = typename P::R;
    using F = typename P::F;
    using Lay = ChunkLayout<P, DK, CH>;
    constexpr int NKT = DK / 16;       // 16-wide key tiles
    constexpr int NCT = CH / 16;       // 16-row chunk tiles
    constexpr int PK = Lay::PK, PC = Lay::PC, PV = Lay::PV;
    constexpr int EPV = 16 / P::kBytes;            // elements per 16-byte vector
    constexpr int VPRQ = DK / EPV;                 // vectors per q/k row
    constexpr int VPRV = kDVT / EPV;               // vectors per v/o tile row
    constexpr int NVQ = (CH * VPRQ + kThreads - 1) / kThreads;
    constexpr int NVV = (CH * VPRV + kThreads - 1) / kThreads;
    constexpr int NPAIR = NCT * (NCT + 1) / 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::bytes];
    R *const Qs = reinterpret_cast<R *>(smem) + Lay::oQ;
    R *const Ks = reinterpret_cast<R *>(smem) + Lay::oK;
    R *const Vs = reinterpret_cast<R *>(smem) + Lay::oV;
    R *const Ls = reinterpret_cast<R *>(smem) + Lay::oL;
    R *const M2s = reinterpret_cast<R *>(smem) + Lay::oM2;
    R *const Ts = reinterpret_cast<R *>(smem) + Lay::oT;
    R *const As = reinterpret_cast<R *>(smem) + Lay::oA;
    R *const M1s = Ls;
    R *const Os = Ts;
    float *const gs = reinterpret_cast<float *>(smem + Lay::nR * P::kBytes);  // g = cumsum log alpha
    float *const egs = gs + CH;      // exp(g)
    float *const egls = egs + CH;    // exp(g_last - g)
    float *const bes = egls + CH;    // beta
    float *const lams = bes + CH;    // lambda

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = wave_id();
    const int r16 = lane & 15;
    const int g4 = lane >> 4;

    // ---- workgroup -> (b, h, value tile); the value tiles of one head share an XCD
    const int nblk = gridDim.x;
    int logical = blockIdx.x;
    if (args.n_dvt > 1 && (nblk & 7) == 0) logical = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int dvt = logical % args.n_dvt;
    const int bh = logical / args.n_dvt;
    const int b = bh / args.H;
    const int h = bh % args.H;
    const int T = args.T, H = args.H, dv = args.dv;
    const int dv0 = dvt * kDVT;

    const R *__restrict__ gq = static_cast<const R *>(args.q);
    const R *__restrict__ gk = static_cast<const R *>(args.k);
    const R *__restrict__ gv = static_cast<const R *>(args.v);
    R *__restrict__ go = static_cast<R *>(args.o);
    auto tok = [&](int t) -> size_t { return (static_cast<size_t>(b) * T + t) * H + h; };

    // ---- state slice: S^T tiles, rows d_k = 16t + 4g + i, column = this wave's value column
    f32x4 sT[NKT];
    const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * wave + r16) * DK;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
        sT[t] = args.S0 ? *reinterpret_cast<const f32x4 *>(args.S0 + srow + 16 * t + 4 * g4) : zero4();

    // ---- raw chunk staging registers (prefetched one chunk ahead, branch-free)
    uint4 rq[NVQ], rk[NVQ], rv[NVV];
    float ra = 1.f, rb = 0.f, rl = 0.f;
    auto gload = [&](int n) {
        const int t0 = n * CH;
        const int last = min(CH, T - t0) - 1;   // >= 0 for every chunk that exists
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = tid + kThreads * j;
            if (CH * VPRQ % kThreads == 0 || vi < CH * VPRQ) {
                const int c = min(vi / VPRQ, last), cv = vi % VPRQ;
                const size_t off = tok(t0 + c) * DK + cv * EPV;
                rq[j] = *reinterpret_cast<const uint4 *>(gq + off);
                rk[j] = *reinterpret_cast<const uint4 *>(gk + off);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = tid + kThreads * j;
            if (CH * VPRV % kThreads == 0 || vi < CH * VPRV) {
                const int c = min(vi / VPRV, last), cv = vi % VPRV;
                rv[j] = *reinterpret_cast<const uint4 *>(gv + tok(t0 + c) * dv + dv0 + cv * EPV);
            }
        }
        {   // every thread loads (clamped) so the loads carry no branch
            const size_t gi = tok(t0 + min(tid & (kWave - 1), last));
            if constexpr (HAS_A) ra = args.alpha[gi];
            rb = args.beta[gi];
            if constexpr (HAS_L) rl = args.lam[gi];
        }
    };
    auto lstore = [&](int clen) {
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = tid + kThreads * j;
            if (CH * VPRQ % kThreads == 0 || vi < CH * VPRQ) {
                const int c = vi / VPRQ, cv = vi % VPRQ;
                *reinterpret_cast<uint4 *>(Qs + c * PK + cv * EPV) = keep_if(c < clen, rq[j]);
                *reinterpret_cast<uint4 *>(Ks + c * PK + cv * EPV) = keep_if(c < clen, rk[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = tid + kThreads * j;
            if (CH * VPRV % kThreads == 0 || vi < CH * VPRV) {
                const int c = vi / VPRV, cv = vi % VPRV;
                *reinterpret_cast<uint4 *>(Vs + c * PV + cv * EPV) = keep_if(c < clen, rv[j]);
            }
        }
        if (wave == 0) {
            // inclusive prefix sum of log(alpha) over the chunk (padding rows add 0)
            const bool ok = lane < clen;
            float x = (HAS_A && ok) ? __logf(ra) : 0.f;
            x = wave_inclusive_sum(x);
            const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), CH - 1));
            if (lane < CH) {
                gs[lane] = x;
                egs[lane] = __expf(x);
                egls[lane] = __expf(glast - x);
                bes[lane] = ok ? rb : 0.f;
                lams[lane] = ok ? rl : 0.f;
            }
        }
    };

    const int NC = (T + CH - 1) / CH;
    if (NC > 0) gload(0);
    // The state and the first chunk's loads complete before the loop.  Otherwise the first
    // use of the state inside the loop is guarded, conservatively, by a wait for every
    // outstanding load, including the next chunk's prefetch.
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)

    for (int n = 0; n < NC; ++n) {
        const int t0 = n * CH;
        const int clen = min(CH, T - t0);
        if (args.Hs) {   // entry state of chunk n, [B][H][NC][d_v][d_k] (kept for the backward)
            R *hs = static_cast<R *>(args.Hs) + (static_cast<size_t>(bh) * NC + n) * dv * DK +
                    static_cast<size_t>(dv0 + 16 * wave + r16) * DK + 4 * g4;
#pragma unroll
            for (int t = 0; t < NKT; ++t) P::st4(hs + 16 * t, sT[t]);
        }
        lstore(clen);
        if (n + 1 < NC) gload(n + 1);
        __syncthreads();

        // ---- Gram blocks: L = sl(diag(beta) X K^T), A = H o Q K^T; then T = (I + L)^-1
        gram_blocks<P, DK, CH, PK, PC, HAS_A, HAS_L>(Qs, Ks, gs, bes, lams, Ls, As, nullptr);
        __syncthreads();
        unit_lower_inverse<P, CH, PC>(Ls, Ts);

        // ---- M1 = (H o T) diag(beta), M2 = -D_g T diag(beta), four columns per lane,
        // lower block triangle only (the other blocks are never read)
        for (int idx = tid; idx < NPAIR * 64; idx += kThreads) {
            int i, j;
            tri_pair(idx >> 6, i, j);
            const int r = 16 * i + ((idx >> 2) & 15);
            const int c0 = 16 * j + 4 * (idx & 3);
            const F tf = P::ld4(Ts + r * PC + c0);
            const f32x4 bc = lds_f32x4(bes + c0);
            const f32x4 gc = lds_f32x4(gs + c0);
            const float gr = gs[r], er = egs[r];
            f32x4 m1, m2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float tb = (c0 + e <= r) ? static_cast<float>(tf[e]) * bc[e] : 0.f;
                m1[e] = HAS_A ? __expf(gr - gc[e]) * tb : tb;
                m2[e] = HAS_A ? -er * tb : -tb;
            }
            P::st4(M1s + r * PC + c0, m1);
            P::st4(M2s + r * PC + c0, m2);
        }
        __syncthreads();

        // ---- state-dependent part: this wave's 16 value columns
        // U~ = M1 V  (initial value of Z)
        f32x4 Z[NCT];
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            Z[mt] = zero4();
#pragma unroll
            for (int s = 0; s <= mt; s += 2) {
                if (s + 1 <= mt)
                    Z[mt] = P::mma2(Z[mt], frag<P>(M1s, PC, 16 * mt, 16 * s), frag<P>(M1s, PC, 16 * mt, 16 * s + 16),
                                    frag_b<P>(Vs, PV, 16 * s, 16 * wave), frag_b<P>(Vs, PV, 16 * s + 16, 16 * wave));
                else
                    Z[mt] = P::mma1(Z[mt], frag<P>(M1s, PC, 16 * mt, 16 * s), frag_b<P>(Vs, PV, 16 * s, 16 * wave));
            }
        }
        // K S^T and Q S^T
        F sTf[NKT];
#pragma unroll
        for (int t = 0; t < NKT; ++t) sTf[t] = P::cvt(sT[t]);
        f32x4 PKs[NCT], PQs[NCT];
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            PKs[mt] = zero4();
            PQs[mt] = zero4();
#pragma unroll
            for (int t = 0; t < NKT; t += 2) {
                PKs[mt] = P::mma2(PKs[mt], frag<P>(Ks, PK, 16 * mt, 16 * t), frag<P>(Ks, PK, 16 * mt, 16 * t + 16),
                                  sTf[t], sTf[t + 1]);
                PQs[mt] = P::mma2(PQs[mt], frag<P>(Qs, PK, 16 * mt, 16 * t), frag<P>(Qs, PK, 16 * mt, 16 * t + 16),
                                  sTf[t], sTf[t + 1]);
            }
        }
        // Z = U~ + M2 (K S^T + diag(lambda) Q S^T)
        F Yf[NCT];
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            f32x4 y = PKs[mt];
            if constexpr (HAS_L) y += lds_f32x4(lams + 16 * mt + 4 * g4) * PQs[mt];
            Yf[mt] = P::cvt(y);
        }
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
#pragma unroll
            for (int s = 0; s <= mt; s += 2) {
                if (s + 1 <= mt)
                    Z[mt] = P::mma2(Z[mt], frag<P>(M2s, PC, 16 * mt, 16 * s), frag<P>(M2s, PC, 16 * mt, 16 * s + 16),
                                    Yf[s], Yf[s + 1]);
                else
                    Z[mt] = P::mma1(Z[mt], frag<P>(M2s, PC, 16 * mt, 16 * s), Yf[s]);
            }
        }
        // O = D_g Q S^T + A Z
        F Zf[NCT], Zd[NCT];
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            Zf[mt] = P::cvt(Z[mt]);
            Zd[mt] = HAS_A ? P::cvt(lds_f32x4(egls + 16 * mt + 4 * g4) * Z[mt]) : Zf[mt];
        }
        f32x4 O[NCT];
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            O[mt] = HAS_A ? lds_f32x4(egs + 16 * mt + 4 * g4) * PQs[mt] : PQs[mt];
#pragma unroll
            for (int s = 0; s <= mt; s += 2) {
                if (s + 1 <= mt)
                    O[mt] = P::mma2(O[mt], frag<P>(As, PC, 16 * mt, 16 * s), frag<P>(As, PC, 16 * mt, 16 * s + 16),
                                    Zf[s], Zf[s + 1]);
                else
                    O[mt] = P::mma1(O[mt], frag<P>(As, PC, 16 * mt, 16 * s), Zf[s]);
            }
        }
        // S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) Z ; K^T blocks via transpose reads of K
        const float dlast = HAS_A ? egs[CH - 1] : 1.f;
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            f32x4 acc = sT[t] * dlast;
#pragma unroll
            for (int s = 0; s < NCT; s += 2) {
                if (s + 1 < NCT)
                    acc = P::mma2(acc, frag_b<P>(Ks, PK, 16 * s, 16 * t), frag_b<P>(Ks, PK, 16 * s + 16, 16 * t),
                                  Zd[s], Zd[s + 1]);
                else
                    acc = P::mma1(acc, frag_b<P>(Ks, PK, 16 * s, 16 * t), Zd[s]);
            }
            sT[t] = acc;
        }
        if (!go) {   // state-only pass: no output; the barrier keeps the next chunk's LDS writes
            __syncthreads();   // behind every wave's reads of this chunk's K
            continue;
        }
        // stage O (the T buffer is dead after the M build), then coalesced row stores
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Os[(16 * mt + 4 * g4 + e) * PV + 16 * wave + r16] = P::from_f32(O[mt][e]);
        }
        __syncthreads();
        for (int vi = tid; vi < CH * VPRV; vi += kThreads) {
            const int c = vi / VPRV, cv = vi % VPRV;
            if (c < clen)
                *reinterpret_cast<uint4 *>(go + tok(t0 + c) * dv + dv0 + cv * EPV) =
                    *reinterpret_cast<const uint4 *>(Os + c * PV + cv * EPV);
        }
        // the next iteration's LDS writes (Q, K, V, gates) do not touch the O staging
        // buffer, and the T writes that reuse it are two barriers away.
    }

    if (args.S_T) {
#pragma unroll
        for (int t = 0; t < NKT; ++t) *reinterpret_cast<f32x4 *>(args.S_T + srow + 16 * t + 4 * g4) = sT[t];
    }
}

template <class P, int DK, int CH>
hipError_t launch_typed(const ChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    if (ha && hl) hipLaunchKernelGGL((chunk_fwd_kernel<P, DK, CH, true, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else if (ha) hipLaunchKernelGGL((chunk_fwd_kernel<P, DK, CH, true, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    else if (hl) hipLaunchKernelGGL((chunk_fwd_kernel<P, DK, CH, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((chunk_fwd_kernel<P, DK, CH, false, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <class P, int DK>
hipError_t launch_dk(int C, const ChunkArgs &a, hipStream_t stream) {
    switch (C) {
        case 16: return launch_typed<P, DK, 16>(a, stream);
        case 32: return launch_typed<P, DK, 32>(a, stream);
        case 64: return launch_typed<P, DK, 64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunk_fwd_supported(int dtype, int dk, int dv, int C) {
    return (dtype == 0 || dtype == 1) && (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
           (C == 16 || C == 32 || C == 64);
}

hipError_t launch_chunk_fwd_states(int dtype, int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    if (dtype == 1) {
        if (C != 16) return launch_chunk_fwd_pipe_states(dk, C, a, stream);
        return dk == 128 ? launch_typed<Bf16, 128, 16>(a, stream) : launch_typed<Bf16, 64, 16>(a, stream);
    }
    return dk == 128 ? launch_dk<F32, 128>(C, a, stream) : launch_dk<F32, 64>(C, a, stream);
}

hipError_t launch_chunk_fwd(int dtype, int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    if (dtype == 1) {
        // C = 32, 64: the pipelined kernel; C = 16 is too short to pair chunk positions
        if (C != 16) return launch_chunk_fwd_pipe(dk, C, a, stream);
        return dk == 128 ? launch_typed<Bf16, 128, 16>(a, stream) : launch_typed<Bf16, 64, 16>(a, stream);
    }
    return dk == 128 ? launch_dk<F32, 128>(C, a, stream) : launch_dk<F32, 64>(C, a, stream);
}

}  // namespace qd
