// QED / GDN-2 layer for gfx950: per-key-channel decay, vector erase and write gates and
// the query-derived erase direction (page "The Query Knows What to Forget" reading notes,
// §2.1 and §2.2, the boxed update), in the d_v x d_k state convention of this library
// (the notes' K x V state transposed, so their S^T x is S x here):
//
//   S_bar = S_{t-1} Diag(exp g_t)
//   a_t   = b_t . k_t + lambda_h (u_t - k_t (k_t . u_t)),   u_t = b_t . q_t
//   r_t   = w_t . v_t - S_bar a_t
//   S_t   = S_bar + r_t k_t^T,       o_t = S_t q_t
//
// lambda_h = 0 is GDN-2.  Two kernels:
//
// qed_step_kernel: one token for N sequences x H heads, the decode form.  Eight lanes
//   share a state row as in the Q-Delta step kernel; the row's exp(g), a, q and k are
//   formed once per lane for its columns (k . u reduced over the eight lanes).
//
// qed_chunk_kernel: the chunked forward.  Within a chunk, with the per-channel cumulative
//   log decay Gm_t = sum_{s<=t} g_s (the recurrence unrolled; derived here, the notes give
//   only the step):
//     (I + L) R = W.V - At S^T,          At_t = a_t . exp(Gm_t)
//     O = Qt S^T + M R,                  Qt_t = q_t . exp(Gm_t)
//     S'^T = diag(exp Gm_C) S^T + Kh^T R,  Kh_j = k_j . exp(Gm_C - Gm_j)
//   with L[t,j] = sum_c a_t[c] k_j[c] exp(Gm_t[c] - Gm_j[c]) (j < t) and M the same with
//   q (j <= t).  L and M are built from 16 x 16 blocks as products of row operands
//   x_t . exp(Gm_t - Gm_r) and column operands k_j . exp(Gm_r - Gm_j): for a block below
//   the diagonal r is the first token of the row block (every factor <= 1); for a
//   diagonal block r is its ninth token, so a factor exceeds 1 by at most eight tokens of
//   decay.  That is the kernel's domain: exp(-(g_s + ... + g_{s+7})) must stay within the
//   fp32 range (per-token log decays above about -11).  T = (I + L)^-1: the diagonal
//   16 x 16 blocks inverted in registers, then the shared block doubling.  The state-
//   dependent part runs on waves 0-3, one wave per 16 value columns holding S^T in MFMA
//   accumulators, one chunk behind the state-independent part (a two-stage pipeline: the
//   decayed operands, w . v and exp(Gm_C) are double-buffered in LDS).
#include "qd_chunk_common.h"
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkThreads = 512;   // chunk kernel: eight waves, four of them on the state
constexpr int kLanesPerRow = 8;
constexpr int kDVT = 64;

constexpr float kLog2e = 1.4426950408889634f;
// 2^x on the transcendental unit (results below the normal range flush to zero, as the
// natural-base form does)
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float group8_sum(float x) {
    x += __shfl_xor(x, 1, kLanesPerRow);
    x += __shfl_xor(x, 2, kLanesPerRow);
    x += __shfl_xor(x, 4, kLanesPerRow);
    return x;
}

// ------------------------------------------------------------------ decode step
template <class P, int DK, int DV>
__global__ __launch_bounds__(kThreads) void qed_step_kernel(const QedStepArgs args) {
    using R = typename P::R;
    constexpr int NG = DK / (4 * kLanesPerRow);
    constexpr int ROWS_PER_PASS = kWave / kLanesPerRow;
    constexpr int ROWS_PER_WAVE = DV / 4;
    constexpr int NPASS = ROWS_PER_WAVE / ROWS_PER_PASS;
    static_assert(NPASS >= 1 && NG >= 1, "unsupported step shape");

    const int nh = blockIdx.x;
    const int h = nh % args.H;
    const int lane = lane_id(), wave = wave_id();
    const int sub = lane % kLanesPerRow, grp = lane / kLanesPerRow;

    const R *gq = static_cast<const R *>(args.q) + static_cast<size_t>(nh) * DK;
    const R *gk = static_cast<const R *>(args.k) + static_cast<size_t>(nh) * DK;
    const R *gv = static_cast<const R *>(args.v) + static_cast<size_t>(nh) * DV;
    const float *gg = args.g + static_cast<size_t>(nh) * DK;
    const float *gb = args.b + static_cast<size_t>(nh) * DK;
    const float *gw = args.w + static_cast<size_t>(nh) * DV;
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

    const float lam = args.lam_h[h];
    f32x4 kk[NG], qq[NG], aa[NG], dec[NG];
    float ku = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NG; ++m) {
        const int c = 4 * (m * kLanesPerRow + sub);
        const f32x4 gm = *reinterpret_cast<const f32x4 *>(gg + c);
        const f32x4 bm = *reinterpret_cast<const f32x4 *>(gb + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kk[m][i] = P::to_f32(gk[c + i]);
            qq[m][i] = P::to_f32(gq[c + i]);
            dec[m][i] = __expf(gm[i]);
            aa[m][i] = bm[i] * qq[m][i];            // u = b . q for now
            ku += kk[m][i] * aa[m][i];
            kq += kk[m][i] * qq[m][i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) aa[m][i] = bm[i] * kk[m][i] + lam * aa[m][i];   // b.k + lambda u
    }
    ku = group8_sum(ku);
    kq = group8_sum(kq);
#pragma unroll
    for (int m = 0; m < NG; ++m) aa[m] -= (lam * ku) * kk[m];                   // - lambda k (k . u)

#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = wave * ROWS_PER_WAVE + p * ROWS_PER_PASS + grp;
        float pred = 0.f, c = 0.f;
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            s[p][m] *= dec[m];                       // S_bar
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pred += s[p][m][i] * aa[m][i];
                c += s[p][m][i] * qq[m][i];
            }
        }
        pred = group8_sum(pred);
        c = group8_sum(c);
        const float r = gw[row] * P::to_f32(gv[row]) - pred;
#pragma unroll
        for (int m = 0; m < NG; ++m)
            *reinterpret_cast<f32x4 *>(S + static_cast<size_t>(row) * DK + 4 * (m * kLanesPerRow + sub)) =
                s[p][m] + r * kk[m];
        if (sub == 0) go[row] = P::from_f32(c + r * kq);   // o = S_bar q + r (k . q)
    }
}

// ------------------------------------------------------------------ chunked forward
template <class P, int DK, int CH>
struct QedLayout {
    static constexpr int PAD = 16 / P::kBytes;
    static constexpr int PK = DK + PAD, PC = CH + PAD, PV = kDVT + PAD;
    static constexpr int PF = DK + 4, PW = kDVT + 4;     // fp32 pitches
    static constexpr int NQ = CH * PK, NCC = CH * PC;
    // element-type arrays: q, k, a; the decayed At, Qt, Kh, two buffers each (the chunk being
    // prepared and the chunk on the state); L, M, T; O staging
    static constexpr int oQ = 0, oK = oQ + NQ, oA = oK + NQ, oAt = oA + NQ, oQt = oAt + 2 * NQ, oKh = oQt + 2 * NQ;
    static constexpr int oL = oKh + 2 * NQ, oM = oL + NCC, oT = oM + NCC, oO = oT + NCC;
    static constexpr int nR = oO + CH * PV;
    // fp32 arrays: Gm (cumulative log decay, base 2); the w . v tile and exp(Gm_C), two
    // buffers each; three slots of partial L and M blocks (one f32x4 per lane and matrix)
    static constexpr int fG = 0, fW = fG + CH * PF, fE = fW + 2 * CH * PW, fP = fE + 2 * DK;
    static constexpr int nF = fP + 3 * 2 * 64 * 4;
    static constexpr int bytes = ((nR * P::kBytes + 15) / 16) * 16 + nF * 4;
    static_assert((PK * P::kBytes) % 16 == 0 && (PC * P::kBytes) % 16 == 0 && (PV * P::kBytes) % 16 == 0,
                  "row pitches keep 16-byte alignment");
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
};

// The key contraction of each 16 x 16 block pair of L and M is cut into NU units of 32
// channels (one MFMA each), computed by waves 4-7.  C = 32 (three pairs): wave 4, 5 and 7
// take all units but the last of pair 0, 1 and 2 and sum that pair, wave 6 takes the last
// unit of every pair (the diagonal pairs 0 and 2 are summed and inverted on different SIMDs;
// wave w runs on SIMD w mod 4).  C = 16 (one pair): unit k on wave 4 + k, summed by wave 4.
template <int NPAIR>
__device__ constexpr int qed_pair_sum_wave(int p) {
    return NPAIR == 3 ? (p == 0 ? 4 : (p == 1 ? 5 : 7)) : 4;
}
template <int NPAIR, int NU>
__device__ constexpr int qed_unit_wave(int p, int k) {
    return NPAIR == 3 ? (k < NU - 1 ? qed_pair_sum_wave<NPAIR>(p) : 6) : 4 + k;
}
// partial-block slot of wave w's share of pair p (every wave that holds a share it does not
// sum itself has one slot per pair)
template <int NPAIR>
__device__ constexpr int qed_part_slot(int w, int p) {
    return NPAIR == 3 ? p : w - 5;
}

template <class P, int DK, int CH>
__global__ __launch_bounds__(kChunkThreads, 1) void qed_chunk_kernel(const QedChunkArgs args) {
    using R = typename P::R;
    using F = typename P::F;
    using Lay = QedLayout<P, DK, CH>;
    constexpr int NKT = DK / 16, NCT = CH / 16;
    constexpr int PK = Lay::PK, PC = Lay::PC, PV = Lay::PV, PF = Lay::PF, PW = Lay::PW;
    constexpr int EPV = 16 / P::kBytes;
    constexpr int VPRV = kDVT / EPV;
    // staging threads per chunk row and key columns per staging thread (at least one 16-byte
    // run of q and k: 8 columns in bf16, 4 in fp32); threads beyond CH * TPR stage nothing
    constexpr int VMIN = EPV > 4 ? EPV : 4;
    constexpr int NT = kChunkThreads;
    constexpr int TPR = (NT / CH < DK / VMIN) ? NT / CH : DK / VMIN;
    constexpr int CPT = DK / TPR;
    static_assert(CPT % 4 == 0 && CPT <= 32, "staging split");
    constexpr int NPAIR = NCT * (NCT + 1) / 2;
    constexpr int NU = NKT / 2;                    // 32-channel units per block pair
    static_assert((NPAIR == 1 || NPAIR == 3) && NU >= 2 && NU <= 4, "C = 16 or 32, d_k = 64 or 128");
    static_assert(2 * DK <= kChunkThreads / 2, "the decay sums run on the state waves");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::bytes];
    R *const Qs = reinterpret_cast<R *>(smem) + Lay::oQ;
    R *const Ks = reinterpret_cast<R *>(smem) + Lay::oK;
    R *const As = reinterpret_cast<R *>(smem) + Lay::oA;
    R *const Ats0 = reinterpret_cast<R *>(smem) + Lay::oAt;   // [2][CH][PK]
    R *const Qts0 = reinterpret_cast<R *>(smem) + Lay::oQt;
    R *const Khs0 = reinterpret_cast<R *>(smem) + Lay::oKh;
    R *const Ls = reinterpret_cast<R *>(smem) + Lay::oL;
    R *const Ms = reinterpret_cast<R *>(smem) + Lay::oM;
    R *const Ts = reinterpret_cast<R *>(smem) + Lay::oT;
    R *const Os = reinterpret_cast<R *>(smem) + Lay::oO;
    float *const fbase = reinterpret_cast<float *>(smem + ((Lay::nR * P::kBytes + 15) / 16) * 16);
    float *const Gs = fbase + Lay::fG;
    float *const WVs0 = fbase + Lay::fW;          // [2][CH][PW]
    float *const eGC0 = fbase + Lay::fE;          // [2][DK]
    f32x4 *const Part = reinterpret_cast<f32x4 *>(fbase + Lay::fP);   // [slot][L, M][lane]

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int r16 = lane & 15, g4 = lane >> 4;

    const int nblk = gridDim.x;
    int logical = blockIdx.x;
    if (args.n_dvt > 1 && (nblk & 7) == 0) logical = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int dvt = logical % args.n_dvt;
    const int bh = logical / args.n_dvt;
    const int b = bh / args.H, h = bh % args.H;
    const int T = args.T, H = args.H, dv = args.dv;
    const int dv0 = dvt * kDVT;
    const float lam = args.lam_h[h];

    const R *__restrict__ gq = static_cast<const R *>(args.q);
    const R *__restrict__ gk = static_cast<const R *>(args.k);
    const R *__restrict__ gv = static_cast<const R *>(args.v);
    R *__restrict__ go = static_cast<R *>(args.o);
    auto tok = [&](int t) -> size_t { return (static_cast<size_t>(b) * T + t) * H + h; };

    // waves 0-3 own value columns [16 wave, 16 wave + 16) and their slice of S^T; the other
    // waves take part in the state-independent work only
    const bool state_wave = wave < 4;
    f32x4 sT[NKT];
    const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * (wave & 3) + r16) * DK;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
        sT[t] = (state_wave && args.S0) ? *reinterpret_cast<const f32x4 *>(args.S0 + srow + 16 * t + 4 * g4) : zero4();
    // settle the entry state here: inside the chunk loop the state registers are written by
    // MFMAs only, and the first product of each step should not wait for the memory counter
    // (which by then also counts the previous step's output stores)
#pragma unroll
    for (int t = 0; t < NKT; ++t) asm volatile("" : : "v"(sT[t]));

    // staging thread -> (row sr, key columns sc0 + 4 TPR j + [0, 4), j < CPT / 4): the TPR
    // threads of a row read each 4-column group of q, k, g and b as one contiguous run, so a
    // load instruction touches no cache line it does not fill.  The next chunk's raw rows are
    // loaded into registers while the current chunk computes (rows past the end are clamped
    // to the last valid row when loaded and zeroed when staged).
    const int sr = tid / TPR, sc0 = (tid % TPR) * 4;
    const bool stager = sr < CH;
    constexpr int GV = CPT / 4;                    // 4-column groups per staging thread
    auto scol = [&](int j) { return sc0 + 4 * TPR * j; };
    constexpr int NVV = (CH * VPRV + NT - 1) / NT;               // v vectors per thread
    constexpr int WPV = EPV / 4;                   // float4 of w per v vector
    F rq[GV], rk[GV];
    uint4 rv[NVV];
    f32x4 rg[GV], rb[GV], rw[NVV][WPV];
    auto gload = [&](int n) {
        const int t0 = n * CH;
        const int last = min(CH, T - t0) - 1;
        if (stager) {
            const size_t base = tok(t0 + min(sr, last)) * DK;
#pragma unroll
            for (int j = 0; j < GV; ++j) {
                rq[j] = P::ld4(gq + base + scol(j));
                rk[j] = P::ld4(gk + base + scol(j));
                rg[j] = *reinterpret_cast<const f32x4 *>(args.g + base + scol(j));
                rb[j] = *reinterpret_cast<const f32x4 *>(args.b + base + scol(j));
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = tid + NT * j;
            if (CH * VPRV % NT == 0 || vi < CH * VPRV) {
                const size_t off = tok(t0 + min(vi / VPRV, last)) * dv + dv0 + (vi % VPRV) * EPV;
                rv[j] = *reinterpret_cast<const uint4 *>(gv + off);
#pragma unroll
                for (int u = 0; u < WPV; ++u) rw[j][u] = *reinterpret_cast<const f32x4 *>(args.w + off + 4 * u);
            }
        }
    };

    // Two-stage pipeline over the chunks: step n prepares chunk n (everything that does not
    // depend on the state) while the state waves run the state-dependent part of chunk n - 1
    // from the buffers chunk n - 1 was prepared into.  Per step, with a barrier after each:
    //   P0  stage chunk n (all waves)
    //   P1  per-channel decay sums (state waves); waves 4-7 load chunk n + 1
    //   P2  decayed operands (all waves), L and M units (waves 4-7) | state part of chunk n - 1
    //   P3  L and M summed, masked, stored, diagonal blocks inverted | chunk n + 1 loaded and
    //       chunk n - 1's output stored (state waves)
    //   P4  block doubling (C = 32)
    const int NC = (T + CH - 1) / CH;
    if (NC > 0) gload(0);
    for (int n = 0; n <= NC; ++n) {
        const bool prep = n < NC;
        const int buf = n & 1;
        R *const Ats = Ats0 + buf * Lay::NQ;
        R *const Qts = Qts0 + buf * Lay::NQ;
        R *const Khs = Khs0 + buf * Lay::NQ;
        float *const WVs = WVs0 + buf * CH * PW;
        float *const eGC = eGC0 + buf * DK;
        const int t0 = n * CH;
        const int clen = min(CH, T - t0);
        const bool ok = sr < clen;   // (false for the threads that stage nothing)

        // ---- P0: stage q, k, a = b.k + lambda (b.q - k (k . b.q)), raw g; w . v tile
        float qf[CPT], kf[CPT], af[CPT];
        if (prep) {
#pragma unroll
            for (int j = 0; j < GV; ++j) {
                const f32x4 q4 = P::f32(rq[j]), k4 = P::f32(rk[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qf[4 * j + i] = ok ? q4[i] : 0.f;
                    kf[4 * j + i] = ok ? k4[i] : 0.f;
                }
            }
            float ku = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                af[c] = rb[c / 4][c % 4] * qf[c];                        // u = b . q
                ku += kf[c] * af[c];
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) af[c] = rb[c / 4][c % 4] * kf[c] + lam * af[c];
            // the TPR threads of a row are consecutive lanes of one wave
            if constexpr (TPR == 16) {
                ku = sum16(ku);
            } else {
#pragma unroll
                for (int off = 1; off < TPR; off <<= 1) ku += __shfl_xor(ku, off, TPR);
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) af[c] -= lam * ku * kf[c];
            if (stager) {
#pragma unroll
                for (int j = 0; j < GV; ++j) {
                    const int c = 4 * j;
                    P::st4(Qs + sr * PK + scol(j), f32x4{qf[c], qf[c + 1], qf[c + 2], qf[c + 3]});
                    P::st4(Ks + sr * PK + scol(j), f32x4{kf[c], kf[c + 1], kf[c + 2], kf[c + 3]});
                    P::st4(As + sr * PK + scol(j), f32x4{af[c], af[c + 1], af[c + 2], af[c + 3]});
                    // log decays in base 2 (g log2 e): every decay factor below is one exp2
                    *reinterpret_cast<f32x4 *>(Gs + sr * PF + scol(j)) = ok ? rg[j] * kLog2e : zero4();
                }
            }
#pragma unroll
            for (int j = 0; j < NVV; ++j) {
                const int vi = tid + NT * j;
                if (CH * VPRV % NT == 0 || vi < CH * VPRV) {
                    const int c = vi / VPRV, cv = vi % VPRV;
                    const R *e = reinterpret_cast<const R *>(&rv[j]);
#pragma unroll
                    for (int u = 0; u < WPV; ++u) {
                        f32x4 wv;
#pragma unroll
                        for (int i = 0; i < 4; ++i) wv[i] = c < clen ? rw[j][u][i] * P::to_f32(e[4 * u + i]) : 0.f;
                        *reinterpret_cast<f32x4 *>(WVs + c * PW + cv * EPV + 4 * u) = wv;
                    }
                }
            }
            __syncthreads();
            // ---- P1: Gm = per-channel cumulative sum of g over the chunk (padding rows add 0).
            // Lanes l and l + 32 of a state wave take the two halves of channel 32 w + l % 32:
            // each sums its half in registers, the second adds the first's total.
            if (!state_wave && n + 1 < NC) gload(n + 1);
            if (tid < 2 * DK) {
                constexpr int HC = CH / 2;
                const int c = 32 * (tid >> 6) + (lane & 31), h = lane >> 5;
                float col[HC];
#pragma unroll
                for (int t = 0; t < HC; ++t) col[t] = Gs[(HC * h + t) * PF + c];
#pragma unroll
                for (int t = 1; t < HC; ++t) col[t] += col[t - 1];
                const float first = __shfl_xor(col[HC - 1], 32);
                const float add = h ? first : 0.f;
#pragma unroll
                for (int t = 0; t < HC; ++t) Gs[(HC * h + t) * PF + c] = col[t] + add;
                if (h) eGC[c] = exp2f_fast(col[HC - 1] + add);
            }
            __syncthreads();
        }

        // ---- P2, state waves: the state-dependent part of chunk n - 1 (this wave's 16 value
        // columns)
        if (state_wave && n > 0) {
            const int pb = buf ^ 1;
            const R *const pAt = Ats0 + pb * Lay::NQ;
            const R *const pQt = Qts0 + pb * Lay::NQ;
            const R *const pKh = Khs0 + pb * Lay::NQ;
            const float *const pWV = WVs0 + pb * CH * PW;
            const float *const peGC = eGC0 + pb * DK;
            F sTf[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) sTf[t] = P::cvt(sT[t]);
            F Ef[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                f32x4 y = zero4();
#pragma unroll
                for (int t = 0; t < NKT; t += 2)
                    y = P::mma2(y, frag<P>(pAt, PK, 16 * mt, 16 * t), frag<P>(pAt, PK, 16 * mt, 16 * t + 16), sTf[t],
                                sTf[t + 1]);
                f32x4 wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[e] = pWV[(16 * mt + 4 * g4 + e) * PW + 16 * wave + r16];
                Ef[mt] = P::cvt(wv - y);
            }
            f32x4 Rr[NCT];
            F Rf[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                Rr[mt] = zero4();
#pragma unroll
                for (int s = 0; s <= mt; s += 2) {   // two 16-position blocks per MFMA
                    if (s + 1 <= mt)
                        Rr[mt] = P::mma2(Rr[mt], frag<P>(Ts, PC, 16 * mt, 16 * s), frag<P>(Ts, PC, 16 * mt, 16 * s + 16),
                                         Ef[s], Ef[s + 1]);
                    else
                        Rr[mt] = P::mma1(Rr[mt], frag<P>(Ts, PC, 16 * mt, 16 * s), Ef[s]);
                }
                Rf[mt] = P::cvt(Rr[mt]);
            }
            f32x4 O[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                O[mt] = zero4();
#pragma unroll
                for (int t = 0; t < NKT; t += 2)
                    O[mt] = P::mma2(O[mt], frag<P>(pQt, PK, 16 * mt, 16 * t), frag<P>(pQt, PK, 16 * mt, 16 * t + 16),
                                    sTf[t], sTf[t + 1]);
#pragma unroll
                for (int s = 0; s <= mt; s += 2) {
                    if (s + 1 <= mt)
                        O[mt] = P::mma2(O[mt], frag<P>(Ms, PC, 16 * mt, 16 * s), frag<P>(Ms, PC, 16 * mt, 16 * s + 16), Rf[s],
                                        Rf[s + 1]);
                    else
                        O[mt] = P::mma1(O[mt], frag<P>(Ms, PC, 16 * mt, 16 * s), Rf[s]);
                }
            }
            // S^T <- diag(exp Gm_C) S^T + Kh^T R
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                f32x4 acc = lds_f32x4(peGC + 16 * t + 4 * g4) * sT[t];
#pragma unroll
                for (int s = 0; s < NCT; s += 2) {
                    if (s + 1 < NCT)
                        acc = P::mma2(acc, frag_b<P>(pKh, PK, 16 * s, 16 * t), frag_b<P>(pKh, PK, 16 * s + 16, 16 * t), Rf[s],
                                      Rf[s + 1]);
                    else
                        acc = P::mma1(acc, frag_b<P>(pKh, PK, 16 * s, 16 * t), Rf[s]);
                }
                sT[t] = acc;
            }
            // output rows through LDS
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) Os[(16 * mt + 4 * g4 + e) * PV + 16 * wave + r16] = P::from_f32(O[mt][e]);
            }
        }
        // ---- P2, chunk n: decayed operands At = a . exp(Gm_t), Qt = q . exp(Gm_t),
        // Kh = k . exp(Gm_C - Gm_t); the L and M units
        f32x4 lacc[NPAIR], macc[NPAIR];
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) lacc[p] = macc[p] = zero4();
        if (prep) {
#pragma unroll
            for (int j = 0; j < (stager ? GV : 0); ++j) {
                const int c = 4 * j;
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(Gs + sr * PF + scol(j));
                const f32x4 gC = *reinterpret_cast<const f32x4 *>(Gs + (CH - 1) * PF + scol(j));
                f32x4 at, qt, kh;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = exp2f_fast(gm[i]);
                    at[i] = af[c + i] * e;
                    qt[i] = qf[c + i] * e;
                    kh[i] = kf[c + i] * exp2f_fast(gC[i] - gm[i]);
                }
                P::st4(Ats + sr * PK + scol(j), at);
                P::st4(Qts + sr * PK + scol(j), qt);
                P::st4(Khs + sr * PK + scol(j), kh);
            }
            if (!state_wave) {
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    int I, J;
                    tri_pair(p, I, J);
                    const int rref = (J < I) ? 16 * I : 16 * I + 8;
                    const int tr = 16 * I + r16, tc = 16 * J + r16;   // this lane's row and column token
                    // scaled operands of one 16-channel step: row a and q, column k
                    auto step = [&](int st, F &fa, F &fq, F &fk) {
                        const int c0 = 16 * st + 4 * g4;
                        const f32x4 gr = *reinterpret_cast<const f32x4 *>(Gs + rref * PF + c0);
                        const f32x4 gt = *reinterpret_cast<const f32x4 *>(Gs + tr * PF + c0);
                        const f32x4 gj = *reinterpret_cast<const f32x4 *>(Gs + tc * PF + c0);
                        const f32x4 xa = P::f32(P::ld4(As + tr * PK + c0));
                        const f32x4 xq = P::f32(P::ld4(Qs + tr * PK + c0));
                        const f32x4 xk = P::f32(P::ld4(Ks + tc * PK + c0));
                        f32x4 ea, ek;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            ea[i] = exp2f_fast(gt[i] - gr[i]);
                            ek[i] = exp2f_fast(gr[i] - gj[i]);
                        }
                        fa = P::cvt(xa * ea);
                        fq = P::cvt(xq * ea);
                        fk = P::cvt(xk * ek);
                    };
                    // formed transposed (K A^T, K Q^T): lane (g, n) gets row 16 I + n and the
                    // columns 16 J + 4 g .. + 3, the MFMA A-operand layout of the block
#pragma unroll
                    for (int k = 0; k < NU; ++k) {
                        if (qed_unit_wave<NPAIR, NU>(p, k) == wave) {
                            F a0, q0, k0, a1, q1, k1;
                            step(2 * k, a0, q0, k0);
                            step(2 * k + 1, a1, q1, k1);
                            lacc[p] = P::mma2(lacc[p], k0, k1, a0, a1);
                            macc[p] = P::mma2(macc[p], k0, k1, q0, q1);
                        }
                    }
                }
                // hand over the shares this wave does not sum itself
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    bool mine = false;
#pragma unroll
                    for (int k = 0; k < NU; ++k) mine = mine || qed_unit_wave<NPAIR, NU>(p, k) == wave;
                    if (mine && wave != qed_pair_sum_wave<NPAIR>(p)) {
                        const int sl = qed_part_slot<NPAIR>(wave, p);
                        Part[(2 * sl) * 64 + lane] = lacc[p];
                        Part[(2 * sl + 1) * 64 + lane] = macc[p];
                    }
                }
            }
        }
        __syncthreads();

        // ---- P3: L and M summed, masked and stored, diagonal blocks inverted | output of
        // chunk n - 1, loads of chunk n + 1
        if (prep && !state_wave) {
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                if (wave == qed_pair_sum_wave<NPAIR>(p)) {
                    f32x4 lsum = lacc[p], msum = macc[p];
#pragma unroll
                    for (int k = 0; k < NU; ++k) {
                        const int w2 = qed_unit_wave<NPAIR, NU>(p, k);
                        bool first = true;                 // count each other wave once
#pragma unroll
                        for (int k2 = 0; k2 < k; ++k2) first = first && qed_unit_wave<NPAIR, NU>(p, k2) != w2;
                        if (w2 != wave && first) {
                            const int sl = qed_part_slot<NPAIR>(w2, p);
                            lsum += Part[(2 * sl) * 64 + lane];
                            msum += Part[(2 * sl + 1) * 64 + lane];
                        }
                    }
                    int I, J;
                    tri_pair(p, I, J);
                    const int r = 16 * I + r16, c0 = 16 * J + 4 * g4;
                    f32x4 lv, mv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lv[e] = (c0 + e < r) ? lsum[e] : 0.f;
                        mv[e] = (c0 + e <= r) ? msum[e] : 0.f;
                    }
                    P::st4(Ls + r * PC + c0, lv);
                    P::st4(Ms + r * PC + c0, mv);
                    if (I == J) {
                        // the diagonal block's inverse (I + L)^-1 at once, in registers (products
                        // of about fp32 accuracy, from L rounded as stored, like the block
                        // doubling's reads)
                        const f32x4 t = invert_unit_lower16<typename AccurateInv<P>::Q>(P::f32(P::cvt(lv)), g4, r16);
#pragma unroll
                        for (int e = 0; e < 4; ++e) Ts[(16 * I + 4 * g4 + e) * PC + 16 * I + r16] = P::from_f32(t[e]);
                    }
                }
            }
        }
        if (state_wave) {
            if (prep && n + 1 < NC) gload(n + 1);
            if (n > 0) {
                const int pt0 = t0 - CH, plen = min(CH, T - pt0);
                for (int vi = tid; vi < CH * VPRV; vi += kChunkThreads / 2) {
                    const int c = vi / VPRV, cv = vi % VPRV;
                    if (c < plen)
                        *reinterpret_cast<uint4 *>(go + tok(pt0 + c) * dv + dv0 + cv * EPV) =
                            *reinterpret_cast<const uint4 *>(Os + c * PV + cv * EPV);
                }
            }
        }
        if (prep) {
            __syncthreads();
            // ---- P4: the block doubling (C = 32: one level)
            if constexpr (NCT >= 2) {
                inverse_level1<P, CH, PC>(Ls, Ts, wave, lane);
                __syncthreads();
            }
        }
    }
    if (state_wave && args.S_T) {
#pragma unroll
        for (int t = 0; t < NKT; ++t) *reinterpret_cast<f32x4 *>(args.S_T + srow + 16 * t + 4 * g4) = sT[t];
    }
}

template <class P, int DK, int DV>
hipError_t launch_qed_step_typed(const QedStepArgs &a, hipStream_t stream) {
    if (a.N * a.H == 0) return hipSuccess;
    hipLaunchKernelGGL((qed_step_kernel<P, DK, DV>), dim3(a.N * a.H), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <class P>
hipError_t launch_qed_step_p(int dk, int dv, const QedStepArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_qed_step_typed<P, 128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_qed_step_typed<P, 128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_qed_step_typed<P, 64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_qed_step_typed<P, 64, 64>(a, stream);
    return hipErrorInvalidValue;
}

template <class P, int DK, int CH>
hipError_t launch_qed_chunk_typed(const QedChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((qed_chunk_kernel<P, DK, CH>), dim3(grid), dim3(kChunkThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool qed_chunk_supported(int dtype, int dk, int dv, int C) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
           ((dtype == 1 && (C == 16 || C == 32)) || (dtype == 0 && C == 16));
}

hipError_t launch_qed_step(int dtype, int dk, int dv, const QedStepArgs &a, hipStream_t stream) {
    return dtype == 1 ? launch_qed_step_p<Bf16>(dk, dv, a, stream) : launch_qed_step_p<F32>(dk, dv, a, stream);
}

hipError_t launch_qed_chunk(int dtype, int dk, int C, const QedChunkArgs &a, hipStream_t stream) {
    if (dtype == 1) {
        if (C == 32) return dk == 128 ? launch_qed_chunk_typed<Bf16, 128, 32>(a, stream)
                                      : launch_qed_chunk_typed<Bf16, 64, 32>(a, stream);
        return dk == 128 ? launch_qed_chunk_typed<Bf16, 128, 16>(a, stream) : launch_qed_chunk_typed<Bf16, 64, 16>(a, stream);
    }
    return dk == 128 ? launch_qed_chunk_typed<F32, 128, 16>(a, stream) : launch_qed_chunk_typed<F32, 64, 16>(a, stream);
}

}  // namespace qd
