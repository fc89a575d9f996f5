// Layer backward for gfx950: gradients of sum(o dO) + sum(S_T dST) with respect to
// q, k, v, alpha, beta, lambda and S0.
//
// The pages define the forward only (Q-Delta reading notes §2.4, the gated update, and
// §2.6, its chunkwise WY/UT form); the backward below is the reverse-mode derivative of
// that chunk form.  Per chunk, with g = cumsum log alpha, G[t][j] = exp(g_t - g_j),
// D_g = diag(exp g), D_r = diag(exp(g_last - g)), X = K + diag(lambda) Q,
// A = G o lower(Q K^T), N = G o strict(X K^T), T_g = (I + diag(beta) N)^-1, the forward is
//     Y = X S^T,  R = V - D_g Y,  Z = T_g diag(beta) R,  O = D_g Q S^T + A Z,
//     S'^T = g_C S^T + K^T D_r Z.
// Three passes:
//   1. the forward over the chunks, keeping every chunk's entry state S^T (the states
//      variant of the forward kernel, no output);
//   2. chunk_bwd_scan_pipe_kernel, the reverse scan: one workgroup per (batch, head, 64 value
//      columns) walks the chunks last to first holding the exit-state gradient dS'^T,
//      stores it per chunk, and writes dV:
//        dZ = A^T dO + D_r K dS'^T,  dV = dR = diag(beta) T_g^T dZ,
//        dS^T = g_C dS'^T + Q^T D_g (dO - diag(lambda) dR) - K^T D_g dR;
//      the last dS^T is dS0;
//   3. chunk_bwd_grad_kernel: chunks are independent of each other; a resident grid of
//      workgroups walks them, prefetching the next chunk's rows into registers, one wave
//      per 16 value columns; from the chunk's S and dS' (read from global memory as MFMA
//      fragments) it recomputes R, Z, dZ, P = T_g^T dZ and the token errors
//      U = R - N Z, and forms dQ, dK, dbeta, dlambda and dalpha:
//        dA = lower(dO Z^T), dL = -strict(P Z^T) (the gradient of diag(beta) N),
//        W_o = dO S, W_p = P S, W_z = Z dS',
//        Mq = G o dA + diag(lambda) dLb,  dLb = diag(beta) (G o dL),
//        dX = dLb K - D_g diag(beta) W_p,
//        dQ = Mq K + D_g (W_o - diag(lambda beta) W_p),
//        dK = Mq^T Q + dLb^T K + D_r W_z + dX,
//        dbeta = rowdot(P, U), dlambda = rowdot(Q, dX),
//        dg = rowsum(dA o A) - colsum(dA o A) + rowsum(dL o beta N) - colsum(dL o beta N)
//             + rowdot(D_g W_o, Q) - rowdot(D_g diag(beta) W_p, X) - rowdot(D_r W_z, K)
//             + [last row] (g_C <dS', S> + sum of rowdot(D_r W_z, K)),
//           where the four pair sums are taken as rowdot(Q, Mq K) + rowdot(K, dLb K)
//           - rowdot(K, Mq^T Q + dLb^T K) (the same sums regrouped; fp32 accumulators and
//           exact q, k instead of rounded A and N),
//        dalpha = (reverse cumulative sum of dg over the chunk) / alpha.
// Both kernels use the element policy of the inputs (bf16 or fp32 MFMA operands, fp32
// accumulation) and the same Gram and triangular-inverse steps as the forward.  A short
// last chunk is padded with alpha = 1, beta = 0 and zero q, k, v, dO rows, which adds
// nothing to any gradient.
#include <atomic>

#include "qd_chunk_common.h"
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kDVT = 64;  // value columns per tile

// ------------------------------------------------------------------ pass 2, pipelined
// The reverse scan as a two-stage software pipeline over the chunks: eight waves per
// (batch, head, 64 value columns) workgroup,
//   scan waves 0-3  the state-gradient chain of chunk n (dZ, dR, dS^T update, dV); wave w
//                   owns value columns [16w, 16w + 16) and keeps its dS'^T slice in
//                   registers;
//   prep waves 4-7  the state-independent work of chunk c = n - 1 (Gram blocks, the
//                   triangular inverse, M1).
// A pipeline step has five intervals separated by workgroup barriers that both roles
// execute:
//   interval  scan (chunk n)                         prep (chunk c = n - 1), C = 64
//   I1        prefetch chunk n - 2 (registers);      Gram blocks (L, A): each wave its
//             dZ, dR                                 diagonal block, whose T it inverts in
//                                                    registers, and one of (1,0), (3,2),
//                                                    (2,0), (2,1)
//   I2        dS^T update                            waves 6, 7: Gram blocks (3,0), (3,1)
//   I3        dV staged in LDS; store half of dS'    T, level 1 (waves 4, 5); M1 of the
//             (the gradient with respect to chunk    diagonal blocks (waves 6, 7)
//             n - 1's exit state)
//   I4        stage chunk n - 2; store the other     T, level 2
//             half of dS'
//   I5        dV stores                              M1 = T_g diag(beta) below the diagonal
// (the stores of dS' are spread over the intervals in which the scan has little to do: the
// vector-memory path takes longer to accept them than the interval's other work)
// At C = 16 and 32 the prep forms every Gram block in I1, the diagonal blocks of T in I2
// and all of M1 in I5.  q, k, dO, A and the gates are double-buffered by chunk parity; M1
// is read by the scan in I1 and rewritten by the prep in I3 and I5; L and T belong to the
// prep.
// One Gram block pair (i, j), j <= i, of gram_blocks: L, A (and -N when Ns is non-null) for
// block (i, j); the callers schedule the pairs themselves.  For a diagonal block and a
// non-null Ts the lane's row of L is already in the MFMA A-operand layout, and the block's
// inverse (I + L)^-1 is formed at once in registers, with products of about fp32 accuracy
// (split bf16 for bf16 data), from L rounded as stored, and written to Ts.
template <class P, int DK, int CH, int PK, int PC, bool HAS_A, bool HAS_L, int PCA = PC>
__device__ __forceinline__ void gram_pair(const typename P::R *Qs, const typename P::R *Ks, const float *gs,
                                          const float *bes, const float *lams, typename P::R *Ls, typename P::R *As,
                                          int i, int j, int lane, typename P::R *Ns = nullptr,
                                          typename P::R *Ts = nullptr) {
    using F = typename P::F;
    constexpr int NKT = DK / 16;
    const int r16 = lane & 15, g4 = lane >> 4;
    f32x4 gq_ = zero4(), gk_ = zero4();
#pragma unroll
    for (int s = 0; s < NKT; s += 2) {
        F a0, a1, q0, q1, k0, k1;
        frag_oct<P>(Ks, PK, 16 * j, 16 * s, a0, a1, lane);
        frag_oct<P>(Qs, PK, 16 * i, 16 * s, q0, q1, lane);
        frag_oct<P>(Ks, PK, 16 * i, 16 * s, k0, k1, lane);
        gq_ = P::mma2(gq_, a0, a1, q0, q1);
        gk_ = P::mma2(gk_, a0, a1, k0, k1);
    }
    const int r = 16 * i + r16;
    const int c0 = 16 * j + 4 * g4;
    const float lr = lams[r], br = bes[r], gr = gs[r];
    const f32x4 gc = lds_f32x4(gs + c0);
    f32x4 lv, av, nv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = c0 + e;
        const float xk = HAS_L ? gk_[e] + lr * gq_[e] : gk_[e];
        const float dec = HAS_A ? __expf(gr - gc[e]) : 1.f;
        lv[e] = (c < r) ? br * xk : 0.f;
        av[e] = (c <= r) ? dec * gq_[e] : 0.f;
        nv[e] = (c < r) ? -dec * xk : 0.f;
    }
    P::st4(Ls + r * PC + c0, lv);
    P::st4(As + r * PCA + c0, av);
    if (Ns) P::st4(Ns + r * PC + c0, nv);
    if (Ts && i == j) {
        // the inverse of L as stored (rounded to the element type), the matrix the block
        // doubling's off-diagonal blocks also read
        const f32x4 t = invert_unit_lower16<typename AccurateInv<P>::Q>(P::f32(P::cvt(lv)), g4, r16);
#pragma unroll
        for (int e = 0; e < 4; ++e) Ts[(16 * i + 4 * g4 + e) * PC + 16 * i + r16] = P::from_f32(t[e]);
    }
}

template <class P, int DK, int CH>
struct ScanPipeLayout {
    static constexpr int PAD = 16 / P::kBytes;
    static constexpr int PK = DK + PAD, PC = CH + PAD, PV = kDVT + PAD;
    static constexpr int NQ = CH * PK, NV = CH * PV, NCC = CH * PC;
    static constexpr int oQ = 0, oK = oQ + 2 * NQ, oD = oK + 2 * NQ, oA = oD + 2 * NV, oM = oA + 2 * NCC;
    static constexpr int oL = oM + NCC, oT = oL + NCC, oV = oT + NCC, nR = oV + NV;
    static constexpr int kGates = 5;   // g, exp(g), exp(g_last - g), beta, lambda
    static constexpr int bytes = nR * P::kBytes + 2 * kGates * CH * 4;
};

template <class P, int DK, int CH, bool HAS_A, bool HAS_L>
__global__ __launch_bounds__(2 * kThreads, 1) void chunk_bwd_scan_pipe_kernel(const BwdArgs args) {
    using R = typename P::R;
    using F = typename P::F;
    using Lay = ScanPipeLayout<P, DK, CH>;
    static_assert(Lay::bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
    constexpr int NKT = DK / 16, NCT = CH / 16;
    constexpr int PK = Lay::PK, PC = Lay::PC, PV = Lay::PV;
    constexpr int PA = PC, PD = PV;                // row pitches of A, M1 and of dO
    constexpr int EPV = 16 / P::kBytes;
    constexpr int VPRQ = DK / EPV, VPRV = kDVT / EPV;
    constexpr int NVQ = (CH * VPRQ + kThreads - 1) / kThreads;
    constexpr int NVV = (CH * VPRV + kThreads - 1) / kThreads;
    constexpr int NPAIR = NCT * (NCT + 1) / 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::bytes];
    R *const base = reinterpret_cast<R *>(smem);
    R *const M1s = base + Lay::oM;
    R *const Ls = base + Lay::oL;
    R *const Ts = base + Lay::oT;
    R *const Vst = base + Lay::oV;                  // dV staging
    float *const gbase = reinterpret_cast<float *>(smem + Lay::nR * P::kBytes);
    auto Qb = [&](int s) { return base + Lay::oQ + s * Lay::NQ; };
    auto Kb = [&](int s) { return base + Lay::oK + s * Lay::NQ; };
    auto Db = [&](int s) { return base + Lay::oD + s * Lay::NV; };
    auto Ab = [&](int s) { return base + Lay::oA + s * Lay::NCC; };
    auto gate = [&](int s, int which) { return gbase + (s * Lay::kGates + which) * CH; };

    const int tid = threadIdx.x, wave = wave_id();
    const bool is_scan = wave < 4;
    const int rw = wave & 3;                       // wave index within its role
    const int rt = tid & (kThreads - 1);           // thread index within its role

    const int nblk = gridDim.x;
    int logical = blockIdx.x;
    if (args.n_dvt > 1 && (nblk & 7) == 0) logical = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int dvt = logical % args.n_dvt;
    const int bh = logical / args.n_dvt;
    const int b = bh / args.H, h = bh % args.H;
    const int T = args.T, H = args.H, dv = args.dv;
    const int dv0 = dvt * kDVT;
    const int NC = (T + CH - 1) / CH;

    const R *__restrict__ gq = static_cast<const R *>(args.q);
    const R *__restrict__ gk = static_cast<const R *>(args.k);
    const R *__restrict__ gdo = static_cast<const R *>(args.dO);
    R *__restrict__ gdv = static_cast<R *>(args.g_v);
    auto tok = [&](int t) -> size_t { return (static_cast<size_t>(b) * T + t) * H + h; };

    // scan role: dS'^T tiles, rows d_k = 16t + 4g + i, column = this wave's value column
    f32x4 sT[NKT];
    {
        const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
        const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * rw + r16) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            sT[t] = (is_scan && args.dST) ? *reinterpret_cast<const f32x4 *>(args.dST + srow + 16 * t + 4 * g4)
                                          : zero4();
    }

    // scan role: registers of one prefetched chunk (rows clamped to the chunk; padding rows
    // are zeroed when staged)
    struct Prefetch {
        uint4 q[NVQ], k[NVQ], d[NVV];
        float a, b, l;
    };
    auto gload = [&](int n, Prefetch &pf) {
        const int t0 = n * CH;
        const int last = min(CH, T - t0) - 1;
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = rt + kThreads * j;
            if (CH * VPRQ % kThreads == 0 || vi < CH * VPRQ) {
                const int c = min(vi / VPRQ, last), cv = vi % VPRQ;
                const size_t off = tok(t0 + c) * DK + cv * EPV;
                pf.q[j] = *reinterpret_cast<const uint4 *>(gq + off);
                pf.k[j] = *reinterpret_cast<const uint4 *>(gk + off);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = rt + kThreads * j;
            if (CH * VPRV % kThreads == 0 || vi < CH * VPRV) {
                const int c = min(vi / VPRV, last), cv = vi % VPRV;
                pf.d[j] = *reinterpret_cast<const uint4 *>(gdo + tok(t0 + c) * dv + dv0 + cv * EPV);
            }
        }
        const size_t gi = tok(t0 + min(rt & (kWave - 1), last));
        pf.a = HAS_A ? args.alpha[gi] : 1.f;
        pf.b = args.beta[gi];
        pf.l = HAS_L ? args.lam[gi] : 0.f;
    };
    auto lstore = [&](int n, const Prefetch &pf) {   // into slot n & 1
        const int s = n & 1, clen = min(CH, T - n * CH);
        R *Qs = Qb(s), *Ks = Kb(s), *Ds = Db(s);
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = rt + kThreads * j;
            if (CH * VPRQ % kThreads == 0 || vi < CH * VPRQ) {
                const int c = vi / VPRQ, cv = vi % VPRQ;
                *reinterpret_cast<uint4 *>(Qs + c * PK + cv * EPV) = keep_if(c < clen, pf.q[j]);
                *reinterpret_cast<uint4 *>(Ks + c * PK + cv * EPV) = keep_if(c < clen, pf.k[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = rt + kThreads * j;
            if (CH * VPRV % kThreads == 0 || vi < CH * VPRV) {
                const int c = vi / VPRV, cv = vi % VPRV;
                *reinterpret_cast<uint4 *>(Ds + c * PD + cv * EPV) = keep_if(c < clen, pf.d[j]);
            }
        }
        if (rw == 0) {
            const int lane = lane_id();
            const bool ok = lane < clen;
            float x = (HAS_A && ok) ? __logf(pf.a) : 0.f;
            x = wave_inclusive_sum(x);
            const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), CH - 1));
            if (lane < CH) {
                gate(s, 0)[lane] = x;
                gate(s, 1)[lane] = __expf(x);
                gate(s, 2)[lane] = __expf(glast - x);
                gate(s, 3)[lane] = ok ? pf.b : 0.f;
                gate(s, 4)[lane] = ok ? pf.l : 0.f;
            }
        }
    };

    // M1 = T_g diag(beta) for eight consecutive columns of one row of block (i, j): item
    // sub in [0, 32) takes row 16 i + sub / 2 and columns 16 j + 8 (sub & 1) .. + 7 (16-byte
    // LDS accesses)
    auto m1_item = [&](int ps, int i, int j, int sub) {
        const float *gs = gate(ps, 0), *bes = gate(ps, 3);
        const int r = 16 * i + (sub >> 1);
        const int c0 = 16 * j + 8 * (sub & 1);
        F tf[2];
        P::ld8(Ts + r * PC + c0, tf[0], tf[1]);
        const float gr = gs[r];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int ch = c0 + 4 * hh;
            const f32x4 bc = lds_f32x4(bes + ch);
            const f32x4 gc = lds_f32x4(gs + ch);
            f32x4 m1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float tb = (ch + e <= r) ? static_cast<float>(tf[hh][e]) * bc[e] : 0.f;
                m1[e] = HAS_A ? __expf(gr - gc[e]) * tb : tb;
            }
            P::st4(M1s + r * PA + ch, m1);
        }
    };

    if (NC > 0 && is_scan) {
        Prefetch pf;
        gload(NC - 1, pf);
        lstore(NC - 1, pf);
    }
    // All loads so far (dS'^T and the first chunk) complete before the loop.  Otherwise the
    // first use of dS'^T inside the loop is guarded, conservatively, by a wait for every
    // outstanding load, including the prefetch issued just before it at every step.
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();

    // scan: the gradient with respect to chunk m's exit state (dS'^T, final after I2), key
    // tiles [t_lo, t_hi)
    auto store_dh = [&](int m, int t_lo, int t_hi) {
        const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
        R *dh = static_cast<R *>(args.dHs) + (static_cast<size_t>(bh) * NC + m) * dv * DK +
                static_cast<size_t>(dv0 + 16 * rw + r16) * DK + 4 * g4;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            if (t >= t_lo && t < t_hi) P::st4(dh + 16 * t, sT[t]);
    };
    // step n: the scan on chunk n (n < NC), the prep on chunk c = n - 1 (c >= 0)
    for (int n = NC; n >= 0; --n) {
        const int c = n - 1;
        const int ss = n & 1, ps = c & 1;
        // lane ids rebuilt from an opaque copy at every step (not hoisted out of the loop)
        int lid_ = threadIdx.x;
        asm volatile("" : "+v"(lid_));
        const int lane = lid_ & (kWave - 1), r16 = lane & 15, g4 = lane >> 4;
        Prefetch pf;                               // scan: chunk n - 2, loaded in I1, staged in I4
        f32x4 dR[NCT];                             // scan: dR = dV of chunk n, I1 to I3

        // ============================================================ I1
        if (is_scan) {
            if (n - 2 >= 0) gload(n - 2, pf);
            if (n < NC) {
                const R *Ks = Kb(ss), *Ds = Db(ss), *As = Ab(ss);
                const float *egls = gate(ss, 2);
                F sTf[NKT];
#pragma unroll
                for (int t = 0; t < NKT; ++t) sTf[t] = P::cvt(sT[t]);
                // dZ = D_r K dS'^T + A^T dO (A^T upper: blocks s >= mt), then dR = M1^T dZ.
                // Software-pipelined by hand: the fragments of row tile mt + 1 are issued
                // before the MFMAs of tile mt, and scheduling fences keep the compiler from
                // sinking each LDS read next to its use.
                F Df[NCT];                             // dO blocks (s, this wave's columns)
#pragma unroll
                for (int s2 = 0; s2 < NCT; ++s2) Df[s2] = frag_b<P>(Ds, PD, 16 * s2, 16 * rw);
                F kf[2][NKT], af[2][NCT];
                auto load_mt = [&](int mt, F(&k)[NKT], F(&a)[NCT]) {
#pragma unroll
                    for (int t = 0; t < NKT; ++t) k[t] = frag<P>(Ks, PK, 16 * mt, 16 * t);
#pragma unroll
                    for (int s2 = 0; s2 < NCT; ++s2)
                        if (s2 >= mt) a[s2] = frag_b<P>(As, PA, 16 * s2, 16 * mt);
                };
                load_mt(0, kf[0], af[0]);
                F mf[NCT][NCT];                        // M1 blocks (s, mt), s >= mt, issued with the last tile
                f32x4 dZ[NCT];
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    if (mt + 1 < NCT) {
                        load_mt(mt + 1, kf[(mt + 1) & 1], af[(mt + 1) & 1]);
                    } else {
#pragma unroll
                        for (int m2 = 0; m2 < NCT; ++m2)
#pragma unroll
                            for (int s2 = m2; s2 < NCT; ++s2) mf[m2][s2] = frag_b<P>(M1s, PA, 16 * s2, 16 * m2);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 kd = zero4();
#pragma unroll
                    for (int t = 0; t < NKT; t += 2) kd = P::mma2(kd, kf[mt & 1][t], kf[mt & 1][t + 1], sTf[t], sTf[t + 1]);
                    f32x4 z = HAS_A ? lds_f32x4(egls + 16 * mt + 4 * g4) * kd : kd;
#pragma unroll
                    for (int s2 = mt; s2 < NCT; s2 += 2) {
                        if (s2 + 1 < NCT)
                            z = P::mma2(z, af[mt & 1][s2], af[mt & 1][s2 + 1], Df[s2], Df[s2 + 1]);
                        else
                            z = P::mma1(z, af[mt & 1][s2], Df[s2]);
                    }
                    dZ[mt] = z;
                    __builtin_amdgcn_sched_barrier(0);
                }
                F dZf[NCT];
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) dZf[mt] = P::cvt(dZ[mt]);
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    dR[mt] = zero4();
#pragma unroll
                    for (int s2 = mt; s2 < NCT; s2 += 2) {
                        if (s2 + 1 < NCT)
                            dR[mt] = P::mma2(dR[mt], mf[mt][s2], mf[mt][s2 + 1], dZf[s2], dZf[s2 + 1]);
                        else
                            dR[mt] = P::mma1(dR[mt], mf[mt][s2], dZf[s2]);
                    }
                }
            }
        } else if (c >= 0) {
            if constexpr (NCT == 4) {
                // two Gram pairs per wave: its diagonal block and one the inverse's levels read;
                // the last two pairs (3, 0) and (3, 1) follow in I2
                const int pi = rw == 0 ? 1 : rw == 1 ? 3 : 2, pj = rw == 0 ? 0 : rw == 1 ? 2 : rw - 2;
                gram_pair<P, DK, CH, PK, PC, HAS_A, HAS_L, PA>(Qb(ps), Kb(ps), gate(ps, 0), gate(ps, 3), gate(ps, 4),
                                                              Ls, Ab(ps), rw, rw, lane, nullptr, Ts);
                gram_pair<P, DK, CH, PK, PC, HAS_A, HAS_L, PA>(Qb(ps), Kb(ps), gate(ps, 0), gate(ps, 3), gate(ps, 4),
                                                              Ls, Ab(ps), pi, pj, lane);
            } else {
                gram_blocks<P, DK, CH, PK, PC, HAS_A, HAS_L, 4, PA>(Qb(ps), Kb(ps), gate(ps, 0), gate(ps, 3),
                                                                    gate(ps, 4), Ls, Ab(ps), nullptr, rw, lane);
            }
        }
        __syncthreads();

        // ============================================================ I2
        if (is_scan) {
            if (n < NC) {
                // dS^T <- g_C dS'^T + Q^T D_g (dO - diag(lambda) dR) - K^T D_g dR
                const R *Qs = Qb(ss), *Ks = Kb(ss), *Ds = Db(ss);
                const float *egs = gate(ss, 1), *lams = gate(ss, 4);
                F Ef[NCT], Ff[NCT];
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    const f32x4 dof = P::f32(frag_b<P>(Ds, PD, 16 * mt, 16 * rw));
                    const f32x4 eg = lds_f32x4(egs + 16 * mt + 4 * g4);
                    f32x4 e = HAS_L ? dof - lds_f32x4(lams + 16 * mt + 4 * g4) * dR[mt] : dof;
                    f32x4 f = -dR[mt];
                    if constexpr (HAS_A) {
                        e = eg * e;
                        f = eg * f;
                    }
                    Ef[mt] = P::cvt(e);
                    Ff[mt] = P::cvt(f);
                }
                const float dlast = HAS_A ? egs[CH - 1] : 1.f;
                // the transposed q and k fragments of key tile t + 1 are issued before the
                // MFMAs of tile t
                F qf[2][NCT], kf[2][NCT];
                auto load_t = [&](int t, F(&qq)[NCT], F(&kk)[NCT]) {
#pragma unroll
                    for (int s2 = 0; s2 < NCT; ++s2) {
                        qq[s2] = frag_b<P>(Qs, PK, 16 * s2, 16 * t);
                        kk[s2] = frag_b<P>(Ks, PK, 16 * s2, 16 * t);
                    }
                };
                load_t(0, qf[0], kf[0]);
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    if (t + 1 < NKT) load_t(t + 1, qf[(t + 1) & 1], kf[(t + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    f32x4 acc = sT[t] * dlast;
#pragma unroll
                    for (int s2 = 0; s2 < NCT; s2 += 2) {
                        if (s2 + 1 < NCT) {
                            acc = P::mma2(acc, qf[t & 1][s2], qf[t & 1][s2 + 1], Ef[s2], Ef[s2 + 1]);
                            acc = P::mma2(acc, kf[t & 1][s2], kf[t & 1][s2 + 1], Ff[s2], Ff[s2 + 1]);
                        } else {
                            acc = P::mma1(acc, qf[t & 1][s2], Ef[s2]);
                            acc = P::mma1(acc, kf[t & 1][s2], Ff[s2]);
                        }
                    }
                    sT[t] = acc;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else if (c >= 0) {
            if constexpr (NCT == 4) {
                if (rw >= 2)
                    gram_pair<P, DK, CH, PK, PC, HAS_A, HAS_L, PA>(Qb(ps), Kb(ps), gate(ps, 0), gate(ps, 3),
                                                                  gate(ps, 4), Ls, Ab(ps), 3, rw - 2, lane);
            } else {
                inverse_diag<P, CH, PC>(Ls, Ts, rw, lane);
            }
        }
        __syncthreads();

        // ============================================================ I3
        if (is_scan) {
            if (n < NC) {
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Vst[(16 * mt + 4 * g4 + e) * PV + 16 * rw + r16] = P::from_f32(dR[mt][e]);
            }
            if (c >= 0) store_dh(c, 0, NKT / 2);
        } else if (c >= 0) {
            inverse_level1<P, CH, PC>(Ls, Ts, rw, lane);
            if constexpr (NCT == 4) {                  // M1 of the diagonal blocks, final since I2
                if (rw >= 2) m1_item(ps, (rt - 128) >> 5, (rt - 128) >> 5, rt & 31);
            }
        }
        __syncthreads();

        // ============================================================ I4
        if (is_scan) {
            if (n - 2 >= 0) lstore(n - 2, pf);     // slot n & 1, which the scan no longer reads
            if (c >= 0) store_dh(c, NKT / 2, NKT);
        } else if (c >= 0) {
            inverse_level2<P, CH, PC>(Ls, Ts, rw, lane);
        }
        __syncthreads();

        // ============================================================ I5
        if (is_scan) {
            if (n < NC) {                          // dV rows (staged in I3, rewritten in the next I3)
                const int t0 = n * CH, clen = min(CH, T - t0);
                for (int vi = rt; vi < CH * VPRV; vi += kThreads) {
                    const int cr = vi / VPRV, cv = vi % VPRV;
                    if (cr < clen)
                        *reinterpret_cast<uint4 *>(gdv + tok(t0 + cr) * dv + dv0 + cv * EPV) =
                            *reinterpret_cast<const uint4 *>(Vst + cr * PV + cv * EPV);
                }
            }

        } else if (c >= 0) {
            // M1 = (H o T) diag(beta) = T_g diag(beta) (lower block triangle)
            if constexpr (NCT == 4) {                  // the six blocks below the diagonal
                if (rt < 192) {
                    const int pr = rt >> 5;            // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
                    const int i = pr == 0 ? 1 : pr < 3 ? 2 : 3, j = pr == 0 ? 0 : pr < 3 ? pr - 1 : pr - 3;
                    m1_item(ps, i, j, rt & 31);
                }
            } else {
                for (int idx = rt; idx < NPAIR * 32; idx += kThreads) {
                    int i, j;
                    tri_pair(idx >> 5, i, j);
                    m1_item(ps, i, j, idx & 31);
                }
            }
        }
        __syncthreads();
    }
    if (is_scan && args.g_S0) {
        const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
        const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * rw + r16) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t) *reinterpret_cast<f32x4 *>(args.g_S0 + srow + 16 * t + 4 * g4) = sT[t];
    }
}

// ------------------------------------------------------------------ pass 3: per-chunk gradients
// One chunk at a time per workgroup, one wave per 16 value columns (DV / 16 waves: all
// value columns at once); the grid is as large as fits the device at once.  LDS holds the chunk's q, k, v, dO rows, Z and P, and the C x C
// matrices; the states S and dS' are read from global memory as MFMA fragments (the
// column-local Y = X S^T and K dS'^T take each wave's 16 rows of S and dS'; the value
// contractions W_o = dO S, W_p = P S, W_z = Z dS' take 4 x 16 blocks of them).
// Four row sums at once.  x holds rows 4g + e (e = 0..3) of the 16 columns a 16-lane group
// spans (the MFMA accumulator layout); lane n of the group gets the sum over the group's
// lanes of row 4g + quad_row(n).  Two exchanges inside each quad leave every lane one of
// the four pair-then-quad partial sums, and two row rotations add the group's four quads:
// five DPP moves for the four sums.
__device__ __forceinline__ int quad_row(int n) { return 2 * (n & 1) + ((n >> 1) & 1); }
__device__ __forceinline__ float rowsum4x16(f32x4 x, int n) {
    const bool b0 = n & 1, b1 = n & 2;
    // lanes n and n ^ 1: even lanes keep rows 0 and 1, odd lanes rows 2 and 3
    const float y0 = (b0 ? x[2] : x[0]) + dpp_mov<0xb1>(b0 ? x[0] : x[2]);
    const float y1 = (b0 ? x[3] : x[1]) + dpp_mov<0xb1>(b0 ? x[1] : x[3]);
    // lanes n and n ^ 2: bit 1 clear keeps the first, set the second
    const float z = (b1 ? y1 : y0) + dpp_mov<0x4e>(b1 ? y0 : y1);
    const float z4 = z + dpp_mov<0x124>(z);          // row_ror:4
    return z4 + dpp_mov<0x128>(z4);                  // row_ror:8
}

template <class P, int DK, int CH, int DV>
struct GradLayout {
    static constexpr int NW = DV / 16;
    static constexpr int PAD = 16 / P::kBytes;
    static constexpr int PK = DK + PAD, PC = CH + PAD, PV = DV + PAD;
    static constexpr int NQ = CH * PK, NV = CH * PV, NCC = CH * PC;
    static_assert(4 * NV >= 2 * NQ, "dO, Z, P and v double as the dQ and dK staging");
    static constexpr int oQ = 0, oK = oQ + NQ, oD = oK + NQ, oZ = oD + NV, oP = oZ + NV, oV = oP + NV;
    static constexpr int oL = oV + NV, oN = oL + NCC, oT = oN + NCC, oA = oT + NCC;
    static constexpr int nR = oA + NCC;
    static constexpr int nF = 6 * CH + 3 * NW * CH + 2 * NW;   // gates; per-wave row partials; scalars
    static constexpr int bytes = nR * P::kBytes + nF * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
};

template <class P, int DK, int CH, int DV, bool HAS_A, bool HAS_L>
__global__ __launch_bounds__(DV * 4, 1) void chunk_bwd_grad_kernel(const BwdArgs args) {
    using R = typename P::R;
    using F = typename P::F;
    using Lay = GradLayout<P, DK, CH, DV>;
    constexpr int NW = Lay::NW, NT = NW * kWave;                 // waves, threads
    constexpr int NKT = DK / 16, NCT = CH / 16, NVT = DV / 16;
    constexpr int NB = NCT * NKT, NBW = (NB + NW - 1) / NW;      // d_k output blocks, per wave
    constexpr int PK = Lay::PK, PC = Lay::PC, PV = Lay::PV;
    constexpr int EPV = 16 / P::kBytes;
    constexpr int VPRQ = DK / EPV, VPRV = DV / EPV;
    constexpr int NPAIR = NCT * (NCT + 1) / 2, PPW = (NPAIR + NW - 1) / NW;
    constexpr int NLQ = (CH * VPRQ + NT - 1) / NT, NLV = (CH * VPRV + NT - 1) / NT;

    __shared__ __attribute__((aligned(16))) unsigned char smem_[Lay::bytes];

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int T = args.T, H = args.H;
    const int NC = (T + CH - 1) / CH;
    const int total = args.B * H * NC;

    const R *__restrict__ gq = static_cast<const R *>(args.q);
    const R *__restrict__ gk = static_cast<const R *>(args.k);
    const R *__restrict__ gv = static_cast<const R *>(args.v);
    const R *__restrict__ gdo = static_cast<const R *>(args.dO);
    R *__restrict__ gdq = static_cast<R *>(args.g_q);
    R *__restrict__ gdk = static_cast<R *>(args.g_k);
    const R *__restrict__ hs0 = static_cast<const R *>(args.Hs);
    const R *__restrict__ dhs0 = static_cast<const R *>(args.dHs);

    // The workgroup walks chunks it, it + gridDim.x, ...  The next chunk's q, k, v, dO rows
    // and (wave 0) the lane's gates are prefetched into registers once the current chunk's
    // global reads are done, so they overlap its last phases: q and k rows after the value
    // contractions, v, dO rows and the gates halfway through the per-d_k-block phase, which
    // has no other global traffic (issued all at once, the loads held the waves at the
    // vector-memory path).  This wave's S^T and dS'^T fragments (S rows 16 wave + l % 16)
    // are loaded right after the rows are staged, and arrive during the Gram blocks and
    // the inverse.
    uint4 xq[NLQ], xk[NLQ], xv[NLV], xd[NLV];
    float xa = 1.f, xb = 0.f, xl = 0.f;
    // part: kFetchQK (q, k rows), kFetchVD (v, dO rows and the gates), or both
    constexpr int kFetchQK = 1, kFetchVD = 2;
    auto fetch = [&](int it, int part) {
        const int n = it % NC, bh = it / NC, b = bh / H, h = bh % H;
        const int t0 = n * CH, clen = min(CH, T - t0);
        auto tok = [&](int t) -> size_t { return (static_cast<size_t>(b) * T + t) * H + h; };
        if (part & kFetchQK)
#pragma unroll
        for (int j = 0; j < NLQ; ++j) {
            const int vi = tid + NT * j;
            xq[j] = xk[j] = make_uint4(0, 0, 0, 0);
            if ((CH * VPRQ % NT == 0 || vi < CH * VPRQ) && vi / VPRQ < clen) {
                const size_t off = tok(t0 + vi / VPRQ) * DK + (vi % VPRQ) * EPV;
                xq[j] = *reinterpret_cast<const uint4 *>(gq + off);
                xk[j] = *reinterpret_cast<const uint4 *>(gk + off);
            }
        }
        if (part & kFetchVD)
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const int vi = tid + NT * j;
            xv[j] = xd[j] = make_uint4(0, 0, 0, 0);
            if ((CH * VPRV % NT == 0 || vi < CH * VPRV) && vi / VPRV < clen) {
                const size_t off = tok(t0 + vi / VPRV) * DV + (vi % VPRV) * EPV;
                xv[j] = *reinterpret_cast<const uint4 *>(gv + off);
                xd[j] = *reinterpret_cast<const uint4 *>(gdo + off);
            }
        }
        if ((part & kFetchVD) && wave == 0) {
            const bool ok = lane < clen;
            const size_t gi = tok(t0 + min(lane, clen - 1));
            xa = (HAS_A && ok) ? args.alpha[gi] : 1.f;
            xb = ok ? args.beta[gi] : 0.f;
            xl = (HAS_L && ok) ? args.lam[gi] : 0.f;
        }
    };

    if (static_cast<int>(blockIdx.x) < total) fetch(blockIdx.x, kFetchQK | kFetchVD);
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
        // Lane ids and the LDS base are rebuilt from opaque copies for every chunk rather
        // than hoisted out of the loop: LDS addresses held across the loop do not fit the
        // register file next to the prefetched rows (they were spilled, and the reloads
        // waited on the state loads in flight).
        int lid_ = threadIdx.x, zoff_ = 0;
        asm volatile("" : "+v"(lid_), "+v"(zoff_));
        const int tid = lid_, lane = lid_ & (kWave - 1), r16 = lane & 15, g4 = lane >> 4;
        unsigned char *const smem = smem_ + zoff_;
        R *const Qs = reinterpret_cast<R *>(smem) + Lay::oQ;
        R *const Ks = reinterpret_cast<R *>(smem) + Lay::oK;
        R *const Vs = reinterpret_cast<R *>(smem) + Lay::oV;
        R *const Ds = reinterpret_cast<R *>(smem) + Lay::oD;    // dO
        R *const Zs = reinterpret_cast<R *>(smem) + Lay::oZ;
        R *const Ps = reinterpret_cast<R *>(smem) + Lay::oP;
        R *const Ls = reinterpret_cast<R *>(smem) + Lay::oL;    // diag(beta) strict(X K^T), later dLb
        R *const Ns = reinterpret_cast<R *>(smem) + Lay::oN;    // -N
        R *const Ts = reinterpret_cast<R *>(smem) + Lay::oT;    // T, then T_g, later Mq
        R *const As = reinterpret_cast<R *>(smem) + Lay::oA;
        R *const Qst = Ds;                                       // dQ staging (after the value phase)
        R *const Kst = Ds + Lay::NQ;                             // dK staging
        float *const gs = reinterpret_cast<float *>(smem + Lay::nR * P::kBytes);
        float *const egs = gs + CH;
        float *const egls = egs + CH;
        float *const bes = egls + CH;
        float *const lams = bes + CH;
        float *const als = lams + CH;
        float *const pdb = als + CH;         // [NW][CH] per-wave row partials: dbeta
        float *const pdl = pdb + NW * CH;    //   dlambda
        float *const pdg = pdl + NW * CH;    //   dg
        float *const psc = pdg + NW * CH;    // [0, NW) <dS', S> per wave, [NW, 2 NW) sum rowdot(D_r W_z, K) per wave

        const int n = it % NC, bh = it / NC, b = bh / H, h = bh % H;
        const int t0 = n * CH;
        const int clen = min(CH, T - t0);
        const R *__restrict__ hs = hs0 + (static_cast<size_t>(bh) * NC + n) * DV * DK;
        const R *__restrict__ dhs = dhs0 + (static_cast<size_t>(bh) * NC + n) * DV * DK;
        auto tok = [&](int t) -> size_t { return (static_cast<size_t>(b) * T + t) * H + h; };

        // ---- stage the prefetched rows and gates
        float sdot = 0.f;
#pragma unroll
        for (int j = 0; j < NLQ; ++j) {
            const int vi = tid + NT * j;
            if (CH * VPRQ % NT == 0 || vi < CH * VPRQ) {
                *reinterpret_cast<uint4 *>(Qs + (vi / VPRQ) * PK + (vi % VPRQ) * EPV) = xq[j];
                *reinterpret_cast<uint4 *>(Ks + (vi / VPRQ) * PK + (vi % VPRQ) * EPV) = xk[j];
            }
        }
#pragma unroll
        for (int j = 0; j < NLV; ++j) {
            const int vi = tid + NT * j;
            if (CH * VPRV % NT == 0 || vi < CH * VPRV) {
                *reinterpret_cast<uint4 *>(Vs + (vi / VPRV) * PV + (vi % VPRV) * EPV) = xv[j];
                *reinterpret_cast<uint4 *>(Ds + (vi / VPRV) * PV + (vi % VPRV) * EPV) = xd[j];
            }
        }
        if (wave == 0) {
            const bool ok = lane < clen;
            float x = (HAS_A && ok) ? __logf(xa) : 0.f;
            x = wave_inclusive_sum(x);
            const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), CH - 1));
            if (lane < CH) {
                gs[lane] = x;
                egs[lane] = __expf(x);
                egls[lane] = __expf(glast - x);
                bes[lane] = xb;
                lams[lane] = xl;
                als[lane] = xa;
            }
        }
        for (int i = tid; i < 3 * NW * CH + 2 * NW; i += NT) pdb[i] = 0.f;
        __syncthreads();

        // ---- L, A, N; T = (I + L)^-1; T_g = H o T in place.  Waves 0 .. NCT - 1 form their
        // diagonal block and invert it in registers; the blocks below the diagonal go to the
        // other waves (round-robin over all waves when there are no others)
        if (wave < NCT)
            gram_pair<P, DK, CH, PK, PC, HAS_A, HAS_L>(Qs, Ks, gs, bes, lams, Ls, As, wave, wave, lane, Ns, Ts);
        constexpr int NOFF = NPAIR - NCT;
#pragma unroll
        for (int q = 0; q < NOFF; ++q) {
            if (wave == (NW > NCT ? NCT + q % (NW - NCT) : q % NW)) {
                int i = 1;
                while (i * (i + 1) / 2 <= q) ++i;
                gram_pair<P, DK, CH, PK, PC, HAS_A, HAS_L>(Qs, Ks, gs, bes, lams, Ls, As, i, q - i * (i - 1) / 2, lane,
                                                           Ns, nullptr);
            }
        }
        // this wave's 16 rows of S and dS', as B operands in octet order (one 16-byte load
        // per lane and 32 keys; the key fragments they meet are read in the same order),
        // issued as each wave finishes its Gram blocks (the waves finish at different times,
        // so the loads reach the vector-memory path spread out)
        F sTf[NKT], dsTf[NKT];
#pragma unroll
        for (int t = 0; t < NKT; t += 2) {
            const size_t off = static_cast<size_t>(16 * wave + r16) * DK + 16 * t + 8 * g4;
            P::ld8(hs + off, sTf[t], sTf[t + 1]);
            P::ld8(dhs + off, dsTf[t], dsTf[t + 1]);
        }
        __syncthreads();
        // the two block-doubling levels of the inverse (the diagonal blocks are done)
        if constexpr (NCT >= 2) {
            inverse_level1<P, CH, PC>(Ls, Ts, wave, lane);
            __syncthreads();
        }
        if constexpr (NCT == 4) {
            inverse_level2<P, CH, PC>(Ls, Ts, wave, lane);
            __syncthreads();
        }
        if constexpr (HAS_A) {
            for (int idx = tid; idx < NPAIR * 64; idx += NT) {
                int i, j;
                tri_pair(idx >> 6, i, j);
                const int r = 16 * i + ((idx >> 2) & 15);
                const int c0 = 16 * j + 4 * (idx & 3);
                const F tf = P::ld4(Ts + r * PC + c0);
                const f32x4 gc = lds_f32x4(gs + c0);
                const float gr = gs[r];
                f32x4 tg;
#pragma unroll
                for (int e = 0; e < 4; ++e) tg[e] = (c0 + e <= r) ? __expf(gr - gc[e]) * static_cast<float>(tf[e]) : 0.f;
                P::st4(Ts + r * PC + c0, tg);
            }
            __syncthreads();
        }

        // ---- column-local part: value columns [16 wave, 16 wave + 16)
        {
            f32x4 Rr[NCT], dZ[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                f32x4 pk = zero4(), pq = zero4(), kd = zero4();
#pragma unroll
                for (int t = 0; t < NKT; t += 2) {
                    F k0, k1;
                    frag_oct<P>(Ks, PK, 16 * mt, 16 * t, k0, k1, lane);
                    pk = P::mma2(pk, k0, k1, sTf[t], sTf[t + 1]);
                    kd = P::mma2(kd, k0, k1, dsTf[t], dsTf[t + 1]);
                    if constexpr (HAS_L) {
                        F q0, q1;
                        frag_oct<P>(Qs, PK, 16 * mt, 16 * t, q0, q1, lane);
                        pq = P::mma2(pq, q0, q1, sTf[t], sTf[t + 1]);
                    }
                }
                const f32x4 y = HAS_L ? pk + lds_f32x4(lams + 16 * mt + 4 * g4) * pq : pk;
                const f32x4 vf = P::f32(frag_b<P>(Vs, PV, 16 * mt, 16 * wave));
                Rr[mt] = HAS_A ? vf - lds_f32x4(egs + 16 * mt + 4 * g4) * y : vf - y;
                dZ[mt] = HAS_A ? lds_f32x4(egls + 16 * mt + 4 * g4) * kd : kd;
            }
            if constexpr (HAS_A) {
#pragma unroll
                for (int t = 0; t < NKT; ++t) {
                    const f32x4 a = P::f32(sTf[t]), d = P::f32(dsTf[t]);
                    sdot += a[0] * d[0] + a[1] * d[1] + a[2] * d[2] + a[3] * d[3];
                }
            }
            // Z = T_g diag(beta) R;  dZ += A^T dO
            F bRf[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) bRf[mt] = P::cvt(lds_f32x4(bes + 16 * mt + 4 * g4) * Rr[mt]);
            f32x4 Z[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                // contractions over the chunk's positions, two 16-position blocks per MFMA
                Z[mt] = zero4();
#pragma unroll
                for (int s = 0; s <= mt; s += 2) {
                    if (s + 1 <= mt)
                        Z[mt] = P::mma2(Z[mt], frag<P>(Ts, PC, 16 * mt, 16 * s), frag<P>(Ts, PC, 16 * mt, 16 * s + 16),
                                        bRf[s], bRf[s + 1]);
                    else
                        Z[mt] = P::mma1(Z[mt], frag<P>(Ts, PC, 16 * mt, 16 * s), bRf[s]);
                }
#pragma unroll
                for (int s = mt; s < NCT; s += 2) {
                    if (s + 1 < NCT)
                        dZ[mt] = P::mma2(dZ[mt], frag_b<P>(As, PC, 16 * s, 16 * mt), frag_b<P>(As, PC, 16 * s + 16, 16 * mt),
                                         frag_b<P>(Ds, PV, 16 * s, 16 * wave), frag_b<P>(Ds, PV, 16 * s + 16, 16 * wave));
                    else
                        dZ[mt] = P::mma1(dZ[mt], frag_b<P>(As, PC, 16 * s, 16 * mt), frag_b<P>(Ds, PV, 16 * s, 16 * wave));
                }
            }
            // P = T_g^T dZ;  U = R - N Z;  dbeta += rowdot(P, U)
            F dZf[NCT], Zf[NCT];
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                dZf[mt] = P::cvt(dZ[mt]);
                Zf[mt] = P::cvt(Z[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < NCT; ++mt) {
                f32x4 Pm = zero4();
#pragma unroll
                for (int s = mt; s < NCT; s += 2) {
                    if (s + 1 < NCT)
                        Pm = P::mma2(Pm, frag_b<P>(Ts, PC, 16 * s, 16 * mt), frag_b<P>(Ts, PC, 16 * s + 16, 16 * mt), dZf[s],
                                     dZf[s + 1]);
                    else
                        Pm = P::mma1(Pm, frag_b<P>(Ts, PC, 16 * s, 16 * mt), dZf[s]);
                }
                f32x4 U = Rr[mt];
#pragma unroll
                for (int s = 0; s <= mt; s += 2) {
                    if (s + 1 <= mt)
                        U = P::mma2(U, frag<P>(Ns, PC, 16 * mt, 16 * s), frag<P>(Ns, PC, 16 * mt, 16 * s + 16),
                                    Zf[s], Zf[s + 1]);
                    else
                        U = P::mma1(U, frag<P>(Ns, PC, 16 * mt, 16 * s), Zf[s]);
                }
                f32x4 pu;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pu[e] = Pm[e] * U[e];
                    const int o = (16 * mt + 4 * g4 + e) * PV + 16 * wave + r16;
                    Zs[o] = P::from_f32(Z[mt][e]);
                    Ps[o] = P::from_f32(Pm[e]);
                }
                // lane r16 < 4 of each 16-lane group stores row 16 mt + 4 g + quad_row(r16)
                const float db = rowsum4x16(pu, r16);
                if (r16 < 4) pdb[wave * CH + 16 * mt + 4 * g4 + quad_row(r16)] = db;
            }
        }
        __syncthreads();

        // ---- value contractions over all d_v: dA = dO Z^T, dL = P Z^T on this wave's lower blocks,
        // formed transposed (Z dO^T, Z P^T): lane (g, n) gets row 16 i + n, columns 16 j + 4 g .. + 3
        f32x4 dAacc[PPW], dLacc[PPW];
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            dAacc[u] = dLacc[u] = zero4();
            const int p = wave + NW * u;
            if (p < NPAIR) {
                int i, j;
                tri_pair(p, i, j);
#pragma unroll
                for (int vv = 0; vv < NVT; vv += 2) {
                    F z0, z1, a0, a1, b0, b1;
                    frag_oct<P>(Zs, PV, 16 * j, 16 * vv, z0, z1, lane);
                    frag_oct<P>(Ds, PV, 16 * i, 16 * vv, a0, a1, lane);
                    frag_oct<P>(Ps, PV, 16 * i, 16 * vv, b0, b1, lane);
                    dAacc[u] = P::mma2(dAacc[u], z0, z1, a0, a1);
                    dLacc[u] = P::mma2(dLacc[u], z0, z1, b0, b1);
                }
            }
        }
        // W_o = dO S, W_p = P S, W_z = Z dS' on this wave's d_k blocks (block index mt * NKT + kk),
        // contracted over the value columns in octet order, and formed transposed (S^T dO^T, ...):
        // lane (g, n) gets row 16 mt + n and the four keys 16 kk + 4 g .. + 3, the layout of the
        // per-d_k-block phase below.  The fragments S[16 vv + 8 g + i][16 kk + l % 16], i = 0..7,
        // come from global memory (rows other waves have just read, so mostly from L2; staging
        // them through LDS measured no faster)
        f32x4 Wo[NBW], Wp[NBW], Wz[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            Wo[j] = Wp[j] = Wz[j] = zero4();
            const int blk = wave + NW * j;
            if (NB % NW == 0 || blk < NB) {
                const int mt = blk / NKT, kk = blk % NKT;
#pragma unroll
                for (int vv = 0; vv < NVT; vv += 2) {
                    const size_t o0 = static_cast<size_t>(16 * vv + 8 * g4) * DK + 16 * kk + r16;
                    const size_t o1 = o0 + static_cast<size_t>(4) * DK;
                    const F s0 = P::ld4_strided(hs + o0, DK), s1 = P::ld4_strided(hs + o1, DK);
                    const F d0 = P::ld4_strided(dhs + o0, DK), d1 = P::ld4_strided(dhs + o1, DK);
                    F a0, a1, b0, b1, c0, c1;
                    frag_oct<P>(Ds, PV, 16 * mt, 16 * vv, a0, a1, lane);
                    frag_oct<P>(Ps, PV, 16 * mt, 16 * vv, b0, b1, lane);
                    frag_oct<P>(Zs, PV, 16 * mt, 16 * vv, c0, c1, lane);
                    Wo[j] = P::mma2(Wo[j], s0, s1, a0, a1);
                    Wp[j] = P::mma2(Wp[j], s0, s1, b0, b1);
                    Wz[j] = P::mma2(Wz[j], d0, d1, c0, c1);
                }
            }
        }
        __syncthreads();   // T_g, L, v, dO, Z, P are free from here on
        // the next chunk's q and k rows (this chunk's global reads are done)
        if (it + static_cast<int>(gridDim.x) < total) fetch(it + gridDim.x, kFetchQK);

        // ---- dA and dL -> Mq = G o dA + diag(lambda) dLb, dLb = diag(beta) (G o dL); each lane
        // has one row and four consecutive columns, stored with one 8-byte write per matrix
#pragma unroll
        for (int u = 0; u < PPW; ++u) {
            const int p = wave + NW * u;
            if (p < NPAIR) {
                int i, j;
                tri_pair(p, i, j);
                const int r = 16 * i + r16;
                const int c0 = 16 * j + 4 * g4;
                const float gr = gs[r], br = bes[r], lr = lams[r];
                const f32x4 gc = lds_f32x4(gs + c0);
                f32x4 mq, lb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = c0 + e;
                    const float G = HAS_A ? __expf(gr - gc[e]) : 1.f;
                    const float da = (c <= r) ? dAacc[u][e] : 0.f;
                    const float dlb = (c < r) ? -br * G * dLacc[u][e] : 0.f;
                    mq[e] = da * G + (HAS_L ? lr * dlb : 0.f);
                    lb[e] = dlb;
                }
                P::st4(Ts + r * PC + c0, mq);
                P::st4(Ls + r * PC + c0, lb);
            }
        }
        __syncthreads();   // Mq and dLb published

        // ---- per d_k block:  MqK = Mq K,  LbK = dLb K,  KT = Mq^T Q + dLb^T K;
        //   dX = LbK - D_g diag(beta) W_p,  dQ = MqK + D_g (W_o - diag(lambda beta) W_p),
        //   dK = KT + D_r W_z + dX;  the decay gradient's pair terms, rowdot(Q, MqK) +
        //   rowdot(K, LbK) - rowdot(K, KT) (the row and column sums of dA o A and dL o beta N
        //   regrouped, from fp32 accumulators and the exact q and k), together with its W
        //   terms, come to rowdot(Q, dQ) + rowdot(K, 2 dX - dK).
        //   Every product is formed transposed (K^T Mq^T, ...), so lane (g, n) holds row
        //   16 mt + n and keys 16 kk + 4 g .. + 3: the row's gates are one value per lane, its
        //   sums over the block's keys are the lane's four plus two cross-group shuffles, and
        //   dQ and dK leave as one 8-byte store per lane.
        float wz = 0.f;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            // halfway: the next chunk's v and dO rows and gates
            if (j == NBW / 2 && it + static_cast<int>(gridDim.x) < total) fetch(it + gridDim.x, kFetchVD);
            const int blk = wave + NW * j;
            if (NB % NW == 0 || blk < NB) {
                const int mt = blk / NKT, kk = blk % NKT;
                const int row = 16 * mt + r16;
                const float eg = egs[row], el = egls[row], bt = bes[row], lm = lams[row];
                // contractions over the chunk's positions, two 16-position blocks per MFMA:
                // s <= mt for Mq K and dLb K, s >= mt for Mq^T Q + dLb^T K
                f32x4 mqk = zero4(), lbk = zero4(), kt = zero4();
#pragma unroll
                for (int s = 0; s < NCT; s += 2) {
                    if (s + 1 <= mt) {
                        const F kb0 = frag_b<P>(Ks, PK, 16 * s, 16 * kk), kb1 = frag_b<P>(Ks, PK, 16 * s + 16, 16 * kk);
                        lbk = P::mma2(lbk, kb0, kb1, frag<P>(Ls, PC, 16 * mt, 16 * s), frag<P>(Ls, PC, 16 * mt, 16 * s + 16));
                        mqk = P::mma2(mqk, kb0, kb1, frag<P>(Ts, PC, 16 * mt, 16 * s), frag<P>(Ts, PC, 16 * mt, 16 * s + 16));
                    } else if (s <= mt) {
                        const F kb = frag_b<P>(Ks, PK, 16 * s, 16 * kk);
                        lbk = P::mma1(lbk, kb, frag<P>(Ls, PC, 16 * mt, 16 * s));
                        mqk = P::mma1(mqk, kb, frag<P>(Ts, PC, 16 * mt, 16 * s));
                    }
                }
#pragma unroll
                for (int s = 0; s < NCT; ++s) {
                    if (s < mt || (s - mt) % 2 != 0) continue;     // pairs (s, s + 1) from s = mt
                    if (s + 1 < NCT) {
                        kt = P::mma2(kt, frag_b<P>(Qs, PK, 16 * s, 16 * kk), frag_b<P>(Qs, PK, 16 * s + 16, 16 * kk),
                                     frag_b<P>(Ts, PC, 16 * s, 16 * mt), frag_b<P>(Ts, PC, 16 * s + 16, 16 * mt));
                        kt = P::mma2(kt, frag_b<P>(Ks, PK, 16 * s, 16 * kk), frag_b<P>(Ks, PK, 16 * s + 16, 16 * kk),
                                     frag_b<P>(Ls, PC, 16 * s, 16 * mt), frag_b<P>(Ls, PC, 16 * s + 16, 16 * mt));
                    } else {
                        kt = P::mma1(kt, frag_b<P>(Qs, PK, 16 * s, 16 * kk), frag_b<P>(Ts, PC, 16 * s, 16 * mt));
                        kt = P::mma1(kt, frag_b<P>(Ks, PK, 16 * s, 16 * kk), frag_b<P>(Ls, PC, 16 * s, 16 * mt));
                    }
                }
                const f32x4 dX = lbk - (eg * bt) * Wp[j];
                const f32x4 dQ = mqk + (HAS_L ? eg * (Wo[j] - (lm * bt) * Wp[j]) : eg * Wo[j]);
                const f32x4 dK = kt + el * Wz[j] + dX;
                const f32x4 qf = P::f32(frag<P>(Qs, PK, 16 * mt, 16 * kk));
                const f32x4 kf = P::f32(frag<P>(Ks, PK, 16 * mt, 16 * kk));
                f32x4 dgp = zero4();
                if constexpr (HAS_A) {
                    // the pair terms plus rowdot(D_g W_o, Q) - rowdot(D_g diag(beta) W_p, X) -
                    // rowdot(D_r W_z, K), regrouped as rowdot(Q, dQ) + rowdot(K, 2 dX - dK)
                    const f32x4 wzk = el * Wz[j] * kf;
                    dgp = qf * dQ + kf * (2.f * dX - dK);
                    wz += wzk[0] + wzk[1] + wzk[2] + wzk[3];
                }
                const f32x4 dlp = HAS_L ? qf * dX : zero4();
                P::st4(Qst + row * PK + 16 * kk + 4 * g4, dQ);
                P::st4(Kst + row * PK + 16 * kk + 4 * g4, dK);
                // row sums over this wave's 16 key columns: the lane's four, then the four lane
                // groups; lanes of group 0 store row 16 mt + n.  When every wave owns one key
                // tile (NW a multiple of NKT), each (wave, row) partial is written once.
                constexpr bool kOnce = NW % NKT == 0;
                const int pr = wave * CH + row;
                auto rowsum = [&](f32x4 v) {
                    float x = (v[0] + v[1]) + (v[2] + v[3]);
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    return x;
                };
                if constexpr (HAS_L) {
                    const float v = rowsum(dlp);
                    if (g4 == 0) {
                        if constexpr (kOnce) pdl[pr] = v;
                        else pdl[pr] += v;
                    }
                }
                if constexpr (HAS_A) {
                    const float v = rowsum(dgp);
                    if (g4 == 0) {
                        if constexpr (kOnce) pdg[pr] = v;
                        else pdg[pr] += v;
                    }
                }
            }
        }
        if constexpr (HAS_A) {
            wz = sum64(wz);
            const float sd = sum64(sdot);
            if (lane == 0) {
                psc[wave] = sd;
                psc[NW + wave] = wz;
            }
        }
        __syncthreads();

        // ---- stores: dQ, dK rows; per-token dbeta, dlambda, dalpha
        for (int vi = tid; vi < CH * VPRQ; vi += NT) {
            const int c = vi / VPRQ, cv = vi % VPRQ;
            if (c < clen) {
                const size_t off = tok(t0 + c) * DK + cv * EPV;
                *reinterpret_cast<uint4 *>(gdq + off) = *reinterpret_cast<const uint4 *>(Qst + c * PK + cv * EPV);
                *reinterpret_cast<uint4 *>(gdk + off) = *reinterpret_cast<const uint4 *>(Kst + c * PK + cv * EPV);
            }
        }
        // per-token sums of the waves' row partials, one quantity per wave: wave 0 dbeta,
        // wave 1 dlambda, wave 2 dalpha (its reverse cumulative sum over the chunk from a
        // DPP prefix sum: the total minus the prefix before the row)
        if (wave <= 2) {
            const float *part = wave == 0 ? pdb : wave == 1 ? pdl : pdg;
            float x = 0.f;
            if (lane < CH) {
#pragma unroll
                for (int w = 0; w < NW; ++w) x += part[w * CH + lane];
            }
            if (wave == 0) {
                if (lane < clen) args.g_beta[tok(t0 + lane)] = x;
            } else if (wave == 1) {
                if (HAS_L && args.g_lam && lane < clen) args.g_lam[tok(t0 + lane)] = x;
            } else if constexpr (HAS_A) {
                if (lane == CH - 1) {
                    float sd = 0.f, wzs = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        sd += psc[w];
                        wzs += psc[NW + w];
                    }
                    x += egs[CH - 1] * sd + wzs;
                }
                // dlog(alpha_t) = sum over the chunk's rows s >= t of dg_s
                const float inc = wave_inclusive_sum(x);
                const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inc), kWave - 1));
                if (args.g_alpha && lane < clen) args.g_alpha[tok(t0 + lane)] = (tot - inc + x) / als[lane];
            }
        }
        __syncthreads();   // the staging buffers and row partials are reused by the next chunk
    }
}

// Persistent grid for a kernel: as many workgroups as fit on the device at once (at most
// the number of work items), each walking items blockIdx.x, blockIdx.x + gridDim.x, ...
// The occupancy figure is cached per device in `cache`, which each kernel instantiation
// owns (a function-local static of its launcher), so instantiations of different block
// size or register use never share an entry.
template <class Kern>
int resident_grid(Kern kernel, int threads, long long items, std::atomic<int> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    int grid = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (grid == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        const int cus = device_cu_count();
        grid = per_cu * (cus > 0 ? cus : 256);
        if (dev >= 0) cache[dev].store(grid, std::memory_order_relaxed);
    }
    return static_cast<int>(items < grid ? items : grid);
}

template <class P, int DK, int CH, bool HAS_A, bool HAS_L>
hipError_t launch_passes(const BwdArgs &a, hipStream_t stream) {
    const int NC = (a.T + CH - 1) / CH;
    const int g2 = a.B * a.H * a.n_dvt;
    hipLaunchKernelGGL((chunk_bwd_scan_pipe_kernel<P, DK, CH, HAS_A, HAS_L>), dim3(g2), dim3(2 * kThreads), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || NC == 0) return err;
    const long long items = static_cast<long long>(a.B) * a.H * NC;
    if (a.dv == 128) {
        static std::atomic<int> cache[kMaxDevices];   // this instantiation's occupancy, per device
        auto kern = chunk_bwd_grad_kernel<P, DK, CH, 128, HAS_A, HAS_L>;
        hipLaunchKernelGGL(kern, dim3(resident_grid(kern, 512, items, cache)), dim3(512), 0, stream, a);
    } else {
        static std::atomic<int> cache[kMaxDevices];
        auto kern = chunk_bwd_grad_kernel<P, DK, CH, 64, HAS_A, HAS_L>;
        hipLaunchKernelGGL(kern, dim3(resident_grid(kern, 256, items, cache)), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <class P, int DK, int CH>
hipError_t launch_gates(const BwdArgs &a, hipStream_t stream) {
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    if (ha && hl) return launch_passes<P, DK, CH, true, true>(a, stream);
    if (ha) return launch_passes<P, DK, CH, true, false>(a, stream);
    if (hl) return launch_passes<P, DK, CH, false, true>(a, stream);
    return launch_passes<P, DK, CH, false, false>(a, stream);
}

template <class P, int DK>
hipError_t launch_chunk(int C, const BwdArgs &a, hipStream_t stream) {
    switch (C) {
        case 16: return launch_gates<P, DK, 16>(a, stream);
        case 32: return launch_gates<P, DK, 32>(a, stream);
        case 64:
            if constexpr (P::kBytes == 2) return launch_gates<P, DK, 64>(a, stream);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool chunk_bwd_supported(int dtype, int dk, int dv, int C) {
    // fp32 C = 64 would exceed the per-chunk kernel's LDS budget
    return (dtype == 0 || dtype == 1) && (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
           (C == 16 || C == 32 || (C == 64 && dtype == 1));
}

size_t chunk_bwd_workspace(int dtype, int B, int T, int H, int dk, int dv, int C) {
    if (B <= 0 || T <= 0 || H <= 0 || C <= 0) return 0;
    const size_t NC = (static_cast<size_t>(T) + C - 1) / C;
    const size_t es = dtype == 1 ? 2 : 4;   // states kept in the input element type
    return 2 * static_cast<size_t>(B) * H * NC * dv * dk * es;
}

hipError_t launch_chunk_bwd(int dtype, int dk, int C, const BwdArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    // pass 1: the forward, keeping the chunk entry states
    ChunkArgs f;
    f.q = a.q; f.k = a.k; f.v = a.v;
    f.alpha = a.alpha; f.beta = a.beta; f.lam = a.lam;
    f.S0 = a.S0; f.o = nullptr; f.S_T = nullptr;
    f.B = a.B; f.T = a.T; f.H = a.H; f.dv = a.dv; f.n_dvt = a.n_dvt;
    f.Hs = a.Hs;
    hipError_t err = hipSuccess;
    if (a.T > 0 && (err = launch_chunk_fwd_states(dtype, dk, C, f, stream)) != hipSuccess) return err;
    if (dtype == 1) return dk == 128 ? launch_chunk<Bf16, 128>(C, a, stream) : launch_chunk<Bf16, 64>(C, a, stream);
    return dk == 128 ? launch_chunk<F32, 128>(C, a, stream) : launch_chunk<F32, 64>(C, a, stream);
}

}  // namespace qd
