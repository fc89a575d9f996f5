// Pipelined chunkwise Q-Delta layer forward for gfx950, bf16 inputs.
//
// Same arithmetic as the sequential kernel in qd_chunk_fwd.hip (Q-Delta reading
// notes §2.6, chunkwise WY/UT form with entry state; see that file for the
// per-chunk formulas), scheduled as a two-stage software pipeline inside one
// workgroup of eight waves:
//
//   scan waves 0-3  run the state-dependent part of chunk n (U~ = M1 V, K S^T and
//                   Q S^T, Z, O, the state update); wave w owns value columns
//                   [16w, 16w + 16) of the 64-wide tile and keeps its S^T slice in
//                   registers for the whole sequence;
//   prep waves 4-7  run the state-independent part of chunk n + 1 (Gram products,
//                   L and A, the UT-transform solve for T, M1 and M2).
// The scan waves also fetch chunk n + 2 from HBM at the end of their busiest phase
// and stage it into LDS at the end of the step.
//
// Every SIMD holds one wave of each role, so the latency of one role's chains is
// hidden behind the other's work.  Each pipeline step has four intervals separated
// by workgroup barriers placed outside the role branches, so both roles always
// execute the same barriers:
//
//   interval  scan (chunk n)                  prep (chunk c = n + 1)
//   I1        U~ = M1 V, K S^T, Q S^T,        Gram blocks, L, A; diagonal T blocks
//             Z = U~ + M2 Y, O (staged);
//             load chunk n + 2 from HBM
//   I2        S^T update, key tiles 0..d_k/32 T level 1 (block doubling)
//   I3        S^T update, the other half      T level 2
//   I4        store O; stage chunk n + 2      M1, M2
//
// Buffers crossing roles are double-buffered by chunk parity (q, k, v, A, gates);
// M1 and M2 are single-buffered because the scan reads them in I1 and the prep
// rewrites them in I4.  LDS: 155 KB for d_k = 128, C = 64.
#include "qd_chunk_common.h"
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kPipeThreads = 512;
constexpr int kRoleThreads = 256;
constexpr int kDVT = 64;

template <int DK, int CH>
struct PipeLayout {
    static constexpr int PAD = 8;                 // 16 bytes of bf16 row padding
    static constexpr int PK = DK + PAD;
    static constexpr int PC = CH + PAD;
    static constexpr int PV = kDVT + PAD;
    static constexpr int NQ = CH * PK;
    static constexpr int NV = CH * PV;
    static constexpr int NCC = CH * PC;
    static constexpr int oQ = 0;                  // [2][NQ]
    static constexpr int oK = oQ + 2 * NQ;        // [2][NQ]
    static constexpr int oV = oK + 2 * NQ;        // [2][NV]
    static constexpr int oA = oV + 2 * NV;        // [2][NCC]
    static constexpr int oM1 = oA + 2 * NCC;
    static constexpr int oM2 = oM1 + NCC;
    static constexpr int oL = oM2 + NCC;
    static constexpr int oT = oL + NCC;
    static constexpr int oO = oT + NCC;           // output staging [NV]
    static constexpr int nR = oO + NV;
    static constexpr int kGates = 5;              // g, exp(g), exp(g_last - g), beta, lambda
    static constexpr int bytes = nR * 2 + 2 * kGates * CH * 4;
    static_assert((PK * 2) % 16 == 0 && (PC * 2) % 16 == 0 && (PV * 2) % 16 == 0, "16-byte row alignment");
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
};

// Gram blocks (i, j) of the prep wave p, diagonal block first; u is a compile-time
// slot index and p is wave-uniform, so this folds to scalar selects (a lookup table
// would become a global load whose wait would also drain the in-flight prefetch).
// Balanced over the four prep waves for C = 64: p0 (0,0) (3,0) (3,1); p1 (1,1) (1,0)
// (3,2); p2 (2,2) (2,0) (2,1); p3 (3,3).  The wave owning a diagonal block inverts it.
template <int NCT>
__device__ __forceinline__ bool prep_block(int p, int u, int &i, int &j) {
    i = -1;
    j = -1;
    if (u == 0) {
        if (p < NCT) { i = p; j = p; }
    } else if constexpr (NCT == 4) {
        if (u == 1) {
            i = (p == 0) ? 3 : p;
            j = (p == 0) ? 0 : (p == 1) ? 0 : (p == 2) ? 0 : -1;
            if (p == 3) i = -1;
        } else {
            i = (p == 3) ? -1 : (p == 2) ? 2 : 3;
            j = (p == 0) ? 1 : (p == 1) ? 2 : 1;
        }
    } else if constexpr (NCT == 2) {
        if (u == 1 && p == 1) { i = 1; j = 0; }
    }
    return i >= 0;
}

template <int DK, int CH, bool HAS_A, bool HAS_L>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_kernel(const ChunkArgs args) {
    using P = Bf16;
    using R = uint16_t;
    using F = bf16x4;
    using Lay = PipeLayout<DK, CH>;
    constexpr int NKT = DK / 16;
    constexpr int NCT = CH / 16;
    constexpr int PK = Lay::PK, PC = Lay::PC, PV = Lay::PV;
    constexpr int EPV = 8;                        // bf16 per 16-byte vector
    constexpr int VPRQ = DK / EPV;
    constexpr int VPRV = kDVT / EPV;
    constexpr int NVQ = (CH * VPRQ + kRoleThreads - 1) / kRoleThreads;
    constexpr int NVV = (CH * VPRV + kRoleThreads - 1) / kRoleThreads;
    constexpr int NPAIR = NCT * (NCT + 1) / 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::bytes];
    R *const base = reinterpret_cast<R *>(smem);
    R *const M1s = base + Lay::oM1;
    R *const M2s = base + Lay::oM2;
    R *const Ls = base + Lay::oL;
    R *const Ts = base + Lay::oT;
    R *const Os = base + Lay::oO;
    float *const gbase = reinterpret_cast<float *>(smem + Lay::nR * 2);
    auto Qb = [&](int s) { return base + Lay::oQ + s * Lay::NQ; };
    auto Kb = [&](int s) { return base + Lay::oK + s * Lay::NQ; };
    auto Vb = [&](int s) { return base + Lay::oV + s * Lay::NV; };
    auto Ab = [&](int s) { return base + Lay::oA + s * Lay::NCC; };
    // gate arrays of slot s: 0 g, 1 exp(g), 2 exp(g_last - g), 3 beta, 4 lambda
    auto gate = [&](int s, int which) { return gbase + (s * Lay::kGates + which) * CH; };

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool is_scan = wave < 4;
    const int rw = wave & 3;                      // wave index within its role
    const int rt = tid & (kRoleThreads - 1);      // thread index within its role
    const int r16 = lane & 15;
    const int g4 = lane >> 4;

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
    const int NC = (T + CH - 1) / CH;
    auto chunk_len = [&](int c) { return min(CH, T - c * CH); };

    // ---- scan role: state slice S^T (rows d_k = 16t + 4g + i, column = own value column)
    f32x4 sT[NKT];
    const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * rw + r16) * DK;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
        sT[t] = (is_scan && args.S0) ? *reinterpret_cast<const f32x4 *>(args.S0 + srow + 16 * t + 4 * g4) : zero4();

    // ---- raw chunk registers of the scan role (loaded at the end of I1, staged in I4)
    uint4 rq[NVQ], rk[NVQ], rv[NVV];
    float ra = 1.f, rb = 0.f, rl = 0.f;
    auto gload = [&](int c) {
        const int t0 = c * CH;
        const int last = chunk_len(c) - 1;
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = rt + kRoleThreads * j;
            if (CH * VPRQ % kRoleThreads == 0 || vi < CH * VPRQ) {
                const int cc = min(vi / VPRQ, last), cv = vi % VPRQ;
                const size_t off = tok(t0 + cc) * DK + cv * EPV;
                rq[j] = *reinterpret_cast<const uint4 *>(gq + off);
                rk[j] = *reinterpret_cast<const uint4 *>(gk + off);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = rt + kRoleThreads * j;
            if (CH * VPRV % kRoleThreads == 0 || vi < CH * VPRV) {
                const int cc = min(vi / VPRV, last), cv = vi % VPRV;
                rv[j] = *reinterpret_cast<const uint4 *>(gv + tok(t0 + cc) * dv + dv0 + cv * EPV);
            }
        }
        {   // every role thread loads (clamped) so the loads carry no branch
            const size_t gi = tok(t0 + min(rt & (kWave - 1), last));
            if constexpr (HAS_A) ra = args.alpha[gi];
            rb = args.beta[gi];
            if constexpr (HAS_L) rl = args.lam[gi];
        }
    };
    auto rstore = [&](int c) {                    // stage chunk c into LDS slot c & 1
        const int s = c & 1;
        const int clen = chunk_len(c);
        R *Qs = Qb(s), *Ks = Kb(s), *Vs = Vb(s);
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int vi = rt + kRoleThreads * j;
            if (CH * VPRQ % kRoleThreads == 0 || vi < CH * VPRQ) {
                const int cc = vi / VPRQ, cv = vi % VPRQ;
                *reinterpret_cast<uint4 *>(Qs + cc * PK + cv * EPV) = keep_if(cc < clen, rq[j]);
                *reinterpret_cast<uint4 *>(Ks + cc * PK + cv * EPV) = keep_if(cc < clen, rk[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int vi = rt + kRoleThreads * j;
            if (CH * VPRV % kRoleThreads == 0 || vi < CH * VPRV) {
                const int cc = vi / VPRV, cv = vi % VPRV;
                *reinterpret_cast<uint4 *>(Vs + cc * PV + cv * EPV) = keep_if(cc < clen, rv[j]);
            }
        }
        if (rw == 0) {                            // first wave of the role: gate prefix sums
            const bool ok = lane < clen;
            float x = (HAS_A && ok) ? __logf(ra) : 0.f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            const float glast = __shfl(x, CH - 1);
            if (lane < CH) {
                gate(s, 0)[lane] = x;
                gate(s, 1)[lane] = __expf(x);
                gate(s, 2)[lane] = __expf(glast - x);
                gate(s, 3)[lane] = ok ? rb : 0.f;
                gate(s, 4)[lane] = ok ? rl : 0.f;
            }
        }
    };

    if (NC == 0) {
        if (is_scan && args.S_T) {
#pragma unroll
            for (int t = 0; t < NKT; ++t) *reinterpret_cast<f32x4 *>(args.S_T + srow + 16 * t + 4 * g4) = sT[t];
        }
        return;
    }

    if (is_scan) {
        gload(0);
        rstore(0);
    }
    __syncthreads();

    // scan-role value carried from I1 to the state update in I2/I3
    F Zd[NCT];

    for (int n = -1; n < NC; ++n) {
        const int c = n + 1;                      // the prep role's chunk
        const int ss = n & 1;                     // scan slot (n >= 0)
        const int ps = c & 1;                     // prep slot

        // ================================================================ I1
        if (is_scan) {
            if (n >= 0) {
                const R *Qs = Qb(ss), *Ks = Kb(ss), *Vs = Vb(ss);
                f32x4 Z[NCT], PQs[NCT];
                F Yf[NCT];
                // U~ = M1 V
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    Z[mt] = zero4();
#pragma unroll
                    for (int s = 0; s <= mt; s += 2) {
                        if (s + 1 <= mt)
                            Z[mt] = P::mma2(Z[mt], frag<P>(M1s, PC, 16 * mt, 16 * s),
                                            frag<P>(M1s, PC, 16 * mt, 16 * s + 16),
                                            frag_b<P>(Vs, PV, 16 * s, 16 * rw), frag_b<P>(Vs, PV, 16 * s + 16, 16 * rw));
                        else
                            Z[mt] = P::mma1(Z[mt], frag<P>(M1s, PC, 16 * mt, 16 * s), frag_b<P>(Vs, PV, 16 * s, 16 * rw));
                    }
                }
                // K S^T, Q S^T, Y = K S^T + diag(lambda) Q S^T
                F sTf[NKT];
#pragma unroll
                for (int t = 0; t < NKT; ++t) sTf[t] = P::cvt(sT[t]);
                const float *lam_s = gate(ss, 4);
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    f32x4 pk = zero4(), pq = zero4();
#pragma unroll
                    for (int t = 0; t < NKT; t += 2) {
                        pk = P::mma2(pk, frag<P>(Ks, PK, 16 * mt, 16 * t), frag<P>(Ks, PK, 16 * mt, 16 * t + 16),
                                     sTf[t], sTf[t + 1]);
                        pq = P::mma2(pq, frag<P>(Qs, PK, 16 * mt, 16 * t), frag<P>(Qs, PK, 16 * mt, 16 * t + 16),
                                     sTf[t], sTf[t + 1]);
                    }
                    PQs[mt] = pq;
                    if constexpr (HAS_L) pk += lds_f32x4(lam_s + 16 * mt + 4 * g4) * pq;
                    Yf[mt] = P::cvt(pk);
                }
                // Z = U~ + M2 Y
                const R *As = Ab(ss);
                const float *eg = gate(ss, 1), *egl = gate(ss, 2);
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
#pragma unroll
                    for (int s = 0; s <= mt; s += 2) {
                        if (s + 1 <= mt)
                            Z[mt] = P::mma2(Z[mt], frag<P>(M2s, PC, 16 * mt, 16 * s),
                                            frag<P>(M2s, PC, 16 * mt, 16 * s + 16), Yf[s], Yf[s + 1]);
                        else
                            Z[mt] = P::mma1(Z[mt], frag<P>(M2s, PC, 16 * mt, 16 * s), Yf[s]);
                    }
                }
                F Zf[NCT];
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    Zf[mt] = P::cvt(Z[mt]);
                    Zd[mt] = HAS_A ? P::cvt(lds_f32x4(egl + 16 * mt + 4 * g4) * Z[mt]) : Zf[mt];
                }
                // O = D_g Q S^T + A Z, staged in LDS for the I4 row stores
#pragma unroll
                for (int mt = 0; mt < NCT; ++mt) {
                    f32x4 o = HAS_A ? lds_f32x4(eg + 16 * mt + 4 * g4) * PQs[mt] : PQs[mt];
#pragma unroll
                    for (int s = 0; s <= mt; s += 2) {
                        if (s + 1 <= mt)
                            o = P::mma2(o, frag<P>(As, PC, 16 * mt, 16 * s), frag<P>(As, PC, 16 * mt, 16 * s + 16),
                                        Zf[s], Zf[s + 1]);
                        else
                            o = P::mma1(o, frag<P>(As, PC, 16 * mt, 16 * s), Zf[s]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        Os[(16 * mt + 4 * g4 + e) * PV + 16 * rw + r16] = P::from_f32(o[e]);
                }
            }
            // fetch chunk n + 2 now, after this role's busiest phase: it is staged into the
            // slot this role frees in I3, in I4 of this step (registers are not loop-carried)
            if (n + 2 < NC) gload(n + 2);
        } else if (c < NC) {
            const R *Qs = Qb(ps), *Ks = Kb(ps);
            R *As = Ab(ps);
            const float *gs = gate(ps, 0), *bes = gate(ps, 3), *lams = gate(ps, 4);
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                int i, j;
                if (prep_block<NCT>(rw, u, i, j)) {
                    // D = K_j Q_i^T, K_j K_i^T: lane owns r = 16i + l%16, c = 16j + 4g + e
                    f32x4 gq_ = zero4(), gk_ = zero4();
#pragma unroll
                    for (int s = 0; s < NKT; s += 2) {
                        const F a0 = frag<P>(Ks, PK, 16 * j, 16 * s);
                        const F a1 = frag<P>(Ks, PK, 16 * j, 16 * s + 16);
                        gq_ = P::mma2(gq_, a0, a1, frag<P>(Qs, PK, 16 * i, 16 * s), frag<P>(Qs, PK, 16 * i, 16 * s + 16));
                        gk_ = P::mma2(gk_, a0, a1, frag<P>(Ks, PK, 16 * i, 16 * s), frag<P>(Ks, PK, 16 * i, 16 * s + 16));
                    }
                    const int r = 16 * i + r16;
                    const int c0 = 16 * j + 4 * g4;
                    const float lr = lams[r], br = bes[r], gr = gs[r];
                    const f32x4 gc = lds_f32x4(gs + c0);
                    f32x4 lv, av;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int cc = c0 + e;
                        const float xk = HAS_L ? gk_[e] + lr * gq_[e] : gk_[e];
                        lv[e] = (cc < r) ? br * xk : 0.f;
                        av[e] = (cc <= r) ? (HAS_A ? __expf(gr - gc[e]) : 1.f) * gq_[e] : 0.f;
                    }
                    P::st4(Ls + r * PC + c0, lv);
                    P::st4(As + r * PC + c0, av);
                    if (u == 0) {
                        // diagonal block i == j == rw, inverted from this wave's registers:
                        // lane (row l%16, group g) holds L[row][4g..4g+3] of the block, and
                        // every L value the forward substitution needs is read with
                        // v_readlane (uniform), so no LDS round trips.  Lane l computes
                        // column l % 16 of T (t_r = e_r - sum_{j<r} L[r][j] t_j); the four
                        // lane groups repeat it.  L is rounded to bf16 as stored in LDS.
                        f32x4 lb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) lb[e] = P::to_f32(P::from_f32(lv[e]));
                        const int o = 16 * i;
                        const int cl = r16;
                        float tv[16];
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            float acc = 0.f;
#pragma unroll
                            for (int jj = 0; jj < rr; ++jj) {
                                const float ljj = __int_as_float(
                                    __builtin_amdgcn_readlane(__float_as_int(lb[jj & 3]), rr + 16 * (jj >> 2)));
                                acc -= ljj * tv[jj];
                            }
                            tv[rr] = (rr == cl) ? 1.f : acc;
                        }
                        if (lane < 16) {
#pragma unroll
                            for (int rr = 0; rr < 16; ++rr) Ts[(o + rr) * PC + o + cl] = P::from_f32(tv[rr]);
                        }
                    }
                }
            }
        }
        __syncthreads();

        auto tstore = [&](int rb_, int cb_, f32x4 val) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Ts[(16 * rb_ + 4 * g4 + e) * PC + 16 * cb_ + r16] = P::from_f32(val[e]);
        };

        // S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) Z, key tiles [t_lo, t_hi)
        auto state_update = [&](int t_lo, int t_hi) {
            const R *Ks = Kb(ss);
            const float dlast = HAS_A ? gate(ss, 1)[CH - 1] : 1.f;
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                if (t < t_lo || t >= t_hi) continue;
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
        };

        // ================================================================ I2
        if (is_scan) {
            if (n >= 0) state_update(0, NKT / 2);
        } else if (c < NC) {
            if constexpr (NCT >= 2) {
                if (rw < NCT / 2) {               // T[2a+1][2a] = -T[2a+1][2a+1] L[2a+1][2a] T[2a][2a]
                    const int rb_ = 2 * rw + 1, cb_ = 2 * rw;
                    const f32x4 x = P::mma1(zero4(), frag<P>(Ls, PC, 16 * rb_, 16 * cb_),
                                            frag_b<P>(Ts, PC, 16 * cb_, 16 * cb_));
                    const f32x4 y = P::mma1(zero4(), frag<P>(Ts, PC, 16 * rb_, 16 * rb_), P::cvt(x));
                    tstore(rb_, cb_, -y);
                }
            }
        }
        __syncthreads();

        // ================================================================ I3
        if (is_scan) {
            if (n >= 0) state_update(NKT / 2, NKT);
        } else if (c < NC) {
            if constexpr (NCT == 4) {             // lower-left 32x32 quadrant of T, one block per wave
                const int ab = 2 + (rw >> 1), cb_ = rw & 1;
                f32x4 acc = zero4();
                for (int m = 2; m <= ab; ++m) {
                    f32x4 x = zero4();
                    for (int kb = cb_; kb <= 1; ++kb)
                        x = P::mma1(x, frag<P>(Ls, PC, 16 * m, 16 * kb), frag_b<P>(Ts, PC, 16 * kb, 16 * cb_));
                    acc = P::mma1(acc, frag<P>(Ts, PC, 16 * ab, 16 * m), P::cvt(x));
                }
                tstore(ab, cb_, -acc);
            }
        }
        __syncthreads();

        // ================================================================ I4
        if (is_scan) {
            if (n >= 0) {
                const int t0 = n * CH, clen = chunk_len(n);
                for (int vi = rt; vi < CH * VPRV; vi += kRoleThreads) {
                    const int cc = vi / VPRV, cv = vi % VPRV;
                    if (cc < clen)
                        *reinterpret_cast<uint4 *>(go + tok(t0 + cc) * dv + dv0 + cv * EPV) =
                            *reinterpret_cast<const uint4 *>(Os + cc * PV + cv * EPV);
                }
            }
            if (n + 2 < NC) rstore(n + 2);            // into slot n & 1, freed in I3
        } else {
            if (c < NC) {
                // M1 = (H o T) diag(beta), M2 = -D_g T diag(beta): one thread per 16-column
                // row segment of the lower block triangle (NPAIR * 16 segments)
                const float *gs = gate(ps, 0), *eg = gate(ps, 1), *bes = gate(ps, 3);
                if (rt < NPAIR * 16) {
                    int i, j;
                    tri_pair(rt >> 4, i, j);
                    const int r = 16 * i + (rt & 15);
                    const int c0 = 16 * j;
                    float tr[16];
                    load_row16<P>(Ts + r * PC + c0, tr);
                    const float gr = gs[r], er = eg[r];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 bc = lds_f32x4(bes + c0 + 4 * q4);
                        const f32x4 gc = lds_f32x4(gs + c0 + 4 * q4);
                        f32x4 m1, m2;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float tb = (c0 + 4 * q4 + e <= r) ? tr[4 * q4 + e] * bc[e] : 0.f;
                            m1[e] = HAS_A ? __expf(gr - gc[e]) * tb : tb;
                            m2[e] = HAS_A ? -er * tb : -tb;
                        }
                        P::st4(M1s + r * PC + c0 + 4 * q4, m1);
                        P::st4(M2s + r * PC + c0 + 4 * q4, m2);
                    }
                }
            }
        }
        __syncthreads();
    }

    if (is_scan && args.S_T) {
#pragma unroll
        for (int t = 0; t < NKT; ++t) *reinterpret_cast<f32x4 *>(args.S_T + srow + 16 * t + 4 * g4) = sT[t];
    }
}

template <int DK, int CH>
hipError_t launch_pipe_typed(const ChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    const dim3 blk(kPipeThreads);
    if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, true>), dim3(grid), blk, 0, stream, a);
    else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, false>), dim3(grid), blk, 0, stream, a);
    else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, true>), dim3(grid), blk, 0, stream, a);
    else hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, false>), dim3(grid), blk, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_pipe(int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    if (dk == 128) {
        switch (C) {
            case 16: return launch_pipe_typed<128, 16>(a, stream);
            case 32: return launch_pipe_typed<128, 32>(a, stream);
            case 64: return launch_pipe_typed<128, 64>(a, stream);
        }
    } else if (dk == 64) {
        switch (C) {
            case 16: return launch_pipe_typed<64, 16>(a, stream);
            case 32: return launch_pipe_typed<64, 32>(a, stream);
            case 64: return launch_pipe_typed<64, 64>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace qd
