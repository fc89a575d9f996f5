// Helpers shared by the chunk-forward kernels.
#pragma once

#include "qd_device.h"

namespace qd {

// Lower-triangle block pair p -> (i, j), j <= i, row-major enumeration.
__device__ __forceinline__ void tri_pair(int p, int &i, int &j) {
    i = 0;
    while ((i + 1) * (i + 2) / 2 <= p) ++i;
    j = p - i * (i + 1) / 2;
}

// 16 consecutive LDS elements (16-byte aligned) as fp32
template <class P>
__device__ __forceinline__ void load_row16(const typename P::R *p, float (&out)[16]) {
    constexpr int EPV = 16 / P::kBytes;
#pragma unroll
    for (int v = 0; v < 16 / EPV; ++v) {
        const uint4 w = *reinterpret_cast<const uint4 *>(p + v * EPV);
        const typename P::R *e = reinterpret_cast<const typename P::R *>(&w);
#pragma unroll
        for (int u = 0; u < EPV; ++u) out[v * EPV + u] = P::to_f32(e[u]);
    }
}

__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
    return ok ? v : make_uint4(0, 0, 0, 0);
}

}  // namespace qd

namespace qd {

// Value of lane k of each group of four lanes (DPP quad permutation).
template <int K>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), K * 0x55, 0xf, 0xf, false));
}

// Products with fp32-like accuracy on the bf16 MFMA: each operand is split into a bf16
// head and a bf16 tail (a = hi + lo to about 2^-16 relative), and a b is formed as
// (hi_a + lo_a) hi_b + (hi_a + lo_a) lo_b, the two halves of each 16x16x32 instruction
// carrying the head and the tail of a.  Two MFMAs per 16x16x16 product, against four
// 16x16x4 fp32 MFMAs.
struct Bf16Split {
    struct F {
        bf16x4 hi, lo;
    };
    __device__ __forceinline__ static F cvt(f32x4 a) {
        F r;
        r.hi = Bf16::cvt(a);
        r.lo = Bf16::cvt(a - Bf16::f32(r.hi));
        return r;
    }
    __device__ __forceinline__ static f32x4 mma1(f32x4 acc, F a, F b) {
        return Bf16::mma2(Bf16::mma2(acc, a.hi, a.lo, b.hi, b.hi), a.hi, a.lo, b.lo, b.lo);
    }
};

// Inverse T of a 16x16 unit lower triangular block I + L, stable block forward substitution:
//   4x4 diagonal blocks inverted in registers (lanes 4j.. of a quad hold rows j),
//   then T21 = -T22 L21 T11 twice (4 -> 8 -> 16) on MFMA.
// In: lv = L[m][4g + e] (lane g = l/16, m = l%16; the MFMA A-operand layout of L, fp32).
// Out: T[4g + e][n] (n = l%16; the accumulator layout).  Both layouts of every partial
// inverse are produced by multiplying in both orders, so no LDS transposes are needed.
// Q: the products' element policy: Bf16 rounds every operand of the substitution to bf16
// (the Q-Delta forward), Bf16Split keeps about 16 bits of each operand on the bf16 MFMA
// (the QED forward and the bf16 backward, whose reverse scan carries the error of T from
// chunk to chunk), F32 computes in fp32 on the fp32 MFMA (fp32 inputs).
template <class Q>
__device__ __forceinline__ f32x4 invert_unit_lower16(f32x4 lv, int g, int m) {
    auto prod = [](f32x4 a, f32x4 b) { return Q::mma1(zero4(), Q::cvt(a), Q::cvt(b)); };
    // 4x4 diagonal blocks.  In the quad of lanes (g, 4g .. 4g+3), lane j holds row j of D
    // (D = the block's strictly lower part); the others hold rows of off-diagonal blocks.
    const int j = m & 3;
    const bool diag = (m >> 2) == g;
    const float d10 = quad_bcast<1>(lv[0]);
    const float d20 = quad_bcast<2>(lv[0]), d21 = quad_bcast<2>(lv[1]);
    const float d30 = quad_bcast<3>(lv[0]), d31 = quad_bcast<3>(lv[1]), d32 = quad_bcast<3>(lv[2]);
    // row j of D^-1 (A layout: lane (g, m) gets T4[m][4g + e])
    f32x4 ra;
    ra[0] = (j == 0) ? 1.f : -lv[0] + lv[1] * d10 + lv[2] * (d20 - d21 * d10);
    ra[1] = (j == 1) ? 1.f : -lv[1] + lv[2] * d21;
    ra[2] = (j == 2) ? 1.f : -lv[2];
    ra[3] = (j == 3) ? 1.f : 0.f;
    // column j of D^-1 (B layout: lane (g, n) gets T4[4g + e][n])
    f32x4 cb;
    cb[0] = (j == 0) ? 1.f : 0.f;
    cb[1] = ((j == 1) ? 1.f : 0.f) - d10 * cb[0];
    cb[2] = ((j == 2) ? 1.f : 0.f) - d20 * cb[0] - d21 * cb[1];
    cb[3] = ((j == 3) ? 1.f : 0.f) - d30 * cb[0] - d31 * cb[1] - d32 * cb[2];
    const f32x4 A4 = diag ? ra : zero4(), B4 = diag ? cb : zero4();
    // 4 -> 8: L restricted to 4x4 blocks (1,0) and (3,2)
    const f32x4 Lm4 = ((m >> 2) == g + 1 && (g & 1) == 0) ? lv : zero4();
    const f32x4 X = prod(Lm4, B4);                   // L' T4
    const f32x4 Y = prod(A4, X);                     // T4 L' T4
    const f32x4 Yt = prod(X, A4);                    // (T4 L' T4)^T
    const f32x4 B8 = B4 - Y, A8 = A4 - Yt;
    // 8 -> 16: L restricted to rows 8..15, columns 0..7
    const f32x4 Lm8 = (m >= 8 && g < 2) ? lv : zero4();
    const f32x4 X2 = prod(Lm8, B8);
    return B8 - prod(A8, X2);
}

// The accurate policy for a kernel's element type: split bf16 products for bf16 data, fp32
// products for fp32 data.
template <class P>
struct AccurateInv {
    using Q = Bf16Split;
};
template <>
struct AccurateInv<F32> {
    using Q = F32;
};

// Gram blocks of one chunk, NW waves over the lower block triangle.  Each block is
// computed transposed (D = K_j Q_i^T gives D[c][r] = (Q K^T)[r][c], r = 16i + l%16,
// c = 16j + 4g + e) so a lane owns four consecutive columns of a row.  Writes
//   L = strictly-lower(diag(beta) X K^T),  X K^T = K K^T + diag(lambda) Q K^T,
//   A = G o lower(Q K^T),   and, when Ns is non-null,  Ns = -N, N = G o strictly-lower(X K^T)
//   (stored negated: its one reader subtracts N Z),
// with G[r][c] = exp(g_r - g_c).  Blocks above the block diagonal are not written.
// wave: index of the calling wave among the NW that share the blocks; lane: its lane id.
// PCA: the row pitch of A (PC, the pitch of L and N, by default).
template <class P, int DK, int CH, int PK, int PC, bool HAS_A, bool HAS_L, int NW = 4, int PCA = PC>
__device__ __forceinline__ void gram_blocks(const typename P::R *Qs, const typename P::R *Ks, const float *gs,
                                            const float *bes, const float *lams, typename P::R *Ls,
                                            typename P::R *As, typename P::R *Ns, int wave = wave_id(),
                                            int lane = lane_id()) {
    using F = typename P::F;
    constexpr int NKT = DK / 16, NCT = CH / 16;
    constexpr int NPAIR = NCT * (NCT + 1) / 2, PPW = (NPAIR + NW - 1) / NW;
    const int r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < PPW; ++u) {
        const int p = wave + NW * u;
        if (p < NPAIR) {
            int i, j;
            tri_pair(p, i, j);
            f32x4 gq_ = zero4(), gk_ = zero4();
            // key contraction in octet order: one 16-byte LDS read per lane and operand
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
        }
    }
}

// T = (I + L)^-1 for the strictly lower CH x CH matrix L in LDS (pitch PC), in three
// stages that each read what the previous one wrote (a barrier between them):
//   1. inverse_diag: the 16 x 16 diagonal blocks by forward substitution over rows
//      (t_r = e_r - sum_{j<r} L[r][j] t_j; wave w < CH / 16 inverts block w, lane l
//      computes column l % 16);
//   2. inverse_level1: T21 = -T22 L21 T11 for the 16-row halves of each 32 x 32 block
//      (waves w < CH / 32);
//   3. inverse_level2 (CH = 64): the lower-left 32 x 32 quadrant, one 16 x 16 block per
//      wave w < 4.
// Only the lower block triangle of T is written; the upper triangle of each diagonal
// block comes out exactly zero.  wave is the caller's index among the waves sharing the
// work, lane its lane id (a caller inside a loop may pass opaque copies, so the per-lane
// constants are not hoisted out of its loop and held in registers).
template <class P, int CH, int PC>
__device__ __forceinline__ void inverse_diag(const typename P::R *Ls, typename P::R *Ts, int wave, int lane) {
    constexpr int NCT = CH / 16;
    if (wave < NCT) {
        const int o = 16 * wave;
        const int c = lane & 15;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float lr[16];
            load_row16<P>(Ls + (o + r) * PC + o, lr);
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int jj = 0; jj < r; ++jj) acc -= lr[jj] * t[jj];
            t[r] = acc;
        }
        if (lane < 16) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Ts[(o + r) * PC + o + c] = P::from_f32(t[r]);
        }
    }
}

// block (rb, cb) of T from an accumulator tile (rows 4g + e, column l % 16)
template <class P, int PC>
__device__ __forceinline__ void inverse_tstore(typename P::R *Ts, int rb, int cb, f32x4 val, int lane) {
    const int r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Ts[(16 * rb + 4 * g4 + e) * PC + 16 * cb + r16] = P::from_f32(val[e]);
}

// T[2a+1][2a] = -T[2a+1][2a+1] L[2a+1][2a] T[2a][2a]
template <class P, int CH, int PC>
__device__ __forceinline__ void inverse_level1(const typename P::R *Ls, typename P::R *Ts, int wave, int lane) {
    constexpr int NCT = CH / 16;
    if constexpr (NCT >= 2) {
        if (wave < NCT / 2) {
            const int rb_ = 2 * wave + 1, cb_ = 2 * wave;
            const f32x4 x = P::mma1(zero4(), frag<P>(Ls, PC, 16 * rb_, 16 * cb_), frag_b<P>(Ts, PC, 16 * cb_, 16 * cb_));
            const f32x4 y = P::mma1(zero4(), frag<P>(Ts, PC, 16 * rb_, 16 * rb_), P::cvt(x));
            inverse_tstore<P, PC>(Ts, rb_, cb_, -y, lane);
        }
    }
}

// lower-left 32x32 quadrant: T[a][c] = -sum_{m=2..a} T[a][m] sum_{k=c..1} L[m][k] T[k][c]
template <class P, int CH, int PC>
__device__ __forceinline__ void inverse_level2(const typename P::R *Ls, typename P::R *Ts, int wave, int lane) {
    constexpr int NCT = CH / 16;
    if constexpr (NCT == 4) {
        if (wave < 4) {
            const int ab = 2 + (wave >> 1), cb_ = wave & 1;
            f32x4 acc = zero4();
            for (int m = 2; m <= ab; ++m) {
                f32x4 x = zero4();
                for (int kb = cb_; kb <= 1; ++kb)
                    x = P::mma1(x, frag<P>(Ls, PC, 16 * m, 16 * kb), frag_b<P>(Ts, PC, 16 * kb, 16 * cb_));
                acc = P::mma1(acc, frag<P>(Ts, PC, 16 * ab, 16 * m), P::cvt(x));
            }
            inverse_tstore<P, PC>(Ts, ab, cb_, -acc, lane);
        }
    }
}

// The three stages with the workgroup barriers between them, by the first four waves
// (every wave must call it: it holds the barriers).  Called after a barrier that
// publishes L; ends with one.
template <class P, int CH, int PC>
__device__ __forceinline__ void unit_lower_inverse(const typename P::R *Ls, typename P::R *Ts, int lane = lane_id()) {
    constexpr int NCT = CH / 16;
    const int wave = wave_id();
    inverse_diag<P, CH, PC>(Ls, Ts, wave, lane);
    __syncthreads();
    if constexpr (NCT >= 2) {
        inverse_level1<P, CH, PC>(Ls, Ts, wave, lane);
        __syncthreads();
    }
    if constexpr (NCT == 4) {
        inverse_level2<P, CH, PC>(Ls, Ts, wave, lane);
        __syncthreads();
    }
}

// x of another lane through a DPP lane pattern (no LDS traffic)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes that share l / 16 (one row of an accumulator tile): lane ^ 1 and
// lane ^ 2 within each quad, then rotations of the 16-lane row by 4 and by 8.
__device__ __forceinline__ float sum16(float x) {
    x += dpp_mov<0xb1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4e>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x128>(x);   // row_ror:8
    return x;
}

// Sum over the wave.
__device__ __forceinline__ float sum64(float x) {
    x = sum16(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

}  // namespace qd
