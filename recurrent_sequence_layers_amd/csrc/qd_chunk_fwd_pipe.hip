// Pipelined chunkwise Q-Delta layer forward for gfx950, bf16 inputs, C = 32 or 64.
//
// Arithmetic: the chunkwise WY/UT form with entry state (Q-Delta reading notes
// §2.6; the per-chunk formulas are listed in qd_chunk_fwd.hip), rearranged so that
// the chunk's decay enters the triangular solve instead of being applied after it:
//
//   L_g = H o strictly-lower(diag(beta) X K^T),   H[r][c] = exp(g_r - g_c)
//   T_g = (I + L_g)^-1 = H o (I + L)^-1           (diagonal scalings commute)
//   M1  = T_g diag(beta)                          (= (H o T) diag(beta))
//   Z   = M1 (V - D_g Y),  Y = K S^T + diag(lambda) Q S^T
//                                                 (M2 = -D_g T diag(beta) = -M1 D_g)
//   O   = D_g Q S^T + A Z,  A = H o (Q K^T) (lower, with diagonal)
//   S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) Z
//
// One workgroup of eight waves owns one (batch, head, 64-wide value tile) and runs a
// two-stage software pipeline over the chunks:
//
//   scan waves 0-3  state-dependent work of chunk n; wave w owns value columns
//                   [16w, 16w + 16) and keeps its slice of S^T (fp32) in registers;
//   prep waves 4-7  state-independent work of chunk c = n + 1 (Gram blocks, L_g, A,
//                   the UT-transform solve, M1).
//
// Every SIMD hosts one wave of each role.  Each role runs its own loop over the chunks,
// with the same four workgroup barriers per step, so that each role's registers are
// allocated for its own code alone.  A step has four intervals:
//
//   interval  scan (chunk n)                         prep (chunk c = n + 1)
//   I1        fetch q, v of chunk n + 2; Y from the  the wave's diagonal Gram block on MFMA,
//             S^T products formed a step ahead;      A and L_g written, its 16x16 block of
//             Z, O (O staged in LDS)                 T_g inverted in registers
//   I2        stage q, v of chunk n + 2 (chunk n's   M1 of the diagonal blocks; four
//             V was last read in I1, its Q a step    off-diagonal Gram blocks
//             earlier); fetch k of chunk n + 2;
//             S^T update over the first half of
//             the keys, then K S^T and Q S^T of
//             chunk n + 1 over those keys
//   I3        the same over the second half          the last two Gram blocks (waves 4,
//                                                    5); block doubling, level 1 (6, 7)
//   I4        stage k and the gate tables of chunk   block doubling, level 2 (C = 64)
//             n + 2 (each scan wave writes part of
//             the tables); store O
//
// Forming K S^T and Q S^T of chunk n + 1 as each key pair of its entry state becomes
// final takes that contraction off the path from one chunk's Z to the next chunk's Z.
//
// LDS layouts (bf16 unless noted):
//   q, k slots [2][C x d_k] in fragment order (see frag_slot);
//   v slots    [2][C][72]   padded rows;
//   A [2], M1  [C x C] in fragment order (see cc_off): one b128 read yields the eight
//                           contraction values a 16x16x32 MFMA pairs with two register
//                           tiles (positions 4g..4g+3 and 16+4g..16+4g+3);
//   L_g        [C][C + 8]   off-diagonal blocks (diagonal blocks stay in registers);
//   T_g        [C][C + 8]   stored transposed (row c holds column c of T_g);
//   O staging  [C][72];  gates [2][5][C] fp32 ([2][7][C] in the raw instances, which add
//                           1/|q| and 1/|k| of each position).
//
// Global traffic uses buffer instructions whose resource is re-based at every chunk:
// the range check returns zeros for rows past the end of the sequence and drops
// their stores, so the tail chunk needs no clamping or masking (it is padded with
// q = k = v = 0, beta = 0, alpha = 1, which leaves the state and valid outputs alone).
#include "qd_chunk_common.h"
#include "qd_device.h"
#include "qd_internal.h"

#include <type_traits>

namespace qd {
namespace {

constexpr int kPipeThreads = 512;
constexpr int kRoleThreads = 256;
constexpr int kDVT = 64;

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// acc += A (16 x 32) B (32 x 16); every bf16 product in this kernel uses this one shape
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// acc += A (16 x 16) B (16 x 16), the same instruction with a zero second slice
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 acc) {
    const bf16x4 z = {};
    return mfma32(cat8(a, z), cat8(b, z), acc);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 lds4(const uint16_t *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ void sts4(uint16_t *p, f32x4 v) {
    *reinterpret_cast<bf16x4 *>(p) = Bf16::cvt(v);
}
// LDS transpose read (8 bytes per lane): within each 16-lane group, lane 4p + q receives
// element q of the four-element chunks read by lanes 4i + p, i = 0..3.
__device__ __forceinline__ bf16x4 lds_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
    // raw buffer (stride 0): accesses at offsets >= bytes read 0 and do not write
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + __expf(-z)); }
// log(alpha) = -softplus(a) = -(max(a, 0) + log(1 + exp(-|a|)))
__device__ __forceinline__ float log_decay_from_logit(float a) {
    return -(fmaxf(a, 0.f) + __logf(1.f + __expf(-fabsf(a))));
}

// Fragment-order layout.  A 16 x 32 tile of an MFMA operand (16 rows, 32 contraction
// values) is one 1 KB block of 64 16-byte slots; lane (g, r) of a b128 read takes slot
// 16 g + (r ^ frag_swz(g)), i.e. row r and contraction values 8g .. 8g + 7 of the
// tile's ordering.  The XOR keeps both access shapes of the kernel free of LDS bank
// conflicts on gfx950 (measured): the b128 fragment reads, where each group of 16
// lanes reads one 256-byte quarter, and the transpose reads of the state update, where
// the four lanes of one row read four different quarters.
__device__ __forceinline__ int frag_swz(int g) { return (12 * g) & 15; }
__device__ __forceinline__ int frag_slot(int g, int r) { return 16 * g + (r ^ frag_swz(g)); }

// A and M1 ([C][C], bf16) in fragment order: block (row tile, 32-column group); inside a
// group, column 16h + 4g + e sits in slot (g, row) at element 4h + e, so one b128 read
// yields the eight contraction values a 16x16x32 MFMA pairs with two register tiles.
template <int CH>
__device__ __forceinline__ int cc_off(int row, int col) {
    const int c = col & 31;
    return ((row >> 4) * (CH / 32) + (col >> 5)) * 512 + 8 * frag_slot((c >> 2) & 3, row & 15) + 4 * (c >> 4) + (c & 3);
}

template <int DK, int CH, int NGATE = 5>
struct PipeLayout {
    static constexpr int NCT = CH / 16;
    static constexpr int PC = CH + 8;             // chunk x chunk rows, 16 bytes of padding
    static constexpr int PV = kDVT + 8;           // v rows and the output staging
    static constexpr int NQ = CH * DK;            // q, k in fragment order (no padding)
    static constexpr int NV = CH * PV;
    static constexpr int NCC = CH * CH;           // A, M1 in fragment order
    static constexpr int NLT = CH * PC;           // L_g, T_g: padded rows
    // bf16 element offsets
    static constexpr int oQ = 0;                  // [2][NQ]
    static constexpr int oK = oQ + 2 * NQ;        // [2][NQ]
    static constexpr int oV = oK + 2 * NQ;        // [2][NV]
    static constexpr int oA = oV + 2 * NV;        // [2][NCC]
    static constexpr int oM1 = oA + 2 * NCC;      // directly after A: both are zeroed together
    static constexpr int oLg = oM1 + NCC;
    static constexpr int oTd = oLg + NLT;
    static constexpr int oO = oTd + NLT;
    static constexpr int nR = oO + NV;
    // byte offset of the fp32 gates
    // g, exp(g), exp(g_last - g), beta, lambda; raw instances add 1/|q| and 1/|k|
    static constexpr int kGates = NGATE;
    static constexpr int oGate = nR * 2;
    static constexpr int bytes = oGate + 2 * kGates * CH * 4;
    static_assert((PC * 2) % 16 == 0 && (PV * 2) % 16 == 0 && oGate % 16 == 0,
                  "16-byte alignment of rows");
    static_assert(bytes <= 160 * 1024, "LDS budget of one gfx950 workgroup exceeded");
};

// Gram blocks (i, j), j <= i, of prep wave P in interval PH (1, 2 or 3).  C = 64: in I1 each
// wave forms its diagonal block (inverted right after its Gram products); in I2 the blocks
// (1,0) and (3,2) that level 1 of the block doubling reads in I3, and (2,0), (2,1); in I3
// (waves 4, 5, beside level 1 on waves 6, 7) the last two, (3,0) and (3,1), which only
// level 2 reads (I4).  C = 32: everything in I1.
template <int NCT, int P, int PH>
struct GramPlan { static constexpr int n = 0; static constexpr int i[4] = {0, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<4, 0, 1> { static constexpr int n = 1; static constexpr int i[4] = {0, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<4, 1, 1> { static constexpr int n = 1; static constexpr int i[4] = {1, 0, 0, 0}, j[4] = {1, 0, 0, 0}; };
template <> struct GramPlan<4, 2, 1> { static constexpr int n = 1; static constexpr int i[4] = {2, 0, 0, 0}, j[4] = {2, 0, 0, 0}; };
template <> struct GramPlan<4, 3, 1> { static constexpr int n = 1; static constexpr int i[4] = {3, 0, 0, 0}, j[4] = {3, 0, 0, 0}; };
template <> struct GramPlan<4, 0, 2> { static constexpr int n = 1; static constexpr int i[4] = {1, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<4, 1, 2> { static constexpr int n = 1; static constexpr int i[4] = {3, 0, 0, 0}, j[4] = {2, 0, 0, 0}; };
template <> struct GramPlan<4, 2, 2> { static constexpr int n = 1; static constexpr int i[4] = {2, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<4, 3, 2> { static constexpr int n = 1; static constexpr int i[4] = {2, 0, 0, 0}, j[4] = {1, 0, 0, 0}; };
template <> struct GramPlan<4, 0, 3> { static constexpr int n = 1; static constexpr int i[4] = {3, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<4, 1, 3> { static constexpr int n = 1; static constexpr int i[4] = {3, 0, 0, 0}, j[4] = {1, 0, 0, 0}; };
template <> struct GramPlan<2, 0, 1> { static constexpr int n = 2; static constexpr int i[4] = {0, 1, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlan<2, 1, 1> { static constexpr int n = 1; static constexpr int i[4] = {1, 0, 0, 0}, j[4] = {1, 0, 0, 0}; };

// The raw instances at C = 32: every off-diagonal block after I1, when the row-norm tables
// that the diagonal blocks write in I1 are there: (1, 0) on wave 6 in I2, beside nothing.
template <int NCT, int P, int PH, bool RAW>
struct GramPlanOf { using type = GramPlan<NCT, P, PH>; };
struct GramPlanDiag0 { static constexpr int n = 1; static constexpr int i[4] = {0, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
struct GramPlan10 { static constexpr int n = 1; static constexpr int i[4] = {1, 0, 0, 0}, j[4] = {0, 0, 0, 0}; };
template <> struct GramPlanOf<2, 0, 1, true> { using type = GramPlanDiag0; };
template <> struct GramPlanOf<2, 2, 2, true> { using type = GramPlan10; };

constexpr int tile_mask(const int (&t)[4], int n) {
    int m = 0;
    for (int b = 0; b < n; ++b) m |= 1 << t[b];
    return m;
}

// RAW: q and k arrive unnormalised and alpha, beta, lambda as logits.  The gates are mapped
// while the chunk is staged into LDS.  q and k are staged as they are: q^ = D_q^-1 q and
// k^ = D_k^-1 k (D = diag(sqrt(|x_t|^2 + 1e-6))) enter every product through per-position
// factors instead, K^ K^T = D_k^-1 K K^T D_k^-1 and so on, applied to the fp32 products.
// |k_t|^2 is the diagonal of the diagonal Gram blocks, |q_t|^2 that of one more product
// Q_i Q_i^T; the diagonal blocks' waves write 1/|q| and 1/|k| to two tables in I1.
// STATES: no output (neither A nor O is formed); keep every chunk's entry state S (bf16,
// [B][H][NC][d_v][d_k], ChunkArgs::Hs, when not null) for the backward.  The entry state of
// chunk n + 1 is stored in I3 and I4 of step n, as its key halves become final; with no O to
// form, the scan's I1 also takes the first quarter of the state update from I2.
// EDA: Erase-then-Delta, DeltaNet (beta = 1) over the interleaved sequence e_1, k_1, e_2,
// k_2, ... read in place: chunk row 2i is an erase token (key e_i, query and value 0) and
// row 2i + 1 the write token (k_i, q_i, v_i) of token i of the chunk's C / 2; outputs are
// stored for the odd rows only.  The staging map gives every wave rows of one parity, so
// the source of the key rows (e or k) is uniform per wave; the query rows of the erase
// tokens are zeroed once and never written.
template <int DK, int CH, bool HAS_A, bool HAS_L, bool RAW, bool STATES = false, bool EDA = false>
struct PipeKernel {
    static_assert(!EDA || (!HAS_A && !HAS_L && !RAW && !STATES), "Erase-then-Delta is the plain beta = 1 delta rule");
    using Lay = PipeLayout<DK, CH, RAW ? 7 : 5>;
    static constexpr int NKT = DK / 16, NKP = DK / 32;
    static constexpr int NCT = CH / 16, NCP = CH / 32;
    static constexpr int PC = Lay::PC, PV = Lay::PV;
    // Key layout of the register tiles: in the pair step u, lane group g supplies the
    // eight keys of quad 4u + g (32 consecutive keys per step).
    __device__ __forceinline__ static int kq(int g, int u) { return 4 * u + g; }
    // q / k element offset of lane (g, r)'s slot in fragment block (row tile mt, step u)
    __device__ __forceinline__ static int qk_off(int mt, int u, int g, int r) {
        return (mt * NKP + u) * 512 + 8 * frag_slot(g, r);
    }

    // Gram blocks of prep wave P for the chunk in slot ps, then the A and L_g epilogue.
    // Block (i, j): D = K_j [Q_i | K_i]^T, so lane (g, n) holds q_r.k_c and k_r.k_c for
    // r = 16i + n, c = 16j + 4g + e.
    // RAW: nqs, nks are the chunk's 1/|q| and 1/|k| tables, written here by the diagonal
    // blocks (I1) and read by the blocks below the diagonal (I2, I3).
    template <int P, int PH>
    __device__ __forceinline__ static void gram(const uint16_t *Qs, const uint16_t *Ks, uint16_t *As, uint16_t *Lg,
                                                uint16_t *Td, const float *gs, const float *bes, const float *lams,
                                                float *nqs, float *nks, int r16, int g4, f32x4 &tdiag) {
        using Plan = typename GramPlanOf<NCT, P, PH, RAW>::type;
        constexpr int NB = Plan::n;
        if constexpr (NB > 0) {
            f32x4 gq[NB], gk[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) { gq[b] = zero4(); gk[b] = zero4(); }
            f32x4 gqq[RAW ? NB : 1];
            if constexpr (RAW) {
#pragma unroll
                for (int b = 0; b < NB; ++b) gqq[b] = zero4();
            }
            // 16-row tiles of K and Q this wave reads (each loaded once per key pair); the
            // tiles of the next key pair are issued before the MFMAs of the current one
            constexpr int kmask = tile_mask(Plan::i, NB) | tile_mask(Plan::j, NB);
            constexpr int qmask = tile_mask(Plan::i, NB);
            bf16x8 kt[2][NCT], qt[2][NCT];
            auto load = [&](int u, bf16x8(&k)[NCT], bf16x8(&q)[NCT]) {
#pragma unroll
                for (int m = 0; m < NCT; ++m) {
                    const int off = qk_off(m, u, g4, r16);
                    if (kmask & (1 << m)) k[m] = lds8(Ks + off);
                    if (qmask & (1 << m)) q[m] = lds8(Qs + off);
                }
            };
            load(0, kt[0], qt[0]);
#pragma unroll
            for (int u = 0; u < NKP; ++u) {
                if (u + 1 < NKP) load(u + 1, kt[(u + 1) & 1], qt[(u + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const bf16x8 a = kt[u & 1][Plan::j[b]];
                    gq[b] = mfma32(a, qt[u & 1][Plan::i[b]], gq[b]);
                    gk[b] = mfma32(a, kt[u & 1][Plan::i[b]], gk[b]);
                    // RAW, diagonal block: Q_i Q_i^T for the squared norms of the block's queries
                    if constexpr (RAW)
                        if (Plan::i[b] == Plan::j[b]) gqq[b] = mfma32(qt[u & 1][Plan::i[b]], qt[u & 1][Plan::i[b]], gqq[b]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int i = Plan::i[b], j = Plan::j[b];
                const int r = 16 * i + r16;
                const int c0 = 16 * j + 4 * g4;
                const float gr = gs[r], br = bes[r];
                const float lr = HAS_L ? lams[r] : 0.f;
                const f32x4 gc = lds_f32x4(gs + c0);
                f32x4 av, lv;
                if constexpr (RAW) {
                    if (i == j) {
                        // the diagonal of the block's K K^T and Q Q^T: lane (n / 4, n), element n % 4
                        if ((r16 >> 2) == g4) {
                            const int e = r16 & 3;
                            const float k2 = e == 0 ? gk[b][0] : e == 1 ? gk[b][1] : e == 2 ? gk[b][2] : gk[b][3];
                            const float q2 = e == 0 ? gqq[b][0] : e == 1 ? gqq[b][1] : e == 2 ? gqq[b][2] : gqq[b][3];
                            nks[r] = __frsqrt_rn(k2 + 1e-6f);
                            nqs[r] = __frsqrt_rn(q2 + 1e-6f);
                        }
                        // the other lanes of the wave read these entries: make the writes
                        // visible across the wave (without this the compiler may hand each
                        // lane its own unwritten value instead of reading the table)
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                        __builtin_amdgcn_wave_barrier();
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    }
                    // written by this wave just above (diagonal block) or by another in I1
                    const float rk = nks[r], rq = nqs[r];
                    const f32x4 rkc = lds_f32x4(nks + c0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int cc = c0 + e;
                        const float f = HAS_A ? __expf(gr - gc[e]) : 1.f;
                        const float qk = gq[b][e] * (rq * rkc[e]);
                        const float kk = gk[b][e] * (rk * rkc[e]);
                        const float xk = HAS_L ? kk + lr * qk : kk;
                        av[e] = (cc <= r) ? f * qk : 0.f;
                        lv[e] = (cc < r) ? (f * br) * xk : 0.f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int cc = c0 + e;
                        const float f = HAS_A ? __expf(gr - gc[e]) : 1.f;
                        const float xk = HAS_L ? gk[b][e] + lr * gq[b][e] : gk[b][e];
                        av[e] = (cc <= r) ? f * gq[b][e] : 0.f;
                        lv[e] = (cc < r) ? (f * br) * xk : 0.f;
                    }
                }
                if constexpr (!STATES) sts4(As + cc_off<CH>(r, c0), av);   // A serves the output only
                if (i == j) {
                    tdiag = invert_unit_lower16<Bf16>(lv, g4, r16);
                    sts4(Td + (16 * i + r16) * PC + 16 * i + 4 * g4, tdiag);   // T_g[16i + 4g + e][16i + n]
                } else {
                    sts4(Lg + r * PC + c0, lv);
                }
            }
        }
    }

    // Block doubling, level 2 (C = 64): block (ab, cb) of the lower-left 32 x 32 quadrant,
    //   T_g[ab][cb] = -sum_m T_g[ab][m] X[m][cb],  X[m][cb] = sum_kb L_g[m][kb] T_g[kb][cb],
    // with M1 = T_g diag(beta) written for it.  The outer product is formed transposed,
    // X^T T_g[ab][m]^T: the X accumulators serve as the A operand (X^T) and the transpose
    // read of T_g[ab][m] (T_g is kept transposed) is the B operand of T_g[ab][m]^T, so each
    // lane ends with four consecutive columns of one row of M1.
    template <int AB, int CB>
    __device__ __forceinline__ static void level2(const uint16_t *Lgs, const uint16_t *Tds, uint16_t *M1s,
                                                  const float *bes, int lane) {
        const int r16 = lane & 15, g4 = lane >> 4, tri = r16 >> 2, trp = r16 & 3;
        // B operands T_g[kb][cb] (kept transposed: row 16 cb + n holds column 16 cb + n)
        const bf16x4 t1 = lds4(Tds + (16 * CB + r16) * PC + 16 + 4 * g4);
        bf16x4 t0 = {};
        if constexpr (CB == 0) t0 = lds4(Tds + r16 * PC + 4 * g4);
        bf16x4 l0[2], l1[2], tt[2];
#pragma unroll
        for (int i = 0; i < AB - 1; ++i) {
            const int m = 2 + i;
            l1[i] = lds4(Lgs + (16 * m + r16) * PC + 16 + 4 * g4);
            if constexpr (CB == 0) l0[i] = lds4(Lgs + (16 * m + r16) * PC + 4 * g4);
            tt[i] = lds_tr(Tds + (16 * m + 4 * g4 + tri) * PC + 16 * AB + 4 * trp);
        }
        bf16x4 xb[2];
#pragma unroll
        for (int i = 0; i < AB - 1; ++i) {
            const f32x4 x = (CB == 0) ? mfma32(cat8(l0[i], l1[i]), cat8(t0, t1), zero4()) : mfma16(l1[i], t1, zero4());
            xb[i] = Bf16::cvt(x);
        }
        const f32x4 acc = (AB == 3) ? mfma32(cat8(xb[0], xb[1]), cat8(tt[0], tt[1]), zero4()) : mfma16(xb[0], tt[0], zero4());
        // lane (g, n): T_g[16 AB + n][16 CB + 4 g + e]
        const f32x4 bc = lds_f32x4(bes + 16 * CB + 4 * g4);
        sts4(M1s + cc_off<CH>(16 * AB + r16, 16 * CB + 4 * g4), -acc * bc);
    }

    // smem: the workgroup's LDS (Lay::bytes); blk, nblk: this workgroup's index within the
    // grid of workgroups that run this instance, and that grid's size
    __device__ static void run(const ChunkArgs &args, unsigned char *smem, int blk, int nblk) {
        constexpr int VPRQ = DK / 8;              // 16-byte vectors per q/k row
        constexpr int VPRV = kDVT / 8;
        constexpr int NVQ = CH * VPRQ / kRoleThreads;
        constexpr int NVV = CH * VPRV / kRoleThreads;
        constexpr int RJV = kRoleThreads / VPRV;
        static_assert(CH * VPRQ % kRoleThreads == 0 && CH * VPRV % kRoleThreads == 0, "whole vectors per thread");

        uint16_t *const base = reinterpret_cast<uint16_t *>(smem);
        uint16_t *const M1s = base + Lay::oM1;
        uint16_t *const Lgs = base + Lay::oLg;
        uint16_t *const Tds = base + Lay::oTd;
        uint16_t *const Os = base + Lay::oO;
        float *const gbase = reinterpret_cast<float *>(smem + Lay::oGate);
        auto Qb = [&](int s) { return base + Lay::oQ + s * Lay::NQ; };
        auto Kb = [&](int s) { return base + Lay::oK + s * Lay::NQ; };
        auto Vb = [&](int s) { return base + Lay::oV + s * Lay::NV; };
        auto Ab = [&](int s) { return base + Lay::oA + s * Lay::NCC; };
        auto gate = [&](int s, int which) { return gbase + (s * Lay::kGates + which) * CH; };

        const int tid = threadIdx.x;
        const int lane = lane_id();
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
        const bool is_scan = wave < 4;
        const int rw = wave & 3;                  // wave index within its role
        const int rt = tid & (kRoleThreads - 1);  // thread index within its role
        const int r16 = lane & 15;
        const int g4 = lane >> 4;

        int logical = blk;
        if (args.n_dvt > 1 && (nblk & 7) == 0) logical = (blk & 7) * (nblk >> 3) + (blk >> 3);
        const int dvt = logical % args.n_dvt;
        const int bh = logical / args.n_dvt;
        const int b = bh / args.H;
        const int h = bh % args.H;
        const int T = args.T, H = args.H, dv = args.dv;
        const int dv0 = dvt * kDVT;
        // rows of the sequence the chunks walk (2T for the interleaved sequence), and tokens
        // of memory per chunk
        const int TS = EDA ? 2 * T : T;
        constexpr int TPC = EDA ? CH / 2 : CH;
        const int NC = (TS + CH - 1) / CH;
        auto chunk_len = [&](int c) { return min(CH, TS - c * CH); };
        auto chunk_tok = [&](int c) { return EDA ? chunk_len(c) / 2 : chunk_len(c); };

        // token 0 of this (batch, head); consecutive tokens are H rows apart
        const size_t tok0 = static_cast<size_t>(b) * T * H + h;
        const uint16_t *const qbase = static_cast<const uint16_t *>(args.q) + tok0 * DK;
        const uint16_t *const kbase = static_cast<const uint16_t *>(args.k) + tok0 * DK;
        // key rows of this wave's staging: the erase directions for the even rows of EDA
        const bool erase_rows = EDA && (rw & 1) == 0;
        const uint16_t *const krows = erase_rows ? static_cast<const uint16_t *>(args.e) + tok0 * DK : kbase;
        // v == null reads as zeros and o == null drops the output (state-only passes of the
        // segmented schedule): their buffer resources get an empty range, so no branch is
        // needed in the loop and no address is formed from a null pointer
        const bool has_v = args.v != nullptr, has_o = args.o != nullptr;
        const uint16_t *const vbase =
            static_cast<const uint16_t *>(has_v ? args.v : args.q) + (has_v ? tok0 * dv + dv0 : 0);
        uint16_t *const obase = has_o ? static_cast<uint16_t *>(args.o) + tok0 * dv + dv0
                                      : static_cast<uint16_t *>(const_cast<void *>(args.q));
        const int rowQ = H * DK * 2, rowV = H * dv * 2, rowG = H * 4;   // bytes between tokens

        // ---- scan role: S^T slice; sT[2u + hh][e] holds key 8 kq(g, u) + 4hh + e of column 16w + l%16
        f32x4 sT[NKT];
        const size_t srow = ((static_cast<size_t>(b) * H + h) * dv + dv0 + 16 * rw + r16) * DK;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            sT[t] = (is_scan && args.S0)
                        ? *reinterpret_cast<const f32x4 *>(args.S0 + srow + 8 * kq(g4, t >> 1) + 4 * (t & 1))
                        : zero4();

        // ---- scan-role prefetch of chunk n + 2: registers, per-lane offsets fixed per chunk.
        // q / k: one wave instruction reads 16 / NKP whole rows; the 16 lanes of a group read
        // four consecutive rows at the four key quads of one fragment step (lane 16G + 4i + g:
        // row 4 (G / NKP) + i, quad kq(g, G % NKP)), so their fragment slots fall on distinct banks.
        // EDA: instruction m = 4j + rw covers rows of parity m & 1 (= rw & 1), 16 / NKP of
        // them two apart; row r is token r / 2 of the chunk.
        const int vv_row = rt / VPRV, vv_col = rt % VPRV;
        int voffQ[NVQ], ldsQ[NVQ], voffV[NVV];
#pragma unroll
        for (int j = 0; j < NVQ; ++j) {
            const int m = 4 * j + rw, loc = 4 * (g4 / NKP) + (r16 >> 2);
            const int row = EDA ? 2 * (16 / NKP) * (m >> 1) + 2 * loc + (m & 1) : m * (16 / NKP) + loc;
            const int u = g4 % NKP, g = r16 & 3;
            voffQ[j] = (EDA ? row >> 1 : row) * rowQ + 16 * kq(g, u);
            ldsQ[j] = qk_off(row >> 4, u, g, row & 15);
        }
        // an offset past every buffer range: loads of it read zeros, stores to it are dropped
        constexpr int kNoRow = 0x7ffffff0;
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int row = vv_row + j * RJV;
            voffV[j] = !EDA ? row * rowV + vv_col * 16 : (row & 1) ? (row >> 1) * rowV + vv_col * 16 : kNoRow;
        }
        const int voffG = (rt & (kWave - 1)) * rowG;
        const int ldsV = vv_row * PV + vv_col * 8;        // + j * RJV * PV

        // Staging of a chunk c into LDS slot c & 1, in two parts with their own registers.
        // q and v: loaded in I1 and written in I2 (the scan reads chunk n's V only in I1 and
        // its Q not at all: its Q S^T is formed a step ahead); k and the gates: loaded in I2
        // and written in I4, once the state update has read chunk n's K and the gate tables.
        struct PrefQV {
            u32x4 q[NVQ], v[NVV];
        };
        struct PrefK {
            u32x4 k[NVQ];
            float a, b, l;
        };
        auto gload_qv = [&](int c, PrefQV &pf) {
            const int clen = chunk_tok(c);
            const size_t t0 = static_cast<size_t>(c) * TPC * H;
            const auto rsq = buffer_rsrc(qbase + t0 * DK, (clen - 1) * rowQ + DK * 2);
            const auto rsv = buffer_rsrc(vbase + (has_v ? t0 * dv : 0), has_v ? (clen - 1) * rowV + kDVT * 2 : 0);
#pragma unroll
            for (int j = 0; j < NVQ; ++j)
                if (!erase_rows) pf.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rsq, voffQ[j], 0, 0);
#pragma unroll
            for (int j = 0; j < NVV; ++j) pf.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rsv, voffV[j], 0, 0);
        };
        auto gload_k = [&](int c, PrefK &pf) {
            const int clen = chunk_tok(c);
            const size_t t0 = static_cast<size_t>(c) * TPC * H;
            const auto rsk = buffer_rsrc(krows + t0 * DK, (clen - 1) * rowQ + DK * 2);
#pragma unroll
            for (int j = 0; j < NVQ; ++j) pf.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rsk, voffQ[j], 0, 0);
            const int gbytes = (clen - 1) * rowG + 4;
            pf.a = 1.f;
            pf.l = 0.f;
            if constexpr (HAS_A)
                pf.a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(args.alpha + tok0 + t0, gbytes), voffG, 0, 0));
            pf.b = 1.f;
            if constexpr (!EDA)
                pf.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(args.beta + tok0 + t0, gbytes), voffG, 0, 0));
            if constexpr (HAS_L)
                pf.l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(args.lam + tok0 + t0, gbytes), voffG, 0, 0));
        };
        auto rstore_qv = [&](int c, const PrefQV &pf) {
            const int s = c & 1;
            uint16_t *Qs = Qb(s), *Vs = Vb(s);
#pragma unroll
            for (int j = 0; j < NVQ; ++j) {
                if (!erase_rows) *reinterpret_cast<u32x4 *>(Qs + ldsQ[j]) = pf.q[j];
            }
#pragma unroll
            for (int j = 0; j < NVV; ++j) *reinterpret_cast<u32x4 *>(Vs + ldsV + j * RJV * PV) = pf.v[j];
        };
        auto rstore_k = [&](int c, const PrefK &pf) {
            const int s = c & 1;
            uint16_t *Ks = Kb(s);
#pragma unroll
            for (int j = 0; j < NVQ; ++j) {
                *reinterpret_cast<u32x4 *>(Ks + ldsQ[j]) = pf.k[j];
            }
            // gates of the chunk, lane = position; every scan wave holds them and writes part
            // of the tables (wave 0: g and beta, 1: exp(g), 2: exp(g_last - g), 3: lambda)
            {
                const bool ok = lane < chunk_len(c);
                if (rw <= 2) {
                    const float la = RAW ? log_decay_from_logit(pf.a) : __logf(pf.a);
                    const float x = wave_inclusive_sum((HAS_A && ok) ? la : 0.f);
                    if (lane < CH) {
                        if (rw == 0) {
                            gate(s, 0)[lane] = x;
                            gate(s, 3)[lane] = ok ? (RAW ? sigmoid_f(pf.b) : pf.b) : 0.f;
                        } else if (rw == 1) {
                            gate(s, 1)[lane] = __expf(x);
                        } else {
                            const float glast =
                                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), CH - 1));
                            gate(s, 2)[lane] = __expf(glast - x);
                        }
                    }
                } else if (lane < CH) {
                    gate(s, 4)[lane] = ok ? ((RAW && HAS_L) ? sigmoid_f(pf.l) : pf.l) : 0.f;
                }
            }
        };

        // A (both slots) and M1 start zeroed: the upper 16x16 block of each 32-wide diagonal
        // pair is read by the scan's paired products and must hold zeros
        for (int i = tid; i < 3 * Lay::NCC / 8; i += kPipeThreads)
            reinterpret_cast<u32x4 *>(base + Lay::oA)[i] = u32x4{0, 0, 0, 0};
        if constexpr (EDA)                        // query rows of the erase tokens, both slots
            for (int i = tid; i < 2 * Lay::NQ / 8; i += kPipeThreads)
                reinterpret_cast<u32x4 *>(base + Lay::oQ)[i] = u32x4{0, 0, 0, 0};

        if (NC == 0) {
            if (is_scan && args.S_T) {
#pragma unroll
                for (int t = 0; t < NKT; ++t)
                    *reinterpret_cast<f32x4 *>(args.S_T + srow + 8 * kq(g4, t >> 1) + 4 * (t & 1)) = sT[t];
            }
            return;
        }

        if (is_scan) {
            PrefQV pq0;
            PrefK pk0;
            gload_qv(0, pq0);
            gload_k(0, pk0);
            rstore_qv(0, pq0);
            rstore_k(0, pk0);
        }
        __syncthreads();

        // The two roles run separate loops with the same four barriers per step, so each
        // role's registers are allocated for its own code: the scan's state and look-ahead
        // products are not live through the prep's code, nor the prep's through the scan's.
        if (is_scan) {
            // K S^T and Q S^T of the chunk the next step's I1 processes, formed in I2 and I3
            // as the key tiles of that chunk's entry state become final
            f32x4 PK_[NCT], PQ[NCT];
            for (int n = -1; n < NC; ++n) {
                const int c = n + 1;              // the chunk whose S^T products are formed ahead
                const int ss = n & 1;             // slot of chunk n
                const int ps = c & 1;             // slot of chunk c
                const int tri = r16 >> 2, trp = r16 & 3;
                PrefQV pfqv;                      // q, v of chunk n + 2, loaded in I1, staged in I2
                PrefK pfk;                        // k and gates of chunk n + 2, loaded in I2, staged in I4
                bf16x4 Zd[NCT];                   // exp(g_last - g) Z, from I1 to I2/I3

                // S^T <- exp(g_last) S^T + K^T diag(exp(g_last - g)) Z for key tiles [t_lo, t_hi).
                // Output row m of tile 2u + hh is key 8 kq(m/4, u) + 4hh + m%4, read from K with
                // the transpose read: lane (g, 4i + p) reads keys 8 kq(p, u) + 4hh.. of position
                // 32s + 4g + i (and + 16), matching the pairing of Zd[2s], Zd[2s + 1].
                auto state_update = [&](int t_lo, int t_hi) {
                    const uint16_t *Ks = Kb(ss);
                    const float dlast = HAS_A ? gate(ss, 1)[CH - 1] : 1.f;
                    bf16x8 zp[NCP];
    #pragma unroll
                    for (int s = 0; s < NCP; ++s) zp[s] = cat8(Zd[2 * s], Zd[2 * s + 1]);
                    bf16x8 kf[2][NCP];
                    auto load = [&](int t, bf16x8(&dst)[NCP]) {
                        // keys 8 kq(trp, t / 2) + 4 (t & 1) .. + 3 of positions 32 s + 4 g4 + tri
                        // and 16 later: slot (trp, 4 g4 + tri) of blocks (2 s, t / 2), (2 s + 1, t / 2)
    #pragma unroll
                        for (int s = 0; s < NCP; ++s) {
                            const uint16_t *p = Ks + qk_off(2 * s, t >> 1, trp, 4 * g4 + tri) + 4 * (t & 1);
                            dst[s] = cat8(lds_tr(p), lds_tr(p + NKP * 512));
                        }
                    };
                    load(t_lo, kf[0]);
    #pragma unroll
                    for (int t = 0; t < NKT; ++t) {
                        if (t < t_lo || t >= t_hi) continue;
                        if (t + 1 < t_hi) load(t + 1, kf[(t + 1 - t_lo) & 1]);
                        __builtin_amdgcn_sched_barrier(0);
                        f32x4 acc = sT[t] * dlast;
    #pragma unroll
                        for (int s = 0; s < NCP; ++s) acc = mfma32(kf[(t - t_lo) & 1][s], zp[s], acc);
                        sT[t] = acc;
                        __builtin_amdgcn_sched_barrier(0);
                    }
                };

                // K S^T and Q S^T of chunk c (slot ps) over the key pairs [u_lo, u_hi), from the
                // state tiles the update has just made final (its entry state); the contraction
                // runs over the pairs in order, so the sums are those of one pass over the keys
                auto lookahead = [&](int u_lo, int u_hi) {
                    const uint16_t *Qn = Qb(ps), *Kn = Kb(ps);
    #pragma unroll
                    for (int u = 0; u < NKP; ++u) {
                        if (u < u_lo || u >= u_hi) continue;
                        const bf16x8 sf = cat8(Bf16::cvt(sT[2 * u]), Bf16::cvt(sT[2 * u + 1]));
                        bf16x8 fk[NCT], fq[NCT];
    #pragma unroll
                        for (int mt = 0; mt < NCT; ++mt) {
                            const int off = qk_off(mt, u, g4, r16);
                            fk[mt] = lds8(Kn + off);
                            if (!STATES || HAS_L) fq[mt] = lds8(Qn + off);
                        }
                        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                        for (int mt = 0; mt < NCT; ++mt) {
                            PK_[mt] = mfma32(fk[mt], sf, PK_[mt]);
                            if (!STATES || HAS_L) PQ[mt] = mfma32(fq[mt], sf, PQ[mt]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                };

                // STATES: the entry state of chunk c (the exit state of chunk n), rounded to bf16,
                // key pairs [u_lo, u_hi): tiles 2u and 2u + 1 hold the eight consecutive keys
                // 8 kq(g, u) .. + 7 of the lane's state row, one 16-byte store, so each store
                // instruction writes 64 contiguous bytes of each of 16 rows
                auto store_entry = [&](int u_lo, int u_hi) {
                    uint16_t *hs = static_cast<uint16_t *>(args.Hs) +
                                   ((static_cast<size_t>(bh) * NC + c) * dv + dv0 + 16 * rw + r16) * DK;
    #pragma unroll
                    for (int u = 0; u < NKP; ++u) {
                        if (u < u_lo || u >= u_hi) continue;
                        *reinterpret_cast<bf16x8 *>(hs + 8 * kq(g4, u)) = cat8(Bf16::cvt(sT[2 * u]), Bf16::cvt(sT[2 * u + 1]));
                    }
                };

                // ======================================================== I1
                if (n + 2 < NC) gload_qv(n + 2, pfqv);   // slot n & 1: its Q is no longer read
                if (n >= 0) {
                    const uint16_t *Vs = Vb(ss), *As = Ab(ss);
                    const float *lam_s = gate(ss, 4), *eg = gate(ss, 1), *egl = gate(ss, 2);
                    // RAW: 1/|q| and 1/|k| of the chunk's positions (the look-ahead products
                    // were formed from the raw q and k)
                    const float *nq = RAW ? gate(ss, 5) : nullptr, *nk = RAW ? gate(ss, 6) : nullptr;
                    // operands of Z: V as the paired B operand (positions 32u + 4g + i and
                    // 32u + 16 + 4g + i) and the M1 fragments
                    bf16x8 Vf[NCP], m1f[NCT][NCP];
#pragma unroll
                    for (int u = 0; u < NCP; ++u) {
                        const uint16_t *p = Vs + (32 * u + 4 * g4 + tri) * PV + 16 * rw + 4 * trp;
                        Vf[u] = cat8(lds_tr(p), lds_tr(p + 16 * PV));
                    }
#pragma unroll
                    for (int m = 0; m < NCT; ++m)
#pragma unroll
                        for (int u = 0; u <= (m >> 1); ++u)
                            m1f[m][u] = lds8(M1s + (m * NCP + u) * 512 + 8 * frag_slot(g4, r16));
                    // Yg = -D_g (K S^T + diag(lambda) Q S^T); the A fragments of O are issued here
                    bf16x8 af[NCT][NCP];
                    if constexpr (!STATES) {
#pragma unroll
                        for (int m = 0; m < NCT; ++m)
#pragma unroll
                            for (int u = 0; u <= (m >> 1); ++u)
                                af[m][u] = lds8(As + (m * NCP + u) * 512 + 8 * frag_slot(g4, r16));
                    }
                    bf16x4 Yg[NCT];
#pragma unroll
                    for (int mt = 0; mt < NCT; ++mt) {
                        f32x4 y = PK_[mt];
                        if constexpr (RAW) y *= lds_f32x4(nk + 16 * mt + 4 * g4);
                        if constexpr (HAS_L && RAW)
                            y += (lds_f32x4(lam_s + 16 * mt + 4 * g4) * lds_f32x4(nq + 16 * mt + 4 * g4)) * PQ[mt];
                        else if constexpr (HAS_L)
                            y += lds_f32x4(lam_s + 16 * mt + 4 * g4) * PQ[mt];
                        if constexpr (HAS_A) y *= lds_f32x4(eg + 16 * mt + 4 * g4);
                        Yg[mt] = Bf16::cvt(-y);
                    }
                    // Z = M1 V + M1 Yg (both products share the M1 fragment)
                    f32x4 Z[NCT];
#pragma unroll
                    for (int mt = 0; mt < NCT; ++mt) {
                        f32x4 z = zero4();
#pragma unroll
                        for (int u = 0; u <= (mt >> 1); ++u) {
                            z = mfma32(m1f[mt][u], Vf[u], z);
                            z = mfma32(m1f[mt][u], cat8(Yg[2 * u], Yg[2 * u + 1]), z);
                        }
                        Z[mt] = z;
                    }
                    bf16x4 Zf[NCT];
#pragma unroll
                    for (int mt = 0; mt < NCT; ++mt) {
                        Zf[mt] = Bf16::cvt(Z[mt]);
                        if constexpr (RAW) {
                            const f32x4 d = lds_f32x4(nk + 16 * mt + 4 * g4);
                            Zd[mt] = Bf16::cvt((HAS_A ? lds_f32x4(egl + 16 * mt + 4 * g4) * d : d) * Z[mt]);
                        } else {
                            Zd[mt] = HAS_A ? Bf16::cvt(lds_f32x4(egl + 16 * mt + 4 * g4) * Z[mt]) : Zf[mt];
                        }
                    }
                    // O = D_g Q S^T + A Z, staged for the row stores of I4
                    if constexpr (!STATES) {
#pragma unroll
                        for (int mt = 0; mt < NCT; ++mt) {
                            f32x4 o = HAS_A ? lds_f32x4(eg + 16 * mt + 4 * g4) * PQ[mt] : PQ[mt];
                            if constexpr (RAW) o *= lds_f32x4(nq + 16 * mt + 4 * g4);
#pragma unroll
                            for (int u = 0; u <= (mt >> 1); ++u) o = mfma32(af[mt][u], cat8(Zf[2 * u], Zf[2 * u + 1]), o);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                Os[(16 * mt + 4 * g4 + e) * PV + 16 * rw + r16] = Bf16::from_f32(o[e]);
                        }
                    } else {
                        // without the output, I1 is short on the scan side: the first quarter
                        // of the state update moves here from I2
                        state_update(0, NKT / 4);
                    }
                }
                __syncthreads();

                // ======================================================== I2
                if (n + 2 < NC) rstore_qv(n + 2, pfqv);  // V of chunk n was read in I1
                if (n + 2 < NC) gload_k(n + 2, pfk);
                if (n >= 0) state_update(STATES ? NKT / 4 : 0, NKT / 2);
                if (c < NC) {
#pragma unroll
                    for (int mt = 0; mt < NCT; ++mt) PK_[mt] = PQ[mt] = zero4();
                    lookahead(0, NKP / 2);
                }
                __syncthreads();

                // ======================================================== I3
                // (the key tiles of the first half became final in I2; the stores of the entry
                // state go to I3 and I4, where the scan has less to do than the prep)
                if (STATES && args.Hs && c < NC) store_entry(0, NKP / 2);
                if (n >= 0) state_update(NKT / 2, NKT);
                if (c < NC) lookahead(NKP / 2, NKP);
                __syncthreads();

                // ======================================================== I4
                if (n + 2 < NC) rstore_k(n + 2, pfk);    // K and gates of chunk n were read up to I3
                if (STATES && args.Hs && c < NC) store_entry(NKP / 2, NKP);
                if (!STATES && n >= 0) {
                    const auto rso = buffer_rsrc(obase + (has_o ? static_cast<size_t>(n) * TPC * H * dv : 0),
                                                 has_o ? (chunk_tok(n) - 1) * rowV + kDVT * 2 : 0);
#pragma unroll
                    for (int j = 0; j < NVV; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4 *>(Os + ldsV + j * RJV * PV),
                                                               rso, voffV[j], 0, 0);
                }
                __syncthreads();
            }
            if (args.S_T) {
#pragma unroll
                for (int t = 0; t < NKT; ++t)
                    *reinterpret_cast<f32x4 *>(args.S_T + srow + 8 * kq(g4, t >> 1) + 4 * (t & 1)) = sT[t];
            }
        } else {
            for (int n = -1; n < NC; ++n) {
                const int c = n + 1;              // the prep role's chunk
                const int ps = c & 1;             // its slot
                const int tri = r16 >> 2, trp = r16 & 3;
                f32x4 tdiag;                      // the wave's diagonal block of T_g, I1 to I2
                // ======================================================== I1
                if (c < NC) {
                const uint16_t *Qs = Qb(ps), *Ks = Kb(ps);
                uint16_t *As = Ab(ps);
                const float *gs = gate(ps, 0), *bes = gate(ps, 3), *lams = gate(ps, 4);
                float *const nqs = RAW ? gate(ps, 5) : nullptr, *const nks = RAW ? gate(ps, 6) : nullptr;
                switch (rw) {
                    case 0: gram<0, 1>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                    case 1: gram<1, 1>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                    case 2: gram<2, 1>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                    default: gram<3, 1>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                }
                }
                __syncthreads();
                // ======================================================== I2
                if (c < NC) {
                if (rw < NCT) {                   // M1 of this wave's diagonal block
                    const int o = 16 * rw;
                    const float bc = gate(ps, 3)[o + r16];
#pragma unroll
                    for (int e = 0; e < 4; ++e) M1s[cc_off<CH>(o + 4 * g4 + e, o + r16)] = Bf16::from_f32(tdiag[e] * bc);
                }
                {
                    const uint16_t *Qs = Qb(ps), *Ks = Kb(ps);
                    uint16_t *As = Ab(ps);
                    const float *gs = gate(ps, 0), *bes = gate(ps, 3), *lams = gate(ps, 4);
                    float *const nqs = RAW ? gate(ps, 5) : nullptr, *const nks = RAW ? gate(ps, 6) : nullptr;
                    switch (rw) {
                        case 0: gram<0, 2>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                        case 1: gram<1, 2>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                        case 2: gram<2, 2>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                        default: gram<3, 2>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag); break;
                    }
                }
                }
                __syncthreads();
                // ======================================================== I3
                if (c < NC && rw < 2) {
                    const uint16_t *Qs = Qb(ps), *Ks = Kb(ps);
                    uint16_t *As = Ab(ps);
                    const float *gs = gate(ps, 0), *bes = gate(ps, 3), *lams = gate(ps, 4);
                    float *const nqs = RAW ? gate(ps, 5) : nullptr, *const nks = RAW ? gate(ps, 6) : nullptr;
                    if (rw == 0) gram<0, 3>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag);
                    else gram<1, 3>(Qs, Ks, As, Lgs, Tds, gs, bes, lams, nqs, nks, r16, g4, tdiag);
                }
                if (c < NC && rw >= 2 && rw - 2 < NCT / 2) {
                    // block doubling, level 1: T_g[2a+1][2a] = -T_g[2a+1][2a+1] L_g[2a+1][2a] T_g[2a][2a]
                    const int aa = 2 * (rw - 2), bb = aa + 1;
                    const f32x4 x = mfma16(lds4(Lgs + (16 * bb + r16) * PC + 16 * aa + 4 * g4),
                                           lds4(Tds + (16 * aa + r16) * PC + 16 * aa + 4 * g4), zero4());
                    const f32x4 y = mfma16(lds_tr(Tds + (16 * bb + 4 * g4 + tri) * PC + 16 * bb + 4 * trp), Bf16::cvt(x),
                                           zero4());
                    if constexpr (NCT == 4) sts4(Tds + (16 * aa + r16) * PC + 16 * bb + 4 * g4, -y);
                    const float bc = gate(ps, 3)[16 * aa + r16];
#pragma unroll
                    for (int e = 0; e < 4; ++e) M1s[cc_off<CH>(16 * bb + 4 * g4 + e, 16 * aa + r16)] = Bf16::from_f32(-y[e] * bc);
                }
                __syncthreads();
                // ======================================================== I4
                if constexpr (NCT == 4) {
                    if (c < NC) {
                    switch (rw) {
                        case 0: level2<2, 0>(Lgs, Tds, M1s, gate(ps, 3), lane); break;
                        case 1: level2<2, 1>(Lgs, Tds, M1s, gate(ps, 3), lane); break;
                        case 2: level2<3, 0>(Lgs, Tds, M1s, gate(ps, 3), lane); break;
                        default: level2<3, 1>(Lgs, Tds, M1s, gate(ps, 3), lane); break;
                    }
                    }
                }
                __syncthreads();
            }
        }
    }
};

template <int DK, int CH, bool HAS_A, bool HAS_L, bool RAW>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_kernel(const ChunkArgs args) {
    using K = PipeKernel<DK, CH, HAS_A, HAS_L, RAW>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::Lay::bytes];
    K::run(args, smem, blockIdx.x, gridDim.x);
}

template <int DK, int CH, bool HAS_A, bool HAS_L>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_states_kernel(const ChunkArgs args) {
    using K = PipeKernel<DK, CH, HAS_A, HAS_L, false, true>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::Lay::bytes];
    K::run(args, smem, blockIdx.x, gridDim.x);
}

template <int DK, int CH>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_eda_kernel(const ChunkArgs args) {
    using K = PipeKernel<DK, CH, false, false, false, false, true>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::Lay::bytes];
    K::run(args, smem, blockIdx.x, gridDim.x);
}

// c ? x : y, field by field (a reference picked among kernel arguments would make the
// compiler copy the arguments to scratch memory)
__device__ __forceinline__ ChunkArgs pick_args(bool c, const ChunkArgs &x, const ChunkArgs &y) {
    ChunkArgs r;
    r.q = c ? x.q : y.q;
    r.k = c ? x.k : y.k;
    r.v = c ? x.v : y.v;
    r.alpha = c ? x.alpha : y.alpha;
    r.beta = c ? x.beta : y.beta;
    r.lam = c ? x.lam : y.lam;
    r.S0 = c ? x.S0 : y.S0;
    r.o = c ? x.o : y.o;
    r.S_T = c ? x.S_T : y.S_T;
    r.B = c ? x.B : y.B;
    r.T = c ? x.T : y.T;
    r.H = c ? x.H : y.H;
    r.dv = c ? x.dv : y.dv;
    r.n_dvt = c ? x.n_dvt : y.n_dvt;
    r.raw = c ? x.raw : y.raw;
    r.Hs = c ? x.Hs : y.Hs;
    r.e = c ? x.e : y.e;
    return r;
}

// The segmented schedule's first launch for a single sequence: workgroups [0, n0) walk the
// first segment with its output from the caller's entry state (a0); the rest run the
// state-only instance over the other segments, the transition maps (am) and then the
// exit states from zero (ag).  The first segment's workgroups have the lowest indices, so
// they are dispatched first and its walk, the longest, starts at once; the state-only
// walks fill the other compute units.  Raw inputs have no state-only instance: their
// state-only walks run the raw instance with the output dropped.
template <int DK, int CH, bool HAS_A, bool HAS_L, bool RAW>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_overlap_kernel(const ChunkArgs a0, const ChunkArgs am,
                                                                                  const ChunkArgs ag, int n0, int nm) {
    using K0 = PipeKernel<DK, CH, HAS_A, HAS_L, RAW>;
    using KS = typename std::conditional<RAW, K0, PipeKernel<DK, CH, HAS_A, HAS_L, false, true>>::type;
    static_assert(static_cast<int>(K0::Lay::bytes) == static_cast<int>(KS::Lay::bytes), "one LDS layout for both instances");
    __shared__ __attribute__((aligned(16))) unsigned char smem[K0::Lay::bytes];
    // each instance's body appears once in the kernel, so the workgroups of the state-only
    // walks (and, for raw inputs, all of them) run the same code: the arguments are picked
    // by the workgroup's range instead
    const int bid = blockIdx.x, ng = static_cast<int>(gridDim.x) - n0 - nm;
    const bool walk_g = bid >= n0 + nm;
    const ChunkArgs as = pick_args(walk_g, ag, am);
    const int bs = walk_g ? bid - n0 - nm : bid - n0, ns = walk_g ? ng : nm;
    if constexpr (RAW) {
        const bool first = bid < n0;
        K0::run(pick_args(first, a0, as), smem, first ? bid : bs, first ? n0 : ns);
    } else {
        if (bid < n0) K0::run(a0, smem, bid, n0);
        else KS::run(as, smem, bs, ns);
    }
}

template <int DK, int CH>
hipError_t launch_pipe_overlap(const ChunkArgs &a0, const ChunkArgs &am, const ChunkArgs &ag, hipStream_t stream) {
    const int n0 = a0.B * a0.H * a0.n_dvt, nm = am.B * am.H * am.n_dvt, ng = ag.B * ag.H * ag.n_dvt;
    if (n0 + nm + ng == 0) return hipSuccess;
    const bool ha = a0.alpha != nullptr, hl = a0.lam != nullptr;
    const dim3 grid(n0 + nm + ng), blk(kPipeThreads);
    if (a0.raw) {
        if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, true, true, true>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, true, false, true>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, false, true, true>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, false, false, true>), grid, blk, 0, stream, a0, am, ag, n0, nm);
    } else {
        if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, true, true, false>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, true, false, false>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, false, true, false>), grid, blk, 0, stream, a0, am, ag, n0, nm);
        else hipLaunchKernelGGL((chunk_fwd_pipe_overlap_kernel<DK, CH, false, false, false>), grid, blk, 0, stream, a0, am, ag, n0, nm);
    }
    return hipGetLastError();
}

template <int DK, int CH>
hipError_t launch_pipe_eda(const ChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_fwd_pipe_eda_kernel<DK, CH>), dim3(grid), dim3(kPipeThreads), 0, stream, a);
    return hipGetLastError();
}

template <int DK, int CH>
hipError_t launch_pipe_states(const ChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    const dim3 blk(kPipeThreads);
    if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_states_kernel<DK, CH, true, true>), dim3(grid), blk, 0, stream, a);
    else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_states_kernel<DK, CH, true, false>), dim3(grid), blk, 0, stream, a);
    else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_states_kernel<DK, CH, false, true>), dim3(grid), blk, 0, stream, a);
    else hipLaunchKernelGGL((chunk_fwd_pipe_states_kernel<DK, CH, false, false>), dim3(grid), blk, 0, stream, a);
    return hipGetLastError();
}

template <int DK, int CH>
hipError_t launch_pipe_typed(const ChunkArgs &a, hipStream_t stream) {
    const int grid = a.B * a.H * a.n_dvt;
    if (grid == 0) return hipSuccess;
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    const dim3 blk(kPipeThreads);
    if (a.raw) {
        if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, true, true>), dim3(grid), blk, 0, stream, a);
        else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, false, true>), dim3(grid), blk, 0, stream, a);
        else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, true, true>), dim3(grid), blk, 0, stream, a);
        else hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, false, true>), dim3(grid), blk, 0, stream, a);
    } else {
        if (ha && hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, true, false>), dim3(grid), blk, 0, stream, a);
        else if (ha) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, true, false, false>), dim3(grid), blk, 0, stream, a);
        else if (hl) hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, true, false>), dim3(grid), blk, 0, stream, a);
        else hipLaunchKernelGGL((chunk_fwd_pipe_kernel<DK, CH, false, false, false>), dim3(grid), blk, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_pipe_eda(int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    if (dk == 128) return C == 64 ? launch_pipe_eda<128, 64>(a, stream) : launch_pipe_eda<128, 32>(a, stream);
    return C == 64 ? launch_pipe_eda<64, 64>(a, stream) : launch_pipe_eda<64, 32>(a, stream);
}

hipError_t launch_chunk_fwd_pipe_overlap(int dk, int C, const ChunkArgs &a0, const ChunkArgs &am, const ChunkArgs &ag,
                                        hipStream_t stream) {
    if (dk == 128) return C == 64 ? launch_pipe_overlap<128, 64>(a0, am, ag, stream) : launch_pipe_overlap<128, 32>(a0, am, ag, stream);
    return C == 64 ? launch_pipe_overlap<64, 64>(a0, am, ag, stream) : launch_pipe_overlap<64, 32>(a0, am, ag, stream);
}

hipError_t launch_chunk_fwd_pipe_states(int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    if (dk == 128) return C == 64 ? launch_pipe_states<128, 64>(a, stream) : launch_pipe_states<128, 32>(a, stream);
    return C == 64 ? launch_pipe_states<64, 64>(a, stream) : launch_pipe_states<64, 32>(a, stream);
}

hipError_t launch_chunk_fwd_pipe(int dk, int C, const ChunkArgs &a, hipStream_t stream) {
    // no output wanted (the state-only passes of the segmented schedule): the instance
    // that forms nothing of O, with no entry states kept when a.Hs is null
    if (!a.raw && a.o == nullptr) return launch_chunk_fwd_pipe_states(dk, C, a, stream);
    if (dk == 128) {
        switch (C) {
            case 32: return launch_pipe_typed<128, 32>(a, stream);
            case 64: return launch_pipe_typed<128, 64>(a, stream);
        }
    } else if (dk == 64) {
        switch (C) {
            case 32: return launch_pipe_typed<64, 32>(a, stream);
            case 64: return launch_pipe_typed<64, 64>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace qd
