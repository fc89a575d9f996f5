// Device-side building blocks for the gfx950 Q-Delta kernels.
//
// Fragment convention (one 64-lane wavefront, MFMA 16x16 tiles):
//   A "fragment" of a 16 x 16 block M (rows m, contraction index k) gives lane l
//   the four values M[l % 16][4 * (l / 16) + i], i = 0..3.
//   A "B-fragment" of a 16 x 16 block N (k x n) gives lane l the four values
//   N[4 * (l / 16) + i][l % 16].
//   The MFMA accumulator of a 16 x 16 output D gives lane l D[4 * (l / 16) + i][l % 16].
// So an accumulator tile is, without moving data, the B-fragment of D (k = row)
// and the A-fragment of D^T.  The kernels chain products through registers this
// way.  A 16x16x32 bf16 MFMA consumes two 16-wide contraction slices at once: its
// A and B operands are the concatenation of the two slices' fragments, in the same
// order for both, so the pairing of contraction indices is consistent whatever
// order the instruction assigns internally.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// ---------------------------------------------------------------- element policies
// Raw storage type R in memory and LDS, fragment type F fed to the MFMA.
struct Bf16 {
    using R = uint16_t;
    using F = bf16x4;
    static constexpr int kBytes = 2;

    __device__ __forceinline__ static float to_f32(R x) {
        return __uint_as_float(static_cast<uint32_t>(x) << 16);
    }
    __device__ __forceinline__ static R from_f32(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
    __device__ __forceinline__ static F cvt(f32x4 a) { return __builtin_convertvector(a, bf16x4); }
    __device__ __forceinline__ static f32x4 f32(F a) { return __builtin_convertvector(a, f32x4); }
    __device__ __forceinline__ static F ld4(const R *p) {      // 4 consecutive elements
        return __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(p));
    }
    __device__ __forceinline__ static F ld4_strided(const R *p, int stride) {
        uint16_t a = p[0], b = p[stride], c = p[2 * stride], d = p[3 * stride];
        uint2 u;
        u.x = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
        u.y = static_cast<uint32_t>(c) | (static_cast<uint32_t>(d) << 16);
        return __builtin_bit_cast(bf16x4, u);
    }
    __device__ __forceinline__ static void st4(R *p, f32x4 a) {
        *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, cvt(a));
    }
    // 8 consecutive elements (p 16-byte aligned) as two halves, one 16-byte access
    __device__ __forceinline__ static void ld8(const R *p, F &lo, F &hi) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        lo = __builtin_bit_cast(bf16x4, make_uint2(u.x, u.y));
        hi = __builtin_bit_cast(bf16x4, make_uint2(u.z, u.w));
    }
    // acc += [A0 A1](16 x 32) [B0; B1](32 x 16)
    __device__ __forceinline__ static f32x4 mma2(f32x4 acc, F a0, F a1, F b0, F b1) {
        bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    // acc += A(16 x 16) B(16 x 16), issued as the same 16x16x32 instruction with a zero
    // second slice.  Every bf16 product uses one MFMA shape.  When one shape takes the
    // other's result as its accumulator, the compiler issues it right behind, with no wait
    // states.  On gfx950 the accumulator is forwarded only within a chain of one
    // instruction, so the later product reads a partly written accumulator and the sums
    // come out wrong.  Alternating the two shapes back to back on one accumulator gave
    // wrong values in every element; with 24 wait states after each product, the values
    // were right.
    __device__ __forceinline__ static f32x4 mma1(f32x4 acc, F a, F b) {
        const F z = {};
        return mma2(acc, a, z, b, z);
    }
};

struct F32 {
    using R = float;
    using F = f32x4;
    static constexpr int kBytes = 4;

    __device__ __forceinline__ static float to_f32(R x) { return x; }
    __device__ __forceinline__ static R from_f32(float x) { return x; }
    __device__ __forceinline__ static F cvt(f32x4 a) { return a; }
    __device__ __forceinline__ static f32x4 f32(F a) { return a; }
    __device__ __forceinline__ static F ld4(const R *p) { return *reinterpret_cast<const f32x4 *>(p); }
    __device__ __forceinline__ static F ld4_strided(const R *p, int stride) {
        f32x4 r;
        r[0] = p[0]; r[1] = p[stride]; r[2] = p[2 * stride]; r[3] = p[3 * stride];
        return r;
    }
    __device__ __forceinline__ static void st4(R *p, f32x4 a) { *reinterpret_cast<f32x4 *>(p) = a; }
    __device__ __forceinline__ static void ld8(const R *p, F &lo, F &hi) {
        lo = ld4(p);
        hi = ld4(p + 4);
    }
    __device__ __forceinline__ static f32x4 mma1(f32x4 acc, F a, F b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
    __device__ __forceinline__ static f32x4 mma2(f32x4 acc, F a0, F a1, F b0, F b1) {
        return mma1(mma1(acc, a0, b0), a1, b1);
    }
};

// ---------------------------------------------------------------- fragment loads
// A-fragment of the 16 x 16 block of a row-major matrix at (row0, col0):
// lane gets M[row0 + l%16][col0 + 4(l/16) .. +3].
template <class P>
__device__ __forceinline__ typename P::F frag(const typename P::R *m, int pitch, int row0, int col0) {
    const int l = lane_id();
    return P::ld4(m + (row0 + (l & 15)) * pitch + col0 + 4 * (l >> 4));
}

// The two halves of a lane's slice of a paired (32-position) product in octet order:
// lane l takes M[row0 + l%16][col0 + 8(l/16) .. +7], lo = +0..3 and hi = +4..7, in one
// 16-byte access.  Pairing frag at col0 and col0 + 16 gives lane group g the positions
// 4g..4g+3 and 16+4g..16+4g+3 instead; either order contracts the same 32 positions, as
// long as both operands of a product use it.  The element offset of each row start and
// col0 must keep 16-byte alignment.
template <class P>
__device__ __forceinline__ void frag_oct(const typename P::R *m, int pitch, int row0, int col0, typename P::F &lo,
                                         typename P::F &hi, int lane) {
    P::ld8(m + (row0 + (lane & 15)) * pitch + col0 + 8 * (lane >> 4), lo, hi);
}

// Fragment of the transpose of the block of a row-major matrix at (row0, col0),
// i.e. lane gets M[row0 + 4(l/16) + i][col0 + l%16], i = 0..3.  Used both as the
// A-fragment of M^T and as the B-fragment of M.
template <class P>
__device__ __forceinline__ typename P::F frag_t(const typename P::R *m, int pitch, int row0, int col0) {
    const int l = lane_id();
    return P::ld4_strided(m + (row0 + 4 * (l >> 4)) * pitch + col0 + (l & 15), pitch);
}

// B-fragment of the 16 x 16 block of a row-major matrix at (row0, col0), i.e. lane l
// gets M[row0 + 4(l/16) + i][col0 + l%16], i = 0..3 (equivalently the A-fragment of
// the block's transpose).  For bf16 this is one LDS transpose read per lane: within
// each group of 16 lanes the instruction hands lane 4p+q element q of the 8-byte
// chunks read by lanes 4i+p, so lane 4i+p of group g reads row 4g+i, columns
// 4p..4p+3.  For fp32 the four values are read one by one.
__device__ __forceinline__ Bf16::F frag_b_bf16(const uint16_t *m, int pitch, int row0, int col0) {
    const int l = lane_id();
    const int g = l >> 4, mm = l & 15;
    const uint16_t *p = m + (row0 + 4 * g + (mm >> 2)) * pitch + col0 + 4 * (mm & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

template <class P>
__device__ __forceinline__ typename P::F frag_b(const typename P::R *m, int pitch, int row0, int col0) {
    if constexpr (P::kBytes == 2) return frag_b_bf16(m, pitch, row0, col0);
    else return frag_t<P>(m, pitch, row0, col0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP row shifts and row
// broadcasts (no LDS round trips).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_src<0x111, 0xf>(x);   // row_shr:1
    x += dpp_src<0x112, 0xf>(x);   // row_shr:2
    x += dpp_src<0x114, 0xf>(x);   // row_shr:4
    x += dpp_src<0x118, 0xf>(x);   // row_shr:8
    x += dpp_src<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_src<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ f32x4 lds_f32x4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

}  // namespace qd
