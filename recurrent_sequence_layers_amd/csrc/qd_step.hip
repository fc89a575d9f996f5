// One recurrent Q-Delta decode step for gfx950 (Q-Delta reading notes §2.4):
//
//   x = k + lambda q
//   for every state row j (value index):
//     e_j  = v_j - alpha (s_j . x)
//     s_j <- alpha s_j + beta e_j k
//     o_j  = alpha (s_j . q) + beta e_j (k . q)      (read-out of the updated row)
//
// The step is bound by one read and one write of the fp32 state.  A workgroup of
// four waves owns one (sequence, head) state; eight lanes share a row, each
// holding d_k / 32 float4 column groups interleaved so that the eight lanes read
// 128 contiguous bytes per load.  Every row of the wave's share is loaded before
// any arithmetic (up to 16 float4 in flight per lane), the two dot products are
// reduced across the eight lanes, and the row is written back in place.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kStepThreads = 256;
constexpr int kLanesPerRow = 8;

__device__ __forceinline__ float group8_sum(float x) {
    x += __shfl_xor(x, 1, kLanesPerRow);
    x += __shfl_xor(x, 2, kLanesPerRow);
    x += __shfl_xor(x, 4, kLanesPerRow);
    return x;
}

// RAW: q and k arrive unnormalised and alpha, beta, lambda as logits (the layer's
// prologue, Q-Delta reading notes §1 and §3.1): q / sqrt(|q|^2 + 1e-6), likewise k;
// beta = sigmoid(b), lambda = sigmoid(l), alpha = exp(-softplus(a)) = 1 / (1 + exp(a)).
template <class P, int DK, int DV, bool HAS_A, bool HAS_L, bool RAW>
__global__ __launch_bounds__(kStepThreads) void step_kernel(const StepArgs args) {
    using R = typename P::R;
    constexpr int NG = DK / (4 * kLanesPerRow);           // float4 column groups per lane
    constexpr int ROWS_PER_PASS = kWave / kLanesPerRow;    // 8 rows per wave per pass
    constexpr int ROWS_PER_WAVE = DV / 4;
    constexpr int NPASS = ROWS_PER_WAVE / ROWS_PER_PASS;
    static_assert(NPASS >= 1 && NG >= 1, "unsupported step shape");

    const int nh = blockIdx.x;
    const int lane = lane_id();
    const int wave = wave_id();
    const int sub = lane % kLanesPerRow;
    const int grp = lane / kLanesPerRow;

    const R *gq = static_cast<const R *>(args.q) + static_cast<size_t>(nh) * DK;
    const R *gk = static_cast<const R *>(args.k) + static_cast<size_t>(nh) * DK;
    const R *gv = static_cast<const R *>(args.v) + static_cast<size_t>(nh) * DV;
    R *go = static_cast<R *>(args.o) + static_cast<size_t>(nh) * DV;
    float *S = args.S + static_cast<size_t>(nh) * DV * DK;

    // state rows first: the loads that matter
    f32x4 s[NPASS][NG];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = wave * ROWS_PER_WAVE + p * ROWS_PER_PASS + grp;
#pragma unroll
        for (int m = 0; m < NG; ++m)
            s[p][m] = *reinterpret_cast<const f32x4 *>(S + static_cast<size_t>(row) * DK + 4 * (m * kLanesPerRow + sub));
    }

    const float alpha = HAS_A ? (RAW ? 1.f / (1.f + __expf(args.alpha[nh])) : args.alpha[nh]) : 1.f;
    const float beta = RAW ? 1.f / (1.f + __expf(-args.beta[nh])) : args.beta[nh];
    const float lam = HAS_L ? (RAW ? 1.f / (1.f + __expf(-args.lam[nh])) : args.lam[nh]) : 0.f;
    f32x4 kk[NG], qq[NG], xx[NG];
#pragma unroll
    for (int m = 0; m < NG; ++m) {
        const int c = 4 * (m * kLanesPerRow + sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kk[m][i] = P::to_f32(gk[c + i]);
            qq[m][i] = P::to_f32(gq[c + i]);
        }
    }
    if constexpr (RAW) {                      // the eight lanes of a row hold all of q and k
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int m = 0; m < NG; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sk += kk[m][i] * kk[m][i];
                sq += qq[m][i] * qq[m][i];
            }
        const float rk = __frsqrt_rn(group8_sum(sk) + 1e-6f), rq = __frsqrt_rn(group8_sum(sq) + 1e-6f);
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            kk[m] *= rk;
            qq[m] *= rq;
        }
    }
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < NG; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xx[m][i] = HAS_L ? kk[m][i] + lam * qq[m][i] : kk[m][i];
            kq += kk[m][i] * qq[m][i];
        }
    kq = group8_sum(kq);

#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int row = wave * ROWS_PER_WAVE + p * ROWS_PER_PASS + grp;
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int m = 0; m < NG; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a += s[p][m][i] * xx[m][i];
                c += s[p][m][i] * qq[m][i];
            }
        }
        a = group8_sum(a);
        c = group8_sum(c);
        const float vj = P::to_f32(gv[row]);
        const float e = vj - alpha * a;          // error along x, from the decayed state
        const float be = beta * e;
#pragma unroll
        for (int m = 0; m < NG; ++m) {
            f32x4 ns;
#pragma unroll
            for (int i = 0; i < 4; ++i) ns[i] = alpha * s[p][m][i] + be * kk[m][i];
            *reinterpret_cast<f32x4 *>(S + static_cast<size_t>(row) * DK + 4 * (m * kLanesPerRow + sub)) = ns;
        }
        if (sub == 0) go[row] = P::from_f32(alpha * c + be * kq);
    }
}

template <class P, int DK, int DV, bool RAW>
void launch_step_gates(const StepArgs &a, hipStream_t stream) {
    const dim3 grid(a.N * a.H), blk(kStepThreads);
    const bool ha = a.alpha != nullptr, hl = a.lam != nullptr;
    if (ha && hl) hipLaunchKernelGGL((step_kernel<P, DK, DV, true, true, RAW>), grid, blk, 0, stream, a);
    else if (ha) hipLaunchKernelGGL((step_kernel<P, DK, DV, true, false, RAW>), grid, blk, 0, stream, a);
    else if (hl) hipLaunchKernelGGL((step_kernel<P, DK, DV, false, true, RAW>), grid, blk, 0, stream, a);
    else hipLaunchKernelGGL((step_kernel<P, DK, DV, false, false, RAW>), grid, blk, 0, stream, a);
}

template <class P, int DK, int DV>
hipError_t launch_step_typed(const StepArgs &a, hipStream_t stream) {
    if (a.N * a.H == 0) return hipSuccess;
    if (a.raw) launch_step_gates<P, DK, DV, true>(a, stream);
    else launch_step_gates<P, DK, DV, false>(a, stream);
    return hipGetLastError();
}

template <class P>
hipError_t launch_step_p(int dk, int dv, const StepArgs &a, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_step_typed<P, 128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_step_typed<P, 128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_step_typed<P, 64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_step_typed<P, 64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool step_supported(int dtype, int dk, int dv) {
    return (dtype == 0 || dtype == 1) && (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

hipError_t launch_step(int dtype, int dk, int dv, const StepArgs &a, hipStream_t stream) {
    return dtype == 1 ? launch_step_p<Bf16>(dk, dv, a, stream) : launch_step_p<F32>(dk, dv, a, stream);
}

}  // namespace qd
