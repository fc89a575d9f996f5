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
