// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace qd {

struct ChunkArgs {
    const void *q, *k, *v;          // [B][T][H][d_k] / [B][T][H][d_v], element type per dtype
    const float *alpha, *beta, *lam; // [B][T][H]; alpha/lam may be null (selects the instance)
    const float *S0;                // [B][H][d_v][d_k] or null
    void *o;                        // [B][T][H][d_v]
    float *S_T;                     // [B][H][d_v][d_k] or null
    int B, T, H, dv;
    int n_dvt;                      // number of 64-wide value-column tiles, d_v / 64
};

struct StepArgs {
    const void *q, *k, *v;          // [N][H][d_k] / [N][H][d_v]
    const float *alpha, *beta, *lam; // [N][H]
    float *S;                       // [N][H][d_v][d_k], in place
    void *o;                        // [N][H][d_v]
    int N, H;
};

// dtype: 0 = fp32, 1 = bf16.  Return hipSuccess or the launch error.
hipError_t launch_chunk_fwd(int dtype, int dk, int C, const ChunkArgs &a, hipStream_t stream);
hipError_t launch_step(int dtype, int dk, int dv, const StepArgs &a, hipStream_t stream);

// bf16 chunk forward, eight-wave pipelined kernel (qd_chunk_fwd_pipe.hip).
hipError_t launch_chunk_fwd_pipe(int dk, int C, const ChunkArgs &a, hipStream_t stream);

// Whether an instance exists for these sizes (checked before launching).
bool chunk_fwd_supported(int dtype, int dk, int dv, int C);
bool step_supported(int dtype, int dk, int dv);

}  // namespace qd
