// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace qd {

// Devices the host-side caches have an entry for (device ids at or above it are simply
// not cached).
constexpr int kMaxDevices = 64;

// Compute units of the current device, read once per device and cached (0 if the query
// fails).  Sizes the segmented schedule and the backward's persistent grid.
int device_cu_count();

struct ChunkArgs {
    const void *q, *k, *v;          // [B][T][H][d_k] / [B][T][H][d_v], element type per dtype;
                                    // v may be null (read as zeros) for the bf16 C = 32, 64 kernel
    const float *alpha, *beta, *lam; // [B][T][H]; alpha/lam may be null (selects the instance)
    const float *S0;                // [B][H][d_v][d_k] or null
    void *o;                        // [B][T][H][d_v]; may be null (not written) for that kernel
    float *S_T;                     // [B][H][d_v][d_k] or null
    int B, T, H, dv;
    int n_dvt;                      // number of 64-wide value-column tiles, d_v / 64
    bool raw = false;               // q, k unnormalised and gates as logits (bf16 C = 32, 64 only)
    void *Hs = nullptr;             // [B][H][NC][d_v][d_k] in the element type: every chunk's entry state
                                    // (generic kernel only)
    const void *e = nullptr;        // [B][T][H][d_k] erase directions (Erase-then-Delta instance only)
};

// Layer backward (qd_chunk_bwd.hip).  Gradients of sum(o dO) + sum(S_T dST).
struct BwdArgs {
    const void *q, *k, *v;          // [B][T][H][d_k] / [B][T][H][d_v]
    const float *alpha, *beta, *lam; // [B][T][H]; alpha/lam may be null
    const float *S0;                // [B][H][d_v][d_k] or null
    const void *dO;                 // [B][T][H][d_v]
    const float *dST;               // [B][H][d_v][d_k] or null
    void *g_q, *g_k, *g_v;          // gradients: [B][T][H][d_k] / [B][T][H][d_v]
    float *g_alpha, *g_beta, *g_lam; // [B][T][H]; g_alpha/g_lam may be null
    float *g_S0;                    // [B][H][d_v][d_k] or null
    void *Hs, *dHs;                 // workspace: [B][H][NC][d_v][d_k] entry states and exit-state gradients,
                                    // in the element type
    int B, T, H, dv;
    int n_dvt;
};

struct StepArgs {
    const void *q, *k, *v;          // [N][H][d_k] / [N][H][d_v]
    const float *alpha, *beta, *lam; // [N][H]
    float *S;                       // [N][H][d_v][d_k], in place
    void *o;                        // [N][H][d_v]
    int N, H;
    bool raw = false;               // q, k unnormalised and gates as logits
};

// QED / GDN-2 (qd_qed.hip): per-key-channel log decay g and erase gate b [..][d_k] fp32,
// write gate w [..][d_v] fp32, strength lam_h [H] fp32.
struct QedChunkArgs {
    const void *q, *k, *v;          // [B][T][H][d_k] / [B][T][H][d_v]
    const float *g, *b, *w;         // [B][T][H][d_k], [B][T][H][d_k], [B][T][H][d_v]
    const float *lam_h;             // [H]
    const float *S0;                // [B][H][d_v][d_k] or null
    void *o;                        // [B][T][H][d_v]
    float *S_T;                     // [B][H][d_v][d_k] or null
    int B, T, H, dv;
    int n_dvt;
};
struct QedStepArgs {
    const void *q, *k, *v;          // [N][H][d_k] / [N][H][d_v]
    const float *g, *b, *w;         // [N][H][d_k], [N][H][d_k], [N][H][d_v]
    const float *lam_h;             // [H]
    float *S;                       // [N][H][d_v][d_k], in place
    void *o;                        // [N][H][d_v]
    int N, H;
};
bool qed_chunk_supported(int dtype, int dk, int dv, int C);
hipError_t launch_qed_chunk(int dtype, int dk, int C, const QedChunkArgs &a, hipStream_t stream);
hipError_t launch_qed_step(int dtype, int dk, int dv, const QedStepArgs &a, hipStream_t stream);

// Erase-then-Delta (qd_eda.hip): erase direction e [..][d_k] in the element type.
struct EdaChunkArgs {
    const void *q, *k, *v, *e;      // [B][T][H][d_k] (q, k, e) / [B][T][H][d_v]
    const float *S0;                // [B][H][d_v][d_k] or null
    void *o;                        // [B][T][H][d_v]
    float *S_T;                     // [B][H][d_v][d_k] or null
    int B, T, H, dv;
};
struct EdaStepArgs {
    const void *q, *k, *v, *e;      // [N][H][d_k] / [N][H][d_v]
    float *S;                       // [N][H][d_v][d_k], in place
    void *o;                        // [N][H][d_v]
    int N, H;
};
size_t eda_chunk_workspace(int dtype, int B, int T, int H, int dk, int dv, int C);
hipError_t launch_eda_chunk(int dtype, int dk, int C, const EdaChunkArgs &a, void *ws, hipStream_t stream);
hipError_t launch_eda_step(int dtype, int dk, int dv, const EdaStepArgs &a, hipStream_t stream);

// dtype: 0 = fp32, 1 = bf16.  Return hipSuccess or the launch error.
hipError_t launch_chunk_fwd(int dtype, int dk, int C, const ChunkArgs &a, hipStream_t stream);
hipError_t launch_step(int dtype, int dk, int dv, const StepArgs &a, hipStream_t stream);

// bf16 chunk forward, eight-wave pipelined kernel (qd_chunk_fwd_pipe.hip), C = 32 or 64;
// the _states variant also writes ChunkArgs::Hs.
hipError_t launch_chunk_fwd_pipe(int dk, int C, const ChunkArgs &a, hipStream_t stream);
hipError_t launch_chunk_fwd_pipe_states(int dk, int C, const ChunkArgs &a, hipStream_t stream);
// One launch of both instances (prepared inputs): a0 walked with its output, am and ag with
// the state-only instance (the segmented schedule's first step for a single sequence).
hipError_t launch_chunk_fwd_pipe_overlap(int dk, int C, const ChunkArgs &a0, const ChunkArgs &am, const ChunkArgs &ag,
                                        hipStream_t stream);
// Erase-then-Delta over the interleaved sequence read in place (ChunkArgs::e; T real tokens;
// beta, alpha, lam unused), bf16 C = 32, 64.
hipError_t launch_chunk_fwd_pipe_eda(int dk, int C, const ChunkArgs &a, hipStream_t stream);

// Segmented schedule (qd_segment.hip) for long sequences over few heads: the number of
// segments P the sequence is cut into (1 = the single-pass schedule), the workspace it
// needs, and the launch sequence.
int chunk_fwd_segments(int dtype, int B, int T, int H, int dk, int dv, int C);
size_t chunk_fwd_segment_workspace(int B, int T, int H, int dk, int dv, int P);
hipError_t launch_chunk_fwd_segmented(int dtype, int dk, int C, const ChunkArgs &a, int P, void *ws,
                                      hipStream_t stream);

// The forward keeping every chunk's entry state (ChunkArgs::Hs, element type) with no
// output (o == null): the eight-wave kernel for bf16 C = 32, 64, else the generic one.
hipError_t launch_chunk_fwd_states(int dtype, int dk, int C, const ChunkArgs &a, hipStream_t stream);

// Backward: workspace size and the three passes (states, reverse scan, per-chunk gradients).
bool chunk_bwd_supported(int dtype, int dk, int dv, int C);
size_t chunk_bwd_workspace(int dtype, int B, int T, int H, int dk, int dv, int C);
hipError_t launch_chunk_bwd(int dtype, int dk, int C, const BwdArgs &a, hipStream_t stream);

// Whether an instance exists for these sizes (checked before launching).
bool chunk_fwd_supported(int dtype, int dk, int dv, int C);
bool step_supported(int dtype, int dk, int dv);

}  // namespace qd
