// C ABI of libqdelta.so: host-side argument checks, then kernel dispatch.
// Every check happens before anything is enqueued; nothing here allocates.
#include "qdelta.h"
#include "qd_internal.h"

#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Buf {
    const void *p;
    size_t n;
};

// Every output must be disjoint from every input and from every other output.  The one
// exception is the in-place state update: the output `same_out` may be exactly the input
// `same_in` (same address; a partial overlap is still rejected).
bool disjoint(std::initializer_list<Buf> ins, std::initializer_list<Buf> outs, const void *same_in = nullptr,
              const void *same_out = nullptr) {
    for (const Buf &o : outs) {
        for (const Buf &i : ins) {
            if (same_in && o.p == same_out && i.p == same_in && o.p == i.p) continue;
            if (overlaps(o.p, o.n, i.p, i.n)) return false;
        }
        for (const Buf &o2 : outs)
            if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return false;
    }
    return true;
}

// ---- scratch of qdelta_chunk_fwd_noalloc
// The segmented schedule's workspace (transition maps, offsets and entry states of the
// segments) for callers that cannot allocate: a file-scope device array that every GPU the
// library runs on holds until the process ends.  Host code never passes the symbol itself
// (on the host it is only a stand-in); it uses the device address hipGetSymbolAddress
// returns for the current device, taken once per device and kept below.  Nothing in it
// needs to start at zero: the schedule writes every byte it later reads (the identity fill
// of the maps, the offsets' zero entry states, the propagation).  Calls that overlap in time
// on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[QDELTA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[qd::kMaxDevices];

// Device address of the current device's scratch array, or null if it cannot be had.
void *device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= qd::kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int qdelta_abi_version(void) { return QDELTA_ABI_VERSION; }

const char *qdelta_status_string(int status) {
    switch (status) {
        case QD_OK: return "ok";
        case QD_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, misaligned or aliased buffer)";
        case QD_ERR_UNSUPPORTED: return "unsupported size or dtype (d_k, d_v in {64,128}; C in {16,32,64}; fp32 or bf16)";
        case QD_ERR_WORKSPACE: return "workspace too small";
        case QD_ERR_HIP: return "HIP runtime error at launch";
        case QD_ERR_SCRATCH_LIMIT:
            return "sizes need more than the 32 MiB scratch qdelta_chunk_fwd_noalloc holds per device";
        default: return "unknown status";
    }
}

size_t qdelta_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C, int dtype) {
    if (B < 0 || T < 0 || H < 0 || !qd::chunk_fwd_supported(dtype, d_k, d_v, C)) return 0;
    // single pass: every chunk intermediate stays in LDS; segmented schedule: the
    // per-segment transition maps and states
    const int P = qd::chunk_fwd_segments(dtype, B, T, H, d_k, d_v, C);
    return qd::chunk_fwd_segment_workspace(B, T, H, d_k, d_v, P);
}

size_t qdelta_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C, int dtype) {
    if (B < 0 || T < 0 || H < 0 || !qd::chunk_bwd_supported(dtype, d_k, d_v, C)) return 0;
    return qd::chunk_bwd_workspace(dtype, B, T, H, d_k, d_v, C);
}

int qdelta_chunk_bwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                     const float *lambda, const float *S0, const void *d_o, const float *dS_T, void *dq, void *dk,
                     void *dv, float *dalpha, float *dbeta, float *dlambda, float *dS0, int B, int T, int H,
                     int d_k, int d_v, int C, int dtype, void *workspace, size_t ws_bytes, void *stream) {
    if (B < 0 || T < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::chunk_bwd_supported(dtype, d_k, d_v, C)) return QD_ERR_UNSUPPORTED;
    const long long bh = static_cast<long long>(B) * H;
    if (bh == 0) return QD_OK;
    const long long nc = (static_cast<long long>(T) + C - 1) / C;
    if (bh * (d_v / 64) > 0x7fffffffLL || bh * nc > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    if ((alpha == nullptr && dalpha != nullptr) || (lambda == nullptr && dlambda != nullptr)) return QD_ERR_INVALID_ARG;
    const long long ntok = bh * T;
    if (ntok > 0 && (!q || !k || !v || !beta || !d_o || !dq || !dk || !dv || !dbeta)) return QD_ERR_INVALID_ARG;
    const size_t need = qd::chunk_bwd_workspace(dtype, B, T, H, d_k, d_v, C);
    if (ws_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return QD_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || !aligned16(S0) || !aligned16(dS_T) || !aligned16(dS0))
        return QD_ERR_INVALID_ARG;
    // every output and the workspace must be disjoint from every input and from one another
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t qk_bytes = static_cast<size_t>(ntok) * d_k * es, v_bytes = static_cast<size_t>(ntok) * d_v * es;
    const size_t g_bytes = static_cast<size_t>(ntok) * 4, st_bytes = static_cast<size_t>(bh) * d_v * d_k * 4;
    if (!disjoint({{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {alpha, g_bytes}, {beta, g_bytes}, {lambda, g_bytes},
                   {S0, st_bytes}, {d_o, v_bytes}, {dS_T, st_bytes}},
                  {{dq, qk_bytes}, {dk, qk_bytes}, {dv, v_bytes}, {dalpha, g_bytes}, {dbeta, g_bytes}, {dlambda, g_bytes},
                   {dS0, st_bytes}, {workspace, need}}))
        return QD_ERR_INVALID_ARG;

    qd::BwdArgs a;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta; a.lam = lambda;
    a.S0 = S0; a.dO = d_o; a.dST = dS_T;
    a.g_q = dq; a.g_k = dk; a.g_v = dv;
    a.g_alpha = dalpha; a.g_beta = dbeta; a.g_lam = dlambda; a.g_S0 = dS0;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    a.Hs = ws;
    a.dHs = ws ? ws + need / 2 : nullptr;
    a.B = B; a.T = T; a.H = H; a.dv = d_v;
    a.n_dvt = d_v / 64;
    const hipError_t err = qd::launch_chunk_bwd(dtype, d_k, C, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

int qdelta_qed_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *b, const float *w,
                         const float *lambda_h, const float *S0, void *o, float *S_T, int B, int T, int H, int d_k,
                         int d_v, int C, int dtype, void *stream) {
    if (B < 0 || T < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::qed_chunk_supported(dtype, d_k, d_v, C)) return QD_ERR_UNSUPPORTED;
    const long long bh = static_cast<long long>(B) * H;
    if (bh == 0) return QD_OK;
    if (bh * (d_v / 64) > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    const long long ntok = bh * T;
    if (!lambda_h || (ntok > 0 && (!q || !k || !v || !g || !b || !w || !o))) return QD_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(g) || !aligned16(b) ||
        !aligned16(S0) || !aligned16(S_T))
        return QD_ERR_INVALID_ARG;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t o_bytes = static_cast<size_t>(ntok) * d_v * es, st_bytes = static_cast<size_t>(bh) * d_v * d_k * 4;
    const size_t qk_bytes = static_cast<size_t>(ntok) * d_k * es, gb_bytes = static_cast<size_t>(ntok) * d_k * 4;
    const size_t w_bytes = static_cast<size_t>(ntok) * d_v * 4;
    if (!disjoint({{q, qk_bytes}, {k, qk_bytes}, {v, o_bytes}, {g, gb_bytes}, {b, gb_bytes}, {w, w_bytes},
                   {lambda_h, H * sizeof(float)}, {S0, st_bytes}},
                  {{o, o_bytes}, {S_T, st_bytes}}, S0, S_T))
        return QD_ERR_INVALID_ARG;
    qd::QedChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.b = b; a.w = w; a.lam_h = lambda_h;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    a.B = B; a.T = T; a.H = H; a.dv = d_v; a.n_dvt = d_v / 64;
    const hipError_t err = qd::launch_qed_chunk(dtype, d_k, C, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

int qdelta_qed_step(const void *q, const void *k, const void *v, const float *g, const float *b, const float *w,
                    const float *lambda_h, float *S, void *o, int N, int H, int d_k, int d_v, int dtype,
                    void *stream) {
    if (N < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::step_supported(dtype, d_k, d_v)) return QD_ERR_UNSUPPORTED;
    const long long nh = static_cast<long long>(N) * H;
    if (nh == 0) return QD_OK;
    if (nh > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    if (!q || !k || !v || !g || !b || !w || !lambda_h || !S || !o) return QD_ERR_INVALID_ARG;
    if (!aligned16(S) || !aligned16(g) || !aligned16(b)) return QD_ERR_INVALID_ARG;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t st_bytes = static_cast<size_t>(nh) * d_v * d_k * 4, o_bytes = static_cast<size_t>(nh) * d_v * es;
    if (!disjoint({{q, static_cast<size_t>(nh) * d_k * es}, {k, static_cast<size_t>(nh) * d_k * es}, {v, o_bytes},
                   {g, static_cast<size_t>(nh) * d_k * 4}, {b, static_cast<size_t>(nh) * d_k * 4},
                   {w, static_cast<size_t>(nh) * d_v * 4}, {lambda_h, H * sizeof(float)}},
                  {{o, o_bytes}, {S, st_bytes}}))
        return QD_ERR_INVALID_ARG;
    qd::QedStepArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.b = b; a.w = w; a.lam_h = lambda_h;
    a.S = S; a.o = o; a.N = N; a.H = H;
    const hipError_t err = qd::launch_qed_step(dtype, d_k, d_v, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

size_t qdelta_eda_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C, int dtype) {
    if (B < 0 || T < 0 || H < 0 || !qd::chunk_fwd_supported(dtype, d_k, d_v, C)) return 0;
    if (static_cast<long long>(B) * T * H == 0) return 0;
    return qd::eda_chunk_workspace(dtype, B, T, H, d_k, d_v, C);
}

int qdelta_eda_chunk_fwd(const void *q, const void *k, const void *v, const void *e, const float *S0, void *o,
                         float *S_T, int B, int T, int H, int d_k, int d_v, int C, int dtype, void *workspace,
                         size_t ws_bytes, void *stream) {
    if (B < 0 || T < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::chunk_fwd_supported(dtype, d_k, d_v, C)) return QD_ERR_UNSUPPORTED;
    const long long bh = static_cast<long long>(B) * H;
    if (bh == 0) return QD_OK;
    if (bh * (d_v / 64) > 0x7fffffffLL || static_cast<long long>(T) * 2 > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    const long long ntok = bh * T;
    if (ntok > 0 && (!q || !k || !v || !e || !o)) return QD_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(e) || !aligned16(o) || !aligned16(S0) ||
        !aligned16(S_T))
        return QD_ERR_INVALID_ARG;
    const size_t need = qdelta_eda_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype);
    if (ws_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return QD_ERR_WORKSPACE;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t qk_bytes = static_cast<size_t>(ntok) * d_k * es, o_bytes = static_cast<size_t>(ntok) * d_v * es;
    const size_t st_bytes = static_cast<size_t>(bh) * d_v * d_k * 4;
    if (!disjoint({{q, qk_bytes}, {k, qk_bytes}, {e, qk_bytes}, {v, o_bytes}, {S0, st_bytes}},
                  {{o, o_bytes}, {S_T, st_bytes}, {workspace, need}}, S0, S_T))
        return QD_ERR_INVALID_ARG;
    qd::EdaChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.e = e; a.S0 = S0; a.o = o; a.S_T = S_T;
    a.B = B; a.T = T; a.H = H; a.dv = d_v;
    const hipError_t err = qd::launch_eda_chunk(dtype, d_k, C, a, workspace, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

int qdelta_eda_step(const void *q, const void *k, const void *v, const void *e, float *S, void *o, int N, int H,
                    int d_k, int d_v, int dtype, void *stream) {
    if (N < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::step_supported(dtype, d_k, d_v)) return QD_ERR_UNSUPPORTED;
    const long long nh = static_cast<long long>(N) * H;
    if (nh == 0) return QD_OK;
    if (nh > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    if (!q || !k || !v || !e || !S || !o) return QD_ERR_INVALID_ARG;
    if (!aligned16(S)) return QD_ERR_INVALID_ARG;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t st_bytes = static_cast<size_t>(nh) * d_v * d_k * 4, o_bytes = static_cast<size_t>(nh) * d_v * es;
    const size_t qk_bytes = static_cast<size_t>(nh) * d_k * es;
    if (!disjoint({{q, qk_bytes}, {k, qk_bytes}, {e, qk_bytes}, {v, o_bytes}}, {{o, o_bytes}, {S, st_bytes}}))
        return QD_ERR_INVALID_ARG;
    qd::EdaStepArgs a;
    a.q = q; a.k = k; a.v = v; a.e = e; a.S = S; a.o = o; a.N = N; a.H = H;
    const hipError_t err = qd::launch_eda_step(dtype, d_k, d_v, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

}  // extern "C"

namespace {

// noalloc: the workspace arguments are ignored and the segmented schedule, when the sizes
// call for it, runs in the library's per-device scratch array instead.
int chunk_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
              const float *lambda, const float *S0, void *o, float *S_T, int B, int T, int H, int d_k, int d_v,
              int C, int dtype, void *workspace, size_t ws_bytes, void *stream, bool raw, bool noalloc = false) {
    if (B < 0 || T < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::chunk_fwd_supported(dtype, d_k, d_v, C)) return QD_ERR_UNSUPPORTED;
    if (raw && (dtype != QD_BF16 || (C != 32 && C != 64))) return QD_ERR_UNSUPPORTED;
    if (noalloc) {
        workspace = nullptr;
        ws_bytes = 0;
        const size_t need = qdelta_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype);
        if (need > QDELTA_NOALLOC_SCRATCH_BYTES) return QD_ERR_SCRATCH_LIMIT;
        if (need > 0 && static_cast<long long>(B) * H > 0) {
            workspace = device_scratch();
            if (!workspace) return QD_ERR_HIP;
            ws_bytes = QDELTA_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (ws_bytes < qdelta_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype)) return QD_ERR_WORKSPACE;
    const long long bh = static_cast<long long>(B) * H;
    if (bh == 0) return QD_OK;
    if (bh * (d_v / 64) > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    const long long ntok = bh * T;
    if (ntok > 0 && (!q || !k || !v || !beta || !o)) return QD_ERR_INVALID_ARG;
    // vector loads need 16-byte aligned rows
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(S0) || !aligned16(S_T))
        return QD_ERR_INVALID_ARG;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t state_bytes = static_cast<size_t>(bh) * d_v * d_k * 4;
    const size_t o_bytes = static_cast<size_t>(ntok) * d_v * es;
    const size_t qk_bytes = static_cast<size_t>(ntok) * d_k * es, g_bytes = static_cast<size_t>(ntok) * 4;
    const int P = qd::chunk_fwd_segments(dtype, B, T, H, d_k, d_v, C);
    const size_t need = qd::chunk_fwd_segment_workspace(B, T, H, d_k, d_v, P);
    if (need > 0 && (!workspace || !aligned16(workspace))) return QD_ERR_WORKSPACE;
    // outputs (and the workspace) disjoint from inputs and each other; S_T == S0 exactly is
    // the allowed in-place case
    if (!disjoint({{q, qk_bytes}, {k, qk_bytes}, {v, o_bytes}, {alpha, g_bytes}, {beta, g_bytes}, {lambda, g_bytes},
                   {S0, state_bytes}},
                  {{o, o_bytes}, {S_T, state_bytes}, {need > 0 ? workspace : nullptr, need}}, S0, S_T))
        return QD_ERR_INVALID_ARG;

    qd::ChunkArgs a;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta; a.lam = lambda;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    a.B = B; a.T = T; a.H = H; a.dv = d_v;
    a.n_dvt = d_v / 64;
    a.raw = raw;
    hipError_t err;
    if (P > 1) {
        err = qd::launch_chunk_fwd_segmented(dtype, d_k, C, a, P, workspace, static_cast<hipStream_t>(stream));
    } else {
        err = qd::launch_chunk_fwd(dtype, d_k, C, a, static_cast<hipStream_t>(stream));
    }
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

int step(const void *q, const void *k, const void *v, const float *alpha, const float *beta, const float *lambda,
         float *S, void *o, int N, int H, int d_k, int d_v, int dtype, void *stream, bool raw) {
    if (N < 0 || H < 0) return QD_ERR_INVALID_ARG;
    if (!qd::step_supported(dtype, d_k, d_v)) return QD_ERR_UNSUPPORTED;
    const long long nh = static_cast<long long>(N) * H;
    if (nh == 0) return QD_OK;
    if (nh > 0x7fffffffLL) return QD_ERR_UNSUPPORTED;
    if (!q || !k || !v || !beta || !S || !o) return QD_ERR_INVALID_ARG;
    if (!aligned16(S)) return QD_ERR_INVALID_ARG;
    const size_t es = dtype == QD_BF16 ? 2 : 4;
    const size_t state_bytes = static_cast<size_t>(nh) * d_v * d_k * 4;
    const size_t o_bytes = static_cast<size_t>(nh) * d_v * es;
    const size_t g_bytes = static_cast<size_t>(nh) * 4;
    if (!disjoint({{q, static_cast<size_t>(nh) * d_k * es}, {k, static_cast<size_t>(nh) * d_k * es}, {v, o_bytes},
                   {alpha, g_bytes}, {beta, g_bytes}, {lambda, g_bytes}},
                  {{o, o_bytes}, {S, state_bytes}}))
        return QD_ERR_INVALID_ARG;

    qd::StepArgs a;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta; a.lam = lambda;
    a.S = S; a.o = o; a.N = N; a.H = H;
    a.raw = raw;
    const hipError_t err = qd::launch_step(dtype, d_k, d_v, a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? QD_OK : QD_ERR_HIP;
}

}  // namespace

extern "C" {

int qdelta_chunk_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                     const float *lambda, const float *S0, void *o, float *S_T, int B, int T, int H, int d_k,
                     int d_v, int C, int dtype, void *workspace, size_t ws_bytes, void *stream) {
    return chunk_fwd(q, k, v, alpha, beta, lambda, S0, o, S_T, B, T, H, d_k, d_v, C, dtype, workspace, ws_bytes,
                     stream, false);
}

int qdelta_chunk_fwd_raw(const void *q, const void *k, const void *v, const float *alpha_logit,
                         const float *beta_logit, const float *lambda_logit, const float *S0, void *o, float *S_T,
                         int B, int T, int H, int d_k, int d_v, int C, int dtype, void *workspace, size_t ws_bytes,
                         void *stream) {
    return chunk_fwd(q, k, v, alpha_logit, beta_logit, lambda_logit, S0, o, S_T, B, T, H, d_k, d_v, C, dtype,
                     workspace, ws_bytes, stream, true);
}

int qdelta_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                             const float *lambda, const float *S0, void *o, float *S_T, int B, int T, int H, int d_k,
                             int d_v, int C, int dtype, void *stream) {
    return chunk_fwd(q, k, v, alpha, beta, lambda, S0, o, S_T, B, T, H, d_k, d_v, C, dtype, nullptr, 0, stream, false,
                     true);
}

int qdelta_step(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                const float *lambda, float *S, void *o, int N, int H, int d_k, int d_v, int dtype, void *stream) {
    return step(q, k, v, alpha, beta, lambda, S, o, N, H, d_k, d_v, dtype, stream, false);
}

int qdelta_step_raw(const void *q, const void *k, const void *v, const float *alpha_logit, const float *beta_logit,
                    const float *lambda_logit, float *S, void *o, int N, int H, int d_k, int d_v, int dtype,
                    void *stream) {
    return step(q, k, v, alpha_logit, beta_logit, lambda_logit, S, o, N, H, d_k, d_v, dtype, stream, true);
}

}  // extern "C"
