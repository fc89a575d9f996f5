"""Python binding of libqdelta.so, the gfx950 Q-Delta layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI declared in ``include/qdelta.h``.  PyTorch supplies device memory and the
HIP stream: every wrapper takes ``stream=None`` (torch's current stream) or a
``torch.cuda.Stream``, enqueues the kernels on it and allocates any output or workspace
it creates while that stream is current.  If the library is not built, the functions raise; there is no
fallback path.

    qdelta_chunk_fwd(q, k, v, alpha, beta, lam, S0=None, C=64, o=None, S_T=None)
        -> (o, S_T)
    qdelta_step(q, k, v, alpha, beta, lam, S, o=None) -> o        (S updated in place)
    qdelta_chunk_bwd(q, k, v, alpha, beta, lam, S0, d_o, dS_T=None, C=64)
        -> dict(dq, dk, dv, dalpha, dbeta, dlam, dS0)
"""
import ctypes
import os

from . import inputs  # noqa: F401  (seeded workload generators)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqdelta.so")

QD_F32, QD_BF16 = 0, 1
# bytes of device scratch qdelta_chunk_fwd_noalloc holds per device (QDELTA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
_lib = None


class QDeltaError(RuntimeError):
    pass


def load_library():
    """Load libqdelta.so (built in-tree by ``python -m recurrent_sequence_layers_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise QDeltaError(f"{LIB_PATH} is missing: build it with "
                          "`python -m recurrent_sequence_layers_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.qdelta_abi_version.restype = i
    lib.qdelta_abi_version.argtypes = []
    lib.qdelta_status_string.restype = ctypes.c_char_p
    lib.qdelta_status_string.argtypes = [i]
    lib.qdelta_chunk_fwd_workspace_bytes.restype = sz
    lib.qdelta_chunk_fwd_workspace_bytes.argtypes = [i] * 7
    lib.qdelta_chunk_fwd.restype = i
    lib.qdelta_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp] + [i] * 7 + [vp, sz, vp]
    lib.qdelta_chunk_fwd_noalloc.restype = i
    lib.qdelta_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp] + [i] * 7 + [vp]
    lib.qdelta_chunk_fwd_raw.restype = i
    lib.qdelta_chunk_fwd_raw.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, fp] + [i] * 7 + [vp, sz, vp]
    lib.qdelta_step.restype = i
    lib.qdelta_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 5 + [vp]
    lib.qdelta_step_raw.restype = i
    lib.qdelta_step_raw.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 5 + [vp]
    lib.qdelta_qed_chunk_fwd.restype = i
    lib.qdelta_qed_chunk_fwd.argtypes = [vp] * 10 + [i] * 7 + [vp]
    lib.qdelta_qed_step.restype = i
    lib.qdelta_qed_step.argtypes = [vp] * 9 + [i] * 5 + [vp]
    lib.qdelta_eda_chunk_fwd_workspace_bytes.restype = sz
    lib.qdelta_eda_chunk_fwd_workspace_bytes.argtypes = [i] * 7
    lib.qdelta_eda_chunk_fwd.restype = i
    lib.qdelta_eda_chunk_fwd.argtypes = [vp] * 7 + [i] * 7 + [vp, sz, vp]
    lib.qdelta_eda_step.restype = i
    lib.qdelta_eda_step.argtypes = [vp] * 6 + [i] * 5 + [vp]
    lib.qdelta_chunk_bwd_workspace_bytes.restype = sz
    lib.qdelta_chunk_bwd_workspace_bytes.argtypes = [i] * 7
    lib.qdelta_chunk_bwd.restype = i
    lib.qdelta_chunk_bwd.argtypes = [vp] * 16 + [i] * 7 + [vp, sz, vp]
    _lib = lib
    return lib


def qdelta_abi_version() -> int:
    return load_library().qdelta_abi_version()


def qdelta_status_string(status: int) -> str:
    return load_library().qdelta_status_string(int(status)).decode()


def qdelta_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype) -> int:
    return int(load_library().qdelta_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, _dtype_code(dtype)))


def _dtype_code(dt) -> int:
    import torch
    if dt in (QD_F32, QD_BF16):
        return dt
    if dt == torch.float32:
        return QD_F32
    if dt == torch.bfloat16:
        return QD_BF16
    raise QDeltaError(f"unsupported dtype {dt}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None, shape=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise QDeltaError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise QDeltaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise QDeltaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise QDeltaError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _launch_stream(stream, device):
    """The stream the kernels are enqueued on: torch's current stream, or the given
    torch.cuda.Stream.  Wrappers allocate their outputs and workspaces while that stream
    is current, so the caching allocator ties those blocks to it: a workspace released on
    return is handed out again only to work ordered after these kernels."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if not isinstance(stream, torch.cuda.Stream):
        raise QDeltaError("stream must be a torch.cuda.Stream or None")
    return stream


def _raise(rc, fn):
    if rc != 0:
        raise QDeltaError(f"{fn}: {qdelta_status_string(rc)} (status {rc})")


def qdelta_chunk_fwd(q, k, v, alpha, beta, lam, S0=None, C: int = 64, o=None, S_T=None,
                     want_state: bool = True, stream=None, workspace=None, raw: bool = False):
    """Layer forward, chunkwise WY/UT form.  q, k [B,T,H,d_k], v [B,T,H,d_v] (fp32 or
    bf16, same dtype); alpha, beta, lam [B,T,H] fp32 (alpha None means 1, lam None
    means 0); S0 [B,H,d_v,d_k] fp32 or None.  Returns (o, S_T); S_T is None when
    want_state is False.  S_T may be passed as S0 for an in-place state update.
    workspace: a device tensor of at least qdelta_chunk_fwd_workspace_bytes(...) bytes
    (long sequences over few heads run a segmented schedule that needs one); when None
    and one is needed, it is allocated here.
    raw: q and k unnormalised and alpha, beta, lam given as logits (qdelta_chunk_fwd_raw:
    the layer's normalisation and gate maps run inside the kernel)."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (B, T, H, dv))
        for name, g in (("alpha", alpha), ("beta", beta), ("lam", lam)):
            _check(g, name, torch.float32, (B, T, H))
        _check(S0, "S0", torch.float32, (B, H, dv, dk))
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (B, T, H, dv))
        if S_T is None and want_state:
            S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
        _check(S_T, "S_T", torch.float32, (B, H, dv, dk))
        code = _dtype_code(dt)
        ws = lib.qdelta_chunk_fwd_workspace_bytes(B, T, H, dk, dv, C, code)
        if ws and workspace is None:
            workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
        fn = lib.qdelta_chunk_fwd_raw if raw else lib.qdelta_chunk_fwd
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(lam), _ptr(S0),
                _ptr(o), _ptr(S_T), B, T, H, dk, dv, int(C), code, ws_ptr, ws_bytes, ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_chunk_fwd_raw" if raw else "qdelta_chunk_fwd")
        return o, S_T


def qdelta_chunk_fwd_noalloc(q, k, v, alpha, beta, lam, S0, o, S_T, C: int = 64, stream=None):
    """qdelta_chunk_fwd for callers that cannot allocate: o and S_T (or None) are supplied
    by the caller and nothing is allocated, here or in the library; the segmented schedule,
    when the sizes call for it, runs in the library's per-device scratch (calls that overlap
    in time on one GPU race on it).  Raises when the sizes need more than
    NOALLOC_SCRATCH_BYTES of it."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (B, T, H, dv))
    for name, g in (("alpha", alpha), ("beta", beta), ("lam", lam)):
        _check(g, name, torch.float32, (B, T, H))
    _check(S0, "S0", torch.float32, (B, H, dv, dk))
    if o is None:
        raise QDeltaError("qdelta_chunk_fwd_noalloc: o must be supplied (nothing is allocated)")
    _check(o, "o", dt, (B, T, H, dv))
    _check(S_T, "S_T", torch.float32, (B, H, dv, dk))
    rc = lib.qdelta_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(lam), _ptr(S0),
                                      _ptr(o), _ptr(S_T), B, T, H, dk, dv, int(C), _dtype_code(dt),
                                      ctypes.c_void_p(s.cuda_stream))
    _raise(rc, "qdelta_chunk_fwd_noalloc")
    return o, S_T


def qdelta_chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype) -> int:
    return int(load_library().qdelta_chunk_bwd_workspace_bytes(B, T, H, d_k, d_v, C, _dtype_code(dtype)))


def qdelta_chunk_bwd(q, k, v, alpha, beta, lam, S0, d_o, dS_T=None, C: int = 64, want_dS0: bool = True,
                     out=None, workspace=None, stream=None):
    """Layer backward: gradients of sum(o * d_o) + sum(S_T * dS_T) for the forward of
    ``qdelta_chunk_fwd`` on the same inputs.  d_o [B,T,H,d_v] in the input dtype; dS_T
    [B,H,d_v,d_k] fp32 or None.  Returns a dict with dq, dk (like q), dv (like v), dbeta,
    and dalpha / dlam (fp32 [B,T,H], None when alpha / lam are None) and dS0 (fp32, None
    unless want_dS0).  ``out`` may supply any of those tensors; ``workspace`` a device
    buffer of at least qdelta_chunk_bwd_workspace_bytes(...) bytes (allocated when None)."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        dev = q.device
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (B, T, H, dv))
        _check(d_o, "d_o", dt, (B, T, H, dv))
        for name, g in (("alpha", alpha), ("beta", beta), ("lam", lam)):
            _check(g, name, torch.float32, (B, T, H))
        _check(S0, "S0", torch.float32, (B, H, dv, dk))
        _check(dS_T, "dS_T", torch.float32, (B, H, dv, dk))
        out = dict(out or {})
        shapes = dict(dq=((B, T, H, dk), dt), dk=((B, T, H, dk), dt), dv=((B, T, H, dv), dt),
                      dbeta=((B, T, H), torch.float32), dalpha=((B, T, H), torch.float32),
                      dlam=((B, T, H), torch.float32), dS0=((B, H, dv, dk), torch.float32))
        wanted = dict(dq=True, dk=True, dv=True, dbeta=True, dalpha=alpha is not None, dlam=lam is not None,
                      dS0=want_dS0)
        for name, (shape, dtype) in shapes.items():
            if not wanted[name]:
                out[name] = None
                continue
            if out.get(name) is None:
                out[name] = torch.empty(shape, dtype=dtype, device=dev)
            _check(out[name], name, dtype, shape)
        code = _dtype_code(dt)
        ws = lib.qdelta_chunk_bwd_workspace_bytes(B, T, H, dk, dv, C, code)
        if ws and workspace is None:
            workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
        rc = lib.qdelta_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(lam), _ptr(S0), _ptr(d_o),
                                  _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]),
                                  _ptr(out["dbeta"]), _ptr(out["dlam"]), _ptr(out["dS0"]), B, T, H, dk, dv, int(C), code,
                                  ws_ptr, ws_bytes, ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_chunk_bwd")
        return out


def qdelta_qed_chunk_fwd(q, k, v, g, b, w, lam_h, S0=None, C: int = 32, o=None, S_T=None, want_state=True,
                         stream=None):
    """QED / GDN-2 layer forward.  q, k [B,T,H,d_k], v [B,T,H,d_v] (fp32 or bf16); g, b
    [B,T,H,d_k], w [B,T,H,d_v], lam_h [H], S0 [B,H,d_v,d_k] fp32.  Returns (o, S_T)."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (B, T, H, dv))
        _check(g, "g", torch.float32, (B, T, H, dk)); _check(b, "b", torch.float32, (B, T, H, dk))
        _check(w, "w", torch.float32, (B, T, H, dv)); _check(lam_h, "lam_h", torch.float32, (H,))
        _check(S0, "S0", torch.float32, (B, H, dv, dk))
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (B, T, H, dv))
        if S_T is None and want_state:
            S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
        _check(S_T, "S_T", torch.float32, (B, H, dv, dk))
        rc = lib.qdelta_qed_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(lam_h), _ptr(S0),
                                      _ptr(o), _ptr(S_T), B, T, H, dk, dv, int(C), _dtype_code(dt), ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_qed_chunk_fwd")
        return o, S_T


def qdelta_qed_step(q, k, v, g, b, w, lam_h, S, o=None, stream=None):
    """One QED / GDN-2 decode step.  q, k [N,H,d_k], v [N,H,d_v]; g, b [N,H,d_k], w [N,H,d_v],
    lam_h [H] fp32; S [N,H,d_v,d_k] fp32 updated in place.  Returns o [N,H,d_v]."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        N, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (N, H, dv))
        _check(g, "g", torch.float32, (N, H, dk)); _check(b, "b", torch.float32, (N, H, dk))
        _check(w, "w", torch.float32, (N, H, dv)); _check(lam_h, "lam_h", torch.float32, (H,))
        _check(S, "S", torch.float32, (N, H, dv, dk))
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (N, H, dv))
        rc = lib.qdelta_qed_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(lam_h), _ptr(S), _ptr(o),
                                 N, H, dk, dv, _dtype_code(dt), ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_qed_step")
        return o


def qdelta_eda_chunk_fwd(q, k, v, e, S0=None, C: int = 64, o=None, S_T=None, want_state=True, workspace=None,
                         stream=None):
    """Erase-then-Delta layer forward.  q, k, e [B,T,H,d_k] (unit-norm), v [B,T,H,d_v], same
    dtype; S0 [B,H,d_v,d_k] fp32.  Returns (o, S_T).  workspace: a device buffer of at least
    qdelta_eda_chunk_fwd_workspace_bytes(...) bytes (allocated here when None)."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(e, "e", dt, q.shape); _check(v, "v", dt, (B, T, H, dv))
        _check(S0, "S0", torch.float32, (B, H, dv, dk))
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (B, T, H, dv))
        if S_T is None and want_state:
            S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q.device)
        _check(S_T, "S_T", torch.float32, (B, H, dv, dk))
        code = _dtype_code(dt)
        ws = lib.qdelta_eda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, C, code)
        if ws and workspace is None:
            workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
        rc = lib.qdelta_eda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv,
                                      int(C), code, ws_ptr, ws_bytes, ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_eda_chunk_fwd")
        return o, S_T


def qdelta_eda_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, dtype) -> int:
    return int(load_library().qdelta_eda_chunk_fwd_workspace_bytes(B, T, H, d_k, d_v, C, _dtype_code(dtype)))


def qdelta_eda_step(q, k, v, e, S, o=None, stream=None):
    """One Erase-then-Delta decode step.  q, k, e [N,H,d_k], v [N,H,d_v]; S [N,H,d_v,d_k] fp32,
    updated in place.  Returns o [N,H,d_v]."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        N, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(e, "e", dt, q.shape); _check(v, "v", dt, (N, H, dv))
        _check(S, "S", torch.float32, (N, H, dv, dk))
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (N, H, dv))
        rc = lib.qdelta_eda_step(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(S), _ptr(o), N, H, dk, dv, _dtype_code(dt),
                                 ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_eda_step")
        return o


def qdelta_step(q, k, v, alpha, beta, lam, S, o=None, stream=None, raw: bool = False):
    """One decode step for N sequences x H heads.  q, k [N,H,d_k], v [N,H,d_v];
    alpha, beta, lam [N,H] fp32 (alpha None means 1, lam None means 0);
    S [N,H,d_v,d_k] fp32, updated in place.  Returns o [N,H,d_v].
    raw: q and k unnormalised and the gates as logits (qdelta_step_raw)."""
    import torch
    lib = load_library()
    s = _launch_stream(stream, q.device)
    with torch.cuda.stream(s):
        N, H, dk = q.shape
        dv = v.shape[-1]
        dt = q.dtype
        _check(q, "q", dt); _check(k, "k", dt, q.shape); _check(v, "v", dt, (N, H, dv))
        for name, g in (("alpha", alpha), ("beta", beta), ("lam", lam)):
            _check(g, name, torch.float32, (N, H))
        _check(S, "S", torch.float32, (N, H, dv, dk))
        if o is None:
            o = torch.empty((N, H, dv), dtype=dt, device=q.device)
        _check(o, "o", dt, (N, H, dv))
        fn = lib.qdelta_step_raw if raw else lib.qdelta_step
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(lam), _ptr(S), _ptr(o),
                N, H, dk, dv, _dtype_code(dt), ctypes.c_void_p(s.cuda_stream))
        _raise(rc, "qdelta_step_raw" if raw else "qdelta_step")
        return o
