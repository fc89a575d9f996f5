"""fp64 CPU oracle for the Q-Delta layer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product package.

Contents
  * ``qdelta_fwd``  -- the token-by-token gated recurrence (C, fp64, OpenMP).
  * ``qdelta_step`` -- one decode step of the same recurrence.
  * ``step_rw``     -- one step with explicit read and write directions.
  * ``qdelta_bwd``  -- gradients of ``qdelta_fwd`` by the hand-derived adjoint of
                       the recurrence, token by token in reverse (C, fp64).
  * ``qed_fwd``     -- the QED / GDN-2 recurrence with per-channel decay and vector
                       erase and write gates (the QED reading notes §2.1-2.2; C, fp64).
  * ``eda_fwd``     -- Erase-then-Delta: erase along e, then a delta write along k (the
                       EDA explainer's core method, as one composed map; C, fp64).
  * ``chunk_form``  -- the chunkwise WY/UT-transform algebra in fp64 numpy
                       (module ``oracle.chunk_form``), used to pin that the
                       chunked algebra reproduces the recurrence.

Source of the rule: the Q-Delta reading notes, §2.4 (the boxed gated update,
evaluated row by row); state convention S in R^{d_v x d_k} from §2.1.
"""
import ctypes
import os

import numpy as np

from .build_oracle import LIB, build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("ORACLE_LIB")      # a separately built copy (the sanitizer test)
    if override:
        lib = ctypes.CDLL(override)
    else:
        src = os.path.join(os.path.dirname(LIB), "qdelta_oracle.c")
        if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(src):
            build()
        lib = ctypes.CDLL(LIB)
    lib.oracle_qdelta_fwd.restype = ctypes.c_int
    lib.oracle_qdelta_fwd.argtypes = [_dp] * 9 + [ctypes.c_int] * 6
    lib.oracle_qdelta_step.restype = ctypes.c_int
    lib.oracle_qdelta_step.argtypes = [_dp] * 8 + [ctypes.c_int] * 5
    lib.oracle_step_rw.restype = None
    lib.oracle_step_rw.argtypes = [_dp] * 5 + [ctypes.c_double, ctypes.c_double, _dp,
                                                ctypes.c_int, ctypes.c_int]
    lib.oracle_qdelta_bwd.restype = ctypes.c_int
    lib.oracle_qdelta_bwd.argtypes = [_dp] * 16 + [ctypes.c_int] * 6
    lib.oracle_qed_fwd.restype = ctypes.c_int
    lib.oracle_qed_fwd.argtypes = [_dp] * 10 + [ctypes.c_int] * 6
    lib.oracle_eda_fwd.restype = ctypes.c_int
    lib.oracle_eda_fwd.argtypes = [_dp] * 7 + [ctypes.c_int] * 6
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a):
    """Contiguous fp64 numpy copy of an array-like (torch tensors are moved to CPU)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def max_threads() -> int:
    return _load().oracle_max_threads()


def qdelta_fwd(q, k, v, alpha, beta, lam, S0=None, nthreads: int = 0, want_o: bool = True):
    """Recurrence forward.  Shapes: q,k [B,T,H,dk]; v [B,T,H,dv]; alpha, beta, lam
    [B,T,H] (alpha None means 1, lam None means 0); S0 [B,H,dv,dk] or None.
    Returns (o [B,T,H,dv] or None, S_T [B,H,dv,dk]) as fp64 numpy arrays."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta, lam, S0 = _f64(alpha), _f64(beta), _f64(lam), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv), dtype=np.float64) if want_o else None
    S_T = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_qdelta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(lam), _ptr(S0), _ptr(o), _ptr(S_T),
                                   B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_qdelta_fwd rejected its arguments")
    return o, S_T


def qdelta_step(q, k, v, alpha, beta, lam, S, nthreads: int = 0):
    """One decode step.  q,k [N,H,dk]; v [N,H,dv]; gates [N,H]; S [N,H,dv,dk].
    Returns (o [N,H,dv], S_new) as fp64 numpy arrays; the input S is not modified."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta, lam = _f64(alpha), _f64(beta), _f64(lam)
    S = _f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((N, H, dv), dtype=np.float64)
    rc = _load().oracle_qdelta_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(lam), _ptr(S), _ptr(o), N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_qdelta_step rejected its arguments")
    return o, S


def step_rw(S, read, write, v, q, alpha: float, beta: float):
    """One step of S <- alpha S + beta (v - alpha S read) write^T, o = S q, for a
    single state S [dv, dk].  Returns (o [dv], S_new [dv, dk])."""
    S = _f64(S).copy()
    read, write, v, q = _f64(read), _f64(write), _f64(v), _f64(q)
    dv, dk = S.shape
    o = np.empty(dv, dtype=np.float64)
    _load().oracle_step_rw(_ptr(S), _ptr(read), _ptr(write), _ptr(v), _ptr(q),
                           float(alpha), float(beta), _ptr(o), dk, dv)
    return o, S


def qdelta_bwd(q, k, v, alpha, beta, lam, S0, dO, dST=None, nthreads: int = 0):
    """Gradients of the loss sum(o * dO) + sum(S_T * dST) with respect to every input
    of ``qdelta_fwd``.  Shapes as ``qdelta_fwd``; dO [B,T,H,dv]; dST [B,H,dv,dk] or
    None (zero).  Returns a dict of fp64 arrays dq, dk, dv, dalpha, dbeta, dlam, dS0
    (dalpha and dlam are taken at alpha = 1 and lambda = 0 when those are None)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta, lam, S0 = _f64(alpha), _f64(beta), _f64(lam), _f64(S0)
    dO, dST = _f64(dO), _f64(dST)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.empty((B, T, H, dk)), dk=np.empty((B, T, H, dk)), dv=np.empty((B, T, H, dv)),
               dalpha=np.empty((B, T, H)), dbeta=np.empty((B, T, H)), dlam=np.empty((B, T, H)),
               dS0=np.empty((B, H, dv, dk)))
    rc = _load().oracle_qdelta_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(lam),
                                   _ptr(S0), _ptr(dO), _ptr(dST),
                                   *[_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "dbeta", "dlam", "dS0")],
                                   B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_qdelta_bwd failed (%d)" % rc)
    return out


def qed_fwd(q, k, v, g, b, w, lam_h, S0=None, nthreads: int = 0, want_o: bool = True):
    """QED / GDN-2 recurrence.  q, k, g, b [B,T,H,dk]; v, w [B,T,H,dv]; lam_h [H] (the
    head's strength; 0 gives GDN-2); S0 [B,H,dv,dk] or None.  State convention as
    ``qdelta_fwd`` (d_v x d_k).  Returns (o [B,T,H,dv] or None, S_T [B,H,dv,dk])."""
    q, k, v, g, b, w = (_f64(t) for t in (q, k, v, g, b, w))
    lam_h, S0 = _f64(lam_h), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv)) if want_o else None
    S_T = np.empty((B, H, dv, dk))
    rc = _load().oracle_qed_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(lam_h), _ptr(S0),
                                _ptr(o), _ptr(S_T), B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_qed_fwd rejected its arguments")
    return o, S_T


def eda_fwd(q, k, v, e, S0=None, nthreads: int = 0, want_o: bool = True):
    """Erase-then-Delta recurrence.  q, k, e [B,T,H,dk] (e unit-norm); v [B,T,H,dv]; S0
    [B,H,dv,dk] or None.  Returns (o [B,T,H,dv] or None, S_T [B,H,dv,dk])."""
    q, k, v, e, S0 = (_f64(t) for t in (q, k, v, e, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv)) if want_o else None
    S_T = np.empty((B, H, dv, dk))
    rc = _load().oracle_eda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(e), _ptr(S0), _ptr(o), _ptr(S_T),
                                B, T, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_eda_fwd rejected its arguments")
    return o, S_T
