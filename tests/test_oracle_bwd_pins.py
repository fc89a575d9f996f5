"""Pins of the oracle's backward (``oracle.qdelta_bwd``, the hand-derived adjoint of
the recurrence) against references that share nothing with that derivation:

  * reverse-mode automatic differentiation (torch, float64, CPU) of the forward
    recurrence written out again here from the Q-Delta reading notes §2.4;
  * central finite differences of the oracle's own forward (a different code path
    through the C library: only the forward step is shared, and that step is pinned
    by the forward pins);
  * the beta = 0 special case, where the layer is a pure decay with closed-form
    gradients;
  * planted mistakes in a copy of the adjoint, each of which the autograd pin rejects.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dlam", "dS0")


def _inputs(B, T, H, dk, dv, seed, alpha=True, lam=True, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    a = np.exp(-np.log1p(np.exp(r.standard_normal((B, T, H)) - 2.0))) if alpha else None
    la = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H)))) if lam else None
    S0 = 0.3 * r.standard_normal((B, H, dv, dk)) if s0 else None
    dO = r.standard_normal((B, T, H, dv))
    dST = r.standard_normal((B, H, dv, dk))
    return q, k, v, a, beta, la, S0, dO, dST


def _autograd(q, k, v, a, beta, la, S0, dO, dST):
    """Gradients of sum(o dO) + sum(S_T dST) by torch autograd of the recurrence
    S_t = alpha S_{t-1} (I - beta x k^T) + beta v k^T, x = k + lambda q, o_t = S_t q."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    leaf = lambda x: None if x is None else torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tb = leaf(q), leaf(k), leaf(v), leaf(beta)
    ta = leaf(a if a is not None else np.ones((B, T, H)))
    tl = leaf(la if la is not None else np.zeros((B, T, H)))
    tS = leaf(S0 if S0 is not None else np.zeros((B, H, dv, dk)))
    loss = torch.zeros((), dtype=torch.float64)
    eye = torch.eye(dk, dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            S = tS[b, h]
            for t in range(T):
                x = tk[b, t, h] + tl[b, t, h] * tq[b, t, h]
                S = ta[b, t, h] * S @ (eye - tb[b, t, h] * torch.outer(x, tk[b, t, h])) \
                    + tb[b, t, h] * torch.outer(tv[b, t, h], tk[b, t, h])
                loss = loss + (S @ tq[b, t, h]) @ torch.tensor(dO[b, t, h])
            loss = loss + (S * torch.tensor(dST[b, h])).sum()
    loss.backward()
    return dict(dq=tq.grad.numpy(), dk=tk.grad.numpy(), dv=tv.grad.numpy(), dalpha=ta.grad.numpy(),
                dbeta=tb.grad.numpy(), dlam=tl.grad.numpy(), dS0=tS.grad.numpy())


def _close(got, ref, rel=1e-11):
    for n in NAMES:
        err = np.abs(got[n] - ref[n]).max()
        scale = max(np.abs(ref[n]).max(), 1e-30)
        assert err <= rel * scale, f"{n}: max abs err {err:.3e} vs scale {scale:.3e}"


@pytest.mark.parametrize("alpha,lam,s0", [(True, True, True), (False, True, True), (True, False, False),
                                          (False, False, True)])
def test_bwd_matches_autograd(alpha, lam, s0):
    """Every gradient equals torch autograd of the recurrence; T = 150 crosses the
    oracle's recomputation stretches (64 tokens) twice and ends mid-stretch."""
    x = _inputs(2, 150, 2, 6, 4, seed=11 + 2 * alpha + lam, alpha=alpha, lam=lam, s0=s0)
    got = oracle.qdelta_bwd(*x)
    ref = _autograd(*x)
    _close(got, ref)


def test_bwd_matches_finite_differences():
    """Directional derivatives of the oracle's forward loss, by central differences,
    equal the inner product of each gradient with the direction."""
    q, k, v, a, beta, la, S0, dO, dST = _inputs(1, 40, 2, 5, 3, seed=3)
    g = oracle.qdelta_bwd(q, k, v, a, beta, la, S0, dO, dST)
    base = dict(q=q, k=k, v=v, alpha=a, beta=beta, lam=la, S0=S0)

    def loss(p):
        o, ST = oracle.qdelta_fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["lam"], p["S0"])
        return float((o * dO).sum() + (ST * dST).sum())

    r = np.random.default_rng(5)
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("alpha", "dalpha"), ("beta", "dbeta"),
                        ("lam", "dlam"), ("S0", "dS0")):
        d = r.standard_normal(base[name].shape)
        eps = 1e-6
        p_hi = dict(base); p_hi[name] = base[name] + eps * d
        p_lo = dict(base); p_lo[name] = base[name] - eps * d
        fd = (loss(p_hi) - loss(p_lo)) / (2 * eps)
        an = float((g[gname] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: fd {fd} vs adjoint {an}"


def test_bwd_beta_zero_closed_form():
    """beta = 0 leaves a pure decay, S_t = gamma_t S0 with gamma_t = prod_{s<=t} alpha_s, so
    o_t = gamma_t S0 q_t and:  dv = dk = dlambda = 0;  dq_t = gamma_t S0^T dO_t;
    dS0 = sum_t gamma_t dO_t q_t^T + gamma_T dST;
    dalpha_s = (sum_{t>=s} gamma_t dO_t.(S0 q_t) + gamma_T <dST, S0>) / alpha_s."""
    q, k, v, a, beta, la, S0, dO, dST = _inputs(2, 30, 2, 6, 5, seed=9)
    beta = np.zeros_like(beta)
    g = oracle.qdelta_bwd(q, k, v, a, beta, la, S0, dO, dST)
    gam = np.cumprod(a, axis=1)                                     # [B, T, H]
    assert np.abs(g["dv"]).max() == 0 and np.abs(g["dk"]).max() == 0 and np.abs(g["dlam"]).max() == 0
    dq = gam[..., None] * np.einsum("bhij,bthi->bthj", S0, dO)
    np.testing.assert_allclose(g["dq"], dq, rtol=0, atol=1e-12)
    dS0 = np.einsum("bth,bthi,bthj->bhij", gam, dO, q) + gam[:, -1][..., None, None] * dST
    np.testing.assert_allclose(g["dS0"], dS0, rtol=0, atol=1e-12)
    per_t = gam * np.einsum("bthi,bhij,bthj->bth", dO, S0, q)       # gamma_t dO_t . S0 q_t
    tail = per_t[:, ::-1].cumsum(axis=1)[:, ::-1] + (gam[:, -1] * np.einsum("bhij,bhij->bh", dST, S0))[:, None]
    np.testing.assert_allclose(g["dalpha"], tail / a, rtol=1e-12, atol=1e-12)


def test_bwd_zero_length_and_no_upstream_gradient():
    """T = 0 passes dST through to dS0; dO = 0 and dST = 0 give all-zero gradients."""
    q, k, v, a, beta, la, S0, dO, dST = _inputs(1, 0, 2, 4, 3, seed=2)
    g = oracle.qdelta_bwd(q, k, v, a, beta, la, S0, dO, dST)
    np.testing.assert_array_equal(g["dS0"], dST)
    q, k, v, a, beta, la, S0, dO, dST = _inputs(1, 20, 2, 4, 3, seed=2)
    g = oracle.qdelta_bwd(q, k, v, a, beta, la, S0, np.zeros_like(dO), None)
    for n in NAMES:
        assert np.abs(g[n]).max() == 0.0, n


# ---------------------------------------------------------------- planted mistakes
SRC = os.path.join(ROOT, "oracle", "qdelta_oracle.c")
BWD_MUTANTS = {
    "readout_grad_uses_entry_state": ("acc += St[(size_t)i * dkn + j] * dot[i];", "acc += P[(size_t)i * dkn + j] * dot[i];"),
    "dbeta_uses_v": ("db += u[i] * gk[i];", "db += vt[i] * gk[i];"),
    "dk_write_term_unscaled": ("dkt[j] = be * acc;", "dkt[j] = acc;"),
    "dalpha_feedback_dropped": ("for (i = 0; i < dvn; ++i) da -= du[i] * px[i];", ""),
    "dx_sign": ("dx[j] = -a * acc;", "dx[j] = a * acc;"),
    "dq_lambda_dropped": ("dqt[j] += la * dx[j];", ""),
    "state_grad_not_decayed": ("G[(size_t)i * dkn + j] = a * G[(size_t)i * dkn + j] - a * du[i] * x[j];",
                               "G[(size_t)i * dkn + j] = G[(size_t)i * dkn + j] - a * du[i] * x[j];"),
    "state_grad_transposed_rank_one": ("- a * du[i] * x[j];", "- a * du[i] * kt[j];"),
}


def _build_bwd(text, tmp, name):
    c, so = os.path.join(tmp, name + ".c"), os.path.join(tmp, name + ".so")
    open(c, "w").write(text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, c],
                   check=True)
    lib = ctypes.CDLL(so)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_qdelta_bwd.restype = ctypes.c_int
    lib.oracle_qdelta_bwd.argtypes = [dp] * 16 + [ctypes.c_int] * 6
    return lib


def _run_bwd(lib, x):
    q, k, v, a, beta, la, S0, dO, dST = x
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.empty((B, T, H, dk)), dk=np.empty((B, T, H, dk)), dv=np.empty((B, T, H, dv)),
               dalpha=np.empty((B, T, H)), dbeta=np.empty((B, T, H)), dlam=np.empty((B, T, H)),
               dS0=np.empty((B, H, dv, dk)))
    dp = ctypes.POINTER(ctypes.c_double)
    p = lambda z: None if z is None else np.ascontiguousarray(z).ctypes.data_as(dp)
    keep = [np.ascontiguousarray(z) if z is not None else None for z in x]
    rc = lib.oracle_qdelta_bwd(*[p(z) for z in keep], *[p(out[n]) for n in NAMES], B, T, H, dk, dv, 1)
    assert rc == 0
    return out


def test_bwd_pins_reject_planted_mistakes():
    text = open(SRC).read()
    x = _inputs(1, 70, 2, 5, 3, seed=21)
    ref = _autograd(*x)
    with tempfile.TemporaryDirectory() as tmp:
        _close(_run_bwd(_build_bwd(text, tmp, "clean"), x), ref)
        for name, (old, new) in BWD_MUTANTS.items():
            assert text.count(old) == 1, name
            got = _run_bwd(_build_bwd(text.replace(old, new), tmp, name), x)
            with pytest.raises(AssertionError):
                _close(got, ref, rel=1e-6)
