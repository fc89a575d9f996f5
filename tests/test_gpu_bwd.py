"""Parity of the layer backward (qdelta_chunk_bwd, through the C ABI) against the fp64
oracle's adjoint of the recurrence (oracle.qdelta_bwd).

Metric per gradient, per (batch, head) slice: max|g - g_ref| / max|g_ref|, worst slice
reported.  Bars: 1e-4 for fp32 inputs (fp32 MFMA, fp32 accumulation) and 2e-2 for
bf16 inputs, the forward's bars.  The kernels round every MFMA operand to bf16 (relative
2^-9) and a gradient is a chain of up to five such products (e.g. dq through Z, P, dL
and K); ordinary inputs measure 6.4e-3 or less.  Only the correlated-keys stress case
keeps a separate, wider bar (see its test).  The oracle consumes fp64 upcasts of exactly
the values handed to the GPU; the full-size workload is compared whole.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_sequence_layers_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
AXES = dict(dq=(1, 3), dk=(1, 3), dv=(1, 3), dalpha=(1,), dbeta=(1,), dlam=(1,), dS0=(2, 3))


def slice_err(y, ref, axes):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(y - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


def dev(x):
    return None if x is None else x.cuda()


def run_bwd(qd, x, dO, dST, C):
    g = qd.qdelta_chunk_bwd(dev(x.q), dev(x.k), dev(x.v), dev(x.alpha), x.beta.cuda(), dev(x.lam), dev(x.S0),
                            dO.cuda(), dev(dST), C=C)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.float().cpu().numpy()) for n, t in g.items()}


def compare(got, x, dO, dST, tol, sel=None):
    errs = {}
    if sel is None:
        ref = oracle.qdelta_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, x.S0, dO, dST)
        for n, r in ref.items():
            if got.get(n) is not None:
                errs[n] = slice_err(got[n], r, AXES[n])
    else:
        for b, h in sel:
            s = lambda t: None if t is None else t[b:b + 1, :, h:h + 1]
            s0 = None if x.S0 is None else x.S0[b:b + 1, h:h + 1]
            st = None if dST is None else dST[b:b + 1, h:h + 1]
            ref = oracle.qdelta_bwd(s(x.q), s(x.k), s(x.v), s(x.alpha), s(x.beta), s(x.lam), s0, s(dO), st)
            for n, r in ref.items():
                if got.get(n) is None:
                    continue
                gs = got[n][b:b + 1, h:h + 1] if n == "dS0" else got[n][b:b + 1, :, h:h + 1]
                errs[n] = max(errs.get(n, 0.0), slice_err(gs, r, AXES[n]))
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (bar {tol:g})", flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    for n, t in got.items():
        if t is not None:
            assert np.isfinite(t).all(), n


CASES = [
    # dtype, B, T, H, dk, dv, C, alpha, lam, S0/dST
    ("f32", 2, 77, 2, 64, 64, 16, "random", "random", True),
    ("f32", 1, 100, 2, 128, 128, 32, "random", "random", True),
    ("f32", 1, 70, 2, 64, 128, 32, "one", "random", True),
    ("f32", 1, 65, 2, 128, 64, 16, "random", "zero", False),
    ("f32", 1, 40, 1, 64, 64, 32, "one", "zero", True),
    ("bf16", 1, 300, 2, 128, 128, 64, "random", "random", True),
    ("bf16", 2, 130, 2, 64, 128, 32, "random", "random", True),
    ("bf16", 1, 90, 3, 128, 64, 16, "random", "random", False),
    ("bf16", 1, 200, 2, 128, 128, 64, "one", "random", True),
    ("bf16", 1, 150, 2, 128, 128, 64, "random", "zero", True),
    ("bf16", 1, 129, 2, 128, 128, 64, "one", "zero", False),
    ("bf16", 1, 64, 2, 64, 64, 64, "random", "random", True),
]


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,C,alpha,lam,state", CASES)
def test_bwd_parity(qd, dtype, B, T, H, dk, dv, C, alpha, lam, state):
    print(f"[bwd] {dtype} B{B} T{T} H{H} dk{dk} dv{dv} C{C} alpha={alpha} lam={lam} state={state}", flush=True)
    x = inputs.chunk_inputs(B, T, H, dk, dv, dtype, seed=T + C, alpha=alpha, lam=lam,
                            s0_std=0.1 if state else None, gates_as_none=True)
    dO, dST = inputs.upstream_grads(B, T, H, dk, dv, dtype, seed=T + 1, dst_std=0.1 if state else None)
    got = run_bwd(qd, x, dO, dST, C)
    assert (got["dalpha"] is None) == (x.alpha is None) and (got["dlam"] is None) == (x.lam is None)
    compare(got, x, dO, dST, TOL[dtype])


@pytest.mark.parametrize("C", [32, 64])
def test_bwd_correlated_keys(qd, C):
    """Keys with mean pairwise cosine about 0.8 (the forward's stress level) make the
    triangular solve ill-conditioned; the forward itself then loses about 1.5e-2 in bf16.
    This stress case has its own bars: dalpha, a reverse cumulative sum over the chunk of
    terms that largely cancel, 6e-2 (measured 3.6-3.9e-2); the other gradients 3e-2
    (dv measured 2.4e-2)."""
    print(f"[bwd] bf16 correlated keys C={C}", flush=True)
    x = inputs.chunk_inputs(1, 256, 2, 128, 128, "bf16", seed=77, s0_std=0.05, key_corr=2.0)
    dO, dST = inputs.upstream_grads(1, 256, 2, 128, 128, "bf16", seed=78, dst_std=0.05)
    got = run_bwd(qd, x, dO, dST, C)
    da = got.pop("dalpha")
    ref = oracle.qdelta_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, x.S0, dO, dST)
    e = slice_err(da, ref["dalpha"], AXES["dalpha"])
    print(f"  dalpha={e:.2e} (bar 6e-2)", flush=True)
    assert e <= 6e-2
    compare(got, x, dO, dST, 3e-2)


def test_bwd_empty_and_single_token(qd):
    """T = 0 gives dS0 = dS_T; T = 1 is one token.  At T = 1 each (batch, head) slice of a
    gate gradient is a single value, so the per-slice relative metric reports that value's
    conditioning: dbeta = sum_i u_i (G k)_i can cancel by three orders of magnitude (the CPU
    test test_single_token_dbeta_is_a_cancelling_dot_product works one such case through in
    fp32).  dbeta is therefore bounded against the scale of its terms, sum_i |u_i (G k)_i|,
    and every other gradient by the usual bar."""
    print("[bwd] T=0 and T=1", flush=True)
    x = inputs.chunk_inputs(1, 0, 2, 64, 64, "f32", seed=1, s0_std=0.1)
    dO, dST = inputs.upstream_grads(1, 0, 2, 64, 64, "f32", seed=2, dst_std=0.1)
    got = run_bwd(qd, x, dO, dST, 16)
    np.testing.assert_array_equal(got["dS0"], dST.numpy())
    x = inputs.chunk_inputs(1, 1, 2, 64, 64, "f32", seed=3, s0_std=0.1)
    dO, dST = inputs.upstream_grads(1, 1, 2, 64, 64, "f32", seed=4, dst_std=0.1)
    got = run_bwd(qd, x, dO, dST, 16)
    ref = oracle.qdelta_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, x.S0, dO, dST)
    f64 = lambda t: t.double().numpy()
    for h in range(2):
        q, k, v = f64(x.q[0, 0, h]), f64(x.k[0, 0, h]), f64(x.v[0, 0, h])
        u = v - float(x.alpha[0, 0, h]) * f64(x.S0[0, h]) @ (k + float(x.lam[0, 0, h]) * q)
        scale = np.abs(u * ((f64(dST[0, h]) + np.outer(f64(dO[0, 0, h]), q)) @ k)).sum()
        err = abs(got["dbeta"][0, 0, h] - ref["dbeta"][0, 0, h])
        print(f"  head {h}: dbeta abs err {err:.2e}, terms' scale {scale:.3f}", flush=True)
        assert err <= 1e-6 * scale
    got.pop("dbeta")
    compare(got, x, dO, dST, TOL["f32"])


def gate_term_scales(x, dO, dST):
    """Per (batch, head): the largest sum of |terms| over the tokens, for the two dot
    products that give the scalar gate gradients in the recurrence's adjoint,
    dbeta_t = sum_i u_i (G k)_i and dlambda_t = sum_j q_j (dx)_j (u the token error,
    G = dLoss/dS_t, dx = -alpha S_{t-1}^T beta G k).  Written out in fp64 numpy for small
    cases; used to bound those gradients where they cancel."""
    f = lambda t: t.double().numpy()
    B, T, H, dk = x.q.shape
    scales = {"dbeta": np.zeros((B, H)), "dlam": np.zeros((B, H))}
    for b in range(B):
        for h in range(H):
            q, k, v = f(x.q[b, :, h]), f(x.k[b, :, h]), f(x.v[b, :, h])
            a = f(x.alpha[b, :, h]) if x.alpha is not None else np.ones(T)
            be = f(x.beta[b, :, h])
            la = f(x.lam[b, :, h]) if x.lam is not None else np.zeros(T)
            S = f(x.S0[b, h]) if x.S0 is not None else np.zeros((v.shape[1], dk))
            states = [S]
            for t in range(T):
                xx = k[t] + la[t] * q[t]
                S = a[t] * (S - be[t] * np.outer(S @ xx, k[t])) + be[t] * np.outer(v[t], k[t])
                states.append(S)
            G = f(dST[b, h]) if dST is not None else np.zeros_like(S)
            do = f(dO[b, :, h])
            for t in range(T - 1, -1, -1):
                P = states[t]
                xx = k[t] + la[t] * q[t]
                G = G + np.outer(do[t], q[t])
                gk = G @ k[t]
                u = v[t] - a[t] * P @ xx
                dx = -a[t] * P.T @ (be[t] * gk)
                scales["dbeta"][b, h] = max(scales["dbeta"][b, h], np.abs(u * gk).sum())
                scales["dlam"][b, h] = max(scales["dlam"][b, h], np.abs(q[t] * dx).sum())
                G = a[t] * G - a[t] * np.outer(be[t] * gk, xx)
    return scales


@pytest.mark.parametrize("dtype,C", [("f32", 16), ("f32", 32), ("bf16", 32), ("bf16", 64)])
def test_bwd_strong_decay(qd, dtype, C):
    """alpha = exp(-softplus(a)), a ~ N(+1, 1): a chunk's cumulative decay reaches the
    bottom of the fp32 range (see the forward's strong-decay test).  Under such decay the
    read-direction gradient dlambda_t = q . dx_t is small (its slice maximum about 0.04,
    against about 1.2 at ordinary decay) while its terms are not, so dbeta and dlambda
    are bounded against their terms' scale (gate_term_scales) at the dtype's bar; every
    other gradient against the usual per-slice metric."""
    print(f"[bwd] strong decay {dtype} C={C}", flush=True)
    x = inputs.chunk_inputs(1, 200, 2, 128, 128, dtype, seed=17 + C, s0_std=0.1, alpha_logit_mean=1.0)
    dO, dST = inputs.upstream_grads(1, 200, 2, 128, 128, dtype, seed=18 + C, dst_std=0.1)
    got = run_bwd(qd, x, dO, dST, C)
    ref = oracle.qdelta_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, x.S0, dO, dST)
    scales = gate_term_scales(x, dO, dST)
    for n in ("dbeta", "dlam"):
        err = np.abs(got[n] - ref[n]).max(axis=1)                    # [B, H]
        rel = float((err / scales[n]).max())
        print(f"  {n}: max abs err / terms' scale = {rel:.2e}, per-slice metric "
              f"{slice_err(got[n], ref[n], AXES[n]):.2e}", flush=True)
        assert rel <= TOL[dtype], n
        got.pop(n)
    compare(got, x, dO, dST, TOL[dtype])


def test_bwd_full_size_whole(qd):
    """B8 T4096 H16 d128 C64 bf16 (the 1.3B-layer shape), every gradient compared whole."""
    print("[bwd] full size B8 T4096 H16 d128 C64 bf16, whole tensors", flush=True)
    x = inputs.workload_inputs("layer_1p3b_bf16", seed=5)
    dO, dST = inputs.upstream_grads(8, 4096, 16, 128, 128, "bf16", seed=6, dst_std=0.02)
    got = run_bwd(qd, x, dO, dST, 64)
    compare(got, x, dO, dST, TOL["bf16"])


def test_bwd_argument_errors(qd):
    print("[bwd] argument errors", flush=True)
    x = inputs.chunk_inputs(1, 64, 2, 64, 64, "f32", seed=1, device="cuda")
    dO, _ = inputs.upstream_grads(1, 64, 2, 64, 64, "f32", seed=2, device="cuda")
    with pytest.raises(qd.QDeltaError, match="unsupported"):
        qd.qdelta_chunk_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, dO, C=64)   # fp32 C = 64
    ws = qd.qdelta_chunk_bwd_workspace_bytes(1, 64, 2, 64, 64, 32, torch.float32)
    assert ws == 2 * 2 * 2 * 64 * 64 * 4
    small = torch.empty(ws - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(qd.QDeltaError, match="workspace"):
        qd.qdelta_chunk_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, dO, C=32, workspace=small)
    with pytest.raises(qd.QDeltaError, match="invalid"):   # an output aliasing an input
        qd.qdelta_chunk_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, dO, C=32, out={"dq": x.q})
