"""Pins of the QED / GDN-2 oracle (``oracle.qed_fwd``) against what the QED reading notes
fix (page "The Query Knows What to Forget", reading notes):

  * the printed two-dimensional example of §2.4, exactly (golden fixture);
  * Eqs. (11)-(12) of §2.3: for one step from the same decayed state, the state and
    output differences between QED and GDN-2 are -lambda k (S_bar^T d)^T and
    -lambda rho S_bar^T d (rho = q^T k);
  * §2.5: the erase factor M = I - k a^T has K-1 unit eigenvalues and 1 - sum_i b_i k_i^2
    (the projection leaves a^T k unchanged), and the printed non-normal counterexample;
  * §2.1: with b = beta 1, w = beta 1, exp(g) = alpha 1 and lambda_h = 0, GDN-2 is Gated
    DeltaNet, which the Q-Delta oracle (pinned separately) computes at lambda = 0;
  * the response of a probe orthogonal to k does not change in one step (§2.3, Eq. 9).
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qed_2d_example.json")


def _one(x):
    return np.asarray(x, dtype=float).reshape(1, 1, 1, -1)


def _rand(B, T, H, dk, dv, seed, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((B, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    g = -np.log1p(np.exp(r.standard_normal((B, T, H, dk)) - 3.0))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H, dk))))
    w = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H, dv))))
    lam = 0.25 / (1.0 + np.exp(-(r.standard_normal(H) - 2.0)))
    S0 = 0.3 * r.standard_normal((B, H, dv, dk)) if s0 else None
    return q, k, v, g, b, w, lam, S0


def test_qed_printed_2d_example():
    """§2.4: K = 2, V = 1, k = (1, 0), q = (0.6, 0.8), b = (0.5, 0.5), S_bar = (2, 3),
    w v = 1, lambda = 0.2: GDN-2 reads 1 and outputs 3.6; QED writes dS = (-0.24, 0),
    reaching S = (1.76, 3) and o = 3.456, 0.144 lower."""
    ex = json.load(open(GOLDEN))
    i, p = ex["inputs"], ex["printed"]
    S_bar = np.array(i["S_bar"]).reshape(1, 1, 1, 2)
    run = lambda lam: oracle.qed_fwd(_one(i["q"]), _one(i["k"]), _one([i["w_times_v"]]), _one([0.0, 0.0]),
                                     _one(i["b"]), _one([1.0]), np.array([lam]), S_bar)
    o0, S0 = run(0.0)
    assert abs(o0.item() - p["baseline_output"]) < 1e-12
    np.testing.assert_allclose(S0.ravel(), i["S_bar"], atol=1e-12)        # baseline residual is zero
    o1, S1 = run(i["lambda"])
    np.testing.assert_allclose(S1.ravel(), p["S_new"], atol=1e-12)
    np.testing.assert_allclose(S1.ravel() - S0.ravel(), p["delta_S"], atol=1e-12)
    assert abs(o1.item() - p["output_new"]) < 1e-12
    assert abs((o0 - o1).item() - p["output_drop"]) < 1e-12


def test_qed_minus_gdn2_one_step():
    """Eqs. (11)-(12): one step from the same S_{t-1}, inputs shared, lambda vs 0."""
    q, k, v, g, b, w, lam, S0 = _rand(1, 1, 3, 7, 5, seed=4)
    o_q, S_q = oracle.qed_fwd(q, k, v, g, b, w, lam, S0)
    o_g, S_g = oracle.qed_fwd(q, k, v, g, b, w, np.zeros_like(lam), S0)
    for h in range(3):
        Sbar = S0[0, h] * np.exp(g[0, 0, h])[None, :]          # d_v x d_k, columns decayed
        kk, qq, bb = k[0, 0, h], q[0, 0, h], b[0, 0, h]
        u = bb * qq
        d = u - kk * (kk @ u)
        rho = qq @ kk
        np.testing.assert_allclose(S_q[0, h] - S_g[0, h], -lam[h] * np.outer(Sbar @ d, kk), atol=1e-13)
        np.testing.assert_allclose(o_q[0, 0, h] - o_g[0, 0, h], -lam[h] * rho * (Sbar @ d), atol=1e-13)


def test_qed_erase_factor_eigenvalues():
    """§2.5: with v = 0 and g = 0 the step maps S to S (I - a k^T) (our convention), so
    running it on S = I exposes the erase factor; its spectrum is K-1 ones and
    1 - sum_i b_i k_i^2, whatever lambda is."""
    dk = 6
    q, k, v, g, b, w, lam, _ = _rand(1, 1, 1, dk, dk, seed=8)
    lam = np.array([0.7])
    _, M = oracle.qed_fwd(q, k, np.zeros_like(v), np.zeros_like(g), b, w, lam, np.eye(dk).reshape(1, 1, dk, dk))
    ev = np.sort(np.linalg.eigvals(M[0, 0]).real)
    e = 1.0 - np.sum(b[0, 0, 0] * k[0, 0, 0] ** 2)
    np.testing.assert_allclose(ev, np.sort(np.r_[np.ones(dk - 1), e]), atol=1e-12)
    assert 0.0 < e < 1.0


def test_qed_non_normal_counterexample():
    """§2.5's counterexample: k = (1, 0), b = (0.5, 0.5), q = (0, 1), lambda = 0.2 give
    M = [[0.5, -0.1], [0, 1]] (the notes' K x K orientation), spectrum {0.5, 1}, and
    |M (0, 1)^T| = sqrt(1.01) > 1."""
    _, Mt = oracle.qed_fwd(_one([0, 1]), _one([1, 0]), _one([0, 0]), _one([0, 0]), _one([0.5, 0.5]),
                           _one([1, 1]), np.array([0.2]), np.eye(2).reshape(1, 1, 2, 2))
    M = Mt[0, 0].T                                      # back to the notes' orientation
    np.testing.assert_allclose(M, [[0.5, -0.1], [0.0, 1.0]], atol=1e-12)
    np.testing.assert_allclose(np.sort(np.linalg.eigvals(M).real), [0.5, 1.0], atol=1e-12)
    assert abs(np.linalg.norm(M @ np.array([0.0, 1.0])) - np.sqrt(1.01)) < 1e-12


def test_gdn2_with_scalar_gates_is_gated_deltanet():
    """§2.1 with b = w = beta 1, Diag(exp g) = alpha I and lambda_h = 0 is Gated DeltaNet:
    the Q-Delta oracle at lambda = 0 (whose own pins fix it) gives the same o and S_T."""
    B, T, H, dk, dv = 2, 40, 2, 8, 5
    q, k, v, _, _, _, _, S0 = _rand(B, T, H, dk, dv, seed=6)
    r = np.random.default_rng(7)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    alpha = np.exp(-np.log1p(np.exp(r.standard_normal((B, T, H)) - 2.0)))
    g = np.repeat(np.log(alpha)[..., None], dk, axis=-1)
    o1, S1 = oracle.qed_fwd(q, k, v, g, np.repeat(beta[..., None], dk, -1), np.repeat(beta[..., None], dv, -1),
                            np.zeros(H), S0)
    o2, S2 = oracle.qdelta_fwd(q, k, v, alpha, beta, None, S0)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(S1, S2, atol=1e-12)


def test_key_orthogonal_probe_unchanged():
    """Eq. (9): the step changes S by r k^T, so a probe x orthogonal to k sees
    S_t x = S_bar x (no decay here, g = 0), for QED as for GDN-2."""
    q, k, v, g, b, w, lam, S0 = _rand(1, 1, 1, 6, 4, seed=12)
    kk = k[0, 0, 0]
    x = np.random.default_rng(1).standard_normal(6)
    x -= kk * (kk @ x)
    _, S = oracle.qed_fwd(q, k, v, np.zeros_like(g), b, w, np.array([0.2]), S0)
    np.testing.assert_allclose(S[0, 0] @ x, S0[0, 0] @ x, atol=1e-13)


# ---------------------------------------------------------------- planted mistakes
import ctypes
import subprocess
import tempfile

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qdelta_oracle.c")
QED_MUTANTS = {
    "project_before_gating": ("for (j = 0; j < dk; ++j) u[j] = bt[j] * qt[j];", "for (j = 0; j < dk; ++j) u[j] = qt[j];"),
    "no_projection": ("lam_h[h] * (u[j] - kt[j] * ku)", "lam_h[h] * u[j]"),
    "lambda_sign": ("bt[j] * kt[j] + lam_h[h] * (u[j]", "bt[j] * kt[j] - lam_h[h] * (u[j]"),
    "erase_ungated": ("a[j] = bt[j] * kt[j] + lam_h", "a[j] = kt[j] + lam_h"),
    "decay_after_read": ("for (j = 0; j < dk; ++j) s[j] = s[j] * exp(gt[j]);              /* S_bar */\n"
                         "            for (j = 0; j < dk; ++j) pred += s[j] * a[j];                     /* (S_bar a)_i */",
                         "for (j = 0; j < dk; ++j) pred += s[j] * a[j];\n"
                         "            for (j = 0; j < dk; ++j) s[j] = s[j] * exp(gt[j]);"),
    "write_gate_dropped": ("r = w[tok * dv + i] * v[tok * dv + i] - pred;", "r = v[tok * dv + i] - pred;"),
    "write_along_a": ("s[j] = s[j] + r * kt[j];                 /* + r k^T */", "s[j] = s[j] + r * a[j];"),
    "readout_before_write": ("for (j = 0; j < dk; ++j) s[j] = s[j] + r * kt[j];                 /* + r k^T */\n"
                             "            for (j = 0; j < dk; ++j) out += s[j] * qt[j];",
                             "for (j = 0; j < dk; ++j) out += s[j] * qt[j];\n"
                             "            for (j = 0; j < dk; ++j) s[j] = s[j] + r * kt[j];"),
}


def _run_qed_lib(lib, x):
    q, k, v, g, b, w, lam, S0 = (None if t is None else np.ascontiguousarray(t, dtype=float) for t in x)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o, S = np.empty((B, T, H, dv)), np.empty((B, H, dv, dk))
    dp = ctypes.POINTER(ctypes.c_double)
    p = lambda z: None if z is None else z.ctypes.data_as(dp)
    assert lib.oracle_qed_fwd(p(q), p(k), p(v), p(g), p(b), p(w), p(lam), p(S0), p(o), p(S), B, T, H, dk, dv, 1) == 0
    return o, S


def _pins_pass(lib):
    """The pins above, restated against a given build of the C source."""
    ex = json.load(open(GOLDEN))
    i, pr = ex["inputs"], ex["printed"]
    S_bar = np.array(i["S_bar"]).reshape(1, 1, 1, 2)
    o1, S1 = _run_qed_lib(lib, (_one(i["q"]), _one(i["k"]), _one([i["w_times_v"]]), _one([0.0, 0.0]), _one(i["b"]),
                                _one([1.0]), np.array([i["lambda"]]), S_bar))
    if abs(o1.item() - pr["output_new"]) > 1e-12 or np.abs(S1.ravel() - pr["S_new"]).max() > 1e-12:
        return False
    q, k, v, g, b, w, lam, S0 = _rand(1, 1, 3, 7, 5, seed=4)
    o_q, S_q = _run_qed_lib(lib, (q, k, v, g, b, w, lam, S0))
    o_g, S_g = _run_qed_lib(lib, (q, k, v, g, b, w, np.zeros_like(lam), S0))
    for h in range(3):
        Sbar = S0[0, h] * np.exp(g[0, 0, h])[None, :]
        kk, qq, bb = k[0, 0, h], q[0, 0, h], b[0, 0, h]
        d = bb * qq - kk * (kk @ (bb * qq))
        if np.abs(S_q[0, h] - S_g[0, h] + lam[h] * np.outer(Sbar @ d, kk)).max() > 1e-12:
            return False
        if np.abs(o_q[0, 0, h] - o_g[0, 0, h] + lam[h] * (qq @ kk) * (Sbar @ d)).max() > 1e-12:
            return False
    # GDN-2 with scalar gates against the Q-Delta oracle at lambda = 0, with decay
    B, T, H, dk, dv = 1, 12, 2, 6, 4
    q, k, v, _, _, _, _, S0 = _rand(B, T, H, dk, dv, seed=6)
    rr = np.random.default_rng(7)
    beta = 1.0 / (1.0 + np.exp(-rr.standard_normal((B, T, H))))
    alpha = np.exp(-np.log1p(np.exp(rr.standard_normal((B, T, H)) - 2.0)))
    o1, S1 = _run_qed_lib(lib, (q, k, v, np.repeat(np.log(alpha)[..., None], dk, -1),
                                np.repeat(beta[..., None], dk, -1), np.repeat(beta[..., None], dv, -1),
                                np.zeros(H), S0))
    o2, S2 = oracle.qdelta_fwd(q, k, v, alpha, beta, None, S0)
    return np.abs(o1 - o2).max() < 1e-12 and np.abs(S1 - S2).max() < 1e-12


def test_qed_pins_reject_planted_mistakes():
    text = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        def build(t, name):
            c, so = os.path.join(tmp, name + ".c"), os.path.join(tmp, name + ".so")
            open(c, "w").write(t)
            subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                            c, "-lm"], check=True)
            lib = ctypes.CDLL(so)
            lib.oracle_qed_fwd.restype = ctypes.c_int
            lib.oracle_qed_fwd.argtypes = [ctypes.POINTER(ctypes.c_double)] * 10 + [ctypes.c_int] * 6
            return lib
        assert _pins_pass(build(text, "clean"))
        for name, (old, new) in QED_MUTANTS.items():
            assert text.count(old) == 1, name
            assert not _pins_pass(build(text.replace(old, new), name)), name
