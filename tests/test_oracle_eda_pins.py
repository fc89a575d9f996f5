"""Pins of the Erase-then-Delta oracle (``oracle.eda_fwd``) against what the EDA
explainer's pseudo-code fixes (page "Erase-then-Delta Attention", core method):

  * step 1 zeroes the state's component along the unit erase direction e: one step
    with k orthogonal to e leaves S_t e = 0;
  * step 2 is the delta write with no beta: with unit k, S_t k = v exactly;
  * with e = 0 (nothing erased) the rule is DeltaNet at beta = 1, which the Q-Delta
    oracle (pinned separately) computes at alpha = 1, lambda = 0;
  * the erase is the delta rule with key e, value 0 and beta = 1, so EDA equals DeltaNet
    run over the interleaved sequence e_1, k_1, e_2, k_2, ... (values 0 at the erase
    tokens), read at the k tokens: the reduction the library's chunk forward uses.
  * planted mistakes in a copy of the oracle are rejected by these pins.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qdelta_oracle.c")


def _rand(B, T, H, dk, dv, seed):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    e = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    S0 = 0.3 * r.standard_normal((B, H, dv, dk))
    return q, k, v, e, S0


def interleaved(q, k, v, e):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    q2 = np.zeros((B, 2 * T, H, dk)); k2 = np.zeros((B, 2 * T, H, dk)); v2 = np.zeros((B, 2 * T, H, dv))
    q2[:, 0::2], q2[:, 1::2] = q, q
    k2[:, 0::2], k2[:, 1::2] = e, k
    v2[:, 1::2] = v
    return q2, k2, v2


def test_erase_zeroes_component_along_e(eda=oracle.eda_fwd):
    q, k, v, e, S0 = _rand(1, 1, 2, 6, 4, seed=3)
    k = k - np.sum(k * e, -1, keepdims=True) * e
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    _, S = eda(q, k, v, e, S0)
    for h in range(2):
        np.testing.assert_allclose(S[0, h] @ e[0, 0, h], 0.0, atol=1e-13)


def test_delta_write_stores_v_along_k(eda=oracle.eda_fwd):
    q, k, v, e, S0 = _rand(1, 1, 2, 6, 4, seed=4)
    o, S = eda(q, k, v, e, S0)
    for h in range(2):
        np.testing.assert_allclose(S[0, h] @ k[0, 0, h], v[0, 0, h], atol=1e-13)
        np.testing.assert_allclose(o[0, 0, h], S[0, h] @ q[0, 0, h], atol=1e-13)


def test_no_erase_is_deltanet_beta_one(eda=oracle.eda_fwd):
    q, k, v, e, S0 = _rand(2, 30, 2, 8, 5, seed=5)
    o1, S1 = eda(q, k, v, np.zeros_like(e), S0)
    o2, S2 = oracle.qdelta_fwd(q, k, v, None, np.ones(q.shape[:3]), None, S0)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(S1, S2, atol=1e-12)


def test_eda_is_deltanet_on_the_interleaved_sequence(eda=oracle.eda_fwd):
    q, k, v, e, S0 = _rand(2, 40, 2, 8, 5, seed=6)
    o1, S1 = eda(q, k, v, e, S0)
    q2, k2, v2 = interleaved(q, k, v, e)
    o2, S2 = oracle.qdelta_fwd(q2, k2, v2, None, np.ones(q2.shape[:3]), None, S0)
    np.testing.assert_allclose(o1, o2[:, 1::2], atol=1e-12)
    np.testing.assert_allclose(S1, S2, atol=1e-12)


EDA_MUTANTS = {
    # the write applied first, then the erase: S (I - k k^T) + v k^T, then times (I - e e^T)
    "write_before_erase": ("            const double coef_k = v[tok * dv + i] - sk + se * ek;\n"
                           "            for (j = 0; j < dk; ++j) s[j] = s[j] - se * et[j] + coef_k * kt[j];",
                           "            const double coef_k = v[tok * dv + i] - sk;\n"
                           "            for (j = 0; j < dk; ++j) s[j] = s[j] + coef_k * kt[j];\n"
                           "            { const double se2 = dot(s, et, dk); for (j = 0; j < dk; ++j) s[j] -= se2 * et[j]; }"),
    "erase_along_k": ("s[j] = s[j] - se * et[j]", "s[j] = s[j] - se * kt[j]"),
    # the delta write's error read from the state before the erase (the cross term dropped)
    "error_from_pre_erase_state": ("v[tok * dv + i] - sk + se * ek;", "v[tok * dv + i] - sk;"),
    "cross_term_sign": ("v[tok * dv + i] - sk + se * ek;", "v[tok * dv + i] - sk - se * ek;"),
    "half_erase": ("s[j] = s[j] - se * et[j]", "s[j] = s[j] - 0.5 * se * et[j]"),
}


def test_eda_pins_reject_planted_mistakes():
    text = open(SRC).read()
    dp = ctypes.POINTER(ctypes.c_double)
    with tempfile.TemporaryDirectory() as tmp:
        def build(t, name):
            c, so = os.path.join(tmp, name + ".c"), os.path.join(tmp, name + ".so")
            open(c, "w").write(t)
            subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so,
                            c, "-lm"], check=True)
            lib = ctypes.CDLL(so)
            lib.oracle_eda_fwd.restype = ctypes.c_int
            lib.oracle_eda_fwd.argtypes = [dp] * 7 + [ctypes.c_int] * 6

            def eda(q, k, v, e, S0):
                q, k, v, e, S0 = (np.ascontiguousarray(x, dtype=float) for x in (q, k, v, e, S0))
                B, T, H, dk = q.shape
                dv = v.shape[-1]
                o, S = np.empty((B, T, H, dv)), np.empty((B, H, dv, dk))
                p = lambda z: z.ctypes.data_as(dp)
                assert lib.oracle_eda_fwd(p(q), p(k), p(v), p(e), p(S0), p(o), p(S), B, T, H, dk, dv, 1) == 0
                return o, S
            return eda

        def passes(eda):
            try:
                for f in (test_erase_zeroes_component_along_e, test_delta_write_stores_v_along_k,
                          test_no_erase_is_deltanet_beta_one, test_eda_is_deltanet_on_the_interleaved_sequence):
                    f(eda)
                return True
            except AssertionError:
                return False
        assert passes(build(text, "clean"))
        for name, (old, new) in EDA_MUTANTS.items():
            assert text.count(old) == 1, name
            assert not passes(build(text.replace(old, new), name)), name
