"""The oracle's pins are discriminating: plant plausible mistakes in a copy of the
oracle source (on the CPU, in a temporary directory), build each mutant, and check
that the independent reference checks reject every one of them while accepting the
unmodified source."""
import ctypes
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qdelta_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden", "qed_2d_example.json")
_dp = ctypes.POINTER(ctypes.c_double)

MUTANTS = {
    # the decay multiplies the whole transition: dropping it from the feedback term
    "feedback_not_decayed": [("alpha * (s[j] - beta * s_read * write[j])", "alpha * s[j] - beta * s_read * write[j]")],
    "write_term_decayed": [("+ beta * v_i * write[j]", "+ alpha * beta * v_i * write[j]")],
    "lambda_sign": [("x[j] = kt[j] + la * qt[j];   /* x_t", "x[j] = kt[j] - la * qt[j];   /* x_t")],
    "lambda_dropped": [("x[j] = kt[j] + la * qt[j];   /* x_t", "x[j] = kt[j] + 0.0 * la * qt[j];   /* x_t")],
    "lambda_normalised": [("x[j] = kt[j] + la * qt[j];   /* x_t",
                           "x[j] = (kt[j] + la * qt[j]) / (1.0 + la);   /* x_t")],
    "write_along_x": [("gated_row_update(s, x, kt, v[tok * dv + i]", "gated_row_update(s, x, x, v[tok * dv + i]")],
    "read_along_k": [("gated_row_update(s, x, kt, v[tok * dv + i]", "gated_row_update(s, kt, kt, v[tok * dv + i]")],
    "readout_along_read_dir": [("o[tok * dv + i] = dot(s, qt, dk);          /* o_t",
                                "o[tok * dv + i] = dot(s, x, dk);          /* o_t"),
                               ("if (o) o[i] = dot(s, q, dk);", "if (o) o[i] = dot(s, read, dk);")],
    "feedback_sign": [("(s[j] - beta * s_read * write[j])", "(s[j] + beta * s_read * write[j])")],
    "readout_before_write": [
        ("            gated_row_update(s, x, kt, v[tok * dv + i], a, be, dk);\n"
         "            if (o) o[tok * dv + i] = dot(s, qt, dk);          /* o_t = S_t q_t */\n",
         "            if (o) o[tok * dv + i] = dot(s, qt, dk);\n"
         "            gated_row_update(s, x, kt, v[tok * dv + i], a, be, dk);\n")],
    "beta_dropped": [("+ beta * v_i * write[j]", "+ v_i * write[j]")],
}


def _build(src_text, tmp, name):
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    open(c, "w").write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", so, c], check=True)
    lib = ctypes.CDLL(so)
    lib.oracle_qdelta_fwd.restype = ctypes.c_int
    lib.oracle_qdelta_fwd.argtypes = [_dp] * 9 + [ctypes.c_int] * 6
    lib.oracle_step_rw.restype = None
    lib.oracle_step_rw.argtypes = [_dp] * 5 + [ctypes.c_double, ctypes.c_double, _dp,
                                                ctypes.c_int, ctypes.c_int]
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _fwd(lib, q, k, v, a, be, la, S0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv)); S = np.empty((B, H, dv, dk))
    args = [np.ascontiguousarray(x) if x is not None else None for x in (q, k, v, a, be, la, S0)]
    assert lib.oracle_qdelta_fwd(*[_p(x) for x in args], _p(o), _p(S), B, T, H, dk, dv, 1) == 0
    return o, S


def _checks(lib):
    """Return the list of reference checks that fail for the oracle library lib."""
    failed = []
    r = np.random.default_rng(99)
    T, dk, dv = 12, 5, 4
    q = r.standard_normal((1, T, 1, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((1, T, 1, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((1, T, 1, dv))
    be = r.uniform(0.2, 0.9, (1, T, 1)); a = r.uniform(0.6, 0.99, (1, T, 1))
    la = r.uniform(0.1, 0.9, (1, T, 1)); S0 = 0.5 * r.standard_normal((1, 1, dv, dk))
    I = np.eye(dk)

    def ref(use_a, use_la):
        S = S0[0, 0].copy(); os_ = []
        for t in range(T):
            kt, qt = k[0, t, 0], q[0, t, 0]
            al = a[0, t, 0] if use_a else 1.0
            x = kt + (la[0, t, 0] if use_la else 0.0) * qt
            S = al * S @ (I - be[0, t, 0] * np.outer(x, kt)) + be[0, t, 0] * np.outer(v[0, t, 0], kt)
            os_.append(S @ qt)
        return np.array(os_), S

    for name, (ua, ul) in {"deltanet": (False, False), "gdn": (True, False), "full": (True, True)}.items():
        o, S = _fwd(lib, q, k, v, a if ua else None, be, la if ul else None, S0)
        oref, Sref = ref(ua, ul)
        if not (np.allclose(o[0, :, 0], oref, atol=1e-11) and np.allclose(S[0, 0], Sref, atol=1e-11)):
            failed.append(name)
    # the hand-computed 2-D step
    o, S = _fwd(lib, np.array([0.6, 0.8]).reshape(1, 1, 1, 2), np.array([1.0, 0.0]).reshape(1, 1, 1, 2),
                np.array([2.0]).reshape(1, 1, 1, 1), np.array([[[0.5]]]), np.array([[[0.5]]]),
                np.array([[[0.5]]]), np.array([2.0, 3.0]).reshape(1, 1, 1, 2))
    if not (abs(o[0, 0, 0, 0] - 1.83) < 1e-12 and np.allclose(S[0, 0, 0], [1.05, 1.5], atol=1e-12)):
        failed.append("hand_2d")
    # the QED page's printed example through the explicit read/write step
    ex = json.load(open(GOLDEN))
    inp, pr = ex["inputs"], ex["printed"]
    kk = np.array(inp["k"]); qq = np.array(inp["q"]); b = np.array(inp["b"])
    u = b * qq; d = u - kk * (kk @ u); read = b * kk + inp["lambda"] * d
    S = np.array([inp["S_bar"]], dtype=np.float64); o = np.empty(1)
    lib.oracle_step_rw(_p(S), _p(read), _p(kk), _p(np.array([inp["w_times_v"]])), _p(qq),
                       1.0, 1.0, _p(o), 2, 1)
    if not (abs(o[0] - pr["output_new"]) < 1e-12 and np.allclose(S[0], pr["S_new"], atol=1e-12)):
        failed.append("qed_printed")
    return failed


def test_unmodified_oracle_passes_all_checks():
    with tempfile.TemporaryDirectory() as tmp:
        assert _checks(_build(open(SRC).read(), tmp, "orig")) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(mutant):
    text = open(SRC).read()
    for old, new in MUTANTS[mutant]:
        assert old in text, f"mutation anchor missing: {old!r}"
        text = text.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        failed = _checks(_build(text, tmp, mutant))
    assert failed, f"mutant {mutant} passed every reference check"
