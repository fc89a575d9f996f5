"""CPU checks of the C ABI: the library loads, exports every function include/qdelta.h
declares, and rejects bad arguments on the host before any device work is enqueued.
No call here reaches a kernel, so these run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdelta.h")

QD_OK, QD_ERR_INVALID_ARG, QD_ERR_UNSUPPORTED, QD_ERR_WORKSPACE, QD_ERR_HIP, QD_ERR_SCRATCH_LIMIT = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdelta_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import recurrent_sequence_layers_amd as qd
    return qd.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qdelta_chunk_fwd", "qdelta_step", "qdelta_chunk_fwd_workspace_bytes",
              "qdelta_status_string", "qdelta_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libqdelta.so does not export {n}"


def test_version_and_status_strings(lib):
    hdr = open(HEADER).read()
    ver = int(re.search(r"#define QDELTA_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.qdelta_abi_version() == ver
    for s in range(6):
        assert lib.qdelta_status_string(s) and b"unknown" not in lib.qdelta_status_string(s)
    assert b"unknown" in lib.qdelta_status_string(99)
    assert lib.qdelta_chunk_fwd_workspace_bytes(8, 4096, 16, 128, 128, 64, 1) == 0


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on these paths


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, alpha=None, beta=FAKE * 4, lam=None, S0=None,
             o=FAKE * 5, S_T=None, B=1, T=4, H=1, d_k=64, d_v=64, C=64, dtype=1, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.qdelta_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["lam"], a["S0"], a["o"],
                                a["S_T"], a["B"], a["T"], a["H"], a["d_k"], a["d_v"], a["C"], a["dtype"],
                                a["ws"], a["ws_bytes"], None)


def test_chunk_fwd_host_side_rejections(lib):
    assert _fwd(lib, d_k=96) == QD_ERR_UNSUPPORTED
    assert _fwd(lib, d_v=256) == QD_ERR_UNSUPPORTED
    assert _fwd(lib, C=48) == QD_ERR_UNSUPPORTED
    assert _fwd(lib, dtype=7) == QD_ERR_UNSUPPORTED
    assert _fwd(lib, B=-1) == QD_ERR_INVALID_ARG
    assert _fwd(lib, T=-3) == QD_ERR_INVALID_ARG
    assert _fwd(lib, q=None) == QD_ERR_INVALID_ARG
    assert _fwd(lib, beta=None) == QD_ERR_INVALID_ARG
    assert _fwd(lib, o=None) == QD_ERR_INVALID_ARG
    assert _fwd(lib, q=FAKE + 2) == QD_ERR_INVALID_ARG            # misaligned
    assert _fwd(lib, o=FAKE) == QD_ERR_INVALID_ARG                # output aliases q
    assert _fwd(lib, S0=FAKE * 64, S_T=FAKE * 64 + 16) == QD_ERR_INVALID_ARG  # partial state overlap
    # nothing to do: B*H == 0 returns OK without launching
    assert _fwd(lib, B=0) == QD_OK
    assert _fwd(lib, H=0, q=None, o=None) == QD_OK


def _step(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, alpha=None, beta=FAKE * 4, lam=None, S=FAKE * 64, o=FAKE * 5,
             N=2, H=2, d_k=128, d_v=128, dtype=1)
    a.update(kw)
    return lib.qdelta_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["lam"], a["S"], a["o"],
                           a["N"], a["H"], a["d_k"], a["d_v"], a["dtype"], None)


def test_step_host_side_rejections(lib):
    assert _step(lib, d_k=32) == QD_ERR_UNSUPPORTED
    assert _step(lib, dtype=3) == QD_ERR_UNSUPPORTED
    assert _step(lib, N=-1) == QD_ERR_INVALID_ARG
    assert _step(lib, S=None) == QD_ERR_INVALID_ARG
    assert _step(lib, S=FAKE * 64 + 4) == QD_ERR_INVALID_ARG
    assert _step(lib, o=FAKE * 64 + 256) == QD_ERR_INVALID_ARG    # output inside the state
    assert _step(lib, N=0) == QD_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import recurrent_sequence_layers_amd as qd
    monkeypatch.setattr(qd, "_lib", None)
    monkeypatch.setattr(qd, "LIB_PATH", str(tmp_path / "libqdelta.so"))
    with pytest.raises(qd.QDeltaError):
        qd.load_library()


# ---------------------------------------------------------------- backward, QED, EDA entry points
def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, alpha=FAKE * 4, beta=FAKE * 5, lam=FAKE * 6, S0=None, d_o=FAKE * 7,
             dS_T=None, dq=FAKE * 8, dk=FAKE * 9, dv=FAKE * 10, dalpha=FAKE * 11, dbeta=FAKE * 12, dlam=FAKE * 13,
             dS0=None, B=1, T=4, H=1, d_k=64, d_v=64, C=32, dtype=1, ws=FAKE * 64, ws_bytes=1 << 20)
    a.update(kw)
    return lib.qdelta_chunk_bwd(*[a[n] for n in ("q", "k", "v", "alpha", "beta", "lam", "S0", "d_o", "dS_T", "dq",
                                                 "dk", "dv", "dalpha", "dbeta", "dlam", "dS0")],
                                a["B"], a["T"], a["H"], a["d_k"], a["d_v"], a["C"], a["dtype"], a["ws"],
                                a["ws_bytes"], None)


def test_chunk_bwd_host_side_rejections(lib):
    assert _bwd(lib, C=64, dtype=0) == QD_ERR_UNSUPPORTED          # fp32 at C = 64
    assert _bwd(lib, d_k=96) == QD_ERR_UNSUPPORTED
    assert _bwd(lib, T=-1) == QD_ERR_INVALID_ARG
    assert _bwd(lib, d_o=None) == QD_ERR_INVALID_ARG
    assert _bwd(lib, dbeta=None) == QD_ERR_INVALID_ARG
    assert _bwd(lib, alpha=None) == QD_ERR_INVALID_ARG             # dalpha given without alpha
    assert _bwd(lib, lam=None) == QD_ERR_INVALID_ARG               # dlambda given without lambda
    assert _bwd(lib, ws=None) == QD_ERR_WORKSPACE
    assert _bwd(lib, ws_bytes=16) == QD_ERR_WORKSPACE
    assert _bwd(lib, dq=FAKE) == QD_ERR_INVALID_ARG                # dq aliases q
    assert _bwd(lib, dk=FAKE * 8) == QD_ERR_INVALID_ARG            # dk aliases dq
    assert _bwd(lib, ws=FAKE * 9) == QD_ERR_INVALID_ARG            # workspace over dk
    assert _bwd(lib, B=0) == QD_OK


def test_chunk_bwd_workspace_formula(lib):
    # entry states and exit-state gradients per chunk, in the element type
    assert lib.qdelta_chunk_bwd_workspace_bytes(2, 100, 3, 64, 128, 32, 1) == 2 * 3 * 4 * 2 * 128 * 64 * 2
    assert lib.qdelta_chunk_bwd_workspace_bytes(2, 100, 3, 64, 128, 32, 0) == 2 * 3 * 4 * 2 * 128 * 64 * 4
    assert lib.qdelta_chunk_bwd_workspace_bytes(2, 0, 3, 64, 128, 32, 1) == 0
    assert lib.qdelta_chunk_bwd_workspace_bytes(2, 100, 3, 64, 128, 64, 0) == 0      # unsupported


def _qed(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, b=FAKE * 5, w=FAKE * 6, lam=FAKE * 7, S0=None, o=FAKE * 8,
             S_T=None, B=1, T=4, H=1, d_k=64, d_v=64, C=32, dtype=1)
    a.update(kw)
    return lib.qdelta_qed_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["b"], a["w"], a["lam"], a["S0"], a["o"],
                                    a["S_T"], a["B"], a["T"], a["H"], a["d_k"], a["d_v"], a["C"], a["dtype"], None)


def test_qed_host_side_rejections(lib):
    assert _qed(lib, C=64) == QD_ERR_UNSUPPORTED
    assert _qed(lib, C=32, dtype=0) == QD_ERR_UNSUPPORTED
    assert _qed(lib, lam=None) == QD_ERR_INVALID_ARG
    assert _qed(lib, g=None) == QD_ERR_INVALID_ARG
    assert _qed(lib, g=FAKE * 4 + 4) == QD_ERR_INVALID_ARG         # misaligned gate rows
    assert _qed(lib, o=FAKE * 6) == QD_ERR_INVALID_ARG             # o aliases w
    assert _qed(lib, B=0) == QD_OK
    assert lib.qdelta_qed_step(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6, None, FAKE * 64, FAKE * 8,
                               2, 2, 64, 64, 1, None) == QD_ERR_INVALID_ARG
    assert lib.qdelta_qed_step(FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 64,
                               FAKE * 8, 0, 2, 64, 64, 1, None) == QD_OK


def _eda(lib, **kw):
    # fp32: the instance that builds the interleaved sequence in a workspace
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, e=FAKE * 4, S0=None, o=FAKE * 5, S_T=None, B=1, T=4, H=1, d_k=64,
             d_v=64, C=32, dtype=0, ws=FAKE * 64, ws_bytes=1 << 20)
    a.update(kw)
    return lib.qdelta_eda_chunk_fwd(a["q"], a["k"], a["v"], a["e"], a["S0"], a["o"], a["S_T"], a["B"], a["T"],
                                    a["H"], a["d_k"], a["d_v"], a["C"], a["dtype"], a["ws"], a["ws_bytes"], None)


def test_eda_host_side_rejections(lib):
    assert _eda(lib, e=None) == QD_ERR_INVALID_ARG
    assert _eda(lib, ws=None) == QD_ERR_WORKSPACE
    assert _eda(lib, o=FAKE * 4) == QD_ERR_INVALID_ARG             # o aliases e
    assert _eda(lib, C=48) == QD_ERR_UNSUPPORTED
    assert _eda(lib, B=0) == QD_OK
    assert _eda(lib, B=0, dtype=1, ws=None, ws_bytes=0) == QD_OK
    # the interleaved sequence and its outputs: 2 B T H ((2 d_k + 2 d_v) e + 4) bytes, the last term rounded up to 16
    assert lib.qdelta_eda_chunk_fwd_workspace_bytes(2, 10, 3, 64, 128, 32, 0) == 2 * 2 * 10 * 3 * ((2 * 64 + 2 * 128) * 4) + 480
    assert lib.qdelta_eda_chunk_fwd_workspace_bytes(2, 10, 3, 64, 128, 16, 1) == 2 * 2 * 10 * 3 * ((2 * 64 + 2 * 128) * 2) + 480
    # bf16 at C = 32, 64 reads the interleaved sequence in place
    assert lib.qdelta_eda_chunk_fwd_workspace_bytes(2, 10, 3, 64, 128, 32, 1) == 0
    assert lib.qdelta_eda_chunk_fwd_workspace_bytes(2, 10, 3, 128, 128, 64, 1) == 0
    assert lib.qdelta_eda_step(FAKE, FAKE * 2, FAKE * 3, None, FAKE * 64, FAKE * 5, 2, 2, 64, 64, 1, None) == QD_ERR_INVALID_ARG


def test_gate_arrays_are_part_of_the_disjointness_check(lib):
    """Every entry point checks each output against every input, the gate arrays
    included; a partial overlap with the state is rejected too."""
    # chunk forward: S_T over alpha, o over lambda, S_T over beta
    assert _fwd(lib, alpha=FAKE * 6, S_T=FAKE * 6) == QD_ERR_INVALID_ARG
    assert _fwd(lib, lam=FAKE * 7, o=FAKE * 7) == QD_ERR_INVALID_ARG
    assert _fwd(lib, S_T=FAKE * 4 - 1024) == QD_ERR_INVALID_ARG       # the state's span covers beta
    # decode step: the state over a gate, the output over a gate
    assert _step(lib, alpha=FAKE * 64 + 64) == QD_ERR_INVALID_ARG
    assert _step(lib, lam=FAKE * 5) == QD_ERR_INVALID_ARG
    # backward: the workspace over beta
    assert _bwd(lib, ws=FAKE * 5) == QD_ERR_INVALID_ARG
    # QED: S_T over the erase gate, and a partial overlap of S_T with S0
    assert _qed(lib, S_T=FAKE * 5) == QD_ERR_INVALID_ARG
    assert _qed(lib, S0=FAKE * 64, S_T=FAKE * 64 + 16) == QD_ERR_INVALID_ARG
    # EDA: the workspace over S0, S_T over q
    assert _eda(lib, S0=FAKE * 32, ws=FAKE * 32) == QD_ERR_INVALID_ARG
    assert _eda(lib, S_T=FAKE) == QD_ERR_INVALID_ARG
