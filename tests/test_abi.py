"""CPU checks of the C ABI: the library loads, exports every function include/qdelta.h
declares, and rejects bad arguments on the host before any device work is enqueued.
No call here reaches a kernel, so these run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdelta.h")

QD_OK, QD_ERR_INVALID_ARG, QD_ERR_UNSUPPORTED, QD_ERR_WORKSPACE, QD_ERR_HIP = range(5)


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
    for s in range(5):
        assert lib.qdelta_status_string(s)
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
