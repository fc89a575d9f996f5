"""qdelta_chunk_fwd_noalloc (through the C ABI) against qdelta_chunk_fwd with a caller
workspace: the same kernels and schedule, so the results must agree bitwise.  Two calls
in a row share the library's per-device scratch, the second on a smaller input, so a
stale scratch from the first would show in the second.  A single-pass shape, which needs
no scratch, and the no-op shapes go through too.

On a 256-CU device the segmented schedule never asks for more than 24 MiB (the product of
segments, batch and heads is capped at 256 * 64 / max(d_k, d_v), times
(d_k^2 + 2 d_v d_k) * 4 bytes per segment), under the 32 MiB the library holds, so the
QD_ERR_SCRATCH_LIMIT path cannot be reached on this hardware; it guards devices with more
compute units.
"""
import ctypes

import pytest
import torch

from recurrent_sequence_layers_amd import inputs

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _pair(qd, B, T, H, d, C, seed, expect_segmented):
    lib = qd.load_library()
    x = inputs.chunk_inputs(B, T, H, d, d, "bf16", seed=seed, s0_std=0.02, device="cuda")
    need = qd.qdelta_chunk_fwd_workspace_bytes(B, T, H, d, d, C, torch.bfloat16)
    print(f"noalloc B={B} T={T} H={H} d={d} C={C}: workspace of the allocating call {need} B", flush=True)
    assert (need > 0) == expect_segmented and need <= qd.NOALLOC_SCRATCH_BYTES
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o_ref = torch.empty_like(x.v)
    S_ref = torch.empty_like(x.S0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    rc = lib.qdelta_chunk_fwd(_p(x.q), _p(x.k), _p(x.v), _p(x.alpha), _p(x.beta), _p(x.lam), _p(x.S0), _p(o_ref),
                              _p(S_ref), B, T, H, d, d, C, 1, _p(ws), ws.numel(), stream)
    assert rc == 0, qd.qdelta_status_string(rc)
    o = torch.full_like(x.v, float("nan"))
    S = torch.full_like(x.S0, float("nan"))
    rc = lib.qdelta_chunk_fwd_noalloc(_p(x.q), _p(x.k), _p(x.v), _p(x.alpha), _p(x.beta), _p(x.lam), _p(x.S0),
                                      _p(o), _p(S), B, T, H, d, d, C, 1, stream)
    assert rc == 0, qd.qdelta_status_string(rc)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_matches_allocating_call_twice_then_smaller(qd):
    # the long-context workload (segmented, 24 MiB of scratch), then a smaller segmented
    # input that uses 3.1 MB of it
    _pair(qd, 1, 65536, 16, 128, 64, seed=501, expect_segmented=True)
    _pair(qd, 1, 8192, 4, 64, 64, seed=502, expect_segmented=True)


def test_noalloc_single_pass_and_empty(qd):
    _pair(qd, 2, 300, 3, 128, 64, seed=503, expect_segmented=False)
    lib = qd.load_library()
    # B * H == 0 is a no-op; invalid sizes are rejected on the host
    assert lib.qdelta_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, None,
                                        0, 10, 2, 128, 128, 64, 1, None) == 0
    assert lib.qdelta_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, None,
                                        1, 10, 2, 96, 128, 64, 1, None) == 2          # QD_ERR_UNSUPPORTED
