"""wkv6_backward_noalloc — the v6 backward for callers that cannot allocate device memory —
against wkv6_backward (the same kernels with a caller workspace for the du staging).

The two entry points run the same arithmetic in the same order (both take the "auto" choice:
the chunked passes for these bf16 inputs, then the sweeps for the units they leave), so their
results must be bitwise equal, which is stricter than the backward's parity bars.  Two
calls in a row go through the library's scratch, the second smaller than the first, so the
second reads none of the first call's staging.
"""
import numpy as np
import pytest
import torch

import rwkv_linear_attention_wkv_amd as wkv
from parity import dev
from wkv_inputs import bf16_round, wkv6_inputs, wkv6_upstream

pytestmark = pytest.mark.gpu


def _call(B, T, H, seed, library_scratch, strong_head=False):
    inp = wkv6_inputs(B, T, H, 64, seed=seed, init_state=B)
    if strong_head:  # head 0's decays beyond the chunked range: the sweeps redo those units
        inp["x"][:, :, :64] = bf16_round(np.random.default_rng(seed).random((B, T, 64), dtype=np.float32) * 3 + 1)
    up = wkv6_upstream(B, T, H, 64, seed=seed + 1)
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    st = dev(inp["state"])
    _, S = wkv.wkv6_forward(*args, state=st, algo="scan")
    return wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=dev(up["d_state"]),
                             library_scratch=library_scratch)


def test_noalloc_backward_matches_workspace_call():
    shapes = [(4, 300, 8, 70), (2, 77, 3, 72)]  # B*H*N = 2048, then 384
    ref = [_call(B, T, H, s, False) for B, T, H, s in shapes]
    got = [_call(B, T, H, s, True) for B, T, H, s in shapes]
    torch.cuda.synchronize()
    names = ("dr", "dk", "dv", "dw", "du", "d_state_in")
    for (B, T, H, _), a, b in zip(shapes, ref, got):
        for name, x, y in zip(names, a, b):
            assert torch.equal(x, y), f"B={B} T={T} H={H}: {name} differs from the workspace call"


def test_noalloc_backward_matches_with_units_left_to_the_sweeps():
    """Units the chunked passes leave to the sweeps stage their du rows in the library's array
    too; two calls in a row, the second smaller."""
    shapes = [(3, 200, 4, 80), (2, 70, 2, 81)]
    ref = [_call(B, T, H, s, False, strong_head=True) for B, T, H, s in shapes]
    got = [_call(B, T, H, s, True, strong_head=True) for B, T, H, s in shapes]
    torch.cuda.synchronize()
    names = ("dr", "dk", "dv", "dw", "du", "d_state_in")
    for (B, T, H, _), a, b in zip(shapes, ref, got):
        for name, x, y in zip(names, a, b):
            assert torch.equal(x, y), f"B={B} T={T} H={H}: {name} differs from the workspace call"


def test_noalloc_backward_rejects_calls_beyond_its_scratch():
    B, T, H = 1025, 1, 16  # B*H*N = 1,049,600 > 1,048,576
    z = torch.zeros((B, T, H * 64), dtype=torch.bfloat16, device="cuda")
    u = torch.zeros(H * 64, device="cuda")
    dy = torch.zeros((B, T, H * 64), device="cuda")
    with pytest.raises(wkv.WkvError, match="scratch"):
        wkv.wkv6_backward(z, z, z, z, u, H, dy, library_scratch=True)
