"""v6 backward (wkv6_backward) against the fp64 oracle's reverse-mode gradients.

The oracle's gradients are pinned to central differences of its forward
(tests/test_oracle_pins.py).  The GPU sweeps compute in fp32.  Metric:
max |g - o| / max(|o|, rms(o)) per gradient.  dr, dk, dv, du and the state
gradient are single recurrences like the forward (measured about 1e-6 at
T=4096): bound 1e-4.  The decay gradient is the reverse running difference of
r * dr~ and k * dk~ over the rest of the sequence; each of those terms carries
its own fp32 rounding (about 1e-6 relative) and they add up over the
sequence while the result is a difference, so its relative error grows with
T over the decay window (measured 1.3e-4 at T=4096 on all 256 units): bound
1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import dev, fp32_relerr, host
from wkv_inputs import wkv6_inputs, wkv6_upstream

pytestmark = pytest.mark.gpu

GRAD_REL = 1e-4
DW_REL = 1e-3


def _gpu(inp, up, state=None, state_map=None, with_dstate=True):
    H = inp["H"]
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    st = dev(state) if state is not None else None
    sm = dev(state_map) if state_map is not None else None
    _, S_final = wkv.wkv6_forward(*args, state=st, state_map=sm, algo="scan")
    ds = dev(up["d_state"]) if with_dstate else None
    return wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_map=sm,
                             state_final=S_final if with_dstate else None, d_state=ds)


def _check(got, ref, what):
    names = ("dr", "dk", "dv", "dw", "du", "d_state")
    for name, g, o in zip(names, got, ref):
        e = fp32_relerr(host(g), o)
        bound = DW_REL if name == "dw" else GRAD_REL
        assert np.all(np.isfinite(host(g))), f"{what} {name}: non-finite"
        assert e <= bound, f"{what} {name}: relative error {e:.3e} > {bound}"


@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (37, "f32"), (100, "bf16"), (129, "f32")])
def test_backward_small(T, dtype):
    inp = wkv6_inputs(2, T, 2, 64, seed=300 + T, dtype=dtype, init_state=2)
    up = wkv6_upstream(2, T, 2, 64, seed=400 + T)
    got = _gpu(inp, up, state=inp["state"])
    torch.cuda.synchronize()
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64,
                                                     up["dy"], state=inp["state"], d_state_out=up["d_state"])
    _check(got, (dr, dk, dv, dx, du, dS), f"T={T} {dtype}")


def test_backward_no_state_gradient_and_mapped_state():
    inp = wkv6_inputs(3, 70, 1, 64, seed=5, init_state=2)
    up = wkv6_upstream(3, 70, 1, 64, seed=6, with_state=False)
    smap = np.array([1, 0, 1], dtype=np.int32)
    got = _gpu(inp, up, state=inp["state"], state_map=smap, with_dstate=False)
    torch.cuda.synchronize()
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 1, 64,
                                                     up["dy"], state=inp["state"], state_map=smap)
    _check(got, (dr, dk, dv, dx, du, dS), "mapped")


def test_backward_zero_state_and_decay_extremes():
    for x_range in [(-6.0, 2.0), (-20.0, -10.0)]:
        inp = wkv6_inputs(2, 50, 2, 64, seed=9, dtype="f32", x_range=x_range)
        up = wkv6_upstream(2, 50, 2, 64, seed=10)
        got = _gpu(inp, up, with_dstate=False)  # no initial state, no final-state gradient
        torch.cuda.synchronize()
        dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64,
                                                         up["dy"])
        _check(got, (dr, dk, dv, dx, du, dS), f"x in {x_range}")


def test_backward_full_shape_sampled():
    """B=8 T=4096 H=32 N=64 (the headline forward shape), checked on sampled (row, head) units."""
    inp = wkv6_inputs(8, 4096, 32, 64, seed=0)
    up = wkv6_upstream(8, 4096, 32, 64, seed=1)
    got = _gpu(inp, up)
    torch.cuda.synchronize()
    units = [(0, 0), (3, 17), (7, 31)]
    dr, dk, dv, dx, du, du_rows, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 32,
                                                           64, up["dy"], d_state_out=up["d_state"], units=units)
    g = [host(t) for t in got[:4]]
    for b, h in units:
        sl = (b, slice(None), slice(h * 64, (h + 1) * 64))
        for name, a, o in zip(("dr", "dk", "dv", "dw"), g, (dr, dk, dv, dx)):
            e = fp32_relerr(a[sl], o[sl])
            assert e <= (DW_REL if name == "dw" else GRAD_REL), f"unit {(b, h)} {name}: {e:.3e}"
        e = fp32_relerr(host(got[5])[b, h], dS[b, h])
        assert e <= GRAD_REL, f"unit {(b, h)} d_state: {e:.3e}"


def test_backward_deterministic_and_empty():
    inp = wkv6_inputs(2, 77, 2, 64, seed=12, init_state=2)
    up = wkv6_upstream(2, 77, 2, 64, seed=13)
    a = _gpu(inp, up, state=inp["state"])
    b = _gpu(inp, up, state=inp["state"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # T = 0: no token gradients, du = 0, the state gradient passes through unchanged
    inp0 = wkv6_inputs(2, 0, 2, 64, seed=1, init_state=2)
    up0 = wkv6_upstream(2, 0, 2, 64, seed=2)
    st = dev(inp0["state"])
    args = [dev(inp0[n]) for n in ("r", "k", "v", "x")] + [dev(inp0["u"]), 2]
    out = wkv.wkv6_backward(*args, dev(up0["dy"]), state=st, state_final=st, d_state=dev(up0["d_state"]))
    torch.cuda.synchronize()
    assert torch.equal(out[4], torch.zeros_like(out[4]))
    assert torch.equal(out[5], dev(up0["d_state"]))
