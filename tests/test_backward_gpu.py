"""v6 backward (wkv6_backward) against the fp64 oracle's reverse-mode gradients.

The oracle's gradients are pinned to central differences of its forward
(tests/test_oracle_pins.py).  The GPU sweeps compute in fp32.  Metric:
max |g - o| / max(|o|, rms(o)) per gradient.  dr, dk, dv, du and the state
gradient are single recurrences like the forward (measured about 1e-6 at
T=4096): bound 1e-4.  The decay gradient is the reverse running difference of
r * dr~ and k * dk~; each of those terms carries its own fp32 rounding (about
1e-6 relative) and their errors add up over the steps walked while the result
is a difference.  The walk restarts from its exact value sum_j G S every 256
tokens (the forward sweep keeps S there), so the error no longer grows with T:
bound 2e-4, checked up to T=16384 and on the restart edges.  With strong decays
(x up to 2, d_t down to exp(-7.4)) the difference cancels within one step as
well: dlam_t = d_t (sum_j G_t S_{t-1}) is small while its two terms are not,
and dx = -exp(x) dlam scales that error up: bound 1e-3 there.
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
DW_REL = 2e-4
DW_REL_STRONG = 1e-3  # decays down to exp(-exp(2)) per step


def _gpu(inp, up, state=None, state_map=None, with_dstate=True):
    H = inp["H"]
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    st = dev(state) if state is not None else None
    sm = dev(state_map) if state_map is not None else None
    _, S_final = wkv.wkv6_forward(*args, state=st, state_map=sm, algo="scan")
    ds = dev(up["d_state"]) if with_dstate else None
    return wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_map=sm,
                             state_final=S_final if with_dstate else None, d_state=ds)


def _check(got, ref, what, dw_bound=DW_REL):
    names = ("dr", "dk", "dv", "dw", "du", "d_state")
    for name, g, o in zip(names, got, ref):
        e = fp32_relerr(host(g), o)
        bound = dw_bound if name == "dw" else GRAD_REL
        print(f"{what} {name}: {e:.3e}")
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


def test_backward_bad_state_map_row_is_skipped():
    """A state_map entry out of range sets the status bit; that batch row's gradients are not
    written, and du sums the other rows only (its share is zero), matching the oracle run on the
    valid rows."""
    inp = wkv6_inputs(3, 70, 2, 64, seed=15, init_state=2)
    up = wkv6_upstream(3, 70, 2, 64, seed=16, with_state=False)
    smap = np.array([1, 7, 0], dtype=np.int32)
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), 2]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=dev(inp["state"]), state_map=dev(smap),
                            dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    good = [0, 2]
    sub = {n: inp[n][good] for n in ("r", "k", "v", "x")}
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(sub["r"], sub["k"], sub["v"], sub["x"], inp["u"], 2, 64,
                                                     up["dy"][good], state=inp["state"], state_map=smap[good])
    _check([t[good] for t in got[:4]] + [got[4], got[5][good]], (dr, dk, dv, dx, du, dS), "bad map row skipped")


def test_backward_zero_state_and_decay_extremes():
    for x_range in [(-6.0, 2.0), (-20.0, -10.0)]:
        inp = wkv6_inputs(2, 50, 2, 64, seed=9, dtype="f32", x_range=x_range)
        up = wkv6_upstream(2, 50, 2, 64, seed=10)
        got = _gpu(inp, up, with_dstate=False)  # no initial state, no final-state gradient
        torch.cuda.synchronize()
        dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64,
                                                         up["dy"])
        _check(got, (dr, dk, dv, dx, du, dS), f"x in {x_range}", DW_REL_STRONG if x_range[1] > 0 else DW_REL)


def test_backward_full_shape():
    """B=8 T=4096 H=32 N=64 (the headline forward shape): every (row, head) unit of every
    gradient, du included, against the oracle."""
    inp = wkv6_inputs(8, 4096, 32, 64, seed=0)
    up = wkv6_upstream(8, 4096, 32, 64, seed=1)
    got = _gpu(inp, up)
    torch.cuda.synchronize()
    ref = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 32, 64, up["dy"],
                               d_state_out=up["d_state"])
    _check(got, (*ref[:5], ref[6]), "B=8 T=4096 H=32")


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


@pytest.mark.parametrize("T,dtype,x_range", [(256, "bf16", None), (257, "f32", None), (1024, "bf16", None),
                                             (2100, "f32", (-6.0, 2.0)), (3103, "bf16", None)])
def test_backward_span_restarts(T, dtype, x_range):
    """T around multiples of the 256-token span at whose ends the decay-gradient walk restarts
    from sum_j G S: none (T=256), one right before the last token, several with a ragged first
    block of the dk/dw sweep, and strong decays (blocks that take the direct form) next to them."""
    kw = {} if x_range is None else {"x_range": x_range}
    inp = wkv6_inputs(2, T, 2, 64, seed=500 + T, dtype=dtype, init_state=2, **kw)
    up = wkv6_upstream(2, T, 2, 64, seed=600 + T)
    got = _gpu(inp, up, state=inp["state"])
    torch.cuda.synchronize()
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64,
                                                     up["dy"], state=inp["state"], d_state_out=up["d_state"])
    _check(got, (dr, dk, dv, dx, du, dS), f"T={T} {dtype}", DW_REL if x_range is None else DW_REL_STRONG)


def test_backward_long_sequence_dw():
    """T=16384 (four times the headline length): the decay gradient stays within 2e-4 (the walk
    restarts every 256 tokens instead of carrying its rounding over the whole sequence)."""
    inp = wkv6_inputs(1, 16384, 2, 64, seed=21, init_state=1)
    up = wkv6_upstream(1, 16384, 2, 64, seed=22)
    got = _gpu(inp, up, state=inp["state"])
    torch.cuda.synchronize()
    ref = oracle.wkv6_backward(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64, up["dy"],
                               state=inp["state"], d_state_out=up["d_state"])
    _check(got, (*ref[:5], ref[6]), "T=16384")
