"""Edge cases of the forward kernels on the GPU: the chunked kernel's decay-range status, grids
far wider than the chip, a long sequence, and wide v4 rows (both of its load paths).

Inputs as the parity tests (seeded; r, k, v ~ N(0, 0.5), u ~ N(0, 0.5), decay parameter
~ U(-6, 0) unless a test says otherwise); every result is compared with the fp64 oracle on the
same inputs, to the bf16-input tolerance (max abs 2e-2, mean abs 5e-3) or, for fp32 inputs, the
fp32 one (max error relative to max(|o|, rms(o)) 2e-5).
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import assert_bf16, assert_fp32, dev, host
from wkv_inputs import wkv4_inputs, wkv6_inputs

pytestmark = pytest.mark.gpu


def _run6(inp, algo, status=None, state=None):
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), inp["H"]]
    return wkv.wkv6_forward(*args, algo=algo, state=state, dev_status=status)


def test_chunked_decay_range_status():
    """Per-token decays of exp(-exp(x)) with x in (1, 4) accumulate far more than the chunked
    kernel's exponent range within a 64-token chunk: the call sets WKV_DEV_DECAY_RANGE (its
    outputs are then not to be used), while the scan on the same inputs matches the oracle and
    sets nothing.  Ordinary decays set no bit."""
    inp = wkv6_inputs(2, 130, 2, 64, seed=41, x_range=(1.0, 4.0))
    st_chunked = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_scan = torch.zeros(1, dtype=torch.int32, device="cuda")
    _run6(inp, "chunked", st_chunked)
    y, S = _run6(inp, "scan", st_scan)
    torch.cuda.synchronize()
    assert int(st_chunked.item()) & wkv.WKV_DEV_DECAY_RANGE
    assert int(st_scan.item()) == 0
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64)
    assert_bf16(host(y), yo, "scan y, strong decay")
    assert_bf16(host(S), So, "scan state, strong decay")
    ok = torch.zeros(1, dtype=torch.int32, device="cuda")
    _run6(wkv6_inputs(2, 130, 2, 64, seed=42), "chunked", ok)
    torch.cuda.synchronize()
    assert int(ok.item()) == 0


@pytest.mark.parametrize("algo", ["scan", "chunked"])
def test_wide_grid(algo):
    """300 batch rows x 3 heads (900 workgroups, several per CU) with a ragged last chunk and
    mapped initial states; sampled (row, head) units against the oracle."""
    B, T, H = 300, 70, 3
    inp = wkv6_inputs(B, T, H, 64, seed=43, init_state=7)
    rng = np.random.default_rng(5)
    smap = rng.integers(0, 7, size=B).astype(np.int32)
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    y, S = wkv.wkv6_forward(*args, state=dev(inp["state"]), state_map=dev(smap), algo=algo)
    torch.cuda.synchronize()
    units = [(0, 0), (1, 2), (150, 1), (298, 0), (299, 2)]
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, 64, state=inp["state"],
                          state_map=smap, units=units)
    yh, Sh = host(y), host(S)
    for b, h in units:
        assert_bf16(yh[b, :, h * 64:(h + 1) * 64], yo[b, :, h * 64:(h + 1) * 64], f"y unit {(b, h)}")
        assert_bf16(Sh[b, h], So[b, h], f"state unit {(b, h)}")


@pytest.mark.parametrize("algo", ["scan", "chunked"])
def test_long_sequence(algo):
    """One head over 16384 tokens (256 chunks, 512 scan blocks) in one call."""
    inp = wkv6_inputs(1, 16384, 1, 64, seed=44)
    y, S = _run6(inp, algo)
    torch.cuda.synchronize()
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 1, 64)
    assert_bf16(host(y), yo, f"{algo} y, T=16384")
    assert_bf16(host(S), So, f"{algo} state, T=16384")
    # far inside the tolerance: no drift over the long carry
    assert np.max(np.abs(host(y) - yo)) < 1e-3


@pytest.mark.parametrize("C", [19200, 19190])
def test_v4_wide_rows(C):
    """v4 rows of 19200 channels (300 channel blocks, straight-line load path) and 19190 (the last
    block partly past the row: guarded path), fp32 with the sigmoid(r) gate and a carried state."""
    inp = wkv4_inputs(2, 40, C, seed=45, with_r=True, init_state=True)
    s = inp["state"].astype(np.float64)
    A0, B0 = s[:, 0] * np.exp(s[:, 2]), s[:, 1] * np.exp(s[:, 2])
    y, st = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["r"]),
                             state=dev(inp["state"]))
    torch.cuda.synchronize()
    yo, Ao, Bo = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"], A0, B0)
    assert_fp32(host(y), yo, f"v4 y C={C}")
    sh = host(st)
    assert_fp32(sh[:, 0] * np.exp(sh[:, 2]) / (sh[:, 1] * np.exp(sh[:, 2])), Ao / Bo, f"v4 A/B C={C}")
