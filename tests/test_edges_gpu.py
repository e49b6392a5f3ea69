"""Edge cases of the forward kernels on the GPU: decays far outside the chunked form's exponent
range (its chunks then run the direct recurrence), grids far wider than the chip, a long
sequence, and wide v4 rows (both of its load paths).

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
from wkv_inputs import bf16_round, bf16_to_f32, wkv4_inputs, wkv5_inputs, wkv6_inputs

pytestmark = pytest.mark.gpu


def _run6(inp, algo, status=None, state=None):
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), inp["H"]]
    return wkv.wkv6_forward(*args, algo=algo, state=state, dev_status=status)


def _strong_decay_case(case):
    """Inputs whose decays reach far past the chunked form's exponent range in some or all of
    their 64-token chunks (the rwkv_ops page's RWKV6_OP call puts no range on w)."""
    if case == "strong":      # every chunk: per-step decay below exp(-e) = 0.066
        return wkv6_inputs(2, 130, 2, 64, seed=41, x_range=(1.0, 4.0), init_state=2)
    if case == "wide":        # some chunks only (an average exp(x) above ~1.08 over a chunk)
        return wkv6_inputs(2, 1000, 3, 64, seed=46, x_range=(-6.0, 2.0), init_state=2)
    inp = wkv6_inputs(2, 333, 2, 64, seed=47, init_state=2)
    x = bf16_to_f32(inp["x"]).copy()
    rng = np.random.default_rng(48)
    x[:, 64:128] = rng.uniform(1.0, 4.0, size=x[:, 64:128].shape)   # exactly chunk 1
    x[0, 200:211, :17] = 60.0    # decay underflows to 0 (exp(-exp(60)))
    x[1, 250:252] = 100.0        # exp(100) overflows fp32: decay exactly 0
    x[:, 320:] = rng.uniform(0.5, 3.0, size=x[:, 320:].shape)        # the ragged last chunk
    inp["x"] = bf16_round(x)
    return inp


@pytest.mark.parametrize("case", ["strong", "wide", "mixed"])
def test_chunked_any_decay_matches_oracle(case):
    """The default algorithm (chunked for bf16, T >= 64) on decays outside its exponent range:
    those chunks run the direct recurrence inside the kernel, so y and the final state match
    the oracle to the bf16-input tolerance, no status bit is set, and the result agrees with
    the scan."""
    inp = _strong_decay_case(case)
    H = inp["H"]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, S = _run6(inp, "auto", st, state=dev(inp["state"]))
    ys, Ss = _run6(inp, "scan", None, state=dev(inp["state"]))
    torch.cuda.synchronize()
    assert wkv.resolve_algo(6, inp["B"], inp["T"], H, 64) == "chunked"
    assert int(st.item()) == 0
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, 64, state=inp["state"])
    assert_bf16(host(y), yo, f"{case}: chunked y")
    assert_bf16(host(S), So, f"{case}: chunked state")
    assert_bf16(host(ys), yo, f"{case}: scan y")
    assert_bf16(host(y), host(ys), f"{case}: chunked vs scan y")


def test_chunked_direct_chunks_layouts_and_determinism():
    """Chunks that run directly give bitwise the same values in head-first layout, their bf16 y
    is the fp32 y rounded, and two runs are bitwise equal."""
    inp = _strong_decay_case("mixed")
    H, B, T = inp["H"], inp["B"], inp["T"]
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    y1, S1 = wkv.wkv6_forward(*args, state=dev(inp["state"]), algo="chunked")
    y2, S2 = wkv.wkv6_forward(*args, state=dev(inp["state"]), algo="chunked")
    yb, _ = wkv.wkv6_forward(*args, state=dev(inp["state"]), algo="chunked", out_dtype=torch.bfloat16)
    hf = [dev(np.ascontiguousarray(inp[n].reshape(B, T, H, 64).transpose(0, 2, 1, 3))) for n in ("r", "k", "v", "x")]
    yh, Sh = wkv.wkv6_forward(*hf, dev(inp["u"]), H, state=dev(inp["state"]), algo="chunked", head_first=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2)
    assert torch.equal(yb, y1.to(torch.bfloat16))
    assert torch.equal(yh.permute(0, 2, 1, 3).reshape(B, T, H * 64), y1) and torch.equal(Sh, S1)


@pytest.mark.parametrize("algo", ["auto", "scan"])
def test_v5_strong_static_decay(algo):
    """v5 with a static decay of exp(-exp(1.5)) on a few channels: every chunk leaves the
    exponent range there and runs directly; the rest of the channels decay weakly."""
    inp = wkv5_inputs(2, 200, 2, 64, seed=49, init_state=2)
    inp["x"] = inp["x"].copy()
    inp["x"][[3, 70, 71, 127]] = 1.5
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), 2]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, S = wkv.wkv5_forward(*args, state=dev(inp["state"]), algo=algo, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], 2, 64, state=inp["state"])
    assert_bf16(host(y), yo, f"v5 {algo} y, strong static decay")
    assert_bf16(host(S), So, f"v5 {algo} state, strong static decay")


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
