"""GPU parity of the HIP kernels against the fp64 oracle (through the C ABI).

Workloads (seeded, synthetic):
  v4  B=1 T=64 C=32 fp32, zero state (small) and B=8 T=1024 C=2048 fp32 with
      the sigmoid(r) gate plus one T=1 decode step carrying (a, b, p);
  v5  B=8 T=4096 H=32 N=64 bf16 (every unit) plus small ragged cases;
  v6  B=4 T=4096 H=40 N=64 and B=8 T=4096 H=32 N=64 bf16 (every unit),
      plus small cases covering ragged tails, T=1, shared / mapped / in-place
      states and fp32 inputs.
Tolerances: fp32 inputs max error relative to max(|o|, rms(o)) <= 2e-5;
bf16 inputs max abs <= 2e-2 and mean abs <= 5e-3, on y and on final states.
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import assert_bf16, assert_fp32, dev, host
from wkv_inputs import wkv4_inputs, wkv5_inputs, wkv6_inputs

pytestmark = pytest.mark.gpu

ALGOS = ["scan", "chunked"]


def _v4_AB(state):
    s = host(state) if isinstance(state, torch.Tensor) else np.asarray(state, dtype=np.float64)
    return s[:, 0] * np.exp(s[:, 2]), s[:, 1] * np.exp(s[:, 2])


def _check_v4_state(state, A_ref, B_ref, what):
    A, Bd = _v4_AB(state)
    rel_b = np.max(np.abs(Bd - B_ref) / np.abs(B_ref))
    assert rel_b <= 2e-5, f"{what}: denominator relative error {rel_b:.3e}"
    assert_fp32(A / Bd, A_ref / B_ref, what + " (A/B)")


# ------------------------------------------------------------------ v4

def test_v4_small_config():
    inp = wkv4_inputs(1, 64, 32, seed=0)
    y, st = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]))
    torch.cuda.synchronize()
    yo, Ao, Bo = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"])
    assert_fp32(host(y), yo, "v4 C0 y")
    _check_v4_state(st, Ao, Bo, "v4 C0 state")
    # from a zero state the first output is v_0 exactly
    assert np.array_equal(host(y)[0, 0], inp["v"][0, 0].astype(np.float64))


def test_v4_full_config_with_decode():
    inp = wkv4_inputs(8, 1024, 2048, seed=0, with_r=True, decode_steps=1)
    y, st = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["r"]))
    d = inp["decode"][0]
    y1, st1 = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(d["k"]), dev(d["v"]), dev(d["r"]), state=st)
    torch.cuda.synchronize()
    yo, Ao, Bo = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"])
    assert_fp32(host(y), yo, "v4 C1 y")
    _check_v4_state(st, Ao, Bo, "v4 C1 state")
    yo1, Ao1, Bo1 = oracle.wkv4(inp["tau"], inp["u"], d["k"], d["v"], d["r"], Ao, Bo)
    assert_fp32(host(y1), yo1, "v4 C1 decode y")
    _check_v4_state(st1, Ao1, Bo1, "v4 C1 decode state")


@pytest.mark.parametrize("B,T,C,dtype,with_r", [(2, 1, 100, "f32", False), (3, 37, 100, "bf16", True),
                                                (1, 300, 64, "f32", True), (2, 773, 128, "bf16", True),
                                                (1, 512, 64, "f32", False), (1, 1024, 192, "bf16", False)])
def test_v4_ragged_and_initial_state(B, T, C, dtype, with_r):
    inp = wkv4_inputs(B, T, C, seed=7, with_r=with_r, dtype=dtype, init_state=True)
    st0 = dev(inp["state"])
    y, st = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["r"]),
                             state=st0)
    # in place: state_out == state_in
    st_inplace = dev(inp["state"])
    y2, _ = wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["r"]),
                             state=st_inplace, state_out=st_inplace)
    torch.cuda.synchronize()
    A0, B0 = _v4_AB(inp["state"])
    yo, Ao, Bo = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"], A0, B0)
    assert_fp32(host(y), yo, "v4 y")
    _check_v4_state(st, Ao, Bo, "v4 state")
    assert torch.equal(y, y2) and torch.equal(st, st_inplace)


def test_v4_zero_tokens_copies_state():
    inp = wkv4_inputs(2, 0, 64, seed=1, init_state=True)
    st0 = dev(inp["state"])
    out = torch.full_like(st0, float("nan"))
    wkv.wkv4_forward(dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), state=st0, state_out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, st0)


# ------------------------------------------------------------------ v5 / v6 helpers

def _run56(version, inp, algo, state=None, state_map=None, **kw):
    H = inp["H"]
    args = [dev(inp["r"]), dev(inp["k"]), dev(inp["v"]), dev(inp["x"]), dev(inp["u"]), H]
    fn = wkv.wkv6_forward if version == 6 else wkv.wkv5_forward
    return fn(*args, state=state, state_map=state_map, algo=algo, **kw)


def _oracle56(inp, state=None, state_map=None, units=None):
    return oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], inp["H"], inp["N"],
                        state=state, state_map=state_map, units=units)


# ------------------------------------------------------------------ v5

@pytest.mark.parametrize("algo", ALGOS)
def test_v5_full_config(algo):
    """B=8 T=4096 H=32: every (row, head) unit against the oracle."""
    inp = wkv5_inputs(8, 4096, 32, 64, seed=0)
    y, S = _run56(5, inp, algo)
    torch.cuda.synchronize()
    yo, So = _oracle56(inp)
    assert_bf16(host(y), yo, f"v5 B=8 T=4096 H=32 {algo} y")
    assert_bf16(host(S), So, f"v5 B=8 T=4096 H=32 {algo} state")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("T", [1, 17, 130])
def test_v5_small_mapped_state(algo, T):
    inp = wkv5_inputs(3, T, 2, 64, seed=T, init_state=2)
    smap = np.array([1, 0, 1], dtype=np.int32)
    y, S = _run56(5, inp, algo, state=dev(inp["state"]), state_map=dev(smap))
    torch.cuda.synchronize()
    yo, So = _oracle56(inp, state=inp["state"], state_map=smap)
    assert_bf16(host(y), yo, "v5 y")
    assert_bf16(host(S), So, "v5 state")


# ------------------------------------------------------------------ v6

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("B,H", [(4, 40), (8, 32)])
def test_v6_full_config(algo, B, H):
    """B=4 H=40 and B=8 H=32 at T=4096: every (row, head) unit against the oracle."""
    inp = wkv6_inputs(B, 4096, H, 64, seed=0)
    y, S = _run56(6, inp, algo)
    torch.cuda.synchronize()
    yo, So = _oracle56(inp)
    assert_bf16(host(y), yo, f"v6 B={B} H={H} {algo} y")
    assert_bf16(host(S), So, f"v6 B={B} H={H} {algo} state")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (63, "bf16"), (64, "f32"), (200, "f32"), (129, "bf16")])
def test_v6_small_cases(algo, T, dtype):
    inp = wkv6_inputs(2, T, 3, 64, seed=100 + T, dtype=dtype, init_state=2)
    if algo == "chunked" and dtype == "f32":
        with pytest.raises(wkv.WkvError):
            _run56(6, inp, algo)
        return
    # 1:1 states
    y, S = _run56(6, inp, algo, state=dev(inp["state"]))
    # shared state (n_state == 1)
    y1, S1 = _run56(6, inp, algo, state=dev(inp["state"][:1]))
    # permuted map
    smap = np.array([1, 0], dtype=np.int32)
    y2, S2 = _run56(6, inp, algo, state=dev(inp["state"]), state_map=dev(smap))
    # in place
    st = dev(inp["state"])
    y3, _ = _run56(6, inp, algo, state=st, state_out=st)
    torch.cuda.synchronize()
    check = assert_bf16
    yo, So = _oracle56(inp, state=inp["state"])
    check(host(y), yo, "v6 y")
    check(host(S), So, "v6 state")
    yo1, So1 = _oracle56(inp, state=inp["state"][:1])
    check(host(y1), yo1, "v6 shared y")
    check(host(S1), So1, "v6 shared state")
    yo2, So2 = _oracle56(inp, state=inp["state"], state_map=smap)
    check(host(y2), yo2, "v6 mapped y")
    check(host(S2), So2, "v6 mapped state")
    assert torch.equal(y3, y) and torch.equal(st, S)


def test_v6_fp32_inputs_tight():
    """fp32 inputs: the scan is far inside the bf16 tolerance (state kept in fp32)."""
    inp = wkv6_inputs(2, 300, 2, 64, seed=5, dtype="f32", init_state=2)
    y, S = _run56(6, inp, "scan", state=dev(inp["state"]))
    torch.cuda.synchronize()
    yo, So = _oracle56(inp, state=inp["state"])
    err = np.max(np.abs(host(y) - yo)) / max(1.0, np.max(np.abs(yo)))
    assert err < 2e-5, err


@pytest.mark.parametrize("x_range", [(-6.0, 2.0), (1.0, 4.0), (-20.0, -10.0)])
def test_v6_scan_decay_extremes(x_range):
    """Strong decays send blocks of the scan to its direct form (a block's decay product below
    2^-80), weak ones keep the rescaled frame: both match the oracle to fp32 accuracy."""
    inp = wkv6_inputs(2, 300, 2, 64, seed=21, dtype="f32", x_range=x_range, init_state=2)
    y, S = _run56(6, inp, "scan", state=dev(inp["state"]))
    torch.cuda.synchronize()
    yo, So = _oracle56(inp, state=inp["state"])
    assert_fp32(host(y), yo, f"v6 y x in {x_range}")
    assert_fp32(host(S), So, f"v6 state x in {x_range}")


def test_v6_bad_state_map_sets_status_and_skips():
    inp = wkv6_inputs(2, 8, 1, 64, seed=3, init_state=2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.full((2, 8, 64), float("nan"), device="cuda")
    smap = dev(np.array([0, 5], dtype=np.int32))
    _run56(6, inp, "scan", state=dev(inp["state"]), state_map=smap, y=y, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    assert torch.isnan(y[1]).all() and not torch.isnan(y[0]).any()


@pytest.mark.parametrize("algo", ALGOS)
def test_v6_deterministic(algo):
    """Two runs on the same inputs are bitwise equal (fixed-order sums, no atomics)."""
    inp = wkv6_inputs(2, 500, 4, 64, seed=9, init_state=2)
    ya, Sa = _run56(6, inp, algo, state=dev(inp["state"]))
    yb, Sb = _run56(6, inp, algo, state=dev(inp["state"]))
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(Sa, Sb)


@pytest.mark.parametrize("split", [96, 111])
def test_v6_split_carry_matches_single_pass(split):
    inp = wkv6_inputs(2, 300, 2, 64, seed=12, init_state=2)
    y, S = _run56(6, inp, "scan", state=dev(inp["state"]))
    part = {k: (inp[k][:, :split] if isinstance(inp[k], np.ndarray) and inp[k].ndim == 3 else inp[k]) for k in inp}
    rest = {k: (inp[k][:, split:] if isinstance(inp[k], np.ndarray) and inp[k].ndim == 3 else inp[k]) for k in inp}
    ya, Sa = _run56(6, part, "scan", state=dev(inp["state"]))
    yb, Sb = _run56(6, rest, "scan", state=Sa)
    torch.cuda.synchronize()
    y2 = torch.cat([ya, yb], dim=1)
    if split % 32 == 0:
        # the scan rescales its state in blocks of 32 tokens from the start of a call: a split on
        # a block boundary walks the same arithmetic, so the results are bitwise equal
        assert torch.equal(y2, y) and torch.equal(Sb, S)
    else:
        # elsewhere the blocks differ and so does the rounding, at the fp32 level
        assert_fp32(host(y2), host(y), "split y vs one pass")
        assert_fp32(host(Sb), host(S), "split state vs one pass")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("side", ["left", "right"])
def test_v6_padding_by_decay_mask(algo, side):
    """The rwkv_ops page's padding convention: padded tokens carry zero r, k, v and a decay
    parameter of -1e9 (decay exactly 1), so they leave the state as it is.  The real tokens'
    outputs and the final state then equal those of the unpadded call."""
    T, P = 100, 37
    inp = wkv6_inputs(2, T, 2, 64, seed=77, init_state=2)
    pad = {}
    for n in ("r", "k", "v", "x"):
        a = inp[n]
        fill = np.zeros((2, P, a.shape[2]), dtype=a.dtype)
        if n == "x":
            fill[:] = 0xCE6E  # bf16 bits of -9.98e8 (the -1e9 mask rounded into bf16)
        pad[n] = np.concatenate([fill, a] if side == "left" else [a, fill], axis=1)
    padded = dict(inp, **pad, T=T + P)
    y, S = _run56(6, inp, algo, state=dev(inp["state"]))
    yp, Sp = _run56(6, padded, algo, state=dev(inp["state"]))
    torch.cuda.synchronize()
    real = yp[:, P:] if side == "left" else yp[:, :T]
    # the two calls group the real tokens into different blocks / chunks, so they agree to the
    # algorithm's own rounding: fp32 for the scan, the bf16-input tolerance for the chunked form
    check = assert_fp32 if algo == "scan" else assert_bf16
    check(host(real), host(y), f"{side} padding y")
    check(host(Sp), host(S), f"{side} padding state")
