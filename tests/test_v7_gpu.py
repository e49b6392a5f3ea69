"""GPU parity of the v7 generalized-delta-rule kernels against the fp64 oracle (through the C ABI):
the token-sequential kernel ("scan") and the 64-token chunked form on MFMA ("chunked", the
default for bf16 inputs with T >= 64).

Inputs (wkv7_inputs, seeded): decay parameter w ~ U(-6, 0) (decay exp(-exp(w))), r, k, v ~ N(0, 0.5), a = -kappa and
b = kappa * beta with a unit kappa per (token, head) and beta ~ U(0, 1); initial states ~ N(0, 0.1).
Tolerances as the other forms: bf16 inputs max abs 2e-2 and mean abs 5e-3 on y and the final
state; fp32 inputs max error relative to max(|o|, rms(o)) 2e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import assert_bf16, assert_fp32, dev, host
from wkv_inputs import bf16_round, bf16_to_f32, wkv7_inputs

pytestmark = pytest.mark.gpu

NAMES = ("r", "w", "k", "v", "a", "b")


def _run(inp, **kw):
    return wkv.wkv7_forward(*(dev(inp[n]) for n in NAMES), inp["H"], **kw)


def _oracle(inp, **kw):
    return oracle.wkv7(*(inp[n] for n in NAMES), inp["H"], inp["N"], **kw)


@pytest.mark.parametrize("T,dtype,algo", [(1, "bf16", "auto"), (17, "f32", "auto"), (130, "bf16", "scan"),
                                          (130, "bf16", "chunked"), (200, "f32", "auto"), (1, "bf16", "chunked"),
                                          (63, "bf16", "chunked")])
def test_v7_small_cases(T, dtype, algo):
    inp = wkv7_inputs(2, T, 3, 64, seed=200 + T, dtype=dtype, init_state=3)
    check = assert_fp32 if dtype == "f32" else assert_bf16
    smap = np.array([2, 0], dtype=np.int32)
    y, S = _run(inp, state=dev(inp["state"]), state_map=dev(smap), algo=algo)
    y1, S1 = _run(inp, state=dev(inp["state"][:1]), algo=algo)         # shared row
    st = dev(inp["state"][:2])
    y2, _ = _run(inp, state=st, state_out=st, algo=algo)               # in place
    y0, S0 = _run(inp, algo=algo)                                      # zero state
    torch.cuda.synchronize()
    yo, So = _oracle(inp, state=inp["state"], state_map=smap)
    check(host(y), yo, "v7 y")
    check(host(S), So, "v7 state")
    yo1, So1 = _oracle(inp, state=inp["state"][:1])
    check(host(y1), yo1, "v7 shared y")
    check(host(S1), So1, "v7 shared state")
    yo2, So2 = _oracle(inp, state=inp["state"][:2])
    check(host(y2), yo2, "v7 in-place y")
    check(host(st), So2, "v7 in-place state")
    yo0, So0 = _oracle(inp)
    check(host(y0), yo0, "v7 zero-state y")
    check(host(S0), So0, "v7 zero-state state")


@pytest.mark.parametrize("T", [8, 9, 63, 64, 65, 128, 129])
def test_v7_block_edges(T):
    """Lengths on either side of the few-token kernel's limit (8 / 9) and of the prefill kernel's
    64-token blocks (one short block, exact multiples, one token past them), fp32 inputs with a
    mapped initial state, against the oracle."""
    inp = wkv7_inputs(3, T, 2, 64, seed=230 + T, dtype="f32", init_state=2)
    smap = np.array([1, 0, 1], dtype=np.int32)
    y, S = _run(inp, state=dev(inp["state"]), state_map=dev(smap))
    torch.cuda.synchronize()
    yo, So = _oracle(inp, state=inp["state"], state_map=smap)
    assert_fp32(host(y), yo, f"v7 y T={T}")
    assert_fp32(host(S), So, f"v7 state T={T}")


@pytest.mark.parametrize("algo", ["scan", "chunked"])
@pytest.mark.parametrize("B,T,H", [(1, 300, 1), (2, 70, 40)])
def test_v7_grid_shapes(B, T, H, algo):
    """A single (row, head) workgroup, and 40 heads (C = 2560), bf16 inputs with zero initial
    state, against the oracle."""
    inp = wkv7_inputs(B, T, H, 64, seed=240 + H)
    y, S = _run(inp, algo=algo)
    torch.cuda.synchronize()
    yo, So = _oracle(inp)
    assert_bf16(host(y), yo, f"v7 y B={B} T={T} H={H}")
    assert_bf16(host(S), So, f"v7 state B={B} T={T} H={H}")


@pytest.mark.parametrize("algo", ["scan", "chunked"])
def test_v7_moderate_full_compare(algo):
    inp = wkv7_inputs(2, 1024, 4, 64, seed=210)
    y, S = _run(inp, algo=algo)
    torch.cuda.synchronize()
    yo, So = _oracle(inp)
    assert_bf16(host(y), yo, "v7 y T=1024")
    assert_bf16(host(S), So, "v7 state T=1024")
    assert np.max(np.abs(host(y) - yo)) < 1e-3


@pytest.mark.parametrize("algo", ["scan", "chunked"])
def test_v7_full_shape(algo):
    """B=8 T=4096 H=32 N=64 bf16 (the bench shape): every (row, head) unit."""
    B, T, H = 8, 4096, 32
    inp = wkv7_inputs(B, T, H, 64, seed=0)
    y, S = _run(inp, algo=algo)
    torch.cuda.synchronize()
    yo, So = _oracle(inp)
    assert_bf16(host(y), yo, f"v7 B=8 T=4096 H=32 {algo} y")
    assert_bf16(host(S), So, f"v7 B=8 T=4096 H=32 {algo} state")
    assert np.max(np.abs(host(y) - yo)) < 1e-3


@pytest.mark.parametrize("T", [64, 65, 127, 128, 129, 191, 200])
def test_v7_chunked_edges(T):
    """The chunked form at its 64-token chunk edges (exact multiples, one past, a ragged last
    chunk), bf16 inputs with a mapped initial state and a bf16 y, against the oracle; the bf16 y
    is the fp32 y rounded, and the result agrees with the scan."""
    inp = wkv7_inputs(3, T, 2, 64, seed=250 + T, init_state=2)
    smap = np.array([1, 0, 1], dtype=np.int32)
    y, S = _run(inp, state=dev(inp["state"]), state_map=dev(smap), algo="chunked")
    yb, Sb = _run(inp, state=dev(inp["state"]), state_map=dev(smap), algo="chunked", out_dtype=torch.bfloat16)
    ys, Ss = _run(inp, state=dev(inp["state"]), state_map=dev(smap), algo="scan")
    torch.cuda.synchronize()
    yo, So = _oracle(inp, state=inp["state"], state_map=smap)
    assert_bf16(host(y), yo, f"chunked y T={T}")
    assert_bf16(host(S), So, f"chunked state T={T}")
    assert torch.equal(yb, y.to(torch.bfloat16)) and torch.equal(Sb, S)
    assert_bf16(host(y), host(ys), f"chunked vs scan y T={T}")


@pytest.mark.parametrize("case", ["strong", "mixed"])
def test_v7_chunked_strong_decays(case):
    """Decays far past the chunked form's exponent range (w ~ U(1, 4): a per-step decay below
    exp(-e)) in every chunk, or in one chunk plus a few tokens whose decay is exactly 0 (w = 100):
    those chunks run the direct recurrence inside the kernel and the result matches the oracle
    with no status bit set."""
    T = 200
    inp = wkv7_inputs(2, T, 2, 64, seed=260, init_state=2)
    rng = np.random.default_rng(10)
    w = bf16_to_f32(inp["w"]).copy()
    if case == "strong":
        w[:] = rng.uniform(1.0, 4.0, size=w.shape)
    else:
        w[:, 64:128] = rng.uniform(1.0, 4.0, size=w[:, 64:128].shape)
        w[1, 150:153] = 100.0
    inp["w"] = bf16_round(w)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, S = _run(inp, state=dev(inp["state"]), algo="chunked", dev_status=st)
    y2, S2 = _run(inp, state=dev(inp["state"]), algo="chunked")
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y, y2) and torch.equal(S, S2)
    yo, So = _oracle(inp, state=inp["state"])
    assert_bf16(host(y), yo, f"{case}: chunked y")
    assert_bf16(host(S), So, f"{case}: chunked state")


def test_v7_decode_steps_carry_the_state():
    """A prompt then T = 1 steps with the state carried equals one pass over all tokens."""
    inp = wkv7_inputs(4, 70, 2, 64, seed=211, init_state=4)
    cut = 66
    pre = dict(inp, **{n: inp[n][:, :cut] for n in NAMES})
    y_pre, S = _run(pre, state=dev(inp["state"]))
    ys = [y_pre]
    for t in range(cut, 70):
        step = dict(inp, **{n: inp[n][:, t:t + 1] for n in NAMES})
        yt, S = _run(step, state=S)
        ys.append(yt)
    torch.cuda.synchronize()
    yo, So = _oracle(inp, state=inp["state"])
    assert_bf16(host(torch.cat(ys, dim=1)), yo, "prompt + decode y")
    assert_bf16(host(S), So, "prompt + decode state")


def test_v7_bf16_out_deterministic_and_empty():
    inp = wkv7_inputs(2, 100, 2, 64, seed=212, init_state=2)
    ya, Sa = _run(inp, state=dev(inp["state"]))
    yb, Sb = _run(inp, state=dev(inp["state"]))
    yc, Sc = _run(inp, state=dev(inp["state"]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(Sa, Sb)
    assert yc.dtype == torch.bfloat16 and torch.equal(yc, ya.to(torch.bfloat16)) and torch.equal(Sc, Sa)
    # T = 0: the state row is copied, nothing else is touched
    e = wkv7_inputs(2, 0, 2, 64, seed=213, init_state=3)
    smap = dev(np.array([2, 1], dtype=np.int32))
    st = dev(e["state"])
    empty = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    _, S0 = wkv.wkv7_forward(empty, empty, empty, empty, empty, empty, 2, state=st, state_map=smap)
    torch.cuda.synchronize()
    assert torch.equal(S0, st[[2, 1]])


def test_v7_plan_repeats_the_eager_call():
    """A pre-marshalled plan, called twice on a carried state (two decode steps in place), gives
    bitwise the outputs and states of two eager calls."""
    inp = wkv7_inputs(4, 1, 3, 64, seed=218, init_state=4)
    toks = [dev(inp[n]) for n in NAMES]
    st_a, st_b = dev(inp["state"]), dev(inp["state"])
    ys_a = []
    for _ in range(2):
        y, _ = wkv.wkv7_forward(*toks, 3, state=st_a, state_out=st_a)
        ys_a.append(y)
    plan = wkv.wkv7_plan(*toks, 3, state=st_b, state_out=st_b)
    ys_b = [plan()[0].clone() for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b)
    for a, b in zip(ys_a, ys_b):
        assert torch.equal(a, b)


def test_v7_bad_state_map_sets_status():
    inp = wkv7_inputs(2, 20, 1, 64, seed=214, init_state=2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.full((2, 20, 64), float("nan"), device="cuda")
    _run(inp, state=dev(inp["state"]), state_map=dev(np.array([1, 9], dtype=np.int32)), y=y, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    assert torch.isnan(y[1]).all() and not torch.isnan(y[0]).any()


@pytest.mark.parametrize("algo", ["scan", "chunked"])
@pytest.mark.parametrize("side", ["left", "right"])
def test_v7_padding_by_decay_parameter(side, algo):
    """The page's padding convention for this operator: padded tokens carry w = -1e9 (decay exactly
    1) and zero r, k, v, a, b, so they leave the state as it was and read zero.  Right padding keeps
    the real tokens' blocks (or chunks), so their outputs and the final state equal the unpadded
    call's bitwise; left padding shifts the 64-token blocks of the scan's rescaled frame (or the
    chunks of the chunked form), so the two agree to that algorithm's rounding: fp32 for the scan,
    the bf16-input tolerance for the chunked form.  The padded outputs are zero."""
    T, P = 150, 9
    inp = wkv7_inputs(2, T, 2, 64, seed=215, init_state=2)
    y, S = _run(inp, state=dev(inp["state"]), algo=algo)
    pad = {n: np.zeros((2, P, 128), dtype=np.uint16) for n in NAMES}
    pad["w"] = bf16_round(np.full((2, P, 128), -1e9, dtype=np.float32))
    if side == "left":
        padded = dict(inp, **{n: np.concatenate([pad[n], inp[n]], axis=1) for n in NAMES})
        real, fill = slice(P, P + T), slice(0, P)
    else:
        padded = dict(inp, **{n: np.concatenate([inp[n], pad[n]], axis=1) for n in NAMES})
        real, fill = slice(0, T), slice(T, T + P)
    yp, Sp = _run(padded, state=dev(inp["state"]), algo=algo)
    torch.cuda.synchronize()
    if side == "right":
        assert torch.equal(yp[:, real], y) and torch.equal(Sp, S)
    else:
        check = assert_fp32 if algo == "scan" else assert_bf16
        check(host(yp[:, real]), host(y), "left padding y")
        check(host(Sp), host(S), "left padding state")
    assert torch.count_nonzero(yp[:, fill]) == 0


def test_v7_direct_form_blocks():
    """Decays strong enough that a 64-token block's decay product falls below 2^-64 (w ~ U(1, 2.5):
    per-step decays exp(-e^1) .. exp(-e^2.5), in the first 70 tokens) send those blocks through the
    direct form; the later blocks take the rescaled frame.  The result matches the oracle."""
    T, S = 200, 70
    inp = wkv7_inputs(2, T, 2, 64, seed=217, dtype="f32", init_state=2)
    rng = np.random.default_rng(9)
    inp["w"][:, :S] = rng.uniform(1.0, 2.5, size=inp["w"][:, :S].shape).astype(np.float32)
    y, St = _run(inp, state=dev(inp["state"]))
    torch.cuda.synchronize()
    yo, So = _oracle(inp, state=inp["state"])
    assert_fp32(host(y), yo, "direct-form blocks y")
    assert_fp32(host(St), So, "direct-form blocks state")


@pytest.mark.parametrize("T,algo", [(1, "auto"), (130, "scan"), (130, "chunked")])
def test_v7_head_first_is_exact(T, algo):
    """Head-first [B, H, T, N] arrays (the operators' head_first flag) give bitwise the token-major
    results, on the prefill kernels (T = 130) and the few-token kernel (T = 1)."""
    B, H = 3, 2
    inp = wkv7_inputs(B, T, H, 64, seed=216 + T, init_state=B)
    y, S = _run(inp, state=dev(inp["state"]), algo=algo)
    hf = [dev(np.ascontiguousarray(inp[n].reshape(B, T, H, 64).transpose(0, 2, 1, 3))) for n in NAMES]
    yh, Sh = wkv.wkv7_forward(*hf, H, state=dev(inp["state"]), head_first=True, algo=algo)
    torch.cuda.synchronize()
    assert yh.shape == (B, H, T, 64)
    assert torch.equal(yh.permute(0, 2, 1, 3).reshape(B, T, H * 64), y) and torch.equal(Sh, S)
