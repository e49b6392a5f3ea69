"""Head-first token layout and bf16 output (the _ex entry points) on the GPU.

Both options change only where values are read and written and how y is
stored, never the arithmetic, so the checks are exact:
  - head-first [B, H, T, N] inputs give bitwise the same y (transposed) and
    final states as [B, T, H, N] inputs;
  - a bf16 y is bitwise the fp32 y rounded to nearest even (torch's own
    float32 -> bfloat16 conversion).
The bf16 y is also compared with the fp64 oracle rounded to bf16: at least
99.9% of the outputs within one bf16 unit in the last place (ulp) of the
rounded oracle value, and every output within half an ulp plus 2e-4 (the fp32
path's own error bound on these inputs) of the oracle.
Inputs as the v5 / v6 parity tests: r, k, v ~ N(0, 0.5), v6 decay parameter
~ U(-6, 0) (v5: U(-6, -0.5)), u ~ N(0, 0.5), initial states ~ N(0, 0.1).
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import assert_bf16, dev, host
from wkv_inputs import varlen_inputs, wkv4_inputs, wkv5_inputs, wkv6_inputs

pytestmark = pytest.mark.gpu

BF16_ABS_FLOOR = 2e-4
BF16_WITHIN_ULP = 0.999


def _bf16_round(o):
    """float64 -> nearest bf16 (through float32, round to nearest even on the 16 dropped bits)."""
    u = np.asarray(o, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def assert_bf16_out(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rb = _bf16_round(ref)
    ulp = _bf16_ulp(rb)
    within = np.abs(got - rb) <= ulp
    frac = float(within.mean()) if within.size else 1.0
    worst = float(np.max(np.abs(got - ref) - 0.5 * ulp)) if ref.size else 0.0
    assert frac >= BF16_WITHIN_ULP, f"{what}: only {frac:.5f} of outputs within 1 bf16 ulp of the oracle"
    assert worst <= BF16_ABS_FLOOR, f"{what}: an output is {worst:.3e} beyond half an ulp (> {BF16_ABS_FLOOR})"
    return frac, worst


def _head_first(a, B, T, H, N):
    """[B, T, H*N] numpy array -> contiguous [B, H, T, N]."""
    return np.ascontiguousarray(np.asarray(a).reshape(B, T, H, N).transpose(0, 2, 1, 3))


def _tok_major(t, B, T, H, N):
    """[B, H, T, N] device tensor -> [B, T, H*N]."""
    return t.permute(0, 2, 1, 3).reshape(B, T, H * N)


def _inputs(version, B, T, H, dtype, seed):
    if version == 6:
        return wkv6_inputs(B, T, H, 64, seed=seed, dtype=dtype, init_state=B + 1)
    return wkv5_inputs(B, T, H, 64, seed=seed, dtype=dtype, init_state=B + 1)


def _call(version, inp, algo, head_first=False, out_dtype=torch.float32, smap=None):
    B, T, H, N = inp["r"].shape[0], inp["r"].shape[1], inp["H"], inp["N"]
    tok = [inp["r"], inp["k"], inp["v"]] + ([inp["x"]] if version == 6 else [])
    if head_first:
        tok = [_head_first(a, B, T, H, N) for a in tok]
    tok = [dev(a) for a in tok]
    fn = wkv.wkv6_forward if version == 6 else wkv.wkv5_forward
    if version == 6:
        args = tok + [dev(inp["u"]), H]
    else:
        args = tok + [dev(inp["x"]), dev(inp["u"]), H]
    return fn(*args, state=dev(inp["state"]), state_map=None if smap is None else dev(smap), algo=algo,
              head_first=head_first, out_dtype=out_dtype)


CASES = [(6, "chunked", 130, "bf16"), (6, "scan", 37, "bf16"), (6, "scan", 70, "f32"),
         (5, "chunked", 200, "bf16"), (5, "scan", 33, "f32")]


@pytest.mark.parametrize("version,algo,T,dtype", CASES)
def test_head_first_and_bf16_out_are_exact(version, algo, T, dtype):
    B, H = 3, 2
    inp = _inputs(version, B, T, H, dtype, seed=300 + T)
    smap = np.array([2, 0, 3], dtype=np.int32)
    y, S = _call(version, inp, algo, smap=smap)
    y_hf, S_hf = _call(version, inp, algo, head_first=True, smap=smap)
    y_b, S_b = _call(version, inp, algo, out_dtype=torch.bfloat16, smap=smap)
    y_hfb, S_hfb = _call(version, inp, algo, head_first=True, out_dtype=torch.bfloat16, smap=smap)
    torch.cuda.synchronize()
    assert y_hf.shape == (B, H, T, 64) and y_b.dtype == torch.bfloat16 and y_hfb.dtype == torch.bfloat16
    assert torch.equal(_tok_major(y_hf, B, T, H, 64), y), "head-first y differs from the token-major y"
    assert torch.equal(S_hf, S) and torch.equal(S_b, S) and torch.equal(S_hfb, S)
    assert torch.equal(y_b, y.to(torch.bfloat16)), "bf16 y is not the fp32 y rounded to nearest even"
    assert torch.equal(_tok_major(y_hfb, B, T, H, 64), y_b)
    # against the oracle
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, 64, state=inp["state"],
                          state_map=smap)
    assert_bf16(host(y), yo, f"v{version} {algo} y")
    assert_bf16(host(S), So, f"v{version} {algo} state")
    assert_bf16_out(host(y_b.float()), yo, f"v{version} {algo} bf16 y")


def test_head_first_zero_tokens_and_bad_map():
    """T = 0 copies the mapped state in either layout; a bad map entry sets the status bit."""
    B, H = 2, 2
    inp = wkv6_inputs(B, 0, H, 64, seed=9, init_state=3)
    st = dev(inp["state"])
    smap = dev(np.array([2, 1], dtype=np.int32))
    empty = torch.empty((B, H, 0, 64), dtype=torch.bfloat16, device="cuda")
    y, S = wkv.wkv6_forward(empty, empty, empty, empty, dev(inp["u"]), H, state=st, state_map=smap,
                            head_first=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y.shape == (B, H, 0, 64)
    assert torch.equal(S, st[[2, 1]])
    inp = wkv6_inputs(B, 70, H, 64, seed=10, init_state=2)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok = [dev(_head_first(inp[n], B, 70, H, 64)) for n in ("r", "k", "v", "x")]
    wkv.wkv6_forward(*tok, dev(inp["u"]), H, state=dev(inp["state"]), state_map=dev(np.array([0, 5], np.int32)),
                     head_first=True, algo="chunked", dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP


def test_headline_shape_head_first_bf16_out():
    """B=8 T=4096 H=32 N=64 bf16 on the chunked kernel: head-first inputs with a bf16 y are exactly the
    token-major fp32 run rounded, and every (row, head) unit matches the oracle."""
    B, T, H, N = 8, 4096, 32, 64
    inp = wkv6_inputs(B, T, H, N, seed=0)
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    y, S = wkv.wkv6_forward(*args, algo="chunked")
    hf = [dev(_head_first(inp[n], B, T, H, N)) for n in ("r", "k", "v", "x")]
    y_hfb, S_hfb = wkv.wkv6_forward(*hf, dev(inp["u"]), H, algo="chunked", head_first=True,
                                     out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(S_hfb, S)
    assert torch.equal(_tok_major(y_hfb, B, T, H, N), y.to(torch.bfloat16))
    yo, So = oracle.wkv56(inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N)
    got = host(_tok_major(y_hfb, B, T, H, N).float())
    assert_bf16_out(got, yo, "headline bf16 y")


@pytest.mark.parametrize("max_len", [1, 8, 64])
def test_varlen_bf16_out_is_rounded_fp32(max_len):
    H, N, S = 2, 64, 40
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, max_len + 1, size=S).astype(np.int32)
    inp = varlen_inputs(S, H, N, seed=61, decode_steps=0, lengths=lengths)
    state = rng.standard_normal((S, H, N, N)).astype(np.float32) * 0.1
    args = [dev(lengths)] + [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    st32, stb = dev(state), dev(state)
    y32 = wkv.wkv6_forward_varlen(*args, st32, max_len=max_len)
    yb = wkv.wkv6_forward_varlen(*args, stb, max_len=max_len, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert yb.dtype == torch.bfloat16
    assert torch.equal(yb, y32.to(torch.bfloat16)) and torch.equal(stb, st32)
    yo, _ = oracle.wkv6_varlen(lengths, inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], H, N, state)
    assert_bf16_out(host(yb.float()), yo, f"varlen max_len={max_len} bf16 y")


@pytest.mark.parametrize("B,T,C,dtype,with_r", [(2, 300, 2048, "bf16", True), (3, 37, 100, "f32", True),
                                                (1, 1024, 192, "bf16", False)])
def test_v4_bf16_out_is_rounded_fp32(B, T, C, dtype, with_r):
    inp = wkv4_inputs(B, T, C, seed=17, with_r=with_r, dtype=dtype, init_state=True)
    args = [dev(inp["tau"]), dev(inp["u"]), dev(inp["k"]), dev(inp["v"]), dev(inp["r"])]
    y32, s32 = wkv.wkv4_forward(*args, state=dev(inp["state"]))
    yb, sb = wkv.wkv4_forward(*args, state=dev(inp["state"]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert yb.dtype == torch.bfloat16
    assert torch.equal(yb, y32.to(torch.bfloat16)) and torch.equal(sb, s32)
    s = inp["state"].astype(np.float64)
    yo, _, _ = oracle.wkv4(inp["tau"], inp["u"], inp["k"], inp["v"], inp["r"], s[:, 0] * np.exp(s[:, 2]),
                           s[:, 1] * np.exp(s[:, 2]))
    assert_bf16_out(host(yb.float()), yo, "v4 bf16 y")
