"""wkv6_forward_train (the chunked v6 forward that also saves the state at every 64-token chunk
boundary) and the chunked backward that takes those states instead of computing them.

Forward: y and the final state must be bitwise those of wkv6_forward(algo="chunked") (the same
kernel code with the state stores added), and every saved state is checked against the fp64
oracle run over the prefix that ends at that boundary: the bf16-input tolerance (2e-2 max abs,
5e-3 mean abs) and a relative bound of 1e-4 (the states come from the hi / lo products, about
2^-17 per term, summed over the chunks before).

Backward with saved states: the chunked bounds of the backward tests (2e-4, dw 2e-3), on the
same cases as the backward without them, plus the cases where the chunked pass itself has to
leave a unit to the sweeps partway through (a chunk out of the exponent range after the pass
has already written later chunks' gradients) or at once (a rejected state_map row).
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import assert_bf16, dev, fp32_relerr, host
from wkv_inputs import bf16_round, wkv6_inputs, wkv6_upstream

pytestmark = pytest.mark.gpu

STATE_REL = 1e-4
GRAD_REL_CHUNKED, DW_REL_CHUNKED = 2e-4, 2e-3
GRAD_REL, DW_REL_STRONG = 1e-4, 1e-3


def _args(inp):
    return [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), inp["H"]]


def _oracle_bwd(inp, up, state=None, state_map=None):
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(
        inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], inp["H"], 64, up["dy"], state=state,
        state_map=state_map, d_state_out=up["d_state"])
    return dr, dk, dv, dx, du, dS


def _check(got, ref, what, grad_bound=GRAD_REL_CHUNKED, dw_bound=DW_REL_CHUNKED, rows=None):
    names = ("dr", "dk", "dv", "dw", "du", "d_state")
    for name, g, o in zip(names, got, ref):
        g = host(g)
        if rows is not None and name != "du":
            g = g[rows]
        e = fp32_relerr(g, o)
        bound = dw_bound if name == "dw" else grad_bound
        print(f"{what} {name}: {e:.3e}")
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        assert e <= bound, f"{what} {name}: relative error {e:.3e} > {bound}"


@pytest.mark.parametrize("T,out_dtype", [(1, torch.float32), (64, torch.float32), (65, torch.float32),
                                         (300, torch.float32), (300, torch.bfloat16)])
def test_forward_train_matches_forward_and_oracle(T, out_dtype):
    inp = wkv6_inputs(2, T, 2, 64, seed=700 + T, init_state=2)
    args = _args(inp)
    st = dev(inp["state"])
    y0, s0 = wkv.wkv6_forward(*args, state=st, algo="chunked", out_dtype=out_dtype)
    y1, s1, cs = wkv.wkv6_forward_train(*args, state=st, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(s0, s1)
    nsave = (T + 63) // 64 - 1
    assert tuple(cs.shape) == (2, 2, nsave, 64, 64)
    for c in range(1, nsave + 1):
        pre = {n: inp[n][:, :64 * c] for n in ("r", "k", "v", "x")}
        _, S = oracle.wkv56(pre["r"], pre["k"], pre["v"], pre["x"], inp["u"], 2, 64, state=inp["state"])
        got = host(cs[:, :, c - 1])
        e = fp32_relerr(got, np.asarray(S))
        print(f"T={T} chunk {c} state: {e:.3e}")
        assert_bf16(got, np.asarray(S), f"T={T} chunk {c} state")
        assert e <= STATE_REL, f"chunk {c} state: {e:.3e}"


def test_forward_train_rejects_what_it_cannot_save():
    inp = wkv6_inputs(1, 100, 1, 64, seed=3, dtype="f32")
    with pytest.raises(wkv.WkvError, match="bf16"):
        wkv.wkv6_forward_train(*_args(inp))
    inp = wkv6_inputs(1, 100, 1, 64, seed=3)
    args = _args(inp)
    r = args[0]
    y = torch.empty((1, 100, 64), device="cuda")
    status = wkv._lib.wkv6_forward_train(1, 100, 1, 64, wkv._ptr(args[0]), wkv._ptr(args[1]), wkv._ptr(args[2]),
                                         wkv._ptr(args[3]), wkv._dtype_code(r), wkv._ptr(args[4]), wkv._ptr(y),
                                         wkv._native.WKV_F32, None, None, 0, None, None, None, wkv._stream(r))
    assert status == wkv._native.WKV_ERR_INVALID_ARG
    assert b"chunk_states" in wkv._lib.wkv_last_error()


@pytest.mark.parametrize("B,T,H,seed", [(2, 65, 2, 1), (2, 128, 2, 4), (2, 300, 2, 2), (3, 1000, 2, 3),
                                        (1, 4097, 3, 5), (64, 128, 8, 6), (8, 4096, 32, 0)])
def test_backward_with_saved_states(B, T, H, seed):
    """Every unit against the oracle, and close to the backward that computes the states itself:
    two whole chunks, ragged last chunks (one token at T=4097), 512 (row, head) units at B=64
    H=8, and B=8 T=4096 H=32 (the headline shape)."""
    inp = wkv6_inputs(B, T, H, 64, seed=seed, init_state=B if seed else None)
    up = wkv6_upstream(B, T, H, 64, seed=seed + 100)
    args = _args(inp)
    st = dev(inp["state"]) if inp["state"] is not None else None
    _, S, cs = wkv.wkv6_forward_train(*args, state=st)
    ds = dev(up["d_state"])
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=ds, chunk_states=cs)
    own = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=ds)
    torch.cuda.synchronize()
    _check(got, _oracle_bwd(inp, up, state=inp["state"]), f"B={B} T={T} H={H} saved")
    for name, a, b in zip(("dr", "dk", "dv", "dw", "du", "d_state"), got, own):
        e = fp32_relerr(host(a), host(b).astype(np.float64))
        print(f"saved vs own {name}: {e:.3e}")
        assert e <= (DW_REL_CHUNKED if name == "dw" else GRAD_REL_CHUNKED)


def test_backward_with_saved_states_leaves_units_to_the_sweeps():
    """Head 1 of every row has decays beyond the chunked range in its first chunk only: the
    chunked pass walks that unit's later chunks, writing their gradients, and leaves it at
    chunk 0, so the sweeps redo it; head 1 of row 2 is out of range in its last chunk (left at
    once).  No status bit; every unit matches."""
    inp = wkv6_inputs(3, 300, 2, 64, seed=51, init_state=3)
    rng = np.random.default_rng(52)
    inp["x"][:, :64, 64:] = bf16_round(rng.random((3, 64, 64), dtype=np.float32) * 1.5 + 0.5)
    inp["x"][2, 256:, 64:] = bf16_round(rng.random((44, 64), dtype=np.float32) * 1.5 + 0.5)
    up = wkv6_upstream(3, 300, 2, 64, seed=53)
    args = _args(inp)
    st = dev(inp["state"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, S, cs = wkv.wkv6_forward_train(*args, state=st, dev_status=status)
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=dev(up["d_state"]),
                            chunk_states=cs, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref = _oracle_bwd(inp, up, state=inp["state"])
    for h, (gb, wb) in ((0, (GRAD_REL_CHUNKED, DW_REL_CHUNKED)), (1, (GRAD_REL, DW_REL_STRONG))):
        cols = slice(64 * h, 64 * (h + 1))
        for name, g, o in zip(("dr", "dk", "dv", "dw"), got[:4], ref[:4]):
            e = fp32_relerr(host(g)[:, :, cols], o[:, :, cols])
            print(f"left head {h} {name}: {e:.3e}")
            assert e <= (wb if name == "dw" else gb), f"head {h} {name}: {e:.3e}"
        e = fp32_relerr(host(got[5])[:, h], ref[5][:, h])
        assert e <= gb, f"head {h} d_state: {e:.3e}"
    assert fp32_relerr(host(got[4]), ref[4]) <= GRAD_REL_CHUNKED


def test_backward_with_saved_states_bad_state_map_row():
    inp = wkv6_inputs(3, 200, 2, 64, seed=61, init_state=2)
    up = wkv6_upstream(3, 200, 2, 64, seed=62, with_state=False)
    smap = np.array([1, 7, 0], dtype=np.int32)
    args = _args(inp)
    st, sm = dev(inp["state"]), dev(smap)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, _, cs = wkv.wkv6_forward_train(*args, state=st, state_map=sm, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    status.zero_()
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_map=sm, chunk_states=cs, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    good = [0, 2]
    sub = {n: inp[n][good] for n in ("r", "k", "v", "x")}
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(sub["r"], sub["k"], sub["v"], sub["x"], inp["u"], 2, 64,
                                                     up["dy"][good], state=inp["state"], state_map=smap[good])
    _check(got, (dr, dk, dv, dx, du, dS), "saved, bad map row skipped", rows=good)


def test_backward_with_saved_states_deterministic():
    inp = wkv6_inputs(2, 333, 2, 64, seed=71, init_state=2)
    up = wkv6_upstream(2, 333, 2, 64, seed=72)
    args = _args(inp)
    st = dev(inp["state"])
    _, S, cs = wkv.wkv6_forward_train(*args, state=st)
    a = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=dev(up["d_state"]), chunk_states=cs)
    b = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=dev(up["d_state"]), chunk_states=cs)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_wide_rows():
    """H=256 (C=16384 channels, 64 KiB per bf16 token row): the chunked passes' row strides and
    store offsets at a width far past the headline's, with and without saved states."""
    inp = wkv6_inputs(1, 130, 256, 64, seed=91, init_state=1)
    up = wkv6_upstream(1, 130, 256, 64, seed=92)
    args = _args(inp)
    st = dev(inp["state"])
    _, S, cs = wkv.wkv6_forward_train(*args, state=st)
    ds = dev(up["d_state"])
    own = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=ds)
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S, d_state=ds, chunk_states=cs)
    torch.cuda.synchronize()
    ref = _oracle_bwd(inp, up, state=inp["state"])
    _check(own, ref, "H=256 own states")
    _check(got, ref, "H=256 saved states")
