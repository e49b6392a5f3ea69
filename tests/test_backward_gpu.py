"""v6 backward (wkv6_backward) against the fp64 oracle's reverse-mode gradients.

The oracle's gradients are pinned to central differences of its forward
(tests/test_oracle_pins.py).  Metric: max |g - o| / max(|o|, rms(o)) per gradient.

Scan path (three fp32 token-sequential sweeps; f32 inputs, T < 64, or algo="scan"):
dr, dk, dv, du and the state gradient are single recurrences like the forward
(measured about 1e-6 at T=4096): bound 1e-4.  The decay gradient is the reverse
running difference of r * dr~ and k * dk~; each of those terms carries its own
fp32 rounding (about 1e-6 relative) and their errors add up over the steps
walked while the result is a difference.  The walk restarts from its exact value
sum_j G S every 256 tokens (the forward sweep keeps S there), so the error no
longer grows with T: bound 2e-4, checked up to T=16384 and on the restart edges.
With strong decays (x up to 2, d_t down to exp(-7.4)) the difference cancels
within one step as well: dlam_t = d_t (sum_j G_t S_{t-1}) is small while its two
terms are not, and dx = -exp(x) dlam scales that error up: bound 1e-3 there.
With x in (1, 4) (d_t below exp(-e) = 0.066 at every step, dx scaled by up to
exp(4) = 55) the same cancellation costs about 1/d_t more: measured 5.0e-3 and
7.7e-3 (dw at most 2.0 there, so about 1e-2 absolute), bound 1.5e-2; the other
gradients keep 1e-4.

Chunked path (64-token chunks on MFMA; bf16 inputs with T >= 64 under "auto"):
every product takes its non-bf16 operands as bf16 hi + lo (about 2^-17
relative each, the product drops lo * lo).  dr, dk, dv, du and the state
gradient measure 3e-5 .. 8.4e-5 (B=8 T=4096 H=32): bound 2e-4.  The decay
gradient is again a difference, now within the chunk: in dlam_m = sum_{t>m}
rb_t . drb_t - sum_{t>=m} kt_t . dkt_t + E, every intra-chunk pair (t, s) that
does not straddle m appears in both sums, through two different products
(dA kt and dA^T rb) rounded independently, so their hi / lo errors do not cancel.
Measured 3e-4 .. 8.1e-4 and flat in T (chunk-local, restarted from E at every
chunk boundary): bound 2e-3.  Units whose decays leave the chunked form's range
are redone by the sweeps (scan bounds), which the mixed cases below check.
"""
import numpy as np
import pytest
import torch

import oracle
import rwkv_linear_attention_wkv_amd as wkv
from parity import dev, fp32_relerr, host
from wkv_inputs import bf16_round, wkv6_inputs, wkv6_upstream

pytestmark = pytest.mark.gpu

GRAD_REL = 1e-4
DW_REL = 2e-4
DW_REL_STRONG = 1e-3  # decays down to exp(-exp(2)) per step
DW_REL_EXTREME = 1.5e-2  # every step's decay below exp(-e)
GRAD_REL_CHUNKED = 2e-4
DW_REL_CHUNKED = 2e-3
CHUNK = 64


def _chunked(algo, dtype, T):
    """Whether the call takes the chunked path (the C API's rule for "auto")."""
    return algo == "chunked" or (algo == "auto" and dtype == "bf16" and T >= CHUNK)


def _bounds(algo, dtype, T, strong=False):
    if _chunked(algo, dtype, T):
        return GRAD_REL_CHUNKED, DW_REL_CHUNKED
    return GRAD_REL, DW_REL_STRONG if strong else DW_REL


def _gpu(inp, up, state=None, state_map=None, with_dstate=True, algo="auto"):
    H = inp["H"]
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), H]
    st = dev(state) if state is not None else None
    sm = dev(state_map) if state_map is not None else None
    _, S_final = wkv.wkv6_forward(*args, state=st, state_map=sm, algo="scan")
    ds = dev(up["d_state"]) if with_dstate else None
    return wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_map=sm,
                             state_final=S_final if with_dstate else None, d_state=ds, algo=algo)


def _check(got, ref, what, bounds):
    grad_bound, dw_bound = bounds
    names = ("dr", "dk", "dv", "dw", "du", "d_state")
    for name, g, o in zip(names, got, ref):
        e = fp32_relerr(host(g), o)
        bound = dw_bound if name == "dw" else grad_bound
        print(f"{what} {name}: {e:.3e} (max |o| {np.abs(o).max():.3e})")
        assert np.all(np.isfinite(host(g))), f"{what} {name}: non-finite"
        assert e <= bound, f"{what} {name}: relative error {e:.3e} > {bound}"


def _oracle(inp, up, state=None, state_map=None, with_dstate=True):
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(
        inp["r"], inp["k"], inp["v"], inp["x"], inp["u"], inp["H"], 64, up["dy"], state=state,
        state_map=state_map, d_state_out=up["d_state"] if with_dstate else None)
    return dr, dk, dv, dx, du, dS


@pytest.mark.parametrize("T,dtype,algo", [(1, "bf16", "auto"), (37, "f32", "auto"), (100, "bf16", "auto"),
                                          (100, "bf16", "scan"), (129, "f32", "auto"), (64, "bf16", "auto"),
                                          (65, "bf16", "auto"), (40, "bf16", "chunked")])
def test_backward_small(T, dtype, algo):
    """Short sequences on both paths: one chunk exactly, one chunk and one token, a single
    ragged chunk (T=40, chunked by request below the "auto" threshold)."""
    inp = wkv6_inputs(2, T, 2, 64, seed=300 + T, dtype=dtype, init_state=2)
    up = wkv6_upstream(2, T, 2, 64, seed=400 + T)
    got = _gpu(inp, up, state=inp["state"], algo=algo)
    torch.cuda.synchronize()
    _check(got, _oracle(inp, up, state=inp["state"]), f"T={T} {dtype} {algo}", _bounds(algo, dtype, T))


@pytest.mark.parametrize("algo", ["auto", "scan"])
def test_backward_no_state_gradient_and_mapped_state(algo):
    inp = wkv6_inputs(3, 70, 1, 64, seed=5, init_state=2)
    up = wkv6_upstream(3, 70, 1, 64, seed=6, with_state=False)
    smap = np.array([1, 0, 1], dtype=np.int32)
    got = _gpu(inp, up, state=inp["state"], state_map=smap, with_dstate=False, algo=algo)
    torch.cuda.synchronize()
    ref = _oracle(inp, up, state=inp["state"], state_map=smap, with_dstate=False)
    _check(got, ref, f"mapped {algo}", _bounds(algo, "bf16", 70))


@pytest.mark.parametrize("algo", ["auto", "scan"])
def test_backward_bad_state_map_row_is_skipped(algo):
    """A state_map entry out of range sets the status bit; that batch row's gradients are not
    defined, and du sums the other rows only (its share is zero), matching the oracle run on the
    valid rows."""
    inp = wkv6_inputs(3, 70, 2, 64, seed=15, init_state=2)
    up = wkv6_upstream(3, 70, 2, 64, seed=16, with_state=False)
    smap = np.array([1, 7, 0], dtype=np.int32)
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), 2]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=dev(inp["state"]), state_map=dev(smap),
                            dev_status=status, algo=algo)
    torch.cuda.synchronize()
    assert int(status.item()) & wkv.WKV_DEV_BAD_STATE_MAP
    good = [0, 2]
    sub = {n: inp[n][good] for n in ("r", "k", "v", "x")}
    dr, dk, dv, dx, du, _, dS = oracle.wkv6_backward(sub["r"], sub["k"], sub["v"], sub["x"], inp["u"], 2, 64,
                                                     up["dy"][good], state=inp["state"], state_map=smap[good])
    _check([t[good] for t in got[:4]] + [got[4], got[5][good]], (dr, dk, dv, dx, du, dS),
           f"bad map row skipped {algo}", _bounds(algo, "bf16", 70))


def test_backward_zero_state_and_decay_extremes():
    for x_range in [(-6.0, 2.0), (-20.0, -10.0)]:
        inp = wkv6_inputs(2, 50, 2, 64, seed=9, dtype="f32", x_range=x_range)
        up = wkv6_upstream(2, 50, 2, 64, seed=10)
        got = _gpu(inp, up, with_dstate=False)  # no initial state, no final-state gradient
        torch.cuda.synchronize()
        _check(got, _oracle(inp, up, with_dstate=False), f"x in {x_range}",
               _bounds("auto", "f32", 50, strong=x_range[1] > 0))


@pytest.mark.parametrize("x_range", [(-6.0, 2.0), (1.0, 4.0)])
def test_backward_chunked_strong_decays(x_range):
    """bf16 inputs under "auto" with decays beyond the chunked form's exponent range: the chunked
    passes leave those units to the sweeps, and every gradient still matches, with no status bit
    (x in (1, 4): every step's decay below exp(-e), the sweeps' decay-gradient bound for that)."""
    inp = wkv6_inputs(2, 200, 2, 64, seed=31, x_range=x_range, init_state=2)
    up = wkv6_upstream(2, 200, 2, 64, seed=32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = [dev(inp[n]) for n in ("r", "k", "v", "x")] + [dev(inp["u"]), 2]
    st = dev(inp["state"])
    _, S_final = wkv.wkv6_forward(*args, state=st, algo="scan")
    got = wkv.wkv6_backward(*args, dev(up["dy"]), state=st, state_final=S_final, d_state=dev(up["d_state"]),
                            dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    _check(got, _oracle(inp, up, state=inp["state"]), f"bf16 x in {x_range}",
           (GRAD_REL, DW_REL_EXTREME) if x_range[0] >= 1.0 else (GRAD_REL_CHUNKED, max(DW_REL_CHUNKED, DW_REL_STRONG)))


def test_backward_chunked_mixed_units():
    """Head 1 of every row has decays that push it to the sweeps while head 0 stays on the chunked
    form: each unit's gradients come from one path, and du (summed over rows) mixes both."""
    inp = wkv6_inputs(3, 300, 2, 64, seed=41, init_state=3)
    strong = np.random.default_rng(42).random((3, 300, 64), dtype=np.float32) * 3.0 + 1.0
    inp["x"][:, :, 64:] = bf16_round(strong)
    up = wkv6_upstream(3, 300, 2, 64, seed=43)
    got = _gpu(inp, up, state=inp["state"])
    torch.cuda.synchronize()
    ref = _oracle(inp, up, state=inp["state"])
    names = ("dr", "dk", "dv", "dw")
    for h, (grad_bound, dw_bound) in ((0, (GRAD_REL_CHUNKED, DW_REL_CHUNKED)), (1, (GRAD_REL, DW_REL_EXTREME))):
        cols = slice(64 * h, 64 * (h + 1))
        for name, g, o in zip(names, got[:4], ref[:4]):
            e = fp32_relerr(host(g)[:, :, cols], o[:, :, cols])
            print(f"mixed head {h} {name}: {e:.3e}")
            assert e <= (dw_bound if name == "dw" else grad_bound), f"head {h} {name}: {e:.3e}"
        e = fp32_relerr(host(got[5])[:, h], ref[5][:, h])
        assert e <= grad_bound, f"head {h} d_state: {e:.3e}"
    e = fp32_relerr(host(got[4]), ref[4])
    print(f"mixed du: {e:.3e}")
    assert e <= GRAD_REL_CHUNKED


@pytest.fixture(scope="module")
def full_shape():
    inp = wkv6_inputs(8, 4096, 32, 64, seed=0)
    up = wkv6_upstream(8, 4096, 32, 64, seed=1)
    return inp, up, _oracle(inp, up)


@pytest.mark.parametrize("algo", ["auto", "scan"])
def test_backward_full_shape(full_shape, algo):
    """B=8 T=4096 H=32 N=64 (the headline forward shape): every (row, head) unit of every
    gradient, du included, against the oracle, on both paths."""
    inp, up, ref = full_shape
    got = _gpu(inp, up, algo=algo)
    torch.cuda.synchronize()
    _check(got, ref, f"B=8 T=4096 H=32 {algo}", _bounds(algo, "bf16", 4096))


@pytest.mark.parametrize("algo", ["auto", "scan"])
def test_backward_deterministic_and_empty(algo):
    inp = wkv6_inputs(2, 77, 2, 64, seed=12, init_state=2)
    up = wkv6_upstream(2, 77, 2, 64, seed=13)
    a = _gpu(inp, up, state=inp["state"], algo=algo)
    b = _gpu(inp, up, state=inp["state"], algo=algo)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # T = 0: no token gradients, du = 0, the state gradient passes through unchanged
    inp0 = wkv6_inputs(2, 0, 2, 64, seed=1, init_state=2)
    up0 = wkv6_upstream(2, 0, 2, 64, seed=2)
    st = dev(inp0["state"])
    args = [dev(inp0[n]) for n in ("r", "k", "v", "x")] + [dev(inp0["u"]), 2]
    out = wkv.wkv6_backward(*args, dev(up0["dy"]), state=st, state_final=st, d_state=dev(up0["d_state"]),
                            algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(out[4], torch.zeros_like(out[4]))
    assert torch.equal(out[5], dev(up0["d_state"]))


@pytest.mark.parametrize("T,dtype,x_range,algo", [(256, "bf16", None, "scan"), (257, "f32", None, "scan"),
                                                  (1024, "bf16", None, "scan"), (2100, "f32", (-6.0, 2.0), "scan"),
                                                  (3103, "bf16", None, "scan"), (3103, "bf16", None, "auto"),
                                                  (2100, "bf16", (-6.0, 0.6), "auto")])
def test_backward_span_restarts(T, dtype, x_range, algo):
    """Scan: T around multiples of the 256-token span at whose ends the decay-gradient walk restarts
    from sum_j G S: none (T=256), one right before the last token, several with a ragged first
    block of the dk/dw sweep, and strong decays (blocks that take the direct form) next to them.
    Chunked: a ragged last chunk, and stronger decays (x up to 0.6, a chunk's log-decay total
    near 18 on average) that still stay within the chunked form's range."""
    kw = {} if x_range is None else {"x_range": x_range}
    inp = wkv6_inputs(2, T, 2, 64, seed=500 + T, dtype=dtype, init_state=2, **kw)
    up = wkv6_upstream(2, T, 2, 64, seed=600 + T)
    got = _gpu(inp, up, state=inp["state"], algo=algo)
    torch.cuda.synchronize()
    bounds = _bounds(algo, dtype, T, strong=x_range is not None)
    if _chunked(algo, dtype, T) and x_range is not None:
        bounds = (bounds[0], max(bounds[1], DW_REL_STRONG))
    _check(got, _oracle(inp, up, state=inp["state"]), f"T={T} {dtype} {algo}", bounds)


@pytest.mark.parametrize("algo", ["scan", "auto"])
def test_backward_long_sequence_dw(algo):
    """T=16384 (four times the headline length).  Scan: the decay gradient stays within 2e-4 (the
    walk restarts every 256 tokens instead of carrying its rounding over the whole sequence).
    Chunked: the same chunk-local bound as at T=64, so nothing grows with T."""
    inp = wkv6_inputs(1, 16384, 2, 64, seed=21, init_state=1)
    up = wkv6_upstream(1, 16384, 2, 64, seed=22)
    got = _gpu(inp, up, state=inp["state"], algo=algo)
    torch.cuda.synchronize()
    _check(got, _oracle(inp, up, state=inp["state"]), f"T=16384 {algo}", _bounds(algo, "bf16", 16384))


@pytest.mark.parametrize("T,algo,saved", [(100, "auto", False), (100, "auto", True), (130, "auto", True),
                                          (65, "auto", False), (100, "scan", False)])
def test_backward_writes_stay_inside_the_outputs(T, algo, saved):
    """The chunked backward stores a ragged last chunk's rows through buffer resources that end at
    its last token (the rows past it are dropped, not branched around).  The last batch row's
    padding rows lie past the end of dr, dk, dv and dw, so each output is handed over at the head
    of a larger buffer whose tail holds a canary: the tail must come back untouched and the
    gradients bitwise equal to the same call on exactly sized outputs."""
    B, H, N = 2, 2, 64
    C = H * N
    inp = wkv6_inputs(B, T, H, N, seed=900 + T, dtype="bf16", init_state=B)
    up = wkv6_upstream(B, T, H, N, seed=950 + T)
    r, k, v, x = (dev(inp[n]) for n in ("r", "k", "v", "x"))
    u, st, dy, dS = dev(inp["u"]), dev(inp["state"]), dev(up["dy"]), dev(up["d_state"])
    cs = None
    if saved:
        _, S_final, cs = wkv.wkv6_forward_train(r, k, v, x, u, H, state=st)
    else:
        _, S_final = wkv.wkv6_forward(r, k, v, x, u, H, state=st, algo="scan")
    ref = wkv.wkv6_backward(r, k, v, x, u, H, dy, state=st, state_final=S_final, d_state=dS, algo=algo,
                            chunk_states=cs)
    n, tail = B * T * C, CHUNK * C  # a whole chunk of rows past the end
    canary = 0x7FBADBAD
    bufs = [torch.full((n + tail,), canary, dtype=torch.int32, device="cuda").view(torch.float32) for _ in range(4)]
    du = torch.empty((C,), dtype=torch.float32, device="cuda")
    du_rows = torch.empty((B, C), dtype=torch.float32, device="cuda")
    d_state_in = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
    p = wkv._ptr
    wkv.check(wkv._lib.wkv6_backward_ex(
        B, T, H, N, p(r), p(k), p(v), p(x), wkv._dtype_code(r), p(u), p(dy), p(st), None, B, p(S_final), p(dS),
        *(p(b) for b in bufs), p(du), p(du_rows), p(d_state_in), p(cs) if cs is not None else None,
        wkv._ALGOS[algo], None, wkv._stream(r)))
    torch.cuda.synchronize()
    for name, b, g in zip(("dr", "dk", "dv", "dw"), bufs, ref[:4]):
        t = b[n:].view(torch.int32)
        assert bool((t == canary).all()), f"{name}: {int((t != canary).sum())} elements past the output written"
        assert torch.equal(b[:n].view(B, T, C), g), f"{name}: differs from the exactly sized call"
    assert torch.equal(du, ref[4]) and torch.equal(d_state_in, ref[5])
