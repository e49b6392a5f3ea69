"""Seeded synthetic inputs shared by the fp64 oracle, the tests and the bench.

This module only draws random numbers and rounds them into the stored input
precision (bf16 round-to-nearest-even).  It contains none of the WKV
arithmetic, so the oracle and the HIP path can both consume its arrays while
sharing no computation.

Distributions follow the workloads the WKV operator is run on:

* v4 (the RWKV-v4 time-mix walk-through, ``RUN_CUDA(B, T, C, time_decay,
  time_first, k, v)`` call): ``time_decay ~ U(-5, 1)`` so the per-step decay
  is ``exp(-exp(time_decay))``, ``time_first (u) ~ N(0, 0.5)``,
  ``k, v ~ N(0, 1)`` and optionally the receptance ``r ~ N(0, 1)`` whose
  sigmoid gates the output, all fp32.
* v5 (multi-head, static decay): ``r, k, v ~ N(0, 0.5)`` rounded to bf16,
  decay parameter ``x ~ U(-6, -0.5)`` per head-channel (fp32, decay
  ``exp(-exp(x))``), ``u ~ N(0, 0.5)`` fp32.
* v6 (the rwkv_ops ``RWKV6_OP`` call table: r, k, v, w of shape
  ``(batch, seq, hidden)``, u of ``(heads, head_size)``): as v5 but the decay
  parameter is per token and channel, ``x ~ U(-6, 0)`` rounded to bf16 like
  r, k, v.
* v6 backward: upstream gradients ``dy ~ N(0, 1)`` fp32 of the output and
  ``dS ~ N(0, 0.1)`` fp32 of the final state (a training step's incoming
  gradients; drawn by their own generator, after the forward inputs).
* varlen serving (the web-rwkv batched-inference section: slots, a per-call
  ``token_chunk_size`` budget): prompt lengths ``~ U{1..2048}`` per slot,
  initial states ``~ N(0, 0.1)`` fp32, per-token inputs as v6.
* v7 (the rwkv_ops ``generalized_delta_rule`` call: r, w, k, v, a, b of shape
  [B, T, H, K]): the decay parameter ``w ~ U(-6, 0)`` (decay
  ``exp(-exp(w))`` between 0.37 and 0.9975, as v6), r, k,
  v ~ N(0, 0.5), and the delta-rule pair of the RWKV-7 time mix: a unit
  direction ``kappa`` per (token, head) (an N(0, 1) vector scaled to length
  1) with ``a = -kappa`` and ``b = kappa * beta``, ``beta ~ U(0, 1)`` per
  channel; all rounded to bf16 when the dtype is bf16.

``N(m, s)`` means standard deviation ``s``.  Every generator uses numpy's
PCG64 (``default_rng(seed)``) with a fixed draw order: lengths, decay
parameter, u, r, k, v, initial state, then decode-step inputs.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "bf16_to_f32", "stored_f32",
    "wkv4_inputs", "wkv5_inputs", "wkv6_inputs", "varlen_inputs", "wkv6_upstream", "wkv7_inputs",
]


def bf16_round(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_f32(a) -> np.ndarray:
    """The exact stored value of an input array as fp32 (bf16 patterns are widened)."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _uniform(rng, shape, lo, hi):
    return rng.random(shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)


def _store(a, dtype):
    if dtype == "bf16":
        return bf16_round(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown input dtype {dtype!r}")


def wkv4_inputs(B, T, C, seed=0, with_r=False, dtype="f32", init_state=False,
                decode_steps=0, tau_range=(-5.0, 1.0)):
    """Inputs of the v4 channel-wise recurrence.

    Returns a dict with ``tau`` (time_decay, [C] fp32), ``u`` (time_first,
    [C] fp32), ``k``, ``v`` and optionally ``r`` ([B, T, C] in ``dtype``),
    ``state`` ([B, 3, C] fp32 planes a, b, p with b > 0, or None) and
    ``decode`` (list of per-step dicts with ``k``, ``v``, ``r`` of shape
    [B, 1, C]).
    """
    rng = np.random.default_rng(seed)
    tau = _uniform(rng, (C,), *tau_range)
    u = _normal(rng, (C,), 0.5)
    r = _store(_normal(rng, (B, T, C), 1.0), dtype) if with_r else None
    k = _store(_normal(rng, (B, T, C), 1.0), dtype)
    v = _store(_normal(rng, (B, T, C), 1.0), dtype)
    state = None
    if init_state:
        a = _normal(rng, (B, C), 1.0)
        b = _uniform(rng, (B, C), 0.5, 2.0)
        p = _uniform(rng, (B, C), -2.0, 2.0)
        state = np.stack([a, b, p], axis=1).astype(np.float32)
    decode = []
    for _ in range(decode_steps):
        step = {"r": _store(_normal(rng, (B, 1, C), 1.0), dtype) if with_r else None}
        step["k"] = _store(_normal(rng, (B, 1, C), 1.0), dtype)
        step["v"] = _store(_normal(rng, (B, 1, C), 1.0), dtype)
        decode.append(step)
    return dict(B=B, T=T, C=C, tau=tau, u=u, r=r, k=k, v=v, state=state,
                decode=decode, dtype=dtype)


def wkv5_inputs(B, T, H, N, seed=0, dtype="bf16", x_range=(-6.0, -0.5),
                init_state=None, state_std=0.1):
    """Inputs of the v5 recurrence (static decay).

    ``x`` is the [H*N] fp32 decay parameter (decay ``exp(-exp(x))``), ``u``
    [H*N] fp32, ``r``, ``k``, ``v`` [B, T, H*N] in ``dtype``.  With
    ``init_state = n`` an [n, H, N, N] fp32 initial state ``~ N(0,
    state_std)`` is drawn.
    """
    C = H * N
    rng = np.random.default_rng(seed)
    x = _uniform(rng, (C,), *x_range)
    u = _normal(rng, (C,), 0.5)
    r = _store(_normal(rng, (B, T, C), 0.5), dtype)
    k = _store(_normal(rng, (B, T, C), 0.5), dtype)
    v = _store(_normal(rng, (B, T, C), 0.5), dtype)
    state = None
    if init_state:
        state = _normal(rng, (init_state, H, N, N), state_std)
    return dict(B=B, T=T, H=H, N=N, x=x, u=u, r=r, k=k, v=v, state=state, dtype=dtype)


def wkv6_inputs(B, T, H, N, seed=0, dtype="bf16", x_range=(-6.0, 0.0),
                init_state=None, state_std=0.1):
    """Inputs of the v6 recurrence (per-token decay).

    As :func:`wkv5_inputs` but ``x`` is [B, T, H*N] stored in ``dtype``.
    """
    C = H * N
    rng = np.random.default_rng(seed)
    x = _store(_uniform(rng, (B, T, C), *x_range), dtype)
    u = _normal(rng, (C,), 0.5)
    r = _store(_normal(rng, (B, T, C), 0.5), dtype)
    k = _store(_normal(rng, (B, T, C), 0.5), dtype)
    v = _store(_normal(rng, (B, T, C), 0.5), dtype)
    state = None
    if init_state:
        state = _normal(rng, (init_state, H, N, N), state_std)
    return dict(B=B, T=T, H=H, N=N, x=x, u=u, r=r, k=k, v=v, state=state, dtype=dtype)


def varlen_inputs(num_slots, H, N, seed=0, max_prompt=2048, decode_steps=256,
                  dtype="bf16", x_range=(-6.0, 0.0), state_std=0.1, lengths=None):
    """Inputs of the batched varlen serving workload.

    Returns ``lengths`` [S] int32 (prompt lengths ``~ U{1..max_prompt}``
    unless given), packed prompt arrays ``x, r, k, v`` of shape
    [sum(lengths), H*N] (slot s occupies rows ``off[s]:off[s]+lengths[s]``
    with ``off`` the exclusive prefix sum), ``u`` [H*N] fp32, ``state``
    [S, H, N, N] fp32 ``~ N(0, state_std)`` and ``decode`` arrays
    ``x, r, k, v`` of shape [decode_steps, S, H*N].
    """
    C = H * N
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_prompt + 1, size=num_slots).astype(np.int32)
    else:
        lengths = np.asarray(lengths, dtype=np.int32)
    total = int(lengths.sum())
    x = _store(_uniform(rng, (total, C), *x_range), dtype)
    u = _normal(rng, (C,), 0.5)
    r = _store(_normal(rng, (total, C), 0.5), dtype)
    k = _store(_normal(rng, (total, C), 0.5), dtype)
    v = _store(_normal(rng, (total, C), 0.5), dtype)
    state = _normal(rng, (num_slots, H, N, N), state_std)
    dec = {}
    dec["x"] = _store(_uniform(rng, (decode_steps, num_slots, C), *x_range), dtype)
    dec["r"] = _store(_normal(rng, (decode_steps, num_slots, C), 0.5), dtype)
    dec["k"] = _store(_normal(rng, (decode_steps, num_slots, C), 0.5), dtype)
    dec["v"] = _store(_normal(rng, (decode_steps, num_slots, C), 0.5), dtype)
    return dict(S=num_slots, H=H, N=N, lengths=lengths, x=x, u=u, r=r, k=k, v=v,
                state=state, decode=dec, dtype=dtype)



def wkv6_upstream(B, T, H, N, seed=0, with_state=True):
    """Upstream gradients of a v6 forward call: ``dy`` [B, T, H*N] ``~ N(0, 1)`` and
    (optionally) ``d_state`` [B, H, N, N] ``~ N(0, 0.1)``, both fp32."""
    rng = np.random.default_rng(seed)
    dy = _normal(rng, (B, T, H * N), 1.0)
    ds = _normal(rng, (B, H, N, N), 0.1) if with_state else None
    return dict(dy=dy, d_state=ds)


def wkv7_inputs(B, T, H, N, seed=0, dtype="bf16", x_range=(-6.0, 0.0), init_state=None, state_std=0.1):
    """Inputs of the v7 generalized delta rule.

    ``r, w, k, v, a, b``: [B, T, H*N] in ``dtype`` (``w`` the decay parameter);
    with ``init_state = n`` an [n, H, N, N] fp32 initial state ``~ N(0,
    state_std)``.  Draw order: decay parameter, r, k, v, kappa, beta, state.
    """
    C = H * N
    rng = np.random.default_rng(seed)
    w = _store(_uniform(rng, (B, T, C), *x_range), dtype)
    r = _store(_normal(rng, (B, T, C), 0.5), dtype)
    k = _store(_normal(rng, (B, T, C), 0.5), dtype)
    v = _store(_normal(rng, (B, T, C), 0.5), dtype)
    kappa = _normal(rng, (B, T, H, N), 1.0)
    kappa /= np.sqrt(np.sum(kappa * kappa, axis=-1, keepdims=True, dtype=np.float32))
    beta = _uniform(rng, (B, T, H, N), 0.0, 1.0)
    a = _store((-kappa).reshape(B, T, C), dtype)
    b = _store((kappa * beta).reshape(B, T, C), dtype)
    state = None
    if init_state:
        state = _normal(rng, (init_state, H, N, N), state_std)
    return dict(B=B, T=T, H=H, N=N, w=w, r=r, k=k, v=v, a=a, b=b, state=state, dtype=dtype)
