"""Helpers of the GPU parity tests: device copies of seeded inputs and the
tolerance checks (fp32: max error relative to max(|o|, rms(o)) <= 2e-5;
bf16 inputs: max abs <= 2e-2 and mean abs <= 5e-3)."""
import numpy as np
import torch

FP32_REL = 2e-5
BF16_MAX = 2e-2
BF16_MEAN = 5e-3


def dev(a, device="cuda"):
    """numpy input (uint16 = bf16 bit patterns) -> device tensor with the same bytes."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def fp32_relerr(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), scale)))


def assert_fp32(got, ref, what=""):
    e = fp32_relerr(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert e <= FP32_REL, f"{what}: max relative error {e:.3e} > {FP32_REL}"
    return e


def assert_bf16(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max abs {mx:.3e} (<= {BF16_MAX}), mean abs {mean:.3e} (<= {BF16_MEAN})"
    return mx, mean
