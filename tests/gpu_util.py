"""Helpers for the GPU parity tests: tensor -> oracle input, error metrics and
the tolerances the comparisons use."""

import numpy as np
import torch

# bf16 inputs: max-abs <= 2e-2 and relative L2 <= 5e-3; fp32 path: rel-L2 <= 1e-5.
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_REL_L2 = 1e-5


def to_oracle(t):
    """CPU numpy view the oracle reads: bf16 as raw uint16 bits, fp32 as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def to_f64(t):
    t = t.detach().cpu()
    return t.double().numpy()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def max_abs(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def assert_bf16_close(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma, rl = max_abs(got, ref), rel_l2(got, ref)
    assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, f"{what}: max-abs {ma:.3e} rel-L2 {rl:.3e}"
    return ma, rl


def assert_f32_close(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rl = rel_l2(got, ref)
    assert rl <= F32_REL_L2, f"{what}: rel-L2 {rl:.3e}"
    return rl


def assert_close(got, ref, fp32_path, what):
    if fp32_path:
        return assert_f32_close(got, ref, what)
    return assert_bf16_close(got, ref, what)
