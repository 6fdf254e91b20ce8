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


class WholeTensorError:
    """Error of one output tensor accumulated over row chunks, so that a call
    whose oracle result is too large to hold at once is still compared over
    every element: max-abs over all elements and rel-L2 = ||got - ref|| /
    ||ref|| over the whole tensor (sums of squares in fp64)."""

    def __init__(self, what):
        self.what = what
        self.err2 = 0.0
        self.ref2 = 0.0
        self.max_abs = 0.0
        self.count = 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (self.what, got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{self.what}: non-finite output"
        diff = got - ref
        self.err2 += float(np.sum(diff * diff))
        self.ref2 += float(np.sum(ref * ref))
        if diff.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(diff))))
        self.count += diff.size

    def rel_l2(self):
        return float(np.sqrt(self.err2) / (np.sqrt(self.ref2) if self.ref2 > 0 else 1.0))

    def assert_bf16(self, expected_count):
        assert self.count == expected_count, f"{self.what}: compared {self.count} of {expected_count}"
        ma, rl = self.max_abs, self.rel_l2()
        assert ma <= BF16_MAX_ABS and rl <= BF16_REL_L2, \
            f"{self.what}: max-abs {ma:.3e} rel-L2 {rl:.3e} over all {self.count} elements"
        return ma, rl


def compare_rows_chunked(O, L, ref_rows, n_rows, what, chunk=2048):
    """Compare a GPU result O [B, H, n_rows, d], L [B, H, n_rows] with the
    oracle over every query row, `chunk` rows at a time: ref_rows(rows) must
    return the oracle's (O, LSE) for those rows of every (batch, head).
    Asserts the bf16 tolerances over the whole tensors and returns
    ((max-abs, rel-L2) of O, (max-abs, rel-L2) of LSE)."""
    eo, el = WholeTensorError(what + " O"), WholeTensorError(what + " LSE")
    Og = O.detach().cpu()
    Lg = L.detach().cpu()
    for a in range(0, n_rows, chunk):
        rows = np.arange(a, min(a + chunk, n_rows))
        Or, Lr = ref_rows(rows)
        eo.add(Og[:, :, a:a + rows.size].double().numpy(), Or)
        el.add(Lg[:, :, a:a + rows.size].double().numpy(), Lr)
    return eo.assert_bf16(O.numel()), el.assert_bf16(L.numel())
