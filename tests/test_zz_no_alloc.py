"""cfg_combine_relmae_noalloc (partial sums in the library's fixed device
array, no caller workspace) against cfg_combine_relmae (caller workspace),
through the C ABI: the same kernels, so the same bits.  Two calls in a row,
the second on a smaller input, so the second reads nothing the first left
behind; then the larger size again."""

import ctypes

import pytest
import torch

import oracle
from attention_attn_block_amd import binding, cfg_combine_relmae
from tests.gpu_util import assert_f32_close, to_f64, to_oracle

pytestmark = pytest.mark.gpu


def noalloc(u, c, s, out, relmae):
    lib = binding.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream(u.device).cuda_stream)
    rc = lib.cfg_combine_relmae_noalloc(u.data_ptr(), c.data_ptr(), out.data_ptr(), u.numel(),
                                        float(s), relmae.data_ptr(), stream)
    assert rc == binding.DIT_OK, binding.status_string(rc)


def test_noalloc_matches_workspace_call():
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(4242)
    sizes = [(1 << 22) + 5, 70001, (1 << 22) + 5]   # large, smaller, large again
    data = {}
    for n in sorted(set(sizes)):
        u = torch.randn(n, generator=g)
        c = u + 0.25 * torch.randn(n, generator=g)
        data[n] = (u, c)
    for k, n in enumerate(sizes):
        print("case noalloc call", k, "n =", n, flush=True)
        u, c = data[n]
        gu, gc = u.to(dev), c.to(dev)
        want_out, want_rm = cfg_combine_relmae(gu, gc, 3.5)
        out = torch.full_like(gu, float("nan"))
        rm = torch.full((4,), float("nan"), device=dev)[:1]
        noalloc(gu, gc, 3.5, out, rm)
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), "out differs from cfg_combine_relmae"
        assert torch.equal(rm, want_rm), (float(rm.item()), float(want_rm.item()))
        assert_f32_close(to_f64(out), oracle.ref_cfg(to_oracle(u), to_oracle(c), 3.5), "noalloc out")
        ref = oracle.ref_cfg_relmae(to_oracle(u), to_oracle(c))
        assert abs(float(rm.item()) - ref) <= 1e-5 * ref
