"""GPU parity of attn_ring_fwd: one device's queries against every KV block of
a ring step, resident in buffers of their own, in one launch.  Against the
oracle's attention over the concatenated keys, every output element."""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_fwd, attn_block_workspace, attn_ring_fwd,
                                      inputs)
from tests.gpu_util import assert_bf16_close, to_f64, to_oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(t):
    return t.to("cuda:0")


def blocks_of(k, v, cuts):
    return ([k[:, :, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])],
            [v[:, :, a:b].contiguous() for a, b in zip(cuts[:-1], cuts[1:])])


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", ["plain", "split", "default"])
def test_ring_2048px_one_launch(out_dtype, mode):
    """The ring share (24 heads, 2048 queries, 8 KV blocks of 2048 keys, d128)
    in one launch: plain grid, forced split, and the library's own choice with
    a workspace (it splits: 256 key tiles per query tile)."""
    w = inputs.ring_2048px()
    q = dev(w["q"])
    ks, vs = [dev(k) for k in w["ks"]], [dev(v) for v in w["vs"]]
    kw = {} if mode == "plain" else {"workspace": attn_block_workspace(q, ks[0]),
                                     "force_split": mode == "split"}
    say("case ring one launch", out_dtype, mode)
    O, L = attn_ring_fwd(q, ks, vs, scale=w["scale"], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    K = torch.cat(w["ks"], dim=2)
    V = torch.cat(w["vs"], dim=2)
    Or, Lr = oracle.ref_attn(to_oracle(w["q"]), to_oracle(K), to_oracle(V), w["scale"])
    assert_bf16_close(to_f64(O), Or, f"ring one launch {mode} O")
    assert_bf16_close(to_f64(L), Lr, f"ring one launch {mode} LSE")


@pytest.mark.parametrize("shape", [
    # (B, H, Nq, block keys, n_blocks, d)
    (1, 3, 500, 300, 3, 128),     # ragged blocks (5 tiles, the last one 44 keys) and queries
    (2, 2, 257, 50, 5, 72),       # one ragged tile per block
    (1, 4, 130, 64, 16, 64),      # sixteen blocks of exactly one tile
    (1, 2, 70, 1, 7, 8),          # one key per block
])
@pytest.mark.parametrize("split", [False, True])
def test_ragged_block_sets(shape, split):
    B, H, Nq, nb_keys, nb, d = shape
    q, k, v = inputs.attn_inputs(B, H, Nq, nb_keys * nb, d, "bf16", seed=nb_keys + 7 * nb + d)
    scale = inputs.default_scale(d)
    cuts = [i * nb_keys for i in range(nb + 1)]
    kb, vb = blocks_of(k, v, cuts)
    gq = dev(q)
    kw = {"workspace": attn_block_workspace(gq, dev(kb[0])), "force_split": True} if split else {}
    say("case ragged block set", shape, split)
    O, L = attn_ring_fwd(gq, [dev(t) for t in kb], [dev(t) for t in vb], scale=scale,
                         out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    assert_bf16_close(to_f64(O), Or, f"block set {shape} O")
    assert_bf16_close(to_f64(L), Lr, f"block set {shape} LSE")


def test_one_block_is_the_block_call():
    """A set of one block gives attn_block_fwd's bits."""
    q, k, v = inputs.attn_inputs(1, 5, 600, 900, 128, "bf16", seed=61)
    q, k, v = dev(q), dev(k), dev(v)
    say("case one-block set")
    O1, L1 = attn_block_fwd(q, k, v, out_dtype=torch.float32)
    O2, L2 = attn_ring_fwd(q, [k], [v], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_repeated_block():
    """The same block twice is attention over the keys listed twice: O as for
    one copy (to rounding) and LSE + ln 2."""
    q, k, v = inputs.attn_inputs(1, 3, 300, 400, 64, "bf16", seed=62)
    scale = inputs.default_scale(64)
    gq, gk, gv = dev(q), dev(k), dev(v)
    say("case repeated block")
    O, L = attn_ring_fwd(gq, [gk, gk], [gv, gv], scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(torch.cat([k, k], 2)),
                             to_oracle(torch.cat([v, v], 2)), scale)
    assert_bf16_close(to_f64(O), Or, "repeated O")
    assert_bf16_close(to_f64(L), Lr, "repeated LSE")
    assert np.allclose(Lr, oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)[1]
                       + np.log(2.0))


@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_every_head_dim(d):
    q, k, v = inputs.attn_inputs(1, 2, 300, 3 * 150, d, "bf16", seed=900 + d)
    scale = inputs.default_scale(d)
    kb, vb = blocks_of(k, v, [0, 150, 300, 450])
    gq = dev(q)
    say("case block set head dim", d)
    for split in (False, True):
        kw = {"workspace": attn_block_workspace(gq, dev(kb[0])), "force_split": True} if split else {}
        O, L = attn_ring_fwd(gq, [dev(t) for t in kb], [dev(t) for t in vb], scale=scale, **kw)
        torch.cuda.synchronize()
        Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
        assert_bf16_close(to_f64(O), Or, f"block set d{d} split={split} O")
        assert_bf16_close(to_f64(L), Lr, f"block set d{d} split={split} LSE")


def test_scores_growing_across_blocks_fall_back():
    """Scores that rise block after block overflow the fast path's reference
    (the first tile's maximum) and take the exact path; plain and split."""
    B, H, Nq, nb_keys, nb, d = 1, 40, 200, 128, 5, 72
    g = torch.Generator().manual_seed(63)
    tile = (torch.arange(nb_keys * nb) // 64).float()
    k = (4.0 * tile)[None, None, :, None] + 0.3 * torch.randn(B, H, nb_keys * nb, d, generator=g)
    q = 1.0 + 0.05 * torch.randn(B, H, Nq, d, generator=g)
    v = torch.randn(B, H, nb_keys * nb, d, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    kb, vb = blocks_of(k, v, [i * nb_keys for i in range(nb + 1)])
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), 0.125)
    gq = dev(q)
    say("case block set growing scores")
    for split in (False, True):
        kw = {"workspace": attn_block_workspace(gq, dev(kb[0])), "force_split": True} if split else {}
        O, L = attn_ring_fwd(gq, [dev(t) for t in kb], [dev(t) for t in vb], scale=0.125,
                             out_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        assert_bf16_close(to_f64(O), Or, f"growing split={split} O")
        assert_bf16_close(to_f64(L), Lr, f"growing split={split} LSE")
