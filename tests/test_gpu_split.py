"""GPU parity of the split launch (attn_block_fwd_ws): a query tile's keys
shared between up to four workgroups, the partials combined through the
caller's workspace.  Against the fp64 oracle; repeated calls must give
identical bits and leave the workspace counters at zero.  The short blocks
force the split (the library takes it on its own only from 6144 keys); the
long blocks run the default choice.  Every output element is compared with
the oracle (the large shapes over chunks of query rows, errors accumulated
over the whole tensors)."""

import numpy as np

import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_fwd, attn_block_fwd_merge, attn_block_workspace,
                                      attn_patch_fwd, inputs)
from attention_attn_block_amd.binding import load
from tests.gpu_util import assert_bf16_close, compare_rows_chunked, to_f64, to_oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(t):
    return t.to("cuda:0")


RECORD_BYTES = 256 + 4 * 256 * (128 + 1) * 4   # one workspace record per 256-row query tile


def counters_zero(ws, B, H, Nq):
    """The arrival counters (first word of each tile's record) are all zero."""
    items = B * H * ((Nq + 255) // 256)
    words = ws[: items * RECORD_BYTES].view(items, RECORD_BYTES)[:, :4].contiguous().view(torch.int32)
    return int(words.abs().sum().item()) == 0


# Shapes whose plain grid (one 256-row query tile per workgroup) leaves part of
# a 256-CU GPU idle, so a forced split is taken.  Pieces per query tile on 256
# CUs: 2 for the first two; 2 or 3 for the next two; 3 or 4 for the last two.
# All but the first are ragged in query rows, keys or both.
SPLIT_SHAPES = [(1, 24, 2048, 2048, 128), (1, 24, 2000, 700, 128), (3, 10, 1111, 517, 72),
                (1, 150, 256, 333, 64), (2, 50, 200, 620, 128), (1, 90, 250, 700, 72)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_split_block_matches_oracle(shape, out_dtype):
    B, H, Nq, Nkv, d = shape
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=Nq + 7 * Nkv + d)
    scale = inputs.default_scale(d)
    say("case split block", shape, out_dtype)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = attn_block_workspace(qd, kd)
    O, L = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=out_dtype, workspace=ws, force_split=True)
    O2, L2 = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=out_dtype, workspace=ws,
                            force_split=True)
    Op, Lp = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2), "split launch is not deterministic"
    assert counters_zero(ws, B, H, Nq), "arrival counters not reset"
    # The combine rounds differently from the one-workgroup path, so some
    # outputs must differ: this shows the split launch ran.
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    assert_bf16_close(to_f64(O), Or, "split O")
    assert_bf16_close(to_f64(L), Lr, "split LSE")


@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_forced_split_every_head_dim(d):
    """The split kernels of every head dim: 150 heads x 256 queries x 333 keys
    (150 query tiles, 6 ragged key tiles each, cut into 2 or 3 pieces)."""
    B, H, Nq, Nkv = 1, 150, 256, 333
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=200 + d)
    scale = inputs.default_scale(d)
    say("case forced split head dim", d)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = attn_block_workspace(qd, kd)
    O, L = attn_block_fwd(qd, kd, vd, scale=scale, workspace=ws, force_split=True)
    Op, Lp = attn_block_fwd(qd, kd, vd, scale=scale)
    torch.cuda.synchronize()
    assert counters_zero(ws, B, H, Nq)
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    assert_bf16_close(to_f64(O), Or, f"split d{d} O")
    assert_bf16_close(to_f64(L), Lr, f"split d{d} LSE")


def test_plain_grid_shape_runs_unsplit():
    """768 query tiles fill three waves of 256 CUs: the workspace call takes
    the plain path and matches attn_block_fwd bit for bit."""
    q, k, v = inputs.attn_inputs(1, 24, 8192, 300, 128, "bf16", seed=11)
    q, k, v = dev(q), dev(k), dev(v)
    say("case split not taken")
    ws = attn_block_workspace(q, k)
    O, L = attn_block_fwd(q, k, v, workspace=ws, force_split=True)
    Op, Lp = attn_block_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(L, Lp)


def test_short_block_runs_unsplit_by_default():
    """Without the force flag a 2048-key block keeps the plain grid."""
    q, k, v = inputs.attn_inputs(1, 24, 2048, 2048, 128, "bf16", seed=12)
    q, k, v = dev(q), dev(k), dev(v)
    say("case split default short")
    ws = attn_block_workspace(q, k)
    O, L = attn_block_fwd(q, k, v, workspace=ws)
    Op, Lp = attn_block_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(L, Lp)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_long_block_splits_by_default_every_row(out_dtype):
    """160 query tiles against 6200 keys (97 tiles, ragged): the default
    choice splits; every output element against the oracle."""
    B, H, Nq, Nkv, d = 1, 20, 2048, 6200, 128
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=21)
    scale = inputs.default_scale(d)
    qd, kd, vd = dev(q), dev(k), dev(v)
    say("case split default long", out_dtype)
    ws = attn_block_workspace(qd, kd)
    O, L = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=out_dtype, workspace=ws)
    Op, Lp = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert counters_zero(ws, B, H, Nq)
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    del Op, Lp
    qo, ko, vo = to_oracle(q), to_oracle(k), to_oracle(v)
    compare_rows_chunked(O, L, lambda rows: oracle.ref_attn(qo, ko, vo, scale, rows=rows), Nq,
                         "long split", chunk=1024)


def test_ulysses_share_video_split_every_row():
    """A Ulysses share of the video workload on 8 devices (3 heads x 32768
    queries x 32768 keys, d128): 384 query tiles, split by default; every
    output element against the oracle."""
    B, H, N, d = 1, 3, 32768, 128
    q, k, v = inputs.attn_inputs(B, H, N, N, d, "bf16", seed=23)
    scale = inputs.default_scale(d)
    qd, kd, vd = dev(q), dev(k), dev(v)
    say("case ulysses share split")
    ws = attn_block_workspace(qd, kd)
    O, L = attn_block_fwd(qd, kd, vd, scale=scale, workspace=ws)
    Op, Lp = attn_block_fwd(qd, kd, vd, scale=scale)
    torch.cuda.synchronize()
    assert counters_zero(ws, B, H, N)
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    del Op, Lp, qd, kd, vd
    qo, ko, vo = to_oracle(q), to_oracle(k), to_oracle(v)
    (ma, rl), _ = compare_rows_chunked(
        O, L, lambda rows: oracle.ref_attn(qo, ko, vo, scale, rows=rows), N, "ulysses split")
    say(f"ulysses every element: O max-abs {ma:.2e} rel-L2 {rl:.2e}")


def test_pipefusion_patch_p8_split_every_row():
    """PipeFusion on 8 devices over the 32768-token video workload: a 4096-query
    patch at p0 = 8192 (24 heads: 384 query tiles), through attn_patch_fwd_ws.
    The spliced buffer bit for bit, every output element against the oracle,
    and the split taken (its bits differ from the plain call's)."""
    w = inputs.video_patch(Np=4096)
    p0, Np = w["p0"], 4096
    say("case pipefusion patch p8 split", tuple(w["k_buf"].shape))
    qp, kp, vp = dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"])
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    ws = attn_block_workspace(qp, kb)
    O, L = attn_patch_fwd(qp, kp, vp, kb, vb, p0, scale=w["scale"], workspace=ws)
    Op, Lp = attn_patch_fwd(qp, kp, vp, kb, vb, p0, scale=w["scale"])   # splice again: same rows
    torch.cuda.synchronize()
    assert counters_zero(ws, 1, 24, Np)
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    assert torch.equal(kb[:, :, p0:p0 + Np], kp) and torch.equal(vb[:, :, p0:p0 + Np], vp)
    del Op, Lp
    qo = to_oracle(w["q_p"])
    _, _, Kn, Vn = oracle.ref_patch(qo, to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                    to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), p0, w["scale"],
                                    rows=np.arange(0))
    assert np.array_equal(to_oracle(kb.cpu()), Kn), "spliced K buffer differs from the oracle's"
    assert np.array_equal(to_oracle(vb.cpu()), Vn), "spliced V buffer differs from the oracle's"
    compare_rows_chunked(O, L, lambda rows: oracle.ref_attn(qo, Kn, Vn, w["scale"], rows=rows),
                         Np, "patch p8 split")


@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_ring_2048px_split_fused(acc_dtype):
    """The ring share (8 KV blocks of 2048 keys, 24 heads, 2048 queries) with
    the merge fused and the split launch, from an empty accumulator whose O
    is NaN, against attention over all 16384 keys."""
    w = inputs.ring_2048px()
    q = dev(w["q"])
    B, H, Nq, d = q.shape
    o_acc = torch.full((B, H, Nq, d), float("nan"), dtype=acc_dtype, device="cuda:0")
    l_acc = torch.full((B, H, Nq), -float("inf"), device="cuda:0")
    ws = attn_block_workspace(q, dev(w["ks"][0]))
    say("case ring split fused", acc_dtype)
    for kj, vj in zip(w["ks"], w["vs"]):
        attn_block_fwd_merge(q, dev(kj), dev(vj), o_acc, l_acc, scale=w["scale"], workspace=ws,
                             force_split=True)
    torch.cuda.synchronize()
    assert counters_zero(ws, B, H, Nq)
    K = torch.cat(w["ks"], dim=2)
    V = torch.cat(w["vs"], dim=2)
    Or, Lr = oracle.ref_attn(to_oracle(w["q"]), to_oracle(K), to_oracle(V), w["scale"])
    assert_bf16_close(to_f64(o_acc), Or, "ring split fused O")
    assert_bf16_close(to_f64(l_acc), Lr, "ring split fused LSE")


def test_workspace_reused_by_a_smaller_call():
    """A workspace sized for the ring share serves a smaller split call next."""
    B, H, Nq, Nkv, d = 1, 24, 2048, 2048, 128
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=5)
    q2, k2, v2 = inputs.attn_inputs(1, 20, 2048, 1000, 128, "bf16", seed=6)
    ws = attn_block_workspace(dev(q), dev(k))
    say("case split workspace reuse")
    attn_block_fwd(dev(q), dev(k), dev(v), out_dtype=torch.float32, workspace=ws, force_split=True)
    O, L = attn_block_fwd(dev(q2), dev(k2), dev(v2), out_dtype=torch.float32, workspace=ws,
                          force_split=True)
    torch.cuda.synchronize()
    assert counters_zero(ws, B, H, Nq)
    Or, Lr = oracle.ref_attn(to_oracle(q2), to_oracle(k2), to_oracle(v2), inputs.default_scale(128))
    assert_bf16_close(to_f64(O), Or, "reuse O")
    assert_bf16_close(to_f64(L), Lr, "reuse LSE")


def test_workspace_reused_across_tile_counts_and_head_dims():
    """One workspace, made for the largest call, serves in turn: 384 query
    tiles at d128, then 192 tiles at d64 (fewer counters, other partial
    sizes), then 384 tiles at d128 again, all through forced splits.  Each
    result against the oracle, every counter back at zero after each call."""
    shapes = [(1, 24, 4096, 700, 128), (1, 24, 2048, 700, 64), (1, 24, 4096, 700, 128)]
    big = inputs.attn_inputs(*shapes[0][:4], shapes[0][4], "bf16", seed=31)
    ws = attn_block_workspace(dev(big[0]), dev(big[1]))
    for n, (B, H, Nq, Nkv, d) in enumerate(shapes):
        q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=31 + n)
        scale = inputs.default_scale(d)
        say("case workspace reuse", n, (B, H, Nq, Nkv, d))
        qd, kd, vd = dev(q), dev(k), dev(v)
        O, L = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=torch.float32, workspace=ws,
                              force_split=True)
        Op, Lp = attn_block_fwd(qd, kd, vd, scale=scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
        assert counters_zero(ws, 1, 24, 4096), f"counters not all zero after call {n}"
        Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
        assert_bf16_close(to_f64(O), Or, f"reuse {n} O")
        assert_bf16_close(to_f64(L), Lr, f"reuse {n} LSE")


def test_fp32_inputs_ignore_the_workspace():
    q, k, v = inputs.attn_inputs(1, 24, 2048, 300, 64, "f32", seed=9)
    q, k, v = dev(q), dev(k), dev(v)
    say("case split f32 inputs")
    ws = attn_block_workspace(q, k)
    O, L = attn_block_fwd(q, k, v, workspace=ws, force_split=True)
    Op, Lp = attn_block_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(L, Lp)
    assert load() is not None
