"""GPU parity of attn_patch_fwd_strided: a PipeFusion patch made of several
evenly spaced runs of buffer rows (a band of spatial rows across every frame
of a video, in frame-major token order), against the oracle's
ref_patch_strided.  The spliced K and V buffers are compared bit for bit and
O and LSE over every element."""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_workspace, attn_patch_fwd,
                                      attn_patch_fwd_strided, inputs)
from tests.gpu_util import assert_bf16_close, compare_rows_chunked, to_f64, to_oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(t):
    return t.to("cuda:0")


def run_and_check(w, out_dtype=torch.bfloat16, workspace=None, what="strided"):
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    O, L = attn_patch_fwd_strided(dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"]), kb, vb, w["p0"],
                                  w["run_len"], w["run_stride"], scale=w["scale"],
                                  out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    Or, Lr, Kn, Vn = oracle.ref_patch_strided(
        to_oracle(w["q_p"]), to_oracle(w["k_p"]), to_oracle(w["v_p"]), to_oracle(w["k_buf"]),
        to_oracle(w["v_buf"]), w["p0"], w["run_len"], w["run_stride"], w["scale"])
    assert np.array_equal(to_oracle(kb.cpu()), Kn), f"{what}: spliced K buffer differs"
    assert np.array_equal(to_oracle(vb.cpu()), Vn), f"{what}: spliced V buffer differs"
    assert_bf16_close(to_f64(O), Or, what + " O")
    assert_bf16_close(to_f64(L), Lr, what + " LSE")
    return O, L


@pytest.mark.parametrize("p", [0, 1, 2, 3])
def test_slab_patch_each_position_small(p):
    """The video recipe shrunk to 4 frames of 8 x 16 patches, 3 heads: patch p
    is spatial rows [2p, 2p + 2) of every frame, 4 runs of 32 tokens."""
    w = inputs.video_slab_patch(p=p, frames=4, height=8, width=16, slab=2, H=3)
    say("case slab patch small", p, w["p0"], w["run_len"], w["run_stride"], w["n_runs"])
    run_and_check(w, torch.float32, what=f"slab p{p}")


def ragged_layout(B, H, N, d, p0, run_len, run_stride, n_runs, seed):
    q_p, k_p, v_p = inputs.attn_inputs(B, H, run_len * n_runs, run_len * n_runs, d, "bf16",
                                       seed=seed)
    _, k_buf, v_buf = inputs.attn_inputs(B, H, 1, N, d, "bf16", seed=seed + 1)
    return dict(q_p=q_p, k_p=k_p, v_p=v_p, k_buf=k_buf, v_buf=v_buf, p0=p0, run_len=run_len,
                run_stride=run_stride, n_runs=n_runs, scale=inputs.default_scale(d))


@pytest.mark.parametrize("layout", [
    # (B, H, N, d, p0, run_len, run_stride, n_runs)
    (2, 3, 600, 128, 13, 37, 100, 5),      # ragged runs and tiles
    (1, 2, 300, 72, 0, 1, 7, 40),          # one-row runs
    (1, 2, 257, 64, 0, 64, 64, 4),         # touching runs: one contiguous range
    (1, 1, 129, 128, 128, 1, 5, 1),        # one run of one row, at the last row
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_ragged_layouts(layout, out_dtype):
    B, H, N, d, p0, run_len, stride, n_runs = layout
    w = ragged_layout(B, H, N, d, p0, run_len, stride, n_runs, seed=N + d + run_len)
    say("case strided layout", layout, out_dtype)
    run_and_check(w, out_dtype, what=f"layout {layout}")


def test_one_run_is_the_contiguous_call():
    """n_runs = 1 is attn_patch_fwd: the same bits."""
    w = inputs.video_patch(N=700, Np=250, p0=111, H=3)
    say("case strided one run = contiguous")
    args = [dev(w[n]) for n in ("q_p", "k_p", "v_p")]
    kb1, vb1 = dev(w["k_buf"]), dev(w["v_buf"])
    kb2, vb2 = kb1.clone(), vb1.clone()
    O1, L1 = attn_patch_fwd(*args, kb1, vb1, w["p0"], scale=w["scale"])
    O2, L2 = attn_patch_fwd_strided(*args, kb2, vb2, w["p0"], 250, 0, scale=w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.equal(kb1, kb2) and torch.equal(vb1, vb2)


@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_every_head_dim(d):
    w = ragged_layout(1, 2, 400, d, 5, 21, 90, 4, seed=800 + d)
    say("case strided head dim", d)
    run_and_check(w, what=f"strided d{d}")


def test_video_slab_patch_full_size_every_row():
    """The video workload (24 heads, 8 frames of 64 x 64, d128) cut into row
    slabs: patch 1 is spatial rows 16..31 of every frame, 8 runs of 1024
    tokens (8192 queries) against the 32768-row buffer.  Spliced buffers bit
    for bit, O and LSE over every element."""
    w = inputs.video_slab_patch(p=1)
    say("case video slab patch full size", w["p0"], w["run_len"], w["run_stride"], w["n_runs"])
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    O, L = attn_patch_fwd_strided(dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"]), kb, vb, w["p0"],
                                  w["run_len"], w["run_stride"], scale=w["scale"])
    torch.cuda.synchronize()
    qo = to_oracle(w["q_p"])
    _, _, Kn, Vn = oracle.ref_patch_strided(qo, to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                            to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), w["p0"],
                                            w["run_len"], w["run_stride"], w["scale"],
                                            rows=np.arange(0))
    assert np.array_equal(to_oracle(kb.cpu()), Kn), "spliced K buffer differs from the oracle's"
    assert np.array_equal(to_oracle(vb.cpu()), Vn), "spliced V buffer differs from the oracle's"
    compare_rows_chunked(O, L, lambda rows: oracle.ref_attn(qo, Kn, Vn, w["scale"], rows=rows),
                         qo.shape[2], "video slab patch")


def test_video_slab_patch_p8_split_every_row():
    """PipeFusion on 8 devices with row-slab patches: 8 spatial rows of every
    frame (8 runs of 512 tokens, 4096 queries: 384 query tiles) through the
    split launch, which it takes by default.  Every element against the
    oracle, and the bits differ from the plain call's."""
    w = inputs.video_slab_patch(p=5, slab=8)
    say("case video slab patch p8 split", w["p0"], w["run_len"], w["run_stride"], w["n_runs"])
    qp, kp, vp = dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"])
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    ws = attn_block_workspace(qp, kb)
    O, L = attn_patch_fwd_strided(qp, kp, vp, kb, vb, w["p0"], w["run_len"], w["run_stride"],
                                  scale=w["scale"], workspace=ws)
    Op, Lp = attn_patch_fwd_strided(qp, kp, vp, kb, vb, w["p0"], w["run_len"], w["run_stride"],
                                    scale=w["scale"])
    torch.cuda.synchronize()
    assert not (torch.equal(O, Op) and torch.equal(L, Lp)), "split launch was not taken"
    del Op, Lp
    qo = to_oracle(w["q_p"])
    _, _, Kn, Vn = oracle.ref_patch_strided(qo, to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                            to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), w["p0"],
                                            w["run_len"], w["run_stride"], w["scale"],
                                            rows=np.arange(0))
    assert np.array_equal(to_oracle(kb.cpu()), Kn), "spliced K buffer differs from the oracle's"
    compare_rows_chunked(O, L, lambda rows: oracle.ref_attn(qo, Kn, Vn, w["scale"], rows=rows),
                         qo.shape[2], "video slab patch p8 split")
