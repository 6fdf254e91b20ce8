"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case compares every output element with the oracle.  The full-size
PipeFusion workload and the long blocks are too large for one oracle call:
the oracle runs over chunks of query rows and the errors are accumulated
over the whole output tensors (max-abs over all elements, rel-L2 over the
whole tensor); the spliced buffer is compared bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_fwd, attn_block_fwd_merge, attn_lse_merge,
                                      attn_patch_fwd, cfg_combine, cfg_combine_relmae, inputs)
from tests.gpu_util import (assert_bf16_close, assert_close, assert_f32_close,
                            compare_rows_chunked, to_f64, to_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no fallback)"
    torch.cuda.init()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def dev(t):
    return t.to("cuda:0")


def run_attn(q, k, v, scale, out_dtype):
    O, L = attn_block_fwd(dev(q), dev(k), dev(v), scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return O, L


def check_attn(q, k, v, scale, out_dtype, what):
    say("case", what, tuple(q.shape), tuple(k.shape), out_dtype)
    O, L = run_attn(q, k, v, scale, out_dtype)
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    fp32 = q.dtype == torch.float32
    assert_close(to_f64(O), Or, fp32, what + " O")
    assert_close(to_f64(L), Lr, fp32, what + " LSE")
    return O, L


# ---------------------------------------------------------------------------
# Workloads at their stated sizes
# ---------------------------------------------------------------------------

def test_tiny_f32_full_and_four_block_merge():
    w = inputs.tiny_f32()
    q, k, v, scale = w["q"], w["k"], w["v"], w["scale"]
    check_attn(q, k, v, scale, torch.float32, "tiny_f32 full")
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    nb = w["blocks"]
    step = k.shape[2] // nb
    say("case tiny_f32 4-block fold")
    acc_o, acc_l = None, None
    for j in range(nb):
        Oj, Lj = run_attn(q, k[:, :, j * step:(j + 1) * step].contiguous(),
                          v[:, :, j * step:(j + 1) * step].contiguous(), scale, torch.float32)
        if acc_o is None:
            acc_o, acc_l = Oj, Lj
        else:
            attn_lse_merge(acc_o, acc_l, Oj, Lj)
    torch.cuda.synchronize()
    assert_f32_close(to_f64(acc_o), Or, "fold O")
    assert_f32_close(to_f64(acc_l), Lr, "fold LSE")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dit_xl_256_attention(out_dtype):
    w = inputs.dit_xl_256()
    check_attn(w["q"], w["k"], w["v"], w["scale"], out_dtype, "dit_xl_256")


def test_dit_xl_256_cfg():
    w = inputs.dit_xl_256()
    say("case dit_xl_256 cfg")
    out = cfg_combine(dev(w["eps_u"]), dev(w["eps_c"]), w["s"])
    torch.cuda.synchronize()
    ref = oracle.ref_cfg(to_oracle(w["eps_u"]), to_oracle(w["eps_c"]), w["s"])
    assert_f32_close(to_f64(out), ref, "cfg")


def test_pixart_1024_attention():
    w = inputs.pixart_1024()
    check_attn(w["q"], w["k"], w["v"], w["scale"], torch.bfloat16, "pixart_1024")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_ring_2048px_eight_blocks_merged(out_dtype):
    """8 sequential block calls folded with 7 merges equal attention over all
    16384 keys.  fp32 partials are the default reading; bf16 partials are
    checked too, against the same tolerances."""
    w = inputs.ring_2048px()
    q = dev(w["q"])
    acc_o = acc_l = None
    say("case ring_2048px", out_dtype)
    for kj, vj in zip(w["ks"], w["vs"]):
        Oj, Lj = attn_block_fwd(q, dev(kj), dev(vj), scale=w["scale"], out_dtype=out_dtype)
        if acc_o is None:
            acc_o, acc_l = Oj, Lj
        else:
            attn_lse_merge(acc_o, acc_l, Oj, Lj)
    torch.cuda.synchronize()
    K = torch.cat(w["ks"], dim=2)
    V = torch.cat(w["vs"], dim=2)
    Or, Lr = oracle.ref_attn(to_oracle(w["q"]), to_oracle(K), to_oracle(V), w["scale"])
    assert_bf16_close(to_f64(acc_o), Or, "ring O")
    assert_bf16_close(to_f64(acc_l), Lr, "ring LSE")


def test_video_patch_full_size_every_row():
    """The PipeFusion workload at its stated size (24 heads, 8192 patch queries
    at p0 = 8192, 32768-row buffer): the spliced buffer bit for bit, and O and
    LSE against the oracle over every element (row chunks of the oracle,
    errors accumulated over the whole tensors)."""
    w = inputs.video_patch()
    p0 = w["p0"]
    Np = w["q_p"].shape[2]
    say("case video_patch full size", tuple(w["k_buf"].shape))
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    kb0, vb0 = kb.clone(), vb.clone()
    O, L = attn_patch_fwd(dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"]), kb, vb, p0,
                          scale=w["scale"])
    torch.cuda.synchronize()
    # the spliced buffer, bit for bit
    kp, vp = dev(w["k_p"]), dev(w["v_p"])
    assert torch.equal(kb[:, :, p0:p0 + Np], kp) and torch.equal(vb[:, :, p0:p0 + Np], vp)
    assert torch.equal(kb[:, :, :p0], kb0[:, :, :p0]) and torch.equal(kb[:, :, p0 + Np:], kb0[:, :, p0 + Np:])
    assert torch.equal(vb[:, :, :p0], vb0[:, :, :p0]) and torch.equal(vb[:, :, p0 + Np:], vb0[:, :, p0 + Np:])
    del kb0, vb0
    qp = to_oracle(w["q_p"])
    _, _, Kn, Vn = oracle.ref_patch(qp, to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                    to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), p0, w["scale"],
                                    rows=np.arange(0))
    assert np.array_equal(to_oracle(kb.cpu()), Kn), "spliced K buffer differs from the oracle's"
    assert np.array_equal(to_oracle(vb.cpu()), Vn), "spliced V buffer differs from the oracle's"
    (ma, rl), (lma, lrl) = compare_rows_chunked(
        O, L, lambda rows: oracle.ref_attn(qp, Kn, Vn, w["scale"], rows=rows), Np, "video_patch")
    say(f"video_patch every element: O max-abs {ma:.2e} rel-L2 {rl:.2e}; LSE {lma:.2e} {lrl:.2e}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_long_ragged_block_every_row(out_dtype):
    """A long KV block whose length is not a multiple of the 64-key tile
    (40 037 keys: 625 full tiles and a 37-row tail) and a ragged query count,
    at the video workload's d = 128: every output element against the oracle."""
    B, H, Nq, Nkv, d = 1, 3, 1000, 40037, 128
    say("case long ragged block", (B, H, Nq, Nkv, d), out_dtype)
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16", seed=77)
    scale = inputs.default_scale(d)
    O, L = run_attn(q, k, v, scale, out_dtype)
    qo, ko, vo = to_oracle(q), to_oracle(k), to_oracle(v)
    compare_rows_chunked(O, L, lambda rows: oracle.ref_attn(qo, ko, vo, scale, rows=rows), Nq,
                         "long ragged block", chunk=500)


# ---------------------------------------------------------------------------
# Edge cases: ragged tiles, odd head dims, tiny and degenerate sizes
# ---------------------------------------------------------------------------

SHAPES = [
    # (B, H, Nq, Nkv, d)
    (1, 1, 1, 1, 64),
    (1, 2, 63, 257, 64),
    (2, 1, 257, 63, 72),
    (1, 1, 1000, 1000, 128),
    (1, 3, 129, 65, 128),
    (1, 1, 5, 300, 8),
    (1, 2, 200, 130, 40),
    (1, 1, 130, 100, 96),
    (1, 1, 64, 64, 120),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_dtype,out_dtype", [
    (torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32), (torch.float32, torch.float32)])
def test_edge_shapes(shape, in_dtype, out_dtype):
    B, H, Nq, Nkv, d = shape
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "bf16" if in_dtype == torch.bfloat16 else "f32",
                                 seed=100 + Nq + Nkv + d)
    check_attn(q, k, v, inputs.default_scale(d), out_dtype, f"edge {shape}")


ALL_HEAD_DIMS = list(range(8, 129, 8))


@pytest.mark.parametrize("d", ALL_HEAD_DIMS)
def test_every_head_dim(d):
    """Every instantiated head dim on a ragged shape (query and key counts not
    multiples of the tiles): bf16 in with bf16 and fp32 out, fp32 in; and two
    KV blocks folded by the fused merge into fp32 and bf16 accumulators."""
    scale = inputs.default_scale(d)
    for out_dtype in (torch.bfloat16, torch.float32):
        q, k, v = inputs.attn_inputs(1, 2, 300, 200, d, "bf16", seed=100 + d)
        check_attn(q, k, v, scale, out_dtype, f"head dim {d}")
    q, k, v = inputs.attn_inputs(1, 2, 130, 90, d, "f32", seed=300 + d)
    check_attn(q, k, v, scale, torch.float32, f"head dim {d} fp32")
    q, k, v = inputs.attn_inputs(1, 2, 300, 200, d, "bf16", seed=400 + d)
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    for acc_dtype in (torch.float32, torch.bfloat16):
        say("case fused merge head dim", d, acc_dtype)
        o_acc = torch.full((1, 2, 300, d), float("nan"), dtype=acc_dtype, device="cuda:0")
        l_acc = torch.full((1, 2, 300), -float("inf"), device="cuda:0")
        for a, b in ((0, 77), (77, 200)):
            attn_block_fwd_merge(dev(q), dev(k[:, :, a:b].contiguous()), dev(v[:, :, a:b].contiguous()),
                                 o_acc, l_acc, scale=scale)
        torch.cuda.synchronize()
        assert_bf16_close(to_f64(o_acc), Or, f"fused d{d} O")
        assert_bf16_close(to_f64(l_acc), Lr, f"fused d{d} LSE")


def test_large_scores_stay_finite():
    """Scores of several hundred (peaked softmax) must not overflow."""
    q, k, v = inputs.attn_inputs(1, 2, 100, 300, 64, "bf16", seed=7)
    q = (q.float() * 8).to(torch.bfloat16)
    k = (k.float() * 8).to(torch.bfloat16)
    check_attn(q, k, v, 0.125, torch.float32, "peaked scores")


def growing_scores_inputs(B, H, Nq, Nkv, d, seed):
    """Every 64-key tile's scores exceed the previous tile's by about 32
    (natural units): key row j is 4 * (j // 64) plus noise, the queries are
    near 1, the scale is 1/8 at d = 64.  Each new tile's weights would pass any
    bound against the running reference, so the rescale runs on every tile."""
    g = torch.Generator().manual_seed(seed)
    tile = (torch.arange(Nkv) // 64).float()
    k = (4.0 * tile)[None, None, :, None] + 0.3 * torch.randn(B, H, Nkv, d, generator=g)
    q = 1.0 + 0.05 * torch.randn(B, H, Nq, d, generator=g)
    v = torch.randn(B, H, Nkv, d, generator=g)
    return (q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16))


def test_rescale_on_every_tile():
    """The rare rescale path, taken on every key tile: plain launch, split
    launch (pieces start with their own reference) and the fused ring step
    over two blocks."""
    from attention_attn_block_amd import attn_block_workspace
    B, H, Nq, Nkv, d = 2, 50, 200, 640, 64
    q, k, v = growing_scores_inputs(B, H, Nq, Nkv, d, seed=77)
    scale = 0.125
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    gq, gk, gv = dev(q), dev(k), dev(v)
    say("case rescale every tile: plain")
    O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(O), Or, "rescale plain O")
    assert_bf16_close(to_f64(L), Lr, "rescale plain LSE")
    say("case rescale every tile: forced split")
    ws = attn_block_workspace(gq, gk)
    O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=torch.float32, workspace=ws,
                          force_split=True)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(O), Or, "rescale split O")
    assert_bf16_close(to_f64(L), Lr, "rescale split LSE")
    say("case rescale every tile: fused ring step over two blocks")
    o_acc = torch.zeros(B, H, Nq, d, dtype=torch.float32, device="cuda:0")
    l_acc = torch.full((B, H, Nq), float("-inf"), dtype=torch.float32, device="cuda:0")
    for lo, hi in ((0, 320), (320, Nkv)):
        attn_block_fwd_merge(gq, gk[:, :, lo:hi].contiguous(), gv[:, :, lo:hi].contiguous(), o_acc,
                             l_acc, scale=scale)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(o_acc), Or, "rescale fused O")
    assert_bf16_close(to_f64(l_acc), Lr, "rescale fused LSE")


@pytest.mark.parametrize("d", [72, 40])
@pytest.mark.parametrize("growth", [0.1, 1.0, 4.0])
def test_ones_row_head_dims_fast_path_and_fallback(d, growth):
    """Head dims that are not a multiple of 32 take the normaliser from the
    PV product's padding rows and bound no weight per tile; a row whose
    scores outgrow the first tile's maximum by 128 (log2 units) overflows
    there and the workgroup reruns with the per-tile bound.  Scores rise by
    about growth * d / 8 (natural units) per 64-key tile over 10 tiles:
    0.1 stays near the first tile's maximum; 1.0 still runs on the fast path
    with weights up to about 2^117 at d = 72, far above the exact path's
    per-tile bound; 4.0 overflows within a few tiles and falls back.  Plain
    launch, forced split and the fused merge over two blocks, against the
    oracle."""
    from attention_attn_block_amd import attn_block_workspace
    B, H, Nq, Nkv = 1, 40, 200, 640
    g = torch.Generator().manual_seed(int(100 * growth) + d)
    tile = (torch.arange(Nkv) // 64).float()
    k = (growth * tile)[None, None, :, None] + 0.3 * torch.randn(B, H, Nkv, d, generator=g)
    q = 1.0 + 0.05 * torch.randn(B, H, Nq, d, generator=g)
    v = torch.randn(B, H, Nkv, d, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    scale = 0.125
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    gq, gk, gv = dev(q), dev(k), dev(v)
    say("case ones-row head dim", d, "growth", growth)
    O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(O), Or, f"d{d} growth {growth} plain O")
    assert_bf16_close(to_f64(L), Lr, f"d{d} growth {growth} plain LSE")
    ws = attn_block_workspace(gq, gk)
    O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=torch.float32, workspace=ws,
                          force_split=True)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(O), Or, f"d{d} growth {growth} split O")
    assert_bf16_close(to_f64(L), Lr, f"d{d} growth {growth} split LSE")
    o_acc = torch.zeros(B, H, Nq, d, dtype=torch.float32, device="cuda:0")
    l_acc = torch.full((B, H, Nq), float("-inf"), dtype=torch.float32, device="cuda:0")
    for lo, hi in ((0, 320), (320, Nkv)):
        attn_block_fwd_merge(gq, gk[:, :, lo:hi].contiguous(), gv[:, :, lo:hi].contiguous(), o_acc,
                             l_acc, scale=scale)
    torch.cuda.synchronize()
    assert_bf16_close(to_f64(o_acc), Or, f"d{d} growth {growth} fused O")
    assert_bf16_close(to_f64(l_acc), Lr, f"d{d} growth {growth} fused LSE")


@pytest.mark.parametrize("Nkv", [30, 100, 1000])
def test_ragged_tile_ignores_stale_lds(Nkv):
    """Key rows past a ragged last tile must not carry over whatever an earlier
    kernel left in LDS.  A first call over all-NaN K/V fills every CU's tile
    buffers with NaN bit patterns; a ragged call right after on the same
    stream must still match the oracle (a stale NaN V row would turn the
    zero weight of a masked key into NaN)."""
    say("case stale-LDS ragged Nkv", Nkv)
    nan = torch.full((1, 32, 4096, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    q0 = torch.zeros(1, 32, 4096, 128, dtype=torch.bfloat16, device="cuda:0")
    q, k, v = inputs.attn_inputs(1, 4, 300, Nkv, 128, "bf16", seed=40 + Nkv)
    gq, gk, gv = dev(q), dev(k), dev(v)
    scale = inputs.default_scale(128)
    attn_block_fwd(q0, nan, nan, scale=scale)          # result discarded
    O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    assert_bf16_close(to_f64(O), Or, f"stale-LDS Nkv={Nkv} O")
    assert_bf16_close(to_f64(L), Lr, f"stale-LDS Nkv={Nkv} LSE")


def test_merge_edge_cases():
    rows, d = 300, 72
    g = torch.Generator().manual_seed(9)
    for dt in (torch.float32, torch.bfloat16):
        say("case merge edges", dt)
        Oa = torch.randn(rows, d, generator=g).to(dt)
        Ob = torch.randn(rows, d, generator=g).to(dt)
        La = torch.randn(rows, generator=g) * 3
        Lb = torch.randn(rows, generator=g) * 3
        La[::7] = -torch.inf          # empty a
        Lb[::5] = -torch.inf          # empty b
        Ob[::5] = torch.nan           # garbage in an empty partial must not leak
        ga, gla = dev(Oa), dev(La)
        attn_lse_merge(ga, gla, dev(Ob), dev(Lb))
        torch.cuda.synchronize()
        Or, Lr = oracle.ref_lse_merge(to_oracle(Oa), to_oracle(La), to_oracle(Ob), to_oracle(Lb))
        both_empty = np.isneginf(Lr)
        got_o, got_l = to_f64(ga), to_f64(gla)
        assert np.array_equal(np.isneginf(got_l), both_empty)
        assert np.all(got_o[both_empty] == 0.0), "two empty partials must give O = 0"
        fin = ~both_empty
        if dt == torch.float32:
            assert_f32_close(got_o[fin], Or[fin], "merge O")
            assert_f32_close(got_l[fin], Lr[fin], "merge LSE")
        else:
            assert_bf16_close(got_o[fin], Or[fin], "merge O bf16")
            assert_bf16_close(got_l[fin], Lr[fin], "merge LSE bf16")
        # rows where b is empty keep a bit for bit
        keep = np.isneginf(to_f64(Lb)) & ~np.isneginf(to_f64(La))
        assert np.array_equal(to_oracle(ga.cpu())[keep], to_oracle(Oa)[keep])


@pytest.mark.parametrize("d", list(range(8, 129, 8)))
def test_merge_and_patch_every_head_dim(d):
    """The merge (fp32 and bf16 partials, with empty rows) and the patch step
    (splice bit for bit, then attention) at every supported head dim."""
    rows = 300
    g = torch.Generator().manual_seed(500 + d)
    for dt in (torch.float32, torch.bfloat16):
        Oa = torch.randn(rows, d, generator=g).to(dt)
        Ob = torch.randn(rows, d, generator=g).to(dt)
        La = torch.randn(rows, generator=g) * 3
        Lb = torch.randn(rows, generator=g) * 3
        La[::7] = -torch.inf
        Lb[::5] = -torch.inf
        ga, gla = dev(Oa), dev(La)
        attn_lse_merge(ga, gla, dev(Ob), dev(Lb))
        torch.cuda.synchronize()
        Or, Lr = oracle.ref_lse_merge(to_oracle(Oa), to_oracle(La), to_oracle(Ob), to_oracle(Lb))
        fin = ~np.isneginf(Lr)
        assert np.array_equal(np.isneginf(to_f64(gla)), ~fin)
        close = assert_f32_close if dt == torch.float32 else assert_bf16_close
        close(to_f64(ga)[fin], Or[fin], f"merge d{d} O")
        close(to_f64(gla)[fin], Lr[fin], f"merge d{d} LSE")
    # patch: 70 fresh rows spliced at row 100 of a 260-row buffer
    q_p, k_p, v_p = inputs.attn_inputs(1, 2, 70, 70, d, "bf16", seed=600 + d)
    _, k_buf, v_buf = inputs.attn_inputs(1, 2, 1, 260, d, "bf16", seed=700 + d)
    scale = inputs.default_scale(d)
    kb, vb = dev(k_buf), dev(v_buf)
    say("case patch head dim", d)
    O, L = attn_patch_fwd(dev(q_p), dev(k_p), dev(v_p), kb, vb, 100, scale=scale)
    torch.cuda.synchronize()
    Or, Lr, Kn, Vn = oracle.ref_patch(to_oracle(q_p), to_oracle(k_p), to_oracle(v_p),
                                      to_oracle(k_buf), to_oracle(v_buf), 100, scale)
    assert np.array_equal(to_oracle(kb.cpu()), Kn) and np.array_equal(to_oracle(vb.cpu()), Vn)
    assert_bf16_close(to_f64(O), Or, f"patch d{d} O")
    assert_bf16_close(to_f64(L), Lr, f"patch d{d} LSE")


def test_merge_in_place_alias():
    """b == a exactly: O unchanged (to rounding), LSE + ln 2."""
    g = torch.Generator().manual_seed(10)
    Oa = torch.randn(500, 128, generator=g)
    La = torch.randn(500, generator=g)
    ga, gla = dev(Oa), dev(La)
    say("case merge alias")
    attn_lse_merge(ga, gla, ga, gla)
    torch.cuda.synchronize()
    Or, Lr = oracle.ref_lse_merge(to_oracle(Oa), to_oracle(La), to_oracle(Oa), to_oracle(La))
    assert_f32_close(to_f64(ga), Or, "alias O")
    assert_f32_close(to_f64(gla), Lr, "alias LSE")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1000, 8192, (1 << 20) + 3])
def test_cfg_sizes(n):
    g = torch.Generator().manual_seed(n)
    u, c = torch.randn(n, generator=g), torch.randn(n, generator=g)
    say("case cfg n =", n)
    out = cfg_combine(dev(u), dev(c), 4.0)
    gu = dev(u)
    cfg_combine(gu, dev(c), 1.0, out=gu)          # in place into eps_u, s = 1 gives eps_c
    torch.cuda.synchronize()
    assert_f32_close(to_f64(out), oracle.ref_cfg(to_oracle(u), to_oracle(c), 4.0), "cfg")
    assert torch.equal(gu.cpu(), c), "s = 1 must return eps_c exactly"


@pytest.mark.parametrize("p", [0, 1, 2, 3])
def test_patch_each_position_small(p):
    """4 patches of a shrunk video buffer (same recipe), every position, ragged patch."""
    N, Np, H = 4 * 300, 300, 3
    w = inputs.video_patch(p0=p * Np, N=N, Np=Np, H=H)
    say("case patch position", p)
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    O, L = attn_patch_fwd(dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"]), kb, vb, w["p0"],
                          scale=w["scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    Or, Lr, Kn, Vn = oracle.ref_patch(to_oracle(w["q_p"]), to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                      to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), w["p0"],
                                      w["scale"])
    assert np.array_equal(to_oracle(kb.cpu()), Kn) and np.array_equal(to_oracle(vb.cpu()), Vn)
    assert_bf16_close(to_f64(O), Or, "patch O")
    assert_bf16_close(to_f64(L), Lr, "patch LSE")


@pytest.mark.parametrize("Np,p0,N", [(1, 0, 50), (1, 49, 50), (50, 0, 50), (17, 33, 50)])
def test_patch_degenerate(Np, p0, N):
    w = inputs.video_patch(p0=p0, N=N, Np=Np, H=2)
    say("case patch degenerate", Np, p0, N)
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    O, L = attn_patch_fwd(dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"]), kb, vb, p0, scale=w["scale"])
    torch.cuda.synchronize()
    Or, Lr, Kn, _ = oracle.ref_patch(to_oracle(w["q_p"]), to_oracle(w["k_p"]), to_oracle(w["v_p"]),
                                     to_oracle(w["k_buf"]), to_oracle(w["v_buf"]), p0, w["scale"])
    assert np.array_equal(to_oracle(kb.cpu()), Kn)
    assert_bf16_close(to_f64(O), Or, "patch O")
    assert_bf16_close(to_f64(L), Lr, "patch LSE")


def test_deterministic_and_stream_ordered():
    """Two runs give identical bits (no LDS races); a side stream orders correctly."""
    q, k, v = inputs.attn_inputs(2, 4, 700, 900, 128, "bf16", seed=3)
    q, k, v = dev(q), dev(k), dev(v)
    say("case determinism")
    O1, L1 = attn_block_fwd(q, k, v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        O2, L2 = attn_block_fwd(q, k, v)
        O2 = O2.clone()
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


# ---------------------------------------------------------------------------
# Fused ring step and the CFG discrepancy signal
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("acc_dtype", [torch.float32, torch.bfloat16])
def test_ring_2048px_fused_merge(acc_dtype):
    """attn_block_fwd_merge over the 8 KV blocks, starting from an empty
    accumulator (LSE = -inf, O full of NaN that must never be read), equals
    attention over all 16384 keys."""
    w = inputs.ring_2048px()
    q = dev(w["q"])
    B, H, Nq, d = q.shape
    o_acc = torch.full((B, H, Nq, d), float("nan"), dtype=acc_dtype, device="cuda:0")
    l_acc = torch.full((B, H, Nq), -float("inf"), device="cuda:0")
    say("case ring fused", acc_dtype)
    for kj, vj in zip(w["ks"], w["vs"]):
        attn_block_fwd_merge(q, dev(kj), dev(vj), o_acc, l_acc, scale=w["scale"])
    torch.cuda.synchronize()
    K = torch.cat(w["ks"], dim=2)
    V = torch.cat(w["vs"], dim=2)
    Or, Lr = oracle.ref_attn(to_oracle(w["q"]), to_oracle(K), to_oracle(V), w["scale"])
    assert_bf16_close(to_f64(o_acc), Or, "ring fused O")
    assert_bf16_close(to_f64(l_acc), Lr, "ring fused LSE")


@pytest.mark.parametrize("shape", [(1, 2, 70, 45, 72), (2, 1, 130, 257, 128), (1, 1, 1, 3, 8)])
def test_fused_merge_uneven_blocks(shape):
    """Three KV blocks of unequal length, fused, against the oracle's fold of
    the same blocks and its full attention; the fp32 path too."""
    B, H, Nq, Nkv, d = shape
    for dt in ("bf16", "f32"):
        q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, dt, seed=Nq + Nkv)
        cuts = [0, Nkv // 3, (2 * Nkv) // 3 + 1, Nkv]
        cuts = sorted(set(min(max(c, 0), Nkv) for c in cuts))
        acc_t = torch.float32
        o_acc = torch.zeros((B, H, Nq, d), dtype=acc_t, device="cuda:0")
        l_acc = torch.full((B, H, Nq), -float("inf"), device="cuda:0")
        say("case fused uneven", shape, dt, cuts)
        for a, b in zip(cuts[:-1], cuts[1:]):
            attn_block_fwd_merge(dev(q), dev(k[:, :, a:b].contiguous()), dev(v[:, :, a:b].contiguous()),
                                 o_acc, l_acc, scale=inputs.default_scale(d))
        torch.cuda.synchronize()
        Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), inputs.default_scale(d))
        assert_close(to_f64(o_acc), Or, dt == "f32", "fused O")
        assert_close(to_f64(l_acc), Lr, dt == "f32", "fused LSE")


@pytest.mark.parametrize("n", [1, 5, 4096, 8192, 4096 * 3 + 7, (1 << 22) + 1])
def test_cfg_relmae(n):
    g = torch.Generator().manual_seed(1000 + n)
    u = torch.randn(n, generator=g)
    c = u + 0.3 * torch.randn(n, generator=g)
    say("case cfg relmae n =", n)
    out, rm = cfg_combine_relmae(dev(u), dev(c), 4.0)
    torch.cuda.synchronize()
    assert_f32_close(to_f64(out), oracle.ref_cfg(to_oracle(u), to_oracle(c), 4.0), "relmae cfg out")
    want = oracle.ref_cfg_relmae(to_oracle(u), to_oracle(c))
    got = float(rm.item())
    assert abs(got - want) <= 1e-5 * abs(want), (got, want)
    # deterministic: a second call gives the same bits
    out2, rm2 = cfg_combine_relmae(dev(u), dev(c), 4.0)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(rm, rm2)


def test_cfg_relmae_dit_xl_256_and_identity():
    w = inputs.dit_xl_256()
    say("case relmae dit_xl_256")
    out, rm = cfg_combine_relmae(dev(w["eps_u"]), dev(w["eps_c"]), w["s"])
    same, rz = cfg_combine_relmae(dev(w["eps_u"]), dev(w["eps_u"]), w["s"])
    zeros, r00 = cfg_combine_relmae(torch.zeros(64, device="cuda:0"), torch.zeros(64, device="cuda:0"), 2.0)
    torch.cuda.synchronize()
    want = oracle.ref_cfg_relmae(to_oracle(w["eps_u"]), to_oracle(w["eps_c"]))
    assert abs(float(rm.item()) - want) <= 1e-5 * want
    assert float(rz.item()) == 0.0 and float(r00.item()) == 0.0
    assert_f32_close(to_f64(out), oracle.ref_cfg(to_oracle(w["eps_u"]), to_oracle(w["eps_c"]), w["s"]), "cfg")


def test_graph_replays_match_eager():
    """The ring fold (fused and unfused), the patch step and the CFG combine
    captured in one HIP graph and replayed several times, with eager work and
    synchronisations between replays, give the eager result every time (the
    library launches kernels only: no memsets, no allocations)."""
    q, k, v = inputs.attn_inputs(1, 4, 300, 3 * 200, 128, "bf16", seed=21)
    q, k, v = dev(q), dev(k), dev(v)
    blocks = [(k[:, :, i * 200:(i + 1) * 200].contiguous(), v[:, :, i * 200:(i + 1) * 200].contiguous())
              for i in range(3)]
    w = inputs.video_patch(N=600, Np=200, p0=200, H=4)
    qp, kp, vp = dev(w["q_p"]), dev(w["k_p"]), dev(w["v_p"])
    kb, vb = dev(w["k_buf"]), dev(w["v_buf"])
    u, c = dev(torch.randn(5000)), dev(torch.randn(5000))
    o_acc = torch.empty(1, 4, 300, 128, device="cuda:0")
    l_acc = torch.empty(1, 4, 300, device="cuda:0")
    o_f = torch.empty_like(o_acc)
    l_f = torch.empty_like(l_acc)
    o_t = torch.empty_like(o_acc)
    l_t = torch.empty_like(l_acc)
    o_p = torch.empty(1, 4, 200, 128, dtype=torch.bfloat16, device="cuda:0")
    l_p = torch.empty(1, 4, 200, device="cuda:0")
    cfg_out = torch.empty_like(u)

    def step():
        attn_block_fwd(q, *blocks[0], out=o_acc, lse=l_acc, out_dtype=torch.float32)
        for kb_, vb_ in blocks[1:]:
            attn_block_fwd(q, kb_, vb_, out=o_t, lse=l_t, out_dtype=torch.float32)
            attn_lse_merge(o_acc, l_acc, o_t, l_t)
        l_f.fill_(-float("inf"))
        for kb_, vb_ in blocks:
            attn_block_fwd_merge(q, kb_, vb_, o_f, l_f)
        attn_patch_fwd(qp, kp, vp, kb, vb, w["p0"], out=o_p, lse=l_p)
        cfg_combine(u, c, 4.0, out=cfg_out)

    say("case graph capture")
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o_acc, l_acc, o_f, l_f, o_p, l_p, cfg_out)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (o_acc, l_acc, o_f, l_f, o_p, l_p, cfg_out):
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o_acc, l_acc, o_f, l_f, o_p, l_p, cfg_out)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
