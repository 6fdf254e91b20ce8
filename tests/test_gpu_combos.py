"""GPU parity over seeded random combinations of the calls' options.

The other GPU tests take each option on its own.  Here every case draws a
shape (B, H, ragged Nq and Nkv, head dim), an output dtype, a launch form and
a score scale from one seeded generator, and compares every output element
with the fp64 oracle:

* plain grid; split launch through a workspace (forced);
* the fused merge: the key range cut in two and folded into a running
  partial that starts empty (LSE = -inf);
* a block set in one launch (attn_ring_fwd), 1-4 equal blocks, plain or split;
* Q scaled by 1 (N(0, 1) scores) or by 6 (peaked rows whose later tiles
  outgrow the first tile's reference max).

A few cases take the fp32 path.  The same is done for the patch step
(contiguous or strided runs, plain or with a workspace; spliced buffers bit
for bit), the LSE merge (random rows, d, dtype and empty rows on either side)
and the CFG combine (odd sizes, any s; the rel-MAE signal too).  Sizes keep
each oracle call well under a second.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_fwd, attn_block_fwd_merge, attn_block_workspace,
                                      attn_lse_merge, attn_patch_fwd, attn_patch_fwd_strided,
                                      attn_ring_fwd, cfg_combine, cfg_combine_relmae, inputs)
from tests.gpu_util import assert_close, assert_f32_close, to_f64, to_oracle

pytestmark = pytest.mark.gpu

N_CASES = 40
FORMS = ("plain", "split", "merge", "ring", "ring_split")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no fallback)"
    torch.cuda.init()
    return torch.device("cuda:0")


def draw(i):
    """Configuration of case i (depends on i only)."""
    r = np.random.RandomState(7000 + i)
    fp32 = i % 10 == 9
    form = "plain" if fp32 else FORMS[r.randint(len(FORMS))]
    n_blocks = int(r.randint(1, 5)) if form.startswith("ring") else 1
    B, H = int(r.randint(1, 3)), int(r.randint(1, 4))
    Nq = int(r.randint(1, 700))
    Nkv_block = int(r.randint(1, 1500 // n_blocks + 1))
    d = 8 * int(r.randint(1, 17))
    out = torch.float32 if fp32 or r.randint(2) else torch.bfloat16
    peak = 6.0 if r.randint(3) == 0 else 1.0
    return dict(fp32=fp32, form=form, n_blocks=n_blocks, B=B, H=H, Nq=Nq, Nkv_block=Nkv_block,
                d=d, out=out, peak=peak, seed=9000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_combination(i):
    c = draw(i)
    print("case", i, c, flush=True)
    B, H, Nq, d = c["B"], c["H"], c["Nq"], c["d"]
    Nkv = c["n_blocks"] * c["Nkv_block"]
    q, k, v = inputs.attn_inputs(B, H, Nq, Nkv, d, "f32" if c["fp32"] else "bf16", c["seed"])
    if c["peak"] != 1.0:
        q = (q.float() * c["peak"]).to(q.dtype)
    scale = inputs.default_scale(d)
    gq, gk, gv = (t.to("cuda:0") for t in (q, k, v))
    form = c["form"]
    if form in ("plain", "split"):
        kw = {"workspace": attn_block_workspace(gq, gk), "force_split": True} if form == "split" else {}
        O, L = attn_block_fwd(gq, gk, gv, scale=scale, out_dtype=c["out"], **kw)
    elif form == "merge":
        O = torch.full((B, H, Nq, d), float("nan"), dtype=c["out"], device="cuda:0")
        L = torch.full((B, H, Nq), -float("inf"), dtype=torch.float32, device="cuda:0")
        cut = Nkv // 2
        for lo, hi in ((0, cut), (cut, Nkv)):
            if hi > lo:
                attn_block_fwd_merge(gq, gk[:, :, lo:hi].contiguous(), gv[:, :, lo:hi].contiguous(),
                                     O, L, scale=scale)
    else:
        nb = c["Nkv_block"]
        ks = [gk[:, :, j * nb:(j + 1) * nb].contiguous() for j in range(c["n_blocks"])]
        vs = [gv[:, :, j * nb:(j + 1) * nb].contiguous() for j in range(c["n_blocks"])]
        kw = ({"workspace": attn_block_workspace(gq, ks[0]), "force_split": True}
              if form == "ring_split" else {})
        O, L = attn_ring_fwd(gq, ks, vs, scale=scale, out_dtype=c["out"], **kw)
    torch.cuda.synchronize()
    Or, Lr = oracle.ref_attn(to_oracle(q), to_oracle(k), to_oracle(v), scale)
    what = f"case {i} ({form}, d={d}, Nq={Nq}, Nkv={Nkv})"
    assert_close(to_f64(O), Or, c["fp32"], what + " O")
    assert_close(to_f64(L), Lr, c["fp32"], what + " LSE")


# ---------------------------------------------------------------------------
# Patch step
# ---------------------------------------------------------------------------

N_PATCH = 16


def draw_patch(i):
    r = np.random.RandomState(7100 + i)
    B, H = int(r.randint(1, 3)), int(r.randint(1, 4))
    d = 8 * int(r.randint(1, 17))
    if r.randint(2):  # strided: n_runs runs of run_len rows, run_stride apart (no overlap)
        n_runs, run_len = int(r.randint(1, 7)), int(r.randint(1, 81))
        run_stride = run_len + int(r.randint(0, 61))
        p0 = int(r.randint(0, 51))
        N = p0 + (n_runs - 1) * run_stride + run_len + int(r.randint(0, 101))
    else:
        N = int(r.randint(1, 1501))
        run_len = int(r.randint(1, N + 1))
        n_runs, run_stride = 1, None
        p0 = int(r.randint(0, N - run_len + 1))
    out = torch.float32 if r.randint(2) else torch.bfloat16
    return dict(B=B, H=H, d=d, N=N, p0=p0, run_len=run_len, run_stride=run_stride, n_runs=n_runs,
                out=out, ws=bool(r.randint(2)), seed=9100 + i)


@pytest.mark.parametrize("i", range(N_PATCH))
def test_random_patch(i):
    c = draw_patch(i)
    print("case patch", i, c, flush=True)
    B, H, d, N = c["B"], c["H"], c["d"], c["N"]
    Np = c["n_runs"] * c["run_len"]
    q_p, k_p, v_p = inputs.attn_inputs(B, H, Np, Np, d, "bf16", seed=c["seed"])
    _, k_buf, v_buf = inputs.attn_inputs(B, H, 1, N, d, "bf16", seed=c["seed"] + 1)
    scale = inputs.default_scale(d)
    gq, gk, gv = (t.to("cuda:0") for t in (q_p, k_p, v_p))
    kb, vb = k_buf.to("cuda:0"), v_buf.to("cuda:0")
    kw = {"workspace": attn_block_workspace(gq, kb)} if c["ws"] else {}
    if c["run_stride"] is None:
        O, L = attn_patch_fwd(gq, gk, gv, kb, vb, c["p0"], scale=scale, out_dtype=c["out"], **kw)
        Or, Lr, Kn, Vn = oracle.ref_patch(to_oracle(q_p), to_oracle(k_p), to_oracle(v_p),
                                          to_oracle(k_buf), to_oracle(v_buf), c["p0"], scale)
    else:
        O, L = attn_patch_fwd_strided(gq, gk, gv, kb, vb, c["p0"], c["run_len"], c["run_stride"],
                                      scale=scale, out_dtype=c["out"], **kw)
        Or, Lr, Kn, Vn = oracle.ref_patch_strided(
            to_oracle(q_p), to_oracle(k_p), to_oracle(v_p), to_oracle(k_buf), to_oracle(v_buf),
            c["p0"], c["run_len"], c["run_stride"], scale)
    torch.cuda.synchronize()
    what = f"patch case {i}"
    assert np.array_equal(to_oracle(kb.cpu()), Kn), what + ": spliced K buffer differs"
    assert np.array_equal(to_oracle(vb.cpu()), Vn), what + ": spliced V buffer differs"
    assert_close(to_f64(O), Or, False, what + " O")
    assert_close(to_f64(L), Lr, False, what + " LSE")


# ---------------------------------------------------------------------------
# LSE merge
# ---------------------------------------------------------------------------

N_MERGE = 12


@pytest.mark.parametrize("i", range(N_MERGE))
def test_random_merge(i):
    r = np.random.RandomState(7200 + i)
    rows, d = int(r.randint(1, 60001)), 8 * int(r.randint(1, 17))
    dt = torch.float32 if r.randint(2) else torch.bfloat16
    p_empty = float(r.choice([0.0, 0.05, 0.5]))
    print("case merge", i, rows, d, dt, p_empty, flush=True)
    g = torch.Generator().manual_seed(9200 + i)
    Oa, Ob = (torch.randn(rows, d, generator=g).to(dt) for _ in range(2))
    La = torch.randn(rows, generator=g) * 3
    Lb = torch.randn(rows, generator=g) * 3
    ea = torch.rand(rows, generator=g) < p_empty
    eb = torch.rand(rows, generator=g) < p_empty
    La[ea] = -float("inf")
    Lb[eb] = -float("inf")
    Oa[ea] = 0  # an empty accumulator holds zeros (two empty partials give 0)
    Or, Lr = oracle.ref_lse_merge(to_oracle(Oa), to_oracle(La), to_oracle(Ob), to_oracle(Lb))
    ga, gla = Oa.to("cuda:0"), La.to("cuda:0")
    attn_lse_merge(ga, gla, Ob.to("cuda:0"), Lb.to("cuda:0"))
    torch.cuda.synchronize()
    got_l = to_f64(gla)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(Lr)), "empty rows differ"
    fin = np.isfinite(Lr)
    assert_close(to_f64(ga), Or, dt == torch.float32, f"merge case {i} O")
    if fin.any():
        assert_close(got_l[fin], Lr[fin], dt == torch.float32, f"merge case {i} LSE")


# ---------------------------------------------------------------------------
# CFG combine
# ---------------------------------------------------------------------------

N_CFG = 8


@pytest.mark.parametrize("i", range(N_CFG))
def test_random_cfg(i):
    r = np.random.RandomState(7300 + i)
    n = int(r.choice([1, 3, 17, 1000, 65537, 1 << 20])) + int(r.randint(0, 5))
    s = float(r.uniform(-2.0, 10.0))
    print("case cfg", i, n, s, flush=True)
    g = torch.Generator().manual_seed(9300 + i)
    u = torch.randn(n, generator=g)
    c = u + 0.5 * torch.randn(n, generator=g)
    out = cfg_combine(u.to("cuda:0"), c.to("cuda:0"), s)
    out2, rm = cfg_combine_relmae(u.to("cuda:0"), c.to("cuda:0"), s)
    torch.cuda.synchronize()
    want = oracle.ref_cfg(to_oracle(u), to_oracle(c), s)
    assert_f32_close(to_f64(out), want, f"cfg case {i}")
    assert torch.equal(out, out2), "cfg_combine and cfg_combine_relmae outputs differ"
    wr = oracle.ref_cfg_relmae(to_oracle(u), to_oracle(c))
    assert abs(float(rm.item()) - wr) <= 1e-5 * abs(wr), (float(rm.item()), wr)
