"""GPU parity over seeded random combinations of the attention calls' options.

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

A few cases take the fp32 path.  Sizes keep each oracle call well under a
second.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_attn_block_amd import (attn_block_fwd, attn_block_fwd_merge, attn_block_workspace,
                                      attn_ring_fwd, inputs)
from tests.gpu_util import assert_close, to_f64, to_oracle

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
