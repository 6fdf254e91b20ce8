"""Write ``oracle_small.json``: oracle outputs on small fixed inputs.

Regression fixture only: it freezes what the fp64 oracle returns today so that
any later change to its arithmetic shows up in the CPU suite.  The inputs are
closed-form integer patterns (no RNG), and every stored value is computed by
``oracle`` alone.  Run from the repository root:

    python -m tests.golden.make_golden
"""

import json
import math
import os

import numpy as np

import oracle


def _pattern(shape, a, b, c):
    idx = np.indices(shape)
    v = (a * idx[-2] + b * idx[-1] + c * idx[1]) % 7 - 3
    return v.astype(np.float64) / 2.0


def compute_cases():
    out = {}
    Q = _pattern((1, 2, 5, 8), 3, 1, 2)
    K = _pattern((1, 2, 9, 8), 2, 5, 1)
    V = _pattern((1, 2, 9, 8), 4, 3, 3)
    O, L = oracle.ref_attn(Q, K, V, 1.0 / math.sqrt(8))
    out["attn_b1h2_q5_k9_d8"] = {"O": O.tolist(), "LSE": L.tolist()}
    parts = [oracle.ref_attn(Q, K[:, :, a:b], V[:, :, a:b], 1.0 / math.sqrt(8))
             for a, b in ((0, 2), (2, 6), (6, 9))]
    Of, Lf = oracle.ref_block_fold(parts)
    out["fold_3_blocks"] = {"O": Of.tolist(), "LSE": Lf.tolist()}
    Op, Lp, Kn, _ = oracle.ref_patch(Q[:, :, :3], K[:, :, :3], V[:, :, :3], K * 0.5, V * 0.5, 4,
                                     1.0 / math.sqrt(8))
    out["patch_np3_p04"] = {"O": Op.tolist(), "LSE": Lp.tolist(), "K_new": Kn.tolist()}
    Ks = _pattern((1, 2, 9, 8), 1, 1, 2)
    Op, Lp, Kn, _ = oracle.ref_patch_strided(Q[:, :, :4], K[:, :, :4], V[:, :, :4], Ks, Ks * 0.25,
                                             1, 2, 5, 1.0 / math.sqrt(8))
    out["patch_strided_2x2_p01_s5"] = {"O": Op.tolist(), "LSE": Lp.tolist(), "K_new": Kn.tolist()}
    u = _pattern((1, 2, 3, 4), 1, 2, 3)
    c = _pattern((1, 2, 3, 4), 3, 1, 1)
    out["cfg_s4"] = {"out": oracle.ref_cfg(u, c, 4.0).tolist(),
                     "relmae": [oracle.ref_cfg_relmae(u, c)]}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(compute_cases(), f, indent=1)
    print("wrote", path)
