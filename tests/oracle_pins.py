"""Pins that tie the fp64 oracle to mathematics other than itself.

Each ``pin_*`` takes an oracle namespace ``o`` (the real ``oracle`` package,
or a deliberately broken copy in the mutation test) and raises AssertionError
when ``o`` is wrong.  The pins are closed forms, invariants, special cases that
reduce to library routines (torch's fp64 scaled-dot-product attention, scipy's
logsumexp) and brute force on tiny inputs.  The pages print no worked example,
so none of the expected values below comes from them.
"""

import math

import numpy as np
import scipy.special
import torch

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def pin_attn_zero_query(o):
    """Q = 0: every score is 0, so O is the per-head mean of V and LSE = ln Nkv."""
    r = _rng(1)
    B, H, Nq, Nkv, d = 2, 3, 5, 7, 4
    Q = np.zeros((B, H, Nq, d))
    K = r.standard_normal((B, H, Nkv, d))
    V = r.standard_normal((B, H, Nkv, d))
    O, L = o.ref_attn(Q, K, V, 0.37)
    _close(O, np.broadcast_to(V.mean(axis=2, keepdims=True), O.shape), 1e-14, "Q=0 mean")
    _close(L, np.full((B, H, Nq), math.log(Nkv)), 1e-14, "Q=0 lse")


def pin_attn_value_ones(o):
    """V = 1: softmax rows sum to one, so O = 1 exactly up to rounding."""
    r = _rng(2)
    Q = r.standard_normal((1, 2, 6, 5)) * 3
    K = r.standard_normal((1, 2, 9, 5)) * 3
    V = np.ones((1, 2, 9, 5))
    O, _ = o.ref_attn(Q, K, V, 0.5)
    _close(O, np.ones_like(O), 1e-13, "V=1")


def pin_attn_one_hot(o):
    """Q = K = A*I with A^2*scale = 64: row i scores 64 at key i and 0 elsewhere,
    so O_i = V_i to within (n-1)e^-64 and LSE = 64 + ln(1 + (n-1)e^-64)."""
    n = 16
    scale = 1.0 / 8.0
    A = math.sqrt(64.0 / scale)
    Q = (A * np.eye(n))[None, None]
    K = Q.copy()
    V = _rng(3).standard_normal((1, 1, n, n))
    O, L = o.ref_attn(Q, K, V, scale)
    _close(O, V, 1e-20 + 1e-12 * np.abs(V).max(), "one-hot O")
    _close(L, np.full((1, 1, n), 64.0 + math.log1p((n - 1) * math.exp(-64.0))), 1e-13, "one-hot lse")


def pin_attn_worked_example(o):
    """Hand-worked case: d = 1, scale = 2, q = 1/2 gives scores ln1, ln2, ln3,
    weights 1/6, 2/6, 3/6; with v = (6, 0, -6) the output is 1 - 3 = -2 and the
    log-sum-exp is ln 6.  A second query q = 0 gives the plain mean 0, ln 3."""
    Q = np.array([0.5, 0.0]).reshape(1, 1, 2, 1)
    K = np.array([0.0, math.log(2.0), math.log(3.0)]).reshape(1, 1, 3, 1)
    V = np.array([6.0, 0.0, -6.0]).reshape(1, 1, 3, 1)
    O, L = o.ref_attn(Q, K, V, 2.0)
    _close(O.ravel(), [-2.0, 0.0], 1e-14, "worked O")
    _close(L.ravel(), [math.log(6.0), math.log(3.0)], 1e-14, "worked lse")


def pin_attn_two_keys(o):
    """Two keys: the weights are the logistic function of the score gap."""
    r = _rng(4)
    d = 3
    q = r.standard_normal(d)
    k = r.standard_normal((2, d))
    v = r.standard_normal((2, 4))
    scale = 0.7
    gap = scale * (q @ (k[0] - k[1]))
    w0 = 1.0 / (1.0 + math.exp(-gap))
    # V has its own width: pad d of q/k up to 4 with zeros so shapes match.
    Q = np.zeros((1, 1, 1, 4)); Q[0, 0, 0, :d] = q
    K = np.zeros((1, 1, 2, 4)); K[0, 0, :, :d] = k
    V = v[None, None]
    O, L = o.ref_attn(Q, K, V, scale)
    _close(O[0, 0, 0], w0 * v[0] + (1 - w0) * v[1], 1e-14, "two-key O")
    s0, s1 = scale * (q @ k[0]), scale * (q @ k[1])
    _close(L.ravel(), [max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))], 1e-14, "two-key lse")


def pin_attn_library(o):
    """Tiny random shapes against torch's fp64 scaled-dot-product attention
    (CPU math path) for O and scipy's logsumexp for the LSE."""
    r = _rng(5)
    for (B, H, Nq, Nkv, d) in [(1, 1, 1, 1, 1), (2, 3, 4, 7, 8), (1, 2, 8, 3, 5), (1, 1, 6, 8, 8)]:
        Q = r.standard_normal((B, H, Nq, d)) * 2
        K = r.standard_normal((B, H, Nkv, d)) * 2
        V = r.standard_normal((B, H, Nkv, d))
        scale = 1.0 / math.sqrt(d) * 1.3
        O, L = o.ref_attn(Q, K, V, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (Q, K, V))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
        _close(O, ref, 1e-13, f"sdpa {B,H,Nq,Nkv,d}")
        S = np.einsum("bhid,bhjd->bhij", Q, K) * scale
        _close(L, scipy.special.logsumexp(S, axis=-1), 1e-13, f"logsumexp {B,H,Nq,Nkv,d}")


def pin_attn_permutation(o):
    """Permuting KV rows jointly changes nothing; permuting Q rows permutes the
    outputs; permuting K alone does change the result."""
    r = _rng(6)
    Q = r.standard_normal((1, 2, 5, 4))
    K = r.standard_normal((1, 2, 9, 4))
    V = r.standard_normal((1, 2, 9, 4))
    O, L = o.ref_attn(Q, K, V, 0.8)
    pk = r.permutation(9)
    O2, L2 = o.ref_attn(Q, K[:, :, pk], V[:, :, pk], 0.8)
    _close(O2, O, 1e-14, "kv perm O")
    _close(L2, L, 1e-14, "kv perm lse")
    pq = r.permutation(5)
    O3, L3 = o.ref_attn(Q[:, :, pq], K, V, 0.8)
    _close(O3, O[:, :, pq], 1e-14, "q perm O")
    _close(L3, L[:, :, pq], 1e-14, "q perm lse")
    O4, _ = o.ref_attn(Q, K[:, :, pk], V, 0.8)
    assert np.max(np.abs(O4 - O)) > 1e-3, "K-only permutation left O unchanged"


def pin_attn_rows(o):
    """Sampled rows equal the same rows of the full computation."""
    r = _rng(7)
    Q = r.standard_normal((2, 2, 11, 4))
    K = r.standard_normal((2, 2, 6, 4))
    V = r.standard_normal((2, 2, 6, 4))
    O, L = o.ref_attn(Q, K, V, 0.5)
    rows = np.array([10, 0, 3])
    Os, Ls = o.ref_attn(Q, K, V, 0.5, rows=rows)
    _close(Os, O[:, :, rows], 0.0, "rows O")
    _close(Ls, L[:, :, rows], 0.0, "rows lse")


def pin_attn_bf16_input(o):
    """bfloat16 bit inputs decode to the same values torch gives for them."""
    r = _rng(8)
    q = torch.from_numpy(r.standard_normal((1, 1, 4, 8)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(r.standard_normal((1, 1, 5, 8)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(r.standard_normal((1, 1, 5, 8)).astype(np.float32)).to(torch.bfloat16)
    bits = [x.view(torch.int16).numpy().view(np.uint16) for x in (q, k, v)]
    O1, L1 = o.ref_attn(*bits, 0.25)
    O2, L2 = o.ref_attn(*(x.double().numpy() for x in (q, k, v)), 0.25)
    _close(O1, O2, 0.0, "bf16 bits O")
    _close(L1, L2, 0.0, "bf16 bits lse")


def pin_decode(o):
    """bfloat16 decode: fixed bit patterns and agreement with torch's widening."""
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F81, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 1.0 + 2.0 ** -7, 2.0 ** -133]
    got = o.decode(bits)
    assert got.dtype == np.float64
    assert list(got) == want, f"decode {got} != {want}"
    assert math.copysign(1.0, got[3]) < 0
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((allbits & 0x7F80) != 0x7F80)
    t = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(o.decode(allbits)[finite], t[finite])


def pin_scale_equivariance(o):
    """Scaling Q by c and the scale by 1/c leaves every score unchanged."""
    r = _rng(9)
    Q = r.standard_normal((1, 3, 4, 6))
    K = r.standard_normal((1, 3, 5, 6))
    V = r.standard_normal((1, 3, 5, 6))
    O1, L1 = o.ref_attn(Q, K, V, 0.4)
    O2, L2 = o.ref_attn(Q * 4.0, K, V, 0.1)
    _close(O1, O2, 1e-14, "scale O")
    _close(L1, L2, 1e-13, "scale lse")


# --------------------------------------------------------------------------
# log-sum-exp merge
# --------------------------------------------------------------------------

def _split_fold(o, Q, K, V, scale, cuts):
    parts = []
    edges = [0] + list(cuts) + [K.shape[2]]
    for a, b in zip(edges[:-1], edges[1:]):
        parts.append(o.ref_attn(Q, K[:, :, a:b], V[:, :, a:b], scale))
    return parts


def pin_merge_fold_equals_full(o):
    """Splitting the keys into k blocks at random cut points and folding the
    block partials with the merge reproduces attention over all keys."""
    r = _rng(10)
    Q = r.standard_normal((2, 2, 5, 8)) * 2
    K = r.standard_normal((2, 2, 40, 8)) * 2
    V = r.standard_normal((2, 2, 40, 8))
    Of, Lf = o.ref_attn(Q, K, V, 0.6)
    for k in (2, 3, 4, 8):
        cuts = np.sort(r.choice(np.arange(1, 40), size=k - 1, replace=False))
        parts = _split_fold(o, Q, K, V, 0.6, cuts)
        O, L = o.ref_block_fold(parts)
        _close(O, Of, 1e-12, f"fold k={k} O")
        _close(L, Lf, 1e-12, f"fold k={k} lse")


def pin_merge_order_free(o):
    """The merge is commutative, and folding the blocks in any order agrees."""
    r = _rng(11)
    Q = r.standard_normal((1, 2, 4, 6))
    K = r.standard_normal((1, 2, 24, 6))
    V = r.standard_normal((1, 2, 24, 6))
    parts = _split_fold(o, Q, K, V, 0.5, [5, 11, 20])
    Oab, Lab = o.ref_lse_merge(*parts[0], *parts[1])
    Oba, Lba = o.ref_lse_merge(*parts[1], *parts[0])
    _close(Oab, Oba, 1e-15, "commute O")
    _close(Lab, Lba, 1e-15, "commute lse")
    O1, L1 = o.ref_block_fold(parts)
    O2, L2 = o.ref_block_fold([parts[i] for i in (3, 1, 0, 2)])
    _close(O1, O2, 1e-12, "reorder O")
    _close(L1, L2, 1e-12, "reorder lse")


def pin_merge_empty(o):
    """An empty partial (LSE = -inf) is the identity on either side; two empty
    partials give O = 0 and LSE = -inf with no NaN, even if O holds garbage."""
    r = _rng(12)
    Oa = r.standard_normal((3, 4))
    La = r.standard_normal(3)
    Ob = np.full((3, 4), np.nan)
    Lb = np.full(3, -np.inf)
    O, L = o.ref_lse_merge(Oa, La, Ob, Lb)
    _close(O, Oa, 0.0, "b empty O")
    _close(L, La, 0.0, "b empty lse")
    O, L = o.ref_lse_merge(Ob, Lb, Oa, La)
    _close(O, Oa, 0.0, "a empty O")
    _close(L, La, 0.0, "a empty lse")
    O, L = o.ref_lse_merge(Ob, Lb, Ob.copy(), Lb.copy())
    assert np.all(O == 0.0) and np.all(np.isneginf(L))


def pin_merge_closed_form(o):
    """Equal log-sum-exps average the outputs and add ln 2; a gap of ln 3
    weights them 3:1."""
    Oa = np.array([[1.0, -2.0]])
    Ob = np.array([[3.0, 6.0]])
    O, L = o.ref_lse_merge(Oa, np.array([0.5]), Ob, np.array([0.5]))
    _close(O, [[2.0, 2.0]], 1e-15, "equal O")
    _close(L, [0.5 + math.log(2.0)], 1e-15, "equal lse")
    O, L = o.ref_lse_merge(Oa, np.array([math.log(3.0)]), Ob, np.array([0.0]))
    _close(O, [[1.5, 0.0]], 1e-15, "3:1 O")
    _close(L, [math.log(4.0)], 1e-15, "3:1 lse")


# --------------------------------------------------------------------------
# patch step
# --------------------------------------------------------------------------

def pin_patch_splice_and_attend(o):
    """With no staleness the patch step is plain self-attention for the patch
    rows; with staleness the returned buffer is the input with exactly the
    patch rows replaced, and the result equals attention over that buffer."""
    r = _rng(13)
    B, H, N, d, Np, p0 = 1, 2, 20, 4, 6, 9
    X = r.standard_normal((B, H, N, d))
    K = r.standard_normal((B, H, N, d))
    V = r.standard_normal((B, H, N, d))
    Of, Lf = o.ref_attn(X, K, V, 0.5)
    O, L, Kn, Vn = o.ref_patch(X[:, :, p0:p0 + Np], K[:, :, p0:p0 + Np], V[:, :, p0:p0 + Np],
                               K, V, p0, 0.5)
    _close(O, Of[:, :, p0:p0 + Np], 1e-14, "patch fresh O")
    _close(L, Lf[:, :, p0:p0 + Np], 1e-14, "patch fresh lse")
    Ks = K + 0.05 * r.standard_normal(K.shape)
    Vs = V + 0.05 * r.standard_normal(V.shape)
    Ks0, Vs0 = Ks.copy(), Vs.copy()
    O, L, Kn, Vn = o.ref_patch(X[:, :, p0:p0 + Np], K[:, :, p0:p0 + Np], V[:, :, p0:p0 + Np],
                               Ks, Vs, p0, 0.5)
    assert np.array_equal(Ks, Ks0) and np.array_equal(Vs, Vs0), "input buffer modified"
    want_k = Ks0.copy(); want_k[:, :, p0:p0 + Np] = K[:, :, p0:p0 + Np]
    want_v = Vs0.copy(); want_v[:, :, p0:p0 + Np] = V[:, :, p0:p0 + Np]
    assert np.array_equal(Kn, want_k) and np.array_equal(Vn, want_v), "splice rows wrong"
    Om, Lm = o.ref_attn(X[:, :, p0:p0 + Np], want_k, want_v, 0.5)
    _close(O, Om, 1e-14, "patch stale O")
    _close(L, Lm, 1e-14, "patch stale lse")
    assert np.max(np.abs(O - Of[:, :, p0:p0 + Np])) > 1e-4, "stale rows had no effect"


def _slab_rows(p0, run_len, run_stride, n_runs):
    """Buffer row of every patch row, listed one by one (patch row j is row
    j % run_len of run j // run_len)."""
    out = []
    for j in range(n_runs * run_len):
        out.append(p0 + (j // run_len) * run_stride + j % run_len)
    return np.array(out, dtype=np.int64)


def pin_patch_strided_fresh_is_self_attention(o):
    """With no staleness a strided patch step gives the patch rows of plain
    self-attention over the whole sequence, whatever the run layout; and a
    single run is the contiguous patch step."""
    r = _rng(16)
    B, H, N, d = 1, 2, 40, 4
    X = r.standard_normal((B, H, N, d))
    K = r.standard_normal((B, H, N, d))
    V = r.standard_normal((B, H, N, d))
    Of, Lf = o.ref_attn(X, K, V, 0.5)
    for p0, run_len, stride, n_runs in ((3, 2, 5, 7), (0, 4, 10, 4), (7, 3, 3, 5), (0, 40, 40, 1)):
        idx = _slab_rows(p0, run_len, stride, n_runs)
        O, L, Kn, Vn = o.ref_patch_strided(X[:, :, idx], K[:, :, idx], V[:, :, idx], K, V, p0,
                                           run_len, stride, 0.5)
        _close(O, Of[:, :, idx], 1e-13, f"strided fresh O {p0, run_len, stride}")
        _close(L, Lf[:, :, idx], 1e-13, f"strided fresh lse {p0, run_len, stride}")
    Ks = K + 0.05 * r.standard_normal(K.shape)
    Vs = V + 0.05 * r.standard_normal(V.shape)
    p0, Np = 11, 9
    a = o.ref_patch_strided(X[:, :, p0:p0 + Np], K[:, :, p0:p0 + Np], V[:, :, p0:p0 + Np], Ks, Vs,
                            p0, Np, 1000, 0.5)
    b = o.ref_patch(X[:, :, p0:p0 + Np], K[:, :, p0:p0 + Np], V[:, :, p0:p0 + Np], Ks, Vs, p0, 0.5)
    for x, y, what in zip(a, b, ("O", "lse", "K", "V")):
        _close(x, y, 0.0, f"one run = contiguous patch {what}")


def pin_patch_strided_splice_rows(o):
    """The returned buffer is the input with exactly the patch rows replaced,
    patch row j landing on buffer row p0 + (j // run_len) * stride + j % run_len
    (rows listed one by one); and the result equals the contiguous patch step
    on a buffer whose rows are reordered so the runs come first: attention does
    not depend on the order of the key rows."""
    r = _rng(17)
    B, H, N, d = 2, 1, 36, 3
    p0, run_len, stride, n_runs = 2, 3, 8, 4
    idx = _slab_rows(p0, run_len, stride, n_runs)
    Np = idx.size
    Qp = r.standard_normal((B, H, Np, d))
    Kp = r.standard_normal((B, H, Np, d))
    Vp = r.standard_normal((B, H, Np, d))
    Ks = r.standard_normal((B, H, N, d))
    Vs = r.standard_normal((B, H, N, d))
    Ks0, Vs0 = Ks.copy(), Vs.copy()
    O, L, Kn, Vn = o.ref_patch_strided(Qp, Kp, Vp, Ks, Vs, p0, run_len, stride, 0.7)
    assert np.array_equal(Ks, Ks0) and np.array_equal(Vs, Vs0), "input buffer modified"
    want_k, want_v = Ks0.copy(), Vs0.copy()
    for j in range(Np):
        want_k[:, :, idx[j]] = Kp[:, :, j]
        want_v[:, :, idx[j]] = Vp[:, :, j]
    assert np.array_equal(Kn, want_k) and np.array_equal(Vn, want_v), "strided splice rows wrong"
    rest = np.array([i for i in range(N) if i not in set(idx.tolist())], dtype=np.int64)
    perm = np.concatenate([idx, rest])
    Oc, Lc, _, _ = o.ref_patch(Qp, Kp, Vp, Ks[:, :, perm], Vs[:, :, perm], 0, 0.7)
    _close(O, Oc, 1e-13, "strided = contiguous on reordered buffer O")
    _close(L, Lc, 1e-13, "strided = contiguous on reordered buffer lse")
    for bad in ((p0, run_len, run_len - 1), (N - 5, run_len, stride), (-1, run_len, stride)):
        try:
            o.ref_patch_strided(Qp, Kp, Vp, Ks, Vs, bad[0], bad[1], bad[2], 0.7)
        except ValueError:
            continue
        raise AssertionError(f"layout {bad} accepted")


# --------------------------------------------------------------------------
# classifier-free guidance
# --------------------------------------------------------------------------

def pin_cfg(o):
    """s = 1 returns eps_c, s = 0 returns eps_u, the result is affine in s, and
    a small exact case: u = 1, c = 3, s = 4 gives 1 + 4*2 = 9."""
    r = _rng(14)
    u = r.standard_normal((2, 4, 3, 3)).astype(np.float32)
    c = r.standard_normal((2, 4, 3, 3)).astype(np.float32)
    _close(o.ref_cfg(u, c, 1.0), c, 0.0, "s=1")
    _close(o.ref_cfg(u, c, 0.0), u, 0.0, "s=0")
    a, b = o.ref_cfg(u, c, 2.0), o.ref_cfg(u, c, 5.0)
    _close(o.ref_cfg(u, c, 3.0), a + (b - a) / 3.0, 1e-12, "affine in s")
    _close(o.ref_cfg(np.array([1.0], np.float32), np.array([3.0], np.float32), 4.0), [9.0], 0.0, "exact")


def pin_cfg_relmae(o):
    """rel-MAE: identical paths give 0; eps_c = 2 eps_u gives 1; eps_c = -eps_u gives 2."""
    u = _rng(15).standard_normal(50)
    assert o.ref_cfg_relmae(u, u) == 0.0
    assert abs(o.ref_cfg_relmae(u, 2 * u) - 1.0) < 1e-14
    assert abs(o.ref_cfg_relmae(u, -u) - 2.0) < 1e-14


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
