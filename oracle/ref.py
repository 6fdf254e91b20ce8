"""Plain fp64 CPU oracle for the DiT attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the entry point's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, constants or
helpers with the HIP library and imports nothing from it.

What is computed, and where it comes from
-----------------------------------------
The pages locate the cost of DiT inference in self-attention over image-patch
tokens, whose work grows with the token count ("xDiT: an Inference Engine for
Diffusion Transformers (DiTs) with Massive Parallelism", abstract).  They name
the schemes that spread that attention over devices -- sequence parallelism
and the patch pipeline PipeFusion (same abstract), Ring, Ulysses and Torus
attention ("SwiftFusion: Scalable Sequence Parallelism for Distributed
Inference of Diffusion Transformers on GPUs", sections 1 and 2) -- and the
classifier-free-guidance split into a conditional and an unconditional path
("Accelerating Diffusion via Hybrid Data-Pipeline Parallelism Based on
Conditional Guidance Scheduling", Technische Zusammenfassung, 2.A).  No page
writes a formula.  Every function below is therefore the textbook definition
of the operation the pages name, written out in fp64:

* ``ref_attn``   softmax(Q K^T * scale) V per (batch, head), plus the natural
                 log-sum-exp of each score row.  No mask, bias or dropout.
* ``ref_lse_merge``  the log-sum-exp identity that combines two partial
                 attention results over disjoint key sets (what a device does
                 when KV blocks arrive one by one around a ring or in Torus
                 chunks).
* ``ref_block_fold``  left fold of ``ref_lse_merge`` over consecutive blocks.
* ``ref_patch``  PipeFusion's per-device step read plainly: the fresh K/V of
                 the device's patch overwrite its rows of the persistent
                 (otherwise stale) KV buffer, then the patch queries attend to
                 the whole buffer.
* ``ref_patch_strided``  the same step for a patch made of several equal runs
                 of rows spaced evenly through the buffer (a row slab of a
                 video that crosses every frame: in frame-major token order
                 it is one run per frame).
* ``ref_cfg``    classifier-free guidance, out = eps_u + s (eps_c - eps_u).

Inputs are numpy arrays.  A ``uint16`` array holds bfloat16 bit patterns and
is decoded exactly (bfloat16 is the upper half of an IEEE binary32); any float
array is widened to float64.  Each function is pinned in the CPU test suite by
closed forms, invariants, library routines and brute force; none is "parity
unpinned".
"""

import numpy as np

__all__ = [
    "decode",
    "ref_attn",
    "ref_lse_merge",
    "ref_block_fold",
    "ref_patch",
    "ref_patch_strided",
    "ref_cfg",
    "ref_cfg_relmae",
]


def decode(x):
    """Widen an input array exactly to float64.

    ``uint16`` is read as bfloat16 bits: shifting them into the high half of a
    32-bit word gives the binary32 value with the same sign, exponent and the
    8 significant bits, which float64 then represents exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        with np.errstate(invalid="ignore"):  # NaN payloads widen as NaN
            return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype.kind == "f":
        return x.astype(np.float64)
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _attn_head(q, k, v, scale):
    """Steps 1-6 of the definition for one (batch, head); all fp64.

    q: [n, d] query rows, k and v: [m, d].  Returns o [n, d] and lse [n].
    """
    s = scale * (q @ k.T)                 # 1. scores s_ij = scale * <q_i, k_j>
    m = s.max(axis=1, keepdims=True)      # 2. row maximum
    e = np.exp(s - m)                     # 3. shifted exponentials
    l = e.sum(axis=1, keepdims=True)      # 4. row normaliser
    o = (e @ v) / l                       # 5. weighted mean of the values
    lse = (m + np.log(l))[:, 0]           # 6. natural log-sum-exp of the row
    return o, lse


def ref_attn(Q, K, V, scale, rows=None):
    """Attention softmax(Q K^T * scale) V and its log-sum-exp, in fp64.

    Q: [B, H, Nq, d]; K, V: [B, H, Nkv, d] (bfloat16 bits as uint16, or float).
    scale: the float the kernel receives, widened exactly.
    rows: optional 1-D array of query-row indices; then only those rows of
    every (b, h) are computed (for sampled checks at full size).
    Returns (O [B, H, nrows, d] float64, LSE [B, H, nrows] float64).
    Decoding is done one head at a time so that large bfloat16 buffers are
    never copied whole into float64.
    """
    B, H, Nq, d = Q.shape
    if K.shape[:2] != (B, H) or V.shape != K.shape or K.shape[3] != d:
        raise ValueError("shape mismatch")
    scale = float(scale)
    sel = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((B, H, sel.size, d), dtype=np.float64)
    L = np.empty((B, H, sel.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            q = decode(Q[b, h][sel])
            k = decode(K[b, h])
            v = decode(V[b, h])
            O[b, h], L[b, h] = _attn_head(q, k, v, scale)
    return O, L


def ref_lse_merge(O_a, L_a, O_b, L_b):
    """Combine two partial attention results over disjoint key sets, in fp64.

    A partial is (O, L): O the normalised output over its keys and L the
    natural log-sum-exp of its scores.  For each row:
      L_b = -inf                -> a (an empty partial is the identity)
      L_a = -inf                -> b
      otherwise  m = max(L_a, L_b),  w_a = exp(L_a - m),  w_b = exp(L_b - m),
                 O = (w_a O_a + w_b O_b) / (w_a + w_b),  L = m + ln(w_a + w_b).
    Both empty gives O = 0 and L = -inf.
    O_*: [..., d]; L_*: [...].  Returns new float64 arrays (O, L).
    """
    Oa, Ob = decode(O_a), decode(O_b)
    La, Lb = decode(L_a), decode(L_b)
    O = np.zeros(np.broadcast_shapes(Oa.shape, Ob.shape), dtype=np.float64)
    L = np.full(np.broadcast_shapes(La.shape, Lb.shape), -np.inf)
    a_empty = np.isneginf(La)
    b_empty = np.isneginf(Lb)
    only_a = b_empty & ~a_empty
    only_b = a_empty & ~b_empty
    both = ~a_empty & ~b_empty
    O[only_a], L[only_a] = Oa[only_a], La[only_a]
    O[only_b], L[only_b] = Ob[only_b], Lb[only_b]
    m = np.maximum(La[both], Lb[both])
    wa = np.exp(La[both] - m)
    wb = np.exp(Lb[both] - m)
    O[both] = (wa[:, None] * Oa[both] + wb[:, None] * Ob[both]) / (wa + wb)[:, None]
    L[both] = m + np.log(wa + wb)
    return O, L


def ref_block_fold(partials):
    """Left fold of ``ref_lse_merge`` over partials [(O_0, L_0), (O_1, L_1), ...].

    The accumulator starts as block 0; blocks 1..k-1 are merged in order, the
    way a ring device folds in each arriving KV block.
    """
    O, L = decode(partials[0][0]), decode(partials[0][1])
    for Ob, Lb in partials[1:]:
        O, L = ref_lse_merge(O, L, Ob, Lb)
    return O, L


def ref_patch(Q_p, K_p, V_p, K_buf, V_buf, p0, scale, rows=None):
    """PipeFusion per-device step: splice the fresh patch, then attend.

    Q_p, K_p, V_p: [B, H, Np, d] (the device's patch); K_buf, V_buf:
    [B, H, N, d], the persistent KV buffer whose rows outside the patch hold
    stale values from the previous denoising step.  Rows [p0, p0 + Np) of the
    buffer are replaced by K_p / V_p (a copy: same dtype, same bits), then the
    patch queries attend to all N rows.
    Returns (O, LSE, K_new, V_new); the input buffers are left untouched.
    """
    Np = Q_p.shape[2]
    N = K_buf.shape[2]
    if not (0 <= p0 and p0 + Np <= N):
        raise ValueError("patch outside the buffer")
    K_new = np.array(K_buf, copy=True)
    V_new = np.array(V_buf, copy=True)
    K_new[:, :, p0:p0 + Np] = K_p
    V_new[:, :, p0:p0 + Np] = V_p
    O, L = ref_attn(Q_p, K_new, V_new, scale, rows=rows)
    return O, L, K_new, V_new


def ref_patch_strided(Q_p, K_p, V_p, K_buf, V_buf, p0, run_len, run_stride, scale, rows=None):
    """PipeFusion per-device step for a patch of several runs of buffer rows.

    The pages let devices hold patches of unequal size ("Spatio-Temporal
    Parallelism for Diffusion Model Inference on Heterogeneous Multi-GPU
    Systems", abstract) and split the image into patches (xDiT abstract) but
    do not fix their shape.  A patch that is a band of spatial rows across
    all frames of a video is, in frame-major token order, not one range of
    the sequence but one run per frame.  Here the patch is n_runs runs of
    run_len rows; run r covers buffer rows
        [p0 + r * run_stride, p0 + r * run_stride + run_len),
    and the device's patch tensors hold the runs back to back, so patch row
    r * run_len + i belongs to buffer row p0 + r * run_stride + i.
    Q_p, K_p, V_p: [B, H, n_runs * run_len, d]; K_buf, V_buf: [B, H, N, d].
    Each run of K_p / V_p is copied over its rows of the buffer, then the
    patch queries attend to all N rows (as ``ref_patch``).
    Returns (O, LSE, K_new, V_new); the input buffers are left untouched.
    """
    Np = Q_p.shape[2]
    N = K_buf.shape[2]
    if run_len < 1 or Np % run_len:
        raise ValueError("the patch is not a whole number of runs")
    n_runs = Np // run_len
    if n_runs > 1 and run_stride < run_len:
        raise ValueError("runs overlap")
    if p0 < 0 or p0 + (n_runs - 1) * run_stride + run_len > N:
        raise ValueError("patch outside the buffer")
    K_new = np.array(K_buf, copy=True)
    V_new = np.array(V_buf, copy=True)
    for r in range(n_runs):
        start = p0 + r * run_stride
        K_new[:, :, start:start + run_len] = K_p[:, :, r * run_len:(r + 1) * run_len]
        V_new[:, :, start:start + run_len] = V_p[:, :, r * run_len:(r + 1) * run_len]
    O, L = ref_attn(Q_p, K_new, V_new, scale, rows=rows)
    return O, L, K_new, V_new


def ref_cfg(eps_u, eps_c, s):
    """Classifier-free guidance in fp64: eps_u + s * (eps_c - eps_u)."""
    u, c = decode(eps_u), decode(eps_c)
    return u + float(s) * (c - u)


def ref_cfg_relmae(eps_u, eps_c):
    """Relative mean absolute discrepancy between the two guidance paths.

    Hybridiff switches its parallel phases on a relative MAE between the
    conditional and unconditional noise predictions ("Accelerating Diffusion
    via Hybrid Data-Pipeline Parallelism ...", Technische Zusammenfassung,
    2.B).  The page gives no formula; the plain reading used here is
    sum|eps_c - eps_u| / sum|eps_u| over the whole tensor, in fp64.
    """
    u, c = decode(eps_u), decode(eps_c)
    return float(np.abs(c - u).sum() / np.abs(u).sum())
