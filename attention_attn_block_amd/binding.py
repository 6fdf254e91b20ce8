"""Thin ctypes binding over libdit_attn.so (argument marshalling only).

Every step of the path runs in the HIP library; torch supplies device memory,
the current stream and output allocation.  If the library is missing or a
call is rejected, an exception is raised -- there is no fallback.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdit_attn.so")

DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_HIP = 0, 1, 2, 3
DIT_F32, DIT_BF16 = 0, 1

EXPORTS = ("attn_block_fwd", "attn_block_fwd_merge", "attn_block_fwd_ws",
           "attn_block_workspace_bytes", "attn_lse_merge", "attn_patch_fwd", "attn_patch_fwd_ws",
           "attn_patch_fwd_strided", "attn_ring_fwd",
           "cfg_combine", "cfg_combine_relmae", "cfg_combine_relmae_noalloc",
           "cfg_combine_relmae_workspace", "dit_status_string")

_lib = None


class DitError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} failed: {text}")
        self.code = code


def load():
    """Load libdit_attn.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m attention_attn_block_amd.build` "
            "(needs hipcc). There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, ll, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float
    L.attn_block_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.attn_block_fwd_merge.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    L.attn_block_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, ll, vp]
    L.attn_block_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_block_workspace_bytes.restype = ll
    L.attn_lse_merge.argtypes = [vp, vp, vp, vp, ll, i, i, vp]
    L.attn_patch_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.attn_patch_fwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, ll,
                                    vp]
    L.attn_patch_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i,
                                         i, vp, ll, vp]
    L.attn_ring_fwd.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, f, i, i, i, vp, ll, vp]
    L.cfg_combine.argtypes = [vp, vp, vp, ll, f, vp]
    L.cfg_combine_relmae.argtypes = [vp, vp, vp, ll, f, vp, vp, vp]
    L.cfg_combine_relmae_noalloc.argtypes = [vp, vp, vp, ll, f, vp, vp]
    L.cfg_combine_relmae_workspace.argtypes = [ll]
    L.cfg_combine_relmae_workspace.restype = ll
    for name in ("attn_block_fwd", "attn_block_fwd_merge", "attn_block_fwd_ws", "attn_lse_merge",
                 "attn_patch_fwd", "attn_patch_fwd_ws", "attn_patch_fwd_strided", "attn_ring_fwd",
                 "cfg_combine",
                 "cfg_combine_relmae",
                 "cfg_combine_relmae_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    L.dit_status_string.argtypes = [ctypes.c_int]
    L.dit_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(code):
    return load().dit_status_string(int(code)).decode()


def _check(fn, code):
    if code != DIT_OK:
        raise DitError(fn, code, status_string(code))


def _dtype(t):
    if t == torch.bfloat16:
        return DIT_BF16
    if t == torch.float32:
        return DIT_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _dev(*ts):
    dev = ts[0].device
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def default_scale(d):
    """1/sqrt(d) rounded to float32."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def attn_block_workspace(q, k):
    """Zero-filled workspace for the split calls (attn_block_fwd,
    attn_block_fwd_merge, attn_patch_fwd and attn_patch_fwd_strided with
    workspace=) of q against k's shape.  Reusable by later calls with no more
    256-row query tiles (B * H * ceil(Nq / 256)), at any head dim, one call at
    a time."""
    B, H, Nq, d = q.shape
    n = load().attn_block_workspace_bytes(B, H, Nq, k.shape[2], d)
    if n <= 0:
        raise ValueError("unsupported attention shape")
    return torch.zeros(n, dtype=torch.uint8, device=q.device)


WS_MERGE, WS_FORCE_SPLIT = 1, 2


def _attn_ws(fn, q, k, v, o, lse, scale, merge, workspace, force_split=False):
    dev = _dev(q, k, v, o, lse, workspace)
    B, H, Nq, d = q.shape
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor (attn_block_workspace)")
    with torch.cuda.device(dev):
        rc = load().attn_block_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, Nq, k.shape[2], d, scale,
                                      _dtype(q.dtype), _dtype(o.dtype),
                                      (WS_MERGE if merge else 0) | (WS_FORCE_SPLIT if force_split else 0),
                                      workspace.data_ptr(), workspace.numel(), _stream(dev))
    _check(fn, rc)


def attn_block_fwd(q, k, v, scale=None, out_dtype=None, out=None, lse=None, workspace=None,
                   force_split=False):
    """(O, LSE) = attention of q [B,H,Nq,d] against k, v [B,H,Nkv,d].  With a
    workspace (attn_block_workspace) the library may share a query tile's
    keys between workgroups to fill the GPU (attn_block_fwd_ws); force_split
    takes that path for short blocks too."""
    dev = _dev(q, k, v)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _dev(q, out, lse)
    if out.shape != (B, H, Nq, d) or out.dtype != out_dtype or lse.shape != (B, H, Nq) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse shape or dtype mismatch")
    if workspace is not None:
        _attn_ws("attn_block_fwd_ws", q, k, v, out, lse, scale, False, workspace, force_split)
        return out, lse
    with torch.cuda.device(dev):
        rc = load().attn_block_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, Nq, Nkv, d, scale, _dtype(q.dtype),
                                   _dtype(out_dtype), _stream(dev))
    _check("attn_block_fwd", rc)
    return out, lse


def attn_block_fwd_merge(q, k, v, o_acc, lse_acc, scale=None, workspace=None, force_split=False):
    """Fold the attention of q against this KV block into (o_acc, lse_acc) in
    place; rows with lse_acc = -inf are empty and take the block's result.
    workspace, force_split: as for attn_block_fwd."""
    dev = _dev(q, k, v, o_acc, lse_acc)
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, H, Nkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes/dtypes disagree")
    if o_acc.shape != (B, H, Nq, d) or lse_acc.shape != (B, H, Nq) \
            or lse_acc.dtype != torch.float32:
        raise ValueError("o_acc/lse_acc shape or dtype mismatch")
    scale = default_scale(d) if scale is None else float(scale)
    if workspace is not None:
        _attn_ws("attn_block_fwd_ws", q, k, v, o_acc, lse_acc, scale, True, workspace, force_split)
        return o_acc, lse_acc
    with torch.cuda.device(dev):
        rc = load().attn_block_fwd_merge(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         o_acc.data_ptr(), lse_acc.data_ptr(), B, H, Nq, Nkv, d,
                                         scale, _dtype(q.dtype), _dtype(o_acc.dtype), _stream(dev))
    _check("attn_block_fwd_merge", rc)
    return o_acc, lse_acc


def attn_lse_merge(o_a, lse_a, o_b, lse_b):
    """In place: (o_a, lse_a) <- merge of a and b.  o_*: [..., d], lse_*: [...]."""
    dev = _dev(o_a, lse_a, o_b, lse_b)
    d = o_a.shape[-1]
    rows = lse_a.numel()
    if o_b.shape != o_a.shape or o_a.dtype != o_b.dtype or lse_b.shape != lse_a.shape \
            or o_a.numel() != rows * d or lse_a.dtype != torch.float32 \
            or lse_b.dtype != torch.float32:
        raise ValueError("merge operand shapes/dtypes disagree")
    with torch.cuda.device(dev):
        rc = load().attn_lse_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                   lse_b.data_ptr(), rows, d, _dtype(o_a.dtype), _stream(dev))
    _check("attn_lse_merge", rc)
    return o_a, lse_a


def attn_patch_fwd(q_p, k_p, v_p, k_buf, v_buf, p0, scale=None, out_dtype=None, out=None,
                   lse=None, workspace=None):
    """Splice k_p/v_p into rows [p0, p0+Np) of k_buf/v_buf (in place), then
    attend q_p to the whole buffer.  Returns (O, LSE).  With a workspace
    (attn_block_workspace(q_p, k_buf)) the attention may take the split
    launch (attn_patch_fwd_ws)."""
    dev = _dev(q_p, k_p, v_p, k_buf, v_buf)
    B, H, Np, d = q_p.shape
    N = k_buf.shape[2]
    if k_p.shape != q_p.shape or v_p.shape != q_p.shape or k_buf.shape != (B, H, N, d) \
            or v_buf.shape != k_buf.shape \
            or len({t.dtype for t in (q_p, k_p, v_p, k_buf, v_buf)}) != 1:
        raise ValueError("patch/buffer shapes or dtypes disagree")
    out_dtype = q_p.dtype if out_dtype is None else out_dtype
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Np, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev)
    _dev(q_p, out, lse)
    if out.shape != (B, H, Np, d) or out.dtype != out_dtype or lse.shape != (B, H, Np) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse shape or dtype mismatch")
    if workspace is not None:
        _dev(q_p, workspace)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor (attn_block_workspace)")
        with torch.cuda.device(dev):
            rc = load().attn_patch_fwd_ws(q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(),
                                          k_buf.data_ptr(), v_buf.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), B, H, Np, N, int(p0), d, scale,
                                          _dtype(q_p.dtype), _dtype(out_dtype),
                                          workspace.data_ptr(), workspace.numel(), _stream(dev))
        _check("attn_patch_fwd_ws", rc)
        return out, lse
    with torch.cuda.device(dev):
        rc = load().attn_patch_fwd(q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(),
                                   k_buf.data_ptr(), v_buf.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, Np, N, int(p0), d, scale,
                                   _dtype(q_p.dtype), _dtype(out_dtype), _stream(dev))
    _check("attn_patch_fwd", rc)
    return out, lse


def attn_patch_fwd_strided(q_p, k_p, v_p, k_buf, v_buf, p0, run_len, run_stride, scale=None,
                           out_dtype=None, out=None, lse=None, workspace=None):
    """Patch step for a patch of several runs of buffer rows: the patch rows
    (q_p, k_p, v_p: [B, H, Np, d], Np a multiple of run_len) are n_runs =
    Np / run_len runs back to back, run r belonging to buffer rows
    [p0 + r * run_stride, +run_len).  Splices each run of k_p/v_p into
    k_buf/v_buf (in place), then attends q_p to the whole buffer.  Returns
    (O, LSE).  workspace: as attn_patch_fwd."""
    dev = _dev(q_p, k_p, v_p, k_buf, v_buf)
    B, H, Np, d = q_p.shape
    N = k_buf.shape[2]
    if k_p.shape != q_p.shape or v_p.shape != q_p.shape or k_buf.shape != (B, H, N, d) \
            or v_buf.shape != k_buf.shape \
            or len({t.dtype for t in (q_p, k_p, v_p, k_buf, v_buf)}) != 1:
        raise ValueError("patch/buffer shapes or dtypes disagree")
    run_len = int(run_len)
    if run_len < 1 or Np % run_len:
        raise ValueError("the patch is not a whole number of runs of run_len rows")
    n_runs = Np // run_len
    out_dtype = q_p.dtype if out_dtype is None else out_dtype
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Np, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev)
    _dev(q_p, out, lse)
    if out.shape != (B, H, Np, d) or out.dtype != out_dtype or lse.shape != (B, H, Np) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse shape or dtype mismatch")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev(q_p, workspace)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor (attn_block_workspace)")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    with torch.cuda.device(dev):
        rc = load().attn_patch_fwd_strided(q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(),
                                           k_buf.data_ptr(), v_buf.data_ptr(), out.data_ptr(),
                                           lse.data_ptr(), B, H, run_len, n_runs, int(run_stride),
                                           N, int(p0), d, scale, _dtype(q_p.dtype),
                                           _dtype(out_dtype), ws_ptr, ws_bytes, _stream(dev))
    _check("attn_patch_fwd_strided", rc)
    return out, lse


def attn_ring_fwd(q, ks, vs, scale=None, out_dtype=None, out=None, lse=None, workspace=None,
                  force_split=False):
    """(O, LSE) = attention of q [B,H,Nq,d] against the concatenation of the
    KV blocks ks[i], vs[i] ([B,H,Nkv_block,d] each, bfloat16, up to 16
    blocks) in one launch.  workspace, force_split: as for attn_block_fwd."""
    if len(ks) != len(vs) or not ks:
        raise ValueError("ks and vs must be equally long, non-empty lists of blocks")
    dev = _dev(q, *ks, *vs)
    B, H, Nq, d = q.shape
    Nkv = ks[0].shape[2]
    for kb, vb in zip(ks, vs):
        if kb.shape != (B, H, Nkv, d) or vb.shape != kb.shape or kb.dtype != q.dtype \
                or vb.dtype != q.dtype:
            raise ValueError("q and the KV blocks disagree in shape or dtype")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _dev(q, out, lse)
    if out.shape != (B, H, Nq, d) or out.dtype != out_dtype or lse.shape != (B, H, Nq) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse shape or dtype mismatch")
    n = len(ks)
    kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in ks])
    vp_ = (ctypes.c_void_p * n)(*[t.data_ptr() for t in vs])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev(q, workspace)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor (attn_block_workspace)")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    with torch.cuda.device(dev):
        rc = load().attn_ring_fwd(q.data_ptr(), kp, vp_, n, out.data_ptr(), lse.data_ptr(), B, H,
                                  Nq, Nkv, d, scale, _dtype(q.dtype), _dtype(out_dtype),
                                  WS_FORCE_SPLIT if force_split else 0, ws_ptr, ws_bytes,
                                  _stream(dev))
    _check("attn_ring_fwd", rc)
    return out, lse


def cfg_combine(eps_u, eps_c, s, out=None):
    """out = eps_u + s * (eps_c - eps_u), float32."""
    dev = _dev(eps_u, eps_c)
    if eps_u.shape != eps_c.shape or eps_u.dtype != torch.float32 or eps_c.dtype != torch.float32:
        raise ValueError("eps_u/eps_c must be float32 tensors of one shape")
    if out is None:
        out = torch.empty_like(eps_u)
    _dev(eps_u, out)
    if out.shape != eps_u.shape or out.dtype != torch.float32:
        raise ValueError("out shape/dtype mismatch")
    with torch.cuda.device(dev):
        rc = load().cfg_combine(eps_u.data_ptr(), eps_c.data_ptr(), out.data_ptr(),
                                eps_u.numel(), float(s), _stream(dev))
    _check("cfg_combine", rc)
    return out


def cfg_combine_relmae(eps_u, eps_c, s, out=None, workspace=None, relmae=None):
    """(out, relmae) with out = eps_u + s (eps_c - eps_u) and relmae =
    sum|eps_c - eps_u| / sum|eps_u| as a one-element float32 device tensor."""
    dev = _dev(eps_u, eps_c)
    if eps_u.shape != eps_c.shape or eps_u.dtype != torch.float32 or eps_c.dtype != torch.float32:
        raise ValueError("eps_u/eps_c must be float32 tensors of one shape")
    n = eps_u.numel()
    if out is None:
        out = torch.empty_like(eps_u)
    nw = load().cfg_combine_relmae_workspace(n)
    if workspace is None:
        workspace = torch.empty(max(nw, 4), dtype=torch.float32, device=dev)
    if relmae is None:
        relmae = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    _dev(eps_u, out, workspace, relmae)
    if out.shape != eps_u.shape or out.dtype != torch.float32 or workspace.numel() < nw \
            or workspace.dtype != torch.float32 or relmae.dtype != torch.float32 \
            or relmae.numel() < 1:
        raise ValueError("out/workspace/relmae shape or dtype mismatch")
    with torch.cuda.device(dev):
        rc = load().cfg_combine_relmae(eps_u.data_ptr(), eps_c.data_ptr(), out.data_ptr(), n,
                                       float(s), workspace.data_ptr(), relmae.data_ptr(),
                                       _stream(dev))
    _check("cfg_combine_relmae", rc)
    return out, relmae
