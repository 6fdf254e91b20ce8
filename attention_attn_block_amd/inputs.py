"""Seeded synthetic inputs for the DiT attention workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic.  It is the one piece shared by the
tests, the benchmark and the smoke check, on both sides of a parity check.

Every tensor is drawn on the CPU with ``torch.Generator().manual_seed(seed)``
as float32 N(0, 1) in the order listed per workload, then rounded to bfloat16
with round-to-nearest-even (``Tensor.to(torch.bfloat16)``) where the workload
is bfloat16.  Layout is [B, H, N, d], contiguous, d innermost.

The workloads stand in for the pages' DiT image and video generation (no
public dataset or benchmark is named there):

* ``tiny_f32``      B1 H1 N256 d64 fp32 (16x16 latent patch grid), split into
                    4 KV blocks of 64 tokens for the merge check.
* ``dit_xl_256``    DiT-XL/2 at 256 px: B2 (cond + uncond) H16 N256 d72 bf16,
                    plus two [2, 4, 32, 32] fp32 noise predictions for the
                    guidance combine (scale 4).
* ``pixart_1024``   PixArt-style 1024 px: B2 H16 N4096 d72 bf16.
* ``ring_2048px``   one sequence-parallel device at 2048 px: B1 H24 d128,
                    a 2048-token query block and 8 KV blocks of 2048 tokens.
* ``video_patch``   one PipeFusion device of a video DiT: B1 H24 d128,
                    N = 32768 (8 frames of 64x64 patches), patch of 8192
                    queries at token offset 8192; the KV buffer holds the
                    fresh K/V plus N(0, 0.05^2) noise (stale), the fresh patch
                    holds the un-noised K/V of its rows.
* ``video_slab_patch``  the same video cut into 4 patches of 16 spatial rows
                    across all 8 frames: in frame-major token order patch p is
                    8 runs of 1024 tokens, one per frame (runs start at
                    p * 1024 + f * 4096); same draws and staleness.
"""

import math

import torch

__all__ = [
    "WORKLOADS",
    "default_scale",
    "randn",
    "attn_inputs",
    "tiny_f32",
    "dit_xl_256",
    "pixart_1024",
    "ring_2048px",
    "video_patch",
    "video_slab_patch",
    "cfg_inputs",
    "make",
]

WORKLOADS = {
    "tiny_f32": dict(seed=1, B=1, H=1, Nq=256, Nkv=256, d=64, dtype="f32", blocks=4),
    "dit_xl_256": dict(seed=2, B=2, H=16, Nq=256, Nkv=256, d=72, dtype="bf16",
                       cfg_shape=(2, 4, 32, 32), cfg_scale=4.0),
    "pixart_1024": dict(seed=3, B=2, H=16, Nq=4096, Nkv=4096, d=72, dtype="bf16"),
    "ring_2048px": dict(seed=4, B=1, H=24, Nq=2048, Nkv=2048, d=128, dtype="bf16", blocks=8),
    "video_patch": dict(seed=5, B=1, H=24, Nq=8192, Nkv=32768, d=128, dtype="bf16",
                        p0=8192, stale_std=0.05),
}


def default_scale(d):
    """1/sqrt(d) rounded to float32, returned as a Python float."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _gen(seed):
    return torch.Generator(device="cpu").manual_seed(int(seed))


def randn(shape, gen, dtype="bf16", std=1.0):
    """float32 N(0, std^2) draw, rounded to ``dtype`` ("bf16" or "f32")."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def attn_inputs(B, H, Nq, Nkv, d, dtype="bf16", seed=0):
    """Q, K, V drawn in that order from one generator."""
    g = _gen(seed)
    q = randn((B, H, Nq, d), g, dtype)
    k = randn((B, H, Nkv, d), g, dtype)
    v = randn((B, H, Nkv, d), g, dtype)
    return q, k, v


def tiny_f32(seed=None):
    w = WORKLOADS["tiny_f32"]
    q, k, v = attn_inputs(w["B"], w["H"], w["Nq"], w["Nkv"], w["d"], "f32",
                          w["seed"] if seed is None else seed)
    return dict(q=q, k=k, v=v, scale=default_scale(w["d"]), blocks=w["blocks"])


def cfg_inputs(shape, seed, gen=None):
    """eps_u then eps_c, float32 N(0, 1)."""
    g = _gen(seed) if gen is None else gen
    u = randn(shape, g, "f32")
    c = randn(shape, g, "f32")
    return u, c


def dit_xl_256(seed=None):
    w = WORKLOADS["dit_xl_256"]
    g = _gen(w["seed"] if seed is None else seed)
    shp_q = (w["B"], w["H"], w["Nq"], w["d"])
    shp_kv = (w["B"], w["H"], w["Nkv"], w["d"])
    q = randn(shp_q, g)
    k = randn(shp_kv, g)
    v = randn(shp_kv, g)
    eps_u, eps_c = cfg_inputs(w["cfg_shape"], None, gen=g)
    return dict(q=q, k=k, v=v, scale=default_scale(w["d"]),
                eps_u=eps_u, eps_c=eps_c, s=w["cfg_scale"])


def pixart_1024(seed=None):
    w = WORKLOADS["pixart_1024"]
    q, k, v = attn_inputs(w["B"], w["H"], w["Nq"], w["Nkv"], w["d"], "bf16",
                          w["seed"] if seed is None else seed)
    return dict(q=q, k=k, v=v, scale=default_scale(w["d"]))


def ring_2048px(seed=None):
    """Q, then K_0, V_0, ..., K_7, V_7."""
    w = WORKLOADS["ring_2048px"]
    g = _gen(w["seed"] if seed is None else seed)
    q = randn((w["B"], w["H"], w["Nq"], w["d"]), g)
    ks, vs = [], []
    for _ in range(w["blocks"]):
        ks.append(randn((w["B"], w["H"], w["Nkv"], w["d"]), g))
        vs.append(randn((w["B"], w["H"], w["Nkv"], w["d"]), g))
    return dict(q=q, ks=ks, vs=vs, scale=default_scale(w["d"]))


def video_patch(seed=None, p0=None, N=None, Np=None, H=None):
    """Patch queries, fresh patch K/V and the stale KV buffer.

    Draw order: Q_p; K and V for all N rows; noise_K, noise_V (std 0.05).
    Buffer = bf16(K + noise), bf16(V + noise) for every row (entirely stale
    before the call); fresh patch = bf16(K), bf16(V) of rows [p0, p0 + Np).
    ``N``, ``Np``, ``H`` and ``p0`` may be shrunk for small parity cases.
    """
    w = WORKLOADS["video_patch"]
    g = _gen(w["seed"] if seed is None else seed)
    B, d = w["B"], w["d"]
    H = w["H"] if H is None else H
    N = w["Nkv"] if N is None else N
    Np = w["Nq"] if Np is None else Np
    p0 = w["p0"] if p0 is None else p0
    q_p = randn((B, H, Np, d), g)
    k = randn((B, H, N, d), g, "f32")
    v = randn((B, H, N, d), g, "f32")
    nk = randn((B, H, N, d), g, "f32", std=w["stale_std"])
    nv = randn((B, H, N, d), g, "f32", std=w["stale_std"])
    k_buf = (k + nk).to(torch.bfloat16)
    v_buf = (v + nv).to(torch.bfloat16)
    k_p = k[:, :, p0:p0 + Np].to(torch.bfloat16).contiguous()
    v_p = v[:, :, p0:p0 + Np].to(torch.bfloat16).contiguous()
    del k, v, nk, nv
    return dict(q_p=q_p, k_p=k_p, v_p=v_p, k_buf=k_buf, v_buf=v_buf, p0=p0,
                scale=default_scale(d))


def video_slab_patch(seed=None, p=1, frames=8, height=64, width=64, slab=16, H=None):
    """A row-slab patch of the video workload: spatial rows [p*slab, (p+1)*slab)
    of every frame.  Tokens are frame-major (frame, row, column), so the patch
    is `frames` runs of slab*width tokens, run f starting at token
    p*slab*width + f*height*width.  Draw order and staleness as video_patch
    (Q_p; K, V for all rows; noise_K, noise_V); the fresh patch holds the
    un-noised K/V of the patch rows, runs back to back.  Returns the tensors
    plus p0, run_len, run_stride and n_runs."""
    w = WORKLOADS["video_patch"]
    g = _gen(w["seed"] if seed is None else seed)
    B, d = w["B"], w["d"]
    H = w["H"] if H is None else H
    N = frames * height * width
    run_len, run_stride, n_runs = slab * width, height * width, frames
    p0 = p * slab * width
    Np = run_len * n_runs
    rows = torch.cat([torch.arange(p0 + f * run_stride, p0 + f * run_stride + run_len)
                      for f in range(n_runs)])
    q_p = randn((B, H, Np, d), g)
    k = randn((B, H, N, d), g, "f32")
    v = randn((B, H, N, d), g, "f32")
    nk = randn((B, H, N, d), g, "f32", std=w["stale_std"])
    nv = randn((B, H, N, d), g, "f32", std=w["stale_std"])
    k_buf = (k + nk).to(torch.bfloat16)
    v_buf = (v + nv).to(torch.bfloat16)
    k_p = k[:, :, rows].to(torch.bfloat16).contiguous()
    v_p = v[:, :, rows].to(torch.bfloat16).contiguous()
    del k, v, nk, nv
    return dict(q_p=q_p, k_p=k_p, v_p=v_p, k_buf=k_buf, v_buf=v_buf, p0=p0, run_len=run_len,
                run_stride=run_stride, n_runs=n_runs, scale=default_scale(d))


def make(name, **kw):
    return {
        "tiny_f32": tiny_f32,
        "dit_xl_256": dit_xl_256,
        "pixart_1024": pixart_1024,
        "ring_2048px": ring_2048px,
        "video_patch": video_patch,
        "video_slab_patch": video_slab_patch,
    }[name](**kw)
