"""CPU tests of the C ABI: the library loads, exports every declared call, and
rejects bad arguments before any HIP call (no GPU needed: a call that reached
the HIP runtime here would return DIT_ERR_HIP, not the validation code)."""

import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

from attention_attn_block_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")

OK, INV, UNS, HIP = 0, 1, 2, 3
F32, BF16 = 0, 1

# Fake, 16-byte aligned, widely spaced device addresses: validation only looks
# at their values.
BASE = 0x7F0000000000
GAP = 1 << 36


def ptr(i, off=0):
    return BASE + i * GAP + off


SPLIT_RECORD_BYTES = 256 + 4 * 256 * (128 + 1) * 4


def split_ws_bytes(B, H, Nq, d):
    """One fixed record per 256-row query tile, whatever the head dim: a
    counter in the first 256 bytes, then four fp32 partials of 256 rows x
    (128 + 1) floats."""
    items = B * H * ((Nq + 255) // 256)
    return items * SPLIT_RECORD_BYTES


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_calls():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings(lib):
    for code in (OK, INV, UNS, HIP):
        s = binding.status_string(code)
        assert s.startswith(["DIT_OK", "DIT_ERR_INVALID_ARG", "DIT_ERR_UNSUPPORTED", "DIT_ERR_HIP"][code])
    assert "unknown" in binding.status_string(17)


# ---------------------------------------------------------------------------
# attn_block_fwd
# ---------------------------------------------------------------------------

def block(lib, **kw):
    a = dict(Q=ptr(0), K=ptr(1), V=ptr(2), O=ptr(3), LSE=ptr(4), B=1, H=2, Nq=100, Nkv=70, d=64,
             scale=0.125, i=BF16, o=BF16)
    a.update(kw)
    return lib.attn_block_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Nq"],
                              a["Nkv"], a["d"], a["scale"], a["i"], a["o"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(K=None), INV), (dict(V=None), INV), (dict(O=None), INV),
    (dict(LSE=None), INV),
    (dict(B=0), INV), (dict(H=-1), INV), (dict(Nq=0), INV), (dict(Nkv=0), INV), (dict(d=0), INV),
    (dict(scale=0.0), INV), (dict(scale=-1.0), INV), (dict(scale=math.nan), INV),
    (dict(scale=math.inf), INV),
    (dict(i=7), INV), (dict(o=-1), INV),
    (dict(Q=ptr(0, 2)), INV), (dict(K=ptr(1, 8)), INV), (dict(O=ptr(3, 4)), INV),
    (dict(LSE=ptr(4, 4)), INV),
    (dict(d=60), UNS), (dict(d=136), UNS), (dict(d=4), UNS),
    (dict(i=F32, o=BF16), UNS),
    (dict(B=1 << 20, H=1 << 12), UNS),
    (dict(O=ptr(0, 64)), INV),                   # O overlaps Q
    (dict(LSE=ptr(3, 256)), INV),                # LSE overlaps O
    (dict(O=ptr(1)), INV),                       # O aliases K
])
def test_attn_block_fwd_rejects(lib, kw, code):
    assert block(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_lse_merge
# ---------------------------------------------------------------------------

def merge(lib, **kw):
    a = dict(Oa=ptr(0), La=ptr(1), Ob=ptr(2), Lb=ptr(3), rows=1000, d=128, t=F32)
    a.update(kw)
    return lib.attn_lse_merge(a["Oa"], a["La"], a["Ob"], a["Lb"], a["rows"], a["d"], a["t"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Oa=None), INV), (dict(La=None), INV), (dict(Ob=None), INV), (dict(Lb=None), INV),
    (dict(rows=0), INV), (dict(rows=-5), INV), (dict(d=0), INV), (dict(t=3), INV),
    (dict(Oa=ptr(0, 4)), INV), (dict(Lb=ptr(3, 8)), INV),
    (dict(d=12), UNS), (dict(d=256), UNS),
    (dict(Ob=ptr(0)), INV),                      # O aliased but LSE not
    (dict(Ob=ptr(0, 512)), INV),                 # partial overlap of O
    (dict(Lb=ptr(1, 16)), INV),                  # partial overlap of LSE
    (dict(La=ptr(0, 1024)), INV),                # LSE_a inside O_a
])
def test_attn_lse_merge_rejects(lib, kw, code):
    assert merge(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_patch_fwd
# ---------------------------------------------------------------------------

def patch(lib, **kw):
    a = dict(Q=ptr(0), Kp=ptr(1), Vp=ptr(2), Kb=ptr(3), Vb=ptr(4), O=ptr(5), L=ptr(6), B=1, H=4,
             Np=64, N=256, p0=64, d=128, scale=0.088, i=BF16, o=BF16)
    a.update(kw)
    return lib.attn_patch_fwd(a["Q"], a["Kp"], a["Vp"], a["Kb"], a["Vb"], a["O"], a["L"], a["B"],
                              a["H"], a["Np"], a["N"], a["p0"], a["d"], a["scale"], a["i"], a["o"],
                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(Kp=None), INV), (dict(Vp=None), INV), (dict(Kb=None), INV),
    (dict(Vb=None), INV), (dict(O=None), INV), (dict(L=None), INV),
    (dict(p0=-1), INV), (dict(p0=200), INV), (dict(Np=257), INV), (dict(Np=0), INV),
    (dict(N=0), INV), (dict(scale=0.0), INV),
    (dict(Kp=ptr(1, 2)), INV), (dict(Vb=ptr(4, 8)), INV),
    (dict(d=100), UNS), (dict(i=F32, o=BF16), UNS),
    (dict(Kp=ptr(3, 4096)), INV),                # fresh patch inside the buffer
    (dict(Vb=ptr(3, 1 << 16)), INV),             # K and V buffers overlap
    (dict(O=ptr(4, 128)), INV),                  # output inside V buffer
])
def test_attn_patch_fwd_rejects(lib, kw, code):
    assert patch(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_patch_fwd_strided
# ---------------------------------------------------------------------------

def strided(lib, **kw):
    a = dict(Q=ptr(0), Kp=ptr(1), Vp=ptr(2), Kb=ptr(3), Vb=ptr(4), O=ptr(5), L=ptr(6), B=1, H=4,
             run_len=64, n_runs=8, stride=512, N=4096, p0=64, d=128, scale=0.088, i=BF16, o=BF16,
             W=None, nbytes=0)
    a.update(kw)
    return lib.attn_patch_fwd_strided(a["Q"], a["Kp"], a["Vp"], a["Kb"], a["Vb"], a["O"], a["L"],
                                      a["B"], a["H"], a["run_len"], a["n_runs"], a["stride"],
                                      a["N"], a["p0"], a["d"], a["scale"], a["i"], a["o"], a["W"],
                                      a["nbytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(Kp=None), INV), (dict(Vb=None), INV), (dict(L=None), INV),
    (dict(run_len=0), INV), (dict(run_len=-4), INV), (dict(n_runs=0), INV), (dict(N=0), INV),
    (dict(p0=-1), INV),
    (dict(stride=63), INV),                      # runs overlap
    (dict(stride=-512), INV),                    # runs backwards
    (dict(p0=449), INV),                         # last run ends one row past the buffer
    (dict(n_runs=9), INV),                       # a ninth run does not fit
    (dict(run_len=1 << 16, n_runs=1 << 15, stride=1 << 16, N=(1 << 31) - 1, p0=0), INV),  # ends at 2^31
    (dict(d=100), UNS), (dict(i=F32, o=BF16), UNS), (dict(scale=math.inf), INV),
    (dict(Kp=ptr(3, 4096)), INV),                # fresh patch inside the buffer
    (dict(O=ptr(4, 128)), INV),                  # output inside the V buffer
    (dict(W=ptr(7)), INV),                       # workspace of 0 bytes
    (dict(W=ptr(7, 16), nbytes=split_ws_bytes(1, 4, 512, 128)), INV),   # misaligned workspace
    (dict(W=ptr(3), nbytes=split_ws_bytes(1, 4, 512, 128)), INV),       # workspace is K_buf
])
def test_attn_patch_fwd_strided_rejects(lib, kw, code):
    assert strided(lib, **kw) == code


def test_attn_patch_fwd_strided_edge_layouts_pass_validation(lib):
    """Layouts at the limits are accepted by the checks: the call then reaches
    the HIP runtime, which fails here without a GPU (DIT_ERR_HIP), not the
    validation codes.  One run ignores the stride; touching runs (stride ==
    run_len) and a last run ending exactly at N are allowed."""
    for kw in (dict(n_runs=1, stride=0, run_len=512), dict(stride=64),
               dict(p0=448), dict(B=1, H=70000, run_len=1, n_runs=1, N=2, p0=1, d=8)):
        assert strided(lib, **kw) == HIP, kw


# ---------------------------------------------------------------------------
# attn_ring_fwd (a ring step's resident KV blocks in one launch)
# ---------------------------------------------------------------------------

def ring(lib, **kw):
    a = dict(Q=ptr(0), O=ptr(1), L=ptr(2), n=8, B=1, H=24, Nq=2048, Nkv=2048, d=128, scale=0.088,
             i=BF16, o=F32, flags=0, W=None, nbytes=0, ks=None, vs=None)
    a.update(kw)
    n = a["n"]
    ks = a["ks"] if a["ks"] is not None else [ptr(3 + j) for j in range(max(n, 0))]
    vs = a["vs"] if a["vs"] is not None else [ptr(20 + j) for j in range(max(n, 0))]
    karr = (ctypes.c_void_p * max(len(ks), 1))(*ks) if ks else None
    varr = (ctypes.c_void_p * max(len(vs), 1))(*vs) if vs else None
    return lib.attn_ring_fwd(a["Q"], karr, varr, n, a["O"], a["L"], a["B"], a["H"], a["Nq"],
                             a["Nkv"], a["d"], a["scale"], a["i"], a["o"], a["flags"], a["W"],
                             a["nbytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(O=None), INV), (dict(L=None), INV),
    (dict(n=0, ks=[], vs=[]), INV), (dict(n=17), INV),
    (dict(ks=[ptr(3)] * 7 + [None]), INV),            # a null block
    (dict(vs=[ptr(20)] * 7 + [ptr(27, 8)]), INV),      # a misaligned block
    (dict(B=0), INV), (dict(Nkv=0), INV), (dict(scale=-1.0), INV), (dict(d=60), UNS),
    (dict(i=F32, o=F32), UNS),                         # fp32 inputs: per-block calls instead
    (dict(Nkv=(1 << 20) + 1), UNS),                    # past the block-length limit
    (dict(flags=1), INV), (dict(flags=4), INV),        # merge flag or unknown flags
    (dict(O=ptr(0, 64)), INV),                         # output overlaps Q
    (dict(O=ptr(9)), INV),                             # output is K block 6
    (dict(L=ptr(25, 128)), INV),                       # LSE inside V block 5
    (dict(W=ptr(30)), INV),                            # workspace of 0 bytes
    (dict(W=ptr(30, 16), nbytes=192 * SPLIT_RECORD_BYTES), INV),   # misaligned workspace
    (dict(W=ptr(4), nbytes=192 * SPLIT_RECORD_BYTES), INV),        # workspace is K block 1
])
def test_attn_ring_fwd_rejects(lib, kw, code):
    assert ring(lib, **kw) == code


def test_attn_ring_fwd_accepts_repeated_blocks(lib):
    """Blocks are read only, so the same block may appear more than once; a
    valid call gets past the checks to the HIP runtime (DIT_ERR_HIP here,
    without a GPU)."""
    assert ring(lib, ks=[ptr(3)] * 8, vs=[ptr(20)] * 8) == HIP
    assert ring(lib, n=16, Nkv=64) == HIP
    assert ring(lib, W=ptr(40), nbytes=192 * SPLIT_RECORD_BYTES, flags=2) == HIP


def test_block_division_is_exact():
    """The kernel finds the block of key tile t of a block set as
    mulhi(t, ceil(2^32 / tpb)) (tpb >= 2 tiles per block); exact for every
    tile index of up to 16 blocks of up to 2^20 keys (the ABI's limits)."""
    import random
    rng = random.Random(5)
    sizes = list(range(2, 200)) + [1 << 14, (1 << 14) - 1, 4096, 8191] + \
        [rng.randrange(2, (1 << 14) + 1) for _ in range(200)]
    for tpb in sizes:
        m = ((1 << 32) + tpb - 1) // tpb
        n_all = 16 * tpb
        probes = set(range(min(n_all, 3000))) | {n_all - 1, n_all - 2, n_all // 2}
        probes |= {rng.randrange(n_all) for _ in range(500)}
        for t in probes:
            assert (t * m) >> 32 == t // tpb, (tpb, t)


# ---------------------------------------------------------------------------
# cfg_combine
# ---------------------------------------------------------------------------

def cfg(lib, **kw):
    a = dict(u=ptr(0), c=ptr(1), o=ptr(2), n=8192, s=4.0)
    a.update(kw)
    return lib.cfg_combine(a["u"], a["c"], a["o"], a["n"], a["s"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), INV), (dict(c=None), INV), (dict(o=None), INV), (dict(n=0), INV),
    (dict(n=-3), INV), (dict(s=math.nan), INV), (dict(s=-math.inf), INV),
    (dict(u=ptr(0, 4)), INV), (dict(o=ptr(2, 8)), INV),
    (dict(o=ptr(0, 16)), INV),                   # out partially overlaps eps_u
    (dict(o=ptr(1, 32)), INV),                   # out partially overlaps eps_c
])
def test_cfg_combine_rejects(lib, kw, code):
    assert cfg(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_block_fwd_merge
# ---------------------------------------------------------------------------

def fused(lib, **kw):
    a = dict(Q=ptr(0), K=ptr(1), V=ptr(2), O=ptr(3), LSE=ptr(4), B=1, H=2, Nq=100, Nkv=70, d=128,
             scale=0.088, i=BF16, o=F32)
    a.update(kw)
    return lib.attn_block_fwd_merge(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"],
                                    a["Nq"], a["Nkv"], a["d"], a["scale"], a["i"], a["o"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), INV), (dict(O=None), INV), (dict(LSE=None), INV), (dict(Nkv=0), INV),
    (dict(scale=-0.5), INV), (dict(o=9), INV), (dict(O=ptr(3, 8)), INV),
    (dict(d=130), UNS), (dict(i=F32, o=BF16), UNS),
    (dict(O=ptr(2, 32)), INV),                   # accumulator overlaps V
    (dict(LSE=ptr(3, 1024)), INV),               # LSE_acc inside O_acc
])
def test_attn_block_fwd_merge_rejects(lib, kw, code):
    assert fused(lib, **kw) == code


# ---------------------------------------------------------------------------
# attn_block_fwd_ws (split launch with a caller workspace)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 24, 2048, 2048, 128), (2, 16, 4096, 4096, 72),
                                   (1, 1, 1, 1, 8), (3, 5, 257, 9, 64)])
def test_block_workspace_bytes(lib, shape):
    B, H, Nq, Nkv, d = shape
    assert lib.attn_block_workspace_bytes(B, H, Nq, Nkv, d) == split_ws_bytes(B, H, Nq, d)


def test_block_workspace_records_do_not_depend_on_the_head_dim(lib):
    """A counter sits at the start of its tile's record for every shape, so the
    counters of one call never fall inside another call's partial slots."""
    sizes = {lib.attn_block_workspace_bytes(1, 24, 2048, 2048, d) for d in range(8, 129, 8)}
    assert sizes == {192 * SPLIT_RECORD_BYTES}
    assert lib.attn_block_workspace_bytes(1, 24, 1024, 2048, 64) == 96 * SPLIT_RECORD_BYTES


def test_block_workspace_bytes_invalid(lib):
    for args in [(0, 1, 1, 1, 64), (1, 0, 1, 1, 64), (1, 1, 0, 1, 64), (1, 1, 1, 0, 64),
                 (1, 1, 1, 1, 60), (1, 1, 1, 1, 136)]:
        assert lib.attn_block_workspace_bytes(*args) == 0


def block_ws(lib, **kw):
    a = dict(Q=ptr(0), K=ptr(1), V=ptr(2), O=ptr(3), LSE=ptr(4), B=1, H=24, Nq=2048, Nkv=2048,
             d=128, scale=0.088, i=BF16, o=F32, flags=0, W=ptr(5), nbytes=None)
    a.update(kw)
    n = split_ws_bytes(a["B"], a["H"], a["Nq"], a["d"]) if a["nbytes"] is None else a["nbytes"]
    return lib.attn_block_fwd_ws(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Nq"],
                                 a["Nkv"], a["d"], a["scale"], a["i"], a["o"], a["flags"], a["W"],
                                 n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), INV),
    (dict(nbytes=split_ws_bytes(1, 24, 2048, 128) - 1), INV),   # short
    (dict(W=ptr(5, 16)), INV),                                   # not 256-byte aligned
    (dict(flags=4), INV), (dict(flags=-1), INV), (dict(flags=8), INV),     # unknown flags
    (dict(W=ptr(4, 256)), INV),                                  # overlaps LSE
    (dict(W=ptr(0, 1 << 20)), INV),                              # inside Q
    (dict(Q=None), INV), (dict(d=60), UNS), (dict(scale=0.0), INV),
    (dict(O=ptr(2, 32)), INV),                                   # output overlaps V
])
def test_attn_block_fwd_ws_rejects(lib, kw, code):
    assert block_ws(lib, **kw) == code


def patch_ws(lib, **kw):
    a = dict(Qp=ptr(0), Kp=ptr(1), Vp=ptr(2), Kb=ptr(3), Vb=ptr(4), O=ptr(5), LSE=ptr(6), B=1, H=24,
             Np=4096, N=32768, p0=8192, d=128, scale=0.088, i=BF16, o=BF16, W=ptr(7), nbytes=None)
    a.update(kw)
    n = split_ws_bytes(a["B"], a["H"], a["Np"], a["d"]) if a["nbytes"] is None else a["nbytes"]
    return lib.attn_patch_fwd_ws(a["Qp"], a["Kp"], a["Vp"], a["Kb"], a["Vb"], a["O"], a["LSE"],
                                 a["B"], a["H"], a["Np"], a["N"], a["p0"], a["d"], a["scale"],
                                 a["i"], a["o"], a["W"], n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), INV),
    (dict(nbytes=split_ws_bytes(1, 24, 4096, 128) - 4), INV),  # short
    (dict(W=ptr(7, 128)), INV),                                  # not 256-byte aligned
    (dict(W=ptr(3, 4096)), INV),                                 # inside K_buf
    (dict(p0=30000), INV),                                       # patch past the buffer end
    (dict(Kp=None), INV), (dict(d=100), UNS),
])
def test_attn_patch_fwd_ws_rejects(lib, kw, code):
    assert patch_ws(lib, **kw) == code


# ---------------------------------------------------------------------------
# cfg_combine_relmae
# ---------------------------------------------------------------------------

def relmae(lib, **kw):
    a = dict(u=ptr(0), c=ptr(1), o=ptr(2), n=8192, s=4.0, w=ptr(3), r=ptr(4))
    a.update(kw)
    return lib.cfg_combine_relmae(a["u"], a["c"], a["o"], a["n"], a["s"], a["w"], a["r"], None)


def test_relmae_workspace_size(lib):
    assert lib.cfg_combine_relmae_workspace(0) == 0
    assert lib.cfg_combine_relmae_workspace(1) == 2
    assert lib.cfg_combine_relmae_workspace(4096) == 2
    assert lib.cfg_combine_relmae_workspace(8192) == 4
    assert lib.cfg_combine_relmae_workspace(4 * 1024 + 4) == 4
    assert lib.cfg_combine_relmae_workspace(1 << 26) == 2 * (1 << 14)


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), INV), (dict(w=None), INV), (dict(r=None), INV), (dict(n=0), INV),
    (dict(s=math.inf), INV), (dict(w=ptr(3, 4)), INV), (dict(r=ptr(4, 8)), INV),
    (dict(o=ptr(1, 16)), INV),                   # out partially overlaps eps_c
    (dict(w=ptr(2, 64)), INV),                   # workspace inside out
    (dict(r=ptr(3)), INV),                       # result aliases the workspace
])
def test_cfg_combine_relmae_rejects(lib, kw, code):
    assert relmae(lib, **kw) == code


def relmae_noalloc(lib, **kw):
    a = dict(u=ptr(0), c=ptr(1), o=ptr(2), n=8192, s=4.0, r=ptr(4))
    a.update(kw)
    return lib.cfg_combine_relmae_noalloc(a["u"], a["c"], a["o"], a["n"], a["s"], a["r"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), INV), (dict(c=None), INV), (dict(o=None), INV), (dict(r=None), INV),
    (dict(n=0), INV), (dict(n=-3), INV), (dict(s=math.nan), INV), (dict(r=ptr(4, 8)), INV),
    (dict(o=ptr(1, 16)), INV),                   # out partially overlaps eps_c
    (dict(r=ptr(2, 64)), INV),                   # result inside out
    (dict(n=(1 << 27) + 1), UNS),                # beyond the library's fixed array
])
def test_cfg_combine_relmae_noalloc_rejects(lib, kw, code):
    assert relmae_noalloc(lib, **kw) == code


# ---------------------------------------------------------------------------
# Python binding: marshalling checks that never reach the library
# ---------------------------------------------------------------------------

def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 1, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_block_fwd(q, q, q)
    with pytest.raises(ValueError):
        binding.cfg_combine(torch.zeros(4), torch.zeros(4), 1.0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.load()
