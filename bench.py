"""Benchmark of the DiT per-device attention step on one MI355X.

One step = one pass of the whole hot path over synthetic DiT-shaped inputs
that are resident in HBM before timing starts:

  1. sequence-parallel (Ring/Torus) share at 2048 px: B1 H24 d128, a 2048-token
     query block against 8 KV blocks of 2048 tokens -> 8 attn_block_fwd calls
     (fp32 partials) folded by 7 attn_lse_merge calls;
  2. PipeFusion share of a video DiT: B1 H24 d128, 8192 patch queries at token
     offset 8192 against a 32768-row KV buffer of fresh and stale blocks ->
     one attn_patch_fwd call (splice + attention);
  3. classifier-free guidance on two [2, 4, 32, 32] fp32 noise predictions,
     s = 4 -> one cfg_combine call.

Prints ONE JSON line.  `value` is attention TFLOP/s over the whole step
(4*B*H*Nq*Nkv*d flops per attention call, divided by the step's wall time,
merges, splice and CFG included).  Per-phase times, the roofline of the
dominant kernel and the fp64 CPU oracle on a bounded sample ride along.

    python bench.py [--gpus 1] [--steps 200] [--warmup 200] [--no-cpu-baseline]

The shader clock needs about half a second of this load to settle at its
steady value; the supplementary workloads (merge and CFG on cold HBM, other
per-device shapes, d = 72 attention) run first, before the warm-up steps, so
the timed steps see the steady-state clock of a GPU under continuous load
(also with a short --warmup).  --no-supplementary skips them.

Phase figures time groups of back-to-back calls between two events, so no
event sits between two kernels of a group; measured peaks of the same GPU (a
matrix-core loop and a streaming copy, libdit_peaks.so) are reported beside
the published ones.
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % of bf16 MFMA peak; merge/CFG GB/s % of HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "attn_fwd_bf16_d128_video_patch_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "attention_attn_block_amd", "csrc", "attn_bf16_kernel.h")
PEAKS_LIB = os.path.join(ROOT, "attention_attn_block_amd", "libdit_peaks.so")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-supplementary", action="store_true")
    return ap.parse_args()


def attn_flops(B, H, Nq, Nkv, d):
    return 4.0 * B * H * Nq * Nkv * d


def kernel_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None if that summary was taken on other kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b:
        return None
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w_patch):
    """fp64 oracle on a bounded sample of the dominant phase: all 24 heads of
    the PipeFusion patch attention, 4096 query rows each, over the full
    32768-row buffer (the splice is a copy and is left out).  The oracle's
    BLAS runs on every core this process may use (its affinity set)."""
    import numpy as np
    import threadpoolctl

    import oracle
    from tests.gpu_util import to_oracle

    rows = np.arange(0, 8192, 2)
    q, kb, vb = to_oracle(w_patch["q_p"]), to_oracle(w_patch["k_buf"]), to_oracle(w_patch["v_buf"])
    B, H, _, d = q.shape
    N = kb.shape[2]
    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
        t0 = time.perf_counter()
        oracle.ref_attn(q, kb, vb, w_patch["scale"], rows=rows)
        dt = time.perf_counter() - t0
    flops = attn_flops(B, H, rows.size, N, d)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": int(threads), "cpu_model": cpu_model(),
            "sample": f"fp64 oracle attention (numpy, BLAS on {threads} threads), B{B} H{H}, "
                      f"{rows.size} of 8192 patch query rows against the full {N}-row buffer, "
                      f"d{d}: {flops / 1e9:.1f} GFLOP in {dt:.1f} s"}


def measured_peaks(torch, dev):
    """Peaks of this GPU measured by libdit_peaks.so: a bf16 matrix-core loop
    (no memory traffic; 2 workgroups of 8 waves per CU) and a streaming copy
    of 1 GiB (read + write counted).  Each is timed over back-to-back
    launches after a warm-up; None if the library is not built."""
    if not os.path.exists(PEAKS_LIB):
        return None
    L = ctypes.CDLL(PEAKS_LIB)
    L.dit_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.dit_peak_mfma_flops.restype = ctypes.c_double
    L.dit_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.dit_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs, iters = 2 * n_cu, 2000
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)

    def run_timed(fn, warm, reps):
        for _ in range(warm):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps   # s per launch

    def mfma():
        assert L.dit_peak_mfma_bf16(wgs, iters, ctypes.c_void_p(sink.data_ptr()), stream) == 0

    t_mfma = run_timed(mfma, 100, 100)
    flops = L.dit_peak_mfma_flops(wgs, iters)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    copy_gbs = {}
    for unroll in (1, 2, 4):
        def copy():
            assert L.dit_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   nbytes, unroll, stream) == 0
        copy_gbs[unroll] = 2 * nbytes / run_timed(copy, 5, 20) / 1e9
    del src, dst, sink
    return {"mfma_bf16_tflops": flops / t_mfma / 1e12, "hbm_copy_gbs": max(copy_gbs.values()),
            "hbm_copy_gbs_by_unroll": copy_gbs,
            "note": f"matrix-core loop: {wgs} workgroups x 8 waves x {4 * iters} rounds of 4 "
                    "independent 32x32x16 bf16 products, 100 launches after 100; copy: 1 GiB, "
                    "16-byte non-temporal, 1, 2 or 4 units per lane (best kept), read + write "
                    "bytes, 20 launches after 5 each"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    rank = int(os.environ.get("RANK", "0"))
    if args.gpus != 1 or world != 1:
        if rank == 0:
            print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
                  "(sharding across devices is described, not built). Use --gpus 1.",
                  file=sys.stderr)
        sys.exit(2)

    import torch

    from attention_attn_block_amd import (attn_block_fwd, attn_lse_merge, attn_patch_fwd,
                                          cfg_combine, inputs, load)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM -------------------------------------------------
    wr = inputs.ring_2048px()
    wp = inputs.video_patch()
    wc = inputs.dit_xl_256()
    q_r = wr["q"].to(dev)
    ks = [k.to(dev) for k in wr["ks"]]
    vs = [v.to(dev) for v in wr["vs"]]
    Br, Hr, Nqr, dr = q_r.shape
    Nkr = ks[0].shape[2]
    o_acc = torch.empty((Br, Hr, Nqr, dr), dtype=torch.float32, device=dev)
    l_acc = torch.empty((Br, Hr, Nqr), dtype=torch.float32, device=dev)
    o_cur, l_cur = torch.empty_like(o_acc), torch.empty_like(l_acc)
    q_p, k_p, v_p = (wp[n].to(dev) for n in ("q_p", "k_p", "v_p"))
    k_buf, v_buf = wp["k_buf"].to(dev), wp["v_buf"].to(dev)
    p0 = wp["p0"]
    Bp, Hp, Np, dp = q_p.shape
    Nb = k_buf.shape[2]
    o_p = torch.empty((Bp, Hp, Np, dp), dtype=torch.bfloat16, device=dev)
    l_p = torch.empty((Bp, Hp, Np), dtype=torch.float32, device=dev)
    eps_u, eps_c = wc["eps_u"].to(dev), wc["eps_c"].to(dev)
    eps_out = torch.empty_like(eps_u)
    s_cfg = wc["s"]
    nblk = len(ks)

    f_ring = nblk * attn_flops(Br, Hr, Nqr, Nkr, dr)
    f_patch = attn_flops(Bp, Hp, Np, Nb, dp)
    f_step = f_ring + f_patch
    merge_bytes = 3 * o_acc.numel() * 4 + 3 * l_acc.numel() * 4     # read a, b; write a
    splice_bytes = 2 * 2 * k_p.numel() * 2                           # K and V, read + write
    cfg_bytes = 3 * eps_u.numel() * 4

    n_ev = 2 * nblk + 2 * (nblk - 1) + 4

    def step(ev=None, patch_ev=None):
        """One step.  `ev` (n_ev events) brackets every call, for the phase
        breakdown; `patch_ev` (2 events) brackets only the patch call, for the
        roofline.  The timed steps carry patch_ev only: an event between every
        pair of kernels costs about 4% of the step."""
        i = 0

        def rec():
            nonlocal i
            if ev is not None:
                ev[i].record()
                i += 1

        for j in range(nblk):
            tgt_o, tgt_l = (o_acc, l_acc) if j == 0 else (o_cur, l_cur)
            rec()
            attn_block_fwd(q_r, ks[j], vs[j], scale=wr["scale"], out_dtype=torch.float32,
                           out=tgt_o, lse=tgt_l)
            rec()
            if j:
                rec()
                attn_lse_merge(o_acc, l_acc, o_cur, l_cur)
                rec()
        rec()
        if patch_ev is not None:
            patch_ev[0].record()
        attn_patch_fwd(q_p, k_p, v_p, k_buf, v_buf, p0, scale=wp["scale"], out=o_p, lse=l_p)
        if patch_ev is not None:
            patch_ev[1].record()
        rec()
        rec()
        cfg_combine(eps_u, eps_c, s_cfg, out=eps_out)
        rec()

    # ---- supplementary and measured peaks, before the warm-up (they also bring
    # the shader clock to its steady state under load) ------------------------------
    supp, peaks = {}, None
    if not args.no_supplementary:
        peaks = measured_peaks(torch, dev)
        supp = supplementary(torch, dev, inputs, q_r, ks, vs, wr["scale"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region ------------------------------------------------------------
    pevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for k in range(args.steps):
        step(patch_ev=pevs[k])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    patch_ms = [a.elapsed_time(b) for a, b in pevs]

    # ---- phase breakdown, after the timed region ---------------------------------
    # The ring share again with each block's partial in a buffer of its own: the
    # 8 block calls run back to back between two events, then the 7 merges
    # (folding blocks 1..7 into block 0's partial, in order) between two more,
    # so no event sits between two kernels of a group.  The per-call event
    # figures of the in-sequence step are kept for comparison (an event pair
    # around each ~14 us merge adds its own overhead).
    n_phase = 10
    parts = [(torch.empty_like(o_acc), torch.empty_like(l_acc)) for _ in range(nblk)]
    grp = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_phase)]
    cfg_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_phase)]
    for k in range(n_phase):
        grp[k][0].record()
        for j in range(nblk):
            attn_block_fwd(q_r, ks[j], vs[j], scale=wr["scale"], out_dtype=torch.float32,
                           out=parts[j][0], lse=parts[j][1])
        grp[k][1].record()
        grp[k][2].record()
        for j in range(1, nblk):
            attn_lse_merge(parts[0][0], parts[0][1], parts[j][0], parts[j][1])
        grp[k][3].record()
        cfg_ev[k][0].record()
        for _ in range(10):
            cfg_combine(eps_u, eps_c, s_cfg, out=eps_out)
        cfg_ev[k][1].record()
    torch.cuda.synchronize()
    ring_ms = [e[0].elapsed_time(e[1]) / nblk for e in grp]
    merge_ms = [e[2].elapsed_time(e[3]) / (nblk - 1) for e in grp]
    cfg_ms = [e[0].elapsed_time(e[1]) / 10 for e in cfg_ev]
    del parts
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n_phase)]
    for k in range(n_phase):
        step(evs[k])
    torch.cuda.synchronize()
    merge_seq_ms = []
    for ev in evs:
        i = 0
        for j in range(nblk):
            i += 2
            if j:
                merge_seq_ms.append(ev[i].elapsed_time(ev[i + 1]))
                i += 2

    def mean(x):
        return sum(x) / len(x)

    ring_us, merge_us, patch_us, cfg_us, merge_seq_us = (
        1e3 * mean(x) for x in (ring_ms, merge_ms, patch_ms, cfg_ms, merge_seq_ms))
    f_block = attn_flops(Br, Hr, Nqr, Nkr, dr)
    patch_tflops = f_patch / (patch_us * 1e-6) / 1e12
    phases = {
        "note": f"means over {n_phase} repetitions after the timed region; ring blocks, merges "
                "and CFG each timed as a group of back-to-back calls between two events",
        "ring_block_attn": {"us_per_call": ring_us, "calls_per_step": nblk,
                            "tflops": f_block / (ring_us * 1e-6) / 1e12,
                            "frac_bf16_peak": f_block / (ring_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                            "note": "8 block calls back to back, fp32 partials"},
        "lse_merge": {"us_per_call": merge_us, "calls_per_step": nblk - 1,
                      "gbs": merge_bytes / (merge_us * 1e-6) / 1e9,
                      "frac_hbm_peak": merge_bytes / (merge_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                      "note": "7 merges back to back, folding the 8 block partials in order"},
        "lse_merge_in_sequence_events": {
            "us_per_call": merge_seq_us, "gbs": merge_bytes / (merge_seq_us * 1e-6) / 1e9,
            "frac_hbm_peak": merge_bytes / (merge_seq_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "note": "each merge of the step bracketed by its own event pair (O_b just written "
                    "by the block call); includes the events' own overhead"},
        "patch_splice_plus_attn": {"us_per_call": patch_us, "tflops": patch_tflops,
                                   "frac_bf16_peak": patch_tflops / PEAK_BF16_TFLOPS,
                                   "note": "events around this call in every timed step"},
        "cfg_combine": {"us_per_call": cfg_us, "gbs": cfg_bytes / (cfg_us * 1e-6) / 1e9,
                        "note": "96 KiB working set, 10 calls back to back: launch-latency bound"},
    }

    roofline = {"bound": "mfma", "achieved": patch_tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": patch_tflops / PEAK_BF16_TFLOPS,
                "traffic": kernel_traffic(),
                "kernel": "attn_fwd_bf16_kernel<128, bf16 out> in attn_patch_fwd "
                          "(8192 queries x 32768 keys x 24 heads; timed with the splice "
                          "that precedes it in the same call)"}
    if peaks:
        roofline["measured_peak"] = peaks["mfma_bf16_tflops"]
        roofline["frac_of_measured_peak"] = patch_tflops / peaks["mfma_bf16_tflops"]
        for name, unit in (("ring_block_attn", "tflops"), ("lse_merge", "gbs"),
                           ("lse_merge_in_sequence_events", "gbs"), ("patch_splice_plus_attn", "tflops")):
            peak = peaks["mfma_bf16_tflops"] if unit == "tflops" else peaks["hbm_copy_gbs"]
            phases[name]["frac_of_measured_peak"] = phases[name][unit] / peak

    value = f_step / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dit_device_step: ring share B1 H24 d128 2048q x 8x2048kv "
                               "(8 block fwd fp32 partials + 7 LSE merges) + PipeFusion share "
                               "B1 H24 d128 8192 patch q x 32768-row fresh/stale KV buffer "
                               "(splice + attention) + CFG combine 2x4x32x32 fp32 s=4",
                   "attn_flops_per_step": f_step, "frac_bf16_peak": value / PEAK_BF16_TFLOPS},
        "roofline": roofline,
        "phases": phases,
        "measured_peaks": peaks,
        "supplementary": supp,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wp)
    print(json.dumps(out), flush=True)


def supplementary(torch, dev, inputs, q_r, ks, vs, ring_scale):
    """Reported beside the step: merge and CFG on cold HBM (rotating buffers
    larger than the 256 MB Infinity Cache), the fused ring step, the ring
    share in one launch over its resident blocks, a long block with few query
    tiles (plain grid vs split launch), the Ulysses and P = 8 PipeFusion
    shares, and the d=72 workloads."""
    from attention_attn_block_amd import (attn_block_fwd, attn_block_fwd_merge, attn_block_workspace,
                                          attn_lse_merge, attn_patch_fwd, attn_ring_fwd,
                                          cfg_combine, cfg_combine_relmae)
    res = {}

    def timed(fn, iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(iters):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters   # us

    # LSE merge, ring-share shape (49152 rows x d128 fp32), 8 rotating sets (608 MB).
    rows, d = 24 * 2048, 128
    sets = [(torch.randn(rows, d, device=dev), torch.randn(rows, device=dev),
             torch.randn(rows, d, device=dev), torch.randn(rows, device=dev)) for _ in range(8)]
    fn = lambda i: attn_lse_merge(*sets[i % 8])
    for i in range(8):
        fn(i)
    us = timed(fn, 64)
    nbytes = 3 * rows * d * 4 + 3 * rows * 4
    res["lse_merge_cold_d128_f32"] = {"us": us, "gbs": nbytes / us / 1e3,
                                      "frac_hbm_peak": nbytes / us / 1e3 / PEAK_HBM_GBS,
                                      "bytes": nbytes}
    del sets

    # CFG combine (and with the rel-MAE signal) at 2^26 floats per tensor (768 MB per call).
    n = 1 << 26
    u, c, o = (torch.randn(n, device=dev) for _ in range(3))
    ws = torch.empty(1 << 16, device=dev)
    rm = torch.empty(4, device=dev)[:1]
    for name, fn in (("cfg_combine_2^26", lambda i: cfg_combine(u, c, 4.0, out=o)),
                     ("cfg_combine_relmae_2^26",
                      lambda i: cfg_combine_relmae(u, c, 4.0, out=o, workspace=ws, relmae=rm))):
        fn(0)
        us = timed(fn, 20)
        nbytes = 3 * n * 4
        res[name] = {"us": us, "gbs": nbytes / us / 1e3, "frac_hbm_peak": nbytes / us / 1e3 / PEAK_HBM_GBS}
    del u, c, o

    # Ring share with the merge fused into the attention epilogue.
    B, H, Nq, dd = q_r.shape
    o_acc = torch.empty((B, H, Nq, dd), dtype=torch.float32, device=dev)
    l_acc = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)

    def ring_fused(i):
        l_acc.fill_(-float("inf"))
        for kj, vj in zip(ks, vs):
            attn_block_fwd_merge(q_r, kj, vj, o_acc, l_acc, scale=ring_scale)

    ring_fused(0)
    us = timed(ring_fused, 20)
    f = len(ks) * attn_flops(B, H, Nq, ks[0].shape[2], dd)
    res["ring_share_fused_merge"] = {"us_per_share": us, "tflops": f / (us * 1e-6) / 1e12,
                                     "frac_bf16_peak": f / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}

    # The whole ring share in one launch over the 8 resident blocks
    # (attn_ring_fwd): plain grid, and the library's choice with a workspace
    # (256 key tiles per query tile: split).
    wsr = attn_block_workspace(q_r, ks[0])
    row = {}
    for tag, kw in (("plain", {}), ("split", {"workspace": wsr})):
        fn = lambda i: attn_ring_fwd(q_r, ks, vs, scale=ring_scale, out=o_acc, lse=l_acc,
                                     out_dtype=torch.float32, **kw)
        for i in range(10):
            fn(i)
        us = timed(fn, 20)
        row[f"{tag}_us_per_share"] = us
        row[f"{tag}_tflops"] = f / (us * 1e-6) / 1e12
        row[f"{tag}_frac_bf16_peak"] = f / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
    res["ring_share_one_launch"] = row
    del wsr

    # Few query tiles against a long block: 20 heads x 2048 queries (160 tiles
    # of 256 rows on 256 CUs) x 16384 keys, plain grid vs the split launch
    # (attn_block_fwd_ws), which shares the tiles' keys over every CU.
    g = torch.Generator(device=dev).manual_seed(7)
    shp = (1, 20, 2048, 16384, 128)
    q = torch.randn(shp[0], shp[1], shp[2], shp[4], device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn(shp[0], shp[1], shp[3], shp[4], device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn(shp[0], shp[1], shp[3], shp[4], device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    wsp = attn_block_workspace(q, k)
    f = attn_flops(shp[0], shp[1], shp[2], shp[3], shp[4])
    row = {"shape_b_h_nq_nkv_d": list(shp)}
    for tag, kw in (("plain", {}), ("split", {"workspace": wsp})):
        fn = lambda i: attn_block_fwd(q, k, v, out=out, lse=lse, out_dtype=torch.float32, **kw)
        for i in range(10):
            fn(i)
        us = timed(fn, 20)
        row[f"{tag}_us"] = us
        row[f"{tag}_tflops"] = f / (us * 1e-6) / 1e12
    res["long_block_160_tiles"] = row
    del q, k, v, out, lse, wsp

    # Ulysses share of the video workload on 8 devices: H/8 = 3 heads against
    # the full 32768-token sequence (384 query tiles: 1.5 waves of workgroups
    # on 256 CUs), bf16 out, plain grid vs split launch.
    shp = (1, 3, 32768, 32768, 128)
    q = torch.randn(shp[0], shp[1], shp[2], shp[4], device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn(shp[0], shp[1], shp[3], shp[4], device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn(shp[0], shp[1], shp[3], shp[4], device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    wsp = attn_block_workspace(q, k)
    f = attn_flops(shp[0], shp[1], shp[2], shp[3], shp[4])
    row = {"shape_b_h_nq_nkv_d": list(shp)}
    for tag, kw in (("plain", {}), ("split", {"workspace": wsp})):
        fn = lambda i: attn_block_fwd(q, k, v, out=out, lse=lse, **kw)
        for i in range(5):
            fn(i)
        us = timed(fn, 10)
        row[f"{tag}_us"] = us
        row[f"{tag}_tflops"] = f / (us * 1e-6) / 1e12
    res["ulysses_share_video_p8"] = row
    del q, k, v, out, lse, wsp

    # PipeFusion on 8 devices over the same 32768-token sequence: a 4096-query
    # patch (24 heads: 384 query tiles, 1.5 waves) spliced at p0 = 8192 and
    # attended to the whole buffer, plain grid vs split launch.
    vp_ = inputs.video_patch(Np=4096)
    q_p, k_p, v_p = (vp_[n].to(dev) for n in ("q_p", "k_p", "v_p"))
    k_buf, v_buf = vp_["k_buf"].to(dev), vp_["v_buf"].to(dev)
    out = torch.empty_like(q_p)
    lse = torch.empty(q_p.shape[:3], dtype=torch.float32, device=dev)
    wsp = attn_block_workspace(q_p, k_buf)
    B, H, Np, dd = q_p.shape
    f = attn_flops(B, H, Np, k_buf.shape[2], dd)
    row = {"shape_b_h_np_n_d": [B, H, Np, k_buf.shape[2], dd], "p0": vp_["p0"]}
    for tag, kw in (("plain", {}), ("split", {"workspace": wsp})):
        fn = lambda i: attn_patch_fwd(q_p, k_p, v_p, k_buf, v_buf, vp_["p0"], scale=vp_["scale"],
                                      out=out, lse=lse, **kw)
        for i in range(5):
            fn(i)
        us = timed(fn, 10)
        row[f"{tag}_us"] = us
        row[f"{tag}_tflops"] = f / (us * 1e-6) / 1e12
    res["pipefusion_patch_video_p8"] = row
    del q_p, k_p, v_p, k_buf, v_buf, out, lse, wsp, vp_

    # d = 72 attention: PixArt-style 1024 px and DiT-XL/2 256 px.
    for name in ("pixart_1024", "dit_xl_256"):
        w = inputs.make(name)
        q, k, v = (w[x].to(dev) for x in ("q", "k", "v"))
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda i: attn_block_fwd(q, k, v, scale=w["scale"], out=out, lse=lse)
        for i in range(300):   # short calls: let the clock settle after the memory-bound runs
            fn(i)
        us = timed(fn, 20)
        B, H, Nq, dd = q.shape
        tf = attn_flops(B, H, Nq, k.shape[2], dd) / (us * 1e-6) / 1e12
        res[f"attn_{name}"] = {"us": us, "tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS}
    return res


if __name__ == "__main__":
    main()
