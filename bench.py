#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the prefill path over one batch: the block mask from
the block scores (top-k or threshold), then the block-sparse forward pass
(its per-row compaction runs inside the forward kernel).  The default
workload is the largest prefill configuration, B4 H32 S8192 D128 with a
top-32 mask of N(0,1) block scores, last two block rows dense, tril,
diagonal forced, causal.

Printed (one JSON line):
* value      — active-block TFLOP/s of the whole step (mask build + forward):
               sum over active blocks of 4*64*64*D flop, divided by the
               measured time per step;
* roofline   — the forward kernel alone against the bf16 dense MFMA peak, its
               time taken per launch with HIP events on the launch stream;
               also the same launch with the 256 MiB last-level cache evicted
               before every call;
* fused_step_ms — the same step as one launch (bsattn_fwd_topk: row
               selection inside the forward kernel), for comparison;
* prefill_other — the other prefill workloads (B2 H16 S4096 D64 top-16, and
               B1 H32 S16384 D128 threshold with long-row split), measured
               the same way;
* decode     — split-KV sparse GQA decode (batch 8, 32 query heads over 8 KV
               heads, D 128, KV lengths U[4096, 32768], up to 64 selected
               blocks): algorithmic HBM bytes per call over its time, with the
               256 MiB last-level cache flushed before every timed call by
               reading a 512 MiB buffer (a read leaves no dirty lines whose
               write-back would land inside the timed call);
* next_rows  — the mask-form and paged-KV variants of that decode (same
               workload and flush), a chunked prefill (the last 1024 of a
               4096-token context), and the XAttention block estimate that
               produces a mask upstream (B1 H32 S16384 D128, stride 8), each
               against its roofline;
* cpu_baseline — the float64 CPU oracle timed on a bounded sample of the
               headline workload on this host (whole (batch, head) slices,
               one slice per worker thread), with the GPU output's error on
               those slices; host CPU model and core count.

Inputs are synthetic (seeded generator) and resident in HBM before timing.
Before its warm-up steps each leg runs its step untimed for half a second, so
that the clocks have left the idle state the input generation leaves them in.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz (published ~2.5 PFLOP/s dense)
HBM_PEAK_GBPS = 8000.0        # 8 TB/s HBM3E
FLOP_PER_BLOCK = lambda D: 4 * 64 * 64 * D   # QK^T and PV on one 64x64 block pair

PROFILE_DIR = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "block_sparse_attention_amd", "csrc")
# the sources a kernel's counters depend on (the forward's issue order lives in a header)
KERNEL_SRC = {
    "prefill": [os.path.join(_CSRC, "prefill.hip"), os.path.join(_CSRC, "item_order.hpp")],
    "decode": [os.path.join(_CSRC, "decode.hip")],
    "xattn": [os.path.join(_CSRC, "xattn.hip")],
}


def _sha(paths) -> str:
    """sha256 of one source, or of several sources' bytes one after another."""
    h = hashlib.sha256()
    for p in ([paths] if isinstance(paths, str) else paths):
        h.update(open(p, "rb").read())
    return h.hexdigest()


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    p = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha256") != _sha(KERNEL_SRC[kernel]):
        return None
    return d.get("traffic_bytes_per_launch")


def _torch():
    import torch
    return torch


def _progress(msg: str) -> None:
    """One line on stderr as each leg finishes (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _gpu_bf16(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _flush_buffer():
    """512 MiB of device memory whose read evicts the 256 MiB last-level cache."""
    torch = _torch()
    flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    return lambda: torch.sum(flush, dim=0, keepdim=True, out=sink)


def _per_call_ms(fn, n, before=None):
    """Average and median ms of n calls of fn, each bracketed by its own HIP
    events on the launch stream; `before` (untimed) runs ahead of each call."""
    torch = _torch()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()   # no collector pause between a call's start event and its launch
    try:
        for a, b in ev:
            if before is not None:
                before()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    ms = [a.elapsed_time(b) for a, b in ev]
    return sum(ms) / len(ms), statistics.median(ms)


def bench_prefill(cfg_name: str, steps: int, warmup: int, flush=None, fused=True):
    torch = _torch()
    import block_sparse_attention_amd as bsa
    from block_sparse_attention_amd import inputs as gen

    cfg = gen.CONFIGS[cfg_name]
    inp = gen.prefill_inputs(cfg, 0)
    scores = torch.from_numpy(inp["scores"]).to("cuda")
    q, k, v = (_gpu_bf16(inp[n]) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    mask = torch.empty((cfg.B, cfg.H, cfg.nb, cfg.nb), dtype=torch.uint8, device="cuda")
    # the long-row split's workspace (zero bytes up to 128 key blocks), allocated once
    ws_bytes = bsa.bsattn_fwd_workspace_bytes(cfg.B, cfg.H, cfg.S, cfg.D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None

    def build_mask():
        if cfg.mask_kind == "topk":
            bsa.bsattn_build_mask_topk(scores, cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal, out=mask)
        else:
            bsa.bsattn_build_mask_threshold(scores, cfg.threshold, cfg.dense_last_two_rows,
                                            cfg.force_diagonal, out=mask)

    build_mask()
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    nb = cfg.nb
    active = int(np.tril(m != 0).sum()) if cfg.is_causal else int((m != 0).sum())
    causal_blocks = cfg.B * cfg.H * nb * (nb + 1) // 2
    diag_blocks = int(np.diagonal(m != 0, axis1=2, axis2=3).sum())
    flops = active * FLOP_PER_BLOCK(cfg.D)
    useful = (active - diag_blocks) * FLOP_PER_BLOCK(cfg.D) + diag_blocks * FLOP_PER_BLOCK(cfg.D) * 2080 / 4096

    stream = torch.cuda.current_stream()

    def timed(fn, n):
        """Average ms per call of n back-to-back calls, HIP events on the launch stream."""
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def fwd():
        bsa.bsattn_fwd(q, k, v, mask, cfg.is_causal, out=out, workspace=ws)

    def step():
        # the whole hot path: the block mask from the scores, then the forward
        # pass on it (per-row compaction inside the forward kernel)
        build_mask()
        fwd()

    def step_fused():
        # the same path in one launch: row selection, compaction and forward
        if cfg.mask_kind == "topk":
            bsa.bsattn_fwd_topk(q, k, v, scores, cfg.topk, cfg.dense_last_two_rows,
                                cfg.force_diagonal, cfg.is_causal, out=out, mask_out=mask,
                                workspace=ws)
        else:
            bsa.bsattn_fwd_threshold(q, k, v, scores, cfg.threshold, cfg.dense_last_two_rows,
                                     cfg.force_diagonal, cfg.is_causal, out=out, mask_out=mask,
                                     workspace=ws)

    _settle(step)
    for _ in range(warmup):
        step()
    # the timed region: `steps` whole steps
    wall0 = time.perf_counter()
    ms_per_step = timed(step, steps)
    wall = time.perf_counter() - wall0
    # the forward kernel alone and the mask build alone, back to back, for the
    # roofline; and the one-launch form of the same step
    fwd_avg = timed(fwd, steps)
    mask_avg = timed(build_mask, steps)
    fused_ms = timed(step_fused, steps) if fused else None
    # the forward with the last-level cache evicted before every call
    flushed = _per_call_ms(fwd, max(10, min(steps, 50)), before=flush) if flush else None
    # leave the two-launch path's output in `out` for the parity sample
    step()
    torch.cuda.synchronize()
    return {
        "cfg": cfg, "active": active, "density": active / causal_blocks, "flops": flops,
        "useful_flops": useful, "ms_per_step": ms_per_step, "wall_s": wall,
        "fused_ms": fused_ms, "fwd_ms_avg": fwd_avg, "mask_ms_avg": mask_avg,
        "fwd_ms_flushed": flushed, "inputs": inp, "mask": m, "out": out,
    }


def _settle(fn, seconds: float = 0.5):
    """Run fn back to back, untimed, for about `seconds` of wall time."""
    torch = _torch()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def _selected_tokens(d, cfg):
    lens = d["lens"]
    sel = 0
    for b in range(cfg.B):
        nbb = -(-int(lens[b]) // 64)
        for h in range(cfg.Hkv):
            for i in d["block_indices"][b, h]:
                if 0 <= i < nbb:
                    sel += min(64, int(lens[b]) - 64 * int(i))
    return sel


def bench_decode(steps: int, warmup: int, form: str = "indices", base=None, page_size: int = 256):
    """Per-call time of one sparse GQA decode call on C5, in the index form
    (packed KV), the mask form, or over a paged KV cache (pages of page_size)."""
    torch = _torch()
    import block_sparse_attention_amd as bsa
    from block_sparse_attention_amd import inputs as gen

    cfg = gen.CONFIGS["C5"]
    d = base if base is not None else gen.decode_inputs(cfg, 0)
    q = _gpu_bf16(d["q"])
    out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=torch.bfloat16, device="cuda")
    sel_tokens = _selected_tokens(d, cfg)
    meta = 0
    if form == "indices":
        k, v = _gpu_bf16(d["k"]), _gpu_bf16(d["v"])
        cu = torch.from_numpy(d["cu_seqlens_k"]).to("cuda")
        idx = torch.from_numpy(d["block_indices"]).to("cuda")
        slots = idx.shape[2]
        meta = idx.numel() * 4 + cu.numel() * 4
        call_args = lambda ns, ws: bsa.bsattn_decode_gqa(q, k, v, cu, idx, num_splits=ns, out=out, workspace=ws)
    elif form == "mask":
        dm = gen.decode_mask_inputs(cfg, 0, base=d)
        k, v = _gpu_bf16(d["k"]), _gpu_bf16(d["v"])
        cu = torch.from_numpy(d["cu_seqlens_k"]).to("cuda")
        bm = torch.from_numpy(dm["block_mask"]).to("cuda")
        slots = bm.shape[2]
        meta = bm.numel() + cu.numel() * 4
        call_args = lambda ns, ws: bsa.bsattn_decode_gqa_mask(q, k, v, cu, bm, num_splits=ns, out=out, workspace=ws)
    else:
        dp = gen.decode_paged_inputs(cfg, 0, page_size=page_size, base=d)
        k, v = _gpu_bf16(dp["k_cache"]), _gpu_bf16(dp["v_cache"])
        sl = torch.from_numpy(dp["cache_seqlens"]).to("cuda")
        tab = torch.from_numpy(dp["block_table"]).to("cuda")
        idx = torch.from_numpy(d["block_indices"]).to("cuda")
        slots = idx.shape[2]
        nsel = int((d["block_indices"] >= 0).sum())
        meta = idx.numel() * 4 + nsel * 4 + sl.numel() * 4
        call_args = lambda ns, ws: bsa.bsattn_decode_gqa_paged(q, k, v, sl, tab, idx, num_splits=ns,
                                                               out=out, workspace=ws)
    ns = bsa.bsattn_decode_default_splits(cfg.B, cfg.Hq, cfg.Hkv, slots, cfg.D)
    ws_bytes = bsa.bsattn_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.D, ns)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    flush = _flush_buffer()

    # algorithmic bytes: selected K and V tokens, q, out, and the selection metadata
    algo_bytes = sel_tokens * 2 * cfg.D * 2 + q.numel() * 2 + out.numel() * 2 + meta

    def call():
        call_args(ns, ws)

    _settle(call)
    for _ in range(warmup):
        call()
    # each timed call follows a read-only pass that evicts the selected K/V
    # from the last-level cache
    avg, med = _per_call_ms(call, steps, before=flush)
    # the time a call adds to a stream of work: (eviction + call) x n minus
    # eviction x n, each timed as one block; the call's dispatch then
    # overlaps the preceding kernel, as it would behind other work
    stream = torch.cuda.current_stream()

    def block(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def both():
        flush()
        call()

    t_both = min(block(both, steps) for _ in range(3))
    t_flush = min(block(flush, steps) for _ in range(3))
    incr = (t_both - t_flush) / steps
    return {"cfg": cfg, "ns": ns, "algo_bytes": algo_bytes, "sel_tokens": sel_tokens,
            "ms_avg": avg, "ms_median": med, "ms_incremental": incr, "inputs": d, "out": out}


def bench_read_ceiling(nbytes: int, steps: int):
    """A plain streaming read of nbytes, timed per call after the same cache
    eviction as the decode: what one read of the decode's byte count reaches
    on this device.  Two forms of the read (a sum over the whole buffer, and a
    sum of each 16 KiB row of it); the faster one is the ceiling."""
    torch = _torch()
    row = 4096
    n = max(row, nbytes // 4 // row * row)
    buf = torch.ones(n, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    rows = torch.zeros(n // row, dtype=torch.float32, device="cuda")
    flush = _flush_buffer()
    forms = {
        "sum": lambda: torch.sum(buf, dim=0, keepdim=True, out=sink),
        "row_sums": lambda: torch.sum(buf.view(-1, row), dim=1, out=rows),
    }
    res = {}
    for name, call in forms.items():
        _settle(call, 0.2)
        avg, med = _per_call_ms(call, steps, before=flush)
        res[name] = {"ms_avg": avg, "GBps": n * 4 / (avg * 1e-3) / 1e9}
    best = max(res, key=lambda k: res[k]["GBps"])
    return {"bytes": n * 4, "ms_avg": res[best]["ms_avg"], "GBps": res[best]["GBps"],
            "form": best, "forms": {k: round(v["GBps"], 1) for k, v in res.items()}}


def bench_mfma_ceiling(steps: int = 20):
    """What bf16 matrix-core work reaches on this device in practice: torch's
    batched GEMM (the vendor BLAS) on contiguous bf16 operands, on the
    XAttention estimator's GEMM shape (32 heads of [2048 x 1024] x [1024 x 2048],
    every product computed) and on one large square product.  A reference
    beside the 2516.6 TFLOP/s nominal peak, not part of any timed step."""
    torch = _torch()
    gen = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for name, (bt, m, k, n) in {"estimator_shape": (32, 2048, 1024, 2048),
                                "square_8192": (1, 8192, 8192, 8192)}.items():
        x = torch.randn(bt, m, k, device="cuda", generator=gen).to(torch.bfloat16).contiguous()
        y = torch.randn(bt, k, n, device="cuda", generator=gen).to(torch.bfloat16).contiguous()
        o = torch.empty(bt, m, n, device="cuda", dtype=torch.bfloat16)

        def mm():
            torch.bmm(x, y, out=o)

        _settle(mm, 0.3)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            mm()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        tf = 2.0 * bt * m * k * n / (ms * 1e-3) / 1e12
        res[name] = {"shape": f"[{bt},{m},{k}] x [{bt},{k},{n}]", "ms": round(ms, 5),
                     "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        del x, y, o
    return res


def bench_launch_floor(steps: int):
    """The per-call timing method's own floor: one trivial kernel (a one-element
    fill) timed exactly as a decode call is, HIP events around it after the
    same cache-evicting read."""
    torch = _torch()
    t = torch.zeros(1, dtype=torch.float32, device="cuda")
    flush = _flush_buffer()
    call = lambda: t.fill_(1.0)
    _settle(call, 0.2)
    avg, med = _per_call_ms(call, steps, before=flush)
    return {"ms_avg": avg, "ms_median": med}


def bench_prefill_chunk(steps: int, warmup: int):
    """Chunked prefill: the last 1024 queries of C2's 4096-token context (Sq 1024,
    Sk 4096), C2's top-16/tril/diagonal mask rows for those query blocks."""
    torch = _torch()
    import block_sparse_attention_amd as bsa
    from block_sparse_attention_amd import inputs as gen

    cfg = gen.CONFIGS["C2"]
    Sq = 1024
    nbq = Sq // 64
    inp = gen.prefill_inputs(cfg, 0)
    # C2's mask from the library's own builder, then its last nbq block rows
    scores = torch.from_numpy(inp["scores"]).to("cuda")
    m_full = bsa.bsattn_build_mask_topk(scores, cfg.topk, cfg.dense_last_two_rows, cfg.force_diagonal)
    mt = m_full[:, :, cfg.nb - nbq:, :].contiguous()
    q = _gpu_bf16(np.ascontiguousarray(inp["q"][:, :, cfg.S - Sq:, :]))
    k, v = _gpu_bf16(inp["k"]), _gpu_bf16(inp["v"])
    out = torch.empty_like(q)
    active = int((mt != 0).sum().item())
    flops = active * FLOP_PER_BLOCK(cfg.D)

    def call():
        bsa.bsattn_fwd_chunk(q, k, v, mt, True, out=out)

    _settle(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"Sq": Sq, "Sk": cfg.S, "active": active, "flops": flops, "ms": ms, "cfg": cfg}


def bench_xattn(steps: int, warmup: int):
    """XAttention block estimate on C3's shape (B1 H32 S16384 D128, its seeded
    q and k), stride 8, threshold 0.9, sink and diagonal kept, causal."""
    torch = _torch()
    import block_sparse_attention_amd as bsa
    from block_sparse_attention_amd import inputs as gen

    cfg = gen.CONFIGS["C3"]
    qkv = gen.prefill_qkv(cfg, 0)
    q, k = _gpu_bf16(qkv["q"]), _gpu_bf16(qkv["k"])
    B, H, S, D = cfg.B, cfg.H, cfg.S, cfg.D
    stride, thr = 8, 0.9
    nb = cfg.nb
    sums = torch.empty((B, H, nb, nb), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, H, nb, nb), dtype=torch.uint8, device="cuda")
    ws = torch.empty(bsa.bsattn_xattn_workspace_bytes(B, H, S, S, stride), dtype=torch.uint8,
                     device="cuda")
    rows = S // stride
    # reshaped GEMM flops over the causally visible reshaped pairs: 2 * (stride * D) each
    flops = B * H * rows * (rows + 1) // 2 * 2 * stride * D

    def est():
        bsa.bsattn_xattn_estimate(q, k, stride, 1.0, thr, True, True, True, block_sums=sums,
                                  out=mask, workspace=ws)

    def timed(fn, n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    _settle(est)
    for _ in range(warmup):
        est()
    ms = timed(est, steps)
    ms_sums = timed(lambda: bsa.bsattn_xattn_block_sums(q, k, stride, 1.0, True, out=sums,
                                                        workspace=ws), steps)
    ms_sel = timed(lambda: bsa.bsattn_build_mask_cumulative(sums, thr, True, True, True, out=mask),
                   steps)
    density = float(mask.float().sum().item()) / (B * H * nb * (nb + 1) / 2)
    return {"flops": flops, "ms": ms, "ms_sums": ms_sums, "ms_select": ms_sel,
            "density": density, "cfg": cfg, "stride": stride, "threshold": thr}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def _host():
    """CPU model and the number of cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline_prefill(res, budget_s: float):
    """Time the oracle (as it stands) on whole (batch, head) slices of the
    workload until the budget is spent, one slice per worker thread (BLAS
    single-threaded in each, numpy releases the GIL in its array loops), and
    compare the GPU output of those slices with it.  Reports active-block
    TFLOP/s of that sample and the sample's parity errors."""
    import concurrent.futures as cf

    from block_sparse_attention_amd import inputs as gen
    from oracle import attention as oa

    cfg = res["cfg"]
    inp, m = res["inputs"], res["mask"]
    model, host_cores = _host()
    workers = max(1, min(host_cores, 16))
    got = res["out"]
    slices = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]

    def one(bh):
        b, h = bh
        q, k, v = (gen.bf16_bits_to_f64(inp[n][b, h]) for n in ("q", "k", "v"))
        return bh, oa.prefill(q[None, None], k[None, None], v[None, None], m[b:b + 1, h:h + 1],
                              cfg.is_causal)[0, 0]

    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:
        limit = None
    done, done_blocks, max_err, sum_err, n_el = [], 0, 0.0, 0.0, 0
    t0 = time.perf_counter()
    try:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            for w0 in range(0, len(slices), workers):
                for (b, h), want in ex.map(one, slices[w0:w0 + workers]):
                    done.append((b, h))
                    done_blocks += int(np.tril(m[b, h] != 0).sum() if cfg.is_causal else (m[b, h] != 0).sum())
                    g = got[b, h].float().cpu().numpy().astype(np.float64)
                    err = np.abs(g - want)
                    max_err = max(max_err, float(err.max()))
                    sum_err += float(err.sum())
                    n_el += err.size
                if time.perf_counter() - t0 >= budget_s:
                    break
    finally:
        if limit is not None:
            limit.unregister() if hasattr(limit, "unregister") else None
    el = time.perf_counter() - t0
    tflops = done_blocks * FLOP_PER_BLOCK(cfg.D) / el / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(done)} of {len(slices)} (batch, head) slices of {cfg.name}, all rows, "
                      f"{done_blocks} active blocks, {el:.1f} s on {workers} worker threads "
                      f"(one slice each, BLAS single-threaded)",
            "host_cpu": model, "host_cores": host_cores,
            "parity_on_sample": {"max_abs": max_err, "mean_abs": sum_err / max(n_el, 1),
                                 "tolerance": {"max_abs": 1e-2, "mean_abs": 1e-3}},
            "seconds": el}


def cpu_baseline_decode(res):
    from block_sparse_attention_amd import inputs as gen
    from oracle import attention as oa
    d = res["inputs"]
    x = {n: gen.bf16_bits_to_f64(d[n]) for n in ("q", "k", "v")}
    t0 = time.perf_counter()
    want = oa.decode_gqa(x["q"], x["k"], x["v"], d["cu_seqlens_k"], d["block_indices"])
    el = time.perf_counter() - t0
    got = res["out"].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    return {"value": res["algo_bytes"] / el / 1e9, "unit": "GB/s", "cores": _blas_threads(),
            "kind": "oracle", "sample": f"whole workload, {el:.2f} s",
            "parity": {"max_abs": float(err.max()), "mean_abs": float(err.mean())}}


def _prefill_entry(res, with_fused=True):
    """The per-workload prefill numbers (step, forward, flushed forward)."""
    cfg = res["cfg"]
    fl = res["flops"]
    e = {
        "workload": _workload_name(cfg),
        "active_blocks": res["active"], "causal_density": round(res["density"], 4),
        "flop_per_launch": fl,
        "ms_per_step": round(res["ms_per_step"], 5),
        "step_tflops": round(fl / (res["ms_per_step"] * 1e-3) / 1e12, 3),
        "fwd_ms_avg": round(res["fwd_ms_avg"], 5),
        "fwd_tflops": round(fl / (res["fwd_ms_avg"] * 1e-3) / 1e12, 3),
        "fwd_frac": round(fl / (res["fwd_ms_avg"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "mask_build_ms_avg": round(res["mask_ms_avg"], 5),
    }
    if res.get("fwd_ms_flushed"):
        avg, med = res["fwd_ms_flushed"]
        e["fwd_ms_cache_evicted"] = round(avg, 5)
        e["fwd_frac_cache_evicted"] = round(fl / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    if with_fused and res.get("fused_ms"):
        e["fused_step_ms"] = round(res["fused_ms"], 5)
    return e


def _workload_name(cfg):
    return (f"{cfg.name} block-sparse prefill: B{cfg.B} H{cfg.H} S{cfg.S} D{cfg.D}, "
            + (f"top-{cfg.topk}" if cfg.mask_kind == "topk" else f"scores > {cfg.threshold}")
            + (", last two rows dense" if cfg.dense_last_two_rows else "")
            + ", tril, diagonal forced, causal; step = mask build + forward")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C4", choices=["C1", "C2", "C3", "C4", "P1"],
                    help="prefill workload of the step (default: the largest, B4 H32 S8192 D128 top-32)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other prefill workloads (C2, C3, C4 besides --config)")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg (profiling runs)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the mask-form / paged decode and chunked-prefill measurements")
    ap.add_argument("--xattn-only", action="store_true",
                    help="only run the XAttention estimate leg (profiling runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 10 times (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(sharding over several GPUs is described, not implemented)", file=sys.stderr)
        return 2

    torch = _torch()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    import block_sparse_attention_amd as bsa
    bsa.load_library()

    if args.copy_mib:
        n = args.copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "launches": 10}), flush=True)
        return 0

    if args.xattn_only:
        xr = bench_xattn(max(10, args.steps // 20), 3)
        print(json.dumps({"xattn_ms": xr["ms"], "block_sums_ms": xr["ms_sums"],
                          "selection_ms": xr["ms_select"]}), flush=True)
        return 0

    if args.no_prefill:
        dres = bench_decode(args.decode_steps, 5)
        gbps = dres["algo_bytes"] / (dres["ms_avg"] * 1e-3) / 1e9
        print(json.dumps({"decode_GBps": round(gbps, 2), "ms_avg": dres["ms_avg"],
                          "num_splits": dres["ns"]}), flush=True)
        return 0

    flush = _flush_buffer()
    res = bench_prefill(args.config, args.steps, args.warmup, flush=flush)
    cfg = res["cfg"]
    value = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
    achieved = res["flops"] / (res["fwd_ms_avg"] * 1e-3) / 1e12
    head = _prefill_entry(res)
    _progress(f"prefill {cfg.name}: {res['ms_per_step']:.4f} ms per step")
    line = {
        "metric": "active-block TFLOP/s (% bf16 MFMA peak) prefill; HBM GB/s sparse GQA decode",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": _workload_name(cfg),
            "batch": cfg.B, "heads": cfg.H, "seq_len": cfg.S, "head_dim": cfg.D, "block": 64,
            "active_blocks": res["active"], "causal_density": round(res["density"], 4),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma", "kernel": "prefill_kernel (bsattn_fwd)",
            "achieved": round(achieved, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": _traffic("prefill", cfg.name),
            "launch_ms_avg": round(res["fwd_ms_avg"], 5),
            "launch_timing": "HIP events around the forward kernel launched back to back, averaged",
            "flop_per_launch": res["flops"],
            "useful_frac": round(res["useful_flops"] / (res["fwd_ms_avg"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "launch_ms_cache_evicted": head.get("fwd_ms_cache_evicted"),
            "frac_cache_evicted": head.get("fwd_frac_cache_evicted"),
        },
        "fused_step_ms": head.get("fused_step_ms"),
        "mask_build_ms_avg": head["mask_build_ms_avg"],
    }

    # the headline's parity sample and oracle baseline, while its inputs are at hand
    cb = None
    if not args.no_cpu:
        cb = cpu_baseline_prefill(res, args.cpu_budget)
        cb.pop("seconds", None)
        cb["value"] = round(cb["value"], 6)
        _progress(f"cpu baseline: {cb['sample']}")
    del res

    if not args.no_other:
        # the other prefill workloads, measured the same way
        other = {}
        for name in ("C2", "C3", "C4"):
            if name == cfg.name:
                continue
            r = bench_prefill(name, max(20, args.steps // 2), max(5, args.warmup // 2), flush=flush)
            other[name] = _prefill_entry(r)
            del r
            _progress(f"prefill {name}: {other[name]['ms_per_step']} ms per step")
        line["prefill_other"] = other

    # what bf16 matrix-core work reaches here in practice (vendor BLAS), beside the nominal peak
    mc = bench_mfma_ceiling()
    line["roofline"]["library_gemm"] = {
        "what": "torch.bmm (vendor BLAS) bf16 rate on this device: the estimator's GEMM shape and "
                "one large square product; a same-box reference for the nominal peak",
        **mc,
        "kernel_vs_square_gemm": round(achieved / mc["square_8192"]["TFLOPs"], 4)}
    _progress(f"library GEMM: {mc['square_8192']['TFLOPs']} TFLOP/s square, "
              f"{mc['estimator_shape']['TFLOPs']} on the estimator shape")

    if not args.no_decode:
        dres = bench_decode(args.decode_steps, 5)
        gbps = dres["algo_bytes"] / (dres["ms_avg"] * 1e-3) / 1e9
        line["decode"] = {
            "workload": "C5 sparse GQA decode: batch 8, 32 query heads over 8 KV heads, D 128, "
                        "KV lengths U[4096, 32768], <= 64 selected 64-token blocks per (batch, KV head)",
            "value": round(gbps, 2), "unit": "GB/s",
            "ms_per_call_avg": round(dres["ms_avg"], 5), "ms_per_call_median": round(dres["ms_median"], 5),
            "num_splits": dres["ns"], "selected_tokens": dres["sel_tokens"],
            "cache": "256 MiB last-level cache flushed before every timed call (512 MiB read)",
            "in_stream": {
                "what": "time one call adds behind the cache-evicting read: (read + call) x n "
                        "minus read x n, each timed as one block of n",
                "ms_per_call": round(dres["ms_incremental"], 5),
                "GBps": round(dres["algo_bytes"] / (dres["ms_incremental"] * 1e-3) / 1e9, 2),
                "frac": round(dres["algo_bytes"] / (dres["ms_incremental"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "roofline": {"bound": "hbm", "kernel": "decode_split_kernel + decode_merge_kernel",
                         "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": _traffic("decode", "C5"),
                         "bytes_per_call": dres["algo_bytes"]},
        }
        _progress(f"decode: {dres['ms_avg']:.4f} ms per call")
        rc = bench_read_ceiling(dres["algo_bytes"], args.decode_steps)
        line["decode"]["read_ceiling"] = {
            "what": "plain streaming read of the same byte count (torch reductions over a buffer: "
                    "whole sum, and per-16-KiB-row sums; the faster), cache evicted before each "
                    "call the same way",
            "GBps": round(rc["GBps"], 2), "ms_per_call_avg": round(rc["ms_avg"], 5),
            "frac_of_peak": round(rc["GBps"] / HBM_PEAK_GBPS, 4), "form": rc["form"],
            "forms_GBps": rc["forms"]}
        lf = bench_launch_floor(args.decode_steps)
        line["decode"]["launch_floor"] = {
            "what": "one trivial kernel (a one-element fill) timed the same way: HIP events "
                    "around it after the same cache-evicting read",
            "ms_per_call_avg": round(lf["ms_avg"], 5), "ms_per_call_median": round(lf["ms_median"], 5)}
        if not args.no_cpu:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(dres)

    if not args.no_next:
        # the next rows of the hot path, each measured the same way as its base row
        nxt = {}
        if not args.no_decode:
            for form in ("mask", "paged"):
                r = bench_decode(args.decode_steps, 5, form=form, base=dres["inputs"])
                gb = r["algo_bytes"] / (r["ms_avg"] * 1e-3) / 1e9
                nxt[f"decode_{form}"] = {
                    "workload": "C5 sparse GQA decode, " + (
                        "mask form: block_mask [8, 8, 512]" if form == "mask"
                        else "paged KV cache: 256-token pages in a shuffled order, block_table [8, 128]"),
                    "value": round(gb, 2), "unit": "GB/s", "ms_per_call_avg": round(r["ms_avg"], 5),
                    "ms_per_call_median": round(r["ms_median"], 5), "num_splits": r["ns"],
                    "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBPS,
                                 "unit": "GB/s", "frac": round(gb / HBM_PEAK_GBPS, 4),
                                 "bytes_per_call": r["algo_bytes"]}}
        _progress("decode mask and paged forms done")
        pc = bench_prefill_chunk(max(20, args.steps // 4), 5)
        _progress(f"chunked prefill: {pc['ms']:.4f} ms")
        tf = pc["flops"] / (pc["ms"] * 1e-3) / 1e12
        nxt["prefill_chunk"] = {
            "workload": f"chunked prefill: the last {pc['Sq']} of {pc['Sk']} positions of C2 "
                        f"(B2 H16 D64, its top-16/tril/diagonal mask rows), causal",
            "value": round(tf, 3), "unit": "TFLOP/s", "ms_per_launch": round(pc["ms"], 5),
            "active_blocks": pc["active"],
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "flop_per_launch": pc["flops"]}}
        xr = bench_xattn(max(10, args.steps // 20), 3)
        tf_all = xr["flops"] / (xr["ms"] * 1e-3) / 1e12
        tf_sums = xr["flops"] / (xr["ms_sums"] * 1e-3) / 1e12
        nxt["xattn_estimate"] = {
            "workload": "XAttention block estimate on C3's shape (B1 H32 S16384 D128, seeded N(0,1) "
                        "q, k): stride 8, threshold 0.9, sink and diagonal kept, causal",
            "value": round(tf_all, 3), "unit": "TFLOP/s (reshaped GEMM flop / whole estimate)",
            "ms_per_call": round(xr["ms"], 5), "ms_block_sums": round(xr["ms_sums"], 5),
            "ms_selection": round(xr["ms_select"], 5), "mask_causal_density": round(xr["density"], 4),
            "roofline": {"bound": "mfma", "kernel": "xattn_lse_kernel + xattn_blocksum_kernel",
                         "achieved": round(tf_sums, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf_sums / BF16_PEAK_TFLOPS, 4), "flop_per_call": xr["flops"],
                         "traffic": _traffic("xattn", "C3"),
                         "vs_library_gemm_same_shape": round(
                             tf_sums / mc["estimator_shape"]["TFLOPs"], 4)}}
        line["next_rows"] = nxt

    if cb is not None:
        line["cpu_baseline"] = cb

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
