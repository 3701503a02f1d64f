#!/usr/bin/env python3
"""Benchmark of one MLA decode step over a paged latent cache on one MI355X.

A step is one pass of the whole hot path on one batch of synthetic input:
  mla_cache_append_query_absorb
                    (B new tokens: W^DKV / W^KR projection, RoPE, paged write;
                     and q~ = W^UK^T q^C, RoPE(q^R) for every query and head)
  mla_decode        (split-KV attention over the latent cache, all heads)
  mla_decode_combine_out_proj
                    (log-sum-exp merge of the splits, then the per-head W^UV
                     up-projection, in one kernel)
--separate runs the five single calls instead (mla_cache_append,
mla_query_absorb, mla_decode, mla_decode_combine, mla_out_proj).
Default workload: DeepSeek-V3 shape, bf16, B=64 sequences of L=4096 cached
tokens, one query token each, H=128, d_c=512, d_R=64, block 64, shuffled page
table.  Inputs are resident in HBM before timing; several copies of the pool
are rotated so the 256 MB last-level cache cannot serve the cache stream.
The timed region launches the calls of a step with only a start and a
stop event (--graph replays one captured HIP graph per step instead); the
per-kernel times, and the decode time the roofline uses, come from a second
pass of the same steps with an event around every call.  Outside the
timed step, the dense layers around it (mla_linear) and chunked prefill over
the latent cache (mla_prefill) are timed on their own.

Prints one JSON line (rank 0).  Metric: KV-tokens/s = sum_b L_b per step / time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense, published
BYTES_PER_KV_TOKEN = {"bf16": 1152, "fp8": 596, "fp8p2": 596, "fp32": 2304}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="v3", choices=["v3", "long", "ragged", "fp8", "fp8p2"])
    p.add_argument("--partitions", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true",
                   help="skip the separate timing of the query projections and W^O (mla_linear)")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the separate timing of chunked prefill over the latent cache (mla_prefill)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--generic", action="store_true", help="force the generic decode kernel")
    p.add_argument("--separate", action="store_true",
                   help="run the five single calls instead of mla_cache_append_query_absorb and "
                        "mla_decode_combine_out_proj")
    p.add_argument("--graph", action="store_true",
                   help="capture each step (per pool copy) into one HIP graph and replay it")
    p.add_argument("--no-calibration", action="store_true",
                   help="skip the achievable-peak calibration (copy kernel, MFMA loop)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (5 times), to "
                        "scale HBM byte counters; prints nothing else")
    return p.parse_args()


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mla_latent_kv_decode_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_src: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    # the kernel's own file plus the shared headers it is compiled with
    if d.get("source_hash") != source_hash(kernel_src, "mla_common.h", "mla_internal.h"):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs the whole hot path on a single "
              f"MI355X (no sharding, no collectives); got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_workloads as W
    import mla_latent_kv_decode_amd as M

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return
    M.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS[args.workload]
    d = cfg.dims
    bs, D, H = d.block_size, d.row, d.num_heads
    lens = W.seq_lens(cfg)
    B, n_q = cfg.batch, cfg.n_q
    table, nblk = W.page_table(lens, bs, cfg.seed)
    kv_tokens = int(lens.sum())
    cdt = {"bf16": M.BF16, "fp8": M.FP8_E4M3, "fp8p2": M.FP8_E4M3_PO2}[cfg.cache_dtype]
    fp8 = cfg.cache_dtype in ("fp8", "fp8p2")
    # the arithmetic type of the decode's matrix products: bf16 MFMA for the
    # bf16 cache and for the e4m3 cache with any tile scales (dequantised to
    # bf16 in LDS); the power-of-two e4m3 cache takes its scores on fp8 MFMA
    # and its output product on bf16 MFMA
    compute_dtype = "fp8+bf16" if cfg.cache_dtype == "fp8p2" and not args.generic else "bf16"
    dims = M.make_dims(H, d.d_latent, d.d_rope, d.d_nope, d.d_v, bs, cdt, M.BF16,
                       flags=M.FLAG_GENERIC_DECODE if args.generic else 0)

    # ---- resident inputs -------------------------------------------------
    elem = 1 if fp8 else 2
    pool_bytes = nblk * bs * D * elem
    n_copies = max(2, math.ceil(1.0e9 / pool_bytes) + 1)
    pools, scales = [], []
    for i in range(n_copies):
        rows = W.cache_rows(nblk * bs, cfg, seed=cfg.seed + 10 + i, device=dev)
        if fp8:
            # synthetic e4m3 bytes: the workload's rows reduced to codes by the
            # library's own cast; the benchmark times decode, not the codec
            # (one scale per row, stored for each of its five tiles; a power
            # of two for the power-of-two format)
            amax = rows.view(-1, D)[:, :].abs().amax(dim=1, keepdim=True).clamp_min(1e-6)
            if cfg.cache_dtype == "fp8p2":
                amax = torch.exp2(torch.ceil(torch.log2(amax / 448.0))) * 448.0
            sc = (amax / 448.0).expand(-1, 5).contiguous()
            pools.append((rows / amax * 448.0).clamp(-448, 448).to(torch.float8_e4m3fn)
                         .view(torch.uint8).view(nblk, bs, D))
            scales.append(sc.view(nblk, bs, 5))
        else:
            pools.append(rows.to(torch.bfloat16).view(nblk, bs, D))
            scales.append(None)
        del rows
    # queries: per head the content part q^C and the un-rotated RoPE part q^R,
    # N(0, 1), absorbed on the GPU every step (W^UK ~ N(0, 1/d_c))
    q_in = W.normal((B, n_q, H, d.d_nope + d.d_rope), cfg.seed + 20, device=dev, dtype=torch.bfloat16)
    w_uk = W.normal((H, d.d_nope, d.d_latent), cfg.seed + 34, std=1 / math.sqrt(d.d_latent),
                    device=dev, dtype=torch.bfloat16)
    q = torch.empty(B, n_q, H, D, dtype=torch.bfloat16, device=dev)
    table_t = torch.from_numpy(table).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    # append inputs: the n_q newest tokens of every sequence
    T = B * n_q
    h = W.normal((T, d.d_model), cfg.seed + 30, device=dev, dtype=torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, cfg.seed + 31, dtype=torch.bfloat16, device=dev)
    w_kr = W.weight(d.d_rope, d.d_model, cfg.seed + 32, dtype=torch.bfloat16, device=dev)
    w_uv = W.normal((H, d.d_v, d.d_latent), cfg.seed + 33, std=1 / math.sqrt(d.d_latent),
                    device=dev, dtype=torch.bfloat16)
    seq_ids = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(n_q)
    positions = (lens_t.repeat_interleave(n_q) - n_q
                 + torch.arange(n_q, dtype=torch.int32, device=dev).repeat(B)).to(torch.int32)
    aws_n = M.mla_cache_append_workspace_size(dims, T, d.d_model)
    aws = torch.empty(aws_n, dtype=torch.uint8, device=dev) if aws_n else None
    G = args.partitions
    ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, G), dtype=torch.uint8, device=dev)
    u = torch.empty(B, n_q, H, d.d_latent, dtype=torch.bfloat16, device=dev)
    o = torch.empty(B * n_q, H, d.d_v, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    # The calls of a step, each a closure over one pool copy.
    def calls(i):
        pool, sc = pools[i % n_copies], scales[i % n_copies]
        decode = lambda: M.mla_decode(dims, q, pool, sc, table_t, lens_t, ws, G)
        if args.separate:
            return [
                lambda: M.mla_cache_append(dims, h, w_dkv, w_kr, seq_ids, positions, table_t, pool, sc, aws),
                lambda: M.mla_query_absorb(dims, q_in, positions, w_uk, q),
                decode,
                lambda: M.mla_decode_combine(dims, ws, lens_t, u, None, G),
                lambda: M.mla_out_proj(dims, u.view(B * n_q, H, d.d_latent), w_uv, o),
            ]
        return [
            lambda: M.mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, seq_ids, positions, table_t, pool,
                                                    sc, aws, q_in, positions, w_uk, q),
            decode,
            lambda: M.mla_decode_combine_out_proj(dims, ws, lens_t, w_uv, o, B, n_q, None, None, G),
        ]
    names = (["append", "query_absorb", "decode", "combine", "out_proj"] if args.separate
             else ["append_query_absorb", "decode", "combine_out_proj"])

    # Achievable peaks on this chip (a plain device copy, a bf16 MFMA loop),
    # measured first; they are reported beside the nominal peaks.
    achievable = None if args.no_calibration else calibrate(M, stream)

    for i in range(args.warmup):
        for c in calls(i):
            c()
    torch.cuda.synchronize()

    # --graph: the calls of a step (per pool copy) are captured once into
    # one HIP graph (they allocate nothing and record no memsets) and a step
    # replays it.  Default: the calls are launched directly.
    if args.graph:
        cap = torch.cuda.Stream()
        runners = []
        for i in range(n_copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for c in calls(i):
                    c()
            runners.append(g.replay)
        for i in range(args.warmup):
            runners[i % n_copies]()
        torch.cuda.synchronize()
        run_step = lambda i: runners[i % n_copies]()
    else:
        def run_step(i):
            for c in calls(i):
                c()

    # ---- timed region: exactly K steps ------------------------------------
    # Only a start and a stop event: an event recorded between two kernels
    # costs the stream several microseconds, so per-kernel times come from a
    # second, separately timed pass below.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        run_step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # ---- per-kernel times: K more steps with an event around every call ----
    nk = len(names)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev = evs[i]
        for k, c in enumerate(calls(i)):
            ev[k].record(stream)
            c()
        ev[nk].record(stream)
    torch.cuda.synchronize()
    per = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(nk)] for e in evs])
    k_ms_evented = per.mean(axis=0)
    step_ms = per.sum(axis=1)  # per step, events included
    # Every call's evented time carries the same event cost; the timed steps
    # carry none (their kernels run back to back), so the cost per call is
    # (evented step - timed step) / calls, and the kernels' own times follow.
    event_ms = max(0.0, (float(step_ms.mean()) - ms_per_step) / nk)
    k_ms = np.maximum(k_ms_evented - event_ms, 0.0)
    # the decode and its merge alone (with the fused W^UV when that is one call)
    dc = [n for n in names if n in ("decode", "combine", "combine_out_proj")]
    dc_ms = float(sum(k_ms[names.index(n)] for n in dc))
    decode_ms = float(k_ms[names.index("decode")])

    # ---- roofline of the dominant kernel (decode) ---------------------------
    # t_roof = max(bytes / HBM peak, flops / MFMA peak of the arithmetic dtype):
    # whichever is larger bounds the kernel and is the one reported.
    bytes_alg = kv_tokens * BYTES_PER_KV_TOKEN[cfg.cache_dtype] + B * n_q * H * D * 2
    flops_qk = kv_tokens * n_q * 2 * H * D
    flops_pv = kv_tokens * n_q * 2 * H * d.d_latent
    flops_alg = flops_qk + flops_pv
    achieved_gbps = bytes_alg / (decode_ms * 1e-3) / 1e9
    achieved_tflops = flops_alg / (decode_ms * 1e-3) / 1e12
    t_hbm = bytes_alg / (HBM_PEAK_GBPS * 1e9)
    if compute_dtype == "fp8+bf16":   # scores at the fp8 peak, the output product at the bf16 peak
        t_mfma = (flops_qk / MFMA_PEAK_TFLOPS["fp8"] + flops_pv / MFMA_PEAK_TFLOPS["bf16"]) / 1e12
        mfma_peak = round(flops_alg / t_mfma / 1e12, 1)   # the mix's effective peak
    else:
        mfma_peak = MFMA_PEAK_TFLOPS[compute_dtype]
        t_mfma = flops_alg / (mfma_peak * 1e12)
    kernel_src = "decode_generic.hip" if args.generic else "decode_mfma.hip"
    traffic = traffic_from_profile(kernel_src, args.workload)
    if t_hbm >= t_mfma:
        roofline = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(achieved_tflops / mfma_peak, 4)}
    roofline.update({"traffic": traffic,
                     "hbm_gbps": round(achieved_gbps, 1), "hbm_frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "mfma_tflops": round(achieved_tflops, 1), "mfma_frac": round(achieved_tflops / mfma_peak, 4),
                     "mfma_dtype": compute_dtype, "t_roof_ms": round(max(t_hbm, t_mfma) * 1e3, 5),
                     "bytes_alg_per_launch": bytes_alg, "flops_alg_per_launch": flops_alg,
                     "kernel_ms": round(decode_ms, 5), "achievable": achievable})

    # ---- the dense layers around the step (outside the timed region) -------
    dense = None if args.no_dense else dense_layers(M, W, dims, d, B * n_q, args.steps, stream)
    prefill = None if args.no_prefill else prefill_chunks(M, W, stream)

    # ---- CPU baseline: the oracle on a bounded sample ----------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, pools[0], scales[0], table, lens, q_in, w_uk, h, w_dkv, w_kr, w_uv,
                           args.cpu_seconds)

    out = {
        "metric": "MLA decode KV-tokens/s (+ achieved HBM GB/s and MFMA TFLOP/s vs roofline)",
        "value": round(kv_tokens * args.steps / (total_ms * 1e-3), 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": compute_dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} L={'ragged' if cfg.seq_len is None else cfg.seq_len} "
                               f"n_q={n_q} H={H} d_c={d.d_latent} d_R={d.d_rope} block={bs} "
                               f"cache={cfg.cache_dtype}",
                   "batch": B, "kv_tokens_per_step": kv_tokens, "n_q": n_q, "cache_dtype": cfg.cache_dtype,
                   "partitions": G, "pool_copies_rotated": n_copies},
        "kernels_ms": {n: round(float(t), 5) for n, t in zip(names, k_ms)},
        "kernels_timing": ("a second pass of K steps with an event around every call, less the events' own "
                           "cost per call: (evented step - timed step) / calls"),
        "kernels_ms_evented": {n: round(float(t), 5) for n, t in zip(names, k_ms_evented)},
        "event_cost_ms_per_call": round(event_ms, 5),
        "evented_step_ms": {"p10": round(float(np.percentile(step_ms, 10)), 5),
                            "median": round(float(np.median(step_ms)), 5),
                            "p90": round(float(np.percentile(step_ms, 90)), 5)},
        "decode_combine_kv_tokens_per_s": {"value": round(kv_tokens / (dc_ms * 1e-3), 1), "calls": dc},
        "decode_kernel": "generic" if args.generic else "default",
        "launch": "hip_graph_replay" if args.graph else "direct",
        "calibration_before_timed_steps": achievable is not None,
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "dense_layers": dense,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def dense_layers(M, W, dims, d, rows, steps, stream):
    """The decoding procedure's dense layers at this batch, timed on their own
    (mla_linear): the query projections c^Q = W^DQ h and [W^UQ_i ; W^QR_i] c^Q
    (head by head, one call), and the output projection W^O.  Each is
    weight-streaming: the figure is weight bytes per launch / launch time
    against the HBM peak; two weight copies alternate so the 256 MB Infinity
    Cache cannot hold the one being read."""
    import torch
    H, dq = d.num_heads, d.d_q
    bf = torch.bfloat16
    layers = {"w_dq": (d.d_model, dq), "w_uq_qr": (dq, H * (d.d_nope + d.d_rope)),
              "w_o": (H * d.d_v, d.d_model)}
    out = {"rows": rows}
    for j, (name, (k, n)) in enumerate(layers.items()):
        x = W.normal((rows, k), 500 + j, device="cuda", dtype=bf)
        ws = [W.weight(n, k, 510 + 2 * j + c, dtype=bf, device="cuda") for c in range(2)]
        y = torch.empty(rows, n, dtype=bf, device="cuda")
        nws = M.mla_linear_workspace_size(dims, rows, n, k)
        wsp = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        for c in range(4):
            M.mla_linear(dims, x, ws[c % 2], y, wsp)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i].record(stream)
            M.mla_linear(dims, x, ws[i % 2], y, wsp)
        evs[steps].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]))
        gbps = n * k * 2 / (ms * 1e-3) / 1e9
        out[name] = {"n": n, "k": k, "ms": round(ms, 5), "weight_gbps": round(gbps, 1),
                     "frac": round(gbps / HBM_PEAK_GBPS, 4)}
        del ws, x, y, wsp
    return out


PREFILL_CHUNKS = ((8192, 1024), (16384, 2048))


def prefill_chunks(M, W, stream, iters=30):
    """Chunked prefill over the latent cache (mla_prefill, bf16, DeepSeek-V3
    dims), timed on its own at two (cached rows T, chunk C) shapes: the last C
    of T rows are the chunk's own tokens.  Algorithmic flops per call: the
    K^C and V expansions, 2 * T * d_c * H * (d_nope + d_v), plus the causal
    attention, 2 * H * (d_nope + d_R + d_v) per visible (query, key) pair,
    sum_j (T - C + j + 1) pairs; against the dense bf16 matrix-core peak."""
    import torch
    cfg = W.CONFIGS["v3"]
    d = cfg.dims
    H, bs = d.num_heads, d.block_size
    dims = M.make_dims(H, d.d_latent, d.d_rope, d.d_nope, d.d_v, bs, M.BF16, M.BF16)
    std = 1 / math.sqrt(d.d_latent)
    w_uk = W.normal((H, d.d_nope, d.d_latent), 601, std=std, device="cuda").to(torch.bfloat16)
    w_uv = W.normal((H, d.d_v, d.d_latent), 602, std=std, device="cuda").to(torch.bfloat16)
    out = {"iters": iters, "dtype": "bf16"}
    for i, (T, C) in enumerate(PREFILL_CHUNKS):
        lens = np.array([T], np.int32)
        table, nblk = W.page_table(lens, bs, 610 + i)
        pool = W.cache_rows(nblk * bs, cfg, seed=620 + i, device="cuda").to(torch.bfloat16).view(nblk, bs, d.row)
        tab = torch.from_numpy(table[0]).cuda()
        q = W.normal((C, H, d.d_nope + d.d_rope), 630 + i, device="cuda").to(torch.bfloat16)
        y = torch.empty(C, H, d.d_v, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(M.mla_prefill_workspace_size(dims, C, T), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            M.mla_prefill(dims, q, pool, tab, T, w_uk, w_uv, y, ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            M.mla_prefill(dims, q, pool, tab, T, w_uk, w_uv, y, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        pairs = C * (T - C) + C * (C + 1) // 2
        flops = 2 * T * d.d_latent * H * (d.d_nope + d.d_v) + 2 * H * (d.d_nope + d.d_rope + d.d_v) * pairs
        tf = flops / (ms * 1e-3) / 1e12
        out[f"T{T}_C{C}"] = {"cached_rows": T, "chunk": C, "ms": round(ms, 5), "flops": flops,
                             "tflops": round(tf, 1), "frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)}
        del pool, q, y, ws
    return out


def calibrate(M, stream):
    """Achievable peaks: a plain 1 GiB device-to-device copy (read + write bytes
    per second) and a bf16 MFMA loop (libmla_calib.so, 2048 workgroups of
    eight waves, four independent accumulators each), 10 launches each, median."""
    import ctypes
    import torch
    out = {}
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ts = []
    for i in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    out["copy_gbps"] = round(2 * n / (float(np.median(ts)) * 1e-3) / 1e9, 1)
    del src, dst
    calib = ctypes.CDLL(os.path.join(os.path.dirname(M.LIB_PATH), "libmla_calib.so"))
    calib.mla_calib_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    wgs, iters = 2048, 256
    sink = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
    ts = []
    for i in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert calib.mla_calib_mfma_loop(iters, wgs, sink.data_ptr(), stream.cuda_stream) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    flops = wgs * 8 * iters * 32 * 32768
    out["mfma_loop_bf16_tflops"] = round(flops / (float(np.median(ts)) * 1e-3) / 1e12, 1)
    out["note"] = "achievable on this chip: device copy (read+write) and a bf16 MFMA loop"
    return out


def cpu_baseline(cfg, pool, sc, table, lens, q_in, w_uk, h, w_dkv, w_kr, w_uv, seconds):
    """The oracle as it stands, in float32 (its dtype argument; parity uses
    float64), on a bounded sample of the same workload: the first few
    sequences' append rows, query absorption, absorbed decode and W^UV.  Three
    runs of about seconds/3 each; the median run's rate is reported."""
    import torch
    from threadpoolctl import threadpool_info
    from oracle import mla_oracle as O

    d = cfg.dims
    bs = d.block_size
    n_seq = 4
    ids = list(range(n_seq))
    host_pool = {"dtype": "fp8" if cfg.cache_dtype in ("fp8", "fp8p2") else cfg.cache_dtype}
    blocks = np.unique(table[ids][table[ids] >= 0])
    data = np.zeros((pool.shape[0],) + tuple(pool.shape[1:]),
                    dtype=np.uint8 if host_pool["dtype"] == "fp8" else np.uint16)
    idx = torch.from_numpy(blocks.astype(np.int64)).to(pool.device)
    raw = pool.index_select(0, idx).cpu()
    data[blocks] = raw.numpy() if host_pool["dtype"] == "fp8" else raw.view(torch.int16).numpy().view(np.uint16)
    host_pool["data"] = data
    if sc is not None:
        s = np.zeros((pool.shape[0], bs, 5), np.float32)
        s[blocks] = sc.index_select(0, idx).cpu().numpy()
        host_pool["scales"] = s

    def f32(t):
        return O.bf16_bits_to_f64(t.detach().cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float32)

    qin = f32(q_in[:n_seq])
    hh = f32(h[:n_seq * cfg.n_q])
    wd, wk, wu, wq = f32(w_dkv), f32(w_kr), f32(w_uv), f32(w_uk)
    scale = O.softmax_scale(d.d_nope, d.d_rope)
    pos = (lens[:n_seq].repeat(cfg.n_q) - 1).astype(np.int64)
    qpos = (lens[:n_seq, None] - cfg.n_q + np.arange(cfg.n_q)[None, :]).astype(np.int64)
    f = np.float32

    def one_rep():
        O.kv_rows(hh, wd, wk, pos, dtype=f)
        qh = O.absorb_query(qin[..., :d.d_nope], qin[..., d.d_nope:], wq, qpos, dtype=f)
        res = O.decode(qh, host_pool, table, lens, bs, d.d_latent, scale, batch_ids=ids, dtype=f)
        O.out_proj(np.concatenate([res[b][0] for b in ids]), wu, dtype=f)

    rates, reps_all = [], []
    for run in range(3):
        reps, t_start = 0, time.perf_counter()
        while True:
            one_rep()
            reps += 1
            el = time.perf_counter() - t_start
            if el >= seconds / 3 or reps >= 1000:
                break
        rates.append(reps * int(lens[:n_seq].sum()) / el)
        reps_all.append(reps)
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else len(os.sched_getaffinity(0))
    lib = f"{blas[0].get('internal_api', '?')} {blas[0].get('version', '')}".strip() if blas else "unknown"
    return {"value": round(float(np.median(rates)), 1), "unit": "KV-tokens/s",
            "cores": threads, "kind": "oracle", "blas": lib,
            "runs": [round(r, 1) for r in rates],
            "sample": f"{n_seq} of {cfg.batch} sequences ({int(lens[:n_seq].sum())} KV-tokens), "
                      f"append rows + query absorption + absorbed decode + W^UV in float32 NumPy "
                      f"({lib}, {threads} threads); median of 3 runs of {reps_all} repetitions"}


if __name__ == "__main__":
    main()
