#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass over every hot-path kernel, on synthetic inputs already
resident in HBM:
  1. tq_set_rows: quantize one 32768-row K and V cache (4 kv heads, d 128,
     turbo3, outlier channels);
  2. tq_attn_decode: one decode token across LAYERS layers, each layer
     attending over its own 32768-cell turbo3 cache (32 q / 4 kv heads,
     bf16 q); the LAYERS caches (>256 MB in total) are cycled so every call
     streams its cache from HBM, and the calls are replayed from a HIP graph;
  3. tq_attn_prefill: 2048 causal rows, 16 q / 8 kv heads, d 256, turbo3;
  4. tq_attn_int8_prompt: 2048 queries x 40000 cells, 8 q / 1 kv head, d 128.
Each phase is timed with HIP events on the stream its kernels run on; the
step time is their sum.  `value` is the decode leg's KV bytes (algorithmic:
packed codes + norms of every key and kv head) per second.

Prints ONE JSON line.  The CPU baseline runs the oracle (oracle/) on a
bounded sample of the decode workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "decode KV GB/s (% HBM peak) at 32K + prefill tokens/s (% MFMA peak)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3

# HBM traffic of one decode call (fused split kernel + merge kernel), from two
# `rocprofv3 --pmc` passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over
# `bench.py --no-cpu-baseline --only decode,copy --steps 2 --warmup 1`, each
# scaled by what the same counter reads for the 256 MiB device copy of that
# run (FETCH_SIZE reads 131088.8 KiB for 262144 KiB copied: x1.99974;
# WRITE_SIZE reads 262144 KiB: x1.0).  Valid only for the decode kernels it
# was taken on: sha256 of their sources (tq_decode.hip, tq_decode_fused4.hip,
# tq_common.h) and of build.py, whose per-source flags shape their code;
# otherwise traffic is reported as null.
DECODE_TRAFFIC = {"sources_sha256": "5a7e501239135a3fe683c41a2bc2bd856c29e853ee53a168c0b48d5233b9d8c3",
                  "fetch_kib": {"decode_fused_kernel": 6542.3, "decode_merge_kernel": 568.5},
                  "write_kib": {"decode_fused_kernel": 1088.0, "decode_merge_kernel": 16.0},
                  "fetch_scale": 1.99974, "write_scale": 1.0}


def decode_traffic_bytes():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in ("csrc/tq_decode.hip", "csrc/tq_decode_fused4.hip", "csrc/tq_common.h", "build.py"):
        with open(os.path.join(here, "quantized_kv_cache_tq_amd", f), "rb") as fh:
            h.update(fh.read())
    t = DECODE_TRAFFIC
    if h.hexdigest() != t["sources_sha256"]:
        return None
    kib = (sum(t["fetch_kib"].values()) * t["fetch_scale"] +
           sum(t["write_kib"].values()) * t["write_scale"])
    return int(round(kib * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of legs: set_rows,decode,prefill,int8 (default: all; extras decode_wide, decode_long, decode_paths, "
                         "decode_types, decode_batch, floor, prefill_rows, int8_140k); "
                         "'copy' adds a 256 MiB device copy used to calibrate HBM counters")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Leg:
    """Times one phase with HIP events on torch's current stream."""

    def __init__(self, name):
        import torch
        self.name = name
        self.pairs = []
        self.torch = torch

    def run(self, fn, record=True):
        if not record:
            fn()
            return
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def mean_ms(self):
        if not self.pairs:
            return None
        return float(np.mean(self.times_ms()))

    def median_ms(self):
        if not self.pairs:
            return None
        return float(np.median(self.times_ms()))


def host_info():
    """Host cores the CPU baseline can use and what it ran on."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["affinity_cpus"] = None
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        info["blas_threads"] = None
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        info["cpu_model"] = None
    return info


def max_abs_rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64).astype(np.float32).astype(np.float64)
    d = got - want
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-300))


def oracle_leg(b, torch, dev, inputs, k_np, v_np, q_np, kc0, vc0, q_dec, ws, scale_dec, kv_bytes_per_call,
               prefill, int8, snap, pf_inputs, d8):
    """The oracle timed on bounded samples of each workload on the host cores,
    and the parity of the GPU results of this run against it."""
    import oracle as o
    log("[bench] cpu baseline: oracle set_rows, decode, prefill and int8 samples")
    host = host_info()
    legs = {}
    parity = {}
    KV, NKV, D = k_np.shape
    # set_rows: the 32K x 4-head K and V caches (vectorized float32 numpy)
    t0 = time.perf_counter()
    okc, ovc = o.new_cache(3, D, NKV, KV), o.new_cache(3, D, NKV, KV)
    o.set_rows(okc, k_np, np.arange(KV))
    o.set_rows(ovc, v_np, np.arange(KV))
    dt = time.perf_counter() - t0
    sr_bytes = 2 * (KV * NKV * D * 4 + KV * NKV * 50)
    legs["set_rows_32k_KV_pair"] = {"s": round(dt, 3), "GBps": round(sr_bytes / dt / 1e9, 4)}
    # decode: two calls at the 32K / GQA-8 shape
    reps = 2
    t0 = time.perf_counter()
    for _ in range(reps):
        ref = o.attn_decode(okc, ovc, KV, q_np.astype(np.float64), scale_dec)
    dt_dec = (time.perf_counter() - t0) / reps
    legs["decode_32k_gqa8"] = {"s_per_call": round(dt_dec, 3), "GBps": round(kv_bytes_per_call / dt_dec / 1e9, 6)}
    # decode parity: one call into a buffer of its own, right before the compare
    chk = torch.empty((q_np.shape[0], D), dtype=torch.float32, device=dev)
    b.tq_attn_decode(kc0, vc0, KV, q_dec, scale_dec, out=chk, workspace=ws)
    torch.cuda.synchronize()
    ma, rl = max_abs_rel_l2(chk.cpu().numpy(), ref)
    parity["decode_32k"] = {"max_abs": ma, "rel_l2": rl}
    # sparse V at the pages' turbo3 threshold: the order-free bound B of the
    # skipped terms and the share of (head, key) weights below tau
    tau = 5e-3
    bnd, n_small = o.sparse_v_bound(okc, ovc, KV, q_np.astype(np.float64), scale_dec, tau)
    chk_s = torch.empty_like(chk)
    b.tq_attn_decode(kc0, vc0, KV, q_dec, scale_dec, out=chk_s, workspace=ws, sparse_v_tau=tau)
    torch.cuda.synchronize()
    dev_s = np.abs(chk_s.cpu().numpy().astype(np.float64) - ref).max(axis=1)
    parity["decode_32k_sparse_v"] = {"tau": tau, "bound_B_max": float(bnd.max()),
                                     "skippable_fraction": float(n_small.sum() / (KV * len(n_small))),
                                     "max_abs_vs_dense_oracle": float(dev_s.max()),
                                     "within_B_plus_2e-3": bool(np.all(dev_s <= bnd + 2e-3))}
    del okc, ovc
    if prefill is not None and pf_inputs is not None:
        # prefill: the last 256 of the 2048 causal rows (dequantize the cache,
        # then float64 attention), against the timed call's output
        pq, pk, pv = pf_inputs
        R, _, PD = pq.shape
        t0 = time.perf_counter()
        pkc, pvc = o.new_cache(3, PD, pk.shape[1], R), o.new_cache(3, PD, pk.shape[1], R)
        o.set_rows(pkc, pk, np.arange(R))
        o.set_rows(pvc, pv, np.arange(R))
        t1 = time.perf_counter()
        n_s = 256
        want = o.attn_prefill(pkc, pvc, R, pq[R - n_s:].astype(np.float64), R - n_s, 1.0 / math.sqrt(PD))
        dt = time.perf_counter() - t1
        legs["prefill_2048_last_256_rows"] = {"s": round(dt, 3), "tokens_per_s": round(n_s / dt, 1),
                                             "quantize_s": round(t1 - t0, 3)}
        ma, rl = max_abs_rel_l2(snap["prefill"][R - n_s:], want)
        parity["prefill_2048_last_256_rows"] = {"max_abs": ma, "rel_l2": rl}
    if int8 is not None and d8 is not None:
        # int8 prompt: the last 64 of the 2048 queries at 40000 cells
        ctx = int8["ctx"]
        n_q8 = d8["q"].shape[0]
        n_s = 64
        t0 = time.perf_counter()
        want = o.attn_int8_prompt(d8["q"][n_q8 - n_s:].astype(np.float64), d8["k8"], d8["v8"], d8["k_scale"],
                                  d8["v_scale"], d8["page_table"], ctx, ctx - n_s, 1.0 / math.sqrt(d8["q"].shape[2]))
        dt = time.perf_counter() - t0
        pairs = n_s * ctx - n_s * (n_s - 1) // 2
        legs["int8_40k_last_64_queries"] = {"s": round(dt, 3),
                                           "GFLOPs": round(4.0 * 128 * d8["q"].shape[1] * pairs / dt / 1e9, 2)}
        ma, rl = max_abs_rel_l2(snap["int8"][n_q8 - n_s:], want)
        parity["int8_40k_last_64_queries"] = {"max_abs": ma, "rel_l2": rl}
    cores = host["blas_threads"] or 1
    return {"cpu_baseline": {"value": legs["decode_32k_gqa8"]["GBps"], "unit": "GB/s", "cores": cores,
                             "kind": "oracle",
                             "sample": f"{reps} numpy decode calls at the 32K / GQA-8 turbo3 shape "
                                       f"({dt_dec:.2f} s per call: unpack, dequantize, float64 attention "
                                       f"through BLAS with {cores} threads); the other legs in 'legs'",
                             "host": host, "legs": legs},
            "parity_check": parity}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(multi-GPU sharding is a design note, not implemented)"}))
        sys.exit(2)
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from quantized_kv_cache_tq_amd import inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    b.load_library()
    only = set(filter(None, args.only.split(",")))
    want = lambda leg: not only or leg in only
    dev = torch.device("cuda:0")
    t_wall0 = time.time()

    # ---------------- decode workload (32 q / 4 kv heads, d 128, 32K, turbo3)
    log("[bench] generating the 32K decode workload")
    q_np, k_np, v_np = inputs.outlier_decode(seed=0)
    KV, NKV, D, NQ = k_np.shape[0], k_np.shape[1], k_np.shape[2], q_np.shape[0]
    k_src = torch.from_numpy(k_np).to(dev)
    v_src = torch.from_numpy(v_np).to(dev)
    idx = torch.arange(KV, dtype=torch.int64, device=dev)
    q_dec = torch.from_numpy(q_np).to(torch.bfloat16).to(dev)
    L = args.layers
    kcs = [b.new_cache(3, D, NKV, KV) for _ in range(L)]
    vcs = [b.new_cache(3, D, NKV, KV) for _ in range(L)]
    b.tq_set_rows(kcs[0], k_src, idx)
    b.tq_set_rows(vcs[0], v_src, idx)
    for i in range(1, L):
        kcs[i].codes.copy_(kcs[0].codes); kcs[i].norms.copy_(kcs[0].norms)
        vcs[i].codes.copy_(vcs[0].codes); vcs[i].norms.copy_(vcs[0].norms)
    torch.cuda.synchronize()
    scale_dec = 1.0 / math.sqrt(D)
    ws_bytes = b.tq_attn_decode_workspace(kcs[0], vcs[0], KV, NQ)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [torch.empty((NQ, D), dtype=torch.float32, device=dev) for _ in range(L)]
    kv_bytes_per_call = 2 * NKV * KV * (48 + 2)      # packed codes + fp16 norm, K and V

    def decode_all():
        for i in range(L):
            b.tq_attn_decode(kcs[i], vcs[i], KV, q_dec, scale_dec, out=outs[i], workspace=ws)

    graph = None
    if want("decode"):
        decode_all()                       # warm, outside capture
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            decode_all()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_all()
        torch.cuda.synchronize()

    # ---------------- prefill workload (2048 rows, 16 q / 8 kv heads, d 256)
    prefill = None
    if want("prefill"):
        try:
            pq, pk, pv = inputs.prefill(seed=0, rows=2048)
            R, PNQ, PD = pq.shape
            PNKV = pk.shape[1]
            pkc, pvc = b.new_cache(3, PD, PNKV, R), b.new_cache(3, PD, PNKV, R)
            pidx = torch.arange(R, dtype=torch.int64, device=dev)
            b.tq_set_rows(pkc, torch.from_numpy(pk).to(dev), pidx)
            b.tq_set_rows(pvc, torch.from_numpy(pv).to(dev), pidx)
            pqt = torch.from_numpy(pq).to(torch.bfloat16).to(dev)
            pws = torch.empty(max(256, b.tq_attn_prefill_workspace(pkc, R, PNQ, R)), dtype=torch.uint8,
                              device=dev)
            pout = torch.empty((R, PNQ, PD), dtype=torch.float32, device=dev)
            pscale = 1.0 / math.sqrt(PD)
            fn = lambda: b.tq_attn_prefill(pkc, pvc, R, pqt, 0, pscale, out=pout, workspace=pws)
            fn()
            torch.cuda.synchronize()
            flops = 4.0 * PD * PNQ * (R * (R + 1) / 2)
            prefill = dict(fn=fn, rows=R, flops=flops)
            # the other two cache types through the same prefill kernel
            # (timed after the steps, not part of a step)
            for bits in (2, 4):
                xk, xv = b.new_cache(bits, PD, PNKV, R), b.new_cache(bits, PD, PNKV, R)
                b.tq_set_rows(xk, torch.from_numpy(pk).to(dev), pidx)
                b.tq_set_rows(xv, torch.from_numpy(pv).to(dev), pidx)
                prefill[f"turbo{bits}"] = (lambda xk=xk, xv=xv: b.tq_attn_prefill(
                    xk, xv, R, pqt, 0, pscale, out=pout, workspace=pws))
            # 128-wide heads, twice the q heads: the same products per call
            hq_, hk_, hv_ = inputs.prefill(seed=1, rows=R, n_q=2 * PNQ, n_kv=PNKV, d=PD // 2)
            hkc, hvc = b.new_cache(3, PD // 2, PNKV, R), b.new_cache(3, PD // 2, PNKV, R)
            b.tq_set_rows(hkc, torch.from_numpy(hk_).to(dev), pidx)
            b.tq_set_rows(hvc, torch.from_numpy(hv_).to(dev), pidx)
            hqt = torch.from_numpy(hq_).to(torch.bfloat16).to(dev)
            hout = torch.empty((R, 2 * PNQ, PD // 2), dtype=torch.float32, device=dev)
            prefill["d128"] = (lambda: b.tq_attn_prefill(hkc, hvc, R, hqt, 0, 1.0 / math.sqrt(PD // 2),
                                                         out=hout, workspace=pws))
        except b.TQError as e:
            log(f"[bench] prefill leg skipped: {e}")

    # ---------------- int8 prompt workload (2048 q x 40000 cells)
    int8 = None
    if want("int8"):
        try:
            d8 = inputs.int8_prompt(seed=0, ctx=40000)
            t = {k_: torch.from_numpy(v_).to(dev) for k_, v_ in d8.items() if not k_.endswith("logical")}
            n_q8, nqh8, dd8 = d8["q"].shape
            ctx8 = 40000
            q08 = ctx8 - n_q8
            ws8 = torch.empty(max(256, b.tq_attn_int8_prompt_workspace(n_q8, nqh8, 1, dd8, ctx8)),
                              dtype=torch.uint8, device=dev)
            out8 = torch.empty((n_q8, nqh8, dd8), dtype=torch.float32, device=dev)
            fn8 = lambda: b.tq_attn_int8_prompt(t["q"], t["k8"], t["v8"], t["k_scale"], t["v_scale"],
                                                t["page_table"], ctx8, q08, 1.0 / math.sqrt(dd8),
                                                out=out8, workspace=ws8)
            fn8()
            torch.cuda.synchronize()
            pairs = sum(min(ctx8, q08 + i + 1) for i in range(n_q8))
            int8 = dict(fn=fn8, flops=4.0 * dd8 * nqh8 * pairs, ctx=ctx8, n_q=n_q8)
        except b.TQError as e:
            log(f"[bench] int8 leg skipped: {e}")

    # ---------------- calibration copy (not part of a step; only with --only copy):
    # a plain device-to-device copy of known size, for scaling HBM counters
    copy = None
    if "copy" in only:
        csrc = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        cdst = torch.empty_like(csrc)
        copy = dict(fn=lambda: cdst.copy_(csrc), nbytes=csrc.numel())

    # ---------------- timed steps
    legs = {n: Leg(n) for n in ("set_rows", "decode", "prefill", "int8", "copy")}

    def step(record):
        if want("set_rows"):
            j = step.i % L
            legs["set_rows"].run(lambda: (b.tq_set_rows(kcs[j], k_src, idx),
                                          b.tq_set_rows(vcs[j], v_src, idx)), record)
        if graph is not None:
            legs["decode"].run(graph.replay, record)
        if prefill is not None:
            legs["prefill"].run(prefill["fn"], record)
        if int8 is not None:
            legs["int8"].run(int8["fn"], record)
        if copy is not None:
            legs["copy"].run(copy["fn"], record)
        step.i += 1
    step.i = 0

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / max(1, args.steps)
    log("[bench] timed region done")
    # the timed calls' outputs, before any extra reuses their buffers (the
    # parity check below compares samples of them with the oracle)
    snap = {}
    if prefill is not None:
        snap["prefill"] = pout.cpu().numpy()
    if int8 is not None:
        snap["int8"] = out8.cpu().numpy()

    # ---------------- extras, timed after the steps (not part of a step)
    def time_eager(fn, reps=10):
        leg = Leg("extra")
        for _ in range(2):
            leg.run(fn, False)
        for _ in range(reps):
            leg.run(fn, True)
        torch.cuda.synchronize()
        return leg.mean_ms()
    extras = {}
    if prefill is not None:
        for bits in (2, 4):
            t_ms = time_eager(prefill[f"turbo{bits}"])
            tf = prefill["flops"] / (t_ms * 1e-3) / 1e12
            extras[f"prefill_turbo{bits}"] = {"us": round(t_ms * 1e3, 2), "TFLOPs": round(tf, 2),
                                              "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        t_ms = time_eager(prefill["d128"])
        tf = prefill["flops"] / (t_ms * 1e-3) / 1e12
        extras["prefill_turbo3_d128_32q8kv"] = {"us": round(t_ms * 1e3, 2), "TFLOPs": round(tf, 2),
                                                "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
    if prefill is not None and want("prefill_rows"):
        # the other two prompt lengths of the prefill workload, 512 and 4096
        # causal rows against as many cells (leg "prefill_rows")
        for R2 in (512, 4096):
            q2_, k2_, v2_ = inputs.prefill(seed=2, rows=R2)
            k2c, v2c = b.new_cache(3, PD, PNKV, R2), b.new_cache(3, PD, PNKV, R2)
            idx2 = torch.arange(R2, dtype=torch.int64, device=dev)
            b.tq_set_rows(k2c, torch.from_numpy(k2_).to(dev), idx2)
            b.tq_set_rows(v2c, torch.from_numpy(v2_).to(dev), idx2)
            q2t = torch.from_numpy(q2_).to(torch.bfloat16).to(dev)
            o2 = torch.empty((R2, PNQ, PD), dtype=torch.float32, device=dev)
            w2 = torch.empty(max(256, b.tq_attn_prefill_workspace(k2c, R2, PNQ, R2)), dtype=torch.uint8, device=dev)
            t_ms = time_eager(lambda: b.tq_attn_prefill(k2c, v2c, R2, q2t, 0, pscale, out=o2, workspace=w2))
            tf = 4.0 * PD * PNQ * (R2 * (R2 + 1) / 2) / (t_ms * 1e-3) / 1e12
            extras[f"prefill_turbo3_{R2}rows"] = {"us": round(t_ms * 1e3, 2),
                                                  "tokens_per_s": round(R2 / (t_ms * 1e-3), 1),
                                                  "TFLOPs": round(tf, 2),
                                                  "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
            del k2c, v2c, q2t, o2, w2
        # the speculative-verify batch: 3 rows at the end of 1024 cells
        q3_, k3_, v3_ = inputs.prefill(seed=3, rows=3, kv_len=1024)
        k3c, v3c = b.new_cache(3, PD, PNKV, 1024), b.new_cache(3, PD, PNKV, 1024)
        idx3 = torch.arange(1024, dtype=torch.int64, device=dev)
        b.tq_set_rows(k3c, torch.from_numpy(k3_).to(dev), idx3)
        b.tq_set_rows(v3c, torch.from_numpy(v3_).to(dev), idx3)
        q3t = torch.from_numpy(q3_).to(torch.bfloat16).to(dev)
        o3 = torch.empty((3, PNQ, PD), dtype=torch.float32, device=dev)
        w3 = torch.empty(max(256, b.tq_attn_prefill_workspace(k3c, 3, PNQ, 1024)), dtype=torch.uint8, device=dev)
        t_ms = time_eager(lambda: b.tq_attn_prefill(k3c, v3c, 1024, q3t, 1021, pscale, out=o3, workspace=w3),
                          reps=50)
        extras["prefill_turbo3_spec_verify_3rows_1024_eager"] = {"us": round(t_ms * 1e3, 2)}
        del k3c, v3c, q3t, o3, w3
    if int8 is not None and want("int8_140k"):
        # the int8 prompt at the longer of the two contexts: 2048 queries at
        # the end of 140000 cells (leg "int8_140k")
        d8l = inputs.int8_prompt(seed=1, ctx=140000)
        tl = {k_: torch.from_numpy(v_).to(dev) for k_, v_ in d8l.items() if not k_.endswith("logical")}
        nql, nqhl, ddl = d8l["q"].shape
        q0l = 140000 - nql
        wsl = torch.empty(max(256, b.tq_attn_int8_prompt_workspace(nql, nqhl, 1, ddl, 140000)), dtype=torch.uint8,
                          device=dev)
        outl = torch.empty((nql, nqhl, ddl), dtype=torch.float32, device=dev)
        t_ms = time_eager(lambda: b.tq_attn_int8_prompt(tl["q"], tl["k8"], tl["v8"], tl["k_scale"], tl["v_scale"],
                                                        tl["page_table"], 140000, q0l, 1.0 / math.sqrt(ddl),
                                                        out=outl, workspace=wsl), reps=5)
        pairs_l = sum(min(140000, q0l + i + 1) for i in range(nql))
        tf = 4.0 * ddl * nqhl * pairs_l / (t_ms * 1e-3) / 1e12
        extras["int8_prompt_140k_2048q"] = {"ms": round(t_ms, 4), "TFLOPs": round(tf, 2),
                                            "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        del tl, outl, wsl
    if graph is not None:
        # sparse V at the pages' turbo3 threshold against the dense call, one
        # 32K cache, eager (launch overhead included in both)
        for tau in (0.0, 5e-3):
            t_ms = time_eager(lambda tau=tau: b.tq_attn_decode(kcs[0], vcs[0], KV, q_dec, scale_dec, out=outs[0],
                                                                workspace=ws, sparse_v_tau=tau), reps=50)
            extras[f"decode_eager_tau_{tau:g}"] = {"us_per_call": round(t_ms * 1e3, 3)}

        def time_graph(calls, reps=5):
            """ms per call of `calls` captured into one graph (warmed first)."""
            for c in calls:
                c()
            torch.cuda.synchronize()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                for c in calls:
                    c()
            torch.cuda.current_stream().wait_stream(st)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for c in calls:
                    c()
            gr.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps / len(calls)

        # 256-wide heads (16 q / 2 kv heads: the bytes of the headline call),
        # and a 256-wide K beside a 128-wide V, over L distinct 32K caches
        # (leg "decode_wide": left out of `--only decode`, whose kernel
        # profiles then hold the headline shape alone)
        for dk, dv in ((256, 256), (256, 128)) if want("decode_wide") else ():
            wq, wk, wv = inputs.outlier_decode(seed=7, kv_len=KV, n_q=16, n_kv=2, d=dk, dv=dv)
            wkc = [b.new_cache(3, dk, 2, KV) for _ in range(L)]
            wvc = [b.new_cache(3, dv, 2, KV) for _ in range(L)]
            b.tq_set_rows(wkc[0], torch.from_numpy(wk).to(dev), idx)
            b.tq_set_rows(wvc[0], torch.from_numpy(wv).to(dev), idx)
            for i in range(1, L):
                wkc[i].codes.copy_(wkc[0].codes); wkc[i].norms.copy_(wkc[0].norms)
                wvc[i].codes.copy_(wvc[0].codes); wvc[i].norms.copy_(wvc[0].norms)
            wqt = torch.from_numpy(wq).to(torch.bfloat16).to(dev)
            wws = torch.empty(b.tq_attn_decode_workspace(wkc[0], wvc[0], KV, 16), dtype=torch.uint8, device=dev)
            wout = [torch.empty((16, dv), dtype=torch.float32, device=dev) for _ in range(L)]
            calls = [lambda i=i: b.tq_attn_decode(wkc[i], wvc[i], KV, wqt, 1.0 / math.sqrt(dk), out=wout[i],
                                                  workspace=wws) for i in range(L)]
            t_ms = time_graph(calls)
            nbytes = KV * 2 * (dk // 128 + dv // 128) * (48 + 2)
            gbps = nbytes / (t_ms * 1e-3) / 1e9
            extras[f"decode_turbo3_32k_k{dk}_v{dv}_16q2kv"] = {
                "us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            del wkc, wvc, wout, wws

        # asymmetric cache of the headline shape (leg "decode_wide"): K in
        # the 8-bit block format beside the turbo3 V, 32 q / 4 kv heads, 32K
        if want("decode_wide"):
            akc = [b.new_cache(8, D, NKV, KV) for _ in range(L)]
            b.tq_set_rows(akc[0], k_src, idx)
            for i in range(1, L):
                akc[i].codes.copy_(akc[0].codes); akc[i].norms.copy_(akc[0].norms)
            aws = torch.empty(b.tq_attn_decode_workspace(akc[0], vcs[0], KV, NQ), dtype=torch.uint8, device=dev)
            calls = [lambda i=i: b.tq_attn_decode(akc[i], vcs[i], KV, q_dec, scale_dec, out=outs[i], workspace=aws)
                     for i in range(L)]
            t_ms = time_graph(calls)
            nbytes = KV * NKV * ((D + 2 * D // 32) + (48 + 2) * D // 128)
            gbps = nbytes / (t_ms * 1e-3) / 1e9
            extras["decode_q8k_turbo3v_32k_gqa8"] = {
                "us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            del akc, aws

        # one query row over a long sequence (leg "decode_long"): 131072
        # cells, 32 q / 4 kv heads, turbo3, L distinct caches (52 MB each),
        # so the launch cost is spread over four times the headline's bytes
        if want("decode_long"):
            LK = 131072
            lq, lk, lv = inputs.outlier_decode(seed=11, kv_len=LK)
            lidx = torch.arange(LK, dtype=torch.int64, device=dev)
            lkc = [b.new_cache(3, D, NKV, LK) for _ in range(L)]
            lvc = [b.new_cache(3, D, NKV, LK) for _ in range(L)]
            b.tq_set_rows(lkc[0], torch.from_numpy(lk).to(dev), lidx)
            b.tq_set_rows(lvc[0], torch.from_numpy(lv).to(dev), lidx)
            del lk, lv
            for i in range(1, L):
                lkc[i].codes.copy_(lkc[0].codes); lkc[i].norms.copy_(lkc[0].norms)
                lvc[i].codes.copy_(lvc[0].codes); lvc[i].norms.copy_(lvc[0].norms)
            lqt = torch.from_numpy(lq).to(torch.bfloat16).to(dev)
            lws = torch.empty(b.tq_attn_decode_workspace(lkc[0], lvc[0], LK, NQ), dtype=torch.uint8, device=dev)
            t_ms = time_graph([lambda i=i: b.tq_attn_decode(lkc[i], lvc[i], LK, lqt, scale_dec, out=outs[i],
                                                            workspace=lws) for i in range(L)])
            nbytes = 2 * NKV * LK * 50
            gbps = nbytes / (t_ms * 1e-3) / 1e9
            extras["decode_turbo3_131072_gqa8"] = {"us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes,
                                                   "GBps": round(gbps, 1),
                                                   "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            del lkc, lvc, lws

        # the two decode kernels side by side (leg "decode_paths"): the
        # matrix-core path and the Q x centroid table path of the decode
        # design on the pages, at 1, 2 and 8 q heads per kv head over 32768
        # cells and at one head over 256 cells
        if want("decode_paths"):
            for n_qh, n_kvh, kvl, LL in ((1, 1, 256, L), (8, 8, 32768, 12), (16, 8, 32768, 12), (NQ, NKV, KV, L)):
                pq_, pk_, pv_ = inputs.outlier_decode(seed=12, kv_len=kvl, n_q=n_qh, n_kv=n_kvh)
                pidx = torch.arange(kvl, dtype=torch.int64, device=dev)
                pkc = [b.new_cache(3, D, n_kvh, kvl) for _ in range(LL)]
                pvc = [b.new_cache(3, D, n_kvh, kvl) for _ in range(LL)]
                b.tq_set_rows(pkc[0], torch.from_numpy(pk_).to(dev), pidx)
                b.tq_set_rows(pvc[0], torch.from_numpy(pv_).to(dev), pidx)
                for i in range(1, LL):
                    pkc[i].codes.copy_(pkc[0].codes); pkc[i].norms.copy_(pkc[0].norms)
                    pvc[i].codes.copy_(pvc[0].codes); pvc[i].norms.copy_(pvc[0].norms)
                pqt = torch.from_numpy(pq_).to(torch.bfloat16).to(dev)
                pout = [torch.empty((n_qh, D), dtype=torch.float32, device=dev) for _ in range(LL)]
                nbytes = 2 * n_kvh * kvl * 50
                row = {"bytes_per_call": nbytes}
                for pname, path in (("matrix", b.TQ_DECODE_MATRIX), ("table", b.TQ_DECODE_TABLE)):
                    pws = torch.empty(b.tq_attn_decode_path_workspace(pkc[0], pvc[0], kvl, n_qh, path),
                                      dtype=torch.uint8, device=dev)
                    t_ms = time_graph([lambda i=i, path=path, pws=pws: b.tq_attn_decode_path(
                        pkc[i], pvc[i], kvl, pqt, scale_dec, path, out=pout[i], workspace=pws) for i in range(LL)])
                    row[f"{pname}_us"] = round(t_ms * 1e3, 3)
                    row[f"{pname}_GBps"] = round(nbytes / (t_ms * 1e-3) / 1e9, 1)
                extras[f"decode_paths_turbo3_{n_qh}q{n_kvh}kv_{kvl}"] = row
                del pkc, pvc, pout

        # turbo2 and turbo4 decode at the headline's heads, 8192 and 32768
        # cells (leg "decode_types"), over L distinct caches each
        if want("decode_types"):
            for bits in (2, 4):
                xkc = [b.new_cache(bits, D, NKV, KV) for _ in range(L)]
                xvc = [b.new_cache(bits, D, NKV, KV) for _ in range(L)]
                b.tq_set_rows(xkc[0], k_src, idx)
                b.tq_set_rows(xvc[0], v_src, idx)
                for i in range(1, L):
                    xkc[i].codes.copy_(xkc[0].codes); xkc[i].norms.copy_(xkc[0].norms)
                    xvc[i].codes.copy_(xvc[0].codes); xvc[i].norms.copy_(xvc[0].norms)
                xws = torch.empty(b.tq_attn_decode_workspace(xkc[0], xvc[0], KV, NQ), dtype=torch.uint8, device=dev)
                for kvl in (8192, KV):
                    t_ms = time_graph([lambda i=i, kvl=kvl: b.tq_attn_decode(xkc[i], xvc[i], kvl, q_dec, scale_dec,
                                                                             out=outs[i], workspace=xws)
                                       for i in range(L)])
                    nbytes = 2 * NKV * kvl * (16 * bits + 2)
                    gbps = nbytes / (t_ms * 1e-3) / 1e9
                    extras[f"decode_turbo{bits}_{kvl}_gqa8"] = {
                        "us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
                del xkc, xvc, xws
            t_ms = time_graph([lambda i=i: b.tq_attn_decode(kcs[i], vcs[i], 8192, q_dec, scale_dec, out=outs[i],
                                                            workspace=ws) for i in range(L)])
            nbytes = 2 * NKV * 8192 * 50
            gbps = nbytes / (t_ms * 1e-3) / 1e9
            extras["decode_turbo3_8192_gqa8"] = {"us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes,
                                                 "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}

        # batched decode (leg "decode_batch"): 8 sequences of mixed lengths
        # (131,072 cells in all), 2 query rows each, 32 q / 4 kv heads, one
        # call per layer over L layer caches in one graph; beside it the same
        # sequences as 8 single-row calls per layer (one row each)
        if want("decode_batch"):
            lens = [32768, 16384, 8192, 4096, 30000, 2000, 12000, 25632]
            starts = np.cumsum([0] + lens[:-1]).tolist()
            NC = int(sum(lens))
            bq_np, bk_np, bv_np = inputs.outlier_decode(seed=8, kv_len=NC)
            bkc = [b.new_cache(3, D, NKV, NC) for _ in range(L)]
            bvc = [b.new_cache(3, D, NKV, NC) for _ in range(L)]
            bidx = torch.arange(NC, dtype=torch.int64, device=dev)
            b.tq_set_rows(bkc[0], torch.from_numpy(bk_np).to(dev), bidx)
            b.tq_set_rows(bvc[0], torch.from_numpy(bv_np).to(dev), bidx)
            for i in range(1, L):
                bkc[i].codes.copy_(bkc[0].codes); bkc[i].norms.copy_(bkc[0].norms)
                bvc[i].codes.copy_(bvc[0].codes); bvc[i].norms.copy_(bvc[0].norms)
            rng = np.random.default_rng(9)
            bq = torch.from_numpy(inputs.bf16_round(rng.standard_normal((8, 2, NQ, D)).astype(np.float32)))
            bq = bq.to(torch.bfloat16).to(dev)
            st = torch.tensor(starts, dtype=torch.int64, device=dev)
            ln = torch.tensor(lens, dtype=torch.int32, device=dev)
            MAXL = max(lens)
            bws = torch.empty(b.tq_attn_decode_batch_workspace(bkc[0], bvc[0], 8, 2, MAXL, NQ), dtype=torch.uint8,
                              device=dev)
            bout = [torch.empty((8, 2, NQ, D), dtype=torch.float32, device=dev) for _ in range(L)]
            calls = [lambda i=i: b.tq_attn_decode_batch(bkc[i], bvc[i], st, ln, MAXL, bq, scale_dec, out=bout[i],
                                                        workspace=bws) for i in range(L)]
            t_ms = time_graph(calls)
            nbytes = NC * NKV * 2 * (48 + 2)
            gbps = nbytes / (t_ms * 1e-3) / 1e9
            extras["decode_batch_8seq_2rows_131k_cells"] = {
                "us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": nbytes, "GBps": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            # the same cells through single-sequence calls (one row each)
            def seq_cache(c, a, n):
                x = b.new_cache(3, D, NKV, n)
                x.codes.copy_(c.codes[:, a:a + n])
                x.norms.copy_(c.norms[:, a:a + n])
                return x
            sk = [[seq_cache(c, a, n) for a, n in zip(starts, lens)] for c in bkc]
            sv = [[seq_cache(c, a, n) for a, n in zip(starts, lens)] for c in bvc]
            sws = torch.empty(max(b.tq_attn_decode_workspace(sk[0][j], sv[0][j], lens[j], NQ) for j in range(8)),
                              dtype=torch.uint8, device=dev)
            sq = bq[:, 1].contiguous()
            sout = torch.empty((NQ, D), dtype=torch.float32, device=dev)
            scalls = [lambda i=i, j=j: b.tq_attn_decode(sk[i][j], sv[i][j], lens[j], sq[j], scale_dec, out=sout,
                                                        workspace=sws) for i in range(L) for j in range(8)]
            t_ms = time_graph(scalls) * 8
            extras["decode_8_single_calls_1row_131k_cells"] = {
                "us_per_layer": round(t_ms * 1e3, 3), "GBps": round(nbytes / (t_ms * 1e-3) / 1e9, 1)}
            del bkc, bvc, bout, sk, sv
            # two rows (speculative verify) over one 32K sequence of the
            # headline caches: 32 (row, head) pairs, two workgroups of sixteen
            st2 = torch.tensor([0], dtype=torch.int64, device=dev)
            ln2 = torch.tensor([KV], dtype=torch.int32, device=dev)
            q2 = torch.from_numpy(inputs.bf16_round(rng.standard_normal((1, 2, NQ, D)).astype(np.float32)))
            q2 = q2.to(torch.bfloat16).to(dev)
            ws2 = torch.empty(b.tq_attn_decode_batch_workspace(kcs[0], vcs[0], 1, 2, KV, NQ), dtype=torch.uint8,
                              device=dev)
            out2 = [torch.empty((1, 2, NQ, D), dtype=torch.float32, device=dev) for _ in range(L)]
            t_ms = time_graph([lambda i=i: b.tq_attn_decode_batch(kcs[i], vcs[i], st2, ln2, KV, q2, scale_dec,
                                                                  out=out2[i], workspace=ws2) for i in range(L)])
            gbps = kv_bytes_per_call / (t_ms * 1e-3) / 1e9
            extras["decode_2rows_32k_gqa8"] = {"us_per_call": round(t_ms * 1e3, 3), "bytes_per_call": kv_bytes_per_call,
                                               "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            del out2, ws2

        # launch and streaming floors (leg "floor"): what one graph-replayed
        # launch of an empty kernel costs, and a kernel that only reads the
        # decode call's bytes once (L distinct buffers, no arithmetic), alone
        # and followed by a second, tiny launch as the split + merge pair is
        fl = None
        if want("floor"):
            import ctypes
            try:
                fl = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(b.__file__)), "lib", "libtq_floor.so"))
            except OSError as e:
                log(f"[bench] floor leg skipped (build the package first): {e}")
        if fl is not None:
            fl.tqf_empty.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            fl.tqf_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            fbufs = [torch.full((kv_bytes_per_call,), i, dtype=torch.uint8, device=dev) for i in range(L)]
            fout = torch.empty(1024 * 64, dtype=torch.float32, device=dev)

            def fcall(rc):
                if rc != 0:
                    raise RuntimeError(f"floor kernel launch failed: hipError {rc}")

            def fs():
                return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            t_ms = time_graph([lambda: fcall(fl.tqf_empty(256, ctypes.c_void_p(fout.data_ptr()), fs()))] * L)
            extras["floor_empty_kernel_256wg"] = {"us_per_launch": round(t_ms * 1e3, 3)}
            for grid in (256, 1024):
                t_ms = time_graph([lambda i=i: fcall(fl.tqf_read(ctypes.c_void_p(fbufs[i].data_ptr()),
                                                                  kv_bytes_per_call, grid,
                                                                  ctypes.c_void_p(fout.data_ptr()), fs()))
                                   for i in range(L)])
                gbps = kv_bytes_per_call / (t_ms * 1e-3) / 1e9
                extras[f"floor_read_{kv_bytes_per_call}B_{grid}wg"] = {
                    "us_per_call": round(t_ms * 1e3, 3), "GBps": round(gbps, 1),
                    "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            t_ms = time_graph([lambda i=i: (fcall(fl.tqf_read(ctypes.c_void_p(fbufs[i].data_ptr()), kv_bytes_per_call,
                                                              1024, ctypes.c_void_p(fout.data_ptr()), fs())),
                                            fcall(fl.tqf_empty(32, ctypes.c_void_p(fout.data_ptr()), fs())))
                               for i in range(L)])
            gbps = kv_bytes_per_call / (t_ms * 1e-3) / 1e9
            extras[f"floor_read_{kv_bytes_per_call}B_then_empty_launch"] = {
                "us_per_call": round(t_ms * 1e3, 3), "GBps": round(gbps, 1),
                "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            del fbufs
    log("[bench] extras done")

    # every leg's time is the median over the timed steps (its mean beside it)
    ms = {n: legs[n].median_ms() for n in legs}
    ms_mean = {n: legs[n].mean_ms() for n in legs}
    step_ms = sum(v_ for n_, v_ in ms.items() if v_ is not None and n_ != "copy")
    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "f16 hi+lo split operands, f32 accumulate (prefill: single f16 operands)",
           "data": "synthetic",
           "config": {"workload": f"turbo3 decode: 32 q / 4 kv heads, head_dim 128, kv 32768, bf16 q, "
                                  f"{L} layers' caches per step; + set_rows of one 32768-row cache, "
                                  f"turbo3 causal prefill 2048 rows (16 q / 8 kv, d 256), "
                                  f"int8 prompt 2048 q x 40000 ctx",
                      "global_batch": 1, "seq_len": KV, "parallelism": "none (1 GPU)"},
           "wall_ms_per_step": round(wall_ms, 4)}
    if ms["decode"] is not None:
        per_call_us = ms["decode"] * 1e3 / L
        gbps = kv_bytes_per_call / (per_call_us * 1e-6) / 1e9
        out["value"] = round(gbps, 2)
        out["decode"] = {"us_per_call": round(per_call_us, 3), "kv_bytes_per_call": kv_bytes_per_call,
                         "GBps": round(gbps, 2), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                         "layers_per_step": L, "us_per_call_mean": round(ms_mean["decode"] * 1e3 / L, 3)}
        out["roofline"] = {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                           "traffic": decode_traffic_bytes(),
                           "kernel": "decode call (decode_fused_kernel + decode_merge_kernel), "
                                     "algorithmic bytes = packed K+V codes and norms"}
    if ms["set_rows"] is not None:
        per_cache_us = ms["set_rows"] * 1e3
        nbytes = 2 * (KV * NKV * D * 4 + KV * NKV * 50)
        out["set_rows"] = {"us_per_32k_KV_pair": round(per_cache_us, 2), "bytes": nbytes,
                           "GBps": round(nbytes / (per_cache_us * 1e-6) / 1e9, 1)}
    if ms["prefill"] is not None:
        t_s = ms["prefill"] * 1e-3
        tflops = prefill["flops"] / t_s / 1e12
        out["prefill"] = {"rows": prefill["rows"], "us": round(ms["prefill"] * 1e3, 2),
                          "tokens_per_s": round(prefill["rows"] / t_s, 1),
                          "TFLOPs": round(tflops, 2), "frac_mfma_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}
    if ms["int8"] is not None:
        t_s = ms["int8"] * 1e-3
        tflops = int8["flops"] / t_s / 1e12
        # the products run on float16 matrix cores with hi and lo operand
        # parts: twice the algorithmic flops are executed
        out["int8_prompt"] = {"ctx": int8["ctx"], "n_q": int8["n_q"], "ms": round(ms["int8"], 4),
                              "TFLOPs": round(tflops, 2),
                              "frac_mfma_f16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                              "frac_mfma_f16_peak_executed": round(2 * tflops / MFMA_F16_PEAK_TFLOPS, 4)}

    if ms["copy"] is not None:
        out["calibration_copy"] = {"bytes_read": copy["nbytes"], "bytes_written": copy["nbytes"],
                                   "us": round(ms["copy"] * 1e3, 2),
                                   "GBps_read_plus_write": round(2 * copy["nbytes"] / (ms["copy"] * 1e-3) / 1e9, 1)}

    # ---------------- CPU baseline and parity: the oracle on bounded samples
    if not args.no_cpu_baseline and want("decode"):
        out.update(oracle_leg(b, torch, dev, inputs, k_np, v_np, q_np, kcs[0], vcs[0], q_dec, ws,
                              scale_dec, kv_bytes_per_call, prefill, int8, snap,
                              (pq, pk, pv) if prefill is not None else None,
                              d8 if int8 is not None else None))
    if extras:
        out["extras"] = extras
    out["wall_s_total"] = round(time.time() - t_wall0, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
