#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: a single
``attn_fwd`` launch (bf16, non-causal) on the FlashAttention-3 ablation shape
(batch 4, seq 8448, 16 heads, head_dim 128).  Inputs are seeded N(0,1) bf16,
resident in HBM before the timed region.  The line also carries the 8-bit path
(quantised inputs, attention kernel alone) on batch 4 / 16 heads / seq 8192 /
d128 when that path is available, the roofline position of the timed kernel and
the float64 CPU oracle timed on a bounded sample of the same workload.

Prints ONE JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0

# sources of the timed kernel; the committed counter summary names their hash
KERNEL_SOURCES = ("attention_attn_fwd_10_amd/csrc/fwd16.hpp", "attention_attn_fwd_10_amd/csrc/common.hpp",
                  "attention_attn_fwd_10_amd/csrc/args.hpp", "attention_attn_fwd_10_amd/csrc/ring.hpp",
                  "attention_attn_fwd_10_amd/csrc/fwd16_d128.hip", "attention_attn_fwd_10_amd/csrc/splitkv.hip",
                  "attention_attn_fwd_10_amd/csrc/api.cpp")
TRAFFIC_PROFILE = "profiles/fwd16_d128_bf16_b4_h16_s8448.md"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, scaled by the factors measured on a plain copy; None when the
    summary was taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip().lstrip("-").strip()
        if ":" in line and line.startswith(("source_sha256", "fetch_kib", "write_kib", "fetch_scale", "write_scale")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    try:
        if vals.get("source_sha256") != kernel_source_hash():
            return None
        return (float(vals["fetch_kib_per_launch"]) * float(vals["fetch_scale"]) +
                float(vals["write_kib_per_launch"]) * float(vals["write_scale"])) * 1024.0
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--causal", action="store_true", help="time the causal variant instead")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp8", action="store_true")
    p.add_argument("--no-int8", action="store_true", help="skip the int8-score leg")
    p.add_argument("--no-bwd", action="store_true", help="skip the backward-pass leg")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--sweep", action="store_true", help="also time the 16384-token seq sweep (extra output)")
    p.add_argument("--no-decode", action="store_true", help="skip the long-cache decoding leg")
    p.add_argument("--no-bias", action="store_true", help="skip the additive-bias leg")
    p.add_argument("--no-points", action="store_true",
                   help="skip the extra workload points (seq-8192 headline, seq-512 GB/s, varlen+paged, causal fp8)")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes and clock")
    p.add_argument("--source-hash", action="store_true", help="print the timed kernel's source hash and exit")
    p.add_argument("--short-points", action="store_true",
                   help="only the short-sequence points (seq 512 at d64/128/256, causal and not) and the varlen "
                        "workload, --warmup then --steps launches each, one JSON line (for counter passes)")
    p.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (calibrates the FETCH_SIZE/WRITE_SIZE counters)")
    return p.parse_args()


def copy_reference(mib):
    """A plain device-to-device copy of known size, run a few times: the HBM
    byte counters read on it give the scale applied to the kernel's readings."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_read": n * 4, "copy_reference_bytes_written": n * 4}))


def time_launches(fn, steps, warmup):
    """Average duration of ``fn`` (one launch on torch's current stream) with HIP
    events bracketing exactly ``steps`` launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, target_s):
    """The float64 oracle (three-pass definition) on whole heads of the same
    workload until about ``target_s`` seconds of CPU work have run.  `cores`
    is the number of BLAS threads the oracle ran on; the host's own core count
    and CPU model are reported beside it."""
    from oracle import attention as OA
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    flops_head = 4.0 * w.seq_q * w.seq_k * w.head_dim / (2 if w.causal else 1)
    t0 = time.perf_counter()
    n = 0
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    while n < len(pairs):
        b, h = pairs[n]
        OA.naive_head(q[b, :, h], k[b, :, h], v[b, :, h], w.scale, w.causal)
        n += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    out = {"value": n * flops_head / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{n} of {len(pairs)} (batch, head) pairs of {w.name}, all rows, float64 numpy "
                     f"three-pass, {dt:.1f} s",
           "host_nproc": os.cpu_count(), "host_affinity_cpus": len(os.sched_getaffinity(0)),
           "cpu_model": cpu_model()}
    # one (batch, head) on one core, beside the threaded figure
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            t1 = time.perf_counter()
            OA.naive_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], w.scale, w.causal)
            out["single_core_s_per_head"] = round(time.perf_counter() - t1, 3)
    except Exception as e:  # pragma: no cover
        out["single_core_s_per_head"] = f"unavailable: {e}"
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    import torch
    import attention_attn_fwd_10_amd as A
    import workloads as W

    if args.short_points:
        print(json.dumps(short_points(A, W, args)), flush=True)
        return

    w = W.WORKLOADS["ablation"]
    if args.causal:
        w = W.Workload(w.name + "_causal", w.batch, w.heads, w.seq_q, w.seq_k, w.head_dim, True, w.seed)
    qs, ks = w.shapes()
    qh, kh, vh = W.qkv_normal(w.seed, qs, ks)
    dev = "cuda"
    q = torch.from_numpy(qh).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(kh).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(vh).to(torch.bfloat16).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device=dev)
    print(f"[bench] inputs ready: {w.name}", file=sys.stderr, flush=True)

    ms = time_launches(lambda: A.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse), args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    algo_bytes = 2 * (2 * w.batch * w.seq_q * w.heads * w.head_dim + 2 * w.batch * w.seq_k * w.heads * w.head_dim) \
        + 4 * w.batch * w.heads * w.seq_q
    print(f"[bench] bf16 fwd {ms:.3f} ms  {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    result = {
        "metric": "attn fwd TFLOPs/s at d128 seq 8k (bf16, fp8) + % of MI355X MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) rounded to bf16, device-resident",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_q": w.seq_q, "seq_k": w.seq_k,
                   "head_dim": w.head_dim, "causal": w.causal, "flops_per_step": w.flops,
                   "flop_convention": "4*B*H*Sq*Sk*D, halved for causal"},
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic(),
                     "kernel": "fwd16_kernel<128, bf16, non-causal, dense wide> (256-row workgroups; the "
                               "step also runs the split tail's merge)",
                     "algorithmic_bytes": algo_bytes},
    }

    if not args.no_fp8:
        result["fp8"] = bench_fp8(A, W, args)

    if not args.no_int8:
        result["int8"] = bench_int8(A, W, args)

    if not args.no_bwd:
        result["bwd"] = bench_bwd(A, W, args, q, k, v, o, lse)

    if not args.no_decode:
        result["decode"] = bench_decode(A, W, args)

    if not args.no_bias:
        result["bias"] = bench_bias(A, W, args)

    if not args.no_points:
        result["points"] = bench_points(A, W, args)

    if not args.no_ceilings:
        result["ceilings"] = measured_ceilings(result)

    if args.sweep:
        result["sweep"] = bench_sweep(A, W, args)

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, qh, kh, vh, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_fp8(A, W, args):
    import torch
    w = W.WORKLOADS["fp8"]
    qs, _ = w.shapes()
    qh, kh, vh = W.qkv_outlier(w.seed, qs)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (qh, kh, vh))
    signs = torch.from_numpy(W.random_signs(4, w.head_dim)).cuda()
    try:
        q8, qsc = A.fp8_quantize(q, 128, signs)
        k8, ksc = A.fp8_quantize(k, 128, signs)
        v8, vsc = A.fp8_quantize(v, 128, None)
        o = torch.empty((w.batch, w.seq_q, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: A.fwd_fp8(q8, qsc, k8, ksc, v8, vsc, 128, w.scale, False, out=o, lse=lse),
                           args.steps, args.warmup)
        ms_q = time_launches(lambda: A.fp8_quantize(q, 128, signs, out=q8, scales=qsc), args.steps, 2)
        # the power-of-two form of the same workload (block scales applied in the MFMAs)
        q8, qsc = A.fp8_quantize_pow2_q(q, w.scale, 128, signs, out=q8, scales=qsc)
        k8, ksc = A.fp8_quantize_pow2(k, 128, signs, out=k8, scales=ksc)
        v8, vsc = A.fp8_quantize_pow2(v, 128, None, out=v8, scales=vsc)
        ms_p2 = time_launches(lambda: A.fwd_fp8_pow2(q8, qsc, k8, ksc, v8, vsc, 128, False, out=o, lse=lse),
                              args.steps, args.warmup)
    except A.AttnError as e:
        return {"available": False, "reason": str(e)}
    tflops = w.flops / (ms * 1e-3) / 1e12
    tf_p2 = w.flops / (ms_p2 * 1e-3) / 1e12
    q_bytes = 2 * q.numel() + q.numel() + 4 * qsc.numel()
    print(f"[bench] fp8 fwd {ms:.3f} ms  {tflops:.1f} TFLOP/s; power-of-two scales {ms_p2:.3f} ms "
          f"{tf_p2:.1f} TFLOP/s", file=sys.stderr, flush=True)
    return {"available": True, "workload": w.name, "ms": round(ms, 4), "tflops": round(tflops, 2),
            "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2), "peak": PEAK_FP8_TFLOPS,
            "quantize_ms_per_tensor": round(ms_q, 4),
            "quantize_gbs": round(q_bytes / (ms_q * 1e-3) / 1e9, 1),
            "end_to_end_ms": round(ms + 3 * ms_q, 4),
            "pow2_scales": {"ms": round(ms_p2, 4), "tflops": round(tf_p2, 2),
                            "pct_of_peak": round(100 * tf_p2 / PEAK_FP8_TFLOPS, 2)}}


def bench_int8(A, W, args):
    """int8 Q/K (block scales + rotation), e4m3 V, on the 8-bit workload;
    int8 and fp8 share the dense 5.0 POP/s peak."""
    import torch
    w = W.WORKLOADS["fp8"]
    qs, _ = w.shapes()
    qh, kh, vh = W.qkv_outlier(w.seed, qs)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (qh, kh, vh))
    signs = torch.from_numpy(W.random_signs(4, w.head_dim)).cuda()
    try:
        q8, qsc = A.int8_quantize(q, 128, signs)
        k8, ksc = A.int8_quantize(k, 128, signs)
        v8, vsc = A.fp8_quantize(v, 128, None)
        o = torch.empty((w.batch, w.seq_q, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: A.fwd_int8(q8, qsc, k8, ksc, v8, vsc, 128, w.scale, False, out=o, lse=lse),
                           args.steps, args.warmup)
        ms_q = time_launches(lambda: A.int8_quantize(q, 128, signs, out=q8, scales=qsc), args.steps, 2)
    except A.AttnError as e:
        return {"available": False, "reason": str(e)}
    tflops = w.flops / (ms * 1e-3) / 1e12
    print(f"[bench] int8 fwd {ms:.3f} ms  {tflops:.1f} TOP/s", file=sys.stderr, flush=True)
    return {"available": True, "workload": w.name, "ms": round(ms, 4), "tops": round(tflops, 2),
            "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2), "peak": PEAK_FP8_TFLOPS,
            "quantize_ms_per_tensor": round(ms_q, 4)}


def bench_bwd(A, W, args, q, k, v, o, lse):
    """attn_bwd on the headline shape (the forward's o and lse as inputs),
    dO ~ N(0,1); FLOPs = 2.5x the forward's (five Sq x Sk x D products)."""
    import torch
    w = W.WORKLOADS["ablation"]
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(w.seed + 1000)).to(torch.bfloat16).cuda()
    A.fwd(q, k, v, w.scale, False, out=o, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((2, w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
    steps = max(3, args.steps // 3)
    ms = time_launches(lambda: A.bwd(q, k, v, o, lse, dout, w.scale, False, dq=dq, dk=dk, dv=dv, workspace=ws),
                       steps, max(2, args.warmup // 3))
    flops = 2.5 * 4.0 * w.batch * w.heads * w.seq_q * w.seq_k * w.head_dim
    tflops = flops / (ms * 1e-3) / 1e12
    # the causal backward beside it (its own forward outputs; FLOPs halved)
    oc, lc = torch.empty_like(o), torch.empty_like(lse)
    A.fwd(q, k, v, w.scale, True, out=oc, lse=lc)
    ms_c = time_launches(lambda: A.bwd(q, k, v, oc, lc, dout, w.scale, True, dq=dq, dk=dk, dv=dv, workspace=ws),
                         steps, max(2, args.warmup // 3))
    tflops_c = flops / 2 / (ms_c * 1e-3) / 1e12
    print(f"[bench] bwd {ms:.3f} ms  {tflops:.1f} TFLOP/s; causal {ms_c:.3f} ms  {tflops_c:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    return {"workload": w.name, "causal": False, "ms": round(ms, 4), "tflops": round(tflops, 2),
            "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
            "ms_causal": round(ms_c, 4), "tflops_causal": round(tflops_c, 2),
            "flop_convention": "10*B*H*Sq*Sk*D (2.5x the forward), halved for causal", "steps": steps}


def bench_decode(A, W, args):
    """One query row per sequence over a long paged cache: the whole-sequence
    kernel (attn_fwd_varlen, one work item per sequence and head) against the
    split-key path (attn_fwd_splitkv).  HBM-bound: reported in GB/s of K and V
    read."""
    import torch
    cfg = W.DECODE
    B, Lq, Lk, H, D, page = (cfg[x] for x in ("n_seq", "seq_q", "seq_k", "heads", "head_dim", "page_size"))
    lens_q, lens_k = [Lq] * B, [Lk] * B
    table, npages = W.paged_layout(cfg["seed_pages"], lens_k, page)
    g = torch.Generator(device="cuda").manual_seed(cfg["seed_values"])
    q = torch.randn((B * Lq, H, D), generator=g, device="cuda").to(torch.bfloat16)
    kp, vp = (torch.randn((npages, page, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(2))
    cu_q = torch.from_numpy(W.cu_seqlens(lens_q)).cuda()
    cu_k = torch.from_numpy(W.cu_seqlens(lens_k)).cuda()
    tab = torch.from_numpy(table).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((H, B * Lq), dtype=torch.float32, device="cuda")
    splits = A.auto_num_splits(B, H, D, B * Lq, Lq, Lk, page)
    ws = torch.empty(A._lib.attn_fwd_splitkv_workspace_bytes(B * Lq, H, D, splits) // 4 + 4, dtype=torch.float32,
                     device="cuda")
    kv_bytes = 2 * B * Lk * H * D * 2
    algo = kv_bytes + 2 * 2 * B * Lq * H * D + 4 * H * B * Lq + 4 * table.size
    steps = max(5, args.steps // 3)
    ms_whole = time_launches(lambda: A.fwd_varlen(q, cu_q, kp, vp, cu_k, Lq, Lk, None, cfg["causal"],
                                                  block_table=tab, page_size=page, out=o, lse=lse), steps, 10)
    ms_split = time_launches(lambda: A.fwd_splitkv(q, cu_q, kp, vp, cu_k, Lq, Lk, None, cfg["causal"],
                                                   block_table=tab, page_size=page, num_splits=splits, out=o,
                                                   lse=lse, workspace=ws), steps, 10)
    gbs = algo / (ms_split * 1e-3) / 1e9
    print(f"[bench] decode: whole {ms_whole:.3f} ms, split x{splits} {ms_split:.3f} ms ({gbs:.0f} GB/s)",
          file=sys.stderr, flush=True)
    return {"workload": f"decode_paged{page}_b{B}_h{H}_sk{Lk}_d{D}", "splits": splits,
            "ms_whole_sequence": round(ms_whole, 4), "ms_split": round(ms_split, 4),
            "gbs_split": round(gbs, 1), "gbs_whole_sequence": round(algo / (ms_whole * 1e-3) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * gbs / 8000.0, 1), "algorithmic_bytes": algo}


def bench_bias(A, W, args):
    """Additive score bias (attn_fwd_bias) on batch 1 x seq 8192 x 16 heads x
    d128: a full [B, H, Sq, Sk] bf16 bias (2 GiB read once) and a per-(head,
    key) bias broadcast over queries, beside the same problem without bias."""
    import torch
    B, S, H, D = 1, 8192, 16, 128
    g = torch.Generator(device="cuda").manual_seed(21)
    q, k, v = (torch.randn((B, S, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    full = torch.randn((B, H, S, S), generator=g, device="cuda").to(torch.bfloat16)
    per_key = torch.randn((1, H, 1, S), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    flops = 4.0 * B * H * S * S * D
    steps = max(5, args.steps // 3)
    out = {"workload": f"bias_b{B}_h{H}_s{S}_d{D}"}
    ms0 = time_launches(lambda: A.fwd(q, k, v, None, False, out=o, lse=lse), steps, 10)
    out["ms_no_bias"] = round(ms0, 4)
    for name, bias in (("full", full), ("per_head_key", per_key)):
        ms = time_launches(lambda: A.fwd_bias(q, k, v, bias, None, False, out=o, lse=lse), steps, 10)
        out[f"ms_{name}"] = round(ms, 4)
        out[f"tflops_{name}"] = round(flops / (ms * 1e-3) / 1e12, 1)
        print(f"[bench] bias {name}: {ms:.3f} ms ({flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s; no bias {ms0:.3f} ms)",
              file=sys.stderr, flush=True)
    out["full_bias_bytes"] = full.numel() * 2
    out["full_bias_gbs"] = round(full.numel() * 2 / (out["ms_full"] * 1e-3) / 1e9, 1)
    del full
    return out


def bench_points(A, W, args):
    """The other workload points the metric and the pages single out, each
    timed with HIP events on device-resident inputs drawn from its seed:
    the d128 seq-8k headline point of the 16384-token sweep (batch 2, 16
    heads, non-causal), the seq-512 d128 points in GB/s (HBM-bound), the
    varlen + paged workload (packed and with 64-token pages), and the 8-bit
    kernel under a causal mask and on the seq-512 shape."""
    import torch
    steps = max(5, args.steps // 3)
    out = {}
    pts = {p.name: p for p in W.seq_sweep_points()}
    for name in ("sweep_s8192_d128_full", "sweep_s8192_d128_causal", "sweep_s512_d128_full",
                 "sweep_s512_d128_causal"):
        w = pts[name]
        qs, _ = w.shapes()
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        q, k, v = (torch.randn(qs, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: A.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse), steps, 10)
        tf = w.flops / (ms * 1e-3) / 1e12
        byts = 4 * q.numel() * 2 + 4 * w.batch * w.heads * w.seq_q
        out[name] = {"batch": w.batch, "heads": w.heads, "seq": w.seq_q, "head_dim": w.head_dim,
                     "causal": w.causal, "ms": round(ms, 4), "tflops": round(tf, 1),
                     "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                     "gbs": round(byts / (ms * 1e-3) / 1e9, 1), "pct_of_hbm_peak": round(100 * byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)}
        print(f"[bench] {name}: {ms:.3f} ms {tf:.1f} TFLOP/s {out[name]['gbs']} GB/s", file=sys.stderr, flush=True)
        del q, k, v, o
    out["varlen_paged"] = bench_varlen(A, W, steps)
    out["fp8_causal"] = bench_fp8_causal(A, W, steps)
    out["fp8_s512"] = bench_fp8_short(A, W, pts["sweep_s512_d128_full"], steps)
    return out


def short_points(A, W, args):
    """The short-sequence points of the 16384-token sweep (seq 512: 32
    sequences, 16 heads, d64/128/256, causal and not) and the varlen workload
    (packed and paged), timed with HIP events; algorithmic bytes are Q, K, V
    read and O, LSE written once.  In launch order, so that a counter pass
    over this run maps its dispatches to the points."""
    import torch
    out = {"metric": "short-sequence forward, algorithmic GB/s", "steps": args.steps, "warmup": args.warmup,
           "points": {}}
    for w in W.seq_sweep_points():
        if w.seq_q != 512:
            continue
        qs, _ = w.shapes()
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        q, k, v = (torch.randn(qs, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: A.fwd(q, k, v, w.scale, w.causal, out=o, lse=lse), args.steps, args.warmup)
        byts = 4 * q.numel() * 2 + 4 * w.batch * w.heads * w.seq_q
        out["points"][w.name] = {"ms": round(ms, 4), "algorithmic_bytes": byts,
                                 "gbs": round(byts / (ms * 1e-3) / 1e9, 1)}
        print(f"[bench] {w.name}: {ms:.4f} ms {out['points'][w.name]['gbs']} GB/s", file=sys.stderr, flush=True)
        del q, k, v, o
    out["varlen_paged"] = bench_varlen(A, W, args.steps, args.warmup)
    return out


def bench_varlen(A, W, steps, warmup=10):
    """32 sequences U{128..4096} (seed 5), 32 heads, d128, causal: packed and
    with 64-token pages at permuted slots."""
    import torch
    cfg = W.VARLEN
    lens = W.varlen_lengths(cfg["seed_lengths"], cfg["n_seq"], cfg["lo"], cfg["hi"])
    H, D, page = cfg["heads"], cfg["head_dim"], cfg["page_size"]
    cu = torch.from_numpy(W.cu_seqlens(lens)).cuda()
    tot = int(lens.sum())
    g = torch.Generator(device="cuda").manual_seed(cfg["seed_values"])
    q, k, v = (torch.randn((tot, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    table, npages = W.paged_layout(cfg["seed_pages"], lens, page)
    # scatter every sequence's keys into its pages (one gather index per token)
    cuh = W.cu_seqlens(lens)
    dst = np.concatenate([table[b, np.arange(int(n)) // page] * page + np.arange(int(n)) % page
                          for b, n in enumerate(lens)])
    src = np.concatenate([cuh[b] + np.arange(int(n)) for b, n in enumerate(lens)])
    kp = torch.zeros((npages * page, H, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    di, si = torch.from_numpy(dst.astype(np.int64)).cuda(), torch.from_numpy(src.astype(np.int64)).cuda()
    kp[di] = k[si]
    vp[di] = v[si]
    kp, vp = kp.view(npages, page, H, D), vp.view(npages, page, H, D)
    tab = torch.from_numpy(table).cuda()
    flops = sum(4.0 * H * int(n) * int(n) * D / 2 for n in lens)
    mx = int(lens.max())
    o = torch.empty_like(q)
    lse = torch.empty((H, tot), dtype=torch.float32, device="cuda")
    byts = 4 * tot * H * D * 2 + 4 * H * tot  # Q, K, V read, O written (bf16); LSE (fp32)
    res = {"workload": f"varlen_32seq_u128_4096_h{H}_d{D}_causal", "tokens": tot, "flops": flops,
           "algorithmic_bytes": byts}
    for name, kk, vv, bt in (("packed", k, v, None), ("paged64", kp, vp, tab)):
        ms = time_launches(lambda: A.fwd_varlen(q, cu, kk, vv, cu, mx, mx, None, True, block_table=bt,
                                                page_size=page if bt is not None else 0, out=o, lse=lse),
                           steps, warmup)
        tf = flops / (ms * 1e-3) / 1e12
        res[f"ms_{name}"] = round(ms, 4)
        res[f"tflops_{name}"] = round(tf, 1)
        res[f"gbs_{name}"] = round(byts / (ms * 1e-3) / 1e9, 1)
        print(f"[bench] varlen {name}: {ms:.3f} ms {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    return res


def bench_fp8_causal(A, W, steps):
    """The 8-bit kernel with a causal mask on the 8-bit workload shape
    (quantised inputs; FLOPs halved)."""
    import torch
    w = W.WORKLOADS["fp8"]
    qs, _ = w.shapes()
    qh, kh, vh = W.qkv_outlier(w.seed, qs)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (qh, kh, vh))
    signs = torch.from_numpy(W.random_signs(4, w.head_dim)).cuda()
    q8, qsc = A.fp8_quantize(q, 128, signs)
    k8, ksc = A.fp8_quantize(k, 128, signs)
    v8, vsc = A.fp8_quantize(v, 128, None)
    del q, k, v
    o = torch.empty((w.batch, w.seq_q, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
    ms = time_launches(lambda: A.fwd_fp8(q8, qsc, k8, ksc, v8, vsc, 128, w.scale, True, out=o, lse=lse), steps, 10)
    tf = w.flops / 2 / (ms * 1e-3) / 1e12
    print(f"[bench] fp8 causal: {ms:.3f} ms {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    return {"workload": w.name + "_causal", "ms": round(ms, 4), "tflops": round(tf, 1),
            "pct_of_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2)}


def bench_fp8_short(A, W, w, steps):
    """The 8-bit kernel (block-128 scales, rotated Q and K) on a short-sequence
    shape of the sweep, non-causal and causal, inputs drawn like the 8-bit
    workload's (0.1 % outliers); beside it the 16-bit kernel on the same
    shape is in the sweep point of that name."""
    import torch
    qs, _ = w.shapes()
    qh, kh, vh = W.qkv_outlier(w.seed, qs)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (qh, kh, vh))
    signs = torch.from_numpy(W.random_signs(4, w.head_dim)).cuda()
    q8, qsc = A.fp8_quantize(q, 128, signs)
    k8, ksc = A.fp8_quantize(k, 128, signs)
    v8, vsc = A.fp8_quantize(v, 128, None)
    del q, k, v
    o = torch.empty((w.batch, w.seq_q, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device="cuda")
    res = {"batch": w.batch, "heads": w.heads, "seq": w.seq_q, "head_dim": w.head_dim}
    for causal in (False, True):
        ms = time_launches(lambda: A.fwd_fp8(q8, qsc, k8, ksc, v8, vsc, 128, w.scale, causal, out=o, lse=lse),
                           steps, 10)
        tf = w.flops / (2 if causal else 1) / (ms * 1e-3) / 1e12
        key = "_causal" if causal else ""
        res["ms" + key] = round(ms, 4)
        res["tflops" + key] = round(tf, 1)
        res["pct_of_peak" + key] = round(100 * tf / PEAK_FP8_TFLOPS, 2)
        print(f"[bench] fp8 seq {w.seq_q}{' causal' if causal else ''}: {ms:.4f} ms {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    return res


def measured_ceilings(result):
    """Sustained clock, matrix-core rates and vector-instruction costs measured
    by libattn_probe.so on this GPU, and what they imply for the timed kernels:
    the datasheet peaks assume 2.4 GHz; the exp2-bound ceiling is the rate at
    which the chip evaluates one exponential per score (4 * D flops per score
    at D = 128)."""
    import ctypes
    path = os.path.join(ROOT, "attention_attn_fwd_10_amd", "libattn_probe.so")
    if not os.path.exists(path):
        return {"available": False, "reason": "libattn_probe.so not built"}
    lib = ctypes.CDLL(path)
    n = 32
    r = (ctypes.c_double * n)()
    rc = lib.attn_probe_ceilings(r, n)
    names = ["exp", "fma", "add", "max3", "cvt_pk_fp8", "cvt_pk_bf16", "rcp"]
    clock = r[10]
    cus = r[18]
    simds = 4 * cus
    out = {"ok": rc == 0, "clock_ghz": round(clock, 3), "cus": int(cus),
           "mfma_bf16_tflops": round(r[7] / 1e12, 1), "mfma_fp8_tflops": round(r[8] / 1e12, 1),
           "mfma_i8_tops": round(r[9] / 1e12, 1)}
    # cycles one wave64 instruction holds its SIMD's vector unit
    for i, nm in enumerate(names):
        out[f"{nm}_cycles_per_wave_instr"] = round(simds * clock * 1e9 * 64 / r[i], 2) if r[i] > 0 else None
    out["exp2_bound_ceiling_tflops_d128"] = round(r[0] * 4 * 128 / 1e12, 1)
    out["overlap_ms"] = {"one_wave_mfma": round(r[11], 4), "one_wave_exp16": round(r[12], 4),
                         "one_wave_mfma_plus_exp8": round(r[13], 4), "one_wave_mfma_plus_exp16": round(r[14], 4),
                         "two_waves_mfma": round(r[15], 4), "two_waves_exp": round(r[16], 4),
                         "two_waves_both": round(r[17], 4)}
    # the timed bf16 and fp8 kernels against the measured (not datasheet) matrix rates
    if clock > 0:
        out["bf16_frac_of_measured_mfma"] = round(result["value"] / (r[7] / 1e12), 4)
        if isinstance(result.get("fp8"), dict) and result["fp8"].get("available"):
            out["fp8_frac_of_measured_mfma"] = round(result["fp8"]["tflops"] / (r[8] / 1e12), 4)
    print(f"[bench] ceilings: clock {clock:.3f} GHz, bf16 MFMA {r[7] / 1e12:.0f} TFLOP/s, "
          f"fp8 {r[8] / 1e12:.0f}, exp {out['exp_cycles_per_wave_instr']} cycles/instr", file=sys.stderr, flush=True)
    return out


def bench_sweep(A, W, args):
    """The 16384-token sequence sweep and the varlen/paged workload (extra
    lines; inputs drawn on the device from the same seeds)."""
    import torch
    out = []
    for w in W.seq_sweep_points():
        qs, ks = w.shapes()
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        q, k, v = (torch.randn(qs, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        ms = time_launches(lambda: A.fwd(q, k, v, w.scale, w.causal), max(5, args.steps // 3), 10)
        tf = w.flops / (ms * 1e-3) / 1e12
        byts = 4 * q.numel() * 2 + 4 * w.batch * w.heads * w.seq_q
        out.append({"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "gbs": round(byts / (ms * 1e-3) / 1e9, 1)})
        print(f"[bench] {w.name}: {ms:.3f} ms {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    # varlen + paged: 32 sequences U{128..4096}, 32 heads, d128, causal, 64-token pages
    cfg = W.VARLEN
    lens = W.varlen_lengths(cfg["seed_lengths"], cfg["n_seq"], cfg["lo"], cfg["hi"])
    H, D, page = cfg["heads"], cfg["head_dim"], cfg["page_size"]
    cu = torch.from_numpy(W.cu_seqlens(lens)).cuda()
    tot = int(lens.sum())
    g = torch.Generator(device="cuda").manual_seed(cfg["seed_values"])
    q, k, v = (torch.randn((tot, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    table, npages = W.paged_layout(cfg["seed_pages"], lens, page)
    kp = torch.zeros((npages, page, H, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    cuh = W.cu_seqlens(lens)
    for b, n in enumerate(lens):
        for t0 in range(0, int(n), page):
            t1 = min(t0 + page, int(n))
            kp[table[b, t0 // page], :t1 - t0] = k[cuh[b] + t0:cuh[b] + t1]
            vp[table[b, t0 // page], :t1 - t0] = v[cuh[b] + t0:cuh[b] + t1]
    tab = torch.from_numpy(table).cuda()
    flops = sum(4.0 * H * int(n) * int(n) * D / 2 for n in lens)
    mx = int(lens.max())
    for name, kk, vv, bt in (("varlen_packed", k, v, None), ("varlen_paged64", kp, vp, tab)):
        ms = time_launches(lambda: A.fwd_varlen(q, cu, kk, vv, cu, mx, mx, None, True, block_table=bt,
                                                page_size=page if bt is not None else 0),
                           max(5, args.steps // 3), 10)
        tf = flops / (ms * 1e-3) / 1e12
        out.append({"workload": f"{name}_32seq_h32_d128_causal", "ms": round(ms, 4), "tflops": round(tf, 1)})
        print(f"[bench] {name}: {ms:.3f} ms {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
    return out


if __name__ == "__main__":
    main()
