"""Benchmark: exact attention forward + backward on one MI355X.

One step = the whole hot path on the headline workload (B8 H16 N4096 d128,
causal, bf16): fa_fwd, then the backward's two stages as fa_bwd runs them
(fa_bwd_dq_dot: dQ with the row-dot D folded in; then fa_bwd_dkdv), all on one
stream with inputs resident in HBM.
W untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; HIP events around each kernel give per-kernel durations.

Prints ONE JSON line.  `value` is fwd+bwd algorithmic TFLOP/s (4d + 10d FLOPs per
(query, key) pair; causal pairs = N(N+1)/2).  `roofline` describes the kernel that
takes the most time per step; `cpu_baseline` times the CPU fp64 oracle on a
time-bounded sample of the same workload's heads.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

from io_aware_exact_attention_amd import accounting as acc
from io_aware_exact_attention_amd import fa355
from io_aware_exact_attention_amd import workloads as wl

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TARGET_FWD_PCT = 50.0       # causal bf16 forward, % of the dense bf16 MFMA peak
TARGET_FWD_BWD_PCT = 35.0   # forward + backward

CALIB_BYTES = 256 << 20     # size of the counter-calibration copy

METRIC = "attention fwd & fwd+bwd TFLOP/s, % bf16 MFMA peak, B8 H16 N4096 d128 causal"

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "io_aware_exact_attention_amd", "csrc")


# The sources that define each path's kernels (their launch shapes come from the
# configuration structs in the same headers).
KERNEL_SOURCES = {
    "bf16": ("fa_device.hpp", "fa_params.hpp", "fa_tiles.hpp", "fa_fwd.hpp", "fa_bwd.hpp"),
    "decode": ("fa_device.hpp", "fa_params.hpp", "fa_tiles.hpp", "fa_decode.hpp"),
    "fp8": ("fa_device.hpp", "fa_params.hpp", "fa_tiles.hpp", "fa_fp8.hpp"),
}


def workload_kind(workload: str) -> str:
    if workload in wl.FP8_WORKLOADS:
        return "fp8"
    if workload in wl.DECODE_WORKLOADS:
        return "decode"
    return "bf16"


def kernel_source_hash(kind: str = "bf16") -> str:
    """sha256 over the sources of one path's kernels: identifies the kernels a
    stored counter summary was taken from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of each kernel, from the committed rocprofv3 PMC summary
    (TCC FETCH_SIZE and WRITE_SIZE in KiB, each scaled by what the same counter
    read for the benchmark's calibration copy of known size).  None when there is
    no summary or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    src, calib, kern = None, None, {}
    with open(path) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "source_sha256":
                src = t[1]
            elif t[0] == "calibration_copy":
                calib = (int(t[2]), float(t[4]), float(t[6]))   # bytes, fetch KiB, write KiB
            elif t[0] == "kernel":
                kern[t[1]] = (float(t[3]), float(t[5]))
    if src != kernel_source_hash(workload_kind(workload)) or calib is None or calib[1] <= 0 or calib[2] <= 0:
        return None
    fetch_scale = calib[0] / (calib[1] * 1024)
    write_scale = calib[0] / (calib[2] * 1024)
    return {k: int(round(fk * 1024 * fetch_scale + wk * 1024 * write_scale))
            for k, (fk, wk) in kern.items()}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=wl.HEADLINE)
    ap.add_argument("--forward", choices=("tiles", "persistent"), default="tiles",
                    help="forward kernel of the dense step: one work-group per tile (fa_fwd) or the "
                         "persistent longest-first kernel (fa_fwd_persistent)")
    ap.add_argument("--max-seqlen", type=int, default=0,
                    help="packed workloads: max_seqlen passed to the kernels (default: the longest "
                         "sequence; a larger value adds only work-groups that find no rows, which "
                         "measures what the grid's empty work-groups cost)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-time budget of the CPU oracle sample (0 disables it)")
    return ap.parse_args()


def calibration_copy(dev):
    """One plain device copy of known size, outside the timed region: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE calibrate the byte counters."""
    calib = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    del calib, calib_dst
    torch.cuda.synchronize()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, w, causal, budget_s: float):
    """Time the fp64 oracle, fwd + bwd, head by head until the budget is used."""
    import oracle   # test infrastructure: only this leg of the benchmark uses it

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    B, N, H, d = x["q"].shape
    done, t_fwd, t_bwd = 0, 0.0, 0.0
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            q, k, v, do = (x[n][sl].contiguous() for n in ("q", "k", "v", "dout"))
            t0 = time.perf_counter()
            oracle.attention_forward(q, k, v, w.scale, causal)
            t1 = time.perf_counter()
            oracle.attention_backward(q, k, v, do, w.scale, causal)
            t_fwd += t1 - t0
            t_bwd += time.perf_counter() - t1
            done += 1
            if t_fwd + t_bwd >= budget_s:
                break
        if t_fwd + t_bwd >= budget_s:
            break
    p = acc.pairs(N, N, causal) * done
    f_fwd, f_bwd = acc.flops_fwd(p, d), acc.flops_bwd(p, d)
    return {
        "value": round((f_fwd + f_bwd) / (t_fwd + t_bwd) / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": torch.get_num_threads(),
        "kind": "oracle",
        "sample": f"{done} of {B * H} (batch, head) slices, forward + backward, float64, "
                  f"{t_fwd + t_bwd:.1f} s",
        "fwd_tflops": round(f_fwd / t_fwd / 1e12, 6),
        "bwd_tflops": round(f_bwd / t_bwd / 1e12, 6),
        "cpu": cpu_model(),
    }


DECODE_METRIC = "split-KV decode HBM GB/s, % of 8 TB/s"


def decode_cpu_baseline(x, w, budget_s: float):
    """Time the fp64 decoding oracle one (sequence, key/value head) group at a time."""
    import oracle   # test infrastructure: only this leg of the benchmark uses it

    torch.set_num_threads(len(os.sched_getaffinity(0)))
    G = w.Hq // w.Hkv
    done, t_total, nbytes = 0, 0.0, 0
    for b in range(w.B):
        for hk in range(w.Hkv):
            hs = slice(hk * G, (hk + 1) * G)
            q = x["q"][b:b + 1, :, hs].contiguous()
            k = x["k"][b:b + 1, :, hk:hk + 1].contiguous()
            v = x["v"][b:b + 1, :, hk:hk + 1].contiguous()
            t0 = time.perf_counter()
            oracle.decode_forward(q, k, v, w.scale, w.causal)
            t_total += time.perf_counter() - t0
            done += 1
            nbytes += 2 * w.Nk * w.d * 2
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hkv} (sequence, key/value head) groups, float64, "
                      f"{t_total:.1f} s",
            "cpu": cpu_model()}


def run_decode(args, w):
    """Decoding workload: one step = fa_fwd_decode (split kernel + merge kernel)."""
    dev = torch.device("cuda", 0)
    x = wl.make_inputs(w.name)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Nq, dtype=torch.float32, device=dev)
    nbytes = fa355.fa_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    call = lambda: fa355.fa_fwd_decode(q, k, v, o, lse, ws, w.scale, w.causal)
    calibration_copy(dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for s in range(args.steps):
        call()
        ev[s + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ts = sorted(ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps))
    ms = sum(ts) / len(ts)
    # compulsory bytes: the cache once, q in, o and lse out
    kv_bytes = 2 * w.B * w.Nk * w.Hkv * w.d * 2
    io_bytes = kv_bytes + 2 * w.B * w.Nq * w.Hq * w.d * 2 + w.B * w.Hq * w.Nq * 4
    pairs = w.B * w.Hq * sum(min(w.Nk, i + w.Nk - w.Nq + 1) if w.causal else w.Nk
                              for i in range(w.Nq))
    gbs = io_bytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    out = {
        "metric": DECODE_METRIC,
        "value": round(io_bytes / wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Nq": w.Nq, "Nk": w.Nk, "Hq": w.Hq,
                   "Hkv": w.Hkv, "d": w.d, "causal": w.causal, "scale": w.scale},
        "decode": {"ms": round(ms, 4), "ms_median": round(ts[len(ts) // 2], 4),
                   "ms_min": round(ts[0], 4), "gbs": round(gbs, 1),
                   "tflops": round(4 * w.d * pairs / (ms * 1e-3) / 1e12, 3),
                   "algorithmic_bytes": io_bytes,
                   "workspace_bytes": nbytes},
        # events bracket both kernels of the entry point (split + merge); the
        # kernel-trace summary in profiles/ separates them
        "roofline": {"kernel": "fa_decode_split_kernel + fa_decode_combine_kernel",
                     "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": (traffic.get("fa_decode_split_kernel", 0) +
                                 traffic.get("fa_decode_combine_kernel", 0)) if traffic else None,
                     "algorithmic_bytes": io_bytes},
        "device": torch.cuda.get_device_name(0),
    }
    out["cpu_baseline"] = decode_cpu_baseline(x, w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(out), flush=True)


FP8_METRIC = "FP8 (e4m3, Hadamard-rotated Q/K) attention forward TFLOP/s, % fp8 MFMA peak, B8 H16 N4096 d128 causal"
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def fp8_cpu_baseline(x, base, budget_s: float):
    """Time the fp64 FP8 oracle (rotate, quantise, attend) one (batch, head) at a time."""
    import oracle.fp8 as of8   # test infrastructure: only this leg of the benchmark uses it

    torch.set_num_threads(len(os.sched_getaffinity(0)))
    B, N, H, d = x["q"].shape
    done, t_total = 0, 0.0
    for b in range(B):
        for h in range(H):
            sl = slice(h, h + 1)
            t0 = time.perf_counter()
            of8.fp8_forward(x["q"][b:b + 1, :, sl], x["k"][b:b + 1, :, sl], x["v"][b:b + 1, :, sl],
                            x["signs"], base.scale, True)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flops = acc.flops_fwd(acc.pairs(N, N, True), d) * done
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{done} of {B * H} (batch, head) slices, FP8 forward (rotation, quantisation, "
                      f"blocked attention, tie bounds), float64, {t_total:.1f} s",
            "cpu": cpu_model()}


def run_fp8(args, w8):
    """FP8 forward: one step = fa_fwd_fp8 (quantisation kernel, attention kernel)."""
    base = wl.WORKLOADS[w8.base]
    dev = torch.device("cuda", 0)
    x = wl.make_inputs(w8.name)
    q, k, v, sg = (x[n].to(dev) for n in ("q", "k", "v", "signs"))
    B, N, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    nbytes = fa355.fa_fp8_workspace_bytes(B, N, N, H, d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    step = lambda: fa355.fa_fwd_fp8(q, k, v, sg, o, lse, ws, base.scale, True, True)
    calibration_copy(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    q8, k8, v8, sc = fa355.fp8_workspace_views(ws, B, N, N, H, d)
    sq, sk, sv = (sc[i].reshape(-1) for i in range(3))
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    attn = lambda: fa355.fa_fwd_fp8_codes(q8, k8, v8, sq, sk, sv, o2, lse2, base.scale / d, True)

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(args.steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        return wall, ts

    wall, ts_step = timed(step)
    for _ in range(2):
        attn()
    _, ts_attn = timed(attn)
    flops = acc.flops_fwd(acc.pairs(N, N, True), d) * B * H
    ms_step = sum(ts_step) / len(ts_step)
    ms_attn = sum(ts_attn) / len(ts_attn)
    rate = flops / (ms_attn * 1e-3) / 1e12
    # compulsory bytes of the attention kernel: codes of q, k, v in, o (bf16) and lse out
    attn_bytes = 3 * B * N * H * d + B * N * H * d * 2 + B * H * N * 4
    # quantisation: q, k, v read once, codes (and 64-row block scales) written
    quant_bytes = 3 * B * N * H * d * 2 + 3 * B * N * H * d
    traffic = measured_traffic(w8.name)
    out = {
        "metric": FP8_METRIC,
        "value": round(flops / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w8.name, "B": B, "H": H, "N": N, "d": d, "causal": True,
                   "scale": base.scale, "rotation": "random-sign Hadamard"},
        "step": {"ms": round(ms_step, 4), "ms_median": round(ts_step[len(ts_step) // 2], 4),
                 "ms_min": round(ts_step[0], 4), "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2)},
        "kernels": {
            "fa_fwd_fp8_kernel": {"ms": round(ms_attn, 4), "ms_median": round(ts_attn[len(ts_attn) // 2], 4),
                                  "ms_min": round(ts_attn[0], 4), "tflops": round(rate, 2),
                                  "algorithmic_bytes": attn_bytes,
                                  "traffic": traffic.get("fa_fwd_fp8_kernel") if traffic else None},
            "fp8_quant_kernel": {
                "ms": round(ms_step - ms_attn, 4),
                "gbs": round(quant_bytes / max((ms_step - ms_attn) * 1e-3, 1e-9) / 1e9, 1),
                "algorithmic_bytes": quant_bytes},
        },
        "roofline": {"kernel": "fa_fwd_fp8_kernel", "bound": "mfma", "achieved": round(rate, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(rate / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic.get("fa_fwd_fp8_kernel") if traffic else None,
                     "algorithmic_bytes": attn_bytes},
        "device": torch.cuda.get_device_name(0),
    }
    out["cpu_baseline"] = fp8_cpu_baseline(x, base, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(out), flush=True)


def run_varlen(args, w):
    """Packed variable-length workload: one step = fa_fwd_varlen + fa_bwd_varlen."""
    dev = torch.device("cuda", 0)
    x = wl.make_inputs(w.name)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    cu = x["cu_seqlens"].to(dev)
    mx = max(x["max_seqlen"], args.max_seqlen)
    nseq = cu.numel() - 1
    causal = w.causal[-1]
    o = torch.empty_like(q)
    lse = torch.empty(nseq, w.H, mx, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa355.fa_bwd_workspace_bytes(nseq, w.H, mx, w.d) // 4, dtype=torch.float32,
                     device=dev)
    calls = [
        lambda: fa355.fa_fwd_varlen(q, k, v, o, lse, cu, cu, mx, mx, w.scale, causal),
        lambda: fa355.fa_bwd_varlen(q, k, v, o, do, lse, dq, dk, dv, ws, cu, cu, mx, mx, w.scale,
                                    causal),
    ]
    calibration_copy(dev)
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for i, c in enumerate(calls):
            c()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    t_fwd = sum(ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)) / args.steps
    t_bwd = sum(ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)) / args.steps
    cnt = acc.varlen_counts(x["lengths"], w.H, w.d, causal)
    f_fwd, f_bwd = cnt["flops_fwd"], cnt["flops_bwd"]
    fwd_tf = f_fwd / (t_fwd * 1e-3) / 1e12
    value = (f_fwd + f_bwd) / wall / 1e12
    out = {
        "metric": METRIC.replace("B8 H16 N4096 d128 causal", "packed varlen"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "H": w.H, "d": w.d, "nseq": nseq,
                   "tokens": int(sum(x["lengths"])), "max_seqlen": mx, "causal": causal},
        "fwd_ms": round(t_fwd, 4),
        "bwd_ms": round(t_bwd, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
        "bwd_tflops": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_hbm_gbs": round(cnt["bytes_fwd"] / (t_fwd * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "fa_fwd_kernel + fa_bwd_* (varlen)", "bound": "mfma",
                     "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "device": torch.cuda.get_device_name(0),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def fa_fwd_kernel_name(B: int, H: int, N: int, causal: bool) -> str:
    """The kernel fa_fwd launches for a dense shape (its documented choice): the
    key-split kernel for causal grids of at most one 128-row query tile per CU (or
    two per CU with at least 16 tiles per sequence), else the persistent kernel
    when the tiles fit two per CU or, causal, when a sequence has at most 32
    tiles, else one work-group per tile."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_tiles = -(-N // 128)
    items = n_tiles * B * H
    if causal and (items <= cus or (items <= 2 * cus and n_tiles >= 16)):
        return "fa_fwd_split_kernel"
    if items <= 2 * cus or (causal and n_tiles <= 32):
        return "fa_fwd_persistent_kernel"
    return "fa_fwd_kernel"


def fa_bwd_pass_kernel_names(B: int, H: int, N: int, causal: bool) -> tuple:
    """The kernels fa_bwd_dq_dot and fa_bwd_dkdv launch for a dense shape (their
    documented choice): each pass on a persistent grid when causal with more
    than two 128-row tiles per CU and either at most eight per CU, or at most 32
    tiles per sequence with items times tiles per sequence at most 512 per CU;
    else one work-group per tile."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = -(-N // 128)
    items = t * B * H
    pers = causal and items > 2 * cus and (items <= 8 * cus or (t <= 32 and items * t <= 512 * cus))
    if pers:
        return "fa_bwd_dq_persistent_kernel", "fa_bwd_dkdv_persistent_kernel"
    return "fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"


def fa_bwd_is_fused(B: int, H: int, N: int, causal: bool) -> bool:
    """Whether fa_bwd runs as the row-dot kernel and one launch holding both
    passes (its documented choice for small dense grids: at most 6 causal or 2
    non-causal dK/dV plus dQ work items of 128 rows per CU)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 2 * (-(-N // 128)) * B * H <= (6 if causal else 2) * cus


def small_config_rates(name: str, causal: bool, steps: int = 50, warmup: int = 10) -> dict:
    """Forward and forward + backward rates of a small dense workload (one that is
    launch- or tail-bound rather than MFMA-bound), timed like the main step with
    HIP events over `steps` back-to-back steps after `warmup` untimed ones."""
    w = wl.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    x = wl.make_inputs(w.name)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    B, N, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa355.fa_bwd_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=dev)
    calls = [
        lambda: fa355.fa_fwd(q, k, v, o, lse, w.scale, causal),
        lambda: fa355.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, w.scale, causal),
    ]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record()
        calls[0]()
        ev[s][1].record()
        for c in calls[1:]:
            c()
    torch.cuda.synchronize()
    t_fwd = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_start.record()
    for _ in range(steps):
        for c in calls:
            c()
    e_end.record()
    torch.cuda.synchronize()
    t_step = e_start.elapsed_time(e_end) / steps
    cnt = acc.dense_counts(B, H, N, d, causal)
    fwd_ms = sum(t_fwd) / len(t_fwd)
    fwd_tf = cnt["flops_fwd"] / (fwd_ms * 1e-3) / 1e12
    step_tf = (cnt["flops_fwd"] + cnt["flops_bwd"]) / (t_step * 1e-3) / 1e12
    return {"shape": f"B{B} H{H} N{N} d{d} {'causal' if causal else 'non-causal'}",
            "fwd_ms": round(fwd_ms, 5), "fwd_ms_min": round(t_fwd[0], 5),
            "fwd_tflops": round(fwd_tf, 2), "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
            "step_ms": round(t_step, 5), "fwd_bwd_tflops": round(step_tf, 2),
            "fwd_bwd_pct_peak": round(100 * step_tf / PEAK_BF16_TFLOPS, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by batch entry and head, which need no communication)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload in wl.FP8_WORKLOADS:
        return run_fp8(args, wl.FP8_WORKLOADS[args.workload])
    if args.workload in wl.DECODE_WORKLOADS:
        return run_decode(args, wl.DECODE_WORKLOADS[args.workload])
    w = wl.WORKLOADS[args.workload]
    if w.varlen:
        return run_varlen(args, w)
    causal = w.causal[-1]
    dev = torch.device("cuda", 0)
    x = wl.make_inputs(w.name)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    B, N, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa355.fa_bwd_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=dev)
    scale = w.scale

    persistent = args.forward == "persistent"
    fused = fa_bwd_is_fused(B, H, N, causal)
    names = ["fa_fwd_persistent_kernel" if persistent else fa_fwd_kernel_name(B, H, N, causal),
             *fa_bwd_pass_kernel_names(B, H, N, causal)]
    fwd = fa355.fa_fwd_persistent if persistent else fa355.fa_fwd
    calls = [   # fa_bwd = fa_bwd_dq_dot, then fa_bwd_dkdv (one kernel each)
        lambda: fwd(q, k, v, o, lse, scale, causal),
        lambda: fa355.fa_bwd_dq_dot(q, k, v, o, do, lse, ws, dq, scale, causal),
        lambda: fa355.fa_bwd_dkdv(q, k, v, do, ws, dk, dv, scale, causal),
    ]
    if fused:   # small grids: fa_bwd is the row-dot kernel, then both passes in one launch
        names = names[:1] + ["fa_bwd_dot_kernel + fa_bwd_fused_kernel"]
        calls = calls[:1] + [lambda: fa355.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale, causal)]
    calibration_copy(dev)

    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for i, c in enumerate(calls):
            c()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    per_step = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
                for i in range(len(calls))]
    kern_ms = [sum(t) / len(t) for t in per_step]

    cnt = acc.dense_counts(B, H, N, d, causal)
    pairs = cnt["pairs"]
    f_fwd, f_bwd = cnt["flops_fwd"], cnt["flops_bwd"]
    # algorithmic FLOPs attributed per kernel (the 10d backward = 2d in dQ + 8d in dK/dV)
    kern_flops = [f_fwd, 2 * d * pairs, 8 * d * pairs] if not fused else [f_fwd, 10 * d * pairs]
    kern = {}
    for n, ms, fl, ts in zip(names, kern_ms, kern_flops, per_step):
        ts = sorted(ts)
        kern[n] = {"ms": round(ms, 4), "ms_median": round(ts[len(ts) // 2], 4), "ms_min": round(ts[0], 4),
                   "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    # algorithmic HBM bytes per launch (each input read once, each output written once):
    # dQ + row-dot reads q, k, v, o, dout, LSE and writes dq, -D, LSE*log2(e);
    # dK/dV reads q, k, v, dout, -D, LSE*log2(e) and writes dk, dv
    tok = B * N * H
    kern_bytes = [cnt["bytes_fwd"], tok * (5 * 2 * d + 4) + tok * (2 * d + 8),
                  tok * (4 * 2 * d + 8) + tok * 2 * 2 * d]
    if fused:   # the row-dot kernel (o, dout, LSE in; -D, LSE*log2(e) out), then the two
        # passes, each reading q, k, v, dout, -D and LSE*log2(e) once (dq; dk, dv out)
        kern_bytes = [kern_bytes[0], tok * (2 * 2 * d + 4 + 8) + tok * (4 * 2 * d + 8 + 2 * d)
                      + tok * (4 * 2 * d + 8 + 2 * 2 * d)]
    traffic = measured_traffic(w.name)
    dom = max(range(len(names)), key=lambda i: kern_ms[i])
    achieved = kern_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    roof = {"kernel": names[dom], "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    def traffic_of(name):   # "a + b": the kernels one entry point launches, summed
        parts = [traffic.get(k) for k in name.split(" + ")] if traffic else [None]
        return sum(parts) if all(t is not None for t in parts) else None

    roof["traffic"] = traffic_of(names[dom])
    roof["algorithmic_bytes"] = kern_bytes[dom]
    for n, b_alg in zip(names, kern_bytes):
        kern[n]["algorithmic_bytes"] = b_alg
        kern[n]["traffic"] = traffic_of(n)

    t_fwd = kern_ms[0]
    t_bwd = sum(kern_ms[1:])
    fwd_tf = f_fwd / (t_fwd * 1e-3) / 1e12
    fb_tf_events = (f_fwd + f_bwd) / ((t_fwd + t_bwd) * 1e-3) / 1e12
    value = (f_fwd + f_bwd) / wall / 1e12
    shape = f"B{B} H{H} N{N} d{d} {'causal' if causal else 'non-causal'}"
    if w.k_scale != 1.0:
        shape += f", K x{w.k_scale:g}"
    out = {
        "metric": METRIC.replace("B8 H16 N4096 d128 causal", shape),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "scale": scale, "forward": args.forward},
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
        "fwd_bwd_tflops_kernels": round(fb_tf_events, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_hbm_gbs": round(cnt["bytes_fwd"] / (t_fwd * 1e-3) / 1e9, 1),
        # the performance targets set for this path on its headline workload
        "targets": {"fwd_pct_peak": TARGET_FWD_PCT, "fwd_bwd_pct_peak": TARGET_FWD_BWD_PCT,
                    "fwd_met": 100 * fwd_tf / PEAK_BF16_TFLOPS >= TARGET_FWD_PCT,
                    "fwd_bwd_met": 100 * value / PEAK_BF16_TFLOPS >= TARGET_FWD_BWD_PCT},
        "kernels": kern,
        "roofline": roof,
        "device": torch.cuda.get_device_name(0),
    }
    if w.name == wl.HEADLINE:
        # the small configurations, after the timed region: launch- and tail-bound
        # shapes whose rates the headline line would not show
        out["small_configs"] = {
            "tiny": small_config_rates("tiny", False),
            "b4_h16_n1024_d64_causal": small_config_rates("b4_h16_n1024_d64", True),
            "b4_h16_n1024_d64_noncausal": small_config_rates("b4_h16_n1024_d64", False),
        }
    if args.cpu_seconds > 0:
        xc = {n: x[n] for n in ("q", "k", "v", "dout")}
        out["cpu_baseline"] = cpu_baseline(xc, w, causal, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
