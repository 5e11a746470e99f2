"""Attention forward throughput on one MI355X, one JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-fp8] [--no-configs] [--no-merge] [--no-decode] [--no-d256]
    python bench.py --sweep | --gemm-calibration | --copy-calibration

A step is one pass of the whole hot path over one batch of synthetic input:
one bf16 attn_fwd launch over B16 H16 N8192 d128 (non-causal), the headline
workload; `value`, `ms_per_step` and `roofline` are that launch's.
Beside it, each in its own object:
  "configs": the other bf16 workloads (B1 H2 N256 d64; causal B4 H16 N2048
             d128; causal window 1024 B2 H32 N16384 d64), each timed with HIP
             events on the launch stream, with its roofline and its accuracy
             against the fp64 oracle on sampled heads;
  "fp8":     the x10-outlier workload at B8 (its configured batch) and at B16
             (the headline shape): attn_fp8_quantize of Q, K, V (per 128-row
             block, and per tensor: the naive baseline) plus the all-E4M3
             attn_fwd; the fp8 PV mode (bf16 scores, E4M3 P and V); RMSE/RMS
             against the unquantised fp64 oracle for each mode;
  "lse_merge", "decode", "decode_paged", "d256": the next-row kernels.
Inputs come from attn_inputs and are resident in HBM before timing.
TFLOP/s counts algorithmic FLOP: 4 * d * (number of allowed query/key pairs).
"cpu_baseline" times the fp64 oracle on a bounded sample of heads of the
headline workload on the host cores (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_FP8_TFLOPS = 5033.2       # dense fp8
PEAK_HBM_GBS = 8000.0
# fp8 PV mode: half the FLOPs on bf16 MFMAs (QK^T), half on fp8 (PV)
PEAK_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_BF16_TFLOPS + 0.5 / PEAK_FP8_TFLOPS)
METRIC = "attn fwd TFLOP/s and % MFMA peak, B16 H16 N8192 d128, bf16 and fp8"
DEFAULT_WORKLOAD = "noncausal_b16h16n8192d128_bf16"
FP8_WORKLOAD = "noncausal_b8h16n8192d128_fp8_outliers"


def allowed_pairs(N: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs in the allowed set of one head."""
    tot = 0
    for i in range(N) if (causal or window >= 0) else ():
        lo = max(0, i - window) if window >= 0 else 0
        hi = i + 1 if causal else (min(N, i + window + 1) if window >= 0 else N)
        tot += max(0, hi - lo)
    return tot if (causal or window >= 0) else N * N


# Sources each profiled kernel is compiled from (its unit, the headers it
# includes, and the build flags), so that a recorded traffic figure is used
# only for the kernel code it was measured on.
KERNEL_SOURCES = {
    "bf16": ["attn_fwd_bf16.hip", "attn_device.h", "attn_internal.h", "../build.py"],
    "fp8": ["attn_fwd_fp8.hip", "attn_device.h", "attn_internal.h", "../build.py"],
}


def strip_c_comments(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed to one
    space (string and character literals kept as they are), so that editing a
    comment does not change the hash of the code a measurement was taken on."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash(kind: str = "bf16") -> str:
    """Hash of the code (comments and layout stripped from the C/C++ files;
    the build script as it is) that the kernel of one kind is compiled from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_attention_forward_attn_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        if not f.endswith(".py"):
            text = strip_c_comments(text)
        h.update((f + "\0" + text).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kind: str = "bf16"):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current sources of that kernel (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(kind):
        return None
    return float(m_bytes.group(1))


def time_launches(fn, steps: int, warmup: int, stream):
    """Run fn `warmup` times, then `steps` times bracketed by synchronize;
    returns (wall ms per step, list of per-launch event ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def cpu_baseline(w, o_gpu, lse_gpu, budget_s: float = 15.0):
    """Time the fp64 oracle on whole heads of the workload until ~budget_s of
    CPU work, and compare the GPU output on those heads. Heads are visited in
    a fixed order that spreads over batches and heads without repeats."""
    import torch
    from attn_inputs import workload_head
    from oracle import attention_rows, max_abs, l1_rel
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    heads, t_oracle, worst_ma, worst_l1, worst_lse = [], 0.0, 0.0, 0.0, 0.0
    nbh = w.B * w.H
    stride = next(s for s in (97, 89, 83, 79, 73, 71, 67, 61, 59, 53, 1) if math.gcd(s, nbh) == 1)
    for i in range(nbh):
        b, h = divmod((i * stride) % nbh, w.H)
        q, k, v = workload_head(w, b, h)
        t0 = time.perf_counter()
        ref_o, ref_lse = attention_rows(q, k, v, w.scale, w.causal, w.window)
        t_oracle += time.perf_counter() - t0
        heads.append((b, h))
        worst_ma = max(worst_ma, max_abs(o_gpu[b, h], ref_o))
        worst_l1 = max(worst_l1, l1_rel(o_gpu[b, h], ref_o))
        worst_lse = max(worst_lse, max_abs(lse_gpu[b, h], ref_lse))
        if t_oracle >= budget_s:
            break
    flop = 4.0 * w.d * allowed_pairs(w.N, w.causal, w.window) * len(heads)
    return {
        "value": flop / t_oracle / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{len(heads)} whole heads (all {w.N} query rows each) of {w.name}, fp64 two-pass "
                  f"attention on torch-CPU, {t_oracle:.1f} s",
        "parity_on_sample": {"max_abs": worst_ma, "l1_rel": worst_l1, "lse_max_abs": worst_lse},
    }


def time_grouped(fn, groups: int, per_group: int, warmup: int, stream):
    """Per-launch ms of back-to-back launches: `groups` groups of `per_group`
    launches, each group between one pair of HIP events on the launch stream;
    returns the per-launch time of every group. For launches of tens of
    microseconds an event pair around each one would add its own gaps."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(per_group):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / per_group)
    return out


def workload_flop(w, B=None) -> float:
    return 4.0 * w.d * allowed_pairs(w.N, w.causal, w.window) * (w.B if B is None else B) * w.H


def mean_ms(ev):
    return sum(ev) / len(ev)


def spread_heads(B, H, count):
    """`count` distinct (b, h) pairs spread over batches and heads."""
    out = []
    for i in range(B * H):
        b, h = i % B, (5 * i + i // B) % H
        if (b, h) not in out:
            out.append((b, h))
        if len(out) == count:
            break
    return out


def bf16_accuracy(w, samples):
    """Worst max-abs, L1-rel and LSE error over the sampled whole heads
    (oracle leg: runs only with the CPU baseline)."""
    from attn_inputs import workload_head
    from oracle import attention_rows, max_abs, l1_rel
    worst = {"max_abs": 0.0, "l1_rel": 0.0, "lse_max_abs": 0.0}
    for (b, h), (ob, lb) in samples.items():
        q, k, v = workload_head(w, b, h)
        ref_o, ref_lse = attention_rows(q, k, v, w.scale, w.causal, w.window)
        worst["max_abs"] = max(worst["max_abs"], max_abs(ob, ref_o))
        worst["l1_rel"] = max(worst["l1_rel"], l1_rel(ob, ref_o))
        worst["lse_max_abs"] = max(worst["lse_max_abs"], max_abs(lb, ref_lse))
    worst["sample"] = f"{len(samples)} whole heads ({w.N} rows each)"
    worst["meets_bar"] = worst["max_abs"] <= 2e-2 and worst["l1_rel"] <= 5e-3
    return worst


def bench_bf16_config(tafa, w, dev, steps, warmup, stream):
    """One bf16 workload: time, TFLOP/s and roofline. Returns the entry and the
    outputs of a few whole heads (host copies) for the oracle leg."""
    import torch
    from attn_inputs import workload_qkv
    q, k, v = workload_qkv(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    run = lambda: tafa.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=o, lse=lse)
    # launches shorter than ~1 ms: groups of back-to-back launches, median group
    groups, per_group = 9, 50
    per_launch = sorted(time_grouped(run, groups, per_group, max(warmup, 20), stream))
    ms = per_launch[groups // 2]
    n = groups * per_group
    flop = workload_flop(w)
    tf = flop / (ms * 1e-3) / 1e12
    samples = {(b, h): (o[b, h].cpu(), lse[b, h].cpu()) for b, h in spread_heads(w.B, w.H, 4)}
    del q, k, v, o, lse
    entry = {
        "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
        "window": w.window, "dtype": "bf16", "launches_timed": n,
        "timing": f"median of {groups} groups of {per_group} back-to-back launches, HIP events",
        "avg_launch_ms": round(ms, 5),
        "tflops": round(tf, 2), "algorithmic_tflop": flop / 1e12,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.name, "bf16")},
    }
    return entry, samples


def fp8_accuracy(w, outs, heads, rows):
    """RMSE/RMS of each mode's sampled output against the unquantised fp64
    oracle, pooled over the sampled rows of the sampled heads (oracle leg)."""
    from attn_inputs import workload_head
    from oracle import attention_rows
    num = {m: 0.0 for m in outs}
    den = 0.0
    for i, (b, h) in enumerate(heads):
        q, k, v = workload_head(w, b, h)
        ref_o, _ = attention_rows(q, k, v, w.scale, w.causal, w.window, rows)
        den += float(ref_o.pow(2).sum())
        for m, o in outs.items():
            num[m] += float((o[i].double() - ref_o).pow(2).sum())
    acc = {m: round(math.sqrt(num[m] / den), 5) for m in outs}
    return {"rmse_rel": acc, "meets_bar": {m: acc[m] <= 3e-2 for m in outs},
            "beats_per_tensor": {m: acc[m] < acc["per_tensor_naive"] for m in outs
                                 if m != "per_tensor_naive"},
            "sample": f"{len(heads)} heads x {len(rows)} rows"}


def bench_fp8(tafa, dev, steps, warmup, stream):
    """The x10-outlier workload: all-E4M3 (per block and per tensor) and the fp8
    PV mode, at B8 (accuracy and speed) and B16 (speed, the headline shape)."""
    import torch
    from attn_inputs import BY_NAME, workload_qkv, rotation_signs
    wf = BY_NAME[FP8_WORKLOAD]
    res = {"workload": wf.name, "dtype": "fp8_e4m3", "accuracy_bar_rmse_rel": 3e-2}
    signs = torch.from_numpy(rotation_signs(wf.seed, wf.d)).to(dev)
    for B in (wf.B, 16):
        print(f"[bench] fp8: generating {wf.name} at B={B}", file=sys.stderr, flush=True)
        q, k, v = workload_qkv(wf, device=dev, B=B)
        bufs = {name: tafa.quantize(t) for name, t in (("q", q), ("k", k), ("v", v))}
        o = torch.empty_like(q)
        lse = torch.empty((B, wf.H, wf.N), dtype=torch.float32, device=dev)
        flop = workload_flop(wf, B)

        def quant(per_tensor=False):
            for name, t in (("q", q), ("k", k), ("v", v)):
                tafa.quantize(t, per_tensor=per_tensor, out=bufs[name][0], descale=bufs[name][1])

        def attn8():
            tafa.fwd(bufs["q"][0], bufs["k"][0], bufs["v"][0], scale=wf.scale,
                     descales=(bufs["q"][1], bufs["k"][1], bufs["v"][1]), out=o, lse=lse)

        def attn_pv():
            tafa.fwd(q, k, bufs["v"][0], scale=wf.scale, descales=(None, None, bufs["v"][1]),
                     out=o, lse=lse)

        def step8():
            quant()
            attn8()

        def quant_rot():
            # incoherent processing: Q and K rotated with the same signs, V plain
            for name, t in (("q", q), ("k", k)):
                tafa.quantize(t, out=bufs[name][0], descale=bufs[name][1], rotation_signs=signs)
            tafa.quantize(v, out=bufs["v"][0], descale=bufs["v"][1])

        print(f"[bench] fp8: timing at B={B}", file=sys.stderr, flush=True)
        quant()
        _, ev_a = time_launches(attn8, steps, warmup, stream)
        _, ev_q = time_launches(quant, steps, warmup, stream)
        wall8, _ = time_launches(step8, steps, warmup, stream)
        _, ev_pv = time_launches(attn_pv, max(1, steps // 2), warmup, stream)
        _, ev_qr = time_launches(quant_rot, steps, warmup, stream)
        quant_rot()
        _, ev_ar = time_launches(attn8, max(1, steps // 2), warmup, stream)
        quant()
        a_ms, q_ms, pv_ms = mean_ms(ev_a), mean_ms(ev_q), mean_ms(ev_pv)
        qr_ms, ar_ms = mean_ms(ev_qr), mean_ms(ev_ar)
        qbytes = 3 * q.numel() * (2 + 1) + 3 * bufs["q"][1].numel() * 4
        a_tf, pv_tf = flop / (a_ms * 1e-3) / 1e12, flop / (pv_ms * 1e-3) / 1e12
        entry = {
            "B": B, "H": wf.H, "N": wf.N, "d": wf.d, "algorithmic_tflop": flop / 1e12,
            "all_e4m3": {
                "avg_launch_ms": round(a_ms, 4), "tflops": round(a_tf, 2),
                "frac_of_dense_fp8_peak": round(a_tf / PEAK_FP8_TFLOPS, 4),
                "quantize_qkv_ms": round(q_ms, 4),
                "quantize_gbs": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
                "quantize_frac_of_hbm_peak": round(qbytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "end_to_end_ms_per_step": round(wall8, 4),
                "end_to_end_tflops": round(flop / (wall8 * 1e-3) / 1e12, 2)},
            "rotated_qk": {
                "what": "incoherent processing: Q and K quantised after a random-sign Hadamard "
                        "rotation (attn_fp8_quantize_rotated), V plainly; the all-E4M3 kernel",
                "avg_launch_ms": round(ar_ms, 4),
                "tflops": round(flop / (ar_ms * 1e-3) / 1e12, 2),
                "frac_of_dense_fp8_peak": round(flop / (ar_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                "quantize_qkv_ms": round(qr_ms, 4),
                "quantize_gbs": round(qbytes / (qr_ms * 1e-3) / 1e9, 1),
                "end_to_end_tflops": round(flop / ((ar_ms + qr_ms) * 1e-3) / 1e12, 2)},
            "pv_mode": {
                "what": "bf16 Q, K (scores on bf16 MFMAs); E4M3 V and P (PV on fp8 MFMAs)",
                "avg_launch_ms": round(pv_ms, 4), "tflops": round(pv_tf, 2),
                "frac_of_dense_fp8_peak": round(pv_tf / PEAK_FP8_TFLOPS, 4),
                "frac_of_mixed_ceiling": round(pv_tf / PEAK_MIXED_TFLOPS, 4),
                "mixed_ceiling_tflops": round(PEAK_MIXED_TFLOPS, 1)},
        }
        if B == wf.B:
            # sampled outputs of each mode, for the oracle leg's RMSE/RMS
            heads = spread_heads(B, wf.H, 8)
            rows = sorted(set(range(0, wf.N, 64)) | {wf.N - 1})
            hi = torch.tensor([b * wf.H + h for b, h in heads], device=dev)
            ri = torch.tensor(rows, device=dev)
            take = lambda t: t.view(B * wf.H, wf.N, wf.d)[hi][:, ri].cpu()
            outs = {}
            attn8()
            outs["per_block"] = take(o)
            attn_pv()
            outs["pv_mode"] = take(o)
            quant(per_tensor=True)
            attn8()
            outs["per_tensor_naive"] = take(o)
            quant_rot()
            attn8()
            outs["rotated_qk"] = take(o)
            quant()
            res["_samples"] = (wf, outs, heads, rows)
        res[f"B{B}"] = entry
        del q, k, v, bufs, o, lse
        torch.cuda.empty_cache()
    b16 = res["B16"]["all_e4m3"]
    res["roofline"] = {"bound": "mfma", "kernel": "attn_fwd_fp8_kernel<128, false>",
                       "achieved": b16["tflops"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                       "frac": b16["frac_of_dense_fp8_peak"],
                       "traffic": recorded_traffic("noncausal_b16h16n8192d128_fp8", "fp8"),
                       "avg_launch_ms": b16["avg_launch_ms"]}
    return res


SWEEP_TOKENS = 131072          # B * N of every sweep point
SWEEP_N = [512, 1024, 2048, 4096, 8192, 16384, 32768]


def run_sweep(tafa, torch, stream):
    """Throughput across sequence lengths at a constant number of tokens per
    batch (B = 131072 / N; H = 32, 16, 8 at d = 64, 128, 256), causal and not,
    for bf16, all-E4M3 fp8 and the fp8 PV mode. Timing only: the inputs are
    seeded normal values drawn on the device (parity is the tests' job).
    Prints a markdown table: TFLOP/s and the fraction of the dense peak of the
    MFMA type that does the work (the PV mode against its mixed ceiling)."""
    gen = torch.Generator(device="cuda:0")
    kinds = [("bf16", 64), ("bf16", 128), ("bf16", 256), ("fp8", 64), ("fp8", 128), ("fp8pv", 128)]
    print("| kind | d | N | B | H | causal | ms per launch | TFLOP/s | fraction of peak |")
    print("|---|---|---|---|---|---|---|---|---|")
    for kind, d in kinds:
        H = {64: 32, 128: 16, 256: 8}[d]
        peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "fp8pv": PEAK_MIXED_TFLOPS}[kind]
        for N in SWEEP_N:
            B = SWEEP_TOKENS // N
            gen.manual_seed(N * 1000 + d)
            q, k, v = [torch.randn(B, H, N, d, generator=gen, device="cuda:0").to(torch.bfloat16)
                       for _ in range(3)]
            descales = None
            if kind == "fp8":
                (q, dq), (k, dk), (v, dv) = [tafa.quantize(t) for t in (q, k, v)]
                descales = (dq, dk, dv)
            elif kind == "fp8pv":
                v, dv = tafa.quantize(v)
                descales = (None, None, dv)
            o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda:0")
            lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda:0")
            for causal in (False, True):
                def launch():
                    tafa.fwd(q, k, v, causal=causal, descales=descales, out=o, lse=lse)
                one = time_grouped(launch, 1, 3, 2, stream)[0]
                per_group = max(3, min(200, int(20.0 / max(one, 1e-3))))
                ms = min(time_grouped(launch, 5, per_group, 2, stream))
                flop = 4.0 * d * allowed_pairs(N, causal, -1) * B * H
                tf = flop / (ms * 1e-3) / 1e12
                print(f"| {kind} | {d} | {N} | {B} | {H} | {int(causal)} | {ms:.4f} | {tf:.1f} | "
                      f"{tf / peak:.3f} |", flush=True)
            del q, k, v, o, lse
            torch.cuda.empty_cache()


def gemm_calibration(tafa, torch, stream):
    """The rate of the platform's library GEMM (hipBLASLt through torch) on
    large square products, bf16 and E4M3, beside the headline attention in
    the same process: a same-box reference for what an LDS-fed MFMA kernel
    reaches at the clock the part holds under load. The bf16 product uses the
    layout hipBLASLt runs fastest here (second operand stored transposed, as
    F.linear passes it); E4M3 runs through torch._scaled_mm with unit scales.
    Prints one JSON line."""
    import torch.nn.functional as F
    from attn_inputs import BY_NAME, workload_qkv
    gen = torch.Generator(device="cuda:0")
    out = {"note": "library GEMM (hipBLASLt via torch), for context; not part of the product path"}
    for n in (8192, 16384):
        gen.manual_seed(n)
        a = torch.randn(n, n, generator=gen, device="cuda:0").to(torch.bfloat16)
        w = torch.randn(n, n, generator=gen, device="cuda:0").to(torch.bfloat16)
        flop = 2.0 * n ** 3
        ms = min(time_grouped(lambda: F.linear(a, w), 3, 10, 2, stream))
        out[f"bf16_gemm_{n}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
        a8, w8 = a.to(torch.float8_e4m3fn), w.to(torch.float8_e4m3fn)
        one = torch.ones((), device="cuda:0")
        ms = min(time_grouped(lambda: torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one,
                                                       out_dtype=torch.bfloat16), 3, 10, 2, stream))
        out[f"fp8_gemm_{n}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
        del a, w, a8, w8
        torch.cuda.empty_cache()
    wl = BY_NAME[DEFAULT_WORKLOAD]
    q, k, v = workload_qkv(wl, device=torch.device("cuda:0"))
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device="cuda:0")
    ms = min(time_grouped(lambda: tafa.fwd(q, k, v, causal=wl.causal, window=wl.window,
                                           scale=wl.scale, out=o, lse=lse), 3, 5, 2, stream))
    att = workload_flop(wl) / (ms * 1e-3) / 1e12
    best = max(out["bf16_gemm_8192_tflops"], out["bf16_gemm_16384_tflops"])
    out[f"attention_{wl.name}_tflops"] = round(att, 1)
    out["attention_over_best_bf16_gemm"] = round(att / best, 3)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-d256", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="only print a markdown table of throughput across sequence lengths "
                         "(bf16 d 64/128/256, fp8, fp8 PV mode; causal and not)")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="only time the library GEMM (bf16 and E4M3, 8192^3 and 16384^3) beside "
                         "the headline attention, for context; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the known-size "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this attention forward runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported; heads shard across GPUs with no exchange, "
              f"so the per-GPU figure is the one-GPU figure).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 2,
                          "copy_bytes_written_per_launch": dst.numel() * 2}))
        return
    import tiled_attention_forward_attn_amd as tafa
    from attn_inputs import BY_NAME, WORKLOADS, workload_qkv
    tafa.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.sweep:
        run_sweep(tafa, torch, stream)
        return
    if args.gemm_calibration:
        gemm_calibration(tafa, torch, stream)
        return

    w = BY_NAME[DEFAULT_WORKLOAD]
    flop = workload_flop(w)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    q, k, v = workload_qkv(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    print(f"[bench] timing bf16 attention, {args.warmup} warmup + {args.steps} steps",
          file=sys.stderr, flush=True)
    run = lambda: tafa.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=o, lse=lse)
    wall_ms, ev = time_launches(run, args.steps, args.warmup, stream)
    kern_ms = mean_ms(ev)
    tflops = flop / (wall_ms * 1e-3) / 1e12
    achieved = flop / (kern_ms * 1e-3) / 1e12
    traffic = recorded_traffic(w.name, "bf16")
    o_host, lse_host = o.cpu(), lse.cpu()
    del q, k, v, o, lse
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "window": w.window, "scale": w.scale,
                   "algorithmic_tflop_per_step": flop / 1e12},
        "frac_of_dense_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16_kernel<128, 64, 1, 8, false>",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "avg_launch_ms": round(kern_ms, 4)},
    }

    oracle_work = []   # (object, workload, sampled outputs) for the oracle leg
    if not args.no_configs:
        line["configs"] = {}
        for wc in WORKLOADS:
            if wc.name == DEFAULT_WORKLOAD or wc.dtype != "bf16":
                continue
            print(f"[bench] timing {wc.name}", file=sys.stderr, flush=True)
            entry, samples = bench_bf16_config(tafa, wc, dev, args.steps, args.warmup, stream)
            line["configs"][wc.name] = entry
            oracle_work.append((entry, wc, samples))
            torch.cuda.empty_cache()

    if not args.no_fp8:
        line["fp8"] = bench_fp8(tafa, dev, args.steps, args.warmup, stream)
        fp8_samples = line["fp8"].pop("_samples")

    if not args.no_d256:
        # head dimension 256: B8 H16 N8192 (the FLOPs of the headline shape)
        Bh, Hh, Nh, dh = 8, 16, 8192, 256
        print(f"[bench] timing bf16 attention B{Bh} H{Hh} N{Nh} d{dh}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(13)
        q2, k2, v2 = [torch.randn((Bh, Hh, Nh, dh), generator=g, device=dev).to(torch.bfloat16)
                      for _ in range(3)]
        o2 = torch.empty_like(q2)
        l2 = torch.empty((Bh, Hh, Nh), dtype=torch.float32, device=dev)
        _, ev_h = time_launches(lambda: tafa.fwd(q2, k2, v2, scale=1 / math.sqrt(dh), out=o2, lse=l2),
                                max(1, args.steps // 2), args.warmup, stream)
        h_ms = sum(ev_h) / len(ev_h)
        hflop = 4.0 * dh * Nh * Nh * Bh * Hh
        line["d256"] = {"workload": f"B{Bh} H{Hh} N{Nh} d{dh} non-causal, bf16",
                        "tflops": round(hflop / (h_ms * 1e-3) / 1e12, 2),
                        "frac_of_dense_bf16_peak": round(hflop / (h_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "avg_launch_ms": round(h_ms, 4)}
        del q2, k2, v2, o2, l2

    if not args.no_merge:
        # attn_lse_merge of R = 4 fp32 partials of the headline shape (the
        # combination a 4-way split of the keys needs): HBM-bound
        R = 4
        rows = w.B * w.H * w.N
        print(f"[bench] timing attn_lse_merge, R={R} partials of {w.name}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(11)
        o_p = torch.randn((R, w.B, w.H, w.N, w.d), generator=g, device=dev, dtype=torch.float32)
        l_p = torch.randn((R, w.B, w.H, w.N), generator=g, device=dev, dtype=torch.float32)
        om = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        lm = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        _, ev_m = time_launches(lambda: tafa.merge(o_p, l_p, out=om, lse=lm), args.steps, args.warmup, stream)
        m_ms = sum(ev_m) / len(ev_m)
        mbytes = R * rows * (4 * w.d + 4) + rows * (2 * w.d + 4)
        line["lse_merge"] = {
            "workload": f"R={R} fp32 partials of B{w.B} H{w.H} N{w.N} d{w.d}",
            "avg_launch_ms": round(m_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(mbytes / (m_ms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(mbytes / (m_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": mbytes},
        }
        del o_p, l_p, om, lm

    if not args.no_decode:
        # attn_decode: one new query per sequence against a 16K-token cache
        Bd, Hd, Nq, Nk, dd = 32, 32, 1, 16384, 128
        print(f"[bench] timing attn_decode B{Bd} H{Hd} Nq{Nq} Nk{Nk} d{dd}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(12)
        qd = torch.randn((Bd, Hd, Nq, dd), generator=g, device=dev).to(torch.bfloat16)
        kd = torch.randn((Bd, Hd, Nk, dd), generator=g, device=dev).to(torch.bfloat16)
        vd = torch.randn((Bd, Hd, Nk, dd), generator=g, device=dev).to(torch.bfloat16)
        sp = tafa.default_splits(Bd, Hd, Nk)
        ws = torch.empty(tafa.load().attn_decode_workspace_bytes(Bd, Hd, Nq, dd, sp), dtype=torch.uint8,
                         device=dev)
        od = torch.empty_like(qd)
        ld = torch.empty((Bd, Hd, Nq), dtype=torch.float32, device=dev)
        _, ev_d = time_launches(lambda: tafa.decode(qd, kd, vd, causal=True, splits=sp, workspace=ws,
                                                    out=od, lse=ld), args.steps, args.warmup, stream)
        d_ms = sum(ev_d) / len(ev_d)
        dbytes = 2 * kd.numel() * 2 + 2 * qd.numel() * 2 + ld.numel() * 4
        line["decode"] = {
            "workload": f"B{Bd} H{Hd} Nq{Nq} Nk{Nk} d{dd} causal, {sp} key chunks per head",
            "avg_ms": round(d_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(dbytes / (d_ms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dbytes / (d_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": dbytes},
        }
        del kd, vd

        # attn_decode_paged: the same step against a paged cache of 64-position
        # pages scattered over the pool in random order
        ps = 64
        print(f"[bench] timing attn_decode_paged B{Bd} H{Hd} Nq{Nq} seq {Nk} d{dd} page {ps}",
              file=sys.stderr, flush=True)
        P = Bd * Nk // ps
        kc = torch.randn((P, Hd, ps, dd), generator=g, device=dev, dtype=torch.bfloat16)
        vc = torch.randn((P, Hd, ps, dd), generator=g, device=dev, dtype=torch.bfloat16)
        table = torch.randperm(P, generator=g, device=dev).to(torch.int32).reshape(Bd, Nk // ps)
        lens = torch.full((Bd,), Nk, dtype=torch.int32, device=dev)
        _, ev_p = time_launches(lambda: tafa.decode_paged(qd, kc, vc, table, lens, causal=True, splits=sp,
                                                          workspace=ws, out=od, lse=ld),
                                args.steps, args.warmup, stream)
        p_ms = sum(ev_p) / len(ev_p)
        pbytes = dbytes + table.numel() * 4 + lens.numel() * 4
        line["decode_paged"] = {
            "workload": f"B{Bd} H{Hd} Nq{Nq} seq_len {Nk} d{dd} causal, {ps}-position pages in random "
                        f"pool order, {sp} key chunks per head",
            "avg_ms": round(p_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(pbytes / (p_ms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(pbytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": pbytes},
        }
        del qd, kc, vc, table, lens, ws, od, ld

    if not args.no_cpu_baseline:
        # the oracle leg: the fp64 oracle timed on host cores, and the accuracy
        # of every timed workload's sampled outputs against it
        print("[bench] timing the fp64 oracle on host cores", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, o_host, lse_host)
        for entry, wc, samples in oracle_work:
            print(f"[bench] oracle: accuracy of {wc.name}", file=sys.stderr, flush=True)
            entry["accuracy_vs_fp64_oracle"] = bf16_accuracy(wc, samples)
        if not args.no_fp8:
            print("[bench] oracle: fp8 RMSE/RMS per mode", file=sys.stderr, flush=True)
            line["fp8"]["B8"]["accuracy_vs_unquantised_fp64_oracle"] = fp8_accuracy(*fp8_samples)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
