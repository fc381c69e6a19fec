#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (all query tiles of all batches and heads),
inputs resident in HBM before timing starts. Prints ONE JSON line on stdout; progress goes to
stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_gqa] [--no-cpu-baseline]
                  [--layout bhnd|bnhd] [--mask none|keep|add] [--backward]

--backward times attn_bwd instead (one step = the dQ kernel and the dK/dV kernel over the whole
workload, given O and LSE from one forward run before timing and a seeded dO), against the
nominal backward flop count 2.5x the forward's (five N x N x D products: dV, dP, dQ, dK and the
recomputed S); the kernels also recompute S and dP a second time, so the MFMA work they issue is
7/5 of that count.

--dtype f32|f16|bf16 replaces the workload's input type (f32: fp32 products on the fp32 matrix
cores, against their 157.3 TFLOP/s dense peak).
--head-dim D replaces the workload's head dimension (16, 32, 64, 128 or 256; scale 1/sqrt(D));
the flop count follows D.
--layout bnhd stores Q, K, V and O as [B, N, H, D] and runs the strided entry point on them.
--mask keep adds an explicit [N, N] uint8 sliding-window mask (key j visible to query i when
|i - j| < 2048) and --mask add an [N, N] additive mask of the input dtype (-|i - j| / 256), both
shared by every batch and head and combined with the workload's own masks; the flop count stays
the nominal one.

Throughput is the nominal forward flop count 4*B*Hq*N^2*D (halved under causal masking) per
second, at the median of the K per-launch times measured with HIP events on the stream the
kernel is launched on (the mean, min, max and the host clock are in the `timing` object). The
roofline object reports that flop rate against the dense 16-bit MFMA peak; `traffic` is the HBM
byte count from rocprofv3 counters recorded in profiles/ for the current sources (null if any of
them changed since). The cpu_baseline object times the fp64 oracle on a bounded sample of whole
(batch, head) slices of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s, bf16 causal N=4096 D=128; % of MFMA dense peak"
METRIC_BWD = "attention bwd TFLOP/s (nominal 2.5x forward flops), bf16 causal N=4096 D=128"
PEAK_TFLOPS_16BIT_DENSE = 2500.0   # MI355X published dense bf16/fp16 MFMA peak
PEAK_TFLOPS_F32_DENSE = 157.3      # MI355X published dense fp32 MFMA peak
PEAK_SOURCE = ("AMD's published MI355X dense (no sparsity) MFMA peaks: 2.5 PFLOP/s bf16/fp16, "
               "157.3 TFLOP/s fp32")
CSRC = os.path.join(ROOT, "scaled_dot_product_fwd_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "attn_fwd.hip")
KERNEL_SRC_BWD = os.path.join(CSRC, "attn_bwd.hip")
# The sources each kind of kernel is compiled from: its own file, the shared device header and
# the C ABI header. A recorded profile belongs to the sources whose fingerprint it names.
SOURCES = {
    "fwd": ["attn_fwd.hip", "attn_common.h", "attn.h"],
    "fwd_f32": ["attn_fwd_f32.hip", "attn_common.h", "attn.h"],
    "bwd": ["attn_bwd.hip", "attn_common.h", "attn.h"],
    "bwd_f32": ["attn_bwd_f32.hip", "attn_common.h", "attn.h"],
}
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def flops(w) -> float:
    f = 4.0 * w.B * w.Hq * w.N * w.N * w.D
    return f / 2 if w.causal else f


def flops_bwd(w) -> float:
    return 2.5 * flops(w)


def effective_flops(w, valid_len) -> float:
    """4 * D flops per (query, visible key) pair actually computed: with padding, sum over the
    batches of the visible pairs of every query row (causal: min(i + 1, valid) keys for row i)."""
    N = w.N
    total = 0
    for b in range(w.B):
        v = N if valid_len is None else min(max(int(valid_len[b]), 0), N)
        if w.causal:
            # rows i < v see i + 1 keys, rows i >= v see v keys
            total += v * (v + 1) // 2 + (N - v) * v
        else:
            total += N * v
    return 4.0 * w.D * w.Hq * total


def code_only(text: bytes) -> bytes:
    """C/C++ source without its comments, every run of white space one blank: what the compiler
    sees, so that an edit of comments or layout keeps a profile current."""
    out = re.sub(rb"/\*.*?\*/|//[^\n]*", b" ", text, flags=re.S)
    return re.sub(rb"\s+", b" ", out).strip()


def source_fingerprint(kind: str) -> str:
    """sha256 over the names and code (comments and layout removed) of the sources a kind of
    kernel is built from."""
    h = hashlib.sha256()
    for name in SOURCES[kind]:
        path = os.path.join(ROOT, "include", name) if name.endswith("attn.h") else \
            os.path.join(CSRC, name)
        with open(path, "rb") as f:
            data = code_only(f.read())
        h.update(name.encode() + b"\0" + str(len(data)).encode() + b"\0" + data)
    return h.hexdigest()


def traffic_for(workload: str, backward: bool = False):
    """HBM bytes per launch (per attn_bwd call with backward) from committed rocprofv3 counter
    runs, if they were taken on the current sources."""
    name = "traffic_%s%s.json" % (workload, "_bwd" if backward else "")
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    fp = t.get("source_fingerprint") or {}
    if fp.get("sha256") != source_fingerprint(fp.get("kind", "bwd" if backward else "fwd")):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, case, target_s: float):
    """Time the oracle on whole (b, hq) slices (so the causal row-length mix is the workload's),
    sized to about target_s seconds; rate scaled by the exact flop share of the sample."""
    import oracle
    q, k, v = case.widened()
    threads = oracle.max_threads()
    heads_total = w.B * w.Hq
    order = np.random.default_rng(0).permutation(heads_total)

    def rows_of(heads):
        return np.concatenate([np.arange(h * w.N, (h + 1) * w.N, dtype=np.int64) for h in heads])

    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, case.scale, case.causal, case.valid_len, rows=rows_of(order[:1]))
    t1 = time.perf_counter() - t0
    nheads = int(max(1, min(heads_total, round(target_s / max(t1, 1e-3)))))
    heads = order[:nheads]
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, case.scale, case.causal, case.valid_len, rows=rows_of(heads))
    dt = time.perf_counter() - t0
    sample_flops = flops(w) * nheads / heads_total
    return {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d (batch, head) slices, all %d query rows each, %.1f s; "
                      "flops scaled by the slice share" % (nheads, heads_total, w.N, dt)}


def cpu_baseline_bwd(w, case, dout_bits, target_s: float):
    """Time the oracle's backward on whole (batch, KV head) groups (every query head of the
    group, all rows), sized to about target_s seconds; rate scaled by the groups' flop share."""
    import oracle
    from scaled_dot_product_fwd_amd import inputs
    threads = oracle.max_threads()
    g = w.Hq // w.Hkv
    groups_total = w.B * w.Hkv
    order = np.random.default_rng(0).permutation(groups_total)

    def run(sel):
        picks = [(int(x) // w.Hkv, int(x) % w.Hkv) for x in sel]
        wd = lambda a: inputs.widen(a, w.dtype)
        qs = wd(np.stack([case.q_bits[b, h * g:(h + 1) * g] for b, h in picks]))
        ks = wd(np.stack([case.k_bits[b, h:h + 1] for b, h in picks]))
        vs = wd(np.stack([case.v_bits[b, h:h + 1] for b, h in picks]))
        ds = wd(np.stack([dout_bits[b, h * g:(h + 1) * g] for b, h in picks]))
        vl = None if case.valid_len is None else case.valid_len[[b for b, _ in picks]]
        t0 = time.perf_counter()
        oracle.attn_bwd(qs, ks, vs, ds, case.scale, case.causal, vl, threads=threads)
        return time.perf_counter() - t0

    # groups run one per thread: time one round of `threads` groups, then size the sample
    n = min(groups_total, threads)
    t1 = run(order[:n])
    rounds = int(max(1, min(groups_total // n, round(target_s / max(t1, 1e-3)))))
    n = min(groups_total, rounds * n)
    dt = run(order[:n])
    sample_flops = flops_bwd(w) * n / groups_total
    return {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "backward of %d of %d (batch, KV head) groups (%d query heads, all %d rows "
                      "each), %.1f s; flops scaled by the group share" % (
                          n, groups_total, g, w.N, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The device's clock settles over the first ~20 launches of this workload (per-launch time
    # falls from ~1.4 ms to ~1.06 ms), so the default warm-up covers that before timing.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="long_gqa")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--layout", choices=("bhnd", "bnhd"), default="bhnd",
                    help="memory layout of Q, K, V and O")
    ap.add_argument("--mask", choices=("none", "keep", "add"), default="none",
                    help="explicit mask to add (see the module docstring)")
    ap.add_argument("--dtype", choices=("f16", "bf16", "f32"), default=None,
                    help="replace the workload's input type")
    ap.add_argument("--head-dim", type=int, default=0, metavar="D",
                    help="replace the workload's head dimension")
    ap.add_argument("--backward", action="store_true",
                    help="time attn_bwd (dQ, dK, dV) instead of the forward")
    ap.add_argument("--no-split", action="store_true",
                    help="keep small grids on one workgroup per query tile (no attn_fwd_ws)")
    ap.add_argument("--log-launches", action="store_true",
                    help="also print every timed launch's time (ms) to stderr")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only; there is no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d MiB three times" % args.copy_calibration)
        return
    import scaled_dot_product_fwd_amd as sdp
    from scaled_dot_product_fwd_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    import dataclasses
    if args.head_dim:
        w = dataclasses.replace(w, D=args.head_dim)
    if args.dtype:
        w = dataclasses.replace(w, dtype=args.dtype)
    log("workload %s: B=%d Hq=%d Hkv=%d N=%d D=%d %s causal=%s padded=%s" % (
        w.name, w.B, w.Hq, w.Hkv, w.N, w.D, w.dtype, w.causal, w.padded))
    case = inputs.make_workload(w)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]

    def dev(bits):
        if w.dtype == "f32":
            return torch.from_numpy(bits.view(np.float32)).cuda()
        return torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()

    q, k, v = dev(case.q_bits), dev(case.k_bits), dev(case.v_bits)
    if args.layout == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    vl = torch.from_numpy(case.valid_len).cuda() if case.valid_len is not None else None
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    amask = None
    if args.mask != "none":
        idx = torch.arange(w.N, device="cuda")
        dist = (idx[:, None] - idx[None, :]).abs()
        if args.mask == "keep":
            amask = dist < 2048
        else:
            amask = (-dist.float() / 256.0).to(tdt)

    # grids too small to fill the device split their key ranges (attn_fwd_ws) into a workspace
    # allocated here, once
    split = not args.no_split and amask is None and w.dtype != "f32"
    n_ws = sdp.attn_fwd_workspace_floats(w.B, w.Hq, w.Hkv, w.N, w.D, w.causal) if split else 0
    fws = torch.empty((n_ws,), dtype=torch.float32, device="cuda") if n_ws > 0 else None
    if n_ws > 0:
        log("key ranges split over workgroups (attn_fwd_ws, %d workspace floats)" % n_ws)

    def step():
        sdp.forward(q, k, v, causal=w.causal, valid_len=vl, scale=w.scale, out=out, lse=lse,
                    stream=stream, layout=args.layout, attn_mask=amask, ws=fws, split=split)

    if args.backward:
        dout_bits = inputs.make_grad(case, [w.c])
        dout = dev(dout_bits)
        if args.layout == "bnhd":
            dout = dout.transpose(1, 2).contiguous()
        step()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        # the workspace with room for the dK/dV split (attn_bwd_ws) where the shape wants one
        ws = torch.empty((sdp.attn_bwd_workspace_floats(w.B, w.Hq, w.Hkv, w.N, w.D),),
                         dtype=torch.float32, device="cuda")

        def step():  # noqa: F811 -- the timed step is the backward
            sdp.backward(q, k, v, out, dout, lse, causal=w.causal, valid_len=vl, scale=w.scale,
                         dq=dq, dk=dk, dv=dv, ws=ws, stream=stream, layout=args.layout,
                         attn_mask=amask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)
    # One HIP event between consecutive launches on the kernel's stream: K per-launch times. The
    # step time is their median (robust to the first launches, which run while the device's
    # clock is still rising); the mean and the host clock around the whole region are reported
    # beside it.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    ms_per_step = float(np.median(per))
    ms_mean = float(per.mean())
    if args.log_launches:
        log("per-launch ms: " + " ".join("%.4f" % x for x in per))
    log("timed %d steps: median %.4f ms, mean %.4f ms, min %.4f, max %.4f ms per step by HIP "
        "events; %.4f ms/step by host clock" % (args.steps, ms_per_step, ms_mean, per.min(),
                                                per.max(), wall * 1e3 / args.steps))
    if torch.isnan(out).any().item():
        raise SystemExit("NaN in the output")
    if args.backward and any(torch.isnan(t).any().item() for t in (dq, dk, dv)):
        raise SystemExit("NaN in the gradients")

    f = flops_bwd(w) if args.backward else flops(w)
    tflops = f / (ms_per_step * 1e-3) / 1e12
    traffic = None
    if args.layout == "bhnd" and amask is None and not args.head_dim and not args.dtype:
        traffic = traffic_for(w.name, backward=args.backward)
    peak = PEAK_TFLOPS_F32_DENSE if w.dtype == "f32" else PEAK_TFLOPS_16BIT_DENSE
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
            "traffic": traffic, "peak_source": PEAK_SOURCE}
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (about %.0f s)" % args.cpu_seconds)
        if args.backward:
            cpu = cpu_baseline_bwd(w, case, dout_bits, args.cpu_seconds)
        else:
            cpu = cpu_baseline(w, case, args.cpu_seconds)
        cpu["value"] = float("%.6g" % cpu["value"])
        log("cpu baseline: %s" % json.dumps(cpu))
    metric = METRIC_BWD if args.backward else METRIC
    # another workload, or a --dtype / --head-dim variant, names its own type and shape
    metric = metric.replace("bf16 causal N=4096 D=128", "%s %sN=%d D=%d" % (
        w.dtype, "causal " if w.causal else "", w.N, w.D))
    line = {
        "metric": metric, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1), rounded to %s)" % w.dtype,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "D": w.D,
                   "causal": w.causal, "padded": w.padded, "scale": w.scale,
                   "layout": args.layout, "explicit_mask": args.mask,
                   "pass": "backward" if args.backward else "forward",
                   "key_split": bool(n_ws > 0) and not args.backward,
                   "flops_per_step": f,
                   "effective_flops_per_step": (
                       (2.5 if args.backward else 1.0) * effective_flops(w, case.valid_len)
                       if w.padded else None)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing": {"statistic": "median of per-launch HIP event times",
                   "median_ms": round(ms_per_step, 5), "mean_ms": round(ms_mean, 5),
                   "min_ms": round(float(per.min()), 5), "max_ms": round(float(per.max()), 5),
                   "mean_tflops": round(f / (ms_mean * 1e-3) / 1e12, 2),
                   "host_ms_per_step": round(wall * 1e3 / args.steps, 5)},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
