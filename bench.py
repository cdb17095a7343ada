"""Throughput of the sliding-window attention forward pass on one MI355X.

One JSON line on stdout.  The headline is causal prefill at T=16384,
W=4096, H_q=32, H_kv=8, d_h=128, bf16 (band-TFLOP/s: 4*d_h FLOP per attended
(query head, key) pair, masked tile work excluded).  The other workloads
(causal prefill B=2 T=32768 W=1024 local-layer shape, ring decode B=64 W=4096,
Longformer B=8 T=4096 r=256, chunked prefill of 512-token chunks over a ring
cache, prefill with attention sinks, dilated prefill, prefill with RoPE applied
inside the call) are reported in "extra".

Timing: inputs resident in HBM, W untimed warm-up launches (and at least
50 ms of them), then K launches
bracketed by torch.cuda.synchronize() and HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes to
the library).  A separate pass then times up to 50 launches one by one for the
median / min / p90 ("launch_ms"); "inputs" gives the generator, seed and the
SHA-256 of the headline's host inputs.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only prefill|local|decode|longformer|chunk|sinks|dilated|rope]
                       [--profile-copy]
"""

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sliding_window_attention_amd import binding as bd  # noqa: E402
from sliding_window_attention_amd import inputs as inp  # noqa: E402

METRIC = "SWA prefill band-TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def causal_pairs(T, W):
    """Attended (query, key) pairs per head of a causal window: sum_t min(t+1, W)."""
    w = min(W, T)
    return T * w - w * (w - 1) // 2


def longformer_pairs(T, r, dil, globals_):
    """Attended pairs per batch row, summed over heads, counted directly from the
    window bounds (global rows attend all T; other rows add the globals outside
    their window)."""
    G = np.asarray(sorted(globals_), dtype=np.int64)
    i = np.arange(T, dtype=np.int64)
    is_g = np.isin(i, G)
    total = 0
    for d in dil:
        k_lo = np.maximum(-r, -(i // d))
        k_hi = np.minimum(r, (T - 1 - i) // d)
        win = k_hi - k_lo + 1
        extra = np.zeros(T, dtype=np.int64)
        for g in G:
            diff = i - g
            inside = (diff % d == 0) & (np.abs(diff) <= r * d)
            extra += (~inside).astype(np.int64)
        total += int(np.where(is_g, T, win + extra).sum())
    return total


def measured_traffic(kernel_key):
    """HBM bytes per dispatch of one kernel, as recorded from rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain-copy calibration) in
    profiles/hbm_traffic.json.  None when the file is missing, the kernel was
    not recorded, or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        k = rec["kernels"][kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    return dict(bytes=k["read_bytes"] + k["write_bytes"], read_bytes=k["read_bytes"],
                write_bytes=k["write_bytes"])


LAUNCH_STATS = {}


def time_launches(fn, steps, warmup, name=None):
    """Average ms per launch over `steps` back-to-back launches (one event pair
    around all of them).  With `name`, a second, separate pass brackets each of
    up to 50 launches with its own event pair and records median / min / p90
    in LAUNCH_STATS[name]; it is not part of the timed average."""
    # at least `warmup` launches and at least 50 ms of them, so that short
    # kernels also reach the steady clock before the timed launches
    t_w = time.perf_counter()
    n_w = 0
    while n_w < warmup or time.perf_counter() - t_w < 0.05:
        fn()
        n_w += 1
        if n_w % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if name is not None:
        n = min(steps, 50)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, b in ev:
            a.record(s)
            fn()
            b.record(s)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        LAUNCH_STATS[name] = dict(n=n, median=round(float(np.median(t)), 4),
                                  min=round(float(t.min()), 4),
                                  p90=round(float(np.quantile(t, 0.9)), 4))
    return e0.elapsed_time(e1) / steps, wall


def inputs_sha256(*tensors):
    """SHA-256 over the raw bytes of the generated host inputs, in order."""
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                 else t.contiguous().view(torch.int16).numpy().tobytes())
    return h.hexdigest()


def bench_prefill(c, steps, warmup, name=None):
    qh, kh, vh = inp.prefill_inputs(c)
    sha = inputs_sha256(qh, kh, vh)
    q, k, v = qh.cuda(), kh.cuda(), vh.cuda()
    del qh, kh, vh
    o = torch.empty_like(q)
    ms, _ = time_launches(lambda: bd.prefill(q, k, v, c.W, out=o), steps, warmup, name)
    flops = 4.0 * c.D * c.Hq * c.B * causal_pairs(c.T, c.W)
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel())
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(ms=ms, tflops=tflops, flops=flops, bytes=nbytes, sha256=sha)


def causal_sink_pairs(T, W, n_sink):
    """Attended pairs per head with n_sink sink tokens: the window pairs plus, for
    every row t >= W, the sinks s < n_sink that lie before its window."""
    extra = sum(min(n_sink, t - W + 1) for t in range(W, T)) if n_sink else 0
    return causal_pairs(T, W) + extra


def bench_prefill_sinks(c, n_sink, steps, warmup):
    q, k, v = (x.cuda() for x in inp.prefill_inputs(c))
    z = torch.from_numpy(np.random.default_rng(c.seed + 7).standard_normal(c.Hq).astype(np.float32))
    z = z.cuda()
    o = torch.empty_like(q)
    ms, _ = time_launches(lambda: bd.prefill_sinks(q, k, v, c.W, n_sink=n_sink, sink_logit=z, out=o),
                          steps, warmup)
    flops = 4.0 * c.D * c.Hq * c.B * causal_sink_pairs(c.T, c.W, n_sink)
    return dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)


def dilated_pairs(T, W, d):
    """Attended pairs per head of the dilated causal window: sum_t min(W, t // d + 1)."""
    t = np.arange(T, dtype=np.int64)
    return int(np.minimum(W, t // d + 1).sum())


def bench_prefill_dilated(c, dil, steps, warmup):
    q, k, v = (x.cuda() for x in inp.prefill_inputs(c))
    o = torch.empty_like(q)
    ms, _ = time_launches(lambda: bd.prefill_dilated(q, k, v, c.W, dil, out=o), steps, warmup)
    flops = 4.0 * c.D * c.B * sum(dilated_pairs(c.T, c.W, d) for d in dil)
    return dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)


def bench_prefill_rope(c, base, steps, warmup):
    q, k, v = (x.cuda() for x in inp.prefill_inputs(c))
    o = torch.empty_like(q)
    ws = torch.empty(bd.prefill_rope_workspace_size(bd.SWA_BF16, c.B, c.T, c.Hkv, c.D),
                     dtype=torch.uint8, device="cuda")
    ms, _ = time_launches(lambda: bd.prefill_rope(q, k, v, c.W, base, out=o, workspace=ws),
                          steps, warmup)
    flops = 4.0 * c.D * c.Hq * c.B * causal_pairs(c.T, c.W)
    return dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12)


def bench_decode(c, steps, warmup):
    q, kc, vc, sp, cur = (x.cuda() for x in inp.decode_inputs(c))
    o = torch.empty_like(q)
    ws = torch.empty(bd.decode_workspace_size(c.B, c.Hq, c.Hkv, c.W, c.D), dtype=torch.uint8,
                     device="cuda")
    ms, _ = time_launches(lambda: bd.decode(q, kc, vc, sp, cur, out=o, workspace=ws), steps, warmup,
                          "decode")
    nbytes = 2 * (q.numel() + kc.numel() + vc.numel() + o.numel()) + 4 * (sp.numel() + cur.numel())
    return dict(ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9, bytes=nbytes)


def bench_longformer(c, steps, warmup):
    q, k, v, dl, g = inp.longformer_inputs(c)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(q)
    ws = torch.empty(max(1, bd.longformer_workspace_size(c.B, c.T, c.H, c.D, g.shape[1])),
                     dtype=torch.uint8, device="cuda")
    ms, _ = time_launches(lambda: bd.longformer(q, k, v, c.r, dl, g, out=o, workspace=ws),
                          steps, warmup, "longformer")
    pairs = c.B * longformer_pairs(c.T, c.r, c.dilation, c.globals_)
    flops = 4.0 * c.D * pairs
    nbytes = 2 * (q.numel() + k.numel() + v.numel() + o.numel())
    t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
    return dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12, pairs=pairs, bytes=nbytes,
                frac_of_roof=t_roof / (ms * 1e-3))


def bench_chunk(c, steps, warmup):
    q, kc, vc, sp, qp = inp.chunk_inputs(c)
    # attended (query token, slot) pairs, counted from the positions
    spn, qpn = sp.numpy().astype(np.int64), qp.numpy().astype(np.int64)
    pairs = 0
    for b in range(c.B):
        s_ = spn[b][None, :]
        t_ = qpn[b][:, None]
        pairs += int(((s_ >= 0) & (s_ > t_ - c.W) & (s_ <= t_)).sum())
    pairs *= c.Hq
    q, kc, vc, sp, qp = q.cuda(), kc.cuda(), vc.cuda(), sp.cuda(), qp.cuda()
    o = torch.empty_like(q)
    ms, _ = time_launches(lambda: bd.prefill_cached(q, kc, vc, sp, qp, c.W, out=o), steps, warmup)
    flops = 4.0 * c.D * pairs
    return dict(ms=ms, tflops=flops / (ms * 1e-3) / 1e12, pairs=pairs)


def cpu_baseline(c):
    """The fp64 oracle as it is, on every third steady-state row (t >= W, W keys
    each) of the headline workload, all heads, run over the host cores by the
    oracle's process pool (one worker per core, one BLAS thread each); scaled
    to band-TFLOP/s.  The wall time includes the workers' start-up."""
    import oracle
    from oracle import pool

    q, k, v = inp.prefill_inputs(c)
    qn, kn, vn = inp.widen(q), inp.widen(k), inp.widen(v)
    rows = np.arange(c.W, c.T, 3)
    cores = pool.host_cores()
    t0 = time.perf_counter()
    pool.run_rows(oracle.swa_prefill, (qn, kn, vn), rows, dict(W=c.W), workers=cores)
    t_used = time.perf_counter() - t0
    flops = 4.0 * c.D * c.Hq * c.W * len(rows)
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{len(rows)} steady-state query rows (every third t >= W, {c.W} keys each) x all "
                       f"{c.Hq} heads of the T={c.T} W={c.W} workload, {t_used:.1f} s wall on "
                       f"{cores} worker processes (one BLAS thread each, start-up included)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "longformer", "local", "chunk",
                                       "sinks", "dilated", "rope"],
                    default="all", help="restrict to one workload (the headline always runs "
                    "unless decode/longformer/local is chosen)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(prefill would shard by key/value-head group or batch with no communication); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bd.lib()

    if args.profile_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    c2 = inp.C2
    main_r = None
    if args.only in ("all", "prefill"):
        main_r = bench_prefill(c2, args.steps, args.warmup, "headline")
    extra = {}
    if args.only in ("all", "local"):
        r3 = bench_prefill(inp.C3, max(5, args.steps // 2), args.warmup)
        extra["prefill_local_layer"] = dict(
            workload="causal SWA prefill B=2 T=32768 W=1024 Hq=32 Hkv=16 d_h=128 bf16, RoPE inputs",
            value=round(r3["tflops"], 2), unit="TFLOP/s", ms=round(r3["ms"], 4),
            frac_mfma_peak=round(r3["tflops"] / PEAK_BF16_TFLOPS, 4))
    if args.only in ("all", "decode"):
        r4 = bench_decode(inp.C4, max(20, args.steps), args.warmup)
        extra["decode"] = dict(
            workload="ring decode B=64 W=4096 Hq=32 Hkv=8 d_h=128 bf16, cur_pos in [4096, 32768)",
            value=round(r4["gbs"], 1), unit="GB/s", ms=round(r4["ms"], 4),
            frac_hbm_peak=round(r4["gbs"] / PEAK_HBM_GBS, 4), bytes=r4["bytes"],
            traffic=measured_traffic("split_mfma_kernel<128, 4, true, 4>@131072"),
            launch_ms=LAUNCH_STATS.get("decode"))
    if args.only in ("all", "longformer"):
        r5 = bench_longformer(inp.C5, max(20, args.steps), args.warmup)
        extra["longformer"] = dict(
            workload="Longformer B=8 T=4096 H=12 d_h=64 r=256, dilation 2 on heads 8-11, globals {0,8}",
            value=round(r5["tflops"], 2), unit="TFLOP/s", ms=round(r5["ms"], 4),
            frac_of_roofline=round(r5["frac_of_roof"], 4), pairs=r5["pairs"],
            traffic_local_pass=measured_traffic("fwd_kernel<64, 1, 4>@786432"),
            launch_ms=LAUNCH_STATS.get("longformer"))

    if args.only in ("all", "chunk"):
        c6 = inp.C6
        r6 = bench_chunk(c6, max(20, args.steps), args.warmup)
        extra["chunked_prefill"] = dict(
            workload=f"chunked prefill over a ring cache B={c6.B} L={c6.L} S={c6.S} W={c6.W} "
                     f"Hq={c6.Hq} Hkv={c6.Hkv} d_h={c6.D} bf16, chunk start in [{c6.p_lo}, {c6.p_hi})",
            value=round(r6["tflops"], 2), unit="TFLOP/s", ms=round(r6["ms"], 4),
            frac_mfma_peak=round(r6["tflops"] / PEAK_BF16_TFLOPS, 4), pairs=r6["pairs"])

    if args.only in ("all", "sinks"):
        r7 = bench_prefill_sinks(c2, 4, max(5, args.steps // 2), args.warmup)
        extra["prefill_sinks"] = dict(
            workload=f"causal SWA prefill with 4 sink tokens and per-head sink scores, "
                     f"B={c2.B} T={c2.T} W={c2.W} Hq={c2.Hq} Hkv={c2.Hkv} d_h={c2.D} bf16",
            value=round(r7["tflops"], 2), unit="TFLOP/s", ms=round(r7["ms"], 4),
            frac_mfma_peak=round(r7["tflops"] / PEAK_BF16_TFLOPS, 4))

    if args.only in ("all", "dilated"):
        dil = [1] * 16 + [2] * 8 + [4] * 8
        r8 = bench_prefill_dilated(c2, dil, max(5, args.steps // 2), args.warmup)
        extra["prefill_dilated"] = dict(
            workload=f"causal SWA prefill with dilation 1 on heads 0-15, 2 on 16-23, 4 on 24-31, "
                     f"B={c2.B} T={c2.T} W={c2.W} Hq={c2.Hq} Hkv={c2.Hkv} d_h={c2.D} bf16",
            value=round(r8["tflops"], 2), unit="TFLOP/s", ms=round(r8["ms"], 4),
            frac_mfma_peak=round(r8["tflops"] / PEAK_BF16_TFLOPS, 4))

    if args.only in ("all", "rope"):
        c3 = dataclasses.replace(inp.C3, rope=False)  # the call applies the rotation
        r9 = bench_prefill_rope(c3, 1.0e4, max(5, args.steps // 2), args.warmup)
        extra["prefill_rope_local_layer"] = dict(
            workload="causal SWA prefill B=2 T=32768 W=1024 Hq=32 Hkv=16 d_h=128 bf16 with RoPE "
                     "(base 1e4) applied inside the call: keys rotated once, queries in registers",
            value=round(r9["tflops"], 2), unit="TFLOP/s", ms=round(r9["ms"], 4),
            frac_mfma_peak=round(r9["tflops"] / PEAK_BF16_TFLOPS, 4))

    if main_r is None:
        print(json.dumps({"partial": args.only, "extra": extra}), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c2)

    ach = main_r["tflops"]
    tr = measured_traffic("fwd_kernel<128, 0, 4>@1048576")
    out = {
        "metric": METRIC,
        "value": round(ach, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal SWA prefill (one launch per step)", "B": c2.B, "T": c2.T,
                   "W": c2.W, "H_q": c2.Hq, "H_kv": c2.Hkv, "d_h": c2.D, "io": "bf16",
                   "accumulate": "fp32"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if tr is None else tr["bytes"],
                     "traffic_detail": tr,
                     "kernel": "fwd_kernel<128, 0 (causal), 4>",
                     "algorithmic_flop_per_launch": main_r["flops"],
                     "algorithmic_bytes_per_launch": main_r["bytes"]},
        "cpu_baseline": cpu,
        "launch_ms": LAUNCH_STATS.get("headline"),
        "inputs": {"generator": "numpy PCG64 standard_normal float32, rounded to bf16 (RNE)",
                   "seed": c2.seed, "sha256_q_k_v": main_r["sha256"]},
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
