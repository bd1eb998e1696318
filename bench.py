#!/usr/bin/env python3
"""Benchmark of dynamic bifocal RoPE attention on one MI355X.

One step = the whole hot path on one batch of synthetic input, inputs already
resident in HBM:
  * 128K bifocal prefill (bf16 in/out, 32 query / 8 KV heads, d 128,
    w_pretrained 32768 so G = 4, w0 2048, theta 1e6, 64 key rows x4):
    jl_bifocal_prefill_prepare (cos/sin table, rotated keys, transposed
    values) then jl_bifocal_prefill_attend (the attention kernel);
  * decode of 16 sequences against full 131072-key caches (same heads).

Prints one JSON line.  `value` is the prefill throughput in TFLOP/s over the
whole prefill call (algorithmic FLOPs = 4 * d * Hq * L(L+1)/2: one logit and
one PV product per causal pair).  The decode rate (algorithmic bytes = K and
V read once plus Q and O) is reported beside it.  `roofline` covers the
dominant kernel (the prefill attention kernel) timed by itself with HIP
events on the stream it runs on; `cpu_baseline` times the fp64 oracle on the
host cores (one worker process per core) on a bounded sample of the same
workloads: random query-row blocks of the prefill, whole sequences of the
decode.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_16BIT = 2500.0   # TFLOP/s, MI355X dense fp16 / bf16 MFMA
PEAK_HBM = 8000.0          # GB/s, MI355X HBM3E
METRIC = "bifocal prefill TFLOP/s @128K (% bf16 MFMA peak); decode HBM GB/s"


def prefill_flops(lens, Hq, d):
    return sum(4.0 * d * Hq * L * (L + 1) / 2 for L in lens)


def decode_bytes(B, L, Hq, Hkv, d, elem=2):
    return B * L * Hkv * d * elem * 2 + 2 * B * Hq * d * elem


def source_digest(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, digest: str):
    """Counter-derived HBM bytes per launch from profiles/, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(kind: str, name: str, wid: int, nworkers: int, budget_s: float):
    """One CPU-baseline worker (a spawned process with one BLAS thread): draws
    its own share of the workload's inputs (untimed), then runs the oracle, as
    it stands, on its units until the budget is spent.  Returns (work, oracle
    seconds, units) with work in FLOP (prefill) or algorithmic bytes (decode)."""
    import numpy as np
    import oracle
    from zero_shot_rope_bifocal_amd import workloads as W
    w = W.WORKLOADS[name]
    t_end = time.perf_counter() + budget_s
    work = secs = 0.0
    units = 0
    if kind == "prefill":
        L, Hq, Hkv, d = w["lens"][0], w["Hq"], w["Hkv"], w["d"]
        r = Hq // Hkv
        kb, vb = W.prefill_kv(name)
        h = wid % Hkv  # this worker's KV head and its query heads
        k = W.as_f64(kb[:, h:h + 1], "bf16")
        v = W.as_f64(vb[:, h:h + 1], "bf16")
        del kb, vb
        rng = np.random.default_rng(1000 + wid)
        while time.perf_counter() < t_end:
            row0 = int(rng.integers(0, L - 8))
            q = W.as_f64(W.prefill_q_rows(name, row0, 8)[:, h * r:(h + 1) * r], "bf16")
            rows = np.arange(row0, row0 + 8)
            t0 = time.perf_counter()
            oracle.bifocal_sequence(q, k, v, rows, L, w["w_pretrained"], w["w0"], w["theta"])
            secs += time.perf_counter() - t0
            work += float(sum(4.0 * d * r * (i + 1) for i in rows))
            units += 1
    else:
        for b in range(wid, w["B"], nworkers):
            if time.perf_counter() >= t_end:
                break
            qb, kb, vb = W.decode_sequence(name, b)
            q, k, v = (W.as_f64(x, "bf16") for x in (qb, kb, vb))
            del qb, kb, vb
            t0 = time.perf_counter()
            oracle.bifocal_decode(q, k, v, np.array([w["L"]], np.int32), w["w_pretrained"], w["w0"], w["theta"])
            secs += time.perf_counter() - t0
            work += float(w["L"] * w["Hkv"] * w["d"] * 2 * 2 + 2 * w["Hq"] * w["d"] * 2)
            units += 1
    return work, secs, units


def cpu_baseline(kind: str, name: str, budget_s: float, workers: int):
    """The oracle on all host cores: `workers` spawned processes, one BLAS
    thread each, every one timing its own oracle calls on its share of the
    workload.  They run side by side, so the throughput is the sum of the
    per-worker rates.  Returns (rate, work done, units, workers)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"  # inherited by the spawned workers only (this process's BLAS is set up)
    try:
        with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
            res = list(ex.map(_oracle_worker, [kind] * workers, [name] * workers, range(workers),
                              [workers] * workers, [budget_s] * workers))
    finally:
        for k, val in env.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    rate = sum(wk / sc for wk, sc, _ in res if sc > 0)
    return rate, sum(r[0] for r in res), sum(r[2] for r in res), workers


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes for the CPU baseline (capped by os.cpu_count())")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run one stage only (for profiling); the JSON line then covers that stage")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-plain", action="store_true",
                    help="skip the plain-RoPE baseline measured after the timed steps")
    ap.add_argument("--no-ie", action="store_true",
                    help="skip the inclusion-exclusion route measured after the timed steps")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU layout is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import zero_shot_rope_bifocal_amd as jl
    from zero_shot_rope_bifocal_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wp_ = W.WORKLOADS["long_bf16"]
    wd = W.WORKLOADS["decode_bf16"]

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    do_prefill = args.only in (None, "prefill")
    do_decode = args.only in (None, "decode")
    L = wp_["lens"][0]
    Hq, Hkv, d = wp_["Hq"], wp_["Hkv"], wp_["d"]
    if do_prefill:
        log("generating 128K prefill inputs")
        pin = W.workload_inputs("long_bf16")
        q = W.to_device(pin["q"], "bf16", dev)
        k = W.to_device(pin["k"], "bf16", dev)
        v = W.to_device(pin["v"], "bf16", dev)
        cu = torch.from_numpy(pin["cu_q"]).to(dev)
        del pin
        o = torch.empty_like(q)
        ws = torch.empty(jl.prefill_workspace_size(jl.JL_BF16, 1, L, L, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    if do_decode:
        log("generating decode inputs (16 x 131072 keys)")
        din = W.workload_inputs("decode_bf16")
        dq = W.to_device(din["q"], "bf16", dev)
        dk = W.to_device(din["k"], "bf16", dev)
        dv = W.to_device(din["v"], "bf16", dev)
        seq = torch.from_numpy(din["seq_L"]).to(dev)
        do = torch.empty_like(dq)
        dws = torch.empty(jl.decode_workspace_size(jl.JL_BF16, wd["B"], wd["L"], wd["Hq"], wd["Hkv"], wd["d"]),
                          dtype=torch.uint8, device=dev)
        # the cos/sin table of every position the caches hold: built once,
        # like a model's RoPE cache, and read by every decode step
        dtab = jl.rope_table(wd["L"], wd["d"], wd["theta"], device=dev)
        dpart = torch.empty(jl.decode_with_table_workspace_size(jl.JL_BF16, wd["B"], wd["L"], wd["Hq"], wd["Hkv"],
                                                                wd["d"]), dtype=torch.uint8, device=dev)
        del din
    if args.copy_mib:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch
        # calibrate the counters against bytes actually moved
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev:
            ev[0].record()
        if do_prefill:
            jl.prefill_prepare(k, v, cu, L, wp_["w_pretrained"], wp_["theta"], Hq=Hq, workspace=ws)
        if ev:
            ev[1].record()
        if do_prefill:
            jl.prefill_attend(q, k, v, cu, L, wp_["w_pretrained"], wp_["w0"], wp_["theta"], ws, out=o)
        if ev:
            ev[2].record()
        if do_decode:
            jl.decode_with_table(dq, dk, dv, seq, wd["w_pretrained"], wd["w0"], dtab, wd["L"], out=do,
                                 workspace=dpart)
        if ev:
            ev[3].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep = [e[0].elapsed_time(e[1]) for e in evs]
    attn = [e[1].elapsed_time(e[2]) for e in evs]
    dec = [e[2].elapsed_time(e[3]) for e in evs]
    tot = [e[0].elapsed_time(e[3]) for e in evs]
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    median = lambda xs: sorted(xs)[len(xs) // 2] if len(xs) % 2 else sum(sorted(xs)[len(xs) // 2 - 1:len(xs) // 2 + 1]) / 2  # noqa: E731
    prep_ms, attn_ms, dec_ms, step_ms = mean(prep), mean(attn), mean(dec), mean(tot)
    fl = prefill_flops(wp_["lens"], Hq, d)
    pre_tflops = fl / ((prep_ms + attn_ms) * 1e-3) / 1e12 if do_prefill else 0.0
    attn_tflops = fl / (attn_ms * 1e-3) / 1e12 if do_prefill else 0.0
    db = decode_bytes(wd["B"], wd["L"], wd["Hq"], wd["Hkv"], wd["d"])
    dec_gbs = db / (dec_ms * 1e-3) / 1e9 if do_decode else 0.0

    # the digests cover the kernel sources and the build flags they are compiled with
    digest = source_digest("zero_shot_rope_bifocal_amd/csrc/prefill_bf16.hip",
                           "zero_shot_rope_bifocal_amd/csrc/jl_device.hpp", "zero_shot_rope_bifocal_amd/build.py")
    traffic = load_traffic("prefill_attn", digest)
    ddigest = source_digest("zero_shot_rope_bifocal_amd/csrc/decode.hip",
                            "zero_shot_rope_bifocal_amd/csrc/jl_device.hpp", "zero_shot_rope_bifocal_amd/build.py")
    dtraffic = load_traffic("decode_split", ddigest)

    # plain RoPE causal attention on the same kernels, after the timed region:
    # prefill with G = 1 and w0 = 0 (every pair at its true position), decode
    # over a pre-rotated cache with every key in the window (no rotation).
    plain = None
    if not args.no_plain:
        log("plain-RoPE baseline")

        def clock(fn, reps=2):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        plain = {"definition": "prefill: same kernels with w_pretrained = L (G = 1) and w0 = 0; decode: "
                               "pre-rotated cache with w0 >= L, i.e. plain RoPE decode over a RoPE cache (no "
                               "table, no key rotation, stored keys on the bf16 MFMA)"}
        if do_prefill:
            jl.prefill_prepare(k, v, cu, L, L, wp_["theta"], Hq=Hq, workspace=ws)
            p_ms = clock(lambda: jl.prefill_attend(q, k, v, cu, L, L, 0, wp_["theta"], ws, out=o))
            plain["prefill_attend_ms"] = round(p_ms, 3)
            plain["prefill_attend_TFLOPs"] = round(fl / (p_ms * 1e-3) / 1e12, 2)
            plain["bifocal_over_plain_prefill_speed"] = round(p_ms / attn_ms, 4)
        if do_decode:
            d_ms = clock(lambda: jl.decode_with_table(dq, dk, dv, seq, wd["w_pretrained"], wd["L"] + 1, dtab, wd["L"],
                                                      out=do, workspace=dpart, prerotated=True), reps=20)
            b_ms = clock(lambda: jl.decode_with_table(dq, dk, dv, seq, wd["w_pretrained"], wd["w0"], dtab, wd["L"],
                                                      out=do, workspace=dpart), reps=20)
            plain["decode_ms"] = round(d_ms, 4)
            plain["bifocal_decode_ms_same_clock"] = round(b_ms, 4)
            plain["bifocal_decode_overhead"] = round(b_ms / d_ms - 1.0, 4)

    # the pages' own route to the same prefill (three passes + LSE merge), on
    # the same inputs, after the timed region
    ie = None
    if not args.no_ie and do_prefill:
        log("inclusion-exclusion route")
        iws = torch.empty(jl.prefill_ie_workspace_size(jl.JL_BF16, 1, L, L, L, Hq, Hkv, d), dtype=torch.uint8,
                          device=dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        run_ie = lambda: jl.prefill_ie(q, k, v, cu, L, wp_["w_pretrained"], wp_["w0"], wp_["theta"],  # noqa: E731
                                       out=o, workspace=iws)
        run_ie()
        torch.cuda.synchronize()
        a.record()
        for _ in range(2):
            run_ie()
        b.record()
        torch.cuda.synchronize()
        ie_ms = a.elapsed_time(b) / 2
        ie = {"definition": "prepare + window pass (true positions) + full causal pass (grouped positions) + "
                            "window pass (grouped positions) + LSE merge, fp32 pass outputs",
              "prefill_ms": round(ie_ms, 3),
              "TFLOPs_equiv": round(fl / (ie_ms * 1e-3) / 1e12, 2),
              "routed_over_ie_speed": round(ie_ms / (prep_ms + attn_ms), 4)}
        del iws

    # decode alone, 50 back-to-back calls after the timed region (median,
    # min): over the prepared table, and building its cos/sin rows per call
    dec50 = dec50_rows = None
    if do_decode and not args.only:
        def fifty(fn):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            d50 = [a.elapsed_time(b) for a, b in ev]
            return [round(median(d50), 4), round(min(d50), 4)]
        dec50 = fifty(lambda: jl.decode_with_table(dq, dk, dv, seq, wd["w_pretrained"], wd["w0"], dtab, wd["L"],
                                                   out=do, workspace=dpart))
        dec50_rows = fifty(lambda: jl.decode(dq, dk, dv, seq, wd["w_pretrained"], wd["w0"], wd["theta"], out=do,
                                             workspace=dws))

    cpu = None
    if not args.no_cpu_baseline:
        # the machine's CPU share for one GPU is 16 cores, whatever os.cpu_count() says
        workers = max(1, min(os.cpu_count() or 1, args.cpu_workers))
        cpu = {"kind": "oracle", "cores": workers, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
               "threads_per_core": 1}
        if do_prefill:
            log(f"cpu baseline, prefill ({workers} workers, {args.cpu_seconds:.0f} s)")
            val, fl, units, _ = cpu_baseline("prefill", "long_bf16", args.cpu_seconds, workers)
            cpu.update(value=val / 1e12, unit="TFLOP/s",
                       sample=f"{units} blocks of 8 consecutive query rows (random starts) x the 4 query heads of "
                              f"one KV head, of the L=131072 prefill against all keys; fp64 numpy oracle; "
                              f"{fl:.3g} FLOP in all")
        if do_decode:
            log(f"cpu baseline, decode ({workers} workers)")
            val, by, units, _ = cpu_baseline("decode", "decode_bf16", max(args.cpu_seconds, 60.0), workers)
            cpu["decode"] = {"value": val / 1e9, "unit": "GB/s", "sample":
                             f"{units} of the 16 sequences of the 16 x 131072 decode, whole (all heads, all keys); "
                             f"fp64 numpy oracle; {by:.3g} algorithmic bytes"}
            if not do_prefill:
                cpu.update(value=val / 1e9, unit="GB/s", sample=cpu["decode"]["sample"])

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": METRIC,
        "value": round(pre_tflops, 2) if do_prefill else round(dec_gbs, 1),
        "unit": "TFLOP/s" if do_prefill else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "prefill L=131072 (32/8 heads, d=128, w_pretrained=32768 -> G=4, w0=2048, theta=1e6, "
                        "64 key rows x4) + decode B=16 x L=131072 (same heads)",
            "io_dtype": "bf16",
            "mfma_operands": "f16 (rotated q/k, p, v), fp32 accumulate",
            "prefill_ms": round(prep_ms + attn_ms, 3) if do_prefill else None,
            "prefill_prepare_ms": round(prep_ms, 3) if do_prefill else None,
            "prefill_attend_ms": round(attn_ms, 3) if do_prefill else None,
            "decode_ms": round(dec_ms, 4) if do_decode else None,
            "prefill_attend_ms_median_min": [round(median(attn), 3), round(min(attn), 3)] if do_prefill else None,
            "decode_ms_median_min": [round(median(dec), 4), round(min(dec), 4)] if do_decode else None,
            "decode_ms_median_min_50": dec50,
            "decode_building_table_rows_ms_median_min_50": dec50_rows,
            "decode_definition": "one step = jl_bifocal_decode_with_table (split-K kernel + combine) over a cos/sin "
                                 "table of all 131072 positions built once before the timed region; "
                                 "jl_bifocal_decode, which builds the rows it reads on every call, is timed beside it",
            "decode_GBps": round(dec_gbs, 1) if do_decode else None,
            "decode_frac_hbm_peak": round(dec_gbs / PEAK_HBM, 4) if do_decode else None,
            "prefill_frac_mfma_peak": round(pre_tflops / PEAK_MFMA_16BIT, 4) if do_prefill else None,
            "stages": args.only or "prefill+decode",
            "gpu": props.name,
            "cu_count": props.multi_processor_count,
            "wall_s_timed": round(wall, 3),
        },
        "roofline": {
            "kernel": "prefill attention (attn_kernel<128,4>)",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_MFMA_16BIT,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_MFMA_16BIT, 4),
            "traffic": traffic,
        } if do_prefill else None,
        "roofline_decode": {
            "kernel": "decode (split + combine over the prepared table)",
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM, 4),
            "traffic": dtraffic,
        } if do_decode else None,
        "cpu_baseline": cpu,
        "plain_rope_baseline": plain,
        "inclusion_exclusion_route": ie,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
