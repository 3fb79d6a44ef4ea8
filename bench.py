"""Throughput of the lightning indexer on one MI355X.

Headline: indexer score + top-k pairs/s of the fused fp8 prefill at
L = 32768 (B=1, H=64, D=128, k=2048, OCP e4m3 with per-row fp32 scales,
causal); a step is one indexer_prefill call over inputs already resident in
HBM.  Alongside, in the same JSON line: paged-decode K-cache GB/s for the
64 x 131072 contiguous workload and the 128-query scattered-page workload,
the roofline of the dominant kernel, and the CPU oracle timed on a bounded
sample of the headline workload (whose rows are also parity-checked against
the GPU output).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer score+top-k pairs/s (prefill L=32K) and decode K-cache GB/s"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

# HBM traffic per launch from two rocprofv3 counter passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) over `bench.py --steps 2 --warmup 1
# --no-cpu-baseline --copy-calibration`.  Each counter is scaled by what it
# reads for a 1 GiB device-to-device copy (FETCH_SIZE 524315.5 KiB, WRITE_SIZE
# 1048576.0 KiB).  A record applies only while the kernel's sources hash to
# the value it was taken at; otherwise traffic is reported as null.
COPY_FETCH_FACTOR = 1048576.0 / 524315.5
COPY_WRITE_FACTOR = 1048576.0 / 1048576.0
_DECODE_SRC = ["csrc/decode_paged.hip", "csrc/select_row.h", "csrc/common.h", "csrc/kernels.h", "build.py"]
_DECODE_SHA = "98816410d2ad66fc654ebd73ea1412957325d177b33375d34187322513b8bb50"
COUNTERS = {
    "prefill": {"sources": ["csrc/prefill_ws.hip", "csrc/rowbuf.h", "csrc/varlen.h", "csrc/common.h", "csrc/kernels.h",
                            "build.py"],
                "sha256": "8716ea67a91e407f862c95a89fba2b4518b2e0d852a0e95bb2dad72b274757d6",
                "fetch_kib": 256229.1, "write_kib": 524378.5},
    # main scan of one decode call, the sample inside it (which re-reads about 1/60 of the cache)
    "decode_scan_w4": {"sources": _DECODE_SRC, "sha256": _DECODE_SHA, "fetch_kib": 556828.7, "write_kib": 2382.2},
    "decode_scan_w5": {"sources": _DECODE_SRC, "sha256": _DECODE_SHA, "fetch_kib": 570465.3, "write_kib": 4139.6},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def up(torch, a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def time_calls(torch, fn, steps, warmup, warm_seconds=0.2, samples=20):
    """Runs fn at least `warmup` times and for at least `warm_seconds` (after
    the host-side input generation the GPU needs a few hundred calls of a
    short op to reach its steady clocks), then
    * exactly `steps` times back to back between one pair of HIP events on
      the current stream (the stream the library launches on), with a device
      synchronisation on both sides: the mean, and the wall time of that
      region;
    * `samples` more calls, each between a pair of events of its own: the
      median and the minimum per call.
    Returns a dict of milliseconds (mean_ms, median_ms, min_ms) and wall_s."""
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < warm_seconds:
        fn()
        done += 1
        if done % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"mean_ms": a.elapsed_time(b) / steps, "median_ms": float(np.median(per)), "min_ms": float(per.min()),
            "wall_s": wall}


def stats(t, scale=1.0, unit="ms"):
    """The timing dict of time_calls in the JSON line's units."""
    return {f"{unit}_mean": t["mean_ms"] * scale, f"{unit}_median": t["median_ms"] * scale,
            f"{unit}_min": t["min_ms"] * scale}


def measured_traffic(name):
    """Calibrated HBM bytes per launch of kernel `name`, or None when its
    sources changed since the counters were taken."""
    import hashlib
    rec = COUNTERS[name]
    pkg = os.path.join(ROOT, "dsa_lightning_indexer_03_amd")
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sha256"]:
        return None
    return (rec["fetch_kib"] * COPY_FETCH_FACTOR + rec["write_kib"] * COPY_WRITE_FACTOR) * 1024.0


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline_prefill(inp, K, gpu_idx, gpu_val, seconds):
    """The oracle as it stands on a time-bounded, seeded sample of rows of
    the headline workload; the sampled rows are also checked against the
    GPU's output of the timed run."""
    from oracle import indexer
    from oracle.check import check_topk_rows

    L = inp["q"].shape[1]
    rng = np.random.default_rng(12345)
    first = [0, K - 2, K - 1, K, L - 1]
    rest = [int(x) for x in rng.permutation(L) if int(x) not in first]
    order = first + rest
    done, pairs, t_oracle = [], 0, 0.0
    chunk = 16
    i = 0
    while i < len(order) and t_oracle < seconds:
        rows = np.array(order[i:i + chunk])
        t0 = time.perf_counter()
        oi, ov, osc = indexer.prefill(inp, K, rows=rows, want_scores=True)
        t_oracle += time.perf_counter() - t0
        check_topk_rows(gpu_idx[rows], gpu_val[rows], osc[0], rows + 1, K, where="bench prefill sample")
        done += rows.tolist()
        pairs += int((rows + 1).sum())
        i += chunk
    threads, api = blas_threads()
    return {"value": pairs / t_oracle, "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} seeded rows of the L=32768 fp8 workload (incl. t=0,{K-2},{K-1},{K},{L-1}); "
                      f"{pairs} causal pairs scored + full-sort top-k in {t_oracle:.1f} s, numpy fp64 with "
                      f"{threads} {api} threads; every sampled row parity-checked against the GPU output"}


# A serving batch of chunked-prefill requests: (position of the chunk's first
# query, chunk length) per sequence; two chunks end exactly at position 131072.
VARLEN_SPEC = [(0, 2048), (8192, 1024), (30000, 512), (60000, 2048), (65500, 512), (100000, 1024),
               (126976, 4096), (129024, 2048)]


def bench_varlen(torch, dsa, dev, args):
    """One call over a ragged batch of chunks (VARLEN_SPEC) against a paged
    fp8 cache whose 64-token pages are scattered by a seeded permutation;
    fp8 queries (with per-row scales) and bf16 queries, H=64, D=128, k=2048.
    Inputs are seeded normals generated on the device."""
    H, D, K = 64, 128, 2048
    B = len(VARLEN_SPEC)
    lens = [q0 + lq for q0, lq in VARLEN_SPEC]
    pages = [(n + 63) // 64 for n in lens]
    mpp, n_pages = max(pages), sum(pages)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    perm = torch.randperm(n_pages, generator=g, device=dev).to(torch.int32)
    table = torch.zeros((B, mpp), dtype=torch.int32, device=dev)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[off:off + n]
        off += n
    kf = torch.randn((n_pages * 64, D), generator=g, device=dev)
    ksc = (kf.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
    kc = (kf / ksc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).view(n_pages, 64, D)
    ksc = ksc.view(n_pages, 64).contiguous()
    del kf
    T = sum(lq for _, lq in VARLEN_SPEC)
    cu = torch.tensor([0] + list(np.cumsum([lq for _, lq in VARLEN_SPEC])), dtype=torch.int32, device=dev)
    q_start = torch.tensor([q0 for q0, _ in VARLEN_SPEC], dtype=torch.int32, device=dev)
    qf = torch.randn((T, H, D), generator=g, device=dev)
    qsc = (qf.abs().amax(dim=2) / 448.0).clamp_min(1e-30)
    q8 = (qf / qsc[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    qb = qf.to(torch.bfloat16)
    del qf
    w = torch.softmax(torch.randn((T, H), generator=g, device=dev), dim=1)
    pairs = sum(lq * q0 + lq * (lq + 1) // 2 for q0, lq in VARLEN_SPEC)
    out = {"what": f"one call over {B} sequences' chunks (q_start, rows) = {VARLEN_SPEC}: T={T} query rows, "
                   f"H={H} D={D} k={K}, against a paged fp8 cache of {sum(lens)} keys in scattered 64-token pages",
           "pairs": pairs}
    for name, qq, qs, peak in (("fp8", q8, qsc, PEAK_FP8_TFLOPS), ("bf16", qb, None, PEAK_BF16_TFLOPS)):
        nws = dsa._lib.load().indexer_prefill_chunk_paged_workspace_bytes(B, T, max(lens), dsa.dtype_code(qq))
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)

        def vstep():
            dsa.prefill_chunk_varlen(qq, qs, w, cu, q_start, kc, ksc, table, K, max(lens), workspace=ws)

        tm = time_calls(torch, vstep, max(args.steps, 10), args.warmup)
        ms = tm["mean_ms"]
        tf = 2.0 * H * D * pairs / (ms * 1e-3) / 1e12
        log(f"prefill varlen chunks, {name} queries: {ms:.3f} ms ({pairs / (ms * 1e-3):.4g} pairs/s, {tf:.0f} TFLOP/s)")
        out[f"{name}_queries"] = {"ms_per_call": ms, **stats(tm), "pairs_per_s": pairs / (ms * 1e-3), "TFLOP/s": tf,
                                  f"frac_of_{name}_peak": tf / peak}
        del ws
    return out


def probe_mfma_peaks(torch, dsa, dev):
    """Measured matrix-core rates of the MFMA shapes the kernels use (the
    probe kernels: long chains of independent MFMAs on every wave of a full
    grid; the best median over two grid sizes)."""
    out = {}
    for kind, name, flop_each, iters in ((0, "fp8_16x16x128_scaled", 65536, 1024), (1, "bf16_16x16x32", 16384, 2048),
                                         (2, "f16_16x16x32", 16384, 2048)):
        best = 0.0
        for blocks in (1024, 2048):
            tm = time_calls(torch, lambda: dsa.probe_mfma(kind, blocks, iters, dev), 5, 2, warm_seconds=0.05,
                            samples=5)
            best = max(best, blocks * 4 * iters * 8 * flop_each / (tm["median_ms"] * 1e-3) / 1e12)
        out[name] = best
    log("measured MFMA peaks (TFLOP/s): " + ", ".join(f"{k} {v:.0f}" for k, v in out.items()))
    return out


def probe_page_read(torch, dsa, dev, kc, ksc, page_ids):
    """Measured read rate of exactly the pages a decode call streams (the
    probe kernel: the scan's load layout, no arithmetic; the best median
    over three grid sizes), GB/s."""
    best = 0.0
    out = torch.empty(4096 * 256, dtype=torch.float32, device=dev)
    for blocks in (1024, 2048, 4096):
        tm = time_calls(torch, lambda: dsa.probe_page_read(kc, ksc, page_ids, blocks, out), 20, 3, warm_seconds=0.1,
                        samples=10)
        best = max(best, page_ids.numel() * 8448 / (tm["median_ms"] * 1e-3) / 1e9)
    return best


def oracle_timings(store, seconds_single):
    """The oracle as it stands, timed on the host over every row (or query)
    of the tiny, bf16 L=8192 and both decode workloads, plus single-thread
    times for the tiny workload (all rows) and a time-bounded seeded row
    sample of the bf16 one; every oracle result is checked against the GPU
    output of the timed run."""
    from oracle import indexer
    from oracle.check import check_topk_rows
    from threadpoolctl import threadpool_limits

    threads, api = blas_threads()
    res = {"threads": threads, "blas": api}

    def prefill_rows(n, rows, what):
        inp, gi, gv, K = store[n]
        t0 = time.perf_counter()
        parts = []
        for a in range(0, rows.size, 512):
            rr = rows[a:a + 512]
            parts.append((rr, indexer.prefill(inp, K, rows=rr, want_scores=True)[2][0]))
        t = time.perf_counter() - t0
        for rr, osc in parts:
            check_topk_rows(gi[rr], gv[rr], osc, rr + 1, K, where=what)
        return t

    for n in (1, 2):
        if n not in store:
            continue
        L = store[n][0]["q"].shape[1]
        t = prefill_rows(n, np.arange(L), f"oracle timing workload {n}")
        pairs = L * (L + 1) // 2
        res[f"workload_{n}"] = {"rows": L, "seconds": t, "pairs_per_s": pairs / t, "cores": threads,
                                "parity": "every row checked against the GPU output"}
        log(f"oracle workload {n}: all {L} rows in {t:.2f} s ({threads} threads)")
    with threadpool_limits(limits=1):
        if 1 in store:
            L = store[1][0]["q"].shape[1]
            t = prefill_rows(1, np.arange(L), "oracle single-thread workload 1")
            res["workload_1_single_thread"] = {"rows": L, "seconds": t, "pairs_per_s": L * (L + 1) // 2 / t,
                                               "cores": 1}
        if 2 in store:
            L = store[2][0]["q"].shape[1]
            rng = np.random.default_rng(2024)
            order = rng.permutation(L)
            done, t, pairs = 0, 0.0, 0
            while done < L and t < seconds_single:
                rr = np.sort(order[done:done + 32])
                t += prefill_rows(2, rr, "oracle single-thread workload 2")
                pairs += int((rr + 1).sum())
                done += rr.size
            res["workload_2_single_thread"] = {"rows": done, "seconds": t, "pairs_per_s": pairs / t, "cores": 1,
                                               "sample": f"{done} seeded rows (time-bounded at {seconds_single} s)"}
            log(f"oracle workload 2, one thread: {done} rows in {t:.1f} s")
    for n in (4, 5):
        if n not in store:
            continue
        d, gi, gv, K = store[n]
        ctx = d["context_lens"].astype(np.int64)
        t, scores = 0.0, []
        for b in range(ctx.size):
            t0 = time.perf_counter()
            o = indexer.decode_scores(d, b)
            indexer.select_topk(o, o.size, K)
            t += time.perf_counter() - t0
            scores.append(o)
        for b, o in enumerate(scores):
            check_topk_rows(gi[b:b + 1], gv[b:b + 1], o[None], np.array([ctx[b]]), K,
                            where=f"oracle timing workload {n} query {b}")
        nbytes = int(ctx.sum()) * 132
        res[f"workload_{n}"] = {"queries": int(ctx.size), "seconds": t, "GB/s": nbytes / t / 1e9, "cores": threads,
                                "parity": "every query checked against the GPU output"}
        log(f"oracle workload {n}: all {ctx.size} queries in {t:.2f} s ({threads} threads)")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip every oracle timing")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="skip the prefill headline (profiling aid)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the probes and every leg but the headline prefill and the decodes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device-to-device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import dsa_lightning_indexer_03_amd as dsa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    store = {}  # workload -> (inputs, GPU idx, GPU scores, k) for the oracle's checks

    result = {"metric": METRIC, "decode_only": True}
    peaks = probe_mfma_peaks(torch, dsa, dev) if not args.no_extra else {}
    inp = gpu_idx = gpu_val = None
    # ---------------- headline: fused fp8 prefill, L = 32768 ----------------
    if not args.decode_only:
        cfg = synth.CONFIGS[3]
        L, H, D, K = cfg["L"], cfg["H"], cfg["D"], cfg["topk"]
        t0 = time.perf_counter()
        inp = synth.config_inputs(3)
        log(f"generated prefill inputs in {time.perf_counter() - t0:.1f} s")
        q, k, w = up(torch, inp["q"], dev), up(torch, inp["k"], dev), up(torch, inp["w"], dev)
        qs, ks = up(torch, inp["q_scale"], dev), up(torch, inp["k_scale"], dev)
        out = {}

        def step():
            out["r"] = dsa.indexer_prefill(q, k, w, K, q_scale=qs, k_scale=ks)

        tm = time_calls(torch, step, args.steps, args.warmup)
        ms_avg, wall = tm["mean_ms"], tm["wall_s"]
        pairs = L * (L + 1) // 2
        flops = 2.0 * H * D * pairs
        achieved = flops / (ms_avg * 1e-3) / 1e12
        log(f"prefill: {ms_avg:.3f} ms/step (median {tm['median_ms']:.3f}, min {tm['min_ms']:.3f}), "
            f"{pairs / (ms_avg * 1e-3):.4g} pairs/s, {achieved:.1f} TFLOP/s")

        gpu_idx = out["r"][0].cpu().numpy()[0]
        gpu_val = out["r"][1].cpu().numpy()[0]

        mp = peaks.get("fp8_16x16x128_scaled")
        result = {
            "metric": METRIC,
            "value": pairs / (ms_avg * 1e-3),
            "unit": "pairs/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_avg,
            "ms_per_step_median": tm["median_ms"],
            "ms_per_step_min": tm["min_ms"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp8_e4m3",
            "data": "synthetic",
            "config": {"workload": "prefill B=1 L=32768 H=64 D=128 k=2048, fp8 e4m3 q/k with per-row fp32 scales, "
                                   "causal s<=t, fused score+top-k (no [L,L] in HBM)",
                       "batch": 1, "L": L, "H": H, "D": D, "topk": K, "seed": 3},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_FP8_TFLOPS, "traffic": measured_traffic("prefill"),
                         "measured_peak": mp, "frac_of_measured_peak": None if not mp else achieved / mp,
                         "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                         "kernel": "prefill_ws_fp8_kernel<4, false, false, false>",
                         "timing": "whole indexer_prefill call (key pre-pass + the kernel), events on the "
                                   "library's stream",
                         "work": f"2*H*D flop per causal pair x {pairs} pairs = {flops:.4g} flop per launch"},
            "wall_s_timed": wall,
        }
        if peaks:
            result["measured_peaks"] = {"mfma_TFLOP/s": peaks}
        # chunked prefill against the paged cache: the sequence's last 4096 tokens
        # (positions 28672 .. 32767) over its 32768 keys in a permuted page pool
        if not args.no_extra:
            q0c, Lqc = L - 4096, 4096
            n_pages = L // 64
            gperm = torch.Generator(device=dev)
            gperm.manual_seed(6)
            perm = torch.randperm(n_pages, generator=gperm, device=dev).to(torch.int32)
            kc = torch.empty((n_pages, 64, D), dtype=torch.uint8, device=dev)
            ksc = torch.empty((n_pages, 64), dtype=torch.float32, device=dev)
            kc[perm.long()] = k.view(n_pages, 64, D)
            ksc[perm.long()] = ks.view(n_pages, 64)
            tab = perm.view(1, n_pages)
            qc, qsc, wc = q[:, q0c:].contiguous(), qs[:, q0c:].contiguous(), w[:, q0c:].contiguous()

            def cstep():
                dsa.prefill_chunk_paged(qc, qsc, wc, kc, ksc, tab, q0c, K)

            tc = time_calls(torch, cstep, max(args.steps, 10), args.warmup)
            cms = tc["mean_ms"]
            cpairs = Lqc * q0c + Lqc * (Lqc + 1) // 2
            ctf = 2.0 * H * D * cpairs / (cms * 1e-3) / 1e12
            log(f"prefill chunk: {cms:.3f} ms for {Lqc} queries at {q0c}.. ({ctf:.0f} TFLOP/s)")
            result["prefill_chunk_paged"] = {
                "what": f"B=1 chunk of {Lqc} fp8 queries at positions {q0c}..{L - 1} of the L={L} workload, "
                        f"scored against its {L} keys in a permuted paged fp8 cache, k={K}",
                "ms_per_call": cms, **stats(tc), "pairs": cpairs, "pairs_per_s": cpairs / (cms * 1e-3),
                "TFLOP/s": ctf, "frac_of_fp8_peak": ctf / PEAK_FP8_TFLOPS,
            }
            del kc, ksc, tab, qc, qsc, wc, perm
        del q, k, w, qs, ks, out
        torch.cuda.empty_cache()
        if not args.no_extra:
            result["prefill_chunk_varlen"] = bench_varlen(torch, dsa, dev, args)
            torch.cuda.empty_cache()

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---------------- decode: contiguous and scattered pages ----------------
    if not args.no_decode:
        dec = {}
        for n in (4, 5):
            c = synth.CONFIGS[n]
            t0 = time.perf_counter()
            d = synth.config_inputs(n)
            log(f"generated decode workload {n} in {time.perf_counter() - t0:.1f} s")
            args_d = [up(torch, d[x], dev) for x in ("q", "w", "k_cache", "k_scale", "block_table", "context_lens")]
            mcl = d["max_pages_per_seq"] * d["page_size"]
            ws = torch.empty(dsa.decode_workspace_bytes(c["B"], mcl, c["H"], c["D"], c["topk"]),
                             dtype=torch.uint8, device=dev)
            dout = {}

            def dstep():
                dout["r"] = dsa.indexer_decode_paged(*args_d, c["topk"], max_context_len=mcl, workspace=ws)

            # a decode call is ~0.2 ms: time at least 200 of them, after 0.5 s of warmup calls
            td = time_calls(torch, dstep, max(args.steps, 200), args.warmup, warm_seconds=0.5)
            dms = td["mean_ms"]
            ctx = d["context_lens"].astype(np.int64)
            nbytes = int(ctx.sum()) * (c["D"] + 4)
            gbs = nbytes / (dms * 1e-3) / 1e9
            rec = {
                "what": ("64 queries x 131072-token contiguous fp8 cache" if n == 4 else
                         "128 queries, ctx ~ U[4096,131072], 64-token pages scattered by a seeded permutation"),
                "kcache_bytes": nbytes, "us_per_call": float(dms * 1e3), **stats(td, 1e3, "us"), "GB/s": gbs,
                "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "topk": c["topk"],
                "scan_traffic_bytes": measured_traffic(f"decode_scan_w{n}"),
            }
            if not args.no_extra:
                # the same pages, read by the probe: the measured bandwidth ceiling of this call
                pids = np.concatenate([d["block_table"][b, :(int(cx) + 63) // 64] for b, cx in enumerate(ctx)])
                peak = probe_page_read(torch, dsa, dev, args_d[2], args_d[3],
                                       torch.from_numpy(pids.astype(np.int32)).to(dev))
                rec.update({"measured_page_read_GB/s": peak, "frac_of_measured_peak": gbs / peak})
            log(f"decode {n}: {dms * 1e3:.1f} us/call (median {td['median_ms'] * 1e3:.1f}, min "
                f"{td['min_ms'] * 1e3:.1f}), {gbs:.0f} GB/s"
                + (f"; page-read probe {rec['measured_page_read_GB/s']:.0f} GB/s" if not args.no_extra else ""))
            dec[f"workload_{n}"] = rec
            store[n] = (d, dout["r"][0].cpu().numpy(), dout["r"][1].cpu().numpy(), c["topk"])
            del args_d, ws, dout
            torch.cuda.empty_cache()
        result["decode"] = dec

    # ---------------- K-cache write path: the decode cache written in one bulk append ----------------
    if not args.no_extra:
        B4, ctx4 = 64, 131072
        T = B4 * ctx4
        g = torch.Generator(device=dev)
        g.manual_seed(4)
        kn = torch.randn((T, 128), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ar = torch.arange(T, device=dev, dtype=torch.int32)
        seq_ids, positions = ar // ctx4, ar % ctx4
        table = torch.arange(B4 * (ctx4 // 64), device=dev, dtype=torch.int32).reshape(B4, ctx4 // 64)
        cache = torch.empty((B4 * ctx4 // 64, 64, 128), dtype=torch.uint8, device=dev)
        scale = torch.empty((B4 * ctx4 // 64, 64), dtype=torch.float32, device=dev)

        def kstep():
            dsa.kcache_append(kn, seq_ids, positions, table, cache, scale)

        tk = time_calls(torch, kstep, max(args.steps, 20), args.warmup)
        kms = tk["mean_ms"]
        nb = T * (256 + 8 + 132)
        # a decode step's append: one new key per sequence (position 7 of each)
        k64 = kn[:B4].contiguous()
        s64 = torch.arange(B4, device=dev, dtype=torch.int32)
        p64 = torch.full((B4,), 7, device=dev, dtype=torch.int32)

        def kstep1():
            dsa.kcache_append(k64, s64, p64, table, cache, scale)

        tk1 = time_calls(torch, kstep1, 200, args.warmup, warm_seconds=0.2)
        log(f"kcache append: {kms:.3f} ms for {T} keys ({nb / (kms * 1e-3) / 1e9:.0f} GB/s); "
            f"64 keys {tk1['mean_ms'] * 1e3:.1f} us")
        result["kcache_append"] = {
            "what": "64 sequences x 131072 bf16 keys quantised to fp8 e4m3 (absmax/448 scale) and written "
                    "through the block table: the decode workload's whole cache in one call",
            "keys": T, "bytes_per_call": nb, "ms_per_call": kms, **stats(tk), "GB/s": nb / (kms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nb / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "work": "per key 256 B bf16 + 8 B sequence/position read, 128 B codes + 4 B scale written",
            "us_per_call_64_keys": tk1["mean_ms"] * 1e3, "us_per_call_64_keys_median": tk1["median_ms"] * 1e3,
        }
        del kn, ar, seq_ids, positions, table, cache, scale, k64, s64, p64
        torch.cuda.empty_cache()

    # ---------------- the selection's consumer: gather of the selected latent rows ----------------
    if not args.no_extra:
        B4, K4, ctx4, row = 64, 2048, 131072, 1024
        n_pages = B4 * ctx4 // 64
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        cache = torch.randint(0, 256, (n_pages, 64, row), generator=g, device=dev, dtype=torch.uint8)
        table = torch.arange(n_pages, device=dev, dtype=torch.int32).reshape(B4, ctx4 // 64)
        gidx = torch.randint(0, ctx4, (B4, K4), generator=g, device=dev, dtype=torch.int32)

        def gstep():
            dsa.topk_gather(cache, table, gidx)

        tg = time_calls(torch, gstep, max(args.steps, 200), args.warmup, warm_seconds=0.2)
        gms = tg["mean_ms"]
        nb = B4 * K4 * (2 * row + 8)
        log(f"topk gather: {gms * 1e3:.1f} us for {B4}x{K4} rows of {row} B ({nb / (gms * 1e-3) / 1e9:.0f} GB/s)")
        result["topk_gather"] = {
            "what": "64 queries x 2048 selected positions gathered from paged 131072-token latent caches "
                    "(1024-byte rows = 512 bf16), random positions",
            "rows": B4 * K4, "bytes_per_call": nb, "us_per_call": gms * 1e3, **stats(tg, 1e3, "us"),
            "GB/s": nb / (gms * 1e-3) / 1e9, "frac_of_hbm_peak": nb / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "work": "per row 1024 B read + 1024 B written + 4 B index + 4 B page id",
        }
        del cache, table, gidx
        torch.cuda.empty_cache()
        # Index Share: one selection gathered from S layers' latent caches in one launch
        S, B6, K6, ctx6 = 8, 16, 2048, 32768
        n6 = B6 * ctx6 // 64
        caches = [torch.randint(0, 256, (n6, 64, row), generator=g, device=dev, dtype=torch.uint8) for _ in range(S)]
        table = torch.randperm(n6, generator=g, device=dev).to(torch.int32).reshape(B6, ctx6 // 64)
        gidx = torch.randint(0, ctx6, (B6, K6), generator=g, device=dev, dtype=torch.int32)
        outs = [torch.empty((B6, K6, row), dtype=torch.uint8, device=dev) for _ in range(S)]

        def lstep():
            dsa.topk_gather_layers(caches, table, gidx, outs=outs)

        tl = time_calls(torch, lstep, max(args.steps, 100), args.warmup, warm_seconds=0.2)
        nb = S * B6 * K6 * 2 * row + B6 * K6 * 8
        log(f"topk gather, {S} layers: {tl['mean_ms'] * 1e3:.1f} us ({nb / (tl['mean_ms'] * 1e-3) / 1e9:.0f} GB/s)")
        result["topk_gather_layers"] = {
            "what": f"Index Share: {B6} queries x {K6} selected positions gathered from {S} layers' paged latent "
                    f"caches ({ctx6}-token contexts, 1024-byte rows, scattered pages) in one launch",
            "bytes_per_call": nb, "us_per_call": tl["mean_ms"] * 1e3, **stats(tl, 1e3, "us"),
            "GB/s": nb / (tl["mean_ms"] * 1e-3) / 1e9,
            "frac_of_hbm_peak": nb / (tl["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "work": "per selected row and layer 1024 B read + 1024 B written; 8 B of index and page id per row",
        }
        del caches, outs, table, gidx
        torch.cuda.empty_cache()

    # ---------------- the other prefill workloads: bf16 L=8192, tiny fp32 ----------------
    if not args.decode_only and not args.no_extra:
        extra = {}
        for n in (2, 1):
            c = synth.CONFIGS[n]
            inp_n = synth.config_inputs(n)
            qn, kn, wn = up(torch, inp_n["q"], dev), up(torch, inp_n["k"], dev), up(torch, inp_n["w"], dev)
            want = n == 1  # the tiny workload also returns its full score matrix
            pout = {}

            def pstep():
                pout["r"] = dsa.indexer_prefill(qn, kn, wn, c["topk"], want_scores=want)

            tp = time_calls(torch, pstep, max(args.steps, 10), args.warmup)
            ms_n = tp["mean_ms"]
            pairs_n = c["L"] * (c["L"] + 1) // 2
            rec = {"what": f"prefill B=1 L={c['L']} H={c['H']} D={c['D']} k={c['topk']} {c['dtype']}"
                           + (" (full score matrix returned)" if want else ", fused"),
                   "ms_per_call": ms_n, **stats(tp), "pairs_per_s": pairs_n / (ms_n * 1e-3)}
            if n == 2:
                tf = 2.0 * c["H"] * c["D"] * pairs_n / (ms_n * 1e-3) / 1e12
                rec.update({"TFLOP/s": tf, "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS})
                if peaks:
                    rec["frac_of_measured_bf16_peak"] = tf / peaks["bf16_16x16x32"]
            extra[f"workload_{n}"] = rec
            store[n] = (inp_n, pout["r"][0].cpu().numpy()[0], pout["r"][1].cpu().numpy()[0], c["topk"])
            log(f"prefill workload {n}: {ms_n:.3f} ms/call")
            del qn, kn, wn, pout
            torch.cuda.empty_cache()
        result["prefill_other"] = extra

        # Long sequences: the fp8 kernel at its largest L (17-bit positions) and
        # the unstaged bf16 kernel (L > 65536).  Inputs are drawn on the device
        # with the recipe of the L=32768 and L=8192 workloads (no needles) and
        # timed only; their parity is tested at L = 65536 / 66000.
        longl = {}
        g = torch.Generator(device=dev)
        for name, L_l, fp8 in (("fp8_L131072", 131072, True), ("bf16_L98304", 98304, False)):
            g.manual_seed(7)
            H_l, D_l, K_l = 64, 128, 2048
            w_l = torch.softmax(torch.randn(1, L_l, H_l, generator=g, device=dev, dtype=torch.float64), -1).float()
            if fp8:
                def quant(x):
                    sc = x.abs().amax(-1, keepdim=True) / 448.0
                    sc = torch.where(sc > 0, sc, torch.ones_like(sc))
                    return (x / sc).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8), sc.squeeze(-1)
                q_l, qs_l = quant(torch.randn(1, L_l, H_l, D_l, generator=g, device=dev))
                k_l, ks_l = quant(torch.randn(1, L_l, D_l, generator=g, device=dev))
            else:
                q_l = torch.randn(1, L_l, H_l, D_l, generator=g, device=dev).to(torch.bfloat16)
                k_l = torch.randn(1, L_l, D_l, generator=g, device=dev).to(torch.bfloat16)
                qs_l = ks_l = None
            torch.cuda.synchronize()

            def lstep_p():
                dsa.indexer_prefill(q_l, k_l, w_l, K_l, q_scale=qs_l, k_scale=ks_l)

            tl = time_calls(torch, lstep_p, 3, 1, warm_seconds=0.0, samples=5)
            pairs_l = L_l * (L_l + 1) // 2
            tf = 2.0 * H_l * D_l * pairs_l / (tl["mean_ms"] * 1e-3) / 1e12
            peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
            longl[name] = {"what": f"prefill B=1 L={L_l} H={H_l} D={D_l} k={K_l} {'fp8 e4m3' if fp8 else 'bf16'}, "
                                   f"device-drawn N(0,1) inputs, softmax head weights",
                           "ms_per_call": tl["mean_ms"], **stats(tl), "pairs_per_s": pairs_l / (tl["mean_ms"] * 1e-3),
                           "TFLOP/s": tf, f"frac_of_{'fp8' if fp8 else 'bf16'}_peak": tf / peak}
            log(f"prefill {name}: {tl['mean_ms']:.2f} ms/call, {tf:.0f} TFLOP/s")
            del q_l, k_l, w_l, qs_l, ks_l
            torch.cuda.empty_cache()
        result["prefill_long"] = longl

    # ---------------- CPU oracle baselines (rank 0, N=1) ----------------
    if not args.no_cpu_baseline and not args.decode_only:
        result["cpu_baseline"] = cpu_baseline_prefill(inp, K, gpu_idx, gpu_val, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.4g} pairs/s")
    if not args.no_cpu_baseline:
        result["oracle_timing"] = oracle_timings(store, seconds_single=10.0)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
