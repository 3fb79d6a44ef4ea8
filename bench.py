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
# reads for a 1 GiB device-to-device copy (FETCH_SIZE 524315 KiB, WRITE_SIZE
# 1048576.0 KiB).  A record applies only while the kernel's sources hash to
# the value it was taken at; otherwise traffic is reported as null.
COPY_FETCH_FACTOR = 1048576.0 / 524315.0
COPY_WRITE_FACTOR = 1048576.0 / 1048576.0
_DECODE_SRC = ["csrc/decode_paged.hip", "csrc/select_row.h", "csrc/common.h", "csrc/kernels.h", "build.py"]
_DECODE_SHA = "b994f09d85857f186da6a3bd56b247d4d0d47b75fa896b0ba2941317424e6e58"
COUNTERS = {
    "prefill": {"sources": ["csrc/prefill_ws.hip", "csrc/rowbuf.h", "csrc/varlen.h", "csrc/common.h", "csrc/kernels.h",
                            "build.py"],
                "sha256": "b707bbef38e6ef71cebf89feeeadd0125e737fd97eb5c1b8f5b2b114bb4971b2",
                "fetch_kib": 255166.1, "write_kib": 524385.8},
    # main scan of one decode call (the sample kernel reads about 1/60 of it)
    "decode_scan_w4": {"sources": _DECODE_SRC, "sha256": _DECODE_SHA, "fetch_kib": 546194.8, "write_kib": 2381.3},
    "decode_scan_w5": {"sources": _DECODE_SRC, "sha256": _DECODE_SHA, "fetch_kib": 556899.7, "write_kib": 4107.8},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def up(torch, a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def time_calls(torch, fn, steps, warmup, warm_seconds=0.2):
    """Runs fn at least `warmup` times and for at least `warm_seconds` (after
    the host-side input generation the GPU needs a few hundred calls of a
    short op to reach its steady clocks), then exactly `steps` times back to
    back between one pair of HIP events on the current stream (the stream
    the library launches on), with a device synchronisation on both sides.
    Returns the mean milliseconds per call and the wall time of the timed
    region."""
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
    return a.elapsed_time(b) / steps, wall


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

        ms, _ = time_calls(torch, vstep, max(args.steps, 10), args.warmup)
        tf = 2.0 * H * D * pairs / (ms * 1e-3) / 1e12
        log(f"prefill varlen chunks, {name} queries: {ms:.3f} ms ({pairs / (ms * 1e-3):.4g} pairs/s, {tf:.0f} TFLOP/s)")
        out[f"{name}_queries"] = {"ms_per_call": ms, "pairs_per_s": pairs / (ms * 1e-3), "TFLOP/s": tf,
                                  f"frac_of_{name}_peak": tf / peak}
        del ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="skip the prefill headline (profiling aid)")
    ap.add_argument("--no-extra", action="store_true", help="skip the bf16 L=8192 and tiny prefill timings")
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

    result = {"metric": METRIC, "decode_only": True}
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

        ms_avg, wall = time_calls(torch, step, args.steps, args.warmup)
        pairs = L * (L + 1) // 2
        flops = 2.0 * H * D * pairs
        achieved = flops / (ms_avg * 1e-3) / 1e12
        log(f"prefill: {ms_avg:.3f} ms/step, {pairs / (ms_avg * 1e-3):.4g} pairs/s, "
            f"{achieved:.1f} TFLOP/s")

        gpu_idx = out["r"][0].cpu().numpy()[0]
        gpu_val = out["r"][1].cpu().numpy()[0]

        result = {
            "metric": METRIC,
            "value": pairs / (ms_avg * 1e-3),
            "unit": "pairs/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms_avg,
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
                         "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                         "kernel": "prefill_ws_fp8_kernel<4, false, false, false>",
                         "work": f"2*H*D flop per causal pair x {pairs} pairs = {flops:.4g} flop per launch"},
            "wall_s_timed": wall,
        }
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

            cms, _ = time_calls(torch, cstep, max(args.steps, 10), args.warmup)
            cpairs = Lqc * q0c + Lqc * (Lqc + 1) // 2
            ctf = 2.0 * H * D * cpairs / (cms * 1e-3) / 1e12
            log(f"prefill chunk: {cms:.3f} ms for {Lqc} queries at {q0c}.. ({ctf:.0f} TFLOP/s)")
            result["prefill_chunk_paged"] = {
                "what": f"B=1 chunk of {Lqc} fp8 queries at positions {q0c}..{L - 1} of the L={L} workload, "
                        f"scored against its {L} keys in a permuted paged fp8 cache, k={K}",
                "ms_per_call": cms, "pairs": cpairs, "pairs_per_s": cpairs / (cms * 1e-3), "TFLOP/s": ctf,
                "frac_of_fp8_peak": ctf / PEAK_FP8_TFLOPS,
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

            def dstep():
                dsa.indexer_decode_paged(*args_d, c["topk"], max_context_len=mcl, workspace=ws)

            # a decode call is ~0.2 ms: time at least 200 of them, after 0.5 s of warmup calls
            dms, _ = time_calls(torch, dstep, max(args.steps, 200), args.warmup, warm_seconds=0.5)
            nbytes = int(d["context_lens"].astype(np.int64).sum()) * (c["D"] + 4)
            gbs = nbytes / (dms * 1e-3) / 1e9
            log(f"decode {n}: {dms * 1e3:.1f} us/call, {gbs:.0f} GB/s")
            dec[f"workload_{n}"] = {
                "what": ("64 queries x 131072-token contiguous fp8 cache" if n == 4 else
                         "128 queries, ctx ~ U[4096,131072], 64-token pages scattered by a seeded permutation"),
                "kcache_bytes": nbytes, "us_per_call": float(dms * 1e3), "GB/s": gbs,
                "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "topk": c["topk"],
                "scan_traffic_bytes": measured_traffic(f"decode_scan_w{n}"),
            }
            del args_d, ws
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

        kms, _ = time_calls(torch, kstep, max(args.steps, 20), args.warmup)
        nb = T * (256 + 8 + 132)
        # a decode step's append: one new key per sequence (position 7 of each)
        k64 = kn[:B4].contiguous()
        s64 = torch.arange(B4, device=dev, dtype=torch.int32)
        p64 = torch.full((B4,), 7, device=dev, dtype=torch.int32)

        def kstep1():
            dsa.kcache_append(k64, s64, p64, table, cache, scale)

        k1ms, _ = time_calls(torch, kstep1, 200, args.warmup, warm_seconds=0.2)
        log(f"kcache append: {kms:.3f} ms for {T} keys ({nb / (kms * 1e-3) / 1e9:.0f} GB/s); "
            f"64 keys {k1ms * 1e3:.1f} us")
        result["kcache_append"] = {
            "what": "64 sequences x 131072 bf16 keys quantised to fp8 e4m3 (absmax/448 scale) and written "
                    "through the block table: the decode workload's whole cache in one call",
            "keys": T, "bytes_per_call": nb, "ms_per_call": kms, "GB/s": nb / (kms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nb / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "work": "per key 256 B bf16 + 8 B sequence/position read, 128 B codes + 4 B scale written",
            "us_per_call_64_keys": k1ms * 1e3,
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

        gms, _ = time_calls(torch, gstep, max(args.steps, 200), args.warmup, warm_seconds=0.2)
        nb = B4 * K4 * (2 * row + 8)
        log(f"topk gather: {gms * 1e3:.1f} us for {B4}x{K4} rows of {row} B ({nb / (gms * 1e-3) / 1e9:.0f} GB/s)")
        result["topk_gather"] = {
            "what": "64 queries x 2048 selected positions gathered from paged 131072-token latent caches "
                    "(1024-byte rows = 512 bf16), random positions",
            "rows": B4 * K4, "bytes_per_call": nb, "us_per_call": gms * 1e3, "GB/s": nb / (gms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nb / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "work": "per row 1024 B read + 1024 B written + 4 B index + 4 B page id",
        }
        del cache, table, gidx
        torch.cuda.empty_cache()

    # ---------------- the other prefill workloads: bf16 L=8192, tiny fp32 ----------------
    if not args.decode_only and not args.no_extra:
        extra = {}
        for n in (2, 1):
            c = synth.CONFIGS[n]
            inp_n = synth.config_inputs(n)
            qn, kn, wn = up(torch, inp_n["q"], dev), up(torch, inp_n["k"], dev), up(torch, inp_n["w"], dev)
            want = n == 1  # the tiny workload also returns its full score matrix

            def pstep():
                dsa.indexer_prefill(qn, kn, wn, c["topk"], want_scores=want)

            ms_n, _ = time_calls(torch, pstep, max(args.steps, 10), args.warmup)
            pairs_n = c["L"] * (c["L"] + 1) // 2
            rec = {"what": f"prefill B=1 L={c['L']} H={c['H']} D={c['D']} k={c['topk']} {c['dtype']}"
                           + (" (full score matrix returned)" if want else ", fused"),
                   "ms_per_call": ms_n, "pairs_per_s": pairs_n / (ms_n * 1e-3)}
            if n == 2:
                tf = 2.0 * c["H"] * c["D"] * pairs_n / (ms_n * 1e-3) / 1e12
                rec.update({"TFLOP/s": tf, "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS})
            extra[f"workload_{n}"] = rec
            log(f"prefill workload {n}: {ms_n:.3f} ms/call")
            del qn, kn, wn
            torch.cuda.empty_cache()
        result["prefill_other"] = extra

    # ---------------- CPU oracle baseline (rank 0, N=1) ----------------
    if not args.no_cpu_baseline and not args.decode_only:
        result["cpu_baseline"] = cpu_baseline_prefill(inp, K, gpu_idx, gpu_val, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.4g} pairs/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
