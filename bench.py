#!/usr/bin/env python3
"""Benchmark of the QSA hot path on one MI355X.

Headline (the JSON line's `value`): query tokens per second of one steady-state
QSA decode step at a 1M-token context, batch 4 x 4 query positions (1 token +
3 multi-token-prediction steps), 32 query / 4 KV heads.  A step is one
qsa_forward call: compression of the newly completed block, indexer scoring of
every earlier micro-block, top-512 selection, expansion and sparse GQA
attention.  Inputs are resident in HBM; the 256 MiB infinity cache and the L2s
are flushed (untimed, by reading a 1 GiB buffer) before every step, as the
other layers of a model would.

The same line carries
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch
                over its HIP-event-timed average duration, against MI355X peak;
  kernels       average duration of every kernel of the step (HIP events on
                the launch stream, via the library's profiling hook);
  prefill       the 1M-context, last-16,384-token-chunk prefill step (batch 1),
                with the indexer-scoring MFMA fraction;
  dense         the dense causal GQA decode comparator at the decode shape;
  cpu_baseline  the CPU oracle timed on a bounded sample of the decode step
                (with its selections checked against the GPU's).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = ("QSA query-tokens/sec at 1M ctx (16K prefill chunk; decode B=4×4) "
          "+ % HBM/MFMA peak")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparator")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--other-configs", action="store_true",
                    help="instead of the headline run: one JSON line per parity workload "
                         "(tiny 4K, 128K decode, 256K prefill chunk), steady-state forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer three times and exit (the reference "
                         "kernel for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# --------------------------------------------------------------------- helpers

def to_dev(a, torch, np):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def kernel_stats(records, n_steps):
    agg = {}
    for name, ms in records:
        s = agg.setdefault(name, [0.0, 0])
        s[0] += ms
        s[1] += 1
    out = {}
    for name, (tot, cnt) in agg.items():
        out[name] = {"avg_us": 1000.0 * tot / cnt, "launches_per_step": cnt / n_steps}
    return out


def timed_steps(step, n, flush, Q, torch):
    """n steps, flush before each (untimed), per-step HIP events; then up to
    20 more steps with the library's per-launch events (carried by each
    kernel's dispatch, so they time the kernel alone; kept out of the step
    times all the same)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        flush()
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    nk = min(n, 20)
    timer = Q.KernelTimer(max_launches=16 * nk + 16)
    with timer:
        for i in range(nk):
            flush()
            step()
    torch.cuda.synchronize()
    return step_ms, kernel_stats(timer.records(), nk), wall


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch,
    each scaled by what the same counter reads for a 1 GiB copy).  None when
    there is no such record or the kernel's source changed since it was
    taken (the record keeps the source file's SHA-256)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "traffic.json")) as f:
            rec = json.load(f).get(kernel)
        if rec is None:
            return None
        with open(os.path.join(here, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return (rec["fetch_kib_per_launch"] * rec["fetch_scale"]
                + rec["write_kib_per_launch"] * rec["write_scale"]) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]


# --------------------------------------------------------------------- legs

def decode_leg(args, Q, W, torch, np, flush):
    log("[bench] decode-1m-b4x4: generating inputs")
    w = W.make(4)
    B, L, Nq = w.batch, w.max_len, w.n_query
    shp = Q.shape(B, L, Nq, w.q_heads, w.kv_heads)
    dev = {n: to_dev(getattr(w, n), torch, np) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = to_dev(w.lens, torch, np)
    prev = to_dev((w.lens - Nq).astype(np.int32), torch, np)
    first = to_dev(((w.lens - Nq) // 4).astype(np.int32), torch, np)
    k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, dev["k_idx"], prev, k_cmp)  # cache state of the previous step
    out = torch.empty((B, Nq, w.q_heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Nq, w.q_heads), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    ws = Q.workspace(shp, Q.OP_FORWARD)

    def step():
        Q.forward(shp, dev["q_idx"], dev["k_idx"], k_cmp, dev["q"], dev["k"], dev["v"], lens,
                  first_block=first, out=out, lse=lse, sel=sel, n_sel=n_sel, ws=ws)

    log(f"[bench] decode: {args.warmup} warmup + {args.steps} timed steps")
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    step_ms, kstats, wall = timed_steps(step, args.steps, flush, Q, torch)
    sel_h = sel.cpu().numpy()
    nsel_h = n_sel.cpu().numpy()
    # algorithmic bytes per step of each kernel
    lens_h = w.lens.astype(np.int64)
    kcmp_bytes = int(sum(((int(l) - 1) // 4) * 128 for l in lens_h))
    union_tokens = 0
    for b in range(B):
        toks = set()
        for i in range(Nq):
            t = int(lens_h[b]) - Nq + i
            bt = t // 4
            for j in sel_h[b, i, :nsel_h[b, i]]:
                toks.update(range(4 * int(j), 4 * int(j) + 4))
            toks.update(range(4 * bt, t + 1))
        union_tokens += len(toks)
    q_bytes = B * Nq * w.q_heads * 128 * 2
    attn_bytes = union_tokens * w.kv_heads * 128 * 2 * 2 + 2 * q_bytes
    algo = {
        "score_table_kernel": ("hbm", kcmp_bytes + B * Nq * 4 * 64 * 2,
                               "compressed keys of every candidate block (128 B each) + indexer queries"),
        "score_stream_kernel": ("hbm", kcmp_bytes + B * Nq * 4 * 64 * 2,
                                "compressed keys of every candidate block + indexer queries"),
        "sparse_attend_kernel": ("hbm", attn_bytes,
                                 "union over each sequence's 4 queries of the gathered K and V rows "
                                 "(4 KV heads x 256 B each) + Q + O"),
        "compress_kernel": ("hbm", B * (512 + 128), "one new block per sequence: 4 keys in, 1 out"),
    }
    return dict(w=w, shp=shp, dev=dev, lens=lens, step_ms=step_ms, kstats=kstats, wall=wall,
                sel=sel_h, n_sel=nsel_h, algo=algo, kcmp_bytes=kcmp_bytes,
                attn_bytes=attn_bytes, out=out)


def dense_leg(args, Q, torch, flush, d):
    shp, dev, lens = d["shp"], d["dev"], d["lens"]
    ws = Q.workspace(shp, Q.OP_DENSE_DECODE)
    out = torch.empty_like(d["out"])

    def step():
        Q.dense_gqa_decode(shp, dev["q"], dev["k"], dev["v"], lens, out=out, ws=ws, want_lse=False)

    flush()
    step()
    torch.cuda.synchronize()
    step_ms, kstats, _ = timed_steps(step, args.dense_steps, flush, Q, torch)
    w = d["w"]
    kv_bytes = int(sum(int(l) for l in w.lens)) * w.kv_heads * 128 * 2 * 2
    ms = sum(step_ms) / len(step_ms)
    return {"ms_per_step": ms, "kernels": kstats,
            "hbm_gbs": kv_bytes / (ms * 1e-3) / 1e9, "kv_bytes": kv_bytes}


def prefill_leg(args, Q, W, torch, np, flush):
    log("[bench] prefill-1m-chunk16k: generating inputs")
    w = W.make(3)
    B, L, Nq = w.batch, w.max_len, w.n_query
    shp = Q.shape(B, L, Nq, w.q_heads, w.kv_heads)
    dev = {n: to_dev(getattr(w, n), torch, np) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = to_dev(w.lens, torch, np)
    prev = to_dev((w.lens - Nq).astype(np.int32), torch, np)
    first = to_dev(((w.lens - Nq) // 4).astype(np.int32), torch, np)
    k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, dev["k_idx"], prev, k_cmp)
    out = torch.empty((B, Nq, w.q_heads, 128), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    ws = Q.workspace(shp, Q.OP_FORWARD)

    def step():
        Q.forward(shp, dev["q_idx"], dev["k_idx"], k_cmp, dev["q"], dev["k"], dev["v"], lens,
                  first_block=first, out=out, sel=sel, n_sel=n_sel, ws=ws, want_lse=False)

    flush()
    step()
    torch.cuda.synchronize()
    log(f"[bench] prefill: {args.prefill_steps} timed steps")
    step_ms, kstats, _ = timed_steps(step, args.prefill_steps, flush, Q, torch)
    t = np.arange(int(w.lens[0]) - Nq, int(w.lens[0]), dtype=np.int64)
    idx_flops = float(np.sum(512.0 * (t // 4)))
    n_tok = 4 * np.minimum(512, t // 4) + (t % 4) + 1
    attn_flops = float(np.sum(n_tok) * w.q_heads * 128 * 4)
    ms = sum(step_ms) / len(step_ms)
    res = {"workload": w.name, "value": Nq / (ms * 1e-3), "unit": "q-tok/s", "ms_per_step": ms,
           "steps": len(step_ms), "kernels": kstats,
           "indexer_flops": idx_flops, "attention_flops": attn_flops}
    sk = kstats.get("score_stream_kernel") or kstats.get("score_table_kernel")
    if sk:
        ach = idx_flops / (sk["avg_us"] * 1e-6) / 1e12
        res["indexer_mfma"] = {"kernel": "score_stream_kernel", "achieved": ach,
                               "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": ach / MFMA_BF16_PEAK_TFLOPS}
    ak = kstats.get("sparse_attend_kernel")
    if ak:
        ach = attn_flops / (ak["avg_us"] * 1e-6) / 1e12
        res["attention_mfma"] = {"achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": ach / MFMA_BF16_PEAK_TFLOPS}
    del dev, k_cmp, out, sel, n_sel, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, d, np):
    """The oracle, untuned, on a bounded sample of the decode step."""
    import threadpoolctl

    import oracle as O

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores))
    w = d["w"]
    Nq = w.n_query
    log(f"[bench] cpu baseline: oracle decode step, {cores} BLAS threads")
    with threadpoolctl.threadpool_limits(cores):
        # compressed-key cache of the previous step, as the GPU had it (untimed)
        caches = {}
        for b in range(w.batch):
            prev = int(w.lens[b]) - Nq
            caches[b] = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[b], prev))
        done = 0
        reps = 0
        match = True
        t0 = time.perf_counter()
        while True:
            for b in range(w.batch):
                length = int(w.lens[b])
                prev = length - Nq
                new = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[b], length, first_block=prev // 4))
                kc = np.concatenate([caches[b][: prev // 4], new])
                for i in range(Nq):
                    t = prev + i
                    s = O.block_scores(O.bf16_bits_to_f64(w.q_idx[b, i]), kc[: t // 4])
                    sel = O.select_blocks(s)
                    tok = O.expand_tokens(sel, t)
                    O.attend(O.bf16_bits_to_f64(w.q[b, i]), O.bf16_bits_to_f64(w.k[b, tok]),
                             O.bf16_bits_to_f64(w.v[b, tok]), w.scale)
                    done += 1
                    if reps == 0:
                        g = d["sel"][b, i, : d["n_sel"][b, i]]
                        match = match and np.array_equal(g, sel)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el > 30:
                break
    return {"value": done / el, "unit": "q-tok/s", "cores": cores, "kind": "oracle",
            "sample": (f"{reps} pass(es) over the 16 decode queries of the 1M-context batch: "
                       "incremental compression of the new block, scoring of every earlier "
                       "block, top-512, expansion and float64 attention; compressed-key cache "
                       "prepared untimed"),
            "seconds": el, "selections_match_gpu": bool(match)}


# --------------------------------------------------------------------- main

def other_configs(Q, W, torch, np, flush):
    """Steady-state forward of the smaller workloads: the compressed-key cache
    holds the blocks before the call's queries, as in the headline legs."""
    for cfg in (0, 1, 2):
        w = W.make(cfg)
        B, L, Nq = w.batch, w.max_len, w.n_query
        shp = Q.shape(B, L, Nq, w.q_heads, w.kv_heads)
        dev = {n: to_dev(getattr(w, n), torch, np) for n in ("q_idx", "k_idx", "q", "k", "v")}
        lens = to_dev(w.lens, torch, np)
        prev = to_dev((w.lens - Nq).astype(np.int32), torch, np)
        first = to_dev(((w.lens - Nq) // 4).astype(np.int32), torch, np)
        k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
        Q.compress_keys(shp, dev["k_idx"], prev, k_cmp)
        out = torch.empty((B, Nq, w.q_heads, 128), dtype=torch.bfloat16, device="cuda")
        sel = torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda")
        n_sel = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
        ws = Q.workspace(shp, Q.OP_FORWARD)

        def step():
            Q.forward(shp, dev["q_idx"], dev["k_idx"], k_cmp, dev["q"], dev["k"], dev["v"], lens,
                      first_block=first, out=out, sel=sel, n_sel=n_sel, ws=ws, want_lse=False)

        for _ in range(3):
            flush()
            step()
        torch.cuda.synchronize()
        step_ms, kstats, _ = timed_steps(step, 50 if Nq <= 64 else 5, flush, Q, torch)
        ms = float(np.median(step_ms))
        idx_flops, kcmp_bytes = 0.0, 0
        for b in range(B):
            t = np.arange(int(w.lens[b]) - Nq, int(w.lens[b]), dtype=np.int64)
            idx_flops += float(np.sum(512.0 * (t // 4)))
            kcmp_bytes += ((int(w.lens[b]) - 1) // 4) * 128
        print(json.dumps({"workload": w.name, "value": B * Nq / (ms * 1e-3), "unit": "q-tok/s",
                          "ms_per_step": ms, "indexer_flops": idx_flops,
                          "kcmp_bytes": kcmp_bytes, "kernels": kstats}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the QSA path here has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import learned_sparse_attention_qsa_amd as Q
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copied 1 GiB three times", flush=True)
        return
    Q.load_library()
    # 1 GiB, four times the infinity cache.  The flush READS it: that evicts the
    # step's inputs from the infinity cache and the L2s and leaves only clean
    # lines behind.  (Writing it would leave ~0.25 GiB of dirty lines whose
    # write-back then competes with the next step's reads, a cost of whatever
    # wrote them, not of this layer.)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    if args.other_configs:
        other_configs(Q, W, torch, np, flush)
        return

    d = decode_leg(args, Q, W, torch, np, flush)
    step_ms = d["step_ms"]
    ms = sum(step_ms) / len(step_ms)
    w = d["w"]
    q_tok = w.batch * w.n_query
    kstats = d["kstats"]
    dom = max(kstats.items(), key=lambda kv: kv[1]["avg_us"] * kv[1]["launches_per_step"])
    dom_name, dom_stat = dom
    roof = None
    if dom_name in d["algo"]:
        bound, step_nbytes, what = d["algo"][dom_name]
        # the algorithmic bytes are per step; a step may split a kernel over launches
        nbytes = step_nbytes / max(dom_stat["launches_per_step"], 1.0)
        ach = nbytes / (dom_stat["avg_us"] * 1e-6) / 1e9
        roof = {"bound": bound, "kernel": dom_name, "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": measured_traffic(dom_name),
                "algorithmic_bytes": nbytes, "bytes_are": what}
    step_bytes = d["kcmp_bytes"] + d["attn_bytes"]
    line = {
        "metric": METRIC,
        "value": q_tok / (ms * 1e-3),
        "unit": "q-tok/s",
        "n_gpus": 1,
        "steps": len(step_ms),
        "warmup": args.warmup,
        "ms_per_step": ms,
        "p10_ms": pct(step_ms, 10),
        "p90_ms": pct(step_ms, 90),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode-1m-b4x4", "batch": w.batch, "context": int(w.max_len),
                   "lens": [int(x) for x in w.lens], "queries_per_seq": w.n_query,
                   "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": 128,
                   "indexer_heads": 4, "indexer_dim": 64, "block": 4, "topk_blocks": 512,
                   "caches_flushed_per_step": True},
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved_gbs": step_bytes / (ms * 1e-3) / 1e9,
                     "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": roof,
        "kernels": kstats,
    }
    if not args.no_dense:
        log("[bench] dense comparator")
        dn = dense_leg(args, Q, torch, flush, d)
        dn["qsa_speedup"] = dn["ms_per_step"] / ms
        line["dense"] = dn
    d_light = {k: d[k] for k in ("w", "sel", "n_sel")}
    del d
    torch.cuda.empty_cache()
    if not args.no_prefill:
        line["prefill"] = prefill_leg(args, Q, W, torch, np, flush)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, d_light, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
