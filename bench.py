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
  roofline      the dominant kernel's algorithmic bytes per launch over its
                average duration (HIP events carried by the kernel's own
                dispatches, over a second pass of the same steps), against
                MI355X peak;
  kernels       average duration of every kernel of the step;
  cold          the same step with the compressed-key cache rebuilt from
                scratch (every block compressed inside the call);
  dense         the dense causal GQA decode comparator at the decode shape;
  prefill       the 1M-context, last-16,384-token-chunk prefill step (batch 1),
                with the indexer's MFMA fraction and the attention's;
  configs       the other three workloads (tiny 4K, 128K decode, 256K prefill
                chunk), steady-state forward, each against its roofline;
  sweep         the decode step (batch 4 x 4) and the last-16K-chunk prefill
                at contexts of 8K, 32K, 128K, 256K and 1M tokens;
  streaming     a whole 1M-token prompt prefilled in 64 chunks of 16,384
                tokens (each compressing only its own micro-blocks), then
                decode steps of 4 tokens appended to the caches;
  ceilings      the part's measured memory ceilings under the path's access
                patterns (cold 128 MiB streaming read, random 256 B / 1 KiB /
                4 KiB gathers over an 8 GiB K/V cache);
  cpu_baseline  the CPU oracle on bounded samples of the decode step and the
                prefill step, per stage, on the host cores.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
       python bench.py --ceilings          (only the memory ceilings)
       python bench.py --copy-calibration  (counter calibration copy)
"""
from __future__ import annotations

import argparse
import json
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


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--cold-steps", type=int, default=3)
    ap.add_argument("--dense-prefill-steps", type=int, default=2)
    ap.add_argument("--page-size", type=int, default=16,
                    help="tokens per page of the paged K/V legs")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged K/V legs")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparator")
    ap.add_argument("--no-configs", action="store_true", help="skip the other three workloads")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the memory ceilings")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 8K..1M context-length sweep of the decode step and prefill chunk")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip the whole-prompt streaming run (1M prompt in 16K chunks, then decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of each oracle sample (decode, prefill)")
    ap.add_argument("--topk-engine", choices=("auto", "table", "stream", "scan"), default="auto",
                    help="force the top-k engine of every leg (default: the library's choice)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the memory ceilings and print them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer three times and exit (the reference "
                         "kernel for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args(argv)


# --------------------------------------------------------------------- helpers

def to_dev(a, torch, np):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def base_name(name: str) -> str:
    """A recorded kernel name without its template arguments."""
    return name.split("<", 1)[0]


def kernel_stats(records, n_steps):
    """Per-kernel average duration (us) and launches per step, keyed by the
    kernel's base name (template instantiations of one kernel are one entry;
    their recorded names are listed under "variants")."""
    agg = {}
    for name, ms in records:
        s = agg.setdefault(base_name(name), [0.0, 0, set()])
        s[0] += ms
        s[1] += 1
        s[2].add(name)
    out = {}
    for name, (tot, cnt, names) in agg.items():
        out[name] = {"avg_us": 1000.0 * tot / cnt, "launches_per_step": cnt / n_steps}
        if names != {name}:
            out[name]["variants"] = sorted(names)
    return out


def timed_steps(step, n, flush, Q, torch):
    """n steps, each after an untimed flush, with HIP events on the stream
    around each step; then the same n steps again with per-kernel HIP events
    carried by each kernel's own dispatch packet (the library's profiling
    hook).  The two passes are separate because the dispatch-carried events
    lengthen the gap between dependent kernels by several microseconds, so
    the step times come from the first pass and the kernel durations from the
    second.  Returns (step times in ms, kernel stats, wall seconds of the
    first pass)."""
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
    nk = min(n, 60)
    timer = Q.KernelTimer(max_launches=16 * nk + 16)
    torch.cuda.synchronize()
    with timer:
        for _ in range(nk):
            flush()
            step()
    return step_ms, kernel_stats(timer.records(), nk), wall


def measured_traffic(kernel, workload=None):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch,
    each scaled by what the same counter reads for a 1 GiB copy).  None when
    there is no such record, when it was taken on another workload than
    `workload` (if given), or when the kernel's source changed since it was
    taken (the record keeps the source file's SHA-256)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "traffic.json")) as f:
            rec = json.load(f).get(kernel)
        if rec is None or (workload is not None and rec.get("workload") != workload):
            return None
        with open(os.path.join(here, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return (rec["fetch_kib_per_launch"] * rec["fetch_scale"]
                + rec["write_kib_per_launch"] * rec["write_scale"]) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def roofline_of(kstats, algo, workload=None):
    """Roofline record of the dominant kernel (largest time per step) of a
    leg.  algo: base kernel name -> (bound, work per step, unit of work,
    description); "hbm" work is bytes, "mfma" work is flop.  `traffic` comes
    from the counters taken on `workload` only."""
    if not kstats:
        return None
    name, st = max(kstats.items(), key=lambda kv: kv[1]["avg_us"] * kv[1]["launches_per_step"])
    if name not in algo:
        return {"kernel": name, "bound": None, "achieved": None, "peak": None,
                "frac": None, "traffic": None, "note": "no algorithmic work recorded"}
    bound, per_step, what = algo[name]
    per_launch = per_step / max(st["launches_per_step"], 1.0)
    sec = st["avg_us"] * 1e-6
    if bound == "hbm":
        ach, peak, unit = per_launch / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = per_launch / sec / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(name, workload)
    rec = {"bound": bound, "kernel": name, "achieved": ach, "peak": peak, "unit": unit,
           "frac": ach / peak, "traffic": traffic,
           "algorithmic_" + ("bytes" if bound == "hbm" else "flop"): per_launch,
           "work_is": what}
    if traffic is not None:
        # the counted HBM bytes per launch over this run's duration
        rec["traffic_gbs"] = traffic / sec / 1e9
        rec["traffic_frac_of_hbm_peak"] = traffic / sec / 1e9 / HBM_PEAK_GBS
    return rec


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]


def decode_bytes(w, sel_h, nsel_h, np):
    """Algorithmic HBM bytes of one decode step: the compressed keys of every
    candidate block (each sequence's 4 queries share the scan), the union per
    sequence of the gathered K and V rows (4 KV heads x 256 B each), Q, O and
    the indexer queries."""
    B, Nq = w.batch, w.n_query
    lens_h = w.lens.astype(np.int64)
    kcmp = int(sum(((int(l) - 1) // 4) * 128 for l in lens_h))
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
    attn = union_tokens * w.kv_heads * 128 * 2 * 2 + 2 * q_bytes
    qidx = B * Nq * 4 * 64 * 2
    return kcmp, attn, qidx


def decode_algo(kcmp, attn, qidx, B):
    return {
        "score_table_kernel": ("hbm", kcmp + qidx,
                               "compressed keys of every candidate block (128 B each) + "
                               "indexer queries"),
        "scan_filter_kernel": ("hbm", kcmp + qidx,
                               "compressed keys of every candidate block (128 B each) + "
                               "indexer queries"),
        "score_stream_kernel": ("hbm", kcmp + qidx,
                                "compressed keys of every candidate block + indexer queries"),
        "sparse_attend_kernel": ("hbm", attn,
                                 "union over each sequence's 4 queries of the gathered K and V "
                                 "rows (4 KV heads x 256 B each) + Q + O"),
        "block_attend_kernel": ("hbm", attn,
                                "union over each sequence's 4 queries of the gathered K and V "
                                "rows (4 KV heads x 256 B each) + Q + O"),
        "compress_kernel": ("hbm", B * (512 + 128), "one new block per sequence: 4 keys in, 1 out"),
    }


def prefill_work(w, np):
    t = np.arange(int(w.lens[0]) - w.n_query, int(w.lens[0]), dtype=np.int64)
    idx_flops = float(np.sum(512.0 * (t // 4)))
    n_tok = 4 * np.minimum(512, t // 4) + (t % 4) + 1
    attn_flops = float(np.sum(n_tok) * w.q_heads * 128 * 4)
    return idx_flops, attn_flops


ENGINE_FLAGS = {"auto": 0, "table": 1, "stream": 2, "scan": 4}


class Workspace:
    """Device tensors of one workload, with the compressed-key cache holding
    every block before the call's queries (the steady state)."""

    flags = 0  # top-k engine flag of every workspace (bench.py --topk-engine)

    def __init__(self, w, Q, torch, np):
        B, L, Nq = w.batch, w.max_len, w.n_query
        self.w = w
        self.shp = Q.shape(B, L, Nq, w.q_heads, w.kv_heads, 0.0, Workspace.flags)
        self.dev = {n: to_dev(getattr(w, n), torch, np) for n in ("q_idx", "k_idx", "q", "k", "v")}
        self.lens = to_dev(w.lens, torch, np)
        prev = to_dev((w.lens - Nq).astype(np.int32), torch, np)
        self.first = to_dev(((w.lens - Nq) // 4).astype(np.int32), torch, np)
        self.k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
        Q.compress_keys(self.shp, self.dev["k_idx"], prev, self.k_cmp)
        self.out = torch.empty((B, Nq, w.q_heads, 128), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((B, Nq, w.q_heads), dtype=torch.float32, device="cuda")
        self.sel = torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda")
        self.n_sel = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
        self.ws = Q.workspace(self.shp, Q.OP_FORWARD)
        self.Q = Q

    def step(self, cold=False):
        d = self.dev
        self.Q.forward(self.shp, d["q_idx"], d["k_idx"], self.k_cmp, d["q"], d["k"], d["v"],
                       self.lens, first_block=None if cold else self.first, out=self.out,
                       lse=self.lse, sel=self.sel, n_sel=self.n_sel, ws=self.ws)


# --------------------------------------------------------------------- legs

def decode_leg(args, Q, W, torch, np, flush):
    log("[bench] decode-1m-b4x4: generating inputs")
    w = W.make(4)
    ws = Workspace(w, Q, torch, np)
    log(f"[bench] decode: {args.warmup} warmup + {args.steps} timed steps")
    for _ in range(args.warmup):
        flush()
        ws.step()
    torch.cuda.synchronize()
    step_ms, kstats, wall = timed_steps(ws.step, args.steps, flush, Q, torch)
    sel_h = ws.sel.cpu().numpy()
    nsel_h = ws.n_sel.cpu().numpy()
    kcmp, attn, qidx = decode_bytes(w, sel_h, nsel_h, np)
    # cold: the whole compressed-key cache rebuilt inside the call
    cold = None
    if args.cold_steps > 0:
        log(f"[bench] decode cold: {args.cold_steps} steps with a full compressed-key rebuild")
        cold_ms, cold_k, _ = timed_steps(lambda: ws.step(cold=True), args.cold_steps, flush, Q,
                                         torch)
        ws.step()  # leave the steady-state cache and selection behind
        torch.cuda.synchronize()
        cold = {"ms_per_step": sum(cold_ms) / len(cold_ms), "steps": len(cold_ms),
                "kernels": cold_k,
                "note": "every block of the 1M-token contexts compressed inside the call "
                        "(k_idx 512 MiB read, k_cmp 128 MiB written), then the step"}
    # selection quality: the share of the dense attention mass (pooled per
    # micro-block, the indexer's training target) that the selection keeps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    teacher = Q.block_teacher(ws.shp, ws.dev["q"], ws.dev["k"], ws.dev["v"], ws.lens)
    ev[1].record()
    recall = Q.teacher_recall(ws.shp, ws.lens, teacher, ws.sel, ws.n_sel).cpu().numpy()
    quality = {"recall_mean": float(recall.mean()), "recall_min": float(recall.min()),
               "teacher_ms": ev[0].elapsed_time(ev[1]),
               "note": "dense attention mass (averaged over heads) on the selected blocks and "
                       "the own block; random synthetic keys, so the mass is spread thinly"}
    del teacher
    torch.cuda.empty_cache()
    # backward passes on the same batch: the sparse attention's gradients
    # (dk/dv added into zeroed float32 caches) and the indexer scores'
    # gradient for a dense dL/ds
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    d_out = torch.randn(ws.out.shape, generator=g, device="cuda").to(torch.bfloat16)
    d_s = torch.randn((w.batch, w.n_query, w.max_len // 4), generator=g, device="cuda")
    dk = torch.zeros(ws.dev["k"].shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    dq_idx = torch.zeros(ws.dev["q_idx"].shape, dtype=torch.float32, device="cuda")
    dk_cmp = torch.zeros(ws.k_cmp.shape, dtype=torch.float32, device="cuda")
    def run_backward():
        Q.sparse_attend_backward(ws.shp, ws.dev["q"], ws.dev["k"], ws.dev["v"], ws.lens, ws.sel,
                                 ws.n_sel, ws.out, ws.lse, d_out, dk=dk, dv=dv)
        Q.index_scores_backward(ws.shp, ws.dev["q_idx"], ws.k_cmp, ws.lens, d_s, dq_idx=dq_idx,
                                dk_cmp=dk_cmp)

    run_backward()  # first launches (code object loading) untimed
    torch.cuda.synchronize()
    # kernel durations from the HIP events each dispatch carries (the
    # attention backward is a fill of dq and the gradient kernel)
    reps = 3
    timer = Q.KernelTimer(max_launches=4 * reps)
    with timer:
        for _ in range(reps):
            run_backward()
    t_att = t_idx = 0.0
    for name, ms in timer.records():
        if name.startswith("index_scores_bwd_kernel"):
            t_idx += ms
        else:
            t_att += ms
    # the indexer backward's algorithmic HBM bytes: each candidate block's
    # compressed key (128 B) and its Nq gradient entries read, its float32
    # dk_cmp row read and written (2 x 256 B), dq_idx read and written once
    nblk = sum((int(n) - 1) // 4 for n in w.lens)
    idx_bytes = nblk * (128 + 4 * w.n_query + 512) + 2 * w.batch * w.n_query * 4 * 64 * 4
    # the attention backward's algorithmic bytes: per (query, KV head) and
    # token of its list, the K and V pieces read (2 x 256 B bf16) and the
    # float32 dk and dv pieces read and written by the adds (2 x 2 x 512 B);
    # q, dO, O and dq are small beside them
    ntok = sum(4 * int(nsel_h[b, i]) + (int(w.lens[b]) - w.n_query + i) % 4 + 1
               for b in range(w.batch) for i in range(w.n_query))
    att_bytes = ntok * w.kv_heads * (2 * 256 + 4 * 512)
    backward = {"attend_backward_us": 1000 * t_att / reps,
                "attend_backward_gbs": att_bytes / (t_att / reps * 1e-3) / 1e9,
                "index_scores_backward_us": 1000 * t_idx / reps,
                "index_scores_backward_gbs": idx_bytes / (t_idx / reps * 1e-3) / 1e9,
                "note": f"kernel time per call, mean of {reps} calls each on the decode batch "
                        "after one untimed call, caches warm (the attention backward: its dq fill "
                        "and gradient kernels); the gradients accumulate into the same buffers; "
                        "dk/dv added atomically, dk_cmp read, added and written back"}
    del d_out, d_s, dk, dv, dq_idx, dk_cmp
    torch.cuda.empty_cache()
    return dict(w=w, ws=ws, step_ms=step_ms, kstats=kstats, wall=wall, sel=sel_h, n_sel=nsel_h,
                quality=quality, backward=backward,
                algo=decode_algo(kcmp, attn, qidx, w.batch), kcmp_bytes=kcmp, attn_bytes=attn,
                qidx_bytes=qidx, cold=cold)


def dense_leg(args, Q, torch, flush, d):
    ws_ = d["ws"]
    shp, dev, lens = ws_.shp, ws_.dev, ws_.lens
    wsp = Q.workspace(shp, Q.OP_DENSE_DECODE)
    out = torch.empty_like(ws_.out)

    def step():
        Q.dense_gqa_decode(shp, dev["q"], dev["k"], dev["v"], lens, out=out, ws=wsp,
                           want_lse=False)

    flush()
    step()
    torch.cuda.synchronize()
    step_ms, kstats, _ = timed_steps(step, args.dense_steps, flush, Q, torch)
    w = d["w"]
    kv_bytes = int(sum(int(l) for l in w.lens)) * w.kv_heads * 128 * 2 * 2
    ms = sum(step_ms) / len(step_ms)
    return {"ms_per_step": ms, "kernels": kstats,
            "hbm_gbs": kv_bytes / (ms * 1e-3) / 1e9, "kv_bytes": kv_bytes,
            "roofline": roofline_of(kstats, {"dense_decode_kernel": ("hbm", kv_bytes,
                                                                     "every K and V row of the "
                                                                     "context")}, w.name)}


def paged_pools(Q, torch, k, v, lens, page, seed):
    """Page pools [n_pages][page][Hkv][128] holding the contiguous caches k, v
    under a seeded random page order, and their page table: the layout a
    paged serving cache leaves after many sequences have come and gone."""
    B, L, Hkv, D = k.shape
    max_pages = (L + page - 1) // page
    need = [(int(n) + page - 1) // page for n in lens]
    n_pages = max(1, sum(need))
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(n_pages, generator=g).to(torch.int64)
    table = torch.zeros((B, max_pages), dtype=torch.int32)
    k_pool = torch.empty((n_pages, page, Hkv, D), dtype=k.dtype, device=k.device)
    v_pool = torch.empty_like(k_pool)
    off = 0
    for b in range(B):
        n, full = need[b], int(lens[b]) // page
        pid = ids[off:off + n]
        off += n
        table[b, :n] = pid.to(torch.int32)
        if full:
            idx = pid[:full].to(k.device)
            k_pool[idx] = k[b, :full * page].view(full, page, Hkv, D)
            v_pool[idx] = v[b, :full * page].view(full, page, Hkv, D)
        if n > full:  # the last, partial page
            rest = int(lens[b]) - full * page
            k_pool[int(pid[full]), :rest] = k[b, full * page:full * page + rest]
            v_pool[int(pid[full]), :rest] = v[b, full * page:full * page + rest]
    torch.cuda.synchronize()
    return k_pool, v_pool, Q.PagedKV(table.to(k.device), page, n_pages)


def paged_decode_leg(args, Q, torch, flush, d, qsa_ms, dense_ms):
    """The decode batch with K/V in page pools: QSA forward and the dense
    decode comparator, both through the page table (the pages' comparison
    is against paged GQA)."""
    ws_ = d["ws"]
    w = d["w"]
    shp, dev, lens = ws_.shp, ws_.dev, ws_.lens
    page = args.page_size
    k_pool, v_pool, pg = paged_pools(Q, torch, dev["k"], dev["v"], w.lens, page, 77)

    def qsa():
        Q.forward_paged(shp, dev["q_idx"], dev["k_idx"], ws_.k_cmp, dev["q"], k_pool, v_pool, pg,
                        lens, first_block=ws_.first, out=ws_.out, lse=ws_.lse, sel=ws_.sel,
                        n_sel=ws_.n_sel, ws=ws_.ws)

    for _ in range(3):
        flush()
        qsa()
    torch.cuda.synchronize()
    q_ms, q_k, _ = timed_steps(qsa, min(args.steps, 50), flush, Q, torch)
    res = {"page_size": page, "n_pages": pg.n_pages,
           "qsa": {"ms_per_step": sum(q_ms) / len(q_ms), "steps": len(q_ms), "kernels": q_k}}
    res["qsa"]["vs_contiguous"] = res["qsa"]["ms_per_step"] / qsa_ms
    if dense_ms is not None:
        wsp = Q.workspace(shp, Q.OP_DENSE_DECODE)
        out = torch.empty_like(ws_.out)

        def dense():
            Q.dense_gqa_decode_paged(shp, dev["q"], k_pool, v_pool, pg, lens, out=out, ws=wsp,
                                     want_lse=False)

        flush()
        dense()
        torch.cuda.synchronize()
        dn_ms, dn_k, _ = timed_steps(dense, args.dense_steps, flush, Q, torch)
        ms = sum(dn_ms) / len(dn_ms)
        kv_bytes = int(sum(int(l) for l in w.lens)) * w.kv_heads * 128 * 2 * 2
        res["dense"] = {"ms_per_step": ms, "kernels": dn_k, "hbm_gbs": kv_bytes / (ms * 1e-3) / 1e9,
                        "vs_contiguous": ms / dense_ms}
        res["qsa_speedup"] = ms / res["qsa"]["ms_per_step"]
    del k_pool, v_pool, pg
    torch.cuda.empty_cache()
    return res


def dense_prefill_flops(w, np):
    """Dense causal attention of the chunk: (t + 1) tokens per query and head,
    QK^T and PV at 2 x 128 flop each per (head, token)."""
    tot = 0
    for b in range(w.batch):
        t = int(w.lens[b]) - w.n_query + np.arange(w.n_query, dtype=np.int64)
        tot += int((t + 1).sum())
    return tot * w.q_heads * 128 * 4


def dense_prefill_leg(args, Q, torch, np, flush, ws, w, qsa_ms):
    """Dense causal GQA over the prefill chunk (the comparator of the pages'
    prefill speedup), contiguous and paged, and the QSA forward over the same
    page pools."""
    shp, dev, lens = ws.shp, ws.dev, ws.lens
    out = torch.empty_like(ws.out)
    flops = dense_prefill_flops(w, np)
    n = args.dense_prefill_steps
    res = {"flops": flops}

    def record(step):
        flush()
        step()
        torch.cuda.synchronize()
        ms_, k_, _ = timed_steps(step, n, flush, Q, torch)
        ms = sum(ms_) / len(ms_)
        rec = {"ms_per_step": ms, "steps": len(ms_), "kernels": k_}
        st = k_.get("dense_prefill_kernel")
        if st:
            ach = flops / (st["avg_us"] * 1e-6) / 1e12
            rec["mfma"] = {"kernel": "dense_prefill_kernel", "achieved": ach,
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / MFMA_BF16_PEAK_TFLOPS}
        return rec

    log(f"[bench] {w.name}: dense prefill comparator, contiguous")
    res["contiguous"] = record(lambda: Q.dense_gqa_prefill(shp, dev["q"], dev["k"], dev["v"], lens,
                                                           out=out, want_lse=False))
    res["qsa_speedup"] = res["contiguous"]["ms_per_step"] / qsa_ms
    if not args.no_paged:
        log(f"[bench] {w.name}: paged ({args.page_size}-token pages)")
        k_pool, v_pool, pg = paged_pools(Q, torch, dev["k"], dev["v"], w.lens, args.page_size, 78)
        res["page_size"] = args.page_size
        res["paged"] = record(lambda: Q.dense_gqa_prefill(shp, dev["q"], k_pool, v_pool, lens,
                                                          paged=pg, out=out, want_lse=False))

        def qsa():
            Q.forward_paged(shp, dev["q_idx"], dev["k_idx"], ws.k_cmp, dev["q"], k_pool, v_pool,
                            pg, lens, first_block=ws.first, out=ws.out, lse=ws.lse, sel=ws.sel,
                            n_sel=ws.n_sel, ws=ws.ws)

        flush()
        qsa()
        torch.cuda.synchronize()
        q_ms, q_k, _ = timed_steps(qsa, args.prefill_steps, flush, Q, torch)
        res["qsa_paged"] = {"ms_per_step": sum(q_ms) / len(q_ms), "steps": len(q_ms),
                            "kernels": q_k}
        res["qsa_paged_speedup"] = res["paged"]["ms_per_step"] / res["qsa_paged"]["ms_per_step"]
        del k_pool, v_pool, pg
        torch.cuda.empty_cache()
    return res


def prefill_record(w, step_ms, kstats, np):
    idx_flops, attn_flops = prefill_work(w, np)
    ms = sum(step_ms) / len(step_ms)
    res = {"workload": w.name, "value": w.batch * w.n_query / (ms * 1e-3), "unit": "q-tok/s",
           "ms_per_step": ms, "steps": len(step_ms), "kernels": kstats,
           "indexer_flops": idx_flops, "attention_flops": attn_flops}
    sk = kstats.get("score_stream_kernel")
    if sk:
        ach = idx_flops / (sk["avg_us"] * 1e-6) / 1e12
        res["indexer_mfma"] = {"kernel": "score_stream_kernel", "achieved": ach,
                               "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                               "traffic": measured_traffic("score_stream_kernel", w.name)}
    ak = kstats.get("sparse_attend_kernel")
    if ak:
        ach = attn_flops / (ak["avg_us"] * 1e-6) / 1e12
        kv_unique = int(w.lens[0]) * w.kv_heads * 128 * 2 * 2
        res["attention_mfma"] = {"kernel": "sparse_attend_kernel", "achieved": ach,
                                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                                 "unique_kv_bytes": kv_unique,
                                 "unique_kv_hbm_frac": kv_unique / (ak["avg_us"] * 1e-6) / 1e9
                                 / HBM_PEAK_GBS,
                                 "traffic": measured_traffic("sparse_attend_kernel", w.name)}
        tr = res["attention_mfma"]["traffic"]
        if tr is not None:
            # the gathered rows the counters saw leave the L2, over this run's duration
            res["attention_mfma"]["traffic_frac_of_hbm_peak"] = (
                tr / (ak["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS)
    return res


def prefill_gather_ceiling(Q, torch, flush, ws, w, ak, reps=3):
    """The prefill attention against the rate at which this part gathers the
    same bytes: every query's selected micro-blocks and its own block, 4 KiB
    of K and 4 KiB of V each (the 4 consecutive token rows of all KV heads),
    read by the plain gather probe in the selection's own order: the bound
    for any kernel that fetches each query's rows once.  Also how often a
    block is chosen (the reuse a block-major kernel could exploit)."""
    B, Nq = w.batch, w.n_query
    sel = ws.sel.to(torch.int64)
    pos = ws.lens.to(torch.int64).view(B, 1) - Nq + torch.arange(Nq, device="cuda").view(1, Nq)
    own = (pos // 4).view(B, Nq, 1)
    seq_blocks = w.max_len // 4
    blk = torch.cat([sel, own], dim=2)
    blk = torch.where(blk < 0, own, blk)  # (rows with fewer than 512 blocks re-read their own)
    idx = (blk + torch.arange(B, device="cuda").view(B, 1, 1) * seq_blocks).reshape(-1).contiguous()
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    best = None
    for wgs in (2048, 8192):
        def probe():
            Q.ceil_gather(ws.dev["k"], idx, 4096, wgs, sink)
            Q.ceil_gather(ws.dev["v"], idx, 4096, wgs, sink)
        probe()
        totals = []
        for _ in range(reps):
            flush()
            timer = Q.KernelTimer(max_launches=4)
            torch.cuda.synchronize()
            with timer:
                probe()
            totals.append(sum(ms for _, ms in timer.records()) * 1000.0)
        us = min(totals)
        if best is None or us < best[0]:
            best = (us, wgs)
    nbytes = idx.numel() * 4096 * 2
    uniq = int(torch.unique(idx).numel())
    return {"probe_us": best[0], "workgroups": best[1], "bytes": nbytes,
            "unique_blocks": uniq, "mean_queries_per_block": idx.numel() / max(uniq, 1),
            "probe_gbs": nbytes / (best[0] * 1e-6) / 1e9,
            "attention_us": ak["avg_us"], "attention_over_probe": ak["avg_us"] / best[0],
            "note": "qsa_ceil_gather over the step's own selection (K then V, 4 KiB blocks); "
                    "the attention also computes, and fetches whole blocks only where the "
                    "selection has them"}


def prefill_leg(args, Q, W, torch, np, flush, cfg=3, steps=None):
    w = W.make(cfg)
    log(f"[bench] {w.name}: inputs ready")
    ws = Workspace(w, Q, torch, np)
    flush()
    ws.step()
    torch.cuda.synchronize()
    n = steps or args.prefill_steps
    log(f"[bench] {w.name}: {n} timed steps")
    step_ms, kstats, _ = timed_steps(ws.step, n, flush, Q, torch)
    res = prefill_record(w, step_ms, kstats, np)
    # needle survival: the share of each query's planted micro-blocks (indexer
    # keys x4) that its selection keeps
    if w.needle_starts and w.needle_starts[0]:
        sel_h, nsel_h = ws.sel.cpu().numpy()[0], ws.n_sel.cpu().numpy()[0]
        blocks = np.array(sorted(j for s in w.needle_starts[0] for j in range(s // 4, s // 4 + 16)))
        hit = np.zeros(w.n_query)
        for i in range(w.n_query):
            hit[i] = np.isin(blocks, sel_h[i, :nsel_h[i]]).mean()
        res["needle_survival"] = {"mean": float(hit.mean()), "min": float(hit.min()),
                                  "spans": len(w.needle_starts[0]), "blocks": int(blocks.size)}
    ak = res["kernels"].get("sparse_attend_kernel")
    if ak:
        res["attention_gather_ceiling"] = prefill_gather_ceiling(Q, torch, flush, ws, w, ak)
    if not args.no_dense:
        res["dense_comparator"] = dense_prefill_leg(args, Q, torch, np, flush, ws, w,
                                                    res["ms_per_step"])
    del ws
    torch.cuda.empty_cache()
    return res, w


def other_configs(Q, W, torch, np, flush):
    """The tiny 4K, 128K decode and 256K prefill-chunk workloads, steady-state
    forward (the compressed-key cache holds the blocks before the call's
    queries), each with its roofline."""
    res = {}
    for cfg in (0, 1, 2):
        w = W.make(cfg)
        ws = Workspace(w, Q, torch, np)
        for _ in range(3):
            flush()
            ws.step()
        torch.cuda.synchronize()
        n = 50 if w.n_query <= 64 else 5
        step_ms, kstats, _ = timed_steps(ws.step, n, flush, Q, torch)
        ms = float(np.median(step_ms))
        if cfg == 2:
            rec = prefill_record(w, step_ms, kstats, np)
            rec["ms_per_step"] = ms
            rec["value"] = w.batch * w.n_query / (ms * 1e-3)
        else:
            sel_h, nsel_h = ws.sel.cpu().numpy(), ws.n_sel.cpu().numpy()
            kcmp, attn, qidx = decode_bytes(w, sel_h, nsel_h, np)
            step_bytes = kcmp + attn + qidx
            rec = {"workload": w.name, "value": w.batch * w.n_query / (ms * 1e-3),
                   "unit": "q-tok/s", "ms_per_step": ms, "steps": n, "kernels": kstats,
                   "step_hbm": {"algorithmic_bytes": step_bytes,
                                "achieved_gbs": step_bytes / (ms * 1e-3) / 1e9,
                                "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                   "roofline": roofline_of(kstats, decode_algo(kcmp, attn, qidx, w.batch),
                                           w.name)}
            if cfg == 0:
                rec["note"] = ("64 queries over a 4,096-token context: too small to load the "
                               "part, so launch and round-trip latencies dominate")
        res[w.name] = rec
        log(f"[bench] {w.name}: {ms * 1e3:.1f} us per step")
        del ws
        torch.cuda.empty_cache()
    return res


def device_inputs(torch, B, L, Nq, Hq, Hkv, seed, positions=None):
    """Seeded synthetic inputs generated on the device (for the sweep and the
    streaming run, whose sizes would take the host generator minutes):
    indexer queries and keys uniform integers in [-8, 8], core Q/K/V
    standard normal, all rounded to bf16 (the integers exactly).  positions:
    query rows to generate (default Nq)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    n = Nq if positions is None else positions
    bf = torch.bfloat16

    def ints(*shape):
        return torch.randint(-8, 9, shape, generator=g, device="cuda", dtype=torch.int32).to(bf)

    def normal(*shape):
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(bf)

    return {"q_idx": ints(B, n, 4, 64), "k_idx": ints(B, L, 64), "q": normal(B, n, Hq, 128),
            "k": normal(B, L, Hkv, 128), "v": normal(B, L, Hkv, 128)}


def sweep(Q, torch, np, flush):
    """The decode step (batch 4 x 4, lens L .. L-3) and the prefill of the last
    16,384 positions (batch 1; the whole prompt when it is shorter) at each
    context length, steady state (the compressed-key cache holds the blocks
    before the call's queries), 32/4 heads, device-generated inputs."""
    res = {}
    for L in (8192, 32768, 131072, 262144, 1048576):
        rec = {}
        for kind in ("decode", "prefill"):
            if kind == "decode":
                B, Nq = 4, 4
                lens_h = np.array([L, L - 1, L - 2, L - 3], np.int32)
            else:
                B, Nq = 1, min(16384, L)
                lens_h = np.array([L], np.int32)
            d = device_inputs(torch, B, L, Nq, 32, 4, seed=L + (0 if kind == "decode" else 1))
            shp = Q.shape(B, L, Nq, 32, 4, 0.0, Workspace.flags)
            lens = torch.from_numpy(lens_h).cuda()
            prev = torch.from_numpy(lens_h - Nq).cuda()
            first = torch.from_numpy((lens_h - Nq) // 4).cuda()
            k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
            if (lens_h - Nq).max() > 0:
                Q.compress_keys(shp, d["k_idx"], prev, k_cmp)
            out = torch.empty((B, Nq, 32, 128), dtype=torch.bfloat16, device="cuda")
            wsp = Q.workspace(shp, Q.OP_FORWARD)

            def step():
                Q.forward(shp, d["q_idx"], d["k_idx"], k_cmp, d["q"], d["k"], d["v"], lens,
                          first_block=first, out=out, ws=wsp, want_lse=False)

            for _ in range(3):
                flush()
                step()
            n = 30 if kind == "decode" else 3
            step_ms, kst, _ = timed_steps(step, n, flush, Q, torch)
            ms = float(np.median(step_ms))
            r = {"ms_per_step": ms, "value": B * Nq / (ms * 1e-3), "unit": "q-tok/s",
                 "kernels": {k: round(v["avg_us"], 2) for k, v in kst.items()}}
            if kind == "decode":
                kcmp_bytes = int(sum(((int(l) - 1) // 4) * 128 for l in lens_h))
                r["kcmp_scan_gbs"] = None
                sk = kst.get("score_table_kernel") or kst.get("scan_filter_kernel")
                if sk:
                    r["kcmp_scan_gbs"] = kcmp_bytes / (sk["avg_us"] * 1e-6) / 1e9
            else:
                t = np.arange(L - Nq, L, dtype=np.int64)
                idx_flops = float(np.sum(512.0 * (t // 4)))
                sk = kst.get("score_stream_kernel")
                if sk:
                    r["indexer_mfma_frac"] = idx_flops / (sk["avg_us"] * 1e-6) / 1e12 \
                        / MFMA_BF16_PEAK_TFLOPS
            rec[kind] = r
            del d, k_cmp, out, wsp
            torch.cuda.empty_cache()
        res[str(L)] = rec
        log(f"[bench] sweep {L}: decode {rec['decode']['ms_per_step'] * 1e3:.1f} us, "
            f"prefill {rec['prefill']['ms_per_step']:.2f} ms")
    return res


def streaming(Q, torch, np, prompt=1 << 20, chunk=16384, steps=16, m=4):
    """A whole prompt of `prompt` tokens prefilled in chunks through
    qsa_forward (each call compressing only its chunk's micro-blocks), then
    `steps` decode steps of m tokens appended to the caches; batch 1, 32/4
    heads, device-generated inputs.  Wall time of the whole prefill and the
    decode steps by HIP events."""
    from learned_sparse_attention_qsa_amd import streaming as S

    total = prompt + steps * m
    cap = (total + 3) // 4 * 4
    d = device_inputs(torch, 1, total, 0, 32, 4, seed=7777, positions=total)
    seq = S.Sequence(cap, 32, 4, flags=Workspace.flags)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    S.prefill(seq, d["q_idx"][0, :prompt], d["k_idx"][0, :prompt], d["q"][0, :prompt],
              d["k"][0, :prompt], d["v"][0, :prompt], chunk)
    ev[1].record()
    for s in range(steps):
        lo = prompt + s * m
        S.decode_step(seq, d["q_idx"][0, lo:lo + m], d["k_idx"][0, lo:lo + m],
                      d["q"][0, lo:lo + m], d["k"][0, lo:lo + m], d["v"][0, lo:lo + m])
    ev[2].record()
    torch.cuda.synchronize()
    pre_ms = ev[0].elapsed_time(ev[1])
    dec_ms = ev[1].elapsed_time(ev[2])
    n_chunks = (prompt + chunk - 1) // chunk
    del d, seq
    torch.cuda.empty_cache()
    return {"prompt_tokens": prompt, "chunk": chunk, "chunks": n_chunks,
            "prefill_ms": pre_ms, "prefill_q_tok_per_s": prompt / (pre_ms * 1e-3),
            "prefill_ms_per_chunk": pre_ms / n_chunks, "decode_steps": steps,
            "decode_tokens_per_step": m, "decode_ms_per_step": dec_ms / steps,
            "decode_q_tok_per_s": steps * m / (dec_ms * 1e-3),
            "note": ("caches not flushed between calls (the run is one continuous stream of "
                     "work); includes the per-chunk appends of K/V and indexer keys")}


def ceilings(Q, torch, flush, reps=10):
    """Memory ceilings under the path's access patterns, each kernel timed by
    the HIP events its own dispatch carries, after an untimed flush."""
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203)

    def run(fn):
        fn()  # one untimed pass: first touch of the buffer's pages
        timer = Q.KernelTimer(max_launches=reps + 2)
        torch.cuda.synchronize()
        with timer:
            for _ in range(reps):
                flush()
                fn()
        recs = timer.records()
        us = sorted(1000.0 * ms for _, ms in recs)
        return us[len(us) // 2]

    out = {}
    scan_bytes = 128 << 20  # one decode step's compressed keys: 4 x 262,143 x 128 B ~ 128 MiB
    buf = torch.empty(scan_bytes, dtype=torch.uint8, device="cuda")
    for wgs in (256, 1024):
        us = run(lambda: Q.ceil_stream_read(buf, wgs, sink))
        out[f"stream_read_128MiB_wg{wgs}"] = {"us": us, "gbs": scan_bytes / (us * 1e-6) / 1e9}
    del buf
    # the decode K/V cache: 4 sequences x 1M tokens x 4 KV heads x 128 dims,
    # K and V: 8 GiB; the gathers read what 16 query rows of 2,048 selected
    # tokens would (random micro-blocks of each row's sequence)
    kv = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    rows, blocks = 16, 512
    seq_tokens = 1 << 20
    blk = torch.randint(0, seq_tokens // 4, (rows, blocks), generator=gen, device="cuda")
    seq = (torch.arange(rows, device="cuda") // 4).view(rows, 1)
    kv_half = 4 << 30
    for row_bytes, name in ((4096, "block_4KiB"), (1024, "token_row_1KiB"), (256, "head_row_256B")):
        # byte offset of K (and V) pieces of every selected block of every row
        base = (seq * (1 << 30) + blk * 4096)  # K half; V half = + 4 GiB
        base = torch.cat([base.reshape(-1), base.reshape(-1) + kv_half])
        per_blk = 4096 // row_bytes
        if row_bytes == 256:
            # one KV head's 256-byte piece of each of the block's 4 tokens
            idx = (base.view(-1, 1) + torch.arange(4, device="cuda").view(1, 4) * 1024) // 256
        else:
            idx = (base.view(-1, 1) + torch.arange(per_blk, device="cuda").view(1, per_blk)
                   * row_bytes) // row_bytes
        idx = idx.reshape(-1).contiguous()
        nbytes = idx.numel() * row_bytes
        us = run(lambda: Q.ceil_gather(kv, idx, row_bytes, 2048, sink))
        out[f"gather_{name}"] = {"us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}
    del kv
    torch.cuda.empty_cache()
    # LDS atomic adds: cycles per wavefront instruction on one SIMD (2,048
    # workgroups of four wavefronts, 256 adds each, over 1,024 SIMDs at 2.4 GHz)
    wgs, iters = 2048, 256
    lsink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    for f32 in (False, True):
        for share in (1, 4, 64):
            us = run(lambda: Q.ceil_lds_atomic(f32, share, wgs, iters, lsink))
            cyc = us * 1e-6 * 2.4e9 / (wgs * 4 * iters / 1024)
            out[f"lds_atomic_{'f32' if f32 else 'u32'}_share{share}"] = {
                "us": us, "cycles_per_wave_instruction": cyc}
    out["note"] = ("kernel durations from dispatch-carried HIP events, median of "
                   f"{reps}, each after a 1 GiB flush; head_row_256B reads one KV head's "
                   "piece of each token (a quarter of the bytes of the others); lds_atomic: "
                   "share = lanes of a wavefront on one LDS address")
    return out


# --------------------------------------------------------------------- CPU oracle

def host_cores():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return aff, max(1, min(16, aff)), model


def cpu_baseline(args, d, w3, np):
    """The oracle as it stands, on bounded samples of the decode step and the
    prefill step, timed per stage on the host cores."""
    import threadpoolctl

    import oracle as O

    aff, threads, model = host_cores()
    log(f"[bench] cpu baseline: oracle on {threads} threads ({aff} CPUs in affinity)")
    w = d["w"]
    Nq = w.n_query
    stages = ("compress", "score", "select", "expand", "attend")
    res = {}
    with threadpoolctl.threadpool_limits(threads):
        # ---- decode: every query of the batch, repeated until the budget is spent
        caches = {}
        for b in range(w.batch):  # the cache of the previous step, as the GPU had it (untimed)
            prev = int(w.lens[b]) - Nq
            caches[b] = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[b], prev))
        tm = dict.fromkeys(stages, 0.0)
        done, reps, match = 0, 0, True
        t0 = time.perf_counter()
        while True:
            for b in range(w.batch):
                length = int(w.lens[b])
                prev = length - Nq
                c0 = time.perf_counter()
                new = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[b], length,
                                                         first_block=prev // 4))
                kc = np.concatenate([caches[b][: prev // 4], new])
                tm["compress"] += time.perf_counter() - c0
                for i in range(Nq):
                    t = prev + i
                    c0 = time.perf_counter()
                    s = O.block_scores(O.bf16_bits_to_f64(w.q_idx[b, i]), kc[: t // 4])
                    c1 = time.perf_counter()
                    sel = O.select_blocks(s)
                    c2 = time.perf_counter()
                    tok = O.expand_tokens(sel, t)
                    c3 = time.perf_counter()
                    O.attend(O.bf16_bits_to_f64(w.q[b, i]), O.bf16_bits_to_f64(w.k[b, tok]),
                             O.bf16_bits_to_f64(w.v[b, tok]), w.scale)
                    c4 = time.perf_counter()
                    tm["score"] += c1 - c0
                    tm["select"] += c2 - c1
                    tm["expand"] += c3 - c2
                    tm["attend"] += c4 - c3
                    done += 1
                    if reps == 0:
                        g = d["sel"][b, i, : d["n_sel"][b, i]]
                        match = match and np.array_equal(g, sel)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res.update({"value": done / el, "unit": "q-tok/s", "cores": threads, "kind": "oracle",
                    "sample": (f"{reps} pass(es) over the 16 decode queries of the 1M-context "
                               "batch: incremental compression of the new block, scoring of "
                               "every earlier block, top-512, expansion and float64 attention; "
                               "compressed-key cache of the earlier tokens prepared untimed"),
                    "seconds": el, "selections_match_gpu": bool(match),
                    "stage_seconds": tm, "affinity_cpus": aff, "cpu_model": model})
        # ---- prefill: queries of the 1M chunk in order until the budget is spent
        if w3 is not None:
            length = int(w3.lens[0])
            Nq3 = w3.n_query
            prev = length - Nq3
            kc_prev = O.bf16_bits_to_f64(O.compress_keys(w3.k_idx[0], prev))  # untimed
            tm3 = dict.fromkeys(stages, 0.0)
            t0 = time.perf_counter()
            new = O.bf16_bits_to_f64(O.compress_keys(w3.k_idx[0], length,
                                                     first_block=prev // 4))
            kc = np.concatenate([kc_prev[: prev // 4], new])
            tm3["compress"] = time.perf_counter() - t0
            done = 0
            while done < Nq3:
                t = prev + done
                c0 = time.perf_counter()
                s = O.block_scores(O.bf16_bits_to_f64(w3.q_idx[0, done]), kc[: t // 4])
                c1 = time.perf_counter()
                sel = O.select_blocks(s)
                c2 = time.perf_counter()
                tok = O.expand_tokens(sel, t)
                c3 = time.perf_counter()
                O.attend(O.bf16_bits_to_f64(w3.q[0, done]), O.bf16_bits_to_f64(w3.k[0, tok]),
                         O.bf16_bits_to_f64(w3.v[0, tok]), w3.scale)
                c4 = time.perf_counter()
                tm3["score"] += c1 - c0
                tm3["select"] += c2 - c1
                tm3["expand"] += c3 - c2
                tm3["attend"] += c4 - c3
                done += 1
                if time.perf_counter() - t0 >= args.cpu_seconds:
                    break
            el = time.perf_counter() - t0
            # the chunk's compression is paid once per 16,384 queries: scale it
            per_query = (el - tm3["compress"]) / done + tm3["compress"] / Nq3
            res["prefill"] = {"value": 1.0 / per_query, "unit": "q-tok/s", "queries": done,
                              "seconds": el, "stage_seconds": tm3,
                              "sample": (f"the first {done} of the 16,384 queries of the "
                                         "1M-context last-chunk prefill, after compressing the "
                                         "chunk's 4,096 new blocks (its cost spread over the "
                                         "whole chunk)")}
    return res


# --------------------------------------------------------------------- main

def main(argv=None):
    args = parse(argv)
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
    Workspace.flags = ENGINE_FLAGS[args.topk_engine]
    # 1 GiB, four times the infinity cache.  The flush READS it: that evicts the
    # step's inputs from the infinity cache and the L2s and leaves only clean
    # lines behind.  (Writing it would leave ~0.25 GiB of dirty lines whose
    # write-back then competes with the next step's reads, a cost of whatever
    # wrote them, not of this layer.)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(Q, torch, flush)}), flush=True)
        return

    d = decode_leg(args, Q, W, torch, np, flush)
    step_ms = d["step_ms"]
    ms = sum(step_ms) / len(step_ms)
    w = d["w"]
    q_tok = w.batch * w.n_query
    step_bytes = d["kcmp_bytes"] + d["attn_bytes"] + d["qidx_bytes"]
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
        "roofline": roofline_of(d["kstats"], d["algo"], w.name),
        "kernels": d["kstats"],
        "cold": d["cold"],
        "selection_quality": d["quality"],
        "backward": d["backward"],
    }
    if not args.no_dense:
        log("[bench] dense comparator")
        dn = dense_leg(args, Q, torch, flush, d)
        dn["qsa_speedup"] = dn["ms_per_step"] / ms
        line["dense"] = dn
    if not args.no_paged:
        log(f"[bench] paged K/V ({args.page_size}-token pages): QSA and the dense comparator")
        line["paged"] = paged_decode_leg(args, Q, torch, flush, d, ms,
                                         None if args.no_dense else line["dense"]["ms_per_step"])
    d_light = {k: d[k] for k in ("w", "sel", "n_sel")}
    del d
    torch.cuda.empty_cache()
    w3 = None
    if not args.no_prefill:
        line["prefill"], w3 = prefill_leg(args, Q, W, torch, np, flush)
        torch.cuda.empty_cache()
    if not args.no_configs:
        line["configs"] = other_configs(Q, W, torch, np, flush)
    if not args.no_sweep:
        line["sweep"] = sweep(Q, torch, np, flush)
    if not args.no_streaming:
        log("[bench] streaming: 1M prompt in 16K chunks, then decode steps")
        line["streaming"] = streaming(Q, torch, np)
    if not args.no_ceilings:
        log("[bench] memory ceilings")
        line["ceilings"] = ceilings(Q, torch, flush)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, d_light, w3, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
