"""Parity at the benchmark shapes, in the launch configuration bench.py times
(the compressed-key cache already holds every block before the call's queries
and the call compresses only the new ones):

  * the 1M-context decode: every query row, selection and output, with the
    automatic top-k engine (table) and with the scan engine;
  * the 256K last-chunk prefill: the selection of every one of the 16,384
    rows, outputs of sampled rows;
  * the 1M last-chunk prefill: the selection of every one of the 16,384
    rows, outputs of sampled rows;
  * the dense 1M comparator: one row of every sequence;
  * the backward passes on the 1M decode batch: every row's dq, dk and dv on
    every token read (zero elsewhere), the indexer gradients of all blocks;
  * paged K/V at the bench's shapes (16-token pages in a shuffled pool): the
    1M decode forward and dense decode, and the 1M-chunk dense prefill, bit
    for bit against the contiguous results; the dense prefill also against
    the oracle on sampled rows.

Selections bit for bit (the oracle's row-batched scorer and selector);
outputs to max-abs <= 2e-2 and rel-L2 <= 1e-2 against the float64 oracle."""
import os
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import check_close, dev_bf16, dev_i32, host_f64_from_bf16, paged_pools_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_bits_np(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(
        np.uint16)


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run_forward(w, flags=0):
    """qsa_forward in the steady state bench.py times: the cache holds the
    blocks of the tokens before the queries, the call compresses from the
    first block those tokens leave incomplete.  flags: the top-k engine (0:
    the automatic choice)."""
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads, flags=flags)
    prev = (w.lens - w.n_query).astype(np.int32)
    first = (prev // 4).astype(np.int32)
    k_idx = dev_bf16(w.k_idx)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, k_idx, dev_i32(prev), k_cmp)
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, dev_bf16(w.q_idx), k_idx, k_cmp, dev_bf16(w.q),
                               dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens),
                               first_block=dev_i32(first), sel=sel, n_sel=n_sel)
    torch.cuda.synchronize()
    return (host_f64_from_bf16(out), lse.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy())


def compare_selections(w, sel, n_sel, rows):
    ref = O.select_rows(w.q_idx, w.k_idx, w.lens, w.n_query, rows, threads=host_threads())
    bad = []
    for b, i in rows:
        want, nw = ref[(b, i)]
        ok = (n_sel[b, i] == nw and np.array_equal(sel[b, i, :nw], want)
              and (sel[b, i, nw:] == -1).all())
        if not ok:
            bad.append((b, i))
    assert not bad, f"{len(bad)} of {len(rows)} rows differ, first {bad[:8]}"


def compare_outputs(w, got, rows):
    out, lse, sel, n_sel = got
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query, queries=rows)
    for b, i in rows:
        want = res["sel"][(b, i)]
        assert n_sel[b, i] == want.shape[0], (b, i)
        np.testing.assert_array_equal(sel[b, i, :want.shape[0]], want, err_msg=f"row {(b, i)}")
        np.testing.assert_allclose(lse[b, i], res["lse"][(b, i)], atol=2e-2, rtol=0)
    check_close(np.stack([out[b, i] for b, i in rows]), np.stack([res["out"][r] for r in rows]))


def sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    nq = w.n_query
    picks = set(range(4)) | set(range(nq - 4, nq))
    picks |= set(int(x) for x in rng.choice(nq, size=n, replace=False))
    return [(0, i) for i in sorted(picks)]


@pytest.mark.parametrize("flags", [0, Q.FLAG_TOPK_SCAN], ids=["auto", "scan"])
def test_decode_1m_every_row(flags):
    # the automatic choice is the table engine; the scan engine (the one for
    # contexts whose score table would not fit) at the same shape
    say(f"decode 1M: inputs (flags {flags})")
    w = W.make(4)
    say("decode 1M: forward")
    got = run_forward(w, flags)
    say("decode 1M: oracle")
    compare_outputs(w, got, [(b, i) for b in range(w.batch) for i in range(w.n_query)])


def test_backward_1m_decode():
    # the backward passes on the batch and in the launch configuration bench.py
    # times them: every query row's dq; dk and dv on every token any query
    # read, and zero elsewhere; the indexer gradients over all 1M blocks
    say("backward 1M: inputs")
    w = W.make(4)
    B, L, Nq, Hq, Hkv = w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads
    shp = Q.shape(B, L, Nq, Hq, Hkv)
    prev = (w.lens - Nq).astype(np.int32)
    lens = dev_i32(w.lens)
    k_idx = dev_bf16(w.k_idx)
    k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, k_idx, dev_i32(prev), k_cmp)
    q, k, v, q_idx = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_bf16(w.q_idx)
    sel = torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((B, Nq), dtype=torch.int32, device="cuda")
    say("backward 1M: forward and backward")
    out, lse, _, _ = Q.forward(shp, q_idx, k_idx, k_cmp, q, k, v, lens,
                               first_block=dev_i32(prev // 4), sel=sel, n_sel=n_sel)
    rng = np.random.default_rng(4243)
    d_out_bits = bf16_bits_np(rng.standard_normal((B, Nq, Hq, 128)).astype(np.float32))
    g = rng.standard_normal((B, Nq, L // 4)).astype(np.float32)
    dq, dk, dv = Q.sparse_attend_backward(shp, q, k, v, lens, sel, n_sel, out, lse,
                                          dev_bf16(d_out_bits))
    dq_idx, dk_cmp = Q.index_scores_backward(shp, q_idx, k_cmp, lens, torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    say("backward 1M: oracle")
    res = O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, Nq)
    want_dq = np.zeros((B, Nq, Hq, 128))
    want_dq_idx = np.zeros((B, Nq, 4, 64))
    dq_h, dq_idx_h = dq.cpu().numpy(), dq_idx.cpu().numpy()
    for b in range(B):
        toks = [res["tok"][(b, i)] for i in range(Nq)]
        union = np.unique(np.concatenate(toks))
        pos = {int(t): n for n, t in enumerate(union)}
        kr = O.bf16_bits_to_f64(w.k[b, union])
        vr = O.bf16_bits_to_f64(w.v[b, union])
        want_dk = np.zeros(kr.shape)
        want_dv = np.zeros(vr.shape)
        kc = O.bf16_bits_to_f64(res["kc"][b])
        want_dkc = np.zeros((L // 4, 64))
        for i in range(Nq):
            rows = np.array([pos[int(t)] for t in toks[i]])
            gq, gk, gv = O.attend_backward(O.bf16_bits_to_f64(w.q[b, i]), kr[rows], vr[rows],
                                           O.bf16_bits_to_f64(d_out_bits[b, i]), w.scale)
            want_dq[b, i] = gq
            np.add.at(want_dk, rows, gk)
            np.add.at(want_dv, rows, gv)
            bt = (int(w.lens[b]) - Nq + i) // 4
            gi, gkc = O.block_scores_backward(O.bf16_bits_to_f64(w.q_idx[b, i]), kc[:bt],
                                              g[b, i, :bt].astype(np.float64))
            want_dq_idx[b, i] = gi
            want_dkc[:bt] += gkc
        ut = torch.from_numpy(union).cuda()
        check_close(dk[b].index_select(0, ut).cpu().numpy(), want_dk)
        check_close(dv[b].index_select(0, ut).cpu().numpy(), want_dv)
        # no other row was touched
        nz = (dk[b] != 0).any(-1).any(-1) | (dv[b] != 0).any(-1).any(-1)
        assert int(nz.sum()) <= union.size and not bool(nz.index_fill(0, ut, False).any())
        got_dkc = dk_cmp[b].cpu().numpy()
        rel = np.linalg.norm(got_dkc - want_dkc) / np.linalg.norm(want_dkc)
        assert rel <= 1e-5, f"dk_cmp of sequence {b}: rel-L2 {rel:.2e}"
    check_close(dq_h, want_dq)
    rel = np.linalg.norm(dq_idx_h - want_dq_idx) / np.linalg.norm(want_dq_idx)
    assert rel <= 1e-5, f"dq_idx: rel-L2 {rel:.2e}"


def test_prefill_256k_every_row_selection():
    say("prefill 256K: inputs")
    w = W.make(2)
    say("prefill 256K: forward")
    got = run_forward(w)
    _, _, sel, n_sel = got
    say("prefill 256K: oracle selections of all 16,384 rows")
    compare_selections(w, sel, n_sel, [(0, i) for i in range(w.n_query)])
    say("prefill 256K: oracle outputs of sampled rows")
    compare_outputs(w, got, sample_rows(w, 40, 1002))


def test_prefill_1m_every_row_selection():
    say("prefill 1M: inputs")
    w = W.make(3)
    say("prefill 1M: forward")
    got = run_forward(w)
    _, _, sel, n_sel = got
    say("prefill 1M: oracle selections of all 16,384 rows")
    compare_selections(w, sel, n_sel, [(0, i) for i in range(w.n_query)])
    say("prefill 1M: oracle outputs of sampled rows")
    compare_outputs(w, got, sample_rows(w, 24, 1003))


def test_dense_decode_1m_one_row_per_sequence():
    say("dense 1M: inputs")
    w = W.make(4)
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    say("dense 1M: kernel")
    out, lse = Q.dense_gqa_decode(shp, dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                  dev_i32(w.lens))
    got = host_f64_from_bf16(out)
    lse_h = lse.cpu().numpy()
    rows = [(b, (3 * b + 1) % w.n_query) for b in range(w.batch)]
    say("dense 1M: oracle")
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query, queries=rows)
    check_close(np.stack([got[b, i] for b, i in rows]), np.stack([ref[r][0] for r in rows]))
    for b, i in rows:
        np.testing.assert_allclose(lse_h[b, i], ref[(b, i)][1], atol=2e-2, rtol=0)


def test_paged_decode_1m_matches_contiguous():
    say("paged decode 1M: inputs")
    w = W.make(4)
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    prev = (w.lens - w.n_query).astype(np.int32)
    first = dev_i32((prev // 4).astype(np.int32))
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, t["k_idx"], dev_i32(prev), k_cmp)
    k_cmp2 = k_cmp.clone()
    say("paged decode 1M: pools")
    k_pool, v_pool, pg = paged_pools_dev(t["k"], t["v"], w.lens, 16, 41)
    say("paged decode 1M: forward, contiguous and paged")
    o1, l1, s1, n1 = Q.forward(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], lens,
                               first_block=first,
                               sel=torch.empty((w.batch, w.n_query, 512), dtype=torch.int32,
                                               device="cuda"),
                               n_sel=torch.empty((w.batch, w.n_query), dtype=torch.int32,
                                                 device="cuda"))
    o2, l2, s2, n2 = Q.forward_paged(shp, t["q_idx"], t["k_idx"], k_cmp2, t["q"], k_pool, v_pool,
                                     pg, lens, first_block=first,
                                     sel=torch.empty_like(s1), n_sel=torch.empty_like(n1))
    say("paged decode 1M: dense comparator, contiguous and paged")
    d1, dl1 = Q.dense_gqa_decode(shp, t["q"], t["k"], t["v"], lens)
    d2, dl2 = Q.dense_gqa_decode_paged(shp, t["q"], k_pool, v_pool, pg, lens)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(n1, n2) and torch.equal(k_cmp, k_cmp2)
    for a, b in ((o1, o2), (l1, l2), (d1, d2), (dl1, dl2)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_dense_prefill_1m_chunk():
    say("dense prefill 1M: inputs")
    w = W.make(3)
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    q, k, v, lens = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens)
    say("dense prefill 1M: contiguous")
    o1, l1 = Q.dense_gqa_prefill(shp, q, k, v, lens)
    say("dense prefill 1M: paged")
    k_pool, v_pool, pg = paged_pools_dev(k, v, w.lens, 16, 42)
    o2, l2 = Q.dense_gqa_prefill(shp, q, k_pool, v_pool, lens, paged=pg)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    got = host_f64_from_bf16(o1)
    lse_h = l1.cpu().numpy()
    rows = [(0, 0), (0, 8191), (0, w.n_query - 1)]
    say("dense prefill 1M: oracle on", rows)
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query, queries=rows)
    check_close(np.stack([got[r] for r in rows]), np.stack([ref[r][0] for r in rows]))
    for r in rows:
        np.testing.assert_allclose(lse_h[r], ref[r][1], atol=2e-2, rtol=0)
