"""Paged K/V: the QSA forward (decode- and prefill-shaped), the sparse
attention and the dense decode comparator read K and V through a page table
over shuffled page pools, and must give bit-identical results to the
contiguous caches (only the addressing differs).  Pool rows past a sequence's length, the pages its
table does not need and the pool's spare pages hold NaN, so a read of
anything outside the valid tokens would show.  The dense prefill comparator
(contiguous and paged) is checked against the float64 oracle on sampled
rows, to the attention tolerance."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import check_close, dev_bf16, dev_i32, host_f64_from_bf16, host_u16

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_pool(k, v, lens, page, seed, spare=3):
    """Page pools holding the contiguous caches k, v ([B][L][Hkv][128]
    host bf16 bits) under a random page permutation.  Returns (k_pool,
    v_pool, PagedKV) on the device."""
    B, L, Hkv, D = k.shape
    max_pages = (L + page - 1) // page
    rng = np.random.default_rng(seed)
    n_pages = B * max_pages + spare
    ids = rng.permutation(n_pages)
    poison = int(ids[-1])  # a spare page: every unneeded table entry points here
    kp = np.full((n_pages, page, Hkv, D), NAN_BF16, dtype=np.uint16)
    vp = np.full((n_pages, page, Hkv, D), NAN_BF16, dtype=np.uint16)
    table = np.full((B, max_pages), poison, dtype=np.int32)
    nxt = 0
    for b in range(B):
        n = int(lens[b])
        for p in range((n + page - 1) // page):
            pid = int(ids[nxt])
            nxt += 1
            table[b, p] = pid
            lo, hi = p * page, min(n, (p + 1) * page)
            kp[pid, :hi - lo] = k[b, lo:hi]
            vp[pid, :hi - lo] = v[b, lo:hi]
    return dev_bf16(kp), dev_bf16(vp), Q.PagedKV(dev_i32(table), page, n_pages)


def bits(t):
    return t.view(torch.int32).cpu().numpy() if t.dtype == torch.float32 else host_u16(t)


@pytest.mark.parametrize("page", [1, 16, 256])
def test_paged_forward_and_attend_match_contiguous(page):
    w = W.make_custom(1100 + page, [6001, 2100, 30002], 5, 16, 2)
    say(f"paged forward: page {page}, lens {list(w.lens)}")
    B, L, Nq = w.batch, w.max_len, w.n_query
    shp = Q.shape(B, L, Nq, 16, 2)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_pool, v_pool, pg = make_pool(w.k, w.v, w.lens, page, 1200 + page)

    def sel_bufs():
        return (torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda"),
                torch.empty((B, Nq), dtype=torch.int32, device="cuda"))

    kc1 = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    kc2 = torch.zeros_like(kc1)
    s1, n1 = sel_bufs()
    s2, n2 = sel_bufs()
    o1, l1, _, _ = Q.forward(shp, t["q_idx"], t["k_idx"], kc1, t["q"], t["k"], t["v"], lens,
                             sel=s1, n_sel=n1)
    o2, l2, _, _ = Q.forward_paged(shp, t["q_idx"], t["k_idx"], kc2, t["q"], k_pool, v_pool, pg,
                                   lens, sel=s2, n_sel=n2)
    o3, l3 = Q.sparse_attend_paged(shp, t["q"], k_pool, v_pool, pg, lens, s1, n1)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(n1, n2)
    np.testing.assert_array_equal(bits(kc1), bits(kc2))
    for o, l in ((o2, l2), (o3, l3)):
        np.testing.assert_array_equal(bits(o), bits(o1))
        np.testing.assert_array_equal(bits(l), bits(l1))
    # and the paged result is the oracle's on a few rows
    rows = [(0, 0), (1, Nq - 1), (2, 2)]
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, Nq, queries=rows)
    got = host_f64_from_bf16(o2)
    check_close(np.stack([got[r] for r in rows]), np.stack([res["out"][r] for r in rows]))


@pytest.mark.parametrize("page", [2, 4, 64])
def test_paged_prefill_forward_matches_contiguous(page):
    # a prefill-shaped call (300 queries x 4 KV heads fill the chip without
    # splits): the stream top-k engine and the attention workgroups that hold
    # all four KV heads of a query, reading the pools through the table
    nq = 300
    w = W.make_custom(1700 + page, [20003, 9001], nq, 32, 4)
    say(f"paged prefill forward: page {page}, lens {list(w.lens)}")
    B, L = w.batch, w.max_len
    shp = Q.shape(B, L, nq, 32, 4)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_pool, v_pool, pg = make_pool(w.k, w.v, w.lens, page, 1800 + page)
    kc1 = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    kc2 = torch.zeros_like(kc1)
    def sel_bufs():
        return (torch.empty((B, nq, 512), dtype=torch.int32, device="cuda"),
                torch.empty((B, nq), dtype=torch.int32, device="cuda"))

    s1, n1 = sel_bufs()
    s2, n2 = sel_bufs()
    o1, l1, _, _ = Q.forward(shp, t["q_idx"], t["k_idx"], kc1, t["q"], t["k"], t["v"], lens,
                             sel=s1, n_sel=n1)
    o2, l2, _, _ = Q.forward_paged(shp, t["q_idx"], t["k_idx"], kc2, t["q"], k_pool, v_pool, pg,
                                   lens, sel=s2, n_sel=n2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(n1, n2)
    np.testing.assert_array_equal(bits(o2), bits(o1))
    np.testing.assert_array_equal(bits(l2), bits(l1))
    rows = [(0, 0), (0, nq - 1), (1, 7), (1, nq - 1)]
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, nq, queries=rows)
    got = host_f64_from_bf16(o2)
    check_close(np.stack([got[r] for r in rows]), np.stack([res["out"][r] for r in rows]))


@pytest.mark.parametrize("page", [1, 16, 4096])
def test_paged_dense_decode_matches_contiguous(page):
    w = W.make_custom(1300 + page, [20001, 9000, 70003, 4], 4, 32, 4)
    say(f"paged dense decode: page {page}, lens {list(w.lens)}")
    B, L, Nq = w.batch, w.max_len, w.n_query
    shp = Q.shape(B, L, Nq, 32, 4)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    lens = dev_i32(w.lens)
    k_pool, v_pool, pg = make_pool(w.k, w.v, w.lens, page, 1400 + page)
    o1, l1 = Q.dense_gqa_decode(shp, q, k, v, lens)
    o2, l2 = Q.dense_gqa_decode_paged(shp, q, k_pool, v_pool, pg, lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o2), bits(o1))
    np.testing.assert_array_equal(bits(l2), bits(l1))
    rows = [(0, 3), (2, 0), (3, 3)]
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, Nq, queries=rows)
    got = host_f64_from_bf16(o2)
    check_close(np.stack([got[r] for r in rows]), np.stack([ref[r][0] for r in rows]))


@pytest.mark.parametrize("hq,hkv", [(32, 4), (8, 8), (24, 4), (64, 1)])
def test_dense_prefill_matches_the_oracle(hq, hkv):
    # 300 queries span several query tiles of a workgroup (256 // G each);
    # the second sequence's first query sees one token; the first is ragged
    nq = 300
    w = W.make_custom(1500 + hq, [5001, nq, 9002], nq, hq, hkv)
    say(f"dense prefill: {hq}/{hkv} heads, lens {list(w.lens)}, {nq} queries")
    B, L = w.batch, w.max_len
    shp = Q.shape(B, L, nq, hq, hkv)
    q, k, v = dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    lens = dev_i32(w.lens)
    o1, l1 = Q.dense_gqa_prefill(shp, q, k, v, lens)
    k_pool, v_pool, pg = make_pool(w.k, w.v, w.lens, 64, 1600 + hq)
    o2, l2 = Q.dense_gqa_prefill(shp, q, k_pool, v_pool, lens, paged=pg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o2), bits(o1))
    np.testing.assert_array_equal(bits(l2), bits(l1))
    qw = 256 // (hq // hkv)
    picks = sorted({0, 1, qw - 1, qw, 2 * qw - 1, nq - 2, nq - 1} & set(range(nq)))
    rows = [(b, i) for b in range(B) for i in picks]
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, nq, queries=rows)
    got = host_f64_from_bf16(o1)
    lse = l1.cpu().numpy()
    check_close(np.stack([got[r] for r in rows]), np.stack([ref[r][0] for r in rows]))
    for r in rows:
        np.testing.assert_allclose(lse[r], ref[r][1], atol=2e-3, rtol=0, err_msg=str(r))
