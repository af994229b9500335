"""Parity of every C-ABI entry point against the CPU oracle, on seeded inputs
of the synthetic workloads and on degenerate inputs.  Indices are compared
bit for bit; attention outputs to max-abs <= 2e-2 and rel-L2 <= 1e-2."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import (check_close, dev_bf16, dev_i32, host_u16, host_f64_from_bf16,
                      padded_sel, padded_tok)

pytestmark = pytest.mark.gpu

ENGINES = [Q.FLAG_TOPK_TABLE, Q.FLAG_TOPK_STREAM, Q.FLAG_TOPK_SCAN]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_const(shape, value):
    f = np.full(shape, value, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def custom(seed=100, lens=(20001, 2000, 60000, 2053), nq=70, hq=16, hkv=2, needles=0,
           max_len=None, parts=("index", "attn")):
    return W.make_custom(seed, list(lens), nq, hq, hkv, max_len=max_len, needles=needles,
                         parts=parts)


def shape_of(w, flags=0):
    return Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads, 0.0, flags)


def gpu_kcmp(w):
    shp = shape_of(w)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, dev_bf16(w.k_idx), dev_i32(w.lens), k_cmp)
    return k_cmp


def oracle_select(w):
    return O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, w.n_query)


# ------------------------------------------------------------------ compress

def test_compress_cfg0_bit_exact():
    say("compress cfg0")
    w = W.make(0, parts=("index",))
    got = host_u16(gpu_kcmp(w))
    want = O.compress_keys(w.k_idx[0], int(w.lens[0]))
    np.testing.assert_array_equal(got[0, :want.shape[0]], want)


def test_compress_partial_range_and_real_values():
    say("compress ragged / first_block / N(0,1) values")
    rng = np.random.default_rng(5)
    B, L = 3, 4096
    lens = np.array([1001, 4096, 37], np.int32)
    first = np.array([0, 100, 3], np.int32)
    # normal-distributed keys exercise the rounding, not just integer sums
    k = (rng.standard_normal((B, L, 64)).astype(np.float32) * 3).view(np.uint32)
    k_idx = ((k + 0x7FFF + ((k >> 16) & 1)) >> 16).astype(np.uint16)
    shp = Q.shape(B, L, 1, 8, 1)
    sentinel = 0x7FC1
    k_cmp = torch.full((B, L // 4, 64), sentinel, dtype=torch.int16, device="cuda")
    Q.compress_keys(shp, dev_bf16(k_idx), dev_i32(lens), k_cmp, dev_i32(first))
    got = host_u16(k_cmp)
    for b in range(B):
        nb = int(lens[b]) // 4
        fb = int(first[b])
        want = O.compress_keys(k_idx[b], int(lens[b]), first_block=fb)
        np.testing.assert_array_equal(got[b, fb:nb], want)
        assert np.all(got[b, :fb] == sentinel) and np.all(got[b, nb:] == sentinel)


# ------------------------------------------------------------------ index + top-k

def run_topk(w, flags, k_cmp=None):
    shp = shape_of(w, flags)
    if k_cmp is None:
        k_cmp = gpu_kcmp(w)
    sel, n_sel = Q.index_topk(shp, dev_bf16(w.q_idx), k_cmp, dev_i32(w.lens))
    return sel.cpu().numpy(), n_sel.cpu().numpy()


def check_topk(w, flags, res=None):
    if res is None:
        res = oracle_select(w)
    want_sel, want_n = padded_sel(res, w.batch, w.n_query, w.lens)
    sel, n_sel = run_topk(w, flags)
    np.testing.assert_array_equal(n_sel, want_n)
    bad = np.argwhere(np.any(sel != want_sel, axis=-1))
    assert bad.shape[0] == 0, f"{bad.shape[0]} rows differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_cfg0(flags):
    say("topk cfg0", flags)
    w = W.make(0, parts=("index",))
    check_topk(w, flags)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_ragged_batch(flags):
    say("topk ragged", flags)
    w = custom(parts=("index",), needles=0)
    check_topk(w, flags)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_needles(flags):
    say("topk needles", flags)
    w = W.make_custom(7, [40000], 200, 8, 1, needles=8, parts=("index",))
    res = oracle_select(w)
    # the planted spans must actually be competitive
    nb = set(j for s in w.needle_starts[0] for j in range(s // 4, s // 4 + 16))
    hits = np.mean([len(nb & set(res["sel"][(0, i)].tolist())) for i in range(200)])
    assert hits > 40
    check_topk(w, flags, res)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_all_zero_keys(flags):
    # every score is 0: the lowest 512 block ids win
    say("topk all-zero", flags)
    w = custom(lens=(9000, 30000), nq=9, parts=("index",))
    w.k_idx[:] = 0
    res = oracle_select(w)
    for (b, i), s in res["sel"].items():
        assert np.array_equal(s, np.arange(512))
    check_topk(w, flags, res)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_all_equal_scores(flags):
    say("topk all-equal", flags)
    w = custom(lens=(12000,), nq=66, parts=("index",))
    w.k_idx[:] = bf16_const(w.k_idx.shape, 1.0)
    w.q_idx[:] = bf16_const(w.q_idx.shape, 1.0)
    check_topk(w, flags)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_ties_at_the_cut(flags):
    # three score values: ~300 blocks score 8, ~6,000 score 4, the rest 0, so
    # the 512th key is a 4 and the lowest-index 4s fill the remainder; the
    # stream engine's candidate list overflows and the whole-row path decides
    say("topk ties at the cut", flags)
    w = custom(lens=(60000, 59999), nq=6, parts=("index",))
    rng = np.random.default_rng(7)
    cls = rng.choice(3, size=(2, w.max_len // 4), p=[0.58, 0.40, 0.02]).astype(np.float32)
    w.k_idx[:] = 0
    w.k_idx[:, 0::4, 0] = (cls.view(np.uint32) >> 16).astype(np.uint16)
    w.q_idx[:] = bf16_const(w.q_idx.shape, 1.0)
    res = oracle_select(w)
    for (b, i), s in res["sel"].items():
        t = int(w.lens[b]) - w.n_query + i
        sc = cls[b, :t // 4]
        n_top = int((sc == 2).sum())
        assert 0 < n_top < 512 and np.array_equal(np.sort(s), s)
        assert set(np.flatnonzero(sc == 2).tolist()) <= set(s.tolist())
    check_topk(w, flags, res)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_increasing_scores(flags):
    # scores grow with the block id: every new block beats the running
    # threshold (worst case for the streaming engine)
    say("topk increasing", flags)
    w = custom(lens=(50000,), nq=5, parts=("index",))
    vals = np.minimum(8, 1 + np.arange(w.max_len) // 6000).astype(np.float32)
    w.k_idx[0] = (np.repeat(vals[:, None], 64, 1).view(np.uint32) >> 16).astype(np.uint16)
    w.q_idx[:] = bf16_const(w.q_idx.shape, 1.0)
    rng = np.random.default_rng(1)
    w.q_idx[0, :, 0, :] = bf16_const((5, 64), 2.0) * (rng.integers(0, 2, (5, 64)) > 0)
    check_topk(w, flags)


@pytest.mark.parametrize("flags", ENGINES)
def test_topk_wide_score_range(flags):
    # a few hundred outlier blocks score up to ~100x the rest, so the table
    # engine's linear bins are coarse and its cutoff bin holds several score
    # values: the bit-level refinement decides (scores stay exact integers)
    say("topk wide range", flags)
    w = custom(seed=41, lens=(90001, 70000), nq=6, parts=("index",))
    rng = np.random.default_rng(41)
    for b in range(w.batch):
        blocks = rng.choice(int(w.lens[b]) // 4 - 64, size=300, replace=False)
        for j, f in zip(blocks, rng.choice([8.0, 64.0], size=blocks.shape[0])):
            rows = w.k_idx[b, 4 * j:4 * j + 4].view(np.uint16).astype(np.uint32) << 16
            vals = rows.view(np.float32) * np.float32(f)
            w.k_idx[b, 4 * j:4 * j + 4] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    check_topk(w, flags)


def scale_blocks(w, b, blocks, f):
    """Multiply the indexer keys of the given micro-blocks of sequence b by f
    (small integers stay exact)."""
    for j in blocks:
        rows = w.k_idx[b, 4 * j:4 * j + 4].astype(np.uint32) << 16
        vals = rows.view(np.float32) * np.float32(f)
        w.k_idx[b, 4 * j:4 * j + 4] = (vals.view(np.uint32) >> 16).astype(np.uint16)


def test_topk_scan_bound_above_the_cut():
    # 100 outlier blocks, 20 of them spread like the scan engine's samples:
    # its sampled bound then lies above all but the outliers, fewer than 512
    # blocks reach it, and the row takes the exact whole-row path
    say("topk scan: bound above the 512th score")
    w = custom(seed=43, lens=(80001,), nq=4, parts=("index",))
    bt_min = (int(w.lens[0]) - w.n_query) // 4
    spread = [i * bt_min // 1024 for i in range(0, 1024, 51)][:20]
    rng = np.random.default_rng(43)
    others = rng.choice(bt_min, size=80, replace=False).tolist()
    scale_blocks(w, 0, sorted(set(spread) | set(others)), 16.0)
    check_topk(w, Q.FLAG_TOPK_SCAN)


def test_topk_scan_segment_overflow():
    # 700 consecutive outlier blocks: one slice holds more candidates than its
    # segment, and the row takes the exact whole-row path
    say("topk scan: segment overflow")
    w = custom(seed=44, lens=(600001,), nq=4, parts=("index",))
    scale_blocks(w, 0, range(70000, 70700), 4.0)
    check_topk(w, Q.FLAG_TOPK_SCAN)


def test_topk_scan_more_candidates_than_the_list_holds():
    # every score is 0 over 15,000 blocks: all are candidates, more than the
    # select's LDS list holds; the lowest 512 ids win
    say("topk scan: candidate list overflow")
    w = custom(lens=(60001,), nq=3, parts=("index",))
    w.k_idx[:] = 0
    check_topk(w, Q.FLAG_TOPK_SCAN)


def test_topk_engines_agree_on_cfg1():
    say("topk cfg1 engines")
    w = W.make(1, parts=("index",))
    k_cmp = gpu_kcmp(w)
    a = run_topk(w, Q.FLAG_TOPK_TABLE, k_cmp)
    b = run_topk(w, Q.FLAG_TOPK_STREAM, k_cmp)
    c = run_topk(w, Q.FLAG_TOPK_SCAN, k_cmp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])
    res = oracle_select(w)
    want_sel, want_n = padded_sel(res, w.batch, w.n_query, w.lens)
    np.testing.assert_array_equal(a[0], want_sel)
    np.testing.assert_array_equal(a[1], want_n)


def test_topk_deterministic():
    say("topk determinism")
    w = custom(lens=(30001,), nq=40, parts=("index",))
    k_cmp = gpu_kcmp(w)
    for flags in ENGINES:
        a = run_topk(w, flags, k_cmp)
        b = run_topk(w, flags, k_cmp)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ expand

def test_expand_bit_exact():
    say("expand")
    w = custom(parts=("index",))
    res = oracle_select(w)
    sel, n_sel = padded_sel(res, w.batch, w.n_query, w.lens)
    want_tok, want_n = padded_tok(res, w.batch, w.n_query)
    tok, n_tok = Q.expand_blocks(shape_of(w), dev_i32(w.lens), dev_i32(sel), dev_i32(n_sel))
    np.testing.assert_array_equal(n_tok.cpu().numpy(), want_n)
    np.testing.assert_array_equal(tok.cpu().numpy(), want_tok)


# ------------------------------------------------------------------ attention

def check_attend_with_oracle_sel(w, res):
    sel, n_sel = padded_sel(res, w.batch, w.n_query, w.lens)
    out, lse = Q.sparse_attend(shape_of(w), dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.lens), dev_i32(sel), dev_i32(n_sel))
    got = host_f64_from_bf16(out)
    lse = lse.cpu().numpy()
    keys = sorted(res["out"].keys())
    ref = np.stack([res["out"][k] for k in keys])
    g = np.stack([got[b, i] for b, i in keys])
    check_close(g, ref)
    ref_lse = np.stack([res["lse"][k] for k in keys])
    g_lse = np.stack([lse[b, i] for b, i in keys])
    assert np.max(np.abs(g_lse - ref_lse)) < 2e-3


def test_sparse_attend_cfg0():
    say("attend cfg0")
    w = W.make(0)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    check_attend_with_oracle_sel(w, res)


@pytest.mark.parametrize("hq,hkv", [(16, 2), (40, 2), (4, 4)])
def test_sparse_attend_head_layouts(hq, hkv):
    say("attend heads", hq, hkv)
    w = custom(lens=(7001, 3003, 2051), nq=12, hq=hq, hkv=hkv)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    check_attend_with_oracle_sel(w, res)


# 8/1: a workgroup per (query, KV head); 32/4 and 4/4: the four KV heads of a
# query in one workgroup (at least 1,024 (query, KV head) units)
@pytest.mark.parametrize("nq,hq,hkv", [(1100, 8, 1), (300, 32, 4), (260, 4, 4)])
def test_sparse_attend_many_rows_single_split(nq, hq, hkv):
    # enough query rows that no split/merge is used
    say("attend many rows", nq, hq, hkv)
    w = W.make_custom(9, [6000], nq, hq, hkv)
    qs = [(0, i) for i in range(0, nq, 37)] + [(0, nq - 1)]
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query, queries=qs)
    sel_all, n_all = padded_sel(O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens,
                                              w.n_query), 1, nq, w.lens)
    out, lse = Q.sparse_attend(shape_of(w), dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                               dev_i32(w.lens), dev_i32(sel_all), dev_i32(n_all))
    got = host_f64_from_bf16(out)
    ref = np.stack([res["out"][k] for k in qs])
    check_close(np.stack([got[b, i] for b, i in qs]), ref)


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("flags", ENGINES)
def test_forward_very_short_sequences(flags):
    # contexts of 4..11 tokens with 4 queries each: the first queries have no
    # completed block before their own (nothing to select, attention over
    # tokens 4 bt .. t only), the later ones select every earlier block
    say("forward very short", flags)
    w = custom(lens=(4, 5, 7, 8, 11), nq=4)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    shp = shape_of(w, flags)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, dev_bf16(w.q_idx), dev_bf16(w.k_idx), k_cmp, dev_bf16(w.q),
                               dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens), sel=sel, n_sel=n_sel)
    want_sel, want_n = padded_sel(res, w.batch, w.n_query, w.lens)
    np.testing.assert_array_equal(n_sel.cpu().numpy(), want_n)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    got = host_f64_from_bf16(out)
    keys = sorted(res["out"].keys())
    check_close(np.stack([got[b, i] for b, i in keys]), np.stack([res["out"][k] for k in keys]))
    g_lse = lse.cpu().numpy()
    assert max(abs(g_lse[b, i] - res["lse"][(b, i)]).max() for b, i in keys) < 2e-3



@pytest.mark.parametrize("flags", ENGINES)
def test_forward_cfg0(flags):
    say("forward cfg0", flags)
    w = W.make(0)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    shp = shape_of(w, flags)
    k_cmp = torch.zeros((1, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((1, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((1, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, dev_bf16(w.q_idx), dev_bf16(w.k_idx), k_cmp, dev_bf16(w.q),
                               dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens), sel=sel, n_sel=n_sel)
    want_sel, want_n = padded_sel(res, 1, w.n_query, w.lens)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    np.testing.assert_array_equal(n_sel.cpu().numpy(), want_n)
    np.testing.assert_array_equal(host_u16(k_cmp)[0, :1024], res["kc"][0])
    got = host_f64_from_bf16(out)
    check_close(np.stack([got[0, i] for i in range(w.n_query)]),
                np.stack([res["out"][(0, i)] for i in range(w.n_query)]))


def test_forward_cfg1_decode_128k():
    # decode-shaped: the key compression runs inside the scoring pass
    say("forward cfg1")
    w = W.make(1)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    shp = shape_of(w)
    sentinel = 0x7fc1
    k_cmp = torch.full((w.batch, w.max_len // 4, 64), sentinel, dtype=torch.int16,
                       device="cuda").view(torch.bfloat16)
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, dev_bf16(w.q_idx), dev_bf16(w.k_idx), k_cmp, dev_bf16(w.q),
                               dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens), sel=sel, n_sel=n_sel)
    want_sel, want_n = padded_sel(res, w.batch, w.n_query, w.lens)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    np.testing.assert_array_equal(n_sel.cpu().numpy(), want_n)
    kc = host_u16(k_cmp)
    for b in range(w.batch):
        nb = int(w.lens[b]) // 4
        np.testing.assert_array_equal(kc[b, :nb], res["kc"][b], err_msg=f"k_cmp of sequence {b}")
        assert (kc[b, nb:] == sentinel).all(), f"k_cmp written past block {nb} of sequence {b}"
    got = host_f64_from_bf16(out)
    keys = sorted(res["out"].keys())
    check_close(np.stack([got[b, i] for b, i in keys]), np.stack([res["out"][k] for k in keys]))


def test_forward_incremental_decode_steps():
    # a decode loop: 4 tokens appended per step, only the new block compressed
    say("forward incremental")
    w = W.make_custom(33, [9000, 9001], 4, 16, 2, max_len=9100)
    shp = shape_of(w)
    k_idx = dev_bf16(w.k_idx)
    k_cmp = torch.zeros((2, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    q_idx, q, k, v = dev_bf16(w.q_idx), dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v)
    lens0 = np.array([8992, 8993], np.int32)
    Q.compress_keys(shp, k_idx, dev_i32(lens0), k_cmp)
    for step in range(3):
        lens = lens0 + 4 * (step + 1)
        prev = lens - 4
        first = (prev // 4).astype(np.int32)
        out, lse, sel, n_sel = Q.forward(shp, q_idx, k_idx, k_cmp, q, k, v, dev_i32(lens),
                                         first_block=dev_i32(first),
                                         sel=torch.empty((2, 4, 512), dtype=torch.int32, device="cuda"),
                                         n_sel=torch.empty((2, 4), dtype=torch.int32, device="cuda"))
        res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, lens, 4)
        want_sel, want_n = padded_sel(res, 2, 4, lens)
        np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
        kc = host_u16(k_cmp)
        for b in range(2):
            np.testing.assert_array_equal(kc[b, :lens[b] // 4], res["kc"][b])
        got = host_f64_from_bf16(out)
        keys = sorted(res["out"].keys())
        check_close(np.stack([got[b, i] for b, i in keys]), np.stack([res["out"][k] for k in keys]))


@pytest.mark.parametrize("nq", [1, 2, 3])
@pytest.mark.parametrize("flags", [0, Q.FLAG_TOPK_SCAN], ids=["auto", "scan"])
def test_forward_decode_odd_query_counts(nq, flags):
    # decode steps of 1-3 query positions (a partial group of 4 in the scan
    # kernels, whose spare rows repeat the last query), in the steady state
    # (the cache holds every block before the step, the call compresses only
    # the new ones); lengths of every residue mod 4, one under the 2,052-token
    # dense range and a 4-token context
    say(f"forward decode nq={nq} flags={flags}")
    lens = np.array([70003, 33334, 131075, 2050, 4 + nq], np.int32)
    w = W.make_custom(60 + nq, list(lens), nq, 16, 2)
    shp = shape_of(w, flags)
    k_idx = dev_bf16(w.k_idx)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    prev = lens - nq
    Q.compress_keys(shp, k_idx, dev_i32(prev), k_cmp)
    out, lse, sel, n_sel = Q.forward(
        shp, dev_bf16(w.q_idx), k_idx, k_cmp, dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
        dev_i32(lens), first_block=dev_i32((prev // 4).astype(np.int32)),
        sel=torch.empty((w.batch, nq, 512), dtype=torch.int32, device="cuda"),
        n_sel=torch.empty((w.batch, nq), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, lens, nq)
    want_sel, want_n = padded_sel(res, w.batch, nq, lens)
    np.testing.assert_array_equal(n_sel.cpu().numpy(), want_n)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
    kc = host_u16(k_cmp)
    for b in range(w.batch):
        np.testing.assert_array_equal(kc[b, :lens[b] // 4], res["kc"][b])
    got = host_f64_from_bf16(out)
    keys = sorted(res["out"].keys())
    check_close(np.stack([got[b, i] for b, i in keys]), np.stack([res["out"][k] for k in keys]))
    lse_h = lse.cpu().numpy()
    for k in keys:
        np.testing.assert_allclose(lse_h[k], res["lse"][k], atol=2e-2, rtol=0, err_msg=str(k))


def test_host_lens_check(monkeypatch):
    # QSA_CHECK=1: the library reads lens back before launching anything and
    # rejects a sequence shorter than its query count or longer than the
    # cache; without it the call trusts lens (the caller's contract)
    say("QSA_CHECK")
    w = W.make_custom(70, [3000, 2500], 4, 16, 2)
    shp = shape_of(w)
    args = (dev_bf16(w.q_idx), dev_bf16(w.k_idx), gpu_kcmp(w), dev_bf16(w.q), dev_bf16(w.k),
            dev_bf16(w.v))
    monkeypatch.setenv("QSA_CHECK", "1")
    out, _ = Q.forward(shp, *args, dev_i32(w.lens))[:2]  # valid: runs
    torch.cuda.synchronize()
    for bad in ([3000, 3], [3000, w.max_len + 4]):
        with pytest.raises(Q.QsaError) as err:
            Q.forward(shp, *args, dev_i32(np.array(bad, np.int32)))
        assert err.value.status == Q.ERR_SHAPE
    monkeypatch.delenv("QSA_CHECK")
    out2, _ = Q.forward(shp, *args, dev_i32(w.lens))[:2]
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


# ------------------------------------------------------------------ dense comparator

@pytest.mark.parametrize("nq", [6, 9])  # 3 and 5 chunks of 16 (query, head) columns per KV head
def test_dense_decode_small(nq):
    say(f"dense small nq={nq}")
    w = custom(lens=(5000, 333, 12), nq=nq, hq=16, hkv=2)
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query)
    out, lse = Q.dense_gqa_decode(shape_of(w), dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                  dev_i32(w.lens))
    got = host_f64_from_bf16(out)
    keys = sorted(ref.keys())
    check_close(np.stack([got[b, i] for b, i in keys]), np.stack([ref[k][0] for k in keys]))
    g_lse = lse.cpu().numpy()
    assert max(abs(g_lse[b, i] - ref[(b, i)][1]).max() for b, i in keys) < 2e-3


def test_dense_decode_cfg1_sampled():
    say("dense cfg1")
    w = W.make(1)
    keys = [(0, 0), (1, 3), (2, 1), (3, 2)]
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query, queries=keys)
    out, _ = Q.dense_gqa_decode(shape_of(w), dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                dev_i32(w.lens))
    got = host_f64_from_bf16(out)
    check_close(np.stack([got[b, i] for b, i in keys]), np.stack([ref[k][0] for k in keys]))


# ------------------------------------------------------------------ timing hook

def test_kernel_timer_records_every_launch():
    # the per-launch events ride in each dispatch: one record per kernel, in
    # launch order, each a positive duration, and the results unchanged
    say("kernel timer")
    w = custom(lens=(9000, 5000), nq=4, hq=16, hkv=2)
    shp = shape_of(w, Q.FLAG_TOPK_TABLE)
    k_cmp = gpu_kcmp(w)
    args = (dev_bf16(w.q_idx), dev_bf16(w.k_idx), k_cmp, dev_bf16(w.q), dev_bf16(w.k),
            dev_bf16(w.v), dev_i32(w.lens))
    out0, _ = Q.forward(shp, *args)[:2]
    timer = Q.KernelTimer(max_launches=16)
    with timer:
        out1, _ = Q.forward(shp, *args)[:2]
    recs = timer.records()
    names = [n for n, _ in recs]
    known = ("compress_kernel", "score_table_kernel", "table_pick_kernel", "sparse_attend_kernel",
             "merge_kernel")
    assert all(n.startswith(known) for n in names), names
    base = [n.split("<")[0] for n in names]  # template instances under their base name
    assert base.index("score_table_kernel") < base.index("table_pick_kernel"), names
    assert any(n.startswith("sparse_attend_kernel") for n in names), names
    assert all(ms > 0.0 for _, ms in recs), recs
    assert torch.equal(out0, out1)
