"""Backward passes against the float64 oracle: the sparse attention's
gradients (dq per query, dk/dv summed over every query and head that reads a
token), the indexer scores' gradients, and the compression's.

Tolerances: attention gradients to the attention tolerance (max-abs 2e-2,
rel-L2 1e-2): the kernel uses the bf16 forward output in D = d_out . out
(2^-9 relative) and float32 sums; indexer gradients are float32 sums of
products of small integers and float32 gradients over up to 10K blocks
(rel-L2 1e-5); the compression's gradient is a copy (bit for bit)."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import check_close, dev_bf16, dev_i32, host_f64_from_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_bits(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


LONG = [6001, 2100, 30002]
SHORT = [5, 7, 70, 1030]


# 8 query heads per KV head and fewer: one eight-head chunk per group; 20
# per KV head: a sixteen-head chunk and a partial one of four.  Short
# contexts: rows with no completed block before them (only their own block's
# 1 to 4 tokens), with fewer than 512 blocks, and a token list of one chunk.
@pytest.mark.parametrize("hq,hkv,lens", [(16, 2, LONG), (32, 4, LONG), (8, 8, LONG), (40, 2, LONG),
                                         (32, 4, SHORT)], ids=["16-2", "32-4", "8-8", "40-2",
                                                               "32-4-short"])
def test_sparse_attend_backward(hq, hkv, lens):
    w = W.make_custom(900 + hq, lens, 5, hq, hkv)
    say(f"attention backward: lens {list(w.lens)}, {hq}/{hkv} heads")
    shp = Q.shape(w.batch, w.max_len, w.n_query, hq, hkv)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], lens,
                               sel=sel, n_sel=n_sel)
    rng = np.random.default_rng(905)
    d_out_bits = bf16_bits(rng.standard_normal((w.batch, w.n_query, hq, 128)).astype(np.float32))
    # dq is written (what the buffer held does not count); dk and dv are added
    dq0 = torch.full((w.batch, w.n_query, hq, 128), 7.0, dtype=torch.float32, device="cuda")
    dq, dk, dv = Q.sparse_attend_backward(shp, t["q"], t["k"], t["v"], lens, sel, n_sel, out, lse,
                                          dev_bf16(d_out_bits), dq=dq0)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    res = O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, w.n_query)
    want_dk = np.zeros(dk.shape)
    want_dv = np.zeros(dv.shape)
    want_dq = np.zeros(dq.shape)
    for b in range(w.batch):
        kr, vr = O.bf16_bits_to_f64(w.k[b]), O.bf16_bits_to_f64(w.v[b])
        for i in range(w.n_query):
            tok = res["tok"][(b, i)]
            g_q, g_k, g_v = O.attend_backward(O.bf16_bits_to_f64(w.q[b, i]), kr[tok], vr[tok],
                                              O.bf16_bits_to_f64(d_out_bits[b, i]), w.scale)
            want_dq[b, i] = g_q
            np.add.at(want_dk[b], tok, g_k)
            np.add.at(want_dv[b], tok, g_v)
    check_close(dq, want_dq, "dq")
    check_close(dk, want_dk, "dk")
    check_close(dv, want_dv, "dv")
    # untouched rows stay exactly zero
    touched = np.zeros(dk.shape[:2], bool)
    for (b, i), tok in res["tok"].items():
        touched[b, tok] = True
    assert (dk[~touched] == 0).all() and (dv[~touched] == 0).all()


# 1 and 4 queries: one workgroup per block slice of a sequence (the dk_cmp rows
# read, added and written back); 6: the eight-query layout; 20: sixteen-query
# workgroups, two per slice (atomic adds to dk_cmp), the second one partial.
# Short contexts: rows with no candidate block, and slices cut short.
@pytest.mark.parametrize("n_query,lens", [(1, [9000, 40001]), (4, [9000, 40001]),
                                          (6, [9000, 40001]), (20, [9000, 40001]),
                                          (5, SHORT), (20, [24, 23, 300])],
                         ids=["1", "4", "6", "20", "5-short", "20-short"])
def test_index_scores_and_compress_backward(n_query, lens):
    w = W.make_custom(910, lens, n_query, 8, 1, parts=("index",))
    say(f"indexer backward: lens {list(w.lens)} n_query {n_query}")
    B, L, Nq = w.batch, w.max_len, w.n_query
    shp = Q.shape(B, L, Nq, 8, 1)
    lens = dev_i32(w.lens)
    k_cmp = torch.zeros((B, L // 4, 64), dtype=torch.bfloat16, device="cuda")
    Q.compress_keys(shp, dev_bf16(w.k_idx), lens, k_cmp)
    rng = np.random.default_rng(911)
    # float32 gradients with full mantissas (the dk_cmp sums split them into
    # three bf16 parts for the matrix cores)
    g = rng.standard_normal((B, Nq, L // 4)).astype(np.float32).astype(np.float64)
    # the gradients are added to what the buffers hold
    base_dq = rng.integers(-4, 5, (B, Nq, 4, 64)).astype(np.float32)
    base_dkc = rng.integers(-4, 5, (B, L // 4, 64)).astype(np.float32)
    dq_idx, dk_cmp = Q.index_scores_backward(shp, dev_bf16(w.q_idx), k_cmp, lens,
                                             torch.from_numpy(g.astype(np.float32)).cuda(),
                                             dq_idx=torch.from_numpy(base_dq).cuda(),
                                             dk_cmp=torch.from_numpy(base_dkc).cuda())
    dk_cmp -= torch.from_numpy(base_dkc).cuda()
    dk_idx = Q.compress_keys_backward(shp, lens, dk_cmp)
    torch.cuda.synchronize()
    dq_idx = dq_idx.cpu().numpy() - base_dq
    dk_cmp_h, dk_idx = dk_cmp.cpu().numpy(), dk_idx.cpu().numpy()
    want_dq = np.zeros(dq_idx.shape)
    want_dkc = np.zeros(dk_cmp_h.shape)
    for b in range(B):
        kc = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[b], int(w.lens[b])))
        for i in range(Nq):
            t = int(w.lens[b]) - Nq + i
            bt = t // 4
            dq_i, dkc_i = O.block_scores_backward(O.bf16_bits_to_f64(w.q_idx[b, i]), kc[:bt],
                                                  g[b, i, :bt])
            want_dq[b, i] = dq_i
            want_dkc[b, :bt] += dkc_i
    for got, want, what in ((dq_idx, want_dq, "dq_idx"), (dk_cmp_h, want_dkc, "dk_cmp")):
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.2e}"
    # the compression's gradient: each completed block's gradient on its four keys
    for b in range(B):
        nb = int(w.lens[b]) // 4
        want = O.compress_keys_backward(dk_cmp_h[b, :nb].astype(np.float64)).astype(np.float32)
        np.testing.assert_array_equal(dk_idx[b, :4 * nb], want)
        assert (dk_idx[b, 4 * nb:] == 0).all()
