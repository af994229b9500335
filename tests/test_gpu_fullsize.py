"""Parity at the benchmark shapes, in the launch configuration bench.py times:
the 1M-context decode (every query row), the 256K and 1M last-chunk prefills
and the dense comparator (sampled rows the oracle computes one by one).
Selections bit for bit; outputs to max-abs <= 2e-2 and rel-L2 <= 1e-2."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import check_close, dev_bf16, dev_i32, host_f64_from_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_forward(w, first_block=None, prev_lens=None):
    """qsa_forward as bench.py calls it: the compressed-key cache already holds
    the previous step's blocks when prev_lens is given."""
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    k_idx = dev_bf16(w.k_idx)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    if prev_lens is not None:
        Q.compress_keys(shp, k_idx, dev_i32(prev_lens), k_cmp)
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, dev_bf16(w.q_idx), k_idx, k_cmp, dev_bf16(w.q),
                               dev_bf16(w.k), dev_bf16(w.v), dev_i32(w.lens),
                               first_block=None if first_block is None else dev_i32(first_block),
                               sel=sel, n_sel=n_sel)
    torch.cuda.synchronize()
    return (host_f64_from_bf16(out), lse.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy())


def compare_rows(w, got, rows):
    out, lse, sel, n_sel = got
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query, queries=rows)
    for b, i in rows:
        want = res["sel"][(b, i)]
        assert n_sel[b, i] == want.shape[0], (b, i)
        np.testing.assert_array_equal(sel[b, i, :want.shape[0]], want, err_msg=f"row {(b, i)}")
        assert (sel[b, i, want.shape[0]:] == -1).all()
        np.testing.assert_allclose(lse[b, i], res["lse"][(b, i)], atol=2e-2, rtol=0)
    check_close(np.stack([out[b, i] for b, i in rows]), np.stack([res["out"][r] for r in rows]))


def sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    nq = w.n_query
    picks = set(range(4)) | set(range(nq - 4, nq))
    picks |= set(int(x) for x in rng.choice(nq, size=n, replace=False))
    return [(0, i) for i in sorted(picks)]


def test_decode_1m_every_row():
    say("decode 1M: inputs")
    w = W.make(4)
    prev = (w.lens - w.n_query).astype(np.int32)
    first = (prev // 4).astype(np.int32)
    say("decode 1M: forward")
    got = run_forward(w, first_block=first, prev_lens=prev)
    say("decode 1M: oracle")
    compare_rows(w, got, [(b, i) for b in range(w.batch) for i in range(w.n_query)])


@pytest.mark.parametrize("cfg", [2, 3])
def test_prefill_chunk_sampled_rows(cfg):
    say(f"prefill cfg{cfg}: inputs")
    w = W.make(cfg)
    say(f"prefill cfg{cfg}: forward")
    got = run_forward(w)
    say(f"prefill cfg{cfg}: oracle")
    compare_rows(w, got, sample_rows(w, 40, 1000 + cfg))


def test_dense_decode_1m_sampled_rows():
    say("dense 1M: inputs")
    w = W.make(4)
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    say("dense 1M: kernel")
    out, lse = Q.dense_gqa_decode(shp, dev_bf16(w.q), dev_bf16(w.k), dev_bf16(w.v),
                                  dev_i32(w.lens))
    got = host_f64_from_bf16(out)
    rows = [(0, 0), (3, 3)]
    say("dense 1M: oracle")
    ref = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query, queries=rows)
    check_close(np.stack([got[b, i] for b, i in rows]), np.stack([ref[r][0] for r in rows]))
