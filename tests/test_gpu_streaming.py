"""Whole-sequence streaming: a prompt prefilled chunk by chunk (the last chunk
ragged), then decode steps of four tokens whose rows are appended to the
caches, each call compressing only the micro-blocks it completes.  Every
chunk's and every step's selections are compared bit for bit with the
oracle, sampled outputs to the attention tolerance, and the compressed-key
cache after the last step bit for bit."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import check_close, dev_bf16, host_f64_from_bf16, host_u16
from learned_sparse_attention_qsa_amd import streaming as S

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_rows(w, length, lo, hi, out, lse, sel, n_sel, sample):
    """Queries at positions lo .. hi-1 of a sequence of `length` tokens."""
    nq = hi - lo
    q_idx = w.q_idx[:, lo:hi]
    rows = [(0, i) for i in range(nq)]
    ref = O.select_rows(q_idx, w.k_idx, np.array([length]), nq, rows, threads=8)
    sel_h = sel.cpu().numpy()[0]
    nsel_h = n_sel.cpu().numpy()[0]
    for _, i in rows:
        want, nw = ref[(0, i)]
        assert nsel_h[i] == nw, (lo, i)
        np.testing.assert_array_equal(sel_h[i, :nw], want, err_msg=f"position {lo + i}")
        assert (sel_h[i, nw:] == -1).all()
    qs = [(0, i) for i in sample]
    res = O.qsa_forward(q_idx, w.k_idx, w.q[:, lo:hi], w.k, w.v, np.array([length]), nq,
                        queries=qs)
    got = host_f64_from_bf16(out)[0]
    check_close(np.stack([got[i] for i in sample]), np.stack([res["out"][r] for r in qs]))
    if lse is not None:
        lse_h = lse.cpu().numpy()[0]
        for i in sample:
            np.testing.assert_allclose(lse_h[i], res["lse"][(0, i)], atol=2e-2, rtol=0)


@pytest.mark.parametrize("flags", [0, Q.FLAG_TOPK_SCAN])
def test_chunked_prefill_then_decode_steps(flags):
    prompt, chunk, steps, m = 18001, 4096, 6, 4
    total = prompt + steps * m
    cap = (total + 3) // 4 * 4
    w = W.make_custom(600, [total], total, 16, 2, max_len=cap)
    seq = S.Sequence(cap, 16, 2, flags=flags)
    dev = {n: dev_bf16(getattr(w, n))[0] for n in ("q_idx", "k_idx", "q", "k", "v")}
    rng = np.random.default_rng(601)
    results = []

    def on_chunk(c, lo, hi, o, lse, sel, n_sel):
        results.append((lo, hi, o.clone(), lse.clone(), sel.clone(), n_sel.clone()))

    say(f"prefill {prompt} tokens in chunks of {chunk}")
    S.prefill(seq, dev["q_idx"][:prompt], dev["k_idx"][:prompt], dev["q"][:prompt],
              dev["k"][:prompt], dev["v"][:prompt], chunk, on_chunk=on_chunk)
    torch.cuda.synchronize()
    assert seq.length == prompt
    for lo, hi, o, lse, sel, n_sel in results:
        say(f"  chunk [{lo}, {hi})")
        sample = sorted(set([0, hi - lo - 1]) | set(rng.choice(hi - lo, 6, replace=False).tolist()))
        check_rows(w, hi, lo, hi, o, lse, sel, n_sel, sample)
    for s in range(steps):
        lo = prompt + s * m
        say(f"decode step {s}: positions [{lo}, {lo + m})")
        o, lse, sel, n_sel = S.decode_step(seq, dev["q_idx"][lo:lo + m], dev["k_idx"][lo:lo + m],
                                           dev["q"][lo:lo + m], dev["k"][lo:lo + m],
                                           dev["v"][lo:lo + m],
                                           sel=torch.empty((1, m, 512), dtype=torch.int32,
                                                           device="cuda"),
                                           n_sel=torch.empty((1, m), dtype=torch.int32,
                                                             device="cuda"))
        torch.cuda.synchronize()
        check_rows(w, lo + m, lo, lo + m, o, lse, sel, n_sel, list(range(m)))
    # the compressed-key cache holds every completed block, as one full compression gives
    want = O.compress_keys(w.k_idx[0], total)
    got = host_u16(seq.k_cmp)[0]
    np.testing.assert_array_equal(got[:want.shape[0]], want)
