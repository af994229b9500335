"""The debug build (lib/libqsa_debug.so, QSA_DEBUG): the kernels' guards on
caller-supplied values count what they catch.  Valid calls give the release
build's results bit for bit and no hits; a selection with ids outside
[0, bt) and counts above min(bt, 512), or a page table with ids outside the
pool, is clamped as in the release build (every access stays in its buffer)
and counted, in the forward kernels and in the attention backward."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import workloads as W
from gpu_util import dev_bf16, dev_i32, host_u16
from learned_sparse_attention_qsa_amd import build as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_forward(w):
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    out, lse, _, _ = Q.forward(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], lens,
                               sel=sel, n_sel=n_sel)
    torch.cuda.synchronize()
    return shp, t, lens, out, lse, sel, n_sel


@pytest.fixture
def debug_library():
    saved = Q._lib
    Q._lib = None
    Q.load_library(B.DEBUG_LIB)
    assert Q.debug_build()
    Q.debug_guard_hits()  # clear
    yield
    Q._lib = saved


def test_valid_calls_match_release_and_hit_nothing():
    w = W.make_custom(1700, [9001, 3002], 6, 16, 2)
    say("release forward", list(w.lens))
    _, _, _, out_r, lse_r, sel_r, _ = run_forward(w)
    saved = Q._lib
    Q._lib = None
    try:
        Q.load_library(B.DEBUG_LIB)
        assert Q.debug_build()
        Q.debug_guard_hits()
        say("debug forward")
        _, _, _, out_d, lse_d, sel_d, _ = run_forward(w)
        assert Q.debug_guard_hits() == 0
    finally:
        Q._lib = saved
    assert torch.equal(sel_r, sel_d)
    np.testing.assert_array_equal(host_u16(out_d), host_u16(out_r))
    np.testing.assert_array_equal(lse_d.cpu().numpy(), lse_r.cpu().numpy())


def test_out_of_range_selection_is_clamped_and_counted(debug_library):
    w = W.make_custom(1701, [9001, 3002], 6, 16, 2)
    shp, t, lens, _, _, sel, n_sel = run_forward(w)
    assert Q.debug_guard_hits() == 0
    bad = sel.clone()
    bad[0, 0, 3] = 1 << 20          # past the row's blocks
    bad[1, 2, 0] = -5               # negative
    bad_n = n_sel.clone()
    bad_n[1, 5] = 700               # more than 512
    say("attention over a corrupted selection")
    out, lse = Q.sparse_attend(shp, t["q"], t["k"], t["v"], lens, bad, bad_n)
    hits = Q.debug_guard_hits()
    assert hits >= 3, hits
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert Q.debug_guard_hits() == 0  # cleared by the read


def test_out_of_range_page_id_is_clamped_and_counted(debug_library):
    w = W.make_custom(1702, [5000], 2, 8, 1)
    B_, L = w.batch, w.max_len
    page = 64
    pages = (L + page - 1) // page
    table = np.arange(pages, dtype=np.int32).reshape(1, pages)
    table[0, 3] = pages + 10        # outside the pool of `pages` pages
    kp = np.zeros((pages, page, 1, 128), dtype=np.uint16)
    vp = np.zeros_like(kp)
    kp.reshape(-1, 1, 128)[:L] = w.k[0]
    vp.reshape(-1, 1, 128)[:L] = w.v[0]
    pg = Q.PagedKV(dev_i32(table), page, pages)
    shp = Q.shape(1, L, 2, 8, 1)
    say("dense decode through a table with a stray page id")
    out, _ = Q.dense_gqa_decode_paged(shp, dev_bf16(w.q), dev_bf16(kp), dev_bf16(vp), pg,
                                      dev_i32(w.lens))
    assert Q.debug_guard_hits() > 0
    assert torch.isfinite(out.float()).all()


def test_backward_over_out_of_range_selection_is_clamped_and_counted(debug_library):
    w = W.make_custom(1703, [9001, 3002], 6, 16, 2)
    shp, t, lens, out, lse, sel, n_sel = run_forward(w)
    assert Q.debug_guard_hits() == 0
    bad = sel.clone()
    bad[0, 0, 3] = 1 << 20          # past the row's blocks
    bad[1, 2, 0] = -5               # negative
    bad_n = n_sel.clone()
    bad_n[1, 5] = 700               # more than 512
    g = torch.Generator(device="cuda")
    g.manual_seed(1703)
    d_out = torch.randn(out.shape, generator=g, device="cuda").to(torch.bfloat16)
    say("attention backward over a corrupted selection")
    dq, dk, dv = Q.sparse_attend_backward(shp, t["q"], t["k"], t["v"], lens, bad, bad_n, out,
                                          lse, d_out)
    hits = Q.debug_guard_hits()
    assert hits >= 3, hits
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
