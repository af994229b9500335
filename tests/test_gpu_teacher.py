"""The indexer's training target and what the selection keeps of it:
qsa_block_teacher (dense attention mass per micro-block, over the heads) and
qsa_teacher_recall against the float64 oracle, and needle survival at varied
depths.

Tolerance: every teacher entry is a sum of at most 4 x Hq terms
exp(z - lse) / Hq computed in float32 from bf16 inputs, with lse from a
float32 dense pass over up to 131K tokens; the relative error of one term is
a few float32 ulps of the logit (|z| ~ 10) plus the lse's error (~1e-6
relative), so each entry is within 1e-5 relative plus 1e-9 absolute of the
exact value, far inside the 1e-4 relative / 1e-7 absolute bound used here;
sums over a row (recall, total mass) within 1e-4."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import oracle as O
import workloads as W
from gpu_util import dev_bf16, dev_i32

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(w):
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    lens = dev_i32(w.lens)
    k_cmp = torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((w.batch, w.n_query, 512), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, w.n_query), dtype=torch.int32, device="cuda")
    _, lse_s, _, _ = Q.forward(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], lens,
                               sel=sel, n_sel=n_sel)
    _, lse_d = Q.dense_gqa_decode(shp, t["q"], t["k"], t["v"], lens)
    teacher = Q.block_teacher(shp, t["q"], t["k"], t["v"], lens)
    recall = Q.teacher_recall(shp, lens, teacher, sel, n_sel)
    torch.cuda.synchronize()
    return (teacher.cpu().numpy(), recall.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy(),
            lse_s.cpu().numpy(), lse_d.cpu().numpy())


@pytest.mark.parametrize("cfg", ["ragged", 1])
def test_teacher_and_recall_match_the_oracle(cfg):
    if cfg == "ragged":
        w = W.make_custom(800, [9001, 3000, 20002], 4, 16, 2)
    else:
        w = W.make(1)
    say(f"teacher: {w.name} lens {list(w.lens)}")
    teacher, recall, sel, n_sel, lse_s, lse_d = gpu_run(w)
    res = O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, w.n_query)
    for b in range(w.batch):
        kr = O.bf16_bits_to_f64(w.k[b])
        for i in range(w.n_query):
            t = int(w.lens[b]) - w.n_query + i
            T = O.block_teacher(O.bf16_bits_to_f64(w.q[b, i]), kr, t, w.scale)
            got = teacher[b, i]
            np.testing.assert_allclose(got[:T.shape[0]], T, rtol=1e-4, atol=1e-7,
                                       err_msg=f"row {(b, i)}")
            assert (got[T.shape[0]:] == 0).all()
            assert abs(got.sum() - 1.0) < 1e-4
            want_sel = res["sel"][(b, i)]
            np.testing.assert_array_equal(sel[b, i, :n_sel[b, i]], want_sel)
            want = O.selection_recall(T, want_sel)
            assert recall[b, i] == pytest.approx(want, abs=1e-4), (b, i)
            # the same share from the two log-sum-exps the GPU computed
            via_lse = float(np.mean(np.exp(lse_s[b, i].astype(np.float64) - lse_d[b, i])))
            assert recall[b, i] == pytest.approx(via_lse, abs=1e-4), (b, i)
            if t + 1 <= 2052:
                assert recall[b, i] == pytest.approx(1.0, abs=1e-4)


def test_needle_survival_at_varied_depths():
    # needle spans (indexer keys x4) near the start, in the middle and near
    # the end of a 60K context: the selection keeps them wherever they are
    L, nq = 60000, 8
    w = W.make_custom(801, [L], nq, 16, 2)
    starts = [256, 12800, 30016, 47104, L - nq - 2048]
    starts = [s // 64 * 64 for s in starts]
    W.plant_needles(w.k_idx, [starts])
    blocks = [j for s in starts for j in range(s // 4, s // 4 + 16)]
    say("needles at", starts)
    _, _, sel, n_sel, _, _ = gpu_run(w)
    res = O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, w.n_query)
    rates = []
    for i in range(nq):
        got = sel[0, i, :n_sel[0, i]]
        np.testing.assert_array_equal(got, res["sel"][(0, i)])
        r = O.needle_survival(got, blocks)
        per_depth = [O.needle_survival(got, range(s // 4, s // 4 + 16)) for s in starts]
        say(f"  query {i}: survival {r:.2f}, by depth {per_depth}")
        rates.append(per_depth)
    # x4 keys put a needle block's score at about four times a typical one:
    # most survive at every depth
    assert np.mean(rates) > 0.5
    assert min(np.mean(rates, axis=0)) > 0.3
