"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values printed on the pages, a hand-worked example, closed forms, brute force,
invariants and library routines.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def bf16(vals):
    """Exact bf16 bit patterns of small integers / simple floats (test input helper)."""
    f = np.asarray(vals, dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- fixtures

def test_page_constants(golden_dir):
    with open(os.path.join(golden_dir, "page_constants.json")) as f:
        c = json.load(f)
    assert O.IDX_HEADS == c["index_query_heads"]["value"]
    assert c["shared_key_heads"]["value"] == 1
    assert O.BLOCK == c["block_tokens"]["value"]
    assert O.TOPK == c["max_blocks"]["value"]
    assert O.TOPK * O.BLOCK == c["token_budget"]["value"]
    # the decode shape of the speed experiment: batch 4, 1 + 3 query positions
    assert W.CONFIGS[4]["n_query"] == c["decode_queries_per_sequence"]["value"]
    assert len(W.CONFIGS[4]["lens"]) == c["decode_batch"]["value"]
    assert len(W.CONFIGS[3]["lens"]) == c["prefill_batch"]["value"]


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        ex = json.load(f)
    k_idx = bf16(ex["k_idx"])
    t = ex["t"]
    kc = O.compress_keys(k_idx, t + 1)
    assert kc.shape == (4, 2)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(kc), np.array(ex["compressed"], float))
    s = O.block_scores(np.array(ex["q_idx"], float), O.bf16_bits_to_f64(kc))
    np.testing.assert_array_equal(s, ex["scores"])
    sel = O.select_blocks(s, ex["k"])
    np.testing.assert_array_equal(sel, ex["sel"])
    tok = O.expand_tokens(sel, t)
    np.testing.assert_array_equal(tok, ex["tok"])


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_closed_forms():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,          # halfway, ties to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,      # halfway, ties to even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above halfway
        -2.5: 0xC020,
        2.0 ** -133: 0x0001,              # smallest subnormal
        2.5 * 2.0 ** -133: 0x0002,        # subnormal tie to even
        3.5e38: 0x7F80,                   # above the largest bf16: inf
        0.0: 0x0000,
        256.0: 0x4380,
        257.0: 0x4380,                    # 257 is halfway between 256 and 258: even
        259.0: 0x4382,
    }
    got = O.f64_to_bf16_bits(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())


def test_bf16_rounding_matches_torch_on_float32_inputs():
    # For float32-representable inputs the definition reduces to torch's
    # float32 -> bfloat16 conversion (round to nearest, ties to even).
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-130, 120, x.shape[0]).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_decode_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(vals)
    back = O.f64_to_bf16_bits(vals[fin])
    # +0/-0 and every finite pattern map back to themselves
    np.testing.assert_array_equal(back, bits[fin])


# ---------------------------------------------------------------- compress

def test_compress_checksum_and_blocks():
    w = W.make_custom(11, [1003], 5, 8, 1, parts=("index",))
    n = int(w.lens[0])
    kc = O.compress_keys(w.k_idx[0], n)
    assert kc.shape == (n // 4, 64)
    vals = O.bf16_bits_to_f64(w.k_idx[0])
    # invariant: total of compressed keys = total of keys of completed blocks
    np.testing.assert_array_equal(O.bf16_bits_to_f64(kc).sum(0), vals[:4 * (n // 4)].sum(0))
    # block-by-block with plain Python ints
    for j in (0, 17, n // 4 - 1):
        rows = [[int(v) for v in vals[4 * j + r]] for r in range(4)]
        want = [sum(col) for col in zip(*rows)]
        assert [int(x) for x in O.bf16_bits_to_f64(kc[j])] == want


def test_compress_first_block_and_rounding():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((64, 64)).astype(np.float32)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    full = O.compress_keys(kb, 64)
    part = O.compress_keys(kb, 64, first_block=5)
    np.testing.assert_array_equal(full[5:], part)
    # non-integer inputs: one rounding of the exact sum (check with Fractions)
    from fractions import Fraction
    vals = O.bf16_bits_to_f64(kb)
    for j in range(16):
        for d in range(0, 64, 9):
            exact = sum(Fraction(vals[4 * j + r, d]) for r in range(4))
            got = Fraction(O.bf16_bits_to_f64(full[j:j + 1, d:d + 1])[0, 0])
            # nearest bf16: no other bf16 value is strictly closer
            f = float(got)
            m, e = math.frexp(f) if f != 0 else (0.0, -200)
            ulp = Fraction(2) ** (max(e - 8, -133)) if f != 0 else Fraction(2) ** -133
            assert abs(got - exact) <= ulp / 2


def test_compress_ignores_partial_block():
    kb = bf16(np.ones((7, 3)))
    kc = O.compress_keys(kb, 7)
    assert kc.shape == (1, 3)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(kc), [[4, 4, 4]])


# ---------------------------------------------------------------- scores

def test_scores_brute_force_python_ints():
    rng = np.random.default_rng(5)
    q = rng.integers(-8, 9, (4, 64))
    kc = rng.integers(-32, 33, (37, 64))
    s = O.block_scores(q.astype(float), kc.astype(float))
    for j in range(37):
        want = 0
        for h in range(4):
            dot = 0
            for d in range(64):
                dot += int(q[h, d]) * int(kc[j, d])
            want += max(0, dot)
        assert s[j] == want


def test_scores_l1_closed_form():
    # heads +e_a, +e_b, -e_a, -e_b turn the score into |kc_a| + |kc_b|
    rng = np.random.default_rng(9)
    kc = rng.integers(-100, 101, (200, 64)).astype(float)
    a, b = 3, 41
    q = np.zeros((4, 64))
    q[0, a] = 1
    q[1, b] = 1
    q[2, a] = -1
    q[3, b] = -1
    np.testing.assert_array_equal(O.block_scores(q, kc), np.abs(kc[:, a]) + np.abs(kc[:, b]))


def test_scores_relu_per_head_not_after_sum():
    # two heads with opposite dots: per-head ReLU keeps the positive one
    q = np.zeros((4, 2))
    q[0] = [1, 0]
    q[1] = [-1, 0]
    kc = np.array([[5.0, 0.0]])
    assert O.block_scores(q, kc)[0] == 5.0


# ---------------------------------------------------------------- select

def brute_topk(s, k):
    if s.shape[0] <= k:
        return np.arange(s.shape[0])
    order = np.lexsort((np.arange(s.shape[0]), -s))  # score desc, index asc
    return np.sort(order[:k])


def test_select_vs_full_sort_tie_heavy():
    rng = np.random.default_rng(21)
    for trial in range(3000):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 40))
        levels = int(rng.integers(1, 5))
        s = rng.integers(0, levels, n).astype(float)
        np.testing.assert_array_equal(O.select_blocks(s, k), brute_topk(s, k))


def test_select_vs_full_sort_k512():
    rng = np.random.default_rng(22)
    for trial in range(60):
        n = int(rng.integers(400, 2000))
        s = rng.integers(0, int(rng.integers(2, 3000)), n).astype(float)
        np.testing.assert_array_equal(O.select_blocks(s, 512), brute_topk(s, 512))


def test_select_special_cases():
    z = np.zeros(5000)
    np.testing.assert_array_equal(O.select_blocks(z), np.arange(512))
    c = np.full(3000, 7.0)
    np.testing.assert_array_equal(O.select_blocks(c), np.arange(512))
    small = np.arange(100, 0, -1).astype(float)
    np.testing.assert_array_equal(O.select_blocks(small), np.arange(100))
    rng = np.random.default_rng(4)
    s = rng.integers(0, 50, 10000).astype(float)
    s[7777] = 1000
    assert 7777 in O.select_blocks(s)
    # exactly 512 candidates: all kept; 513: one dropped (the lowest, last index on ties)
    np.testing.assert_array_equal(O.select_blocks(np.ones(512)), np.arange(512))
    np.testing.assert_array_equal(O.select_blocks(np.ones(513)), np.arange(512))


def test_select_invariant_under_key_scaling():
    # multiplying every indexer key by 4 scales all scores by 4: same selection
    w = W.make_custom(12, [6000], 3, 8, 1, parts=("index",))
    kc1 = O.bf16_bits_to_f64(O.compress_keys(w.k_idx[0], 6000))
    q = O.bf16_bits_to_f64(w.q_idx[0, 0])
    s1 = O.block_scores(q, kc1)
    s4 = O.block_scores(q, 4 * kc1)
    np.testing.assert_array_equal(s4, 4 * s1)
    np.testing.assert_array_equal(O.select_blocks(s1), O.select_blocks(s4))


# ---------------------------------------------------------------- row-batched scoring and selection

def test_scores_rows_brute_force_python_ints():
    rng = np.random.default_rng(15)
    q = rng.integers(-8, 9, (5, 4, 64))
    kc = rng.integers(-32, 33, (23, 64))
    s = O.block_scores_rows(q.astype(float), kc.astype(float))
    assert s.shape == (5, 23)
    for i in range(5):
        for j in range(23):
            want = 0
            for h in range(4):
                want += max(0, sum(int(q[i, h, d]) * int(kc[j, d]) for d in range(64)))
            assert s[i, j] == want


def test_select_rows_vs_full_sort_ragged_candidates():
    # every row has its own candidate count bt; columns at or past bt are ignored
    rng = np.random.default_rng(31)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        m = int(rng.integers(1, 400))
        k = int(rng.integers(1, 50))
        levels = int(rng.integers(1, 6))
        s = rng.integers(0, levels, (n, m)).astype(float)
        bt = rng.integers(0, m + 1, n)
        bt[0] = m
        sel, n_sel = O.select_blocks_rows(s, bt, k)
        for i in range(n):
            want = brute_topk(s[i, :bt[i]], k)
            assert n_sel[i] == want.shape[0]
            np.testing.assert_array_equal(sel[i, :n_sel[i]], want)
            assert (sel[i, n_sel[i]:] == -1).all()


def test_select_rows_k512_matches_per_row_select():
    rng = np.random.default_rng(32)
    s = rng.integers(0, 40, (6, 3000)).astype(float)
    bt = np.array([3000, 2999, 513, 512, 100, 2048])
    sel, n_sel = O.select_blocks_rows(s, bt, 512)
    for i in range(6):
        want = brute_topk(s[i, :bt[i]], 512)
        np.testing.assert_array_equal(sel[i, :n_sel[i]], want)


def test_select_rows_end_to_end_matches_single_query_path():
    # the batched path through select_rows gives the per-query oracle's selections
    w = W.make_custom(14, [5000, 3100], 37, 8, 1, parts=("index",))
    rows = [(b, i) for b in range(2) for i in range(37)]
    got = O.select_rows(w.q_idx, w.k_idx, w.lens, w.n_query, rows, chunk=16, threads=2)
    ref = O.qsa_forward(w.q_idx, w.k_idx, None, None, None, w.lens, w.n_query)
    for r in rows:
        np.testing.assert_array_equal(got[r][0], ref["sel"][r])
        assert got[r][1] == ref["sel"][r].shape[0]


# ---------------------------------------------------------------- tail / expand

@pytest.mark.parametrize("n", [4093, 4094, 4095, 4096, 1, 2, 3, 4, 5])
def test_tail_by_length_mod4(n):
    t = n - 1
    bt = t // 4
    rng = np.random.default_rng(n)
    s = rng.integers(0, 100, bt).astype(float)
    sel = O.select_blocks(s)
    tok = O.expand_tokens(sel, t)
    tail = t - 4 * bt + 1
    assert tail == (n - 1) % 4 + 1
    assert tok.shape[0] == 4 * min(512, bt) + tail
    assert tok[-1] == t and tok.max() == t
    np.testing.assert_array_equal(tok[-tail:], np.arange(4 * bt, t + 1))
    assert np.all(np.diff(tok) > 0)
    assert tok.shape[0] <= O.TOPK * O.BLOCK + O.BLOCK


# ---------------------------------------------------------------- attention

def sdpa_ref(q, k, v, scale, causal_pos=None):
    """torch's SDPA (float64, CPU) as the textbook routine: q [Hq][D], k/v [n][Hkv][D]."""
    hq, hkv = q.shape[0], k.shape[1]
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    qq = torch.from_numpy(q)[:, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return out[:, 0, :].numpy()


def test_attend_matches_sdpa():
    rng = np.random.default_rng(31)
    for hq, hkv, n in [(8, 1, 37), (32, 4, 300), (4, 4, 1), (6, 2, 9)]:
        q = rng.standard_normal((hq, 128))
        k = rng.standard_normal((n, hkv, 128))
        v = rng.standard_normal((n, hkv, 128))
        o, lse = O.attend(q, k, v, 0.088)
        np.testing.assert_allclose(o, sdpa_ref(q, k, v, 0.088), rtol=1e-12, atol=1e-12)
        # lse against its closed form for head 0
        z = 0.088 * (k[:, 0, :] @ q[0])
        assert abs(lse[0] - math.log(np.exp(z).sum())) < 1e-10


def test_attend_special_cases():
    rng = np.random.default_rng(32)
    q = rng.standard_normal((8, 128))
    v = rng.standard_normal((20, 2, 128))
    o, lse = O.attend(q, np.zeros((20, 2, 128)), v, 0.1)
    np.testing.assert_allclose(o[:4], np.broadcast_to(v[:, 0].mean(0), (4, 128)), atol=1e-14)
    np.testing.assert_allclose(o[4:], np.broadcast_to(v[:, 1].mean(0), (4, 128)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(20), atol=1e-14)
    k = rng.standard_normal((20, 2, 128))
    o, _ = O.attend(q, k, np.full((20, 2, 128), 3.25), 0.1)
    np.testing.assert_allclose(o, 3.25, atol=1e-13)
    k = np.zeros((20, 2, 128))
    k[13, :, :] = 50 * q[0] / np.linalg.norm(q[0])
    o, _ = O.attend(q[:1], k[:, :1], v[:, :1], 1.0)
    np.testing.assert_allclose(o[0], v[13, 0], atol=1e-12)


def test_qsa_equals_dense_for_short_context():
    # every context of at most 2,052 tokens keeps all its blocks: QSA == dense causal
    w = W.make_custom(41, [2052, 1500, 7], 6, 16, 2)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, 6)
    dense = O.dense_decode(w.q, w.k, w.v, w.lens, 6)
    for key, (o, lse) in dense.items():
        b, i = key
        t = int(w.lens[b]) - 6 + i
        if t < 0:
            continue
        np.testing.assert_array_equal(res["tok"][key], np.arange(t + 1))
        np.testing.assert_allclose(res["out"][key], o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(res["lse"][key], lse, rtol=0, atol=1e-12)
    # and the dense oracle against torch's causal SDPA
    b, i = 0, 5
    t = int(w.lens[b]) - 6 + i
    q = O.bf16_bits_to_f64(w.q[b, i])
    k = O.bf16_bits_to_f64(w.k[b, :t + 1])
    v = O.bf16_bits_to_f64(w.v[b, :t + 1])
    np.testing.assert_allclose(dense[(b, i)][0], sdpa_ref(q, k, v, 1 / math.sqrt(128)),
                               rtol=1e-12, atol=1e-12)


def test_qsa_differs_from_dense_beyond_2052():
    w = W.make_custom(42, [2053], 1, 8, 1)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, 1)
    tok = res["tok"][(0, 0)]
    assert tok.shape[0] == 2049  # 512 blocks + a one-token tail (t = 2052)
    assert 2052 in tok


# ---------------------------------------------------------------- teacher, recall, survival

def test_teacher_brute_force_and_mass():
    rng = np.random.default_rng(70)
    hq, hkv, t = 4, 2, 13
    q = rng.standard_normal((hq, 8))
    k = rng.standard_normal((t + 1, hkv, 8))
    scale = 0.3
    T = O.block_teacher(q, k, t, scale)
    assert T.shape == (t // 4 + 1,)
    want = np.zeros(t // 4 + 1)
    for h in range(hq):
        logits = [scale * sum(q[h, d] * k[s, h // 2, d] for d in range(8)) for s in range(t + 1)]
        mx = max(logits)
        e = [math.exp(x - mx) for x in logits]
        for s in range(t + 1):
            want[s // 4] += e[s] / sum(e) / hq
    np.testing.assert_allclose(T, want, rtol=1e-12, atol=1e-15)
    assert abs(T.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("t", [4095, 4096, 4097, 4098])
def test_teacher_uniform_keys(t):
    # K = 0: every position equally likely, so a block holds 4/(t+1) and the
    # query's own block (t mod 4) + 1 of t + 1
    q = np.random.default_rng(t).standard_normal((8, 16))
    k = np.zeros((t + 1, 1, 16))
    T = O.block_teacher(q, k, t, 0.1)
    np.testing.assert_allclose(T[:-1], 4.0 / (t + 1), rtol=1e-12)
    assert T[-1] == pytest.approx((t % 4 + 1) / (t + 1), rel=1e-12)


def test_recall_is_the_lse_gap_and_one_for_short_contexts():
    # the teacher mass on the attended tokens, per head, is exp(lse_sparse -
    # lse_dense): the attention oracle's two log-sum-exps give it independently
    w = W.make_custom(71, [3000], 3, 8, 2)
    res = O.qsa_forward(w.q_idx, w.k_idx, w.q, w.k, w.v, w.lens, w.n_query)
    dense = O.dense_decode(w.q, w.k, w.v, w.lens, w.n_query)
    kr = O.bf16_bits_to_f64(w.k[0])
    for i in range(3):
        t = 3000 - 3 + i
        qi = O.bf16_bits_to_f64(w.q[0, i])
        T = O.block_teacher(qi, kr, t, w.scale)
        rec = O.selection_recall(T, res["sel"][(0, i)])
        via_lse = float(np.mean(np.exp(res["lse"][(0, i)] - dense[(0, i)][1])))
        assert 0.0 < rec < 1.0
        assert rec == pytest.approx(via_lse, rel=1e-9)
    short = W.make_custom(72, [2052], 2, 8, 1)
    r2 = O.qsa_forward(short.q_idx, short.k_idx, short.q, short.k, short.v, short.lens, 2)
    for i in range(2):
        t = 2050 + i
        T = O.block_teacher(O.bf16_bits_to_f64(short.q[0, i]), O.bf16_bits_to_f64(short.k[0]), t,
                            short.scale)
        assert O.selection_recall(T, r2["sel"][(0, i)]) == pytest.approx(1.0, abs=1e-12)


def test_needle_survival_counts_kept_planted_blocks():
    sel = np.array([3, 5, 9, 40, 41])
    assert O.needle_survival(sel, [40, 41, 42, 43]) == 0.5
    assert O.needle_survival(sel, []) == 1.0
    assert O.needle_survival(sel, [5]) == 1.0


# ---------------------------------------------------------------- gradients

def _fd(f, x, eps=1e-6):
    """Central finite differences of a scalar function of an array."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        g[i] = (f(xp) - f(xm)) / (2 * eps)
    return g


def test_attend_backward_finite_differences():
    rng = np.random.default_rng(80)
    hq, hkv, n, d = 4, 2, 7, 6
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((hq, d))
    scale = 0.7
    dq, dk, dv = O.attend_backward(q, k, v, do, scale)
    loss = lambda qq, kk, vv: float(np.sum(O.attend(qq, kk, vv, scale)[0] * do))
    np.testing.assert_allclose(dq, _fd(lambda x: loss(x, k, v), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, _fd(lambda x: loss(q, x, v), k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, _fd(lambda x: loss(q, k, x), v), rtol=1e-6, atol=1e-8)


def test_attend_backward_matches_torch_autograd():
    rng = np.random.default_rng(81)
    hq, hkv, n, d = 8, 2, 40, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((n, hkv, d))
    v = rng.standard_normal((n, hkv, d))
    do = rng.standard_normal((hq, d))
    scale = 0.25
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)   # [hq][n][d]
    vv = tv.repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    p = torch.softmax(scale * torch.einsum("hd,hnd->hn", tq, kk), dim=-1)
    o = torch.einsum("hn,hnd->hd", p, vv)
    o.backward(torch.tensor(do))
    dq, dk, dv = O.attend_backward(q, k, v, do, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_block_scores_backward_finite_differences():
    rng = np.random.default_rng(82)
    q = rng.standard_normal((4, 8))
    kc = rng.standard_normal((11, 8))
    g = rng.standard_normal(11)
    dq, dkc = O.block_scores_backward(q, kc, g)
    loss = lambda qq, kk: float(np.dot(O.block_scores(qq, kk), g))
    np.testing.assert_allclose(dq, _fd(lambda x: loss(x, kc), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dkc, _fd(lambda x: loss(q, x), kc), rtol=1e-6, atol=1e-8)


def test_compress_backward_is_the_sum_adjoint():
    # <compress(k), a> = <k, compress_backward(a)> for any k, a (exact sums)
    rng = np.random.default_rng(83)
    k = rng.integers(-8, 9, (40, 64)).astype(np.float64)
    a = rng.standard_normal((10, 64))
    kc = O.bf16_bits_to_f64(O.compress_keys(bf16(k), 40))
    assert np.sum(kc * a) == pytest.approx(np.sum(k * O.compress_keys_backward(a)), rel=1e-12)
