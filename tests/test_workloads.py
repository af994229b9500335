"""The seeded input generators: determinism, value ranges, needle structure."""
import numpy as np

import oracle as O
import workloads as W


def test_same_seed_same_bytes_any_thread_count():
    a = W.make_custom(5, [20000, 9000], 7, 16, 2, needles=0, threads=1)
    b = W.make_custom(5, [20000, 9000], 7, 16, 2, needles=0, threads=4)
    for name in ("q_idx", "k_idx", "q", "k", "v"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = W.make_custom(6, [20000, 9000], 7, 16, 2)
    assert not np.array_equal(a.k_idx, c.k_idx)


def test_chunked_generation_crosses_chunks():
    n = W.CHUNK + 1000
    x = W.gen_tensor(3, 1, (n,), "int", threads=3)
    y = W.gen_tensor(3, 1, (n,), "int", threads=1)
    assert np.array_equal(x, y)


def test_value_ranges():
    w = W.make_custom(8, [5000], 16, 8, 1)
    qi = O.bf16_bits_to_f64(w.q_idx)
    ki = O.bf16_bits_to_f64(w.k_idx)
    for arr in (qi, ki):
        assert arr.min() == -8 and arr.max() == 8
        assert np.all(arr == np.round(arr))
    # all 17 integer values appear, roughly uniformly
    counts = np.bincount((ki.astype(int) + 8).ravel(), minlength=17)
    assert counts.min() > 0.8 * counts.mean()
    q = O.bf16_bits_to_f64(w.q)
    assert abs(q.mean()) < 0.05 and abs(q.std() - 1) < 0.05


def test_needles():
    w = W.make_custom(2, [40000], 4, 8, 1, needles=8, parts=("index",))
    starts = w.needle_starts[0]
    assert len(starts) == 8 and len(set(starts)) == 8
    assert all(s % 64 == 0 and s + 64 <= 40000 - 16384 for s in starts)
    plain = W.make_custom(2, [40000], 4, 8, 1, needles=0, parts=("index",))
    ki, kp = O.bf16_bits_to_f64(w.k_idx[0]), O.bf16_bits_to_f64(plain.k_idx[0])
    mask = np.zeros(40000, bool)
    for s in starts:
        mask[s:s + 64] = True
    assert np.array_equal(ki[mask], 4 * kp[mask])
    assert np.array_equal(ki[~mask], kp[~mask])


def test_config_shapes():
    c = W.CONFIGS
    assert c[3]["lens"] == [1 << 20] and c[3]["n_query"] == 16384
    assert c[4]["lens"] == [1048576, 1048575, 1048574, 1048573]
    assert [l % 4 for l in c[1]["lens"]] == [0, 3, 2, 1]
    w = W.make(0)
    assert w.q_idx.shape == (1, 64, 4, 64) and w.k.shape == (1, 4096, 1, 128)
    t = int(w.lens[0]) - w.n_query + np.arange(w.n_query)
    assert sorted(np.bincount((t % 4).astype(int))) == [16, 16, 16, 16]
