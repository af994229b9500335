"""Seeded synthetic inputs for the QSA hot path.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no compression, scoring, selection or attention), so
both the CPU oracle and the GPU path can be fed from it without sharing any
of the computation they are checked on.

Every array is generated in fixed-size chunks; chunk ``c`` of tensor ``t`` of
workload ``w`` draws from ``numpy.random.default_rng([w, t, c])`` (PCG64), so
the bytes are identical however many threads produce them.

Shapes and value distributions follow the speed experiment described on
"Qwen's million-token window has a 2,048-token keyhole" (section "Three speed
claims, three different experiments"): a 1M-token context, a last-chunk
prefill at batch one, and a batch-four decode with three extra
multi-token-prediction steps (four query positions per sequence).  The
indexer layout (four query heads, one shared key head) and the four-token
micro-blocks come from the section "A million-token window with a selective
view" of the same page.

Layouts (all row-major, bf16 carried as uint16 bit patterns):
  q_idx  [B][Nq][4][64]      indexer queries
  k_idx  [B][Lmax][64]       indexer keys (one shared head)
  q      [B][Nq][Hq][128]    core-attention queries
  k, v   [B][Lmax][Hkv][128] core-attention key/value cache (token-major)
  lens   [B] int32           tokens in each sequence, query tokens included

Query i of sequence b sits at position t = lens[b] - Nq + i.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

IDX_HEADS = 4
IDX_DIM = 64
HEAD_DIM = 128

CHUNK = 1 << 22  # elements per generator chunk

# tensor ids used in the seed tuple
T_Q_IDX, T_K_IDX, T_Q, T_K, T_V, T_NEEDLE = 0, 1, 2, 3, 4, 5

# The five benchmark shapes.  "needles": number of 64-token spans per
# sequence whose indexer keys are multiplied by four.
CONFIGS = {
    0: dict(name="tiny-4k", lens=[4096], n_query=64, q_heads=8, kv_heads=1, needles=0),
    1: dict(name="decode-128k-b4x4", lens=[131072, 131071, 131070, 131069], n_query=4,
            q_heads=32, kv_heads=4, needles=0),
    2: dict(name="prefill-256k-chunk16k", lens=[262144], n_query=16384, q_heads=32,
            kv_heads=4, needles=8),
    3: dict(name="prefill-1m-chunk16k", lens=[1048576], n_query=16384, q_heads=32,
            kv_heads=4, needles=8),
    4: dict(name="decode-1m-b4x4", lens=[1048576, 1048575, 1048574, 1048573], n_query=4,
            q_heads=32, kv_heads=4, needles=0),
}

NEEDLE_TOKENS = 64      # tokens per planted span (16 micro-blocks)
NEEDLE_GAIN = 4         # indexer-key multiplier inside a span
NEEDLE_GUARD = 16384    # spans lie before the last 16,384 positions


@dataclass
class Workload:
    name: str
    lens: np.ndarray            # int32 [B]
    max_len: int
    n_query: int
    q_heads: int
    kv_heads: int
    q_idx: np.ndarray | None = None   # uint16 [B][Nq][4][64]
    k_idx: np.ndarray | None = None   # uint16 [B][Lmax][64]
    q: np.ndarray | None = None       # uint16 [B][Nq][Hq][128]
    k: np.ndarray | None = None       # uint16 [B][Lmax][Hkv][128]
    v: np.ndarray | None = None       # uint16 [B][Lmax][Hkv][128]
    needle_starts: list = field(default_factory=list)  # per sequence, token offsets

    @property
    def batch(self) -> int:
        return int(self.lens.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / np.sqrt(HEAD_DIM)


def _threads(threads: int | None) -> int:
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); returns uint16 bits."""
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _small_int_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Small integers are exact in bf16: the float32 bit pattern's top half."""
    return (x.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _fill(out_flat: np.ndarray, seed_head: tuple, kind: str, threads: int) -> None:
    n = out_flat.shape[0]
    n_chunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng(list(seed_head) + [c])
        if kind == "int":
            vals = rng.integers(-8, 9, hi - lo, dtype=np.int8)
            out_flat[lo:hi] = _small_int_to_bf16_bits(vals)
        else:
            vals = rng.standard_normal(hi - lo, dtype=np.float32)
            out_flat[lo:hi] = _f32_to_bf16_bits(vals)

    if n_chunks <= 1 or threads <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(n_chunks)))


def gen_tensor(seed_id: int, tensor_id: int, shape: tuple, kind: str,
               threads: int | None = None) -> np.ndarray:
    """Seeded uint16 bf16-bit tensor: kind "int" = uniform integers in [-8, 8],
    kind "normal" = N(0, 1) rounded to bf16."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    _fill(out, (seed_id, tensor_id), kind, _threads(threads))
    return out.reshape(shape)


def needle_starts_for(seed_id: int, length: int, n_spans: int, b: int) -> list:
    """Token offsets of the planted spans of sequence b: 64-aligned, disjoint,
    all before the last NEEDLE_GUARD positions (so every chunk query sees them)."""
    if n_spans == 0:
        return []
    slots = max(0, (length - NEEDLE_GUARD)) // NEEDLE_TOKENS
    if slots < n_spans:
        raise ValueError("sequence too short for its needle spans")
    rng = np.random.default_rng([seed_id, T_NEEDLE, b])
    picks = rng.choice(slots, size=n_spans, replace=False)
    return sorted(int(p) * NEEDLE_TOKENS for p in picks)


def plant_needles(k_idx: np.ndarray, starts_per_seq: list) -> None:
    """Multiply the indexer keys of every planted span by NEEDLE_GAIN, in place.
    Values stay small integers, so the bf16 patterns remain exact."""
    for b, starts in enumerate(starts_per_seq):
        for s in starts:
            seg = k_idx[b, s:s + NEEDLE_TOKENS]
            f = (seg.astype(np.uint32) << np.uint32(16)).view(np.float32) * NEEDLE_GAIN
            k_idx[b, s:s + NEEDLE_TOKENS] = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def make_custom(seed_id: int, lens, n_query: int, q_heads: int, kv_heads: int,
                max_len: int | None = None, needles: int = 0, parts=("index", "attn"),
                threads: int | None = None, name: str = "custom") -> Workload:
    lens = np.asarray(lens, dtype=np.int32)
    if max_len is None:
        max_len = int(lens.max()) if lens.size else 4
    max_len = (max_len + 3) // 4 * 4
    B = int(lens.shape[0])
    w = Workload(name=name, lens=lens, max_len=max_len, n_query=n_query,
                 q_heads=q_heads, kv_heads=kv_heads)
    th = _threads(threads)
    if "index" in parts:
        w.q_idx = gen_tensor(seed_id, T_Q_IDX, (B, n_query, IDX_HEADS, IDX_DIM), "int", th)
        w.k_idx = gen_tensor(seed_id, T_K_IDX, (B, max_len, IDX_DIM), "int", th)
        if needles:
            w.needle_starts = [needle_starts_for(seed_id, int(lens[b]), needles, b)
                               for b in range(B)]
            plant_needles(w.k_idx, w.needle_starts)
    if "attn" in parts:
        w.q = gen_tensor(seed_id, T_Q, (B, n_query, q_heads, HEAD_DIM), "normal", th)
        w.k = gen_tensor(seed_id, T_K, (B, max_len, kv_heads, HEAD_DIM), "normal", th)
        w.v = gen_tensor(seed_id, T_V, (B, max_len, kv_heads, HEAD_DIM), "normal", th)
    return w


def make(cfg_id: int, parts=("index", "attn"), threads: int | None = None) -> Workload:
    """The benchmark workload `cfg_id` (0..4), generated deterministically."""
    c = CONFIGS[cfg_id]
    return make_custom(cfg_id, c["lens"], c["n_query"], c["q_heads"], c["kv_heads"],
                       needles=c["needles"], parts=parts, threads=threads, name=c["name"])
