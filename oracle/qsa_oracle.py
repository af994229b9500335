"""Plain, slow CPU oracle of the Qwen Sparse Attention (QSA) hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  It shares no code
with the HIP library.

Arithmetic is float64 / int64.  Every step follows the method as described on
the page "Qwen's million-token window has a 2,048-token keyhole" (cronfeed.work,
English edition; its Chinese twin "Qwen 的百万 token 窗口，只有一道 2,048 token
的锁孔" states the same facts):

  * the opening section: each sparse-attention query picks up to 2,048
    earlier tokens, grouped in at most 512 micro-blocks of four tokens, and
    also takes the unfinished block at the sequence tail;
  * section "A million-token window with a selective view": the indexer has
    four query heads and one shared key head, compresses keys four at a time,
    ranks the micro-blocks, expands the winners back to token positions and
    runs core attention only there; the 2,048-token budget does not grow
    with the context;
  * section "Three speed claims, three different experiments": the baseline
    is grouped-query attention, so core attention is GQA.

The pages give no formula for the compression, the block score, the tie
rule or the softmax scale.  The readings used here (each one listed with its
reason in the design notes of this repository) are:

  compress   kc[j] = sum_{r<4} k_idx[4j + r], exact, then one
             round-to-nearest-even to bf16;
  score      s[i][j] = sum_{h<4} max(0, q_idx[i,h] . kc[j]), no scale;
  candidates completed blocks strictly before the query's own block,
             j < bt = floor(t / 4);
  select     keep all candidates when bt <= 512, else the 512 best under
             (score descending, block index ascending);
  tail       the query's own block, tokens 4*bt .. t (1 to 4 tokens);
  attend     softmax(scale * q . k) over the gathered tokens, query head h
             reading KV head floor(h / (Hq / Hkv)), scale = 1/sqrt(128).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 4          # tokens per micro-block
TOPK = 512         # micro-blocks kept per query (2,048-token budget)
IDX_HEADS = 4      # indexer query heads (one shared key head)
IDX_DIM = 64       # indexer head dimension
HEAD_DIM = 128     # core attention head dimension


# --------------------------------------------------------------------------
# bf16 <-> float64
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns: the bf16 pattern is the top half of the
    float32 pattern of the same number."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); uint16 bits.

    bf16 keeps 8 significant bits and float32's exponent range.  A finite
    x = m * 2**e with 0.5 <= |m| < 1 is rounded to a multiple of its quantum
    2**(e - 8), or of 2**-133 (the subnormal quantum) when x is that small;
    np.rint rounds halves to even.  Results above the largest bf16 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x) & (x != 0.0)
    v = np.where(finite, x, 1.0)
    _, e = np.frexp(v)                           # |v| = m * 2**e, m in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)              # exponent of the bf16 quantum
    r = np.ldexp(np.rint(np.ldexp(v, -q_exp)), q_exp)
    max_bf16 = math.ldexp(255.0, 120)            # (2 - 2**-7) * 2**127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, v), r)
    out = np.where(finite, r, x)
    f32 = out.astype(np.float32)                 # exact: every result is a bf16 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# The four method steps
# --------------------------------------------------------------------------

def compress_keys(k_idx_bits: np.ndarray, n_tokens: int, first_block: int = 0) -> np.ndarray:
    """Compressed indexer keys of blocks first_block .. floor(n_tokens/4) - 1.

    The indexer folds each run of four keys into one micro-block key (section
    "A million-token window with a selective view").  Reading: the micro-block
    key is the sum of its four token keys, formed exactly and rounded once to
    bf16.
    Returns uint16 bf16 bits, shape [n_blocks - first_block][64].
    """
    n_blocks = n_tokens // BLOCK
    rows = bf16_bits_to_f64(k_idx_bits[first_block * BLOCK:n_blocks * BLOCK])
    sums = np.zeros((n_blocks - first_block, rows.shape[-1]), dtype=np.float64)
    for r in range(BLOCK):
        sums += rows[r::BLOCK]
    return f64_to_bf16_bits(sums)


def block_scores(q_idx: np.ndarray, kc: np.ndarray) -> np.ndarray:
    """Indexer score of every compressed block for one query.

    q_idx: float64 [4][64] (the four indexer query heads); kc: float64
    [n_blocks][64] (compressed keys of the shared key head).
    s[j] = sum over heads of max(0, q_h . kc[j]).  The pages say only that the
    indexer scores and ranks the blocks; the sum of per-head ReLU scores is the
    reading adopted.  Exact for the small-integer inputs used here (every
    partial sum is an integer far below 2**53).
    """
    per_head = kc @ q_idx.T                      # [n_blocks][4]
    return np.maximum(per_head, 0.0).sum(axis=1)


def select_blocks(scores: np.ndarray, k: int = TOPK) -> np.ndarray:
    """Top-k micro-blocks of one query, ascending block ids (int64).

    Up to 512 blocks are kept (opening section of the page: a 2,048-token
    budget in at most 512 four-token micro-blocks).  With no more than k
    candidates all are kept.  Otherwise v is the k-th largest score; every
    block scoring above v is kept and the rest of the budget goes to the
    lowest-numbered blocks scoring exactly v (the tie rule is a reading: the
    pages state none).
    """
    n = scores.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    v = np.partition(scores, n - k)[n - k]       # k-th largest value
    above = np.nonzero(scores > v)[0]
    ties = np.nonzero(scores == v)[0]            # ascending block ids
    chosen = np.concatenate([above, ties[:k - above.shape[0]]])
    return np.sort(chosen).astype(np.int64)


def expand_tokens(sel: np.ndarray, t: int) -> np.ndarray:
    """Token positions attended by the query at position t.

    The kept blocks are turned back into the token positions they cover, and
    the unfinished block at the tail is added (opening section and section "A
    million-token window with a selective view").  Reading: the tail is the query's own
    block, tokens 4*floor(t/4) .. t, which holds 1 to 4 tokens.
    """
    bt = t // BLOCK
    parts = [np.arange(BLOCK * int(j), BLOCK * int(j) + BLOCK, dtype=np.int64) for j in sel]
    parts.append(np.arange(BLOCK * bt, t + 1, dtype=np.int64))
    return np.sort(np.concatenate(parts))


def attend(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float):
    """Grouped-query softmax attention of one query token over gathered rows.

    q: float64 [Hq][D]; k_rows, v_rows: float64 [n][Hkv][D].  Query head h
    reads KV head floor(h / (Hq / Hkv)).  Returns (o [Hq][D], lse [Hq]) with
    lse = ln sum_s exp(scale * q_h . k_s).  Core attention over the selected
    positions is GQA because the pages' dense baseline is grouped-query
    attention (section "Three speed claims, three different experiments").
    """
    hq = q.shape[0]
    hkv = k_rows.shape[1]
    group = hq // hkv
    o = np.zeros((hq, q.shape[1]), dtype=np.float64)
    lse = np.full(hq, -np.inf, dtype=np.float64)
    if k_rows.shape[0] == 0:
        return o, lse
    for h in range(hq):
        g = h // group
        z = scale * (k_rows[:, g, :] @ q[h])
        m = z.max()
        p = np.exp(z - m)
        denom = p.sum()
        o[h] = (p @ v_rows[:, g, :]) / denom
        lse[h] = m + math.log(denom)
    return o, lse


# --------------------------------------------------------------------------
# The same scoring and selection for many query rows at once
# --------------------------------------------------------------------------

def block_scores_rows(q_idx: np.ndarray, kc: np.ndarray) -> np.ndarray:
    """Indexer scores of every compressed block for n queries of one sequence.

    q_idx: float64 [n][4][64]; kc: float64 [m][64].  Returns float64 [n][m]
    with s[i][j] = sum over heads of max(0, q_idx[i, h] . kc[j]): the score of
    block_scores, for n rows in one matrix product (the indexer ranks the
    micro-blocks per query, section "A million-token window with a selective
    view").  Exact for the small-integer inputs used here.
    """
    n = q_idx.shape[0]
    per_head = (q_idx.reshape(n * IDX_HEADS, -1) @ kc.T).reshape(n, IDX_HEADS, kc.shape[0])
    return np.maximum(per_head, 0.0).sum(axis=1)


def select_blocks_rows(scores: np.ndarray, bt: np.ndarray, k: int = TOPK):
    """Top-k selection of select_blocks for n rows at once.

    scores: float64 [n][m] (non-negative); bt: int [n], row i's candidates are
    blocks 0 .. bt[i] - 1 (later columns are ignored).  Returns (sel int64
    [n][k] ascending, padded with -1; n_sel int64 [n]).  Per row: all
    candidates when bt <= k; otherwise v is the k-th largest candidate score,
    every block above v is kept and the rest of the budget goes to the
    lowest-numbered blocks scoring exactly v.
    """
    n, m = scores.shape
    bt = np.minimum(np.asarray(bt, dtype=np.int64), m)
    sel = np.full((n, k), -1, dtype=np.int64)
    n_sel = np.minimum(bt, k)
    short = bt <= k
    for i in np.nonzero(short)[0]:
        sel[i, :bt[i]] = np.arange(bt[i])
    rows = np.nonzero(~short)[0]
    if rows.size == 0:
        return sel, n_sel
    # blocks at or past a row's own block score -1, below every candidate
    s = np.where(np.arange(m)[None, :] < bt[rows, None], scores[rows], -1.0)
    v = np.partition(s, m - k, axis=1)[:, m - k]          # k-th largest per row
    above = s > v[:, None]
    equal = s == v[:, None]
    need = k - above.sum(axis=1)
    keep = above | (equal & (np.cumsum(equal, axis=1) <= need[:, None]))
    r_idx, j_idx = np.nonzero(keep)                        # row-major: ascending j
    sel[rows] = j_idx.reshape(rows.size, k)
    return sel, n_sel


def select_rows(q_idx_bits, k_idx_bits, lens, n_query: int, rows, k: int = TOPK,
                chunk: int | None = None, threads: int = 1):
    """Selections of the given (b, i) query rows, computed with the row-batched
    scorer and selector (chunks of `chunk` rows of one sequence, by default
    about 2**24 scores per chunk, on `threads` threads).
    Returns {(b, i): (sel ascending int64, n_sel)}."""
    from concurrent.futures import ThreadPoolExecutor

    by_seq = {}
    for b, i in rows:
        by_seq.setdefault(int(b), []).append(int(i))
    out = {}
    for b, idxs in by_seq.items():
        length = int(lens[b])
        kc = bf16_bits_to_f64(compress_keys(k_idx_bits[b], length))
        idxs = sorted(set(idxs))
        step = chunk or max(8, (1 << 24) // max(1, length // BLOCK))
        parts = [idxs[c:c + step] for c in range(0, len(idxs), step)]

        def work(part):
            t = length - n_query + np.asarray(part, dtype=np.int64)
            q = bf16_bits_to_f64(q_idx_bits[b, part])
            m = int(t.max()) // BLOCK
            s = block_scores_rows(q, kc[:m])
            sel, n_sel = select_blocks_rows(s, t // BLOCK, k)
            return [((b, i), (sel[r, :n_sel[r]], int(n_sel[r]))) for r, i in enumerate(part)]

        if threads > 1 and len(parts) > 1:
            with ThreadPoolExecutor(threads) as ex:
                for res in ex.map(work, parts):
                    out.update(res)
        else:
            for part in parts:
                out.update(work(part))
    return out


# --------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------

def query_positions(length: int, n_query: int) -> np.ndarray:
    """Positions of the n_query query tokens: the last n_query of the sequence."""
    return np.arange(length - n_query, length, dtype=np.int64)


def qsa_forward(q_idx_bits, k_idx_bits, q_bits, k_bits, v_bits, lens, n_query: int,
                scale: float | None = None, queries=None, k: int = TOPK):
    """Run the oracle over a batch.

    Arrays are uint16 bf16 bits in the layouts of the synthetic workloads.
    ``queries`` optionally restricts the work to a list of (b, i) pairs.
    Returns a dict with, per computed (b, i): sel, tok, out (float64 [Hq][128]),
    lse, and per sequence the compressed keys kc (uint16 bits).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    B = len(lens)
    if queries is None:
        queries = [(b, i) for b in range(B) for i in range(n_query)]
    res = {"sel": {}, "tok": {}, "out": {}, "lse": {}, "kc": {}}
    by_seq = {}
    for b, i in queries:
        by_seq.setdefault(b, []).append(i)
    for b, idxs in by_seq.items():
        length = int(lens[b])
        kc_bits = compress_keys(k_idx_bits[b], length)
        res["kc"][b] = kc_bits
        kc = bf16_bits_to_f64(kc_bits)
        pos = query_positions(length, n_query)
        for i in idxs:
            t = int(pos[i])
            qi = bf16_bits_to_f64(q_idx_bits[b, i])
            bt = t // BLOCK
            s = block_scores(qi, kc[:bt])
            sel = select_blocks(s, k)
            tok = expand_tokens(sel, t)
            o = lse = None
            if q_bits is not None:
                kr = bf16_bits_to_f64(k_bits[b, tok])
                vr = bf16_bits_to_f64(v_bits[b, tok])
                o, lse = attend(bf16_bits_to_f64(q_bits[b, i]), kr, vr, scale)
            res["sel"][(b, i)] = sel
            res["tok"][(b, i)] = tok
            res["out"][(b, i)] = o
            res["lse"][(b, i)] = lse
    return res


def dense_decode(q_bits, k_bits, v_bits, lens, n_query: int, scale: float | None = None,
                 queries=None):
    """Dense causal GQA over every earlier position (the comparator of the
    speed experiment: grouped-query attention over the full context).
    Returns {(b, i): (out, lse)}."""
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    B = len(lens)
    if queries is None:
        queries = [(b, i) for b in range(B) for i in range(n_query)]
    out = {}
    for b, i in queries:
        t = int(lens[b]) - n_query + i
        kr = bf16_bits_to_f64(k_bits[b, :t + 1])
        vr = bf16_bits_to_f64(v_bits[b, :t + 1])
        out[(b, i)] = attend(bf16_bits_to_f64(q_bits[b, i]), kr, vr, scale)
    return out


# --------------------------------------------------------------------------
# The indexer's training target and what the selection keeps of it
# --------------------------------------------------------------------------

def block_teacher(q: np.ndarray, k_rows: np.ndarray, t: int, scale: float) -> np.ndarray:
    """Dense attention mass of every micro-block for the query at position t.

    The indexer learns from the full-attention distribution (page "Qwen's
    million-token window has a 2,048-token keyhole", section "The indexer is
    trained, not bolted on").  Reading: the target is that distribution
    pooled per micro-block and averaged over the core query heads,
      T[j] = (1/Hq) sum_h sum_{s in block j, s <= t} softmax_h(scale q_h . k_s),
    over blocks 0 .. floor(t/4), the last one holding only tokens up to t.
    q: float64 [Hq][D]; k_rows: float64 [>= t+1][Hkv][D] (the sequence's keys).
    Returns float64 [floor(t/4) + 1]; it sums to 1.
    """
    hq = q.shape[0]
    hkv = k_rows.shape[1]
    group = hq // hkv
    n = t + 1
    bt = t // BLOCK
    pooled = np.zeros(bt + 1, dtype=np.float64)
    for h in range(hq):
        z = scale * (k_rows[:n, h // group, :] @ q[h])
        p = np.exp(z - z.max())
        p /= p.sum()
        pooled += np.bincount(np.arange(n) // BLOCK, weights=p, minlength=bt + 1)
    return pooled / hq


def selection_recall(teacher: np.ndarray, sel: np.ndarray) -> float:
    """Share of the teacher's mass on the positions QSA attends to: the kept
    micro-blocks and the query's own block (always attended, opening section
    of the page)."""
    return float(teacher[np.asarray(sel, dtype=np.int64)].sum() + teacher[-1])


def needle_survival(sel: np.ndarray, needle_blocks) -> float:
    """Share of the planted micro-blocks that the selection keeps (the pages
    ask whether the evidence a long-context task needs survives the
    selection: section "What a serious evaluation should preserve")."""
    nb = np.asarray(sorted(needle_blocks), dtype=np.int64)
    if nb.size == 0:
        return 1.0
    return float(np.isin(nb, np.asarray(sel, dtype=np.int64)).mean())


# --------------------------------------------------------------------------
# Gradients (the indexer and the backbone are trained together)
# --------------------------------------------------------------------------

def attend_backward(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, d_out: np.ndarray,
                    scale: float):
    """Gradient of attend()'s output o with respect to q, the gathered k rows
    and the gathered v rows, given d_out = dL/do (float64 [Hq][D]).

    The indexer and the model are trained together (page "Qwen's million-token
    window has a 2,048-token keyhole", section "The indexer is trained, not
    bolted on"), so the sparse attention needs its backward pass; it is the
    softmax-attention gradient over the gathered rows only: with p the softmax
    of z = scale q_h . k_s, dp_s = d_out_h . v_s and ds_s = p_s (dp_s -
    sum_r p_r dp_r),
      dq_h = scale sum_s ds_s k_s,  dk_s += scale ds_s q_h,  dv_s += p_s d_out_h
    (query head h reading KV head floor(h / (Hq / Hkv))).
    Returns (dq [Hq][D], dk [n][Hkv][D], dv [n][Hkv][D]).
    """
    hq, hkv = q.shape[0], k_rows.shape[1]
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_rows)
    dv = np.zeros_like(v_rows)
    for h in range(hq):
        g = h // group
        z = scale * (k_rows[:, g, :] @ q[h])
        p = np.exp(z - z.max())
        p /= p.sum()
        dp = v_rows[:, g, :] @ d_out[h]
        ds = p * (dp - np.dot(p, dp))
        dq[h] = scale * (ds @ k_rows[:, g, :])
        dk[:, g, :] += scale * np.outer(ds, q[h])
        dv[:, g, :] += np.outer(p, d_out[h])
    return dq, dk, dv


def block_scores_backward(q_idx: np.ndarray, kc: np.ndarray, g: np.ndarray):
    """Gradient of block_scores() (s_j = sum_h max(0, q_h . kc_j)) given
    g = dL/ds (float64 [n]): dq_h = sum_j g_j [q_h . kc_j > 0] kc_j and
    dkc_j = sum_h g_j [q_h . kc_j > 0] q_h (the ReLU's derivative taken as 0
    at 0).  Returns (dq [4][64], dkc [n][64])."""
    per_head = kc @ q_idx.T                      # [n][4]
    w = (per_head > 0.0) * g[:, None]            # [n][4]
    return w.T @ kc, w @ q_idx


def compress_keys_backward(d_kc: np.ndarray) -> np.ndarray:
    """Gradient of compress_keys()'s sum with respect to the token keys: each
    of a block's four keys receives the block's gradient (the bf16 rounding
    is taken as the identity, as it is for the configurations' exact sums).
    d_kc: float64 [m][64] -> [4m][64]."""
    return np.repeat(d_kc, BLOCK, axis=0)
