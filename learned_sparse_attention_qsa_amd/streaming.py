"""Whole-sequence streaming over the QSA C ABI: a long prompt prefilled chunk
by chunk, then decode steps that append new tokens to the caches.

The speed experiment behind the layer measures a last-chunk prefill and a
batch-four decode with three extra multi-token-prediction steps (page "Qwen's
million-token window has a 2,048-token keyhole", section "Three speed claims,
three different experiments"); a serving stack reaches both states by
running the whole prompt through the layer in chunks and then decoding.
This module is that outer loop, host-side orchestration only: every chunk
and every step is one qsa_forward call, which compresses just the micro-blocks
the chunk or step completes (first_block) and leaves the earlier ones in the
caller's compressed-key cache.

A sequence here is batch-1 state with a fixed capacity: the indexer keys,
compressed keys and core K/V of every token so far.  Appending a token's
rows is a device copy into the caches (the model's projections produce them);
nothing is allocated per chunk or step after construction except the outputs
the caller does not provide.
"""
from __future__ import annotations

import torch

from . import (BLOCK, HEAD_DIM, IDX_DIM, IDX_HEADS, OP_FORWARD, TOPK, forward, shape,
               workspace_bytes)


class Sequence:
    """Caches of one sequence (batch 1) with room for `capacity` tokens."""

    def __init__(self, capacity: int, q_heads: int, kv_heads: int, device="cuda",
                 flags: int = 0):
        if capacity <= 0 or capacity % BLOCK:
            raise ValueError("capacity must be a positive multiple of 4")
        self.capacity = capacity
        self.q_heads, self.kv_heads = q_heads, kv_heads
        self.flags = flags
        self.device = torch.device(device)
        bf = torch.bfloat16
        self.k_idx = torch.zeros((1, capacity, IDX_DIM), dtype=bf, device=device)
        self.k_cmp = torch.zeros((1, capacity // BLOCK, IDX_DIM), dtype=bf, device=device)
        self.k = torch.zeros((1, capacity, kv_heads, HEAD_DIM), dtype=bf, device=device)
        self.v = torch.zeros((1, capacity, kv_heads, HEAD_DIM), dtype=bf, device=device)
        self.length = 0
        self._ws = None
        # (length, first block) of the current call, as device int32 scalars
        self._lens = torch.zeros(1, dtype=torch.int32, device=device)
        self._first = torch.zeros(1, dtype=torch.int32, device=device)

    def append(self, k_idx, k, v) -> None:
        """Write the rows of n new tokens (k_idx [n][64], k and v [n][Hkv][128])
        at the end of the caches."""
        n = k_idx.shape[0]
        if self.length + n > self.capacity:
            raise ValueError("sequence capacity exceeded")
        s = slice(self.length, self.length + n)
        self.k_idx[0, s].copy_(k_idx)
        self.k[0, s].copy_(k)
        self.v[0, s].copy_(v)
        self.length += n

    def _workspace(self, shp):
        need = workspace_bytes(shp, OP_FORWARD)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws if need else None

    def attend_last(self, q_idx, q, done: int, out=None, lse=None, sel=None, n_sel=None):
        """One qsa_forward call for the last n tokens of the sequence (q_idx
        [n][4][64], q [n][Hq][128]); `done` tokens (a multiple of 4 or not)
        were in the sequence at the previous call, so the call compresses the
        micro-blocks from done // 4 on.  Returns (out, lse, sel, n_sel) with
        a leading batch dimension of 1."""
        n = q_idx.shape[0]
        shp = shape(1, self.capacity, n, self.q_heads, self.kv_heads, 0.0, self.flags)
        self._lens.fill_(self.length)
        self._first.fill_(done // BLOCK)
        return forward(shp, q_idx.view(1, n, IDX_HEADS, IDX_DIM), self.k_idx, self.k_cmp,
                       q.view(1, n, self.q_heads, HEAD_DIM), self.k, self.v, self._lens,
                       first_block=self._first, out=out, lse=lse, sel=sel, n_sel=n_sel,
                       ws=self._workspace(shp))


def prefill(seq: Sequence, q_idx, k_idx, q, k, v, chunk: int, on_chunk=None):
    """Chunked prefill of a prompt of n tokens: for each chunk of at most
    `chunk` tokens, its rows are appended and its queries attend over
    everything up to themselves.  q_idx [n][4][64], k_idx [n][64], q
    [n][Hq][128], k and v [n][Hkv][128].  Returns out [n][Hq][128] (bf16);
    on_chunk(c, lo, hi, out, lse, sel, n_sel), when given, sees each chunk's
    results (with its selection) right after its call was enqueued."""
    n = q_idx.shape[0]
    out = torch.empty((n, seq.q_heads, HEAD_DIM), dtype=torch.bfloat16, device=seq.device)
    for c, lo in enumerate(range(0, n, chunk)):
        hi = min(n, lo + chunk)
        done = seq.length
        seq.append(k_idx[lo:hi], k[lo:hi], v[lo:hi])
        sel = n_sel = None
        if on_chunk is not None:
            sel = torch.empty((1, hi - lo, TOPK), dtype=torch.int32, device=seq.device)
            n_sel = torch.empty((1, hi - lo), dtype=torch.int32, device=seq.device)
        o, lse, sel, n_sel = seq.attend_last(q_idx[lo:hi], q[lo:hi], done,
                                             out=out[lo:hi].view(1, hi - lo, seq.q_heads,
                                                                 HEAD_DIM),
                                             sel=sel, n_sel=n_sel)
        if on_chunk is not None:
            on_chunk(c, lo, hi, o, lse, sel, n_sel)
    return out


def decode_step(seq: Sequence, q_idx, k_idx, q, k, v, out=None, lse=None, sel=None,
                n_sel=None):
    """One decode step of m new tokens (one accepted token plus the
    multi-token-prediction positions): their rows are appended, and their
    queries attend over the sequence so far; only the micro-blocks the step
    completes are compressed.  Shapes as in prefill with n = m."""
    done = seq.length
    seq.append(k_idx, k, v)
    return seq.attend_last(q_idx, q, done, out=out, lse=lse, sel=sel, n_sel=n_sel)
