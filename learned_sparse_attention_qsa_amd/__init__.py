"""Python binding of libqsa, the Qwen Sparse Attention (QSA) hot path for
AMD MI355X (gfx950).

This module only marshals arguments: torch tensors supply device memory and
the current HIP stream, and every step of the path runs in the HIP kernels of
``lib/libqsa.so``.  If the library has not been built, every call raises;
there is no CPU fallback.

Names follow the C ABI in ``include/qsa.h``.  Tensors are torch CUDA (HIP)
tensors, contiguous: bf16 data as ``torch.bfloat16`` (or int16 bit patterns),
int32 for lens / sel / tok.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QSA_LIBRARY selects another build of the same library (the sanitized one)
LIB_PATH = os.environ.get("QSA_LIBRARY") or os.path.join(_HERE, "lib", "libqsa.so")

IDX_HEADS = 4
IDX_DIM = 64
BLOCK = 4
TOPK = 512
HEAD_DIM = 128
MAX_TOK = TOPK * BLOCK + BLOCK

OK, ERR_NULL, ERR_ALIGN, ERR_SHAPE, ERR_WORKSPACE, ERR_DEVICE, ERR_HIP, ERR_SCRATCH = range(8)
NOALLOC_SCRATCH_BYTES = 64 << 20
(OP_COMPRESS, OP_INDEX_TOPK, OP_EXPAND, OP_SPARSE_ATTEND, OP_FORWARD, OP_DENSE_DECODE,
 OP_BLOCK_TEACHER) = range(7)
FLAG_TOPK_TABLE = 1
FLAG_TOPK_STREAM = 2
FLAG_TOPK_SCAN = 4

# Every symbol include/qsa.h declares.
EXPORTS = (
    "qsa_workspace_bytes",
    "qsa_status_string",
    "qsa_compress_keys",
    "qsa_index_topk",
    "qsa_expand_blocks",
    "qsa_sparse_attend",
    "qsa_forward",
    "qsa_forward_noalloc",
    "qsa_dense_gqa_decode",
    "qsa_sparse_attend_paged",
    "qsa_forward_paged",
    "qsa_dense_gqa_decode_paged",
    "qsa_dense_gqa_prefill",
    "qsa_block_teacher",
    "qsa_teacher_recall",
    "qsa_sparse_attend_backward",
    "qsa_index_scores_backward",
    "qsa_compress_keys_backward",
    "qsa_debug_build",
    "qsa_debug_guard_hits",
    "qsa_profile_attach",
    "qsa_profile_detach",
    "qsa_profile_kernel_name",
    # include/qsa_ceilings.h: memory-system ceilings for benchmarks
    "qsa_ceil_stream_read",
    "qsa_ceil_gather",
    "qsa_ceil_lds_atomic",
)


class QsaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("n_query", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class QsaPagedKV(ctypes.Structure):
    _fields_ = [
        ("page_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("n_pages", ctypes.c_int32),
    ]


class PagedKV:
    """A page table (device int32 [B][max_pages]) over K/V page pools
    [n_pages][page_size][Hkv][128]; keeps the table tensor alive."""

    def __init__(self, page_table: torch.Tensor, page_size: int, n_pages: int):
        if page_table.dtype != torch.int32 or page_table.dim() != 2:
            raise ValueError("page_table must be int32 [B][max_pages]")
        if not page_table.is_contiguous():
            raise ValueError("page_table must be contiguous")
        self.page_table = page_table
        self.page_size = int(page_size)
        self.n_pages = int(n_pages)
        self.c = QsaPagedKV(page_table.data_ptr(), self.page_size, page_table.shape[1],
                            self.n_pages)


class QsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m learned_sparse_attention_qsa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    sp = ctypes.POINTER(QsaShape)
    lib.qsa_workspace_bytes.argtypes = [sp, i32]
    lib.qsa_workspace_bytes.restype = sz
    lib.qsa_status_string.argtypes = [i32]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_compress_keys.argtypes = [sp, vp, vp, vp, vp, vp]
    lib.qsa_index_topk.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_expand_blocks.argtypes = [sp, vp, vp, vp, vp, vp, vp]
    lib.qsa_sparse_attend.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_forward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_dense_gqa_decode.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_forward_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    pp = ctypes.POINTER(QsaPagedKV)
    lib.qsa_sparse_attend_paged.argtypes = [sp, vp, vp, vp, pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_forward_paged.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.qsa_dense_gqa_decode_paged.argtypes = [sp, vp, vp, vp, pp, vp, vp, vp, vp, sz, vp]
    lib.qsa_dense_gqa_prefill.argtypes = [sp, vp, vp, vp, pp, vp, vp, vp, vp]
    lib.qsa_block_teacher.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qsa_teacher_recall.argtypes = [sp, vp, vp, vp, vp, vp, vp]
    lib.qsa_sparse_attend_backward.argtypes = [sp] + [vp] * 13
    lib.qsa_index_scores_backward.argtypes = [sp] + [vp] * 7
    lib.qsa_compress_keys_backward.argtypes = [sp, vp, vp, vp, vp]
    for name in EXPORTS[2:18]:
        getattr(lib, name).restype = i32
    lib.qsa_debug_build.argtypes = []
    lib.qsa_debug_build.restype = i32
    lib.qsa_debug_guard_hits.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.qsa_debug_guard_hits.restype = i32
    lib.qsa_profile_attach.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.qsa_profile_attach.restype = i32
    lib.qsa_profile_detach.argtypes = []
    lib.qsa_profile_detach.restype = i32
    lib.qsa_profile_kernel_name.argtypes = [i32]
    lib.qsa_profile_kernel_name.restype = ctypes.c_char_p
    lib.qsa_ceil_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.qsa_ceil_stream_read.restype = i32
    lib.qsa_ceil_gather.argtypes = [vp, vp, ctypes.c_int64, i32, i32, vp, vp]
    lib.qsa_ceil_gather.restype = i32
    lib.qsa_ceil_lds_atomic.argtypes = [i32, i32, i32, i32, vp, vp]
    lib.qsa_ceil_lds_atomic.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().qsa_status_string(status).decode()


def shape(batch: int, max_len: int, n_query: int, q_heads: int, kv_heads: int,
          scale: float = 0.0, flags: int = 0) -> QsaShape:
    return QsaShape(batch, max_len, n_query, q_heads, kv_heads, scale, flags)


def workspace_bytes(shp: QsaShape, op: int) -> int:
    return int(load_library().qsa_workspace_bytes(ctypes.byref(shp), op))


def workspace(shp: QsaShape, op: int, device="cuda") -> torch.Tensor | None:
    n = workspace_bytes(shp, op)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


# ------------------------------------------------------------------ helpers

def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str) -> None:
    if status != OK:
        raise QsaError(status, what)


def _need(t: torch.Tensor, name: str, shape_, dtypes) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape_):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape_)}")


_BF = (torch.bfloat16, torch.int16)
_I32 = (torch.int32,)


def _ws(shp, op, ws, device):
    need = workspace_bytes(shp, op)
    if need == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ------------------------------------------------------------------ entry points

def compress_keys(shp: QsaShape, k_idx, lens, k_cmp, first_block=None) -> torch.Tensor:
    B, L = shp.batch, shp.max_len
    _need(k_idx, "k_idx", (B, L, IDX_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    if first_block is not None:
        _need(first_block, "first_block", (B,), _I32)
    st = load_library().qsa_compress_keys(ctypes.byref(shp), _p(k_idx), _p(lens), _p(first_block),
                                          _p(k_cmp), _stream(k_idx.device))
    _check(st, "qsa_compress_keys")
    return k_cmp


def index_topk(shp: QsaShape, q_idx, k_cmp, lens, sel=None, n_sel=None, ws=None):
    B, L, Nq = shp.batch, shp.max_len, shp.n_query
    dev = q_idx.device
    _need(q_idx, "q_idx", (B, Nq, IDX_HEADS, IDX_DIM), _BF)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    if sel is None:
        sel = torch.empty((B, Nq, TOPK), dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty((B, Nq), dtype=torch.int32, device=dev)
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    ws, nb = _ws(shp, OP_INDEX_TOPK, ws, dev)
    st = load_library().qsa_index_topk(ctypes.byref(shp), _p(q_idx), _p(k_cmp), _p(lens), _p(sel),
                                       _p(n_sel), _p(ws), nb, _stream(dev))
    _check(st, "qsa_index_topk")
    return sel, n_sel


def expand_blocks(shp: QsaShape, lens, sel, n_sel, tok=None, n_tok=None):
    B, Nq = shp.batch, shp.n_query
    dev = sel.device
    _need(lens, "lens", (B,), _I32)
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    if tok is None:
        tok = torch.empty((B, Nq, MAX_TOK), dtype=torch.int32, device=dev)
    if n_tok is None:
        n_tok = torch.empty((B, Nq), dtype=torch.int32, device=dev)
    _need(tok, "tok", (B, Nq, MAX_TOK), _I32)
    _need(n_tok, "n_tok", (B, Nq), _I32)
    st = load_library().qsa_expand_blocks(ctypes.byref(shp), _p(lens), _p(sel), _p(n_sel), _p(tok),
                                          _p(n_tok), _stream(dev))
    _check(st, "qsa_expand_blocks")
    return tok, n_tok


def sparse_attend(shp: QsaShape, q, k, v, lens, sel, n_sel, out=None, lse=None, ws=None,
                  want_lse: bool = True):
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    if out is None:
        out = torch.empty((B, Nq, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    _need(out, "out", (B, Nq, Hq, HEAD_DIM), _BF)
    if lse is None and want_lse:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, Nq, Hq), (torch.float32,))
    ws, nb = _ws(shp, OP_SPARSE_ATTEND, ws, dev)
    st = load_library().qsa_sparse_attend(ctypes.byref(shp), _p(q), _p(k), _p(v), _p(lens),
                                          _p(sel), _p(n_sel), _p(out), _p(lse), _p(ws), nb,
                                          _stream(dev))
    _check(st, "qsa_sparse_attend")
    return out, lse


def forward(shp: QsaShape, q_idx, k_idx, k_cmp, q, k, v, lens, first_block=None, out=None,
            lse=None, sel=None, n_sel=None, ws=None, want_lse: bool = True):
    """Compress (blocks [first_block, lens/4)) -> score + top-k -> expand ->
    sparse attention, one call.  Returns (out, lse, sel, n_sel)."""
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q_idx, "q_idx", (B, Nq, IDX_HEADS, IDX_DIM), _BF)
    _need(k_idx, "k_idx", (B, L, IDX_DIM), _BF)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    if first_block is not None:
        _need(first_block, "first_block", (B,), _I32)
    if out is None:
        out = torch.empty((B, Nq, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=dev)
    if (sel is None) != (n_sel is None):
        raise ValueError("give both sel and n_sel, or neither")
    if sel is not None:
        _need(sel, "sel", (B, Nq, TOPK), _I32)
        _need(n_sel, "n_sel", (B, Nq), _I32)
    ws, nb = _ws(shp, OP_FORWARD, ws, dev)
    st = load_library().qsa_forward(ctypes.byref(shp), _p(q_idx), _p(k_idx), _p(k_cmp),
                                    _p(first_block), _p(q), _p(k), _p(v), _p(lens), _p(out),
                                    _p(lse), _p(sel), _p(n_sel), _p(ws), nb, _stream(dev))
    _check(st, "qsa_forward")
    return out, lse, sel, n_sel


def forward_noalloc(shp: QsaShape, q_idx, k_idx, k_cmp, q, k, v, lens, out, first_block=None,
                    lse=None, sel=None, n_sel=None):
    """qsa_forward_noalloc: forward() without a workspace; the library's own
    per-GPU scratch array serves instead.  Outputs are caller-given (nothing
    is allocated here either).  Returns (out, lse, sel, n_sel)."""
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    _need(q_idx, "q_idx", (B, Nq, IDX_HEADS, IDX_DIM), _BF)
    _need(k_idx, "k_idx", (B, L, IDX_DIM), _BF)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    _need(out, "out", (B, Nq, Hq, HEAD_DIM), _BF)
    if first_block is not None:
        _need(first_block, "first_block", (B,), _I32)
    if lse is not None:
        _need(lse, "lse", (B, Nq, Hq), (torch.float32,))
    if (sel is None) != (n_sel is None):
        raise ValueError("give both sel and n_sel, or neither")
    if sel is not None:
        _need(sel, "sel", (B, Nq, TOPK), _I32)
        _need(n_sel, "n_sel", (B, Nq), _I32)
    st = load_library().qsa_forward_noalloc(ctypes.byref(shp), _p(q_idx), _p(k_idx), _p(k_cmp),
                                            _p(first_block), _p(q), _p(k), _p(v), _p(lens),
                                            _p(out), _p(lse), _p(sel), _p(n_sel),
                                            _stream(q.device))
    _check(st, "qsa_forward_noalloc")
    return out, lse, sel, n_sel


def dense_gqa_decode(shp: QsaShape, q, k, v, lens, out=None, lse=None, ws=None,
                     want_lse: bool = True):
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    if out is None:
        out = torch.empty((B, Nq, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=dev)
    ws, nb = _ws(shp, OP_DENSE_DECODE, ws, dev)
    st = load_library().qsa_dense_gqa_decode(ctypes.byref(shp), _p(q), _p(k), _p(v), _p(lens),
                                             _p(out), _p(lse), _p(ws), nb, _stream(dev))
    _check(st, "qsa_dense_gqa_decode")
    return out, lse


def _need_pools(k, v, paged: PagedKV, shp: QsaShape) -> None:
    pool = (paged.n_pages, paged.page_size, shp.kv_heads, HEAD_DIM)
    _need(k, "k_pool", pool, _BF)
    _need(v, "v_pool", pool, _BF)
    _need(paged.page_table, "page_table", (shp.batch, paged.page_table.shape[1]), _I32)


def _attn_outputs(shp, dev, out, lse, want_lse):
    B, Nq, Hq = shp.batch, shp.n_query, shp.q_heads
    if out is None:
        out = torch.empty((B, Nq, Hq, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    _need(out, "out", (B, Nq, Hq, HEAD_DIM), _BF)
    if lse is None and want_lse:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, Nq, Hq), (torch.float32,))
    return out, lse


def sparse_attend_paged(shp: QsaShape, q, k_pool, v_pool, paged: PagedKV, lens, sel, n_sel,
                        out=None, lse=None, ws=None, want_lse: bool = True):
    """sparse_attend with K/V read through a page table."""
    B, Nq, Hq = shp.batch, shp.n_query, shp.q_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need_pools(k_pool, v_pool, paged, shp)
    _need(lens, "lens", (B,), _I32)
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    out, lse = _attn_outputs(shp, dev, out, lse, want_lse)
    ws, nb = _ws(shp, OP_SPARSE_ATTEND, ws, dev)
    st = load_library().qsa_sparse_attend_paged(ctypes.byref(shp), _p(q), _p(k_pool),
                                                _p(v_pool), ctypes.byref(paged.c), _p(lens),
                                                _p(sel), _p(n_sel), _p(out), _p(lse), _p(ws), nb,
                                                _stream(dev))
    _check(st, "qsa_sparse_attend_paged")
    return out, lse


def forward_paged(shp: QsaShape, q_idx, k_idx, k_cmp, q, k_pool, v_pool, paged: PagedKV, lens,
                  first_block=None, out=None, lse=None, sel=None, n_sel=None, ws=None,
                  want_lse: bool = True):
    """forward with the core K/V read through a page table (the indexer caches
    stay per sequence).  Returns (out, lse, sel, n_sel)."""
    B, L, Nq, Hq = shp.batch, shp.max_len, shp.n_query, shp.q_heads
    dev = q.device
    _need(q_idx, "q_idx", (B, Nq, IDX_HEADS, IDX_DIM), _BF)
    _need(k_idx, "k_idx", (B, L, IDX_DIM), _BF)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need_pools(k_pool, v_pool, paged, shp)
    _need(lens, "lens", (B,), _I32)
    if first_block is not None:
        _need(first_block, "first_block", (B,), _I32)
    out, lse = _attn_outputs(shp, dev, out, lse, want_lse)
    if (sel is None) != (n_sel is None):
        raise ValueError("give both sel and n_sel, or neither")
    if sel is not None:
        _need(sel, "sel", (B, Nq, TOPK), _I32)
        _need(n_sel, "n_sel", (B, Nq), _I32)
    ws, nb = _ws(shp, OP_FORWARD, ws, dev)
    st = load_library().qsa_forward_paged(ctypes.byref(shp), _p(q_idx), _p(k_idx), _p(k_cmp),
                                          _p(first_block), _p(q), _p(k_pool), _p(v_pool),
                                          ctypes.byref(paged.c), _p(lens), _p(out), _p(lse),
                                          _p(sel), _p(n_sel), _p(ws), nb, _stream(dev))
    _check(st, "qsa_forward_paged")
    return out, lse, sel, n_sel


def dense_gqa_decode_paged(shp: QsaShape, q, k_pool, v_pool, paged: PagedKV, lens, out=None,
                           lse=None, ws=None, want_lse: bool = True):
    B, Nq, Hq = shp.batch, shp.n_query, shp.q_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need_pools(k_pool, v_pool, paged, shp)
    _need(lens, "lens", (B,), _I32)
    out, lse = _attn_outputs(shp, dev, out, lse, want_lse)
    ws, nb = _ws(shp, OP_DENSE_DECODE, ws, dev)
    st = load_library().qsa_dense_gqa_decode_paged(ctypes.byref(shp), _p(q), _p(k_pool),
                                                   _p(v_pool), ctypes.byref(paged.c), _p(lens),
                                                   _p(out), _p(lse), _p(ws), nb, _stream(dev))
    _check(st, "qsa_dense_gqa_decode_paged")
    return out, lse


def dense_gqa_prefill(shp: QsaShape, q, k, v, lens, paged: PagedKV | None = None, out=None,
                      lse=None, want_lse: bool = True):
    """Dense causal GQA for many queries (a prefill chunk); k and v are the
    contiguous caches, or the page pools of `paged`."""
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    if paged is None:
        _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
        _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    else:
        _need_pools(k, v, paged, shp)
    _need(lens, "lens", (B,), _I32)
    out, lse = _attn_outputs(shp, dev, out, lse, want_lse)
    st = load_library().qsa_dense_gqa_prefill(ctypes.byref(shp), _p(q), _p(k), _p(v),
                                              ctypes.byref(paged.c) if paged else None, _p(lens),
                                              _p(out), _p(lse), _stream(dev))
    _check(st, "qsa_dense_gqa_prefill")
    return out, lse


def debug_build() -> bool:
    """True when the loaded library was built with QSA_DEBUG."""
    return bool(load_library().qsa_debug_build())


def debug_guard_hits() -> int:
    """Caller-supplied values the kernels' guards caught since the previous
    call (debug builds; 0 otherwise).  Waits for the device."""
    n = ctypes.c_uint64(0)
    _check(load_library().qsa_debug_guard_hits(ctypes.byref(n)), "qsa_debug_guard_hits")
    return int(n.value)


def ceil_stream_read(buf: torch.Tensor, workgroups: int, sink: torch.Tensor) -> None:
    """Streaming read of the whole of `buf` (qsa_ceil_stream_read)."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda):
        raise ValueError("buf and sink must be contiguous GPU tensors")
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().qsa_ceil_stream_read(_p(buf), nbytes, workgroups, _p(sink),
                                               _stream(buf.device)), "qsa_ceil_stream_read")


def ceil_gather(base: torch.Tensor, row_index: torch.Tensor, row_bytes: int, workgroups: int,
                sink: torch.Tensor) -> None:
    """Random gather of row_bytes-byte pieces row_index[i] of `base`
    (qsa_ceil_gather); every piece must lie inside `base`."""
    if not (base.is_cuda and base.is_contiguous() and row_index.is_cuda and sink.is_cuda):
        raise ValueError("base, row_index and sink must be GPU tensors")
    if row_index.dtype != torch.int64 or not row_index.is_contiguous():
        raise ValueError("row_index must be contiguous int64")
    nbytes = base.numel() * base.element_size()
    n = row_index.numel()
    if n and (int(row_index.min()) < 0 or (int(row_index.max()) + 1) * row_bytes > nbytes):
        raise ValueError("a gathered piece lies outside base")
    _check(load_library().qsa_ceil_gather(_p(base), _p(row_index), n, row_bytes, workgroups,
                                          _p(sink), _stream(base.device)), "qsa_ceil_gather")


def ceil_lds_atomic(f32: bool, share: int, workgroups: int, iters: int,
                    sink: torch.Tensor) -> None:
    """LDS atomic adds with `share` lanes per address (qsa_ceil_lds_atomic);
    sink holds at least `workgroups` words."""
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink must be a GPU tensor of at least `workgroups` words")
    _check(load_library().qsa_ceil_lds_atomic(int(f32), share, workgroups, iters, _p(sink),
                                              _stream(sink.device)), "qsa_ceil_lds_atomic")


def block_teacher(shp: QsaShape, q, k, v, lens, teacher=None, ws=None):
    """qsa_block_teacher: dense attention mass per micro-block, averaged over
    the heads; returns teacher [B][Nq][Lmax/4] float32."""
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    if teacher is None:
        teacher = torch.empty((B, Nq, L // BLOCK), dtype=torch.float32, device=dev)
    _need(teacher, "teacher", (B, Nq, L // BLOCK), (torch.float32,))
    ws, nb = _ws(shp, OP_BLOCK_TEACHER, ws, dev)
    st = load_library().qsa_block_teacher(ctypes.byref(shp), _p(q), _p(k), _p(v), _p(lens),
                                          _p(teacher), _p(ws), nb, _stream(dev))
    _check(st, "qsa_block_teacher")
    return teacher


def teacher_recall(shp: QsaShape, lens, teacher, sel, n_sel, recall=None):
    """qsa_teacher_recall: share of each row's teacher mass on its kept blocks
    and its own block; returns recall [B][Nq] float32."""
    B, L, Nq = shp.batch, shp.max_len, shp.n_query
    dev = teacher.device
    _need(lens, "lens", (B,), _I32)
    _need(teacher, "teacher", (B, Nq, L // BLOCK), (torch.float32,))
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    if recall is None:
        recall = torch.empty((B, Nq), dtype=torch.float32, device=dev)
    _need(recall, "recall", (B, Nq), (torch.float32,))
    st = load_library().qsa_teacher_recall(ctypes.byref(shp), _p(lens), _p(teacher), _p(sel),
                                           _p(n_sel), _p(recall), _stream(dev))
    _check(st, "qsa_teacher_recall")
    return recall


def _f32(t, name, shape_):
    _need(t, name, shape_, (torch.float32,))


def sparse_attend_backward(shp: QsaShape, q, k, v, lens, sel, n_sel, out, lse, d_out,
                           dq=None, dk=None, dv=None):
    """qsa_sparse_attend_backward.  dq is written; dk and dv (float32) are
    added into (zero-filled here when not given).  Returns (dq, dk, dv)."""
    B, L, Nq, Hq, Hkv = shp.batch, shp.max_len, shp.n_query, shp.q_heads, shp.kv_heads
    dev = q.device
    _need(q, "q", (B, Nq, Hq, HEAD_DIM), _BF)
    _need(k, "k", (B, L, Hkv, HEAD_DIM), _BF)
    _need(v, "v", (B, L, Hkv, HEAD_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    _need(sel, "sel", (B, Nq, TOPK), _I32)
    _need(n_sel, "n_sel", (B, Nq), _I32)
    _need(out, "out", (B, Nq, Hq, HEAD_DIM), _BF)
    _f32(lse, "lse", (B, Nq, Hq))
    _need(d_out, "d_out", (B, Nq, Hq, HEAD_DIM), _BF)
    if dq is None:
        dq = torch.empty((B, Nq, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros((B, L, Hkv, HEAD_DIM), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.zeros((B, L, Hkv, HEAD_DIM), dtype=torch.float32, device=dev)
    _f32(dq, "dq", (B, Nq, Hq, HEAD_DIM))
    _f32(dk, "dk", (B, L, Hkv, HEAD_DIM))
    _f32(dv, "dv", (B, L, Hkv, HEAD_DIM))
    st = load_library().qsa_sparse_attend_backward(
        ctypes.byref(shp), _p(q), _p(k), _p(v), _p(lens), _p(sel), _p(n_sel), _p(out), _p(lse),
        _p(d_out), _p(dq), _p(dk), _p(dv), _stream(dev))
    _check(st, "qsa_sparse_attend_backward")
    return dq, dk, dv


def index_scores_backward(shp: QsaShape, q_idx, k_cmp, lens, d_scores, dq_idx=None,
                          dk_cmp=None):
    """qsa_index_scores_backward; dq_idx and dk_cmp (float32) are added into
    (zero-filled here when not given).  Returns (dq_idx, dk_cmp)."""
    B, L, Nq = shp.batch, shp.max_len, shp.n_query
    dev = q_idx.device
    _need(q_idx, "q_idx", (B, Nq, IDX_HEADS, IDX_DIM), _BF)
    _need(k_cmp, "k_cmp", (B, L // BLOCK, IDX_DIM), _BF)
    _need(lens, "lens", (B,), _I32)
    _f32(d_scores, "d_scores", (B, Nq, L // BLOCK))
    if dq_idx is None:
        dq_idx = torch.zeros((B, Nq, IDX_HEADS, IDX_DIM), dtype=torch.float32, device=dev)
    if dk_cmp is None:
        dk_cmp = torch.zeros((B, L // BLOCK, IDX_DIM), dtype=torch.float32, device=dev)
    _f32(dq_idx, "dq_idx", (B, Nq, IDX_HEADS, IDX_DIM))
    _f32(dk_cmp, "dk_cmp", (B, L // BLOCK, IDX_DIM))
    st = load_library().qsa_index_scores_backward(ctypes.byref(shp), _p(q_idx), _p(k_cmp),
                                                  _p(lens), _p(d_scores), _p(dq_idx),
                                                  _p(dk_cmp), _stream(dev))
    _check(st, "qsa_index_scores_backward")
    return dq_idx, dk_cmp


def compress_keys_backward(shp: QsaShape, lens, dk_cmp, dk_idx=None):
    """qsa_compress_keys_backward; dk_idx (float32) is added into."""
    B, L = shp.batch, shp.max_len
    dev = dk_cmp.device
    _need(lens, "lens", (B,), _I32)
    _f32(dk_cmp, "dk_cmp", (B, L // BLOCK, IDX_DIM))
    if dk_idx is None:
        dk_idx = torch.zeros((B, L, IDX_DIM), dtype=torch.float32, device=dev)
    _f32(dk_idx, "dk_idx", (B, L, IDX_DIM))
    st = load_library().qsa_compress_keys_backward(ctypes.byref(shp), _p(lens), _p(dk_cmp),
                                                   _p(dk_idx), _stream(dev))
    _check(st, "qsa_compress_keys_backward")
    return dk_idx


class KernelTimer:
    """Times every kernel the library launches on this thread with a pair of
    HIP events carried by the kernel's own dispatch (qsa_profile_attach), for
    benchmarks.  Use as a context manager; afterwards `records()` lists
    (kernel name, milliseconds of execution) in launch order."""

    def __init__(self, max_launches: int = 512):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_launches)]
        for e in self.events:  # materialise the HIP events
            e.record()
        torch.cuda.synchronize()
        self._handles = (ctypes.c_void_p * len(self.events))(
            *[ctypes.c_void_p(e.cuda_event) for e in self.events])
        self._names = []

    def __enter__(self):
        _check(load_library().qsa_profile_attach(self._handles, len(self.events)),
               "qsa_profile_attach")
        return self

    def __exit__(self, *exc):
        lib = load_library()
        n = lib.qsa_profile_detach()
        self._names = [lib.qsa_profile_kernel_name(i).decode() for i in range(n)]
        return False

    def records(self):
        torch.cuda.synchronize()
        return [(name, self.events[2 * i].elapsed_time(self.events[2 * i + 1]))
                for i, name in enumerate(self._names)]

