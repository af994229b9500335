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
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libqsa.so")

IDX_HEADS = 4
IDX_DIM = 64
BLOCK = 4
TOPK = 512
HEAD_DIM = 128
MAX_TOK = TOPK * BLOCK + BLOCK

OK, ERR_NULL, ERR_ALIGN, ERR_SHAPE, ERR_WORKSPACE, ERR_DEVICE, ERR_HIP = range(7)
OP_COMPRESS, OP_INDEX_TOPK, OP_EXPAND, OP_SPARSE_ATTEND, OP_FORWARD, OP_DENSE_DECODE = range(6)
FLAG_TOPK_TABLE = 1
FLAG_TOPK_STREAM = 2

# Every symbol include/qsa.h declares.
EXPORTS = (
    "qsa_workspace_bytes",
    "qsa_status_string",
    "qsa_compress_keys",
    "qsa_index_topk",
    "qsa_expand_blocks",
    "qsa_sparse_attend",
    "qsa_forward",
    "qsa_dense_gqa_decode",
    "qsa_profile_attach",
    "qsa_profile_detach",
    "qsa_profile_kernel_name",
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
    for name in EXPORTS[2:8]:
        getattr(lib, name).restype = i32
    lib.qsa_profile_attach.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.qsa_profile_attach.restype = i32
    lib.qsa_profile_detach.argtypes = []
    lib.qsa_profile_detach.restype = i32
    lib.qsa_profile_kernel_name.argtypes = [i32]
    lib.qsa_profile_kernel_name.restype = ctypes.c_char_p
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


def default_scale() -> float:
    return 1.0 / math.sqrt(HEAD_DIM)
