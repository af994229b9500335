"""The C-ABI library: it loads, exports every symbol include/qsa.h declares,
and rejects bad host-visible arguments before touching a device.  No compute
call is made here (CPU-only)."""
import ctypes
import os
import re

import pytest

import learned_sparse_attention_qsa_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if fn.endswith(".h"):
            with open(os.path.join(inc, fn)) as f:
                names |= set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", f.read()))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = Q.load_library()
    declared = header_symbols()
    assert len(declared) == 26
    assert sorted(Q.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    seen = set()
    for st in range(8):
        s = Q.status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert Q.status_string(99) == "unknown status"


def test_workspace_sizes():
    dec = Q.shape(4, 1 << 20, 4, 32, 4)
    assert Q.workspace_bytes(dec, Q.OP_COMPRESS) == 0
    assert Q.workspace_bytes(dec, Q.OP_EXPAND) == 0
    # the decode shape takes the score table engine: 16 rows x 262,144 blocks x 4 B
    assert Q.workspace_bytes(dec, Q.OP_INDEX_TOPK) >= 16 * 262144 * 4
    assert Q.workspace_bytes(dec, Q.OP_FORWARD) >= Q.workspace_bytes(dec, Q.OP_INDEX_TOPK)
    scan = Q.shape(4, 1 << 20, 4, 32, 4, flags=Q.FLAG_TOPK_SCAN)
    # the scan engine: candidate segments of 64 slices x 512 keys per row
    assert Q.workspace_bytes(scan, Q.OP_INDEX_TOPK) == 16 * 64 * (512 * 8 + 4)
    # beyond a 512 MiB score table the decode shape takes the scan engine
    long_dec = Q.shape(4, 1 << 26, 4, 32, 4)   # a 1 GiB table: 2,048 slices of 8,192 blocks
    assert Q.workspace_bytes(long_dec, Q.OP_INDEX_TOPK) == 16 * 2048 * (512 * 8 + 4)
    pre = Q.shape(1, 1 << 20, 16384, 32, 4)
    # prefill uses the streaming engine: no score table (would be 16 GiB)
    assert Q.workspace_bytes(pre, Q.OP_INDEX_TOPK) < 3 << 30
    assert Q.workspace_bytes(pre, Q.OP_SPARSE_ATTEND) == 0
    forced = Q.shape(1, 1 << 16, 16384, 32, 4, flags=Q.FLAG_TOPK_TABLE)
    assert Q.workspace_bytes(forced, Q.OP_INDEX_TOPK) >= 16384 * 16384 * 4
    assert Q.workspace_bytes(Q.shape(1, 6, 1, 8, 1), Q.OP_INDEX_TOPK) == 0  # invalid shape


BAD_SHAPES = [
    Q.shape(1, 6, 1, 8, 1),          # max_len not a multiple of 4
    Q.shape(1, 0, 0, 8, 1),          # empty cache
    Q.shape(1, 8, 9, 8, 1),          # more queries than positions
    Q.shape(1, 8, 1, 8, 3),          # Hq % Hkv != 0
    Q.shape(1, 8, 1, 0, 1),          # no heads
    Q.shape(-1, 8, 1, 8, 1),         # negative batch
    Q.shape(1, 8, 1, 130, 2),        # group of 65 heads
    Q.shape(1, 8, 1, 8, 1, flags=3),  # both engines forced
    Q.shape(1, 8, 1, 8, 1, flags=8),  # unknown flag
    Q.shape(1, 8, 1, 8, 1, flags=5),  # table and scan engines forced
    Q.shape(1, 8, 1, 8, 1, flags=6),  # stream and scan engines forced
    Q.shape(1, (1 << 30) + 4, 1, 8, 1),  # beyond 2^30 tokens
]

FAKE = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced: errors come first
MISALIGNED = ctypes.c_void_p((1 << 20) + 8)


def call(name, shp, *ptrs):
    lib = Q.load_library()
    return getattr(lib, name)(ctypes.byref(shp), *ptrs)


@pytest.mark.parametrize("shp", BAD_SHAPES)
def test_bad_shapes_rejected(shp):
    assert call("qsa_index_topk", shp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == Q.ERR_SHAPE
    assert call("qsa_compress_keys", shp, FAKE, FAKE, None, FAKE, None) == Q.ERR_SHAPE
    assert call("qsa_sparse_attend", shp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                1 << 30, None) == Q.ERR_SHAPE
    assert call("qsa_dense_gqa_decode", shp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                None) == Q.ERR_SHAPE


def test_null_and_alignment_rejected():
    shp = Q.shape(2, 4096, 4, 8, 1)
    assert call("qsa_compress_keys", shp, None, FAKE, None, FAKE, None) == Q.ERR_NULL
    assert call("qsa_compress_keys", shp, MISALIGNED, FAKE, None, FAKE, None) == Q.ERR_ALIGN
    assert call("qsa_index_topk", shp, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == Q.ERR_NULL
    assert call("qsa_expand_blocks", shp, FAKE, FAKE, FAKE, None, FAKE, None) == Q.ERR_NULL
    assert call("qsa_sparse_attend", shp, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                1 << 30, None) == Q.ERR_ALIGN
    # forward: sel_out without n_sel_out
    assert call("qsa_forward", shp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                FAKE, None, FAKE, 1 << 30, None) == Q.ERR_NULL


def test_workspace_rejected():
    shp = Q.shape(2, 4096, 4, 8, 1)
    need = Q.workspace_bytes(shp, Q.OP_INDEX_TOPK)
    assert need > 0
    assert call("qsa_index_topk", shp, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == Q.ERR_WORKSPACE
    assert call("qsa_index_topk", shp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == Q.ERR_WORKSPACE
    assert call("qsa_index_topk", shp, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, need, None) == Q.ERR_ALIGN
    dn = Q.workspace_bytes(shp, Q.OP_DENSE_DECODE)
    assert call("qsa_dense_gqa_decode", shp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, dn - 1,
                None) == Q.ERR_WORKSPACE


def test_empty_batches_are_noops():
    # B = 0 or Nq = 0: nothing to do, OK without touching pointers or a device
    assert call("qsa_index_topk", Q.shape(0, 8, 1, 8, 1), None, None, None, None, None, None, 0, None) == Q.OK
    assert call("qsa_sparse_attend", Q.shape(3, 8, 0, 8, 1), None, None, None, None, None, None,
                None, None, None, 0, None) == Q.OK
    assert call("qsa_compress_keys", Q.shape(0, 8, 1, 8, 1), None, None, None, None, None) == Q.OK


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(Q, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        Q.load_library(str(tmp_path / "nope.so"))


def test_ceiling_probes_reject_bad_arguments():
    lib = Q.load_library()
    sink = FAKE
    assert lib.qsa_ceil_stream_read(None, 1024, 4, sink, None) == Q.ERR_NULL
    assert lib.qsa_ceil_stream_read(MISALIGNED, 1024, 4, sink, None) == Q.ERR_ALIGN
    assert lib.qsa_ceil_stream_read(FAKE, 1000, 4, sink, None) == Q.ERR_ALIGN
    assert lib.qsa_ceil_stream_read(FAKE, 1024, 0, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_stream_read(FAKE, 0, 4, sink, None) == Q.OK
    assert lib.qsa_ceil_gather(FAKE, FAKE, 10, 1000, 4, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_gather(FAKE, FAKE, 10, 8, 4, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_gather(FAKE, FAKE, -1, 256, 4, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_gather(FAKE, None, 10, 256, 4, sink, None) == Q.ERR_NULL
    assert lib.qsa_ceil_gather(FAKE, FAKE, 0, 256, 4, sink, None) == Q.OK
    assert lib.qsa_ceil_lds_atomic(0, 1, 4, 16, None, None) == Q.ERR_NULL
    assert lib.qsa_ceil_lds_atomic(2, 1, 4, 16, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_lds_atomic(0, 3, 4, 16, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_lds_atomic(1, 64, 0, 16, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_lds_atomic(1, 64, 4, 0, sink, None) == Q.ERR_SHAPE
    assert lib.qsa_ceil_lds_atomic(1, 64, 4, 4097, sink, None) == Q.ERR_SHAPE


def test_noalloc_rejects_shapes_beyond_its_scratch_before_any_launch():
    lib = Q.load_library()
    big = Q.shape(1, 1 << 20, 16384, 32, 4)   # a 16K-query prefill chunk's workspace
    assert Q.workspace_bytes(big, Q.OP_FORWARD) > Q.NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 12 + [None]
    assert lib.qsa_forward_noalloc(ctypes.byref(big), *args) == Q.ERR_SCRATCH
    assert lib.qsa_forward_noalloc(None, *args) == Q.ERR_NULL
    dec = Q.shape(4, 1 << 20, 4, 32, 4)        # the 1M-context decode fits
    assert 0 < Q.workspace_bytes(dec, Q.OP_FORWARD) <= Q.NOALLOC_SCRATCH_BYTES
    bad = Q.shape(1, 6, 1, 8, 1)               # max_len not a multiple of 4
    assert lib.qsa_forward_noalloc(ctypes.byref(bad), *args) == Q.ERR_SHAPE
    assert Q.status_string(Q.ERR_SCRATCH).startswith("shape needs more scratch")


def test_paged_descriptor_rejected_before_any_launch():
    lib = Q.load_library()
    shp = Q.shape(2, 4096, 4, 8, 1)
    table = Q.QsaPagedKV(FAKE.value, 16, 256, 600)    # 256 pages of 16 tokens cover 4,096
    ok = ctypes.byref(table)
    ws = Q.workspace_bytes(shp, Q.OP_SPARSE_ATTEND)

    def attend(kv):
        return lib.qsa_sparse_attend_paged(ctypes.byref(shp), FAKE, FAKE, FAKE, kv, FAKE, FAKE,
                                           FAKE, FAKE, None, FAKE, max(ws, 16), None)

    assert attend(None) == Q.ERR_NULL
    for ps, mp, npg in ((12, 512, 600), (0, 256, 600), (1 << 21, 1, 1), (16, 255, 600),
                        (16, 256, 0), (16, 0, 600)):
        bad = Q.QsaPagedKV(FAKE.value, ps, mp, npg)
        assert attend(ctypes.byref(bad)) == Q.ERR_SHAPE, (ps, mp, npg)
    mis = Q.QsaPagedKV(FAKE.value + 2, 16, 256, 600)
    assert attend(ctypes.byref(mis)) == Q.ERR_ALIGN
    assert lib.qsa_dense_gqa_decode_paged(ctypes.byref(shp), FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                          None, FAKE, 1 << 30, None) == Q.ERR_NULL
    assert lib.qsa_forward_paged(ctypes.byref(shp), *([FAKE] * 7), None, *([FAKE] * 5),
                                 FAKE, 1 << 30, None) == Q.ERR_NULL
    short = Q.QsaPagedKV(FAKE.value, 64, 63, 600)     # 63 pages of 64 tokens < 4,096
    assert lib.qsa_dense_gqa_prefill(ctypes.byref(shp), FAKE, FAKE, FAKE, ctypes.byref(short),
                                     FAKE, FAKE, None, None) == Q.ERR_SHAPE
    # prefill without a table takes contiguous caches; empty work is a no-op
    assert lib.qsa_dense_gqa_prefill(ctypes.byref(Q.shape(3, 8, 0, 8, 1)), None, None, None,
                                     None, None, None, None, None) == Q.OK
    assert lib.qsa_dense_gqa_prefill(ctypes.byref(shp), None, FAKE, FAKE, ok, FAKE, FAKE,
                                     None, None) == Q.ERR_NULL


def test_debug_entry_points_without_a_device():
    from learned_sparse_attention_qsa_amd import build as B
    lib = Q.load_library()
    assert lib.qsa_debug_build() == 0
    n = ctypes.c_uint64(7)
    assert lib.qsa_debug_guard_hits(ctypes.byref(n)) == Q.OK and n.value == 0
    assert lib.qsa_debug_guard_hits(None) == Q.ERR_NULL
    if not os.path.exists(B.DEBUG_LIB):
        B.build_debug()
    dbg = ctypes.CDLL(B.DEBUG_LIB)
    dbg.qsa_debug_build.restype = ctypes.c_int32
    dbg.qsa_debug_guard_hits.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    assert dbg.qsa_debug_build() == 1
    assert dbg.qsa_debug_guard_hits(None) == Q.ERR_NULL
