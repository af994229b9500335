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
    with open(os.path.join(ROOT, "include", "qsa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = Q.load_library()
    declared = header_symbols()
    assert len(declared) == 11
    assert sorted(Q.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    seen = set()
    for st in range(7):
        s = Q.status_string(st)
        assert s and s not in seen
        seen.add(s)
    assert Q.status_string(99) == "unknown status"


def test_workspace_sizes():
    dec = Q.shape(4, 1 << 20, 4, 32, 4)
    assert Q.workspace_bytes(dec, Q.OP_COMPRESS) == 0
    assert Q.workspace_bytes(dec, Q.OP_EXPAND) == 0
    # the score table of the decode shape: 16 rows x 262,144 blocks x 4 B
    assert Q.workspace_bytes(dec, Q.OP_INDEX_TOPK) >= 16 * 262144 * 4
    assert Q.workspace_bytes(dec, Q.OP_FORWARD) >= Q.workspace_bytes(dec, Q.OP_INDEX_TOPK)
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
