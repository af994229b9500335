"""qsa_forward_noalloc against qsa_forward: the same selections bit for bit
and the same outputs within the attention tolerance, on two calls in a row
(the second with a smaller input, so it runs on scratch the first one left
behind), and no device memory allocated by the calls.  The entry point's
first call on a device takes the device address of the library's scratch
array, and the runtime places the array then; that set-up call comes first,
and the free device memory must not change across the compared calls."""
import sys

import numpy as np
import pytest
import torch

import learned_sparse_attention_qsa_amd as Q
import workloads as W
from gpu_util import check_close, dev_bf16, dev_i32, host_f64_from_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(w):
    shp = Q.shape(w.batch, w.max_len, w.n_query, w.q_heads, w.kv_heads)
    t = {n: dev_bf16(getattr(w, n)) for n in ("q_idx", "k_idx", "q", "k", "v")}
    t["lens"] = dev_i32(w.lens)
    return shp, t


def outputs(w):
    B, Nq, Hq = w.batch, w.n_query, w.q_heads
    return (torch.empty((B, Nq, Hq, 128), dtype=torch.bfloat16, device="cuda"),
            torch.empty((B, Nq, Hq), dtype=torch.float32, device="cuda"),
            torch.empty((B, Nq, 512), dtype=torch.int32, device="cuda"),
            torch.empty((B, Nq), dtype=torch.int32, device="cuda"),
            torch.zeros((w.batch, w.max_len // 4, 64), dtype=torch.bfloat16, device="cuda"))


def test_noalloc_matches_forward_twice_second_smaller():
    cases = [W.make_custom(501, [40001, 9000, 70002], 4, 32, 4),   # decode-shaped, 3 sequences
             W.make_custom(502, [6003], 2, 16, 2)]                 # then a smaller one
    runs = []
    for w in cases:
        shp, t = inputs(w)
        need = Q.workspace_bytes(shp, Q.OP_FORWARD)
        assert 0 < need <= Q.NOALLOC_SCRATCH_BYTES
        ref = outputs(w)
        got = outputs(w)
        runs.append((w, shp, t, ref, got))
    # reference results through qsa_forward
    for w, shp, t, ref, _ in runs:
        say(f"forward: lens {list(w.lens)}, {w.n_query} queries")
        out, lse, sel, n_sel, k_cmp = ref
        Q.forward(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], t["lens"],
                  out=out, lse=lse, sel=sel, n_sel=n_sel)
    torch.cuda.synchronize()
    # set-up call (first on this device): the smaller case, into spare outputs
    w, shp, t, _, _ = runs[1]
    spare = outputs(w)
    Q.forward_noalloc(shp, t["q_idx"], t["k_idx"], spare[4], t["q"], t["k"], t["v"], t["lens"],
                      spare[0])
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for w, shp, t, _, got in runs:
        say(f"noalloc: lens {list(w.lens)}, {w.n_query} queries")
        out, lse, sel, n_sel, k_cmp = got
        Q.forward_noalloc(shp, t["q_idx"], t["k_idx"], k_cmp, t["q"], t["k"], t["v"], t["lens"],
                          out, lse=lse, sel=sel, n_sel=n_sel)
        torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device memory changed by {free0 - free1} bytes"
    for w, shp, t, ref, got in runs:
        r_out, r_lse, r_sel, r_nsel, r_kc = ref
        g_out, g_lse, g_sel, g_nsel, g_kc = got
        np.testing.assert_array_equal(g_nsel.cpu().numpy(), r_nsel.cpu().numpy())
        np.testing.assert_array_equal(g_sel.cpu().numpy(), r_sel.cpu().numpy())
        np.testing.assert_array_equal(g_kc.view(torch.int16).cpu().numpy(),
                                      r_kc.view(torch.int16).cpu().numpy())
        check_close(host_f64_from_bf16(g_out), host_f64_from_bf16(r_out))
        np.testing.assert_allclose(g_lse.cpu().numpy(), r_lse.cpu().numpy(), atol=2e-2, rtol=0)
