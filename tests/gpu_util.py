"""Helpers for the GPU parity tests: host <-> device marshalling and the
tolerance check.  Expected values always come from oracle/."""
import numpy as np
import torch

import oracle as O

DEV = "cuda"
MAX_ABS = 2e-2
REL_L2 = 1e-2


def dev_bf16(a) -> torch.Tensor:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64_from_bf16(t: torch.Tensor) -> np.ndarray:
    return O.bf16_bits_to_f64(host_u16(t))


def check_close(got: np.ndarray, ref: np.ndarray, what: str = "out"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got))
    assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    return max_abs, rel


def padded_sel(res, B, Nq, lens):
    """Oracle selections as the library lays them out: [B][Nq][512] ascending,
    padded with -1, plus n_sel."""
    sel = np.full((B, Nq, O.TOPK), -1, dtype=np.int32)
    n_sel = np.zeros((B, Nq), dtype=np.int32)
    for (b, i), s in res["sel"].items():
        sel[b, i, :s.shape[0]] = s
        n_sel[b, i] = s.shape[0]
    return sel, n_sel


def padded_tok(res, B, Nq):
    tok = np.full((B, Nq, O.TOPK * O.BLOCK + O.BLOCK), -1, dtype=np.int32)
    n_tok = np.zeros((B, Nq), dtype=np.int32)
    for (b, i), t in res["tok"].items():
        tok[b, i, :t.shape[0]] = t
        n_tok[b, i] = t.shape[0]
    return tok, n_tok


def paged_pools_dev(k, v, lens, page, seed):
    """Page pools [n_pages][page][Hkv][128] holding the device caches k, v
    ([B][L][Hkv][128]) under a seeded random page order, and their page
    table (a Q.PagedKV)."""
    import learned_sparse_attention_qsa_amd as Q
    B, L, Hkv, D = k.shape
    max_pages = (L + page - 1) // page
    need = [(int(n) + page - 1) // page for n in lens]
    n_pages = max(1, sum(need))
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(n_pages, generator=g)
    table = torch.zeros((B, max_pages), dtype=torch.int32)
    k_pool = torch.empty((n_pages, page, Hkv, D), dtype=k.dtype, device=k.device)
    v_pool = torch.empty_like(k_pool)
    off = 0
    for b in range(B):
        n, full = need[b], int(lens[b]) // page
        pid = ids[off:off + n]
        off += n
        table[b, :n] = pid.to(torch.int32)
        if full:
            idx = pid[:full].to(k.device)
            k_pool[idx] = k[b, :full * page].view(full, page, Hkv, D)
            v_pool[idx] = v[b, :full * page].view(full, page, Hkv, D)
        if n > full:
            rest = int(lens[b]) - full * page
            k_pool[int(pid[full]), :rest] = k[b, full * page:full * page + rest]
            v_pool[int(pid[full]), :rest] = v[b, full * page:full * page + rest]
    return k_pool, v_pool, Q.PagedKV(table.to(k.device), page, n_pages)
