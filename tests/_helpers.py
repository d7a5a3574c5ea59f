"""Shared test plumbing: paged caches on the device, oracle-side views of the
same bytes, and the comparison rules (index sets bit-exact; stage-1 kept
sets bit-exact except boundary swaps whose oracle score gap is under 1e-6
relative, which are counted; outputs within 1e-3 absolute)."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from sparse_kv_cache_hsa_amd import synth

OUT_ATOL = 1e-3
NEAR_TIE_REL = 1e-6


def lib():
    from sparse_kv_cache_hsa_amd import rkv
    rkv.load_library()
    return rkv


def make_cache(Hkv: int, d: int, P: int, max_pages: int, pages_per_seq, dtype, seed: int,
               device="cuda"):
    """Empty paged cache with a seeded, shuffled block layout."""
    rkv = lib()
    B = len(pages_per_seq)
    table, nblk = synth.page_table(seed, B, pages_per_seq, max_pages)
    kp = torch.zeros((nblk, Hkv, P, d), dtype=dtype, device=device)
    vp = torch.zeros_like(kp)
    cache = rkv.PagedCache(kp, vp, table.to(device))
    summ = torch.zeros((B, Hkv, 2, d, max_pages), dtype=dtype, device=device)
    return cache, summ


def fill_cache(g, cache, summ, K, V, lens):
    """Writes logical rows K/V [B, Hkv, Lmax, d] (device) for rows [0, lens)
    into the cache and summaries with the library's append."""
    rkv = lib()
    B = K.shape[0]
    n_old = torch.zeros(B, dtype=torch.int32, device=K.device)
    n_new = torch.tensor(lens, dtype=torch.int32, device=K.device)
    rkv.rkv_append_summaries(g, cache, n_old, n_new, max(1, K.shape[2]), summ, k_src=K, v_src=V)


def bits(t: torch.Tensor):
    return synth.to_bits(t)


def oracle_summaries(k_rows_bits, P, NP, d):
    if NP == 0:
        z = np.zeros((1, d), k_rows_bits.dtype)
        return z, z.copy()
    return oracle.summaries_rebuild(k_rows_bits, P)


def gpu_summaries(summ: torch.Tensor, b: int, h: int, NP: int):
    """[NP, d] max and min of sequence b, head h from the device layout."""
    s = summ[b, h, :, :, :NP].transpose(1, 2).contiguous()
    return bits(s[0]), bits(s[1])


def check_kept(gpu_kept: np.ndarray, ora_kept: np.ndarray, ora_pooled: np.ndarray, w: int):
    """Stage-1 kept sets: the window tail must match; prefix mismatches are
    allowed only as boundary swaps with an oracle score gap < 1e-6 relative.
    Returns the number of such swaps."""
    keep = len(ora_kept)
    assert len(gpu_kept) == keep
    np.testing.assert_array_equal(gpu_kept[keep - w:], ora_kept[keep - w:])
    K = keep - w
    g, o = set(gpu_kept[:K].tolist()), set(ora_kept[:K].tolist())
    diff = g ^ o
    if not diff:
        np.testing.assert_array_equal(gpu_kept, ora_kept)
        return 0
    thr = float(ora_pooled[ora_kept[:K]].min())
    for t in diff:
        gap = abs(float(ora_pooled[t]) - thr)
        assert gap <= NEAR_TIE_REL * abs(thr), (t, float(ora_pooled[t]), thr)
    assert np.all(np.diff(gpu_kept) > 0)
    return len(diff)


def max_abs_err(gpu_out: torch.Tensor, ora_out: np.ndarray) -> float:
    return float(np.abs(gpu_out.detach().cpu().double().numpy() - ora_out).max())


def scale_for(d: int) -> float:
    return synth.head_dim_scale(d)


def n_pages(n: int, P: int) -> int:
    return (n + P - 1) // P


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["OUT_ATOL", "NEAR_TIE_REL", "lib", "make_cache", "fill_cache", "bits",
           "oracle_summaries", "gpu_summaries", "check_kept", "max_abs_err", "scale_for",
           "n_pages", "ceil_div", "math"]
