"""Pins of the oracle's page summaries (O3): element-wise max/min per page
("RocketKV-adapted -- Two-Stage Compression", section "Where it sits"),
checked against numpy's reductions, and incremental append bit-identical to
a rebuild, token by token and in chunks (section "Evidence")."""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_cache_hsa_amd import synth


def rows(n, d, dtype, seed):
    x = torch.randn((n, d), generator=torch.Generator().manual_seed(seed)) * 3
    return synth.to_bits(x.to(dtype))


def as_float(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,P", [(1, 16), (16, 16), (17, 16), (100, 8), (257, 32), (50, 1)])
def test_rebuild_matches_numpy_reduction(dtype, n, P):
    d = 24
    k = rows(n, d, dtype, n * 7 + P)
    smax, smin = oracle.summaries_rebuild(k, P)
    kf = as_float(k)
    assert smax.shape == ((n + P - 1) // P, d)
    for p in range(smax.shape[0]):
        page = kf[p * P:min(n, p * P + P)]
        np.testing.assert_array_equal(as_float(smax[p]), page.max(axis=0))
        np.testing.assert_array_equal(as_float(smin[p]), page.min(axis=0))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("P", [1, 5, 16])
def test_append_token_by_token_equals_rebuild(dtype, P):
    n, d = 123, 16
    k = rows(n, d, dtype, 11)
    np_ = (n + P - 1) // P
    smax = np.zeros((np_, d), k.dtype)
    smin = np.zeros((np_, d), k.dtype)
    for t in range(n):
        oracle.summaries_append(k, t, t + 1, P, smax, smin)
        rmax, rmin = oracle.summaries_rebuild(k[:t + 1], P)
        np.testing.assert_array_equal(smax[:rmax.shape[0]], rmax)
        np.testing.assert_array_equal(smin[:rmin.shape[0]], rmin)


@pytest.mark.parametrize("chunks", [[0, 7, 8, 40, 41, 200], [0, 64, 128, 200], [0, 3, 200]])
def test_append_chunks_equals_rebuild(chunks):
    P, d = 16, 8
    k = rows(200, d, torch.bfloat16, 5)
    smax = np.zeros((13, d), np.uint16)
    smin = np.zeros((13, d), np.uint16)
    for a, b in zip(chunks[:-1], chunks[1:]):
        oracle.summaries_append(k, a, b, P, smax, smin)
    rmax, rmin = oracle.summaries_rebuild(k, P)
    np.testing.assert_array_equal(smax, rmax)
    np.testing.assert_array_equal(smin, rmin)


def test_signed_zero_keeps_first_occurrence():
    # +0 and -0 compare equal; both routes must keep the earliest row's bits
    k = np.array([[0.0], [-0.0], [0.0], [-0.0], [-1.0], [-0.0]], dtype=np.float32)
    rmax, rmin = oracle.summaries_rebuild(k, 6)
    smax = np.zeros((1, 1), np.float32)
    smin = np.zeros((1, 1), np.float32)
    for t in range(6):
        oracle.summaries_append(k, t, t + 1, 6, smax, smin)
    assert smax.view(np.uint32)[0, 0] == rmax.view(np.uint32)[0, 0] == 0  # +0 (row 0)
    assert smin[0, 0] == rmin[0, 0] == -1.0


def test_values_invariant_to_row_order_within_page():
    P, d = 8, 32
    k = rows(64, d, torch.float32, 3)
    perm = np.concatenate([p * P + np.random.default_rng(p).permutation(P) for p in range(8)])
    a = oracle.summaries_rebuild(k, P)
    b = oracle.summaries_rebuild(k[perm], P)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
