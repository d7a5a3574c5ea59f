"""Pins of the oracle's SnapKV++ stage-1 eviction (O2).  The paper's abstract
names SnapKV++ (adaptive pooling size, GQA compatibility); the atlas.scime.ai
summary ("Approach") gives a large pooling kernel and group-level selection;
"RocketKV-adapted" ("The problem this solves") says stage 1 reuses SnapKV's
observation-window scoring.  Checks:
  - the scores equal the window queries' causal softmax probabilities summed
    over queries and heads, against torch's fp64 softmax;
  - pooling equals scipy's maximum filter; the kept set equals numpy's sort
    of the pooled scores plus the window;
  - G = 1 with pooling 1 is plain SnapKV scoring; the group score is the sum
    of its heads' scores; keep >= L keeps everything; a planted needle
    survives."""
import numpy as np
import pytest
import scipy.ndimage
import torch

import oracle
from sparse_kv_cache_hsa_amd import synth


def make(G, w, L, d, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    q = synth.to_bits((torch.randn((G, w, d), generator=g)).to(dtype))
    k = synth.to_bits((torch.randn((L, d), generator=g) * 1.5).to(dtype))
    return q, k


def to_f64(a):
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return torch.from_numpy(a.astype(np.float64))


def reference_scores(q, k, scale, causal=True):
    G, w, d = q.shape
    L = k.shape[0]
    qt, kt = to_f64(q), to_f64(k)
    A = torch.zeros(L - w, dtype=torch.float64)
    for j in range(G):
        for i in range(w):
            last = L - w + i if causal else L - 1
            p = torch.softmax((kt[:last + 1] @ qt[j, i]) * scale, dim=0)
            A += p[:L - w]
    return A.numpy()


def expected_keep(pooled, keep, L, w):
    order = np.lexsort((np.arange(len(pooled)), -pooled.astype(np.float64)))
    return np.concatenate([np.sort(order[:keep - w]), np.arange(L - w, L)])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("G,w,L", [(1, 4, 90), (2, 8, 300), (4, 16, 257)])
def test_scores_are_summed_causal_softmax(dtype, G, w, L):
    d = 16
    q, k = make(G, w, L, d, G * 100 + L, dtype)
    scale = synth.head_dim_scale(d)
    kept, A, pooled = oracle.snapkv_group(q, k, 5, w + 20, scale)
    ref = reference_scores(q, k, scale)
    np.testing.assert_allclose(A, ref, rtol=2e-5, atol=1e-9)
    # the causal mask matters at this size: dropping it changes the scores
    assert np.abs(reference_scores(q, k, scale, causal=False) - ref).max() > 1e-4 * ref.max()


@pytest.mark.parametrize("pool", [1, 3, 7, 63])
def test_pooling_is_max_filter_and_keep_is_sorted_topk(pool):
    G, w, L, d = 2, 8, 400, 16
    q, k = make(G, w, L, d, pool)
    keep = 60
    kept, A, pooled = oracle.snapkv_group(q, k, pool, keep, 0.25)
    np.testing.assert_array_equal(
        pooled, scipy.ndimage.maximum_filter1d(A, size=pool, mode="nearest"))
    np.testing.assert_array_equal(kept, expected_keep(pooled, keep, L, w))
    assert len(kept) == keep and np.all(np.diff(kept) > 0)


def test_plain_snapkv_special_case():
    # one query head per KV head and no pooling: keep the top window scores
    q, k = make(1, 6, 200, 8, 7)
    kept, A, pooled = oracle.snapkv_group(q, k, 1, 40, 0.3)
    np.testing.assert_array_equal(pooled, A)
    np.testing.assert_array_equal(kept, expected_keep(A, 40, 200, 6))


def test_group_score_is_sum_of_head_scores():
    G, w, L, d = 4, 8, 150, 16
    q, k = make(G, w, L, d, 9)
    _, A, _ = oracle.snapkv_group(q, k, 3, 30, 0.25)
    acc = np.zeros(L - w, np.float32)
    for j in range(G):
        _, Aj, _ = oracle.snapkv_group(q[j:j + 1], k, 3, 30, 0.25)
        acc = acc + Aj
    np.testing.assert_array_equal(A, acc)


def test_keep_at_least_prompt_keeps_everything():
    q, k = make(2, 8, 50, 8, 11)
    for keep in (50, 80):
        kept, _, _ = oracle.snapkv_group(q, k, 63, keep, 0.3)
        np.testing.assert_array_equal(kept, np.arange(50))


def test_keep_equal_window_keeps_only_window():
    q, k = make(2, 8, 50, 8, 12)
    kept, _, _ = oracle.snapkv_group(q, k, 3, 8, 0.3)
    np.testing.assert_array_equal(kept, np.arange(42, 50))


def test_planted_needle_survives():
    G, w, L, d = 4, 16, 2000, 32
    q, k = make(G, w, L, d, 13)
    u = np.random.default_rng(0).standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    q = q + 2.0 * np.sqrt(d) * u                     # window queries point at u
    k[777] = 3.0 * np.sqrt(d) * u                    # the needle key
    kept, _, pooled = oracle.snapkv_group(q.astype(np.float32), k, 63, 64, 1 / np.sqrt(d))
    assert 777 in kept
    assert np.argmax(pooled) in range(777 - 31, 777 + 32)


def test_invalid_arguments():
    q, k = make(2, 8, 50, 8, 1)
    with pytest.raises(oracle.OracleError):
        oracle.snapkv_group(q, k, 4, 20, 0.3)        # even pooling kernel
    with pytest.raises(oracle.OracleError):
        oracle.snapkv_group(q, k, 3, 5, 0.3)         # keep below the window


# ---- chunked prefill (the budget re-enforced across calls) ------------------
def _chunks(G, w, d, lens, seed, dtype=torch.float32):
    qs, ks = [], []
    for t, n in enumerate(lens):
        q, k = make(G, w, n, d, seed + t, dtype)
        qs.append(q)
        ks.append(k)
    return qs, ks


def test_chunked_single_chunk_is_plain_eviction():
    qs, ks = _chunks(4, 8, 32, [400], 71)
    (kept, pooled, pos), = oracle.snapkv_chunked_group(qs, ks, 7, [100], 0.2)
    k2, _, p2 = oracle.snapkv_group(qs[0], ks[0], 7, 100, 0.2)
    np.testing.assert_array_equal(kept, k2)
    np.testing.assert_array_equal(pos, k2)
    np.testing.assert_array_equal(pooled, p2)


def test_chunked_budget_window_and_order():
    """After every call: min(keep, rows so far + chunk) rows kept, positions
    ascending, the chunk's last w rows kept, earlier positions only from rows
    kept before (evicted rows never come back)."""
    w, lens, keeps = 8, [300, 120, 500, 90], [150, 150, 200, 120]
    qs, ks = _chunks(2, w, 32, lens, 81)
    res = oracle.snapkv_chunked_group(qs, ks, 5, keeps, 0.2)
    held, start = set(), 0
    for (kept, _, pos), n, keep in zip(res, lens, keeps):
        L = len(held) + n
        assert len(pos) == min(keep, L)
        assert np.all(np.diff(pos) > 0)
        end = start + n
        assert set(range(end - w, end)) <= set(pos.tolist())
        assert set(p for p in pos.tolist() if p < start) <= held
        held, start = set(pos.tolist()), end


def test_chunked_without_pressure_keeps_everything():
    lens = [50, 60, 70]
    qs, ks = _chunks(1, 4, 16, lens, 91)
    res = oracle.snapkv_chunked_group(qs, ks, 3, [1000] * 3, 0.25)
    np.testing.assert_array_equal(res[-1][2], np.arange(sum(lens)))


def test_chunked_second_call_scores_the_concatenation():
    """Call 2 scores exactly the kept rows of call 1 followed by chunk 2,
    against the window of chunk 2 (fp64 causal softmax reference)."""
    G, w, d = 2, 8, 32
    qs, ks = _chunks(G, w, d, [200, 100], 101)
    res = oracle.snapkv_chunked_group(qs, ks, 1, [80, 90], 0.2)
    cat = np.concatenate([ks[0][res[0][0]], ks[1]])
    ref = reference_scores(qs[1], cat, 0.2)
    np.testing.assert_allclose(res[1][1], ref, rtol=2e-5, atol=1e-9)
