"""Pins of the oracle's RocketKV-MT turn view (oracle.mt_turn_view): per
turn, SnapKV++ over the whole retained history with the turn's window
queries picks the turn's view, and nothing is deleted
("RocketKV: Accelerating Long-Context LLM Inference via Two-Stage KV Cache
Compression" (atlas.scime.ai), "Approach", "Limitations"; "RocketKV-adapted --
Two-Stage Compression", "Should you use this?").  Checks:
  - keep >= L makes the view the whole history, so HSA over the view is HSA
    over the full cache (the multi-turn workload without a filter);
  - the view is SnapKV++'s kept set of the same bytes, re-derived here from
    the scores by a numpy sort;
  - a row left out of turn 1's view returns in turn 2's when turn 2's
    queries point at it, while the chunked-prefill composition (stage-1
    budget re-enforced, evicted rows gone) can never bring it back."""
import numpy as np
import torch

import oracle
from sparse_kv_cache_hsa_amd import synth

G, w, d, P, POOL = 4, 8, 32, 8, 5


def rows(n, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return synth.to_bits(torch.randn((n, d), generator=g) * scale)


def queries(seed, direction=None, strength=0.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((G, w, d), generator=g)
    if direction is not None:
        q = q + strength * direction
    return synth.to_bits(q)


def test_keep_everything_is_the_full_history():
    scale = synth.head_dim_scale(d)
    k = rows(300, 1)
    v = rows(300, 2)
    kept, _ = oracle.mt_turn_view(queries(3), k, POOL, 10_000, scale)
    np.testing.assert_array_equal(kept, np.arange(300))
    q = rows(G, 4)
    smax, smin = oracle.summaries_rebuild(k[kept], P)
    a = oracle.hsa_group(q, k[kept], v[kept], smax, smin, 300, P, 8, 6, scale)
    smax2, smin2 = oracle.summaries_rebuild(k, P)
    b = oracle.hsa_group(q, k, v, smax2, smin2, 300, P, 8, 6, scale)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_view_is_the_sorted_top_of_the_pooled_scores():
    scale = synth.head_dim_scale(d)
    k = rows(500, 5)
    keep = 120
    kept, pooled = oracle.mt_turn_view(queries(6), k, POOL, keep, scale)
    L = len(k)
    order = np.lexsort((np.arange(L - w), -pooled.astype(np.float64)))
    want = np.concatenate([np.sort(order[:keep - w]), np.arange(L - w, L)])
    np.testing.assert_array_equal(kept, want)


def test_left_out_row_returns_in_a_later_turn():
    scale = synth.head_dim_scale(d)
    L1 = 400
    hist = rows(L1, 7)
    u = torch.randn(d, generator=torch.Generator().manual_seed(8))
    u = u / u.norm()
    # a needle row at position 50 along u; turn 1's queries point away
    needle = 50
    kf = torch.from_numpy((hist.astype(np.uint32) << 16).view(np.float32)) \
        if hist.dtype == np.uint16 else torch.from_numpy(hist.copy())
    kf[needle] = 4.0 * np.sqrt(d) * u
    hist = synth.to_bits(kf)
    keep = 60
    kept1, _ = oracle.mt_turn_view(queries(9, -u, 3.0), hist, POOL, keep, scale)
    assert needle not in kept1
    # turn 2 appends rows and its queries point at the needle
    hist2 = np.concatenate([hist, rows(100, 10)])
    kept2, _ = oracle.mt_turn_view(queries(11, u, 3.0), hist2, POOL, keep, scale)
    assert needle in kept2
    # with permanent eviction (chunked prefill) the row is gone after turn 1
    chunks = oracle.snapkv_chunked_group([queries(9, -u, 3.0), queries(11, u, 3.0)],
                                         [hist, rows(100, 10)], POOL, [keep, keep], scale)
    assert needle not in chunks[0][2] and needle not in chunks[1][2]
