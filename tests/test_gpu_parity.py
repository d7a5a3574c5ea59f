"""GPU parity of every librkv entry point against the CPU oracle on small and
ragged shapes: page summaries (bit-exact), HSA channel/page selection and page
scores (bit-exact), attention outputs (within 1e-3), SnapKV++ kept sets (gap
rule) and the compacted cache.  Inputs are seeded; both sides read the same
bytes."""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_cache_hsa_amd import synth, workloads

from _helpers import (OUT_ATOL, bits, check_kept, fill_cache, gpu_summaries, lib, make_cache,
                      max_abs_err, n_pages, oracle_summaries, scale_for)

pytestmark = pytest.mark.gpu
F32, BF16 = torch.float32, torch.bfloat16


def rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


# (dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages)
DECODE_CASES = [
    (F32, 1, 2, 4, 64, 16, 16, 16, [2048], 136),
    (BF16, 3, 2, 4, 128, 16, 32, 8, [1000, 17, 1], 64),
    (BF16, 2, 1, 8, 128, 1, 32, 64, [300, 129], 512),
    (F32, 2, 3, 1, 64, 7, 64, 5, [100, 0], 32),
    (BF16, 1, 4, 2, 64, 32, 8, 200, [1500], 64),
    (BF16, 2, 8, 4, 128, 16, 32, 64, [5000, 4100], 400),
    (BF16, 1, 2, 4, 128, 8, 16, 32, [1359], 200),
    (F32, 1, 2, 2, 128, 32, 128, 1024, [8000], 260),
    (BF16, 1, 1, 4, 128, 4, 32, 50, [20000], 5000),
    (F32, 4, 2, 8, 64, 3, 5, 7, [1, 2, 3, 250], 100),
    # the largest page size, one channel and one page, a cache filled to
    # exactly its capacity (max_pages * P rows)
    (BF16, 2, 2, 4, 128, 256, 1, 1, [3000, 256], 16),
    (BF16, 3, 2, 2, 64, 16, 1, 1, [1, 16, 17], 4),
    (BF16, 2, 2, 4, 128, 16, 32, 64, [2048, 2047], 128),
    # k2 in (128, 256] over several selection chunks: the rank-ordered
    # candidate merge with four keys per lane
    (BF16, 1, 2, 4, 128, 8, 32, 200, [4000], 600),
    # a RocketKV-MT view's shape: 128 pages of 32 rows selected, more rows
    # than one block's table, so split-K shares of at most 2,048 rows
    (BF16, 2, 8, 4, 128, 32, 32, 128, [6500, 5001], 208),
    # groups of 8 query heads: 8-wave fused blocks, one per unit at 192 units
    (BF16, 24, 8, 8, 128, 16, 32, 64, [1000 + 41 * i for i in range(24)], 128),
    (F32, 24, 8, 8, 64, 16, 16, 32, [800 + 13 * i for i in range(24)], 72),
    # token-level selection (page 1) with k2 above 1,024, up to the limit
    (BF16, 1, 2, 4, 128, 1, 32, 2000, [5000], 5100),
    (F32, 1, 1, 2, 64, 1, 8, 4096, [4500], 4600),
    # the fixed-stride staging of 32 channels at its edges: exactly 512
    # pages (staged at the fixed stride), 513 pages (summaries read from
    # memory), and a page capacity that is not a multiple of 8 (staged at
    # the packed stride)
    (BF16, 2, 2, 4, 128, 16, 32, 64, [8192, 8100], 520),
    (BF16, 1, 2, 4, 128, 16, 32, 64, [8193], 520),
    (BF16, 1, 2, 4, 128, 16, 32, 64, [3000], 190),
    # bf16 at head_dim 128 with groups of 1 and 2 query heads (the
    # attention merge's per-head lane sums; groups of 4 and 8 take the
    # four-heads-per-swap form), ragged rows
    (BF16, 2, 2, 1, 128, 16, 32, 32, [700, 333], 64),
    (BF16, 3, 2, 2, 128, 8, 16, 24, [900, 17, 260], 128),
]


def run_decode_case(case, seed, q_override=None, k_override=None, mode="decode", opts=None):
    """mode: "decode" (rkv_hsa_decode on a filled cache) or "step" (the cache
    holds rows [0, n-1) and rkv_decode_step appends row n-1 itself).  opts:
    execution options (rkv_opts) passed to the decode call and used to size
    its workspace."""
    rkv = lib()
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = case
    Lmax = max(max(lens), 1)
    K = k_override if k_override is not None else rand((B, Hkv, Lmax, d), seed, dtype, 1.5)
    V = rand((B, Hkv, Lmax, d), seed + 1, dtype)
    q = q_override if q_override is not None else rand((B, Hkv * G, d), seed + 2, dtype)
    g = rkv.gqa(Hkv, G, d)
    pages = [min(max_pages, n_pages(n, P) + 1) for n in lens]
    cache, summ = make_cache(Hkv, d, P, max_pages, pages, dtype, seed)
    Kd, Vd, qd = K.cuda(), V.cuda(), q.cuda()
    if mode == "step":
        fill_cache(g, cache, summ, Kd, Vd, [max(n - 1, 0) for n in lens])
        last = torch.tensor([max(n - 1, 0) for n in lens])
        k_new = torch.stack([Kd[b, :, last[b]] for b in range(B)]).contiguous()
        v_new = torch.stack([Vd[b, :, last[b]] for b in range(B)]).contiguous()
    else:
        fill_cache(g, cache, summ, Kd, Vd, lens)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hkv * G, d), float("nan"), device="cuda")
    chan = torch.full((B, Hkv, k1), -7, dtype=torch.int32, device="cuda")
    pidx = torch.full((B, Hkv, k2), -7, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, Hkv, max_pages), dtype=torch.float32, device="cuda")
    ws = rkv.hsa_workspace(g, B, P, max_pages, k1, k2, "cuda", opts)
    scale = scale_for(d)
    if mode == "step":
        rkv.rkv_decode_step(g, qd, k_new, v_new, cache, seq, summ, k1, k2, scale, out, ws,
                            chan_idx=chan, page_idx=pidx, page_scores=scores, opts=opts)
    else:
        rkv.rkv_hsa_decode(g, qd, cache, seq, summ, k1, k2, scale, out, ws, chan_idx=chan,
                           page_idx=pidx, page_scores=scores, opts=opts)
    torch.cuda.synchronize()
    if mode == "step":
        # the appended row sits in the pool at its page's block
        for b in range(B):
            n = lens[b]
            if n == 0:
                continue
            blk = int(cache.page_table[b, (n - 1) // P])
            for h in range(Hkv):
                assert torch.equal(cache.k_pool[blk, h, (n - 1) % P].cpu(), K[b, h, n - 1]), (b, h)
                assert torch.equal(cache.v_pool[blk, h, (n - 1) % P].cpu(), V[b, h, n - 1]), (b, h)
    worst = 0.0
    for b in range(B):
        n = lens[b]
        NP = n_pages(n, P)
        for h in range(Hkv):
            kb, vb = bits(K[b, h, :max(n, 1)]), bits(V[b, h, :max(n, 1)])
            smax, smin = oracle_summaries(bits(K[b, h, :n]), P, NP, d)
            gmax, gmin = gpu_summaries(summ, b, h, NP)
            if NP:
                np.testing.assert_array_equal(gmax, smax)
                np.testing.assert_array_equal(gmin, smin)
            c_o, p_o, S_o, out_o = oracle.hsa_group(bits(q[b, h * G:(h + 1) * G]), kb, vb, smax,
                                                    smin, n, P, k1, k2, scale)
            np.testing.assert_array_equal(chan[b, h].cpu().numpy(), c_o)
            np.testing.assert_array_equal(pidx[b, h].cpu().numpy(), p_o)
            np.testing.assert_array_equal(scores[b, h, :NP].cpu().numpy().view(np.uint32),
                                          S_o.view(np.uint32))
            err = max_abs_err(out[b, h * G:(h + 1) * G], out_o)
            assert err <= OUT_ATOL, (b, h, err)
            worst = max(worst, err)
    return worst, out


PATH_OPTS = {
    "auto": {},
    "fused": {"form": 2},
    "splitk": {"form": 3},
    "split": {"form": 1},
    "split-legacy": {"form": 1, "select_radix": 1},
    "split-chunk64": {"form": 1, "select_chunk": 64},
}


def path_opts(name):
    return lib().make_opts(**PATH_OPTS[name])


@pytest.fixture(params=list(PATH_OPTS))
def path(request):
    """Which implementation rkv_hsa_decode / rkv_decode_step dispatch to,
    as explicit rkv_opts: the default rule, the fused kernel with one block
    per unit, the fused kernel split K-wise (plus the merge), or the
    standalone kernels (with several selection chunks: rank-ordered
    candidates and the rank-search merge by default, "split-legacy" the
    radix top-k and radix merge, "split-chunk64" 64-page chunks, whose
    candidates take the radix merge when there are too many lists)."""
    return request.param


def case_mode(case, opts=None):
    """The decode form the library picks for a case and options."""
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = case
    rkv = lib()
    return rkv.decode_mode(rkv.gqa(Hkv, G, d), B, P, max_pages, k2, k1,
                           rkv.RKV_F32 if dtype == F32 else rkv.RKV_BF16, opts)


def fused_supported(case):
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = case
    return G <= 8 and max_pages <= 2048 and k2 * P <= 2048


@pytest.mark.parametrize("ci", range(len(DECODE_CASES)))
@pytest.mark.parametrize("mode", ["decode", "step"])
def test_decode_matches_oracle(ci, mode, path):
    case = DECODE_CASES[ci]
    opts = path_opts(path)
    if path == "fused" and not fused_supported(case):
        pytest.skip("shape outside the fused kernel's limits (dispatches to the split path)")
    if path == "splitk" and case_mode(case, opts) != 3:
        pytest.skip("shape outside the split-K fused kernel's limits")
    run_decode_case(case, 1000 + ci, mode=mode, opts=opts)


# A batch large enough for the fused kernel by default (B * Hkv >= 192).
BIG_CASE = (BF16, 24, 8, 4, 128, 16, 32, 64, [4000 + 37 * i for i in range(24)], 320)


def test_splitk_appended_row_read_by_a_later_split():
    """Split-K fused path, one page per split: the appended row's key points
    along the group's queries, so its page (the highest selected index) is
    attended by the last split, not by the block that stores the row.  The
    output must match the oracle, and the pool must hold the new row."""
    opts = path_opts("splitk")
    case = (BF16, 2, 2, 4, 128, 16, 32, 16, [1000, 777], 80)
    assert case_mode(case, opts) == 3
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = case
    K = rand((B, Hkv, max(lens), d), 4100, dtype, 1.5)
    q = rand((B, Hkv * G, d), 4102, dtype)
    for b in range(B):
        for h in range(Hkv):
            qs = q[b, h * G:(h + 1) * G].float().sum(0)
            K[b, h, lens[b] - 1] = (8.0 * qs / qs.norm()).to(dtype)
    run_decode_case(case, 4100, q_override=q, k_override=K, mode="step", opts=opts)


def test_decode_large_batch_default_path():
    run_decode_case(BIG_CASE, 77, mode="step")


def test_fused_and_split_select_identically():
    outs = []
    for name, form in (("fused", 2), ("splitk", 3), ("split", 1)):
        opts = path_opts(name)
        assert case_mode(BIG_CASE, opts) == form
        outs.append(run_decode_case(BIG_CASE, 78, mode="step", opts=opts)[1].clone())
    for o in outs[1:]:
        assert (outs[0] - o).abs().max().item() < 1e-5


def test_decode_ties_zero_query_and_identical_keys():
    case = (BF16, 2, 2, 4, 128, 16, 32, 8, [700, 333], 64)
    q = torch.zeros((2, 8, 128), dtype=BF16)
    run_decode_case(case, 7, q_override=q)
    K = rand((2, 2, 1, 128), 8, BF16).expand(2, 2, 700, 128).contiguous()
    run_decode_case(case, 9, k_override=K)


def test_decode_is_deterministic():
    case = DECODE_CASES[5]
    _, a = run_decode_case(case, 42)
    _, b = run_decode_case(case, 42)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_append_in_chunks_matches_rebuild(dtype):
    rkv = lib()
    B, Hkv, d, P, max_pages = 3, 2, 64, 16, 40
    g = rkv.gqa(Hkv, 2, d)
    lens = [600, 37, 1]
    K = rand((B, Hkv, 600, d), 5, dtype)
    V = rand((B, Hkv, 600, d), 6, dtype)
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages] * B, dtype, 3)
    Kd, Vd = K.cuda(), V.cuda()
    done = [0] * B
    for step, chunk in enumerate([1, 15, 16, 100, 3, 1000]):
        new = [min(lens[b], done[b] + chunk) for b in range(B)]
        mx = max(max(nn - o for nn, o in zip(new, done)), 1)
        src_k = torch.zeros((B, Hkv, mx, d), dtype=dtype, device="cuda")
        src_v = torch.zeros_like(src_k)
        for b in range(B):
            src_k[b, :, :new[b] - done[b]] = Kd[b, :, done[b]:new[b]]
            src_v[b, :, :new[b] - done[b]] = Vd[b, :, done[b]:new[b]]
        rkv.rkv_append_summaries(g, cache, torch.tensor(done, dtype=torch.int32, device="cuda"),
                                 torch.tensor(new, dtype=torch.int32, device="cuda"), mx, summ,
                                 k_src=src_k, v_src=src_v)
        done = new
    torch.cuda.synchronize()
    table = cache.page_table.cpu()
    for b in range(B):
        NP = n_pages(lens[b], P)
        for h in range(Hkv):
            smax, smin = oracle.summaries_rebuild(bits(K[b, h, :lens[b]]), P)
            gmax, gmin = gpu_summaries(summ, b, h, NP)
            np.testing.assert_array_equal(gmax, smax)
            np.testing.assert_array_equal(gmin, smin)
            for p in range(NP):  # rows landed in the right blocks
                rows = cache.k_pool[table[b, p], h, :min(P, lens[b] - p * P)].cpu()
                assert torch.equal(rows, K[b, h, p * P:p * P + rows.shape[0]])
    # rebuild from the pool (no copy-in) gives the same bits
    summ2 = torch.zeros_like(summ)
    rkv.rkv_append_summaries(g, cache, torch.zeros(B, dtype=torch.int32, device="cuda"),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), 600, summ2)
    torch.cuda.synchronize()
    assert torch.equal(summ.view(torch.int16 if dtype == BF16 else torch.int32),
                       summ2.view(torch.int16 if dtype == BF16 else torch.int32))


@pytest.mark.parametrize("form", ["fused", "splitk", "split"])
def test_tiny_workload_decode_loop(form):
    """The tiny fp32 workload end to end: 2,048 cached rows, 32 decode steps,
    each appending its token and decoding in one rkv_decode_step call."""
    opts = path_opts(form)
    rkv = lib()
    wl = workloads.TINY
    B, Hkv, G, d, P = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim, wl.page_size
    n0 = wl.cache_len
    cap = n0 + wl.decode_steps
    max_pages = n_pages(cap, P)
    g = rkv.gqa(Hkv, G, d)
    k0, v0 = wl.prompt_kv(0, 0, n0)
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages], wl.dtype, 1)
    fill_cache(g, cache, summ, k0[None].cuda(), v0[None].cuda(), [n0])
    K = np.zeros((cap, d), np.float32)
    V = np.zeros((cap, d), np.float32)
    Ko = [K.copy() for _ in range(Hkv)]
    Vo = [V.copy() for _ in range(Hkv)]
    smax = [np.zeros((max_pages, d), np.float32) for _ in range(Hkv)]
    smin = [np.zeros((max_pages, d), np.float32) for _ in range(Hkv)]
    for h in range(Hkv):
        Ko[h][:n0], Vo[h][:n0] = k0[h].numpy(), v0[h].numpy()
        oracle.summaries_append(Ko[h], 0, n0, P, smax[h], smin[h])
    ws = rkv.hsa_workspace(g, B, P, max_pages, wl.k1, wl.k2, "cuda", opts)
    out = torch.zeros((B, Hkv * G, d), device="cuda")
    pidx = torch.zeros((B, Hkv, wl.k2), dtype=torch.int32, device="cuda")
    chan = torch.zeros((B, Hkv, wl.k1), dtype=torch.int32, device="cuda")
    scale = scale_for(d)
    n = n0
    for step in range(wl.decode_steps):
        kt, vt, qt = wl.decode_tokens(0, step, torch.tensor([n]))
        seq = torch.tensor([n + 1], dtype=torch.int32, device="cuda")
        rkv.rkv_decode_step(g, qt.cuda(), kt.cuda(), vt.cuda(), cache, seq, summ, wl.k1, wl.k2,
                            scale, out, ws, chan_idx=chan, page_idx=pidx, opts=opts)
        torch.cuda.synchronize()
        for h in range(Hkv):
            Ko[h][n], Vo[h][n] = kt[0, h].numpy(), vt[0, h].numpy()
            oracle.summaries_append(Ko[h], n, n + 1, P, smax[h], smin[h])
            c_o, p_o, _, out_o = oracle.hsa_group(qt[0, h * G:(h + 1) * G].numpy(), Ko[h], Vo[h],
                                                  smax[h], smin[h], n + 1, P, wl.k1, wl.k2, scale)
            np.testing.assert_array_equal(chan[0, h].cpu().numpy(), c_o)
            np.testing.assert_array_equal(pidx[0, h].cpu().numpy(), p_o)
            assert max_abs_err(out[0, h * G:(h + 1) * G], out_o) <= OUT_ATOL
        n += 1


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("pool", [1, 7, 63])
def test_prefill_evict_matches_oracle(dtype, pool):
    rkv = lib()
    B, Hkv, G, d, w, P = 3, 2, 4, 64, 16, 16
    lens = [500, 1700, 3000]
    keeps = [100, 300, 3000 if pool == 1 else 500]   # one case keeps everything
    L_max = max(lens)
    g = rkv.gqa(Hkv, G, d)
    K = rand((B, Hkv, L_max, d), 21 + pool, dtype, 1.5)
    V = rand((B, Hkv, L_max, d), 22 + pool, dtype)
    Q = rand((B, Hkv * G, w, d), 23 + pool, dtype)
    max_pages = n_pages(max(keeps), P) + 2
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages] * B, dtype, 4)
    keep_eff = [min(k, L) for k, L in zip(keeps, lens)]
    kept = torch.full((B, Hkv, max(keep_eff)), -7, dtype=torch.int32, device="cuda")
    pooled = torch.zeros((B, Hkv, L_max), dtype=torch.float32, device="cuda")
    seq_out = torch.zeros(B, dtype=torch.int32, device="cuda")
    scale = scale_for(d)
    rkv.rkv_prefill_evict(g, lens, keeps, Q.cuda(), K.cuda(), V.cuda(), w, pool, scale, cache,
                          summaries=summ, kept_idx=kept, pooled_scores=pooled,
                          seq_lens_out=seq_out)
    torch.cuda.synchronize()
    assert seq_out.cpu().tolist() == keep_eff
    table = cache.page_table.cpu()
    swaps = 0
    for b in range(B):
        L, ke = lens[b], keep_eff[b]
        for h in range(Hkv):
            kb = bits(K[b, h, :L])
            k_o, A_o, pl_o = oracle.snapkv_group(bits(Q[b, h * G:(h + 1) * G]), kb, pool, keeps[b],
                                                 scale)
            gk = kept[b, h].cpu().numpy()
            assert np.all(gk[ke:] == -1)
            unit_swaps = 0
            if keeps[b] < L:
                gp = pooled[b, h, :L - w].cpu().numpy()
                np.testing.assert_allclose(gp, pl_o, rtol=1e-5, atol=0)
                unit_swaps = check_kept(gk[:ke], k_o, pl_o, w)
                swaps += unit_swaps
            else:
                np.testing.assert_array_equal(gk[:ke], k_o)
            # the compacted cache holds the kept rows in order: the oracle's
            # set when the sets agree, else (a near-tie swap) the GPU's own
            rows_k = torch.stack([cache.k_pool[table[b, r // P], h, r % P] for r in range(ke)])
            rows_v = torch.stack([cache.v_pool[table[b, r // P], h, r % P] for r in range(ke)])
            sel = k_o if unit_swaps == 0 else gk[:ke]
            idx = torch.from_numpy(sel.astype(np.int64))
            assert torch.equal(rows_k.cpu(), K[b, h, idx])
            assert torch.equal(rows_v.cpu(), V[b, h, idx])
            if unit_swaps == 0:
                smax, smin = oracle.summaries_rebuild(bits(K[b, h, idx]), P)
                gmax, gmin = gpu_summaries(summ, b, h, n_pages(ke, P))
                np.testing.assert_array_equal(gmax, smax)
                np.testing.assert_array_equal(gmin, smin)
    print(f"near-tie boundary swaps: {swaps}")


# The pages' ablation axes as parameterisations of the same kernels: Quest-only
# (k1 = d: every channel, so the page bound is the full box bound), SparQ-only
# (page size 1: the bound is the partial dot product of the k1 channels) and
# Exact-TopK (both: the exact GQA-summed score of every token).
PARAM_CASES = {
    "quest": (BF16, 2, 8, 4, 128, 16, 128, 32, [3000, 2000], 200),
    "sparq": (BF16, 2, 8, 4, 128, 1, 32, 256, [1500, 700], 1600),
    "exact": (BF16, 2, 8, 4, 128, 1, 128, 512, [1800, 900], 1900),
}


@pytest.mark.parametrize("name", sorted(PARAM_CASES))
@pytest.mark.parametrize("mode", ["decode", "step"])
def test_selection_parameterisations(name, mode, path):
    case = PARAM_CASES[name]
    opts = path_opts(path)
    if path == "fused" and not fused_supported(case):
        pytest.skip("shape outside the fused kernel's limits")
    if path == "splitk" and case_mode(case, opts) != 3:
        pytest.skip("shape outside the split-K fused kernel's limits")
    run_decode_case(case, 3000 + len(name), mode=mode, opts=opts)


def test_exact_topk_is_the_top_of_the_true_scores():
    """With P = 1 and k1 = d the selected tokens are the k2 largest exact
    scores sum_j q_j . k_t (checked in float64 away from near ties)."""
    rkv = lib()
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = PARAM_CASES["exact"]
    Lmax = max(lens)
    K = rand((B, Hkv, Lmax, d), 91, dtype, 1.5)
    q = rand((B, Hkv * G, d), 92, dtype)
    g = rkv.gqa(Hkv, G, d)
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages] * B, dtype, 9)
    fill_cache(g, cache, summ, K.cuda(), K.cuda(), lens)
    pidx = torch.zeros((B, Hkv, k2), dtype=torch.int32, device="cuda")
    ws = rkv.hsa_workspace(g, B, P, max_pages, k1, k2, "cuda")
    rkv.rkv_hsa_select(g, q.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"), P, summ,
                       k1, k2, pidx, ws)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(Hkv):
            s = (q[b, h * G:(h + 1) * G].double() @ K[b, h, :lens[b]].double().T).sum(0).numpy()
            order = np.argsort(-s, kind="stable")
            kth, nxt = s[order[k2 - 1]], s[order[k2]]
            if abs(kth - nxt) <= 1e-5 * abs(kth):
                continue  # float64 and the fp32 order may rank a near tie differently
            np.testing.assert_array_equal(pidx[b, h].cpu().numpy(), np.sort(order[:k2]))


def test_selection_overlap_measurement_runs():
    """The overlap measurement on the tiny workload: exact top-k agrees with
    itself and every method's recall and attention mass are fractions."""
    from sparse_kv_cache_hsa_amd import overlap
    res = overlap.measure(workloads.TINY, steps=2)
    assert res["exact"]["recall_vs_exact_min"] == 1.0
    for m in ("hsa", "quest", "sparq", "exact"):
        for key in ("recall_vs_exact_mean", "attention_mass_mean"):
            assert 0.0 <= res[m][key] <= 1.0 + 1e-6


def _random_cases(n, seed):
    """Seeded shape combinations inside the documented limits."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        dtype = BF16 if rng.random() < 0.7 else F32
        d = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 3, 8]))
        B = int(rng.integers(1, 5))
        P = int(rng.choice([1, 2, 3, 8, 16, 32, 64]))
        k1 = int(rng.integers(1, d + 1))
        lens = [int(x) for x in rng.integers(0, 2500, B)]
        need = max(n_pages(n, P) for n in lens) + 1
        max_pages = int(min(2048, need + rng.integers(0, 8)))
        lens = [min(n, max_pages * P) for n in lens]
        k2 = int(rng.integers(1, min(300, max(2, need)) + 1))
        cases.append((dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages))
    return cases


RANDOM_CASES = _random_cases(16, 2024)


@pytest.mark.parametrize("ci", range(len(RANDOM_CASES)))
@pytest.mark.parametrize("mode", ["decode", "step"])
def test_random_shapes_match_oracle(ci, mode, path):
    case = RANDOM_CASES[ci]
    opts = path_opts(path)
    if path == "fused" and not fused_supported(case):
        pytest.skip("shape outside the fused kernel's limits")
    if path == "splitk" and case_mode(case, opts) != 3:
        pytest.skip("shape outside the split-K fused kernel's limits")
    run_decode_case(case, 5000 + ci, mode=mode, opts=opts)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_prefill_evict_chunked_matches_oracle(dtype):
    """Three prefill chunks per sequence with the budget re-enforced after
    each: kept rows (positions in the concatenation, gap rule), the cache
    rows and the summaries against the oracle's composition."""
    rkv = lib()
    B, Hkv, G, d, w, P, pool = 2, 2, 4, 64, 16, 16, 7
    chunk_lens = [[700, 500, 600], [300, 900, 40]]
    keeps = [[400, 400, 500], [250, 600, 620]]
    n_calls = 3
    C_max = max(max(c) for c in chunk_lens)
    g = rkv.gqa(Hkv, G, d)
    scale = scale_for(d)
    max_pages = 48
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages] * B, dtype, 6)
    table = cache.page_table.cpu()
    # the oracle's state per (sequence, head): original positions and rows
    state = {(b, h): (np.zeros(0, np.int64), None, None) for b in range(B) for h in range(Hkv)}
    live = {u: True for u in state}
    n_cached = [0] * B
    offsets = [0] * B
    swaps = 0
    for t in range(n_calls):
        cl = [chunk_lens[b][t] for b in range(B)]
        kp = [keeps[b][t] for b in range(B)]
        Kc = rand((B, Hkv, C_max, d), 300 + t, dtype, 1.5)
        Vc = rand((B, Hkv, C_max, d), 400 + t, dtype)
        Q = rand((B, Hkv * G, w, d), 500 + t, dtype)
        L = [n_cached[b] + cl[b] for b in range(B)]
        keep_eff = [min(kp[b], L[b]) for b in range(B)]
        kept = torch.full((B, Hkv, max(keep_eff)), -7, dtype=torch.int32, device="cuda")
        seq_out = torch.zeros(B, dtype=torch.int32, device="cuda")
        rkv.rkv_prefill_evict_chunk(g, n_cached, cl, kp, Q.cuda(), Kc.cuda(), Vc.cuda(), w, pool,
                                    scale, cache, summaries=summ, kept_idx=kept,
                                    seq_lens_out=seq_out)
        torch.cuda.synchronize()
        assert seq_out.cpu().tolist() == keep_eff
        for b in range(B):
            for h in range(Hkv):
                pos, rk, rv = state[(b, h)]
                kc, vc = bits(Kc[b, h, :cl[b]]), bits(Vc[b, h, :cl[b]])
                cat_k = kc if rk is None else np.concatenate([rk, kc])
                cat_v = vc if rv is None else np.concatenate([rv, vc])
                cpos = np.concatenate([pos, offsets[b] + np.arange(cl[b])])
                k_o, _, pl_o = oracle.snapkv_group(bits(Q[b, h * G:(h + 1) * G]), cat_k, pool,
                                                   kp[b], scale)
                if not live[(b, h)]:
                    continue
                gk = kept[b, h, :keep_eff[b]].cpu().numpy()
                s = check_kept(gk, k_o, pl_o, w) if kp[b] < L[b] else 0
                if kp[b] >= L[b]:
                    np.testing.assert_array_equal(gk, k_o)
                swaps += s
                if s:
                    live[(b, h)] = False
                    continue
                state[(b, h)] = (cpos[k_o], cat_k[k_o], cat_v[k_o])
                # the cache holds the kept rows in order, and their summaries
                ke = keep_eff[b]
                rows_k = torch.stack([cache.k_pool[table[b, r // P], h, r % P] for r in range(ke)])
                np.testing.assert_array_equal(bits(rows_k.cpu()), cat_k[k_o])
                smax, smin = oracle.summaries_rebuild(cat_k[k_o], P)
                gmax, gmin = gpu_summaries(summ, b, h, n_pages(ke, P))
                np.testing.assert_array_equal(gmax, smax)
                np.testing.assert_array_equal(gmin, smin)
        n_cached = keep_eff
        offsets = [offsets[b] + cl[b] for b in range(B)]
    print(f"chunked eviction near-tie swaps: {swaps}")
    assert sum(live.values()) >= len(live) - 1


@pytest.mark.parametrize("form", ["fused", "splitk", "split"])
def test_device_status_word(form):
    """Device-side inputs the kernels must clamp or skip are reported in the
    optional status word (rkv_opts.status): a row count beyond the cache's
    capacity (RKV_DEV_LENGTH), a page-table entry outside the pool
    (RKV_DEV_BLOCK) and, for rkv_hsa_attend, a page index outside the
    sequence (RKV_DEV_PAGE).  Clean calls leave the word at zero, and the
    sequences with valid inputs still match the oracle."""
    rkv = lib()
    dtype, B, Hkv, G, d, P, k1, k2, max_pages = BF16, 2, 2, 4, 128, 16, 32, 4, 8
    lens = [100, 50]
    K = rand((B, Hkv, 128, d), 61, dtype, 1.5)
    V = rand((B, Hkv, 128, d), 62, dtype)
    q = rand((B, Hkv * G, d), 63, dtype)
    g = rkv.gqa(Hkv, G, d)
    cache, summ = make_cache(Hkv, d, P, max_pages, [max_pages] * B, dtype, 64)
    fill_cache(g, cache, summ, K.cuda(), V.cuda(), lens)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    opts = lib().make_opts(**PATH_OPTS[form], status=status)
    ws = rkv.hsa_workspace(g, B, P, max_pages, k1, k2, "cuda", opts)
    out = torch.zeros((B, Hkv * G, d), device="cuda")
    pidx = torch.zeros((B, Hkv, k2), dtype=torch.int32, device="cuda")
    scale = scale_for(d)
    qd = q.cuda()

    def decode(seq_lens):
        status.zero_()
        rkv.rkv_hsa_decode(g, qd, cache, torch.tensor(seq_lens, dtype=torch.int32, device="cuda"),
                           summ, k1, k2, scale, out, ws, page_idx=pidx, opts=opts)
        torch.cuda.synchronize()
        return int(status.item())

    def check_seq(b):
        n = lens[b]
        for h in range(Hkv):
            smax, smin = oracle.summaries_rebuild(bits(K[b, h, :n]), P)
            _, p_o, _, out_o = oracle.hsa_group(bits(q[b, h * G:(h + 1) * G]), bits(K[b, h, :n]),
                                                bits(V[b, h, :n]), smax, smin, n, P, k1, k2, scale)
            np.testing.assert_array_equal(pidx[b, h].cpu().numpy(), p_o)
            assert max_abs_err(out[b, h * G:(h + 1) * G], out_o) <= OUT_ATOL

    assert decode(lens) == 0
    check_seq(0)
    check_seq(1)
    # sequence 0 claims more rows than max_pages * P = 128
    assert decode([200, 50]) == rkv.RKV_DEV_LENGTH
    check_seq(1)
    assert decode([-3, 50]) == rkv.RKV_DEV_LENGTH
    check_seq(1)
    # a page of sequence 0 points outside the pool; k2 = 4 of its 7 pages
    # with one of them broken must touch it for some head or not at all, so
    # every page is made selectable by asking for all of them
    saved = cache.page_table.clone()
    cache.page_table[0, 2] = cache.k_pool.shape[0] + 5
    status.zero_()
    k2_all = 8
    ws_all = rkv.hsa_workspace(g, B, P, max_pages, k1, k2_all, "cuda", opts)
    pidx_all = torch.zeros((B, Hkv, k2_all), dtype=torch.int32, device="cuda")
    rkv.rkv_hsa_decode(g, qd, cache, torch.tensor(lens, dtype=torch.int32, device="cuda"), summ,
                       k1, k2_all, scale, out, ws_all, page_idx=pidx_all, opts=opts)
    torch.cuda.synchronize()
    assert int(status.item()) == rkv.RKV_DEV_BLOCK
    cache.page_table.copy_(saved)
    # rkv_hsa_attend with a page index outside sequence 1's 4 pages
    bad = pidx.clone()
    bad[1, 0, 0] = 6
    status.zero_()
    rkv.rkv_hsa_attend(g, qd, cache, torch.tensor(lens, dtype=torch.int32, device="cuda"), bad,
                       k2, scale, out, ws, opts=opts)
    torch.cuda.synchronize()
    assert int(status.item()) == rkv.RKV_DEV_PAGE
    # an append whose row counts exceed the capacity
    status.zero_()
    rkv.rkv_append_summaries(g, cache, torch.tensor([100, 50], dtype=torch.int32, device="cuda"),
                             torch.tensor([300, 50], dtype=torch.int32, device="cuda"), 8,
                             torch.zeros_like(summ), opts=opts)
    torch.cuda.synchronize()
    assert int(status.item()) == rkv.RKV_DEV_LENGTH
