"""rkv_decode_step_static (the library's static device scratch as workspace)
against rkv_decode_step (a caller workspace), through the C ABI, on two calls
in a row, the second with a smaller input: the channel and page index sets,
the appended cache rows and page summaries must be bit-exact and the outputs
within 1e-3 (the same kernels run, so they agree bit for bit)."""
import numpy as np
import pytest
import torch

from _helpers import OUT_ATOL, fill_cache, lib, make_cache, n_pages, scale_for

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def run_both(case, seed, opts=None):
    """One decode step (append + HSA) through both entry points on two
    identical copies of a filled cache."""
    rkv = lib()
    dtype, B, Hkv, G, d, P, k1, k2, lens, max_pages = case
    Lmax = max(lens)
    K = rand((B, Hkv, Lmax, d), seed, dtype, 1.5).cuda()
    V = rand((B, Hkv, Lmax, d), seed + 1, dtype).cuda()
    q = rand((B, Hkv * G, d), seed + 2, dtype).cuda()
    g = rkv.gqa(Hkv, G, d)
    pages = [min(max_pages, n_pages(n, P) + 1) for n in lens]
    res = []
    for static in (False, True):
        cache, summ = make_cache(Hkv, d, P, max_pages, pages, dtype, seed)
        fill_cache(g, cache, summ, K, V, [n - 1 for n in lens])
        last = [n - 1 for n in lens]
        k_new = torch.stack([K[b, :, last[b]] for b in range(B)]).contiguous()
        v_new = torch.stack([V[b, :, last[b]] for b in range(B)]).contiguous()
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out = torch.full((B, Hkv * G, d), float("nan"), device="cuda")
        chan = torch.full((B, Hkv, k1), -7, dtype=torch.int32, device="cuda")
        pidx = torch.full((B, Hkv, k2), -7, dtype=torch.int32, device="cuda")
        if static:
            rkv.rkv_decode_step_static(g, q, k_new, v_new, cache, seq, summ, k1, k2, scale_for(d),
                                       out, chan_idx=chan, page_idx=pidx, opts=opts)
        else:
            ws = rkv.hsa_workspace(g, B, P, max_pages, k1, k2, "cuda", opts)
            rkv.rkv_decode_step(g, q, k_new, v_new, cache, seq, summ, k1, k2, scale_for(d), out,
                                ws, chan_idx=chan, page_idx=pidx, opts=opts)
        torch.cuda.synchronize()
        res.append((out, chan, pidx, cache, summ))
    (o0, c0, p0, cache0, s0), (o1, c1, p1, cache1, s1) = res
    assert torch.equal(c0, c1)
    assert torch.equal(p0, p1)
    assert (o0 - o1).abs().max().item() <= OUT_ATOL
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
    assert torch.equal(cache0.k_pool.view(torch.int16), cache1.k_pool.view(torch.int16))
    assert torch.equal(cache0.v_pool.view(torch.int16), cache1.v_pool.view(torch.int16))
    assert torch.equal(s0.view(torch.int16), s1.view(torch.int16))


def test_static_scratch_matches_workspace_call():
    rkv = lib()
    # a batch that fills the chip (the fused kernel), then a smaller input on
    # the standalone kernels, whose candidates and partials use the scratch
    big = (BF16, 24, 8, 4, 128, 16, 32, 64, [4000 + 37 * i for i in range(24)], 320)
    small = (BF16, 3, 2, 4, 128, 16, 32, 40, [1000, 517, 2200], 160)
    run_both(big, 11)
    run_both(small, 12, opts=rkv.make_opts(form=rkv.RKV_FORM_STANDALONE))
