"""GPU parity of the multi-turn view (rkv_turn_filter, RocketKV-MT's "retain
evicted tokens for later turns") against oracle.mt_turn_view.  Per turn:
the turn's rows are appended to the full cache, SnapKV++ over the whole
history picks the view (kept set bit-exact up to near-tie swaps; view rows
and summaries bit-exact), then decode steps run on the view (channels and
pages bit-exact, outputs within 1e-3) while every new token also goes to the
full cache.  A needle row left out of turn 1's view returns in turn 2's when
turn 2's queries point at it."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import OUT_ATOL, bits, check_kept, gpu_summaries, lib, make_cache, n_pages, \
    scale_for

pytestmark = pytest.mark.gpu
F32, BF16 = torch.float32, torch.bfloat16


def randn(shape, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_turn_filter_matches_oracle(dtype):
    rkv = lib()
    B, Hkv, G, d, P, w, pool, k1, k2 = 2, 2, 4, 64, 16, 16, 7, 16, 8
    hist0 = [900, 1300]
    turn_rows = [200, 150]
    keep = [300, 400]
    turns, steps = 3, 4
    g = rkv.gqa(Hkv, G, d)
    scale = scale_for(d)
    cap_full = max(hist0) + turns * (max(turn_rows) + steps)
    full_pages = n_pages(cap_full, P)
    view_pages = n_pages(max(keep) + steps, P) + 1
    full, _ = make_cache(Hkv, d, P, full_pages, [full_pages] * B, dtype, 21)
    full_summ = torch.zeros((B, Hkv, 2, d, full_pages), dtype=dtype, device="cuda")
    view, view_summ = make_cache(Hkv, d, P, view_pages, [view_pages] * B, dtype, 22)
    # needles: rows of sequence 0 along u; turn 1's queries point away from
    # them, turn 2's at them
    u = randn(d, 23)
    u = u / u.norm()
    needles = [150, 400, 650, 800]
    Kh = [randn((Hkv, hist0[b], d), 30 + b) * 1.2 for b in range(B)]
    Vh = [randn((Hkv, hist0[b], d), 40 + b) for b in range(B)]
    for r in needles:
        Kh[0][:, r] = 4.0 * d ** 0.5 * u
    K_all = [k.to(dtype) for k in Kh]          # the oracle's full history per sequence
    V_all = [v.to(dtype) for v in Vh]
    n = [0] * B

    def append_full(kr, vr):
        """Appends kr/vr (per sequence [Hkv, m_b, d]) to the full cache."""
        m = max(x.shape[1] for x in kr)
        src_k = torch.zeros((B, Hkv, max(m, 1), d), dtype=dtype)
        src_v = torch.zeros_like(src_k)
        for b in range(B):
            src_k[b, :, :kr[b].shape[1]] = kr[b]
            src_v[b, :, :vr[b].shape[1]] = vr[b]
        n_old = torch.tensor(n, dtype=torch.int32, device="cuda")
        n_new = torch.tensor([n[b] + kr[b].shape[1] for b in range(B)], dtype=torch.int32,
                             device="cuda")
        rkv.rkv_append_summaries(g, full, n_old, n_new, max(m, 1), full_summ,
                                 k_src=src_k.cuda(), v_src=src_v.cuda())
        for b in range(B):
            n[b] += kr[b].shape[1]

    append_full(K_all, V_all)
    swaps = 0
    needle_in = []
    for t in range(turns):
        if t > 0:
            kr = [(randn((Hkv, turn_rows[b], d), 100 * t + b) * 1.2).to(dtype) for b in range(B)]
            vr = [randn((Hkv, turn_rows[b], d), 100 * t + 50 + b).to(dtype) for b in range(B)]
            append_full(kr, vr)
            K_all = [torch.cat([K_all[b], kr[b]], 1) for b in range(B)]
            V_all = [torch.cat([V_all[b], vr[b]], 1) for b in range(B)]
        sign = -1.0 if t == 0 else 1.0
        qw = (randn((B, Hkv * G, w, d), 200 + t) + sign * 3.0 * u).to(dtype)
        kept = torch.full((B, Hkv, max(keep)), -7, dtype=torch.int32, device="cuda")
        pooled = torch.zeros((B, Hkv, max(n)), dtype=torch.float32, device="cuda")
        vlen = torch.zeros(B, dtype=torch.int32, device="cuda")
        rkv.rkv_turn_filter(g, n, keep, qw.cuda(), w, pool, scale, full, view,
                            view_summaries=view_summ, kept_idx=kept, pooled_scores=pooled,
                            view_lens_out=vlen)
        torch.cuda.synchronize()
        assert vlen.cpu().tolist() == [min(k, m) for k, m in zip(keep, n)]
        table = view.page_table.cpu()
        views = {}
        for b in range(B):
            for h in range(Hkv):
                kb = bits(K_all[b][h])
                k_o, pl_o = oracle.mt_turn_view(bits(qw[b, h * G:(h + 1) * G]), kb, pool, keep[b],
                                                scale)
                gk = kept[b, h, :keep[b]].cpu().numpy()
                s = check_kept(gk, k_o, pl_o, w)
                swaps += s
                if b == 0:
                    needle_in.append(np.isin(needles, k_o))
                if s:
                    continue
                rows = torch.stack([view.k_pool[table[b, r // P], h, r % P]
                                    for r in range(keep[b])]).cpu()
                np.testing.assert_array_equal(bits(rows), kb[k_o])
                smax, smin = oracle.summaries_rebuild(kb[k_o], P)
                gmax, gmin = gpu_summaries(view_summ, b, h, n_pages(keep[b], P))
                np.testing.assert_array_equal(gmax, smax)
                np.testing.assert_array_equal(gmin, smin)
                views[(b, h)] = [kb[k_o], bits(V_all[b][h])[k_o]]
        # decode steps on the view; every token also goes to the full cache
        ws = rkv.hsa_workspace(g, B, P, view_pages, k1, k2, "cuda")
        vl = [min(k, m) for k, m in zip(keep, n)]
        for s_ in range(steps):
            kt = randn((B, Hkv, d), 300 + 10 * t + s_).to(dtype)
            vt = randn((B, Hkv, d), 400 + 10 * t + s_).to(dtype)
            qt = randn((B, Hkv * G, d), 500 + 10 * t + s_).to(dtype)
            seq = torch.tensor([x + 1 for x in vl], dtype=torch.int32, device="cuda")
            out = torch.zeros((B, Hkv * G, d), device="cuda")
            chan = torch.zeros((B, Hkv, k1), dtype=torch.int32, device="cuda")
            pidx = torch.zeros((B, Hkv, k2), dtype=torch.int32, device="cuda")
            rkv.rkv_decode_step(g, qt.cuda(), kt.cuda(), vt.cuda(), view, seq, view_summ, k1, k2,
                                scale, out, ws, chan_idx=chan, page_idx=pidx)
            append_full([kt[b][:, None] for b in range(B)], [vt[b][:, None] for b in range(B)])
            K_all = [torch.cat([K_all[b], kt[b][:, None]], 1) for b in range(B)]
            V_all = [torch.cat([V_all[b], vt[b][:, None]], 1) for b in range(B)]
            torch.cuda.synchronize()
            vl = [x + 1 for x in vl]
            for (b, h), (vk, vv) in views.items():
                vk = np.concatenate([vk, bits(kt[b, h])[None]])
                vv = np.concatenate([vv, bits(vt[b, h])[None]])
                views[(b, h)] = [vk, vv]
                smax, smin = oracle.summaries_rebuild(vk, P)
                c_o, p_o, _, out_o = oracle.hsa_group(bits(qt[b, h * G:(h + 1) * G]), vk, vv,
                                                      smax, smin, vl[b], P, k1, k2, scale)
                np.testing.assert_array_equal(chan[b, h].cpu().numpy(), c_o)
                np.testing.assert_array_equal(pidx[b, h].cpu().numpy(), p_o)
                err = float(np.abs(out[b, h * G:(h + 1) * G].cpu().double().numpy() - out_o).max())
                assert err <= OUT_ATOL, (t, s_, b, h, err)
    # needle rows out of turn 1's view are back in turn 2's (both heads)
    for h in range(Hkv):
        assert not needle_in[h].all() and needle_in[Hkv + h].all(), needle_in
    print(f"turn-filter near-tie swaps: {swaps}")
