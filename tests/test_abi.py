"""Host-side checks of librkv without a GPU: it loads, exports every function
include/rkv.h declares, was built from the current sources, computes the
adaptive split like the oracle, and rejects bad arguments before touching
the device."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rkv_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(rkv_lib):
    lib = rkv_lib.load_library()
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(rkv_lib.EXPORTED)


def test_build_id_matches_sources(rkv_lib):
    from sparse_kv_cache_hsa_amd import build
    assert rkv_lib.load_library().rkv_build_id().decode() == build.source_hash()


@pytest.mark.parametrize("c", [1.0, 1.25, 2.0, 7.0, 16.0, 31.99, 64.0, 428.0, 1024.0, 3e5])
@pytest.mark.parametrize("L,w", [(0, 0), (1, 0), (32768, 32), (109568, 32), (16384, 32), (10, 32)])
def test_split_matches_oracle_bitwise(rkv_lib, c, L, w):
    assert rkv_lib.rkv_split_ratio(c, L, w) == oracle.split_ratio(c, L, w)


def test_split_rejects_bad_ratio(rkv_lib):
    for c in (0.99, float("nan"), float("inf"), -1.0):
        with pytest.raises(rkv_lib.RkvError) as e:
            rkv_lib.rkv_split_ratio(c, 10, 0)
        assert e.value.status == rkv_lib.RKV_EINVAL


def _call_decode(lib, g, dtype=0, B=1, P=16, max_pages=8, k1=8, k2=4, scale=0.125,
                 ws_bytes=1 << 20, null_q=False, null_out=False, num_blocks=64):
    fake = 0x10000  # never dereferenced: every case below fails a host check
    cache = lib.rkv_paged_cache(fake, fake, fake, num_blocks, P, max_pages)
    return lib.load_library().rkv_hsa_decode(
        ctypes.byref(g) if g is not None else None, dtype, B, None if null_q else fake,
        ctypes.byref(cache), fake, fake, k1, k2, scale, None if null_out else fake,
        None, None, None, fake, ws_bytes, None, None)


def test_decode_argument_checks(rkv_lib):
    L = rkv_lib
    g = L.gqa(8, 4, 128)
    assert _call_decode(L, None) == L.RKV_EINVAL
    assert _call_decode(L, L.gqa(8, 3, 128)) == L.RKV_EUNSUPPORTED
    assert _call_decode(L, L.gqa(8, 4, 96)) == L.RKV_EUNSUPPORTED
    assert _call_decode(L, g, dtype=7) == L.RKV_EUNSUPPORTED
    assert _call_decode(L, g, B=0) == L.RKV_EINVAL
    assert _call_decode(L, g, k1=0) == L.RKV_EINVAL
    assert _call_decode(L, g, k1=129) == L.RKV_EINVAL
    assert _call_decode(L, g, k2=0) == L.RKV_EINVAL
    assert _call_decode(L, g, k2=L.RKV_MAX_K2 + 1) == L.RKV_EINVAL
    assert _call_decode(L, g, P=0) == L.RKV_EINVAL
    assert _call_decode(L, g, P=300) == L.RKV_EUNSUPPORTED
    assert _call_decode(L, g, scale=0.0) == L.RKV_EINVAL
    assert _call_decode(L, g, scale=float("nan")) == L.RKV_EINVAL
    assert _call_decode(L, g, null_q=True) == L.RKV_EINVAL
    assert _call_decode(L, g, null_out=True) == L.RKV_EINVAL
    assert _call_decode(L, g, ws_bytes=16) == L.RKV_EWORKSPACE
    # a pool of 2^32 - 1 rows or more: the kernels' 32-bit row units
    # cannot name its rows (8 heads x 16 rows per block)
    assert _call_decode(L, g, num_blocks=(0xFFFFFFFF - 1) // 128 + 1) == L.RKV_EUNSUPPORTED
    assert _call_decode(L, g, num_blocks=(0xFFFFFFFF - 1) // 128, ws_bytes=16) == L.RKV_EWORKSPACE


def test_workspace_sizes(rkv_lib):
    L = rkv_lib
    g = L.gqa(8, 4, 128)
    a = L.rkv_hsa_workspace_bytes(g, 1, 16, 256, 32, 32)
    b = L.rkv_hsa_workspace_bytes(g, 32, 16, 400, 32, 64)
    assert a > 0 and b > 0
    # batch 1 (8 units) runs the split-K fused kernel: 16 splits of two pages,
    # each a (max, sum, acc[128]) partial per query head in fp32
    assert a >= 8 * 16 * 4 * (128 + 2) * 4
    # the split-K partials fit for every batch, also where the default rule
    # picks another form (the options can force split-K there)
    for (Hkv, G, d, B, k2) in [(8, 4, 128, 24, 64), (8, 4, 128, 32, 64), (8, 4, 128, 1, 32),
                               (2, 4, 64, 1, 16), (1, 4, 128, 200, 1024), (3, 1, 64, 4, 7)]:
        units = B * Hkv
        want = min(k2, -(-128 // units))
        pps = -(-k2 // want)
        nsp = -(-k2 // pps)
        need = units * nsp * G * (d + 2) * 4
        assert L.rkv_hsa_workspace_bytes(L.gqa(Hkv, G, d), B, 16, 400, 32, k2) >= need
    # the workspace follows the options only, never the environment: the
    # same arguments give the same size; a larger split-K target needs more
    os.environ["RKV_FUSED"] = "0"
    os.environ["RKV_SPLITK_BLOCKS"] = "4096"
    try:
        assert L.rkv_hsa_workspace_bytes(g, 1, 16, 256, 32, 32) == a
    finally:
        del os.environ["RKV_FUSED"], os.environ["RKV_SPLITK_BLOCKS"]
    big = L.rkv_hsa_workspace_bytes(g, 1, 16, 256, 32, 32, L.make_opts(splitk_blocks=256))
    assert big >= a + 8 * 16 * 4 * (128 + 2) * 4
    e1 = L.rkv_prefill_evict_workspace_bytes(g, 1, 32768, 32)
    # logits for 128 window rows over 32K keys dominate: 4 B each
    assert e1 >= 8 * 32768 * 128 * 4
    assert L.rkv_prefill_evict_workspace_bytes(L.gqa(8, 3, 128), 1, 100, 8) == 0


def test_evict_argument_checks(rkv_lib):
    L = rkv_lib
    lib = L.load_library()
    g = L.gqa(2, 2, 64)
    fake = 0x10000
    cache = L.rkv_paged_cache(fake, fake, fake, 64, 16, 4)

    def call(lens, keeps, w=8, pool=7, L_max=100, stride=0, ws=1 << 30):
        B = len(lens)
        return lib.rkv_prefill_evict(
            ctypes.byref(g), 0, B, (ctypes.c_int32 * B)(*lens), (ctypes.c_int32 * B)(*keeps),
            L_max, w, pool, 0.125, fake, fake, fake, ctypes.byref(cache), None,
            fake if stride else None, stride, None, None, fake, ws, None, None)

    assert call([50], [20], pool=4) == L.RKV_EINVAL          # even pooling kernel
    assert call([50], [5]) == L.RKV_EINVAL                   # keep below window
    assert call([150], [20]) == L.RKV_EINVAL                 # prompt longer than L_max
    assert call([100], [80]) == L.RKV_ECAPACITY              # 80 rows > 4 pages x 16
    assert call([50], [20], stride=10) == L.RKV_EINVAL       # kept_idx row too short
    assert call([50], [20], ws=100) == L.RKV_EWORKSPACE
    assert call([50] * 200, [20] * 200) == L.RKV_EUNSUPPORTED  # batch above the limit


def test_evict_chunk_argument_checks(rkv_lib):
    L = rkv_lib
    lib = L.load_library()
    g = L.gqa(2, 2, 64)
    fake = 0x10000
    cache = L.rkv_paged_cache(fake, fake, fake, 64, 16, 4)

    def call(n_cached, chunks, keeps, w=8, C_max=100, ws=1 << 30):
        B = len(chunks)
        arr = lambda xs: (ctypes.c_int32 * B)(*xs)
        return lib.rkv_prefill_evict_chunk(
            ctypes.byref(g), 0, B, arr(n_cached), arr(chunks), arr(keeps), C_max, w, 7, 0.125,
            fake, fake, fake, ctypes.byref(cache), None, None, 0, None, None, fake, ws, None, None)

    assert call([40], [30], [20], w=40) == L.RKV_EINVAL     # evicting with a chunk below w
    assert call([40], [120], [20]) == L.RKV_EINVAL          # chunk longer than C_max
    assert call([-1], [30], [20]) == L.RKV_EINVAL           # negative row count
    assert call([70], [30], [20]) == L.RKV_ECAPACITY        # 70 cached rows > 4 pages x 16
    assert call([40], [30], [20], ws=100) == L.RKV_EWORKSPACE
    assert lib.rkv_prefill_evict_chunk_workspace_bytes(ctypes.byref(g), 1, 70, 8) > 0


def test_decode_mode_rule(rkv_lib):
    """Which decode form runs (host-only query): the documented rule, forms
    forced through rkv_opts, and argument errors.  The environment plays no
    part."""
    L = rkv_lib
    S, F, K = L.RKV_FORM_STANDALONE, L.RKV_FORM_FUSED, L.RKV_FORM_SPLITK
    g = L.gqa(8, 4, 128)
    os.environ["RKV_FUSED"] = "0"
    try:
        assert L.decode_mode(g, 32, 16, 400, 64, 32) == F      # 256 units fill the chip
    finally:
        del os.environ["RKV_FUSED"]
    assert L.decode_mode(g, 1, 16, 216, 32, 32) == K       # batch 1: split-K
    assert L.decode_mode(g, 4, 32, 4400, 128, 32) == S     # beyond the fused page limit
    assert L.decode_mode(g, 1, 16, 600, 32, 32) == S       # stage too small for 600 pages
    assert L.decode_mode(L.gqa(2, 8, 128), 1, 16, 64, 16, 16) == K   # G = 8: 8-wave blocks
    assert L.decode_mode(L.gqa(2, 8, 128), 1, 16, 600, 16, 16) == S  # their stage: 512 pages
    assert L.decode_mode(L.gqa(32, 8, 128), 8, 16, 400, 64, 32) == F
    assert L.decode_mode(L.gqa(2, 4, 64), 1, 16, 130, 16, 16, L.RKV_F32) == K
    # a selection of more rows than one block's table (128 pages x 32 rows):
    # split-K, each share within the table
    assert L.decode_mode(g, 4, 32, 208, 128, 32) == K
    assert L.decode_mode(g, 32, 32, 208, 128, 32) == K
    o = L.make_opts
    assert L.decode_mode(g, 32, 16, 400, 64, 32, opts=o(form=S)) == S
    assert L.decode_mode(g, 32, 16, 400, 64, 32, opts=o(form=K)) == K
    assert L.decode_mode(g, 1, 16, 600, 32, 32, opts=o(form=K)) == S   # not past the stage
    assert L.decode_mode(g, 1, 16, 216, 32, 32, opts=o(form=F)) == F
    assert L.decode_mode(g, 4, 32, 4400, 128, 32, opts=o(form=F)) == S  # not past the limits
    assert L.decode_mode(g, 4, 32, 208, 128, 32, opts=o(form=F)) == S   # rows beyond one block
    assert L.decode_mode(g, 1, 16, 216, 32, 32, opts=o(form=L.RKV_FORM_AUTO)) == K
    lib = L.load_library()
    assert lib.rkv_decode_mode(ctypes.byref(g), 1, 0, 16, 100, 8, 8, None) == L.RKV_EINVAL
    assert lib.rkv_decode_mode(ctypes.byref(g), 1, 1, 16, 100, 0, 8, None) == L.RKV_EINVAL
    assert lib.rkv_decode_mode(ctypes.byref(g), 7, 1, 16, 100, 8, 8, None) == L.RKV_EUNSUPPORTED
    assert lib.rkv_decode_mode(None, 1, 1, 16, 100, 8, 8, None) == L.RKV_EINVAL


def test_no_environment_lookups_in_the_library():
    """Every choice the library makes comes from its arguments: no source
    file reads the environment."""
    csrc = os.path.join(ROOT, "sparse_kv_cache_hsa_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert "getenv" not in text and "environ" not in text, name


def test_static_decode_rejects_oversized_shapes(rkv_lib):
    """rkv_decode_step_static refuses shapes whose workspace exceeds the
    static scratch (before any device work)."""
    L = rkv_lib
    lib = L.load_library()
    g = L.gqa(8, 4, 128)
    B, P, max_pages, k1, k2 = 4096, 16, 4096, 32, 1024
    assert L.rkv_hsa_workspace_bytes(g, B, P, max_pages, k1, k2) > L.RKV_STATIC_SCRATCH_BYTES
    fake = 0x10000  # never dereferenced: the size check fails first
    cache = L.rkv_paged_cache(fake, fake, fake, 64, P, max_pages)
    st = lib.rkv_decode_step_static(ctypes.byref(g), L.RKV_BF16, B, fake, None, None,
                                    ctypes.byref(cache), fake, fake, k1, k2, 0.1, fake, None,
                                    None, None, None, None)
    assert st == L.RKV_ESCRATCH
    assert lib.rkv_status_string(st).decode().startswith("shapes need more")
    # argument errors still come first
    assert lib.rkv_decode_step_static(None, L.RKV_BF16, 1, fake, None, None, ctypes.byref(cache),
                                      fake, fake, k1, 8, 0.1, fake, None, None, None, None,
                                      None) == L.RKV_EINVAL


def test_turn_filter_argument_checks(rkv_lib):
    L = rkv_lib
    lib = L.load_library()
    g = L.gqa(2, 2, 64)
    fake = 0x10000
    full = L.rkv_paged_cache(fake, fake, fake, 64, 16, 20)   # 320 rows
    view = L.rkv_paged_cache(fake, fake, fake, 64, 16, 4)    # 64 rows

    def call(n_rows, keeps, w=8, pool=7, ws=1 << 30, stride=0):
        B = len(n_rows)
        arr = lambda xs: (ctypes.c_int32 * B)(*xs)
        return lib.rkv_turn_filter(ctypes.byref(g), 0, B, arr(n_rows), arr(keeps), w, pool,
                                   0.125, fake, ctypes.byref(full), ctypes.byref(view), None,
                                   fake if stride else None, stride, None, None, fake, ws, None,
                                   None)

    assert call([200], [40], pool=4) == L.RKV_EINVAL       # even pooling kernel
    assert call([200], [5]) == L.RKV_EINVAL                # keep below the window
    assert call([400], [40]) == L.RKV_ECAPACITY            # history beyond the full cache
    assert call([200], [80]) == L.RKV_ECAPACITY            # view beyond its capacity
    # keep >= n copies the whole history, which must fit the view
    assert call([70], [100]) == L.RKV_ECAPACITY
    assert call([200], [40], stride=10) == L.RKV_EINVAL    # kept_idx row too short
    assert call([200], [40], ws=100) == L.RKV_EWORKSPACE
    assert L.rkv_turn_filter_workspace_bytes(g, 1, 320, 8) > 0


def test_read_probe_argument_checks(rkv_lib):
    """The read probe rejects a null buffer or sink, an unaligned buffer and
    an empty read on the host, before any launch (the pointers below are
    never dereferenced)."""
    L = rkv_lib.load_library()
    sink = ctypes.c_void_p(4096)
    assert L.rkv_read_probe(None, None, 1, sink, None) == rkv_lib.RKV_EINVAL
    assert L.rkv_read_probe(ctypes.c_void_p(4096), None, 1, None, None) == rkv_lib.RKV_EINVAL
    assert L.rkv_read_probe(ctypes.c_void_p(4100), None, 1, sink, None) == rkv_lib.RKV_EINVAL
    assert L.rkv_read_probe(ctypes.c_void_p(4096), None, 0, sink, None) == rkv_lib.RKV_EINVAL
