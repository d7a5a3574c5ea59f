"""Thin ctypes binding of librkv (the C ABI in include/rkv.h).

Argument marshalling only: every step of the decode path runs in librkv's
HIP kernels.  Tensors are torch CUDA tensors (PyTorch supplies device memory
and the current stream); dtypes map float32 -> RKV_F32, bfloat16 -> RKV_BF16.
The library is loaded on first use and must have been built from the
sources next to it (``sparse_kv_cache_hsa_amd.build``); a missing or stale
build raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import torch

from . import build as _build

RKV_OK = 0
RKV_EINVAL = -1
RKV_EWORKSPACE = -2
RKV_ECAPACITY = -3
RKV_EUNSUPPORTED = -4
RKV_EHIP = -5
RKV_ESCRATCH = -6
RKV_STATIC_SCRATCH_BYTES = 16 << 20
RKV_F32 = 0
RKV_BF16 = 1
RKV_MAX_K2 = 4096
RKV_MAX_EVICT_BATCH = 128
RKV_FORM_AUTO = 0
RKV_FORM_STANDALONE = 1
RKV_FORM_FUSED = 2
RKV_FORM_SPLITK = 3
RKV_DEV_LENGTH = 1
RKV_DEV_BLOCK = 2
RKV_DEV_PAGE = 4
RKV_READ_PROBE_CHUNK = 4096
RKV_READ_PROBE_BLOCKS = 2048
RKV_READ_PROBE_SINK_WORDS = RKV_READ_PROBE_BLOCKS * 4

EXPORTED = (
    "rkv_status_string", "rkv_build_id", "rkv_split_ratio",
    "rkv_prefill_evict_workspace_bytes", "rkv_prefill_evict", "rkv_append_summaries",
    "rkv_hsa_workspace_bytes", "rkv_hsa_select", "rkv_hsa_attend", "rkv_hsa_decode",
    "rkv_decode_step", "rkv_prefill_evict_chunk_workspace_bytes", "rkv_prefill_evict_chunk",
    "rkv_decode_mode", "rkv_decode_step_static", "rkv_turn_filter_workspace_bytes",
    "rkv_turn_filter", "rkv_read_probe",
)


class RkvError(RuntimeError):
    def __init__(self, where: str, status: int, text: str):
        super().__init__(f"{where}: status {status} ({text})")
        self.status = status


class rkv_gqa(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class rkv_paged_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


RKV_TRACE_SLOTS = 32


class rkv_opts(ctypes.Structure):
    _fields_ = [("form", ctypes.c_int32), ("splitk_blocks", ctypes.c_int32),
                ("select_chunk", ctypes.c_int32), ("select_radix", ctypes.c_int32),
                ("attend_variant", ctypes.c_int32), ("attend_pages", ctypes.c_int32),
                ("status", ctypes.c_void_p), ("trace", ctypes.c_void_p)]


def make_opts(form: int = RKV_FORM_AUTO, splitk_blocks: int = 0, select_chunk: int = 0,
              select_radix: int = 0, attend_variant: int = 0, attend_pages: int = 0,
              status: torch.Tensor | None = None,
              trace: torch.Tensor | None = None) -> rkv_opts:
    """Execution options (include/rkv.h rkv_opts).  status: optional device
    int32 tensor of one element that receives RKV_DEV_* flags.  trace:
    optional device int64 tensor of RKV_TRACE_SLOTS stamps per block, written
    only by the phase-timing build."""
    if status is not None:
        _need(status, "status", torch.int32)
    if trace is not None:
        _need(trace, "trace", torch.int64)
    return rkv_opts(int(form), int(splitk_blocks), int(select_chunk), int(select_radix),
                    int(attend_variant), int(attend_pages), _ptr(status), _ptr(trace))


def _opt(o: rkv_opts | None):
    return None if o is None else ctypes.byref(o)


_LOCK = threading.Lock()
_LIB = None


def load_library(path: str | None = None, check_build_id: bool = True):
    """Loads librkv.so (once).  Raises if it is missing or stale."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = path or _build.LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        i32, i64, f32, f64, vp, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t)
        P = ctypes.POINTER
        G, C, O = P(rkv_gqa), P(rkv_paged_cache), P(rkv_opts)
        lib.rkv_status_string.argtypes = [ctypes.c_int]
        lib.rkv_status_string.restype = ctypes.c_char_p
        lib.rkv_build_id.argtypes = []
        lib.rkv_build_id.restype = ctypes.c_char_p
        lib.rkv_split_ratio.argtypes = [f64, i64, i64, P(f64), P(f64), P(f64), P(i64)]
        lib.rkv_split_ratio.restype = ctypes.c_int
        lib.rkv_prefill_evict_workspace_bytes.argtypes = [G, i32, i64, i32]
        lib.rkv_prefill_evict_workspace_bytes.restype = sz
        lib.rkv_prefill_evict.argtypes = [G, i32, i32, P(i32), P(i32), i64, i32, i32, f32, vp,
                                          vp, vp, C, vp, vp, i32, vp, vp, vp, sz, vp, O]
        lib.rkv_prefill_evict.restype = ctypes.c_int
        lib.rkv_prefill_evict_chunk_workspace_bytes.argtypes = [G, i32, i64, i32]
        lib.rkv_prefill_evict_chunk_workspace_bytes.restype = sz
        lib.rkv_prefill_evict_chunk.argtypes = [G, i32, i32, P(i32), P(i32), P(i32), i64, i32,
                                                i32, f32, vp, vp, vp, C, vp, vp, i32, vp, vp,
                                                vp, sz, vp, O]
        lib.rkv_prefill_evict_chunk.restype = ctypes.c_int
        lib.rkv_turn_filter_workspace_bytes.argtypes = [G, i32, i64, i32]
        lib.rkv_turn_filter_workspace_bytes.restype = sz
        lib.rkv_turn_filter.argtypes = [G, i32, i32, P(i32), P(i32), i32, i32, f32, vp, C, C, vp,
                                        vp, i32, vp, vp, vp, sz, vp, O]
        lib.rkv_turn_filter.restype = ctypes.c_int
        lib.rkv_append_summaries.argtypes = [G, i32, i32, C, vp, vp, i32, vp, vp, vp, vp, O]
        lib.rkv_append_summaries.restype = ctypes.c_int
        lib.rkv_hsa_workspace_bytes.argtypes = [G, i32, i32, i32, i32, i32, O]
        lib.rkv_hsa_workspace_bytes.restype = sz
        lib.rkv_decode_mode.argtypes = [G, i32, i32, i32, i32, i32, i32, O]
        lib.rkv_decode_mode.restype = ctypes.c_int
        lib.rkv_hsa_select.argtypes = [G, i32, i32, vp, vp, i32, i32, vp, i32, i32, vp, vp, vp,
                                       vp, sz, vp, O]
        lib.rkv_hsa_select.restype = ctypes.c_int
        lib.rkv_hsa_attend.argtypes = [G, i32, i32, vp, C, vp, vp, i32, f32, vp, vp, sz, vp, O]
        lib.rkv_hsa_attend.restype = ctypes.c_int
        lib.rkv_hsa_decode.argtypes = [G, i32, i32, vp, C, vp, vp, i32, i32, f32, vp, vp, vp,
                                       vp, vp, sz, vp, O]
        lib.rkv_hsa_decode.restype = ctypes.c_int
        lib.rkv_decode_step.argtypes = [G, i32, i32, vp, vp, vp, C, vp, vp, i32, i32, f32, vp,
                                        vp, vp, vp, vp, sz, vp, O]
        lib.rkv_decode_step.restype = ctypes.c_int
        lib.rkv_decode_step_static.argtypes = [G, i32, i32, vp, vp, vp, C, vp, vp, i32, i32, f32,
                                               vp, vp, vp, vp, vp, O]
        lib.rkv_decode_step_static.restype = ctypes.c_int
        lib.rkv_read_probe.argtypes = [vp, vp, i64, vp, vp]
        lib.rkv_read_probe.restype = ctypes.c_int
        if check_build_id:
            built = lib.rkv_build_id().decode()
            want = _build.source_hash()
            if built != want:
                raise RuntimeError(f"{path} was built from other sources (build id {built}, "
                                   f"sources {want}); run __graft_entry__.build() again")
        _LIB = lib
        return lib


def _check(where: str, status: int) -> None:
    if status != RKV_OK:
        raise RkvError(where, status, load_library().rkv_status_string(status).decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RKV_F32
    if t.dtype == torch.bfloat16:
        return RKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor | None, name: str, dtype=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def gqa(n_kv_heads: int, group: int, head_dim: int) -> rkv_gqa:
    return rkv_gqa(int(n_kv_heads), int(group), int(head_dim))


@dataclass
class PagedCache:
    """A paged KV cache as librkv sees it (tensors are caller-owned)."""
    k_pool: torch.Tensor      # [num_blocks, Hkv, P, d]
    v_pool: torch.Tensor      # [num_blocks, Hkv, P, d]
    page_table: torch.Tensor  # [B, max_pages] int32

    @property
    def page_size(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def c_struct(self) -> rkv_paged_cache:
        _need(self.k_pool, "k_pool")
        _need(self.v_pool, "v_pool", self.k_pool.dtype)
        _need(self.page_table, "page_table", torch.int32)
        return rkv_paged_cache(self.k_pool.data_ptr(), self.v_pool.data_ptr(),
                               self.page_table.data_ptr(), int(self.k_pool.shape[0]),
                               self.page_size, self.max_pages)

    def row_slice(self, b0: int, b1: int) -> "PagedCache":
        """The same pools with the page-table rows of sequences [b0, b1)."""
        return PagedCache(self.k_pool, self.v_pool, self.page_table[b0:b1])


def decode_mode(g: rkv_gqa, B: int, page_size: int, max_pages: int, k2: int, k1: int = 1,
                dtype: int = RKV_BF16, opts: rkv_opts | None = None) -> int:
    """How rkv_decode_step runs for these shapes and options
    (rkv_decode_mode, the rule documented in include/rkv.h):
    RKV_FORM_STANDALONE, RKV_FORM_FUSED (one block per (sequence, KV head))
    or RKV_FORM_SPLITK (the fused kernel split K-wise, plus the merge)."""
    mode = load_library().rkv_decode_mode(ctypes.byref(g), dtype, B, page_size, max_pages, k1, k2,
                                          _opt(opts))
    if mode < 0:
        _check("rkv_decode_mode", mode)
    return mode


def fused_path(g: rkv_gqa, B: int, page_size: int, max_pages: int, k2: int, k1: int = 1,
               dtype: int = RKV_BF16, opts: rkv_opts | None = None) -> bool:
    """Whether rkv_decode_step runs as the fused kernel with one block per
    (sequence, KV head)."""
    return decode_mode(g, B, page_size, max_pages, k2, k1, dtype, opts) == RKV_FORM_FUSED


# ---- entry points (same names as the C ABI) ---------------------------------

def rkv_split_ratio(c: float, L: int, w: int = 0):
    """Returns (r, c_evict, c_hsa, keep)."""
    r, ce, ch = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    keep = ctypes.c_int64()
    _check("rkv_split_ratio", load_library().rkv_split_ratio(
        float(c), int(L), int(w), ctypes.byref(r), ctypes.byref(ce), ctypes.byref(ch),
        ctypes.byref(keep)))
    return r.value, ce.value, ch.value, keep.value


def rkv_prefill_evict_workspace_bytes(g: rkv_gqa, B: int, L_max: int, w: int) -> int:
    return int(load_library().rkv_prefill_evict_workspace_bytes(ctypes.byref(g), B, L_max, w))


def rkv_prefill_evict(g: rkv_gqa, prompt_lens, keep, q_win: torch.Tensor, k: torch.Tensor,
                      v: torch.Tensor, w: int, pool_kernel: int, scale: float,
                      cache: PagedCache, summaries: torch.Tensor | None = None,
                      kept_idx: torch.Tensor | None = None,
                      pooled_scores: torch.Tensor | None = None,
                      seq_lens_out: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, opts: rkv_opts | None = None) -> None:
    """SnapKV++ eviction.  prompt_lens/keep: host sequences of ints (length B);
    q_win [B, Hq, w, d]; k, v [B, Hkv, L_max, d]."""
    _need(k, "k")
    _need(v, "v", k.dtype)
    _need(q_win, "q_win", k.dtype)
    _need(summaries, "summaries", k.dtype, optional=True)
    _need(kept_idx, "kept_idx", torch.int32, optional=True)
    _need(pooled_scores, "pooled_scores", torch.float32, optional=True)
    _need(seq_lens_out, "seq_lens_out", torch.int32, optional=True)
    B, L_max = int(k.shape[0]), int(k.shape[2])
    lens = (ctypes.c_int32 * B)(*[int(x) for x in prompt_lens])
    keeps = (ctypes.c_int32 * B)(*[int(x) for x in keep])
    if ws is None:
        ws = torch.empty(rkv_prefill_evict_workspace_bytes(g, B, L_max, w), dtype=torch.uint8,
                         device=k.device)
    _need(ws, "ws")
    cs = cache.c_struct()
    stride = int(kept_idx.shape[-1]) if kept_idx is not None else 0
    _check("rkv_prefill_evict", load_library().rkv_prefill_evict(
        ctypes.byref(g), _dtype_code(k), B, lens, keeps, L_max, int(w), int(pool_kernel),
        float(scale), q_win.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(cs),
        _ptr(summaries), _ptr(kept_idx), stride, _ptr(pooled_scores), _ptr(seq_lens_out),
        ws.data_ptr(), ws.numel(), _stream(), _opt(opts)))


def rkv_prefill_evict_chunk_workspace_bytes(g: rkv_gqa, B: int, L_max: int, w: int) -> int:
    return int(load_library().rkv_prefill_evict_chunk_workspace_bytes(ctypes.byref(g), B, L_max,
                                                                      w))


def rkv_prefill_evict_chunk(g: rkv_gqa, n_cached, chunk_lens, keep, q_win: torch.Tensor,
                            k_chunk: torch.Tensor, v_chunk: torch.Tensor, w: int,
                            pool_kernel: int, scale: float, cache: PagedCache,
                            summaries: torch.Tensor | None = None,
                            kept_idx: torch.Tensor | None = None,
                            pooled_scores: torch.Tensor | None = None,
                            seq_lens_out: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None,
                            opts: rkv_opts | None = None) -> None:
    """SnapKV++ eviction over the cached rows followed by a prefill chunk.
    n_cached/chunk_lens/keep: host sequences of ints (length B); q_win
    [B, Hq, w, d] (the chunk's last w queries); k_chunk, v_chunk
    [B, Hkv, C_max, d].  kept_idx and pooled_scores index the concatenated
    sequence; pooled_scores is [B, Hkv, max(n_cached + chunk_lens)]."""
    _need(k_chunk, "k_chunk")
    _need(v_chunk, "v_chunk", k_chunk.dtype)
    _need(q_win, "q_win", k_chunk.dtype)
    _need(summaries, "summaries", k_chunk.dtype, optional=True)
    _need(kept_idx, "kept_idx", torch.int32, optional=True)
    _need(pooled_scores, "pooled_scores", torch.float32, optional=True)
    _need(seq_lens_out, "seq_lens_out", torch.int32, optional=True)
    B, C_max = int(k_chunk.shape[0]), int(k_chunk.shape[2])
    nc = (ctypes.c_int32 * B)(*[int(x) for x in n_cached])
    cl = (ctypes.c_int32 * B)(*[int(x) for x in chunk_lens])
    keeps = (ctypes.c_int32 * B)(*[int(x) for x in keep])
    L_max = max(1, max(int(a) + int(c) for a, c in zip(n_cached, chunk_lens)))
    if ws is None:
        ws = torch.empty(rkv_prefill_evict_chunk_workspace_bytes(g, B, L_max, w),
                         dtype=torch.uint8, device=k_chunk.device)
    _need(ws, "ws")
    cs = cache.c_struct()
    stride = int(kept_idx.shape[-1]) if kept_idx is not None else 0
    _check("rkv_prefill_evict_chunk", load_library().rkv_prefill_evict_chunk(
        ctypes.byref(g), _dtype_code(k_chunk), B, nc, cl, keeps, C_max, int(w),
        int(pool_kernel), float(scale), q_win.data_ptr(), k_chunk.data_ptr(),
        v_chunk.data_ptr(), ctypes.byref(cs), _ptr(summaries), _ptr(kept_idx), stride,
        _ptr(pooled_scores), _ptr(seq_lens_out), ws.data_ptr(), ws.numel(), _stream(), _opt(opts)))


def rkv_turn_filter_workspace_bytes(g: rkv_gqa, B: int, L_max: int, w: int) -> int:
    return int(load_library().rkv_turn_filter_workspace_bytes(ctypes.byref(g), B, L_max, w))


def rkv_turn_filter(g: rkv_gqa, n_rows, keep, q_win: torch.Tensor, w: int, pool_kernel: int,
                    scale: float, full: PagedCache, view: PagedCache,
                    view_summaries: torch.Tensor | None = None,
                    kept_idx: torch.Tensor | None = None,
                    pooled_scores: torch.Tensor | None = None,
                    view_lens_out: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, opts: rkv_opts | None = None) -> None:
    """RocketKV-MT's per-turn view: SnapKV++ over the first n_rows[b] rows of
    `full` (only read) with the turn's last w queries q_win [B, Hq, w, d];
    the kept rows go to `view`.  n_rows/keep: host sequences of ints."""
    _need(q_win, "q_win", full.k_pool.dtype)
    _need(view_summaries, "view_summaries", full.k_pool.dtype, optional=True)
    _need(kept_idx, "kept_idx", torch.int32, optional=True)
    _need(pooled_scores, "pooled_scores", torch.float32, optional=True)
    _need(view_lens_out, "view_lens_out", torch.int32, optional=True)
    B = int(q_win.shape[0])
    nr = (ctypes.c_int32 * B)(*[int(x) for x in n_rows])
    kp = (ctypes.c_int32 * B)(*[int(x) for x in keep])
    if ws is None:
        ws = torch.empty(rkv_turn_filter_workspace_bytes(g, B, max(1, max(int(x) for x in n_rows)),
                                                         w), dtype=torch.uint8,
                         device=q_win.device)
    _need(ws, "ws")
    fs, vs = full.c_struct(), view.c_struct()
    stride = int(kept_idx.shape[-1]) if kept_idx is not None else 0
    _check("rkv_turn_filter", load_library().rkv_turn_filter(
        ctypes.byref(g), _dtype_code(q_win), B, nr, kp, int(w), int(pool_kernel), float(scale),
        q_win.data_ptr(), ctypes.byref(fs), ctypes.byref(vs), _ptr(view_summaries),
        _ptr(kept_idx), stride, _ptr(pooled_scores), _ptr(view_lens_out), ws.data_ptr(),
        ws.numel(), _stream(), _opt(opts)))


def rkv_append_summaries(g: rkv_gqa, cache: PagedCache, n_old: torch.Tensor,
                         n_new: torch.Tensor, max_new_rows: int, summaries: torch.Tensor,
                         k_src: torch.Tensor | None = None,
                         v_src: torch.Tensor | None = None,
                         opts: rkv_opts | None = None) -> None:
    """Fold rows [n_old, n_new) into the page summaries, first copying them
    from k_src/v_src [B, Hkv, max_new_rows, d] into the cache when given."""
    _need(n_old, "n_old", torch.int32)
    _need(n_new, "n_new", torch.int32)
    _need(summaries, "summaries", cache.k_pool.dtype)
    _need(k_src, "k_src", cache.k_pool.dtype, optional=True)
    _need(v_src, "v_src", cache.k_pool.dtype, optional=True)
    cs = cache.c_struct()
    _check("rkv_append_summaries", load_library().rkv_append_summaries(
        ctypes.byref(g), _dtype_code(summaries), int(n_old.shape[0]), ctypes.byref(cs),
        n_old.data_ptr(), n_new.data_ptr(), int(max_new_rows), _ptr(k_src), _ptr(v_src),
        summaries.data_ptr(), _stream(), _opt(opts)))


def rkv_hsa_workspace_bytes(g: rkv_gqa, B: int, page_size: int, max_pages: int, k1: int,
                            k2: int, opts: rkv_opts | None = None) -> int:
    return int(load_library().rkv_hsa_workspace_bytes(ctypes.byref(g), B, page_size,
                                                      max_pages, k1, k2, _opt(opts)))


def hsa_workspace(g: rkv_gqa, B: int, page_size: int, max_pages: int, k1: int, k2: int,
                  device, opts: rkv_opts | None = None) -> torch.Tensor:
    return torch.zeros(rkv_hsa_workspace_bytes(g, B, page_size, max_pages, k1, k2, opts),
                       dtype=torch.uint8, device=device)


def rkv_hsa_select(g: rkv_gqa, q: torch.Tensor, seq_lens: torch.Tensor, page_size: int,
                   summaries: torch.Tensor, k1: int, k2: int, page_idx: torch.Tensor,
                   ws: torch.Tensor, chan_idx: torch.Tensor | None = None,
                   page_scores: torch.Tensor | None = None,
                   opts: rkv_opts | None = None) -> None:
    _need(q, "q")
    _need(seq_lens, "seq_lens", torch.int32)
    _need(summaries, "summaries", q.dtype)
    _need(page_idx, "page_idx", torch.int32)
    _need(chan_idx, "chan_idx", torch.int32, optional=True)
    _need(page_scores, "page_scores", torch.float32, optional=True)
    _need(ws, "ws")
    max_pages = int(summaries.shape[-1])
    _check("rkv_hsa_select", load_library().rkv_hsa_select(
        ctypes.byref(g), _dtype_code(q), int(q.shape[0]), q.data_ptr(), seq_lens.data_ptr(),
        int(page_size), max_pages, summaries.data_ptr(), int(k1), int(k2), _ptr(chan_idx),
        page_idx.data_ptr(), _ptr(page_scores), ws.data_ptr(), ws.numel(), _stream(), _opt(opts)))


def rkv_hsa_attend(g: rkv_gqa, q: torch.Tensor, cache: PagedCache, seq_lens: torch.Tensor,
                   page_idx: torch.Tensor, k2: int, scale: float, out: torch.Tensor,
                   ws: torch.Tensor, opts: rkv_opts | None = None) -> None:
    _need(q, "q", cache.k_pool.dtype)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(page_idx, "page_idx", torch.int32)
    _need(out, "out", torch.float32)
    _need(ws, "ws")
    cs = cache.c_struct()
    _check("rkv_hsa_attend", load_library().rkv_hsa_attend(
        ctypes.byref(g), _dtype_code(q), int(q.shape[0]), q.data_ptr(), ctypes.byref(cs),
        seq_lens.data_ptr(), page_idx.data_ptr(), int(k2), float(scale), out.data_ptr(),
        ws.data_ptr(), ws.numel(), _stream(), _opt(opts)))


def rkv_hsa_decode(g: rkv_gqa, q: torch.Tensor, cache: PagedCache, seq_lens: torch.Tensor,
                   summaries: torch.Tensor, k1: int, k2: int, scale: float, out: torch.Tensor,
                   ws: torch.Tensor, chan_idx: torch.Tensor | None = None,
                   page_idx: torch.Tensor | None = None,
                   page_scores: torch.Tensor | None = None,
                   opts: rkv_opts | None = None) -> None:
    _need(q, "q", cache.k_pool.dtype)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(summaries, "summaries", q.dtype)
    _need(out, "out", torch.float32)
    _need(chan_idx, "chan_idx", torch.int32, optional=True)
    _need(page_idx, "page_idx", torch.int32, optional=True)
    _need(page_scores, "page_scores", torch.float32, optional=True)
    _need(ws, "ws")
    cs = cache.c_struct()
    _check("rkv_hsa_decode", load_library().rkv_hsa_decode(
        ctypes.byref(g), _dtype_code(q), int(q.shape[0]), q.data_ptr(), ctypes.byref(cs),
        seq_lens.data_ptr(), summaries.data_ptr(), int(k1), int(k2), float(scale),
        out.data_ptr(), _ptr(chan_idx), _ptr(page_idx), _ptr(page_scores), ws.data_ptr(),
        ws.numel(), _stream(), _opt(opts)))


def rkv_decode_step(g: rkv_gqa, q: torch.Tensor, k_new: torch.Tensor | None,
                    v_new: torch.Tensor | None, cache: PagedCache, seq_lens: torch.Tensor,
                    summaries: torch.Tensor, k1: int, k2: int, scale: float, out: torch.Tensor,
                    ws: torch.Tensor, chan_idx: torch.Tensor | None = None,
                    page_idx: torch.Tensor | None = None,
                    page_scores: torch.Tensor | None = None,
                    opts: rkv_opts | None = None) -> None:
    """Append the new token (row seq_lens-1 from k_new/v_new [B, Hkv, d]) and
    run HSA decode, in one call per layer."""
    _need(q, "q", cache.k_pool.dtype)
    _need(k_new, "k_new", q.dtype, optional=True)
    _need(v_new, "v_new", q.dtype, optional=True)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(summaries, "summaries", q.dtype)
    _need(out, "out", torch.float32)
    _need(chan_idx, "chan_idx", torch.int32, optional=True)
    _need(page_idx, "page_idx", torch.int32, optional=True)
    _need(page_scores, "page_scores", torch.float32, optional=True)
    _need(ws, "ws")
    cs = cache.c_struct()
    _check("rkv_decode_step", load_library().rkv_decode_step(
        ctypes.byref(g), _dtype_code(q), int(q.shape[0]), q.data_ptr(), _ptr(k_new),
        _ptr(v_new), ctypes.byref(cs), seq_lens.data_ptr(), summaries.data_ptr(), int(k1),
        int(k2), float(scale), out.data_ptr(), _ptr(chan_idx), _ptr(page_idx),
        _ptr(page_scores), ws.data_ptr(), ws.numel(), _stream(), _opt(opts)))


def rkv_decode_step_static(g: rkv_gqa, q: torch.Tensor, k_new: torch.Tensor | None,
                           v_new: torch.Tensor | None, cache: PagedCache, seq_lens: torch.Tensor,
                           summaries: torch.Tensor, k1: int, k2: int, scale: float,
                           out: torch.Tensor, chan_idx: torch.Tensor | None = None,
                           page_idx: torch.Tensor | None = None,
                           page_scores: torch.Tensor | None = None,
                           opts: rkv_opts | None = None) -> None:
    """rkv_decode_step with the library's static device scratch as the
    workspace (no allocation; calls that overlap on one GPU race)."""
    _need(q, "q", cache.k_pool.dtype)
    _need(k_new, "k_new", q.dtype, optional=True)
    _need(v_new, "v_new", q.dtype, optional=True)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(summaries, "summaries", q.dtype)
    _need(out, "out", torch.float32)
    _need(chan_idx, "chan_idx", torch.int32, optional=True)
    _need(page_idx, "page_idx", torch.int32, optional=True)
    _need(page_scores, "page_scores", torch.float32, optional=True)
    cs = cache.c_struct()
    _check("rkv_decode_step_static", load_library().rkv_decode_step_static(
        ctypes.byref(g), _dtype_code(q), int(q.shape[0]), q.data_ptr(), _ptr(k_new),
        _ptr(v_new), ctypes.byref(cs), seq_lens.data_ptr(), summaries.data_ptr(), int(k1),
        int(k2), float(scale), out.data_ptr(), _ptr(chan_idx), _ptr(page_idx),
        _ptr(page_scores), _stream(), _opt(opts)))


def rkv_read_probe(buf: torch.Tensor, sink: torch.Tensor, offsets: torch.Tensor | None = None,
                   n_chunks: int | None = None, check_offsets: bool = True) -> None:
    """Measurement helper: reads RKV_READ_PROBE_CHUNK-byte chunks of buf (a
    device tensor, consecutive chunks, or the ones starting at the int64
    byte offsets) and stores per-wave XORs of the words read into sink
    (uint32 words as an int32 tensor of RKV_READ_PROBE_SINK_WORDS).  The
    library does not check device offsets; check_offsets does it here (a
    host synchronisation: pass False inside a timed loop once a call with
    the same offsets has checked them)."""
    if not buf.is_cuda or not sink.is_cuda:
        raise ValueError("rkv_read_probe: buf and sink must be device tensors")
    if sink.dtype != torch.int32 or sink.numel() < RKV_READ_PROBE_SINK_WORDS:
        raise ValueError("rkv_read_probe: sink must be int32 with RKV_READ_PROBE_SINK_WORDS words")
    nbytes = buf.numel() * buf.element_size()
    if offsets is not None:
        _need(offsets, "offsets", torch.int64)
        n = offsets.numel() if n_chunks is None else int(n_chunks)
        if n > offsets.numel():
            raise ValueError("rkv_read_probe: more chunks than offsets")
        if check_offsets and n > 0:
            o = offsets[:n]
            bad = ((o < 0) | (o % 16 != 0) | (o + RKV_READ_PROBE_CHUNK > nbytes)).any()
            if bool(bad.item()):
                raise ValueError("rkv_read_probe: an offset is unaligned or its chunk leaves buf")
    else:
        n = nbytes // RKV_READ_PROBE_CHUNK if n_chunks is None else int(n_chunks)
        if n * RKV_READ_PROBE_CHUNK > nbytes:
            raise ValueError("rkv_read_probe: buf holds fewer chunks than asked for")
    _check("rkv_read_probe", load_library().rkv_read_probe(
        buf.data_ptr(), _ptr(offsets), n, sink.data_ptr(), _stream()))
