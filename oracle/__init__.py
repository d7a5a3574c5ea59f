"""CPU oracle for the RocketKV decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it.

The arithmetic lives in ``rkv_oracle.c`` (plain C, compiled here with gcc and
``-ffp-contract=off``); this module only builds it and marshals numpy arrays.
Arrays are fp32 (``np.float32``) or bf16 stored as raw bits (``np.uint16``).

Parity status: every function is pinned by ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rkv_oracle.c")
_LOCK = threading.Lock()
_LIB = None

OK = 0
EINVAL = -1


def _src_hash() -> str:
    with open(_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _sanitized() -> bool:
    """RKV_ORACLE_SANITIZE=1 loads a build under AddressSanitizer and
    UndefinedBehaviorSanitizer (the process must preload libasan)."""
    return os.environ.get("RKV_ORACLE_SANITIZE", "") == "1"


def _lib_path(sanitize: bool = False) -> str:
    tag = "liboracle-asan-" if sanitize else "liboracle-"
    return os.path.join(_HERE, f"{tag}{_src_hash()}.so")


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile rkv_oracle.c into a shared library named after its content;
    sanitize=True: with -fsanitize=address,undefined, every UB report fatal."""
    path = _lib_path(sanitize)
    if force or not os.path.exists(path):
        tmp = path + f".tmp{os.getpid()}"
        cmd = ["gcc", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-fno-builtin", "-Wall", "-o", tmp, _SRC, "-lm"]
        if sanitize:
            cmd[1:1] = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all"]
        else:
            cmd[1:1] = ["-O2"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
        prefix = "liboracle-asan-" if sanitize else "liboracle-"
        for name in os.listdir(_HERE):
            if not (name.startswith(prefix) and name.endswith(".so")):
                continue
            if not sanitize and name.startswith("liboracle-asan-"):
                continue
            if os.path.join(_HERE, name) != path:
                try:
                    os.remove(os.path.join(_HERE, name))
                except OSError:
                    pass
    return path


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            lib = ctypes.CDLL(build(sanitize=_sanitized()))
            i64, i32, f32, f64, vp = (ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_void_p)
            P = ctypes.POINTER
            lib.rkvo_split_ratio.argtypes = [f64, i64, i64, P(f64), P(f64), P(f64), P(i64)]
            lib.rkvo_split_ratio.restype = i32
            lib.rkvo_summaries_rebuild.argtypes = [vp, i32, i64, i32, i32, vp, vp]
            lib.rkvo_summaries_rebuild.restype = None
            lib.rkvo_summaries_append.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
            lib.rkvo_summaries_append.restype = None
            lib.rkvo_snapkv_group.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, i64, f32,
                                              vp, vp, vp]
            lib.rkvo_snapkv_group.restype = i32
            lib.rkvo_hsa_group.argtypes = [vp, vp, vp, i32, vp, vp, i64, i32, i32, i32, i32,
                                           i32, f64, vp, vp, vp, vp]
            lib.rkvo_hsa_group.restype = i32
            _LIB = lib
    return _LIB


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _p(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


class OracleError(RuntimeError):
    pass


def split_ratio(c: float, L: int, w: int = 0):
    """Adaptive split: returns (r, c_evict, c_hsa, keep)."""
    r, c1, c2 = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    keep = ctypes.c_int64()
    rc = _lib().rkvo_split_ratio(float(c), int(L), int(w), ctypes.byref(r), ctypes.byref(c1),
                                 ctypes.byref(c2), ctypes.byref(keep))
    if rc != OK:
        raise OracleError(f"split_ratio: status {rc}")
    return r.value, c1.value, c2.value, keep.value


def summaries_rebuild(k: np.ndarray, P: int):
    """Page max/min summaries of rows k[n, d]; returns (smax, smin) [NP, d]."""
    k = _c(k)
    n, d = k.shape
    np_ = (n + P - 1) // P
    smax = np.zeros((np_, d), dtype=k.dtype)
    smin = np.zeros((np_, d), dtype=k.dtype)
    _lib().rkvo_summaries_rebuild(_p(k), _dt(k), n, d, P, _p(smax), _p(smin))
    return smax, smin


def summaries_append(k: np.ndarray, n_old: int, n_new: int, P: int,
                     smax: np.ndarray, smin: np.ndarray) -> None:
    """Fold rows [n_old, n_new) of k into smax/smin in place (arrays sized for
    at least ceil(n_new/P) pages)."""
    k = _c(k)
    assert smax.flags.c_contiguous and smin.flags.c_contiguous
    assert smax.dtype == k.dtype and smin.dtype == k.dtype
    assert smax.shape[0] * P >= n_new and k.shape[0] >= n_new
    _lib().rkvo_summaries_append(_p(k), _dt(k), int(n_old), int(n_new), k.shape[1], P,
                                 _p(smax), _p(smin))


def snapkv_group(q_win: np.ndarray, k: np.ndarray, pool_kernel: int, keep: int,
                 scale: float):
    """SnapKV++ for one KV head group.  q_win [G, w, d], k [L, d].
    Returns (kept[keep'] int32, A[L-w] fp32, pooled[L-w] fp32), keep' = min(keep, L)."""
    q_win, k = _c(q_win), _c(k)
    assert q_win.dtype == k.dtype
    G, w, d = q_win.shape
    L = k.shape[0]
    keep_eff = min(int(keep), L)
    npre = max(L - w, 0)
    kept = np.full(max(keep_eff, 1), -1, dtype=np.int32)
    A = np.zeros(max(npre, 1), dtype=np.float32)
    pooled = np.zeros(max(npre, 1), dtype=np.float32)
    rc = _lib().rkvo_snapkv_group(_p(q_win), _p(k), _dt(k), L, d, G, w, int(pool_kernel),
                                  keep_eff, ctypes.c_float(scale), _p(A), _p(pooled), _p(kept))
    if rc != OK:
        raise OracleError(f"snapkv_group: status {rc}")
    return kept[:keep_eff], A[:npre], pooled[:npre]


def snapkv_chunked_group(q_wins, k_chunks, pool_kernel: int, keeps, scale: float):
    """SnapKV++ across the calls of a chunked prefill, for one KV head group
    ("RocketKV-adapted -- Two-Stage Compression", "Evidence": the stage-1
    budget is re-enforced across chunked-prefill calls).  Reading: call t
    appends chunk t (keys k_chunks[t] [C_t, d]) to the rows kept so far and
    applies snapkv_group to that concatenation with the chunk's last w
    queries q_wins[t] [G, w, d] and budget keeps[t].
    Returns one (kept, pooled, kept_positions) per call: kept indexes the
    concatenation, kept_positions are original prompt positions."""
    rows = np.asarray(k_chunks[0])[:0]
    pos = np.zeros(0, np.int64)
    off = 0
    out = []
    for q, kc, keep in zip(q_wins, k_chunks, keeps):
        kc = np.asarray(kc)
        cat = np.concatenate([rows, kc])
        cpos = np.concatenate([pos, off + np.arange(len(kc), dtype=np.int64)])
        off += len(kc)
        kept, _, pooled = snapkv_group(q, cat, pool_kernel, keep, scale)
        rows, pos = cat[kept], cpos[kept]
        out.append((kept, pooled, pos.copy()))
    return out


def mt_turn_view(q_win: np.ndarray, k_hist: np.ndarray, pool_kernel: int, keep: int,
                 scale: float):
    """RocketKV-MT's per-turn candidate view for one KV head group.

    "RocketKV: Accelerating Long-Context LLM Inference via Two-Stage KV Cache
    Compression" (atlas.scime.ai), "Approach" and "Limitations": RocketKV-MT
    retains the tokens stage 1 would evict for later turns, so it saves
    memory traffic but no KV storage; "RocketKV-adapted -- Two-Stage
    Compression", "Should you use this?": it skips permanent eviction so that
    earlier-turn tokens survive.  Reading (the pages give no per-turn rule):
    at the start of a turn, after the turn's rows are appended to the full
    history k_hist [L, d] (never shortened), SnapKV++ scores the whole
    history with the turn's last w queries q_win [G, w, d] and keeps `keep`
    rows; those rows, in ascending position, are the turn's view that HSA
    decodes over; nothing is deleted, so a row left out of one turn's view
    can be in the next one's.  Returns (kept, pooled) as snapkv_group."""
    kept, _, pooled = snapkv_group(q_win, k_hist, pool_kernel, keep, scale)
    return kept, pooled


def hsa_group(q: np.ndarray, k: np.ndarray, v: np.ndarray, smax: np.ndarray,
              smin: np.ndarray, n: int, P: int, k1: int, k2: int, scale: float):
    """HSA decode for one KV head group.  q [G, d]; k, v [>=n, d]; summaries
    [>=NP, d].  Returns (chan[k1], pages[k2] (-1 padded), S[NP] fp32, out[G, d] fp64)."""
    q, k, v, smax, smin = _c(q), _c(k), _c(v), _c(smax), _c(smin)
    assert q.dtype == k.dtype == v.dtype == smax.dtype == smin.dtype
    G, d = q.shape
    np_ = (n + P - 1) // P
    chan = np.zeros(k1, dtype=np.int32)
    pages = np.zeros(k2, dtype=np.int32)
    S = np.zeros(max(np_, 1), dtype=np.float32)
    out = np.zeros((G, d), dtype=np.float64)
    rc = _lib().rkvo_hsa_group(_p(q), _p(k), _p(v), _dt(k), _p(smax), _p(smin), int(n), d, G,
                               int(P), int(k1), int(k2), float(scale), _p(chan), _p(pages),
                               _p(S), _p(out))
    if rc != OK:
        raise OracleError(f"hsa_group: status {rc}")
    return chan, pages, S[:np_], out
