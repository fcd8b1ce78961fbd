"""fp64 CPU oracle for DFlash block attention.

TEST INFRASTRUCTURE ONLY: nothing on the product path may import, call, link
or execute anything in this package.  Its users are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

``block_attn_f64`` wraps the plain C implementation in ``oracle_f64.c`` (see
its header for the definition it follows); ``brute.py`` holds an independent
pure-Python formulation for tiny inputs.  Neither shares anything with the
HIP path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_f64.c")
_LIB = os.path.join(_HERE, "liboracle_f64.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle_f64.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                               "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def is_built() -> bool:
    """The compiled library exists and is newer than its source."""
    return os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)


def bind(path: str):
    """Load a compiled oracle library and declare its signature."""
    lib = ctypes.CDLL(path)
    f = lib.oracle_block_attn_f64
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_double, P, ctypes.c_int64, P, ctypes.c_int32]
    f.restype = ctypes.c_int
    if hasattr(lib, "oracle_block_attn_spans_f64"):
        g = lib.oracle_block_attn_spans_f64
        g.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_double, P, ctypes.c_int64, P, ctypes.c_int32]
        g.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = bind(_LIB)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def block_attn_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx_lens, block_lens, causal,
                   Hq: int, Hkv: int, D: int, window: int, scale: float,
                   rows: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                   lib=None, spans=None) -> np.ndarray:
    """Exact attention in fp64.

    q: uint16 bf16 bits [total_q, Hq, D]; k, v: uint16 [total_kv, Hkv, D] (logical,
    request-major); ctx_lens/block_lens int [B]; causal uint8 [B] or None (all
    non-causal).  Returns float64 [total_q, Hq, D], or [len(rows), D] when ``rows``
    lists packed (token * Hq + head) indices.  ``lib`` selects another build of
    the same source (tests use it to check that the pins catch planted mistakes).
    ``spans``: optional bidirectional spans, a per-request list of (start, end)
    key-position pairs (sorted, disjoint), see oracle_f64.c.
    """
    lib = _load() if lib is None else lib
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    blk = np.ascontiguousarray(block_lens, dtype=np.int32)
    B = int(ctx.shape[0])
    cz = None if causal is None else np.ascontiguousarray(causal, dtype=np.uint8)
    total_q = int(blk.sum())
    total_kv = int(ctx.astype(np.int64).sum() + blk.astype(np.int64).sum())
    assert q.shape == (total_q, Hq, D), (q.shape, total_q, Hq, D)
    assert k.shape == (total_kv, Hkv, D) and v.shape == k.shape, (k.shape, total_kv)
    if rows is None:
        out = np.empty((total_q, Hq, D), dtype=np.float64)
        rr, nr = None, 0
    else:
        rr = np.ascontiguousarray(rows, dtype=np.int64)
        nr = int(rr.shape[0])
        out = np.empty((nr, D), dtype=np.float64)
    th = default_threads() if threads is None else int(threads)
    if spans is None:
        rc = lib.oracle_block_attn_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(ctx), _ptr(blk), _ptr(cz), B, Hq, Hkv, D,
                                       int(window), float(scale), _ptr(rr), nr, _ptr(out), th)
    else:
        offs, flat = spans_csr(spans, B)
        rc = lib.oracle_block_attn_spans_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(ctx), _ptr(blk), _ptr(cz), _ptr(offs),
                                             _ptr(flat), B, Hq, Hkv, D, int(window), float(scale), _ptr(rr), nr,
                                             _ptr(out), th)
    if rc != 0:
        raise RuntimeError(f"oracle_block_attn_f64 failed with code {rc}")
    return out


def spans_csr(spans, B: int):
    """Per-request span lists -> (offsets int32 [B+1], pairs int32 [num_spans, 2])."""
    offs = np.zeros(B + 1, dtype=np.int32)
    flat = []
    for r in range(B):
        lst = list(spans[r]) if r < len(spans) else []
        offs[r + 1] = offs[r] + len(lst)
        flat.extend(lst)
    pairs = np.asarray(flat, dtype=np.int32).reshape(-1, 2) if flat else np.zeros((1, 2), dtype=np.int32)
    return offs, np.ascontiguousarray(pairs)


def run_workload(wl, rows: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                 spans=None) -> np.ndarray:
    """Oracle output for a ``workloads.Workload`` (uses its logical K/V)."""
    return block_attn_f64(wl.q, wl.k, wl.v, wl.ctx_lens, wl.block_lens, wl.causal, wl.Hq, wl.Hkv, wl.D,
                          wl.window, wl.scale, rows=rows, threads=threads, spans=spans)
