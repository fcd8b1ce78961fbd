"""DFlash block attention on MI355X (gfx950).

Thin Python layer over the C ABI of ``libdflash_attn.so`` (declared in
include/dflash_block_attn.h).  Functions carry the C names and only marshal
arguments; ``block_attn`` adds the allocation of ``out`` and the workspace
with torch (device memory and the current stream are the only things torch
provides here).

The operation: each request's block of 1 + num_speculative_tokens queries
attends to the request's context K/V plus the block's own K/V, non-causally
by default, with a per-request causal flag and an optional sliding window
(kenforever1 "DFlash + Gemma 4 31B-it" notes, "why non-causal attention is
needed"; vLLM PR #43445 report).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import _lib
from ._lib import (DFLASH_ERR_HIP, DFLASH_ERR_INVALID_ARGUMENT, DFLASH_ERR_UNSUPPORTED,  # noqa: F401
                   DFLASH_ERR_WORKSPACE_TOO_SMALL, DFLASH_KERNEL_AUTO, DFLASH_KERNEL_MFMA, DFLASH_KERNEL_REFERENCE,
                   DFLASH_MERGE_AUTO, DFLASH_MERGE_COMBINE_KERNEL, DFLASH_MERGE_IN_KERNEL, DFLASH_OK,
                   dflash_batch_desc, dflash_plan_info)


class DFlashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{dflash_status_string(status)} ({status}): {message}")
        self.status = status


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(status: int) -> None:
    if status != DFLASH_OK:
        raise DFlashError(status, dflash_last_error_message())


# ---- the C names -----------------------------------------------------------
def dflash_abi_version() -> int:
    return _lib.load().dflash_abi_version()


# bits of dflash_debug_checks_result (include/dflash_block_attn.h)
DFLASH_DEBUG_NEGATIVE_LENGTH = 1
DFLASH_DEBUG_BEYOND_PAGE_TABLE = 2
DFLASH_DEBUG_BAD_PAGE_ID = 4
DFLASH_DEBUG_TOTAL_Q_MISMATCH = 8
DFLASH_DEBUG_ABOVE_HINT = 16
DFLASH_DEBUG_BAD_SPAN_OFFSETS = 32


def dflash_set_debug_checks(on: bool) -> bool:
    """Switch the device-side value checks for later calls; returns the previous setting."""
    return bool(_lib.load().dflash_set_debug_checks(1 if on else 0))


def dflash_debug_checks_result():
    """(bits, first_request) of the checked calls since the last query; synchronises and clears."""
    bits = ctypes.c_uint32(0)
    req = ctypes.c_int32(-1)
    _check(_lib.load().dflash_debug_checks_result(ctypes.byref(bits), ctypes.byref(req)))
    return bits.value, req.value


def dflash_block_conv(x, base, delta, block_lens, num_reqs: int, total_q: int, channels: int, groups: int,
                       taps: int, out, stream: Optional[int]) -> int:
    """Raw call: DFlash2 in-block grouped dynamic depthwise convolution; status code out."""
    return _lib.load().dflash_block_conv(_ptr(x), _ptr(base), _ptr(delta), _ptr(block_lens), num_reqs, total_q,
                                          channels, groups, taps, _ptr(out), stream)


def block_conv(x, base, delta, block_lens, *, groups: int, out=None):
    """DFlash2 block convolution on torch device tensors (bf16); returns ``out``.

    x: [total_q, C]; base: [taps, C]; delta: [total_q, taps, groups];
    block_lens: int32 [B].  Runs on torch's current stream.
    """
    import torch

    total_q, C = x.shape
    taps = base.shape[0]
    if out is None:
        out = torch.empty_like(x)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(dflash_block_conv(x, base, delta, block_lens, block_lens.shape[0], total_q, C, groups, taps, out, stream))
    return out


def dflash_stream_read(buf, nbytes: int, sink, stream) -> int:
    """Measurement helper: one streaming read of nbytes at buf (see the C header)."""
    return _lib.load().dflash_stream_read(_ptr(buf), nbytes, _ptr(sink), stream)


def dflash_timeline_set_buffer(buf, nbytes: int) -> int:
    """Timeline build only: per-workgroup stamps of later attention launches go to buf
    (see the C header).  Raises if the loaded library is not the timeline build."""
    lib = _lib.load()
    if not hasattr(lib, "dflash_timeline_set_buffer"):
        raise RuntimeError(f"{_lib.LIB_PATH} is not the timeline build (python -m non_causal_block_amd.build --timeline)")
    return lib.dflash_timeline_set_buffer(_ptr(buf), nbytes)


def dflash_status_string(status: int) -> str:
    return _lib.load().dflash_status_string(status).decode()


def dflash_last_error_message() -> str:
    return _lib.load().dflash_last_error_message().decode()


def dflash_block_attn_supports(n_heads: int, n_kv_heads: int, head_dim: int) -> bool:
    return bool(_lib.load().dflash_block_attn_supports(n_heads, n_kv_heads, head_dim))


def dflash_block_attn_workspace_size(desc: dflash_batch_desc, n_heads: int, n_kv_heads: int, head_dim: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.load().dflash_block_attn_workspace_size(ctypes.byref(desc), n_heads, n_kv_heads, head_dim,
                                                        ctypes.byref(out)))
    return int(out.value)


def dflash_block_attn_plan(desc: dflash_batch_desc, n_heads: int, n_kv_heads: int, head_dim: int) -> dflash_plan_info:
    info = dflash_plan_info()
    _check(_lib.load().dflash_block_attn_plan(ctypes.byref(desc), n_heads, n_kv_heads, head_dim, ctypes.byref(info)))
    return info


def dflash_block_attn(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads: int, n_kv_heads: int,
                      head_dim: int, causal, window: int, scale: float, out, stream: Optional[int],
                      desc: dflash_batch_desc) -> int:
    """Raw call: tensors (or raw device addresses) in, status code out."""
    return _lib.load().dflash_block_attn(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(ctx_lens),
                                         _ptr(block_lens), n_heads, n_kv_heads, head_dim, _ptr(causal), window,
                                         scale, _ptr(out), stream, ctypes.byref(desc))


def dflash_block_attn_noalloc(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads: int, n_kv_heads: int,
                              head_dim: int, causal, window: int, scale: float, out, stream: Optional[int],
                              desc: dflash_batch_desc) -> int:
    """Raw call on the library's static scratch (no workspace, nothing allocated); status code out."""
    return _lib.load().dflash_block_attn_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                                                 _ptr(ctx_lens), _ptr(block_lens), n_heads, n_kv_heads, head_dim,
                                                 _ptr(causal), window, scale, _ptr(out), stream, ctypes.byref(desc))


def dflash_noalloc_scratch_bytes() -> int:
    return int(_lib.load().dflash_noalloc_scratch_bytes())


def dflash_block_attn_spans(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads: int, n_kv_heads: int,
                            head_dim: int, causal, span_offsets, spans, num_spans: int, window: int, scale: float,
                            out, stream: Optional[int], desc: dflash_batch_desc) -> int:
    """Raw call with bidirectional spans in causal requests; status code out."""
    return _lib.load().dflash_block_attn_spans(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                                               _ptr(ctx_lens), _ptr(block_lens), n_heads, n_kv_heads, head_dim,
                                               _ptr(causal), _ptr(span_offsets), _ptr(spans), num_spans, window,
                                               scale, _ptr(out), stream, ctypes.byref(desc))


def dflash_block_kv_append(k_new, v_new, k_pages, v_pages, page_table, ctx_lens, block_lens, n_kv_heads: int,
                           head_dim: int, stream: Optional[int], desc: dflash_batch_desc) -> int:
    """Raw call: write the block K/V rows into their pages; status code out."""
    return _lib.load().dflash_block_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                              _ptr(page_table), _ptr(ctx_lens), _ptr(block_lens), n_kv_heads,
                                              head_dim, stream, ctypes.byref(desc))


def dflash_block_attn_append(q, k_new, v_new, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads: int,
                             n_kv_heads: int, head_dim: int, causal, window: int, scale: float, out,
                             stream: Optional[int], desc: dflash_batch_desc) -> int:
    """Raw call: append the block K/V, then attend (one stream); status code out."""
    return _lib.load().dflash_block_attn_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                                _ptr(page_table), _ptr(ctx_lens), _ptr(block_lens), n_heads,
                                                n_kv_heads, head_dim, _ptr(causal), window, scale, _ptr(out), stream,
                                                ctypes.byref(desc))


# ---- convenience -------------------------------------------------------------
def make_desc(*, num_reqs: int, total_q: int, max_block_len: int, total_kv_len: int, page_size: int,
              max_pages_per_req: int, num_pages: int, kernel: int = DFLASH_KERNEL_AUTO, num_workgroups: int = 0,
              num_cus: int = 0, merge_mode: int = DFLASH_MERGE_AUTO) -> dflash_batch_desc:
    d = dflash_batch_desc()
    d.num_reqs = num_reqs
    d.total_q = total_q
    d.max_block_len = max_block_len
    d.total_kv_len = total_kv_len
    d.page_size = page_size
    d.max_pages_per_req = max_pages_per_req
    d.num_pages = num_pages
    d.kernel = kernel
    d.num_workgroups = num_workgroups
    d.num_cus = num_cus
    d.merge_mode = merge_mode
    return d


def block_attn(q, k_pages, v_pages, page_table, ctx_lens, block_lens, *, causal=None, window: int = 0,
               scale: Optional[float] = None, out=None, max_block_len: int = 0, total_kv_len: int = 0,
               kernel: int = DFLASH_KERNEL_AUTO, num_workgroups: int = 0, workspace=None, span_offsets=None,
               spans=None, merge_mode: int = DFLASH_MERGE_AUTO):
    """Block attention on torch device tensors; returns ``out`` (bf16 [total_q, Hq, D]).

    q: bf16 [total_q, Hq, D]; k_pages/v_pages: bf16 [num_pages, page_size, Hkv, D];
    page_table: int32 [B, max_pages_per_req]; ctx_lens/block_lens: int32 [B];
    causal: uint8 [B] or None.  ``max_block_len``/``total_kv_len`` are host hints
    (0 = unknown).  ``span_offsets`` (int32 [B+1]) with ``spans`` (int32 [S, 2])
    add bidirectional spans to causal requests (dflash_block_attn_spans).  Runs on
    torch's current stream.  A caller-given ``workspace`` (uint8 device tensor) must
    have been zero-filled once before its first use; one allocated here is.
    """
    import torch

    total_q, Hq, D = q.shape
    num_pages, page_size, Hkv, D2 = k_pages.shape
    if D2 != D or v_pages.shape != k_pages.shape:
        raise ValueError("q / k_pages / v_pages head_dim or shape mismatch")
    B = ctx_lens.shape[0]
    desc = make_desc(num_reqs=B, total_q=total_q, max_block_len=max_block_len, total_kv_len=total_kv_len,
                     page_size=page_size, max_pages_per_req=page_table.shape[1], num_pages=num_pages,
                     kernel=kernel, num_workgroups=num_workgroups, merge_mode=merge_mode)
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device=q.device)
    need = dflash_block_attn_workspace_size(desc, Hq, Hkv, D)
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if span_offsets is not None:
        num_spans = 0 if spans is None else spans.shape[0]
        _check(dflash_block_attn_spans(q, k_pages, v_pages, page_table, ctx_lens, block_lens, Hq, Hkv, D, causal,
                                       span_offsets, spans if num_spans else None, num_spans, window, scale, out,
                                       stream, desc))
        return out
    _check(dflash_block_attn(q, k_pages, v_pages, page_table, ctx_lens, block_lens, Hq, Hkv, D, causal, window,
                             scale, out, stream, desc))
    return out
