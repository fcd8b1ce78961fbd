"""Helpers for the GPU tests: upload a seeded workload, call the C ABI, compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import non_causal_block_amd as nb
import workloads

# parity tolerances on bf16 outputs vs the fp64 oracle (fp32 accumulation)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# relative RMS error: the absolute bounds alone would pass an all-zero output at long
# contexts (output std ~ sqrt(e/T)); bf16 rounding alone gives ~2^-9
REL_RMS = 1e-2


def dev():
    return torch.device("cuda", 0)


def bf16_tensor(bits: np.ndarray, device=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device or dev())


def upload(wl: workloads.Workload) -> dict:
    d = dev()
    return dict(
        q=bf16_tensor(wl.q, d), k=bf16_tensor(wl.k_pages, d), v=bf16_tensor(wl.v_pages, d),
        pt=torch.from_numpy(wl.page_table).to(d), ctx=torch.from_numpy(wl.ctx_lens).to(d),
        blk=torch.from_numpy(wl.block_lens).to(d), causal=torch.from_numpy(wl.causal).to(d),
    )


def run(wl: workloads.Workload, t: dict = None, *, kernel=nb.DFLASH_KERNEL_AUTO, num_workgroups=0,
        hints=True, causal_none=False, out=None, spans=None, merge_mode=nb.DFLASH_MERGE_AUTO) -> torch.Tensor:
    """``spans``: per-request (start, end) lists -> dflash_block_attn_spans."""
    t = t or upload(wl)
    so = sp = None
    if spans is not None:
        offs = np.zeros(wl.B + 1, dtype=np.int32)
        offs[1:] = np.cumsum([len(x) for x in spans])
        flat = np.asarray([p for x in spans for p in x], dtype=np.int32).reshape(-1, 2)
        so = torch.from_numpy(offs).to(dev())
        sp = torch.from_numpy(np.ascontiguousarray(flat)).to(dev()) if flat.shape[0] else None
    o = nb.block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"],
                      causal=None if causal_none else t["causal"], window=wl.window, scale=wl.scale, out=out,
                      max_block_len=int(wl.block_lens.max()) if (hints and wl.B) else 0,
                      total_kv_len=wl.total_kv if hints else 0, kernel=kernel, num_workgroups=num_workgroups,
                      span_offsets=so, spans=sp, merge_mode=merge_mode)
    torch.cuda.synchronize()
    return o


def to_f64(o: torch.Tensor) -> np.ndarray:
    return o.float().cpu().numpy().astype(np.float64)


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    rms_ref = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    return dict(max_abs=float(err.max()) if err.size else 0.0, mean_abs=float(err.mean()) if err.size else 0.0,
                rel_rms=(math.sqrt(float(np.mean(err * err))) / rms_ref) if rms_ref > 0 else 0.0,
                finite=bool(np.isfinite(got).all()))


# Full-size parity results of this session (workload, kernel, metrics, oracle wall time),
# printed as a table at the end of the run (conftest.py) and written as JSON to the file
# named by DFLASH_PARITY_REPORT when that is set.
PARITY_REPORT: list = []


def record(workload: str, kernel: str, m: dict, oracle_s: float, rows: int) -> None:
    PARITY_REPORT.append(dict(workload=workload, kernel=kernel, rows=rows, oracle_s=oracle_s, **m))


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    m = metrics(got, ref)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_abs"] <= MAX_ABS, f"{what}: {m}"
    assert m["mean_abs"] <= MEAN_ABS, f"{what}: {m}"
    assert m["rel_rms"] <= REL_RMS, f"{what}: {m}"
    return m
