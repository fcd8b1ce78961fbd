"""dflash_block_attn_noalloc: the call on the library's static scratch (needs an MI355X).

Through the C ABI, two calls in a row -- the head_dim-512 global layer (B = 4 x 9,
L ~ U[8192, 32768]: the largest workload the scratch is sized for), then a smaller
one (the head_dim-128 draft step) -- each compared element by element with
dflash_block_attn on a caller-owned workspace with the same merge path (bitwise:
same kernels, same plan) and with the fp64 oracle (the parity bounds).  A call
needing more scratch than the library holds is refused before anything runs.
"""
import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import oracle
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _desc(wl):
    return nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                        total_kv_len=wl.total_kv, page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                        num_pages=wl.num_pages, merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL)


def _both(wl):
    t = H.upload(wl)
    stream = torch.cuda.current_stream().cuda_stream
    d = _desc(wl)
    out_na = torch.full((wl.total_q, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=H.dev())
    st = nb.dflash_block_attn_noalloc(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                      t["causal"], wl.window, wl.scale, out_na, stream, d)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    d2 = _desc(wl)
    need = nb.dflash_block_attn_workspace_size(d2, wl.Hq, wl.Hkv, wl.D)
    assert 0 < need <= nb.dflash_noalloc_scratch_bytes()
    ws = torch.zeros(need, dtype=torch.uint8, device=H.dev())
    d2.workspace, d2.workspace_bytes = ws.data_ptr(), ws.numel()
    out_ws = torch.empty_like(out_na)
    st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D, t["causal"],
                              wl.window, wl.scale, out_ws, stream, d2)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    return out_na, out_ws


def test_noalloc_two_calls_in_a_row_match_the_workspace_call():
    big = workloads.make("c3_global_d512")
    small = workloads.make("c1_tiny_d128")
    for wl in (big, small):
        out_na, out_ws = _both(wl)
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), wl.name
        rows = None
        if wl.total_q * wl.Hq > 600:
            rows = np.sort(np.random.default_rng(5).choice(wl.total_q * wl.Hq, size=600, replace=False))
        ref = oracle.run_workload(wl, rows=rows)
        got = H.to_f64(out_na).reshape(-1, wl.D)
        H.assert_parity(got if rows is None else got[rows], ref.reshape(-1, wl.D), f"noalloc {wl.name}")


def test_noalloc_refuses_more_than_its_scratch():
    wl = workloads.make("c1_tiny_d128")
    t = H.upload(wl)
    d = _desc(wl)
    # a forced grid whose partial slots exceed the static scratch
    d.num_workgroups = 1 << 20
    need = nb.dflash_block_attn_workspace_size(d, wl.Hq, wl.Hkv, wl.D)
    assert need > nb.dflash_noalloc_scratch_bytes()
    out = torch.full((wl.total_q, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=H.dev())
    st = nb.dflash_block_attn_noalloc(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                      t["causal"], wl.window, wl.scale, out, torch.cuda.current_stream().cuda_stream, d)
    assert st == nb.DFLASH_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in nb.dflash_last_error_message()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing ran
