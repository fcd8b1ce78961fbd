"""Debug checks of device-side values (dflash_set_debug_checks): a valid call
reports nothing and matches the unchecked call bitwise; a call whose page table,
block lengths or span offsets break the contract is reported and does nothing.

Every bad value below stays inside the memory the test allocated (a page id past
desc->num_pages but inside the page arrays, a total_q hint off by one), so even a
kernel that ignored the checks would touch only valid memory.
"""
import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _checks_on():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prev = nb.dflash_set_debug_checks(True)
    nb.dflash_debug_checks_result()  # start from a clear state
    yield
    nb.dflash_debug_checks_result()
    nb.dflash_set_debug_checks(prev)


def _call(wl, t, *, num_pages=None, total_q=None, out=None, span_offsets=None, spans=None):
    d = H.dev()
    desc = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q if total_q is None else total_q,
                        max_block_len=int(wl.block_lens.max()), total_kv_len=wl.total_kv,
                        page_size=wl.page_size, max_pages_per_req=wl.page_table.shape[1],
                        num_pages=wl.num_pages if num_pages is None else num_pages)
    need = nb.dflash_block_attn_workspace_size(desc, wl.Hq, wl.Hkv, wl.D)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=d)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    out = torch.full((wl.total_q, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=d) if out is None else out
    stream = torch.cuda.current_stream().cuda_stream
    if span_offsets is None:
        st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                  t["causal"], wl.window, wl.scale, out, stream, desc)
    else:
        st = nb.dflash_block_attn_spans(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                        t["causal"], span_offsets, spans, 0 if spans is None else spans.shape[0],
                                        wl.window, wl.scale, out, stream, desc)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    return out


def _workload():
    # identity page ids: the 4 extra pages are the last ids, so "num_pages - 2" excludes only them
    return workloads.build(3, 16, 4, 256, [300, 40, 1000], [9, 16, 9], [0, 1, 0], seed=41, extra_pages=4,
                           permute_pages=False)


def test_valid_call_reports_nothing_and_matches_unchecked():
    wl = _workload()
    t = H.upload(wl)
    got = _call(wl, t).cpu()
    assert nb.dflash_debug_checks_result() == (0, -1)
    nb.dflash_set_debug_checks(False)
    ref = _call(wl, t).cpu()
    nb.dflash_set_debug_checks(True)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_page_id_past_num_pages_is_reported_and_nothing_runs():
    wl = _workload()
    t = H.upload(wl)
    # request 2's 10th page points at the last page of the arrays, which the desc
    # declares out of range (num_pages is passed two short)
    pt = wl.page_table.copy()
    pt[2, 10] = wl.num_pages - 1
    t["pt"] = torch.from_numpy(pt).to(H.dev())
    out = _call(wl, t, num_pages=wl.num_pages - 2)
    bits, req = nb.dflash_debug_checks_result()
    assert bits & nb.DFLASH_DEBUG_BAD_PAGE_ID and req == 2
    assert bool((out.float() == 7.0).all())  # untouched


def test_total_q_mismatch_is_reported():
    wl = _workload()
    t = H.upload(wl)
    out = torch.full((wl.total_q + 1, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=H.dev())
    out = _call(wl, t, total_q=wl.total_q + 1, out=out)
    bits, _ = nb.dflash_debug_checks_result()
    assert bits & nb.DFLASH_DEBUG_TOTAL_Q_MISMATCH
    assert bool((out.float() == 7.0).all())


def test_bad_span_offsets_are_reported():
    wl = _workload()
    t = H.upload(wl)
    spans = torch.tensor([[300, 305], [40, 50]], dtype=torch.int32, device=H.dev())
    offs = torch.tensor([0, 1, 3, 2], dtype=torch.int32, device=H.dev())  # decreasing, past num_spans
    out = _call(wl, t, span_offsets=offs, spans=spans)
    bits, req = nb.dflash_debug_checks_result()
    assert bits & nb.DFLASH_DEBUG_BAD_SPAN_OFFSETS and req == 1
    assert bool((out.float() == 7.0).all())


def test_append_with_bad_page_id_writes_nothing():
    wl = _workload()
    k_new, v_new, kp, vp = workloads.split_block_kv(wl)
    d = H.dev()
    kpt, vpt = H.bf16_tensor(kp, d), H.bf16_tensor(vp, d)
    before = kpt.clone()
    pt = wl.page_table.copy()
    blk_page = (int(wl.ctx_lens[0]) + 3) // wl.page_size  # a page holding block 0's positions
    pt[0, blk_page] = wl.num_pages - 1
    desc = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                        total_kv_len=wl.total_kv, page_size=wl.page_size,
                        max_pages_per_req=wl.page_table.shape[1], num_pages=wl.num_pages - 2)
    st = nb.dflash_block_kv_append(H.bf16_tensor(k_new, d), H.bf16_tensor(v_new, d), kpt, vpt,
                                   torch.from_numpy(pt).to(d), torch.from_numpy(wl.ctx_lens).to(d),
                                   torch.from_numpy(wl.block_lens).to(d), wl.Hkv, wl.D,
                                   torch.cuda.current_stream().cuda_stream, desc)
    assert st == nb.DFLASH_OK
    bits, req = nb.dflash_debug_checks_result()
    assert bits & nb.DFLASH_DEBUG_BAD_PAGE_ID and req == 0
    assert torch.equal(kpt.view(torch.int16), before.view(torch.int16))
