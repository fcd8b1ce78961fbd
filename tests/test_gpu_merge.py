"""The split-KV merge inside the MFMA attention kernel (needs an MI355X).

The pieces of a split unit are merged by the workgroups that computed them,
coordinated through counters at the start of the caller's workspace: every call
must leave those counters at zero, agree with the separate combine kernel, and
stay correct when the grid is larger than what the chip runs at once (waiting
workgroups then give up after a bounded time and the unit's last piece merges
the rest).  Every call goes through the C ABI.
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


def _call(wl, t, ws, *, num_workgroups=0, separate=False, out=None):
    """separate: merge with the combine kernel; else inside the attention kernel."""
    d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                     total_kv_len=wl.total_kv, page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                     num_pages=wl.num_pages, num_workgroups=num_workgroups,
                     merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL if separate else nb.DFLASH_MERGE_IN_KERNEL)
    plan = nb.dflash_block_attn_plan(d, wl.Hq, wl.Hkv, wl.D)
    assert ws.numel() >= plan.workspace_bytes
    d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
    if out is None:
        out = torch.empty((wl.total_q, wl.Hq, wl.D), dtype=torch.bfloat16, device=H.dev())
    st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D, t["causal"],
                              wl.window, wl.scale, out, torch.cuda.current_stream().cuda_stream, d)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    return out, plan


# the merge counters' region at the start of the workspace, the same for every grid:
# a finish count, then an arrival word per workgroup and two give-up flags per workgroup
# for up to 16384 workgroups (merge.h)
CTR_BYTES = 4 * (64 + 3 * 16384)


def _counters(ws):
    return ws[:CTR_BYTES].view(torch.int32).cpu().numpy()


def _within_one_ulp(a, b, what):
    """bf16 results of the same fp32 sum taken in two orders: they differ by at most one
    unit in the last place (an ulp of a bf16 value x is at most 2^-7 |x|) plus what
    reordering an fp32 sum of at most a few hundred terms of size <= 1 can move a
    cancelling result by (1e-6 absolute)."""
    excess = np.abs(a - b) - (2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)
    worst = int(np.argmax(excess))
    assert excess.flat[worst] <= 0, f"{what}: {a.flat[worst]!r} vs {b.flat[worst]!r} at flat index {worst}"


CASES = [
    # (name, kwargs for workloads.make or build args, grids)
    ("c2", dict(name="c2_paged_d256", ctx_cap=1500), (0, 2, 7, 64, 300)),
    ("c4", dict(name="c4_causal_window_d256", B=4), (0, 3, 50)),
    ("c1", dict(name="c1_tiny_d128"), (0, 2, 5, 40)),
    ("c3", dict(name="c3_global_d512", ctx_cap=3000), (0, 5, 64, 256)),
    ("c5", dict(name="c5_mixed_d512", ctx_cap=900, B=10), (0, 9, 100)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_in_kernel_merge_matches_combine_kernel(case):
    """Same partials, same merge arithmetic: at head_dim <= 256 the combine kernel
    merges each row in the same order as the in-kernel merge, so the outputs are
    bitwise equal; at head_dim 512 the combine may deal a row's pieces over four
    waves (a different summation order), so they agree to the bf16 rounding of the
    output (one ulp)."""
    label, kw, grids = CASES[case]
    kw = dict(kw)
    wl = workloads.make(kw.pop("name"), **kw)
    ref = oracle.run_workload(wl)
    t = H.upload(wl)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=H.dev())
    for nwg in grids:
        fused, plan = _call(wl, t, ws, num_workgroups=nwg)
        sep, plan2 = _call(wl, t, ws, num_workgroups=nwg, separate=True)
        torch.cuda.synchronize()
        assert plan2.merge_in_kernel == 0
        assert plan.merge_in_kernel == (1 if plan.num_workgroups > 1 else 0)
        H.assert_parity(H.to_f64(fused), ref, f"{label} fused wg={nwg}")
        H.assert_parity(H.to_f64(sep), ref, f"{label} separate wg={nwg}")
        if wl.D <= 256:
            assert torch.equal(fused.view(torch.int16), sep.view(torch.int16)), (label, nwg)
        else:
            _within_one_ulp(H.to_f64(fused), H.to_f64(sep), f"{label} wg={nwg}")
        assert not _counters(ws).any(), f"{label} wg={nwg}: counters not cleared"


def test_workspace_reused_across_shapes_back_to_back():
    """One zero-filled workspace serves calls of different shapes and grids, queued
    back to back with no synchronisation between them: each call finds the counters
    the previous one cleared."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=H.dev())
    jobs = []
    for name, kw, nwg in (("c2_paged_d256", dict(ctx_cap=1200), 0), ("c3_global_d512", dict(ctx_cap=2500), 0),
                          ("c2_paged_d256", dict(ctx_cap=1200), 37), ("c1_tiny_d128", {}, 0),
                          ("c3_global_d512", dict(ctx_cap=2500), 200), ("c4_causal_window_d256", dict(B=3), 0)):
        wl = workloads.make(name, **kw)
        jobs.append((wl, H.upload(wl), nwg))
    outs = [_call(wl, t, ws, num_workgroups=nwg) for wl, t, nwg in jobs]
    torch.cuda.synchronize()
    for (wl, _, nwg), (out, plan) in zip(jobs, outs):
        H.assert_parity(H.to_f64(out), oracle.run_workload(wl), f"{wl.name} wg={nwg}")
    assert not _counters(ws).any()


def test_repeated_calls_are_bitwise_equal():
    """The merge is deterministic: which wave claims which row changes from call to
    call, the arithmetic of a row does not."""
    wl = workloads.make("c3_global_d512", ctx_cap=6000)
    t = H.upload(wl)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=H.dev())
    first, plan = _call(wl, t, ws)
    outs = [_call(wl, t, ws)[0] for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))
    assert not _counters(ws).any()


@pytest.mark.parametrize("D", [128, 512])
def test_grid_larger_than_the_chip(D):
    """More workgroups than run at once: pieces of a unit may sit in workgroups that
    start only after others finished.  Waiting workgroups leave after the bounded
    wait, and the unit's last piece merges what is left; the result is unchanged."""
    wl = workloads.build(2, 8, 2, D, [20000, 700], [9, 5], [0, 1], seed=41)
    ref = oracle.run_workload(wl)
    t = H.upload(wl)
    props = torch.cuda.get_device_properties(0)
    nwg = 6 * props.multi_processor_count
    d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=9, total_kv_len=wl.total_kv,
                     page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req, num_pages=wl.num_pages,
                     num_workgroups=nwg, merge_mode=nb.DFLASH_MERGE_IN_KERNEL)
    ws = torch.zeros(nb.dflash_block_attn_plan(d, wl.Hq, wl.Hkv, wl.D).workspace_bytes, dtype=torch.uint8,
                     device=H.dev())
    out, plan = _call(wl, t, ws, num_workgroups=nwg)
    sep, _ = _call(wl, t, ws, num_workgroups=nwg, separate=True)
    torch.cuda.synchronize()
    assert plan.num_workgroups == nwg and plan.merge_in_kernel == 1
    H.assert_parity(H.to_f64(out), ref, f"D={D} grid {nwg}")
    _within_one_ulp(H.to_f64(out), H.to_f64(sep), f"D={D} grid {nwg}")
    assert not _counters(ws).any()


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("nwg", [24, 200])
def test_combine_directory_rows_of_no_request(nwg, D):
    """The combine kernel finds each output row's pieces in a directory that the attention
    kernel writes on every call (one entry per row of the total_q hint).  Rows past the
    blocks' sum belong to no request: a call must leave them alone even when an earlier
    call on the same workspace had real rows there, and a call whose blocks are all empty
    must leave every row alone.  24 workgroups split each unit a few ways (rows per wave
    in the combine), 200 many (at head_dim 512, a workgroup per row)."""
    big = workloads.build(3, 8, 2, D, [3000, 900, 2000], [9, 9, 9], [0, 1, 0], seed=51)
    small = workloads.build(2, 8, 2, D, [2500, 1200], [9, 4], [1, 0], seed=52)
    empty = workloads.build(2, 8, 2, D, [300, 100], [0, 0], [0, 0], seed=53)
    extra = 5

    def call(wl, t, ws, total_q, out):
        d = nb.make_desc(num_reqs=wl.B, total_q=total_q, max_block_len=9, total_kv_len=wl.total_kv,
                         page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req, num_pages=wl.num_pages,
                         num_workgroups=nwg, merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL)
        plan = nb.dflash_block_attn_plan(d, wl.Hq, wl.Hkv, wl.D)
        assert plan.combine_workgroups > 0 and ws.numel() >= plan.workspace_bytes
        d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
        st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                  t["causal"], wl.window, wl.scale, out, torch.cuda.current_stream().cuda_stream, d)
        assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
        torch.cuda.synchronize()
        return plan

    tb, ts, te = H.upload(big), H.upload(small), H.upload(empty)
    te["q"] = ts["q"]  # no row of it is read: every block is empty
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=H.dev())
    out_b = torch.empty((big.total_q, big.Hq, big.D), dtype=torch.bfloat16, device=H.dev())
    call(big, tb, ws, big.total_q, out_b)
    H.assert_parity(H.to_f64(out_b), oracle.run_workload(big), f"big, grid {nwg}")

    nq = small.total_q + extra
    out_s = torch.full((nq, small.Hq, small.D), 7.0, dtype=torch.bfloat16, device=H.dev())
    call(small, ts, ws, nq, out_s)
    H.assert_parity(H.to_f64(out_s[:small.total_q]), oracle.run_workload(small), f"small, grid {nwg}")
    assert torch.all(out_s[small.total_q:] == 7.0), "rows of no request were written"

    out_e = torch.full((4, empty.Hq, empty.D), 7.0, dtype=torch.bfloat16, device=H.dev())
    call(empty, te, ws, 4, out_e)
    assert torch.all(out_e == 7.0), "a call with empty blocks wrote output rows"


def test_combine_directory_more_than_64_requests():
    """As above with 130 requests, where each run is located over several 64-request chunks
    of the length arrays and the run holding the last tile sums the blocks in a pass of
    its own: an earlier call with more query tokens leaves real entries in the rows that
    the later call's larger total_q hint covers but no request owns."""
    rng = np.random.default_rng(91)
    B = 130
    L = rng.integers(0, 400, size=B)
    c = rng.integers(0, 2, size=B)
    n_big = rng.integers(1, 10, size=B)
    n_small = np.minimum(n_big, rng.integers(0, 6, size=B))
    big = workloads.build(B, 8, 2, 128, L, n_big, c, seed=92)
    small = workloads.build(B, 8, 2, 128, L, n_small, c, seed=93)
    assert small.total_q < big.total_q
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device=H.dev())
    for nwg in (24, 200):
        for wl, total_q in ((big, big.total_q), (small, big.total_q)):
            t = H.upload(wl)
            d = nb.make_desc(num_reqs=wl.B, total_q=total_q, max_block_len=int(wl.block_lens.max()),
                             total_kv_len=wl.total_kv, page_size=wl.page_size,
                             max_pages_per_req=wl.max_pages_per_req, num_pages=wl.num_pages,
                             num_workgroups=nwg, merge_mode=nb.DFLASH_MERGE_COMBINE_KERNEL)
            plan = nb.dflash_block_attn_plan(d, wl.Hq, wl.Hkv, wl.D)
            assert plan.combine_workgroups > 0 and ws.numel() >= plan.workspace_bytes
            d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
            out = torch.full((total_q, wl.Hq, wl.D), 7.0, dtype=torch.bfloat16, device=H.dev())
            st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                      t["causal"], wl.window, wl.scale, out, torch.cuda.current_stream().cuda_stream,
                                      d)
            assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
            torch.cuda.synchronize()
            H.assert_parity(H.to_f64(out[:wl.total_q]), oracle.run_workload(wl), f"B=130 grid {nwg}")
            assert torch.all(out[wl.total_q:] == 7.0), "rows of no request were written"
