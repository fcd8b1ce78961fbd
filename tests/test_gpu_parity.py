"""HIP path vs the fp64 oracle on the same seeded inputs (needs an MI355X).

Every call goes through the C ABI (non_causal_block_amd -> libdflash_attn.so).
Tolerances: max|err| <= 2e-2 and mean|err| <= 2e-3 on bf16 outputs, plus a
relative RMS error <= 1e-2 (tests/gpu_helpers.py).
"""
import time

import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import oracle
import workloads
from tests import error_model
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KERNELS = [("mfma", nb.DFLASH_KERNEL_MFMA), ("ref", nb.DFLASH_KERNEL_REFERENCE)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the oracle library was compiled at session start, before the GPU was touched


KNAMES = {nb.DFLASH_KERNEL_AUTO: "auto", nb.DFLASH_KERNEL_MFMA: "mfma", nb.DFLASH_KERNEL_REFERENCE: "ref"}


def _full(name, kernel, report=True, **kw):
    """Every output element of the workload against the oracle; full-size runs go into the
    session's parity report."""
    wl = workloads.make(name, **kw)
    t0 = time.perf_counter()
    ref = oracle.run_workload(wl)
    oracle_s = time.perf_counter() - t0
    got = H.to_f64(H.run(wl, kernel=kernel))
    m = H.assert_parity(got, ref, f"{name} kernel={kernel}")
    if report:
        H.record(name, KNAMES.get(kernel, str(kernel)), m, oracle_s, int(ref.shape[0] * ref.shape[1]))
    return m


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_c1_tiny_d128(kname, kernel):
    _full("c1_tiny_d128", kernel)


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_c2_paged_d256(kname, kernel):
    _full("c2_paged_d256", kernel)


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_c3_global_d512(kname, kernel):
    _full("c3_global_d512", kernel)


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_c4_causal_window_d256(kname, kernel):
    _full("c4_causal_window_d256", kernel)


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_c5_mixed_d512_reduced(kname, kernel):
    _full("c5_mixed_d512", kernel, report=False, ctx_cap=1500)


# target-side verification on a hybrid model: local sliding-window and global layers
def test_verify_local_window_d256():
    _full("v_local_window_d256", nb.DFLASH_KERNEL_MFMA)


def test_verify_global_d512():
    _full("v_global_d512", nb.DFLASH_KERNEL_MFMA)


def test_c5_mixed_d512_full_every_row():
    """The full-size mixed batch (B = 64, lognormal contexts up to 131072 keys) in the
    benchmark's launch configuration, every output element against the fp64 oracle
    (about 9 s of oracle time on 16 host threads)."""
    _full("c5_mixed_d512", nb.DFLASH_KERNEL_AUTO)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
EDGE = [
    # (Hq, Hkv, D, ctx_lens, block_lens, causal, window, page_size)
    (4, 1, 128, [0, 1, 15, 16, 17, 31, 32, 33], [1, 2, 9, 16, 1, 2, 9, 16], [0, 1, 0, 1, 0, 1, 0, 1], 0, 16),
    (8, 8, 256, [0, 5, 40], [3, 0, 7], [1, 0, 1], 0, 16),          # Hq == Hkv, an empty block
    (32, 4, 512, [100, 63, 64], [16, 9, 1], [0, 1, 0], 0, 16),     # 128 rows: two row groups
    (16, 2, 64, [70, 3], [5, 4], [1, 0], 0, 16),                   # head_dim 64 (padded)
    (16, 2, 136, [70, 3], [5, 4], [1, 0], 0, 16),                  # head_dim 136 (padded)
    (16, 4, 264, [130, 9], [9, 16], [0, 1], 0, 16),                # head_dim 264 (padded 512)
    (8, 2, 128, [50, 200, 7], [9, 5, 4], [1, 1, 0], 1, 16),        # window 1: only itself
    (8, 2, 128, [50, 200, 7], [9, 5, 4], [1, 0, 1], 2, 16),
    (8, 2, 128, [50, 200, 7], [9, 5, 4], [1, 0, 1], 16, 16),
    (8, 2, 128, [50, 200, 7], [9, 5, 4], [0, 0, 0], 17, 16),       # non-causal + window
    (8, 2, 128, [50, 200, 7], [9, 5, 4], [1, 1, 1], 300, 16),      # window wider than the context
    (8, 2, 256, [333, 77], [9, 9], [0, 1], 0, 8),                  # page size 8
    (8, 2, 256, [333, 77], [9, 9], [0, 1], 40, 32),                # page size 32
    (8, 2, 128, [0], [1], [0], 0, 16),                             # a single key
    (12, 3, 128, [1000, 2, 515], [15, 16, 9], [1, 0, 1], 100, 16),
    (6, 2, 128, [700, 33], [9, 5], [0, 1], 0, 16),                 # Hq not a multiple of the combine's rows per wave
    (3, 3, 64, [400, 90], [7, 3], [1, 0], 0, 16),                  # Hq == Hkv == 3, head_dim 64
    (16, 2, 264, [300, 41], [9, 10], [0, 1], 0, 16),               # 72 rows at padded head_dim 512: five row tiles
]


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_edges(case, kname, kernel):
    Hq, Hkv, D, L, n, c, W, P = EDGE[case]
    wl = workloads.build(len(L), Hq, Hkv, D, L, n, c, window=W, seed=100 + case, page_size=P, extra_pages=2)
    ref = oracle.run_workload(wl)
    for nwg in (0, 1, 5):
        got = H.to_f64(H.run(wl, kernel=kernel, num_workgroups=nwg))
        H.assert_parity(got, ref, f"edge {case} kernel={kname} wg={nwg}")


def test_causal_null_means_all_noncausal():
    wl = workloads.build(3, 8, 2, 128, [40, 9, 100], [9, 4, 9], [0, 0, 0], seed=5)
    ref = oracle.run_workload(wl)
    got = H.to_f64(H.run(wl, causal_none=True))
    H.assert_parity(got, ref, "causal=NULL")


def test_no_hints():
    wl = workloads.make("c2_paged_d256", ctx_cap=900)
    ref = oracle.run_workload(wl)
    H.assert_parity(H.to_f64(H.run(wl, hints=False)), ref, "no hints")


# ---------------------------------------------------------------------------
# key-set membership: a dominant key planted at each mask edge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_spike_at_mask_edges(kname, kernel):
    """Query i's logit for one key is made huge.  If the key is visible the output is
    that key's value row; if not, the output ignores it.  Keys probed: the block's
    own i and i+1 (causal edge), and the window edges lo-1 and lo."""
    Hq, Hkv, D, L, n, W = 4, 1, 128, 70, 6, 9
    for causal in (0, 1):
        for target_rel in ("self", "next", "lo", "lo-1"):
            rng = np.random.default_rng(11)
            wl = workloads.build(1, Hq, Hkv, D, [L], [n], [causal], window=W, seed=3)
            k = workloads.bf16_bits_to_f32(wl.k).astype(np.float32) * 0.05
            q = np.zeros((n, Hq, D), np.float32)
            for i in range(n):
                p = L + i
                tgt = {"self": p, "next": p + 1, "lo": p - W + 1, "lo-1": p - W}[target_rel]
                if not (0 <= tgt < L + n):
                    continue
                # one distinct direction per query position
                dirv = np.zeros(D, np.float32)
                dirv[i % D] = 1.0
                k[tgt, 0] += 4.0 * dirv
                q[i, :, :] = 30.0 * dirv
            wl.k = workloads.f32_to_bf16_bits(k)
            wl.q = workloads.f32_to_bf16_bits(q)
            wl.k_pages = workloads.scatter_to_pages(wl.k, wl.kv_lens, wl.page_table, wl.num_pages, wl.page_size, True)
            ref = oracle.run_workload(wl)
            got = H.to_f64(H.run(wl, kernel=kernel))
            H.assert_parity(got, ref, f"spike causal={causal} target={target_rel}")


def test_extreme_logit_range_recomputes_exactly():
    """Logits that climb by far more than 2^32 along the context: the lazy reference
    is abandoned and the segment recomputed with the exact row max."""
    Hq, Hkv, D = 4, 1, 128
    for L in (40, 700, 3000):
        wl = workloads.build(2, Hq, Hkv, D, [L, 33], [9, 5], [0, 1], seed=21)
        k = workloads.bf16_bits_to_f32(wl.k).astype(np.float32)
        # key norms grow along the sequence: later tiles have much larger logits
        ramp = np.linspace(0.0, 200.0, k.shape[0], dtype=np.float32)
        k[:, 0, 0] = ramp
        q = workloads.bf16_bits_to_f32(wl.q).astype(np.float32)
        q[:, :, 0] = 8.0
        wl.k = workloads.f32_to_bf16_bits(k)
        wl.q = workloads.f32_to_bf16_bits(q)
        wl.k_pages = workloads.scatter_to_pages(wl.k, wl.kv_lens, wl.page_table, wl.num_pages, wl.page_size, True)
        ref = oracle.run_workload(wl)
        for nwg in (0, 1, 3):
            got = H.to_f64(H.run(wl, num_workgroups=nwg))
            H.assert_parity(got, ref, f"extreme L={L} wg={nwg}")


# ---------------------------------------------------------------------------
# properties of the GPU path itself
# ---------------------------------------------------------------------------
def test_split_invariance():
    """Any split of the key ranges over workgroups gives the oracle's result, and the
    splits agree with each other element by element within the bound the rounding
    steps allow (tests/error_model.py: bf16 weights rounded against each piece's own
    reference maximum, bf16 partials, the final bf16 rounding)."""
    wl = workloads.make("c3_global_d512", ctx_cap=4000)
    ref = oracle.run_workload(wl)
    bound = error_model.split_bound(ref, error_model.split_sigma(wl))
    t = H.upload(wl)
    base = H.to_f64(H.run(wl, t, num_workgroups=1))
    H.assert_parity(base, ref, "split 1")
    for nwg in (2, 3, 7, 64, 256, 1000):
        for mode in (nb.DFLASH_MERGE_COMBINE_KERNEL, nb.DFLASH_MERGE_IN_KERNEL):
            got = H.to_f64(H.run(wl, t, num_workgroups=nwg, merge_mode=mode))
            H.assert_parity(got, ref, f"split {nwg} merge {mode}")
            excess = np.abs(got - base) - bound
            worst = int(np.argmax(excess))
            assert excess.flat[worst] <= 0, (nwg, mode, got.flat[worst], base.flat[worst], bound.flat[worst])


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_more_than_64_requests(kname, kernel):
    """130 requests: the kernels locate runs and tokens over several 64-request
    chunks of the length arrays (the one-load path covers at most 64)."""
    rng = np.random.default_rng(77)
    B = 130
    L = rng.integers(0, 400, size=B)
    n = rng.integers(0, 10, size=B)
    c = rng.integers(0, 2, size=B)
    wl = workloads.build(B, 8, 2, 128, L, n, c, seed=78)
    ref = oracle.run_workload(wl)
    for nwg in (0, 37):
        got = H.to_f64(H.run(wl, kernel=kernel, num_workgroups=nwg))
        H.assert_parity(got, ref, f"B=130 kernel={kname} wg={nwg}")


@pytest.mark.parametrize("merge", ["combine", "in-kernel"])
@pytest.mark.parametrize("D,L0", [(128, 8000), (512, 12000)])
def test_combine_over_more_than_64_pieces(D, L0, merge):
    """A unit split over hundreds of workgroups: the combine merges its pieces in
    rounds of 64 (rescaling earlier rounds to the running maximum).  One long request
    and one kv-head, so 600 workgroups take about one tile each.  At head_dim 128 one
    wave merges four rows; at head_dim 512 a workgroup merges one row with every
    fourth piece per wave (375 pieces: more than 64 per wave)."""
    wl = workloads.build(2, 8, 1, D, [L0, 300], [9, 5], [0, 1], seed=31)
    ref = oracle.run_workload(wl)
    mode = nb.DFLASH_MERGE_COMBINE_KERNEL if merge == "combine" else nb.DFLASH_MERGE_IN_KERNEL
    for nwg in (150, 600):
        got = H.to_f64(H.run(wl, num_workgroups=nwg, merge_mode=mode))
        H.assert_parity(got, ref, f"many pieces D={D} wg={nwg} merge={merge}")


def test_page_permutation_invariance_is_bitwise():
    a = workloads.make("c2_paged_d256", ctx_cap=1200)
    b = workloads.build(a.B, a.Hq, a.Hkv, a.D, a.ctx_lens, a.block_lens, a.causal, seed=999, extra_pages=5)
    # same logical data, different physical pages
    b.q, b.k, b.v = a.q, a.k, a.v
    b.k_pages = workloads.scatter_to_pages(b.k, b.kv_lens, b.page_table, b.num_pages, b.page_size, True)
    b.v_pages = workloads.scatter_to_pages(b.v, b.kv_lens, b.page_table, b.num_pages, b.page_size, True)
    oa = H.run(a).cpu()
    ob = H.run(b).cpu()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_determinism_is_bitwise():
    wl = workloads.make("c4_causal_window_d256")
    t = H.upload(wl)
    o1 = H.run(wl, t).cpu()
    o2 = H.run(wl, t).cpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name,B", [("c5_mixed_d512", 12), ("c2_paged_d256", 8)])
@pytest.mark.parametrize("mode", [nb.DFLASH_MERGE_COMBINE_KERNEL, nb.DFLASH_MERGE_IN_KERNEL])
def test_poison_and_guard_bands(mode, name, B):
    """NaN page tails and unused pages never reach the output; rows of `out` outside
    the call's range are never written, and nothing outside the call's workspace is
    written (guard bands on both sides of it).  Head_dim 256 with the combine kernel
    also covers the merge directory at the workspace's end."""
    wl = workloads.make(name, ctx_cap=700, B=B)   # pages are NaN-poisoned
    ref = oracle.run_workload(wl)
    t = H.upload(wl)
    guard = 7
    big = torch.full((wl.total_q + 2 * guard, wl.Hq, wl.D), 3.0, dtype=torch.bfloat16, device=H.dev())
    inner = big[guard:guard + wl.total_q]
    for nwg in (0, 9, 60):
        d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                         total_kv_len=wl.total_kv, page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                         num_pages=wl.num_pages, num_workgroups=nwg, merge_mode=mode)
        need = nb.dflash_block_attn_workspace_size(d, wl.Hq, wl.Hkv, wl.D)
        gb = 1 << 16
        wsbig = torch.full((need + 2 * gb,), 0xA5, dtype=torch.uint8, device=H.dev())
        wsbig[gb:gb + need].zero_()
        d.workspace, d.workspace_bytes = wsbig.data_ptr() + gb, need
        st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D,
                                  t["causal"], wl.window, wl.scale, inner, torch.cuda.current_stream().cuda_stream, d)
        assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
        torch.cuda.synchronize()
        H.assert_parity(H.to_f64(inner), ref, f"poison wg={nwg}")
        assert torch.all(big[:guard] == 3.0) and torch.all(big[guard + wl.total_q:] == 3.0)
        assert torch.all(wsbig[:gb] == 0xA5) and torch.all(wsbig[gb + need:] == 0xA5), f"workspace guard wg={nwg}"


def test_timing_events_are_recorded():
    wl = workloads.make("c1_tiny_d128")
    t = H.upload(wl)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()  # torch creates the HIP event on first record
    ev1.record()
    torch.cuda.synchronize()
    assert ev0.cuda_event and ev1.cuda_event
    d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=9, total_kv_len=wl.total_kv,
                     page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req, num_pages=wl.num_pages)
    need = nb.dflash_block_attn_workspace_size(d, wl.Hq, wl.Hkv, wl.D)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=H.dev())
    d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
    d.event_attn_begin, d.event_attn_end = ev0.cuda_event, ev1.cuda_event
    out = torch.empty((wl.total_q, wl.Hq, wl.D), dtype=torch.bfloat16, device=H.dev())
    st = nb.dflash_block_attn(t["q"], t["k"], t["v"], t["pt"], t["ctx"], t["blk"], wl.Hq, wl.Hkv, wl.D, t["causal"],
                              wl.window, wl.scale, out, torch.cuda.current_stream().cuda_stream, d)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    assert ev0.elapsed_time(ev1) > 0
    H.assert_parity(H.to_f64(out), oracle.run_workload(wl), "events")


def test_plan_on_device():
    wl = workloads.make("c3_global_d512")
    d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=9, total_kv_len=wl.total_kv,
                     page_size=16, max_pages_per_req=wl.max_pages_per_req, num_pages=wl.num_pages)
    p = nb.dflash_block_attn_plan(d, wl.Hq, wl.Hkv, wl.D)
    props = torch.cuda.get_device_properties(0)
    assert p.kernel == nb.DFLASH_KERNEL_MFMA and p.rows_per_unit == 80
    assert p.num_workgroups % props.multi_processor_count == 0
