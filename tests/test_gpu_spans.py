"""Bidirectional spans in causal requests (the multimodal-prefix mask) on the
HIP path, through dflash_block_attn_spans, against the fp64 oracle.

Parity bar as everywhere: max|err| <= 2e-2, mean|err| <= 2e-3, relative RMS
<= 1e-2.  At long contexts one extra visible key moves an output by far less
than that, so membership is probed with planted dominant keys, and the span
that covers a whole block is checked bitwise against the non-causal call.
"""
import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import oracle
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KERNELS = [("mfma", nb.DFLASH_KERNEL_MFMA), ("ref", nb.DFLASH_KERNEL_REFERENCE)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the oracle library was compiled at session start, before the GPU was touched


SMALL = [
    # (Hq, Hkv, D, ctx_lens, block_lens, causal, window)
    (8, 2, 128, [0, 5, 40, 130, 17], [16, 9, 9, 16, 1], [1, 1, 0, 1, 1], 0),
    (32, 4, 512, [300, 64, 1000], [9, 16, 9], [1, 1, 1], 0),        # two row groups at 16 x 8 rows
    (16, 4, 256, [700, 90, 2000, 5], [16, 9, 16, 9], [1, 0, 1, 1], 64),
    (12, 3, 136, [33, 250], [15, 9], [1, 1], 0),                     # padded head_dim
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_random_spans_parity(case, kname, kernel):
    Hq, Hkv, D, L, n, c, W = SMALL[case]
    wl = workloads.build(len(L), Hq, Hkv, D, L, n, c, window=W, seed=300 + case)
    for sseed in range(3):
        spans = workloads.draw_spans(wl.ctx_lens, wl.block_lens, seed=50 * case + sseed, max_prefix_span=64)
        ref = oracle.run_workload(wl, spans=spans)
        for nwg in (0, 1, 5):
            got = H.to_f64(H.run(wl, kernel=kernel, num_workgroups=nwg, spans=spans))
            H.assert_parity(got, ref, f"spans case {case} sseed {sseed} kernel={kname} wg={nwg}")


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_span_over_the_block_equals_non_causal_bitwise(kname, kernel):
    wl = workloads.build(4, 16, 4, 256, [100, 0, 37, 900], [9, 16, 5, 9], [1, 1, 1, 1], window=50, seed=8)
    t = H.upload(wl)
    spans = [[(max(0, int(L) - 3), int(L + n))] for L, n in zip(wl.ctx_lens, wl.block_lens)]
    a = H.run(wl, t, kernel=kernel, spans=spans).cpu()
    t_nc = dict(t, causal=torch.zeros_like(t["causal"]))
    b = H.run(wl, t_nc, kernel=kernel).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_no_spans_or_context_spans_equal_plain_causal_bitwise(kname, kernel):
    wl = workloads.build(3, 8, 2, 128, [60, 200, 9], [9, 9, 16], [1, 1, 1], seed=9)
    t = H.upload(wl)
    plain = H.run(wl, t, kernel=kernel).cpu().view(torch.int16)
    for spans in ([[], [], []], [[(0, 60)], [(5, 7), (100, 200)], []]):
        got = H.run(wl, t, kernel=kernel, spans=spans).cpu().view(torch.int16)
        assert torch.equal(got, plain), spans


@pytest.mark.parametrize("kname,kernel", KERNELS)
def test_spike_at_span_edges(kname, kernel):
    """Query i's logit for one key is made huge: the output is that key's value row
    when the key is visible and ignores it otherwise.  Keys probed around a span
    [s, e) that covers block positions: e - 1 (visible from inside the span), e
    (never visible from before it), and the key after the query for a query
    outside every span."""
    Hq, Hkv, D, L, n = 4, 1, 128, 70, 12
    s, e = L + 3, L + 8
    for target_rel in ("end-1", "end", "next"):
        wl = workloads.build(1, Hq, Hkv, D, [L], [n], [1], seed=3)
        k = workloads.bf16_bits_to_f32(wl.k).astype(np.float32) * 0.05
        q = np.zeros((n, Hq, D), np.float32)
        for i in range(n):
            p = L + i
            tgt = {"end-1": e - 1, "end": e, "next": p + 1}[target_rel]
            if not (0 <= tgt < L + n):
                continue
            dirv = np.zeros(D, np.float32)
            dirv[i % D] = 1.0
            k[tgt, 0] += 4.0 * dirv
            q[i, :, :] = 30.0 * dirv
        wl.k = workloads.f32_to_bf16_bits(k)
        wl.q = workloads.f32_to_bf16_bits(q)
        wl.k_pages = workloads.scatter_to_pages(wl.k, wl.kv_lens, wl.page_table, wl.num_pages, wl.page_size, True)
        spans = [[(s, e)]]
        ref = oracle.run_workload(wl, spans=spans)
        got = H.to_f64(H.run(wl, kernel=kernel, spans=spans))
        H.assert_parity(got, ref, f"span spike target={target_rel}")


def test_verify_global_d512_with_spans_sampled():
    """The causal global-layer verification workload at full size (L ~ U[8192, 32768],
    D 512) with seeded spans, in the default launch configuration; the oracle
    computes every row of the requests whose spans widen some block query's range,
    and 300 random rows."""
    wl = workloads.make("v_global_d512")
    spans = workloads.draw_spans(wl.ctx_lens, wl.block_lens, seed=77)
    out = H.to_f64(H.run(wl, spans=spans)).reshape(-1, wl.D)
    qs = wl.q_start
    widened = [r for r in range(wl.B) if any(e - 1 > max(s, int(wl.ctx_lens[r])) for s, e in spans[r])]
    assert len(widened) >= 2, widened
    pick = set()
    for r in widened:
        for t in range(qs[r], qs[r + 1]):
            pick.update(range(t * wl.Hq, (t + 1) * wl.Hq))
    rng = np.random.default_rng(1)
    pick.update(rng.choice(wl.total_q * wl.Hq, size=300, replace=False).tolist())
    rows = np.array(sorted(pick), dtype=np.int64)
    ref = oracle.run_workload(wl, rows=rows, spans=spans)
    H.assert_parity(out[rows], ref, "v_global_d512 spans sampled")
