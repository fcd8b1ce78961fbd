"""Block K/V append on the GPU, append + attention in one call, and graph capture.

* dflash_block_kv_append writes exactly the block slots: the whole page arrays
  equal the oracle's append, bit for bit (every other slot keeps its poison).
* dflash_block_attn_append on context-only pages equals the fp64 oracle's
  attention over the full workload (same tolerances as every parity test).
* The whole call captured into a HIP graph (torch.cuda.CUDAGraph) at each
  block-aligned capture size (9, 18, 36, 72 query tokens) replays correctly: three
  replays, each after eager work that restores the context-only pages and clears
  the output, each bit-identical to the eager call.
* Where the append is fused into the attention launch (MFMA kernel, pages of >= 16
  keys), output and pages equal those of the two separate calls, bit for bit.
"""
import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import oracle
import workloads
from gpu_helpers import assert_parity, bf16_tensor, dev, to_f64
from oracle.append import block_kv_append

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Hq, Hkv, D, ctx_lens, block_lens, causal, window, page_size)
    (1, 8, 2, 128, [512], [9], [0], 0, 16),                                   # C1 shape
    (4, 32, 8, 256, [1100, 2000, 1500, 4000], [9, 9, 9, 9], [0, 0, 0, 0], 0, 16),
    (3, 16, 4, 512, [0, 37, 300], [5, 16, 1], [1, 0, 1], 0, 16),
    (5, 8, 2, 64, [3, 70, 0, 15, 16], [4, 0, 9, 1, 16], [0, 1, 0, 1, 0], 0, 8),  # page 8, an empty block
    (2, 8, 8, 136, [33, 60], [9, 3], [1, 1], 20, 32),
]


def _setup(i):
    B, Hq, Hkv, D, ctx, blk, c, W, P = CASES[i]
    wl = workloads.build(B, Hq, Hkv, D, ctx, blk, c, window=W, seed=400 + i, page_size=P, extra_pages=2)
    return (wl, *workloads.split_block_kv(wl))


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _desc(wl, workspace=None):
    d = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                     total_kv_len=wl.total_kv, page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                     num_pages=wl.num_pages)
    need = nb.dflash_block_attn_workspace_size(d, wl.Hq, wl.Hkv, wl.D)
    ws = workspace if workspace is not None else torch.zeros(max(need, 256), dtype=torch.uint8, device=dev())
    d.workspace, d.workspace_bytes = ws.data_ptr(), ws.numel()
    return d, ws


def _inputs(wl, k_new, v_new, kc, vc):
    d = dev()
    return dict(q=bf16_tensor(wl.q, d), kn=bf16_tensor(k_new, d), vn=bf16_tensor(v_new, d), kp=bf16_tensor(kc, d),
                vp=bf16_tensor(vc, d), pt=torch.from_numpy(wl.page_table).to(d),
                ctx=torch.from_numpy(wl.ctx_lens).to(d), blk=torch.from_numpy(wl.block_lens).to(d),
                causal=torch.from_numpy(wl.causal).to(d),
                out=torch.empty((wl.total_q, wl.Hq, wl.D), dtype=torch.bfloat16, device=d))


def _attn_append(wl, t, desc, stream):
    return nb.dflash_block_attn_append(t["q"], t["kn"], t["vn"], t["kp"], t["vp"], t["pt"], t["ctx"], t["blk"],
                                       wl.Hq, wl.Hkv, wl.D, t["causal"], wl.window, wl.scale, t["out"], stream, desc)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_append_writes_exactly_the_block_slots(case):
    wl, k_new, v_new, kc, vc = _setup(case)
    want_k, want_v = block_kv_append(kc, vc, k_new, v_new, wl.page_table, wl.ctx_lens, wl.block_lens)
    t = _inputs(wl, k_new, v_new, kc, vc)
    desc, _ = _desc(wl)
    st = nb.dflash_block_kv_append(t["kn"], t["vn"], t["kp"], t["vp"], t["pt"], t["ctx"], t["blk"], wl.Hkv, wl.D,
                                   torch.cuda.current_stream().cuda_stream, desc)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(t["kp"]), want_k)
    assert np.array_equal(_bits(t["vp"]), want_v)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attn_append_matches_oracle(case):
    wl, k_new, v_new, kc, vc = _setup(case)
    t = _inputs(wl, k_new, v_new, kc, vc)
    desc, _ = _desc(wl)
    st = _attn_append(wl, t, desc, torch.cuda.current_stream().cuda_stream)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    assert np.array_equal(_bits(t["kp"]), wl.k_pages) and np.array_equal(_bits(t["vp"]), wl.v_pages)
    assert_parity(to_f64(t["out"]), oracle.run_workload(wl), f"append case {case}")


def _draft_step(shape: str, B: int):
    """A draft step at a block-aligned capture size: B requests x block 9 (9, 18, 36 or 72
    query tokens), request shapes of the C1 (head_dim 128) and C2 (head_dim 256) workloads."""
    rng = np.random.default_rng(2000 + B)
    if shape == "c1":
        Hq, Hkv, D, ctx = 8, 2, 128, np.full(B, 512)
    else:
        Hq, Hkv, D, ctx = 32, 8, 256, rng.integers(1024, 4097, size=B)
    wl = workloads.build(B, Hq, Hkv, D, ctx, np.full(B, 9), np.zeros(B, dtype=np.uint8), seed=2100 + B)
    return (wl, *workloads.split_block_kv(wl))


@pytest.mark.parametrize("shape", ["c1", "c2"])
@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_graph_capture_replays_match_eager(shape, B):
    """The whole draft step captured into a HIP graph at each capture size replays
    bit-identically to the eager call, three times, with eager work (pages restored,
    output cleared) and synchronisations between the replays."""
    wl, k_new, v_new, kc, vc = _draft_step(shape, B)
    t = _inputs(wl, k_new, v_new, kc, vc)
    kc_dev, vc_dev = t["kp"].clone(), t["vp"].clone()
    desc, ws = _desc(wl)
    side = torch.cuda.Stream()
    # eager reference (also warms the library's per-device caches before capture)
    with torch.cuda.stream(side):
        assert _attn_append(wl, t, desc, side.cuda_stream) == nb.DFLASH_OK
    torch.cuda.synchronize()
    out_eager, kp_eager, vp_eager = t["out"].clone(), t["kp"].clone(), t["vp"].clone()
    assert_parity(to_f64(out_eager), oracle.run_workload(wl), "eager")
    assert np.array_equal(_bits(kp_eager), wl.k_pages) and np.array_equal(_bits(vp_eager), wl.v_pages)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        st = _attn_append(wl, t, desc, side.cuda_stream)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    for rep in range(3):
        t["kp"].copy_(kc_dev)
        t["vp"].copy_(vc_dev)
        t["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(t["out"].view(torch.int16), out_eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(t["kp"].view(torch.int16), kp_eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(t["vp"].view(torch.int16), vp_eager.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_append_equals_append_then_attention(case):
    """dflash_block_attn_append (one launch where the append is fused) against the two
    separate calls on the same inputs: the same output and the same pages, bit for bit."""
    wl, k_new, v_new, kc, vc = _setup(case)
    stream = torch.cuda.current_stream().cuda_stream
    t1 = _inputs(wl, k_new, v_new, kc, vc)
    desc, _ = _desc(wl)
    assert _attn_append(wl, t1, desc, stream) == nb.DFLASH_OK, nb.dflash_last_error_message()
    t2 = _inputs(wl, k_new, v_new, kc, vc)
    desc2, _ = _desc(wl)
    st = nb.dflash_block_kv_append(t2["kn"], t2["vn"], t2["kp"], t2["vp"], t2["pt"], t2["ctx"], t2["blk"], wl.Hkv,
                                   wl.D, stream, desc2)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    st = nb.dflash_block_attn(t2["q"], t2["kp"], t2["vp"], t2["pt"], t2["ctx"], t2["blk"], wl.Hq, wl.Hkv, wl.D,
                              t2["causal"], wl.window, wl.scale, t2["out"], stream, desc2)
    assert st == nb.DFLASH_OK, nb.dflash_last_error_message()
    torch.cuda.synchronize()
    assert torch.equal(t1["out"].view(torch.int16), t2["out"].view(torch.int16))
    assert torch.equal(t1["kp"].view(torch.int16), t2["kp"].view(torch.int16))
    assert torch.equal(t1["vp"].view(torch.int16), t2["vp"].view(torch.int16))
