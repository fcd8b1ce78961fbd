"""Seeded input generator: determinism, bf16 rounding, paging layout, poisoning."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-40, np.inf, -np.inf], np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_arrays():
    a = workloads.make("c2_paged_d256", ctx_cap=64, B=3)
    b = workloads.make("c2_paged_d256", ctx_cap=64, B=3)
    for f in ("q", "k", "v", "k_pages", "v_pages", "page_table", "ctx_lens", "block_lens", "causal"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_reduced_variant_keeps_full_size_length_draws():
    cfg = workloads.CONFIGS["c5_mixed_d512"]
    rng = np.random.Generator(np.random.PCG64(workloads.default_seed("c5_mixed_d512")))
    ctx = workloads._draw_ctx(rng, cfg.ctx_law, cfg.B)
    red = workloads.make("c5_mixed_d512", ctx_cap=50, B=8)
    assert np.array_equal(red.ctx_lens, np.minimum(ctx[:8], 50))


def test_config_laws():
    for name in ("c2_paged_d256", "c3_global_d512", "c5_mixed_d512", "c4_causal_window_d256"):
        cfg = workloads.CONFIGS[name]
        rng = np.random.Generator(np.random.PCG64(workloads.default_seed(name)))
        ctx = workloads._draw_ctx(rng, cfg.ctx_law, cfg.B)
        law = cfg.ctx_law
        if law[0] == "uniform":
            assert ctx.min() >= law[1] and ctx.max() <= law[2]
        if law[0] == "lognormal":
            assert ctx.min() >= law[3] and ctx.max() <= law[4]
        if law[0] == "fixed":
            assert (ctx == law[1]).all()


def test_paging_is_a_bijection_and_poisons_the_rest():
    wl = workloads.make("c2_paged_d256", ctx_cap=100, B=4)
    P = wl.page_size
    used = []
    for r in range(wl.B):
        T = int(wl.kv_lens[r])
        npg = (T + P - 1) // P
        assert (wl.page_table[r, :npg] >= 0).all() and (wl.page_table[r, npg:] == -1).all()
        used.extend(wl.page_table[r, :npg].tolist())
        base = int(wl.kv_start[r])
        for j in range(T):
            pg = wl.page_table[r, j // P]
            assert np.array_equal(wl.k_pages[pg, j % P], wl.k[base + j])
            assert np.array_equal(wl.v_pages[pg, j % P], wl.v[base + j])
        # tail slots of the last page are NaN
        for j in range(T, npg * P):
            pg = wl.page_table[r, j // P]
            assert (wl.k_pages[pg, j % P] == workloads.BF16_NAN).all()
    assert len(set(used)) == len(used)
    unused = sorted(set(range(wl.num_pages)) - set(used))
    assert len(unused) == 1
    assert (wl.k_pages[unused[0]] == workloads.BF16_NAN).all()


def test_values_are_standard_normal():
    wl = workloads.make("c3_global_d512", ctx_cap=2000, B=2)
    x = workloads.bf16_bits_to_f32(wl.k).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_draw_spans_are_sorted_disjoint_and_inside_the_request():
    ctx = np.array([0, 5, 100, 20000, 3, 0], dtype=np.int32)
    blk = np.array([16, 9, 0, 9, 1, 0], dtype=np.int32)
    hits = 0
    for seed in range(40):
        spans = workloads.draw_spans(ctx, blk, seed=seed)
        assert spans == workloads.draw_spans(ctx, blk, seed=seed)
        assert len(spans) == len(ctx)
        for L, n, lst in zip(ctx.tolist(), blk.tolist(), spans):
            end = 0
            for s, e in lst:
                assert end <= s < e <= L + n
                end = e
                hits += e > L and n > 0
    assert hits > 20   # spans reach into blocks often enough to matter
