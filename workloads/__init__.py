"""Seeded synthetic workloads for DFlash block attention.

This module only draws random inputs and lays them out in memory.  It holds
none of the attention arithmetic: both the fp64 oracle (``oracle/``) and the
HIP path (``non_causal_block_amd``) consume what it produces, and neither is
imported here.

Shapes follow the pages' workloads:
  * a request's block is ``1 + num_speculative_tokens`` queries (9 for 8
    speculative tokens; 16 for 15), kenforever1 "DFlash + Gemma 4 31B-it"
    notes, sections "why non-causal attention" and the PR #52 change table;
  * global layers use head_dim 512, same notes, section "Gemma 4 31B-it
    structure";
  * causal / sliding-window variants, vLLM PR #43445 report, "motivation".
The five configurations below are the synthetic stand-ins for those
workloads (GQA, bf16 values ~ N(0,1), paged KV with 16-token pages); two more
(``v_*``) are the target's verification of the same blocks on a hybrid model.

Recipe (fixed, so that every consumer sees identical arrays):
  numpy ``Generator(PCG64(seed))``; draw order lengths -> speculative token
  counts -> causal flags -> page permutation -> Q -> K -> V.  Values are
  float32 N(0,1) rounded to bf16 (round to nearest even).  Q/K/V are drawn
  request by request in chunks of at most ``_CHUNK_ROWS`` rows, K and V as
  logical ``[T_r, Hkv, D]`` blocks (context keys followed by the block's own
  keys).  Lognormal contexts use sigma = 1 (natural log).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
_CHUNK_ROWS = 8192


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    # context length law: ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    ctx_law: tuple
    # speculative tokens per request: tuple of allowed k values (block = 1 + k)
    spec_k: tuple
    # causal law: ("all", bool) | ("bernoulli", p)
    causal_law: tuple
    window: int = 0
    page_size: int = 16
    permute_pages: bool = True
    description: str = ""


CONFIGS = {
    "c1_tiny_d128": Config(
        "c1_tiny_d128", B=1, Hq=8, Hkv=2, D=128, ctx_law=("fixed", 512), spec_k=(8,),
        causal_law=("all", False), permute_pages=False,
        description="non-causal, B=1, block 9, L=512, Hq 8 / Hkv 2, D 128, contiguous KV"),
    "c2_paged_d256": Config(
        "c2_paged_d256", B=8, Hq=32, Hkv=8, D=256, ctx_law=("uniform", 1024, 4096), spec_k=(8,),
        causal_law=("all", False),
        description="non-causal, B=8 x block 9, L~U[1024,4096], Hq 32 / Hkv 8, D 256, paged+permuted"),
    "c3_global_d512": Config(
        "c3_global_d512", B=4, Hq=32, Hkv=4, D=512, ctx_law=("uniform", 8192, 32768), spec_k=(8,),
        causal_law=("all", False),
        description="non-causal global layer, B=4 x block 9, L~U[8192,32768], Hq 32 / Hkv 4, D 512, paged"),
    "c4_causal_window_d256": Config(
        "c4_causal_window_d256", B=16, Hq=32, Hkv=8, D=256, ctx_law=("fixed", 16384), spec_k=(15,),
        causal_law=("all", True), window=1024, permute_pages=False,
        description="causal sliding window W=1024, B=16 x block 16, L=16384, Hq 32 / Hkv 8, D 256"),
    "c5_mixed_d512": Config(
        "c5_mixed_d512", B=64, Hq=32, Hkv=8, D=512, ctx_law=("lognormal", 4096, 1.0, 256, 131072),
        spec_k=(4, 8, 15), causal_law=("bernoulli", 0.25),
        description="mixed batch B=64, k in {4,8,15}, lognormal L (median 4096), 25% causal, D 512, paged"),
    # Target-side verification of the same blocks on a hybrid model: the verifier runs
    # many local sliding-window layers and periodic global layers at head_dim 512
    # (kenforever1 notes, "Gemma 4 31B-it structure"), each over the 1 + k block
    # causally.  The pages give no window size or head counts: W = 1024 and the head
    # counts of the configurations above are readings.
    "v_local_window_d256": Config(
        "v_local_window_d256", B=8, Hq=32, Hkv=8, D=256, ctx_law=("uniform", 8192, 32768), spec_k=(8,),
        causal_law=("all", True), window=1024,
        description="verify, local sliding-window layer: causal, W=1024, B=8 x block 9, L~U[8192,32768], "
                    "Hq 32 / Hkv 8, D 256, paged"),
    "v_global_d512": Config(
        "v_global_d512", B=8, Hq=32, Hkv=4, D=512, ctx_law=("uniform", 8192, 32768), spec_k=(8,),
        causal_law=("all", True),
        description="verify, global layer: causal, B=8 x block 9, L~U[8192,32768], Hq 32 / Hkv 4, D 512, paged"),
}
CONFIG_ORDER = list(CONFIGS)
SEED_BASE = 1000


def default_seed(name: str) -> int:
    return SEED_BASE + CONFIG_ORDER.index(name)


# ----------------------------------------------------------------------------
# workload container
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    window: int
    scale: float
    ctx_lens: np.ndarray      # int32 [B]
    block_lens: np.ndarray    # int32 [B]
    causal: np.ndarray        # uint8 [B]
    q: np.ndarray             # uint16 (bf16 bits) [total_q, Hq, D]
    k: np.ndarray             # uint16 [total_kv, Hkv, D], logical, request-major
    v: np.ndarray             # uint16 [total_kv, Hkv, D]
    page_size: int
    page_table: np.ndarray    # int32 [B, max_pages_per_req], -1 past the last page
    k_pages: np.ndarray       # uint16 [num_pages, page_size, Hkv, D]
    v_pages: np.ndarray

    @property
    def total_q(self) -> int:
        return int(self.block_lens.sum())

    @property
    def kv_lens(self) -> np.ndarray:
        return self.ctx_lens.astype(np.int64) + self.block_lens.astype(np.int64)

    @property
    def total_kv(self) -> int:
        return int(self.kv_lens.sum())

    @property
    def q_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.block_lens.astype(np.int64))])

    @property
    def kv_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.kv_lens)])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def max_pages_per_req(self) -> int:
        return int(self.page_table.shape[1])


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------
def _draw_ctx(rng: np.random.Generator, law: tuple, B: int) -> np.ndarray:
    kind = law[0]
    if kind == "fixed":
        return np.full(B, law[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(law[1], law[2], size=B, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = law[1:]
        x = np.exp(rng.normal(math.log(median), sigma, size=B))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(f"unknown context law {law}")


def _draw_causal(rng: np.random.Generator, law: tuple, B: int) -> np.ndarray:
    if law[0] == "all":
        return np.full(B, 1 if law[1] else 0, dtype=np.uint8)
    if law[0] == "bernoulli":
        return (rng.random(B) < law[1]).astype(np.uint8)
    raise ValueError(f"unknown causal law {law}")


def _draw_bf16(rng: np.random.Generator, shape: tuple) -> np.ndarray:
    """N(0,1) float32 rounded to bf16, drawn in row chunks along axis 0."""
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    for s in range(0, rows, _CHUNK_ROWS):
        e = min(rows, s + _CHUNK_ROWS)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32))
    return out


def page_layout(kv_lens: np.ndarray, page_size: int, rng: Optional[np.random.Generator],
                extra_pages: int = 0):
    """Page table for the given per-request KV lengths.

    Logical page j of request r holds keys [j*page_size, (j+1)*page_size).  Physical
    page ids are 0..num_pages-1, assigned in request order (identity) or through a
    seeded permutation when ``rng`` is given.  ``extra_pages`` unused pages are added
    (they are never referenced by the table).
    """
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = kv_lens.shape[0]
    npg = (kv_lens + page_size - 1) // page_size
    used = int(npg.sum())
    num_pages = used + int(extra_pages)
    max_pages = max(1, int(npg.max()) if B else 1)
    phys = np.arange(num_pages, dtype=np.int64)
    if rng is not None:
        phys = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for r in range(B):
        table[r, : npg[r]] = phys[off: off + npg[r]]
        off += int(npg[r])
    return table, num_pages


def scatter_to_pages(logical: np.ndarray, kv_lens: np.ndarray, table: np.ndarray, num_pages: int,
                     page_size: int, poison: bool) -> np.ndarray:
    """Copy logical rows [total_kv, Hkv, D] into pages [num_pages, page_size, Hkv, D]."""
    Hkv, D = logical.shape[1], logical.shape[2]
    pages = np.empty((num_pages, page_size, Hkv, D), dtype=np.uint16)
    pages.fill(BF16_NAN if poison else 0)
    flat = pages.reshape(num_pages * page_size, Hkv, D)
    off = 0
    for r, T in enumerate(np.asarray(kv_lens, dtype=np.int64)):
        T = int(T)
        if T == 0:
            continue
        keys = np.arange(T, dtype=np.int64)
        phys_rows = table[r, keys // page_size].astype(np.int64) * page_size + keys % page_size
        flat[phys_rows] = logical[off: off + T]
        off += T
    return pages


def block_conv_inputs(block_lens, channels: int, groups: int, taps: int, seed: int):
    """Seeded inputs of DFlash2's in-block convolution, as bf16 bits.

    x ~ N(0, 1) [total_q, channels]; base ~ N(0, 1/taps) [taps, channels] and
    delta ~ N(0, 1/taps) [total_q, taps, groups] (so an output sums taps terms of
    unit-order size); draw order x -> base -> delta.  The scales are readings: the
    page gives the formula, not the coefficient statistics.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    total_q = int(np.sum(block_lens))
    x = f32_to_bf16_bits(rng.standard_normal((total_q, channels), dtype=np.float32))
    s = np.float32(1.0 / math.sqrt(taps))
    base = f32_to_bf16_bits(rng.standard_normal((taps, channels), dtype=np.float32) * s)
    delta = f32_to_bf16_bits(rng.standard_normal((total_q, taps, groups), dtype=np.float32) * s)
    return x, base, delta


def draw_spans(ctx_lens, block_lens, seed: int, max_prefix_span: int = 512):
    """Seeded bidirectional spans (the multimodal-prefix mask), one list per request.

    Each request gets, each with probability 1/2, in position order and disjoint:
    an image span inside the context (length U[1, max_prefix_span]); a span that
    starts within 16 positions before the block (or at its start) and ends
    U-uniformly inside the block or at its end; and one more span inside the
    rest of the block.  Only spans that hold block positions change a block
    query's mask; the context-only span is there to exercise the lookup.  The
    mix is a reading: the pages name the mask, not a span-length law.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for L, n in zip(np.asarray(ctx_lens).tolist(), np.asarray(block_lens).tolist()):
        T, lst, pos = L + n, [], 0
        if L > 0 and rng.random() < 0.5:
            s = int(rng.integers(0, L))
            e = min(L, s + int(rng.integers(1, max_prefix_span + 1)))
            lst.append((s, e))
            pos = e
        if n > 0 and rng.random() < 0.5:
            s = int(rng.integers(max(pos, L - 16), L + 1))
            e = int(rng.integers(max(s, L) + 1, T + 1))
            lst.append((s, e))
            pos = e
        if pos < T and max(pos, L) < T and rng.random() < 0.5:
            s = int(rng.integers(max(pos, L), T))
            e = int(rng.integers(s + 1, T + 1))
            lst.append((s, e))
        out.append(lst)
    return out


def split_block_kv(wl: "Workload"):
    """The block tokens' K/V rows and pages that hold only the context.

    Returns (k_new, v_new, k_pages_ctx, v_pages_ctx): k_new / v_new are bf16 bits
    [total_q, Hkv, D] -- row t is block token t - q_start[r] of its request,
    packed in request order like q -- and the page arrays equal wl.k_pages /
    wl.v_pages except that every block slot is NaN-poisoned (the state of the
    cache before a draft step writes its block).
    """
    kv_start = wl.kv_start
    rows = []
    for r in range(wl.B):
        L, n = int(wl.ctx_lens[r]), int(wl.block_lens[r])
        rows.extend(range(int(kv_start[r]) + L, int(kv_start[r]) + L + n))
    rows = np.asarray(rows, dtype=np.int64)
    k_new = np.ascontiguousarray(wl.k[rows])
    v_new = np.ascontiguousarray(wl.v[rows])
    k_ctx = wl.k.copy()
    v_ctx = wl.v.copy()
    k_ctx[rows] = BF16_NAN
    v_ctx[rows] = BF16_NAN
    k_pages = scatter_to_pages(k_ctx, wl.kv_lens, wl.page_table, wl.num_pages, wl.page_size, True)
    v_pages = scatter_to_pages(v_ctx, wl.kv_lens, wl.page_table, wl.num_pages, wl.page_size, True)
    return k_new, v_new, k_pages, v_pages


def build(B: int, Hq: int, Hkv: int, D: int, ctx_lens, block_lens, causal, *, window: int = 0,
          scale: Optional[float] = None, seed: int = 0, page_size: int = 16, permute_pages: bool = True,
          poison: bool = True, extra_pages: int = 0, name: str = "custom",
          rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw Q/K/V for explicitly given lengths and flags, then page K/V."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64).reshape(B)
    block_lens = np.asarray(block_lens, dtype=np.int64).reshape(B)
    causal = np.asarray(causal, dtype=np.uint8).reshape(B)
    kv_lens = ctx_lens + block_lens
    table, num_pages = page_layout(kv_lens, page_size, rng if permute_pages else None, extra_pages)
    total_q = int(block_lens.sum())
    q = np.empty((total_q, Hq, D), dtype=np.uint16)
    qs = 0
    for r in range(B):
        n = int(block_lens[r])
        if n:
            q[qs: qs + n] = _draw_bf16(rng, (n, Hq, D))
        qs += n
    kv = []
    for which in range(2):
        arr = np.empty((int(kv_lens.sum()), Hkv, D), dtype=np.uint16)
        off = 0
        for r in range(B):
            T = int(kv_lens[r])
            if T:
                arr[off: off + T] = _draw_bf16(rng, (T, Hkv, D))
            off += T
        kv.append(arr)
    k, v = kv
    k_pages = scatter_to_pages(k, kv_lens, table, num_pages, page_size, poison)
    v_pages = scatter_to_pages(v, kv_lens, table, num_pages, page_size, poison)
    return Workload(
        name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, window=int(window),
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        ctx_lens=ctx_lens.astype(np.int32), block_lens=block_lens.astype(np.int32), causal=causal,
        q=q, k=k, v=v, page_size=page_size, page_table=table, k_pages=k_pages, v_pages=v_pages)


def make(name: str, seed: Optional[int] = None, *, ctx_cap: Optional[int] = None, B: Optional[int] = None,
         poison: bool = True, extra_pages: int = 1) -> Workload:
    """Draw one of the named configurations.

    ``ctx_cap`` clips every context length (a reduced-length variant of the same
    configuration, used where the oracle must finish in seconds); ``B`` keeps only
    the first B requests' lengths (drawn from the full-size law first, so the
    draws of the kept requests are those of the full configuration).
    """
    cfg = CONFIGS[name]
    seed = default_seed(name) if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = _draw_ctx(rng, cfg.ctx_law, cfg.B)
    ks = np.asarray(cfg.spec_k)
    kk = ks[rng.integers(0, len(ks), size=cfg.B)] if len(ks) > 1 else np.full(cfg.B, ks[0])
    causal = _draw_causal(rng, cfg.causal_law, cfg.B)
    nB = cfg.B if B is None else int(B)
    ctx, kk, causal = ctx[:nB], kk[:nB], causal[:nB]
    if ctx_cap is not None:
        ctx = np.minimum(ctx, int(ctx_cap))
    return build(nB, cfg.Hq, cfg.Hkv, cfg.D, ctx, 1 + kk, causal, window=cfg.window,
                 seed=seed, page_size=cfg.page_size, permute_pages=cfg.permute_pages, poison=poison,
                 extra_pages=extra_pages, name=name if (ctx_cap is None and B is None) else name + "_reduced",
                 rng=rng)
