// decomp.h -- how a call's work is cut into equal runs of key tiles.
//
// Host code (the planner) and every kernel include this one header, so the
// attention kernels, the split-KV combine and the planner derive the same
// key ranges, windows and split points from the same lengths.  (A split
// schedule computed from facts that differ from the kernel's -- for instance
// one that ignores sliding-window layers -- is what broke the FlashAttention
// split-KV combine in vLLM PR #52816's review thread, prhub summary, "review
// highlights" and "risks".)
//
// Work model.  A request r with n > 0 queries and G = Hq/Hkv q-heads per
// kv-head has n*G query rows per kv-head, numbered row = i*G + j (block query
// i, head j of the group).  Rows are cut into groups of at most `rmax`.  A
// *unit* is (request, kv-head, row group); all of its rows see keys drawn from
// the request's union key range [lo, T): lo is the first query's window start
// (0 without a window), rounded down to a multiple of the tile size `tk`.  The
// range is cut into ceil((T - lo)/tk) tiles.  Units are laid out request by
// request, kv-head-major inside a request, and every workgroup w of the P
// attention workgroups takes the tiles [w*tpw, (w+1)*tpw) of that flat order,
// tpw = ceil(total/P).  A unit whose tiles all fall to one workgroup is
// finished there; otherwise every workgroup that touched it leaves a partial
// (normalised output + log2-sum-exp) in one of its two slots:
//     slot 0 -- the unit was the first one in the workgroup's run,
//     slot 1 -- the unit was the last one (and not also the first).
// Units strictly inside a run are always whole.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DFL_HD __host__ __device__ __forceinline__
#else
#define DFL_HD inline
#endif

namespace dflash {

struct Decomp {
    int32_t B;       // requests
    int32_t Hkv;     // kv-heads
    int32_t G;       // q-heads per kv-head
    int32_t window;  // <= 0: none
    int32_t rmax;    // rows per unit (row group size)
    int32_t tk;      // keys per tile
    int32_t P;       // attention workgroups
};

struct ReqGeom {
    int32_t kv_lo;    // first key of tile 0 (multiple of tk)
    int32_t T;        // keys of the request (L + n)
    int32_t ntiles;   // tiles per unit
    int32_t ngroups;  // row groups per kv-head
};

DFL_HD ReqGeom req_geom(int32_t L, int32_t n, const Decomp& d)
{
    ReqGeom g;
    g.T = L + n;
    if (n <= 0) {
        g.kv_lo = 0;
        g.ntiles = 0;
        g.ngroups = 0;
        return g;
    }
    int32_t lo = 0;
    if (d.window > 0) {
        lo = L - d.window + 1;  // window start of the block's first query (position L)
        if (lo < 0)
            lo = 0;
    }
    lo = (lo / d.tk) * d.tk;
    g.kv_lo = lo;
    g.ntiles = (g.T - lo + d.tk - 1) / d.tk;
    g.ngroups = (n * d.G + d.rmax - 1) / d.rmax;
    return g;
}

// Tiles of all units of one request.
DFL_HD int64_t req_work(const ReqGeom& g, const Decomp& d)
{
    return (int64_t)d.Hkv * g.ngroups * g.ntiles;
}

DFL_HD int64_t tiles_per_wg(int64_t total, int32_t P)
{
    return (total + P - 1) / P;
}

// Visible key range of one query row (inclusive), independent of tiling.
DFL_HD void query_range(int32_t L, int32_t n, int32_t i, bool causal, int32_t window, int32_t& lo, int32_t& hi)
{
    const int32_t p = L + i;
    hi = causal ? p : L + n - 1;
    lo = 0;
    if (window > 0) {
        lo = p - window + 1;
        if (lo < 0)
            lo = 0;
    }
}

// High end of a causal row's range once bidirectional spans are applied: a
// query at position p inside a span [s, e) also sees the span's later keys
// (the mm-prefix case -- a multimodal prefix is attended as a whole while
// text stays causal; kenforever1 "DFlash + Gemma 4 31B-it" notes, section on
// MooreThreads/vllm-musa PR #52).  The request's spans are entries
// offs[r] .. offs[r+1]-1 of `spans` ((start, end) pairs); entries outside
// [0, num_spans) are ignored, and the result never passes T - 1.  Any order
// and any overlap give the same answer: the largest end among the spans that
// hold p.
DFL_HD int32_t span_high(const int32_t* offs, const int32_t* spans, int32_t num_spans, int32_t r, int32_t p,
                         int32_t T, int32_t hi)
{
    int32_t w0 = offs[r], w1 = offs[r + 1];
    w0 = w0 < 0 ? 0 : w0;
    w1 = w1 > num_spans ? num_spans : w1;
    for (int32_t w = w0; w < w1; ++w) {
        const int32_t s = spans[2 * w], e = spans[2 * w + 1];
        if (s <= p && p < e && e - 1 > hi)
            hi = e - 1;
    }
    return hi < T - 1 ? hi : T - 1;
}

}  // namespace dflash
