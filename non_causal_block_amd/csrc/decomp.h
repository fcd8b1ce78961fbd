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
// tpw = ceil(total/P).
//
// Set-up charge.  Starting a unit costs a workgroup more than a tile: loading
// the unit's queries and first pages, and writing its output or partial at
// the end.  A run that crosses from one unit into the next pays that twice, so
// the flat order gives every unit `ov` virtual tiles in front of its real
// ones: a unit spans uwork = ov + ntiles flat positions, virtual position v
// being real tile v - ov (none for v < ov).  A run whose part of a unit holds
// only virtual positions does nothing there.  ov = 0 is the plain split.
//
// A unit whose real tiles all fall to one workgroup is finished there;
// otherwise every workgroup that holds some of its real tiles leaves a
// partial (normalised output + log2-sum-exp) in one of its two slots:
//     slot 0 -- the unit was the first one with real tiles in the run,
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
    int32_t ov;      // virtual set-up tiles charged at the start of every unit
};

struct ReqGeom {
    int32_t kv_lo;    // first key of tile 0 (multiple of tk)
    int32_t T;        // keys of the request (L + n)
    int32_t ntiles;   // real tiles per unit
    int32_t uwork;    // flat positions per unit: ov + ntiles (0 without queries)
    int32_t ngroups;  // row groups per kv-head
};

DFL_HD ReqGeom req_geom(int32_t L, int32_t n, const Decomp& d)
{
    ReqGeom g;
    g.T = L + n;
    if (n <= 0) {
        g.kv_lo = 0;
        g.ntiles = 0;
        g.uwork = 0;
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
    g.uwork = d.ov + g.ntiles;
    g.ngroups = (n * d.G + d.rmax - 1) / d.rmax;
    return g;
}

// Flat positions of all units of one request.
DFL_HD int64_t req_work(const ReqGeom& g, const Decomp& d)
{
    return (int64_t)d.Hkv * g.ngroups * g.uwork;
}

// The part of one unit that a run [pos, end) covers, for pos inside a request
// whose flat range starts at rbase: unit index, real tiles [t0, t1) (empty
// when the part holds only virtual positions) and the flat position after it.
struct Segment {
    int32_t unit;
    int32_t t0;
    int32_t t1;
    int64_t next;
};

DFL_HD Segment run_segment(const ReqGeom& g, int64_t rbase, int64_t pos, int64_t end, int32_t ov)
{
    Segment s;
    s.unit = (int32_t)((pos - rbase) / g.uwork);
    const int64_t ustart = rbase + (int64_t)s.unit * g.uwork;
    const int64_t uend = ustart + g.uwork;
    s.next = end < uend ? end : uend;
    const int64_t v0 = pos - ustart - ov;
    const int64_t v1 = s.next - ustart - ov;
    s.t0 = (int32_t)(v0 > 0 ? v0 : 0);
    s.t1 = (int32_t)(v1 > 0 ? v1 : 0);
    return s;
}

// Workgroups [kf, kl] hold real tiles of the unit whose flat range starts at
// `us`; kf == kl means one workgroup finished it whole.
DFL_HD void unit_pieces(const ReqGeom& g, int64_t us, int32_t ov, int64_t tpw, int64_t& kf, int64_t& kl)
{
    kf = (us + ov) / tpw;
    kl = (us + g.uwork - 1) / tpw;
}

// Slot holding workgroup k's partial of the unit starting at `us`: 1 when the
// run began before the unit (it then holds real tiles of an earlier unit --
// every unit ends with a real tile), else 0.
DFL_HD int piece_slot(int64_t k, int64_t us, int64_t tpw)
{
    return k * tpw < us ? 1 : 0;
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
// query at position p inside a span [s, e) also sees the span's later keys.
// This rule is a reading: kenforever1 "DFlash + Gemma 4 31B-it" notes, section
// on MooreThreads/vllm-musa PR #52, only name the backend's mm-prefix support;
// the rule is the plainest mask in which a multimodal prefix is attended as a
// whole while text stays causal.  The request's spans are entries
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
