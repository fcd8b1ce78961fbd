// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decomp.h"

namespace dflash {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// 64-bit value broadcast/shift helpers built from 32-bit lane shuffles.
__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int delta)
{
    int lo = __shfl_up((int)(uint32_t)(uint64_t)v, delta);
    int hi = __shfl_up((int)(uint32_t)((uint64_t)v >> 32), delta);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t shfl_i64(int64_t v, int src)
{
    int lo = __shfl((int)(uint32_t)(uint64_t)v, src);
    int hi = __shfl((int)(uint32_t)((uint64_t)v >> 32), src);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int64_t t = shfl_up_i64(x, off);
        if (lane >= off)
            x += t;
    }
    return x;
}

// Work of request r (0 when r is out of range).
__device__ __forceinline__ int64_t req_work_at(const int32_t* __restrict__ ctx_lens,
                                               const int32_t* __restrict__ block_lens, int32_t r, const Decomp& d)
{
    if (r >= d.B)
        return 0;
    ReqGeom g = req_geom(ctx_lens[r], block_lens[r], d);
    return req_work(g, d);
}

// Total tiles of the call; every lane of the wave gets the same value.
__device__ __forceinline__ int64_t wave_total_work(const int32_t* __restrict__ ctx_lens,
                                                   const int32_t* __restrict__ block_lens, const Decomp& d)
{
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int32_t base = 0; base < d.B; base += 64) {
        int64_t w = req_work_at(ctx_lens, block_lens, base + lane, d);
        acc += shfl_i64(wave_inclusive_scan(w), 63);
    }
    return acc;
}

// Request containing flat tile `pos` (0 <= pos < total) and the number of tiles
// before it.  Requests with no work are skipped.  Wave-uniform result.
__device__ __forceinline__ void wave_find_request(const int32_t* __restrict__ ctx_lens,
                                                  const int32_t* __restrict__ block_lens, const Decomp& d,
                                                  int64_t pos, int32_t& r_out, int64_t& base_out)
{
    const int lane = threadIdx.x & 63;
    int64_t carry = 0;
    for (int32_t base = 0; base < d.B; base += 64) {
        int64_t w = req_work_at(ctx_lens, block_lens, base + lane, d);
        int64_t incl = wave_inclusive_scan(w) + carry;
        // first lane whose inclusive prefix exceeds pos
        unsigned long long m = __ballot(incl > pos);
        if (m) {
            int src = __ffsll((long long)m) - 1;
            r_out = base + src;
            base_out = shfl_i64(incl - w, src);
            return;
        }
        carry = shfl_i64(incl, 63);
    }
    r_out = d.B;  // not reached for pos < total
    base_out = carry;
}

// Request owning packed query token t, with its first token index.  Wave-uniform.
__device__ __forceinline__ void wave_find_token(const int32_t* __restrict__ block_lens, int32_t B, int64_t t,
                                                int32_t& r_out, int64_t& qstart_out)
{
    const int lane = threadIdx.x & 63;
    int64_t carry = 0;
    for (int32_t base = 0; base < B; base += 64) {
        int64_t n = (base + lane < B) ? (int64_t)block_lens[base + lane] : 0;
        int64_t incl = wave_inclusive_scan(n) + carry;
        unsigned long long m = __ballot(incl > t);
        if (m) {
            int src = __ffsll((long long)m) - 1;
            r_out = base + src;
            qstart_out = shfl_i64(incl - n, src);
            return;
        }
        carry = shfl_i64(incl, 63);
    }
    r_out = B;
    qstart_out = carry;
}

// Prefix of work over requests [0, r).  Wave-uniform.
__device__ __forceinline__ int64_t wave_work_before(const int32_t* __restrict__ ctx_lens,
                                                    const int32_t* __restrict__ block_lens, const Decomp& d, int32_t r)
{
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int32_t base = 0; base < r; base += 64) {
        int64_t w = (base + lane < r) ? req_work_at(ctx_lens, block_lens, base + lane, d) : 0;
        acc += shfl_i64(wave_inclusive_scan(w), 63);
    }
    return acc;
}

// First request of a workgroup's run, with what the kernels need of it.
struct RunStart {
    int32_t r;       // request holding the run's first tile
    int64_t rbase;   // flat work before request r
    int64_t qstart;  // query tokens before request r
    int32_t L, n;    // its lengths
    bool causal;     // its causal flag (false without a flag array)
};

// The run of workgroup wg: total work, its flat range [begin, end), and its first
// request.  For up to 64 requests everything, the causal flags included, comes from
// one load of the request arrays (one memory round trip before the first segment);
// larger batches take the general helpers.  When begin >= end `rs` is not set.
// qtotal: the query tokens of all requests when the run holds the last tile (end ==
// total) or there is no work at all, else -1.  Wave-uniform.
__device__ __forceinline__ void wave_locate_run(const int32_t* __restrict__ ctx_lens,
                                                const int32_t* __restrict__ block_lens,
                                                const uint8_t* __restrict__ causal, const Decomp& d, int32_t wg,
                                                int64_t& total, int64_t& begin, int64_t& end, RunStart& rs,
                                                int64_t& qtotal)
{
    const int lane = threadIdx.x & 63;
    if (d.B <= 64) {
        const bool live = lane < d.B;
        const int32_t L = live ? ctx_lens[lane] : 0;
        const int32_t n = live ? block_lens[lane] : 0;
        const int32_t c = (live && causal) ? (int32_t)causal[lane] : 0;
        const int64_t w = live ? req_work(req_geom(L, n, d), d) : 0;
        const int64_t wincl = wave_inclusive_scan(w);
        const int64_t qincl = wave_inclusive_scan((int64_t)n);
        total = shfl_i64(wincl, 63);
        const int64_t tpw = tiles_per_wg(total, d.P);
        begin = (int64_t)wg * tpw;
        end = min(total, begin + tpw);
        qtotal = (end == total || total == 0) ? shfl_i64(qincl, 63) : -1;
        if (begin >= end)
            return;
        const unsigned long long m = __ballot(wincl > begin);
        const int src = __ffsll((long long)m) - 1;
        rs.r = src;
        rs.rbase = shfl_i64(wincl - w, src);
        rs.qstart = shfl_i64(qincl - n, src);
        rs.L = __shfl(L, src);
        rs.n = __shfl(n, src);
        rs.causal = __shfl(c, src) != 0;
        return;
    }
    total = wave_total_work(ctx_lens, block_lens, d);
    const int64_t tpw = tiles_per_wg(total, d.P);
    begin = (int64_t)wg * tpw;
    end = min(total, begin + tpw);
    qtotal = -1;
    if (end == total || total == 0) {
        qtotal = 0;
        for (int32_t base = 0; base < d.B; base += 64) {
            const int64_t nn = (base + lane < d.B) ? (int64_t)block_lens[base + lane] : 0;
            qtotal += shfl_i64(wave_inclusive_scan(nn), 63);
        }
    }
    if (begin >= end)
        return;
    wave_find_request(ctx_lens, block_lens, d, begin, rs.r, rs.rbase);
    int64_t q = 0;
    for (int32_t base = 0; base < rs.r; base += 64) {
        const int64_t nn = (base + lane < rs.r) ? (int64_t)block_lens[base + lane] : 0;
        q += shfl_i64(wave_inclusive_scan(nn), 63);
    }
    rs.qstart = q;
    rs.L = ctx_lens[rs.r];
    rs.n = block_lens[rs.r];
    rs.causal = causal ? causal[rs.r] != 0 : false;
}

// One pass over the request arrays, 64 requests per step (one load round for up to
// 64 requests): the request holding packed query token t with its first token, the
// flat work before it, and the call's total work.  r_out = B for a token past the
// end.  Wave-uniform.
__device__ __forceinline__ void wave_locate_token(const int32_t* __restrict__ ctx_lens,
                                                  const int32_t* __restrict__ block_lens, const Decomp& d, int64_t t,
                                                  int32_t& r_out, int64_t& qstart_out, int64_t& wbefore_out,
                                                  int64_t& total_out)
{
    const int lane = threadIdx.x & 63;
    int64_t qcarry = 0, wcarry = 0;
    bool found = false;
    r_out = d.B;
    qstart_out = 0;
    wbefore_out = 0;
    for (int32_t base = 0; base < d.B; base += 64) {
        const int32_t r = base + lane;
        const bool live = r < d.B;
        const int32_t L = live ? ctx_lens[r] : 0;
        const int32_t n = live ? block_lens[r] : 0;
        const int64_t w = live ? req_work(req_geom(L, n, d), d) : 0;
        const int64_t qincl = wave_inclusive_scan((int64_t)n) + qcarry;
        const int64_t wincl = wave_inclusive_scan(w) + wcarry;
        const unsigned long long m = __ballot(qincl > t);
        if (!found && m) {
            const int src = __ffsll((long long)m) - 1;
            r_out = base + src;
            qstart_out = shfl_i64(qincl - n, src);
            wbefore_out = shfl_i64(wincl - w, src);
            found = true;
        }
        qcarry = shfl_i64(qincl, 63);
        wcarry = shfl_i64(wincl, 63);
    }
    total_out = wcarry;
}

// Logical workgroup index: consecutive logical indices are placed on the same XCD
// (the dispatcher deals workgroups round-robin over 8 XCDs), so the workgroups
// that share a unit share that XCD's L2 for the unit's Q rows.
__device__ __forceinline__ int32_t logical_wg(int32_t bid, int32_t P)
{
    constexpr int32_t kXcd = 8;
    if (P % kXcd != 0)
        return bid;
    return (bid % kXcd) * (P / kXcd) + bid / kXcd;
}

// Kernel arguments shared by the attention kernels.
struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k_pages;
    const uint16_t* v_pages;
    const int32_t* page_table;
    const int32_t* ctx_lens;
    const int32_t* block_lens;
    const uint8_t* causal;
    const int32_t* span_offsets;  // [B+1] or nullptr: bidirectional spans of causal requests
    const int32_t* spans;         // [num_spans][2] (start, end) key positions
    int32_t num_spans;
    uint16_t* out;
    uint16_t* part_o;  // bf16 [P][2][rmax][Dp]: normalised partial outputs
    float* part_lse;   // [P][2][rmax]
    // Counters of the in-kernel merge of split units (layout in merge.h); zero before
    // the launch and zero again after it.  nullptr: the kernel leaves the partials for
    // the combine kernel.
    uint32_t* ctr;
    // Fused block K/V append (APPEND instances only): the block's K/V rows, bf16
    // [total_q][Hkv][D] in request order; writable views of the pages; and the element
    // offsets k_new - k_pages and (v_new - v_pages) - (k_new - k_pages).
    const uint16_t* k_new;
    const uint16_t* v_new;
    uint16_t* k_dst;
    uint16_t* v_dst;
    int64_t app_dk;
    int64_t app_dv;
    Decomp d;
    int32_t Hq;
    int32_t D;         // real head_dim
    int32_t Dp;        // padded head_dim (partial row stride)
    int32_t page_shift;
    int32_t max_pages_per_req;
    float scale_log2;  // scale * log2(e)
    const uint32_t* dbg;  // debug-check state or nullptr: when it is non-zero the kernel does nothing
    // Merge directory for the combine kernel, one entry per output row (token * Hq +
    // q-head) of [0, total_rows): written in full by every launch whose partials that
    // kernel merges, nullptr otherwise.  Entry (x, y): x = first piece's workgroup kf | that
    // piece's slot << 31; y = pieces np (bits 0-23) | the row's index inside its unit << 24.
    // np = 1: the unit was finished whole (nothing to merge); np = 0: a row of no request.
    uint2* dir;
    int64_t total_rows;  // total_q hint * Hq (rows of `dir`)
#ifdef DFLASH_TIMELINE
    // Timeline build only: per-workgroup wall-clock stamps (layout in attn_mfma_kernel.h),
    // or nullptr for none.
    uint64_t* timeline;
#endif
};

// Merge-directory entries (AttnArgs::dir).
__device__ __forceinline__ uint2 dir_pack(int64_t kf, int slot0, int64_t np, int32_t rin)
{
    return make_uint2((uint32_t)kf | ((uint32_t)slot0 << 31), (uint32_t)np | ((uint32_t)rin << 24));
}

struct DirEntry {
    int64_t kf;   // first piece's workgroup
    int64_t np;   // pieces (0: no request's row, 1: finished whole)
    int slot0;    // slot of the first piece's partial (the later pieces use slot 0)
    int32_t rin;  // row inside its unit
};

__device__ __forceinline__ DirEntry dir_unpack(uint2 e)
{
    DirEntry r;
    r.kf = e.x & 0x7fffffffu;
    r.slot0 = (int)(e.x >> 31);
    r.np = e.y & 0xffffffu;
    r.rin = (int32_t)(e.y >> 24);
    return r;
}

struct CombineArgs {
    const int32_t* ctx_lens;
    const int32_t* block_lens;
    const uint16_t* part_o;  // bf16 [P][2][rmax][Dp]
    const float* part_lse;
    uint16_t* out;
    Decomp d;
    int32_t Hq;
    int32_t D;
    int32_t Dp;
    int64_t total_rows;  // total_q hint * Hq
    const uint32_t* dbg;  // as in AttnArgs
    // the attention kernel's merge directory (AttnArgs::dir), or nullptr: then each row's
    // pieces are derived from the request arrays
    const uint2* dir;
};

struct ConvArgs {
    const uint16_t* x;      // bf16 [total_q][C]
    const uint16_t* base;   // bf16 [taps][C]
    const uint16_t* delta;  // bf16 [total_q][taps][G]
    const int32_t* block_lens;
    uint16_t* out;          // bf16 [total_q][C]
    int32_t B;
    int32_t C;
    int32_t G;
    int32_t taps;
    int32_t total_rows;     // total_q (grid rows; rows past sum(block_lens) do nothing)
};

struct AppendArgs {
    const uint16_t* k_new;  // bf16 [total_q][Hkv][D], block tokens in request order
    const uint16_t* v_new;
    uint16_t* k_pages;      // bf16 [num_pages][page][Hkv][D]
    uint16_t* v_pages;
    const int32_t* page_table;
    const int32_t* ctx_lens;
    const int32_t* block_lens;
    int32_t B;
    int32_t Hkv;
    int32_t D;
    int32_t page_shift;
    int32_t max_pages_per_req;
    int64_t total_rows;  // total_q * Hkv
    const uint32_t* dbg;  // as in AttnArgs
};

// Debug checks of the device-side values a call relies on (debug_checks.hip).
struct ValidateArgs {
    const int32_t* page_table;
    const int32_t* ctx_lens;
    const int32_t* block_lens;
    const int32_t* span_offsets;  // or nullptr
    int32_t B;
    int32_t page_size;
    int32_t max_pages_per_req;
    int32_t window;         // attention window (<= 0: none); sets the first page attention reads
    int32_t tile_keys;      // key tile of the attention kernel (the first key read is a multiple)
    int32_t from_block;     // 1: only the block's own positions are touched (append alone)
    int64_t num_pages;
    int64_t total_q;        // desc->total_q
    int32_t max_block_len;  // hint (0 = none)
    int32_t num_spans;
    int64_t total_kv_len;   // hint (0 = none)
    uint32_t* state;        // [0] sticky error bits, [1] lowest failing request
};

}  // namespace dflash
