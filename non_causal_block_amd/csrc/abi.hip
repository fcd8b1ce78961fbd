// abi.hip -- the C ABI: host validation, planning and kernel launch.
//
// The operation and its arguments are described in include/dflash_block_attn.h.
// Host-checkable mistakes are rejected before anything is enqueued and the
// library never silently runs a different mask: a backend that cannot honour
// the non-causal block must refuse it (kenforever1 "DFlash + Gemma 4 31B-it"
// notes, "why non-causal attention is needed"; vLLM PR #43445 report, "key
// code", the non-causal assertion and its message).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dflash_block_attn.h"
#include "decomp.h"
#include "kernels.h"
#include "merge.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Debug checks of device-side values: off unless DFLASH_DEBUG_CHECKS=1 in the
// environment at the first call, or switched by dflash_set_debug_checks.
std::atomic<int> g_debug_checks{-1};

bool debug_checks_on()
{
    int v = g_debug_checks.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("DFLASH_DEBUG_CHECKS");
        const int want = (e && e[0] == '1') ? 1 : 0;
        int expected = -1;
        g_debug_checks.compare_exchange_strong(expected, want);
        v = g_debug_checks.load(std::memory_order_relaxed);
    }
    return v == 1;
}

// The debug state word of the current device when checks are on, else nullptr.
int debug_state(uint32_t** out)
{
    *out = nullptr;
    if (!debug_checks_on())
        return DFLASH_OK;
    if (dflash::debug_state_ptr(out) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "debug checks: cannot locate the device state word");
    return DFLASH_OK;
}

int ilog2(int64_t x)
{
    int s = 0;
    while ((int64_t(1) << s) < x)
        ++s;
    return s;
}

// Compute-unit count per device, queried once per device.
constexpr int kMaxDevices = 64;
std::mutex g_cu_mu;
int g_cu_count[kMaxDevices] = {0};

int device_cus(int* out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(DFLASH_ERR_HIP, "no current HIP device to plan for (set desc->num_cus to plan without one)");
    if (dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_cu_mu);
        if (g_cu_count[dev] > 0) {
            *out = g_cu_count[dev];
            return DFLASH_OK;
        }
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return fail(DFLASH_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed on device %d", dev);
    if (dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_cu_mu);
        g_cu_count[dev] = cus;
    }
    *out = cus;
    return DFLASH_OK;
}

// Fewest key tiles per attention workgroup for the reference kernel and for steps
// above the small-step bound below: a workgroup walks its tiles one after another,
// so short runs (and a combine over more pieces) finish soonest; large steps fill
// the chip long before this bound matters.
constexpr int kMinTilesPerWg = 2;
// Set-up charge of a unit in the work split (decomp.h), in tiles: what one more
// unit in a run costs the MFMA kernel (queries and first pages in, output or
// partial out -- about 3.5 tiles' time at head_dim 512 and 80 rows, measured).
// Runs shorter than kChargeMinTiles tiles are latency-bound: a second unit in one
// of them doubles that workgroup's time, so they get a charge of 2, which keeps
// a two- or three-tile run from reaching into the next unit's real tiles (a draft
// step of one request, head_dim 128: attention 12.9 -> 11.3 us; 0 and 1 measured
// slower).
constexpr int kSegmentCharge = 3;
constexpr int kSegmentChargeShort = 2;
// Five row tiles at head_dim 512 (72-80 rows per unit): set-up plus epilogue take about
// 3.6 tiles' time (4.2 + 4.5 us against 2.44 us per tile), so a charge of 4 balances the
// runs that cross into a second unit.  The B = 4 x 9 global layer's call measured 1-2 us
// faster with it in five A/B runs (0.8-2.0 us), 5 was level with 3, and the B = 8 x 9
// global verify layer was level; at four row tiles (about 3.1 tiles of set-up) 3 stays.
constexpr int kSegmentChargeWide = 4;
constexpr int kChargeMinTiles = 16;
constexpr size_t kAlign = 256;
// Largest grid the automatic choice always merges split units in (besides the small steps
// below, this matters for forced grids): a small draft step is launch
// bound, and merging in the attention kernel saves the second launch (C1's step: 18.4 ->
// 16.7 us per call); larger grids pay more for the in-kernel merge's coherent publish and
// waits than for a second kernel (C2 48.7 vs 60.0 us, C3 138.7 vs 147.4 us; A/B on one box).
constexpr int kMergeInKernelAutoWgs = 64;
// A step at head_dim <= 256 whose work -- key tiles plus every unit's set-up charge --
// comes to at most this many tiles per compute unit is latency-bound (a draft step: a
// few requests, short contexts).  The automatic choice merges its split units inside the
// attention kernel: with runs of one to three tiles a second launch costs more than the
// coherent merge.  Where kMinTilesPerWg would give it more than kMergeInKernelAutoWgs
// workgroups, it runs one per CU instead.  Measured per call (block append + attention,
// GPU time, two boxes) against kMinTilesPerWg's grid and the combine kernel: head_dim 128
// with 4 and 8 requests of 512 context keys 18.7-20.9 -> 17.7-20.0 and 18.9-21.5 ->
// 16.3-19.0 us; head_dim 256, one request of 2.6K keys, 21.6-23.8 -> 21.0-23.3 us.  With
// 1 or 2 requests kMinTilesPerWg gives at most 64 workgroups, which measured as fast as
// one per CU or up to 0.5 us faster.  At head_dim 512 the in-kernel merge is slower even
// for small steps (one request of 2048 keys: 33.7 -> 39.9 us), so those keep the
// general rule.
constexpr int kSmallStepTilesPerWg = 3;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

#ifdef DFLASH_TIMELINE
// Timeline build: the caller's stamp buffer (dflash_timeline_set_buffer), used by the
// MFMA attention kernel of every later call whose grid it holds (8 words per workgroup).
std::mutex g_timeline_mu;
uint64_t* g_timeline = nullptr;
size_t g_timeline_bytes = 0;

uint64_t* timeline_buffer(int64_t P)
{
    std::lock_guard<std::mutex> lk(g_timeline_mu);
    return g_timeline && g_timeline_bytes >= (size_t)P * 8 * sizeof(uint64_t) ? g_timeline : nullptr;
}
#endif

struct Plan {
    int kernel = 0;
    int P = 0;
    int tk = 0;
    int rmax = 0;
    int row_tiles = 0;
    int Dp = 0;
    int combine_wgs = 0;
    int combine_pps = 16;  // partial rows each combine lane requests together
    int combine_lpr = 64;  // combine lanes per output row
    bool combine_rows = false;  // one output row per combine workgroup, pieces over its waves
    bool merge_in_kernel = false;  // the MFMA kernel merges split units itself (no combine launch)
    int ov = 0;
    size_t ctr_bytes = 0;  // merge counters at the start of the workspace
    size_t off_o = 0;
    size_t off_lse = 0;
    size_t off_dir = 0;  // merge directory (MFMA kernel), 0 = none
    bool use_dir = false;  // the attention kernel writes it for the rows-per-wave combine
    size_t ws_bytes = 0;
    bool empty = false;
};

int check_shape(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim)
{
    if (n_heads < 1 || n_kv_heads < 1)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "n_heads (%d) and n_kv_heads (%d) must be >= 1", n_heads, n_kv_heads);
    if (n_heads % n_kv_heads != 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "n_heads (%d) must be a multiple of n_kv_heads (%d)", n_heads,
                    n_kv_heads);
    if (head_dim <= 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "head_dim (%d) must be positive", head_dim);
    if (head_dim > 512)
        return fail(DFLASH_ERR_UNSUPPORTED, "head_dim %d > 512 is not supported (head_size <= 512)", head_dim);
    if (head_dim % 8 != 0)
        return fail(DFLASH_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 8", head_dim);
    return DFLASH_OK;
}

int make_plan(const dflash_batch_desc* desc, int32_t Hq, int32_t Hkv, int32_t D, Plan* p)
{
    if (!desc)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "desc is NULL");
    int st = check_shape(Hq, Hkv, D);
    if (st != DFLASH_OK)
        return st;
    if (desc->num_reqs < 0 || desc->total_q < 0 || desc->max_block_len < 0 || desc->total_kv_len < 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "negative count in desc (num_reqs %d, total_q %d, max_block_len %d)",
                    desc->num_reqs, desc->total_q, desc->max_block_len);
    if (!is_pow2(desc->page_size) || desc->page_size > 1024)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two in [1, 1024]", desc->page_size);
    if (desc->max_pages_per_req < 1)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "max_pages_per_req %d must be >= 1", desc->max_pages_per_req);
    if (desc->num_pages < 1)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "num_pages %lld must be >= 1", (long long)desc->num_pages);
    // one page of one of k_pages / v_pages is addressed with 32-bit element offsets
    if ((int64_t)desc->page_size * Hkv * D >= ((int64_t)1 << 31))
        return fail(DFLASH_ERR_UNSUPPORTED, "page_size * n_kv_heads * head_dim = %lld elements per page; must be < 2^31",
                    (long long)desc->page_size * Hkv * D);
    if (desc->kernel < DFLASH_KERNEL_AUTO || desc->kernel > DFLASH_KERNEL_MFMA)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "unknown kernel selector %d", desc->kernel);
    if (desc->num_workgroups < 0 || desc->num_cus < 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "num_workgroups / num_cus must be >= 0");
    if (desc->merge_mode < DFLASH_MERGE_AUTO || desc->merge_mode > DFLASH_MERGE_IN_KERNEL)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "unknown merge_mode %d", desc->merge_mode);

    *p = Plan();
    if (desc->num_reqs == 0 || desc->total_q == 0) {
        p->empty = true;
        return DFLASH_OK;
    }
    const int32_t G = Hq / Hkv;
    const int kernel = desc->kernel == DFLASH_KERNEL_AUTO ? DFLASH_KERNEL_MFMA : desc->kernel;
    int occ = 1;
    if (kernel == DFLASH_KERNEL_MFMA) {
        p->Dp = D <= 128 ? 128 : (D <= 256 ? 256 : 512);
        p->tk = dflash::mfma_tile_keys();
        const int rt_max = dflash::mfma_max_row_tiles(p->Dp);
        int rt = rt_max;
        if (desc->max_block_len > 0) {
            const int64_t rows = (int64_t)desc->max_block_len * G;
            rt = (int)std::min<int64_t>(rt_max, (rows + 15) / 16);
        }
        p->row_tiles = rt;
        p->rmax = 16 * rt;
    } else {
        p->Dp = D;
        p->tk = dflash::ref_tile_keys();
        p->rmax = dflash::ref_rows_per_unit();
        p->row_tiles = 0;
    }
    p->kernel = kernel;

    int cus = desc->num_cus;
    if (cus == 0) {
        st = device_cus(&cus);
        if (st != DFLASH_OK)
            return st;
        // resident workgroups per CU of the chosen kernel on this device
        const int q = kernel == DFLASH_KERNEL_MFMA ? dflash::mfma_wgs_per_cu(p->Dp, p->row_tiles, D == p->Dp)
                                                   : dflash::ref_wgs_per_cu();
        if (q > 0)
            occ = q;
    }
    int64_t P = (int64_t)cus * occ;
    bool small_step = false;
    if (desc->total_kv_len > 0) {
        const int64_t B = desc->num_reqs;
        const int64_t keys = desc->total_kv_len;
        int64_t groups = 1;
        if (desc->max_block_len > 0)
            groups = ((int64_t)desc->max_block_len * G + p->rmax - 1) / p->rmax;
        const int64_t tiles = (int64_t)Hkv * groups * (keys / p->tk + B);
        P = std::min<int64_t>(P, std::max<int64_t>(1, (tiles + kMinTilesPerWg - 1) / kMinTilesPerWg));
        const int64_t work = tiles + (int64_t)Hkv * groups * B * kSegmentChargeShort;
        small_step = kernel == DFLASH_KERNEL_MFMA && p->Dp <= 256 && work <= (int64_t)kSmallStepTilesPerWg * cus;
        if (small_step && P > kMergeInKernelAutoWgs)
            P = cus;
    }
    if (desc->num_workgroups > 0)
        P = desc->num_workgroups;
    if (P > (1 << 20))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "num_workgroups %lld too large", (long long)P);
    p->P = (int)P;
    if (kernel == DFLASH_KERNEL_MFMA && desc->total_kv_len > 0) {
        int64_t groups = 1;
        if (desc->max_block_len > 0)
            groups = ((int64_t)desc->max_block_len * G + p->rmax - 1) / p->rmax;
        const int64_t tiles = (int64_t)Hkv * groups * (desc->total_kv_len / p->tk);
        p->ov = tiles >= (int64_t)kChargeMinTiles * P ? kSegmentCharge : kSegmentChargeShort;
        if (p->ov == kSegmentCharge && p->row_tiles == 5 && p->Dp == 512)
            p->ov = kSegmentChargeWide;
    }
    if (p->P > 1) {
        // [merge counters, a fixed layout for every grid (merge.h)]
        // [bf16 partials [P][2][rmax][Dp]] [fp32 log-sum-exps [P][2][rmax]]
        const bool want = desc->merge_mode == DFLASH_MERGE_IN_KERNEL ||
                          (desc->merge_mode == DFLASH_MERGE_AUTO && (small_step || p->P <= kMergeInKernelAutoWgs));
        p->merge_in_kernel = kernel == DFLASH_KERNEL_MFMA && want && p->P <= dflash::kMergeMaxWgs;
        p->ctr_bytes = align_up((size_t)dflash::kCtrWords * sizeof(int32_t));
        const size_t o_bytes = (size_t)p->P * 2 * p->rmax * p->Dp * sizeof(uint16_t);
        p->off_o = p->ctr_bytes;
        p->off_lse = p->off_o + align_up(o_bytes);
        p->ws_bytes = p->off_lse + align_up((size_t)p->P * 2 * p->rmax * sizeof(float));
        if (kernel == DFLASH_KERNEL_MFMA) {
            // [merge directory: one 8-byte entry per output row, written by the attention
            // kernel for the combine kernel; present whatever the merge mode, so the
            // workspace size does not depend on it]
            p->off_dir = p->ws_bytes;
            p->ws_bytes = p->off_dir + align_up((size_t)desc->total_q * Hq * 8);
        }
        if (p->merge_in_kernel)
            return DFLASH_OK;
        p->combine_lpr = kernel == DFLASH_KERNEL_MFMA ? dflash::combine_lanes_per_row(p->Dp, Hq) : 64;
        p->combine_wgs = dflash::combine_grid((int64_t)desc->total_q * Hq, p->combine_lpr);
        // Expected pieces per split unit: the runs over the units, plus the two that
        // straddle each unit's ends.  Few pieces and many output rows want the lean
        // combine (more resident waves); many pieces want all rows in one round.
        int64_t units = (int64_t)desc->num_reqs * Hkv;
        if (desc->max_block_len > 0)
            units *= ((int64_t)desc->max_block_len * G + p->rmax - 1) / p->rmax;
        const int64_t pieces = P / std::max<int64_t>(1, units) + 2;
        p->combine_pps = pieces <= 4 ? 4 : pieces <= 8 ? 8 : 16;
        // Units split more ways than one wave requests in one round (head_dim 512 at long
        // contexts): a workgroup per output row, its four waves taking every fourth piece.
        const int64_t rows = (int64_t)desc->total_q * Hq;
        if (p->combine_lpr == 64 && pieces > 16 && rows <= 0x7fffffff) {
            p->combine_rows = true;
            p->combine_wgs = (int)rows;
        }
        // The combine finds each row's pieces in the merge directory: one load instead of a
        // pass over the request arrays, a reload of the row's lengths and the work-split
        // arithmetic (calls, A/B on one box: the causal window-1024 workload of 16 x 16
        // queries 43.8 -> 42.0 us, B = 8 x 9 at L ~ U[1024, 4096] 46.9 -> 46.3 us, the
        // head_dim-512 global layer at B = 4 x 9 128.1 -> 126.6 us).
        p->use_dir = p->off_dir != 0;
    }
    return DFLASH_OK;
}

// A validated attention call: the plan and the kernel arguments.
struct AttnCall {
    Plan plan;
    dflash::AttnArgs args;
    dflash::ValidateArgs check;  // used when args.dbg is set
};

dflash::ValidateArgs validate_args(const int32_t* page_table, const int32_t* ctx_lens, const int32_t* block_lens,
                                   const int32_t* span_offsets, int32_t num_spans, int32_t window, int32_t tile_keys,
                                   bool from_block, const dflash_batch_desc* desc, uint32_t* state)
{
    dflash::ValidateArgs v;
    v.page_table = page_table;
    v.ctx_lens = ctx_lens;
    v.block_lens = block_lens;
    v.span_offsets = span_offsets;
    v.B = desc->num_reqs;
    v.page_size = desc->page_size;
    v.max_pages_per_req = desc->max_pages_per_req;
    v.window = window;
    v.tile_keys = tile_keys > 0 ? tile_keys : 1;
    v.from_block = from_block ? 1 : 0;
    v.num_pages = desc->num_pages;
    v.total_q = desc->total_q;
    v.max_block_len = desc->max_block_len;
    v.num_spans = span_offsets ? num_spans : 0;
    v.total_kv_len = desc->total_kv_len;
    v.state = state;
    return v;
}

int attn_prepare(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                 const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads, int32_t n_kv_heads,
                 int32_t head_dim, const uint8_t* causal, const int32_t* span_offsets, const int32_t* spans,
                 int32_t num_spans, int32_t window, float scale, void* out, const dflash_batch_desc* desc,
                 AttnCall* call)
{
    Plan& p = call->plan;
    int st = make_plan(desc, n_heads, n_kv_heads, head_dim, &p);
    if (st != DFLASH_OK)
        return st;
    if (!std::isfinite(scale))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (span_offsets) {
        if (num_spans < 0)
            return fail(DFLASH_ERR_INVALID_ARGUMENT, "num_spans %d must be >= 0", num_spans);
        if (num_spans > 0 && !spans)
            return fail(DFLASH_ERR_INVALID_ARGUMENT, "spans is NULL with num_spans %d", num_spans);
        if ((reinterpret_cast<uintptr_t>(span_offsets) & 3u) || (reinterpret_cast<uintptr_t>(spans) & 3u))
            return fail(DFLASH_ERR_INVALID_ARGUMENT, "span_offsets and spans must be 4-byte aligned");
    }
    if (p.empty)
        return DFLASH_OK;
    if (!q || !k_pages || !v_pages || !page_table || !ctx_lens || !block_lens || !out)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "NULL device pointer (q %p, k_pages %p, v_pages %p, page_table %p, "
                    "ctx_lens %p, block_lens %p, out %p)", q, k_pages, v_pages, page_table, ctx_lens, block_lens, out);
    auto mis16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) != 0; };
    if (mis16(q) || mis16(k_pages) || mis16(v_pages) || mis16(out))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "q, k_pages, v_pages and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(page_table) & 3u) || (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(block_lens) & 3u))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "page_table, ctx_lens and block_lens must be 4-byte aligned");
    if (p.ws_bytes > 0) {
        if (!desc->workspace || desc->workspace_bytes < p.ws_bytes)
            return fail(DFLASH_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes at %p; this call needs %zu bytes",
                        desc->workspace_bytes, desc->workspace, p.ws_bytes);
        if (reinterpret_cast<uintptr_t>(desc->workspace) % kAlign)
            return fail(DFLASH_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kAlign);
    }

    dflash::AttnArgs& a = call->args;
    a.q = static_cast<const uint16_t*>(q);
    a.k_pages = static_cast<const uint16_t*>(k_pages);
    a.v_pages = static_cast<const uint16_t*>(v_pages);
    a.page_table = page_table;
    a.ctx_lens = ctx_lens;
    a.block_lens = block_lens;
    a.causal = causal;
    a.span_offsets = span_offsets;
    a.spans = span_offsets ? spans : nullptr;
    a.num_spans = span_offsets ? num_spans : 0;
    a.out = static_cast<uint16_t*>(out);
    char* ws = static_cast<char*>(desc->workspace);
    a.part_o = p.ws_bytes ? reinterpret_cast<uint16_t*>(ws + p.off_o) : nullptr;
    a.part_lse = p.ws_bytes ? reinterpret_cast<float*>(ws + p.off_lse) : nullptr;
    a.ctr = p.merge_in_kernel ? reinterpret_cast<uint32_t*>(ws) : nullptr;
    a.dir = p.use_dir ? reinterpret_cast<uint2*>(ws + p.off_dir) : nullptr;
    a.total_rows = (int64_t)desc->total_q * n_heads;
    a.k_new = a.v_new = nullptr;  // set by dflash_block_attn_append for the fused launch
    a.k_dst = a.v_dst = nullptr;
    a.app_dk = a.app_dv = 0;
    a.d.B = desc->num_reqs;
    a.d.Hkv = n_kv_heads;
    a.d.G = n_heads / n_kv_heads;
    a.d.window = window;
    a.d.rmax = p.rmax;
    a.d.tk = p.tk;
    a.d.P = p.P;
    a.d.ov = p.ov;
    a.Hq = n_heads;
    a.D = head_dim;
    a.Dp = p.Dp;
    a.page_shift = ilog2(desc->page_size);
    a.max_pages_per_req = desc->max_pages_per_req;
    a.scale_log2 = scale * 1.4426950408889634f;
    uint32_t* dbg = nullptr;
    st = debug_state(&dbg);
    if (st != DFLASH_OK)
        return st;
    a.dbg = dbg;
#ifdef DFLASH_TIMELINE
    a.timeline = timeline_buffer(p.P);
#endif
    if (dbg)
        call->check = validate_args(page_table, ctx_lens, block_lens, span_offsets, num_spans, window, p.tk, false,
                                    desc, dbg);
    return DFLASH_OK;
}

int attn_launch(const AttnCall& call, const dflash_batch_desc* desc, hipStream_t s, bool validate = true,
                bool fused_append = false)
{
    const Plan& p = call.plan;
    const dflash::AttnArgs& a = call.args;
    if (a.dbg && validate) {
        const hipError_t ev = dflash::launch_validate(call.check, s);
        if (ev != hipSuccess)
            return fail(DFLASH_ERR_HIP, "debug-check kernel launch failed: %s", hipGetErrorString(ev));
    }
    if (desc->event_attn_begin && hipEventRecord(static_cast<hipEvent_t>(desc->event_attn_begin), s) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "hipEventRecord(event_attn_begin) failed");
    hipError_t e = fused_append ? dflash::launch_attn_mfma_append(a, p.Dp, p.row_tiles, s)
                   : p.kernel == DFLASH_KERNEL_MFMA ? dflash::launch_attn_mfma(a, p.Dp, p.row_tiles, s)
                                                    : dflash::launch_attn_ref(a, s);
    if (e != hipSuccess)
        return fail(DFLASH_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
    if (desc->event_attn_end && hipEventRecord(static_cast<hipEvent_t>(desc->event_attn_end), s) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "hipEventRecord(event_attn_end) failed");
    if (p.combine_wgs > 0) {
        dflash::CombineArgs c;
        c.ctx_lens = a.ctx_lens;
        c.block_lens = a.block_lens;
        c.part_o = a.part_o;
        c.part_lse = a.part_lse;
        c.dir = a.dir;
        c.out = a.out;
        c.d = a.d;
        c.Hq = a.Hq;
        c.D = a.D;
        c.Dp = p.Dp;
        c.total_rows = (int64_t)desc->total_q * a.Hq;
        c.dbg = a.dbg;
        e = p.combine_rows ? dflash::launch_combine_rows(c, s)
                           : dflash::launch_combine(c, p.combine_wgs, p.combine_pps, p.combine_lpr, s);
        if (e != hipSuccess)
            return fail(DFLASH_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
    }
    return DFLASH_OK;
}

int append_prepare(const void* k_new, const void* v_new, void* k_pages, void* v_pages, const int32_t* page_table,
                   const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_kv_heads, int32_t head_dim,
                   const dflash_batch_desc* desc, dflash::AppendArgs* a)
{
    if (!desc)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "desc is NULL");
    int st = check_shape(n_kv_heads, n_kv_heads, head_dim);
    if (st != DFLASH_OK)
        return st;
    if (desc->num_reqs < 0 || desc->total_q < 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "negative count in desc (num_reqs %d, total_q %d)", desc->num_reqs,
                    desc->total_q);
    if (!is_pow2(desc->page_size) || desc->page_size > 1024)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "page_size %d must be a power of two in [1, 1024]", desc->page_size);
    if (desc->max_pages_per_req < 1)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "max_pages_per_req %d must be >= 1", desc->max_pages_per_req);
    a->total_rows = (desc->num_reqs == 0) ? 0 : (int64_t)desc->total_q * n_kv_heads;
    if (a->total_rows == 0)
        return DFLASH_OK;
    if (!k_new || !v_new || !k_pages || !v_pages || !page_table || !ctx_lens || !block_lens)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "NULL device pointer (k_new %p, v_new %p, k_pages %p, v_pages %p, "
                    "page_table %p, ctx_lens %p, block_lens %p)", k_new, v_new, k_pages, v_pages, page_table,
                    ctx_lens, block_lens);
    auto mis16 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) != 0; };
    if (mis16(k_new) || mis16(v_new) || mis16(k_pages) || mis16(v_pages))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "k_new, v_new, k_pages and v_pages must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(page_table) & 3u) || (reinterpret_cast<uintptr_t>(ctx_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(block_lens) & 3u))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "page_table, ctx_lens and block_lens must be 4-byte aligned");
    a->k_new = static_cast<const uint16_t*>(k_new);
    a->v_new = static_cast<const uint16_t*>(v_new);
    a->k_pages = static_cast<uint16_t*>(k_pages);
    a->v_pages = static_cast<uint16_t*>(v_pages);
    a->page_table = page_table;
    a->ctx_lens = ctx_lens;
    a->block_lens = block_lens;
    a->B = desc->num_reqs;
    a->Hkv = n_kv_heads;
    a->D = head_dim;
    a->page_shift = ilog2(desc->page_size);
    a->max_pages_per_req = desc->max_pages_per_req;
    uint32_t* dbg = nullptr;
    st = debug_state(&dbg);
    if (st != DFLASH_OK)
        return st;
    a->dbg = dbg;
    return DFLASH_OK;
}

}  // namespace

namespace dflash {

// The thread's last-error text, for entry points in other translation units.
int set_last_error(int status, const char* msg)
{
    return fail(status, "%s", msg);
}

}  // namespace dflash

extern "C" {

int dflash_abi_version(void) { return DFLASH_ABI_VERSION; }

#ifdef DFLASH_TIMELINE
int dflash_timeline_set_buffer(void* buf, size_t bytes)
{
    if ((buf == nullptr) != (bytes == 0) || reinterpret_cast<uintptr_t>(buf) % 8)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "timeline buffer: NULL with 0 bytes, or 8-byte aligned with > 0");
    std::lock_guard<std::mutex> lk(g_timeline_mu);
    g_timeline = static_cast<uint64_t*>(buf);
    g_timeline_bytes = bytes;
    return DFLASH_OK;
}
#endif

int dflash_block_conv(const void* x, const void* base, const void* delta, const int32_t* block_lens,
                       int32_t num_reqs, int32_t total_q, int32_t channels, int32_t groups, int32_t taps, void* out,
                       void* stream)
{
    if (num_reqs < 0 || total_q < 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: negative num_reqs (%d) or total_q (%d)", num_reqs, total_q);
    if (total_q > 65535)
        return fail(DFLASH_ERR_UNSUPPORTED, "block_conv: total_q %d > 65535 (one grid row per position)", total_q);
    if (channels < 2 || channels % 2 != 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: channels (%d) must be even and >= 2", channels);
    if (groups < 1 || channels % groups != 0)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: groups (%d) must divide channels (%d)", groups, channels);
    if (taps < 1 || taps > 1024)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: taps (%d) must be in [1, 1024]", taps);
    if (num_reqs == 0 || total_q == 0)
        return DFLASH_OK;
    if (!x || !base || !delta || !block_lens || !out)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: NULL device pointer");
    if ((reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(base) & 3u) ||
        (reinterpret_cast<uintptr_t>(out) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 1u) ||
        (reinterpret_cast<uintptr_t>(block_lens) & 3u))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "block_conv: x, base, out and block_lens must be 4-byte aligned, "
                    "delta 2-byte aligned");
    dflash::ConvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.base = static_cast<const uint16_t*>(base);
    a.delta = static_cast<const uint16_t*>(delta);
    a.block_lens = block_lens;
    a.out = static_cast<uint16_t*>(out);
    a.B = num_reqs;
    a.C = channels;
    a.G = groups;
    a.taps = taps;
    a.total_rows = total_q;
    const hipError_t e = dflash::launch_block_conv(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DFLASH_ERR_HIP, "block_conv launch failed: %s", hipGetErrorString(e));
    return DFLASH_OK;
}

int dflash_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream)
{
    if (bytes == 0)
        return DFLASH_OK;
    if (!buf || !sink)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "stream_read: buf and sink must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "stream_read: buf and bytes must be 16-byte multiples, sink 4-byte aligned");
    int cus = 0;
    const int st = device_cus(&cus);
    if (st != DFLASH_OK)
        return st;
    // four workgroups per compute unit keep enough 16-byte loads in flight
    const int64_t need = (int64_t)((bytes / 16 + 255) / 256);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(need, (int64_t)cus * 4));
    const hipError_t e = dflash::launch_stream_read(buf, bytes, sink, grid, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DFLASH_ERR_HIP, "stream_read launch failed: %s", hipGetErrorString(e));
    return DFLASH_OK;
}

const char* dflash_status_string(int status)
{
    switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported";
    case DFLASH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DFLASH_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char* dflash_last_error_message(void) { return g_last_error; }

int dflash_set_debug_checks(int on)
{
    const int prev = debug_checks_on() ? 1 : 0;
    g_debug_checks.store(on ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

int dflash_debug_checks_result(uint32_t* bits, int32_t* first_request)
{
    if (!bits || !first_request)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "debug checks: bits and first_request must be non-NULL");
    uint32_t* p = nullptr;
    if (dflash::debug_state_ptr(&p) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "debug checks: cannot locate the device state word");
    if (hipDeviceSynchronize() != hipSuccess)
        return fail(DFLASH_ERR_HIP, "debug checks: hipDeviceSynchronize failed");
    uint32_t host[2] = {0, 0};
    if (hipMemcpy(host, p, sizeof host, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "debug checks: reading the state word failed");
    const uint32_t clear[2] = {0u, 0x7fffffffu};
    if (hipMemcpy(p, clear, sizeof clear, hipMemcpyHostToDevice) != hipSuccess)
        return fail(DFLASH_ERR_HIP, "debug checks: clearing the state word failed");
    *bits = host[0];
    *first_request = host[0] ? (int32_t)host[1] : -1;
    return DFLASH_OK;
}

int dflash_block_attn_supports(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim)
{
    char saved[sizeof g_last_error];
    memcpy(saved, g_last_error, sizeof saved);
    const int ok = check_shape(n_heads, n_kv_heads, head_dim) == DFLASH_OK;
    memcpy(g_last_error, saved, sizeof saved);
    return ok ? 1 : 0;
}

int dflash_block_attn_workspace_size(const dflash_batch_desc* desc, int32_t n_heads, int32_t n_kv_heads,
                                     int32_t head_dim, size_t* bytes)
{
    if (!bytes)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "bytes is NULL");
    Plan p;
    const int st = make_plan(desc, n_heads, n_kv_heads, head_dim, &p);
    if (st != DFLASH_OK)
        return st;
    *bytes = p.ws_bytes;
    return DFLASH_OK;
}

int dflash_block_attn_plan(const dflash_batch_desc* desc, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                           dflash_plan_info* info)
{
    if (!info)
        return fail(DFLASH_ERR_INVALID_ARGUMENT, "plan is NULL");
    Plan p;
    const int st = make_plan(desc, n_heads, n_kv_heads, head_dim, &p);
    if (st != DFLASH_OK)
        return st;
    info->kernel = p.kernel;
    info->num_workgroups = p.P;
    info->tile_keys = p.tk;
    info->rows_per_unit = p.rmax;
    info->head_dim_padded = p.Dp;
    info->combine_workgroups = p.combine_wgs;
    info->merge_in_kernel = p.merge_in_kernel ? 1 : 0;
    info->workspace_bytes = p.ws_bytes;
    return DFLASH_OK;
}

int dflash_block_attn(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                      const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads, int32_t n_kv_heads,
                      int32_t head_dim, const uint8_t* causal, int32_t window, float scale, void* out,
                      void* stream, const dflash_batch_desc* desc)
{
    AttnCall c;
    const int st = attn_prepare(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads, n_kv_heads, head_dim,
                                causal, nullptr, nullptr, 0, window, scale, out, desc, &c);
    if (st != DFLASH_OK || c.plan.empty)
        return st;
    return attn_launch(c, desc, static_cast<hipStream_t>(stream));
}

int dflash_block_attn_spans(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                            const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, const uint8_t* causal, const int32_t* span_offsets,
                            const int32_t* spans, int32_t num_spans, int32_t window, float scale, void* out,
                            void* stream, const dflash_batch_desc* desc)
{
    AttnCall c;
    const int st = attn_prepare(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads, n_kv_heads, head_dim,
                                causal, span_offsets, spans, num_spans, window, scale, out, desc, &c);
    if (st != DFLASH_OK || c.plan.empty)
        return st;
    return attn_launch(c, desc, static_cast<hipStream_t>(stream));
}

int dflash_block_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                           const int32_t* page_table, const int32_t* ctx_lens, const int32_t* block_lens,
                           int32_t n_kv_heads, int32_t head_dim, void* stream, const dflash_batch_desc* desc)
{
    dflash::AppendArgs a;
    const int st = append_prepare(k_new, v_new, k_pages, v_pages, page_table, ctx_lens, block_lens, n_kv_heads,
                                  head_dim, desc, &a);
    if (st != DFLASH_OK || a.total_rows == 0)
        return st;
    if (a.dbg) {
        const dflash::ValidateArgs v =
            validate_args(page_table, ctx_lens, block_lens, nullptr, 0, 0, 1, true, desc, const_cast<uint32_t*>(a.dbg));
        const hipError_t ev = dflash::launch_validate(v, static_cast<hipStream_t>(stream));
        if (ev != hipSuccess)
            return fail(DFLASH_ERR_HIP, "debug-check kernel launch failed: %s", hipGetErrorString(ev));
    }
    const hipError_t e = dflash::launch_kv_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DFLASH_ERR_HIP, "append kernel launch failed: %s", hipGetErrorString(e));
    return DFLASH_OK;
}

int dflash_block_attn_append(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                             const int32_t* page_table, const int32_t* ctx_lens, const int32_t* block_lens,
                             int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, const uint8_t* causal,
                             int32_t window, float scale, void* out, void* stream, const dflash_batch_desc* desc)
{
    // both halves are validated before either is enqueued
    dflash::AppendArgs ap;
    int st = append_prepare(k_new, v_new, k_pages, v_pages, page_table, ctx_lens, block_lens, n_kv_heads, head_dim,
                            desc, &ap);
    if (st != DFLASH_OK)
        return st;
    AttnCall c;
    st = attn_prepare(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads, n_kv_heads, head_dim, causal,
                      nullptr, nullptr, 0, window, scale, out, desc, &c);
    if (st != DFLASH_OK)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (ap.dbg) {
        const dflash::ValidateArgs v =
            c.plan.empty ? validate_args(page_table, ctx_lens, block_lens, nullptr, 0, 0, 1, true, desc,
                                         const_cast<uint32_t*>(ap.dbg))
                         : c.check;
        const hipError_t ev = dflash::launch_validate(v, s);
        if (ev != hipSuccess)
            return fail(DFLASH_ERR_HIP, "debug-check kernel launch failed: %s", hipGetErrorString(ev));
    }
    // The MFMA kernel with pages of >= 16 keys takes the append into its own launch: it
    // reads the block's K/V rows from k_new / v_new and writes them into the pages.
    const bool fused = !c.plan.empty && c.plan.kernel == DFLASH_KERNEL_MFMA && c.args.page_shift >= 4;
    if (fused) {
        c.args.k_new = ap.k_new;
        c.args.v_new = ap.v_new;
        c.args.k_dst = ap.k_pages;
        c.args.v_dst = ap.v_pages;
        const intptr_t dk = reinterpret_cast<intptr_t>(ap.k_new) - reinterpret_cast<intptr_t>(ap.k_pages);
        const intptr_t dv = reinterpret_cast<intptr_t>(ap.v_new) - reinterpret_cast<intptr_t>(ap.v_pages);
        c.args.app_dk = (int64_t)(dk / 2);  // all four are 16-byte aligned
        c.args.app_dv = (int64_t)((dv - dk) / 2);
        return attn_launch(c, desc, s, /*validate=*/false, /*fused_append=*/true);
    }
    if (ap.total_rows > 0) {
        const hipError_t e = dflash::launch_kv_append(ap, s);
        if (e != hipSuccess)
            return fail(DFLASH_ERR_HIP, "append kernel launch failed: %s", hipGetErrorString(e));
    }
    if (c.plan.empty)
        return DFLASH_OK;
    return attn_launch(c, desc, s, /*validate=*/false);
}

}  // extern "C"
