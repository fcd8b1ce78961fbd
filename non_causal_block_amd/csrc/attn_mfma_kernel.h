// attn_mfma_kernel.h -- the MFMA (matrix-core) block-attention kernel for gfx950.
//
// Included by attn_mfma.hip (plain masks) and attn_mfma_spans.hip (masks with
// bidirectional spans): the two sets of instances compile in parallel, and the
// span lookup costs the plain instances nothing.
//
// What it computes: kenforever1 "DFlash + Gemma 4 31B-it" notes, "why
// non-causal attention is needed" -- each request's block of 1+k queries
// attends, as a whole, to the context K/V plus the block's own K/V; the
// causal variant lets query i see only itself and keys to its left; vLLM PR
// #43445 (report, "implementation") makes causality a per-request flag and
// adds sliding-window DFlash.  Global layers need head_dim 512 (notes,
// "Gemma 4 31B-it structure").
//
// How (gfx950, wave64, 4 waves per workgroup, one wave per SIMD):
//  * Work: decomp.h -- each workgroup takes an equal run of 32-key tiles over
//    all (request, kv-head, row group) units; all G q-heads of a kv-head and
//    all n block queries share every K/V byte (rows = n*G, tiled by 16).
//  * The head dimension is split over the 4 waves (DW = Dp/4 each).  Wave w
//    streams only its d-slice of every key, 16 bytes per lane so that one load
//    covers whole slices of several keys, into registers one tile ahead, and
//    from there into wave-private LDS tiles (K swizzled for the MFMA-order
//    reads, V for the transposing reads).  V is requested apart from K; up to
//    head_dim 256 it is also staged just before the PV product, so that each
//    half of the next tile has a whole step to arrive.
//  * S^T = K Q^T per wave over its d-slice with v_mfma_f32_16x16x32_bf16
//    (A = K, rows = keys; B = Q^T, held for the whole unit); the four partial
//    S^T tiles are summed through LDS by the wave that owns the row tile, which
//    applies the mask, runs the softmax (exp2; max over lanes with
//    xor-shuffles) and publishes P^T in exactly the MFMA B-operand layout.
//  * O^T += V^T P^T per wave for its d-slice (A = V^T gathered from LDS, B =
//    P^T from LDS), fp32 accumulators in registers.
//  * No rescaling of the accumulators: a row's reference max is its first
//    visible tile's max, kept while later tiles stay within 2^32 of it (the
//    probabilities then fit bf16/fp32 comfortably).  A tile beyond that
//    (extreme logit ranges only) abandons the segment; after its run the
//    workgroup recomputes such segments with each row's exact max found by a
//    K-only pass.  Numerator and denominator share the reference, so the
//    result is the same softmax either way.
//  * Keys past the request's end are read as its last key (T - 1) instead, so
//    page-tail garbage (possibly NaN) is never loaded; their logits are masked,
//    so their weight is exactly zero.
//  * Epilogue: a unit finished inside the workgroup writes bf16 output;
//    otherwise its piece is a bf16 normalised partial + fp32 log2-sum-exp in the
//    workgroup's workspace slot.  With merge counters (AttnArgs::ctr) the pieces'
//    own workgroups merge each split unit after their runs (merge.h); without
//    them combine.hip does.
#pragma once

#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "merge.h"

namespace dflash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Waves per workgroup: the head dimension is split over them (DP / WAVES d each).
// Four, one per SIMD.  An 8-way split at head_dim 512 (two waves per SIMD, 80
// accumulators each) passes the same tests but ran about 5% slower on C3: the
// barriers keep both waves of a SIMD in the same phase, and each row-tile owner
// then sums twice as many partial products.
constexpr int waves_for(int /*dp*/) { return 4; }
template <int DP>
constexpr int threads_for = waves_for(DP) * 64;
constexpr int kTK = 32;              // keys per tile (two 16-key MFMA tiles)
constexpr float kLazyBound = 32.0f;  // log2 units a row max may exceed its reference by
constexpr int kLazy = 0, kMaxScan = 1, kFixed = 2;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p)
{
    return *reinterpret_cast<const u32x4_t*>(p);
}

// K/V rows are read once per call: a streaming (nontemporal) load does not
// allocate them in the caches, which keeps the last-level cache from evicting
// (and writing back) other data on their account.
__device__ __forceinline__ u32x4_t ldg16_stream(const uint16_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane 4q+r
// receives element r of the 8-byte rows addressed by lanes q, q+4, q+8, q+12.
__device__ __forceinline__ u32x2_t ds_read_tr16(const unsigned char* p)
{
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
    return __builtin_bit_cast(u32x2_t, v);
}

// Max over the four 16-lane groups (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap instructions, which stay in the VALU instead of going through LDS.
__device__ __forceinline__ float max_across_groups(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float m = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    // gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even)
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

template <int DP, int RT>
struct Cfg {
    static constexpr int WAVES = waves_for(DP);
    static constexpr int THREADS = WAVES * 64;
    static constexpr int DW = DP / WAVES;  // d per wave
    static constexpr int KS = DW / 32;      // QK^T k-steps per wave
    static constexpr int DT = DW / 16;      // PV d-tiles per wave
    static constexpr int ROWS = 16 * RT;
    static constexpr int NOWN = (RT + WAVES - 1) / WAVES;  // row tiles owned per wave
    // K/V loads: a key's d-slice is NCH 16-byte chunks, read by NCH consecutive lanes, so
    // one load instruction covers KPI whole slices (256 contiguous bytes per key at
    // head_dim 512); a 32-key tile takes NI loads each of K and V per wave.
    static constexpr int NCH = DW / 8;
    static constexpr int KPI = 64 / NCH;
    static constexpr int NI = kTK / KPI;
    static constexpr int KSH = NCH == 16 ? 0 : NCH == 8 ? 1 : 2;
    // K tile, row-major [key][d_local] in 16-byte chunks; chunk c of row r sits at
    // c ^ ((r >> KSH) % NCH), which keeps both the row-wise stores and the MFMA-order
    // reads (16 keys at one chunk) free of bank conflicts.
    static constexpr int KROW = DW * 2;
    static __device__ __forceinline__ int kofs(int row, int chunk)
    {
        return row * KROW + 16 * (chunk ^ ((row >> KSH) & (NCH - 1)));
    }
    // V tile, row-major [key][d_local], addressed in 8-byte chunks.  A transposing
    // read touches four key rows of 32 bytes per 16-lane group (eight rows per
    // 32-lane pass).  Rows of 256 bytes XOR the chunk index with 4*(row % 8), which
    // puts the eight rows of a pass on distinct banks; shorter rows get a 32-byte pad.
    static constexpr bool VSWZ = DW * 2 == 256;
    static constexpr int VROW = VSWZ ? DW * 2 : DW * 2 + 32;
    static __device__ __forceinline__ int vofs(int row, int chunk)
    {
        return row * VROW + 8 * (VSWZ ? chunk ^ ((row & 7) << 2) : chunk);
    }
    // LDS layout (bytes)
    static constexpr int SX_BYTES = WAVES * 2 * RT * 64 * 16;  // partial S^T [wave][h][b][lane]
    static constexpr int PX_BYTES = RT * 64 * 16;               // P^T (B operand) [b][lane]
    static constexpr int V_BYTES_PER_WAVE = kTK * VROW;
    static constexpr int V_BYTES = WAVES * V_BYTES_PER_WAVE;
    static constexpr int K_BYTES_PER_WAVE = kTK * KROW;
    static constexpr int K_BYTES = WAVES * K_BYTES_PER_WAVE;
    static constexpr int ROWF_BYTES = ROWS * 4;
    static constexpr int OFF_SX = 0;
    static constexpr int OFF_PX = OFF_SX + SX_BYTES;
    static constexpr int OFF_V = OFF_PX + PX_BYTES;
    static constexpr int OFF_K = OFF_V + V_BYTES;
    static constexpr int OFF_LSUM = OFF_K + K_BYTES;
    static constexpr int OFF_MREF = OFF_LSUM + ROWF_BYTES;
    static constexpr int OFF_FLAG = OFF_MREF + ROWF_BYTES;
    // the split units of the run, for the in-kernel merge: [2 slots][16] int64
    static constexpr int OFF_REC = OFF_FLAG + 16 * 4;
    static constexpr int LDS_BYTES = OFF_REC + 2 * 16 * 8;
    // Epilogue staging of the unit's normalised rows as bf16, [row][d] with a 32-byte
    // pad per row, in the bytes the tile loop no longer uses (everything below LSUM).
    static constexpr int SROW = DP * 2 + 32;
    static constexpr int OFF_STAGE = 0;
    static_assert(ROWS * SROW <= OFF_LSUM, "epilogue staging must fit below the row sums");
    static_assert(KS >= 1 && DT >= 1, "head_dim too small for the d-split");
    static_assert(NCH >= 4 && NCH <= 16 && KPI * NCH == 64 && NI * KPI == kTK, "load geometry");
    static_assert(RT <= 14, "flag array (the last two words carry the merge decision)");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// EXACT: head_dim == DP, so every d-chunk exists and no lane needs masking.
// SPANS: causal rows may be widened by bidirectional spans (a.span_offsets).
// APPEND: the block's own K/V (keys L..T-1) are read from a.k_new / a.v_new instead of
// the pages, and the workgroup that finishes a (request, kv-head)'s last tile writes them
// into the pages (the block K/V append of a draft step, fused into the same launch).
// WIDEPG: pages hold at least 16 keys, so a 32-key tile lies in at most two pages
// whose ids are wave-uniform.  (Smaller pages are a separate instance: a runtime
// branch between the two ways of locating keys made the compiler wait for the
// tile's LDS stores before every key address on the common path.)
template <int DP, int RT, bool EXACT, bool SPANS, bool WIDEPG, bool APPEND>
__global__ __launch_bounds__(threads_for<DP>) void attn_mfma_kernel(AttnArgs a)
{
    using C = Cfg<DP, RT>;
    constexpr int WAVES = C::WAVES;
    constexpr int KS = C::KS;
    constexpr int DT = C::DT;
    constexpr int DW = C::DW;
    constexpr int NOWN = C::NOWN;
    constexpr bool LATE_V = DP <= 256;  // where V is staged and requested (see the tile step)
    // Otherwise V of the next tile is requested after this wave's S^T products, or, where a
    // wave owns two row tiles, after the first barrier.
    constexpr bool V_AFTER_BARRIER = !LATE_V && RT > WAVES;
    // The merge directory (AttnArgs::dir) is written by every instance when the planner
    // passes one (every launch whose partials the combine kernel merges).
    constexpr bool DIR = true;

    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
#ifdef DFLASH_TIMELINE
    // Timeline build: the 100 MHz wall clock when the workgroup starts, when its first
    // tile loop starts and when its last one ends; its tile count.  Written with the
    // end of its last epilogue (before any in-kernel merge) to
    // timeline[8 * logical workgroup + {0, 1, 2, 3, 4}].
    const uint64_t tl_start = wall_clock64();
    uint64_t tl_loop0 = 0, tl_loop1 = 0, tl_tiles = 0;
#endif
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    f32x4_t* sx = reinterpret_cast<f32x4_t*>(lds + C::OFF_SX);
    u32x4_t* px = reinterpret_cast<u32x4_t*>(lds + C::OFF_PX);
    float* lsum_s = reinterpret_cast<float*>(lds + C::OFF_LSUM);
    float* mref_s = reinterpret_cast<float*>(lds + C::OFF_MREF);
    int* flag_s = reinterpret_cast<int*>(lds + C::OFF_FLAG);

    // The tile size and the rows per unit are fixed by the instance (the planner sets the
    // same values); as constants, the work-split arithmetic divides by them with shifts and
    // multiplications instead of division sequences.
    Decomp d = a.d;
    d.tk = kTK;
    d.rmax = C::ROWS;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int grp4 = lane >> 4;
    const int wbase = wave * DW;  // first d of this wave's slice
    unsigned char* vls = lds + C::OFF_V + wave * C::V_BYTES_PER_WAVE;
    unsigned char* kls = lds + C::OFF_K + wave * C::K_BYTES_PER_WAVE;
    constexpr int NI = C::NI;
    constexpr int KPI = C::KPI;
    const int kl = lane / C::NCH;  // key of this lane within a load's KPI keys
    const int sl = lane % C::NCH;  // 16-byte chunk of this lane within the key's d-slice
    // this lane's chunk exists (always, unless head_dim < padded head_dim); an absent one
    // reads the row start, finite data that meets a zero Q chunk or an unstored column
    const bool lval = EXACT || wbase + 8 * sl < a.D;

    const int32_t wg = logical_wg(blockIdx.x, d.P);
    const int32_t D = a.D;
    const int32_t G = d.G;
    const int32_t psize = 1 << a.page_shift;

    // d-chunks of this lane that exist (all of them unless head_dim < padded head_dim)
    bool dval[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        dval[s] = EXACT || (wbase + 32 * s + 8 * grp4 < D);

    int64_t total, begin, end, qtotal;
    RunStart first;
    wave_locate_run(a.ctx_lens, a.block_lens, a.causal, d, wg, total, begin, end, first, qtotal);
    if (DIR && total == 0 && a.dir && wg == 0) {
        // no request has queries: every row of the merge directory is no request's
        for (int64_t R = threadIdx.x; R < a.total_rows; R += C::THREADS)
            a.dir[R] = make_uint2(0u, 0u);
    }
    if (begin >= end)
        return;
    // The split units this run holds a piece of (slot 0: its first unit, slot 1: its
    // last), kept in LDS for the in-kernel merge after the run (registers are full in
    // the tile loop): per slot [0] the unit's first flat position, [1] its first
    // workgroup (which names its counters), [2] its pieces, [3] the query tokens before
    // its request, [4] its first row, [5] its rows, [6] its kv-head, [8] the arrival word
    // before this piece's arrival; [7] of slot 0 is the run length per workgroup.
    int64_t* rec_s = reinterpret_cast<int64_t*>(lds + C::OFF_REC);
    int have_rec = 0;
    // What the epilogues and the end of the run need, kept in LDS rather than in registers
    // through the tile loop: [7] the run length per workgroup, [12] the query tokens of
    // all requests if this run holds the last tile (else -1), [13] the merge directory's
    // rows, [14] its address (0: none).
    if (threadIdx.x == 0 && (DIR || a.ctr))
        rec_s[7] = tiles_per_wg(total, d.P);
    if (DIR && threadIdx.x == 0) {
        rec_s[12] = qtotal;
        rec_s[13] = a.total_rows;
        rec_s[14] = reinterpret_cast<int64_t>(a.dir);
    }
    // Segments of this workgroup's run that a lazy pass abandoned (bit i: i-th segment;
    // segments past 63 share the overflow flag and are all recomputed).
    uint64_t redo_mask = 0;
    bool redo_overflow = false;

    f32x4_t o[DT][RT];
    float m_run[NOWN];
    float l_run[NOWN];

    // Walks the run; phase 0 runs every segment lazily, phase 1 recomputes abandoned ones.
    auto walk = [&](auto phase_tag) {
        constexpr int PHASE = decltype(phase_tag)::value;
        int32_t r = first.r;
        int64_t rbase = first.rbase;
        int64_t qstart = first.qstart;
        // lengths and flag of request r (the first request's come with the run)
        int32_t L = first.L, n = first.n;
        bool is_causal = first.causal;
        int64_t pos = begin;
        int seg = 0;
        while (pos < end) {
            const ReqGeom g = req_geom(L, n, d);
            const int64_t w = req_work(g, d);
            if (pos >= rbase + w) {
                // pos < end <= total work, so request r + 1 exists
                rbase += w;
                qstart += n;
                ++r;
                L = a.ctx_lens[r];
                n = a.block_lens[r];
                is_causal = a.causal ? (a.causal[r] != 0) : false;
                continue;
            }
            const Segment sg = run_segment(g, rbase, pos, end, d.ov);
            pos = sg.next;
            if (sg.t0 >= sg.t1)
                continue;  // only set-up positions of this unit: nothing to do here
            const int32_t unit = sg.unit;
            // segment bounds are wave-uniform; readfirstlane lets the compiler keep the tile
            // loop in scalar control flow with exact memory-counter waits
            const int32_t t0 = __builtin_amdgcn_readfirstlane(sg.t0);
            const int32_t t1 = __builtin_amdgcn_readfirstlane(sg.t1);
            const int this_seg = seg++;
            if constexpr (PHASE == 1) {
                const bool redo = this_seg < 64 ? ((redo_mask >> this_seg) & 1u) != 0 : redo_overflow;
                if (!redo)
                    continue;
            }
            const int32_t kvh = unit / g.ngroups;
            const int32_t grp = unit % g.ngroups;
            const int slot = (this_seg == 0) ? 0 : 1;
            const bool whole = (t0 == 0 && t1 == g.ntiles);
            const int32_t row0 = grp * d.rmax;
            const int32_t rows_here = min(d.rmax, n * G - row0);
            const int32_t T = g.T;
            const int32_t* pt = a.page_table + (int64_t)r * a.max_pages_per_req;
            // element offset of kv-head kvh inside a key row; d-chunks past head_dim
            // address the row start instead (never past the row), and are zeroed
            const int64_t head_off = (int64_t)kvh * D;

            // Tile keys are located in two steps so that no wait lands on loads in flight:
            // tile_page() reads, one tile ahead, the page-table entry of key lane % 32 of the
            // tile, clamped to the request's last key T - 1; tile_rows() hands each lane the
            // entries of its NI keys when the tile's K/V are requested -- two lane reads when
            // a page holds at least 16 keys, else a shuffle per key.  Keys past the end read
            // key T - 1 (a real key, so finite; its logit is masked), which keeps every load
            // in bounds and away from page-tail garbage.
            auto tile_page = [&](int32_t t) -> int32_t {
                const int32_t key = g.kv_lo + t * kTK + (lane & 31);
                return pt[(key < T ? key : T - 1) >> a.page_shift];
            };
            const int32_t hkvd = d.Hkv * D;  // elements per key row
            // element offset of this lane's 16 bytes inside a key row (< hkvd)
            const int32_t lane_off = (int32_t)head_off + (lval ? wbase + 8 * sl : 0);
            // APPEND: keys from app_from on are the block's own, read from k_new / v_new:
            // element offsets relative to k_pages (v_pages for V, which adds app_dv)
            const int32_t app_from = APPEND ? L : INT32_MAX;
            const int64_t app_base = APPEND ? a.app_dk + (qstart - L) * (int64_t)hkvd + lane_off : 0;
            uint32_t blkmask = 0;  // APPEND: bit i -- this lane's i-th key of the tile is a block key
            auto tile_rows = [&](int32_t t, int32_t pgl, int64_t (&rows)[NI]) {
                const int32_t k0 = g.kv_lo + t * kTK;
                if constexpr (APPEND)
                    blkmask = 0;
                if constexpr (WIDEPG) {
                    // Keys 0-15 of the tile lie in the page of its key 0, keys 16-31 in that
                    // of its key 16 (tiles start at multiples of 32; a clamped key T - 1
                    // lies in the page tile_page() read for its half).  A page's first
                    // element comes from one wave-uniform product; a key adds its place in
                    // the page, which fits 32 bits (page_size * Hkv * D < 2^31 is checked
                    // on the host).
                    const uint32_t p0 = (uint32_t)__builtin_amdgcn_readlane(pgl, 0);
                    const uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane(pgl, 16);
                    const uint32_t page_elems = (uint32_t)psize * (uint32_t)hkvd;
                    const int64_t base0 = (int64_t)((uint64_t)p0 * page_elems);
                    const int64_t base1 = (int64_t)((uint64_t)p1 * page_elems);
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int32_t key = min(k0 + i * KPI + kl, T - 1);
                        const uint32_t inpg = (uint32_t)(key & (psize - 1)) * (uint32_t)hkvd + (uint32_t)lane_off;
                        rows[i] = (((i * KPI) & 16) ? base1 : base0) + inpg;
                        if constexpr (APPEND) {
                            const bool blk = key >= app_from;
                            rows[i] = blk ? app_base + (int64_t)key * hkvd : rows[i];
                            blkmask |= (blk ? 1u : 0u) << i;
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        const int32_t page = __builtin_amdgcn_ds_bpermute(4 * (i * KPI + kl), pgl);
                        const int32_t key = min(k0 + i * KPI + kl, T - 1);
                        const uint64_t slot = (uint64_t)(uint32_t)page * (uint32_t)psize + (uint32_t)(key & (psize - 1));
                        rows[i] = (int64_t)(slot * (uint32_t)hkvd) + lane_off;
                    }
                }
            };

            // Page entries of the segment's first two tiles, requested before Q so that
            // waiting for them never waits for Q (which is needed only at the first product).
            const int32_t pg_first = tile_page(t0);
            const int32_t pg_second = tile_page(t0 + 1);
            __builtin_amdgcn_sched_barrier(0);

            // ---------------- Q^T (B operand) for the unit ----------------
            // All of the unit's Q chunks are requested here; padding rows and absent d-chunks
            // (which read a real row) are zeroed only after the first tile's K/V requests
            // (q_mask below), so that nothing waits for Q before those go out.  Zeroing each
            // row tile as it arrived made the compiler wait for every row tile's loads in
            // turn (five dependent rounds at head_dim 512) before the first K/V request.
            bf16x8_t qf[RT][KS];
#pragma unroll
            for (int b = 0; b < RT; ++b) {
                const int32_t row = b * 16 + l16;
                const bool rv = row < rows_here;
                const int32_t rr = row0 + (rv ? row : 0);
                const int32_t qi = rr / G;
                const int32_t qj = rr % G;
                const uint16_t* qrow = a.q + ((qstart + qi) * a.Hq + (int64_t)kvh * G + qj) * D;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    qf[b][s] = as_bf16x8(ldg16(qrow + (dval[s] ? wbase + 32 * s + 8 * grp4 : 0)));
            }
            auto q_mask = [&]() {
#pragma unroll
                for (int b = 0; b < RT; ++b) {
                    const bool rv = b * 16 + l16 < rows_here;
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        u32x4_t x = __builtin_bit_cast(u32x4_t, qf[b][s]);
                        const bool keep = rv && dval[s];
                        x[0] = keep ? x[0] : 0u;
                        x[1] = keep ? x[1] : 0u;
                        x[2] = keep ? x[2] : 0u;
                        x[3] = keep ? x[3] : 0u;
                        qf[b][s] = as_bf16x8(x);
                    }
                }
            };


            float m_fix[NOWN];
            // Visible key range [rlo, rhi] of this lane's query row in each owned row tile, and
            // the keys [ilo, ihi] every real row of the tile sees: a tile inside that range
            // needs no mask (padding rows then get finite weights that reach no output).
            int32_t rlo[NOWN], rhi[NOWN], ilo[NOWN], ihi[NOWN];
#pragma unroll
            for (int ob = 0; ob < NOWN; ++ob) {
                m_fix[ob] = -INFINITY;
                const int32_t row = (ob * WAVES + wave) * 16 + l16;
                const bool rv = row < rows_here;
                const int32_t qi = (row0 + (rv ? row : 0)) / G;
                query_range(L, n, qi, is_causal, d.window, rlo[ob], rhi[ob]);
                if (SPANS && is_causal)
                    rhi[ob] = span_high(a.span_offsets, a.spans, a.num_spans, r, L + qi, T, rhi[ob]);
                int32_t lo_all = rv ? rlo[ob] : INT32_MIN;
                int32_t hi_all = rv ? rhi[ob] : INT32_MAX;
                if (!rv)
                    rhi[ob] = -1;  // padding row: nothing visible
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    lo_all = max(lo_all, __shfl_xor(lo_all, off));
                    hi_all = min(hi_all, __shfl_xor(hi_all, off));
                }
                ilo[ob] = __builtin_amdgcn_readfirstlane(lo_all);
                ihi[ob] = __builtin_amdgcn_readfirstlane(hi_all);
            }

            // One pass over the segment's tiles (MODE kLazy, kMaxScan or kFixed).  Returns
            // true when a kLazy pass met a tile beyond its reference bound.
            auto run_pass = [&](auto mode_tag) -> bool {
                constexpr int MODE = decltype(mode_tag)::value;
                if constexpr (MODE != kMaxScan) {
#pragma unroll
                    for (int c = 0; c < DT; ++c)
#pragma unroll
                        for (int b = 0; b < RT; ++b)
                            o[c][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int ob = 0; ob < NOWN; ++ob) {
                    m_run[ob] = MODE == kFixed ? m_fix[ob] : -INFINITY;
                    l_run[ob] = 0.f;
                }
                bool aborted = false;

                int64_t rows[NI];  // element offsets of this lane's 16 bytes of each key it loads
                int32_t pg_next;
                u32x4_t kr[NI], vr[NI];
                auto issue = [&](const uint16_t* base, u32x4_t (&dst)[NI]) {
#pragma unroll
                    for (int i = 0; i < NI; ++i)
                        dst[i] = ldg16_stream(base + rows[i]);
                };
                // V: as K, except that block keys (APPEND) are read from v_new
                auto issue_v = [&](u32x4_t (&dst)[NI]) {
                    if constexpr (APPEND) {
#pragma unroll
                        for (int i = 0; i < NI; ++i)
                            dst[i] = ldg16_stream(a.v_pages + rows[i] + (((blkmask >> i) & 1u) ? a.app_dv : 0));
                    } else {
                        issue(a.v_pages, dst);
                    }
                };

                // One 32-key tile per step.  At the top of step t the registers holding K of
                // tile t are written to LDS and at once refilled with K of tile t+1, which so
                // has a whole step to arrive.  V is requested apart from K, so that the two
                // halves of the workgroup's 64 KB do not queue at the address unit at once
                // (both at the top measured 12% slower on C3).  Up to head_dim 256 (LATE_V)
                // V(t) goes to LDS just before the PV product and V(t+1) is requested there,
                // so V too has a whole step and waiting for K(t) never waits for V(t)
                // (C2 40.4 vs 42.5 us, A/B on one box).  At head_dim 512, V(t) goes to LDS
                // with K(t) and V(t+1) is requested after the S^T product: the late form
                // keeps V's registers live across that product, and measured 1-2% slower
                // (C5, the global verify layer) with C3 unchanged.  With five row tiles
                // (one wave owns two) V(t+1) goes out after the first barrier instead:
                // C3 120.3 vs 121.7 us, the global verify layer 192.2 vs 194.6 us, while
                // four row tiles (C5) measured 0.6% slower that way (A/B on one box).  Inside the loop every request is
                // unconditional (keys past the request read its last key, page entries are
                // read at clamped indices): the loop has no divergent branches and each wait
                // on the memory counter is exact.  The issue order (page entries, K, V) is pinned with
                // scheduling barriers, here and in the loop: the compiler's waits at the
                // loop head are exact only if both paths into it issue in the same order.
                tile_rows(t0, pg_first, rows);
                pg_next = pg_second;
                __builtin_amdgcn_sched_barrier(0);
                issue(a.k_pages, kr);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (MODE != kMaxScan)
                    issue_v(vr);
                __builtin_amdgcn_sched_barrier(0);
                q_mask();  // idempotent: a second pass over the segment zeroes the same lanes
                __builtin_amdgcn_sched_barrier(0);
                // One tile; PF: also request the next one (every tile but the segment's last).
                auto step = [&](const int32_t t, auto pf_tag) {
                    constexpr bool PF = decltype(pf_tag)::value;
                    const int32_t k0 = g.kv_lo + t * kTK;
                    // (1) this wave's K slice (and, unless LATE_V, its V slice) -> LDS
                    // [key][d_local].  Keys past the request hold its last key and d past
                    // head_dim the row start: finite values whose weight (masked logit) or
                    // output column (never stored) is 0.
                    if constexpr (MODE != kMaxScan && !LATE_V) {
#pragma unroll
                        for (int i = 0; i < NI; ++i)
                            *reinterpret_cast<u32x4_t*>(vls + C::vofs(i * KPI + kl, 2 * sl)) = vr[i];
                    }
#pragma unroll
                    for (int i = 0; i < NI; ++i)
                        *reinterpret_cast<u32x4_t*>(kls + C::kofs(i * KPI + kl, sl)) = kr[i];
                    // request tile t+1 (page entries of t+2 first, so that waiting for them
                    // later never waits for K/V)
                    if constexpr (PF) {
                        tile_rows(t + 1, pg_next, rows);
                        pg_next = tile_page(t + 2);
                        __builtin_amdgcn_sched_barrier(0);
                        issue(a.k_pages, kr);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // (2) partial S^T over this wave's d-slice (absent d: Q is zero there and K
                    //     finite; absent keys are masked below).  A operand: key 16h + l16,
                    //     d chunk 4s + grp4 of the slice.
                    if constexpr (LATE_V) {
                        // one 16-key half at a time: V(t)'s registers are live here
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            bf16x8_t kb[KS];
#pragma unroll
                            for (int s = 0; s < KS; ++s)
                                kb[s] = as_bf16x8(
                                    *reinterpret_cast<const u32x4_t*>(kls + C::kofs(16 * h + l16, 4 * s + grp4)));
#pragma unroll
                            for (int b = 0; b < RT; ++b) {
                                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int s = 0; s < KS; ++s)
                                    acc = mfma16(kb[s], qf[b][s], acc);
                                sx[((wave * 2 + h) * RT + b) * 64 + lane] = acc;
                            }
                        }
                    } else {
                        bf16x8_t kb[2][KS];
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int s = 0; s < KS; ++s)
                                kb[h][s] = as_bf16x8(
                                    *reinterpret_cast<const u32x4_t*>(kls + C::kofs(16 * h + l16, 4 * s + grp4)));
#pragma unroll
                        for (int b = 0; b < RT; ++b) {
                            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s = 0; s < KS; ++s) {
                                acc0 = mfma16(kb[0][s], qf[b][s], acc0);
                                acc1 = mfma16(kb[1][s], qf[b][s], acc1);
                            }
                            sx[((wave * 2 + 0) * RT + b) * 64 + lane] = acc0;
                            sx[((wave * 2 + 1) * RT + b) * 64 + lane] = acc1;
                        }
                        // V of tile t+1, requested after this wave's products
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (MODE != kMaxScan && PF && !V_AFTER_BARRIER)
                            issue_v(vr);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    __syncthreads();
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (MODE != kMaxScan && PF && V_AFTER_BARRIER) {
                        issue_v(vr);  // ... or after the barrier
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // (3) owners: reduce, mask, softmax, publish P^T
#pragma unroll
                    for (int ob = 0; ob < NOWN; ++ob) {
                        const int b = ob * WAVES + wave;
                        if (b < RT) {
                            // partials are requested four at a time before any is summed, so that
                            // the LDS latency is paid once per four
                            float z[8];
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                                for (int w0 = 0; w0 < WAVES; w0 += 4) {
                                    f32x4_t part[4];
#pragma unroll
                                    for (int ww = 0; ww < 4; ++ww)
                                        part[ww] = sx[(((w0 + ww) * 2 + h) * RT + b) * 64 + lane];
                                    acc += (part[0] + part[1]) + (part[2] + part[3]);
                                }
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    z[h * 4 + e] = acc[e];
                            }
                            float tmax = -INFINITY;
                            if (k0 >= ilo[ob] && k0 + kTK - 1 <= ihi[ob]) {
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    z[e] *= a.scale_log2;
                                    tmax = fmaxf(tmax, z[e]);
                                }
                            } else {
                                const int32_t lo = rlo[ob], hi = rhi[ob];
#pragma unroll
                                for (int h = 0; h < 2; ++h)
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        const int32_t key = k0 + 16 * h + 4 * grp4 + e;
                                        const bool vis = key >= lo && key <= hi;
                                        const float zz = vis ? z[h * 4 + e] * a.scale_log2 : -INFINITY;
                                        z[h * 4 + e] = zz;
                                        tmax = fmaxf(tmax, zz);
                                    }
                            }
                            tmax = max_across_groups(tmax);
                            if constexpr (MODE == kMaxScan) {
                                m_fix[ob] = fmaxf(m_fix[ob], tmax);
                            } else {
                                const float m_old = m_run[ob];
                                float m_new = m_old;
                                bool over = false;
                                if constexpr (MODE == kLazy) {
                                    const bool first = m_old == -INFINITY;
                                    over = !first && tmax > m_old + kLazyBound;
                                    m_new = first ? tmax : m_old;
                                }
                                const float mu = (m_new == -INFINITY) ? 0.f : m_new;
                                u32x4_t pk;
                                // the denominator sums the same bf16-rounded weights PV uses
                                // (a dot product of each packed pair with (1, 1))
                                const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
                                float psum = l_run[ob];
#pragma unroll
                                for (int e2 = 0; e2 < 4; ++e2) {
                                    const uint32_t w2 = pack_bf16x2(__builtin_amdgcn_exp2f(z[2 * e2] - mu),
                                                                    __builtin_amdgcn_exp2f(z[2 * e2 + 1] - mu));
                                    pk[e2] = w2;
                                    psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2), ones, psum,
                                                                          false);
                                }
                                l_run[ob] = psum;
                                m_run[ob] = m_new;
                                px[b * 64 + lane] = pk;
                                if constexpr (MODE == kLazy) {
                                    const unsigned long long anyover = __ballot(over);
                                    if (lane == 0)
                                        flag_s[b] = anyover ? 1 : 0;
                                }
                            }
                        }
                    }
                    __syncthreads();
                    if constexpr (MODE == kMaxScan)
                        return;
                    if constexpr (MODE == kLazy) {
                        int anyover = 0;
#pragma unroll
                        for (int b = 0; b < RT; ++b)
                            anyover |= flag_s[b];
                        aborted = __builtin_amdgcn_readfirstlane(anyover) != 0;
                    }
                    // (4) LATE_V: this wave's V slice of tile t -> LDS (the wave's own tile: no
                    // barrier), and V of tile t+1 requested into the freed registers
                    if constexpr (LATE_V) {
#pragma unroll
                        for (int i = 0; i < NI; ++i)
                            *reinterpret_cast<u32x4_t*>(vls + C::vofs(i * KPI + kl, 2 * sl)) = vr[i];
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (PF)
                            issue_v(vr);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // (5) O^T += V^T P^T for this wave's d-slice
                    // A operand V^T: lane l holds d = 16c + l%16 at key slots 4*grp4 + 0..3
                    // and 16 + 4*grp4 + 0..3 (the key order of P^T).  Transposing reads:
                    // lane j of group grp4 addresses key 4*grp4 + j/4 (and +16) at
                    // d = 16c + 4*(j%4).  All reads are issued before the first product.
                    bf16x8_t pb[RT];
#pragma unroll
                    for (int b = 0; b < RT; ++b)
                        pb[b] = as_bf16x8(px[b * 64 + lane]);
                    const int vrow = 4 * grp4 + (l16 >> 2);
                    u32x2_t vt[DT][2];
#pragma unroll
                    for (int c = 0; c < DT; ++c) {
                        vt[c][0] = ds_read_tr16(vls + C::vofs(vrow, 4 * c + (l16 & 3)));
                        vt[c][1] = ds_read_tr16(vls + C::vofs(vrow + 16, 4 * c + (l16 & 3)));
                    }
#pragma unroll
                    for (int c = 0; c < DT; ++c) {
                        const u32x4_t va = {vt[c][0][0], vt[c][0][1], vt[c][1][0], vt[c][1][1]};
                        const bf16x8_t vb = as_bf16x8(va);
#pragma unroll
                        for (int b = 0; b < RT; ++b)
                            o[c][b] = mfma16(vb, pb[b], o[c][b]);
                    }
                };
                // An abandoned lazy segment leaves by the loop condition only: an exit between
                // the softmax and the PV product would make the compiler keep a second copy of
                // every accumulator.  The tile that triggered it still runs its (discarded) PV.
                int32_t t = t0;
                for (; t + 1 < t1 && !aborted; ++t)
                    step(t, std::true_type{});
                // The last tile requests nothing: a request for a tile past the segment would
                // hold its registers, and so the epilogue, until it landed.
                if (t < t1 && !aborted)
                    step(t, std::false_type{});
                // wait for the last tile's LDS traffic of every wave before anything reuses it
                __syncthreads();
                return aborted;
            };

#ifdef DFLASH_TIMELINE
            if (tl_loop0 == 0)
                tl_loop0 = wall_clock64();
            tl_tiles += t1 - t0;
#endif
            if constexpr (PHASE == 0) {
                if (run_pass(std::integral_constant<int, kLazy>{})) {
                    if (this_seg < 64)
                        redo_mask |= (uint64_t)1 << this_seg;
                    else
                        redo_overflow = true;
                    continue;  // recomputed after the run
                }
            } else {
                run_pass(std::integral_constant<int, kMaxScan>{});
                run_pass(std::integral_constant<int, kFixed>{});
            }

#ifdef DFLASH_TIMELINE
            tl_loop1 = wall_clock64();
#endif
            // ---------------- epilogue ----------------
#pragma unroll
            for (int ob = 0; ob < NOWN; ++ob) {
                const int b = ob * WAVES + wave;
                if (b < RT) {
                    float l = l_run[ob];
                    l += __shfl_xor(l, 16);
                    l += __shfl_xor(l, 32);
                    if (grp4 == 0) {
                        lsum_s[b * 16 + l16] = l;
                        mref_s[b * 16 + l16] = m_run[ob];
                    }
                }
            }
            __syncthreads();
            // Stage the normalised rows as bf16 (rows [row][d]) in the LDS the tile loop no
            // longer uses, then write whole rows with contiguous 16-byte-per-lane stores: a
            // store straight from the MFMA layout would scatter 16 short row pieces.
            unsigned char* stage = lds + C::OFF_STAGE;
#pragma unroll
            for (int b = 0; b < RT; ++b) {
                const float l = lsum_s[b * 16 + l16];
                const float inv = l > 0.f ? 1.f / l : 0.f;
                unsigned char* srow = stage + (b * 16 + l16) * C::SROW + (wbase + 4 * grp4) * 2;
#pragma unroll
                for (int c = 0; c < DT; ++c) {
                    const f32x4_t v = o[c][b] * inv;
                    const u32x2_t pk2 = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    *reinterpret_cast<u32x2_t*>(srow + 32 * c) = pk2;
                }
            }
            __syncthreads();
            constexpr int CPR = DP / 8;    // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;  // rows per wave instruction
            const int rsub = lane / CPR;
            const int ch = lane % CPR;
            if (!whole) {
                // A partial: bf16 rows of this workgroup's slot (a normalised partial is a
                // convex combination of bf16 values, so bf16 holds its range; its rounding
                // is that of the output itself).  Head-dim columns past D land in the
                // slot's row padding, which the combine never reads; padding rows are not
                // stored at all (every workgroup writes its partial at about the same
                // time, so these bytes are paid at the end of the kernel).
                const int64_t sbase = ((int64_t)wg * 2 + slot) * d.rmax;
#pragma unroll
                for (int r0 = wave * RPI; r0 < C::ROWS; r0 += WAVES * RPI) {
                    const int row = r0 + rsub;
                    if (row < rows_here) {
                        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(stage + row * C::SROW + ch * 16);
                        uint16_t* dst = a.part_o + (sbase + row) * DP + ch * 8;
                        // merged in this kernel by other workgroups: coherent stores; merged by
                        // the combine kernel: streaming stores (read once, from HBM)
                        if (a.ctr)
                            store16_coherent(dst, __builtin_bit_cast(uint4, x));
                        else
                            __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(dst));
                    }
                }
                // Merge directory (AttnArgs::dir): the unit's second piece writes its rows'
                // entries.  That run began inside the unit, less than one run length past its
                // first real tile, so the first piece is the previous workgroup.  It is a run
                // inside the unit unless the unit has two pieces, so the work stays off the
                // runs that cross into a second unit, which end last.
                if (DIR && slot == 0 && t0 > 0) {
                    uint2* const dirp = reinterpret_cast<uint2*>(rec_s[14]);
                    const int64_t tpw = rec_s[7];
                    if (dirp && t0 <= tpw) {
                        const int64_t us = rbase + (int64_t)unit * g.uwork;
                        const int64_t kf = wg - 1;
                        const int64_t kl = (us + g.uwork - 1) / tpw;
                        const uint2 e = dir_pack(kf, kf * tpw < us ? 1 : 0, kl - kf + 1, 0);
                        const int64_t nrows = rec_s[13];
                        for (int row = threadIdx.x; row < rows_here; row += C::THREADS) {
                            const int32_t rr = row0 + row;
                            const int64_t R = (qstart + rr / G) * a.Hq + (int64_t)kvh * G + rr % G;
                            if (R < nrows)  // (total_q below the blocks' sum breaks the contract)
                                dirp[R] = make_uint2(e.x, e.y | ((uint32_t)row << 24));
                        }
                    }
                }
                if (wave == 0 && grp4 == 0) {
#pragma unroll
                    for (int b = 0; b < RT; ++b) {
                        const float l = lsum_s[b * 16 + l16];
                        const float lse = l > 0.f ? mref_s[b * 16 + l16] + log2f(l) : -INFINITY;
                        if (a.ctr)
                            store_f32_coherent(a.part_lse + sbase + b * 16 + l16, lse);
                        else
                            a.part_lse[sbase + b * 16 + l16] = lse;
                    }
                }

            } else {
                // The whole unit was here: bf16 output rows, real rows and columns only.
#pragma unroll
                for (int r0 = wave * RPI; r0 < C::ROWS; r0 += WAVES * RPI) {
                    const int row = r0 + rsub;
                    if (row < rows_here && (EXACT || ch * 8 < D)) {
                        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(stage + row * C::SROW + ch * 16);
                        const int32_t rr = row0 + row;
                        const int32_t qi = rr / G;
                        const int32_t qj = rr % G;
                        const int64_t R = (qstart + qi) * a.Hq + (int64_t)kvh * G + qj;
                        *reinterpret_cast<u32x4_t*>(a.out + R * D + ch * 8) = x;
                        if constexpr (DIR) {
                            uint2* const dirp = reinterpret_cast<uint2*>(rec_s[14]);
                            if (ch == 0 && dirp && R < rec_s[13])
                                dirp[R] = make_uint2(0u, 1u);  // merge directory: nothing to merge
                        }
                    }
                }
            }
            __syncthreads();
            if constexpr (APPEND) {
                // the workgroup holding the last tile of the first row group writes the block's
                // K/V rows of this kv-head into their page slots (each (token, kv-head) row once)
                if (grp == 0 && t1 == g.ntiles) {
                    const int32_t nch = D / 8;  // 16-byte chunks per row
                    for (int32_t c = threadIdx.x; c < n * nch; c += C::THREADS) {
                        const int32_t i = c / nch;
                        const int32_t ch = c % nch;
                        const int32_t p = L + i;
                        const int64_t page = pt[p >> a.page_shift];
                        const int64_t dst = ((page << a.page_shift) + (p & (psize - 1))) * hkvd + head_off + ch * 8;
                        const int64_t src = (qstart + i) * (int64_t)hkvd + head_off + ch * 8;
                        *reinterpret_cast<u32x4_t*>(a.k_dst + dst) = ldg16(a.k_new + src);
                        *reinterpret_cast<u32x4_t*>(a.v_dst + dst) = ldg16(a.v_new + src);
                    }
                }
            }
            if (!whole && a.ctr) {
                // record the piece; it is counted in after the run (below), when its stores
                // have long completed -- a wait for them here would stall the run
                if (threadIdx.x == 0) {
                    const int64_t us = rbase + (int64_t)unit * g.uwork;
                    const int64_t tpw = rec_s[7];
                    int64_t kf, kl;
                    unit_pieces(g, us, d.ov, tpw, kf, kl);
                    int64_t* rp = rec_s + 16 * slot;
                    rp[0] = us;
                    rp[1] = kf;
                    rp[2] = kl - kf + 1;
                    rp[3] = qstart;
                    rp[4] = row0;
                    rp[5] = rows_here;
                    rp[6] = kvh;
                }
                have_rec |= 1 << slot;
            }
        }
    };

    walk(std::integral_constant<int, 0>{});
    if (DIR && rec_s[14] != 0 && rec_s[12] >= 0) {
        // the run holding the last tile: rows of tokens past the last request's block
        // (total_q larger than the blocks' sum) belong to no request
        uint2* const dirp = reinterpret_cast<uint2*>(rec_s[14]);
        for (int64_t R = rec_s[12] * a.Hq + threadIdx.x; R < rec_s[13]; R += C::THREADS)
            dirp[R] = make_uint2(0u, 0u);
    }
    if (redo_mask != 0 || redo_overflow)
        walk(std::integral_constant<int, 1>{});
#ifdef DFLASH_TIMELINE
    if (threadIdx.x == 0 && a.timeline) {
        uint64_t* tp = a.timeline + (int64_t)logical_wg(blockIdx.x, d.P) * 8;
        tp[0] = tl_start;
        tp[1] = tl_loop0;
        tp[2] = tl_loop1;
        tp[3] = wall_clock64();
        tp[4] = tl_tiles;
    }
#endif
    if (!a.ctr)
        return;  // the combine kernel merges the partials

    // ---------------- in-kernel merge of the split units (merge.h) ----------------
    // An item is the rows one wave merges at once (LPR lanes per row, 8 head-dim
    // elements per lane).  Piece j of a unit merges items j, j + np, ...; its waves
    // take every fourth of those.
    constexpr int LPR = DP / 8;
    constexpr int RPW = 64 / LPR;
    const int rg = lane / LPR;
    const int32_t d0 = (lane % LPR) * 8;
    const bool dlive = EXACT || d0 < D;
    // publish: every wave's partial rows and log-sum-exps have completed (vmcnt 0) before
    // the barrier; then the pieces are counted in
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (have_rec & (1 << s))
                rec_s[16 * s + 8] = __hip_atomic_fetch_add(a.ctr + kCtrArrive + rec_s[16 * s + 1], 1u,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // the records in LDS
    const int64_t tpw = rec_s[7];
    auto merge_items = [&](const int64_t* rp, int64_t j) {
        const int64_t us = rp[0], kf = rp[1], np = rp[2], qs = rp[3];
        const int32_t row0 = (int32_t)rp[4], rows = (int32_t)rp[5], kvh = (int32_t)rp[6];
        const int64_t nitems = (rows + RPW - 1) / RPW;
        for (int64_t it = j + np * wave; it < nitems; it += np * WAVES) {
            const int32_t rin = (int32_t)it * RPW + rg;
            const bool live = rin < rows;
            float acc[8];
            const float W = merge_pieces<LPR, 16, true>(a.part_o, a.part_lse, d.rmax, DP, kf, np, np, us, tpw, rin,
                                                        live, dlive, d0, acc);
            if (live && dlive) {
                const int32_t rr = row0 + rin;
                const int32_t qi = rr / G;
                const int32_t qj = rr % G;
                store_merged(a.out + ((qs + qi) * a.Hq + (int64_t)kvh * G + qj) * D + d0, acc, W);
            }
        }
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if (!(have_rec & (1 << s)))
            continue;
        const int64_t* rp = rec_s + 16 * s;
        const int64_t us = rp[0], kf = rp[1], np = rp[2];
        const uint32_t old = (uint32_t)rp[8];
        const int64_t me = logical_wg(blockIdx.x, d.P);
        const bool last = (int64_t)(old & kArriveMask) == np - 1;
        bool mine = true;
        if (!last) {
            // wave 0 waits for the unit (or gives up) for the whole workgroup
            if (wave == 0) {
                const bool go = wave_wait_or_give_up(a.ctr + kCtrArrive + kf, (uint32_t)np,
                                                     a.ctr + kCtrGaveUp + 2 * me + s);
                if (lane == 0)
                    flag_s[14 + s] = go ? 1 : 0;
            }
            __syncthreads();
            mine = flag_s[14 + s] != 0;
        }
        if (mine)
            merge_items(rp, me - kf);
        if (last && (old >> 16) != 0) {
            // some pieces gave up before the unit completed: merge their items too
            for (int64_t base = 0; base < np; base += 64) {
                const int64_t k = kf + base + lane;
                uint32_t g = 0;
                if (base + lane < np)
                    g = __hip_atomic_load(a.ctr + kCtrGaveUp + 2 * k + piece_slot(k, us, tpw), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                unsigned long long m = __ballot(g != 0);
                while (m) {
                    const int b = __ffsll((long long)m) - 1;
                    m &= m - 1;
                    merge_items(rp, base + b);
                }
            }
        }
        unit_depart(a.ctr, kf, np, [&](int64_t k) { return piece_slot(k, us, tpw); });
    }
}

// Raises a kernel's dynamic-LDS limit once per device (not on every launch: a call
// being captured into a graph then enqueues nothing but the launch itself).
template <int DP, int RT, bool EXACT, bool SPANS, bool WIDEPG, bool APPEND = false>
static hipError_t ensure_lds_limit()
{
    using C = Cfg<DP, RT>;
    if (C::LDS_BYTES <= 64 * 1024)
        return hipSuccess;
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(attn_mfma_kernel<DP, RT, EXACT, SPANS, WIDEPG, APPEND>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <int DP, int RT, bool EXACT, bool SPANS, bool WIDEPG, bool APPEND>
static hipError_t launch_one(const AttnArgs& a, hipStream_t stream)
{
    using C = Cfg<DP, RT>;
    const hipError_t e = ensure_lds_limit<DP, RT, EXACT, SPANS, WIDEPG, APPEND>();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((attn_mfma_kernel<DP, RT, EXACT, SPANS, WIDEPG, APPEND>), dim3(a.d.P), dim3(C::THREADS),
                       C::LDS_BYTES, stream, a);
    return hipGetLastError();
}

template <int DP, bool EXACT, bool SPANS, bool WIDEPG, bool APPEND>
static hipError_t launch_rt(const AttnArgs& a, int row_tiles, hipStream_t stream)
{
    switch (row_tiles) {
    case 1: return launch_one<DP, 1, EXACT, SPANS, WIDEPG, APPEND>(a, stream);
    case 2: return launch_one<DP, 2, EXACT, SPANS, WIDEPG, APPEND>(a, stream);
    case 3: return launch_one<DP, 3, EXACT, SPANS, WIDEPG, APPEND>(a, stream);
    case 4: return launch_one<DP, 4, EXACT, SPANS, WIDEPG, APPEND>(a, stream);
    case 5: return launch_one<DP, 5, EXACT, SPANS, WIDEPG, APPEND>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <bool SPANS, bool WIDEPG, bool APPEND = false>
static hipError_t launch_dp(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream)
{
    switch (dpad) {
    case 128: return a.D == 128 ? launch_rt<128, true, SPANS, WIDEPG, APPEND>(a, row_tiles, stream)
                                : launch_rt<128, false, SPANS, WIDEPG, APPEND>(a, row_tiles, stream);
    case 256: return a.D == 256 ? launch_rt<256, true, SPANS, WIDEPG, APPEND>(a, row_tiles, stream)
                                : launch_rt<256, false, SPANS, WIDEPG, APPEND>(a, row_tiles, stream);
    case 512: return a.D == 512 ? launch_rt<512, true, SPANS, WIDEPG, APPEND>(a, row_tiles, stream)
                                : launch_rt<512, false, SPANS, WIDEPG, APPEND>(a, row_tiles, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dflash
