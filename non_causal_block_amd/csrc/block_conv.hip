// block_conv.hip -- DFlash2's in-block grouped dynamic depthwise convolution.
//
// prhub summary of vLLM PR #52816 ("DFlash2: local convolution + candidate
// selector"), section "motivation": every proposal position of a draft block
// sees earlier positions of the same block through
//     out[i,c] = sum_t (base[t,c] + delta[i,t,g(c)]) * x[i-t,c],
// with taps that fall before the block's first position set to zero (no second
// backbone pass is needed).  base is a static per-tap, per-channel kernel,
// delta a per-position, per-tap, per-channel-group correction computed upstream;
// channels form contiguous groups, g(c) = c / (channels / groups).
//
// Rows of x / delta / out are block positions packed in request order (request
// r's block occupies rows q_start[r] .. q_start[r] + n_r - 1, like q in the block
// attention).  block_conv_kernel: one thread per (row, channel pair); the
// workgroup's row locates its request, the thread sums taps t = 0 .. min(i, taps-1)
// in that order in fp32 (bf16 in, bf16 out, round to nearest even), re-reading x,
// base and delta through the caches.  block_conv_tiled_kernel (below) serves
// taps <= 16 whenever a workgroup's 512 channels span at most 64 groups, reading
// every input once per workgroup and taking two taps per bf16 dot product.
#include "device_common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kConvThreads = 128;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two fp32 values to a bf16 pair (lo, hi), rounded to nearest even by the hardware conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){lo, hi}, bf16x2));
}

__global__ __launch_bounds__(kConvThreads) void block_conv_kernel(ConvArgs a)
{
    const int64_t row = blockIdx.y;
    const int64_t cp = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;  // channel pair
    // the request whose block holds this row (the same for the whole workgroup),
    // found by a wave-wide scan of block_lens
    int32_t r;
    int64_t qs;
    wave_find_token(a.block_lens, a.B, row, r, qs);
    if (r >= a.B || cp * 2 >= a.C)
        return;
    const int32_t i = (int32_t)(row - qs);
    const int64_t c0 = cp * 2;
    const int32_t per_group = a.C / a.G;
    const int32_t g0 = (int32_t)(c0 / per_group);
    const int32_t g1 = (int32_t)((c0 + 1) / per_group);
    const uint32_t* x = reinterpret_cast<const uint32_t*>(a.x);
    const uint32_t* base = reinterpret_cast<const uint32_t*>(a.base);
    const int64_t cw = a.C / 2;  // channel pairs per row
    const uint16_t* dl = a.delta + row * a.taps * a.G;
    float acc0 = 0.f, acc1 = 0.f;
    const int32_t tmax = min(i, a.taps - 1);
#pragma unroll 4
    for (int32_t t = 0; t <= tmax; ++t) {
        const uint32_t xw = x[(row - t) * cw + cp];
        const uint32_t bw = base[(int64_t)t * cw + cp];
        const float d0 = __uint_as_float((uint32_t)dl[t * a.G + g0] << 16);
        const float d1 = __uint_as_float((uint32_t)dl[t * a.G + g1] << 16);
        acc0 = fmaf(bf16_lo(bw) + d0, bf16_lo(xw), acc0);
        acc1 = fmaf(bf16_hi(bw) + d1, bf16_hi(xw), acc1);
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(a.out);
    o[row * cw + cp] = pack_bf16x2(acc0, acc1);
}

// Tap-pair form, for taps <= 16: one wave per (request, 64 channel pairs), four waves
// per workgroup on adjacent channels.  Each product of two bf16 values is exact in
// fp32, so the sum over taps splits into  sum_t base[t,c] x[i-t,c]  and
// sum_t delta[i,t,g] x[i-t,c],  and two taps at a time go through one bf16 dot product
// with fp32 accumulation: the lane packs (x[j,c], x[j-1,c]) once per row j, the tap pairs
// (base[t,c], base[t+1,c]) once per launch, and reads (delta[i,t,g], delta[i,t+1,g]) from
// LDS, where the workgroup stages the groups its channels belong to with taps
// contiguous (zero past `taps`).  Positions go 16 at a time; the lane keeps the previous
// 16 rows of x for the taps that reach back, zero before the block.
constexpr int kTileThreads = 256;
constexpr int kTilePairs = 64 * (kTileThreads / 64);  // channel pairs per workgroup
constexpr int kTilePos = 16;
constexpr int kTileTaps = 16;
constexpr int kTileGroups = 64;

// groups a workgroup's kTilePairs channel pairs can touch (host and device agree)
__host__ __device__ inline int32_t tile_groups_max(int64_t C, int32_t G)
{
    const int64_t per_group = C / G;
    const int64_t span = (2 * kTilePairs + per_group - 1) / per_group + 1;
    return (int32_t)(span < G ? span : G);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// One chunk of 16 positions.  xr[k] holds row c0 - 16 + k (k < 16: the previous chunk,
// zero before the block); FIRST (c0 == 0) skips the tap pairs that lie wholly before it.
template <int TPP, bool FIRST>
__device__ __forceinline__ void conv_chunk(const uint32_t (&xr)[32], const uint32_t (&blo)[TPP],
                                           const uint32_t (&bhi)[TPP], const uint32_t* d0, const uint32_t* d1,
                                           int32_t dstride, uint32_t* orow, int64_t cw, int32_t cnt, bool live)
{
    constexpr int K0 = FIRST ? 16 : 16 - 2 * (TPP - 1);
    uint32_t plo[32], phi[32];
#pragma unroll
    for (int k = K0; k < 32; ++k) {
        plo[k] = lo_pair(xr[k], xr[k - 1]);
        phi[k] = hi_pair(xr[k], xr[k - 1]);
    }
#pragma unroll
    for (int i = 0; i < kTilePos; ++i) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int tp = 0; tp < TPP; ++tp) {
            if (FIRST && 2 * tp > i)
                continue;
            const int k = 16 + i - 2 * tp;
            a0 = dot2(blo[tp], plo[k], a0);
            a1 = dot2(bhi[tp], phi[k], a1);
            a0 = dot2(d0[i * dstride + tp], plo[k], a0);
            a1 = dot2(d1[i * dstride + tp], phi[k], a1);
        }
        if (live && i < cnt)
            orow[i * cw] = pack_bf16x2(a0, a1);
    }
}

template <int TPP>
__global__ __launch_bounds__(kTileThreads) void block_conv_tiled_kernel(ConvArgs a)
{
    constexpr int TPAD = 2 * TPP;      // staged taps per (position, group)
    extern __shared__ uint32_t dsh[];  // [position][group - g_lo][tap pair]
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    // Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its own L2.
    // Renumber so that XCD x runs a contiguous range of (request, tile) ids: a request's
    // tiles then share one L2, and its delta rows and block_lens prefix are fetched once.
    const int32_t nwg = (int32_t)(gridDim.x * gridDim.y);
    const int32_t lin = (int32_t)(blockIdx.y * gridDim.x + blockIdx.x);
    const int32_t xcd = lin & 7, per = nwg >> 3, extra = nwg & 7;
    const int32_t logical = xcd * per + min(xcd, extra) + (lin >> 3);
    const int32_t r = logical / (int32_t)gridDim.x;
    const int32_t cw = (int32_t)(a.C / 2);  // channel pairs per row
    const int32_t P0 = (logical - r * (int32_t)gridDim.x) * kTilePairs;
    const int32_t cp = P0 + wave * 64 + lane;
    const bool live = cp < cw;
    const int32_t cpc = live ? cp : cw - 1;  // clamped: loads stay in bounds
    const uint32_t* x = reinterpret_cast<const uint32_t*>(a.x);
    const uint32_t* base = reinterpret_cast<const uint32_t*>(a.base);
    uint32_t blo[TPP], bhi[TPP];
#pragma unroll
    for (int tp = 0; tp < TPP; ++tp) {
        const uint32_t b0 = 2 * tp < a.taps ? base[(int64_t)(2 * tp) * cw + cpc] : 0u;
        const uint32_t b1 = 2 * tp + 1 < a.taps ? base[(int64_t)(2 * tp + 1) * cw + cpc] : 0u;
        blo[tp] = lo_pair(b0, b1);
        bhi[tp] = hi_pair(b0, b1);
    }
    // first row of request r: prefix of block_lens[0 .. r) (one load round for r < 64)
    int64_t qs = 0;
    for (int32_t b0 = 0; b0 < r; b0 += 64) {
        const int64_t nn = (b0 + lane < r) ? (int64_t)a.block_lens[b0 + lane] : 0;
        qs += shfl_i64(wave_inclusive_scan(nn), 63);
    }
    const int32_t n = a.block_lens[r];
    if (n <= 0)
        return;
    const int32_t per_group = (int32_t)(a.C / a.G);
    const int32_t g_lo = 2 * P0 / per_group;
    const int32_t g_hi = (2 * min(P0 + kTilePairs, cw) - 1) / per_group;
    const int32_t ng = g_hi - g_lo + 1;  // <= tile_groups_max(C, G)
    const int32_t gl0 = 2 * cpc / per_group - g_lo;
    const int32_t gl1 = (2 * cpc + 1) / per_group - g_lo;
    const int32_t lg = ng > 1 ? 32 - __clz(ng - 1) : 0;  // ceil(log2(ng))
    const int32_t dstride = ng * TPP;  // u32 words per staged position
    const uint32_t* d0 = dsh + gl0 * TPP;
    const uint32_t* d1 = dsh + gl1 * TPP;
    uint16_t* dsh16 = reinterpret_cast<uint16_t*>(dsh);
    uint32_t xr[32];
#pragma unroll
    for (int k = 0; k < 16; ++k)
        xr[k] = 0u;  // before the block
    for (int32_t c0 = 0; c0 < n; c0 += kTilePos) {
        const int32_t cnt = min(kTilePos, n - c0);
        const int64_t row0 = qs + c0;
#pragma unroll
        for (int i = 0; i < kTilePos; ++i)
            xr[16 + i] = i < cnt ? x[(row0 + i) * cw + cpc] : 0u;
        if (c0 > 0)
            __syncthreads();  // the previous chunk's delta reads are done
        // delta[row0 + i, t, g_lo + gl] -> dsh16[(i * ng + gl) * TPAD + t].  Element e of the
        // chunk is (gl, t, i) = (e mod 2^lg, (e >> lg) mod TPAD, e >> lg / TPAD), 2^lg >= ng:
        // consecutive threads take consecutive groups (contiguous in memory), and each thread
        // issues 8 loads before it writes any of them.
        const uint16_t* src = a.delta + row0 * a.taps * a.G + g_lo;
        const int32_t total = (kTilePos * TPAD) << lg;
        for (int32_t e0 = 0; e0 < total; e0 += 8 * kTileThreads) {
            uint16_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int32_t e = e0 + u * kTileThreads + (int32_t)threadIdx.x;
                const int32_t gl = e & ((1 << lg) - 1);
                const int32_t t = (e >> lg) % TPAD;
                const int32_t i = (e >> lg) / TPAD;
                v[u] = (e < total && gl < ng && i < cnt && t < a.taps) ? src[(int64_t)(i * a.taps + t) * a.G + gl]
                                                                      : (uint16_t)0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int32_t e = e0 + u * kTileThreads + (int32_t)threadIdx.x;
                const int32_t gl = e & ((1 << lg) - 1);
                if (e < total && gl < ng)
                    dsh16[((e >> lg) / TPAD * ng + gl) * TPAD + (e >> lg) % TPAD] = v[u];
            }
        }
        __syncthreads();
        uint32_t* orow = reinterpret_cast<uint32_t*>(a.out) + row0 * cw + cpc;
        if (c0 == 0)
            conv_chunk<TPP, true>(xr, blo, bhi, d0, d1, dstride, orow, cw, cnt, live);
        else
            conv_chunk<TPP, false>(xr, blo, bhi, d0, d1, dstride, orow, cw, cnt, live);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            xr[k] = xr[16 + k];
    }
}

}  // namespace

hipError_t launch_block_conv(const ConvArgs& a, hipStream_t stream)
{
    const int64_t pairs = a.C / 2;
    if (a.taps <= kTileTaps && tile_groups_max(a.C, a.G) <= kTileGroups && a.B <= 65535 && a.C < (int64_t(1) << 30)) {
        dim3 grid((unsigned)((pairs + kTilePairs - 1) / kTilePairs), (unsigned)a.B);
        const int tpp = a.taps <= 4 ? 2 : a.taps <= 8 ? 4 : 8;
        const size_t lds = sizeof(uint32_t) * kTilePos * tpp * tile_groups_max(a.C, a.G);
        if (tpp == 2)
            hipLaunchKernelGGL(block_conv_tiled_kernel<2>, grid, dim3(kTileThreads), lds, stream, a);
        else if (tpp == 4)
            hipLaunchKernelGGL(block_conv_tiled_kernel<4>, grid, dim3(kTileThreads), lds, stream, a);
        else
            hipLaunchKernelGGL(block_conv_tiled_kernel<8>, grid, dim3(kTileThreads), lds, stream, a);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((pairs + kConvThreads - 1) / kConvThreads), (unsigned)a.total_rows);
    hipLaunchKernelGGL(block_conv_kernel, grid, dim3(kConvThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dflash
