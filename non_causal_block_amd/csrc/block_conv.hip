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
// attention).  One thread per (row, channel pair): the workgroup's row locates
// its request, the thread sums taps t = 0 .. min(i, taps-1) in that order in fp32
// (bf16 in, bf16 out, round to nearest even).  The taps' loads are independent,
// and every re-read of x, base and delta across threads is a cache hit.
#include "device_common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kConvThreads = 128;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
    o[row * cw + cp] = (uint32_t)f32_to_bf16(acc0) | ((uint32_t)f32_to_bf16(acc1) << 16);
}

}  // namespace

hipError_t launch_block_conv(const ConvArgs& a, hipStream_t stream)
{
    const int64_t pairs = a.C / 2;
    dim3 grid((unsigned)((pairs + kConvThreads - 1) / kConvThreads), (unsigned)a.total_rows);
    hipLaunchKernelGGL(block_conv_kernel, grid, dim3(kConvThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dflash
