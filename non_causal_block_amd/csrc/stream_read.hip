// stream_read.hip -- a plain streaming read of a device buffer, the measured
// achievable read bandwidth that block-attention throughput is compared with
// (one pass reads every byte once; nothing else is computed).  It also serves
// as a cache flush: a read-only pass over a buffer several times the size of
// the last-level cache evicts earlier data without leaving dirty lines.
#include "device_common.h"
#include "kernels.h"

namespace dflash {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane

// Workgroup w reads its own contiguous run of 32 KB blocks; in each block wave v
// reads 8 KB (eight 1 KB rows, one 16-byte load per lane per row), so every load
// instruction covers 1 KB of consecutive bytes and a lane keeps eight in flight.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                                     uint32_t* __restrict__ sink)
{
    constexpr size_t kBlock16 = (size_t)kStreamThreads * kStreamUnroll;  // 16-byte units per block
    const size_t nblocks = n16 / kBlock16;
    const size_t per_wg = (nblocks + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per_wg;
    const size_t b1 = b0 + per_wg < nblocks ? b0 + per_wg : nblocks;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (size_t b = b0; b < b1; ++b) {
        const u32x4_t* p = buf + b * kBlock16 + (size_t)wave * 64 * kStreamUnroll + lane;
        u32x4_t x[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            x[u] = __builtin_nontemporal_load(p + 64 * u);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            acc ^= x[u];
    }
    // the tail past the last whole block, spread over the grid
    for (size_t i = nblocks * kBlock16 + (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * kStreamThreads)
        acc ^= __builtin_nontemporal_load(buf + i);
    // XOR of every 32-bit word the wave read, folded into sink[0] by one atomic per
    // wave: the pass cannot be elided and its result checks that each word was read once
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v ^= (uint32_t)__shfl_xor((int)v, off);
    if (lane == 0)
        atomicXor(sink, v);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                       static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace dflash
