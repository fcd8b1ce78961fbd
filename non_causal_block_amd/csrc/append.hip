// append.hip -- writes each request's block K/V into the paged cache.
//
// The block's own keys sit at positions L .. L+n-1 of request r (L = ctx_lens[r],
// n = block_lens[r]), in the same paged cache as the context: the drafter's
// block queries attend to the context K/V together with the block's K/V
// (kenforever1 "DFlash + Gemma 4 31B-it" notes, "why non-causal attention is
// needed").  Row t of k_new / v_new (rows packed in request order, like q) is
// block token i = t - q_start[r] of request r and lands in page
// page_table[r][(L+i) / page_size], slot (L+i) % page_size.
//
// One wave per (token, kv-head) row: each lane moves one 16-byte chunk of the
// head_dim*2-byte row for K and for V (head_dim <= 512, so one pass).
#include "device_common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kAppendRowsPerWg = 4;  // one wave each

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a)
{
    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kAppendRowsPerWg + wave;
    if (row >= a.total_rows)
        return;
    const int64_t t = row / a.Hkv;
    const int32_t h = (int32_t)(row % a.Hkv);
    int32_t r;
    int64_t qstart;
    wave_find_token(a.block_lens, a.B, t, r, qstart);
    if (r >= a.B)
        return;  // a row past the last block token
    const int32_t pos = a.ctx_lens[r] + (int32_t)(t - qstart);
    const int32_t page = a.page_table[(int64_t)r * a.max_pages_per_req + (pos >> a.page_shift)];
    const int64_t slot = (int64_t)page * (1 << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
    const int64_t dst = (slot * a.Hkv + h) * a.D;
    const int64_t src = (t * a.Hkv + h) * a.D;
    if (lane < a.D / 8) {
        const u32x4_t k = *reinterpret_cast<const u32x4_t*>(a.k_new + src + 8 * lane);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.v_new + src + 8 * lane);
        *reinterpret_cast<u32x4_t*>(a.k_pages + dst + 8 * lane) = k;
        *reinterpret_cast<u32x4_t*>(a.v_pages + dst + 8 * lane) = v;
    }
}

}  // namespace

int append_grid(int64_t total_rows)
{
    return (int)((total_rows + kAppendRowsPerWg - 1) / kAppendRowsPerWg);
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_append_kernel, dim3(append_grid(a.total_rows)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dflash
