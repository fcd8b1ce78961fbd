// debug_checks.hip -- optional checks of the device-side values a call relies on.
//
// Page ids, lengths and span offsets live in device memory, so the host cannot
// validate them; out-of-range values are undefined behaviour on the fast path.
// With debug checks on, a one-workgroup kernel checks them first and records any
// failure in a sticky state word; every later kernel of the call reads that word
// and does nothing when it is set, so a bad page id is never dereferenced.
#include <limits.h>

#include "device_common.h"
#include "kernels.h"

namespace dflash {

// [0]: error bits (DFLASH_DEBUG_* in the public header), [1]: lowest failing request.
__device__ __align__(16) uint32_t g_debug_state[4] = {0u, (uint32_t)INT_MAX, 0u, 0u};

constexpr int kValidateThreads = 256;

__global__ __launch_bounds__(kValidateThreads) void validate_kernel(ValidateArgs a)
{
    __shared__ uint32_t s_bits[kValidateThreads / 64];
    __shared__ int32_t s_bad[kValidateThreads / 64];
    __shared__ long long s_q[kValidateThreads / 64];
    __shared__ long long s_kv[kValidateThreads / 64];
    const int tid = threadIdx.x;
    uint32_t bits = 0;
    int32_t bad = INT_MAX;
    int64_t qsum = 0, kvsum = 0;
    for (int32_t r = tid; r < a.B; r += kValidateThreads) {
        const int32_t L = a.ctx_lens[r];
        const int32_t n = a.block_lens[r];
        uint32_t b = 0;
        if (L < 0 || n < 0) {
            b |= 1u;
        } else {
            const int64_t T = (int64_t)L + n;
            qsum += n;
            kvsum += T;
            if (a.max_block_len > 0 && n > a.max_block_len)
                b |= 16u;
            if (T > (int64_t)a.max_pages_per_req * a.page_size) {
                b |= 2u;
            } else if (n > 0) {
                // the pages a kernel of the call reads or writes: from the first key the
                // attention reads (or the block start for an append alone) to the last key
                int64_t lo = 0;
                if (a.from_block) {
                    lo = L;
                } else {
                    if (a.window > 0)
                        lo = L - a.window + 1 > 0 ? L - a.window + 1 : 0;
                    lo = lo / a.tile_keys * a.tile_keys;
                }
                const int64_t p0 = lo / a.page_size;
                const int64_t p1 = (T + a.page_size - 1) / a.page_size;
                const int32_t* row = a.page_table + (int64_t)r * a.max_pages_per_req;
                for (int64_t j = p0; j < p1; ++j) {
                    const int32_t p = row[j];
                    if (p < 0 || (int64_t)p >= a.num_pages) {
                        b |= 4u;
                        break;
                    }
                }
            }
        }
        if (a.span_offsets) {
            const int32_t o0 = a.span_offsets[r], o1 = a.span_offsets[r + 1];
            if (o0 < 0 || o1 < o0 || o1 > a.num_spans)
                b |= 32u;
        }
        if (b) {
            bits |= b;
            bad = min(bad, r);
        }
    }
    // workgroup reduction: wave shuffles, then one value per wave through LDS
    for (int off = 32; off >= 1; off >>= 1) {
        bits |= (uint32_t)__shfl_xor((int)bits, off);
        bad = min(bad, __shfl_xor(bad, off));
        qsum += shfl_i64(qsum, (threadIdx.x & 63) ^ off);
        kvsum += shfl_i64(kvsum, (threadIdx.x & 63) ^ off);
    }
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
        s_bits[wave] = bits;
        s_bad[wave] = bad;
        s_q[wave] = qsum;
        s_kv[wave] = kvsum;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kValidateThreads / 64; ++w) {
            bits |= s_bits[w];
            bad = min(bad, s_bad[w]);
            qsum += s_q[w];
            kvsum += s_kv[w];
        }
        if (qsum != a.total_q)
            bits |= 8u;
        if (a.total_kv_len > 0 && kvsum > a.total_kv_len)
            bits |= 16u;
        if (bits) {
            atomicOr(&a.state[0], bits);
            atomicMin(reinterpret_cast<int*>(&a.state[1]), bad == INT_MAX ? a.B : bad);
        }
    }
}

hipError_t debug_state_ptr(uint32_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    constexpr int kMaxDev = 64;
    static uint32_t* cache[kMaxDev] = {};
    if (dev >= 0 && dev < kMaxDev && __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE)) {
        *out = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
        return hipSuccess;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_state));
    if (e != hipSuccess)
        return e;
    if (dev >= 0 && dev < kMaxDev)
        __atomic_store_n(&cache[dev], static_cast<uint32_t*>(p), __ATOMIC_RELEASE);
    *out = static_cast<uint32_t*>(p);
    return hipSuccess;
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kValidateThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dflash
