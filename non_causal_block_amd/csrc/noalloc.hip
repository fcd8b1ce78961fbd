// noalloc.hip -- dflash_block_attn_noalloc: block attention with the library's own
// static scratch in place of a caller-provided workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The scratch is one file-scope device array per GPU, of kScratchBytes.  Host code never
// passes the array's name to a kernel (in host code it is a host-side stand-in): its
// device address is taken once per device with hipGetSymbolAddress, with that device
// current, and only that address is used.  Every call on a GPU shares the array and the
// array keeps the last call's partials; calls that overlap on one GPU race.  The split
// pieces are merged by the combine kernel, which reads only partial rows the same call
// wrote, so nothing in the scratch has to start at zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>

#include "dflash_block_attn.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(48) << 20;  // covers the head_dim-512 global layer at B = 4 x 9
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the scratch on the current device (looked up once per device).
int scratch_ptr(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return dflash::set_last_error(DFLASH_ERR_HIP, "noalloc: no usable current HIP device");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[256];
            snprintf(msg, sizeof msg, "noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                     hipGetErrorString(e));
            return dflash::set_last_error(DFLASH_ERR_HIP, msg);
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_noalloc_scratch_bytes(void) { return kScratchBytes; }

int dflash_block_attn_noalloc(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                              const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, const uint8_t* causal, int32_t window,
                              float scale, void* out, void* stream, const dflash_batch_desc* desc)
{
    if (!desc)
        return dflash_block_attn(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads, n_kv_heads,
                                 head_dim, causal, window, scale, out, stream, desc);  // reports the NULL desc
    dflash_batch_desc d;
    memcpy(&d, desc, sizeof d);
    d.merge_mode = DFLASH_MERGE_COMBINE_KERNEL;
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    size_t need = 0;
    int st = dflash_block_attn_workspace_size(&d, n_heads, n_kv_heads, head_dim, &need);
    if (st != DFLASH_OK)
        return st;
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "noalloc: this call needs %zu bytes of scratch; the library's static scratch holds %zu "
                 "(use dflash_block_attn with a workspace)", need, kScratchBytes);
        return dflash::set_last_error(DFLASH_ERR_WORKSPACE_TOO_SMALL, msg);
    }
    if (need > 0) {
        void* p = nullptr;
        st = scratch_ptr(&p);
        if (st != DFLASH_OK)
            return st;
        d.workspace = p;
        d.workspace_bytes = kScratchBytes;
    }
    return dflash_block_attn(q, k_pages, v_pages, page_table, ctx_lens, block_lens, n_heads, n_kv_heads, head_dim,
                             causal, window, scale, out, stream, &d);
}

}  // extern "C"
