// attn_ref.hip -- the plain VALU block-attention kernel (any head_dim <= 512).
//
// A deliberately simple second implementation next to the MFMA kernel: the
// same work split (decomp.h) and partial format, but scalar fp32 dot products
// and a textbook online softmax, one 16-key tile at a time.  Kept for
// head_dims without an MFMA instantiation and as a cross-check of the fast
// kernel on the GPU.
//
// Semantics: kenforever1 "DFlash + Gemma 4 31B-it" notes, "why non-causal
// attention is needed" (non-causal block over context + block keys; causal =
// self and left); vLLM PR #43445 report (per-request causal flag, sliding
// window).
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace dflash {

constexpr int kRefRows = 16;   // rows per unit
constexpr int kRefTile = 16;   // keys per tile
constexpr int kRefMaxD = 512;
constexpr int kRefThreads = 256;

__global__ __launch_bounds__(kRefThreads) void attn_ref_kernel(AttnArgs a)
{
    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
    __shared__ __attribute__((aligned(16))) uint16_t q_s[kRefRows][kRefMaxD];
    __shared__ __attribute__((aligned(16))) uint16_t k_s[kRefTile][kRefMaxD];
    __shared__ __attribute__((aligned(16))) uint16_t v_s[kRefTile][kRefMaxD];
    __shared__ float z_s[kRefRows][kRefTile];
    __shared__ float alpha_s[kRefRows];
    __shared__ float m_s[kRefRows];
    __shared__ float l_s[kRefRows];
    __shared__ int64_t krow_s[kRefTile];  // element offset of each tile key's row for this kv-head, -1 = none

    const Decomp& d = a.d;
    const int tid = threadIdx.x;
    const int32_t wg = logical_wg(blockIdx.x, d.P);
    const int32_t D = a.D;
    const int32_t G = d.G;
    const int32_t psize = 1 << a.page_shift;

    int64_t total, begin, end;
    RunStart first;
    int64_t qtotal;
    wave_locate_run(a.ctx_lens, a.block_lens, a.causal, d, wg, total, begin, end, first, qtotal);
    if (begin >= end)
        return;
    int32_t r = first.r;
    int64_t rbase = first.rbase, qstart = first.qstart;  // its work and first query token

    int64_t pos = begin;
    int nseg = 0;
    while (pos < end) {
        const int32_t L = a.ctx_lens[r];
        const int32_t n = a.block_lens[r];
        const ReqGeom g = req_geom(L, n, d);
        const int64_t w = req_work(g, d);
        if (pos >= rbase + w) {
            rbase += w;
            qstart += n;
            ++r;
            continue;
        }
        const Segment sg = run_segment(g, rbase, pos, end, d.ov);
        pos = sg.next;
        if (sg.t0 >= sg.t1)
            continue;  // only set-up positions of this unit
        const int32_t unit = sg.unit;
        const int32_t t0 = sg.t0;
        const int32_t t1 = sg.t1;
        const int32_t kvh = unit / g.ngroups;
        const int32_t grp = unit % g.ngroups;
        const int slot = (nseg++ == 0) ? 0 : 1;  // first unit with real tiles in the run: slot 0
        const bool whole = (t0 == 0 && t1 == g.ntiles);
        const bool is_causal = a.causal ? (a.causal[r] != 0) : false;
        const int32_t row0 = grp * d.rmax;
        const int32_t rows_here = min(d.rmax, n * G - row0);

        // ---- Q rows of this unit ----
        for (int c = tid; c < kRefRows * (kRefMaxD / 8); c += kRefThreads) {
            const int rho = c / (kRefMaxD / 8);
            const int part = c % (kRefMaxD / 8);
            uint4 val = make_uint4(0, 0, 0, 0);
            if (rho < rows_here && part * 8 < D) {
                const int32_t rr = row0 + rho;
                const int32_t i = rr / G;
                const int32_t j = rr % G;
                const uint16_t* src = a.q + ((qstart + i) * a.Hq + (int64_t)kvh * G + j) * D + part * 8;
                val = *reinterpret_cast<const uint4*>(src);
            }
            *reinterpret_cast<uint4*>(&q_s[rho][part * 8]) = val;
        }
        if (tid < kRefRows) {
            m_s[tid] = -INFINITY;
            l_s[tid] = 0.f;
        }
        float o[kRefRows][2];
#pragma unroll
        for (int rho = 0; rho < kRefRows; ++rho) {
            o[rho][0] = 0.f;
            o[rho][1] = 0.f;
        }
        __syncthreads();

        for (int32_t t = t0; t < t1; ++t) {
            const int32_t k0 = g.kv_lo + t * kRefTile;
            if (tid < kRefTile) {
                const int32_t key = k0 + tid;
                int64_t rowoff = -1;
                if (key < g.T) {
                    const int64_t page = a.page_table[(int64_t)r * a.max_pages_per_req + (key >> a.page_shift)];
                    rowoff = ((page * psize + (key & (psize - 1))) * d.Hkv + kvh) * (int64_t)D;
                }
                krow_s[tid] = rowoff;
            }
            __syncthreads();
            for (int c = tid; c < kRefTile * (kRefMaxD / 8); c += kRefThreads) {
                const int kk = c / (kRefMaxD / 8);
                const int part = c % (kRefMaxD / 8);
                uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
                const int64_t ro = krow_s[kk];
                if (ro >= 0 && part * 8 < D) {
                    kv = *reinterpret_cast<const uint4*>(a.k_pages + ro + part * 8);
                    vv = *reinterpret_cast<const uint4*>(a.v_pages + ro + part * 8);
                }
                *reinterpret_cast<uint4*>(&k_s[kk][part * 8]) = kv;
                *reinterpret_cast<uint4*>(&v_s[kk][part * 8]) = vv;
            }
            __syncthreads();
            {
                // one (row, key) logit per thread
                const int rho = tid / kRefTile;
                const int kk = tid % kRefTile;
                const int32_t key = k0 + kk;
                float z = -INFINITY;
                if (rho < rows_here && krow_s[kk] >= 0) {
                    const int32_t i = (row0 + rho) / G;
                    int32_t lo, hi;
                    query_range(L, n, i, is_causal, d.window, lo, hi);
                    if (is_causal && a.span_offsets)
                        hi = span_high(a.span_offsets, a.spans, a.num_spans, r, L + i, L + n, hi);
                    if (key >= lo && key <= hi) {
                        float s = 0.f;
                        for (int32_t dd = 0; dd < D; ++dd)
                            s = fmaf(bf16_to_f32(q_s[rho][dd]), bf16_to_f32(k_s[kk][dd]), s);
                        z = s * a.scale_log2;
                    }
                }
                z_s[rho][kk] = z;
            }
            __syncthreads();
            if (tid < kRefRows) {
                float tmax = -INFINITY;
                for (int kk = 0; kk < kRefTile; ++kk)
                    tmax = fmaxf(tmax, z_s[tid][kk]);
                const float m_old = m_s[tid];
                const float m_new = fmaxf(m_old, tmax);
                const float mu = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = exp2f(m_old - mu);
                float sum = 0.f;
                for (int kk = 0; kk < kRefTile; ++kk) {
                    const float p = exp2f(z_s[tid][kk] - mu);
                    z_s[tid][kk] = p;
                    sum += p;
                }
                l_s[tid] = l_s[tid] * alpha + sum;
                m_s[tid] = m_new;
                alpha_s[tid] = alpha;
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int32_t dd = tid + c * kRefThreads;
                if (dd < D) {
#pragma unroll
                    for (int rho = 0; rho < kRefRows; ++rho) {
                        float acc = o[rho][c] * alpha_s[rho];
                        for (int kk = 0; kk < kRefTile; ++kk)
                            acc = fmaf(z_s[rho][kk], bf16_to_f32(v_s[kk][dd]), acc);
                        o[rho][c] = acc;
                    }
                }
            }
            __syncthreads();
        }

        // ---- epilogue ----
        const int64_t sbase = ((int64_t)wg * 2 + slot) * d.rmax;
#pragma unroll
        for (int rho = 0; rho < kRefRows; ++rho) {
            if (rho >= rows_here)
                break;
            const float l = l_s[rho];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const int32_t rr = row0 + rho;
            const int32_t i = rr / G;
            const int32_t j = rr % G;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int32_t dd = tid + c * kRefThreads;
                if (dd < D) {
                    if (whole)
                        a.out[((qstart + i) * a.Hq + (int64_t)kvh * G + j) * D + dd] = f32_to_bf16(o[rho][c] * inv);
                    else
                        a.part_o[(sbase + rho) * a.Dp + dd] = f32_to_bf16(o[rho][c] * inv);
                }
            }
            if (!whole && tid == 0)
                a.part_lse[sbase + rho] = l > 0.f ? m_s[rho] + log2f(l) : -INFINITY;
        }
        __syncthreads();
    }
}

hipError_t launch_attn_ref(const AttnArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(attn_ref_kernel, dim3(a.d.P), dim3(kRefThreads), 0, stream, a);
    return hipGetLastError();
}

int ref_rows_per_unit() { return kRefRows; }

int ref_wgs_per_cu()
{
    static std::atomic<int> cached{-1};  // queried once (one architecture)
    int blocks = cached.load(std::memory_order_acquire);
    if (blocks >= 0)
        return blocks;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_ref_kernel, kRefThreads, 0) != hipSuccess)
        return 0;
    cached.store(blocks, std::memory_order_release);
    return blocks;
}
int ref_tile_keys() { return kRefTile; }

}  // namespace dflash
