// combine.hip -- merges split-KV partial results into the bf16 output.
//
// A unit (request, kv-head, row group) whose key tiles were spread over
// several attention workgroups left one partial per workgroup: the output
// normalised by its own softmax sum, o_s, and lse_s = log2 of that sum in
// the shifted scaled-log2 domain the kernels use.  The exact result is the
// sum-weighted mean
//     out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M),   M = max_s lse_s,
// with pieces that saw no visible key (lse = -inf) weighing zero.  The
// FlashAttention split-KV combine is the prior art named in vLLM PR #52816's
// review (prhub summary, "review highlights"); this one is written for the
// 9..72 query rows and head_dim up to 512 of a DFlash step: one wave per
// output row, 8 consecutive head-dim elements per lane.
#include "device_common.h"
#include "kernels.h"

namespace dflash {

constexpr int kCombineRowsPerWg = 4;  // one wave each

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const Decomp& d = a.d;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kCombineRowsPerWg + wave;
    if (row >= a.total_rows)
        return;
    const int64_t t = row / a.Hq;
    const int32_t h = (int32_t)(row % a.Hq);

    int32_t r;
    int64_t qstart;
    wave_find_token(a.block_lens, d.B, t, r, qstart);
    if (r >= d.B)
        return;  // token past the real total
    const int32_t L = a.ctx_lens[r];
    const int32_t n = a.block_lens[r];
    const ReqGeom g = req_geom(L, n, d);
    const int64_t total = wave_total_work(a.ctx_lens, a.block_lens, d);
    const int64_t tpw = tiles_per_wg(total, d.P);
    const int64_t rbase = wave_work_before(a.ctx_lens, a.block_lens, d, r);

    const int32_t i = (int32_t)(t - qstart);
    const int32_t kvh = h / d.G;
    const int32_t j = h % d.G;
    const int32_t rowreq = i * d.G + j;
    const int32_t grp = rowreq / d.rmax;
    const int32_t rin = rowreq % d.rmax;
    const int32_t unit = kvh * g.ngroups + grp;
    const int64_t us = rbase + (int64_t)unit * g.ntiles;
    const int64_t ue = us + g.ntiles;
    const int64_t kf = us / tpw;
    const int64_t kl = (ue - 1) / tpw;
    if (kf == kl)
        return;  // finished inside one workgroup, already written

    float M = -INFINITY;
    for (int64_t k = kf; k <= kl; ++k) {
        const int slot = (k == kf && us != k * tpw) ? 1 : 0;
        M = fmaxf(M, a.part_lse[(k * 2 + slot) * d.rmax + rin]);
    }
    const int32_t d0 = lane * 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    float W = 0.f;
    for (int64_t k = kf; k <= kl; ++k) {
        const int slot = (k == kf && us != k * tpw) ? 1 : 0;
        const int64_t prow = (k * 2 + slot) * d.rmax + rin;
        const float lse = a.part_lse[prow];
        const float w = (lse == -INFINITY) ? 0.f : exp2f(lse - M);
        W += w;
        if (d0 < a.D && w != 0.f) {
            const float4* src = reinterpret_cast<const float4*>(a.part_o + prow * a.Dp + d0);
            const float4 x0 = src[0];
            const float4 x1 = src[1];
            acc[0] = fmaf(w, x0.x, acc[0]);
            acc[1] = fmaf(w, x0.y, acc[1]);
            acc[2] = fmaf(w, x0.z, acc[2]);
            acc[3] = fmaf(w, x0.w, acc[3]);
            acc[4] = fmaf(w, x1.x, acc[4]);
            acc[5] = fmaf(w, x1.y, acc[5]);
            acc[6] = fmaf(w, x1.z, acc[6]);
            acc[7] = fmaf(w, x1.w, acc[7]);
        }
    }
    if (d0 < a.D) {
        const float inv = W > 0.f ? 1.f / W : 0.f;
        uint16_t* dst = a.out + (t * a.Hq + h) * (int64_t)a.D + d0;
        uint4 packed;
        packed.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
        packed.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
        packed.z = (uint32_t)f32_to_bf16(acc[4] * inv) | ((uint32_t)f32_to_bf16(acc[5] * inv) << 16);
        packed.w = (uint32_t)f32_to_bf16(acc[6] * inv) | ((uint32_t)f32_to_bf16(acc[7] * inv) << 16);
        *reinterpret_cast<uint4*>(dst) = packed;
    }
}

int combine_grid(int64_t total_rows)
{
    return (int)((total_rows + kCombineRowsPerWg - 1) / kCombineRowsPerWg);
}

hipError_t launch_combine(const CombineArgs& a, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dflash
