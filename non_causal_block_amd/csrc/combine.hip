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
    const int64_t us = rbase + (int64_t)unit * g.uwork;
    int64_t kf, kl;
    unit_pieces(g, us, d.ov, tpw, kf, kl);
    if (kf == kl)
        return;  // finished inside one workgroup, already written

    // piece weights, lane-parallel: lane j holds piece kf + j (+ 64 per round)
    const int64_t npieces = kl - kf + 1;
    float M = -INFINITY;
    for (int64_t base = 0; base < npieces; base += 64) {
        const int64_t k = kf + base + lane;
        if (k <= kl) {
            const int slot = piece_slot(k, us, tpw);
            M = fmaxf(M, a.part_lse[(k * 2 + slot) * d.rmax + rin]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        M = fmaxf(M, __shfl_xor(M, off));

    const int32_t d0 = lane * 8;
    const bool dlive = d0 < a.D;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    float W = 0.f;
    for (int64_t base = 0; base < npieces; base += 64) {
        const int64_t kq = kf + base + lane;
        float wl = 0.f;
        if (kq <= kl) {
            const int slot = piece_slot(kq, us, tpw);
            const float lse = a.part_lse[(kq * 2 + slot) * d.rmax + rin];
            wl = (lse == -INFINITY) ? 0.f : exp2f(lse - M);
        }
        W += wl;
        const int cnt = (int)min<int64_t>(64, npieces - base);
        // four pieces per step keep eight 16-byte loads of each lane in flight
        for (int j0 = 0; j0 < cnt; j0 += 4) {
            float wj[4];
            float4 x0[4], x1[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = min(j0 + u, cnt - 1);
                wj[u] = (j0 + u < cnt) ? __shfl(wl, j) : 0.f;
                const int64_t k = kf + base + j;
                const int slot = piece_slot(k, us, tpw);
                const int64_t prow = (k * 2 + slot) * d.rmax + rin;
                if (dlive && wj[u] != 0.f) {
                    const float4* src = reinterpret_cast<const float4*>(a.part_o + prow * a.Dp + d0);
                    x0[u] = src[0];
                    x1[u] = src[1];
                } else {
                    x0[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                    x1[u] = x0[u];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[0] = fmaf(wj[u], x0[u].x, acc[0]);
                acc[1] = fmaf(wj[u], x0[u].y, acc[1]);
                acc[2] = fmaf(wj[u], x0[u].z, acc[2]);
                acc[3] = fmaf(wj[u], x0[u].w, acc[3]);
                acc[4] = fmaf(wj[u], x1[u].x, acc[4]);
                acc[5] = fmaf(wj[u], x1[u].y, acc[5]);
                acc[6] = fmaf(wj[u], x1[u].z, acc[6]);
                acc[7] = fmaf(wj[u], x1[u].w, acc[7]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        W += __shfl_xor(W, off);
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
