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
constexpr int kPiecesPerStep = 16;   // partial rows requested together by each lane

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
    const Decomp& d = a.d;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kCombineRowsPerWg + wave;
    if (row >= a.total_rows)
        return;
    const int64_t t = row / a.Hq;
    const int32_t h = (int32_t)(row % a.Hq);

    int32_t r;
    int64_t qstart, rbase, total;
    wave_locate_token(a.ctx_lens, a.block_lens, d, t, r, qstart, rbase, total);
    if (r >= d.B)
        return;  // token past the real total
    const int32_t L = a.ctx_lens[r];
    const int32_t n = a.block_lens[r];
    const ReqGeom g = req_geom(L, n, d);
    const int64_t tpw = tiles_per_wg(total, d.P);

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

    // Lane j holds piece kf + j (+ 64 per round).  The log-sum-exps and the partial rows
    // are requested together (rows of pieces that saw no key hold zeros, so they need no
    // guard), and the weights are formed once everything has arrived.
    const int64_t npieces = kl - kf + 1;
    const int32_t d0 = lane * 8;
    const bool dlive = d0 < a.D;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    float M = -INFINITY;
    float W = 0.f;
    for (int64_t base = 0; base < npieces; base += 64) {
        const int64_t kq = kf + base + lane;
        const float lse = kq <= kl ? a.part_lse[(kq * 2 + piece_slot(kq, us, tpw)) * d.rmax + rin] : -INFINITY;
        const int cnt = (int)min<int64_t>(64, npieces - base);
        float wl = 0.f;
        for (int j0 = 0; j0 < cnt; j0 += kPiecesPerStep) {
            uint4 x[kPiecesPerStep];
#pragma unroll
            for (int u = 0; u < kPiecesPerStep; ++u) {
                const int jj = min(j0 + u, cnt - 1);
                const int64_t k = kf + base + jj;
                const int64_t prow = (k * 2 + piece_slot(k, us, tpw)) * d.rmax + rin;
                x[u] = (dlive && j0 + u < cnt) ? *reinterpret_cast<const uint4*>(a.part_o + prow * a.Dp + d0)
                                               : make_uint4(0, 0, 0, 0);
            }
            if (j0 == 0) {
                // weights of this round, formed while the rows above are in flight; what
                // earlier rounds summed (more than 64 pieces only) is rescaled to the new max
                float mr = lse;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1)
                    mr = fmaxf(mr, __shfl_xor(mr, off));
                const float m_new = fmaxf(M, mr);
                if (base > 0 && m_new > M) {
                    const float sc = exp2f(M - m_new);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[e] *= sc;
                    W *= sc;
                }
                M = m_new;
                wl = (lse == -INFINITY) ? 0.f : exp2f(lse - M);
                W += wl;
            }
#pragma unroll
            for (int u = 0; u < kPiecesPerStep; ++u) {
                const float wj = (j0 + u < cnt) ? __shfl(wl, min(j0 + u, cnt - 1)) : 0.f;
                const uint32_t w4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // bf16 -> fp32 is exact: the bits move to the high half
                    acc[2 * e] = fmaf(wj, __uint_as_float(w4[e] << 16), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(wj, __uint_as_float(w4[e] & 0xffff0000u), acc[2 * e + 1]);
                }
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
