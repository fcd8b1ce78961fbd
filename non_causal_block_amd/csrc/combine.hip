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
// 9..72 query rows and head_dim up to 512 of a DFlash step, 8 consecutive
// head-dim elements per lane.  combine_kernel gives an output row 16, 32 or 64
// lanes of a wave; combine_row_kernel gives a row a whole workgroup, its four
// waves taking every fourth piece, for units split many ways at head_dim 512.
#include "device_common.h"
#include "kernels.h"
#include "merge.h"

namespace dflash {

constexpr int kCombineWavesPerWg = 4;

// PPS: partial rows each lane requests together.  More rows in flight pay one latency
// for a unit split many ways; fewer keep the registers low enough for many resident
// waves when there are many rows and few pieces each.
// LPR: lanes per output row (8 head-dim elements each): 64 / LPR rows share a wave,
// so head_dim 128 or 256 does not leave most lanes idle.  All rows of a wave belong
// to one token (the planner uses LPR < 64 only when Hq is a multiple of 64 / LPR).
template <int PPS, int LPR>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    constexpr int RPW = 64 / LPR;
    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
    const Decomp& d = a.d;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rg = lane / LPR;  // row of this lane within the wave
    const int sl = lane % LPR;  // lane within the row's group
    const int64_t row0 = ((int64_t)blockIdx.x * kCombineWavesPerWg + wave) * RPW;
    if (row0 >= a.total_rows)
        return;
    const int64_t t = row0 / a.Hq;
    const int32_t h = (int32_t)(row0 % a.Hq) + rg;

    int64_t kf, np, us, tpw;
    int32_t rin;
    if (a.dir) {
        // the attention kernel's directory: pieces kf .. kf+np-1; piece_slot(k, kf + slot0, 1)
        // then gives the first piece's slot and slot 0 for the later ones
        const DirEntry e = dir_unpack(a.dir[row0 + rg]);
        kf = e.kf;
        np = e.kf + e.np <= d.P ? e.np : 0;  // (always within the grid for this call's entries)
        us = kf + e.slot0;
        tpw = 1;
        rin = e.rin;
    } else {
        int32_t r;
        int64_t qstart, rbase, total;
        wave_locate_token(a.ctx_lens, a.block_lens, d, t, r, qstart, rbase, total);
        if (r >= d.B)
            return;  // token past the real total
        const int32_t L = a.ctx_lens[r];
        const int32_t n = a.block_lens[r];
        const ReqGeom g = req_geom(L, n, d);
        tpw = tiles_per_wg(total, d.P);

        const int32_t i = (int32_t)(t - qstart);
        const int32_t kvh = h / d.G;
        const int32_t j = h % d.G;
        const int32_t rowreq = i * d.G + j;
        const int32_t grp = rowreq / d.rmax;
        rin = rowreq % d.rmax;
        const int32_t unit = kvh * g.ngroups + grp;
        us = rbase + (int64_t)unit * g.uwork;
        int64_t kl;
        unit_pieces(g, us, d.ov, tpw, kf, kl);
        np = kl - kf + 1;
    }
    // a unit finished inside one workgroup is already written; its lanes only take
    // part in the wave's shuffles
    const bool split = np > 1;
    if (!__any(split))
        return;
    const int64_t npieces = split ? np : 0;
    // loop bounds common to the wave (one row per wave: already uniform)
    int64_t max_np = npieces;
    if constexpr (RPW > 1) {
#pragma unroll
        for (int off = 32; off >= LPR; off >>= 1)
            max_np = max(max_np, shfl_i64(max_np, lane ^ off));
    }

    const int32_t d0 = sl * 8;
    const bool dlive = split && d0 < a.D;
    float acc[8];
    const float W = merge_pieces<LPR, PPS>(a.part_o, a.part_lse, d.rmax, a.Dp, kf, npieces, max_np, us, tpw, rin,
                                           split, dlive, d0, acc);
    if (dlive)
        store_merged(a.out + (t * a.Hq + h) * (int64_t)a.D + d0, acc, W);
}

// One output row per workgroup, its pieces dealt over the four waves (wave w takes
// pieces w, w + 4, ...), for head_dim up to 512 (64 lanes x 8 elements).  A unit split
// many ways (16 to 30 pieces at the long-context head_dim-512 shapes) then needs one
// load round per wave instead of two for a single wave; the four partial sums, each
// with its own running max, meet in LDS and wave 0 writes the row.
// DIRK: the row's pieces come from the attention kernel's merge directory (a.dir), else
// from the request arrays.  Both instances are held to at most 96 registers (5 waves per
// SIMD; the directory instance needs 70), so that at least 1280 workgroups fit on the
// chip at once (C3's 1152 rows): at 4 waves per SIMD the last rows wait for a second
// round (C3's call 1.7 us slower, A/B on one box).
template <int PPS, bool DIRK>
__global__ __launch_bounds__(256, 5) void combine_row_kernel(CombineArgs a)
{
    constexpr int NW = kCombineWavesPerWg;
    __shared__ float s_m[NW], s_w[NW];
    __shared__ float s_acc[NW - 1][8][64];
    if (a.dbg && *a.dbg != 0u)
        return;  // debug checks found a bad device-side value: touch nothing
    const Decomp& d = a.d;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = blockIdx.x;  // the grid has exactly total_rows workgroups
    const int64_t t = row / a.Hq;
    const int32_t h = (int32_t)(row % a.Hq);

    int64_t kf, np, us, tpw;
    int32_t rin;
    if constexpr (DIRK) {
        // pieces kf .. kf+np-1; piece_slot(k, kf + slot0, 1) then gives the first piece's
        // slot and slot 0 for the later ones
        const DirEntry e = dir_unpack(a.dir[row]);
        if (e.np <= 1 || e.kf + e.np > d.P)
            return;  // no request's row, or finished whole (always within the grid)
        kf = e.kf;
        np = e.np;
        us = kf + e.slot0;
        tpw = 1;
        rin = e.rin;
    } else {
        int32_t r;
        int64_t qstart, rbase, total;
        wave_locate_token(a.ctx_lens, a.block_lens, d, t, r, qstart, rbase, total);
        if (r >= d.B)
            return;  // token past the real total (the same for every wave of the workgroup)
        const int32_t L = a.ctx_lens[r];
        const int32_t n = a.block_lens[r];
        const ReqGeom g = req_geom(L, n, d);
        tpw = tiles_per_wg(total, d.P);
        const int32_t rowreq = (int32_t)(t - qstart) * d.G + h % d.G;
        rin = rowreq % d.rmax;
        const int32_t unit = (h / d.G) * g.ngroups + rowreq / d.rmax;
        us = rbase + (int64_t)unit * g.uwork;
        int64_t kl;
        unit_pieces(g, us, d.ov, tpw, kf, kl);
        if (kf == kl)
            return;  // finished inside one attention workgroup: already written
        np = kl - kf + 1;
    }
    const int64_t cnt = np > wave ? (np - wave + NW - 1) / NW : 0;  // this wave's pieces
    const int32_t d0 = lane * 8;
    const bool dlive = d0 < a.D;
    auto prow = [&](int64_t m) {  // partial row of the wave's m-th piece
        const int64_t k = kf + wave + (int64_t)NW * m;
        return (k * 2 + piece_slot(k, us, tpw)) * d.rmax + rin;
    };

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    float M = -INFINITY;
    float W = 0.f;
    for (int64_t base = 0; base < cnt; base += 64) {
        const int64_t mq = base + lane;  // lane mq holds the log-sum-exp of piece mq
        const float lse = mq < cnt ? a.part_lse[prow(mq)] : -INFINITY;
        const int c = (int)min<int64_t>(64, cnt - base);
        float wl = 0.f;
        for (int j0 = 0; j0 < c; j0 += PPS) {
            uint4 x[PPS];
#pragma unroll
            for (int u = 0; u < PPS; ++u)
                x[u] = (dlive && j0 + u < c) ? *reinterpret_cast<const uint4*>(a.part_o + prow(base + j0 + u) * a.Dp + d0)
                                             : make_uint4(0, 0, 0, 0);
            if (j0 == 0) {
                // weights of this round, formed while its rows are in flight; what earlier
                // rounds summed (more than 64 pieces per wave only) moves to the new max
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
            for (int u = 0; u < PPS; ++u) {
                const float wsh = __shfl(wl, min(j0 + u, 63));
                const float wj = (j0 + u < c) ? wsh : 0.f;
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
    if (lane == 0) {
        s_m[wave] = M;  // -inf for a wave with no pieces (its W and acc are 0)
        s_w[wave] = W;
    }
    if (wave > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s_acc[wave - 1][e][lane] = acc[e];
    }
    __syncthreads();
    if (wave != 0)
        return;
    // at least one piece saw a key (every query sees itself), so the common max is finite
    float Mt = s_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        Mt = fmaxf(Mt, s_m[w]);
    const float sc0 = M == -INFINITY ? 0.f : exp2f(M - Mt);
    float tot = sc0 * W;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] *= sc0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float sc = s_m[w] == -INFINITY ? 0.f : exp2f(s_m[w] - Mt);
        tot = fmaf(sc, s_w[w], tot);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = fmaf(sc, s_acc[w - 1][e][lane], acc[e]);
    }
    if (dlive) {
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        uint16_t* dst = a.out + (t * a.Hq + h) * (int64_t)a.D + d0;
        uint4 packed;
        packed.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
        packed.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
        packed.z = (uint32_t)f32_to_bf16(acc[4] * inv) | ((uint32_t)f32_to_bf16(acc[5] * inv) << 16);
        packed.w = (uint32_t)f32_to_bf16(acc[6] * inv) | ((uint32_t)f32_to_bf16(acc[7] * inv) << 16);
        *reinterpret_cast<uint4*>(dst) = packed;
    }
}

hipError_t launch_combine_rows(const CombineArgs& a, hipStream_t stream)
{
    if (a.total_rows <= 0 || a.total_rows > 0x7fffffff || a.Dp > 512)
        return hipErrorInvalidValue;
    if (a.dir)
        hipLaunchKernelGGL((combine_row_kernel<8, true>), dim3((unsigned)a.total_rows), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((combine_row_kernel<8, false>), dim3((unsigned)a.total_rows), dim3(256), 0, stream, a);
    return hipGetLastError();
}

int combine_lanes_per_row(int dpad, int32_t n_heads)
{
    const int lpr = dpad <= 128 ? 16 : dpad <= 256 ? 32 : 64;
    return n_heads % (64 / lpr) == 0 ? lpr : 64;
}

int combine_grid(int64_t total_rows, int lanes_per_row)
{
    const int64_t rows_per_wg = (int64_t)kCombineWavesPerWg * (64 / lanes_per_row);
    return (int)((total_rows + rows_per_wg - 1) / rows_per_wg);
}

template <int LPR>
static hipError_t launch_lpr(const CombineArgs& a, int grid, int pps, hipStream_t stream)
{
    switch (pps) {
    case 4: hipLaunchKernelGGL((combine_kernel<4, LPR>), dim3(grid), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((combine_kernel<8, LPR>), dim3(grid), dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((combine_kernel<16, LPR>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int grid, int pieces_per_step, int lanes_per_row, hipStream_t stream)
{
    switch (lanes_per_row) {
    case 16: return launch_lpr<16>(a, grid, pieces_per_step, stream);
    case 32: return launch_lpr<32>(a, grid, pieces_per_step, stream);
    case 64: return launch_lpr<64>(a, grid, pieces_per_step, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dflash
