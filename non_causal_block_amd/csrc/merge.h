// merge.h -- the split-KV merge of one output row, shared by the standalone
// combine kernel (combine.hip) and the in-kernel merge of the MFMA attention
// kernel (attn_mfma_kernel.h).
//
// A unit (request, kv-head, row group) whose key tiles were spread over
// several attention workgroups left one partial per workgroup: the output
// normalised by its own softmax sum, o_s (bf16), and lse_s = log2 of that sum
// in the shifted scaled-log2 domain the kernels use (fp32).  The exact result
// is the sum-weighted mean
//     out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M),   M = max_s lse_s,
// with pieces that saw no visible key (lse = -inf, o = 0) weighing zero: softmax
// over a union of disjoint key sets.  The FlashAttention split-KV combine is the
// prior art named in vLLM PR #52816's review (prhub summary, "review
// highlights").
#pragma once

#include "device_common.h"

namespace dflash {

// Partial row of piece k (workgroup k's slot) for row `rin` of the unit whose flat
// range starts at `us`; rows of a slot are rmax apart, slots of a workgroup 2*rmax.
__device__ __forceinline__ int64_t partial_row(int64_t k, int64_t us, int64_t tpw, int32_t rmax, int32_t rin)
{
    return (k * 2 + piece_slot(k, us, tpw)) * rmax + rin;
}

// Merges pieces kf .. kf+np-1 of one row per LPR-lane group of the wave: lane sl of a
// group accumulates head-dim elements [8 sl, 8 sl + 8) into acc (fp32, relative to the
// running max) and the group's total weight is returned.  Lane sl also holds piece
// base + sl's log-sum-exp in each round of LPR pieces; the rows of a round are requested
// PPS at a time, together with (and before the use of) the round's log-sum-exps, so the
// weights are formed while the rows are in flight.  `max_np` is the largest np of the
// wave's groups (loop bounds must be wave-uniform); rows with np = 0 or !live take part
// in the shuffles only.  `dlive`: this lane's 8 elements exist (d0 < head_dim).
// 16 bytes at an agent-coherent point: two 8-byte relaxed atomic accesses at agent
// scope, which gfx950 performs past the per-XCD L2 (no cache maintenance needed).
__device__ __forceinline__ void store16_coherent(void* dst, uint4 x)
{
    uint64_t* p = reinterpret_cast<uint64_t*>(dst);
    __hip_atomic_store(p, ((uint64_t)x.y << 32) | x.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, ((uint64_t)x.w << 32) | x.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 load16_coherent(const void* src)
{
    const uint64_t* p = reinterpret_cast<const uint64_t*>(src);
    const uint64_t a = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}

__device__ __forceinline__ float load_f32_coherent(const float* src)
{
    return __uint_as_float(
        __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ void store_f32_coherent(float* dst, float v)
{
    __hip_atomic_store(reinterpret_cast<uint32_t*>(dst), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// COH: the partials were written in this same kernel by other workgroups and are read
// with coherent loads; otherwise (a later kernel) with plain ones.
template <int LPR, int PPS, bool COH = false>
__device__ __forceinline__ float merge_pieces(const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
                                              int32_t rmax, int32_t Dp, int64_t kf, int64_t np, int64_t max_np,
                                              int64_t us, int64_t tpw, int32_t rin, bool live, bool dlive, int32_t d0,
                                              float (&acc)[8])
{
    const int lane = threadIdx.x & 63;
    const int sl = lane % LPR;
    const int gbase = lane - sl;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.f;
    float M = -INFINITY;
    float W = 0.f;
    for (int64_t base = 0; base < max_np; base += LPR) {
        const int64_t kq = kf + base + sl;
        float lse = -INFINITY;
        if (live && base + sl < np) {
            const float* src = part_lse + partial_row(kq, us, tpw, rmax, rin);
            lse = COH ? load_f32_coherent(src) : *src;
        }
        const int cnt = live ? (int)max<int64_t>(0, min<int64_t>(LPR, np - base)) : 0;
        int max_cnt = cnt;
        if constexpr (LPR < 64) {
#pragma unroll
            for (int off = 32; off >= LPR; off >>= 1)
                max_cnt = max(max_cnt, __shfl_xor(max_cnt, off));
        }
        float wl = 0.f;
        for (int j0 = 0; j0 < max_cnt; j0 += PPS) {
            uint4 x[PPS];
#pragma unroll
            for (int u = 0; u < PPS; ++u) {
                const int64_t k = kf + base + j0 + u;
                x[u] = make_uint4(0, 0, 0, 0);
                if (dlive && live && j0 + u < cnt) {
                    const uint16_t* src = part_o + partial_row(k, us, tpw, rmax, rin) * Dp + d0;
                    x[u] = COH ? load16_coherent(src) : *reinterpret_cast<const uint4*>(src);
                }
            }
            if (j0 == 0) {
                // weights of this round, formed while the rows above are in flight; what
                // earlier rounds summed (more than LPR pieces only) moves to the new max
                float mr = lse;
#pragma unroll
                for (int off = LPR / 2; off >= 1; off >>= 1)
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
                const int src = gbase + min(j0 + u, LPR - 1);
                const float wsh = __shfl(wl, src);
                const float wj = (j0 + u < cnt) ? wsh : 0.f;
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
    for (int off = LPR / 2; off >= 1; off >>= 1)
        W += __shfl_xor(W, off);
    return W;
}

// acc / W rounded to bf16 (round to nearest even), 16 bytes at dst.
__device__ __forceinline__ void store_merged(uint16_t* dst, const float (&acc)[8], float W)
{
    const float inv = W > 0.f ? 1.f / W : 0.f;
    uint4 packed;
    packed.x = (uint32_t)f32_to_bf16(acc[0] * inv) | ((uint32_t)f32_to_bf16(acc[1] * inv) << 16);
    packed.y = (uint32_t)f32_to_bf16(acc[2] * inv) | ((uint32_t)f32_to_bf16(acc[3] * inv) << 16);
    packed.z = (uint32_t)f32_to_bf16(acc[4] * inv) | ((uint32_t)f32_to_bf16(acc[5] * inv) << 16);
    packed.w = (uint32_t)f32_to_bf16(acc[6] * inv) | ((uint32_t)f32_to_bf16(acc[7] * inv) << 16);
    *reinterpret_cast<uint4*>(dst) = packed;
}

// ---- in-kernel merge: counters in the caller's workspace ----------------------------
//
// A split unit is named by its first workgroup kf (at most one split unit starts in
// any run).  Each piece's workgroup publishes its partial with coherent stores, waits
// until they have completed (vmcnt 0), and counts itself in the unit's arrival word
// (low 16 bits; an atomic add whose old value tells the unit's last arrival).  The
// unit's merge items -- the rows one wave merges at once -- are dealt to its pieces in
// turn: piece j (workgroup kf + j) merges items j, j + np, j + 2 np, ...  A piece whose
// workgroup is not the last arrival waits for the unit to complete and then merges its
// items; the last arrival merges its own at once.  Nothing in the grid waits without a
// bound: a piece whose wait runs out (kMergeWaitTicks -- possible only when the grid
// does not fit on the chip at once) raises its give-up flag and registers itself in
// the arrival word's high bits with a compare-and-swap that succeeds only while the
// unit is incomplete; the last arrival, whose add returns those registrations, then
// merges the items of every piece that gave up.  (A piece whose registration lost the
// race to the completion merges its items itself; the last arrival may then merge them
// too, writing the same bits.)  When a piece is done with the unit it counts itself in
// the unit's departure word; the last to leave clears the unit's words, which nothing
// of this call reads again, for the next call.  No cache maintenance is needed: every
// access to published data or counters is coherent at agent scope.

constexpr long long kMergeWaitTicks = 5000;  // 50 us of the 100 MHz constant clock
constexpr uint32_t kArriveMask = 0xffffu;     // arrivals; give-ups are counted above
constexpr uint32_t kGiveUp = 0x10000u;

// Counter layout (int32 words at the start of the workspace), the same for every grid
// size so that partials of one call never land on counters of another call that shares
// the workspace: [kCtrArrive + k] arrival word and [kCtrDepart + k] departure count of
// the unit whose first workgroup is k, [kCtrGaveUp + 2 k + s] give-up flag of workgroup
// k's slot s.  Grids of more than kMergeMaxWgs workgroups use the separate combine
// kernel.
constexpr int32_t kMergeMaxWgs = 16384;
constexpr int32_t kCtrArrive = 64;
constexpr int32_t kCtrDepart = kCtrArrive + kMergeMaxWgs;
constexpr int32_t kCtrGaveUp = kCtrDepart + kMergeMaxWgs;
constexpr int32_t kCtrWords = kCtrGaveUp + 2 * kMergeMaxWgs;

// Waits until every piece of the unit has arrived (lane 0 polls, the wave follows).
// On a timeout the piece gives up unless the unit completed meanwhile.  Returns true
// when the caller merges its own items, false when it gave up.
__device__ __forceinline__ bool wave_wait_or_give_up(uint32_t* arrive, uint32_t np, uint32_t* gave_up)
{
    const int lane = threadIdx.x & 63;
    const long long t0 = wall_clock64();
    for (int iter = 0; iter < (1 << 16); ++iter) {
        uint32_t v = 0;
        if (lane == 0)
            v = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = __builtin_amdgcn_readfirstlane(v);
        if ((v & kArriveMask) >= np)
            return true;
        if (wall_clock64() - t0 > kMergeWaitTicks)
            break;
        __builtin_amdgcn_s_sleep(2);
    }
    // raise the flag first (completed before the registration below), then register
    // while the unit is still incomplete
    uint32_t res = 1;
    if (lane == 0) {
        __hip_atomic_store(gave_up, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the flag is out
        uint32_t v = __hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every failed swap saw the word change (an arrival or another give-up): at
        // most 2 np rounds
        for (int k = 0; k < 1 << 16; ++k) {
            if ((v & kArriveMask) >= np)
                break;  // completed after all
            uint32_t expected = v;
            if (__hip_atomic_compare_exchange_strong(arrive, &expected, v + kGiveUp, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                res = 0;
                break;
            }
            v = expected;
        }
    }
    return __builtin_amdgcn_readfirstlane(res) != 0;
}

// The calling workgroup is done with the unit whose pieces are workgroups kf .. kf+np-1
// (all its waves must be: the barrier).  The unit's last piece to leave clears the
// unit's arrival and departure words and its pieces' give-up flags; slot_of(k) is the
// slot piece k used.
template <typename SlotOf>
__device__ __forceinline__ void unit_depart(uint32_t* ctr, int64_t kf, int64_t np, SlotOf slot_of)
{
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t old = 0;
        if (threadIdx.x == 0)
            old = __hip_atomic_fetch_add(ctr + kCtrDepart + kf, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if ((int64_t)old == np - 1) {
            for (int64_t j = threadIdx.x; j < np; j += 64)
                __hip_atomic_store(ctr + kCtrGaveUp + 2 * (kf + j) + slot_of(kf + j), 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (threadIdx.x == 0) {
                __hip_atomic_store(ctr + kCtrArrive + kf, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctr + kCtrDepart + kf, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

}  // namespace dflash
