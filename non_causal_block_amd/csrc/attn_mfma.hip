// attn_mfma.hip -- instances of the MFMA block-attention kernel (attn_mfma_kernel.h)
// for plain masks, the dispatch between plain and span instances, and the
// occupancy queries the planner uses.
#include "attn_mfma_kernel.h"

namespace dflash {

hipError_t launch_attn_mfma(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream)
{
    if (a.page_shift < 4)
        return launch_attn_mfma_small_pages(a, dpad, row_tiles, stream);
    if (a.span_offsets)
        return launch_attn_mfma_spans(a, dpad, row_tiles, stream);
    return launch_dp<false, true>(a, dpad, row_tiles, stream);
}

// Resident workgroups per CU, queried once per kernel instance (the library runs on
// one architecture, so the answer does not depend on the device).  The span and
// small-page instances differ only in a few instructions and share the plain ones'
// launch shape; the planner's count is an upper bound on workgroups in flight,
// not something the kernel relies on.
template <int DP, int RT, bool EXACT>
static int occupancy_one()
{
    static std::atomic<int> cached{-1};
    int blocks = cached.load(std::memory_order_acquire);
    if (blocks >= 0)
        return blocks;
    if (ensure_lds_limit<DP, RT, EXACT, false, true>() != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_mfma_kernel<DP, RT, EXACT, false, true, false>,
                                                     Cfg<DP, RT>::THREADS, Cfg<DP, RT>::LDS_BYTES) != hipSuccess)
        return 0;
    cached.store(blocks, std::memory_order_release);
    return blocks;
}

template <int DP, bool EXACT>
static int occupancy_rt(int row_tiles)
{
    switch (row_tiles) {
    case 1: return occupancy_one<DP, 1, EXACT>();
    case 2: return occupancy_one<DP, 2, EXACT>();
    case 3: return occupancy_one<DP, 3, EXACT>();
    case 4: return occupancy_one<DP, 4, EXACT>();
    case 5: return occupancy_one<DP, 5, EXACT>();
    default: return 0;
    }
}

int mfma_tile_keys() { return kTK; }
int mfma_max_row_tiles(int /*dpad*/) { return 5; }

int mfma_wgs_per_cu(int dpad, int row_tiles, bool exact)
{
    switch (dpad) {
    case 128: return exact ? occupancy_rt<128, true>(row_tiles) : occupancy_rt<128, false>(row_tiles);
    case 256: return exact ? occupancy_rt<256, true>(row_tiles) : occupancy_rt<256, false>(row_tiles);
    case 512: return exact ? occupancy_rt<512, true>(row_tiles) : occupancy_rt<512, false>(row_tiles);
    default: return 0;
    }
}

}  // namespace dflash
