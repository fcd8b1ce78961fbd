// attn_mfma_small_pages.hip -- instances of the MFMA block-attention kernel
// (attn_mfma_kernel.h) for KV pages of fewer than 16 keys, with and without
// bidirectional spans.  A 32-key tile then spans several pages, so each lane
// fetches the page id of its own keys from the tile's page entries.
#include "attn_mfma_kernel.h"

namespace dflash {

hipError_t launch_attn_mfma_small_pages(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream)
{
    if (a.span_offsets)
        return launch_dp<true, false>(a, dpad, row_tiles, stream);
    return launch_dp<false, false>(a, dpad, row_tiles, stream);
}

}  // namespace dflash
