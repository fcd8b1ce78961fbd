// attn_mfma_append.hip -- instances of the MFMA block-attention kernel
// (attn_mfma_kernel.h) with the block K/V append fused in: the block's queries attend to
// the context K/V together with the block's own K/V (kenforever1 "DFlash + Gemma 4
// 31B-it" notes, "why non-causal attention is needed"), which are read straight from the
// draft step's new K/V rows and written into their page slots by the same launch.
// Pages of at least 16 keys, no spans.
#include "attn_mfma_kernel.h"

namespace dflash {

hipError_t launch_attn_mfma_append(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream)
{
    if (a.page_shift < 4 || a.span_offsets || !a.k_new || !a.v_new || !a.k_dst || !a.v_dst)
        return hipErrorInvalidValue;
    return launch_dp<false, true, true>(a, dpad, row_tiles, stream);
}

}  // namespace dflash
