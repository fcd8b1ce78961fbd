// attn_mfma_spans.hip -- instances of the MFMA block-attention kernel
// (attn_mfma_kernel.h) whose causal rows may be widened by bidirectional spans
// (the multimodal-prefix mask of kenforever1's "DFlash + Gemma 4 31B-it" notes,
// section on MooreThreads/vllm-musa PR #52).
#include "attn_mfma_kernel.h"

namespace dflash {

hipError_t launch_attn_mfma_spans(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream)
{
    return launch_dp<true, true>(a, dpad, row_tiles, stream);
}

}  // namespace dflash
