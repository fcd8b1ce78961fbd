// kernels.h -- launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace dflash {

// Plain VALU kernel.
hipError_t launch_attn_ref(const AttnArgs& a, hipStream_t stream);
int ref_rows_per_unit();
int ref_tile_keys();
int ref_wgs_per_cu();  // resident workgroups per CU on the current device (0 if unknown)

// MFMA kernel.  `row_tiles` is the number of 16-row MFMA tiles per unit
// (rows per unit = 16 * row_tiles); `dpad` is 128, 256 or 512.
hipError_t launch_attn_mfma(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream);
// the same with bidirectional spans (a.span_offsets non-null); attn_mfma_spans.hip
hipError_t launch_attn_mfma_spans(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream);
// the same with the block K/V append fused in (pages of >= 16 keys, no spans); attn_mfma_append.hip
hipError_t launch_attn_mfma_append(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream);
// the same for pages of fewer than 16 keys (a.page_shift < 4); attn_mfma_small_pages.hip
hipError_t launch_attn_mfma_small_pages(const AttnArgs& a, int dpad, int row_tiles, hipStream_t stream);
int mfma_tile_keys();
int mfma_max_row_tiles(int dpad);
int mfma_wgs_per_cu(int dpad, int row_tiles, bool exact);  // on the current device (0 if unknown)

// Split-KV combine.
// lanes per output row (16, 32 or 64) for a padded head_dim and head count
int combine_lanes_per_row(int dpad, int32_t n_heads);
int combine_grid(int64_t total_rows, int lanes_per_row);
// pieces_per_step 4, 8 or 16
hipError_t launch_combine(const CombineArgs& a, int grid, int pieces_per_step, int lanes_per_row, hipStream_t stream);
// one output row per workgroup, pieces dealt over its four waves (head_dim <= 512); grid = total_rows
hipError_t launch_combine_rows(const CombineArgs& a, hipStream_t stream);

// block K/V rows -> their pages (one wave per (token, kv-head) row)
int append_grid(int64_t total_rows);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

// DFlash2 in-block grouped dynamic depthwise convolution
hipError_t launch_block_conv(const ConvArgs& a, hipStream_t stream);

// records `msg` as the calling thread's last error (dflash_last_error_message); returns status
int set_last_error(int status, const char* msg);

// debug checks: the per-device state word (static device memory) and the checking kernel
hipError_t debug_state_ptr(uint32_t** out);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream);

// streaming read of bytes (a multiple of 16) with grid workgroups, XOR of all words into *sink
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t stream);

}  // namespace dflash
