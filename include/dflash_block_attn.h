/*
 * dflash_block_attn.h -- C ABI of the MI355X (gfx950) DFlash block-attention library.
 *
 * The operation (kenforever1, "DFlash + Gemma 4 31B-it" notes, sections "what
 * DFlash is" and "why non-causal attention is needed"):  a block-diffusion
 * drafter proposes a block of 1 + num_speculative_tokens query tokens per
 * request.  The block's queries (bonus token + mask tokens) attend to the
 * request's context K/V -- computed from the target model's hidden states --
 * together with the block's own K/V, as one whole block, with no left-to-right
 * restriction.  That non-causal mode is the default; vLLM PR #43445 ("Allow
 * causal DFlash", sections "implementation" and "key code") adds a per-request
 * causal flag that the attention backend interprets, and sliding-window
 * DFlash variants exist (same report, "motivation").  Gemma 4 31B's global
 * layers use head_dim 512, so the backend must take head sizes up to 512
 * (kenforever1 notes, "Gemma 4 31B-it structure" and the PR #52 change table).
 *
 * Per request r: L = ctx_lens[r] context keys, n = block_lens[r] block queries,
 * T = L + n keys (the block's own K/V are keys L..L+n-1; the caller has written
 * them to the paged cache before the call).  Query i sits at position p = L+i.
 * For q-head h the kv-head is h / (n_heads / n_kv_heads) (contiguous groups).
 * Query i sees keys j with
 *     lo_i <= j <= hi_i,   hi_i = causal[r] ? p : T-1,
 *     lo_i = window > 0 ? max(0, p - window + 1) : 0
 * and its output is the softmax(scale * q.k)-weighted mean of those keys' V.
 *
 * All functions are thread-safe.  None of them allocates device memory,
 * synchronises a stream or reads device memory from the host.
 */
#ifndef DFLASH_BLOCK_ATTN_H
#define DFLASH_BLOCK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 2

/* Return codes. */
typedef enum {
    DFLASH_OK = 0,
    DFLASH_ERR_INVALID_ARGUMENT = 1,   /* a host-checkable argument is wrong; nothing was enqueued */
    DFLASH_ERR_UNSUPPORTED = 2,        /* valid problem this library does not run (e.g. head_dim > 512) */
    DFLASH_ERR_WORKSPACE_TOO_SMALL = 3,/* desc->workspace_bytes below dflash_block_attn_workspace_size */
    DFLASH_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} dflash_status;

/* Merge of split-KV pieces (desc->merge_mode).  AUTO merges inside the attention kernel for
   small steps -- head_dim <= 256 and at most 3 key tiles of work per compute unit (run on
   at most one workgroup per CU), or a grid of at most 64 workgroups: launch-bound draft
   steps, where a second kernel is a large part of the call -- and with the combine kernel
   otherwise (measured faster there). */
#define DFLASH_MERGE_AUTO 0
#define DFLASH_MERGE_COMBINE_KERNEL 1
#define DFLASH_MERGE_IN_KERNEL 2

/* Kernel selection (desc->kernel). */
#define DFLASH_KERNEL_AUTO 0       /* the MFMA kernel where it applies, else the reference kernel */
#define DFLASH_KERNEL_REFERENCE 1  /* plain VALU kernel: any head_dim <= 512, slow; for checking */
#define DFLASH_KERNEL_MFMA 2       /* MFMA kernel: instantiated for head_dim 128/256/512, other
                                      head_dims run on the next larger one with zero-filled lanes */

/*
 * Host-side facts about one call.  Everything here is host memory; nothing in it
 * is read from the device.  Hints that bound device-side values only steer the
 * plan (work split, grid); results do not depend on them, except total_q, which
 * must be >= sum(block_lens) (rows past total_q are not combined).
 */
typedef struct {
    int32_t num_reqs;          /* B >= 0: entries in ctx_lens / block_lens / causal / page_table rows */
    int32_t total_q;           /* >= sum(block_lens): rows of q and out                                 */
    int32_t max_block_len;     /* >= max(block_lens) (0 = unknown); picks the row tiling                 */
    int64_t total_kv_len;      /* >= sum(ctx_lens + block_lens) (0 = unknown); sizes the work split      */
    int32_t page_size;         /* tokens per KV page, a power of two in [1, 1024] (16 is the tuned one); \
                                  page_size * n_kv_heads * head_dim must be < 2^31 (else UNSUPPORTED)  */
    int32_t max_pages_per_req; /* row stride (entries) of page_table, >= 1                               */
    int64_t num_pages;         /* rows of k_pages / v_pages, >= 1                                        */
    int32_t kernel;            /* DFLASH_KERNEL_* (0 = auto)                                             */
    int32_t num_workgroups;    /* 0 = planner decides; >= 1 forces the attention grid (tests)            */
    int32_t num_cus;           /* 0 = query the current device; > 0 plans for that many compute units    */
    void*   workspace;         /* device scratch owned by the caller, 256-byte aligned, zero-filled     \
                                  once before its first use (see below)                                  */
    size_t  workspace_bytes;   /* its size; must be >= dflash_block_attn_workspace_size(...)             */
    void*   event_attn_begin;  /* optional hipEvent_t recorded on `stream` right before the attention   */
    void*   event_attn_end;    /*   kernel and right after it (not around the combine); NULL = none     */
    int32_t merge_mode;        /* how split-KV pieces are merged: DFLASH_MERGE_AUTO (0, the planner     \
                                  picks), DFLASH_MERGE_COMBINE_KERNEL (1, a second kernel) or          \
                                  DFLASH_MERGE_IN_KERNEL (2, the MFMA attention kernel itself; the      \
                                  reference kernel always uses the combine kernel)                       */
} dflash_batch_desc;

/* What the planner decided for a call (dflash_block_attn_plan). */
typedef struct {
    int32_t kernel;            /* DFLASH_KERNEL_REFERENCE or DFLASH_KERNEL_MFMA                         */
    int32_t num_workgroups;    /* attention workgroups; each takes an equal run of key tiles             */
    int32_t tile_keys;         /* keys per tile                                                         */
    int32_t rows_per_unit;     /* query rows (block query x q-head of one kv-head) handled together    */
    int32_t head_dim_padded;   /* head_dim rounded up to the kernel's instantiation                      */
    int32_t combine_workgroups;/* grid of the split-KV combine kernel (0 = not launched)                 */
    int32_t merge_in_kernel;   /* 1: split-KV pieces are merged inside the attention kernel             */
    size_t  workspace_bytes;   /* scratch the call needs                                                */
} dflash_plan_info;

/*
 * dflash_block_attn -- block attention for a batch of requests.
 *
 *   q           device bf16 [total_q][n_heads][head_dim]; requests' blocks packed in order
 *   k_pages     device bf16 [num_pages][page_size][n_kv_heads][head_dim]
 *   v_pages     device bf16, same layout as k_pages
 *   page_table  device int32 [num_reqs][max_pages_per_req]; entry j of row r is the physical page
 *               holding keys [j*page_size, (j+1)*page_size) of request r; entries at or past
 *               ceil((L+n)/page_size) are never read
 *   ctx_lens    device int32 [num_reqs], L >= 0
 *   block_lens  device int32 [num_reqs], n >= 0 (n = 0: the request produces nothing)
 *   n_heads     Hq >= 1;  n_kv_heads  Hkv >= 1 with Hq % Hkv == 0
 *   head_dim    D, a multiple of 8 in [8, 512]
 *   causal      device uint8 [num_reqs] (non-zero = causal) or NULL = every request non-causal
 *   window      sliding window in keys (<= 0: none), applies to every request of the call
 *   scale       logit scale (finite), usually 1/sqrt(head_dim)
 *   out         device bf16 [total_q][n_heads][head_dim]; written, never read
 *   stream      hipStream_t to enqueue on (NULL = null stream)
 *   desc        host struct above
 *
 * Output rows are rounded to bf16 with round-to-nearest-even from fp32 accumulation.  When a
 * request's keys are split over several workgroups, each piece's normalised output is kept in
 * bf16 in the workspace (with an fp32 log-sum-exp) and the pieces are merged in fp32 (softmax
 * over a union of disjoint key sets).
 *
 * The call is asynchronous: it validates, enqueues one attention kernel -- which, for small grids
 * or when desc->merge_mode asks for it, also merges the split pieces -- or the attention kernel
 * followed by a combine kernel, and returns.  Buffers must stay valid until the stream has run the work.
 *
 * Workspace: the caller allocates dflash_block_attn_workspace_size bytes and zero-fills them
 * once (hipMemset, torch.zeros) before the first call that uses them.  The merge keeps
 * counters at the start of the workspace; every call leaves them zero again when it has run,
 * so no call needs a memset (graph capture).  After a call that did not run to completion
 * (a launch failure, a device fault) zero-fill it again.  Calls that may run at the same time
 * (different streams) need distinct workspaces.
 *
 * On a non-OK return from validation nothing is enqueued and `out` is untouched.
 * Device-side values outside the stated ranges (negative lengths, page ids >= num_pages,
 * L+n beyond max_pages_per_req*page_size) are undefined behaviour.
 */
int dflash_block_attn(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                      const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads, int32_t n_kv_heads,
                      int32_t head_dim, const uint8_t* causal, int32_t window, float scale, void* out,
                      void* stream, const dflash_batch_desc* desc);

/*
 * dflash_block_attn with bidirectional spans inside causal requests, for a
 * multimodal prefix.  kenforever1 "DFlash + Gemma 4 31B-it" notes, section on
 * MooreThreads/vllm-musa PR #52, only name the backend's mm-prefix support and
 * warn that arbitrary partial 2D masks are not fully covered; the rule below is
 * this library's reading (the plainest mask in which an image prefix is attended
 * as a whole while text stays causal).  A query at position p of a causal request that lies in
 * one of the request's spans [s, e) also sees the keys after it up to e - 1:
 * its visible range becomes [lo, max(p, e - 1)] (lo from the window as before).
 * Positions count keys of the request from 0 (context 0..L-1, block L..L+n-1).
 *   span_offsets  device int32 [num_reqs + 1] or NULL (= dflash_block_attn):
 *                 request r's spans are entries span_offsets[r] .. span_offsets[r+1]-1
 *   spans         device int32 [num_spans][2], (start, end) pairs, end exclusive;
 *                 may be NULL when num_spans == 0
 *   num_spans     entries of `spans`; the kernels skip entries outside [0, num_spans)
 * Spans of non-causal requests change nothing.  Spans may come in any order and
 * may overlap (the largest end among those holding p counts); ranges are clipped
 * to the request's keys.  Other arguments, errors and asynchrony as for
 * dflash_block_attn; both span pointers must be 4-byte aligned.
 */
int dflash_block_attn_spans(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                            const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, const uint8_t* causal, const int32_t* span_offsets,
                            const int32_t* spans, int32_t num_spans, int32_t window, float scale, void* out,
                            void* stream, const dflash_batch_desc* desc);

/*
 * Block K/V append: writes each request's block K/V into the paged cache, the
 * step that must precede the attention (the block's queries attend to the
 * context K/V together with the block's own K/V -- kenforever1 notes, "why
 * non-causal attention is needed" -- and those keys live in the same cache at
 * positions L .. L+n-1).  Row t of k_new / v_new is block token i = t - q_start[r]
 * of request r (rows packed in request order, exactly like q); it is copied to
 * page page_table[r][(L+i) / page_size], slot (L+i) % page_size, kv-head h.
 *   k_new, v_new     device bf16 [desc->total_q, n_kv_heads, head_dim], 16-byte aligned
 *   k_pages, v_pages device bf16 [num_pages, page_size, n_kv_heads, head_dim]; only
 *                    the block slots are written
 *   page_table, ctx_lens, block_lens, desc  as for dflash_block_attn (desc->total_q
 *                    must equal sum(block_lens); workspace and events are not used)
 * Host-checkable errors return before anything is enqueued.  Page-table entries
 * that the block positions need must be valid page ids (undefined otherwise).
 */
int dflash_block_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                           const int32_t* page_table, const int32_t* ctx_lens, const int32_t* block_lens,
                           int32_t n_kv_heads, int32_t head_dim, void* stream, const dflash_batch_desc* desc);

/*
 * dflash_block_kv_append followed by dflash_block_attn on the same stream: one
 * call per draft step, graph-capturable (it allocates nothing, synchronises
 * nothing and enqueues only kernel launches).  Both halves are validated before
 * either is enqueued; arguments as for the two calls.  With the MFMA kernel and
 * pages of at least 16 keys the two are one launch: the attention reads the
 * block's own K/V from k_new / v_new and writes them into the pages itself (the
 * result, pages included, is the same as the two calls').
 */
int dflash_block_attn_append(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                             const int32_t* page_table, const int32_t* ctx_lens, const int32_t* block_lens,
                             int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, const uint8_t* causal,
                             int32_t window, float scale, void* out, void* stream, const dflash_batch_desc* desc);

/*
 * dflash_block_attn for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same operation,
 * arguments, layouts and errors, but the scratch comes from a static array inside the
 * library -- desc->workspace and desc->workspace_bytes are ignored, and the split-KV pieces
 * are always merged by the combine kernel (desc->merge_mode is ignored).  The array holds
 * dflash_noalloc_scratch_bytes() bytes (48 MiB) on every GPU the library runs on, for the
 * life of the process; a call that needs more (dflash_block_attn_workspace_size) returns
 * DFLASH_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call on one GPU shares
 * the array: calls that may overlap on one GPU (different streams, or host threads) race
 * and must not be issued.  Nothing is allocated, freed or synchronised.
 */
int dflash_block_attn_noalloc(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                              const int32_t* ctx_lens, const int32_t* block_lens, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, const uint8_t* causal, int32_t window,
                              float scale, void* out, void* stream, const dflash_batch_desc* desc);

/* Bytes of the static scratch dflash_block_attn_noalloc uses on each GPU. */
size_t dflash_noalloc_scratch_bytes(void);

/* Scratch bytes dflash_block_attn needs for this desc and shape (desc->workspace is ignored). */
int dflash_block_attn_workspace_size(const dflash_batch_desc* desc, int32_t n_heads, int32_t n_kv_heads,
                                     int32_t head_dim, size_t* bytes);

/* The plan dflash_block_attn would use (host only; nothing is launched). */
int dflash_block_attn_plan(const dflash_batch_desc* desc, int32_t n_heads, int32_t n_kv_heads,
                           int32_t head_dim, dflash_plan_info* plan);

/*
 * 1 if the library runs this head configuration -- in both non-causal and causal
 * mode and with any window -- else 0.  A backend must declare non-causal support
 * rather than silently run a causal mask (kenforever1 notes, "why non-causal
 * attention is needed"; vLLM PR #43445 report, "key code", the non-causal
 * assertion).
 */
int dflash_block_attn_supports(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim);

/* Static text for a dflash_status value. */
const char* dflash_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* dflash_last_error_message(void);

/* DFLASH_ABI_VERSION of the built library. */
int dflash_abi_version(void);

/*
 * Debug checks of device-side values.  Lengths, page ids and span offsets live in
 * device memory, so the host cannot check them, and out-of-range values are
 * undefined behaviour on the normal path.  With checks on, every attention / append
 * call first runs a one-workgroup kernel over them.  On a failure it sets bits in a
 * sticky per-device state word, and every kernel of that call then does nothing:
 * `out`, the pages and the workspace are left untouched, and no bad page id is
 * dereferenced.  The checks cost one small launch per call.  They are off unless
 * DFLASH_DEBUG_CHECKS=1 is in the environment at the first call.
 *
 * Bits: a request's pages are those a kernel of the call reads or writes, i.e. from
 * the first key the attention reads (window start, tile-aligned) or from the block
 * start for an append alone, to the request's last key.
 */
#define DFLASH_DEBUG_NEGATIVE_LENGTH   1u  /* ctx_lens[r] < 0 or block_lens[r] < 0                     */
#define DFLASH_DEBUG_BEYOND_PAGE_TABLE 2u  /* L + n > max_pages_per_req * page_size                     */
#define DFLASH_DEBUG_BAD_PAGE_ID       4u  /* a page the call touches is outside [0, desc->num_pages)   */
#define DFLASH_DEBUG_TOTAL_Q_MISMATCH  8u  /* sum(block_lens) != desc->total_q                          */
#define DFLASH_DEBUG_ABOVE_HINT       16u  /* a block above max_block_len, or sum(L+n) > total_kv_len   */
#define DFLASH_DEBUG_BAD_SPAN_OFFSETS 32u  /* span_offsets not non-decreasing within [0, num_spans]     */

/* Switches the checks on (non-zero) or off for later calls; returns the previous setting. */
int dflash_set_debug_checks(int on);

/*
 * Synchronises the current device, stores the OR of the bits set by all checked calls
 * since the last query in *bits, and stores the lowest failing request index in
 * *first_request (-1 when no bit is set).  Then it clears the state.  Calls whose checks
 * fail do nothing, so with checks on a non-zero result means some call was skipped.
 * Returns DFLASH_ERR_HIP without a device.
 */
int dflash_debug_checks_result(uint32_t* bits, int32_t* first_request);

/*
 * DFlash2 in-block grouped dynamic depthwise convolution (prhub summary of vLLM
 * PR #52816, "DFlash2: local convolution + candidate selector", section
 * "motivation"): for every request's block of n positions and every channel c,
 *     out[i,c] = sum_{t=0}^{taps-1} (base[t,c] + delta[i,t,g(c)]) * x[i-t,c],
 * where taps reaching before the block's first position (i - t < 0) are zero and
 * g(c) = c / (channels / groups) (contiguous channel groups).
 *   x      device bf16 [total_q, channels]; rows are block positions packed in
 *          request order (request r: rows q_start[r] .. q_start[r] + n_r - 1)
 *   base   device bf16 [taps, channels]
 *   delta  device bf16 [total_q, taps, groups]
 *   block_lens device int32 [num_reqs]; their sum must equal total_q
 *   out    device bf16 [total_q, channels] (written; must not alias x)
 * fp32 accumulation over t in increasing order, bf16 result rounded to nearest
 * even.  channels even, groups dividing channels, 1 <= taps <= 1024,
 * total_q <= 65535.  Host-checkable errors return before anything is
 * enqueued; asynchronous on `stream`.
 */
int dflash_block_conv(const void* x, const void* base, const void* delta, const int32_t* block_lens,
                       int32_t num_reqs, int32_t total_q, int32_t channels, int32_t groups, int32_t taps, void* out,
                       void* stream);

/*
 * Measurement helper, not part of the attention: reads `bytes` of device memory
 * at `buf` once, with the same streaming (nontemporal) 16-byte loads the
 * attention kernel uses for K/V, and XORs every 32-bit word it read into
 * sink[0] (one atomic per wavefront; clear sink[0] first to get the XOR of the
 * buffer).  Timing it gives the achievable HBM read bandwidth that K/V GB/s is
 * reported against, next to the 8 TB/s specification; a pass over a buffer
 * larger than the last-level cache is also a flush that leaves no dirty lines.
 *   buf    device pointer, 16-byte aligned; bytes a multiple of 16 (0 is a no-op)
 *   sink   device uint32_t[1], caller-owned
 *   stream hipStream_t (NULL = default stream); asynchronous, stream-ordered
 * Returns DFLASH_ERR_INVALID_ARGUMENT for a NULL/misaligned pointer or size,
 * DFLASH_ERR_HIP if the launch fails.
 */
int dflash_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef DFLASH_TIMELINE
/*
 * dflash_timeline_set_buffer -- exported only by the timeline build of the library
 * (libdflash_attn_timeline.so, compiled with -DDFLASH_TIMELINE; the product library
 * does not have it).  A measurement aid: every later MFMA attention launch whose grid
 * of P workgroups fits in `bytes` (P * 64) writes, per logical workgroup w, the 100 MHz
 * wall clock (wall_clock64) at buf[8w + 0] its start, [8w + 1] its first tile loop's
 * start, [8w + 2] its last tile loop's end, [8w + 3] the end of its last epilogue
 * (before any in-kernel merge), and [8w + 4] its key-tile count.  Workgroups without
 * tiles leave [1] and [2] zero.  buf: device memory, caller-owned, 8-byte aligned;
 * NULL with bytes = 0 turns the stamps off.  DFLASH_ERR_INVALID_ARGUMENT otherwise.
 */
int dflash_timeline_set_buffer(void* buf, size_t bytes);
#endif

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_BLOCK_ATTN_H */
