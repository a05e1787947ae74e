/*
 * rld.h -- C ABI of the routed LoRA delta library (librld.so, gfx950).
 *
 * For a batch of rows, each row names an adapter slot; the library adds that
 * adapter's LoRA delta to the row's output in place:
 *
 *     xa    = bf16(x_i @ A_s^T)              shrink, to a BF16 scratch
 *     delta = bf16(xa @ B_s^T)               expand
 *     out_i = bf16(f32(out_i) + scale_s * f32(delta))   fold (fp32 multiply,
 *                                            rounded, then fp32 add, rounded)
 *
 * Both contractions run at the pool's padded max_rank.  Sources: the routed-LoRA
 * pages "Function apply_lora_bgmv" (description, STRIDES and GRAPH-SAFE
 * paragraphs), "Module lora_delta" (LoraPair, LoraRoute), the lora_delta.rs
 * listing (LoraPair, LoraRoute and apply_lora_bgmv doc comments) and "Module
 * moe_lora_grouped" (moe_lora_grouped_down, moe_lora_gather_bgmv,
 * pack_expert_tables, grouped_down_wc, grouped_down_windows,
 * gather_bgmv_grids, gather_row_token, MLG_M_TILE).
 *
 * Conventions shared by every entry point
 *   - BF16 tensors are passed as void* and hold IEEE bfloat16 bit patterns.
 *   - All sizes and strides are in elements, not bytes.
 *   - Device pointers are raw HIP device addresses; the caller owns every
 *     buffer.  Device entry points allocate nothing, never synchronise and
 *     never read device memory on the host, so a sequence of calls can be
 *     captured into a HIP graph; the launch shape depends only on the host
 *     arguments.  `stream` is a hipStream_t (NULL = the default stream).
 *   - Return value: RLD_OK (0) or a negative status.  Argument errors are
 *     detected before any launch; a launch error is reported as RLD_ELAUNCH
 *     and its HIP code is kept for rld_last_hip_error().
 *   - Alignment (RLD_EALIGN otherwise): k_in, n_out, max_rank and all row
 *     strides and element offsets are multiples of 8; x, xa and base_out
 *     pointers are 16-byte aligned; A/B pool addresses in the tables are
 *     16-byte aligned (checked by the pack helpers, which are the supported
 *     way to build tables).  max_rank <= 128 (RLD_EUNSUPPORTED otherwise).
 *   - Device-side values the host cannot see (slot ids, expert ids, token
 *     ids, offsets) are never trusted for addressing: a row whose slot is < 0
 *     or >= max_loras, whose table entries are 0, whose expert or token is out
 *     of range, or that lies in no expert span is a base row.  A base row's
 *     output is left untouched and its xa row is written as zeros.
 */
#ifndef RLD_H
#define RLD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RLD_OK 0
#define RLD_EINVAL (-1)       /* null required pointer, zero or inconsistent size   */
#define RLD_EALIGN (-2)       /* size, stride, offset or pointer not aligned (above) */
#define RLD_EUNSUPPORTED (-3) /* e.g. max_rank > 128, or more than 2^30 work items   */
#define RLD_ELAUNCH (-4)      /* a kernel launch failed; see rld_last_hip_error()    */
#define RLD_ENOSPACE (-5)     /* xa or workspace smaller than the call needs          */

#define RLD_MAX_RANK 128
#define RLD_M_TILE 64 /* rows per m-tile of the grouped path (MLG_M_TILE) */

/* Routing tables of one (layer, module): LoraRoute.  All three tables are
 * device arrays of max_loras entries, fixed when the pool is packed.
 * a_table[s] / b_table[s] are device addresses of slot s's padded A
 * ([max_rank, k_in] row-major BF16, zero rows past the adapter's rank) and B
 * ([n_out, max_rank] row-major BF16, zero columns past the rank); 0 means the
 * slot does not adapt this module.  scale_table[s] is the fp32 scale. */
typedef struct rld_route {
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  uint32_t max_loras;
  uint32_t k_in;
  uint32_t n_out;
  uint32_t max_rank;
} rld_route;

/* One adapted module without routing (LoraPair, "Module lora_delta"): device
 * addresses of A ([max_rank, k_in] row-major BF16, zero rows past the
 * adapter's rank) and B ([n_out, max_rank] row-major BF16, zero columns past
 * the rank), and the fp32 scale. */
typedef struct rld_pair {
  const void* a;
  const void* b;
  float scale;
  uint32_t k_in;
  uint32_t n_out;
  uint32_t max_rank;
} rld_pair;

/* Expert routing tables of one MoE projection (MoeExpertRoute, widened to a
 * [max_loras][num_experts] table so a mixed batch can name its adapter per
 * row): entry s*num_experts + e holds adapter slot s's pair for expert e. */
typedef struct rld_moe_route {
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  uint32_t max_loras;
  uint32_t num_experts;
  uint32_t k_in;
  uint32_t n_out;
  uint32_t max_rank;
} rld_moe_route;

/* One adapted module of one adapter, as installed in a pool. */
typedef struct rld_adapter_entry {
  uint32_t slot;      /* adapter slot, < max_loras                              */
  int32_t expert;     /* expert id for MoE tables; ignored by rld_route_pack    */
  uint64_t a_addr;    /* device address of the padded A, 16-byte aligned, != 0 */
  uint64_t b_addr;    /* device address of the padded B, 16-byte aligned, != 0 */
  uint32_t rank;      /* true rank, 1..max_rank                                 */
  float alpha;        /* lora_alpha                                             */
  int32_t use_rslora; /* nonzero: scale = alpha/sqrt(rank); else alpha/rank      */
} rld_adapter_entry;

/* ---------------------------------------------------------------- host ---- */

/* LoraPair scale (lora_delta.rs, LoraPair doc comment): alpha/rank, or
 * alpha/sqrt(rank) with use_rslora, computed in double and rounded once to
 * float.  RLD_EINVAL if rank == 0 or out is NULL. */
int rld_scale(float alpha, uint32_t rank, int use_rslora, float* out);

/* Adapter install, PEFT tensors stored as F16 ("Module lora_delta": A/B kept
 * verbatim, converted F16 -> BF16 on the host at load): dst[i] = the BF16
 * value nearest to the F16 value src[i], ties to even.  Every F16 value is in
 * BF16's normal range, so only the significand is rounded; +-0 and +-Inf are
 * kept, a NaN becomes a quiet NaN with its sign.  Host memory, bit patterns;
 * src and dst may be the same array.  RLD_EINVAL on NULL with n > 0. */
int rld_f16_to_bf16_host(const uint16_t* src, uint16_t* dst, size_t n);

/* Pool layout of one PEFT pair ("Module lora_delta", LoraPair; lora_delta.rs
 * header invariants): a [rank, k_in] -> a_pad [max_rank, k_in] with zero rows
 * after rank; b [n_out, rank] -> b_pad [n_out, max_rank] with zero columns
 * after rank.  Host memory, BF16 bits.  RLD_EINVAL on NULL or rank > max_rank. */
int rld_pad_adapter_host(const uint16_t* a, const uint16_t* b, uint32_t rank, uint32_t k_in,
                         uint32_t n_out, uint32_t max_rank, uint16_t* a_pad, uint16_t* b_pad);

/* Slot route tables of one module (LoraRoute: "built at pool pack time").
 * Writes host arrays a_out/b_out/scale_out of max_loras entries: 0/0/0.0f for
 * slots without an entry; a repeated slot keeps the last entry.  The caller
 * uploads them.  RLD_EINVAL on slot >= max_loras, rank 0 or > max_rank, or a
 * zero address; RLD_EALIGN on an address that is not 16-byte aligned. */
int rld_route_pack(const rld_adapter_entry* entries, size_t n_entries, uint32_t max_loras,
                   uint32_t max_rank, uint64_t* a_out, uint64_t* b_out, float* scale_out);

/* MoE tables [max_loras * num_experts] (same rules per (slot, expert);
 * RLD_EINVAL on expert < 0 or >= num_experts). */
int rld_moe_tables_pack(const rld_adapter_entry* entries, size_t n_entries, uint32_t max_loras,
                        uint32_t num_experts, uint32_t max_rank, uint64_t* a_out, uint64_t* b_out,
                        float* scale_out);

/* pack_expert_tables ("Module moe_lora_grouped"): dense [n_experts] tables
 * indexed by expert id from (expert_id, a, b, scale) entries; n_experts = max
 * id + 1; 0/0/0.0f where unadapted; a repeated id keeps the last entry.
 * *n_experts_out = 0 for no entries (the page's None).  RLD_ENOSPACE if
 * n_experts would exceed cap. */
int rld_pack_expert_tables(const uint32_t* expert_ids, const uint64_t* a_addrs,
                           const uint64_t* b_addrs, const float* scales, size_t n_entries,
                           uint32_t cap, uint64_t* a_out, uint64_t* b_out, float* scale_out,
                           uint32_t* n_experts_out);

/* grouped_down_windows: contiguous [start, end) windows of at most cap rows
 * covering 0..total_rows.  *count = number of windows (0 when total_rows is
 * 0); RLD_ENOSPACE if more than max_windows; RLD_EINVAL if cap == 0. */
int rld_grouped_windows(uint32_t total_rows, uint32_t cap, uint32_t* starts, uint32_t* ends,
                        uint32_t max_windows, uint32_t* count);

/* grouped_down_wc: m-tiles of one window, max(1, ceil((row_end-row_offset)/64));
 * 0 if row_end < row_offset. */
uint32_t rld_grouped_wc(uint32_t row_offset, uint32_t row_end);

/* gather_row_token: owning token of flat (token, top-k position) row `row`:
 * row / top_k (0 if top_k == 0). */
uint32_t rld_gather_row_token(uint32_t row, uint32_t top_k);

/* gather_bgmv_grids: the exact launch shapes of the gather shrink and expand
 * for these host constants: out[0..2] shrink grid, out[3..5] shrink block,
 * out[6..8] expand grid, out[9..11] expand block.  They depend only on the
 * arguments, so a captured graph's shape is fixed.  (The shapes are this
 * library's own, not the page's 4-outputs-per-block grids.) */
int rld_gather_grids(uint32_t max_rank, uint32_t n_out, uint32_t n_rows, uint32_t out[12]);

/* -------------------------------------------------------------- device ---- */

/* Bytes of workspace the BGMV entry points need for a call with these sizes:
 * the fp32 partial sums of the k_in split ([chunks][n][max_rank], chunks of
 * 256 for max_rank <= 16 and 512 above); 0 when k_in fits one chunk (then no
 * workspace is needed and NULL may be passed) or when k_in, max_rank or
 * max_loras is 0.
 *
 * Workspace contract (rld_bgmv_shrink and rld_bgmv):
 *   - device memory, 16-byte aligned, of workspace_bytes >= the size above;
 *     one buffer as large as the largest call serves calls of every shape;
 *   - its contents need no initialisation and carry nothing between calls;
 *   - calls that share a workspace must not run at the same time (same stream,
 *     or otherwise ordered). */
size_t rld_bgmv_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank,
                                uint32_t max_loras);

/* Routed BGMV shrink (apply_lora_bgmv, kernel 1): for every row i < n with an
 * active slot s = seq_slot[i], xa[i, k] = bf16(sum_c x[i*x_row_stride + c] *
 * A_s[k, c]) for k < max_rank; xa rows of base rows are zeros.  With a k_in
 * split this is two launches on the stream (the shrink, then the chunk
 * reduce).
 *   x        device BF16, row i at x + i*x_row_stride, k_in elements read
 *   seq_slot device int32 [n], contents may change between calls
 *   xa       device BF16 [n, max_rank] (row stride max_rank), written
 *   workspace see rld_bgmv_workspace_bytes (RLD_ENOSPACE if smaller)
 * n == 0 is a no-op.  The per-row result does not depend on n or on the
 * other rows, so a batched call is bit-identical to n one-row calls. */
int rld_bgmv_shrink(const rld_route* route, const void* x, uint32_t x_row_stride,
                    const int32_t* seq_slot, uint32_t n, void* xa, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Routed BGMV expand + fold (apply_lora_bgmv, kernel 2): for every row with
 * an active slot, delta = bf16(xa[i,:] @ B_s^T) and
 * base_out[i*out_row_stride + j] = bf16(f32(base) + scale_s * f32(delta_j))
 * for j < n_out.  Nothing outside [0, n_out) of each row is touched, so the
 * fold can land inside an interleaved [Q|K|V] row (pass base_out offset to the
 * K or V region and the full row stride). */
int rld_bgmv_expand_fold(const rld_route* route, const void* xa, const int32_t* seq_slot,
                         uint32_t n, void* base_out, uint32_t out_row_stride, void* stream);

/* apply_lora_bgmv: the results of rld_bgmv_shrink then rld_bgmv_expand_fold
 * on the same stream (xa written, outputs folded), bit for bit.  At
 * max_rank <= 16, k_in <= 4096 and n <= 256 with few enough (slot, column
 * group) items (decode batches of the attention shapes) this is one launch
 * instead of three: each block recomputes its slot's xa in the shrink's
 * summation order and expands its columns from LDS; the workspace is then
 * unused, but the workspace arguments are checked as for the two stages.
 * rld_bgmv_launches gives the count for a call. */
int rld_bgmv(const rld_route* route, const void* x, uint32_t x_row_stride,
             const int32_t* seq_slot, uint32_t n, void* base_out, uint32_t out_row_stride,
             void* xa, void* workspace, size_t workspace_bytes, void* stream);

/* Kernel launches of rld_bgmv (one route: routes = &route, nroutes = 1) or of
 * rld_bgmv_multi over these routes, for a batch of n rows: 1 in the one-pass
 * form, 3 with a k_in split (shrink, chunk reduce, expand), 2 without one.
 * 0 for n == 0 or routes the calls reject (a missing table, a zero dimension,
 * one that is not a multiple of 8, max_rank above RLD_MAX_RANK, routes of
 * different k_in or max_rank, nroutes outside 1..4).  The one-pass form is
 * taken at max_rank <= 16, k_in <= 4096 and n <= 256 when the routes'
 * (slot, 512 output columns) items number at most 256. */
int rld_bgmv_launches(const rld_route* const* routes, uint32_t nroutes, uint32_t n);

/* rld_bgmv for callers that cannot allocate: code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc.  The same fold, bit for
 * bit, with the xa arena and the k-split partials in a fixed device array of
 * RLD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * (until the process ends) instead of caller buffers.  The call allocates
 * nothing; its first call with a device current looks up that device's copy.
 *   route, x, x_row_stride, seq_slot, n, base_out, out_row_stride, stream:
 *                   as rld_bgmv
 * RLD_ENOSPACE (before anything runs) when the call needs more scratch than
 * RLD_NOALLOC_SCRATCH_BYTES: the xa arena, n * max_rank * 2 bytes rounded up to
 * a multiple of 256, plus rld_bgmv_workspace_bytes(n, k_in, max_rank, 1) (at
 * k_in 12288 and max_rank 64, up to 1337 rows).  Nothing in the scratch must
 * start at zero: every call
 * writes all it reads.  All calls on one GPU share its scratch, which keeps the
 * last call's contents: calls that may overlap on one GPU (different streams
 * without ordering) race, so issue them on one stream or order them. */
#define RLD_NOALLOC_SCRATCH_BYTES (8u << 20)
int rld_bgmv_noalloc(const rld_route* route, const void* x, uint32_t x_row_stride,
                     const int32_t* seq_slot, uint32_t n, void* base_out,
                     uint32_t out_row_stride, void* stream);

/* Several routed BGMV folds over the same rows (apply_lora_bgmv once per
 * route, as a layer's q, k and v, or gate and up, read one input): one shrink,
 * one chunk reduce (k_in split only) and one expand launch serve every route,
 * instead of that many per route (in rld_bgmv's one-pass form, one launch).
 *   routes          host array [nroutes] of routes, 1 <= nroutes <= 4
 *                   (RLD_EUNSUPPORTED above); all with the same k_in and
 *                   max_rank (RLD_EINVAL otherwise); max_loras and n_out may
 *                   differ
 *   x, seq_slot, n  as rld_bgmv, shared by every route
 *   base_out, out_row_stride, xa
 *                   host arrays [nroutes]: route r folds into base_out[r]
 *                   (row stride out_row_stride[r]) through its own xa[r]
 *                   (device BF16 [n, max_rank]); as rld_bgmv otherwise
 *   workspace       rld_bgmv_multi_workspace_bytes(n, k_in, max_rank, nroutes)
 *                   bytes (route r's partials at r times the single-route
 *                   size), under the single-route contract
 * Route r's results are bit-identical to rld_bgmv on that route alone.  The
 * outputs of different routes must not overlap; n == 0 is a no-op. */
size_t rld_bgmv_multi_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank,
                                      uint32_t nroutes);
int rld_bgmv_multi(const rld_route* const* routes, uint32_t nroutes, const void* x,
                   uint32_t x_row_stride, const int32_t* seq_slot, uint32_t n,
                   void* const* base_out, const uint32_t* out_row_stride, void* const* xa,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace the unrouted entry points need for m rows: the same k_in
 * split as the BGMV path (rld_bgmv_workspace_bytes(m, k_in, max_rank, 1)),
 * under the same contract.  0 when k_in fits one chunk. */
size_t rld_lora_workspace_bytes(uint32_t m, uint32_t k_in, uint32_t max_rank);

/* Unrouted single-adapter shrink (apply_lora_delta, lora_delta.rs): for every
 * row i < m, xa[i, k] = bf16(sum_c x[i*x_row_stride + c] * A[k, c]) for
 * k < max_rank.
 *   x   device BF16, row i at x + i*x_row_stride (the page asks for
 *       contiguous rows; any stride >= k_in works here)
 *   xa  device BF16 [m, max_rank], written
 * One launch shape serves every m (the page's m == 1 GEMV pair, its row loop
 * up to lora_gemv_max_m rows and its GEMM path are one path here).  A row's
 * summation order depends only on (k_in, max_rank) and is the same as in the
 * routed BGMV shrink, so m rows are bit-identical to m one-row calls and to a
 * routed call with every row on a slot holding this pair. */
int rld_lora_shrink(const rld_pair* pair, const void* x, uint32_t x_row_stride, uint32_t m,
                    void* xa, void* workspace, size_t workspace_bytes, void* stream);

/* Unrouted expand + fold (apply_lora_delta's expand and bf16_scaled_add, fused):
 * delta = bf16(xa[i,:] @ B^T) and base_out[i*out_row_stride + j] =
 * bf16(f32(base) + scale * f32(delta_j)) for j < n_out, every row i < m.
 * Nothing outside [0, n_out) of a row is touched. */
int rld_lora_expand_fold(const rld_pair* pair, const void* xa, uint32_t m, void* base_out,
                         uint32_t out_row_stride, void* stream);

/* apply_lora_delta: rld_lora_shrink then rld_lora_expand_fold on the same
 * stream.  m == 0 is a no-op. */
int rld_lora_delta(const rld_pair* pair, const void* x, uint32_t x_row_stride, uint32_t m,
                   void* base_out, uint32_t out_row_stride, void* xa, void* workspace,
                   size_t workspace_bytes, void* stream);

/* MoE decode gather-fold shrink (moe_lora_gather_bgmv): flat row rho < n_rows
 * (rho = token*top_k + position) uses expert e = indices[rho] and adapter slot
 * s = row_adapter[rho / top_k] (row_adapter NULL: every row uses slot 0).
 * xa [n_rows, max_rank]. */
int rld_moe_gather_shrink(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                          const int32_t* indices, const int32_t* row_adapter, uint32_t top_k,
                          uint32_t n_rows, void* xa, void* stream);

/* MoE decode gather-fold expand + fold into base_out rows (flat row order). */
int rld_moe_gather_expand_fold(const rld_moe_route* route, const void* xa, const int32_t* indices,
                               const int32_t* row_adapter, uint32_t top_k, uint32_t n_rows,
                               void* base_out, uint32_t out_row_stride, void* stream);

/* moe_lora_gather_bgmv: gather shrink then expand + fold. */
int rld_moe_gather(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                   const int32_t* indices, const int32_t* row_adapter, uint32_t top_k,
                   uint32_t n_rows, void* base_out, uint32_t out_row_stride, void* xa,
                   void* stream);

/* Bytes of workspace rld_moe_grouped_shrink needs for a window of window_rows
 * rows: the fp32 partial sums of its k_in split ([chunks][window_rows]
 * [max_rank], chunks = ceil(k_in / 512)) plus 16 bytes of counter per (slot,
 * expert) pair.  Returns 0 when k_in is one chunk -- k_in <= 1024, or
 * k_in <= 2048 with max_rank <= 32 -- (no workspace needed, NULL may be
 * passed) or when any size is 0.  Workspace contract:
 *   - device memory, 16-byte aligned, of workspace_bytes >= the size above;
 *     one buffer as large as the largest call needs serves every window and
 *     route, if the same workspace_bytes is passed every time (the counters
 *     sit at the end of the buffer, keyed by pair);
 *   - zero-filled once before its first use (e.g. hipMemset at allocation);
 *     every call leaves the counters at zero again; do not write them;
 *   - calls that share a workspace must not run at the same time. */
size_t rld_moe_grouped_workspace_bytes(uint32_t window_rows, uint32_t k_in, uint32_t max_rank,
                                       uint32_t max_loras, uint32_t num_experts);

/* MoE grouped fold shrink for ONE chunk window [row_offset, row_end) of the
 * expert-sorted rows (moe_lora_grouped_down):
 *   expert_offsets   device int32 [num_experts_off + 1], non-decreasing prefix
 *                    sum; row r belongs to the expert e with
 *                    off[e] <= r < off[e+1]
 *   sorted_token_ids device int32, sorted row -> token; may be NULL when
 *                    x_gather == 0 and row_adapter == NULL.  When given, every
 *                    row's token is read and a row whose token is outside
 *                    [0, num_tokens) is a base row (in the shrink, the expand
 *                    and the combined calls alike, whether or not x is gathered)
 *   num_experts_off  entries of expert_offsets minus one; may exceed the
 *                    route's num_experts, and rows of experts past the table
 *                    are base rows
 *   row_adapter      device int32 [num_tokens] adapter slot per token, or NULL
 *                    (every row on slot 0)
 *   x                x_gather == 0: sorted rows, row r at x + r*x_row_stride;
 *                    x_gather != 0: token-major rows, x + t*x_row_stride with
 *                    t = sorted_token_ids[r]
 *   xa               device BF16 [xa_rows_cap, max_rank]; row r is written at
 *                    the window-local row r - row_offset; rows that do not
 *                    fold are written as zeros
 *   workspace        see rld_moe_grouped_workspace_bytes (RLD_ENOSPACE if
 *                    workspace_bytes is smaller than it for this window)
 * The launch shape depends only on the host arguments (route sizes and the
 * window), so a captured call replays with new routing contents; an empty
 * window (row_end == row_offset) launches nothing and returns RLD_OK.  A
 * row's xa depends only on its own x row, so a full-window call and the union
 * of its chunk windows are bit-identical.
 * RLD_EUNSUPPORTED if max_loras * num_experts > 2048 (the per-launch pair
 * list) or num_experts_off >= 1024 (offsets staged on chip); RLD_ENOSPACE if
 * row_end - row_offset > xa_rows_cap. */
int rld_moe_grouped_shrink(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                           int x_gather, uint32_t num_tokens, const int32_t* expert_offsets,
                           uint32_t num_experts_off, const int32_t* sorted_token_ids,
                           const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end,
                           void* xa, uint32_t xa_rows_cap, void* workspace,
                           size_t workspace_bytes, void* stream);

/* MoE grouped fold expand + fold of the same window into the sorted base_out
 * ([te, out_row_stride] BF16, row r folded in place). */
int rld_moe_grouped_expand_fold(const rld_moe_route* route, const void* xa, uint32_t num_tokens,
                                const int32_t* expert_offsets, uint32_t num_experts_off,
                                const int32_t* sorted_token_ids, const int32_t* row_adapter,
                                uint32_t row_offset, uint32_t row_end, void* base_out,
                                uint32_t out_row_stride, void* stream);

/* moe_lora_grouped_down for one window: shrink then expand + fold, with the
 * results of the two calls above (xa written the same way, base_out folded
 * bit-identically).  When 1024 < k_in <= 2048, max_rank <= 32 and
 * n_out <= 768 both stages run in one launch, each block folding the rows it
 * has just contracted; otherwise it is the two launches. */
int rld_moe_grouped(const rld_moe_route* route, const void* x, uint32_t x_row_stride,
                    int x_gather, uint32_t num_tokens, const int32_t* expert_offsets,
                    uint32_t num_experts_off, const int32_t* sorted_token_ids,
                    const int32_t* row_adapter, uint32_t row_offset, uint32_t row_end,
                    void* base_out, uint32_t out_row_stride, void* xa, uint32_t xa_rows_cap,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Two projections that read the same x rows under the same routing -- a gated
 * FFN's gate and up -- over one window: the results of rld_moe_grouped(route_a,
 * ..., base_a, os_a, xa_a, ...) followed by rld_moe_grouped(route_b, ...,
 * base_b, os_b, xa_b, ...), bit for bit.  When both routes have the same k_in,
 * max_rank, max_loras and num_experts, 1024 < k_in <= 2048, max_rank <= 32,
 * both n_out <= 768 and max_loras * num_experts <= 512, it is one launch that
 * shares the row scan between the projections; otherwise it is those two
 * calls (the workspace then serves them in turn).  A (slot, expert) pair that
 * only one route adapts folds in that projection alone; xa rows of the other
 * are written as zeros.  Errors as rld_moe_grouped for either route. */
int rld_moe_grouped_pair(const rld_moe_route* route_a, const rld_moe_route* route_b,
                         const void* x, uint32_t x_row_stride, int x_gather, uint32_t num_tokens,
                         const int32_t* expert_offsets, uint32_t num_experts_off,
                         const int32_t* sorted_token_ids, const int32_t* row_adapter,
                         uint32_t row_offset, uint32_t row_end, void* base_a, uint32_t os_a,
                         void* base_b, uint32_t os_b, void* xa_a, void* xa_b,
                         uint32_t xa_rows_cap, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------ diagnostics -- */

const char* rld_status_string(int status);
/* HIP error code of the last failed launch on this thread (0 if none). */
int rld_last_hip_error(void);
const char* rld_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RLD_H */
