/*
 * pagedkv.h -- C ABI of the paged KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * The method (web pages, cited by title and section):
 *  - "KV Cache Optimization and PagedAttention" (cracklab.in): each token's K and V are
 *    stored once and reused by every later token; the cache is split into small
 *    fixed-size blocks held in any free physical blocks, with a per-request block
 *    table mapping logical to physical blocks as an operating system's page table maps pages; requests with a common
 *    prefix can point at the same physical blocks (copy-on-write).
 *  - "PagedAttention: Optimizing KV Cache Utilization in Large Language Models"
 *    (fromzero2ai.dev): "The Mechanics of PagedAttention" (logical blocks, physical
 *    blocks, page table; blocks granted as tokens are generated, K/V written into scattered
 *    blocks), "The Math: Block Attention Calculation" (softmax(q.K^T / sqrt(d_k)) with the
 *    keys located through the page table), "Conclusion" (blocks can run out
 *    mid-generation; block size trades table lookups against final-block waste).
 *  - "KV Cache Management" (ai360xpert.com): "The Solution: PagedAttention (vLLM)" (one
 *    block at a time, the next need not be adjacent), "The Bonus: Zero-Copy Sharing",
 *    "What to Read Next" (8-bit KV cache).
 *
 * Conventions shared by every entry point
 *  - All functions return PA_OK (0) or a negative status; on a negative status
 *    pa_last_error() returns a message for the calling thread and nothing was enqueued
 *    (device calls) or changed (allocator calls).
 *  - Device pointers are borrowed for the duration of the enqueued work only; the caller
 *    owns every buffer and keeps it alive until the stream has passed the call.  The
 *    library allocates no device memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Work is enqueued
 *    asynchronously; launch failures return PA_ERR_DEVICE.
 *  - Tensors are dense and row-major (C order) in the shapes stated; device pointers must
 *    be 16-byte aligned.
 *
 * Cache layout (the pages fix none): k_cache and v_cache are each
 *     [num_blocks][num_kv_heads][block_size][head_dim]
 * of the cache storage type; token slot s lives in block s / block_size at row
 * s % block_size.  One (block, head) tile is one contiguous span of
 * block_size * head_dim elements.  An MXFP4 cache ("8-bit or 4-bit": "KV Cache Management",
 * "Watch Out For") keeps the same [num_blocks][num_kv_heads] tiles, each of
 *     block_size * head_dim / 2 bytes of E2M1 codes, row-major [block_size][head_dim / 2], two
 *       per byte (the even dim in the low nibble), then
 *     block_size * head_dim / 32 bytes of E8M0 scales, row-major [block_size][head_dim / 32]
 * (one scale 2^(byte - 127) per 32 consecutive dims of a token row; 0xFF is NaN).
 *
 * Supported combinations (others return PA_ERR_UNSUPPORTED):
 *   (q / K,V input / out, cache) in {(f32, f32), (bf16, bf16), (bf16, fp8 e4m3), (bf16, mxfp4)},
 *   and for pa_kv_write also (f32 K,V input, fp8 e4m3 cache),
 *   head_dim in {64, 128}, block_size in {8, 16, 32, 128},
 *   num_q_heads / num_kv_heads in {1, 4, 8}.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status and types */

#define PA_OK               0
#define PA_ERR_INVALID     -1   /* bad argument: shape, pointer, id, contract violation  */
#define PA_ERR_UNSUPPORTED -2   /* valid but not built: dtype / head_dim / block / group */
#define PA_ERR_NO_BLOCKS   -3   /* the allocator's free queue cannot cover the request   */
#define PA_ERR_DEVICE      -4   /* a HIP runtime call or kernel launch failed            */

#define PA_DTYPE_F32      0     /* IEEE binary32                                          */
#define PA_DTYPE_BF16     1     /* bfloat16                                               */
#define PA_DTYPE_FP8_E4M3 2     /* OCP FP8 E4M3FN (bias 7, max 448, no inf), cache only   */
#define PA_DTYPE_MXFP4    3     /* OCP MXFP4: E2M1 codes, E8M0 scale per 32 dims; cache only */

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);

/* Library ABI version; bumped on any signature change. */
int32_t pa_abi_version(void);

/* ---------------------------------------------------------------- KV write
 *
 * Slot-mapped write of new tokens' K and V into their physical blocks ("The Mechanics of
 * PagedAttention": the K/V vectors are written into the blocks even when those are
 * scattered).  For every token t with slot_mapping[t] >= 0 and every KV head h:
 *     k_cache[s / block_size][h][s % block_size][:] = enc_h(k[t][h][:]),  s = slot_mapping[t]
 * and the same for v.  enc is a bit copy when cache_dtype == in_dtype; for an fp8 cache
 * (in_dtype bf16 or f32) enc_h(x) = e4m3_round_nearest_even_saturate(float32(x / k_scale[h]))
 * (v_scale for v): the float32 quotient is correctly rounded, magnitudes beyond 448
 * saturate to 448, NaN stays NaN.  For an MXFP4 cache (in_dtype bf16, k_scale = v_scale =
 * NULL) each 32 dims of a row are one block: E = floor(log2(max |x|)) - 2 clamped to
 * [-127, 127] (-127 for a block of zeros), codes = e2m1_round_nearest_even_saturate(x / 2^E),
 * scale byte E + 127; a block with NaN or infinity stores scale 0xFF and zero codes.
 *
 *  k, v          device, [num_tokens][num_kv_heads][head_dim] of in_dtype
 *  slot_mapping  device, int64 [num_tokens]; < 0 means "skip this token" (padding)
 *  k_cache, v_cache  device, cache layout above, of cache_dtype
 *  k_scale, v_scale  device, float32 [num_kv_heads]; required for an fp8 cache, else NULL
 *
 * Contract (not checked on the device; out-of-range slots are skipped, never written):
 * slots are < num_blocks * block_size and pairwise distinct within one call.  The write
 * never touches a slot that is not listed.
 */
int pa_kv_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int32_t in_dtype, int32_t cache_dtype,
                const float* k_scale, const float* v_scale, void* stream);

/* ---------------------------------------------------------------- decode attention
 *
 * Decode attention through the block table ("The Math: Block Attention Calculation").
 * For request b with L = seq_lens[b] cached tokens (the new token included) and query head
 * h, with KV head g = h / (num_q_heads / num_kv_heads):
 *     K_j = dec(k_cache[block_tables[b][j / block_size]][g][j % block_size][:]),  j < L
 *     s_j = scale * <q[b][h][:], K_j>
 *     out[b][h][:] = sum_j softmax(s)_j * V_j            (one softmax over all L keys)
 * dec is exact (fp8: e4m3 value times k_scale[g] / v_scale[g]).  Scores, softmax and the
 * weighted sum are accumulated in float32; out is rounded to nearest even in q's dtype.
 * L = 0 gives out = 0.  Slots at positions >= L are never read (they may hold anything).
 *
 * Long contexts are split into partitions of `partition_tokens` logical tokens; each partition
 * is reduced to (max score, sum of exponentials, unnormalised weighted sum) and the
 * partitions are merged by rescaling to the largest maximum (log-sum-exp).  An explicit
 * partition_tokens > 0 is rounded up to a multiple of max(64, block_size).  0 chooses it
 * automatically (pa_decode_partition_tokens gives the value): with fewer (request, KV head)
 * pairs than S = the device's compute units (bf16, f32 caches) or twice that (fp8, 4-bit
 * caches), each request is cut into ceil(S / pairs) equal partitions of
 * ceil(max_seq_len / parts) tokens (one or two work-groups per compute unit); otherwise
 * partitions are 512 tokens.  For a given partition size the result depends only on logical
 * positions, so it is bit-identical under any physical placement of the blocks.
 *
 *  out           device, [num_seqs][num_q_heads][head_dim] of q_dtype
 *  q             device, [num_seqs][num_q_heads][head_dim] of q_dtype
 *  k_cache, v_cache  device, cache layout above, num_blocks blocks, of cache_dtype
 *  block_tables  device, int32 [num_seqs][max_blocks_per_seq]; entries past
 *                ceil(L / block_size) are ignored
 *  seq_lens      device, int32 [num_seqs]
 *  max_seq_len   host upper bound of seq_lens (sizes the grid and the workspace)
 *  workspace     device scratch of at least pa_decode_workspace_bytes(...) bytes, or NULL
 *                (then each request is reduced in a single partition, which is correct but
 *                slow for long contexts).  It holds the partitions' partial results and merge
 *                ticket counters: the last work-group of each group of 16 partitions of a
 *                request and KV head merges that group, and with more than one group the last
 *                group-merger merges the groups, all in the same launch.  The ticket counters
 *                (and two counters that hand out work items on long, few-request batches)
 *                sit at the start of the workspace, in a region whose place and size depend
 *                only on (num_seqs, num_q_heads, max_seq_len), and every call leaves them at
 *                zero.  Zero the workspace (pa_decode_workspace_init) before its first use and
 *                whenever it is reused with a different (num_seqs, num_q_heads, max_seq_len);
 *                calls that differ only in num_kv_heads, head_dim, block_size,
 *                partition_tokens, cache_dtype or the device's compute units (all of which
 *                change the partition count and the partial rows' layout, never the ticket
 *                region) need no re-zeroing.  Calls that share a workspace must not run
 *                concurrently (order them on one stream).
 *
 * Device-side faults are turned into loud results instead of out-of-bounds accesses: a
 * request whose L exceeds max_seq_len or max_blocks_per_seq * block_size, or whose table
 * holds a block id outside [0, num_blocks) within its first ceil(L / block_size) entries,
 * gets out = NaN for all its heads.
 */
int64_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, int32_t partition_tokens,
                                  int32_t block_size, int32_t cache_dtype);

/* The partition size in tokens that pa_decode uses for these sizes and cache type on the
 * current device (partition_tokens as passed to pa_decode; 0 = automatic), or a negative
 * status. */
int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                   int32_t partition_tokens, int32_t block_size, int32_t cache_dtype);

/* Zero a decode workspace (a store kernel on `stream`; no memset node is recorded, so this
 * may be captured in a graph).  workspace_bytes must be a multiple of 4. */
int pa_decode_workspace_init(void* workspace, int64_t workspace_bytes, void* stream);

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, float scale,
              int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
              const float* k_scale, const float* v_scale,
              void* workspace, int64_t workspace_bytes, int32_t partition_tokens, void* stream);

/* ---------------------------------------------------------------- append and decode in one launch
 *
 * One decode step of a layer in one launch: the slot-mapped write of each request's new token
 * ("The Mechanics of PagedAttention": the new K/V are written into the request's physical
 * block, wherever it is) and the decode over the tokens including it ("The Math: Block
 * Attention Calculation").  For every request b with L = seq_lens[b] >= 1 and every KV head h,
 * the token at logical position L - 1 is written through the block table --
 *     slot = block_tables[b][(L - 1) / block_size] * block_size + (L - 1) % block_size
 * -- with k_new[b][h][:] and v_new[b][h][:] exactly as pa_kv_write writes a slot (bit copy,
 * fp8 quantisation with k_scale / v_scale, or MXFP4), and then out is computed as pa_decode
 * computes it.  The result (cache bytes and out) is bit-identical to pa_kv_write of those
 * slots followed by pa_decode with the same arguments.  Only the one wave that reads position
 * L - 1 touches the row: over bf16 caches it stores the row when it reaches that position and
 * uses the new values for it directly; over fp8 and MXFP4 caches it writes the row before its
 * first load and waits for the stores.
 *  k_new, v_new  device, [num_seqs][num_kv_heads][head_dim] of q_dtype (bf16), 16-byte aligned
 *  the other arguments as pa_decode; the caches are written (position L - 1 only).
 * Contract: the caller has appended the token in the allocator (pa_seq_append or
 * pa_batch_append, copy-on-write pairs copied), so position L - 1 maps to a slot that belongs
 * to this request alone.  Float32 caches are not supported (PA_ERR_UNSUPPORTED: use the two
 * calls).  A table entry outside [0, num_blocks) at position L - 1 is not written; the request's
 * output is NaN as in pa_decode. */
int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens, float scale, int32_t block_size,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_seq_len, int32_t q_dtype,
                     int32_t cache_dtype, const float* k_scale, const float* v_scale, void* workspace,
                     int64_t workspace_bytes, int32_t partition_tokens, void* stream);

/* ---------------------------------------------------------------- decode without allocation
 *
 * For callers that cannot allocate device memory or hand the library a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation, arguments and results as pa_decode (bit for bit: the same kernels and
 * partitions) without (workspace, workspace_bytes): the split-K partials and merge tickets live
 * in a static device array of PA_NOALLOC_SCRATCH_BYTES inside the library, which every device
 * the library runs on holds until the process ends.
 *  - Sizes whose pa_decode_workspace_bytes(...) exceeds PA_NOALLOC_SCRATCH_BYTES return
 *    PA_ERR_INVALID with nothing enqueued (128 MiB holds, for example, 256 requests x 32 q heads
 *    up to 8192 tokens in 512-token partitions, or 2 x 64 heads at 131072 tokens).
 *  - Nothing is allocated or freed: no hipMalloc, hipFree or allocating library routine.  The
 *    first call on a device, with that device current, looks the array's address up once.
 *  - Every call on one device shares that device's array, which keeps the last call's
 *    contents.  When a call's ticket counters reach past the bytes earlier calls left at zero,
 *    the call first clears them with a store kernel on `stream` (no memset node).
 *  - Calls that overlap on one device (on different streams, or from several threads without
 *    ordering on one stream) race on the array and give undefined results. */
#define PA_NOALLOC_SCRATCH_BYTES (128 * 1024 * 1024)

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, float scale,
                      int32_t block_size, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_seq_len, int32_t q_dtype, int32_t cache_dtype,
                      const float* k_scale, const float* v_scale, int32_t partition_tokens, void* stream);

/* ---------------------------------------------------------------- prefill attention
 *
 * Attention of several new tokens per request through the block table, causal: the step
 * before decode, where a prompt's (or a chunk of it) keys and values are computed once and
 * stored ("KV Cache Management", "Why Does This Exist?") and a token's attention covers every
 * token before it ("KV Cache Optimization and PagedAttention", first paragraph).  The new
 * tokens' K/V are written first (pa_kv_write), so for request b with L = seq_lens[b] cached
 * tokens and n = query_start[b+1] - query_start[b] new ones (its last n tokens), new token i
 * (q row query_start[b] + i) sits at logical position L - n + i and, for every query head h
 * with KV head g = h / (num_q_heads / num_kv_heads):
 *     out[query_start[b] + i][h][:] = sum_{j <= L - n + i} softmax_j(scale * <q_i, K_j>) V_j
 * with K_j, V_j read through the table as in pa_decode.  Tokens before the new ones (a cached
 * prefix, earlier chunks) are read from the cache like the new ones.  Scores, softmax and
 * sums in float32 (the weights multiplied into V rounded to bf16, and the denominator sums
 * those rounded weights); out rounded to nearest even.
 *
 *  out, q        device, [num_query_tokens][num_q_heads][head_dim] bf16
 *  query_start   device, int32 [num_seqs + 1], non-decreasing, query_start[num_seqs] <=
 *                num_query_tokens (rows of request b: query_start[b] .. query_start[b+1]-1)
 *  seq_lens      device, int32 [num_seqs], L >= n
 *  block_tables  device, int32 [num_seqs][max_blocks_per_seq]
 *  max_query_len host upper bound of n; max_seq_len host upper bound of L
 *
 *  k_scale, v_scale  device, float32 [num_kv_heads]: required for an fp8 cache (K_j, V_j are
 *                then the stored values times the head's scale, as in pa_decode), ignored
 *                otherwise; an MXFP4 cache carries its own scales
 *
 * Supported: bf16 q; bf16, fp8 E4M3 or MXFP4 cache; head_dim {64, 128}, block_size {8, 16, 32,
 * 128}, num_q_heads / num_kv_heads in {1, 4, 8}.  One kernel launch; no workspace.  A request whose
 * query range is inconsistent (decreasing, negative or past num_query_tokens) is not written;
 * one with n > L, n > max_query_len, L > max_seq_len or L > max_blocks_per_seq * block_size,
 * or whose table holds an id outside [0, num_blocks) where positions are read, gets NaN in the
 * rows of the query tiles that cover it (n > max_query_len: its first max_query_len rows). */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
               float scale, int32_t block_size, int32_t num_seqs, int64_t num_query_tokens,
               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
               int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_seq_len,
               int32_t q_dtype, int32_t cache_dtype, const float* k_scale, const float* v_scale,
               void* stream);

/* ---------------------------------------------------------------- block copy
 *
 * Whole-block copies for copy-on-write ("KV Cache Optimization and PagedAttention", prose
 * on shared prefix blocks and copy-on-write): for each pair i,
 *     k_cache[src_dst[2i+1]] = k_cache[src_dst[2i]]   (all heads, rows and dims), same for v.
 *  src_dst  device, int64 [num_pairs][2] (src, dst); destinations pairwise distinct and
 *           never a source of another pair in the same call; pairs with an id outside
 *           [0, num_blocks) are skipped.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst, int32_t num_pairs,
                   int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t cache_dtype, void* stream);

/* ---------------------------------------------------------------- block-table upload
 *
 * The host -> device leg of the block-table export: the tables live in the host allocator
 * ("KV Cache Optimization and PagedAttention", prose on paging: each request's table maps its
 * logical blocks to physical ones), and every decode step hands the changed rows, lengths and
 * new tokens' slots to the device before the step's writes and decodes.
 *     dst[0 .. bytes) = src[0 .. bytes)
 * by one kernel on `stream`, so the copy is ordered with the stream's kernels on one queue, with
 * no copy engine and no cross-queue wait.  The kernel reads src with system-scope loads, which
 * bypass the device caches: it sees what the host wrote to pinned memory before the call.
 *  dst, src  16-byte aligned; each range must lie inside one HIP allocation, device memory or
 *            pinned host memory allocated by HIP (checked before the launch; pageable host
 *            memory gives PA_ERR_INVALID).  The ranges must not overlap.
 *  bytes     a multiple of 16, below 2^31.
 * The caller keeps src unchanged until the stream has passed the call (e.g. one pinned buffer
 * per step in flight). */
int pa_upload(void* dst, const void* src, int64_t bytes, void* stream);

/* ---------------------------------------------------------------- measurement reference
 *
 * Plain streaming reads, the references the decode's HBM rate is set against on the same device
 * and at the same sizes (the decode is a bandwidth-bound read of the cache, "The Math: Block
 * Attention Calculation": every step reads each request's whole cached history).  Every byte of
 * [src, src + bytes) is loaded once with non-temporal 16-byte loads by one work-group of four
 * waves per compute unit; the loaded words are folded per lane and nothing is written (the sink
 * is written only when a fold equals one fixed constant, which keeps the loads live).
 *  pattern     PA_PROBE_GRID: a grid-stride sweep (the whole device reads one compact window at
 *              a time); PA_PROBE_RANGES: work-group j reads its own contiguous range of 4 KiB
 *              tiles (the decode's partitions, without a block table); PA_PROBE_TILES: passes of
 *              two tiles taken through tile_order, split over work-groups and waves as the
 *              decode's uniform grid splits its passes, each pass moved straight to LDS (given
 *              the K and V tiles of every pass of a decode, its memory traffic without its
 *              arithmetic)
 *  src         device, 16-byte aligned; bytes a multiple of 16 (GRID) or of 4096 (RANGES,
 *              TILES), else PA_ERR_INVALID
 *  tile_order, order_len  PA_PROBE_TILES: device, int32 [order_len] (even), the indices of src's
 *              4 KiB tiles to read, two per pass (entries outside [0, bytes / 4096) are clamped
 *              into it); else ignored
 *  sink        device, at least 4 x (compute units) bytes (else PA_ERR_INVALID)
 * Enqueued on `stream`; computes nothing the caller reads. */
#define PA_PROBE_GRID 0
#define PA_PROBE_RANGES 1
#define PA_PROBE_TILES 2
int pa_probe_read(const void* src, int64_t bytes, int32_t pattern, const int32_t* tile_order, int64_t order_len,
                  void* sink, int64_t sink_bytes, void* stream);

/* ---------------------------------------------------------------- tensor-view entry points
 *
 * pa_kv_write and pa_decode over non-owning tensor views, for callers that hold shapes and
 * strides rather than loose sizes.  Each view is checked on the host -- dtype, rank, shape
 * agreement between the arguments, C-contiguity -- before the plain entry point is called with
 * the sizes read from the views; a mismatch returns PA_ERR_INVALID (or PA_ERR_UNSUPPORTED)
 * naming the argument, with nothing enqueued.  Same computation and results as the plain calls.
 *
 *  pa_tensor  data: device pointer; dtype: PA_DTYPE_*; ndim, shape[0 .. ndim), stride[0 .. ndim)
 *             in elements (C-contiguous: stride[ndim-1] = 1, stride[i] = stride[i+1] * shape[i+1]).
 *             An MXFP4 cache is given as dtype PA_DTYPE_MXFP4 with the logical shape
 *             [num_blocks][num_kv_heads][block_size][head_dim] and all strides 0 (its tiles are
 *             packed as the cache layout above states).
 *  pa_opts    nullable; zero fields take the defaults: stream NULL, no workspace (one partition
 *             per request), partition_tokens 0 (automatic), max_seq_len 0 (the table's capacity,
 *             max_blocks_per_seq * block_size), k_scale / v_scale NULL (required for fp8 caches).
 */
#define PA_DTYPE_I32 4          /* int32 index tensor (block tables, lengths)                */
#define PA_DTYPE_I64 5          /* int64 index tensor (slot mapping)                         */

typedef struct {
    void* data;
    int32_t dtype;
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} pa_tensor;

typedef struct {
    void* stream;
    void* workspace;
    int64_t workspace_bytes;
    int32_t partition_tokens;
    int32_t max_seq_len;
    const float* k_scale;
    const float* v_scale;
} pa_opts;

/* k, v: [num_tokens][num_kv_heads][head_dim]; slot_mapping: int64 [num_tokens]; caches as above. */
int pa_kv_write_t(const pa_tensor* k, const pa_tensor* v, const pa_tensor* slot_mapping, pa_tensor* k_cache,
                  pa_tensor* v_cache, const pa_opts* opts);

/* out, q: [num_seqs][num_q_heads][head_dim]; caches [num_blocks][num_kv_heads][block_size][head_dim];
 * block_tables: int32 [num_seqs][max_blocks_per_seq]; seq_lens: int32 [num_seqs]. */
int pa_decode_t(pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                const pa_tensor* block_tables, const pa_tensor* seq_lens, float scale, int32_t block_size,
                const pa_opts* opts);

/* ---------------------------------------------------------------- host block allocator
 *
 * CPU-only bookkeeping of the block pool; never touches the device.  One handle is used
 * by one thread at a time.  Rules:
 *  - a free FIFO queue (initial order given, identity if NULL); grants pop the head,
 *    releases push to the tail (the pages let any free block be granted; FIFO is this library's choice);
 *  - blocks are granted on demand: appending token n of a sequence takes a new block when
 *    n % block_size == 0 ("The Solution: PagedAttention (vLLM)");
 *  - slot of token n = block * block_size + n % block_size;
 *  - fork(parent, child) makes child share all of parent's blocks (refcount + 1 each)
 *    ("The Bonus: Zero-Copy Sharing");
 *  - copy-on-write: appending into a partially filled last block with refcount > 1 first
 *    moves the sequence to a fresh block and reports the (old, new) pair, which the caller
 *    copies with pa_copy_blocks before writing; shared blocks are never written;
 *  - free(seq) drops one reference of each of its blocks in logical order; blocks reaching
 *    zero join the free queue tail in that order;
 *  - any operation that cannot be completed (PA_ERR_NO_BLOCKS, unknown or duplicate ids)
 *    changes nothing; PA_ERR_NO_BLOCKS from an append or a swap-in also counts one
 *    exhaustion event ("Conclusion": blocks can run out mid-generation; preemption is the
 *    caller's decision);
 *  - preemption by swapping ("Conclusion": a preempted request's KV cache is recomputed or
 *    swapped): a second pool of host blocks, with its own FIFO queue (identity order) and
 *    refcounts, holds the blocks of swapped-out sequences (pa_swap_out / pa_swap_in below).
 *    A swapped-out sequence can only be swapped in, freed or queried.
 */
typedef struct pa_allocator pa_allocator;

typedef struct {
    int64_t free_blocks;        /* blocks in the free queue                              */
    int64_t used_blocks;        /* blocks with refcount > 0                              */
    int64_t total_refs;         /* sum of refcounts = resident sequences' table entries  */
    int64_t exhaustion_events;  /* appends and swap-ins refused with PA_ERR_NO_BLOCKS    */
    int64_t waste_slots;        /* sum over resident sequences of ceil(n/bs)*bs - n      */
    int64_t num_seqs;           /* live sequences (resident and swapped out)             */
    int64_t host_free_blocks;   /* host pool: blocks in its free queue                   */
    int64_t host_used_blocks;   /* host pool: blocks with refcount > 0                   */
    int64_t swapped_seqs;       /* sequences whose blocks are in the host pool           */
    int64_t cached_blocks;      /* prefix cache: device blocks registered under content  */
    int64_t cache_hit_blocks;   /* prefix cache: blocks taken from the cache by prompts  */
    int64_t cache_evictions;    /* prefix cache: registered blocks handed out again      */
} pa_alloc_stats_t;

/* num_blocks > 0, block_size > 0; initial_free_order: host int32 [num_blocks], a
 * permutation of 0..num_blocks-1, or NULL.  *out receives a handle owned by the caller. */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                    pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

int pa_seq_add(pa_allocator* a, int64_t seq_id);

/* Append n_tokens to one sequence.  slots_out: host int64 [n_tokens]; cow_out: host int64
 * [2] receiving (src, dst) when *n_cow_out == 1 (at most one copy per append). */
int pa_seq_append(pa_allocator* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                  int64_t* cow_out, int32_t* n_cow_out);

/* Append n_tokens[i] to each of n_seqs distinct sequences, in order, all or nothing.
 * slots_out: host int64 [sum n_tokens] (sequence-major); cow_out: host int64
 * [2 * n_seqs]; *n_cow_out receives the number of (src, dst) pairs written. */
int pa_batch_append(pa_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                    int32_t n_seqs, int64_t* slots_out, int64_t* cow_out, int32_t* n_cow_out);

int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);
int pa_seq_free(pa_allocator* a, int64_t seq_id);

/* ---------------------------------------------------------------- prefix caching
 *
 * "KV Cache Management", "The Bonus: Zero-Copy Sharing": the KV cache of a system prompt that
 * many users share is computed and stored once, and every user's block table points at the
 * same block; "KV Cache Optimization and PagedAttention", first paragraph, names this prefix
 * caching.  Here a block is registered under its content -- the whole token prefix from
 * token 0 to the block's end -- when a sequence whose token ids are all known fills it.
 * Rules:
 *  - content is compared exactly (token ids and the whole prefix before them);
 *  - a block whose content is already registered to another block is not registered;
 *  - a registered block at refcount 0 stays registered while it waits in the free queue; when
 *    the queue hands it out again its registration is dropped (eviction, in release order);
 *  - only sequences created empty or by pa_seq_add_prompt and grown by pa_seq_append_tokens
 *    have known token ids; pa_seq_append / pa_batch_append make them unknown for good (no
 *    later block of that sequence is registered); fork copies the parent's state; a
 *    swapped-in sequence's blocks are fresh and unregistered, later ones are registered. */

/* Create sequence seq_id holding the n_tokens prompt tokens: from block 0 on, every block
 * whose content equals the prompt's prefix is taken from the cache (refcount + 1; a free one
 * leaves the free queue), stopping at the first block that is not registered; *n_cached_out
 * receives the tokens so covered (a multiple of block_size), whose K/V the caller does not
 * write.  The remaining n_tokens - *n_cached_out tokens are appended as by
 * pa_seq_append_tokens; slots_out (host int64 [n_tokens - *n_cached_out]) receives their
 * slots.  PA_ERR_NO_BLOCKS (nothing changed, one exhaustion event) if the free blocks not
 * taken as hits cannot hold the rest. */
int pa_seq_add_prompt(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                      int32_t* n_cached_out, int64_t* slots_out);

/* pa_seq_append with the new tokens' ids (host int32 [n_tokens]): every block the append
 * fills is registered under its content. */
int pa_seq_append_tokens(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                         int64_t* slots_out, int64_t* cow_out, int32_t* n_cow_out);

/* registered[b] = 1 if device block b is registered in the prefix cache, else 0 (host int32
 * [num_blocks]). */
int pa_alloc_dump_cached(const pa_allocator* a, int32_t* registered);

/* Rows of physical block ids for the given sequences, padded with -1, and their token
 * counts.  tables_out: host int32 [n_seqs][max_blocks]; seq_lens_out: host int32 [n_seqs].
 * PA_ERR_INVALID if a sequence holds more than max_blocks blocks. */
int pa_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs,
                    int32_t max_blocks, int32_t* tables_out, int32_t* seq_lens_out);

int pa_alloc_stats(const pa_allocator* a, pa_alloc_stats_t* out);

/* Full state for comparison: refcounts [num_blocks], free queue in order (n_free entries
 * of a buffer of num_blocks). */
int pa_alloc_dump(const pa_allocator* a, int32_t* refcounts, int32_t* free_order,
                  int32_t* n_free);

/* ---------------------------------------------------------------- preemption by swapping
 *
 * "PagedAttention: Optimizing KV Cache Utilization in Large Language Models", "Conclusion":
 * when blocks run out mid-generation, requests are preempted and their KV cache is
 * recomputed or swapped.  Swapping here moves whole blocks between the device pool and a
 * pool of the same block shape in pinned host memory, bit for bit, so a request resumes
 * with exactly the cache it had (and, decode being independent of block placement, exactly
 * the outputs it would have had).
 *
 * (Re)creates the host pool with num_host_blocks blocks (ids 0..num_host_blocks-1, free
 * queue in identity order).  PA_ERR_INVALID while any sequence is swapped out. */
int pa_alloc_set_host_blocks(pa_allocator* a, int32_t num_host_blocks);

/* Swap out the n_seqs listed sequences (distinct, resident).  Their blocks are walked in
 * list order, each in logical order; every distinct device block gets one host block from
 * the host queue head and the pair (device id, host id) is written to pairs_out (host int64
 * [max_pairs][2]) in that order; each reference moves to the host block, and the device
 * reference is dropped as pa_seq_free would (blocks reaching 0 join the device queue tail).
 * A block also held by a resident sequence stays allocated for it and is copied.  The caller
 * copies the pairs with pa_swap_blocks (device pool -> host pool) on the stream that later
 * writes the freed blocks, before those writes.  PA_ERR_NO_BLOCKS if the host queue holds
 * fewer blocks than the distinct blocks; PA_ERR_INVALID if they exceed max_pairs. */
int pa_swap_out(pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int64_t* pairs_out,
                int32_t max_pairs, int32_t* n_pairs_out);

/* Swap the listed sequences (distinct, swapped out) back in: the mirror image of
 * pa_swap_out, with pairs (host id, device id), device blocks from the device queue head and
 * host blocks reaching 0 joining the host queue tail.  The caller copies the pairs with
 * pa_swap_blocks (host pool -> device pool) before the sequences' next decode.
 * PA_ERR_NO_BLOCKS (one exhaustion event) if the device queue is too short. */
int pa_swap_in(pa_allocator* a, const int64_t* seq_ids, int32_t n_seqs, int64_t* pairs_out,
               int32_t max_pairs, int32_t* n_pairs_out);

/* 1 if the sequence is swapped out, 0 if resident, negative status if unknown. */
int pa_seq_is_swapped(const pa_allocator* a, int64_t seq_id);

/* Host pool state: refcounts [num_host_blocks], free queue in order (*n_free entries). */
int pa_alloc_dump_host(const pa_allocator* a, int32_t* refcounts, int32_t* free_order,
                       int32_t* n_free);

/* Whole-block copies between two pools of the same block shape, either of which may be
 * device memory or pinned host memory (allocated by HIP, e.g. hipHostMalloc): for each pair
 * i with both ids in range,
 *     dst_k[src_dst[2i+1]] = src_k[src_dst[2i]]   (all heads, rows and dims), same for v.
 * The copy is one kernel on `stream` that reads and writes host memory directly over the
 * host link (no staging).  Every pointer (the four pools over their whole extent and
 * src_dst over 2 * num_pairs entries) is checked before the launch to lie inside one HIP
 * allocation, device or pinned host; pageable host memory gives PA_ERR_INVALID.
 *  src_dst  device or pinned host int64 [num_pairs][2]; destinations pairwise distinct;
 *           pairs with an id outside [0, src_num_blocks) / [0, dst_num_blocks) are skipped. */
int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int64_t* src_dst, int32_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t cache_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
