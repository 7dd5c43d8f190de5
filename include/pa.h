/*
 * pa.h -- C ABI of the paged-KV attention library (libpa.so) for AMD gfx950.
 *
 * Five operations, all defined on the pages this library follows:
 *
 *   pa_decode       attention of one query token per head over a KV cache kept
 *                   in fixed-size physical blocks, found through a per-sequence
 *                   block table and bounded by per-sequence context lengths
 *                   (page "vLLM推理引擎架构：PagedAttention机制与高吞吐推理",
 *                   section 2.3 "PagedAttention Kernel": the kernel takes
 *                   output, query, key_cache, value_cache, block_tables,
 *                   context_lens and block_size, fills the caller's output,
 *                   locates each token's block through the table and
 *                   accumulates attention across blocks; the logical-to-physical
 *                   translation itself is section 5.1 of page
 *                   "vLLM框架中的KV cache优化与PagedAttention机制详解").
 *   pa_decode_layers  pa_decode over several layers' caches in one launch,
 *                   all layers sharing the block tables.
 *   pa_prefill      the same attention for several query tokens per sequence
 *                   (a prompt chunk, or draft tokens being verified), each
 *                   token seeing the context up to its own position; the
 *                   query tensor of the same section holds one row per token.
 *   pa_cache_write  scatter of new tokens' K/V rows into physical slots
 *                   (slot = block * block_size + offset, the address rule of
 *                   page "Paged KVCache：大模型推理显存管理优化方案", section 2.3).
 *   pa_copy_blocks  copies of whole blocks, between or within pools: the
 *                   private copy a sequence takes of a shared block before
 *                   writing into it (section 5.1, step 4, of the first page
 *                   above), and the swap of blocks between GPU memory and host
 *                   memory (section 5 of the page just cited).
 *
 * Conventions shared by every entry point
 *   - Every buffer is device memory owned by the caller.  No call allocates or
 *     frees device memory, and no call synchronises with the host: work is
 *     enqueued on opts->stream (NULL = the null stream) and the call returns.
 *     A call enqueues kernel launches only (no memset, no copy), and every
 *     kernel leaves its workspace counters at zero, so calls may be captured
 *     into a HIP graph on a capturing stream and the graph replayed on the
 *     same buffers.
 *   - Tensors are described by pa_tensor: a device pointer, a pa_dtype, a rank
 *     and per-dimension sizes and strides counted in ELEMENTS.  The last
 *     dimension must be contiguous (stride 1); the data pointer and every
 *     other stride (in bytes) must be multiples of 16.
 *   - Errors are returned as pa_status; a thread-local message with the
 *     details is available from pa_last_error().  Validation happens on the
 *     host before anything is enqueued, so a non-OK return enqueued nothing
 *     (except PA_ERR_HIP, reported if a launch itself fails).
 *   - Contents of device memory are trusted: a block-table entry outside
 *     [0, num_blocks) or a context length above max_blocks_per_seq *
 *     block_size does not fault -- the kernel clamps it -- but the result for
 *     that sequence is then unspecified.
 *   - Debugging: with PA_FLAG_VALIDATE in opts->flags a call first copies the
 *     index and scale arrays it reads (block tables, context lengths, slot
 *     mappings, query_start_loc, block pairs, per-head scales) to the host,
 *     after the stream's earlier work, and checks every entry the contract
 *     above leaves unspecified; the first bad one is returned as
 *     PA_ERR_BAD_INDEX, with its position in pa_last_error(), and nothing is
 *     enqueued.  Such a call waits for the stream (the one exception to "no
 *     call synchronises"), and is refused with PA_ERR_ARG on a stream that is
 *     being captured.  The pages treat these entries as faults reported to the
 *     owner of the mapping: an unmapped page-table entry faults (page
 *     "Paged KVCache：大模型推理显存管理优化方案", section 2.3), and a request
 *     the block pool cannot serve raises an error (page
 *     "vLLM推理引擎架构：PagedAttention机制与高吞吐推理", section 2.2).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_API __attribute__((visibility("default")))

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3, /* OCP e4m3fn: bias 7, max 448, no infinities, NaN = S.1111.111 */
  PA_I32 = 4,
  PA_I64 = 5,
} pa_dtype;

typedef struct pa_tensor {
  void *data;        /* device pointer */
  int32_t dtype;     /* pa_dtype */
  int32_t ndim;      /* number of valid entries in shape/stride, 1..5 */
  int64_t shape[5];
  int64_t stride[5]; /* in elements */
} pa_tensor;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_DTYPE = -2,       /* unsupported dtype or dtype combination */
  PA_ERR_SHAPE = -3,       /* ranks or sizes disagree */
  PA_ERR_LAYOUT = -4,      /* inner dimension not contiguous, or misaligned */
  PA_ERR_UNSUPPORTED = -5, /* head_dim / block_size / group size outside the built set */
  PA_ERR_WORKSPACE = -6,   /* workspace missing, misaligned or smaller than pa_decode_workspace_size() */
  PA_ERR_ARG = -7,         /* a scalar argument out of range (scale, partition size, ...) */
  PA_ERR_HIP = -8,         /* the HIP runtime reported an error while enqueuing */
  PA_ERR_BAD_INDEX = -9,   /* PA_FLAG_VALIDATE: an index or scale array entry the results would not survive */
} pa_status;

/* opts->flags bits */
#define PA_FLAG_VALIDATE 1u /* check the index and scale arrays on the host first (see the conventions above) */

/* Options common to both operations.  A NULL opts means all defaults. */
typedef struct pa_opts {
  float k_scale;          /* fp8 caches: stored value = code * k_scale; ignored otherwise.  0 = 1.0 */
  float v_scale;          /* likewise for the value cache.  0 = 1.0 */
  int32_t partition_size; /* decode: tokens per split-context work unit, a multiple of block_size;
                             0 = library choice (a few dozen tokens) */
  int32_t num_workers;    /* decode: wavefronts that share the work (rounded up to a multiple of 4);
                             0 = library choice for the current device */
  uint32_t flags;         /* 0 or PA_FLAG_VALIDATE; other bits are reserved and must be 0 */
  uint32_t reserved;      /* must be 0 */
  void *workspace;        /* decode: device scratch of >= pa_decode_workspace_size() bytes */
  size_t workspace_bytes;
  void *stream;           /* hipStream_t the work is enqueued on; NULL = null stream */
  /* fp8 caches, finer scales: NULL, or fp32 arrays with one scale per kv head
   * (pa_decode_layers: [layers, num_kv_heads], layer-major; pa_decode,
   * pa_prefill, pa_cache_write: [num_kv_heads]), in device memory
   * or pinned host memory.  The stored value of kv head h is then
   * code * k_head_scales[h] (v_head_scales[h] for the value cache), so that
   * heads of small magnitude keep their precision (the precision per attention
   * head of section 8.2 of page "vLLM框架中的KV cache优化与PagedAttention机制详解";
   * the fp8 KV cache of page "大模型推理KV Cache内存管理与PagedAttention分页显存实战").
   * Both or neither; with them k_scale and v_scale must be 0.  The contents are
   * trusted like the block tables: finite and > 0, else results are unspecified. */
  const float *k_head_scales;
  const float *v_head_scales;
  /* fp8 caches, one scale per (physical block, kv head): NULL, or fp32 arrays
   * [num_blocks, num_kv_heads] (pa_decode_layers: [layers, num_blocks,
   * num_kv_heads]) in device memory or pinned host memory.  The stored value
   * of kv head h in block b is then code * k_block_scales[b * num_kv_heads + h]
   * (v_block_scales for the value cache): a block's tokens share a scale, so
   * it can follow the magnitude of the tokens a block holds (the per-head
   * precision of section 8.2 of page "vLLM框架中的KV cache优化与PagedAttention机制详解",
   * at the grain of the pool's blocks).  pa_decode, pa_decode_layers,
   * pa_prefill and pa_cache_write take them (the cache write quantises each
   * new row with its destination block's scales).
   * Both or neither, and not with per-head scales; with them k_scale and
   * v_scale must be 0.  Trusted like the per-head scales. */
  const float *k_block_scales;
  const float *v_block_scales;
} pa_opts;

/* Number of workers pa_decode launches for this request (0 = the library's
 * choice for the current device).  Always a positive multiple of 4. */
PA_API int32_t pa_decode_num_workers(int32_t requested);

/* Bytes of workspace pa_decode needs: two partial-result slots per worker,
 * each holding for every query head of a group a running max, a running sum
 * and an unnormalised head_dim-long output (fp32), from the workspace's
 * start; one int32 merge counter per (sequence, kv head) at its end (in the
 * last bytes of workspace_bytes rounded down to 256).  num_workers as in
 * pa_opts (0 = default).
 * The workspace belongs to the caller: it must be zero-filled once before its
 * first use.  Every pa_decode call leaves its counters at zero again and
 * garbage only in its slots, whose extent depends on the group size
 * (num_heads / num_kv_heads), head_dim and num_workers alone; so calls that
 * agree on those three may share one workspace whatever their number of
 * sequences (or layers), each sized for its own request.  A call with another
 * group size, head_dim or worker count may lay its counters over earlier
 * slots: zero-fill the workspace again before it.  One workspace serves one
 * pa_decode at a time (calls that overlap on different streams need separate
 * workspaces). */
PA_API size_t pa_decode_workspace_size(int64_t num_seqs, int64_t num_heads, int64_t num_kv_heads,
                                       int64_t head_dim, int32_t num_workers);

/*
 * pa_decode -- paged attention decode.
 *
 *   out          [num_seqs, num_heads, head_dim], dtype = q's dtype or PA_F32.
 *                out[s, h, :] = softmax_t(scale * q[s,h,:] . K_t) . V_t over the
 *                first context_lens[s] tokens t of sequence s, where token t
 *                lives at k_cache[block_tables[s, t / block_size], t % block_size,
 *                h / (num_heads / num_kv_heads), :] (and likewise in v_cache).
 *                A sequence with context length 0 gets zeros.
 *   q            [num_seqs, num_heads, head_dim]: PA_F32, PA_F16 or PA_BF16.
 *   k_cache,
 *   v_cache      [num_blocks, block_size, num_kv_heads, head_dim], same shape and
 *                dtype: PA_F32 / PA_F16 / PA_BF16 equal to q's dtype, or PA_FP8_E4M3
 *                with an F16 or BF16 q (values are code * opts->k_scale / v_scale,
 *                or code * the kv head's entry of opts->k_head_scales / v_head_scales).
 *   block_tables [num_seqs, max_blocks_per_seq] PA_I32; only the first
 *                ceil(context_lens[s] / block_size) entries of row s are read.
 *   context_lens [num_seqs] PA_I32.
 *   block_size   tokens per block: 16 or 32; must equal k_cache.shape[1].
 *   scale        softmax scale (finite, > 0).
 *   num_kv_heads must equal k_cache.shape[2] and divide num_heads.
 *   head_dim     (q.shape[2]) 64 or 128.
 *   opts         workspace (required), stream, fp8 scales, work split.
 * Work: one launch of num_workers persistent wavefronts.  The contexts of all
 * (sequence, kv head) pairs are cut into work units of partition_size tokens
 * and every worker takes an equal contiguous share of the units; a context
 * that two or more workers share is merged by log-sum-exp in the same launch
 * by whichever of them finishes last.
 */
PA_API pa_status pa_decode(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache, pa_tensor block_tables,
                           pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                           const pa_opts *opts);

/*
 * pa_decode_append -- one decode step in one launch: the cache write of every
 * sequence's new token (pa_cache_write) followed by pa_decode, fused so that
 * the step pays one launch (the batched translation of section 5.2 of page
 * "vLLM框架中的KV cache优化与PagedAttention机制详解", which cuts kernel launches;
 * the new token's slot from the allocator of section 2.2 of page
 * "vLLM推理引擎架构：PagedAttention机制与高吞吐推理").
 *   out, q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
 *   num_kv_heads, opts   as pa_decode (one layer).
 *   k_new, v_new   [num_seqs, num_kv_heads, head_dim], the caches' dtype
 *                  (PA_F32, PA_F16 or PA_BF16; fp8 caches are refused with
 *                  PA_ERR_UNSUPPORTED -- use pa_cache_write then pa_decode).
 *   slot_mapping   [num_seqs] PA_I32 or PA_I64: the slot of sequence s's new
 *                  token, which is the token at position context_lens[s] - 1,
 *                  i.e. block_tables[s][(L-1) / block_size] * block_size +
 *                  (L-1) % block_size for L = context_lens[s].
 * Effect: rows k_new[s], v_new[s] are copied to their slot and out is
 * pa_decode's result over the updated cache: the decode reads the new token's
 * K/V from k_new/v_new directly instead of from the slot being written.  For
 * groups of four or more query heads per kv head on 16-bit caches the result
 * is pa_decode's bit for bit (the new token takes its place in its chunk).
 * For groups of one or two and for fp32 caches the new token enters its
 * softmax first instead of last, so the sums run in another order and the
 * result equals pa_decode's up to fp32 rounding.  A slot < 0 or past the
 * pool is skipped, as in pa_cache_write (for
 * instance a last token that lies in a block already stored and shared with
 * other sequences): nothing is written and the decode reads position L - 1
 * from the cache as it stands.  If a slot is not the one of position L - 1, or
 * two sequences share a slot, the result is unspecified.  A sequence with
 * context length 0 has no new token: nothing is written for it and its output
 * is zeros.
 */
PA_API pa_status pa_decode_append(pa_tensor out, pa_tensor q, pa_tensor k_new, pa_tensor v_new, pa_tensor k_cache,
                                  pa_tensor v_cache, pa_tensor slot_mapping, pa_tensor block_tables,
                                  pa_tensor context_lens, int32_t block_size, float scale, int32_t num_kv_heads,
                                  const pa_opts *opts);

/*
 * pa_decode_static -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *   Arguments as pa_decode; opts->workspace must be NULL and
 *   opts->workspace_bytes 0 (else PA_ERR_ARG).  The workspace is instead a
 *   device array owned by the library, pa_decode_static_scratch_bytes()
 *   (24 MiB) on each device it runs on, held until the process ends.  A
 *   request whose pa_decode_workspace_size() exceeds it returns
 *   PA_ERR_WORKSPACE before anything is enqueued (at the default worker count
 *   that allows, for instance, 65535 sequences x 32 kv heads with 8 query
 *   heads of 128 dims per kv head).
 *   The first call on a device looks the array up and enqueues one kernel on
 *   opts->stream that clears it; every decode leaves its counters at zero
 *   again, so calls of any batch size follow without a clear.  A call whose
 *   counters would overlap partial-result slots used since the last clear
 *   (another group size, head_dim or worker count; see
 *   pa_decode_workspace_size) enqueues the clear again first.  No call
 *   allocates or frees memory.  Every call on one device
 *   shares that device's array: calls that overlap on one device (other
 *   streams, other host threads) race and must be serialised by the caller.
 *   The results are pa_decode's, bit for bit.
 */
PA_API size_t pa_decode_static_scratch_bytes(void);
PA_API pa_status pa_decode_static(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache,
                                  pa_tensor block_tables, pa_tensor context_lens, int32_t block_size, float scale,
                                  int32_t num_kv_heads, const pa_opts *opts);

/*
 * pa_decode_layers -- pa_decode for several layers of the same batch in one
 * launch (the translation of many lookups batched into one call, section 5.2
 * of page "vLLM框架中的KV cache优化与PagedAttention机制详解").
 *
 *   out, q          [layers, num_seqs, num_heads, head_dim]
 *   k_caches,
 *   v_caches        [layers, num_blocks, block_size, num_kv_heads, head_dim]:
 *                   one pool per layer, block b of every layer holding the same
 *                   tokens, so that the block tables and context lengths --
 *                   [num_seqs, max_blocks_per_seq] and [num_seqs], shared by all
 *                   layers -- address every layer.
 *   everything else as pa_decode; each layer's result is exactly pa_decode's
 *   on that layer's q, caches and out.  The layer stride of each tensor must be
 *   a multiple of 16 bytes.
 *   opts->workspace: pa_decode_workspace_size(layers * num_seqs, ...) bytes.
 *   opts->k_head_scales / v_head_scales (fp8 caches): [layers, num_kv_heads].
 * Work: one launch; the (layer, sequence) pairs are the items of pa_decode's
 * split, so the launch's fixed cost and its finishing spread are paid once for
 * all layers.
 */
PA_API pa_status pa_decode_layers(pa_tensor out, pa_tensor q, pa_tensor k_caches, pa_tensor v_caches,
                                  pa_tensor block_tables, pa_tensor context_lens, int32_t block_size, float scale,
                                  int32_t num_kv_heads, const pa_opts *opts);

/*
 * pa_prefill -- paged attention for several causal query tokens per sequence.
 *
 *   q               [num_tokens, num_heads, head_dim] PA_F16 or PA_BF16: the
 *                   query rows of every sequence of the step, sequence after
 *                   sequence.
 *   query_start_loc [num_seqs + 1] PA_I32, non-decreasing, from 0 to
 *                   num_tokens: rows query_start_loc[s] .. query_start_loc[s+1]-1
 *                   belong to sequence s.
 *   context_lens    [num_seqs] PA_I32: tokens of sequence s in the cache,
 *                   the step's own tokens included (their K/V rows written
 *                   first, e.g. by pa_cache_write).
 *   out             [num_tokens, num_heads, head_dim], q's dtype or PA_F32.
 *                   With n = the rows of sequence s and L = context_lens[s],
 *                   row j (0 <= j < n) is the token at position p = L - n + j:
 *                   out[row, h, :] = softmax_t(scale * q[row,h,:] . K_t) . V_t
 *                   over positions t = 0 .. p, K_t / V_t found through the
 *                   block table as in pa_decode.  n = 1 is pa_decode's result;
 *                   n = L is causal attention over a whole prompt.  Requires
 *                   n <= L; a row whose position would be negative gets zeros.
 *   k_cache,
 *   v_cache         [num_blocks, block_size, num_kv_heads, head_dim]: q's dtype,
 *                   or PA_FP8_E4M3 (values code * opts->k_scale / v_scale, or
 *                   code * the kv head's entry of opts->k_head_scales /
 *                   v_head_scales, as in pa_decode).
 *   block_tables    [num_seqs, max_blocks_per_seq] PA_I32, as in pa_decode.
 *   block_size      16 or 32; num_kv_heads divides num_heads; head_dim 64 or 128.
 *   opts            stream, fp8 scales, optional workspace (partition_size and
 *                   num_workers are ignored; flags as in pa_opts).
 *   opts->workspace NULL, or device memory of pa_prefill_workspace_size()
 *                   bytes, 256-byte aligned, zero-filled before its first use
 *                   and left at zero by every call.  With it, steps of few
 *                   query rows per sequence hand their (tile, kv head) pairs to
 *                   workgroups as they free up, longest context first; without
 *                   it the pairs are dealt round-robin.  The results are the
 *                   same either way, bit for bit.  One workspace serves one
 *                   call at a time.
 * The contents of query_start_loc are trusted like the block tables: values
 * outside [0, num_tokens] are clamped, never followed out of bounds.
 * Work: one launch.  Steps averaging more than 32 (query row, query head)
 * pairs per sequence: a workgroup per (sequence, kv head, tile of 64 or 128
 * such pairs), streaming the positions its last row sees.  Smaller steps
 * (speculative verification): one persistent workgroup per compute unit; the
 * four wavefronts of a workgroup split one tile's keys.
 */
PA_API pa_status pa_prefill(pa_tensor out, pa_tensor q, pa_tensor k_cache, pa_tensor v_cache,
                            pa_tensor block_tables, pa_tensor context_lens, pa_tensor query_start_loc,
                            int32_t block_size, float scale, int32_t num_kv_heads, const pa_opts *opts);

/* Bytes of the optional pa_prefill workspace (one pair counter, padded). */
PA_API size_t pa_prefill_workspace_size(void);

/*
 * pa_cache_write -- scatter new tokens into the paged cache.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim]; dtype equal to the
 *                 cache's, or PA_F32 / PA_F16 / PA_BF16 for an fp8 cache.
 *   k_cache,
 *   v_cache       [num_blocks, block_size, num_kv_heads, head_dim], same shape/dtype.
 *   slot_mapping  [num_tokens] PA_I64 or PA_I32.  Token n goes to block
 *                 slot / block_size, offset slot % block_size.  Slots < 0 and
 *                 slots >= num_blocks * block_size are skipped.  Slots must be
 *                 distinct (duplicates race); writing into a block that several
 *                 sequences share is the caller's responsibility.
 * Same-dtype writes copy the bytes.  fp8 writes store
 * round-to-nearest-even(x / scale) saturated to +-448 (NaN stays NaN), the
 * division done in fp32, with scale = opts->k_scale / v_scale, or the scale of
 * the row's kv head when opts->k_head_scales / v_head_scales are given
 * ([num_kv_heads] each; ignored, like the per-tensor scales, when k is itself
 * FP8_E4M3 and its codes are copied).
 */
PA_API pa_status pa_cache_write(pa_tensor k, pa_tensor v, pa_tensor k_cache, pa_tensor v_cache,
                                pa_tensor slot_mapping, const pa_opts *opts);

/*
 * pa_copy_blocks -- copy whole blocks from one pool to another (or within one).
 *
 *   dst_k_cache, dst_v_cache  [dst_blocks, block_size, num_kv_heads, head_dim]
 *   src_k_cache, src_v_cache  [src_blocks, block_size, num_kv_heads, head_dim]
 *                             any one dtype for all four; the same block shape;
 *                             each block one contiguous run of bytes (the cache
 *                             layout of pa_decode); K and V pools of a side have
 *                             the same number of blocks and block stride.  Each
 *                             pool is device memory or pinned host memory
 *                             (hipHostMalloc, torch pin_memory): a swap-out
 *                             copies device -> host, a swap-in host -> device,
 *                             copy-on-write device -> device in one pool (pass
 *                             the same tensors as source and destination).
 *   block_mapping             [num_pairs, 2] PA_I64 or PA_I32, device or pinned
 *                             host memory: pair (s, d) makes K and V block d of
 *                             the destination a byte copy of block s of the
 *                             source.  Pairs with an id < 0 or past its pool are
 *                             skipped.  Destinations must be distinct and, within
 *                             one pool, no destination may also be a source;
 *                             otherwise the result is unspecified (never a fault).
 *   opts                      stream and flags only.
 * Errors: PA_ERR_ARG if a pointer is neither device memory nor pinned host
 * memory (pageable host memory is refused before anything is enqueued).
 * Work: one launch, a workgroup per (pair, K or V, 16 KB of the block).
 */
PA_API pa_status pa_copy_blocks(pa_tensor dst_k_cache, pa_tensor dst_v_cache, pa_tensor src_k_cache,
                                pa_tensor src_v_cache, pa_tensor block_mapping, const pa_opts *opts);

/*
 * pa_stream_read -- a plain streaming read of one buffer, for measurement.
 *
 * Not a step of the attention path.  A decode step gathers each sequence's
 * K/V range through its block table (page "vLLM框架中的KV cache优化与
 * PagedAttention机制详解", section 5.1) and reads each of those bytes once, so
 * its practical ceiling is the rate at which the part can stream-read memory
 * far larger than its caches; this call measures that rate with the same
 * 16-byte loads.
 *
 *   buf              device memory (or pinned host memory), 16-byte aligned,
 *                    `bytes` long; read once, never written.
 *   bytes            > 0, a multiple of 16.
 *   num_workgroups   1 .. 65536 workgroups of 256 threads, reading the buffer
 *                    grid-stride in 16-byte vectors.
 *   loads_in_flight  1, 4 or 8 vectors each thread loads before it uses any.
 *   nontemporal      non-zero: non-temporal loads (the kind the decode
 *                    kernels use for K/V rows); zero: ordinary loads.
 *   partials         [num_workgroups] uint32, device memory, caller-owned:
 *                    partials[w] becomes the XOR of the 32-bit words workgroup
 *                    w read, so the XOR of all partials is the XOR of every
 *                    32-bit word of the buffer, whatever the launch shape.
 *   opts             stream only (NULL = null stream, flags 0).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_LAYOUT, PA_ERR_ARG,
 * PA_ERR_UNSUPPORTED as named above, before anything is enqueued.
 * Work: one launch.
 */
PA_API pa_status pa_stream_read(const void *buf, int64_t bytes, int32_t num_workgroups, int32_t loads_in_flight,
                                int32_t nontemporal, uint32_t *partials, const pa_opts *opts);

/* Static description of a status code. */
PA_API const char *pa_status_string(pa_status s);

/* Thread-local detail for the last non-OK status returned on this thread. */
PA_API const char *pa_last_error(void);

/* Library version, "major.minor.patch". */
PA_API const char *pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
