/*
 * pkv.h -- C ABI of libpkv: paged KV-cache input preparation, KV-cache write
 * and paged variable-length causal attention for AMD Instinct MI355X (gfx950).
 *
 * One step of paged LLM serving runs these calls on one HIP stream (the
 * index derivation first, the KV write before the attention that reads it):
 *
 *   pkv_prepare_inputs         flat-batch index tensors from the scheduler's
 *                              per-request token counts and block tables;
 *   pkv_prepare_input_ids      the step's input token ids gathered from the
 *                              per-request token table, and the mask of
 *                              requests whose sampled token is discarded;
 *   pkv_kv_cache_write         each new token's K and V rows into the block
 *                              pool at its slot;
 *   pkv_kv_cache_write_fp8     the same into an FP8 E4M3 pool with a scale
 *                              per pool;
 *   pkv_paged_attention_varlen causal attention of every query row of the
 *                              step (prefill chunks and single-token decodes
 *                              alike, in one launch) over its request's
 *                              context, read through the block table;
 *   pkv_paged_attention_varlen_fp8  the same over FP8 pools;
 *   pkv_paged_attention_plan / pkv_paged_attention_run  the attention call in
 *                              two halves: the work list once per batch,
 *                              then any number of calls over it (one per
 *                              model layer);
 *   pkv_prepare_inputs_and_plan  pkv_prepare_inputs and
 *                              pkv_paged_attention_plan of one step in a
 *                              single launch;
 *   pkv_copy_blocks            whole-block copies in both pools (copy-on-write
 *                              of a shared block);
 *   pkv_zero_blocks            whole-block clears in both pools (freshly
 *                              allocated blocks).
 *
 * Two more calls describe the build: pkv_debug_checks_enabled and
 * pkv_debug_check_flags (the checked build, libpkv_checked.so, validates
 * every call's device data first; see PKV_ERR_DEVICE_DATA below).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers must be device memory (or memory the
 *   device can address) owned by the caller.  The library allocates nothing,
 *   keeps no device state between calls, never synchronises, never reads
 *   device memory from the host, and only enqueues work on `stream`
 *   (a hipStream_t; NULL means the default stream).  Calls are reentrant:
 *   host threads may call any entry point concurrently.
 *   (The checked build is the exception: it reads a check word back and
 *   synchronises `stream` once per call, and its calls share one device
 *   check word, so checked calls must not run concurrently.)
 * - Host-side validation covers the scalar arguments and null pointers only;
 *   it returns a status and enqueues nothing on failure.  Device-side
 *   contents are preconditions (listed per call).  Where a precondition on
 *   device data is broken the kernels still never touch memory outside the
 *   buffers described here; the affected outputs are then unspecified.
 * - Integer index tensors are int32 except slot_mapping (int64, -1 = no
 *   write).  Block pools are two separate tensors:
 *     K pool: [num_blocks][num_kv_heads][head_dim * block_size], each
 *             (block, head) run in slabs of 32 dims: element (dim, t) at
 *             ((dim / 32) * block_size + t) * 32 + dim % 32 (when 32 does
 *             not divide head_dim the slab spans all dims: then the run is
 *             plain [block_size][head_dim])
 *     V pool: [num_blocks][num_kv_heads][head_dim * block_size], each
 *             (block, head) run in tiles of 16 dims x 4 tokens:
 *             element (dim, t) at ((dim / 16) * (block_size / 4) + t / 4) * 64
 *             + (dim % 16) * 4 + t % 4 (when 16 does not divide head_dim the
 *             tile spans all dims, when 4 does not divide block_size all
 *             tokens: then the run is plain [head_dim][block_size])
 *   The pages leave the cache layout to the kernel ("Inside vLLM: Following
 *   One Request from the API to GPU Execution", Part 5, which notes that
 *   different write/read kernel pairs use different layouts).  A K slab of
 *   a 16-token block is 1 KB (16-bit elements) holding, for each token, 32
 *   contiguous dims: one wave-wide 16-byte load reads a whole slab, the
 *   operand of one 32-deep step of the Q.K contraction, as 8 full cache
 *   lines (token-major rows would take 16 half lines), and a token's row of
 *   128 16-bit values spans 4 runs of 64 bytes.  In a V tile the 4 tokens
 *   of one dimension are one contiguous run, the operand unit of the P.V
 *   contraction over tokens, and a single token's row of 128 16-bit values
 *   spans 8 cache lines of 128 bytes per head (a dim-major run would spread
 *   it over 32, each partly written).
 * - Ordering: the KV write of a step must be enqueued before the attention
 *   that reads it, on the same stream or behind an event.  The pages make the
 *   same requirement explicit with a dummy data dependency ("Inside vLLM...",
 *   Part 4).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes  */
  PKV_ERR_UNSUPPORTED = 2, /* a valid argument the library has no kernel for  */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  PKV_ERR_LAUNCH = 4,      /* the HIP runtime rejected a kernel launch         */
  PKV_ERR_DEVICE_DATA = 5, /* checked build only: device data broke a
                              precondition (see pkv_debug_check_flags)        */
  PKV_ERR_SCRATCH_LIMIT = 6 /* pkv_paged_attention_varlen_noalloc: the sizes
                              need more than PKV_NOALLOC_SCRATCH_BYTES        */
} pkv_status;

/*
 * The checked build (libpkv_checked.so, compiled with PKV_DEBUG_CHECKS)
 * exports the same entry points.  Each first runs a validation kernel on the
 * device data it is given, on `stream`, waits for it (the checked build does
 * synchronise), and returns PKV_ERR_DEVICE_DATA without launching anything
 * else when a precondition is broken; pkv_debug_check_flags() then returns
 * the failed checks as these bits.  The regular build never checks device
 * data and never returns PKV_ERR_DEVICE_DATA.
 */
#define PKV_CHECK_COUNTS 0x001u    /* negative token counts, or their sum != num_tokens */
#define PKV_CHECK_BLOCK_ID 0x002u  /* a table entry the call reads is outside
                                      [0, num_blocks), or its column is past the row   */
#define PKV_CHECK_SLOT 0x004u      /* a slot outside [-1, num_blocks * block_size)     */
#define PKV_CHECK_SLOT_DUP 0x008u  /* two rows of one write share a slot (checked up
                                      to 65536 rows)                                   */
#define PKV_CHECK_QSL 0x010u       /* query_start_loc negative, decreasing, or past
                                      num_tokens                                       */
#define PKV_CHECK_LENGTHS 0x020u   /* q_len > seq_len, seq_len > max_seq_len or
                                      q_len > max_query_len                            */
#define PKV_CHECK_ROW 0x040u       /* input ids: a row's request or position outside
                                      the token table (other than a -1, -1 padding row) */
#define PKV_CHECK_PAIRS 0x080u     /* block copies: a destination repeated or also a
                                      source (checked up to 65536 pairs)               */
#define PKV_CHECK_SCALE 0x100u     /* an FP8 scale not finite and positive             */
#define PKV_CHECK_PLAN 0x200u      /* pkv_paged_attention_run: the workspace holds no
                                      work list for these sizes and this batch          */

typedef enum pkv_dtype {
  PKV_F32 = 0,  /* IEEE binary32                                   */
  PKV_BF16 = 1  /* bfloat16 (top 16 bits of binary32); fp32 accumulate */
} pkv_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* pkv_status_string(pkv_status status);

/* 1 in the checked build, 0 in the regular one. */
int32_t pkv_debug_checks_enabled(void);

/* Checked build: the PKV_CHECK_* bits of the last call that returned
 * PKV_ERR_DEVICE_DATA in this process (0 before any; not per thread).
 * Regular build: always 0. */
uint32_t pkv_debug_check_flags(void);

/*
 * pkv_prepare_inputs -- flat-batch index tensors for one step.
 *
 * Follows "Building the Batch", sections "How they are computed" and
 * "Reading and writing the KV cache", and "vLLM's Model Runner -- the
 * Persistent Batch, in Source", "The two things this method returns".  With
 * nst = num_scheduled_tokens, nct = num_computed_tokens, for request r:
 *   query_start_loc[0] = 0, query_start_loc[r+1] = query_start_loc[r] + nst[r]
 *   seq_lens[r]        = nct[r] + nst[r]
 *   logits_indices[r]  = query_start_loc[r+1] - 1
 * and for the t-th scheduled token of r, at flat row i = query_start_loc[r] + t:
 *   req_indices[i]  = r
 *   positions[i]    = nct[r] + t
 *   slot_mapping[i] = block_table[r][positions[i] / block_size] * block_size
 *                     + positions[i] % block_size
 * query_start_loc[num_reqs+1 .. qsl_len-1] = the token total, so the array is
 * non-decreasing and padding "requests" have an empty row range.
 *
 * Arguments (device pointers unless stated):
 *   num_scheduled_tokens, num_computed_tokens  int32 [num_reqs], >= 0
 *   block_table     int32 [num_reqs][bt_row_stride]; a request reads only
 *                   columns < bt_row_stride
 *   num_reqs        host, >= 0;  num_tokens host, = sum(num_scheduled_tokens)
 *   qsl_len         host, >= num_reqs + 1
 *   block_size      host, >= 1
 *   num_blocks      host, size of the block pool; slots are checked against it
 *   req_indices, positions  int32 [num_tokens]  (out)
 *   slot_mapping    int64 [num_tokens]          (out)
 *   query_start_loc int32 [qsl_len]             (out)
 *   seq_lens, logits_indices int32 [num_reqs]   (out)
 * Device-data behaviour: a token whose block-table column is >= bt_row_stride
 * or whose block id is outside [0, num_blocks) gets slot -1 (no write).  If
 * sum(num_scheduled_tokens) differs from num_tokens, rows past the device sum
 * get req_indices = positions = -1 and slot -1.
 * Errors: PKV_ERR_INVALID_ARG for null pointers (outputs of size 0 may be
 * NULL), negative sizes, qsl_len < num_reqs + 1, block_size < 1,
 * bt_row_stride < 1 when num_tokens > 0; PKV_ERR_LAUNCH.
 */
pkv_status pkv_prepare_inputs(const int32_t* num_scheduled_tokens,
                              const int32_t* num_computed_tokens, const int32_t* block_table,
                              int64_t bt_row_stride, int32_t num_reqs, int32_t num_tokens,
                              int32_t qsl_len, int32_t block_size, int64_t num_blocks,
                              int32_t* req_indices, int32_t* positions, int64_t* slot_mapping,
                              int32_t* query_start_loc, int32_t* seq_lens,
                              int32_t* logits_indices, void* stream);

/*
 * pkv_prepare_input_ids -- the step's input token ids and discard mask.
 *
 * Follows "Building the Batch", "How they are computed" (request r's tokens
 * are row r of a table of row_width columns, so its token at position p is
 * element r * row_width + p of the table read flat) and "vLLM's Model Runner
 * -- the Persistent Batch, in Source", "The batch contains rows that must not
 * be sampled" (a request still short of its known token count after this
 * pass is mid-prefill; its sampled token is dropped).  For every flat row i
 * with r = req_indices[i], p = positions[i]:
 *   token_indices[i] = r * row_width + p
 *   input_ids[i]     = token_table[token_indices[i]]
 * and for every request r:
 *   discard_request_mask[r] = seq_lens[r] < num_tokens_total[r] ? 1 : 0
 * req_indices, positions and seq_lens are the outputs of pkv_prepare_inputs
 * for the same step (enqueue that call first).
 *
 * Arguments (device pointers unless stated):
 *   token_table     int32 [num_reqs or more][row_width], row r = request r
 *   row_width       host, >= 1, the longest sequence a request may reach
 *   num_reqs        host, >= 0;  num_tokens host, >= 0
 *   req_indices, positions  int32 [num_tokens]
 *   seq_lens, num_tokens_total  int32 [num_reqs]
 *   token_indices   int64 [num_tokens] (out), or NULL when not wanted
 *   input_ids       int32 [num_tokens] (out)
 *   discard_request_mask  uint8 [num_reqs] (out), 0 or 1
 * Device-data behaviour: a row with r outside [0, num_reqs) or p outside
 * [0, row_width) (padding rows from pkv_prepare_inputs have -1 in both) gets
 * token_indices = -1 and input_ids = -1; nothing outside the table is read.
 * Errors: PKV_ERR_INVALID_ARG for negative sizes, row_width < 1, null
 * pointers to non-empty arrays; PKV_ERR_LAUNCH.
 */
pkv_status pkv_prepare_input_ids(const int32_t* token_table, int64_t row_width,
                                 int32_t num_reqs, const int32_t* req_indices,
                                 const int32_t* positions, int32_t num_tokens,
                                 const int32_t* seq_lens, const int32_t* num_tokens_total,
                                 int64_t* token_indices, int32_t* input_ids,
                                 uint8_t* discard_request_mask, void* stream);

/*
 * pkv_kv_cache_write -- scatter this step's K and V rows into the block pool.
 *
 * Follows "Inside vLLM: Following One Request from the API to GPU Execution",
 * Part 5: for token i the K and V vectors go to the cache slot
 * slot_mapping[i] = physical_block * block_size + in_block_offset; the write
 * is token-granular while reads are block-granular.  For every i with
 * s = slot_mapping[i] in [0, num_blocks * block_size) and every kv head h:
 *   K pool element (dim, s % block_size) of run (s / block_size, h)
 *     = key[i][h][dim] for every dim (slab order above)
 *   V pool element (dim, s % block_size) of run (s / block_size, h)
 *     = value[i][h][dim] for every dim (tiled order above)
 * Bytes are copied unchanged.  Slots < 0 (padding rows) and slots past the
 * pool are skipped.
 *
 * Arguments (device pointers unless stated):
 *   key, value      [num_tokens][num_kv_heads][head_dim] of `dtype`; row i
 *                   starts at element i * key_row_stride (value_row_stride);
 *                   heads and dims are contiguous within a row; row starts
 *                   must be 16-byte aligned
 *   key_cache, value_cache  the K and V pools (layouts above), 16-byte aligned
 *   num_blocks      host, blocks in each pool
 *   slot_mapping    int64 [num_tokens]
 *   num_tokens, num_kv_heads, head_dim, block_size   host
 *   dtype           PKV_F32 or PKV_BF16
 * Preconditions: slots are unique within a call (two tokens with the same slot
 * leave either row there).
 * Errors: PKV_ERR_INVALID_ARG (null pointers with num_tokens > 0, sizes < 1,
 * row strides < num_kv_heads * head_dim); PKV_ERR_UNSUPPORTED when
 * head_dim * element size is not a multiple of 16 bytes or head_dim > 256;
 * PKV_ERR_LAUNCH.
 */
pkv_status pkv_kv_cache_write(const void* key, const void* value, int64_t key_row_stride,
                              int64_t value_row_stride, void* key_cache, void* value_cache,
                              int64_t num_blocks, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, pkv_dtype dtype, void* stream);

/*
 * pkv_kv_cache_write_fp8 -- pkv_kv_cache_write into an FP8 cache.
 *
 * Follows "Inside vLLM: Following One Request from the API to GPU
 * Execution", Part 5 (the write call takes kv_cache_dtype, k_scale and
 * v_scale next to the pools) and "How vLLM Works Internally: A Deep Dive",
 * "FP8 KV Cache" (the cache is stored in FP8 instead of 16-bit floats).
 * Reading of the pages: the FP8 format is OCP E4M3 (no infinities, largest
 * finite 448) and each pool has one scale.  For every i with
 * s = slot_mapping[i] in [0, num_blocks * 16), every kv head h and dim c:
 *   K byte (s / 16, h, s % 16, c) = e4m3(key[i][h][c] / *k_scale)
 *   V byte (s / 16, h, s % 16, c) = e4m3(value[i][h][c] / *v_scale)
 * where the division is binary32 and e4m3() rounds to the nearest code, ties
 * to even, saturating finite magnitudes beyond 448 (NaN stays NaN).  A code
 * reads back as its E4M3 value times the scale.
 *
 * FP8 pool layouts (bytes; block_size 16, head_dim a multiple of 64):
 *   K pool: [num_blocks][num_kv_heads][head_dim * 16], each (block, head) run
 *           ordered [dim / 64][token][dim % 64]: slabs of 64 dims, 1 KB each,
 *           one 16-byte load of the attention kernels per slab and lane
 *   V pool: [num_blocks][num_kv_heads][head_dim * 16], each (block, head) run
 *           ordered [dim / 64][token / 4][dim % 16][(dim / 16) % 4][token % 4],
 *           so 16 consecutive bytes hold 4 tokens of 4 dims 16 apart -- one
 *           16-byte load of the attention kernels.
 *
 * Arguments (device pointers unless stated):
 *   key, value      [num_tokens][num_kv_heads][head_dim] of `dtype` (PKV_BF16 or
 *                   PKV_F32); row i starts at element i * key_row_stride
 *                   (value_row_stride); heads and dims contiguous in a row
 *   key_cache, value_cache  the FP8 pools above, 16-byte aligned
 *   num_blocks      host, blocks in each pool
 *   slot_mapping    int64 [num_tokens]; < 0 (padding) or past the pool: skipped
 *   num_tokens, num_kv_heads, head_dim, block_size   host
 *   k_scale, v_scale  float32 scalars, positive and finite (preconditions)
 * Preconditions: slots unique within a call.
 * Errors: PKV_ERR_INVALID_ARG (null pointers with num_tokens > 0, sizes < 1,
 * row strides < num_kv_heads * head_dim, misaligned pointers);
 * PKV_ERR_UNSUPPORTED (block_size != 16, head_dim not a multiple of 64 or
 * > 256); PKV_ERR_LAUNCH.
 */
pkv_status pkv_kv_cache_write_fp8(const void* key, const void* value, int64_t key_row_stride,
                                  int64_t value_row_stride, void* key_cache, void* value_cache,
                                  int64_t num_blocks, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, pkv_dtype dtype, const float* k_scale,
                                  const float* v_scale, void* stream);

/*
 * pkv_paged_attention_workspace_bytes -- device workspace that
 * pkv_paged_attention_varlen needs for these host-side sizes (the work list
 * and, for long decode contexts split into partitions, the per-partition
 * partial results).  The arguments mean what they mean there; split_tokens = 0
 * selects the library's own partition size, which depends on the current
 * device's CU count (call this with the device of the attention call
 * current).  Returns 0 for invalid sizes.
 */
size_t pkv_paged_attention_workspace_bytes(int32_t num_reqs, int32_t num_tokens,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_query_len,
                                           int32_t max_seq_len, int32_t split_tokens,
                                           pkv_dtype dtype);

/*
 * pkv_paged_attention_varlen -- causal attention over a flat, variable-length
 * batch whose K/V history lives in a block-paged pool.
 *
 * Follows "How vLLM Works Internally: A Deep Dive", "How the Kernel Works"
 * (look up the block table, fetch K from scattered blocks, scores, softmax,
 * weighted sum of V) and "PagedAttention V1/V2" (a second pass that reduces
 * per-partition partial softmax results, used here for long decode
 * contexts); "Inside vLLM...", Part 5 (the read call takes the query, both
 * pools, the output, query_start_loc as the query boundaries, seq_lens as the
 * visible K length and the block table).  For request r with
 * q_len = query_start_loc[r+1] - query_start_loc[r] and L = seq_lens[r], the
 * query at flat row i = query_start_loc[r] + t sits at absolute position
 * p = L - q_len + t and sees keys 0..p.  For q head h and kv head
 * g = h / (num_q_heads / num_kv_heads):
 *   out[i][h][:] = sum_{j<=p} softmax_j(scale * q[i][h] . K_r[j][g]) V_r[j][g][:]
 * where K_r[j] / V_r[j] is token j % block_size of physical block
 * block_table[r][j / block_size].  Rows of the same step that belong to long
 * prompt chunks and to single-token decodes are handled by one launch.
 *
 * Arguments (device pointers unless stated):
 *   q               [num_tokens][num_q_heads][head_dim] of `dtype`, row i at
 *                   element i * q_row_stride, 16-byte aligned rows
 *   key_cache, value_cache  the K and V pools, num_blocks blocks each
 *   out             [num_tokens][num_q_heads][head_dim] of `dtype`, row stride
 *                   out_row_stride elements, 16-byte aligned rows (written)
 *   query_start_loc int32 [num_reqs + 1], non-decreasing, last <= num_tokens;
 *                   rows from query_start_loc[num_reqs] to num_tokens - 1
 *                   are padding rows of a step captured at a fixed size
 *                   ("Building the Batch", "Padding, after all that"): they
 *                   belong to no request and the bf16 path leaves their
 *                   output untouched (the fp32 path writes zeros there)
 *   seq_lens        int32 [num_reqs]
 *   block_table     int32 [num_reqs][bt_row_stride]; request r reads columns
 *                   0 .. ceil(seq_lens[r] / block_size) - 1, all < bt_row_stride
 *   num_reqs, num_tokens    host
 *   max_query_len, max_seq_len  host upper bounds of the device values (they
 *                   size the launch and the workspace)
 *   num_q_heads, num_kv_heads  host; num_q_heads % num_kv_heads == 0
 *   head_dim        host, 64 or 128
 *   block_size      host, 16
 *   scale           host, the softmax scale (1/sqrt(head_dim) for plain models),
 *                   finite and > 0
 *   dtype           PKV_BF16 (MFMA path) or PKV_F32 (fp32 vector path)
 *   split_tokens    host, partition size (tokens) for splitting one long
 *                   decode context over several workgroups; 0 = automatic
 *                   (partitions only when requests x kv heads is below the
 *                   current device's CU count, into about one item per CU:
 *                   size the workspace with the same device current);
 *                   otherwise a positive multiple of 32
 *   workspace, workspace_bytes  device scratch of at least
 *                   pkv_paged_attention_workspace_bytes(...) bytes, 256-byte
 *                   aligned; its contents on entry do not matter
 * Preconditions: 1 <= q_len <= seq_len for every request with q_len > 0;
 * block ids in range for every column a request reads.  A row that sees no key
 * (only when seq_len < q_len) is written as zeros; a block id outside
 * [0, num_blocks) contributes no keys.  bf16 output is the fp32 result
 * rounded to nearest even.
 * Errors: PKV_ERR_INVALID_ARG (null pointers, sizes, num_q_heads not a
 * multiple of num_kv_heads, row strides too small, split_tokens not a
 * multiple of 32, scale not finite and positive); PKV_ERR_UNSUPPORTED
 * (head_dim not 64/128, block_size not 16, more than 16 q heads per kv head,
 * or more than 2^24 - 1 workgroups: one per (request, kv head, context
 * partition), one per prompt tile and, when the batch may hold prompt tiles,
 * one more per CU -- only reachable with tiny forced partitions of very long
 * contexts); PKV_ERR_WORKSPACE; PKV_ERR_LAUNCH.
 */
pkv_status pkv_paged_attention_varlen(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, int32_t split_tokens, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_varlen_fp8 -- pkv_paged_attention_varlen over FP8 E4M3
 * pools written by pkv_kv_cache_write_fp8 ("How vLLM Works Internally: A Deep
 * Dive", "FP8 KV Cache").  Every K element reads as its E4M3 value times
 * *k_scale and every V element as its E4M3 value times *v_scale; the result is
 * then exactly what pkv_paged_attention_varlen defines over those values.
 * q and out are bf16 (the dtype is implied); the pools use the FP8 layouts of
 * pkv_kv_cache_write_fp8; k_scale, v_scale are device float32 scalars,
 * positive and finite (preconditions).  The other arguments, the workspace
 * (same size as for bf16) and the errors are those of
 * pkv_paged_attention_varlen; null scales give PKV_ERR_INVALID_ARG.
 */
pkv_status pkv_paged_attention_varlen_fp8(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, const float* k_scale, const float* v_scale, int32_t split_tokens,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_plan, pkv_paged_attention_run -- pkv_paged_attention_varlen
 * in two halves.  Every layer of a model runs attention over the same batch:
 * the same query_start_loc, seq_lens, block table and sizes, with its own q,
 * pools and output.  The plan half derives the call's work list (the order
 * of prompt tiles and decode partitions) from query_start_loc and seq_lens
 * into `workspace`; the run half executes attention over that list.  One plan
 * per batch, then one run per layer, does the same work as one
 * pkv_paged_attention_varlen per layer without re-deriving the list.
 *
 * pkv_paged_attention_plan: arguments as for pkv_paged_attention_varlen
 * (those it takes); q, pools, table and scale are not needed.  The fp32 path
 * has no work list: the call then only validates its arguments.
 * pkv_paged_attention_run: arguments as for pkv_paged_attention_varlen, plus
 * k_scale and v_scale: both null for 16-bit pools, or both device float32
 * scalars for FP8 pools (dtype PKV_BF16; see pkv_paged_attention_varlen_fp8).
 * Precondition: `workspace` holds the work list of a plan (or of a
 * pkv_paged_attention_varlen* call) made with the same query_start_loc and
 * seq_lens contents and the same num_reqs, num_tokens, max_query_len,
 * max_seq_len, num_q_heads, num_kv_heads, head_dim, dtype and split_tokens,
 * on the same device, enqueued earlier on the same stream (or ordered before
 * it), with no other
 * call using the workspace in between.  Runs over one workspace must not
 * overlap: they share its partition buffers.  The checked build verifies the
 * list's record of the sizes and a checksum of the batch (PKV_CHECK_PLAN);
 * the regular build relies on the precondition, and with a stale list the
 * result is unspecified (the kernels still stay inside their buffers).
 * Errors: as for pkv_paged_attention_varlen; PKV_ERR_INVALID_ARG when only
 * one scale is given, or scales with dtype PKV_F32.
 */
pkv_status pkv_paged_attention_plan(const int32_t* query_start_loc, const int32_t* seq_lens,
                                    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len,
                                    int32_t max_seq_len, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                                    int32_t split_tokens, void* workspace,
                                    size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attention_run(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, const float* k_scale, const float* v_scale,
    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_prepare_inputs_and_plan -- pkv_prepare_inputs followed by
 * pkv_paged_attention_plan over the query_start_loc and seq_lens it writes,
 * in one launch.  In "vLLM's Model Runner -- the Persistent Batch, in
 * Source" ("The Forward Pass", "One method, four jobs") the model runner
 * builds the step's input tensors and then its attention metadata inside
 * one input-preparation block; here the attention metadata is the work
 * list.  Two calls back to back pay a launch boundary that one launch does
 * not.
 * Arguments: those of pkv_prepare_inputs, then those of
 * pkv_paged_attention_plan that are not outputs of the prepare half
 * (max_query_len .. workspace_bytes).  Results: identical to the two calls:
 * the same index tensors, and a work list in `workspace` that any
 * pkv_paged_attention_run precondition accepts (the order of items of equal
 * rank may differ between any two plans, as it may between two plan calls).
 * With dtype PKV_F32, or an empty batch, only the prepare half runs and
 * `workspace` is not touched.  The checked build (libpkv_checked.so) runs
 * the two calls one after the other, each with its device-data checks.
 * Errors: those of either call, checked on the host before anything is
 * enqueued.
 */
pkv_status pkv_prepare_inputs_and_plan(
    const int32_t* num_scheduled_tokens, const int32_t* num_computed_tokens,
    const int32_t* block_table, int64_t bt_row_stride, int32_t num_reqs, int32_t num_tokens,
    int32_t qsl_len, int32_t block_size, int64_t num_blocks, int32_t* req_indices,
    int32_t* positions, int64_t* slot_mapping, int32_t* query_start_loc, int32_t* seq_lens,
    int32_t* logits_indices, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype, int32_t split_tokens,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attention_varlen_noalloc -- pkv_paged_attention_varlen for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace.  The work list and the split-KV partials live in a static
 * device array of PKV_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one
 * per GPU, held from the library's first use on that GPU until the process
 * ends; the call allocates nothing and calls no allocating routine.  Inputs
 * and outputs are the caller's, exactly as for pkv_paged_attention_varlen
 * (same arguments minus workspace / workspace_bytes, same kernels and the
 * same results).  All calls on one GPU share that GPU's array and leave their
 * data in it: two calls that overlap in time on one GPU (different streams,
 * or host threads without ordering) race and their results are unspecified;
 * calls ordered on one stream are fine.  The array's contents on entry do not
 * matter (everything a call reads there it wrote first).  The current device
 * must be the device of `stream`.
 * Errors: those of pkv_paged_attention_varlen except PKV_ERR_WORKSPACE, and
 * PKV_ERR_SCRATCH_LIMIT when pkv_paged_attention_workspace_bytes(...) of the
 * same sizes exceeds PKV_NOALLOC_SCRATCH_BYTES, checked on the host before
 * any device access.  That need is 16 bytes per work item plus, when decode
 * contexts are split, 64 * (head_dim + 2) bytes per (request, kv head,
 * partition) slot (the partition count is that of the longest context).
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

pkv_status pkv_paged_attention_varlen_noalloc(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, int32_t split_tokens, void* stream);

/*
 * pkv_copy_blocks -- copy-on-write of whole blocks, both pools at once.
 *
 * Follows "How vLLM Works Internally: A Deep Dive", "Copy-on-Write for Beam
 * Search": before a beam writes into a block that other beams still share,
 * the block's contents move to a newly allocated block that the beam's table
 * then points to.  For every pair k, with (src, dst) = (block_pairs[2k],
 * block_pairs[2k+1]), every byte of block dst in the K pool becomes the byte
 * of block src in the K pool, and likewise in the V pool.  A block is the
 * contiguous run of block_bytes bytes at offset id * block_bytes of a pool,
 * which holds for every pool layout of this library (bf16, float32 and FP8
 * alike): block_bytes = num_kv_heads * block_size * head_dim * element size.
 *
 * Arguments (device pointers unless stated):
 *   key_cache, value_cache  the two pools, num_blocks blocks each, 16-byte
 *                   aligned
 *   num_blocks      host, >= 0;  block_bytes host, >= 16, a multiple of 16
 *   block_pairs     int32 [num_pairs][2]: (source, destination)
 *   num_pairs       host, >= 0
 * Device-data preconditions: the destinations are distinct and none is also
 * a source (a copy-on-write target is a freshly allocated block); sources may
 * repeat (one block forked to several beams).  The copies then do not
 * interact, and the result equals applying the pairs one after another.  A
 * pair with an id outside [0, num_blocks) is skipped.
 * Errors: PKV_ERR_INVALID_ARG for negative sizes, block_bytes < 16, null
 * pointers when num_pairs > 0; PKV_ERR_UNSUPPORTED for block_bytes not a
 * multiple of 16, unaligned pools, or more than 2^24 - 1 workgroups
 * (2 * ceil(block_bytes / 16384) per pair); PKV_ERR_LAUNCH.
 */
pkv_status pkv_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           int64_t block_bytes, const int32_t* block_pairs, int32_t num_pairs,
                           void* stream);

/*
 * pkv_zero_blocks -- clear whole blocks in both pools.
 *
 * Follows "Inside vLLM: Following One Request from the API to GPU
 * Execution", Part 2 (new_block_ids_to_zero): blocks handed to a request for
 * the first time are cleared before the forward pass, so bytes left by an
 * earlier owner (NaNs included) never reach attention.  Every byte of every
 * listed block becomes 0 in both pools (0 is +0.0 in bf16, float32 and E4M3).
 * Arguments and errors as for pkv_copy_blocks, with block_ids int32
 * [num_ids] in place of the pairs; ids may repeat; an id outside
 * [0, num_blocks) is skipped.  Kernel stores only (no memset node), so the
 * call may be captured in a HIP graph.
 */
pkv_status pkv_zero_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           int64_t block_bytes, const int32_t* block_ids, int32_t num_ids,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
