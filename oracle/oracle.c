/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the paged KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no header, helper or constant with the
 * HIP library: every layout rule below is written out here on its own.
 *
 * Three functions, each the plain definition from the pages:
 *
 *   orc_prepare    -- the flat-batch index tensors ("Building the Batch",
 *                     sections "How they are computed" and "Reading and
 *                     writing the KV cache"; "vLLM's Model Runner -- the
 *                     Persistent Batch, in Source", "The two things this
 *                     method returns").
 *   orc_kv_write   -- each new token's K and V row copied to the cache slot
 *                     named by slot_mapping ("Inside vLLM: Following One
 *                     Request from the API to GPU Execution", Part 5, the
 *                     write path through slot_mapping).
 *   orc_attention  -- per request, gather the logical blocks named by the
 *                     block table into contiguous K and V, then naive causal
 *                     softmax attention in fp64 ("How vLLM Works Internally:
 *                     A Deep Dive", "How the Kernel Works", its four steps;
 *                     "Inside vLLM...", Part 5, the block_table read loop).
 *   orc_input_ids  -- token ids gathered from the per-request token table at
 *                     positions + request * row width, and the mask of
 *                     requests whose sampled token is discarded ("Building
 *                     the Batch", "How they are computed"; "vLLM's Model
 *                     Runner...", "The batch contains rows that must not be
 *                     sampled").
 *   orc_copy_blocks, orc_zero_blocks
 *                  -- whole-block copy for copy-on-write ("How vLLM Works
 *                     Internally: A Deep Dive", "Copy-on-Write for Beam
 *                     Search", step 3) and clearing of newly allocated blocks
 *                     ("Inside vLLM...", Part 2: new_block_ids_to_zero).
 *   orc_kv_write_fp8, orc_attention_kv
 *                  -- the same write and read with an FP8 cache: each stored
 *                     element is an FP8 E4M3 code of the value divided by a
 *                     per-tensor scale, read back as code value times scale
 *                     ("How vLLM Works Internally: A Deep Dive", "FP8 KV
 *                     Cache"; "Inside vLLM...", Part 5: the write call takes
 *                     kv_cache_dtype, k_scale and v_scale).
 *
 * Cache layout (an interface fact, not part of the method; the pages leave the
 * layout open): both pools are [num_blocks][num_kv_heads][run], one run of
 * head_dim x block_size elements per (block, head).  A 16-bit or fp32 K run
 * is [dim / 32][token][dim % 32] (slabs of 32 dims, see orc_k_elem); a V run
 * holds tiles of 16 dims x 4 tokens, [dim / 16][token / 4][dim % 16]
 * [token % 4] (see orc_v_elem).
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *   - causal alignment: the query at in-chunk offset t of a request with
 *     q_len new tokens and seq_len total tokens sits at absolute position
 *     p = seq_len - q_len + t (= num_computed_tokens + t) and sees keys
 *     0..p inclusive;
 *   - GQA: q head h reads kv head h / (num_q_heads / num_kv_heads);
 *   - slot -1 in slot_mapping means "no write" (a padding row);
 *   - the query_start_loc entries past num_reqs are filled with the token
 *     total so the array stays non-decreasing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1      /* null pointer or non-positive size            */
#define ORC_ERR_RANGE 2    /* block id, logical block or slot out of range  */
#define ORC_ERR_DUP 3      /* two tokens name the same cache slot           */
#define ORC_ERR_PRECOND 4  /* q_len > seq_len, or a row outside the batch   */
#define ORC_ERR_NOMEM 5

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2  /* cache elements: FP8 E4M3 codes, one scale per pool */

/* ------------------------------------------------------------------------ */
/* prepare                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * For requests r = 0..R-1 in order (nst = num_scheduled_tokens,
 * nct = num_computed_tokens):
 *   qsl[0] = 0, qsl[r+1] = qsl[r] + nst[r]           (prefix sum of the chunk
 *                                                      lengths)
 *   seq_lens[r] = nct[r] + nst[r]                     (length once this step's
 *                                                      tokens are in the cache)
 *   logits_indices[r] = qsl[r+1] - 1                  (last row of the request)
 *   for t in 0..nst[r]-1, row i = qsl[r] + t:
 *     req_indices[i] = r
 *     positions[i]   = nct[r] + t                     (computed tokens + offset
 *                                                      inside the chunk)
 *     slot[i] = block_table[r][positions[i] / bs] * bs + positions[i] % bs
 *   qsl[R+1 .. qsl_len-1] = T                         (non-decreasing tail)
 * Returns ORC_ERR_RANGE when a needed block-table column is >= bt_cols or a
 * block id lies outside [0, num_blocks).  *num_tokens_out receives T.
 */
int orc_prepare(const int32_t* nst, const int32_t* nct, const int32_t* block_table,
                int64_t bt_stride, int32_t bt_cols, int32_t num_reqs, int32_t qsl_len,
                int32_t block_size, int64_t num_blocks, int32_t* req_indices,
                int32_t* positions, int64_t* slot_mapping, int32_t* qsl, int32_t* seq_lens,
                int32_t* logits_indices, int64_t* num_tokens_out) {
  if (!nst || !nct || !qsl || !seq_lens || !logits_indices || num_reqs < 0 ||
      qsl_len < num_reqs + 1 || block_size <= 0)
    return ORC_ERR_ARG;
  qsl[0] = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (nst[r] < 0 || nct[r] < 0) return ORC_ERR_ARG;
    qsl[r + 1] = qsl[r] + nst[r];
    seq_lens[r] = nct[r] + nst[r];
    logits_indices[r] = qsl[r + 1] - 1;
  }
  const int32_t total = qsl[num_reqs];
  for (int32_t k = num_reqs + 1; k < qsl_len; ++k) qsl[k] = total;
  if (num_tokens_out) *num_tokens_out = total;
  if (total > 0 && (!req_indices || !positions || !slot_mapping)) return ORC_ERR_ARG;
  for (int32_t r = 0; r < num_reqs; ++r) {
    for (int32_t t = 0; t < nst[r]; ++t) {
      const int32_t i = qsl[r] + t;
      const int32_t pos = nct[r] + t;
      req_indices[i] = r;
      positions[i] = pos;
      const int32_t logical = pos / block_size;
      if (!block_table || logical >= bt_cols) return ORC_ERR_RANGE;
      const int32_t phys = block_table[(int64_t)r * bt_stride + logical];
      if (phys < 0 || phys >= num_blocks) return ORC_ERR_RANGE;
      slot_mapping[i] = (int64_t)phys * block_size + pos % block_size;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* input ids and discard mask                                                */
/* ------------------------------------------------------------------------ */

/*
 * The token table holds one row of row_width (the longest sequence a request
 * may reach) token ids per request of the step, request r in row r.  For
 * every flat row i:
 *   token_indices[i] = positions[i] + req_indices[i] * row_width
 *   input_ids[i]     = token_table[token_indices[i]]   (the table read as flat)
 * and for every request r:
 *   discard[r] = 1 if seq_lens[r] < num_tokens_total[r] else 0
 * (seq_lens = computed + scheduled tokens, num_tokens_total = the request's
 * known token count: a request still short of it is mid-prefill, and the token
 * sampled from its last row is thrown away).  Returns ORC_ERR_RANGE when a row's
 * request is outside [0, num_reqs) or its position outside [0, row_width).
 */
int orc_input_ids(const int32_t* token_table, int64_t row_width, int32_t num_reqs,
                  const int32_t* req_indices, const int32_t* positions, int32_t num_tokens,
                  const int32_t* seq_lens, const int32_t* num_tokens_total,
                  int64_t* token_indices, int32_t* input_ids, uint8_t* discard) {
  if (num_reqs < 0 || num_tokens < 0 || row_width <= 0) return ORC_ERR_ARG;
  if (num_tokens > 0 && (!token_table || !req_indices || !positions || !token_indices ||
                         !input_ids))
    return ORC_ERR_ARG;
  if (num_reqs > 0 && (!seq_lens || !num_tokens_total || !discard)) return ORC_ERR_ARG;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t r = req_indices[i], p = positions[i];
    if (r < 0 || r >= num_reqs || p < 0 || p >= row_width) return ORC_ERR_RANGE;
    token_indices[i] = (int64_t)p + (int64_t)r * row_width;
    input_ids[i] = token_table[token_indices[i]];
  }
  for (int32_t r = 0; r < num_reqs; ++r) discard[r] = seq_lens[r] < num_tokens_total[r] ? 1 : 0;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* block copy and zeroing                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Every pool keeps a block as one contiguous run of block_bytes bytes (all kv
 * heads of one block: num_kv_heads * block_size * head_dim elements, whatever
 * the order inside), so both operations are plain byte moves.
 *
 * orc_copy_blocks: for each pair k, block pairs[2k+1] of both pools becomes a
 * byte copy of block pairs[2k] (the pairs are applied in order).
 * orc_zero_blocks: every byte of the listed blocks of both pools becomes 0.
 * Both return ORC_ERR_RANGE for a block id outside [0, num_blocks).
 */
int orc_copy_blocks(uint8_t* key_cache, uint8_t* value_cache, int64_t num_blocks,
                    int64_t block_bytes, const int32_t* pairs, int32_t num_pairs) {
  if (num_blocks < 0 || block_bytes <= 0 || num_pairs < 0) return ORC_ERR_ARG;
  if (num_pairs > 0 && (!key_cache || !value_cache || !pairs)) return ORC_ERR_ARG;
  for (int32_t k = 0; k < num_pairs; ++k) {
    const int64_t src = pairs[2 * k], dst = pairs[2 * k + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return ORC_ERR_RANGE;
  }
  for (int32_t k = 0; k < num_pairs; ++k) {
    const int64_t src = pairs[2 * k], dst = pairs[2 * k + 1];
    memmove(key_cache + dst * block_bytes, key_cache + src * block_bytes, (size_t)block_bytes);
    memmove(value_cache + dst * block_bytes, value_cache + src * block_bytes, (size_t)block_bytes);
  }
  return ORC_OK;
}

int orc_zero_blocks(uint8_t* key_cache, uint8_t* value_cache, int64_t num_blocks,
                    int64_t block_bytes, const int32_t* block_ids, int32_t num_ids) {
  if (num_blocks < 0 || block_bytes <= 0 || num_ids < 0) return ORC_ERR_ARG;
  if (num_ids > 0 && (!key_cache || !value_cache || !block_ids)) return ORC_ERR_ARG;
  for (int32_t k = 0; k < num_ids; ++k)
    if (block_ids[k] < 0 || block_ids[k] >= num_blocks) return ORC_ERR_RANGE;
  for (int32_t k = 0; k < num_ids; ++k) {
    memset(key_cache + (int64_t)block_ids[k] * block_bytes, 0, (size_t)block_bytes);
    memset(value_cache + (int64_t)block_ids[k] * block_bytes, 0, (size_t)block_bytes);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* kv_write                                                                  */
/* ------------------------------------------------------------------------ */

/* Element of (block, head, token, dim) in a 16-bit or fp32 K pool.  Each
 * (block, head) run of head_dim * block_size elements is cut into slabs of
 * KW dims, ordered [dim / KW][token][dim % KW], with KW = 32 -- or KW =
 * head_dim when 32 does not divide it (then the run is plain [token][dim]).
 * An interface fact of the library's pools. */
static int64_t orc_k_elem(int64_t block, int32_t head, int32_t tok, int32_t dim,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim) {
  const int32_t kw = head_dim % 32 == 0 ? 32 : head_dim;
  const int64_t run = (block * num_kv_heads + head) * (int64_t)head_dim * block_size;
  return run + ((int64_t)(dim / kw) * block_size + tok) * kw + dim % kw;
}

/* Element of (block, head, token, dim) in a 16-bit or fp32 V pool.  Each
 * (block, head) run of head_dim * block_size elements is cut into tiles of
 * DW dims x TG tokens, ordered [dim / DW][token / TG][dim % DW][token % TG],
 * with DW = 16 and TG = 4 -- or DW = head_dim when 16 does not divide it,
 * and TG = block_size when 4 does not divide it (then the run is plain
 * [dim][token]).  An interface fact of the library's pools. */
static int64_t orc_v_elem(int64_t block, int32_t head, int32_t tok, int32_t dim,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim) {
  const int32_t dw = head_dim % 16 == 0 ? 16 : head_dim;
  const int32_t tg = block_size % 4 == 0 ? 4 : block_size;
  const int64_t run = (block * num_kv_heads + head) * (int64_t)head_dim * block_size;
  const int64_t tile = (int64_t)(dim / dw) * (block_size / tg) + tok / tg;
  return run + tile * dw * tg + (int64_t)(dim % dw) * tg + tok % tg;
}

static int cmp_i64(const void* a, const void* b) {
  const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/*
 * For every token i with slot s = slot_mapping[i] >= 0 and every kv head h:
 * K row key[i][h][:] goes to block s / bs, in-block offset s % bs, head h of
 * the K pool; the V row likewise to the V pool.  The bytes are copied as they
 * are (a write, no arithmetic).  key/value rows are [T][num_kv_heads][head_dim]
 * with a row stride (elements between consecutive tokens) of key_row_stride /
 * value_row_stride.  Rejects slots outside the pool and duplicate slots.
 */
int orc_kv_write(const void* key, const void* value, int64_t key_row_stride,
                 int64_t value_row_stride, void* key_cache, void* value_cache,
                 int64_t num_blocks, const int64_t* slot_mapping, int32_t num_tokens,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t elem_bytes) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      (elem_bytes != 2 && elem_bytes != 4))
    return ORC_ERR_ARG;
  if (num_tokens == 0) return ORC_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return ORC_ERR_ARG;
  const int64_t pool_slots = num_blocks * block_size;
  int64_t* seen = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_tokens);
  if (!seen) return ORC_ERR_NOMEM;
  int32_t n_seen = 0;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    if (s >= pool_slots) { free(seen); return ORC_ERR_RANGE; }
    seen[n_seen++] = s;
  }
  qsort(seen, (size_t)n_seen, sizeof(int64_t), cmp_i64);
  for (int32_t k = 1; k < n_seen; ++k)
    if (seen[k] == seen[k - 1]) { free(seen); return ORC_ERR_DUP; }
  free(seen);

  const char* ksrc = (const char*)key;
  const char* vsrc = (const char*)value;
  char* kdst = (char*)key_cache;
  char* vdst = (char*)value_cache;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    const int64_t block = s / block_size;
    const int32_t off = (int32_t)(s % block_size);
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      for (int32_t c = 0; c < head_dim; ++c) {
        const int64_t src_k = (int64_t)i * key_row_stride + (int64_t)h * head_dim + c;
        const int64_t src_v = (int64_t)i * value_row_stride + (int64_t)h * head_dim + c;
        const int64_t dk = orc_k_elem(block, h, off, c, num_kv_heads, block_size, head_dim);
        const int64_t dv = orc_v_elem(block, h, off, c, num_kv_heads, block_size, head_dim);
        memcpy(kdst + dk * elem_bytes, ksrc + src_k * elem_bytes, (size_t)elem_bytes);
        memcpy(vdst + dv * elem_bytes, vsrc + src_v * elem_bytes, (size_t)elem_bytes);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* FP8 cache                                                                 */
/* ------------------------------------------------------------------------ */

static double orc_load(const void* base, int64_t idx, int32_t dtype);

/*
 * FP8 E4M3 in the OCP 8-bit floating point format (the "fn" variant: no
 * infinities).  Bit 7 is the sign, bits 6..3 the exponent field E (bias 7),
 * bits 2..0 the mantissa M.  E = 1..15 encodes (1 + M/8) * 2^(E-7), except
 * E = 15 with M = 7, which is NaN; E = 0 encodes the subnormal (M/8) * 2^-6.
 * The largest finite magnitude is 1.75 * 2^8 = 448.  The pages name the FP8
 * cache but not the format; E4M3 with a per-tensor scale is the plainest
 * reading of an "fp8" cache dtype that comes with k_scale and v_scale.
 */
double orc_fp8_decode(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -mag : mag;
}

/*
 * The E4M3 code of x: the nearest representable value, ties to the even
 * mantissa; finite magnitudes at or above 448 saturate to +-448 (there is no
 * infinity to round to); NaN gives the NaN code with x's sign.
 */
uint8_t orc_fp8_encode(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  const double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  /* spacing of representable values around a: 2^(k-3) in the binade
   * [2^k, 2^(k+1)) for k >= -6, and 2^-9 below 2^-6 (the subnormals) */
  int k;
  frexp(a, &k);
  k -= 1;
  const double q = (k < -6) ? ldexp(1.0, -9) : ldexp(1.0, k - 3);
  const double v = rint(a / q) * q; /* a / q is exact; rint rounds half to even */
  if (v == 0.0) return sign;
  if (v < ldexp(1.0, -6)) return sign | (uint8_t)(v / ldexp(1.0, -9));
  int e;
  frexp(v, &e);
  e -= 1; /* v in [2^e, 2^(e+1)) */
  const int m = (int)(v / ldexp(1.0, e - 3)) - 8;
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* Byte of (block, head, token, dim) in an FP8 K pool (block_size 16, head_dim
 * a multiple of 64).  Each (block, head) run of head_dim * 16 bytes is laid
 * out as [dim / 64][token][dim % 64]: slabs of 64 dims, one 64-byte row per
 * token.  An interface fact of the library's pools. */
static int64_t orc_k8_byte(int64_t block, int32_t head, int32_t tok, int32_t dim,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim) {
  const int64_t run = (block * num_kv_heads + head) * (int64_t)head_dim * block_size;
  return run + ((int64_t)(dim / 64) * block_size + tok) * 64 + dim % 64;
}

/* Byte of (block, head, token, dim) in an FP8 V pool (block_size 16, head_dim
 * a multiple of 64).  Each (block, head) run of head_dim * 16 bytes is laid
 * out as [dim / 64][token / 4][dim % 16][(dim / 16) % 4][token % 4]: sixteen
 * consecutive bytes hold four tokens of four dims 16 apart.  An interface
 * fact of the library's pools (the pages leave the layout open). */
static int64_t orc_v8_byte(int64_t block, int32_t head, int32_t tok, int32_t dim,
                           int32_t num_kv_heads, int32_t block_size, int32_t head_dim) {
  const int64_t run = (block * num_kv_heads + head) * (int64_t)head_dim * block_size;
  const int32_t within =
      ((((dim / 64) * 4 + tok / 4) * 16 + dim % 16) * 4 + (dim / 16) % 4) * 4 + tok % 4;
  return run + within;
}

/*
 * The FP8 form of orc_kv_write: for every token i with slot s >= 0 and every
 * kv head h and dim c, the K pool byte of (s / bs, h, s % bs, c) becomes
 * orc_fp8_encode(k / k_scale) with k = key[i][h][c] and the division done in
 * binary32, and the V pool byte likewise with v_scale.  key/value hold
 * elem_bytes = 2 (bf16) or 4 (fp32) elements.  block_size must be 16 and
 * head_dim a multiple of 64; k_scale and v_scale positive and finite.
 * Rejects slots outside the pool and duplicate slots.
 */
int orc_kv_write_fp8(const void* key, const void* value, int64_t key_row_stride,
                     int64_t value_row_stride, uint8_t* key_cache, uint8_t* value_cache,
                     int64_t num_blocks, const int64_t* slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t elem_bytes, float k_scale, float v_scale) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 64 != 0 ||
      block_size != 16 || (elem_bytes != 2 && elem_bytes != 4) || !(k_scale > 0.0f) ||
      !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
    return ORC_ERR_ARG;
  if (num_tokens == 0) return ORC_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return ORC_ERR_ARG;
  const int64_t pool_slots = num_blocks * block_size;
  int64_t* seen = (int64_t*)malloc(sizeof(int64_t) * (size_t)num_tokens);
  if (!seen) return ORC_ERR_NOMEM;
  int32_t n_seen = 0;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    if (s >= pool_slots) { free(seen); return ORC_ERR_RANGE; }
    seen[n_seen++] = s;
  }
  qsort(seen, (size_t)n_seen, sizeof(int64_t), cmp_i64);
  for (int32_t k = 1; k < n_seen; ++k)
    if (seen[k] == seen[k - 1]) { free(seen); return ORC_ERR_DUP; }
  free(seen);

  const int32_t dtype = (elem_bytes == 2) ? ORC_BF16 : ORC_F32;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0) continue;
    const int64_t block = s / block_size;
    const int32_t off = (int32_t)(s % block_size);
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      for (int32_t c = 0; c < head_dim; ++c) {
        const int64_t src_k = (int64_t)i * key_row_stride + (int64_t)h * head_dim + c;
        const int64_t src_v = (int64_t)i * value_row_stride + (int64_t)h * head_dim + c;
        const float kq = (float)orc_load(key, src_k, dtype) / k_scale;
        const float vq = (float)orc_load(value, src_v, dtype) / v_scale;
        key_cache[orc_k8_byte(block, h, off, c, num_kv_heads, block_size, head_dim)] =
            orc_fp8_encode(kq);
        value_cache[orc_v8_byte(block, h, off, c, num_kv_heads, block_size, head_dim)] =
            orc_fp8_encode(vq);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */

/* Exact widening of one stored element to fp64.  bf16 is the top half of an
 * IEEE binary32, so shifting its 16 bits up gives the same value as fp32. */
static double orc_load(const void* base, int64_t idx, int32_t dtype) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  int32_t req;      /* request index                              */
  int32_t kv_head;  /* kv head                                    */
  int32_t first;    /* first entry in the sorted selection        */
  int32_t count;    /* number of selected rows in this work item  */
} orc_item;

typedef struct {
  int32_t row;  /* flat row index                  */
  int32_t sel;  /* position in the caller's list   */
  int32_t req;  /* request owning the row          */
} orc_sel;

static int cmp_sel(const void* a, const void* b) {
  const orc_sel* x = (const orc_sel*)a;
  const orc_sel* y = (const orc_sel*)b;
  if (x->req != y->req) return (x->req > y->req) - (x->req < y->req);
  return (x->row > y->row) - (x->row < y->row);
}

/*
 * out[k][h][:] for each selected flat row rows[k] (all T rows when rows is
 * NULL, in which case num_rows must equal qsl[num_reqs]) and each q head h:
 *
 *   r   = the request with qsl[r] <= row < qsl[r+1]
 *   L   = seq_lens[r], q_len = qsl[r+1] - qsl[r], t = row - qsl[r]
 *   p   = L - q_len + t                                  (absolute position)
 *   g   = h / (num_q_heads / num_kv_heads)
 *   Kr, Vr = the request's first p+1 cache rows for head g, gathered in
 *            logical order: token j comes from physical block
 *            block_table[r][j / bs], in-block offset j % bs
 *   s_j = scale * sum_c q[row][h][c] * Kr[j][c]          for j = 0..p
 *   w_j = exp(s_j - max_j s_j)
 *   out = sum_j w_j * Vr[j][:] / sum_j w_j
 *
 * Everything is fp64; inputs (fp32 or bf16) are widened exactly.  q rows are
 * [T][num_q_heads][head_dim] with row stride q_row_stride elements.
 * Returns ORC_ERR_PRECOND when q_len > seq_len for a request that has a
 * selected row, ORC_ERR_RANGE when a needed table column or block id is out of
 * range.  num_threads <= 0 uses the OpenMP default.
 */
/*
 * orc_attention_kv is orc_attention with the cache dtype given apart from the
 * query dtype: kv_dtype = ORC_FP8 reads every K element as
 * orc_fp8_decode(byte) * k_scale (V likewise with v_scale) from the FP8 pool
 * layouts above; any other kv_dtype must equal dtype and ignores the scales.
 * The widening is exact in fp64, so the attention arithmetic is unchanged.
 */
int orc_attention_kv(const void* q, int64_t q_row_stride, const void* key_cache,
                     const void* value_cache, int32_t dtype, int32_t kv_dtype, double k_scale,
                     double v_scale, const int32_t* qsl, const int32_t* seq_lens,
                     const int32_t* block_table, int64_t bt_stride, int32_t bt_cols,
                     int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int64_t num_blocks, double scale,
                     const int32_t* rows, int32_t num_rows, double* out, int32_t num_threads) {
  if (!q || !key_cache || !value_cache || !qsl || !seq_lens || !block_table || !out ||
      num_reqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_rows < 0 || num_q_heads % num_kv_heads != 0 ||
      (dtype != ORC_F32 && dtype != ORC_BF16) ||
      (kv_dtype != dtype && kv_dtype != ORC_FP8) ||
      (kv_dtype == ORC_FP8 && (block_size != 16 || head_dim % 64 != 0)))
    return ORC_ERR_ARG;
  const int32_t total_rows = qsl[num_reqs];
  if (!rows && num_rows != total_rows) return ORC_ERR_ARG;
  if (num_rows == 0) return ORC_OK;
  const int32_t group = num_q_heads / num_kv_heads;

  /* Tag every selected row with its request, then sort by (request, row). */
  orc_sel* sel = (orc_sel*)malloc(sizeof(orc_sel) * (size_t)num_rows);
  if (!sel) return ORC_ERR_NOMEM;
  for (int32_t k = 0; k < num_rows; ++k) {
    const int32_t row = rows ? rows[k] : k;
    if (row < 0 || row >= total_rows) { free(sel); return ORC_ERR_PRECOND; }
    int32_t lo = 0, hi = num_reqs - 1; /* last r with qsl[r] <= row */
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (qsl[mid] <= row) lo = mid; else hi = mid - 1;
    }
    while (lo < num_reqs - 1 && qsl[lo + 1] <= row) ++lo;
    sel[k].row = row;
    sel[k].sel = k;
    sel[k].req = lo;
  }
  qsort(sel, (size_t)num_rows, sizeof(orc_sel), cmp_sel);

  /* Check the preconditions and cut the selection into work items:
   * (request, kv head, up to 16 consecutive selected rows). */
  const int32_t chunk = 16;
  int32_t n_items = 0;
  for (int32_t k = 0; k < num_rows;) {
    const int32_t r = sel[k].req;
    const int32_t q_len = qsl[r + 1] - qsl[r];
    const int32_t L = seq_lens[r];
    if (q_len > L) { free(sel); return ORC_ERR_PRECOND; }
    int32_t e = k;
    while (e < num_rows && sel[e].req == r) ++e;
    int32_t max_pos = L - q_len + (sel[e - 1].row - qsl[r]);
    const int32_t needed_blocks = max_pos / block_size + 1;
    if (needed_blocks > bt_cols) { free(sel); return ORC_ERR_RANGE; }
    for (int32_t j = 0; j < needed_blocks; ++j) {
      const int32_t b = block_table[(int64_t)r * bt_stride + j];
      if (b < 0 || b >= num_blocks) { free(sel); return ORC_ERR_RANGE; }
    }
    n_items += num_kv_heads * ((e - k + chunk - 1) / chunk);
    k = e;
  }
  orc_item* items = (orc_item*)malloc(sizeof(orc_item) * (size_t)n_items);
  if (!items) { free(sel); return ORC_ERR_NOMEM; }
  int32_t it = 0;
  for (int32_t k = 0; k < num_rows;) {
    const int32_t r = sel[k].req;
    int32_t e = k;
    while (e < num_rows && sel[e].req == r) ++e;
    for (int32_t g = 0; g < num_kv_heads; ++g)
      for (int32_t c = k; c < e; c += chunk) {
        items[it].req = r;
        items[it].kv_head = g;
        items[it].first = c;
        items[it].count = (e - c < chunk) ? (e - c) : chunk;
        ++it;
      }
    k = e;
  }

  int status = ORC_OK;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
#pragma omp parallel
  {
    double* Kr = NULL;
    double* Vr = NULL;
    double* s = NULL;
    int64_t cap = 0;
#pragma omp for schedule(dynamic, 1)
    for (int32_t w = 0; w < n_items; ++w) {
      const orc_item item = items[w];
      const int32_t r = item.req, g = item.kv_head;
      const int32_t q_len = qsl[r + 1] - qsl[r];
      const int32_t L = seq_lens[r];
      const orc_sel* last = &sel[item.first + item.count - 1];
      const int32_t n_keys = L - q_len + (last->row - qsl[r]) + 1;
      if (n_keys > cap) {
        free(Kr); free(Vr); free(s);
        cap = n_keys;
        Kr = (double*)malloc(sizeof(double) * (size_t)cap * head_dim);
        Vr = (double*)malloc(sizeof(double) * (size_t)cap * head_dim);
        s = (double*)malloc(sizeof(double) * (size_t)cap);
        if (!Kr || !Vr || !s) {
#pragma omp atomic write
          status = ORC_ERR_NOMEM;
          cap = 0;
          continue;
        }
      }
      /* Gather: logical token j lives in block_table[r][j / bs] at j % bs. */
      for (int32_t j = 0; j < n_keys; ++j) {
        const int64_t phys = block_table[(int64_t)r * bt_stride + j / block_size];
        const int32_t off = j % block_size;
        for (int32_t c = 0; c < head_dim; ++c) {
          if (kv_dtype == ORC_FP8) {
            Kr[(int64_t)j * head_dim + c] =
                orc_fp8_decode(((const uint8_t*)key_cache)[orc_k8_byte(
                    phys, g, off, c, num_kv_heads, block_size, head_dim)]) * k_scale;
            Vr[(int64_t)j * head_dim + c] =
                orc_fp8_decode(((const uint8_t*)value_cache)[orc_v8_byte(
                    phys, g, off, c, num_kv_heads, block_size, head_dim)]) * v_scale;
          } else {
            Kr[(int64_t)j * head_dim + c] = orc_load(
                key_cache, orc_k_elem(phys, g, off, c, num_kv_heads, block_size, head_dim),
                dtype);
            Vr[(int64_t)j * head_dim + c] = orc_load(
                value_cache, orc_v_elem(phys, g, off, c, num_kv_heads, block_size, head_dim),
                dtype);
          }
        }
      }
      for (int32_t k = item.first; k < item.first + item.count; ++k) {
        const int32_t row = sel[k].row;
        const int32_t p = L - q_len + (row - qsl[r]);
        for (int32_t h = g * group; h < (g + 1) * group; ++h) {
          double* o = out + ((int64_t)sel[k].sel * num_q_heads + h) * head_dim;
          const int64_t qbase = (int64_t)row * q_row_stride + (int64_t)h * head_dim;
          double m = -INFINITY;
          for (int32_t j = 0; j <= p; ++j) {
            double acc = 0.0;
            for (int32_t c = 0; c < head_dim; ++c)
              acc += orc_load(q, qbase + c, dtype) * Kr[(int64_t)j * head_dim + c];
            s[j] = scale * acc;
            if (s[j] > m) m = s[j];
          }
          double denom = 0.0;
          for (int32_t j = 0; j <= p; ++j) {
            s[j] = exp(s[j] - m);
            denom += s[j];
          }
          for (int32_t c = 0; c < head_dim; ++c) o[c] = 0.0;
          for (int32_t j = 0; j <= p; ++j) {
            const double wj = s[j] / denom;
            for (int32_t c = 0; c < head_dim; ++c) o[c] += wj * Vr[(int64_t)j * head_dim + c];
          }
        }
      }
    }
    free(Kr); free(Vr); free(s);
  }
  free(items);
  free(sel);
  return status;
}

int orc_attention(const void* q, int64_t q_row_stride, const void* key_cache,
                  const void* value_cache, int32_t dtype, const int32_t* qsl,
                  const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride,
                  int32_t bt_cols, int32_t num_reqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int64_t num_blocks, double scale,
                  const int32_t* rows, int32_t num_rows, double* out, int32_t num_threads) {
  return orc_attention_kv(q, q_row_stride, key_cache, value_cache, dtype, dtype, 1.0, 1.0, qsl,
                          seq_lens, block_table, bt_stride, bt_cols, num_reqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, scale, rows, num_rows,
                          out, num_threads);
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
