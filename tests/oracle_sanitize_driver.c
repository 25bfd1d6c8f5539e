/*
 * oracle_sanitize_driver.c -- runs every oracle entry point on small ragged
 * inputs, valid and invalid, so that a build of oracle.c with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py) sees every
 * loop bound and error path.  Test infrastructure: it links oracle.c and
 * nothing else.  Exits 0 when every call returns the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_prepare(const int32_t*, const int32_t*, const int32_t*, int64_t, int32_t, int32_t,
                int32_t, int32_t, int64_t, int32_t*, int32_t*, int64_t*, int32_t*, int32_t*,
                int32_t*, int64_t*);
int orc_input_ids(const int32_t*, int64_t, int32_t, const int32_t*, const int32_t*, int32_t,
                  const int32_t*, const int32_t*, int64_t*, int32_t*, uint8_t*);
int orc_copy_blocks(uint8_t*, uint8_t*, int64_t, int64_t, const int32_t*, int32_t);
int orc_zero_blocks(uint8_t*, uint8_t*, int64_t, int64_t, const int32_t*, int32_t);
int orc_kv_write(const void*, const void*, int64_t, int64_t, void*, void*, int64_t,
                 const int64_t*, int32_t, int32_t, int32_t, int32_t, int32_t);
int orc_kv_write_fp8(const void*, const void*, int64_t, int64_t, uint8_t*, uint8_t*, int64_t,
                     const int64_t*, int32_t, int32_t, int32_t, int32_t, int32_t, float, float);
double orc_fp8_decode(uint8_t);
uint8_t orc_fp8_encode(float);
int orc_attention_kv(const void*, int64_t, const void*, const void*, int32_t, int32_t, double,
                     double, const int32_t*, const int32_t*, const int32_t*, int64_t, int32_t,
                     int32_t, int32_t, int32_t, int32_t, int32_t, int64_t, double,
                     const int32_t*, int32_t, double*, int32_t);
int orc_attention(const void*, int64_t, const void*, const void*, int32_t, const int32_t*,
                  const int32_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t,
                  int32_t, int32_t, int64_t, double, const int32_t*, int32_t, double*, int32_t);

static int failures = 0;

static void expect(const char* what, int got, int ok) {
  if ((got == 0) != ok) {
    fprintf(stderr, "%s: status %d, expected %s\n", what, got, ok ? "0" : "an error");
    ++failures;
  }
}

/* exact-size heap copies, so the sanitizer sees any read past an array */
static void* dup_bytes(const void* src, size_t n) {
  void* p = malloc(n ? n : 1);
  if (n) memcpy(p, src, n);
  return p;
}

int main(void) {
  enum { R = 3, T = 10, H = 2, HQ = 4, D = 64, BS = 16, NB = 6, COLS = 2 };
  const int32_t nst_v[R] = {2, 5, 3}, nct_v[R] = {14, 0, 9};
  const int32_t bt_v[R * COLS] = {4, 1, 0, -1, 5, -1};
  int32_t* nst = dup_bytes(nst_v, sizeof nst_v);
  int32_t* nct = dup_bytes(nct_v, sizeof nct_v);
  int32_t* bt = dup_bytes(bt_v, sizeof bt_v);
  int32_t* req = malloc(T * 4);
  int32_t* pos = malloc(T * 4);
  int64_t* slot = malloc(T * 8);
  int32_t* qsl = malloc((R + 1 + 2) * 4);
  int32_t* sl = malloc(R * 4);
  int32_t* li = malloc(R * 4);
  int64_t nt = 0;
  expect("prepare", orc_prepare(nst, nct, bt, COLS, COLS, R, R + 3, BS, NB, req, pos, slot, qsl,
                                sl, li, &nt), 1);
  int32_t* bad_bt = dup_bytes(bt_v, sizeof bt_v);
  bad_bt[0] = NB; /* out of the pool */
  expect("prepare, block out of range",
         orc_prepare(nst, nct, bad_bt, COLS, COLS, R, R + 1, BS, NB, req, pos, slot, qsl, sl, li,
                     &nt), 0);

  /* input ids over a 3 x 40 token table */
  int32_t* table = malloc(R * 40 * 4);
  for (int i = 0; i < R * 40; ++i) table[i] = 7 * i;
  int32_t* total = dup_bytes(sl, R * 4);
  total[1] += 3;
  int64_t* tok_idx = malloc(T * 8);
  int32_t* ids = malloc(T * 4);
  uint8_t* discard = malloc(R);
  expect("input ids", orc_input_ids(table, 40, R, req, pos, T, sl, total, tok_idx, ids, discard),
         1);
  expect("input ids, narrow table",
         orc_input_ids(table, 10, R, req, pos, T, sl, total, tok_idx, ids, discard), 0);

  /* bf16 (2-byte) and fp32 (4-byte) pools, written then read */
  for (int eb = 2; eb <= 4; eb += 2) {
    const size_t pool = (size_t)NB * H * BS * D * eb;
    uint8_t* kc = calloc(pool, 1);
    uint8_t* vc = calloc(pool, 1);
    uint8_t* key = malloc((size_t)T * H * D * eb);
    uint8_t* val = malloc((size_t)T * H * D * eb);
    for (size_t i = 0; i < (size_t)T * H * D * eb; ++i) {
      key[i] = (uint8_t)(eb == 2 ? (i & 1 ? 0x3f : 0x80) : (i % 4 == 3 ? 0x3f : 0));
      val[i] = key[i];
    }
    for (size_t i = 0; i < pool; ++i) kc[i] = vc[i] = key[i % ((size_t)T * H * D * eb)];
    expect("kv write", orc_kv_write(key, val, H * D, H * D, kc, vc, NB, slot, T, H, D, BS, eb), 1);
    int64_t* dupslot = dup_bytes(slot, T * 8);
    dupslot[3] = dupslot[2];
    expect("kv write, duplicate slot",
           orc_kv_write(key, val, H * D, H * D, kc, vc, NB, dupslot, T, H, D, BS, eb), 0);
    uint8_t* q = malloc((size_t)T * HQ * D * eb);
    memcpy(q, key, (size_t)T * H * D * eb);
    memcpy(q + (size_t)T * H * D * eb, key, (size_t)T * H * D * eb);
    double* out = malloc((size_t)T * HQ * D * sizeof(double));
    const double scale = 0.125;
    expect("attention", orc_attention(q, HQ * D, kc, vc, eb == 2 ? 1 : 0, qsl, sl, bt, COLS, COLS,
                                      R, HQ, H, D, BS, NB, scale, NULL, T, out, 2), 1);
    const int32_t rows_v[3] = {9, 0, 4};
    int32_t* rows = dup_bytes(rows_v, sizeof rows_v);
    expect("attention, row subset", orc_attention(q, HQ * D, kc, vc, eb == 2 ? 1 : 0, qsl, sl, bt,
                                                  COLS, COLS, R, HQ, H, D, BS, NB, scale, rows,
                                                  3, out, 1), 1);
    int32_t* bad_sl = dup_bytes(sl, R * 4);
    bad_sl[1] = 2; /* q_len 5 > seq_len 2 */
    expect("attention, q_len > seq_len",
           orc_attention(q, HQ * D, kc, vc, eb == 2 ? 1 : 0, qsl, bad_sl, bt, COLS, COLS, R, HQ,
                         H, D, BS, NB, scale, NULL, T, out, 1), 0);
    const int32_t pairs_v[4] = {0, 3, 2, 5};
    int32_t* pairs = dup_bytes(pairs_v, sizeof pairs_v);
    expect("copy blocks", orc_copy_blocks(kc, vc, NB, (int64_t)H * BS * D * eb, pairs, 2), 1);
    pairs[3] = NB;
    expect("copy blocks, out of range",
           orc_copy_blocks(kc, vc, NB, (int64_t)H * BS * D * eb, pairs, 2), 0);
    const int32_t zid_v[3] = {1, 1, 5};
    int32_t* zid = dup_bytes(zid_v, sizeof zid_v);
    expect("zero blocks", orc_zero_blocks(kc, vc, NB, (int64_t)H * BS * D * eb, zid, 3), 1);
    zid[0] = -1;
    expect("zero blocks, out of range",
           orc_zero_blocks(kc, vc, NB, (int64_t)H * BS * D * eb, zid, 3), 0);
    free(kc); free(vc); free(key); free(val); free(dupslot); free(q); free(out); free(rows);
    free(bad_sl); free(pairs); free(zid);
  }

  /* FP8: every code through the codec, then a write and a read over FP8 pools */
  for (int c = 0; c < 256; ++c) {
    const double x = orc_fp8_decode((uint8_t)c);
    if (x == x && orc_fp8_encode((float)x) != (uint8_t)c && (c & 0x7f) != 0) {
      fprintf(stderr, "fp8 code %d does not round-trip\n", c);
      ++failures;
    }
  }
  {
    const size_t pool = (size_t)NB * H * BS * D;
    uint8_t* kc = calloc(pool, 1);
    uint8_t* vc = calloc(pool, 1);
    uint16_t* key = malloc((size_t)T * H * D * 2);
    for (int i = 0; i < T * H * D; ++i) key[i] = (uint16_t)(0x3c00 + (i % 97));
    expect("fp8 write", orc_kv_write_fp8(key, key, H * D, H * D, kc, vc, NB, slot, T, H, D, BS, 2,
                                         0.0125f, 0.02f), 1);
    uint16_t* q = malloc((size_t)T * HQ * D * 2);
    for (int i = 0; i < T * HQ * D; ++i) q[i] = (uint16_t)(0x3c00 + (i % 31));
    double* out = malloc((size_t)T * HQ * D * sizeof(double));
    expect("fp8 attention", orc_attention_kv(q, HQ * D, kc, vc, 1, 2, 0.0125, 0.02, qsl, sl, bt,
                                             COLS, COLS, R, HQ, H, D, BS, NB, 0.125, NULL, T,
                                             out, 2), 1);
    free(kc); free(vc); free(key); free(q); free(out);
  }

  free(nst); free(nct); free(bt); free(bad_bt); free(req); free(pos); free(slot); free(qsl);
  free(sl); free(li); free(table); free(total); free(tok_idx); free(ids); free(discard);
  if (failures) fprintf(stderr, "%d unexpected statuses\n", failures);
  return failures ? 1 : 0;
}
