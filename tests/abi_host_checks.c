/*
 * Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against the library's host code (the kernels are
 * not needed: every call here either only computes sizes and plans or is
 * rejected by validation before anything is enqueued).  Device pointers are
 * fake addresses that are never dereferenced.
 *
 * Exit status 0 when every expectation holds; the sanitizers abort the
 * process on the first error they find.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ka_attn.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

/* A rejected call must say why. */
#define REJECTS(call, code)                                            \
  do {                                                                 \
    const ka_status st_ = (call);                                      \
    if (st_ != (code)) {                                               \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, \
              (int)st_, (int)(code), ka_attn_last_error());            \
      ++failures;                                                      \
    } else if (ka_attn_last_error()[0] == '\0') {                      \
      fprintf(stderr, "%s:%d: %s gave no reason\n", __FILE__, __LINE__, #call); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static ka_attn_shape shape(int b, int hq, int hkv, int d, int c, int dt) {
  ka_attn_shape s;
  s.batch = b;
  s.num_q_heads = hq;
  s.num_kv_heads = hkv;
  s.head_dim = d;
  s.capacity = c;
  s.kv_dtype = dt;
  return s;
}

#define FAKE ((void*)(uintptr_t)0x1000)
#define FAKEF ((float*)(uintptr_t)0x10000000)  /* inputs */
#define FAKEO ((float*)(uintptr_t)0x40000000)  /* outputs, far from the inputs */

/* Shapes at the edges of what the ABI accepts, and beyond. */
static const int kBatches[] = {1, 3, 4096, INT_MAX};
static const int kHeads[][2] = {{1, 1}, {8, 1}, {8, 2}, {64, 8}, {1 << 20, 1}, {INT_MAX, 1}};
static const int kDims[] = {64, 128, 256};
static const int kCaps[] = {64, 4160, 16448, 131072};
static const int kRows[] = {-1, 0, 1, 2, 15, 16, 17, 255, 768, 769, 4096, 131072, INT_MAX};

static void size_queries(void) {
  for (unsigned bi = 0; bi < sizeof kBatches / sizeof *kBatches; ++bi)
    for (unsigned hi = 0; hi < sizeof kHeads / sizeof *kHeads; ++hi)
      for (unsigned di = 0; di < sizeof kDims / sizeof *kDims; ++di)
        for (unsigned ci = 0; ci < sizeof kCaps / sizeof *kCaps; ++ci)
          for (int dt = 0; dt < 3; ++dt) {
            const ka_attn_shape s =
                shape(kBatches[bi], kHeads[hi][0], kHeads[hi][1], kDims[di], kCaps[ci], dt);
            const size_t cb = ka_attn_cache_bytes(&s);
            const int c = kCaps[ci];
            for (unsigned ri = 0; ri < sizeof kRows / sizeof *kRows; ++ri) {
              const int r = kRows[ri];
              const size_t pw = ka_attn_prefill_workspace_bytes(&s, r);
              const size_t fw = ka_attn_append_prefill_workspace_bytes(&s, r);
              const size_t dw = ka_attn_decode_workspace_bytes(&s, r);
              (void)dw;
              const size_t rw = ka_attn_prefill_ragged_workspace_bytes(&s, (int64_t)r * 3);
              (void)rw;
              const int starts[] = {0, 1, c / 2, c - 1, c, INT_MAX};
              for (unsigned si = 0; si < sizeof starts / sizeof *starts; ++si) {
                const size_t need = ka_attn_prefill_workspace_need(&s, starts[si], r);
                const size_t fneed = ka_attn_append_prefill_workspace_need(&s, starts[si], r);
                /* a valid call never needs more than the bound for its rows */
                if (cb != 0 && r > 0 && (long long)starts[si] + r <= c) {
                  EXPECT(need <= pw);
                  EXPECT(fneed <= fw && need <= fneed);
                }
              }
              ka_attn_memory m;
              memset(&m, 0, sizeof m);
              const ka_status st = ka_attn_session_memory(&s, r, &m);
              if (st == KA_OK) {
                EXPECT(m.cache_bytes == 2 * cb);
                EXPECT(m.total_bytes >= m.cache_bytes);
              }
            }
            /* ragged tables: B host entries are read only when the shape is valid */
            if (cb != 0 && kBatches[bi] <= 4096) {
              static int32_t st[4096], rows[4096];
              for (int b = 0; b < kBatches[bi]; ++b) {
                st[b] = (b * 37) % c;
                rows[b] = (b % 5 == 0) ? 0 : 1 + (b * 13) % (c - st[b]);
              }
              const size_t need = ka_attn_prefill_ragged_workspace_need(&s, st, rows);
              long long total = 0;
              for (int b = 0; b < kBatches[bi]; ++b) total += rows[b];
              EXPECT(need <= ka_attn_prefill_ragged_workspace_bytes(&s, total));
            }
          }
}

static void rejections(void) {
  const ka_attn_shape ok = shape(2, 8, 1, 256, 4160, KA_DTYPE_BF16);
  const ka_attn_shape bad[] = {
      shape(0, 8, 1, 256, 4160, 1),       shape(2, 0, 1, 256, 4160, 1),
      shape(2, 8, 0, 256, 4160, 1),       shape(2, 8, 3, 256, 4160, 1),
      shape(2, 8, 1, 96, 4160, 1),        shape(2, 8, 1, 256, 4100, 1),
      shape(2, 8, 1, 256, 0, 1),          shape(2, 8, 1, 256, 131136, 1),
      shape(2, 8, 1, 256, 4160, 3),       shape(2, 8, 1, 256, 4160, -1),
      shape(INT_MAX, INT_MAX, INT_MAX, 256, 131072, 0),
  };
  const int32_t ctx_ok[2] = {10, 20}, ctx_zero[2] = {0, 5}, ctx_big[2] = {4161, 5};
  const int32_t st_ok[2] = {0, 100}, rw_ok[2] = {10, 10}, rw_neg[2] = {-1, 3};
  const int32_t st_big[2] = {4159, 0}, rw_big[2] = {2, 1};

  for (unsigned i = 0; i < sizeof bad / sizeof *bad; ++i) {
    const ka_attn_shape* s = &bad[i];
    EXPECT(ka_attn_cache_bytes(s) == 0);
    EXPECT(ka_attn_append_kv(s, FAKE, FAKE, FAKEF, FAKEF, 0, 1, NULL) != KA_OK);
    EXPECT(ka_attn_prefill_chunk(s, FAKEF, FAKE, FAKE, FAKEO, 0, 1, 0.1f, FAKE, 1 << 30, NULL) !=
           KA_OK);
    EXPECT(ka_attn_decode(s, FAKEF, FAKE, FAKE, FAKEO, ctx_ok, 0.1f, FAKE, 1 << 30, NULL) != KA_OK);
    EXPECT(ka_attn_decode_step(s, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, ctx_ok, 0.1f, FAKE,
                               1 << 30, NULL) != KA_OK);
    EXPECT(ka_attn_decode_step_noalloc(s, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, ctx_ok, 0.1f,
                                       NULL) != KA_OK);
    EXPECT(ka_attn_prefill_ragged(s, FAKEF, FAKE, FAKE, FAKEO, st_ok, rw_ok, 0.1f, FAKE, 1 << 30,
                                  NULL) != KA_OK);
    EXPECT(ka_attn_append_kv_ragged(s, FAKE, FAKE, FAKEF, FAKEF, NULL, NULL, st_ok, rw_ok, NULL) !=
           KA_OK);
    EXPECT(ka_attn_rope_rows(s, FAKEF, FAKEO, FAKEF, FAKEF, 1, NULL) != KA_OK);
    ka_attn_memory m;
    EXPECT(ka_attn_session_memory(s, 768, &m) != KA_OK);
    EXPECT(ka_attn_prefill_workspace_bytes(s, 768) == 0);
    EXPECT(ka_attn_decode_workspace_bytes(s, 100) == 0);
  }
  REJECTS(ka_attn_append_kv(NULL, FAKE, FAKE, FAKEF, FAKEF, 0, 1, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_kv(&ok, NULL, FAKE, FAKEF, FAKEF, 0, 1, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_kv(&ok, FAKE, FAKE, FAKEF, FAKEF, -1, 1, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_kv(&ok, FAKE, FAKE, FAKEF, FAKEF, 0, -1, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_kv(&ok, FAKE, FAKE, FAKEF, FAKEF, 4100, 61, NULL), KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_append_kv(&ok, FAKE, FAKE, FAKEF, FAKEF, INT_MAX, INT_MAX, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_append_kv_rope(&ok, FAKE, FAKE, FAKEF, FAKEF, NULL, FAKEF, 0, 1, NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_rope_rows(&ok, FAKEF, FAKEO, FAKEF, FAKEF, -1, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, 4000, 161, 0.1f, FAKE, 1 << 30, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, INT_MAX, INT_MAX, 0.1f, FAKE, 0,
                                NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, 0, 16, NAN, FAKE, 1 << 30, NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, 0, 16, -1.f, FAKE, 1 << 30, NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, 0, 16, INFINITY, FAKE, 1 << 30,
                                NULL),
          KA_ERR_INVALID_ARGUMENT);
  {
    const size_t need = ka_attn_prefill_workspace_need(&ok, 3000, 768);
    EXPECT(need > 0);
    if (need > 0)
      REJECTS(ka_attn_prefill_chunk(&ok, FAKEF, FAKE, FAKE, FAKEO, 3000, 768, 0.1f, FAKE, need - 1,
                                    NULL),
              KA_ERR_WORKSPACE);
  }
  REJECTS(ka_attn_append_prefill_chunk(&ok, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, 4000, 161, 0.1f,
                                       FAKE, 1 << 30, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_append_prefill_chunk(&ok, FAKEF, NULL, FAKEF, FAKE, FAKE, FAKEO, 0, 16, 0.1f, FAKE,
                                       1 << 30, NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_prefill_chunk(&ok, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEF, 0, 16, 0.1f, FAKE,
                                       1 << 30, NULL),
          KA_ERR_INVALID_ARGUMENT);
  {
    const size_t need = ka_attn_append_prefill_workspace_need(&ok, 3000, 768);
    EXPECT(need > 0 && need <= ka_attn_append_prefill_workspace_bytes(&ok, 768));
    if (need > 0)
      REJECTS(ka_attn_append_prefill_chunk(&ok, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, 3000, 768,
                                           0.1f, FAKE, need - 1, NULL),
              KA_ERR_WORKSPACE);
  }
  REJECTS(ka_attn_decode(&ok, FAKEF, FAKE, FAKE, FAKEO, NULL, 0.1f, FAKE, 1 << 30, NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_decode(&ok, FAKEF, FAKE, FAKE, FAKEO, ctx_zero, 0.1f, FAKE, 1 << 30, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_decode(&ok, FAKEF, FAKE, FAKE, FAKEO, ctx_big, 0.1f, FAKE, 1 << 30, NULL),
          KA_ERR_OUT_OF_RANGE);
  {
    const int32_t ctx[2] = {4096, 4096};
    const size_t need = ka_attn_decode_workspace_bytes(&ok, 4096);
    EXPECT(need > 0);
    if (need > 0)
      REJECTS(ka_attn_decode(&ok, FAKEF, FAKE, FAKE, FAKEO, ctx, 0.1f, FAKE, need - 1, NULL),
              KA_ERR_WORKSPACE);
  }
  {
    const int32_t pos_neg[2] = {-1, 3}, pos_big[2] = {4160, 3};
    REJECTS(ka_attn_decode_step(&ok, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, pos_neg, 0.1f, FAKE,
                                1 << 30, NULL),
            KA_ERR_OUT_OF_RANGE);
    REJECTS(ka_attn_decode_step(&ok, FAKEF, FAKEF, FAKEF, FAKE, FAKE, FAKEO, pos_big, 0.1f, FAKE,
                                1 << 30, NULL),
            KA_ERR_OUT_OF_RANGE);
    REJECTS(ka_attn_decode_step(&ok, FAKEF, NULL, FAKEF, FAKE, FAKE, FAKEO, ctx_ok, 0.1f, FAKE,
                                1 << 30, NULL),
            KA_ERR_INVALID_ARGUMENT);
  }
  REJECTS(ka_attn_prefill_ragged(&ok, FAKEF, FAKE, FAKE, FAKEO, st_ok, rw_neg, 0.1f, FAKE, 1 << 30,
                                 NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_prefill_ragged(&ok, FAKEF, FAKE, FAKE, FAKEO, st_big, rw_big, 0.1f, FAKE,
                                 1 << 30, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_prefill_ragged(&ok, FAKEF, FAKE, FAKE, FAKEO, NULL, rw_ok, 0.1f, FAKE, 1 << 30,
                                 NULL),
          KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_append_kv_ragged(&ok, FAKE, FAKE, FAKEF, FAKEF, NULL, NULL, st_big, rw_big, NULL),
          KA_ERR_OUT_OF_RANGE);
  REJECTS(ka_attn_session_memory(&ok, 768, NULL), KA_ERR_INVALID_ARGUMENT);
  REJECTS(ka_attn_session_memory(&ok, -1, NULL), KA_ERR_INVALID_ARGUMENT);
  {
    const ka_attn_shape dst = shape(2, 8, 1, 256, 8256, KA_DTYPE_BF16);
    const ka_attn_shape other = shape(2, 8, 1, 256, 8256, KA_DTYPE_F32);
    REJECTS(ka_attn_cache_resize(&ok, FAKE, FAKE, &dst, FAKE, FAKE, 4161, NULL),
            KA_ERR_OUT_OF_RANGE);
    REJECTS(ka_attn_cache_resize(&ok, FAKE, FAKE, &other, FAKE, FAKE, 10, NULL),
            KA_ERR_INVALID_ARGUMENT);
    REJECTS(ka_attn_cache_resize(&ok, FAKE, FAKE, &dst, FAKE, FAKE, -1, NULL),
            KA_ERR_INVALID_ARGUMENT);
    REJECTS(ka_attn_cache_resize(NULL, FAKE, FAKE, &dst, FAKE, FAKE, 1, NULL),
            KA_ERR_INVALID_ARGUMENT);
  }
}

static void limits(void) {
  ka_attn_shape a = shape(1, KA_ATTN_MAX_Q_HEADS + 1, 1, 64, 64, KA_DTYPE_F32);
  EXPECT(ka_attn_cache_bytes(&a) == 0);
  REJECTS(ka_attn_append_kv(&a, FAKE, FAKE, FAKEF, FAKEF, 0, 1, NULL), KA_ERR_OUT_OF_RANGE);
  a = shape(KA_ATTN_MAX_BATCH + 1, 8, 1, 64, 64, KA_DTYPE_F32);
  EXPECT(ka_attn_cache_bytes(&a) == 0);
  REJECTS(ka_attn_append_kv(&a, FAKE, FAKE, FAKEF, FAKEF, 0, 1, NULL), KA_ERR_OUT_OF_RANGE);
  a = shape(1, 8, 1, 64, KA_ATTN_MAX_CAPACITY + 64, KA_DTYPE_F32);
  REJECTS(ka_attn_append_kv(&a, FAKE, FAKE, FAKEF, FAKEF, 0, 1, NULL), KA_ERR_OUT_OF_RANGE);
  /* the largest shape: every size still exact */
  a = shape(KA_ATTN_MAX_BATCH, KA_ATTN_MAX_Q_HEADS, KA_ATTN_MAX_Q_HEADS, 256, KA_ATTN_MAX_CAPACITY,
            KA_DTYPE_F32);
  EXPECT(ka_attn_cache_bytes(&a) == (size_t)KA_ATTN_MAX_BATCH * KA_ATTN_MAX_Q_HEADS *
                                        KA_ATTN_MAX_CAPACITY * 256 * 4);
  ka_attn_memory m;
  EXPECT(ka_attn_session_memory(&a, 768, &m) == KA_OK);
  EXPECT(m.total_bytes >= m.cache_bytes && m.cache_bytes == 2 * ka_attn_cache_bytes(&a));
  EXPECT(ka_attn_prefill_workspace_bytes(&a, KA_ATTN_MAX_CAPACITY) >=
         ka_attn_prefill_workspace_need(&a, 0, KA_ATTN_MAX_CAPACITY));
  EXPECT(ka_attn_prefill_ragged_workspace_bytes(&a, INT64_MAX) >=
         ka_attn_prefill_ragged_workspace_bytes(&a, 768));
  (void)ka_attn_decode_workspace_bytes(&a, KA_ATTN_MAX_CAPACITY);
}

static void strings(void) {
  for (int code = -3; code < 10; ++code) {
    const char* s = ka_attn_status_string(code);
    EXPECT(s != NULL && strlen(s) > 0);
  }
  EXPECT(strcmp(ka_attn_status_string(KA_OK), "KA_OK") == 0);
  EXPECT(ka_attn_abi_version() == KA_ATTN_ABI_VERSION);
  EXPECT(ka_attn_decode_step_noalloc_max_bytes() > 0);
}

int main(void) {
  size_queries();
  rejections();
  limits();
  strings();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
