/*
 * Sanitizer driver for the host side of libsps: the sizing arithmetic, the
 * argument and shape checks, the status strings and the thread-local error
 * message. Every call made here returns before any device work (NULL
 * handles, bad sizes, too-small workspaces, or pure sizing calls), so the
 * driver needs no GPU. Built with -fsanitize=address,undefined and no
 * recovery (the library's host code too), an out-of-bounds access, a leak
 * or a signed overflow in that arithmetic ends the run with a report.
 */
#include <limits.h>
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sps.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);         \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

static int is_status(sps_status s) { return s <= 0 && s >= SPS_ERR_UNSUPPORTED; }

/* reads the whole message, so the sanitizer sees every byte */
static size_t msg_len(void) {
  const char *m = sps_last_error_message();
  CHECK(m != NULL);
  return strlen(m);
}

static void sizing_grid(void) {
  const int64_t ns[] = {0, 1, 1023, 1024, 1025, 8191, 8192, 2000000, 2147483646LL,
                        2147483647LL, 2147483648LL, INT64_MAX, -1, INT64_MIN};
  const int64_t ds[] = {1, 30522, 1200000, 2147483646LL, 2147483647LL, INT64_MAX, 0, -1};
  const int64_t zs[] = {0, 1, 86000000, (1LL << 29) - 65, (1LL << 29) - 64, 2147483647LL,
                        INT64_MAX, -1};
  const int32_t cs[] = {INT32_MIN, -1, 0, 1, 7, 1024, 1025, 8192, 1048576, 1048577, INT32_MAX};
  int ok = 0;
  for (size_t a = 0; a < sizeof ns / sizeof *ns; ++a)
    for (size_t b = 0; b < sizeof ds / sizeof *ds; ++b)
      for (size_t c = 0; c < sizeof zs / sizeof *zs; ++c)
        for (size_t d = 0; d < sizeof cs / sizeof *cs; ++d) {
          size_t p = 1, s = 1;
          sps_status st = sps_items_workspace_size(ns[a], ds[b], zs[c], cs[d], &p, &s);
          CHECK(is_status(st));
          if (st == SPS_OK) {
            ++ok;
            CHECK(p % 256 == 0 && s % 256 == 0 && p > 0 && s > 0);
          } else {
            CHECK(msg_len() > 0);
          }
        }
  CHECK(ok > 0);
  for (int64_t z = -2; z < 40; ++z) {
    size_t n = 0;
    CHECK(sps_bsc_offsets_bytes(z, &n) == (z < 0 ? SPS_ERR_INVALID_ARGUMENT : SPS_OK));
    if (z >= 0) CHECK(n % 4 == 0 && n * 8 >= (size_t)(10 * z));
  }
  const int64_t big[] = {715827882LL, 715827883LL, 2147483647LL, INT64_MAX / 10,
                         INT64_MAX / 10 + 1, INT64_MAX};
  for (size_t k = 0; k < sizeof big / sizeof *big; ++k) {
    size_t n = 0;
    sps_status st = sps_bsc_offsets_bytes(big[k], &n);
    CHECK(st == (big[k] <= 715827882LL ? SPS_OK : SPS_ERR_OVERFLOW));
  }
}

static void null_handles(void) {
  void *out = (void *)1;
  CHECK(sps_prepare(NULL, 8192, NULL, 0, NULL, 0, NULL, (sps_items **)&out) ==
        SPS_ERR_INVALID_ARGUMENT);
  CHECK(out == NULL);
  CHECK(sps_prepare(NULL, 8192, NULL, 0, NULL, 0, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_prepare_queries(NULL, NULL, NULL, 0, NULL, (sps_queries **)&out) ==
        SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_chunk(NULL, NULL, 0, NULL, 8192, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_chunk_static(NULL, NULL, 0, NULL, 8192, NULL, NULL) ==
        SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_stream(NULL, NULL, 0, 1, NULL, 8192, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_stream_host(NULL, NULL, 0, 1, NULL, 8192, NULL, NULL, 8192, NULL, NULL,
                               NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_chunk_threshold(NULL, NULL, 0, 0.5f, NULL, 0, NULL, NULL, NULL) ==
        SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_cosine_chunk_half(NULL, NULL, 0, NULL, 8192, NULL, NULL) ==
        SPS_ERR_INVALID_ARGUMENT);
  int64_t a = 0, b = 0, c = 0;
  int32_t d = 0, e = 0, f = 0;
  CHECK(sps_items_info(NULL, &a, &b, &c, &d, &e) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_items_slices(NULL, &d, &e, &c) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_items_heavy_dims(NULL, NULL, &f, 1, &f) == SPS_ERR_INVALID_ARGUMENT);
  size_t z = 0;
  CHECK(sps_items_half_workspace_size(NULL, &z) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_items_enable_half(NULL, NULL, 0, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_queries_workspace_size(NULL, 10, 10, 10, &z) == SPS_ERR_INVALID_ARGUMENT);
  const float *inv = NULL;
  CHECK(sps_queries_inv_norms(NULL, &inv) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_row_inv_norms(NULL, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_validate_csr(NULL, NULL, NULL, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_bsc_decode(NULL, NULL, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_bsc_encode_sizes(NULL, NULL, NULL, NULL, NULL) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(sps_bsc_encode(NULL, NULL, NULL, 0, NULL, 0, NULL) == SPS_ERR_INVALID_ARGUMENT);
  sps_items_destroy(NULL);
  sps_queries_destroy(NULL);
  CHECK(msg_len() > 0);
}

/* CSR shapes with placeholder device addresses: every case is rejected on
 * the host, before the addresses could be used */
static void csr_shapes(void) {
  sps_items *out = NULL;
  const int32_t *P = (const int32_t *)0x1000, *I = (const int32_t *)0x2000;
  const float *V = (const float *)0x3000;
  struct {
    sps_csr m;
    int32_t chunk;
    void *ws;
    size_t wsb;
    sps_status want;
  } cases[] = {
      {{10, 100, 5, P, I, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{10, 0, 5, P, I, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{10, 100, 5, P, NULL, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{10, 100, 5, NULL, I, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{-1, 100, 5, P, I, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{10, 100, -5, P, I, V}, 8192, NULL, 0, SPS_ERR_INVALID_ARGUMENT},
      {{2147483648LL, 100, 5, P, I, V}, 8192, NULL, 0, SPS_ERR_OVERFLOW},
      {{10, INT64_MAX, 5, P, I, V}, 8192, NULL, 0, SPS_ERR_OVERFLOW},
      {{10, 100, INT64_MAX, P, I, V}, 8192, NULL, 0, SPS_ERR_OVERFLOW},
      {{10, 100, 5, P, I, V}, 0, (void *)0x10000, 16, SPS_ERR_INVALID_ARGUMENT},
      {{10, 100, 5, P, I, V}, 1048577, (void *)0x10000, 16, SPS_ERR_INVALID_ARGUMENT},
      {{10, 100, 5, P, I, V}, 8192, (void *)0x10000, 16, SPS_ERR_WORKSPACE_TOO_SMALL},
  };
  for (size_t k = 0; k < sizeof cases / sizeof *cases; ++k) {
    sps_status st = sps_prepare(&cases[k].m, cases[k].chunk, cases[k].ws, cases[k].wsb,
                                cases[k].ws ? (void *)0x20000 : NULL, cases[k].wsb, NULL, &out);
    if (st != cases[k].want) fprintf(stderr, "case %zu: status %d\n", k, (int)st);
    CHECK(st == cases[k].want);
    CHECK(out == NULL);
    CHECK(msg_len() > 0);
  }
}

static void *other_thread(void *arg) {
  (void)arg;
  size_t p, s;
  CHECK(sps_items_workspace_size(-1, 1, 1, 1, &p, &s) == SPS_ERR_INVALID_ARGUMENT);
  CHECK(strstr(sps_last_error_message(), "negative") != NULL);
  return NULL;
}

int main(void) {
  for (int code = 1; code >= -12; --code) {
    const char *s = sps_status_string((sps_status)code);
    CHECK(s != NULL && strlen(s) > 0);
  }
  sizing_grid();
  null_handles();
  csr_shapes();
  /* the error message is per thread: another thread's failure leaves ours */
  size_t p, s;
  CHECK(sps_items_workspace_size(10, 10, 0, 8192, NULL, &s) == SPS_ERR_INVALID_ARGUMENT);
  pthread_t th;
  CHECK(pthread_create(&th, NULL, other_thread, NULL) == 0);
  CHECK(pthread_join(th, NULL) == 0);
  CHECK(strstr(sps_last_error_message(), "NULL") != NULL);
  (void)p;
  puts("libsps host code: clean");
  return 0;
}
