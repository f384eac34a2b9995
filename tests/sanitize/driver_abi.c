/* Host-side driver of libm3ssm's validation paths, for a build of the
 * library whose host code carries AddressSanitizer and UndefinedBehavior-
 * Sanitizer.  Every call below returns before any HIP call (a query, or an
 * argument the host rejects), so no GPU is needed.  Pointers passed as
 * "device" memory are aligned fake addresses the host code never
 * dereferences.  Exit status 0 when every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "m3ssm.h"

static int fails = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);      \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static m3_dims dims(int64_t b, int64_t t, int64_t h, int64_t p, int64_t n, int64_t r) {
  m3_dims d = {b, t, h, p, n, r};
  return d;
}

int main(void) {
  for (int c = -2; c < 10; ++c) EXPECT(m3_status_string((m3_status)c) != NULL);
  EXPECT(m3_version() == M3SSM_VERSION);

  /* workspace queries over a sweep of shapes, including huge and negative
   * sizes: 0 (invalid or unsupported) or a multiple of 256 */
  static const int64_t bs[] = {-1, 0, 1, 3, 64, 1ll << 20, 1ll << 40};
  static const int64_t ts[] = {-5, 0, 1, 63, 64, 65, 1000, 16384, 1ll << 31, 1ll << 45};
  static const int64_t hs[] = {0, 1, 2, 16, 64, 1021, 1ll << 33};
  static const int64_t ps[] = {8, 16, 32, 64, 128, 256};
  static const int64_t ns[] = {2, 15, 16, 30, 32, 48, 64, 96, 128, 256, 512};
  static const int64_t rs[] = {0, 1, 2, 3, 4};
  static const int chunks[] = {-16, 0, 1, 16, 32, 48, 64, 128, 256};
  size_t queries = 0;
  for (size_t ib = 0; ib < sizeof bs / sizeof *bs; ++ib)
    for (size_t it = 0; it < sizeof ts / sizeof *ts; ++it)
      for (size_t ih = 0; ih < sizeof hs / sizeof *hs; ++ih)
        for (size_t ip = 0; ip < sizeof ps / sizeof *ps; ++ip)
          for (size_t in = 0; in < sizeof ns / sizeof *ns; ++in)
            for (size_t ir = 0; ir < sizeof rs / sizeof *rs; ++ir) {
              m3_dims d = dims(bs[ib], ts[it], hs[ih], ps[ip], ns[in], rs[ir]);
              for (int dt = 0; dt < 3; ++dt) {
                for (size_t ic = 0; ic < sizeof chunks / sizeof *chunks; ++ic) {
                  size_t w = m3_prefill_workspace_size(&d, chunks[ic], (m3_dtype)dt);
                  EXPECT(w % 256 == 0);
                  ++queries;
                }
                size_t wb = m3_backward_workspace_size(&d, (m3_dtype)dt);
                (void)wb;
                ++queries;
              }
            }
  EXPECT(m3_prefill_workspace_size(NULL, 64, M3_BF16) == 0);
  EXPECT(m3_backward_workspace_size(NULL, M3_BF16) == 0);

  /* rejected calls */
  unsigned char* dev = (unsigned char*)(uintptr_t)0x10000000u; /* never dereferenced */
  m3_dims d = dims(2, 100, 2, 64, 64, 1);
  size_t need = m3_prefill_workspace_size(&d, 64, M3_BF16);
  EXPECT(need > 0);
  EXPECT(m3_prefill(NULL, M3_BF16, 64, dev, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                    dev, dev, dev, (float*)dev, dev, need, NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill(&d, M3_BF16, 64, NULL, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                    dev, dev, dev, (float*)dev, dev, need, NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill(&d, M3_BF16, 64, dev + 2, (float*)dev, (float*)dev, (float*)dev,
                    (float*)dev, dev, dev, dev, (float*)dev, dev, need,
                    NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill(&d, M3_BF16, 64, dev, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                    dev, dev, dev, (float*)dev, dev, need - 256, NULL) == M3_ERR_WORKSPACE);
  EXPECT(m3_prefill(&d, M3_BF16, 64, dev, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                    dev, dev, dev, (float*)dev, dev + 16, need, NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill(&d, M3_BF16, 24, dev, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                    dev, dev, dev, (float*)dev, dev, need, NULL) == M3_ERR_NOT_SUPPORTED);
  EXPECT(m3_prefill(&d, (m3_dtype)7, 64, dev, (float*)dev, (float*)dev, (float*)dev,
                    (float*)dev, dev, dev, dev, (float*)dev, dev, need,
                    NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill_from_state(&d, M3_BF16, 64, (float*)dev, dev, NULL, dev, (float*)dev,
                               (float*)dev, (float*)dev, (float*)dev, dev, dev, dev,
                               (float*)dev, dev, need, NULL) == M3_ERR_INVALID_VALUE);
  /* h_final partially overlapping h0 */
  EXPECT(m3_prefill_from_state(&d, M3_BF16, 64, (float*)dev, NULL, NULL, dev, (float*)dev,
                               (float*)dev, (float*)dev, (float*)dev, dev, dev, dev,
                               (float*)(dev + 256), dev, need, NULL) == M3_ERR_INVALID_VALUE);
  m3_dims dd = dims(4, 1, 2, 64, 128, 4);
  EXPECT(m3_decode_step(&dd, M3_BF16, NULL, (float*)dev, dev, dev, dev, dev, dev, (float*)dev,
                        (float*)dev, (float*)dev, (float*)dev, dev, NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_decode_step(&dd, M3_BF16, (float*)(dev + 4), (float*)dev, dev, dev, dev, dev, dev,
                        (float*)dev, (float*)dev, (float*)dev, (float*)dev, dev,
                        NULL) == M3_ERR_INVALID_VALUE);
  m3_dims db = dims(1, 8, 2, 64, 48, 2);
  EXPECT(m3_block_prepass(&db, M3_BF16, dev, dev, dev, (float*)dev, (float*)dev, (float*)dev,
                          (float*)dev, (float*)dev, 1e-6f, dev, dev, dev,
                          NULL) == M3_ERR_NOT_SUPPORTED);
  m3_dims dp = dims(1, 8, 2, 64, 64, 2);
  EXPECT(m3_block_postpass(&dp, M3_BF16, NULL, (float*)dev, dev, NULL) == M3_ERR_INVALID_VALUE);
  m3_dims dw = dims(1, 64, 2, 64, 64, 1);
  EXPECT(m3_backward(&dw, M3_BF16, dev, (float*)dev, (float*)dev, NULL, (float*)dev, dev, dev,
                     dev, NULL, (float*)dev, (float*)dev, (float*)dev, (float*)dev, (float*)dev,
                     (float*)dev, (float*)dev, dev, 1u << 30, NULL) != M3_SUCCESS);
  EXPECT(m3_prefill_workspace_error(NULL, 4096, 0, NULL, NULL) == M3_ERR_INVALID_VALUE);
  EXPECT(m3_prefill_workspace_error(dev + 4, 4096, 0, NULL, NULL) == M3_ERR_INVALID_VALUE);

  printf("driver_abi: %zu workspace queries, %d failures\n", queries, fails);
  return fails ? 1 : 0;
}
