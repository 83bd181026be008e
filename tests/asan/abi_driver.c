/* Host-layer checks of the C ABI (include/tsr.h) for a build of the library
 * whose host code carries AddressSanitizer: every class of invalid argument
 * on every entry point, and sampler_init's failure and success paths. Exit
 * status 0 when every check holds; AddressSanitizer aborts the run on an
 * invalid access in the host layer. Needs no GPU (where one is present, the
 * init path runs to the end and the handle is destroyed again). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tsr.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "abi_driver: check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static tsr_params P(double t, int k, double p, double m, int mode) {
  tsr_params x;
  x.temperature = t;
  x.top_k = k;
  x.top_p = p;
  x.min_p = m;
  x.filter_mode = mode;
  return x;
}

int main(void) {
  /* error strings: every code, known or not */
  for (int c = -3; c < 64; ++c) {
    const char* s = sampler_strerror(c);
    CHECK(s != NULL && strlen(s) > 0);
  }

  /* sampler_init: argument errors leave *out NULL */
  tsr_handle h = (tsr_handle)(uintptr_t)0x10;
  CHECK(sampler_init(NULL, 0, 1, 1, 1, 0) == TSR_EINVAL);
  CHECK(sampler_init(&h, 0, 0, 10, 1, 0) == TSR_EINVAL && h == NULL);
  h = (tsr_handle)(uintptr_t)0x10;
  CHECK(sampler_init(&h, 0, 10, 0, 1, 0) == TSR_EINVAL && h == NULL);
  CHECK(sampler_init(&h, 0, 10, 10, 33, 0) == TSR_EINVAL && h == NULL);
  CHECK(sampler_init(&h, 0, -5, 10, 1, 0) == TSR_EINVAL && h == NULL);
  CHECK(sampler_init(&h, -1, 10, 10, 1, 0) != TSR_OK && h == NULL);
  CHECK(sampler_init(&h, 1 << 20, 10, 10, 1, 0) != TSR_OK && h == NULL);

  /* a real init: a device error without a GPU, else a handle that is freed */
  int rc = sampler_init(&h, 0, 64, 4096, 4, 7);
  if (rc == TSR_OK) {
    CHECK(h != NULL);
    CHECK(sampler_destroy(h) == TSR_OK);
  } else {
    CHECK(rc == TSR_EDEVICE || rc == TSR_ENOMEM);
    CHECK(h == NULL);
  }
  CHECK(sampler_destroy(NULL) == TSR_OK);

  /* every call with a NULL handle */
  const tsr_params ok = P(1.0, 0, 1.0, 0.0, TSR_JOINT);
  int32_t out[8] = {0};
  CHECK(sample_rows(NULL, NULL, TSR_F32, 1, 1, 1, &ok, 0, out, NULL, NULL) == TSR_EINVAL);
  CHECK(greedy_argmax(NULL, NULL, TSR_F32, 1, 1, 1, out, NULL, NULL) == TSR_EINVAL);
  CHECK(sample_rows_masked(NULL, NULL, TSR_F32, 1, 1, 1, NULL, 0, &ok, 0, out, NULL, NULL,
                           NULL) == TSR_EINVAL);
  tsr_constraints cs;
  memset(&cs, 0, sizeof cs);
  cs.repetition_penalty = 1.0;
  CHECK(sample_rows_ex(NULL, NULL, TSR_F32, 1, 1, 1, &cs, &ok, 0, out, NULL, NULL, NULL) ==
        TSR_EINVAL);
  CHECK(spec_verify(NULL, NULL, NULL, TSR_F32, NULL, 1, 1, 1, &ok, 0, out, out, NULL, NULL) ==
        TSR_EINVAL);
  CHECK(tree_verify(NULL, NULL, NULL, TSR_F32, NULL, NULL, 1, 2, 1, &ok, 0, out, out, out, NULL,
                    NULL) == TSR_EINVAL);
  CHECK(beam_step(NULL, NULL, TSR_F32, 1, 4, 1, 1, NULL, out, out, NULL, NULL, NULL) ==
        TSR_EINVAL);
  CHECK(sampler_philox(NULL, NULL, 1, NULL, NULL) == TSR_EINVAL);

  /* spec_verify_noalloc needs no handle: each argument class is rejected
   * before any device work (the pointers are never dereferenced on the host) */
  float dummy[64];
  int32_t toks[64], acc[8];
  const tsr_params bad[] = {P(-1.0, 0, 1.0, 0.0, 0), P(NAN, 0, 1.0, 0.0, 0),
                            P(INFINITY, 0, 1.0, 0.0, 0), P(1e-31, 0, 1.0, 0.0, 0),
                            P(1.0, 0, -0.1, 0.0, 0), P(1.0, 0, NAN, 0.0, 0),
                            P(1.0, 0, 1.0, INFINITY, 0), P(1.0, 0, 1.0, 0.0, 7)};
  for (unsigned i = 0; i < sizeof bad / sizeof bad[0]; ++i)
    CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_F32, toks, 2, 2, 8, &bad[i], 0, toks, acc,
                              NULL, NULL) == TSR_EINVAL);
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_F32, toks, 2, 2, 8, NULL, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* no params */
  CHECK(spec_verify_noalloc(0, 1, NULL, dummy, TSR_F32, toks, 2, 2, 8, &ok, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* no target */
  CHECK(spec_verify_noalloc(0, 1, dummy, NULL, TSR_F32, toks, 2, 2, 8, &ok, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* T > 0 needs q */
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, 5, toks, 2, 2, 8, &ok, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* dtype */
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_F32, toks, 2, 0, 8, &ok, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* K < 1 */
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_F32, toks, 2, 33, 8, &ok, 0, toks, acc, NULL,
                            NULL) == TSR_EINVAL);                       /* K > 32 */
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_F32, toks, 16385, 1, 8, &ok, 0, toks, acc,
                            NULL, NULL) == TSR_EINVAL);                 /* rows */
  CHECK(spec_verify_noalloc(0, 1, (char*)dummy + 2, dummy, TSR_F32, toks, 2, 2, 8, &ok, 0, toks,
                            acc, NULL, NULL) == TSR_EINVAL);            /* misaligned */
  CHECK(spec_verify_noalloc(0, 1, dummy, dummy, TSR_BF16, toks, 2, 2, 65537, &ok, 0, toks, acc,
                            NULL, NULL) == TSR_EUNSUPPORTED);           /* wider than its path */
  printf("abi_driver: ok\n");
  return 0;
}
