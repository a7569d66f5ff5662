/* A plain C99 caller of libecco's C ABI: the header compiles as C, the
 * library links, and the host-side calls behave as declared.  No device is
 * touched: every device call below is refused by its argument checks, which
 * run before any HIP call. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ecco.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      return 1;                                                  \
    }                                                            \
  } while (0)

int main(void) {
  /* tables: 15 evenly spaced centroids (exact in FP16), every code 4 bits */
  float cent[ECCO_N_PATTERNS * ECCO_N_CENTROIDS];
  uint8_t len[ECCO_N_PATTERNS * ECCO_N_CODEBOOKS * ECCO_N_SYMBOLS];
  for (int p = 0; p < ECCO_N_PATTERNS; ++p)
    for (int k = 0; k < ECCO_N_CENTROIDS; ++k) cent[p * ECCO_N_CENTROIDS + k] = (float)(k - 7) / 8.0f;
  memset(len, 4, sizeof(len));
  const size_t tsize = ecco_tables_size();
  CHECK(tsize > 0);
  void* blob = malloc(tsize);
  CHECK(blob != NULL);
  CHECK(ecco_tables_build(cent, len, blob) == ECCO_OK);
  CHECK(ecco_tables_validate(blob) == ECCO_OK);
  float cent2[ECCO_N_PATTERNS * ECCO_N_CENTROIDS];
  uint8_t len2[ECCO_N_PATTERNS * ECCO_N_CODEBOOKS * ECCO_N_SYMBOLS];
  CHECK(ecco_tables_get(blob, cent2, len2) == ECCO_OK);
  CHECK(memcmp(cent, cent2, sizeof(cent)) == 0 && memcmp(len, len2, sizeof(len)) == 0);
  ((uint8_t*)blob)[0] ^= 1u;          /* a damaged header is refused */
  CHECK(ecco_tables_validate(blob) == ECCO_ETABLES);
  len[5] = 1;                         /* a code length below 2 */
  CHECK(ecco_tables_build(cent, len, blob) == ECCO_ETABLES);
  CHECK(ecco_tables_build(NULL, len, blob) == ECCO_EINVAL);

  /* per-tensor scale: amax / 448, and 1 for a zero or non-finite amax */
  CHECK(ecco_tensor_scale_from_amax(448.0f) == 1.0f);
  CHECK(ecco_tensor_scale_from_amax(0.0f) == 1.0f);
  CHECK(ecco_tensor_scale_from_amax(INFINITY) == 1.0f);

  /* device calls refused by their argument checks */
  void* fake = (void*)(uintptr_t)(1u << 20);
  CHECK(ecco_amax(NULL, 8, (float*)fake, NULL) == ECCO_EINVAL);
  CHECK(ecco_amax((const uint16_t*)fake, 0, (float*)fake, NULL) == ECCO_ESIZE);
  CHECK(ecco_amax_many(NULL, 1, NULL) == ECCO_EINVAL);
  ecco_amax_job_t aj = {(const uint16_t*)fake, 100, (float*)((char*)fake + 2)};
  CHECK(ecco_amax_many(&aj, 1, NULL) == ECCO_EALIGN);
  CHECK(ecco_amax_many(&aj, 0, NULL) == ECCO_ESIZE);
  CHECK(ecco_encode((const uint16_t*)fake, 1, 1, 128, 1, fake, 0.0f, fake, NULL, NULL) == ECCO_EINVAL);
  CHECK(ecco_decode((const char*)fake + 32, 1, 1, 1, 128, fake, 1.0f, (uint16_t*)fake, NULL) == ECCO_EALIGN);
  CHECK(ecco_decode_gemv(fake, fake, 1.0f, 4, 100, (const uint16_t*)fake, 1, (float*)fake, NULL) == ECCO_ESIZE);
  CHECK(ecco_decode_many(NULL, 1, NULL) == ECCO_EINVAL);
  CHECK(ecco_strerror(ECCO_EALIGN) != NULL && ecco_strerror(12345) != NULL);
  free(blob);
  printf("ok\n");
  return 0;
}
