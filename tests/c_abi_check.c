/* Plain-C client of include/int8mm.h: compiles as C99 against the header,
 * links libint8mm.so and drives every entry point through its host-side
 * argument checks (no call here reaches the GPU).  Prints one line per
 * check; the Python test compares them. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "int8mm.h"

#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
#define FAKE_WS ((void*)(uintptr_t)0x7F0000100000ull)

int main(void) {
  printf("ld %lld\n", (long long)int8_weight_ld(70));
  printf("bytes %lld\n", (long long)int8_weight_bytes(300, 70));
  printf("ws_ok %d\n", int8_matmul_workspace_size(40, 64, 40) > 0);
  printf("ws_bad %d\n", (int)int8_matmul_workspace_size(8, INT8MM_MAX_K + 1, 8));
  printf("prepare %d\n", int8_prepare_weight(NULL, 4, 8, FAKE, FAKE, NULL));
  printf("matmul %d\n", int8_matmul(FAKE, 4, 8, FAKE, FAKE, 4, NAN, FAKE, FAKE_WS, 1u << 30, NULL));
  printf("linear %d\n", int8_linear(FAKE, -1, 8, FAKE, FAKE, 4, NULL, 6.0f, FAKE, FAKE_WS,
                                    1u << 30, NULL));
  printf("stages %d\n", int8_matmul_stages(FAKE, 4, 8, FAKE, FAKE, 4, 6.0f, NULL, NULL, NULL, NULL,
                                           NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL));
  printf("profiled %d\n", int8_matmul_profiled(FAKE, 4, 8, FAKE, FAKE, 4, -1.0f, FAKE, FAKE_WS,
                                               1u << 30, NULL, NULL, NULL));
  printf("colmax %d\n", int8_column_absmax(FAKE, 4, 8, NULL, FAKE_WS, 1u << 30, NULL));
  {
    const float thr[2] = {6.0f, NAN};
    printf("counts %d\n", int8_outlier_counts(FAKE, 8, thr, 2, FAKE, NULL));
  }
  printf("empty %d\n", int8_matmul(NULL, 0, 8, NULL, FAKE, 4, 6.0f, NULL, NULL, 0, NULL));
  printf("strerror %s\n", int8mm_strerror(INT8MM_EWORKSPACE));
  printf("hiperr [%s]\n", int8mm_last_hip_error());
  return 0;
}
