/* A plain C99 caller of the C ABI: it includes include/hattn.h, links libhattn.so and
 * calls the entry points that need no GPU (presets, sizes, the schedule, argument
 * validation, status strings).  Exits 0 and prints "ok" when every check holds, else
 * prints the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "hattn.h"

#define CHECK(cond)                                       \
  do {                                                    \
    if (!(cond)) {                                        \
      printf("failed: %s (line %d)\n", #cond, __LINE__);  \
      return 1;                                           \
    }                                                     \
  } while (0)

int main(void) {
  hattn_layer_cfg s, f;
  int dummy = 0;
  CHECK(hattn_cfg_preset(HATTN_SLIDING, &s) == HATTN_OK);
  CHECK(hattn_cfg_preset(HATTN_FULL, &f) == HATTN_OK);
  CHECK(hattn_cfg_preset(HATTN_FULL, NULL) == HATTN_ERR_NULL);
  CHECK(s.kind == HATTN_SLIDING && s.n_q_heads == 16 && s.n_kv_heads == 4 && s.head_dim == 256);
  CHECK(s.window == 512 && s.rot_dim == 256 && s.rope_theta == 1e4 && s.softmax_scale == 1.0f / 16);
  CHECK(f.window == 0 && f.rot_dim == 64 && f.rope_theta == 5e6 && f.reserved == 0);

  /* Sliding decode workspace: the ring split's partials (8 splits up to B = 8, 4 above;
   * 4 heads x (256 + 2) floats each) and one counter per (sequence, KV head). */
  CHECK(hattn_decode_workspace_bytes(&s, 1, 512) == (size_t)1 * 4 * 8 * 4 * 258 * 4 + 1 * 4 * 4);
  CHECK(hattn_decode_workspace_bytes(&s, 32, 512) == (size_t)32 * 4 * 4 * 4 * 258 * 4 + 32 * 4 * 4);
  CHECK(hattn_decode_workspace_bytes(&s, 32, 513) == 0);
  CHECK(hattn_decode_workspace_bytes(&f, 32, 131136) > 0);

  /* The layer schedule: every fourth layer (l % 4 == 3) is full-causal. */
  for (int l = 0; l < 36; ++l)
    CHECK(hattn_model_layer_kind(l) == (l % 4 == 3 ? HATTN_FULL : HATTN_SLIDING));
  {
    size_t per[36], total = 0;
    CHECK(hattn_model_kv_bytes(36, 1, 1048576, per, &total) == HATTN_OK);
    /* 9 full layers x 2^20 keys and 27 rings x 512 slots, 4096 bytes of K and V each. */
    CHECK(total == (size_t)4096 * (9 * 1048576 + 27 * 512));
    CHECK(per[3] == (size_t)4096 * 1048576 && per[0] == (size_t)4096 * 512);
  }

  /* Argument validation happens before anything touches a device. */
  CHECK(hattn_decode(&f, NULL, &dummy, &dummy, 4096, &dummy, 1, &dummy, &dummy, NULL, &dummy,
                     1 << 20, 0, NULL) == HATTN_ERR_NULL);
  CHECK(hattn_decode(&f, &dummy, &dummy, &dummy, 4096, &dummy, 0, &dummy, &dummy, NULL, NULL, 0,
                     0, NULL) == HATTN_OK);  /* B = 0: nothing to do */
  CHECK(hattn_prefill(NULL, &dummy, &dummy, &dummy, 8, &dummy, 1, 1, &dummy, &dummy, NULL, 0,
                      NULL) == HATTN_ERR_NULL);

  for (int st = 0; st <= HATTN_ERR_SCRATCH; ++st) {
    const char* msg = hattn_status_string((hattn_status)st);
    CHECK(msg != NULL && strlen(msg) > 0);
  }
  printf("ok\n");
  return 0;
}
