/*
 * A C program that uses libfp8kv.so through include/fp8kv.h alone: the ABI
 * version, status strings, the kernel-family choice, the workspace size and
 * the documented argument errors.  Every call here returns before anything
 * is launched, so no GPU is needed; the device addresses are fake (aligned,
 * never dereferenced).  Exit status 0 means every check held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8kv.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      return 1;                                                            \
    }                                                                      \
  } while (0)

static int decode(void* ws, size_t ws_bytes, int32_t batch, int32_t hq, int32_t hkv, float k_scale,
                  const uint32_t* tags, const uint32_t* expected) {
  void* dev = (void*)(uintptr_t)0x100000; /* 256-byte aligned */
  return paged_decode_attn((const uint16_t*)dev, dev, dev, FP8KV_KV_FP8_E4M3, k_scale, 1.0f,
                           (const int32_t*)dev, 513, (const int32_t*)dev, tags, expected,
                           (uint16_t*)dev, (uint8_t*)dev, ws, ws_bytes, batch, hq, hkv, 128, 64, 16416,
                           0.08838835f, 0, NULL);
}

int main(void) {
  void* dev = (void*)(uintptr_t)0x100000;
  CHECK(fp8kv_abi_version() == FP8KV_ABI_VERSION);
  CHECK(fp8kv_status_string(FP8KV_OK) != NULL);
  CHECK(strlen(fp8kv_status_string(FP8KV_ERR_WORKSPACE)) > 0);

  /* kernel family: matrix cores for groups of 5..16, VALU below, -1 when invalid */
  CHECK(paged_decode_attn_path(64, 8) == 1);
  CHECK(paged_decode_attn_path(8, 2) == 0);
  CHECK(paged_decode_attn_path(0, 8) == -1);

  /* workspace: deterministic, grows with the batch */
  const size_t ws = paged_decode_attn_workspace_size(32, 64, 8, 128, 64, 513, 0);
  CHECK(ws > 0);
  CHECK(paged_decode_attn_workspace_size(32, 64, 8, 128, 64, 513, 0) == ws);
  CHECK(paged_decode_attn_workspace_size(64, 64, 8, 128, 64, 513, 0) > ws);

  /* argument errors, each with every other argument valid */
  CHECK(decode(dev, ws, 0, 64, 8, 1.0f, NULL, NULL) == FP8KV_ERR_SHAPE);          /* batch 0 */
  CHECK(decode(dev, ws, 32, 63, 8, 1.0f, NULL, NULL) == FP8KV_ERR_SHAPE);         /* heads do not divide */
  CHECK(decode(dev, ws, 32, 64, 2, 1.0f, NULL, NULL) == FP8KV_ERR_UNSUPPORTED);   /* group 32 > 16 */
  CHECK(decode(dev, ws, 32, 64, 8, NAN, NULL, NULL) == FP8KV_ERR_SCALE);          /* scale not finite */
  CHECK(decode(dev, ws, 32, 64, 8, 1.0f, (const uint32_t*)dev, NULL) == FP8KV_ERR_TAGS);
  CHECK(decode(NULL, ws, 32, 64, 8, 1.0f, NULL, NULL) == FP8KV_ERR_NULL);         /* no workspace */
  CHECK(decode(dev, ws - 1, 32, 64, 8, 1.0f, NULL, NULL) == FP8KV_ERR_WORKSPACE); /* one byte short */

  /* a whole step: the decode's errors first, then the append's (its rows' pointers only when n_rows > 0) */
  CHECK(paged_decode_step(NULL, NULL, NULL, NULL, 0, (const uint16_t*)dev, dev, dev, FP8KV_KV_FP8_E4M3, 1.0f, 1.0f,
                          (const int32_t*)dev, 513, (const int32_t*)dev, NULL, NULL, (uint16_t*)dev, (uint8_t*)dev,
                          dev, ws - 1, 32, 64, 8, 128, 64, 16416, 0.08838835f, 0, NULL, NULL, NULL) ==
        FP8KV_ERR_WORKSPACE);
  CHECK(paged_decode_step(NULL, NULL, NULL, NULL, 32, (const uint16_t*)dev, dev, dev, FP8KV_KV_FP8_E4M3, 1.0f,
                          1.0f, (const int32_t*)dev, 513, (const int32_t*)dev, NULL, NULL, (uint16_t*)dev,
                          (uint8_t*)dev, dev, ws, 32, 64, 8, 128, 64, 16416, 0.08838835f, 0, NULL, NULL,
                          NULL) == FP8KV_ERR_NULL);

  /* append: nothing to do is valid (and launches nothing); a head count past the limit is not */
  CHECK(kv_quant_append(NULL, NULL, NULL, NULL, NULL, 1, 1, 1.0f, 1.0f, NULL, NULL, 1, 0, 8, 128, 64,
                        FP8KV_KV_FP8_E4M3, NULL) == FP8KV_OK);
  CHECK(kv_quant_append((const uint16_t*)dev, (const uint16_t*)dev, (const int32_t*)dev, (const int32_t*)dev,
                        (const int32_t*)dev, 1, 1, 1.0f, 1.0f, dev, dev, 1, 1, 65536, 128, 64,
                        FP8KV_KV_FP8_E4M3, NULL) == FP8KV_ERR_SHAPE);

  /* INT4 GEMV: at most FP8KV_INT4_MAX_M activation rows, K a multiple of the group */
  CHECK(int4_gemv((const uint16_t*)dev, (const uint32_t*)dev, (const uint16_t*)dev, (uint16_t*)dev,
                  FP8KV_INT4_MAX_M + 1, 128, 128, NULL) == FP8KV_ERR_SHAPE);
  CHECK(int4_gemv((const uint16_t*)dev, (const uint32_t*)dev, (const uint16_t*)dev, (uint16_t*)dev, 1, 128,
                  FP8KV_INT4_GROUP + 1, NULL) == FP8KV_ERR_SHAPE);

  printf("C ABI checks passed\n");
  return 0;
}
