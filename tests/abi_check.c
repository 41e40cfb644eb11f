/* The C ABI from plain C (C99): include the public header, link the library,
 * and check the host-side contract of every entry point - sizes, argument
 * validation before any launch, status strings. Nothing here reaches a GPU:
 * every call either returns a validation error or does nothing (zero
 * tokens), so it runs on a machine without one. Prints the failures and
 * exits with their count. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flint_attn.h"

static int failures = 0, checks = 0;

#define CHECK(cond)                                                         \
  do {                                                                      \
    ++checks;                                                               \
    if (!(cond)) {                                                          \
      ++failures;                                                           \
      fprintf(stderr, "abi_check: line %d: %s\n", __LINE__, #cond);         \
    }                                                                       \
  } while (0)

/* an aligned, non-NULL address that no call dereferences */
#define FAKE ((void*)(uintptr_t)(1u << 20))
#define FAKE_AT(off) ((void*)((uintptr_t)(1u << 20) + (off)))

static int fwd(void* q, int32_t T, int32_t heads, int32_t window, size_t ws_bytes) {
  return flint_attn_fwd(q, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, T, heads, 4, 128,
                        window, 1, 1.0e6f, 1.0e-6f, FAKE, ws_bytes, FAKE, NULL);
}

int main(void) {
  /* sizes */
  const size_t ws = flint_attn_workspace_bytes(8192, 1, 8192, 4, 128);
  CHECK(ws > 0);
  CHECK(flint_attn_workspace_bytes(-1, 1, 8192, 4, 128) == 0);
  CHECK(flint_attn_workspace_bytes(8192, 1, 8192, 8, 128) == 0);
  CHECK(flint_attn_workspace_bytes(16384, 1, 16384, 4, 128) > ws);
  CHECK(flint_attn_f16_workspace_bytes(8192, 1, 8192, 4, 128) >= ws + (size_t)8192 * 32 * 128 * 2);
  CHECK(flint_attn_bwd_workspace_bytes(8192, 1, 8192, 4, 128) > 0);
  CHECK(flint_attn_decode_workspace_bytes(64, 8192) > 0);
  CHECK(flint_attn_bshd_plan_bytes(2, 4) >= 4 * (8 + 6 * 8));
  CHECK(flint_attn_bshd_plan_bytes(-1, 4) == 0);
  CHECK(flint_attn_workspace_bytes(FLINT_MAX_SEQLEN, 1, FLINT_MAX_SEQLEN, 4, 128) > 0);
  CHECK(flint_attn_workspace_bytes(FLINT_MAX_SEQLEN, 1, FLINT_MAX_SEQLEN + 1, 4, 128) == 0);
  CHECK(flint_attn_bwd_workspace_bytes(64, 1, FLINT_MAX_SEQLEN + 1, 4, 128) == 0);

  /* the forward on the static scratch: host checks before any launch */
  CHECK(flint_attn_fwd_static(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 1 << 20, 1 << 20,
                              32, 4, 128, 0, 0, 1.0e6f, 1.0e-6f, FAKE, NULL) == FLINT_ERR_TOO_LARGE);
  CHECK(flint_attn_fwd_static(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 16, 4,
                              128, 0, 0, 1.0e6f, 1.0e-6f, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);
  CHECK(flint_attn_fwd_static(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, -1, 32, 4,
                              128, 0, 0, 1.0e6f, 1.0e-6f, FAKE, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_fwd_static(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 0, 0, 32, 4,
                              128, 0, 0, 1.0e6f, 1.0e-6f, NULL, NULL) == FLINT_OK);

  /* which attention kernel a forward launches: a host-side query */
  CHECK(flint_attn_fwd_kernel(0, 1) == 0);
  CHECK(flint_attn_fwd_kernel(-1, 1) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_fwd_kernel(64, 0) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_fwd_kernel(64, 1) == FLINT_KERNEL_SPLIT);
  CHECK(flint_attn_fwd_kernel(8192, 1) == FLINT_KERNEL_WIDE);

  /* forward: validation before any launch */
  CHECK(fwd(NULL, 64, 32, 513, ws) == FLINT_ERR_NULL);
  CHECK(fwd(FAKE, 64, 16, 513, ws) == FLINT_ERR_UNSUPPORTED);
  CHECK(fwd(FAKE, 64, 32, -1, ws) == FLINT_ERR_VALUE);
  CHECK(fwd(FAKE, -1, 32, 513, ws) == FLINT_ERR_SHAPE);
  CHECK(fwd(FAKE_AT(8), 64, 32, 513, ws) == FLINT_ERR_ALIGN);
  CHECK(fwd(FAKE, 64, 32, 513, 16) == FLINT_ERR_WORKSPACE);
  CHECK(fwd(NULL, 0, 32, 513, 0) == FLINT_OK); /* zero tokens: nothing to do */
  CHECK(flint_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, FLINT_MAX_SEQLEN + 1, 64, 32,
                       4, 128, 0, 0, 1.0e6f, 1.0e-6f, FAKE, ws, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);
  CHECK(flint_attn_fwd_phases(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 32, 4,
                              128, 513, 1, 1.0e6f, 1.0e-6f, FAKE, ws, FAKE, NULL, 0) == FLINT_ERR_VALUE);
  CHECK(flint_attn_fwd_phases(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 32, 4,
                              128, 513, 1, 1.0e6f, 1.0e-6f, FAKE, ws, FAKE, NULL,
                              FLINT_PHASE_ALL + 1) == FLINT_ERR_VALUE);
  CHECK(flint_attn_fwd_lse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 32, 4,
                           128, 513, 1, 1.0e6f, 1.0e-6f, FAKE, ws, FAKE, NULL, NULL) == FLINT_ERR_NULL);
  CHECK(flint_attn_fwd_f16(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 32, 8,
                           128, 513, 1, 1.0e6f, 1.0e-6f, FAKE, ws, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);
  CHECK(flint_attn_fwd_f16(NULL, NULL, NULL, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 0, 0, 32, 4, 128,
                           513, 1, 1.0e6f, 1.0e-6f, NULL, 0, NULL, NULL) == FLINT_OK);

  /* backward */
  CHECK(flint_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, -1, 32, 4, 128,
                       513, 1, 1.0e6f, 1.0e-6f, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                       FAKE, FAKE, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, 64, 64, 16, 4, 128,
                       513, 1, 1.0e6f, 1.0e-6f, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                       FAKE, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);
  CHECK(flint_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, 1, FLINT_MAX_SEQLEN + 1, 64, 32,
                       4, 128, 0, 0, 1.0e6f, 1.0e-6f, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                       FAKE, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);

  /* decode */
  CHECK(flint_attn_kv_append(FAKE, FAKE, FAKE, NULL, FAKE, 0, 1, FAKE, FAKE, 64, 4, 128, 0, 0,
                             1.0e6f, 1.0e-6f, FAKE, (size_t)1 << 20, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_kv_append(FAKE, FAKE, FAKE, NULL, FAKE, 2, 1, FAKE, FAKE, 33, 4, 128, 0, 0,
                             1.0e6f, 1.0e-6f, FAKE, (size_t)1 << 20, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 2, FAKE, FAKE, 64, 32, 4,
                          64, 0, 0, 1.0e6f, 1.0e-6f, FAKE, (size_t)1 << 20, FAKE,
                          NULL) == FLINT_ERR_UNSUPPORTED);

  /* projections */
  CHECK(flint_proj_qkv(FAKE, FAKE, FAKE, FAKE, 64, 2050, 32, 4, 128, FAKE, FAKE, FAKE, NULL) ==
        FLINT_ERR_UNSUPPORTED);
  CHECK(flint_proj_qkv(NULL, FAKE, FAKE, FAKE, 64, 2048, 32, 4, 128, FAKE, FAKE, FAKE, NULL) ==
        FLINT_ERR_NULL);
  CHECK(flint_proj_out(NULL, NULL, 0, 2048, 32, 128, NULL, NULL) == FLINT_OK);
  CHECK(flint_proj_out(FAKE, FAKE, 64, 2000, 32, 128, FAKE, NULL) == FLINT_ERR_UNSUPPORTED);

  /* BSHD documents and padding */
  CHECK(flint_attn_bshd_plan(FAKE, FAKE, -1, 4, FAKE, 1u << 20, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_bshd_plan(FAKE, FAKE, 2, 4, NULL, 1u << 20, NULL) == FLINT_ERR_NULL);
  CHECK(flint_attn_bshd_plan(FAKE, FAKE, 2, 4, FAKE, 8, NULL) == FLINT_ERR_WORKSPACE);
  CHECK(flint_attn_copy_rows(FAKE, FAKE, 4, 6, 0u, FAKE, NULL) == FLINT_ERR_SHAPE);
  CHECK(flint_attn_copy_rows(NULL, NULL, 0, 16, 0u, NULL, NULL) == FLINT_OK);

  /* helpers */
  CHECK(flint_attn_seqused_from_mask(FAKE, -1, 4, FAKE, FAKE, NULL) == FLINT_ERR_SHAPE);
  {
    int32_t flags = 0;
    CHECK(flint_attn_device_status(NULL, NULL, &flags) == FLINT_ERR_NULL);
  }
  {
    const char* seen[10];
    int st;
    for (st = 0; st >= -9; --st) {
      int j;
      const char* m = flint_attn_strerror(st);
      CHECK(m != NULL && strlen(m) > 0);
      for (j = 0; j < -st; ++j) CHECK(m == NULL || strcmp(m, seen[j]) != 0);
      seen[-st] = m ? m : "";
    }
  }

  printf("abi_check: %d checks, %d failed\n", checks, failures);
  return failures;
}
