/* The library's C ABI used from plain C: the header compiles as C99 and the
 * host-side calls (version, workspace size queries, argument validation)
 * behave as the header states.  No GPU work is launched. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ring_attn.h"

static int failures = 0;

static void check(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s (last error: %s)\n", what, ra_last_error());
    ++failures;
  }
}

int main(void) {
  const char* v = ra_version();
  check(v != NULL && strlen(v) > 0, "ra_version returns a string");

  /* workspace queries: a valid forward ring needs a workspace, P = 1 needs none */
  size_t nb = ring_attn_fwd_ws_bytes(1, 32, 32, 32768, 128, 8, RA_BF16);
  check(nb > 0 && nb != SIZE_MAX, "fwd workspace of the 32k prefill");
  check(ring_attn_fwd_ws_bytes(1, 32, 32, 32768, 128, 1, RA_BF16) == 0, "no workspace with one host");
  check(ring_attn_fwd_ws_bytes(1, 32, 32, 32769, 128, 8, RA_BF16) == SIZE_MAX, "N % P != 0 is refused");
  check(strstr(ra_last_error(), "multiple of P") != NULL, "the refusal says why");
  check(ring_attn_bwd_share_ws_bytes(1, 4, 4, 1048576, 128, 8, RA_BF16) != SIZE_MAX, "backward share workspace");
  check(ring_attn_decode_ws_bytes(16, 32, 8, 262144, 128, 8) != SIZE_MAX, "decode workspace");

  /* argument checks return before anything is launched */
  check(ring_attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 2, 1, 64, 64, 4, 1, RA_CONTIGUOUS, 0.125f, RA_BF16, NULL,
                      NULL, 0) == RA_EINVAL,
        "null tensors are refused");
  ra_mask_desc md;
  memset(&md, 0, sizeof md);
  md.B = 1; md.H = 2; md.Hkv = 1; md.d = 64; md.Lq = 16; md.Lkv = 16; md.scale = 0.125f;
  md.dtype = RA_BF16; md.causal = 1; md.layout = RA_CONTIGUOUS; md.P = 4; md.q_rank = 5; md.kv_rank = 0;
  ra_kv_block kv = {(const void*)256, (const void*)512};
  check(ring_attn_step((const void*)768, kv, (float*)1024, (float*)1280, (float*)1536, &md, NULL) == RA_EINVAL,
        "a rank past the ring is refused");
  check(ring_attn_bwd_step((const void*)768, (const void*)1024, (const float*)1280, kv, (float*)1536,
                           (float*)1792, (float*)2048, &md, NULL) == RA_EINVAL,
        "the backward step refuses it too");
  check(lse_merge(NULL, NULL, NULL, NULL, 0, 64, NULL) == RA_OK, "merging zero rows is a no-op");

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
