/* A plain C client of the library's C ABI (no Python, no GPU).  It includes
 * include/sv.h, links libsv.so and exercises the host-side entry points:
 * workspace sizing, status strings, tree-builder sizing and argument checks
 * that return before any launch.  Exit status 0 when every check holds; the
 * first failing check is printed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sv.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond, \
              sv_last_error());                                            \
      return 1;                                                            \
    }                                                                      \
  } while (0)

int main(void) {
  /* fake, never dereferenced device addresses: every call below fails or
     returns before launching */
  void* fake = (void*)(uintptr_t)0x100000;
  const int32_t* fi = (const int32_t*)fake;

  sv_tree t;
  memset(&t, 0, sizeof t);
  t.B = 32;
  t.T_max = 65;
  t.parent = fi;
  t.num_nodes = fi;
  t.tokens = fi;

  sv_attn_args a;
  memset(&a, 0, sizeof a);
  a.Hq = 64; a.Hkv = 8; a.D = 128; a.L_max = 8192 + 128; a.dtype = SV_BF16;
  a.q = a.k_new = a.v_new = a.k_cache = a.v_cache = fake;
  a.prefix_len = fi; a.out = fake;

  sv_accept_args c;
  memset(&c, 0, sizeof c);
  c.V = 128256; c.logit_dtype = SV_BF16; c.sibling_mode = SV_SIB_WITHOUT_REPLACEMENT;
  c.target_logits = fake; c.q_probs = (const float*)fake; c.temperature = (const float*)fake;
  c.u_accept = (const float*)fake; c.u_sample = (const float*)fake;
  c.out_tokens = (int32_t*)fake; c.out_nodes = (int32_t*)fake; c.out_count = (int32_t*)fake;

  /* sizing: the step's workspace covers both calls */
  size_t wa = sv_workspace_bytes(&t, &a, NULL);
  size_t wc = sv_workspace_bytes(&t, NULL, &c);
  size_t wb = sv_workspace_bytes(&t, &a, &c);
  CHECK(wc > 0);
  CHECK(wb >= wa && wb >= wc);
  CHECK(wb % 256 == 0);

  /* host-visible errors come back before any launch */
  sv_attn_args bad = a;
  bad.D = 96;
  CHECK(sv_workspace_bytes(&t, &bad, NULL) == 0);
  CHECK(strlen(sv_last_error()) > 0);
  CHECK(sv_tree_attn(&t, (const uint64_t*)fake, fi, &bad, fake, wb, NULL) == SV_E_UNSUPPORTED);
  bad = a;
  bad.Hq = 60;
  CHECK(sv_tree_attn(&t, (const uint64_t*)fake, fi, &bad, fake, wb, NULL) == SV_E_SHAPE);
  CHECK(sv_spec_accept(&t, (int32_t*)fake, &c, NULL, wb, NULL) == SV_E_WORKSPACE);
  CHECK(sv_tree_mask_build(NULL, NULL, NULL, NULL, NULL) == SV_E_NULL);
  sv_tree big = t;
  big.T_max = 257;
  CHECK(sv_tree_mask_build(&big, (uint64_t*)fake, (int32_t*)fake, (int32_t*)fake, NULL) == SV_E_UNSUPPORTED);

  /* every status code has a description */
  for (int s = -6; s <= 10; ++s) CHECK(strcmp(sv_status_string((sv_status)s), "unknown status") != 0);
  CHECK(strcmp(sv_status_string((sv_status)99), "unknown status") == 0);

  /* the tree builder's state size, and its limits */
  sv_eagle2_cfg e = {32, 128256, 8, 6, 64};
  size_t sb = sv_eagle2_state_bytes(&e);
  CHECK(sb > 0 && sb % 256 == 0);
  sv_eagle2_cfg eb = e;
  eb.k = 17;
  CHECK(sv_eagle2_state_bytes(&eb) == 0);
  CHECK(sv_eagle2_expand(&e, fake, sb, 6, (const float*)fake, NULL, NULL, NULL) == SV_E_SHAPE);
  CHECK(sv_eagle2_begin(&e, fake, sb - 1, fi, NULL) == SV_E_WORKSPACE);

  /* an empty batch needs nothing and launches nothing */
  sv_tree empty = t;
  empty.B = 0;
  empty.parent = empty.num_nodes = empty.tokens = NULL;
  CHECK(sv_tree_mask_build(&empty, NULL, NULL, NULL, NULL) == SV_OK);

  printf("C ABI host checks passed: workspace %zu bytes, tree-builder state %zu bytes\n", wb, sb);
  return 0;
}
