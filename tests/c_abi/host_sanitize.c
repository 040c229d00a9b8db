/* Host-side checks of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only).  Every compute call here is built
 * to fail argument validation, so nothing reaches the device: the launch
 * functions of this build abort if called.  The pointers are fake,
 * never-dereferenced device addresses.  Exit status 0 when every call
 * returned the expected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                              \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

static void* P(int i) { return (void*)(uintptr_t)(0x7F0000000000ull + (uint64_t)i * (64ull << 20)); }

int main(void) {
  const int D = 128;
  kda_fused_opts o;
  memset(&o, 0, sizeof o);
  o.l2_eps = 1e-6f;
  o.rms_eps = 1e-6f;
  /* status strings and the precondition word */
  for (int s = 0; s <= 7; ++s)
    if (!kda_status_string((kda_status)s) || !kda_status_string((kda_status)s)[0]) ++failures;
  EXPECT(kda_last_precondition_flags(), 0);
  /* workspace queries, including sizes that must be refused */
  if (kda_chunk_fwd_workspace_bytes(1, 8192, 96, D, D, KDA_DTYPE_BF16, NULL) == 0) ++failures;
  if (kda_chunk_fwd_workspace_bytes(64, 1000000, 96, D, D, KDA_DTYPE_BF16, NULL) == 0) ++failures;
  EXPECT(kda_chunk_fwd_workspace_bytes(0, 10, 2, D, D, KDA_DTYPE_BF16, NULL), 0);
  EXPECT(kda_chunk_fwd_workspace_bytes(1, -5, 2, D, D, KDA_DTYPE_BF16, NULL), 0);
  EXPECT(kda_chunk_fwd_workspace_bytes(1, 10, 2, 64, D, KDA_DTYPE_BF16, NULL), 0);
  EXPECT(kda_chunk_fwd_workspace_bytes(1, 10, 2, D, D, (kda_dtype)7, NULL), 0);
  EXPECT(kda_chunk_fwd_workspace_bytes(0x7FFFFFFF, 10, 0x7FFFFFFF, D, D, KDA_DTYPE_BF16, NULL), 0);
  o.factor_budget_mib = -1;
  EXPECT(kda_chunk_fwd_workspace_bytes(1, 10, 2, D, D, KDA_DTYPE_BF16, &o), 0);
  o.factor_budget_mib = 64;
  if (kda_chunk_fwd_workspace_bytes(1, 8192, 96, D, D, KDA_DTYPE_BF16, &o) == 0) ++failures;
  o.factor_budget_mib = 0;
  o.segment_tokens = 100;
  EXPECT(kda_chunk_fwd_workspace_bytes(1, 1000, 2, D, D, KDA_DTYPE_BF16, &o), 0);
  o.segment_tokens = 64;
  if (kda_chunk_fwd_workspace_bytes(1, 1000, 2, D, D, KDA_DTYPE_BF16, &o) == 0) ++failures;
  o.segment_tokens = 0;
  if (kda_chunk_bwd_workspace_bytes(3, 1000, 2, D, D, KDA_DTYPE_F32) == 0) ++failures;
  EXPECT(kda_chunk_bwd_workspace_bytes(1, 10, 2, 64, D, KDA_DTYPE_BF16), 0);
  EXPECT(kda_chunk_bwd_workspace_bytes(0x7FFFFFFF, 1, 0x7FFFFFFF, D, D, KDA_DTYPE_BF16), 0);

  /* kda_chunk_fwd: every call fails validation */
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, 64, D, KDA_DTYPE_BF16, NULL, P(5), P(6),
                       P(8), 32u << 20, 0), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 2, 10, 2, D, D, KDA_DTYPE_BF16, NULL, P(5), P(6),
                       P(8), 32u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, NULL, P(0), P(6),
                       P(8), 32u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, NULL, P(5), P(6),
                       NULL, 0, 0), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), P(0), NULL, 1, 256, 2, D, D, KDA_DTYPE_BF16, NULL, P(5), P(0),
                       P(8), 32u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd((char*)P(0) + 8, P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, NULL,
                       P(5), P(6), P(8), 32u << 20, 0), KDA_ERR_INVALID_ARG);
  o.l2_eps = -1.f;
  EXPECT(kda_chunk_fwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, &o, P(5), P(6),
                       P(8), 32u << 20, 0), KDA_ERR_INVALID_ARG);
  o.l2_eps = 1e-6f;
  /* the no-allocation prefill: sizes past its scratch array, bad sizes */
  EXPECT(kda_chunk_fwd_noalloc(P(0), P(1), P(2), P(3), P(4), NULL, P(7), 64, 256, 96, D, D, KDA_DTYPE_BF16, NULL,
                               P(5), NULL, 0), KDA_ERR_SCRATCH);
  EXPECT(kda_chunk_fwd_noalloc(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, -1, 2, D, D, KDA_DTYPE_BF16, NULL,
                               P(5), NULL, 0), KDA_ERR_INVALID_ARG);
  /* backward */
  EXPECT(kda_chunk_bwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, P(5), NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, P(0),
                       P(7), P(8), P(9), P(10), NULL, P(11), 64u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, P(5), NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, P(6),
                       P(7), P(8), P(9), P(10), NULL, NULL, 0, 0), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_bwd(P(0), P(1), P(2), P(3), P(4), NULL, NULL, NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, P(6),
                       P(7), P(8), P(9), P(10), NULL, P(11), 64u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd_saved(P(0), P(1), P(2), P(3), P(4), NULL, NULL, P(5), NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16,
                             P(0), P(7), P(8), P(9), P(10), NULL, P(11), 64u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd_saved(P(0), P(1), P(2), P(3), P(4), NULL, NULL, P(5), NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16,
                             P(6), P(7), P(8), P(9), P(10), NULL, NULL, 0, 0), KDA_ERR_WORKSPACE);
  /* the training forward */
  EXPECT(kda_chunk_fwd_save(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, P(1), NULL,
                            P(11), 64u << 20, 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_fwd_save(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, D, KDA_DTYPE_BF16, P(6), NULL,
                            NULL, 0, 0), KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_save(P(0), P(1), P(2), P(3), P(4), NULL, NULL, 1, 10, 2, D, 64, KDA_DTYPE_BF16, P(6), NULL,
                            P(11), 64u << 20, 0), KDA_ERR_UNSUPPORTED);
  /* decode and replay */
  EXPECT(kda_decode_step(P(0), P(1), P(2), P(3), P(4), P(5), 2, 2, D, D, KDA_DTYPE_BF16, P(1), 0),
         KDA_ERR_INVALID_ARG);
  EXPECT(kda_decode_step(P(0), P(1), P(2), P(3), P(4), P(5), 2, 2, D, 64, KDA_DTYPE_BF16, P(6), 0),
         KDA_ERR_UNSUPPORTED);
  EXPECT(kda_decode_replay(P(0), P(1), P(1), P(2), P(3), P(4), P(5), P(7), 2, 4, 2, D, D, KDA_DTYPE_BF16, NULL, NULL,
                           NULL, P(6), 0), KDA_ERR_INVALID_ARG);
  EXPECT(kda_decode_replay(P(0), P(0), P(1), P(2), P(3), P(4), P(5), P(7), 2, 17, 2, D, D, KDA_DTYPE_BF16, NULL,
                           NULL, NULL, P(6), 0), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_decode_replay(P(0), NULL, P(1), P(2), P(3), P(4), P(5), P(7), 2, 4, 2, D, D, KDA_DTYPE_BF16, NULL, NULL,
                           NULL, NULL, 0), KDA_OK);
  if (failures) fprintf(stderr, "%d failed check(s)\n", failures);
  else printf("host sanitizer checks passed\n");
  return failures ? 1 : 0;
}
