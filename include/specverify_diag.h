/*
 * specverify_diag.h -- diagnostics of libspecverify for tests (no GPU work).
 *
 * spec_diag_access_check walks, on the host, every kernel launch that
 * spec_verify would make for a pass of B sequences with gamma drafts over a
 * target of the given shape: the weight-registration layout (MFMA tiles),
 * the launch plan each GEMM would take (stacked, plain or wide MFMA, or the
 * vector-FMA path), and the workspace layout of spec_workspace_size.  For
 * every buffer a kernel reads or writes (weights, split activations,
 * residual, activations, logits, per-unit statistics, wide partial sums and
 * LDS tiles) it evaluates the kernel's own address formulas at the block,
 * wave, lane and k-step that reach the lowest and highest element, and
 * checks both against the buffer's extent.  No device memory is allocated
 * and nothing is launched, so it runs on machines without a GPU.
 *
 *   d, ffn, n_blocks, vocab, wdtype   the target's shape, as in
 *                                     spec_weights_desc
 *   mfma_min_rows, flags              the description's mfma_min_rows and
 *                                     SPEC_FLAG_* flags (bf16 only)
 *   B, gamma                          the pass
 *   shrink_bytes                      0 in use; > 0 checks against workspace
 *                                     buffers that many bytes short (a
 *                                     planted inconsistency, so a test can
 *                                     show that the check catches one)
 *   msg, msg_len                      host buffer (may be NULL) that receives
 *                                     the first out-of-range access, if any
 *   checks                            host out (may be NULL): ranges checked
 *
 * Returns SPEC_OK when every access lies inside its buffer, SPEC_EINVAL
 * when one does not (described in msg) or the arguments are invalid
 * (including shrink_bytes < 0),
 * SPEC_EDTYPE for an unknown wdtype.
 */
#ifndef SPECVERIFY_DIAG_H
#define SPECVERIFY_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

#ifdef __cplusplus
extern "C" {
#endif

spec_status spec_diag_access_check(int32_t d, int32_t ffn, int32_t n_blocks, int32_t vocab,
                                   int32_t wdtype, int32_t mfma_min_rows, uint32_t flags,
                                   int32_t B, int32_t gamma, int32_t shrink_bytes, char* msg,
                                   size_t msg_len, int64_t* checks);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_DIAG_H */
