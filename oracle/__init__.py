"""Float64 CPU oracle for the speculative-decoding target-verification step.

TEST INFRASTRUCTURE, NOT PRODUCT.  Only the test-suite, the package smoke
check and the CPU-baseline leg of the benchmark may import this package.  The
HIP library never calls it, and it shares no code, header, table or helper with
the HIP library.

It is written from the text of five web pages on speculative decoding, cited
in docstrings by page title and section:

  [LAT] "Speculative decoding" explainer, lattice-ai-eng.pages.dev
        (acceptance rule, worked example "blue"/"green", expected-tokens
        formula, reference implementation ``speculative_generate``)
  [PIG] "Speculative decoding" guide, herodthegreater.github.io/pigeon
        (sections "How it works", "Why the output is exactly p", "Speed",
        "When it breaks")
  [SSD] "Build a Speculative Decoding Engine to Cut LLM Latency by 3x",
        scalablesystem.dev (sections "The Accept/Reject Mechanism",
        "Speculation Depth Tuning and Tree Drafting", "Batch-Level
        Speculation", "Quality, Evaluation, and Guardrails")
  [KIS] "Speculative Decoding: How to Make an LLM 3x Faster by Letting a
        Smaller Model Guess Its Homework", kishorek.dev
  [ACI] "Speculative Decoding: Speeding Sequential Generation",
        aicomputerinstitute.com (sections "Why Generation Is Slow: A Roofline
        View", "Expected Tokens per Verification Round: Chain vs. Tree")

Counter-based randoms follow Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11), Philox4x64-10.

Modules:
  philox  -- Philox4x64-10 and the uniforms r, u of one verification row
  model   -- the synthetic target: RMSNorm / up / SiLU / down / residual MLP
             blocks, then the LM head
  rule    -- temperature, top-p, the ratio test, residual resampling, bonus,
             greedy branch, and the margin, slack and token band of every decision
  verify  -- spec_verify / spec_verify_from_logits over a batch
  tree    -- greedy verification of a draft tree: ancestor mask, depths,
             the walk down passing children
  control -- the gamma controller and the ragged repack of a batch
  attention -- the new rows' attention over a KV-cached prefix (chain or
             tree mask, grouped-query heads) and the KV commit

Parity status of each part (what pins it) is listed in the module docstrings.
"""

from .philox import philox4x64_10, row_uniforms, PURPOSE_VERIFY, PURPOSE_DRAFT
from .model import bf16_to_f64, as_f64, rmsnorm, silu, forward
from .rule import (warp_logits, warp_probs, nucleus_mask, accept_test,
                   inverse_cdf, cdf_band, verify_row, verify_row_greedy, MARGIN, TopP,
                   Decision)
from .verify import spec_verify, spec_verify_from_logits, VerifyResult
from . import attention, control, tree

__all__ = [
    "philox4x64_10", "row_uniforms", "PURPOSE_VERIFY", "PURPOSE_DRAFT",
    "bf16_to_f64", "as_f64", "rmsnorm", "silu", "forward",
    "warp_logits", "warp_probs", "nucleus_mask", "accept_test", "inverse_cdf",
    "cdf_band", "verify_row", "verify_row_greedy", "MARGIN", "TopP", "Decision",
    "spec_verify", "spec_verify_from_logits", "VerifyResult",
]
