"""CPU oracle for the Sparse Gated Attention hot path -- TEST INFRASTRUCTURE.

This package is the slow, obviously correct reference the HIP library is
checked against. It is test infrastructure, not part of the product: only
the tests, the package smoke check and the bench's CPU-baseline leg import
it. The product path never calls it and has no CPU fallback.

Modules:
  formats  exact decoders for fp32 / bf16 / E4M3FN / E8M0 / MXFP8 storage
  quant    encoders into those formats and the cache append (new tokens
           quantised into caller-chosen cache rows)
  sga      the four steps (index scores, top-k, sparse MLA, gate), the whole
           path, and a dense causal MLA reference
  kl       the indexer's KL loss over the sparse selection and its gradients
  case     glue that decodes a generated case (sga_inputs.SgaCase) for `sga`

Parity status: every function is pinned by tests that do not reuse it
(format code points and an independent library cast, brute force on tiny
inputs, closed forms, a library attention routine, invariants). The choice
of ReLU inside the indexer is a reading of the pages (they print no
formula): that single modelling choice is "parity unpinned" by the pages.
"""

from . import formats, kl, quant, sga  # noqa: F401
