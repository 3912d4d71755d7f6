"""CPU oracle for one GPT training step and the hashed n-gram tables.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the bench's CPU-baseline
leg may import this package.  The product path (the HIP library and its binding) never calls
it, and it shares no code with that path: plain numpy, float64 unless the caller asks for
float32 storage on the large workloads, written from the pages' definitions:

* model math: "$1000 tier nanochat run" discussion (nanochat #8), the GPT class a commenter
  posted there (apply_rotary_emb, norm, MLP, CausalSelfAttention, Block, GPT.forward,
  _precompute_rotary_embeddings), with the modded-nanogpt README's recipe (rotary, RMSNorm
  without affine parameters, ReLU^2) deciding the MLP activation;
* hashed tables and their sparse optimizer: the decoder-rtx posts by Chris McCormick
  (baseline 4: bigram tables added to x0 and to values, a frozen trigram table projected into
  values, an optimizer with no first moment and one magnitude per row, inlined in backward).

Every function here is pinned by tests under tests/ against something other than itself
(finite differences, closed forms, brute force, library routines).
"""
from . import model, tables  # noqa: F401
