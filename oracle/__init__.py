"""Float64 CPU oracle for the LoRA layer backward.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, calls or links it, and shares no code with it.

Sources (web pages, cited by title and section):
  [FFN]   Hesper API docs, "FFN Backward GPU Kernels" (Hesper.Training.FFNBackward)
  [ATTN]  Hesper API docs, "Attention Backward GPU Kernels"
          (Hesper.Training.AttentionBackward)
  [ENT]   entrenar source, train/transformer_trainer/wgpu_backward.rs
          (aprender-train 0.34.0): cpu_adamw, LayerActivations,
          backward_through_layers

Modules:
  backward  the backward pass, one function per step, formula-shaped
  forward   the float64 layer forward whose gradient the backward computes;
            it turns seeded draws into consistent saved activations and is the
            function the finite-difference pins differentiate
  fd        central finite differences
  bitlinear the packed ternary (BitLinear) weight format of the decode layer:
            packing, unpacking and the transposed product
  lmhead    the lm_head backward upstream of the stack: softmax cross-entropy
            over the vocabulary, grad_hidden, and AdamW on the lm_head weight

Every function is pinned by tests/test_oracle_*.py (finite differences,
closed forms, invariants, special cases reducing to library routines).  The
one thing no pin can fix is the choice among readings where the pages
disagree (which forward is differentiated); those readings are listed in the
module docstrings below and in the design notes.
"""
from . import backward, bitlinear, forward, fd, lmhead  # noqa: F401
