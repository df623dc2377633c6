"""CPU reference (oracle) for the P-EAGLE parallel-drafting draft forward.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run this package. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

It is a plain, slow, float64 implementation written from the pages that describe
the method:

- P-EAGLE guide of the speculators documentation ("P-EAGLE"): sections
  "Architecture", "COD Sampling", "Inference Process", "Key Parameters".
- NeMo Automodel pull request 2376, "feat(speculative): add P-EAGLE
  parallel-drafting training for EAGLE-3 drafts": the PR description
  (implementation, checkpoint contract, parity section) and the commit message of
  the RoPE fix (gather cos/sin by position value).
- snxtyle/P_Eagle README: the packed-batch structure (``cu_seqlens``).

Modules:

- ``cod``       COD retained sets and the draft row layout.
- ``fuse``      fc projection of the aux hidden states, mask_hidden / ptd
                substitution at depths >= 1.
- ``rope``      rotary embedding gathered by position value.
- ``attention`` the multi-depth draft attention, with an explicit dense mask.
- ``decode``    the same attention at inference: K new rows per request at one base
                position over a KV cache (the flat [context, mask_1 ..] layout).
- ``layer``     the first draft layer's attention inputs: RMSNorm of the embedding and
                hidden halves, their concatenation, the QKV projection.
- ``verify``    greedy verification and the longest accepted prefix, the d2t variant and
                sampling acceptance.
- ``loss``      the depth-weighted cross-entropy of the draft rows and its gradient.

Inputs are bf16 bit patterns (uint16) or integer arrays; ``bf16`` converts the
bit patterns to float64 exactly.

Parity pins: every function is checked by ``tests/test_oracle_*.py`` against
closed forms, published test outputs, library routines, independent formulations
or brute force. The SplitMix64 hash is pinned by the generator's published
outputs for seed 0.
"""
from . import bf16, cod, fuse, rope, attention, decode, layer, verify, loss  # noqa: F401
