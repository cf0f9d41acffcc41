"""Plain fp64 CPU oracle for batched speculative-decoding verification.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import, call or execute anything in this
package.  The product path (the HIP library and its Python binding) never
does, and this package imports nothing from it: the two share no code.

Modules
  rng     SplitMix64 uniforms from the published definition
  verify  greedy, sampling and tree-greedy verification in float64, with the
          per-decision margins used to classify disagreements
  serving rejected-draft masks for KV-cache trimming and a draft tree's parent
          array from its list of choices
"""
from . import rng, serving, verify  # noqa: F401
