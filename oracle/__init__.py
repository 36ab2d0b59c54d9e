"""CPU oracles (fp64): the Lightweight DC layer and MUDD layer mixing.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the CPU
baseline of the benchmark.  The product path never imports, calls or links it,
and it imports nothing from the product path.

Modules:
  ldc_oracle  blocked numpy float64 forward/backward (the oracle proper)
  bruteforce  dense torch float64 forward for pinning on tiny inputs
  mudd_oracle float64 multiway dynamic dense (MUDD) layer mixing, forward
              and backward

Parity status: every function here is pinned by CPU tests (brute force,
library special cases, closed forms, invariants, finite differences and a
hand-worked example); none is "parity unpinned".
"""
