"""fp64 CPU oracle for the gated delta-rule forward engine.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP kernels or their host
library (no common headers, helpers, tables or generators); the two sides
meet only in the seeded input arrays, which both read.

Sources ("the pages"):
  * Kaczmarz Linear Attention (reading notes): §1.1 gated delta rule,
    §2.1 tokenwise step and Algorithm 1, §2.2-2.4 projection / line search /
    proximal forms, §2.5 chunkwise form (Eqs. 6-9).
  * Preconditioned DeltaNet (reading notes): §2.2 exact ATK and
    Sherman-Morrison (Eqs. 3-5, Thm 3.1), §2.3 diagonal statistic and its
    counterexample, §2.4 trainable preconditioner (Eq. 9), §2.5 decay
    variants, §2.6 two-key chunk form (Eq. 6), §2.7 single-step spectrum.
  * Kalman Delta Networks (reading notes): §1.1 unified family, §2.2 exact
    Kalman filter (Eqs. 12-17), §2.4 diagonal KDN (Eqs. 23-30), §2.5
    information scaling, §2.6 Mobius scan (Eqs. 32-39).

Modules:
  recurrence  the plain token-by-token recurrence (the oracle proper)
  exact       the same recurrence and its chunkwise form in exact rationals
  chunkwise   the chunkwise (triangular-system) form in fp64, to pin the
              chunk equations against the recurrence
  kalman      textbook dense Kalman filter and ridge regression (pins)
  backward    gradients of the recurrence by a reverse sweep (training's
              backpropagation through the same recurrence)

Every function here has a pin in tests/ (worked examples printed on the
pages, closed forms, invariants, library special cases); none is
"parity unpinned".
"""
