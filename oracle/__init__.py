"""CPU oracle for the row-L2 ops -- TEST INFRASTRUCTURE, not a product path.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it, and it never calls the
GPU library: the two share no code.

What is here:

* :mod:`oracle.bf16` -- round-to-nearest-even to bfloat16 from float64, and
  bf16/fp32 helpers.
* :mod:`oracle.rows` -- the three ops written out from their definitions in
  float64, rounding to bf16 only at the rounding points the pages name:
  ``l2_rows``, ``slerp_rows`` (TensorFold PR #1260, the commit that adds the two
  unit-sphere row kernels) and ``weight_rownorm_gain`` (DragonScale README,
  "What DragonScale changes", the W_eff formula).
* :mod:`oracle.brute` -- the same definitions in exact rational arithmetic
  (``fractions``) with 60-digit ``decimal`` square roots, for tiny rows; it
  pins the float64 oracle.
* :mod:`oracle.check` -- the tolerance checks: the 1-bf16-ulp / 2e-6 relative
  contract, and the strict admissible-set check (float64 value at the bf16
  rounding points, widened by the spread an fp32 run may have; TensorFold PR
  #1260, the kernel-contract check of the row kernels).

Every function is pinned by tests that do not restate it: closed forms, exact
brute force, invariants, and special cases that reduce to a library routine.
"""
