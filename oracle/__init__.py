"""CPU oracle for the fused int4 Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the build
entry point and the CPU-baseline leg of the benchmark may import or run this
package.  The GPU library never calls it and it never calls the GPU library;
the two share nothing but the seeded input generators in ``synth``.

``oracle.moe`` is the plain definition of the layer in float64 numpy.
``oracle.brute`` is an independent pure-Python float64 evaluation of the same
definition for tiny shapes (a dense formulation that runs every expert on
every token), used to pin ``oracle.moe``.

Parity status of each function is stated in its docstring; every function
here is pinned by tests/test_oracle.py (brute force, closed forms,
invariants, special cases that reduce to library routines, and the page's
printed sweep table for the routing statistics).
"""
from . import moe, brute  # noqa: F401
