"""ORACLE — test infrastructure, not part of the product.

A plain, slow, float64 CPU implementation of the E(3)-equivariant edge convolution (forward,
exact vector-Jacobian product, per-irrep linear, bf16-rounded MLP operands, per-edge path
subsets) and of the node-local product ladder (oracle/ladder.py), written from the definitions,
used to check the HIP library.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
It shares no code, tables or constants with tensor_product_gnn_amd/ (which never imports it);
the two meet only through the seeded input generators in tensor_product_gnn_amd/workloads.py,
which hold none of the method's arithmetic.

Modules
  so3   real SH (Cartesian real form), Racah CG + real-basis transform, Wigner-D, path order.
  conv  radial basis, radial MLP, forward, backward (exact VJP), linear, forces.

Every function is pinned by tests/test_oracle_*.py against printed values (Table C1 of the
FlashCart page), closed forms, invariants, library routines (scipy) or brute force.
"""
from . import so3, conv  # noqa: F401
