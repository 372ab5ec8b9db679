"""fp64 CPU oracle of the CSA/HCA hybrid compressed attention layer.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never imports it, and
it imports nothing from the product path.
"""
from . import numerics, csa_oracle  # noqa: F401
