"""The oracle: a plain, slow, fp64 CPU definition of the routed MoE layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the package entry's smoke check and
the benchmark's CPU-baseline leg may import or call anything in this package.
The product path (the HIP kernels, the C-ABI library and its Python binding)
never imports it, and this package imports nothing from the product path: the
two share no code. Both sides receive their inputs from the seeded synthetic
generator in `synth`, which holds none of the method's arithmetic.

Modules:
  mx   -- exact E2M1 / E4M3 / E8M0 codecs, MX block quantisation, BF16 rounding
  moe  -- route, permute, grouped W1 + fused epilogue, grouped W2, combine,
          the whole layer, and a brute-force dense evaluation

Every function is pinned by the `-m "not gpu"` tests in tests/test_oracle_*.py
against code tables, library conversions, closed forms, brute force and exact
metamorphic relations. No function is left "parity unpinned".
"""
from . import mx, moe  # noqa: F401
from .moe import (route, permute, gather_rows, grouped_w1, grouped_w2, combine,  # noqa: F401
                  moe_layer, dense_layer, concat_transposed, algorithmic_bytes,
                  algorithmic_flops)
