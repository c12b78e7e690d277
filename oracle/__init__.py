"""CPU oracle for the block-scaled FP8 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers), and it never consumes a value
produced by the HIP library.

What it computes, and where the pages define it:

* ``formats``  -- the OCP e4m3 ("float8_e4m3fn") codec and bf16 rounding.
  Admin Guide ("DeepSeek-V3 Administrator & Developer Guide", doccompiler),
  section 8.5.1 (448 is the largest e4m3fn magnitude); DocSearch index of the
  DeepSeek-V3 README, item 10 (``fmt: e4m3`` is ``torch.float8_e4m3fn``).
* ``quant``    -- per-token, per-128-channel activation quantisation
  (Admin Guide 8.5.1; User Guide FAQ "What is scale_fmt: ue8m0?"), the 128x128
  weight block-scale format with zero padding (DocSearch item 3), weight
  dequantisation (Admin Guide 8.5.2), and the weight block quantiser that
  produces that format from real-valued weights.
* ``gemm``     -- the block-scaled product with per-K-block rescaling
  (Admin Guide 8.5.3 and 6.3), and its per-expert grouped form (Admin Guide
  6.4 and 8.4).
* ``glue``     -- SiLU(g) * u between the up and down projections
  (Admin Guide 1.2, MLP / Expert rows).
* ``moe``      -- the routed-expert steps around the grouped product: the row
  order of the (token, slot) pairs, the gathered act_quant and the weighted
  bf16 combine (Admin Guide 6.4 and 8.4).

Precision: the pages fix fp32 for the quantisers (the data are converted to fp32 first), so
those run in IEEE binary32 through NumPy float32 scalars/arrays, whose
arithmetic is correctly rounded.  The products are formed in fp64.

Pins: every function here is pinned by ``tests/test_oracle_*.py`` against
something other than itself (torch's own float8/bfloat16 casts, exact rational
arithmetic, closed forms, invariants, brute force).  ``glue.silu_mul`` is
pinned only against fp64 closed forms at a few points and a Fraction-free
second evaluation; see its docstring.
"""

from . import formats, quant, gemm, glue, moe  # noqa: F401

BLOCK = 128
