"""CPU oracle for latent-space MLA decode -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy implementations of what the decode path computes, written
from the method's definition on the "Mla Analysis" page (sections "Absorption
Trick (FlashMLA)", "Cost Models", "Tensor Shapes") and the FlashMLA-2 newsletter
page (section "Architectural Analysis": FP8 latent cache, the sorted block
scheduler that balances sequence partitions across compute units).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package. The product
path (the HIP library and its Python binding) never does, and this package shares
no code with it: it imports nothing from ``mla_latent_space_amd``. Inputs reach it
as plain arrays produced by the seeded generator module.

Modules:
  mla   -- latent-form decode, explicit (decompressed) form, e4m3fn decoder and
           the FP8-to-BF16 scaling, split combine, cost models.
  plan  -- the split-plan definition (sort by length, equal-cost contiguous
           chunks), used to check the device planner bit for bit.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(library cross-checks -- torch's float8 and bfloat16 casts for the number formats --,
closed forms, brute force, invariants, printed values, and for the cost models an
independent tensor inventory), and each pin group has a planted-mistake test that
must fail it. No function is "parity unpinned".
"""
