"""CPU oracle for the deferred MoE finalize: TEST INFRASTRUCTURE.

Plain, slow, obviously-correct numpy code that states what the HIP library
must compute. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it; the library and its binding
never do, and this package imports nothing from them (the two share no
code; only the seeded input generators serve both).

``formats``  - bf16 / OCP E4M3 / UE8M0 helpers from the format definitions.
``finalize`` - finalize, residual + RMSNorm and UE8M0 quant, in an fp64
               "truth" mode and an fp32 "mirror" mode.
``routing``  - the sigmoid top-k gate and packed-word producer that feed it.
``act_quant`` - standalone 1 x 128 FP8 activation quant, power-of-two
               (UE8M0) and continuous (amax / 448) scale policies.

Every function is pinned by CPU tests to something other than itself
(closed forms, exhaustive enumeration, exact rational arithmetic, library
routines, invariants); see ``tests/test_oracle_*.py``.
"""
from . import act_quant, finalize, formats, routing  # noqa: F401
