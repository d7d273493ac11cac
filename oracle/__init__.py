"""CPU oracle for the SVDQuant W4A4 + low-rank linear (INT4, and its FP4
variant in MXFP4), a user LoRA merged into its low-rank branch, the AWQ
W4A16 linear and the GELU between the MLP projections.

TEST INFRASTRUCTURE ONLY.  It may be imported, called or executed only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product library (``w4a4_rank_corrected_smooth_amd``)
never imports it, and the two share no code, headers, helpers or tables;
the only common dependency is the seeded input generator ``synth``, which
holds none of the method's arithmetic.
"""
from . import svdquant, awq, glue, mxfp4, lora  # noqa: F401
