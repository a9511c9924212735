"""CPU oracle for the W4A16 group-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check of the
entry module and the benchmark's CPU-baseline leg do.  It shares no code with
the HIP library (no kernels, headers, tables or helpers); the only module both
sides use is ``synthetic`` (seeded input generators, which hold none of the
method's arithmetic).

See ``oracle/w4_oracle.py`` for the functions and the passages they follow.
"""
from .w4_oracle import *  # noqa: F401,F403
from .w4a8_oracle import *  # noqa: F401,F403
