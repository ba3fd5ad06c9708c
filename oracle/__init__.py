"""fp64 CPU oracle of the InfLLM-V2 sparse attention forward path.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP library.
"""
from .infv2_oracle import *  # noqa: F401,F403
from . import infv2_oracle as impl  # noqa: F401
