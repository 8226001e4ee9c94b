"""CPU oracle (test infrastructure only): a plain, slow, independent
implementation of the quantized projection used to check the HIP library.
Only tests, the smoke check and the benchmark's CPU-baseline leg import it."""
from .qlin_oracle import *  # noqa: F401,F403
from .qlin_oracle import __all__  # noqa: F401
