"""CPU oracle (float64 numpy) of the flow-matching action expert.

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The product path never
does, and it shares no code with the HIP kernels.
"""
from . import denoise, quant  # noqa: F401
