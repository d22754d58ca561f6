"""CPU oracle (test infrastructure): plain float64 / exact-rational reference of the
residual binarization, the matmul-free product and the binary-codebook variant.
Only tests, the smoke check and the bench's CPU-baseline leg use it."""
from .rb_oracle import *  # noqa: F401,F403
