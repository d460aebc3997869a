"""CPU oracle for compressed-KV sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and nothing here imports the product path.
"""
from .ckv_oracle import *  # noqa: F401,F403
from .hc_oracle import (HC_EPS, HC_N, HC_SINKHORN_ITERS, hc_post, hc_pre, hc_split,  # noqa: F401
                        sigmoid, sinkhorn)
