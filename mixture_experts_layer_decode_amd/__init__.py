"""MI355X (gfx950) decode-step Mixture-of-Experts layer.

The layer runs in hand-written HIP kernels behind the C ABI of
``libmoe_decode.so`` (include/moe_decode.h); this package is the Python
binding (argument marshalling only) and its build script.
"""
from .binding import (BF16, F32, FP8_E4M3, PATH_AUTO, PATH_GEMV, PATH_MFMA, ROUTER_AUTO,
                      ROUTER_GEMV, ROUTER_MFMA, SIGMOID, SOFTMAX,
                      STAGES, Context, MoeError, check_config, dtype_code, forward_noalloc,
                      last_error, load_library, make_config)

__all__ = ["BF16", "F32", "FP8_E4M3", "PATH_AUTO", "PATH_GEMV", "PATH_MFMA", "ROUTER_AUTO",
           "ROUTER_GEMV", "ROUTER_MFMA", "SIGMOID", "SOFTMAX",
           "STAGES", "Context", "MoeError", "check_config", "dtype_code", "forward_noalloc",
           "last_error", "load_library", "make_config"]
