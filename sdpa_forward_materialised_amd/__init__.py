"""MI355X-native materialised-probability SDPA forward.

``fwd(q, k, v, attn_mask=None, is_causal=False, scale=None, enable_gqa=False)``
returns ``(O, P, LSE)``: the attention output, the full probability map and
the float32 row log-sum-exp, computed by hand-written gfx950 HIP kernels in
``libsdpa_math.so`` (C ABI declared in ``include/sdpa_math.h``). This package
is argument marshalling only; torch supplies device memory and streams.
"""

from ._binding import (EXPORTS, LIB_PATH, PATHS, SdpaMathFunction, bwd, fwd, fwd_noalloc, fwd_varlen,  # noqa: F401
                       PreparedFwd, kernel_name, last_error, load_library, plan, prepare_fwd, probe_copy, probe_fill, sdpa_math, version)

__all__ = ["fwd", "fwd_noalloc", "fwd_varlen", "bwd", "sdpa_math", "SdpaMathFunction", "plan", "kernel_name", "prepare_fwd", "PreparedFwd", "version", "last_error",
           "load_library", "LIB_PATH", "PATHS", "EXPORTS"]
