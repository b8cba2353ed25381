"""MI355X-native DARKFormer positive-random-feature attention (forward pass).

The compute lives in libdarkprf.so (hand-written HIP kernels for gfx950) behind
the C ABI of include/darkprf.h; `binding` is a thin ctypes layer over it.
"""
from .binding import (  # noqa: F401
    DarkPrfDesc,
    DarkPrfError,
    dark_prf_decode_step,
    dark_prf_fwd,
    dark_prf_omega,
    dark_prf_proj_tag,
    dark_prf_status_str,
    dark_prf_timing_begin,
    dark_prf_timing_end,
    dark_prf_workspace_bytes,
    decode_step,
    make_desc,
    prf_attention,
)
