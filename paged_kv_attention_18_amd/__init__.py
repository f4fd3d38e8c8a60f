"""MI355X (gfx950) paged-attention forward: HIP kernels behind a C ABI.

``binding`` holds the ctypes face of ``include/pa.h``; ``synth`` draws seeded
synthetic inputs; ``build`` compiles ``libpa.so``.
"""
from . import synth  # noqa: F401
from .binding import (Attention, PaError, for_problem, pa_create, pa_describe, pa_destroy,  # noqa: F401
                      pa_forward, pa_get_device_error, pa_read_timing, pa_set_timing, pa_status_string,
                      run_problem)
