"""MI355X-native hierarchical (R-top-k) beam-search selection step.

The product is librtopk.so (include/rtopk.h): HIP kernels for gfx950 behind a
C ABI. This package holds its sources (csrc/), the in-tree build (_build), the
ctypes binding (rtopk) and seeded synthetic inputs (synth).
"""
from .rtopk import (  # noqa: F401
    RTOPK_BF16, RTOPK_F16, RTOPK_F32, RtopkError, beam_step, debug_step, rtopk_beam_step,
    rtopk_beam_step_ws, rtopk_debug_step, rtopk_last_error, rtopk_plan, rtopk_release,
    rtopk_set_override, rtopk_workspace_bytes,
)
