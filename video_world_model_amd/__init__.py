"""QuantWM 2-bit KV cache for MI355X (gfx950): HIP kernels behind a C ABI
(include/qwm.h) and a thin ctypes binding (``video_world_model_amd.qwm``)."""

from . import qwm  # noqa: F401
from .qwm import Cache, QwmError, lib  # noqa: F401
