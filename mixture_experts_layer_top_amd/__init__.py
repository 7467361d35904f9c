"""MI355X-native MoE expert-layer forward: HIP kernels for gfx950 behind a
C ABI (libmoe.so), with a ctypes binding and a driver for the whole layer."""
from .inputs import CONFIGS, LayerConfig, make_layer  # noqa: F401
from . import _lib  # noqa: F401  (loads libmoe.so lazily, on first call)
