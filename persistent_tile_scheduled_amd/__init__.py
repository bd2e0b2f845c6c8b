"""MI355X-native persistent, tile-scheduled batch-1 decode engine.

libdec.so (built from csrc/ by `python -m persistent_tile_scheduled_amd.build`) holds the
ahead-of-time planner, the persistent HIP engine kernel for gfx950 and the C ABI of
include/dec.h. `binding` is its ctypes binding; `engine.DecodeEngine` wraps it with torch
device memory and streams.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
