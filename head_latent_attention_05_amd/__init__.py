"""MLA decode with weight absorption on MI355X (gfx950): libmla + thin bindings.

    binding  -- ctypes wrappers of the C ABI in include/mla.h
    step     -- a device-resident decode/prefill step over the four calls
    synth    -- seeded synthetic inputs (shared by tests, benchmark and oracle checks)
    build    -- compiles libmla.so for gfx950
"""
from .binding import MlaConfig, MlaError, load  # noqa: F401
