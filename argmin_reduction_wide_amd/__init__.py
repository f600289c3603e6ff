"""MI355X (gfx950) ArgMax / ArgMin (last or middle axis) and cummax / cummin with indices.

The computation runs in the HIP library ``libargreduce.so`` (C ABI: include/argreduce.h);
``binding`` marshals arguments into it. Importing this package loads nothing; the library
is loaded on first use and its absence is an error, never a fallback.
"""
from .binding import (  # noqa: F401
    ArgreduceError,
    argmax,
    argmin,
    argreduce_axis,
    argreduce_axis_plan,
    argreduce_axis_scratch_bytes,
    argreduce_debug_force_path,
    argreduce_debug_set_capacity,
    argreduce_lastaxis,
    argreduce_plan,
    argreduce_scan_lastaxis,
    argreduce_scan_plan,
    argreduce_scan_scratch_bytes,
    argreduce_scratch_bytes,
    cummax,
    cummin,
)
