"""The CPython fast-call marshalling module (CPU only): it is built beside the library, bound
to the library's entry points, and returns exactly the status codes the ctypes calls return
for the same arguments; malformed Python arguments raise before the library is called. No
kernel is launched: every case here is rejected by the library's host-side checks or is a
no-op."""
import os

import pytest

import argmin_reduction_wide_amd.binding as B
from argmin_reduction_wide_amd import build as hip_build

FAKE = 1 << 20  # an aligned, never-dereferenced address


@pytest.fixture
def fast():
    assert os.path.exists(hip_build.fast_binding_path()), "built with the library"
    m = B.fast()
    assert m is not None
    yield m
    B.argreduce_debug_set_capacity(0)


def test_reductions_route_through_the_fast_module(fast):
    assert B.entry_point("argreduce_lastaxis") is fast.argreduce_lastaxis
    assert B.entry_point("argreduce_axis") is fast.argreduce_axis
    assert B.entry_point("argreduce_scan_lastaxis") is fast.argreduce_scan_lastaxis


LASTAXIS_CASES = [
    (FAKE, B.F32, -1, 10, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 4, 0, B.MAX, FAKE, 0, 0, 0),
    (FAKE, 7, 4, 10, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 4, 10, 4, FAKE, 0, 0, 0),
    (FAKE, B.F16, 1 << 40, 1 << 30, B.MAX, FAKE, 0, 0, 0),
    (0, B.F32, 2, 8, B.MAX, FAKE, 0, 0, 0),
    (FAKE + 2, B.F32, 2, 8, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 8, B.MAX, FAKE + 4, 0, 0, 0),
    (0, B.F32, 0, 8, B.MAX, 0, 0, 0, 0),                      # rows == 0: a no-op
    (FAKE, B.F32, 1, 202048, B.MAX, FAKE, FAKE, 100, 0),       # scratch too small
    (FAKE, B.I32, 4, 10, B.MAX, FAKE, 0, 0, 0),                # integer formats: scan only
]


@pytest.mark.parametrize("args", LASTAXIS_CASES)
def test_lastaxis_status_codes_match_ctypes(fast, args):
    B.argreduce_debug_set_capacity(256 * 2048)
    assert fast.argreduce_lastaxis(*args) == B.lib().argreduce_lastaxis(*args)


AXIS_CASES = [
    (FAKE, B.F32, -1, 8, 4, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 0, 4, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 8, 0, B.MAX, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 1 << 31, 4, B.MAX, FAKE, 0, 0, 0),        # axis beyond INT32_MAX
    (FAKE, 9, 2, 8, 4, B.MAX, FAKE, 0, 0, 0),
    (0, B.F32, 0, 8, 4, B.MAX, 0, 0, 0, 0),                    # outer == 0: a no-op
]


@pytest.mark.parametrize("args", AXIS_CASES)
def test_axis_status_codes_match_ctypes(fast, args):
    assert fast.argreduce_axis(*args) == B.lib().argreduce_axis(*args)


SCAN_CASES = [
    (FAKE, B.F32, -1, 8, B.MAX, FAKE, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 0, B.MAX, FAKE, FAKE, 0, 0, 0),
    (FAKE, B.F32, 2, 8, B.MAX_LAST, FAKE, FAKE, 0, 0, 0),      # scan: MAX / MIN only
    (FAKE, B.F32, 2, 8, B.MAX, FAKE, FAKE + 4, 0, 0, 0),       # misaligned indices
    (FAKE, B.F32, 2, 8, B.MAX, FAKE, FAKE, 0, 0, 0),           # overlap with x
    (0, B.F32, 0, 8, B.MAX, 0, 0, 0, 0, 0),
]


@pytest.mark.parametrize("args", SCAN_CASES)
def test_scan_status_codes_match_ctypes(fast, args):
    assert fast.argreduce_scan_lastaxis(*args) == B.lib().argreduce_scan_lastaxis(*args)


def test_hook_status_codes_match_ctypes(fast):
    h = B.lib()
    for args in [(FAKE + 8, 64, FAKE, 1, 0), (FAKE, 60, FAKE, 1, 0), (FAKE, 64, FAKE, 0, 0),
                 (FAKE, 64, FAKE, 70000, 0), (0, 64, FAKE, 1, 0)]:
        assert fast.argreduce_debug_launch_read(*args) == h.argreduce_debug_launch_read(*args)
    assert fast.argreduce_debug_launch_store(FAKE + 4, 0) == h.argreduce_debug_launch_store(FAKE + 4, 0)
    assert fast.argreduce_debug_launch_store(0, 0) == h.argreduce_debug_launch_store(0, 0)


def test_malformed_python_arguments_raise(fast):
    with pytest.raises(TypeError):
        fast.argreduce_lastaxis(FAKE, B.F32, 2, 8)
    with pytest.raises(TypeError):
        fast.argreduce_lastaxis("x", B.F32, 2, 8, B.MAX, FAKE, 0, 0, 0)
    with pytest.raises(TypeError):
        fast.argreduce_axis(FAKE, B.F32, 2, 8, 4, B.MAX, FAKE, 0, 0, 0, 0)
    with pytest.raises(OverflowError):
        fast.argreduce_lastaxis(FAKE, B.F32, 1 << 70, 8, B.MAX, FAKE, 0, 0, 0)
    with pytest.raises(OverflowError):
        fast.argreduce_lastaxis(FAKE, B.F32, 2, 8, B.MAX, FAKE, 0, -1, 0)
    with pytest.raises(ValueError):
        fast.bind(0, 0, 0, 0, 0, 0)  # refused, and the existing binding stays
    assert fast.argreduce_lastaxis(0, B.F32, 0, 8, B.MAX, 0, 0, 0, 0) == 0
