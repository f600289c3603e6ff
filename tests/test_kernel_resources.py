"""Registers, LDS and residency of the built gfx950 kernels, read from the code-object
metadata of the library (CPU only), and the split plans checked against them.

The split path's finalizing workgroup waits for the other workgroups of its row. The
automatic plans launch at most one device wave of 256-thread workgroups (CUs * 2048 / 256)
and the split kernel (k_split) is compiled for eight waves per SIMD, so every workgroup of such a grid is
resident at once on an otherwise idle device: no wait depends on the order in which the
dispatcher starts workgroups. These tests pin both halves of that argument.
"""
import os
import re

import pytest

import argmin_reduction_wide_amd.binding as B
import kernel_resources as K

MI355X_THREADS = 256 * 2048
H200_THREADS = 132 * 2048
LDS_PER_CU = 160 * 1024
THREADS_PER_CU = 2048
BLOCK = 256
FMT = {B.F32: "F32", B.F16: "F16", B.BF16: "BF16", B.F64: "F64"}


@pytest.fixture(scope="module")
def kernels():
    return K.kernels(B.LIB_PATH)


def blocks_per_cu(k: dict) -> int:
    """Workgroups of 256 threads (four waves, one per SIMD) of kernel k one CU holds."""
    lds = k[".group_segment_fixed_size"]
    by_lds = LDS_PER_CU // lds if lds else THREADS_PER_CU // BLOCK
    return min(K.waves_per_simd(k), by_lds, THREADS_PER_CU // BLOCK)


VW = {"F32": 4, "F16": 8, "BF16": 8, "F64": 2}


def split_kernels(kernels, fmt: str, unroll: int) -> list[dict]:
    """The k_split<fmt, op, unroll, mode> instances, every op and scan mode (general,
    aligned, span)."""
    pat = re.compile(rf"k_splitINS_\d+{fmt}ELi\dELi{unroll}ELi[012]EEE")
    return [k for k in kernels if pat.search(k[".name"])]


def split_modes(fmt: str, unroll: int) -> int:
    """Scan modes built per op: the span scan only where a lane holds at most 32 elements."""
    return 3 if unroll * VW[fmt] <= 32 else 2


def test_every_format_op_and_unroll_of_the_split_kernel_is_present(kernels):
    for fmt in FMT.values():
        for u in (1, 2, 4, 8):
            assert len(split_kernels(kernels, fmt, u)) == 4 * split_modes(fmt, u), (fmt, u)


def test_split_kernel_holds_a_full_cu(kernels):
    """Every k_split instance: at most 64 VGPRs (eight waves per SIMD), no private
    (spill) memory, LDS for eight workgroups per CU."""
    ks = [k for k in kernels if "k_split" in k[".name"]]
    assert len(ks) == sum(4 * split_modes(f, u) for f in FMT.values() for u in (1, 2, 4, 8))
    for k in ks:
        assert k[".wavefront_size"] == 64
        assert K.waves_per_simd(k) == 8, (k[".name"], k[".vgpr_count"])
        assert k[".private_segment_fixed_size"] == 0, k[".name"]
        assert blocks_per_cu(k) == THREADS_PER_CU // BLOCK, k[".name"]


def test_no_kernel_uses_private_memory(kernels):
    """No kernel spills registers to memory or keeps a stack (SGPR spills into VGPR lanes,
    as in the unaligned long-row scan, use no memory)."""
    for k in kernels:
        assert k[".private_segment_fixed_size"] == 0, k[".name"]
        assert not k.get(".uses_dynamic_stack", False), k[".name"]


def test_every_kernel_argument_is_preloaded(kernels):
    """Each kernel's own arguments fit the SGPRs the hardware preloads at wave launch (at
    most 14 dwords here): an argument beyond them would be read from kernel-argument memory
    by every wave, which with arguments kept in host memory is a read across PCIe per wave."""
    for k in kernels:
        assert k[".preload_dwords"] is not None, k[".name"]
        assert K.explicit_arg_bytes(k) <= 4 * k[".preload_dwords"], (
            k[".name"], K.explicit_arg_bytes(k), k[".preload_dwords"])


SHAPES = [(r, c) for r in (1, 2, 3, 8, 32, 100, 255, 256, 1000)
          for c in (1000, 4096, 32000, 65537, 202048, 500000, 1 << 20, 3 << 20, 1 << 24,
                    (1 << 31) - 1)]


@pytest.mark.parametrize("cap", [MI355X_THREADS, H200_THREADS, 16 * 2048, 2048])
def test_automatic_split_plans_fit_one_resident_wave(kernels, cap):
    """For every automatic split plan, the grid is at most what the device holds at once of
    the very kernel instance it launches (CUs = capacity / 2048)."""
    B.argreduce_debug_set_capacity(cap)
    try:
        cus = cap // THREADS_PER_CU
        seen = 0
        for dtype, fmt in FMT.items():
            for rows, cols in SHAPES:
                p = B.argreduce_plan(rows, cols, dtype)
                if p["path"] != B.PATH_SPLIT:
                    continue
                seen += 1
                inst = split_kernels(kernels, fmt, p["unroll"])
                resident = cus * min(blocks_per_cu(k) for k in inst)
                assert p["grid_blocks"] <= resident, (cap, rows, cols, fmt, p, resident)
        assert seen > 0
    finally:
        B.argreduce_debug_set_capacity(0)


def test_fp64_split_at_a_full_device_wave(kernels):
    """[8, 1048576] and [32, 262144] fp64 at MI355X capacity: 2048 workgroups of U = 8, the
    largest automatic split grids, all resident."""
    B.argreduce_debug_set_capacity(MI355X_THREADS)
    try:
        for rows, cols in [(8, 1 << 20), (32, 1 << 18)]:
            p = B.argreduce_plan(rows, cols, B.F64)
            assert p["path"] == B.PATH_SPLIT and p["unroll"] == 8, p
            assert p["grid_blocks"] == 2048 == MI355X_THREADS // BLOCK
            assert all(blocks_per_cu(k) == 8 for k in split_kernels(kernels, "F64", 8))
    finally:
        B.argreduce_debug_set_capacity(0)


def test_metadata_reader_sees_both_sources(kernels):
    names = " ".join(k[".name"] for k in kernels)
    for kernel in ("k_narrow", "k_subwave", "k_blocks", "k_split", "k_axis", "k_axis_merge",
                   "k_wide", "k_cum", "k_read_floor"):
        assert kernel in names, kernel
    assert os.path.getsize(B.LIB_PATH) > 0
