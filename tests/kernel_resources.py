"""Register, LDS and spill figures of the kernels in the built HIP library, read from the
gfx950 code objects that hipcc embedded in it (no GPU needed).

The library's .hip_fatbin section holds one clang offload bundle per HIP source; each
bundle holds a host entry and the gfx950 code object, an ELF whose NT_AMDGPU_METADATA note
is a msgpack map with one record per kernel (".name", ".vgpr_count", ".sgpr_count",
".agpr_count", ".group_segment_fixed_size", ".private_segment_fixed_size",
".vgpr_spill_count", ...).
"""
from __future__ import annotations

import struct

import msgpack

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32
VGPRS_PER_SIMD_LANE = 512  # gfx950 VGPR file per lane of a SIMD (unified with AGPRs)
VGPR_GRANULE = 8
MAX_WAVES_PER_SIMD = 8


def _section_headers(elf: bytes) -> list[tuple]:
    """(name, type, addr, offset, size, link, entsize) of every section of a 64-bit
    little-endian ELF."""
    assert elf[:4] == b"\x7fELF" and elf[4] == 2 and elf[5] == 1, "not an ELF64 LE file"
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + k * shentsize) for k in range(shnum)]
    stroff = hdrs[shstrndx][4]
    out = []
    for h in hdrs:
        name_off, stype, _, addr, off, size, link, _, _, entsize = h
        end = elf.index(b"\0", stroff + name_off)
        out.append((elf[stroff + name_off:end].decode(), stype, addr, off, size, link, entsize))
    return out


def _sections(elf: bytes) -> dict[str, tuple[int, int, int]]:
    """name -> (type, offset, size) of every section of a 64-bit little-endian ELF."""
    return {h[0]: (h[1], h[3], h[4]) for h in _section_headers(elf)}


def _code_objects(lib_bytes: bytes, arch: str) -> list[bytes]:
    sec = _sections(lib_bytes)
    _, off, size = sec[".hip_fatbin"]
    blob = lib_bytes[off:off + size]
    objs = []
    pos = blob.find(BUNDLE_MAGIC)
    while pos >= 0:
        n = struct.unpack_from("<Q", blob, pos + len(BUNDLE_MAGIC))[0]
        p = pos + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            eoff, esize, tsize = struct.unpack_from("<QQQ", blob, p)
            triple = blob[p + 24:p + 24 + tsize].decode()
            p += 24 + tsize
            if arch in triple and esize > 0:
                objs.append(blob[pos + eoff:pos + eoff + esize])
        pos = blob.find(BUNDLE_MAGIC, p)
    return objs


def _metadata(code_object: bytes) -> dict:
    for stype, off, size in _sections(code_object).values():
        if stype != 7:  # SHT_NOTE
            continue
        p = off
        while p < off + size:
            namesz, descsz, ntype = struct.unpack_from("<III", code_object, p)
            name = code_object[p + 12:p + 12 + namesz].rstrip(b"\0")
            desc_at = p + 12 + ((namesz + 3) & ~3)
            if name == b"AMDGPU" and ntype == NT_AMDGPU_METADATA:
                return msgpack.unpackb(code_object[desc_at:desc_at + descsz], raw=False,
                                       strict_map_key=False)
            p = desc_at + ((descsz + 3) & ~3)
    raise ValueError("no AMDGPU metadata note in the code object")


def _kernel_descriptors(code_object: bytes) -> dict[str, bytes]:
    """symbol name (without ".kd") -> the 64-byte kernel descriptor, from the symbol table."""
    hdrs = _section_headers(code_object)
    out = {}
    for name, stype, _, off, size, link, entsize in hdrs:
        if stype != 2:  # SHT_SYMTAB
            continue
        stroff = hdrs[link][3]
        for k in range(size // entsize):
            st_name, _, _, shndx, value, sz = struct.unpack_from("<IBBHQQ", code_object, off + k * entsize)
            end = code_object.index(b"\0", stroff + st_name)
            sym = code_object[stroff + st_name:end].decode()
            if sym.endswith(".kd") and sz == 64:
                sec = hdrs[shndx]
                at = sec[3] + (value - sec[2])
                out[sym[:-3]] = code_object[at:at + 64]
    return out


def kernels(lib_path: str, arch: str = "gfx950") -> list[dict]:
    """One metadata record per kernel of every ``arch`` code object in the library, with
    ".preload_dwords" added: the kernel-argument dwords the descriptor has the hardware
    preload into SGPRs at wave launch (KERNARG_PRELOAD_SPEC_LENGTH, bits 0-6 of the 16-bit
    field at byte 58 of the descriptor); arguments beyond them are loaded from memory."""
    with open(lib_path, "rb") as f:
        data = f.read()
    objs = _code_objects(data, arch)
    if not objs:
        raise ValueError(f"no {arch} code object in {lib_path}")
    out = []
    for co in objs:
        kds = _kernel_descriptors(co)
        for k in _metadata(co)["amdhsa.kernels"]:
            kd = kds.get(k[".symbol"][:-3] if k[".symbol"].endswith(".kd") else k[".symbol"])
            k[".preload_dwords"] = None if kd is None else struct.unpack_from("<H", kd, 58)[0] & 0x7F
            out.append(k)
    return out


def explicit_arg_bytes(k: dict) -> int:
    """Bytes of a kernel's own arguments (the hidden ones the runtime appends excluded)."""
    args = [a for a in k[".args"] if not a[".value_kind"].startswith("hidden")]
    return max((a[".offset"] + a[".size"] for a in args), default=0)


def waves_per_simd(k: dict) -> int:
    """Waves of this kernel one SIMD holds at once, as its registers allow (VGPRs and AGPRs
    share one file of 512 per lane; allocation in granules of 8)."""
    regs = k[".vgpr_count"] + k.get(".agpr_count", 0)
    regs = max(VGPR_GRANULE, -(-regs // VGPR_GRANULE) * VGPR_GRANULE)
    return min(MAX_WAVES_PER_SIMD, VGPRS_PER_SIMD_LANE // regs)
