"""Checks on the gfx950 assembly of the decode kernels (CPU only: hipcc
cross-compiles).

The decode loops stream K/V with several tiles in flight per wave.  A full
drain of the vector-memory counter (s_waitcnt vmcnt(0)) inside a loop would
stall every prefetch; the compiler inserts one whenever a register that an
in-flight load or store still uses gets reused, so these checks guard the
code shapes that avoid it.  They also pin register use and the absence of
scratch (spill) memory.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_03_amd import build as B

hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(hipcc), reason="hipcc not available")


def device_asm(src, tmp_path, defines=()):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [hipcc, *B.HIPCC_FLAGS, *defines, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernel_body(asm, name_part):
    m = re.search(r"^(_Z\S*" + name_part + r"\S*):\s*;.*$", asm, re.M)
    assert m, f"kernel {name_part} not found"
    start = m.end()
    end = asm.index("s_endpgm", start)
    body = asm[start:asm.index(".Lfunc_end", start)]
    return body


def meta(asm, name_part, key):
    """A field of the kernel's own entry in the code-object metadata (the
    entry runs from its "- .agpr_count" line to the next entry)."""
    sym = re.search(r"^(_Z\S*" + name_part + r"\S*):", asm, re.M).group(1)
    at = asm.index(f".name:           {sym}")
    start = asm.rfind("  - .agpr_count:", 0, at)
    end = asm.find("  - .agpr_count:", at)
    block = asm[start:end if end > 0 else at + 4000]
    return int(re.search(rf"\.{key}:\s+(\d+)", block).group(1))


@pytest.fixture(scope="module")
def flat_asm(tmp_path_factory):
    return device_asm("pa_decode_flat.hip", tmp_path_factory.mktemp("isa"))


@pytest.fixture(scope="module")
def part_asm(tmp_path_factory):
    return device_asm("pa_decode.hip", tmp_path_factory.mktemp("isa"))


def tile_loops(body):
    """{loop header: text of every block of that loop} for the loops that
    issue 16-byte tile loads, from the compiler's loop annotations (a header
    block says "Loop Header", member blocks say "in Loop: Header=BB..")."""
    blocks = re.split(r"^(?=\.LBB\d+_\d+:)", body, flags=re.M)
    loops = {}
    for blk in blocks:
        first = blk.split("\n", 2)
        head = "\n".join(first[:2])
        m = re.match(r"\.LBB(\d+_\d+):", blk)
        if not m:
            continue
        if "Loop Header" in head:
            key = "BB" + m.group(1)
        else:
            h = re.search(r"in Loop: Header=(BB\d+_\d+)", head)
            if not h:
                continue
            key = h.group(1)
        loops[key] = loops.get(key, "") + blk
    return {k: v for k, v in loops.items() if "buffer_load_dwordx4" in v}


@pytest.mark.parametrize("append", [0, 1])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("policy", [2, 0])
def test_flat_loop_never_drains_loads(flat_asm, D, policy, append):
    """The flat decode (and its instantiation with the fused append) keeps
    its load ring going: no full drain of the load counter once blocks are
    consumed."""
    body = kernel_body(flat_asm, f"pa_decode_flat_kernelILi{D}ELi{policy}ELb0ELb{append}E")
    loops = tile_loops(body)
    assert loops, "no tile loop found"
    for label, text in loops.items():
        assert "vmcnt(0)" not in text, f"full load drain inside loop {label}"
    # nor anywhere once blocks are being consumed
    assert "vmcnt(0)" not in body[body.index("v_dot2"):]
    # the tiles are fetched as 16-byte buffer loads, non-temporal by default
    nt = re.search(r"buffer_load_dwordx4 .* offen( offset:\d+)? nt", body)
    assert bool(nt) == (policy == 2)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("policy", [2, 0])
def test_partition_loop_never_drains_loads(part_asm, D, policy):
    body = kernel_body(part_asm, f"pa_decode_part_kernelILi{D}ELi{policy}E")
    loops = tile_loops(body)
    assert loops, "no tile loop found"
    for label, text in loops.items():
        assert "vmcnt(0)" not in text, f"full load drain inside loop {label}"


def test_no_spills_and_register_budget(flat_asm, part_asm):
    for asm, name in ((flat_asm, "pa_decode_flat_kernelILi128ELi2ELb0ELb0E"),
                      (flat_asm, "pa_decode_flat_kernelILi128ELi2ELb0ELb1E"),
                      (part_asm, "pa_decode_part_kernelILi128E")):
        assert meta(asm, name, "vgpr_spill_count") == 0
        assert meta(asm, name, "private_segment_fixed_size") == 0
    # two waves per SIMD for the flat kernel (<= 256 VGPRs), with or without
    # the fused append, three for the partitioned one (<= 168)
    for append in (0, 1):
        name = f"pa_decode_flat_kernelILi128ELi2ELb0ELb{append}E"
        assert meta(flat_asm, name, "vgpr_count") <= 256
    assert meta(part_asm, "pa_decode_part_kernelILi128E", "vgpr_count") <= 168


@pytest.fixture(scope="module")
def grouped_asm(tmp_path_factory):
    return device_asm("pa_decode_grouped.hip", tmp_path_factory.mktemp("isa"))


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("policy", [2, 0])
def test_grouped_ring_keeps_a_tile_in_flight(grouped_asm, D, policy):
    """The grouped decode's tile loop (the one issuing the MFMAs) never
    drains its loads, and no wait in it leaves less than one tile (2*D/32
    loads) in flight; both products run on the matrix cores."""
    body = kernel_body(grouped_asm, f"pa_decode_grouped_kernelILi{D}ELi{policy}E")
    rings = [t for t in tile_loops(body).values() if "v_mfma" in t]
    assert len(rings) == 1, "expected one MFMA tile loop"
    ring = rings[0]
    assert "vmcnt(0)" not in ring
    waits = [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", ring)]
    assert waits and min(waits) >= 2 * (D // 32)
    assert "v_mfma_f32_16x16x32_f16" in ring and "v_mfma_f32_16x16x16_f16" in ring
    nt = re.search(r"buffer_load_dwordx4 .* offen( offset:\d+)? nt", ring)
    assert bool(nt) == (policy == 2)


def test_grouped_no_spills_and_register_budget(grouped_asm):
    for D in (128, 64):
        name = f"pa_decode_grouped_kernelILi{D}E"
        assert meta(grouped_asm, name, "vgpr_spill_count") == 0
        assert meta(grouped_asm, name, "private_segment_fixed_size") == 0
        # two waves per SIMD: VGPRs and AGPRs share the 512-entry file (the
        # metadata's vgpr_count already counts the AGPRs after the VGPRs)
        assert meta(grouped_asm, name, "vgpr_count") <= 256


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return device_asm("pa_prefill.hip", tmp_path_factory.mktemp("isa"))


@pytest.mark.parametrize("multi", [False, True])
@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("D", [128, 64])
def test_prefill_ring_keeps_a_tile_in_flight(prefill_asm, D, append, multi):
    """The prefill's tile loop: 32x32x16 MFMAs, the K/V buffer resources stay
    scalar (no waterfall loop around a load), and no wait drains the loads.
    Without the append, tiles are copied straight into LDS (buffer_load ...
    lds) and every wait leaves the next pair's copies (2 x D/64 per thread)
    in flight; with it, they come through a register ring in which three
    tiles (D/64 16-byte loads per thread and tile) stay in flight at every
    wait, through the per-tile choice of source (rows or pools) and the pool
    writes.  Items of several heads (multi) run the same loops with the head
    boundaries inside: there the ring's waits for the next head's queries
    still leave the two tiles fetched last in flight."""
    name = f"pa_prefill_kernelILi{D}ELb{int(append)}ELb{int(multi)}E"
    body = kernel_body(prefill_asm, name)
    # the ring is the loop with the most MFMAs (the item loop around it
    # holds the first pair's score products and waits for each item's start)
    rings = [t for t in tile_loops(body).values() if "v_mfma" in t]
    assert rings, "no MFMA tile loop"
    ring = max(rings, key=lambda t: t.count("v_mfma"))
    assert ring.count("v_mfma") >= 4 * (D // 32)
    assert "v_mfma_f32_32x32x16_f16" in ring
    assert "s_cbranch_execnz" not in ring
    assert "vmcnt(0)" not in ring
    waits = [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", ring)]
    if append:
        assert waits and min(waits) >= (2 if multi else 3) * (D // 64)
    else:
        assert re.search(r"buffer_load_dwordx4 .* lds", ring)
        assert waits and min(waits) >= 2 * (D // 64)
    assert meta(prefill_asm, name, "vgpr_spill_count") == 0
    assert meta(prefill_asm, name, "private_segment_fixed_size") == 0
    assert meta(prefill_asm, name, "vgpr_count") <= 256


@pytest.mark.parametrize("D", [128, 64])
def test_contiguous_flat_loop_never_drains_loads(flat_asm, D):
    """The same flat kernel addressing contiguous rows: same load ring, no
    drain, no spill."""
    name = f"pa_decode_flat_kernelILi{D}ELi2ELb1ELb0E"
    body = kernel_body(flat_asm, name)
    loops = tile_loops(body)
    assert loops
    for label, text in loops.items():
        assert "vmcnt(0)" not in text, f"full load drain inside loop {label}"
    assert "vmcnt(0)" not in body[body.index("v_dot2"):]
    assert meta(flat_asm, name, "vgpr_spill_count") == 0
    assert meta(flat_asm, name, "vgpr_count") <= 256
