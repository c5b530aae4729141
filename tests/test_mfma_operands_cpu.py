"""Register placement of the matrix instructions in the compiled kernels (CPU).

A matrix instruction whose destination quad starts above its accumulator
input while sharing registers with it (for example destination a[28:31] with
accumulator a[26:29]) overwrote the accumulator's last element before the
instruction had read it: the fp32 chunk kernel then divided rows 3 mod 4 by
a wrong normaliser.  The compiler emits such placements when an accumulator
array is indexed by a run-time count and rotates through registers; the
kernels keep those counts compile-time.  Overlaps in the other direction
(destination below the accumulator) are read before they are written and
pass the GPU parity tests, so only the harmful direction is rejected here.
Every source that issues matrix instructions is compiled to gfx950
assembly with the library's own flags and scanned.
"""
import concurrent.futures as cf
import re
import shutil

import pytest

from kernelized_linear_attention_la_amd import build

MFMA_SOURCES = ["la_mfma.hip", "la_mfma_seg.hip", "la_favor.hip", "la_backward_mfma.hip",
                "la_gla_chunk.hip", "la_delta_chunk.hip", "la_f32mma.hip"]
_MFMA = re.compile(r"(v_mfma\S*)\s+([av])\[(\d+):(\d+)\],\s*[^,]+,\s*[^,]+,\s*([av])\[(\d+):(\d+)\]")

pytestmark = pytest.mark.skipif(not (shutil.which("hipcc") or __import__("os").path.exists("/opt/rocm/bin/hipcc")),
                                reason="hipcc is not installed")


def harmful_overlaps(asm: str):
    """(line, text) of matrix instructions whose destination starts inside and above their accumulator."""
    bad = []
    for ln, line in enumerate(asm.splitlines(), 1):
        m = _MFMA.search(line)
        if not m:
            continue
        dfile, d0, d1 = m.group(2), int(m.group(3)), int(m.group(4))
        cfile, c0, c1 = m.group(5), int(m.group(6)), int(m.group(7))
        if dfile == cfile and c0 < d0 <= c1:
            bad.append((ln, line.strip()))
    return bad


def test_scanner_flags_the_harmful_direction_only():
    asm = "\n".join([
        "v_mfma_f32_16x16x4_f32 a[28:31], v53, v4, a[26:29]",   # harmful
        "v_mfma_f32_16x16x4_f32 a[6:9], v29, v30, a[8:11]",     # read before written
        "v_mfma_f32_16x16x4_f32 a[24:27], v53, v5, a[24:27]",   # in place
        "v_mfma_f32_16x16x32_bf16 v[6:9], v[0:3], v[12:15], v[4:7]",  # harmful, VGPRs
        "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], 0",  # zero accumulator
    ])
    assert [b[0] for b in harmful_overlaps(asm)] == [1, 4]


def test_no_matrix_instruction_overwrites_its_unread_accumulator():
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        asms = dict(zip(MFMA_SOURCES, ex.map(build.device_asm, MFMA_SOURCES)))
    found = {src: harmful_overlaps(a)[:5] for src, a in asms.items()}
    assert sum("v_mfma" in a for a in asms.values()) == len(MFMA_SOURCES)
    assert not any(found.values()), found
