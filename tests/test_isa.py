"""Checks on the gfx950 assembly of the library's own kernels (CPU only: compiles the device pass).

The LDS-DMA loads are inline assembly that writes M0 ahead of each `buffer_load ... lds`; the
compiler is told M0 is clobbered but treats it as reserved, so the kernels are only correct if no
compiler-generated instruction relies on M0.  This test pins that: every M0 write is one of ours,
directly followed by its LDS-DMA load, and no instruction reads M0 otherwise.
"""
import re

import pytest

from attention_backward_sdpa_amd import build


@pytest.fixture(scope="module")
def asm():
    return build.device_assembly()


def _instructions(text):
    out = []
    for line in text.splitlines():
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append(t)
    return out


def test_m0_written_only_for_lds_dma(asm):
    ins = _instructions(asm)
    n_dma = 0
    for i, t in enumerate(ins):
        if not re.search(r"\bm0\b", t):
            continue
        # the asm's scalar operand may land in any SGPR, vcc_lo/vcc_hi included
        assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", t), f"unexpected M0 use: {t}"
        nxt = ins[i + 1]
        assert re.match(r"buffer_load_dword(x4)? v\d+, s\[\d+:\d+\], 0 offen (sc1 )?lds", nxt), \
            f"M0 write not followed by its LDS-DMA load: {t} / {nxt}"
        n_dma += 1
    assert n_dma > 0
    # every LDS-DMA load is preceded by its own M0 write
    n_lds_loads = sum(1 for t in ins if re.match(r"buffer_load_dword\w* .* lds$", t))
    assert n_lds_loads == n_dma

