"""Host model of the record addressing of the gate/up and down tiles: for
every supported shape and width, the largest byte any lane touches stays
inside its section (so inside the record), including the clamped positions
past a ragged end.  The lane layout is the kernels' own: a row of `cols`
columns at b bits is cols*b/128 16-byte chunks; 2^lg lanes share a row
(lg = ceil(log2(chunks)), at most 6); lane li of a row takes chunks li,
li + 2^lg, ...; positions past the row or past the last row load row 0 /
chunk 0 instead.  The scale/bias word of chunk c is word c/2 (4-bit) or c
(2-bit) of the row's group words."""
import math

import pytest

from bit_dequant_expert_route_amd import synth


def _max_offsets(rows, cols, bits, nch, npass):
    cpr = cols * bits // 128
    lg = min(6, max(0, math.ceil(math.log2(cpr))) if cpr > 1 else 0)
    rpp = 64 >> lg
    wpr = cols * bits // 32
    gpr = cols // 64
    rows_per_wave = npass * rpp
    waves = (rows + rows_per_wave - 1) // rows_per_wave
    max_code = max_sb = 0
    for wave in (0, waves - 1):
        row0 = wave * rows_per_wave
        for lane in range(64):
            li, rip = lane & ((1 << lg) - 1), lane >> lg
            for p in range(npass):
                r = row0 + p * rpp + rip
                for j in range(nch):
                    c = li + (j << lg)
                    inside = r < rows and c < cpr
                    rr, cc = (r, c) if inside else (0, 0)
                    max_code = max(max_code, (rr * wpr + cc * 4) * 4 + 16)
                    g = cc // 2 if bits == 4 else cc
                    max_sb = max(max_sb, (rr * gpr + g) * 4 + 4)
    return max_code, max_sb


def _nch(cols, bits):
    cpr = cols * bits // 128
    lpr = 64 if cpr >= 64 else 1 << max(0, math.ceil(math.log2(cpr)) if cpr > 1 else 0)
    n = (cpr + lpr - 1) // lpr
    return 1 if n <= 1 else (2 if n <= 2 else 4)


@pytest.mark.parametrize("bits", [4, 2])
def test_tile_reads_stay_inside_their_sections(bits):
    for H in range(64, 8192 + 1, 64 * 7):
        for I in (64, 128, 192, 320, 1024, 4096, 8192):
            lay = synth.record_layout(H, I, bits)
            codes_gu = I * H * bits // 8
            sb_gu = I * (H // 64) * 4
            codes_dn = H * I * bits // 8
            sb_dn = H * (I // 64) * 4
            for npass in (1, 2, 4):
                nch = _nch(H, bits)
                if nch >= 4 and npass > 1:
                    continue
                mc, ms = _max_offsets(I, H, bits, nch, npass)
                assert mc <= codes_gu and ms <= sb_gu, (H, I, bits, npass, mc, ms)
                assert lay.gate_codes + mc <= lay.up_codes and lay.up_sb + ms <= lay.down_sb
                nch = _nch(I, bits)
                if nch >= 4 and npass > 1:
                    continue
                mc, ms = _max_offsets(H, I, bits, nch, npass)
                assert mc <= codes_dn and ms <= sb_dn, (H, I, bits, npass, mc, ms)
                assert lay.down_sb + ms <= lay.total
