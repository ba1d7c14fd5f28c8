"""Host emulation of the decode streaming kernel's whole-line weight loads.

An MFMA 16x16x32 operand needs 16 weight rows in one instruction (lane
c16 + 16 q holds row c16, 16-byte chunk q of a 64-byte block), so a direct
load covers half of each 128-byte line. The kernel instead reads each line of
a 16-row tile with two loads of 8 whole rows (`line_offsets` in decode.hip)
and forms the operands with DPP moves (`line_pick`: a bank-masked move for the
first half of the line, a row rotation by 8 and a bank-masked move for the
second). These tests replay that lane map on the host, lane by lane, and check
that every load reads 8 whole lines and that every operand lane receives the
chunk the MFMA layout needs. The GPU parity tests check the kernel itself.
"""
import pytest

LANES = 64


def dpp(old, src, ctrl, bank_mask):
    """v_mov_b32_dpp with row_mask 0xF: quad_perm identity (0xE4) or
    row_ror:8 (0x128); lanes outside bank_mask keep `old`."""
    out = []
    for lane in range(LANES):
        c16, row0 = lane & 15, lane & ~15
        src_lane = lane if ctrl == 0xE4 else row0 | ((c16 + 8) & 15)
        out.append(src[src_lane] if (bank_mask >> (c16 >> 2)) & 1 else old[lane])
    return out


def line_pick(a, b, hi):
    if not hi:
        return dpp(a, b, 0xE4, 0xC)
    r = dpp(a, a, 0x128, 0xF)
    return dpp(r, b, 0x128, 0xC)


def line_loads(qs, hs, line_base):
    """(row, byte) each lane loads from the line at line_base: line_offsets
    with row0 = 0 gives lane (c16, q) chunk qs q + hs (first load, c16 >= 8;
    second load, c16 < 8) or qs q (otherwise); bf16 rows: qs = 16, hs = 64."""
    first = [((lane & 15) & 7, line_base + qs * (lane >> 4) + (hs if (lane & 15) >= 8 else 0)) for lane in range(LANES)]
    second = [(((lane & 15) & 7) + 8, line_base + qs * (lane >> 4) + (hs if (lane & 15) < 8 else 0)) for lane in range(LANES)]
    return first, second


@pytest.mark.parametrize("line", [0, 1])
def test_each_load_reads_eight_whole_lines(line):
    for load in line_loads(16, 64, 128 * line):
        rows = {}
        for row, byte in load:
            rows.setdefault(row, set()).add(byte)
        assert len(rows) == 8
        for chunks in rows.values():
            assert chunks == {128 * line + 16 * c for c in range(8)}


@pytest.mark.parametrize("line", [0, 1])
def test_bf16_operands_match_the_mfma_layout(line):
    a, b = line_loads(16, 64, 128 * line)
    for hi in (0, 1):
        t = 2 * line + hi  # MFMA t of the 256-byte k-step: bytes [64 t, 64 t + 64) of each row
        got = line_pick(a, b, hi)
        for lane in range(LANES):
            assert got[lane] == (lane & 15, 64 * t + 16 * (lane >> 4)), (t, lane)


def test_a_wrong_rotation_is_caught():
    # the check is not vacuous: picking the second half without the rotation
    a, b = line_loads(16, 64, 0)
    got = dpp(a, b, 0xE4, 0xC)  # the hi = 0 pick used for hi = 1
    assert any(got[lane] != (lane & 15, 64 + 16 * (lane >> 4)) for lane in range(LANES))
