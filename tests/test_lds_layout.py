"""LDS layouts of the attention kernel's K/V tiles, checked on the CPU with a
model of the 64 four-byte LDS banks: the operand reads of one hardware pass
must touch each bank with at most one distinct word (16 lanes per pass for
16-byte reads, 32 lanes for the 8-byte transposing reads).

The address arithmetic below restates the kernel's read offsets (K: lane l32
reads row kt*32 + l32 at column 2c + hi; V: lane group q = lane / 16 reads
rows 4 (q / 2) + i / 4 and units 4 dt + 2 (q % 2) + (i % 4) / 2).  The d = 72
placement tables are read from the kernel source itself."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "attention_attn_block_amd", "csrc", "attn_bf16_kernel.h")
BANKS = 64


def v9_tables():
    txt = open(SRC).read()
    out = []
    for fn in ("v9_slot", "v9_unit"):
        body = txt[txt.index(f"int {fn}(int r"):]
        body = body[:body.index("return")]
        words = [int(w, 16) for w in re.findall(r"0x([0-9a-f]+)ull", body)]
        assert len(words) == 4
        out.append([[(w >> (4 * i)) & 15 for i in range(9)] for w in words])
    return out


def extra_cycles(lane_words, lanes_per_pass):
    extra = 0
    for p0 in range(0, 64, lanes_per_pass):
        banks = {}
        for lane in range(p0, p0 + lanes_per_pass):
            for w in lane_words[lane]:
                banks.setdefault(w % BANKS, set()).add(w)
        if banks:
            extra += max(len(s) for s in banks.values()) - 1
    return extra


def v_pass_words(kOct, slot, dt, row0):
    words = []
    for lane in range(64):
        q, i = lane >> 4, lane & 15
        row = row0 + 4 * (q >> 1) + (i >> 2)
        unit = 4 * dt + 2 * (q & 1) + ((i & 3) >> 1)
        elem = (row * kOct + slot(row, unit)) * 8 + 4 * (i & 1)      # bf16 elements
        words.append([elem // 2, elem // 2 + 1])                       # two 4-byte words
    return words


def k_pass_words(kOct, slot, kt, c, half_tail):
    """K operand reads: lane (l32, hi) reads unit slot(row, 2c + hi) mod kOct
    of row kt * 32 + l32.  In a half-filled last chunk (half_tail) the upper
    half-wave's unit index wraps to a real unit of the row (its Q operand is
    zero), so every lane reads."""
    words = []
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        row = kt * 32 + l32
        base = (row * kOct + slot(row, 2 * c + hi) % kOct) * 4         # 16-byte unit -> 4 words
        words.append([base, base + 1, base + 2, base + 3])
    return words


def test_v9_tables_are_inverse_permutations():
    slot, unit = v9_tables()
    for r in range(4):
        assert sorted(slot[r]) == list(range(9))
        assert all(unit[r][slot[r][u]] == u for u in range(9))


def ones_skew():
    txt = open(SRC).read()
    m = re.search(r"constexpr int kOnesSkew = (\d+);", txt)
    assert m
    return int(m.group(1))


def v_pass_words_ones(kOct, slot, dt, row0):
    """As v_pass_words, with the reads of padding rows (unit >= kOct) sent to
    the ones region: two buffers (of 64 kOct + 16 units) plus the skew past
    the V buffer, at the pass's chunk offset (row0 rows of kOct units)."""
    pad = 2 * (64 * kOct + 16) + ones_skew()
    words = []
    for lane in range(64):
        q, i = lane >> 4, lane & 15
        row = row0 + 4 * (q >> 1) + (i >> 2)
        unit = 4 * dt + 2 * (q & 1) + ((i & 3) >> 1)
        if unit >= kOct:
            elem = (pad + row0 * kOct) * 8 + 4 * (i & 1)
        else:
            elem = (row * kOct + slot(row, unit)) * 8 + 4 * (i & 1)
        words.append([elem // 2, elem // 2 + 1])
    return words


def test_d72_v_reads_conflict_free():
    slot_t, _ = v9_tables()
    slot = lambda r, u: slot_t[r & 3][u]
    for dt in range(3):
        for row0 in range(0, 64, 8):
            assert extra_cycles(v_pass_words_ones(9, slot, dt, row0), 32) == 0, (dt, row0)
    # the plain row-major layout it replaces does conflict
    plain = lambda r, u: u
    assert sum(extra_cycles(v_pass_words(9, plain, dt, 0), 32) for dt in range(2)) > 0


def test_d72_k_reads_conflict_free():
    ident = lambda r, g: g
    for kt in range(2):
        for c in range(5):
            assert extra_cycles(k_pass_words(9, ident, kt, c, c == 4), 16) == 0, (kt, c)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_d128_xor_swizzles_conflict_free(kind):
    if kind == "k":
        sw = lambda r, g: g ^ (r & 15)
        for kt in range(2):
            for c in range(8):
                assert extra_cycles(k_pass_words(16, sw, kt, c, False), 16) == 0
    else:
        sw = lambda r, u: u ^ (4 * (r & 3))
        for dt in range(4):
            assert extra_cycles(v_pass_words(16, sw, dt, 0), 32) == 0


def test_staged_fp32_output_layout():
    """The fp32 epilogue at d = 128 passes each wave's 32 rows through an 8 KB
    LDS slice, two 32-column tiles (64 columns, 16 units of 16 bytes) at a
    time: lane (l32, hi) writes unit u = 8 dd + 2 q4 + hi (columns 4u..4u+3 of
    the half) of row l32 at slot l32 * 16 + (u ^ (l32 % 16)); read pass it,
    lane L takes unit c = L % 16 of row r = 4 it + L / 16 from slot
    r * 16 + (c ^ (r % 16)) and stores it to global memory.  Checked: the
    writes fill the slice once, every read gets row r's columns 4c..4c+3,
    neither side meets a bank twice in a 16-lane pass, each store instruction
    covers whole 128-byte lines, and the eight slices fit the tile buffers."""
    txt = open(SRC).read()
    assert "slice[l32 * 16 + (u ^ (l32 & 15))]" in txt
    assert "slice[r * 16 + (c ^ (r & 15))]" in txt
    assert "const int u = dd * 8 + 2 * q4 + hi;" in txt
    assert "const int r = it * 4 + (lane >> 4), c = lane & 15;" in txt
    assert 8 * 512 <= 4 * (64 * 16 + 16)
    holds = {}
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        for dd in range(2):
            for q4 in range(4):
                u = dd * 8 + 2 * q4 + hi
                slot = l32 * 16 + (u ^ (l32 & 15))
                assert slot not in holds
                holds[slot] = (l32, 4 * u)
    assert sorted(holds) == list(range(512))
    # one write instruction per (dd, q4): 16-byte stores, 16 lanes per pass
    for dd in range(2):
        for q4 in range(4):
            words = []
            for lane in range(64):
                l32, hi = lane & 31, lane >> 5
                u = dd * 8 + 2 * q4 + hi
                s = l32 * 16 + (u ^ (l32 & 15))
                words.append([4 * s + k for k in range(4)])
            assert extra_cycles(words, 16) == 0, (dd, q4)
    for it in range(8):
        words, lines = [], set()
        for lane in range(64):
            r, c = it * 4 + (lane >> 4), lane & 15
            s = r * 16 + (c ^ (r & 15))
            assert holds[s] == (r, 4 * c)
            words.append([4 * s + k for k in range(4)])
            byte = r * 128 * 4 + 4 * c * 4            # global offset inside the half, row stride 512 B
            lines.add(byte // 128)
        assert extra_cycles(words, 16) == 0, it
        assert len(lines) == 8                         # 64 lanes x 16 B = 8 whole lines


def test_staged_bf16_output_layout_d72():
    """The bf16 epilogue at d = 72 writes each lane's pieces (4 bf16 at
    columns d0 = 32 dt + 8 q4 + 4 hi < 72 of row l32) into a linear copy of
    the wave's 32 output rows and then copies that out in 16-byte units.
    Checked: the pieces cover every row's 72 columns exactly once, a unit
    never straddles two rows (row = unit / 9), the units cover the copy once,
    and eight copies fit the four tile buffers."""
    txt = open(SRC).read()
    assert "slice + (l32 * D + d0) * 2" in txt
    assert "q_base + unit / (D / 8) < Nq" in txt
    D, k_dtiles = 72, 3
    cover = {}
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        for dt in range(k_dtiles):
            for q4 in range(4):
                d0 = dt * 32 + 8 * q4 + 4 * hi
                if d0 < D:
                    for e in range(4):
                        key = (l32, d0 + e)
                        assert key not in cover
                        cover[key] = (l32 * D + d0 + e) * 2
    assert sorted(cover) == [(r, c) for r in range(32) for c in range(D)]
    assert sorted(cover.values()) == list(range(0, 32 * D * 2, 2))   # a linear copy
    units = 32 * D * 2 // 16
    for unit in range(units):
        first, last = unit * 16 // 2, unit * 16 // 2 + 7                # bf16 elements
        assert first // D == last // D == unit // (D // 8)
    k_buf_units = 64 * (D // 8) + 16
    assert 8 * 32 * D * 2 <= 4 * k_buf_units * 16
