"""The K/V tile loads of the attention kernel, replayed on the CPU: for every
head dim and for tiles of 32, 64 and 128 keys, no lane may read a row past
the tile or write an LDS unit past the tile, and every unit of the tile must
be written exactly once.  The operand reads must stay inside the buffer
(tile plus slack).

The replay restates the kernel's index arithmetic (the loads of `dma_tile`:
wave w of the loading group issues load j to units 64 (4 j + w) .. +63, lane
i the unit 64 (4 j + w) + i, which holds row p / kOct of the tile).  The
lines it restates are read from the kernel source and must be present there
verbatim, so a change to the kernel's guard fails this test until the replay
follows it.  A 32-key tile at an odd number of 16-byte units per row (for
example d = 72) is not a whole number of 64-unit wave loads: without the
per-lane guard the last wave load writes past the tile, which the replay
shows as well."""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "attention_attn_block_amd", "csrc", "attn_bf16_kernel.h")

GUARD_LINES = [
    "const int first_unit = 64 * ((kDmaThreads / 64) * j + wvl);",
    "const bool lane_in = (kTileUnits % 64 == 0) || dtid + kDmaThreads * j < kTileUnits;",
    "if (kTileUnits % kDmaThreads == 0 || (first_unit < kTileUnits && lane_in)) {",
    "const int pu = dtid + kDmaThreads * j;",
    "constexpr int kBufUnits = kTileUnits + 16;",
    "static constexpr int kKLoads = (kKItems + kDmaThreads - 1) / kDmaThreads;",
]


def source():
    return open(SRC).read()


def constant(name):
    m = re.search(rf"constexpr int {name} = (\d+);", source())
    assert m, name
    return int(m.group(1))


def test_guard_lines_present():
    txt = " ".join(source().split())
    for line in GUARD_LINES:
        assert " ".join(line.split()) in txt, line


def replay(D, kBc, kDmaThreads, lane_guard=True):
    """Return (writes, bad) for one tile: the LDS units written (with the
    tile row each one reads) and a list of violations."""
    kOct = D // 8
    kTileUnits = kBc * kOct
    kBufUnits = kTileUnits + 16
    kKLoads = (kBc * kOct + kDmaThreads - 1) // kDmaThreads
    written = {}
    bad = []
    for wv in range(kDmaThreads // 64):
        for lane in range(64):
            dtid = 64 * wv + lane
            for j in range(kKLoads):
                first_unit = 64 * ((kDmaThreads // 64) * j + wv)
                lane_in = (kTileUnits % 64 == 0) or (dtid + kDmaThreads * j < kTileUnits)
                if not lane_guard:
                    lane_in = True
                if not (kTileUnits % kDmaThreads == 0 or (first_unit < kTileUnits and lane_in)):
                    continue
                unit = first_unit + lane
                pu = dtid + kDmaThreads * j
                row = pu // kOct
                if unit != pu:
                    bad.append(("lds unit differs from the unit the source offset names", unit, pu))
                if unit >= kTileUnits:
                    bad.append(("write past the tile", unit, kTileUnits))
                if unit >= kBufUnits:
                    bad.append(("write past the buffer", unit, kBufUnits))
                if row >= kBc:
                    bad.append(("read past the tile's rows", row, kBc))
                written[unit] = written.get(unit, 0) + 1
    for u in range(kTileUnits):
        if written.get(u, 0) != 1:
            bad.append(("unit not written exactly once", u, written.get(u, 0)))
    return written, bad


HEAD_DIMS = list(range(8, 129, 8))


@pytest.mark.parametrize("kBc", [32, 64, 128])
@pytest.mark.parametrize("D", HEAD_DIMS)
def test_tile_loads_stay_in_bounds(D, kBc):
    _, bad = replay(D, kBc, constant("kDmaThreads"))
    assert not bad, bad[:5]


def test_built_tile_size():
    assert constant("kBc") == 64 and constant("kDmaThreads") == 256


def test_replay_catches_a_missing_lane_guard():
    """The wave-level guard alone writes past 32-key tiles at odd unit counts."""
    _, bad = replay(72, 32, constant("kDmaThreads"), lane_guard=False)
    assert any(b[0] == "write past the buffer" for b in bad)
    assert any(b[0] == "read past the tile's rows" for b in bad)


def v9_slot_table():
    txt = source()
    body = txt[txt.index("int v9_slot(int r"):]
    body = body[:body.index("return")]
    words = [int(w, 16) for w in re.findall(r"0x([0-9a-f]+)ull", body)]
    return [[(w >> (4 * i)) & 15 for i in range(9)] for w in words]


def ones_skew():
    m = re.search(r"constexpr int kOnesSkew = (\d+);", source())
    assert m
    return int(m.group(1))


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_operand_reads_stay_in_buffer(D):
    """K operand reads (row kt * 32 + l32, unit (2c + hi) ^ swz mod kOct) and
    the transposing V reads (rows 4 (q / 2) + i / 4 of each 8-key half chunk,
    units 4 dt + 2 (q % 2) + (i % 4) / 2, swizzled) of a 64-key tile, every
    chunk: all inside the tile plus its 16-unit slack.  When d is not a
    multiple of 32, the reads of units past the row (padding rows of O^T) go
    to the ones region after the four buffers; from either V buffer they must
    land inside it."""
    kBc = constant("kBc")
    kOct = D // 8
    kTileUnits = kBc * kOct
    kBufUnits = kTileUnits + 16
    ones_row = D % 32 != 0
    assert ("constexpr bool kOnesRow = (D % 32) != 0;" in source())
    ones_units = kBufUnits + ones_skew() + 56 * kOct + 1 if ones_row else 0
    for vbuf in (0, 1):                       # V buffers sit at units (2 + vbuf) * kBufUnits
        base = (2 + vbuf) * kBufUnits
        for lane in range(64):
            q, i = lane >> 4, lane & 15
            for dt in range((D + 31) // 32):
                u = 4 * dt + 2 * (q & 1) + ((i & 3) >> 1)
                if not (ones_row and u >= kOct):
                    continue
                for ch in range(kBc // 16):
                    for up in (0, 8):
                        first = base * 8 + (2 * kBufUnits + ones_skew()) * 8 + 4 * (i & 1) \
                            + (16 * ch + up) * kOct * 8
                        assert 4 * kBufUnits * 8 <= first
                        assert first + 3 < (4 * kBufUnits + ones_units) * 8, (D, vbuf, lane, dt, ch)
    kChunks = (D + 15) // 16
    kDTiles = (D + 31) // 32
    kCH = kBc // 16
    v9 = v9_slot_table()
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        for kt in range(kBc // 32):
            for c in range(kChunks):
                unit = (kt * 32 + l32) * kOct + (2 * c + hi) % kOct   # swizzle permutes within the row
                assert unit < kTileUnits
        q, i = lane >> 4, lane & 15
        v_row = 4 * (q >> 1) + (i >> 2)
        for dt in range(kDTiles):
            u = 4 * dt + 2 * (q & 1) + ((i & 3) >> 1)
            if ones_row and u >= kOct:
                continue                      # checked above: the ones region
            if kOct == 9:
                slot = v9[v_row & 3][u]
            elif kOct in (8, 16):
                sv = 4 * (v_row & 3) if kOct == 16 else 4 * ((v_row >> 1) & 1)
                slot = u ^ sv
            else:
                slot = u
            for ch in range(kCH):
                for up in (0, 8):
                    row = v_row + 16 * ch + up
                    last_elem = (row * kOct + slot) * 8 + 4 * (i & 1) + 3
                    assert last_elem < kBufUnits * 8, (D, lane, dt, ch, up)
