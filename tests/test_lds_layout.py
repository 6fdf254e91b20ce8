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
    words = []
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        if half_tail and hi:
            words.append([])
            continue
        row = kt * 32 + l32
        base = (row * kOct + slot(row, 2 * c + hi)) * 4                # 16-byte unit -> 4 words
        words.append([base, base + 1, base + 2, base + 3])
    return words


def test_v9_tables_are_inverse_permutations():
    slot, unit = v9_tables()
    for r in range(4):
        assert sorted(slot[r]) == list(range(9))
        assert all(unit[r][slot[r][u]] == u for u in range(9))


def test_d72_v_reads_conflict_free():
    slot_t, _ = v9_tables()
    slot = lambda r, u: slot_t[r & 3][u if u < 9 else 8]
    for dt in range(3):
        for row0 in range(0, 64, 8):
            assert extra_cycles(v_pass_words(9, slot, dt, row0), 32) == 0, (dt, row0)
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
