"""Host check of the integer-weight remap tables (CPU only).

The kernels turn INT4 codes into E4M3 codes and pairs of INT2 codes into
bytes of two E2M1 codes with byte permutes (v_perm_b32) over two 8-byte
tables whose results are XORed.  This test reads the table constants from the
device header, runs the same steps on the CPU with the instruction's
documented byte selection (selector 0-7: a source byte, 8-11: bit 7 of source
byte 1, 3, 5, 7 repeated, 12: 0x00, 13-15: 0xFF), and checks every code and
many random words against the oracle's value tables: the remapped float code
must have the integer code's value.
"""
import os
import re

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "block_scaled_precision_mxgemm_amd", "csrc", "mxg_device.h")


def _tables(func: str):
    src = open(HEADER).read()
    body = src[src.index("void " + func + "("):]
    body = body[:body.index("\n}\n")]
    vals = dict(re.findall(r"\b([LH][01]) = (0x[0-9A-Fa-f]+)u", body))
    return [int(vals[k], 16) for k in ("L0", "L1", "H0", "H1")]


def _perm(s0: int, s1: int, sel: int) -> int:
    src = [(s1 >> (8 * i)) & 0xFF for i in range(4)] + [(s0 >> (8 * i)) & 0xFF for i in range(4)]
    out = 0
    for i in range(4):
        k = (sel >> (8 * i)) & 0xFF
        if k >= 13:
            v = 0xFF
        elif k == 12:
            v = 0
        elif k >= 8:
            v = 0xFF if src[2 * (k - 8) + 1] & 0x80 else 0
        else:
            v = src[k]
        out |= v << (8 * i)
    return out


def _remap(x: int, t):
    s = x >> 4
    lo = _perm(s, x, 0x05010400) & 0x0F0F0F0F
    hi = _perm(s, x, 0x07030602) & 0x0F0F0F0F
    look = lambda i: _perm(t[1], t[0], i) ^ _perm(t[3], t[2], i ^ 0x08080808)  # noqa: E731
    return look(lo), look(hi)


def _words(seed=7, n=4000):
    rng = np.random.default_rng(seed)
    fixed = [0, 0xFFFFFFFF, 0x88888888, 0x77777777, 0x76543210, 0xFEDCBA98, 0x89ABCDEF, 0x01234567]
    # every nibble value at every position
    fixed += [(v * 0x11111111) & 0xFFFFFFFF for v in range(16)]
    return fixed + [int(v) for v in rng.integers(0, 2 ** 32, n, dtype=np.uint64)]


def test_int4_remap_gives_e4m3_of_the_same_value():
    t = _tables("int4x8_to_e4m3")
    e4m3 = oracle.e4m3_table()
    int4 = oracle.int4_table()
    for x in _words():
        lo, hi = _remap(x, t)
        out = [(lo >> (8 * i)) & 0xFF for i in range(4)] + [(hi >> (8 * i)) & 0xFF for i in range(4)]
        for i in range(8):
            n = (x >> (4 * i)) & 15
            assert e4m3[out[i]] == int4[n], (hex(x), i, hex(out[i]))


def test_int2_remap_gives_e2m1_of_the_same_value():
    t = _tables("int2x16_to_e2m1")
    e2m1 = oracle.e2m1_table()
    int2 = oracle.int2_table()
    for x in _words(seed=11):
        lo, hi = _remap(x, t)
        nib = [(lo >> (4 * i)) & 15 for i in range(8)] + [(hi >> (4 * i)) & 15 for i in range(8)]
        for i in range(16):
            c = (x >> (2 * i)) & 3
            assert e2m1[nib[i]] == int2[c], (hex(x), i, nib[i])


def test_table_error_is_caught():
    # a planted table mistake (one byte of the negative half) must fail
    t = _tables("int4x8_to_e4m3")
    t[2] ^= 0x00000100
    e4m3 = oracle.e4m3_table()
    int4 = oracle.int4_table()
    lo, _ = _remap(0x00000009, t)
    assert e4m3[lo & 0xFF] != int4[9]
