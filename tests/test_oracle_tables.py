"""Pins for the oracle's decode tables (CPU only).

Each table is compared with an implementation that is not the oracle's:
torch's float8_e4m3fn / float8_e8m0fnu dtypes (byte views), numpy's float16,
and the OCP MX E2M1 value list stored in tests/golden.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden_rows


def test_e4m3_table_matches_torch_fn_dtype():
    ours = oracle.e4m3_table()
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zero of code 0x80
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_page_facts():
    # RIGEL summary, section 3: saturates at +-448, no infinity encoding.
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert not np.isinf(t).any()
    assert sorted(np.flatnonzero(np.isnan(t)).tolist()) == [0x7F, 0xFF]
    # the OCP FN variant (bias 7), not the bias-8 "fnuz" variant: 0x38 is 1.0
    assert t[0x38] == 1.0 and t[0x01] == 2.0 ** -9


def test_e2m1_table_matches_golden():
    rows = read_golden_rows("e2m1_values.txt")
    assert len(rows) == 16
    t = oracle.e2m1_table()
    for code, val in rows:
        c = int(code, 16)
        v = float(val)
        assert t[c] == v
        assert math.copysign(1.0, t[c]) == math.copysign(1.0, v)


def test_e2m1_is_subset_of_e4m3():
    # every E2M1 magnitude is exactly representable in E4M3 (torch table)
    e4 = set(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
             .to(torch.float64).numpy()[:0x7F].tolist())
    for v in oracle.e2m1_table():
        assert abs(v) in e4


def test_ue8m0_table_matches_torch_e8m0_dtype():
    ours = oracle.ue8m0_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_fp16_decode_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    # sample the whole range with a stride plus all specials and subnormals
    idx = np.concatenate([np.arange(0, 65536, 97), np.arange(0, 1024), np.arange(31 * 1024, 32 * 1024),
                          np.arange(32768, 32768 + 1024), np.arange(63 * 1024, 64 * 1024)])
    for i in np.unique(idx):
        o = oracle.fp16_value(int(i))
        r = ref[i]
        if np.isnan(r):
            assert math.isnan(o)
        else:
            assert o == r and math.copysign(1.0, o) == math.copysign(1.0, r)
