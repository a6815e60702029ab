"""Pins for the oracle's block-scaled fp8 payload (E4M3 codes + one float32 scale per
128 elements; the format reading is documented in oracle/__init__.py).

The codec is pinned against the field definitions by hand-derived codes, by an
exhaustive nearest-value brute force over all 254 finite codes, by the exact
midpoints between neighbouring codes (round half to even), and by round trips; the
block quantizer by its defining properties (the block maximum lands on +-448, the
error stays within half a step, zero blocks stay zero)."""
import numpy as np
import pytest

import oracle


def test_e4m3_hand_derived_codes():
    # value = (1 + m/8) * 2^(e-7) for exponent field e >= 1, (m/8) * 2^-6 for e = 0
    cases = [
        (448.0, 0x7E),          # e=15, m=6: 1.75 * 2^8, the largest finite value
        (-448.0, 0xFE),
        (1.0, 0x38),            # e=7, m=0
        (0.5, 0x30),            # e=6
        (3.0, 0x44),            # 1.5 * 2^1: e=8, m=4
        (2.0 ** -6, 0x08),      # smallest normal: e=1, m=0
        (2.0 ** -9, 0x01),      # smallest subnormal: m=1
        (7 * 2.0 ** -9, 0x07),  # largest subnormal
        (0.0, 0x00),
        (-0.0, 0x80),
        (1e9, 0x7E),            # saturates
        (464.0, 0x7E),          # between 448 and the NaN pattern: saturates
        (-1e9, 0xFE),
    ]
    got = oracle.e4m3_encode(np.array([v for v, _ in cases], dtype=np.float32))
    assert [int(c) for c in got] == [c for _, c in cases]


def test_e4m3_decode_table():
    vals = oracle.e4m3_decode(np.arange(256))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    finite = np.delete(np.arange(256), [0x7F, 0xFF])
    assert not np.any(np.isnan(vals[finite]))
    pos = vals[1:0x7F]
    assert np.all(np.diff(pos) > 0)                  # codes 1..126 strictly increasing
    assert pos[0] == 2.0 ** -9 and pos[-1] == 448.0
    assert np.array_equal(vals[0x80:0xFF], -vals[0:0x7F])


def test_e4m3_round_trip_every_code():
    codes = np.delete(np.arange(256), [0x7F, 0xFF]).astype(np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_e4m3_midpoints_round_to_even():
    vals = oracle.e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)
    for c in range(0, 0x7E):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)           # exact: <= 5 significant bits
        assert float(mid) == (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert int(oracle.e4m3_encode([mid])[0]) == want, c
        assert int(oracle.e4m3_encode([-mid])[0]) == 0x80 | want, c


def test_e4m3_nearest_by_brute_force():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-460, 460, 4000), rng.normal(0, 1, 4000),
                        rng.normal(0, 0.01, 2000)]).astype(np.float32)
    codes = oracle.e4m3_encode(v)
    table = oracle.e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)   # non-negative finite
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    best = np.abs(table[None, :] - a[:, None]).min(axis=1)
    got = oracle.e4m3_decode(codes).astype(np.float64)
    assert np.all(np.abs(np.abs(got) - a) == best)
    assert np.all((codes >= 0x80) == np.signbit(v))


def test_block_quantizer_properties():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, (6, 512)).astype(np.float32)
    x[2, 128:256] = 0.0                                   # an all-zero block
    x[3, :128] = 0.0
    x[3, 5] = -3.5                                        # a single non-zero element
    x[4] *= 1e-3
    codes, scales = oracle.quantize_blocks_fp8(x)
    assert codes.dtype == np.uint8 and scales.shape == (6, 4)
    amax = np.abs(x.reshape(6, 4, 128)).max(axis=2)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    assert scales[2, 1] == 0 and np.all(codes[2, 128:256] == 0)
    assert codes[3, 5] == 0xFE                           # the block max lands on -448
    back = oracle.dequantize_blocks_fp8(codes, scales)
    # within half a step: 2^-4 relative for normal codes, half the subnormal step else
    step = np.repeat(scales, 128, axis=1).astype(np.float64) * 2.0 ** -10
    err = np.abs(back.astype(np.float64) - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, step) * (1 + 1e-6))
    # every block's largest magnitude maps to +-448 exactly
    cb = codes.reshape(6, 4, 128)
    for t in range(6):
        for b in range(4):
            if scales[t, b] > 0:
                i = np.argmax(np.abs(x.reshape(6, 4, 128)[t, b]))
                assert cb[t, b, i] & 0x7F == 0x7E
