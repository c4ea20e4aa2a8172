"""Pins of the oracle's e4m3 codec against the format definition and an independent
implementation (torch's float8_e4m3fn cast)."""
import math
import os

import numpy as np
import torch

from oracle import e4m3_decode, e4m3_encode, e4m3_table, E4M3_MAX

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def test_decode_matches_published_code_points():
    for code, val in _golden_rows():
        got = float(e4m3_decode(code))
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_table_shape_of_format():
    t = e4m3_table()
    finite = t[~np.isnan(t)]
    assert len(finite) == 254
    assert np.nanmax(t) == E4M3_MAX == 448.0
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # codes 0..0x7E ascend
    assert np.array_equal(t[0x80:0xFF], -pos)       # sign-magnitude


def test_encode_decode_identity_on_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def _bruteforce(x):
    """Nearest finite e4m3 value by exhaustive search, ties to the even code."""
    pos = e4m3_table()[:0x7F]
    out = np.empty(len(x), dtype=np.uint8)
    for i, xv in enumerate(np.asarray(x, dtype=np.float64)):
        a = abs(xv)
        dist = np.abs(pos - a)
        best = np.flatnonzero(dist == dist.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if math.copysign(1, xv) < 0 else 0)
    return out


def _probe_values():
    rng = np.random.default_rng(0)
    t = e4m3_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    vals = []
    for base in np.concatenate([t, mids]).astype(np.float32):
        u = np.array([base], dtype=np.float32).view(np.uint32)[0]
        for dlt in range(-3, 4):
            vals.append(np.array([max(int(u) + dlt, 0)], dtype=np.uint32).view(np.float32)[0])
    # a strided sweep over every fp32 bit pattern in [0, 480]
    top = np.array([480.0], dtype=np.float32).view(np.uint32)[0]
    sweep = np.arange(0, int(top) + 1, 104729, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([np.array(vals, dtype=np.float32), sweep,
                           rng.uniform(0, 480, 2000).astype(np.float32),
                           np.array([464.0, 470.0, 479.9, 1e6, 1e-30], dtype=np.float32)])
    return np.concatenate([vals, -vals])


def test_encode_equals_bruteforce_nearest_even_saturating():
    x = _probe_values()
    assert np.array_equal(e4m3_encode(x), _bruteforce(x))


def test_rounding_ties_and_saturation():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even mantissa wins
    assert e4m3_encode(np.float32(1.0625)) == 0x38
    assert e4m3_encode(np.float32(1.1875)) == 0x3A        # between 0x39 and 0x3A
    assert e4m3_encode(np.float32(2.0 ** -10)) == 0x00     # half the smallest subnormal
    assert e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02
    assert e4m3_encode(np.float32(464.0)) == 0x7E          # saturates to 448
    assert e4m3_encode(np.float32(-1e9)) == 0xFE
    assert e4m3_encode(np.float32(np.nan)) == 0x7F


def test_agrees_with_torch_float8_cast_below_overflow():
    x = _probe_values()
    x = x[np.abs(x) < 464.0]
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)
