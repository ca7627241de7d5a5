"""Pins for the oracle's number formats and roundings (CPU only).

The pages name the formats (E4M3FN weights in ninfer PR #167 "Measured"; E2M1
codes with E4M3 per-16 scales in ninfer PR #160) but print no tables, so the
oracle's codecs are pinned against what the formats' definitions fix:
torch's float8_e4m3fn decode and cast (a library routine), the E2M1 value
set, a brute-force nearest-value search, and exact rational rounding.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def all_finite_bf16_as_f32():
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    return f[np.isfinite(f)]


def brute_nearest(values, table_codes, table_vals):
    """Nearest representable magnitude by exhaustive search; ties to the even
    code; the largest value absorbs everything above it."""
    # Anything above twice the largest value is nearest to the largest value;
    # clipping keeps every fp64 distance below exact (no absorption of the
    # table values into a huge magnitude).
    top = float(table_vals.max())
    a = np.minimum(np.abs(values.astype(np.float64)), 2 * top)[:, None]
    d = np.abs(a - table_vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer an even code
    even = (table_codes[None, :] % 2 == 0)
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    return table_codes[idx]


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert math.copysign(1.0, ours[0x80]) == -1.0
    # magnitudes strictly increase with the code, so the encoder's search is valid
    assert np.all(np.diff(ours[:0x7F]) > 0)


def test_e2m1_decode_is_the_format_value_set():
    # 1 sign, 2 exponent, 1 mantissa bit: the eight magnitudes of the format
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ours = oracle.E2M1_TABLE
    assert list(ours[:8]) == mags
    assert list(-ours[8:]) == mags
    assert math.copysign(1.0, ours[8]) == -1.0
    # every E2M1 value is also an E4M3 value (a format nesting the tables must respect)
    e4 = set(oracle.E4M3_TABLE[~np.isnan(oracle.E4M3_TABLE)].tolist())
    assert all(v in e4 for v in ours)


def test_e4m3_encode_round_trip_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


def test_e2m1_encode_round_trip_every_code():
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c


def _oracle_e4m3_codes(vals):
    return np.array([oracle.e4m3_encode(float(v)) for v in vals], dtype=np.int64)


def _oracle_e2m1_codes(vals):
    return np.array([oracle.e2m1_encode(float(v)) for v in vals], dtype=np.int64)


def _neighbourhood(points):
    """Each point and its float32 neighbours one ulp either side."""
    p = np.asarray(points, dtype=np.float32)
    return np.concatenate([p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(-np.inf))])


def test_e4m3_encode_vs_brute_force_all_bf16():
    vals = all_finite_bf16_as_f32()
    codes = np.arange(127)
    ref = brute_nearest(vals, codes, oracle.E4M3_TABLE[:127]) | np.where(np.signbit(vals), 0x80, 0)
    # the oracle's quantizer with a unit scale encodes x / 1 = x: vectorised path
    x16 = (vals.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    q = oracle.quantize_rows_with_scale(x16, np.float32(1.0))[0]
    assert np.array_equal(q.astype(np.int64), ref)


def test_e4m3_encode_vs_brute_force_midpoints():
    mags = oracle.E4M3_TABLE[:127]
    mids = (mags[:-1] + mags[1:]) / 2
    pts = _neighbourhood(np.concatenate([mids, -mids, [448.0, 464.0, 500.0, 1e30, 2.0 ** -10, 2.0 ** -11]]))
    ref = brute_nearest(pts, np.arange(127), mags) | np.where(np.signbit(pts), 0x80, 0)
    assert np.array_equal(_oracle_e4m3_codes(pts), ref)


def test_e4m3_encode_matches_torch_cast_below_saturation():
    vals = all_finite_bf16_as_f32()
    vals = vals[np.abs(vals) < 464]
    mags = oracle.E4M3_TABLE[:127]
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([vals, _neighbourhood(np.concatenate([mids, -mids]))])
    ref = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(_oracle_e4m3_codes(vals), ref)


def test_e4m3_saturates_and_keeps_sign():
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(464.0) == 0x7E      # tie between 448 and 512: even code
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9: even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 (x 2^-9): even


def test_e2m1_encode_vs_brute_force():
    mags = oracle.E2M1_TABLE[:8]
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([all_finite_bf16_as_f32(),
                           _neighbourhood(np.concatenate([mids, -mids, [6.0, 7.0, 8.0]]))])
    ref = brute_nearest(vals, np.arange(8), mags) | np.where(np.signbit(vals), 0x8, 0)
    assert np.array_equal(_oracle_e2m1_codes(vals), ref)
    # ties: 0.25 -> 0, 0.75 -> 1.0 (code 2), 1.25 -> 1.0, 2.5 -> 2, 5 -> 4
    assert [oracle.e2m1_encode(v) for v in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0, 2, 2, 4, 4, 6, 6]


def _bf16_exact_round(y: float) -> int:
    """Nearest bf16 to the exact value of y by comparing rational distances to
    the bf16 neighbours; ties to the even bit pattern."""
    fy = Fraction(y)
    sign = 0x8000 if math.copysign(1.0, y) < 0 else 0
    a = abs(fy)
    # candidates: bf16 patterns bracketing a (found via a float32 estimate)
    base = int(np.array([abs(y)], np.float32).view(np.uint32)[0] >> 16)
    best = None
    for h in range(max(0, base - 2), min(0x7F80, base + 3) + 1):
        v = Fraction(float((np.array([h << 16], np.uint32)).view(np.float32)[0])) if h < 0x7F80 else None
        if v is None:
            continue
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and h % 2 == 0):
            best = (d, h)
    return sign | best[1]


def test_bf16_from_f64_matches_exact_rational_rounding():
    rng = np.random.default_rng(7)
    ys = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000))
    # exact ties and near-ties between adjacent bf16 values
    for h in rng.integers(0x0080, 0x7F00, 300):
        lo = float(np.array([int(h) << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(int(h) + 1) << 16], np.uint32).view(np.float32)[0])
        mid = (lo + hi) / 2
        ys += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid]
    for y in ys:
        assert oracle.bf16_from_f64(y) == _bf16_exact_round(float(y)), y


def test_bf16_from_f64_is_one_rounding_not_two():
    # y just above a bf16 midpoint but rounding to the midpoint in fp32: a
    # double rounding via fp32 would tie to even (down); a single rounding goes up.
    lo = 1.0
    ulp = 2.0 ** -7
    y = lo + ulp / 2 + 2.0 ** -40
    assert np.float32(y) == np.float32(lo + ulp / 2)
    assert oracle.bf16_from_f64(y) == 0x3F81
