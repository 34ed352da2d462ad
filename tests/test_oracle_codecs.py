"""Pins of the oracle's element decoders against the format definitions and
torch's own casts (library routines independent of the oracle)."""
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3fn_table_matches_torch_cast_all_codes():
    table = oracle.e4m3fn_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(table[c]), c
        else:
            assert table[c] == ref[c], (c, table[c], ref[c])
            assert math.copysign(1.0, table[c]) == math.copysign(1.0, ref[c]), c


def test_e4m3fn_values_from_format_definition():
    """Codes whose values the OCP 8-bit floating point format fixes (fixture
    tests/golden/e4m3fn_values.json lists each with its derivation)."""
    with open(os.path.join(GOLDEN, "e4m3fn_values.json")) as f:
        fixture = json.load(f)
    for entry in fixture["values"]:
        got = oracle.e4m3fn_table()[int(entry["code"], 16)]
        want = entry["value"]
        if want == "nan":
            assert math.isnan(got), entry
        else:
            assert got == float(want), entry
            assert math.copysign(1.0, got) == math.copysign(1.0, float(want)), entry


def test_e4m3fn_table_is_monotone_and_symmetric():
    t = oracle.e4m3fn_table()
    pos = t[0:0x7F]  # 0x00..0x7E: +0 .. 448, strictly increasing
    assert np.all(np.diff(pos) > 0)
    assert np.all(t[0x80:0xFF] == -t[0x00:0x7F])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t[np.r_[0:0x7F, 0x80:0xFF]]).all()


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        got = oracle.bf16_to_f64(int(b))
        if math.isnan(r):
            assert math.isnan(got)
        else:
            assert got == r


# ---- E4M3FN encoder (used by the quantising write)

def test_e4m3fn_encoder_round_trips_every_finite_code():
    table = oracle.e4m3fn_table()
    finite = [c for c in range(256) if not math.isnan(table[c])]
    codes = oracle.e4m3fn_encode(table[finite].astype(np.float32))
    assert codes.tolist() == finite


def test_e4m3fn_encoder_matches_torch_cast_in_range():
    """torch's float -> float8_e4m3fn cast rounds to nearest even; it does not
    saturate, so the comparison covers |y| < 464 (the midpoint above 448)."""
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-12.0, np.log2(463.9), size=200_000))
    y = (mags * rng.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    y = np.concatenate([y, np.float32([0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -9, 463.99997])])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(y), ref)


def test_e4m3fn_encoder_ties_go_to_even_mantissa():
    """The midpoint of two neighbouring finite codes (exact in binary32) goes to
    the one whose mantissa LSB is 0, on both signs."""
    table = oracle.e4m3fn_table()
    for c in range(0, 0x7E):
        mid = np.float32((table[c] + table[c + 1]) / 2)
        assert float(mid) == (table[c] + table[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        got = oracle.e4m3fn_encode(np.array([mid, -mid], dtype=np.float32))
        assert got.tolist() == [even, 0x80 | even], (c, float(mid))


def test_e4m3fn_encoder_saturates_and_keeps_nan_and_signed_zero():
    y = np.array([448.0, 449.0, 464.0, 465.0, 1e30, np.inf, -449.0, -1e30, -np.inf,
                  np.nan, -np.nan, 0.0, -0.0, 1e-30, -1e-30], dtype=np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE,
            0x7F, 0xFF, 0x00, 0x80, 0x00, 0x80]
    assert oracle.e4m3fn_encode(y).tolist() == want


def test_e4m3fn_encoder_picks_a_nearest_code():
    """Brute force against the decode table: no finite code is nearer to y
    than the chosen one."""
    table = oracle.e4m3fn_table()
    finite = np.array([table[c] for c in range(0x7F)])
    rng = np.random.default_rng(12)
    y = rng.uniform(-500.0, 500.0, size=3000).astype(np.float32)
    codes = oracle.e4m3fn_encode(y)
    for yi, c in zip(y, codes):
        val = table[c]
        best = np.min(np.abs(finite - abs(float(yi))))
        assert abs(abs(val) - abs(float(yi))) == best
        assert (c >= 0x80) == (yi < 0)
