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
