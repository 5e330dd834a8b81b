"""Pins of the oracle's number formats against the format definitions and torch's casts."""
import math
import os

import numpy as np
import torch

import oracle
from oracle.formats import bf16_bits_to_f64, e4m3_decode, e4m3_decode_table, e4m3_encode

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    # signed zeros decode with their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_e4m3_landmarks_from_format_definition():
    table = e4m3_decode_table()
    n = 0
    for line in open(os.path.join(GOLD, "e4m3fn_landmarks.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        code = int(code, 16)
        if val == "nan":
            assert math.isnan(table[code])
        else:
            assert table[code] == float(val), hex(code)
            assert math.copysign(1.0, table[code]) == math.copysign(1.0, float(val))
        n += 1
    assert n == 15


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()


def test_e4m3_structure():
    t = e4m3_decode_table()
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()  # positive codes strictly increasing
    assert (t[0x80:0xFF] == -t[0:0x7F]).all()  # sign symmetry
    assert pos.max() == oracle.E4M3_MAX == 448.0
    assert pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert (e4m3_encode(vals) == codes).all()


def test_e4m3_encode_midpoints_round_to_even():
    t = e4m3_decode_table()
    for c in range(0, 0x7E):
        mid = np.float32((t[c] + t[c + 1]) / 2)  # exact in fp32 (<= 5 significant bits)
        assert float(mid) == (t[c] + t[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert int(e4m3_encode(mid)) == want, hex(c)
        assert int(e4m3_encode(-mid)) == want | 0x80
        # just off the midpoint goes to the nearer neighbour
        assert int(e4m3_encode(np.nextafter(mid, np.float32(0)))) == c
        assert int(e4m3_encode(np.nextafter(mid, np.float32(1e9)))) == c + 1


def test_e4m3_encode_saturates_and_nan():
    y = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert e4m3_encode(y).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert int(e4m3_encode(np.float32(np.nan))) == 0x7F
    assert int(e4m3_encode(np.float32(-np.nan))) in (0x7F, 0xFF)
    assert int(e4m3_encode(np.float32(0.0))) == 0x00
    assert int(e4m3_encode(np.float32(-0.0))) == 0x80
    assert int(e4m3_encode(np.float32(2.0 ** -10))) == 0x00  # tie between 0 and the smallest subnormal
    assert int(e4m3_encode(np.float32(-(2.0 ** -11)))) == 0x80


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 3,
        (rng.standard_normal(200_000) * 0.01).astype(np.float32),
        rng.uniform(-447.9, 447.9, 200_000).astype(np.float32),
    ])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (e4m3_encode(y) == ref).all()
