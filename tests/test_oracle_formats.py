"""Pins of the oracle's number formats against published tables, a library and brute force."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as fm
import synth.inputs as si

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_e4m3fn_published_code_points():
    for code, val in _table("e4m3fn_codes.txt"):
        got = fm.dec_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), code
            assert np.signbit(got) == val.startswith("-"), code


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fm.dec_e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert nan.sum() == 2


def _all_bf16_within(limit):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # drop inf / NaN patterns
    v = fm.bf16_to_f64(bits)
    ok = np.abs(v) <= limit
    return v[ok]


def test_e4m3fn_encode_exhaustive_brute_force():
    """Every bf16 value with |v| <= 448 against a nearest-code search (ties to even code)."""
    v = _all_bf16_within(448.0)
    codes = np.arange(256, dtype=np.uint8)
    dec = fm.dec_e4m3fn(codes)
    fin = np.isfinite(dec)
    cand_codes = codes[fin]
    cand = dec[fin]
    got = fm.enc_e4m3fn_rne(v)
    # brute force in chunks
    for lo in range(0, v.size, 4096):
        vv = v[lo:lo + 4096]
        dist = np.abs(vv[:, None] - cand[None, :])
        best = dist.min(axis=1, keepdims=True)
        tie = dist == best
        # among equally near codes prefer an even mantissa (code LSB 0), and the
        # sign of v (the value -0 vs +0 distinction only matters at zero)
        score = tie * (1 + ((cand_codes[None, :] & 1) == 0) * 2
                       + ((cand_codes[None, :] >> 7) == np.signbit(vv)[:, None]))
        want = cand_codes[np.argmax(score, axis=1)]
        g = got[lo:lo + 4096]
        assert np.array_equal(fm.dec_e4m3fn(g), fm.dec_e4m3fn(want)), lo
        assert np.array_equal(g, want), lo


def test_e4m3fn_encode_matches_torch_cast():
    v = _all_bf16_within(448.0)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fm.enc_e4m3fn_rne(v), ref)


def test_e4m3fn_encode_ties_and_limits():
    # 1.0625 is halfway 1.0 / 1.125 -> even (1.0); 1.1875 halfway 1.125 / 1.25 -> 1.25
    # 2^-10 halfway 0 / 2^-9 -> 0; 3*2^-11 -> 2^-9 (nearest); 3*2^-10 halfway 2^-9 / 2^-8 -> 2^-8
    assert list(fm.enc_e4m3fn_rne(np.array([1.0625, 1.1875, 448.0, 2.0 ** -10, 3 * 2.0 ** -11,
                                            3 * 2.0 ** -10, -0.0]))) == [0x38, 0x3A, 0x7E, 0x00, 0x01, 0x02, 0x80]
    with pytest.raises(ValueError):
        fm.enc_e4m3fn_rne(np.array([449.0]))


def test_e2m1_published_table():
    for nib, val in _table("e2m1_table.txt"):
        got = fm.dec_e2m1(np.array([int(nib, 16)], np.uint8))[0]
        assert got == float(val) and np.signbit(got) == val.startswith("-"), nib


def test_e8m0():
    assert fm.dec_e8m0(np.array([127], np.uint8))[0] == 1.0
    assert fm.dec_e8m0(np.array([0], np.uint8))[0] == 2.0 ** -127
    assert fm.dec_e8m0(np.array([254], np.uint8))[0] == 2.0 ** 127
    assert np.isnan(fm.dec_e8m0(np.array([255], np.uint8))[0])


def test_nibble_order_low_first():
    p = np.array([[0x21, 0xF7]], np.uint8)
    assert list(fm.unpack_nibbles(p)[0]) == [0x1, 0x2, 0x7, 0xF]
    # element 2i low nibble: [0.5, 1, 6, -6] with scale byte 127 -> unchanged
    d = fm.dequant_mxfp4(np.tile(p, (1, 8)), np.array([[127]], np.uint8))
    assert list(d[0, :4]) == [0.5, 1.0, 6.0, -6.0]


def test_mxfp4_roundtrip_exact_on_grid():
    """Values already on the e2m1 grid times a power of two survive encode/decode."""
    rng = np.random.default_rng(1)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    vals = rng.choice(mags, size=(8, 64)) * rng.choice([-1, 1], size=(8, 64))
    vals[:, 0] = 6.0  # pins each block's exponent: floor(log2 6) - 2 = 0
    vals[:, 32] = -4.0
    vals = (vals * np.float32(2.0 ** -7)).astype(np.float32)
    packed, sc = si._encode_mxfp4(vals)
    assert np.array_equal(fm.dequant_mxfp4(packed, sc), vals.astype(np.float64))


def test_mxfp4_roundtrip_error_bound():
    """Gaussian rows: error <= half the e2m1 grid step at the element's magnitude
    (steps 0.5/1/2 below 2/4/6 times the block scale), or saturation above 6."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    packed, sc = si._encode_mxfp4(w)
    d = fm.dequant_mxfp4(packed, sc)
    scale = np.repeat(fm.dec_e8m0(sc), 32, axis=-1)
    a = np.abs(w.astype(np.float64)) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(d - w) / scale
    bound = np.where(a <= 6, step / 2, a - 6)
    assert np.all(err <= bound + 1e-12)


def test_bf16_roundtrip_and_rne():
    assert fm.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16)).tolist() == [1.0, -2.0, 0.0, -0.0]
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    got = fm.f64_to_bf16_rne(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -3.0]))
    assert got.tolist() == [0x3F80, 0x3F82, 0xC040]
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(100000) * 10).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fm.f64_to_bf16_rne(v.astype(np.float64)), ref)
