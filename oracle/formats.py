"""Number formats of the a8w4 MoE layer, decoded and encoded from first principles.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
never does.

The pages name the formats only: routed experts stored as MXFP4, activations
in fp8 ("a8w4") [InferenceX PR 3430 "[AMD][MI35X] 0926 DSV4 sglang mtp
agentic", Additional detail section; FlyDSL issue 978 "Investigate MegaMoEV2
end-to-end throughput gap vs V1 on 8xMI355X", Test environment].  The bit
layouts below are the public OCP definitions those names refer to:

* fp8 E4M3FN (OCP 8-bit floating point): 1 sign, 4 exponent (bias 7),
  3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448;
  subnormals are m * 2^-9.
* e2m1 (OCP MX v1.0 FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit;
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* e8m0 (OCP MX v1.0 scale): 2^(b - 127); b = 255 is NaN.
* bf16: the upper 16 bits of an IEEE binary32.

Everything is evaluated in float64, where all these values are exact.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def dec_e4m3fn(codes) -> np.ndarray:
    """fp8 E4M3FN byte -> float64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    v = np.where(e == 0, sub, nor)
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def enc_e4m3fn_rne(v) -> np.ndarray:
    """float64 -> fp8 E4M3FN, round to nearest, ties to even mantissa.

    Defined for finite |v| <= 448 (the layer never produces more: every value
    is divided by a power of two chosen to bring the block maximum to <= 448).
    The sign of zero is kept.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3fn encode: input outside [-448, 448]")
    neg = np.signbit(v)
    a = np.abs(v)
    # subnormal range (a < 2^-6): integer multiples of 2^-9; m == 8 is 2^-6,
    # which is exactly code 0x08, so the code is the rounded multiple itself.
    sub_code = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal range: a = mant * 2^E with mant in [1, 2)
    fr, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex.astype(np.int64) - 1
    mant = fr * 2.0
    m = np.rint((mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    m = np.where(carry, 0, m)
    E = np.where(carry, E + 1, E)
    nor_code = ((E + 7) << 3) | m
    code = np.where(a < 2.0 ** -6, sub_code, nor_code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def dec_e2m1(nibbles) -> np.ndarray:
    """e2m1 nibble (0..15) -> float64, computed from the bit fields."""
    n = np.asarray(nibbles, dtype=np.uint8).astype(np.int64)
    s = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    v = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2((e - 1).astype(np.float64)))
    return s * v


def dec_e8m0(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2((b - 127).astype(np.float64)))


def unpack_nibbles(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] nibbles; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mxfp4(packed, scales) -> np.ndarray:
    """MXFP4 rows -> float64: element k of a row = e2m1(k) * 2^(scale[k // 32] - 127)."""
    vals = dec_e2m1(unpack_nibbles(packed))
    sc = dec_e8m0(scales)
    return vals * np.repeat(sc, 32, axis=-1)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v) -> np.ndarray:
    """float64 -> bf16 bits: round to f32 (nearest-even), then f32 -> bf16 (nearest-even)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)
