"""The rounding of gfx950's block-scaled MFMA instruction, measured: the
allowance (oracle.moe.MFMA_REL, 2^-14 of the sum of absolute products per
instruction) behind the GEMM tolerances of the parity tests.

V_MFMA_SCALE_F32_16X16X128_F8F6F4 does not return the float32 rounding of
the exact sum.  A test-only probe (tests/probe/mfma_probe.hip) runs it on
MXFP4 x fp8 operands placed directly in the instruction's lanes, and each
case compares the 16 x 16 results with exact sums (float64; the products are
exact).  What it shows:
  * inside one 32-element scale block the products are aligned to the
    block's largest and the bits more than about 14 below its leading bit are
    dropped (a product 2^-12 of the largest loses part of itself, one below
    2^-16 vanishes), while the four blocks are combined at float32
    precision.  For any operands the error of one instruction is therefore
    at most, per block, (non-zero products - 1) x 2^(floor(log2 of its
    largest |product|) - 13), plus float32 roundings: asserted on random,
    cancelling, wide-range and accumulator cases;
  * relative to the sum of absolute products that model allows up to
    31 x 2^-13 for adversarial blocks (uniformly random codes reach 1.9e-4),
    but operands drawn like the layer's (N(0, 1) token rows quantised per 128
    columns, SwiGLU-shaped act rows, N(0, 0.02) MXFP4 weights) stay well
    inside 2^-14: asserted, one instruction and K = 2048 chains;
  * chains of 16 and 56 instructions (K = 2048 and 7168, the layer's widths)
    stay within oracle.moe.gemm_error_bound.
Every case prints its worst ratio.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import moe as om

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libmfma_probe.so")
FP8_OK = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # every code but NaN


def _say(*a):
    print(*a, flush=True)


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with `python -m tests.probe.build`")
    L = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    L.mfma_probe_chain.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int, P]
    L.mfma_probe_chain.restype = ctypes.c_int
    return L


def _values(codes, scales, dec):
    """float64 [.., 16, 128] of element codes [.., 16, 128] and e8m0 scales [.., 16, 4]."""
    return dec(codes) * np.repeat(fm.dec_e8m0(scales), 32, axis=-1)


def run(A, sa, B, sb, C):
    """Chains on the GPU.  A: e2m1 codes [nprob, n, 16, 128]; sa: [nprob, n, 16, 4];
    B: fp8 codes [nprob, n, 16, 128]; sb likewise; C: f32 [nprob, 16, 16].
    Returns the GPU's D [nprob, 16, 16] (float64) and the exact D."""
    nprob, n = A.shape[:2]
    lane = np.arange(64)
    r, g = lane % 16, lane // 16
    # A: lane l -> row r, K [32 g, 32 g + 32), element 2i low nibble of byte i
    ka = 32 * g[:, None] + np.arange(32)[None, :]                       # [64, 32]
    a_el = A[:, :, r[:, None], ka]                                      # [nprob, n, 64, 32]
    a_lane = (a_el[..., 0::2] | (a_el[..., 1::2] << 4)).astype(np.uint8)
    # B: lane l -> column r, K [16 g, +16) then [64 + 16 g, +16)
    kb = np.concatenate([16 * g[:, None] + np.arange(16)[None, :], 64 + 16 * g[:, None] + np.arange(16)[None, :]], 1)
    b_lane = B[:, :, r[:, None], kb].astype(np.uint8)                   # [nprob, n, 64, 32]
    sa_lane = sa[:, :, r, g].astype(np.int32)
    sb_lane = sb[:, :, r, g].astype(np.int32)
    el = np.arange(4)
    c_lane = C[:, 4 * g[:, None] + el[None, :], r[:, None]].astype(np.float32)   # [nprob, 64, 4]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")  # noqa: E731
    ta, tb, tsa, tsb, tc = dev(a_lane), dev(b_lane), dev(sa_lane), dev(sb_lane), dev(c_lane)
    td = torch.zeros((nprob, 64, 4), dtype=torch.float32, device="cuda")
    rc = _lib().mfma_probe_chain(ta.data_ptr(), tb.data_ptr(), tsa.data_ptr(), tsb.data_ptr(), tc.data_ptr(),
                                 td.data_ptr(), nprob, n, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    d_lane = td.cpu().numpy().astype(np.float64)
    D = np.zeros((nprob, 16, 16))
    D[:, 4 * g[:, None] + el[None, :], r[:, None]] = d_lane
    av = _values(A, sa, fm.dec_e2m1)                                    # [nprob, n, 16, 128]
    bv = _values(B, sb, fm.dec_e4m3fn)
    prod = av[:, :, :, None, :] * bv[:, :, None, :, :]                  # [nprob, n, 16, 16, 128] (exact)
    exact = C.astype(np.float64) + prod.sum(axis=(1, 4))
    mag = np.abs(prod).sum(axis=(1, 4))
    return D, exact, mag


def _rand(rng, nprob, n, lo=120, hi=134):
    A = rng.integers(0, 16, (nprob, n, 16, 128)).astype(np.uint8)
    B = rng.choice(FP8_OK, (nprob, n, 16, 128)).astype(np.uint8)
    sa = rng.integers(lo, hi, (nprob, n, 16, 4)).astype(np.uint8)
    sb = rng.integers(lo, hi, (nprob, n, 16, 4)).astype(np.uint8)
    return A, sa, B, sb


def block_model_bound(A, sa, B, sb, C):
    """The measured model of one instruction (chains of n = 1): per 32-element
    block, (non-zero products - 1) x 2^(floor(log2 max |product|) - 13), plus
    2^-22 (|C| + sum |products|) for the float32 combination of the blocks and
    the accumulator."""
    av = _values(A, sa, fm.dec_e2m1)[:, 0]                              # [nprob, 16, 128]
    bv = _values(B, sb, fm.dec_e4m3fn)[:, 0]
    p = np.abs(av[:, :, None, :] * bv[:, None, :, :]).reshape(av.shape[0], 16, 16, 4, 32)
    mx_ = p.max(-1)
    cnt = (p > 0).sum(-1)
    e = np.floor(np.log2(np.where(mx_ > 0, mx_, 1.0)))
    trunc = np.where(cnt > 0, (cnt - 1) * np.exp2(e - 13), 0.0).sum(-1)
    return trunc + 2.0 ** -22 * (np.abs(C.astype(np.float64)) + p.sum(axis=(-1, -2)))


def _ratio(D, exact, mag, C=None):
    """|D - exact| over the instruction allowance's base (sum of |products|)."""
    err = np.abs(D - exact)
    if C is not None:  # the accumulator input's own float32 rounding is allowed on top
        err = np.maximum(err - om.F32_U * np.abs(exact), 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(mag > 0, err / mag, np.where(err > 0, np.inf, 0.0))
    return float(r.max())


def test_single_instruction_random_and_cancelling():
    rng = np.random.default_rng(1)
    A, sa, B, sb = _rand(rng, 256, 1)
    C = np.zeros((256, 16, 16), np.float32)
    D, ex, mag = run(A, sa, B, sb, C)
    r1 = _ratio(D, ex, mag)
    assert np.all(np.abs(D - ex) <= block_model_bound(A, sa, B, sb, C))
    # products cancelling in pairs: K 64..127 repeat K 0..63 with the A sign
    # flipped (scale blocks 2, 3 equal to 0, 1), the last pair left whole
    A2, sa2, B2, sb2 = _rand(rng, 256, 1)
    A2[..., 64:] = A2[..., :64] ^ 8
    A2[..., 127] = A2[..., 63]
    B2[..., 64:] = B2[..., :64]
    sa2[..., 2:] = sa2[..., :2]
    sb2[..., 2:] = sb2[..., :2]
    D, ex, mag = run(A2, sa2, B2, sb2, C)
    r2 = _ratio(D, ex, mag)
    assert np.all(np.abs(D - ex) <= block_model_bound(A2, sa2, B2, sb2, C))
    _say(f"[mfma] one instruction, uniformly random codes: {r1:.3e}; cancelling pairs {r2:.3e} of sum|a w| "
         f"(within the block model; the layer's allowance is {om.MFMA_REL:.3e})")


def test_characterise_two_products():
    """Where the instruction loses the smaller of two products: one product of
    2688 (6 x 448) and one of 2^-j times it, in the same 32-block or in
    another block.  Printed, and held to the block model."""
    rows = []
    for where in ("same block", "other block"):
        for j in (4, 8, 10, 12, 13, 14, 16, 18, 20, 24):
            nprob = 1
            A = np.zeros((nprob, 1, 16, 128), np.uint8)
            B = np.zeros((nprob, 1, 16, 128), np.uint8)
            sa = np.full((nprob, 1, 16, 4), 127, np.uint8)
            sb = np.full((nprob, 1, 16, 4), 127, np.uint8)
            A[..., 0] = 7                            # 6.0
            B[..., 0] = 0x7E                         # 448
            k = 1 if where == "same block" else 32
            A[..., k] = 7                            # 6.0
            B[..., k] = 0x7E                         # 448, scaled down by 2^-j through the scale byte
            if where == "same block":
                # scale the small product through its fp8 code instead: 448 * 2^-j on the fp8 grid
                B[..., k] = fm.enc_e4m3fn_rne(np.array([448.0 * 2.0 ** -j]))[0] if j <= 17 else 0x01
            else:
                sb[..., 1] = 127 - j
            C = np.zeros((nprob, 16, 16), np.float32)
            D, ex, mag = run(A, sa, B, sb, C)
            assert np.all(np.abs(D - ex) <= block_model_bound(A, sa, B, sb, C))
            big = 2688.0
            small = float(ex[0, 0, 0] - big)
            err = float(D[0, 0, 0] - ex[0, 0, 0])
            rows.append((where, j, small / big, err / small if small else 0.0))
    for w, j, rel, frac in rows:
        _say(f"[mfma] two products, {w}: small/big = {rel:.3e}: error = {frac:+.3e} of the small product")


def _layer_operands(rng, nprob, n, act_like):
    """Operands drawn as the layer draws them: B (token side) N(0, 1) rows, or
    SwiGLU-shaped silu(g) u for GEMM2, quantised per 128 columns by the a4
    rule; A (weights) N(0, 0.02) encoded to MXFP4 by the OCP rule."""
    import synth
    K = 128 * n
    B = np.zeros((nprob, n, 16, 128), np.uint8)
    sb = np.zeros((nprob, n, 16, 4), np.uint8)
    A = np.zeros((nprob, n, 16, 128), np.uint8)
    sa = np.zeros((nprob, n, 16, 4), np.uint8)
    for p in range(nprob):
        if act_like:
            g, u = rng.normal(0, 1.5, (16, K)), rng.normal(0, 1.5, (16, K))
            x = om.silu(g) * u
        else:
            x = rng.normal(0, 1, (16, K))
        q, s = om.quant_blocks(x)                                  # e8m0 per 128, e4m3fn codes
        B[p] = q.reshape(16, n, 128).transpose(1, 0, 2)
        sb[p] = np.repeat(s.reshape(16, n, 1), 4, axis=2).transpose(1, 0, 2)
        w, ws = synth.inputs._encode_mxfp4(rng.normal(0, 0.02, (16, K)).astype(np.float32))
        codes = np.stack([w & 15, w >> 4], axis=-1).reshape(16, K)
        A[p] = codes.reshape(16, n, 128).transpose(1, 0, 2)
        sa[p] = ws.reshape(16, n, 4).transpose(1, 0, 2)
    return A, sa, B, sb


@pytest.mark.parametrize("act_like", [False, True])
def test_layer_operands_within_the_allowance(act_like):
    """The allowance covers operands drawn like the layer's (GEMM1: N(0, 1)
    token rows; GEMM2: SwiGLU-shaped act rows), one instruction and K = 2048
    chains."""
    rng = np.random.default_rng(11 + act_like)
    worst = {}
    for n, nprob in ((1, 256), (16, 16)):
        A, sa, B, sb = _layer_operands(rng, nprob, n, act_like)
        C = np.zeros((nprob, 16, 16), np.float32)
        D, ex, mag = run(A, sa, B, sb, C)
        worst[n] = _ratio(D, ex, mag)
        bound = (om.MFMA_REL + n * om.F32_U * (1 + 4 * om.MFMA_REL)) * mag
        assert np.all(np.abs(D - ex) <= bound)
    _say(f"[mfma] layer operands ({'GEMM2 act' if act_like else 'GEMM1 tokens'}): one instruction "
         f"{worst[1]:.3e}, K = 2048 chain {worst[16]:.3e} of sum|a w| (allowance {om.MFMA_REL:.3e})")


@pytest.mark.parametrize("shift", [8, 12, 16, 20, 23, 26])
def test_single_instruction_wide_dynamic_range(shift):
    """One product about 2^shift larger than the 96 others (K block 0 holds only
    it): small products that an internal alignment to the largest would cut
    short."""
    rng = np.random.default_rng(100 + shift)
    nprob = 128
    A, sa, B, sb = _rand(rng, nprob, 1, 126, 129)
    A[..., 0] = 7                           # e2m1 6.0 at K = 0
    B[..., 0] = 0x7E                        # fp8 448 at K = 0
    sa[..., 0] = np.minimum(sa[..., 0].astype(np.int32) + shift, 254).astype(np.uint8)
    A[..., 1:32] = 0
    C = np.zeros((nprob, 16, 16), np.float32)
    D, ex, mag = run(A, sa, B, sb, C)
    r = _ratio(D, ex, mag)
    _say(f"[mfma] dynamic range 2^{shift}+: {r:.3e} of sum|a w|")
    assert r <= om.MFMA_REL and np.all(np.abs(D - ex) <= block_model_bound(A, sa, B, sb, C))


@pytest.mark.parametrize("c_scale", [2.0 ** 12, 2.0 ** -12])
def test_single_instruction_with_accumulator(c_scale):
    rng = np.random.default_rng(7)
    A, sa, B, sb = _rand(rng, 128, 1, 125, 129)
    C = (rng.normal(0, 1, (128, 16, 16)) * c_scale).astype(np.float32)
    D, ex, mag = run(A, sa, B, sb, C)
    r = _ratio(D, ex, mag, C)
    _say(f"[mfma] accumulator ~{c_scale:g}, uniformly random codes: {r:.3e} of sum|a w| beyond one float32 "
         f"rounding")
    assert np.all(np.abs(D - ex) <= block_model_bound(A, sa, B, sb, C))


@pytest.mark.parametrize("n", [16, 56])
def test_chains_within_the_gemm_bound(n):
    rng = np.random.default_rng(n)
    nprob = 16
    A, sa, B, sb = _rand(rng, nprob, n, 124, 130)
    C = np.zeros((nprob, 16, 16), np.float32)
    D, ex, mag = run(A, sa, B, sb, C)
    bound = (om.MFMA_REL + n * om.F32_U * (1 + 4 * om.MFMA_REL)) * mag   # oracle.moe.gemm_error_bound
    worst = float((np.abs(D - ex) / mag).max())
    _say(f"[mfma] chain of {n} (K = {128 * n}): {worst:.3e} of sum|a w| (bound "
         f"{om.MFMA_REL + n * om.F32_U:.3e})")
    assert np.all(np.abs(D - ex) <= bound)
