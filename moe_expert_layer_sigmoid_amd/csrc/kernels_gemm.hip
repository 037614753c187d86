// Grouped expert GEMMs on block-scaled fp8 x MXFP4 MFMA (gfx950):
//   a5  GEMM1 (gate/up) + SwiGLU + fp8 requant
//   a6  GEMM2 (down) into an f32 row buffer (the combine reads it)
// The operator runs GEMM1 then GEMM2 on the routed experts, with fp8
// activations on MXFP4 experts [sglang PR 47065 "Use the aiter MegaMoE small-
// and large-input paths", intro; InferenceX PR 3430, Additional detail section].
//
// Weight-streaming design for few rows per expert ("swap-AB"): the MFMA's
// 16-row A side is 16 weight rows, its 16-column B side is 16 token rows of
// one expert.  Each wave owns four 16-row weight tiles and streams them from
// HBM once per 16 tokens; the token operand is read from the bucketed fp8
// buffer (L2-resident).
//
// Operand layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (measured on gfx950):
//  - e2m1 operand: lane l holds row l%16, K elements [32g, 32g+32), g = l/16,
//    packed two per byte (low nibble first) in its 4 low dwords;
//  - e4m3 operand: lane l holds row l%16, K [16g, 16g+16) in dwords 0-3 and
//    K [64+16g, 64+16g+16) in dwords 4-7;
//  - scales: lane l supplies the e8m0 scale of row l%16, K block g (32 wide),
//    op_sel choosing the byte of the scale register;
//  - result: lane l, element r holds D[4g + r][l%16].
// The K order inside one instruction is free as long as both operands and the
// scales agree, so lane group g takes NI consecutive 32-blocks of the weight
// row per step (NI*16 contiguous bytes and NI scale bytes) and the token
// operand is gathered to match.

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

template <int NI>
__device__ __forceinline__ int load_scales(rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (NI == 4) return buf_load4(r, voff, soff);
  else if constexpr (NI == 2) return buf_load2(r, voff, soff);
  else return buf_load1(r, voff, soff);
}

template <int I>
__device__ __forceinline__ v4f mfma_i(v4i a, v8i b, v4f c, int sa, int sb) {
  return mfma_fp4_fp8<I>(a, b, c, sa, sb);
}

template <int IA, int IB>
__device__ __forceinline__ v4f mfma_ij(v4i a, v8i b, v4f c, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, kFmtFp4, kFmtFp8, IA, sa, IB, sb);
}

// Registers of one K step of NT weight tiles against one token tile: the
// weight bytes and scales of each tile (A side) and the token bytes and scale
// (B side).  Steps are double-buffered so that the loads of step st + 2 are in
// flight while step st + 1 is waited for.
union V8 {
  v8i v;
  v4i h[2];
};

template <int NI, int NT>
struct Stage {
  v4i a[NT][NI];
  int sa[NT];
  V8 b[NI];
  int sb;
};

// Addressing of one wave's operands: buffer resources (scalar registers) plus
// 32-bit per-lane offsets; the K step enters as a uniform offset.
template <int NT>
struct Operands {
  rsrc_t w;           // weights of the slot
  rsrc_t ws;          // weight scales of the slot
  rsrc_t x;           // the rows of the token tile
  rsrc_t xs;          // their 128-column scales
  uint32_t woff[NT];  // row * K/2 + g * NI * 16
  uint32_t soff[NT];  // row * K/32 + g * NI
  uint32_t xlo, xhi;  // token row * K + (g & 1) * 16 + {(g >> 1), 2 + (g >> 1)} * NI * 32
  uint32_t xsoff;     // token row * K/128 + (g * NI) / 4
};

template <int NI, int NT>
__device__ __forceinline__ void load_stage(Stage<NI, NT>& S, const Operands<NT>& O, int st,
                                           const bool (&live)[NT]) {
  const uint32_t kb = (uint32_t)st * 4 * NI;  // first 32-block of the step
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    if (!live[rt]) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) S.a[rt][i] = buf_load16(O.w, O.woff[rt] + i * 16, kb * 16);
    S.sa[rt] = load_scales<NI>(O.ws, O.soff[rt], kb);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    S.b[i].h[0] = buf_load16(O.x, O.xlo + i * 32, kb * 32);
    S.b[i].h[1] = buf_load16(O.x, O.xhi + i * 32, kb * 32);
  }
  S.sb = buf_load1(O.xs, O.xsoff, kb / 4);
}

template <int NI, int NT>
__device__ __forceinline__ void mma_stage(v4f (&acc)[NT], const Stage<NI, NT>& S, const bool (&live)[NT]) {
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    if (!live[rt]) continue;
    acc[rt] = mfma_i<0>(S.a[rt][0], S.b[0].v, acc[rt], S.sa[rt], S.sb);
    if constexpr (NI > 1) acc[rt] = mfma_i<1>(S.a[rt][1], S.b[1].v, acc[rt], S.sa[rt], S.sb);
    if constexpr (NI > 2) acc[rt] = mfma_i<2>(S.a[rt][2], S.b[2].v, acc[rt], S.sa[rt], S.sb);
    if constexpr (NI > 3) acc[rt] = mfma_i<3>(S.a[rt][3], S.b[3].v, acc[rt], S.sa[rt], S.sb);
  }
}

// All nst K steps of one token tile, two register stages deep: the loads of
// step st + 2 are issued right after step st's MFMAs, so while step st + 1 is
// waited for, the next step's bytes are already in flight.  For an even step
// count the loop has no branches: its last two loads re-read the last two
// steps (L2 hits) and are never used.
template <int NI, int NT, bool EVEN>
__device__ __forceinline__ void stream_k(v4f (&acc)[NT], const Operands<NT>& O, int nst, const bool (&live)[NT]) {
  Stage<NI, NT> s0, s1;
  load_stage<NI, NT>(s0, O, 0, live);
  if (!EVEN && nst == 1) {
    mma_stage<NI, NT>(acc, s0, live);
    return;
  }
  load_stage<NI, NT>(s1, O, 1, live);
  if constexpr (EVEN) {
    for (int st = 0; st < nst; st += 2) {
      mma_stage<NI, NT>(acc, s0, live);
      load_stage<NI, NT>(s0, O, min(st + 2, nst - 2), live);
      mma_stage<NI, NT>(acc, s1, live);
      load_stage<NI, NT>(s1, O, min(st + 3, nst - 1), live);
    }
  } else {
  int st = 0;
  for (; st + 3 < nst; st += 2) {
    mma_stage<NI, NT>(acc, s0, live);
    load_stage<NI, NT>(s0, O, st + 2, live);
    mma_stage<NI, NT>(acc, s1, live);
    load_stage<NI, NT>(s1, O, st + 3, live);
  }
  // st + 3 == nst: three steps left
  mma_stage<NI, NT>(acc, s0, live);
  load_stage<NI, NT>(s0, O, st + 2, live);
  mma_stage<NI, NT>(acc, s1, live);
  mma_stage<NI, NT>(acc, s0, live);
  }
}

// ---------------------------------------------------------------------------
// Main case (K a multiple of 1024): natural K order, two MFMAs per 256-wide
// step.  MFMA i of step st covers 32-blocks st*8 + 4i + [0, 4), lane group g
// holding block st*8 + 4i + g, so each weight load reads 64 contiguous bytes
// per row across the four lane groups.  One 16-byte scale load per tile covers
// two steps (bytes 8h + 4i + g, picked with v_perm), and one token-scale dword
// covers two steps (128-column block 2st + i, picked with op_sel).
// ---------------------------------------------------------------------------
template <int NT>
struct QOperands {
  rsrc_t w, ws, x, xs;
  uint32_t woff[NT];  // row * K/2 + 16 g
  uint32_t soff[NT];  // row * K/32
  uint32_t xlo, xhi;  // token row * K + 16 g, + 64
  uint32_t xsoff;     // token row * K/128
  uint32_t sel;       // v_perm selector: byte g of the low dword, byte g of the high dword
};

struct QStage {
  v4i a[4][2];
  V8 b[2];
};

template <int NT>
__device__ __forceinline__ void q_load(QStage& S, const QOperands<NT>& O, int st) {
  const uint32_t wo = (uint32_t)st * 128, xo = (uint32_t)st * 256;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    S.a[rt][0] = buf_load16(O.w, O.woff[rt], wo);
    S.a[rt][1] = buf_load16(O.w, O.woff[rt] + 64, wo);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    S.b[i].h[0] = buf_load16(O.x, O.xlo + i * 128, xo);
    S.b[i].h[1] = buf_load16(O.x, O.xhi + i * 128, xo);
  }
}

// scales of steps st0 and st0 + 1 (st0 even)
template <int NT>
struct QScales {
  v4i sa[NT];
  int sb;
};

template <int NT>
__device__ __forceinline__ void q_load_scales(QScales<NT>& S, const QOperands<NT>& O, int st0) {
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) S.sa[rt] = buf_load16(O.ws, O.soff[rt], (uint32_t)st0 * 8);
  S.sb = buf_load4(O.xs, O.xsoff, (uint32_t)st0 * 2);
}

// MFMAs of step st0 + H (H = 0, 1) with stage S and the pair's scales
template <int NT, int H>
__device__ __forceinline__ void q_mma(v4f (&acc)[NT], const QStage& S, const QScales<NT>& C, uint32_t sel) {
  int sa[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
    sa[rt] = (int)__builtin_amdgcn_perm((uint32_t)C.sa[rt][2 * H + 1], (uint32_t)C.sa[rt][2 * H], sel);
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) acc[rt] = mfma_ij<0, 2 * H>(S.a[rt][0], S.b[0].v, acc[rt], sa[rt], C.sb);
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) acc[rt] = mfma_ij<1, 2 * H + 1>(S.a[rt][1], S.b[1].v, acc[rt], sa[rt], C.sb);
}

// nst a multiple of 4.  Operand stages run two steps ahead, scale pairs two
// to four steps ahead; the loop has no branches (its last loads re-read the
// final steps and are never used).
template <int NT>
__device__ __forceinline__ void stream_k_quad(v4f (&acc)[NT], const QOperands<NT>& O, int nst) {
  QStage s0, s1;
  QScales<NT> c0, c1;
  q_load_scales<NT>(c0, O, 0);
  q_load<NT>(s0, O, 0);
  q_load<NT>(s1, O, 1);
  q_load_scales<NT>(c1, O, 2);
  for (int st = 0; st < nst; st += 4) {
    q_mma<NT, 0>(acc, s0, c0, O.sel);
    q_load<NT>(s0, O, min(st + 2, nst - 2));
    q_mma<NT, 1>(acc, s1, c0, O.sel);
    q_load<NT>(s1, O, min(st + 3, nst - 1));
    q_load_scales<NT>(c0, O, min(st + 4, nst - 4));
    q_mma<NT, 0>(acc, s0, c1, O.sel);
    q_load<NT>(s0, O, min(st + 4, nst - 2));
    q_mma<NT, 1>(acc, s1, c1, O.sel);
    q_load<NT>(s1, O, min(st + 5, nst - 1));
    q_load_scales<NT>(c1, O, min(st + 6, nst - 2));
  }
}

__device__ __forceinline__ uint32_t perm_sel(int g) { return (uint32_t)g | ((uint32_t)(4 + g) << 8) | 0x0c0c0000u; }

// Per-lane offsets of the token operand for token row `tok` of the tile.
template <int NI, int NT>
__device__ __forceinline__ void token_offsets(Operands<NT>& O, uint32_t tok, uint32_t K, int g) {
  const uint32_t row = tok * K + (uint32_t)(g & 1) * 16;
  O.xlo = row + (uint32_t)(g >> 1) * NI * 32;
  O.xhi = row + (uint32_t)(2 + (g >> 1)) * NI * 32;
  O.xsoff = tok * (K / kActBlock) + (uint32_t)(g * NI) / 4;
}

// ---------------------------------------------------------------------------
// a5: one block per (local slot s, 128-column block fb of F).  Wave w owns gate
// rows fb*128 + 32w + [0, 32) and the matching up rows F + ..., so SwiGLU pairs
// registers of the same lane; the requant amax over the 128 columns is reduced
// across the four waves in LDS.
// ---------------------------------------------------------------------------
template <int NI, bool EVEN, bool QUAD>
__global__ __launch_bounds__(256, 3) void k_gemm1_stream(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                      const int32_t* __restrict__ offsets,
                                                      const uint8_t* __restrict__ w1, const uint8_t* __restrict__ w1s,
                                                      uint8_t* __restrict__ aq, uint8_t* __restrict__ as_, int H,
                                                      int F) {
  __shared__ float s_amax[4][16];
  const int nfb = F / kActBlock;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nfb, fb = item - s * nfb;
  const int row0 = offsets[s];
  const int n = offsets[s + 1] - row0;
  if (n <= 0) return;  // block-uniform: an idle expert reads no weights
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int f0 = fb * kActBlock + wave * 32;
  const uint32_t KB = (uint32_t)H / 2, KS = (uint32_t)H / 32;
  Operands<4> O;
  O.w = make_rsrc(w1 + (size_t)s * 2 * F * KB, 2u * F * KB);
  O.ws = make_rsrc(w1s + (size_t)s * 2 * F * KS, 2u * F * KS);
  const int wrow[4] = {f0 + l16, f0 + 16 + l16, F + f0 + l16, F + f0 + 16 + l16};
  if constexpr (!QUAD) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      O.woff[rt] = (uint32_t)wrow[rt] * KB + (uint32_t)(g * NI) * 16;
      O.soff[rt] = (uint32_t)wrow[rt] * KS + (uint32_t)(g * NI);
    }
  }
  QOperands<4> Q;
  if constexpr (QUAD) {
    Q.w = O.w;
    Q.ws = O.ws;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Q.woff[rt] = (uint32_t)wrow[rt] * KB + (uint32_t)g * 16;
      Q.soff[rt] = (uint32_t)wrow[rt] * KS;
    }
    Q.sel = perm_sel(g);
  }
  const int nst = H / (128 * NI);
  const int nb = H / kActBlock;
  const bool live[4] = {true, true, true, true};
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const uint32_t nrow = (uint32_t)min(16, n - tt0);
    O.x = make_rsrc(xq + (size_t)(row0 + tt0) * H, nrow * H);
    O.xs = make_rsrc(xs + (size_t)(row0 + tt0) * nb, nrow * nb);
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (QUAD) {
      const uint32_t tr = tv ? (uint32_t)l16 : 0u;
      Q.x = O.x;
      Q.xs = O.xs;
      Q.xlo = tr * (uint32_t)H + (uint32_t)g * 16;
      Q.xhi = Q.xlo + 64;
      Q.xsoff = tr * (uint32_t)nb;
      stream_k_quad<4>(acc, Q, H / 256);
    } else {
      token_offsets<NI, 4>(O, tv ? (uint32_t)l16 : 0u, (uint32_t)H, g);
      stream_k<NI, 4, EVEN>(acc, O, nst, live);
    }
    // SwiGLU: acc[0]/acc[2] are gate/up of columns f0 + 4g + r, acc[1]/acc[3] of f0 + 16 + 4g + r
    float act[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      act[r] = silu(acc[0][r]) * acc[2][r];
      act[4 + r] = silu(acc[1][r]) * acc[3][r];
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(act[i]));
    am = fmaxf(am, __shfl_xor(am, 16));
    am = fmaxf(am, __shfl_xor(am, 32));
    if (g == 0) s_amax[wave][l16] = am;
    __syncthreads();
    am = fmaxf(fmaxf(s_amax[0][l16], s_amax[1][l16]), fmaxf(s_amax[2][l16], s_amax[3][l16]));
    __syncthreads();
    const int e = scale_exp(am);
    if (tv) {
      uint8_t* ap = aq + (size_t)(row0 + tok) * F + f0 + 4 * g;
      *reinterpret_cast<uint32_t*>(ap) =
          pack4_fp8(ldexpf(act[0], -e), ldexpf(act[1], -e), ldexpf(act[2], -e), ldexpf(act[3], -e));
      *reinterpret_cast<uint32_t*>(ap + 16) =
          pack4_fp8(ldexpf(act[4], -e), ldexpf(act[5], -e), ldexpf(act[6], -e), ldexpf(act[7], -e));
      if (wave == 0 && g == 0) as_[(size_t)(row0 + tok) * nfb + fb] = (uint8_t)(e + 127);
    }
  }
}

// ---------------------------------------------------------------------------
// a6: one block per (local slot s, 256-row block of H).  Wave w owns rows
// hb*256 + 64w + [0, 64) as four 16-row tiles; y rows are f32 [rows, H].
// ---------------------------------------------------------------------------
template <int NI, bool EVEN, bool QUAD>
__global__ __launch_bounds__(256, 3) void k_gemm2_stream(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_,
                                                      const int32_t* __restrict__ offsets,
                                                      const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s,
                                                      float* __restrict__ y, int H, int F) {
  const int nhb = (H + 255) / 256;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nhb, hb = item - s * nhb;
  const int row0 = offsets[s];
  const int n = offsets[s + 1] - row0;
  if (n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int h0 = hb * 256 + wave * 64;
  if (h0 >= H) return;  // wave-uniform (H is a multiple of 128)
  const uint32_t KB = (uint32_t)F / 2, KS = (uint32_t)F / 32;
  Operands<4> O;
  O.w = make_rsrc(w2 + (size_t)s * H * KB, (uint32_t)H * KB);
  O.ws = make_rsrc(w2s + (size_t)s * H * KS, (uint32_t)H * KS);
  bool live[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    live[rt] = h0 + 16 * rt < H;
    const uint32_t row = live[rt] ? (uint32_t)(h0 + 16 * rt + l16) : 0u;
    O.woff[rt] = row * KB + (uint32_t)(g * NI) * 16;
    O.soff[rt] = row * KS + (uint32_t)(g * NI);
  }
  QOperands<4> Q;
  if constexpr (QUAD) {  // H is a multiple of 256 here: every tile is live
    Q.w = O.w;
    Q.ws = O.ws;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t row = (uint32_t)(h0 + 16 * rt + l16);
      Q.woff[rt] = row * KB + (uint32_t)g * 16;
      Q.soff[rt] = row * KS;
    }
    Q.sel = perm_sel(g);
  }
  const int nst = F / (128 * NI);
  const int nb = F / kActBlock;
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const uint32_t nrow = (uint32_t)min(16, n - tt0);
    O.x = make_rsrc(aq + (size_t)(row0 + tt0) * F, nrow * F);
    O.xs = make_rsrc(as_ + (size_t)(row0 + tt0) * nb, nrow * nb);
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (QUAD) {
      const uint32_t tr = tv ? (uint32_t)l16 : 0u;
      Q.x = O.x;
      Q.xs = O.xs;
      Q.xlo = tr * (uint32_t)F + (uint32_t)g * 16;
      Q.xhi = Q.xlo + 64;
      Q.xsoff = tr * (uint32_t)nb;
      stream_k_quad<4>(acc, Q, F / 256);
    } else {
      token_offsets<NI, 4>(O, tv ? (uint32_t)l16 : 0u, (uint32_t)F, g);
      stream_k<NI, 4, EVEN>(acc, O, nst, live);
    }
    if (tv) {
      float* yr = y + (size_t)(row0 + tok) * H + h0 + 4 * g;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (!live[rt]) continue;
        *reinterpret_cast<float4*>(yr + 16 * rt) = make_float4(acc[rt][0], acc[rt][1], acc[rt][2], acc[rt][3]);
      }
    }
  }
}

// 32-blocks per lane group per step.  Two (a 256-wide K step) when the step
// count comes out even, which keeps the branch-free pipelined loop within the
// register budget of 3 waves per SIMD; otherwise one.
#ifndef MOE_STREAM_NI
#define MOE_STREAM_NI 2
#endif
static int pick_ni(int K) {
  return (MOE_STREAM_NI >= 2 && (K / 128) % 4 == 0) ? 2 : 1;
}

hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* w1,
                               const uint8_t* w1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                               hipStream_t st) {
  dim3 grid(P_local * (F / kActBlock));
  if (H % 1024 == 0) k_gemm1_stream<2, true, true><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F);
  else if (pick_ni(H) == 2)
    k_gemm1_stream<2, true, false><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F);
  else if ((H / 128) % 2 == 0)
    k_gemm1_stream<1, true, false><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F);
  else k_gemm1_stream<1, false, false><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* w2,
                               const uint8_t* w2s, float* y, int H, int F, int P_local, hipStream_t st) {
  dim3 grid(P_local * ((H + 255) / 256));
  if (F % 1024 == 0 && H % 256 == 0)
    k_gemm2_stream<2, true, true><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F);
  else if (pick_ni(F) == 2) k_gemm2_stream<2, true, false><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F);
  else if ((F / 128) % 2 == 0) k_gemm2_stream<1, true, false><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F);
  else k_gemm2_stream<1, false, false><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F);
  return hipGetLastError();
}

}  // namespace moe
