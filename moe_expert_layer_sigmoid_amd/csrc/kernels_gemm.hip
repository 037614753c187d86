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
// row per step (NI*16 contiguous bytes, one scale dword when NI = 4) and the
// token operand is gathered to match.

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

template <int NI>
__device__ __forceinline__ int load_scales(const uint8_t* p) {
  if constexpr (NI == 4) return *reinterpret_cast<const int*>(p);
  else if constexpr (NI == 2) return (int)*reinterpret_cast<const uint16_t*>(p);
  else return (int)*p;
}

template <int I>
__device__ __forceinline__ v4f mfma_i(v4i a, v8i b, v4f c, int sa, int sb) {
  return mfma_fp4_fp8<I>(a, b, c, sa, sb);
}

// One K step of four weight tiles against one token tile.
//  wp[rt]: this lane's weight bytes for the step (NI*16 bytes)
//  sp[rt]: this lane's weight scale bytes for the step (NI bytes)
//  xp:     token row + (g & 1) * 16; blocks are addressed relative to kbase
template <int NI, int NT>
__device__ __forceinline__ void step_4tiles(v4f (&acc)[NT], const uint8_t* (&wp)[NT],
                                            const uint8_t* (&sp)[NT], const uint8_t* xp, int kbase,
                                            int g, int sbv, const bool (&live)[NT]) {
  v4i a[NT][NI];
  int sa[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    if (!live[rt]) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) a[rt][i] = *reinterpret_cast<const v4i*>(wp[rt] + i * 16);
    sa[rt] = load_scales<NI>(sp[rt]);
  }
  v8i b[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    v4i lo = *reinterpret_cast<const v4i*>(xp + (size_t)(kbase + (g >> 1) * NI + i) * 32);
    v4i hi = *reinterpret_cast<const v4i*>(xp + (size_t)(kbase + (2 + (g >> 1)) * NI + i) * 32);
    b[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    if (!live[rt]) continue;
    acc[rt] = mfma_i<0>(a[rt][0], b[0], acc[rt], sa[rt], sbv);
    if constexpr (NI > 1) acc[rt] = mfma_i<1>(a[rt][1], b[1], acc[rt], sa[rt], sbv);
    if constexpr (NI > 2) acc[rt] = mfma_i<2>(a[rt][2], b[2], acc[rt], sa[rt], sbv);
    if constexpr (NI > 3) acc[rt] = mfma_i<3>(a[rt][3], b[3], acc[rt], sa[rt], sbv);
  }
}

// ---------------------------------------------------------------------------
// a5: one block per (local slot s, 128-column block fb of F).  Wave w owns gate
// rows fb*128 + 32w + [0, 32) and the matching up rows F + ..., so SwiGLU pairs
// registers of the same lane; the requant amax over the 128 columns is reduced
// across the four waves in LDS.
// ---------------------------------------------------------------------------
template <int NI>
__global__ __launch_bounds__(256) void k_gemm1_stream(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
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
  const size_t KB = (size_t)H / 2, KS = (size_t)H / 32;
  const uint8_t* wb = w1 + (size_t)s * 2 * F * KB;
  const uint8_t* sb = w1s + (size_t)s * 2 * F * KS;
  const int wrow[4] = {f0 + l16, f0 + 16 + l16, F + f0 + l16, F + f0 + 16 + l16};
  const int nst = H / (128 * NI);
  const int nb = H / kActBlock;
  const bool live[4] = {true, true, true, true};
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const size_t xr = (size_t)(row0 + (tv ? tok : 0));
    const uint8_t* xp = xq + xr * H + (g & 1) * 16;
    const uint8_t* xsp = xs + xr * nb;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < nst; ++st) {
      const int kbase = st * 4 * NI;
      const uint8_t* wp[4];
      const uint8_t* sp[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        wp[rt] = wb + (size_t)wrow[rt] * KB + (size_t)(kbase + g * NI) * 16;
        sp[rt] = sb + (size_t)wrow[rt] * KS + kbase + g * NI;
      }
      const int sbv = xsp[(kbase + g * NI) / 4];
      step_4tiles<NI, 4>(acc, wp, sp, xp, kbase, g, sbv, live);
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
template <int NI>
__global__ __launch_bounds__(256) void k_gemm2_stream(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_,
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
  const size_t KB = (size_t)F / 2, KS = (size_t)F / 32;
  const uint8_t* wb = w2 + (size_t)s * H * KB;
  const uint8_t* sb = w2s + (size_t)s * H * KS;
  bool live[4];
  int wrow[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    live[rt] = h0 + 16 * rt < H;
    wrow[rt] = live[rt] ? h0 + 16 * rt + l16 : 0;
  }
  const int nst = F / (128 * NI);
  const int nb = F / kActBlock;
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const size_t xr = (size_t)(row0 + (tv ? tok : 0));
    const uint8_t* xp = aq + xr * F + (g & 1) * 16;
    const uint8_t* xsp = as_ + xr * nb;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < nst; ++st) {
      const int kbase = st * 4 * NI;
      const uint8_t* wp[4];
      const uint8_t* sp[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        wp[rt] = wb + (size_t)wrow[rt] * KB + (size_t)(kbase + g * NI) * 16;
        sp[rt] = sb + (size_t)wrow[rt] * KS + kbase + g * NI;
      }
      const int sbv = xsp[(kbase + g * NI) / 4];
      step_4tiles<NI, 4>(acc, wp, sp, xp, kbase, g, sbv, live);
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

static int pick_ni(int K) {
  int nb = K / 128;
  return (nb % 4 == 0) ? 4 : (nb % 2 == 0 ? 2 : 1);
}

hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* w1,
                               const uint8_t* w1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                               hipStream_t st) {
  dim3 grid(P_local * (F / kActBlock));
  switch (pick_ni(H)) {
    case 4: k_gemm1_stream<4><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F); break;
    case 2: k_gemm1_stream<2><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F); break;
    default: k_gemm1_stream<1><<<grid, 256, 0, st>>>(xq, xs, offsets, w1, w1s, aq, as, H, F); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* w2,
                               const uint8_t* w2s, float* y, int H, int F, int P_local, hipStream_t st) {
  dim3 grid(P_local * ((H + 255) / 256));
  switch (pick_ni(F)) {
    case 4: k_gemm2_stream<4><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F); break;
    case 2: k_gemm2_stream<2><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F); break;
    default: k_gemm2_stream<1><<<grid, 256, 0, st>>>(aq, as, offsets, w2, w2s, y, H, F); break;
  }
  return hipGetLastError();
}

}  // namespace moe
