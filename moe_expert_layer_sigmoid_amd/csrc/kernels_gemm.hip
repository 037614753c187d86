// Grouped expert GEMMs on block-scaled fp8 x MXFP4 MFMA (gfx950), and the
// one-time repack of MXFP4 weights into MFMA-operand order (moe_layout.hpp):
//   a5  GEMM1 (gate/up) + SwiGLU + fp8 requant
//   a6  GEMM2 (down) into an f32 row buffer (the combine reads it)
// The operator runs GEMM1 then GEMM2 on the routed experts, with fp8
// activations on MXFP4 experts [sglang PR 47065 "Use the aiter MegaMoE small-
// and large-input paths", intro; InferenceX PR 3430, Additional detail section].
//
// Weight-streaming design for few rows per expert ("swap-AB"): the MFMA's
// 16-row A side is 16 weight rows, its 16-column B side is 16 token rows of
// one expert.  Each wave owns four 16-row weight tiles and streams them from
// HBM once per 16 tokens, two K steps ahead, as contiguous 1 KB loads; the
// token rows come from the bucketed fp8 buffer (L2-resident) and their
// 128-column scales are staged in LDS once per token tile.
//
// Operand layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (measured on gfx950):
//  - e2m1 operand: lane l holds row l%16, K elements [32g, 32g+32), g = l/16,
//    packed two per byte (low nibble first) in its 4 low dwords;
//  - e4m3 operand: lane l holds row l%16, K [16g, 16g+16) in dwords 0-3 and
//    K [64+16g, 64+16g+16) in dwords 4-7;
//  - scales: lane l supplies the e8m0 scale of row l%16, K block g (32 wide),
//    op_sel choosing the byte of the scale register;
//  - result: lane l, element r holds D[4g + r][l%16].

#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_layout.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Repack (pure byte movement, see moe_layout.hpp)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack_data(const uint8_t* __restrict__ w, uint8_t* __restrict__ pw,
                                                   uint32_t P, uint32_t R, uint32_t K, uint32_t S4) {
  const uint32_t tiles = R / 16;
  const size_t n = (size_t)P * tiles * S4 * 128;  // 16-byte chunks
  const size_t KB = K / 2;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (size_t)gridDim.x * blockDim.x) {
    const uint32_t lane = c % 64, i = (c / 64) % 2;
    const uint32_t st = (c / 128) % S4;
    const size_t tile = (c / (128ull * S4)) % tiles;
    const size_t slot = c / (128ull * S4 * tiles);
    const uint32_t r = lane % 16, g = lane / 16;
    const uint32_t blk = st * 8 + 4 * i + g;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (blk * 32 < K) v = *reinterpret_cast<const uint4*>(w + (slot * R + tile * 16 + r) * KB + (size_t)blk * 16);
    *reinterpret_cast<uint4*>(pw + c * 16) = v;
  }
}

__global__ __launch_bounds__(256) void k_pack_scales(const uint8_t* __restrict__ ws, uint8_t* __restrict__ ps,
                                                     uint32_t P, uint32_t R, uint32_t K, uint32_t S4) {
  const uint32_t tiles = R / 16, nq = S4 / 4, KS = K / 32;
  const size_t n = (size_t)P * tiles * nq * 64;  // 8-byte chunks
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (size_t)gridDim.x * blockDim.x) {
    const uint32_t lane = c % 64;
    const uint32_t q = (c / 64) % nq;
    const size_t tile = (c / (64ull * nq)) % tiles;
    const size_t slot = c / (64ull * nq * tiles);
    const uint32_t r = lane % 16, g = lane / 16;
    const uint8_t* row = ws + (slot * R + tile * 16 + r) * KS;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {  // byte b = 2 * j + i
      const uint32_t j = b / 2, i = b % 2;
      const uint32_t blk = (4 * q + j) * 8 + 4 * i + g;
      const uint32_t v = blk < KS ? row[blk] : 0u;
      if (b < 4) lo |= v << (8 * b);
      else hi |= v << (8 * (b - 4));
    }
    *reinterpret_cast<uint2*>(ps + c * 8) = make_uint2(lo, hi);
  }
}

hipError_t launch_pack(const uint8_t* w, const uint8_t* ws, uint8_t* pw, uint8_t* ps, int P, int R, int K,
                       hipStream_t st) {
  const PackGeom g = pack_geom((uint32_t)R, (uint32_t)K);
  k_pack_data<<<2048, 256, 0, st>>>(w, pw, (uint32_t)P, (uint32_t)R, (uint32_t)K, g.steps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_pack_scales<<<1024, 256, 0, st>>>(ws, ps, (uint32_t)P, (uint32_t)R, (uint32_t)K, g.steps);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming core
// ---------------------------------------------------------------------------
union V8 {
  v8i v;
  v4i h[2];
};

template <int IA, int IB>
__device__ __forceinline__ v4f mfma_ij(v4i a, v8i b, v4f c, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, kFmtFp4, kFmtFp8, IA, sa, IB, sb);
}

// One wave's operands: packed weight tiles (A) and one token tile (B).
struct SOps {
  rsrc_t w;            // packed data of the slot
  rsrc_t ws;           // packed scales of the slot
  rsrc_t x;            // the token tile's rows
  uint32_t wt[4];      // tile * data_tile + 16 * lane
  uint32_t wst[4];     // tile * scale_tile + 8 * lane
  uint32_t xlo, xhi;   // token row * K + 16 g, + 64
  const uint8_t* sxs;  // LDS: this lane's token's 128-column scales (zero-padded)
};

struct SStage {
  v4i a[4][2];
  V8 b[2];
};

__device__ __forceinline__ void s_load(SStage& S, const SOps& O, int st) {
  const uint32_t wo = (uint32_t)st * 2048, xo = (uint32_t)st * 256;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    S.a[rt][0] = buf_load16(O.w, O.wt[rt], wo);
    S.a[rt][1] = buf_load16(O.w, O.wt[rt] + 1024, wo);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    S.b[i].h[0] = buf_load16(O.x, O.xlo + i * 128, xo);
    S.b[i].h[1] = buf_load16(O.x, O.xhi + i * 128, xo);
  }
}

struct SScales {
  int lo[4], hi[4];  // steps 4q, 4q+1 (lo) and 4q+2, 4q+3 (hi) of each tile
};

__device__ __forceinline__ void s_load_scales(SScales& C, const SOps& O, int q) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const v2i v = buf_load8(O.ws, O.wst[rt], (uint32_t)q * 512);
    C.lo[rt] = v.x;
    C.hi[rt] = v.y;
  }
}

// Step with in-quad index J (0..3): A scale byte 2 * (J % 2) + i of the
// (lo | hi) dword, B scale byte 2 * (J % 2) + i of the pair's dword `sb`.
template <int J>
__device__ __forceinline__ void s_mma(v4f (&acc)[4], const SStage& S, const SScales& C, int sb) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int sa = (J < 2) ? C.lo[rt] : C.hi[rt];
    acc[rt] = mfma_ij<2 * (J % 2), 2 * (J % 2)>(S.a[rt][0], S.b[0].v, acc[rt], sa, sb);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int sa = (J < 2) ? C.lo[rt] : C.hi[rt];
    acc[rt] = mfma_ij<2 * (J % 2) + 1, 2 * (J % 2) + 1>(S.a[rt][1], S.b[1].v, acc[rt], sa, sb);
  }
}

// All S4 (a multiple of 4) steps of one token tile.  Operand stages run two
// steps ahead, scale quads one quad ahead; the loop has no branches (its last
// loads re-read the final steps and are never used).
__device__ __forceinline__ void stream_tile(v4f (&acc)[4], const SOps& O, int S4) {
  SStage s0, s1;
  SScales c0, c1;
  const int nq = S4 / 4;
  s_load_scales(c0, O, 0);
  s_load(s0, O, 0);
  s_load(s1, O, 1);
  s_load_scales(c1, O, min(1, nq - 1));
  for (int st = 0; st < S4; st += 4) {
    const int sb0 = *reinterpret_cast<const int*>(O.sxs + 2 * st);
    const int sb1 = *reinterpret_cast<const int*>(O.sxs + 2 * st + 4);
    s_mma<0>(acc, s0, c0, sb0);
    s_load(s0, O, min(st + 2, S4 - 2));
    s_mma<1>(acc, s1, c0, sb0);
    s_load(s1, O, min(st + 3, S4 - 1));
    s_mma<2>(acc, s0, c0, sb1);
    s_load(s0, O, min(st + 4, S4 - 2));
    s_mma<3>(acc, s1, c0, sb1);
    s_load(s1, O, min(st + 5, S4 - 1));
    c0 = c1;
    s_load_scales(c1, O, min(st / 4 + 2, nq - 1));
  }
}

// Stage the token tile's 128-column scales in LDS: rows of 2 * S4 bytes,
// zero beyond K/128 (padded steps).
__device__ __forceinline__ void stage_token_scales(uint8_t* s_xs, const uint8_t* xs, int nrow, int nb, int S4) {
  const int pitch = 2 * S4;
  for (int i = threadIdx.x; i < 16 * pitch; i += blockDim.x) {
    const int r = i / pitch, c = i - r * pitch;
    s_xs[i] = (r < nrow && c < nb) ? xs[(size_t)r * nb + c] : (uint8_t)0;
  }
}

constexpr int kMaxSteps = 64;  // K <= 16384

// ---------------------------------------------------------------------------
// a5: one block per (local slot s, 128-column block fb of F).  Wave w owns the
// gate tiles of columns fb*128 + 32w + [0, 32) and the matching up tiles, so
// SwiGLU pairs registers of the same lane; the requant amax over the 128
// columns is reduced across the four waves in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 3) void k_gemm1_stream(const uint8_t* __restrict__ xq,
                                                         const uint8_t* __restrict__ xs,
                                                         const int32_t* __restrict__ offsets,
                                                         const uint8_t* __restrict__ pw1,
                                                         const uint8_t* __restrict__ pw1s, uint8_t* __restrict__ aq,
                                                         uint8_t* __restrict__ as_, int H, int F) {
  __shared__ float s_amax[4][16];
  __shared__ __align__(16) uint8_t s_xs[16 * 2 * kMaxSteps];
  const int nfb = F / kActBlock;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nfb, fb = item - s * nfb;
  const int row0 = offsets[s];
  const int n = offsets[s + 1] - row0;
  if (n <= 0) return;  // block-uniform: an idle expert reads no weights
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const PackGeom G = pack_geom(2u * F, (uint32_t)H);
  const int S4 = (int)G.steps;
  const int nb = H / kActBlock;
  const int f0 = fb * kActBlock + wave * 32;
  SOps O;
  O.w = make_rsrc(pw1 + (size_t)s * G.data_slot, (uint32_t)G.data_slot);
  O.ws = make_rsrc(pw1s + (size_t)s * G.scale_slot, (uint32_t)G.scale_slot);
  const int tile[4] = {f0 / 16, f0 / 16 + 1, (F + f0) / 16, (F + f0) / 16 + 1};
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    O.wt[rt] = (uint32_t)tile[rt] * (uint32_t)G.data_tile + 16u * lane;
    O.wst[rt] = (uint32_t)tile[rt] * (uint32_t)G.scale_tile + 8u * lane;
  }
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const int nrow = min(16, n - tt0);
    __syncthreads();  // previous tile's readers of s_xs / s_amax are done
    stage_token_scales(s_xs, xs + (size_t)(row0 + tt0) * nb, nrow, nb, S4);
    __syncthreads();
    const uint32_t tr = tv ? (uint32_t)l16 : 0u;
    O.x = make_rsrc(xq + (size_t)(row0 + tt0) * H, (uint32_t)nrow * H);
    O.xlo = tr * (uint32_t)H + (uint32_t)g * 16;
    O.xhi = O.xlo + 64;
    O.sxs = s_xs + tr * 2 * S4;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_tile(acc, O, S4);
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
__global__ __launch_bounds__(256, 3) void k_gemm2_stream(const uint8_t* __restrict__ aq,
                                                         const uint8_t* __restrict__ as_,
                                                         const int32_t* __restrict__ offsets,
                                                         const uint8_t* __restrict__ pw2,
                                                         const uint8_t* __restrict__ pw2s, float* __restrict__ y,
                                                         int H, int F) {
  __shared__ __align__(16) uint8_t s_xs[16 * 2 * kMaxSteps];
  const int nhb = (H + 255) / 256;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nhb, hb = item - s * nhb;
  const int row0 = offsets[s];
  const int n = offsets[s + 1] - row0;
  if (n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int h0 = hb * 256 + wave * 64;
  const bool live = h0 < H;  // wave-uniform; H is a multiple of 128 so a live wave has 4 full tiles
  const PackGeom G = pack_geom((uint32_t)H, (uint32_t)F);
  const int S4 = (int)G.steps;
  const int nb = F / kActBlock;
  SOps O;
  O.w = make_rsrc(pw2 + (size_t)s * G.data_slot, (uint32_t)G.data_slot);
  O.ws = make_rsrc(pw2s + (size_t)s * G.scale_slot, (uint32_t)G.scale_slot);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const uint32_t tile = live ? (uint32_t)(h0 / 16 + rt) : 0u;
    O.wt[rt] = tile * (uint32_t)G.data_tile + 16u * lane;
    O.wst[rt] = tile * (uint32_t)G.scale_tile + 8u * lane;
  }
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const int nrow = min(16, n - tt0);
    __syncthreads();
    stage_token_scales(s_xs, as_ + (size_t)(row0 + tt0) * nb, nrow, nb, S4);
    __syncthreads();
    if (!live) continue;
    const uint32_t tr = tv ? (uint32_t)l16 : 0u;
    O.x = make_rsrc(aq + (size_t)(row0 + tt0) * F, (uint32_t)nrow * F);
    O.xlo = tr * (uint32_t)F + (uint32_t)g * 16;
    O.xhi = O.xlo + 64;
    O.sxs = s_xs + tr * 2 * S4;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_tile(acc, O, S4);
    if (tv) {
      float* yr = y + (size_t)(row0 + tok) * H + h0 + 4 * g;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        *reinterpret_cast<float4*>(yr + 16 * rt) = make_float4(acc[rt][0], acc[rt][1], acc[rt][2], acc[rt][3]);
    }
  }
}

hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                               const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                               hipStream_t st) {
  k_gemm1_stream<<<P_local * (F / kActBlock), 256, 0, st>>>(xq, xs, offsets, pw1, pw1s, aq, as, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                               const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  k_gemm2_stream<<<P_local * ((H + 255) / 256), 256, 0, st>>>(aq, as, offsets, pw2, pw2s, y, H, F);
  return hipGetLastError();
}

}  // namespace moe
