// a16w4 variant: bf16 activations on the MXFP4 experts, no activation
// quantisation [InferenceX PR 3430 "[AMD][MI35X] 0926 DSV4 sglang mtp
// agentic", Additional detail section: the non-EP arms run MXFP4 experts with
// bf16 activations].  gfx950's block-scaled MFMA takes fp8/fp6/fp4 operands
// only, so each weight block is expanded to bf16 in registers (exactly: an
// e2m1 value times its e8m0 scale is a bf16 with at most two significant
// bits; byte-table lookups, about 2.5 integer instructions per value) and
// multiplied on the bf16 16x16x32 MFMA.
//
// One block of 4 waves per (local slot, 64 output columns); wave w owns 16
// columns: for GEMM1 the gate tile and the matching up tile (SwiGLU pairs
// registers of the same lane), for GEMM2 one tile of H.  The packed weight
// layout of the a8w4 kernels is read as is: lane 16 g + r of half-step i of K
// step st holds row r's 32-block b = 8 st + 4 i + g, and MFMA m of that
// half-step takes elements [8 m, 8 m + 8) of every lane's block -- the K order
// is a permutation of the block's columns, applied to the token operand too
// (lane 16 g + c loads token c's bf16 columns 32 b + 8 m + [0, 8)).  The
// slot's rows are taken 16 at a time, each pass streaming the weights again
// (the variant is meant for small token counts).

#include <hip/hip_runtime.h>

#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_layout.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kA16Cols = 64;  // output columns per block (16 per wave)

// bf16 bits of the eight e2m1 magnitudes v = 0 ... 7 under scale byte sb, as
// byte tables for v_perm: low bytes in l0 (v = 0..3) and l1 (v = 4..7), high
// bytes in h0 / h1.  The value is 2^(sb-127) times {0, 1/2, 1, 3/2, 2, 3, 4, 6},
// i.e. bits 0 (v = 0) and c + 64 v' with c = (sb - 1) << 7, v' = 0 for v = 1
// and v for v >= 2: the low byte depends only on the parity of sb - 1 and the
// high byte is (sb - 1) / 2 plus a carry of 0, 1 or 2.  Exact for scale bytes
// 2 ... 252, where every value is a normal bf16 (the high byte stays below 128).
struct Bf16Tab {
  uint32_t l0, l1, h0, h1;
};

__device__ __forceinline__ Bf16Tab bf16_tables(uint32_t sb) {
  const uint32_t odd = (sb - 1u) & 1u, hb = ((sb - 1u) >> 1) & 0x7Fu;
  Bf16Tab t;
  t.l0 = odd ? 0x40008000u : 0xC0800000u;
  t.l1 = odd ? 0x4000C080u : 0xC0804000u;
  t.h0 = hb * 0x01010100u + (odd ? 0x01010000u : 0u);
  t.h1 = hb * 0x01010101u + (odd ? 0x02020101u : 0x01010101u);
  return t;
}

// Elements [8 m, 8 m + 8) of a lane's 32-element block (dword `a` = dword m
// of its 16 bytes, element 2 q in the low nibble of byte q) as a bf16 operand:
// byte-table lookups of the magnitudes (v_perm selectors 0-3 pick the second
// source, 4-7 the first), the sign bits or-ed into the high bytes, then the
// low / high bytes interleaved into four dwords of two bf16 each.
__device__ __forceinline__ v4i expand8(uint32_t a, const Bf16Tab& t) {
  const uint32_t ve = a & 0x07070707u, vo = (a >> 4) & 0x07070707u;  // even / odd elements
  const uint32_t le = __builtin_amdgcn_perm(t.l1, t.l0, ve);
  const uint32_t he = __builtin_amdgcn_perm(t.h1, t.h0, ve) | ((a << 4) & 0x80808080u);
  const uint32_t lo = __builtin_amdgcn_perm(t.l1, t.l0, vo);
  const uint32_t ho = __builtin_amdgcn_perm(t.h1, t.h0, vo) | (a & 0x80808080u);
  const uint32_t e02 = __builtin_amdgcn_perm(he, le, 0x05010400u);  // elements 0, 2
  const uint32_t e46 = __builtin_amdgcn_perm(he, le, 0x07030602u);  // elements 4, 6
  const uint32_t o13 = __builtin_amdgcn_perm(ho, lo, 0x05010400u);  // elements 1, 3
  const uint32_t o57 = __builtin_amdgcn_perm(ho, lo, 0x07030602u);  // elements 5, 7
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(o13, e02, 0x05040100u);
  r[1] = (int)__builtin_amdgcn_perm(o13, e02, 0x07060302u);
  r[2] = (int)__builtin_amdgcn_perm(o57, e46, 0x05040100u);
  r[3] = (int)__builtin_amdgcn_perm(o57, e46, 0x07060302u);
  return r;
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

// G1: h = W1 x (bf16 input rows of the slot's pairs), act = bf16(silu(gate) up)
// into act rows [rows, F].  G2: y = W2 act into y rows [rows, H] (f32).
template <bool G1>
__global__ __launch_bounds__(256) void k_gemm_a16(const uint16_t* __restrict__ src, uint32_t src_bytes,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ pair_of_row, int k,
                                                 const uint8_t* __restrict__ pw, const uint8_t* __restrict__ pws,
                                                 uint16_t* __restrict__ act, float* __restrict__ y, int H, int F) {
  constexpr int NW = G1 ? 2 : 1;  // weight tiles per wave
  const int K = G1 ? H : F, R = G1 ? 2 * F : H, ncol = G1 ? F : H;
  const int nfb = ncol / kA16Cols;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nfb, fb = item - s * nfb;
  const int row0 = offsets[s], n = offsets[s + 1] - row0;
  if (n <= 0) return;  // block-uniform: an idle expert reads no weights
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int c0 = fb * kA16Cols + wave * 16;
  const PackGeom G = pack_geom((uint32_t)R, (uint32_t)K);
  const int S4 = (int)G.steps;
  const uint8_t* wd[NW];
  const uint8_t* wsc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int tile = (j == 0 ? c0 : F + c0) / 16;
    wd[j] = pw + (size_t)s * G.data_slot + (size_t)tile * G.data_tile + lane * 16;
    wsc[j] = pws + (size_t)s * G.scale_slot + (size_t)tile * G.scale_tile + lane * 8;
  }
  const rsrc_t xr = make_rsrc(src, src_bytes);

  for (int tt = 0; tt < n; tt += 16) {
    const int rr = tt + r16;
    const bool valid = rr < n;
    uint32_t boff = src_bytes;  // past the buffer: zeros
    if (valid) {
      const int srow = G1 ? pair_of_row[row0 + rr] / k : row0 + rr;
      boff = (uint32_t)srow * (uint32_t)K * 2u;
    }
    v4f acc[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    v2i sc[NW];
    for (int st = 0; st < S4; ++st) {
      if ((st & 3) == 0) {
#pragma unroll
        for (int j = 0; j < NW; ++j) sc[j] = *reinterpret_cast<const v2i*>(wsc[j] + (size_t)(st >> 2) * 512);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v4i a[NW], b[4];
#pragma unroll
        for (int j = 0; j < NW; ++j) a[j] = *reinterpret_cast<const v4i*>(wd[j] + (size_t)st * 2048 + i * 1024);
        const int col = (8 * st + 4 * i + g) * 32;  // this lane's block, in elements
        // blocks past K (padding of the packed layout) take zeros
        const uint32_t o = col < K ? boff + (uint32_t)col * 2u : src_bytes;
#pragma unroll
        for (int m = 0; m < 4; ++m) b[m] = buf_load16(xr, o + 16u * m, 0);
        const int bi = 2 * (st & 3) + i;  // scale byte of this half-step
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          const uint32_t sb = ((uint32_t)(bi < 4 ? sc[j].x : sc[j].y) >> (8 * (bi & 3))) & 0xFFu;
          const Bf16Tab tab = bf16_tables(sb);
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[j] = mfma_bf16(expand8((uint32_t)a[j][m], tab), b[m], acc[j]);
        }
      }
    }
    if (!valid) continue;
    // lane (g, r16) holds rows 4 g + q of each weight tile for token row rr
    const size_t orow = (size_t)(row0 + rr);
    if (G1) {
      uint32_t p[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float a0 = silu(acc[0][2 * q]) * acc[NW - 1][2 * q];
        const float a1 = silu(acc[0][2 * q + 1]) * acc[NW - 1][2 * q + 1];
        p[q] = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
      }
      *reinterpret_cast<uint2*>(act + orow * F + c0 + 4 * g) = make_uint2(p[0], p[1]);
    } else {
      *reinterpret_cast<v4f*>(y + orow * H + c0 + 4 * g) = acc[0];
    }
  }
}

}  // namespace

hipError_t launch_gemm1_a16(const uint16_t* x, int T, const int32_t* offsets, const int32_t* pair_of_row, int k,
                            const uint8_t* pw1, const uint8_t* pw1s, uint16_t* act, int H, int F, int P_local,
                            hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * (F / kA16Cols));
  k_gemm_a16<true><<<grid, 256, 0, st>>>(x, (uint32_t)((size_t)T * H * 2), offsets, pair_of_row, k, pw1, pw1s, act,
                                         nullptr, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_a16(const uint16_t* act, int rows_max, const int32_t* offsets, const uint8_t* pw2,
                            const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * (H / kA16Cols));
  k_gemm_a16<false><<<grid, 256, 0, st>>>(act, (uint32_t)((size_t)rows_max * F * 2), offsets, nullptr, 1, pw2, pw2s,
                                          nullptr, y, H, F);
  return hipGetLastError();
}

}  // namespace moe
