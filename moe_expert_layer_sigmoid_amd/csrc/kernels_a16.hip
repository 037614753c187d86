// a16w4 variant: bf16 activations on the MXFP4 experts, no activation
// quantisation [InferenceX PR 3430 "[AMD][MI35X] 0926 DSV4 sglang mtp
// agentic", Additional detail section: the non-EP arms run MXFP4 experts with
// bf16 activations].  gfx950's block-scaled MFMA takes fp8/fp6/fp4 operands
// only, so each weight block is expanded to bf16 in registers (exactly: an
// e2m1 value times its e8m0 scale is a bf16 with at most two significant
// bits; the hardware conversion, two values per instruction) and multiplied
// on the bf16 16x16x32 MFMA.
//
// One block of 4 waves per (local slot, 128 columns of F | 256 rows of H);
// wave w owns four weight tiles: for GEMM1 two gate tiles and the matching up
// tiles (SwiGLU pairs registers of the same lane), for GEMM2 64 rows of H.  The packed weight
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
#include "moe_pairs.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Output columns per block: GEMM1 32 per wave (two gate and two up tiles),
// GEMM2 64 per wave (four tiles of H).
template <bool G1>
constexpr int a16_cols() {
  return G1 ? 128 : 256;
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Elements [8 m, 8 m + 8) of a lane's 32-element block (dword `a` = dword m
// of its 16 bytes, element 2 q in the low nibble of byte q) as a bf16
// operand: gfx950's v_cvt_scalef32_pk_bf16_fp4 turns byte q into the two bf16
// e2m1(code) * scale, low nibble in the low half.  `scale` = 2^(sb - 127) as
// an f32; every product is exact for scale bytes 2 ... 252 (an e2m1 value
// times a power of two has at most two significant bits).
__device__ __forceinline__ v4i expand8(uint32_t a, float scale) {
  v4i r;
  r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, scale, 0));
  r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, scale, 1));
  r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, scale, 2));
  r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, scale, 3));
  return r;
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

// G1: h = W1 x (bf16 input rows of the slot's pairs), act = bf16(silu(gate) up)
// into act rows [rows, F].  G2: y = W2 act into y rows [rows, H] (f32).
// Bucketed (PAIRS false): the slot's rows are [offsets[s], offsets[s+1]), row r
// of token pair_of_row[r] / k.  Pair-indexed (PAIRS true): act and y rows are
// pair rows [T k, .], the token of pair p is p / k; GEMM1 lists the pairs p
// with phys[p] == p0 + s (ascending) itself and the slot's first block leaves
// their count in counts[s] and the list at plist + s * stride, which GEMM2
// reads.
template <bool G1, bool PAIRS>
__global__ __launch_bounds__(256, 3) void k_gemm_a16(const uint16_t* __restrict__ src, uint32_t src_bytes,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ pair_of_row,
                                                 const int32_t* __restrict__ phys, int np, int p0,
                                                 int32_t* __restrict__ counts, int32_t* __restrict__ plist,
                                                 int stride, int k,
                                                 const uint8_t* __restrict__ pw, const uint8_t* __restrict__ pws,
                                                 uint16_t* __restrict__ act, float* __restrict__ y, int H, int F) {
  __shared__ int s_list[PAIRS ? kPairMaxT : 1];
  __shared__ int s_cnt[2][4];
  constexpr int NW = 4;  // weight tiles per wave
  constexpr int kA16Cols = a16_cols<G1>(), WC = kA16Cols / 4;  // columns per block / wave
  const int K = G1 ? H : F, R = G1 ? 2 * F : H, ncol = G1 ? F : H;
  const int nfb = (ncol + kA16Cols - 1) / kA16Cols;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nfb, fb = item - s * nfb;
  int row0 = 0, n;
  if (PAIRS && G1) {
    n = min(slot_pairs(phys, np, p0 + s, s_list, kPairMaxT, s_cnt), kPairMaxT);  // block-wide (barriers)
    if (fb == 0) {
      if (threadIdx.x == 0) counts[s] = n;
      for (int i = threadIdx.x; i < n; i += blockDim.x) plist[(size_t)s * stride + i] = s_list[i];
    }
  } else if (PAIRS) {
    n = min(counts[s], kPairMaxT);
    for (int i = threadIdx.x; i < n; i += blockDim.x) s_list[i] = plist[(size_t)s * stride + i];
    __syncthreads();
  } else {
    row0 = offsets[s];
    n = offsets[s + 1] - row0;
  }
  if (n <= 0) return;  // block-uniform: an idle expert reads no weights
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int c0 = fb * kA16Cols + wave * WC;
  if (c0 >= ncol) return;  // wave-uniform (the last GEMM2 block when H % 256 == 128); no barriers below
  const PackGeom G = pack_geom((uint32_t)R, (uint32_t)K);
  const int S4 = (int)G.steps;
  // weights through a buffer over the slot's packed data: a load at the
  // buffer's size (the prefetch past the last K step) reads zeros and no memory
  const uint32_t wbytes = (uint32_t)G.data_slot;
  const rsrc_t wr = make_rsrc(pw + (size_t)s * G.data_slot, wbytes);
  uint32_t wt[NW];
  const uint8_t* wsc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    // GEMM1: gate tiles of columns c0, c0 + 16, then the matching up tiles
    const int tile = G1 ? (j >= 2 ? F : 0) / 16 + (c0 + 16 * (j & 1)) / 16 : (c0 + 16 * j) / 16;
    wt[j] = (uint32_t)tile * (uint32_t)G.data_tile + (uint32_t)lane * 16u;
    wsc[j] = pws + (size_t)s * G.scale_slot + (size_t)tile * G.scale_tile + lane * 8;
  }
  const rsrc_t xr = make_rsrc(src, src_bytes);
  const int ng = S4 / 4;  // scale groups of four K steps (S4 is a multiple of 4)

  for (int tt = 0; tt < n; tt += 16) {
    const int rr = tt + r16;
    const bool valid = rr < n;
    uint32_t boff = src_bytes;  // past the buffer: zeros
    int orow_i = 0;
    if (valid) {
      const int pr = PAIRS ? s_list[rr] : (G1 ? pair_of_row[row0 + rr] : row0 + rr);
      orow_i = PAIRS ? pr : row0 + rr;
      const int srow = G1 ? pr / k : (PAIRS ? pr : row0 + rr);
      boff = (uint32_t)srow * (uint32_t)K * 2u;
    }
    // operands of one half-step h (K step h / 2, half h % 2): the wave's
    // weight tiles and the token rows; h = 2 S4 (the prefetch past the end)
    // reads zeros
    struct Stage {
      v4i a[NW];
      v4i b[4];
    };
    auto load_stage = [&](Stage& S, int h) {
      const bool live = h < 2 * S4;
#pragma unroll
      for (int j = 0; j < NW; ++j)  // streamed once per call: non-temporal
        S.a[j] = buf_load16_p<2>(wr, live ? wt[j] : wbytes, live ? (uint32_t)h * 1024u : 0u);
      const int col = (4 * h + g) * 32;  // this lane's block, in elements
      // blocks past K (padding of the packed layout, or past the last step) take zeros
      const uint32_t o = col < K ? boff + (uint32_t)col * 2u : src_bytes;
#pragma unroll
      for (int m = 0; m < 4; ++m) S.b[m] = buf_load16(xr, o + 16u * m, 0);
    };
    auto load_sc = [&](v2i(&sc)[NW], int grp) {
#pragma unroll
      for (int j = 0; j < NW; ++j) sc[j] = *reinterpret_cast<const v2i*>(wsc[j] + (size_t)grp * 512);
    };
    v4f acc[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    // half-step bi (0..7) of the current scale group: scale byte bi of each tile
    auto mma = [&](const Stage& S, const v2i(&sc)[NW], int bi) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const uint32_t sb = ((uint32_t)(bi < 4 ? sc[j].x : sc[j].y) >> (8 * (bi & 3))) & 0xFFu;
        const float scale = __uint_as_float(sb << 23);  // 2^(sb - 127); 0 for sb = 0 (zero padding)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[j] = mfma_bf16(expand8((uint32_t)S.a[j][m], scale), S.b[m], acc[j]);
      }
    };
    // two half-steps in registers: h + 1 loads while h multiplies
    Stage s0, s1;
    v2i scc[NW], scn[NW];
    load_sc(scc, 0);
    load_stage(s0, 0);
    // (scheduling barriers keep each prefetch ahead of the previous stage's
    // multiplies: the scheduler would otherwise sink the loads and wait early)
    for (int q = 0; q < ng; ++q) {
      const int h = 8 * q;
      load_sc(scn, min(q + 1, ng - 1));
      load_stage(s1, h + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(s0, scc, 0);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s0, h + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma(s1, scc, 1);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s1, h + 3);
      __builtin_amdgcn_sched_barrier(0);
      mma(s0, scc, 2);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s0, h + 4);
      __builtin_amdgcn_sched_barrier(0);
      mma(s1, scc, 3);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s1, h + 5);
      __builtin_amdgcn_sched_barrier(0);
      mma(s0, scc, 4);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s0, h + 6);
      __builtin_amdgcn_sched_barrier(0);
      mma(s1, scc, 5);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s1, h + 7);
      __builtin_amdgcn_sched_barrier(0);
      mma(s0, scc, 6);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(s0, h + 8);
      __builtin_amdgcn_sched_barrier(0);
      mma(s1, scc, 7);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NW; ++j) scc[j] = scn[j];
    }
    if (!valid) continue;
    // lane (g, r16) holds rows 4 g + q of each weight tile for token row rr
    const size_t orow = (size_t)orow_i;
    if (G1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {  // columns c0 + 16 u + 4 g + [0, 4)
        uint32_t p[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float a0 = silu(acc[u][2 * q]) * acc[2 + u][2 * q];
          const float a1 = silu(acc[u][2 * q + 1]) * acc[2 + u][2 * q + 1];
          p[q] = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
        }
        *reinterpret_cast<uint2*>(act + orow * F + c0 + 16 * u + 4 * g) = make_uint2(p[0], p[1]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NW; ++j) *reinterpret_cast<v4f*>(y + orow * H + c0 + 16 * j + 4 * g) = acc[j];
    }
  }
}

}  // namespace

hipError_t launch_gemm1_a16(const uint16_t* x, int T, const int32_t* offsets, const int32_t* pair_of_row, int k,
                            const uint8_t* pw1, const uint8_t* pw1s, uint16_t* act, int H, int F, int P_local,
                            hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * (F / a16_cols<true>()));
  k_gemm_a16<true, false><<<grid, 256, 0, st>>>(x, (uint32_t)((size_t)T * H * 2), offsets, pair_of_row, nullptr, 0, 0,
                                                nullptr, nullptr, 0, k, pw1, pw1s, act, nullptr, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_a16(const uint16_t* act, int rows_max, const int32_t* offsets, const uint8_t* pw2,
                            const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * ((H + a16_cols<false>() - 1) / a16_cols<false>()));
  k_gemm_a16<false, false><<<grid, 256, 0, st>>>(act, (uint32_t)((size_t)rows_max * F * 2), offsets, nullptr, nullptr,
                                                 0, 0, nullptr, nullptr, 0, 1, pw2, pw2s, nullptr, y, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm1_a16_pairs(const uint16_t* x, int T, int k, const int32_t* phys, int p0, const uint8_t* pw1,
                                  const uint8_t* pw1s, uint16_t* act, int32_t* counts, int32_t* plist, int stride,
                                  int H, int F, int P_local, hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * (F / a16_cols<true>()));
  k_gemm_a16<true, true><<<grid, 256, 0, st>>>(x, (uint32_t)((size_t)T * H * 2), nullptr, nullptr, phys, T * k, p0,
                                               counts, plist, stride, k, pw1, pw1s, act, nullptr, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_a16_pairs(const uint16_t* act, int T, int k, const int32_t* counts, const int32_t* plist,
                                  int stride, const uint8_t* pw2, const uint8_t* pw2s, float* y, int H, int F,
                                  int P_local, hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * ((H + a16_cols<false>() - 1) / a16_cols<false>()));
  // the GEMM2 instance only reads counts and plist (the casts are for the shared signature)
  k_gemm_a16<false, true><<<grid, 256, 0, st>>>(act, (uint32_t)((size_t)T * k * F * 2), nullptr, nullptr, nullptr, 0,
                                                0, const_cast<int32_t*>(counts), const_cast<int32_t*>(plist), stride,
                                                1, pw2, pw2s, nullptr, y, H, F);
  return hipGetLastError();
}

}  // namespace moe
