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

// Operands of K step st; `gofs` moves the weight tiles to another group of
// the wave's tiles (a uniform byte offset).
template <int WAUX>
__device__ __forceinline__ void s_load(SStage& S, const SOps& O, int st, uint32_t gofs = 0) {
  const uint32_t wo = (uint32_t)st * 2048 + gofs, xo = (uint32_t)st * 256;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    S.a[rt][0] = buf_load16_p<WAUX>(O.w, O.wt[rt], wo);
    S.a[rt][1] = buf_load16_p<WAUX>(O.w, O.wt[rt] + 1024, wo);
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

__device__ __forceinline__ void s_load_scales(SScales& C, const SOps& O, int q, uint32_t gofs = 0) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const v2i v = buf_load8(O.ws, O.wst[rt], (uint32_t)q * 512 + gofs);
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

// One token tile against G groups of four weight tiles each (group g at
// byte offsets g * gd in the data and g * sgd in the scales), streamed back
// to back: all S4 (a multiple of 4) K steps of group 0, then of group 1, ...
// Operand stages run two steps ahead and scale quads one quad ahead across
// group boundaries, so the pipeline never drains between groups; the loop has
// no branches (its last loads re-read the final steps and are never used).
// After a group's last step epi(g, acc) consumes its results and acc restarts
// at zero.  WAUX: cache policy of the weight loads.
template <int WAUX, int G, typename Epi>
__device__ __forceinline__ void stream_groups(v4f (&acc)[4], const SOps& O, int S4, uint32_t gd, uint32_t sgd,
                                              Epi&& epi) {
  SStage s0, s1;
  SScales c0, c1;
  const int nq = S4 / 4, NQ = G * nq, V = G * S4;
  static_assert(G == 1 || G == 2, "one or two groups");
  auto ld = [&](SStage& S, int v) {
    const int g = (G > 1 && v >= S4) ? 1 : 0;
    s_load<WAUX>(S, O, v - g * S4, g ? gd : 0u);
  };
  auto ldsc = [&](SScales& C, int q) {
    const int g = (G > 1 && q >= nq) ? 1 : 0;
    s_load_scales(C, O, q - g * nq, g ? sgd : 0u);
  };
  ldsc(c0, 0);
  ld(s0, 0);
  ld(s1, 1);
  ldsc(c1, min(1, NQ - 1));
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    for (int q = 0; q < nq; ++q) {
      const int st = 4 * q, v = g * S4 + st, vq = g * nq + q;
      const int sb0 = *reinterpret_cast<const int*>(O.sxs + 2 * st);
      const int sb1 = *reinterpret_cast<const int*>(O.sxs + 2 * st + 4);
      s_mma<0>(acc, s0, c0, sb0);
      ld(s0, min(v + 2, V - 2));
      s_mma<1>(acc, s1, c0, sb0);
      ld(s1, min(v + 3, V - 1));
      s_mma<2>(acc, s0, c0, sb1);
      ld(s0, min(v + 4, V - 2));
      s_mma<3>(acc, s1, c0, sb1);
      ld(s1, min(v + 5, V - 1));
      c0 = c1;
      ldsc(c1, min(vq + 2, NQ - 1));
    }
    epi(g, acc);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

// One group: all S4 steps of one token tile, results left in acc.
template <int WAUX>
__device__ __forceinline__ void stream_tile(v4f (&acc)[4], const SOps& O, int S4) {
  v4f res[4];
  stream_groups<WAUX, 1>(acc, O, S4, 0u, 0u, [&](int, const v4f(&a)[4]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) res[rt] = a[rt];
  });
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = res[rt];
}

constexpr int kMaxSteps = 64;    // K <= 16384

// Cache policy of the streamed weight loads: non-temporal (each weight byte
// is read once per call).  Measured on the decode share (512 tokens, 48
// slots): GEMM1 5.4 -> 6.3 TB/s, GEMM2 (512-row blocks) 4.9 -> 5.2 TB/s.
#ifndef MOE_G1_WAUX
#define MOE_G1_WAUX 2
#endif
#ifndef MOE_G2_WAUX
#define MOE_G2_WAUX 2
#endif
constexpr int kPairRows = kPairMaxT;  // rows of one slot on the pair-indexed path

// The pairs (t, j) whose physical slot is q, ascending, into list[0, cap);
// returns their number (the same in every thread).  256 threads; each
// iteration covers 1024 pairs, four consecutive ones per thread, placed by
// ballots within a wavefront and by the wavefront totals across the block.
__device__ __forceinline__ int4 pairs4(const int32_t* __restrict__ phys, int np, int i0) {
  if (i0 + 3 < np) return *reinterpret_cast<const int4*>(phys + i0);
  int4 v;
  v.x = i0 < np ? phys[i0] : -1;
  v.y = i0 + 1 < np ? phys[i0 + 1] : -1;
  v.z = i0 + 2 < np ? phys[i0 + 2] : -1;
  v.w = i0 + 3 < np ? phys[i0 + 3] : -1;
  return v;
}

__device__ int slot_pairs(const int32_t* __restrict__ phys, int np, int q, int* list, int cap, int (*s_cnt)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int run = 0, buf = 0;
  int4 cur = pairs4(phys, np, 4 * tid);
  for (int base = 0; base < np; base += 1024) {
    const int i0 = base + 4 * tid;
    const int4 nxt = base + 1024 < np ? pairs4(phys, np, i0 + 1024) : int4{-1, -1, -1, -1};  // one ahead
    const int v[4] = {cur.x, cur.y, cur.z, cur.w};
    int before = 0, total = 0;
    bool f[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f[m] = v[m] == q;
      const uint64_t bal = __ballot(f[m]);
      before += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      total += __popcll(bal);
    }
    if (lane == 0) s_cnt[buf][wave] = total;
    __syncthreads();
    int pos = run + before, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int cw = s_cnt[buf][w];
      pos += w < wave ? cw : 0;
      all += cw;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (f[m]) {
        if (pos < cap) list[pos] = i0 + m;
        ++pos;
      }
    run += all;
    buf ^= 1;
    cur = nxt;
  }
  __syncthreads();  // the list is complete
  return run;
}

// Stage a token tile's 128-column scales in LDS: 16 rows of 2 * S4 bytes,
// zero beyond K/128 (padded steps) and beyond the tile's rows.
template <typename Src>
__device__ __forceinline__ void stage_token_scales(uint8_t* s_xs, const uint8_t* xs, int nrow, int nb, int S4,
                                                   Src src) {
  const int pitch = 2 * S4;
  for (int i = threadIdx.x; i < 16 * pitch; i += blockDim.x) {
    const int r = i / pitch, c = i - r * pitch;
    s_xs[i] = (r < nrow && c < nb) ? xs[(size_t)src(r) * nb + c] : (uint8_t)0;
  }
}

// Rows of one slot for the streaming GEMMs.  Bucketed: the slot's rows are
// [offsets[s], offsets[s+1]) of the per-row buffers (input and output share
// the index).  Pair-indexed: the slot's pairs p (ascending), input row
// p / div (div = k for GEMM1's per-token activations, 1 for GEMM2), output
// row p.
template <bool PAIRS>
struct SlotRows {
  int n, row0, div;
  const int* list;
  __device__ int src(int r) const { return PAIRS ? list[r] / div : row0 + r; }
  __device__ int dst(int r) const { return PAIRS ? list[r] : row0 + r; }
};

template <bool PAIRS>
__device__ __forceinline__ SlotRows<PAIRS> slot_rows(const int32_t* offsets, const int32_t* phys, int np, int q,
                                                     int s, int div, int* list, int (*s_cnt)[4]) {
  SlotRows<PAIRS> R;
  R.div = div;
  R.list = list;
  if (PAIRS) {
    R.row0 = 0;
    R.n = min(slot_pairs(phys, np, q, list, kPairRows, s_cnt), kPairRows);
  } else {
    R.row0 = offsets[s];
    R.n = offsets[s + 1] - R.row0;
  }
  return R;
}

// The token operand of one 16-row tile: a buffer over the input rows and
// this lane's byte offsets.  Lanes past the tile's rows read zeros (pair-
// indexed: an offset past the buffer) or row 0 of the tile (bucketed); their
// results are never stored.
template <bool PAIRS>
__device__ __forceinline__ void token_operand(SOps& O, const uint8_t* x, const SlotRows<PAIRS>& R, int tt0, int nrow,
                                              int nsrc, int K, int l16, int g) {
  const bool tv = l16 < nrow;
  if (PAIRS) {
    const uint32_t lim = (uint32_t)nsrc * (uint32_t)K;
    O.x = make_rsrc(x, lim);
    O.xlo = tv ? (uint32_t)R.src(tt0 + l16) * (uint32_t)K + (uint32_t)g * 16 : lim;
  } else {
    O.x = make_rsrc(x + (size_t)(R.row0 + tt0) * K, (uint32_t)nrow * K);
    O.xlo = (tv ? (uint32_t)l16 : 0u) * (uint32_t)K + (uint32_t)g * 16;
  }
  O.xhi = O.xlo + 64;
}

// ---------------------------------------------------------------------------
// a5: one block per (local slot s, 128-column block fb of F).  Wave w owns the
// gate tiles of columns fb*128 + 32w + [0, 32) and the matching up tiles, so
// SwiGLU pairs registers of the same lane; the requant amax over the 128
// columns is reduced across the four waves in LDS.
//   bucketed (PAIRS false): xq/xs rows and aq/as rows from `offsets`;
//   pair-indexed (PAIRS true): xq/xs are per-token rows [nsrc = T], aq/as
//   per-pair rows [T*k]; the slot's pairs come from phys[0, np).
// ---------------------------------------------------------------------------
template <bool PAIRS>
__global__ __launch_bounds__(256, 3) void k_gemm1_stream(const uint8_t* __restrict__ xq,
                                                         const uint8_t* __restrict__ xs,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ phys, int np, int k, int p0,
                                                         int nsrc, const uint8_t* __restrict__ pw1,
                                                         const uint8_t* __restrict__ pw1s, uint8_t* __restrict__ aq,
                                                         uint8_t* __restrict__ as_, int32_t* __restrict__ counts,
                                                         int H, int F) {
  __shared__ float s_amax[4][16];
  __shared__ __align__(16) uint8_t s_xs[16 * 2 * kMaxSteps];
  __shared__ int s_list[PAIRS ? kPairRows : 1];
  __shared__ int s_cnt[2][4];
  const int nfb = F / kActBlock;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nfb, fb = item - s * nfb;
  const SlotRows<PAIRS> R = slot_rows<PAIRS>(offsets, phys, np, p0 + s, s, k, s_list, s_cnt);
  const int n = R.n;
  if (PAIRS && fb == 0 && threadIdx.x == 0) counts[s] = n;
  if (n <= 0) return;  // block-uniform: an idle expert reads no weights
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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
    stage_token_scales(s_xs, xs, nrow, nb, S4, [&](int r) { return R.src(tt0 + r); });
    __syncthreads();
    token_operand<PAIRS>(O, xq, R, tt0, nrow, nsrc, H, l16, g);
    O.sxs = s_xs + (tv ? l16 : 0) * 2 * S4;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_tile<MOE_G1_WAUX>(acc, O, S4);
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
      const size_t d = (size_t)R.dst(tok);
      uint8_t* ap = aq + d * F + f0 + 4 * g;
      *reinterpret_cast<uint32_t*>(ap) =
          pack4_fp8(ldexpf(act[0], -e), ldexpf(act[1], -e), ldexpf(act[2], -e), ldexpf(act[3], -e));
      *reinterpret_cast<uint32_t*>(ap + 16) =
          pack4_fp8(ldexpf(act[4], -e), ldexpf(act[5], -e), ldexpf(act[6], -e), ldexpf(act[7], -e));
      if (wave == 0 && g == 0) as_[d * nfb + fb] = (uint8_t)(e + 127);
    }
  }
}

// ---------------------------------------------------------------------------
// a6: one block per (local slot s, 512-row block of H).  Wave w owns rows
// hb*512 + 128w + [0, 128) as two groups of four 16-row tiles, streamed back
// to back (512-row blocks fill the chip in one round at three blocks per CU:
// 7168 / 512 * 48 slots = 672 blocks).  y rows are f32 [rows, H] (bucketed
// rows, or pair rows with the act rows pair-indexed too).
// ---------------------------------------------------------------------------
constexpr int kG2Rows = 512;

template <bool PAIRS>
__global__ __launch_bounds__(256, 3) void k_gemm2_stream(const uint8_t* __restrict__ aq,
                                                         const uint8_t* __restrict__ as_,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ phys, int np, int p0, int nsrc,
                                                         const uint8_t* __restrict__ pw2,
                                                         const uint8_t* __restrict__ pw2s, float* __restrict__ y,
                                                         int H, int F) {
  __shared__ __align__(16) uint8_t s_xs[16 * 2 * kMaxSteps];
  __shared__ int s_list[PAIRS ? kPairRows : 1];
  __shared__ int s_cnt[2][4];
  const int nhb = (H + kG2Rows - 1) / kG2Rows;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int s = item / nhb, hb = item - s * nhb;
  const SlotRows<PAIRS> R = slot_rows<PAIRS>(offsets, phys, np, p0 + s, s, 1, s_list, s_cnt);
  const int n = R.n;
  if (n <= 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int h0 = hb * kG2Rows + wave * 128;
  const bool live = h0 < H;  // wave-uniform; H is a multiple of 128 so a live wave has 8 full tiles
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
  const uint32_t gd = 4u * (uint32_t)G.data_tile, sgd = 4u * (uint32_t)G.scale_tile;
  for (int tt0 = 0; tt0 < n; tt0 += 16) {
    const int tok = tt0 + l16;
    const bool tv = tok < n;
    const int nrow = min(16, n - tt0);
    __syncthreads();
    stage_token_scales(s_xs, as_, nrow, nb, S4, [&](int r) { return R.src(tt0 + r); });
    __syncthreads();
    if (!live) continue;
    token_operand<PAIRS>(O, aq, R, tt0, nrow, nsrc, F, l16, g);
    O.sxs = s_xs + (tv ? l16 : 0) * 2 * S4;
    float* yr = tv ? y + (size_t)R.dst(tok) * H + h0 + 4 * g : nullptr;
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_groups<MOE_G2_WAUX, 2>(acc, O, S4, gd, sgd, [&](int grp, const v4f(&a)[4]) {
      if (tv) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          *reinterpret_cast<float4*>(yr + 64 * grp + 16 * rt) = make_float4(a[rt][0], a[rt][1], a[rt][2], a[rt][3]);
      }
    });
  }
}

hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                               const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                               hipStream_t st) {
  k_gemm1_stream<false><<<P_local * (F / kActBlock), 256, 0, st>>>(xq, xs, offsets, nullptr, 0, 1, 0, 0, pw1, pw1s,
                                                                   aq, as, nullptr, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                               const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  k_gemm2_stream<false><<<P_local * ((H + kG2Rows - 1) / kG2Rows), 256, 0, st>>>(aq, as, offsets, nullptr, 0, 0, 0, pw2, pw2s, y,
                                                                     H, F);
  return hipGetLastError();
}

hipError_t launch_gemm1_pairs(const uint8_t* xq_tok, const uint8_t* xs_tok, const int32_t* phys, int T, int k, int p0,
                              const uint8_t* pw1, const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int32_t* counts,
                              int H, int F, int P_local, hipStream_t st) {
  k_gemm1_stream<true><<<P_local * (F / kActBlock), 256, 0, st>>>(xq_tok, xs_tok, nullptr, phys, T * k, k, p0, T,
                                                                  pw1, pw1s, aq, as, counts, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_pairs(const uint8_t* aq, const uint8_t* as, const int32_t* phys, int T, int k, int p0,
                              const uint8_t* pw2, const uint8_t* pw2s, float* y, int H, int F, int P_local,
                              hipStream_t st) {
  k_gemm2_stream<true><<<P_local * ((H + kG2Rows - 1) / kG2Rows), 256, 0, st>>>(aq, as, nullptr, phys, T * k, p0, T * k, pw2,
                                                                    pw2s, y, H, F);
  return hipGetLastError();
}

// ===========================================================================
// Large-M path: persistent tiled kernel.
//
// Work item = (local slot s, token block of BM = 128 * TG rows, weight block
// of 256 rows: 128 gate + 128 up columns for GEMM1, 256 rows of H for
// GEMM2).  Items are listed per slot (token blocks from the slot's row count,
// read on the device) and dealt to the 8 XCDs in contiguous ranges, so the
// weight blocks of one token block run on one XCD and share its rows in L2.
//
// Block = 4 * TG waves; wave (wg, tg) owns four 16-row weight tiles (group
// wg) against eight 16-token tiles (group tg): 32 accumulators of 16x16.
// K advances 128 per stage (one MFMA per tile pair).  The token rows of a
// stage (BM x 128 B) are staged through LDS, double-buffered, pitch 144 B so
// that the 16 tokens a ds_read_b128 touches fall in distinct bank groups; the
// weight tiles stream from HBM into registers two stages ahead.
// ===========================================================================
constexpr int kLPitch = 144;

template <int TG>
struct LShared {
  uint8_t b[2][128 * TG * kLPitch];   // token stage buffers
  uint8_t xs[128 * TG * 128];          // 128-column scales of the block's tokens (K <= 16384)
  float amax[TG][4][128];              // GEMM1 requant: per-token amax of each weight group
  int prefix[1025];                    // exclusive prefix of token blocks per slot
};

// Token block count prefix over slots, computed by every block (P_local <= 1024).
template <int TG>
__device__ __forceinline__ int block_prefix(LShared<TG>& S, const int32_t* offsets, int P_local) {
  constexpr int BM = 128 * TG;
  const int tid = threadIdx.x;
  for (int p = tid; p < P_local; p += blockDim.x) {
    const int n = offsets[p + 1] - offsets[p];
    S.prefix[p + 1] = (n + BM - 1) / BM;
  }
  if (tid == 0) S.prefix[0] = 0;
  __syncthreads();
  if (tid == 0) {  // P_local serial adds: negligible next to one item
    int run = 0;
    for (int p = 1; p <= P_local; ++p) {
      run += S.prefix[p];
      S.prefix[p] = run;
    }
  }
  __syncthreads();
  return S.prefix[P_local];
}

template <int TG, bool G1>
__global__ __launch_bounds__(256 * TG, 1) void k_tiled(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const int32_t* __restrict__ offsets,
    int P_local, const uint8_t* __restrict__ pw, const uint8_t* __restrict__ pws, uint8_t* __restrict__ aq,
    uint8_t* __restrict__ as_, float* __restrict__ y, int H, int F) {
  constexpr int BM = 128 * TG;
  __shared__ LShared<TG> S;
  const int K = G1 ? H : F;
  const int R = G1 ? 2 * F : H;
  const int nblk = G1 ? F / kActBlock : (H + 255) / 256;
  const int nb = K / kActBlock;      // 128-wide K stages (real)
  const PackGeom Gm = pack_geom((uint32_t)R, (uint32_t)K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int l16 = lane & 15, g = lane >> 4;
  const int wg = wave & 3, tg = wave >> 2;

  const int nitems = block_prefix<TG>(S, offsets, P_local) * nblk;
  // contiguous item range per XCD; blocks of one XCD stride through it
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int chunk = (nitems + 7) / 8;
  const int i0 = xcd * chunk, i1 = min(nitems, i0 + chunk);

  for (int item = i0 + lb; item < i1; item += nper) {
    const int tb = item / nblk, wb = item - tb * nblk;
    // slot of token block tb: last s with prefix[s] <= tb
    int lo = 0, hi = P_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (S.prefix[mid] <= tb) lo = mid;
      else hi = mid - 1;
    }
    const int s = lo;
    const int bm = tb - S.prefix[s];
    const int n = offsets[s + 1] - offsets[s];
    const int r0 = offsets[s] + bm * BM;
    const int nvalid = min(BM, n - bm * BM);

    // weight tiles of this wave
    int tile[4];
    bool wlive = true;
    if (G1) {
      const int f0 = wb * kActBlock + wg * 32;
      tile[0] = f0 / 16; tile[1] = f0 / 16 + 1; tile[2] = (F + f0) / 16; tile[3] = (F + f0) / 16 + 1;
    } else {
      const int h0 = wb * 256 + wg * 64;
      wlive = h0 < H;  // H is a multiple of 128: a live wave has four full tiles
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) tile[rt] = wlive ? h0 / 16 + rt : 0;
    }
    const rsrc_t Wr = make_rsrc(pw + (size_t)s * Gm.data_slot, (uint32_t)Gm.data_slot);
    const rsrc_t Sr = make_rsrc(pws + (size_t)s * Gm.scale_slot, (uint32_t)Gm.scale_slot);
    uint32_t wt[4], wst[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      wt[rt] = (uint32_t)tile[rt] * (uint32_t)Gm.data_tile + 16u * lane;
      wst[rt] = (uint32_t)tile[rt] * (uint32_t)Gm.scale_tile + 8u * lane;
    }
    const int ntt = min(8, max(0, (nvalid - tg * 128 + 15) / 16));  // token tiles of this wave

    __syncthreads();  // the previous item is done with S.b / S.xs / S.amax
    for (int i = tid; i < BM * nb; i += blockDim.x) {
      const int t = i / nb, c = i - t * nb;
      S.xs[t * nb + c] = t < nvalid ? xs[(size_t)(r0 + t) * nb + c] : (uint8_t)0;
    }
    // token stage loader: 16-byte chunks, 8 per token row; two register sets
    // so that a stage's rows are loaded three stages before use and written
    // to LDS one stage before use
    const rsrc_t Xr = make_rsrc(xq + (size_t)r0 * K, (uint32_t)nvalid * K);
    uint4 breg0[4], breg1[4];
    auto b_load = [&](uint4 (&br)[4], int stg) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = tid + j * 256 * TG;  // chunk: token c / 8, piece c % 8
        const int t = c >> 3, pc = c & 7;
        br[j] = __builtin_bit_cast(uint4, buf_load16(Xr, (uint32_t)t * K + pc * 16, (uint32_t)stg * 128));
      }
    };
    auto b_store = [&](const uint4 (&br)[4], int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = tid + j * 256 * TG;
        const int t = c >> 3, pc = c & 7;
        *reinterpret_cast<uint4*>(&S.b[buf][t * kLPitch + pc * 16]) = br[j];
      }
    };
    v4i a0[4], a1[4];
    auto a_load = [&](v4i (&a)[4], int stg) {
      const uint32_t so = (uint32_t)(stg >> 1) * 2048 + (uint32_t)(stg & 1) * 1024;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = buf_load16(Wr, wt[rt], so);
    };
    v2i scur[4], snext[4];
    auto s_loadq = [&](v2i (&sc)[4], int grp) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sc[rt] = buf_load8(Sr, wst[rt], (uint32_t)grp * 512);
    };

    v4f acc[4][8];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[rt][tt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int ngrp = Gm.steps / 4;  // scale groups of 8 stages
    // prologue: rows of stages 0 and 1 to LDS, stage 2 in flight; weights of stages 0, 1
    b_load(breg0, 0);
    if (nb > 1) b_load(breg1, 1);
    s_loadq(scur, 0);
    s_loadq(snext, min(1, ngrp - 1));
    if (wlive) {
      a_load(a0, 0);
      if (nb > 1) a_load(a1, 1);
    }
    b_store(breg0, 0);
    if (nb > 1) b_store(breg1, 1);
    if (nb > 2) b_load(breg0, 2);

    auto stage = [&](const v4i (&a)[4], int stg) {
      const int buf = stg & 1;
      if (wlive) {
        const int sh = 8 * (stg & 3);
        int sa[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) sa[rt] = (int)((uint32_t)((stg & 4) ? scur[rt].y : scur[rt].x) >> sh);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          if (tt >= ntt) continue;  // wave-uniform
          const int tok = tg * 128 + tt * 16 + l16;
          const uint8_t* bp = &S.b[buf][tok * kLPitch + g * 16];
          V8 b;
          b.h[0] = *reinterpret_cast<const v4i*>(bp);
          b.h[1] = *reinterpret_cast<const v4i*>(bp + 64);
          const int sb = S.xs[tok * nb + stg];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[rt][tt] = mfma_ij<0, 0>(a[rt], b.v, acc[rt][tt], sa[rt], sb);
          // keep the operand reads of one token tile next to its MFMAs
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // Stage stg reads LDS buffer stg & 1.  At its start (after the barrier)
    // the rows of stage stg + 1 go from registers to the other buffer, whose
    // readers (stage stg - 1) are past the barrier; the rows of stage stg + 3
    // are requested into the register set just emptied.
    for (int stg = 0; stg < nb; stg += 2) {
      __syncthreads();
      if (stg > 0 && stg + 1 < nb) b_store(breg1, 1);
      if (stg + 3 < nb) b_load(breg1, stg + 3);
      stage(a0, stg);
      if (wlive && stg + 2 < nb) a_load(a0, stg + 2);
      if (stg + 1 < nb) {
        __syncthreads();
        if (stg + 2 < nb) b_store(breg0, 0);
        if (stg + 4 < nb) b_load(breg0, stg + 4);
        stage(a1, stg + 1);
        if (wlive && stg + 3 < nb) a_load(a1, stg + 3);
      }
      if (((stg + 2) & 7) == 0) {  // next scale group
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) scur[rt] = snext[rt];
        s_loadq(snext, min((stg + 2) / 8 + 1, ngrp - 1));
      }
    }

    // ---- epilogue
    if (G1) {
      // SwiGLU in place: acc[0] / acc[1] become act of the gate tiles' columns
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[0][tt][r] = silu(acc[0][tt][r]) * acc[2][tt][r];
          acc[1][tt][r] = silu(acc[1][tt][r]) * acc[3][tt][r];
        }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fmaxf(fabsf(acc[0][tt][r]), fabsf(acc[1][tt][r])));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0) S.amax[tg][wg][tt * 16 + l16] = m;
      }
      __syncthreads();
      const int nfb = F / kActBlock;
      const int f0 = wb * kActBlock + wg * 32;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tl = tt * 16 + l16;
        const int tok = tg * 128 + tl;
        if (tt >= ntt || tok >= nvalid) continue;
        const float am = fmaxf(fmaxf(S.amax[tg][0][tl], S.amax[tg][1][tl]),
                               fmaxf(S.amax[tg][2][tl], S.amax[tg][3][tl]));
        const int e = scale_exp(am);
        uint8_t* ap = aq + (size_t)(r0 + tok) * F + f0 + 4 * g;
        *reinterpret_cast<uint32_t*>(ap) = pack4_fp8(ldexpf(acc[0][tt][0], -e), ldexpf(acc[0][tt][1], -e),
                                                     ldexpf(acc[0][tt][2], -e), ldexpf(acc[0][tt][3], -e));
        *reinterpret_cast<uint32_t*>(ap + 16) = pack4_fp8(ldexpf(acc[1][tt][0], -e), ldexpf(acc[1][tt][1], -e),
                                                          ldexpf(acc[1][tt][2], -e), ldexpf(acc[1][tt][3], -e));
        if (wg == 0 && g == 0) as_[(size_t)(r0 + tok) * nfb + wb] = (uint8_t)(e + 127);
      }
    } else if (wlive) {
      const int h0 = wb * 256 + wg * 64;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tok = tg * 128 + tt * 16 + l16;
        if (tt >= ntt || tok >= nvalid) continue;
        float* yr = y + (size_t)(r0 + tok) * H + h0 + 4 * g;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          *reinterpret_cast<float4*>(yr + 16 * rt) =
              make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
      }
    }
  }
}

static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

hipError_t launch_gemm1_tiled(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                              const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                              hipStream_t st) {
  k_tiled<1, true><<<num_cus() / 8 * 8, 256, 0, st>>>(xq, xs, offsets, P_local, pw1, pw1s, aq, as, nullptr, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  k_tiled<1, false><<<num_cus() / 8 * 8, 256, 0, st>>>(aq, as, offsets, P_local, pw2, pw2s, nullptr, nullptr, y, H,
                                                       F);
  return hipGetLastError();
}

}  // namespace moe
