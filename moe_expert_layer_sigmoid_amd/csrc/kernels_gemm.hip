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
#include "moe_pairs.hpp"

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

// `p`, with the compiler kept from assuming it is the same value as before
// (it stops loop-invariant code motion of what is derived from it).
template <typename T>
__device__ __forceinline__ T* opaque(T* p) {
  asm volatile("" : "+s"(p));
  return p;
}

template <int IA, int IB>
__device__ __forceinline__ v4f mfma_ij(v4i a, v8i b, v4f c, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, kFmtFp4, kFmtFp8, IA, sa, IB, sb);
}

// One wave's operands: packed weight tiles (A) and NT token tiles (B) that
// share each weight load.  UT: the tile offsets wt / wst are wave-uniform
// (scalar registers) and the lane's own offset is wl / sl; otherwise wt / wst
// hold the lane's full offsets.  (GEMM2 takes the uniform form, GEMM1 the
// per-lane one: with these, each fits its 168-register budget without
// spilling.)
template <int NT, bool UT = false>
struct SOps {
  rsrc_t w;                // packed data of the slot
  rsrc_t ws;               // packed scales of the slot
  rsrc_t x;                // the token rows
  uint32_t wl;             // UT: 16 * lane, the lane's bytes in a 1 KB weight load
  uint32_t sl;             // UT: 8 * lane, the lane's bytes in a 512 B scale load
  uint32_t wt[4];          // tile * data_tile (+ 16 * lane unless UT)
  uint32_t wst[4];         // tile * scale_tile (+ 8 * lane unless UT)
  uint32_t xlo[NT];        // per token tile: token row * K + 16 g (past the buffer: zeros)
  uint32_t kx;             // K of the token rows (bytes)
  uint32_t lim;            // the token buffer's size: offsets from here read zeros
  const uint8_t* sxs[NT];  // LDS: this lane's token's 128-column scales (zero-padded)
};

template <int NT>
struct SStage {
  v4i a[4][2];
  V8 b[NT][2];
};

// Operands of K step st; `gofs` moves the weight tiles to another group of
// the wave's tiles (a uniform byte offset).  dead: a load past the stream's
// last step, issued only to keep the loop free of branches and never used;
// it goes through a zero-sized buffer (no memory access, zeros back at once)
// so that a later wait for the stream's loads does not wait for a re-read.
template <int WAUX, int NT, bool UT>
__device__ __forceinline__ void s_load(SStage<NT>& S, const SOps<NT, UT>& O, int st, uint32_t gofs = 0,
                                       bool dead = false) {
  const uint32_t wo = (uint32_t)st * 2048 + gofs, xo = (uint32_t)st * 256;
  const rsrc_t W = dead ? make_rsrc(nullptr, 0u) : O.w;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if constexpr (UT) {
      S.a[rt][0] = buf_load16_p<WAUX>(W, O.wl, O.wt[rt] + wo);
      S.a[rt][1] = buf_load16_p<WAUX>(W, O.wl, O.wt[rt] + wo + 1024);
    } else {
      S.a[rt][0] = buf_load16_p<WAUX>(W, O.wt[rt], wo);
      S.a[rt][1] = buf_load16_p<WAUX>(W, O.wt[rt] + 1024, wo);
    }
  }
  // Steps past K (the packed weights pad K to a multiple of 1024) take zero
  // tokens, not the bytes after the row: those may belong to rows nothing
  // wrote (pair rows of remote pairs) and hold fp8 NaN codes, which a zero
  // weight would not cancel.  Each 128-column half-step is whole (K is a
  // multiple of 128), so the test is uniform.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool live = !dead && xo + (uint32_t)i * 128 < O.kx;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t b = live ? O.xlo[n] : O.lim;
      S.b[n][i].h[0] = buf_load16(O.x, b + i * 128, xo);
      S.b[n][i].h[1] = buf_load16(O.x, b + 64 + i * 128, xo);
    }
  }
}

struct SScales {
  int lo[4], hi[4];  // steps 4q, 4q+1 (lo) and 4q+2, 4q+3 (hi) of each tile
};

template <int NT, bool UT>
__device__ __forceinline__ void s_load_scales(SScales& C, const SOps<NT, UT>& O, int q, uint32_t gofs = 0) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const v2i v = UT ? buf_load8(O.ws, O.sl, O.wst[rt] + (uint32_t)q * 512 + gofs)
                     : buf_load8(O.ws, O.wst[rt], (uint32_t)q * 512 + gofs);
    C.lo[rt] = v.x;
    C.hi[rt] = v.y;
  }
}

// Step with in-quad index J (0..3): A scale byte 2 * (J % 2) + i of the
// (lo | hi) dword, B scale byte 2 * (J % 2) + i of token tile n's dword sb[n].
template <int J, int NT>
__device__ __forceinline__ void s_mma(v4f (&acc)[4][NT], const SStage<NT>& S, const SScales& C, const int (&sb)[NT]) {
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int sa = (J < 2) ? C.lo[rt] : C.hi[rt];
      acc[rt][n] = mfma_ij<2 * (J % 2), 2 * (J % 2)>(S.a[rt][0], S.b[n][0].v, acc[rt][n], sa, sb[n]);
    }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int sa = (J < 2) ? C.lo[rt] : C.hi[rt];
      acc[rt][n] = mfma_ij<2 * (J % 2) + 1, 2 * (J % 2) + 1>(S.a[rt][1], S.b[n][1].v, acc[rt][n], sa, sb[n]);
    }
}

// NT token tiles against G groups of four weight tiles each (group g at
// byte offsets g * gd in the data and g * sgd in the scales), streamed back
// to back: all S4 (a multiple of 4) K steps of group 0, then of group 1, ...
// Operand stages run two steps ahead and scale quads one quad ahead across
// group boundaries (each quad's scales issued before the previous quad's
// operand loads), so the pipeline never drains between quads or groups; the loop has
// no branches (its last loads, past the final step, go through a zero-sized
// buffer and are never used).
// After a group's last step epi(g, acc) consumes its results and acc restarts
// at zero.  WAUX: cache policy of the weight loads.  The S4 steps are steps
// st0 .. st0 + S4 - 1 of K (st0 a multiple of 4: a range of whole quads).
template <int WAUX, int G, int NT, bool UT, typename Epi>
__device__ __forceinline__ void stream_groups(v4f (&acc)[4][NT], const SOps<NT, UT>& O, int S4, uint32_t gd, uint32_t sgd,
                                              int st0, Epi&& epi) {
  SStage<NT> s0, s1;
  SScales c0, c1;
  const int nq = S4 / 4, NQ = G * nq, V = G * S4;
  static_assert(G == 1 || G == 2, "one or two groups");
  auto ld = [&](SStage<NT>& S, int v) {  // v >= V: a dead load (past the stream's end)
    const bool dead = v >= V;
    const int vv = dead ? V - 1 : v;
    const int g = (G > 1 && vv >= S4) ? 1 : 0;
    s_load<WAUX>(S, O, st0 + vv - g * S4, g ? gd : 0u, dead);
  };
  auto ldsc = [&](SScales& C, int q) {
    const int g = (G > 1 && q >= nq) ? 1 : 0;
    s_load_scales(C, O, (st0 >> 2) + q - g * nq, g ? sgd : 0u);
  };
  ldsc(c1, 0);
  ld(s0, 0);
  ld(s1, 1);
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    for (int q = 0; q < nq; ++q) {
      const int st = 4 * q, v = g * S4 + st, vq = g * nq + q;
      // this quad's scales, loaded a quad ahead and before that quad's operand
      // loads: waiting for them (the copy) never waits for operands in flight,
      // which a scale load issued after them would make it do
      c0 = c1;
      ldsc(c1, min(vq + 1, NQ - 1));
      __builtin_amdgcn_sched_barrier(0);
      int sb0[NT], sb1[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        sb0[n] = *reinterpret_cast<const int*>(O.sxs[n] + 2 * (st0 + st));
        sb1[n] = *reinterpret_cast<const int*>(O.sxs[n] + 2 * (st0 + st) + 4);
      }
      s_mma<0>(acc, s0, c0, sb0);
      ld(s0, v + 2);
      s_mma<1>(acc, s1, c0, sb0);
      ld(s1, v + 3);
      s_mma<2>(acc, s0, c0, sb1);
      ld(s0, v + 4);
      s_mma<3>(acc, s1, c0, sb1);
      ld(s1, v + 5);
    }
    epi(g, acc);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[rt][n] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

// One group: S4 steps (from step st0) of NT token tiles, results left in acc.
template <int WAUX, int NT, bool UT>
__device__ __forceinline__ void stream_tile(v4f (&acc)[4][NT], const SOps<NT, UT>& O, int S4, int st0) {
  v4f res[4][NT];
  stream_groups<WAUX, 1>(acc, O, S4, 0u, 0u, st0, [&](int, const v4f(&a)[4][NT]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int n = 0; n < NT; ++n) res[rt][n] = a[rt][n];
  });
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[rt][n] = res[rt][n];
}

constexpr int kMaxSteps = 64;    // K <= 16384

// Cache policy of the streamed weight loads: non-temporal (each weight byte
// is read once per call).  Measured on the decode share (512 tokens, 48
// slots): GEMM1 5.4 -> 6.3 TB/s, GEMM2 (then in 512-row blocks) 4.9 -> 5.2 TB/s.
constexpr int kWeightAux = 2;
// Cache policy of device-coherent loads and stores (sc1).
constexpr int kCoherent = 16;
constexpr int kPairRows = kPairMaxT;  // rows of one slot on the pair-indexed path


// Stage the token tiles' 128-column scales in LDS: `rows` rows of 2 * S4
// bytes, zero beyond K/128 (padded steps) and beyond the tiles' rows.
template <typename Src>
__device__ __forceinline__ void stage_token_scales(uint8_t* s_xs, const uint8_t* xs, int nrow, int nb, int S4,
                                                   int rows, Src src) {
  // 16 threads per row: no division by the run-time pitch
  const int pitch = 2 * S4;
  for (int r = (int)(threadIdx.x >> 4); r < rows; r += (int)(blockDim.x >> 4)) {
    const bool ok = r < nrow;
    const uint8_t* row = xs + (ok ? (size_t)src(r) * nb : 0);
    for (int c = threadIdx.x & 15; c < pitch; c += 16) s_xs[r * pitch + c] = (ok && c < nb) ? row[c] : (uint8_t)0;
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

// Pair-indexed GEMM2: the slot's pair list as GEMM1 left it (counts[s]
// entries, at most kPairRows, at plist + s * stride), staged in LDS.
template <bool PAIRS>
__device__ __forceinline__ SlotRows<PAIRS> listed_rows(const int32_t* counts, const int32_t* plist, int stride, int s,
                                                       int* list) {
  SlotRows<PAIRS> R;
  R.div = 1;
  R.row0 = 0;
  R.list = list;
  R.n = min(counts[s], kPairRows);
  const int32_t* src = plist + (size_t)s * stride;
  for (int i = threadIdx.x; i < R.n; i += blockDim.x) list[i] = src[i];
  __syncthreads();
  return R;
}

// The token operand of NT 16-row tiles (rows tt0 .. tt0 + nrow - 1 of the
// slot): a buffer over the input rows and this lane's byte offsets.  Lanes
// past the rows read zeros (an offset past the buffer); their results are
// never stored.
template <bool PAIRS, int NT, bool UT>
__device__ __forceinline__ void token_operand(SOps<NT, UT>& O, const uint8_t* x, const SlotRows<PAIRS>& R, int tt0,
                                              int nrow, int nsrc, int K, int l16, int g) {
  const uint32_t lim = PAIRS ? (uint32_t)nsrc * (uint32_t)K : (uint32_t)nrow * (uint32_t)K;
  O.x = PAIRS ? make_rsrc(x, lim) : make_rsrc(x + (size_t)(R.row0 + tt0) * K, lim);
  O.kx = (uint32_t)K;
  O.lim = lim;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = n * 16 + l16;
    const uint32_t row = PAIRS ? (uint32_t)R.src(tt0 + (r < nrow ? r : 0)) : (uint32_t)r;
    O.xlo[n] = r < nrow ? row * (uint32_t)K + (uint32_t)g * 16 : lim;
  }
}

// ---------------------------------------------------------------------------
// a5: one block per (local slot s, 128-column block fb of F, K range ks).
// Wave w owns the gate tiles of columns fb*128 + 32w + [0, 32) and the
// matching up tiles, so SwiGLU pairs registers of the same lane; the requant
// amax over the 128 columns is reduced across the four waves in LDS.
//   bucketed (PAIRS false): xq/xs rows and aq/as rows from `offsets`;
//   pair-indexed (PAIRS true): xq/xs are per-token rows [nsrc = T], aq/as
//   per-pair rows [T*k]; the slot's pairs come from phys[0, np), and the
//   slot's first block leaves its count in counts[s] and (plist non-null)
//   its list at plist + s * stride for GEMM2.
// Split K (ks_n > 1, pair-indexed decode shares whose few touched slots would
// otherwise stream on a few CUs): block ks takes quads [ks nq / ks_n,
// (ks + 1) nq / ks_n) of the nq K quads and stores its f32 partial sums at
// part + (ks * np + pair) * 2F; the last of the ks_n blocks of (s, fb) to
// finish (a device-scope counter, cnt[s * nfb + fb], zero before the call and
// left zero) adds the partials in ascending ks and runs SwiGLU and the requant.
// The partials are stored and loaded device-coherent (sc1: past the XCD's
// L2), so ordering them around the counter takes only waits for completion,
// not the whole-L2 write-back and invalidation a device-scope fence costs.
// ---------------------------------------------------------------------------
// NT 16-row token tiles share each pass over the block's weights (a slot
// with more rows streams its weights once per 16 NT rows); NT = 2 needs more
// registers and runs two blocks per CU instead of three.
template <bool PAIRS, int NT, bool SM = false>
__global__ __launch_bounds__(256, NT == 1 && !SM ? 3 : 2) void k_gemm1_stream(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs_in, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ phys_in, int np, int k, int p0, int nsrc, const uint8_t* __restrict__ pw1,
    const uint8_t* __restrict__ pw1s, uint8_t* __restrict__ aq, uint8_t* __restrict__ as_,
    int32_t* __restrict__ counts, int32_t* __restrict__ plist, int stride, int H, int F, int ks_arg,
    float* __restrict__ part, int32_t* __restrict__ cnt, int nvs_arg, int P_local, int32_t* __restrict__ tlist) {
  constexpr int kRows = 16 * NT;  // token rows per pass
  // SM (pair-indexed decode shares): split K and touched-slot rows; the
  // other forms compile neither
  const int ks_n = SM ? ks_arg : 1;
  const int nvs = SM ? nvs_arg : P_local;
  const bool vmap = SM && nvs < P_local;  // block rows are the touched slots, not all slots
  __shared__ float s_amax[4][kRows];
  __shared__ __align__(16) uint8_t s_xs[kRows * 2 * kMaxSteps];
  __shared__ int s_list[PAIRS ? kPairRows : 1];
  __shared__ int s_cnt[2][4];
  __shared__ int s_last;
  __shared__ uint32_t s_bits[SM ? kTouchedWords : 1];
  const int nfb = F / kActBlock;
  // split K: consecutive blocks (ks fastest) on different XCDs, so that the
  // few touched slots spread over the chip; otherwise XCD-contiguous items
  const int item = ks_n > 1 ? (int)blockIdx.x : xcd_item(blockIdx.x, gridDim.x);
  const int jv = item / (nfb * ks_n), sub = item - jv * nfb * ks_n;
  const int fb = sub / ks_n, ks = sub - fb * ks_n;
  int ntouched = 0;
  if constexpr (SM) {
    if (vmap) {
      ntouched = touched_bits(phys_in, np, p0, P_local, s_bits);
      if (jv == 0 && fb == 0 && ks == 0)  // slots no block lists: count 0; the touched list for GEMM2
        for (int i = threadIdx.x; i < P_local; i += blockDim.x) {
          if ((s_bits[i >> 5] >> (i & 31)) & 1u) {
            if (tlist) tlist[1 + bit_rank(s_bits, i)] = i;
          } else {
            counts[i] = 0;
          }
          if (i == 0 && tlist) tlist[0] = ntouched;
        }
    }
  }
  // one slot: its pairs, then this block's columns and K range of them.  The
  // base pointers pass through opaque() so that the per-lane addresses built
  // from them stay inside the loop over slots instead of living across it.
  auto run_slot = [&](const int s) {
    __syncthreads();  // the previous slot's readers of s_list / s_amax are done
    const int32_t* phys = opaque(phys_in);
    const uint8_t* xs = opaque(xs_in);
    const SlotRows<PAIRS> R = slot_rows<PAIRS>(offsets, phys, np, p0 + s, s, k, s_list, s_cnt);
    const int n = R.n;
    if (PAIRS && fb == 0 && ks == 0) {
      if (threadIdx.x == 0) counts[s] = n;
      if (plist)
        for (int i = threadIdx.x; i < n; i += blockDim.x) plist[(size_t)s * stride + i] = s_list[i];
    }
    if (n <= 0) return;  // block-uniform: an idle expert reads no weights
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const PackGeom G = pack_geom(2u * F, (uint32_t)H);
    const int S4 = (int)G.steps;
    const int nq = S4 / 4, q0 = ks * nq / ks_n, q1 = (ks + 1) * nq / ks_n;
    const int nb = H / kActBlock;
    const int f0 = fb * kActBlock + wave * 32;
    SOps<NT> O;
    O.w = make_rsrc(pw1 + (size_t)s * G.data_slot, (uint32_t)G.data_slot);
    O.ws = make_rsrc(pw1s + (size_t)s * G.scale_slot, (uint32_t)G.scale_slot);
    const int tile[4] = {f0 / 16, f0 / 16 + 1, (F + f0) / 16, (F + f0) / 16 + 1};
  #pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      O.wt[rt] = (uint32_t)tile[rt] * (uint32_t)G.data_tile + 16u * lane;
      O.wst[rt] = (uint32_t)tile[rt] * (uint32_t)G.scale_tile + 8u * lane;
    }
    // partial sums of pair row `row`, tile rt: 4 consecutive f32 at columns
    // tile*16 + 4g, as a byte offset into Pr (ks_n np rows of 2F f32)
    const rsrc_t Pr = make_rsrc(part, SM && ks_n > 1 ? (uint32_t)ks_n * (uint32_t)np * (uint32_t)(8 * F) : 0u);
    auto part_at = [&](int kk, int row, int rt) -> uint32_t {
      return (((uint32_t)kk * (uint32_t)np + (uint32_t)row) * (uint32_t)(2 * F) + (uint32_t)(tile[rt] * 16 + 4 * g)) * 4u;
    };
    // SwiGLU, the requant amax over the block's 128 columns, fp8 codes and the scale
    auto epilogue = [&](const v4f (&acc)[4][NT], int tt0, int nrow) {
      // acc[0]/acc[2] are gate/up of columns f0 + 4g + r, acc[1]/acc[3] of f0 + 16 + 4g + r
      float act[NT][8];
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          act[t][r] = silu(acc[0][t][r]) * acc[2][t][r];
          act[t][4 + r] = silu(acc[1][t][r]) * acc[3][t][r];
        }
        float am = 0.0f;
  #pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(act[t][i]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        if (g == 0) s_amax[wave][t * 16 + l16] = am;
      }
      __syncthreads();
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int r = t * 16 + l16;
        const float am = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
        const int e = scale_exp(am);
        if (r < nrow) {
          const size_t d = (size_t)R.dst(tt0 + r);
          uint8_t* ap = aq + d * F + f0 + 4 * g;
          *reinterpret_cast<uint32_t*>(ap) =
              pack4_fp8(ldexpf(act[t][0], -e), ldexpf(act[t][1], -e), ldexpf(act[t][2], -e), ldexpf(act[t][3], -e));
          *reinterpret_cast<uint32_t*>(ap + 16) =
              pack4_fp8(ldexpf(act[t][4], -e), ldexpf(act[t][5], -e), ldexpf(act[t][6], -e), ldexpf(act[t][7], -e));
          if (wave == 0 && g == 0) as_[d * nfb + fb] = (uint8_t)(e + 127);
        }
      }
    };
    for (int tt0 = 0; tt0 < n; tt0 += kRows) {
      const int nrow = min(kRows, n - tt0);
      __syncthreads();  // previous pass's readers of s_xs / s_amax are done
      stage_token_scales(s_xs, xs, nrow, nb, S4, kRows, [&](int r) { return R.src(tt0 + r); });
      __syncthreads();
      token_operand<PAIRS, NT, false>(O, xq, R, tt0, nrow, nsrc, H, l16, g);
  #pragma unroll
      for (int t = 0; t < NT; ++t) O.sxs[t] = s_xs + (t * 16 + l16) * 2 * S4;
      v4f acc[4][NT];
  #pragma unroll
      for (int rt = 0; rt < 4; ++rt)
  #pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = v4f{0.f, 0.f, 0.f, 0.f};
      stream_tile<kWeightAux>(acc, O, 4 * (q1 - q0), 4 * q0);
      if (ks_n == 1) {
        epilogue(acc, tt0, nrow);
      } else {
  #pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int r = t * 16 + l16;
          if (r < nrow) {
            const int row = R.dst(tt0 + r);
  #pragma unroll
            for (int rt = 0; rt < 4; ++rt)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[rt][t]), Pr, part_at(ks, row, rt), 0,
                                                     kCoherent);
          }
        }
      }
    }
    if (ks_n == 1) return;
    // this block's partials are complete (coherent stores), then it counts
    // itself in; the last block of (s, fb) reads the others' and finishes
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      const int before = __hip_atomic_fetch_add(cnt + s * nfb + fb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = before == ks_n - 1;
      if (s_last) __hip_atomic_store(cnt + s * nfb + fb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    for (int tt0 = 0; tt0 < n; tt0 += kRows) {
      const int nrow = min(kRows, n - tt0);
      __syncthreads();  // previous pass's readers of s_amax are done
      v4f acc[4][NT];
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int r = t * 16 + l16;
        const int row = r < nrow ? R.dst(tt0 + r) : 0;
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          v4f v = v4f{0.f, 0.f, 0.f, 0.f};
          if (r < nrow)
            for (int kk = 0; kk < ks_n; ++kk)
              v += __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(Pr, part_at(kk, row, rt), 0, kCoherent));
          acc[rt][t] = v;
        }
      }
      epilogue(acc, tt0, nrow);
    }
  };
  // block row jv: slot jv, or (vmap) touched slots number jv, jv + nvs, ...
  for (int jj = jv;; jj += nvs) {
    int s = jj;
    if (vmap) {
      if (jj >= ntouched) break;
      s = nth_bit(s_bits, P_local, jj);
    }
    run_slot(s);
    if (!vmap) break;
  }
}

// ---------------------------------------------------------------------------
// a6: one block per (local slot s, block of 256 rows of H).  Wave w owns rows
// hb*256 + 64w + [0, 64) as one group of four 16-row tiles.  7168 / 256 * 48
// slots = 1344 blocks at three per CU: blocks of 512 rows (two groups per wave,
// one round over the chip) measured 5-8% slower at 512-1536 tokens.  y rows
// are f32 [rows, H] (bucketed rows, or pair rows with the act rows
// pair-indexed too; the slot's pairs then come from GEMM1's counts and lists,
// or with plist null from phys as in GEMM1).  Split K (pair-indexed only,
// ks_n > 1): block ks takes quads [ks nq / ks_n, (ks + 1) nq / ks_n) and
// writes its partial y at y + ks * ystride; the combine adds them.
// ---------------------------------------------------------------------------
constexpr int kG2Rows = 256;  // rows of H per block

template <bool PAIRS, int NT, bool SM = false>
__global__ __launch_bounds__(256, NT == 1 ? 3 : 2) void k_gemm2_stream(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as_, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ phys, int np, int p0, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ plist, int stride, int nsrc, const uint8_t* __restrict__ pw2,
    const uint8_t* __restrict__ pw2s, float* __restrict__ y, int H, int F, SingleRows sr, int ks_arg,
    size_t ystride, int nvs_arg, int P_local, const int32_t* __restrict__ tlist) {
  constexpr int kRows = 16 * NT;  // token rows per pass
  const int ks_n = SM ? ks_arg : 1;  // SM: as in GEMM1
  const bool vmap = SM && plist && tlist && nvs_arg < P_local;  // rows: GEMM1's touched slots
  const int nvs = vmap ? nvs_arg : P_local;
  __shared__ __align__(16) uint8_t s_xs[kRows * 2 * kMaxSteps];
  __shared__ int s_list[PAIRS ? kPairRows : 1];
  __shared__ int s_cnt[2][4];
  const int nhb = (H + kG2Rows - 1) / kG2Rows;
  const int item = ks_n > 1 ? (int)blockIdx.x : xcd_item(blockIdx.x, gridDim.x);  // as in GEMM1
  const int jv = item / (nhb * ks_n), sub = item - jv * nhb * ks_n;
  const int hb = sub / ks_n, ks = sub - hb * ks_n;
  y += (size_t)ks * ystride;
  // one slot: this block's rows of H and K range of it
  auto run_slot = [&](const int s) {
    __syncthreads();  // the previous slot's readers of s_list are done
    const SlotRows<PAIRS> R = (PAIRS && plist) ? listed_rows<PAIRS>(counts, plist, stride, s, s_list)
                                               : slot_rows<PAIRS>(offsets, phys, np, p0 + s, s, 1, s_list, s_cnt);
    const int n = R.n;
    if (n <= 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int h0 = hb * kG2Rows + wave * 64;
    const bool live = h0 < H;  // wave-uniform; H is a multiple of 128, so a live wave has 4 full tiles
    const PackGeom G = pack_geom((uint32_t)H, (uint32_t)F);
    const int S4 = (int)G.steps;
    const int nq = S4 / 4, q0 = ks * nq / ks_n, q1 = (ks + 1) * nq / ks_n;
    const int nb = F / kActBlock;
    SOps<NT, true> O;
    O.w = make_rsrc(pw2 + (size_t)s * G.data_slot, (uint32_t)G.data_slot);
    O.ws = make_rsrc(pw2s + (size_t)s * G.scale_slot, (uint32_t)G.scale_slot);
    O.wl = 16u * lane;
    O.sl = 8u * lane;
  #pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t tile = live ? (uint32_t)(h0 / 16 + rt) : 0u;
      O.wt[rt] = tile * (uint32_t)G.data_tile;
      O.wst[rt] = tile * (uint32_t)G.scale_tile;
    }
    const uint32_t gd = 4u * (uint32_t)G.data_tile, sgd = 4u * (uint32_t)G.scale_tile;
    for (int tt0 = 0; tt0 < n; tt0 += kRows) {
      const int nrow = min(kRows, n - tt0);
      __syncthreads();
      stage_token_scales(s_xs, as_, nrow, nb, S4, kRows, [&](int r) { return R.src(tt0 + r); });
      __syncthreads();
      if (!live) continue;
      token_operand<PAIRS, NT, true>(O, aq, R, tt0, nrow, nsrc, F, l16, g);
      // y through a buffer: pair rows index all of y (T k H 4 bytes < 2^31 for
      // T <= 1024), bucketed rows the pass's own rows; lanes past the rows
      // store beyond the buffer, which drops them
      const uint32_t ylim = (PAIRS ? (uint32_t)nsrc : (uint32_t)nrow) * (uint32_t)H * 4u;
      const rsrc_t Yr = PAIRS ? make_rsrc(y, ylim) : make_rsrc(y + (size_t)(R.row0 + tt0) * H, ylim);
      // bucketed rows of tokens with exactly one local pair: the output row
      // bf16(fma(w, y, 0)) instead of y (sr.rtok null: none)
      // (one offset per lane: into y, or into out when ow >= 0, the routing
      // weight of a single-pair row; routing weights are never negative)
      const rsrc_t Or = make_rsrc(sr.out, sr.rtok ? sr.out_bytes : 0u);
      uint32_t off[NT];
      float ow[NT];
  #pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int r = t * 16 + l16;
        O.sxs[t] = s_xs + r * 2 * S4;
        const uint32_t row = PAIRS ? (uint32_t)R.dst(tt0 + (r < nrow ? r : 0)) : (uint32_t)r;
        int tok = -1;
        if constexpr (!PAIRS) {
          if (sr.rtok != nullptr && r < nrow) tok = sr.rtok[R.row0 + tt0 + r];
        }
        ow[t] = tok >= 0 ? sr.rw[R.row0 + tt0 + r] : -1.0f;
        off[t] = tok >= 0 ? ((uint32_t)tok * (uint32_t)H + (uint32_t)(h0 + 4 * g)) * 2u
                          : (r < nrow ? (row * (uint32_t)H + (uint32_t)(h0 + 4 * g)) * 4u : ylim);
      }
      v4f acc[4][NT];
  #pragma unroll
      for (int rt = 0; rt < 4; ++rt)
  #pragma unroll
        for (int t = 0; t < NT; ++t) acc[rt][t] = v4f{0.f, 0.f, 0.f, 0.f};
      stream_groups<kWeightAux, 1>(acc, O, 4 * (q1 - q0), gd, sgd, 4 * q0, [&](int grp, const v4f(&a)[4][NT]) {
  #pragma unroll
        for (int t = 0; t < NT; ++t)
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            // column offsets go into the lane offset, soffset stays 0: the
            // compiler guards the store data of a 16-byte buffer store against
            // the next VALU write only when soffset is not a register, and
            // gfx950 needs that guard (a register soffset here let the next
            // instruction's write reach the stored data)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, a[rt][t]), Yr,
                                                   (ow[t] < 0.0f ? off[t] : ylim) + (uint32_t)(64 * grp + 16 * rt) * 4u,
                                                   0, 0);
            if constexpr (!PAIRS) {
              const v4f& v = a[rt][t];
              const v2i o = {(int)((uint32_t)f32_to_bf16(fmaf(ow[t], v[0], 0.0f)) |
                                   ((uint32_t)f32_to_bf16(fmaf(ow[t], v[1], 0.0f)) << 16)),
                             (int)((uint32_t)f32_to_bf16(fmaf(ow[t], v[2], 0.0f)) |
                                   ((uint32_t)f32_to_bf16(fmaf(ow[t], v[3], 0.0f)) << 16))};
              __builtin_amdgcn_raw_buffer_store_b64(
                  o, Or, (ow[t] >= 0.0f ? off[t] : sr.out_bytes) + (uint32_t)(64 * grp + 16 * rt) * 2u, 0, 0);
            }
          }
      });
    }
  };
  const int ntouched = vmap ? tlist[0] : 0;
  for (int jj = jv;; jj += nvs) {
    if (vmap && jj >= ntouched) break;
    run_slot(vmap ? tlist[1 + jj] : jj);
    if (!vmap) break;
  }
}

hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                               const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local, int nt,
                               hipStream_t st) {
  const unsigned grid = (unsigned)(P_local * (F / kActBlock));
  if (nt >= 2)
    k_gemm1_stream<false, 2><<<grid, 256, 0, st>>>(xq, xs, offsets, nullptr, 0, 1, 0, 0, pw1, pw1s, aq, as, nullptr,
                                                    nullptr, 0, H, F, 1, nullptr, nullptr, P_local, P_local, nullptr);
  else
    k_gemm1_stream<false, 1><<<grid, 256, 0, st>>>(xq, xs, offsets, nullptr, 0, 1, 0, 0, pw1, pw1s, aq, as, nullptr,
                                                    nullptr, 0, H, F, 1, nullptr, nullptr, P_local, P_local, nullptr);
  return hipGetLastError();
}

// returns the K split it ran with (1 unless the decode-share form ran)
template <bool PAIRS>
static int gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const int32_t* phys, int np,
                         int p0, const int32_t* counts, const int32_t* plist, int stride, int nsrc, const uint8_t* pw2,
                         const uint8_t* pw2s, float* y, int H, int F, int P_local, int nt, SingleRows sr, int ks_n,
                         int nvs, const int32_t* tlist, hipStream_t st) {
  // the decode-share form (split K, touched rows) only with one token tile
  const bool sm = PAIRS && nt < 2 && (ks_n > 1 || (plist && tlist && nvs < P_local));
  if (!sm) ks_n = 1;
  const int rows = (sm && plist && tlist && nvs < P_local) ? nvs : P_local;
  const unsigned grid = (unsigned)(rows * ((H + kG2Rows - 1) / kG2Rows) * ks_n);
  const size_t ystride = (size_t)nsrc * (size_t)H;
  if (sm)
    k_gemm2_stream<PAIRS, 1, PAIRS><<<grid, 256, 0, st>>>(aq, as, offsets, phys, np, p0, counts, plist, stride, nsrc,
                                                           pw2, pw2s, y, H, F, sr, ks_n, ystride, rows, P_local, tlist);
  else if (nt >= 2)
    k_gemm2_stream<PAIRS, 2><<<grid, 256, 0, st>>>(aq, as, offsets, phys, np, p0, counts, plist, stride, nsrc, pw2,
                                                    pw2s, y, H, F, sr, 1, ystride, rows, P_local, tlist);
  else
    k_gemm2_stream<PAIRS, 1><<<grid, 256, 0, st>>>(aq, as, offsets, phys, np, p0, counts, plist, stride, nsrc, pw2,
                                                    pw2s, y, H, F, sr, 1, ystride, rows, P_local, tlist);
  return ks_n;
}

hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                               const uint8_t* pw2s, float* y, int H, int F, int P_local, int nt, SingleRows sr,
                               hipStream_t st) {
  gemm2_stream<false>(aq, as, offsets, nullptr, 0, 0, nullptr, nullptr, 0, 0, pw2, pw2s, y, H, F, P_local, nt, sr, 1,
                      P_local, nullptr, st);
  return hipGetLastError();
}

hipError_t launch_gemm1_pairs(const uint8_t* xq_tok, const uint8_t* xs_tok, const int32_t* phys, int T, int k, int p0,
                              const uint8_t* pw1, const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int32_t* counts,
                              int32_t* plist, int stride, int H, int F, int P_local, int nt, int ks_n, float* part,
                              int32_t* cnt, int nvs, int32_t* tlist, hipStream_t st) {
  // the decode-share form (split K, touched rows) only with one token tile
  const bool sm = nt < 2 && (ks_n > 1 || nvs < P_local);
  const int rows = sm && nvs < P_local ? nvs : P_local;
  const unsigned grid = (unsigned)(rows * (F / kActBlock) * (sm ? ks_n : 1));
  if (sm)
    k_gemm1_stream<true, 1, true><<<grid, 256, 0, st>>>(xq_tok, xs_tok, nullptr, phys, T * k, k, p0, T, pw1, pw1s, aq,
                                                         as, counts, plist, stride, H, F, ks_n, part, cnt, rows, P_local,
                                                         tlist);
  else if (nt >= 2)
    k_gemm1_stream<true, 2><<<grid, 256, 0, st>>>(xq_tok, xs_tok, nullptr, phys, T * k, k, p0, T, pw1, pw1s, aq, as,
                                                   counts, plist, stride, H, F, 1, part, cnt, rows, P_local, tlist);
  else
    k_gemm1_stream<true, 1><<<grid, 256, 0, st>>>(xq_tok, xs_tok, nullptr, phys, T * k, k, p0, T, pw1, pw1s, aq, as,
                                                   counts, plist, stride, H, F, 1, part, cnt, rows, P_local, tlist);
  return hipGetLastError();
}

hipError_t launch_gemm2_pairs(const uint8_t* aq, const uint8_t* as, const int32_t* phys, int T, int k, int p0,
                              const int32_t* counts, const int32_t* plist, int stride, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, int nt, int ks_n, int nvs,
                              const int32_t* tlist, hipStream_t st) {
  gemm2_stream<true>(aq, as, nullptr, phys, T * k, p0, counts, plist, stride, T * k, pw2, pw2s, y, H, F, P_local, nt,
                     SingleRows{nullptr, nullptr, nullptr, 0u}, ks_n, nvs, tlist, st);  // nt < 2 whenever ks_n > 1
  return hipGetLastError();
}

}  // namespace moe
