// Large-M path: persistent grouped GEMMs for many rows per expert (block-
// scaled fp8 x MXFP4 MFMA on gfx950).  Same arithmetic as the streaming
// kernels (a5 GEMM1 + SwiGLU + fp8 requant, a6 GEMM2 into f32 rows), tiled
// for MFMA throughput: the pages' persistent large-input path serves extend
// steps of at least 1024 tokens per rank [sglang PR 47065 "Use the aiter
// MegaMoE small- and large-input paths", Modifications].
//
// Both kernels are persistent: one block per CU walks the work items of its
// XCD's contiguous range (block b runs on XCD b % 8), token block fastest, so
// the items that run at the same time on one XCD share their weight block in
// that XCD's L2.  K advances 128 per stage (one V_MFMA_SCALE_F32_16X16X128_
// F8F6F4 per tile pair); two waves share each SIMD, so that one wave's LDS
// and barrier waits are filled by the other's MFMAs.
//  - Token rows and weight tiles: direct-to-LDS DMA (buffer_load_dwordx4 ...
//    lds) into a ring of stages issued ahead of use; each token row of 128
//    bytes is stored with its eight 16-byte pieces permuted so that the
//    B-operand reads of a 16-token tile hit distinct banks; a weight tile
//    (the packed layout is the MFMA operand order) is read back with one
//    ds_read_b128 per lane.
//  - Stage barriers are bare s_barrier with explicit vmcnt waits: the
//    generic workgroup barrier would drain every load in flight.
//  - k_gemm2_tiled (a6): items of 128 tokens x 256 rows of H; wave (wq, th)
//    owns rows 64 wq .. + 63 against the token tiles of half th; a ring of
//    four stages, three in flight; weight scales by DMA too; y tiles of an
//    item written during the next item's stages.
//  - k_gemm1_w (a5): items of 128 tokens x 512 weight rows (the gate and up
//    rows of 256 columns of F); wave w owns 32 columns against all eight
//    token tiles; a ring of three stages, two in flight; weight scales in
//    registers; SwiGLU + fp8 requant epilogue.

#include <type_traits>

#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_layout.hpp"

namespace moe {

constexpr int kTM = 128;           // token rows per block tile
constexpr int kTN = 256;           // weight rows per block tile (4 waves x 4 tiles)
constexpr int kRing = 4;           // token stages resident in LDS
constexpr int kAhead = kRing - 1;  // token stages in flight ahead of use
constexpr int kStage = kTM * 128;  // bytes of one token stage
constexpr int kWStage = 16 * 1024; // bytes of one weight stage (16 tiles x 64 lanes x 16 B)
constexpr int kSGroup = 16 * 512;  // bytes of one scale group (16 tiles, 8 stages)
constexpr int kMaxStages = 64;     // K <= 8192
constexpr int kNW = 8;             // waves per block: two per SIMD (measured 7% faster than one)
constexpr int kWPS = kNW / 4;      // waves per SIMD = token groups of the block tile
constexpr int kTT = 8 / kWPS;      // 16-token tiles per wave
constexpr int kXI = 16 / kNW;      // token DMA instructions per wave per stage (1 KB each)
constexpr int kWI = 4 / kWPS;      // weight DMA instructions per wave per stage
constexpr int kSI = 2 / kWPS;      // scale DMA instructions per wave per scale group

// vmcnt accounting.  A stage's DMA is waited for at the start of the stage
// three later; after it the wave has issued two more stages of DMA (kXI +
// kWI each) and one y store per stage: three.  Scale-group DMA and
// token-scale loads only add to the count, which keeps the wait sufficient.
// (Scale groups are issued at least three stages before their first use,
// with three stages of DMA after them by then.)
constexpr int kVmWait = 2 * (kXI + kWI) + 3;

// Physical 16-byte piece of logical piece p in the stage row of the token at
// position r (mod 16) of its tile: p ^ swz(r).  Measured on gfx950 for the
// B-operand reads (16 rows x one piece per ds_read_b128 quarter): r & 7 reads
// at 1.6x the rate of an XOR that also folds in bit 3, and 3x unswizzled rows.
__device__ __forceinline__ int swz(int r) { return r & 7; }

__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) const uint8_t* lds_u8_t;

// LDS reads of the hot loop, issued as instructions the compiler does not
// track: it would otherwise treat every read of an LDS object that a DMA
// targets as dependent on all DMA in flight and drain the DMA queue.  Their
// results are waited for explicitly (lgkm_wait) before use.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_u8_t)(const uint8_t*)p;
}
__device__ __forceinline__ v4i lds_read16(const void* p) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr(p)));
  return v;
}
// ds_read_b128 at LDS address `a` + OFS (an immediate, < 65536)
template <int OFS>
__device__ __forceinline__ v4i lds_read16_at(uint32_t a) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFS));
  return v;
}
__device__ __forceinline__ v2i lds_read8(const void* p) {
  v2i v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(lds_addr(p)));
  return v;
}
#define MOE_LGKM_WAIT(n) asm volatile("s_waitcnt lgkmcnt(" #n ")" ::: "memory")
// Arguments of __builtin_amdgcn_raw_ptr_buffer_load_lds: (buffer, LDS base,
// bytes per lane, voffset, soffset, immediate offset, cache policy).
#ifndef MOE_TILED_WAUX
#define MOE_TILED_WAUX 0
#endif
constexpr int kWeightNt = MOE_TILED_WAUX;  // weights: default policy (each weight stage is read by every token block)

union V8T {
  v8i v;
  v4i h[2];
};

// One work item: wave-uniform scalars only (per-lane DMA offsets are lane
// constants plus uniform parts).
struct TItem {
  int live;      // an item (0: every DMA of it reads zeros)
  int wlive;     // the wave's weight tiles exist (GEMM2's partial last block)
  int s, wb, r0, nvalid;
  int tl[2];     // the wave's weight tiles: tl[0], tl[0] + 1, tl[1], tl[1] + 1
};

// GEMM2 (a6): y rows [bucket rows, H] f32 from the requantised act rows.
__global__ __launch_bounds__(kNW * 64, 1) void k_gemm2_tiled(const uint8_t* __restrict__ xq,
                                                             const uint8_t* __restrict__ xs,
                                                             const int32_t* __restrict__ offsets, int P_local,
                                                             const uint8_t* __restrict__ pw,
                                                             const uint8_t* __restrict__ pws, float* __restrict__ y,
                                                             int H, int F) {
  // DMA rings: one LDS object per ring slot, so that the compiler's LDS-DMA
  // tracking sees that the slot a stage reads is not the one just refilled
  // slot: kTM token rows x 128 B (swizzled), then 16 weight tiles x 1 KB
  __shared__ __align__(16) uint8_t r0s[kStage + kWStage], r1s[kStage + kWStage], r2s[kStage + kWStage],
      r3s[kStage + kWStage];
  __shared__ __align__(16) uint8_t sring[2 * kSGroup];      // [2 groups][16 tiles x 512 B]
  __shared__ __align__(16) uint8_t s_xs[kTM * kMaxStages];  // [stage][16][8] token scales
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t* const xring[kRing] = {r0s, r1s, r2s, r3s};
  uint8_t* const wring[kRing] = {r0s + kStage, r1s + kStage, r2s + kStage, r3s + kStage};
  const int K = F, R = H;
  const int nwb = (H + kTN - 1) / kTN;
  const int nst = K / 128;               // stages with data (K is a multiple of 128)
  const int nst4 = (nst + 3) & ~3;       // stages run per item: whole ring turns
  const PackGeom Gm = pack_geom((uint32_t)R, (uint32_t)K);
  const int ngrp = (int)Gm.steps / 4;    // scale groups (8 stages each); 8 ngrp >= nst4
  int* s_pre = reinterpret_cast<int*>(lds);  // [P_local + 1] items before slot
  int* s_off = s_pre + P_local + 1;           // [P_local + 1] bucket offsets
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 3, th = kWPS == 1 ? 0 : wave >> 2;  // weight quarter (SIMD), token group
  const int l16 = lane & 15, g = lane >> 4;
  const int sw = swz(l16);

  for (int p = tid; p <= P_local; p += blockDim.x) s_off[p] = offsets[p];
  __syncthreads();
  for (int p = tid; p < P_local; p += blockDim.x) s_pre[p + 1] = (s_off[p + 1] - s_off[p] + kTM - 1) / kTM * nwb;
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int p = 1; p <= P_local; ++p) {
      run += s_pre[p];
      s_pre[p] = run;
    }
  }
  __syncthreads();
  const int nitems = s_pre[P_local];
  // a contiguous item range per XCD (block b runs on XCD b % 8)
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int chunk = (nitems + 7) / 8;
  const int i0 = xcd * chunk, i1 = min(nitems, i0 + chunk);
  if (i0 + lb >= i1) return;  // block-uniform: no item for this block

  // lane constants of the DMA offsets
  uint32_t xt[kXI], xp[kXI];  // token DMA instruction wave + kNW m: token row and byte offset of the lane's piece
#pragma unroll
  for (int m = 0; m < kXI; ++m) {
    const int t = 8 * (wave + kNW * m) + (lane >> 3);
    xt[m] = (uint32_t)t;
    xp[m] = 16u * (uint32_t)((lane & 7) ^ swz(t & 15));
  }
  const uint32_t wlane = 16u * lane;                                            // weight tile: lane's 16 bytes
  const uint32_t slane = (uint32_t)(lane >> 5) * (uint32_t)Gm.scale_tile + 16u * (lane & 31);  // scales of tiles 2h + lane / 32
  const uint32_t wlim = (uint32_t)Gm.data_slot, slim = (uint32_t)Gm.scale_slot;  // past a slot: zeros

  auto decode = [&](int item) {
    TItem it;
    it.live = item < i1;
    int s = 0, wb = 0, tb = 0, n = 0;
    if (it.live) {
      int lo = 0, hi = P_local - 1;  // slot: last s with s_pre[s] <= item
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= item) lo = mid;
        else hi = mid - 1;
      }
      s = lo;
      n = s_off[s + 1] - s_off[s];
      const int ntb = (n + kTM - 1) / kTM;
      const int local = item - s_pre[s];
      wb = local / ntb;
      tb = local - wb * ntb;
    }
    // wave-uniform by construction; readfirstlane tells the compiler
    it.s = __builtin_amdgcn_readfirstlane(s);
    it.wb = __builtin_amdgcn_readfirstlane(wb);
    it.r0 = __builtin_amdgcn_readfirstlane(s_off[s] + tb * kTM);
    it.nvalid = __builtin_amdgcn_readfirstlane(it.live ? min(kTM, n - tb * kTM) : 0);
    it.live = __builtin_amdgcn_readfirstlane(it.live);
    it.wlive = it.live && wb * kTN + wq * 64 < H;  // H is a multiple of 128
    const int h0 = it.wb * kTN + wq * 64;         // rows h0 .. h0 + 63
    it.tl[0] = h0 / 16;
    it.tl[1] = h0 / 16 + 2;
    return it;
  };

  // DMA issue.  Every stage moves the same number of instructions (past the
  // data: offsets beyond the buffer, which read zeros and move nothing).
  auto dma_x = [&](const TItem it, uint8_t* slot, int q) {  // token stage q
    const bool live = it.live && q < nst;
    const uint32_t xlim = (uint32_t)it.nvalid * (uint32_t)K;
    const rsrc_t Xr = make_rsrc(xq + (size_t)it.r0 * K, xlim);
#pragma unroll
    for (int m = 0; m < kXI; ++m) {
      const uint32_t vo = (live && xt[m] < (uint32_t)it.nvalid) ? xt[m] * (uint32_t)K + xp[m] : xlim;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (lds_ptr_t)(slot + (wave + kNW * m) * 1024), 16, vo,
                                               live ? (uint32_t)q * 128u : 0u, 0, 0);
    }
  };
  auto dma_w = [&](const TItem it, uint8_t* slot, int q) {  // this wave's share of its quarter's tiles of stage q
    const bool live = it.wlive && q < nst;
    const rsrc_t Wr = make_rsrc(pw + (size_t)it.s * Gm.data_slot, wlim);
    const uint32_t so = (uint32_t)(q >> 1) * 2048u + (uint32_t)(q & 1) * 1024u;
#pragma unroll
    for (int i = 0; i < kWI; ++i) {
      const int rt = th * kWI + i;  // tl[] picked by selects: a runtime index would put the item in scratch
      const uint32_t tile = (uint32_t)(((rt >> 1) ? it.tl[1] : it.tl[0]) + (rt & 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Wr, (lds_ptr_t)(slot + wq * 4096 + rt * 1024), 16,
                                               live ? wlane : wlim, live ? tile * (uint32_t)Gm.data_tile + so : 0u, 0,
                                               kWeightNt);
    }
  };
  auto dma_s = [&](const TItem it, int grp, int par) {  // this wave's share of its quarter's scales of group grp
    const bool live = it.wlive && grp < ngrp;
    const rsrc_t Sr = make_rsrc(pws + (size_t)it.s * Gm.scale_slot, slim);
    uint8_t* slot = sring + par * kSGroup + wq * 2048;
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
      const int h = th * kSI + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Sr, (lds_ptr_t)(slot + h * 1024), 16, live ? slane : slim,
                                               live ? (uint32_t)(h ? it.tl[1] : it.tl[0]) * (uint32_t)Gm.scale_tile + (uint32_t)grp * 512u : 0u,
                                               0, 0);
    }
  };
  // The item's token scales, stage-major: byte tt of lane record [q][r] is
  // the scale of token 16 tt + r at stage q (one 8-byte read gives a lane all
  // eight); stages past the data hold 0.  kTPR threads per token row.  Rows of
  // a multiple of 4 bytes are fetched as dwords into registers well ahead of
  // use (relaxed atomic loads: issued where written, not sunk to the use);
  // other widths are read byte by byte when stored.
  constexpr int kTPR = kNW * 64 / kTM;             // threads per token row
  constexpr int kXsPer = kMaxStages / 4 / kTPR;    // dwords per thread
  const bool xs_dw = (nst & 3) == 0;
  auto xs_fetch = [&](const TItem it, uint32_t (&v)[kXsPer]) {
    const int t = tid / kTPR;
    const bool ok = xs_dw && it.live && t < it.nvalid;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(xs + (size_t)(it.r0 + t) * nst);
#pragma unroll
    for (int j = 0; j < kXsPer; ++j) {
      const int d = (tid % kTPR) + kTPR * j;  // dword of the row
      v[j] = (ok && 4 * d < nst) ? __hip_atomic_load(src + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    }
  };
  auto xs_store = [&](const TItem it, const uint32_t (&v)[kXsPer]) {
    const int t = tid / kTPR;
    uint8_t* dst = s_xs + (t & 15) * 8 + (t >> 4);
    if (xs_dw) {
#pragma unroll
      for (int j = 0; j < kXsPer; ++j) {
        const int d = (tid % kTPR) + kTPR * j;
        if (4 * d < nst4) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) dst[(4 * d + bb) * kTM] = (uint8_t)(v[j] >> (8 * bb));
        }
      }
    } else {
      const bool ok = it.live && t < it.nvalid;
      const uint8_t* src = xs + (size_t)(it.r0 + t) * nst;
      for (int c = tid % kTPR; c < nst4; c += kTPR) dst[c * kTM] = (ok && c < nst) ? src[c] : (uint8_t)0;
    }
  };

  const int o_lo = (g ^ sw) * 16, o_hi = ((g + 4) ^ sw) * 16;
  v2i sc[4];  // weight scales of the current group: byte q % 8 scales stage q
  v4f acc[4][kTT];
  constexpr int kTile = 16 * 128;  // bytes of one 16-token tile of a stage

  // B operand (token tile tt of this wave's group) from the stage's rows
  auto ldb = [&](V8T& b, uint32_t blo, uint32_t bhi, auto ttc) {
    constexpr int o = decltype(ttc)::value * kTile;
    b.h[0] = lds_read16_at<o>(blo);
    b.h[1] = lds_read16_at<o>(bhi);
  };

  // this wave's kTT token tiles of stage q (tiles past the block's rows hold zeros)
  auto compute = [&](bool wlive, const uint8_t* xs_slot, const uint8_t* w_slot, int q) {
    if (!wlive) return;
    // LDS reads in issue order (they complete in order): weights (4), token
    // scales (1), token tiles 0 and 1 (2 + 2), then tile tt + 2's two reads
    // before tile tt's MFMAs.  Tile tt's operands are complete once at most
    // the reads of the two later tiles are outstanding.  Addresses are one
    // register each plus immediate offsets.
    const uint32_t aa = lds_addr(w_slot + wq * 4096 + lane * 16);
    const uint8_t* xg = xs_slot + th * kTT * kTile + l16 * 128;
    const uint32_t blo = lds_addr(xg + o_lo), bhi = lds_addr(xg + o_hi);
    v4i a[4];
    a[0] = lds_read16_at<0>(aa);
    a[1] = lds_read16_at<1024>(aa);
    a[2] = lds_read16_at<2048>(aa);
    a[3] = lds_read16_at<3072>(aa);
    const v2i sbw = lds_read8(s_xs + q * kTM + l16 * 8);
    V8T b[3];
    ldb(b[0], blo, bhi, std::integral_constant<int, 0>{});
    ldb(b[1], blo, bhi, std::integral_constant<int, 1>{});
    int sa[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) sa[rt] = (int)((uint32_t)((q & 4) ? sc[rt].y : sc[rt].x) >> (8 * (q & 3)));
    MOE_LGKM_WAIT(4);  // weights and token scales are in
    __builtin_amdgcn_sched_barrier(0);
    int sb[kTT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
      const int t8 = th * kTT + tt;  // byte of the 8-tile record
      sb[tt] = (int)(((uint32_t)(t8 < 4 ? sbw.x : sbw.y) >> (8 * (t8 & 3))) & 0xFFu);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt + 2 < kTT) ldb(b[(tt + 2) % 3], blo, bhi, std::integral_constant<int, tt + 2>{});
      if constexpr (tt + 2 < kTT) MOE_LGKM_WAIT(4);
      else if constexpr (tt + 1 < kTT) MOE_LGKM_WAIT(2);
      else MOE_LGKM_WAIT(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][tt] = mfma_fp4_fp8<0>(a[rt], b[tt % 3].v, acc[rt][tt], sa[rt], sb[tt]);
      __builtin_amdgcn_sched_barrier(0);
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    tile(std::integral_constant<int, 2>{});
    tile(std::integral_constant<int, 3>{});
    if constexpr (kTT == 8) {
      tile(std::integral_constant<int, kTT == 8 ? 4 : 0>{});
      tile(std::integral_constant<int, kTT == 8 ? 5 : 0>{});
      tile(std::integral_constant<int, kTT == 8 ? 6 : 0>{});
      tile(std::integral_constant<int, kTT == 8 ? 7 : 0>{});
    }
  };

  // GEMM2 writes an item's y tiles during the next item's stages, one
  // 16x16 tile per stage and wave, instead of all at the item's end: the
  // items of all CUs end together, and their y rows written at once stall
  // every CU on the write burst (measured: 9.1k -> 3.4k clocks per item
  // with the burst removed).  yst holds the previous item's results not yet
  // stored, the next token tile first (a shift after every fourth store
  // keeps every register index a constant); a store past the previous item
  // (or with none) lands out of range and is dropped.
  v4f yst[4][kTT];
  rsrc_t Yp = make_rsrc(y, 0u);  // the previous item's rows
  uint32_t yp_lane = 0;          // this lane's byte offset within them (tile 0, rt 0)
  auto ystore = [&](auto rtc, int q) {  // tile (rt, q / 4) of the previous item; q % 4 == rt
    constexpr int rt = decltype(rtc)::value;
    const int tt = q >> 2;
    const uint32_t off = tt < kTT ? yp_lane + (uint32_t)tt * 16u * (uint32_t)H * 4u + 64u * rt : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, yst[rt][0]), Yp, off, 0, 0);
    if constexpr (rt == 3) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j + 1 < kTT; ++j) yst[r][j] = yst[r][j + 1];
    }
  };
  auto ystore_rt = [&](int q) {  // runtime rt = q % 4
    switch (q & 3) {
      case 0: ystore(std::integral_constant<int, 0>{}, q); break;
      case 1: ystore(std::integral_constant<int, 1>{}, q); break;
      case 2: ystore(std::integral_constant<int, 2>{}, q); break;
      default: ystore(std::integral_constant<int, 3>{}, q); break;
    }
  };

  // ---- first item: its token scales, first scale group and first stages
  TItem cur = decode(i0 + lb);
  int gpar = 0;  // scale slot of the current item's group 0
  {
    uint32_t v[kXsPer];
    xs_fetch(cur, v);
    xs_store(cur, v);
  }
  __syncthreads();
  dma_s(cur, 0, 0);
#pragma unroll
  for (int q = 0; q < kAhead; ++q) {
    dma_x(cur, xring[q], q);
    dma_w(cur, wring[q], q);
    ystore(std::integral_constant<int, 0>{}, 4 * kTT);  // nothing yet: the per-stage count
  }

  for (int item = i0 + lb; item < i1; item += nper) {
    // the next item: decoded now; its first stages and first scale group are
    // moved in during this item's last stages, its token scales fetched into
    // registers at the start of the last four (stored at the item boundary)
    const TItem nxt = decode(item + nper);

#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) acc[rt][tt] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage (ring slot u = q % kRing, a compile-time constant): wait for
    // its rows and weights (own DMA, then everyone's via the barrier, which
    // also retires the slot the next DMA refills), issue stage q + 3 (of
    // this item or, past its end, of the next), compute stage q
    auto stage = [&](auto uc, int q) {
      constexpr int u = decltype(uc)::value;
      asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kVmWait) : "memory");
      bare_barrier();
      if ((q & 7) == 0 && cur.wlive) {  // a new scale group (its DMA was issued at least three stages ago)
        const uint8_t* sp = sring + ((gpar + (q >> 3)) & 1) * kSGroup + wq * 2048 + lane * 8;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) sc[rt] = lds_read8(sp + (rt >> 1) * 1024 + (rt & 1) * 512);
        MOE_LGKM_WAIT(0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((q & 7) == 4 && (q >> 3) + 1 < ngrp) dma_s(cur, (q >> 3) + 1, (gpar + (q >> 3) + 1) & 1);
      if (q == nst4 - 3) dma_s(nxt, 0, (gpar + ngrp) & 1);
      if (q + kAhead < nst4) {
        dma_x(cur, xring[(u + kAhead) % kRing], q + kAhead);
        dma_w(cur, wring[(u + kAhead) % kRing], q + kAhead);
      } else {
        dma_x(nxt, xring[(u + kAhead) % kRing], q + kAhead - nst4);
        dma_w(nxt, wring[(u + kAhead) % kRing], q + kAhead - nst4);
      }
      ystore(std::integral_constant<int, u>{}, q);  // q % 4 == u: stage loops start at multiples of 4
      compute(cur.wlive, xring[u], wring[u], q);
    };
    for (int q0 = 0; q0 < nst4 - 4; q0 += 4) {
      stage(std::integral_constant<int, 0>{}, q0);
      stage(std::integral_constant<int, 1>{}, q0 + 1);
      stage(std::integral_constant<int, 2>{}, q0 + 2);
      stage(std::integral_constant<int, 3>{}, q0 + 3);
    }
    // the last four stages, outside the loop: the compiler then counts the
    // loads issued after the token-scale fetch exactly and waits for that
    // fetch alone at the boundary
    uint32_t xsn[kXsPer];
    xs_fetch(nxt, xsn);
    stage(std::integral_constant<int, 0>{}, nst4 - 4);
    stage(std::integral_constant<int, 1>{}, nst4 - 3);
    stage(std::integral_constant<int, 2>{}, nst4 - 2);
    stage(std::integral_constant<int, 3>{}, nst4 - 1);

    // ---- epilogue: the previous item's tiles not stored by this item's
    // stages (fewer than 4 kTT stages), then this item's results take their
    // place
    for (int q = nst4; q < 4 * kTT; ++q) ystore_rt(q);
    const int h0 = cur.wb * kTN + wq * 64;
    // waves without weight tiles (a partial last block of H) store nothing: zero-sized buffer
    Yp = make_rsrc(y + (size_t)cur.r0 * H, cur.wlive ? (uint32_t)cur.nvalid * (uint32_t)H * 4u : 0u);
    yp_lane = ((uint32_t)(th * kTT * 16 + l16) * (uint32_t)H + (uint32_t)(cur.wlive ? h0 + 4 * g : 0)) * 4u;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) yst[rt][tt] = acc[rt][tt];
    // item boundary: every wave is done with this item's token scales; the
    // next item's go in (visible after the next stage barrier)
    bare_barrier();
    xs_store(nxt, xsn);
    MOE_LGKM_WAIT(0);
    cur = nxt;
    gpar = (gpar + ngrp) & 1;
  }
  for (int q = 0; q < 4 * kTT; ++q) ystore_rt(q);  // the last item's results
}

// ---------------------------------------------------------------------------
// GEMM1 (a5) on 128-token x 512-row tiles.  Eight waves, two per SIMD; wave
// w owns the gate and up tiles of 32 columns of F (four 16-row weight tiles)
// against all eight 16-token tiles: 32 accumulators (128 registers).  A
// stage of 128 K is 32 MFMAs per wave over 48 KB of DMA per block (16 KB
// tokens + 32 KB weights): twice the MFMA work per stage barrier and per
// byte moved of the 128 x 256 tile, and fewer LDS reads per MFMA.  Weight
// scales come into registers (four 8-byte loads per wave per eight stages,
// issued seven stages ahead); the ring holds three stages, two in flight.
// Work item = (slot, block of 256 columns of F, token block of 128 rows).
// ---------------------------------------------------------------------------
constexpr int kG1W = 8;                    // waves
constexpr int kG1Ring = 3;                 // ring stages
constexpr int kG1Ahead = kG1Ring - 1;      // stages in flight ahead of use
constexpr int kG1WStage = 32 * 1024;       // weight bytes per stage (32 tiles x 1 KB)
constexpr int kG1Cols = 256;               // act columns per item (512 weight rows)
constexpr int kG1XI = kStage / 1024 / kG1W;  // token DMA instructions per wave per stage (2)
constexpr int kG1WI = 4;                   // weight DMA instructions per wave per stage
// A stage's DMA is waited for at the start of the stage two later, with one
// more stage of DMA issued after it; the epilogue's stores (3 per token tile)
// follow the DMA of the next item's first two stages.
constexpr int kG1Vm = kG1XI + kG1WI;
constexpr int kG1Epi = 3 * 8;
constexpr size_t kG1StaticLds = (size_t)kG1Ring * (kStage + kG1WStage) + kTM * kMaxStages;
static size_t g1w_lds(int P_local) { return kG1W * kTM * sizeof(float) + 2 * (size_t)(P_local + 1) * sizeof(int); }

__global__ __launch_bounds__(kG1W * 64, 1) void k_gemm1_w(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                          const int32_t* __restrict__ offsets, int P_local,
                                                          const uint8_t* __restrict__ pw,
                                                          const uint8_t* __restrict__ pws, uint8_t* __restrict__ aq,
                                                          uint8_t* __restrict__ as_, int H, int F) {
  __shared__ __align__(16) uint8_t g0s[kStage + kG1WStage], g1s[kStage + kG1WStage], g2s[kStage + kG1WStage];
  __shared__ __align__(16) uint8_t s_xs[kTM * kMaxStages];  // [stage][16][8] token scales
  extern __shared__ __align__(16) uint8_t lds[];
  const int K = H, R = 2 * F;
  const int nwb = (F + kG1Cols - 1) / kG1Cols;
  const int nst = K / 128;
  const int nst4 = (nst + 3) & ~3;
  const PackGeom Gm = pack_geom((uint32_t)R, (uint32_t)K);
  const int ngrp = (int)Gm.steps / 4;  // scale words of 8 stages
  float* s_amax = reinterpret_cast<float*>(lds);            // [8 waves][kTM]
  int* s_pre = reinterpret_cast<int*>(s_amax + kG1W * kTM);  // [P_local + 1] items before slot
  int* s_off = s_pre + P_local + 1;                         // [P_local + 1] bucket offsets
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int sw = swz(l16);

  for (int p = tid; p <= P_local; p += blockDim.x) s_off[p] = offsets[p];
  __syncthreads();
  for (int p = tid; p < P_local; p += blockDim.x) s_pre[p + 1] = (s_off[p + 1] - s_off[p] + kTM - 1) / kTM * nwb;
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int p = 1; p <= P_local; ++p) {
      run += s_pre[p];
      s_pre[p] = run;
    }
  }
  __syncthreads();
  const int nitems = s_pre[P_local];
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int chunk = (nitems + 7) / 8;
  const int i0 = xcd * chunk, i1 = min(nitems, i0 + chunk);
  if (i0 + lb >= i1) return;  // block-uniform: no item for this block

  uint32_t xt[kG1XI], xp[kG1XI];  // token DMA instruction wave + 8m: token row, byte offset of the lane's piece
#pragma unroll
  for (int m = 0; m < kG1XI; ++m) {
    const int t = 8 * (wave + kG1W * m) + (lane >> 3);
    xt[m] = (uint32_t)t;
    xp[m] = 16u * (uint32_t)((lane & 7) ^ swz(t & 15));
  }
  const uint32_t wlane = 16u * lane, slane = 8u * lane;
  const uint32_t wlim = (uint32_t)Gm.data_slot, slim = (uint32_t)Gm.scale_slot;

  auto decode = [&](int item) {
    TItem it;
    it.live = item < i1;
    int s = 0, wb = 0, tb = 0, n = 0;
    if (it.live) {
      int lo = 0, hi = P_local - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= item) lo = mid;
        else hi = mid - 1;
      }
      s = lo;
      n = s_off[s + 1] - s_off[s];
      const int ntb = (n + kTM - 1) / kTM;
      const int local = item - s_pre[s];
      wb = local / ntb;
      tb = local - wb * ntb;
    }
    it.s = __builtin_amdgcn_readfirstlane(s);
    it.wb = __builtin_amdgcn_readfirstlane(wb);
    it.r0 = __builtin_amdgcn_readfirstlane(s_off[s] + tb * kTM);
    it.nvalid = __builtin_amdgcn_readfirstlane(it.live ? min(kTM, n - tb * kTM) : 0);
    it.live = __builtin_amdgcn_readfirstlane(it.live);
    const int c0 = it.wb * kG1Cols + wave * 32;  // this wave's 32 columns of F
    it.wlive = it.live && c0 < F;               // F is a multiple of 128
    it.tl[0] = c0 / 16;                          // gate tiles tl[0], tl[0] + 1
    it.tl[1] = (F + c0) / 16;                    // up tiles tl[1], tl[1] + 1
    return it;
  };

  auto dma_x = [&](const TItem it, uint8_t* slot, int q) {  // token stage q
    const bool live = it.live && q < nst;
    const uint32_t xlim = (uint32_t)it.nvalid * (uint32_t)K;
    const rsrc_t Xr = make_rsrc(xq + (size_t)it.r0 * K, xlim);
#pragma unroll
    for (int m = 0; m < kG1XI; ++m) {
      const uint32_t vo = (live && xt[m] < (uint32_t)it.nvalid) ? xt[m] * (uint32_t)K + xp[m] : xlim;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (lds_ptr_t)(slot + (wave + kG1W * m) * 1024), 16, vo,
                                               live ? (uint32_t)q * 128u : 0u, 0, 0);
    }
  };
  // Loads of nothing (no item, no tiles, past K) go through a zero-sized
  // buffer, so the lane offsets stay loop constants.
  auto dma_w = [&](const TItem it, uint8_t* slot, int q) {  // this wave's four weight tiles of stage q
    const bool live = it.wlive && q < nst;
    const rsrc_t Wr = make_rsrc(pw + (size_t)it.s * Gm.data_slot, live ? wlim : 0u);
    const uint32_t so = (uint32_t)(q >> 1) * 2048u + (uint32_t)(q & 1) * 1024u;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t tile = (uint32_t)(((a >> 1) ? it.tl[1] : it.tl[0]) + (a & 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Wr, (lds_ptr_t)(slot + wave * 4096 + a * 1024), 16, wlane,
                                               live ? tile * (uint32_t)Gm.data_tile + so : 0u, 0, kWeightNt);
    }
  };
  // the four tiles' scales of group grp (stages 8 grp .. 8 grp + 7): byte q % 8 scales stage q
  auto load_scales = [&](const TItem it, int grp, v2i (&sc)[4]) {
    const bool live = it.wlive && grp < ngrp;
    const rsrc_t Sr = make_rsrc(pws + (size_t)it.s * Gm.scale_slot, live ? slim : 0u);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t tile = (uint32_t)(((a >> 1) ? it.tl[1] : it.tl[0]) + (a & 1));
      sc[a] = buf_load8(Sr, slane, live ? tile * (uint32_t)Gm.scale_tile + (uint32_t)grp * 512u : 0u);
    }
  };

  constexpr int kTPR = kG1W * 64 / kTM;          // threads per token row
  constexpr int kXsPer = kMaxStages / 4 / kTPR;  // dwords per thread
  const bool xs_dw = (nst & 3) == 0;
  auto xs_fetch = [&](const TItem it, uint32_t (&v)[kXsPer]) {
    const int t = tid / kTPR;
    const bool ok = xs_dw && it.live && t < it.nvalid;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(xs + (size_t)(it.r0 + t) * nst);
#pragma unroll
    for (int j = 0; j < kXsPer; ++j) {
      const int d = (tid % kTPR) + kTPR * j;
      v[j] = (ok && 4 * d < nst) ? __hip_atomic_load(src + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    }
  };
  auto xs_store = [&](const TItem it, const uint32_t (&v)[kXsPer]) {
    const int t = tid / kTPR;
    uint8_t* dst = s_xs + (t & 15) * 8 + (t >> 4);
    if (xs_dw) {
#pragma unroll
      for (int j = 0; j < kXsPer; ++j) {
        const int d = (tid % kTPR) + kTPR * j;
        if (4 * d < nst4) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) dst[(4 * d + bb) * kTM] = (uint8_t)(v[j] >> (8 * bb));
        }
      }
    } else {
      const bool ok = it.live && t < it.nvalid;
      const uint8_t* src = xs + (size_t)(it.r0 + t) * nst;
      for (int c = tid % kTPR; c < nst4; c += kTPR) dst[c * kTM] = (ok && c < nst) ? src[c] : (uint8_t)0;
    }
  };

  const int o_lo = (g ^ sw) * 16, o_hi = ((g + 4) ^ sw) * 16;
  v2i scc[4], scn[4];  // weight scales: the current group, the next one
  v4f acc[4][8];
  constexpr int kTile = 16 * 128;

  auto ldb = [&](V8T& b, uint32_t blo, uint32_t bhi, auto ttc) {
    constexpr int o = decltype(ttc)::value * kTile;
    b.h[0] = lds_read16_at<o>(blo);
    b.h[1] = lds_read16_at<o>(bhi);
  };
  // stage q: LDS reads in issue order (they complete in order): weights (4),
  // token scales (1), token tiles 0 and 1 (2 + 2), then tile tt + 2's two
  // reads before tile tt's four MFMAs.
  auto compute = [&](bool wlive, const uint8_t* xs_slot, const uint8_t* w_slot, int q) {
    if (!wlive) return;
    const uint32_t aa = lds_addr(w_slot + wave * 4096 + lane * 16);
    const uint32_t blo = lds_addr(xs_slot + l16 * 128 + o_lo), bhi = lds_addr(xs_slot + l16 * 128 + o_hi);
    v4i a[4];
    a[0] = lds_read16_at<0>(aa);
    a[1] = lds_read16_at<1024>(aa);
    a[2] = lds_read16_at<2048>(aa);
    a[3] = lds_read16_at<3072>(aa);
    const v2i sbw = lds_read8(s_xs + q * kTM + l16 * 8);
    V8T b[3];
    ldb(b[0], blo, bhi, std::integral_constant<int, 0>{});
    ldb(b[1], blo, bhi, std::integral_constant<int, 1>{});
    int sa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = (int)((uint32_t)((q & 4) ? scc[i].y : scc[i].x) >> (8 * (q & 3)));
    MOE_LGKM_WAIT(4);  // weights and token scales are in
    __builtin_amdgcn_sched_barrier(0);
    int sb[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) sb[tt] = (int)(((uint32_t)(tt < 4 ? sbw.x : sbw.y) >> (8 * (tt & 3))) & 0xFFu);
    __builtin_amdgcn_sched_barrier(0);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt + 2 < 8) ldb(b[(tt + 2) % 3], blo, bhi, std::integral_constant<int, tt + 2>{});
      if constexpr (tt + 2 < 8) MOE_LGKM_WAIT(4);
      else if constexpr (tt + 1 < 8) MOE_LGKM_WAIT(2);
      else MOE_LGKM_WAIT(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][tt] = mfma_fp4_fp8<0>(a[i], b[tt % 3].v, acc[i][tt], sa[i], sb[tt]);
      __builtin_amdgcn_sched_barrier(0);
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    tile(std::integral_constant<int, 2>{});
    tile(std::integral_constant<int, 3>{});
    tile(std::integral_constant<int, 4>{});
    tile(std::integral_constant<int, 5>{});
    tile(std::integral_constant<int, 6>{});
    tile(std::integral_constant<int, 7>{});
  };

  auto ring = [&](int i) -> uint8_t* { return i == 0 ? g0s : (i == 1 ? g1s : g2s); };  // a select: no table of LDS addresses

  // ---- first item: its token scales, first scale group and first stages
  TItem cur = decode(i0 + lb);
  bool after_epi = false;  // an epilogue's stores are in flight (every item but the first)
  {
    uint32_t v[kXsPer];
    xs_fetch(cur, v);
    xs_store(cur, v);
  }
  load_scales(cur, 0, scn);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kG1Ahead; ++q) {
    dma_x(cur, ring(q), q);
    dma_w(cur, ring(q) + kStage, q);
  }
  int slot = 0;  // ring slot of the current stage

  for (int item = i0 + lb; item < i1; item += nper) {
    const TItem nxt = decode(item + nper);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[i][tt] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage: wait for its DMA (own, then everyone's via the barrier,
    // which also retires the slot the next DMA refills), issue stage q + 2
    // (of this item or, past its end, of the next), compute stage q
    auto stage = [&](int q) {
      if (after_epi && q < kG1Ahead)
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kG1Vm + kG1Epi) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kG1Vm) : "memory");
      bare_barrier();
      if ((q & 7) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) scc[i] = scn[i];
      }
      // the next scale group, of this item or the next item's first; issued
      // before the stage's DMA, so that any wait the compiler places for it
      // leaves that DMA in flight
      if ((q & 7) == 1) {
        if ((q >> 3) + 1 < ngrp && 8 * ((q >> 3) + 1) < nst4) load_scales(cur, (q >> 3) + 1, scn);
        else load_scales(nxt, 0, scn);
      }
      uint8_t* const fill = ring(slot == 0 ? kG1Ring - 1 : slot - 1);  // the slot read by stage q - 1
      if (q + kG1Ahead < nst4) {
        dma_x(cur, fill, q + kG1Ahead);
        dma_w(cur, fill + kStage, q + kG1Ahead);
      } else {
        dma_x(nxt, fill, q + kG1Ahead - nst4);
        dma_w(nxt, fill + kStage, q + kG1Ahead - nst4);
      }
      compute(cur.wlive, ring(slot), ring(slot) + kStage, q);
      slot = slot == kG1Ring - 1 ? 0 : slot + 1;
    };
    for (int q0 = 0; q0 < nst4 - 4; q0 += 4) {
      stage(q0);
      stage(q0 + 1);
      stage(q0 + 2);
      stage(q0 + 3);
    }
    uint32_t xsn[kXsPer];
    xs_fetch(nxt, xsn);
    stage(nst4 - 4);
    stage(nst4 - 3);
    stage(nst4 - 2);
    stage(nst4 - 1);

    // ---- epilogue: SwiGLU in place (acc[0..1] become act of the gate
    // tiles' columns), the requant amax over 128 columns (this wave's 32 and
    // the three other waves of its group of four), fp8 codes and scales
    // through buffers sized to the item's rows
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
      if (g == 0) s_amax[wave * kTM + tt * 16 + l16] = m;
    }
    MOE_LGKM_WAIT(0);
    bare_barrier();
    {
      const int nfb = F / kActBlock;
      const int c0 = cur.wb * kG1Cols + wave * 32;
      const rsrc_t Ar = make_rsrc(aq + (size_t)cur.r0 * F, cur.wlive ? (uint32_t)cur.nvalid * (uint32_t)F : 0u);
      const uint32_t slim_as = (uint32_t)cur.nvalid * (uint32_t)nfb;
      const rsrc_t Sr = make_rsrc(as_ + (size_t)cur.r0 * nfb, cur.wlive ? slim_as : 0u);
      const float* am0 = s_amax + (wave & ~3) * kTM;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tok = tt * 16 + l16;
        const int e = scale_exp(fmaxf(fmaxf(am0[tok], am0[kTM + tok]), fmaxf(am0[2 * kTM + tok], am0[3 * kTM + tok])));
        const uint32_t ao = (uint32_t)tok * (uint32_t)F + (uint32_t)(c0 + 4 * g);
        __builtin_amdgcn_raw_buffer_store_b32(pack4_fp8(ldexpf(acc[0][tt][0], -e), ldexpf(acc[0][tt][1], -e),
                                                        ldexpf(acc[0][tt][2], -e), ldexpf(acc[0][tt][3], -e)),
                                              Ar, ao, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(pack4_fp8(ldexpf(acc[1][tt][0], -e), ldexpf(acc[1][tt][1], -e),
                                                        ldexpf(acc[1][tt][2], -e), ldexpf(acc[1][tt][3], -e)),
                                              Ar, ao + 16u, 0, 0);
        const uint32_t so = ((wave & 3) == 0 && g == 0) ? (uint32_t)tok * (uint32_t)nfb + (uint32_t)(c0 / kActBlock)
                                                        : slim_as;
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(e + 127), Sr, so, 0, 0);
      }
    }
    after_epi = true;
    bare_barrier();  // every wave is done with this item's token scales and amax
    xs_store(nxt, xsn);
    MOE_LGKM_WAIT(0);
    cur = nxt;
  }
}

static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

constexpr size_t kTiledStaticLds = (size_t)kRing * (kStage + kWStage) + 2 * kSGroup + kTM * kMaxStages;

// dynamic LDS of the GEMM2 kernel: the item prefix and the bucket offsets
static size_t tiled_lds(int P_local) { return 2 * (size_t)(P_local + 1) * sizeof(int); }

bool tiled_fits(int H, int F, int P_local) {
  return H / 128 <= kMaxStages && F / 128 <= kMaxStages && kTiledStaticLds + tiled_lds(P_local) <= kTiledLdsMax &&
         kG1StaticLds + g1w_lds(P_local) <= kTiledLdsMax;
}

// Dynamic LDS above the default limit is opted into per kernel and device,
// once per size.
static hipError_t grant_lds(const void* fn, size_t lds, size_t (&granted)[64]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || lds > granted[dev]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) granted[dev] = lds;
  }
  return hipSuccess;
}

hipError_t launch_gemm1_tiled(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                              const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                              hipStream_t st) {
  const size_t lds = g1w_lds(P_local);
  static size_t granted[64] = {};
  hipError_t e = grant_lds(reinterpret_cast<const void*>(&k_gemm1_w), lds, granted);
  if (e != hipSuccess) return e;
  k_gemm1_w<<<num_cus() / 8 * 8, kG1W * 64, lds, st>>>(xq, xs, offsets, P_local, pw1, pw1s, aq, as, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm2_tiled(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  const size_t lds = tiled_lds(P_local);
  static size_t granted[64] = {};
  hipError_t e = grant_lds(reinterpret_cast<const void*>(&k_gemm2_tiled), lds, granted);
  if (e != hipSuccess) return e;
  k_gemm2_tiled<<<num_cus() / 8 * 8, kNW * 64, lds, st>>>(aq, as, offsets, P_local, pw2, pw2s, y, H, F);
  return hipGetLastError();
}

}  // namespace moe
