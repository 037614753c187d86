// Large-M path: persistent grouped GEMMs for many rows per expert (block-
// scaled fp8 x MXFP4 MFMA on gfx950).  Same arithmetic as the streaming
// kernels (a5 GEMM1 + SwiGLU + fp8 requant, a6 GEMM2 into f32 rows), tiled
// for MFMA throughput: the pages' persistent large-input path serves extend
// steps of at least 1024 tokens per rank [sglang PR 47065 "Use the aiter
// MegaMoE small- and large-input paths", Modifications].
//
// Work item = (local slot s, weight block of 256 rows, token block of 128
// rows of the slot's bucket), token block fastest, so the items that run at
// the same time on one XCD share their weight block in that XCD's L2.  The
// grid is one block per CU; each block walks items of its XCD's contiguous
// range.
//
// Block = 4 waves, one block per CU: one wave per SIMD, so the 32
// accumulator tiles live in AGPRs next to a deep operand pipeline in VGPRs.
// Wave w owns four 16-row weight tiles (GEMM1: the gate and up tiles of 32
// columns of F; GEMM2: 64 rows of H) against the eight 16-token tiles of the
// block: 32 accumulators of 16x16 (128 registers).  K advances 128 per stage
// (one V_MFMA_SCALE_F32_16X16X128_F8F6F4 per tile pair).
//  - Token rows: direct-to-LDS DMA (buffer_load_dwordx4 ... lds), a ring of
//    kRing stages issued kRing - 1 stages ahead; each stage row of 128 bytes
//    is stored with its eight 16-byte pieces XOR-swizzled so the B-operand
//    reads of a 16-token tile hit distinct banks.
//  - Weight tiles: streamed from HBM straight into registers (the packed
//    layout is the MFMA operand order), three stages ahead.
//  - Stage barriers are bare s_barrier with explicit vmcnt waits: the
//    generic workgroup barrier would drain every load in flight.

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

// DMA instructions a wave issues after a stage's own (4 token + 4 weight) by
// the time that stage is consumed: two more stages of 8.  Scale-group DMA
// only adds to the count, which keeps the wait sufficient.  (Scale groups are
// issued four stages before their first use, with at least 24 DMA
// instructions after them by then: complete under the same wait.)
#define MOE_TILED_VMCNT "16"

// Physical 16-byte piece of logical piece p in the stage row of the token at
// position r (mod 16) of its tile: p ^ swz(r).  Eight consecutive tokens, and
// sixteen, land on distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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

template <bool G1>
__global__ __launch_bounds__(256, 1) void k_grouped(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                    const int32_t* __restrict__ offsets, int P_local,
                                                    const uint8_t* __restrict__ pw, const uint8_t* __restrict__ pws,
                                                    uint8_t* __restrict__ aq, uint8_t* __restrict__ as_,
                                                    float* __restrict__ y, int H, int F) {
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
  const int K = G1 ? H : F;
  const int R = G1 ? 2 * F : H;
  const int nwb = G1 ? F / kActBlock : (H + kTN - 1) / kTN;
  const int nst = K / 128;               // stages with data (K is a multiple of 128)
  const int nst4 = (nst + 3) & ~3;       // stages run per item: whole ring turns
  const PackGeom Gm = pack_geom((uint32_t)R, (uint32_t)K);
  const int ngrp = (int)Gm.steps / 4;    // scale groups (8 stages each); 8 ngrp >= nst4
  float* s_amax = reinterpret_cast<float*>(lds);            // [4][kTM]
  int* s_pre = reinterpret_cast<int*>(s_amax + 4 * kTM);    // [P_local + 1] items before slot
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
  // a contiguous item range per XCD (block b runs on XCD b % 8)
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int chunk = (nitems + 7) / 8;
  const int i0 = xcd * chunk, i1 = min(nitems, i0 + chunk);
  if (i0 + lb >= i1) return;  // block-uniform: no item for this block

  // lane constants of the DMA offsets
  uint32_t xt[4], xp[4];  // token DMA instruction wave + 4m: token row and byte offset of the lane's piece
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 8 * (wave + 4 * m) + (lane >> 3);
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
    it.wlive = it.live && (G1 || wb * kTN + wave * 64 < H);  // H is a multiple of 128
    if (G1) {  // gate and up tiles of columns f0 .. f0 + 31
      const int f0 = it.wb * kActBlock + wave * 32;
      it.tl[0] = f0 / 16;
      it.tl[1] = (F + f0) / 16;
    } else {   // rows h0 .. h0 + 63
      const int h0 = it.wb * kTN + wave * 64;
      it.tl[0] = h0 / 16;
      it.tl[1] = h0 / 16 + 2;
    }
    return it;
  };

  // DMA issue.  Every stage moves the same number of instructions (past the
  // data: offsets beyond the buffer, which read zeros and move nothing).
  auto dma_x = [&](const TItem it, uint8_t* slot, int q) {  // token stage q
    const bool live = it.live && q < nst;
    const uint32_t xlim = (uint32_t)it.nvalid * (uint32_t)K;
    const rsrc_t Xr = make_rsrc(xq + (size_t)it.r0 * K, xlim);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t vo = (live && xt[m] < (uint32_t)it.nvalid) ? xt[m] * (uint32_t)K + xp[m] : xlim;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (lds_ptr_t)(slot + (wave + 4 * m) * 1024), 16, vo,
                                               live ? (uint32_t)q * 128u : 0u, 0, 0);
    }
  };
  auto dma_w = [&](const TItem it, uint8_t* slot, int q) {  // this wave's four weight tiles of stage q
    const bool live = it.wlive && q < nst;
    const rsrc_t Wr = make_rsrc(pw + (size_t)it.s * Gm.data_slot, wlim);
    const uint32_t so = (uint32_t)(q >> 1) * 2048u + (uint32_t)(q & 1) * 1024u;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t tile = (uint32_t)(it.tl[rt >> 1] + (rt & 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Wr, (lds_ptr_t)(slot + wave * 4096 + rt * 1024), 16,
                                               live ? wlane : wlim, live ? tile * (uint32_t)Gm.data_tile + so : 0u, 0,
                                               kWeightNt);
    }
  };
  auto dma_s = [&](const TItem it, int grp, int par) {  // this wave's scales of group grp into slot par
    const bool live = it.wlive && grp < ngrp;
    const rsrc_t Sr = make_rsrc(pws + (size_t)it.s * Gm.scale_slot, slim);
    uint8_t* slot = sring + par * kSGroup + wave * 2048;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Sr, (lds_ptr_t)(slot + h * 1024), 16, live ? slane : slim,
                                               live ? (uint32_t)it.tl[h] * (uint32_t)Gm.scale_tile + (uint32_t)grp * 512u : 0u,
                                               0, 0);
  };
  // The item's token scales, stage-major: byte tt of lane record [q][r] is
  // the scale of token 16 tt + r at stage q (one 8-byte read gives a lane all
  // eight); stages past the data hold 0.  Two threads per token row.  Rows of
  // a multiple of 4 bytes are fetched as dwords into registers well ahead of
  // use (relaxed atomic loads: issued where written, not sunk to the use);
  // other widths are read byte by byte when stored.
  constexpr int kXsPer = kMaxStages / 8;  // dwords per thread
  const bool xs_dw = (nst & 3) == 0;
  auto xs_fetch = [&](const TItem it, uint32_t (&v)[kXsPer]) {
    const int t = tid >> 1;
    const bool ok = xs_dw && it.live && t < it.nvalid;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(xs + (size_t)(it.r0 + t) * nst);
#pragma unroll
    for (int j = 0; j < kXsPer; ++j) {
      const int d = (tid & 1) + 2 * j;  // dword of the row
      v[j] = (ok && 4 * d < nst) ? __hip_atomic_load(src + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    }
  };
  auto xs_store = [&](const TItem it, const uint32_t (&v)[kXsPer]) {
    const int t = tid >> 1;
    uint8_t* dst = s_xs + (t & 15) * 8 + (t >> 4);
    if (xs_dw) {
#pragma unroll
      for (int j = 0; j < kXsPer; ++j) {
        const int d = (tid & 1) + 2 * j;
        if (4 * d < nst4) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) dst[(4 * d + bb) * kTM] = (uint8_t)(v[j] >> (8 * bb));
        }
      }
    } else {
      const bool ok = it.live && t < it.nvalid;
      const uint8_t* src = xs + (size_t)(it.r0 + t) * nst;
      for (int c = tid & 1; c < nst4; c += 2) dst[c * kTM] = (ok && c < nst) ? src[c] : (uint8_t)0;
    }
  };

  const int o_lo = (g ^ sw) * 16, o_hi = ((g + 4) ^ sw) * 16;
  v2i sc[4];  // weight scales of the current group: byte q % 8 scales stage q
  v4f acc[4][8];

  // all eight token tiles of stage q (tiles past the block's rows hold zeros)
  auto compute = [&](bool wlive, const uint8_t* xs_slot, const uint8_t* w_slot, int q) {
    if (!wlive) return;
    // LDS reads in issue order (they complete in order): weights (4), token
    // scales (1), token tiles 0 and 1 (2 + 2), then tile tt + 2's two reads
    // before tile tt's MFMAs.  Tile tt's operands are complete once at most
    // the reads of the two later tiles are outstanding.  Addresses are one
    // register each plus immediate offsets.
    const uint32_t aa = lds_addr(w_slot + wave * 4096 + lane * 16);
    const uint32_t blo = lds_addr(xs_slot + l16 * 128 + o_lo), bhi = lds_addr(xs_slot + l16 * 128 + o_hi);
    v4i a[4];
    a[0] = lds_read16_at<0>(aa);
    a[1] = lds_read16_at<1024>(aa);
    a[2] = lds_read16_at<2048>(aa);
    a[3] = lds_read16_at<3072>(aa);
    const v2i sbw = lds_read8(s_xs + q * kTM + l16 * 8);
    V8T b[3];
    b[0].h[0] = lds_read16_at<0>(blo);
    b[0].h[1] = lds_read16_at<0>(bhi);
    b[1].h[0] = lds_read16_at<2048>(blo);
    b[1].h[1] = lds_read16_at<2048>(bhi);
    int sa[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) sa[rt] = (int)((uint32_t)((q & 4) ? sc[rt].y : sc[rt].x) >> (8 * (q & 3)));
    MOE_LGKM_WAIT(4);  // weights and token scales are in
    __builtin_amdgcn_sched_barrier(0);
    int sb[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) sb[tt] = (int)(((uint32_t)(tt < 4 ? sbw.x : sbw.y) >> (8 * (tt & 3))) & 0xFFu);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      if (tt + 2 < 8) {
        constexpr int kTile = 16 * 128;
        switch (tt) {  // immediate offsets of tile tt + 2
          case 0: b[2].h[0] = lds_read16_at<2 * kTile>(blo); b[2].h[1] = lds_read16_at<2 * kTile>(bhi); break;
          case 1: b[0].h[0] = lds_read16_at<3 * kTile>(blo); b[0].h[1] = lds_read16_at<3 * kTile>(bhi); break;
          case 2: b[1].h[0] = lds_read16_at<4 * kTile>(blo); b[1].h[1] = lds_read16_at<4 * kTile>(bhi); break;
          case 3: b[2].h[0] = lds_read16_at<5 * kTile>(blo); b[2].h[1] = lds_read16_at<5 * kTile>(bhi); break;
          case 4: b[0].h[0] = lds_read16_at<6 * kTile>(blo); b[0].h[1] = lds_read16_at<6 * kTile>(bhi); break;
          case 5: b[1].h[0] = lds_read16_at<7 * kTile>(blo); b[1].h[1] = lds_read16_at<7 * kTile>(bhi); break;
        }
      }
      if (tt < 6) MOE_LGKM_WAIT(4);
      else if (tt == 6) MOE_LGKM_WAIT(2);
      else MOE_LGKM_WAIT(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][tt] = mfma_fp4_fp8<0>(a[rt], b[tt % 3].v, acc[rt][tt], sa[rt], sb[tt]);
      __builtin_amdgcn_sched_barrier(0);
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
  dma_x(cur, xring[0], 0);
  dma_w(cur, wring[0], 0);
  dma_x(cur, xring[1], 1);
  dma_w(cur, wring[1], 1);
  dma_x(cur, xring[2], 2);
  dma_w(cur, wring[2], 2);

  for (int item = i0 + lb; item < i1; item += nper) {
    // the next item: decoded now; its first stages and first scale group are
    // moved in during this item's last stages, its token scales fetched into
    // registers at the start of the last four (stored at the item boundary)
    const TItem nxt = decode(item + nper);

#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[rt][tt] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage (ring slot u = q % kRing, a compile-time constant): wait for
    // its rows and weights (own DMA, then everyone's via the barrier, which
    // also retires the slot the next DMA refills), issue stage q + 3 (of
    // this item or, past its end, of the next), compute stage q
    auto stage = [&](auto uc, int q) {
      constexpr int u = decltype(uc)::value;
      asm volatile("s_waitcnt vmcnt(" MOE_TILED_VMCNT ")" ::: "memory");
      bare_barrier();
      if ((q & 7) == 0 && cur.wlive) {  // a new scale group (its DMA was issued at least three stages ago)
        const uint8_t* sp = sring + ((gpar + (q >> 3)) & 1) * kSGroup + wave * 2048 + lane * 8;
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

    // ---- epilogue (LDS exchanges use bare barriers: the next item's DMA
    // stays in flight)
    const int ntt = (cur.nvalid + 15) / 16;
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
        if (g == 0) s_amax[wave * kTM + tt * 16 + l16] = m;
      }
      MOE_LGKM_WAIT(0);
      bare_barrier();
      const int nfb = F / kActBlock;
      const int f0 = cur.wb * kActBlock + wave * 32;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tok = tt * 16 + l16;
        if (tt >= ntt || tok >= cur.nvalid) continue;
        const float am = fmaxf(fmaxf(s_amax[tok], s_amax[kTM + tok]), fmaxf(s_amax[2 * kTM + tok], s_amax[3 * kTM + tok]));
        const int e = scale_exp(am);
        uint8_t* ap = aq + (size_t)(cur.r0 + tok) * F + f0 + 4 * g;
        *reinterpret_cast<uint32_t*>(ap) = pack4_fp8(ldexpf(acc[0][tt][0], -e), ldexpf(acc[0][tt][1], -e),
                                                     ldexpf(acc[0][tt][2], -e), ldexpf(acc[0][tt][3], -e));
        *reinterpret_cast<uint32_t*>(ap + 16) = pack4_fp8(ldexpf(acc[1][tt][0], -e), ldexpf(acc[1][tt][1], -e),
                                                          ldexpf(acc[1][tt][2], -e), ldexpf(acc[1][tt][3], -e));
        if (wave == 0 && g == 0) as_[(size_t)(cur.r0 + tok) * nfb + cur.wb] = (uint8_t)(e + 127);
      }
    } else if (cur.wlive) {
      const int h0 = cur.wb * kTN + wave * 64;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int tok = tt * 16 + l16;
        if (tt >= ntt || tok >= cur.nvalid) continue;
        float* yr = y + (size_t)(cur.r0 + tok) * H + h0 + 4 * g;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          *reinterpret_cast<float4*>(yr + 16 * rt) =
              make_float4(acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]);
      }
    }
    // item boundary: every wave is done with this item's token scales and
    // amax; the next item's scales go in (visible after the next stage barrier)
    bare_barrier();
    xs_store(nxt, xsn);
    MOE_LGKM_WAIT(0);
    cur = nxt;
    gpar = (gpar + ngrp) & 1;
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

// dynamic LDS: the requant amax, the item prefix and the bucket offsets
static size_t tiled_lds(int P_local) { return 4 * kTM * sizeof(float) + 2 * (size_t)(P_local + 1) * sizeof(int); }

bool tiled_fits(int H, int F, int P_local) {
  return H / 128 <= kMaxStages && F / 128 <= kMaxStages && kTiledStaticLds + tiled_lds(P_local) <= kTiledLdsMax;
}

template <bool G1>
static hipError_t launch_grouped(const uint8_t* x, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw,
                                 const uint8_t* pws, uint8_t* aq, uint8_t* as, float* y, int H, int F, int P_local,
                                 hipStream_t st) {
  const size_t lds = tiled_lds(P_local);
  // dynamic LDS above the default limit is opted into per device, once per size
  static size_t granted[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || lds > granted[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_grouped<G1>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) granted[dev] = lds;
  }
  k_grouped<G1><<<num_cus() / 8 * 8, 256, lds, st>>>(x, xs, offsets, P_local, pw, pws, aq, as, y, H, F);
  return hipGetLastError();
}

hipError_t launch_gemm1_tiled(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                              const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                              hipStream_t st) {
  return launch_grouped<true>(xq, xs, offsets, pw1, pw1s, aq, as, nullptr, H, F, P_local, st);
}

hipError_t launch_gemm2_tiled(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st) {
  return launch_grouped<false>(aq, as, offsets, pw2, pw2s, nullptr, nullptr, y, H, F, P_local, st);
}

}  // namespace moe
