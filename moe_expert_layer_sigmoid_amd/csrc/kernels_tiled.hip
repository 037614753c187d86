// Large-M path: persistent grouped GEMMs for many rows per expert (block-
// scaled fp8 x MXFP4 MFMA on gfx950).  Same arithmetic as the streaming
// kernels (a5 GEMM1 + SwiGLU + fp8 requant, a6 GEMM2 into f32 rows), tiled
// for MFMA throughput: the pages' persistent large-input path serves extend
// steps of at least 1024 tokens per rank [sglang PR 47065 "Use the aiter
// MegaMoE small- and large-input paths", Modifications].
//
// One kernel template, k_tiled<G1>, for both GEMMs.  It is persistent: one
// block per CU walks the work items of its XCD's contiguous range (block b
// runs on XCD b % 8), token block fastest, so the items that run at the same
// time on one XCD share their weight block in that XCD's L2.
//  - Item: 128 tokens of a slot's bucket x 512 weight rows (GEMM1: the gate
//    and up rows of 256 columns of F; GEMM2: 512 rows of H).  Eight waves,
//    two per SIMD; wave w owns four 16-row weight tiles (GEMM1: gate and up
//    of 32 columns; GEMM2: 64 rows) against all eight 16-token tiles: 32
//    accumulators (128 registers).  Two waves per SIMD let one wave's LDS
//    and barrier waits be filled by the other's MFMAs.
//  - K advances 128 per stage (one V_MFMA_SCALE_F32_16X16X128_F8F6F4 per
//    tile pair): 32 MFMAs per wave per stage over 48 KB moved into LDS.
//  - Token rows and weight tiles: direct-to-LDS DMA (buffer_load_dwordx4 ...
//    lds) into a ring of three stages, two in flight; each token row of 128
//    bytes is stored with its eight 16-byte pieces permuted so that the
//    B-operand reads of a 16-token tile hit distinct banks; a weight tile
//    (the packed layout is the MFMA operand order) is read back with one
//    ds_read_b128 per lane.  Weight scales come into registers.
//  - A stage's DMA is issued by half of the waves (by stage parity), so
//    that while they wait for the CU's address unit to take it the other
//    wave of each SIMD runs its MFMAs; the item loop is compiled once per
//    half, each copy with a fixed DMA pattern.
//  - Stage barriers are bare s_barrier with explicit vmcnt waits: the
//    generic workgroup barrier would drain every load in flight.
//  - Epilogue: GEMM1 SwiGLU + fp8 requant, GEMM2 y rows in f32; its stores
//    are issued after the next item's first DMA, whose waits do not drain
//    them.  (Measured at the EP-shaped prefill share: stages of ~2750 clocks
//    for 2048 clocks of MFMA per SIMD; GEMM2's items are short, K = 2048,
//    and its epilogue, ~1 GB of y and output rows per call, is a fifth of
//    each item.)

#include <atomic>
#include <mutex>
#include <type_traits>

#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_layout.hpp"

namespace moe {

constexpr int kTM = 128;           // token rows per block tile
constexpr int kStage = kTM * 128;  // bytes of one token stage (128 rows x 128 K)
constexpr int kMaxStages = 64;     // K <= 8192

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
// ds_read_b128 at LDS address `a` + OFS (an immediate, < 65536)
template <int OFS>
__device__ __forceinline__ v4i lds_read16_at(uint32_t a) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFS));
  return v;
}
// ds_write_b64 of `v` at LDS address `a` + OFS (an immediate)
template <int OFS>
__device__ __forceinline__ void lds_write8_at(uint32_t a, v2i v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(a), "v"(v), "i"(OFS) : "memory");
}
__device__ __forceinline__ v2i lds_read8(const void* p) {
  v2i v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(lds_addr(p)));
  return v;
}
#define MOE_LGKM_WAIT(n) asm volatile("s_waitcnt lgkmcnt(" #n ")" ::: "memory")
// Arguments of __builtin_amdgcn_raw_ptr_buffer_load_lds: (buffer, LDS base,
// bytes per lane, voffset, soffset, immediate offset, cache policy).
// Weight cache policy (a kernel template argument, WNT): the default when the
// slots have several token blocks, since each weight stage is then read by
// every token block of the slot (non-temporal loads dropped the L2 hit rate
// from 77 % to 53 % at ~1000 rows per slot and cost 3 % there); non-temporal
// when a slot's rows fit about one block, where nothing re-reads the weights
// (GEMM1 -5 % at 62 rows per slot).
constexpr int kWeightNtLoads = 2;

union V8T {
  v8i v;
  v4i h[2];
};

// One work item: wave-uniform scalars only (per-lane DMA offsets are lane
// constants plus uniform parts).
struct TItem {
  int live;      // an item (0: every DMA of it reads zeros)
  int wlive;     // the wave's weight tiles exist (a partial last block)
  int s, wb, r0, nvalid;
  int tl[2];     // the wave's weight tiles: tl[0], tl[0] + 1, tl[1], tl[1] + 1
};

constexpr int kWaves = 8;                      // waves per block
constexpr int kIssuers = kWaves / 2;           // waves that issue one stage's DMA
constexpr int kRing = 3;                       // ring stages
constexpr int kAhead = kRing - 1;              // stages in flight ahead of use
constexpr int kWStage = 32 * 1024;             // weight bytes per stage (32 tiles x 1 KB)
constexpr int kCols = 256;                     // GEMM1: act columns per item (512 weight rows)
constexpr int kXI = kStage / 1024 / kIssuers;  // token DMA instructions per issuing wave per stage (4)
// Each stage's DMA (16 token and 32 weight instructions of 1 KB) is issued by
// one half of the waves: waves 0-3 for even stages, 4-7 for odd ones, wave
// u + 4h covering the token pieces u, u + 4, ... and the weight tiles of
// waves u and u + 4.  A wave stalls while its DMA instructions queue for the
// CU's address unit (about 900 clocks for a stage's 48); with the issue split
// by stage parity the other wave of each SIMD runs its MFMAs meanwhile.
// A stage's DMA is waited for, by the waves that issued it, at the start of
// the stage two later (vmcnt 0: their weight-scale loads of the stage between
// are waited for with it), except that an epilogue's stores (GEMM1: 3 per
// token tile; GEMM2: 4 of y and 2 of bf16 output rows per token tile) follow
// the DMA of the next item's first two stages and stay in flight.
template <bool G1>
constexpr int kEpiStores = G1 ? 3 * 8 : 6 * 8;
// GEMM2's bf16 output rows pass through LDS on their way out: per wave, 16
// rows of 64 bf16 values with a padded pitch (in the ring slot that no DMA
// targets at the item's end).
constexpr int kOutPitch = 144;
static_assert(kEpiStores<false> <= 63, "vmcnt range");
static_assert(kWaves * 16 * kOutPitch <= kStage + kWStage, "output rows fit one ring slot");
constexpr size_t kStaticLds = (size_t)kRing * (kStage + kWStage) + kTM * kMaxStages;
// dynamic LDS: the requant amax, the item prefix and the bucket offsets
static size_t tiled_lds(int P_local) { return kWaves * kTM * sizeof(float) + 2 * (size_t)(P_local + 1) * sizeof(int); }

template <bool G1, int WNT>
__global__ __launch_bounds__(kWaves * 64, 1) void k_tiled(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                        const int32_t* __restrict__ offsets, int P_local,
                                                        const uint8_t* __restrict__ pw, const uint8_t* __restrict__ pws,
                                                        uint8_t* __restrict__ aq, uint8_t* __restrict__ as_,
                                                        float* __restrict__ y, int H, int F, SingleRows sr) {
  __shared__ __align__(16) uint8_t g0s[kStage + kWStage], g1s[kStage + kWStage], g2s[kStage + kWStage];
  __shared__ __align__(16) uint8_t s_xs[kTM * kMaxStages];  // [stage][16][8] token scales
  extern __shared__ __align__(16) uint8_t lds[];
  const int K = G1 ? H : F, R = G1 ? 2 * F : H;
  const int nwb = G1 ? (F + kCols - 1) / kCols : (H + 2 * kCols - 1) / (2 * kCols);
  const int nst = K / 128;
  const int nst4 = (nst + 3) & ~3;
  const PackGeom Gm = pack_geom((uint32_t)R, (uint32_t)K);
  const int ngrp = (int)Gm.steps / 4;  // scale words of 8 stages
  float* s_amax = reinterpret_cast<float*>(lds);               // [8 waves][kTM]
  int* s_pre = reinterpret_cast<int*>(s_amax + kWaves * kTM);  // [P_local + 1] items before slot
  // GEMM2: the current item's rows of single-pair tokens (the GEMM1 amax area):
  // s_rinf[r] = token of row r (or -1), s_rinf[kTM + r] = its routing weight
  int* s_rinf = reinterpret_cast<int*>(lds);
  int* s_off = s_pre + P_local + 1;                            // [P_local + 1] bucket offsets
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

  // token DMA instruction u + 4m of an issuing wave (u = wave & 3) moves
  // rows 8 (u + 4m) .. + 7: the lane's row is xt0 + 32m, its piece's byte
  // offset xp (row & 15 does not depend on m)
  const int iu = wave & (kIssuers - 1), igrp = wave / kIssuers;
  const uint32_t xt0 = (uint32_t)(8 * iu + (lane >> 3));
  const uint32_t xp = 16u * (uint32_t)((lane & 7) ^ swz((int)(xt0 & 15)));
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
    if (G1) {
      const int c0 = it.wb * kCols + wave * 32;  // this wave's 32 columns of F
      it.wlive = it.live && c0 < F;               // F is a multiple of 128
      it.tl[0] = c0 / 16;                          // gate tiles tl[0], tl[0] + 1
      it.tl[1] = (F + c0) / 16;                    // up tiles tl[1], tl[1] + 1
    } else {
      const int h0 = it.wb * 2 * kCols + wave * 64;  // this wave's 64 rows of H
      it.wlive = it.live && h0 < H;                   // H is a multiple of 128
      it.tl[0] = h0 / 16;
      it.tl[1] = h0 / 16 + 2;
    }
    return it;
  };

  auto dma_x = [&](const TItem it, uint8_t* slot, int q) {  // this wave's token pieces of stage q
    const bool live = it.live && q < nst;
    const uint32_t xlim = (uint32_t)it.nvalid * (uint32_t)K;
    const rsrc_t Xr = make_rsrc(xq + (size_t)it.r0 * K, xlim);
#pragma unroll
    for (int m = 0; m < kXI; ++m) {
      const uint32_t t = xt0 + 32u * (uint32_t)m;
      const uint32_t vo = (live && t < (uint32_t)it.nvalid) ? t * (uint32_t)K + xp : xlim;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Xr, (lds_ptr_t)(slot + (iu + kIssuers * m) * 1024), 16, vo,
                                               live ? (uint32_t)q * 128u : 0u, 0, 0);
    }
  };
  // Loads of nothing (no item, no tiles, past K) go through a zero-sized
  // buffer, so the lane offsets stay loop constants.
  auto dma_w = [&](const TItem it, uint8_t* slot, int q) {  // the weight tiles of waves iu and iu + 4, stage q
    const uint32_t so = (uint32_t)(q >> 1) * 2048u + (uint32_t)(q & 1) * 1024u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int w = iu + kIssuers * h;
      int t0, t1;
      bool wl;
      if (G1) {
        const int c0 = it.wb * kCols + w * 32;  // wave w's 32 columns of F: gate tiles t0, t0 + 1, up t1, t1 + 1
        wl = c0 < F;
        t0 = c0 / 16;
        t1 = (F + c0) / 16;
      } else {
        const int h0 = it.wb * 2 * kCols + w * 64;  // wave w's 64 rows of H: tiles t0 .. t0 + 3
        wl = h0 < H;
        t0 = h0 / 16;
        t1 = t0 + 2;
      }
      const bool live = it.live && wl && q < nst;
      const rsrc_t Wr = make_rsrc(pw + (size_t)it.s * Gm.data_slot, live ? wlim : 0u);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t tile = (uint32_t)(((a >> 1) ? t1 : t0) + (a & 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(Wr, (lds_ptr_t)(slot + w * 4096 + a * 1024), 16, wlane,
                                                 live ? tile * (uint32_t)Gm.data_tile + so : 0u, 0, WNT);
      }
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

  constexpr int kTPR = kWaves * 64 / kTM;          // threads per token row
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

  // GEMM2: row info of an item's rows (threads 0..127: token or -1,
  // 128..255: routing weight), fetched early and stored after the barrier
  // that ends the previous item
  const bool fuse = !G1 && sr.rtok != nullptr;
  auto rinf_fetch = [&](const TItem it) -> int {
    const int r = tid & (kTM - 1);
    int v = -1;
    if (fuse && tid < 2 * kTM && it.live && r < it.nvalid)
      v = tid < kTM ? __hip_atomic_load(sr.rtok + it.r0 + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                    : __hip_atomic_load(reinterpret_cast<const int*>(sr.rw) + it.r0 + r, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    return v;
  };
  auto rinf_store = [&](int v) {
    if (!G1 && tid < 2 * kTM) s_rinf[tid] = v;
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

  // The item loop in one copy per half of the waves (GRP = wave / 4), so that
  // each copy's DMA pattern is fixed: the compiler's waits for the weight
  // scales then count the DMA issued after them instead of draining it.
  auto run = [&](auto grpc) {
  constexpr int GRP = decltype(grpc)::value;
  // ---- first item: its token scales, first scale group and first stages
  TItem cur = decode(i0 + lb);
  bool after_epi = false;  // an epilogue's stores are in flight (every item but the first)
  {
    uint32_t v[kXsPer];
    xs_fetch(cur, v);
    xs_store(cur, v);
    rinf_store(rinf_fetch(cur));
  }
  load_scales(cur, 0, scn);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kAhead; ++q) {
    if ((q & 1) == GRP) {
      dma_x(cur, ring(q), q);
      dma_w(cur, ring(q) + kStage, q);
    }
  }
  int slot = 0;  // ring slot of the current stage

  for (int item = i0 + lb; item < i1; item += nper) {
    const TItem nxt = decode(item + nper);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[i][tt] = v4f{0.f, 0.f, 0.f, 0.f};

    // one stage (q of parity P): its issuing waves wait for its DMA, the
    // barrier makes it everyone's (and retires the slot the next DMA
    // refills); the same waves issue stage q + 2 (of this item or, past its
    // end, of the next); every wave computes stage q
    auto stage = [&](int q, auto pc) {
      constexpr int P = decltype(pc)::value;
      constexpr bool iss = GRP == P;
      if constexpr (iss) {
        if (after_epi && q < kAhead)
          asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kEpiStores<G1>) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
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
      if constexpr (iss) {
        uint8_t* const fill = ring(slot == 0 ? kRing - 1 : slot - 1);  // the slot read by stage q - 1
        if (q + kAhead < nst4) {
          dma_x(cur, fill, q + kAhead);
          dma_w(cur, fill + kStage, q + kAhead);
        } else {
          dma_x(nxt, fill, q + kAhead - nst4);
          dma_w(nxt, fill + kStage, q + kAhead - nst4);
        }
      }
      compute(cur.wlive, ring(slot), ring(slot) + kStage, q);
      slot = slot == kRing - 1 ? 0 : slot + 1;
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int q0 = 0; q0 < nst4 - 4; q0 += 4) {
      stage(q0, P0{});
      stage(q0 + 1, P1{});
      stage(q0 + 2, P0{});
      stage(q0 + 3, P1{});
    }
    uint32_t xsn[kXsPer];
    xs_fetch(nxt, xsn);
    const int rinfn = rinf_fetch(nxt);
    stage(nst4 - 4, P0{});
    stage(nst4 - 3, P1{});
    stage(nst4 - 2, P0{});
    stage(nst4 - 1, P1{});

    if (!G1) {
      // ---- GEMM2 epilogue.  Rows of tokens with two or more local pairs (all
      // rows without the fusion): f32 y through a buffer sized to the item's
      // rows (zero-sized for waves past H).  Rows of tokens with exactly one
      // local pair: bf16(fma(w, y, 0)) into their output row, regrouped
      // through LDS so that each lane stores 16 consecutive values.  Every
      // store is issued by every lane (an unused one lands past its buffer),
      // so the count the next stages' waits rely on is exact; the next
      // stages' waits do not drain them.
      const int h0 = cur.wb * 2 * kCols + wave * 64;
      const uint32_t ylim = cur.wlive ? (uint32_t)cur.nvalid * (uint32_t)H * 4u : 0u;
      const rsrc_t Yr = make_rsrc(y + (size_t)cur.r0 * H, ylim);
      const uint32_t olim = (fuse && cur.wlive) ? sr.out_bytes : 0u;
      const rsrc_t Or = make_rsrc(sr.out, olim);
      bare_barrier();  // every wave is done reading the last stage's ring slot
      const uint8_t* tr = ring(slot == 0 ? kRing - 1 : slot - 1) + wave * (16 * kOutPitch);
      const uint32_t trw = lds_addr(tr + l16 * kOutPitch + 8 * g);   // row l16, values 16 i + 4 g ..
      const uint32_t trr = lds_addr(tr + l16 * kOutPitch + 32 * g);  // row l16, values 16 g .. 16 g + 15
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int row = tt * 16 + l16;
        const int tok = s_rinf[row];  // -1: y (no fusion, several local pairs, or past the rows)
        const float wgt = __int_as_float(s_rinf[kTM + row]);
        const uint32_t yo =
            tok < 0 ? ((uint32_t)row * (uint32_t)H + (uint32_t)(cur.wlive ? h0 + 4 * g : 0)) * 4u : ylim;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[i][tt]), Yr, yo + 64u * i, 0, 0);
        v2i o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i].x = (int)((uint32_t)f32_to_bf16(fmaf(wgt, acc[i][tt][0], 0.0f)) |
                         ((uint32_t)f32_to_bf16(fmaf(wgt, acc[i][tt][1], 0.0f)) << 16));
          o[i].y = (int)((uint32_t)f32_to_bf16(fmaf(wgt, acc[i][tt][2], 0.0f)) |
                         ((uint32_t)f32_to_bf16(fmaf(wgt, acc[i][tt][3], 0.0f)) << 16));
        }
        lds_write8_at<0>(trw, o[0]);
        lds_write8_at<32>(trw, o[1]);
        lds_write8_at<64>(trw, o[2]);
        lds_write8_at<96>(trw, o[3]);
        MOE_LGKM_WAIT(0);
        const v4i r0 = lds_read16_at<0>(trr), r1 = lds_read16_at<16>(trr);
        MOE_LGKM_WAIT(0);
        const uint32_t oo = tok >= 0 ? ((uint32_t)tok * (uint32_t)H + (uint32_t)(h0 + 16 * g)) * 2u : olim;
        __builtin_amdgcn_raw_buffer_store_b128(r0, Or, oo, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(r1, Or, oo + 16u, 0, 0);
      }
    } else {
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
        const int c0 = cur.wb * kCols + wave * 32;
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
    }
    after_epi = true;
    bare_barrier();  // every wave is done with this item's token scales, amax and row info
    xs_store(nxt, xsn);
    rinf_store(rinfn);
    MOE_LGKM_WAIT(0);
    cur = nxt;
  }
  };
  if (igrp == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});
}

// Compute units of the current device, looked up once per device.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_num_cus[kMaxDevices];

static int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices) {
    const int n = g_num_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < kMaxDevices) g_num_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool tiled_fits(int H, int F, int P_local) {
  return H / 128 <= kMaxStages && F / 128 <= kMaxStages && kStaticLds + tiled_lds(P_local) <= kTiledLdsMax;
}

// Dynamic LDS above the default limit is opted into per kernel and device,
// once per size (the largest granted so far), under a lock: callers on other
// threads may launch on the same device.
static std::mutex g_lds_mu;

static hipError_t grant_lds(const void* fn, size_t lds, size_t (&granted)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_lds_mu);
  if (dev < 0 || dev >= kMaxDevices || lds > granted[dev]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) granted[dev] = lds;
  }
  return hipSuccess;
}

template <bool G1, int WNT>
static hipError_t run_tiled(const uint8_t* x, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw,
                            const uint8_t* pws, uint8_t* aq, uint8_t* as, float* y, int H, int F, int P_local,
                            SingleRows sr, hipStream_t st) {
  const size_t lds = tiled_lds(P_local);
  static size_t granted[kMaxDevices] = {};  // one table per kernel instantiation
  hipError_t e = grant_lds(reinterpret_cast<const void*>(&k_tiled<G1, WNT>), lds, granted);
  if (e != hipSuccess) return e;
  k_tiled<G1, WNT><<<num_cus() / 8 * 8, kWaves * 64, lds, st>>>(x, xs, offsets, P_local, pw, pws, aq, as, y, H, F, sr);
  return hipGetLastError();
}

hipError_t launch_gemm1_tiled(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                              const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                              bool nt_weights, hipStream_t st) {
  const SingleRows none{nullptr, nullptr, nullptr, 0u};
  return nt_weights ? run_tiled<true, kWeightNtLoads>(xq, xs, offsets, pw1, pw1s, aq, as, nullptr, H, F, P_local, none, st)
                    : run_tiled<true, 0>(xq, xs, offsets, pw1, pw1s, aq, as, nullptr, H, F, P_local, none, st);
}

hipError_t launch_gemm2_tiled(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, SingleRows sr,
                              bool nt_weights, hipStream_t st) {
  return nt_weights ? run_tiled<false, kWeightNtLoads>(aq, as, offsets, pw2, pw2s, nullptr, nullptr, y, H, F, P_local, sr, st)
                    : run_tiled<false, 0>(aq, as, offsets, pw2, pw2s, nullptr, nullptr, y, H, F, P_local, sr, st);
}

}  // namespace moe
