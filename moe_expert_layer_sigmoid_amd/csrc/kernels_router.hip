// Router projection in front of routing: logits[t][e] = sum_k x[t][k] w_gate[e][k]
// with bf16 operands and f32 accumulation, on gfx950's bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  The gate is stored in BF16 [InferenceX PR 3430
// "[AMD][MI35X] 0926 DSV4 sglang mtp agentic", Additional detail section].
//
// A block (8 waves) computes 128 experts x (16 NB) tokens: stages of 128 K
// columns go global -> registers -> LDS, each row's 256 bytes read by 16
// consecutive threads (whole 128-byte lines), double-buffered in LDS with one
// barrier per stage (a bare s_barrier after the block's LDS writes: the
// generic barrier would drain the global loads in flight), the global loads
// of the next three stages in flight while the current one computes.  The
// waves split the tile 4 (experts) x 2 (tokens), or 8 x 1 for a single token
// tile; operands come from LDS in the natural 16x16x32 order (lane 16 g + r:
// row r, columns 8 g + [0, 8) of the 32-column slice), rows
// padded to 272 bytes so that a 16-lane phase of ds_read_b128 hits 16
// distinct bank groups.  The result tile lands as C[row 4 g + i][column r] in
// lane 16 g + r: four consecutive experts of one token, one 16-byte store.
// For few tokens the K range is split over several blocks writing partial
// sums that k_router_reduce adds in split order (a fixed order).

#include <hip/hip_runtime.h>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRouterWaves = 8;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}

constexpr int kRouterDepth = 3;         // stages of global loads in flight

// Staged rows: BK bf16 columns (2 BK bytes) plus 16 bytes of padding, so that
// the 16 rows of a 16-lane ds_read_b128 phase fall on distinct banks (row
// strides of 68 and 36 dwords map 16 rows onto 16 distinct 4-bank groups).
template <int BK>
constexpr int router_row() {
  return 2 * BK + 16;
}

template <int NB, int BM, int BK>
struct RouterSmem {
  uint8_t a[2][BM * router_row<BK>()];
  uint8_t b[2][16 * NB * router_row<BK>()];
};

// NB: token tiles of 16 per block; BM: experts per block; BK: K columns per stage.
template <int NB, int BM, int BK>
__global__ void __launch_bounds__(64 * kRouterWaves)
    k_router_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, float* __restrict__ out, int T,
                  int E, int H, int klen, int gx, int gy, int tiles) {
  constexpr int kRouterBM = BM, kRouterBK = BK, kRouterRow = router_row<BK>();
  constexpr int PR = BK / 8;                                    // 16-byte pieces per staged row
  constexpr int BN = 16 * NB;                                   // tokens per block
  constexpr int NT = 64 * kRouterWaves;                         // threads
  constexpr int WN = NB >= 2 ? 2 : 1;                           // waves along tokens
  constexpr int WM = kRouterWaves / WN;                         // waves along experts
  constexpr int TI = kRouterBM / (16 * WM);                     // expert tiles per wave
  constexpr int TJ = NB / WN;                                   // token tiles per wave
  constexpr int PA = kRouterBM * PR / NT;                       // 16-byte pieces per thread: A
  constexpr int PB = (BN * PR + NT - 1) / NT;                   // and B (the last may be partial)
  static_assert(TI * 16 * WM == BM && PA * NT == BM * PR && NT % PR == 0, "router tile shape");
  __shared__ __align__(16) RouterSmem<NB, BM, BK> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;
  // XCD-aware tile order: the hardware deals blocks round-robin to the 8 XCDs,
  // so block b runs on XCD b % 8; give each XCD a contiguous range of tiles
  // (experts fastest), so the expert blocks that share a token slab share
  // that XCD's L2.
  const int per = (tiles + kXcds - 1) / kXcds;
  const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= tiles) return;  // whole block
  const int bx = tile % gx, by = (tile / gx) % gy, bz = tile / (gx * gy);
  const int e0 = bx * kRouterBM, t0 = by * BN, kb = bz * klen;
  const int stages = (min(H, kb + klen) - kb) / kRouterBK;  // H, klen: multiples of 128

  // this thread's pieces: piece index i = tid + NT q -> row i / PR, bytes 16 (i % PR)
  const int pcol = tid % PR;
  const v4i* ga[PA];
  const v4i* gb[PB];
#pragma unroll
  for (int q = 0; q < PA; ++q) {
    const int row = min(e0 + (tid + NT * q) / PR, E - 1);  // rows past E: a valid row, results not stored
    ga[q] = reinterpret_cast<const v4i*>(wg + (size_t)row * H + kb) + pcol;
  }
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int row = min(t0 + min((tid + NT * q) / PR, BN - 1), T - 1);
    gb[q] = reinterpret_cast<const v4i*>(x + (size_t)row * H + kb) + pcol;
  }
  // kRouterDepth register sets of staged pieces: the global loads of stage
  // s + kRouterDepth are issued while stage s computes (set (s + 1) % depth
  // is refilled right after its pieces went to LDS).
  constexpr int D = kRouterDepth;
  v4i ra[D][PA], rb[D][PB];
  auto fetch = [&](int set, int st) {
    const int o = min(st, stages - 1) * (kRouterBK / 8);  // past the end: an unused re-read
#pragma unroll
    for (int q = 0; q < PA; ++q) ra[set][q] = ga[q][o];
#pragma unroll
    for (int q = 0; q < PB; ++q) rb[set][q] = gb[q][o];
  };
  auto stash = [&](int set, int buf) {
#pragma unroll
    for (int q = 0; q < PA; ++q)
      *reinterpret_cast<v4i*>(sm.a[buf] + ((tid + NT * q) / PR) * kRouterRow + pcol * 16) = ra[set][q];
#pragma unroll
    for (int q = 0; q < PB; ++q)
      if (tid + NT * q < BN * PR)
        *reinterpret_cast<v4i*>(sm.b[buf] + ((tid + NT * q) / PR) * kRouterRow + pcol * 16) = rb[set][q];
  };

  v4f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int m = 0; m < kRouterBK / 32; ++m) {
      const int cb = m * 64 + g * 16;  // bytes: columns 32 m + 8 g
      v4i a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const v4i*>(sm.a[buf] + (16 * (TI * wm + i) + r) * kRouterRow + cb);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const v4i*>(sm.b[buf] + (16 * (TJ * wn + j) + r) * kRouterRow + cb);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d) fetch(d, d);
  stash(0, 0);
  fetch(0, D);
  __syncthreads();
  for (int s0 = 0; s0 < stages; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s0 + d;  // uniform
      const int nxt = (d + 1) % D;
      if (st < stages) compute(st & 1);
      __builtin_amdgcn_sched_barrier(0);
      // stage st + 1 from its set into the other buffer (read last before the
      // previous barrier), then refill that set with stage st + 1 + D
      if (st + 1 < stages) stash(nxt, (st + 1) & 1);
      fetch(nxt, st + 1 + D);
      __builtin_amdgcn_sched_barrier(0);
      // a bare barrier: the generic one would also drain the global loads in flight
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  }

  float* o = out + (size_t)bz * T * E;
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int t = t0 + 16 * (TJ * wn + j) + r;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int e = e0 + 16 * (TI * wm + i) + 4 * g;
      float* p = o + (size_t)t * E + e;
      if (vec && e + 3 < E) {
        *reinterpret_cast<v4f*>(p) = acc[i][j];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < E) p[q] = acc[i][j][q];
      }
    }
  }
}

// logits = sum over s of part[s] (s ascending), n = T * E values; 16-byte
// accesses when every split starts 16-byte aligned (n % 4 == 0).  S is at
// most SMAX (an instantiated bound: the loads of all splits are in flight at
// once, so the bound is kept near S).
template <int SMAX>
__global__ void __launch_bounds__(256) k_router_reduce(const float* __restrict__ part, float* __restrict__ logits,
                                                       size_t n, int S) {
  const size_t n4 = (n & 3) == 0 ? n / 4 : 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    // every split's value in flight at once, then added in split order
    v4f v[SMAX];
#pragma unroll
    for (int z = 0; z < SMAX; ++z)
      v[z] = z < S ? reinterpret_cast<const v4f*>(part + (size_t)z * n)[i] : v4f{0.f, 0.f, 0.f, 0.f};
    v4f s = v[0];
#pragma unroll
    for (int z = 1; z < SMAX; ++z)
      if (z < S) s += v[z];
    reinterpret_cast<v4f*>(logits)[i] = s;
  }
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float s = part[i];
    for (int z = 1; z < S; ++z) s += part[(size_t)z * n + i];
    logits[i] = s;
  }
}

}  // namespace

RouterPlan router_plan(int T, int E, int H) {
  RouterPlan p;
  p.ni = T >= kRouterHugeT ? 16 : (T >= kRouterLargeT ? 8 : (T >= kRouterMidT ? 4 : 1));  // token tiles per block
  p.bm = p.ni == 16 ? kRouterWideBM : 128;
  p.gx = (E + p.bm - 1) / p.bm;
  p.gy = (T + 16 * p.ni - 1) / (16 * p.ni);
  const int blocks = p.gx * p.gy;
  int S = blocks >= kRouterMinBlocks ? 1 : (kRouterMinBlocks + blocks - 1) / blocks;
  const int kmax = H / 128;  // at least 128 columns of K per split
  S = S < 1 ? 1 : (S > kRouterMaxSplits ? kRouterMaxSplits : S);
  if (S > kmax) S = kmax;
  p.klen = (H / 128 + S - 1) / S * 128;
  p.splits = (H + p.klen - 1) / p.klen;
  return p;
}

size_t router_partial_bytes(int T_max, int E, int H) {
  // splits <= ceil(kRouterMinBlocks / blocks) and blocks >= gx * T / (16 ni), so
  // splits * T <= kRouterMinBlocks * 16 ni / gx + T for every T <= T_max; the
  // larger bound of the two tile heights (ni <= 8 with 128 experts, ni = 16 with
  // the wide tiles)
  (void)H;
  const size_t g128 = (size_t)(E + 127) / 128, gw = (size_t)(E + kRouterWideBM - 1) / kRouterWideBM;
  const size_t a = (size_t)kRouterMinBlocks * 16 * 8 / g128, b = (size_t)kRouterMinBlocks * 16 * 16 / gw;
  const size_t tok = (a > b ? a : b) + 1 + (size_t)T_max;
  return tok * E * sizeof(float);
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wg, float* logits, float* partial, int T, int E, int H,
                         hipStream_t st) {
  const RouterPlan p = router_plan(T, E, H);
  float* dst = p.splits > 1 ? partial : logits;
  const int tiles = p.gx * p.gy * p.splits;
  dim3 grid((tiles + kXcds - 1) / kXcds * kXcds), block(64 * kRouterWaves);
  if (p.ni == 16)
    hipLaunchKernelGGL((k_router_gemm<16, kRouterWideBM, 64>), grid, block, 0, st, x, wg, dst, T, E, H, p.klen, p.gx,
                       p.gy, tiles);
  else if (p.ni == 8)
    hipLaunchKernelGGL((k_router_gemm<8, 128, 128>), grid, block, 0, st, x, wg, dst, T, E, H, p.klen, p.gx, p.gy,
                       tiles);
  else if (p.ni == 4)
    hipLaunchKernelGGL((k_router_gemm<4, 128, 128>), grid, block, 0, st, x, wg, dst, T, E, H, p.klen, p.gx, p.gy,
                       tiles);
  else
    hipLaunchKernelGGL((k_router_gemm<1, 128, 128>), grid, block, 0, st, x, wg, dst, T, E, H, p.klen, p.gx, p.gy,
                       tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t n = (size_t)T * E;
  const size_t want = (n / 4 + 255) / 256 + 1;
  const int blocks = (int)(want < 2048 ? want : 2048);
  static_assert(kRouterMaxSplits <= 16, "reduce instantiations");
  if (p.splits <= 4)
    hipLaunchKernelGGL(k_router_reduce<4>, dim3(blocks), dim3(256), 0, st, partial, logits, n, p.splits);
  else if (p.splits <= 8)
    hipLaunchKernelGGL(k_router_reduce<8>, dim3(blocks), dim3(256), 0, st, partial, logits, n, p.splits);
  else
    hipLaunchKernelGGL(k_router_reduce<16>, dim3(blocks), dim3(256), 0, st, partial, logits, n, p.splits);
  return hipGetLastError();
}

}  // namespace moe
