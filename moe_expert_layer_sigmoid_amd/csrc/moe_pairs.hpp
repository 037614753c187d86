// Pair listing of the pair-indexed (small-input) path, shared by the a8w4
// streaming GEMMs and the a16w4 GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

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

__device__ __forceinline__ int slot_pairs(const int32_t* __restrict__ phys, int np, int q, int* list, int cap, int (*s_cnt)[4]) {
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

// The local slots [0, P_local) that hold a pair of phys[0, np) (slot ids
// from p0 on) as a bitmap in LDS, bits[0, ceil(P_local / 32)); returns how
// many (the same in every thread).  P_local <= 32 * kTouchedWords.
constexpr int kTouchedWords = 32;
__device__ __forceinline__ int touched_bits(const int32_t* __restrict__ phys, int np, int p0, int P_local,
                                            uint32_t* bits) {
  const int nw = (P_local + 31) >> 5;
  for (int i = threadIdx.x; i < nw; i += blockDim.x) bits[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    const int p = phys[i] - p0;
    if (p >= 0 && p < P_local) atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  int n = 0;
  for (int w = 0; w < nw; ++w) n += __popc(bits[w]);
  return n;
}
// The slot of set bit number j (ascending; 0 <= j < the number set).
__device__ __forceinline__ int nth_bit(const uint32_t* bits, int P_local, int j) {
  const int nw = (P_local + 31) >> 5;
  for (int w = 0; w < nw; ++w) {
    uint32_t b = bits[w];
    const int c = __popc(b);
    if (j < c) {
      for (; j > 0; --j) b &= b - 1u;
      return w * 32 + __builtin_ctz(b);
    }
    j -= c;
  }
  return -1;
}
// The number of set bits below slot i.
__device__ __forceinline__ int bit_rank(const uint32_t* bits, int i) {
  int r = 0;
  for (int w = 0; w < (i >> 5); ++w) r += __popc(bits[w]);
  return r + __popc(bits[i >> 5] & ((1u << (i & 31)) - 1u));
}

}  // namespace moe
