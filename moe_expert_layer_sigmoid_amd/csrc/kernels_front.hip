// Routing, EPLB remap + load recording, bucketing, activation quantisation /
// dispatch, and the weighted combine: the integer and elementwise steps of the
// fused MoE layer, as gfx950 kernels.
//
// Pages: the operator runs quant, dispatch, GEMM1, GEMM2 and combine [sglang
// PR 47065 "Use the aiter MegaMoE small- and large-input paths", intro]; top-6
// routing [sglang PR 35619 "Aiter/FlyDSL MegaMoEv2 backend for DeepSeek-V4",
// "Four settings that silently break it"]; fused EPLB remap + recording in
// prefill [same page, Summary]; per-physical-expert counts behind EPLB
// [FlyDSL issue 978, Data-quality gates].

#include <climits>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// a1 route.  Each of the k rounds takes the argmax of the token's logits
// (largest logit, lower id on ties) and retires the winner's entry (set to
// -inf; inputs are finite).  Weights: sigmoid of the chosen logits over their
// sum, in f32, the sum being a DPP tree over the lanes j < k that hold choice j.
//  - route64, one wavefront per token (the fused small-M front, where the
//    chain's latency counts): lane l holds logits l, l + 64, ...; a round is a
//    scan of the lane's own entries, a DPP reduction inside each 16-lane row
//    and a scalar pick among the four row winners (read with readlane).
//  - route16, one 16-lane row per token, four tokens per wavefront (the
//    standalone routing pass over many tokens, where throughput counts):
//    lane l of the row holds logits l, l + 16, ...; the DPP reduction inside
//    the row leaves the winner in every lane, with no cross-row step.  On the
//    prefill share of 65,536 tokens (384 experts, top-6) it took about 1 %
//    off the forward; in the fused front its longer per-lane scan cost
//    1-2 us at one token.
// Both give the same choices and weights bit for bit (the same comparisons,
// and the weights' sum in the same order, lane 0's tree).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
constexpr int kRor8 = 0x128, kRor4 = 0x124, kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// (bv, bi) <- the better of itself and its DPP partner's.
template <int CTRL>
__device__ __forceinline__ void take_better(float& bv, int& bi) {
  const float ov = dppf<CTRL>(bv);
  const int oi = dpp<CTRL>(bi);
  const bool take = better(ov, oi, bv, bi);
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

template <int CTRL>
__device__ __forceinline__ float add_partner(float v) {
  return v + dppf<CTRL>(v);
}

// Route one token per wavefront (`row`: its logits).  Lane j < k returns
// choice j and its weight.
template <int EPL>
__device__ __forceinline__ void route64(const float* __restrict__ row, int E, int k, int lane, int& my_id,
                                        float& my_w) {
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  my_id = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int i = 1; i < EPL; ++i) {
      const bool t = v[i] > bv;  // ascending ids: strict > keeps the lower id
      bv = t ? v[i] : bv;
      bi = t ? lane + 64 * i : bi;
    }
    take_better<kRor8>(bv, bi);
    take_better<kRor4>(bv, bi);
    take_better<kQuadSwap2>(bv, bi);
    take_better<kQuadSwap1>(bv, bi);
    float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int si = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
      const int ri = __builtin_amdgcn_readlane(bi, 16 * r);
      if (better(rv, ri, sv, si)) {
        sv = rv;
        si = ri;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = (lane + 64 * i == si) ? -INFINITY : v[i];
    if (lane == j) {
      my_id = si;
      my_l = sv;
    }
  }
  const float s = lane < k ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
  float sum = add_partner<kRor8>(s);
  sum = add_partner<kRor4>(sum);
  sum = add_partner<kQuadSwap2>(sum);
  sum = add_partner<kQuadSwap1>(sum);
  sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), 0));
  my_w = s / sum;
}

// Route the token of this lane's 16-lane row (`row`: its logits; EPL logits
// per lane).  Lane l16 < k of the row returns choice l16 and its weight; the
// weights' sum is the row's DPP tree as its lane 0 adds it (the other lanes
// add in other orders), so every choice of the token divides by one value.
template <int EPL>
__device__ __forceinline__ void route16(const float* __restrict__ row, int E, int k, int l16, int& my_id,
                                        float& my_w) {
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = l16 + 16 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  my_id = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = v[0];
    int bi = l16;
#pragma unroll
    for (int i = 1; i < EPL; ++i) {
      const bool t = v[i] > bv;  // ascending ids: strict > keeps the lower id
      bv = t ? v[i] : bv;
      bi = t ? l16 + 16 * i : bi;
    }
    take_better<kRor8>(bv, bi);
    take_better<kRor4>(bv, bi);
    take_better<kQuadSwap2>(bv, bi);
    take_better<kQuadSwap1>(bv, bi);
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = (l16 + 16 * i == bi) ? -INFINITY : v[i];
    if (l16 == j) {
      my_id = bi;
      my_l = bv;
    }
  }
  const float s = l16 < k ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
  float sum = add_partner<kRor8>(s);
  sum = add_partner<kRor4>(sum);
  sum = add_partner<kQuadSwap2>(sum);
  sum = add_partner<kQuadSwap1>(sum);
  sum = __shfl(sum, (int)(threadIdx.x & 63) & ~15);
  my_w = s / sum;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
  const int l16 = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (t >= T) return;  // uniform over the token's 16-lane row
  int id;
  float wt;
  route16<4 * EPL>(logits + (size_t)t * E, E, k, l16, id, wt);  // EPL: logits per lane of 64
  if (l16 < k) {
    ids[(size_t)t * k + l16] = id;
    w[(size_t)t * k + l16] = wt;
  }
}

// Logits per lane, rounded up to an instantiated size (E <= 1024).
static int route_epl(int E) {
  const int e = (E + 63) / 64;
  if (e <= 1) return 1;
  if (e <= 2) return 2;
  if (e <= 4) return 4;
  if (e <= 6) return 6;
  if (e <= 8) return 8;
  if (e <= 12) return 12;
  return 16;
}

#define MOE_ROUTE_CASES(X) X(1) X(2) X(4) X(6) X(8) X(12) X(16)

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const unsigned nb = (unsigned)((T + 15) / 16);
  switch (route_epl(E)) {
#define X(N) \
  case N: k_route<N><<<nb, 256, 0, st>>>(logits, T, E, k, ids, w); break;
    MOE_ROUTE_CASES(X)
#undef X
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2 + a3 (part 1): per chunk of 64 tokens, optionally remap logical -> physical
// expert, then count.  One wavefront walks the chunk's pairs in (t, j) order,
// 64 at a time: a pair's rank is the count of its slot before the group (an
// LDS histogram) plus the lanes below it with the same slot (a ballot per
// distinct local slot of the group), after which the group's pairs add
// themselves to the histogram.
// The histogram then gives the chunk's counts per slot.  Both results are
// deterministic: the order of the adds only matters for their sum.
// (Counting every slot against every pair, per thread, took 7 us of LDS
// broadcasts per chunk and the ranks 12 us more.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_count(int T, int k, const int32_t* __restrict__ ids,
                                               const int32_t* __restrict__ rep_count,
                                               const int32_t* __restrict__ rep_slots, int R_max,
                                               uint32_t token_id_base, int32_t* __restrict__ phys, int do_remap,
                                               int P_total, int p0, int P_local, int32_t* __restrict__ partial,
                                               int32_t* __restrict__ rank) {
  __shared__ int4 s_phys4[kChunkTokens * 16 / 4];
  __shared__ int s_hist[1024];  // P_total <= 1024
  int* s_phys = reinterpret_cast<int*>(s_phys4);
  const int c = blockIdx.x;
  const int t0 = c * kChunkTokens;
  const int nt = min(kChunkTokens, T - t0);
  const int np = nt * k;
  const int np4 = (np + 3) / 4;
  const size_t pr0 = (size_t)t0 * k;
  for (int i = threadIdx.x; i < np4 * 4; i += blockDim.x) {
    int p = -1;  // padding never matches a slot
    if (i < np) {
      if (do_remap) {
        const int e = ids[pr0 + i];
        const uint32_t h = fmix32(token_id_base + (uint32_t)(t0 + i / k));
        p = rep_slots[(size_t)e * R_max + replica(h, rep_count[e], R_max)];
        phys[pr0 + i] = p;
      } else {
        p = phys[pr0 + i];
      }
    }
    s_phys[i] = p;
  }
  for (int q = threadIdx.x; q < P_total; q += blockDim.x) s_hist[q] = 0;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int i0 = 0; i0 < np; i0 += 64) {
      const int i = i0 + lane;
      const int q = i < np ? s_phys[i] : -1;
      const bool inb = q >= 0 && q < P_total;  // slots outside the table count nowhere
      int r = inb ? s_hist[q] : 0;
      if (rank) {
        // the lower lanes with the same slot, for the local pairs only: one
        // round per distinct local slot of the group (its lanes found by
        // ballot), not one per lane
        const bool loc = i < np && q >= p0 && q < p0 + P_local;
        uint64_t pending = __ballot(loc);
        while (pending) {  // wave-uniform
          const int lead = __builtin_ctzll(pending);
          const int qv = __builtin_amdgcn_readlane(q, lead);
          const uint64_t m = __ballot(q == qv);
          if (q == qv) r += __popcll(m & ((1ull << lane) - 1ull));
          pending &= ~m;
        }
        if (loc) rank[pr0 + i] = r;
      }
      // every lane has read its count before any adds (one wavefront: LDS
      // operations run in order)
      if (inb) atomicAdd(&s_hist[q], 1);
    }
  }
  __syncthreads();
  if (partial)
    for (int q = threadIdx.x; q < P_total; q += blockDim.x) partial[(size_t)c * P_total + q] = s_hist[q];
}

hipError_t launch_count(int T, int k, const int32_t* ids, const int32_t* rep_count, const int32_t* rep_slots,
                        int R_max, uint32_t token_id_base, int32_t* phys, bool do_remap, int P_total, int p0,
                        int P_local, int32_t* partial, int32_t* rank, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (P_total > 1024) return hipErrorInvalidValue;  // the kernel's LDS histogram
  int nch = (T + kChunkTokens - 1) / kChunkTokens;
  k_count<<<nch, 256, 0, st>>>(T, k, ids, rep_count, rep_slots, R_max, token_id_base, phys, do_remap ? 1 : 0,
                               P_total, p0, P_local, partial, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2 / a3 (part 2): blocks of 1024 threads sum the chunk partials.  Block 0,
// local slots: counts, exclusive-scan offsets, and per-(chunk, slot) base
// rows, the work split as (slot, chunk-range) so the serial part per thread
// is nch / NG loads.  Blocks 1.., all slots: load_hist += totals, 64 slots
// per block, each slot's chunks split over 16 threads (integer sums: the
// result does not depend on the split).  The loops over chunks keep up to
// kScanBatch independent loads in flight (one load per step waited for each
// line in turn).
// ---------------------------------------------------------------------------
constexpr int kHistSlotsPerBlock = 64;
constexpr int kScanBatch = 16;  // chunk loads a thread keeps in flight
__global__ __launch_bounds__(1024) void k_scan(int nch, int P_total, int p0, int P_local,
                                               const int32_t* __restrict__ partial, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ base,
                                               int32_t* __restrict__ load_hist) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[1024];
  const int tid = threadIdx.x;
  if (counts && blockIdx.x == 0) {
    // NG thread groups per local slot; P_local <= 1024
    int NG = 1024 / P_local;
    if (NG > nch) NG = nch;
    if (NG < 1) NG = 1;
    const int s = tid % P_local, g = tid / P_local;
    const bool act = g < NG;
    const int per = (nch + NG - 1) / NG;
    const int c0 = g * per, c1 = min(nch, c0 + per);
    int sum = 0;
    if (act)
      for (int c = c0; c < c1; c += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? partial[(size_t)(c + u) * P_total + p0 + s] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) sum += v[u];
      }
    if (act) s_part[g * P_local + s] = sum;
    __syncthreads();
    if (tid < P_local) {  // exclusive prefix over groups, total per slot
      int run = 0;
      for (int gg = 0; gg < NG; ++gg) {
        int v = s_part[gg * P_local + tid];
        s_part[gg * P_local + tid] = run;
        run += v;
      }
      s_tot[tid] = run;
    }
    __syncthreads();
    // exclusive scan of slot totals (Hillis-Steele over P_local <= 1024)
    int v = tid < P_local ? s_tot[tid] : 0;
    for (int off = 1; off < 1024; off <<= 1) {
      __syncthreads();
      int o = (tid >= off && tid < P_local) ? s_tot[tid - off] : 0;
      __syncthreads();
      if (tid < P_local) s_tot[tid] += o;
    }
    __syncthreads();
    if (tid < P_local) {
      counts[tid] = v;
      offsets[tid] = s_tot[tid] - v;
      if (tid == P_local - 1) offsets[P_local] = s_tot[tid];
    }
    if (act) {
      // offsets[s] (exclusive prefix of slot totals) + counts of earlier chunk groups
      int run = (s > 0 ? s_tot[s - 1] : 0) + s_part[g * P_local + s];
      for (int c = c0; c < c1; c += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? partial[(size_t)(c + u) * P_total + p0 + s] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
          if (c + u < c1) base[(size_t)(c + u) * P_local + s] = run;
          run += v[u];
        }
      }
    }
  }
  if (load_hist && blockIdx.x > 0) {
    constexpr int NG = 1024 / kHistSlotsPerBlock;
    const int q = ((int)blockIdx.x - 1) * kHistSlotsPerBlock + tid % kHistSlotsPerBlock, g = tid / kHistSlotsPerBlock;
    int sum = 0;
    if (q < P_total)
      for (int c = g; c < nch; c += kScanBatch * NG) {
        int v[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
          v[u] = c + u * NG < nch ? partial[(size_t)(c + u * NG) * P_total + q] : 0;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) sum += v[u];
      }
    s_part[tid] = sum;
    __syncthreads();
    if (tid < kHistSlotsPerBlock && q < P_total) {
      int tot = 0;
      for (int gg = 0; gg < NG; ++gg) tot += s_part[gg * kHistSlotsPerBlock + tid];
      load_hist[q] += tot;
    }
  }
}

hipError_t launch_scan(int nch, int P_total, int p0, int P_local, const int32_t* partial, int32_t* counts,
                       int32_t* offsets, int32_t* base, int32_t* load_hist, hipStream_t st) {
  const unsigned nhist = load_hist ? (unsigned)((P_total + kHistSlotsPerBlock - 1) / kHistSlotsPerBlock) : 0u;
  k_scan<<<1 + nhist, 1024, 0, st>>>(nch, P_total, p0, P_local, partial, counts, offsets, base, load_hist);
  return hipGetLastError();
}

// a4 arithmetic for one lane's 8 columns of a 128-column block (16 lanes per
// block), on eight bf16 values already loaded (zeros for columns past H):
// e = smallest integer with amax <= 448 * 2^e over the block, codes
// RNE e4m3fn(x * 2^-e).
__device__ __forceinline__ int quant8_raw(const uint4 raw, uint2& q) {
  float v[8];
  const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(wd[i] << 16);
    v[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) am = fmaxf(am, __shfl_xor(am, off));
  const int e = scale_exp(am);
  q.x = pack4_fp8(ldexpf(v[0], -e), ldexpf(v[1], -e), ldexpf(v[2], -e), ldexpf(v[3], -e));
  q.y = pack4_fp8(ldexpf(v[4], -e), ldexpf(v[5], -e), ldexpf(v[6], -e), ldexpf(v[7], -e));
  return e;
}

// The same, loading the lane's 8 columns (`ok` false: zeros).
__device__ __forceinline__ int quant8(const uint16_t* __restrict__ src, bool ok, uint2& q) {
  return quant8_raw(ok ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0), q);
}

// ---------------------------------------------------------------------------
// a3 (part 3) + a4: one wavefront per (token, kQC 512-column chunks).  Lanes
// j < k resolve the row of pair (t, j) (base of its chunk and slot + rank;
// the wave of chunk 0 also writes the row maps); the wave then loads all its
// columns at once (one 16-byte load per lane and chunk) and quantises each
// 128-column block: 16 lanes per block, 8 bf16 per lane; the block amax gives
// the e8m0 exponent, codes are RNE e4m3fn of x * 2^-e; the same bytes go to
// every local row of the token.  Tokens without a local pair read nothing.
// ---------------------------------------------------------------------------
constexpr int kQC = 4;  // 512-column chunks per wavefront (quantise)
constexpr int kCC = 4;  // 512-column chunks per wavefront (combine; 2 and 7 measured the same)

__global__ __launch_bounds__(256) void k_quant(int T, int H, int k, const uint16_t* __restrict__ x,
                                               const int32_t* __restrict__ phys, int p0, int P_local,
                                               const int32_t* __restrict__ base, const int32_t* __restrict__ rank,
                                               uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                               int32_t* __restrict__ row_of_pair, int32_t* __restrict__ pair_of_row,
                                               const float* __restrict__ w, int32_t* __restrict__ rtok,
                                               float* __restrict__ rw) {
  const int lane = threadIdx.x & 63;
  const int nb = H / kActBlock;
  const int ng = (H + 512 * kQC - 1) / (512 * kQC);
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = wid / ng, grp = wid - t * ng;
  if (t >= T) return;  // wave-uniform
  int myrow = -1;
  if (lane < k) {
    const size_t pr = (size_t)t * k + lane;
    const int p = phys[pr];
    if (p >= p0 && p < p0 + P_local) {
      const int s = p - p0;
      myrow = base[(size_t)(t / kChunkTokens) * P_local + s] + rank[pr];
      if (grp == 0) pair_of_row[myrow] = (int32_t)pr;
    }
    if (grp == 0) row_of_pair[pr] = myrow;
  }
  if (rtok && grp == 0) {  // the single-pair row map (as k_single_rows)
    const int nloc = __popcll(__ballot(myrow >= 0));
    if (myrow >= 0) {
      rtok[myrow] = nloc == 1 ? t : -1;
      rw[myrow] = w[(size_t)t * k + lane];
    }
  }
  int rows[16];
  bool any = false;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int r = __shfl(myrow, j);
    rows[j] = j < k ? r : -1;
    any |= rows[j] >= 0;
  }
  if (!any) return;
  const int sub = lane & 15;  // 8 columns each
  uint4 raw[kQC];
  bool ok[kQC];
#pragma unroll
  for (int c = 0; c < kQC; ++c) {  // all loads first
    const int b = (grp * kQC + c) * 4 + (lane >> 4);
    ok[c] = b < nb;
    raw[c] = ok[c] ? *reinterpret_cast<const uint4*>(x + (size_t)t * H + b * kActBlock + sub * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < kQC; ++c) {
    const int b = (grp * kQC + c) * 4 + (lane >> 4);
    uint2 q;
    const int e = quant8_raw(raw[c], q);
    if (ok[c]) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (rows[j] < 0) continue;  // wave-uniform
        const size_t r = (size_t)rows[j];
        *reinterpret_cast<uint2*>(xq + r * H + b * kActBlock + sub * 8) = q;
        if (sub == 0) xs[r * nb + b] = (uint8_t)(e + 127);
      }
    }
  }
}

hipError_t launch_quant(int T, int H, int k, const uint16_t* x, const int32_t* phys, int p0, int P_local,
                        const int32_t* base, const int32_t* rank, uint8_t* xq, uint8_t* xs, int32_t* row_of_pair,
                        int32_t* pair_of_row, hipStream_t st, const float* w, int32_t* rtok, float* rw) {
  if (T == 0) return hipSuccess;
  const int ng = (H + 512 * kQC - 1) / (512 * kQC);
  const long waves = (long)T * ng;
  k_quant<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(T, H, k, x, phys, p0, P_local, base, rank, xq, xs,
                                                       row_of_pair, pair_of_row, w, rtok, rw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a7, tokens with exactly one local pair: their output row is one term,
// bf16(fma(w, y, 0)), which the bucketed GEMM2 kernels write themselves from
// their accumulators (the combine then skips those tokens, and their f32 y
// row is never written or read).  One thread per token: rtok[row] = t for the
// row of such a token, -1 for the rows of tokens with two or more local
// pairs; rw[row] = the pair's routing weight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_single_rows(int T, int k, const int32_t* __restrict__ row_of_pair,
                                                     const float* __restrict__ w, int32_t* __restrict__ rtok,
                                                     float* __restrict__ rw) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* rp = row_of_pair + (size_t)t * k;
  int n = 0;
  for (int j = 0; j < k; ++j) n += rp[j] >= 0;
  for (int j = 0; j < k; ++j) {
    const int r = rp[j];
    if (r >= 0) {
      rtok[r] = n == 1 ? t : -1;
      rw[r] = w[(size_t)t * k + j];
    }
  }
}

hipError_t launch_single_rows(int T, int k, const int32_t* row_of_pair, const float* w, int32_t* rtok, float* rw,
                              hipStream_t st) {
  if (T == 0) return hipSuccess;
  k_single_rows<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(T, k, row_of_pair, w, rtok, rw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a7 combine: one wavefront per (token, kCC 512-column chunks), 8 columns per
// lane and chunk; out[t] = sum over local j ascending of w[t][j] *
// y[row(t, j)] (f32 fma chain), rounded to bf16 (nearest even).  A row's
// loads for all the wave's chunks are issued together.  With skip_single,
// tokens with exactly one local pair are left alone (GEMM2 wrote them).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_pair,
                                                 const float* __restrict__ w, uint16_t* __restrict__ out,
                                                 int skip_single) {
  const int lane = threadIdx.x & 63;
  const int ng = (H + 512 * kCC - 1) / (512 * kCC);
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = wid / ng, grp = wid - t * ng;
  if (t >= T) return;
  int myrow = -1;
  float myw = 0.0f;
  if (lane < k) {
    myrow = row_of_pair[(size_t)t * k + lane];
    myw = w[(size_t)t * k + lane];
  }
  int rows[16];
  float ws[16];
  int nloc = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int r = __shfl(myrow, j);
    ws[j] = __shfl(myw, j);
    rows[j] = j < k ? r : -1;
    nloc += rows[j] >= 0;
  }
  if (skip_single && nloc == 1) return;  // wave-uniform: GEMM2 wrote this row
  float a[kCC][8];
#pragma unroll
  for (int c = 0; c < kCC; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[c][i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (rows[j] < 0) continue;  // wave-uniform
    float4 v[kCC][2];
#pragma unroll
    for (int c = 0; c < kCC; ++c) {
      const int h = (grp * kCC + c) * 512 + lane * 8;
      const float* yr = y + (size_t)rows[j] * H + h;
      v[c][0] = h < H ? *reinterpret_cast<const float4*>(yr) : make_float4(0.f, 0.f, 0.f, 0.f);
      v[c][1] = h < H ? *reinterpret_cast<const float4*>(yr + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int c = 0; c < kCC; ++c) {
      a[c][0] = fmaf(ws[j], v[c][0].x, a[c][0]);
      a[c][1] = fmaf(ws[j], v[c][0].y, a[c][1]);
      a[c][2] = fmaf(ws[j], v[c][0].z, a[c][2]);
      a[c][3] = fmaf(ws[j], v[c][0].w, a[c][3]);
      a[c][4] = fmaf(ws[j], v[c][1].x, a[c][4]);
      a[c][5] = fmaf(ws[j], v[c][1].y, a[c][5]);
      a[c][6] = fmaf(ws[j], v[c][1].z, a[c][6]);
      a[c][7] = fmaf(ws[j], v[c][1].w, a[c][7]);
    }
  }
#pragma unroll
  for (int c = 0; c < kCC; ++c) {
    const int h = (grp * kCC + c) * 512 + lane * 8;
    if (h >= H) continue;
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(a[c][0]) | ((uint32_t)f32_to_bf16(a[c][1]) << 16);
    o.y = (uint32_t)f32_to_bf16(a[c][2]) | ((uint32_t)f32_to_bf16(a[c][3]) << 16);
    o.z = (uint32_t)f32_to_bf16(a[c][4]) | ((uint32_t)f32_to_bf16(a[c][5]) << 16);
    o.w = (uint32_t)f32_to_bf16(a[c][6]) | ((uint32_t)f32_to_bf16(a[c][7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + h) = o;
  }
}

hipError_t launch_combine(int T, int H, int k, const float* y, const int32_t* row_of_pair, const float* w,
                          uint16_t* out, bool skip_single, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const long waves = (long)T * ((H + 512 * kCC - 1) / (512 * kCC));
  k_combine<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(T, H, k, y, row_of_pair, w, out, skip_single ? 1 : 0);
  return hipGetLastError();
}

// ===========================================================================
// Small-M path front and back ends.  The small-input path keeps (token, j)
// pair order instead of bucket rows: the GEMM blocks list their slot's pairs
// themselves, so no scan or permute runs between routing and GEMM1.
// ===========================================================================

// a1 + a2 + a4 in one launch.  Blocks [0, nr) route 16 tokens each (one per
// wavefront), remap them and count the chunk's pairs per physical slot into
// partial[chunk][P_total]; the replica tables are staged in LDS while the
// logits load when they fit.  Blocks [nr, ...) quantise every token (one
// wavefront per token and 512 columns) into per-token rows xq_tok / xs_tok.
constexpr int kFrontThreads = 1024;
constexpr int kRepLds = 4096;  // replica-table entries staged in LDS

//
// With a device token count (t_dev != NULL) the grid covers the capacity T
// and only the first min(*t_dev, T) tokens are valid: the pairs of the other
// tokens get phys = -1 (no slot), so the GEMMs list none of them, the combine
// writes +0 rows for them and the load record skips them.
template <int EPL>
__global__ __launch_bounds__(kFrontThreads) void k_front(
    int T, int E, int k, int H, const float* __restrict__ logits, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ rep_count, const int32_t* __restrict__ rep_slots, int R_max,
    uint32_t token_id_base, int P_total, int nr, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ phys, int32_t* __restrict__ partial, uint8_t* __restrict__ xq_tok,
    uint8_t* __restrict__ xs_tok, const int32_t* __restrict__ t_dev, int32_t* __restrict__ zero, int nzero) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Tcap = T;
  if (t_dev) T = __builtin_amdgcn_readfirstlane(min(max(*t_dev, 0), Tcap));
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += kFrontThreads) zero[i] = 0;
  if ((int)blockIdx.x < nr) {
    __shared__ int s_rc[1024];
    __shared__ int s_rs[kRepLds];
    __shared__ int s_phys[16 * 16];
    const bool lds_tab = E * R_max <= kRepLds;
    for (int i = threadIdx.x; i < E; i += kFrontThreads) s_rc[i] = rep_count[i];
    if (lds_tab)
      for (int i = threadIdx.x; i < E * R_max; i += kFrontThreads) s_rs[i] = rep_slots[i];
    const int t = blockIdx.x * 16 + wave;
    const bool tv = t < T;  // wave-uniform
    int id = 0;
    float wt = 0.0f;
    if (tv) route64<EPL>(logits + (size_t)t * E, E, k, lane, id, wt);
    __syncthreads();  // replica tables staged
    int p = -1;       // never matches a slot
    if (tv && lane < k) {
      const size_t pr = (size_t)t * k + lane;
      const uint32_t h = fmix32(token_id_base + (uint32_t)t);
      const int r = replica(h, s_rc[id], R_max);
      p = lds_tab ? s_rs[id * R_max + r] : rep_slots[(size_t)id * R_max + r];
      ids[pr] = id;
      w[pr] = wt;
      phys[pr] = p;
    } else if (t < Tcap && lane < k) {
      phys[(size_t)t * k + lane] = -1;  // past the device token count: no slot
    }
    if (lane < k) s_phys[wave * k + lane] = p;
    __syncthreads();
    const int np = 16 * k;
    for (int q = threadIdx.x; q < P_total; q += kFrontThreads) {
      int cnt = 0;
      for (int i = 0; i < np; ++i) cnt += s_phys[i] == q;  // same address in every lane: a broadcast
      partial[(size_t)blockIdx.x * P_total + q] = cnt;
    }
    return;
  }
  const int nb = H / kActBlock;
  const int nc = (nb + 3) / 4;
  const int wid = ((int)blockIdx.x - nr) * 16 + wave;
  const int t = wid / nc, ch = wid - t * nc;
  if (t >= T) return;  // wave-uniform
  const int b = ch * 4 + (lane >> 4);
  const bool ok = b < nb;
  const int sub = lane & 15;
  uint2 q;
  const int e = quant8(x + (size_t)t * H + b * kActBlock + sub * 8, ok, q);
  if (ok) {
    *reinterpret_cast<uint2*>(xq_tok + (size_t)t * H + b * kActBlock + sub * 8) = q;
    if (sub == 0) xs_tok[(size_t)t * nb + b] = (uint8_t)(e + 127);
  }
}

hipError_t launch_front(int T, int E, int k, int H, const float* logits, const uint16_t* x, const int32_t* rep_count,
                        const int32_t* rep_slots, int R_max, uint32_t token_id_base, int P_total, int32_t* ids,
                        float* w, int32_t* phys, int32_t* partial, uint8_t* xq_tok, uint8_t* xs_tok,
                        hipStream_t st, const int32_t* t_dev, int32_t* zero, int nzero) {
  if (T == 0) return hipSuccess;
  const int nr = (T + 15) / 16;
  // xq_tok == NULL: routing blocks only (callers that take bf16 rows)
  const long waves = xq_tok ? (long)T * ((H / kActBlock + 3) / 4) : 0;
  const unsigned grid = (unsigned)(nr + (waves + 15) / 16);
  switch (route_epl(E)) {
#define X(N)                                                                                                   \
  case N:                                                                                                      \
    k_front<N><<<grid, kFrontThreads, 0, st>>>(T, E, k, H, logits, x, rep_count, rep_slots, R_max,             \
                                               token_id_base, P_total, nr, ids, w, phys, partial, xq_tok,     \
                                               xs_tok, t_dev, zero, nzero);                                   \
    break;
    MOE_ROUTE_CASES(X)
#undef X
  }
  return hipGetLastError();
}

// a7 over pair-indexed GEMM2 rows: out[t] = bf16_rne(sum over local j,
// ascending, of w[t][j] * y[t * k + j]) (the same f32 fma chain as
// k_combine; y of a pair is the sum of GEMM2's ky K-range partials,
// ascending, when it split K).  Extra blocks after the ncomb combine blocks finish the load
// record: nred blocks add the routing blocks' chunk counts into load_hist
// (64 slots per block, four chunk groups per slot reduced in LDS), and the
// last block turns the per-slot counts (written by GEMM1) into offsets.
__global__ __launch_bounds__(256) void k_combine_pairs(int T, int H, int k, const float* __restrict__ y,
                                                       const int32_t* __restrict__ phys, int p0, int P_local,
                                                       const float* __restrict__ w, uint16_t* __restrict__ out,
                                                       int ncomb, int nred, const int32_t* __restrict__ partial,
                                                       int nch, int P_total, int32_t* __restrict__ load_hist,
                                                       const int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets, int ky) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= ncomb) {
    const int r = (int)blockIdx.x - ncomb;
    if (r < nred) {
      __shared__ int s_red[4][64];
      const int ql = tid & 63, cg = tid >> 6;
      const int q = 64 * r + ql;
      int sum = 0;
      if (q < P_total)
        for (int c = cg; c < nch; c += 4) sum += partial[(size_t)c * P_total + q];
      s_red[cg][ql] = sum;
      __syncthreads();
      if (cg == 0 && q < P_total) load_hist[q] += (s_red[0][ql] + s_red[1][ql]) + (s_red[2][ql] + s_red[3][ql]);
      return;
    }
    // offsets: thread i scans slots [4i, 4i + 4), then a Hillis-Steele scan of the 256 partial sums
    __shared__ int s_scan[256];
    int loc[4], run = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = 4 * tid + u;
      loc[u] = run;
      run += sl < P_local ? counts[sl] : 0;
    }
    s_scan[tid] = run;
    for (int off = 1; off < 256; off <<= 1) {
      __syncthreads();
      const int o = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += o;
    }
    __syncthreads();
    const int before = tid > 0 ? s_scan[tid - 1] : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = 4 * tid + u;
      if (sl < P_local) offsets[sl] = before + loc[u];
    }
    if (tid == blockDim.x - 1) offsets[P_local] = s_scan[tid];
    return;
  }
  const int lane = tid & 63;
  const int nc = (H + 511) / 512;
  const int wid = blockIdx.x * 4 + (tid >> 6);
  const int t = wid / nc, ch = wid - t * nc;
  if (t >= T) return;
  int mine = 0;
  float myw = 0.0f;
  if (lane < k) {
    const int p = phys[(size_t)t * k + lane];
    mine = p >= p0 && p < p0 + P_local;
    myw = w[(size_t)t * k + lane];
  }
  const uint64_t local = __ballot(mine);
  float ws[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) ws[j] = __shfl(myw, j);
  const int h = ch * 512 + lane * 8;
  if (h >= H) return;
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float wj = ws[j];
    if (j >= k || !((local >> j) & 1u)) continue;  // wave-uniform
    const float* yr = y + ((size_t)t * k + j) * H + h;
    float4 y0 = *reinterpret_cast<const float4*>(yr);
    float4 y1 = *reinterpret_cast<const float4*>(yr + 4);
    for (int kk = 1; kk < ky; ++kk) {  // GEMM2's K partials, ascending
      const float* yk = yr + (size_t)kk * T * k * H;
      const float4 u0 = *reinterpret_cast<const float4*>(yk);
      const float4 u1 = *reinterpret_cast<const float4*>(yk + 4);
      y0.x += u0.x;
      y0.y += u0.y;
      y0.z += u0.z;
      y0.w += u0.w;
      y1.x += u1.x;
      y1.y += u1.y;
      y1.z += u1.z;
      y1.w += u1.w;
    }
    a[0] = fmaf(wj, y0.x, a[0]);
    a[1] = fmaf(wj, y0.y, a[1]);
    a[2] = fmaf(wj, y0.z, a[2]);
    a[3] = fmaf(wj, y0.w, a[3]);
    a[4] = fmaf(wj, y1.x, a[4]);
    a[5] = fmaf(wj, y1.y, a[5]);
    a[6] = fmaf(wj, y1.z, a[6]);
    a[7] = fmaf(wj, y1.w, a[7]);
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(a[4]) | ((uint32_t)f32_to_bf16(a[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(a[6]) | ((uint32_t)f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + h) = o;
}

hipError_t launch_combine_pairs(int T, int H, int k, const float* y, const int32_t* phys, int p0, int P_local,
                                const float* w, uint16_t* out, const int32_t* partial, int nch, int P_total,
                                int32_t* load_hist, const int32_t* counts, int32_t* offsets, hipStream_t st,
                                int ky) {
  if (T == 0) return hipSuccess;
  const long waves = (long)T * ((H + 511) / 512);
  const int ncomb = (int)((waves + 3) / 4);
  const int nred = load_hist ? (P_total + 63) / 64 : 0;
  k_combine_pairs<<<(unsigned)(ncomb + nred + 1), 256, 0, st>>>(T, H, k, y, phys, p0, P_local, w, out, ncomb, nred,
                                                                partial, nch, P_total, load_hist, counts, offsets, ky);
  return hipGetLastError();
}

}  // namespace moe
