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
// a1 route: one wavefront per token.  Lane l holds logits l, l+64, ...; each of
// the k rounds takes a wave-wide argmax (largest logit, lower id on ties) over
// the entries not yet taken.  Weights: sigmoid of the chosen logits divided by
// their sum, in f32.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const float* row = logits + (size_t)t * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  uint32_t taken = 0;
  int my_id = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = lane + 64 * i;
      bool ok = e < E && !((taken >> i) & 1u);
      if (ok && (bi == INT_MAX || v[i] > bv)) {  // ascending e: strict > keeps the lower id
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      bool take = (oi != INT_MAX) && (bi == INT_MAX || ov > bv || (ov == bv && oi < bi));
      if (take) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_id = bi;
      my_l = bv;
    }
  }
  float s = lane < k ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
  float sum = s;
#pragma unroll
  for (int off = 1; off <= 32; off <<= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = s / sum;
  }
}

template <int EPL>
static hipError_t route_epl(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  k_route<EPL><<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int epl = (E + 63) / 64;
  switch (epl) {
    case 1: return route_epl<1>(logits, T, E, k, ids, w, st);
    case 2: return route_epl<2>(logits, T, E, k, ids, w, st);
    case 3: return route_epl<3>(logits, T, E, k, ids, w, st);
    case 4: return route_epl<4>(logits, T, E, k, ids, w, st);
    case 5: case 6: return route_epl<6>(logits, T, E, k, ids, w, st);
    case 7: case 8: return route_epl<8>(logits, T, E, k, ids, w, st);
    case 9: case 10: case 11: case 12: return route_epl<12>(logits, T, E, k, ids, w, st);
    default: return route_epl<16>(logits, T, E, k, ids, w, st);
  }
}

// ---------------------------------------------------------------------------
// a2 + a3 (part 1): per chunk of 64 tokens, optionally remap logical -> physical
// expert, then count.  No atomics: thread q counts the chunk's pairs equal to
// slot q (a broadcast read of each pair id from LDS), and thread s < P_local
// walks the chunk's pairs in (t, j) order handing out consecutive ranks for
// local slot p0 + s.  Both results are deterministic by construction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_count(int T, int k, const int32_t* __restrict__ ids,
                                               const int32_t* __restrict__ rep_count,
                                               const int32_t* __restrict__ rep_slots, int R_max,
                                               uint32_t token_id_base, int32_t* __restrict__ phys, int do_remap,
                                               int P_total, int p0, int P_local, int32_t* __restrict__ partial,
                                               int32_t* __restrict__ rank) {
  __shared__ int4 s_phys4[kChunkTokens * 16 / 4];
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
        int e = ids[pr0 + i];
        uint32_t h = fmix32(token_id_base + (uint32_t)(t0 + i / k));
        int r = (int)(h % (uint32_t)rep_count[e]);
        p = rep_slots[(size_t)e * R_max + r];
        phys[pr0 + i] = p;
      } else {
        p = phys[pr0 + i];
      }
    }
    s_phys[i] = p;
  }
  __syncthreads();
  if (partial) {
    for (int q = threadIdx.x; q < P_total; q += blockDim.x) {
      int cnt = 0;
#pragma unroll 8
      for (int i = 0; i < np4; ++i) {
        const int4 v = s_phys4[i];  // same address in every lane: a broadcast
        cnt += (v.x == q) + (v.y == q) + (v.z == q) + (v.w == q);
      }
      partial[(size_t)c * P_total + q] = cnt;
    }
  }
  if (rank) {
    for (int s = threadIdx.x; s < P_local; s += blockDim.x) {
      const int q = p0 + s;
      int r = 0;
      for (int i = 0; i < np4; ++i) {
        const int4 v = s_phys4[i];
        if (v.x == q) rank[pr0 + 4 * i] = r++;
        if (v.y == q) rank[pr0 + 4 * i + 1] = r++;
        if (v.z == q) rank[pr0 + 4 * i + 2] = r++;
        if (v.w == q) rank[pr0 + 4 * i + 3] = r++;
      }
    }
  }
}

hipError_t launch_count(int T, int k, const int32_t* ids, const int32_t* rep_count, const int32_t* rep_slots,
                        int R_max, uint32_t token_id_base, int32_t* phys, bool do_remap, int P_total, int p0,
                        int P_local, int32_t* partial, int32_t* rank, hipStream_t st) {
  if (T == 0) return hipSuccess;
  int nch = (T + kChunkTokens - 1) / kChunkTokens;
  k_count<<<nch, 256, 0, st>>>(T, k, ids, rep_count, rep_slots, R_max, token_id_base, phys, do_remap ? 1 : 0,
                               P_total, p0, P_local, partial, rank);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2 / a3 (part 2): one block of 1024 threads sums the chunk partials.
// Local slots: counts, exclusive-scan offsets, and per-(chunk, slot) base rows.
// All slots: load_hist += totals.  Work is split as (slot, chunk-range) so the
// serial part per thread is nch / NG loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_scan(int nch, int P_total, int p0, int P_local,
                                               const int32_t* __restrict__ partial, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ base,
                                               int32_t* __restrict__ load_hist) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[1024];
  const int tid = threadIdx.x;
  if (counts) {
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
      for (int c = c0; c < c1; ++c) sum += partial[(size_t)c * P_total + p0 + s];
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
      for (int c = c0; c < c1; ++c) {
        base[(size_t)c * P_local + s] = run;
        run += partial[(size_t)c * P_total + p0 + s];
      }
    }
  }
  if (load_hist) {
    for (int q = tid; q < P_total; q += 1024) {
      int sum = 0;
      for (int c = 0; c < nch; ++c) sum += partial[(size_t)c * P_total + q];
      load_hist[q] += sum;
    }
  }
}

hipError_t launch_scan(int nch, int P_total, int p0, int P_local, const int32_t* partial, int32_t* counts,
                       int32_t* offsets, int32_t* base, int32_t* load_hist, hipStream_t st) {
  k_scan<<<1, 1024, 0, st>>>(nch, P_total, p0, P_local, partial, counts, offsets, base, load_hist);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a3 (part 3) + a4: one wavefront per (token, 512-column chunk).  Lanes j < k
// resolve the row of pair (t, j) (base of its chunk and slot + rank; the
// chunk-0 wave also writes the row maps), then the wave quantises its four
// 128-column blocks: 16 lanes per block, 8 bf16 per lane; the block amax gives
// the e8m0 exponent, codes are RNE e4m3fn of x * 2^-e; the same bytes go to
// every local row of the token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant(int T, int H, int k, const uint16_t* __restrict__ x,
                                               const int32_t* __restrict__ phys, int p0, int P_local,
                                               const int32_t* __restrict__ base, const int32_t* __restrict__ rank,
                                               uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                               int32_t* __restrict__ row_of_pair, int32_t* __restrict__ pair_of_row) {
  const int lane = threadIdx.x & 63;
  const int nb = H / kActBlock;
  const int nc = (nb + 3) / 4;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = wid / nc, ch = wid - t * nc;
  if (t >= T) return;  // wave-uniform
  int myrow = -1;
  if (lane < k) {
    const size_t pr = (size_t)t * k + lane;
    const int p = phys[pr];
    if (p >= p0 && p < p0 + P_local) {
      const int s = p - p0;
      myrow = base[(size_t)(t / kChunkTokens) * P_local + s] + rank[pr];
      if (ch == 0) pair_of_row[myrow] = (int32_t)pr;
    }
    if (ch == 0) row_of_pair[pr] = myrow;
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
  const int b = ch * 4 + (lane >> 4);
  const bool ok = b < nb;
  const int sub = lane & 15;  // 8 columns each
  float v[8];
  if (ok) {
    uint4 raw = *reinterpret_cast<const uint4*>(x + (size_t)t * H + b * kActBlock + sub * 8);
    uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(wd[i] << 16);
      v[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) am = fmaxf(am, __shfl_xor(am, off));
  const int e = scale_exp(am);
  uint2 q;
  q.x = pack4_fp8(ldexpf(v[0], -e), ldexpf(v[1], -e), ldexpf(v[2], -e), ldexpf(v[3], -e));
  q.y = pack4_fp8(ldexpf(v[4], -e), ldexpf(v[5], -e), ldexpf(v[6], -e), ldexpf(v[7], -e));
  if (ok) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (rows[j] < 0) continue;  // wave-uniform
      const size_t r = (size_t)rows[j];
      *reinterpret_cast<uint2*>(xq + r * H + b * kActBlock + sub * 8) = q;
      if (sub == 0) xs[r * nb + b] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_quant(int T, int H, int k, const uint16_t* x, const int32_t* phys, int p0, int P_local,
                        const int32_t* base, const int32_t* rank, uint8_t* xq, uint8_t* xs, int32_t* row_of_pair,
                        int32_t* pair_of_row, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nc = (H / kActBlock + 3) / 4;
  const long waves = (long)T * nc;
  k_quant<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(T, H, k, x, phys, p0, P_local, base, rank, xq, xs,
                                                       row_of_pair, pair_of_row);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a7 combine: one wavefront per (token, 512-column chunk), 8 columns per lane;
// out[t] = sum over local j ascending of w[t][j] * y[row(t, j)] (f32 fma
// chain), rounded to bf16 (nearest even).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_pair,
                                                 const float* __restrict__ w, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int nc = (H + 511) / 512;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = wid / nc, ch = wid - t * nc;
  if (t >= T) return;
  int myrow = -1;
  float myw = 0.0f;
  if (lane < k) {
    myrow = row_of_pair[(size_t)t * k + lane];
    myw = w[(size_t)t * k + lane];
  }
  int rows[16];
  float ws[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int r = __shfl(myrow, j);
    ws[j] = __shfl(myw, j);
    rows[j] = j < k ? r : -1;
  }
  const int h = ch * 512 + lane * 8;
  if (h >= H) return;
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (rows[j] < 0) continue;  // wave-uniform
    const float* yr = y + (size_t)rows[j] * H + h;
    const float4 y0 = *reinterpret_cast<const float4*>(yr);
    const float4 y1 = *reinterpret_cast<const float4*>(yr + 4);
    a[0] = fmaf(ws[j], y0.x, a[0]);
    a[1] = fmaf(ws[j], y0.y, a[1]);
    a[2] = fmaf(ws[j], y0.z, a[2]);
    a[3] = fmaf(ws[j], y0.w, a[3]);
    a[4] = fmaf(ws[j], y1.x, a[4]);
    a[5] = fmaf(ws[j], y1.y, a[5]);
    a[6] = fmaf(ws[j], y1.z, a[6]);
    a[7] = fmaf(ws[j], y1.w, a[7]);
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(a[4]) | ((uint32_t)f32_to_bf16(a[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(a[6]) | ((uint32_t)f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + h) = o;
}

hipError_t launch_combine(int T, int H, int k, const float* y, const int32_t* row_of_pair, const float* w,
                          uint16_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const long waves = (long)T * ((H + 511) / 512);
  k_combine<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(T, H, k, y, row_of_pair, w, out);
  return hipGetLastError();
}

}  // namespace moe
