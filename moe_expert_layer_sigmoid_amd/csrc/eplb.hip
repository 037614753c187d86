// EPLB rebalance from the recorded slot loads (host) and the weight migration
// it implies (device copy kernel).
//
// The pages run EPLB with redundant physical experts, rebalance every few
// hundred steps from the loads the fused remap/record step counts, and check
// that rebalancing and migrations happen [sglang PR 35619 "Aiter/FlyDSL
// MegaMoEv2 backend for DeepSeek-V4", Summary and reviewer reproduction;
// FlyDSL issue 978 "Investigate MegaMoEV2 end-to-end throughput gap vs V1 on
// 8xMI355X", Benchmark plan and Data-quality gates].  They give no placement
// algorithm; the one below is a plain greedy reading (see moe.h).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/moe.h"
#include "moe_device.hpp"
#include "moe_layout.hpp"

using namespace moe;

namespace {

// share_a > share_b for shares L_a / c_a and L_b / c_b, exactly.
inline bool share_gt(int64_t La, int64_t ca, int64_t Lb, int64_t cb) { return La * cb > Lb * ca; }

struct Replica {
  int64_t L, c;
  int32_t e, i;
};

// ---------------------------------------------------------------------------
// Migration: slot s of the local weights takes logical expert src[s]'s bytes
// from the pool when src[s] >= 0.  One block copies one 16 KB chunk of one
// slot; the chunks of a slot run over its four packed buffers in turn.
// ---------------------------------------------------------------------------

constexpr int kMigThreads = 256;
constexpr size_t kMigChunk = kMigThreads * 4 * 16;

struct MigBufs {
  const uint8_t* src[4];
  uint8_t* dst[4];
  size_t bytes[4];    // per slot (= per pool expert), multiples of 16
  uint32_t first[5];  // first chunk index of each buffer within a slot
};

__global__ void __launch_bounds__(kMigThreads) k_migrate(MigBufs b, const int32_t* __restrict__ src_expert,
                                                         int n_pool) {
  const int slot = blockIdx.y;
  const int e = src_expert[slot];
  if (e < 0 || e >= n_pool) return;
  const uint32_t c = blockIdx.x;
  int w = 0;
  while (w < 3 && c >= b.first[w + 1]) ++w;
  const size_t off = (size_t)(c - b.first[w]) * kMigChunk;
  const size_t n = b.bytes[w];
  const v4i* s = reinterpret_cast<const v4i*>(b.src[w] + (size_t)e * n + off);
  v4i* d = reinterpret_cast<v4i*>(b.dst[w] + (size_t)slot * n + off);
  const size_t left = (n - off) / 16;
  v4i v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t q = (size_t)u * kMigThreads + threadIdx.x;
    if (q < left) v[u] = __builtin_nontemporal_load(s + q);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t q = (size_t)u * kMigThreads + threadIdx.x;
    if (q < left) __builtin_nontemporal_store(v[u], d + q);
  }
}

bool al16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int moe_eplb_rebalance(int32_t E, int32_t P_total, int32_t n_ranks, int32_t R_max, const int32_t* load_hist,
                       const int32_t* slot_expert_old, int32_t* rep_count, int32_t* rep_slots,
                       int32_t* slot_expert_new) {
  if (!load_hist || !slot_expert_old || !rep_count || !rep_slots || !slot_expert_new) return MOE_ERR_INVALID_ARG;
  if (E < 1 || n_ranks < 1 || R_max < 1 || P_total < E || P_total % n_ranks) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || P_total > 1024 || R_max > 64) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)E * R_max < P_total) return MOE_ERR_INVALID_ARG;
  for (int s = 0; s < P_total; ++s)
    if (slot_expert_old[s] < -1 || slot_expert_old[s] >= E || load_hist[s] < 0) return MOE_ERR_INVALID_ARG;

  // 1. logical loads
  std::vector<int64_t> L(E, 0);
  for (int s = 0; s < P_total; ++s)
    if (slot_expert_old[s] >= 0) L[slot_expert_old[s]] += load_hist[s];

  // 2. replica counts: one more to the largest share below the cap
  std::vector<int64_t> c(E, 1);
  for (int n = P_total - E; n > 0; --n) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (c[e] >= R_max) continue;
      if (best < 0 || share_gt(L[e], c[e], L[best], c[best])) best = e;
    }
    ++c[best];  // E * R_max >= P_total keeps a candidate
  }

  // 3. replicas by descending share to the least-loaded rank with room,
  //    preferring ranks without a copy
  std::vector<Replica> reps;
  reps.reserve(P_total);
  for (int e = 0; e < E; ++e)
    for (int i = 0; i < c[e]; ++i) reps.push_back({L[e], c[e], e, i});
  std::sort(reps.begin(), reps.end(), [](const Replica& a, const Replica& b) {
    if (share_gt(a.L, a.c, b.L, b.c)) return true;
    if (share_gt(b.L, b.c, a.L, a.c)) return false;
    return a.e != b.e ? a.e < b.e : a.i < b.i;
  });
  const int per = P_total / n_ranks;
  std::vector<double> load(n_ranks, 0.0);
  std::vector<int> fill(n_ranks, 0);
  std::vector<uint8_t> holds((size_t)n_ranks * E, 0);
  std::vector<int> rank_of(P_total);  // placement order -> rank
  for (int q = 0; q < P_total; ++q) {
    const int e = reps[q].e;
    int best = -1;
    for (int r = 0; r < n_ranks; ++r) {
      if (fill[r] == per) continue;
      if (best < 0) {
        best = r;
        continue;
      }
      const bool hr = holds[(size_t)r * E + e], hb = holds[(size_t)best * E + e];
      if (hr != hb) {
        if (!hr) best = r;
      } else if (load[r] < load[best]) {
        best = r;
      }
    }
    rank_of[q] = best;
    ++fill[best];
    load[best] += (double)reps[q].L / (double)reps[q].c;
    holds[(size_t)best * E + e] = 1;
  }

  // 4. inside each rank: keep a slot that held the same expert, fill the rest
  //    in ascending slot order
  for (int s = 0; s < P_total; ++s) slot_expert_new[s] = -1;
  std::vector<int> waiting;
  for (int r = 0; r < n_ranks; ++r) {
    waiting.clear();
    const int s0 = r * per;
    for (int q = 0; q < P_total; ++q) {
      if (rank_of[q] != r) continue;
      const int e = reps[q].e;
      int keep = -1;
      for (int s = s0; s < s0 + per; ++s)
        if (slot_expert_old[s] == e && slot_expert_new[s] < 0) {
          keep = s;
          break;
        }
      if (keep >= 0)
        slot_expert_new[keep] = e;
      else
        waiting.push_back(e);
    }
    size_t w = 0;
    for (int s = s0; s < s0 + per && w < waiting.size(); ++s)
      if (slot_expert_new[s] < 0) slot_expert_new[s] = waiting[w++];
  }

  for (int e = 0; e < E; ++e) {
    rep_count[e] = 0;
    for (int r = 0; r < R_max; ++r) rep_slots[(size_t)e * R_max + r] = -1;
  }
  for (int s = 0; s < P_total; ++s) {
    const int e = slot_expert_new[s];
    rep_slots[(size_t)e * R_max + rep_count[e]++] = s;
  }
  return MOE_OK;
}

int moe_eplb_migrate(const moe_dims_t* d, const int32_t* src_expert, int32_t n_pool, const uint8_t* pool_pw1,
                     const uint8_t* pool_pw1s, const uint8_t* pool_pw2, const uint8_t* pool_pw2s, uint8_t* pw1,
                     uint8_t* pw1s, uint8_t* pw2, uint8_t* pw2s, moe_stream_t stream) {
  if (moe_workspace_bytes(d) == 0) return MOE_ERR_INVALID_ARG;
  if (n_pool < 1 || n_pool > 1024) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {src_expert, pool_pw1, pool_pw1s, pool_pw2, pool_pw2s, pw1, pw1s, pw2, pw2s};
  for (const void* p : ptrs)
    if (!al16(p)) return MOE_ERR_INVALID_ARG;
  const PackGeom g1 = pack_geom(2 * d->F, d->H), g2 = pack_geom(d->H, d->F);
  MigBufs b;
  b.src[0] = pool_pw1, b.src[1] = pool_pw1s, b.src[2] = pool_pw2, b.src[3] = pool_pw2s;
  b.dst[0] = pw1, b.dst[1] = pw1s, b.dst[2] = pw2, b.dst[3] = pw2s;
  b.bytes[0] = g1.data_slot, b.bytes[1] = g1.scale_slot, b.bytes[2] = g2.data_slot, b.bytes[3] = g2.scale_slot;
  b.first[0] = 0;
  for (int w = 0; w < 4; ++w) b.first[w + 1] = b.first[w] + (uint32_t)((b.bytes[w] + kMigChunk - 1) / kMigChunk);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_migrate, dim3(b.first[4], d->P_local), dim3(kMigThreads), 0, st, b, src_expert, n_pool);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
