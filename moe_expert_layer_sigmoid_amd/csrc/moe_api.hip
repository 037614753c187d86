// C ABI of libmoe: host-side validation, workspace layout and the launch
// sequences of the fused MoE layer (see include/moe.h for the contract).

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/moe.h"
#include "moe_device.hpp"
#include "moe_internal.hpp"
#include "moe_layout.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t ids, w, phys, rank, partial, base, counts, offsets, rop, por, xq, xs, aq, as, y, plist, rtok, rw, kcnt, tlist,
      total;
};

// Split K of the pair-indexed GEMMs at decode shares (few touched slots,
// each otherwise streamed by a few CUs): ks K ranges per block with
// ks * T <= kSplitRows (measured at 7168 x 2048, top-6 of 384: 1 token
// 50 -> 39 us, 8 tokens 65 -> 46 us; at 64 tokens a split of 2 was slower).  GEMM1's partials ([ks][T k][2F] f32) and GEMM2's
// partial y ([ks][T k][H] f32) share the y region, which holds
// max(T_max, kSplitRows) k rows of H.
constexpr int kSplitRows = 32;
size_t y_rows(const moe_dims_t* d) { return (size_t)(d->T_max > kSplitRows ? d->T_max : kSplitRows) * d->k; }
// (The decode-share form runs with one token tile per pass: none of it
// where the streaming GEMMs take two.)
int stream_tiles(const moe_dims_t* d);
int split_k1(const moe_dims_t* d) {
  if (d->T <= 0 || stream_tiles(d) >= 2) return 1;
  const long nq = pack_geom(2u * d->F, (uint32_t)d->H).steps / 4;
  long ks = kSplitRows / d->T;
  const long fit = (long)(y_rows(d) * d->H / ((size_t)d->T * d->k * 2 * d->F));  // partials within the y region
  ks = ks < nq ? ks : nq;
  ks = ks < fit ? ks : fit;
  return ks > 1 ? (int)ks : 1;
}
// Block rows of the pair-indexed GEMMs: twice the expected number of
// touched local slots (T k P_local / P_total under uniform routing), at
// least 8, at most P_local (then every slot has its row, as at large T).
int touched_rows(const moe_dims_t* d) {
  if (stream_tiles(d) >= 2) return d->P_local;
  const long e = ((long)d->T * d->k * d->P_local + d->P_total - 1) / d->P_total;
  long v = 2 * e > 8 ? 2 * e : 8;
  return (int)(v < d->P_local ? v : d->P_local);
}
int split_k2(const moe_dims_t* d) {
  if (d->T <= 0 || stream_tiles(d) >= 2) return 1;
  const long nq = pack_geom((uint32_t)d->H, (uint32_t)d->F).steps / 4;
  long ks = kSplitRows / d->T;
  const long fit = (long)(y_rows(d) / ((size_t)d->T * d->k));  // partial y within the y region
  ks = ks < nq ? ks : nq;
  ks = ks < fit ? ks : fit;
  return ks > 1 ? (int)ks : 1;
}

// One workspace serves every call; regions are sized by T_max.
Layout layout_of(const moe_dims_t* d) {
  Layout L{};
  const size_t TK = (size_t)d->T_max * d->k;
  const size_t nch = ((size_t)d->T_max + kChunkTokens - 1) / kChunkTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += round_up(bytes, kAlign);
    return o;
  };
  L.ids = take(TK * 4);
  L.w = take(TK * 4);
  L.phys = take(TK * 4);
  L.rank = take(TK * 4);
  // chunk counts: 64-token chunks (staged and large-M), 16-token chunks (small-M)
  const size_t nch16 = ((size_t)(d->T_max < kPairMaxT ? d->T_max : kPairMaxT) + kFrontTokens - 1) / kFrontTokens;
  L.partial = take((nch > nch16 ? nch : nch16) * d->P_total * 4);
  L.base = take(nch * d->P_local * 4);
  L.counts = take((size_t)d->P_local * 4);
  L.offsets = take(((size_t)d->P_local + 1) * 4);
  L.rop = take(TK * 4);
  L.por = take(TK * 4);
  L.xq = take(TK * d->H);
  L.xs = take(TK * (d->H / kActBlock));
  L.aq = take(TK * d->F);
  L.as = take(TK * (d->F / kActBlock));
  L.y = take(y_rows(d) * d->H * 4);
  // per-slot pair lists of the pair-indexed GEMMs (GEMM1 -> GEMM2)
  L.plist = take((size_t)d->P_local * pair_list_stride(d->T_max, d->k) * 4);
  // bucketed rows of single-pair tokens (GEMM2 writes their output rows)
  L.rtok = take(TK * 4);
  L.rw = take(TK * 4);
  // split-K GEMM1 counters, one per (slot, 128 columns of F)
  L.kcnt = take((size_t)d->P_local * (d->F / kActBlock) * 4);
  // the pair-indexed GEMMs' touched-slot list (count, then slots)
  L.tlist = take(((size_t)d->P_local + 1) * 4);
  L.total = off;
  return L;
}

int check_dims(const moe_dims_t* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->T_max < 0 || d->T > d->T_max) return MOE_ERR_INVALID_ARG;
  if (d->T_max > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (d->H <= 0 || d->F <= 0 || d->H % 128 || d->F % 128) return MOE_ERR_INVALID_ARG;
  if (d->H > 16384 || d->F > 16384) return MOE_ERR_UNSUPPORTED;
  if (d->E < 1 || d->k < 1 || d->k > d->E) return MOE_ERR_INVALID_ARG;
  if (d->E > 1024 || d->k > 16) return MOE_ERR_UNSUPPORTED;
  if (d->P_total < 1 || d->P_local < 1 || d->p0 < 0 || d->p0 + d->P_local > d->P_total) return MOE_ERR_INVALID_ARG;
  if (d->P_total > 1024) return MOE_ERR_UNSUPPORTED;
  if (d->R_max < 1) return MOE_ERR_INVALID_ARG;
  if (d->R_max > 64) return MOE_ERR_UNSUPPORTED;
  if (d->small_m_max < 0 || d->large_m_min < 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dev_ok(const void* p) { return p != nullptr && aligned(p); }
bool opt_ok(const void* p) { return p == nullptr || aligned(p); }

int check_ws(const moe_dims_t* d, void* ws, size_t bytes) {
  size_t need = layout_of(d).total;
  if (need == 0) return MOE_OK;
  if (!ws || bytes < need) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws % kAlign) != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                         \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

int nchunks(int T) { return (T + kChunkTokens - 1) / kChunkTokens; }

// Mean (token, expert) pairs per physical slot, routing being near-uniform
// for this layer's workloads.
double mean_rows(const moe_dims_t* d) { return (double)d->T * d->k / d->P_total; }
// Token tiles per weight pass of the streaming GEMMs: two once a slot's rows
// commonly exceed one 16-row tile.
int stream_tiles(const moe_dims_t* d) { return mean_rows(d) > 10.0 ? 2 : 1; }
// The large-input path streams weights while the slots' rows fit about one
// two-tile pass (the 128-token tiles of the persistent kernels would be mostly
// empty and their weight stream latency-bound), and runs the tiled kernels
// beyond.
// (Measured at d_model 7168, d_ff 2048, 384 experts, top-6: streaming 0.26 vs
// tiled 0.36 ms at 1024 tokens (16 rows per slot), 0.35 vs 0.37 ms at 1536
// (24), 0.49 vs 0.37 ms at 2048 (32).)
constexpr double kStreamMaxRows = 24.0;
bool tiled_gemms(moe_path_t p, const moe_dims_t* d) { return p == MOE_PATH_LARGE_M && mean_rows(d) > kStreamMaxRows; }
// The tiled GEMMs stream the weights non-temporally while a slot averages at
// most 96 rows (mostly one 128-token block, nothing re-reads its weights):
// GEMM1 -5 % at 62 rows per slot, unchanged at 126, 3 % slower at ~1000.
constexpr double kTiledNtMaxRows = 96.0;
bool tiled_nt_weights(const moe_dims_t* d) { return mean_rows(d) <= kTiledNtMaxRows; }

// GEMM kernels of a path: weight streaming for few rows per expert, the
// persistent tiled kernels for many.
hipError_t gemm1(moe_path_t p, const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                 const uint8_t* pw1s, uint8_t* aq, uint8_t* as, const moe_dims_t* d, hipStream_t st) {
  if (tiled_gemms(p, d))
    return launch_gemm1_tiled(xq, xs, offsets, pw1, pw1s, aq, as, d->H, d->F, d->P_local, tiled_nt_weights(d), st);
  return launch_gemm1_stream(xq, xs, offsets, pw1, pw1s, aq, as, d->H, d->F, d->P_local, stream_tiles(d), st);
}
hipError_t gemm2(moe_path_t p, const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                 const uint8_t* pw2s, float* y, SingleRows sr, const moe_dims_t* d, hipStream_t st) {
  if (tiled_gemms(p, d))
    return launch_gemm2_tiled(aq, as, offsets, pw2, pw2s, y, d->H, d->F, d->P_local, sr, tiled_nt_weights(d), st);
  return launch_gemm2_stream(aq, as, offsets, pw2, pw2s, y, d->H, d->F, d->P_local, stream_tiles(d), sr, st);
}
// GEMM2 + combine on bucketed rows.  Tokens with exactly one local pair get
// their output row from GEMM2 itself (bf16(fma(w, y, 0)), the combine's
// arithmetic for one term) and the combine skips them, whenever the output's
// byte offsets fit the kernels' 32-bit buffer offsets (T H 2 < 2^32).
hipError_t gemm2_combine(moe_path_t p, const uint8_t* aq, const uint8_t* as, const int32_t* offsets,
                         const uint8_t* pw2, const uint8_t* pw2s, const int32_t* rop, const float* w, uint16_t* out,
                         void* ws, const moe_dims_t* d, hipStream_t st) {
  const Layout L = layout_of(d);
  float* y = at<float>(ws, L.y);
  const bool fuse = (uint64_t)d->T * (uint64_t)d->H * 2u < (1ull << 32);
  SingleRows sr{nullptr, nullptr, nullptr, 0u};
  if (fuse) {
    int32_t* rtok = at<int32_t>(ws, L.rtok);
    float* rw = at<float>(ws, L.rw);
    hipError_t e = launch_single_rows(d->T, d->k, rop, w, rtok, rw, st);
    if (e != hipSuccess) return e;
    sr = SingleRows{rtok, rw, out, (uint32_t)((uint64_t)d->T * d->H * 2u)};
  }
  hipError_t e = gemm2(p, aq, as, offsets, pw2, pw2s, y, sr, d, st);
  if (e != hipSuccess) return e;
  return launch_combine(d->T, d->H, d->k, y, rop, w, out, fuse, st);
}
// The component GEMM calls pick by token count like MOE_PATH_AUTO.
moe_path_t gemm_path(const moe_dims_t* d) {
  return moe_select_path(d) == MOE_PATH_LARGE_M ? MOE_PATH_LARGE_M : MOE_PATH_SMALL_M;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_dims_t* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return layout_of(dims).total;
}

moe_path_t moe_select_path(const moe_dims_t* d) {
  if (!d) return MOE_PATH_AUTO;
  const int small = d->small_m_max > 0 ? d->small_m_max : 512;
  const int large = d->large_m_min > 0 ? d->large_m_min : 1024;
  if (d->T <= small && d->T <= kPairMaxT) return MOE_PATH_SMALL_M;
  if (d->T >= large && tiled_fits(d->H, d->F, d->P_local)) return MOE_PATH_LARGE_M;
  return MOE_PATH_STAGED;
}

size_t moe_packed_bytes(const moe_dims_t* d, int which) {
  if (check_dims(d) != MOE_OK) return 0;
  const PackGeom g1 = pack_geom(2u * d->F, (uint32_t)d->H), g2 = pack_geom((uint32_t)d->H, (uint32_t)d->F);
  switch (which) {
    case 0: return g1.data_slot * d->P_local;
    case 1: return g1.scale_slot * d->P_local;
    case 2: return g2.data_slot * d->P_local;
    case 3: return g2.scale_slot * d->P_local;
    default: return 0;
  }
}

int moe_pack_weights(const moe_dims_t* d, const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2, const uint8_t* w2s,
                     uint8_t* pw1, uint8_t* pw1s, uint8_t* pw2, uint8_t* pw2s, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  const void* ps[] = {w1, w1s, w2, w2s, pw1, pw1s, pw2, pw2s};
  for (const void* p : ps)
    if (!dev_ok(p)) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY(launch_pack(w1, w1s, pw1, pw1s, d->P_local, 2 * d->F, d->H, st));
  MOE_TRY(launch_pack(w2, w2s, pw2, pw2s, d->P_local, d->H, d->F, st));
  return MOE_OK;
}

int32_t moe_replica_of(uint32_t token_id, int32_t rep_count, int32_t R_max) {
  return replica(fmix32(token_id), rep_count, R_max < 1 ? 1 : R_max);
}

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH: return "dims need more workspace than the fixed scratch of moe_forward_noalloc";
    default: return "unknown status";
  }
}

int moe_route(const moe_dims_t* d, const float* logits, int32_t* topk_ids, float* topk_w, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(logits) || !dev_ok(topk_ids) || !dev_ok(topk_w)) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  return hip_status(launch_route(logits, d->T, d->E, d->k, topk_ids, topk_w, (hipStream_t)stream));
}

int moe_eplb_remap_record(const moe_dims_t* d, const int32_t* topk_ids, const int32_t* rep_count,
                          const int32_t* rep_slots, int32_t* phys_ids, int32_t* load_hist, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(topk_ids) || !dev_ok(rep_count) || !dev_ok(rep_slots) || !dev_ok(phys_ids) || !opt_ok(load_hist))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  Layout L = layout_of(d);
  int32_t* partial = load_hist ? at<int32_t>(ws, L.partial) : nullptr;
  MOE_TRY(launch_count(d->T, d->k, topk_ids, rep_count, rep_slots, d->R_max, d->token_id_base, phys_ids, true,
                       d->P_total, d->p0, d->P_local, partial, nullptr, st));
  if (load_hist)
    MOE_TRY(launch_scan(nchunks(d->T), d->P_total, d->p0, d->P_local, partial, nullptr, nullptr, nullptr, load_hist,
                        st));
  return MOE_OK;
}

int moe_quant_permute(const moe_dims_t* d, const uint16_t* x, const int32_t* phys_ids, uint8_t* xq, uint8_t* xs,
                      int32_t* counts, int32_t* offsets, int32_t* row_of_pair, int32_t* pair_of_row, void* ws,
                      size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(x) || !dev_ok(phys_ids) || !dev_ok(xq) || !dev_ok(xs) || !dev_ok(counts) || !dev_ok(offsets) ||
      !dev_ok(row_of_pair) || !dev_ok(pair_of_row))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  Layout L = layout_of(d);
  int32_t* partial = at<int32_t>(ws, L.partial);
  int32_t* rank = at<int32_t>(ws, L.rank);
  int32_t* base = at<int32_t>(ws, L.base);
  MOE_TRY(launch_count(d->T, d->k, nullptr, nullptr, nullptr, d->R_max, d->token_id_base,
                       const_cast<int32_t*>(phys_ids), false, d->P_total, d->p0, d->P_local, partial, rank, st));
  MOE_TRY(launch_scan(nchunks(d->T), d->P_total, d->p0, d->P_local, partial, counts, offsets, base, nullptr, st));
  MOE_TRY(launch_quant(d->T, d->H, d->k, x, phys_ids, d->p0, d->P_local, base, rank, xq, xs, row_of_pair,
                       pair_of_row, st));
  return MOE_OK;
}

int moe_grouped_gemm1_swiglu(const moe_dims_t* d, const uint8_t* xq, const uint8_t* xs, const int32_t* offsets,
                             const uint8_t* pw1, const uint8_t* pw1s, uint8_t* aq, uint8_t* as, void* ws,
                             size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(xq) || !dev_ok(xs) || !dev_ok(offsets) || !dev_ok(pw1) || !dev_ok(pw1s) || !dev_ok(aq) || !dev_ok(as))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  if (d->T == 0) return MOE_OK;
  return hip_status(gemm1(gemm_path(d), xq, xs, offsets, pw1, pw1s, aq, as, d, (hipStream_t)stream));
}

int moe_grouped_gemm2_combine(const moe_dims_t* d, const uint8_t* aq, const uint8_t* as, const int32_t* offsets,
                              const uint8_t* pw2, const uint8_t* pw2s, const int32_t* row_of_pair,
                              const float* topk_w, uint16_t* out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(aq) || !dev_ok(as) || !dev_ok(offsets) || !dev_ok(pw2) || !dev_ok(pw2s) || !dev_ok(row_of_pair) ||
      !dev_ok(topk_w) || !dev_ok(out))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY(gemm2_combine(gemm_path(d), aq, as, offsets, pw2, pw2s, row_of_pair, topk_w, out, ws, d, st));
  return MOE_OK;
}

int moe_grouped_gemm1_swiglu_pairs(const moe_dims_t* d, const uint8_t* xq_tok, const uint8_t* xs_tok,
                                   const int32_t* phys_ids, const uint8_t* pw1, const uint8_t* pw1s, uint8_t* aq_pair,
                                   uint8_t* as_pair, int32_t* counts, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(xq_tok) || !dev_ok(xs_tok) || !dev_ok(phys_ids) || !dev_ok(pw1) || !dev_ok(pw1s) ||
      !dev_ok(aq_pair) || !dev_ok(as_pair) || !dev_ok(counts))
    return MOE_ERR_INVALID_ARG;
  if (d->T > kPairMaxT) return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return MOE_OK;
  return hip_status(launch_gemm1_pairs(xq_tok, xs_tok, phys_ids, d->T, d->k, d->p0, pw1, pw1s, aq_pair, as_pair,
                                       counts, nullptr, 0, d->H, d->F, d->P_local, stream_tiles(d), 1, nullptr,
                                       nullptr, d->P_local, nullptr, (hipStream_t)stream));
}

int moe_grouped_gemm2_combine_pairs(const moe_dims_t* d, const uint8_t* aq_pair, const uint8_t* as_pair,
                                    const int32_t* phys_ids, const uint8_t* pw2, const uint8_t* pw2s,
                                    const float* topk_w, const int32_t* counts, int32_t* offsets, uint16_t* out,
                                    void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(aq_pair) || !dev_ok(as_pair) || !dev_ok(phys_ids) || !dev_ok(pw2) || !dev_ok(pw2s) ||
      !dev_ok(topk_w) || !dev_ok(counts) || !dev_ok(offsets) || !dev_ok(out))
    return MOE_ERR_INVALID_ARG;
  if (d->T > kPairMaxT) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  float* y = at<float>(ws, layout_of(d).y);
  const int ks2 = split_k2(d);
  MOE_TRY(launch_gemm2_pairs(aq_pair, as_pair, phys_ids, d->T, d->k, d->p0, nullptr, nullptr, 0, pw2, pw2s, y, d->H,
                             d->F, d->P_local, stream_tiles(d), ks2, d->P_local, nullptr, st));
  MOE_TRY(launch_combine_pairs(d->T, d->H, d->k, y, phys_ids, d->p0, d->P_local, topk_w, out, nullptr, 0,
                               d->P_total, nullptr, counts, offsets, st, ks2));
  return MOE_OK;
}

}  // extern "C"

namespace {

// moe_forward; t_dev (device, nullable) = the device token count of
// moe_forward_small_m (SMALL_M only).
int forward_impl(const moe_dims_t* d, moe_path_t path, const int32_t* t_dev, const uint16_t* x, const float* logits,
                 const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                 const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist, uint16_t* out,
                 const moe_taps_t* taps, moe_path_t* chosen, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_LARGE_M) return MOE_ERR_INVALID_ARG;
  if (!dev_ok(x) || !dev_ok(logits) || !dev_ok(pw1) || !dev_ok(pw1s) || !dev_ok(pw2) || !dev_ok(pw2s) ||
      !dev_ok(rep_count) || !dev_ok(rep_slots) || !opt_ok(load_hist) || !dev_ok(out))
    return MOE_ERR_INVALID_ARG;
  if (taps) {
    const void* tp[] = {taps->topk_ids, taps->topk_w,  taps->phys_ids, taps->counts,  taps->offsets,
                        taps->row_of_pair, taps->pair_of_row, taps->xq, taps->xs, taps->aq,
                        taps->as, taps->xq_tok, taps->xs_tok, taps->aq_pair, taps->as_pair};
    for (const void* p : tp)
      if (!opt_ok(p)) return MOE_ERR_INVALID_ARG;
  }
  if ((rc = check_ws(d, ws, ws_bytes))) return rc;
  const moe_path_t p = path == MOE_PATH_AUTO ? moe_select_path(d) : path;
  if (p == MOE_PATH_SMALL_M && d->T > kPairMaxT) return MOE_ERR_UNSUPPORTED;
  if (p == MOE_PATH_LARGE_M && !tiled_fits(d->H, d->F, d->P_local)) return MOE_ERR_UNSUPPORTED;
  if (chosen) *chosen = p;
  if (d->T == 0) return MOE_OK;

  hipStream_t st = (hipStream_t)stream;
  Layout L = layout_of(d);
  auto pick = [&](auto* tap, size_t off) -> decltype(tap) {
    return tap ? tap : reinterpret_cast<decltype(tap)>(static_cast<char*>(ws) + off);
  };
  const moe_taps_t none{};
  const moe_taps_t& tp = taps ? *taps : none;
  int32_t* ids = pick(tp.topk_ids, L.ids);
  float* w = pick(tp.topk_w, L.w);
  int32_t* phys = pick(tp.phys_ids, L.phys);
  int32_t* counts = pick(tp.counts, L.counts);
  int32_t* offsets = pick(tp.offsets, L.offsets);
  int32_t* rop = pick(tp.row_of_pair, L.rop);
  int32_t* por = pick(tp.pair_of_row, L.por);
  uint8_t* xq = pick(tp.xq, L.xq);
  uint8_t* xs = pick(tp.xs, L.xs);
  uint8_t* aq = pick(tp.aq, L.aq);
  uint8_t* as = pick(tp.as, L.as);
  int32_t* rank = at<int32_t>(ws, L.rank);
  int32_t* partial = at<int32_t>(ws, L.partial);
  int32_t* base = at<int32_t>(ws, L.base);
  float* y = at<float>(ws, L.y);
  auto mark = [&](void* ev) { return ev ? hipEventRecord(static_cast<hipEvent_t>(ev), st) : hipSuccess; };

  if (p == MOE_PATH_SMALL_M) {
    // pair-indexed: per-token activations in the xq/xs regions, pair rows in aq/as/y
    uint8_t* xq_tok = pick(tp.xq_tok, L.xq);
    uint8_t* xs_tok = pick(tp.xs_tok, L.xs);
    uint8_t* aq_p = pick(tp.aq_pair, L.aq);
    uint8_t* as_p = pick(tp.as_pair, L.as);
    const int ks1 = split_k1(d), ks2 = split_k2(d), nvs = touched_rows(d);
    int32_t* kcnt = at<int32_t>(ws, L.kcnt);
    int32_t* tlist = at<int32_t>(ws, L.tlist);
    MOE_TRY(launch_front(d->T, d->E, d->k, d->H, logits, x, rep_count, rep_slots, d->R_max, d->token_id_base,
                         d->P_total, ids, w, phys, partial, xq_tok, xs_tok, st, t_dev, ks1 > 1 ? kcnt : nullptr,
                         ks1 > 1 ? d->P_local * (d->F / kActBlock) : 0));
    const int nt = stream_tiles(d);
    int32_t* plist = at<int32_t>(ws, L.plist);
    const int stride = pair_list_stride(d->T_max, d->k);
    MOE_TRY(mark(tp.gemm1_events[0]));
    MOE_TRY(launch_gemm1_pairs(xq_tok, xs_tok, phys, d->T, d->k, d->p0, pw1, pw1s, aq_p, as_p, counts, plist, stride,
                               d->H, d->F, d->P_local, nt, ks1, y, kcnt, nvs, tlist, st));
    MOE_TRY(mark(tp.gemm1_events[1]));
    MOE_TRY(mark(tp.gemm2_events[0]));
    MOE_TRY(launch_gemm2_pairs(aq_p, as_p, phys, d->T, d->k, d->p0, counts, plist, stride, pw2, pw2s, y, d->H, d->F,
                               d->P_local, nt, ks2, nvs, tlist, st));
    MOE_TRY(mark(tp.gemm2_events[1]));
    MOE_TRY(launch_combine_pairs(d->T, d->H, d->k, y, phys, d->p0, d->P_local, w, out, partial,
                                 (d->T + kFrontTokens - 1) / kFrontTokens, d->P_total, load_hist, counts, offsets,
                                 st, ks2));
    return MOE_OK;
  }

  MOE_TRY(launch_route(logits, d->T, d->E, d->k, ids, w, st));
  MOE_TRY(launch_count(d->T, d->k, ids, rep_count, rep_slots, d->R_max, d->token_id_base, phys, true, d->P_total,
                       d->p0, d->P_local, partial, rank, st));
  MOE_TRY(launch_scan(nchunks(d->T), d->P_total, d->p0, d->P_local, partial, counts, offsets, base, load_hist, st));
  // GEMM2 writes the output rows of single-pair tokens itself (their row
  // map from the quantise pass) whenever the output's byte offsets fit its
  // 32-bit buffer offsets
  const bool fuse = (uint64_t)d->T * (uint64_t)d->H * 2u < (1ull << 32);
  int32_t* rtok = fuse ? at<int32_t>(ws, L.rtok) : nullptr;
  float* rw = fuse ? at<float>(ws, L.rw) : nullptr;
  MOE_TRY(launch_quant(d->T, d->H, d->k, x, phys, d->p0, d->P_local, base, rank, xq, xs, rop, por, st, w, rtok, rw));
  MOE_TRY(mark(tp.gemm1_events[0]));
  MOE_TRY(gemm1(p, xq, xs, offsets, pw1, pw1s, aq, as, d, st));
  MOE_TRY(mark(tp.gemm1_events[1]));
  SingleRows sr{nullptr, nullptr, nullptr, 0u};
  if (fuse) sr = SingleRows{rtok, rw, out, (uint32_t)((uint64_t)d->T * d->H * 2u)};
  MOE_TRY(mark(tp.gemm2_events[0]));
  MOE_TRY(gemm2(p, aq, as, offsets, pw2, pw2s, y, sr, d, st));
  MOE_TRY(mark(tp.gemm2_events[1]));
  MOE_TRY(launch_combine(d->T, d->H, d->k, y, rop, w, out, fuse, st));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_dims_t* d, moe_path_t path, const uint16_t* x, const float* logits, const uint8_t* pw1,
                const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s, const int32_t* rep_count,
                const int32_t* rep_slots, int32_t* load_hist, uint16_t* out, const moe_taps_t* taps,
                moe_path_t* chosen, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return forward_impl(d, path, nullptr, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, load_hist, out, taps,
                      chosen, ws, ws_bytes, stream);
}

int moe_forward_small_m(const moe_dims_t* d, const int32_t* num_tokens, const uint16_t* x, const float* logits,
                        const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                        const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist, uint16_t* out,
                        const moe_taps_t* taps, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (!num_tokens || ((uintptr_t)num_tokens & 3u)) return MOE_ERR_INVALID_ARG;
  return forward_impl(d, MOE_PATH_SMALL_M, num_tokens, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots,
                      load_hist, out, taps, nullptr, ws, ws_bytes, stream);
}

size_t moe_router_workspace_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return round_up(router_partial_bytes(d->T_max, d->E, d->H), kAlign);
}

int moe_router_logits(const moe_dims_t* d, const uint16_t* x, const uint16_t* w_gate, float* logits, void* ws,
                      size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc != MOE_OK) return rc;
  if (!dev_ok(x) || !dev_ok(w_gate) || !dev_ok(logits)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_router_workspace_bytes(d);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws % kAlign) != 0) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(launch_router(x, w_gate, logits, static_cast<float*>(ws), d->T, d->E, d->H, st));
}

size_t moe_a16w4_workspace_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return layout_of(d).total + round_up((size_t)d->T_max * d->k * d->F * 2, kAlign);
}

int moe_forward_a16w4(const moe_dims_t* d, const uint16_t* x, const float* logits, const uint8_t* pw1,
                      const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s, const int32_t* rep_count,
                      const int32_t* rep_slots, int32_t* load_hist, uint16_t* out, const moe_taps_t* taps,
                      uint16_t* act_tap, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dev_ok(x) || !dev_ok(logits) || !dev_ok(pw1) || !dev_ok(pw1s) || !dev_ok(pw2) || !dev_ok(pw2s) ||
      !dev_ok(rep_count) || !dev_ok(rep_slots) || !opt_ok(load_hist) || !dev_ok(out) || !opt_ok(act_tap))
    return MOE_ERR_INVALID_ARG;
  if (taps) {
    const void* tp[] = {taps->topk_ids, taps->topk_w, taps->phys_ids, taps->counts, taps->offsets,
                        taps->row_of_pair, taps->pair_of_row};
    for (const void* p : tp)
      if (!opt_ok(p)) return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe_a16w4_workspace_bytes(d);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws % kAlign) != 0) return MOE_ERR_INVALID_ARG;
  if ((size_t)d->T_max * d->H * 2 >= (1u << 31) || (size_t)d->T_max * d->k * d->F * 2 >= (1u << 31))
    return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return MOE_OK;

  hipStream_t st = (hipStream_t)stream;
  Layout L = layout_of(d);
  auto pick = [&](auto* tap, size_t off) -> decltype(tap) {
    return tap ? tap : reinterpret_cast<decltype(tap)>(static_cast<char*>(ws) + off);
  };
  const moe_taps_t none{};
  const moe_taps_t& tp = taps ? *taps : none;
  int32_t* ids = pick(tp.topk_ids, L.ids);
  float* w = pick(tp.topk_w, L.w);
  int32_t* phys = pick(tp.phys_ids, L.phys);
  int32_t* counts = pick(tp.counts, L.counts);
  int32_t* offsets = pick(tp.offsets, L.offsets);
  int32_t* rop = pick(tp.row_of_pair, L.rop);
  int32_t* por = pick(tp.pair_of_row, L.por);
  uint16_t* act = act_tap ? act_tap : at<uint16_t>(ws, L.total);
  int32_t* rank = at<int32_t>(ws, L.rank);
  int32_t* partial = at<int32_t>(ws, L.partial);
  int32_t* base = at<int32_t>(ws, L.base);
  float* y = at<float>(ws, L.y);
  if (d->T <= kPairMaxT) {
    // pair-indexed rows as the a8w4 small-input path: the fused front (routing
    // and remap only), GEMMs listing their slot's pairs, combine + record
    MOE_TRY(launch_front(d->T, d->E, d->k, d->H, logits, x, rep_count, rep_slots, d->R_max, d->token_id_base,
                         d->P_total, ids, w, phys, partial, nullptr, nullptr, st));
    int32_t* plist = at<int32_t>(ws, L.plist);
    const int stride = pair_list_stride(d->T_max, d->k);
    MOE_TRY(launch_gemm1_a16_pairs(x, d->T, d->k, phys, d->p0, pw1, pw1s, act, counts, plist, stride, d->H, d->F,
                                   d->P_local, st));
    MOE_TRY(launch_gemm2_a16_pairs(act, d->T, d->k, counts, plist, stride, pw2, pw2s, y, d->H, d->F, d->P_local, st));
    MOE_TRY(launch_combine_pairs(d->T, d->H, d->k, y, phys, d->p0, d->P_local, w, out, partial,
                                 (d->T + kFrontTokens - 1) / kFrontTokens, d->P_total, load_hist, counts, offsets,
                                 st));
    return MOE_OK;
  }
  // bucketed rows: routing, remap + record, buckets as in the a8w4 layer; the
  // row maps come from the bucketed quantise kernel (its fp8 rows unused)
  MOE_TRY(launch_route(logits, d->T, d->E, d->k, ids, w, st));
  MOE_TRY(launch_count(d->T, d->k, ids, rep_count, rep_slots, d->R_max, d->token_id_base, phys, true, d->P_total,
                       d->p0, d->P_local, partial, rank, st));
  MOE_TRY(launch_scan(nchunks(d->T), d->P_total, d->p0, d->P_local, partial, counts, offsets, base, load_hist, st));
  MOE_TRY(launch_quant(d->T, d->H, d->k, x, phys, d->p0, d->P_local, base, rank, at<uint8_t>(ws, L.xq),
                       at<uint8_t>(ws, L.xs), rop, por, st));
  MOE_TRY(launch_gemm1_a16(x, d->T, offsets, por, d->k, pw1, pw1s, act, d->H, d->F, d->P_local, st));
  MOE_TRY(launch_gemm2_a16(act, d->T_max * d->k, offsets, pw2, pw2s, y, d->H, d->F, d->P_local, st));
  MOE_TRY(launch_combine(d->T, d->H, d->k, y, rop, w, out, false, st));
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free variant of moe_forward: the workspace is a file-scope
// device array, one copy per GPU, that lives as long as the process.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): its device address is resolved once per device
// with hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (resolved on the first
// call there).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_dims_t* d, moe_path_t path, const uint16_t* x, const float* logits,
                                   const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                                   const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist,
                                   uint16_t* out, moe_path_t* chosen, moe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (layout_of(d).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return forward_impl(d, path, nullptr, x, logits, pw1, pw1s, pw2, pw2s, rep_count, rep_slots, load_hist, out,
                      nullptr, chosen, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
