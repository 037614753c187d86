// Host-side launch wrappers of the libmoe kernels (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Front kernels (kernels_front.hip)
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t st);

// Remap (optional), per-chunk histogram partials and local ranks.
//  do_remap: phys = rep_slots[e][fmix32(base + t) % rep_count[e]] from ids; else phys is input.
//  partial:  [nch, P_total] counts per chunk of 64 tokens (nullable)
//  rank:     [T*k] rank of each local pair among the chunk's pairs of its slot (nullable)
hipError_t launch_count(int T, int k, const int32_t* ids, const int32_t* rep_count, const int32_t* rep_slots,
                        int R_max, uint32_t token_id_base, int32_t* phys, bool do_remap, int P_total, int p0,
                        int P_local, int32_t* partial, int32_t* rank, hipStream_t st);

// Sum chunk partials: counts/offsets/base of local slots (when counts != NULL)
// and load_hist += totals over all slots (when load_hist != NULL).
hipError_t launch_scan(int nch, int P_total, int p0, int P_local, const int32_t* partial, int32_t* counts,
                       int32_t* offsets, int32_t* base, int32_t* load_hist, hipStream_t st);

// Row assignment + fp8 quantisation + dispatch of each token to its local rows.
// rtok (nullable): also the single-pair row map launch_single_rows writes
// (rtok / rw from the routing weights w).
hipError_t launch_quant(int T, int H, int k, const uint16_t* x, const int32_t* phys, int p0, int P_local,
                        const int32_t* base, const int32_t* rank, uint8_t* xq, uint8_t* xs,
                        int32_t* row_of_pair, int32_t* pair_of_row, hipStream_t st, const float* w = nullptr,
                        int32_t* rtok = nullptr, float* rw = nullptr);

// skip_single: leave tokens with exactly one local pair alone (the bucketed
// GEMM2 kernels wrote their rows, given launch_single_rows's row map).
hipError_t launch_combine(int T, int H, int k, const float* y, const int32_t* row_of_pair, const float* w,
                          uint16_t* out, bool skip_single, hipStream_t st);
// Row map of tokens with exactly one local pair, for GEMM2 to write their
// output rows: rtok [rows] = token (or -1: two or more local pairs), rw
// [rows] = routing weight.
hipError_t launch_single_rows(int T, int k, const int32_t* row_of_pair, const float* w, int32_t* rtok, float* rw,
                              hipStream_t st);
// The output rows GEMM2 writes for single-pair tokens (nullable rtok: none).
struct SingleRows {
  const int32_t* rtok;
  const float* rw;
  uint16_t* out;
  uint32_t out_bytes;  // T H 2 (< 2^32)
};

// Small-M path (pair-indexed rows).  Front: routing, remap, per-16-token
// chunk counts partial[ceil(T/16), P_total], and every token quantised into
// xq_tok [T, H] / xs_tok [T, H/128].  t_dev (nullable, device): a token count
// read on the device; tokens from min(*t_dev, T) on get phys = -1 (idle).
// xq_tok == NULL: no quantisation blocks (xs_tok ignored).  zero (nullable):
// nzero int32 set to 0 (the split-K GEMM1's counters).
constexpr int kFrontTokens = 16;
hipError_t launch_front(int T, int E, int k, int H, const float* logits, const uint16_t* x, const int32_t* rep_count,
                        const int32_t* rep_slots, int R_max, uint32_t token_id_base, int P_total, int32_t* ids,
                        float* w, int32_t* phys, int32_t* partial, uint8_t* xq_tok, uint8_t* xs_tok, hipStream_t st,
                        const int32_t* t_dev = nullptr, int32_t* zero = nullptr, int nzero = 0);
// Combine of pair rows y [T*k, H] (the sum over ks of the ky partials at
// y + ks * T*k*H, ascending, when GEMM2 split K), plus load_hist += the
// front's chunk counts (load_hist nullable) and offsets from the per-slot
// counts GEMM1 wrote.
hipError_t launch_combine_pairs(int T, int H, int k, const float* y, const int32_t* phys, int p0, int P_local,
                                const float* w, uint16_t* out, const int32_t* partial, int nch, int P_total,
                                int32_t* load_hist, const int32_t* counts, int32_t* offsets, hipStream_t st,
                                int ky = 1);

// GEMM kernels (kernels_gemm.hip).  Weights are in the packed layout of
// moe_layout.hpp; launch_pack converts one natural MXFP4 matrix set
// [P, R, K/2] + [P, R, K/32] into it.
hipError_t launch_pack(const uint8_t* w, const uint8_t* ws, uint8_t* pw, uint8_t* ps, int P, int R, int K,
                       hipStream_t st);
// Streaming GEMMs: `nt` (1 or 2) 16-row token tiles share each pass over a
// block's weights.
hipError_t launch_gemm1_stream(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                               const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local, int nt,
                               hipStream_t st);
hipError_t launch_gemm2_stream(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                               const uint8_t* pw2s, float* y, int H, int F, int P_local, int nt, SingleRows sr,
                               hipStream_t st);
// Pair-indexed GEMMs: GEMM1's blocks list their slot's pairs from phys
// [T*k], read per-token rows xq_tok/xs_tok and write pair rows aq/as
// [T*k, F]; GEMM2 reads those and writes pair rows y [T*k, H].  T <= 1024.
constexpr int kPairMaxT = 1024;
// GEMM1 also leaves each slot's pair count in counts [P_local] and (plist
// non-null) its pair list at plist + s * stride (stride =
// pair_list_stride(T_max, k)), which GEMM2 takes instead of listing the
// pairs from phys again (with plist null GEMM2 lists them itself).
inline int pair_list_stride(int T_max, int k) {
  const long tk = (long)T_max * k;
  return (int)(tk < kPairMaxT ? tk : kPairMaxT);
}
// Split K (ks_n > 1, at most the number of 1024-element K quads): GEMM1's
// partial sums go to part [ks_n][T*k][2F] f32 and cnt [P_local * F/128]
// (zero before the call, left zero) counts finished blocks; GEMM2 writes
// ks_n partial y at y + ks * T*k*H, which the combine adds.
// Touched-slot rows (nvs < P_local): nvs block rows instead of P_local, row j
// taking the touched slots j, j + nvs, ... (ascending slot order); GEMM1 also
// zeroes the counts of untouched slots and leaves the touched list in tlist
// [1 + P_local] (count first), from which GEMM2 (with plist) takes its slots.
hipError_t launch_gemm1_pairs(const uint8_t* xq_tok, const uint8_t* xs_tok, const int32_t* phys, int T, int k, int p0,
                              const uint8_t* pw1, const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int32_t* counts,
                              int32_t* plist, int stride, int H, int F, int P_local, int nt, int ks_n, float* part,
                              int32_t* cnt, int nvs, int32_t* tlist, hipStream_t st);
hipError_t launch_gemm2_pairs(const uint8_t* aq, const uint8_t* as, const int32_t* phys, int T, int k, int p0,
                              const int32_t* counts, const int32_t* plist, int stride, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, int nt, int ks_n, int nvs,
                              const int32_t* tlist, hipStream_t st);
// Large-M: persistent tiled kernels.  Their LDS (operand rings plus the
// block's token scales) must fit a CU's 160 KB, which holds for
// H, F <= 8192: tiled_fits(H, F, P_local).
constexpr size_t kTiledLdsMax = 160 * 1024;
bool tiled_fits(int H, int F, int P_local);
// Large-M: persistent tiled kernels (grid = one block per CU, items decoded
// on the device from offsets).
// nt_weights: stream the weights with non-temporal loads (slots of about one
// 128-token block, where no other block of the slot re-reads them).
hipError_t launch_gemm1_tiled(const uint8_t* xq, const uint8_t* xs, const int32_t* offsets, const uint8_t* pw1,
                              const uint8_t* pw1s, uint8_t* aq, uint8_t* as, int H, int F, int P_local,
                              bool nt_weights, hipStream_t st);
hipError_t launch_gemm2_tiled(const uint8_t* aq, const uint8_t* as, const int32_t* offsets, const uint8_t* pw2,
                              const uint8_t* pw2s, float* y, int H, int F, int P_local, SingleRows sr,
                              bool nt_weights, hipStream_t st);

// Router projection (kernels_router.hip): logits [T, E] f32 = x [T, H] bf16 times
// w_gate [E, H] bf16 transposed.  Plan: blocks of 128 experts x 16 ni tokens
// (ni = 8 from kRouterLargeT tokens, 4 from kRouterMidT, else 1); the K range is
// split over `splits` blocks until the grid has kRouterMinBlocks blocks (at most
// kRouterMaxSplits, each split at least 128 columns), the partial sums going to
// `partial` [splits, T, E] and a reduce kernel adding them in split order.
// (Measured at 384 experts, d_model 7168: 512 tokens in 64-token tiles take
// 17.5 us, in 16-token tiles 26.7 us -- each token tile reads the whole gate
// -- and in 128-token tiles 21.9 us; 512 blocks and 32 splits 23.3 us.)
// From kRouterHugeT tokens the tiles are kRouterWideBM experts x 256 tokens in
// 64-column stages (the gate is re-read once per 256 tokens, x once per 192
// experts).
constexpr int kRouterHugeT = 4096;
constexpr int kRouterWideBM = 192;
constexpr int kRouterLargeT = 4096;
constexpr int kRouterMidT = 256;
constexpr int kRouterMinBlocks = 256;
constexpr int kRouterMaxSplits = 16;
struct RouterPlan {
  int ni, bm, gx, gy, splits, klen;
};
RouterPlan router_plan(int T, int E, int H);
// Bytes of `partial` any T <= T_max needs (an upper bound).
size_t router_partial_bytes(int T_max, int E, int H);
hipError_t launch_router(const uint16_t* x, const uint16_t* wg, float* logits, float* partial, int T, int E, int H,
                         hipStream_t st);

// a16w4 variant (kernels_a16.hip): bf16 rows on MXFP4 experts, weights
// expanded to bf16 in registers, bf16 MFMA.  GEMM1 reads the bf16 input row of
// each bucketed row's token (pair_of_row / k) and writes bf16 act rows
// [rows, F]; GEMM2 reads those and writes f32 y rows [rows, H].  Byte sizes of
// the inputs (T H 2 and rows_max F 2) must stay below 2^31.
hipError_t launch_gemm1_a16(const uint16_t* x, int T, const int32_t* offsets, const int32_t* pair_of_row, int k,
                            const uint8_t* pw1, const uint8_t* pw1s, uint16_t* act, int H, int F, int P_local,
                            hipStream_t st);
hipError_t launch_gemm2_a16(const uint16_t* act, int rows_max, const int32_t* offsets, const uint8_t* pw2,
                            const uint8_t* pw2s, float* y, int H, int F, int P_local, hipStream_t st);
// The same on pair-indexed rows (T <= kPairMaxT): act [T k, F] and y [T k, H]
// by pair; GEMM1's blocks list their slot's pairs from phys and leave counts
// and lists as launch_gemm1_pairs does, GEMM2 takes them.
hipError_t launch_gemm1_a16_pairs(const uint16_t* x, int T, int k, const int32_t* phys, int p0, const uint8_t* pw1,
                                  const uint8_t* pw1s, uint16_t* act, int32_t* counts, int32_t* plist, int stride,
                                  int H, int F, int P_local, hipStream_t st);
hipError_t launch_gemm2_a16_pairs(const uint16_t* act, int T, int k, const int32_t* counts, const int32_t* plist,
                                  int stride, const uint8_t* pw2, const uint8_t* pw2s, float* y, int H, int F,
                                  int P_local, hipStream_t st);

}  // namespace moe
