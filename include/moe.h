/*
 * moe.h -- C ABI of libmoe: one MI355X's share of a fused Mixture-of-Experts
 * layer (sigmoid top-k routing, EPLB remap + load recording, fp8 activations
 * on MXFP4 experts), as hand-written HIP kernels for gfx950.
 *
 * What the layer is, from the pages:
 *  - The MegaMoEV2 operator runs quant, dispatch, GEMM1, GEMM2 and combine;
 *    its small-input path does all of them in one kernel for up to 512 tokens
 *    per rank, and its persistent large-input path serves extend steps of at
 *    least 1024 tokens [sglang PR 47065 "[Perf] [AMD] dsv4: Use the aiter
 *    MegaMoE small- and large-input paths", intro and Modifications].
 *  - Activations are fp8 and routed experts MXFP4 ("a8w4") [InferenceX PR 3430
 *    "[AMD][MI35X] 0926 DSV4 sglang mtp agentic", Additional detail section].
 *  - Each token picks its top-6 routed experts [sglang PR 35619 "Aiter/FlyDSL
 *    MegaMoEv2 backend for DeepSeek-V4", "Four settings that silently break
 *    it", item 2].
 *  - Prefill fuses the EPLB logical-to-physical remap with load recording
 *    [same page, Summary]; EPLB runs with redundant physical experts
 *    [FlyDSL issue 978 "Investigate MegaMoEV2 end-to-end throughput gap vs V1
 *    on 8xMI355X", Benchmark plan].
 *  The pages print no formula; the readings used for the unstated steps are:
 *  sigmoid scores and renormalised top-k weights, replica = MurmurHash3
 *  fmix32(global token id) mod replica count, e8m0 per-128-column activation
 *  scales, SwiGLU between the GEMMs, routing weights applied in the combine.
 *
 * Conventions for every call
 *  - Pointers other than `dims`, `taps` and `chosen` are DEVICE pointers owned
 *    by the caller; they must be 16-byte aligned.  The library allocates
 *    nothing and keeps no state between calls (moe_forward_noalloc's scratch
 *    is a fixed array of the library's device code, not an allocation).
 *  - Every call is asynchronous on `stream` (NULL = the default stream); it
 *    never synchronises the host and never prints.
 *  - Arguments are validated on the host before any launch; a failed check
 *    returns a negative moe_status_t and launches nothing.  A launch error
 *    becomes MOE_ERR_HIP.  Finite inputs, expert ids in [0, E) and replica
 *    tables whose entries lie in [0, P_total) are the caller's contract.
 *  - T == 0 is valid and launches nothing (the outputs have no rows).
 *  - Calls on one workspace must not overlap in time; use one workspace per
 *    stream for concurrent calls.
 *
 * Layouts (row-major, C order):
 *  logits   f32  [T, E]
 *  x        bf16 [T, H]                 (uint16 bit patterns)
 *  w1       u8   [P_local, 2F, H/2]     MXFP4: e2m1 pairs, element 2i in the low
 *                                       nibble; rows [0, F) gate, [F, 2F) up
 *  w1s      u8   [P_local, 2F, H/32]    e8m0 scale of each 32-element block along K
 *  w2       u8   [P_local, H, F/2]
 *  w2s      u8   [P_local, H, F/32]
 *  pw1, pw1s, pw2, pw2s                 the same weights repacked by
 *                                       moe_pack_weights (sizes: moe_packed_bytes):
 *    each 16-row tile, each 256-wide K step, each of the step's two
 *    16x16x128 MFMAs: 64 lanes x 16 bytes, lane 16g + r holding row r,
 *    32-block 8 step + 4 i + g; scales per tile and 4 steps: 64 lanes x 8
 *    bytes, byte 2 (step % 4) + i of lane 16g + r = scale of row r, block
 *    8 step + 4 i + g.  K is padded with zero blocks to a multiple of 1024.
 *  rep_count  i32 [E]                   replicas of each logical expert (>= 1)
 *  rep_slots  i32 [E, R_max]            physical slot of replica r of expert e
 *  load_hist  i32 [P_total]             += pairs per physical slot (nullable)
 *  topk_ids i32 [T, k], topk_w f32 [T, k], phys_ids i32 [T, k]
 *  counts   i32 [P_local], offsets i32 [P_local + 1]
 *  row_of_pair i32 [T*k] (-1: remote pair), pair_of_row i32 [T_max*k]
 *  xq u8 [T_max*k, H] (fp8 e4m3fn), xs u8 [T_max*k, H/128] (e8m0)
 *  aq u8 [T_max*k, F], as u8 [T_max*k, F/128]
 *  out bf16 [T, H]
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad shape or misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2, /* a size beyond the limits below */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_bytes */
  MOE_ERR_HIP = -4,         /* a kernel launch failed */
  MOE_ERR_SCRATCH = -5      /* moe_forward_noalloc: the dims need more than its fixed scratch */
} moe_status_t;

typedef enum {
  MOE_PATH_AUTO = 0,    /* SMALL_M if T <= min(small_m_max, 1024), LARGE_M if T >= large_m_min,
                           else STAGED */
  MOE_PATH_SMALL_M = 1, /* four launches in (token, j) pair order: route + remap + quant of every
                           token; GEMM1 and GEMM2 weight streaming, each block listing its slot's
                           pairs itself; combine + load record.  No bucket scan or permute.
                           T <= 1024 (else MOE_ERR_UNSUPPORTED). */
  MOE_PATH_STAGED = 2,  /* the component calls in sequence (bucketed rows, weight streaming) */
  MOE_PATH_LARGE_M = 3  /* bucketed rows, persistent tiled GEMMs once the mean rows per physical
                           slot (T k / P_total) exceed 24, weight streaming below */
} moe_path_t;

/* Problem sizes of one call.  Limits: 0 <= T <= T_max <= 1<<20; H, F
 * multiples of 128, each in [128, 16384]; 1 <= E <= 1024; 1 <= k <= min(E, 16);
 * 1 <= P_total <= 1024; 0 <= p0, 1 <= P_local, p0 + P_local <= P_total;
 * 1 <= R_max <= 64.  Without EPLB: P_total = E, R_max = 1, rep_slots[e] = e. */
typedef struct {
  int32_t T, T_max;
  int32_t H, F, E, k;
  int32_t P_total, p0, P_local, R_max;
  uint32_t token_id_base;  /* global id of token 0; the remap hashes global ids */
  int32_t small_m_max;     /* 0 -> 512  [sglang PR 47065, intro]            */
  int32_t large_m_min;     /* 0 -> 1024 [sglang PR 47065, Modifications]    */
} moe_dims_t;

/* Optional device copies of intermediate results for parity checks, and
 * timing hooks; any member may be NULL.  Shapes as in the layout table above.  Every path
 * writes topk_ids, topk_w, phys_ids, counts and offsets.  STAGED and
 * LARGE_M (bucketed rows) write row_of_pair, pair_of_row, xq, xs, aq, as;
 * SMALL_M writes instead the per-token activations xq_tok u8 [T, H] /
 * xs_tok u8 [T, H/128] (every token, local pairs or not) and the per-pair
 * act rows aq_pair u8 [T*k, F] / as_pair u8 [T*k, F/128] (rows of local
 * pairs only). */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* phys_ids;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_of_pair;
  int32_t* pair_of_row;
  uint8_t* xq;
  uint8_t* xs;
  uint8_t* aq;
  uint8_t* as;
  uint8_t* xq_tok;
  uint8_t* xs_tok;
  uint8_t* aq_pair;
  uint8_t* as_pair;
  /* Timing hooks (HOST values: hipEvent_t handles created by the caller, any
   * may be NULL): moe_forward records gemm1_events[0] / [1] on `stream` right
   * before / after its GEMM1 launch and gemm2_events likewise around GEMM2,
   * so that a caller can time those kernels inside the whole forward. */
  void* gemm1_events[2];
  void* gemm2_events[2];
} moe_taps_t;

/* Bytes of device workspace every call below needs for `dims` (sized by
 * T_max, independent of T).  Returns 0 for invalid dims. */
size_t moe_workspace_bytes(const moe_dims_t* dims);

/* The path MOE_PATH_AUTO takes for `dims`: small-input at most small_m_max
 * tokens, large-input from large_m_min tokens, staged in between
 * [sglang PR 47065, intro and Modifications; the aiter commit note on the
 * three-state large-input switch]. */
moe_path_t moe_select_path(const moe_dims_t* dims);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* Bytes of a packed weight buffer for `dims` over all P_local slots:
 * which = 0 pw1, 1 pw1s, 2 pw2, 3 pw2s.  Returns 0 for invalid arguments. */
size_t moe_packed_bytes(const moe_dims_t* dims, int which);

/* Repack MXFP4 expert weights (natural layout above) into the MFMA-operand
 * order the GEMM kernels stream: every weight load of a wavefront becomes one
 * contiguous 1 KB and one 8-byte scale load covers four K steps of a tile.
 * Pure byte movement, run once when weights are loaded (like the checkpoint
 * conversion that produced the MXFP4 experts [InferenceX PR 3430, Additional
 * detail section]).  Output buffers must not overlap the inputs. */
int moe_pack_weights(const moe_dims_t* dims, const uint8_t* w1, const uint8_t* w1s, const uint8_t* w2,
                     const uint8_t* w2s, uint8_t* pw1, uint8_t* pw1s, uint8_t* pw2, uint8_t* pw2s,
                     moe_stream_t stream);

/* a1. Top-k routing [sglang PR 35619, "Four settings that silently break it"].
 * For each token: the k largest logits (descending, equal logits to the lower
 * expert id); weight_j = sigmoid(l_j) / sum_i sigmoid(l_i) in f32. */
int moe_route(const moe_dims_t* dims, const float* logits, int32_t* topk_ids, float* topk_w,
              moe_stream_t stream);

/* a2. EPLB logical -> physical remap with load recording [sglang PR 35619,
 * Summary; FlyDSL issue 978, Data-quality gates].
 * phys[t][j] = rep_slots[e][fmix32(token_id_base + t) mod rep_count[e]],
 * e = topk_ids[t][j]; if load_hist != NULL, load_hist[p] += number of pairs
 * with phys == p (all T*k pairs, every slot).  Deterministic, no atomics. */
int moe_eplb_remap_record(const moe_dims_t* dims, const int32_t* topk_ids, const int32_t* rep_count,
                          const int32_t* rep_slots, int32_t* phys_ids, int32_t* load_hist,
                          void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The replica a2 sends a token to (host utility, no device call): the index
 * r in [0, rep_count) of rep_slots[e][r] for global token id `token_id` of an
 * expert with `rep_count` replicas, r = fmix32(token_id) mod rep_count
 * (MurmurHash3's 32-bit finaliser).  The kernels use the same rule; a
 * rep_count outside [1, R_max] (a broken table) is clamped into that range
 * there and here, so that no table read leaves the expert's row. */
int32_t moe_replica_of(uint32_t token_id, int32_t rep_count, int32_t R_max);

/* a3 + a4. Bucket this GPU's pairs by local slot and quantise + dispatch the
 * activations [sglang PR 47065, intro: "quant, dispatch"].
 * Local pairs have p0 <= phys < p0 + P_local; slot s = phys - p0 owns rows
 * [offsets[s], offsets[s+1]), filled in ascending (t, j).  Row r holds token
 * pair_of_row[r] / k quantised per 128 columns: scale byte e + 127 with e the
 * smallest integer such that amax <= 448 * 2^e, codes RNE_e4m3fn(x * 2^-e). */
int moe_quant_permute(const moe_dims_t* dims, const uint16_t* x, const int32_t* phys_ids,
                      uint8_t* xq, uint8_t* xs, int32_t* counts, int32_t* offsets,
                      int32_t* row_of_pair, int32_t* pair_of_row,
                      void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* a5. GEMM1 + SwiGLU + fp8 requant, grouped by slot [sglang PR 47065, intro].
 * For each row r of slot s: h = W1_s a_r (f32 accumulation of block-scaled
 * fp8 x MXFP4 products); act_f = silu(h_f) * h_{F+f}; act requantised with
 * the a4 rule per 128 columns into aq / as.  `offsets` as from a3; weights
 * packed by moe_pack_weights. */
int moe_grouped_gemm1_swiglu(const moe_dims_t* dims, const uint8_t* xq, const uint8_t* xs,
                             const int32_t* offsets, const uint8_t* pw1, const uint8_t* pw1s,
                             uint8_t* aq, uint8_t* as, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/* a6 + a7. GEMM2 and the routing-weighted combine [sglang PR 47065, intro].
 * y_r = W2_s dequant(aq_r) (f32); out[t] = bf16_rne(sum over local j, ascending,
 * of topk_w[t][j] * y[row_of_pair[t*k+j]]); tokens with no local pair get +0. */
int moe_grouped_gemm2_combine(const moe_dims_t* dims, const uint8_t* aq, const uint8_t* as,
                              const int32_t* offsets, const uint8_t* pw2, const uint8_t* pw2s,
                              const int32_t* row_of_pair, const float* topk_w, uint16_t* out,
                              void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* a5 on the small-input path's pair-indexed rows (what MOE_PATH_SMALL_M runs
 * between its front end and GEMM2) [sglang PR 47065, intro].  Same arithmetic
 * as moe_grouped_gemm1_swiglu; the rows of slot s are the pairs p (ascending)
 * with phys_ids[p] == p0 + s, listed by each block itself.  Inputs: per-token
 * activations xq_tok u8 [T, H] / xs_tok u8 [T, H/128] (the a4 rule) and
 * phys_ids [T*k]; outputs: act rows aq_pair u8 [T*k, F] / as_pair
 * u8 [T*k, F/128] (rows of local pairs only; others untouched) and
 * counts i32 [P_local].  T <= 1024, else MOE_ERR_UNSUPPORTED.  No workspace. */
int moe_grouped_gemm1_swiglu_pairs(const moe_dims_t* dims, const uint8_t* xq_tok, const uint8_t* xs_tok,
                                   const int32_t* phys_ids, const uint8_t* pw1, const uint8_t* pw1s,
                                   uint8_t* aq_pair, uint8_t* as_pair, int32_t* counts, moe_stream_t stream);

/* a6 + a7 on pair-indexed rows: y_p = W2_s dequant(aq_pair_p) for every local
 * pair p (f32, in the workspace), then out as in moe_grouped_gemm2_combine
 * with row(t, j) = t*k + j; `offsets` i32 [P_local + 1] receives the
 * exclusive scan of `counts`.  T <= 1024, else MOE_ERR_UNSUPPORTED. */
int moe_grouped_gemm2_combine_pairs(const moe_dims_t* dims, const uint8_t* aq_pair, const uint8_t* as_pair,
                                    const int32_t* phys_ids, const uint8_t* pw2, const uint8_t* pw2s,
                                    const float* topk_w, const int32_t* counts, int32_t* offsets, uint16_t* out,
                                    void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The whole layer, a1..a7, on `path` (MOE_PATH_AUTO: moe_select_path).
 * rep_count / rep_slots describe the replica table; load_hist (nullable) is
 * accumulated as in a2 (pass NULL in decode: recording is prefill-only
 * [sglang PR 35619, Summary]).  `chosen` (host, nullable) receives the path
 * taken.  `taps` (host struct of device pointers, nullable) receives copies
 * of the intermediates. */
int moe_forward(const moe_dims_t* dims, moe_path_t path, const uint16_t* x, const float* logits,
                const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist,
                uint16_t* out, const moe_taps_t* taps, moe_path_t* chosen,
                void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* a16w4 variant of the whole layer: bf16 activations on the MXFP4 experts,
 * no activation quantisation (the pages' non-EP arms run the MXFP4 experts
 * with bf16 activations [InferenceX PR 3430, Additional detail section]).
 * Routing, remap + record and buckets as moe_forward; GEMM1 takes each
 * bucketed row's bf16 input row as is (products exact, f32 accumulation),
 * act = silu(gate) * up rounded to bf16 (nearest even), GEMM2 on the bf16
 * act, combine as moe_forward.  The weight scale bytes of non-zero MXFP4
 * elements must lie in [2, 252] (every value then a normal bf16; the caller's
 * contract like finite inputs).  Rows: T <= 1024 takes pair-indexed rows as
 * MOE_PATH_SMALL_M (four launches), larger T bucketed rows as the staged
 * path (seven launches).  taps (nullable): topk_ids, topk_w, phys_ids,
 * counts, offsets as moe_forward, and for bucketed rows also row_of_pair,
 * pair_of_row (other members ignored); act_tap (nullable, device): bf16 act
 * rows [T_max*k, F], in bucket order for bucketed rows, by pair t*k+j for
 * pair-indexed rows (rows of remote pairs unspecified).  Workspace:
 * moe_a16w4_workspace_bytes(dims).  T * H * 2 and T_max * k * F * 2 bytes
 * must stay below 2^31 (else MOE_ERR_UNSUPPORTED).  Asynchronous on
 * `stream`. */
size_t moe_a16w4_workspace_bytes(const moe_dims_t* dims);
int moe_forward_a16w4(const moe_dims_t* dims, const uint16_t* x, const float* logits, const uint8_t* pw1,
                      const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s, const int32_t* rep_count,
                      const int32_t* rep_slots, int32_t* load_hist, uint16_t* out, const moe_taps_t* taps,
                      uint16_t* act_tap, void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The small-input path with the token count on the device, for captured
 * graphs: decode graphs are captured per token-count bucket and must also
 * run idle (zero-token) steps [sglang PR 35619, Summary: graph-safe idle
 * handling; sglang PR 47065, Modifications: DP-synchronised buckets for the
 * captured graphs, forward_small_m(max_tokens=)].  dims->T is the bucket
 * capacity (<= 1024; every launch shape follows it); num_tokens (DEVICE, i32,
 * 4-byte aligned) holds the step's valid count n, read by the kernels, so one
 * capture serves every n in [0, dims->T] (values outside are clamped).  The
 * first n tokens go through the layer exactly as moe_forward(MOE_PATH_SMALL_M)
 * with T = n computes them; rows [n, T) of `out` are written as +0; load_hist
 * (nullable) counts only the first n tokens' pairs; taps hold the first n
 * tokens' intermediates (phys_ids of the others = -1, the rest unspecified).
 * Other arguments and errors as moe_forward.  Launches no memset and
 * allocates nothing, so the four launches can be captured into a graph. */
int moe_forward_small_m(const moe_dims_t* dims, const int32_t* num_tokens, const uint16_t* x, const float* logits,
                        const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                        const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist, uint16_t* out,
                        const moe_taps_t* taps, void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Router projection in front of a1: logits[t][e] = sum_k x[t][k] w_gate[e][k]
 * (bf16 x bf16 products, f32 accumulation in an unspecified order).  The
 * gate is stored in BF16 [InferenceX PR 3430, Additional detail section];
 * routing then takes the top-k of these logits (moe_route / moe_forward).
 * Layouts: x bf16 [T, H] (as everywhere), w_gate bf16 [E, H] (one row per
 * logical expert, no bias), logits f32 [T, E].  Only dims->T, T_max, H, E
 * matter (the other fields must still be valid dims).  Workspace: at least
 * moe_router_workspace_bytes(dims) bytes, 256-byte aligned (split-K partial
 * sums; sized by T_max).  T == 0 launches nothing.  Asynchronous on `stream`;
 * one or two launches. */
size_t moe_router_workspace_bytes(const moe_dims_t* dims);
int moe_router_logits(const moe_dims_t* dims, const uint16_t* x, const uint16_t* w_gate, float* logits,
                      void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* EPLB rebalance: a new replica table from the loads recorded by a2 (host
 * call; every pointer is a HOST pointer; no stream, no device memory).
 * The pages run EPLB with redundant physical experts and rebalance every few
 * hundred steps from the recorded per-expert loads [sglang PR 35619,
 * Summary and reviewer reproduction; FlyDSL issue 978, Benchmark plan and
 * Data-quality gates]; they give no placement algorithm.  This one:
 *  1. L_e = sum of load_hist[s] over the slots s with slot_expert_old[s] == e
 *     (slots holding -1 are ignored);
 *  2. every expert gets one replica; P_total - E times, the expert with the
 *     largest L_e / c_e (exact comparison) among those with c_e < R_max gets
 *     one more, equal shares to the lower e;
 *  3. replicas in descending L_e / c_e (then e, then replica index) go one by
 *     one to the rank (slots [r P_total/n_ranks, (r+1) P_total/n_ranks)) with
 *     a free slot that does not hold e yet, else any rank with a free slot,
 *     the one with the smallest load (f64 sum of the shares placed on it,
 *     in placement order), then the lower rank;
 *  4. inside a rank a replica keeps a slot that held e in the old map (the
 *     lowest first), so that it needs no migration; the others fill the
 *     rank's remaining slots in ascending order, in placement order.
 * Inputs: load_hist i32 [P_total] (>= 0; the histogram of all ranks' tokens
 * in a multi-GPU job), slot_expert_old i32 [P_total] (expert of each slot,
 * -1 = empty).  Outputs: rep_count i32 [E], rep_slots i32 [E, R_max] (each
 * expert's slots ascending, -1 padded; the table moe_forward takes with this
 * R_max), slot_expert_new i32 [P_total].  Requires E <= P_total,
 * P_total % n_ranks == 0 and E * R_max >= P_total; MOE_ERR_INVALID_ARG
 * otherwise (nothing written). */
int moe_eplb_rebalance(int32_t E, int32_t P_total, int32_t n_ranks, int32_t R_max, const int32_t* load_hist,
                       const int32_t* slot_expert_old, int32_t* rep_count, int32_t* rep_slots,
                       int32_t* slot_expert_new);

/* EPLB weight migration for this GPU's slots (the pages' data-quality gates
 * check that rebalances and migrations take place [FlyDSL issue 978,
 * Data-quality gates]).  For each local slot s
 * (s < dims->P_local) with src_expert[s] >= 0, the packed weights of slot s
 * (pw1, pw1s, pw2, pw2s, layout of moe_pack_weights) become a byte copy of
 * logical expert src_expert[s]'s packed weights in the pool; slots with -1
 * keep their bytes.  The pool holds n_pool experts packed by moe_pack_weights
 * (a pack with P_local = n_pool): on one GPU it stands in for the peer or
 * host memory a multi-GPU job would fetch experts from.  src_expert: DEVICE
 * i32 [P_local]; entries >= n_pool are skipped.  Only dims->H, F, P_local
 * matter; the pool and the slots must not overlap.  Asynchronous on
 * `stream`, one launch. */
int moe_eplb_migrate(const moe_dims_t* dims, const int32_t* src_expert, int32_t n_pool, const uint8_t* pool_pw1,
                     const uint8_t* pool_pw1s, const uint8_t* pool_pw2, const uint8_t* pool_pw2s, uint8_t* pw1,
                     uint8_t* pw1s, uint8_t* pw2, uint8_t* pw2s, moe_stream_t stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, paths, results and errors as
 * moe_forward with taps = NULL; the workspace is instead a fixed device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, that
 * each GPU the library runs on holds until the process ends.  The first call
 * on a device resolves that device's copy (the calling thread's current
 * device must be the stream's device).  Dims whose moe_workspace_bytes exceed
 * the scratch return MOE_ERR_SCRATCH before any launch (at d_model 7168,
 * d_ff 2048, top-6: T_max up to 587 tokens).  The call allocates nothing and
 * needs no part of the scratch to start at zero (every kernel writes what it
 * reads), but all calls on one GPU share that GPU's scratch, which keeps the
 * last call's contents: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_forward_noalloc(const moe_dims_t* dims, moe_path_t path, const uint16_t* x, const float* logits,
                        const uint8_t* pw1, const uint8_t* pw1s, const uint8_t* pw2, const uint8_t* pw2s,
                        const int32_t* rep_count, const int32_t* rep_slots, int32_t* load_hist, uint16_t* out,
                        moe_path_t* chosen, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
