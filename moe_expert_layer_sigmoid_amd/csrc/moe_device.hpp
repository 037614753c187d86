// Device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kActBlock = 128;   // activation scale block (columns)
constexpr int kChunkTokens = 64; // tokens per counting chunk

// MFMA operand format codes of the block-scaled f8f6f4 instructions.
constexpr int kFmtFp8 = 0;  // e4m3fn
constexpr int kFmtFp4 = 4;  // e2m1

// MurmurHash3's 32-bit finaliser (Appleby, public domain): the replica hash
// of the EPLB remap.
__host__ __device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Replica index of a token hash for an expert with `count` replicas: h mod
// count.  A count outside [1, R_max] breaks the caller's contract; it is
// clamped so that the replica-table read stays inside the expert's row.
__host__ __device__ __forceinline__ int replica(uint32_t h, int count, int R_max) {
  const int c = count < 1 ? 1 : (count > R_max ? R_max : count);
  return (int)(h % (uint32_t)c);
}

// Smallest integer e with amax <= 448 * 2^e (0 when amax == 0), clamped to
// [-127, 127].  With amax = f * 2^x, f in [0.5, 1) and 448 = 0.875 * 2^9:
// e = x - 9 when f <= 0.875, else x - 8.  Exact for every finite amax.
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  float f = frexpf(amax, &x);
  int e = x - 9 + (f > 0.875f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four f32 values (each |v| <= 448) -> four e4m3fn codes, round to nearest
// even, packed little-endian (v0 in the low byte).
__device__ __forceinline__ uint32_t pack4_fp8(float v0, float v1, float v2, float v3) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, p, true);
  return (uint32_t)p;
}

// f32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// silu(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (each within
// about one ulp): a few ulps overall, far inside the accumulation error of the
// GEMM that produced g.  Very negative g: e^-g overflows to inf, 1/inf = 0.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Block index -> work item such that consecutive items land on the same XCD.
// The hardware deals workgroups round-robin over the 8 XCDs (block b runs on
// XCD b % 8); items of one expert share activation rows, so keeping them on
// one XCD keeps those rows in that XCD's L2.
__device__ __forceinline__ int xcd_item(int b, int nblk) {
  const int nx = 8;
  int xcd = b % nx, idx = b / nx;
  int q = nblk / nx, rem = nblk % nx;
  return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Buffer resource of `bytes` bytes at `p` (gfx9 descriptor word 3: raw
// 32-bit dwords, no swizzle).  Buffer loads address it as base + lane offset
// (VGPR) + uniform offset (SGPR) + immediate, and return 0 outside
// [0, bytes) instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ v4i buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 16-byte load with cache-policy bits `AUX` (2: non-temporal, for data read
// once such as streamed weights).
template <int AUX>
__device__ __forceinline__ v4i buf_load16_p(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
__device__ __forceinline__ v2i buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ int buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ int buf_load2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ int buf_load1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Block-scaled 16x16x128 MFMA, A = MXFP4 (e2m1, 32 K-elements in the 4 low
// dwords of each lane), B = fp8 e4m3fn, f32 accumulate.  Lane l supplies
// row/column l % 16 and scale block l / 16; `OPSEL_A` picks the byte of
// `sa` that holds this lane's A scale, B's scale is the low byte of `sb`.
template <int OPSEL_A>
__device__ __forceinline__ v4f mfma_fp4_fp8(v4i a, v8i b, v4f c, int sa, int sb) {
  v8i a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, kFmtFp4, kFmtFp8, OPSEL_A, sa, 0, sb);
}

}  // namespace moe
