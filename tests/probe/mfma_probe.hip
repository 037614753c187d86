// Test probe, not part of libmoe: runs chains of gfx950's block-scaled
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 (A = MXFP4 e2m1, B = fp8 e4m3fn, f32
// accumulation) on operands given directly in the instruction's lane order,
// so that a test can compare the hardware's float32 results with exact sums.
//
// Lane order (lane l, g = l / 16): A holds row l % 16, K elements
// [32 g, 32 g + 32) as 16 bytes (element 2i in the low nibble of byte i);
// B holds column l % 16, K [16 g, 16 g + 16) in bytes 0-15 and
// K [64 + 16 g, 64 + 16 g + 16) in bytes 16-31; lane l's scale bytes are the
// e8m0 scales of row / column l % 16 for K block g (32 wide); the f32
// accumulator element r of lane l is D[4 g + r][l % 16].
#include <hip/hip_runtime.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Block b runs problem b: a chain of n instructions starting from c.
__global__ __launch_bounds__(64) void k_mfma_chain(const v4i* __restrict__ a, const v8i* __restrict__ b,
                                                   const int* __restrict__ sa, const int* __restrict__ sb,
                                                   const v4f* __restrict__ c, v4f* __restrict__ d, int n) {
  const int l = threadIdx.x;
  const size_t p = blockIdx.x;
  v4f acc = c[p * 64 + l];
  for (int i = 0; i < n; ++i) {
    const size_t o = (p * n + i) * 64 + l;
    const v4i av = a[o];
    const v8i a8 = {av.x, av.y, av.z, av.w, 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b[o], acc, 4, 0, 0, sa[o], 0, sb[o]);
  }
  d[p * 64 + l] = acc;
}

// a: [nprob, n, 64] x 16 bytes, b: [nprob, n, 64] x 32 bytes, sa / sb:
// [nprob, n, 64] i32 (scale in the low byte), c / d: [nprob, 64] x 4 f32.
// Device pointers, 32-byte aligned.  Returns 0, -1 for bad arguments (nothing
// launched), -4 for a launch error.
extern "C" int mfma_probe_chain(const void* a, const void* b, const int* sa, const int* sb, const float* c, float* d,
                                int nprob, int n, void* stream) {
  if (!a || !b || !sa || !sb || !c || !d || nprob < 1 || nprob > 65536 || n < 1 || n > 4096) return -1;
  k_mfma_chain<<<nprob, 64, 0, (hipStream_t)stream>>>(static_cast<const v4i*>(a), static_cast<const v8i*>(b), sa, sb,
                                                      reinterpret_cast<const v4f*>(c), reinterpret_cast<v4f*>(d), n);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
