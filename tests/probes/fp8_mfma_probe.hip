// Test probe (not part of the library): one 32x32x64 FP8 (e4m3) matrix
// product on gfx950, to measure how far its fp32 sums lie from the exact sum
// of the 64 products.  The FP8-QK variant's parity bar depends on that
// distance.  a: 32 rows x 64 e4m3 codes, b: 32 columns x 64 codes (row-major,
// k innermost); d: 32 x 32 fp32, d[i][j] = sum_k a[i][k] * b[j][k].  Lane l
// feeds row / column l % 32 and the k-slice 32 * (l / 32) .. +31 of both
// operands (any k assignment common to A and B gives the same products).
// The output layout of the 32x32 family: lane l holds column l % 32, rows
// 8 * (r / 4) + 4 * (l / 32) + r % 4 for register r.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void fp8_mfma_probe(const uint8_t* a, const uint8_t* b, float* d) {
  const int l = threadIdx.x, r32 = l % 32, h = l / 32;
  i32x8_t av, bv;
  for (int w = 0; w < 8; ++w) {
    av[w] = *(const int*)(a + r32 * 64 + 32 * h + 4 * w);
    bv[w] = *(const int*)(b + r32 * 64 + 32 * h + 4 * w);
  }
  f32x16_t acc = {};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 16; ++r) d[(8 * (r / 4) + 4 * h + r % 4) * 32 + r32] = acc[r];
}

extern "C" int fp8_mfma_probe_run(const void* a, const void* b, void* d, void* stream) {
  hipLaunchKernelGGL(fp8_mfma_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                     (const uint8_t*)b, (float*)d);
  return (int)hipGetLastError();
}
