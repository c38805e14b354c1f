// Test probe (not part of the library): issue costs of the instructions the
// softmax and the two products of the attention kernels are made of, on
// gfx950, and the shader clock under a full-chip matrix load.
//
// rate_kernel: every wave runs `iters` rounds of one instruction kind on
// independent chains (8 VALU chains, or 4 matrix accumulators, so that no
// instruction waits for the one before it) and writes the shader cycle
// counter (s_memtime) before and after the loop to cyc[2 wave], cyc[2 wave +
// 1].  Cycles per instruction = (after - before) / count
// with count = iters * 64 for the VALU kinds (4 rounds of 16 chains) and
// iters * 32 for the matrix kinds (8 rounds of 4 accumulators).  kinds:
//   0 v_fma_f32            1 v_exp_f32          2 v_cvt_pk_fp8_f32
//   3 MFMA 32x32x16 bf16   4 MFMA 32x32x32 i8   5 MFMA 32x32x64 f8f6f4 (e4m3)
//   6 one bf16 MFMA + 8 v_fma_f32 (8 chains) per step (the overlap of the
//     two pipes)
//   8 v_exp_f32 and v_fma_f32 alternating on separate chains (16 of each:
//     whether the transcendental unit runs beside the FMA)
//  13 MFMA 32x32x16 bf16 on one accumulator: each product adds onto the
//     previous one's result (the dependent issue rate)
//  14 one bf16 MFMA + 4 v_exp_f32 (8 chains) per step: whether exponentials
//     run beside the products as FMAs do
// lds_kernel: every wave streams 16-byte LDS reads (ds_read_b128, kind 9) or
//   8-byte transposing reads (ds_read_b64_tr_b16, kind 10) from consecutive
//   addresses of a 64 KB tile, 8 in flight; the workgroup's span over the bytes
//   its waves read is the CU's LDS read bandwidth.
// feed_kernel: every wave runs rounds of 16 bf16 32x32x16 products whose A
//   operand comes from LDS, read two products ahead (kind 11: one 16-byte
//   read per product; kind 12: two 8-byte transposing reads), the order
//   pinned by scheduling barriers: how busy LDS-fed products keep the matrix
//   unit.
// split_kernel (kind 15): the first half of a workgroup's waves run the bf16
//   product rounds of kind 3, the second half three times as many rounds of
//   kind 1 (exponentials), so each product wave shares its SIMD with
//   exponential waves for its whole run; every wave also writes the SIMD it
//   ran on (bits 5:4 of the hardware ID register) to sink[n + wave], n the
//   number of waves: whether exponentials on one wave slow another wave's
//   products.
// clock_kernel: every wave runs bf16 MFMA chains for `iters` rounds and
// writes its shader cycles and its 100 MHz real-time ticks (s_memrealtime),
// so cycles / ticks * 100 MHz is the clock the chip ran at under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__device__ __forceinline__ void run_rounds(int iters, float a, float b, float* out) {
  if constexpr (KIND == 8) {
    float x[16], y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = a + (float)i * b;
      y[i] = b + (float)i * a;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i)  // one asm statement per pair keeps them alternating
          asm volatile("v_exp_f32 %0, %0\n\tv_fma_f32 %1, %1, %2, %3" : "+v"(x[i]), "+v"(y[i]) : "v"(a), "v"(b));
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i] + y[i];
    *out = s;
  } else if constexpr (KIND <= 2) {
    // 16 chains: a wave64 VALU result is ready only several instructions
    // later, and a single wave must not wait for it
    float x[16];
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[i] = a + (float)i * b;
      w[i] = __float_as_uint(x[i]);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (KIND == 0) x[i] = __builtin_fmaf(x[i], a, b);
          if constexpr (KIND == 1) x[i] = __builtin_amdgcn_exp2f(x[i]);
          if constexpr (KIND == 2) w[i] = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(w[i]), b, w[i], false);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += KIND == 2 ? __uint_as_float(w[i]) : x[i];
    *out = s;
  } else {
    f32x16 acc[4];
    i32x16 iacc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[c][r] = a;
        iacc[c][r] = c;
      }
    bf16x8 av, bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      av[e] = (__bf16)a;
      bv[e] = (__bf16)b;
    }
    const i32x4 ai = {1, 2, 3, 4}, bi = {5, 6, 7, (int)threadIdx.x};
    const i32x8 a8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      (int)threadIdx.x};
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = a + (float)i * b;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (KIND == 3 || KIND == 6)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
          if constexpr (KIND == 13) acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[0], 0, 0, 0);
          if constexpr (KIND == 14) {
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * (c & 1) + i] = __builtin_amdgcn_exp2f(x[4 * (c & 1) + i]);
          }
          if constexpr (KIND == 4) iacc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, bi, iacc[c], 0, 0, 0);
          if constexpr (KIND == 5)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, acc[c], 0, 0, 0, 0, 0, 0);
          if constexpr (KIND == 6) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], a, b);
          }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0] + (float)iacc[c][0];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += x[i];
    *out = s;
  }
}

template <int KIND>
__global__ void rate_kernel(int iters, float a, float b, unsigned long long* cyc, float* sink) {
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  float s;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  run_rounds<KIND>(iters, a, b, &s);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) {
    cyc[2 * wave] = t0;
    cyc[2 * wave + 1] = t1;
    sink[wave] = s;
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short __attribute__((address_space(3))) lds_short;
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

template <bool TR>
__global__ void lds_kernel(int iters, unsigned long long* cyc, float* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[16384];  // 64 KB
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) tile[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  uint32_t acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    uint32_t v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (TR) {
        // 512 consecutive bytes per instruction, 128 windows: byte offsets < 65536
        const int off = (((it * 8 + u) & 127) * 512 + lane * 8) / 4;
        const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off));
        const uint2 w = __builtin_bit_cast(uint2, r);
        v[u][0] = w.x;
        v[u][1] = w.y;
        v[u][2] = v[u][3] = 0u;
      } else {
        // 1 KB consecutive bytes per instruction, 64 windows: byte offsets < 65536
        const int off = (((it * 8 + u) & 63) * 1024 + lane * 16) / 4;
        const uint4 w = *(const uint4*)(tile + off);
        v[u][0] = w.x;
        v[u][1] = w.y;
        v[u][2] = w.z;
        v[u][3] = w.w;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    cyc[2 * wave] = t0;
    cyc[2 * wave + 1] = t1;
  }
  sink[wave * 64 + lane] = (float)acc;
}

template <bool TR>
__global__ void feed_kernel(int iters, unsigned long long* cyc, float* sink) {
  constexpr int kDepth = 2;
  __shared__ __attribute__((aligned(16))) uint32_t tile[16384];  // 64 KB
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) tile[i] = 0x3f803f80u ^ (uint32_t)(i & 7);
  __syncthreads();
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x & 63, w4 = (threadIdx.x / 64) & 3;
  f32x16 acc[2] = {};
  bf16x8 bv;
#pragma unroll
  for (int e = 0; e < 8; ++e) bv[e] = (__bf16)(0.001f * (float)lane);
  int it = 0;
  // operand of product k in round it: rows move with it, so no read is loop-invariant
  auto rd = [&](int k) -> uint4 {
    if constexpr (TR) {
      // byte offsets < 15 * 1024 + 504 + 512 + 8 <= 65536
      const int o1 = (((k + it) & 15) * 1024 + lane * 8) / 4, o2 = o1 + 512 / 4;
      const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + o1)));
      const uint2 y = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + o2)));
      return uint4{x.x, x.y, y.x, y.y};
    } else {
      // byte offsets < 15 * 1024 + 1008 + 16 + 3 * 16384 <= 65536
      return *(const uint4*)(tile + (((k + it) & 15) * 1024 + lane * 16) / 4 + w4 * 4096);
    }
  };
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (it = 0; it < iters; ++it) {
    uint4 buf[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) buf[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      acc[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, buf[k % kDepth]), bv, acc[k & 1],
                                                           0, 0, 0);
      if (k + kDepth < 16) buf[k % kDepth] = rd(k + kDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    cyc[2 * wave] = t0;
    cyc[2 * wave + 1] = t1;
  }
  sink[wave * 64 + lane] = acc[0][0] + acc[1][5];
}

__global__ void split_kernel(int iters, float a, float b, unsigned long long* cyc, float* sink) {
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int n = gridDim.x * (blockDim.x / 64);
  const bool products = (int)(threadIdx.x / 64) < (int)(blockDim.x / 128);  // wave-uniform
  float s;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  if (products) run_rounds<3>(iters, a, b, &s);
  else run_rounds<1>(3 * iters, a, b, &s);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  // HW_ID register, all 32 bits: (31 << 11) | (0 << 6) | 4
  const unsigned hwid = __builtin_amdgcn_s_getreg(0xF804);
  if ((threadIdx.x & 63) == 0) {
    cyc[2 * wave] = t0;
    cyc[2 * wave + 1] = t1;
    sink[wave] = s;
    sink[n + wave] = (float)((hwid >> 4) & 3);
  }
}

__global__ void clock_kernel(int iters, float a, float b, unsigned long long* out, float* sink) {
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  float s;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  run_rounds<3>(iters, a, b, &s);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) {
    out[2 * wave] = t1 - t0;
    out[2 * wave + 1] = r1 - r0;
    sink[wave] = s;
  }
}

// cyc: device array of 2 * wgs * waves_per_wg entries;
// sink: device array of 64 * wgs * waves_per_wg floats.  kind 7 = clock_kernel.
extern "C" int issue_rate_probe_run(int kind, int wgs, int waves_per_wg, int iters, void* cyc, void* sink,
                                    void* stream) {
  if (wgs < 1 || waves_per_wg < 1 || waves_per_wg > 16 || iters < 1) return -1;
  const dim3 grid(wgs), block(64 * waves_per_wg);
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* c = (unsigned long long*)cyc;
  float* k = (float*)sink;
  const float a = 0.999f, b = 1e-3f;
  switch (kind) {
    case 0: hipLaunchKernelGGL(rate_kernel<0>, grid, block, 0, s, iters, a, b, c, k); break;
    case 1: hipLaunchKernelGGL(rate_kernel<1>, grid, block, 0, s, iters, a, b, c, k); break;
    case 2: hipLaunchKernelGGL(rate_kernel<2>, grid, block, 0, s, iters, a, b, c, k); break;
    case 3: hipLaunchKernelGGL(rate_kernel<3>, grid, block, 0, s, iters, a, b, c, k); break;
    case 4: hipLaunchKernelGGL(rate_kernel<4>, grid, block, 0, s, iters, a, b, c, k); break;
    case 5: hipLaunchKernelGGL(rate_kernel<5>, grid, block, 0, s, iters, a, b, c, k); break;
    case 6: hipLaunchKernelGGL(rate_kernel<6>, grid, block, 0, s, iters, a, b, c, k); break;
    case 7: hipLaunchKernelGGL(clock_kernel, grid, block, 0, s, iters, a, b, c, k); break;
    case 8: hipLaunchKernelGGL(rate_kernel<8>, grid, block, 0, s, iters, a, b, c, k); break;
    case 9: hipLaunchKernelGGL(lds_kernel<false>, grid, block, 0, s, iters, c, k); break;
    case 10: hipLaunchKernelGGL(lds_kernel<true>, grid, block, 0, s, iters, c, k); break;
    case 11: hipLaunchKernelGGL(feed_kernel<false>, grid, block, 0, s, iters, c, k); break;
    case 12: hipLaunchKernelGGL(feed_kernel<true>, grid, block, 0, s, iters, c, k); break;
    case 13: hipLaunchKernelGGL(rate_kernel<13>, grid, block, 0, s, iters, a, b, c, k); break;
    case 14: hipLaunchKernelGGL(rate_kernel<14>, grid, block, 0, s, iters, a, b, c, k); break;
    case 15:
      if (waves_per_wg % 2 != 0) return -1;
      hipLaunchKernelGGL(split_kernel, grid, block, 0, s, iters, a, b, c, k);
      break;
    default: return -1;
  }
  return (int)hipGetLastError();
}
