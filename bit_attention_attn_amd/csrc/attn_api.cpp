// attn_api.cpp -- the extern "C" entry points declared in include/attn.h.
//
// Every argument check runs before any HIP call, so an invalid call returns
// its status without touching the device.  There is no fallback: shapes,
// dtypes or devices the kernels do not cover are errors.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn_internal.hpp"

// ---- fixed scratch of attn_bwd_noalloc ---------------------------------
// Callers that cannot allocate device memory use attn_bwd_noalloc, whose one
// scratch buffer (D = rowsum(dO * O), one fp32 per query row, fully written
// by the first kernel of every call before any kernel reads it) lives in
// this fixed device array: one copy per GPU, held until the process ends.
// Calls that overlap on one GPU share it and race.
constexpr size_t kBwdScratchBytes = (size_t)ATTN_BWD_NOALLOC_MAX_ROWS * sizeof(float);  // 16 MiB
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

attn_status check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 96 && d != 128) return ATTN_ERR_HEADDIM;
  const int64_t elems = (int64_t)B * H * N * d;
  if (elems >= kMaxElems) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// A block bias (or its gradient) is fp32 [B,H,nb,nb], nb = ceil(N/64).  The
// tensor obeys the per-tensor rule (< 2^31 elements), and the forward kernels
// address one head's nb*nb values with 32-bit byte offsets through a buffer
// descriptor, so nb*nb*4 must stay below 2^32 (nb <= 32767, N <= 2,097,088).
attn_status check_bias_size(int B, int H, int N) {
  const int64_t nb = ((int64_t)N + 63) / 64;
  if ((int64_t)B * H * nb * nb >= kMaxElems) return ATTN_ERR_SHAPE;
  if (nb * nb * 4 >= ((int64_t)1 << 32)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

attn_status check_common(void* o, float* lse, int B, int H, int N, int d, int causal, float scale,
                         const float* bias) {
  if (o == nullptr) return ATTN_ERR_NULL;
  attn_status s = check_shape(B, H, N, d);
  if (s != ATTN_OK) return s;
  if (bias != nullptr && (s = check_bias_size(B, H, N)) != ATTN_OK) return s;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_ARG;
  if (!aligned(o, 16)) return ATTN_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
  if (bias && !aligned(bias, 4)) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// 0 unknown, 1 gfx950, 2 other / unavailable; per device ordinal.
std::atomic<int> g_dev_ok[64];

attn_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
  if (dev < 64) {
    const int known = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return ATTN_OK;
    if (known == 2) return ATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

attn_status fwd16(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, int d, int causal, float scale, const float* bias, int out_dtype,
                  void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr) return ATTN_ERR_NULL;
  attn_status s = check_common(o, lse, B, H, N, d, causal, scale, bias);
  if (s != ATTN_OK) return s;
  const int in_dtype = bf16 ? ATTN_DTYPE_BF16 : ATTN_DTYPE_F16;
  if (out_dtype != in_dtype && out_dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_ALIGN;
  s = check_device();
  if (s != ATTN_OK) return s;
  attn::FwdArgs a{q, k, v, o, lse, bias, B, H, N, d, causal, scale,
                  out_dtype == ATTN_DTYPE_F32 ? attn::kOutF32 : (bf16 ? attn::kOutBF16 : attn::kOutF16)};
  if (attn::launch_fwd16(a, bf16, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

// Strides of a strided call (n tensors, 3 strides each): every stride
// non-negative and a multiple of 8 elements (16-byte rows), token strides at
// least d, and `extra` rows past N still addressable with 32-bit byte
// offsets from a head's base.
attn_status check_strides(const long long* st, int n, int N, int d, int extra) {
  for (int t = 0; t < n; ++t) {
    for (int i = 0; i < 3; ++i) {
      const long long x = st[3 * t + i];
      if (x < 0 || x > (1LL << 31)) return ATTN_ERR_ARG;
      if (x % 8 != 0) return ATTN_ERR_ALIGN;
    }
    if (st[3 * t + 2] < d) return ATTN_ERR_ARG;
    if ((long long)(N + extra) * st[3 * t + 2] * 2 >= (1LL << 32)) return ATTN_ERR_SHAPE;
  }
  return ATTN_OK;
}

attn_status fwd16_strided(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int N, int d, const long long* strides, const int* cu_seqlens, int causal,
                          float scale, const float* bias, int out_dtype, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || strides == nullptr) return ATTN_ERR_NULL;
  attn_status s = check_common(o, lse, B, H, N, d, causal, scale, bias);
  if (s != ATTN_OK) return s;
  const int in_dtype = bf16 ? ATTN_DTYPE_BF16 : ATTN_DTYPE_F16;
  if (out_dtype != in_dtype && out_dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_ALIGN;
  if (cu_seqlens != nullptr && !aligned(cu_seqlens, 4)) return ATTN_ERR_ALIGN;
  // the key and value loads of the last block read whole 64-row blocks, up
  // to 63 rows past N, which must stay addressable with 32-bit byte offsets
  // from a head's base (the buffer descriptor returns zeros for them)
  s = check_strides(strides, 4, N, d, 64);
  if (s != ATTN_OK) return s;
  s = check_device();
  if (s != ATTN_OK) return s;
  attn::FwdArgs a{q, k, v, o, lse, bias, B, H, N, d, causal, scale,
                  out_dtype == ATTN_DTYPE_F32 ? attn::kOutF32 : (bf16 ? attn::kOutBF16 : attn::kOutF16)};
  a.general = true;
  for (int i = 0; i < 12; ++i) a.strides[i] = strides[i];
  a.cu = cu_seqlens;
  if (attn::launch_fwd16(a, bf16, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

void* bwd_scratch();

// noalloc: the workspace comes from the library's fixed device array (the
// workspace arguments are ignored; shapes that need more than it holds are
// ATTN_ERR_WORKSPACE)
attn_status bwd16(bool bf16, const void* q, const void* k, const void* v, const void* o, int o_dtype,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dbias, int B, int H,
                  int N, int d, int causal, float scale, const float* bias, int grad_dtype, void* workspace,
                  size_t workspace_bytes, void* stream, bool noalloc = false) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return ATTN_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 96 && d != 128) return ATTN_ERR_HEADDIM;
  if ((int64_t)B * H * N * d >= kMaxElems) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_ARG;
  const int in_dtype = bf16 ? ATTN_DTYPE_BF16 : ATTN_DTYPE_F16;
  if (grad_dtype != in_dtype && grad_dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (o_dtype != in_dtype && o_dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if ((bias != nullptr || dbias != nullptr) && check_bias_size(B, H, N) != ATTN_OK) return ATTN_ERR_SHAPE;
  if (noalloc) {
    if (attn_bwd_workspace_size(B, H, N, d) > kBwdScratchBytes) return ATTN_ERR_WORKSPACE;
  } else if (workspace == nullptr || workspace_bytes < attn_bwd_workspace_size(B, H, N, d)) {
    return ATTN_ERR_WORKSPACE;
  }
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(ptr, 16)) return ATTN_ERR_ALIGN;
  if (!aligned(lse, 4) || (!noalloc && !aligned(workspace, 256)) || (bias && !aligned(bias, 4)) ||
      (dbias && !aligned(dbias, 4)))
    return ATTN_ERR_ALIGN;
  attn_status s = check_device();
  if (s != ATTN_OK) return s;
  if (noalloc && (workspace = bwd_scratch()) == nullptr) return ATTN_ERR_HIP;
  attn::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, dbias, bias, static_cast<float*>(workspace),
                  B, H, N, d, causal, scale,
                  grad_dtype == ATTN_DTYPE_F32 ? attn::kOutF32 : (bf16 ? attn::kOutBF16 : attn::kOutF16),
                  o_dtype == ATTN_DTYPE_F32};
  if (attn::launch_bwd16(a, bf16, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

// Device address of the current device's copy of `scratch` (host code must
// not use the array's name, which is a host-side stand-in): looked up once
// per device, with that device current, on its first use; nullptr on a HIP
// error.
std::atomic<void*> g_scratch_ptr[64];

void* bwd_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < 64) {
    void* known = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (known != nullptr) return known;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
  if (dev < 64) g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

attn_status prep8(const void* q, const void* k, const void* v, int in_dtype, int B, int H, int N, int d,
                  const long long* strides, const int* cu_seqlens, void* workspace, size_t workspace_bytes,
                  void* stream, int fmt) {
  if (q == nullptr || k == nullptr || v == nullptr) return ATTN_ERR_NULL;
  attn_status s = check_shape(B, H, N, d);
  if (s != ATTN_OK) return s;
  if (in_dtype != ATTN_DTYPE_F16 && in_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_ERR_ALIGN;
  if (workspace == nullptr) return ATTN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return ATTN_ERR_ALIGN;
  if (workspace_bytes < attn::sage8_layout(B, H, N, d).total) return ATTN_ERR_WORKSPACE;
  if (cu_seqlens != nullptr && !aligned(cu_seqlens, 4)) return ATTN_ERR_ALIGN;
  int64_t st[9];
  if (strides != nullptr) {
    // the column statistics read whole 256-row chunks, up to 255 rows past N
    s = check_strides(strides, 3, N, d, 256);
    if (s != ATTN_OK) return s;
    for (int i = 0; i < 9; ++i) st[i] = strides[i];
  }
  s = check_device();
  if (s != ATTN_OK) return s;
  if (attn::launch_sage8_prep(q, k, v, in_dtype == ATTN_DTYPE_BF16, B, H, N, d, strides ? st : nullptr, cu_seqlens,
                              workspace, static_cast<hipStream_t>(stream), fmt) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status fwd8(const void* workspace, void* o, float* lse, int B, int H, int N, int d, int causal, float scale,
                 const float* bias, int out_dtype, const long long* o_strides, const int* cu_seqlens, void* stream,
                 bool qk_fp8) {
  if (workspace == nullptr) return ATTN_ERR_WORKSPACE;
  attn_status s = check_common(o, lse, B, H, N, d, causal, scale, bias);
  if (s != ATTN_OK) return s;
  if (out_dtype != ATTN_DTYPE_F16 && out_dtype != ATTN_DTYPE_BF16 && out_dtype != ATTN_DTYPE_F32)
    return ATTN_ERR_DTYPE;
  if (!aligned(workspace, 256)) return ATTN_ERR_ALIGN;
  if (cu_seqlens != nullptr && !aligned(cu_seqlens, 4)) return ATTN_ERR_ALIGN;
  if (o_strides != nullptr) {
    s = check_strides(o_strides, 1, N, d, 0);
    if (s != ATTN_OK) return s;
  }
  s = check_device();
  if (s != ATTN_OK) return s;
  attn::FwdArgs a{nullptr, nullptr, nullptr, o, lse, bias, B, H, N, d, causal, scale,
                  out_dtype == ATTN_DTYPE_F32 ? attn::kOutF32
                                              : (out_dtype == ATTN_DTYPE_BF16 ? attn::kOutBF16 : attn::kOutF16)};
  if (o_strides != nullptr) {
    a.general = true;
    for (int i = 0; i < 3; ++i) a.strides[9 + i] = o_strides[i];
  }
  a.cu = cu_seqlens;
  if (attn::launch_fwd_sage8(workspace, a, static_cast<hipStream_t>(stream), qk_fp8) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

attn_status fwd_q8(const void* workspace, const void* v, int v_dtype, void* o, float* lse, int B, int H, int N,
                   int d, int causal, float scale, const float* bias, int out_dtype, void* stream) {
  if (workspace == nullptr) return ATTN_ERR_WORKSPACE;
  if (v == nullptr) return ATTN_ERR_NULL;
  attn_status s = check_common(o, lse, B, H, N, d, causal, scale, bias);
  if (s != ATTN_OK) return s;
  if (v_dtype != ATTN_DTYPE_F16 && v_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (out_dtype != v_dtype && out_dtype != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (!aligned(workspace, 256)) return ATTN_ERR_ALIGN;
  if (!aligned(v, 16)) return ATTN_ERR_ALIGN;
  s = check_device();
  if (s != ATTN_OK) return s;
  const bool bf16 = v_dtype == ATTN_DTYPE_BF16;
  attn::FwdArgs a{nullptr, nullptr, v, o, lse, bias, B, H, N, d, causal, scale,
                  out_dtype == ATTN_DTYPE_F32 ? attn::kOutF32 : (bf16 ? attn::kOutBF16 : attn::kOutF16)};
  if (attn::launch_fwd_q8(workspace, a, bf16, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                         int N, int d, int causal, float scale, const float* bias, int out_dtype,
                         void* stream) {
  return fwd16(false, q, k, v, o, lse, B, H, N, d, causal, scale, bias, out_dtype, stream);
}

attn_status attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                          int N, int d, int causal, float scale, const float* bias, int out_dtype,
                          void* stream) {
  return fwd16(true, q, k, v, o, lse, B, H, N, d, causal, scale, bias, out_dtype, stream);
}

attn_status attn_fwd_strided_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int N, int d, const long long* strides, const int* cu_seqlens, int causal,
                                 float scale, const float* bias, int out_dtype, void* stream) {
  return fwd16_strided(false, q, k, v, o, lse, B, H, N, d, strides, cu_seqlens, causal, scale, bias, out_dtype,
                       stream);
}

attn_status attn_fwd_strided_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                  int N, int d, const long long* strides, const int* cu_seqlens, int causal,
                                  float scale, const float* bias, int out_dtype, void* stream) {
  return fwd16_strided(true, q, k, v, o, lse, B, H, N, d, strides, cu_seqlens, causal, scale, bias, out_dtype,
                       stream);
}

size_t attn_sage8_workspace_size(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != ATTN_OK) return 0;
  return attn::sage8_layout(B, H, N, d).total;
}

int attn_sage8_workspace_layout(int B, int H, int N, int d, size_t* out, int n) {
  if (check_shape(B, H, N, d) != ATTN_OK || out == nullptr || n <= 0) return 0;
  const attn::Sage8Layout L = attn::sage8_layout(B, H, N, d);
  const size_t vals[9] = {L.qq, L.kq, L.vq, L.sq, L.sk, L.sv, L.kmean, (size_t)L.nblk * 64, (size_t)L.nblk};
  const int m = n < 9 ? n : 9;
  for (int i = 0; i < m; ++i) out[i] = vals[i];
  return m;
}

attn_status attn_k_smooth_quant(const void* q, const void* k, const void* v, int in_dtype, int B, int H,
                                int N, int d, void* workspace, size_t workspace_bytes, void* stream) {
  return prep8(q, k, v, in_dtype, B, H, N, d, nullptr, nullptr, workspace, workspace_bytes, stream, attn::kPrepInt8);
}

attn_status attn_k_smooth_quant_fp8qk(const void* q, const void* k, const void* v, int in_dtype, int B, int H,
                                      int N, int d, void* workspace, size_t workspace_bytes, void* stream) {
  return prep8(q, k, v, in_dtype, B, H, N, d, nullptr, nullptr, workspace, workspace_bytes, stream, attn::kPrepFp8);
}

attn_status attn_fwd_sage8(const void* workspace, void* o, float* lse, int B, int H, int N, int d,
                           int causal, float scale, const float* bias, int out_dtype, void* stream) {
  return fwd8(workspace, o, lse, B, H, N, d, causal, scale, bias, out_dtype, nullptr, nullptr, stream, false);
}

attn_status attn_fwd_sage8_fp8qk(const void* workspace, void* o, float* lse, int B, int H, int N, int d,
                                 int causal, float scale, const float* bias, int out_dtype, void* stream) {
  return fwd8(workspace, o, lse, B, H, N, d, causal, scale, bias, out_dtype, nullptr, nullptr, stream, true);
}

attn_status attn_fwd_sage8_pv16(const void* workspace, const void* v, int v_dtype, void* o, float* lse, int B,
                                int H, int N, int d, int causal, float scale, const float* bias, int out_dtype,
                                void* stream) {
  return fwd_q8(workspace, v, v_dtype, o, lse, B, H, N, d, causal, scale, bias, out_dtype, stream);
}

attn_status attn_k_smooth_quant_strided(const void* q, const void* k, const void* v, int in_dtype, int B, int H,
                                        int N, int d, const long long* strides, const int* cu_seqlens,
                                        int qk_format, void* workspace, size_t workspace_bytes, void* stream) {
  if (strides == nullptr) return ATTN_ERR_NULL;
  if (qk_format != ATTN_QK_INT8 && qk_format != ATTN_QK_FP8 && qk_format != ATTN_QK_INT8_NO_V) return ATTN_ERR_ARG;
  const int fmt = qk_format == ATTN_QK_FP8 ? attn::kPrepFp8
                  : qk_format == ATTN_QK_INT8_NO_V ? attn::kPrepInt8NoV : attn::kPrepInt8;
  return prep8(q, k, v, in_dtype, B, H, N, d, strides, cu_seqlens, workspace, workspace_bytes, stream, fmt);
}

attn_status attn_fwd_sage8_strided(const void* workspace, void* o, float* lse, int B, int H, int N, int d,
                                   const long long* o_strides, const int* cu_seqlens, int causal, float scale,
                                   const float* bias, int out_dtype, int qk_format, void* stream) {
  if (o_strides == nullptr) return ATTN_ERR_NULL;
  if (qk_format != ATTN_QK_INT8 && qk_format != ATTN_QK_FP8) return ATTN_ERR_ARG;
  return fwd8(workspace, o, lse, B, H, N, d, causal, scale, bias, out_dtype, o_strides, cu_seqlens, stream,
              qk_format == ATTN_QK_FP8);
}

size_t attn_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 96 && d != 128)) return 0;
  if ((int64_t)B * H * N * d >= kMaxElems) return 0;
  return ((size_t)B * H * N * sizeof(float) + 255) & ~(size_t)255;
}

attn_status attn_bwd_f16(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, float* dbias, int B, int H, int N,
                         int d, int causal, float scale, const float* bias, int grad_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return bwd16(false, q, k, v, o, o_dtype, dout, lse, dq, dk, dv, dbias, B, H, N, d, causal, scale, bias, grad_dtype,
               workspace, workspace_bytes, stream);
}

attn_status attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* dbias, int B, int H, int N,
                          int d, int causal, float scale, const float* bias, int grad_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return bwd16(true, q, k, v, o, o_dtype, dout, lse, dq, dk, dv, dbias, B, H, N, d, causal, scale, bias, grad_dtype,
               workspace, workspace_bytes, stream);
}

attn_status attn_bwd_noalloc(int in_dtype, const void* q, const void* k, const void* v, const void* o, int o_dtype,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dbias, int B,
                             int H, int N, int d, int causal, float scale, const float* bias, int grad_dtype,
                             void* stream) {
  if (in_dtype != ATTN_DTYPE_F16 && in_dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  return bwd16(in_dtype == ATTN_DTYPE_BF16, q, k, v, o, o_dtype, dout, lse, dq, dk, dv, dbias, B, H, N, d, causal,
               scale, bias, grad_dtype, nullptr, 0, stream, true);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: B, H, N must be >= 1 and each tensor < 2^31 elements";
    case ATTN_ERR_HEADDIM: return "ATTN_ERR_HEADDIM: head dimension must be 64, 96 or 128";
    case ATTN_ERR_DTYPE: return "ATTN_ERR_DTYPE: unsupported input/output dtype";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: pointer not aligned (tensors 16 B, workspace 256 B)";
    case ATTN_ERR_ARG: return "ATTN_ERR_ARG: invalid argument (causal must be 0/1, scale finite)";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_DEVICE: return "ATTN_ERR_DEVICE: current device is not gfx950 (MI355X)";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown attn_status";
  }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
