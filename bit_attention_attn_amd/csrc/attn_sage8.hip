// attn_sage8.hip -- the 8-bit (SageAttention-style) path on gfx950.
//
// Page 1 ("SageAttention", claim vs reality section): the first product
// Q K^T runs on INT8 matrix units after K is mean-centred (softmax is
// shift-invariant, so the centring changes no output), the softmax output P
// lies in [0, 1] and goes to FP8 for the second product P V, and the two are
// combined with a two-level accumulation.
//
// Preparation (HBM-bound, three kernels):
//   colstats  per 256-token chunk of each (b,h): fp64 column sums of K and
//             fp32 column absmax of V.
//   finalize  per (b,h), 256 threads: kmean = (sum of chunk sums) / N rounded
//             once to fp32; V scale = absmax/448 and its inverse 448/absmax
//             (1 if 0).
//   quant     per 64-row block: Q and K - kmean to INT8 with one fp32 scale
//             per block (scale = absmax/127, code = rne(x * (127/absmax)),
//             clamp +-127); V to e4m3 (code = e4m3_rne(v * inv)), written
//             through LDS into the per-block transposed layout that the P V
//             product reads.
// Forward: S^T = Kq Qq^T on 32x32x32 INT8 MFMA (int32, exact, read as fp32
// through an offset), scaled by sq*sk*scale*log2(e) per 64x64 block; online
// softmax in base 2 with a lazy running maximum (raised only when a block
// maximum exceeds it by more than kTau8 = 2); P^ = e4m3(448 * 2^(t - m -
// kTau8)) <= 448 becomes the B operand of a 32x32x64 FP8 MFMA straight from
// the S^T registers; V^T comes from the prepared tile.  Level one of the
// accumulation is the fp32 sum over the 64 keys of a block inside one matrix
// instruction, level two the fp32 running output carried across blocks.  The
// normaliser l sums the fp32 values of P before they are quantised; the V
// scales and 1/l are applied once.
#include "attn_common.hpp"
#include "attn_internal.hpp"

#include <math.h>

namespace attn {

namespace {

constexpr int kQB = 64;        // rows per INT8 scale block (and keys per block)
constexpr int kChunk = 256;    // tokens per column-statistics chunk
// threads of the preparation kernels: a multiple of the 16-byte chunks per
// row (D/8), so every thread keeps one chunk column (192 at d = 96)
template <int D>
constexpr int prep_threads() { return D == 96 ? 192 : 256; }
constexpr float kTau8 = 2.0f;  // lazy-rescale threshold of the 8-bit path (log2 units)
// log2(448) - kTau8: P^ = e4m3(2^(t - m + kPlog)) stays <= 448
constexpr float kPlog = 6.807354922057604f;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

Sage8Layout sage8_layout(int B, int H, int N, int d) {
  Sage8Layout L{};
  const size_t bh = (size_t)B * H;
  const size_t np = (size_t)((N + 127) / 128) * 128;  // tokens padded to whole 128-row tiles
  L.nblk = (int)(np / kQB);
  L.nchunk = (N + kChunk - 1) / kChunk;
  size_t off = 0;
  L.qq = off; off = align256(off + bh * np * d);
  L.kq = off; off = align256(off + bh * np * d);
  L.vq = off; off = align256(off + bh * np * d);
  L.sq = off; off = align256(off + bh * L.nblk * sizeof(float));
  L.sk = off; off = align256(off + bh * L.nblk * sizeof(float));
  L.sv = off; off = align256(off + bh * d * sizeof(float));
  L.vinv = off; off = align256(off + bh * d * sizeof(float));
  L.kmean = off; off = align256(off + bh * d * sizeof(float));
  L.kpart = off; off = align256(off + bh * (size_t)L.nchunk * d * sizeof(double));
  L.vpart = off; off = align256(off + bh * (size_t)L.nchunk * d * sizeof(float));
  L.total = off;
  return L;
}

namespace {

// Position of key k (0..63 in its block) inside the lane order of the P^T
// operand: the S^T accumulator gives lane half h the keys 32T + 8g + 4h + u
// (register r = 4g + u of tile T); byte e = 16T + r of half h is the key at
// position 32h + e.
__device__ __forceinline__ int key_pos(int k) {
  const int T = k >> 5, kin = k & 31;
  const int h = (kin >> 2) & 1, g = kin >> 3, u = kin & 3;
  return 32 * h + 16 * T + 4 * g + u;
}

// ---- colstats: grid (nchunk, B*H), prep_threads<D>() threads --------------------------
// Input layout: element strides (batch, head, token) of q, k, v, d contiguous.
// cu (nullable, device int32 [B+1]) packs the sequences along the token axis:
// batch entry b is tokens cu[b] .. cu[b+1]-1 (at most N of them), and every
// statistic of the recipe (K mean, V channel scales, 64-row blocks) is taken
// over that sequence alone, so its workspace slot is the one it would get on
// its own.
struct PrepIn {
  int H;
  int64_t s[9];
  const int* cu;
};

// Sequence of batch entry b: its length (<= N) and the element offset of its
// first row of tensor t (0: q, 1: k, 2: v) at head h.
__device__ __forceinline__ int seq_span(const PrepIn& in, int b, int h, int N, int t, int64_t& base) {
  if (in.cu == nullptr) {
    base = b * in.s[3 * t] + h * in.s[3 * t + 1];
    return N;
  }
  const int t0 = in.cu[b];
  base = (int64_t)t0 * in.s[3 * t + 2] + h * in.s[3 * t + 1];
  return max(0, min(in.cu[b + 1] - t0, N));
}

// NOV: Q and K only (the INT8-score variant with the 16-bit P V product
// reads no FP8 V): V is neither read nor summarised.
template <int D, bool BF16, bool NOV>
__global__ __launch_bounds__(256) void sage8_colstats(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                      int N, double* __restrict__ kpart,
                                                      float* __restrict__ vpart, int nchunk, PrepIn in) {
  constexpr int kCpr = D / 8;                        // 16-byte chunks per row
  constexpr int kRows = prep_threads<D>() / kCpr;    // rows per pass
  __shared__ double ssum[kRows][D];
  __shared__ float smax[kRows][D];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, ch = tid % kCpr, rg = tid / kCpr;
  const int b = bh / in.H, h = bh - b * in.H;
  const uint32_t ksn = (uint32_t)in.s[5], vsn = (uint32_t)in.s[8];  // token strides
  int64_t kb0, vb0;
  const int n_k = seq_span(in, b, h, N, 1, kb0);
  seq_span(in, b, h, N, 2, vb0);
  double acc[8];
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] = 0.0;
    mx[e] = 0.f;
  }
  // buffer loads: rows past the sequence read zeros, which change neither
  // the sums nor the absolute maxima, so the row loop has a fixed trip count
  // (the byte offsets stay below 2^32 for rows up to N + kChunk: checked by
  // the caller)
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(k + kb0, (uint32_t)n_k * ksn * 2);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(v + vb0, (uint32_t)n_k * vsn * 2);
  const uint32_t kvoff = 2u * (rg * ksn + 8u * ch), vvoff = 2u * (rg * vsn + 8u * ch);  // row rg, chunk ch
  const int n0 = chunk * kChunk;
#pragma unroll
  for (int i = 0; i < kChunk / kRows; ++i) {
    const uint32_t n = (uint32_t)(n0 + i * kRows);
    const u32x4_t kx = buffer_load16(krs, kvoff, n * ksn * 2);
    const u32x4_t vx = NOV ? u32x4_t{0u, 0u, 0u, 0u} : buffer_load16(vrs, vvoff, n * vsn * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t kb = (uint16_t)(kx[e >> 1] >> (16 * (e & 1)));
      const uint16_t vb = (uint16_t)(vx[e >> 1] >> (16 * (e & 1)));
      acc[e] += (double)in_to_f32<BF16>(kb);
      mx[e] = fmaxf(mx[e], fabsf(in_to_f32<BF16>(vb)));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ssum[rg][ch * 8 + e] = acc[e];
    smax[rg][ch * 8 + e] = mx[e];
  }
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
    float m = 0.f;
    for (int g = 0; g < kRows; ++g) {
      s += ssum[g][tid];
      m = fmaxf(m, smax[g][tid]);
    }
    kpart[((size_t)bh * nchunk + chunk) * D + tid] = s;
    if (!NOV) vpart[((size_t)bh * nchunk + chunk) * D + tid] = m;
  }
}

// ---- finalize: grid (B*H, D/32), 256 threads.  Block (bh, y) owns channels
// 32y .. 32y+31; thread (g, c) adds the partials of chunks g, g + 8, ... of
// channel 32y + c with four independent accumulators (the loads of a thread
// are independent, so they overlap), then the 8 groups combine through LDS.
// The fp64 partials are sums of fp16 / bf16 values, which fp64 adds exactly
// at these magnitudes, so the order of the additions does not change kmean.
template <int D, bool NOV>
__global__ __launch_bounds__(256) void sage8_finalize(const double* __restrict__ kpart, const float* __restrict__ vpart,
                                                    int nchunk, int N, float* __restrict__ kmean,
                                                    float* __restrict__ sv, float* __restrict__ vinv, PrepIn in) {
  constexpr int kG = 8;  // chunk groups of 32 threads
  __shared__ double ssum[kG][32];
  __shared__ float smax[kG][32];
  const int bh = blockIdx.x, cl = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int c = 32 * blockIdx.y + cl;
  const double* kp = kpart + (size_t)bh * nchunk * D + c;
  const float* vp = vpart + (size_t)bh * nchunk * D + c;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  int ch = g;
  for (; ch + 3 * kG < nchunk; ch += 4 * kG) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] += kp[(size_t)(ch + u * kG) * D];
      if (!NOV) m[u] = fmaxf(m[u], vp[(size_t)(ch + u * kG) * D]);
    }
  }
#pragma unroll
  for (int u = 0; u < 3; ++u)  // at most three chunks remain
    if (ch + u * kG < nchunk) {
      s[u] += kp[(size_t)(ch + u * kG) * D];
      if (!NOV) m[u] = fmaxf(m[u], vp[(size_t)(ch + u * kG) * D]);
    }
  ssum[g][cl] = (s[0] + s[1]) + (s[2] + s[3]);
  smax[g][cl] = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  __syncthreads();
  if (g == 0) {
    double t = 0.0;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      t += ssum[i][cl];
      mx = fmaxf(mx, smax[i][cl]);
    }
    int64_t base;
    const int n = seq_span(in, bh / in.H, 0, N, 1, base);
    kmean[(size_t)bh * D + c] = n > 0 ? (float)(t / (double)n) : 0.f;
    if (!NOV) {
      sv[(size_t)bh * D + c] = mx > 0.f ? __fdiv_rn(mx, 448.0f) : 1.0f;
      vinv[(size_t)bh * D + c] = mx > 0.f ? __fdiv_rn(448.0f, mx) : 1.0f;
    }
  }
}

// Block-wide max of a non-negative float over NW waves.
template <int NW>
__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
  return m;
}

__device__ __forceinline__ uint32_t q8(float y, float inv) {
  float r = rintf(y * inv);
  r = fminf(fmaxf(r, -127.f), 127.f);
  return (uint32_t)((int)r & 0xFF);
}

// e4m3 code (round to nearest even) of y * inv, |y * inv| <= 448
__device__ __forceinline__ uint32_t f8(float y, float inv) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(y * inv, 0.f, 0, false) & 0xFF;
}

// ---- quant: grid (nblk, B*H), prep_threads<D>() threads --------------------------------
// QKFP8: Q and smoothed K go to e4m3 with scale amax / 448 per block (the
// FP8-QK variant) instead of INT8 with amax / 127.  NOV: V is not touched.
template <int D, bool BF16, bool QKFP8, bool NOV>
__global__ __launch_bounds__(256) void sage8_quant(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, int N, int np, int nblk,
                                                   const float* __restrict__ kmean, const float* __restrict__ vinv,
                                                   int8_t* __restrict__ qq, int8_t* __restrict__ kq,
                                                   uint8_t* __restrict__ vq, float* __restrict__ sq,
                                                   float* __restrict__ sk, PrepIn in) {
  constexpr int kThreads = prep_threads<D>();
  constexpr int kCpr = D / 8;
  constexpr int kRows = kThreads / kCpr;  // rows per pass
  constexpr int kPass = kQB / kRows;      // passes over the 64-row block
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t vt[D][kQB];  // transposed, permuted V codes
  // heads in reverse order: the column statistics pass ran head by head, so
  // its last heads' K and V are the ones most likely still in the device's
  // last-level cache when this pass reads them again (measured: 3.8% less
  // time at 1x32x32768 and 4x32x4096, d = 128)
  const int blk = blockIdx.x, bh = gridDim.y - 1 - blockIdx.y;
  const int tid = threadIdx.x, ch = tid % kCpr, rg = tid / kCpr;
  const int b = bh / in.H, h = bh - b * in.H;
  int64_t qb0, kb0, vb0;
  const int n_seq = seq_span(in, b, h, N, 0, qb0);
  seq_span(in, b, h, N, 1, kb0);
  seq_span(in, b, h, N, 2, vb0);
  const uint16_t* qh = q + qb0;
  const uint16_t* kh = k + kb0;
  const uint16_t* vh = v + vb0;
  const size_t headp = (size_t)bh * np * D;
  const int n0 = blk * kQB;

  float xq[kPass][8], xk[kPass][8];
  float km[8], vi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    km[e] = kmean[(size_t)bh * D + ch * 8 + e];
    vi[e] = NOV ? 0.f : vinv[(size_t)bh * D + ch * 8 + e];
  }
  float aq = 0.f, ak = 0.f;
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int r = rg + i * kRows, n = n0 + r;
    u32x4_t qx = {0u, 0u, 0u, 0u}, kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (n < n_seq) {
      qx = *(const u32x4_t*)(qh + n * in.s[2] + ch * 8);
      kx = *(const u32x4_t*)(kh + n * in.s[5] + ch * 8);
      if (!NOV) vx = *(const u32x4_t*)(vh + n * in.s[8] + ch * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t qb = (uint16_t)(qx[e >> 1] >> (16 * (e & 1)));
      const uint16_t kb = (uint16_t)(kx[e >> 1] >> (16 * (e & 1)));
      const uint16_t vb = (uint16_t)(vx[e >> 1] >> (16 * (e & 1)));
      xq[i][e] = in_to_f32<BF16>(qb);
      xk[i][e] = n < n_seq ? in_to_f32<BF16>(kb) - km[e] : 0.f;
      aq = fmaxf(aq, fabsf(xq[i][e]));
      ak = fmaxf(ak, fabsf(xk[i][e]));
      // V code, byte-scattered into the transposed tile
      if (!NOV) {
        const float t = in_to_f32<BF16>(vb) * vi[e];
        const uint32_t code = n < n_seq ? (__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.f, 0, false) & 0xFF) : 0u;
        vt[ch * 8 + e][key_pos(r)] = (uint8_t)code;
      }
    }
  }
  aq = block_max<kThreads / 64>(aq, red);
  ak = block_max<kThreads / 64>(ak, red);
  constexpr float kQmax = QKFP8 ? 448.0f : 127.0f;
  const float inv_q = aq > 0.f ? __fdiv_rn(kQmax, aq) : 1.0f;
  const float inv_k = ak > 0.f ? __fdiv_rn(kQmax, ak) : 1.0f;
  if (tid == 0) {
    sq[(size_t)bh * nblk + blk] = aq > 0.f ? __fdiv_rn(aq, kQmax) : 1.0f;
    sk[(size_t)bh * nblk + blk] = ak > 0.f ? __fdiv_rn(ak, kQmax) : 1.0f;
  }
  auto code = [&](float y, float inv) { return QKFP8 ? f8(y, inv) : q8(y, inv); };
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int r = rg + i * kRows, n = n0 + r;
    u32x2_t wq, wk;
    wq[0] = code(xq[i][0], inv_q) | code(xq[i][1], inv_q) << 8 | code(xq[i][2], inv_q) << 16 |
            code(xq[i][3], inv_q) << 24;
    wq[1] = code(xq[i][4], inv_q) | code(xq[i][5], inv_q) << 8 | code(xq[i][6], inv_q) << 16 |
            code(xq[i][7], inv_q) << 24;
    wk[0] = code(xk[i][0], inv_k) | code(xk[i][1], inv_k) << 8 | code(xk[i][2], inv_k) << 16 |
            code(xk[i][3], inv_k) << 24;
    wk[1] = code(xk[i][4], inv_k) | code(xk[i][5], inv_k) << 8 | code(xk[i][6], inv_k) << 16 |
            code(xk[i][7], inv_k) << 24;
    *(u32x2_t*)(qq + headp + (size_t)n * D + ch * 8) = wq;
    *(u32x2_t*)(kq + headp + (size_t)n * D + ch * 8) = wk;
  }
  if (NOV) return;
  __syncthreads();
  // V tile: D rows of 64 bytes, contiguous per block -> 16-byte stores
  uint8_t* vdst = vq + headp + (size_t)blk * kQB * D;
  for (int idx = tid; idx < D * kQB / 16; idx += kThreads) {
    const int row = idx / (kQB / 16), c16 = idx % (kQB / 16);
    *(u32x4_t*)(vdst + row * kQB + c16 * 16) = *(const u32x4_t*)(&vt[row][c16 * 16]);
  }
}

template <int D, bool BF16, bool QKFP8, bool NOV>
hipError_t prep_impl(const void* q, const void* k, const void* v, int B, int H, int N, const int64_t* strides,
                     const int* cu, void* ws, hipStream_t stream) {
  const Sage8Layout L = sage8_layout(B, H, N, D);
  PrepIn in;
  in.H = H;
  in.cu = cu;
  for (int t = 0; t < 3; ++t) {
    in.s[3 * t + 0] = strides ? strides[3 * t + 0] : (int64_t)H * N * D;
    in.s[3 * t + 1] = strides ? strides[3 * t + 1] : (int64_t)N * D;
    in.s[3 * t + 2] = strides ? strides[3 * t + 2] : D;
  }
  char* w = static_cast<char*>(ws);
  const int bh = B * H;
  const int np = L.nblk * kQB;
  hipLaunchKernelGGL((sage8_colstats<D, BF16, NOV>), dim3(L.nchunk, bh), dim3(prep_threads<D>()), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N,
                     reinterpret_cast<double*>(w + L.kpart), reinterpret_cast<float*>(w + L.vpart), L.nchunk, in);
  hipLaunchKernelGGL((sage8_finalize<D, NOV>), dim3(bh, D / 32), dim3(256), 0, stream,
                     reinterpret_cast<const double*>(w + L.kpart), reinterpret_cast<const float*>(w + L.vpart),
                     L.nchunk, N, reinterpret_cast<float*>(w + L.kmean), reinterpret_cast<float*>(w + L.sv),
                     reinterpret_cast<float*>(w + L.vinv), in);
  hipLaunchKernelGGL((sage8_quant<D, BF16, QKFP8, NOV>), dim3(L.nblk, bh), dim3(prep_threads<D>()), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), N, np, L.nblk,
                     reinterpret_cast<const float*>(w + L.kmean), reinterpret_cast<const float*>(w + L.vinv),
                     reinterpret_cast<int8_t*>(w + L.qq), reinterpret_cast<int8_t*>(w + L.kq),
                     reinterpret_cast<uint8_t*>(w + L.vq), reinterpret_cast<float*>(w + L.sq),
                     reinterpret_cast<float*>(w + L.sk), in);
  return hipGetLastError();
}

// =========================================================================
// Forward
// =========================================================================

struct Fwd8Params {
  const int8_t* qq;
  const int8_t* kq;
  const uint8_t* vq;
  const float* sq;
  const float* sv;
  const float* kmean;
  void* o;
  float* lse;
  int N, np, nblk;
  int nq;      // query tiles per head
  int nbh;     // B*H
  int nb;      // ceil(N/64), bias blocks per side
  int ntiles;  // B*H*nq
  float c;     // scale * log2(e), never 0
  int out_kind;
  int H;
  int64_t os[3];  // element strides (batch, head, token) of O
  int lpt;        // causal: items heaviest first across the heads (work_queue)
  const int* cu;  // VARLEN: packed sequences, device int32 [B+1]
};

constexpr int kNW8 = 4;                // waves per workgroup
constexpr int kBM8 = 32 * kNW8;        // queries per workgroup
constexpr int kThreads8 = 64 * kNW8;

// K tile: 64 keys x D bytes; V tile: D rows (channels) x 64 bytes, the
// block's keys in operand order.  Both are unpadded and filled straight from
// global memory by 16-byte buffer loads into LDS: one instruction writes the
// 64 consecutive 16-byte chunks of a wave, so the layout is chosen by which
// global chunk each lane fetches.  Within a row the 16-byte chunks are
// rotated by a per-row amount (k_rot, v_rot), so the 16-byte operand reads
// of 16 consecutive rows at one logical chunk fall on distinct banks
// (rows of 128 bytes: banks repeat every 2 rows, so the rotation is row/2
// mod 8; 64 bytes: every 4 rows, row/4 mod 4; 96 bytes: rows 8 apart share
// banks, row/8 mod 2).  The rotation depends on the row's low bits only, so
// rows 32 apart (the two 32-key halves) rotate alike.
template <int D>
struct Fwd8Smem {
  static constexpr int kKC = D / 16;  // 16-byte chunks per K row
  static constexpr int kKTile = kQB * D;
  static constexpr int kVTile = D * kQB;
  static constexpr int kBytes = 2 * (kKTile + kVTile);
};
// rotation of K row r (mod kKC) and of V row r (mod 4)
template <int D>
__device__ __forceinline__ int k_rot(int r) {
  return D == 128 ? (r >> 1) & 7 : D == 64 ? (r >> 2) & 3 : (r >> 3) & 1;
}
__device__ __forceinline__ int v_rot(int r) { return (r >> 2) & 3; }
// LDS byte offset of logical chunk c of K row r
template <int D>
__device__ __forceinline__ uint32_t k_pos(int r, int c) {
  constexpr int C = D / 16;
  const int x = c + k_rot<D>(r);
  return (uint32_t)(r * D + 16 * (x >= C ? x - C : x));
}
__device__ __forceinline__ uint32_t v_pos(int r, int c) { return (uint32_t)(r * kQB + 16 * ((c + v_rot(r)) & 3)); }



// (the first conversion's high half is overwritten by the second, so any
// register serves as its old value: a's bits, which need no extra move)
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_uint(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// BIAS: a block bias is given (adds the block-sparse skip).  The bias and
// the K block scales come as their own restrict arguments: their reads,
// uniform and never written by the kernel, then compile to scalar loads,
// which do not share the in-order vector-load counter with the K/V prefetch.
// QKFP8: Qq and Kq hold e4m3 codes (the FP8-QK variant) and S^T = Kq Qq^T
// runs on the FP8 32x32x64 instruction, with no offset on the accumulators.
// VARLEN: batch entry b is the packed sequence of tokens cu[b] .. cu[b+1]-1
// (its workspace slot prepared from that sequence alone): its length bounds
// the keys and rows, its rows of O start at token cu[b], and with BIAS its
// blocks are those of [b, h] of the bias, counted from that token.
template <int D, bool CAUSAL, bool BIAS, bool QKFP8, bool VARLEN>
__global__ __launch_bounds__(kThreads8, 3) void fwd8_kernel(Fwd8Params p, const float* __restrict__ bias,
                                                            const float* __restrict__ sk) {
  using S = Fwd8Smem<D>;
  constexpr int kKTile = S::kKTile, kVTile = S::kVTile, kKC = S::kKC;
  constexpr int kDT = D / 32;  // 32-row tiles of O^T
  constexpr int kKS = D / 32;  // 16-byte Q chunks per lane (INT8: one per 32-deep k-step;
                               // FP8: two per 64-deep k-step)
  // FP8: D / 64 full 64-deep steps; at d = 96 a last step covers channels
  // 64..95 with half of each lane's 32 operand bytes zero (kHalf8)
  constexpr int kFull8 = D / 64;
  constexpr bool kHalf8 = QKFP8 && D % 64 != 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::kBytes];
  uint8_t* const kl = smem;               // 2 K tiles
  uint8_t* const vl = smem + 2 * kKTile;  // 2 V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Loop over (b, h, query tile) work items (work_queue: per-XCD queues,
  // balanced heavy-first order when the grid is persistent).
  const WorkQueue wq = work_queue(p.nbh, p.nq, p.lpt);
  for (int round = 0;; ++round) {
  int bh, tq;
  if (!work_item(wq, round, p.nq, bh, tq)) break;
  const int qt = CAUSAL ? p.nq - 1 - tq : tq;  // heaviest tiles first
  const int N = VARLEN ? max(0, min(p.cu[bh / p.H + 1] - p.cu[bh / p.H], p.N)) : p.N;
  const int q0 = qt * kBM8;
  if (VARLEN && q0 >= N) continue;  // past a shorter sequence's end
  const int qw0 = q0 + wave * 32;
  const size_t headp = (size_t)bh * p.np * D;
  const int8_t* __restrict__ Qq = p.qq + headp;
  const int8_t* __restrict__ Kq = p.kq + headp;
  const uint8_t* __restrict__ Vq = p.vq + headp;

  // Qq^T as the B operand: lane holds Qq[qw0 + l32][32kk + 16hf .. +15]
  // (INT8, and the half FP8 step), or bytes 64(kk/2) + 32hf + 16(kk%2) ..
  // +15 (a full FP8 step, 32 bytes per 64-deep step); rows up to the padded
  // length are valid zero codes.
  u32x4_t qf[kKS];
#pragma unroll
  for (int kk = 0; kk < kKS; ++kk) {
    const int col = (QKFP8 && kk < 2 * kFull8) ? 64 * (kk >> 1) + 32 * hf + 16 * (kk & 1) : 32 * kk + 16 * hf;
    qf[kk] = *(const u32x4_t*)(Qq + (size_t)(qw0 + l32) * D + col);
  }
  const float sqw = p.sq[(size_t)bh * p.nblk + qw0 / kQB];

  const int kend = CAUSAL ? min(N, q0 + kBM8) : N;
  const int nkb = (kend + kQB - 1) / kQB;
  const int wave_last = CAUSAL ? min(nkb - 1, qw0 / kQB) : nkb - 1;
  const bool wave_has_rows = qw0 < N;

  // loader: K tile 64*D bytes and V tile D*64 bytes, 16-byte chunks written
  // straight into LDS.  Round i of wave w fills LDS chunks i*256 + 64w ..
  // +63 of a tile; lane l fetches the global chunk that belongs at LDS chunk
  // i*256 + tid (row p / kKC, inverse rotation for K; row p / 4 for V).
  // The per-lane byte offsets inside a block are fixed; the block offset
  // kb*64*D is uniform (buffer loads: base and size in scalar registers).
  constexpr int kChunks = kQB * D / 16;  // 16-byte chunks per tile
  constexpr int kNld = (kChunks + kThreads8 - 1) / kThreads8;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kq, (uint32_t)p.np * D);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vq, (uint32_t)p.np * D);
  uint32_t kvo[kNld], vvo[kNld];
#pragma unroll
  for (int i = 0; i < kNld; ++i) {
    const int pc = i * kThreads8 + tid;
    const int kr = pc / kKC, kp = pc % kKC;
    int kc = kp - k_rot<D>(kr);
    kc = kc < 0 ? kc + kKC : kc;
    kvo[i] = (uint32_t)(kr * D + 16 * kc);
    const int vr = pc / 4;
    vvo[i] = (uint32_t)(vr * kQB + 16 * ((pc - v_rot(vr)) & 3));
  }
  auto load_kv = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < kNld; ++i) {
      if (kChunks % kThreads8 != 0 && i * kThreads8 + wave * 64 >= kChunks) continue;  // wave-uniform
      const int c0 = 16 * (i * kThreads8 + wave * 64);
      buffer_load16_lds(krs, kl + buf * kKTile + c0, kvo[i], kb * kQB * D);
      buffer_load16_lds(vrs, vl + buf * kVTile + c0, vvo[i], kb * kQB * D);
    }
  };
  // operand read offsets inside a tile: K rows 32T + l32 at the logical
  // chunks of k-step kk (INT8 and the half FP8 step: 2kk + hf; a full FP8
  // step: 4kk + 2hf and +1), V rows
  // 32dt + l32 at chunks 2hf and 2hf + 1
  // (row 32 + l32 rotates like row l32: the second 32-row half is 32*D
  // bytes further)
  uint32_t ko[kKS];
#pragma unroll
  for (int kk = 0; kk < kKS; ++kk)
    ko[kk] = (QKFP8 && kk < 2 * kFull8) ? k_pos<D>(l32, 4 * (kk >> 1) + 2 * hf + (kk & 1))
                                         : k_pos<D>(l32, 2 * kk + hf);
  auto kofs = [&](int T, int kk) -> uint32_t { return ko[kk] + 32 * T * D; };
  const uint32_t vo0 = v_pos(l32, 2 * hf), vo1 = v_pos(l32, 2 * hf + 1);

  f32x16_t o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) o[dt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const unsigned long long magic_v = magic_pair();  // (loop-invariant: see magic_tile)
  const float c = p.c;
  const bool pos = c > 0.f;
  const float sent = pos ? -INFINITY : INFINITY;
  const float* skrow = sk + (size_t)bh * p.nblk;  // K block scales (scalar reads)

  // ---- block-sparse skip (with a bias only): a key block gated off (bias
  // -inf) for every query block of this tile is neither loaded nor computed;
  // a wave skips blocks gated off for its own query block.  The bias values
  // a step needs are read a step ahead.
  constexpr int kRows = kBM8 / kQB;  // 64-query blocks per tile
  const int rw = wave * 32 / kQB;    // this wave's query block in the tile
  BlockGate<kRows> gate(BIAS ? bias + (size_t)bh * p.nb * p.nb : bias, p.nb, q0 / kQB, nkb, rw);

  // ---- one key block: the next active block (jn) loads while block jc,
  // staged in buffer buf, computes; braw is this wave's bias of block jc
  auto step = [&](int jc, int jn, int buf, float braw) {
    const bool more = jn < nkb;
    if (more) load_kv(jn, buf ^ 1);
    if (wave_has_rows && jc <= wave_last && (!BIAS || braw != -INFINITY)) {
      f32x16_t s[2];
      if constexpr (QKFP8) {
        // ---- S^T = Kq Qq^T in fp32 from e4m3 codes (A: 32 bytes of a K
        // row per 64-deep step, B: the matching 32 bytes of the Q row)
        const uint8_t* Ks = kl + buf * kKTile;
        s[0] = s[1] = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < kFull8; ++kk)
#pragma unroll
          for (int T = 0; T < 2; ++T) {
            const u32x4_t a0 = *(const u32x4_t*)(Ks + kofs(T, 2 * kk));
            const u32x4_t a1 = *(const u32x4_t*)(Ks + kofs(T, 2 * kk + 1));
            const u32x4_t b0 = qf[2 * kk], b1 = qf[2 * kk + 1];
            const i32x8_t aop = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            const i32x8_t bop = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                 (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            s[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, s[T], 0, 0, 0, 0, 0, 0);
          }
        if constexpr (kHalf8) {
          // channels 64..95: lane half hf gives channels 64 + 16hf .. +15 as
          // its k-slice's first 16 bytes, zeros (e4m3 +0) as the other 16, in
          // both operands, so the padding adds exact zeros
          const u32x4_t b0 = qf[2 * kFull8];
#pragma unroll
          for (int T = 0; T < 2; ++T) {
            const u32x4_t a0 = *(const u32x4_t*)(Ks + kofs(T, 2 * kFull8));
            const i32x8_t aop = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], 0, 0, 0, 0};
            const i32x8_t bop = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], 0, 0, 0, 0};
            s[T] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, s[T], 0, 0, 0, 0, 0, 0);
          }
        }
      } else {
        // ---- S^T = Kq Qq^T on top of the offset, exact
        const uint8_t* Ks = kl + buf * kKTile;
        i32x16_t si[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) si[T] = magic_tile(magic_v);
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk)
#pragma unroll
          for (int T = 0; T < 2; ++T) {
            const u32x4_t a = *(const u32x4_t*)(Ks + kofs(T, kk));
            si[T] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                                          __builtin_bit_cast(i32x4_t, qf[kk]), si[T], 0, 0, 0);
          }
#pragma unroll
        for (int T = 0; T < 2; ++T) s[T] = __builtin_bit_cast(f32x16_t, si[T]);
      }
      // INT8: s = kMagic + S_int; base 2: t = S_int * f + bias*log2(e)
      //       = s * f + g,  g = bias*log2(e) - kMagic * f.  FP8: s = S, g = bias*log2(e).
      const float f = (sqw * skrow[jc]) * c;
      if ((CAUSAL && jc == wave_last) || (jc + 1) * kQB > N) {
        const int kb0 = jc * kQB, qi = qw0 + l32;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb0 + 32 * T + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool m = (CAUSAL && key > qi) || key >= N;
            s[T][r] = m ? sent : s[T][r];
          }
      }
      const float bl = BIAS ? braw * kLog2e : 0.f;
      const float g = QKFP8 ? bl : fmaf(-kMagic, f, bl);
      // (three-input max / min: one instruction per two scores)
      float a0;
      if (pos) {
        a0 = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fmaxf(fmaxf(a0, s[0][r]), s[1][r]);
        a0 = xor32_max(a0);
      } else {
        a0 = fminf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fminf(fminf(a0, s[0][r]), s[1][r]);
        a0 = xor32_min(a0);
      }
      const float m_blk = (a0 == sent) ? -INFINITY : fmaf(a0, f, g);
      const bool need = m_blk > m_run + kTau8;
      if (__any(need)) {
        const float m_new = need ? m_blk : m_run;
        // rows that keep their maximum keep alpha = 1 (also a row still at -inf)
        const float alpha = need ? exp2_approx(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      const float kc = (g - ((m_run == -INFINITY) ? 0.f : m_run)) + kPlog;
      // ---- P^ in e4m3 as the B operand (byte e = 16T + r); the row sum
      // adds the fp32 values before quantisation
      uint32_t pw[8];
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int T = w >> 2, r0 = 4 * (w & 3);
        const float e0 = exp2_approx(fmaf(s[T][r0], f, kc)), e1 = exp2_approx(fmaf(s[T][r0 + 1], f, kc));
        const float e2 = exp2_approx(fmaf(s[T][r0 + 2], f, kc)), e3 = exp2_approx(fmaf(s[T][r0 + 3], f, kc));
        lsum += (e0 + e1) + (e2 + e3);
        pw[w] = pack_fp8x4(e0, e1, e2, e3);
      }
      l_run += lsum;
      const i32x8_t bop = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                           (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
      // ---- O^T += Vq^T P^T over the 64 keys (one FP8 instruction per d tile)
      const uint8_t* Vs = vl + buf * kVTile;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const u32x4_t a0v = *(const u32x4_t*)(Vs + 32 * dt * kQB + vo0);
        const u32x4_t a1v = *(const u32x4_t*)(Vs + 32 * dt * kQB + vo1);
        const i32x8_t aop = {(int)a0v[0], (int)a0v[1], (int)a0v[2], (int)a0v[3],
                             (int)a1v[0], (int)a1v[1], (int)a1v[2], (int)a1v[3]};
        o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, o[dt], 0, 0, 0, 0, 0, 0);
      }
    }
    // the next block's loads into LDS are complete before any wave reads them
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  // The first block is staged unconditionally (a valid block even when every
  // block is gated off), after the Q loads (the scheduling barrier): its wait
  // for the global loads then also covers Q, so no wait on Q lands inside the
  // loop, where (the counter being in order) it would also wait for the next
  // block's prefetch every iteration.
  int j0 = 0;
  if constexpr (BIAS) j0 = gate.first();
  __builtin_amdgcn_sched_barrier(0);
  load_kv(min(j0, nkb - 1), 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if constexpr (BIAS) {
    // the wave's bias of block jc, then the next visited block (a wave whose
    // query block is past the last one has no rows and ignores its bias)
    int jc = j0;
    float wb = jc < nkb ? gate.wave_bias(jc) : -INFINITY;
    int jn = gate.next();
    for (int buf = 0; jc < nkb; buf ^= 1) {
      const float wb_next = jn < nkb ? gate.wave_bias(jn) : -INFINITY;
      step(jc, jn, buf, wb);
      const int jnn = gate.next();
      jc = jn;
      jn = jnn;
      wb = wb_next;
    }
  } else {
    for (int j = 0; j < nkb; ++j) step(j, j + 1, j & 1, 0.f);
  }

  // ---- epilogue: O = acc * sv[d] / l; LSE = (m + log2 l - kPlog) ln 2 plus
  // the shift scale * sq * (Qq . kmean) that the centring of K removed from
  // every score of the row (O does not depend on it)
  const float l_tot = xor32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int qi = qw0 + l32;
  if (p.lse != nullptr) {
    // the Q codes are read again here rather than kept from the prologue,
    // so no register has to survive the main loop for this
    const float* kmh = p.kmean + (size_t)bh * D;
    float dot = 0.f;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      const u32x4_t qc = *(const u32x4_t*)(Qq + (size_t)(qw0 + l32) * D + 32 * kk + 16 * hf);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float qv = QKFP8 ? __builtin_amdgcn_cvt_f32_fp8((int)(qc[e >> 2] >> (8 * (e & 3))), 0)
                               : (float)(int)(int8_t)(qc[e >> 2] >> (8 * (e & 3)));
        dot = fmaf(qv, kmh[32 * kk + 16 * hf + e], dot);
      }
    }
    dot = xor32_sum(dot);
    if (hf == 0 && qi < N)
      p.lse[(size_t)bh * p.N + qi] =
          l_tot > 0.f ? (m_run + __log2f(l_tot) - kPlog + c * (sqw * dot)) * kLn2 : -INFINITY;
  }
  // lane (l32, hf) holds d = 32dt + 8g + 4hf + u of query qi: 16-byte (fp32)
  // or 8-byte (fp16 / bf16) stores straight from the accumulators
  const float* svh = p.sv + (size_t)bh * D;
  const int ob = bh / p.H;
  const int64_t orow = (VARLEN ? (int64_t)p.cu[ob] * p.os[2] : ob * p.os[0]) + (bh - ob * p.H) * p.os[1] +
                       (int64_t)qi * p.os[2];
  if (qi < N)
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hf;
      const f32x4_t svv = *(const f32x4_t*)(svh + d);
      const f32x4_t w = {o[dt][4 * g] * svv[0] * inv, o[dt][4 * g + 1] * svv[1] * inv,
                         o[dt][4 * g + 2] * svv[2] * inv, o[dt][4 * g + 3] * svv[3] * inv};
      if (p.out_kind == kOutF32) {
        *(f32x4_t*)(reinterpret_cast<float*>(p.o) + orow + d) = w;
      } else if (p.out_kind == kOutBF16) {
        *(u32x2_t*)(reinterpret_cast<uint16_t*>(p.o) + orow + d) = u32x2_t{pack2<true>(w[0], w[1]), pack2<true>(w[2], w[3])};
      } else {
        *(u32x2_t*)(reinterpret_cast<uint16_t*>(p.o) + orow + d) = u32x2_t{pack2<false>(w[0], w[1]), pack2<false>(w[2], w[3])};
      }
    }
  }  // work items
}

template <int D, bool CAUSAL, bool BIAS, bool QKFP8, bool VARLEN = false>
hipError_t fwd8_impl(const void* ws, const FwdArgs& a, hipStream_t stream) {
  const Sage8Layout L = sage8_layout(a.B, a.H, a.N, D);
  const char* w = static_cast<const char*>(ws);
  Fwd8Params p;
  p.qq = reinterpret_cast<const int8_t*>(w + L.qq);
  p.kq = reinterpret_cast<const int8_t*>(w + L.kq);
  p.vq = reinterpret_cast<const uint8_t*>(w + L.vq);
  p.sq = reinterpret_cast<const float*>(w + L.sq);
  p.sv = reinterpret_cast<const float*>(w + L.sv);
  p.kmean = reinterpret_cast<const float*>(w + L.kmean);
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.nblk = L.nblk;
  p.np = L.nblk * kQB;
  p.nq = (a.N + kBM8 - 1) / kBM8;
  p.nb = (a.N + 63) / 64;
  p.nbh = a.B * a.H;
  p.ntiles = a.B * a.H * p.nq;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  if (p.c == 0.f) p.c = 1.17549435e-38f;
  p.out_kind = a.out_kind;
  p.H = a.H;
  p.os[0] = a.general ? a.strides[9] : (int64_t)a.H * a.N * D;
  p.os[1] = a.general ? a.strides[10] : (int64_t)a.N * D;
  p.os[2] = a.general ? a.strides[11] : D;
  p.cu = a.cu;
  // One workgroup per tile.  Causal tiles differ in cost: with few items per
  // resident slot they start heaviest first across the heads (measured +10%
  // at 4x32x4096 over the persistent balanced order, which with 5.3 rounds
  // per slot leaves the last rounds uneven), else head by head (L2 sharing).
  const int grid = p.ntiles;
  p.lpt = !CAUSAL ? 0
                  : sorted_order(reinterpret_cast<const void*>(&fwd8_kernel<D, CAUSAL, BIAS, QKFP8, VARLEN>),
                                 kThreads8, p.nbh, p.nq);
  hipLaunchKernelGGL((fwd8_kernel<D, CAUSAL, BIAS, QKFP8, VARLEN>), dim3(grid), dim3(kThreads8), 0, stream, p, a.bias,
                     reinterpret_cast<const float*>(w + L.sk));
  return hipGetLastError();
}

}  // namespace

namespace {
template <bool QKFP8, bool NOV>
hipError_t prep_q(const void* q, const void* k, const void* v, bool bf16, int B, int H, int N, int d,
                  const int64_t* st, const int* cu, void* ws, hipStream_t stream) {
  if (d == 64) return bf16 ? prep_impl<64, true, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream)
                           : prep_impl<64, false, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream);
  if (d == 96) return bf16 ? prep_impl<96, true, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream)
                           : prep_impl<96, false, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream);
  return bf16 ? prep_impl<128, true, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream)
              : prep_impl<128, false, QKFP8, NOV>(q, k, v, B, H, N, st, cu, ws, stream);
}
}  // namespace

hipError_t launch_sage8_prep(const void* q, const void* k, const void* v, bool bf16, int B, int H, int N, int d,
                             const int64_t* strides, const int* cu, void* ws, hipStream_t stream, int fmt) {
  if (fmt == kPrepFp8) return prep_q<true, false>(q, k, v, bf16, B, H, N, d, strides, cu, ws, stream);
  if (fmt == kPrepInt8NoV) return prep_q<false, true>(q, k, v, bf16, B, H, N, d, strides, cu, ws, stream);
  return prep_q<false, false>(q, k, v, bf16, B, H, N, d, strides, cu, ws, stream);
}

namespace {
template <int D, bool QKFP8>
hipError_t fwd8_d(const void* ws, const FwdArgs& a, hipStream_t stream) {
  // packed sequences: the bias blocks of sequence b are [b, h] of the
  // [B,H,nb,nb] bias, counted from its first token
  if (a.cu && a.bias) return a.causal ? fwd8_impl<D, true, true, QKFP8, true>(ws, a, stream)
                                      : fwd8_impl<D, false, true, QKFP8, true>(ws, a, stream);
  if (a.cu) return a.causal ? fwd8_impl<D, true, false, QKFP8, true>(ws, a, stream)
                            : fwd8_impl<D, false, false, QKFP8, true>(ws, a, stream);
  if (a.bias) return a.causal ? fwd8_impl<D, true, true, QKFP8>(ws, a, stream)
                              : fwd8_impl<D, false, true, QKFP8>(ws, a, stream);
  return a.causal ? fwd8_impl<D, true, false, QKFP8>(ws, a, stream) : fwd8_impl<D, false, false, QKFP8>(ws, a, stream);
}
}  // namespace

hipError_t launch_fwd_sage8(const void* ws, const FwdArgs& a, hipStream_t stream, bool qk_fp8) {
  if (qk_fp8) {
    if (a.d == 64) return fwd8_d<64, true>(ws, a, stream);
    if (a.d == 96) return fwd8_d<96, true>(ws, a, stream);
    return fwd8_d<128, true>(ws, a, stream);
  }
  if (a.d == 64) return fwd8_d<64, false>(ws, a, stream);
  if (a.d == 96) return fwd8_d<96, false>(ws, a, stream);
  return fwd8_d<128, false>(ws, a, stream);
}

}  // namespace attn
