// attn_bwd.hip -- backward of the fused attention (fp16/bf16) on gfx950: the
// row statistic D = rowsum(dO * O) and the query-side kernel (dQ).
//
// The backward recomputes the score tile from Q, K and the forward's LSE
// instead of storing it (page 3, "FlashAttention", the glossary paragraph:
// the backward pass recomputes the cheap intermediates; page 4,
// "FlashAttention (TR)": tiling and the single fused kernel).  With
// P = exp(s - LSE) the exact probabilities, for a loss L and dO = dL/dO:
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O),
//   dQ = scale * dS K,   dK = scale * dS^T Q,   dbias = block sums of dS
// (the bias enters the scores unscaled, as the log-form gate of page 5,
// "SAS").  This file computes D and dQ; the key side (dK, dV, dbias) is in
// attn_bwd_kv.hip.
//
// dQ kernel: a workgroup of 8 waves x 32 queries per (b, h, query tile),
// the layout of the forward kernel.  Per 64-key block, in halves of 32 keys:
//   S^T = K Q^T and dP^T = V dO^T (32x32x16 MFMA; K and V rows from LDS,
//       Q and dO rows held in registers as the B operands);
//   P^T = exp2(c S^T + bias*log2e - LSE*log2e), dS^T = P^T (dP^T - D),
//       one query per lane column, so LSE and D are one value per lane;
//   dQ^T += K^T dS^T: dS^T goes from the accumulator registers straight into
//       the B operand, K^T comes from the row-major K tile by the
//       transposing LDS read (the forward's P V step with K in place of V).
// A block is one straight-line body (the scores of both halves first, then
// each half's dS next to the other half's products); the mask is a second
// copy of that body, used on the blocks past the start of the workgroup's
// causal diagonal and on a ragged last block.
#include "attn_common.hpp"
#include "attn_internal.hpp"

#include <type_traits>

#include <math.h>

namespace attn {
namespace {

constexpr int kBN = 64;  // keys per block

// threads per row of the D kernel: D/8 rounded up to a power of two, so a
// row's threads are consecutive lanes of one wave (d = 96: 12 chunks on 16
// threads, the last 4 adding nothing)
template <int D>
constexpr int delta_tpr() { return D <= 64 ? 8 : 16; }

// ---- D = rowsum(dO * O) in fp32, one row per delta_tpr<D>() consecutive
// threads; O in the input dtype or (OF32) fp32 ---------------------------------
template <int D, bool BF16, bool OF32>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
  constexpr int kCpr = D / 8;               // 8-element chunks per row (8, 12 or 16)
  constexpr int kTpr = delta_tpr<D>();      // threads per row
  constexpr int kRows = 256 / kTpr;         // rows per workgroup
  static_assert(kCpr <= kTpr && (kTpr & (kTpr - 1)) == 0, "row threads");
  const int tid = threadIdx.x, ch = tid % kTpr;
  const int64_t row = (int64_t)blockIdx.x * kRows + tid / kTpr;
  float acc = 0.f;
  if (row < rows && ch < kCpr) {
    const u32x4_t b = *(const u32x4_t*)(dout + row * D + ch * 8);
    float ov[8];
    if constexpr (OF32) {
      const f32x4_t a0 = *(const f32x4_t*)(static_cast<const float*>(o) + row * D + ch * 8);
      const f32x4_t a1 = *(const f32x4_t*)(static_cast<const float*>(o) + row * D + ch * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = a0[e];
        ov[4 + e] = a1[e];
      }
    } else {
      const u32x4_t a = *(const u32x4_t*)(static_cast<const uint16_t*>(o) + row * D + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = in_to_f32<BF16>((uint16_t)(a[e >> 1] >> (16 * (e & 1))));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(ov[e], in_to_f32<BF16>((uint16_t)(b[e >> 1] >> (16 * (e & 1)))), acc);
  }
  // the kTpr threads of a row are consecutive lanes of one wave
#pragma unroll
  for (int off = kTpr / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && ch == 0) delta[row] = acc;
}

struct BwdQParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  void* dq;
  int N;
  int nq;   // query tiles per head
  int nbh;  // B*H
  int nb;   // ceil(N/64)
  float c;  // scale * log2(e), never 0
  float scale;
  int out_f32;
  int lpt;  // causal: items heaviest first across the heads (work_queue)
};

template <int D, bool BF16, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdQParams p, const float* __restrict__ bias) {
  constexpr int NW = 8, kWQ = 32, kBM = NW * kWQ, kThreads = 64 * NW;
  constexpr int kKS = D / 16;  // k-steps over d
  constexpr int kDT = D / 32;  // 32-row tiles of dQ^T
  constexpr int kCpr = D / 8;  // 16-byte chunks per row
  // K rows are read both ways (rows for the scores, transposing reads for
  // dQ); the padding is the fastest of a sweep of 8 to 40 elements at
  // d = 128, faster than 32 at d = 64, and 16 beats 24 and 40 at d = 96.
  // V rows are read as rows only.
  constexpr int kKRow = D == 96 ? D + 16 : D + 24;
  constexpr int kVRow = D + 8;
  constexpr int kKTile = kBN * kKRow, kVTile = kBN * kVRow;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (kKTile + kVTile)];
  uint16_t* const kl = smem;
  uint16_t* const vl = smem + 2 * kKTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int N = p.N;

  const WorkQueue wq = work_queue(p.nbh, p.nq, p.lpt);
  for (int round = 0;; ++round) {
  int bh, tq;
  if (!work_item(wq, round, p.nq, bh, tq)) break;
  const int qt = CAUSAL ? p.nq - 1 - tq : tq;  // heaviest tiles first
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kWQ;
  const size_t head = (size_t)bh * N * D;
  const int qi = qw0 + l32;
  const int qrow = min(qi, N - 1);  // rows past N compute garbage that is never stored

  // Q and dO rows as B operands: lane holds row qi, d = 16kk + 8hf .. +7
  u32x4_t qf[kKS], df[kKS];
#pragma unroll
  for (int kk = 0; kk < kKS; ++kk) {
    qf[kk] = *(const u32x4_t*)(p.q + head + (size_t)qrow * D + 16 * kk + 8 * hf);
    df[kk] = *(const u32x4_t*)(p.dout + head + (size_t)qrow * D + 16 * kk + 8 * hf);
  }
  const float lse = p.lse[(size_t)bh * N + qrow];
  // a row with no visible key (LSE = -inf) has P = 0 everywhere
  const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
  const float dlt = p.delta[(size_t)bh * N + qrow];

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
  const int nkb = (kend + kBN - 1) / kBN;
  const int wave_last = CAUSAL ? min(nkb - 1, qw0 / kBN) : nkb - 1;
  const bool wave_has_rows = qw0 < N;
  const float* bias_row = HAS_BIAS ? bias + ((size_t)bh * p.nb + min(qw0 / kBN, p.nb - 1)) * p.nb : nullptr;

  // loader (as in the forward): chunk tid + i*threads of a block at byte
  // 16*tid + kb*64*D*2 + 16*i*threads; rows past N read zeros.  At d = 96 a
  // block is 768 chunks, so the second round covers only the first 256
  // threads (the others' loads are never stored).
  constexpr int kChunks = kBN * kCpr;
  constexpr int kNst = (kChunks + kThreads - 1) / kThreads;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(p.k + head, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(p.v + head, (uint32_t)N * D * 2);
  const uint32_t voff = 16u * tid;
  u32x4_t kst[kNst], vst[kNst];
  auto load_kv = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      kst[i] = buffer_load16(krs, voff, kb * kBN * D * 2 + 16 * i * kThreads);
      vst[i] = buffer_load16(vrs, voff, kb * kBN * D * 2 + 16 * i * kThreads);
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCpr, ch = idx % kCpr;
      if (kChunks % kThreads != 0 && idx >= kChunks) continue;
      *(u32x4_t*)(kl + buf * kKTile + row * kKRow + ch * 8) = kst[i];
      *(u32x4_t*)(vl + buf * kVTile + row * kVRow + ch * 8) = vst[i];
    }
  };

  f32x16_t acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16_t{};
  const float c = p.c;

  // transposing-read coordinates (K^T operand): this lane addresses row
  // 16kk + tkey (and +8) at column 32dt + tcol
  const int g16 = lane >> 4, t16 = lane & 15;
  const int tkey = 4 * hf + (t16 >> 2);
  const int tcol = 16 * (g16 & 1) + 4 * (t16 & 3);

  // S^T and dP^T of key half T (32 keys) of staged block buf
  auto scores = [&](int buf, int T, f32x16_t& s, f32x16_t& dp) {
    const uint16_t* Ks = kl + buf * kKTile + (32 * T + l32) * kKRow + 8 * hf;
    const uint16_t* Vs = vl + buf * kVTile + (32 * T + l32) * kVRow + 8 * hf;
    s = f32x16_t{};
    dp = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      s = mfma32x32x16<BF16>(*(const u32x4_t*)(Ks + 16 * kk), qf[kk], s);
      dp = mfma32x32x16<BF16>(*(const u32x4_t*)(Vs + 16 * kk), df[kk], dp);
    }
  };
  // dS^T of half T in the register order of the B operand: pb[t] holds keys
  // 32T + 16t + 4hf + {0..3} and 32T + 16t + 8 + 4hf + {0..3}.  MASK: keys
  // the causal mask or the end of the sequence hide get dS = 0.
  auto probs = [&](auto mask_tag, int j, int T, float off, const f32x16_t& s, const f32x16_t& dp,
                   u32x4_t (&pb)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 8 * t + e + u;
          const float pr = exp2_approx(fmaf(s[r], c, off));
          ds[u] = pr * (dp[r] - dlt);
          if constexpr (MASK) {
            const int key = j * kBN + 32 * T + 8 * (r >> 2) + 4 * hf + (r & 3);
            if ((CAUSAL && key > qi) || key >= N) ds[u] = 0.f;
          }
        }
        pb[t][e >> 1] = pack2<BF16>(ds[0], ds[1]);
      }
  };
  // dQ^T += K^T dS^T over half T (K^T by the transposing LDS read)
  auto accum = [&](int buf, int T, const u32x4_t (&pb)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* kt = kl + buf * kKTile + (32 * T + 16 * t + tkey) * kKRow + tcol;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const u32x2_t lo = lds_read_tr16(kt + 32 * dt);
        const u32x2_t hi = lds_read_tr16(kt + 32 * dt + 8 * kKRow);
        const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
        acc[dt] = mfma32x32x16<BF16>(a, pb[t], acc[dt]);
      }
    }
  };
  // One staged block of 64 keys in one straight-line body: the scores of
  // both halves first, then each half's softmax next to the other half's
  // products.  MASK: the body for blocks the causal diagonal or the end of
  // the sequence cut through.
  auto block = [&](auto mask_tag, int j, int buf) {
    const float bl = HAS_BIAS ? bias_row[j] * kLog2e : 0.f;
    const float off = bl - lse2;  // exponent of P: c*S + off
    f32x16_t s0, dp0, s1, dp1;
    u32x4_t pb0[2], pb1[2];
    scores(buf, 0, s0, dp0);
    scores(buf, 1, s1, dp1);
    probs(mask_tag, j, 0, off, s0, dp0, pb0);
    accum(buf, 0, pb0);
    probs(mask_tag, j, 1, off, s1, dp1, pb1);
    accum(buf, 1, pb1);
  };

  __builtin_amdgcn_sched_barrier(0);
  load_kv(0);
  store_kv(0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  // The key loop in two segments, each with one body: the blocks before the
  // workgroup's causal diagonal (unmasked; all of them without a causal
  // mask, but a ragged last block), then the rest (masked).  The bodies
  // switch only between the segments.
  const int jm = CAUSAL ? min(q0 / kBN, nkb) : (N % kBN != 0 ? nkb - 1 : nkb);
  auto segment = [&](auto mask_tag, int jb, int je) {
    for (int j = jb; j < je; ++j) {
      const bool more = j + 1 < nkb;
      if (more) load_kv(j + 1);
      if (wave_has_rows && j <= wave_last && (!HAS_BIAS || bias_row[j] != -INFINITY)) block(mask_tag, j, j & 1);
      if (more) store_kv((j + 1) & 1);
      __syncthreads();
    }
  };
  segment(std::false_type{}, 0, jm);
  segment(std::true_type{}, jm, nkb);

  // ---- epilogue: dQ = scale * acc; lane (l32, hf) holds d = 32dt + 8g +
  // 4hf .. +3 of query qi
  if (qi < N) {
    const size_t orow = head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        const f32x4_t w = {acc[dt][4 * g] * p.scale, acc[dt][4 * g + 1] * p.scale,
                           acc[dt][4 * g + 2] * p.scale, acc[dt][4 * g + 3] * p.scale};
        if (p.out_f32) {
          *(f32x4_t*)(reinterpret_cast<float*>(p.dq) + orow + d) = w;
        } else {
          *(u32x2_t*)(reinterpret_cast<uint16_t*>(p.dq) + orow + d) =
              u32x2_t{pack2<BF16>(w[0], w[1]), pack2<BF16>(w[2], w[3])};
        }
      }
  }
  }  // work items
}

template <int D, bool BF16>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  constexpr int kRowsPerBlock = 256 / delta_tpr<D>();
  const dim3 dgrid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (a.o_f32)
    hipLaunchKernelGGL((bwd_delta_kernel<D, BF16, true>), dgrid, dim3(256), 0, stream, a.o,
                       static_cast<const uint16_t*>(a.dout), a.delta, rows);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<D, BF16, false>), dgrid, dim3(256), 0, stream, a.o,
                       static_cast<const uint16_t*>(a.dout), a.delta, rows);
  BwdQParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.N = a.N;
  p.nq = (a.N + 255) / 256;
  p.nbh = a.B * a.H;
  p.nb = (a.N + 63) / 64;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  if (p.c == 0.f) p.c = 1.17549435e-38f;
  p.scale = a.scale;
  p.out_f32 = a.grad_kind == kOutF32;
  const dim3 grid(p.nq * p.nbh), block(512);
  p.lpt = 0;
  if (a.causal) {
    p.lpt = sorted_order(a.bias ? reinterpret_cast<const void*>(&bwd_dq_kernel<D, BF16, true, true>)
                                : reinterpret_cast<const void*>(&bwd_dq_kernel<D, BF16, true, false>),
                         512, p.nbh, p.nq);
    if (a.bias) hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, true, true>), grid, block, 0, stream, p, a.bias);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, true, false>), grid, block, 0, stream, p, a.bias);
  } else {
    if (a.bias) hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, false, true>), grid, block, 0, stream, p, a.bias);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, false, false>), grid, block, 0, stream, p, a.bias);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd16(const BwdArgs& a, bool bf16, hipStream_t stream) {
  hipError_t e;
  if (a.d == 64) e = bf16 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
  else if (a.d == 96) e = bf16 ? launch_d<96, true>(a, stream) : launch_d<96, false>(a, stream);
  else e = bf16 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  if (e != hipSuccess) return e;
  return launch_bwd16_kv(a, bf16, stream);
}

}  // namespace attn
