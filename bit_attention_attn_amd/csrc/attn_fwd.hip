// attn_fwd.hip -- fused attention forward for fp16/bf16 inputs on gfx950.
//
// Computes O = softmax(scale * Q K^T + mask + bias) V (page 4, "FlashAttention
// (TR)": the attention formula; tiling into on-chip blocks; online softmax
// with a running maximum and running sum; one fused kernel that writes only
// the final result) without forming the N x N score matrix anywhere.
//
// Work split: one workgroup of 4 waves per (b, h, 128-query tile); each wave
// owns 32 queries.  Keys and values stream through LDS in blocks of 64,
// double buffered: the global loads of block j+1 are in flight while block j
// is computed.
//
// Per key block and wave:
//   S^T = K Q^T on the matrix cores (32x32x16, fp32 accumulation).  Computing
//       the transpose puts one query per lane column, so the row maximum and
//       row sum over keys reduce inside a lane plus one lane-half exchange.
//   softmax in base 2: the scale is folded into c = scale*log2(e); the bias
//       (natural-log units) is one scalar per 64x64 block, so the block
//       maximum of c*S + bias is c*max(S) + bias.
//   The running maximum is raised only when a block maximum exceeds it by
//       more than kTau (P then stays <= 2^kTau, exact in fp16/bf16 range),
//       which skips most rescales of the output accumulator.
//   O^T += V^T P^T: P^T comes straight from the S^T accumulator registers as
//       the B operand (the key order inside a lane is a permutation applied
//       to both operands); V^T is read from the row-major V tile with the
//       transposing LDS read.
// The output is normalised once, staged through LDS and written with
// coalesced 16-byte stores.
#include "attn_common.hpp"
#include "attn_internal.hpp"

#include <math.h>

namespace attn {
namespace {

constexpr int kBM = 128;      // queries per workgroup
constexpr int kBN = 64;       // keys per block
constexpr int kThreads = 256; // 4 waves
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

struct Fwd16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const float* bias;
  int N;
  int nq;      // query tiles per head
  int nb;      // ceil(N/64), bias blocks per side
  int ntiles;  // B*H*nq
  float c;     // scale * log2(e)
  int out_f32;
};

template <int D>
struct Fwd16Smem {
  static constexpr int kRow = D + 8;       // padded row, elements
  static constexpr int kTile = kBN * kRow; // elements per K or V tile
  static constexpr int kElems = 4 * kTile; // two buffers of (K, V)
};

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd16_kernel(Fwd16Params p) {
  using S = Fwd16Smem<D>;
  constexpr int kRow = S::kRow;
  constexpr int kTile = S::kTile;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::kElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, p.ntiles);
  const int bh = tile / p.nq;
  int qt = tile - bh * p.nq;
  if (CAUSAL) qt = p.nq - 1 - qt;  // heaviest tiles first
  const int N = p.N;
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Q = p.q + head;
  const uint16_t* __restrict__ K = p.k + head;
  const uint16_t* __restrict__ V = p.v + head;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[qi][16kk + 8hf .. +7].
  u32x4_t qf[D / 16];
  {
    const bool ok = qi < N;
    const uint16_t* src = Q + (size_t)(ok ? qi : 0) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4_t x = *(const u32x4_t*)(src + 16 * kk);
      qf[kk] = ok ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
  const int nkb = (kend + kBN - 1) / kBN;

  // Loader: a 64 x D tile is 64*D/8 chunks of 16 bytes.
  constexpr int kCpr = D / 8;
  constexpr int kNld = kBN * kCpr / kThreads;
  u32x4_t kr[kNld], vr[kNld];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kNld; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / kCpr, ch = idx % kCpr;
      const int key = kb * kBN + row;
      if (key < N) {
        kr[i] = *(const u32x4_t*)(K + (size_t)key * D + ch * 8);
        vr[i] = *(const u32x4_t*)(V + (size_t)key * D + ch * 8);
      } else {
        kr[i] = u32x4_t{0u, 0u, 0u, 0u};
        vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * 2 * kTile;
#pragma unroll
    for (int i = 0; i < kNld; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / kCpr, ch = idx % kCpr;
      *(u32x4_t*)(ks + row * kRow + ch * 8) = kr[i];
      *(u32x4_t*)(ks + kTile + row * kRow + ch * 8) = vr[i];
    }
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m_run = -INFINITY;  // running max, log2 units (same in both lane halves)
  float l_run = 0.f;        // this lane's partial row sum
  const float c = p.c;
  const bool pos = c >= 0.f;
  // a wave whose queries all lie past N computes nothing (it still loads and
  // synchronises); the clamp keeps its bias row inside the tensor
  const bool wave_has_rows = qw0 < N;
  const int qb64 = min(qw0 >> 6, p.nb - 1);
  const float* bias_row = p.bias ? p.bias + ((size_t)bh * p.nb + (size_t)qb64) * p.nb : nullptr;

  // transposing-read coordinates for the V^T operand
  const int g16 = lane >> 4, t16 = lane & 15;
  const int vkey = 4 * hf + (t16 >> 2);
  const int vcol = 16 * (g16 & 1) + 4 * (t16 & 3);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < nkb; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkb) load_tile(j + 1);
    const int kbase = j * kBN;
    const bool active = wave_has_rows && (!CAUSAL || kbase <= qw0 + 31);
    if (active) {
      const uint16_t* Ks = smem + buf * 2 * kTile;
      const uint16_t* Vs = Ks + kTile;

      // ---- S^T = K Q^T for keys [kbase, kbase+64): two 32-key tiles
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const u32x4_t a = *(const u32x4_t*)(Ks + (32 * T + l32) * kRow + 16 * kk + 8 * hf);
          s[T] = mfma32x32x16<BF16>(a, qf[kk], s[T]);
        }
      }

      // ---- mask (diagonal and tail blocks only)
      const bool need_mask = (CAUSAL && kbase + kBN - 1 > qw0) || (kbase + kBN > N);
      const float sent = pos ? -INFINITY : INFINITY;
      uint32_t mbits = 0u;
      if (need_mask) {
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 32 * T + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool m = (CAUSAL && key > qi) || key >= N;
            if (m) {
              s[T][r] = sent;
              mbits |= 1u << (16 * T + r);
            }
          }
      }

      // ---- block maximum of c*S (+ bias, constant over the block)
      float mx;
      if (pos) {
        float a0 = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fmaxf(a0, fmaxf(s[0][r], s[1][r]));
        mx = xor32_max(a0);
      } else {
        float a0 = fminf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fminf(a0, fminf(s[0][r], s[1][r]));
        mx = xor32_min(a0);
      }
      const float bl = bias_row ? bias_row[j] * kLog2e : 0.f;
      const float m_blk = (mx == sent) ? -INFINITY : fmaf(mx, c, bl);

      // ---- lazy rescale of the running state
      const bool need = m_blk > m_run + kTau;
      if (__any(need)) {
        const float m_new = need ? m_blk : m_run;
        const float alpha = exp2_approx(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      const float kc = bl - ((m_run == -INFINITY) ? 0.f : m_run);

      // ---- P = exp2(c*S + bias - m), packed as the B operand of O^T += V^T P^T
      u32x4_t pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int T = kk >> 1, t = kk & 1;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * t + e;
          float p0 = exp2_approx(fmaf(s[T][r], c, kc));
          float p1 = exp2_approx(fmaf(s[T][r + 1], c, kc));
          if (need_mask) {
            p0 = (mbits >> (16 * T + r)) & 1u ? 0.f : p0;
            p1 = (mbits >> (16 * T + r + 1)) & 1u ? 0.f : p1;
          }
          lsum += p0 + p1;
          pb[kk][e >> 1] = pack2<BF16>(p0, p1);
        }
      }
      l_run += lsum;

      // ---- O^T += V^T P^T; V^T via transposing reads of the row-major tile
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const uint16_t* vp = Vs + (16 * kk + vkey) * kRow + 32 * dt + vcol;
          const u32x2_t lo = lds_read_tr16(vp);
          const u32x2_t hi = lds_read_tr16(vp + 8 * kRow);
          const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
          o[dt] = mfma32x32x16<BF16>(a, pb[kk], o[dt]);
        }
      }
    }
    if (j + 1 < nkb) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, LSE, stage through LDS, coalesced stores
  const float l_tot = xor32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (p.lse != nullptr && hf == 0 && qi < N)
    p.lse[(size_t)bh * N + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;

  if (p.out_f32) {
    constexpr int kSt = D + 4;  // floats per staged row
    float* st = reinterpret_cast<float*>(smem) + wave * 32 * kSt;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        f32x4_t w = {o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                     o[dt][4 * g + 3] * inv};
        *(f32x4_t*)(st + l32 * kSt + d) = w;
      }
    __syncthreads();
    float* O = reinterpret_cast<float*>(p.o) + head;
    constexpr int kCh = D / 4;  // 16-byte chunks per row
#pragma unroll
    for (int it = 0; it < 32 * kCh / 64; ++it) {
      const int idx = lane + 64 * it;
      const int row = idx / kCh, ch = idx % kCh;
      const int q = qw0 + row;
      if (q < N) *(f32x4_t*)(O + (size_t)q * D + 4 * ch) = *(const f32x4_t*)(st + row * kSt + 4 * ch);
    }
  } else {
    constexpr int kSt = D + 8;  // 16-bit elements per staged row
    uint16_t* st = smem + wave * 32 * kSt;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        u32x2_t w = {pack2<BF16>(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                     pack2<BF16>(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2_t*)(st + l32 * kSt + d) = w;
      }
    __syncthreads();
    uint16_t* O = reinterpret_cast<uint16_t*>(p.o) + head;
    constexpr int kCh = D / 8;
#pragma unroll
    for (int it = 0; it < 32 * kCh / 64; ++it) {
      const int idx = lane + 64 * it;
      const int row = idx / kCh, ch = idx % kCh;
      const int q = qw0 + row;
      if (q < N) *(u32x4_t*)(O + (size_t)q * D + 8 * ch) = *(const u32x4_t*)(st + row * kSt + 8 * ch);
    }
  }
}

template <int D, bool BF16, bool CAUSAL>
hipError_t launch_impl(const FwdArgs& a, hipStream_t stream) {
  Fwd16Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.bias = a.bias;
  p.N = a.N;
  p.nq = (a.N + kBM - 1) / kBM;
  p.nb = (a.N + 63) / 64;
  p.ntiles = a.B * a.H * p.nq;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  p.out_f32 = a.out_kind == kOutF32;
  hipLaunchKernelGGL((fwd16_kernel<D, BF16, CAUSAL>), dim3(p.ntiles), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, bool CAUSAL>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_impl<64, BF16, CAUSAL>(a, stream) : launch_impl<128, BF16, CAUSAL>(a, stream);
}

}  // namespace

hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.causal ? launch_d<true, true>(a, stream) : launch_d<true, false>(a, stream);
  return a.causal ? launch_d<false, true>(a, stream) : launch_d<false, false>(a, stream);
}

}  // namespace attn
