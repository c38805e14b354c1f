// attn_fwd.hip -- fused attention forward for fp16/bf16 inputs on gfx950.
//
// Computes O = softmax(scale * Q K^T + mask + bias) V (page 4, "FlashAttention
// (TR)": the attention formula; tiling into on-chip blocks; online softmax
// with a running maximum and running sum; one fused kernel that writes only
// the final result) without forming the N x N score matrix anywhere.
//
// Work split: a workgroup of NW waves per (b, h, query tile); each wave
// owns QS x 32 queries (QS MFMA column tiles, so one K or V operand read from
// LDS feeds QS matrix instructions).  Two waves share each SIMD (from two
// workgroups when NW = 4, from one when NW = 8), so one wave's softmax runs
// on the vector ALU while the other's products run on the matrix cores.
// Keys and values stream through LDS in blocks of 64; the global loads of a
// future block are in flight while the current one is computed, and (dense
// layout, no bias) the next work item's Q rows and first block load during
// the current item's last block.
//
// Per key block and wave:
//   S^T = K Q^T (32x32x16 MFMA, fp32 accumulation): one query per lane
//       column, so the row maximum and row sum over keys reduce inside a lane
//       plus one exchange between the two lane halves.
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
// The output is normalised once and stored straight from the accumulators.
// The grid is persistent: as many workgroups as fit on the device at once,
// each looping over work items in a balanced heavy-first order.
#include "attn_common.hpp"
#include "attn_internal.hpp"

#include <math.h>
#include <stdlib.h>

#include <atomic>

namespace attn {
namespace {

constexpr int kBN = 64;       // keys per block
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// Tiling: QS query tiles of 32 per wave, NW waves per workgroup.  Block
// j+1 (K and V) is loaded during block j into the other of two buffers.
template <int QS, int NW>
struct Tiling {
  static constexpr int kWQ = 32 * QS;            // queries per wave
  static constexpr int kBM = NW * kWQ;           // queries per workgroup
  static constexpr int kThreads = 64 * NW;
  static constexpr int kKbuf = 2;
  static constexpr int kVbuf = 2;
};

struct Fwd16Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int N;
  int nq;      // query tiles per head
  int nbh;     // B*H
  int nb;      // ceil(N/64), bias blocks per side
  int ntiles;  // B*H*nq
  float c;     // scale * log2(e), never 0
  int out_f32;
  // general layout (strided entry point only): element strides (batch, head,
  // token) of q, k, v, o with d contiguous, and optional packed sequences
  // (cu: sequence b holds tokens cu[b] .. cu[b+1]-1; N is the longest)
  int H;
  const int* cu;
  int64_t qs[3], ks[3], vs[3], os[3];
};

template <int D, int QS, int NW>
struct Fwd16Smem {
  using T = Tiling<QS, NW>;
  // Padded rows.  K: 16 bytes of padding, so the 16-byte operand reads of 16
  // consecutive rows fall on distinct banks.  V: the transposing reads touch
  // 4 consecutive rows x 64 bytes per half wave; a row stride of 288 bytes
  // (d = 128) or 192 bytes (d = 64) spreads them over the banks (measured
  // on gfx950: 107 B/clk/CU against 62 B/clk/CU at a 272-byte stride).
  static constexpr int kKRow = D + 8;
  // V rows of 288 bytes at d = 128 and 96, 192 bytes at d = 64
  static constexpr int kVRow = D == 64 ? D + 32 : 144;
  static constexpr int kKTile = kBN * kKRow;
  static constexpr int kVTile = kBN * kVRow;
  static constexpr int kElems = T::kKbuf * kKTile + T::kVbuf * kVTile;
};

// Kernel variants by input layout: contiguous without a bias (the plain loop
// over key blocks), contiguous with a block bias (adds the block-sparse skip)
// and the general strided / packed-sequence layout (no bias).
enum Mode { kDense = 0, kBias = 1, kGen = 2 };

// The block bias comes as its own restrict argument: its reads, uniform and
// never written by the kernel, then compile to scalar loads, which do not
// share the in-order vector-load counter with the K/V prefetch.
template <int D, bool BF16, bool CAUSAL, int QS, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd16_kernel(Fwd16Params p, const float* __restrict__ bias) {
  constexpr bool GEN = MODE == kGen, HAS_BIAS = MODE == kBias;
  using TL = Tiling<QS, NW>;
  using S = Fwd16Smem<D, QS, NW>;
  constexpr int kWQ = TL::kWQ, kBM = TL::kBM, kThreads = TL::kThreads;
  constexpr int kKbuf = TL::kKbuf, kVbuf = TL::kVbuf;
  constexpr int kKRow = S::kKRow, kVRow = S::kVRow;
  constexpr int kKTile = S::kKTile, kVTile = S::kVTile;
  constexpr int kCpr = D / 8;  // 16-byte chunks of data per row
  constexpr int kDT = D / 32;  // 32-row tiles of O^T
  constexpr int kKS = D / 16;  // k-steps of S^T = K Q^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::kElems];
  uint16_t* const kbase_lds = smem;                   // kKbuf K tiles
  uint16_t* const vbase_lds = smem + kKbuf * kKTile;  // kVbuf V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Loop over (b, h, query tile) work items (work_queue: per-XCD queues,
  // balanced heavy-first order when the grid is persistent).
  const WorkQueue wq = work_queue(p.nbh, p.nq);
  constexpr bool DENSE = MODE == kDense;
  constexpr int kNst = kBN * kCpr / kThreads;
  u32x4_t qf[QS][kKS];
  u32x4_t kst[kNst], vst[kNst];
  // Dense layout without a bias: the next work item's Q rows and first K/V
  // block are loaded during the current item's last block, so a new item
  // starts without waiting for global memory (pre: qf and kst/vst already
  // hold this item's Q and block 0).
  bool pre = false;
  for (int round = 0;; ++round) {
  int bh, tq;
  if (!work_item(wq, round, p.nq, bh, tq)) break;
  int bh_n = 0, tq_n = 0;
  const bool has_next = DENSE && work_item(wq, round + 1, p.nq, bh_n, tq_n);
  const int qt = CAUSAL ? p.nq - 1 - tq : tq;  // heaviest tiles first
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kWQ;
  // this head's row 0 (elements) and row strides; the dense layout is
  // [B,H,N,d] contiguous
  int N = p.N;
  int64_t qoff, koff, voff0, ooff;
  int qsn = D, ksn = D, vsn = D, osn = D;
  if constexpr (GEN) {
    const int b = bh / p.H, h = bh - b * p.H;
    int64_t t0 = 0;
    if (p.cu != nullptr) {
      t0 = p.cu[b];
      N = max(0, min(p.cu[b + 1] - p.cu[b], p.N));
    }
    qoff = (p.cu ? t0 * p.qs[2] : b * p.qs[0]) + h * p.qs[1];
    koff = (p.cu ? t0 * p.ks[2] : b * p.ks[0]) + h * p.ks[1];
    voff0 = (p.cu ? t0 * p.vs[2] : b * p.vs[0]) + h * p.vs[1];
    ooff = (p.cu ? t0 * p.os[2] : b * p.os[0]) + h * p.os[1];
    qsn = (int)p.qs[2];
    ksn = (int)p.ks[2];
    vsn = (int)p.vs[2];
    osn = (int)p.os[2];
    if (q0 >= N) continue;  // this sequence is shorter than the tile start
  } else {
    qoff = koff = voff0 = ooff = (int64_t)bh * N * D;
  }
  const uint16_t* __restrict__ Q = p.q + qoff;
  const uint16_t* __restrict__ K = p.k + koff;
  const uint16_t* __restrict__ V = p.v + voff0;

  // Q^T as the B operand of S^T = K Q^T: for query sub-tile qs the lane holds
  // Q[qw0 + 32qs + l32][16kk + 8hf .. +7].  Rows past N read row N-1 (their
  // results are never stored).
  if (!(DENSE && pre)) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int row = min(qw0 + 32 * qs + l32, N - 1);
      const uint16_t* src = Q + (size_t)row * qsn + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) qf[qs][kk] = *(const u32x4_t*)(src + 16 * kk);
    }
  }

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
  const int nkb = (kend + kBN - 1) / kBN;
  // last key block this wave computes (causal: its diagonal block)
  const int wave_last = CAUSAL ? min(nkb - 1, qw0 / kBN) : nkb - 1;
  const bool wave_has_rows = qw0 < N;

  // ---- loader: a 64 x D tile is 64*D/8 chunks of 16 bytes, staged through
  // registers.  Chunk tid + i*threads of block kb sits at byte
  // 16*tid + (kb*64*D*2 + 16*i*threads) of the head: a buffer load with one
  // per-lane offset and a uniform one; key rows past N read zeros (masked
  // later), so every load is unconditional.
  // (general layout: key rows ksn / vsn elements apart, so each chunk has its
  // own per-lane offset and the block offset is kb*64 rows)
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K, (uint32_t)N * ksn * 2);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V, (uint32_t)N * vsn * 2);
  const uint32_t voff = 16u * tid;
  uint32_t kvo[kNst], vvo[kNst];
  if constexpr (GEN) {
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCpr, ch = idx % kCpr;
      kvo[i] = (uint32_t)(row * ksn * 2 + ch * 16);
      vvo[i] = (uint32_t)(row * vsn * 2 + ch * 16);
    }
  }
  auto load_k = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      if constexpr (GEN) kst[i] = buffer_load16(krs, kvo[i], (uint32_t)(kb * kBN) * ksn * 2);
      else kst[i] = buffer_load16(krs, voff, kb * kBN * D * 2 + 16 * i * kThreads);
    }
  };
  auto load_v = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      if constexpr (GEN) vst[i] = buffer_load16(vrs, vvo[i], (uint32_t)(kb * kBN) * vsn * 2);
      else vst[i] = buffer_load16(vrs, voff, kb * kBN * D * 2 + 16 * i * kThreads);
    }
  };
  auto store_k = [&](int buf) {
    uint16_t* ks = kbase_lds + buf * kKTile;
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCpr, ch = idx % kCpr;
      *(u32x4_t*)(ks + row * kKRow + ch * 8) = kst[i];
    }
  };
  auto store_v = [&](int buf) {
    uint16_t* vs = vbase_lds + buf * kVTile;
#pragma unroll
    for (int i = 0; i < kNst; ++i) {
      const int idx = tid + i * kThreads, row = idx / kCpr, ch = idx % kCpr;
      *(u32x4_t*)(vs + row * kVRow + ch * 8) = vst[i];
    }
  };

  // ---- per-wave online-softmax state
  f32x16_t o[kDT][QS];
  float m_run[QS], l_run[QS];  // running max (log2 units, equal in both lane halves), partial sums
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) o[dt][qs] = f32x16_t{};
    m_run[qs] = -INFINITY;
    l_run[qs] = 0.f;
  }
  const float c = p.c;
  const bool pos = c > 0.f;
  const float sent = pos ? -INFINITY : INFINITY;

  // transposing-read coordinates for the V^T operand: this lane addresses row
  // 16kk + vkey (and +8) at column 32dt + vcol
  const int g16 = lane >> 4, t16 = lane & 15;
  const int vkey = 4 * hf + (t16 >> 2);
  const int vcol = 16 * (g16 & 1) + 4 * (t16 & 3);

  // ---- S^T = K Q^T for one key block (two 32-key tiles x QS query tiles)
  auto qk = [&](int buf, f32x16_t (&s)[2][QS]) {
    const uint16_t* Ks = kbase_lds + buf * kKTile + l32 * kKRow + 8 * hf;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) s[0][qs] = s[1][qs] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        // row 32T + l32, columns 16kk + 8hf .. +7
        const u32x4_t a = *(const u32x4_t*)(Ks + 32 * T * kKRow + 16 * kk);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[T][qs] = mfma32x32x16<BF16>(a, qf[qs][kk], s[T][qs]);
      }
  };

  // ---- masking of the causal diagonal block and the tail block (keys past
  // N): masked scores become +-inf, so c*S is -inf and P = exp2(-inf) = 0.
  auto apply_mask = [&](int j, f32x16_t (&s)[2][QS]) {
    const int kb0 = j * kBN;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + 32 * T + 8 * (r >> 2) + 4 * hf + (r & 3);
          const int qi = qw0 + 32 * qs + l32;
          const bool m = (CAUSAL && key > qi) || key >= N;
          s[T][qs][r] = m ? sent : s[T][qs][r];
        }
  };
  auto needs_mask = [&](int j) { return (CAUSAL && j == wave_last) || (j + 1) * kBN > N; };

  // ---- block maximum and lazy rescale of the running state; returns the
  // exponent offsets kc = bias - m (log2 units) of the block
  auto block_max = [&](f32x16_t (&s)[2][QS], float (&kc)[QS], float braw) {
    const float bl = HAS_BIAS ? braw * kLog2e : 0.f;
    float m_blk[QS];
    bool need_any = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float a0;
      if (pos) {
        a0 = fmaxf(s[0][qs][0], s[1][qs][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fmaxf(a0, fmaxf(s[0][qs][r], s[1][qs][r]));
        a0 = xor32_max(a0);
      } else {
        a0 = fminf(s[0][qs][0], s[1][qs][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) a0 = fminf(a0, fminf(s[0][qs][r], s[1][qs][r]));
        a0 = xor32_min(a0);
      }
      m_blk[qs] = (a0 == sent) ? -INFINITY : fmaf(a0, c, bl);
      need_any |= m_blk[qs] > m_run[qs] + kTau;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const bool need = m_blk[qs] > m_run[qs] + kTau;
        const float m_new = need ? m_blk[qs] : m_run[qs];
        const float alpha = need ? exp2_approx(m_run[qs] - m_new) : 1.f;
        l_run[qs] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) o[dt][qs] *= alpha;
        m_run[qs] = m_new;
      }
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) kc[qs] = bl - ((m_run[qs] == -INFINITY) ? 0.f : m_run[qs]);
  };

  // ---- P = exp2(c*S + bias - m) as the B operand of O^T += V^T P^T.  Masked
  // scores are +-inf, so c*S is -inf and P is 0 (c is never 0: the host
  // passes the smallest normal float for a zero scale).  The row sum adds
  // the rounded P values the product uses.
  u32x4_t pb[4][QS];
  auto softmax_p = [&](f32x16_t (&s)[2][QS], const float (&kc)[QS]) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float lsum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int T = kk >> 1, t = kk & 1;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * t + e;
          const float p0 = exp2_approx(fmaf(s[T][qs][r], c, kc[qs]));
          const float p1 = exp2_approx(fmaf(s[T][qs][r + 1], c, kc[qs]));
          const uint32_t pk = pack2<BF16>(p0, p1);
          lsum = sum2_acc<BF16>(pk, lsum);
          pb[kk][qs][e >> 1] = pk;
        }
      }
      l_run[qs] += lsum;
    }
  };
  auto pv = [&](int buf) {
    const uint16_t* Vs = vbase_lds + buf * kVTile + vkey * kVRow + vcol;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const uint16_t* vp = Vs + 16 * kk * kVRow + 32 * dt;
        const u32x2_t lo = lds_read_tr16(vp);
        const u32x2_t hi = lds_read_tr16(vp + 8 * kVRow);
        const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) o[dt][qs] = mfma32x32x16<BF16>(a, pb[kk][qs], o[dt][qs]);
      }
    }
  };

  // ---- block-sparse skip (with a bias only): a key block whose gate is 0
  // (bias -inf) for every query block of this tile adds nothing to any of
  // its rows, so it is neither loaded nor computed; a wave skips blocks gated
  // off for its own query block.  The bias values a step needs are read a
  // step ahead, so their latency hides behind a block's products.
  constexpr int kRows = kBM / kBN;  // 64-query blocks per tile (2 or 4)
  const int rw = wave * kWQ / kBN;  // this wave's query block in the tile
  BlockGate<kRows> gate(HAS_BIAS ? bias + (size_t)bh * p.nb * p.nb : bias, p.nb, q0 / kBN, nkb, rw);

  f32x16_t sc[2][QS];
  // ---- one key block: the next active block (jn) loads while block jc,
  // staged in buffer buf, computes; braw is this wave's bias of block jc
  auto step = [&](int jc, int jn, int buf, float braw) {
    const bool more = jn < nkb;
    if (more) {
      load_k(jn);
      load_v(jn);
    }
    if (wave_has_rows && jc <= wave_last && (!HAS_BIAS || braw != -INFINITY)) {
      qk(buf, sc);
      if (needs_mask(jc)) apply_mask(jc, sc);
      float kc[QS];
      block_max(sc, kc, braw);
      softmax_p(sc, kc);
      pv(buf);
    }
    if (more) {
      store_k(buf ^ 1);
      store_v(buf ^ 1);
    }
    __syncthreads();
  };
  // The first block is staged unconditionally (a valid block even when every
  // block is gated off), and its loads are issued after the Q loads (the
  // scheduling barrier): its wait for the global loads then also covers Q,
  // so no wait on Q lands inside the loop, where (the counter being in
  // order) it would also wait for the next block's prefetch every iteration.
  int j0 = 0;
  if constexpr (HAS_BIAS) j0 = gate.first();
  __builtin_amdgcn_sched_barrier(0);
  if (!(DENSE && pre)) {
    load_k(min(j0, nkb - 1));
    load_v(min(j0, nkb - 1));
  }
  store_k(0);
  store_v(0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if constexpr (HAS_BIAS) {
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
    // every block is active (the plain counted loop schedules measurably
    // better than the general one)
    for (int j = 0; j + 1 < nkb; ++j) step(j, j + 1, j & 1, 0.f);
    // the last block: the next item's Q rows and first K/V block are
    // loaded meanwhile (Q after this block's last use of it)
    {
      const int jc = nkb - 1, buf = jc & 1;
      const int qt_n = CAUSAL ? p.nq - 1 - tq_n : tq_n;
      const int qw0_n = qt_n * kBM + wave * kWQ;
      const size_t off_n = (size_t)bh_n * N * D;
      if (has_next) {
        const __amdgpu_buffer_rsrc_t krn = buffer_rsrc(p.k + off_n, (uint32_t)N * D * 2);
        const __amdgpu_buffer_rsrc_t vrn = buffer_rsrc(p.v + off_n, (uint32_t)N * D * 2);
#pragma unroll
        for (int i = 0; i < kNst; ++i) {
          kst[i] = buffer_load16(krn, voff, 16 * i * kThreads);
          vst[i] = buffer_load16(vrn, voff, 16 * i * kThreads);
        }
      }
      const bool work = wave_has_rows && jc <= wave_last;
      if (work) qk(buf, sc);
      if (has_next) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const int row = min(qw0_n + 32 * qs + l32, N - 1);
          const uint16_t* src = p.q + off_n + (size_t)row * D + 8 * hf;
#pragma unroll
          for (int kk = 0; kk < kKS; ++kk) qf[qs][kk] = *(const u32x4_t*)(src + 16 * kk);
        }
      }
      if (work) {
        if (needs_mask(jc)) apply_mask(jc, sc);
        float kc[QS];
        block_max(sc, kc, 0.f);
        softmax_p(sc, kc);
        pv(buf);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: normalise, LSE, stores straight from the accumulators
  // (lane (l32, hf) holds d = 32dt + 8g + 4hf .. +3 of query qw0 + 32qs + l32)
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const float l_tot = xor32_sum(l_run[qs]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int qi = qw0 + 32 * qs + l32;
    if (qi < N) {
      if (p.lse != nullptr && hf == 0)
        p.lse[(size_t)bh * p.N + qi] = l_tot > 0.f ? (m_run[qs] + __log2f(l_tot)) * kLn2 : -INFINITY;
      const size_t orow = (size_t)ooff + (size_t)qi * osn;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * hf;
          const f32x4_t w4 = {o[dt][qs][4 * g] * inv, o[dt][qs][4 * g + 1] * inv, o[dt][qs][4 * g + 2] * inv,
                              o[dt][qs][4 * g + 3] * inv};
          if (p.out_f32) {
            *(f32x4_t*)(reinterpret_cast<float*>(p.o) + orow + d) = w4;
          } else {
            *(u32x2_t*)(reinterpret_cast<uint16_t*>(p.o) + orow + d) =
                u32x2_t{pack2<BF16>(w4[0], w4[1]), pack2<BF16>(w4[2], w4[3])};
          }
        }
    }
  }
  pre = has_next;
  }  // work items
}

template <int D, bool BF16, bool CAUSAL, int QS, int NW, int MODE>
hipError_t launch_impl(const FwdArgs& a, hipStream_t stream) {
  using TL = Tiling<QS, NW>;
  Fwd16Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.nq = (a.N + TL::kBM - 1) / TL::kBM;
  p.nb = (a.N + 63) / 64;
  p.nbh = a.B * a.H;
  p.ntiles = a.B * a.H * p.nq;
  // c = scale*log2(e).  A zero scale is passed as the smallest normal float:
  // masked scores are +-inf and inf*0 would be NaN, while any finite score
  // below 2^100 in magnitude times 2^-126 is below an ulp of the exponent.
  p.c = (float)((double)a.scale * 1.4426950408889634);
  if (p.c == 0.f) p.c = 1.17549435e-38f;
  p.out_f32 = a.out_kind == kOutF32;
  p.H = a.H;
  p.cu = a.cu;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = a.strides[i];
    p.ks[i] = a.strides[3 + i];
    p.vs[i] = a.strides[6 + i];
    p.os[i] = a.strides[9 + i];
  }
  // Causal tiles differ in cost, so a persistent grid with the balanced
  // heavy-first order pays where it applies (measured +7% at 4x32x4096,
  // d = 128); equal-cost non-causal tiles run one workgroup per item
  // (persistent was 5% slower).
  // (packed sequences of different lengths: one workgroup per tile; the
  // balance argument of the persistent queues assumes equal heads)
  const int grid = (CAUSAL && !(MODE == kGen && a.cu))
                       ? persistent_grid(reinterpret_cast<const void*>(&fwd16_kernel<D, BF16, CAUSAL, QS, NW, MODE>),
                                         TL::kThreads, p.nbh, p.nq)
                       : p.ntiles;
  if (grid <= 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd16_kernel<D, BF16, CAUSAL, QS, NW, MODE>), dim3(grid), dim3(TL::kThreads), 0, stream, p, a.bias);
  return hipGetLastError();
}

// Tiling per head dimension.  ATTN_FWD16_TILING selects another variant, to
// compare them on the GPU.  Measured on MI355X (TFLOPS; prefill 4x32x4096 /
// long-context 1x32x32768, causal, d = 128; DiT-gated 2x24x16384, d = 64):
//   d = 128: QS1 NW8 (default) 743 / 1085; QS1 NW4 688 / 1003.  Tried and
//     dropped: software-pipelined S of block j+1 next to the softmax of block j
//     (653 / 1030); two wave groups in ping-pong phases (596 / 950: a product
//     phase has one matrix-issuing wave per SIMD, LDS waits are exposed);
//     waves staggered by one product (701 / 983, and register spills).
//   d = 64: QS2 NW4 (default) 936-950; QS1 NW4 854.
int tiling_override() {
  static const int v = [] {
    const char* e = getenv("ATTN_FWD16_TILING");
    return e ? atoi(e) : -1;
  }();
  return v;
}

template <bool BF16, bool CAUSAL, int MODE>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  const int t = tiling_override();
  if (a.d == 64) {
    if (t == 1) return launch_impl<64, BF16, CAUSAL, 1, 4, MODE>(a, stream);
    return launch_impl<64, BF16, CAUSAL, 2, 4, MODE>(a, stream);
  }
  // d = 96: a 64 x 96 tile is 768 16-byte chunks, which 4 waves split evenly
  if (a.d == 96) return launch_impl<96, BF16, CAUSAL, 1, 4, MODE>(a, stream);
  if (t == 1) return launch_impl<128, BF16, CAUSAL, 1, 4, MODE>(a, stream);
  return launch_impl<128, BF16, CAUSAL, 1, 8, MODE>(a, stream);
}

template <bool BF16, bool CAUSAL>
hipError_t launch_g(const FwdArgs& a, hipStream_t stream) {
  if (a.general) return launch_d<BF16, CAUSAL, kGen>(a, stream);
  return a.bias ? launch_d<BF16, CAUSAL, kBias>(a, stream) : launch_d<BF16, CAUSAL, kDense>(a, stream);
}

}  // namespace

// Workgroups of `kernel` resident at once on the current device (a multiple
// of 8 when at least 8), cached per kernel and device; -1 on a HIP error.
int resident_slots(const void* kernel, int threads) {
  struct Entry { const void* k; int dev; int slots; };
  static Entry cache[64];
  static std::atomic<int> used{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const int n = used.load(std::memory_order_acquire);
  for (int i = 0; i < n && i < 64; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].slots;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  int slots = per_cu * cus;
  if (slots >= 8) slots &= ~7;
  if (slots <= 0) return -1;
  const int i = used.fetch_add(1, std::memory_order_acq_rel);
  if (i < 64) cache[i] = Entry{kernel, dev, slots};
  return slots;
}

int sorted_order(const void* kernel, int threads, int nbh, int nq, int per_slot) {
  const int slots = resident_slots(kernel, threads);
  if (slots <= 0 || (int64_t)nbh * nq >= (int64_t)per_slot * slots) return 0;
  static const int forced = [] {
    const char* e = getenv("ATTN_LPT_GROUP");
    return e ? atoi(e) : 0;
  }();
  if (forced > 0) return forced;
  // heads per group: the smallest power of two with at least two items per
  // slot of an XCD in a group (measured on the 8-bit forward, against one
  // group of all of an XCD's heads: 4x32x4096 +3% and HBM reads 438 MB
  // instead of 1103 with groups of 8; 2x32x8192 +1% with groups of 4)
  const int per_xcd = slots >= 8 ? slots / 8 : slots;
  const int need = (2 * per_xcd + nq - 1) / nq;
  int g = 1;
  while (g < need) g *= 2;
  return g;
}

int persistent_grid(const void* kernel, int threads, int nbh, int nq) {
  const int items = nbh * nq;
  const int slots = resident_slots(kernel, threads);
  if (slots <= 0) return -1;
  // Persistent only when the alternating order of the per-XCD queues
  // balances exactly (2 x slots per XCD a multiple of the tiles per head,
  // heads spread evenly over the XCDs) and there is more than one round;
  // else one workgroup per item, where the hardware dispatch balances.
  const bool balanced = (nbh & 7) == 0 && slots % 8 == 0 && (2 * (slots / 8)) % nq == 0;
  return (balanced && items > slots) ? slots : items;
}

hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.causal ? launch_g<true, true>(a, stream) : launch_g<true, false>(a, stream);
  return a.causal ? launch_g<false, true>(a, stream) : launch_g<false, false>(a, stream);
}

}  // namespace attn
