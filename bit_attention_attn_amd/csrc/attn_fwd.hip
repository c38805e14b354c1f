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
// workgroups when NW = 4, from one when NW = 8; three, from three 4-wave
// workgroups, for INT8 scores at d = 128 on long sequences), so one wave's
// softmax runs on the vector ALU while another's products run on the matrix
// cores.
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
//   Lazy rescale: P stays <= 2^kTau (well inside the fp16/bf16 range)
//       against a running maximum m that is raised only when needed, which
//       skips most rescales of the output accumulator.  Two forms:
//     - block maximum first (d = 96, 128): m is raised when the block
//       maximum exceeds it by more than kTau;
//     - speculative (d = 64, two query tiles per wave): P is computed against
//       m as it stands, with no block maximum.  P >= 0, so if every lane's
//       partial sum of the block's P stays <= 2^kTau no single P exceeds it
//       and the block is done; otherwise (and on a row's first block, where m
//       is still -inf) the block maximum is taken, m is raised to it, the
//       running state rescaled and P recomputed.  This saves the maximum
//       tree on most blocks but keeps the P V products from starting before
//       the last exponential; measured on MI355X, +6% at d = 64 (twice the
//       softmax work per matrix instruction) and -2% at d = 128.
//   O^T += V^T P^T: P^T comes straight from the S^T accumulator registers as
//       the B operand (the key order inside a lane is a permutation applied
//       to both operands); V^T is read from the row-major V tile with the
//       transposing LDS read.
// The output is normalised once and stored straight from the accumulators.
// Causal launches whose tiles balance over the resident slots use a
// persistent grid (as many workgroups as fit on the device at once, each
// looping over work items in a balanced heavy-first order); the others run
// one workgroup per work item.
#include "attn_common.hpp"
#include "attn_internal.hpp"

#include <math.h>

#include <mutex>

namespace attn {
namespace {

constexpr int kBN = 64;       // keys per block
constexpr float kTau = 8.0f;  // lazy-rescale bound, log2 units: P <= 2^kTau
constexpr float kSumCap = 256.0f;  // 2^kTau

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
  // INT8 scores (Q8 kernels): the prepared INT8 Q and centred K [B,H,np,d],
  // the Q block scales [B,H,nblk] and the K mean [B,H,d] (the K block scales
  // come as their own kernel argument)
  const int8_t* qq;
  const int8_t* kq;
  const float* sq;
  const float* kmean;
  int np, nblk;
};

// K and V tiles of one 64-key block, unpadded and filled straight from
// global memory by 16-byte buffer loads into LDS: one instruction writes the
// 64 consecutive 16-byte chunks of a wave, so the layout is set by which
// global chunk each lane fetches.  Within a row the 16-byte chunks are
// rotated by a per-row amount so that the operand reads spread over the
// banks:
//   K (16-bit, read 16 bytes per lane, 16 consecutive rows at one logical
//     chunk): rows of 256 bytes (d = 128) all start on bank 0, so the chunk
//     rotates by r mod 16; rows of 128 bytes (d = 64) repeat every 2 rows,
//     r/2; rows of 192 bytes (d = 96) every 4 rows, r/4.
//   K (INT8, Q8 kernels): rows of D bytes, rotated by r/2 (d = 128), r/4
//     (d = 64), r/8 (d = 96).
//   V (16-bit, transposing reads: each group of 16 lanes reads 4 consecutive
//     rows, 32 bytes each): rows of 256 bytes rotate by 4(r mod 4) chunks,
//     rows of 128 bytes by 4((r/2) mod 2); rows of 192 bytes already start
//     on different banks.
// Every rotation is a function of the row's low bits only, so it is the same
// for rows 32 apart (the two 32-key halves) and 8 or 16 apart (the two
// halves of a transposing read, successive k-steps): one per-lane offset per
// logical chunk serves all of them.
template <int D, int QS, int NW, bool Q8 = false>
struct Fwd16Smem {
  using T = Tiling<QS, NW>;
  static constexpr int kKRowB = Q8 ? D : 2 * D;  // bytes per K row
  static constexpr int kVRowB = 2 * D;           // bytes per V row
  static constexpr int kKC = kKRowB / 16;        // 16-byte chunks per K row
  static constexpr int kVC = kVRowB / 16;        // 16-byte chunks per V row
  static constexpr int kKTile = kBN * kKRowB;    // bytes
  static constexpr int kVTile = kBN * kVRowB;
  static constexpr int kBytes = T::kKbuf * kKTile + T::kVbuf * kVTile;
  __device__ static __forceinline__ int k_rot(int r) {
    if constexpr (Q8) return D == 128 ? (r >> 1) & 7 : D == 64 ? (r >> 2) & 3 : (r >> 3) & 1;
    else return D == 128 ? r & 15 : D == 64 ? (r >> 1) & 7 : (r >> 2) & 3;
  }
  __device__ static __forceinline__ int v_rot(int r) {
    return D == 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0;
  }
  // LDS byte offsets of logical 16-byte chunk c of row r
  __device__ static __forceinline__ uint32_t k_pos(int r, int c) {
    const int x = c + k_rot(r);
    return (uint32_t)(r * kKRowB + 16 * (x >= kKC ? x - kKC : x));
  }
  __device__ static __forceinline__ uint32_t v_pos(int r, int c) {
    const int x = c + v_rot(r);
    return (uint32_t)(r * kVRowB + 16 * (x >= kVC ? x - kVC : x));
  }
};

// Kernel variants by input layout: contiguous without a bias (the plain loop
// over key blocks), contiguous with a block bias (adds the block-sparse skip)
// and the general strided / packed-sequence layout without and with a block
// bias.  A packed sequence takes its bias blocks from [b, h] of the
// [B,H,nb,nb] bias, counted from its own first token (nb from the longest
// length).
enum Mode { kDense = 0, kBias = 1, kGen = 2, kGenBias = 3 };

// The block bias comes as its own restrict argument: its reads, uniform and
// never written by the kernel, then compile to scalar loads, which do not
// share the in-order vector-load counter with the K/V prefetch.
//
// Q8: the scores come from the 8-bit preparation instead (page 1,
// "SageAttention": the first product in INT8 after K is mean-centred), as
// S^T = Kq Qq^T on the 32x32x32 INT8 instruction with the accumulators
// started from the bit pattern of 1.5 * 2^23 (|S| < 2^22, so the int32 result
// read as fp32 is exactly 1.5 * 2^23 + S), dequantised per 64 x 64 block by
// f = sq * sk * scale * log2(e) folded into the exponent; P and V stay in the
// 16-bit input format for the second product, exactly as in the 16-bit path.
// Workgroups per CU the register budget is set for: 8 waves per CU (two per
// SIMD), or three 4-wave workgroups for the INT8-score instance at d = 128.
template <int D, int NW, bool Q8>
constexpr int kMinBlocks = (Q8 && D == 128 && NW == 4) ? 3 : 8 / NW;

template <int D, bool BF16, bool CAUSAL, int QS, int NW, int MODE, bool Q8 = false>
__global__ __launch_bounds__(64 * NW, (kMinBlocks<D, NW, Q8>)) void fwd16_kernel(Fwd16Params p,
                                                                                  const float* __restrict__ bias,
                                                                                  const float* __restrict__ sk) {
  constexpr bool GEN = MODE == kGen || MODE == kGenBias, HAS_BIAS = MODE == kBias || MODE == kGenBias;
  static_assert(!(Q8 && GEN), "INT8 scores take the dense layout");
  using TL = Tiling<QS, NW>;
  using S = Fwd16Smem<D, QS, NW, Q8>;
  constexpr int kWQ = TL::kWQ, kBM = TL::kBM, kThreads = TL::kThreads;
  constexpr int kKbuf = TL::kKbuf;
  constexpr int kKTile = S::kKTile, kVTile = S::kVTile;
  constexpr int kDT = D / 32;  // 32-row tiles of O^T
  constexpr int kKS = D / 16;  // k-steps of S^T = K Q^T (Q8: D/32 of them)
  constexpr int kChunksK = kBN * S::kKC, kChunksV = kBN * S::kVC;  // 16-byte chunks per tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[S::kBytes];
  uint8_t* const kbase_lds = smem;                   // kKbuf K tiles
  uint8_t* const vbase_lds = smem + kKbuf * kKTile;  // kVbuf V tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Loop over (b, h, query tile) work items (work_queue: per-XCD queues,
  // balanced heavy-first order when the grid is persistent).
  const WorkQueue wq = work_queue(p.nbh, p.nq);
  constexpr bool DENSE = MODE == kDense;
  constexpr int kNK = (kChunksK + kThreads - 1) / kThreads, kNV = kChunksV / kThreads;
  static_assert(kChunksV % kThreads == 0, "V tiles split evenly over the threads");
  u32x4_t qf[QS][kKS];
  // Dense layout without a bias: the next work item's Q rows and first K/V
  // block are loaded during the current item's last block, so a new item
  // starts without waiting for global memory (pre: qf and the LDS buffer b0
  // already hold this item's Q and block 0).
  bool pre = false;
  int b0 = 0;  // LDS buffer of the item's first block
  for (int round = 0;; ++round) {
  int bh, tq;
  if (!work_item(wq, round, p.nq, bh, tq)) break;
  int bh_n = 0, tq_n = 0;
  const bool has_next = DENSE && !Q8 && work_item(wq, round + 1, p.nq, bh_n, tq_n);
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
  // (Q8: the lane holds Qq[row][32kk + 16hf .. +15], one 32-deep step each)
  const int8_t* __restrict__ Qq = Q8 ? p.qq + (size_t)bh * p.np * D : nullptr;
  if constexpr (Q8) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int row = min(qw0 + 32 * qs + l32, N - 1);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qf[qs][kk] = *(const u32x4_t*)(Qq + (size_t)row * D + 32 * kk + 16 * hf);
    }
  } else if (!(DENSE && pre)) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const int row = min(qw0 + 32 * qs + l32, N - 1);
      const uint16_t* src = Q + (size_t)row * qsn + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) qf[qs][kk] = *(const u32x4_t*)(src + 16 * kk);
    }
  }
  // Q8: the wave's queries lie in one 64-row block; its scale and the K
  // block scales (scalar reads) dequantise the scores
  const float sqw = Q8 ? p.sq[(size_t)bh * p.nblk + min(qw0, N - 1) / kBN] : 1.f;
  const float* skrow = Q8 ? sk + (size_t)bh * p.nblk : nullptr;

  const int kend = CAUSAL ? min(N, q0 + kBM) : N;
  const int nkb = (kend + kBN - 1) / kBN;
  // last key block this wave computes (causal: its diagonal block)
  const int wave_last = CAUSAL ? min(nkb - 1, qw0 / kBN) : nkb - 1;
  const bool wave_has_rows = qw0 < N;

  // ---- loader: 16-byte buffer loads straight into LDS.  Round i of wave w
  // fills LDS chunks i*threads + 64w .. +63 of a tile; lane l fetches the
  // global chunk that belongs at LDS chunk p = i*threads + tid (row p / C,
  // logical chunk by the inverse rotation).  The per-lane byte offsets inside
  // a block are fixed; the block offset kb*64 rows is uniform.  Key rows past
  // N read zeros (the buffer descriptor's range check), so every load is
  // unconditional and the V rows past N hold zeros.
  const int krb = Q8 ? D : 2 * ksn, vrb = 2 * vsn;  // global bytes between K / V rows
  const __amdgpu_buffer_rsrc_t krs =
      Q8 ? buffer_rsrc(p.kq + (size_t)bh * p.np * D, (uint32_t)p.np * D) : buffer_rsrc(K, (uint32_t)N * ksn * 2);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V, (uint32_t)N * vsn * 2);
  uint32_t kvo[kNK], vvo[kNV];
#pragma unroll
  for (int i = 0; i < kNK; ++i) {
    const int pc = i * kThreads + tid, row = pc / S::kKC;
    int c = pc % S::kKC - S::k_rot(row);
    c = c < 0 ? c + S::kKC : c;
    kvo[i] = (uint32_t)(row * krb + 16 * c);
  }
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int pc = i * kThreads + tid, row = pc / S::kVC;
    int c = pc % S::kVC - S::v_rot(row);
    c = c < 0 ? c + S::kVC : c;
    vvo[i] = (uint32_t)(row * vrb + 16 * c);
  }
  auto load_kv = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < kNK; ++i) {
      if (kChunksK % kThreads != 0 && i * kThreads + wave * 64 >= kChunksK) continue;  // wave-uniform
      buffer_load16_lds(krs, kbase_lds + buf * kKTile + 16 * (i * kThreads + wave * 64), kvo[i],
                        (uint32_t)(kb * kBN) * krb);
    }
#pragma unroll
    for (int i = 0; i < kNV; ++i)
      buffer_load16_lds(vrs, vbase_lds + buf * kVTile + 16 * (i * kThreads + wave * 64), vvo[i],
                        (uint32_t)(kb * kBN) * vrb);
  };

  // operand read offsets inside a tile (the rotation depends on the row's
  // low bits only): K row l32 at logical chunk 2kk + hf (16-bit: 8 elements
  // per k-step of 16; INT8: 16 bytes per k-step of 32), the other 32-row
  // half 32 rows further; V row vkey (the transposing read's row, k-step
  // rows 16 further, the second half 8 further) at the chunk holding column
  // 32dt + vcol.
  const int g16 = lane >> 4, t16 = lane & 15;
  const int vkey = 4 * hf + (t16 >> 2);
  const int vcol = 16 * (g16 & 1) + 4 * (t16 & 3);
  uint32_t ko[kKS];
#pragma unroll
  for (int kk = 0; kk < kKS; ++kk) ko[kk] = S::k_pos(l32, 2 * kk + hf);
  uint32_t vo[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) vo[dt] = S::v_pos(vkey, (32 * dt + vcol) / 8) + 2 * (vcol % 8);

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
  constexpr bool kSpec = QS == 2;  // speculative softmax (the d = 64 tiling)
  // INT8 scores: the accumulators' start value from one register pair (see
  // magic_tile) at d = 64; at d = 128 that measured 8-9% slower than the
  // per-block splat
  constexpr bool kMagicReg = Q8 && QS == 2;
  const unsigned long long magic_v = kMagicReg ? magic_pair() : 0ull;
  const float sent = pos ? -INFINITY : INFINITY;


  // ---- S^T = K Q^T for one key block (two 32-key tiles x QS query tiles)
  auto qk = [&](int buf, f32x16_t (&s)[2][QS]) {
    if constexpr (Q8) {
      // S^T = Kq Qq^T on top of the offset, exact (A: 16 bytes of a K row per
      // 32-deep step, B: the matching bytes of the Q row)
      const uint8_t* Ks8 = kbase_lds + buf * kKTile;
      i32x16_t si[2][QS];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          if constexpr (kMagicReg) {
            si[T][qs] = magic_tile(magic_v);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) si[T][qs][r] = kMagicBits;
          }
        }
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const u32x4_t a = *(const u32x4_t*)(Ks8 + ko[kk] + 32 * T * S::kKRowB);
#pragma unroll
          for (int qs = 0; qs < QS; ++qs)
            si[T][qs] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                                              __builtin_bit_cast(i32x4_t, qf[qs][kk]), si[T][qs],
                                                              0, 0, 0);
        }
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[T][qs] = __builtin_bit_cast(f32x16_t, si[T][qs]);
      return;
    }
    const uint8_t* Ks = kbase_lds + buf * kKTile;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) s[0][qs] = s[1][qs] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        // row 32T + l32, columns 16kk + 8hf .. +7
        const u32x4_t a = *(const u32x4_t*)(Ks + ko[kk] + 32 * T * S::kKRowB);
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

  // ---- block maximum: raises the running maximum to it where it is larger
  // by more than tau, rescales the running state, and returns the exponent
  // offsets kc = g0 - m (log2 units) of the block.  g0: the block's additive
  // term (the bias in log2 units; for INT8 scores also the offset
  // 1.5 * 2^23 * cf taken off); cf: the scale of the block's raw scores in
  // log2 units (c, or for INT8 scores c * sq * sk).
  auto block_max = [&](f32x16_t (&s)[2][QS], float (&kc)[QS], float g0, float cf, float tau) {
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
      m_blk[qs] = (a0 == sent) ? -INFINITY : fmaf(a0, cf, g0);
      need_any |= m_blk[qs] > m_run[qs] + tau;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const bool need = m_blk[qs] > m_run[qs] + tau;
        const float m_new = need ? m_blk[qs] : m_run[qs];
        const float alpha = need ? exp2_approx(m_run[qs] - m_new) : 1.f;
        l_run[qs] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) o[dt][qs] *= alpha;
        m_run[qs] = m_new;
      }
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) kc[qs] = g0 - ((m_run[qs] == -INFINITY) ? 0.f : m_run[qs]);
  };

  // ---- P = exp2(c*S + bias - m) as the B operand of O^T += V^T P^T.  Masked
  // scores are +-inf, so c*S is -inf and P is 0 (c is never 0: the host
  // passes the smallest normal float for a zero scale).  ls: the lane's sum
  // of the rounded P values the product uses.
  u32x4_t pb[4][QS];
  auto softmax_p = [&](f32x16_t (&s)[2][QS], const float (&kc)[QS], float cf, float (&ls)[QS]) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float lsum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int T = kk >> 1, t = kk & 1;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * t + e;
          const float p0 = exp2_approx(fmaf(s[T][qs][r], cf, kc[qs]));
          const float p1 = exp2_approx(fmaf(s[T][qs][r + 1], cf, kc[qs]));
          const uint32_t pk = pack2<BF16>(p0, p1);
          lsum = sum2_acc<BF16>(pk, lsum);
          pb[kk][qs][e >> 1] = pk;
        }
      }
      ls[qs] = lsum;
    }
  };
  // ---- the block's P: the block maximum first, or (speculative form) P
  // against the running maximum and the block maximum only when a lane's
  // partial sum shows a P above 2^kTau could be present (or m is still -inf)
  auto softmax_block = [&](f32x16_t (&s)[2][QS], float braw, float cf) {
    const float bl = HAS_BIAS ? braw * kLog2e : 0.f;
    const float g0 = Q8 ? fmaf(-kMagic, cf, bl) : bl;
    float kc[QS], ls[QS];
    if constexpr (!kSpec) {
      block_max(s, kc, g0, cf, kTau);
      softmax_p(s, kc, cf, ls);
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) l_run[qs] += ls[qs];
      return;
    }
    bool slow = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      kc[qs] = g0 - m_run[qs];
      slow |= m_run[qs] == -INFINITY;
    }
    if (!__any(slow)) {
      softmax_p(s, kc, cf, ls);
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) slow |= ls[qs] > kSumCap;
    }
    if (__any(slow)) {
      block_max(s, kc, g0, cf, 0.f);
      softmax_p(s, kc, cf, ls);
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) l_run[qs] += ls[qs];
  };
  auto pv = [&](int buf) {
    const uint8_t* Vs = vbase_lds + buf * kVTile;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        const uint8_t* vp = Vs + vo[dt] + 16 * kk * S::kVRowB;
        const u32x2_t lo = lds_read_tr16(vp);
        const u32x2_t hi = lds_read_tr16(vp + 8 * S::kVRowB);
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
    if (more) load_kv(jn, buf ^ 1);
    if (wave_has_rows && jc <= wave_last && (!HAS_BIAS || braw != -INFINITY)) {
      qk(buf, sc);
      if (needs_mask(jc)) apply_mask(jc, sc);
      const float cf = Q8 ? (sqw * skrow[jc]) * c : c;
      softmax_block(sc, braw, cf);
      pv(buf);
    }
    // the next block's loads into LDS are complete before any wave reads them
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
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
    b0 = 0;
    load_kv(min(j0, nkb - 1), 0);
  }
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
    for (int j = 0; j + 1 < nkb; ++j) step(j, j + 1, (b0 + j) & 1, 0.f);
    // the last block: the next item's Q rows and first K/V block are
    // loaded meanwhile (Q after this block's last use of it)
    {
      const int jc = nkb - 1, buf = (b0 + jc) & 1;
      const int qt_n = CAUSAL ? p.nq - 1 - tq_n : tq_n;
      const int qw0_n = qt_n * kBM + wave * kWQ;
      const size_t off_n = (size_t)bh_n * N * D;
      if (has_next) {
        // the next item's block 0 into the other buffer, free since this
        // item's second-to-last block
        const __amdgpu_buffer_rsrc_t krn = buffer_rsrc(p.k + off_n, (uint32_t)N * D * 2);
        const __amdgpu_buffer_rsrc_t vrn = buffer_rsrc(p.v + off_n, (uint32_t)N * D * 2);
#pragma unroll
        for (int i = 0; i < kNK; ++i)
          buffer_load16_lds(krn, kbase_lds + (buf ^ 1) * kKTile + 16 * (i * kThreads + wave * 64), kvo[i], 0);
#pragma unroll
        for (int i = 0; i < kNV; ++i)
          buffer_load16_lds(vrn, vbase_lds + (buf ^ 1) * kVTile + 16 * (i * kThreads + wave * 64), vvo[i], 0);
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
        const float cf = Q8 ? (sqw * skrow[jc]) * c : c;
        softmax_block(sc, 0.f, cf);
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
    // INT8 scores: centring K shifted every score of the row by
    // scale * sq * (Qq . kmean); the LSE adds it back (the Q codes are read
    // again here rather than kept live across the loop)
    float shift = 0.f;
    if constexpr (Q8) {
      if (p.lse != nullptr) {
        const float* kmh = p.kmean + (size_t)bh * D;
        const int row = min(qi, N - 1);
        float dot = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          const u32x4_t qc = *(const u32x4_t*)(Qq + (size_t)row * D + 32 * kk + 16 * hf);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            dot = fmaf((float)(int)(int8_t)(qc[e >> 2] >> (8 * (e & 3))), kmh[32 * kk + 16 * hf + e], dot);
        }
        shift = c * (sqw * xor32_sum(dot));
      }
    }
    if (qi < N) {
      if (p.lse != nullptr && hf == 0)
        p.lse[(size_t)bh * p.N + qi] = l_tot > 0.f ? (m_run[qs] + __log2f(l_tot) + shift) * kLn2 : -INFINITY;
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
  b0 = (b0 + nkb) & 1;
  }  // work items
}

// ws: the 8-bit preparation's workspace (Q8 only)
template <int D, bool BF16, bool CAUSAL, int QS, int NW, int MODE, bool Q8 = false>
hipError_t launch_impl(const FwdArgs& a, hipStream_t stream, const void* ws = nullptr) {
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
  const float* sk = nullptr;
  p.qq = p.kq = nullptr;
  p.sq = p.kmean = nullptr;
  p.np = p.nblk = 0;
  if constexpr (Q8) {
    const Sage8Layout L = sage8_layout(a.B, a.H, a.N, D);
    const char* w = static_cast<const char*>(ws);
    p.qq = reinterpret_cast<const int8_t*>(w + L.qq);
    p.kq = reinterpret_cast<const int8_t*>(w + L.kq);
    p.sq = reinterpret_cast<const float*>(w + L.sq);
    p.kmean = reinterpret_cast<const float*>(w + L.kmean);
    sk = reinterpret_cast<const float*>(w + L.sk);
    p.nblk = L.nblk;
    p.np = L.nblk * kBN;
  }
  // Causal tiles differ in cost, so a persistent grid with the balanced
  // heavy-first order pays where it applies (measured +7% at 4x32x4096,
  // d = 128); equal-cost non-causal tiles run one workgroup per item
  // (persistent was 5% slower).
  // (packed sequences of different lengths: one workgroup per tile; the
  // balance argument of the persistent queues assumes equal heads)
  const int grid = (CAUSAL && !((MODE == kGen || MODE == kGenBias) && a.cu))
                       ? persistent_grid(reinterpret_cast<const void*>(&fwd16_kernel<D, BF16, CAUSAL, QS, NW, MODE, Q8>),
                                         TL::kThreads, p.nbh, p.nq)
                       : p.ntiles;
  if (grid <= 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd16_kernel<D, BF16, CAUSAL, QS, NW, MODE, Q8>), dim3(grid), dim3(TL::kThreads), 0, stream, p,
                     a.bias, sk);
  return hipGetLastError();
}

// Tiling per head dimension, measured on MI355X (TFLOPS; prefill 4x32x4096 /
// long-context 1x32x32768, causal, d = 128; DiT-gated 2x24x16384, d = 64):
//   d = 128: QS1 NW8 743 / 1085 against QS1 NW4 688 / 1003.  Tried and
//     dropped: software-pipelined S of block j+1 next to the softmax of block j
//     (653 / 1030); two wave groups in ping-pong phases (596 / 950: a product
//     phase has one matrix-issuing wave per SIMD, LDS waits are exposed);
//     waves staggered by one product (701 / 983, and register spills).
//   d = 64: QS2 NW4 936-950 against QS1 NW4 854.
template <bool BF16, bool CAUSAL, int MODE>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_impl<64, BF16, CAUSAL, 2, 4, MODE>(a, stream);
  // d = 96: a 64 x 96 tile is 768 16-byte chunks, which 4 waves split evenly
  if (a.d == 96) return launch_impl<96, BF16, CAUSAL, 1, 4, MODE>(a, stream);
  return launch_impl<128, BF16, CAUSAL, 1, 8, MODE>(a, stream);
}

template <bool BF16, bool CAUSAL>
hipError_t launch_g(const FwdArgs& a, hipStream_t stream) {
  if (a.general) return a.bias ? launch_d<BF16, CAUSAL, kGenBias>(a, stream) : launch_d<BF16, CAUSAL, kGen>(a, stream);
  return a.bias ? launch_d<BF16, CAUSAL, kBias>(a, stream) : launch_d<BF16, CAUSAL, kDense>(a, stream);
}

// INT8 scores with the 16-bit P V product: the tilings of the 16-bit path.
template <bool BF16, bool CAUSAL, int MODE>
hipError_t launch_q8_d(const void* ws, const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_impl<64, BF16, CAUSAL, 2, 4, MODE, true>(a, stream, ws);
  if (a.d == 96) return launch_impl<96, BF16, CAUSAL, 1, 4, MODE, true>(a, stream, ws);
  // d = 128: 4-wave workgroups, three per CU (three waves per SIMD from
  // independent workgroups; 163 VGPRs, 48 KB of LDS) on long sequences;
  // measured +3.4% at 1x32x32768, -0.3% at 4x32x4096 and -1.4% at 2x32x8192
  // against 8-wave workgroups (two waves per SIMD)
  if (a.N >= 16384) return launch_impl<128, BF16, CAUSAL, 1, 4, MODE, true>(a, stream, ws);
  return launch_impl<128, BF16, CAUSAL, 1, 8, MODE, true>(a, stream, ws);
}

template <bool BF16, bool CAUSAL>
hipError_t launch_q8_g(const void* ws, const FwdArgs& a, hipStream_t stream) {
  return a.bias ? launch_q8_d<BF16, CAUSAL, kBias>(ws, a, stream) : launch_q8_d<BF16, CAUSAL, kDense>(ws, a, stream);
}

}  // namespace

// Workgroups of `kernel` resident at once on the current device (a multiple
// of 8 when at least 8), cached per kernel and device; -1 on a HIP error.
// The cache is shared by every host thread that launches: entries are
// looked up and added under one lock (the occupancy query itself runs
// outside it; two threads that miss together both query and the first
// stores the same value).
int resident_slots(const void* kernel, int threads) {
  struct Entry { const void* k; int dev; int slots; };
  static Entry cache[64];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].slots;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  int slots = per_cu * cus;
  if (slots >= 8) slots &= ~7;
  if (slots <= 0) return -1;
  std::lock_guard<std::mutex> lock(mu);
  bool known = false;
  for (int i = 0; i < used; ++i) known = known || (cache[i].k == kernel && cache[i].dev == dev);
  if (!known && used < 64) cache[used++] = Entry{kernel, dev, slots};
  return slots;
}

int sorted_order(const void* kernel, int threads, int nbh, int nq, int per_slot) {
  const int slots = resident_slots(kernel, threads);
  if (slots <= 0 || (int64_t)nbh * nq >= (int64_t)per_slot * slots) return 0;
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

hipError_t launch_fwd_q8(const void* ws, const FwdArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.causal ? launch_q8_g<true, true>(ws, a, stream) : launch_q8_g<true, false>(ws, a, stream);
  return a.causal ? launch_q8_g<false, true>(ws, a, stream) : launch_q8_g<false, false>(ws, a, stream);
}

}  // namespace attn
