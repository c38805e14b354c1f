// attn_common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// Register layouts used throughout (verified on gfx950 for the 32x32 MFMA
// family): for D = A*B with A of 32 rows and B of 32 columns,
//   A operand: lane l holds row (l % 32), a lane-half-specific slice of k;
//   B operand: lane l holds column (l % 32), the same k slice as A;
//   C/D:       lane l holds column (l % 32) and rows
//              8*(r/4) + 4*(l/32) + (r%4) for register r = 0..15.
// Because k is a reduction index, any assignment of k to (lane half,
// element) works as long as A and B agree; the kernels exploit this to feed
// the accumulator of one product straight into the next as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// INT8 score products start their accumulators from the bit pattern of
// 1.5 * 2^23: with |S| < 2^22 (true for d <= 128: 128 * 127^2 < 2^22) the
// int32 sum 0x4B400000 + S read as fp32 is exactly 12582912 + S, so the
// scores leave the matrix unit as floats and the offset is folded into the
// exponent.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

// 32x32x16 MFMA on 16-bit inputs packed as 4 dwords per lane.
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two fp32 values to a packed pair of 16-bit floats, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  f32x2_t v = {x, y};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
}

// acc + x.lo + x.hi for a packed pair of 16-bit floats (one dot-product
// instruction against the pair (1, 1)).
template <bool BF16>
__device__ __forceinline__ float sum2_acc(uint32_t x, float acc) {
  if constexpr (BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                           __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), __builtin_bit_cast(f16x2_t, 0x3C003C00u),
                                  acc, false);
  }
}

// Values of this lane and of its partner (lane ^ 32).  With both operands
// equal, permlane32_swap returns (x[l], x[l^32]) in some order per lane, so
// max/sum of the pair is the reduction over the two lane halves.  The two
// results are first copied into plain integers: bit-casting the builtin's
// result elements directly to float lowers both to the first element.
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  const uint32_t u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t u0 = p[0];
  const uint32_t u1 = p[1];
  a = __uint_as_float(u0);
  b = __uint_as_float(u1);
}
__device__ __forceinline__ float xor32_max(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor32_min(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fminf(a, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return a + b;
}

// One fp16 / bf16 value (raw bits) to fp32, exactly.
template <bool BF16>
__device__ __forceinline__ float in_to_f32(uint16_t x) {
  if constexpr (BF16) {
    return __uint_as_float((uint32_t)x << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, x);
  }
}

// Transposing LDS read of four 16-bit values.  Within each group of 16 lanes,
// lane 4a+b receives element b of the 8-byte rows addressed by lanes a, a+4,
// a+8 and a+12 of the group (verified on gfx950).
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer access: base and size in scalar registers, a per-lane byte
// offset and a uniform byte offset; loads past `bytes` return zeros.  The
// third descriptor word selects 32-bit data (required for untyped loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// One 16-byte buffer load per lane straight into LDS: the wave's 64 chunks
// land at lds + 16 * lane (lds wave-uniform: it goes to M0; verified on
// gfx950).  The LDS write happens when the load returns; the vector-memory
// counter covers it.  The intrinsic exists only in the device pass.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                                  uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8) that waits for every outstanding vector memory
// operation and for nothing else.  Placed after a kernel's prologue loads, it
// tells the compiler's wait tracking that those loads are done, so no wait on
// them is left inside the main loop (where, the counter being in order, it
// would also wait for the loads that prefetch the next block).
constexpr int kWaitVm0 = 0x0F70;

// The INT8 score accumulators' start value, kMagicBits in all 16 registers
// of a 32x32 tile, built from one vector register pair made once per
// kernel.  From a splat of the constant the compiler rebuilds the 16-register
// tuple in scalar registers and copies it over at every key block; from a
// loop-invariant register pair it keeps one tuple live and feeds it to the
// first product of every block as its C operand (no per-block moves).
__device__ __forceinline__ unsigned long long magic_pair() {
  unsigned long long v = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("v_mov_b64 %0, %1" : "=v"(v) : "s"(((unsigned long long)kMagicBits << 32) | (unsigned)kMagicBits));
#endif
  return v;
}
__device__ __forceinline__ i32x16_t magic_tile(unsigned long long pair) {
  typedef unsigned long long u64x8_t __attribute__((ext_vector_type(8)));
  u64x8_t m;
#pragma unroll
  for (int r = 0; r < 8; ++r) m[r] = pair;
  return __builtin_bit_cast(i32x16_t, m);
}

// Block-sparse gating by a per-head [nb x nb] block bias (fp32, natural-log
// units; -inf gates a 64 x 64 block off).  A workgroup tile spans kRows
// query blocks starting at qb_lo; a key block is visited when its bias is
// not -inf for at least one of them.  The gate holds a chunk of 64 key
// blocks: a bit mask of the visited ones (one ballot per query block) and,
// in lane i, the bias of key block cb + i for the wave's own query block, so
// stepping to the next block costs a few scalar instructions and one lane
// read; a new chunk is read once per 64 key blocks.  Reads go through a
// buffer resource: reads past the head return 0 and are masked out.
template <int kRows>
struct BlockGate {
  __amdgpu_buffer_rsrc_t rs;
  int nb, nkb, qb_lo, rw;
  int cb;         // first key block of the chunk held (a multiple of 64)
  uint64_t rest;  // visited blocks of the chunk not yet returned (bit i: cb + i)
  float wv;       // lane i: bias of key block cb + i for query block qb_lo + rw

  // head: this head's bias; nkb: key blocks of the tile; rw: the wave's
  // query block within the tile
  __device__ __forceinline__ BlockGate(const float* head, int nb_, int qb_lo_, int nkb_, int rw_)
      : nb(nb_), nkb(nkb_), qb_lo(qb_lo_), rw(rw_), cb(0), rest(0), wv(-INFINITY) {
    rs = buffer_rsrc(head, (uint32_t)nb * (uint32_t)nb * 4u);
  }
  __device__ void load_chunk(int c) {
    const int lane = threadIdx.x & 63;
    cb = c;
    rest = 0;
    wv = -INFINITY;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (qb_lo + r >= nb) break;
      const float x = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * (uint32_t)lane,
                                                      4u * (uint32_t)((qb_lo + r) * nb + c), 0));
      rest |= __ballot(c + lane < nkb && x != -INFINITY);
      if (r == rw) wv = x;
    }
  }
  // the next visited key block in increasing order (nkb when none is left);
  // the chunk held afterwards contains it
  __device__ __forceinline__ int next() {
    while (rest == 0) {
      if (cb + 64 >= nkb) return nkb;
      load_chunk(cb + 64);
    }
    const int t = (int)__builtin_ctzll(rest);
    rest &= rest - 1;
    return cb + t;
  }
  // the first visited key block (nkb when none)
  __device__ __forceinline__ int first() {
    load_chunk(0);
    return next();
  }
  // the wave's bias of key block j, which the chunk held must contain
  __device__ __forceinline__ float wave_bias(int j) const {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), j - cb));
  }
};

// Work items (b*h, query tile) of a (possibly persistent) grid.  Workgroups
// are handed to the 8 XCDs round-robin, so workgroup w runs on XCD w % 8.
// When B*H is a multiple of 8, XCD x owns the heads x, x+8, ... (a head's
// keys and values stay in one L2) and serves them head by head, tiles in
// order (heaviest first for causal callers), with the n workgroups on it as
// slots: in round k, slot s takes queue entry k*n + s, or k*n + n-1-s in odd
// rounds.  This pairs entries e and 2n-1-e; when 2n is a multiple of the
// tiles per head those two tiles cost the same together for every pair, so
// the slots are balanced (the host makes the grid persistent only then:
// also every slot must get whole pairs of rounds).
// With one workgroup per item the order is XCD-grouped, head-major (the
// concurrent workgroups share one head's keys and values in L2), or with
// lpt tile-major across the XCD's heads: tile position 0 of every head, then
// position 1, ...  The dispatcher starts the workgroups in that order as
// slots free up, which for causal tiles (position 0 the heaviest) is list
// scheduling heaviest first.  The host asks for it when there are few items
// per slot, where the balance matters more than the L2 sharing
// (sorted_order).
struct WorkQueue {
  int nslot, slot, qlen, xcd, split, lpt;
};
__device__ __forceinline__ WorkQueue work_queue(int nbh, int nq, int lpt = 0) {
  const int G = gridDim.x, w = blockIdx.x;
  WorkQueue q;
  q.split = (nbh & 7) == 0 && (G & 7) == 0;
  q.nslot = q.split ? G >> 3 : G;
  q.slot = q.split ? w >> 3 : w;
  q.qlen = (q.split ? nbh >> 3 : nbh) * nq;
  q.xcd = w & 7;
  q.lpt = q.nslot >= q.qlen ? lpt : 0;  // one workgroup per item
  return q;
}
// Returns false when the workgroup is done; else the head bh and the tile
// position r within the head (causal callers process tile nq-1-r).
__device__ __forceinline__ bool work_item(const WorkQueue& q, int round, int nq, int& bh, int& r) {
  if (q.lpt) {
    // groups of lpt heads in turn, tile-major within a group
    if (round > 0 || q.slot >= q.qlen) return false;
    const int nh = q.qlen / nq;  // heads served by this queue
    const int g = min(q.lpt, nh), per = g * nq;
    const int grp = q.slot / per, h0 = grp * g, gh = min(g, nh - h0);
    const int jj = q.slot - grp * per;
    r = jj / gh;
    const int hl = h0 + (jj - r * gh);
    bh = q.split ? q.xcd + 8 * hl : hl;
    return true;
  }
  const int j = round * q.nslot + ((round & 1) ? q.nslot - 1 - q.slot : q.slot);
  if (j >= q.qlen) return false;
  const int hl = j / nq;
  r = j - hl * nq;
  bh = q.split ? q.xcd + 8 * hl : hl;
  return true;
}

}  // namespace attn
