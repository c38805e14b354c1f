// attn_internal.hpp -- launch interface between the C ABI layer and the
// kernels.  Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

enum OutKind : int { kOutF16 = 0, kOutBF16 = 1, kOutF32 = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;         // nullable
  const float* bias;  // nullable, [B,H,nb,nb]
  int B, H, N, d;
  int causal;
  float scale;
  int out_kind;       // OutKind
  // general layout (16-bit strided entry point): element strides (batch,
  // head, token) of q, k, v, o; cu (nullable, device) packs sequences
  bool general = false;
  int64_t strides[12] = {};
  const int* cu = nullptr;
};

// Grid for a launch over nbh * nq (head, query tile) items: the number of
// workgroups of `kernel` resident at once on the current device (CUs x
// workgroups per CU, a multiple of 8) when the persistent per-XCD queues
// balance exactly and there is more than one round, else nbh * nq (one
// workgroup per item); -1 on a HIP error.
int persistent_grid(const void* kernel, int threads, int nbh, int nq);
// Whether a one-workgroup-per-item causal launch of nbh * nq items should
// start its items heaviest first across the heads (work_queue's lpt order):
// when there are fewer than 10 items per resident workgroup slot, the
// balance of the last rounds matters more than L2 sharing.  Measured on the
// 8-bit forward: +10% at 5.3 items per slot (4x32x4096), -1.4% at 10.7
// (1x32x32768).
// Returns the number of heads per group of that order (0: head-major).
int sorted_order(const void* kernel, int threads, int nbh, int nq, int per_slot = 10);

// 16-bit path (fp16 when bf16 == false).
hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t stream);

// Backward of the 16-bit path: gradients of a loss L given dO = dL/dO and the
// forward's O and LSE.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // forward output, input dtype or fp32 (o_f32)
  const void* dout;   // dL/dO, input dtype
  const float* lse;   // forward LSE [B,H,N], natural log
  void* dq;
  void* dk;
  void* dv;
  float* dbias;       // nullable, [B,H,nb,nb], overwritten
  const float* bias;  // nullable, [B,H,nb,nb]
  float* delta;       // workspace [B,H,N]: rowsum(dO * O)
  int B, H, N, d;
  int causal;
  float scale;
  int grad_kind;      // OutKind of dq, dk, dv
  bool o_f32;         // o holds fp32 values
};
hipError_t launch_bwd16(const BwdArgs& a, bool bf16, hipStream_t stream);
// the key-side kernel (dK, dV, dbias), built without the VGPR-form option
hipError_t launch_bwd16_kv(const BwdArgs& a, bool bf16, hipStream_t stream);

// 8-bit path.
struct Sage8Layout {
  // byte offsets inside the workspace, each 256-byte aligned
  size_t qq, kq, vq, sq, sk, sv, vinv, kmean, kpart, vpart;
  size_t total;
  int nblk;    // 64-row blocks of the token count padded to a multiple of 128
  int nchunk;  // token chunks of the column reductions
};
Sage8Layout sage8_layout(int B, int H, int N, int d);
// fmt: kPrepInt8 (the INT8 recipe), kPrepFp8 (Q and K in e4m3 blocks, the
// FP8-QK variant) or kPrepInt8NoV (INT8 Q and K only, for the
// 16-bit P V variant: V's statistics, codes and regions are not touched);
// the forward must be told the format the preparation wrote.
// strides: element strides (batch, head, token) of q, k, v with d
// contiguous (9 values); nullptr for contiguous [B,H,N,d].
// cu (nullable, device int32 [B+1]): packed sequences along the token axis
// (the batch strides are then unused); each fills its own workspace slot.
enum PrepFormat : int { kPrepInt8 = 0, kPrepFp8 = 1, kPrepInt8NoV = 2 };
hipError_t launch_sage8_prep(const void* q, const void* k, const void* v, bool bf16, int B, int H,
                             int N, int d, const int64_t* strides, const int* cu, void* ws, hipStream_t stream,
                             int fmt);
// INT8 scores from the workspace of launch_sage8_prep (INT8 format) with the
// 16-bit P V product: a.v is the 16-bit V [B,H,N,d] (fp16 unless bf16), O
// contiguous [B,H,N,d]; a.q and a.k are unused.
hipError_t launch_fwd_q8(const void* ws, const FwdArgs& a, bool bf16, hipStream_t stream);
// O is written with the element strides a.strides[9..11] (batch, head,
// token) when a.general, else contiguous [B,H,N,d].  With a.cu (packed
// sequences) batch entry b writes its rows from token a.cu[b], and a block
// bias is read at [b, h] with block indices counted from that token.
hipError_t launch_fwd_sage8(const void* ws, const FwdArgs& a, hipStream_t stream, bool qk_fp8);

}  // namespace attn
