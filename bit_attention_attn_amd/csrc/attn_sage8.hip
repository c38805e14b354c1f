// attn_sage8.hip -- 8-bit path: workspace layout (kernels follow).
#include "attn_common.hpp"
#include "attn_internal.hpp"

namespace attn {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Sage8Layout sage8_layout(int B, int H, int N, int d) {
  Sage8Layout L{};
  const size_t bh = (size_t)B * H;
  const size_t np = (size_t)((N + 127) / 128) * 128;  // tokens padded to whole 128-row tiles
  L.nblk = (int)(np / 64);
  L.nchunk = (N + 255) / 256;
  size_t off = 0;
  L.qq = off; off = align256(off + bh * np * d);
  L.kq = off; off = align256(off + bh * np * d);
  L.vq = off; off = align256(off + bh * np * d);
  L.sq = off; off = align256(off + bh * L.nblk * sizeof(float));
  L.sk = off; off = align256(off + bh * L.nblk * sizeof(float));
  L.sv = off; off = align256(off + bh * d * sizeof(float));
  L.kmean = off; off = align256(off + bh * d * sizeof(float));
  L.kpart = off; off = align256(off + bh * (size_t)L.nchunk * d * sizeof(double));
  L.vpart = off; off = align256(off + bh * (size_t)L.nchunk * d * sizeof(float));
  L.total = off;
  return L;
}

hipError_t launch_sage8_prep(const void*, const void*, const void*, bool, int, int, int, int, void*,
                             hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_fwd_sage8(const void*, const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
