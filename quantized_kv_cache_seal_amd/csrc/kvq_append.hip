// Append: sink copy or rotation + tq6_0 staging write, one wave per
// (token, KV head, K|V) vector.
//
// SJ-KVaRN 2.1 items 1-2: the first 128 tokens stay at 16 bits; every later
// token's key and value are rotated (2.2) and written to the staging ring as
// tq6_0 (98 bytes per 128 values).  With f16 staging (section 4.1's 16-bit
// alternative) a later token is copied to its ring slot as it is.
#include "kvq_encode.h"

namespace kvq {

__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const Layout& y = a.y;
  const int t = blockIdx.x;
  const int h = blockIdx.y >> 1, kv = blockIdx.y & 1;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int s = a.slot[b];
  const int64_t pos = a.pos0[b] + t;
  const uint16_t* src = (kv ? a.v : a.k) + (((int64_t)b * a.n_tok + t) * y.H + h) * (int64_t)y.D;
  if (pos < kSink) {
    uint16_t* dst = (uint16_t*)(a.arena + y.off_sink) + sink_elem(y, s, a.layer, h, kv, (int)pos);
    for (int i = lane; i < y.D; i += 64) dst[i] = src[i];
    return;
  }
  const int slot = (int)((pos - kSink) % y.cap);
  if (y.f16ring) {
    uint16_t* dst = (uint16_t*)(a.arena + rcode_off(y, s, a.layer, h, kv, slot));
    for (int i = lane; i < y.D; i += 64) dst[i] = src[i];
    return;
  }
  uint8_t* codes = a.arena + rcode_off(y, s, a.layer, h, kv, slot);
  uint16_t* scales = (uint16_t*)(a.arena + rscale_off(y, s, a.layer, h, kv, slot));
  if (y.D == 128) {
    float deq[2];
    encode_chunk<2>(src, codes, scales, lane, a.signs, true, deq);
  } else {
    for (int c = 0; c < y.D / 256; ++c) {
      float deq[4];
      encode_chunk<4>(src + 256 * c, codes + 2 * kQBytes * c, scales + 2 * c, lane, a.signs, false, deq);
    }
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  dim3 grid(a.n_tok, 2 * a.y.H, a.n_seqs);
  hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
