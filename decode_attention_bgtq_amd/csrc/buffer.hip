// fp16 sink and recent-window buffers of the packed cache (the Block-GTQ
// README's AIME "withbuffer" setting: 4 attention-sink tokens and a 128-token
// recent window kept in fp16): the copy of new tokens into them.  The decode
// side is the buffered merge (merge.h).  Definitions: include/bgtq.h.
#include <algorithm>

#include "device.h"
#include "host.h"
#include "merge.h"

namespace bgtq {

// Block x < n_a: new token i = x, copied to sink row t0 + i; block x >= n_a:
// new token i = i_r + (x - n_a), copied to ring row (t0 + i) % n_recent.  One
// 16-byte chunk per thread and step over the n_kv_heads rows of the token.
__global__ __launch_bounds__(256) void buffer_append_kernel(const uint4 *__restrict__ k, const uint4 *__restrict__ v,
                                                            int64_t n_new, int64_t t0, int hkv, uint4 *k_sink,
                                                            uint4 *v_sink, int n_sink, uint4 *k_recent,
                                                            uint4 *v_recent, int n_recent, int n_a, int64_t i_r) {
  const int b = blockIdx.y;
  const bool sink = (int)blockIdx.x < n_a;
  const int64_t i = sink ? (int64_t)blockIdx.x : i_r + ((int64_t)blockIdx.x - n_a);
  const int64_t t = t0 + i;
  const int per = hkv * (kHeadDim / 8);  // 16-byte chunks of one token's rows
  const uint4 *ks = k + ((size_t)b * n_new + i) * per, *vs = v + ((size_t)b * n_new + i) * per;
  for (int c = threadIdx.x; c < per; c += blockDim.x) {
    const int h = c / (kHeadDim / 8), w = c % (kHeadDim / 8);
    const uint4 kx = ks[c], vx = vs[c];
    size_t dst;
    uint4 *kd, *vd;
    if (sink) {
      dst = (((size_t)b * hkv + h) * n_sink + t) * (kHeadDim / 8) + w;
      kd = k_sink, vd = v_sink;
    } else {
      dst = (((size_t)b * hkv + h) * n_recent + (size_t)(t % n_recent)) * (kHeadDim / 8) + w;
      kd = k_recent, vd = v_recent;
    }
    kd[dst] = kx;
    vd[dst] = vx;
  }
}

}  // namespace bgtq

using namespace bgtq;

extern "C" {

bgtq_status bgtq_buffer_append(const uint16_t *k, const uint16_t *v, int32_t batch, int64_t n_new, int64_t t0,
                               int32_t n_kv_heads, uint16_t *k_sink, uint16_t *v_sink, int32_t n_sink,
                               uint16_t *k_recent, uint16_t *v_recent, int32_t n_recent, bgtq_stream stream) {
  const char *nm = "bgtq_buffer_append";
  if (n_sink < 0 || n_sink > kMaxSink || n_recent < 0 || n_recent > kMaxRecent)
    return fail(BGTQ_EINVAL, std::string(nm) + ": n_sink must be 0..64 and n_recent 0..65536");
  if (batch < 1 || batch > 65535 || n_kv_heads < 1 || n_new < 0 || t0 < 0)
    return fail(BGTQ_EINVAL, std::string(nm) + ": batch 1..65535, n_kv_heads >= 1, n_new >= 0, t0 >= 0");
  if ((n_sink && (!k_sink || !v_sink)) || (n_recent && (!k_recent || !v_recent)))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null buffer with a non-zero count");
  if (n_new && (!k || !v)) return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_sink | (uintptr_t)v_sink | (uintptr_t)k_recent |
       (uintptr_t)v_recent) & 15)
    return fail(BGTQ_EINVAL, std::string(nm) + ": every pointer must be 16-byte aligned");
  // new tokens that reach the sink: t0 + i < n_sink; the ring: the last n_recent
  const int64_t n_a64 = t0 < n_sink ? std::min<int64_t>(n_new, n_sink - t0) : 0;
  const int64_t i_r = n_recent ? std::max<int64_t>(0, n_new - n_recent) : n_new;
  const int64_t n_b = n_new - i_r;
  const int n_a = (int)n_a64;
  if (n_a + n_b == 0) return BGTQ_OK;
  const dim3 grid((unsigned)(n_a + n_b), batch);
  buffer_append_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(
      (const uint4 *)k, (const uint4 *)v, n_new, t0, n_kv_heads, (uint4 *)k_sink, (uint4 *)v_sink, n_sink,
      (uint4 *)k_recent, (uint4 *)v_recent, n_recent, n_a, i_r);
  return launch_status(nm);
}

}  // extern "C"
