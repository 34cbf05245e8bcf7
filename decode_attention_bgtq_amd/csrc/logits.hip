// Key logits read from the packed key cache alone (K-only).
//
// "RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract: the method
// is judged by how well the quantised keys keep the RoPE query-key logits,
// with the keys alone quantised (K-only) at 2 and 3 bits per coordinate; the
// Block-GTQ README's per-layer diagnostic takes that error over the last
// positions of each layer.  This entry point returns the logits q . k_hat of
// a block of queries against a range of cache tokens, computed from the
// library's own packed keys, so that the diagnostic is taken from the cache
// the decode reads.
//
// A TurboQuant-MSE key group is stored in its rotated space, so the logit is
// taken there: q . k_hat = sum_g n_g sum_i (Pi_g q_g)_i c_w[code_i] / sqrt(d_g),
// with the rotated queries Pi_g q_g from bgtq_rotate_queries (group order).
#include <cmath>

#include "device.h"
#include "host.h"

namespace bgtq {

struct LogitArgs {
  const uint8_t *consts;
  const float *q_rot;  // [batch][n_q][n_q_heads][128], group order
  const uint32_t *kc;
  const uint16_t *kn;
  TileMap map;
  int64_t t0, n_k;
  int32_t n_q;
  int32_t tile0;  // first cache tile of the token range
  float *logits;  // [batch][n_q_heads][n_q][n_k]
};

// One workgroup of four waves per (cache tile, KV head, sequence).
//  1. The tile's keys are rebuilt in the rotated space of their groups,
//     khat[p][token] = n_g * c_w[code_p] / sqrt(d_g) for group-order position p
//     (0 past the coded positions), fp32, in LDS: thread (token, quarter) the
//     positions 32 quarter .. 32 quarter + 31 of its token.  The key words are
//     staged in LDS first ([word][token], two zero rows after the last word)
//     so that a code that crosses a word boundary reads both words.
//  2. Every lane keeps its token's 128 values in registers; wave w takes the
//     query rows (query n, head of the group) r = w, w + 4, ..., each one a
//     wave-uniform row of q_rot, and writes one logit per token.
__global__ __launch_bounds__(256) void logits_kernel(const LogitArgs a) {
  __shared__ float khat[kHeadDim][kTile];
  __shared__ uint32_t words[kMaxWK + 2][kTile];
  __shared__ float cs[kMaxGroups][16];  // c_w[code] / sqrt(d_g) per group
  const ConstHeader *hd = hdr_of(a.consts);
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tile = a.tile0 + (int)blockIdx.x;
  const int tid = threadIdx.x, tok = tid & 63, wave = tid >> 6;
  const KvhDesc *kd = (const KvhDesc *)(a.consts + hd->off_kvh) + kvh;
  const int wk = hd->wk, G = hd->group, hq = hd->n_q_heads;
  const int64_t ti = tile_at(a.map, b, kvh, tile);
  for (int idx = tid; idx < (kMaxWK + 2) * kTile; idx += 256) {
    const int j = idx / kTile, t = idx % kTile;
    words[j][t] = j < wk ? a.kc[(size_t)ti * wk * kTile + (size_t)j * kTile + t] : 0u;
  }
  if (tid < kMaxGroups * 16) {
    const int g = tid >> 4, c = tid & 15;
    float v = 0.f;
    if (g < kd->n_groups) {
      const KGroupDesc &gd = kd->g[g];
      if (c < (1 << gd.w)) v = (float)(hd->cent[gd.w - 1][c] / sqrt((double)gd.d));
    }
    cs[g][c] = v;
  }
  __syncthreads();
  {
    const uint16_t *nrm = a.kn + ((size_t)ti * kTile + tok) * 4;
    int g = 0;
    for (int p = wave * 32; p < wave * 32 + 32; ++p) {
      float v = 0.f;
      if (p < kd->d_nz) {
        while (p >= kd->g[g].pos + kd->g[g].d) ++g;
        const KGroupDesc &gd = kd->g[g];
        const int bit = gd.bit_off + gd.w * (p - gd.pos), wi = bit >> 5, sh = bit & 31;
        const uint64_t pair = (uint64_t)words[wi][tok] | ((uint64_t)words[wi + 1][tok] << 32);
        const uint32_t code = (uint32_t)(pair >> sh) & ((1u << gd.w) - 1u);
        v = h2f(nrm[4 - gd.w]) * cs[g][code];
      }
      khat[p][tok] = v;
    }
  }
  __syncthreads();
  float kr[kHeadDim];
#pragma unroll
  for (int i = 0; i < kHeadDim; ++i) kr[i] = khat[i][tok];
  const int64_t pos = (int64_t)tile * kTile + tok;
  const bool valid = pos >= a.t0 && pos < a.t0 + a.n_k;
  const int rows = a.n_q * G;
  for (int r = wave; r < rows; r += 4) {
    const int n = r / G, h = kvh * G + r % G;
    const float *qr = a.q_rot + (((size_t)b * a.n_q + n) * hq + h) * kHeadDim;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < kHeadDim; i += 4) {
      s0 = fmaf(qr[i], kr[i], s0);
      s1 = fmaf(qr[i + 1], kr[i + 1], s1);
      s2 = fmaf(qr[i + 2], kr[i + 2], s2);
      s3 = fmaf(qr[i + 3], kr[i + 3], s3);
    }
    if (valid) a.logits[(((size_t)b * hq + h) * a.n_q + n) * a.n_k + (pos - a.t0)] = (s0 + s1) + (s2 + s3);
  }
}

}  // namespace bgtq

using namespace bgtq;

extern "C" bgtq_status bgtq_key_logits(const bgtq_plan *plan, const void *dev_consts, const float *q_rot,
                                       int32_t n_q, const uint32_t *k_codes, const uint16_t *k_norms,
                                       int64_t capacity, int32_t batch, int64_t t0, int64_t n_k, float *logits,
                                       bgtq_stream stream) {
  if (!plan || !dev_consts || !q_rot || !k_norms || !logits)
    return fail(BGTQ_EINVAL, "bgtq_key_logits: null pointer");
  const Plan &p = plan->p;
  if (p.hdr.wk > 0 && !k_codes) return fail(BGTQ_EINVAL, "bgtq_key_logits: null k_codes");
  if (batch < 1 || batch > 65535 || n_q < 1) return fail(BGTQ_EINVAL, "bgtq_key_logits: batch 1..65535, n_q >= 1");
  if (capacity < 1 || t0 < 0 || n_k < 0 || t0 + n_k > capacity)
    return fail(BGTQ_ECAPACITY, "bgtq_key_logits: tokens [t0, t0 + n_k) must lie in [0, capacity)");
  if (n_k == 0) return BGTQ_OK;
  const int64_t tile0 = t0 / kTile, tile1 = (t0 + n_k - 1) / kTile;
  LogitArgs a{};
  a.consts = (const uint8_t *)dev_consts;
  a.q_rot = q_rot;
  // plans without key bits have no key words; the kernel reads none (wk = 0)
  a.kc = k_codes;
  a.kn = k_norms;
  a.map = contiguous_map(p.desc.n_kv_heads, capacity);
  a.t0 = t0;
  a.n_k = n_k;
  a.n_q = n_q;
  a.tile0 = (int32_t)tile0;
  a.logits = logits;
  const dim3 grid((unsigned)(tile1 - tile0 + 1), p.desc.n_kv_heads, batch);
  logits_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(a);
  return launch_status("bgtq_key_logits");
}
