// fp16 decode attention over an uncompressed KV cache on gfx950: the baseline
// the packed-cache path is compared with ("RoPE-Aware Bit Allocation for
// KV-Cache Quantization", Abstract: the packed path against fp16
// FlashAttention-2 decode at 128K; Block-GTQ README, end-to-end decode
// benchmark).  Same split-sequence structure as the packed decode, same online
// softmax and split merge, fp32 accumulation:
//  * one workgroup of 4 waves per (split, KV head, sequence); per 64-token tile
//    of a wave, the logits on the 16x16x32 fp16 matrix cores (fp16 products,
//    fp32 sums): per group of 16 tokens and 32 coordinates one product whose B
//    operand is 16 bytes of a key row per lane (each load instruction reads 64
//    contiguous bytes of 16 rows) and whose A operand (the queries, from LDS)
//    has its rows at the token group's row block, so that the four groups'
//    results land in one accumulator with lane = token (a lane-per-row read
//    of the keys moved 8x the key bytes through the caches);
//  * the softmax weights go to the wave's LDS row; lane (j, c) then sums the
//    value rows of the tokens 4u + j, u < 16, over its 8 coordinates 8c..8c+7
//    (16-byte loads, fp32 accumulation), and the four token phases j are
//    added with lane shuffles;
//  * the waves merge into one partial per split, the merge kernel combines
//    the splits.
#include <algorithm>
#include <cmath>

#include "device.h"
#include "host.h"
#include "merge.h"

namespace bgtq {

constexpr int kF16Waves = 4;
constexpr int kF16Threads = 64 * kF16Waves;
constexpr float kF16RescaleSlack = 8.f;  // log2 units, as in the packed decode

struct F16Args {
  const uint16_t *q;  // [batch][hq][128]
  const uint16_t *k;  // [batch][capacity][hkv][128]
  const uint16_t *v;  // [batch][capacity][hkv][128]
  const int32_t *seq_lens;
  float *part;        // split partials [batch][hq][n_splits][kPartStride]
  int64_t capacity, max_seq_len;
  int hkv, hq, tiles_per_split, n_splits;
  float kscale;       // softmax scale * log2(e)
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int G>
__global__ __launch_bounds__(kF16Threads) void f16_decode_kernel(const F16Args a) {
  constexpr int P = (G + 3) / 4;  // passes of four heads
  // A operands [pass][token group][32-coordinate chunk][lane]: lane l holds row
  // l % 16 = 4 tg' + m (head 4 pass + m if tg' is the token group, else zero),
  // coordinates 32 kc + 8 (l / 16) .. + 7
  // (after the tile loop the same LDS holds the wave merge: four workgroups
  // per compute unit fit with eight heads)
  constexpr int kQaBytes = P * 16 * 64 * 16, kMrgBytes = kF16Waves * G * kPartStride * 4;
  __shared__ __attribute__((aligned(16))) uint8_t qa_mrg[kQaBytes > kMrgBytes ? kQaBytes : kMrgBytes];
  f16x8(*qa)[4][4][64] = (f16x8(*)[4][4][64])qa_mrg;
  float *mrg = (float *)qa_mrg;
  __shared__ __attribute__((aligned(16))) float pw[kF16Waves][G][kTile];     // softmax weights
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t *qg = a.q + ((size_t)b * a.hq + (size_t)kvh * G) * kHeadDim;
  for (int i = tid; i < P * 16 * 64; i += kF16Threads) {
    const int l = i & 63, kc = (i >> 6) & 3, tg = (i >> 8) & 3, pass = i >> 10;
    const int r = l & 15, h = 4 * pass + (r & 3);
    f16x8 v;
    if ((r >> 2) == tg && h < G) {
      const uint4 w = *(const uint4 *)(qg + (size_t)h * kHeadDim + 32 * kc + 8 * (l >> 4));
      v = __builtin_bit_cast(f16x8, w);
    } else {
      v = (f16x8){0, 0, 0, 0, 0, 0, 0, 0};
    }
    qa[pass][tg][kc][l] = v;
  }
  int64_t seq = a.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > a.max_seq_len ? a.max_seq_len : seq);
  __syncthreads();

  const int ntile = (int)((seq + kTile - 1) / kTile);
  const int tile_lo = split * a.tiles_per_split;
  const int tile_hi = min(tile_lo + a.tiles_per_split, ntile);
  const size_t tstride = (size_t)a.hkv * kHeadDim;  // elements between consecutive tokens
  const uint16_t *kb = a.k + ((size_t)b * a.capacity * a.hkv + kvh) * kHeadDim;
  const uint16_t *vb = a.v + ((size_t)b * a.capacity * a.hkv + kvh) * kHeadDim;
  const int j = lane >> 4, d0 = 8 * (lane & 15);
  float mrun[G], lsum[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mrun[h] = -INFINITY, lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  for (int tile = tile_lo + wave; tile < tile_hi; tile += kF16Waves) {
    // ---- logits: token group tg = lanes' tokens 16 tg .. 16 tg + 15; lane l
    // reads 16 bytes of row 16 tg + l % 16 at byte 64 kc + 16 (l / 16) (rows
    // past the sequence read its last token); the result has lane = token
    const int64_t t = (int64_t)tile * kTile + lane;
    const bool valid = t < seq;
    uint4 kv[4][4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int64_t tr = (int64_t)tile * kTile + 16 * tg + (lane & 15);
      const uint4 *kr = (const uint4 *)(kb + (size_t)(tr < seq ? tr : seq - 1) * tstride) + (lane >> 4);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) kv[tg][kc] = kr[4 * kc];
    }
    f32x4 sacc[P];
#pragma unroll
    for (int pass = 0; pass < P; ++pass) {
      sacc[pass] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          sacc[pass] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[pass][tg][kc][lane],
                                                             __builtin_bit_cast(f16x8, kv[tg][kc]), sacc[pass], 0, 0, 0);
    }
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = sacc[h >> 2][h & 3];
    // ---- online softmax (log2 domain), lazy rescale as in the packed decode
    float l[G];
    bool up = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = valid ? sc[h] * a.kscale : -INFINITY;
      up = up || l[h] > mrun[h] + kF16RescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(mrun[h], wave_max(l[h]));
        const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mn);
        lsum[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        mrun[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = __builtin_amdgcn_exp2f(l[h] - mrun[h]);
      lsum[h] += p;
      pw[wave][h][lane] = p;
    }
    wave_sync_lds();
    // ---- values: lane (j, c) takes tokens 4u + j and coordinates 8c .. 8c + 7
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tt = 4 * u + j;
      const int64_t tok = (int64_t)tile * kTile + tt;
      const uint4 vv = *(const uint4 *)(vb + (size_t)(tok < seq ? tok : seq - 1) * tstride + d0);
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = pw[wave][h][tt];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h][2 * e] = fmaf(p, h2f((uint16_t)(w4[e] & 0xFFFFu)), acc[h][2 * e]);
          acc[h][2 * e + 1] = fmaf(p, h2f((uint16_t)(w4[e] >> 16)), acc[h][2 * e + 1]);
        }
      }
    }
    wave_sync_lds();  // the weights row is rewritten by the next tile
  }
  // ---- the four token phases of each coordinate, then the waves of the split
  __syncthreads();  // every wave is past its last read of the query operands
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = wave_sum(lsum[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16);
      acc[h][e] += __shfl_xor(acc[h][e], 32);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float *rr = mrg + (wave * G + h) * kPartStride;
    if (lane == 0) rr[0] = mrun[h], rr[1] = lsum[h];
    if (j == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rr[4 + d0 + e] = acc[h][e];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += kF16Threads) {
    const int h = idx / kHeadDim, i = idx % kHeadDim;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kF16Waves; ++w) mx = fmaxf(mx, mrg[(w * G + h) * kPartStride]);
    float s = 0.f, lt = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kF16Waves; ++w) {
        const float *rr = mrg + (w * G + h) * kPartStride;
        const float f = __builtin_amdgcn_exp2f(rr[0] - mx);
        s = fmaf(f, rr[4 + i], s);
        lt = fmaf(f, rr[1], lt);
      }
    }
    float *o = a.part + ((((size_t)b * a.hq + (size_t)kvh * G + h) * a.n_splits) + split) * kPartStride;
    o[4 + i] = s;
    if (i == 0) o[0] = mx, o[1] = lt;
  }
}

typedef void (*f16_fn)(const F16Args);

f16_fn pick_f16(int g) {
  switch (g) {
    case 1: return f16_decode_kernel<1>;
    case 2: return f16_decode_kernel<2>;
    case 4: return f16_decode_kernel<4>;
    default: return f16_decode_kernel<8>;
  }
}

struct F16Layout {
  int n_splits, tiles_per_split;
  size_t total;
};

F16Layout f16_layout(int batch, int hkv, int hq, int64_t max_seq_len) {
  F16Layout d{};
  const int tiles = (int)((max_seq_len + kTile - 1) / kTile);
  const int target = 4 * device_cus();  // four workgroups of four waves per CU
  int s = (target + batch * hkv - 1) / (batch * hkv);
  s = std::max(1, std::min({s, (tiles + 2 * kF16Waves - 1) / (2 * kF16Waves), kMaxSplits}));
  const int tps = (tiles + s - 1) / s;
  d.n_splits = (tiles + tps - 1) / tps;
  d.tiles_per_split = tps;
  d.total = (((size_t)batch * hq * d.n_splits * kPartStride * 4) + 255) & ~(size_t)255;
  return d;
}

}  // namespace bgtq

using namespace bgtq;

extern "C" {

bgtq_status bgtq_fp16_decode_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                            int64_t max_seq_len, size_t *bytes) {
  if (!bytes) return fail(BGTQ_EINVAL, "bgtq_fp16_decode_workspace_size: null pointer");
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || max_seq_len < 1)
    return fail(BGTQ_EINVAL, "bgtq_fp16_decode_workspace_size: sizes must be positive");
  *bytes = f16_layout(batch, n_kv_heads, n_q_heads, max_seq_len).total;
  return BGTQ_OK;
}

bgtq_status bgtq_fp16_decode_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads, int64_t capacity,
                                  const int32_t *seq_lens, int64_t max_seq_len, float softmax_scale,
                                  uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream) {
  if (!q || !k || !v || !seq_lens || !out || !workspace) return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: null pointer");
  if (batch < 1 || batch > 65535) return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: batch must be 1..65535");
  if (n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: query heads per KV head must be 1, 2, 4 or 8");
  if (max_seq_len < 1 || max_seq_len > capacity)
    return fail(BGTQ_ECAPACITY, "bgtq_fp16_decode_attn: max_seq_len must be in [1, capacity]");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: softmax_scale must be positive and finite");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15)
    return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: q, k and v must be 16-byte aligned");
  if ((uintptr_t)workspace & 255) return fail(BGTQ_EINVAL, "bgtq_fp16_decode_attn: workspace must be 256-byte aligned");
  const F16Layout lay = f16_layout(batch, n_kv_heads, n_q_heads, max_seq_len);
  if (ws_bytes < lay.total) return fail(BGTQ_EWORKSPACE, "bgtq_fp16_decode_attn: workspace too small");
  F16Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.part = (float *)workspace;
  a.capacity = capacity;
  a.max_seq_len = max_seq_len;
  a.hkv = n_kv_heads;
  a.hq = n_q_heads;
  a.tiles_per_split = lay.tiles_per_split;
  a.n_splits = lay.n_splits;
  a.kscale = softmax_scale * 1.4426950408889634f;
  hipStream_t st = (hipStream_t)stream;
  pick_f16(G)<<<dim3(lay.n_splits, n_kv_heads, batch), kF16Threads, 0, st>>>(a);
  const bgtq_status s = launch_status("bgtq_fp16_decode_attn");
  if (s != BGTQ_OK) return s;
  merge_kernel<false><<<dim3(n_q_heads, batch), kMergeThreads, 0, st>>>(nullptr, (const float *)workspace,
                                                                       lay.n_splits, G, n_q_heads, out,
                                                                       MergeBuf{});
  return launch_status("bgtq_fp16_decode_attn (merge)");
}

}  // extern "C"
