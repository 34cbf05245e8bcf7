// Split merge of the decode kernels: log-sum-exp combination of the per-split
// partials (m, l, acc[128]) of each query head, normalisation and, for the
// packed path, the un-rotation of the value space ("RoPE-Aware Bit Allocation
// for KV-Cache Quantization", Abstract: packed-cache serving path).  Internal
// header.
#pragma once

#include "device.h"

namespace bgtq {

constexpr int kPartStride = 132;  // m, l, pad, pad, acc[128]
constexpr int kMaxSplits = 256;
constexpr int kMaxSink = 64, kMaxRecent = 65536;  // fp16 buffer bounds (sink, recent window)

// One workgroup of 512 threads (8 waves) per (query head, sequence).  Every
// global load is issued first: each wave loads the (m, l) of every split (lane
// s, s + 64, ...), lane l of wave w the split accumulators of coordinate
// k = 16 w + (l % 16) for the splits s = l / 16 (mod 4) (up to kMergeRegs of
// them in registers), and (ROT) thread t a quarter (32 values) of row t / 4 of
// Pi_V^T.  Then, without a workgroup barrier: M = max_s m_s and
// w_s = 2^(m_s - M) / (sum_s 2^(m_s - M) l_s c) in every wave (a copy per
// wave in LDS), y[k] = sum_s w_s acc_s[k] by the four split groups of the lanes
// of k and a cross-lane sum.  After one barrier, out[j] = sum_k Pi_V[k][j] y[k]
// (ROT: the packed path, c = sqrt(128) for the centroid scale; four threads per
// j) or out[k] = y[k] (c = 1).
//
// With BUF (the fp16 sink and recent window), the merge also attends to the
// buffered fp16 tokens of its head: thread t takes token rows t / 8 (+ 64 per
// round, the loads of three rounds issued together) and the 16 coordinates
// 16 (t % 8) .. of the key and value; the
// logit is the sum over the 8 threads of a row; each thread keeps a running
// (max, sum, 16 value sums), combined over the rows of a wave by cross-lane
// steps and over the waves in LDS.  The packed result y (normalised by its own
// sum) and the buffer's are then mixed by their shares of the total softmax
// mass.
constexpr int kMergeThreads = 512;
constexpr int kBufRows = kMergeThreads / 8;  // buffered token rows per round
constexpr int kBufRounds = 3;                // rounds whose loads are issued together (192 tokens)
constexpr int kMergeRegs = 16;  // split accumulators per lane loaded before the weights (n_splits <= 64)

struct MergeBuf {
  const uint16_t *q;                    // [batch][hq][128]
  const uint16_t *k_sink, *v_sink;      // [batch][hkv][n_sink][128]
  const uint16_t *k_recent, *v_recent;  // [batch][hkv][n_recent][128], token t in row t % n_recent
  const int32_t *seq_lens;
  int64_t max_seq_len;
  int n_sink, n_recent, hkv, seq_add;
  float kscale;  // softmax scale in log2 units
};

// Running softmax state of one thread over its buffered tokens: maximum logit
// (log2 units), sum of 2^(l - m) and the 16 value sums.
struct BufState {
  float m, l, a[16];
};

__device__ __forceinline__ void buf_combine(BufState &s, float om, float ol, const float *oa) {
  const float mn = fmaxf(s.m, om);
  if (mn == -INFINITY) return;
  const float f0 = __builtin_amdgcn_exp2f(s.m - mn), f1 = __builtin_amdgcn_exp2f(om - mn);
  s.l = s.l * f0 + ol * f1;
#pragma unroll
  for (int i = 0; i < 16; ++i) s.a[i] = s.a[i] * f0 + oa[i] * f1;
  s.m = mn;
}

// The buffered tokens of sequence b for the query head of this workgroup:
// sink rows [0, min(n_sink, T)), then the window tokens [max(n_sink, T - n_recent), T).
__device__ __forceinline__ void buf_rows(const MergeBuf &bf, int b, int kvh, int tid, BufState &st,
                                         const float *qv) {
  const int64_t sr = (int64_t)bf.seq_lens[b] + bf.seq_add;
  const int64_t seq = sr < 0 ? 0 : (sr > bf.max_seq_len ? bf.max_seq_len : sr);
  const int64_t n_s = seq < bf.n_sink ? seq : bf.n_sink;
  const int64_t r0 = seq - bf.n_recent > bf.n_sink ? seq - bf.n_recent : bf.n_sink;
  const int64_t n_f = n_s + (seq > r0 ? seq - r0 : 0);
  const int row = tid >> 3, part = tid & 7;
  const size_t hb = (size_t)b * bf.hkv + kvh;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) st.a[i] = 0.f;
  // ring row of the first window token (the window's tokens are consecutive, fewer than n_recent)
  const int64_t slot0 = n_f > n_s ? r0 % bf.n_recent : 0;
  for (int64_t c0 = 0; c0 < n_f; c0 += kBufRows * kBufRounds) {
    // every load of the pass first (rows past the end re-read the last one), then the rows
    uint4 kx[kBufRounds][2], vx[kBufRounds][2];
#pragma unroll
    for (int u = 0; u < kBufRounds; ++u) {
      const int64_t f = c0 + u * kBufRows + row, fc = f < n_f ? f : n_f - 1;
      int64_t slot = slot0 + (fc - n_s);
      slot = slot >= bf.n_recent ? slot - bf.n_recent : slot;
      const bool sink = fc < n_s;
      const size_t off = (hb * (sink ? bf.n_sink : bf.n_recent) + (sink ? fc : slot)) * kHeadDim;
      const uint4 *kp = (const uint4 *)((sink ? bf.k_sink : bf.k_recent) + off) + 2 * part;
      const uint4 *vp = (const uint4 *)((sink ? bf.v_sink : bf.v_recent) + off) + 2 * part;
      kx[u][0] = kp[0], kx[u][1] = kp[1], vx[u][0] = vp[0], vx[u][1] = vp[1];
    }
#pragma unroll
    for (int u = 0; u < kBufRounds; ++u) {
      const uint32_t kw[8] = {kx[u][0].x, kx[u][0].y, kx[u][0].z, kx[u][0].w,
                              kx[u][1].x, kx[u][1].y, kx[u][1].z, kx[u][1].w};
      const uint32_t vw[8] = {vx[u][0].x, vx[u][0].y, vx[u][0].z, vx[u][0].w,
                              vx[u][1].x, vx[u][1].y, vx[u][1].z, vx[u][1].w};
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s = fmaf(qv[2 * i], h2f((uint16_t)(kw[i] & 0xFFFFu)), s);
        s = fmaf(qv[2 * i + 1], h2f((uint16_t)(kw[i] >> 16)), s);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      if (c0 + u * kBufRows + row < n_f) {
        float va[16];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          va[2 * i] = h2f((uint16_t)(vw[i] & 0xFFFFu)), va[2 * i + 1] = h2f((uint16_t)(vw[i] >> 16));
        buf_combine(st, s, 1.f, va);  // one token: (logit, 1, its value)
      }
    }
  }
  // rows of the wave (lane bits 3..5)
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const float om = __shfl_xor(st.m, off), ol = __shfl_xor(st.l, off);
    float oa[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) oa[i] = __shfl_xor(st.a[i], off);
    buf_combine(st, om, ol, oa);
  }
}

template <bool ROT, bool BUF = false>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *__restrict__ pvt_all,
                                                              const float *__restrict__ part, int n_splits,
                                                              int group, int hq, uint16_t *__restrict__ out,
                                                              const MergeBuf bf) {
  constexpr int kWaves = kMergeThreads / 64;
  static_assert(!BUF || ROT, "the buffered merge is the packed path's");
  __shared__ float wsm[kWaves][kMaxSplits];
  __shared__ __attribute__((aligned(16))) float ys[kHeadDim];
  __shared__ float bsm[BUF ? kWaves : 1][8][18];  // per wave and coordinate block: m, l, 16 value sums
  const int hqi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvh = hqi / group;
  const float *ph = part + ((size_t)b * hq + hqi) * (size_t)n_splits * kPartStride;
  // rotation quarter: output j = tid / 4, k in [32 (tid % 4), 32 (tid % 4) + 32)
  const int j = tid >> 2, kq = tid & 3;
  float4 pr[8];
  if constexpr (ROT) {
    const float4 *row = (const float4 *)(pvt_all + ((size_t)kvh * kHeadDim + j) * kHeadDim + 32 * kq);
#pragma unroll
    for (int u = 0; u < 8; ++u) pr[u] = row[u];
  }
  float2 ml[kMaxSplits / 64];
#pragma unroll
  for (int r = 0; r < kMaxSplits / 64; ++r) {
    const int sp = lane + 64 * r;
    ml[r] = sp < n_splits ? *(const float2 *)(ph + (size_t)sp * kPartStride) : make_float2(-INFINITY, 0.f);
  }
  const int k = 16 * wave + (lane & 15), sg = lane >> 4;
  const float *pv = ph + 4 + k;
  float av[kMergeRegs];
#pragma unroll
  for (int u = 0; u < kMergeRegs; ++u) {
    const int sp = sg + 4 * u;
    av[u] = pv[(size_t)(sp < n_splits ? sp : 0) * kPartStride];
  }
  if constexpr (BUF) {
    // this thread's 16 query coordinates, in log2 units
    const uint4 *qp = (const uint4 *)(bf.q + ((size_t)b * hq + hqi) * kHeadDim) + 2 * (tid & 7);
    const uint4 q0 = qp[0], q1 = qp[1];
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float qv[16];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qv[2 * i] = h2f((uint16_t)(qw[i] & 0xFFFFu)) * bf.kscale, qv[2 * i + 1] = h2f((uint16_t)(qw[i] >> 16)) * bf.kscale;
    BufState bs;
    buf_rows(bf, b, kvh, tid, bs, qv);
    if (lane < 8) {
      bsm[wave][lane][0] = bs.m;
      bsm[wave][lane][1] = bs.l;
#pragma unroll
      for (int i = 0; i < 16; ++i) bsm[wave][lane][2 + i] = bs.a[i];
    }
  }
  // ---- weights, per wave
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxSplits / 64; ++r) m = fmaxf(m, ml[r].x);
  const float mx = wave_max(m);
  float l = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxSplits / 64; ++r)
    if (ml[r].x != -INFINITY) l = fmaf(__builtin_amdgcn_exp2f(ml[r].x - mx), ml[r].y, l);
  const float lsum = wave_sum(l);
  const float inv = lsum > 0.f ? 1.0f / (lsum * (ROT ? sqrtf((float)kHeadDim) : 1.f)) : 0.f;
#pragma unroll
  for (int r = 0; r < kMaxSplits / 64; ++r)
    wsm[wave][lane + 64 * r] = ml[r].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[r].x - mx) * inv;
  wave_sync_lds();
  // ---- y[k]: split group sg of the lanes of k, then the sum over the four groups
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeRegs; ++u) {
    const int sp = sg + 4 * u;
    if (sp < n_splits) acc = fmaf(wsm[wave][sp], av[u], acc);
  }
  for (int c0 = sg + 4 * kMergeRegs; c0 < n_splits; c0 += 4 * kMergeRegs) {
    float v[kMergeRegs];
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u) v[u] = pv[(size_t)min(c0 + 4 * u, n_splits - 1) * kPartStride];
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u)
      if (c0 + 4 * u < n_splits) acc = fmaf(wsm[wave][c0 + 4 * u], v[u], acc);
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if constexpr (!ROT) {
    if (sg == 0) out[((size_t)b * hq + hqi) * kHeadDim + k] = __builtin_bit_cast(uint16_t, (_Float16)acc);
    return;
  }
  if (sg == 0) ys[k] = acc;
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const float4 y = *(const float4 *)(ys + 32 * kq + 4 * u);
    o = fmaf(pr[u].x, y.x, o);
    o = fmaf(pr[u].y, y.y, o);
    o = fmaf(pr[u].z, y.z, o);
    o = fmaf(pr[u].w, y.w, o);
  }
  o += __shfl_xor(o, 1);
  o += __shfl_xor(o, 2);
  if constexpr (BUF) {
    // the buffer's (max, sum, value sum of coordinate j) over the waves, then
    // the two results mixed by their shares of the softmax mass
    const int jb = j >> 4, ji = j & 15;
    float bm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) bm = fmaxf(bm, bsm[w][jb][0]);
    float bl = 0.f, ba = 0.f;
    if (bm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(bsm[w][jb][0] - bm);
        bl = fmaf(f, bsm[w][jb][1], bl);
        ba = fmaf(f, bsm[w][jb][2 + ji], ba);
      }
    }
    const float mm = fmaxf(mx, bm);
    const float ep = lsum > 0.f ? __builtin_amdgcn_exp2f(mx - mm) * lsum : 0.f;
    const float eb = bl > 0.f ? __builtin_amdgcn_exp2f(bm - mm) * bl : 0.f;
    const float tot = ep + eb;
    o = tot > 0.f ? (ep * o + (bl > 0.f ? eb * (ba / bl) : 0.f)) / tot : 0.f;
  }
  if (kq == 0) out[((size_t)b * hq + hqi) * kHeadDim + j] = __builtin_bit_cast(uint16_t, (_Float16)o);
}

}  // namespace bgtq
