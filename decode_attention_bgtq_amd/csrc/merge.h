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
constexpr int kMergeThreads = 512;
constexpr int kMergeRegs = 16;  // split accumulators per lane loaded before the weights (n_splits <= 64)

template <bool ROT>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *__restrict__ pvt_all,
                                                              const float *__restrict__ part, int n_splits,
                                                              int group, int hq, uint16_t *__restrict__ out) {
  constexpr int kWaves = kMergeThreads / 64;
  __shared__ float wsm[kWaves][kMaxSplits];
  __shared__ __attribute__((aligned(16))) float ys[kHeadDim];
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
  if (kq == 0) out[((size_t)b * hq + hqi) * kHeadDim + j] = __builtin_bit_cast(uint16_t, (_Float16)o);
}

}  // namespace bgtq
