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

// One workgroup of 512 threads per (query head, sequence).  Every global load
// is issued first: thread t holds the split accumulators of coordinate t % 128
// for the splits s = t / 128 (mod 4) (up to kMergeRegs of them in registers),
// the (m, l) of split t, and (ROT) a quarter (32 values) of row t / 4 of Pi_V^T.
// Then: M = max_s m_s, w_s = 2^(m_s - M) / (sum_s 2^(m_s - M) l_s c),
// y = sum_s w_s acc_s, and out[j] = sum_k Pi_V[k][j] y[k] (ROT: the packed
// path, c = sqrt(128) for the centroid scale; four threads per j) or out[j] =
// y[j] (c = 1).
constexpr int kMergeThreads = 512;
constexpr int kMergeRegs = 16;  // split accumulators per thread loaded before the weights (n_splits <= 64)

template <bool ROT>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *__restrict__ pvt_all,
                                                              const float *__restrict__ part, int n_splits,
                                                              int group, int hq, uint16_t *__restrict__ out) {
  __shared__ float wsm[kMaxSplits];
  __shared__ __attribute__((aligned(16))) float ys[4 * kHeadDim];
  __shared__ float red[2 * (kMergeThreads / 64)];
  const int hqi = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvh = hqi / group;
  const float *ph = part + ((size_t)b * hq + hqi) * (size_t)n_splits * kPartStride;
  // rotation quarter: output j = tid / 4, k in [32 (tid % 4), 32 (tid % 4) + 32)
  const int j = tid >> 2, kq = tid & 3;
  const float4 *row = (const float4 *)(pvt_all + ((size_t)kvh * kHeadDim + j) * kHeadDim + 32 * kq);
  float4 pr[8];
  if constexpr (ROT) {
#pragma unroll
    for (int u = 0; u < 8; ++u) pr[u] = row[u];
  }
  float m = -INFINITY, l = 0.f;
  if (tid < n_splits) {
    const float2 ml = *(const float2 *)(ph + (size_t)tid * kPartStride);
    m = ml.x;
    l = ml.y;
  }
  const int i = tid & (kHeadDim - 1), par = tid >> 7;
  const float *pv = ph + 4 + i;
  float av[kMergeRegs];
#pragma unroll
  for (int u = 0; u < kMergeRegs; ++u) {
    const int sp = par + 4 * u;
    av[u] = pv[(size_t)(sp < n_splits ? sp : 0) * kPartStride];
  }
  const float wm = wave_max(m);
  if (lane == 0) red[wave] = wm;
  __syncthreads();
  float mx = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  const float f = (mx == -INFINITY || m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
  const float wl = wave_sum(f * l);
  if (lane == 0) red[kMergeThreads / 64 + wave] = wl;
  __syncthreads();
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) lsum += red[kMergeThreads / 64 + w];
  const float inv = lsum > 0.f ? 1.0f / (lsum * (ROT ? sqrtf((float)kHeadDim) : 1.f)) : 0.f;
  if (tid < n_splits) wsm[tid] = f * inv;
  __syncthreads();
  {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u) {
      const int sp = par + 4 * u;
      if (sp < n_splits) acc = fmaf(wsm[sp], av[u], acc);
    }
    // further splits: chunks of kMergeRegs independent loads
    for (int c0 = par + 4 * kMergeRegs; c0 < n_splits; c0 += 4 * kMergeRegs) {
      float v[kMergeRegs];
#pragma unroll
      for (int u = 0; u < kMergeRegs; ++u) v[u] = pv[(size_t)min(c0 + 4 * u, n_splits - 1) * kPartStride];
#pragma unroll
      for (int u = 0; u < kMergeRegs; ++u)
        if (c0 + 4 * u < n_splits) acc = fmaf(wsm[c0 + 4 * u], v[u], acc);
    }
    ys[par * kHeadDim + i] = acc;
  }
  __syncthreads();
  if constexpr (!ROT) {
    if (tid < kHeadDim) {
      const float o = ys[tid] + ys[kHeadDim + tid] + ys[2 * kHeadDim + tid] + ys[3 * kHeadDim + tid];
      out[((size_t)b * hq + hqi) * kHeadDim + tid] = __builtin_bit_cast(uint16_t, (_Float16)o);
    }
    return;
  }
  float o = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = 32 * kq + 4 * u;
    const float y0 = ys[k] + ys[kHeadDim + k] + ys[2 * kHeadDim + k] + ys[3 * kHeadDim + k];
    const float y1 = ys[k + 1] + ys[kHeadDim + k + 1] + ys[2 * kHeadDim + k + 1] + ys[3 * kHeadDim + k + 1];
    const float y2 = ys[k + 2] + ys[kHeadDim + k + 2] + ys[2 * kHeadDim + k + 2] + ys[3 * kHeadDim + k + 2];
    const float y3 = ys[k + 3] + ys[kHeadDim + k + 3] + ys[2 * kHeadDim + k + 3] + ys[3 * kHeadDim + k + 3];
    o = fmaf(pr[u].x, y0, o);
    o = fmaf(pr[u].y, y1, o);
    o = fmaf(pr[u].z, y2, o);
    o = fmaf(pr[u].w, y3, o);
  }
  o += __shfl_xor(o, 1);
  o += __shfl_xor(o, 2);
  if (kq == 0) out[((size_t)b * hq + hqi) * kHeadDim + j] = __builtin_bit_cast(uint16_t, (_Float16)o);
}

}  // namespace bgtq
