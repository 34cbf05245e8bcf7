// Query preparation for the fused decode: rotation of the queries once per
// key width group (fp32 MFMA, the only matrix-core use) and the per-chunk
// lookup tables of q_rot x centroid ("RoPE-Aware Bit Allocation for KV-Cache
// Quantization", Abstract; Block-GTQ README, backend table).  Internal header,
// shared by the decode launches and the fused decode step.
#pragma once

#include "device.h"

namespace bgtq {

constexpr int kPrepWaves = 8;
constexpr int kPrepThreads = 64 * kPrepWaves;

typedef float f4v __attribute__((ext_vector_type(4)));

// q_rot[h][pos_g + i] = sum_k Pi_g[i][k] q[h][coord_g[k]] for the key groups of
// one KV head.  qg [8][128]: the queries gathered into group order
// (qg[h][pos_g + k] = q[h][coord_g[k]]), rows h >= G zero.  qs [G][128]: the
// rotated queries in group order.  16x16x4 fp32 MFMA tiles with the query
// heads as columns; the (group, 16-row tile) pairs of all groups are spread
// over the `waves` waves, and each wave issues every operand load of a tile
// before its first MFMA (clamped addresses, zero-masked values).
__device__ __forceinline__ void rotate_queries(const ConstHeader *hd, const KvhDesc *kd, int G,
                                               const float *qg, float *qs, int wave, int waves,
                                               int lane) {
  const int n = lane & 15, kq = lane >> 4;
  int ng = kd->n_groups, tiles[kMaxGroups + 1];
  tiles[0] = 0;
  for (int gi = 0; gi < kMaxGroups; ++gi) tiles[gi + 1] = tiles[gi] + (gi < ng ? (kd->g[gi].d + 15) >> 4 : 0);
  for (int t = wave; t < tiles[kMaxGroups]; t += waves) {
    int gi = 0;
    while (t >= tiles[gi + 1]) ++gi;
    const int d = kd->g[gi].d, pos = kd->g[gi].pos;
    const float *pi = (const float *)((const uint8_t *)hd + hd->off_rot32_k) + kd->g[gi].rot32;
    const int ia = 16 * (t - tiles[gi]) + n;
    const int ic = ia < d ? ia : d - 1;
    float a[kHeadDim / 4];
#pragma unroll
    for (int s = 0; s < kHeadDim / 4; ++s) {
      const int kk = 4 * s + kq;
      a[s] = pi[(size_t)ic * d + (kk < d ? kk : d - 1)];
    }
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kHeadDim / 4; ++s) {
      const int kk = 4 * s + kq;
      if (4 * s < d) {  // wave-uniform
        const float av = (ia < d && kk < d) ? a[s] : 0.f;
        const float bq = qg[(n & 7) * kHeadDim + pos + (kk < d ? kk : d - 1)];
        const float bv = kk < d ? bq : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = ia - n + 4 * kq + r;
      if (i < d && n < G) qs[n * kHeadDim + pos + i] = acc[r];
    }
  }
}

// qg[h][p] = q[h][coord[p]] for p < d_nz, else 0, for h < 8 (rows h >= G zero).
__device__ __forceinline__ void gather_queries(const KvhDesc *kd, int G, const uint16_t *qb, float *qg, int tid,
                                               int threads) {
  const int dnz = kd->d_nz;
  for (int i = tid; i < 8 * kHeadDim; i += threads) {
    const int h = i >> 7, p = i & (kHeadDim - 1);
    const int pc = p < dnz ? p : 0;
    const int hc = h < G ? h : 0;
    const float v = h2f(qb[hc * kHeadDim + kd->coord[pc]]);
    qg[i] = (h < G && p < dnz) ? v : 0.f;
  }
}

struct PrepArgs {
  const uint8_t *consts;
  const uint16_t *q;
  uint8_t *out;
  int64_t off_kvh, off_build, stride;
  int hkv, hq, win, table_bytes, chunks_per_wg;
  float kscale;
};

// One workgroup per (KV head, sequence, slice): the query-dependent state that every split
// of the stream kernel shares.  Each workgroup rotates the G queries once per
// key group (fp32 MFMA) and builds the lookup tables of its slice of the
// width-1..3 chunks: per chunk, fac_h * kscale / sqrt(d_g) * sum_r
// q_rot[h][pos + r] * c_w[code_r] over every value of the chunk's window, as
// fp16.  fac_h is the power of two that brings
// max_g(kscale c_max,w / sqrt(d_g)) * sum_p |q_rot[h][p]| (over the positions
// of those groups, summed in a fixed order so that every slice finds the same
// factor) below 2^14.  Slice 0 also writes the 4-bit group queries scaled by
// kscale / sqrt(d4) and 1 / fac_h.
template <int G>
__device__ __forceinline__ void prep_role(const PrepArgs &a, int kvh, int b, int slice) {
  constexpr int lg = GLog<G>::v - 1;  // log2 G
  __shared__ KvhDesc kds;
  __shared__ float qg[8 * kHeadDim];
  __shared__ float qs[G * kHeadDim];
  __shared__ uint32_t bld[kMaxChunks];
  __shared__ float cs[64 + kMaxGroups];
  __shared__ float hsum[G];
  const uint8_t *consts = a.consts;
  const ConstHeader *hd = hdr_of(consts);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t *out = a.out + ((size_t)b * a.hkv + kvh) * (size_t)a.stride;
  // ---- round 1: descriptor, queries (natural order, in the rotated-query area), centroids, build words
  {
    const uint32_t *src = (const uint32_t *)((const KvhDesc *)(consts + a.off_kvh) + kvh);
    for (int i = tid; i < (int)(sizeof(KvhDesc) / 4); i += kPrepThreads) ((uint32_t *)&kds)[i] = src[i];
    const uint16_t *qb = a.q + ((size_t)b * a.hq + (size_t)kvh * G) * kHeadDim;
    for (int i = tid; i < G * kHeadDim; i += kPrepThreads) qs[i] = h2f(qb[i]);
    if (tid < 64) cs[tid] = (float)hd->cent[tid >> 4][tid & 15];
    if (tid < kMaxChunks) bld[tid] = ((const uint32_t *)(consts + a.off_build))[kvh * kMaxChunks + tid];
  }
  __syncthreads();
  const int nch = kds.n_chunks, d4 = kds.d4, dnz = kds.d_nz;
  if (tid < kds.n_groups) cs[64 + tid] = a.kscale / sqrtf((float)kds.g[tid].d);
  {
    // group order: qg[h][p] = q[h][coord[p]] (rows h >= G and positions >= d_nz zero)
    const int p = tid & (kHeadDim - 1);
    const int cp = kds.coord[p < dnz ? p : 0];
    for (int i = tid; i < 8 * kHeadDim; i += kPrepThreads) {
      const int h = i >> 7;
      const float v = qs[(h < G ? h : 0) * kHeadDim + cp];
      qg[i] = (h < G && p < dnz) ? v : 0.f;
    }
  }
  __syncthreads();
  // ---- round 2: rotation rows
  rotate_queries(hd, &kds, G, qg, qs, wave, kPrepWaves, lane);
  __syncthreads();
  // per head: sum of |q_rot| over the table groups, one wave per head, fixed order
  for (int h = wave; h < G; h += kPrepWaves) {
    float v = 0.f;
    for (int p = d4 + lane; p < dnz; p += 64) v += fabsf(qs[h * kHeadDim + p]);
    v = wave_sum(v);
    if (lane == 0) hsum[h] = v;
  }
  if (slice == 0) {
    float *q4 = (float *)(out + a.table_bytes);
    const float s4 = d4 > 0 ? a.kscale / sqrtf((float)d4) : 0.f;
    for (int idx = tid; idx < G * kHeadDim; idx += kPrepThreads) {
      const int h = idx >> 7, r = idx & (kHeadDim - 1);
      q4[idx] = r < d4 ? qs[h * kHeadDim + r] * s4 : 0.f;
    }
  }
  __syncthreads();
  float smax = 0.f;
  for (int gi = 0; gi < kds.n_groups; ++gi) {
    const int w = kds.g[gi].w;
    if (w < 4) smax = fmaxf(smax, cs[64 + gi] * fabsf(cs[16 * (w - 1) + (1 << w) - 1]));
  }
  float fac[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = smax * hsum[h];
    int e = 0;
    (void)frexpf(m, &e);
    e = m > 0.f ? e : 0;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    fac[h] = ldexpf(1.f, 14 - e);
    if (slice == 0 && tid == h) ((float *)(out + a.table_bytes + G * kHeadDim * 4))[h] = ldexpf(1.f, e - 14);
  }
  const int ne = 1 << a.win, sh = a.win + lg;
  const int c_lo = slice * a.chunks_per_wg;
  const int c_hi = min(nch, c_lo + a.chunks_per_wg);
  _Float16 *tab = (_Float16 *)out;
  for (int idx = (c_lo << sh) + tid; idx < (c_hi << sh); idx += kPrepThreads) {
    const int h = idx & (G - 1), f = (idx >> lg) & (ne - 1), c = idx >> sh;
    const uint32_t bw = bld[c];
    const int pos = bw & 255, m = (bw >> 8) & 15, w = (bw >> 12) & 7, gi = (bw >> 15) & 3;
    const float *cw = cs + 16 * (w - 1);
    const float *qh = qs + h * kHeadDim + pos;
    const int mask = (1 << w) - 1;
    float acc = 0.f;
    for (int r = 0; r < m; ++r) acc = fmaf(qh[r], cw[(f >> (w * r)) & mask], acc);
    float fh = fac[0];
#pragma unroll
    for (int k = 1; k < G; ++k) fh = h == k ? fac[k] : fh;
    tab[idx] = (_Float16)(fh * (cs[64 + gi] * acc));
  }
}

}  // namespace bgtq
