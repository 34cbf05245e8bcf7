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

// q_rot[h][p] = sum_k R[p][k] qg[h][k]: the rotation of every key width group
// at once, R being the head's block-diagonal matrix of the group rotations
// (rows and columns in group order, zero outside the blocks and past d_nz).
// qg [8][128]: the queries in group order, rows h >= G zero; qs [G][128].
// 16x16x4 fp32 MFMA tiles, the query heads as columns; the 8 row tiles of 16
// are spread over the WAVES waves (8 / WAVES tiles each).  The operand rows of R are fetched by
// rot_rows (addresses independent of the descriptor), the MFMAs run in
// rot_tiles.
template <int WAVES>
struct RotRows {
  static constexpr int nt = 8 / WAVES;  // row tiles per wave
  float a[nt][kHeadDim / 4];
};

template <int WAVES>
__device__ __forceinline__ void rot_rows(const float *R, int wave, int lane, RotRows<WAVES> &rr) {
  const int n = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
#pragma unroll
    for (int s = 0; s < kHeadDim / 4; ++s) rr.a[t2][s] = R[(16 * t + n) * kHeadDim + 4 * s + kq];
  }
}

template <int WAVES>
__device__ __forceinline__ void rot_tiles(const RotRows<WAVES> &rr, int G, const float *qg, float *qs, int wave,
                                          int lane) {
  const int n = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    {
      f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kHeadDim / 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(rr.a[t2][s], qg[(n & 7) * kHeadDim + 4 * s + kq], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n < G) qs[n * kHeadDim + 16 * t + 4 * kq + r] = acc[r];
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
  int64_t off_kvh, off_build, off_rot32, stride;
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
  // ---- one round of loads: descriptor, queries (natural order, in the
  // rotated-query area), centroids and build words first, then the rotation
  // rows (fixed addresses), so that staging the former waits for them only.
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  static_assert(kDescWords <= kPrepThreads && G * kHeadDim <= 2 * kPrepThreads, "one pass of staging loads");
  const uint32_t dw = ((const uint32_t *)((const KvhDesc *)(consts + a.off_kvh) + kvh))[min(tid, kDescWords - 1)];
  const uint16_t *qb = a.q + ((size_t)b * a.hq + (size_t)kvh * G) * kHeadDim;
  const uint16_t q0 = qb[min(tid, G * kHeadDim - 1)];
  const uint16_t q1 = qb[min(tid + kPrepThreads, G * kHeadDim - 1)];
  const float c0 = (float)hd->cent[(tid >> 4) & 3][tid & 15];
  const uint32_t bw0 = ((const uint32_t *)(consts + a.off_build))[kvh * kMaxChunks + (tid & (kMaxChunks - 1))];
  RotRows<kPrepWaves> rr;
  rot_rows<kPrepWaves>((const float *)(consts + a.off_rot32) + (size_t)kvh * kHeadDim * kHeadDim, wave, lane, rr);
  if (tid < kDescWords) ((uint32_t *)&kds)[tid] = dw;
  if (tid < G * kHeadDim) qs[tid] = h2f(q0);
  if (tid + kPrepThreads < G * kHeadDim) qs[tid + kPrepThreads] = h2f(q1);
  if (tid < 64) cs[tid] = c0;
  if (tid < kMaxChunks) bld[tid] = bw0;
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
  rot_tiles<kPrepWaves>(rr, G, qg, qs, wave, lane);
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
