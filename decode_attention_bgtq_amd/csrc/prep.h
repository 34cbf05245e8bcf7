// Query preparation for the fused decode: rotation of the queries once per
// key width group (fp32 MFMA) and their matrix-core operands for the stream
// kernel ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract;
// Block-GTQ README, backend table).  Internal header, shared by the decode
// launches and the fused decode step.
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
  int64_t off_kvh, off_rot32, stride;
  int hkv, hq;
  float kscale;
};

template <int G>
struct PrepOut {  // byte offsets in one (sequence, KV head) block of the prep output
  static constexpr int nq = (G + 3) / 4;            // query-head quads
  static constexpr int q4 = 0;                      // fp32 [G][128]
  static constexpr int qr = G * kHeadDim * 4;       // fp16 [kMaxKSteps][nq][4][4]
  static constexpr int rinv = qr + kMaxKSteps * nq * 32;  // fp32 [G]
  static constexpr int bytes = rinv + G * 4;
};

// One workgroup per (KV head, sequence): the query-dependent state that every
// split of the stream kernel shares.  The G queries are rotated once per key
// group (fp32 MFMA, block-diagonal rotation) and written as
//  * q4[h][r] = kscale / sqrt(d4) q_rot[h][r] for the 4-bit group (r < d4, else 0);
//  * qr[k][quad][m][i] = fp16(fac_h kscale / sqrt(d_g) q_rot[h][pos_g + 4 s + i]),
//    h = 4 quad + m, for k-step k = (group g, step s) of the width-1..3 groups
//    (0 past the group, for h >= G and for k past the head's k-steps);
//  * rinv[h] = 1 / fac_h, fac_h the power of two that brings the largest
//    |kscale / sqrt(d_g) q_rot[h][p]| over those groups to [2^13, 2^14).
template <int G>
__device__ __forceinline__ void prep_role(const PrepArgs &a, int kvh, int b) {
  typedef PrepOut<G> PO;
  __shared__ KvhDesc kds;
  __shared__ float qg[8 * kHeadDim];
  __shared__ float qs[G * kHeadDim];
  __shared__ float gsc[kHeadDim];  // kscale / sqrt(d_g) of the group of each position
  __shared__ float hmax[G];
  const uint8_t *consts = a.consts;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t *out = a.out + ((size_t)b * a.hkv + kvh) * (size_t)a.stride;
  // ---- one round of loads: descriptor and queries (natural order, in the
  // rotated-query area) first, then the rotation rows (fixed addresses), so
  // that staging the former waits for them only.
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  static_assert(kDescWords <= kPrepThreads && G * kHeadDim <= 2 * kPrepThreads, "one pass of staging loads");
  const uint32_t dw = ((const uint32_t *)((const KvhDesc *)(consts + a.off_kvh) + kvh))[min(tid, kDescWords - 1)];
  const uint16_t *qb = a.q + ((size_t)b * a.hq + (size_t)kvh * G) * kHeadDim;
  const uint16_t q0 = qb[min(tid, G * kHeadDim - 1)];
  const uint16_t q1 = qb[min(tid + kPrepThreads, G * kHeadDim - 1)];
  RotRows<kPrepWaves> rr;
  rot_rows<kPrepWaves>((const float *)(consts + a.off_rot32) + (size_t)kvh * kHeadDim * kHeadDim, wave, lane, rr);
  if (tid < kDescWords) ((uint32_t *)&kds)[tid] = dw;
  if (tid < G * kHeadDim) qs[tid] = h2f(q0);
  if (tid + kPrepThreads < G * kHeadDim) qs[tid + kPrepThreads] = h2f(q1);
  __syncthreads();
  const int d4 = kds.d4, dnz = kds.d_nz;
  {
    // group order: qg[h][p] = q[h][coord[p]] (rows h >= G and positions >= d_nz zero)
    const int p = tid & (kHeadDim - 1);
    const int cp = kds.coord[p < dnz ? p : 0];
    for (int i = tid; i < 8 * kHeadDim; i += kPrepThreads) {
      const int h = i >> 7;
      const float v = qs[(h < G ? h : 0) * kHeadDim + cp];
      qg[i] = (h < G && p < dnz) ? v : 0.f;
    }
    if (tid < kHeadDim) {
      float sc = 0.f;
      for (int gi = 0; gi < kds.n_groups; ++gi)
        if (tid >= kds.g[gi].pos && tid < kds.g[gi].pos + kds.g[gi].d) sc = a.kscale / sqrtf((float)kds.g[gi].d);
      gsc[tid] = sc;
    }
  }
  __syncthreads();
  rot_tiles<kPrepWaves>(rr, G, qg, qs, wave, lane);
  __syncthreads();
  // per head: the largest scaled |q_rot| over the width-1..3 groups, one wave per head
  for (int h = wave; h < G; h += kPrepWaves) {
    float v = 0.f;
    for (int p = d4 + lane; p < dnz; p += 64) v = fmaxf(v, fabsf(qs[h * kHeadDim + p] * gsc[p]));
    v = wave_max(v);
    if (lane == 0) hmax[h] = v;
  }
  {
    float *q4 = (float *)(out + PO::q4);
    const float s4 = d4 > 0 ? a.kscale / sqrtf((float)d4) : 0.f;
    for (int idx = tid; idx < G * kHeadDim; idx += kPrepThreads) {
      const int h = idx >> 7, r = idx & (kHeadDim - 1);
      q4[idx] = r < d4 ? qs[h * kHeadDim + r] * s4 : 0.f;
    }
  }
  __syncthreads();
  float fac[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = hmax[h];
    int e = 0;
    (void)frexpf(m, &e);
    e = m > 0.f ? e : 0;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    fac[h] = ldexpf(1.f, 14 - e);
    if (tid == h) ((float *)(out + PO::rinv))[h] = ldexpf(1.f, e - 14);
  }
  // k-step operand rows, in group order 3, 2, 1
  _Float16 *qr = (_Float16 *)(out + PO::qr);
  for (int idx = tid; idx < kMaxKSteps * PO::nq * 16; idx += kPrepThreads) {
    const int i = idx & 3, m = (idx >> 2) & 3, quad = (idx >> 4) % PO::nq, k = (idx >> 4) / PO::nq;
    const int h = 4 * quad + m;
    int p = -1, k0 = 0;
    for (int gi = 0; gi < kds.n_groups; ++gi) {
      const KGroupDesc &g = kds.g[gi];
      if (g.w == 4) continue;
      const int ns = (g.d + 3) >> 2;
      if (k >= k0 && k < k0 + ns && 4 * (k - k0) + i < g.d) p = g.pos + 4 * (k - k0) + i;
      k0 += ns;
    }
    float v = 0.f;
    if (h < G && p >= 0) {
      float fh = fac[0];
#pragma unroll
      for (int u = 1; u < G; ++u) fh = h == u ? fac[u] : fh;
      v = fh * (gsc[p] * qs[h * kHeadDim + p]);
    }
    qr[idx] = (_Float16)v;
  }
}

}  // namespace bgtq
