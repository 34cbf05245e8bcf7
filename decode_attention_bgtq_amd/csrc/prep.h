// Query preparation for the fused decode: rotation of the queries once per
// key width group and their matrix-core operands for the tile loop
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract; Block-GTQ
// README, backend table).  Internal header.  The decode kernel prepares the
// queries of its (sequence, KV head) in its own prologue from the group
// rotations stored as bands (fp32 VALU); the query-rotation entry point rotates
// batches of queries with fp32 MFMA over the block-diagonal matrix.
#pragma once

#include "device.h"

namespace bgtq {

typedef float f4v __attribute__((ext_vector_type(4)));

// q_rot[h][p] = sum_k R[p][k] qg[h][k]: the rotation of every key width group
// at once, R being the head's block-diagonal matrix of the group rotations
// (rows and columns in group order, zero outside the blocks and past d_nz).
// qg [8][128]: the queries in group order, rows h >= G zero; qs [G][128].
// 16x16x4 fp32 MFMA tiles, the query heads as columns; the 8 row tiles of 16
// are spread over the WAVES waves (8 / WAVES tiles each).  Step (u, e) of a
// tile contracts column 16 u + 4 kq + e in the lanes of quarter kq (the sum
// runs over every column once), so that A and B are read as float4.  The
// operand rows of R are fetched by rot_rows (addresses independent of the
// group layout), the MFMAs run in rot_tiles.
template <int WAVES>
struct RotRows {
  static constexpr int nt = 8 / WAVES;  // row tiles per wave
  float4 a[nt][kHeadDim / 16];
};

template <int WAVES>
__device__ __forceinline__ void rot_rows(const float *R, int wave, int lane, RotRows<WAVES> &rr) {
  const int n = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    const float4 *row = (const float4 *)(R + (16 * t + n) * kHeadDim + 4 * kq);
#pragma unroll
    for (int u = 0; u < kHeadDim / 16; ++u) rr.a[t2][u] = row[4 * u];
  }
}

template <int WAVES>
__device__ __forceinline__ void rot_tiles(const RotRows<WAVES> &rr, int G, const float *qg, float *qs, int wave,
                                          int lane) {
  const int n = lane & 15, kq = lane >> 4;
  const float4 *bq = (const float4 *)(qg + (n & 7) * kHeadDim + 4 * kq);
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kHeadDim / 16; ++u) {
      const float4 a = rr.a[t2][u], b = bq[4 * u];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n < G) qs[n * kHeadDim + 16 * t + 4 * kq + r] = acc[r];
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

// Byte offsets of the prepared query state in the decode kernel's LDS, relative
// to its start.
template <int G>
struct PrepOut {
  static constexpr int nq = (G + 3) / 4;                  // query-head quads
  static constexpr int q4 = 0;                            // fp32 [G][128]
  static constexpr int qr = G * kHeadDim * 4;             // fp16 [kMaxKSteps][nq][4][4]
  static constexpr int rinv = qr + kMaxKSteps * nq * 32;  // fp32 [G]
  static constexpr int bytes = (rinv + G * 4 + 15) & ~15;
};

// LDS scratch of the preparation (prologue only), byte offsets from its base.
template <int G>
struct PrepScratch {
  static constexpr int kds = 0;                                 // KvhDesc
  static constexpr int qs = ((int)sizeof(KvhDesc) + 15) & ~15;  // fp32 [G][128], natural coordinate order
  static constexpr int hm = qs + G * kHeadDim * 4;              // fp32 [8 waves][G]
  static constexpr int bytes = (hm + 8 * G * 4 + 15) & ~15;
};

// Global loads of the preparation, issued at the start of the prologue so that
// their latency overlaps the first cache tile's.  Thread t works on row
// p = t / 4 of the head's group-order rotation and on its columns
// k = 2 (t % 4) + 8 u + e (u < 16, e < 2).
struct PrepLoads {
  uint2 row;         // row table entry of p (band offset; d_g, pos_g, width, first k-step)
  uint32_t dw;       // one word of the KvhDesc
  uint16_t q0, q1;   // two query values (natural order)
  float2 r[16];      // Pi_g[p - pos_g][k], 0 past d_g
};

template <int G>
__device__ __forceinline__ void prep_load_row(PrepLoads &l, const uint2 *rows, const KvhDesc *kd, const uint16_t *qb,
                                              int tid) {
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  static_assert(kDescWords <= 512 && G * kHeadDim <= 1024, "one pass of staging loads (512 threads)");
  l.row = rows[tid >> 2];
  l.dw = ((const uint32_t *)kd)[min(tid, kDescWords - 1)];
  l.q0 = qb[min(tid, G * kHeadDim - 1)];
  l.q1 = qb[min(tid + 512, G * kHeadDim - 1)];
}

// The band of row p (addresses depend on the row entry): unconditional loads at
// clamped addresses, zeroed past d_g.
__device__ __forceinline__ void prep_load_band(PrepLoads &l, const float *band, int tid) {
  const int d = (int)(l.row.y & 255u), kq = tid & 3;
  const float2 *src = (const float2 *)(band + l.row.x);
  const int last = d > 1 ? (d - 2) >> 1 : 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) l.r[u] = src[min(kq + 4 * u, last)];
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (2 * kq + 8 * u >= d) l.r[u] = make_float2(0.f, 0.f);
}

// The query-dependent state of one (sequence, KV head), built in LDS by a
// workgroup of 512 threads from the loads above.  The G queries are rotated
// once per key group, q_rot[h][p] = sum_k Pi_g[p - pos_g][k] q[h][coord[pos_g + k]]
// (fp32; four threads per row, each a quarter of the columns, summed by DPP), and
// written as
//  * q4[h][p] = kscale / sqrt(d4) q_rot[h][p] for the 4-bit group (p < d4, else 0);
//  * qr[k][quad][m][i] = fp16(fac_h kscale / sqrt(d_g) q_rot[h][pos_g + 4 s + i]),
//    h = 4 quad + m, for k-step k = (group g, step s) of the width-1..3 groups
//    (0 past the group, for h >= G and for k past the head's k-steps);
//  * rinv[h] = 1 / fac_h, fac_h the power of two that brings the largest
//    |kscale / sqrt(d_g) q_rot[h][p]| over those groups to [2^13, 2^14).
// `out` and `scr` are LDS addresses (PrepOut and PrepScratch layouts).  Ends
// with a workgroup barrier.
template <int G>
__device__ __forceinline__ void prep_build_rows(const PrepLoads &l, uint8_t *out, uint8_t *scr, float kscale,
                                                int tid, int wave, int lane) {
  typedef PrepOut<G> PO;
  typedef PrepScratch<G> PS;
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  const KvhDesc &kds = *(const KvhDesc *)(scr + PS::kds);
  float *qs = (float *)(scr + PS::qs), *hm = (float *)(scr + PS::hm);
  // ---- stage the descriptor and the queries; clear the k-step operands
  if (tid < kDescWords) ((uint32_t *)(scr + PS::kds))[tid] = l.dw;
  if (tid < G * kHeadDim) qs[tid] = h2f(l.q0);
  if (tid + 512 < G * kHeadDim) qs[tid + 512] = h2f(l.q1);
  constexpr int kQrVec = kMaxKSteps * PO::nq * 32 / 16;
  for (int i = tid; i < kQrVec; i += 512) ((uint4 *)(out + PO::qr))[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  // ---- rotation of row p: this thread's quarter of the columns, then the quad sum
  const int p = tid >> 2, kq = tid & 3;
  const int d = (int)(l.row.y & 255u), pos = (int)((l.row.y >> 8) & 255u), w = (int)((l.row.y >> 16) & 7u);
  const int kb = (int)(l.row.y >> 19);
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int k = 2 * kq + 8 * u;
    if (k < d) {  // d is even: k + 1 < d too
      const int c0 = kds.coord[pos + k], c1 = kds.coord[pos + k + 1];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h] = fmaf(l.r[u].x, qs[h * kHeadDim + c0], acc[h]);
        acc[h] = fmaf(l.r[u].y, qs[h * kHeadDim + c1], acc[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc[h] += dpp_f<0xB1>(acc[h]);  // quad_perm [1,0,3,2]
    acc[h] += dpp_f<0x4E>(acc[h]);  // quad_perm [2,3,0,1]
  }
  const float gsc = d > 0 ? kscale / sqrtf((float)d) : 0.f;
  // 4-bit rows -> q4 (every row written: 0 outside the 4-bit group); heads kq, kq + 4
  float *q4 = (float *)(out + PO::q4);
#pragma unroll
  for (int h = 0; h < G; ++h)
    if ((h & 3) == kq) q4[h * kHeadDim + p] = w == 4 ? acc[h] * gsc : 0.f;
  // per head: the largest scaled |q_rot| over the width-1..3 rows (wave, then workgroup)
  const bool low = d > 0 && w < 4;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wave_max(low ? fabsf(acc[h] * gsc) : 0.f);
    if (lane == 0) hm[wave * G + h] = v;
  }
  __syncthreads();
  // ---- power-of-two operand scale per head; k-step operands of the width-1..3 rows
  _Float16 *qr = (_Float16 *)(out + PO::qr);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = 0.f;
#pragma unroll
    for (int wv = 0; wv < 8; ++wv) m = fmaxf(m, hm[wv * G + h]);
    int e = 0;
    (void)frexpf(m, &e);
    e = m > 0.f ? e : 0;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    if (tid == h) ((float *)(out + PO::rinv))[h] = ldexpf(1.f, e - 14);
    if (low && (h & 3) == kq) {
      const int r = p - pos, k = kb + (r >> 2);
      qr[((k * PO::nq + (h >> 2)) * 4 + (h & 3)) * 4 + (r & 3)] = (_Float16)(ldexpf(1.f, 14 - e) * (acc[h] * gsc));
    }
  }
  __syncthreads();
}

}  // namespace bgtq
