// Query preparation for the fused decode: rotation of the queries once per
// key width group and their matrix-core operands for the tile loop
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract; Block-GTQ
// README, backend table).  Internal header.  The preparation kernel (and the
// serving step's front kernel) prepares the queries of each (sequence, KV
// head) once per call, and the query-rotation entry point rotates batches of
// queries, both with fp32 MFMA over the block-diagonal matrix of the group
// rotations.
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
// runs over every column once), so that A and B are read as float4; four
// accumulators (u mod 4) keep four MFMA chains in flight.  The operand rows of
// R are fetched by rot_rows (addresses independent of the group layout), the
// MFMAs run in rot_tiles.  With more than 8 waves, waves 8 and up compute no tile.
template <int WAVES>
struct RotRows {
  static constexpr int nt = WAVES >= 8 ? 1 : 8 / WAVES;  // row tiles per wave
  float4 a[nt][kHeadDim / 16];
};

template <int WAVES>
__device__ __forceinline__ void rot_rows(const float *R, int wave, int lane, RotRows<WAVES> &rr) {
  const int n = lane & 15, kq = lane >> 4;
  // waves 8 and up load the first 16 bytes of R in every lane and never use
  // them: the loads are unconditional (so that the wait for a later load never
  // has to assume the longer queue of a skipped branch) but cost one line
  const bool idle = WAVES > 8 && wave >= 8;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    const float4 *row = (const float4 *)(R + (idle ? 0 : (16 * t + n) * kHeadDim + 4 * kq));
#pragma unroll
    for (int u = 0; u < kHeadDim / 16; ++u) rr.a[t2][u] = row[idle ? 0 : 4 * u];
  }
}

// The preparation fetches only the nonzero part of R: the row-table
// entries of the lane's rows first (rot_keys; y = d_g | pos_g << 8 | ..., 0
// past d_nz), then (rot_rows_sparse) the lane's four columns of each step
// from R when they meet its row's group [pos_g, pos_g + d_g), else from the
// plan's zero block (one line for every lane), so that the zero blocks of R
// are not read.  For the 128K workload's plans that is under a third of R.
template <int WAVES>
struct RotKeys {
  uint32_t y[RotRows<WAVES>::nt];
};

template <int WAVES>
__device__ __forceinline__ void rot_keys(const uint2 *rowk, int wave, int lane, RotKeys<WAVES> &rk) {
  const int n = lane & 15;
  const bool idle = WAVES > 8 && wave >= 8;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) rk.y[t2] = rowk[idle ? 0 : 16 * (wave + t2 * WAVES) + n].y;
}

template <int WAVES>
__device__ __forceinline__ void rot_rows_sparse(const float *R, const float *zero, const RotKeys<WAVES> &rk, int wave,
                                                int lane, RotRows<WAVES> &rr) {
  const int n = lane & 15, kq = lane >> 4;
  const bool idle = WAVES > 8 && wave >= 8;
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    const int dg = (int)(rk.y[t2] & 255u), pg = (int)((rk.y[t2] >> 8) & 255u);
    const float *row = R + (16 * t + n) * kHeadDim + 4 * kq;
#pragma unroll
    for (int u = 0; u < kHeadDim / 16; ++u) {
      const int c = 16 * u + 4 * kq;
      const bool need = !idle && c < pg + dg && c + 4 > pg;
      rr.a[t2][u] = *(const float4 *)(need ? row + 16 * u : zero);
    }
  }
}

template <int WAVES>
__device__ __forceinline__ void rot_tiles(const RotRows<WAVES> &rr, int G, const float *qg, float *qs, int wave,
                                          int lane) {
  const int n = lane & 15, kq = lane >> 4;
  if (WAVES > 8 && wave >= 8) return;
  const float4 *bq = (const float4 *)(qg + (n & 7) * kHeadDim + 4 * kq);
#pragma unroll
  for (int t2 = 0; t2 < RotRows<WAVES>::nt; ++t2) {
    const int t = wave + t2 * WAVES;
    f4v acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int u = 0; u < kHeadDim / 16; ++u) {
      const float4 a = rr.a[t2][u], b = bq[4 * u];
      f4v &c = acc[u & 3];
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
    }
    const f4v sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n < G) qs[n * kHeadDim + 16 * t + 4 * kq + r] = sum[r];
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

// LDS scratch of the preparation (before the tile loop), byte offsets from its base.
template <int G>
struct PrepScratch {
  static constexpr int kds = 0;                                  // KvhDesc words
  static constexpr int qn = ((int)sizeof(KvhDesc) + 15) & ~15;   // fp32 [G][128], natural coordinate order
  static constexpr int qg = qn + G * kHeadDim * 4;               // fp32 [8][128], group order, rows h >= G zero
  static constexpr int qs = qg + 8 * kHeadDim * 4;               // fp32 [G][128], rotated, group order
  static constexpr int hm = qs + G * kHeadDim * 4;               // fp32 [16 waves][G]
  static constexpr int bytes = (hm + 16 * G * 4 + 15) & ~15;
};

// The query preparation of one (sequence, KV head) by a workgroup of
// 64 WAVES threads: the G queries rotated once per key width group and turned
// into the tile loop's operands, in the PrepOut layout:
//  * q4[h][p] = kscale / sqrt(d4) q_rot[h][p] for the 4-bit group (0 elsewhere);
//  * qr[k][quad][m][i] = fp16(fac_h kscale / sqrt(d_g) q_rot[h][pos_g + 4 s + i]),
//    h = 4 quad + m, for k-step k = (group g, step s) of the width-1..3 groups
//    (0 past the group, for h >= G and past the head's k-steps);
//  * rinv[h] = 1 / fac_h, fac_h the power of two that brings the largest
//    |kscale / sqrt(d_g) q_rot[h][p]| over those groups to [2^13, 2^14).
// No global address depends on loaded data: prep_issue loads the queries in
// natural order, the head's descriptor and the row table entry of row
// p = tid % 128, prep_issue_rot the head's block-diagonal fp32 rotation as
// 16-row MFMA operand tiles.  prep_stage puts the descriptor and the queries
// into LDS (waiting for prep_issue's loads only); prep_build then gathers the
// queries into group order, rotates them on the matrix cores (rot_tiles, the
// first use of the rotation) and writes the operands; it ends with a workgroup
// barrier.
template <int G, int WAVES>
struct PrepIn {
  static constexpr int T = 64 * WAVES;
  static constexpr int nq = (G * kHeadDim + T - 1) / T;  // query values per thread
  uint32_t dw;                                             // one word of the KvhDesc
  uint16_t qv[nq];
  uint2 row;  // row table entry of p: y = d_g | pos_g << 8 | w << 16 | first k-step << 19
  RotKeys<WAVES> rk;
  RotRows<WAVES> rr;
};

// qb: the KV head's first query head; gr <= G heads are real (a group of 3, 5,
// 6 or 7 runs as the next power of two): rows h >= gr repeat row gr - 1, so
// that every row is a valid query and the decode's extra rows are never read.
template <int G, int WAVES>
__device__ __forceinline__ void prep_issue(PrepIn<G, WAVES> &in, const uint8_t *consts, int kvh,
                                           const uint16_t *qb, int gr, int tid, int wave, int lane) {
  typedef PrepIn<G, WAVES> PI;
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  static_assert(kDescWords <= PI::T, "one round of descriptor loads");
  const ConstHeader *hd = hdr_of(consts);
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  in.dw = ((const uint32_t *)kd)[min(tid, kDescWords - 1)];
#pragma unroll
  for (int u = 0; u < PI::nq; ++u) {
    const int i = min(tid + u * PI::T, G * kHeadDim - 1);
    in.qv[u] = qb[min(i / kHeadDim, gr - 1) * kHeadDim + i % kHeadDim];
  }
  in.row = ((const uint2 *)(consts + hd->off_rowk))[(size_t)kvh * kHeadDim + (tid & (kHeadDim - 1))];
}

// The row-table entries of the lane's rotation rows: the first loads of the prologue.
template <int G, int WAVES>
__device__ __forceinline__ void prep_issue_keys(PrepIn<G, WAVES> &in, const uint8_t *consts, int kvh, int wave,
                                                int lane) {
  const ConstHeader *hd = hdr_of(consts);
  rot_keys<WAVES>((const uint2 *)(consts + hd->off_rowk) + (size_t)kvh * kHeadDim, wave, lane, in.rk);
}

template <int G, int WAVES>
__device__ __forceinline__ void prep_issue_rot(PrepIn<G, WAVES> &in, const uint8_t *consts, int64_t off_zero, int kvh,
                                               int wave, int lane) {
  const ConstHeader *hd = hdr_of(consts);
  rot_rows_sparse<WAVES>((const float *)(consts + hd->off_rot32_k) + (size_t)kvh * kHeadDim * kHeadDim,
                         (const float *)(consts + off_zero), in.rk, wave, lane, in.rr);
}

// `out` and `scr`: LDS (PrepOut and PrepScratch layouts).
template <int G, int WAVES>
__device__ __forceinline__ void prep_stage(const PrepIn<G, WAVES> &in, uint8_t *out, uint8_t *scr, int tid) {
  typedef PrepOut<G> PO;
  typedef PrepScratch<G> PS;
  typedef PrepIn<G, WAVES> PI;
  constexpr int kDescWords = (int)(sizeof(KvhDesc) / 4);
  float *qn = (float *)(scr + PS::qn);
  if (tid < kDescWords) ((uint32_t *)(scr + PS::kds))[tid] = in.dw;
#pragma unroll
  for (int u = 0; u < PI::nq; ++u)
    if (tid + u * PI::T < G * kHeadDim) qn[tid + u * PI::T] = h2f(in.qv[u]);
  for (int i = tid; i < (PO::rinv - PO::qr) / 16; i += PI::T) ((uint4 *)(out + PO::qr))[i] = make_uint4(0u, 0u, 0u, 0u);
}

// `out` and `scr`: LDS (PrepOut and PrepScratch layouts).
template <int G, int WAVES>
__device__ __forceinline__ void prep_build(const PrepIn<G, WAVES> &in, uint8_t *out, uint8_t *scr, float kscale,
                                           int tid, int wave, int lane) {
  typedef PrepOut<G> PO;
  typedef PrepScratch<G> PS;
  typedef PrepIn<G, WAVES> PI;
  float *qn = (float *)(scr + PS::qn), *qg = (float *)(scr + PS::qg), *qs = (float *)(scr + PS::qs);
  float *hm = (float *)(scr + PS::hm);
  __syncthreads();
  // ---- gather into group order: qg[h][p] = q[h][coord[p]] for p < d_nz
  const KvhDesc &kds = *(const KvhDesc *)(scr + PS::kds);
  const int dnz = kds.d_nz;
  for (int i = tid; i < 8 * kHeadDim; i += PI::T) {
    const int h = i >> 7, pp = i & (kHeadDim - 1);
    qg[i] = (h < G && pp < dnz) ? qn[min(h, G - 1) * kHeadDim + kds.coord[pp < dnz ? pp : 0]] : 0.f;
  }
  __syncthreads();
  rot_tiles<WAVES>(in.rr, G, qg, qs, wave, lane);
  __syncthreads();
  // ---- operands of row p for heads hsel, hsel + T / 128, ...
  constexpr int kSel = PI::T / kHeadDim;                     // head strides over the threads
  constexpr int kHpt = (G + kSel - 1) / kSel;                // heads per thread
  const int p = tid & (kHeadDim - 1), hsel = tid >> 7;
  const int d = (int)(in.row.y & 255u), pos = (int)((in.row.y >> 8) & 255u), w = (int)((in.row.y >> 16) & 7u);
  const int kb = (int)(in.row.y >> 19);
  const float gsc = d > 0 ? kscale / sqrtf((float)d) : 0.f;
  const bool low = d > 0 && w < 4;
  float v[kHpt];
#pragma unroll
  for (int j = 0; j < kHpt; ++j) {
    const int h = hsel + kSel * j;
    v[j] = h < G ? qs[h * kHeadDim + p] * gsc : 0.f;
    if (h < G) ((float *)(out + PO::q4))[h * kHeadDim + p] = w == 4 ? v[j] : 0.f;
  }
  // per head: the largest scaled |q_rot| over the width-1..3 rows; the rows of
  // head selector hsel are waves 2 hsel and 2 hsel + 1
#pragma unroll
  for (int j = 0; j < kHpt; ++j) {
    const float m = wave_max(low ? fabsf(v[j]) : 0.f);
    const int h = hsel + kSel * j;
    if (lane == 0 && h < G) hm[wave * G + h] = m;
  }
  __syncthreads();
  _Float16 *qr = (_Float16 *)(out + PO::qr);
#pragma unroll
  for (int j = 0; j < kHpt; ++j) {
    const int h = hsel + kSel * j;
    if (h < G) {
      const float m = fmaxf(hm[(2 * hsel) * G + h], hm[(2 * hsel + 1) * G + h]);
      int e = 0;
      (void)frexpf(m, &e);
      e = m > 0.f ? e : 0;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
      if (p == 0) ((float *)(out + PO::rinv))[h] = ldexpf(1.f, e - 14);
      if (low) {
        const int r = p - pos, k = kb + (r >> 2);
        qr[((k * PO::nq + (h >> 2)) * 4 + (h & 3)) * 4 + (r & 3)] = (_Float16)(ldexpf(1.f, 14 - e) * v[j]);
      }
    }
  }
  __syncthreads();
}

}  // namespace bgtq
