// Append of a few tokens to the packed cache: one workgroup of 512 threads per
// (tile, KV head, sequence).  TurboQuant-MSE per key width group / for the
// values ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract;
// Block-GTQ README, introduction).  Internal header, shared by the append
// kernels and the fused decode step.
#pragma once

#include "device.h"

namespace bgtq {

constexpr int kAppendThreads = 512;

struct AppendArgs {
  const uint8_t *consts;
  const uint16_t *x;  // [rows][n_kv_heads][128] fp16
  uint32_t *codes;
  uint16_t *norms;
  TileMap map;                  // tile addresses (contiguous or paged)
  int64_t off_kvh, off_rot64;  // off_rot64: K group area or Pi_V^T area
  int hkv, wk, v_bits;
};

// One DPP step of a wave sum of doubles: v + (v moved by the DPP pattern; lanes
// the pattern does not write add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
  return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes of a wave of integers below 2^40 held as doubles (every
// partial sum is an integer below 2^47, so the fp64 additions are exact and the
// order does not matter): quad, half-row, row steps, then the row broadcasts;
// the total is read from lane 63.
__device__ __forceinline__ uint64_t wave_sum_int40(uint64_t x) {
  double v = (double)x;
  v = dpp_add_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add_f64<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add_f64<0x140, 0xF>(v);  // row_mirror
  v = dpp_add_f64<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_add_f64<0x143, 0xC>(v);  // row_bcast:31
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return (uint64_t)__builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Tokens lo..hi-1 of cache tile `tile` of (sequence b, KV head kvh); token t
// comes from row row0 + (t - lo) of x.  Thread (p, q) owns group-order
// position p = tid % 128 and the k-quarter q = tid / 128 of its group's
// rotation row; that quarter of the fp64 rotation row is loaded into registers
// once, before the token loop, and the four partial dot products are added in
// quarter order.  Group norms are exact: the fp16 squares as integers
// (|x| 2^24)^2, split at bit 40 and summed per wave (DPP steps on the halves
// below 2^40, added exactly in fp64), then rounded once to float64.  Codes are OR-ed into the token's key words in LDS.
template <bool IS_V>
__device__ __forceinline__ void append_role(const AppendArgs &a, int64_t tile, int kvh, int b, int lo, int hi,
                                            int64_t row0) {
  __shared__ KvhDesc kds;
  __shared__ double thr_s[4][16];
  __shared__ double part[4][kHeadDim];
  __shared__ float xn[kHeadDim];
  __shared__ float xg[kHeadDim];
  __shared__ uint64_t gsum[2][kMaxGroups][2];
  __shared__ uint32_t words[kMaxWK];
  __shared__ double nrm[kMaxGroups];
  __shared__ uint16_t n16[4];
  const ConstHeader *hd = hdr_of(a.consts);
  const int hkv = a.hkv, tid = threadIdx.x, lane = tid & 63;
  const int p = tid & (kHeadDim - 1), qtr = tid >> 7;
  const int64_t tix = tile_at(a.map, b, kvh, tile);
  if (tix < 0) return;  // a paged table entry outside the pool: nothing is written (uniform per workgroup)
  const size_t base = (size_t)tix;
  // ---- descriptor, thresholds and the first token into LDS
  if (!IS_V) {
    const uint32_t *src = (const uint32_t *)((const KvhDesc *)(a.consts + a.off_kvh) + kvh);
    for (int i = tid; i < (int)(sizeof(KvhDesc) / 4); i += kAppendThreads) ((uint32_t *)&kds)[i] = src[i];
  }
  if (tid < 64) thr_s[tid >> 4][tid & 15] = hd->thr[tid >> 4][tid & 15];
  if (tid < kHeadDim) xn[tid] = h2f(a.x[((size_t)row0 * hkv + kvh) * kHeadDim + tid]);
  __syncthreads();
  const int n_groups = IS_V ? 1 : kds.n_groups;
  const int d_nz = IS_V ? kHeadDim : kds.d_nz;
  int gi = 0;
  if (!IS_V)
    while (gi + 1 < n_groups && p >= kds.g[gi + 1].pos) ++gi;
  const int w = IS_V ? a.v_bits : kds.g[gi].w;
  const int d = IS_V ? kHeadDim : kds.g[gi].d;
  const int pos = IS_V ? 0 : kds.g[gi].pos;
  const int i = p - pos < d ? p - pos : d - 1;
  const double *pt = (const double *)(a.consts + a.off_rot64) +
                     (IS_V ? (size_t)kvh * kHeadDim * kHeadDim : (size_t)kds.g[gi].rot64);
  const int kq = (d + 3) >> 2, k0 = qtr * kq, k1 = min(d, k0 + kq);
  double ar[kHeadDim / 4];
#pragma unroll
  for (int j = 0; j < kHeadDim / 4; ++j) ar[j] = pt[(size_t)min(k0 + j, d - 1) * d + i];
  const int cp = IS_V ? p : (p < d_nz ? (int)kds.coord[p] : 0);
  const int boff = IS_V ? 0 : kds.g[gi].bit_off + w * (p - pos);  // first bit of position p's code

  for (int t = lo; t < hi; ++t) {
    if (t > lo) {
      __syncthreads();
      if (tid < kHeadDim) xn[tid] = h2f(a.x[((size_t)(row0 + t - lo) * hkv + kvh) * kHeadDim + tid]);
      __syncthreads();
    }
    if (tid < kHeadDim) xg[p] = p < d_nz ? xn[cp] : 0.f;
    if (tid < kMaxWK) words[tid] = 0u;
    if (tid < 4) n16[tid] = 0;  // slots of absent widths stay zero
    // exact per-group sums of squares: waves 0 and 1 hold the 128 positions
    if (tid < kHeadDim) {
      uint64_t shi = 0, slo = 0;
      if (p < d_nz) {
        const uint64_t u = (uint64_t)(fabsf(xn[cp]) * 16777216.0f);  // |x| 2^24, exact for fp16 inputs
        const u128 sq = (u128)u * u;
        shi = (uint64_t)(sq >> 40);
        slo = (uint64_t)sq & ((1ull << 40) - 1);
      }
      for (int g = 0; g < n_groups; ++g) {
        const uint64_t h = wave_sum_int40(g == gi ? shi : 0), l = wave_sum_int40(g == gi ? slo : 0);
        if (lane == 0) gsum[tid >> 6][g][0] = h, gsum[tid >> 6][g][1] = l;
      }
    }
    __syncthreads();
    {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < kHeadDim / 4; ++j) {
        const int k = k0 + j;
        const float xv = xg[pos + min(k, d - 1)];
        if (k < k1) acc = fma(ar[j], (double)xv, acc);
      }
      part[qtr][p] = acc;
    }
    if (tid < n_groups) {
      const u128 s = (((u128)(gsum[0][tid][0] + gsum[1][tid][0])) << 40) + (u128)(gsum[0][tid][1] + gsum[1][tid][1]);
      const double nn = sqrt(ldexp(u128_to_f64(s), -48));
      nrm[tid] = nn;
      n16[IS_V ? 0 : 4 - kds.g[tid].w] = f64_to_f16(nn);
    }
    __syncthreads();
    if (tid < d_nz) {
      const double acc = ((part[0][p] + part[1][p]) + part[2][p]) + part[3][p];
      const double nn = nrm[gi];
      const double y = nn > 0.0 ? acc / nn : 0.0;
      const double z = sqrt((double)d) * y;
      const int nthr = (1 << w) - 1;
      uint32_t code = 0;
      for (int kk = 0; kk < nthr; ++kk) code += thr_s[w - 1][kk] < z ? 1u : 0u;
      if (!IS_V) {
        const int wi = boff >> 5, sh = boff & 31;
        atomicOr(&words[wi], code << sh);
        if (sh + w > 32) atomicOr(&words[wi + 1], code >> (32 - sh));
      } else {
        const int vb = a.v_bits, wv = 2 * vb;
        const int bit = vb * t, wj = bit >> 5, sb = bit & 31;
        const uint64_t c = (uint64_t)code << sb, m = ((1ull << vb) - 1) << sb;
        uint32_t *dst = a.codes + (base * kHeadDim + p) * wv + wj;
        dst[0] = (dst[0] & ~(uint32_t)m) | (uint32_t)c;
        if (sb + vb > 32) dst[1] = (dst[1] & ~(uint32_t)(m >> 32)) | (uint32_t)(c >> 32);
      }
    }
    if (!IS_V) {
      __syncthreads();
      if (tid < a.wk) a.codes[(base * a.wk + tid) * kTile + t] = words[tid];
      if (tid == 0) {
        uint2 nv;
        nv.x = (uint32_t)n16[0] | ((uint32_t)n16[1] << 16);
        nv.y = (uint32_t)n16[2] | ((uint32_t)n16[3] << 16);
        *(uint2 *)(a.norms + (base * kTile + t) * 4) = nv;
      }
    } else if (tid == 0) {
      a.norms[base * kTile + t] = n16[0];
    }
  }
}

}  // namespace bgtq
