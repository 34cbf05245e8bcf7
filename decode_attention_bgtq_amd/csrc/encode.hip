// TurboQuant-MSE encode of keys (per equal-width group, Block-GTQ widths) and
// values (one group at the uniform width) into the packed cache, on gfx950
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract: TQ-MSE as
// the base encoder, KxVy budgets; Block-GTQ README, introduction).  The group
// order, quantiser and bit layout are defined in include/bgtq.h.
#include "append.h"
#include "device.h"
#include "host.h"

namespace bgtq {

// Prefill path: one workgroup per (tile, KV head, sequence), every token of the
// tile and every group at once: exact group norms (four threads per token),
// then the fp64 rotation and the quantiser with a 4 x 8 register tile per work
// item (rows x tokens), the work items of all groups spread over the threads.
template <bool IS_V>
__global__ __launch_bounds__(256) void encode_kernel(const uint8_t *__restrict__ consts,
                                                     const uint16_t *__restrict__ x, const TileMap map,
                                                     int64_t t0, int64_t n_new,
                                                     uint32_t *__restrict__ codes,
                                                     uint16_t *__restrict__ norms) {
  __shared__ float xs[kTile][kHeadDim + 1];
  __shared__ uint8_t cs[kTile][kHeadDim];
  __shared__ double nrm[kMaxGroups][kTile];
  __shared__ uint16_t nrm16[kTile][4];
  __shared__ int16_t cds[kHeadDim];  // the head's group-order coordinates (keys)
  __shared__ double thr_s[4][16];    // interior thresholds of the b-bit quantisers, row b - 1
  const ConstHeader *hd = hdr_of(consts);
  const int hkv = hd->n_kv_heads;
  const int64_t tile = t0 / kTile + blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t tok0 = tile * kTile;
  const int lo = (int)(std::max(t0, tok0) - tok0);
  const int hi = (int)(std::min(t0 + n_new, tok0 + kTile) - tok0);
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int64_t tix = tile_at(map, b, kvh, tile);
  if (tix < 0) return;  // a paged table entry outside the pool: nothing is written (uniform per workgroup)

  // the tile's rows into LDS as floats (zero outside [lo, hi)): 16-byte loads,
  // all issued before the first use (rows outside the range re-read row lo)
  constexpr int kChunks = kTile * kHeadDim / 8 / 256;  // 16-byte chunks per thread
  uint4 xv[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int idx = tid + 256 * j, t = idx >> 4, c8 = idx & 15;
    const int tt = (t >= lo && t < hi) ? t : lo;
    const int64_t row = (int64_t)b * n_new + (tok0 + tt - t0);
    xv[j] = *(const uint4 *)(x + ((size_t)row * hkv + kvh) * kHeadDim + 8 * c8);
  }
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int idx = tid + 256 * j, t = idx >> 4, c8 = idx & 15;
    const bool in = t >= lo && t < hi;
    const uint32_t w4[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xs[t][8 * c8 + 2 * e] = in ? h2f((uint16_t)(w4[e] & 0xFFFFu)) : 0.f;
      xs[t][8 * c8 + 2 * e + 1] = in ? h2f((uint16_t)(w4[e] >> 16)) : 0.f;
    }
  }
  if (tid < kTile * 4) nrm16[tid >> 2][tid & 3] = 0;
  if (!IS_V && tid < kHeadDim) cds[tid] = kd->coord[tid];
  if (!IS_V && tid < 64) thr_s[tid >> 4][tid & 15] = hd->thr[tid >> 4][tid & 15];
  __syncthreads();

  // ---- the groups (keys: up to four, in width order; values: one of 128)
  const int n_groups = IS_V ? 1 : kd->n_groups;
  int gw[kMaxGroups], gd[kMaxGroups], gpos[kMaxGroups], gpre[kMaxGroups];
  const double *gpt[kMaxGroups];
  int total_rb = 0;  // row blocks of four over every group
#pragma unroll
  for (int gi = 0; gi < kMaxGroups; ++gi) {
    const bool on = gi < n_groups;
    gw[gi] = !on ? 1 : IS_V ? hd->v_bits : kd->g[gi].w;
    gd[gi] = !on ? 0 : IS_V ? kHeadDim : kd->g[gi].d;
    gpos[gi] = !on ? 0 : IS_V ? 0 : kd->g[gi].pos;
    gpt[gi] = IS_V ? (const double *)(consts + hd->off_rot64_v) + (size_t)kvh * kHeadDim * kHeadDim
                   : (const double *)(consts + hd->off_rot64_k) + (on ? kd->g[gi].rot64 : 0);
    gpre[gi] = total_rb;
    total_rb += (gd[gi] + 3) / 4;
  }

  // ---- group norms, exact: |x| 2^24 = h 2^20 + l with h, l < 2^20 integers
  // (h = floor(|x| 16), l = its fraction times 2^20, both exact in fp32), so
  // x^2 2^48 = h^2 2^40 + 2 h l 2^20 + l^2; the three sums are 64-bit
  // integers.  Four threads per token, each every fourth coordinate, then the
  // total rounded once to double.
  {
    const int t = tid >> 2, q = tid & 3;
#pragma unroll
    for (int gi = 0; gi < kMaxGroups; ++gi) {
      if (gi >= n_groups) break;
      unsigned long long A = 0, B = 0, C = 0;
      for (int k = q; k < gd[gi]; k += 4) {
        const int c = IS_V ? k : cds[gpos[gi] + k];
        const float f = fabsf(xs[t][c]) * 16.f;
        const uint32_t h = (uint32_t)f;
        const uint32_t l = (uint32_t)((f - (float)h) * 1048576.f);
        A += (unsigned long long)h * h;
        B += (unsigned long long)h * l;
        C += (unsigned long long)l * l;
      }
      A += __shfl_xor(A, 1);
      B += __shfl_xor(B, 1);
      C += __shfl_xor(C, 1);
      A += __shfl_xor(A, 2);
      B += __shfl_xor(B, 2);
      C += __shfl_xor(C, 2);
      if (q == 0) {
        const u128 ss = ((u128)A << 40) + ((u128)B << 21) + (u128)C;
        const double nn = sqrt(ldexp(u128_to_f64(ss), -48));
        nrm[gi][t] = nn;
        nrm16[t][IS_V ? 0 : 4 - gw[gi]] = f64_to_f16(nn);
      }
    }
  }
  __syncthreads();

  // ---- rotation and quantiser.  Keys, every group at once: work item = (row
  // block of four rows of a group, block of eight tokens), a 4 x 8 register tile
  // each.
  const auto sel = [](const int (&a)[kMaxGroups], int gi) {
    return gi == 0 ? a[0] : gi == 1 ? a[1] : gi == 2 ? a[2] : a[3];
  };
  if constexpr (IS_V) {
    // values: Y = Pi X^T on the matrix cores (v_mfma_f64_16x16x4f64: A = 16
    // rows x 4 columns of Pi in lane r + 16 k, B = 4 coordinates x 16 tokens in
    // lane t + 16 k, D = rows lane / 16 + 4 e of token lane % 16, checked on the
    // device); wave w takes row tiles 2w and 2w + 1 and the four token tiles
    const double *pt = gpt[0];  // Pi^T [k][i]
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lk = lane >> 4;
    typedef double d4v __attribute__((ext_vector_type(4)));
    d4v acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) acc[a][bt] = (d4v){0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
    for (int k0 = 0; k0 < kHeadDim; k0 += 4) {
      const int k = k0 + lk;
      double av[2], bv[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = pt[(size_t)k * kHeadDim + 16 * (2 * wave + a) + lr];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) bv[bt] = (double)xs[16 * bt + lr][k];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) acc[a][bt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[bt], acc[a][bt], 0, 0, 0);
    }
    const int w = gw[0];
    const double *thr = hd->thr[w - 1];
    const double sd = sqrt((double)kHeadDim);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int t = 16 * bt + lr;
        const double nn = nrm[0][t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * (2 * wave + a) + lk + 4 * e;
          const double y = nn > 0.0 ? acc[a][bt][e] / nn : 0.0;
          const double z = sd * y;
          int code = 0;
          for (int kk = 0; kk < (1 << w) - 1; ++kk) code += thr[kk] < z ? 1 : 0;
          cs[t][i] = (uint8_t)code;
        }
      }
  } else {
    for (int item = tid; item < total_rb * 8; item += 256) {
      const int grb = item >> 3, tb = item & 7;
      int gi = 0;
  #pragma unroll
      for (int jg = 1; jg < kMaxGroups; ++jg) gi += (jg < n_groups && grb >= gpre[jg]) ? 1 : 0;
      const int w = sel(gw, gi), d = sel(gd, gi), pos = sel(gpos, gi);
      const double *pt = gi == 0 ? gpt[0] : gi == 1 ? gpt[1] : gi == 2 ? gpt[2] : gpt[3];
      const int i0 = 4 * (grb - sel(gpre, gi)), u0 = 8 * tb;
      double acc[4][8];
  #pragma unroll
      for (int r = 0; r < 4; ++r)
  #pragma unroll
        for (int u = 0; u < 8; ++u) acc[r][u] = 0.0;
  #pragma unroll 4
      for (int k = 0; k < d; ++k) {
        const int c = IS_V ? k : cds[pos + k];
        // unconditional loads (rows past d re-read row d - 1 and are zeroed), so
        // that the loads of the unrolled iterations are issued together
        double pr[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double pv = pt[(size_t)k * d + min(i0 + r, d - 1)];
          pr[r] = i0 + r < d ? pv : 0.0;
        }
  #pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double xv = (double)xs[u0 + u][c];
  #pragma unroll
          for (int r = 0; r < 4; ++r) acc[r][u] = fma(pr[r], xv, acc[r][u]);
        }
      }
      // keys: a wave mixes groups of different widths, so the thresholds come from
      // LDS by bisection; values: one width, the thresholds read through the
      // scalar cache and counted
      const double *thr = IS_V ? hd->thr[w - 1] : thr_s[w - 1];
      const double sd = sqrt((double)d);
  #pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double nn = nrm[gi][u0 + u];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (i0 + r >= d) continue;
          const double y = nn > 0.0 ? acc[r][u] / nn : 0.0;
          const double z = sd * y;
          // code = #{k : thr[k] < z} over the ascending thresholds
          int code = 0;
          if constexpr (IS_V) {
            for (int kk = 0; kk < (1 << w) - 1; ++kk) code += thr[kk] < z ? 1 : 0;
          } else {
            for (int step = 1 << (w - 1); step > 0; step >>= 1) code += thr[code + step - 1] < z ? step : 0;
          }
          cs[u0 + u][pos + i0 + r] = (uint8_t)code;
        }
      }
    }
  }
  __syncthreads();

  const size_t base = (size_t)tix;
  if (!IS_V) {
    // key words: work item (token t, word wi), lanes = tokens; word wi holds the
    // stream bits [32 wi, 32 wi + 32): the codes of every group that overlap them
    const int wk = hd->wk;
    int gbo[kMaxGroups];
#pragma unroll
    for (int gi = 0; gi < kMaxGroups; ++gi) gbo[gi] = gi < n_groups ? kd->g[gi].bit_off : 0;
    for (int item = tid; item < kTile * wk; item += 256) {
      const int t = item & (kTile - 1), wi = item >> 6;
      if (t < lo || t >= hi) continue;
      const int b0 = 32 * wi;
      uint64_t val = 0;
#pragma unroll
      for (int gi = 0; gi < kMaxGroups; ++gi) {
        if (gi >= n_groups) break;
        const int w = gw[gi], bo = gbo[gi], e = bo + gd[gi] * w;
        if (e <= b0 || bo >= b0 + 32) continue;
        const int k0 = bo >= b0 ? 0 : (b0 - bo) / w;
        const int k1 = min(gd[gi], (b0 + 32 - bo + w - 1) / w);
        for (int k = k0; k < k1; ++k) {
          const int off = bo + k * w - b0;  // may be negative for a code straddling the word start
          const uint64_t cv = cs[t][gpos[gi] + k];
          val |= off >= 0 ? cv << off : cv >> (-off);
        }
      }
      codes[(base * wk + wi) * kTile + t] = (uint32_t)val;
    }
    if (tid >= lo && tid < hi) {
      uint2 nv;
      nv.x = (uint32_t)nrm16[tid][0] | ((uint32_t)nrm16[tid][1] << 16);
      nv.y = (uint32_t)nrm16[tid][2] | ((uint32_t)nrm16[tid][3] << 16);
      *(uint2 *)(norms + (base * kTile + tid) * 4) = nv;
    }
  } else {
    const int vb = hd->v_bits, wv = 2 * vb;
    for (int idx = tid; idx < kHeadDim * wv; idx += 256) {
      const int ci = idx / wv, wi = idx % wv;
      const int b0 = 32 * wi, b1 = b0 + 32;
      uint64_t val = 0, mask = 0;
      for (int t = b0 / vb; t * vb < b1 && t < kTile; ++t) {
        const int off = t * vb - b0;
        const uint64_t cm = (1ull << vb) - 1;
        const uint64_t cv = t >= lo && t < hi ? (uint64_t)cs[t][ci] : 0;
        const uint64_t mv = t >= lo && t < hi ? cm : 0;
        if (off >= 0) {
          val |= cv << off;
          mask |= mv << off;
        } else {
          val |= cv >> (-off);
          mask |= mv >> (-off);
        }
      }
      const uint32_t m32 = (uint32_t)mask, v32 = (uint32_t)val;
      uint32_t *dst = codes + (base * kHeadDim + ci) * wv + wi;
      if (m32 == 0xFFFFFFFFu) *dst = v32;
      else if (m32) *dst = (*dst & ~m32) | (v32 & m32);
    }
    if (tid >= lo && tid < hi) norms[base * kTile + tid] = nrm16[tid][0];
  }
}

// Append path for a few tokens per tile (uniform start t0 for the batch): one
// workgroup per (tile, KV head, sequence), see append_role.
template <bool IS_V>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(const AppendArgs a, int64_t t0, int64_t n_new) {
  const int64_t tile = t0 / kTile + blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int64_t tok0 = tile * kTile;
  const int lo = (int)(std::max(t0, tok0) - tok0);
  const int hi = (int)(std::min(t0 + n_new, tok0 + kTile) - tok0);
  append_role<IS_V>(a, tile, kvh, b, lo, hi, (int64_t)b * n_new + (tok0 + lo - t0));
}

AppendArgs append_args(const Plan &p, const uint8_t *consts, const uint16_t *x, uint32_t *codes, uint16_t *norms,
                       const TileMap &map, bool is_v) {
  AppendArgs a;
  a.consts = consts;
  a.x = x;
  a.codes = codes;
  a.norms = norms;
  a.map = map;
  a.off_kvh = p.hdr.off_kvh;
  a.off_rot64 = is_v ? p.hdr.off_rot64_v : p.hdr.off_rot64_k;
  a.hkv = p.desc.n_kv_heads;
  a.wk = p.hdr.wk;
  a.v_bits = p.desc.v_bits;
  return a;
}

}  // namespace bgtq

using namespace bgtq;

namespace {

bgtq_status encode_common(bool is_v, const bgtq_plan *plan, const void *dev_consts, const uint16_t *x,
                          int32_t batch, int64_t capacity, int64_t t0, int64_t n_new, uint32_t *codes,
                          uint16_t *norms, bgtq_stream stream, const bgtq_pages *pages = nullptr) {
  const char *nm = pages ? (is_v ? "bgtq_encode_v_paged" : "bgtq_encode_k_paged") : (is_v ? "bgtq_encode_v" : "bgtq_encode_k");
  if (pages) {
    const bgtq_status ps = pages_check(pages, nm);
    if (ps != BGTQ_OK) return ps;
    capacity = (int64_t)kTile * pages->max_pages;
  }
  const bool no_codes = !is_v && plan && plan->p.hdr.wk == 0;  // zero-bit keys store no code words
  if (!plan || !dev_consts || (!codes && !no_codes) || !norms || (!x && n_new > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (batch < 1 || n_new < 0 || capacity < 0) return fail(BGTQ_EINVAL, std::string(nm) + ": bad batch or count");
  if (t0 < 0 || t0 + n_new > capacity) return fail(BGTQ_ECAPACITY, std::string(nm) + ": tokens beyond capacity");
  if ((uintptr_t)x & 15) return fail(BGTQ_EINVAL, std::string(nm) + ": k / v must be 16-byte aligned");
  if (n_new == 0 || no_codes) return BGTQ_OK;  // zero-bit keys: the caller's zero norms stand
  const TileMap map = pages ? paged_map(plan->p, pages) : contiguous_map(plan->p.desc.n_kv_heads, capacity);
  const int64_t first = t0 / kTile, last = (t0 + n_new - 1) / kTile;
  if (last - first + 1 > 0x7FFFFFFF || batch > 65535 || plan->p.desc.n_kv_heads > 65535)
    return fail(BGTQ_EINVAL, std::string(nm) + ": grid too large");
  const dim3 grid((unsigned)(last - first + 1), plan->p.desc.n_kv_heads, batch);
  const uint8_t *c = (const uint8_t *)dev_consts;
  hipStream_t st = (hipStream_t)stream;
  const bool small = n_new <= 8;  // a few tokens per tile: dot-product path
  if (is_v) {
    if (small) append_kernel<true><<<grid, kAppendThreads, 0, st>>>(append_args(plan->p, c, x, codes, norms, map, true), t0, n_new);
    else encode_kernel<true><<<grid, 256, 0, st>>>(c, x, map, t0, n_new, codes, norms);
  } else {
    if (small) append_kernel<false><<<grid, kAppendThreads, 0, st>>>(append_args(plan->p, c, x, codes, norms, map, false), t0, n_new);
    else encode_kernel<false><<<grid, 256, 0, st>>>(c, x, map, t0, n_new, codes, norms);
  }
  return launch_status(nm);
}

}  // namespace

extern "C" {

bgtq_status bgtq_encode_k(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k, int32_t batch,
                          int64_t capacity, int64_t t0, int64_t n_new, uint32_t *k_codes, uint16_t *k_norms,
                          bgtq_stream stream) {
  return encode_common(false, plan, dev_consts, k, batch, capacity, t0, n_new, k_codes, k_norms, stream);
}

bgtq_status bgtq_encode_v(const bgtq_plan *plan, const void *dev_consts, const uint16_t *v, int32_t batch,
                          int64_t capacity, int64_t t0, int64_t n_new, uint32_t *v_codes, uint16_t *v_norms,
                          bgtq_stream stream) {
  return encode_common(true, plan, dev_consts, v, batch, capacity, t0, n_new, v_codes, v_norms, stream);
}

bgtq_status bgtq_encode_k_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *k, int32_t batch,
                                const bgtq_pages *pages, int64_t t0, int64_t n_new, uint32_t *k_codes,
                                uint16_t *k_norms, bgtq_stream stream) {
  if (!pages) return fail(BGTQ_EINVAL, "bgtq_encode_k_paged: null pages");
  return encode_common(false, plan, dev_consts, k, batch, 0, t0, n_new, k_codes, k_norms, stream, pages);
}

bgtq_status bgtq_encode_v_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *v, int32_t batch,
                                const bgtq_pages *pages, int64_t t0, int64_t n_new, uint32_t *v_codes,
                                uint16_t *v_norms, bgtq_stream stream) {
  if (!pages) return fail(BGTQ_EINVAL, "bgtq_encode_v_paged: null pages");
  return encode_common(true, plan, dev_consts, v, batch, 0, t0, n_new, v_codes, v_norms, stream, pages);
}

}  // extern "C"
