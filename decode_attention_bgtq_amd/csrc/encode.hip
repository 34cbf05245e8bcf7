// TurboQuant-MSE encode of keys (per equal-width group, Block-GTQ widths) and
// values (one group at the uniform width) into the packed cache, on gfx950
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract: TQ-MSE as
// the base encoder, KxVy budgets; Block-GTQ README, introduction).  The group
// order, quantiser and bit layout are defined in include/bgtq.h.
#include "device.h"
#include "host.h"

namespace bgtq {

// Prefill path: one workgroup per (tile, KV head, sequence), every token of the
// tile at once.  fp64 rotation with a 4 x 8 register tile per thread (rows x
// tokens).
template <bool IS_V>
__global__ __launch_bounds__(256) void encode_kernel(const uint8_t *__restrict__ consts,
                                                     const uint16_t *__restrict__ x, int64_t tiles_cap,
                                                     int64_t t0, int64_t n_new,
                                                     uint32_t *__restrict__ codes,
                                                     uint16_t *__restrict__ norms) {
  __shared__ float xs[kTile][kHeadDim + 1];
  __shared__ uint8_t cs[kTile][kHeadDim];
  __shared__ double nrm[kTile];
  __shared__ uint16_t nrm16[kTile][4];
  const ConstHeader *hd = hdr_of(consts);
  const int hkv = hd->n_kv_heads;
  const int64_t tile = t0 / kTile + blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t tok0 = tile * kTile;
  const int lo = (int)(std::max(t0, tok0) - tok0);
  const int hi = (int)(std::min(t0 + n_new, tok0 + kTile) - tok0);
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;

  for (int idx = tid; idx < kTile * kHeadDim; idx += 256) {
    const int t = idx >> 7, c = idx & 127;
    float v = 0.f;
    if (t >= lo && t < hi) {
      const int64_t row = (int64_t)b * n_new + (tok0 + t - t0);
      v = h2f(x[((size_t)row * hkv + kvh) * kHeadDim + c]);
    }
    xs[t][c] = v;
  }
  if (tid < kTile * 4) nrm16[tid >> 2][tid & 3] = 0;
  __syncthreads();

  const int n_groups = IS_V ? 1 : kd->n_groups;
  for (int gi = 0; gi < n_groups; ++gi) {
    const int w = IS_V ? hd->v_bits : kd->g[gi].w;
    const int d = IS_V ? kHeadDim : kd->g[gi].d;
    const int pos = IS_V ? 0 : kd->g[gi].pos;
    const double *pt = IS_V ? (const double *)(consts + hd->off_rot64_v) + (size_t)kvh * kHeadDim * kHeadDim
                            : (const double *)(consts + hd->off_rot64_k) + kd->g[gi].rot64;
    if (tid < kTile) {
      u128 s = 0;
      for (int k = 0; k < d; ++k) {
        const int c = IS_V ? k : kd->coord[pos + k];
        const double a = fabs((double)xs[tid][c]) * 16777216.0;
        const uint64_t u = (uint64_t)a;
        s += (u128)u * u;
      }
      const double nn = sqrt(ldexp(u128_to_f64(s), -48));
      nrm[tid] = nn;
      nrm16[tid][IS_V ? 0 : 4 - w] = f64_to_f16(nn);
    }
    __syncthreads();
    const int rb = tid & 31, tb = tid >> 5;
    const int i0 = rb * 4, u0 = tb * 8;
    if (i0 < d) {
      double acc[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[r][u] = 0.0;
      for (int k = 0; k < d; ++k) {
        const int c = IS_V ? k : kd->coord[pos + k];
        double p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = (i0 + r < d) ? pt[(size_t)k * d + i0 + r] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double xv = (double)xs[u0 + u][c];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r][u] = fma(p[r], xv, acc[r][u]);
        }
      }
      const int nthr = (1 << w) - 1;
      const double *thr = hd->thr[w - 1];
      const double sd = sqrt((double)d);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double nn = nrm[u0 + u];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (i0 + r >= d) continue;
          const double y = nn > 0.0 ? acc[r][u] / nn : 0.0;
          const double z = sd * y;
          int code = 0;
          for (int kk = 0; kk < nthr; ++kk) code += thr[kk] < z ? 1 : 0;
          cs[u0 + u][pos + i0 + r] = (uint8_t)code;
        }
      }
    }
    __syncthreads();
  }

  const size_t base = ((size_t)b * hkv + kvh) * (size_t)tiles_cap + (size_t)tile;
  if (!IS_V) {
    const int wk = hd->wk;
    if (tid >= lo && tid < hi) {
      uint64_t accb = 0;
      int nb = 0, word = 0;
      for (int gi = 0; gi < kd->n_groups; ++gi) {
        const int w = kd->g[gi].w, d = kd->g[gi].d, pos = kd->g[gi].pos;
        for (int i = 0; i < d; ++i) {
          accb |= (uint64_t)cs[tid][pos + i] << nb;
          nb += w;
          if (nb >= 32) {
            codes[(base * wk + word) * kTile + tid] = (uint32_t)accb;
            ++word;
            accb >>= 32;
            nb -= 32;
          }
        }
      }
      for (; word < wk; ++word) {  // only reached for an empty stream tail
        codes[(base * wk + word) * kTile + tid] = (uint32_t)accb;
        accb = 0;
      }
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

// Append path for a few tokens: one workgroup of 512 threads per (tile, KV
// head, sequence), the tile's new tokens one after another.  Thread (p, q)
// owns group-order position p = tid % 128 and the k-quarter q = tid / 128 of
// its group's rotation row; its quarter of the fp64 rotation row is loaded
// into registers once, before the token loop, so the loads of all threads are
// in flight together.  The four partial dot products are added in quarter
// order.
constexpr int kAppendThreads = 512;

template <bool IS_V>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(const uint8_t *__restrict__ consts,
                                                                const uint16_t *__restrict__ x, int64_t tiles_cap,
                                                                int64_t t0, int64_t n_new,
                                                                uint32_t *__restrict__ codes,
                                                                uint16_t *__restrict__ norms) {
  __shared__ double part[4][kHeadDim];
  __shared__ float xg[kHeadDim];
  __shared__ uint8_t cs[kHeadDim];
  __shared__ u128 red[kMaxGroups][kHeadDim];
  __shared__ double nrm[kMaxGroups];
  __shared__ uint16_t n16[4];
  const ConstHeader *hd = hdr_of(consts);
  const int hkv = hd->n_kv_heads;
  const int64_t tile = t0 / kTile + blockIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int p = tid & (kHeadDim - 1), qtr = tid >> 7;
  const int64_t tok0 = tile * kTile;
  const int lo = (int)(std::max(t0, tok0) - tok0);
  const int hi = (int)(std::min(t0 + n_new, tok0 + kTile) - tok0);
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const size_t base = ((size_t)b * hkv + kvh) * (size_t)tiles_cap + (size_t)tile;
  const int n_groups = IS_V ? 1 : kd->n_groups;
  const int d_nz = IS_V ? kHeadDim : kd->d_nz;
  // position p's group, its place in the group, width and rotation
  int gi = 0;
  if (!IS_V)
    while (gi + 1 < n_groups && p >= kd->g[gi + 1].pos) ++gi;
  const int w = IS_V ? hd->v_bits : kd->g[gi].w;
  const int d = IS_V ? kHeadDim : kd->g[gi].d;
  const int pos = IS_V ? 0 : kd->g[gi].pos;
  const int i = p - pos < d ? p - pos : d - 1;
  const double *pt = IS_V ? (const double *)(consts + hd->off_rot64_v) + (size_t)kvh * kHeadDim * kHeadDim
                          : (const double *)(consts + hd->off_rot64_k) + kd->g[gi].rot64;
  const int kq = (d + 3) >> 2, k0 = qtr * kq, k1 = min(d, k0 + kq);
  double a[kHeadDim / 4];
#pragma unroll
  for (int j = 0; j < kHeadDim / 4; ++j) {
    const int k = min(k0 + j, d - 1);
    a[j] = pt[(size_t)k * d + i];
  }
  const int cp = IS_V ? p : (p < d_nz ? (int)kd->coord[p] : 0);

  for (int t = lo; t < hi; ++t) {
    const int64_t row = (int64_t)b * n_new + (tok0 + t - t0);
    if (tid < kHeadDim) xg[p] = p < d_nz ? h2f(x[((size_t)row * hkv + kvh) * kHeadDim + cp]) : 0.f;
    if (tid < 4) n16[tid] = 0;
    __syncthreads();
    // exact per-group sums of squares: one tree over 128 positions, a slot per group
    if (tid < kHeadDim) {
      u128 sq = 0;
      if (p < d_nz) {
        const uint64_t u = (uint64_t)(fabs((double)xg[p]) * 16777216.0);
        sq = (u128)u * u;
      }
#pragma unroll
      for (int g = 0; g < kMaxGroups; ++g) red[g][p] = g == gi ? sq : (u128)0;
    }
    {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < kHeadDim / 4; ++j) {
        const int k = k0 + j;
        const float xv = xg[pos + min(k, d - 1)];
        if (k < k1) acc = fma(a[j], (double)xv, acc);
      }
      part[qtr][p] = acc;
    }
    __syncthreads();
    for (int s = 64; s > 0; s >>= 1) {
      if (tid < s) {
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g) red[g][tid] += red[g][tid + s];
      }
      __syncthreads();
    }
    if (tid < n_groups) {
      const double nn = sqrt(ldexp(u128_to_f64(red[tid][0]), -48));
      nrm[tid] = nn;
      n16[IS_V ? 0 : 4 - kd->g[tid].w] = f64_to_f16(nn);
    }
    __syncthreads();
    if (tid < d_nz) {
      const double acc = ((part[0][p] + part[1][p]) + part[2][p]) + part[3][p];
      const double nn = nrm[gi];
      const double y = nn > 0.0 ? acc / nn : 0.0;
      const double z = sqrt((double)d) * y;
      const int nthr = (1 << w) - 1;
      const double *thr = hd->thr[w - 1];
      int code = 0;
      for (int kk = 0; kk < nthr; ++kk) code += thr[kk] < z ? 1 : 0;
      cs[p] = (uint8_t)code;
    }
    __syncthreads();
    if (!IS_V) {
      const int wk = hd->wk;
      if (tid < wk) {  // word tid of this token's key stream
        uint64_t word = 0;
        for (int g = 0; g < kd->n_groups; ++g) {
          const int gw = kd->g[g].w, gd = kd->g[g].d, gp = kd->g[g].pos, off = kd->g[g].bit_off;
          const int r0 = 32 * tid > off ? (32 * tid - off) / gw : 0;  // first code that can reach the word
          for (int r = r0; r < gd; ++r) {
            const int bit = off + gw * r - 32 * tid;
            if (bit >= 32) break;
            if (bit <= -gw) continue;
            const uint64_t c = cs[gp + r];
            word |= bit >= 0 ? c << bit : c >> (-bit);
          }
        }
        codes[(base * wk + tid) * kTile + t] = (uint32_t)word;
      }
      if (tid == 0) {
        uint2 nv;
        nv.x = (uint32_t)n16[0] | ((uint32_t)n16[1] << 16);
        nv.y = (uint32_t)n16[2] | ((uint32_t)n16[3] << 16);
        *(uint2 *)(norms + (base * kTile + t) * 4) = nv;
      }
    } else if (tid < kHeadDim) {
      const int vb = hd->v_bits, wv = 2 * vb;
      const int bit = vb * t, wi = bit >> 5, sh = bit & 31;
      const uint64_t c = (uint64_t)cs[p] << sh, m = ((1ull << vb) - 1) << sh;
      uint32_t *dst = codes + (base * kHeadDim + p) * wv + wi;
      dst[0] = (dst[0] & ~(uint32_t)m) | (uint32_t)c;
      if (sh + vb > 32) dst[1] = (dst[1] & ~(uint32_t)(m >> 32)) | (uint32_t)(c >> 32);
      if (tid == 0) norms[base * kTile + t] = n16[0];
    }
    __syncthreads();
  }
}

}  // namespace bgtq

using namespace bgtq;

namespace {

bgtq_status encode_common(bool is_v, const bgtq_plan *plan, const void *dev_consts, const uint16_t *x,
                          int32_t batch, int64_t capacity, int64_t t0, int64_t n_new, uint32_t *codes,
                          uint16_t *norms, bgtq_stream stream) {
  const char *nm = is_v ? "bgtq_encode_v" : "bgtq_encode_k";
  const bool no_codes = !is_v && plan && plan->p.hdr.wk == 0;  // zero-bit keys store no code words
  if (!plan || !dev_consts || (!codes && !no_codes) || !norms || (!x && n_new > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (batch < 1 || n_new < 0 || capacity < 0) return fail(BGTQ_EINVAL, std::string(nm) + ": bad batch or count");
  if (t0 < 0 || t0 + n_new > capacity) return fail(BGTQ_ECAPACITY, std::string(nm) + ": tokens beyond capacity");
  if (n_new == 0 || no_codes) return BGTQ_OK;  // zero-bit keys: the caller's zero norms stand
  const int64_t tiles_cap = (capacity + kTile - 1) / kTile;
  const int64_t first = t0 / kTile, last = (t0 + n_new - 1) / kTile;
  if (last - first + 1 > 0x7FFFFFFF || batch > 65535 || plan->p.desc.n_kv_heads > 65535)
    return fail(BGTQ_EINVAL, std::string(nm) + ": grid too large");
  const dim3 grid((unsigned)(last - first + 1), plan->p.desc.n_kv_heads, batch);
  const uint8_t *c = (const uint8_t *)dev_consts;
  hipStream_t st = (hipStream_t)stream;
  const bool small = n_new <= 8;  // a few tokens per tile: dot-product path
  if (is_v) {
    if (small) append_kernel<true><<<grid, kAppendThreads, 0, st>>>(c, x, tiles_cap, t0, n_new, codes, norms);
    else encode_kernel<true><<<grid, 256, 0, st>>>(c, x, tiles_cap, t0, n_new, codes, norms);
  } else {
    if (small) append_kernel<false><<<grid, kAppendThreads, 0, st>>>(c, x, tiles_cap, t0, n_new, codes, norms);
    else encode_kernel<false><<<grid, 256, 0, st>>>(c, x, tiles_cap, t0, n_new, codes, norms);
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

}  // extern "C"
