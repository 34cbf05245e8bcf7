// Host-side plan for the Block-GTQ packed-KV path: Lloyd-Max codebooks,
// seeded Haar rotations, key group maps, decode k-step descriptors and tables,
// and the device constant image.  Pure host C++ (no HIP calls).
//
// Method sources: "RoPE-Aware Bit Allocation for KV-Cache Quantization",
// Abstract (TurboQuant-MSE as the base encoder, per-(layer, KV head) integer
// widths); Block-GTQ README introduction (grouping by width under a fixed
// average budget).  The quantiser, rotation and layout details the pages leave
// open are fixed as follows and restated in bgtq.h:
//  * b-bit Lloyd-Max quantiser of N(0,1) (Lloyd 1957, Max 1960) in double,
//    made exactly odd-symmetric, applied to sqrt(d_g) * y.
//  * Rotations: SplitMix64 (Steele, Lea, Flood 2014) absorbing (seed, layer,
//    kvh, tensor, width, d); Box-Muller Gaussians filled row-major; Householder
//    QR, Pi = Q diag(sign R_ii) with sign(0) = +1 (Mezzadri 2007).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace bgtq {
namespace {

// ---------------------------------------------------------------- codebooks
double gauss_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

// P(a <= X < b), X ~ N(0,1); upper-tail form when both ends are positive.
double gauss_mass(double a, double b) {
  const double r2 = std::sqrt(2.0);
  if (a >= 0.0) return 0.5 * (std::erfc(a / r2) - std::erfc(b / r2));
  if (b <= 0.0) return 0.5 * (std::erfc(-b / r2) - std::erfc(-a / r2));
  return 1.0 - 0.5 * std::erfc(-a / r2) - 0.5 * std::erfc(b / r2);
}

Codebook make_codebook(int bits) {
  const int n = 1 << bits;
  std::vector<double> c(n), t(n + 1), nc(n);
  for (int k = 0; k < n; ++k) c[k] = -2.0 + 4.0 * (k + 0.5) / n;
  for (int it = 0; it < 100000; ++it) {
    t[0] = -INFINITY;
    t[n] = INFINITY;
    for (int k = 1; k < n; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double move = 0.0;
    for (int k = 0; k < n; ++k) {
      nc[k] = (gauss_pdf(t[k]) - gauss_pdf(t[k + 1])) / gauss_mass(t[k], t[k + 1]);
      move = std::max(move, std::fabs(nc[k] - c[k]));
    }
    c = nc;
    if (move <= 1e-15) break;
  }
  std::vector<double> s(n);
  for (int k = 0; k < n; ++k) s[k] = (c[k] - c[n - 1 - k]) / 2.0;
  Codebook cb;
  cb.c = s;
  cb.t.resize(n - 1);
  for (int k = 1; k < n; ++k) cb.t[k - 1] = 0.5 * (s[k - 1] + s[k]);
  // D(b) = 1 - sum_k p_k c_k^2, summed with Neumaier compensation
  double sum = 0.0, comp = 0.0;
  for (int k = 0; k < n; ++k) {
    const double lo = k ? cb.t[k - 1] : -INFINITY, hi = k < n - 1 ? cb.t[k] : INFINITY;
    const double term = gauss_mass(lo, hi) * s[k] * s[k];
    const double tt = sum + term;
    comp += std::fabs(sum) >= std::fabs(term) ? (sum - tt) + term : (term - tt) + sum;
    sum = tt;
  }
  cb.d = 1.0 - (sum + comp);
  return cb;
}

// ---------------------------------------------------------------- rotations
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Stream {
  uint64_t s = 0;
  void absorb(uint64_t f) { s = sm_mix((s ^ f) + kGamma); }
  uint64_t next() {
    s += kGamma;
    return sm_mix(s);
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
};

// Haar rotation of size d for the given stream fields, row-major Pi[i][k].
std::vector<double> haar(uint64_t seed, int layer, int kvh, int tensor, int width, int d) {
  Stream st;
  const uint64_t fields[6] = {seed, (uint64_t)(int64_t)layer, (uint64_t)kvh, (uint64_t)tensor,
                              (uint64_t)width, (uint64_t)d};
  for (uint64_t f : fields) st.absorb(f);
  std::vector<double> a((size_t)d * d);
  for (size_t i = 0; i < a.size(); i += 2) {
    const double u1 = st.uniform(), u2 = st.uniform();
    const double r = std::sqrt(-2.0 * std::log(1.0 - u1));
    a[i] = r * std::cos(2.0 * M_PI * u2);
    a[i + 1] = r * std::sin(2.0 * M_PI * u2);
  }
  // Householder QR: a <- R, q <- H_0 H_1 ... H_{d-1}
  std::vector<double> q((size_t)d * d, 0.0), v(d);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  std::vector<double> diag(d);
  for (int j = 0; j < d; ++j) {
    double nrm2 = 0.0;
    for (int i = j; i < d; ++i) nrm2 += a[(size_t)i * d + j] * a[(size_t)i * d + j];
    const double nrm = std::sqrt(nrm2);
    if (nrm == 0.0) {
      diag[j] = 0.0;
      continue;
    }
    const double x0 = a[(size_t)j * d + j];
    const double alpha = x0 >= 0.0 ? -nrm : nrm;
    double vn2 = 0.0;
    for (int i = j; i < d; ++i) {
      v[i] = a[(size_t)i * d + j] - (i == j ? alpha : 0.0);
      vn2 += v[i] * v[i];
    }
    if (vn2 == 0.0) {
      diag[j] = x0;
      continue;
    }
    const double beta = 2.0 / vn2;
    for (int k = j; k < d; ++k) {
      double s = 0.0;
      for (int i = j; i < d; ++i) s += v[i] * a[(size_t)i * d + k];
      s *= beta;
      for (int i = j; i < d; ++i) a[(size_t)i * d + k] -= s * v[i];
    }
    for (int r = 0; r < d; ++r) {
      double s = 0.0;
      for (int i = j; i < d; ++i) s += q[(size_t)r * d + i] * v[i];
      s *= beta;
      for (int i = j; i < d; ++i) q[(size_t)r * d + i] -= s * v[i];
    }
    diag[j] = a[(size_t)j * d + j];
  }
  for (int r = 0; r < d; ++r)
    for (int k = 0; k < d; ++k)
      if (diag[k] < 0.0) q[(size_t)r * d + k] = -q[(size_t)r * d + k];
  return q;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// float64 -> fp16 bits, round to nearest even (finite inputs of any size).
uint16_t f16_bits(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < std::ldexp(1.0, -14)) return sign | (uint16_t)std::nearbyint(std::ldexp(a, 24));  // 1024 = min normal
  int e = 0;
  const double f = std::frexp(a, &e);  // a = f 2^e, f in [0.5, 1)
  double m = std::nearbyint((2.0 * f - 1.0) * 1024.0);
  int ex = e - 1;
  if (m >= 1024.0) m = 0.0, ++ex;
  if (ex > 15) return sign | 0x7C00;
  return sign | (uint16_t)((ex + 15) << 10) | (uint16_t)m;
}

// Value lookup table of width vb: for a code byte (or 6-bit pair for vb = 3)
// of one coordinate, the fp16 centroids of its tokens packed in pairs.
std::vector<uint32_t> value_table(int vb) {
  uint16_t c16[16];
  const Codebook &cb = codebook(vb);
  for (int k = 0; k < (1 << vb); ++k) c16[k] = f16_bits(cb.c[k]);
  std::vector<uint32_t> t;
  if (vb == 1) {
    for (int y = 0; y < 256; ++y)
      for (int u = 0; u < 4; ++u) t.push_back(c16[(y >> (2 * u)) & 1] | ((uint32_t)c16[(y >> (2 * u + 1)) & 1] << 16));
  } else if (vb == 2) {
    for (int y = 0; y < 256; ++y) {
      t.push_back(c16[y & 3] | ((uint32_t)c16[(y >> 2) & 3] << 16));
      t.push_back(c16[(y >> 4) & 3] | ((uint32_t)c16[(y >> 6) & 3] << 16));
    }
  } else if (vb == 3) {
    for (int y = 0; y < 64; ++y) t.push_back(c16[y & 7] | ((uint32_t)c16[(y >> 3) & 7] << 16));
  } else {
    for (int y = 0; y < 256; ++y) t.push_back(c16[y & 15] | ((uint32_t)c16[(y >> 4) & 15] << 16));
  }
  return t;
}

}  // namespace

const Codebook &codebook(int bits) {
  static std::once_flag once;
  static Codebook books[4];
  std::call_once(once, [] {
    for (int b = 1; b <= 4; ++b) books[b - 1] = make_codebook(b);
  });
  return books[bits - 1];
}

bgtq_status build_plan(const bgtq_plan_desc &d, Plan &p, std::string &err) {
  const int hkv = d.n_kv_heads, hq = d.n_q_heads;
  if (hkv < 1 || hq < 1 || hq % hkv) {
    err = "n_q_heads must be a positive multiple of n_kv_heads";
    return BGTQ_EINVAL;
  }
  const int G = hq / hkv;
  if (G > 8) {
    err = "at most 8 query heads per KV head";
    return BGTQ_EINVAL;
  }
  if (d.head_dim != kHeadDim) {
    err = "head_dim must be 128";
    return BGTQ_EINVAL;
  }
  if (!d.k_bits) {
    err = "k_bits is NULL";
    return BGTQ_EINVAL;
  }
  if (d.rope_pairing != BGTQ_ROPE_HALF && d.rope_pairing != BGTQ_ROPE_INTERLEAVED) {
    err = "rope_pairing must be BGTQ_ROPE_HALF or BGTQ_ROPE_INTERLEAVED";
    return BGTQ_EINVAL;
  }
  if (d.k_avg_bits < 0 || d.k_avg_bits > 4 || d.v_bits < 1 || d.v_bits > 4) {
    err = "k_avg_bits must be 0..4 and v_bits 1..4";
    return BGTQ_EBUDGET;
  }
  p.desc = d;
  p.bits.assign(d.k_bits, d.k_bits + (size_t)hkv * kBlocks);
  p.desc.k_bits = nullptr;
  for (int h = 0; h < hkv; ++h) {
    int sum = 0;
    for (int j = 0; j < kBlocks; ++j) {
      const int b = p.bits[(size_t)h * kBlocks + j];
      if (b < 0 || b > 4) {
        err = "k_bits entries must be 0..4";
        return BGTQ_EBUDGET;
      }
      sum += b;
    }
    if (sum != d.k_avg_bits * kBlocks) {
      err = "a row of k_bits does not sum to k_avg_bits * 64";
      return BGTQ_EBUDGET;
    }
  }
  const int wk = 4 * d.k_avg_bits;

  // groups, coordinates, bit offsets, rotations; block j holds coordinates (j, j+64) half-split
  // or (2j, 2j+1) interleaved, next to each other in its group
  const bool inter = d.rope_pairing == BGTQ_ROPE_INTERLEAVED;
  p.kvh.assign(hkv, KvhDesc{});
  p.rot_k.clear();
  p.rot_v.clear();
  int64_t rot64_k = 0, rot32_k = 0;
  for (int h = 0; h < hkv; ++h) {
    KvhDesc &kd = p.kvh[h];
    std::memset(&kd, 0, sizeof(kd));
    int pos = 0, bit = 0;
    for (int w = 4; w >= 1; --w) {
      int dg = 0;
      for (int j = 0; j < kBlocks; ++j)
        if (p.bits[(size_t)h * kBlocks + j] == w) {
          kd.coord[pos + dg++] = (int16_t)(inter ? 2 * j : j);
          kd.coord[pos + dg++] = (int16_t)(inter ? 2 * j + 1 : j + kBlocks);
        }
      if (!dg) continue;
      KGroupDesc &g = kd.g[kd.n_groups++];
      g.w = w;
      g.d = dg;
      g.pos = pos;
      g.bit_off = bit;
      g.rot64 = rot64_k;
      g.rot32 = rot32_k;
      rot64_k += (int64_t)dg * dg;
      rot32_k += (int64_t)dg * dg;
      p.rot_k.push_back(haar(d.seed, d.layer, h, 0, w, dg));
      pos += dg;
      bit += w * dg;
    }
    kd.d_nz = pos;
    p.rot_v.push_back(haar(d.seed, d.layer, h, 1, d.v_bits, kHeadDim));
  }

  // decode k-steps of the width-1..3 groups (four positions each)
  std::vector<int> kbase((size_t)hkv * kMaxGroups, 0);  // first k-step of each width-1..3 group
  int max_ksteps = 0;
  for (int h = 0; h < hkv; ++h) {
    KvhDesc &kd = p.kvh[h];
    int c = 0;
    kd.d4 = (kd.n_groups > 0 && kd.g[0].w == 4) ? kd.g[0].d : 0;
    kd.n4blk = (kd.d4 + 15) / 16;
    kd.n4w = (kd.d4 + 7) / 8;
    kd.gbit = 0;
    int cfirst[3] = {-1, -1, -1};  // first k-step of the width-3, 2, 1 groups
    for (int gi = 0; gi < kd.n_groups; ++gi) {
      const KGroupDesc &g = kd.g[gi];
      if (g.w == 4) continue;  // one matrix-core step per code in the decode
      const int rg = 3 - g.w;  // rest-group index
      cfirst[rg] = c;
      kbase[(size_t)h * kMaxGroups + gi] = c;
      kd.gbit |= (uint32_t)g.bit_off << (10 * rg);
      c += (g.d + 3) / 4;
      if (c > kMaxKSteps) {
        err = "internal: too many k-steps";
        return BGTQ_EINVAL;
      }
    }
    kd.n_ksteps = c;
    max_ksteps = std::max(max_ksteps, c);
    // k-step boundaries of the width-3, 2, 1 groups (an absent group is an empty range)
    int bnd[4];
    bnd[3] = c;
    for (int rg = 2; rg >= 0; --rg) bnd[rg] = cfirst[rg] >= 0 ? cfirst[rg] : bnd[rg + 1];
    kd.cgrp = (uint32_t)bnd[0] | ((uint32_t)bnd[1] << 8) | ((uint32_t)bnd[2] << 16) | ((uint32_t)bnd[3] << 24);
  }

  // constant image
  ConstHeader &hd = p.hdr;
  std::memset(&hd, 0, sizeof(hd));
  hd.n_kv_heads = hkv;
  hd.n_q_heads = hq;
  hd.group = G;
  hd.head_dim = kHeadDim;
  hd.k_avg_bits = d.k_avg_bits;
  hd.v_bits = d.v_bits;
  hd.wk = wk;
  hd.wv = 2 * d.v_bits;
  hd.max_ksteps = max_ksteps;
  for (int b = 1; b <= 4; ++b) {
    const Codebook &cb = codebook(b);
    for (int k = 0; k < (1 << b); ++k) hd.cent[b - 1][k] = cb.c[k];
    for (int k = 0; k < (1 << b) - 1; ++k) hd.thr[b - 1][k] = cb.t[k];
    hd.dist[b] = cb.d;
  }
  hd.dist[0] = 1.0;
  size_t off = align256(sizeof(ConstHeader));
  hd.off_kvh = off;
  off = align256(off + sizeof(KvhDesc) * hkv);
  hd.off_rot64_k = off;
  off = align256(off + 8 * (size_t)rot64_k);
  hd.off_rot32_k = off;
  off = align256(off + 4 * (size_t)hkv * kHeadDim * kHeadDim);
  hd.off_rot64_v = off;
  off = align256(off + 8 * (size_t)hkv * kHeadDim * kHeadDim);
  hd.off_rot32_v = off;
  off = align256(off + 4 * (size_t)hkv * kHeadDim * kHeadDim);
  const std::vector<uint32_t> vlut = value_table(d.v_bits);
  hd.off_dtab = off;
  off = align256(off + kDtabBytes);
  hd.off_vlut = off;
  hd.vlut_bytes = 4 * (int64_t)vlut.size();
  off = align256(off + 4 * vlut.size());
  hd.off_rowk = off;
  off = align256(off + 8 * (size_t)hkv * kHeadDim);
  hd.off_zero = off;
  off = align256(off + kZeroBytes);
  hd.total_bytes = off;

  p.image.assign(off, 0);
  uint8_t *img = p.image.data();
  std::memcpy(img, &hd, sizeof(hd));
  std::memcpy(img + hd.off_kvh, p.kvh.data(), sizeof(KvhDesc) * hkv);
  double *r64k = (double *)(img + hd.off_rot64_k);
  float *r32k = (float *)(img + hd.off_rot32_k);
  size_t gidx = 0;
  for (int h = 0; h < hkv; ++h)
    for (int gi = 0; gi < p.kvh[h].n_groups; ++gi, ++gidx) {
      const KGroupDesc &g = p.kvh[h].g[gi];
      const std::vector<double> &pi = p.rot_k[gidx];
      for (int i = 0; i < g.d; ++i)
        for (int k = 0; k < g.d; ++k) {
          r64k[g.rot64 + (int64_t)k * g.d + i] = pi[(size_t)i * g.d + k];
          r32k[((size_t)h * kHeadDim + g.pos + i) * kHeadDim + g.pos + k] = (float)pi[(size_t)i * g.d + k];
        }
    }
  {
    // per group-order row of the key rotation: its group's size, position, width and first k-step
    uint32_t *rowk = (uint32_t *)(img + hd.off_rowk);
    for (int h = 0; h < hkv; ++h)
      for (int gi = 0; gi < p.kvh[h].n_groups; ++gi) {
        const KGroupDesc &g = p.kvh[h].g[gi];
        const uint32_t kb = g.w < 4 ? (uint32_t)kbase[(size_t)h * kMaxGroups + gi] : 0u;
        for (int i = 0; i < g.d; ++i) {
          const size_t r = (size_t)h * kHeadDim + g.pos + i;
          rowk[2 * r] = (uint32_t)i;
          rowk[2 * r + 1] = (uint32_t)g.d | ((uint32_t)g.pos << 8) | ((uint32_t)g.w << 16) | (kb << 19);
        }
      }
  }
  {
    uint8_t *dt = img + hd.off_dtab;
    float *c4 = (float *)(dt + kDtabC4);
    const Codebook &cb4 = codebook(4);
    for (int e = 0; e < 256; ++e) {
      c4[2 * e] = (float)cb4.c[e & 15];
      c4[2 * e + 1] = (float)cb4.c[e >> 4];
    }
    uint16_t *t2 = (uint16_t *)(dt + kDtabT2), *t1 = (uint16_t *)(dt + kDtabT1), *t3 = (uint16_t *)(dt + kDtabT3);
    const Codebook &cb1 = codebook(1), &cb2 = codebook(2), &cb3 = codebook(3);
    for (int y = 0; y < 256; ++y)
      for (int k = 0; k < 4; ++k) t2[4 * y + k] = f16_bits(cb2.c[(y >> (2 * k)) & 3]);
    for (int y = 0; y < 16; ++y)
      for (int k = 0; k < 4; ++k) t1[4 * y + k] = f16_bits(cb1.c[(y >> k) & 1]);
    for (int y = 0; y < 64; ++y)
      for (int k = 0; k < 2; ++k) t3[2 * y + k] = f16_bits(cb3.c[(y >> (3 * k)) & 7]);
  }
  std::memcpy(img + hd.off_vlut, vlut.data(), 4 * vlut.size());
  double *r64v = (double *)(img + hd.off_rot64_v);
  float *r32v = (float *)(img + hd.off_rot32_v);
  for (int h = 0; h < hkv; ++h) {
    const std::vector<double> &pi = p.rot_v[h];
    const size_t base = (size_t)h * kHeadDim * kHeadDim;
    for (int i = 0; i < kHeadDim; ++i)
      for (int k = 0; k < kHeadDim; ++k) {
        r64v[base + (size_t)k * kHeadDim + i] = pi[(size_t)i * kHeadDim + k];
        r32v[base + (size_t)k * kHeadDim + i] = (float)pi[(size_t)i * kHeadDim + k];
      }
  }
  return BGTQ_OK;
}

}  // namespace bgtq
