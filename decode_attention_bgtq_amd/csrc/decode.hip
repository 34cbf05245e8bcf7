// Fused decode attention over the packed Block-GTQ cache on gfx950 (the
// packed-cache serving path of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", Abstract, and of the Block-GTQ README backend table).
//
// Two launches per call:
//  stream  one workgroup per (split of the sequence, KV head, sequence).
//          Prologue: rotates the G queries of the KV head once per key width
//          group with fp32 MFMA (the only matrix-core use) and builds in LDS,
//          per lookup chunk of the key stream, a table of
//          scale * sum_r q_rot[h][pos + r] * centroid_w[code_r] / sqrt(d_g) over
//          every value of the chunk's stream window.  Per 64-token tile: lane =
//          token reads the key words (coalesced, word-major) and sums table
//          entries times group norms into log2-domain logits; online softmax
//          with wavefront reductions; lane = value coordinate accumulates fp16
//          (p * value norm) token pairs against fp16 centroid pairs from an LDS
//          table (v_dot2, fp32 accumulate) in the rotated value space.  Writes
//          one partial (m, l, acc) per split and query head.
//  merge   one workgroup per (sequence, KV head): log-sum-exp merge of the
//          splits, normalisation, un-rotation by Pi_V^T, fp16 output.
#include "device.h"
#include "host.h"

namespace bgtq {

constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kPartStride = 132;  // m, l, pad, pad, acc[128]
constexpr int kMaxSplits = 256;

typedef float f4v __attribute__((ext_vector_type(4)));

// LDS access by raw byte offset.  The stream kernel has no static LDS, so its
// dynamic allocation starts at offset 0 (checked on the host before launch).
template <typename T>
__device__ __forceinline__ T lds_at(uint32_t off) {
  typedef uint32_t u2v __attribute__((ext_vector_type(2)));
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, *(const __attribute__((address_space(3))) uint32_t *)(size_t)off);
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, *(const __attribute__((address_space(3))) u2v *)(size_t)off);
  } else {
    static_assert(sizeof(T) == 16, "LDS reads of 4, 8 or 16 bytes");
    return __builtin_bit_cast(T, *(const __attribute__((address_space(3))) u4v *)(size_t)off);
  }
}

// q_rot[h][pos_g + i] = sum_k Pi_g[i][k] q[h][coord_g[k]] for the key groups of
// one KV head; qin [G][128] natural order, qs [G][128] group order (zeroed by
// the caller past d_nz).  16x16x4 fp32 MFMA tiles, the G heads as columns;
// `waves` waves of the workgroup share the row tiles.
__device__ __forceinline__ void rotate_queries(const ConstHeader *hd, const KvhDesc *kd, int G,
                                               const float *qin, float *qs, int wave, int waves,
                                               int lane) {
  for (int gi = 0; gi < kd->n_groups; ++gi) {
    const KGroupDesc g = kd->g[gi];
    const float *pi = (const float *)((const uint8_t *)hd + hd->off_rot32_k) + g.rot32;
    const int n = lane & 15, kq = lane >> 4;
    for (int i0 = 16 * wave; i0 < g.d; i0 += 16 * waves) {
      f4v acc = {0.f, 0.f, 0.f, 0.f};
      const int ia = i0 + n;
      const int ic = ia < g.d ? ia : g.d - 1;
#pragma unroll 8
      for (int k0 = 0; k0 < g.d; k0 += 4) {
        const int kk = k0 + kq;
        const int kcl = kk < g.d ? kk : g.d - 1;
        const float a0 = pi[(size_t)ic * g.d + kcl];
        const float b0 = qin[(n & 7) * kHeadDim + kd->coord[g.pos + kcl]];
        const float a = (ia < g.d && kk < g.d) ? a0 : 0.f;
        const float bv = (kk < g.d && n < G) ? b0 : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * kq + r;
        if (i < g.d && n < G) qs[n * kHeadDim + g.pos + i] = acc[r];
      }
    }
  }
}

// Rotated queries only (the bgtq_rotate_queries entry point): one workgroup
// per (KV head, sequence).
__global__ __launch_bounds__(256) void qrot_kernel(const uint8_t *__restrict__ consts,
                                                   const uint16_t *__restrict__ q, float *__restrict__ qrot) {
  __shared__ float qs[8 * kHeadDim];
  __shared__ float qin[8 * kHeadDim];
  const ConstHeader *hd = hdr_of(consts);
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = hd->group, hq = hd->n_q_heads;
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int tid = threadIdx.x;
  const uint16_t *qb = q + ((size_t)b * hq + (size_t)kvh * G) * kHeadDim;
  const int nq = G * kHeadDim;
  for (int i = tid; i < 8 * kHeadDim; i += 256) {
    qs[i] = 0.f;
    qin[i] = i < nq ? h2f(qb[i]) : 0.f;
  }
  __syncthreads();
  rotate_queries(hd, kd, G, qin, qs, tid >> 6, 4, tid & 63);
  __syncthreads();
  for (int idx = tid; idx < nq; idx += 256) qrot[((size_t)b * hq + (size_t)kvh * G) * kHeadDim + idx] = qs[idx];
}

// ------------------------------------------------------------------ stream

struct StreamSmem {
  int vlut, pbuf, scratch, total;
};

// LDS layout: [key tables | wave merge area] [value table] [P pairs per wave]
//             [prologue scratch: qin, qs (G x 128 floats each), build words]
template <int G, int VB>
__host__ __device__ constexpr StreamSmem stream_layout(int table_bytes) {
  StreamSmem s{};
  const int merge = kStreamWaves * G * kPartStride * 4;
  int r0 = table_bytes > merge ? table_bytes : merge;
  r0 = (r0 + 15) & ~15;
  s.vlut = r0;
  s.pbuf = s.vlut + VLut<VB>::entries * VLut<VB>::bytes;
  s.scratch = s.pbuf + kStreamWaves * 32 * G * 4;
  s.total = s.scratch + 2 * G * kHeadDim * 4 + kMaxChunks * 4;
  return s;
}

template <int VB, int WK>
struct TileRegs {
  uint32_t w[WK];
  uint2 nr;
  uint32_t nv;
  uint32_t va[2 * VB], vb[2 * VB];
};

// All loads unconditional (addresses clamped into valid memory, unused words
// zeroed afterwards) so that the compiler can count outstanding loads across
// the software pipeline.  kc / wkl are the key words and their count, or the
// norm array and 1 for zero-bit keys.  `base` is wave-uniform.
template <int VB, int WK>
__device__ __forceinline__ void load_tile(TileRegs<VB, WK> &r, const uint32_t *__restrict__ kc,
                                          const uint16_t *__restrict__ kn, const uint32_t *__restrict__ vc,
                                          const uint16_t *__restrict__ vn, size_t base, int wk, int wkl,
                                          int lane) {
  const uint32_t *kt = kc + base * wkl * kTile;
#pragma unroll
  for (int j = 0; j < WK; ++j) {
    const uint32_t v = kt[(size_t)min(j, wkl - 1) * kTile + lane];
    r.w[j] = j < wk ? v : 0u;
  }
  r.nr = *(const uint2 *)(kn + base * kTile * 4 + lane * 4);
  r.nv = vn[base * kTile + lane];
  const uint32_t *vt = vc + base * kHeadDim * (2 * VB);
  const uint32_t *p0 = vt + lane * (2 * VB);
  const uint32_t *p1 = p0 + 64 * (2 * VB);
  if constexpr (VB == 1) {
    const uint2 a = *(const uint2 *)p0, c = *(const uint2 *)p1;
    r.va[0] = a.x, r.va[1] = a.y, r.vb[0] = c.x, r.vb[1] = c.y;
  } else if constexpr (VB == 2) {
    const uint4 a = *(const uint4 *)p0, c = *(const uint4 *)p1;
    r.va[0] = a.x, r.va[1] = a.y, r.va[2] = a.z, r.va[3] = a.w;
    r.vb[0] = c.x, r.vb[1] = c.y, r.vb[2] = c.z, r.vb[3] = c.w;
  } else if constexpr (VB == 3) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const uint2 a = *(const uint2 *)(p0 + 2 * k), c = *(const uint2 *)(p1 + 2 * k);
      r.va[2 * k] = a.x, r.va[2 * k + 1] = a.y, r.vb[2 * k] = c.x, r.vb[2 * k + 1] = c.y;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 a = *(const uint4 *)(p0 + 4 * k), c = *(const uint4 *)(p1 + 4 * k);
      r.va[4 * k] = a.x, r.va[4 * k + 1] = a.y, r.va[4 * k + 2] = a.z, r.va[4 * k + 3] = a.w;
      r.vb[4 * k] = c.x, r.vb[4 * k + 1] = c.y, r.vb[4 * k + 2] = c.z, r.vb[4 * k + 3] = c.w;
    }
  }
}

template <int G>
__device__ __forceinline__ void lds_entry(uint32_t a, float (&t)[G]) {
  if constexpr (G == 1) {
    t[0] = lds_at<float>(a);
  } else if constexpr (G == 2) {
    const float2 v = lds_at<float2>(a);
    t[0] = v.x, t[1] = v.y;
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const float4 v = lds_at<float4>(a + 16 * q4);
      t[4 * q4 + 0] = v.x, t[4 * q4 + 1] = v.y, t[4 * q4 + 2] = v.z, t[4 * q4 + 3] = v.w;
    }
  }
}

template <int G>
__device__ __forceinline__ void lds_pairs(uint32_t a, uint32_t (&o)[G]) {
  if constexpr (G == 1) {
    o[0] = lds_at<uint32_t>(a);
  } else if constexpr (G == 2) {
    const uint2 v = lds_at<uint2>(a);
    o[0] = v.x, o[1] = v.y;
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const uint4 v = lds_at<uint4>(a + 16 * q4);
      o[4 * q4 + 0] = v.x, o[4 * q4 + 1] = v.y, o[4 * q4 + 2] = v.z, o[4 * q4 + 3] = v.w;
    }
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// acc0/acc1[h] += <p' pair of head h, centroid pair> for token pair `pair`
template <int G>
__device__ __forceinline__ void pair_accum(uint32_t pbuf, int pair, uint32_t c0, uint32_t c1,
                                           float (&acc0)[G], float (&acc1)[G]) {
  uint32_t pv[G];
  lds_pairs<G>(pbuf + pair * G * 4, pv);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc0[h] = dot2(pv[h], c0, acc0[h]);
    acc1[h] = dot2(pv[h], c1, acc1[h]);
  }
}

struct StreamState {
  uint32_t dv0, dv1;  // lane l: lookup descriptor of chunk l (dv0) and l + 64 (dv1)
  uint32_t av;        // lane jj: first chunk anchored at key word jj-1
  uint32_t fmask;     // window mask shifted to the entry offset (held in a VGPR)
  int wk;
  int64_t seq;
};

// One key chunk: funnel-shift the window out of (hi, lo), look up the table
// entry of every head, accumulate norm * entry.
template <int G>
__device__ __forceinline__ void key_chunk(uint32_t dsc, uint32_t hi, uint32_t lo, uint32_t fmask,
                                          const float (&nf)[4], float &ncur, float (&lg)[G]) {
  if (dsc & kChunkStart) {
    const uint32_t slot = (dsc >> 24) & 3;
    ncur = slot == 0 ? nf[0] : slot == 1 ? nf[1] : slot == 2 ? nf[2] : nf[3];
  }
  const uint32_t t = __builtin_amdgcn_alignbit(hi, lo, dsc);
  float tv[G];
  lds_entry<G>((t & fmask) | (dsc & kChunkTableMask), tv);
#pragma unroll
  for (int h = 0; h < G; ++h) lg[h] = fmaf(ncur, tv[h], lg[h]);
}

template <int G, int VB, int WK>
__device__ __forceinline__ void process_tile(const TileRegs<VB, WK> &r, int tile, const StreamState &st,
                                             uint32_t vlut, uint32_t pbuf, float (&mrun)[G], float (&lsum)[G],
                                             float (&acc0)[G], float (&acc1)[G], int lane) {
  // ---- keys: lane = token; log2-domain logits from the chunk tables
  const float nf[4] = {h2f((uint16_t)(r.nr.x & 0xFFFF)), h2f((uint16_t)(r.nr.x >> 16)),
                       h2f((uint16_t)(r.nr.y & 0xFFFF)), h2f((uint16_t)(r.nr.y >> 16))};
  float lg[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lg[h] = 0.f;
  float ncur = 0.f;
#pragma unroll
  for (int jj = 0; jj <= WK; ++jj) {
    if (jj <= st.wk) {
      const uint32_t lo = jj ? r.w[jj - 1] : 0u, hi = jj < WK ? r.w[jj] : 0u;
      const int c0 = __builtin_amdgcn_readlane((int)st.av, jj);
      const int c1 = __builtin_amdgcn_readlane((int)st.av, jj + 1);
      const int m1 = c1 < 64 ? c1 : 64;
      for (int c = c0; c < m1; ++c)
        key_chunk<G>((uint32_t)__builtin_amdgcn_readlane((int)st.dv0, c), hi, lo, st.fmask, nf, ncur, lg);
      for (int c = c0 > 64 ? c0 : 64; c < c1; ++c)
        key_chunk<G>((uint32_t)__builtin_amdgcn_readlane((int)st.dv1, c - 64), hi, lo, st.fmask, nf, ncur, lg);
    }
  }
  const bool valid = (int64_t)tile * kTile + lane < st.seq;
  const float nv = h2f((uint16_t)r.nv);
  float alpha[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = valid ? lg[h] : -INFINITY;
    const float mn = fmaxf(mrun[h], wave_max(l));
    alpha[h] = __builtin_amdgcn_exp2f(mrun[h] - mn);
    const float p = __builtin_amdgcn_exp2f(l - mn);
    lsum[h] = fmaf(lsum[h], alpha[h], p);
    mrun[h] = mn;
    *(__attribute__((address_space(3))) _Float16 *)(size_t)(pbuf + ((lane >> 1) * G + h) * 4 + (lane & 1) * 2) =
        (_Float16)(p * nv);
  }
  wave_sync_lds();
  // ---- values: lane = coordinates lane and lane + 64
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc0[h] *= alpha[h];
    acc1[h] *= alpha[h];
  }
  if constexpr (VB == 3) {
#pragma unroll
    for (int y = 0; y < 32; ++y) {
      const int bit = 6 * y, wi = bit >> 5, sh = bit & 31;
      uint32_t s0, s1;
      if (sh <= 26) {
        s0 = (r.va[wi] >> sh) & 63u;
        s1 = (r.vb[wi] >> sh) & 63u;
      } else {
        s0 = __builtin_amdgcn_alignbit(r.va[wi + 1], r.va[wi], sh) & 63u;
        s1 = __builtin_amdgcn_alignbit(r.vb[wi + 1], r.vb[wi], sh) & 63u;
      }
      pair_accum<G>(pbuf, y, lds_at<uint32_t>(vlut + 4 * s0), lds_at<uint32_t>(vlut + 4 * s1), acc0, acc1);
    }
  } else if constexpr (VB == 4) {
#pragma unroll
    for (int y = 0; y < 32; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      pair_accum<G>(pbuf, y, lds_at<uint32_t>(vlut + 4 * s0), lds_at<uint32_t>(vlut + 4 * s1), acc0, acc1);
    }
  } else if constexpr (VB == 2) {
#pragma unroll
    for (int y = 0; y < 16; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint2 e0 = lds_at<uint2>(vlut + 8 * s0), e1 = lds_at<uint2>(vlut + 8 * s1);
      pair_accum<G>(pbuf, 2 * y, e0.x, e1.x, acc0, acc1);
      pair_accum<G>(pbuf, 2 * y + 1, e0.y, e1.y, acc0, acc1);
    }
  } else {
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint4 e0 = lds_at<uint4>(vlut + 16 * s0), e1 = lds_at<uint4>(vlut + 16 * s1);
      pair_accum<G>(pbuf, 4 * y + 0, e0.x, e1.x, acc0, acc1);
      pair_accum<G>(pbuf, 4 * y + 1, e0.y, e1.y, acc0, acc1);
      pair_accum<G>(pbuf, 4 * y + 2, e0.z, e1.z, acc0, acc1);
      pair_accum<G>(pbuf, 4 * y + 3, e0.w, e1.w, acc0, acc1);
    }
  }
  wave_sync_lds();
}

template <int G, int VB, int WK>
__global__ __launch_bounds__(kStreamThreads) void decode_stream_kernel(
    const uint8_t *__restrict__ consts, const uint16_t *__restrict__ q, const uint32_t *__restrict__ kc,
    const uint16_t *__restrict__ kn, const uint32_t *__restrict__ vc, const uint16_t *__restrict__ vn,
    int64_t tiles_cap, const int32_t *__restrict__ seq_lens, int64_t max_seq_len, int tiles_per_split,
    float kscale, float *__restrict__ part, int n_splits) {
  constexpr int L = GLog<G>::v;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const ConstHeader *hd = hdr_of(consts);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hkv = hd->n_kv_heads, hq = hd->n_q_heads;
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int win = hd->lut_window;
  const int nch = kd->n_chunks;
  const StreamSmem sm = stream_layout<G, VB>(hd->max_chunks << (win + L));
  const uint32_t pbuf = (uint32_t)(sm.pbuf + wave * 32 * G * 4);

  // ---- prologue: rotated queries and key lookup tables of this head
  {
    float *qin = (float *)(smem + sm.scratch);
    float *qs = qin + G * kHeadDim;
    uint32_t *bld = (uint32_t *)(qs + G * kHeadDim);
    const uint16_t *qb = q + ((size_t)b * hq + (size_t)kvh * G) * kHeadDim;
    for (int i = tid; i < G * kHeadDim; i += kStreamThreads) {
      qin[i] = h2f(qb[i]);
      qs[i] = 0.f;
    }
    const uint32_t *bsrc = (const uint32_t *)(consts + hd->off_build) + kd->chunk_base;
    if (tid < nch) bld[tid] = bsrc[tid];
    __syncthreads();
    rotate_queries(hd, kd, G, qin, qs, wave, kStreamWaves, lane);
    __syncthreads();
    const int ne = 1 << win;
    float *tab = (float *)smem;
    for (int idx = tid; idx < nch * ne * G; idx += kStreamThreads) {
      const int h = idx % G, f = (idx / G) % ne, c = idx / (G * ne);
      const uint32_t bw = bld[c];
      const int pos = bw & 255, m = (bw >> 8) & 15, w = (bw >> 12) & 7, gi = (bw >> 15) & 3;
      float s = 0.f;
      for (int r = 0; r < m; ++r)
        s = fmaf(qs[h * kHeadDim + pos + r], (float)hd->cent[w - 1][(f >> (w * r)) & ((1 << w) - 1)], s);
      tab[idx] = kscale / sqrtf((float)kd->g[gi].d) * s;
    }
  }
  // value table: fp16 centroid pairs for the tokens of one code chunk
  {
    uint16_t c16[1 << VB];
#pragma unroll
    for (int k = 0; k < (1 << VB); ++k) c16[k] = f64_to_f16(hd->cent[VB - 1][k]);
    uint32_t *vl = (uint32_t *)(smem + sm.vlut);
    for (int y = tid; y < VLut<VB>::entries; y += kStreamThreads) {
      if constexpr (VB == 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          vl[4 * y + u] = (uint32_t)c16[(y >> (2 * u)) & 1] | ((uint32_t)c16[(y >> (2 * u + 1)) & 1] << 16);
      } else if constexpr (VB == 2) {
        vl[2 * y + 0] = (uint32_t)c16[y & 3] | ((uint32_t)c16[(y >> 2) & 3] << 16);
        vl[2 * y + 1] = (uint32_t)c16[(y >> 4) & 3] | ((uint32_t)c16[(y >> 6) & 3] << 16);
      } else if constexpr (VB == 3) {
        vl[y] = (uint32_t)c16[y & 7] | ((uint32_t)c16[(y >> 3) & 7] << 16);
      } else {
        vl[y] = (uint32_t)c16[y & 15] | ((uint32_t)c16[(y >> 4) & 15] << 16);
      }
    }
  }
  StreamState st;
  {
    int64_t s = seq_lens[b];
    st.seq = s < 0 ? 0 : (s > max_seq_len ? max_seq_len : s);
    const uint32_t *lk = (const uint32_t *)(consts + hd->off_lookup) + kd->chunk_base;
    st.dv0 = lane < nch ? lk[lane] : 0u;
    st.dv1 = lane + 64 < nch ? lk[lane + 64] : 0u;
    st.av = lane <= kMaxWK + 1 ? (uint32_t)kd->anchor[lane] : 0u;
    st.fmask = (uint32_t)__builtin_amdgcn_mov_dpp((int)(((1u << win) - 1) << L), 0xE4, 0xF, 0xF, false);
    st.wk = hd->wk;
  }
  __syncthreads();

  const int ntile = (int)((st.seq + kTile - 1) / kTile);
  const int tile_lo = split * tiles_per_split;
  const int tile_hi = min(tile_lo + tiles_per_split, ntile);
  float mrun[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mrun[h] = -INFINITY, lsum[h] = 0.f, acc0[h] = 0.f, acc1[h] = 0.f;

  const size_t head_base = ((size_t)b * hkv + kvh) * (size_t)tiles_cap;
  const uint32_t *ksrc = st.wk ? kc : (const uint32_t *)kn;
  const int wkl = st.wk ? st.wk : 1;
  const uint32_t vlut = (uint32_t)sm.vlut;
  TileRegs<VB, WK> ra, rb;
  int tile = tile_lo + wave;
  if (tile < tile_hi) {
    load_tile(ra, ksrc, kn, vc, vn, head_base + tile, st.wk, wkl, lane);
    for (;;) {
      load_tile(rb, ksrc, kn, vc, vn, head_base + min(tile + kStreamWaves, tile_hi - 1), st.wk, wkl, lane);
      process_tile<G, VB, WK>(ra, tile, st, vlut, pbuf, mrun, lsum, acc0, acc1, lane);
      tile += kStreamWaves;
      if (tile >= tile_hi) break;
      load_tile(ra, ksrc, kn, vc, vn, head_base + min(tile + kStreamWaves, tile_hi - 1), st.wk, wkl, lane);
      process_tile<G, VB, WK>(rb, tile, st, vlut, pbuf, mrun, lsum, acc0, acc1, lane);
      tile += kStreamWaves;
      if (tile >= tile_hi) break;
    }
  }

  // ---- merge the waves of this split into one partial per query head
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = wave_sum(lsum[h]);
  __syncthreads();
  float *mrg = (float *)smem;  // [waves][G][kPartStride]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float *rr = mrg + (wave * G + h) * kPartStride;
    if (lane == 0) rr[0] = mrun[h], rr[1] = lsum[h];
    rr[4 + lane] = acc0[h];
    rr[4 + 64 + lane] = acc1[h];
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += kStreamThreads) {
    const int h = idx / kHeadDim, i = idx % kHeadDim;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) mx = fmaxf(mx, mrg[(w * G + h) * kPartStride]);
    float s = 0.f, l = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kStreamWaves; ++w) {
        const float *rr = mrg + (w * G + h) * kPartStride;
        const float f = __builtin_amdgcn_exp2f(rr[0] - mx);
        s = fmaf(f, rr[4 + i], s);
        l = fmaf(f, rr[1], l);
      }
    }
    float *o = part + (((size_t)b * hq + (size_t)kvh * G + h) * n_splits + split) * kPartStride;
    o[4 + i] = s;
    if (i == 0) o[0] = mx, o[1] = l;
  }
}

// One workgroup per (sequence, KV head): log-sum-exp merge of the splits of
// its G query heads, normalisation and un-rotation by Pi_V^T, fp16 output.
__global__ __launch_bounds__(kStreamThreads) void merge_kernel(const uint8_t *__restrict__ consts,
                                                             const float *__restrict__ part, int n_splits,
                                                             uint16_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) float ws_s[8 * kMaxSplits];
  __shared__ float ls_s[8 * kMaxSplits];
  __shared__ __attribute__((aligned(16))) float ys[8 * kHeadDim];
  const ConstHeader *hd = hdr_of(consts);
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = hd->group, hq = hd->n_q_heads;
  const int gs = G * n_splits;
  const size_t pbase = ((size_t)b * hq + (size_t)kvh * G) * n_splits;
  for (int idx = tid; idx < gs; idx += kStreamThreads) {
    const float2 ml = *(const float2 *)(part + (pbase + idx) * kPartStride);
    ws_s[idx] = ml.x;
    ls_s[idx] = ml.y;
  }
  __syncthreads();
  if (tid < G) {  // per head: max, then weights exp2(m_s - M) / (L sqrt(128))
    float mx = -INFINITY;
    for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ws_s[tid * n_splits + s]);
    float l = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float f = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ws_s[tid * n_splits + s] - mx);
      ws_s[tid * n_splits + s] = f;
      l = fmaf(f, ls_s[tid * n_splits + s], l);
    }
    const float inv = l > 0.f ? 1.0f / (l * sqrtf((float)kHeadDim)) : 0.f;
    for (int s = 0; s < n_splits; ++s) ws_s[tid * n_splits + s] *= inv;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += kStreamThreads) {
    const int h = idx / kHeadDim, i = idx % kHeadDim;
    const float *p = part + (pbase + (size_t)h * n_splits) * kPartStride + 4 + i;
    const float *wv = ws_s + h * n_splits;
    float a = 0.f;
#pragma unroll 16
    for (int s = 0; s < n_splits; ++s) a = fmaf(wv[s], p[(size_t)s * kPartStride], a);
    ys[idx] = a;
  }
  __syncthreads();
  const float *pvt = (const float *)(consts + hd->off_rot32_v) + (size_t)kvh * kHeadDim * kHeadDim;
  for (int idx = tid; idx < G * kHeadDim; idx += kStreamThreads) {
    const int h = idx / kHeadDim, j = idx % kHeadDim;
    const float4 *row = (const float4 *)(pvt + (size_t)j * kHeadDim);  // Pi_V[k][j], k = 0..127
    const float4 *yv = (const float4 *)(ys + h * kHeadDim);
    float o = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < kHeadDim / 4; ++k4) {
      const float4 pv = row[k4], y4 = yv[k4];
      o = fmaf(pv.x, y4.x, o);
      o = fmaf(pv.y, y4.y, o);
      o = fmaf(pv.z, y4.z, o);
      o = fmaf(pv.w, y4.w, o);
    }
    out[((size_t)b * hq + (size_t)kvh * G + h) * kHeadDim + j] = __builtin_bit_cast(uint16_t, (_Float16)o);
  }
}

// ------------------------------------------------------------------ host

typedef void (*stream_fn)(const uint8_t *, const uint16_t *, const uint32_t *, const uint16_t *, const uint32_t *,
                          const uint16_t *, int64_t, const int32_t *, int64_t, int, float, float *, int);

template <int G, int VB>
stream_fn pick_wk(int wk) {
  if (wk <= 8) return decode_stream_kernel<G, VB, 8>;
  if (wk <= 12) return decode_stream_kernel<G, VB, 12>;
  return decode_stream_kernel<G, VB, 16>;
}

template <int G>
stream_fn pick_vb(int vb, int wk) {
  switch (vb) {
    case 1: return pick_wk<G, 1>(wk);
    case 2: return pick_wk<G, 2>(wk);
    case 3: return pick_wk<G, 3>(wk);
    default: return pick_wk<G, 4>(wk);
  }
}

stream_fn pick_stream(int g, int vb, int wk) {
  switch (g) {
    case 1: return pick_vb<1>(vb, wk);
    case 2: return pick_vb<2>(vb, wk);
    case 4: return pick_vb<4>(vb, wk);
    default: return pick_vb<8>(vb, wk);
  }
}

int stream_smem_bytes(int g, int vb, int table_bytes) {
#define BGTQ_SM(G_, VB_) \
  if (g == G_ && vb == VB_) return stream_layout<G_, VB_>(table_bytes).total;
  BGTQ_SM(1, 1) BGTQ_SM(1, 2) BGTQ_SM(1, 3) BGTQ_SM(1, 4)
  BGTQ_SM(2, 1) BGTQ_SM(2, 2) BGTQ_SM(2, 3) BGTQ_SM(2, 4)
  BGTQ_SM(4, 1) BGTQ_SM(4, 2) BGTQ_SM(4, 3) BGTQ_SM(4, 4)
  BGTQ_SM(8, 1) BGTQ_SM(8, 2) BGTQ_SM(8, 3) BGTQ_SM(8, 4)
#undef BGTQ_SM
  return -1;
}

struct DecodeLayout {
  int n_splits, tiles_per_split;
  size_t total;  // workspace bytes (split partials)
};

DecodeLayout decode_layout(const Plan &p, int batch, int64_t max_seq_len) {
  DecodeLayout d{};
  const int tiles = (int)((max_seq_len + kTile - 1) / kTile);
  const int hkv = p.desc.n_kv_heads, hq = p.desc.n_q_heads;
  const int target = 2 * device_cus();
  int s = (target + batch * hkv - 1) / (batch * hkv);
  s = std::max(1, std::min({s, (tiles + 2 * kStreamWaves - 1) / (2 * kStreamWaves), kMaxSplits}));
  const int tps = (tiles + s - 1) / s;
  d.n_splits = (tiles + tps - 1) / tps;
  d.tiles_per_split = tps;
  d.total = (((size_t)batch * hq * d.n_splits * kPartStride * 4) + 255) & ~(size_t)255;
  return d;
}

// The stream kernels address LDS from offset 0: they must have no static LDS.
bool stream_static_lds_ok(stream_fn fn) {
  static std::mutex mu;
  static std::vector<stream_fn> checked;
  std::lock_guard<std::mutex> lk(mu);
  for (stream_fn f : checked)
    if (f == fn) return true;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, (const void *)fn) != hipSuccess || attr.sharedSizeBytes != 0) return false;
  checked.push_back(fn);
  return true;
}

}  // namespace bgtq

using namespace bgtq;

extern "C" {

bgtq_status bgtq_rotate_queries(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q, int32_t batch,
                                float *q_rot, bgtq_stream stream) {
  if (!plan || !dev_consts || !q || !q_rot) return fail(BGTQ_EINVAL, "bgtq_rotate_queries: null pointer");
  if (batch < 1 || batch > 65535) return fail(BGTQ_EINVAL, "bgtq_rotate_queries: batch must be 1..65535");
  const dim3 grid(plan->p.desc.n_kv_heads, batch);
  qrot_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const uint8_t *)dev_consts, q, q_rot);
  return launch_status("bgtq_rotate_queries");
}

bgtq_status bgtq_decode_workspace_size(const bgtq_plan *plan, int32_t batch, int64_t max_seq_len, size_t *bytes) {
  if (!plan || !bytes) return fail(BGTQ_EINVAL, "bgtq_decode_workspace_size: null pointer");
  if (batch < 1 || max_seq_len < 1) return fail(BGTQ_EINVAL, "bgtq_decode_workspace_size: batch, max_seq_len >= 1");
  *bytes = decode_layout(plan->p, batch, max_seq_len).total;
  return BGTQ_OK;
}

bgtq_status bgtq_decode_attn(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                             const uint32_t *k_codes, const uint16_t *k_norms, const uint32_t *v_codes,
                             const uint16_t *v_norms, int64_t capacity, const int32_t *seq_lens, int32_t batch,
                             int64_t max_seq_len, float softmax_scale, uint16_t *out, void *workspace,
                             size_t ws_bytes, bgtq_stream stream) {
  if (!plan || !dev_consts || !q || !k_norms || !v_codes || !v_norms || !seq_lens || !out || !workspace ||
      (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, "bgtq_decode_attn: null pointer");
  if (batch < 1 || batch > 65535) return fail(BGTQ_EINVAL, "bgtq_decode_attn: batch must be 1..65535");
  if (max_seq_len < 1 || max_seq_len > capacity)
    return fail(BGTQ_ECAPACITY, "bgtq_decode_attn: max_seq_len must be in [1, capacity]");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(BGTQ_EINVAL, "bgtq_decode_attn: softmax_scale must be positive and finite");
  if ((uintptr_t)workspace & 255) return fail(BGTQ_EINVAL, "bgtq_decode_attn: workspace must be 256-byte aligned");
  const Plan &p = plan->p;
  const DecodeLayout lay = decode_layout(p, batch, max_seq_len);
  if (ws_bytes < lay.total) return fail(BGTQ_EWORKSPACE, "bgtq_decode_attn: workspace too small");
  const int G = p.hdr.group, vb = p.hdr.v_bits;
  const int table_bytes = p.hdr.max_chunks << (p.hdr.lut_window + p.hdr.lut_entry_log2);
  const int smem = stream_smem_bytes(G, vb, table_bytes);
  stream_fn fn = pick_stream(G, vb, p.hdr.wk);
  if (!stream_static_lds_ok(fn)) return fail(BGTQ_EDEVICE, "bgtq_decode_attn: stream kernel has static LDS");
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return fail(BGTQ_EDEVICE, "bgtq_decode_attn: lookup tables exceed the LDS limit");
  }
  hipStream_t st = (hipStream_t)stream;
  float *part = (float *)workspace;
  const int64_t tiles_cap = (capacity + kTile - 1) / kTile;
  const float kscale = softmax_scale * 1.4426950408889634f;  // logits in log2 units
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    Prof &pr = prof();
    std::lock_guard<std::mutex> lk(pr.mu);
    if (pr.on) {
      if (!pr.pool.empty()) {
        e0 = pr.pool.back().first;
        e1 = pr.pool.back().second;
        pr.pool.pop_back();
      } else if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        return fail(BGTQ_EDEVICE, "bgtq_decode_attn: event creation failed");
      }
    }
  }
  if (e0) (void)hipEventRecord(e0, st);
  const dim3 grid(lay.n_splits, p.desc.n_kv_heads, batch);
  fn<<<grid, kStreamThreads, smem, st>>>((const uint8_t *)dev_consts, q, k_codes, k_norms, v_codes, v_norms,
                                         tiles_cap, seq_lens, max_seq_len, lay.tiles_per_split, kscale, part,
                                         lay.n_splits);
  bgtq_status s = launch_status("bgtq_decode_attn (stream)");
  if (e1) {
    (void)hipEventRecord(e1, st);
    Prof &pr = prof();
    std::lock_guard<std::mutex> lk(pr.mu);
    pr.pending.emplace_back(e0, e1);
  }
  if (s != BGTQ_OK) return s;
  merge_kernel<<<dim3(p.desc.n_kv_heads, batch), kStreamThreads, 0, st>>>((const uint8_t *)dev_consts, part,
                                                                         lay.n_splits, out);
  return launch_status("bgtq_decode_attn (merge)");
}

}  // extern "C"
