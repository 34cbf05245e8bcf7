// Fused decode attention over the packed Block-GTQ cache on gfx950 (the
// packed-cache serving path of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", Abstract, and of the Block-GTQ README backend table).
//
// Two launches per call:
//  prep    one workgroup per (sequence, KV head): rotates the G queries of the
//          KV head once per key width group with fp32 MFMA (the only matrix-core
//          use) and builds, per lookup chunk of the key stream, a table of
//          scale * sum_r q_rot[h][pos + r] * centroid_w[code_r] / sqrt(d_g) for
//          every value of the chunk's stream window;
//  stream  one workgroup per (split of the sequence, KV head, sequence): copies
//          the tables to LDS; per 64-token tile, lane = token reads the key words
//          (coalesced, word-major) and sums table entries times group norms into
//          log2-domain logits; online softmax with wavefront reductions; lane =
//          value coordinate accumulates fp16 (p * value norm) pairs against fp16
//          centroid pairs from an LDS table (v_dot2, fp32 accumulate) in the
//          rotated value space.  The last workgroup of a (sequence, KV head)
//          merges the splits (log-sum-exp), normalises, un-rotates by Pi_V^T and
//          writes fp16.
#include "device.h"
#include "host.h"

namespace bgtq {

constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kPartStride = 132;  // m, l, pad, pad, acc[128]

// ------------------------------------------------------------------ prep

__global__ __launch_bounds__(256) void prep_kernel(const uint8_t *__restrict__ consts,
                                                   const uint16_t *__restrict__ q, float *__restrict__ qrot,
                                                   float *__restrict__ tables, uint32_t *__restrict__ counters,
                                                   float kscale, int tbl_stride, int build_tables) {
  __shared__ float qs[8][kHeadDim];    // rotated queries, group order
  __shared__ float qin[8][kHeadDim];   // input queries, natural order
  __shared__ float cent[4][16];
  __shared__ uint32_t bld_s[kMaxChunks];
  __shared__ float kap_s[kMaxGroups];
  const ConstHeader *hd = hdr_of(consts);
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = hd->group, hq = hd->n_q_heads, hkv = hd->n_kv_heads;
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nch = kd->n_chunks;
  for (int i = tid; i < 8 * kHeadDim; i += 256) {
    (&qs[0][0])[i] = 0.f;
    const int h = i / kHeadDim;
    (&qin[0][0])[i] = h < G ? h2f(q[((size_t)b * hq + (size_t)kvh * G) * kHeadDim + i]) : 0.f;
  }
  if (tid < 64) cent[tid >> 4][tid & 15] = (float)hd->cent[tid >> 4][tid & 15];
  if (tid < nch) bld_s[tid] = ((const uint32_t *)(consts + hd->off_build))[kd->chunk_base + tid];
  if (tid < kd->n_groups) kap_s[tid] = kscale / sqrtf((float)kd->g[tid].d);
  __syncthreads();

  // q_rot = Pi_g q[coords of g] for every group, the G query heads as MFMA columns
  typedef float f4 __attribute__((ext_vector_type(4)));
  for (int gi = 0; gi < kd->n_groups; ++gi) {
    const KGroupDesc g = kd->g[gi];
    const float *pi = (const float *)(consts + hd->off_rot32_k) + g.rot32;
    const int n = lane & 15, kq = lane >> 4;
    for (int i0 = 16 * wave; i0 < g.d; i0 += 64) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      const int ia = i0 + n;
#pragma unroll 8
      for (int k0 = 0; k0 < g.d; k0 += 4) {
        const int kk = k0 + kq;
        const float a = (ia < g.d && kk < g.d) ? pi[(size_t)ia * g.d + kk] : 0.f;
        const float bv = (kk < g.d && n < G) ? qin[n][kd->coord[g.pos + kk]] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * kq + r;
        if (i < g.d && n < G) qs[n][g.pos + i] = acc[r];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += 256)
    qrot[((size_t)b * hq + (size_t)kvh * G) * kHeadDim + idx] = qs[idx / kHeadDim][idx % kHeadDim];
  if (!build_tables) return;

  // key lookup tables of this (sequence, KV head): [chunk][window value][head]
  const int ne = 1 << hd->lut_window;
  float *tab = tables + ((size_t)b * hkv + kvh) * (size_t)tbl_stride;
  for (int idx = tid; idx < nch * ne * G; idx += 256) {
    const int h = idx % G, f = (idx / G) % ne, c = idx / (G * ne);
    const uint32_t bw = bld_s[c];
    const int pos = bw & 255, m = (bw >> 8) & 15, w = (bw >> 12) & 7, gi = (bw >> 15) & 3;
    float s = 0.f;
    for (int r = 0; r < m; ++r) s = fmaf(qs[h][pos + r], cent[w - 1][(f >> (w * r)) & ((1 << w) - 1)], s);
    tab[idx] = kap_s[gi] * s;
  }
  if (tid == 0) counters[(size_t)b * hkv + kvh] = 0u;
}

// ------------------------------------------------------------------ stream

struct StreamSmem {
  int vlut, pbuf, total;
};

template <int G, int VB>
__host__ __device__ constexpr StreamSmem stream_layout(int table_bytes) {
  StreamSmem s{};
  const int merge = kStreamWaves * G * kPartStride * 4;
  int r0 = table_bytes > merge ? table_bytes : merge;
  r0 = (r0 + 15) & ~15;
  s.vlut = r0;
  s.pbuf = s.vlut + VLut<VB>::entries * VLut<VB>::bytes;
  s.total = s.pbuf + kStreamWaves * 32 * G * 4;
  return s;
}

template <int VB, int WK>
struct TileRegs {
  uint32_t w[WK];
  uint2 nr;
  uint32_t nv;
  uint32_t va[2 * VB], vb[2 * VB];
};

template <int VB, int WK>
__device__ __forceinline__ void load_tile(TileRegs<VB, WK> &r, const uint32_t *__restrict__ kc,
                                          const uint16_t *__restrict__ kn, const uint32_t *__restrict__ vc,
                                          const uint16_t *__restrict__ vn, size_t base, int wk, int lane) {
#pragma unroll
  for (int j = 0; j < WK; ++j) r.w[j] = j < wk ? kc[(base * wk + j) * kTile + lane] : 0u;
  r.nr = *(const uint2 *)(kn + (base * kTile + lane) * 4);
  r.nv = vn[base * kTile + lane];
  const uint32_t *p0 = vc + (base * kHeadDim + lane) * (2 * VB);
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
__device__ __forceinline__ void lds_entry(const uint8_t *smem, uint32_t a, float (&t)[G]) {
  if constexpr (G == 1) {
    t[0] = *(const float *)(smem + a);
  } else if constexpr (G == 2) {
    const float2 v = *(const float2 *)(smem + a);
    t[0] = v.x, t[1] = v.y;
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const float4 v = *(const float4 *)(smem + a + 16 * q4);
      t[4 * q4 + 0] = v.x, t[4 * q4 + 1] = v.y, t[4 * q4 + 2] = v.z, t[4 * q4 + 3] = v.w;
    }
  }
}

template <int G>
__device__ __forceinline__ void lds_pairs(const uint8_t *p, uint32_t (&o)[G]) {
  if constexpr (G == 1) {
    o[0] = *(const uint32_t *)p;
  } else if constexpr (G == 2) {
    const uint2 v = *(const uint2 *)p;
    o[0] = v.x, o[1] = v.y;
  } else {
#pragma unroll
    for (int q4 = 0; q4 < G / 4; ++q4) {
      const uint4 v = *(const uint4 *)(p + 16 * q4);
      o[4 * q4 + 0] = v.x, o[4 * q4 + 1] = v.y, o[4 * q4 + 2] = v.z, o[4 * q4 + 3] = v.w;
    }
  }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// acc0/acc1[h] += <p' pair of head h, centroid pair> for token pair `pair`
template <int G>
__device__ __forceinline__ void pair_accum(const uint8_t *pb, int pair, uint32_t c0, uint32_t c1,
                                           float (&acc0)[G], float (&acc1)[G]) {
  uint32_t pv[G];
  lds_pairs<G>(pb + pair * G * 4, pv);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc0[h] = dot2(pv[h], c0, acc0[h]);
    acc1[h] = dot2(pv[h], c1, acc1[h]);
  }
}

struct StreamState {
  uint32_t dv;      // lane l: lookup descriptors 2l, 2l+1 (16 bits each)
  uint32_t av;      // lane jj: first chunk anchored at key word jj-1
  uint32_t fmask;   // window mask shifted to the entry offset
  int tshift;       // log2 of the bytes of one table
  int wk;
  int64_t seq;
};

template <int G, int VB, int WK>
__device__ __forceinline__ void process_tile(const TileRegs<VB, WK> &r, int tile, const StreamState &st,
                                             const uint8_t *smem, const uint8_t *vlut, uint8_t *pbuf,
                                             float (&mrun)[G], float (&lsum)[G], float (&acc0)[G],
                                             float (&acc1)[G], int lane) {
  // ---- keys: lane = token; log2-domain logits from the chunk tables
  const float nf0 = h2f((uint16_t)(r.nr.x & 0xFFFF)), nf1 = h2f((uint16_t)(r.nr.x >> 16));
  const float nf2 = h2f((uint16_t)(r.nr.y & 0xFFFF)), nf3 = h2f((uint16_t)(r.nr.y >> 16));
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
      for (int c = c0; c < c1; ++c) {
        const uint32_t pw = (uint32_t)__builtin_amdgcn_readlane((int)st.dv, c >> 1);
        const uint32_t dsc = (c & 1) ? (pw >> 16) : (pw & 0xFFFFu);
        if (dsc & kChunkStart) {
          const uint32_t slot = (dsc >> 12) & 3;
          ncur = slot == 0 ? nf0 : slot == 1 ? nf1 : slot == 2 ? nf2 : nf3;
        }
        const uint32_t t = __builtin_amdgcn_alignbit(hi, lo, (dsc >> 7) & 31);
        const uint32_t a = (t & st.fmask) | ((dsc & 127u) << st.tshift);
        float tv[G];
        lds_entry<G>(smem, a, tv);
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h] = fmaf(ncur, tv[h], lg[h]);
      }
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
    *(_Float16 *)(pbuf + ((lane >> 1) * G + h) * 4 + (lane & 1) * 2) = (_Float16)(p * nv);
  }
  wave_sync_lds();
  // ---- values: lane = coordinates lane and lane + 64
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc0[h] *= alpha[h];
    acc1[h] *= alpha[h];
  }
  if constexpr (VB == 3) {
    const uint32_t *vl = (const uint32_t *)vlut;
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
      pair_accum<G>(pbuf, y, vl[s0], vl[s1], acc0, acc1);
    }
  } else if constexpr (VB == 4) {
    const uint32_t *vl = (const uint32_t *)vlut;
#pragma unroll
    for (int y = 0; y < 32; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      pair_accum<G>(pbuf, y, vl[s0], vl[s1], acc0, acc1);
    }
  } else if constexpr (VB == 2) {
    const uint2 *vl = (const uint2 *)vlut;
#pragma unroll
    for (int y = 0; y < 16; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint2 e0 = vl[s0], e1 = vl[s1];
      pair_accum<G>(pbuf, 2 * y, e0.x, e1.x, acc0, acc1);
      pair_accum<G>(pbuf, 2 * y + 1, e0.y, e1.y, acc0, acc1);
    }
  } else {
    const uint4 *vl = (const uint4 *)vlut;
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const uint32_t s0 = (r.va[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint32_t s1 = (r.vb[y >> 2] >> (8 * (y & 3))) & 255u;
      const uint4 e0 = vl[s0], e1 = vl[s1];
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
    const uint8_t *__restrict__ consts, const float *__restrict__ tables, const uint32_t *__restrict__ kc,
    const uint16_t *__restrict__ kn, const uint32_t *__restrict__ vc, const uint16_t *__restrict__ vn,
    int64_t tiles_cap, const int32_t *__restrict__ seq_lens, int64_t max_seq_len, int tiles_per_split,
    int tbl_stride, float *__restrict__ part, uint32_t *__restrict__ counters, uint16_t *__restrict__ out,
    int n_splits) {
  constexpr int L = GLog<G>::v;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;
  const ConstHeader *hd = hdr_of(consts);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hkv = hd->n_kv_heads, hq = hd->n_q_heads;
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int win = hd->lut_window;
  const int nch = kd->n_chunks;
  const StreamSmem sm = stream_layout<G, VB>(hd->max_chunks << (win + L));
  const uint8_t *vlut = smem + sm.vlut;
  uint8_t *pbuf = smem + sm.pbuf + wave * 32 * G * 4;

  StreamState st;
  {
    int64_t s = seq_lens[b];
    st.seq = s < 0 ? 0 : (s > max_seq_len ? max_seq_len : s);
  }
  const int ntile = (int)((st.seq + kTile - 1) / kTile);
  const int tile_lo = split * tiles_per_split;
  const int tile_hi = min(tile_lo + tiles_per_split, ntile);

  // tables of this (sequence, KV head) into LDS
  {
    const int n16 = (nch << (win + L)) >> 4;
    const uint4 *src = (const uint4 *)(tables + ((size_t)b * hkv + kvh) * (size_t)tbl_stride);
    uint4 *dst = (uint4 *)smem;
    for (int i0 = 0; i0 < n16; i0 += 8 * kStreamThreads) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kStreamThreads + tid;
        if (i < n16) v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kStreamThreads + tid;
        if (i < n16) dst[i] = v[u];
      }
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
  {
    const uint32_t *lk = (const uint32_t *)(consts + hd->off_lookup) + (kd->chunk_base >> 1);
    st.dv = 2 * lane < nch ? lk[lane] : 0u;
    st.av = lane <= kMaxWK + 1 ? (uint32_t)kd->anchor[lane] : 0u;
    st.fmask = (uint32_t)((1 << win) - 1) << L;
    st.tshift = win + L;
    st.wk = hd->wk;
  }
  __syncthreads();

  float mrun[G], lsum[G], acc0[G], acc1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mrun[h] = -INFINITY, lsum[h] = 0.f, acc0[h] = 0.f, acc1[h] = 0.f;

  const size_t head_base = ((size_t)b * hkv + kvh) * (size_t)tiles_cap;
  TileRegs<VB, WK> ra, rb;
  int tile = tile_lo + wave;
  if (tile < tile_hi) load_tile(ra, kc, kn, vc, vn, head_base + tile, st.wk, lane);
  for (;;) {
    if (tile >= tile_hi) break;
    if (tile + kStreamWaves < tile_hi) load_tile(rb, kc, kn, vc, vn, head_base + tile + kStreamWaves, st.wk, lane);
    process_tile<G, VB, WK>(ra, tile, st, smem, vlut, pbuf, mrun, lsum, acc0, acc1, lane);
    tile += kStreamWaves;
    if (tile >= tile_hi) break;
    if (tile + kStreamWaves < tile_hi) load_tile(ra, kc, kn, vc, vn, head_base + tile + kStreamWaves, st.wk, lane);
    process_tile<G, VB, WK>(rb, tile, st, smem, vlut, pbuf, mrun, lsum, acc0, acc1, lane);
    tile += kStreamWaves;
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
  // ---- the last split of this (sequence, KV head) merges all splits
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[(size_t)b * hkv + kvh], 1u);
    s_last = prev == (uint32_t)(n_splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  float *ws_s = (float *)smem;                     // [G][n_splits] split weights
  float *ys = ws_s + ((G * n_splits + 3) & ~3);    // [G][128], 16-byte aligned
  const size_t pbase = ((size_t)b * hq + (size_t)kvh * G) * n_splits;
  for (int idx = tid; idx < G * n_splits; idx += kStreamThreads) ws_s[idx] = part[(pbase + idx) * kPartStride];
  __syncthreads();
  if (tid < G) {  // per head: max, then weights exp2(m_s - M) / (L sqrt(128))
    float mx = -INFINITY;
    for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ws_s[tid * n_splits + s]);
    float l = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float f = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ws_s[tid * n_splits + s] - mx);
      ws_s[tid * n_splits + s] = f;
      l = fmaf(f, part[(pbase + (size_t)tid * n_splits + s) * kPartStride + 1], l);
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
  if (tid == 0) counters[(size_t)b * hkv + kvh] = 0u;
}

// ------------------------------------------------------------------ host

typedef void (*stream_fn)(const uint8_t *, const float *, const uint32_t *, const uint16_t *, const uint32_t *,
                          const uint16_t *, int64_t, const int32_t *, int64_t, int, int, float *, uint32_t *,
                          uint16_t *, int);

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
  int n_splits, tiles_per_split, tbl_stride;  // tbl_stride in floats
  size_t off_tables, off_part, off_counters, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(const Plan &p, int batch, int64_t max_seq_len) {
  DecodeLayout d{};
  const int tiles = (int)((max_seq_len + kTile - 1) / kTile);
  const int hkv = p.desc.n_kv_heads, hq = p.desc.n_q_heads;
  const int target = 2 * device_cus();
  int s = (target + batch * hkv - 1) / (batch * hkv);
  s = std::max(1, std::min({s, (tiles + 2 * kStreamWaves - 1) / (2 * kStreamWaves), 256}));
  const int tps = (tiles + s - 1) / s;
  d.n_splits = (tiles + tps - 1) / tps;
  d.tiles_per_split = tps;
  d.tbl_stride = p.hdr.max_chunks * (1 << p.hdr.lut_window) * p.hdr.group;
  d.tbl_stride = (d.tbl_stride + 63) & ~63;
  size_t off = align256((size_t)batch * hq * kHeadDim * 4);  // rotated queries
  d.off_tables = off;
  off = align256(off + (size_t)batch * hkv * d.tbl_stride * 4);
  d.off_part = off;
  off = align256(off + (size_t)batch * hq * d.n_splits * kPartStride * 4);
  d.off_counters = off;
  d.total = align256(off + (size_t)batch * hkv * 4);
  return d;
}

}  // namespace bgtq

using namespace bgtq;

extern "C" {

bgtq_status bgtq_rotate_queries(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q, int32_t batch,
                                float *q_rot, bgtq_stream stream) {
  if (!plan || !dev_consts || !q || !q_rot) return fail(BGTQ_EINVAL, "bgtq_rotate_queries: null pointer");
  if (batch < 1 || batch > 65535) return fail(BGTQ_EINVAL, "bgtq_rotate_queries: batch must be 1..65535");
  const dim3 grid(plan->p.desc.n_kv_heads, batch);
  prep_kernel<<<grid, 256, 0, (hipStream_t)stream>>>((const uint8_t *)dev_consts, q, q_rot, nullptr, nullptr,
                                                      0.f, 0, 0);
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
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return fail(BGTQ_EDEVICE, "bgtq_decode_attn: lookup tables exceed the LDS limit");
  }
  hipStream_t st = (hipStream_t)stream;
  uint8_t *ws = (uint8_t *)workspace;
  float *qrot = (float *)ws;
  float *tables = (float *)(ws + lay.off_tables);
  float *part = (float *)(ws + lay.off_part);
  uint32_t *counters = (uint32_t *)(ws + lay.off_counters);
  const float kscale = softmax_scale * 1.4426950408889634f;  // logits in log2 units
  prep_kernel<<<dim3(p.desc.n_kv_heads, batch), 256, 0, st>>>((const uint8_t *)dev_consts, q, qrot, tables,
                                                              counters, kscale, lay.tbl_stride, 1);
  bgtq_status s = launch_status("bgtq_decode_attn (prep)");
  if (s != BGTQ_OK) return s;
  const int64_t tiles_cap = (capacity + kTile - 1) / kTile;
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
  fn<<<grid, kStreamThreads, smem, st>>>((const uint8_t *)dev_consts, tables, k_codes, k_norms, v_codes, v_norms,
                                         tiles_cap, seq_lens, max_seq_len, lay.tiles_per_split, lay.tbl_stride, part,
                                         counters, out, lay.n_splits);
  s = launch_status("bgtq_decode_attn (stream)");
  if (e1) {
    (void)hipEventRecord(e1, st);
    Prof &pr = prof();
    std::lock_guard<std::mutex> lk(pr.mu);
    pr.pending.emplace_back(e0, e1);
  }
  return s;
}

}  // extern "C"
