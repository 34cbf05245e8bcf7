// Fused decode attention over the packed Block-GTQ cache on gfx950 (the
// packed-cache serving path of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", Abstract, and of the Block-GTQ README backend table).
//
// Two launches per call.  The decode kernel, one workgroup of 16 waves (one
// per CU; 8 waves where four waves per SIMD do not fit) per (split of the
// sequence, KV head, sequence):
//  prologue  the plan's decode tables into LDS; the G queries of the KV head
//            rotated once per key width group (fp32 MFMA over the head's
//            block-diagonal rotation) into the scaled 4-bit-group queries and
//            the k-step operands of the width-1..3 groups (prep.h), in LDS.
//            The first tile is requested once the small loads of the
//            preparation have arrived, so that they are not queued behind it.
//  tiles     per 64-token tile (lane = token): key words read coalesced
//            (word-major); logits on the matrix cores (the 4-bit group one
//            fp32 4x4x1 step per code, the width-1..3 groups one fp16 4x4x4
//            k-step per four codes, both with LDS centroid lookups, the
//            lookups of the next batch in flight during the products) times
//            the group norms, in log2 units; online softmax with wavefront
//            reductions; the value codes (lane = coordinate) accumulated on the
//            matrix cores against the fp16 softmax weights in the rotated value
//            space.  The waves of a workgroup merge into one partial
//            (m, l, acc[128]) per query head.
// The merge kernel, one workgroup per (query head, sequence): log-sum-exp
// merge of the splits, normalisation, un-rotation by Pi_V^T, fp16 output.
// (Merging inside the decode kernel, by the last workgroup to arrive, costs
// more: its chain of device-coherent stores, atomics and loads sits on the
// critical path at the end of the grid.)
#include <hip/hip_ext.h>

#include "device.h"
#include "host.h"
#include "merge.h"
#include "prep.h"

namespace bgtq {

constexpr int64_t kMaxSeqLen = 0x7FFFFFFFLL - kTile;  // token positions of the decode fit 32 bits
constexpr float kRescaleSlack = 8.f;  // log2 units: softmax weights within a tile stay below 2^8


// Waves per SIMD the register allocation aims at: four (two workgroups per CU,
// at most 128 VGPRs) up to four query heads per KV head unless the key and
// value words of two tiles take too many registers; two for eight heads.
template <int G, int VB, int WK>
struct StreamOcc {
  static constexpr bool four = G <= 4 && (WK + 2 * VB <= 18 || (WK == 16 && VB <= 2));
  static constexpr int v = four ? 4 : (G <= 4 ? 3 : 2);
};

// Waves per workgroup: one workgroup of 16 waves per CU where four waves per
// SIMD fit (one query preparation per CU, every wave of the CU the same age),
// else workgroups of 8 waves.
template <int G, int VB, int WK>
struct StreamCfg {
  static constexpr int waves = StreamOcc<G, VB, WK>::four ? 16 : 8;
  static constexpr int threads = 64 * waves;
  static constexpr int per_cu = StreamOcc<G, VB, WK>::v * 4 / waves;  // resident workgroups per CU (by waves)
};

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

// Rotated queries only (the bgtq_rotate_queries entry point): one workgroup
// per (KV head, sequence).
__global__ __launch_bounds__(256) void qrot_kernel(const uint8_t *__restrict__ consts,
                                                   const uint16_t *__restrict__ q, float *__restrict__ qrot) {
  __shared__ __attribute__((aligned(16))) float qs[8 * kHeadDim];
  __shared__ __attribute__((aligned(16))) float qg[8 * kHeadDim];
  const ConstHeader *hd = hdr_of(consts);
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = hd->group, hq = hd->n_q_heads;
  const KvhDesc *kd = (const KvhDesc *)(consts + hd->off_kvh) + kvh;
  const int tid = threadIdx.x;
  const uint16_t *qb = q + ((size_t)b * hq + (size_t)kvh * G) * kHeadDim;
  const int nq = G * kHeadDim;
  RotRows<4> rr;
  rot_rows<4>((const float *)(consts + hd->off_rot32_k) + (size_t)kvh * kHeadDim * kHeadDim, tid >> 6, tid & 63, rr);
  gather_queries(kd, G, qb, qg, tid, 256);
  __syncthreads();
  rot_tiles<4>(rr, G, qg, qs, tid >> 6, tid & 63);
  __syncthreads();
  for (int idx = tid; idx < nq; idx += 256) qrot[((size_t)b * hq + (size_t)kvh * G) * kHeadDim + idx] = qs[idx];
}

// ------------------------------------------------------------------ stream

// LDS layout of the decode kernel (bytes, fixed offsets that the compiler
// folds into the LDS instruction offsets):
//   [0, kDtabBytes)  decode tables of the plan: 4-bit centroid pairs (c4),
//                    four fp16 centroids of a width-2 byte (t2) / width-1
//                    nibble (t1), two of six width-3 bits (t3)
//   [q4, +G 512)     4-bit group queries: G x 128 fp32, scaled, zero past d4
//   [qr, ..)         k-step query operands of the width-1..3 groups (PrepOut)
//   [rinv, ..)       per head: 1 / the power-of-two scale of its k-step operands
//   [vlut, ..)       value table
//   [pt, ..)         per wave: the tile's softmax weights x value norm, fp16 [G][64]
//   [kw, ..)         per wave: the tile's key words [WK + 2][64] (the last two rows zero)
// The decode and value tables are copied from global memory in the prologue,
// the prepared queries built there (prep_build, with its scratch from pt on);
// after the tile loop the area from 0 is reused for the wave merge.  Past
// `total`: 16 spare bytes that take the stores of the copy falling outside the
// tables.
template <int G, int VB, int WK = kMaxWK>
struct StreamLds {
  static constexpr int c4 = kDtabC4, t2 = kDtabT2, t1 = kDtabT1, t3 = kDtabT3;
  static constexpr int q4 = kDtabBytes;
  static constexpr int qr = q4 + PrepOut<G>::qr;
  static constexpr int rinv = q4 + PrepOut<G>::rinv;
  static constexpr int vlut = q4 + PrepOut<G>::bytes;
  static constexpr int pt = (vlut + VLut<VB>::entries * VLut<VB>::bytes + 15) & ~15;
  static constexpr int W = StreamCfg<G, VB, WK>::waves;
  static constexpr int kw = pt + W * G * kTile * 2;
  static constexpr int kw_rows = WK + 2;  // key words of the tile, then two zero rows
  static constexpr int end = kw + W * kw_rows * kTile * 4;
  static constexpr int merge = W * G * kPartStride * 4;
  static constexpr int total = end > merge ? end : merge;
  static constexpr int spare = total, alloc = total + 16;
  static_assert(t2 % 2048 == 0 && t1 % 128 == 0 && t3 % 256 == 0, "table bases above the index bits");
  static_assert(q4 % 16 == 0 && vlut % 16 == 0 && kw % 16 == 0, "16-byte aligned areas");
  static constexpr int scr = pt;  // query-preparation scratch (before the tile loop)
  static_assert(scr + PrepScratch<G>::bytes <= total, "preparation scratch inside the allocation");
};

template <int VB, int WK>
struct TileRegs {
  uint32_t w[WK];
  uint2 nr;
  uint32_t nv;
  uint32_t va[2 * VB], vb[2 * VB];
};

// The tile's loads: wave-uniform base addresses (scalar registers) plus the
// lane's offset, so that the compiler keeps one offset register per array.
// Branch-free: a plan without key words (every block at zero bits) reads the
// plan's block of zeros for every tile (`kstride` 0).  The loads are
// non-temporal (streaming): the cache is read once per call, and keeping it
// out of the caches' retained lines leaves the plan's constant image
// (rotations, tables) cached for the prologues and the merge kernel (the
// decode call measured 2.4 us shorter at the 128K layer).
typedef uint32_t ntu4 __attribute__((ext_vector_type(4)));
typedef uint32_t ntu2 __attribute__((ext_vector_type(2)));
template <int VB, int WK>
__device__ __forceinline__ void load_tile(TileRegs<VB, WK> &r, const uint32_t *__restrict__ kc, size_t kstride,
                                          const uint16_t *__restrict__ kn, const uint32_t *__restrict__ vc,
                                          const uint16_t *__restrict__ vn, size_t base, int lane) {
  const uint32_t *kt = kc + base * kstride;
#pragma unroll
  for (int j = 0; j < WK; ++j) r.w[j] = __builtin_nontemporal_load(kt + j * kTile + lane);
  const ntu2 nr = __builtin_nontemporal_load((const ntu2 *)(kn + base * kTile * 4 + lane * 4));
  r.nr = make_uint2(nr.x, nr.y);
  r.nv = __builtin_nontemporal_load(vn + base * kTile + lane);
  const uint32_t *vt = vc + base * kHeadDim * (2 * VB);
  const uint32_t *p0 = vt + lane * (2 * VB);
  const uint32_t *p1 = p0 + 64 * (2 * VB);
  if constexpr (VB == 1) {
    const ntu2 a = __builtin_nontemporal_load((const ntu2 *)p0), c = __builtin_nontemporal_load((const ntu2 *)p1);
    r.va[0] = a.x, r.va[1] = a.y, r.vb[0] = c.x, r.vb[1] = c.y;
  } else if constexpr (VB == 2) {
    const ntu4 a = __builtin_nontemporal_load((const ntu4 *)p0), c = __builtin_nontemporal_load((const ntu4 *)p1);
    r.va[0] = a.x, r.va[1] = a.y, r.va[2] = a.z, r.va[3] = a.w;
    r.vb[0] = c.x, r.vb[1] = c.y, r.vb[2] = c.z, r.vb[3] = c.w;
  } else if constexpr (VB == 3) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const ntu2 a = __builtin_nontemporal_load((const ntu2 *)(p0 + 2 * k)),
                 c = __builtin_nontemporal_load((const ntu2 *)(p1 + 2 * k));
      r.va[2 * k] = a.x, r.va[2 * k + 1] = a.y, r.vb[2 * k] = c.x, r.vb[2 * k + 1] = c.y;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const ntu4 a = __builtin_nontemporal_load((const ntu4 *)(p0 + 4 * k)),
                 c = __builtin_nontemporal_load((const ntu4 *)(p1 + 4 * k));
      r.va[4 * k] = a.x, r.va[4 * k + 1] = a.y, r.va[4 * k + 2] = a.z, r.va[4 * k + 3] = a.w;
      r.vb[4 * k] = c.x, r.vb[4 * k + 1] = c.y, r.vb[4 * k + 2] = c.z, r.vb[4 * k + 3] = c.w;
    }
  }
}

struct StreamState {
  uint32_t kwl;       // LDS byte address of this lane's word 0 in this wave's key-word rows
  uint32_t qrl;       // LDS byte address of this lane's row in k-step 0's query operand
  uint32_t cgrp;      // first k-step of the width-3, 2, 1 groups (bytes 0..2), k-step count (byte 3)
  uint32_t gbit;      // first stream bit of the width-3, 2, 1 groups (10 bits each)
  uint32_t ptw;       // LDS byte offset of this wave's weight rows
  int wk, n4w;
  int lo;       // first token of the packed range
  uint32_t nv;  // tokens in the packed range [lo, lo + nv)
  int64_t seq;  // end of the packed range (may be below lo: an empty range)
};

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
template <int G>
struct VQuads {
  static constexpr int v = (G + 3) / 4;  // matrix-core registers of 4 query heads
};

// Key word J holds codes 8 J .. 8 J + 7, two per byte (low nibble first).  The
// words are pipelined: the four lookups of word J + 1 (and the query operand of
// its block of 16 codes) are issued before the products of word J.
template <int WK, int J>
__device__ __forceinline__ void key4_lookups(const uint32_t (&w)[WK], uint32_t c4l, float2 (&cp)[4]) {
  const uint32_t word = w[J];
#pragma unroll
  for (int by = 0; by < 4; ++by) cp[by] = lds_at<float2>(c4l + (((word >> (8 * by)) & 255u) << 3));
}

template <int G, int VB, int BLK>
__device__ __forceinline__ void key4_query(int lane, float (&qa)[VQuads<G>::v]) {
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g)
    qa[g] = lds_at<float>(StreamLds<G, VB>::q4 +
                          (uint32_t)(((4 * g + (lane & 3)) & (G - 1)) * kHeadDim + 16 * BLK + (lane >> 2)) * 4);
}

template <int G, int J>
__device__ __forceinline__ void key4_products(const float2 (&cp)[4], const float (&qa)[VQuads<G>::v],
                                              f4v (&a4)[VQuads<G>::v]) {
  constexpr int S0 = 8 * (J & 1);
#define BGTQ_K4(BY)                                                                          \
  _Pragma("unroll") for (int g = 0; g < VQuads<G>::v; ++g) {                                 \
    a4[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(qa[g], cp[BY].x, a4[g], 4, S0 + 2 * BY, 0);     \
    a4[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(qa[g], cp[BY].y, a4[g], 4, S0 + 2 * BY + 1, 0); \
  }
  BGTQ_K4(0) BGTQ_K4(1) BGTQ_K4(2) BGTQ_K4(3)
#undef BGTQ_K4
}

// Word J (< n4w) with its lookups in cx and the query operand of its block in qx;
// word J + 1's go to cy / qy (the query operand only at a block boundary).
template <int G, int VB, int WK, int J>
__device__ __forceinline__ void key4_words(const uint32_t (&w)[WK], int n4w, int lane, uint32_t c4l, float2 (&cx)[4],
                                           float2 (&cy)[4], float (&qx)[VQuads<G>::v], float (&qy)[VQuads<G>::v],
                                           f4v (&a4)[VQuads<G>::v]) {
  if constexpr (J < WK) {
    if (J < n4w) {
      if constexpr (J + 1 < WK) {
        key4_lookups<WK, J + 1>(w, c4l, cy);
        if constexpr ((J & 1) == 1) key4_query<G, VB, (J + 1) / 2>(lane, qy);
      }
      __builtin_amdgcn_sched_barrier(0);
      key4_products<G, J>(cx, qx, a4);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr ((J & 1) == 1)
        key4_words<G, VB, WK, J + 1>(w, n4w, lane, c4l, cy, cx, qy, qx, a4);
      else
        key4_words<G, VB, WK, J + 1>(w, n4w, lane, c4l, cy, cx, qx, qy, a4);
    }
  }
}

// 4-bit group on the matrix cores, one v_mfma_f32_4x4x1f32 per code r (16 blocks
// of 4 x 4 x 1): block k is lanes 4k .. 4k + 3 = tokens 4k .. 4k + 3, its B operand
// the token's centroid c4[code_r] (centroid pairs at LDS byte 8 x code byte) and
// its output row m head m, so the token's lane keeps
// a4[h] in register h.  The A operand, head m's query value of code r, is
// broadcast from block r % 16 of a register whose lane 4k + m holds code
// 16 (r / 16) + k (CBSZ 4, ABID r % 16).
template <int G, int VB, int WK>
__device__ __forceinline__ void key4_group(const uint32_t (&w)[WK], int n4w, int lane, uint32_t c4l,
                                           f4v (&a4)[VQuads<G>::v]) {
  if (n4w > 0) {
    float2 cx[4], cy[4];
    float qx[VQuads<G>::v], qy[VQuads<G>::v];
    key4_lookups<WK, 0>(w, c4l, cx);
    key4_query<G, VB, 0>(lane, qx);
    key4_words<G, VB, WK, 0>(w, n4w, lane, c4l, cx, cy, qx, qy, a4);
  }
}

// Width-1..3 groups on the matrix cores: per k-step (four positions of one
// group), v_mfma_f32_4x4x4f16 adds sum_i q[m][i] c[code_i] for every token.
// Block k is lanes 4k .. 4k + 3 = tokens; its B operand is the token's four
// fp16 centroids, looked up from the k-step's 4w code bits, and every block
// takes the same A operand, head m's four scaled query values, from the LDS
// operand row of the k-step (lane 4k + m reads row m).
//
// The key words of the tile are staged in LDS (this wave's rows [word][lane],
// two zero rows past the last word), so that a group's bits can be re-read
// from its first word b (a per-head value) and realigned to bit 0:
// al[i] = bits [32 i, 32 i + 32) of the group = alignbit(W[b + i + 1], W[b + i],
// shift).  K-step s then sits at the static bits [4 w s, 4 w s + 4 w) of al.
template <int W>
struct KStep {
  static constexpr int bits = 4 * W;
  // highest aligned register that k-step s touches
  static constexpr int last_reg(int s) { return (bits * s + bits - 1) / 32; }
};

template <int W, int S>
__device__ __forceinline__ uint32_t kstep_bits(const uint32_t (&al)[13]) {
  constexpr int lo = KStep<W>::bits * S, i = lo / 32, off = lo % 32;
  if constexpr (off + KStep<W>::bits <= 32)
    return al[i] >> off;
  else
    return __builtin_amdgcn_alignbit(al[i + 1], al[i], off);
}

template <int G, int VB, int W>
__device__ __forceinline__ h4v kstep_b(uint32_t t) {
  typedef StreamLds<G, VB> Lds;
  if constexpr (W == 3)
    return __builtin_bit_cast(h4v, (u2v){lds_at<uint32_t>(Lds::t3 + ((t << 2) & 0xFCu)),
                                         lds_at<uint32_t>(Lds::t3 + ((t >> 4) & 0xFCu))});
  else if constexpr (W == 2)
    return lds_at<h4v>(Lds::t2 + ((t & 255u) << 3));
  else
    return lds_at<h4v>(Lds::t1 + ((t & 15u) << 3));
}

// K-steps S, S + 1, ... of the group of width W (ns of them), reading aligned
// register i of the group when the first k-step needs it.
template <int G, int VB, int W, int S>
__device__ __forceinline__ void kgroup_steps(uint32_t (&wd)[14], uint32_t (&al)[13], uint32_t wa, uint32_t sh,
                                             uint32_t qa, int ns, f4v (&acc)[VQuads<G>::v]) {
  if constexpr (S < 32) {
    if (S >= ns) return;
    constexpr int hi = KStep<W>::last_reg(S), lo = S == 0 ? 0 : KStep<W>::last_reg(S - 1) + 1;
#pragma unroll
    for (int i = lo; i <= hi; ++i) {
      wd[i + 1] = lds_at<uint32_t>(wa + 256 * (i + 1));
      al[i] = __builtin_amdgcn_alignbit(wd[i + 1], wd[i], sh);
    }
    const h4v bq = kstep_b<G, VB, W>(kstep_bits<W, S>(al));
#pragma unroll
    for (int g = 0; g < VQuads<G>::v; ++g)
      acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(lds_at<h4v>(qa + (S * VQuads<G>::v + g) * 32), bq, acc[g], 0, 0, 0);
    kgroup_steps<G, VB, W, S + 1>(wd, al, wa, sh, qa, ns, acc);
  }
}

// The k-steps of the width-(3 - R) group.
template <int G, int VB, int WK, int R>
__device__ __forceinline__ void key_group(const StreamState &st, f4v (&acc)[VQuads<G>::v]) {
  constexpr int W = 3 - R;
  const int cb = (st.cgrp >> (8 * R)) & 255, ce = (st.cgrp >> (8 * R + 8)) & 255;
  if (cb >= ce) return;
  const uint32_t bit = (st.gbit >> (10 * R)) & 1023u;
  const uint32_t wa = st.kwl + (bit >> 5) * 256;
  const uint32_t qa = st.qrl + (uint32_t)cb * (VQuads<G>::v * 32);
  uint32_t wd[14], al[13];
  wd[0] = lds_at<uint32_t>(wa);
  // The k-step count is opaque per tile, so that the compiler evaluates each
  // k-step's guard where it is used instead of keeping all of them live.
  int ns = ce - cb;
  asm volatile("" : "+s"(ns));
  kgroup_steps<G, VB, W, 0>(wd, al, wa, bit & 31u, qa, ns, acc);
}

// In-place maximum over the 64 lanes of each v[h] (every lane receives it):
// fused DPP max steps, heads interleaved so that consecutive steps of one head
// are at least two instructions apart.
#define BGTQ_MX(V, CTL) "v_max_f32_dpp %" #V ", %" #V ", %" #V " " CTL " bank_mask:0xf\n\t"
#define BGTQ_MX4(CTL) BGTQ_MX(0, CTL) BGTQ_MX(1, CTL) BGTQ_MX(2, CTL) BGTQ_MX(3, CTL)
#define BGTQ_MX2(CTL) BGTQ_MX(0, CTL) "s_nop 0\n\t" BGTQ_MX(1, CTL)
template <int G>
__device__ __forceinline__ void wave_max_heads(float (&v)[G]) {
  if constexpr (G == 1) {
    asm("s_nop 1\n\t" BGTQ_MX(0, "quad_perm:[1,0,3,2] row_mask:0xf") "s_nop 1\n\t"
        BGTQ_MX(0, "quad_perm:[2,3,0,1] row_mask:0xf") "s_nop 1\n\t" BGTQ_MX(0, "row_half_mirror row_mask:0xf")
        "s_nop 1\n\t" BGTQ_MX(0, "row_mirror row_mask:0xf") "s_nop 1\n\t" BGTQ_MX(0, "row_bcast:15 row_mask:0xa")
        "s_nop 1\n\t" BGTQ_MX(0, "row_bcast:31 row_mask:0xc")
        : "+v"(v[0]));
  } else if constexpr (G == 2) {
    asm("s_nop 1\n\t" BGTQ_MX2("quad_perm:[1,0,3,2] row_mask:0xf") "s_nop 0\n\t"
        BGTQ_MX2("quad_perm:[2,3,0,1] row_mask:0xf") "s_nop 0\n\t" BGTQ_MX2("row_half_mirror row_mask:0xf")
        "s_nop 0\n\t" BGTQ_MX2("row_mirror row_mask:0xf") "s_nop 0\n\t" BGTQ_MX2("row_bcast:15 row_mask:0xa")
        "s_nop 0\n\t" BGTQ_MX2("row_bcast:31 row_mask:0xc")
        : "+v"(v[0]), "+v"(v[1]));
  } else {
#pragma unroll
    for (int g = 0; g < G; g += 4) {
      asm("s_nop 1\n\t" BGTQ_MX4("quad_perm:[1,0,3,2] row_mask:0xf") BGTQ_MX4("quad_perm:[2,3,0,1] row_mask:0xf")
              BGTQ_MX4("row_half_mirror row_mask:0xf") BGTQ_MX4("row_mirror row_mask:0xf")
                  BGTQ_MX4("row_bcast:15 row_mask:0xa") BGTQ_MX4("row_bcast:31 row_mask:0xc")
          : "+v"(v[g]), "+v"(v[g + 1]), "+v"(v[g + 2]), "+v"(v[g + 3]));
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
    v[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[h]), 63));
}
#undef BGTQ_MX2
#undef BGTQ_MX4
#undef BGTQ_MX

// Value accumulation on the matrix cores: per tile, acc[h][i] += sum_t P'[h][t] v[t][i]
// with P' = softmax weight x value norm (fp16) and v the fp16 centroids of the
// lane's coordinate i, as 16 steps of v_mfma_f32_4x4x4f16 (16 blocks of 4 x 4,
// K = 4 tokens).  Block k of a step is lanes 4k .. 4k + 3: its B operand is the
// four tokens of coordinate (lane) and its output row m is head m, so lane i
// keeps acc[h][i] in register h.  The A operand (P' of tokens 4S .. 4S + 3) is
// broadcast from block S (CBSZ 4, ABID S), whose lane 4S + m holds head m.
template <int BIT, int N>
__device__ __forceinline__ uint32_t bits6(const uint32_t (&c)[N]) {
  constexpr int wi = BIT >> 5, sh = BIT & 31;
  if constexpr (sh <= 26)
    return (c[wi] >> sh) & 63u;
  else
    return __builtin_amdgcn_alignbit(c[wi + 1], c[wi], sh) & 63u;
}

// B operand of step S: the fp16 centroids of tokens 4S .. 4S + 3 (bits 4 VB S ..
// 4 VB (S + 1) of the coordinate's code stream) from the value table.
template <int VB, int S>
__device__ __forceinline__ h4v v_operand(const uint32_t (&c)[2 * VB], uint32_t vlut) {
  if constexpr (VB == 1) {  // entry = one byte (8 tokens) x 16 bytes
    const uint32_t y = (c[S >> 3] >> (8 * ((S >> 1) & 3))) & 255u;
    return lds_at<h4v>(vlut + 16 * y + 8 * (S & 1));
  } else if constexpr (VB == 2) {  // entry = one byte (4 tokens) x 8 bytes
    const uint32_t y = (c[S >> 2] >> (8 * (S & 3))) & 255u;
    return lds_at<h4v>(vlut + 8 * y);
  } else if constexpr (VB == 3) {  // entry = 6 bits (2 tokens) x 4 bytes
    const uint32_t y0 = bits6<12 * S>(c), y1 = bits6<12 * S + 6>(c);
    return __builtin_bit_cast(h4v, (u2v){lds_at<uint32_t>(vlut + 4 * y0), lds_at<uint32_t>(vlut + 4 * y1)});
  } else {  // entry = one byte (2 tokens) x 4 bytes
    const uint32_t w = c[S >> 1] >> (16 * (S & 1));
    return __builtin_bit_cast(h4v, (u2v){lds_at<uint32_t>(vlut + 4 * (w & 255u)),
                                         lds_at<uint32_t>(vlut + 4 * ((w >> 8) & 255u))});
  }
}

// The 16 steps in batches of kVBatch: the lookups of batch k + 1 are issued
// before the products of batch k, so that the wave keeps 2 kVBatch lookups in
// flight instead of waiting for each one.
constexpr int kVBatch = 4;

template <int VB, int S, int N>
__device__ __forceinline__ void v_lookups(const uint32_t (&va)[2 * VB], const uint32_t (&vb)[2 * VB], uint32_t vlut,
                                          h4v (&b0)[kVBatch], h4v (&b1)[kVBatch]) {
  if constexpr (N < kVBatch) {
    b0[N] = v_operand<VB, S + N>(va, vlut);
    b1[N] = v_operand<VB, S + N>(vb, vlut);
    v_lookups<VB, S, N + 1>(va, vb, vlut, b0, b1);
  }
}

template <int G, int S, int N>
__device__ __forceinline__ void v_products(const h4v (&b0)[kVBatch], const h4v (&b1)[kVBatch],
                                           const h4v (&pa)[VQuads<G>::v], f4v (&acc0)[VQuads<G>::v],
                                           f4v (&acc1)[VQuads<G>::v]) {
  if constexpr (N < kVBatch) {
#pragma unroll
    for (int g = 0; g < VQuads<G>::v; ++g) {
      acc0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa[g], b0[N], acc0[g], 4, S + N, 0);
      acc1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa[g], b1[N], acc1[g], 4, S + N, 0);
    }
    v_products<G, S, N + 1>(b0, b1, pa, acc0, acc1);
  }
}

// Batch starting at step S, whose lookups are in (x0, x1); the next batch's go to (y0, y1).
template <int G, int VB, int S>
__device__ __forceinline__ void v_mfma_steps(const uint32_t (&va)[2 * VB], const uint32_t (&vb)[2 * VB], uint32_t vlut,
                                             const h4v (&pa)[VQuads<G>::v], h4v (&x0)[kVBatch],
                                             h4v (&x1)[kVBatch], h4v (&y0)[kVBatch], h4v (&y1)[kVBatch],
                                             f4v (&acc0)[VQuads<G>::v], f4v (&acc1)[VQuads<G>::v]) {
  if constexpr (S < kTile / 4) {
    if constexpr (S + kVBatch < kTile / 4) v_lookups<VB, S + kVBatch, 0>(va, vb, vlut, y0, y1);
    __builtin_amdgcn_sched_barrier(0);
    v_products<G, S, 0>(x0, x1, pa, acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    v_mfma_steps<G, VB, S + kVBatch>(va, vb, vlut, pa, y0, y1, x0, x1, acc0, acc1);
  }
}

template <int G, int VB, int WK>
__device__ __forceinline__ void process_tile(const TileRegs<VB, WK> &r, int tile, const StreamState &st,
                                             const float (&rinv)[G], float (&mrun)[G], float (&mth)[G],
                                             float (&lsum)[G], f4v (&acc0)[VQuads<G>::v],
                                             f4v (&acc1)[VQuads<G>::v], int lane) {
  // ---- keys, lane = token.  4-bit group: one fp32 step per code.
  f4v a4[VQuads<G>::v];
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g) a4[g] = (f4v){0.f, 0.f, 0.f, 0.f};
  key4_group<G, VB, WK>(r.w, st.n4w, lane, (uint32_t)StreamLds<G, VB, WK>::c4, a4);
  // widths 3, 2, 1 (norm slots 1, 2, 3): fp16 k-steps, lr = sum_w n_w acc_w,
  // from the key words staged in this wave's LDS rows
#pragma unroll
  for (int j = 0; j < WK; ++j)
    *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * j) = r.w[j];
  float lr[G];
  {
    f4v ak[VQuads<G>::v];
#define BGTQ_KG(R, NORM)                                                              \
  {                                                                                   \
    _Pragma("unroll") for (int g = 0; g < VQuads<G>::v; ++g) ak[g] = (f4v){0.f, 0.f, 0.f, 0.f}; \
    key_group<G, VB, WK, R>(st, ak);                                                  \
    const float nw = h2f((uint16_t)(NORM));                                           \
    _Pragma("unroll") for (int h = 0; h < G; ++h) lr[h] = R == 0 ? nw * ak[h >> 2][h & 3] : fmaf(nw, ak[h >> 2][h & 3], lr[h]); \
  }
    BGTQ_KG(0, r.nr.x >> 16) BGTQ_KG(1, r.nr.y & 0xFFFFu) BGTQ_KG(2, r.nr.y >> 16)
#undef BGTQ_KG
  }
  // token positions fit 32 bits (max_seq_len < 2^31 - 64); below lo wraps to a large unsigned value
  const bool valid = (uint32_t)(tile * kTile + lane - st.lo) < st.nv;
  const float n4 = h2f((uint16_t)(r.nr.x & 0xFFFF));  // norm slot 0: the 4-bit group
  const float nv = h2f((uint16_t)r.nv);
  // ---- online softmax (log2 domain), rescaled lazily: the running maximum
  // moves (with the wave maximum, the rescale of the sums and the
  // accumulators) only when a logit exceeds it by more than kRescaleSlack, so
  // p = 2^(l - m) stays below 2^kRescaleSlack.  P' = p * value norm, fp16, to
  // the wave's LDS rows [h][token].
  float l[G];
  bool up = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = valid ? fmaf(n4, a4[h >> 2][h & 3], lr[h] * rinv[h]) : -INFINITY;
    up = up || l[h] > mth[h];
  }
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) mx[h] = l[h];
    wave_max_heads<G>(mx);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(mrun[h], mx[h]);
      const float alpha = __builtin_amdgcn_exp2f(mrun[h] - mn);
      lsum[h] *= alpha;
      acc0[h >> 2][h & 3] *= alpha;
      acc1[h >> 2][h & 3] *= alpha;
      // wave-uniform: kept in scalar registers
      mrun[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn)));
      mth[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn + kRescaleSlack)));
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p = __builtin_amdgcn_exp2f(l[h] - mrun[h]);
    lsum[h] += p;
    *(__attribute__((address_space(3))) _Float16 *)(size_t)(st.ptw + h * (2 * kTile) + 2 * lane) = (_Float16)(p * nv);
  }
  // A operands: lane 4k + m holds head m's weights of tokens 4k .. 4k + 3 (heads
  // past G repeat a valid row; their output rows are never read)
  h4v pa[VQuads<G>::v];
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g)
    pa[g] = lds_at<h4v>(st.ptw + ((4 * g + (lane & 3)) & (G - 1)) * (2 * kTile) + (lane >> 2) * 8);
  // ---- values: lane = coordinates lane and lane + 64
  typedef StreamLds<G, VB, WK> L;
  const uint32_t vlut = (uint32_t)L::vlut;
  h4v x0[kVBatch], x1[kVBatch], y0[kVBatch], y1[kVBatch];
  v_lookups<VB, 0, 0>(r.va, r.vb, vlut, x0, x1);
  v_mfma_steps<G, VB, 0>(r.va, r.vb, vlut, pa, x0, x1, y0, y1, acc0, acc1);
}


// ------------------------------------------------------------------ decode kernel

// Launch arguments (by value; the host fills in what it knows so that the
// kernel starts without dependent loads).
struct DecodeArgs {
  const uint8_t *consts;
  const uint16_t *q;
  const uint32_t *kc;
  const uint16_t *kn;
  const uint32_t *vc;
  const uint16_t *vn;
  const int32_t *seq_lens;
  float *part;  // split partials [batch][hq][n_splits][kPartStride]
  const int32_t *table;  // paged pools: block table [batch][max_pages], else null
  int64_t head_stride, seq_stride;  // tile index = kvh * head_stride + b * seq_stride + page
  int max_pages, n_pages;
  int64_t max_seq_len, off_kvh, off_dtab, off_vlut, off_zero;
  int hkv, hq, wk, tiles_base, tiles_extra, n_splits;  // split s: tiles_base + (s < tiles_extra) tiles
  int seq_add;  // sequence length = seq_lens[b] + seq_add (1 when seq_lens holds the new token's position)
  int n_sink, n_recent;  // tokens [0, n_sink) and [T - n_recent, T) are served from fp16 buffers, not here
  float kscale;  // softmax scale in log2 units
};

template <int G, int VB, int WK>
__global__ __attribute__((amdgpu_flat_work_group_size(1, StreamCfg<G, VB, WK>::threads)))
__attribute__((amdgpu_waves_per_eu(StreamOcc<G, VB, WK>::v)))
void decode_kernel(const DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint8_t *consts = a.consts;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const KvhDesc *kd = (const KvhDesc *)(consts + a.off_kvh) + kvh;
  typedef StreamLds<G, VB, WK> Lds;
  constexpr int kStreamWaves = StreamCfg<G, VB, WK>::waves, kStreamThreads = StreamCfg<G, VB, WK>::threads;

  // ---- prologue loads, in this order so that waiting for an earlier group
  // does not wait for a later one (loads complete in order): the sequence
  // length and the head's group fields, the row-table entries of the
  // rotation rows, the query preparation's inputs, the plan's decode and
  // value tables (16 bytes per thread and round), the nonzero part of the
  // rotation (addressed from the row-table entries), then the first tile.
  const int64_t seq_raw = (int64_t)a.seq_lens[b] + a.seq_add;
  const int n4w = kd->n4w;
  const uint32_t cgrp = kd->cgrp, gbit = kd->gbit;
  PrepIn<G, kStreamWaves> pin;
  prep_issue_keys<G, kStreamWaves>(pin, consts, kvh, wave, lane);
  prep_issue<G, kStreamWaves>(pin, consts, kvh, a.q + ((size_t)b * a.hq + (size_t)kvh * G) * kHeadDim, tid, wave,
                              lane);
  constexpr int n0 = kDtabBytes >> 4;
  constexpr int n1 = n0 + ((VLut<VB>::entries * VLut<VB>::bytes) >> 4);
  constexpr int kRounds = (n1 + kStreamThreads - 1) / kStreamThreads;
  const uint4 *cs0 = (const uint4 *)(consts + a.off_dtab), *cs1 = (const uint4 *)(consts + a.off_vlut) - n0;
  static_assert(kRounds <= 2 && n0 <= kStreamThreads, "at most two rounds of the table copy");
  const int i0 = min(tid, n1 - 1), i1 = min(tid + kStreamThreads, n1 - 1);
  const uint4 cr0 = *(i0 < n0 ? cs0 + i0 : cs1 + i0);
  uint4 cr1 = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (kRounds == 2) cr1 = *(cs1 + i1);
  prep_issue_rot<G, kStreamWaves>(pin, consts, a.off_zero, kvh, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  // the tables, descriptor and queries into LDS before the first tile is
  // requested (waiting for these loads only), so that they are not queued
  // behind the grid's tile requests
  const auto tab_at = [](int i) { return i < n0 ? 16 * i : i < n1 ? Lds::vlut + 16 * (i - n0) : Lds::spare; };
  *(uint4 *)(smem + tab_at(tid)) = cr0;
  if constexpr (kRounds == 2) *(uint4 *)(smem + tab_at(tid + kStreamThreads)) = cr1;
  prep_stage<G, kStreamWaves>(pin, smem + Lds::q4, smem + Lds::scr, tid);
  StreamState st;
  __builtin_amdgcn_sched_barrier(0);  // keep the staging ahead of the tile request
  // ---- tiles of this wave: tile_lo + wave, + W, ... (W waves); double-buffered
  // registers.  The first is requested now, before the query preparation, its
  // range bounded by max_seq_len (in memory).
  const int tile_lo = split * a.tiles_base + min(split, a.tiles_extra);
  const int tile_end =
      min(tile_lo + a.tiles_base + (split < a.tiles_extra ? 1 : 0), (int)((a.max_seq_len + kTile - 1) / kTile));
  // tile index = head_base + page; page = tile (contiguous) or the block
  // table's entry (paged; clamped into the pool, read one tile ahead)
  const size_t head_base = (size_t)kvh * a.head_stride + (size_t)b * a.seq_stride;
  const bool paged = a.table != nullptr;
  const int32_t *btab = paged ? a.table + (size_t)b * a.max_pages : nullptr;
  const auto page_of = [&](int t) -> size_t {
    return (size_t)min((uint32_t)__builtin_amdgcn_readfirstlane(btab[t]), (uint32_t)(a.n_pages - 1));
  };
  const bool kzero = a.wk == 0;
  // (zero-key plans run the 4-word kernel: the plan's zero block is one such tile)
  static_assert(4 * kTile * 4 == kZeroBytes, "zero block of one 4-word tile");
  const uint32_t *kcodes = kzero ? (const uint32_t *)(consts + a.off_zero) : a.kc;
  const size_t kstride = kzero ? 0 : (size_t)WK * kTile;
  TileRegs<VB, WK> ra, rb;
  int tile = tile_lo + wave;
  size_t pn = 0;  // paged: page of the wave's next tile
  if (paged) {
    load_tile(ra, kcodes, kstride, a.kn, a.vc, a.vn, head_base + page_of(min(tile, tile_end - 1)), lane);
    pn = page_of(min(tile + kStreamWaves, tile_end - 1));
  } else {
    load_tile(ra, kcodes, kstride, a.kn, a.vc, a.vn, head_base + min(tile, tile_end - 1), lane);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the queries of this (sequence, KV head), rotated and scaled (ends with a barrier)
  prep_build<G, kStreamWaves>(pin, smem + Lds::q4, smem + Lds::scr, a.kscale, tid, wave, lane);
  st.seq = (seq_raw < 0 ? 0 : (seq_raw > a.max_seq_len ? a.max_seq_len : seq_raw)) - a.n_recent;
  st.lo = a.n_sink;
  st.nv = (uint32_t)(st.seq > st.lo ? st.seq - st.lo : 0);
  st.wk = a.wk;
  st.kwl = (uint32_t)(Lds::kw + wave * (Lds::kw_rows * kTile * 4) + lane * 4);
  st.qrl = (uint32_t)Lds::qr + (uint32_t)(lane & 3) * 8;
  st.ptw = (uint32_t)(Lds::pt + wave * (G * kTile * 2));
  st.n4w = n4w;
  st.cgrp = cgrp;
  st.gbit = gbit;
  // the two zero rows past the key words (this lane's column, read by this lane only)
  *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * WK) = 0u;
  *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * (WK + 1)) = 0u;
  float rinv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) rinv[h] = lds_at<float>(Lds::rinv + 4 * h);

  const int ntile = (int)((st.seq + kTile - 1) / kTile);
  const int tile_hi = min(tile_end, ntile);
  float mrun[G], mth[G], lsum[G];  // running maximum, rescale threshold mrun + kRescaleSlack, sum
  f4v acc0[VQuads<G>::v], acc1[VQuads<G>::v];
#pragma unroll
  // The running maximum starts finite, far below any logit, so that a tile
  // without a valid token (all logits -inf; possible below the packed range's
  // first token) gives p = 2^(-inf) = 0 rather than 2^(-inf + inf).
  for (int h = 0; h < G; ++h) mrun[h] = -0x1p100f, mth[h] = -0x1p100f, lsum[h] = 0.f;
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g) acc0[g] = (f4v){0.f, 0.f, 0.f, 0.f}, acc1[g] = acc0[g];
  // One copy of the tile body (the instruction cache holds the loop): the
  // next tile's registers are requested before the current one is processed
  // and moved into place after it.  (Two copies with alternating register
  // sets raise the register count past the occupancy limit.)
  for (; tile < tile_hi; tile += kStreamWaves) {
    const int tn = min(tile + kStreamWaves, tile_hi - 1);
    size_t bn = head_base + tn;
    if (paged) {  // (the prefetched page belongs to tn except on the last pass, whose load is not used)
      bn = head_base + pn;
      pn = page_of(min(tile + 2 * kStreamWaves, tile_hi - 1));
    }
    load_tile(rb, kcodes, kstride, a.kn, a.vc, a.vn, bn, lane);
    process_tile<G, VB, WK>(ra, tile, st, rinv, mrun, mth, lsum, acc0, acc1, lane);
    ra = rb;
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
    rr[4 + lane] = acc0[h >> 2][h & 3];
    rr[4 + 64 + lane] = acc1[h >> 2][h & 3];
  }
  __syncthreads();
  const size_t head0 = (size_t)b * a.hq + (size_t)kvh * G;  // first query head of this (sequence, KV head)
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
    float *o = a.part + ((head0 + h) * a.n_splits + split) * kPartStride;
    o[4 + i] = s;
    if (i == 0) o[0] = mx, o[1] = l;
  }
}

// ------------------------------------------------------------------ host
// ------------------------------------------------------------------ host

typedef void (*decode_fn)(const DecodeArgs);

// The decode kernel of a plan shape with its launch parameters.
struct DecodeKernel {
  decode_fn fn;
  int smem, waves, per_cu;
};

template <int G, int VB, int WK>
DecodeKernel kernel_of() {
  return {decode_kernel<G, VB, WK>, StreamLds<G, VB, WK>::alloc, StreamCfg<G, VB, WK>::waves,
          StreamCfg<G, VB, WK>::per_cu};
}

// Key words per token: 4 avg_bits exactly (zero-bit plans run the 4-word kernel
// with the key words zero).
template <int G, int VB>
DecodeKernel pick_wk(int wk) {
  if (wk <= 4) return kernel_of<G, VB, 4>();
  if (wk <= 8) return kernel_of<G, VB, 8>();
  if (wk <= 12) return kernel_of<G, VB, 12>();
  return kernel_of<G, VB, 16>();
}

template <int G>
DecodeKernel pick_vb(int vb, int wk) {
  switch (vb) {
    case 1: return pick_wk<G, 1>(wk);
    case 2: return pick_wk<G, 2>(wk);
    case 3: return pick_wk<G, 3>(wk);
    default: return pick_wk<G, 4>(wk);
  }
}

DecodeKernel pick_decode(int g, int vb, int wk) {
  switch (g) {
    case 1: return pick_vb<1>(vb, wk);
    case 2: return pick_vb<2>(vb, wk);
    case 4: return pick_vb<4>(vb, wk);
    default: return pick_vb<8>(vb, wk);
  }
}

// Workspace: the split partials [batch][hq][n_splits][kPartStride] f32.
struct DecodeLayout {
  int n_splits, tiles_base, tiles_extra;  // split s covers tiles_base + (s < tiles_extra) tiles
  size_t total;
};


DecodeLayout decode_layout(const Plan &p, int batch, int64_t max_seq_len) {
  DecodeLayout d{};
  const int tiles = (int)((max_seq_len + kTile - 1) / kTile);
  const int hkv = p.desc.n_kv_heads, hq = p.desc.n_q_heads;
  const DecodeKernel k = pick_decode(p.hdr.group, p.hdr.v_bits, p.hdr.wk);
  const int target = std::max(1, k.per_cu) * device_cus();  // one round of resident workgroups
  // (short sequences: at least one tile per wave, the latency-bound case
  // measured faster than two tiles per wave)
  int s = (target + batch * hkv - 1) / (batch * hkv);
  s = std::max(1, std::min({s, (tiles + k.waves - 1) / k.waves, kMaxSplits}));
  // tiles dealt out evenly: the first tiles % s splits take one tile more, so
  // that (with a multiple of the wave count per split) no wave but those of
  // the first splits has a tile more than the others
  d.n_splits = s;
  d.tiles_base = tiles / s;
  d.tiles_extra = tiles % s;
  d.total = (((size_t)batch * hq * d.n_splits * kPartStride * 4) + 255) & ~(size_t)255;
  return d;
}

// The decode kernels address LDS from offset 0: they must have no static LDS.
bool decode_static_lds_ok(decode_fn fn) {
  static std::mutex mu;
  static std::vector<decode_fn> checked;
  std::lock_guard<std::mutex> lk(mu);
  for (decode_fn f : checked)
    if (f == fn) return true;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, (const void *)fn) != hipSuccess || attr.sharedSizeBytes != 0) return false;
  checked.push_back(fn);
  return true;
}

float kscale_of(float softmax_scale) { return softmax_scale * 1.4426950408889634f; }  // logits in log2 units

bgtq_status decode_check(const Plan &p, int64_t capacity, int32_t batch, int64_t max_seq_len, float softmax_scale,
                         const void *workspace, size_t ws_bytes, const char *nm) {
  if (batch < 1 || batch > 65535) return fail(BGTQ_EINVAL, std::string(nm) + ": batch must be 1..65535");
  if (max_seq_len < 1 || max_seq_len > capacity)
    return fail(BGTQ_ECAPACITY, std::string(nm) + ": max_seq_len must be in [1, capacity]");
  if (max_seq_len > kMaxSeqLen) return fail(BGTQ_EINVAL, std::string(nm) + ": max_seq_len must be below 2^31 - 64");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(BGTQ_EINVAL, std::string(nm) + ": softmax_scale must be positive and finite");
  if ((uintptr_t)workspace & 255) return fail(BGTQ_EINVAL, std::string(nm) + ": workspace must be 256-byte aligned");
  if (ws_bytes < decode_layout(p, batch, max_seq_len).total)
    return fail(BGTQ_EWORKSPACE, std::string(nm) + ": workspace too small");
  return BGTQ_OK;
}

bgtq_status decode_launch(const Plan &p, const DecodeCall &c) {
  const DecodeLayout lay = decode_layout(p, c.batch, c.max_seq_len);
  const int G = p.hdr.group, vb = p.hdr.v_bits;
  const DecodeKernel k = pick_decode(G, vb, p.hdr.wk);
  const int smem = k.smem;
  decode_fn fn = k.fn;
  if (!decode_static_lds_ok(fn)) return fail(BGTQ_EDEVICE, "decode: kernel has static LDS");
  if (smem > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return fail(BGTQ_EDEVICE, "decode: LDS request above the limit");
  }
  hipStream_t st = (hipStream_t)c.stream;
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
        return fail(BGTQ_EDEVICE, "decode: event creation failed");
      }
    }
  }
  uint8_t *ws = (uint8_t *)c.workspace;
  DecodeArgs a;
  a.consts = (const uint8_t *)c.dev_consts;
  a.q = c.q;
  a.kc = c.k_codes;
  a.kn = c.k_norms;
  a.vc = c.v_codes;
  a.vn = c.v_norms;
  a.seq_lens = c.seq_lens;
  a.part = (float *)ws;
  const TileMap map = c.pages ? paged_map(p, c.pages) : contiguous_map(p.desc.n_kv_heads, c.capacity);
  a.table = map.table;
  a.head_stride = map.head_stride;
  a.seq_stride = map.seq_stride;
  a.max_pages = map.max_pages;
  a.n_pages = map.n_pages;
  a.max_seq_len = c.max_seq_len;
  a.off_kvh = p.hdr.off_kvh;
  a.off_dtab = p.hdr.off_dtab;
  a.off_vlut = p.hdr.off_vlut;
  a.off_zero = p.hdr.off_zero;
  a.hkv = p.desc.n_kv_heads;
  a.hq = p.desc.n_q_heads;
  a.wk = p.hdr.wk;
  a.tiles_base = lay.tiles_base;
  a.tiles_extra = lay.tiles_extra;
  a.n_splits = lay.n_splits;
  a.seq_add = c.seq_add;
  a.n_sink = c.n_sink;
  a.n_recent = c.n_recent;
  a.kscale = kscale_of(c.softmax_scale);
  const dim3 grid(lay.n_splits, p.desc.n_kv_heads, c.batch);
  // With profiling on, the events are bound to the launch itself, so their elapsed time is the
  // kernel's own start-to-end time (no queue packets of their own around the kernel).
  if (e0)
    hipExtLaunchKernelGGL(fn, grid, dim3(64 * k.waves), (uint32_t)smem, st, e0, e1, 0, a);
  else
    fn<<<grid, 64 * k.waves, smem, st>>>(a);
  const bgtq_status s = launch_status("decode");
  if (e1) {
    Prof &pr = prof();
    std::lock_guard<std::mutex> lk(pr.mu);
    pr.pending.emplace_back(e0, e1);
  }
  if (s != BGTQ_OK) return s;
  const float *pvt = (const float *)((const uint8_t *)c.dev_consts + p.hdr.off_rot32_v);
  const dim3 mgrid(p.desc.n_q_heads, c.batch);
  if (c.n_sink || c.n_recent) {
    const MergeBuf bf{c.q,        c.k_sink,      c.v_sink,    c.k_recent, c.v_recent, c.seq_lens,
                      c.max_seq_len, c.n_sink, c.n_recent, p.desc.n_kv_heads, c.seq_add, a.kscale};
    merge_kernel<true, true><<<mgrid, kMergeThreads, 0, st>>>(pvt, (const float *)ws, lay.n_splits, G,
                                                               p.desc.n_q_heads, c.out, bf);
  } else {
    merge_kernel<true><<<mgrid, kMergeThreads, 0, st>>>(pvt, (const float *)ws, lay.n_splits, G, p.desc.n_q_heads,
                                                        c.out, MergeBuf{});
  }
  return launch_status("decode (merge)");
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
  const bgtq_status v = decode_check(plan->p, capacity, batch, max_seq_len, softmax_scale, workspace, ws_bytes,
                                     "bgtq_decode_attn");
  if (v != BGTQ_OK) return v;
  DecodeCall c{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, seq_lens, 0, batch, max_seq_len,
               softmax_scale, out, workspace, stream};
  return decode_launch(plan->p, c);
}

bgtq_status bgtq_decode_attn_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                   const uint32_t *k_codes, const uint16_t *k_norms, const uint32_t *v_codes,
                                   const uint16_t *v_norms, const bgtq_pages *pages, const int32_t *seq_lens,
                                   int32_t batch, int64_t max_seq_len, float softmax_scale, uint16_t *out,
                                   void *workspace, size_t ws_bytes, bgtq_stream stream) {
  const char *nm = "bgtq_decode_attn_paged";
  if (!plan || !dev_consts || !q || !k_norms || !v_codes || !v_norms || !seq_lens || !out || !workspace ||
      (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  const bgtq_status ps = pages_check(pages, nm);
  if (ps != BGTQ_OK) return ps;
  const int64_t capacity = (int64_t)kTile * pages->max_pages;
  const bgtq_status v = decode_check(plan->p, capacity, batch, max_seq_len, softmax_scale, workspace, ws_bytes, nm);
  if (v != BGTQ_OK) return v;
  DecodeCall c{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, seq_lens, 0, batch, max_seq_len,
               softmax_scale, out, workspace, stream};
  c.pages = pages;
  return decode_launch(plan->p, c);
}

bgtq_status bgtq_decode_attn_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                      const uint32_t *k_codes, const uint16_t *k_norms, const uint32_t *v_codes,
                                      const uint16_t *v_norms, int64_t capacity, const int32_t *seq_lens,
                                      int32_t batch, int64_t max_seq_len, float softmax_scale,
                                      const uint16_t *k_sink, const uint16_t *v_sink, int32_t n_sink,
                                      const uint16_t *k_recent, const uint16_t *v_recent, int32_t n_recent,
                                      uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream) {
  const char *nm = "bgtq_decode_attn_buffered";
  if (!plan || !dev_consts || !q || !k_norms || !v_codes || !v_norms || !seq_lens || !out || !workspace ||
      (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (n_sink < 0 || n_sink > kMaxSink || n_recent < 0 || n_recent > kMaxRecent)
    return fail(BGTQ_EINVAL, std::string(nm) + ": n_sink must be 0..64 and n_recent 0..65536");
  if ((n_sink && (!k_sink || !v_sink)) || (n_recent && (!k_recent || !v_recent)))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null buffer with a non-zero count");
  if (((uintptr_t)k_sink | (uintptr_t)v_sink | (uintptr_t)k_recent | (uintptr_t)v_recent | (uintptr_t)q) & 15)
    return fail(BGTQ_EINVAL, std::string(nm) + ": q and the buffers must be 16-byte aligned");
  const bgtq_status v = decode_check(plan->p, capacity, batch, max_seq_len, softmax_scale, workspace, ws_bytes, nm);
  if (v != BGTQ_OK) return v;
  DecodeCall c{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, seq_lens, 0, batch, max_seq_len,
               softmax_scale, out, workspace, stream};
  c.k_sink = k_sink;
  c.v_sink = v_sink;
  c.k_recent = k_recent;
  c.v_recent = v_recent;
  c.n_sink = n_sink;
  c.n_recent = n_recent;
  return decode_launch(plan->p, c);
}

}  // extern "C"
