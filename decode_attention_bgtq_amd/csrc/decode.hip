// Fused decode attention over the packed Block-GTQ cache on gfx950 (the
// packed-cache serving path of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", Abstract, and of the Block-GTQ README backend table).
//
// Three launches per call.
//  prep_kernel    one workgroup of 8 waves per (KV head, sequence): the G
//                 queries rotated once per key width group (fp32 MFMA over the
//                 head's block-diagonal rotation, prep.h), scaled into the
//                 4-bit-group operands and the k-step operands of the
//                 width-1..3 groups, written as the decode kernel's register
//                 image (one 64-lane row per register).  In the serving step
//                 the same workgroups run beside the new token's append
//                 (step_front_kernel).
//  decode_kernel  one workgroup per CU (16 waves, or 12 where four waves per
//                 SIMD do not fit the registers) per (split of the sequence,
//                 KV head, sequence).  Prologue: the plan's decode tables into
//                 LDS (lookup rows), the query registers from the image, the
//                 first tiles requested.  Per 64-token tile (lane = token):
//                 key words read coalesced (word-major); logits on the matrix
//                 cores (the 4-bit group one fp32 4x4x1 step per code, or for
//                 eight heads split-fp16 16x16x32 products per 16 codes, the
//                 width-1..3 groups one fp16 4x4x4 k-step per four codes, all
//                 with LDS centroid lookups, the lookups of the next batch in
//                 flight during the products) times the group norms, in log2
//                 units; online softmax with wavefront reductions; the value
//                 codes (lane = coordinate) accumulated on the matrix cores
//                 against the fp16 softmax weights in the rotated value space.
//                 The waves of a workgroup merge into one partial
//                 (m, l, acc[128]) per query head.
//  merge_kernel   one workgroup per (query head, sequence): log-sum-exp merge
//                 of the splits, normalisation, un-rotation by Pi_V^T, fp16
//                 output.
// (Merging inside the decode kernel, by the last workgroup to arrive, costs
// more: its chain of device-coherent stores, atomics and loads sits on the
// critical path at the end of the grid.)
#include <hip/hip_ext.h>

#include "append.h"
#include "device.h"
#include "host.h"
#include "merge.h"
#include "prep.h"

namespace bgtq {

constexpr int64_t kMaxSeqLen = 0x7FFFFFFFLL - kTile;  // token positions of the decode fit 32 bits
constexpr float kRescaleSlack = 8.f;  // log2 units: softmax weights between rescales stay below 2^8
                                      // (less for value norms of 128 and above)


// Waves per SIMD the register allocation aims at: four (at most 128 VGPRs) up
// to four query heads per KV head unless the key and value words of two tiles
// and the query registers take too many registers, else three (at most 168);
// eight heads keep their query operands in LDS (QueryRegs below) to fit three,
// except with the widest tiles (two waves, query operands in registers).
template <int G, int VB, int WK>
struct StreamOcc {
  static constexpr bool four =
      G <= 4 && (VB <= 2 ? WK + 2 * VB <= 16 : WK + 2 * VB <= (G <= 2 ? 14 : 10));
  static constexpr int v = four ? 4 : (G <= 4 || VB <= 2 || WK + 2 * VB <= 18) ? 3 : 2;
  static constexpr bool qlds = G > 4 && v == 3;  // query operands in LDS
};

// Waves per workgroup: one workgroup per CU (one copy of the lookup rows per
// CU, every wave of the CU the same age), StreamOcc::v waves per SIMD.
template <int G, int VB, int WK>
struct StreamCfg {
  static constexpr int waves = 4 * StreamOcc<G, VB, WK>::v;
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
//   [0, 2560)        k-step tables of the plan: four fp16 centroids of a
//                    width-2 byte (t2) / width-1 nibble (t1), two of six
//                    width-3 bits (t3)
//   [rep, +64 KB)    lookup rows: row e (256 bytes) holds, in its first 128
//                    bytes, the value-table entry of index e once per lane
//                    slot (16 slots of 8 bytes, or 32 of 4 bytes) and, in its
//                    last 128 bytes, the 4-bit centroid pair of code byte e
//                    once per lane slot (16 slots of 8 bytes).  Lane l reads
//                    slot l mod 16 (32): the 16 (32) lanes that the LDS
//                    serves together read 16 (32) different bank pairs
//                    (banks), whatever their indices, so the random lookups
//                    take no bank conflicts; the row address is the code
//                    byte moved to bits 8..15 and the slot offset put below
//                    it, one v_perm_b32.
//   [vcomp, ..)      one-bit value table (16 bytes per code byte), VB = 1 only
//   [kw, ..)         per wave: the tile's key words [WK + 2][64] (the last two rows zero)
//   [qimg, ..)       query operands in LDS only: the (sequence, KV head)'s query
//                    register image (the preparation kernel's rows, read by
//                    each lane from its own column)
// The tables are copied (and replicated) from the plan's constant image in
// the prologue; after the tile loop the area from 0 is reused for the wave
// merge.
template <int G, int VB, int WK = kMaxWK>
struct StreamLds {
  static constexpr int t2 = 0, t1 = 2048, t3 = 2304, kt_bytes = 2560;
  static constexpr int rep = kt_bytes, rep_bytes = 256 * 256;
  static constexpr int vslot = VB == 2 ? 8 : 4;                 // bytes per value slot (VB 2..4)
  static constexpr int vcomp = rep + rep_bytes;
  static constexpr int W = StreamCfg<G, VB, WK>::waves;
  static constexpr int kw = vcomp + (VB == 1 ? VLut<1>::entries * VLut<1>::bytes : 0);
  static constexpr int kw_rows = WK + 2;  // key words of the tile, then two zero rows
  static constexpr bool qlds = StreamOcc<G, VB, WK>::qlds;
  static constexpr int qimg = kw + W * kw_rows * kTile * 4;
  static constexpr int qimg_bytes = qlds ? 3 * 2 * 2 * kTile * 8 + 256 + 8 * kTile * 16 : 0;
  static constexpr int end = qimg + qimg_bytes;
  static constexpr int merge = W * G * kPartStride * 4;
  static constexpr int total = end > merge ? end : merge;
  static constexpr int alloc = total;
  static_assert(t2 % 2048 == 0 && t1 % 128 == 0 && t3 % 256 == 0 && rep % 256 == 0, "table bases above the index bits");
  static_assert(rep < 65536, "lookup rows addressed by the instruction offset plus a 16-bit row address");
  static_assert(kw % 16 == 0 && qimg % 16 == 0, "16-byte aligned areas");
  static_assert(alloc <= 160 * 1024, "LDS of one CU");
};

// Row address of a lookup: code byte K of `word` at bits 8..15, the lane's
// slot offset `slot` (below 256) in bits 0..7 (v_perm_b32: result byte 0 is
// byte 0 of `slot`, byte 1 is byte K of `word`, bytes 2 and 3 are zero).
template <int K>
__device__ __forceinline__ uint32_t row_addr(uint32_t word, uint32_t slot) {
  return __builtin_amdgcn_perm(word, slot, 0x0C0C0400u | ((uint32_t)K << 8));
}

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
  uint32_t kwb;       // (16x16x32 4-bit group) of row lane / 32, token lane % 16 in those rows
  uint32_t vslot;     // this lane's slot offset in the value half of a lookup row
  uint32_t c4slot;    // this lane's slot offset in the centroid-pair half of a lookup row
  uint32_t cgrp;      // first k-step of the width-3, 2, 1 groups (bytes 0..2), k-step count (byte 3)
  uint32_t gbit;      // first stream bit of the width-3, 2, 1 groups (10 bits each)
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

// The prepared queries of the tile loop.  The matrix-core A operands are
// broadcast from one block of 4 lanes to all 16 (CBSZ 4, ABID b), so one
// register holds the operands of 16 steps:
//  q4[k][g]     lane 4b + m: head 4g + m's scaled query of 4-bit code 16k + b
//  kq[r][j][g]  lane 4b + m: head 4g + m's four fp16 query values of k-step
//               16j + b of the width-(3 - r) group
// They stay in registers for the whole loop (L false), or (eight heads at three
// waves per SIMD) are read from the image in LDS next to their use, which
// leaves the registers of the third wave; those kernels take the 4-bit group
// on the 16x16x32 matrix cores (key4_wide) instead of the q4 steps.
template <int G, bool L>
struct QueryRegs;

template <int G>
struct QueryRegs<G, false> {
  static constexpr int VQ = VQuads<G>::v;
  float q4[8][VQ];
  h4v kq[3][2][VQ];
};

template <int G>
struct QueryRegs<G, true> {
  uint32_t kqa;  // LDS byte address of the lane's column of kq[0][0][0]
  uint32_t qaa;  // LDS byte address of the lane's qa operand of chunk 0
};

template <int G, int K>
__device__ __forceinline__ void query_q4(const QueryRegs<G, false> &qr, float (&o)[VQuads<G>::v]) {
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g) o[g] = qr.q4[K][g];
}

template <int G, int R>
__device__ __forceinline__ void query_kq(const QueryRegs<G, false> &qr, h4v (&o)[2][VQuads<G>::v]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int g = 0; g < VQuads<G>::v; ++g) o[j][g] = qr.kq[R][j][g];
}

template <int G, int R>
__device__ __forceinline__ void query_kq(const QueryRegs<G, true> &qr, h4v (&o)[2][VQuads<G>::v]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int g = 0; g < VQuads<G>::v; ++g)
      o[j][g] = *(const __attribute__((address_space(3))) h4v *)(size_t)(qr.kqa +
                                                                      ((2 * R + j) * VQuads<G>::v + g) * kTile * 8);
}

// Key word J holds codes 8 J .. 8 J + 7, two per byte (low nibble first).  The
// words are pipelined: the four lookups of word J + 1 are issued before the
// products of word J.  A lookup reads the centroid pair of its code byte from
// the lane's slot of the byte's lookup row.
template <int G, int VB, int WK, int J>
__device__ __forceinline__ void key4_lookups(const uint32_t (&w)[WK], uint32_t c4slot, float2 (&cp)[4]) {
  typedef StreamLds<G, VB, WK> L;
  const uint32_t word = w[J];
  cp[0] = lds_at<float2>(L::rep + row_addr<0>(word, c4slot));
  cp[1] = lds_at<float2>(L::rep + row_addr<1>(word, c4slot));
  cp[2] = lds_at<float2>(L::rep + row_addr<2>(word, c4slot));
  cp[3] = lds_at<float2>(L::rep + row_addr<3>(word, c4slot));
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

// Word J (< n4w) with its lookups in cx and its query operands in qx; word
// J + 1's go to cy and qy.
template <int G, int VB, int WK, int J, class QR>
__device__ __forceinline__ void key4_words(const uint32_t (&w)[WK], int n4w, uint32_t c4slot, float2 (&cx)[4],
                                           float2 (&cy)[4], float (&qx)[VQuads<G>::v], float (&qy)[VQuads<G>::v],
                                           const QR &qr, f4v (&a4)[VQuads<G>::v]) {
  if constexpr (J < WK) {
    if (J < n4w) {
      if constexpr (J + 1 < WK) {
        key4_lookups<G, VB, WK, J + 1>(w, c4slot, cy);
        query_q4<G, ((J + 1) >> 1) & 7>(qr, qy);
      }
      __builtin_amdgcn_sched_barrier(0);
      key4_products<G, J>(cx, qx, a4);
      __builtin_amdgcn_sched_barrier(0);
      key4_words<G, VB, WK, J + 1>(w, n4w, c4slot, cy, cx, qy, qx, qr, a4);
    }
  }
}

// 4-bit group on the matrix cores, one v_mfma_f32_4x4x1f32 per code r (16 blocks
// of 4 x 4 x 1): block k is lanes 4k .. 4k + 3 = tokens 4k .. 4k + 3, its B operand
// the token's centroid c4[code_r] and its output row m head m, so the token's
// lane keeps a4[h] in register h.  The A operand, head m's query value of
// code r, is broadcast from block r % 16 of q4[r / 16] (CBSZ 4, ABID r % 16).
template <int G, int VB, int WK, class QR>
__device__ __forceinline__ void key4_group(const uint32_t (&w)[WK], int n4w, uint32_t c4slot, const QR &qr,
                                           f4v (&a4)[VQuads<G>::v]) {
  if (n4w > 0) {
    float2 cx[4], cy[4];
    float qx[VQuads<G>::v], qy[VQuads<G>::v];
    key4_lookups<G, VB, WK, 0>(w, c4slot, cx);
    query_q4<G, 0>(qr, qx);
    key4_words<G, VB, WK, 0>(w, n4w, c4slot, cx, cy, qx, qy, qr, a4);
  }
}

// 4-bit group of the eight-head kernels that read their query operands from
// LDS, on the 16x16x32 fp16 matrix cores with the query and the centroid each
// split into two fp16 parts, q = q_hi + q_lo (q scaled per head by a power of
// two into fp16 range) and c = c_hi + c_lo: q_hi c_hi + q_hi c_lo + q_lo c_hi
// keeps ~22 bits of every product (the logits of the widest group need more
// than fp16 operands give), at a quarter of the fp32 steps' matrix-core time.
// Per chunk of 16 codes and token group tg (tokens 16 tg .. 16 tg + 15), one
// product D += A B:
//  A (16 x 32, the chunk's qa operand from the image in LDS): row 4r + j is
//    head 2r + j / 2 with part j % 2 (q_hi, q_lo); k-slots 8 kb .. 8 kb + 7
//    are codes 8 (kb / 2) .. + 7 of the chunk against c_hi (kb even) or c_lo
//    (kb odd), where the q_lo rows are zero;
//  B (32 x 16): lane 16 kb + n holds token 16 tg + n's key word 2 chunk + kb / 2
//    (from this wave's key-word rows in LDS), its four code bytes looked up as
//    fp16 pairs, c_hi or c_lo by the lane's slot (the two halves of an 8-byte
//    lookup slot);
//  D: lane 16 r + n, register j: head 2r + j / 2, part j % 2, token 16 tg + n.
// The parts are added in the lane; two 4 x 4 transposes of 16-lane row blocks
// over the four token groups (permlane16 / permlane32 swaps) then put head h
// of token t into lane t (a4[h / 4][h % 4]), the layout of the other groups.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void rows_transpose(float (&x)[4]) {
  uint32_t a0 = __builtin_bit_cast(uint32_t, x[0]), a1 = __builtin_bit_cast(uint32_t, x[1]);
  uint32_t a2 = __builtin_bit_cast(uint32_t, x[2]), a3 = __builtin_bit_cast(uint32_t, x[3]);
  auto p = __builtin_amdgcn_permlane16_swap(a0, a1, false, false);
  a0 = p[0], a1 = p[1];
  p = __builtin_amdgcn_permlane16_swap(a2, a3, false, false);
  a2 = p[0], a3 = p[1];
  p = __builtin_amdgcn_permlane32_swap(a0, a2, false, false);
  a0 = p[0], a2 = p[1];
  p = __builtin_amdgcn_permlane32_swap(a1, a3, false, false);
  a1 = p[0], a3 = p[1];
  x[0] = __builtin_bit_cast(float, a0), x[1] = __builtin_bit_cast(float, a1);
  x[2] = __builtin_bit_cast(float, a2), x[3] = __builtin_bit_cast(float, a3);
}

template <class L>
__device__ __forceinline__ h8v wide_b(uint32_t word, uint32_t slot) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 v = {lds_at<uint32_t>(L::rep + row_addr<0>(word, slot)), lds_at<uint32_t>(L::rep + row_addr<1>(word, slot)),
                lds_at<uint32_t>(L::rep + row_addr<2>(word, slot)), lds_at<uint32_t>(L::rep + row_addr<3>(word, slot))};
  return __builtin_bit_cast(h8v, v);
}

// kwb: LDS byte address of (row lane / 32, token lane % 16) of this wave's key
// words; qaa: of the lane's qa operand of chunk 0; slot: the lane's lookup slot.
template <int G, int VB, int WK>
__device__ __forceinline__ void key4_wide(int n4w, uint32_t kwb, uint32_t qaa, uint32_t slot, f4v (&a4)[2]) {
  typedef StreamLds<G, VB, WK> L;
  f4v acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = (f4v){0.f, 0.f, 0.f, 0.f};
  const int nch = (n4w + 1) >> 1;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c >= nch) break;
    const h8v a = *(const __attribute__((address_space(3))) h8v *)(size_t)(qaa + c * 64 * 16);
    uint32_t wd[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wd[t] = lds_at<uint32_t>(kwb + c * 512 + t * 64);
    h8v bb[2];  // B operands of token groups t (in use) and t + 1 (in flight)
    bb[0] = wide_b<L>(wd[0], slot);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 1 < 4) bb[(t + 1) & 1] = wide_b<L>(wd[t + 1], slot);
      __builtin_amdgcn_sched_barrier(0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb[t & 1], acc[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float u0[4], u1[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) u0[t] = acc[t][0] + acc[t][1], u1[t] = acc[t][2] + acc[t][3];
  rows_transpose(u0);  // u0[r]: head 2r
  rows_transpose(u1);  // u1[r]: head 2r + 1
  a4[0] = (f4v){u0[0], u1[0], u0[1], u1[1]};
  a4[1] = (f4v){u0[2], u1[2], u0[3], u1[3]};
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
                                             const h4v (&kq)[2][VQuads<G>::v], int ns, f4v (&acc)[VQuads<G>::v]) {
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
      acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(kq[S >> 4][g], bq, acc[g], 4, S & 15, 0);
    kgroup_steps<G, VB, W, S + 1>(wd, al, wa, sh, kq, ns, acc);
  }
}

// The k-steps of the width-(3 - R) group; the query operand of k-step S is
// broadcast from block S % 16 of kq[R][S / 16].
template <int G, int VB, int WK, int R, class QR>
__device__ __forceinline__ void key_group(const StreamState &st, const QR &qr, f4v (&acc)[VQuads<G>::v]) {
  constexpr int W = 3 - R;
  const int cb = (st.cgrp >> (8 * R)) & 255, ce = (st.cgrp >> (8 * R + 8)) & 255;
  if (cb >= ce) return;
  const uint32_t bit = (st.gbit >> (10 * R)) & 1023u;
  const uint32_t wa = st.kwl + (bit >> 5) * 256;
  uint32_t wd[14], al[13];
  wd[0] = lds_at<uint32_t>(wa);
  h4v kq[2][VQuads<G>::v];
  query_kq<G, R>(qr, kq);
  // The k-step count is opaque per tile, so that the compiler evaluates each
  // k-step's guard where it is used instead of keeping all of them live.
  int ns = ce - cb;
  asm volatile("" : "+s"(ns));
  kgroup_steps<G, VB, W, 0>(wd, al, wa, bit & 31u, kq, ns, acc);
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
// 4 VB (S + 1) of the coordinate's code stream), from the lane's slot of the
// lookup rows (VB 2..4; `slot` is the lane's slot offset) or from the compact
// one-bit table.
template <class L, int VB, int S>
__device__ __forceinline__ h4v v_operand(const uint32_t (&c)[2 * VB], uint32_t slot) {
  if constexpr (VB == 1) {  // entry = one byte (8 tokens) x 16 bytes
    const uint32_t y = (c[S >> 3] >> (8 * ((S >> 1) & 3))) & 255u;
    return lds_at<h4v>(L::vcomp + 16 * y + 8 * (S & 1));
  } else if constexpr (VB == 2) {  // row = one byte (4 tokens), 8-byte slots
    return lds_at<h4v>(L::rep + row_addr<S & 3>(c[S >> 2], slot));
  } else if constexpr (VB == 3) {  // row = 6 bits (2 tokens), 4-byte slots
    const uint32_t y0 = bits6<12 * S>(c), y1 = bits6<12 * S + 6>(c);
    return __builtin_bit_cast(h4v, (u2v){lds_at<uint32_t>(L::rep + ((y0 << 8) | slot)),
                                         lds_at<uint32_t>(L::rep + ((y1 << 8) | slot))});
  } else {  // row = one byte (2 tokens), 4-byte slots
    return __builtin_bit_cast(h4v, (u2v){lds_at<uint32_t>(L::rep + row_addr<2 * (S & 1)>(c[S >> 1], slot)),
                                         lds_at<uint32_t>(L::rep + row_addr<2 * (S & 1) + 1>(c[S >> 1], slot))});
  }
}

// The 16 steps in batches of kVBatch: the lookups of batch k + 1 are issued
// before the products of batch k, so that the wave keeps 2 kVBatch lookups in
// flight instead of waiting for each one.
constexpr int kVBatch = 4;

template <class L, int VB, int S, int N>
__device__ __forceinline__ void v_lookups(const uint32_t (&va)[2 * VB], const uint32_t (&vb)[2 * VB], uint32_t slot,
                                          h4v (&b0)[kVBatch], h4v (&b1)[kVBatch]) {
  if constexpr (N < kVBatch) {
    b0[N] = v_operand<L, VB, S + N>(va, slot);
    b1[N] = v_operand<L, VB, S + N>(vb, slot);
    v_lookups<L, VB, S, N + 1>(va, vb, slot, b0, b1);
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
template <int G, class L, int VB, int S>
__device__ __forceinline__ void v_mfma_steps(const uint32_t (&va)[2 * VB], const uint32_t (&vb)[2 * VB], uint32_t slot,
                                             const h4v (&pa)[VQuads<G>::v], h4v (&x0)[kVBatch],
                                             h4v (&x1)[kVBatch], h4v (&y0)[kVBatch], h4v (&y1)[kVBatch],
                                             f4v (&acc0)[VQuads<G>::v], f4v (&acc1)[VQuads<G>::v]) {
  if constexpr (S < kTile / 4) {
    if constexpr (S + kVBatch < kTile / 4) v_lookups<L, VB, S + kVBatch, 0>(va, vb, slot, y0, y1);
    __builtin_amdgcn_sched_barrier(0);
    v_products<G, S, 0>(x0, x1, pa, acc0, acc1);
    __builtin_amdgcn_sched_barrier(0);
    v_mfma_steps<G, L, VB, S + kVBatch>(va, vb, slot, pa, y0, y1, x0, x1, acc0, acc1);
  }
}

template <int G, int VB, int WK, class QR>
__device__ __forceinline__ void process_tile(const TileRegs<VB, WK> &r, int tile, const StreamState &st,
                                             const QR &qr, const float (&rinv)[G], const float (&rinv4)[G],
                                             float (&mrun)[G],
                                             float (&mth)[G], float (&lsum)[G], f4v (&acc0)[VQuads<G>::v],
                                             f4v (&acc1)[VQuads<G>::v], int lane) {
  // ---- keys, lane = token.  4-bit group: one fp32 step per code, or (query
  // operands in LDS) the split-fp16 16x16x32 products from the staged words.
  // The key words are staged in this wave's LDS rows for the k-steps of
  // widths 3, 2, 1 (norm slots 1, 2, 3): lr = sum_w n_w acc_w.
  constexpr bool kWide = StreamLds<G, VB, WK>::qlds;
  f4v a4[VQuads<G>::v];
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g) a4[g] = (f4v){0.f, 0.f, 0.f, 0.f};
  if constexpr (!kWide) key4_group<G, VB, WK>(r.w, st.n4w, st.c4slot, qr, a4);
#pragma unroll
  for (int j = 0; j < WK; ++j)
    *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * j) = r.w[j];
  if constexpr (kWide) key4_wide<G, VB, WK>(st.n4w, st.kwb, qr.qaa, st.c4slot, a4);
  float lr[G];
  {
    f4v ak[VQuads<G>::v];
#define BGTQ_KG(R, NORM)                                                              \
  {                                                                                   \
    _Pragma("unroll") for (int g = 0; g < VQuads<G>::v; ++g) ak[g] = (f4v){0.f, 0.f, 0.f, 0.f}; \
    key_group<G, VB, WK, R>(st, qr, ak);                                              \
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
  // accumulators) only when a logit exceeds it by more than the token's
  // slack, kRescaleSlack less dv = clamp(E - 21, 0, 8) for the exponent field
  // E of the token's fp16 value norm.  Without a rescale p = 2^(l - m) stays
  // below 2^(8 - dv), so P' = p * value norm stays below 2^15 (the norm is
  // below 2^(E - 14)); after one, p <= 1 and P' <= the norm.  So the fp16
  // operand P' is finite for every finite norm.
  const float dv = (float)min(max((int)((r.nv >> 10) & 31u) - 21, 0), 8);
  float l[G];
  bool up = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = valid ? fmaf(kWide ? n4 * rinv4[h] : n4, a4[h >> 2][h & 3], lr[h] * rinv[h]) : -INFINITY;
    up = up || l[h] + dv > mth[h];
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
  _Float16 pw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p = __builtin_amdgcn_exp2f(l[h] - mrun[h]);
    lsum[h] += p;
    pw[h] = (_Float16)(p * nv);
  }
  // A operands: lane 4k + m holds head m's weights of tokens 4k .. 4k + 3 (heads
  // past G repeat a valid row; their output rows are never read): the 4 x 4
  // block (token, head) of a lane quad transposed, first the 2 x 2 blocks
  // within lane pairs, then the pairs across the quad
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
  const bool lo2 = (lane & 2) == 0;
  h4v pa[VQuads<G>::v];
#pragma unroll
  for (int g = 0; g < VQuads<G>::v; ++g) {
    const uint32_t d0 = __builtin_bit_cast(uint32_t, (h2v){pw[(4 * g) & (G - 1)], pw[(4 * g + 1) & (G - 1)]});
    const uint32_t d1 = __builtin_bit_cast(uint32_t, (h2v){pw[(4 * g + 2) & (G - 1)], pw[(4 * g + 3) & (G - 1)]});
    const uint32_t n0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    const uint32_t n1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, true);
    const uint32_t e0 = __builtin_amdgcn_perm(n0, d0, sel), e1 = __builtin_amdgcn_perm(n1, d1, sel);
    const uint32_t p0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)e0, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)e1, 0x4E, 0xF, 0xF, true);
    pa[g] = __builtin_bit_cast(h4v, (u2v){lo2 ? e0 : p1, lo2 ? p0 : e1});
  }
  // ---- values: lane = coordinates lane and lane + 64
  typedef StreamLds<G, VB, WK> L;
  h4v x0[kVBatch], x1[kVBatch], y0[kVBatch], y1[kVBatch];
  v_lookups<L, VB, 0, 0>(r.va, r.vb, st.vslot, x0, x1);
  v_mfma_steps<G, L, VB, 0>(r.va, r.vb, st.vslot, pa, x0, x1, y0, y1, acc0, acc1);
}


// ------------------------------------------------------------------ query preparation

// The decode kernel's query registers (QueryRegs) of one (sequence, KV head)
// as the preparation kernel writes them to the workspace: one 64-lane row per
// register, so that the decode kernel loads each register with one coalesced
// load whose address does not depend on loaded data.
//
// Eight heads also get the 4-bit group as the A operands of the 16x16x32 fp16
// products (qa, see key4_wide); the kernels that keep their query operands in
// LDS copy the image up to q4 (kq, the scales and qa) and read the rest of
// their operands there.
template <int G>
struct QueryImage {
  static constexpr int VQ = VQuads<G>::v;
  static constexpr bool wide = G == 8;
  static constexpr int kq = 0;                               // h4v [3][2][VQ][64]
  static constexpr int rinv = kq + 3 * 2 * VQ * kTile * 8;   // float [G]: 1 / the k-step operands' scale;
  static constexpr int rinv4 = rinv + 128;                   // float [G]: 1 / the qa operands' scale
  static constexpr int qa = rinv + 256;                      // (eight heads) fp16 [8 chunks][64][8]
  static constexpr int q4 = qa + (wide ? 8 * kTile * 16 : 0);  // float [8][VQ][64]
  static constexpr int bytes = q4 + 8 * VQ * kTile * 4;
  static constexpr int lds_bytes = q4;
  static_assert(bytes % 256 == 0 && G <= 32, "256-byte slots");
};

constexpr int kPrepWaves = 8;

struct PrepArgs {
  const uint8_t *consts;
  const uint16_t *q;
  int hq, hkv, gr;  // gr: query heads per KV head (at most G)
  int64_t off_zero;
  float kscale;
  uint8_t *images;
};

// The G queries of (KV head, sequence) rotated once per key width group and
// scaled (prep.h, in LDS), then rearranged into the register image of the
// pair's slot; 8 waves.
template <int G>
__device__ __forceinline__ void prep_role(const PrepArgs &pa, int kvh, int b) {
  typedef PrepOut<G> PO;
  typedef QueryImage<G> QI;
  constexpr int VQ = VQuads<G>::v, T = 64 * kPrepWaves;
  __shared__ __attribute__((aligned(16))) uint8_t out[PO::bytes];
  __shared__ __attribute__((aligned(16))) uint8_t scr[PrepScratch<G>::bytes];
  const uint8_t *consts = pa.consts;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  PrepIn<G, kPrepWaves> pin;
  prep_issue_keys<G, kPrepWaves>(pin, consts, kvh, wave, lane);
  prep_issue<G, kPrepWaves>(pin, consts, kvh, pa.q + ((size_t)b * pa.hq + (size_t)kvh * pa.gr) * kHeadDim, pa.gr,
                            tid, wave, lane);
  prep_issue_rot<G, kPrepWaves>(pin, consts, pa.off_zero, kvh, wave, lane);
  prep_stage<G, kPrepWaves>(pin, out, scr, tid);
  prep_build<G, kPrepWaves>(pin, out, scr, pa.kscale, tid, wave, lane);  // ends with a barrier
  const KvhDesc &kds = *(const KvhDesc *)(scr + PrepScratch<G>::kds);
  uint8_t *img = pa.images + ((size_t)b * pa.hkv + kvh) * QI::bytes;
  // q4[k][g][l]: head 4g + (l & 3) (repeating a valid head past G), code 16k + l / 4
  for (int i = tid; i < 8 * VQ * kTile; i += T) {
    const int l = i & 63, g = (i >> 6) % VQ, k = (i >> 6) / VQ;
    const int h = (4 * g + (l & 3)) & (G - 1);
    ((float *)(img + QI::q4))[i] = ((const float *)(out + PO::q4))[h * kHeadDim + 16 * k + (l >> 2)];
  }
  // kq[r][j][g][l]: k-step 16j + l / 4 of the width-(3 - r) group, head 4g + (l & 3)
  for (int i = tid; i < 6 * VQ * kTile; i += T) {
    const int l = i & 63, g = (i >> 6) % VQ, rj = (i >> 6) / VQ, r = rj >> 1, j = rj & 1;
    const int cb = (int)((kds.cgrp >> (8 * r)) & 255u);
    const int k = min(cb + 16 * j + (l >> 2), kMaxKSteps - 1);
    ((uint2 *)(img + QI::kq))[i] = ((const uint2 *)(out + PO::qr))[(k * VQ + g) * 4 + (l & 3)];
  }
  if (tid < G) ((float *)(img + QI::rinv))[tid] = ((const float *)(out + PO::rinv))[tid];
  if constexpr (QI::wide) {
    // qa: the 4-bit group as the 16x16x32 A operands (key4_wide), head h's
    // values scaled by the power of two fac[h] that brings their largest
    // magnitude to [2^13, 2^14) and split as q = q_hi + q_lo in fp16.
    // Wave h finds head h's scale (eight waves, eight heads).
    static_assert(kPrepWaves == G, "one wave per head");
    float *fac = (float *)(scr + PrepScratch<G>::hm);
    const float *q4 = (const float *)(out + PO::q4);
    const float m = wave_max(fmaxf(fabsf(q4[wave * kHeadDim + lane]), fabsf(q4[wave * kHeadDim + lane + 64])));
    int e = 0;
    (void)frexpf(m, &e);
    e = m > 0.f ? e : 0;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
    if (lane == 0) {
      fac[wave] = ldexpf(1.f, 14 - e);
      ((float *)(img + QI::rinv4))[wave] = ldexpf(1.f, e - 14);
    }
    __syncthreads();
    // element i = (chunk c, lane l, e): row l % 16 = 4r + j is head 2r + j / 2,
    // part j % 2; k-slot 8 (l / 16) + e is code 16 c + 8 (l / 32) + e against
    // c_hi (l / 16 even) or c_lo (odd; the q_lo rows are zero there)
    // (one 16-byte operand per thread and round)
    for (int i = tid; i < 8 * kTile; i += T) {
      const int l = i & 63, c = i >> 6;
      const int row = l & 15, kb = l >> 4;
      const int h = 2 * (row >> 2) + ((row >> 1) & 1);
      const float f = fac[h];
      const float *src = q4 + h * kHeadDim + 16 * c + 8 * (kb >> 1);
      h8v o;
#pragma unroll
      for (int el = 0; el < 8; ++el) {
        const float v = src[el] * f;
        const _Float16 hi = (_Float16)v, lo = (_Float16)(v - (float)hi);
        o[el] = (row & 1) == 0 ? hi : ((kb & 1) ? (_Float16)0.f : lo);
      }
      ((h8v *)(img + QI::qa))[i] = o;
    }
  }
}

// One workgroup per (KV head, sequence).
template <int G>
__global__ __launch_bounds__(64 * kPrepWaves) void prep_kernel(const PrepArgs pa) {
  prep_role<G>(pa, blockIdx.x, blockIdx.y);
}

static_assert(kAppendThreads == 64 * kPrepWaves, "one workgroup size for all roles");

// The buffered step's copy of the new token of sequence b into the fp16 sink
// (row pos[b] when below n_sink) and recent window (ring row pos[b] %
// n_recent); a sequence with pos[b] < 0 copies nothing.
struct BufCopy {
  const uint4 *k, *v;  // [batch][hkv][128] fp16, 16-byte chunks
  uint4 *k_sink, *v_sink, *k_recent, *v_recent;
  int n_sink, n_recent;
};

__device__ __forceinline__ void buffer_copy_role(const BufCopy &bc, const int32_t *__restrict__ pos, int hkv, int b) {
  const int64_t t = pos[b];
  if (t < 0) return;  // uniform per workgroup
  const int per = hkv * (kHeadDim / 8);
  for (int c = threadIdx.x; c < per; c += blockDim.x) {
    const int h = c / (kHeadDim / 8), w = c % (kHeadDim / 8);
    const uint4 kx = bc.k[(size_t)b * per + c], vx = bc.v[(size_t)b * per + c];
    if (t < bc.n_sink) {
      const size_t dst = (((size_t)b * hkv + h) * bc.n_sink + t) * (kHeadDim / 8) + w;
      bc.k_sink[dst] = kx;
      bc.v_sink[dst] = vx;
    }
    if (bc.n_recent > 0) {
      const size_t dst = (((size_t)b * hkv + h) * bc.n_recent + (size_t)(t % bc.n_recent)) * (kHeadDim / 8) + w;
      bc.k_recent[dst] = kx;
      bc.v_recent[dst] = vx;
    }
  }
}

// The front of a serving step in one launch: the new token's key and value
// appended to the cache and the queries prepared, side by side (the two are
// independent; the decode kernel after them needs both).  Workgroups [0, n):
// key append of (sequence, KV head) = (r / hkv, r % hkv); [n, 2n): value
// append; [2n, 3n): query preparation.  n = batch * hkv.  A buffered step adds
// [3n, 3n + batch): the fp16 buffer copy of sequence role - 3n (read only by
// the merge, two launches later).
template <int G>
__global__ __launch_bounds__(64 * kPrepWaves) void step_front_kernel(const PrepArgs pa, const AppendArgs ka,
                                                                     const AppendArgs va,
                                                                     const int32_t *__restrict__ pos,
                                                                     int64_t capacity, int n, const BufCopy bc) {
  const int role = blockIdx.x, hkv = ka.hkv;
  if (role >= 3 * n) {
    buffer_copy_role(bc, pos, hkv, role - 3 * n);
    return;
  }
  const int r = role < n ? role : role < 2 * n ? role - n : role - 2 * n;
  const int kvh = r % hkv, b = r / hkv;
  if (role >= 2 * n) {
    prep_role<G>(pa, kvh, b);
    return;
  }
  const int64_t t = pos[b];
  if (t < 0 || t >= capacity) return;  // uniform per workgroup
  const int64_t tile = t / kTile;
  const int lo = (int)(t - tile * kTile);
  if (role < n) {
    if (ka.wk > 0) append_role<false>(ka, tile, kvh, b, lo, lo + 1, b);
  } else {
    append_role<true>(va, tile, kvh, b, lo, lo + 1, b);
  }
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
  const uint8_t *qimg;   // prepared query registers [batch][hkv] (QueryImage)
  const int32_t *table;  // paged pools: block table [batch][max_pages], else null
  int64_t head_stride, seq_stride;  // tile index = kvh * head_stride + b * seq_stride + page
  int max_pages, n_pages;
  int64_t max_seq_len, off_kvh, off_dtab, off_vlut, off_zero;
  int hkv, hq, wk, tiles_base, tiles_extra, n_splits;  // split s: tiles_base + (s < tiles_extra) tiles
  int group;  // query heads per KV head (at most the kernel's G: the rows past it are not written)
  int seq_add;  // sequence length = seq_lens[b] + seq_add (1 when seq_lens holds the new token's position)
  int n_sink, n_recent;  // tokens [0, n_sink) and [T - n_recent, T) are served from fp16 buffers, not here
  float kscale;  // softmax scale in log2 units
};

// Issue priority of a wave from the tiles it has left after the current one.
// The SIMD's arbiter favours older waves, so at equal priority the four waves
// of a SIMD finish one after another (about 1.6 us apart at the 128K layer)
// and the last ones run alone, unable to fill the SIMD; a wave that is behind
// gets the higher priority, so that the waves of a SIMD finish together.
__device__ __forceinline__ void wave_priority(int rem) {
  if (rem >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (rem == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (rem == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

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

  // ---- prologue: every load first, none of them addressed from loaded data
  // (loads complete in order, so waiting for an earlier group does not wait
  // for a later one): the plan's tables, this (sequence, KV head)'s prepared
  // query registers, then the wave's first tile.  The tables go into LDS as
  // soon as they arrive; after the barrier the second tile is requested.
  // (Requesting both tiles at once queues every wave's table loads behind
  // twice the tile traffic: the barrier came 2 us later at the 128K layer.)
  const int64_t seq_raw = (int64_t)a.seq_lens[b] + a.seq_add;
  const int n4w = kd->n4w;
  const uint32_t cgrp = kd->cgrp, gbit = kd->gbit;
  // the plan's tables: the compact k-step tables (bytes 2048 .. 4608 of the
  // image's decode tables: t2, t1, t3) and, for each lookup row, the entry to
  // replicate into its slots -- thread (row e, part p): p 0, 1 the value-table
  // entry e (VB 2..4), p 2, 3 the 4-bit centroid pair of code byte e
  constexpr int kRowRounds = (256 * 4 + kStreamThreads - 1) / kStreamThreads;
  constexpr int kVEntries = VLut<VB>::entries;
  const uint8_t *dtab = consts + a.off_dtab, *vtab = consts + a.off_vlut;
  const uint4 ktab = *((const uint4 *)(dtab + 2048) + min(tid, Lds::kt_bytes / 16 - 1));
  uint2 rsrc[kRowRounds];
#pragma unroll
  for (int rr = 0; rr < kRowRounds; ++rr) {
    const int e = min((tid >> 2) + rr * (kStreamThreads / 4), 255), part = tid & 3;
    if (part >= 2)
      rsrc[rr] = *(const uint2 *)(dtab + 8 * e);
    else if constexpr (VB == 2)
      rsrc[rr] = *(const uint2 *)(vtab + 8 * e);
    else if constexpr (VB >= 3)
      rsrc[rr] = make_uint2(*(const uint32_t *)(vtab + 4 * min(e, kVEntries - 1)), 0u);
    else
      rsrc[rr] = make_uint2(0u, 0u);
  }
  uint4 vcomp = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (VB == 1) vcomp = *((const uint4 *)vtab + min(tid, kVEntries - 1));
  // the prepared query registers (QueryRegs), one coalesced row per register
  constexpr int VQ = VQuads<G>::v;
  typedef QueryImage<G> QI;
  const uint8_t *img = a.qimg + ((size_t)b * a.hkv + kvh) * QI::bytes;
  QueryRegs<G, Lds::qlds> qr;
  constexpr int kImg16 = Lds::qimg_bytes / 16;  // 16-byte pieces of the image copied to LDS (eight heads)
  constexpr int kImgRounds = (kImg16 + kStreamThreads - 1) / kStreamThreads;
  static_assert(kImgRounds <= 2, "two rounds of image loads");
  uint4 qimg0 = make_uint4(0u, 0u, 0u, 0u), qimg1 = qimg0;  // (scalars: an array of them went to scratch)
  if constexpr (Lds::qlds) {
    static_assert(QI::lds_bytes == Lds::qimg_bytes && QI::wide, "query image in LDS");
    qimg0 = ((const uint4 *)img)[min(tid, kImg16 - 1)];
    if constexpr (kImgRounds > 1) qimg1 = ((const uint4 *)img)[min(tid + kStreamThreads, kImg16 - 1)];
    qr.kqa = (uint32_t)(Lds::qimg + QI::kq + lane * 8);
    qr.qaa = (uint32_t)(Lds::qimg + QI::qa + lane * 16);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int g = 0; g < VQ; ++g) qr.q4[k][g] = ((const float *)(img + QI::q4))[(k * VQ + g) * kTile + lane];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < VQ; ++g)
          qr.kq[r][j][g] =
              __builtin_bit_cast(h4v, ((const uint2 *)(img + QI::kq))[((2 * r + j) * VQ + g) * kTile + lane]);
  }
  float rinv[G], rinv4[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    rinv[h] = ((const float *)(img + QI::rinv))[h];
    rinv4[h] = Lds::qlds ? ((const float *)(img + QI::rinv4))[h] : 1.f;
  }
  // ---- tiles of this wave: tile_lo + wave, + W, ... (W waves); two in flight
  // in registers, their range bounded by max_seq_len (in memory)
  const int tile_lo = split * a.tiles_base + min(split, a.tiles_extra);
  const int tile_end =
      min(tile_lo + a.tiles_base + (split < a.tiles_extra ? 1 : 0), (int)((a.max_seq_len + kTile - 1) / kTile));
  // tile index = head_base + page; page = tile (contiguous) or the block
  // table's entry (paged; clamped into the pool)
  const size_t head_base = (size_t)kvh * a.head_stride + (size_t)b * a.seq_stride;
  const bool paged = a.table != nullptr;
  const int32_t *btab = paged ? a.table + (size_t)b * a.max_pages : nullptr;
  const auto page_of = [&](int t) -> size_t {
    return (size_t)min((uint32_t)__builtin_amdgcn_readfirstlane(btab[t]), (uint32_t)(a.n_pages - 1));
  };
  const auto base_of = [&](int t, int hi) -> size_t {
    const int tc = min(t, hi - 1);
    return head_base + (paged ? page_of(tc) : (size_t)tc);
  };
  const bool kzero = a.wk == 0;
  // (zero-key plans run the 4-word kernel: the plan's zero block is one such tile)
  static_assert(4 * kTile * 4 == kZeroBytes, "zero block of one 4-word tile");
  const uint32_t *kcodes = kzero ? (const uint32_t *)(consts + a.off_zero) : a.kc;
  const size_t kstride = kzero ? 0 : (size_t)WK * kTile;
  TileRegs<VB, WK> ra, rb;
  int tile = tile_lo + wave;
  load_tile(ra, kcodes, kstride, a.kn, a.vc, a.vn, base_of(tile, tile_end), lane);
  // paged: the page of the tile after next, read one tile ahead of its load
  size_t pnext = paged ? page_of(min(tile + 2 * kStreamWaves, tile_end - 1)) : 0;
  __builtin_amdgcn_sched_barrier(0);
  if (tid < Lds::kt_bytes / 16) *(uint4 *)(smem + 16 * tid) = ktab;
#pragma unroll
  for (int rr = 0; rr < kRowRounds; ++rr) {
    const int e = (tid >> 2) + rr * (kStreamThreads / 4), part = tid & 3;
    if (e >= 256) break;
    uint2 v = rsrc[rr];
    if (Lds::qlds && part >= 2) {  // the pair (c, c') as fp16 (c_hi, c'_hi) and (c_lo, c'_lo)
      const float c0 = __builtin_bit_cast(float, v.x), c1 = __builtin_bit_cast(float, v.y);
      const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
      const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
      typedef _Float16 h2t __attribute__((ext_vector_type(2)));
      v = make_uint2(__builtin_bit_cast(uint32_t, (h2t){h0, h1}), __builtin_bit_cast(uint32_t, (h2t){l0, l1}));
    }
    // 64 bytes of row e: slots of 8 bytes (two copies per 16-byte store) or of 4 bytes (four)
    const uint4 q = (part >= 2 || VB == 2) ? make_uint4(v.x, v.y, v.x, v.y) : make_uint4(v.x, v.x, v.x, v.x);
    uint4 *dst = (uint4 *)(smem + Lds::rep + 256 * e + 64 * part);
    if (part >= 2 || VB >= 2) {
      dst[0] = q;
      dst[1] = q;
      dst[2] = q;
      dst[3] = q;
    }
  }
  if constexpr (VB == 1)
    if (tid < kVEntries) *(uint4 *)(smem + Lds::vcomp + 16 * tid) = vcomp;
  if constexpr (Lds::qlds) {
    if (tid < kImg16) *(uint4 *)(smem + Lds::qimg + 16 * tid) = qimg0;
    if (kImgRounds > 1 && tid + kStreamThreads < kImg16)
      *(uint4 *)(smem + Lds::qimg + 16 * (tid + kStreamThreads)) = qimg1;
  }
  StreamState st;
  st.seq = (seq_raw < 0 ? 0 : (seq_raw > a.max_seq_len ? a.max_seq_len : seq_raw)) - a.n_recent;
  st.lo = a.n_sink;
  st.nv = (uint32_t)(st.seq > st.lo ? st.seq - st.lo : 0);
  st.wk = a.wk;
  st.kwl = (uint32_t)(Lds::kw + wave * (Lds::kw_rows * kTile * 4) + lane * 4);
  st.kwb = (uint32_t)(Lds::kw + wave * (Lds::kw_rows * kTile * 4) + (lane >> 5) * kTile * 4 + (lane & 15) * 4);
  st.vslot = (uint32_t)(lane & (128 / Lds::vslot - 1)) * Lds::vslot;
  st.c4slot = 128u + (uint32_t)(lane & 15) * 8u + (Lds::qlds ? 4u * (uint32_t)((lane >> 4) & 1) : 0u);
  st.n4w = n4w;
  st.cgrp = cgrp;
  st.gbit = gbit;
  // the two zero rows past the key words (this lane's column, read by this lane only)
  *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * WK) = 0u;
  *(__attribute__((address_space(3))) uint32_t *)(size_t)(st.kwl + 256 * (WK + 1)) = 0u;
  __syncthreads();
  load_tile(rb, kcodes, kstride, a.kn, a.vc, a.vn, base_of(tile + kStreamWaves, tile_end), lane);

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
  // tile after next is requested once the next one has moved into place, so
  // that one tile is in flight while one is processed.  (Two copies with
  // alternating register sets raise the register count past the occupancy
  // limit.)
  for (; tile < tile_hi; tile += kStreamWaves) {
    wave_priority((tile_hi - 1 - tile) / kStreamWaves);
    process_tile<G, VB, WK>(ra, tile, st, qr, rinv, rinv4, mrun, mth, lsum, acc0, acc1, lane);
    ra = rb;
    if (tile + 2 * kStreamWaves < tile_hi) {
      const size_t bn = head_base + (paged ? pnext : (size_t)(tile + 2 * kStreamWaves));
      load_tile(rb, kcodes, kstride, a.kn, a.vc, a.vn, bn, lane);
      if (paged) pnext = page_of(min(tile + 3 * kStreamWaves, tile_hi - 1));
    }
  }

  __builtin_amdgcn_s_setprio(0);
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
  const size_t head0 = (size_t)b * a.hq + (size_t)kvh * a.group;  // first query head of this (sequence, KV head)
  for (int idx = tid; idx < a.group * kHeadDim; idx += kStreamThreads) {
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

// The kernel instance of a group size: 3 heads run as 4, 5..7 as 8.
int kernel_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : 8; }

DecodeKernel pick_decode(int g, int vb, int wk) {
  switch (kernel_group(g)) {
    case 1: return pick_vb<1>(vb, wk);
    case 2: return pick_vb<2>(vb, wk);
    case 4: return pick_vb<4>(vb, wk);
    default: return pick_vb<8>(vb, wk);
  }
}

// Workspace: the split partials [batch][hq][n_splits][kPartStride] f32, then
// the prepared query registers [batch][hkv] (QueryImage).
struct DecodeLayout {
  int n_splits, tiles_base, tiles_extra;  // split s covers tiles_base + (s < tiles_extra) tiles
  size_t img_off, total;
};

size_t query_image_bytes(int g) {
  switch (kernel_group(g)) {
    case 1: return QueryImage<1>::bytes;
    case 2: return QueryImage<2>::bytes;
    case 4: return QueryImage<4>::bytes;
    default: return QueryImage<8>::bytes;
  }
}


DecodeLayout decode_layout(const Plan &p, int batch, int64_t max_seq_len) {
  DecodeLayout d{};
  const int tiles = (int)((max_seq_len + kTile - 1) / kTile);
  const int hkv = p.desc.n_kv_heads, hq = p.desc.n_q_heads;
  const DecodeKernel k = pick_decode(p.hdr.group, p.hdr.v_bits, p.hdr.wk);
  const int target = std::max(1, k.per_cu) * device_cus();  // one round of resident workgroups
  // (short sequences: at least one tile per wave, the latency-bound case
  // measured faster than two tiles per wave; for the 12-wave kernels one tile
  // per 8 waves, the grid of their former 8-wave workgroups: with fewer
  // workgroups the 32K eight-head layer's kernel took 15.4 us instead of 13.9)
  const int per_split = k.waves == 12 ? 8 : k.waves;
  int s = (target + batch * hkv - 1) / (batch * hkv);
  s = std::max(1, std::min({s, (tiles + per_split - 1) / per_split, kMaxSplits}));
  // tiles dealt out evenly: the first tiles % s splits take one tile more, so
  // that (with a multiple of the wave count per split) no wave but those of
  // the first splits has a tile more than the others
  d.n_splits = s;
  d.tiles_base = tiles / s;
  d.tiles_extra = tiles % s;
  d.img_off = (((size_t)batch * hq * d.n_splits * kPartStride * 4) + 255) & ~(size_t)255;
  d.total = d.img_off + (size_t)batch * hkv * query_image_bytes(p.hdr.group);
  return d;
}

// Once per (kernel, device): the decode kernels address LDS from offset 0, so
// they must have no static LDS; and their dynamic LDS above 64 KB must be
// allowed.  Later calls find the pair in the list.
bgtq_status decode_kernel_ready(decode_fn fn, int smem) {
  static std::mutex mu;
  static std::vector<std::pair<decode_fn, int>> ready;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BGTQ_EDEVICE, "decode: no current device");
  std::lock_guard<std::mutex> lk(mu);
  for (const auto &r : ready)
    if (r.first == fn && r.second == dev) return BGTQ_OK;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, (const void *)fn) != hipSuccess || attr.sharedSizeBytes != 0)
    return fail(BGTQ_EDEVICE, "decode: kernel has static LDS");
  if (smem > 65536 &&
      hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem) != hipSuccess)
    return fail(BGTQ_EDEVICE, "decode: LDS request above the limit");
  ready.emplace_back(fn, dev);
  return BGTQ_OK;
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
  const bgtq_status ks = decode_kernel_ready(fn, smem);
  if (ks != BGTQ_OK) return ks;
  hipStream_t st = (hipStream_t)c.stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  {
    Prof &pr = prof();
    std::lock_guard<std::mutex> lk(pr.mu);
    if (pr.on && !(c.no_alloc && pr.pool.empty())) {
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
  a.qimg = ws + lay.img_off;
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
  a.group = G;
  // the queries of every (sequence, KV head), rotated and scaled into the
  // decode kernel's register image (in a serving step, side by side with the
  // new token's append)
  {
    const PrepArgs pa{a.consts, c.q, a.hq, a.hkv, G, a.off_zero, a.kscale, ws + lay.img_off};
    if (c.step) {
      const int n = c.batch * p.desc.n_kv_heads;
      const StepAppend &sa = *c.step;
      const bool copy = sa.n_sink > 0 || sa.n_recent > 0;
      const BufCopy bc{(const uint4 *)sa.k_new, (const uint4 *)sa.v_new, (uint4 *)sa.k_sink, (uint4 *)sa.v_sink,
                       (uint4 *)sa.k_recent, (uint4 *)sa.v_recent, sa.n_sink, sa.n_recent};
      const unsigned blocks = (unsigned)(3 * n + (copy ? c.batch : 0));
#define BGTQ_FRONT(GK) \
  step_front_kernel<GK><<<blocks, 64 * kPrepWaves, 0, st>>>(pa, *sa.ka, *sa.va, sa.pos, sa.capacity, n, bc)
      switch (kernel_group(G)) {
        case 1: BGTQ_FRONT(1); break;
        case 2: BGTQ_FRONT(2); break;
        case 4: BGTQ_FRONT(4); break;
        default: BGTQ_FRONT(8); break;
      }
#undef BGTQ_FRONT
    } else {
      const dim3 pgrid(p.desc.n_kv_heads, c.batch);
      switch (kernel_group(G)) {
        case 1: prep_kernel<1><<<pgrid, 64 * kPrepWaves, 0, st>>>(pa); break;
        case 2: prep_kernel<2><<<pgrid, 64 * kPrepWaves, 0, st>>>(pa); break;
        case 4: prep_kernel<4><<<pgrid, 64 * kPrepWaves, 0, st>>>(pa); break;
        default: prep_kernel<8><<<pgrid, 64 * kPrepWaves, 0, st>>>(pa); break;
      }
    }
    const bgtq_status ps = launch_status(c.step ? "decode step (append and query preparation)"
                                                : "decode (query preparation)");
    if (ps != BGTQ_OK) return ps;
  }
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

// ------------------------------------------------------------------ no-allocation entry

// Scratch of bgtq_decode_attn_noalloc: the split partials of the decode, in a
// file-scope device array (each device that runs the library holds its own
// copy until the process ends).  In host code `scratch` is a host-side
// stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device (resolved on the device's
// first call, with that device current).
static bgtq_status scratch_address(void **out) {
  static std::mutex mu;
  static std::vector<void *> addr;  // by device ordinal
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(BGTQ_EDEVICE, "bgtq_decode_attn_noalloc: no device");
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(BGTQ_EDEVICE, std::string("bgtq_decode_attn_noalloc: scratch address: ") + hipGetErrorString(e));
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return BGTQ_OK;
}

}  // namespace bgtq

using namespace bgtq;

// The buffered decode on a contiguous cache (pages null) or a paged pool.
static bgtq_status decode_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                   const uint32_t *k_codes, const uint16_t *k_norms, const uint32_t *v_codes,
                                   const uint16_t *v_norms, int64_t capacity, const bgtq_pages *pages,
                                   const int32_t *seq_lens, int32_t batch, int64_t max_seq_len, float softmax_scale,
                                   const uint16_t *k_sink, const uint16_t *v_sink, int32_t n_sink,
                                   const uint16_t *k_recent, const uint16_t *v_recent, int32_t n_recent,
                                   uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream,
                                   const char *nm) {
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
  c.pages = pages;
  return decode_launch(plan->p, c);
}

extern "C" {

size_t bgtq_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

bgtq_status bgtq_decode_attn_noalloc(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                     const uint32_t *k_codes, const uint16_t *k_norms, const uint32_t *v_codes,
                                     const uint16_t *v_norms, int64_t capacity, const int32_t *seq_lens,
                                     int32_t batch, int64_t max_seq_len, float softmax_scale, uint16_t *out,
                                     bgtq_stream stream) {
  const char *nm = "bgtq_decode_attn_noalloc";
  if (!plan || !dev_consts || !q || !k_norms || !v_codes || !v_norms || !seq_lens || !out ||
      (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (batch < 1 || max_seq_len < 1) return fail(BGTQ_EINVAL, std::string(nm) + ": batch, max_seq_len >= 1");
  if (decode_layout(plan->p, batch, max_seq_len).total > kNoAllocScratchBytes)
    return fail(BGTQ_EWORKSPACE, std::string(nm) + ": the split partials exceed the 4 MiB scratch");
  void *ws = nullptr;
  const bgtq_status sa = scratch_address(&ws);
  if (sa != BGTQ_OK) return sa;
  const bgtq_status v =
      decode_check(plan->p, capacity, batch, max_seq_len, softmax_scale, ws, kNoAllocScratchBytes, nm);
  if (v != BGTQ_OK) return v;
  DecodeCall c{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, seq_lens, 0, batch, max_seq_len,
               softmax_scale, out, ws, stream};
  c.no_alloc = true;
  return decode_launch(plan->p, c);
}

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
  return decode_buffered(plan, dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, nullptr, seq_lens, batch,
                         max_seq_len, softmax_scale, k_sink, v_sink, n_sink, k_recent, v_recent, n_recent, out,
                         workspace, ws_bytes, stream, "bgtq_decode_attn_buffered");
}

bgtq_status bgtq_decode_attn_paged_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                            const uint32_t *k_codes, const uint16_t *k_norms,
                                            const uint32_t *v_codes, const uint16_t *v_norms,
                                            const bgtq_pages *pages, const int32_t *seq_lens, int32_t batch,
                                            int64_t max_seq_len, float softmax_scale, const uint16_t *k_sink,
                                            const uint16_t *v_sink, int32_t n_sink, const uint16_t *k_recent,
                                            const uint16_t *v_recent, int32_t n_recent, uint16_t *out,
                                            void *workspace, size_t ws_bytes, bgtq_stream stream) {
  const char *nm = "bgtq_decode_attn_paged_buffered";
  const bgtq_status ps = pages_check(pages, nm);
  if (ps != BGTQ_OK) return ps;
  return decode_buffered(plan, dev_consts, q, k_codes, k_norms, v_codes, v_norms, (int64_t)kTile * pages->max_pages,
                         pages, seq_lens, batch, max_seq_len, softmax_scale, k_sink, v_sink, n_sink, k_recent,
                         v_recent, n_recent, out, workspace, ws_bytes, stream, nm);
}

}  // extern "C"
