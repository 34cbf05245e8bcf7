// Device helpers shared by the HIP kernels (gfx950).  Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace bgtq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned __int128 u128;

// ============================================================ device helpers

// fp16 bit pattern -> |x| * 2^24 as an exact integer (finite inputs).
__device__ __forceinline__ uint64_t f16_mag_units(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  return e == 0 ? (uint64_t)m : ((uint64_t)(1024u + m) << (e - 1));
}

// Round-to-nearest-even conversion of an unsigned 128-bit integer to double.
__device__ __forceinline__ double u128_to_f64(u128 x) {
  const uint64_t hi = (uint64_t)(x >> 64), lo = (uint64_t)x;
  if (hi == 0 && (lo >> 53) == 0) return (double)lo;
  const int msb = hi ? 127 - __builtin_clzll(hi) : 63 - __builtin_clzll(lo);
  const int sh = msb - 52;  // >= 1
  const uint64_t mant = (uint64_t)(x >> sh);
  const u128 rem = x & (((u128)1 << sh) - 1);
  const u128 half = (u128)1 << (sh - 1);
  uint64_t m = mant;
  if (rem > half || (rem == half && (m & 1))) ++m;
  return ldexp((double)m, sh);
}

// IEEE binary16 bits of a double with one round-to-nearest-even step.
__device__ __forceinline__ uint16_t f64_to_f16(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int ex = (int)((u >> 52) & 0x7FF);
  const uint64_t man = u & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
  if (ex == 0) return sign;  // double subnormals are far below fp16 range
  const int e = ex - 1023;
  const uint64_t m = (1ull << 52) | man;
  if (e >= -14) {
    uint64_t q = m >> 42;
    const uint64_t rem = m & ((1ull << 42) - 1), half = 1ull << 41;
    if (rem > half || (rem == half && (q & 1))) ++q;
    int ee = e;
    if (q == 2048) {
      q = 1024;
      ++ee;
    }
    if (ee > 15) return sign | 0x7C00u;
    return sign | (uint16_t)(((ee + 15) << 10) | (q & 1023));
  }
  const int sh = 28 - e;  // > 42
  if (sh >= 64) return sign;
  uint64_t q = m >> sh;
  const uint64_t rem = m & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  return sign | (uint16_t)q;
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}

// Max over the 64 lanes of a wave, returned to every lane.  Floats are mapped
// to integers with the same order (negative values have their magnitude bits
// flipped) so that each step is a single integer max with a DPP operand; the
// inputs are finite or -inf.
__device__ __forceinline__ float wave_max(float x) {
  const int i = __builtin_bit_cast(int, x);
  int v = i ^ ((i >> 31) & 0x7FFFFFFF);
  v = max(v, dpp_i<0xB1>(v));        // quad_perm [1,0,3,2]
  v = max(v, dpp_i<0x4E>(v));        // quad_perm [2,3,0,1]
  v = max(v, dpp_i<0x141>(v));       // row_half_mirror
  v = max(v, dpp_i<0x140>(v));       // row_mirror
  v = max(v, dpp_i<0x142, 0xA>(v));  // row_bcast:15
  v = max(v, dpp_i<0x143, 0xC>(v));  // row_bcast:31
  v = __builtin_amdgcn_readlane(v, 63);
  return __builtin_bit_cast(float, v ^ ((v >> 31) & 0x7FFFFFFF));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  // rows hold their sum in every lane; add the four rows
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tile index of logical tile j of (sequence b, KV head kvh), or -1 when a
// paged table entry is outside the pool (writers skip such tiles).
__device__ __forceinline__ int64_t tile_at(const TileMap &m, int b, int kvh, int64_t j) {
  int64_t page = j;
  if (m.table) {
    const int32_t e = m.table[(size_t)b * m.max_pages + j];
    if (e < 0 || e >= m.n_pages) return -1;
    page = e;
  }
  return (int64_t)kvh * m.head_stride + (int64_t)b * m.seq_stride + page;
}

__device__ __forceinline__ const ConstHeader *hdr_of(const uint8_t *c) {
  return (const ConstHeader *)c;
}

template <int VB> struct VLut;  // value lookup table: entries x bytes
template <> struct VLut<1> { static constexpr int entries = 256, bytes = 16; };
template <> struct VLut<2> { static constexpr int entries = 256, bytes = 8; };
template <> struct VLut<3> { static constexpr int entries = 64, bytes = 4; };
template <> struct VLut<4> { static constexpr int entries = 256, bytes = 4; };

}  // namespace bgtq
