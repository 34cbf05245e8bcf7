// Calibration rows of the Block-GTQ path on gfx950: the label-free RoPE-block
// energy and the greedy integer bit allocation ("RoPE-Aware Bit Allocation for
// KV-Cache Quantization", Abstract; Block-GTQ README, introduction and
// calibration paragraph).  Definitions: include/bgtq.h.
#include <cmath>
#include <cstring>

#include "device.h"
#include "host.h"

namespace bgtq {

// Eight workgroups of 256 threads per KV head: workgroup p owns the sixteen
// coordinates of blocks 8p .. 8p + 7 (coordinates 8p .. 8p + 7 and 64 + 8p ..
// 64 + 8p + 7 half-split, 16p .. 16p + 15 interleaved), thread (phase, half)
// eight of them (one 16-byte load per token and head) over the tokens t = phase
// (mod 128).  Sums of squares are exact: |x| 2^24 = u = h 2^20 + l (h, l <
// 2^20), u^2 = h^2 2^40 + 2 h l 2^20 + l^2, the three sums in 64-bit integers
// folded into 128-bit totals every kFold tokens; integer sums do not depend on
// their order, so the split over threads and workgroups changes no bit.
constexpr int kEnergyThreads = 256, kEnergySplit = kBlocks / 8, kEnergyPhases = kEnergyThreads / 2, kFold = 4096;

__device__ __forceinline__ void sq_split(uint64_t u, uint64_t &a, uint64_t &b, uint64_t &c) {
  const uint64_t h = u >> 20, l = u & 0xFFFFFu;
  a += h * h;
  b += h * l;
  c += l * l;
}

__device__ __forceinline__ u128 sq_fold(uint64_t &a, uint64_t &b, uint64_t &c) {
  const u128 s = ((u128)a << 40) + ((u128)b << 21) + (u128)c;
  a = b = c = 0;
  return s;
}

// The eight fp16 values of a 16-byte load into the sums of their squares.
__device__ __forceinline__ void sq_split8(const uint4 v, uint64_t (&s)[8][3]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 8; ++i)
    sq_split(f16_mag_units((uint16_t)(w[i >> 1] >> (16 * (i & 1)))), s[i][0], s[i][1], s[i][2]);
}

__global__ __launch_bounds__(kEnergyThreads) void energy_kernel(const uint16_t *__restrict__ q,
                                                                const uint16_t *__restrict__ k, int64_t n,
                                                                int hq, int hkv, int inter,
                                                                double *__restrict__ energy) {
  __shared__ u128 red[kEnergyThreads][8];
  __shared__ u128 tot[2][16];
  const int kvh = blockIdx.x, p = blockIdx.y, tid = threadIdx.x, half = tid & 1, ph = tid >> 1;
  const int G = hq / hkv;
  const int off = inter ? 16 * p + 8 * half : (half ? kBlocks + 8 * p : 8 * p);
  uint64_t sq[8][3] = {}, sk[8][3] = {};
  u128 aq[8] = {}, ak[8] = {};
  int cnt = 0;
  for (int64_t t = ph; t < n; t += kEnergyPhases) {
    const uint16_t *qt = q + ((size_t)t * hq + (size_t)kvh * G) * kHeadDim + off;
    for (int hh = 0; hh < G; ++hh) sq_split8(*(const uint4 *)(qt + (size_t)hh * kHeadDim), sq);
    sq_split8(*(const uint4 *)(k + ((size_t)t * hkv + kvh) * kHeadDim + off), sk);
    if (++cnt == kFold) {  // (at most kFold * G terms below 2^40 in each 64-bit sum)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        aq[i] += sq_fold(sq[i][0], sq[i][1], sq[i][2]);
        ak[i] += sq_fold(sk[i][0], sk[i][1], sk[i][2]);
      }
      cnt = 0;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    aq[i] += sq_fold(sq[i][0], sq[i][1], sq[i][2]);
    ak[i] += sq_fold(sk[i][0], sk[i][1], sk[i][2]);
  }
  // per coordinate over the phases: slot h * 8 + i is coordinate i of half h
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tid][i] = r ? ak[i] : aq[i];
    __syncthreads();
    if (tid < 16) {
      u128 s = 0;
      for (int f = 0; f < kEnergyPhases; ++f) s += red[2 * f + (tid >> 3)][tid & 7];
      tot[r][tid] = s;
    }
    __syncthreads();
  }
  if (tid < 8) {  // block 8p + tid: its two coordinates' slots
    const int a = inter ? 2 * tid : tid, b = inter ? 2 * tid + 1 : 8 + tid;
    const double eq = ldexp(u128_to_f64(tot[0][a] + tot[0][b]), -48) / (double)(n * G);
    const double ek = ldexp(u128_to_f64(tot[1][a] + tot[1][b]), -48) / (double)n;
    energy[(size_t)kvh * kBlocks + 8 * p + tid] = eq * ek;
  }
}

// ============================================================ (2) allocation

// One wave per KV head; lane j owns block j.  The greedy's result is the top
// avg * 64 of the marginal gains g[j][b] = E_j (D(b) - D(b + 1)), b < 4, in the
// order (gain descending, block ascending, width ascending): each block's gains
// are non-increasing in b, so the greedy takes them in that order, and a tie
// between blocks goes to the lower block as in the greedy.  Each candidate's
// rank in that order is counted against all 256; block j gets one bit per
// candidate of rank < avg * 64.
__global__ __launch_bounds__(64) void allocate_kernel(const double *__restrict__ energy, int avg,
                                                      int8_t *__restrict__ bits, double dd0, double dd1,
                                                      double dd2, double dd3) {
  __shared__ double gs[kBlocks * 4];
  const int kvh = blockIdx.x, lane = threadIdx.x;
  const double e = energy[(size_t)kvh * kBlocks + lane];
  const double g[4] = {e * dd0, e * dd1, e * dd2, e * dd3};
#pragma unroll
  for (int b = 0; b < 4; ++b) gs[lane * 4 + b] = g[b];
  __syncthreads();
  int rank[4] = {0, 0, 0, 0};
  for (int i = 0; i < kBlocks * 4; ++i) {
    const double o = gs[i];
    const int j2 = i >> 2, b2 = i & 3;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      rank[b] += (o > g[b] || (o == g[b] && (j2 < lane || (j2 == lane && b2 < b)))) ? 1 : 0;
  }
  int nb = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) nb += rank[b] < avg * kBlocks ? 1 : 0;
  bits[(size_t)kvh * kBlocks + lane] = (int8_t)nb;
}

}  // namespace bgtq

using namespace bgtq;

extern "C" {

bgtq_status bgtq_energy(const uint16_t *q_cal, const uint16_t *k_cal, int64_t n_cal, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t rope_pairing, double *energy,
                        bgtq_stream stream) {
  if (!q_cal || !k_cal || !energy) return fail(BGTQ_EINVAL, "bgtq_energy: null pointer");
  if (n_cal < 1 || n_cal > (1 << 22)) return fail(BGTQ_EINVAL, "bgtq_energy: n_cal must be 1..2^22");
  if (head_dim != kHeadDim) return fail(BGTQ_EINVAL, "bgtq_energy: head_dim must be 128");
  if (n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(BGTQ_EINVAL, "bgtq_energy: n_q_heads must be a positive multiple of n_kv_heads");
  if (rope_pairing != BGTQ_ROPE_HALF && rope_pairing != BGTQ_ROPE_INTERLEAVED)
    return fail(BGTQ_EINVAL, "bgtq_energy: rope_pairing must be BGTQ_ROPE_HALF or BGTQ_ROPE_INTERLEAVED");
  if (n_q_heads / n_kv_heads > 1024)
    return fail(BGTQ_EINVAL, "bgtq_energy: at most 1024 query heads per KV head");
  if (((uintptr_t)q_cal | (uintptr_t)k_cal) & 15u)
    return fail(BGTQ_EINVAL, "bgtq_energy: q_cal and k_cal must be 16-byte aligned");
  const dim3 grid(n_kv_heads, kEnergySplit);
  energy_kernel<<<grid, kEnergyThreads, 0, (hipStream_t)stream>>>(q_cal, k_cal, n_cal, n_q_heads, n_kv_heads,
                                                                   rope_pairing, energy);
  return launch_status("bgtq_energy");
}

// The distortion drops D(b) - D(b + 1), b = 0..3, of the library's codebooks.
static void distortion_drops(double dd[4]) {
  double dist[5] = {1.0, 0, 0, 0, 0};
  for (int b = 1; b <= 4; ++b) dist[b] = codebook(b).d;
  for (int b = 0; b < 4; ++b) dd[b] = dist[b] - dist[b + 1];
}

bgtq_status bgtq_allocate(const double *energy, int32_t n_kv_heads, int32_t n_blocks, int32_t avg_bits,
                          int8_t *bits) {
  if (!energy || !bits) return fail(BGTQ_EINVAL, "bgtq_allocate: null pointer");
  if (n_blocks != kBlocks || n_kv_heads < 1) return fail(BGTQ_EINVAL, "bgtq_allocate: n_blocks must be 64");
  if (avg_bits < 0 || avg_bits > 4) return fail(BGTQ_EBUDGET, "bgtq_allocate: avg_bits must be 0..4");
  for (int64_t i = 0; i < (int64_t)n_kv_heads * kBlocks; ++i)
    if (!(energy[i] >= 0.0) || !std::isfinite(energy[i]))
      return fail(BGTQ_EINVAL, "bgtq_allocate: energies must be finite and non-negative");
  double dd[4];
  distortion_drops(dd);
  // The greedy as stated: from all zeros, avg_bits * 64 times one more bit to
  // the block of largest gain E_j (D(b_j) - D(b_j + 1)) among blocks below 4
  // bits, the lowest j on a tie.
  for (int h = 0; h < n_kv_heads; ++h) {
    const double *e = energy + (size_t)h * kBlocks;
    int8_t b[kBlocks] = {};
    for (int step = 0; step < avg_bits * kBlocks; ++step) {
      int best = -1;
      double gbest = 0.0;
      for (int j = 0; j < kBlocks; ++j) {
        if (b[j] >= 4) continue;
        const double g = e[j] * dd[b[j]];
        if (best < 0 || g > gbest) best = j, gbest = g;
      }
      ++b[best];
    }
    std::memcpy(bits + (size_t)h * kBlocks, b, kBlocks);
  }
  return BGTQ_OK;
}

bgtq_status bgtq_allocate_device(const double *energy, int32_t n_kv_heads, int32_t n_blocks, int32_t avg_bits,
                                 int8_t *bits, bgtq_stream stream) {
  if (!energy || !bits) return fail(BGTQ_EINVAL, "bgtq_allocate_device: null pointer");
  if (n_blocks != kBlocks || n_kv_heads < 1) return fail(BGTQ_EINVAL, "bgtq_allocate_device: n_blocks must be 64");
  if (avg_bits < 0 || avg_bits > 4) return fail(BGTQ_EBUDGET, "bgtq_allocate_device: avg_bits must be 0..4");
  double dd[4];
  distortion_drops(dd);
  allocate_kernel<<<n_kv_heads, 64, 0, (hipStream_t)stream>>>(energy, avg_bits, bits, dd[0], dd[1], dd[2], dd[3]);
  return launch_status("bgtq_allocate_device");
}

}  // extern "C"
