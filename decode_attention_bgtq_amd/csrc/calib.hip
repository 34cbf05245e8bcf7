// Calibration rows of the Block-GTQ path on gfx950: the label-free RoPE-block
// energy and the greedy integer bit allocation ("RoPE-Aware Bit Allocation for
// KV-Cache Quantization", Abstract; Block-GTQ README, introduction and
// calibration paragraph).  Definitions: include/bgtq.h.
#include "device.h"
#include "host.h"

namespace bgtq {

// One workgroup of 1024 threads per KV head: thread (phase, coordinate) takes
// the tokens t = phase (mod 8).  Sums of squares are exact: |x| 2^24 = u =
// h 2^20 + l (h, l < 2^20), u^2 = h^2 2^40 + 2 h l 2^20 + l^2, the three sums in
// 64-bit integers folded into 128-bit totals every kFold tokens; then per block
// over its two coordinates (j, j+64) half-split or (2j, 2j+1) interleaved.
constexpr int kEnergyThreads = 1024, kEnergyPhases = kEnergyThreads / kHeadDim, kFold = 4096;

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

__global__ __launch_bounds__(kEnergyThreads) void energy_kernel(const uint16_t *__restrict__ q,
                                                                const uint16_t *__restrict__ k, int64_t n,
                                                                int hq, int hkv, int inter,
                                                                double *__restrict__ energy) {
  __shared__ u128 sq[kEnergyThreads], sk[kEnergyThreads];
  const int kvh = blockIdx.x, tid = threadIdx.x, c = tid & 127, ph = tid >> 7;
  const int G = hq / hkv;
  u128 aq = 0, ak = 0;
  uint64_t qa = 0, qb = 0, qc = 0, ka = 0, kb = 0, kc = 0;
  int cnt = 0;
  for (int64_t t = ph; t < n; t += kEnergyPhases) {
    const uint16_t *qt = q + ((size_t)t * hq + (size_t)kvh * G) * kHeadDim + c;
    for (int hh = 0; hh < G; ++hh) sq_split(f16_mag_units(qt[(size_t)hh * kHeadDim]), qa, qb, qc);
    sq_split(f16_mag_units(k[((size_t)t * hkv + kvh) * kHeadDim + c]), ka, kb, kc);
    if (++cnt == kFold) {  // (at most kFold * G terms below 2^40 in each 64-bit sum)
      aq += sq_fold(qa, qb, qc);
      ak += sq_fold(ka, kb, kc);
      cnt = 0;
    }
  }
  aq += sq_fold(qa, qb, qc);
  ak += sq_fold(ka, kb, kc);
  sq[tid] = aq;
  sk[tid] = ak;
  __syncthreads();
  if (tid < kBlocks) {
    const int j = tid, a = inter ? 2 * j : j, b = inter ? 2 * j + 1 : j + kBlocks;
    u128 tq = 0, tk = 0;
#pragma unroll
    for (int p = 0; p < kEnergyPhases; ++p) {
      tq += sq[p * kHeadDim + a] + sq[p * kHeadDim + b];
      tk += sk[p * kHeadDim + a] + sk[p * kHeadDim + b];
    }
    const double eq = ldexp(u128_to_f64(tq), -48) / (double)(n * G);
    const double ek = ldexp(u128_to_f64(tk), -48) / (double)n;
    energy[(size_t)kvh * kBlocks + j] = eq * ek;
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
  energy_kernel<<<n_kv_heads, kEnergyThreads, 0, (hipStream_t)stream>>>(q_cal, k_cal, n_cal, n_q_heads, n_kv_heads,
                                                                         rope_pairing, energy);
  return launch_status("bgtq_energy");
}

bgtq_status bgtq_allocate(const double *energy, int32_t n_kv_heads, int32_t n_blocks, int32_t avg_bits,
                          int8_t *bits, bgtq_stream stream) {
  if (!energy || !bits) return fail(BGTQ_EINVAL, "bgtq_allocate: null pointer");
  if (n_blocks != kBlocks || n_kv_heads < 1) return fail(BGTQ_EINVAL, "bgtq_allocate: n_blocks must be 64");
  if (avg_bits < 0 || avg_bits > 4) return fail(BGTQ_EBUDGET, "bgtq_allocate: avg_bits must be 0..4");
  double dist[5] = {1.0, 0, 0, 0, 0};
  for (int b = 1; b <= 4; ++b) dist[b] = codebook(b).d;
  allocate_kernel<<<n_kv_heads, 64, 0, (hipStream_t)stream>>>(energy, avg_bits, bits, dist[0] - dist[1],
                                                               dist[1] - dist[2], dist[2] - dist[3],
                                                               dist[3] - dist[4]);
  return launch_status("bgtq_allocate");
}

}  // extern "C"
