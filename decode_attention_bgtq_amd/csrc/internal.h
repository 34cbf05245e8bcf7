// Internal definitions shared by the host plan (plan.cpp) and the HIP kernels
// (calib.hip, encode.hip, decode.hip, step.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/bgtq.h"

namespace bgtq {

constexpr int kHeadDim = 128;
constexpr int kBlocks = 64;
constexpr int kTile = 64;
constexpr int kMaxGroups = 4;
constexpr int kMaxWK = 16;          // key words per token at 4 bits per coordinate
constexpr int kMaxKSteps = 36;      // bound on the width-1..3 k-steps of one head (at most 33)
constexpr int kZeroBytes = 4 * 64 * 4;  // one tile of four key words

// Decode k-steps of the key groups of width 1..3 (the 4-bit group takes one
// matrix-core step per code).  A k-step is four consecutive positions of one
// group (a group's last step may hold two; its query operand is zero past the
// group): its codes are the 4w stream bits that start at its first position's
// bit, code k at bits [w k, w (k + 1)).  K-steps are numbered through the
// groups of width 3, 2, 1.

// Decode tables shared by every head of a plan, copied as one block into LDS:
// 4-bit centroid pairs of a code byte (float2 [256]); four fp16 centroids of a
// width-2 code byte [256] and of a width-1 code nibble [16]; two fp16 centroids
// of six width-3 code bits [64].  Offsets in bytes.
constexpr int kDtabC4 = 0, kDtabT2 = 2048, kDtabT1 = 4096, kDtabT3 = 4352, kDtabBytes = 4608;

struct KGroupDesc {
  int32_t w;        // width 1..4
  int32_t d;        // coordinates in the group
  int32_t pos;      // first position in group order
  int32_t bit_off;  // first bit in the key stream
  int64_t rot64;    // element offset of Pi^T (double, [k][i]) in the K double-rotation area
  int64_t rot32;    // unused (the float rotations are one block-diagonal matrix per head)
};

struct KvhDesc {
  int32_t n_groups;
  int32_t d_nz;
  int32_t n_ksteps;            // k-steps of the width-1..3 groups
  uint32_t gbit;               // bits [10r, 10r+10): first stream bit of the width-(3-r) group (0 if absent)
  int32_t d4;                  // coordinates of the 4-bit group (group 0 when present), else 0
  int32_t n4blk;               // 16-code blocks of the 4-bit group, ceil(d4 / 16)
  int32_t n4w;                 // key words holding 4-bit codes, ceil(d4 / 8)
  uint32_t cgrp;               // byte r (r = 0..2): first k-step of the width-(3-r) group; byte 3 = n_ksteps
  KGroupDesc g[kMaxGroups];
  int16_t coord[kHeadDim];     // original coordinate of each group-order position
};

// Where logical tile j of (sequence b, KV head h) lives in a cache array of
// tiles: contiguous caches [batch][n_kv_heads][tiles_cap] (no table; page = j,
// head_stride = tiles_cap, seq_stride = n_kv_heads * tiles_cap) or paged pools
// [n_kv_heads][n_pages] (page = table[b][j], head_stride = n_pages,
// seq_stride = 0).  Tile index = h * head_stride + b * seq_stride + page.
struct TileMap {
  const int32_t *table;  // device int32 [batch][max_pages], or null
  int64_t head_stride, seq_stride;
  int32_t max_pages, n_pages;
};

inline TileMap contiguous_map(int n_kv_heads, int64_t capacity) {
  const int64_t tiles = (capacity + kTile - 1) / kTile;
  return TileMap{nullptr, tiles, (int64_t)n_kv_heads * tiles, 0, 0};
}

// Device constant image header.  All offsets are bytes from the image start.
struct ConstHeader {
  int32_t n_kv_heads, n_q_heads, group, head_dim;
  int32_t k_avg_bits, v_bits, wk, wv;
  int32_t max_ksteps;        // largest k-step count over heads
  int32_t pad0;
  int64_t off_kvh;           // KvhDesc[n_kv_heads]
  int64_t off_rot64_k;       // double area (Pi^T per K group)
  int64_t off_rot32_k;       // float [n_kv_heads][128][128]: block-diagonal R, R[pos_g + i][pos_g + k] = Pi_g[i][k]
  int64_t off_rot64_v;       // double [n_kv_heads][128][128], Pi_V^T ([k][i])
  int64_t off_rot32_v;       // float [n_kv_heads][128][128], Pi_V^T ([j][k] = Pi_V[k][j])
  int64_t off_dtab;          // decode tables, kDtabBytes (layout above)
  int64_t off_vlut;          // value-width table: fp16 centroid pairs of the tokens of one code chunk
  int64_t vlut_bytes;
  int64_t off_rowk;          // uint2 [n_kv_heads][128]: per group-order row p of the key rotation, x = row
                             // within its group, y = d_g | pos_g << 8 | w << 16 | kbase << 19
                             // (kbase: first k-step of a width-1..3 group); y = 0 past d_nz
  int64_t off_zero;          // kZeroBytes of zeros: the key words of every tile for a plan without key bits
  int64_t total_bytes;
  double thr[4][16];         // interior thresholds of the b-bit quantiser, row b-1
  double cent[4][16];        // centroids, row b-1
  double dist[8];            // D(0..4)
};

struct Codebook {
  std::vector<double> c, t;
  double d;
};

// Host-side plan (immutable after creation).
struct Plan {
  bgtq_plan_desc desc{};
  std::vector<int8_t> bits;             // [Hkv][64]
  std::vector<KvhDesc> kvh;
  std::vector<std::vector<double>> rot_k;  // per (kvh, group) Pi row-major
  std::vector<std::vector<double>> rot_v;  // per kvh Pi_V row-major
  std::vector<uint8_t> image;           // device constant image
  ConstHeader hdr{};
};

const Codebook &codebook(int bits);  // Lloyd-Max for N(0,1), bits 1..4
bgtq_status build_plan(const bgtq_plan_desc &d, Plan &p, std::string &err);

}  // namespace bgtq

struct bgtq_plan {
  bgtq::Plan p;
};
