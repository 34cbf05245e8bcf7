// Internal definitions shared by the host plan (plan.cpp) and the HIP kernels
// (bgtq.hip).  Not part of the public ABI.
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
constexpr int kMaxChunks = 128;     // bound on lookup chunks per head (widths 1..3)

// Decode lookup-table chunk descriptors, for the key groups of width 1..3 (the
// 4-bit group is summed directly from its centroids).  A chunk is a run of m
// consecutive codes of one key group (m * w <= window bits).  Its table, one
// fp16 entry per query head of the group, is indexed by the `window` stream
// bits starting at the chunk's first bit.
//
// lookup (32 bits): [0,5) funnel shift that brings the chunk's window to bit
//   log2(entry bytes), [5,23) byte offset of the chunk's table in LDS,
//   [23] first chunk of a group, [24,26) norm slot (4 - width)
// build (32 bits): [0,8) first code position (group order), [8,12) codes m,
//   [12,15) width w, [15,17) group index
constexpr uint32_t kChunkStart = 1u << 23;
constexpr uint32_t kChunkTableMask = 0x007FFFE0u;
constexpr int kLutBudget = 64 * 1024;  // LDS bytes for one head's key tables

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
  int32_t n_chunks;
  int32_t chunk_base;          // index of this head's first chunk in the chunk arrays (head * kMaxChunks)
  int32_t d4;                  // coordinates of the 4-bit group (group 0 when present), else 0
  int32_t n4blk;               // 16-code blocks of the 4-bit group, ceil(d4 / 16)
  int32_t n4w;                 // key words holding 4-bit codes, ceil(d4 / 8)
  uint32_t cgrp;               // byte r (r = 0..3): first chunk of the width-(3-r) group; byte 3 = n_chunks
  uint32_t jrng;               // bits [10r, 10r+5) / [10r+5, 10r+10): first / last word slot jj of group r's chunks
  KGroupDesc g[kMaxGroups];
  int16_t coord[kHeadDim];     // original coordinate of each group-order position
  int16_t pad_[4];
  int32_t anchor[kMaxWK + 2];  // chunks anchored at word jj-1 are [anchor[jj], anchor[jj+1])
};

// Device constant image header.  All offsets are bytes from the image start.
struct ConstHeader {
  int32_t n_kv_heads, n_q_heads, group, head_dim;
  int32_t k_avg_bits, v_bits, wk, wv;
  int32_t lut_window;        // key lookup window bits (4 or 6)
  int32_t lut_entry_log2;    // log2 of the table entry size in bytes (2 * group: fp16 per head)
  int32_t max_chunks;        // largest chunk count over heads
  int32_t pad0;
  int64_t off_kvh;           // KvhDesc[n_kv_heads]
  int64_t off_lookup;        // uint32 [total chunks]
  int64_t off_build;         // uint32 [total chunks]
  int64_t off_rot64_k;       // double area (Pi^T per K group)
  int64_t off_rot32_k;       // float [n_kv_heads][128][128]: block-diagonal R, R[pos_g + i][pos_g + k] = Pi_g[i][k]
  int64_t off_rot64_v;       // double [n_kv_heads][128][128], Pi_V^T ([k][i])
  int64_t off_rot32_v;       // float [n_kv_heads][128][128], Pi_V^T ([j][k] = Pi_V[k][j])
  int64_t off_c4;            // float2 [256]: (c4[b & 15], c4[b >> 4]), 4-bit centroid pairs of a code byte
  int64_t off_vlut;          // value-width table: fp16 centroid pairs of the tokens of one code chunk
  int64_t vlut_bytes;
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
  std::vector<uint32_t> lookup, build;  // chunk descriptors (see above)
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
