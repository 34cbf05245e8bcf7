// Host-side helpers shared by the ABI translation units.  Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"

namespace bgtq {

bgtq_status fail(bgtq_status s, const std::string &m);
bgtq_status launch_status(const char *what);
int device_cus();

// Events bracketing the decode kernel while profiling is on.
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending, pool;
};
Prof &prof();

struct AppendArgs;

// A serving step's append of the new token (launched with the query
// preparation): the key and value arguments, each sequence's position.
struct StepAppend {
  const AppendArgs *ka, *va;
  const int32_t *pos;
  int64_t capacity;
  // buffered step: the new token (rows [batch][hkv][128]) also copied into the
  // fp16 sink (row pos[b] when below n_sink) and recent window (ring row
  // pos[b] % n_recent); counts 0: no copy
  const uint16_t *k_new = nullptr, *v_new = nullptr;
  uint16_t *k_sink = nullptr, *v_sink = nullptr, *k_recent = nullptr, *v_recent = nullptr;
  int n_sink = 0, n_recent = 0;
};

// Decode launches shared by bgtq_decode_attn and bgtq_decode_step.
struct DecodeCall {
  const void *dev_consts;
  const uint16_t *q;
  const uint32_t *k_codes;
  const uint16_t *k_norms;
  const uint32_t *v_codes;
  const uint16_t *v_norms;
  int64_t capacity;
  const int32_t *seq_lens;
  int seq_add;
  int32_t batch;
  int64_t max_seq_len;
  float softmax_scale;
  uint16_t *out;
  void *workspace;
  bgtq_stream stream;
  // paged pool (null: the contiguous layout)
  const bgtq_pages *pages = nullptr;
  // fp16 sink and recent window (counts 0: none)
  const uint16_t *k_sink = nullptr, *v_sink = nullptr, *k_recent = nullptr, *v_recent = nullptr;
  int n_sink = 0, n_recent = 0;
  // no HIP allocation of any kind in this call (no profiling events are created)
  bool no_alloc = false;
  // a serving step: the new token is appended in the launch that prepares the queries
  const StepAppend *step = nullptr;
};
bgtq_status decode_check(const Plan &p, int64_t capacity, int32_t batch, int64_t max_seq_len, float softmax_scale,
                         const void *workspace, size_t ws_bytes, const char *nm);
bgtq_status decode_launch(const Plan &p, const DecodeCall &c);  // the fused decode kernel

AppendArgs append_args(const Plan &p, const uint8_t *consts, const uint16_t *x, uint32_t *codes, uint16_t *norms,
                       const TileMap &map, bool is_v);

// Paged pools: argument checks and the tile map of a pool.
inline bgtq_status pages_check(const bgtq_pages *pg, const char *nm) {
  if (!pg || !pg->block_table) return fail(BGTQ_EINVAL, std::string(nm) + ": null pages or block table");
  if (pg->max_pages < 1 || pg->n_pages < 1 || (int64_t)pg->max_pages * kTile > ((int64_t)1 << 40))
    return fail(BGTQ_EINVAL, std::string(nm) + ": max_pages and n_pages must be >= 1");
  return BGTQ_OK;
}

inline TileMap paged_map(const Plan &, const bgtq_pages *pg) {
  return TileMap{pg->block_table, pg->n_pages, 0, pg->max_pages, pg->n_pages};
}

}  // namespace bgtq
