// Fused decode step: the new token's key and value appended to the packed
// cache, then the fused decode over the cache including that token
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract:
// packed-cache serving; Block-GTQ README, backend table).  The append runs in
// the launch that prepares the queries (decode.hip, step_front_kernel).
#include "append.h"
#include "device.h"
#include "host.h"

using namespace bgtq;

namespace {

bgtq_status step_common(const char *nm, const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                        const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos, int32_t batch,
                        int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms, uint32_t *v_codes,
                        uint16_t *v_norms, int64_t capacity, const bgtq_pages *pages, float softmax_scale,
                        uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream) {
  if (!plan || !dev_consts || !q || !k_new || !v_new || !pos || !k_norms || !v_codes || !v_norms || !out ||
      !workspace || (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  const Plan &p = plan->p;
  const bgtq_status v = decode_check(p, capacity, batch, max_seq_len, softmax_scale, workspace, ws_bytes, nm);
  if (v != BGTQ_OK) return v;
  const int n = batch * p.desc.n_kv_heads;
  if ((int64_t)n * 3 > 0x7FFFFFFF) return fail(BGTQ_EINVAL, std::string(nm) + ": grid too large");
  const TileMap map = pages ? paged_map(p, pages) : contiguous_map(p.desc.n_kv_heads, capacity);
  const uint8_t *c = (const uint8_t *)dev_consts;
  const AppendArgs ka = append_args(p, c, k_new, k_codes, k_norms, map, false);
  const AppendArgs va = append_args(p, c, v_new, v_codes, v_norms, map, true);
  const StepAppend sa{&ka, &va, pos, capacity};
  DecodeCall dc{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, pos, 1, batch, max_seq_len,
                softmax_scale, out, workspace, stream};
  dc.pages = pages;
  dc.step = &sa;
  return decode_launch(p, dc);
}

}  // namespace

extern "C" {

bgtq_status bgtq_decode_step(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                             const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos, int32_t batch,
                             int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms, uint32_t *v_codes,
                             uint16_t *v_norms, int64_t capacity, float softmax_scale, uint16_t *out,
                             void *workspace, size_t ws_bytes, bgtq_stream stream) {
  return step_common("bgtq_decode_step", plan, dev_consts, q, k_new, v_new, pos, batch, max_seq_len, k_codes,
                     k_norms, v_codes, v_norms, capacity, nullptr, softmax_scale, out, workspace, ws_bytes, stream);
}

bgtq_status bgtq_decode_step_paged(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                   const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                   int32_t batch, int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms,
                                   uint32_t *v_codes, uint16_t *v_norms, const bgtq_pages *pages,
                                   float softmax_scale, uint16_t *out, void *workspace, size_t ws_bytes,
                                   bgtq_stream stream) {
  const bgtq_status ps = pages_check(pages, "bgtq_decode_step_paged");
  if (ps != BGTQ_OK) return ps;
  return step_common("bgtq_decode_step_paged", plan, dev_consts, q, k_new, v_new, pos, batch, max_seq_len,
                     k_codes, k_norms, v_codes, v_norms, (int64_t)kTile * pages->max_pages, pages, softmax_scale,
                     out, workspace, ws_bytes, stream);
}

}  // extern "C"
