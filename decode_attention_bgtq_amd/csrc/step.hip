// Fused decode step: the new token's key and value appended to the packed
// cache, then the fused decode over the cache including that token
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract:
// packed-cache serving; Block-GTQ README, backend table).  The append runs in
// the launch that prepares the queries (decode.hip, step_front_kernel).
#include "append.h"
#include "device.h"
#include "host.h"
#include "merge.h"

using namespace bgtq;

namespace {

// fp16 sink and recent-window buffers of a buffered step (n_sink = n_recent = 0: none).
struct StepBuffers {
  uint16_t *k_sink = nullptr, *v_sink = nullptr, *k_recent = nullptr, *v_recent = nullptr;
  int32_t n_sink = 0, n_recent = 0;
};

bgtq_status step_common(const char *nm, const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                        const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos, int32_t batch,
                        int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms, uint32_t *v_codes,
                        uint16_t *v_norms, int64_t capacity, const bgtq_pages *pages, float softmax_scale,
                        uint16_t *out, void *workspace, size_t ws_bytes, bgtq_stream stream,
                        const StepBuffers &bf = StepBuffers()) {
  if (!plan || !dev_consts || !q || !k_new || !v_new || !pos || !k_norms || !v_codes || !v_norms || !out ||
      !workspace || (!k_codes && plan->p.hdr.wk > 0))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null pointer");
  if (bf.n_sink < 0 || bf.n_sink > kMaxSink || bf.n_recent < 0 || bf.n_recent > kMaxRecent)
    return fail(BGTQ_EINVAL, std::string(nm) + ": n_sink must be 0..64 and n_recent 0..65536");
  if ((bf.n_sink && (!bf.k_sink || !bf.v_sink)) || (bf.n_recent && (!bf.k_recent || !bf.v_recent)))
    return fail(BGTQ_EINVAL, std::string(nm) + ": null buffer with a non-zero count");
  if (((uintptr_t)bf.k_sink | (uintptr_t)bf.v_sink | (uintptr_t)bf.k_recent | (uintptr_t)bf.v_recent |
       (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)q) & 15)
    return fail(BGTQ_EINVAL, std::string(nm) + ": q, the new token and the buffers must be 16-byte aligned");
  const Plan &p = plan->p;
  const bgtq_status v = decode_check(p, capacity, batch, max_seq_len, softmax_scale, workspace, ws_bytes, nm);
  if (v != BGTQ_OK) return v;
  const int n = batch * p.desc.n_kv_heads;
  if ((int64_t)n * 3 > 0x7FFFFFFF) return fail(BGTQ_EINVAL, std::string(nm) + ": grid too large");
  const TileMap map = pages ? paged_map(p, pages) : contiguous_map(p.desc.n_kv_heads, capacity);
  const uint8_t *c = (const uint8_t *)dev_consts;
  const AppendArgs ka = append_args(p, c, k_new, k_codes, k_norms, map, false);
  const AppendArgs va = append_args(p, c, v_new, v_codes, v_norms, map, true);
  StepAppend sa{&ka, &va, pos, capacity};
  DecodeCall dc{dev_consts, q, k_codes, k_norms, v_codes, v_norms, capacity, pos, 1, batch, max_seq_len,
                softmax_scale, out, workspace, stream};
  dc.pages = pages;
  dc.step = &sa;
  if (bf.n_sink || bf.n_recent) {
    // the new token into the fp16 buffers in the step's front launch (the buffered merge reads them)
    sa.k_new = k_new, sa.v_new = v_new;
    sa.k_sink = bf.k_sink, sa.v_sink = bf.v_sink, sa.k_recent = bf.k_recent, sa.v_recent = bf.v_recent;
    sa.n_sink = bf.n_sink, sa.n_recent = bf.n_recent;
    dc.k_sink = bf.k_sink;
    dc.v_sink = bf.v_sink;
    dc.k_recent = bf.k_recent;
    dc.v_recent = bf.v_recent;
    dc.n_sink = bf.n_sink;
    dc.n_recent = bf.n_recent;
  }
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

bgtq_status bgtq_decode_step_buffered(const bgtq_plan *plan, const void *dev_consts, const uint16_t *q,
                                      const uint16_t *k_new, const uint16_t *v_new, const int32_t *pos,
                                      int32_t batch, int64_t max_seq_len, uint32_t *k_codes, uint16_t *k_norms,
                                      uint32_t *v_codes, uint16_t *v_norms, int64_t capacity, float softmax_scale,
                                      uint16_t *k_sink, uint16_t *v_sink, int32_t n_sink, uint16_t *k_recent,
                                      uint16_t *v_recent, int32_t n_recent, uint16_t *out, void *workspace,
                                      size_t ws_bytes, bgtq_stream stream) {
  StepBuffers bf;
  bf.k_sink = k_sink, bf.v_sink = v_sink, bf.k_recent = k_recent, bf.v_recent = v_recent;
  bf.n_sink = n_sink, bf.n_recent = n_recent;
  return step_common("bgtq_decode_step_buffered", plan, dev_consts, q, k_new, v_new, pos, batch, max_seq_len,
                     k_codes, k_norms, v_codes, v_norms, capacity, nullptr, softmax_scale, out, workspace, ws_bytes,
                     stream, bf);
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
