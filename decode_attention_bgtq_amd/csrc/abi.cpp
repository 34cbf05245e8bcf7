// Host side of the C ABI: errors, plans, inspection and profiling.
#include <atomic>
#include <cmath>
#include <cstring>
#include <new>

#include "host.h"

namespace bgtq {
namespace {
thread_local std::string g_err;
}  // namespace

bgtq_status fail(bgtq_status s, const std::string &m) {
  g_err = m;
  return s;
}

bgtq_status launch_status(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGTQ_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return BGTQ_OK;
}

// Compute units of the current device, queried once per device (the launch
// shapes of every call depend on it; the attribute query is not free).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

Prof &prof() {
  static Prof p;
  return p;
}

const char *last_error() { return g_err.c_str(); }

}  // namespace bgtq

using namespace bgtq;

extern "C" {

int32_t bgtq_abi_version(void) { return BGTQ_ABI_VERSION; }

const char *bgtq_last_error(void) { return last_error(); }

bgtq_status bgtq_plan_create(const bgtq_plan_desc *desc, bgtq_plan **out) {
  if (!desc || !out) return fail(BGTQ_EINVAL, "bgtq_plan_create: null pointer");
  *out = nullptr;
  bgtq_plan *p = new (std::nothrow) bgtq_plan();
  if (!p) return fail(BGTQ_EINVAL, "bgtq_plan_create: out of host memory");
  std::string err;
  const bgtq_status s = build_plan(*desc, p->p, err);
  if (s != BGTQ_OK) {
    delete p;
    return fail(s, "bgtq_plan_create: " + err);
  }
  *out = p;
  return BGTQ_OK;
}

void bgtq_plan_destroy(bgtq_plan *plan) { delete plan; }

bgtq_status bgtq_plan_sizes(const bgtq_plan *plan, int32_t batch, int64_t capacity, bgtq_sizes *out) {
  if (!plan || !out) return fail(BGTQ_EINVAL, "bgtq_plan_sizes: null pointer");
  if (batch < 1 || capacity < 0) return fail(BGTQ_EINVAL, "bgtq_plan_sizes: batch >= 1, capacity >= 0");
  const Plan &p = plan->p;
  const uint64_t tiles = (uint64_t)((capacity + kTile - 1) / kTile);
  const uint64_t bh = (uint64_t)batch * p.desc.n_kv_heads;
  out->consts = p.image.size();
  out->k_codes = bh * tiles * p.hdr.wk * kTile * 4;
  out->k_norms = bh * tiles * kTile * 4 * 2;
  out->v_codes = bh * tiles * kHeadDim * p.hdr.wv * 4;
  out->v_norms = bh * tiles * kTile * 2;
  return BGTQ_OK;
}

bgtq_status bgtq_plan_upload(const bgtq_plan *plan, void *dev_consts, bgtq_stream stream) {
  if (!plan || !dev_consts) return fail(BGTQ_EINVAL, "bgtq_plan_upload: null pointer");
  if ((uintptr_t)dev_consts & 255) return fail(BGTQ_EINVAL, "bgtq_plan_upload: dev_consts must be 256-byte aligned");
  const hipError_t e = hipMemcpyAsync(dev_consts, plan->p.image.data(), plan->p.image.size(),
                                      hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BGTQ_EDEVICE, std::string("bgtq_plan_upload: ") + hipGetErrorString(e));
  return BGTQ_OK;
}

bgtq_status bgtq_codebook(int32_t bits, double *centroids, double *thresholds, double *distortion) {
  if (bits < 1 || bits > 4) return fail(BGTQ_EINVAL, "bgtq_codebook: bits must be 1..4");
  const Codebook &cb = codebook(bits);
  if (centroids) std::memcpy(centroids, cb.c.data(), sizeof(double) * cb.c.size());
  if (thresholds) std::memcpy(thresholds, cb.t.data(), sizeof(double) * cb.t.size());
  if (distortion) *distortion = cb.d;
  return BGTQ_OK;
}

bgtq_status bgtq_plan_rotation(const bgtq_plan *plan, int32_t kvh, int32_t tensor, int32_t width, double *out,
                               int32_t *dim) {
  if (!plan || !dim) return fail(BGTQ_EINVAL, "bgtq_plan_rotation: null pointer");
  const Plan &p = plan->p;
  if (kvh < 0 || kvh >= p.desc.n_kv_heads || (tensor != 0 && tensor != 1))
    return fail(BGTQ_EINVAL, "bgtq_plan_rotation: bad head or tensor");
  if (tensor == 1) {
    if (width != p.desc.v_bits) {
      *dim = 0;
      return BGTQ_OK;
    }
    *dim = kHeadDim;
    if (out) std::memcpy(out, p.rot_v[kvh].data(), sizeof(double) * kHeadDim * kHeadDim);
    return BGTQ_OK;
  }
  size_t gidx = 0;
  for (int h = 0; h < kvh; ++h) gidx += p.kvh[h].n_groups;
  for (int gi = 0; gi < p.kvh[kvh].n_groups; ++gi)
    if (p.kvh[kvh].g[gi].w == width) {
      const int d = p.kvh[kvh].g[gi].d;
      *dim = d;
      if (out) std::memcpy(out, p.rot_k[gidx + gi].data(), sizeof(double) * d * d);
      return BGTQ_OK;
    }
  *dim = 0;
  return BGTQ_OK;
}

bgtq_status bgtq_plan_bits(const bgtq_plan *plan, int8_t *bits) {
  if (!plan || !bits) return fail(BGTQ_EINVAL, "bgtq_plan_bits: null pointer");
  std::memcpy(bits, plan->p.bits.data(), plan->p.bits.size());
  return BGTQ_OK;
}

bgtq_status bgtq_profile_enable(int32_t on) {
  Prof &pr = prof();
  std::lock_guard<std::mutex> lk(pr.mu);
  pr.on = on != 0;
  return BGTQ_OK;
}

bgtq_status bgtq_profile_read(double *stream_kernel_ms, int64_t *launches) {
  if (!stream_kernel_ms || !launches) return fail(BGTQ_EINVAL, "bgtq_profile_read: null pointer");
  Prof &pf = prof();
  std::lock_guard<std::mutex> lk(pf.mu);
  double total = 0.0;
  int64_t n = 0;
  for (auto &ev : pf.pending) {
    if (hipEventSynchronize(ev.second) != hipSuccess) return fail(BGTQ_EDEVICE, "bgtq_profile_read: event wait failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
      return fail(BGTQ_EDEVICE, "bgtq_profile_read: elapsed time failed");
    total += ms;
    ++n;
    pf.pool.push_back(ev);
  }
  pf.pending.clear();
  *stream_kernel_ms = total;
  *launches = n;
  return BGTQ_OK;
}

}  // extern "C"
