// Host offload of cached per-layer metadata (the anchor residual R) with a
// one-layer-ahead prefetch (research walkthrough page, method step 5; paper
// landing page, Table 8). Pinned host blobs, two device slots used in turn,
// and events that order the copies against the compute stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>
#include <new>
#include <vector>

#include "mcsparse.h"


namespace mcs {
// shared with mcs_api.cpp through the same thread-local slot
void set_last_error(const char *msg);
}

struct mcs_rcache {
  int32_t n_layers = 0;
  size_t bytes = 0;
  char *host = nullptr;
  void *slot[2] = {nullptr, nullptr};
  hipEvent_t ready[2] = {nullptr, nullptr};  // prefetch into the slot finished
  hipEvent_t freed[2] = {nullptr, nullptr};  // the slot's last reader finished
  hipStream_t reader[2] = {nullptr, nullptr};
  bool acquired[2] = {false, false};          // the slot has a reader since its last prefetch
  int32_t slot_layer[2] = {-1, -1};
  std::vector<char> stored;
  // per layer: the last store's D2H copy into the blob finished, and the
  // last prefetch's H2D copy out of the blob finished. A prefetch waits for
  // the first and a store for the second, so the two may run on any streams.
  std::vector<hipEvent_t> store_done, fetch_done;
  std::vector<char> fetch_pending;
};

namespace {

// two events per layer order stores against prefetches
constexpr int32_t kMaxLayers = 1 << 16;

mcs_status_t fail(mcs_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  mcs::set_last_error(buf);
  return st;
}

mcs_status_t hipfail(hipError_t e, const char *what) {
  return fail(MCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call, what)                   \
  do {                                        \
    const hipError_t _e = (call);             \
    if (_e != hipSuccess) return hipfail(_e, what); \
  } while (0)

mcs_status_t check_layer(const mcs_rcache *c, int32_t layer) {
  if (!c) return fail(MCS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (layer < 0 || layer >= c->n_layers)
    return fail(MCS_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, c->n_layers);
  return MCS_OK;
}

void release(mcs_rcache *c) {
  for (hipEvent_t e : c->store_done)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->fetch_done)
    if (e) (void)hipEventDestroy(e);
  for (int s = 0; s < 2; ++s) {
    if (c->ready[s]) (void)hipEventDestroy(c->ready[s]);
    if (c->freed[s]) (void)hipEventDestroy(c->freed[s]);
    if (c->slot[s]) (void)hipFree(c->slot[s]);
  }
  if (c->host) (void)hipHostFree(c->host);
  delete c;
}

}  // namespace

extern "C" {

mcs_status_t mcs_rcache_create(int32_t n_layers, size_t bytes_per_layer, mcs_rcache_t **out) {
  if (!out) return fail(MCS_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (n_layers < 1 || n_layers > kMaxLayers)
    return fail(MCS_ERR_INVALID_ARGUMENT, "n_layers %d outside [1, %d]", n_layers, kMaxLayers);
  if (bytes_per_layer == 0 || bytes_per_layer % 16)
    return fail(MCS_ERR_INVALID_ARGUMENT, "bytes_per_layer must be a positive multiple of 16");
  size_t host_bytes;
  if (__builtin_mul_overflow((size_t)n_layers, bytes_per_layer, &host_bytes))
    return fail(MCS_ERR_INVALID_ARGUMENT, "n_layers * bytes_per_layer overflows");
  mcs_rcache *c = new (std::nothrow) mcs_rcache();
  if (!c) return fail(MCS_ERR_INVALID_ARGUMENT, "out of host memory for the cache state");
  c->n_layers = n_layers;
  c->bytes = bytes_per_layer;
  try {
    c->stored.assign(n_layers, 0);
    c->fetch_pending.assign(n_layers, 0);
    c->store_done.assign(n_layers, nullptr);
    c->fetch_done.assign(n_layers, nullptr);
  } catch (const std::bad_alloc &) {
    delete c;
    return fail(MCS_ERR_INVALID_ARGUMENT, "out of host memory for %d layer flags", n_layers);
  }
  hipError_t e = hipHostMalloc((void **)&c->host, host_bytes, hipHostMallocDefault);
  for (int32_t l = 0; l < n_layers && e == hipSuccess; ++l) {
    e = hipEventCreateWithFlags(&c->store_done[l], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->fetch_done[l], hipEventDisableTiming);
  }
  for (int s = 0; s < 2 && e == hipSuccess; ++s) {
    e = hipMalloc(&c->slot[s], bytes_per_layer);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ready[s], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->freed[s], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    release(c);
    return hipfail(e, "mcs_rcache_create");
  }
  *out = c;
  return MCS_OK;
}

mcs_status_t mcs_rcache_store(mcs_rcache_t *c, int32_t layer, const void *src, mcs_stream_t stream) {
  const mcs_status_t st = check_layer(c, layer);
  if (st != MCS_OK) return st;
  if (!src) return fail(MCS_ERR_INVALID_ARGUMENT, "src is NULL");
  // a prefetch of this layer may still be reading the blob
  if (c->fetch_pending[layer])
    HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, c->fetch_done[layer], 0), "mcs_rcache_store");
  HIP_TRY(hipMemcpyAsync(c->host + (size_t)layer * c->bytes, src, c->bytes, hipMemcpyDeviceToHost,
                         (hipStream_t)stream),
          "mcs_rcache_store");
  HIP_TRY(hipEventRecord(c->store_done[layer], (hipStream_t)stream), "mcs_rcache_store");
  c->stored[layer] = 1;
  return MCS_OK;
}

mcs_status_t mcs_rcache_prefetch(mcs_rcache_t *c, int32_t layer, mcs_stream_t stream) {
  const mcs_status_t st = check_layer(c, layer);
  if (st != MCS_OK) return st;
  if (!c->stored[layer]) return fail(MCS_ERR_STATE, "layer %d was never stored", layer);
  const int s = layer & 1;
  if (c->acquired[s]) {
    // everything enqueued so far on the stream that last acquired this slot
    // (its reader kernels) must finish before the slot is overwritten
    HIP_TRY(hipEventRecord(c->freed[s], c->reader[s]), "mcs_rcache_prefetch");
    HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, c->freed[s], 0), "mcs_rcache_prefetch");
    c->acquired[s] = false;
  }
  // an earlier prefetch into this slot, on whatever stream, has finished
  // writing it (otherwise the two copies would race on the slot)
  if (c->slot_layer[s] >= 0)
    HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, c->ready[s], 0), "mcs_rcache_prefetch");
  // the blob's last store has landed in host memory
  HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, c->store_done[layer], 0), "mcs_rcache_prefetch");
  HIP_TRY(hipMemcpyAsync(c->slot[s], c->host + (size_t)layer * c->bytes, c->bytes, hipMemcpyHostToDevice,
                         (hipStream_t)stream),
          "mcs_rcache_prefetch");
  HIP_TRY(hipEventRecord(c->ready[s], (hipStream_t)stream), "mcs_rcache_prefetch");
  HIP_TRY(hipEventRecord(c->fetch_done[layer], (hipStream_t)stream), "mcs_rcache_prefetch");
  c->fetch_pending[layer] = 1;
  c->slot_layer[s] = layer;
  return MCS_OK;
}

mcs_status_t mcs_rcache_acquire(mcs_rcache_t *c, int32_t layer, mcs_stream_t stream, const void **dev_ptr) {
  const mcs_status_t st = check_layer(c, layer);
  if (st != MCS_OK) return st;
  if (!dev_ptr) return fail(MCS_ERR_INVALID_ARGUMENT, "dev_ptr is NULL");
  const int s = layer & 1;
  if (c->slot_layer[s] != layer) return fail(MCS_ERR_STATE, "layer %d is not the last prefetch into its slot", layer);
  HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, c->ready[s], 0), "mcs_rcache_acquire");
  c->reader[s] = (hipStream_t)stream;
  c->acquired[s] = true;
  *dev_ptr = c->slot[s];
  return MCS_OK;
}

mcs_status_t mcs_rcache_host_ptr(mcs_rcache_t *c, int32_t layer, const void **host_ptr) {
  const mcs_status_t st = check_layer(c, layer);
  if (st != MCS_OK) return st;
  if (!host_ptr) return fail(MCS_ERR_INVALID_ARGUMENT, "host_ptr is NULL");
  *host_ptr = c->host + (size_t)layer * c->bytes;
  return MCS_OK;
}

mcs_status_t mcs_rcache_destroy(mcs_rcache_t *c) {
  if (!c) return fail(MCS_ERR_INVALID_ARGUMENT, "cache is NULL");
  const hipError_t e = hipDeviceSynchronize();
  release(c);
  if (e != hipSuccess) return hipfail(e, "mcs_rcache_destroy");
  return MCS_OK;
}

}  // extern "C"
