// Host-offloaded gradient shard with two device slots (blog "数据并行与 ZeRO：
// 三级分片各省多少", section 分片放到 CPU：两个缓冲就够): the gradient shard
// lives in pinned host memory; chunk c of it passes through device slot c % 2.
// While chunk c's reduction runs on the caller's compute stream, the previous
// chunk's result streams to the host on a device-to-host side stream and the
// next chunk's host values stream in on a host-to-device side stream.
//
// Ordering (all by HIP events, never by host waits):
//   staging[s] is written by the H2D copy and by the reduce kernel and read by
//   the reduce kernel (accumulate), the D2H copy and the Adam kernel, so
//     - the H2D into staging[s] waits for the last D2H from it and the last
//       kernel that used it;
//     - a non-accumulating reduce into staging[s] waits for the last D2H from it;
//     - the D2H from staging[s] waits for the reduce kernel that wrote it;
//     - every kernel on slot s waits for the previous one (directly, or
//       through the H2D that it waits for), so kernel_done[s] covers all of
//       them even when the caller changes compute streams between calls.
//   host chunk c is written by its D2H and read by its H2D, so
//     - an H2D of chunk c waits for the last D2H into chunk c;
//     - a D2H into chunk c waits for the last H2D out of chunk c.
//   The contribution slot is consumed by the reduce kernel on the compute
//   stream, so the caller's next writes on that stream follow it in order.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "kernels.h"
#include "validate.h"

namespace zero {
int fail(int status, const char* msg);
int hip_status(hipError_t err, const char* where);
void set_path(bool vec);
}  // namespace zero

using namespace zero;

namespace {

struct Ev {
  hipEvent_t e = nullptr;
  bool recorded = false;
};

// Debug knobs (environment, read at creation): a host-side delay inserted on
// the side streams before every copy, and NaN-poisoning of a staging buffer
// once its D2H copy is done.  Both leave correct results unchanged.
struct Debug {
  int delay_us = 0;
  bool poison = false;
};

void host_sleep(void* arg) {
  const int us = *static_cast<int*>(arg);
  std::this_thread::sleep_for(std::chrono::microseconds(us));
}

}  // namespace

struct zero_offload {
  int device = 0;
  int n_ranks = 0;
  int64_t shard = 0, chunk = 0, n_chunks = 0;
  float* host = nullptr;
  uint16_t* contrib[2] = {nullptr, nullptr};
  float* stage[2] = {nullptr, nullptr};
  hipStream_t h2d = nullptr, d2h = nullptr;
  Ev h2d_done[2], d2h_done[2], kernel_done[2];
  std::vector<Ev> host_written, host_read;
  std::vector<int> last_mb;  // last micro-batch reduced per chunk, -1 = none
  Debug dbg;
  int delay_arg = 0;
};

namespace {

hipError_t record(Ev& ev, hipStream_t s) {
  hipError_t err = hipEventRecord(ev.e, s);
  if (err == hipSuccess) ev.recorded = true;
  return err;
}

hipError_t wait(hipStream_t s, const Ev& ev) {
  return ev.recorded ? hipStreamWaitEvent(s, ev.e, 0) : hipSuccess;
}

hipError_t maybe_delay(zero_offload* h, hipStream_t s) {
  if (h->dbg.delay_us <= 0) return hipSuccess;
  return hipLaunchHostFunc(s, host_sleep, &h->delay_arg);
}

#define ZCHK(expr)                                   \
  do {                                               \
    hipError_t _e = (expr);                          \
    if (_e != hipSuccess) return hip_status(_e, #expr); \
  } while (0)

int check_device(zero_offload* h) {
  int dev = -1;
  ZCHK(hipGetDevice(&dev));
  if (dev != h->device) return fail(ZERO_ERR_STATE, "offload: called with another current device");
  return ZERO_OK;
}

// Copy host chunk c into staging[s] on the H2D stream, then make `compute`
// wait for it.
int stream_in(zero_offload* h, int64_t c, int s, int64_t len, hipStream_t compute) {
  ZCHK(wait(h->h2d, h->d2h_done[s]));
  ZCHK(wait(h->h2d, h->kernel_done[s]));
  ZCHK(wait(h->h2d, h->host_written[c]));
  ZCHK(maybe_delay(h, h->h2d));
  ZCHK(hipMemcpyAsync(h->stage[s], h->host + c * h->chunk, len * sizeof(float),
                      hipMemcpyHostToDevice, h->h2d));
  ZCHK(record(h->h2d_done[s], h->h2d));
  ZCHK(record(h->host_read[c], h->h2d));
  ZCHK(wait(compute, h->h2d_done[s]));
  return ZERO_OK;
}

}  // namespace

extern "C" {

int zero_offload_create(int n_ranks, int64_t shard_numel, int64_t chunk_numel,
                        float* host_shard_pinned, uint16_t* const slot_contrib[2],
                        float* const slot_f32[2], zero_offload** out) {
  Err e;
  if (!out) return fail(ZERO_ERR_ARG, "offload_create: NULL output handle");
  *out = nullptr;
  int st = check_offload_create(n_ranks, shard_numel, chunk_numel, host_shard_pinned, slot_contrib,
                                slot_f32, e);
  if (st) return fail(st, e.msg);
  zero_offload* h = new (std::nothrow) zero_offload();
  if (!h) return fail(ZERO_ERR_SIZE, "offload_create: out of host memory");
  h->n_ranks = n_ranks;
  h->shard = shard_numel;
  h->chunk = chunk_numel;
  h->n_chunks = (shard_numel + chunk_numel - 1) / chunk_numel;
  h->host = host_shard_pinned;
  for (int s = 0; s < 2; ++s) {
    h->contrib[s] = slot_contrib[s];
    h->stage[s] = slot_f32[s];
  }
  const char* d = getenv("ZERO_OFFLOAD_DEBUG_DELAY_US");
  h->dbg.delay_us = d ? atoi(d) : 0;
  h->delay_arg = h->dbg.delay_us;
  const char* p = getenv("ZERO_OFFLOAD_DEBUG_POISON");
  h->dbg.poison = p && atoi(p) != 0;
  auto cleanup = [&](int status) {
    zero_offload_destroy(h);
    return status;
  };
  try {
    h->host_written.resize(h->n_chunks);
    h->host_read.resize(h->n_chunks);
    h->last_mb.assign(h->n_chunks, -1);
  } catch (const std::bad_alloc&) {   // nothing may propagate through the C ABI
    zero_offload_destroy(h);
    return fail(ZERO_ERR_SIZE, "offload_create: out of host memory");
  }
  hipError_t err = hipGetDevice(&h->device);
  if (err == hipSuccess) {
    // pageable memory would turn every asynchronous copy of the shard into a
    // synchronous one: only pinned host memory (known to the runtime) is taken
    void* mapped = nullptr;
    if (hipHostGetDevicePointer(&mapped, host_shard_pinned, 0) != hipSuccess || !mapped) {
      (void)hipGetLastError();
      return cleanup(fail(ZERO_ERR_ARG, "offload_create: the host shard is not pinned host memory "
                                        "(hipHostMalloc or a pinned torch tensor)"));
    }
  }
  if (err == hipSuccess) err = hipStreamCreateWithFlags(&h->h2d, hipStreamNonBlocking);
  if (err == hipSuccess) err = hipStreamCreateWithFlags(&h->d2h, hipStreamNonBlocking);
  for (int s = 0; s < 2 && err == hipSuccess; ++s) {
    Ev* evs[3] = {&h->h2d_done[s], &h->d2h_done[s], &h->kernel_done[s]};
    for (Ev* ev : evs)
      if (err == hipSuccess) err = hipEventCreateWithFlags(&ev->e, hipEventDisableTiming);
  }
  for (int64_t c = 0; c < h->n_chunks && err == hipSuccess; ++c) {
    err = hipEventCreateWithFlags(&h->host_written[c].e, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&h->host_read[c].e, hipEventDisableTiming);
  }
  if (err != hipSuccess) return cleanup(hip_status(err, "zero_offload_create"));
  *out = h;
  return ZERO_OK;
}

int zero_offload_stream(zero_offload* h, int op, int64_t chunk, int micro_batch,
                        const float* rank_weights, float* master, float* exp_avg,
                        float* exp_avg_sq, uint16_t* bf16_out, const zero_adam_hparams* hp,
                        void* compute_stream) {
  TraceRange tr("zero_offload_stream");
  if (!h) return fail(ZERO_ERR_ARG, "offload_stream: NULL handle");
  if (op != ZERO_OFFLOAD_REDUCE && op != ZERO_OFFLOAD_ADAM && op != ZERO_OFFLOAD_REDUCE_ADAM)
    return fail(ZERO_ERR_ARG, "offload_stream: unknown op");
  if (chunk < 0 || chunk >= h->n_chunks) return fail(ZERO_ERR_STATE, "offload_stream: chunk out of range");
  int st = check_device(h);
  if (st) return st;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  const int s = static_cast<int>(chunk & 1);
  const int64_t off = chunk * h->chunk;
  const int64_t len = (h->shard - off < h->chunk) ? h->shard - off : h->chunk;

  if (op == ZERO_OFFLOAD_REDUCE) {
    if (micro_batch < 0) return fail(ZERO_ERR_ARG, "offload_stream: micro_batch < 0");
    if (micro_batch > 0 && h->last_mb[chunk] != micro_batch - 1)
      return fail(ZERO_ERR_STATE, "offload_stream: micro-batch out of order for this chunk");
    if (!rank_weights) return fail(ZERO_ERR_ARG, "offload_stream: NULL rank_weights");
    const uint16_t* g[ZERO_MAX_RANKS];
    for (int r = 0; r < h->n_ranks; ++r) g[r] = h->contrib[s] + r * h->chunk;
    float* outp[1] = {h->stage[s]};
    Err e;
    st = check_reduce_scatter(reinterpret_cast<const void* const*>(g), rank_weights, h->n_ranks, len, outp,
                              1, micro_batch > 0, e);
    if (st) return fail(st, e.msg);
    // staging[s] must be free of its previous D2H reader before it is written
    if (micro_batch > 0) {
      st = stream_in(h, chunk, s, len, cs);
      if (st) return st;
    } else {
      ZCHK(wait(cs, h->d2h_done[s]));
      ZCHK(wait(cs, h->kernel_done[s]));   // an update still reading staging[s] on another stream
    }
    RsParams p;
    memset(&p, 0, sizeof p);
    p.shard = len;
    p.n_ranks = h->n_ranks;
    bool vec = (len % 4) == 0 && aligned16(h->stage[s]);
    for (int r = 0; r < h->n_ranks; ++r) {
      p.g[r] = g[r];
      p.w[r] = rank_weights[r];
      vec = vec && aligned8(g[r]);
    }
    p.out[0] = h->stage[s];
    set_path(vec);
    ZCHK(launch_reduce_scatter(p, 1, micro_batch > 0, vec, cs));
    ZCHK(record(h->kernel_done[s], cs));
    // stream the chunk's new value to the host
    ZCHK(wait(h->d2h, h->kernel_done[s]));
    ZCHK(wait(h->d2h, h->host_read[chunk]));
    ZCHK(maybe_delay(h, h->d2h));
    ZCHK(hipMemcpyAsync(h->host + off, h->stage[s], len * sizeof(float), hipMemcpyDeviceToHost,
                        h->d2h));
    if (h->dbg.poison) ZCHK(launch_fill_u32(reinterpret_cast<uint32_t*>(h->stage[s]), 0x7FC00000u, len, h->d2h));
    ZCHK(record(h->d2h_done[s], h->d2h));
    ZCHK(record(h->host_written[chunk], h->d2h));
    h->last_mb[chunk] = micro_batch;
    return ZERO_OK;
  }

  if (op == ZERO_OFFLOAD_REDUCE_ADAM) {
    // the last micro-batch, reduced and applied in one pass; its sum never
    // goes to the host
    if (micro_batch < 0) return fail(ZERO_ERR_ARG, "offload_stream: micro_batch < 0");
    if (micro_batch > 0 && h->last_mb[chunk] != micro_batch - 1)
      return fail(ZERO_ERR_STATE, "offload_stream: micro-batch out of order for this chunk");
    if (!rank_weights || !master || !exp_avg || !exp_avg_sq || !bf16_out)
      return fail(ZERO_ERR_ARG, "offload_stream: NULL weights or state pointer");
    const uint16_t* g[ZERO_MAX_RANKS];
    for (int r = 0; r < h->n_ranks; ++r) g[r] = h->contrib[s] + r * h->chunk;
    float* pm[1] = {master + off};
    float* mm[1] = {exp_avg + off};
    float* vm[1] = {exp_avg_sq + off};
    uint16_t* bm[1] = {bf16_out + off};
    const float* acc[1] = {h->stage[s]};
    Err e;
    st = check_reduce_scatter_adam(g, rank_weights, h->n_ranks, len, 1, pm, mm, vm, bm,
                                   micro_batch > 0 ? acc : nullptr, nullptr, hp, e);
    if (st) return fail(st, e.msg);
    if (micro_batch > 0) {
      st = stream_in(h, chunk, s, len, cs);
      if (st) return st;
    } else {
      // staging[s] is not used, but kernel_done[s] is recorded again below:
      // keep it after every earlier kernel on the slot, whatever its stream
      ZCHK(wait(cs, h->kernel_done[s]));
    }
    FusedParams p;
    memset(&p, 0, sizeof p);
    p.shard = len;
    p.n_ranks = h->n_ranks;
    adam_scalars(hp, &p.s, e);
    bool vec = (len % 4) == 0;
    for (int r = 0; r < h->n_ranks; ++r) {
      p.g[r] = g[r];
      p.w[r] = rank_weights[r];
      vec = vec && aligned8(g[r]);
    }
    p.p[0] = pm[0];
    p.m[0] = mm[0];
    p.v[0] = vm[0];
    p.b[0] = bm[0];
    p.gacc[0] = micro_batch > 0 ? h->stage[s] : nullptr;
    vec = vec && aligned16(p.p[0]) && aligned16(p.m[0]) && aligned16(p.v[0]) && aligned8(p.b[0]) &&
          aligned16(p.gacc[0]);
    set_path(vec);
    ZCHK(launch_fused(p, 1, false, vec, cs));
    ZCHK(record(h->kernel_done[s], cs));
    h->last_mb[chunk] = -1;   // the accumulation of this chunk is consumed
    return ZERO_OK;
  }

  // ADAM: stream the accumulated chunk back and update the device-resident state
  if (h->last_mb[chunk] < 0) return fail(ZERO_ERR_STATE, "offload_stream: ADAM on a chunk never reduced");
  if (!master || !exp_avg || !exp_avg_sq || !bf16_out)
    return fail(ZERO_ERR_ARG, "offload_stream: NULL state pointer");
  Err e;
  st = check_adam(master + off, exp_avg + off, exp_avg_sq + off, bf16_out + off, h->stage[s], len, hp, e);
  if (st) return fail(st, e.msg);
  st = stream_in(h, chunk, s, len, cs);
  if (st) return st;
  AdamParams a;
  memset(&a, 0, sizeof a);
  a.p = master + off;
  a.m = exp_avg + off;
  a.v = exp_avg_sq + off;
  a.b = bf16_out + off;
  a.g = h->stage[s];
  a.n = len;
  adam_scalars(hp, &a.s, e);
  const bool vec = aligned16(a.p) && aligned16(a.m) && aligned16(a.v) && aligned16(a.g) &&
                   aligned8(a.b);
  set_path(vec);
  ZCHK(launch_adam(a, vec, cs));
  ZCHK(record(h->kernel_done[s], cs));
  h->last_mb[chunk] = -1;   // the accumulation of this chunk is consumed, as after REDUCE_ADAM
  return ZERO_OK;
}

int zero_offload_sync(zero_offload* h) {
  if (!h) return fail(ZERO_ERR_ARG, "offload_sync: NULL handle");
  int st = check_device(h);
  if (st) return st;
  for (int s = 0; s < 2; ++s)
    if (h->kernel_done[s].recorded) ZCHK(hipEventSynchronize(h->kernel_done[s].e));
  ZCHK(hipStreamSynchronize(h->h2d));
  ZCHK(hipStreamSynchronize(h->d2h));
  return ZERO_OK;
}

int zero_offload_destroy(zero_offload* h) {
  if (!h) return ZERO_OK;
  int status = ZERO_OK;
  if (h->h2d) {
    if (hipStreamSynchronize(h->h2d) != hipSuccess) status = ZERO_ERR_HIP;
  }
  if (h->d2h) {
    if (hipStreamSynchronize(h->d2h) != hipSuccess) status = ZERO_ERR_HIP;
  }
  for (int s = 0; s < 2; ++s) {
    if (h->kernel_done[s].recorded) hipEventSynchronize(h->kernel_done[s].e);
    Ev* evs[3] = {&h->h2d_done[s], &h->d2h_done[s], &h->kernel_done[s]};
    for (Ev* ev : evs)
      if (ev->e) hipEventDestroy(ev->e);
  }
  for (auto& ev : h->host_written)
    if (ev.e) hipEventDestroy(ev.e);
  for (auto& ev : h->host_read)
    if (ev.e) hipEventDestroy(ev.e);
  if (h->h2d) hipStreamDestroy(h->h2d);
  if (h->d2h) hipStreamDestroy(h->d2h);
  delete h;
  return status;
}

}  // extern "C"
