// C ABI entry points of libzero (declared in include/zero.h): validate on the
// host, pick the 16-byte or element-wise kernel path, launch on the caller's
// stream.  No call allocates, frees or synchronises.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "validate.h"

namespace zero {

thread_local char g_last_error[320] = "";
thread_local int g_last_vec = -1;

int fail(int status, const char* msg) {
  snprintf(g_last_error, sizeof g_last_error, "%s", msg);
  return status;
}

int hip_status(hipError_t err, const char* where) {
  if (err == hipSuccess) return ZERO_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(err));
  return ZERO_ERR_HIP;
}

void set_path(bool vec) { g_last_vec = vec ? 1 : 0; }

// Optional ROCTX ranges around the device entry points (ZERO_ROCTX=1 in the
// environment when the library is first used): ROCm's roctx library is
// loaded at run time, so nothing is linked or called when tracing is off.
// rocprofv3 --marker-trace then shows one range per call on the host
// timeline.
namespace {
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

const Roctx& roctx() {
  static const Roctx r = [] {
    Roctx x;
    const char* e = std::getenv("ZERO_ROCTX");
    if (!e || std::atoi(e) == 0) return x;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) return x;
    x.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    x.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!x.push || !x.pop) x = Roctx();
    return x;
  }();
  return r;
}
}  // namespace

TraceRange::TraceRange(const char* name) : on_(roctx().push != nullptr) {
  if (on_) roctx().push(name);
}
TraceRange::~TraceRange() {
  if (on_) roctx().pop();
}

int tracing_enabled() { return roctx().push != nullptr ? 1 : 0; }

}  // namespace zero

using namespace zero;

extern "C" {

const char* zero_status_string(int status) {
  switch (status) {
    case ZERO_OK: return "ZERO_OK";
    case ZERO_ERR_ARG: return "ZERO_ERR_ARG: invalid argument";
    case ZERO_ERR_ALIGN: return "ZERO_ERR_ALIGN: misaligned pointer";
    case ZERO_ERR_SIZE: return "ZERO_ERR_SIZE: inconsistent sizes";
    case ZERO_ERR_HIP: return "ZERO_ERR_HIP: HIP runtime error";
    case ZERO_ERR_STATE: return "ZERO_ERR_STATE: offload handle used out of order";
    default: return "unknown zero_status";
  }
}

const char* zero_last_error(void) { return g_last_error; }

int zero_last_path_vectorized(void) { return g_last_vec; }

int zero_tracing_enabled(void) { return tracing_enabled(); }

int zero_adam_scalars_compute(const zero_adam_hparams* hp, zero_adam_scalars* out) {
  Err e;
  int st = adam_scalars(hp, out, e);
  return st ? fail(st, e.msg) : ZERO_OK;
}

int zero_rank_weights(const int64_t* counts, int n_ranks, float* weights_out) {
  Err e;
  int st = rank_weights(counts, n_ranks, weights_out, e);
  return st ? fail(st, e.msg) : ZERO_OK;
}

int zero_shard_layout(const int64_t* numels, int n_tensors, int n_shards, int64_t* psi,
                      int64_t* psi_pad, int64_t* shard_numel) {
  Err e;
  int st = shard_layout(numels, n_tensors, n_shards, psi, psi_pad, shard_numel, e);
  return st ? fail(st, e.msg) : ZERO_OK;
}

int zero_reduce_scatter(const uint16_t* const* rank_grads, const float* rank_weights, int n_ranks,
                        int64_t numel, float* const* shards_out, int n_shards, int accumulate,
                        void* stream) {
  TraceRange tr("zero_reduce_scatter");
  Err e;
  int st = check_reduce_scatter(reinterpret_cast<const void* const*>(rank_grads), rank_weights,
                                n_ranks, numel, shards_out, n_shards, accumulate, e);
  if (st) return fail(st, e.msg);
  if (numel == 0) return ZERO_OK;
  RsParams p;
  memset(&p, 0, sizeof p);
  p.shard = numel / n_shards;
  p.n_ranks = n_ranks;
  bool vec = (p.shard % 4) == 0;
  for (int r = 0; r < n_ranks; ++r) {
    p.g[r] = rank_grads[r];
    p.w[r] = rank_weights[r];
    vec = vec && aligned8(rank_grads[r]);
  }
  for (int k = 0; k < n_shards; ++k) {
    p.out[k] = shards_out[k];
    vec = vec && aligned16(shards_out[k]);
  }
  set_path(vec);
  return hip_status(launch_reduce_scatter(p, n_shards, accumulate != 0, vec,
                                          static_cast<hipStream_t>(stream)),
                    "zero_reduce_scatter");
}

// The update once its buffers (and hyper-parameters or device scalars) are
// checked: the optional gradient scale's checks, then the launch with the host
// scalars `s` or, when sdev is given, the device struct read when it runs.
static int adam_checked(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* bf16_out, const float* grad,
                        const float* grad_scale, int64_t n, const zero_adam_scalars& s,
                        const zero_adam_scalars* sdev, void* stream, const char* where) {
  if (n == 0) return ZERO_OK;
  if (grad_scale) {
    Err e;
    int st = check_adam_scale(grad_scale, master, exp_avg, exp_avg_sq, bf16_out, n, e);
    if (st) return fail(st, e.msg);
  }
  AdamParams a;
  memset(&a, 0, sizeof a);
  a.p = master;
  a.m = exp_avg;
  a.v = exp_avg_sq;
  a.b = bf16_out;
  a.g = grad;
  a.gscale = grad_scale;
  a.n = n;
  a.s = s;
  a.sdev = sdev;
  const bool vec = aligned16(master) && aligned16(exp_avg) && aligned16(exp_avg_sq) &&
                   aligned16(grad) && aligned8(bf16_out);
  set_path(vec);
  return hip_status(launch_adam(a, vec, static_cast<hipStream_t>(stream)), where);
}

static int adam_common(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* bf16_out,
                       const float* grad, const float* grad_scale, int64_t n,
                       const zero_adam_hparams* hp, void* stream, const char* where) {
  Err e;
  int st = check_adam(master, exp_avg, exp_avg_sq, bf16_out, grad, n, hp, e);
  if (st) return fail(st, e.msg);
  zero_adam_scalars sc;
  memset(&sc, 0, sizeof sc);
  adam_scalars(hp, &sc, e);
  return adam_checked(master, exp_avg, exp_avg_sq, bf16_out, grad, grad_scale, n, sc, nullptr, stream, where);
}

int zero_reduce_scatter_f32(const float* const* rank_grads, const float* rank_weights, int n_ranks,
                            int64_t numel, float* const* shards_out, int n_shards, int accumulate,
                            void* stream) {
  TraceRange tr("zero_reduce_scatter_f32");
  Err e;
  int st = check_reduce_scatter(reinterpret_cast<const void* const*>(rank_grads), rank_weights, n_ranks,
                                numel, shards_out, n_shards, accumulate, e, 4);
  if (st) return fail(st, e.msg);
  if (numel == 0) return ZERO_OK;
  RsParams p;
  memset(&p, 0, sizeof p);
  p.shard = numel / n_shards;
  p.n_ranks = n_ranks;
  bool vec = (p.shard % 4) == 0;
  for (int r = 0; r < n_ranks; ++r) {
    p.g[r] = reinterpret_cast<const uint16_t*>(rank_grads[r]);
    p.w[r] = rank_weights[r];
    vec = vec && aligned16(rank_grads[r]);
  }
  for (int k = 0; k < n_shards; ++k) {
    p.out[k] = shards_out[k];
    vec = vec && aligned16(shards_out[k]);
  }
  set_path(vec);
  return hip_status(launch_reduce_scatter_f32(p, n_shards, accumulate != 0, vec,
                                              static_cast<hipStream_t>(stream)),
                    "zero_reduce_scatter_f32");
}

int zero_adam_shard_step(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* bf16_out,
                         const float* grad, int64_t n, const zero_adam_hparams* hp, void* stream) {
  TraceRange tr("zero_adam_shard_step");
  return adam_common(master, exp_avg, exp_avg_sq, bf16_out, grad, nullptr, n, hp, stream,
                     "zero_adam_shard_step");
}

int zero_adam_shard_step_scaled(float* master, float* exp_avg, float* exp_avg_sq,
                                uint16_t* bf16_out, const float* grad, const float* grad_scale,
                                int64_t n, const zero_adam_hparams* hp, void* stream) {
  TraceRange tr("zero_adam_shard_step_scaled");
  if (!grad_scale && n > 0) return fail(ZERO_ERR_ARG, "adam_scaled: NULL grad_scale");
  return adam_common(master, exp_avg, exp_avg_sq, bf16_out, grad, grad_scale, n, hp, stream,
                     "zero_adam_shard_step_scaled");
}

// Both norm entry points: checks, then the two norm launches with `partials`
// (a caller workspace of workspace_len doubles, or the library's own array).
static int norm_common(const float* const* shards, int n_shards, int64_t shard_numel, double* partials,
                       int64_t partials_len, double* norm_sq_out, float max_norm, float* clip_coef_out,
                       void* stream, const char* where) {
  Err e;
  int st = check_grad_norm(shards, n_shards, shard_numel, partials, partials_len, norm_sq_out, max_norm,
                           clip_coef_out, e);
  if (st) return fail(st, e.msg);
  NormParams p;
  memset(&p, 0, sizeof p);
  p.n = shard_numel;
  p.n_shards = n_shards;
  p.partials = partials;
  p.out = norm_sq_out;
  p.coef = clip_coef_out;
  p.max_norm = max_norm;
  bool vec = true;
  for (int k = 0; k < n_shards; ++k) {
    p.x[k] = shards[k];
    vec = vec && aligned16(shards[k]);
  }
  set_path(vec);
  return hip_status(launch_norm(p, vec, static_cast<hipStream_t>(stream)), where);
}

int zero_grad_norm_sq(const float* const* shards, int n_shards, int64_t shard_numel,
                      double* workspace, int64_t workspace_len, double* norm_sq_out,
                      float max_norm, float* clip_coef_out, void* stream) {
  TraceRange tr("zero_grad_norm_sq");
  return norm_common(shards, n_shards, shard_numel, workspace, workspace_len, norm_sq_out, max_norm,
                     clip_coef_out, stream, "zero_grad_norm_sq");
}

int zero_grad_norm_sq_no_alloc(const float* const* shards, int n_shards, int64_t shard_numel,
                               double* norm_sq_out, float max_norm, float* clip_coef_out,
                               void* stream) {
  TraceRange tr("zero_grad_norm_sq_no_alloc");
  double* scratch_dev = nullptr;
  int st = hip_status(norm_scratch_device_ptr(&scratch_dev), "zero_grad_norm_sq_no_alloc: scratch address");
  if (st) return st;
  if (n_shards >= 1 && n_shards <= ZERO_MAX_RANKS &&
      static_cast<int64_t>(n_shards) * ZERO_NORM_BLOCKS > kNormScratchDoubles)
    return fail(ZERO_ERR_SIZE, "grad_norm_no_alloc: the partial sums exceed the library's array");
  return norm_common(shards, n_shards, shard_numel, scratch_dev, kNormScratchDoubles, norm_sq_out, max_norm,
                     clip_coef_out, stream, "zero_grad_norm_sq_no_alloc");
}

int zero_adam_shard_step_dev(float* master, float* exp_avg, float* exp_avg_sq, uint16_t* bf16_out,
                             const float* grad, const float* grad_scale, int64_t n,
                             const zero_adam_scalars* scalars_dev, void* stream) {
  TraceRange tr("zero_adam_shard_step_dev");
  Err e;
  int st = check_adam_dev(master, exp_avg, exp_avg_sq, bf16_out, grad, n, scalars_dev, e);
  if (st) return fail(st, e.msg);
  zero_adam_scalars unused;
  memset(&unused, 0, sizeof unused);
  return adam_checked(master, exp_avg, exp_avg_sq, bf16_out, grad, grad_scale, n, unused, scalars_dev, stream,
                      "zero_adam_shard_step_dev");
}

static int fused_common(const uint16_t* const* rank_grads, const float* rank_weights, int n_ranks,
                        int64_t numel, int n_shards, float* const* master, float* const* exp_avg,
                        float* const* exp_avg_sq, uint16_t* const* bf16_out,
                        const float* const* grad_acc, float* const* grad_out, const zero_adam_scalars& s,
                        const zero_adam_scalars* sdev, void* stream, const char* where) {
  FusedParams p;
  memset(&p, 0, sizeof p);
  p.shard = numel / n_shards;
  p.n_ranks = n_ranks;
  p.s = s;
  p.sdev = sdev;
  bool vec = (p.shard % 4) == 0;
  for (int r = 0; r < n_ranks; ++r) {
    p.g[r] = rank_grads[r];
    p.w[r] = rank_weights[r];
    vec = vec && aligned8(rank_grads[r]);
  }
  for (int k = 0; k < n_shards; ++k) {
    p.p[k] = master[k];
    p.m[k] = exp_avg[k];
    p.v[k] = exp_avg_sq[k];
    p.b[k] = bf16_out[k];
    p.gout[k] = grad_out ? grad_out[k] : nullptr;
    p.gacc[k] = grad_acc ? grad_acc[k] : nullptr;
    vec = vec && aligned16(p.p[k]) && aligned16(p.m[k]) && aligned16(p.v[k]) && aligned8(p.b[k]) &&
          aligned16(p.gout[k]) && aligned16(p.gacc[k]);
  }
  set_path(vec);
  return hip_status(launch_fused(p, n_shards, grad_out != nullptr, vec, static_cast<hipStream_t>(stream)),
                    where);
}

int zero_reduce_scatter_adam_dev(const uint16_t* const* rank_grads, const float* rank_weights,
                                 int n_ranks, int64_t numel, int n_shards, float* const* master,
                                 float* const* exp_avg, float* const* exp_avg_sq,
                                 uint16_t* const* bf16_out, const float* const* grad_acc,
                                 float* const* grad_out, const zero_adam_scalars* scalars_dev,
                                 void* stream) {
  TraceRange tr("zero_reduce_scatter_adam_dev");
  Err e;
  int st = check_reduce_scatter_adam_dev(rank_grads, rank_weights, n_ranks, numel, n_shards, master,
                                         exp_avg, exp_avg_sq, bf16_out, grad_acc, grad_out, scalars_dev, e);
  if (st) return fail(st, e.msg);
  if (numel == 0) return ZERO_OK;
  zero_adam_scalars unused;
  memset(&unused, 0, sizeof unused);
  return fused_common(rank_grads, rank_weights, n_ranks, numel, n_shards, master, exp_avg, exp_avg_sq,
                      bf16_out, grad_acc, grad_out, unused, scalars_dev, stream, "zero_reduce_scatter_adam_dev");
}

// The ring must be pinned host memory mapped for the device, with all
// ring_len structs inside that one allocation: the kernel reads it through
// the device mapping, and a pageable or short ring would fault there.  On
// success *dev_ring is the ring's device-visible address.
static int pinned_ring(const zero_adam_scalars* ring, int ring_len, const zero_adam_scalars** dev_ring) {
  hipPointerAttribute_t at;
  memset(&at, 0, sizeof at);
  if (hipPointerGetAttributes(&at, ring) != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer ||
      !at.hostPointer) {
    (void)hipGetLastError();  // leave no error behind for the next launch check to report
    return fail(ZERO_ERR_ARG, "zero_adam_scalars_fetch: ring_host is not pinned host memory (hipHostMalloc)");
  }
  void* start = nullptr;
  size_t size = 0;
  if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR,
                             reinterpret_cast<hipDeviceptr_t>(const_cast<zero_adam_scalars*>(ring))) != hipSuccess ||
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE,
                             reinterpret_cast<hipDeviceptr_t>(const_cast<zero_adam_scalars*>(ring))) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ZERO_ERR_ARG, "zero_adam_scalars_fetch: the ring's pinned allocation could not be determined");
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(start), hi = lo + size;
  const uintptr_t r0 = reinterpret_cast<uintptr_t>(ring);
  const uintptr_t r1 = r0 + static_cast<uintptr_t>(ring_len) * sizeof(zero_adam_scalars);
  if (r0 < lo || r1 > hi || r1 < r0)
    return fail(ZERO_ERR_ARG, "zero_adam_scalars_fetch: ring_len structs do not fit in the ring's pinned allocation");
  // the device address of `ring`, whether the runtime reports the pointers of
  // the allocation's start or of the queried address
  const intptr_t off = static_cast<intptr_t>(r0 - reinterpret_cast<uintptr_t>(at.hostPointer));
  *dev_ring = reinterpret_cast<const zero_adam_scalars*>(static_cast<char*>(at.devicePointer) + off);
  return ZERO_OK;
}

int zero_adam_scalars_fetch(const zero_adam_scalars* ring_host, int ring_len, uint32_t* cursor_dev,
                            zero_adam_scalars* scalars_dev, void* stream) {
  TraceRange tr("zero_adam_scalars_fetch");
  Err e;
  int st = check_scalars_fetch(ring_host, ring_len, cursor_dev, scalars_dev, e);
  if (st) return fail(st, e.msg);
  const zero_adam_scalars* dev_ring = nullptr;
  st = pinned_ring(ring_host, ring_len, &dev_ring);
  if (st) return st;
  return hip_status(launch_scalars_fetch(dev_ring, ring_len, cursor_dev, scalars_dev, static_cast<hipStream_t>(stream)),
                    "zero_adam_scalars_fetch");
}

int zero_reduce_scatter_adam(const uint16_t* const* rank_grads, const float* rank_weights,
                             int n_ranks, int64_t numel, int n_shards, float* const* master,
                             float* const* exp_avg, float* const* exp_avg_sq,
                             uint16_t* const* bf16_out, const float* const* grad_acc,
                             float* const* grad_out, const zero_adam_hparams* hp, void* stream) {
  TraceRange tr("zero_reduce_scatter_adam");
  Err e;
  int st = check_reduce_scatter_adam(rank_grads, rank_weights, n_ranks, numel, n_shards, master,
                                     exp_avg, exp_avg_sq, bf16_out, grad_acc, grad_out, hp, e);
  if (st) return fail(st, e.msg);
  if (numel == 0) return ZERO_OK;
  zero_adam_scalars sc;
  adam_scalars(hp, &sc, e);
  return fused_common(rank_grads, rank_weights, n_ranks, numel, n_shards, master, exp_avg, exp_avg_sq,
                      bf16_out, grad_acc, grad_out, sc, nullptr, stream, "zero_reduce_scatter_adam");
}

int zero_all_gather_layer(const void* const* shards, int n_shards, int64_t shard_bytes,
                          void* full_view, void* stream) {
  TraceRange tr("zero_all_gather_layer");
  Err e;
  int st = check_all_gather(shards, n_shards, shard_bytes, full_view, e);
  if (st) return fail(st, e.msg);
  if (shard_bytes == 0) return ZERO_OK;
  GatherParams p;
  memset(&p, 0, sizeof p);
  p.dst = full_view;
  p.shard_bytes = shard_bytes;
  uintptr_t bits = reinterpret_cast<uintptr_t>(full_view) | static_cast<uintptr_t>(shard_bytes);
  for (int k = 0; k < n_shards; ++k) {
    p.src[k] = shards[k];
    bits |= reinterpret_cast<uintptr_t>(shards[k]);
  }
  const int path = (bits & 15u) == 0 ? GATHER_V16 : (bits & 3u) == 0 ? GATHER_U32 : GATHER_U8;
  set_path(path == GATHER_V16);
  return hip_status(launch_gather(p, n_shards, path, static_cast<hipStream_t>(stream)),
                    "zero_all_gather_layer");
}

}  // extern "C"
