// Internal launch interface between the C ABI (zero_api.cpp, offload.cpp) and
// the gfx950 kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/zero.h"

namespace zero {

struct RsParams {
  const uint16_t* g[ZERO_MAX_RANKS];  // rank contributions, numel BF16 each
  float w[ZERO_MAX_RANKS];            // rank weights
  float* out[ZERO_MAX_RANKS];         // owner shards, `shard` FP32 each
  int64_t shard;                      // elements per owner shard
  int n_ranks;
};

struct AdamParams {
  float* p;
  float* m;
  float* v;
  uint16_t* b;
  const float* g;
  const float* gscale;  // device scalar multiplying g (gradient clipping), or NULL
  int64_t n;
  zero_adam_scalars s;
  const zero_adam_scalars* sdev;  // device copy of the scalars (read when the kernel runs), or NULL
};

// Fixed number of partial sums per shard for the gradient norm, so that the
// summation order never depends on the device.
constexpr int kNormBlocks = ZERO_NORM_BLOCKS;

// Doubles of the library-owned partial-sum array of zero_grad_norm_sq_no_alloc
// (one array per GPU): room for every shard's partial sums.
constexpr int kNormScratchDoubles = ZERO_NORM_SCRATCH_DOUBLES;
static_assert(kNormScratchDoubles >= ZERO_MAX_RANKS * kNormBlocks, "scratch holds every partial sum");

struct NormParams {
  const float* x[ZERO_MAX_RANKS];  // shards
  int64_t n;                       // elements per shard
  double* partials;                // n_shards * gx doubles
  double* out;                     // sum of squares
  float* coef;                     // clip coefficient, or NULL
  float max_norm;
  int gx;                          // partial sums per shard
  int n_shards;
};

struct FusedParams {
  const uint16_t* g[ZERO_MAX_RANKS];  // rank contributions, n_shards*shard BF16 each
  float w[ZERO_MAX_RANKS];
  float* p[ZERO_MAX_RANKS];           // per owner: master, m, v (FP32), working shard (BF16)
  float* m[ZERO_MAX_RANKS];
  float* v[ZERO_MAX_RANKS];
  uint16_t* b[ZERO_MAX_RANKS];
  float* gout[ZERO_MAX_RANKS];        // per owner: reduced gradient out, or all NULL
  const float* gacc[ZERO_MAX_RANKS];  // per owner: accumulator added to the reduction, or all NULL
  int64_t shard;
  int n_ranks;
  zero_adam_scalars s;
  const zero_adam_scalars* sdev;  // device copy of the scalars, or NULL
};

struct GatherParams {
  const void* src[ZERO_MAX_RANKS];
  void* dst;
  int64_t shard_bytes;
};

// Each launcher enqueues on `stream` and returns hipSuccess or the launch
// error.  `vec` selects the vector path; the caller has checked its alignment
// conditions: reduce-scatter and fused: shard % 4 == 0, BF16 contribution and
// working-shard pointers 8-byte aligned, FP32 pointers 16-byte aligned;
// Adam: n % 4 tail handled in-kernel, FP32 pointers 16-byte and the BF16
// output 8-byte aligned.
hipError_t launch_reduce_scatter(const RsParams& p, int n_shards, bool accumulate, bool vec,
                                 hipStream_t stream);
// Same with FP32 contributions: p.g holds float pointers (cast).
hipError_t launch_reduce_scatter_f32(const RsParams& p, int n_shards, bool accumulate, bool vec,
                                     hipStream_t stream);
hipError_t launch_adam(const AdamParams& p, bool vec, hipStream_t stream);
hipError_t launch_fused(const FusedParams& p, int n_shards, bool write_grad, bool vec,
                        hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, int n_shards, int path, hipStream_t stream);
// Two passes: per-(block, shard) partial sums of squares, then one block
// folds them in index order and derives the clip coefficient.
hipError_t launch_norm(NormParams& p, bool vec, hipStream_t stream);

// Device address of the current device's partial-sum array for the norm
// (kNormScratchDoubles doubles, 256-byte aligned).  Looked up once per device
// with that device current and cached; allocates nothing.
hipError_t norm_scratch_device_ptr(double** out);

// zero_adam_scalars_fetch: ring is the device-visible address of the pinned
// host ring, ring_len a power of two.
hipError_t launch_scalars_fetch(const zero_adam_scalars* ring, int ring_len, uint32_t* cursor,
                                zero_adam_scalars* out, hipStream_t stream);

// Fill n 32-bit words with `value` (used to poison released staging buffers
// in the offload engine's debug mode).
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t stream);

// Gather path selector: 16-byte, 4-byte or 1-byte units.
enum { GATHER_V16 = 0, GATHER_U32 = 1, GATHER_U8 = 2 };

// A ROCTX range for the lifetime of the object when tracing is on
// (ZERO_ROCTX=1); a no-op otherwise.
class TraceRange {
 public:
  explicit TraceRange(const char* name);
  ~TraceRange();
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;

 private:
  bool on_;
};
int tracing_enabled();

}  // namespace zero
