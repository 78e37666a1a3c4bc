// Host-only argument checks of the C ABI (no HIP dependency, so they can be
// built with g++ and run under the host sanitizers).  Every function returns
// ZERO_OK or a negative zero_status and writes a message into `err`.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/zero.h"

namespace zero {

struct Err {
  char msg[256];
  Err() { msg[0] = 0; }
};

int set_err(Err& e, int status, const char* fmt, ...);

// [lo, hi) byte ranges of device buffers, used for the overlap checks.
struct Range {
  uintptr_t lo, hi;
};
bool overlaps(Range a, Range b);

// elem_bytes: 2 for BF16 contributions, 4 for FP32 contributions.
int check_reduce_scatter(const void* const* rank_grads, const float* rank_weights,
                         int n_ranks, int64_t numel, float* const* shards_out, int n_shards,
                         int accumulate, Err& e, int elem_bytes = 2);

int check_adam_hparams(const zero_adam_hparams* hp, Err& e);

int check_adam(const float* master, const float* exp_avg, const float* exp_avg_sq,
               const uint16_t* bf16_out, const float* grad, int64_t n,
               const zero_adam_hparams* hp, Err& e);

// The same checks without the hyper-parameters (buffers only), and the
// device-scalar forms: the scalars non-NULL, 4-byte aligned, outside every
// buffer the update writes.
int check_adam_buffers(const float* master, const float* exp_avg, const float* exp_avg_sq,
                       const uint16_t* bf16_out, const float* grad, int64_t n, Err& e);
int check_adam_dev(const float* master, const float* exp_avg, const float* exp_avg_sq,
                   const uint16_t* bf16_out, const float* grad, int64_t n,
                   const zero_adam_scalars* scalars_dev, Err& e);
int check_reduce_scatter_adam_buffers(const uint16_t* const* rank_grads, const float* rank_weights,
                                      int n_ranks, int64_t numel, int n_shards, float* const* master,
                                      float* const* exp_avg, float* const* exp_avg_sq,
                                      uint16_t* const* bf16_out, const float* const* grad_acc,
                                      float* const* grad_out, Err& e);
int check_reduce_scatter_adam_dev(const uint16_t* const* rank_grads, const float* rank_weights,
                                  int n_ranks, int64_t numel, int n_shards, float* const* master,
                                  float* const* exp_avg, float* const* exp_avg_sq,
                                  uint16_t* const* bf16_out, const float* const* grad_acc,
                                  float* const* grad_out, const zero_adam_scalars* scalars_dev, Err& e);
// zero_adam_scalars_fetch without the memory-type check (which needs the
// runtime): non-NULL, 4-byte aligned, ring_len a power of two in 1..65536,
// no overlap between ring, cursor and scalars.
int check_scalars_fetch(const zero_adam_scalars* ring_host, int ring_len, const uint32_t* cursor_dev,
                        const zero_adam_scalars* scalars_dev, Err& e);
// The device scale of zero_adam_shard_step_scaled: non-NULL, 4-byte aligned,
// outside every buffer the update writes.
int check_adam_scale(const float* grad_scale, const float* master, const float* exp_avg,
                     const float* exp_avg_sq, const uint16_t* bf16_out, int64_t n, Err& e);
int check_all_gather(const void* const* shards, int n_shards, int64_t shard_bytes,
                     const void* full_view, Err& e);

int check_offload_create(int n_ranks, int64_t shard_numel, int64_t chunk_numel,
                         const float* host_shard, uint16_t* const slot_contrib[2],
                         float* const slot_f32[2], Err& e);

// Scalars the update kernel uses (binary32 values, see zero_adam_scalars).
int adam_scalars(const zero_adam_hparams* hp, zero_adam_scalars* out, Err& e);

int rank_weights(const int64_t* counts, int n_ranks, float* out, Err& e);

int shard_layout(const int64_t* numels, int n_tensors, int n_shards, int64_t* psi,
                 int64_t* psi_pad, int64_t* shard_numel, Err& e);

int check_reduce_scatter_adam(const uint16_t* const* rank_grads, const float* rank_weights,
                              int n_ranks, int64_t numel, int n_shards, float* const* master,
                              float* const* exp_avg, float* const* exp_avg_sq,
                              uint16_t* const* bf16_out, const float* const* grad_acc,
                              float* const* grad_out, const zero_adam_hparams* hp, Err& e);

int check_grad_norm(const float* const* shards, int n_shards, int64_t shard_numel,
                    const double* workspace, int64_t workspace_len, const double* norm_sq_out,
                    float max_norm, const float* clip_coef_out, Err& e);

// Alignment tests for the kernels' vector paths.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

}  // namespace zero
