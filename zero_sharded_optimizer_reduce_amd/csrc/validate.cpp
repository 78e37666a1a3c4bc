// Host-only argument checks and host-side scalars of the C ABI.
#include "validate.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace zero {

int set_err(Err& e, int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(e.msg, sizeof e.msg, fmt, ap);
  va_end(ap);
  return status;
}

bool overlaps(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

static Range range_of(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

static bool mul_overflows(int64_t a, int64_t b) {
  return a != 0 && b > INT64_MAX / a;
}

int check_reduce_scatter(const void* const* rank_grads, const float* rank_weights,
                         int n_ranks, int64_t numel, float* const* shards_out, int n_shards,
                         int accumulate, Err& e, int elem_bytes) {
  if (!rank_grads || !rank_weights || !shards_out)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter: NULL pointer table or weights");
  if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter: n_ranks=%d outside [1,%d]", n_ranks, ZERO_MAX_RANKS);
  if (n_shards < 1 || n_shards > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter: n_shards=%d outside [1,%d]", n_shards, ZERO_MAX_RANKS);
  if (numel < 0) return set_err(e, ZERO_ERR_ARG, "reduce_scatter: numel=%lld < 0", (long long)numel);
  if (accumulate != 0 && accumulate != 1)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter: accumulate must be 0 or 1");
  if (numel % n_shards != 0)
    return set_err(e, ZERO_ERR_SIZE, "reduce_scatter: numel=%lld not divisible by n_shards=%d",
                   (long long)numel, n_shards);
  if (mul_overflows(numel, 4)) return set_err(e, ZERO_ERR_SIZE, "reduce_scatter: numel too large");
  const int64_t shard = numel / n_shards;
  // an empty reduction touches no buffer, so its pointers may be NULL (as
  // PyTorch's empty tensors are)
  if (numel == 0) return ZERO_OK;
  for (int r = 0; r < n_ranks; ++r) {
    if (!rank_grads[r]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter: rank_grads[%d] is NULL", r);
    if (reinterpret_cast<uintptr_t>(rank_grads[r]) & static_cast<uintptr_t>(elem_bytes - 1))
      return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter: rank_grads[%d] not %d-byte aligned", r, elem_bytes);
  }
  for (int k = 0; k < n_shards; ++k) {
    if (!shards_out[k]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter: shards_out[%d] is NULL", k);
    if (reinterpret_cast<uintptr_t>(shards_out[k]) & 3u)
      return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter: shards_out[%d] not 4-byte aligned", k);
  }
  for (int k = 0; k < n_shards; ++k) {
    Range ok = range_of(shards_out[k], shard * 4);
    for (int j = k + 1; j < n_shards; ++j)
      if (overlaps(ok, range_of(shards_out[j], shard * 4)))
        return set_err(e, ZERO_ERR_ARG, "reduce_scatter: shards_out[%d] and [%d] overlap", k, j);
    for (int r = 0; r < n_ranks; ++r)
      if (overlaps(ok, range_of(rank_grads[r], numel * elem_bytes)))
        return set_err(e, ZERO_ERR_ARG, "reduce_scatter: shards_out[%d] overlaps rank_grads[%d]", k, r);
  }
  return ZERO_OK;
}

int check_reduce_scatter_adam(const uint16_t* const* rank_grads, const float* rank_weights,
                              int n_ranks, int64_t numel, int n_shards, float* const* master,
                              float* const* exp_avg, float* const* exp_avg_sq,
                              uint16_t* const* bf16_out, const float* const* grad_acc,
                              float* const* grad_out, const zero_adam_hparams* hp, Err& e) {
  int st = check_adam_hparams(hp, e);
  if (st) return st;
  return check_reduce_scatter_adam_buffers(rank_grads, rank_weights, n_ranks, numel, n_shards, master,
                                           exp_avg, exp_avg_sq, bf16_out, grad_acc, grad_out, e);
}

int check_reduce_scatter_adam_dev(const uint16_t* const* rank_grads, const float* rank_weights,
                                  int n_ranks, int64_t numel, int n_shards, float* const* master,
                                  float* const* exp_avg, float* const* exp_avg_sq,
                                  uint16_t* const* bf16_out, const float* const* grad_acc,
                                  float* const* grad_out, const zero_adam_scalars* scalars_dev, Err& e) {
  int st = check_reduce_scatter_adam_buffers(rank_grads, rank_weights, n_ranks, numel, n_shards, master,
                                             exp_avg, exp_avg_sq, bf16_out, grad_acc, grad_out, e);
  if (st) return st;
  if (!scalars_dev) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: NULL device scalars");
  if (reinterpret_cast<uintptr_t>(scalars_dev) & 3u)
    return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: device scalars not 4-byte aligned");
  if (numel == 0) return ZERO_OK;
  const int64_t shard = numel / n_shards;
  const Range sc = range_of(scalars_dev, sizeof(zero_adam_scalars));
  for (int k = 0; k < n_shards; ++k) {
    const Range outs[5] = {range_of(master[k], shard * 4), range_of(exp_avg[k], shard * 4),
                           range_of(exp_avg_sq[k], shard * 4), range_of(bf16_out[k], shard * 2),
                           range_of(grad_out ? grad_out[k] : nullptr, grad_out ? shard * 4 : 0)};
    for (const Range& r : outs)
      if (overlaps(sc, r))
        return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: device scalars overlap an output of owner %d", k);
  }
  return ZERO_OK;
}

int check_reduce_scatter_adam_buffers(const uint16_t* const* rank_grads, const float* rank_weights,
                                      int n_ranks, int64_t numel, int n_shards, float* const* master,
                                      float* const* exp_avg, float* const* exp_avg_sq,
                                      uint16_t* const* bf16_out, const float* const* grad_acc,
                                      float* const* grad_out, Err& e) {
  if (!rank_grads || !rank_weights || !master || !exp_avg || !exp_avg_sq || !bf16_out)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: NULL pointer table or weights");
  if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: n_ranks=%d outside [1,%d]", n_ranks, ZERO_MAX_RANKS);
  if (n_shards < 1 || n_shards > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: n_shards=%d outside [1,%d]", n_shards, ZERO_MAX_RANKS);
  if (numel < 0) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: numel < 0");
  if (numel % n_shards != 0)
    return set_err(e, ZERO_ERR_SIZE, "reduce_scatter_adam: numel=%lld not divisible by n_shards=%d",
                   (long long)numel, n_shards);
  if (mul_overflows(numel, 4)) return set_err(e, ZERO_ERR_SIZE, "reduce_scatter_adam: numel too large");
  if (numel == 0) return ZERO_OK;
  const int64_t shard = numel / n_shards;
  // outputs: per owner master, m, v, bf16 and (optionally) grad_out; inputs:
  // the rank contributions and the accumulators.  acc_of_out[i] / acc_of_in[j]
  // name the owner whose grad_out / grad_acc the range is (-1 otherwise).
  Range outs[ZERO_MAX_RANKS * 5], ins[ZERO_MAX_RANKS * 2];
  int out_owner[ZERO_MAX_RANKS * 5], in_owner[ZERO_MAX_RANKS * 2];
  int no = 0, ni = 0;
  for (int r = 0; r < n_ranks; ++r) {
    if (!rank_grads[r]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: rank_grads[%d] is NULL", r);
    if (reinterpret_cast<uintptr_t>(rank_grads[r]) & 1u)
      return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: rank_grads[%d] not 2-byte aligned", r);
    in_owner[ni] = -1;
    ins[ni++] = range_of(rank_grads[r], numel * 2);
  }
  for (int k = 0; k < n_shards; ++k) {
    const void* f32s[3] = {master[k], exp_avg[k], exp_avg_sq[k]};
    for (const void* q : f32s) {
      if (!q) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: NULL state of owner %d", k);
      if (reinterpret_cast<uintptr_t>(q) & 3u)
        return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: FP32 state of owner %d misaligned", k);
      out_owner[no] = -1;
      outs[no++] = range_of(q, shard * 4);
    }
    if (!bf16_out[k]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: bf16_out[%d] is NULL", k);
    if (reinterpret_cast<uintptr_t>(bf16_out[k]) & 1u)
      return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: bf16_out[%d] misaligned", k);
    out_owner[no] = -1;
    outs[no++] = range_of(bf16_out[k], shard * 2);
    if (grad_out) {
      if (!grad_out[k]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: grad_out[%d] is NULL", k);
      if (reinterpret_cast<uintptr_t>(grad_out[k]) & 3u)
        return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: grad_out[%d] misaligned", k);
      out_owner[no] = k;
      outs[no++] = range_of(grad_out[k], shard * 4);
    }
    if (grad_acc) {
      if (!grad_acc[k]) return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: grad_acc[%d] is NULL", k);
      if (reinterpret_cast<uintptr_t>(grad_acc[k]) & 3u)
        return set_err(e, ZERO_ERR_ALIGN, "reduce_scatter_adam: grad_acc[%d] misaligned", k);
      in_owner[ni] = k;
      ins[ni++] = range_of(grad_acc[k], shard * 4);
    }
  }
  for (int i = 0; i < no; ++i) {
    for (int j = i + 1; j < no; ++j)
      if (overlaps(outs[i], outs[j]))
        return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: two output buffers overlap");
    for (int j = 0; j < ni; ++j) {
      // the one permitted alias: grad_out[k] == grad_acc[k] exactly (each
      // element is read, then written, by the same lane)
      const bool in_place = out_owner[i] >= 0 && out_owner[i] == in_owner[j] &&
                            outs[i].lo == ins[j].lo && outs[i].hi == ins[j].hi;
      if (!in_place && overlaps(outs[i], ins[j]))
        return set_err(e, ZERO_ERR_ARG, "reduce_scatter_adam: an output overlaps an input");
    }
  }
  return ZERO_OK;
}

int check_grad_norm(const float* const* shards, int n_shards, int64_t shard_numel,
                    const double* workspace, int64_t workspace_len, const double* norm_sq_out,
                    float max_norm, const float* clip_coef_out, Err& e) {
  if (!shards || !workspace || !norm_sq_out)
    return set_err(e, ZERO_ERR_ARG, "grad_norm: NULL shard table, workspace or output");
  if (n_shards < 1 || n_shards > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "grad_norm: n_shards=%d outside [1,%d]", n_shards, ZERO_MAX_RANKS);
  if (shard_numel < 0) return set_err(e, ZERO_ERR_ARG, "grad_norm: shard_numel < 0");
  if (mul_overflows(shard_numel, 4)) return set_err(e, ZERO_ERR_SIZE, "grad_norm: shard_numel too large");
  if (workspace_len < static_cast<int64_t>(n_shards) * ZERO_NORM_BLOCKS)
    return set_err(e, ZERO_ERR_SIZE, "grad_norm: workspace needs n_shards*%d doubles", ZERO_NORM_BLOCKS);
  if (clip_coef_out && !(max_norm > 0.0f))
    return set_err(e, ZERO_ERR_ARG, "grad_norm: max_norm must be > 0 when a clip coefficient is requested");
  const uintptr_t a8 = reinterpret_cast<uintptr_t>(workspace) | reinterpret_cast<uintptr_t>(norm_sq_out);
  if (a8 & 7u) return set_err(e, ZERO_ERR_ALIGN, "grad_norm: workspace or output not 8-byte aligned");
  if (clip_coef_out && (reinterpret_cast<uintptr_t>(clip_coef_out) & 3u))
    return set_err(e, ZERO_ERR_ALIGN, "grad_norm: clip_coef_out not 4-byte aligned");
  Range outs[3] = {range_of(workspace, workspace_len * 8), range_of(norm_sq_out, 8),
                   range_of(clip_coef_out, clip_coef_out ? 4 : 0)};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j])) return set_err(e, ZERO_ERR_ARG, "grad_norm: outputs overlap");
  for (int k = 0; k < n_shards; ++k) {
    if (shard_numel > 0 && !shards[k]) return set_err(e, ZERO_ERR_ARG, "grad_norm: shards[%d] is NULL", k);
    if (reinterpret_cast<uintptr_t>(shards[k]) & 3u)
      return set_err(e, ZERO_ERR_ALIGN, "grad_norm: shards[%d] not 4-byte aligned", k);
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[i], range_of(shards[k], shard_numel * 4)))
        return set_err(e, ZERO_ERR_ARG, "grad_norm: an output overlaps shards[%d]", k);
  }
  return ZERO_OK;
}

int check_adam_hparams(const zero_adam_hparams* hp, Err& e) {
  if (!hp) return set_err(e, ZERO_ERR_ARG, "adam: NULL hyper-parameters");
  if (hp->step < 1) return set_err(e, ZERO_ERR_ARG, "adam: step=%lld < 1", (long long)hp->step);
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return set_err(e, ZERO_ERR_ARG, "adam: betas must lie in [0, 1)");
  return ZERO_OK;
}

int check_adam(const float* master, const float* exp_avg, const float* exp_avg_sq,
               const uint16_t* bf16_out, const float* grad, int64_t n,
               const zero_adam_hparams* hp, Err& e) {
  int st = check_adam_hparams(hp, e);
  if (st) return st;
  return check_adam_buffers(master, exp_avg, exp_avg_sq, bf16_out, grad, n, e);
}

int check_scalars_fetch(const zero_adam_scalars* ring_host, int ring_len, const uint32_t* cursor_dev,
                        const zero_adam_scalars* scalars_dev, Err& e) {
  if (!ring_host || !cursor_dev || !scalars_dev) return set_err(e, ZERO_ERR_ARG, "scalars_fetch: NULL pointer");
  if (ring_len < 1 || ring_len > (1 << 16) || (ring_len & (ring_len - 1)) != 0)
    return set_err(e, ZERO_ERR_ARG, "scalars_fetch: ring_len=%d is not a power of two in 1..65536", ring_len);
  if ((reinterpret_cast<uintptr_t>(ring_host) | reinterpret_cast<uintptr_t>(cursor_dev) |
       reinterpret_cast<uintptr_t>(scalars_dev)) & 3u)
    return set_err(e, ZERO_ERR_ALIGN, "scalars_fetch: pointers must be 4-byte aligned");
  const Range ring = range_of(ring_host, static_cast<int64_t>(ring_len) * sizeof(zero_adam_scalars));
  const Range cur = range_of(cursor_dev, sizeof(uint32_t));
  const Range out = range_of(scalars_dev, sizeof(zero_adam_scalars));
  if (overlaps(cur, out) || overlaps(ring, out) || overlaps(ring, cur))
    return set_err(e, ZERO_ERR_ARG, "scalars_fetch: ring, cursor and scalars must not overlap");
  return ZERO_OK;
}

int check_adam_dev(const float* master, const float* exp_avg, const float* exp_avg_sq,
                   const uint16_t* bf16_out, const float* grad, int64_t n,
                   const zero_adam_scalars* scalars_dev, Err& e) {
  int st = check_adam_buffers(master, exp_avg, exp_avg_sq, bf16_out, grad, n, e);
  if (st) return st;
  if (!scalars_dev) return set_err(e, ZERO_ERR_ARG, "adam: NULL device scalars");
  if (reinterpret_cast<uintptr_t>(scalars_dev) & 3u)
    return set_err(e, ZERO_ERR_ALIGN, "adam: device scalars not 4-byte aligned");
  if (n == 0) return ZERO_OK;
  const Range sc = range_of(scalars_dev, sizeof(zero_adam_scalars));
  const Range outs[4] = {range_of(master, n * 4), range_of(exp_avg, n * 4), range_of(exp_avg_sq, n * 4),
                         range_of(bf16_out, n * 2)};
  for (const Range& r : outs)
    if (overlaps(sc, r)) return set_err(e, ZERO_ERR_ARG, "adam: device scalars overlap a buffer the update writes");
  return ZERO_OK;
}

int check_adam_buffers(const float* master, const float* exp_avg, const float* exp_avg_sq,
                       const uint16_t* bf16_out, const float* grad, int64_t n, Err& e) {
  if (n < 0) return set_err(e, ZERO_ERR_ARG, "adam: n=%lld < 0", (long long)n);
  if (n == 0) return ZERO_OK;  // touches no buffer; NULL pointers allowed
  if (!master || !exp_avg || !exp_avg_sq || !bf16_out || !grad)
    return set_err(e, ZERO_ERR_ARG, "adam: NULL buffer");
  if (mul_overflows(n, 4)) return set_err(e, ZERO_ERR_SIZE, "adam: n too large");
  const void* f32s[4] = {master, exp_avg, exp_avg_sq, grad};
  for (const void* p : f32s)
    if (reinterpret_cast<uintptr_t>(p) & 3u)
      return set_err(e, ZERO_ERR_ALIGN, "adam: FP32 buffer not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(bf16_out) & 1u)
    return set_err(e, ZERO_ERR_ALIGN, "adam: bf16_out not 2-byte aligned");
  Range rs[5] = {range_of(master, n * 4), range_of(exp_avg, n * 4), range_of(exp_avg_sq, n * 4),
                 range_of(grad, n * 4), range_of(bf16_out, n * 2)};
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(rs[i], rs[j])) return set_err(e, ZERO_ERR_ARG, "adam: buffers %d and %d overlap", i, j);
  return ZERO_OK;
}

int check_adam_scale(const float* grad_scale, const float* master, const float* exp_avg,
                     const float* exp_avg_sq, const uint16_t* bf16_out, int64_t n, Err& e) {
  if (!grad_scale) return set_err(e, ZERO_ERR_ARG, "adam: NULL grad_scale");
  if (reinterpret_cast<uintptr_t>(grad_scale) & 3u)
    return set_err(e, ZERO_ERR_ALIGN, "adam: grad_scale not 4-byte aligned");
  // every workgroup reads the scale while others write the state: it must not
  // lie inside a buffer the update writes
  const Range sc = range_of(grad_scale, 4);
  const Range outs[4] = {range_of(master, n * 4), range_of(exp_avg, n * 4), range_of(exp_avg_sq, n * 4),
                         range_of(bf16_out, n * 2)};
  for (const Range& r : outs)
    if (overlaps(sc, r)) return set_err(e, ZERO_ERR_ARG, "adam: grad_scale overlaps a buffer the update writes");
  return ZERO_OK;
}

int check_all_gather(const void* const* shards, int n_shards, int64_t shard_bytes,
                     const void* full_view, Err& e) {
  if (!shards) return set_err(e, ZERO_ERR_ARG, "all_gather: NULL shard table");
  if (n_shards < 1 || n_shards > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "all_gather: n_shards=%d outside [1,%d]", n_shards, ZERO_MAX_RANKS);
  if (shard_bytes < 0) return set_err(e, ZERO_ERR_ARG, "all_gather: shard_bytes < 0");
  if (shard_bytes == 0) return ZERO_OK;  // touches no buffer; NULL pointers allowed
  if (!full_view) return set_err(e, ZERO_ERR_ARG, "all_gather: NULL view");
  if (mul_overflows(shard_bytes, n_shards)) return set_err(e, ZERO_ERR_SIZE, "all_gather: size overflow");
  Range view = range_of(full_view, shard_bytes * n_shards);
  for (int k = 0; k < n_shards; ++k) {
    if (!shards[k]) return set_err(e, ZERO_ERR_ARG, "all_gather: shards[%d] is NULL", k);
    if (overlaps(view, range_of(shards[k], shard_bytes)))
      return set_err(e, ZERO_ERR_ARG, "all_gather: shards[%d] overlaps the view", k);
  }
  return ZERO_OK;
}

int check_offload_create(int n_ranks, int64_t shard_numel, int64_t chunk_numel,
                         const float* host_shard, uint16_t* const slot_contrib[2],
                         float* const slot_f32[2], Err& e) {
  if (!host_shard || !slot_contrib || !slot_f32 || !slot_contrib[0] || !slot_contrib[1] ||
      !slot_f32[0] || !slot_f32[1])
    return set_err(e, ZERO_ERR_ARG, "offload_create: NULL buffer");
  if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "offload_create: n_ranks=%d outside [1,%d]", n_ranks, ZERO_MAX_RANKS);
  if (shard_numel < 1 || chunk_numel < 1)
    return set_err(e, ZERO_ERR_ARG, "offload_create: sizes must be positive");
  if (mul_overflows(chunk_numel, 2 * (int64_t)n_ranks) || mul_overflows(shard_numel, 4))
    return set_err(e, ZERO_ERR_SIZE, "offload_create: size overflow");
  if ((shard_numel - 1) / chunk_numel + 1 > ZERO_OFFLOAD_MAX_CHUNKS)
    return set_err(e, ZERO_ERR_SIZE, "offload_create: more than %d chunks", ZERO_OFFLOAD_MAX_CHUNKS);
  for (int s = 0; s < 2; ++s) {
    if (reinterpret_cast<uintptr_t>(slot_contrib[s]) & 1u || reinterpret_cast<uintptr_t>(slot_f32[s]) & 3u)
      return set_err(e, ZERO_ERR_ALIGN, "offload_create: slot %d misaligned", s);
  }
  if (reinterpret_cast<uintptr_t>(host_shard) & 3u)
    return set_err(e, ZERO_ERR_ALIGN, "offload_create: host shard misaligned");
  Range rs[4] = {range_of(slot_contrib[0], chunk_numel * 2 * n_ranks),
                 range_of(slot_contrib[1], chunk_numel * 2 * n_ranks),
                 range_of(slot_f32[0], chunk_numel * 4), range_of(slot_f32[1], chunk_numel * 4)};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(rs[i], rs[j])) return set_err(e, ZERO_ERR_ARG, "offload_create: slots overlap");
  return ZERO_OK;
}

int adam_scalars(const zero_adam_hparams* hp, zero_adam_scalars* out, Err& e) {
  int st = check_adam_hparams(hp, e);
  if (st) return st;
  if (!out) return set_err(e, ZERO_ERR_ARG, "adam_scalars: NULL output");
  const float b1 = hp->beta1, b2 = hp->beta2;
  out->lr = hp->lr;
  out->beta1 = b1;
  out->beta2 = b2;
  out->one_minus_beta1 = 1.0f - b1;  // binary32 subtraction, exact for b1 in [1/2, 1]
  out->one_minus_beta2 = 1.0f - b2;
  out->bias_correction1 = static_cast<float>(1.0 - std::pow(static_cast<double>(b1), static_cast<double>(hp->step)));
  out->bias_correction2 = static_cast<float>(1.0 - std::pow(static_cast<double>(b2), static_cast<double>(hp->step)));
  out->eps = hp->eps;
  out->weight_decay = hp->weight_decay;
  return ZERO_OK;
}

int rank_weights(const int64_t* counts, int n_ranks, float* out, Err& e) {
  if (!out) return set_err(e, ZERO_ERR_ARG, "rank_weights: NULL output");
  if (n_ranks < 1 || n_ranks > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "rank_weights: n_ranks=%d outside [1,%d]", n_ranks, ZERO_MAX_RANKS);
  if (!counts) {
    for (int r = 0; r < n_ranks; ++r) out[r] = static_cast<float>(1.0 / static_cast<double>(n_ranks));
    return ZERO_OK;
  }
  int64_t total = 0;
  for (int r = 0; r < n_ranks; ++r) {
    if (counts[r] < 0) return set_err(e, ZERO_ERR_ARG, "rank_weights: counts[%d] < 0", r);
    if (counts[r] > INT64_MAX - total) return set_err(e, ZERO_ERR_SIZE, "rank_weights: sum overflows");
    total += counts[r];
  }
  if (total == 0) return set_err(e, ZERO_ERR_ARG, "rank_weights: counts sum to 0");
  for (int r = 0; r < n_ranks; ++r)
    out[r] = static_cast<float>(static_cast<double>(counts[r]) / static_cast<double>(total));
  return ZERO_OK;
}

int shard_layout(const int64_t* numels, int n_tensors, int n_shards, int64_t* psi,
                 int64_t* psi_pad, int64_t* shard_numel, Err& e) {
  if (!psi || !psi_pad || !shard_numel || (n_tensors > 0 && !numels) || n_tensors < 0)
    return set_err(e, ZERO_ERR_ARG, "shard_layout: NULL pointer or negative n_tensors");
  if (n_shards < 1 || n_shards > ZERO_MAX_RANKS)
    return set_err(e, ZERO_ERR_ARG, "shard_layout: n_shards=%d outside [1,%d]", n_shards, ZERO_MAX_RANKS);
  int64_t total = 0;
  for (int i = 0; i < n_tensors; ++i) {
    if (numels[i] < 0) return set_err(e, ZERO_ERR_ARG, "shard_layout: numels[%d] < 0", i);
    if (numels[i] > INT64_MAX / 8 - total) return set_err(e, ZERO_ERR_SIZE, "shard_layout: overflow");
    total += numels[i];
  }
  const int64_t q = static_cast<int64_t>(n_shards) * 256;
  const int64_t pad = ((total + q - 1) / q) * q;
  *psi = total;
  *psi_pad = pad;
  *shard_numel = pad / n_shards;
  return ZERO_OK;
}

}  // namespace zero
