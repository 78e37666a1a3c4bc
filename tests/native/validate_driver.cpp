// Host-only driver for the C ABI's argument checks, built with g++ and the
// address/undefined-behaviour sanitizers (no HIP, no device).  Exercises every
// check with valid, boundary and invalid arguments; prints "ok" on success.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../zero_sharded_optimizer_reduce_amd/csrc/validate.h"

using namespace zero;

static int fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);       \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  Err e;
  // reduce-scatter
  const void* g4[4] = {P(0x10000), P(0x20000), P(0x30000), P(0x40000)};
  float* o4[4] = {(float*)P(0x100000), (float*)P(0x110000), (float*)P(0x120000), (float*)P(0x130000)};
  float w4[4] = {0.25f, 0.25f, 0.25f, 0.25f};
  EXPECT(check_reduce_scatter(g4, w4, 4, 1024, o4, 4, 0, e) == ZERO_OK);
  EXPECT(check_reduce_scatter(g4, w4, 4, 1024, o4, 4, 1, e, 4) == ZERO_OK);
  EXPECT(check_reduce_scatter(g4, w4, 0, 1024, o4, 4, 0, e) == ZERO_ERR_ARG);
  EXPECT(check_reduce_scatter(g4, w4, 4, 1023, o4, 4, 0, e) == ZERO_ERR_SIZE);
  EXPECT(check_reduce_scatter(g4, w4, 4, INT64_MAX - 3, o4, 4, 0, e) != ZERO_OK);
  EXPECT(check_reduce_scatter(nullptr, w4, 4, 1024, o4, 4, 0, e) == ZERO_ERR_ARG);
  const void* gbad[4] = {P(0x10001), P(0x20000), P(0x30000), P(0x40000)};
  EXPECT(check_reduce_scatter(gbad, w4, 4, 1024, o4, 4, 0, e) == ZERO_ERR_ALIGN);
  float* oover[4] = {(float*)P(0x10100), (float*)P(0x110000), (float*)P(0x120000), (float*)P(0x130000)};
  EXPECT(check_reduce_scatter(g4, w4, 4, 1024, oover, 4, 0, e) == ZERO_ERR_ARG);
  EXPECT(std::strstr(e.msg, "overlap") != nullptr);
  // Adam
  zero_adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1};
  float* p = (float*)P(0x100000);
  float* m = (float*)P(0x200000);
  float* v = (float*)P(0x300000);
  uint16_t* b = (uint16_t*)P(0x400000);
  float* gr = (float*)P(0x500000);
  EXPECT(check_adam(p, m, v, b, gr, 4096, &hp, e) == ZERO_OK);
  EXPECT(check_adam(p, p + 16, v, b, gr, 4096, &hp, e) == ZERO_ERR_ARG);
  EXPECT(check_adam(nullptr, nullptr, nullptr, nullptr, nullptr, 0, &hp, e) == ZERO_OK);
  zero_adam_hparams bad = hp;
  bad.step = 0;
  EXPECT(check_adam(p, m, v, b, gr, 16, &bad, e) == ZERO_ERR_ARG);
  bad = hp;
  bad.beta2 = 1.0f;
  EXPECT(check_adam(p, m, v, b, gr, 16, &bad, e) == ZERO_ERR_ARG);
  // the device scale of the clipped update
  const float* gs = (const float*)P(0x600000);
  EXPECT(check_adam_scale(gs, p, m, v, b, 4096, e) == ZERO_OK);
  EXPECT(check_adam_scale(nullptr, p, m, v, b, 4096, e) == ZERO_ERR_ARG);
  EXPECT(check_adam_scale((const float*)P(0x600002), p, m, v, b, 4096, e) == ZERO_ERR_ALIGN);
  EXPECT(check_adam_scale(p + 4095, p, m, v, b, 4096, e) == ZERO_ERR_ARG);       // last master element
  EXPECT(check_adam_scale((const float*)(b + 2046), p, m, v, b, 4096, e) == ZERO_ERR_ARG);  // inside bf16_out
  EXPECT(check_adam_scale(p + 4096, p, m, v, b, 4096, e) == ZERO_OK);            // just past master
  EXPECT(check_adam_scale(gr, p, m, v, b, 4096, e) == ZERO_OK);                  // inside the read-only gradient
  // device scalars of the graph-capturable update
  const zero_adam_scalars* sd = (const zero_adam_scalars*)P(0x700000);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, sd, e) == ZERO_OK);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, nullptr, e) == ZERO_ERR_ARG);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, (const zero_adam_scalars*)P(0x700002), e) == ZERO_ERR_ALIGN);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, (const zero_adam_scalars*)(v + 100), e) == ZERO_ERR_ARG);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, (const zero_adam_scalars*)(p + 4096 - 4), e) == ZERO_ERR_ARG);
  EXPECT(check_adam_dev(p, m, v, b, gr, 4096, (const zero_adam_scalars*)(gr + 8), e) == ZERO_OK);
  EXPECT(check_adam_dev(p, p + 16, v, b, gr, 4096, sd, e) == ZERO_ERR_ARG);   // buffers still checked
  // the scalar ring of captured steps (memory types are checked by the entry point itself)
  {
    const zero_adam_scalars* ring = (const zero_adam_scalars*)P(0x900000);
    uint32_t* cur = (uint32_t*)P(0xa00000);
    zero_adam_scalars* out = (zero_adam_scalars*)P(0xb00000);
    EXPECT(check_scalars_fetch(ring, 1, cur, out, e) == ZERO_OK);
    EXPECT(check_scalars_fetch(ring, 8, cur, out, e) == ZERO_OK);
    EXPECT(check_scalars_fetch((const zero_adam_scalars*)P(0x10000000), 1 << 16, cur, out, e) == ZERO_OK);
    EXPECT(check_scalars_fetch(ring, 1 << 16, cur, out, e) == ZERO_ERR_ARG);   // 2.4 MB reach cursor and scalars
    EXPECT(check_scalars_fetch(ring, 0, cur, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, 6, cur, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, 1 << 17, cur, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, -4, cur, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(nullptr, 8, cur, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, 8, nullptr, out, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, 8, cur, nullptr, e) == ZERO_ERR_ARG);
    EXPECT(check_scalars_fetch(ring, 8, (uint32_t*)P(0xa00002), out, e) == ZERO_ERR_ALIGN);
    EXPECT(check_scalars_fetch(ring, 8, (uint32_t*)P(0xb00020), out, e) == ZERO_ERR_ARG);   // cursor in scalars
    EXPECT(check_scalars_fetch(ring, 8, (uint32_t*)P(0xb00024), out, e) == ZERO_OK);        // just past them
    EXPECT(check_scalars_fetch(ring, 8, (uint32_t*)P(0x900000 + 7 * 36), out, e) == ZERO_ERR_ARG);  // in the ring
  }
  {
    const uint16_t* gg[2] = {(const uint16_t*)P(0x10000), (const uint16_t*)P(0x20000)};
    float wts[2] = {0.5f, 0.5f};
    float* mp[2] = {(float*)P(0x100000), (float*)P(0x110000)};
    float* mm[2] = {(float*)P(0x200000), (float*)P(0x210000)};
    float* mv[2] = {(float*)P(0x300000), (float*)P(0x310000)};
    uint16_t* mb[2] = {(uint16_t*)P(0x400000), (uint16_t*)P(0x410000)};
    float* go[2] = {(float*)P(0x500000), (float*)P(0x510000)};
    EXPECT(check_reduce_scatter_adam_dev(gg, wts, 2, 2048, 2, mp, mm, mv, mb, nullptr, go, sd, e) == ZERO_OK);
    EXPECT(check_reduce_scatter_adam_dev(gg, wts, 2, 2048, 2, mp, mm, mv, mb, nullptr, go, nullptr, e) ==
           ZERO_ERR_ARG);
    EXPECT(check_reduce_scatter_adam_dev(gg, wts, 2, 2048, 2, mp, mm, mv, mb, nullptr, go,
                                         (const zero_adam_scalars*)(go[1] + 10), e) == ZERO_ERR_ARG);
    EXPECT(check_reduce_scatter_adam_dev(gg, wts, 2, 2048, 2, mp, mm, mv, mb, nullptr, go,
                                         (const zero_adam_scalars*)(mb[0] + 2), e) == ZERO_ERR_ARG);
  }
  // scalars
  zero_adam_scalars sc;
  EXPECT(adam_scalars(&hp, &sc, e) == ZERO_OK);
  EXPECT(sc.bias_correction1 == sc.one_minus_beta1);
  hp.step = 1000000000000LL;  // bias corrections saturate to 1
  EXPECT(adam_scalars(&hp, &sc, e) == ZERO_OK && sc.bias_correction1 == 1.0f);
  // weights and layout
  int64_t counts[4] = {4096, 3072, 4096, 2048};
  float w[4];
  EXPECT(rank_weights(counts, 4, w, e) == ZERO_OK);
  { float w16[16]; EXPECT(rank_weights(nullptr, 16, w16, e) == ZERO_OK && w16[15] == 0.0625f); }
  int64_t zeros[2] = {0, 0};
  EXPECT(rank_weights(zeros, 2, w, e) == ZERO_ERR_ARG);
  int64_t huge[2] = {INT64_MAX, 5};
  EXPECT(rank_weights(huge, 2, w, e) == ZERO_ERR_SIZE);
  int64_t numels[3] = {5, 7, 0};
  int64_t psi, pad, s;
  EXPECT(shard_layout(numels, 3, 4, &psi, &pad, &s, e) == ZERO_OK && psi == 12 && pad == 1024 && s == 256);
  int64_t big[2] = {INT64_MAX / 8, INT64_MAX / 8};
  EXPECT(shard_layout(big, 2, 4, &psi, &pad, &s, e) == ZERO_ERR_SIZE);
  // all-gather
  const void* sh[2] = {P(0x10000), P(0x20000)};
  EXPECT(check_all_gather(sh, 2, 4096, P(0x100000), e) == ZERO_OK);
  EXPECT(check_all_gather(sh, 2, 4096, P(0x10800), e) == ZERO_ERR_ARG);
  // fused
  const uint16_t* fg[1] = {(const uint16_t*)P(0x10000000)};
  float* fp[1] = {p};
  float* fm[1] = {m};
  float* fv[1] = {v};
  uint16_t* fb[1] = {b};
  const float* facc[1] = {gr};
  float* fout[1] = {gr};
  hp.step = 3;
  EXPECT(check_reduce_scatter_adam(fg, w4, 1, 1024, 1, fp, fm, fv, fb, facc, fout, &hp, e) == ZERO_OK);
  float* fout2[1] = {gr + 4};
  EXPECT(check_reduce_scatter_adam(fg, w4, 1, 1024, 1, fp, fm, fv, fb, facc, fout2, &hp, e) == ZERO_ERR_ARG);
  // gradient norm
  const float* ns[2] = {(const float*)P(0x100000), (const float*)P(0x200000)};
  double* ws = (double*)P(0x1000000);
  double* out = (double*)P(0x2000000);
  EXPECT(check_grad_norm(ns, 2, 4096, ws, 2048, out, 1.0f, nullptr, e) == ZERO_OK);
  EXPECT(check_grad_norm(ns, 2, 4096, ws, 2047, out, 1.0f, nullptr, e) == ZERO_ERR_SIZE);
  EXPECT(check_grad_norm(ns, 2, 4096, ws, 2048, out, 0.0f, (float*)P(0x3000000), e) == ZERO_ERR_ARG);
  // offload
  uint16_t* slots[2] = {(uint16_t*)P(0x100000), (uint16_t*)P(0x900000)};
  float* stage[2] = {(float*)P(0x2000000), (float*)P(0x3000000)};
  EXPECT(check_offload_create(4, 1 << 20, 1 << 18, (const float*)P(0x5000), slots, stage, e) == ZERO_OK);
  uint16_t* slots_over[2] = {(uint16_t*)P(0x100000), (uint16_t*)P(0x800000)};
  EXPECT(check_offload_create(4, 1 << 20, 1 << 20, (const float*)P(0x5000), slots_over, stage, e) == ZERO_ERR_ARG);
  // at most ZERO_OFFLOAD_MAX_CHUNKS chunks (the handle holds two events per chunk)
  uint16_t* small_slots[2] = {(uint16_t*)P(0x100000), (uint16_t*)P(0x200000)};
  float* small_stage[2] = {(float*)P(0x300000), (float*)P(0x400000)};
  EXPECT(check_offload_create(4, 65536LL * 16, 16, (const float*)P(0x5000), small_slots, small_stage, e) == ZERO_OK);
  EXPECT(check_offload_create(4, 65536LL * 16 + 1, 16, (const float*)P(0x5000), small_slots, small_stage, e) ==
         ZERO_ERR_SIZE);
  EXPECT(check_offload_create(4, 2000000000LL, 1, (const float*)P(0x5000), small_slots, small_stage, e) ==
         ZERO_ERR_SIZE);
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
