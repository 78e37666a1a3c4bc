// gfx950 kernels of the sharded update: reduce-scatter, fused Adam owner
// update, all-gather copy.  All three are HBM-streaming kernels (no data
// reuse, a few FLOPs per byte), so they use no MFMA and compute nothing in
// LDS: each lane moves 16-byte (or 8-byte BF16) vectors with non-temporal
// loads and stores, and the grid covers the whole array, one tile per
// workgroup, so that the workgroups in flight sweep a narrow window of every
// array in dispatch order (the loops are grid-stride only beyond the grid
// cap).  Workgroup sizes and residency caps are per kernel (see the launch
// constants below).
//
// Floating point: the file is compiled with FP contraction off (also forced
// below), so every multiply and add is its own binary32 rounding; '/' and
// sqrtf are the correctly rounded forms (hipcc's default).  The arithmetic is
// therefore the same, operation for operation, as the definitions cited at
// each kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kernels.h"

#pragma clang fp contract(off)

namespace zero {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

// ------------------------------------------------------------------ helpers
// A BF16 value is the high half of a binary32, so widening is a shift (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Round-to-nearest-even binary32 -> bfloat16 (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t to_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(to_bf16(lo)) | (static_cast<uint32_t>(to_bf16(hi)) << 16);
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T v, T* p) { __builtin_nontemporal_store(v, p); }

// Streamed output stores with a cache policy the compiler's builtin cannot
// set.  With SC1 a workgroup writes its tile through a buffer descriptor based
// at the tile's first element (workgroup-uniform, so the descriptor lives in
// scalar registers and every lane offset is below 4 KiB), with the store bits
// nt and sc1 (device scope); without it the plain non-temporal store is used.
// Same-box A/B on MI355X: with sc1 the update, the fused kernel (without the
// gradient output), the accumulate-mode reduce and the gather ran 1.0-3.6%
// faster; the plain reduce, the FP32-contribution reduce and the fused kernel
// storing the gradient ran 0.4-1.8% slower, so they keep the plain store
// (system scope, sc0|sc1, measured the same as sc1).
// The buffer forms are compiler intrinsics (not inline assembly), so the
// compiler schedules them and resolves their register hazards.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
constexpr int kRawBufferFlags = 0x00020000;   // dword 3 of a raw buffer descriptor: 32-bit data format
constexpr int kStoreNtSc1 = 2 | 16;           // cache-policy operand: nt | sc1

template <typename T, bool SC1>
struct TileOut {
  T* global;                  // the tile's first element
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ TileOut(T* base, int64_t count) : global(base) {
    if constexpr (SC1)
      rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(count * static_cast<int64_t>(sizeof(T))),
                                               kRawBufferFlags);
  }
  // element j of the tile (0 <= j < count)
  __device__ __forceinline__ void store(T v, int j) const {
    if constexpr (!SC1) {
      __builtin_nontemporal_store(v, global + j);
    } else if constexpr (sizeof(T) == 16) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), rsrc, j * 16, 0, kStoreNtSc1);
    } else if constexpr (sizeof(T) == 8) {
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), rsrc, j * 8, 0, kStoreNtSc1);
    } else {
      __builtin_nontemporal_store(v, global + j);
    }
  }
};

// Elements of the tile that starts `left` elements before the end of an array.
__device__ __forceinline__ int64_t tile_len(int64_t left, int bs) { return left < bs ? left : bs; }

// ------------------------------------------------------------ reduce-scatter
// Owner k, element i (global index j = k*shard + i):
//   red = w_0*x_0[j]; red = red + w_r*x_r[j] for r = 1..N-1 (rank order),
// optionally out = out + red.  Contributions of one parameter are combined
// element-wise and never mixed with other parameters; the owner receives only
// its slice (slide "分担数据，与分担保存责任，是两个动作", note 原 N48).
//
// Vector path: each lane reduces 4 consecutive elements: one 8-byte BF16 load
// per rank, one 16-byte FP32 store, so every load and store instruction of a
// wave covers one contiguous span (16-byte loads with two strided 16-byte
// stores measured 5% slower: the stores then cover half lines).  A workgroup
// takes one tile of BS vectors per loop iteration; lanes past the end of the
// shard skip the whole body, so a lane's N contribution loads sit in one
// basic block and are all in flight before the first wait (a guard per load
// made the compiler wait for each load before issuing the next: 10-16%
// slower).

// The 4 reduced values of one lane; x[r] holds rank r's 4 BF16 values.
template <int NMAX>
__device__ __forceinline__ f32x4 reduce4(const u32x2 (&x)[NMAX], int n, const float* w) {
  const float w0 = w[0];
  float a0 = w0 * bf16_lo(x[0].x), a1 = w0 * bf16_hi(x[0].x);
  float a2 = w0 * bf16_lo(x[0].y), a3 = w0 * bf16_hi(x[0].y);
#pragma unroll
  for (int r = 1; r < NMAX; ++r) {
    if (r < n) {
      const float wr = w[r];
      a0 = a0 + wr * bf16_lo(x[r].x);
      a1 = a1 + wr * bf16_hi(x[r].x);
      a2 = a2 + wr * bf16_lo(x[r].y);
      a3 = a3 + wr * bf16_hi(x[r].y);
    }
  }
  return f32x4{a0, a1, a2, a3};
}

template <int NMAX>
__device__ __forceinline__ f32x4 reduce4(const f32x4 (&x)[NMAX], int n, const float* w) {
  f32x4 a = w[0] * x[0];
#pragma unroll
  for (int r = 1; r < NMAX; ++r)
    if (r < n) a = a + w[r] * x[r];
  return a;
}

// FP32 contributions (gradients stored in FP32): 16-byte load per rank.
template <int N, bool ACC, int BS>
__global__ __launch_bounds__(BS) void rs_f32_vec_kernel(RsParams p) {
  constexpr int NMAX = N > 0 ? N : ZERO_MAX_RANKS;
  const int n = N > 0 ? N : p.n_ranks;
  const int k = blockIdx.y;
  const int64_t nvec = p.shard >> 2;
  const int64_t off = static_cast<int64_t>(k) * nvec;
  f32x4* __restrict__ out = reinterpret_cast<f32x4*>(p.out[k]);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * BS + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * BS) {
    f32x4 x[NMAX];
#pragma unroll
    for (int r = 0; r < NMAX; ++r)
      if (r < n) x[r] = ld_nt(reinterpret_cast<const f32x4*>(p.g[r]) + off + i);
    f32x4 a = reduce4<NMAX>(x, n, p.w);
    if (ACC) a = out[i] + a;
    st_nt(a, out + i);
  }
}

template <bool ACC>
__global__ __launch_bounds__(kBlock) void rs_f32_scalar_kernel(RsParams p) {
  const int k = blockIdx.y;
  const int64_t base = static_cast<int64_t>(k) * p.shard;
  float* __restrict__ out = p.out[k];
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < p.shard;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    const float* const* g = reinterpret_cast<const float* const*>(p.g);
    float a = p.w[0] * g[0][base + i];
    for (int r = 1; r < p.n_ranks; ++r) a = a + p.w[r] * g[r][base + i];
    out[i] = ACC ? out[i] + a : a;
  }
}

template <int N, bool ACC, int BS>
__global__ __launch_bounds__(BS) void rs_vec_kernel(RsParams p) {
  constexpr int NMAX = N > 0 ? N : ZERO_MAX_RANKS;
  const int n = N > 0 ? N : p.n_ranks;
  const int k = blockIdx.y;
  const int64_t nvec = p.shard >> 2;
  const int64_t off = static_cast<int64_t>(k) * nvec;
  f32x4* __restrict__ out = reinterpret_cast<f32x4*>(p.out[k]);
  const int64_t step = static_cast<int64_t>(gridDim.x) * BS;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * BS; tile < nvec; tile += step) {
    const int64_t i = tile + threadIdx.x;
    if (i < nvec) {
      const TileOut<f32x4, ACC> o(out + tile, tile_len(nvec - tile, BS));
      u32x2 x[NMAX];
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        if (r < n) x[r] = ld_nt(reinterpret_cast<const u32x2*>(p.g[r]) + off + i);
      f32x4 prev;
      if (ACC) prev = out[i];
      // Keep the scheduler from starting the conversion of rank 0's values
      // (and waiting for them) before the last load is issued.
      __builtin_amdgcn_sched_barrier(0);
      f32x4 a = reduce4<NMAX>(x, n, p.w);
      if (ACC) a = prev + a;
      o.store(a, threadIdx.x);
    }
  }
}

// Element-at-a-time path for shards whose length or pointers do not allow
// 16-byte vectors.  Same arithmetic, same order.
template <bool ACC>
__global__ __launch_bounds__(kBlock) void rs_scalar_kernel(RsParams p) {
  const int k = blockIdx.y;
  const int64_t base = static_cast<int64_t>(k) * p.shard;
  float* __restrict__ out = p.out[k];
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < p.shard;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    float a = p.w[0] * bf16_at(p.g[0], base + i);
    for (int r = 1; r < p.n_ranks; ++r) a = a + p.w[r] * bf16_at(p.g[r], base + i);
    out[i] = ACC ? out[i] + a : a;
  }
}

// ---------------------------------------------------------------- Adam update
// The owner's update of its master weight p, first moment m and second moment
// v with the reduced gradient g (slide, note 原 N48; essay "把训练账本放进多张
// 设备", section 从持久状态开始记账): bias-corrected Adam with decoupled decay.
// WD: 0 no decay term, 1 decay term, 2 the scalars come from device memory and
// the term is applied when their weight_decay is non-zero (a uniform branch),
// exactly as the host decides it for 0 and 1.
template <int WD>
__device__ __forceinline__ zero_adam_scalars step_scalars(const zero_adam_scalars& by_value,
                                                          const zero_adam_scalars* dev) {
  if (WD == 2) return *dev;
  return by_value;
}

template <int WD>
__device__ __forceinline__ void adam_elem(float& p, float& m, float& v, float g,
                                          const zero_adam_scalars& s) {
  const float m1 = s.beta1 * m + s.one_minus_beta1 * g;
  const float gg = g * g;
  const float v1 = s.beta2 * v + s.one_minus_beta2 * gg;
  const float m_hat = m1 / s.bias_correction1;
  const float v_hat = v1 / s.bias_correction2;
  const float denom = sqrtf(v_hat) + s.eps;
  float u = m_hat / denom;
  if (WD == 1 || (WD == 2 && s.weight_decay != 0.0f)) u = u + s.weight_decay * p;
  p = p - s.lr * u;
  m = m1;
  v = v1;
}

// One pass: read g, p, m, v (16 B/param), write p, m, v and the BF16 working
// weight (14 B/param).  Vector path: 4 elements per 16-byte access, one
// tile of BS vectors per workgroup and loop iteration, lanes past the end
// skipping the whole body; the n % 4 tail goes element-wise.  SC: the gradient
// is first multiplied by the device scalar *gscale (the clip coefficient).
template <int WD, bool SC, int BS>
__global__ __launch_bounds__(BS) void adam_vec_kernel(AdamParams a) {
  const zero_adam_scalars s = step_scalars<WD>(a.s, a.sdev);
  const int64_t nvec = a.n >> 2;
  f32x4* __restrict__ P = reinterpret_cast<f32x4*>(a.p);
  f32x4* __restrict__ M = reinterpret_cast<f32x4*>(a.m);
  f32x4* __restrict__ V = reinterpret_cast<f32x4*>(a.v);
  const f32x4* __restrict__ G = reinterpret_cast<const f32x4*>(a.g);
  u32x2* __restrict__ B = reinterpret_cast<u32x2*>(a.b);
  const float c = SC ? *a.gscale : 1.0f;
  const int64_t step = static_cast<int64_t>(gridDim.x) * BS;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * BS; tile < nvec; tile += step) {
    const int64_t i = tile + threadIdx.x;
    if (i < nvec) {
      const int64_t len = tile_len(nvec - tile, BS);
      const TileOut<f32x4, true> oP(P + tile, len), oM(M + tile, len), oV(V + tile, len);
      const TileOut<u32x2, true> oB(B + tile, len);
      f32x4 g = ld_nt(G + i);
      const f32x4 pv = ld_nt(P + i), mv = ld_nt(M + i), vv = ld_nt(V + i);
      if (SC) g = g * c;
      float pe[4] = {pv.x, pv.y, pv.z, pv.w};
      float me[4] = {mv.x, mv.y, mv.z, mv.w};
      float ve[4] = {vv.x, vv.y, vv.z, vv.w};
      const float ge[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) adam_elem<WD>(pe[e], me[e], ve[e], ge[e], s);
      oP.store(f32x4{pe[0], pe[1], pe[2], pe[3]}, threadIdx.x);
      oM.store(f32x4{me[0], me[1], me[2], me[3]}, threadIdx.x);
      oV.store(f32x4{ve[0], ve[1], ve[2], ve[3]}, threadIdx.x);
      oB.store(u32x2{to_bf16x2(pe[0], pe[1]), to_bf16x2(pe[2], pe[3])}, threadIdx.x);
    }
  }
  const int64_t tail = a.n - (nvec << 2);
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const int64_t i = (nvec << 2) + threadIdx.x;
    float pe = a.p[i], me = a.m[i], ve = a.v[i];
    adam_elem<WD>(pe, me, ve, SC ? a.g[i] * c : a.g[i], s);
    a.p[i] = pe;
    a.m[i] = me;
    a.v[i] = ve;
    a.b[i] = to_bf16(pe);
  }
}

template <int WD, bool SC>
__global__ __launch_bounds__(kBlock) void adam_scalar_kernel(AdamParams a) {
  const zero_adam_scalars s = step_scalars<WD>(a.s, a.sdev);
  const float c = SC ? *a.gscale : 1.0f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < a.n;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    float pe = a.p[i], me = a.m[i], ve = a.v[i];
    adam_elem<WD>(pe, me, ve, SC ? a.g[i] * c : a.g[i], s);
    a.p[i] = pe;
    a.m[i] = me;
    a.v[i] = ve;
    a.b[i] = to_bf16(pe);
  }
}

// ------------------------------------------------------ global gradient norm
// Sum of squares of the reduced gradient shards in FP64 (each square of a
// binary32 value is exact in binary64, so only the additions round), with a
// summation order fixed by the element count alone: lane-sequential partial
// sums over a grid-stride pattern of a fixed number of blocks, a butterfly
// across the 64 lanes of a wave, the 4 waves of a block in order, then one
// block folding the per-block partial sums in index order.  Repeated calls
// give the same bits on any device.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ double block_sum(double x) {
  __shared__ double part[kBlock / 64];
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[w] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i) t += part[i];
  }
  return t;  // valid in thread 0
}

template <bool VEC>
__global__ __launch_bounds__(kBlock) void norm_partial_kernel(NormParams p) {
  const int k = blockIdx.y;
  const float* __restrict__ x = p.x[k];
  double acc = 0.0;
  if (VEC) {
    const int64_t nvec = p.n >> 2;
    const f32x4* __restrict__ X = reinterpret_cast<const f32x4*>(x);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nvec;
         i += static_cast<int64_t>(gridDim.x) * kBlock) {
      const f32x4 v = ld_nt(X + i);
      acc += static_cast<double>(v.x) * static_cast<double>(v.x);
      acc += static_cast<double>(v.y) * static_cast<double>(v.y);
      acc += static_cast<double>(v.z) * static_cast<double>(v.z);
      acc += static_cast<double>(v.w) * static_cast<double>(v.w);
    }
    const int64_t tail = p.n - (nvec << 2);
    if (blockIdx.x == 0 && threadIdx.x < tail) {
      const double e = x[(nvec << 2) + threadIdx.x];
      acc += e * e;
    }
  } else {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < p.n;
         i += static_cast<int64_t>(gridDim.x) * kBlock) {
      const double e = x[i];
      acc += e * e;
    }
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) p.partials[static_cast<int64_t>(k) * gridDim.x + blockIdx.x] = t;
}

// Partial sums of zero_grad_norm_sq_no_alloc: one array per GPU, held until the
// process ends.  Host code never uses this name as an address: it is a
// host-side stand-in for the symbol, and the device address comes from
// norm_scratch_device_ptr.
static __device__ __align__(256) double scratch[kNormScratchDoubles];

__global__ __launch_bounds__(kBlock) void norm_final_kernel(NormParams p) {
  const int64_t total = static_cast<int64_t>(p.n_shards) * p.gx;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < total; i += kBlock) acc += p.partials[i];
  const double t = block_sum(acc);
  if (threadIdx.x == 0) {
    p.out[0] = t;
    if (p.coef) {
      const double c = static_cast<double>(p.max_norm) / (sqrt(t) + 1e-6);
      p.coef[0] = static_cast<float>(c < 1.0 ? c : 1.0);
    }
  }
}

// ------------------------------------------------ fused reduce-scatter + Adam
// The reduce-scatter and the owner update in one pass (blog "数据并行与 ZeRO：
// 三级分片各省多少", section 三级分片: ZeRO-1 places the optimizer step between
// the reduce-scatter and the all-gather).  The reduced gradient is formed in
// registers with exactly the reduce-scatter kernel's arithmetic and handed to
// the same update, so the results are bit-identical to the two kernels run
// one after the other; it is written out only when gout is given.  ACC: the
// gradient is gacc + red (the reduce kernel's accumulate mode: the last
// micro-batch of an accumulation updates directly).  Bytes per parameter
// (N=4): 8 (contributions) + 12 (state) read, 12 (state) + 2 (BF16) written
// = 34, against 12 + 30 = 42 for the two kernels.
template <int N, int WD, bool WG, bool ACC, int BS>
__global__ __launch_bounds__(BS) void fused_vec_kernel(FusedParams p) {
  const zero_adam_scalars s = step_scalars<WD>(p.s, p.sdev);
  constexpr int NMAX = N > 0 ? N : ZERO_MAX_RANKS;
  const int n = N > 0 ? N : p.n_ranks;
  const int k = blockIdx.y;
  const int64_t nvec = p.shard >> 2;
  const int64_t off = static_cast<int64_t>(k) * nvec;
  f32x4* __restrict__ P = reinterpret_cast<f32x4*>(p.p[k]);
  f32x4* __restrict__ M = reinterpret_cast<f32x4*>(p.m[k]);
  f32x4* __restrict__ V = reinterpret_cast<f32x4*>(p.v[k]);
  u32x2* __restrict__ B = reinterpret_cast<u32x2*>(p.b[k]);
  f32x4* __restrict__ GO = reinterpret_cast<f32x4*>(p.gout[k]);
  const f32x4* __restrict__ GA = reinterpret_cast<const f32x4*>(p.gacc[k]);
  const int64_t step = static_cast<int64_t>(gridDim.x) * BS;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * BS; tile < nvec; tile += step) {
    const int64_t i = tile + threadIdx.x;
    if (i < nvec) {
      const int64_t len = tile_len(nvec - tile, BS);
      const TileOut<f32x4, !WG> oP(P + tile, len), oM(M + tile, len), oV(V + tile, len);
      const TileOut<u32x2, !WG> oB(B + tile, len);
      u32x2 x[NMAX];
#pragma unroll
      for (int r = 0; r < NMAX; ++r)
        if (r < n) x[r] = ld_nt(reinterpret_cast<const u32x2*>(p.g[r]) + off + i);
      const f32x4 pv = ld_nt(P + i), mv = ld_nt(M + i), vv = ld_nt(V + i);
      f32x4 g = reduce4<NMAX>(x, n, p.w);
      if (ACC) g = ld_nt(GA + i) + g;
      if (WG) st_nt(g, GO + i);
      float pe[4] = {pv.x, pv.y, pv.z, pv.w};
      float me[4] = {mv.x, mv.y, mv.z, mv.w};
      float ve[4] = {vv.x, vv.y, vv.z, vv.w};
      const float ge[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) adam_elem<WD>(pe[e], me[e], ve[e], ge[e], s);
      oP.store(f32x4{pe[0], pe[1], pe[2], pe[3]}, threadIdx.x);
      oM.store(f32x4{me[0], me[1], me[2], me[3]}, threadIdx.x);
      oV.store(f32x4{ve[0], ve[1], ve[2], ve[3]}, threadIdx.x);
      oB.store(u32x2{to_bf16x2(pe[0], pe[1]), to_bf16x2(pe[2], pe[3])}, threadIdx.x);
    }
  }
}

template <int WD>
__global__ __launch_bounds__(kBlock) void fused_scalar_kernel(FusedParams p) {
  const zero_adam_scalars s = step_scalars<WD>(p.s, p.sdev);
  const int k = blockIdx.y;
  const int64_t base = static_cast<int64_t>(k) * p.shard;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < p.shard;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    float g = p.w[0] * bf16_at(p.g[0], base + i);
    for (int r = 1; r < p.n_ranks; ++r) g = g + p.w[r] * bf16_at(p.g[r], base + i);
    if (p.gacc[k]) g = p.gacc[k][i] + g;
    if (p.gout[k]) p.gout[k][i] = g;
    float pe = p.p[k][i], me = p.m[k][i], ve = p.v[k][i];
    adam_elem<WD>(pe, me, ve, g, s);
    p.p[k][i] = pe;
    p.m[k][i] = me;
    p.v[k][i] = ve;
    p.b[k][i] = to_bf16(pe);
  }
}

// ---------------------------------------------------------------- all-gather
// The full view is the owners' shards concatenated in owner order (essay,
// section ZeRO-3 的一次完整计算; slide, note 原 N47).  Owner k = blockIdx.y.
template <typename T, int BS>
__global__ __launch_bounds__(BS) void gather_kernel(GatherParams p) {
  const int k = blockIdx.y;
  const int64_t n = p.shard_bytes / static_cast<int64_t>(sizeof(T));
  const T* __restrict__ src = reinterpret_cast<const T*>(p.src[k]);
  T* __restrict__ dst = reinterpret_cast<T*>(static_cast<char*>(p.dst) + k * p.shard_bytes);
  const int64_t step = static_cast<int64_t>(gridDim.x) * BS;
  constexpr bool kSc1 = sizeof(T) == 16;   // the 16-byte path stores with nt | sc1
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * BS; tile < n; tile += step) {
    const int64_t i = tile + threadIdx.x;
    if (i < n) {
      const TileOut<T, kSc1> o(dst + tile, tile_len(n - tile, BS));
      o.store(ld_nt(src + i), threadIdx.x);
    }
  }
}

// ------------------------------------------- scalars of a captured step
// One lane copies slot (*cursor mod len) of the host ring into *out and
// advances the cursor.  The host rewrites ring slots between replays, so the
// ring is read with system-scope loads (never served from a GPU cache); the
// cursor, written only here, with agent-scope ones.  len is a power of two.
constexpr int kScalarWords = static_cast<int>(sizeof(zero_adam_scalars) / sizeof(uint32_t));
static_assert(sizeof(zero_adam_scalars) == kScalarWords * sizeof(uint32_t), "scalars are 32-bit words");

__global__ __launch_bounds__(64) void scalars_fetch_kernel(const uint32_t* ring, uint32_t len, uint32_t* cursor,
                                                           uint32_t* out) {
  if (threadIdx.x != 0) return;
  const uint32_t c = __hip_atomic_load(cursor, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t* src = ring + static_cast<size_t>(c & (len - 1)) * kScalarWords;
  uint32_t w[kScalarWords];
#pragma unroll
  for (int i = 0; i < kScalarWords; ++i) w[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
  for (int i = 0; i < kScalarWords; ++i) out[i] = w[i];
  __hip_atomic_store(cursor, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kBlock) void fill_u32_kernel(uint32_t* p, uint32_t value, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    p[i] = value;
}

// -------------------------------------------------------------- launch shape
// Launch shape, chosen by measurement on MI355X: one tile per workgroup (the
// grid covers the whole array).  The dispatcher issues workgroups in index
// order, so the tiles in flight at any moment form a narrow moving window of
// each array, which keeps HBM row locality high; a persistent grid that
// sweeps the arrays in a grid-stride loop measured 5-15% slower on every
// kernel here.  The grid-stride loops stay so that a capped grid (the
// ZERO_BLOCKS_PER_CU tuning override, or arrays beyond kMaxGridX tiles) is
// still covered.
constexpr int64_t kMaxGridX = int64_t(1) << 24;

int blocks_per_cu() {
  static int v = [] {
    const char* s = getenv("ZERO_BLOCKS_PER_CU");
    int x = s ? atoi(s) : 0;
    return (x >= 1 && x <= 64) ? x : 0;
  }();
  return v;
}

// Compute units of the current device, cached per device (calls from several
// threads may fill a slot concurrently; they store the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Blocks along x for `units` work items per owner, each block covering bs of
// them per loop iteration.
unsigned grid_x(int64_t units, int n_y, int bs = kBlock) {
  const int64_t per_iter = bs;
  int64_t need = (units + per_iter - 1) / per_iter;
  int64_t cap = kMaxGridX;
  if (blocks_per_cu() > 0) cap = static_cast<int64_t>(device_cus()) * blocks_per_cu() / (n_y > 0 ? n_y : 1);
  if (cap < 1) cap = 1;
  if (need > cap) need = cap;
  if (need < 1) need = 1;
  return static_cast<unsigned>(need);
}

// Workgroup sizes of the streaming kernels, chosen by same-box A/B runs on
// MI355X (256 is used where the size made no measurable difference).
constexpr int kRsBlock = 128;
constexpr int kAdamBlock = 64;
constexpr int kFusedBlock = 64;
constexpr int kGatherBlock = 64;

// Residency caps.  The update and the fused kernel use no LDS, but their
// launches reserve this many bytes of it per workgroup, so that at most
// 160 KiB / bytes workgroups (one wave each) are resident per CU: 10 for the
// update (8 streams) and for the fused kernel (11 streams), 8 for the fused
// kernel that also stores the reduced gradient (12 streams).  With fewer
// requests in flight the HBM keeps more row hits: measured on MI355X, the
// update goes from 6.1-6.2 TB/s uncapped to 6.72-6.75 TB/s, the fused kernel
// from 5.8-6.0 to 6.65 TB/s (same-box sweeps: update 14/12/10 per CU
// 6.64/6.72/6.74 TB/s; fused 12/10/8 6.57/6.65/6.64, storing the gradient
// 10/8 6.46/6.50).  The plain reduce (5 streams) and the gather (2) are
// fastest without a cap.  The byte counts are multiples of 1 KiB and give the
// same count under any allocation granularity up to 1 KiB.
constexpr unsigned kAdamResidencyLds = 16 * 1024;        // 160 / 16 -> 10 workgroups
constexpr unsigned kFusedResidencyLds = 16 * 1024;       // 160 / 16 -> 10 workgroups
constexpr unsigned kFusedGradResidencyLds = 20 * 1024;   // 160 / 20 -> 8 workgroups
// The reduce in accumulate mode (6 streams) and with FP32 contributions
// (5 streams of 16-byte loads) are fastest with 64-lane workgroups capped at
// 20 and 16 per CU: 6.14 -> 6.4 and 6.1 -> 6.4 TB/s on the 7B-layer shards.
constexpr int kRsAccBlock = 64;
constexpr unsigned kRsAccResidencyLds = 8 * 1024;    // 160 / 8 -> 20 workgroups
constexpr int kRsF32Block = 64;
constexpr unsigned kRsF32ResidencyLds = 10 * 1024;   // 160 / 10 -> 16 workgroups

// Owner k's parameters for a 1-D launch: contribution pointers moved to the
// owner's slice (elem_units = shard length in units of p.g's element type).
RsParams owner_slice(const RsParams& p, int k, int64_t elem_units) {
  RsParams q = p;
  for (int r = 0; r < p.n_ranks; ++r) q.g[r] = p.g[r] + static_cast<int64_t>(k) * elem_units;
  q.out[0] = p.out[k];
  return q;
}

// One launch per owner: measured 3% faster on MI355X than one 2-D launch over
// all owners (the in-flight window then never straddles two owners' buffers).
template <int N, bool ACC>
hipError_t rs_vec_launch(const RsParams& p, int n_shards, hipStream_t s) {
  for (int k = 0; k < n_shards; ++k) {
    const RsParams q = owner_slice(p, k, p.shard);
    constexpr int bs = ACC ? kRsAccBlock : kRsBlock;
    dim3 grid(grid_x(p.shard >> 2, 1, bs), 1);
    hipLaunchKernelGGL((rs_vec_kernel<N, ACC, bs>), grid, dim3(bs), ACC ? kRsAccResidencyLds : 0u, s, q);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <bool ACC>
hipError_t rs_dispatch(const RsParams& p, int n_shards, bool vec, hipStream_t s) {
  if (!vec) {
    dim3 grid(grid_x(p.shard, n_shards), n_shards);
    hipLaunchKernelGGL((rs_scalar_kernel<ACC>), grid, dim3(kBlock), 0, s, p);
    return hipGetLastError();
  }
  switch (p.n_ranks) {
    case 1: return rs_vec_launch<1, ACC>(p, n_shards, s);
    case 2: return rs_vec_launch<2, ACC>(p, n_shards, s);
    case 4: return rs_vec_launch<4, ACC>(p, n_shards, s);
    case 8: return rs_vec_launch<8, ACC>(p, n_shards, s);
    default: return rs_vec_launch<0, ACC>(p, n_shards, s);
  }
}

}  // namespace

hipError_t launch_reduce_scatter(const RsParams& p, int n_shards, bool accumulate, bool vec,
                                 hipStream_t stream) {
  return accumulate ? rs_dispatch<true>(p, n_shards, vec, stream)
                    : rs_dispatch<false>(p, n_shards, vec, stream);
}

template <int N, bool ACC>
hipError_t rs_f32_vec_launch(const RsParams& p, int n_shards, hipStream_t s) {
  for (int k = 0; k < n_shards; ++k) {
    const RsParams q = owner_slice(p, k, 2 * p.shard);   // FP32 elements = 2 BF16 units
    dim3 grid(grid_x(p.shard >> 2, 1, kRsF32Block), 1);
    hipLaunchKernelGGL((rs_f32_vec_kernel<N, ACC, kRsF32Block>), grid, dim3(kRsF32Block), kRsF32ResidencyLds, s, q);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <bool ACC>
hipError_t rs_f32_dispatch(const RsParams& p, int n_shards, bool vec, hipStream_t s) {
  if (!vec) {
    dim3 grid(grid_x(p.shard, n_shards), n_shards);
    hipLaunchKernelGGL((rs_f32_scalar_kernel<ACC>), grid, dim3(kBlock), 0, s, p);
    return hipGetLastError();
  }
  switch (p.n_ranks) {
    case 4: return rs_f32_vec_launch<4, ACC>(p, n_shards, s);
    default: return rs_f32_vec_launch<0, ACC>(p, n_shards, s);
  }
}

hipError_t launch_reduce_scatter_f32(const RsParams& p, int n_shards, bool accumulate, bool vec,
                                     hipStream_t stream) {
  return accumulate ? rs_f32_dispatch<true>(p, n_shards, vec, stream)
                    : rs_f32_dispatch<false>(p, n_shards, vec, stream);
}

template <int N, int WD, bool WG, bool ACC>
hipError_t fused_vec_launch(const FusedParams& p, int n_shards, hipStream_t s) {
  dim3 grid(grid_x(p.shard >> 2, n_shards, kFusedBlock), n_shards);
  hipLaunchKernelGGL((fused_vec_kernel<N, WD, WG, ACC, kFusedBlock>), grid, dim3(kFusedBlock),
                     WG ? kFusedGradResidencyLds : kFusedResidencyLds, s, p);
  return hipGetLastError();
}

template <int WD, bool WG, bool ACC>
hipError_t fused_dispatch_n(const FusedParams& p, int n_shards, hipStream_t s) {
  switch (p.n_ranks) {
    case 1: return fused_vec_launch<1, WD, WG, ACC>(p, n_shards, s);
    case 2: return fused_vec_launch<2, WD, WG, ACC>(p, n_shards, s);
    case 4: return fused_vec_launch<4, WD, WG, ACC>(p, n_shards, s);
    case 8: return fused_vec_launch<8, WD, WG, ACC>(p, n_shards, s);
    default: return fused_vec_launch<0, WD, WG, ACC>(p, n_shards, s);
  }
}

template <int WD>
hipError_t fused_dispatch_wd(const FusedParams& p, bool write_grad, bool acc, hipStream_t s) {
  if (write_grad)
    return acc ? fused_dispatch_n<WD, true, true>(p, 1, s) : fused_dispatch_n<WD, true, false>(p, 1, s);
  return acc ? fused_dispatch_n<WD, false, true>(p, 1, s) : fused_dispatch_n<WD, false, false>(p, 1, s);
}

// The decay mode of the update kernels: 2 when the scalars are read from
// device memory (decided in the kernel), else 1 or 0 from the host value.
int decay_mode(const zero_adam_scalars& s, const zero_adam_scalars* sdev) {
  if (sdev) return 2;
  return s.weight_decay != 0.0f ? 1 : 0;
}

hipError_t launch_fused(const FusedParams& p, int n_shards, bool write_grad, bool vec, hipStream_t s) {
  const int wd = decay_mode(p.s, p.sdev);
  if (!vec) {
    dim3 grid(grid_x(p.shard, n_shards), n_shards);
    if (wd == 2)
      hipLaunchKernelGGL((fused_scalar_kernel<2>), grid, dim3(kBlock), 0, s, p);
    else if (wd == 1)
      hipLaunchKernelGGL((fused_scalar_kernel<1>), grid, dim3(kBlock), 0, s, p);
    else
      hipLaunchKernelGGL((fused_scalar_kernel<0>), grid, dim3(kBlock), 0, s, p);
    return hipGetLastError();
  }
  const bool acc = p.gacc[0] != nullptr;
  // One launch per owner (contribution pointers moved to the owner's slice):
  // measured 3% faster on MI355X than one 2-D launch over all owners, whose
  // in-flight window straddles two owners' buffers at every owner boundary.
  for (int k = 0; k < n_shards; ++k) {
    FusedParams q = p;
    for (int r = 0; r < p.n_ranks; ++r) q.g[r] = p.g[r] + static_cast<int64_t>(k) * p.shard;
    q.p[0] = p.p[k];
    q.m[0] = p.m[k];
    q.v[0] = p.v[k];
    q.b[0] = p.b[k];
    q.gout[0] = p.gout[k];
    q.gacc[0] = p.gacc[k];
    hipError_t err;
    if (wd == 2)
      err = fused_dispatch_wd<2>(q, write_grad, acc, s);
    else if (wd == 1)
      err = fused_dispatch_wd<1>(q, write_grad, acc, s);
    else
      err = fused_dispatch_wd<0>(q, write_grad, acc, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int WD, bool SC>
hipError_t adam_launch(const AdamParams& a, bool vec, hipStream_t s) {
  if (vec) {
    dim3 grid(grid_x(a.n >> 2, 1, kAdamBlock));
    hipLaunchKernelGGL((adam_vec_kernel<WD, SC, kAdamBlock>), grid, dim3(kAdamBlock),
                       kAdamResidencyLds, s, a);
  } else {
    dim3 grid(grid_x(a.n, 1));
    hipLaunchKernelGGL((adam_scalar_kernel<WD, SC>), grid, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

template <int WD>
hipError_t adam_launch_sc(const AdamParams& a, bool vec, hipStream_t s) {
  return a.gscale ? adam_launch<WD, true>(a, vec, s) : adam_launch<WD, false>(a, vec, s);
}

hipError_t launch_adam(const AdamParams& a, bool vec, hipStream_t s) {
  const int wd = decay_mode(a.s, a.sdev);
  if (wd == 2) return adam_launch_sc<2>(a, vec, s);
  if (wd == 1) return adam_launch_sc<1>(a, vec, s);
  return adam_launch_sc<0>(a, vec, s);
}

hipError_t launch_norm(NormParams& p, bool vec, hipStream_t s) {
  const int64_t units = vec ? (p.n >> 2) : p.n;
  int64_t gx = (units + kBlock - 1) / kBlock;
  if (gx > kNormBlocks) gx = kNormBlocks;
  if (gx < 1) gx = 1;
  p.gx = static_cast<int>(gx);
  dim3 grid(p.gx, p.n_shards);
  if (vec)
    hipLaunchKernelGGL((norm_partial_kernel<true>), grid, dim3(kBlock), 0, s, p);
  else
    hipLaunchKernelGGL((norm_partial_kernel<false>), grid, dim3(kBlock), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t norm_scratch_device_ptr(double** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<double*> cache[kMaxDevices];
  static std::mutex lookup;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  double* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(lookup);
    p = cache[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      // with `dev` current: this device's copy of the array
      err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<double*>(addr);
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_gather(const GatherParams& p, int n_shards, int path, hipStream_t s) {
  constexpr int bs = kGatherBlock;
  if (path == GATHER_V16) {
    dim3 grid(grid_x(p.shard_bytes / 16, n_shards, bs), n_shards);
    hipLaunchKernelGGL((gather_kernel<u32x4, bs>), grid, dim3(bs), 0, s, p);
  } else if (path == GATHER_U32) {
    dim3 grid(grid_x(p.shard_bytes / 4, n_shards, bs), n_shards);
    hipLaunchKernelGGL((gather_kernel<uint32_t, bs>), grid, dim3(bs), 0, s, p);
  } else {
    dim3 grid(grid_x(p.shard_bytes, n_shards, bs), n_shards);
    hipLaunchKernelGGL((gather_kernel<uint8_t, bs>), grid, dim3(bs), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_scalars_fetch(const zero_adam_scalars* ring, int ring_len, uint32_t* cursor,
                                zero_adam_scalars* out, hipStream_t s) {
  hipLaunchKernelGGL(scalars_fetch_kernel, dim3(1), dim3(64), 0, s, reinterpret_cast<const uint32_t*>(ring),
                     static_cast<uint32_t>(ring_len), cursor, reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_x(n, 1)), dim3(kBlock), 0, s, p, value, n);
  return hipGetLastError();
}

}  // namespace zero
