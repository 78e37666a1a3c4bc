// A C++ caller of libzero that uses only include/zero.h and the HIP runtime
// (no Python, no PyTorch): it allocates its own device buffers, calls the
// device entry points on its own stream, and checks results that need no
// oracle:
//   - the fused reduce-scatter + update equals the two separate calls, bit for
//     bit, on a ragged multi-tile shard (vector path) and an odd one
//     (element path);
//   - a reduction of small integers times 2^-10 with weights 1/4 is exact;
//   - the all-gather equals a host-side concatenation;
//   - a zero gradient with zero decay at t = 1 leaves the master weights
//     unchanged and the moments zero;
//   - invalid arguments return the documented status and write nothing;
//   - the workspace-free gradient norm equals the workspace form bit for bit
//     on two consecutive calls (the second smaller), and both give the exact
//     sum of squares of small integers times 2^-10.
// Built as a shared library and called through one exported function, so the
// test process runs it without starting another program.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "zero.h"

namespace {

char g_msg[512];

#define FAIL(...)                                  \
  do {                                             \
    std::snprintf(g_msg, sizeof g_msg, __VA_ARGS__); \
    return 1;                                      \
  } while (0)

#define HIPOK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_));    \
  } while (0)

#define ZOK(x)                                                                \
  do {                                                                        \
    int s_ = (x);                                                             \
    if (s_ != ZERO_OK) FAIL("%s -> %s (%s)", #x, zero_status_string(s_), zero_last_error()); \
  } while (0)

uint32_t xorshift(uint32_t& s) {
  s ^= s << 13;
  s ^= s >> 17;
  s ^= s << 5;
  return s;
}

// A finite BF16 bit pattern with magnitude in [2^-20, 2^-4): random sign and
// mantissa, exponent field in [107, 123).
uint16_t random_bf16(uint32_t& s) {
  const uint32_t r = xorshift(s);
  const uint32_t sign = (r >> 31) & 1u, exp = 107u + ((r >> 7) & 15u), man = r & 0x7Fu;
  return static_cast<uint16_t>((sign << 15) | (exp << 7) | man);
}

float bits_f32(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

// The BF16 pattern of a float that BF16 represents exactly (its low 16 bits are zero).
uint16_t exact_bf16(float x) {
  uint32_t b;
  std::memcpy(&b, &x, 4);
  return static_cast<uint16_t>(b >> 16);
}

struct Dev {
  std::vector<void*> ptrs;
  ~Dev() {
    for (void* p : ptrs) (void)hipFree(p);
  }
  template <typename T>
  T* alloc(size_t n) {
    void* p = nullptr;
    if (hipMalloc(&p, n * sizeof(T) + 16) != hipSuccess) return nullptr;
    ptrs.push_back(p);
    return static_cast<T*>(p);
  }
};

template <typename T>
int upload(T* d, const std::vector<T>& h) {
  return hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) == hipSuccess ? 0 : 1;
}

template <typename T>
std::vector<T> download(const T* d, size_t n) {
  std::vector<T> h(n);
  if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) h.clear();
  return h;
}

// Fused call == reduce-scatter then per-owner update, bit for bit.
int check_fused_equals_separate(hipStream_t st, int64_t per_shard, uint32_t seed) {
  const int n = 4;
  const int64_t numel = per_shard * n;
  Dev dev;
  uint32_t s = seed;
  std::vector<uint16_t*> g(n);
  for (int r = 0; r < n; ++r) {
    g[r] = dev.alloc<uint16_t>(numel);
    if (!g[r]) FAIL("hipMalloc");
    std::vector<uint16_t> h(numel);
    for (auto& x : h) x = random_bf16(s);
    if (upload(g[r], h)) FAIL("upload");
  }
  float w[n];
  const int64_t counts[n] = {4096, 3072, 4096, 2048};
  ZOK(zero_rank_weights(counts, n, w));
  // two identical owner states: A for the separate calls, B for the fused call
  float *pA[n], *mA[n], *vA[n], *gA[n], *pB[n], *mB[n], *vB[n], *gB[n];
  uint16_t *bA[n], *bB[n];
  for (int k = 0; k < n; ++k) {
    std::vector<float> p(per_shard), m(per_shard), v(per_shard);
    for (int64_t i = 0; i < per_shard; ++i) {
      p[i] = bits_f32(static_cast<uint32_t>(random_bf16(s)) << 16) * 64.0f;
      m[i] = bits_f32(static_cast<uint32_t>(random_bf16(s)) << 16) * 0.125f;
      const float q = bits_f32(static_cast<uint32_t>(random_bf16(s)) << 16);
      v[i] = q * q;
    }
    float** dst[8] = {&pA[k], &mA[k], &vA[k], &gA[k], &pB[k], &mB[k], &vB[k], &gB[k]};
    for (float** d : dst) {
      *d = dev.alloc<float>(per_shard);
      if (!*d) FAIL("hipMalloc");
    }
    bA[k] = dev.alloc<uint16_t>(per_shard);
    bB[k] = dev.alloc<uint16_t>(per_shard);
    if (!bA[k] || !bB[k]) FAIL("hipMalloc");
    if (upload(pA[k], p) || upload(mA[k], m) || upload(vA[k], v) || upload(pB[k], p) || upload(mB[k], m) ||
        upload(vB[k], v))
      FAIL("upload");
  }
  zero_adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, 7};
  ZOK(zero_reduce_scatter(g.data(), w, n, numel, gA, n, 0, st));
  for (int k = 0; k < n; ++k) ZOK(zero_adam_shard_step(pA[k], mA[k], vA[k], bA[k], gA[k], per_shard, &hp, st));
  ZOK(zero_reduce_scatter_adam(g.data(), w, n, numel, n, pB, mB, vB, bB, nullptr, gB, &hp, st));
  HIPOK(hipStreamSynchronize(st));
  for (int k = 0; k < n; ++k) {
    const float* a[4] = {pA[k], mA[k], vA[k], gA[k]};
    const float* b[4] = {pB[k], mB[k], vB[k], gB[k]};
    for (int j = 0; j < 4; ++j) {
      auto x = download(a[j], per_shard), y = download(b[j], per_shard);
      if (x.empty() || y.empty()) FAIL("download");
      if (std::memcmp(x.data(), y.data(), per_shard * 4) != 0)
        FAIL("fused != separate: owner %d array %d (per_shard %lld)", k, j, (long long)per_shard);
    }
    auto x = download(bA[k], per_shard), y = download(bB[k], per_shard);
    if (x.empty() || y.empty() || std::memcmp(x.data(), y.data(), per_shard * 2) != 0)
      FAIL("fused != separate: owner %d BF16 shard", k);
  }
  return 0;
}

// Small integers times 2^-10 with weights 1/4: every product and partial sum
// is representable, so each owner's shard is the exact mean.
int check_exact_reduce(hipStream_t st) {
  const int n = 4;
  const int64_t per_shard = 3 * 1024 + 8, numel = per_shard * n;
  Dev dev;
  uint32_t s = 12345u;
  std::vector<std::vector<int>> ints(n, std::vector<int>(numel));
  std::vector<uint16_t*> g(n);
  for (int r = 0; r < n; ++r) {
    std::vector<uint16_t> h(numel);
    for (int64_t i = 0; i < numel; ++i) {
      ints[r][i] = static_cast<int>(xorshift(s) % 255u) - 127;
      h[i] = exact_bf16(static_cast<float>(ints[r][i]) * (1.0f / 1024.0f));
    }
    g[r] = dev.alloc<uint16_t>(numel);
    if (!g[r] || upload(g[r], h)) FAIL("upload");
  }
  float w[n];
  ZOK(zero_rank_weights(nullptr, n, w));
  float* out[n];
  for (int k = 0; k < n; ++k) {
    out[k] = dev.alloc<float>(per_shard);
    if (!out[k]) FAIL("hipMalloc");
  }
  ZOK(zero_reduce_scatter(g.data(), w, n, numel, out, n, 0, st));
  HIPOK(hipStreamSynchronize(st));
  for (int k = 0; k < n; ++k) {
    auto h = download(out[k], per_shard);
    if (h.empty()) FAIL("download");
    for (int64_t i = 0; i < per_shard; ++i) {
      const int64_t j = k * per_shard + i;
      const int sum = ints[0][j] + ints[1][j] + ints[2][j] + ints[3][j];
      const double exact = static_cast<double>(sum) / 4096.0;
      if (static_cast<double>(h[i]) != exact)
        FAIL("exact reduce: owner %d element %lld: %.9g != %.9g", k, (long long)i, h[i], exact);
    }
  }
  return 0;
}

int check_all_gather(hipStream_t st) {
  const int n = 3;
  const int64_t shard_bytes = 4096 * 16 + 6;  // ragged: byte path for the tail
  Dev dev;
  uint32_t s = 777u;
  std::vector<uint8_t> all;
  const void* src[n];
  for (int k = 0; k < n; ++k) {
    std::vector<uint8_t> h(shard_bytes);
    for (auto& b : h) b = static_cast<uint8_t>(xorshift(s));
    uint8_t* d = dev.alloc<uint8_t>(shard_bytes);
    if (!d || upload(d, h)) FAIL("upload");
    src[k] = d;
    all.insert(all.end(), h.begin(), h.end());
  }
  uint8_t* view = dev.alloc<uint8_t>(n * shard_bytes);
  if (!view) FAIL("hipMalloc");
  ZOK(zero_all_gather_layer(src, n, shard_bytes, view, st));
  HIPOK(hipStreamSynchronize(st));
  auto h = download(view, n * shard_bytes);
  if (h.size() != all.size() || std::memcmp(h.data(), all.data(), all.size()) != 0)
    FAIL("all-gather != concatenation");
  return 0;
}

// g = 0, wd = 0, m = v = 0, t = 1: m' = v' = 0 and u = 0/(0 + eps) = 0, so p' = p.
int check_zero_gradient(hipStream_t st) {
  const int64_t n = 5000;
  Dev dev;
  uint32_t s = 99u;
  std::vector<float> p(n), zeros(n, 0.0f);
  // BF16-exact values (a power-of-two scale keeps them so): RNE(p) is then p's high half
  for (auto& x : p) x = bits_f32(static_cast<uint32_t>(random_bf16(s)) << 16) * 64.0f;
  float *dp = dev.alloc<float>(n), *dm = dev.alloc<float>(n), *dv = dev.alloc<float>(n), *dg = dev.alloc<float>(n);
  uint16_t* db = dev.alloc<uint16_t>(n);
  if (!dp || !dm || !dv || !dg || !db) FAIL("hipMalloc");
  if (upload(dp, p) || upload(dm, zeros) || upload(dv, zeros) || upload(dg, zeros)) FAIL("upload");
  zero_adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1};
  ZOK(zero_adam_shard_step(dp, dm, dv, db, dg, n, &hp, st));
  HIPOK(hipStreamSynchronize(st));
  auto p2 = download(dp, n), m2 = download(dm, n), v2 = download(dv, n);
  auto b2 = download(db, n);
  if (p2.empty() || m2.empty() || v2.empty() || b2.empty()) FAIL("download");
  if (std::memcmp(p2.data(), p.data(), n * 4) != 0) FAIL("zero gradient changed the master weights");
  for (int64_t i = 0; i < n; ++i) {
    if (m2[i] != 0.0f || v2[i] != 0.0f) FAIL("zero gradient: moments not zero at %lld", (long long)i);
    if (b2[i] != exact_bf16(p[i])) FAIL("zero gradient: BF16 shard differs at %lld", (long long)i);
  }
  return 0;
}

// Invalid arguments: the documented status, nothing written.
int check_errors(hipStream_t st) {
  Dev dev;
  const int64_t n = 1024;
  uint16_t* g = dev.alloc<uint16_t>(4 * n);
  float* out = dev.alloc<float>(4 * n);
  if (!g || !out) FAIL("hipMalloc");
  const std::vector<float> sentinel(4 * n, 42.0f);
  if (upload(out, sentinel)) FAIL("upload");
  const uint16_t* gr[1] = {g};
  float w[1] = {1.0f};
  float* o3[3] = {out, out + n, out + 2 * n};
  // numel not divisible by n_shards
  int s = zero_reduce_scatter(gr, w, 1, 1000, o3, 3, 0, st);
  if (s != ZERO_ERR_SIZE) FAIL("numel %% n_shards: got %d, want ZERO_ERR_SIZE", s);
  // NULL contribution pointer
  const uint16_t* gnull[1] = {nullptr};
  s = zero_reduce_scatter(gnull, w, 1, 3 * n, o3, 3, 0, st);
  if (s != ZERO_ERR_ARG) FAIL("NULL contribution: got %d, want ZERO_ERR_ARG", s);
  // too many ranks
  s = zero_reduce_scatter(gr, w, ZERO_MAX_RANKS + 1, 3 * n, o3, 3, 0, st);
  if (s != ZERO_ERR_ARG) FAIL("n_ranks > max: got %d, want ZERO_ERR_ARG", s);
  // an FP32 output that is not 4-byte aligned
  float* mis[1] = {reinterpret_cast<float*>(reinterpret_cast<char*>(out) + 2)};
  s = zero_reduce_scatter(gr, w, 1, n, mis, 1, 0, st);
  if (s != ZERO_ERR_ALIGN) FAIL("misaligned output: got %d, want ZERO_ERR_ALIGN", s);
  // the output overlapping the contribution
  float* alias[1] = {reinterpret_cast<float*>(g)};
  s = zero_reduce_scatter(gr, w, 1, n, alias, 1, 0, st);
  if (s != ZERO_ERR_ARG) FAIL("aliased output: got %d, want ZERO_ERR_ARG", s);
  // Adam: step 0 is rejected
  zero_adam_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 0};
  s = zero_adam_shard_step(out, out + n, out + 2 * n, reinterpret_cast<uint16_t*>(out + 3 * n), out,
                           n / 2, &hp, st);
  if (s == ZERO_OK) FAIL("Adam with step 0 (and an aliased gradient) accepted");
  HIPOK(hipStreamSynchronize(st));
  auto h = download(out, 4 * n);
  if (h.empty() || std::memcmp(h.data(), sentinel.data(), sentinel.size() * 4) != 0)
    FAIL("a rejected call wrote to its output");
  if (!zero_status_string(ZERO_ERR_ALIGN) || !zero_last_error()) FAIL("status strings missing");
  return 0;
}

// Sum of squares of k * 2^-10 for integers |k| <= 50: every square and every
// partial sum is exact in binary64, so any summation order gives sum(k^2) * 2^-20.
int norm_case(hipStream_t st, int n_shards, int64_t numel, uint32_t seed) {
  Dev dev;
  uint32_t s = seed;
  const float* shards[ZERO_MAX_RANKS];
  int64_t ksq = 0;
  for (int k = 0; k < n_shards; ++k) {
    std::vector<float> h(numel);
    for (auto& x : h) {
      const int kk = static_cast<int>(xorshift(s) % 101u) - 50;
      x = static_cast<float>(kk) * 0x1p-10f;
      ksq += static_cast<int64_t>(kk) * kk;
    }
    float* d = dev.alloc<float>(numel);
    if (!d || upload(d, h)) FAIL("upload");
    shards[k] = d;
  }
  double* ws = dev.alloc<double>(static_cast<size_t>(n_shards) * ZERO_NORM_BLOCKS);
  double* out = dev.alloc<double>(2);
  float* coef = dev.alloc<float>(2);
  if (!ws || !out || !coef) FAIL("hipMalloc");
  ZOK(zero_grad_norm_sq(shards, n_shards, numel, ws, static_cast<int64_t>(n_shards) * ZERO_NORM_BLOCKS, out,
                        0.5f, coef, st));
  ZOK(zero_grad_norm_sq_no_alloc(shards, n_shards, numel, out + 1, 0.5f, coef + 1, st));
  HIPOK(hipStreamSynchronize(st));
  auto o = download(out, 2);
  auto c = download(coef, 2);
  if (o.size() != 2 || c.size() != 2) FAIL("download");
  if (std::memcmp(&o[0], &o[1], 8) != 0 || std::memcmp(&c[0], &c[1], 4) != 0)
    FAIL("norm without workspace != with workspace (%d shards of %lld)", n_shards, (long long)numel);
  if (o[0] != static_cast<double>(ksq) * 0x1p-20)
    FAIL("norm %.17g != exact %.17g", o[0], static_cast<double>(ksq) * 0x1p-20);
  return 0;
}

int check_norm_no_alloc(hipStream_t st) {
  if (norm_case(st, 3, 4096 * 5 + 4, 4242u)) return 1;   // vector path, several blocks per shard
  if (norm_case(st, 1, 7, 17u)) return 1;                // smaller: one shard, one block, element tail
  // too many shards: rejected before anything runs
  double* out = nullptr;
  if (hipMalloc(&out, 8) != hipSuccess) FAIL("hipMalloc");
  const float* many[ZERO_MAX_RANKS + 1] = {};
  const int s = zero_grad_norm_sq_no_alloc(many, ZERO_MAX_RANKS + 1, 0, out, 0.0f, nullptr, st);
  (void)hipFree(out);
  if (s != ZERO_ERR_ARG) FAIL("norm_no_alloc with %d shards: got %d, want ZERO_ERR_ARG", ZERO_MAX_RANKS + 1, s);
  return 0;
}

}  // namespace

extern "C" int zero_native_abi_check(char* msg, int msg_len) {
  g_msg[0] = '\0';
  hipStream_t st = nullptr;
  int rc = 0;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) {
    std::snprintf(g_msg, sizeof g_msg, "hipStreamCreateWithFlags failed");
    rc = 1;
  }
  if (!rc) rc = check_fused_equals_separate(st, 3 * 4096 + 4, 1u);
  if (!rc) rc = check_fused_equals_separate(st, 1001, 2u);
  if (!rc) rc = check_exact_reduce(st);
  if (!rc) rc = check_all_gather(st);
  if (!rc) rc = check_zero_gradient(st);
  if (!rc) rc = check_errors(st);
  if (!rc) rc = check_norm_no_alloc(st);
  if (st) (void)hipStreamDestroy(st);
  if (msg && msg_len > 0) std::snprintf(msg, static_cast<size_t>(msg_len), "%s", rc ? g_msg : "ok");
  return rc;
}
