// Error reporting, kernel timing and the device-wide prefix sum.
#include <atomic>
#include <mutex>
#include <vector>

#include "common.h"

namespace mlip {

// ---------------------------------------------------------------- errors ---
static thread_local char g_err[1024] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

// ------------------------------------------------------------- profiling ---
static const char *kClassNames[K_NUM_CLASSES] = {
    "graph",          "embed_aggregate",     "gemm_dense",         "route_dispatch",
    "gemm_expert_up", "gemm_expert_down",    "combine",            "readout",
    "gemm_expert_vjp_down", "gemm_expert_vjp_up", "edge_vjp", "attn_fwd",
    "attn_vjp_recv", "attn_vjp_send", "tri_fwd", "tri_vjp_recv", "tri_vjp_send",
    "gemm_expert_tan", "gemm_wgrad", "edge_tan", "moe_tan", "attn_tan", "gemm_expert_pair"};

// Profiling state is process-wide and guarded by g_prof_mu, so host threads
// may call the library concurrently with profiling on; each scope keeps its
// own event pair and files the record only when both events are recorded.
struct ProfRec {
  int k;
  hipEvent_t a, b;
};
static std::mutex g_prof_mu;
static std::atomic<bool> g_prof{false};
static std::atomic<uint64_t> g_prof_mask{~uint64_t(0)};   // classes timed while profiling is on
static std::vector<std::pair<hipEvent_t, hipEvent_t>> g_pool;
static std::vector<ProfRec> g_recs;
static double g_ms[K_NUM_CLASSES];
static int64_t g_cnt[K_NUM_CLASSES];

ProfScope::ProfScope(KClass kk, hipStream_t ss) : k(kk), s(ss) {
  if (!g_prof.load(std::memory_order_relaxed) ||
      !((g_prof_mask.load(std::memory_order_relaxed) >> int(kk)) & 1))
    return;
  std::pair<hipEvent_t, hipEvent_t> ev;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_pool.empty()) {
      ev = g_pool.back();
      g_pool.pop_back();
      slot = 1;
    }
  }
  if (slot < 0) {
    if (hipEventCreate(&ev.first) != hipSuccess) return;
    if (hipEventCreate(&ev.second) != hipSuccess) {
      (void)hipEventDestroy(ev.first);
      return;
    }
  }
  if (hipEventRecord(ev.first, s) != hipSuccess) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_pool.push_back(ev);
    slot = -1;
    return;
  }
  a = ev.first;
  b = ev.second;
  slot = 1;
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  const bool ok = hipEventRecord(b, s) == hipSuccess;
  std::lock_guard<std::mutex> lock(g_prof_mu);
  if (ok) g_recs.push_back({int(k), a, b});
  else g_pool.push_back({a, b});
}

// callers hold g_prof_mu
static int resolve_profile_locked() {
  for (auto &r : g_recs) {
    MLIP_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    MLIP_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    g_ms[r.k] += ms;
    g_cnt[r.k] += 1;
    g_pool.push_back({r.a, r.b});
  }
  g_recs.clear();
  return MLIP_OK;
}

}  // namespace mlip

using namespace mlip;

extern "C" {

const char *mlip_last_error(void) { return g_err; }
int mlip_version(void) { return 1; }

int mlip_profile_enable(int enable) {
  g_prof.store(enable != 0);
  return MLIP_OK;
}

int mlip_profile_select(uint64_t class_mask) {
  g_prof_mask.store(class_mask);
  return MLIP_OK;
}

int mlip_profile_reset(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  int rc = resolve_profile_locked();
  for (int i = 0; i < K_NUM_CLASSES; ++i) {
    g_ms[i] = 0.0;
    g_cnt[i] = 0;
  }
  return rc;
}

int mlip_profile_count(void) { return K_NUM_CLASSES; }

int mlip_profile_get(int idx, const char **name, int64_t *launches, double *total_ms) {
  MLIP_CHECK_ARG(idx >= 0 && idx < K_NUM_CLASSES, "profile index %d out of range", idx);
  std::lock_guard<std::mutex> lock(g_prof_mu);
  int rc = resolve_profile_locked();
  if (rc != MLIP_OK) return rc;
  if (name) *name = kClassNames[idx];
  if (launches) *launches = g_cnt[idx];
  if (total_ms) *total_ms = g_ms[idx];
  return MLIP_OK;
}

}  // extern "C"

namespace mlip {

// ------------------------------------------------------------------ scan ---
// Three passes over 1024-element tiles: tile sums, a scan of the tile sums
// (one workgroup, serial over chunks of 1024 tiles), then the tile scans.
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_PER_THREAD = 4;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_PER_THREAD;

// Exclusive scan of one value per thread over a 256-thread block.
__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t *total, int32_t *lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int32_t wave_off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SCAN_THREADS / 64; ++w) {
    int32_t s = lds[w];
    if (w < wave) wave_off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wave_off + x - v;
}

__global__ void __launch_bounds__(SCAN_THREADS) scan_tile_sums(const int32_t *__restrict__ in,
                                                               int64_t n, int32_t *__restrict__ sums) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  int64_t base = int64_t(blockIdx.x) * SCAN_TILE + int64_t(threadIdx.x) * SCAN_PER_THREAD;
  int32_t v = 0;
#pragma unroll
  for (int j = 0; j < SCAN_PER_THREAD; ++j)
    if (base + j < n) v += in[base + j];
  int32_t tot;
  block_exclusive_scan(v, &tot, lds);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(SCAN_THREADS) scan_sums(int32_t *__restrict__ sums, int64_t nt) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  int32_t carry = 0;
  for (int64_t c0 = 0; c0 < nt; c0 += SCAN_TILE) {
    int64_t base = c0 + int64_t(threadIdx.x) * SCAN_PER_THREAD;
    int32_t v[SCAN_PER_THREAD];
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER_THREAD; ++j) {
      v[j] = (base + j < nt) ? sums[base + j] : 0;
      s += v[j];
    }
    int32_t tot;
    int32_t off = block_exclusive_scan(s, &tot, lds) + carry;
#pragma unroll
    for (int j = 0; j < SCAN_PER_THREAD; ++j) {
      if (base + j < nt) sums[base + j] = off;
      off += v[j];
    }
    carry += tot;
  }
}

__global__ void __launch_bounds__(SCAN_THREADS) scan_apply(const int32_t *in, int32_t *out,
                                                           int64_t n, const int32_t *__restrict__ sums,
                                                           int write_total) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  int64_t base = int64_t(blockIdx.x) * SCAN_TILE + int64_t(threadIdx.x) * SCAN_PER_THREAD;
  int32_t v[SCAN_PER_THREAD];
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < SCAN_PER_THREAD; ++j) {
    v[j] = (base + j < n) ? in[base + j] : 0;
    s += v[j];
  }
  int32_t tot;
  int32_t off = block_exclusive_scan(s, &tot, lds) + (sums ? sums[blockIdx.x] : 0);
#pragma unroll
  for (int j = 0; j < SCAN_PER_THREAD; ++j) {
    if (base + j < n) out[base + j] = off;
    off += v[j];
  }
  if (write_total && blockIdx.x == gridDim.x - 1 && threadIdx.x == SCAN_THREADS - 1) out[n] = off;
}

size_t scan_tmp_elems(int64_t n) { return size_t(cdiv(n, SCAN_TILE)) + 1; }

__global__ void scan_zero_total(int32_t *out) { out[0] = 0; }

__global__ void __launch_bounds__(SCAN_THREADS) scan_single(const int32_t *in, int32_t *out,
                                                            int64_t n, int write_total) {
  __shared__ int32_t lds[SCAN_THREADS / 64];
  int32_t carry = 0;
  for (int64_t c0 = 0; c0 < n; c0 += SCAN_TILE) {
    const int64_t base = c0 + int64_t(threadIdx.x) * SCAN_PER_THREAD;
    int32_t v[SCAN_PER_THREAD];
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER_THREAD; ++j) {
      v[j] = (base + j < n) ? in[base + j] : 0;
      sum += v[j];
    }
    int32_t tot;
    int32_t off = block_exclusive_scan(sum, &tot, lds) + carry;
#pragma unroll
    for (int j = 0; j < SCAN_PER_THREAD; ++j) {
      if (base + j < n) out[base + j] = off;
      off += v[j];
    }
    carry += tot;
  }
  if (write_total && threadIdx.x == 0) out[n] = carry;
}

int exclusive_scan(const int32_t *in, int32_t *out, int64_t n, bool write_total, int32_t *tmp,
                   hipStream_t stream) {
  if (n <= 0) {
    if (write_total) {
      scan_zero_total<<<1, 1, 0, stream>>>(out);
      MLIP_LAUNCHED();
    }
    return MLIP_OK;
  }
  int64_t nt = cdiv(n, SCAN_TILE);
  if (nt > 1 && nt <= 64) {
    // small arrays: one workgroup walks the tiles with a running carry
    scan_single<<<1, SCAN_THREADS, 0, stream>>>(in, out, n, write_total ? 1 : 0);
    MLIP_LAUNCHED();
    return MLIP_OK;
  }
  if (nt > 1) {
    scan_tile_sums<<<dim3(unsigned(nt)), dim3(SCAN_THREADS), 0, stream>>>(in, n, tmp);
    MLIP_LAUNCHED();
    scan_sums<<<dim3(1), dim3(SCAN_THREADS), 0, stream>>>(tmp, nt);
    MLIP_LAUNCHED();
  }
  scan_apply<<<dim3(unsigned(nt)), dim3(SCAN_THREADS), 0, stream>>>(in, out, n, nt > 1 ? tmp : nullptr,
                                                                    write_total ? 1 : 0);
  MLIP_LAUNCHED();
  return MLIP_OK;
}

}  // namespace mlip
