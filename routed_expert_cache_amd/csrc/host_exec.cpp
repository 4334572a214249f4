// Host executor for the host set C: the experts a cache step leaves to the
// CPU are evaluated here, on a persistent pool of threads, from the same
// packed rows of the pinned host pool that fills copy to the GPU.
//
// [FT] section "q* 策略": the misses not filled are computed by the CPU in
// parallel with the GPU and the two partial sums are added.  [OSDI] section
// 4.2: FP8 weights stay as stored; the CPU expands the codes with bit
// operations, dots each 128-wide block first and multiplies it by its scale
// once (post-scaling).  [OSDI] section 4.3: an expert is gate, up and down
// projections, down reads SiLU(gate) * up.
//
// Packed rows (the brick format of the GPU slots): a matrix W [N][K] is a run
// of 1 KB bricks of 16 rows x KB columns (KB = 32 BF16 or 64 E4M3), brick
// (t, kt) at (t * (K / KB) + kt) KB; the 16-byte chunk c = 16 j + r of a
// brick holds W[16 t + r][KB kt + (KB / 4) j + e].  Gate/up rows interleave:
// packed row 16 t + r is gate row 8 t + r (r < 8) or up row 8 t + r - 8.
//
// Work of one call, in two passes over the thread pool: (1) every (host
// expert, brick row) pair -> 8 features of h for every token that picked
// the expert, in FP32; (2) every 16-row block of y_host -> for each token,
// the gate-weighted down products of its host experts summed in pick order.
// Each output is summed by one thread in a fixed order: the same bits on
// every call, with any number of threads.
#include "../../include/moe.h"

#include <hip/hip_runtime_api.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include <pthread.h>
#include <sched.h>

#include <cctype>
#include <cstdio>
#include <cstdlib>
#include <string>

namespace moe {
void set_error(const char* fmt, ...);   // the library's per-thread error message
void clear_error();
}  // namespace moe

#define HX_FAIL(code, ...)         \
  do {                             \
    ::moe::set_error(__VA_ARGS__); \
    return code;                   \
  } while (0)

namespace {

// ------------------------------------------------------------ E4M3 decoding
// E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
// subnormal (m * 2^-9); 0x7F / 0xFF are NaN; there are no infinities.
inline float e4m3_to_f32(uint8_t c) {
  const uint32_t s = (uint32_t)(c >> 7) << 31, e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if ((c & 0x7Fu) == 0x7Fu) {
    uint32_t nan = s | 0x7FC00000u;
    std::memcpy(&v, &nan, 4);
    return v;
  }
  if (e == 0) {
    v = (float)m * (1.0f / 512.0f);
    return s ? -v : v;
  }
  const uint32_t bits = s | ((e + 120u) << 23) | (m << 20);
  std::memcpy(&v, &bits, 4);
  return v;
}

inline float bf16_to_f32(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline float silu(float a) { return a / (1.0f + std::exp(-a)); }

// ------------------------------------------------------------ brick-row dot
// acc[r] (16 rows) += sum over the brick row's K of W[r][k] * v[k], for one
// vector v (FP32, length K).  FP8: each 128-wide K block is dotted on its
// own and multiplied by sc(row half, block) before it is added.
struct RowScale {               // FP8 scale of a 16-row brick row at K block b
  const float* lo;              // rows 0..7: lo[b]
  const float* hi;              // rows 8..15: hi[b]
};

void dot_rows_bf16_scalar(const uint16_t* brow, int nkt, const float* v, float* acc) {
  for (int kt = 0; kt < nkt; ++kt) {
    const uint16_t* b = brow + (size_t)kt * 512;
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) {
        const uint16_t* w = b + (16 * j + r) * 8;
        const float* x = v + 32 * kt + 8 * j;
        float s = 0.f;
        for (int e = 0; e < 8; ++e) s += bf16_to_f32(w[e]) * x[e];
        acc[r] += s;
      }
  }
}

void dot_rows_fp8_scalar(const uint8_t* brow, int nkt, const float* v, RowScale sc, float* acc) {
  float blk[16];
  for (int kt = 0; kt < nkt; ++kt) {
    if ((kt & 1) == 0) std::fill(blk, blk + 16, 0.f);
    const uint8_t* b = brow + (size_t)kt * 1024;
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) {
        const uint8_t* w = b + (16 * j + r) * 16;
        const float* x = v + 64 * kt + 16 * j;
        float s = 0.f;
        for (int e = 0; e < 16; ++e) s += e4m3_to_f32(w[e]) * x[e];
        blk[r] += s;
      }
    if ((kt & 1) == 1 || kt == nkt - 1) {
      const int bk = kt >> 1;
      for (int r = 0; r < 16; ++r) acc[r] += (r < 8 ? sc.lo[bk] : sc.hi[bk]) * blk[r];
    }
  }
}

__attribute__((target("avx512f,avx512bw"))) inline __m512 bf16x16_to_f32(__m256i h) {
  return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
}

// 16 E4M3 codes -> 16 floats equal to 2^-8 times their values.  With its
// 7 magnitude bits shifted up by 7, an E4M3 code is the FP16 pattern of
// value * 2^-8 (exponent bias 15 = 7 + 8; E4M3 subnormals land on FP16
// subnormals with the same mantissa), so one FP16 -> FP32 conversion expands
// 16 codes exactly; the callers fold the 2^8 into the block scale.  The NaN
// codes (0x7F, 0xFF) are patched to NaN.
__attribute__((target("avx512f,avx512bw,avx512vl"))) inline __m512 e4m3x16_to_f32_div256(__m128i c8) {
  const __m256i c = _mm256_cvtepu8_epi16(c8);
  const __m256i mag = _mm256_and_si256(c, _mm256_set1_epi16(0x7F));
  const __m256i sign = _mm256_slli_epi16(_mm256_and_si256(c, _mm256_set1_epi16(0x80)), 8);
  const __m256i h = _mm256_or_si256(sign, _mm256_slli_epi16(mag, 7));
  const __mmask16 nan = _mm256_cmpeq_epi16_mask(mag, _mm256_set1_epi16(0x7F));
  return _mm512_mask_blend_ps(nan, _mm512_cvtph_ps(h), _mm512_set1_ps(__builtin_nanf("")));
}

// Lane layout of the AVX-512 accumulators: a[q] holds rows 2q, 2q + 1, one
// 8-wide K chunk each (BF16), or rows q (FP8: 16-wide chunk); the horizontal
// sums at the end give the row sums.
__attribute__((target("avx512f,avx512bw"))) void dot_rows_bf16_avx512(const uint16_t* brow, int nkt, const float* v,
                                                                       float* acc) {
  __m512 a[8];
  for (int q = 0; q < 8; ++q) a[q] = _mm512_setzero_ps();
  for (int kt = 0; kt < nkt; ++kt) {
    const uint16_t* b = brow + (size_t)kt * 512;
    for (int j = 0; j < 4; ++j) {
      const __m256 x8 = _mm256_loadu_ps(v + 32 * kt + 8 * j);
      const __m512 x16 = _mm512_castpd_ps(
          _mm512_insertf64x4(_mm512_castps_pd(_mm512_castps256_ps512(x8)), _mm256_castps_pd(x8), 1));
      const uint16_t* w = b + 16 * j * 8;   // rows 0..15, 8 values each: 256 bytes
      for (int q = 0; q < 8; ++q) {
        const __m512 wf = bf16x16_to_f32(_mm256_loadu_si256((const __m256i*)(w + 16 * q)));
        a[q] = _mm512_fmadd_ps(wf, x16, a[q]);
      }
    }
  }
  for (int q = 0; q < 8; ++q) {
    const __m256 lo = _mm512_castps512_ps256(a[q]);
    const __m256 hi = _mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(a[q]), 1));
    float t0[8], t1[8];
    _mm256_storeu_ps(t0, lo);
    _mm256_storeu_ps(t1, hi);
    float s0 = 0.f, s1 = 0.f;
    for (int e = 0; e < 8; ++e) {
      s0 += t0[e];
      s1 += t1[e];
    }
    acc[2 * q] += s0;
    acc[2 * q + 1] += s1;
  }
}

__attribute__((target("avx512f,avx512bw,avx512vl"))) void dot_rows_fp8_avx512(const uint8_t* brow, int nkt,
                                                                               const float* v, RowScale sc, float* acc) {
  __m512 t[16], blk[16];
  for (int r = 0; r < 16; ++r) t[r] = _mm512_setzero_ps();
  for (int kt = 0; kt < nkt; ++kt) {
    if ((kt & 1) == 0)
      for (int r = 0; r < 16; ++r) blk[r] = _mm512_setzero_ps();
    const uint8_t* b = brow + (size_t)kt * 1024;
    for (int j = 0; j < 4; ++j) {
      const __m512 x = _mm512_loadu_ps(v + 64 * kt + 16 * j);
      for (int r = 0; r < 16; ++r) {
        const __m512 wf = e4m3x16_to_f32_div256(_mm_loadu_si128((const __m128i*)(b + (16 * j + r) * 16)));
        blk[r] = _mm512_fmadd_ps(wf, x, blk[r]);
      }
    }
    if ((kt & 1) == 1 || kt == nkt - 1) {
      const int bk = kt >> 1;
      // the codes were expanded as 2^-8 times their values: scale by 2^8 too (exact)
      const __m512 slo = _mm512_set1_ps(256.0f * sc.lo[bk]), shi = _mm512_set1_ps(256.0f * sc.hi[bk]);
      for (int r = 0; r < 16; ++r) t[r] = _mm512_fmadd_ps(r < 8 ? slo : shi, blk[r], t[r]);
    }
  }
  for (int r = 0; r < 16; ++r) acc[r] += _mm512_reduce_add_ps(t[r]);
}

bool have_avx512() {
  static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                         __builtin_cpu_supports("avx512vl");
  return ok;
}

// ------------------------------------------------------------ core placement
// The pages run the host set on a resident pool of threads pinned to
// physical cores ([FT] section "Graph 内的 CPU 执行分支").  The plan: the
// CPUs this process may use, one per physical core first (the lowest CPU of
// each core's SMT siblings), cores on the GPU's NUMA node before the others,
// then the remaining SMT siblings in the same order; thread i takes entry
// i (modulo the list).
std::vector<int> parse_cpulist(const std::string& s) {
  std::vector<int> out;
  size_t i = 0;
  while (i < s.size()) {
    while (i < s.size() && (s[i] < '0' || s[i] > '9')) ++i;
    if (i >= s.size()) break;
    int a = 0;
    while (i < s.size() && s[i] >= '0' && s[i] <= '9') a = 10 * a + (s[i++] - '0');
    int b = a;
    if (i < s.size() && s[i] == '-') {
      ++i;
      b = 0;
      while (i < s.size() && s[i] >= '0' && s[i] <= '9') b = 10 * b + (s[i++] - '0');
    }
    for (int c = a; c <= b && c < 65536; ++c) out.push_back(c);
  }
  return out;
}

std::string read_line(const std::string& path) {
  std::string out;
  if (FILE* f = std::fopen(path.c_str(), "r")) {
    char buf[4096];
    if (std::fgets(buf, sizeof buf, f)) out = buf;
    std::fclose(f);
  }
  return out;
}

int gpu_numa_node() {
  int dev = 0;
  char bus[64] = {0};
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetPCIBusId(bus, sizeof bus, dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  std::string id(bus);
  for (char& ch : id) ch = (char)std::tolower((unsigned char)ch);
  const std::string v = read_line("/sys/bus/pci/devices/" + id + "/numa_node");
  return v.empty() ? -1 : std::atoi(v.c_str());
}

std::vector<int> core_plan(int* node_out) {
  cpu_set_t set;
  CPU_ZERO(&set);
  std::vector<int> allowed;
  if (sched_getaffinity(0, sizeof set, &set) == 0)
    for (int c = 0; c < CPU_SETSIZE; ++c)
      if (CPU_ISSET(c, &set)) allowed.push_back(c);
  const int node = gpu_numa_node();
  *node_out = node;
  std::vector<int> local;
  if (node >= 0) local = parse_cpulist(read_line("/sys/devices/system/node/node" + std::to_string(node) + "/cpulist"));
  auto is_local = [&](int c) { return std::find(local.begin(), local.end(), c) != local.end(); };
  // rank 0: the first allowed sibling of its core; rank r: the r-th
  std::vector<std::pair<int, int>> keyed;   // (sibling rank * 2 + remote, cpu)
  for (int c : allowed) {
    std::vector<int> sib = parse_cpulist(
        read_line("/sys/devices/system/cpu/cpu" + std::to_string(c) + "/topology/thread_siblings_list"));
    int rank = 0;
    for (int s2 : sib)
      if (s2 < c && std::find(allowed.begin(), allowed.end(), s2) != allowed.end()) ++rank;
    keyed.push_back({rank * 2 + (is_local(c) ? 0 : 1), c});
  }
  std::stable_sort(keyed.begin(), keyed.end(),
                   [](const std::pair<int, int>& a, const std::pair<int, int>& b) { return a.first < b.first; });
  std::vector<int> out;
  for (auto& kc : keyed) out.push_back(kc.second);
  return out;
}

void pin_self(int cpu) {
  if (cpu < 0) return;
  cpu_set_t set;
  CPU_ZERO(&set);
  CPU_SET(cpu, &set);
  (void)pthread_setaffinity_np(pthread_self(), sizeof set, &set);
}

// ------------------------------------------------------------ thread pool
// run(n_items, f): f(item) for every item in [0, n_items), spread over the
// pool; returns when all are done.  Unpinned, the pool is n - 1 worker
// threads plus the calling thread.  Pinned (cpus given), it is n worker
// threads, worker i on cpus[i], and the calling thread only waits: a caller
// that also took items would run wherever the OS put it, possibly on a
// pinned worker's core, and every pass would wait for the two sharing it.
class Pool {
 public:
  Pool(int n, const std::vector<int>& cpus) : n_(n), caller_works_(cpus.empty()) {
    for (int i = caller_works_ ? 1 : 0; i < n_; ++i) {
      const int cpu = cpus.empty() ? -1 : cpus[(size_t)i % cpus.size()];
      th_.emplace_back([this, cpu] {
        pin_self(cpu);
        loop();
      });
    }
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
      ++gen_;
      gen_seen_.store(gen_, std::memory_order_release);
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  int size() const { return n_; }
  void run(int n_items, const std::function<void(int)>& f) {
    {
      std::lock_guard<std::mutex> lk(mu_);
      f_ = &f;
      n_items_ = n_items;
      next_.store(0);
      busy_ = (int)th_.size();
      ++gen_;
      gen_seen_.store(gen_, std::memory_order_release);
    }
    cv_.notify_all();
    if (caller_works_) work();
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [this] { return busy_ == 0; });
    f_ = nullptr;
  }

 private:
  void work() {
    for (;;) {
      const int i = next_.fetch_add(1);
      if (i >= n_items_) break;
      (*f_)(i);
    }
  }
  // A worker spins for about kSpin before it sleeps, so calls that come one
  // layer apart find it awake (a sleeping thread takes tens of microseconds
  // to wake).
  static constexpr auto kSpin = std::chrono::microseconds(250);
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      const auto t0 = std::chrono::steady_clock::now();
      while (gen_seen_.load(std::memory_order_acquire) == seen &&
             std::chrono::steady_clock::now() - t0 < kSpin)
        _mm_pause();
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_ != seen; });
        seen = gen_;
        if (stop_) return;
      }
      work();
      {
        std::lock_guard<std::mutex> lk(mu_);
        if (--busy_ == 0) done_cv_.notify_one();
      }
    }
  }
  int n_;
  bool caller_works_;
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_, done_cv_;
  uint64_t gen_ = 0;
  std::atomic<uint64_t> gen_seen_{0};   // gen_, readable without the lock (the spin)
  bool stop_ = false;
  int busy_ = 0;
  int n_items_ = 0;
  std::atomic<int> next_{0};
  const std::function<void(int)>* f_ = nullptr;
};

}  // namespace

struct HostCall {             // the arguments of one moe_host_forward
  moe_host_pool pool;
  int32_t wtype, H, I;
  const uint16_t* x;
  const int32_t* ids;
  const int32_t* pick_slot;
  const float* w;
  int32_t T, k;
  float* y_host;
};

struct SignalJob {             // a call that waits for `ready`, then publishes `done`
  HostCall call;
  const volatile uint32_t* ready;
  volatile uint32_t* done;
  uint32_t seq;
};

struct moe_host_exec {
  Pool pool;
  bool simd;                   // the AVX-512 path
  std::mutex call_mu;          // one call at a time per executor
  std::vector<float> xs;       // [T][H] x in FP32
  std::vector<float> hbuf;     // [n_pairs][I] h in FP32
  HostCall queued{};           // the call an enqueued host function runs (persistent: graphs replay it)
  std::atomic<int32_t> status{MOE_OK};   // first failure of an enqueued run
  uint64_t n_calls = 0, ns = 0;          // calls with host picks, time spent in them
  // the dispatcher thread of moe_host_forward_signal (started by its first call)
  std::thread dispatcher;
  std::mutex q_mu;
  std::condition_variable q_cv;
  std::vector<SignalJob> q;
  bool q_stop = false;
  std::vector<int> cpus;       // CPU of thread i (0: the dispatcher), empty when not pinned
  int numa_node = -1;
  moe_host_exec(int n, bool s, const std::vector<int>& c, int node)
      : pool(n, c), simd(s), cpus(c), numa_node(node) {}
  ~moe_host_exec() {
    if (dispatcher.joinable()) {
      {
        std::lock_guard<std::mutex> lk(q_mu);
        q_stop = true;
      }
      q_cv.notify_all();
      dispatcher.join();
    }
  }
};

extern "C" moe_status moe_host_exec_create(int32_t n_threads, uint32_t flags, moe_host_exec_t* out) {
  ::moe::clear_error();
  if (!out) HX_FAIL(MOE_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (n_threads < 1 || n_threads > 1024) HX_FAIL(MOE_ERR_ARG, "n_threads %d not in [1, 1024]", n_threads);
  if (flags & ~(MOE_HOST_PORTABLE | MOE_HOST_PIN)) HX_FAIL(MOE_ERR_ARG, "bad flags %u", flags);
  std::vector<int> cpus;
  int node = -1;
  if (flags & MOE_HOST_PIN) {
    cpus = core_plan(&node);
    if (cpus.empty()) HX_FAIL(MOE_ERR_STATE, "no CPU in this process's affinity set");
    std::vector<int> per_thread;
    for (int i = 0; i < n_threads; ++i) per_thread.push_back(cpus[(size_t)i % cpus.size()]);
    cpus.swap(per_thread);
  }
  moe_host_exec* h =
      new (std::nothrow) moe_host_exec(n_threads, have_avx512() && !(flags & MOE_HOST_PORTABLE), cpus, node);
  if (!h) HX_FAIL(MOE_ERR_NO_SPACE, "out of host memory");
  *out = h;
  return MOE_OK;
}

extern "C" moe_status moe_host_exec_destroy(moe_host_exec_t h) {
  ::moe::clear_error();
  delete h;
  return MOE_OK;
}

extern "C" int32_t moe_host_exec_simd(moe_host_exec_t h) { return h && h->simd ? 512 : 0; }

extern "C" moe_status moe_host_exec_cpus(moe_host_exec_t h, int32_t* cpus, int32_t n, int32_t* numa_node) {
  ::moe::clear_error();
  if (!h || (n > 0 && !cpus)) HX_FAIL(MOE_ERR_ARG, "null argument");
  for (int i = 0; i < n; ++i) cpus[i] = (i < h->pool.size() && !h->cpus.empty()) ? h->cpus[(size_t)i] : -1;
  if (numa_node) *numa_node = h->numa_node;
  return MOE_OK;
}

extern "C" moe_status moe_host_forward(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H,
                                       int32_t I, const uint16_t* x, const int32_t* ids, const int32_t* pick_slot,
                                       const float* w, int32_t T, int32_t k, float* y_host) {
  ::moe::clear_error();
  if (!h || !pool || !y_host) HX_FAIL(MOE_ERR_ARG, "null executor, pool or y_host");
  if (T < 0 || k < 1) HX_FAIL(MOE_ERR_SHAPE, "bad T=%d k=%d", T, k);
  if (wtype != MOE_W_BF16 && wtype != MOE_W_FP8_B128) HX_FAIL(MOE_ERR_ARG, "bad wtype %d", wtype);
  const bool fp8 = wtype == MOE_W_FP8_B128;
  const int KB = fp8 ? 64 : 32;
  if (H <= 0 || I <= 0 || H % KB || I % KB || I % 8 || (fp8 && (H % 128 || I % 128)))
    HX_FAIL(MOE_ERR_SHAPE, "host executor needs H, I multiples of %d and I %% 8 == 0 (H=%d I=%d)", fp8 ? 128 : 32, H, I);
  if (T == 0) return MOE_OK;
  if (!x || !ids || !pick_slot || !w || !pool->w_gate_up || !pool->w_down) HX_FAIL(MOE_ERR_ARG, "null argument");
  if (fp8 && (!pool->s_gate || !pool->s_up || !pool->s_down)) HX_FAIL(MOE_ERR_ARG, "FP8 pool without scales");
  std::lock_guard<std::mutex> lk(h->call_mu);

  // the host picks, token-major in pick order: pair p = (token, pick)
  std::vector<int> pt, pj;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j)
      if (pick_slot[t * k + j] < 0) {
        if (ids[t * k + j] < 0) HX_FAIL(MOE_ERR_ARG, "host pick (%d, %d) has id %d", t, j, ids[t * k + j]);
        pt.push_back(t);
        pj.push_back(j);
      }
  std::memset(y_host, 0, sizeof(float) * (size_t)T * H);
  const int n_pairs = (int)pt.size();
  if (n_pairs == 0) return MOE_OK;

  const auto t_start = std::chrono::steady_clock::now();
  h->xs.resize((size_t)T * H);
  for (size_t i = 0; i < (size_t)T * H; ++i) h->xs[i] = bf16_to_f32(x[i]);
  h->hbuf.resize((size_t)n_pairs * I);
  const bool simd = h->simd;
  const int nkt_gu = H / KB, nkt_dn = I / KB;
  const size_t brick_row_gu = (size_t)nkt_gu * 1024, brick_row_dn = (size_t)nkt_dn * 1024;

  // (1) gate/up: item = (pair, brick row t of I/8): gate/up rows 8t..8t+7
  const int RA = I / 8;
  h->pool.run(n_pairs * RA, [&](int item) {
    const int p = item / RA, t = item - p * RA;
    const int id = ids[pt[p] * k + pj[p]];
    const char* brow = (const char*)pool->w_gate_up[id] + (size_t)t * brick_row_gu;
    const float* v = h->xs.data() + (size_t)pt[p] * H;
    float acc[16] = {0};
    if (fp8) {
      const int nbk = H / 128, rb = (8 * t) / 128;
      const RowScale sc{pool->s_gate[id] + (size_t)rb * nbk, pool->s_up[id] + (size_t)rb * nbk};
      if (simd)
        dot_rows_fp8_avx512((const uint8_t*)brow, nkt_gu, v, sc, acc);
      else
        dot_rows_fp8_scalar((const uint8_t*)brow, nkt_gu, v, sc, acc);
    } else {
      if (simd)
        dot_rows_bf16_avx512((const uint16_t*)brow, nkt_gu, v, acc);
      else
        dot_rows_bf16_scalar((const uint16_t*)brow, nkt_gu, v, acc);
    }
    float* hp = h->hbuf.data() + (size_t)p * I + 8 * t;
    for (int r = 0; r < 8; ++r) hp[r] = silu(acc[r]) * acc[8 + r];
  });

  // (2) down: item = 16-row block of y_host; for each token, its host pairs in pick order
  h->pool.run(H / 16, [&](int blk) {
    float acc[16];
    for (int p0 = 0; p0 < n_pairs;) {
      const int t = pt[p0];
      int p1 = p0;
      while (p1 < n_pairs && pt[p1] == t) ++p1;
      float yt[16] = {0};
      for (int p = p0; p < p1; ++p) {
        const int id = ids[t * k + pj[p]];
        const char* brow = (const char*)pool->w_down[id] + (size_t)blk * brick_row_dn;
        const float* v = h->hbuf.data() + (size_t)p * I;
        std::fill(acc, acc + 16, 0.f);
        if (fp8) {
          const int nbk = I / 128;
          const float* s = pool->s_down[id] + (size_t)((16 * blk) / 128) * nbk;
          const RowScale sc{s, s};
          if (simd)
            dot_rows_fp8_avx512((const uint8_t*)brow, nkt_dn, v, sc, acc);
          else
            dot_rows_fp8_scalar((const uint8_t*)brow, nkt_dn, v, sc, acc);
        } else {
          if (simd)
            dot_rows_bf16_avx512((const uint16_t*)brow, nkt_dn, v, acc);
          else
            dot_rows_bf16_scalar((const uint16_t*)brow, nkt_dn, v, acc);
        }
        const float wp = w[t * k + pj[p]];
        for (int r = 0; r < 16; ++r) yt[r] += wp * acc[r];
      }
      std::memcpy(y_host + (size_t)t * H + 16 * blk, yt, sizeof(yt));
      p0 = p1;
    }
  });
  h->n_calls += 1;
  h->ns += (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t_start)
               .count();
  return MOE_OK;
}

extern "C" moe_status moe_host_exec_stats(moe_host_exec_t h, uint64_t* calls, uint64_t* ns) {
  ::moe::clear_error();
  if (!h || !calls || !ns) HX_FAIL(MOE_ERR_ARG, "null argument");
  std::lock_guard<std::mutex> lk(h->call_mu);
  *calls = h->n_calls;
  *ns = h->ns;
  return MOE_OK;
}

// ------------------------------------------------------------ stream-ordered form
namespace {
void host_call_fn(void* p) {
  moe_host_exec* h = static_cast<moe_host_exec*>(p);
  const HostCall& c = h->queued;
  const moe_status st = moe_host_forward(h, &c.pool, c.wtype, c.H, c.I, c.x, c.ids, c.pick_slot, c.w, c.T, c.k,
                                         c.y_host);
  if (st != MOE_OK) {
    int32_t ok = MOE_OK;
    h->status.compare_exchange_strong(ok, st);
  }
}
}  // namespace

extern "C" moe_status moe_host_forward_enqueue(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H,
                                               int32_t I, const uint16_t* x, const int32_t* ids,
                                               const int32_t* pick_slot, const float* w, int32_t T, int32_t k,
                                               float* y_host, hipStream_t stream) {
  ::moe::clear_error();
  if (!h || !pool) HX_FAIL(MOE_ERR_ARG, "null executor or pool");
  h->queued = HostCall{*pool, wtype, H, I, x, ids, pick_slot, w, T, k, y_host};
  const hipError_t e = hipLaunchHostFunc(stream, host_call_fn, h);
  if (e != hipSuccess) HX_FAIL(MOE_ERR_HIP, "hipLaunchHostFunc failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_host_exec_status(moe_host_exec_t h) {
  if (!h) return MOE_ERR_ARG;
  return (moe_status)h->status.exchange(MOE_OK);
}

// ------------------------------------------------------------ signalled form
namespace {
constexpr auto kReadyTimeout = std::chrono::seconds(2);

void dispatch_loop(moe_host_exec* h) {
  for (;;) {
    SignalJob job;
    bool stopping;
    {
      std::unique_lock<std::mutex> lk(h->q_mu);
      h->q_cv.wait(lk, [&] { return h->q_stop || !h->q.empty(); });
      if (h->q.empty()) return;   // stopping with nothing queued
      job = h->q.front();
      h->q.erase(h->q.begin());
      stopping = h->q_stop;
    }
    // wait (bounded) until the stream has written this call's inputs; a
    // stopping executor abandons the call but still releases the GPU
    const auto t0 = std::chrono::steady_clock::now();
    bool ready = !stopping;
    while (ready && (int32_t)(*job.ready - job.seq) < 0) {
      if (std::chrono::steady_clock::now() - t0 > kReadyTimeout) {
        ready = false;
        break;
      }
      _mm_pause();
    }
    std::atomic_thread_fence(std::memory_order_acquire);
    moe_status st = MOE_ERR_STATE;
    if (ready) {
      const HostCall& c = job.call;
      st = moe_host_forward(h, &c.pool, c.wtype, c.H, c.I, c.x, c.ids, c.pick_slot, c.w, c.T, c.k, c.y_host);
    }
    if (st != MOE_OK) {
      int32_t ok = MOE_OK;
      h->status.compare_exchange_strong(ok, st);
    }
    std::atomic_thread_fence(std::memory_order_release);   // y_host before `done`
    *job.done = job.seq;
  }
}
}  // namespace

extern "C" moe_status moe_host_forward_signal(moe_host_exec_t h, const moe_host_pool* pool, int32_t wtype, int32_t H,
                                              int32_t I, const uint16_t* x, const int32_t* ids,
                                              const int32_t* pick_slot, const float* w, int32_t T, int32_t k,
                                              float* y_host, const uint32_t* ready, uint32_t* done, uint32_t seq) {
  ::moe::clear_error();
  if (!h || !pool || !ready || !done) HX_FAIL(MOE_ERR_ARG, "null executor, pool or signal word");
  {
    std::lock_guard<std::mutex> lk(h->q_mu);
    if (!h->dispatcher.joinable()) h->dispatcher = std::thread(dispatch_loop, h);
    h->q.push_back(SignalJob{HostCall{*pool, wtype, H, I, x, ids, pick_slot, w, T, k, y_host}, ready, done, seq});
  }
  h->q_cv.notify_one();
  return MOE_OK;
}
