// Shared expert-slot cache: the per-layer decision kernel, the fused fill
// copy, and the host side of the cache handle.
//
// [FT] section "Device-side 缓存控制": one kernel per MoE layer deduplicates
// the routed experts, classifies them against the residency table, derives
// the fill count q from the bandwidth ratio, selects victim slots and
// rewrites each logical route to a physical slot or a "host" flag; victim
// discovery is one scan that yields the K least recently used candidates, of
// which the first q are consumed; control lives in fixed-shape buffers with
// device-resident valid counts, and one fixed-shape launch applies the
// source/destination list to every bank.
// [FT] section "语义感知专家缓存": one LRU residency space shared by all MoE
// layers; hits refresh recency, fills admit, eviction takes the least
// recently needed.  [FT] section "q* 策略": q* = m B_P / B_H rounded, at least
// one fill; the host set leaves residency untouched.
//
// Readings where the pages are silent: ascending-id dedup; per-call tick with
// in-call rank (hits then fills, ascending id); hit slots are never victims;
// victims ordered by (stamp, slot), empty slots (stamp 0) first; fill i goes
// to victim i.
#include <stdarg.h>
#include <string.h>

#include <vector>

#include "common.h"

namespace moe {

// ---------------------------------------------------------------- errors
static thread_local char g_err[512];
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = 0; }

moe_status check_slots(const moe_slots* s) {
  if (!s) MOE_FAIL(MOE_ERR_ARG, "slots is NULL");
  if (s->wtype != MOE_W_BF16 && s->wtype != MOE_W_FP8_B128) MOE_FAIL(MOE_ERR_ARG, "bad wtype %d", s->wtype);
  if (s->H <= 0 || s->I <= 0 || s->n_slots <= 0) MOE_FAIL(MOE_ERR_SHAPE, "bad slot shape");
  int q = s->wtype == MOE_W_FP8_B128 ? 128 : 32;
  if (s->H % q || s->I % q) MOE_FAIL(MOE_ERR_SHAPE, "H and I must be multiples of %d (H=%d I=%d)", q, s->H, s->I);
  if (!s->w_gate || !s->w_up || !s->w_down) MOE_FAIL(MOE_ERR_ARG, "null weight bank");
  if (!aligned16(s->w_gate) || !aligned16(s->w_up) || !aligned16(s->w_down))
    MOE_FAIL(MOE_ERR_ARG, "weight banks must be 16-byte aligned");
  if (s->wtype == MOE_W_FP8_B128) {
    if (!s->s_gate || !s->s_up || !s->s_down) MOE_FAIL(MOE_ERR_ARG, "null scale bank");
    if (!aligned16(s->s_gate) || !aligned16(s->s_up) || !aligned16(s->s_down))
      MOE_FAIL(MOE_ERR_ARG, "scale banks must be 16-byte aligned");
  }
  return MOE_OK;
}

constexpr int kThreads = 1024;        // decision kernel: one workgroup
constexpr int kUMax = 1024;           // T_max * k <= 1024
constexpr int kEMax = 4096;
constexpr int kCMax = 16384;
constexpr uint64_t kSent = ~0ull;
constexpr int kSmallQ = 32;           // tournament selection up to this many victims

enum { ERR_BAD_ID = 1, ERR_TICK = 2, ERR_TABLE = 3 };

struct CacheDev {
  int32_t* id_slot;     // [L*E]
  int32_t* slot_id;     // [C]   -1 empty, -2 reserved, else logical id
  uint64_t* stamp;      // [C]
  uint64_t* tick;       // [1]
  uint64_t* counters;   // [8]
  int32_t* error;       // [1]
  int32_t* seed_list;   // [2*C + 8] scratch for seeding: ids, slots, counts
  const uint64_t* host_tab;  // [nb][L*E] device-visible host pointers
  int L, E, C;
  uint32_t bp, bh;
};

struct StepArgs {
  const int32_t* ids;
  int layer, T, k, U_max;
  moe_step_out out;
};

// ---------------------------------------------------------------- device utils
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o < v ? o : v;
  }
  return v;
}

// Block-wide stable compaction step: every thread offers `flag`; returns the
// thread's output position (valid if flag) and writes the total to *total.
// `wsum` is LDS scratch of 16 ints.  Contains two barriers.
__device__ int block_compact(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t b = __ballot(flag);
  int pre = __popcll(b & lanemask_lt());
  if (lane == 0) wsum[wv] = __popcll(b);
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < kThreads / 64; ++i) {
    int c = wsum[i];
    base += (i < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + pre;
}

// ---------------------------------------------------------------- decision kernel
__global__ __launch_bounds__(kThreads) void cache_decide_kernel(CacheDev cd, StepArgs a) {
  extern __shared__ uint64_t keys[];          // [C]
  __shared__ uint32_t bm[kEMax / 32];
  __shared__ int uniq[kUMax];                 // local expert index, ascending
  __shared__ int uslot[kUMax];                // slot of uniq[i] after the step, -1 = host
  __shared__ int hit_list[kUMax];             // positions into uniq
  __shared__ int miss_list[kUMax];
  __shared__ int victims[kUMax];
  __shared__ uint64_t cand[16 * kSmallQ];
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ int sh[8];                       // 0 u, 1 h, 2 m, 3 q*, 4 q, 5 n_cand
  __shared__ uint64_t sh64[4];                // 0 tick, 1 radix prefix, 2 key OR

  const int tid = threadIdx.x;
  const int E = cd.E, C = cd.C, layer = a.layer;
  const int P = a.T * a.k;
  const int lbase = layer * E;

  for (int i = tid; i < (E + 31) / 32; i += kThreads) bm[i] = 0;
  if (tid == 0) {
    sh64[0] = *cd.tick;
    sh64[2] = 0;
  }
  __syncthreads();

  // 1. dedup: bitmap of the routed experts of this layer
  for (int p = tid; p < P; p += kThreads) {
    int e = a.ids[p];
    if (e < 0 || e >= E)
      atomicOr(cd.error, 1 << ERR_BAD_ID);
    else
      atomicOr(&bm[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  int u = 0;
  for (int base = 0; base < E; base += kThreads) {
    int e = base + tid;
    bool f = e < E && ((bm[e >> 5] >> (e & 31)) & 1u);
    int tot;
    int pos = block_compact(f, wsum, &tot);
    if (f) uniq[u + pos] = e;
    u += tot;
  }
  __syncthreads();   // uniq[] is read below by threads of other waves

  // 2. classify against the residency table
  bool is_hit = false;
  int my_slot = -1;
  if (tid < u) {
    my_slot = cd.id_slot[lbase + uniq[tid]];
    if (my_slot >= C) {
      atomicOr(cd.error, 1 << ERR_TABLE);
      my_slot = -1;
    }
    is_hit = my_slot >= 0;
  }
  int h, m;
  int hp = block_compact(tid < u && is_hit, wsum, &h);
  int mp = block_compact(tid < u && !is_hit, wsum, &m);
  if (tid < u) {
    if (is_hit) {
      hit_list[hp] = tid;
      uslot[tid] = my_slot;
    } else {
      miss_list[mp] = tid;
      uslot[tid] = -1;
    }
  }
  __syncthreads();   // hit_list / miss_list / uslot are read by other waves

  // 3. q* = clamp(round(m bp / bh), 1, m)
  int qs = 0;
  if (m > 0) {
    uint64_t q0 = (2ull * (uint64_t)m * cd.bp + cd.bh) / (2ull * cd.bh);
    qs = (int)(q0 < 1 ? 1 : (q0 > (uint64_t)m ? (uint64_t)m : q0));
  }

  // 4. one scan over the slots: keys (stamp << 20 | slot) of the candidates
  int q = 0;
  if (qs > 0) {
    int ncand = 0;
    uint64_t kor = 0;
    for (int s = tid; s < C; s += kThreads) {
      int sid = cd.slot_id[s];
      bool pinned_hit = false;
      if (sid >= 0) {
        int sl = sid - lbase;
        pinned_hit = sl >= 0 && sl < E && ((bm[sl >> 5] >> (sl & 31)) & 1u);
      }
      uint64_t key = kSent;
      if (sid != -2 && !pinned_hit) {
        key = (cd.stamp[s] << 20) | (uint64_t)s;
        ++ncand;
        kor |= key;
      }
      keys[s] = key;
    }
    if (tid == 0) sh[5] = 0;
    __syncthreads();
    atomicAdd(&sh[5], ncand);
    if (kor) atomicOr((unsigned long long*)&sh64[2], (unsigned long long)kor);
    __syncthreads();
    q = qs < sh[5] ? qs : sh[5];

    if (q > 0 && q <= kSmallQ) {
      // tournament: each wave extracts its q smallest keys, then wave 0 merges
      const int lane = tid & 63, wv = tid >> 6;
      for (int r = 0; r < q; ++r) {
        uint64_t best = kSent;
        int bs = -1;
        for (int s = tid; s < C; s += kThreads) {
          uint64_t kk = keys[s];
          if (kk < best) {
            best = kk;
            bs = s;
          }
        }
        uint64_t wmin = wave_min_u64(best);
        if (wmin != kSent && best == wmin) keys[bs] = kSent;   // keys are unique
        if (lane == 0) cand[wv * kSmallQ + r] = wmin;
      }
      __syncthreads();
      if (wv == 0) {
        const int NC = 16 * q;
        for (int r = 0; r < q; ++r) {
          uint64_t best = kSent;
          int bi = -1;
          for (int i = lane; i < NC; i += 64) {
            int idx = (i / q) * kSmallQ + (i % q);
            uint64_t kk = cand[idx];
            if (kk < best) {
              best = kk;
              bi = idx;
            }
          }
          uint64_t wmin = wave_min_u64(best);
          if (wmin != kSent && best == wmin) cand[bi] = kSent;
          if (lane == 0) victims[r] = (int)(wmin & 0xFFFFFull);
        }
      }
      __syncthreads();
    } else if (q > 0) {
      // MSD radix select of the q-th smallest key, 8 bits per pass
      uint64_t kor_all = sh64[2];
      int top = 63 - __builtin_clzll(kor_all | 1ull);
      int start = (top / 8) * 8;
      if (tid == 0) {
        sh64[1] = 0;
        sh[6] = q;
      }
      __syncthreads();
      for (int shift = start; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
        __syncthreads();
        const uint64_t prefix = sh64[1];
        const uint64_t himask = (shift + 8 >= 64) ? 0ull : (~0ull << (shift + 8));
        for (int s = tid; s < C; s += kThreads) {
          uint64_t kk = keys[s];
          if (kk != kSent && (kk & himask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1);
        }
        __syncthreads();
        if (tid < 64) {
          // wave 0: inclusive scan over 256 bins, 4 per lane
          int c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
          int lsum = c0 + c1 + c2 + c3;
          int incl = lsum;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            int o = __shfl_up(incl, d, 64);
            if (tid >= d) incl += o;
          }
          int excl = incl - lsum;
          int need = sh[6];
          if (excl < need && incl >= need) {
            int c[4] = {c0, c1, c2, c3};
            int cum = excl, dgt = 0;
            for (int j = 0; j < 4; ++j) {
              if (cum + c[j] >= need) {
                dgt = 4 * tid + j;
                break;
              }
              cum += c[j];
            }
            sh[6] = need - cum;
            sh64[1] = prefix | ((uint64_t)dgt << shift);
          }
        }
        __syncthreads();
      }
      const uint64_t thr = sh64[1];   // exactly the q-th smallest key
      if (tid == 0) sh[7] = 0;
      __syncthreads();
      for (int s = tid; s < C; s += kThreads) {
        uint64_t kk = keys[s];
        if (kk != kSent && kk <= thr) {
          int pos = atomicAdd(&sh[7], 1);   // exactly q keys are <= thr
          if (pos < q) victims[pos] = s;
        }
      }
      __syncthreads();
      // order the q victims by key: rank sort
      int myv = -1;
      int myrank = 0;
      if (tid < q) {
        myv = victims[tid];
        uint64_t mk = keys[myv];
        for (int j = 0; j < q; ++j) myrank += keys[victims[j]] < mk;
      }
      __syncthreads();
      if (tid < q) victims[myrank] = myv;
      __syncthreads();
    }
  }

  // 5. table update: fill i -> victim i
  const uint64_t tick = sh64[0];
  if (tid < q) {
    int v = victims[tid];
    int f = lbase + uniq[miss_list[tid]];
    int old = cd.slot_id[v];
    if (old >= 0) cd.id_slot[old] = -1;
    cd.slot_id[v] = f;
    cd.id_slot[f] = v;
    uslot[miss_list[tid]] = v;
    a.out.fill_id[tid] = f;
    a.out.fill_slot[tid] = v;
    a.out.fill_evicted[tid] = old;
    cd.stamp[v] = (tick << 16) | (uint64_t)(1 + h + tid);
  }
  if (tid < h) cd.stamp[uslot[hit_list[tid]]] = (tick << 16) | (uint64_t)(1 + tid);
  __syncthreads();

  // 6. outputs: rewrite picks, lists, counts
  for (int p = tid; p < P; p += kThreads) {
    int e = a.ids[p];
    int slot = -1;
    if (e >= 0 && e < E) {
      int lo = 0, hi = u - 1;
      while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (uniq[mid] < e) lo = mid + 1; else hi = mid;
      }
      slot = uslot[lo];
    }
    a.out.pick_slot[p] = slot;
  }
  if (tid < a.U_max) {
    a.out.uniq[tid] = tid < u ? lbase + uniq[tid] : -1;
    a.out.is_hit[tid] = tid < u ? (is_hit ? 1 : 0) : -1;
  }
  for (int i = tid; i < a.U_max; i += kThreads) {
    if (i >= q) {
      a.out.fill_id[i] = -1;
      a.out.fill_slot[i] = -1;
      a.out.fill_evicted[i] = -1;
    }
    int hi = i + q;
    a.out.host_id[i] = (hi < m) ? lbase + uniq[miss_list[hi]] : -1;
  }
  if (tid == 0) {
    int* cnt = a.out.counts;
    cnt[MOE_CNT_UNIQ] = u;
    cnt[MOE_CNT_HIT] = h;
    cnt[MOE_CNT_MISS] = m;
    cnt[MOE_CNT_QSTAR] = qs;
    cnt[MOE_CNT_FILL] = q;
    cnt[MOE_CNT_HOST] = m - q;
    cnt[6] = layer;
    cnt[7] = 0;
    *cd.tick = tick + 1;
    if (tick + 1 >= (1ull << 28)) atomicOr(cd.error, 1 << ERR_TICK);
    cd.counters[0] += 1;
    cd.counters[1] += (uint64_t)u;
    cd.counters[2] += (uint64_t)h;
    cd.counters[3] += (uint64_t)m;
    cd.counters[4] += (uint64_t)q;
    cd.counters[5] += (uint64_t)(m - q);
  }
}

// ---------------------------------------------------------------- fused fill copy
struct FillArgs {
  const int32_t* fill_id;
  const int32_t* fill_slot;
  const int32_t* n_fill;        // device count
  const uint64_t* host_tab;     // [nb][LE]
  int LE, C, nb;
  char* dst[6];
  uint64_t bytes[6];
};

__global__ __launch_bounds__(256) void cache_fill_kernel(FillArgs a) {
  const int n = *a.n_fill;
  const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t gsz = (size_t)gridDim.x * blockDim.x;
  for (int f = 0; f < n; ++f) {
    const int id = a.fill_id[f];
    const int slot = a.fill_slot[f];
    if (id < 0 || id >= a.LE || slot < 0 || slot >= a.C) continue;
    for (int b = 0; b < a.nb; ++b) {
      const char* src = reinterpret_cast<const char*>(a.host_tab[(size_t)b * a.LE + id]);
      char* dst = a.dst[b] + (size_t)slot * a.bytes[b];
      if ((a.bytes[b] & 15) == 0) {
        const size_t n16 = a.bytes[b] >> 4;
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
        u32x4* d4 = reinterpret_cast<u32x4*>(dst);
        size_t i = gtid;
        for (; i + 3 * gsz < n16; i += 4 * gsz) {
          u32x4 v0 = __builtin_nontemporal_load(s4 + i);
          u32x4 v1 = __builtin_nontemporal_load(s4 + i + gsz);
          u32x4 v2 = __builtin_nontemporal_load(s4 + i + 2 * gsz);
          u32x4 v3 = __builtin_nontemporal_load(s4 + i + 3 * gsz);
          d4[i] = v0;
          d4[i + gsz] = v1;
          d4[i + 2 * gsz] = v2;
          d4[i + 3 * gsz] = v3;
        }
        for (; i < n16; i += gsz) d4[i] = __builtin_nontemporal_load(s4 + i);
      } else {
        const size_t n4 = a.bytes[b] >> 2;
        const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
        uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
        for (size_t i = gtid; i < n4; i += gsz) d1[i] = s1[i];
      }
    }
  }
}

// ---------------------------------------------------------------- init / seed kernels
__global__ void cache_reset_kernel(CacheDev cd, int keep_reserved) {
  const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t gsz = (size_t)gridDim.x * blockDim.x;
  for (size_t i = gtid; i < (size_t)cd.L * cd.E; i += gsz) cd.id_slot[i] = -1;
  for (size_t s = gtid; s < (size_t)cd.C; s += gsz) {
    if (!(keep_reserved && cd.slot_id[s] == -2)) cd.slot_id[s] = -1;
    cd.stamp[s] = 0;
  }
  if (gtid == 0) {
    *cd.tick = 1;
    for (int i = 0; i < 8; ++i) cd.counters[i] = 0;
    *cd.error = 0;
  }
}

// after reset: slot i <- seed id i (single thread per entry; ids distinct)
__global__ void cache_seed_kernel(CacheDev cd, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    int id = cd.seed_list[i];
    if (id < 0 || id >= cd.L * cd.E || cd.slot_id[i] == -2) {
      atomicOr(cd.error, 1 << ERR_BAD_ID);
      cd.seed_list[cd.C + i] = -1;       // the fill copy skips this entry
      return;
    }
    cd.slot_id[i] = id;
    cd.id_slot[id] = i;
    cd.stamp[i] = 1 + (uint64_t)i;
    cd.seed_list[cd.C + i] = i;
  }
  if (i == 0) cd.seed_list[2 * cd.C] = n;
}

// reserve (mark=-2) or release (mark=-1) slots [first, first+n)
__global__ void cache_mark_kernel(CacheDev cd, int first, int n, int mark) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    int s = first + i;
    int old = cd.slot_id[s];
    if (old >= 0) cd.id_slot[old] = -1;
    cd.slot_id[s] = mark;
    cd.stamp[s] = 0;
  }
}

}  // namespace moe

// ================================================================ host side
struct moe_cache {
  moe_cache_cfg cfg;
  moe_slots slots;
  moe::CacheDev dev;
  int nb;
  moe::BankBytes bb;
  std::vector<const void*> host_ptr[6];   // host-visible pool pointers (for DMA)
  int lds_bytes;
  int U_max;
  bool has_prefill;
};

using namespace moe;

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct WsLayout {
  size_t id_slot, slot_id, stamp, tick, counters, error, seed, host_tab, total;
};
static WsLayout ws_layout(const moe_cache_cfg* c, int nb) {
  WsLayout w{};
  size_t off = 0;
  size_t LE = (size_t)c->L * c->E;
  w.id_slot = off; off = align_up(off + 4 * LE, 256);
  w.slot_id = off; off = align_up(off + 4 * (size_t)c->C, 256);
  w.stamp = off; off = align_up(off + 8 * (size_t)c->C, 256);
  w.tick = off; off = align_up(off + 8, 256);
  w.counters = off; off = align_up(off + 64, 256);
  w.error = off; off = align_up(off + 4, 256);
  w.seed = off; off = align_up(off + 4 * (2 * (size_t)c->C + 8), 256);
  w.host_tab = off; off = align_up(off + 8 * (size_t)nb * LE, 256);
  w.total = off;
  return w;
}

static moe_status check_cfg(const moe_cache_cfg* c) {
  if (!c) MOE_FAIL(MOE_ERR_ARG, "cfg is NULL");
  if (c->L < 1 || c->E < 1 || c->E > kEMax || c->k < 1 || c->k > c->E || c->T_max < 1 ||
      (int64_t)c->T_max * c->k > kUMax || c->C < 1 || c->C > kCMax)
    MOE_FAIL(MOE_ERR_SHAPE, "cache cfg out of range (L=%d E=%d k=%d T_max=%d C=%d; E<=%d, T_max*k<=%d, C<=%d)",
             c->L, c->E, c->k, c->T_max, c->C, kEMax, kUMax, kCMax);
  if ((int64_t)c->L * c->E > (1 << 30)) MOE_FAIL(MOE_ERR_SHAPE, "L*E too large");
  if (c->bh == 0) MOE_FAIL(MOE_ERR_ARG, "bh must be > 0");
  return MOE_OK;
}

extern "C" const char* moe_last_error(void) { return moe::g_err; }

extern "C" moe_status moe_cache_workspace_bytes(const moe_cache_cfg* cfg, size_t* bytes) {
  clear_error();
  moe_status st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) MOE_FAIL(MOE_ERR_ARG, "bytes is NULL");
  *bytes = ws_layout(cfg, 6).total;
  return MOE_OK;
}

extern "C" moe_status moe_cache_create(const moe_cache_cfg* cfg, const moe_slots* slots,
                                       const moe_host_pool* host, void* dev_ws, size_t ws_bytes,
                                       hipStream_t stream, moe_cache_t* out) {
  clear_error();
  moe_status st = check_cfg(cfg);
  if (st) return st;
  if (!out || !host || !dev_ws) MOE_FAIL(MOE_ERR_ARG, "null argument");
  *out = nullptr;
  if ((st = check_slots(slots))) return st;
  if (slots->n_slots != cfg->C) MOE_FAIL(MOE_ERR_SHAPE, "slots->n_slots (%d) != cfg->C (%d)", slots->n_slots, cfg->C);
  if (reinterpret_cast<uintptr_t>(dev_ws) & 255) MOE_FAIL(MOE_ERR_ARG, "workspace must be 256-byte aligned");
  const int nb = slots->wtype == MOE_W_FP8_B128 ? 6 : 3;
  WsLayout L = ws_layout(cfg, 6);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);

  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  int lds_max = 0;
  MOE_HIP(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  const int lds_static = 32 * 1024;   // bound on the kernel's static LDS (about 26 KB)
  const int lds_dyn = 8 * cfg->C;
  if (lds_dyn + lds_static > lds_max)
    MOE_FAIL(MOE_ERR_SHAPE, "C=%d needs %d B of LDS; device allows %d", cfg->C, lds_dyn + lds_static, lds_max);

  const void* const* tabs[6] = {host->w_gate, host->w_up, host->w_down,
                                (const void* const*)host->s_gate, (const void* const*)host->s_up,
                                (const void* const*)host->s_down};
  const size_t LE = (size_t)cfg->L * cfg->E;
  std::vector<uint64_t> htab((size_t)nb * LE);
  moe_cache* c = new moe_cache();
  for (int b = 0; b < nb; ++b) {
    if (!tabs[b]) {
      delete c;
      MOE_FAIL(MOE_ERR_ARG, "host pool table %d is NULL", b);
    }
    c->host_ptr[b].resize(LE);
    const void* last_base = nullptr;
    void* last_dev = nullptr;
    size_t last_size = 0;
    for (size_t i = 0; i < LE; ++i) {
      const void* p = tabs[b][i];
      if (!p) {
        delete c;
        MOE_FAIL(MOE_ERR_ARG, "host pool pointer (bank %d, id %zu) is NULL", b, i);
      }
      c->host_ptr[b][i] = p;
      // resolve the device-visible address; reuse the last allocation's range
      const char* pc = (const char*)p;
      if (last_base && pc >= (const char*)last_base && pc < (const char*)last_base + last_size) {
        htab[b * LE + i] = (uint64_t)((char*)last_dev + (pc - (const char*)last_base));
        continue;
      }
      hipPointerAttribute_t attr;
      hipError_t e = hipPointerGetAttributes(&attr, p);
      if (e != hipSuccess || attr.type != hipMemoryTypeHost || !attr.devicePointer) {
        (void)hipGetLastError();
        delete c;
        MOE_FAIL(MOE_ERR_NOT_PINNED, "host pool pointer (bank %d, id %zu) is not pinned host memory", b, i);
      }
      htab[b * LE + i] = (uint64_t)attr.devicePointer;
      void* abase = nullptr;
      size_t asize = 0;
      if (hipMemGetAddressRange((hipDeviceptr_t*)&abase, &asize, (hipDeviceptr_t)attr.devicePointer) == hipSuccess &&
          abase) {
        last_dev = abase;
        last_base = pc - ((char*)attr.devicePointer - (char*)abase);
        last_size = asize;
      } else {
        (void)hipGetLastError();
        last_base = nullptr;
      }
    }
  }

  char* ws = (char*)dev_ws;
  c->cfg = *cfg;
  c->slots = *slots;
  c->nb = nb;
  c->bb = bank_bytes(slots->wtype, slots->H, slots->I);
  c->lds_bytes = lds_dyn;
  c->U_max = cfg->T_max * cfg->k < cfg->E ? cfg->T_max * cfg->k : cfg->E;
  c->has_prefill = false;
  CacheDev& d = c->dev;
  d.id_slot = (int32_t*)(ws + L.id_slot);
  d.slot_id = (int32_t*)(ws + L.slot_id);
  d.stamp = (uint64_t*)(ws + L.stamp);
  d.tick = (uint64_t*)(ws + L.tick);
  d.counters = (uint64_t*)(ws + L.counters);
  d.error = (int32_t*)(ws + L.error);
  d.seed_list = (int32_t*)(ws + L.seed);
  d.host_tab = (const uint64_t*)(ws + L.host_tab);
  d.L = cfg->L;
  d.E = cfg->E;
  d.C = cfg->C;
  d.bp = cfg->bp;
  d.bh = cfg->bh;

  hipError_t e = hipFuncSetAttribute((const void*)cache_decide_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_dyn);
  if (e != hipSuccess) {
    delete c;
    MOE_FAIL(MOE_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  e = hipMemcpyAsync((void*)d.host_tab, htab.data(), htab.size() * 8, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    cache_reset_kernel<<<64, 256, 0, stream>>>(d, 0);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    delete c;
    MOE_FAIL(MOE_ERR_HIP, "cache init: %s", hipGetErrorString(e));
  }
  *out = c;
  return MOE_OK;
}

static moe_status launch_fill(moe_cache* c, const int32_t* fill_id, const int32_t* fill_slot,
                              const int32_t* n_fill, hipStream_t stream) {
  FillArgs f{};
  f.fill_id = fill_id;
  f.fill_slot = fill_slot;
  f.n_fill = n_fill;
  f.host_tab = c->dev.host_tab;
  f.LE = c->cfg.L * c->cfg.E;
  f.C = c->cfg.C;
  f.nb = c->nb;
  void* bases[6] = {c->slots.w_gate, c->slots.w_up, c->slots.w_down,
                    c->slots.s_gate, c->slots.s_up, c->slots.s_down};
  for (int b = 0; b < c->nb; ++b) {
    f.dst[b] = (char*)bases[b];
    f.bytes[b] = c->bb.b[b];
  }
  cache_fill_kernel<<<512, 256, 0, stream>>>(f);
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_cache_seed(moe_cache_t c, const int32_t* host_ids, int32_t n, uint32_t flags,
                                     hipStream_t stream) {
  clear_error();
  if (!c) MOE_FAIL(MOE_ERR_ARG, "cache is NULL");
  if (n < 0 || n > c->cfg.C) MOE_FAIL(MOE_ERR_SHAPE, "seed count %d outside [0, C=%d]", n, c->cfg.C);
  if (n > 0 && !host_ids) MOE_FAIL(MOE_ERR_ARG, "host_ids is NULL");
  if (c->has_prefill) MOE_FAIL(MOE_ERR_STATE, "cannot seed while a prefill pool holds slots");
  {
    std::vector<char> seen((size_t)c->cfg.L * c->cfg.E, 0);
    for (int i = 0; i < n; ++i) {
      int id = host_ids[i];
      if (id < 0 || (size_t)id >= seen.size()) MOE_FAIL(MOE_ERR_ARG, "seed id %d out of range", id);
      if (seen[id]) MOE_FAIL(MOE_ERR_ARG, "seed id %d repeated", id);
      seen[id] = 1;
    }
  }
  CacheDev d = c->dev;
  cache_reset_kernel<<<64, 256, 0, stream>>>(d, 1);
  MOE_LAUNCHED();
  if (n > 0) MOE_HIP(hipMemcpyAsync(d.seed_list, host_ids, 4 * (size_t)n, hipMemcpyHostToDevice, stream));
  cache_seed_kernel<<<(n + 255) / 256 + 1, 256, 0, stream>>>(d, n);
  MOE_LAUNCHED();
  if (!(flags & MOE_STEP_NO_COPY) && n > 0) {
    moe_status st = launch_fill(c, d.seed_list, d.seed_list + c->cfg.C, d.seed_list + 2 * c->cfg.C, stream);
    if (st) return st;
  }
  MOE_HIP(hipStreamSynchronize(stream));
  return MOE_OK;
}

extern "C" moe_status moe_cache_step(moe_cache_t c, int32_t layer, const int32_t* ids, int32_t T, uint32_t flags,
                                     const moe_step_out* out, hipStream_t stream) {
  clear_error();
  if (!c || !ids || !out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (layer < 0 || layer >= c->cfg.L) MOE_FAIL(MOE_ERR_SHAPE, "layer %d outside [0, %d)", layer, c->cfg.L);
  if (T < 1 || T > c->cfg.T_max) MOE_FAIL(MOE_ERR_SHAPE, "T=%d outside [1, T_max=%d]", T, c->cfg.T_max);
  if (!out->pick_slot || !out->uniq || !out->is_hit || !out->fill_id || !out->fill_slot || !out->fill_evicted ||
      !out->host_id || !out->counts)
    MOE_FAIL(MOE_ERR_ARG, "a moe_step_out buffer is NULL");
  StepArgs a;
  a.ids = ids;
  a.layer = layer;
  a.T = T;
  a.k = c->cfg.k;
  a.U_max = c->U_max;
  a.out = *out;
  cache_decide_kernel<<<1, kThreads, c->lds_bytes, stream>>>(c->dev, a);
  MOE_LAUNCHED();
  if (!(flags & MOE_STEP_NO_COPY))
    return launch_fill(c, out->fill_id, out->fill_slot, out->counts + MOE_CNT_FILL, stream);
  return MOE_OK;
}

extern "C" moe_status moe_cache_fill(moe_cache_t c, const moe_step_out* out, hipStream_t stream) {
  clear_error();
  if (!c || !out || !out->fill_id || !out->fill_slot || !out->counts) MOE_FAIL(MOE_ERR_ARG, "null argument");
  return launch_fill(c, out->fill_id, out->fill_slot, out->counts + MOE_CNT_FILL, stream);
}

extern "C" moe_status moe_cache_read_state(moe_cache_t c, int32_t* slot_id, uint64_t* stamp, int32_t* id_slot,
                                           uint64_t* tick, uint64_t* counters, hipStream_t stream) {
  clear_error();
  if (!c) MOE_FAIL(MOE_ERR_ARG, "cache is NULL");
  const CacheDev& d = c->dev;
  if (slot_id) MOE_HIP(hipMemcpyAsync(slot_id, d.slot_id, 4 * (size_t)d.C, hipMemcpyDeviceToHost, stream));
  if (stamp) MOE_HIP(hipMemcpyAsync(stamp, d.stamp, 8 * (size_t)d.C, hipMemcpyDeviceToHost, stream));
  if (id_slot) MOE_HIP(hipMemcpyAsync(id_slot, d.id_slot, 4 * (size_t)d.L * d.E, hipMemcpyDeviceToHost, stream));
  if (tick) MOE_HIP(hipMemcpyAsync(tick, d.tick, 8, hipMemcpyDeviceToHost, stream));
  if (counters) MOE_HIP(hipMemcpyAsync(counters, d.counters, 48, hipMemcpyDeviceToHost, stream));
  MOE_HIP(hipStreamSynchronize(stream));
  return MOE_OK;
}

extern "C" moe_status moe_cache_error(moe_cache_t c, int32_t* code, hipStream_t stream) {
  clear_error();
  if (!c || !code) MOE_FAIL(MOE_ERR_ARG, "null argument");
  MOE_HIP(hipMemcpyAsync(code, c->dev.error, 4, hipMemcpyDeviceToHost, stream));
  MOE_HIP(hipStreamSynchronize(stream));
  int32_t zero = 0;
  MOE_HIP(hipMemcpyAsync(c->dev.error, &zero, 4, hipMemcpyHostToDevice, stream));
  MOE_HIP(hipStreamSynchronize(stream));
  return MOE_OK;
}

extern "C" moe_status moe_cache_destroy(moe_cache_t c) {
  clear_error();
  if (!c) return MOE_OK;
  if (c->has_prefill) MOE_FAIL(MOE_ERR_STATE, "destroy the prefill pool first");
  delete c;
  return MOE_OK;
}

// ================================================================ prefill double buffer
struct moe_prefill {
  moe_cache* c;
  int first;               // first reserved slot
  int E;
  int buf_layer[2];
  hipEvent_t ready[2], released[2];
  bool released_recorded[2];
};

extern "C" moe_status moe_prefill_create(moe_cache_t c, moe_prefill_t* out) {
  clear_error();
  if (!c || !out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  *out = nullptr;
  if (c->has_prefill) MOE_FAIL(MOE_ERR_STATE, "the cache already has a prefill pool");
  const int E = c->cfg.E;
  if (2 * E > c->cfg.C) MOE_FAIL(MOE_ERR_NO_SPACE, "two full-layer buffers need %d slots; the pool has %d", 2 * E, c->cfg.C);
  moe_prefill* p = new moe_prefill();
  p->c = c;
  p->E = E;
  p->first = c->cfg.C - 2 * E;
  for (int b = 0; b < 2; ++b) {
    p->buf_layer[b] = -1;
    p->released_recorded[b] = false;
    hipError_t e1 = hipEventCreateWithFlags(&p->ready[b], hipEventDisableTiming);
    hipError_t e2 = hipEventCreateWithFlags(&p->released[b], hipEventDisableTiming);
    if (e1 != hipSuccess || e2 != hipSuccess) {
      delete p;
      MOE_FAIL(MOE_ERR_HIP, "hipEventCreate failed");
    }
  }
  cache_mark_kernel<<<(2 * E + 255) / 256, 256, 0, 0>>>(c->dev, p->first, 2 * E, -2);
  MOE_LAUNCHED();
  MOE_HIP(hipDeviceSynchronize());
  c->has_prefill = true;
  *out = p;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_prefetch(moe_prefill_t p, int32_t layer, hipStream_t copy_stream) {
  clear_error();
  if (!p) MOE_FAIL(MOE_ERR_ARG, "pool is NULL");
  moe_cache* c = p->c;
  if (layer < 0 || layer >= c->cfg.L) MOE_FAIL(MOE_ERR_SHAPE, "layer %d outside [0, %d)", layer, c->cfg.L);
  const int b = layer & 1;
  if (p->released_recorded[b]) MOE_HIP(hipStreamWaitEvent(copy_stream, p->released[b], 0));
  const int E = p->E;
  const int slot0 = p->first + b * E;
  void* bases[6] = {c->slots.w_gate, c->slots.w_up, c->slots.w_down,
                    c->slots.s_gate, c->slots.s_up, c->slots.s_down};
  for (int k = 0; k < c->nb; ++k) {
    const size_t sz = c->bb.b[k];
    char* dst = (char*)bases[k] + (size_t)slot0 * sz;
    const std::vector<const void*>& hp = c->host_ptr[k];
    int e = 0;
    while (e < E) {
      // coalesce runs of experts whose host bytes are contiguous
      const char* src = (const char*)hp[(size_t)layer * E + e];
      int run = 1;
      while (e + run < E && (const char*)hp[(size_t)layer * E + e + run] == src + (size_t)run * sz) ++run;
      MOE_HIP(hipMemcpyAsync(dst + (size_t)e * sz, src, (size_t)run * sz, hipMemcpyHostToDevice, copy_stream));
      e += run;
    }
  }
  MOE_HIP(hipEventRecord(p->ready[b], copy_stream));
  p->buf_layer[b] = layer;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_acquire(moe_prefill_t p, int32_t layer, hipStream_t compute, moe_slots* view) {
  clear_error();
  if (!p || !view) MOE_FAIL(MOE_ERR_ARG, "null argument");
  const int b = layer & 1;
  if (layer < 0 || p->buf_layer[b] != layer)
    MOE_FAIL(MOE_ERR_STATE, "layer %d was not prefetched into buffer %d", layer, b);
  MOE_HIP(hipStreamWaitEvent(compute, p->ready[b], 0));
  moe_cache* c = p->c;
  const int slot0 = p->first + b * p->E;
  moe_slots v = c->slots;
  v.n_slots = p->E;
  v.w_gate = (char*)c->slots.w_gate + (size_t)slot0 * c->bb.b[0];
  v.w_up = (char*)c->slots.w_up + (size_t)slot0 * c->bb.b[1];
  v.w_down = (char*)c->slots.w_down + (size_t)slot0 * c->bb.b[2];
  if (c->nb == 6) {
    v.s_gate = (float*)((char*)c->slots.s_gate + (size_t)slot0 * c->bb.b[3]);
    v.s_up = (float*)((char*)c->slots.s_up + (size_t)slot0 * c->bb.b[4]);
    v.s_down = (float*)((char*)c->slots.s_down + (size_t)slot0 * c->bb.b[5]);
  }
  *view = v;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_release(moe_prefill_t p, int32_t layer, hipStream_t compute) {
  clear_error();
  if (!p) MOE_FAIL(MOE_ERR_ARG, "pool is NULL");
  const int b = layer & 1;
  if (layer < 0 || p->buf_layer[b] != layer) MOE_FAIL(MOE_ERR_STATE, "layer %d does not own buffer %d", layer, b);
  MOE_HIP(hipEventRecord(p->released[b], compute));
  p->released_recorded[b] = true;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_destroy(moe_prefill_t p, hipStream_t stream) {
  clear_error();
  if (!p) return MOE_OK;
  moe_cache* c = p->c;
  MOE_HIP(hipDeviceSynchronize());
  cache_mark_kernel<<<(2 * p->E + 255) / 256, 256, 0, stream>>>(c->dev, p->first, 2 * p->E, -1);
  MOE_LAUNCHED();
  MOE_HIP(hipStreamSynchronize(stream));
  for (int b = 0; b < 2; ++b) {
    (void)hipEventDestroy(p->ready[b]);
    (void)hipEventDestroy(p->released[b]);
  }
  c->has_prefill = false;
  delete p;
  return MOE_OK;
}
