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

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

#include <chrono>
#include <cmath>
#include <functional>

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
  if (s->I % 8) MOE_FAIL(MOE_ERR_SHAPE, "I must be a multiple of 8");
  if (!s->w_gate_up || !s->w_down) MOE_FAIL(MOE_ERR_ARG, "null weight bank");
  if (!aligned16(s->w_gate_up) || !aligned16(s->w_down))
    MOE_FAIL(MOE_ERR_ARG, "weight banks must be 16-byte aligned");
  if (s->wtype == MOE_W_FP8_B128) {
    if (!s->s_gate || !s->s_up || !s->s_down) MOE_FAIL(MOE_ERR_ARG, "null scale bank");
    if (!aligned16(s->s_gate) || !aligned16(s->s_up) || !aligned16(s->s_down))
      MOE_FAIL(MOE_ERR_ARG, "scale banks must be 16-byte aligned");
  }
  return MOE_OK;
}

constexpr int kDT = 1024;             // decision kernel: one workgroup of 16 waves
constexpr int kDW = kDT / 64;
constexpr int kUMax = 1024;           // T_max * k <= 1024
static_assert(kUMax == kDT, "the decision kernel holds one routed pick per thread");
constexpr int kEMax = 4096;
constexpr int kCMax = 16384;

enum { ERR_BAD_ID = 1, ERR_TICK = 2, ERR_TABLE = 3, ERR_LAYER = 4 };

struct CacheDev {
  int32_t* id_slot;     // [L*E]
  int32_t* slot_id;     // [C]   -1 empty, -2 reserved, else logical id
  uint64_t* stamp;      // [C]
  int32_t* order;       // [C]   non-reserved slots in ascending (stamp, slot): the LRU order
  int32_t* n_ord;       // [1]   entries of `order`
  uint64_t* tick;       // [1]
  uint64_t* counters;   // [8]
  int32_t* error;       // [1]
  int32_t* seed_list;   // [2*C + 8] scratch for seeding: ids, slots, counts
  int32_t* set_list;    // [2*kUMax] scratch of on-demand loading: expert set, its picks
  const uint64_t* host_tab;  // [nb][L*E] device-visible host pointers
  int L, E, C;
  uint32_t bp, bh;
};

struct StepArgs {
  const int32_t* ids;     // routed ids [T*k] (input, or written when routing in the kernel)
  const float* logits;    // [T*E] when routing in the kernel
  float* w;               // [T*k] gate weights when routing in the kernel
  const int32_t* d_layer; // device scalar holding the layer, or NULL: `layer` below
  int layer, T, k, U_max;
  int fill_all;           // q* = m (on-demand loading) instead of the bandwidth split
  moe_step_out out;
};

// ---------------------------------------------------------------- device utils
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Staging batch of the decision kernel: 2 words per thread.
constexpr int kStageB = 2048;
static_assert(kStageB % kDT == 0, "whole staging rows");

// Exclusive prefix (for wave wv) and total of the 16 per-wave counts cnt[0..15]
// in LDS: lane l reads cnt[l & 15], four DPP row shifts inside each row of 16
// lanes make the inclusive prefix, and two lane reads pick out the results.
__device__ __forceinline__ void wave_counts_prefix(const int* cnt, int wv, int& excl, int& total) {
  static_assert(kDW == 16, "one count per lane of a DPP row");
  int v = cnt[threadIdx.x & 15];
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  total = __builtin_amdgcn_readlane(v, 15);
  excl = wv ? __builtin_amdgcn_readlane(v, wv - 1) : 0;
}
__host__ __device__ constexpr int round_stage(int n) { return (n + kStageB - 1) / kStageB * kStageB; }

// Dynamic LDS of the decision kernel (sizes rounded up to whole staging
// batches, so the staging writes need no bounds test): slot_id [C] | LRU
// order [C] as 16-bit slot numbers | id_slot row of the layer [E] | hit
// bitmap [ceil(C/32)].
__host__ __device__ inline int decide_lds_bytes(int C, int E) {
  return 6 * round_stage(C) + 4 * round_stage(E) + 4 * ((C + 31) / 32);
}

// ---------------------------------------------------------------- decision kernel
// LRU order array: the slots sorted by (stamp, slot), reserved slots left out.
// Victims are the first q entries that hold no hit of this call, found in one
// ordered scan; the new order is the other entries in place, then the hits
// (rank order), then the filled victims: exactly the (stamp, slot) order after
// the new stamps, since every new stamp exceeds all older ones.
// Every table the decision reads (the order, slot_id, the layer's id_slot
// row, the routed ids) is staged into LDS up front with all loads in flight
// together; the rest of the kernel reads only LDS, so its barriers wait for
// LDS traffic only and its global stores drain in the background.
// One workgroup of 16 waves: with one wave per SIMD the kernel's dependent
// LDS and ballot chains left the SIMDs idle; four waves per SIMD overlap them.
// VPL > 0: the kernel routes first (the router of route_topk_kernel, one
// wave per token, VPL logits per lane) while the table loads are in flight,
// and writes ids and gate weights as well.
template <int VPL>
__global__ __launch_bounds__(kDT) void cache_decide_kernel(CacheDev cd, StepArgs a) {
  extern __shared__ int dyn[];
  __shared__ uint32_t bm[kEMax / 32];          // routed experts of this layer
  // uniq: local expert index, ascending; uslot: slot of uniq[i] when hit,
  // else -1; hit_list, miss_list: positions into uniq; victims.  Before the
  // classification the same memory is the router's per-wave scratch.
  __shared__ __align__(16) int s_lists[5 * kUMax];
  static_assert(5 * kUMax * 4 >= kDW * 96 * 8, "router scratch fits the lists");
  int* const uniq = s_lists;
  int* const uslot = s_lists + kUMax;
  int* const hit_list = s_lists + 2 * kUMax;
  int* const miss_list = s_lists + 3 * kUMax;
  int* const victims = s_lists + 4 * kUMax;
  __shared__ int s_cnt[kEMax / kDT][2][kDW];   // per (row, kind, wave): routed, hit
  __shared__ int s_cc[2][kStageB / kDT][kDW];  // per (chunk parity, row, wave): LRU candidates
  __shared__ int s_pid[VPL > 0 ? kUMax : 1];   // the router's picks

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = cd.E, C = cd.C;
  const int T = a.T, k = a.k, P = T * k;
  constexpr int V = kStageB / kDT, NEM = kEMax / kDT;
  const int Cp = round_stage(C), Ep = round_stage(E);
  int* sl = dyn;                                               // slot_id before the step
  uint16_t* ord = reinterpret_cast<uint16_t*>(dyn + Cp);       // LRU order before the step
  int* row = dyn + Cp + Cp / 2;                                // id_slot[lbase + e]; after step 5 the new slot
  uint32_t* hitbm = reinterpret_cast<uint32_t*>(row + Ep);

  // 0. stage.  The layer scalar is loaded first (a load of 0 bytes when the
  //    layer comes as an argument), then what does not depend on the layer:
  //    the router's logits (or the routed ids) ahead of the tables, so that
  //    routing can run while the table loads are in flight, then the LRU
  //    order and the slot table; the layer's id_slot row is issued as soon
  //    as the layer has arrived.  An invalid layer reads no row and is
  //    handled after the staging (the loads stay unconditional).  Buffer
  //    loads past the end return 0; entries of `order` past n_ord are not
  //    used.  All loads are vector loads, so each wait below is for a
  //    prefix of them in issue order.
  const int layer_ld = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.d_layer, a.d_layer ? 4u : 0u), 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  auto row_of = [&](int t) {
    return make_rsrc(a.logits + (size_t)(t < T ? t : 0) * E, t < T ? 4u * (uint32_t)E : 0u);
  };
  uint32_t kraw[VPL > 0 ? VPL : 1], kc[VPL > 0 ? VPL : 1], ac = 0;
  int pid = 0;
  if constexpr (VPL > 0)
    topk_load<VPL>(row_of(wv), kraw);
  else
    pid = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.ids, 4u * (uint32_t)P), 4 * tid, 0, 0);
  const __amdgpu_buffer_rsrc_t r_ord = make_rsrc(cd.order, 4u * (uint32_t)C);
  const __amdgpu_buffer_rsrc_t r_sl = make_rsrc(cd.slot_id, 4u * (uint32_t)C);
  int32_t vo[V], vs[V], vr[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    vo[j] = __builtin_amdgcn_raw_buffer_load_b32(r_ord, 4 * (j * kDT + tid), 0, 0);
    vs[j] = __builtin_amdgcn_raw_buffer_load_b32(r_sl, 4 * (j * kDT + tid), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t tick = *cd.tick;      // uniform, consumed late
  const int n_ord = *cd.n_ord;
  uint64_t ctr[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) ctr[i] = cd.counters[i];
  // the layer comes from device memory, so one captured step serves any
  // layer (layer_ld is 0 when it comes as an argument: no branch on the load)
  const int layer = __builtin_amdgcn_readfirstlane(layer_ld) + (a.d_layer ? 0 : a.layer);
  const bool bad_layer = layer < 0 || layer >= cd.L;
  const int lbase = bad_layer ? 0 : layer * E;
  const __amdgpu_buffer_rsrc_t r_row = make_rsrc(cd.id_slot + lbase, bad_layer ? 0u : 4u * (uint32_t)E);
#pragma unroll
  for (int j = 0; j < V; ++j) vr[j] = __builtin_amdgcn_raw_buffer_load_b32(r_row, 4 * (j * kDT + tid), 0, 0);
  __builtin_amdgcn_sched_barrier(0);   // nothing below moves above the row loads
  if constexpr (VPL > 0) {
    topk_keys_of<VPL>(kraw, E, kc, ac);
    // wave wv routes tokens wv, wv + 16, ...; the next token's logits load
    // while this one is picked (a buffer of 0 bytes past the last token) and
    // are waited for only when there is a next token: that wait also covers
    // the stores issued in between, which a last token need not wait for.
    for (int t = wv; t < T; t += kDW) {
      const bool more = t + kDW < T;   // uniform
      uint32_t rn[VPL];
      topk_load<VPL>(row_of(more ? t + kDW : T), rn);
      int id;
      float wt;
      topk_pick_fast<VPL>(kc, ac, E, k, reinterpret_cast<uint2*>(s_lists) + 96 * wv, id, wt);
      if (lane < k && !bad_layer) {   // a bad layer leaves ids and w unwritten
        const_cast<int32_t*>(a.ids)[t * k + lane] = id;
        a.w[t * k + lane] = wt;
        s_pid[t * k + lane] = id;
      }
      if (more) topk_keys_of<VPL>(rn, E, kc, ac);
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j * kDT + tid;
    ord[i] = (uint16_t)(i < n_ord ? vo[j] : 0);   // entries past n_ord read as slot 0
    sl[i] = vs[j];
    row[i] = vr[j];
  }
  for (int b0 = kStageB; b0 < Cp; b0 += kStageB) {   // pools of more than kStageB slots
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int o = 4 * (b0 + j * kDT + tid);
      vo[j] = __builtin_amdgcn_raw_buffer_load_b32(r_ord, o, 0, 0);
      vs[j] = __builtin_amdgcn_raw_buffer_load_b32(r_sl, o, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      ord[b0 + j * kDT + tid] = (uint16_t)(b0 + j * kDT + tid < n_ord ? vo[j] : 0);
      sl[b0 + j * kDT + tid] = vs[j];
    }
  }
  for (int b0 = kStageB; b0 < Ep; b0 += kStageB) {   // layers of more than kStageB experts
#pragma unroll
    for (int j = 0; j < V; ++j) vr[j] = __builtin_amdgcn_raw_buffer_load_b32(r_row, 4 * (b0 + j * kDT + tid), 0, 0);
#pragma unroll
    for (int j = 0; j < V; ++j) row[b0 + j * kDT + tid] = vr[j];
  }
  if (bad_layer) {   // uniform: nothing is decided, every pick goes to the host
    if (tid == 0) atomicOr(cd.error, 1 << ERR_LAYER);
    for (int p = tid; p < P; p += kDT) a.out.pick_slot[p] = -1;
    for (int i = tid; i < a.U_max; i += kDT) {
      a.out.uniq[i] = a.out.is_hit[i] = a.out.host_id[i] = -1;
      a.out.fill_id[i] = a.out.fill_slot[i] = a.out.fill_evicted[i] = -1;
    }
    if (tid < MOE_CNT_N) a.out.counts[tid] = tid == 6 ? layer : 0;
    return;
  }
  for (int i = tid; i < (E + 31) / 32; i += kDT) bm[i] = 0;
  for (int i = tid; i < (C + 31) / 32; i += kDT) hitbm[i] = 0;
  lds_barrier();
  if constexpr (VPL > 0) pid = tid < P ? s_pid[tid] : 0;

  // 1. dedup: bitmap of the routed experts (one pick per thread)
  if (tid < P) {
    if (pid < 0 || pid >= E)
      atomicOr(cd.error, 1 << ERR_BAD_ID);
    else
      atomicOr(&bm[pid >> 5], 1u << (pid & 31));
  }
  lds_barrier();

  // 2. one ordered pass over the layer's experts, e = j*kDT + tid: routed
  //    (unique, ascending), and hit when the residency table holds it.  The
  //    ranks among the unique, hit and missed experts come from ballots and
  //    per-(row, wave) counts, with one barrier between counting and placing;
  //    the classification of each thread's experts stays in registers.
  const int NE = (E + kDT - 1) / kDT;
  int cs[NEM];
  uint64_t cbR[NEM], cbH[NEM];
#pragma unroll
  for (int j = 0; j < NEM; ++j) {
    if (j < NE) {
      const int e = j * kDT + tid;
      const int ee = e < E ? e : 0;
      const uint32_t word = bm[ee >> 5];
      const int s = row[ee];                           // row is padded: ee is in range
      const int owner = sl[(s >= 0 && s < C) ? s : 0];
      const bool rt = e < E && ((word >> (ee & 31)) & 1u) != 0;
      const bool valid = s >= 0 && s < C && owner == lbase + e;
      if (rt && s >= 0 && !valid) atomicOr(cd.error, 1 << ERR_TABLE);   // a broken entry counts as a miss
      cs[j] = rt ? (valid ? s : -1) : -2;
      cbR[j] = __ballot(rt);
      cbH[j] = __ballot(rt && valid);
      s_cnt[j][0][wv] = __popcll(cbR[j]);   // every lane writes the same value: no branch
      s_cnt[j][1][wv] = __popcll(cbH[j]);
    }
  }
  lds_barrier();
  int u = 0, h = 0;   // routed and hit experts before the current row
#pragma unroll
  for (int j = 0; j < NEM; ++j) {
    if (j < NE) {
      int pu, tu, ph, th;
      wave_counts_prefix(&s_cnt[j][0][0], wv, pu, tu);
      wave_counts_prefix(&s_cnt[j][1][0], wv, ph, th);
      const int e = j * kDT + tid;
      const int s = cs[j];
      if (s != -2) {
        const int r = u + pu + __popcll(cbR[j] & lanemask_lt());
        const int rh = h + ph + __popcll(cbH[j] & lanemask_lt());
        uniq[r] = e;
        uslot[r] = s;
        a.out.is_hit[r] = s >= 0 ? 1 : 0;
        if (s >= 0) {
          hit_list[rh] = r;
          atomicOr(&hitbm[s >> 5], 1u << (s & 31));
        } else {
          miss_list[r - rh] = r;
          row[e] = -1;   // host unless step 5 fills it
        }
      }
      u += tu;
      h += th;
    }
  }
  const int m = u - h;
  for (int i = u + tid; i < a.U_max; i += kDT) a.out.is_hit[i] = -1;

  // 3. q* = clamp(round(m bp / bh), 1, m), or m when every miss is to be filled
  int qs = 0;
  if (m > 0 && a.fill_all) {
    qs = m;
  } else if (m > 0) {
    const uint64_t q0 = (2ull * (uint64_t)m * cd.bp + cd.bh) / (2ull * cd.bh);
    qs = (int)(q0 < 1 ? 1 : (q0 > (uint64_t)m ? (uint64_t)m : q0));
  }
  // every hit slot is in the order (it is occupied, so not reserved):
  // the candidates are the other n_ord - h entries
  const int n_cand = n_ord - h;
  const int q = qs < n_cand ? qs : n_cand;
  lds_barrier();   // hit bitmap and lists complete

  // 4. one ordered scan of the LRU order: the first q non-hit entries are the
  //    victims; the others keep their relative order in the new order.
  //    Chunks of kStageB entries, i = b0 + j*kDT + tid, one barrier each.
  {
    int before = 0;   // candidates before the current row
    for (int b0 = 0; b0 < n_ord; b0 += kStageB) {
      const int cb = (b0 / kStageB) & 1;   // count buffers alternate between chunks
      int sv[V];
      uint32_t hw[V];
      uint64_t bc[V];
#pragma unroll
      for (int j = 0; j < V; ++j) sv[j] = ord[b0 + j * kDT + tid];   // padded, 0 past n_ord
#pragma unroll
      for (int j = 0; j < V; ++j) hw[j] = hitbm[sv[j] >> 5];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const bool cand = (b0 + j * kDT + tid < n_ord) & (((hw[j] >> (sv[j] & 31)) & 1u) == 0);
        bc[j] = __ballot(cand);
        s_cc[cb][j][wv] = __popcll(bc[j]);   // every lane writes the same value: no branch
      }
      lds_barrier();
#pragma unroll
      for (int j = 0; j < V; ++j) {
        int pre, tot;
        wave_counts_prefix(&s_cc[cb][j][0], wv, pre, tot);
        if ((bc[j] >> lane) & 1ull) {
          const int r = before + pre + __popcll(bc[j] & lanemask_lt());
          if (r < q)
            victims[r] = sv[j];
          else
            cd.order[r - q] = sv[j];
        }
        before += tot;
      }
    }
  }
  lds_barrier();   // victims complete

  // 5. table update: fill i -> victim i; stamps; tail of the new order
  for (int i = tid; i < q; i += kDT) {
    const int v = victims[i];
    const int e = uniq[miss_list[i]];
    const int f = lbase + e;
    const int old = sl[v];
    if (old >= 0) cd.id_slot[old] = -1;
    cd.slot_id[v] = f;
    cd.id_slot[f] = v;
    row[e] = v;
    a.out.fill_id[i] = f;
    a.out.fill_slot[i] = v;
    a.out.fill_evicted[i] = old;
    cd.stamp[v] = (tick << 16) | (uint64_t)(1 + h + i);
    cd.order[n_cand - q + h + i] = v;
  }
  for (int r = tid; r < h; r += kDT) {
    const int s = uslot[hit_list[r]];
    cd.stamp[s] = (tick << 16) | (uint64_t)(1 + r);
    cd.order[n_cand - q + r] = s;
  }
  lds_barrier();

  // 6. outputs: rewrite picks (row holds each routed expert's slot after the
  //    step, -1 for the host), lists, counts
  if (tid < P) a.out.pick_slot[tid] = (pid >= 0 && pid < E) ? row[pid] : -1;
  for (int i = tid; i < a.U_max; i += kDT) {
    a.out.uniq[i] = i < u ? lbase + uniq[i] : -1;
    if (i >= q) {
      a.out.fill_id[i] = -1;
      a.out.fill_slot[i] = -1;
      a.out.fill_evicted[i] = -1;
    }
    const int hi = i + q;
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
    const uint64_t add[6] = {1, (uint64_t)u, (uint64_t)h, (uint64_t)m, (uint64_t)q, (uint64_t)(m - q)};
#pragma unroll
    for (int i = 0; i < 6; ++i) cd.counters[i] = ctr[i] + add[i];
  }
}

// Rebuild the LRU order from the stamps (set-up paths only: reset, seed,
// reserve, release, hand-over, resize): rank of each non-reserved slot by
// (stamp, slot).  The keys are staged through LDS a tile at a time, so each
// thread compares its slots against every other slot from LDS; a reserved
// slot's key is the maximum and never counts.
constexpr int kOrdTile = 2048;
__global__ __launch_bounds__(1024) void cache_order_kernel(CacheDev cd) {
  __shared__ uint64_t key[kOrdTile];
  __shared__ int cnt;
  constexpr uint64_t kNone = ~0ull;
  const int C = cd.C, tid = threadIdx.x;
  if (tid == 0) cnt = 0;
  constexpr int kPer = kCMax / 1024;   // slots per thread at most
  uint64_t ks[kPer];
  int rank[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int sidx = tid + u * 1024;
    ks[u] = (sidx < C && cd.slot_id[sidx] != -2) ? cd.stamp[sidx] : kNone;
    rank[u] = 0;
  }
  for (int t0 = 0; t0 < C; t0 += kOrdTile) {
    __syncthreads();
    for (int t = tid; t < kOrdTile; t += 1024) {
      const int ti = t0 + t;
      key[t] = (ti < C && cd.slot_id[ti] != -2) ? cd.stamp[ti] : kNone;
    }
    __syncthreads();
    const int nt = C - t0 < kOrdTile ? C - t0 : kOrdTile;
    for (int t = 0; t < nt; ++t) {
      const uint64_t kt = key[t];
      const int ti = t0 + t;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (u * 1024 >= C) break;   // uniform: only the slot columns that exist
        const int sidx = tid + u * 1024;
        rank[u] += (kt < ks[u]) || (kt == ks[u] && ti < sidx);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int sidx = tid + u * 1024;
    if (sidx < C && ks[u] != kNone) {
      cd.order[rank[u]] = sidx;
      atomicAdd(&cnt, 1);
    }
  }
  __syncthreads();
  if (tid == 0) *cd.n_ord = cnt;
}

// ---------------------------------------------------------------- fused fill copy
struct FillArgs {
  const int32_t* fill_id;
  const int32_t* fill_slot;
  const int32_t* n_fill;        // device count
  const uint64_t* host_tab;     // [nb][LE]
  int LE, C, nb;
  char* dst[5];
  uint64_t bytes[5];
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

// On-demand loading of a prefill batch: the set of experts the batch routes
// to, written as n_set ids (whole rows of k for the decision kernel): the
// routed experts ascending, then the first of them repeated (the decision's
// dedup removes repeats; a set with no valid id is all -1).
__global__ __launch_bounds__(1024) void prefill_set_kernel(CacheDev cd, const int32_t* __restrict__ ids, int64_t P,
                                                           int n_set) {
  __shared__ uint32_t bm[kEMax / 32];
  __shared__ int wpre[kEMax / 32 + 1];
  const int E = cd.E, nw = (E + 31) / 32, tid = threadIdx.x;
  for (int i = tid; i < nw; i += 1024) bm[i] = 0;
  __syncthreads();
  for (int64_t p = tid; p < P; p += 1024) {
    const int e = ids[p];
    if (e < 0 || e >= E)
      atomicOr(cd.error, 1 << ERR_BAD_ID);
    else
      atomicOr(&bm[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (tid == 0) {   // at most 128 words
    int acc = 0;
    for (int w = 0; w < nw; ++w) {
      wpre[w] = acc;
      acc += __popc(bm[w]);
    }
    wpre[nw] = acc;
  }
  __syncthreads();
  int* set = cd.set_list;
  const int U = wpre[nw];
  int first = -1;
  for (int w = 0; w < nw && first < 0; ++w)
    if (bm[w]) first = 32 * w + __builtin_ctz(bm[w]);
  for (int w = tid; w < nw; w += 1024) {
    uint32_t bits = bm[w];
    int r = wpre[w];
    while (bits) {
      set[r++] = 32 * w + __builtin_ctz(bits);
      bits &= bits - 1;
    }
  }
  for (int i = U + tid; i < n_set; i += 1024) set[i] = first;
}

// After the decision: each pick of the batch goes to its expert's slot if the
// expert is now resident (it is then in G = H u F), else to the host (-1).
__global__ __launch_bounds__(256) void prefill_pick_kernel(CacheDev cd, const int32_t* __restrict__ ids, int64_t P,
                                                           int layer, int32_t* __restrict__ pick_slot) {
  const int E = cd.E;
  const int32_t* row = cd.id_slot + (size_t)layer * E;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < P; p += (int64_t)gridDim.x * 256) {
    const int e = ids[p];
    pick_slot[p] = (e >= 0 && e < E) ? row[e] : -1;
  }
}

// End of prefill: slot first + b*E + e of buffer b takes expert e of layer
// lay[b] (-1: the buffer holds nothing) with stamp (tick << 16) | (1 + pos[b]*E
// + e), pos[b] being the buffer's rank in load order; an expert already
// resident elsewhere keeps its slot and takes the stamp, leaving the buffer
// slot empty.  The tick then advances by one.
constexpr int kMaxRing = 64;
struct AdoptArgs {
  int first, n_buf;
  int lay[kMaxRing], pos[kMaxRing];
};

__global__ __launch_bounds__(1024) void cache_adopt_kernel(CacheDev cd, AdoptArgs a) {
  const uint64_t tick = *cd.tick;
  const int E = cd.E;
  for (int i = threadIdx.x; i < a.n_buf * E; i += 1024) {
    const int b = i / E, e = i - b * E, s = a.first + i;
    const int layer = a.lay[b];
    if (layer < 0) {
      cd.slot_id[s] = -1;
      cd.stamp[s] = 0;
      continue;
    }
    const int lid = layer * E + e;
    const uint64_t st = (tick << 16) | (uint64_t)(1 + a.pos[b] * E + e);
    const int old = cd.id_slot[lid];
    if (old >= 0 && old < cd.C && cd.slot_id[old] == lid) {
      cd.stamp[old] = st;
      cd.slot_id[s] = -1;
      cd.stamp[s] = 0;
    } else {
      cd.slot_id[s] = lid;
      cd.id_slot[lid] = s;
      cd.stamp[s] = st;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    *cd.tick = tick + 1;
    if (tick + 1 >= (1ull << 28)) atomicOr(cd.error, 1 << ERR_TICK);
  }
}

// ---------------------------------------------------------------- resize
// Tables of the resized cache `nd` (Cn slots, fresh workspace) from those of
// `od` (C slots; no slot reserved): the min(residents, Cn) most recent
// residents (the tail of od's LRU order, where every resident follows every
// empty slot) are kept with their stamps; one below Cn stays in its slot, the
// others move, ascending by old slot, to the free slots below Cn, ascending.
// The copies to make are listed in nd.seed_list: sources [0, Cn),
// destinations [Cn, 2Cn), count at 2Cn; every kept resident when copy_all (the
// banks move to new memory), else only the movers.  One workgroup; each
// thread owns a contiguous chunk of slot numbers, so ranks are chunk prefix
// sums.
__global__ __launch_bounds__(1024) void cache_resize_kernel(CacheDev od, CacheDev nd, int copy_all) {
  __shared__ uint8_t keep[kCMax];
  __shared__ uint16_t free_list[kCMax];
  __shared__ int c_free[1024], c_list[1024], c_move[1024];
  __shared__ int n_res;
  const int tid = threadIdx.x, C = od.C, Cn = nd.C;
  const int S = C > Cn ? C : Cn;
  const int ch = (S + 1023) / 1024;
  const int s0 = tid * ch < S ? tid * ch : S;
  const int s1 = s0 + ch < S ? s0 + ch : S;
  if (tid == 0) n_res = 0;
  for (int x = tid; x < S; x += 1024) keep[x] = 0;
  __syncthreads();
  int nr = 0;
  for (int x = tid; x < C; x += 1024) nr += od.slot_id[x] >= 0 ? 1 : 0;
  atomicAdd(&n_res, nr);
  __syncthreads();
  const int n_ord = *od.n_ord;
  const int n_keep = n_res < Cn ? n_res : Cn;
  for (int i = n_ord - n_keep + tid; i < n_ord; i += 1024) keep[od.order[i]] = 1;
  __syncthreads();
  int nf = 0, nl = 0, nm = 0;
  for (int x = s0; x < s1; ++x) {
    const bool kp = x < C && keep[x];
    nf += (x < Cn && !kp) ? 1 : 0;
    nm += (kp && x >= Cn) ? 1 : 0;
    nl += (kp && (copy_all || x >= Cn)) ? 1 : 0;
  }
  c_free[tid] = nf;
  c_list[tid] = nl;
  c_move[tid] = nm;
  __syncthreads();
  if (tid == 0) {
    int af = 0, al = 0, am = 0;
    for (int t = 0; t < 1024; ++t) {
      const int f = c_free[t], l = c_list[t], m = c_move[t];
      c_free[t] = af;
      c_list[t] = al;
      c_move[t] = am;
      af += f;
      al += l;
      am += m;
    }
    nd.seed_list[2 * Cn] = al;
  }
  __syncthreads();
  int rf = c_free[tid];
  for (int x = s0; x < s1; ++x)
    if (x < Cn && !(x < C && keep[x])) free_list[rf++] = (uint16_t)x;
  for (int x = tid; x < Cn; x += 1024) {
    nd.slot_id[x] = -1;
    nd.stamp[x] = 0;
  }
  for (size_t i = tid; i < (size_t)od.L * od.E; i += 1024) nd.id_slot[i] = -1;
  __syncthreads();
  int rl = c_list[tid], rm = c_move[tid];
  for (int x = s0; x < s1; ++x) {
    if (!(x < C && keep[x])) continue;
    const int dst = x < Cn ? x : (int)free_list[rm++];
    const int id = od.slot_id[x];
    nd.slot_id[dst] = id;
    nd.stamp[dst] = od.stamp[x];
    nd.id_slot[id] = dst;
    if (copy_all || x >= Cn) {
      nd.seed_list[rl] = x;
      nd.seed_list[Cn + rl] = dst;
      ++rl;
    }
  }
  if (tid == 0) {
    *nd.tick = *od.tick;
    for (int i = 0; i < 8; ++i) nd.counters[i] = od.counters[i];
    *nd.error = *od.error;
  }
}

// Copy every bank of each listed slot from the old banks to the new ones.
// Sources and destinations are distinct slots (destinations were free), so
// the copies are independent: each workgroup copies whole experts, with
// eight 16-byte loads per thread in flight, and every workgroup streams at
// once.
struct MoveArgs {
  const int32_t* src;
  const int32_t* dst;
  const int32_t* n;
  int nb;
  const char* from[5];
  char* to[5];
  uint64_t bytes[5];
};

__global__ __launch_bounds__(256) void slot_move_kernel(MoveArgs a) {
  const int n = *a.n;
  for (int f = blockIdx.x; f < n; f += gridDim.x) {
    const size_t s = (size_t)a.src[f], d = (size_t)a.dst[f];
    for (int b = 0; b < a.nb; ++b) {
      const char* src = a.from[b] + s * a.bytes[b];
      char* dst = a.to[b] + d * a.bytes[b];
      if ((a.bytes[b] & 15) == 0) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
        u32x4* d4 = reinterpret_cast<u32x4*>(dst);
        const size_t n16 = a.bytes[b] >> 4;
        size_t i = threadIdx.x;
        for (; i + 7 * 256 < n16; i += 8 * 256) {
          u32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(s4 + i + u * 256);
#pragma unroll
          for (int u = 0; u < 8; ++u) d4[i + u * 256] = v[u];
        }
        for (; i < n16; i += 256) d4[i] = __builtin_nontemporal_load(s4 + i);
      } else {
        const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
        uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
        for (size_t i = threadIdx.x; i < (a.bytes[b] >> 2); i += 256) d1[i] = s1[i];
      }
    }
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
  std::vector<const void*> host_ptr[5];   // host-visible pool pointers (for DMA)
  int lds_bytes;
  int U_max;
  bool has_prefill;
  char* ws;                // the caller's workspace and its used bytes
  size_t ws_used;
};

using namespace moe;

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct WsLayout {
  size_t id_slot, slot_id, stamp, order, n_ord, tick, counters, error, seed, set, host_tab, total;
};
static WsLayout ws_layout(const moe_cache_cfg* c, int nb) {
  WsLayout w{};
  size_t off = 0;
  size_t LE = (size_t)c->L * c->E;
  w.id_slot = off; off = align_up(off + 4 * LE, 256);
  w.slot_id = off; off = align_up(off + 4 * (size_t)c->C, 256);
  w.stamp = off; off = align_up(off + 8 * (size_t)c->C, 256);
  w.order = off; off = align_up(off + 4 * (size_t)c->C, 256);
  w.n_ord = off; off = align_up(off + 4, 256);
  w.tick = off; off = align_up(off + 8, 256);
  w.counters = off; off = align_up(off + 64, 256);
  w.error = off; off = align_up(off + 4, 256);
  w.seed = off; off = align_up(off + 4 * (2 * (size_t)c->C + 8), 256);
  w.set = off; off = align_up(off + 4 * 2 * (size_t)kUMax, 256);
  w.host_tab = off; off = align_up(off + 8 * (size_t)nb * LE, 256);
  w.total = off;
  return w;
}

static CacheDev make_dev(char* ws, const WsLayout& L, const moe_cache_cfg* cfg) {
  CacheDev d{};
  d.id_slot = (int32_t*)(ws + L.id_slot);
  d.slot_id = (int32_t*)(ws + L.slot_id);
  d.stamp = (uint64_t*)(ws + L.stamp);
  d.order = (int32_t*)(ws + L.order);
  d.n_ord = (int32_t*)(ws + L.n_ord);
  d.tick = (uint64_t*)(ws + L.tick);
  d.counters = (uint64_t*)(ws + L.counters);
  d.error = (int32_t*)(ws + L.error);
  d.seed_list = (int32_t*)(ws + L.seed);
  d.set_list = (int32_t*)(ws + L.set);
  d.host_tab = (const uint64_t*)(ws + L.host_tab);
  d.L = cfg->L;
  d.E = cfg->E;
  d.C = cfg->C;
  d.bp = cfg->bp;
  d.bh = cfg->bh;
  return d;
}

// The decision kernels' dynamic-LDS limit is a per-function attribute shared
// by every cache of the process: raise it to the largest size asked for.
static std::mutex g_lds_mu;
static int g_decide_lds = 0;
static hipError_t ensure_decide_lds(int bytes) {
  std::lock_guard<std::mutex> lk(g_lds_mu);
  if (bytes <= g_decide_lds) return hipSuccess;
  const void* fns[] = {(const void*)cache_decide_kernel<0>, (const void*)cache_decide_kernel<1>,
                       (const void*)cache_decide_kernel<2>, (const void*)cache_decide_kernel<4>,
                       (const void*)cache_decide_kernel<8>, (const void*)cache_decide_kernel<16>};
  for (const void* fn : fns) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  g_decide_lds = bytes;
  return hipSuccess;
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
  *bytes = ws_layout(cfg, 5).total;
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
  const int nb = slots->wtype == MOE_W_FP8_B128 ? 5 : 2;
  WsLayout L = ws_layout(cfg, 5);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);

  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  int lds_max = 0;
  MOE_HIP(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  const int lds_static = 32 * 1024;   // bound on the kernel's static LDS (about 21 KB)
  const int lds_dyn = decide_lds_bytes(cfg->C, cfg->E);
  if (lds_dyn + lds_static > lds_max)
    MOE_FAIL(MOE_ERR_SHAPE, "C=%d needs %d B of LDS; device allows %d", cfg->C, lds_dyn + lds_static, lds_max);

  const void* const* tabs[5] = {host->w_gate_up, host->w_down, (const void* const*)host->s_gate,
                                (const void* const*)host->s_up, (const void* const*)host->s_down};
  const size_t LE = (size_t)cfg->L * cfg->E;
  std::vector<uint64_t> htab((size_t)nb * LE);  // nb <= 5
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
  c->ws = ws;
  c->ws_used = L.total;
  c->dev = make_dev(ws, L, cfg);
  const CacheDev& d = c->dev;
  hipError_t e = ensure_decide_lds(lds_dyn);
  if (e != hipSuccess) {
    delete c;
    MOE_FAIL(MOE_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  e = hipMemcpyAsync((void*)d.host_tab, htab.data(), htab.size() * 8, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) {
    cache_reset_kernel<<<64, 256, 0, stream>>>(d, 0);
    cache_order_kernel<<<1, 1024, 0, stream>>>(d);
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

static moe_status launch_fill_to(moe_cache* c, const moe_slots& dst, const int32_t* fill_id,
                                 const int32_t* fill_slot, const int32_t* n_fill, hipStream_t stream) {
  FillArgs f{};
  f.fill_id = fill_id;
  f.fill_slot = fill_slot;
  f.n_fill = n_fill;
  f.host_tab = c->dev.host_tab;
  f.LE = c->cfg.L * c->cfg.E;
  f.C = dst.n_slots;
  f.nb = c->nb;
  void* bases[5] = {dst.w_gate_up, dst.w_down, dst.s_gate, dst.s_up, dst.s_down};
  for (int b = 0; b < c->nb; ++b) {
    f.dst[b] = (char*)bases[b];
    f.bytes[b] = c->bb.b[b];
  }
  cache_fill_kernel<<<512, 256, 0, stream>>>(f);
  MOE_LAUNCHED();
  return MOE_OK;
}

static moe_status launch_fill(moe_cache* c, const int32_t* fill_id, const int32_t* fill_slot,
                              const int32_t* n_fill, hipStream_t stream) {
  return launch_fill_to(c, c->slots, fill_id, fill_slot, n_fill, stream);
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
  cache_order_kernel<<<1, 1024, 0, stream>>>(d);
  MOE_LAUNCHED();
  if (!(flags & MOE_STEP_NO_COPY) && n > 0) {
    moe_status st = launch_fill(c, d.seed_list, d.seed_list + c->cfg.C, d.seed_list + 2 * c->cfg.C, stream);
    if (st) return st;
  }
  MOE_HIP(hipStreamSynchronize(stream));
  return MOE_OK;
}

static moe_status check_step(moe_cache_t c, const int32_t* d_layer, int32_t T, const moe_step_out* out) {
  if (!c || !out || !d_layer) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (reinterpret_cast<uintptr_t>(d_layer) & 3) MOE_FAIL(MOE_ERR_ARG, "d_layer must be 4-byte aligned");
  if (T < 1 || T > c->cfg.T_max) MOE_FAIL(MOE_ERR_SHAPE, "T=%d outside [1, T_max=%d]", T, c->cfg.T_max);
  if (!out->pick_slot || !out->uniq || !out->is_hit || !out->fill_id || !out->fill_slot || !out->fill_evicted ||
      !out->host_id || !out->counts)
    MOE_FAIL(MOE_ERR_ARG, "a moe_step_out buffer is NULL");
  return MOE_OK;
}

extern "C" moe_status moe_cache_step(moe_cache_t c, const int32_t* d_layer, const int32_t* ids, int32_t T,
                                     uint32_t flags, const moe_step_out* out, hipStream_t stream) {
  clear_error();
  moe_status st = check_step(c, d_layer, T, out);
  if (st) return st;
  if (!ids) MOE_FAIL(MOE_ERR_ARG, "ids is NULL");
  StepArgs a{};
  a.ids = ids;
  a.d_layer = d_layer;
  a.T = T;
  a.k = c->cfg.k;
  a.U_max = c->U_max;
  a.fill_all = (flags & MOE_STEP_FILL_ALL) != 0;
  a.out = *out;
  cache_decide_kernel<0><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  MOE_LAUNCHED();
  if (!(flags & MOE_STEP_NO_COPY))
    return launch_fill(c, out->fill_id, out->fill_slot, out->counts + MOE_CNT_FILL, stream);
  return MOE_OK;
}

extern "C" moe_status moe_cache_route_step(moe_cache_t c, const int32_t* d_layer, const float* logits, int32_t T,
                                           int32_t* ids, float* w, uint32_t flags, const moe_step_out* out,
                                           hipStream_t stream) {
  clear_error();
  moe_status st = check_step(c, d_layer, T, out);
  if (st) return st;
  if (!logits || !ids || !w) MOE_FAIL(MOE_ERR_ARG, "null argument");
  const int E = c->cfg.E, k = c->cfg.k;
  if (E > 1024 || k > 32) MOE_FAIL(MOE_ERR_SHAPE, "routing in the step needs E <= 1024 and k <= 32 (E=%d k=%d)", E, k);
  StepArgs a{};
  a.ids = ids;
  a.logits = logits;
  a.w = w;
  a.d_layer = d_layer;
  a.T = T;
  a.k = k;
  a.U_max = c->U_max;
  a.fill_all = (flags & MOE_STEP_FILL_ALL) != 0;
  a.out = *out;
  if (E <= 64)
    cache_decide_kernel<1><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  else if (E <= 128)
    cache_decide_kernel<2><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  else if (E <= 256)
    cache_decide_kernel<4><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  else if (E <= 512)
    cache_decide_kernel<8><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  else
    cache_decide_kernel<16><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
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

extern "C" moe_status moe_cache_prefill_load(moe_cache_t c, int32_t layer, const int32_t* ids, int32_t T,
                                             uint32_t flags, const moe_step_out* out, int32_t* pick_slot,
                                             hipStream_t stream) {
  clear_error();
  if (!c || !out || !ids || !pick_slot) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (layer < 0 || layer >= c->cfg.L) MOE_FAIL(MOE_ERR_SHAPE, "layer %d outside [0, %d)", layer, c->cfg.L);
  if (T < 1) MOE_FAIL(MOE_ERR_SHAPE, "T=%d < 1", T);
  const int E = c->cfg.E, k = c->cfg.k;
  const int rows = (E + k - 1) / k;
  if (rows > c->cfg.T_max)
    MOE_FAIL(MOE_ERR_SHAPE, "on-demand loading passes a layer's expert set as %d rows of k; T_max is %d", rows,
             c->cfg.T_max);
  if (!out->uniq || !out->is_hit || !out->fill_id || !out->fill_slot || !out->fill_evicted || !out->host_id ||
      !out->counts)
    MOE_FAIL(MOE_ERR_ARG, "a moe_step_out buffer is NULL");
  const int64_t P = (int64_t)T * k;
  prefill_set_kernel<<<1, 1024, 0, stream>>>(c->dev, ids, P, rows * k);
  MOE_LAUNCHED();
  StepArgs a{};
  a.ids = c->dev.set_list;
  a.layer = layer;
  a.T = rows;
  a.k = k;
  a.U_max = c->U_max;
  a.fill_all = 1;
  a.out = *out;
  a.out.pick_slot = c->dev.set_list + kUMax;   // picks of the set itself: not the caller's
  cache_decide_kernel<0><<<1, kDT, c->lds_bytes, stream>>>(c->dev, a);
  MOE_LAUNCHED();
  const int64_t blocks = (P + 255) / 256 < 2048 ? (P + 255) / 256 : 2048;
  prefill_pick_kernel<<<(unsigned)blocks, 256, 0, stream>>>(c->dev, ids, P, layer, pick_slot);
  MOE_LAUNCHED();
  if (!(flags & MOE_STEP_NO_COPY))
    return launch_fill(c, out->fill_id, out->fill_slot, out->counts + MOE_CNT_FILL, stream);
  return MOE_OK;
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

extern "C" moe_status moe_cache_resize(moe_cache_t c, const moe_slots* slots, void* dev_ws, size_t ws_bytes,
                                       hipStream_t stream) {
  clear_error();
  if (!c || !dev_ws) MOE_FAIL(MOE_ERR_ARG, "null argument");
  moe_status st = check_slots(slots);
  if (st) return st;
  if (c->has_prefill) MOE_FAIL(MOE_ERR_STATE, "cannot resize while a prefill pool holds slots");
  if (slots->wtype != c->slots.wtype || slots->H != c->slots.H || slots->I != c->slots.I)
    MOE_FAIL(MOE_ERR_ARG, "the new slots must have the cache's weight type, H and I");
  moe_cache_cfg ncfg = c->cfg;
  ncfg.C = slots->n_slots;
  if ((st = check_cfg(&ncfg))) return st;
  if (reinterpret_cast<uintptr_t>(dev_ws) & 255) MOE_FAIL(MOE_ERR_ARG, "workspace must be 256-byte aligned");
  const WsLayout L = ws_layout(&ncfg, 5);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* nws = (char*)dev_ws;
  // address ranges as integers: the two allocations are unrelated objects
  const auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(nws, L.total, c->ws, c->ws_used))
    MOE_FAIL(MOE_ERR_ARG, "the new workspace overlaps the cache's current one");
  int dev = 0, lds_max = 0;
  MOE_HIP(hipGetDevice(&dev));
  MOE_HIP(hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  const int lds_dyn = decide_lds_bytes(ncfg.C, ncfg.E);
  if (lds_dyn + 32 * 1024 > lds_max)
    MOE_FAIL(MOE_ERR_SHAPE, "C=%d needs %d B of LDS; device allows %d", ncfg.C, lds_dyn + 32 * 1024, lds_max);
  // banks: all in place (same base) or all in new memory that does not overlap the old
  const void* ob[5] = {c->slots.w_gate_up, c->slots.w_down, c->slots.s_gate, c->slots.s_up, c->slots.s_down};
  const void* nbk[5] = {slots->w_gate_up, slots->w_down, slots->s_gate, slots->s_up, slots->s_down};
  int same = 0;
  for (int b = 0; b < c->nb; ++b) {
    if (ob[b] == nbk[b]) {
      ++same;
      continue;
    }
    const size_t bo = (size_t)c->cfg.C * c->bb.b[b], bn = (size_t)ncfg.C * c->bb.b[b];
    if (overlap(nbk[b], bn, ob[b], bo)) MOE_FAIL(MOE_ERR_ARG, "bank %d of the new slots overlaps the old one", b);
  }
  if (same != 0 && same != c->nb) MOE_FAIL(MOE_ERR_ARG, "move every bank or none");
  const int copy_all = same == 0;

  CacheDev nd = make_dev(nws, L, &ncfg);
  MOE_HIP(ensure_decide_lds(lds_dyn));
  const size_t LE = (size_t)c->cfg.L * c->cfg.E;
  MOE_HIP(hipMemcpyAsync((void*)nd.host_tab, c->dev.host_tab, 8 * (size_t)c->nb * LE, hipMemcpyDeviceToDevice,
                         stream));
  cache_resize_kernel<<<1, 1024, 0, stream>>>(c->dev, nd, copy_all);
  cache_order_kernel<<<1, 1024, 0, stream>>>(nd);
  MoveArgs m{};
  m.src = nd.seed_list;
  m.dst = nd.seed_list + ncfg.C;
  m.n = nd.seed_list + 2 * ncfg.C;
  m.nb = c->nb;
  for (int b = 0; b < c->nb; ++b) {
    m.from[b] = (const char*)ob[b];
    m.to[b] = (char*)nbk[b];
    m.bytes[b] = c->bb.b[b];
  }
  slot_move_kernel<<<512, 256, 0, stream>>>(m);
  MOE_LAUNCHED();
  MOE_HIP(hipStreamSynchronize(stream));
  c->cfg = ncfg;
  c->slots = *slots;
  c->dev = nd;
  c->lds_bytes = lds_dyn;
  c->ws = nws;
  c->ws_used = L.total;
  return MOE_OK;
}

// ================================================================ prefill full-layer buffers
struct moe_prefill {
  moe_cache* c;
  int first;               // first reserved slot
  int E;
  int D;                   // buffers: layer l uses buffer l % D
  uint64_t n_loads;        // prefetches so far (load order of the buffers)
  std::vector<int> buf_layer;
  std::vector<uint64_t> buf_load;
  std::vector<hipEvent_t> ready, released;
  std::vector<char> released_recorded;   // released[b] has been recorded at least once
  std::vector<char> buf_free;            // the layer buffer b holds (if any) has been released since its prefetch
  ~moe_prefill() {
    for (hipEvent_t e : ready) if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : released) if (e) (void)hipEventDestroy(e);
  }
};

extern "C" moe_status moe_prefill_create_ring(moe_cache_t c, int32_t depth, moe_prefill_t* out) {
  clear_error();
  if (!c || !out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  *out = nullptr;
  if (depth < 2 || depth > kMaxRing) MOE_FAIL(MOE_ERR_SHAPE, "ring depth %d outside [2, %d]", depth, kMaxRing);
  if (c->has_prefill) MOE_FAIL(MOE_ERR_STATE, "the cache already has a prefill pool");
  const int E = c->cfg.E;
  if ((int64_t)depth * E > c->cfg.C)
    MOE_FAIL(MOE_ERR_NO_SPACE, "%d full-layer buffers need %lld slots; the pool has %d", depth,
             (long long)depth * E, c->cfg.C);
  moe_prefill* p = new moe_prefill();
  p->c = c;
  p->E = E;
  p->D = depth;
  p->n_loads = 0;
  p->first = c->cfg.C - depth * E;
  p->buf_layer.assign(depth, -1);
  p->buf_load.assign(depth, 0);
  p->ready.assign(depth, nullptr);
  p->released.assign(depth, nullptr);
  p->released_recorded.assign(depth, 0);
  p->buf_free.assign(depth, 1);
  for (int b = 0; b < depth; ++b) {
    hipError_t e1 = hipEventCreateWithFlags(&p->ready[b], hipEventDisableTiming);
    hipError_t e2 = hipEventCreateWithFlags(&p->released[b], hipEventDisableTiming);
    if (e1 != hipSuccess || e2 != hipSuccess) {
      delete p;
      MOE_FAIL(MOE_ERR_HIP, "hipEventCreate failed");
    }
  }
  cache_mark_kernel<<<(depth * E + 255) / 256, 256, 0, 0>>>(c->dev, p->first, depth * E, -2);
  cache_order_kernel<<<1, 1024, 0, 0>>>(c->dev);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete p;
    MOE_FAIL(MOE_ERR_HIP, "reserving the buffers: %s", hipGetErrorString(e));
  }
  c->has_prefill = true;
  *out = p;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_create(moe_cache_t c, moe_prefill_t* out) {
  return moe_prefill_create_ring(c, 2, out);
}

extern "C" moe_status moe_prefill_prefetch(moe_prefill_t p, int32_t layer, hipStream_t copy_stream) {
  clear_error();
  if (!p) MOE_FAIL(MOE_ERR_ARG, "pool is NULL");
  moe_cache* c = p->c;
  if (layer < 0 || layer >= c->cfg.L) MOE_FAIL(MOE_ERR_SHAPE, "layer %d outside [0, %d)", layer, c->cfg.L);
  const int b = layer % p->D;
  // the copy may only overwrite the buffer once the layer it holds is released:
  // waiting on an older release would let the copy overwrite weights that
  // the compute stream is still reading
  if (!p->buf_free[b])
    MOE_FAIL(MOE_ERR_STATE, "buffer %d still holds layer %d, which has not been released", b, p->buf_layer[b]);
  if (p->released_recorded[b]) MOE_HIP(hipStreamWaitEvent(copy_stream, p->released[b], 0));
  const int E = p->E;
  const int slot0 = p->first + b * E;
  void* bases[5] = {c->slots.w_gate_up, c->slots.w_down, c->slots.s_gate, c->slots.s_up, c->slots.s_down};
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
  p->buf_load[b] = ++p->n_loads;
  p->buf_free[b] = 0;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_acquire(moe_prefill_t p, int32_t layer, hipStream_t compute, moe_slots* view) {
  clear_error();
  if (!p || !view) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (layer < 0) MOE_FAIL(MOE_ERR_STATE, "layer %d was not prefetched", layer);
  const int b = layer % p->D;
  if (p->buf_layer[b] != layer) MOE_FAIL(MOE_ERR_STATE, "layer %d was not prefetched into buffer %d", layer, b);
  MOE_HIP(hipStreamWaitEvent(compute, p->ready[b], 0));
  moe_cache* c = p->c;
  const int slot0 = p->first + b * p->E;
  moe_slots v = c->slots;
  v.n_slots = p->E;
  v.w_gate_up = (char*)c->slots.w_gate_up + (size_t)slot0 * c->bb.b[0];
  v.w_down = (char*)c->slots.w_down + (size_t)slot0 * c->bb.b[1];
  if (c->nb == 5) {
    v.s_gate = (float*)((char*)c->slots.s_gate + (size_t)slot0 * c->bb.b[2]);
    v.s_up = (float*)((char*)c->slots.s_up + (size_t)slot0 * c->bb.b[3]);
    v.s_down = (float*)((char*)c->slots.s_down + (size_t)slot0 * c->bb.b[4]);
  }
  *view = v;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_release(moe_prefill_t p, int32_t layer, hipStream_t compute) {
  clear_error();
  if (!p) MOE_FAIL(MOE_ERR_ARG, "pool is NULL");
  if (layer < 0) MOE_FAIL(MOE_ERR_STATE, "layer %d does not own a buffer", layer);
  const int b = layer % p->D;
  if (p->buf_layer[b] != layer) MOE_FAIL(MOE_ERR_STATE, "layer %d does not own buffer %d", layer, b);
  MOE_HIP(hipEventRecord(p->released[b], compute));
  p->released_recorded[b] = 1;
  p->buf_free[b] = 1;
  return MOE_OK;
}

// Ends the pool: keep = the buffers' layers become residents, else the
// buffers return to the LRU empty.
static moe_status prefill_end(moe_prefill_t p, bool keep, hipStream_t stream) {
  moe_cache* c = p->c;
  MOE_HIP(hipDeviceSynchronize());   // every prefetch has landed and no kernel reads the buffers
  AdoptArgs a{};
  a.first = p->first;
  a.n_buf = p->D;
  std::vector<std::pair<uint64_t, int>> loads;
  for (int b = 0; b < p->D; ++b) {
    a.lay[b] = keep ? p->buf_layer[b] : -1;
    if (a.lay[b] >= 0) loads.push_back({p->buf_load[b], b});
  }
  std::sort(loads.begin(), loads.end());
  for (size_t i = 0; i < loads.size(); ++i) a.pos[loads[i].second] = (int)i;
  if (keep) {
    cache_adopt_kernel<<<1, 1024, 0, stream>>>(c->dev, a);
  } else {
    cache_mark_kernel<<<(p->D * p->E + 255) / 256, 256, 0, stream>>>(c->dev, p->first, p->D * p->E, -1);
  }
  cache_order_kernel<<<1, 1024, 0, stream>>>(c->dev);
  MOE_LAUNCHED();
  MOE_HIP(hipStreamSynchronize(stream));
  c->has_prefill = false;
  delete p;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_finish(moe_prefill_t p, hipStream_t stream) {
  clear_error();
  if (!p) MOE_FAIL(MOE_ERR_ARG, "pool is NULL");
  return prefill_end(p, true, stream);
}

extern "C" moe_status moe_prefill_destroy(moe_prefill_t p, hipStream_t stream) {
  clear_error();
  if (!p) return MOE_OK;
  return prefill_end(p, false, stream);
}

// ================================================================ bandwidth calibration
// [FT] section "q* 策略": B_P and B_H are measured on the deployed machine,
// with the deployed tensor shapes, and feed the split; [FT] section "挑战二":
// the right split between transfer and host execution is a property of the
// machine.  B_P is measured through the path decode fills take (the fused
// fill kernel reading mapped pinned memory) and through the DMA engines
// (hipMemcpyAsync, the path of the prefill buffers); B_H through the host
// executor evaluating experts of the pool as a decode step's host set.
extern "C" moe_status moe_calibrate_bandwidth(moe_cache_t c, moe_host_exec_t hx, const int32_t* ids, int32_t n,
                                              const moe_slots* scratch, int32_t reps, hipStream_t stream,
                                              moe_bandwidth* out) {
  clear_error();
  if (!c || !ids || !scratch || !out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (n < 1 || n > c->cfg.C || reps < 1 || reps > 1000)
    MOE_FAIL(MOE_ERR_SHAPE, "calibration needs 1 <= n <= C (%d) and 1 <= reps <= 1000 (n=%d reps=%d)", c->cfg.C, n,
             reps);
  moe_status st = check_slots(scratch);
  if (st) return st;
  if (scratch->wtype != c->slots.wtype || scratch->H != c->slots.H || scratch->I != c->slots.I ||
      scratch->n_slots < n)
    MOE_FAIL(MOE_ERR_SHAPE, "scratch slots must match the cache's weight type, H and I and hold n = %d experts", n);
  const int LE = c->cfg.L * c->cfg.E;
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= LE) MOE_FAIL(MOE_ERR_ARG, "id %d out of range", ids[i]);
  *out = moe_bandwidth{};
  size_t expert_bytes = 0;
  for (int b = 0; b < c->nb; ++b) expert_bytes += c->bb.b[b];
  out->expert_bytes = (double)expert_bytes;
  const double bytes = (double)expert_bytes * n;

  // the fill list: ids -> scratch slots 0 .. n-1, in the cache's seed scratch
  std::vector<int32_t> list(2 * (size_t)n + 1);
  for (int i = 0; i < n; ++i) {
    list[i] = ids[i];
    list[n + i] = i;
  }
  list[2 * n] = n;
  int32_t* dl = c->dev.seed_list;
  MOE_HIP(hipMemcpyAsync(dl, list.data(), 4 * list.size(), hipMemcpyHostToDevice, stream));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  MOE_HIP(hipEventCreate(&e0));
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    MOE_FAIL(MOE_ERR_HIP, "hipEventCreate failed");
  }
  auto timed = [&](const std::function<moe_status()>& body, double* ms) -> moe_status {
    moe_status s1 = body();   // warm-up
    if (s1) return s1;
    if (hipEventRecord(e0, stream) != hipSuccess) MOE_FAIL(MOE_ERR_HIP, "hipEventRecord failed");
    for (int r = 0; r < reps; ++r)
      if ((s1 = body())) return s1;
    if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
      MOE_FAIL(MOE_ERR_HIP, "event wait failed");
    float f = 0.f;
    if (hipEventElapsedTime(&f, e0, e1) != hipSuccess) MOE_FAIL(MOE_ERR_HIP, "hipEventElapsedTime failed");
    *ms = f;
    return MOE_OK;
  };
  double ms_fill = 0, ms_dma = 0;
  st = timed([&] { return launch_fill_to(c, *scratch, dl, dl + n, dl + 2 * n, stream); }, &ms_fill);
  void* bases[5] = {scratch->w_gate_up, scratch->w_down, scratch->s_gate, scratch->s_up, scratch->s_down};
  if (!st)
    st = timed(
        [&]() -> moe_status {
          for (int i = 0; i < n; ++i)
            for (int b = 0; b < c->nb; ++b)
              MOE_HIP(hipMemcpyAsync((char*)bases[b] + (size_t)i * c->bb.b[b], c->host_ptr[b][ids[i]], c->bb.b[b],
                                     hipMemcpyHostToDevice, stream));
          return MOE_OK;
        },
        &ms_dma);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st) return st;
  out->fill_GBps = bytes * reps / (ms_fill * 1e-3) / 1e9;
  out->dma_GBps = bytes * reps / (ms_dma * 1e-3) / 1e9;
  out->bp = (uint32_t)std::max(1.0, std::floor(out->fill_GBps * 10.0 + 0.5));

  if (hx) {
    // the host executor on decode-shaped calls: one token, k = min(8, n) host
    // picks per call, cycling through the ids
    const int H = c->slots.H, I = c->slots.I;
    const int k = n < 8 ? n : 8;
    moe_host_pool pool{};
    pool.w_gate_up = c->host_ptr[0].data();
    pool.w_down = c->host_ptr[1].data();
    if (c->nb == 5) {
      pool.s_gate = (const float* const*)c->host_ptr[2].data();
      pool.s_up = (const float* const*)c->host_ptr[3].data();
      pool.s_down = (const float* const*)c->host_ptr[4].data();
    }
    std::vector<uint16_t> x((size_t)H, 0x3f80);   // 1.0 in BF16
    std::vector<int32_t> pid(k), pick(k, -1);
    std::vector<float> w(k, 1.0f / k), y((size_t)H);
    auto one = [&](int call) -> moe_status {
      for (int j = 0; j < k; ++j) pid[j] = ids[(call * k + j) % n];
      return moe_host_forward(hx, &pool, c->slots.wtype, H, I, x.data(), pid.data(), pick.data(), w.data(), 1, k,
                              y.data());
    };
    if ((st = one(0))) return st;
    const auto t0 = std::chrono::steady_clock::now();
    for (int r = 0; r < reps; ++r)
      if ((st = one(r + 1))) return st;
    const double sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    out->host_GBps = (double)expert_bytes * k * reps / sec / 1e9;
    out->bh = (uint32_t)std::max(1.0, std::floor(out->host_GBps * 10.0 + 0.5));
  }
  return MOE_OK;
}
