// Grouped SwiGLU expert evaluation of G = H u F, the weight packing, and the
// partial-sum merge.
//
// [FT] section "执行顺序与工程细节": after the cache update and the copy of F the
// GPU evaluates all of G as one grouped computation.  [OSDI] section 4.3: an
// expert is gate, up and down projections, down reads SiLU(gate) * up.
// [OSDI] section 4.2: FP8 weights are kept as stored, expanded in registers,
// dotted first and multiplied by the shared block scale once per block
// (post-scaling: scale * sum(w x) = sum(scale * w * x)).
//
// Weights live in 1 KB MFMA bricks (see below), so every weight load of a
// wave is one contiguous 1 KB segment.
// Decode (T <= 16): every slot in G is streamed once from HBM; the brick is
// the MFMA A operand and the (up to 16) tokens are B, so one read of a slot
// serves the whole batch.  One launch: gate/up + SwiGLU into h, then down
// with the per-token gate weights (and the merge with the host partial sum).
// Prefill (any T): (token, pick) pairs counting-sorted by slot, a grouped
// MFMA GEMM for gate/up with the SwiGLU epilogue, a grouped MFMA GEMM for
// down with the gate-weight epilogue into per-pair rows, and a combine that
// sums each token's k rows in pick order.
#include "common.h"

#include <algorithm>
#include <type_traits>
#include <atomic>
#include <mutex>

namespace moe {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// position of element r (0..15) of a 16-group after the even/odd permutation
__device__ __forceinline__ int perm16(int r) { return (r & 1) ? 8 + (r >> 1) : (r >> 1); }

// 16 BF16 (8 dwords, natural order) -> even elements then odd elements
__device__ __forceinline__ void split_even_odd(const u32x4& a, const u32x4& b, u32x4& ev, u32x4& od) {
  ev[0] = (a[0] & 0xFFFFu) | (a[1] << 16);
  ev[1] = (a[2] & 0xFFFFu) | (a[3] << 16);
  ev[2] = (b[0] & 0xFFFFu) | (b[1] << 16);
  ev[3] = (b[2] & 0xFFFFu) | (b[3] << 16);
  od[0] = (a[0] >> 16) | (a[1] & 0xFFFF0000u);
  od[1] = (a[2] >> 16) | (a[3] & 0xFFFF0000u);
  od[2] = (b[0] >> 16) | (b[1] & 0xFFFF0000u);
  od[3] = (b[2] >> 16) | (b[3] & 0xFFFF0000u);
}

// ================================================================ brick format
// A matrix W [N][K] is stored as 1 KB bricks of 16 rows x KB columns (KB = 32
// BF16 or 64 E4M3): brick (t, kt) at byte offset (t * (K/KB) + kt) * 1024,
// lane l = 16 j + r of an MFMA operand at l * 16 within it, holding
// W[16t + r][KB kt + (KB/4) j + e].  A brick is therefore one MFMA 16x16x32
// operand (A for weights-as-rows, B for weights-as-columns) read with one
// contiguous 1 KB wave load.  The gate/up bank packs the 2I-row matrix whose
// row 16t + r is gate row 8t + r (r < 8) or up row 8t + r - 8 (r >= 8).

__global__ __launch_bounds__(256) void pack_kernel(int fp8, int H, int I, int n, const char* __restrict__ wg,
                                                   const char* __restrict__ wu, const char* __restrict__ wd,
                                                   char* __restrict__ gu, char* __restrict__ dp) {
  const int el = fp8 ? 1 : 2, KB = fp8 ? 64 : 32;
  const size_t gu_chunks = (size_t)2 * I * H * el / 16, d_chunks = (size_t)H * I * el / 16;
  const size_t per = gu_chunks + d_chunks;
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= per * n) return;
  const size_t e = c / per;
  size_t rem = c % per;
  const int lane = (int)(rem & 63), r = lane & 15, j = lane >> 4;
  const size_t brick = rem >> 6;
  if (rem < gu_chunks) {
    const int nkt = H / KB;
    const int t = (int)(brick / nkt), kt = (int)(brick % nkt);
    const int row = 8 * t + (r & 7);
    const int col = KB * kt + (KB / 4) * j;
    const char* src = (r < 8 ? wg : wu) + ((e * I + row) * (size_t)H + col) * el;
    *reinterpret_cast<u32x4*>(gu + e * gu_chunks * 16 + rem * 16) = ld16(src);
  } else {
    rem -= gu_chunks;
    const size_t b2 = rem >> 6;
    const int nkt = I / KB;
    const int t = (int)(b2 / nkt), kt = (int)(b2 % nkt);
    const int row = 16 * t + r;
    const int col = KB * kt + (KB / 4) * j;
    const char* src = wd + ((e * H + row) * (size_t)I + col) * el;
    *reinterpret_cast<u32x4*>(dp + e * d_chunks * 16 + rem * 16) = ld16(src);
  }
}

// ================================================================ decode
// The launch is a grid of resident workgroups that walk a task list
// round-robin.  Every weight and activation load is a raw buffer load whose
// offset is pushed past the buffer's end when the step does not exist, so the
// hardware returns zeros without touching memory: each wave issues one fixed
// sequence of loads, kept D steps (2 bricks each) ahead of the MFMAs in a
// register ring, with no branch around any load.
constexpr int kDecTok = 16;     // MFMA N: tokens of one decode call
constexpr int kDecPmax = 256;   // T * k picks
constexpr int kDecPPL = kDecPmax / 64;
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past the end of every decode buffer

struct DecArgs {
  const void* w_gu;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int H, I, n_slots, T, k;
  const uint16_t* x;         // [T][H]
  const int32_t* pick_slot;  // [T*k]
  const float* w;            // [T*k]
  float* y;                  // [T][H] GPU partial sum, or NULL
  const float* y_host;       // [T][H] host partial sum (merge), or NULL
  float* y_out;              // [T][H] y + y_host (merge), or NULL
  uint16_t* y_bf16;          // [T][H] BF16 of y_out (merge), or NULL
  uint16_t* h;               // workspace [G_max][16][I] BF16
  int G_max;
  int phase;                 // 0: both projections in one launch; a split pair: 1 gate/up only, then 2 down only;
                             // 3: down only, with the waits of 0 (nothing raises their signal: a test of the bound)
  uint32_t poll_limit;       // polls of a bounded wait before it gives up
};

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// device scope (sc1): sees the write-through stores of other XCDs without an L2 invalidate
__device__ __forceinline__ u32x4 bload_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16));
}
__device__ __forceinline__ u32x4 bload_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
// Offset v if c, else past the end of the buffer.  The empty asm keeps the
// choice a register select: without it the compiler may split the load into
// two branches writing one register, and order them with a full wait on all
// loads in flight.
__device__ __forceinline__ uint32_t oob_sel(bool c, uint32_t v) {
  uint32_t o = c ? v : kOOB;
  asm volatile("" : "+v"(o));
  return o;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Group plan, computed by one wave: groups are the distinct valid slots of
// pick_slot in order of first appearance.  s_gslot[g] = slot of group g; if
// s_gw is not NULL, s_gw[g*16 + t] = gate weight of token t's pick of group g
// (0 if token t did not pick it).  Writes *s_G.  s_tab is LDS scratch of
// kPlanTab words: an open-addressing table slot -> earliest pick holding it
// (key in the high half, pick index in the low half, so atomicMin keeps the
// earliest pick).  No barrier inside.
constexpr int kPlanTab = 2 * kDecPmax;
__device__ void wave_plan(const int32_t* __restrict__ pick_slot, const float* __restrict__ w, int P, int k,
                          int n_slots, int G_max, int* s_gslot, float* s_gw, int* s_G, unsigned long long* s_tab) {
  const int lane = threadIdx.x & 63;
  constexpr unsigned long long kEmpty = ~0ull;
  int sl[kDecPPL], hs[kDecPPL];
  float pw[kDecPPL];   // gate weights, loaded with the slots: one memory round trip for both
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    const int p = lane + 64 * h;
    const int s = p < P ? pick_slot[p] : -1;
    pw[h] = (s_gw && p < P) ? w[p] : 0.f;
    sl[h] = (s >= 0 && s < n_slots) ? s : -1;
  }
  for (int i = lane; i < kPlanTab; i += 64) s_tab[i] = kEmpty;
  if (s_gw)
    for (int i = lane; i < G_max * kDecTok; i += 64) s_gw[i] = 0.f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    hs[h] = -1;
    if (sl[h] < 0) continue;
    const unsigned long long want = ((unsigned long long)(uint32_t)sl[h] << 32) | (uint32_t)(lane + 64 * h);
    int pos = (int)(((uint32_t)sl[h] * 2654435761u) >> 23) & (kPlanTab - 1);
    for (int probe = 0; probe < kPlanTab; ++probe) {
      unsigned long long cur = atomicCAS(&s_tab[pos], kEmpty, want);
      if (cur == kEmpty || (cur >> 32) == (uint32_t)sl[h]) {
        if (cur != kEmpty) atomicMin(&s_tab[pos], want);
        hs[h] = pos;
        break;
      }
      pos = (pos + 1) & (kPlanTab - 1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  int fq[kDecPPL];
  bool first[kDecPPL];
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    fq[h] = hs[h] >= 0 ? (int)(uint32_t)s_tab[hs[h]] : lane + 64 * h;
    first[h] = hs[h] >= 0 && fq[h] == lane + 64 * h;
  }
  uint64_t m[kDecPPL];
  int base[kDecPPL + 1];
  base[0] = 0;
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    m[h] = __ballot(first[h]);
    base[h + 1] = base[h] + __popcll(m[h]);
  }
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    if (hs[h] < 0) continue;
    const int f = fq[h];
    int g = 0;
#pragma unroll
    for (int h2 = 0; h2 < kDecPPL; ++h2)
      if ((f >> 6) == h2) g = base[h2] + __popcll(m[h2] & ((1ull << (f & 63)) - 1ull));
    if (first[h]) s_gslot[g] = sl[h];
    if (s_gw) s_gw[g * kDecTok + (lane + 64 * h) / k] = pw[h];
  }
  if (lane == 0) *s_G = base[kDecPPL];
}

// ---------------------------------------------------------------- fused decode
// One launch evaluates both projections: a grid of resident workgroups walks
// one task list round-robin, first the gate/up tasks (group g, brick row t),
// then the down tasks (one 16-row block of y each, over every (group, K)
// step).  A workgroup takes its tasks in list order, so every gate/up task is
// finished or in progress before any workgroup waits for one.  The waves of a
// workgroup split a task's K steps and meet in LDS at its end, so every
// output element is summed by one workgroup in a fixed order: y is written
// with plain stores and has the same bits on every run; the merge with the
// host partial sum happens in the same place ([FT] section "q* 策略": the two
// partial sums are added).
//
// Hand-over without a reset launch.  A gate/up task writes its h values with
// device-coherent (write-through) stores, waits for them, and counts itself
// in done[g]; the task that completes group g (old value I/8 - 1) clears
// done[g] and counts the group in `all`; the task that completes the last
// group clears `all` and raises go[b] for every workgroup b that holds a
// down task.  A down workgroup first loads the weights of its first D steps,
// then polls its own go[b] (one address per poller, so the polls stay off
// the streams' memory channels), clears it, and only then loads h.  Every
// control word is back at 0 when the launch ends, so a workspace that starts
// zero-filled stays valid.  A poll is bounded: on time-out the workgroup
// flags the workspace error word and goes on.
constexpr int kCtrlStride = 16;                     // one control word per 64 bytes
constexpr int kDecGridMax = 4096;                   // go flags
constexpr uint32_t kPollLimit = 1u << 22;

struct DecWsDev {
  uint32_t* err;          // [1] sticky error word
  uint32_t* done;         // [kDecPmax * kCtrlStride] per-group count of finished gate/up tasks
  uint32_t* all;          // [1] finished groups
  uint32_t* go;           // [kDecGridMax * kCtrlStride] per-workgroup start signal of the down phase
};

// DR: rows of y per down task.
//  16: one brick row per task; each wave streams its (group, K step) pairs
//      through a register ring D steps deep, weights before the start signal
//      and h after it.
//  32: (FP8) the same with two brick rows per task, each h load
//      serving both.
//   8: (BF16) half a brick row per task (the task's slice of a brick is one
//      128-byte line per K chunk), for calls whose down work is small: every
//      wave issues ALL of its down weights into registers when its gate/up
//      tasks are done (at most kDecResSteps steps of 4 bricks), so they stream
//      while the second round of gate/up tasks runs; after the start
//      signal the workgroup copies h into LDS in one round trip of
//      device-scope loads (no L2 invalidate), so the only memory latency left
//      between the signal and y is that copy.  Each of a step's two 16-byte
//      loads per lane holds the 8-row slices of two bricks (lanes 16j + r,
//      r < 8: the first, r >= 8: the second): against the first brick's h the
//      product's rows 0-7 are that brick's sums, against the second's its
//      rows 8-15 are; two accumulators collect them and the valid halves are
//      added at the end.
constexpr int kDecResSteps = 6;          // down steps per wave held in registers (DR = 8)
constexpr int kDecResH = 32 * 1024;      // bytes of LDS for h (DR = 8): G * T * I * 2 at most

// (RG = 4: the register budget of two workgroups per CU is asked for
// explicitly; left to itself the compiler takes 134 VGPRs, one per CU)
// HDEV: the down phase reads h with device-scope loads instead of one L2
// invalidate per workgroup and ordinary loads (cheaper when h is small: T = 1).
template <bool FP8, int D, int NW, int DR, int RG = 1, bool HDEV = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RG == 4 ? 4 : 1)))
void dec_fused_kernel(DecArgs a, DecWsDev c) {
  static_assert(DR == 16 || DR == 32 || (DR == 8 && !FP8), "down tasks of 16 or 32 rows, or 8 (BF16 only)");
  static_assert(RG == 1 || ((RG == 2 || RG == 4) && DR != 8), "gate/up tasks of one, two or four brick rows");
  constexpr int NRB = DR == 32 ? 2 : 1;   // brick rows per down task (DR >= 16)
  __shared__ __align__(16) uint16_t s_h[DR == 8 ? kDecResH / 2 : 8];
  __shared__ int s_gslot[kDecPmax];
  __shared__ float s_gw[kDecPmax * kDecTok];
  __shared__ int s_G;
  __shared__ unsigned long long s_tab[kPlanTab];
  __shared__ f32x4 red[2][NW][64];
  // the second brick row of a gate/up or down task
  __shared__ f32x4 redB[RG > 1 || NRB > 1 ? 2 : 1][NW][RG > 1 || NRB > 1 ? 64 : 1];
  // the third and fourth brick rows of a gate/up task (RG = 4), one buffer:
  // wave 0 sums them before a second barrier releases it
  __shared__ f32x4 red4[RG == 4 ? 2 : 1][NW][RG == 4 ? 64 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I, T = a.T;
  if (wv == 0) wave_plan(a.pick_slot, a.w, T * a.k, a.k, a.n_slots, a.G_max, s_gslot, s_gw, &s_G, s_tab);
  __syncthreads();
  const int G = s_G;
  const bool tok = r < T;
  constexpr int XN = FP8 ? 4 : 2;
  const int RA = I / 8;                          // gate/up brick rows
  const int RAT = RA / RG;                       // gate/up tasks per group (the host checks RG | RA)
  // (a split pair: the first launch takes only the gate/up tasks, the
  // second only the down tasks, which then find h complete and wait for nothing)
  const int nA = a.phase >= 2 ? 0 : G * RAT, nB = a.phase == 1 ? 0 : H / DR;
  const bool waits = a.phase == 0 || a.phase == 3;   // the down phase waits for the start signal
  const int b0 = (int)blockIdx.x, gs = (int)gridDim.x;
  // the gate/up tasks go round-robin over the whole grid (the fewest per
  // compute unit at most); the down tasks start at workgroup nA % gs, the
  // first one with one gate/up task fewer
  const int myA = nA > b0 ? (nA - b0 + gs - 1) / gs : 0;
  const int tb0 = (b0 - nA % gs + gs) % gs;                               // my first down task
  const int myB = nB > tb0 ? (nB - tb0 + gs - 1) / gs : 0;

  // DR == 8: the down task's weights (every step of every wave) go into
  // registers when phase A is done, before the wait for the start signal
  const int rnkt = I / 32;
  const int rSB = (rnkt + 3) >> 2;               // down steps of 4 bricks
  const int rn = G * rSB;                        // 0: no pick on the GPU, no start signal comes
  const int rSWB = (rn + NW - 1) / NW;           // <= kDecResSteps (checked by the host)
  u32x4 wv2[DR == 8 ? kDecResSteps : 1][2];
  float f1[DR == 8 ? kDecResSteps : 1];
  // ================= phase A: gate/up + SwiGLU
  // A task is RG brick rows (RG x 16 gate/up rows) of one group: each step
  // loads the x operand once for all RG rows, so x is re-read from the
  // caches once per RG rows (it is as large as the FP8 weights of two rows
  // at T = 16; FP8 uses RG = 2, and RG = 4 from T = 8 on).
  {
    u32x4 wb[D][RG][2], ob[D][XN];   // weight bricks and x of D steps
    const int nkt = FP8 ? H / 64 : H / 32;
    const int S = (nkt + 1) >> 1;
    const int SW = (S + NW - 1) / NW;
    const int s_lo = wv * SW;
    const size_t gu_bytes = (size_t)2 * I * H * (FP8 ? 1 : 2);
    const int nsteps = myA * SW;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(T * H * 2));
    const __amdgpu_buffer_rsrc_t hw = make_rsrc(a.h, (uint32_t)(2u * a.G_max * kDecTok * I));
    const __amdgpu_buffer_rsrc_t gow = make_rsrc(c.go, (uint32_t)(4u * kDecGridMax * kCtrlStride));
    float sb[D][2];
    int i_tk = 0, i_l = 0;
    auto issue = [&](int d) {
      const int task = b0 + i_tk * gs;
      const int s = s_lo + i_l;
      const bool ok = i_tk < myA && s < S;
      const int tt = ok ? task : 0;
      const int g = tt / RAT, t = (tt - g * RAT) * RG;   // first brick row of the task
      const int slot = ok ? __builtin_amdgcn_readfirstlane(s_gslot[g]) : 0;   // slot 0 always exists
      const __amdgpu_buffer_rsrc_t wr =
          make_rsrc((const char*)a.w_gu + (size_t)slot * gu_bytes + (size_t)t * nkt * 1024,
                    (uint32_t)(RG * nkt * 1024));
      const uint32_t wo = oob_sel(ok, (uint32_t)s * 2048u + lane * 16u);
#pragma unroll
      for (int rr = 0; rr < RG; ++rr) {
        wb[d][rr][0] = bload_nt(wr, oob_sel(ok, wo + (uint32_t)(rr * nkt * 1024)));
        wb[d][rr][1] = bload_nt(wr, oob_sel(ok, wo + (uint32_t)(rr * nkt * 1024) + 1024u));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int k0 = FP8 ? 128 * s + 64 * b : 64 * s + 32 * b;
        const bool xo = ok && tok && k0 < H;
        const uint32_t off = oob_sel(xo, (uint32_t)(r * H + k0 + (FP8 ? 16 : 8) * j) * 2u);
        if (FP8) {
          ob[d][2 * b] = bload(xr, off);
          ob[d][2 * b + 1] = bload(xr, oob_sel(xo, off + 16u));
        } else {
          ob[d][b] = bload(xr, off);
        }
      }
      if (FP8) {   // block scales of the gate rows and of the up rows at this K step (one 128-row
                   // block holds every row of the task: 16 brick rows share it and RG divides 16)
        const size_t si = ((size_t)slot * (I / 128) + (8 * t) / 128) * (H / 128) + (ok ? s : 0);
        sb[d][0] = a.s_gate[si];
        sb[d][1] = a.s_up[si];
      }
      if (++i_l == SW) {
        i_l = 0;
        ++i_tk;
      }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    f32x4 acc[RG];
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) acc[rr] = f32x4{0, 0, 0, 0};
    int c_tk = 0, c_l = 0;
    for (int i0 = 0; i0 < nsteps; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (i0 + d < nsteps) {
#pragma unroll
          for (int rr = 0; rr < RG; ++rr) {
            if (!FP8) {
              acc[rr] = mfma16x16x32(wb[d][rr][0], ob[d][0], acc[rr]);
              acc[rr] = mfma16x16x32(wb[d][rr][1], ob[d][1], acc[rr]);
            } else {
              f32x4 p = {0, 0, 0, 0};
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                u32x4 lo, hi;
                e4m3x16_to_bf16_nat(wb[d][rr][b], lo, hi);
                p = mfma16x16x32(lo, ob[d][2 * b], p);
                p = mfma16x16x32(hi, ob[d][2 * b + 1], p);
              }
              const float sc = j < 2 ? sb[d][0] : sb[d][1];
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[rr][q] += sc * p[q];
            }
          }
          if (c_l == SW - 1) {   // end of a task: reduce over the waves, SwiGLU, h, count
            const int task = b0 + c_tk * gs;
            const int g = task / RAT, t = (task - g * RAT) * RG;
            f32x4(&rb)[NW][64] = red[c_tk & 1];
            rb[wv][lane] = acc[0];
            if constexpr (RG > 1) redB[c_tk & 1][wv][lane] = acc[1];
            if constexpr (RG == 4) {
              red4[0][wv][lane] = acc[2];
              red4[1][wv][lane] = acc[3];
            }
            __syncthreads();
            // a brick row's partials summed over the waves (gate lanes j < 2,
            // the up value of the same feature at lane + 32)
            auto row_sum = [&](auto& rx, f32x4& Gv, f32x4& Uv) {
              Gv = rx[0][lane];
              Uv = rx[0][lane + 32];
#pragma unroll
              for (int w2 = 1; w2 < NW; ++w2) {
                Gv += rx[w2][lane];
                Uv += rx[w2][lane + 32];
              }
            };
            f32x4 G4[RG == 4 ? 2 : 1], U4[RG == 4 ? 2 : 1];
            if constexpr (RG == 4) {
              if (wv == 0 && j < 2) {
                row_sum(red4[0], G4[0], U4[0]);
                row_sum(red4[1], G4[1], U4[1]);
              }
              __syncthreads();   // red4 is free for the next task's partials
            }
            if (wv == 0) {
              // SwiGLU of one brick row's sums, store its h
              auto row_emit = [&](const f32x4& Gv, const f32x4& Uv, int rr) {
                const uint32_t h01 = f32_to_bf16_rne(silu_f32(Gv[0]) * Uv[0]) |
                                     ((uint32_t)f32_to_bf16_rne(silu_f32(Gv[1]) * Uv[1]) << 16);
                const uint32_t h23 = f32_to_bf16_rne(silu_f32(Gv[2]) * Uv[2]) |
                                     ((uint32_t)f32_to_bf16_rne(silu_f32(Gv[3]) * Uv[3]) << 16);
                // device-coherent store (written through to memory), so no L2 write-back is needed
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{h01, h23}, hw, (uint32_t)((((size_t)g * kDecTok + r) * I + 8 * (t + rr) + 4 * j) * 2), 0, 16);
              };
              auto row_out = [&](auto& rx, int rr) {
                f32x4 Gv, Uv;
                row_sum(rx, Gv, Uv);
                row_emit(Gv, Uv, rr);
              };
              if (j < 2 && tok) {
                row_out(red[c_tk & 1], 0);
                if constexpr (RG > 1) row_out(redB[c_tk & 1], 1);
                if constexpr (RG == 4) {
                  row_emit(G4[0], U4[0], 2);
                  row_emit(G4[1], U4[1], 3);
                }
              }
              __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the stores above have completed
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // and stay before the count
              bool last = false;
              if (lane == 0 && atomicAdd(&c.done[g * kCtrlStride], 1u) == (uint32_t)RAT - 1u) {
                // no other task of g is left: clear its counter for the next launch
                __hip_atomic_store(&c.done[g * kCtrlStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = atomicAdd(c.all, 1u) == (uint32_t)G - 1u;
                if (last) __hip_atomic_store(c.all, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
              if (__ballot(last)) {   // every group is done: start the down phase
                // one store per workgroup holding a down task (a second store
                // could land after that workgroup cleared its flag)
                for (int bb = lane; bb < gs; bb += 64)
                  if ((bb - nA % gs + gs) % gs < nB)
                    __builtin_amdgcn_raw_buffer_store_b32(1u, gow, (uint32_t)(bb * kCtrlStride * 4), 0, 16);
              }
            }
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) acc[rr] = f32x4{0, 0, 0, 0};
            c_l = 0;
            ++c_tk;
          } else {
            ++c_l;
          }
        }
        issue(d);
      }
    }
  }
  if constexpr (DR == 8) {
    const size_t dn_bytes = (size_t)H * I * 2;
    const int t = tb0;
    const int t16 = t >> 1;
    const uint32_t lo = (uint32_t)(r >> 3) * 1024u + (uint32_t)(16 * j + 8 * (t & 1) + (r & 7)) * 16u;
#pragma unroll
    for (int d = 0; d < kDecResSteps; ++d) {
      const int q = wv * rSWB + d;
      const bool ok = myB > 0 && d < rSWB && q < rn;
      const int qq = ok ? q : 0;
      const int g = qq / rSB, s = qq - g * rSB;
      const int slot = ok ? __builtin_amdgcn_readfirstlane(s_gslot[g]) : 0;
      const __amdgpu_buffer_rsrc_t wr =
          make_rsrc((const char*)a.w_down + (size_t)slot * dn_bytes + (size_t)t16 * rnkt * 1024, (uint32_t)(rnkt * 1024));
      const uint32_t wo = oob_sel(ok, (uint32_t)s * 4096u + lo);
      wv2[d][0] = bload_nt(wr, wo);
      wv2[d][1] = bload_nt(wr, oob_sel(ok, wo + 2048u));
      f1[d] = ok ? s_gw[g * kDecTok + r] : 0.f;
    }
  }

  // ================= phase B: down projection + gate weights (+ merge)
  if (DR == 8 && myB > 0) {
    // one 8-row task (myB == 1): rows 8t .. 8t+7 of y; its weights are in wv2
    const int t = tb0;
    f32x4 yh = {0, 0, 0, 0};
    if (wv == 0 && a.y_host && tok && j < 2)
      yh = *reinterpret_cast<const f32x4*>(a.y_host + (size_t)r * H + 8 * t + 4 * j);
    if (wv == 0 && rn > 0 && waits) {   // wait for the start signal of the down phase (bounded)
      uint32_t* flag = c.go + (size_t)b0 * kCtrlStride;
      uint32_t it = 0;
      for (;;) {
        uint32_t v = 0;
        if (lane == 0) v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__shfl(v, 0, 64)) break;
        if (++it >= a.poll_limit) {
          if (lane == 0) atomicOr(c.err, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      if (lane == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // no acquire fence (on gfx950 an L2 invalidate): h is read below with
      // device-scope loads, which see the write-through h stores of other XCDs
    }
    __syncthreads();
    // h rows of the T tokens of every group -> LDS [g][t][I]: every load of a
    // thread (16 bytes each, at most kHL) is issued before the first LDS write
    {
      constexpr int kHL = kDecResH / 16 / (NW * 64);
      const int n16 = G * T * (I / 8);
      const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.h, (uint32_t)(2u * a.G_max * kDecTok * I));
      u32x4 hv[kHL];
#pragma unroll
      for (int u = 0; u < kHL; ++u) {
        const int i = tid + u * NW * 64;
        const int row = i / (I / 8), k8 = i - row * (I / 8);
        const int g = row / T, tt = row - g * T;
        hv[u] = bload_dev(hr, oob_sel(i < n16, (uint32_t)(((g * kDecTok + tt) * I + 8 * k8) * 2)));
      }
#pragma unroll
      for (int u = 0; u < kHL; ++u) {
        const int i = tid + u * NW * 64;
        if (i < n16) *reinterpret_cast<u32x4*>(&s_h[(size_t)i * 8]) = hv[u];
      }
    }
    __syncthreads();
    // A 16-byte load of a step holds the 8-row slices of two bricks (the first
    // in the accumulator's rows 0-7, the second in rows 8-15).  Against the h
    // of the first brick, rows 0-7 of the product are that brick's sums (rows
    // 8-15 are unused products); against the h of the second, rows 8-15 are.
    // acc_e and acc_o collect the two, and the valid halves are added at the
    // end.  Lanes of tokens >= T read token 0's h: their columns are never
    // stored.  Missing steps and bricks past I are skipped by uniform branches.
    f32x4 acc_e = {0, 0, 0, 0}, acc_o = {0, 0, 0, 0};
    const u32x4 z = {0, 0, 0, 0};
    const int hl = (tok ? r : 0) * I + 8 * j;
#pragma unroll
    for (int d = 0; d < kDecResSteps; ++d) {
      const int q = wv * rSWB + d;
      if (d < rSWB && q < rn) {
        const int g = q / rSB, s = q - g * rSB;
        const uint16_t* hg = s_h + (size_t)g * T * I + hl;
        u32x4 hb[4];   // h of bricks 4s .. 4s+3 (zero past I)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int k0 = 32 * (4 * s + b);
          const u32x4 v = *reinterpret_cast<const u32x4*>(hg + (k0 < I ? k0 : 0));   // in the row either way
          hb[b] = k0 < I ? v : z;
        }
        f32x4 pe = mfma16x16x32(wv2[d][0], hb[0], f32x4{0, 0, 0, 0});
        f32x4 po = mfma16x16x32(wv2[d][0], hb[1], f32x4{0, 0, 0, 0});
        pe = mfma16x16x32(wv2[d][1], hb[2], pe);
        po = mfma16x16x32(wv2[d][1], hb[3], po);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc_e[e] += f1[d] * pe[e];
          acc_o[e] += f1[d] * po[e];
        }
      }
    }
    const f32x4 acc = j < 2 ? acc_e : acc_o;   // rows 0-7 of acc_e, rows 8-15 of acc_o
    // sum the waves' partials (rows 0-7 and 8-15 of each) in a fixed order, store y
    f32x4(&rb)[NW][64] = red[0];
    rb[wv][lane] = acc;
    __syncthreads();
    if (wv == 0 && tok && j < 2) {
      f32x4 Y = rb[0][lane] + rb[0][lane + 32];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) Y += rb[w2][lane] + rb[w2][lane + 32];
      const size_t o = (size_t)r * H + 8 * t + 4 * j;
      if (a.y) *reinterpret_cast<f32x4*>(a.y + o) = Y;
      if (a.y_out) {
        const f32x4 M = Y + yh;
        *reinterpret_cast<f32x4*>(a.y_out + o) = M;
        if (a.y_bf16) {
          const uint32_t lo2 = f32_to_bf16_rne(M[0]) | ((uint32_t)f32_to_bf16_rne(M[1]) << 16);
          const uint32_t hi2 = f32_to_bf16_rne(M[2]) | ((uint32_t)f32_to_bf16_rne(M[3]) << 16);
          *reinterpret_cast<u32x2*>(a.y_bf16 + o) = u32x2{lo2, hi2};
        }
      }
    }
  } else if (myB > 0) {
    // A down task is NRB brick rows of y: each step loads the h operand once
    // for all of them (at T = 16, h is twice the FP8 weight bytes per row).
    u32x4 wb[D][NRB][2], ob[D][XN];   // weight bricks and h of D steps
    const int nkt = FP8 ? I / 64 : I / 32;
    const int SB = (nkt + 1) >> 1;
    const int n = G * SB;                       // (group, K step) pairs of every task
    const int SWB = (n + NW - 1) / NW;          // of one wave
    const size_t dn_bytes = (size_t)H * I * (FP8 ? 1 : 2);
    const int nsteps = myB * SWB;
    const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.h, (uint32_t)(2u * a.G_max * kDecTok * I));
    float fb[D];
    int qg[D], qs[D];
    bool qok[D];
    int i_tk = 0, i_l = 0;
    auto issue_w = [&](int d) {   // weights of the next step; remembers its (group, step)
      const int t = tb0 + i_tk * gs;   // DR-row block of y
      const int q = wv * SWB + i_l;
      const bool ok = i_tk < myB && q < n;
      const int qq = ok ? q : 0;
      const int g = qq / SB, s = qq - g * SB;
      const int slot = ok ? __builtin_amdgcn_readfirstlane(s_gslot[g]) : 0;
      const int tr = ok ? t : 0;
      const __amdgpu_buffer_rsrc_t wr = make_rsrc(
          (const char*)a.w_down + (size_t)slot * dn_bytes + (size_t)tr * NRB * nkt * 1024, (uint32_t)(NRB * nkt * 1024));
      const uint32_t wo = oob_sel(ok, (uint32_t)s * 2048u + lane * 16u);
#pragma unroll
      for (int rr = 0; rr < NRB; ++rr) {
        wb[d][rr][0] = bload_nt(wr, oob_sel(ok, wo + (uint32_t)(rr * nkt * 1024)));
        wb[d][rr][1] = bload_nt(wr, oob_sel(ok, wo + (uint32_t)(rr * nkt * 1024) + 1024u));
      }
      float f = ok ? s_gw[g * kDecTok + r] : 0.f;
      // (the NRB brick rows lie in one 128-row scale block: 16 NRB divides 128)
      if (FP8) f *= a.s_down[((size_t)slot * (H / 128) + (16 * NRB * tr) / 128) * (I / 128) + s];
      fb[d] = f;
      qg[d] = g;
      qs[d] = s;
      qok[d] = ok;
      if (++i_l == SWB) {
        i_l = 0;
        ++i_tk;
      }
    };
    auto issue_h = [&](int d) {   // the h operand of the step issue_w(d) took
      const int g = qg[d], s = qs[d];
      const uint32_t hrow = (uint32_t)((g * kDecTok + r) * I);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int k0 = FP8 ? 128 * s + 64 * b : 64 * s + 32 * b;
        const bool ho = qok[d] && tok && k0 < I;
        const uint32_t off = oob_sel(ho, (hrow + k0 + (FP8 ? 16 : 8) * j) * 2u);
        if (FP8 && HDEV) {
          ob[d][2 * b] = bload_dev(hr, off);
          ob[d][2 * b + 1] = bload_dev(hr, oob_sel(ho, off + 16u));
        } else if (FP8) {
          ob[d][2 * b] = bload(hr, off);
          ob[d][2 * b + 1] = bload(hr, oob_sel(ho, off + 16u));
        } else {
          ob[d][b] = bload(hr, off);
        }
      }
    };
    // the end of a task: sum the waves' partials in wave order, store y
    // and the merged output (lanes 16j + r: token r, rows DR t + 16 rr + 4j .. + 3)
    f32x4 yh[NRB];   // host partial of the current task (wave 0)
#pragma unroll
    for (int rr = 0; rr < NRB; ++rr) yh[rr] = f32x4{0, 0, 0, 0};
    auto load_yh = [&](int tk) {
      if (wv == 0 && a.y_host && tok) {
        const int t = tb0 + tk * gs;
#pragma unroll
        for (int rr = 0; rr < NRB; ++rr)
          yh[rr] = *reinterpret_cast<const f32x4*>(a.y_host + (size_t)r * H + DR * t + 16 * rr + 4 * j);
      }
    };
    auto finish = [&](int tk, const f32x4 (&acc)[NRB]) {
      const int t = tb0 + tk * gs;
      red[tk & 1][wv][lane] = acc[0];
      if constexpr (NRB > 1) redB[tk & 1][wv][lane] = acc[NRB - 1];
      __syncthreads();
      auto out_row = [&](auto& rb, int rr) {
        f32x4 Y = rb[0][lane];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) Y += rb[w2][lane];
        const size_t o = (size_t)r * H + DR * t + 16 * rr + 4 * j;
        if (a.y) *reinterpret_cast<f32x4*>(a.y + o) = Y;
        if (a.y_out) {
          const f32x4 M = Y + yh[rr];
          *reinterpret_cast<f32x4*>(a.y_out + o) = M;
          if (a.y_bf16) {
            const uint32_t lo = f32_to_bf16_rne(M[0]) | ((uint32_t)f32_to_bf16_rne(M[1]) << 16);
            const uint32_t hi = f32_to_bf16_rne(M[2]) | ((uint32_t)f32_to_bf16_rne(M[3]) << 16);
            *reinterpret_cast<u32x2*>(a.y_bf16 + o) = u32x2{lo, hi};
          }
        }
      };
      if (wv == 0 && tok) {
        out_row(red[tk & 1], 0);
        if constexpr (NRB > 1) out_row(redB[tk & 1], 1);
      }
    };
    if (SWB == 0) {   // no pick on the GPU: y = 0, y_out = y_host
      f32x4 z[NRB];
#pragma unroll
      for (int rr = 0; rr < NRB; ++rr) z[rr] = f32x4{0, 0, 0, 0};
      for (int tk = 0; tk < myB; ++tk) {
        load_yh(tk);
        finish(tk, z);
      }
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) issue_w(d);
      load_yh(0);
      // wait for the start signal of the down phase (bounded)
      if (wv == 0 && waits) {
        uint32_t* flag = c.go + (size_t)b0 * kCtrlStride;
        uint32_t it = 0;
        for (;;) {
          uint32_t v = 0;
          if (lane == 0) v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (__shfl(v, 0, 64)) break;
          if (++it >= a.poll_limit) {
            if (lane == 0) atomicOr(c.err, 1u);
            break;
          }
          __builtin_amdgcn_s_sleep(16);
        }
        if (lane == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // h written on other XCDs is read from memory: one L2 invalidate per
        // workgroup, then ordinary loads that the XCD's L2 serves to every
        // down workgroup on it (device-scope loads re-read h from memory each
        // time, which costs more than the invalidate once T is large; HDEV
        // takes them instead)
        if constexpr (!HDEV) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
#pragma unroll
      for (int d = 0; d < D; ++d) issue_h(d);
      f32x4 acc[NRB];
#pragma unroll
      for (int rr = 0; rr < NRB; ++rr) acc[rr] = f32x4{0, 0, 0, 0};
      int c_tk = 0, c_l = 0;
      for (int i0 = 0; i0 < nsteps; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          if (i0 + d < nsteps) {
            const float f = fb[d];
#pragma unroll
            for (int rr = 0; rr < NRB; ++rr) {
              f32x4 p = {0, 0, 0, 0};
              if (!FP8) {
                p = mfma16x16x32(wb[d][rr][0], ob[d][0], p);
                p = mfma16x16x32(wb[d][rr][1], ob[d][1], p);
              } else {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                  u32x4 lo, hi;
                  e4m3x16_to_bf16_nat(wb[d][rr][b], lo, hi);
                  p = mfma16x16x32(lo, ob[d][2 * b], p);
                  p = mfma16x16x32(hi, ob[d][2 * b + 1], p);
                }
              }
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[rr][q] += f * p[q];
            }
            if (c_l == SWB - 1) {
              finish(c_tk, acc);
#pragma unroll
              for (int rr = 0; rr < NRB; ++rr) acc[rr] = f32x4{0, 0, 0, 0};
              c_l = 0;
              ++c_tk;
              if (c_tk < myB) load_yh(c_tk);
            } else {
              ++c_l;
            }
          }
          issue_w(d);
          issue_h(d);
        }
      }
    }
  }
}

// ================================================================ prefill
// (token, pick) pairs are counting-sorted by slot in three launches (per
// workgroup histograms, one scan, scatter), then two grouped GEMMs walk a
// tile list: tile = (slot, 128 or 64 sorted pairs) x (512 bank rows).  The
// weight bricks are the MFMA A operand and the tokens' rows the B operand;
// both go from memory straight into LDS stages.  Each wave owns 128 bank
// rows, so the accumulator of a lane holds 4 consecutive bank
// rows of one token: SwiGLU pairs a gate lane with the up lane 32 away, and
// the outputs leave registers as 8-byte stores.  Gate/up writes h [P][I]
// (BF16); down writes the gate-weighted rows o [P][H] (BF16); a last launch
// sums each token's k rows in pick order.
constexpr int kSortChunk = 2048;   // least pairs per counting workgroup
constexpr int kSortMaxChunks = 32; // counting workgroups at most
constexpr int kSortMaxSlots = 4096;
constexpr int kPfRows = 512;       // bank rows per tile (8 waves x 64)

struct PfArgs {
  const void* w_gu;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int H, I, n_slots, T, k, P, tm, max_mtiles, chunk;
  const uint16_t* x;
  const int32_t* pick_slot;
  const float* w;
  float* y;              // [T][H] GPU partial sum, or NULL
  const float* y_host;   // merge: [T][H] host partial sum, or NULL
  float* y_out;          // merge: y + y_host, or NULL
  uint16_t* y_bf16;      // merge: BF16 of y_out, or NULL
  // workspace
  int32_t* hist;         // [n_chunks][n_slots] counts, then bases
  int32_t* cnt;          // [n_slots]
  int32_t* off;          // [n_slots]
  int32_t* mtoff;        // [n_slots] first M tile of each slot
  int32_t* n_mtiles;     // [1]
  int32_t* tile_slot;    // [max_mtiles]
  int32_t* tile_m0;      // [max_mtiles]
  int32_t* sorted_pair;  // [P]
  int32_t* pair_pos;     // [P]
  uint16_t* h;           // [P][I] BF16
  uint16_t* o;           // [P][H] BF16
};

// pass 1: histogram of the chunk's pairs by slot
__global__ __launch_bounds__(256) void pf_count_kernel(PfArgs a) {
  __shared__ int hs[kSortMaxSlots];
  const int tid = threadIdx.x, S = a.n_slots;
  for (int s = tid; s < S; s += 256) hs[s] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * a.chunk, p1 = min(a.P, p0 + a.chunk);
  for (int p = p0 + tid; p < p1; p += 256) {
    const int s = a.pick_slot[p];
    if (s >= 0 && s < S) atomicAdd(&hs[s], 1);
  }
  __syncthreads();
  int32_t* row = a.hist + (size_t)blockIdx.x * S;
  for (int s = tid; s < S; s += 256) row[s] = hs[s];
}

// pass 2 (one workgroup): slot totals and segment offsets, per-chunk bases
// (hist is overwritten with the first sorted position of each chunk's pairs
// of each slot), and the list of M tiles (slot, first row) in slot order.
// Thread t takes the R = ceil(S / 1024) consecutive slots from t R; each
// slot's column of chunk counts is read with raw buffer loads whose offset
// leaves the buffer for a missing chunk (reading zero), so a column's loads
// issue back to back.  n_chunks * S <= kSortMaxChunks * kSortMaxSlots keeps
// every byte offset below the out-of-range one.
__global__ __launch_bounds__(1024) void pf_scan_kernel(PfArgs a, int n_chunks) {
  __shared__ int wsum[16], wsum2[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int S = a.n_slots, TM = a.tm;
  static_assert(kSortMaxSlots <= 4 * 1024, "four slots per thread at most");
  const int R = (S + 1023) / 1024;   // at most kSortMaxSlots / 1024 = 4
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.hist, (uint32_t)(4u * n_chunks * S));
  auto column = [&](int s, int (&col)[kSortMaxChunks]) {
#pragma unroll
    for (int w = 0; w < kSortMaxChunks; ++w)
      col[w] = (int)__builtin_amdgcn_raw_buffer_load_b32(
          hr, (int)oob_sel(s < S && w < n_chunks, (uint32_t)((w * S + s) * 4)), 0, 0);
  };
  int c[4], tc[4], ls = 0, lt = 0;
  for (int i = 0; i < 4; ++i) {
    c[i] = tc[i] = 0;
    if (i >= R) continue;
    int col[kSortMaxChunks];
    column(tid * R + i, col);
    int v = 0;
#pragma unroll
    for (int w = 0; w < kSortMaxChunks; ++w) v += col[w];
    c[i] = v;
    tc[i] = (v + TM - 1) / TM;
    ls += v;
    lt += tc[i];
  }
  int is = ls, it = lt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o1 = __shfl_up(is, d, 64), o2 = __shfl_up(it, d, 64);
    if (lane >= d) {
      is += o1;
      it += o2;
    }
  }
  if (lane == 63) {
    wsum[wv] = is;
    wsum2[wv] = it;
  }
  __syncthreads();
  int bs = 0, bt = 0;
  for (int w = 0; w < wv; ++w) {
    bs += wsum[w];
    bt += wsum2[w];
  }
  int es = bs + is - ls, et = bt + it - lt;   // exclusive prefix of this thread's first slot
  for (int i = 0; i < R; ++i) {
    const int s = tid * R + i;
    if (s < S) {
      a.cnt[s] = c[i];
      a.off[s] = es;
      a.mtoff[s] = et;
      int col[kSortMaxChunks];
      column(s, col);
      int b = es;
#pragma unroll
      for (int w = 0; w < kSortMaxChunks; ++w)
        if (w < n_chunks) {
          a.hist[(size_t)w * S + s] = b;
          b += col[w];
        }
      for (int q = 0; q < tc[i]; ++q)
        if (et + q < a.max_mtiles) {
          a.tile_slot[et + q] = s;
          a.tile_m0[et + q] = q * TM;
        }
    }
    es += c[i];
    et += tc[i];
  }
  if (tid == 1023) *a.n_mtiles = min(et, a.max_mtiles);
}

// pass 3: scatter each chunk's pairs to their sorted positions
__global__ __launch_bounds__(256) void pf_scatter_kernel(PfArgs a) {
  __shared__ int cur[kSortMaxSlots];
  const int tid = threadIdx.x, S = a.n_slots;
  const int32_t* row = a.hist + (size_t)blockIdx.x * S;
  for (int s = tid; s < S; s += 256) cur[s] = row[s];
  __syncthreads();
  const int p0 = blockIdx.x * a.chunk, p1 = min(a.P, p0 + a.chunk);
  for (int p = p0 + tid; p < p1; p += 256) {
    const int s = a.pick_slot[p];
    int pos = -1;
    if (s >= 0 && s < S) {
      pos = atomicAdd(&cur[s], 1);
      a.sorted_pair[pos] = p;
    }
    a.pair_pos[p] = pos;
  }
}

// Grouped GEMM.  Tile = (M tile of one slot: TM sorted pairs) x (512 bank
// rows).  Eight waves, two per SIMD; wave w owns bank rows [64 w, 64 w + 64)
// of the tile (four brick rows) against every pair of the tile, so no two
// waves need the same weights.  K advances one weight brick per step.
// The weight bricks are already MFMA A-operand images: each wave streams its
// four bricks of a step from memory straight into registers (one contiguous
// 1 KB wave load each), D steps ahead of the MFMAs in a register ring.  Only
// the token operand goes through LDS: the token bricks of SPS steps form a
// stage, loaded from memory straight into LDS (buffer loads with an LDS
// destination; FP8: lane (r, j) of a token brick fetches 16 bytes of its
// pair's row, so the LDS image is the B operand; BF16: a stage's loads
// fetch whole 128-byte lines of the rows into a swizzled image, described
// at pf_line_row), NSTG stages deep, one barrier per stage.  A wave reads
// the token bricks of step st+1 from LDS while the
// MFMAs of step st run (each brick's register is re-read right after the
// MFMAs that take it are issued).  FP8: a weight brick is 64 K of E4M3
// codes, expanded exactly to two BF16 operands in registers; the partial
// sums of a 128-K scale block (two steps) are multiplied by the block's
// scale once (post-scaling).  Every load past the last step, or of a pair
// row past the tile's, is a buffer load pushed out of range: it returns
// zeros without touching memory, so each wave issues the same loads on every
// step and the waits are constants.  Tiles are ordered (slot, bank-row
// block, M tile) and taken in order per XCD (workgroup b runs on XCD b % 8),
// so the M tiles sharing a block of weights run side by side and share it
// through that XCD's L2.
typedef __attribute__((address_space(3))) void* lds_ptr;
template <int AUX>
__device__ __forceinline__ void bload_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, AUX);
}
constexpr int kPfWaves = 8;
constexpr int kPfWaveRows = kPfRows / kPfWaves;   // 64 bank rows (four brick rows) per wave

// BF16 token stages in whole lines.  The two steps of a stage take 64 K of
// each pair row: one 128-byte line.  A token brick with lane (r, j) fetching
// 16 bytes per step would ask for 16 half lines per load; instead load s of
// a stage brings rows 8 s .. 8 s + 7 of the wave's token group, eight lanes
// a row and every line whole.  Such a load writes its 1 KB of LDS in lane
// order, so the lane -> (row, chunk) map sets the image, and the 16-byte
// chunks are XOR-swizzled by the row so that the operand reads of one step
// (lane (r, j) takes chunk 4 s + j of row r) fall on distinct banks in every
// 8 and every 16 lanes: chunk c of row 8 u + q sits in 16-byte slot
// 64 u + 8 (q ^ u) + (c ^ q) of the group's 2 KB.
__device__ __forceinline__ int pf_line_row(int lane, int u) { return 8 * u + ((lane >> 3) ^ u); }
__device__ __forceinline__ int pf_line_chunk(int lane, int u) { return (lane & 7) ^ ((lane >> 3) ^ u); }
__device__ __forceinline__ uint32_t pf_line_slot(int lane, int s) {   // the operand slot of lane (r, j) at step s
  const int r = lane & 15, j = lane >> 4, u = r >> 3, q = r & 7;
  return (uint32_t)(64 * u + 8 * (q ^ u) + ((4 * s + j) ^ q));
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(kPfWaves * 64, 1) void pf_gemm_kernel(PfArgs a) {
  constexpr int TM = FP8 ? 64 : 128;         // pairs per tile
  constexpr int NTG = TM / 16;               // token groups (MFMA N blocks)
  constexpr int TBS = FP8 ? 2 * NTG : NTG;   // token bricks per step (FP8: K halves of 32)
  constexpr int KS = FP8 ? 64 : 32;          // K per step = one weight brick
  constexpr int WB = kPfWaveRows / 16;       // weight brick rows per wave
  constexpr int SPS = 2;                     // steps per LDS stage (one barrier each)
  constexpr int NSTG = 4;                    // stages in LDS
  constexpr int D = FP8 ? 2 : 4;             // weight register ring, in steps (FP8 also holds the block sums)
  constexpr int SB = SPS * TBS;              // token bricks per stage
  static_assert(TBS == kPfWaves, "each wave loads one token brick per step: SPS per stage");
  static_assert(SPS == 2 && (FP8 || SPS * KS * 2 == 128), "a BF16 stage spans one 128-byte line of each row");
  static_assert(D % SPS == 0, "a loop body of D steps holds whole stages");
  __shared__ __attribute__((aligned(1024))) char Ls[NSTG][SB * 1024];

  const int K = GATEUP ? a.H : a.I;
  const int NROWS = GATEUP ? 2 * a.I : a.H;           // bank rows
  const int NB = (NROWS + kPfRows - 1) / kPfRows;
  const int ntiles = *a.n_mtiles * NB;
  const int Q = (ntiles + 7) / 8;
  const int xcd = blockIdx.x & 7, sq = blockIdx.x >> 3;
  if (sq >= Q) return;
  const int tau = xcd * Q + sq;
  if (tau >= ntiles) return;
  // tau / NB falls inside the slot's run of M tiles because each slot's
  // block of tiles is NB times its M tiles.
  const int slot = a.tile_slot[tau / NB];
  const int nm = (a.cnt[slot] + TM - 1) / TM;
  const int lam = tau - a.mtoff[slot] * NB;
  const int nb = lam / nm, mt = a.mtoff[slot] + (lam - nb * nm);
  const int m0 = a.tile_m0[mt];
  const int seg = a.off[slot];
  const int mrows = min(TM, a.cnt[slot] - m0);
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nkt = K / KS;                                  // steps
  const int row0 = nb * kPfRows + kPfWaveRows * wv;        // first bank row of this wave
  const bool rows_ok = row0 < NROWS;                       // NROWS is a multiple of 128
  const int t0 = rows_ok ? row0 / 16 : 0;                  // first brick row of this wave

  const size_t bank_bytes = (size_t)(GATEUP ? 2 : 1) * a.I * a.H * (FP8 ? 1 : 2);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc((const char*)(GATEUP ? a.w_gu : a.w_down) + (size_t)slot * bank_bytes +
                                                   (size_t)t0 * nkt * 1024,
                                               rows_ok ? (uint32_t)(WB * nkt * 1024) : 0u);
  const uint16_t* tsrc = GATEUP ? a.x : a.h;
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(tsrc, (uint32_t)((size_t)(GATEUP ? a.T : a.P) * K * 2));
  // This wave's token brick of every step: brick q = wv (BF16: token group
  // wv; FP8: group wv / 2, K half wv & 1).  Lane (r, j) fetches 16 bytes of
  // pair row 16 g + r: a row of x (gate/up: the pair's token) or of h (down:
  // the pair itself).  FP8 halves follow the expansion of a weight brick:
  // lane j of the low operand holds K 16 j .. 16 j + 7 of the step, of the
  // high one 16 j + 8 .. 16 j + 15.
  // BF16 stages hold whole lines instead (pf_line_row and the notes above
  // it): load s of a stage brings rows 8 s .. 8 s + 7 of group wv.
  int srow[SPS];
  uint32_t tkoff[SPS];
#pragma unroll
  for (int s = 0; s < SPS; ++s) {
    const int prow = 16 * (FP8 ? wv >> 1 : wv) + (FP8 ? r : pf_line_row(lane, s));
    srow[s] = prow < mrows ? (GATEUP ? a.sorted_pair[seg + m0 + prow] / a.k : seg + m0 + prow) : -1;
    tkoff[s] = FP8 ? (uint32_t)(16 * j + 8 * (wv & 1)) : (uint32_t)(8 * pf_line_chunk(lane, s));
  }
  auto issue_tok = [&](int sg) {   // stage sg -> LDS buffer sg % NSTG
    char* stage = Ls[sg % NSTG];
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      const int st = FP8 ? sg * SPS + s : sg * SPS;   // BF16: the stage's first step (the line spans both)
      bload_lds<0>(trs, stage + (FP8 ? s * TBS + wv : 2 * wv + s) * 1024,
                   oob_sel(srow[s] >= 0 && st < nkt,
                           (uint32_t)(((size_t)(srow[s] < 0 ? 0 : srow[s]) * K + st * KS + tkoff[s]) * 2)));
    }
  };
  u32x4 wr[D][WB];
  auto issue_w = [&](int st, u32x4 (&dst)[WB]) {   // weight bricks of step st (zeros past the last)
#pragma unroll
    for (int i = 0; i < WB; ++i) dst[i] = bload(wrs, oob_sel(st < nkt, (uint32_t)((i * nkt + st) * 1024 + lane * 16)));
  };
  // FP8 block scales: wave-uniform pointers read with scalar loads; gate/up
  // lanes j < 2 hold gate rows and j >= 2 up rows (32 features in one block)
  const float* scp = nullptr;
  const float* scq = nullptr;
  if (FP8) {
    const int nbk = K / 128;
    if (GATEUP) {
      const size_t o = ((size_t)slot * (a.I / 128) + (8 * t0) / 128) * nbk;
      scp = a.s_gate + o;
      scq = a.s_up + o;
    } else {
      scp = scq = a.s_down + ((size_t)slot * (a.H / 128) + (16 * t0) / 128) * nbk;
    }
  }
  float s_g = 0.f, s_u = 0.f;

  f32x4 acc[WB][NTG];
  f32x4 part[FP8 ? WB : 1][FP8 ? NTG : 1];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) acc[i][tg] = f32x4{0, 0, 0, 0};

  // Token operands are read from LDS with asm so that the compiler, which
  // cannot tell the stage being read from the stages still being filled by
  // the LDS-destination loads, does not wait for every load in flight; the
  // asm wait that follows ties the registers.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)&Ls[0][0];
  u32x4 tk[TBS];
  const uint32_t rofs[2] = {FP8 ? (uint32_t)lane * 16u : pf_line_slot(lane, 0) * 16u,
                            FP8 ? (uint32_t)lane * 16u : pf_line_slot(lane, 1) * 16u};
  auto rd_tok = [&](int st, int q) {
    const uint32_t addr = lds0 + (uint32_t)(((st / SPS) % NSTG) * SB * 1024 +
                                            (FP8 ? ((st % SPS) * TBS + q) * 1024 : q * 2048)) + rofs[st % SPS];
    asm volatile("ds_read_b128 %0, %1" : "=v"(tk[q]) : "v"(addr));
  };
  auto wait_tok = [&]() {   // every LDS read and scalar load issued so far has returned
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(tk[0]), "+v"(tk[1]), "+v"(tk[2]), "+v"(tk[3]), "+v"(tk[4]), "+v"(tk[5]), "+v"(tk[6]),
                   "+v"(tk[7]));
  };
  // Loads issued after the token loads of stage e + 1, at the end of stage e
  // (the wait may not exceed it): in the steady state the weights of
  // (NSTG - 1) SPS steps and the token loads of NSTG - 2 stages; at the
  // first stage ends, whose next stages came with the prologue, the
  // prologue's later token and weight loads plus WB per step run so far and
  // SPS per earlier stage end (that count grows by WB SPS per stage end).
  constexpr int kWaitSS = WB * SPS * (NSTG - 1) + SPS * (NSTG - 2);
  constexpr int kWait0 = SPS * (NSTG - 2) + WB * D + WB * (SPS - 1);
  constexpr int kWait1 = kWait0 + WB * SPS < kWaitSS ? kWait0 + WB * SPS : kWaitSS;
  constexpr int kWait2 = kWait1 + WB * SPS < kWaitSS ? kWait1 + WB * SPS : kWaitSS;
  static_assert(kWaitSS < 64, "vmcnt counts to 63");

  auto step = [&](int st, auto dc) {
    constexpr int d = decltype(dc)::value;                  // st % D
    constexpr bool ODD = (d & 1) != 0;                      // st % 2 (D is even)
    constexpr bool STAGE_END = (d % SPS) == SPS - 1;        // step st + 1 starts a new stage
    wait_tok();
    if constexpr (FP8 && ODD) asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(s_g), "+s"(s_u));   // the block's scales
    if constexpr (STAGE_END) {
      // the wait counts assume the loads stay in program order around it:
      // nothing is scheduled across this block
      __builtin_amdgcn_sched_barrier(0);
      const int e = st / SPS;                               // stage ending; stage e + 1 must be in
      if (e == 0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait0));
      else if (e == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait1));
      else if (e == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait2));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitSS));
      __builtin_amdgcn_s_barrier();
      issue_tok(e + NSTG);                                   // into the buffer of stage e, now free
      __builtin_amdgcn_sched_barrier(0);
    }
    if (st < nkt) {
      if constexpr (!FP8) {
#pragma unroll
        for (int q = 0; q < TBS; ++q) {
#pragma unroll
          for (int i = 0; i < WB; ++i) acc[i][q] = mfma16x16x32(wr[d][i], tk[q], acc[i][q]);
          rd_tok(st + 1, q);
        }
      } else {
        if constexpr (!ODD) {   // first step of a 128-K block: its two scales, zero partial sums
          asm volatile("s_load_dword %0, %1, 0x0" : "=s"(s_g) : "s"(scp + (st >> 1)));
          asm volatile("s_load_dword %0, %1, 0x0" : "=s"(s_u) : "s"(scq + (st >> 1)));
#pragma unroll
          for (int i = 0; i < WB; ++i)
#pragma unroll
            for (int tg = 0; tg < NTG; ++tg) part[i][tg] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {   // the low K halves of the step, then the high ones
          u32x4 op[WB];
#pragma unroll
          for (int i = 0; i < WB; ++i) {
            u32x4 lo, hi;
            e4m3x16_to_bf16_nat(wr[d][i], lo, hi);
            op[i] = h ? hi : lo;
          }
#pragma unroll
          for (int tg = 0; tg < NTG; ++tg) {
#pragma unroll
            for (int i = 0; i < WB; ++i) part[i][tg] = mfma16x16x32(op[i], tk[2 * tg + h], part[i][tg]);
            rd_tok(st + 1, 2 * tg + h);
          }
        }
        if constexpr (ODD) {
          const float sc = j < 2 ? s_g : s_u;
#pragma unroll
          for (int i = 0; i < WB; ++i)
#pragma unroll
            for (int tg = 0; tg < NTG; ++tg)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][tg][e] += sc * part[i][tg][e];
        }
      }
    }
    issue_w(st + D, wr[d]);
  };

  for (int sg = 0; sg < NSTG; ++sg) issue_tok(sg);
#pragma unroll
  for (int d = 0; d < D; ++d) issue_w(d, wr[d]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(SPS * (NSTG - 1) + WB * D));   // stage 0 is in
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int q = 0; q < TBS; ++q) rd_tok(0, q);
  const int nloop = (nkt + D - 1) / D * D;
  for (int st0 = 0; st0 < nloop; st0 += D) {
    step(st0, std::integral_constant<int, 0>{});
    step(st0 + 1, std::integral_constant<int, 1>{});
    if constexpr (D == 4) {
      step(st0 + 2, std::integral_constant<int, 2>{});
      step(st0 + 3, std::integral_constant<int, 3 % D>{});
    }
  }
  wait_tok();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load into LDS or registers outlives the loop
  if (!rows_ok) return;

  // ---- epilogue.  acc[i][tg][e] at lane (r, j): bank row 16 (t0 + i) + 4 j + e,
  // pair row 16 tg + r.
  if (GATEUP) {
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) {
      const int row = 16 * tg + r;
#pragma unroll
      for (int i = 0; i < WB; ++i) {
        // lanes j and j ^ 2 (32 apart) hold the gate and the up rows of the
        // same 4 features; each computes two of them: j < 2 the first two
        // (sending its gate of the last two), j >= 2 the last two (sending
        // its up of the first two), so every lane evaluates 2 SiLUs, not 4
        const f32x4 v = acc[i][tg];
        const bool lo = j < 2;
        const float r0 = __shfl_xor(lo ? v[2] : v[0], 32, 64), r1 = __shfl_xor(lo ? v[3] : v[1], 32, 64);
        const float g0 = lo ? v[0] : r0, g1 = lo ? v[1] : r1, u0 = lo ? r0 : v[2], u1 = lo ? r1 : v[3];
        if (row < mrows) {
          const int f = 8 * (t0 + i) + 4 * (j & 1) + (lo ? 0 : 2);   // the lane's first feature
          const uint32_t h01 = f32_to_bf16_rne(silu_f32(g0) * u0) | ((uint32_t)f32_to_bf16_rne(silu_f32(g1) * u1) << 16);
          *reinterpret_cast<uint32_t*>(a.h + (size_t)(seg + m0 + row) * a.I + f) = h01;
        }
      }
    }
  } else {
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) {
      const int row = 16 * tg + r;
      if (row < mrows) {
        const int pos = seg + m0 + row;
        const float wp = a.w[a.sorted_pair[pos]];
#pragma unroll
        for (int i = 0; i < WB; ++i) {
          const int c = 16 * (t0 + i) + 4 * j;
          const uint32_t o01 = f32_to_bf16_rne(wp * acc[i][tg][0]) | ((uint32_t)f32_to_bf16_rne(wp * acc[i][tg][1]) << 16);
          const uint32_t o23 = f32_to_bf16_rne(wp * acc[i][tg][2]) | ((uint32_t)f32_to_bf16_rne(wp * acc[i][tg][3]) << 16);
          *reinterpret_cast<u32x2*>(a.o + (size_t)pos * a.H + c) = u32x2{o01, o23};
        }
      }
    }
  }
}

// A wave-uniform pointer held in a vector register, moved to scalar registers.
__device__ __forceinline__ const float* uniform_ptr(const float* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const float*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Tiles per workgroup of the down GEMM at most (their descriptors and gate
// weights live in LDS).
template <bool FP8>
struct PfMeta {
  static constexpr int kTiles = FP8 ? 80 : 64;
};

// The down GEMM as a persistent kernel.  Its K (I) is short, so in the
// one-tile-per-workgroup form a tile's start (the first stages' latency)
// and end (the stores of its rows of o) took as long as its K steps.  Here
// a workgroup runs on each CU and walks its share of the tiles (every R-th
// tile of its XCD's run, so that neighbouring tiles still share their
// weights through the L2) as one pipeline: the token stages and the weight
// ring run on into the next tile while the MFMAs finish the current one,
// and a tile's stores drain while the next tile computes.  Each tile is the
// same computation as in pf_gemm_kernel (the same steps, the same order of
// the sums), so o is the same to the bit.
template <bool FP8>
__global__ __launch_bounds__(kPfWaves * 64, 1) void pf_down_kernel(PfArgs a) {
  constexpr int TM = FP8 ? 64 : 128;         // pairs per tile
  constexpr int NTG = TM / 16;               // token groups (MFMA N blocks)
  constexpr int TBS = FP8 ? 2 * NTG : NTG;   // token bricks per step (FP8: K halves of 32)
  constexpr int KS = FP8 ? 64 : 32;          // K per step = one weight brick
  constexpr int WB = kPfWaveRows / 16;       // weight brick rows per wave
  constexpr int SPS = 2;                     // steps per LDS stage (one barrier each)
  constexpr int NSTG = 4;                    // stages in LDS
  constexpr int D = 2;                       // weight register ring, in steps (2: the registers the
                                             // tile-to-tile state needs besides it)
  constexpr int SB = SPS * TBS;              // token bricks per stage
  constexpr int MT = PfMeta<FP8>::kTiles;    // tiles per workgroup at most
  static_assert(TBS == kPfWaves, "each wave loads one token brick per step: SPS per stage");
  static_assert(SPS == 2 && (FP8 || SPS * KS * 2 == 128), "a BF16 stage spans one 128-byte line of each row");
  static_assert(D % SPS == 0, "a loop body of D steps holds whole stages");
  __shared__ __attribute__((aligned(1024))) char Ls[NSTG][SB * 1024];
  __shared__ int4 s_desc[MT];                // per tile: slot, first sorted pair, pair rows, bank-row block
  __shared__ float s_wp[MT][TM];             // per tile and pair row: the pair's gate weight (0 past the tile)
  const auto desc = [&](int i) __attribute__((always_inline)) {             // a tile's descriptor, wave-uniform
    const int4 v = s_desc[i];
    return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
  };

  const int K = a.I;
  const int NROWS = a.H;                              // bank rows
  const int NB = (NROWS + kPfRows - 1) / kPfRows;
  const int ntiles = *a.n_mtiles * NB;
  const int Q = (ntiles + 7) / 8;
  const int R = (int)gridDim.x >> 3;                  // workgroups per XCD
  const int xcd = blockIdx.x & 7, sq = blockIdx.x >> 3;
  // my tiles: tau = xcd Q + sq + i R for i = 0, 1, ... (the XCD's run of
  // tiles, ordered (slot, bank-row block, M tile), dealt round-robin to its
  // workgroups, so neighbouring tiles share their weights through the L2)
  const int tlim = min(Q, ntiles - xcd * Q);
  const int nt_w = sq < tlim ? (tlim - sq + R - 1) / R : 0;
  if (nt_w == 0 || nt_w > MT) return;   // the host sizes the grid so that nt_w <= MT
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int nkt = K / KS;                                  // K steps of a tile
  const int nkp = (nkt + D - 1) / D * D;                   // the same padded to whole loop bodies
  const size_t bank_bytes = (size_t)a.I * a.H * (FP8 ? 1 : 2);

  // ---- metadata of every tile of this workgroup into LDS (once)
  for (int i = tid; i < nt_w; i += kPfWaves * 64) {
    const int tau = xcd * Q + sq + i * R;
    // tau / NB falls inside the slot's run of M tiles because each slot's
    // block of tiles is NB times its M tiles.
    const int slot = a.tile_slot[tau / NB];
    const int cnt = a.cnt[slot];
    const int nm = (cnt + TM - 1) / TM;
    const int lam = tau - a.mtoff[slot] * NB;
    const int nb = lam / nm, mt = a.mtoff[slot] + (lam - nb * nm);
    const int m0 = a.tile_m0[mt];
    s_desc[i] = make_int4(slot, a.off[slot] + m0, min(TM, cnt - m0), nb);
  }
  __syncthreads();
  for (int e = tid; e < nt_w * TM; e += kPfWaves * 64) {
    const int i = e / TM, p = e - i * TM;
    const int4 d4 = s_desc[i];
    s_wp[i][p] = p < d4.z ? a.w[a.sorted_pair[d4.y + p]] : 0.f;
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t trs = make_rsrc(a.h, (uint32_t)((size_t)a.P * K * 2));
  // Three streams walk the workgroup's steps (every tile's nkp steps in a
  // row): the token loads NSTG stages ahead, the weight loads D steps ahead,
  // and the MFMAs.  Each keeps its own tile, advanced when it crosses into
  // the next; loads of padding steps (k >= nkt) are pushed out of range.
  // Token stream: this wave's token brick of every step (brick q = wv; BF16:
  // token group wv, FP8: group wv / 2, K half wv & 1); lane (r, j) fetches 16
  // bytes of the h row of pair row 16 g + r.
  // BF16 stages hold whole lines (pf_line_row): load s of a stage brings
  // rows 8 s .. 8 s + 7 of group wv, for both steps of the stage.
  int prow[SPS];
  uint32_t tkoff[SPS];
#pragma unroll
  for (int s = 0; s < SPS; ++s) {
    prow[s] = 16 * (FP8 ? wv >> 1 : wv) + (FP8 ? r : pf_line_row(lane, s));
    tkoff[s] = FP8 ? (uint32_t)(16 * j + 8 * (wv & 1)) : (uint32_t)(8 * pf_line_chunk(lane, s));
  }
  int t_i = -1, t_k = 0, t_st = 0;   // tile, its K step and the step overall of the next token step
  int srow[SPS] = {-1, -1};
  auto t_enter = [&](int i) __attribute__((always_inline)) {
    t_i = i;
    t_k = 0;
    const int4 d4 = desc(i);
#pragma unroll
    for (int s = 0; s < SPS; ++s) srow[s] = prow[s] < d4.z ? d4.y + prow[s] : -1;
  };
  auto issue_tok = [&](int sg) __attribute__((always_inline)) {   // stage sg -> LDS buffer sg % NSTG
    char* stage = Ls[sg % NSTG];
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      // a stage never spans two tiles (nkp is a multiple of SPS), so the
      // tile changes only at s = 0
      if (t_k == nkp && t_i + 1 < nt_w) t_enter(t_i + 1);   // past the last tile: loads nothing
      const int kst = FP8 ? t_k : t_k - s;                   // BF16: the stage's first step (the line spans both)
      const bool live = t_st < nt_w * nkp && kst < nkt && srow[s] >= 0;
      bload_lds<0>(trs, stage + (FP8 ? s * TBS + wv : 2 * wv + s) * 1024,
                   oob_sel(live, (uint32_t)(((size_t)(srow[s] < 0 ? 0 : srow[s]) * K + kst * KS + tkoff[s]) * 2)));
      ++t_k;
      ++t_st;
    }
  };
  // Weight stream: the wave's WB brick rows of the tile's bank-row block.
  int w_i = -1, w_k = 0, w_st = 0;   // tile, its K step, and the step overall
  __amdgpu_buffer_rsrc_t wrs = make_rsrc(a.w_gu, 0u);
  auto w_enter = [&](int i) __attribute__((always_inline)) {
    w_i = i;
    w_k = 0;
    const int4 d4 = desc(i);
    const int row0 = d4.w * kPfRows + kPfWaveRows * wv;
    const bool rows_ok = row0 < NROWS;   // NROWS is a multiple of 128
    const int t0 = rows_ok ? row0 / 16 : 0;
    wrs = make_rsrc((const char*)a.w_down + (size_t)d4.x * bank_bytes + (size_t)t0 * nkt * 1024,
                    rows_ok ? (uint32_t)(WB * nkt * 1024) : 0u);
  };
  u32x4 wr[D][WB];
  auto issue_w = [&](u32x4 (&dst)[WB]) {   // weight bricks of the next weight step (zeros past the last)
    if (w_k == nkp && w_i + 1 < nt_w) w_enter(w_i + 1);
    const bool live = w_st < nt_w * nkp && w_k < nkt;
#pragma unroll
    for (int i = 0; i < WB; ++i) dst[i] = bload(wrs, oob_sel(live, (uint32_t)((i * nkt + w_k) * 1024 + lane * 16)));
    ++w_k;
    ++w_st;
  };

  // MFMA stream: the tile being accumulated.
  int c_i = 0, c_k = 0;
  int t0c = 0;            // first brick row of this wave in the compute tile
  bool rows_okc = false;
  const float* scp = nullptr;   // FP8 block scales of the compute tile (wave-uniform, scalar loads)
  const float* scq = nullptr;
  auto c_enter = [&](int i) __attribute__((always_inline)) {
    c_i = i;
    c_k = 0;
    const int4 d4 = desc(i);
    const int row0 = d4.w * kPfRows + kPfWaveRows * wv;
    rows_okc = row0 < NROWS;
    t0c = rows_okc ? row0 / 16 : 0;
    if (FP8) {
      const int nbk = K / 128;
      scp = scq = a.s_down + ((size_t)d4.x * (a.H / 128) + (16 * t0c) / 128) * nbk;
    }
  };

  f32x4 acc[WB][NTG];
  f32x4 part[FP8 ? WB : 1][FP8 ? NTG : 1];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) acc[i][tg] = f32x4{0, 0, 0, 0};

  // Token operands are read from LDS with asm so that the compiler, which
  // cannot tell the stage being read from the stages still being filled by
  // the LDS-destination loads, does not wait for every load in flight; the
  // asm wait that follows ties the registers.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr)&Ls[0][0];
  u32x4 tk[TBS];
  const uint32_t rofs[2] = {FP8 ? (uint32_t)lane * 16u : pf_line_slot(lane, 0) * 16u,
                            FP8 ? (uint32_t)lane * 16u : pf_line_slot(lane, 1) * 16u};
  auto rd_tok = [&](int st, int q) __attribute__((always_inline)) {
    const uint32_t addr = lds0 + (uint32_t)(((st / SPS) % NSTG) * SB * 1024 +
                                            (FP8 ? ((st % SPS) * TBS + q) * 1024 : q * 2048)) + rofs[st % SPS];
    asm volatile("ds_read_b128 %0, %1" : "=v"(tk[q]) : "v"(addr));
  };
  auto wait_tok = [&]() __attribute__((always_inline)) {   // every LDS read and scalar load issued so far has returned
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(tk[0]), "+v"(tk[1]), "+v"(tk[2]), "+v"(tk[3]), "+v"(tk[4]), "+v"(tk[5]), "+v"(tk[6]),
                   "+v"(tk[7]));
  };

  // The tile's rows of o from the accumulators: acc[i][tg][e] at lane (r, j)
  // is bank row 16 (t0 + i) + 4 j + e of pair row 16 tg + r, times the pair's
  // gate weight.  Buffer stores over the tile's rows (pair rows past the tile
  // pushed out of range): no branch, and the same stores on every tile.
  // They are the only memory operations besides the streams' loads: at the
  // next stage ends they make the waits below (counts of loads only) wait
  // for more, never for less.
  auto epilogue = [&]() __attribute__((always_inline)) {
    const int4 d4 = desc(__builtin_amdgcn_readfirstlane(c_i));
    const int pair0 = d4.y, mrows = d4.z;
    const bool rows_ok = __builtin_amdgcn_readfirstlane((int)rows_okc) != 0;
    const int t0e = __builtin_amdgcn_readfirstlane(t0c);
    const __amdgpu_buffer_rsrc_t os =
        make_rsrc(a.o + (size_t)pair0 * a.H, rows_ok ? (uint32_t)(mrows * a.H * 2) : 0u);
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) {
      const int row = 16 * tg + r;
      const float wp = s_wp[c_i][row];   // 0 past the tile's rows
#pragma unroll
      for (int i = 0; i < WB; ++i) {
        const int c = 16 * (t0e + i) + 4 * j;
        const uint32_t o01 = f32_to_bf16_rne(wp * acc[i][tg][0]) | ((uint32_t)f32_to_bf16_rne(wp * acc[i][tg][1]) << 16);
        const uint32_t o23 = f32_to_bf16_rne(wp * acc[i][tg][2]) | ((uint32_t)f32_to_bf16_rne(wp * acc[i][tg][3]) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{o01, o23}, os,
                                              oob_sel(row < mrows, (uint32_t)((row * a.H + c) * 2)), 0, 0);
      }
    }
  };

  // Loads issued after the token loads of stage e + 1, at the end of stage e
  // (the wait may not exceed it): in the steady state the weights of
  // (NSTG - 1) SPS steps and the token loads of NSTG - 2 stages; at the
  // first stage ends, whose next stages came with the prologue, the
  // prologue's later token and weight loads plus WB per step run so far and
  // SPS per earlier stage end (that count grows by WB SPS per stage end).
  // The epilogues' stores only add to these counts.
  constexpr int kWaitSS = WB * SPS * (NSTG - 1) + SPS * (NSTG - 2);
  constexpr int kWait0 = SPS * (NSTG - 2) + WB * D + WB * (SPS - 1);
  constexpr int kWait1 = kWait0 + WB * SPS < kWaitSS ? kWait0 + WB * SPS : kWaitSS;
  constexpr int kWait2 = kWait1 + WB * SPS < kWaitSS ? kWait1 + WB * SPS : kWaitSS;
  static_assert(kWaitSS < 64, "vmcnt counts to 63");

  // s_g, s_u: the FP8 block scales, loaded at the even step of a loop body
  // and used at its odd step (never carried from one body to the next)
  auto step = [&](int st, auto dc, float& s_g, float& s_u) __attribute__((always_inline)) {
    constexpr int d = decltype(dc)::value;                  // st % D
    constexpr bool ODD = (d & 1) != 0;                      // st % 2 (D is even)
    constexpr bool STAGE_END = (d % SPS) == SPS - 1;        // step st + 1 starts a new stage
    const int ck = __builtin_amdgcn_readfirstlane(c_k);     // K step of the tile (wave-uniform)
    wait_tok();
    if constexpr (FP8 && !ODD) {   // first step of a 128-K block: its two scales (padding steps read the last block's)
      const int blk = min(ck >> 1, K / 128 - 1);
      asm volatile("s_load_dword %0, %1, 0x0" : "=s"(s_g) : "s"(uniform_ptr(scp + blk)));
      asm volatile("s_load_dword %0, %1, 0x0" : "=s"(s_u) : "s"(uniform_ptr(scq + blk)));
    }
    if constexpr (FP8 && ODD) asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(s_g), "+s"(s_u));   // the block's scales
    if constexpr (STAGE_END) {
      // the wait counts assume the loads stay in program order around it:
      // nothing is scheduled across this block
      __builtin_amdgcn_sched_barrier(0);
      const int e = st / SPS;                               // stage ending; stage e + 1 must be in
      if (e == 0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait0));
      else if (e == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait1));
      else if (e == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWait2));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWaitSS));
      __builtin_amdgcn_s_barrier();
      issue_tok(e + NSTG);                                   // into the buffer of stage e, now free
      __builtin_amdgcn_sched_barrier(0);
    }
    // every step runs its MFMAs: a padding step (K step >= nkt) multiplies the
    // zeros its out-of-range loads returned, so no branch separates the token
    // reads (whose registers are in flight until the next wait) from the MFMAs
    if constexpr (!FP8) {
#pragma unroll
      for (int q = 0; q < TBS; ++q) {
#pragma unroll
        for (int i = 0; i < WB; ++i) acc[i][q] = mfma16x16x32(wr[d][i], tk[q], acc[i][q]);
        rd_tok(st + 1, q);
      }
    } else {
      if constexpr (!ODD) {   // first step of a 128-K block: zero partial sums
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int tg = 0; tg < NTG; ++tg) part[i][tg] = f32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {   // the low K halves of the step, then the high ones
        u32x4 op[WB];
#pragma unroll
        for (int i = 0; i < WB; ++i) {
          u32x4 lo, hi;
          e4m3x16_to_bf16_nat(wr[d][i], lo, hi);
          op[i] = h ? hi : lo;
        }
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg) {
#pragma unroll
          for (int i = 0; i < WB; ++i) part[i][tg] = mfma16x16x32(op[i], tk[2 * tg + h], part[i][tg]);
          rd_tok(st + 1, 2 * tg + h);
        }
      }
      if constexpr (ODD) {
        const float sc = j < 2 ? s_g : s_u;
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int tg = 0; tg < NTG; ++tg)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][tg][e] += sc * part[i][tg][e];
      }
    }
    issue_w(wr[d]);
    if (++c_k == nkp) {   // the tile is complete: its outputs, then the next tile
      epilogue();
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg) acc[i][tg] = f32x4{0, 0, 0, 0};
      if (c_i + 1 < nt_w) c_enter(c_i + 1);
    }
  };

  t_enter(0);
  w_enter(0);
  c_enter(0);
  for (int sg = 0; sg < NSTG; ++sg) issue_tok(sg);
#pragma unroll
  for (int d = 0; d < D; ++d) issue_w(wr[d]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(SPS * (NSTG - 1) + WB * D));   // stage 0 is in
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int q = 0; q < TBS; ++q) rd_tok(0, q);
  const int nsteps = nt_w * nkp;
  for (int st0 = 0; st0 < nsteps; st0 += D) {
    float s_g, s_u;   // defined at the even step when it is a real step (padding steps come in pairs)
    step(st0, std::integral_constant<int, 0>{}, s_g, s_u);
    step(st0 + 1, std::integral_constant<int, 1>{}, s_g, s_u);
    if constexpr (D == 4) {
      step(st0 + 2, std::integral_constant<int, 2>{}, s_g, s_u);
      step(st0 + 3, std::integral_constant<int, 3 % D>{}, s_g, s_u);
    }
  }
  wait_tok();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load into LDS or registers outlives the loop
}

// y[t] = sum_j o[pos(t, j)] in pick order (deterministic), 8 outputs per thread
__global__ __launch_bounds__(256) void pf_combine_kernel(PfArgs a) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = a.H / 8;
  if (gid >= (size_t)a.T * per_row) return;
  const int t = (int)(gid / per_row), c = (int)(gid % per_row) * 8;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int jj = 0; jj < a.k; ++jj) {
    const int pos = a.pair_pos[(size_t)t * a.k + jj];
    if (pos >= 0) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.o + (size_t)pos * a.H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[2 * q] += __uint_as_float(v[q] << 16);
        s[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
      }
    }
  }
  const size_t o = (size_t)t * a.H + c;
  const f32x4 y0 = {s[0], s[1], s[2], s[3]}, y1 = {s[4], s[5], s[6], s[7]};
  if (a.y) {
    *reinterpret_cast<f32x4*>(a.y + o) = y0;
    *reinterpret_cast<f32x4*>(a.y + o + 4) = y1;
  }
  if (a.y_out) {   // merge with the host partial sum
    const f32x4 m0 = y0 + *reinterpret_cast<const f32x4*>(a.y_host + o);
    const f32x4 m1 = y1 + *reinterpret_cast<const f32x4*>(a.y_host + o + 4);
    *reinterpret_cast<f32x4*>(a.y_out + o) = m0;
    *reinterpret_cast<f32x4*>(a.y_out + o + 4) = m1;
    if (a.y_bf16) {
      const uint32_t b0 = f32_to_bf16_rne(m0[0]) | ((uint32_t)f32_to_bf16_rne(m0[1]) << 16);
      const uint32_t b1 = f32_to_bf16_rne(m0[2]) | ((uint32_t)f32_to_bf16_rne(m0[3]) << 16);
      const uint32_t b2 = f32_to_bf16_rne(m1[0]) | ((uint32_t)f32_to_bf16_rne(m1[1]) << 16);
      const uint32_t b3 = f32_to_bf16_rne(m1[2]) | ((uint32_t)f32_to_bf16_rne(m1[3]) << 16);
      *reinterpret_cast<u32x4*>(a.y_bf16 + o) = u32x4{b0, b1, b2, b3};
    }
  }
}

// ================================================================ merge
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ yg, const float* __restrict__ yh,
                                                    size_t n4, size_t n, float* yo, uint16_t* yb) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(yg + 4 * i) + *reinterpret_cast<const f32x4*>(yh + 4 * i);
    *reinterpret_cast<f32x4*>(yo + 4 * i) = v;
    if (yb) {
      uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
      uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<u32x2*>(yb + 4 * i) = u32x2{lo, hi};
    }
  }
  if (i == 0) {
    for (size_t t = 4 * n4; t < n; ++t) {
      float v = yg[t] + yh[t];
      yo[t] = v;
      if (yb) yb[t] = f32_to_bf16_rne(v);
    }
  }
}

// ================================================================ E4M3 expansion utility
// The same conversion the decode path runs in registers, exposed so that it
// can be checked code by code.
__global__ __launch_bounds__(256) void e4m3_expand_kernel(const uint8_t* __restrict__ codes, uint16_t* __restrict__ out,
                                                          int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= n) return;
  u32x4 q = {0, 0, 0, 0};
  uint8_t b[16];
  for (int t = 0; t < 16; ++t) b[t] = (i + t < n) ? codes[i + t] : 0;
  for (int t = 0; t < 4; ++t)
    q[t] = (uint32_t)b[4 * t] | ((uint32_t)b[4 * t + 1] << 8) | ((uint32_t)b[4 * t + 2] << 16) |
           ((uint32_t)b[4 * t + 3] << 24);
  u32x4 lo, hi;
  e4m3x16_to_bf16_nat(q, lo, hi);
  for (int t = 0; t < 16; ++t) {
    if (i + t >= n) break;
    const uint32_t v = t < 8 ? lo[t >> 1] : hi[(t - 8) >> 1];
    out[i + t] = (uint16_t)((t & 1) ? (v >> 16) : (v & 0xFFFFu));
  }
}

// ================================================================ workspace layouts
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecWs {
  size_t err, done, all, go, h, total;
};
static DecWs dec_ws(int T_max, int k, int H, int I, int n_slots) {
  DecWs w{};
  int G = T_max * k < n_slots ? T_max * k : n_slots;
  size_t off = 0;
  w.err = off; off = align256(off + 4);
  w.done = off; off = align256(off + 4 * (size_t)kDecPmax * kCtrlStride);
  w.all = off; off = align256(off + 4);
  w.go = off; off = align256(off + 4 * (size_t)kDecGridMax * kCtrlStride);
  w.h = off; off = align256(off + 2 * (size_t)G * kDecTok * I);
  w.total = off;
  return w;
}

// Resident workgroups per CU of each decode kernel, and the CU count, per device.
struct DecOcc {
  int cus = 0;
  int fu[2][2] = {{0, 0}, {0, 0}};   // [FP8][8-row down tasks]
  int fu_rg2 = 0;                    // FP8 with two brick rows per gate/up task
  int fu_rb2 = 0;                    // ... and per down task
  int fu_rg4 = 0;                    // FP8, four brick rows per gate/up task, two per down task
  int fu_rg2h = 0;                   // FP8 two-row gate/up tasks, device-scope h loads
  int fu_rb2h = 0;                   // ... and two-row down tasks
};
// Register-ring depths in 2-brick steps.  Deeper rings put more bytes in
// flight per wave, but past a few KB per wave the launch as a whole streams
// slower (measured: BF16 T = 16 2 steps 83.5 us against 4 steps 87.4 us;
// BF16 T = 1 with resident down weights 3 steps 19.5 us against 4 steps
// 20.5 us; FP8 two-row tasks 1 step 41.9 / 120.1 / 338.5 us at T = 1 / 4 /
// 16 against 2 steps 48.4 / 134.9 / 352.0 us).
constexpr int kDecD_BF16 = 2;      // 16-row down tasks
constexpr int kDecD_RES = 2;       // register-resident down weights (DR = 8; 3: 17.9 -> 17.5 us at 7 groups back to back)
constexpr int kDecD_FP8 = 3;       // FP8, one brick row per gate/up task (steps carry twice the x operand)
constexpr int kDecD_FP8_RG2 = 1;   // FP8, two brick rows per gate/up task
constexpr int kDecW = 8;   // waves per workgroup
static std::atomic<int> g_dec_grid_override{0};   // decode forward grid, 0: automatic
static std::mutex g_occ_mu;
static DecOcc g_occ[64];
static moe_status dec_occupancy(DecOcc* out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) MOE_FAIL(MOE_ERR_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_occ_mu);
  DecOcc& o = g_occ[dev];
  if (!o.cus) {
    int cus = 0;
    MOE_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu[0][0], dec_fused_kernel<false, kDecD_BF16, kDecW, 16>, kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu[1][0], dec_fused_kernel<true, kDecD_FP8, kDecW, 16>, kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu[0][1], dec_fused_kernel<false, kDecD_RES, kDecW, 8>, kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu_rg2, dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 16, 2>,
                                                         kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu_rb2, dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 2>,
                                                         kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.fu_rg4, dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 4>,
                                                         kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &o.fu_rg2h, dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 16, 2, true>, kDecW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &o.fu_rb2h, dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 2, true>, kDecW * 64, 0));
    o.fu[1][1] = 0;   // the register-resident form is BF16 only (FP8 steps need more registers than it has)
    for (int i = 0; i < 2; ++i)
      if (o.fu[i][0] < 1) o.fu[i][0] = 1;
    o.cus = cus > 0 ? cus : 1;
  }
  *out = o;
  return MOE_OK;
}

struct PfWs {
  size_t hist, cnt, off, mtoff, nt, tslot, tm0, sp, pp, h, o, total;
  int max_mtiles, n_chunks, tm, chunk;
};
static PfWs pf_ws(int T_max, int k, int H, int I, int n_slots, bool fp8) {
  PfWs w{};
  size_t P = (size_t)T_max * k;
  w.tm = fp8 ? 64 : 128;
  w.max_mtiles = (int)((P + w.tm - 1) / w.tm) + n_slots;
  w.chunk = kSortChunk;
  while ((P + w.chunk - 1) / w.chunk > (size_t)kSortMaxChunks) w.chunk *= 2;
  w.n_chunks = (int)((P + w.chunk - 1) / w.chunk);
  size_t off = 0;
  w.hist = off; off = align256(off + 4 * (size_t)w.n_chunks * n_slots);
  w.cnt = off; off = align256(off + 4 * (size_t)n_slots);
  w.off = off; off = align256(off + 4 * (size_t)n_slots);
  w.mtoff = off; off = align256(off + 4 * (size_t)n_slots);
  w.nt = off; off = align256(off + 4);
  w.tslot = off; off = align256(off + 4 * (size_t)w.max_mtiles);
  w.tm0 = off; off = align256(off + 4 * (size_t)w.max_mtiles);
  w.sp = off; off = align256(off + 4 * P);
  w.pp = off; off = align256(off + 4 * P);
  w.h = off; off = align256(off + 2 * P * I);
  w.o = off; off = align256(off + 2 * P * H);
  w.total = off;
  return w;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_forward_workspace_bytes(int32_t T_max, int32_t k, int32_t H, int32_t I, int32_t n_slots,
                                                  uint32_t mode, size_t* bytes) {
  clear_error();
  if (!bytes) MOE_FAIL(MOE_ERR_ARG, "bytes is NULL");
  if (T_max < 1 || k < 1 || H < 1 || I < 1 || n_slots < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad sizes");
  if (mode == MOE_FWD_DECODE || mode == MOE_FWD_DECODE_SPLIT) {
    if (T_max > kDecTok || T_max * k > kDecPmax)
      MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T_max <= %d and T_max*k <= %d", kDecTok, kDecPmax);
    *bytes = dec_ws(T_max, k, H, I, n_slots).total;
  } else if (mode == MOE_FWD_PREFILL) {
    if (n_slots > kSortMaxSlots) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs n_slots <= %d", kSortMaxSlots);
    const size_t b16 = pf_ws(T_max, k, H, I, n_slots, false).total, b8 = pf_ws(T_max, k, H, I, n_slots, true).total;
    *bytes = b16 > b8 ? b16 : b8;
  } else {
    MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  }
  return MOE_OK;
}

extern "C" moe_status moe_pack_weights(int32_t wtype, int32_t H, int32_t I, int32_t n, const void* w_gate,
                                      const void* w_up, const void* w_down, void* w_gate_up, void* w_down_packed,
                                      hipStream_t stream) {
  clear_error();
  if (wtype != MOE_W_BF16 && wtype != MOE_W_FP8_B128) MOE_FAIL(MOE_ERR_ARG, "bad wtype %d", wtype);
  const int q = wtype == MOE_W_FP8_B128 ? 128 : 32;
  if (H <= 0 || I <= 0 || n < 0 || H % q || I % q || I % 8)
    MOE_FAIL(MOE_ERR_SHAPE, "pack needs H, I multiples of %d and I %% 8 == 0 (H=%d I=%d n=%d)", q, H, I, n);
  if (n == 0) return MOE_OK;
  if (!w_gate || !w_up || !w_down || !w_gate_up || !w_down_packed) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(w_gate_up) || !aligned16(w_down_packed))
    MOE_FAIL(MOE_ERR_ARG, "pack buffers must be 16-byte aligned");
  const size_t el = wtype == MOE_W_FP8_B128 ? 1 : 2;
  const size_t chunks = (size_t)n * 3 * I * H * el / 16;
  pack_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, stream>>>(wtype == MOE_W_FP8_B128, H, I, n, (const char*)w_gate,
                                                                      (const char*)w_up, (const char*)w_down,
                                                                      (char*)w_gate_up, (char*)w_down_packed);
  MOE_LAUNCHED();
  return MOE_OK;
}

// run_forward's mode for moe_decode_wait_test (not a public mode: the public
// calls take only these)
constexpr uint32_t kFwdDecodeWaitTest = 0x80000000u;
static bool public_mode(uint32_t mode) {
  return mode == MOE_FWD_DECODE || mode == MOE_FWD_PREFILL || mode == MOE_FWD_DECODE_SPLIT;
}

static moe_status run_forward(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot, const float* w,
                              int32_t T, int32_t k, float* y, const float* y_host, float* y_out, uint16_t* y_bf16,
                              void* ws, size_t ws_bytes, uint32_t mode, hipStream_t stream,
                              uint32_t polls = kPollLimit) {
  moe_status st = check_slots(slots);
  if (st) return st;
  if (T < 0 || k < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad T=%d k=%d", T, k);
  if (T == 0) return MOE_OK;
  if (!x || !pick_slot || !w || !ws) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(x) || (y && !aligned16(y)) || (y_host && !aligned16(y_host)) || (y_out && !aligned16(y_out)) ||
      (y_bf16 && !aligned16(y_bf16)))
    MOE_FAIL(MOE_ERR_ARG, "x and the outputs must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) & 255) MOE_FAIL(MOE_ERR_ARG, "workspace must be 256-byte aligned");
  const bool fp8 = slots->wtype == MOE_W_FP8_B128;
  const int H = slots->H, I = slots->I;
  char* wsb = (char*)ws;

  if (mode == MOE_FWD_DECODE || mode == MOE_FWD_DECODE_SPLIT || mode == kFwdDecodeWaitTest) {
    if (T > kDecTok || T * k > kDecPmax)
      MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T <= %d and T*k <= %d (T=%d k=%d)", kDecTok, kDecPmax, T, k);
    if (fp8 && H > 16384) MOE_FAIL(MOE_ERR_SHAPE, "FP8 decode mode needs H <= 16384 (H=%d)", H);
    DecWs L = dec_ws(T, k, H, I, slots->n_slots);
    if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
    DecOcc occ;
    moe_status os = dec_occupancy(&occ);
    if (os) return os;
    DecArgs a{};
    a.w_gu = slots->w_gate_up; a.w_down = slots->w_down;
    a.s_gate = slots->s_gate; a.s_up = slots->s_up; a.s_down = slots->s_down;
    a.H = H; a.I = I; a.n_slots = slots->n_slots; a.T = T; a.k = k;
    a.x = x; a.pick_slot = pick_slot; a.w = w; a.y = y;
    a.y_host = y_host; a.y_out = y_out; a.y_bf16 = y_bf16;
    a.h = (uint16_t*)(wsb + L.h);
    a.G_max = T * k < slots->n_slots ? T * k : slots->n_slots;
    a.poll_limit = polls;
    DecWsDev c{};
    c.err = (uint32_t*)(wsb + L.err);
    c.done = (uint32_t*)(wsb + L.done);
    c.all = (uint32_t*)(wsb + L.all);
    c.go = (uint32_t*)(wsb + L.go);
    const int f = fp8 ? 1 : 0;
    // FP8: two brick rows per gate/up task, so each x load serves both (x is
    // 2 B x T per K against 1 B per weight row); measured faster at T = 1, 4
    // and 16 (at T = 1 it also halves the task ends)
    const bool rg2 = fp8 && (I / 8) % 2 == 0 && occ.fu_rg2 >= occ.fu[1][0];
    // FP8 from T = 2 on: two brick rows per down task too, so each h load
    // serves both (h is 2 B x T per K against 1 B per weight row; measured
    // at T = 16: 333 -> 281 us, T = 4: 121 -> 111 us, T = 2: 67.5 -> 64.4 us)
    const bool rb2 = rg2 && T >= 2 && occ.fu_rb2 >= occ.fu[1][0];
    // from T = 8 on, also four brick rows per gate/up task, so x is re-read
    // once per four rows (measured at T = 16: 285 -> 247 us; at T = 4 slower)
    const bool rg4 = rb2 && T >= 8 && (I / 8) % 4 == 0 && occ.fu_rg4 >= occ.fu[1][0];
    const long tasks = (long)a.G_max * (I / 8) / (rg4 ? 4 : rg2 ? 2 : 1) + 2L * (H / 16);
    // the grid: every workgroup resident at once (the down phase waits for
    // the last gate/up task), at most one workgroup per task
    const auto grid = [&](int per_cu) {
      return (unsigned)std::min<long>(std::min<long>(tasks, (long)occ.cus * per_cu), kDecGridMax);
    };
    // 8-row down tasks with register-resident weights and h in LDS when every
    // down task fits in one round of that form's grid, a wave's steps fit its
    // registers and h fits the LDS
    const long res_steps = ((long)a.G_max * ((I / (fp8 ? 64 : 32) + 3) / 4) + kDecW - 1) / kDecW;
    const int ov = g_dec_grid_override.load(std::memory_order_relaxed);
    const bool dr8 = !fp8 && (long)(H / 8) <= (ov > 0 ? (long)ov : (long)grid(occ.fu[0][1])) &&
                     res_steps <= kDecResSteps && (long)a.G_max * T * I * 2 <= kDecResH;
    // (FP8 two-row tasks: two workgroups per CU, the one-row form's
    // occupancy, although three fit: measured 120 / 339 us at T = 4 / 16
    // against 125 / 364 us with three)
    const unsigned g1 = ov > 0 ? (unsigned)ov : grid(rg2 ? occ.fu[1][0] : dr8 ? occ.fu[0][1] : occ.fu[f][0]);
    // MOE_FWD_DECODE_SPLIT: the same kernel twice (gate/up, then down)
    const int ph0 = mode == MOE_FWD_DECODE ? 0 : mode == kFwdDecodeWaitTest ? 3 : 1;
    const int ph1 = mode == MOE_FWD_DECODE_SPLIT ? 2 : ph0;
    for (int ph = ph0; ph <= ph1; ++ph) {
      a.phase = ph;
      if (rg4)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 4><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (rb2 && T <= 4 && occ.fu_rb2h >= occ.fu[1][0])   // (device-scope h loads: T = 2 63.7 -> 62.6 us,
                                                                // T = 4 98.6 -> 98.1 us, 8 and 13 groups)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 2, true><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (rb2)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 2><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (rg2 && T == 1 && occ.fu_rb2h >= occ.fu[1][0])   // T = 1: two-row down tasks too, device-scope h
                                                               // loads (4 groups: 36.9 -> 35.5 us; 3: 31.7 -> 30.8)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 32, 2, true><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (rg2 && T == 1 && occ.fu_rg2h >= occ.fu[1][0])   // (device-scope h loads: T = 1 41.8 -> 40.2 us,
                                                               // T = 4 119.6 -> 121.3 us)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 16, 2, true><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (rg2)
        dec_fused_kernel<true, kDecD_FP8_RG2, kDecW, 16, 2><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (fp8)
        dec_fused_kernel<true, kDecD_FP8, kDecW, 16><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else if (dr8)
        dec_fused_kernel<false, kDecD_RES, kDecW, 8><<<g1, kDecW * 64, 0, stream>>>(a, c);
      else
        dec_fused_kernel<false, kDecD_BF16, kDecW, 16><<<g1, kDecW * 64, 0, stream>>>(a, c);
      MOE_LAUNCHED();
    }
    return MOE_OK;
  }
  if (mode != MOE_FWD_PREFILL) MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  if (slots->n_slots > kSortMaxSlots) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs n_slots <= %d", kSortMaxSlots);
  if (H % 128 || I % 64) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs H %% 128 == 0 and I %% 64 == 0");
  PfWs L = pf_ws(T, k, H, I, slots->n_slots, fp8);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if ((size_t)T * H * 2 >= 0x80000000ull || (size_t)T * k * (size_t)(H > I ? H : I) * 2 >= 0x80000000ull)
    MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs T*H*2 and T*k*max(H,I)*2 below 2^31 bytes");
  PfArgs a{};
  a.w_gu = slots->w_gate_up; a.w_down = slots->w_down;
  a.s_gate = slots->s_gate; a.s_up = slots->s_up; a.s_down = slots->s_down;
  a.H = H; a.I = I; a.n_slots = slots->n_slots; a.T = T; a.k = k; a.P = T * k;
  a.tm = L.tm; a.max_mtiles = L.max_mtiles; a.chunk = L.chunk;
  a.x = x; a.pick_slot = pick_slot; a.w = w; a.y = y;
  a.y_host = y_host; a.y_out = y_out; a.y_bf16 = y_bf16;
  a.hist = (int32_t*)(wsb + L.hist);
  a.cnt = (int32_t*)(wsb + L.cnt);
  a.off = (int32_t*)(wsb + L.off);
  a.mtoff = (int32_t*)(wsb + L.mtoff);
  a.n_mtiles = (int32_t*)(wsb + L.nt);
  a.tile_slot = (int32_t*)(wsb + L.tslot);
  a.tile_m0 = (int32_t*)(wsb + L.tm0);
  a.sorted_pair = (int32_t*)(wsb + L.sp);
  a.pair_pos = (int32_t*)(wsb + L.pp);
  a.h = (uint16_t*)(wsb + L.h);
  a.o = (uint16_t*)(wsb + L.o);
  pf_count_kernel<<<L.n_chunks, 256, 0, stream>>>(a);
  pf_scan_kernel<<<1, 1024, 0, stream>>>(a, L.n_chunks);
  pf_scatter_kernel<<<L.n_chunks, 256, 0, stream>>>(a);
  // The persistent down GEMM's grid: R workgroups per XCD, one per CU where
  // the tiles allow, more when a workgroup would hold more tiles than its LDS
  // tables do (the tile count is known on the device; max_mtiles bounds it).
  DecOcc occ;
  moe_status os = dec_occupancy(&occ);
  if (os) return os;
  const int mt_lds = fp8 ? PfMeta<true>::kTiles : PfMeta<false>::kTiles;
  const auto pgrid = [&](long tiles) {
    const long q = (tiles + 7) / 8;                       // tiles per XCD at most
    long rr = std::max<long>(1, occ.cus / 8);
    rr = std::max<long>(rr, (q + mt_lds - 1) / mt_lds);   // at most mt_lds tiles per workgroup
    rr = std::min<long>(rr, std::max<long>(1, q));
    return (unsigned)(8 * rr);
  };
  const long gu_tiles = (long)L.max_mtiles * ((2 * I + kPfRows - 1) / kPfRows);
  const long dn_tiles = (long)L.max_mtiles * ((H + kPfRows - 1) / kPfRows);
  // gate/up: one tile per workgroup, the dispatcher balancing the CUs (its
  // long K hides a tile's start and end); down: the persistent kernel, since
  // its short K leaves them exposed (measured per BF16 layer 0.787 ms
  // against 0.813 ms with one-tile workgroups for both; per FP8 layer 6.57
  // against 6.75 ms)
  const unsigned g1 = (unsigned)(8 * ((gu_tiles + 7) / 8)), g2 = pgrid(dn_tiles);
  if (fp8) {
    pf_gemm_kernel<true, true><<<g1, kPfWaves * 64, 0, stream>>>(a);
    pf_down_kernel<true><<<g2, kPfWaves * 64, 0, stream>>>(a);
  } else {
    pf_gemm_kernel<false, true><<<g1, kPfWaves * 64, 0, stream>>>(a);
    pf_down_kernel<false><<<g2, kPfWaves * 64, 0, stream>>>(a);
  }
  const size_t ncomb = ((size_t)T * (H / 8) + 255) / 256;
  pf_combine_kernel<<<(unsigned)ncomb, 256, 0, stream>>>(a);
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_expert_forward(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                         const float* w, int32_t T, int32_t k, float* y, void* ws, size_t ws_bytes,
                                         uint32_t mode, hipStream_t stream) {
  clear_error();
  if (!public_mode(mode)) MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  if (T > 0 && !y) MOE_FAIL(MOE_ERR_ARG, "y is NULL");
  return run_forward(slots, x, pick_slot, w, T, k, y, nullptr, nullptr, nullptr, ws, ws_bytes, mode, stream);
}

extern "C" moe_status moe_expert_forward_merge(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                               const float* w, int32_t T, int32_t k, float* y_gpu,
                                               const float* y_host, float* y_out, uint16_t* y_out_bf16, void* ws,
                                               size_t ws_bytes, uint32_t mode, hipStream_t stream) {
  clear_error();
  if (!public_mode(mode)) MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  if (T > 0 && (!y_host || !y_out)) MOE_FAIL(MOE_ERR_ARG, "y_host and y_out are required");
  return run_forward(slots, x, pick_slot, w, T, k, y_gpu, y_host, y_out, y_out_bf16, ws, ws_bytes, mode, stream);
}

extern "C" moe_status moe_decode_wait_test(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                           const float* w, int32_t T, int32_t k, float* y, void* ws, size_t ws_bytes,
                                           uint32_t polls, hipStream_t stream) {
  clear_error();
  if (polls < 1 || polls > kPollLimit) MOE_FAIL(MOE_ERR_ARG, "polls %u outside [1, %u]", polls, kPollLimit);
  if (T > 0 && !y) MOE_FAIL(MOE_ERR_ARG, "y is NULL");
  return run_forward(slots, x, pick_slot, w, T, k, y, nullptr, nullptr, nullptr, ws, ws_bytes, kFwdDecodeWaitTest,
                     stream, polls);
}

extern "C" moe_status moe_decode_grid_override(int32_t n_workgroups) {
  clear_error();
  if (n_workgroups < 0 || n_workgroups > kDecGridMax)
    MOE_FAIL(MOE_ERR_ARG, "n_workgroups %d outside [0, %d]", n_workgroups, kDecGridMax);
  g_dec_grid_override.store(n_workgroups, std::memory_order_relaxed);
  return MOE_OK;
}

// ================================================================ allocation-free decode
// For callers that cannot allocate (hipGraph capture, serving loops, harnesses
// that forbid hipMalloc): the decode workspace lives in this file-scope
// device array.  Each GPU the library runs on holds its own copy until the
// process ends; its device address is looked up once per device and kept.
namespace moe {
constexpr size_t kStaticCtrlBytes = 512u << 10;                       // error word, counters, start flags
constexpr size_t kStaticScratchBytes = (8u << 20) + kStaticCtrlBytes;  // + h: 8 MiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

static moe_status scratch_ptr(void** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) MOE_FAIL(MOE_ERR_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) MOE_FAIL(MOE_ERR_HIP, "hipGetSymbolAddress returned NULL for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace moe

extern "C" moe_status moe_expert_forward_merge_static(const moe_slots* slots, const uint16_t* x,
                                                      const int32_t* pick_slot, const float* w, int32_t T, int32_t k,
                                                      float* y_gpu, const float* y_host, float* y_out,
                                                      uint16_t* y_out_bf16, hipStream_t stream) {
  clear_error();
  moe_status st = check_slots(slots);
  if (st) return st;
  if (T < 0 || k < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad T=%d k=%d", T, k);
  if (T == 0) return MOE_OK;
  if (!y_host || !y_out) MOE_FAIL(MOE_ERR_ARG, "y_host and y_out are required");
  if (T > kDecTok || T * k > kDecPmax)
    MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T <= %d and T*k <= %d (T=%d k=%d)", kDecTok, kDecPmax, T, k);
  const DecWs L = dec_ws(T, k, slots->H, slots->I, slots->n_slots);
  if (L.h > kStaticCtrlBytes || L.total > kStaticScratchBytes)
    MOE_FAIL(MOE_ERR_NO_SPACE,
             "this call needs %zu bytes of workspace; the static scratch holds %zu (h of min(T*k, n_slots) * 16 * I "
             "BF16 values must fit 8 MiB)",
             L.total, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws))) return st;
  // the hand-over words must start at zero: a call whose wait timed out may
  // have left one set, so they are cleared (a kernel, not a memset, so that
  // the call can be captured) before every call
  const size_t ctrl_words = L.h / 4;
  zero_words_kernel<<<(unsigned)std::min<size_t>((ctrl_words + 255) / 256, 256), 256, 0, stream>>>((uint32_t*)ws,
                                                                                                  ctrl_words);
  MOE_LAUNCHED();
  return run_forward(slots, x, pick_slot, w, T, k, y_gpu, y_host, y_out, y_out_bf16, ws, kStaticScratchBytes,
                     MOE_FWD_DECODE, stream);
}

extern "C" moe_status moe_merge_partial(const float* y_gpu, const float* y_host, int32_t T, int32_t H, float* y_out,
                                        uint16_t* y_out_bf16, hipStream_t stream) {
  clear_error();
  if (T < 0 || H < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad T=%d H=%d", T, H);
  if (T == 0) return MOE_OK;
  if (!y_gpu || !y_host || !y_out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(y_gpu) || !aligned16(y_host) || !aligned16(y_out) || (y_out_bf16 && (reinterpret_cast<uintptr_t>(y_out_bf16) & 7)))
    MOE_FAIL(MOE_ERR_ARG, "y_gpu, y_host, y_out must be 16-byte aligned and y_out_bf16 8-byte aligned");
  const size_t n = (size_t)T * H, n4 = n / 4;
  const size_t blocks = n4 ? (n4 + 255) / 256 : 1;
  merge_kernel<<<(unsigned)blocks, 256, 0, stream>>>(y_gpu, y_host, n4, n, y_out, y_out_bf16);
  MOE_LAUNCHED();
  return MOE_OK;
}

namespace moe {
// Plain streaming read: U non-temporal 16-byte loads per thread in flight,
// grid-stride, folded with XOR and one atomic per workgroup.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* sink) {
  const size_t gsz = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * gsz < n; i += U * gsz) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * gsz);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += gsz) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + (blockIdx.x & 255), acc);
}
}  // namespace moe

extern "C" moe_status moe_stream_read_cfg(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg, int32_t unroll,
                                          hipStream_t stream) {
  clear_error();
  if (bytes == 0) return MOE_OK;
  if (!src || !sink) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(src) || (bytes & 15)) MOE_FAIL(MOE_ERR_ARG, "src must be 16-byte aligned and bytes a multiple of 16");
  if (n_wg < 1 || n_wg > 65536) MOE_FAIL(MOE_ERR_SHAPE, "n_wg %d outside [1, 65536]", n_wg);
  const u32x4* p = (const u32x4*)src;
  const size_t n = bytes / 16;
  switch (unroll) {
    case 1: stream_read_kernel<1><<<n_wg, 256, 0, stream>>>(p, n, sink); break;
    case 2: stream_read_kernel<2><<<n_wg, 256, 0, stream>>>(p, n, sink); break;
    case 4: stream_read_kernel<4><<<n_wg, 256, 0, stream>>>(p, n, sink); break;
    case 8: stream_read_kernel<8><<<n_wg, 256, 0, stream>>>(p, n, sink); break;
    case 16: stream_read_kernel<16><<<n_wg, 256, 0, stream>>>(p, n, sink); break;
    default: MOE_FAIL(MOE_ERR_ARG, "unroll %d not in {1, 2, 4, 8, 16}", unroll);
  }
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  return moe_stream_read_cfg(src, bytes, sink, 512, 4, stream);
}

extern "C" moe_status moe_e4m3_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, hipStream_t stream) {
  clear_error();
  if (n < 0) MOE_FAIL(MOE_ERR_SHAPE, "n < 0");
  if (n == 0) return MOE_OK;
  if (!codes || !out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  const int64_t threads = (n + 15) / 16;
  e4m3_expand_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(codes, out, n);
  MOE_LAUNCHED();
  return MOE_OK;
}
