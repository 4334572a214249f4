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
// serves the whole batch.  Two launches: gate/up + SwiGLU into h, then down
// with the per-token gate weights.
// Prefill (any T): (token, pick) pairs counting-sorted by slot, a grouped
// MFMA GEMM for gate/up with the SwiGLU epilogue, a grouped MFMA GEMM for
// down with the gate-weight epilogue into per-pair rows, and a combine that
// sums each token's k rows in pick order.
#include "common.h"

#include <algorithm>
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
// Both launches are grids of resident workgroups that walk a task list
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
  float* y;                  // [T][H]
  uint16_t* h;               // workspace [G_max][16][I] BF16
  int G_max;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
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
#pragma unroll
  for (int h = 0; h < kDecPPL; ++h) {
    const int p = lane + 64 * h;
    const int s = p < P ? pick_slot[p] : -1;
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
    if (s_gw) s_gw[g * kDecTok + (lane + 64 * h) / k] = w[lane + 64 * h];
  }
  if (lane == 0) *s_G = base[kDecPPL];
}

// gate/up + SwiGLU.  Task (group g, brick row t): 16 rows of the gate/up bank
// (gate rows 8t..8t+7 above the same up rows) over all H.  The NW waves take
// 1/NW of the row's 2-brick steps each and meet in LDS, where wave 0 forms
// h[g][token][8t..8t+7] = silu(gate) * up in BF16.  A workgroup's tasks form
// one continuous step sequence per wave, so the loads of the next task are in
// flight while the current one is reduced.  The first pass of workgroups also
// zeroes y for the down launch.
template <bool FP8, int D, int NW>
__global__ __launch_bounds__(NW * 64) void dec_gu_kernel(DecArgs a) {
  __shared__ int s_gslot[kDecPmax];
  __shared__ int s_G;
  __shared__ unsigned long long s_tab[kPlanTab];
  __shared__ f32x4 red[2][NW][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I, T = a.T;
  for (int i = blockIdx.x * NW * 64 + tid; i < T * H; i += gridDim.x * NW * 64) a.y[i] = 0.f;
  if (wv == 0) wave_plan(a.pick_slot, a.w, T * a.k, a.k, a.n_slots, a.G_max, s_gslot, nullptr, &s_G, s_tab);
  __syncthreads();
  const int G = s_G;
  const int RA = I / 8;
  const int nkt = FP8 ? H / 64 : H / 32;     // bricks per row
  const int S = (nkt + 1) >> 1;              // 2-brick steps per row
  const int SW = (S + NW - 1) / NW;          // steps per wave per task
  const int s_lo = wv * SW;
  const size_t gu_bytes = (size_t)2 * I * H * (FP8 ? 1 : 2);
  const int ntask = G * RA;
  const int ntk = ntask > (int)blockIdx.x ? (ntask - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
  const int nsteps = ntk * SW;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)(T * H * 2));
  const bool tok = r < T;
  constexpr int XN = FP8 ? 4 : 2;
  u32x4 wb[D][2], xb[D][XN];
  float sb[D][2];
  int i_tk = 0, i_l = 0;   // issue position: task of this workgroup, step within the wave's share
  auto issue = [&](int d) {
    const int task = (int)blockIdx.x + i_tk * (int)gridDim.x;
    const int s = s_lo + i_l;
    const bool ok = i_tk < ntk && s < S;
    const int tt = ok ? task : 0;
    const int g = tt / RA, t = tt - g * RA;
    const int slot = ok ? __builtin_amdgcn_readfirstlane(s_gslot[g]) : 0;   // slot 0 always exists
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc((const char*)a.w_gu + (size_t)slot * gu_bytes + (size_t)t * nkt * 1024, (uint32_t)(nkt * 1024));
    const uint32_t wo = oob_sel(ok, (uint32_t)s * 2048u + lane * 16u);
    wb[d][0] = bload_nt(wr, wo);
    wb[d][1] = bload_nt(wr, oob_sel(ok, wo + 1024u));
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int k0 = FP8 ? 128 * s + 64 * b : 64 * s + 32 * b;
      const bool xo = ok && tok && k0 < H;
      const uint32_t off = oob_sel(xo, (uint32_t)(r * H + k0 + (FP8 ? 16 : 8) * j) * 2u);
      if (FP8) {
        xb[d][2 * b] = bload(xr, off);
        xb[d][2 * b + 1] = bload(xr, oob_sel(xo, off + 16u));
      } else {
        xb[d][b] = bload(xr, off);
      }
    }
    if (FP8) {   // block scales of the gate rows and of the up rows at this K step (scalar loads)
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
  f32x4 acc = {0, 0, 0, 0};
  int c_tk = 0, c_l = 0;
  for (int i0 = 0; i0 < nsteps; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (i0 + d < nsteps) {
        if (!FP8) {
          acc = mfma16x16x32(wb[d][0], xb[d][0], acc);
          acc = mfma16x16x32(wb[d][1], xb[d][1], acc);
        } else {
          f32x4 p = {0, 0, 0, 0};
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            u32x4 lo, hi;
            e4m3x16_to_bf16_nat(wb[d][b], lo, hi);
            p = mfma16x16x32(lo, xb[d][2 * b], p);
            p = mfma16x16x32(hi, xb[d][2 * b + 1], p);
          }
          const float sc = j < 2 ? sb[d][0] : sb[d][1];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] += sc * p[q];
        }
        if (c_l == SW - 1) {   // end of a task: reduce over the waves, SwiGLU, h
          const int task = (int)blockIdx.x + c_tk * (int)gridDim.x;
          const int g = task / RA, t = task - g * RA;
          f32x4(&rb)[NW][64] = red[c_tk & 1];
          rb[wv][lane] = acc;
          __syncthreads();
          if (wv == 0 && j < 2 && tok) {
            f32x4 Gv = rb[0][lane], Uv = rb[0][lane + 32];
#pragma unroll
            for (int w2 = 1; w2 < NW; ++w2) {
              Gv += rb[w2][lane];
              Uv += rb[w2][lane + 32];
            }
            uint16_t* hrow = a.h + ((size_t)g * kDecTok + r) * I + 8 * t + 4 * j;
            const uint32_t h01 = f32_to_bf16_rne(silu_f32(Gv[0]) * Uv[0]) | ((uint32_t)f32_to_bf16_rne(silu_f32(Gv[1]) * Uv[1]) << 16);
            const uint32_t h23 = f32_to_bf16_rne(silu_f32(Gv[2]) * Uv[2]) | ((uint32_t)f32_to_bf16_rne(silu_f32(Gv[3]) * Uv[3]) << 16);
            *reinterpret_cast<u32x2*>(hrow) = u32x2{h01, h23};
          }
          acc = f32x4{0, 0, 0, 0};
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

// down projection + gate weights.  Task (brick row t of H, half): the output
// row's steps over (group, 2-brick K step) are split in two halves; the NW
// waves take 1/NW of the half each, scale each step's sum by the token's gate
// weight (and the FP8 block scale), meet in LDS, and wave 0 adds the 16 x T
// partial into y, zeroed by the gate/up launch.  Exactly two additions land on
// each y element and two additions into 0 commute exactly, so y has the same
// bits whichever half lands first.  Continuous per-wave step sequence as in
// the gate/up launch.
template <bool FP8, int D, int NW>
__global__ __launch_bounds__(NW * 64) void dec_dn_kernel(DecArgs a) {
  __shared__ int s_gslot[kDecPmax];
  __shared__ float s_gw[kDecPmax * kDecTok];
  __shared__ int s_G;
  __shared__ unsigned long long s_tab[kPlanTab];
  __shared__ f32x4 red[2][NW][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I, T = a.T;
  if (wv == 0) wave_plan(a.pick_slot, a.w, T * a.k, a.k, a.n_slots, a.G_max, s_gslot, s_gw, &s_G, s_tab);
  __syncthreads();
  const int G = s_G;
  const int nkt = FP8 ? I / 64 : I / 32;     // bricks per (row, slot)
  const int SB = (nkt + 1) >> 1;             // steps per (row, group)
  const int n = G * SB;                      // steps per output row
  const int SWB = ((n + 1) / 2 + NW - 1) / NW;   // steps per wave per task (larger half)
  const size_t dn_bytes = (size_t)H * I * (FP8 ? 1 : 2);
  const int ntask = 2 * (H / 16);
  const int ntk = ntask > (int)blockIdx.x ? (ntask - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
  const int nsteps = ntk * SWB;
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.h, (uint32_t)(2u * a.G_max * kDecTok * I));
  const bool tok = r < T;
  constexpr int XN = FP8 ? 4 : 2;
  u32x4 wb[D][2], hb[D][XN];
  float fb[D];
  int i_tk = 0, i_l = 0;
  auto issue = [&](int d) {
    const int task = (int)blockIdx.x + i_tk * (int)gridDim.x;
    const int t = task >> 1, half = task & 1;
    const int lo = half ? n / 2 : 0, hi = half ? n : n / 2;
    const int q = lo + wv * SWB + i_l;
    const bool ok = i_tk < ntk && i_l < SWB && wv * SWB + i_l < hi - lo;
    (void)q;
    const int qq = ok ? q : 0;
    const int g = qq / SB, s = qq - g * SB;
    const int slot = ok ? __builtin_amdgcn_readfirstlane(s_gslot[g]) : 0;   // slot 0 always exists
    const int tr = ok ? t : 0;
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc((const char*)a.w_down + (size_t)slot * dn_bytes + (size_t)tr * nkt * 1024, (uint32_t)(nkt * 1024));
    const uint32_t wo = oob_sel(ok, (uint32_t)s * 2048u + lane * 16u);
    wb[d][0] = bload_nt(wr, wo);
    wb[d][1] = bload_nt(wr, oob_sel(ok, wo + 1024u));
    const uint32_t hrow = (uint32_t)((g * kDecTok + r) * I);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int k0 = FP8 ? 128 * s + 64 * b : 64 * s + 32 * b;
      const bool ho = ok && tok && k0 < I;
      const uint32_t off = oob_sel(ho, (hrow + k0 + (FP8 ? 16 : 8) * j) * 2u);
      if (FP8) {
        hb[d][2 * b] = bload(hr, off);
        hb[d][2 * b + 1] = bload(hr, oob_sel(ho, off + 16u));
      } else {
        hb[d][b] = bload(hr, off);
      }
    }
    float f = ok ? s_gw[g * kDecTok + r] : 0.f;
    if (FP8) f *= a.s_down[((size_t)slot * (H / 128) + (16 * tr) / 128) * (I / 128) + s];
    fb[d] = f;
    if (++i_l == SWB) {
      i_l = 0;
      ++i_tk;
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d);
  f32x4 acc = {0, 0, 0, 0};
  int c_tk = 0, c_l = 0;
  for (int i0 = 0; i0 < nsteps; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (i0 + d < nsteps) {
        f32x4 p = {0, 0, 0, 0};
        if (!FP8) {
          p = mfma16x16x32(wb[d][0], hb[d][0], p);
          p = mfma16x16x32(wb[d][1], hb[d][1], p);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            u32x4 lo, hi;
            e4m3x16_to_bf16_nat(wb[d][b], lo, hi);
            p = mfma16x16x32(lo, hb[d][2 * b], p);
            p = mfma16x16x32(hi, hb[d][2 * b + 1], p);
          }
        }
        const float f = fb[d];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += f * p[q];
        if (c_l == SWB - 1) {   // end of a task: reduce over the waves, add into y
          const int task = (int)blockIdx.x + c_tk * (int)gridDim.x;
          const int t = task >> 1;
          f32x4(&rb)[NW][64] = red[c_tk & 1];
          rb[wv][lane] = acc;
          __syncthreads();
          if (wv == 0 && tok) {
            f32x4 Y = rb[0][lane];
#pragma unroll
            for (int w2 = 1; w2 < NW; ++w2) Y += rb[w2][lane];
            float* yr = a.y + (size_t)r * H + 16 * t + 4 * j;
#pragma unroll
            for (int q = 0; q < 4; ++q) atomicAdd(yr + q, Y[q]);
          }
          acc = f32x4{0, 0, 0, 0};
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

// ================================================================ prefill
constexpr int kBM = 128;          // rows (pairs) per tile
constexpr int kPfThreads = 256;   // 4 waves, 2 x 2, 64 x 64 each

struct PfArgs {
  const void* w_gu;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int H, I, n_slots, T, k, P, max_tiles;
  const uint16_t* x;
  const int32_t* pick_slot;
  const float* w;
  float* y;
  // workspace
  int32_t* cnt;          // [n_slots]
  int32_t* off;          // [n_slots]
  int32_t* n_tiles;      // [1]
  int32_t* tile_slot;    // [max_tiles]
  int32_t* tile_m0;      // [max_tiles]
  int32_t* sorted_pair;  // [P]
  int32_t* pair_pos;     // [P]
  uint16_t* h;           // [P][I]
  float* o;              // [P][H]
};

// counting sort of the (token, pick) pairs by slot; one workgroup
__global__ __launch_bounds__(1024) void pf_sort_kernel(PfArgs a) {
  __shared__ int cnt[4096];
  __shared__ int base[4096];
  __shared__ int wsum[16];
  __shared__ int wsum2[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int S = a.n_slots;
  for (int s = tid; s < S; s += 1024) cnt[s] = 0;
  __syncthreads();
  for (int p = tid; p < a.P; p += 1024) {
    int s = a.pick_slot[p];
    if (s >= 0 && s < S) atomicAdd(&cnt[s], 1);
  }
  __syncthreads();
  // exclusive scans of counts and of tile counts; thread handles 4 slots
  int c[4], tcount[4], ls = 0, lt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int s = tid * 4 + i;
    c[i] = s < S ? cnt[s] : 0;
    tcount[i] = (c[i] + kBM - 1) / kBM;
    ls += c[i];
    lt += tcount[i];
  }
  int is = ls, it = lt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o1 = __shfl_up(is, d, 64), o2 = __shfl_up(it, d, 64);
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
  int bs = 0, bt = 0, tot_t = 0;
  for (int w2 = 0; w2 < 16; ++w2) {
    if (w2 < wv) {
      bs += wsum[w2];
      bt += wsum2[w2];
    }
    tot_t += wsum2[w2];
  }
  int es = bs + is - ls, et = bt + it - lt;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int s = tid * 4 + i;
    if (s < S) {
      base[s] = es;
      a.off[s] = es;
      a.cnt[s] = c[i];
      for (int q = 0; q < tcount[i]; ++q) {
        if (et + q < a.max_tiles) {
          a.tile_slot[et + q] = s;
          a.tile_m0[et + q] = q * kBM;
        }
      }
    }
    es += c[i];
    et += tcount[i];
  }
  if (tid == 0) *a.n_tiles = tot_t < a.max_tiles ? tot_t : a.max_tiles;
  __syncthreads();
  for (int p = tid; p < a.P; p += 1024) {
    int s = a.pick_slot[p];
    int pos = -1;
    if (s >= 0 && s < S) {
      pos = atomicAdd(&base[s], 1);
      a.sorted_pair[pos] = p;
    }
    a.pair_pos[p] = pos;
  }
}

// Grouped GEMM tile C[128 pairs x 128 weight rows] over one slot's segment;
// weights are bricks read as MFMA B operands.  GATEUP: A = gathered x rows,
// B = gate/up brick rows (16 B-rows = 8 gate + 8 up of the same outputs),
// epilogue h = silu(g) * u (BF16).  DOWN: A = h rows of the segment, B =
// W_down bricks, epilogue o = w_pair * acc (FP32).  Global -> register ->
// LDS staging is double-buffered: the next K step's loads are in flight while
// the current one computes.  FP8 bricks are expanded exactly to BF16 when
// read from LDS; the 128 x 128 scale multiplies the block partial once.
template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(kPfThreads) void pf_gemm_kernel(PfArgs a) {
  constexpr int BK = FP8 ? 128 : 64;           // one FP8 scale block per step; 2 bricks per 16 B-rows
  constexpr int KB = FP8 ? 64 : 32;            // brick K width
  constexpr int ASTR = BK + 8;                 // A row stride in LDS (BF16 elements)
  constexpr int A_ELEMS = kBM * ASTR;
  constexpr int B_BYTES = 16 * 1024;           // 8 groups of 16 B-rows x 2 bricks
  constexpr int ACH = kBM * BK / 16;           // 16-element A chunks per step
  constexpr int ACT = ACH / kPfThreads;        // per thread
  constexpr int BCT = (B_BYTES / 16) / kPfThreads;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][A_ELEMS];
  __shared__ __attribute__((aligned(16))) char Bs[2][B_BYTES];
  __shared__ int rowtok[kBM];

  const int tile = blockIdx.x;
  if (tile >= *a.n_tiles) return;
  const int slot = a.tile_slot[tile];
  const int m0 = a.tile_m0[tile];
  const int seg = a.off[slot];
  const int mrows = min(kBM, a.cnt[slot] - m0);
  const int K = GATEUP ? a.H : a.I;
  const int nkt = K / KB;
  const int n0 = blockIdx.y * 128;             // first B row (gate/up rows or H rows)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int r = lane & 15, j = lane >> 4;

  if (tid < kBM) {
    int pr = -1;
    if (tid < mrows) pr = GATEUP ? a.sorted_pair[seg + m0 + tid] / a.k : seg + m0 + tid;
    rowtok[tid] = pr;
  }
  const char* bbase = (const char*)(GATEUP ? a.w_gu : a.w_down) +
                      (size_t)slot * (GATEUP ? 2 : 1) * a.I * a.H * (FP8 ? 1 : 2) + (size_t)(n0 / 16) * nkt * 1024;
  float sc_lane = 1.f;
  const float* scp = nullptr;
  if (FP8) {
    const int nbk = K / 128;
    if (GATEUP)   // B column r of a 16-row group: gate (r < 8) or up; all 64 outputs share one scale row block
      scp = (r < 8 ? a.s_gate : a.s_up) + ((size_t)slot * (a.I / 128) + (n0 / 2) / 128) * nbk;
    else
      scp = a.s_down + ((size_t)slot * (a.H / 128) + n0 / 128) * nbk;
  }
  const uint16_t* asrc = GATEUP ? a.x : a.h;
  const int astride = GATEUP ? a.H : a.I;
  __syncthreads();

  u32x4 ra[ACT][2], rb[BCT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int c = 0; c < ACT; ++c) {
      const int ch = tid + c * kPfThreads;
      const int row = ch / (BK / 16), kc = (ch % (BK / 16)) * 16;
      const int src = rowtok[row];
      if (src >= 0) {
        const uint16_t* p = asrc + (size_t)src * astride + k0 + kc;
        ra[c][0] = ld16(p);
        ra[c][1] = ld16(p + 8);
      } else {
        ra[c][0] = u32x4{0, 0, 0, 0};
        ra[c][1] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int c = 0; c < BCT; ++c) {
      const int ch = tid + c * kPfThreads;     // brick bi = ch / 64 (group bi/2, sub bi%2), lane ch % 64
      const int bi = ch >> 6, gi = bi >> 1, sub = bi & 1;
      rb[c] = ld16_nt(bbase + ((size_t)gi * nkt + k0 / KB + sub) * 1024 + (ch & 63) * 16);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < ACT; ++c) {
      const int ch = tid + c * kPfThreads;
      const int row = ch / (BK / 16), kc = (ch % (BK / 16)) * 16;
      uint16_t* d = &As[buf][row * ASTR + kc];
      if (FP8) {
        u32x4 ev, od;
        split_even_odd(ra[c][0], ra[c][1], ev, od);
        *reinterpret_cast<u32x4*>(d) = ev;
        *reinterpret_cast<u32x4*>(d + 8) = od;
      } else {
        *reinterpret_cast<u32x4*>(d) = ra[c][0];
        *reinterpret_cast<u32x4*>(d + 8) = ra[c][1];
      }
    }
#pragma unroll
    for (int c = 0; c < BCT; ++c) {
      const int ch = tid + c * kPfThreads;
      *reinterpret_cast<u32x4*>(&Bs[buf][ch * 16]) = rb[c];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0, 0, 0, 0};

  gload(0);
  lstore(0);
  __syncthreads();
  const int nsteps = K / BK;
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) gload((st + 1) * BK);
    if (!FP8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *reinterpret_cast<const u32x4*>(&As[buf][(wm * 64 + mi * 16 + r) * ASTR + ks * 32 + j * 8]);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          bfr[ni] = *reinterpret_cast<const u32x4*>(&Bs[buf][((wn * 4 + ni) * 2 + ks) * 1024 + lane * 16]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16x16x32(af[mi], bfr[ni], acc[mi][ni]);
      }
    } else {
      f32x4 part[4][4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) part[mi][ni] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 ae[4], ao[4], be[4], bo[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const uint16_t* p = &As[buf][(wm * 64 + mi * 16 + r) * ASTR + hh * 64 + j * 16];
          ae[mi] = *reinterpret_cast<const u32x4*>(p);
          ao[mi] = *reinterpret_cast<const u32x4*>(p + 8);
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const u32x4 q = *reinterpret_cast<const u32x4*>(&Bs[buf][((wn * 4 + ni) * 2 + hh) * 1024 + lane * 16]);
          e4m3x16_to_bf16(q, be[ni], bo[ni]);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            part[mi][ni] = mfma16x16x32(ae[mi], be[ni], part[mi][ni]);
            part[mi][ni] = mfma16x16x32(ao[mi], bo[ni], part[mi][ni]);
          }
      }
      sc_lane = scp[st];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mi][ni][i] += sc_lane * part[mi][ni][i];
    }
    if (st + 1 < nsteps) {
      lstore(buf ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue.  Lane holds C[row = 4j + i][col = r] of each 16x16 tile.
  if (GATEUP) {
    // col r < 8: gate, r >= 8: up of output 8*(n0/16 + wn*4 + ni) + (r & 7)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = acc[mi][ni][i];
          const float u = __shfl_xor(v, 8, 64);
          const int row = wm * 64 + mi * 16 + 4 * j + i;
          if (r < 8 && row < mrows) {
            const int io = n0 / 2 + (wn * 4 + ni) * 8 + r;
            a.h[(size_t)(seg + m0 + row) * a.I + io] = f32_to_bf16_rne(silu_f32(v) * u);
          }
        }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + mi * 16 + 4 * j + i;
        if (row < mrows) {
          const int pos = seg + m0 + row;
          const float wp = a.w[a.sorted_pair[pos]];
          float* orow = a.o + (size_t)pos * a.H + n0 + wn * 64;
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) orow[ni * 16 + r] = wp * acc[mi][ni][i];
        }
      }
  }
}

// y[t] = sum_j o[pos(t, j)] in pick order (deterministic)
__global__ __launch_bounds__(256) void pf_combine_kernel(PfArgs a) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = a.H / 4;
  if (gid >= (size_t)a.T * per_row) return;
  const int t = (int)(gid / per_row), c = (int)(gid % per_row) * 4;
  f32x4 s = {0, 0, 0, 0};
  for (int jj = 0; jj < a.k; ++jj) {
    const int pos = a.pair_pos[(size_t)t * a.k + jj];
    if (pos >= 0) s += *reinterpret_cast<const f32x4*>(a.o + (size_t)pos * a.H + c);
  }
  *reinterpret_cast<f32x4*>(a.y + (size_t)t * a.H + c) = s;
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
  size_t h, total;
};
static DecWs dec_ws(int T_max, int k, int H, int I, int n_slots) {
  DecWs w{};
  int G = T_max * k < n_slots ? T_max * k : n_slots;
  size_t off = 0;
  w.h = off; off = align256(off + 2 * (size_t)G * kDecTok * I);
  w.total = off;
  return w;
}

// Resident workgroups per CU of each decode kernel, and the CU count, per device.
struct DecOcc {
  int cus = 0;
  int gu[2] = {0, 0}, dn[2] = {0, 0};
};
constexpr int kDecD_BF16 = 4, kDecD_FP8 = 4;   // register-ring depth in 2-brick steps (gate/up)
constexpr int kDnD_BF16 = 4, kDnD_FP8 = 4;     // (down)
constexpr int kGuW = 4, kDnW = 16;              // waves per workgroup
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
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.gu[0], dec_gu_kernel<false, kDecD_BF16, kGuW>, kGuW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.gu[1], dec_gu_kernel<true, kDecD_FP8, kGuW>, kGuW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.dn[0], dec_dn_kernel<false, kDnD_BF16, kDnW>, kDnW * 64, 0));
    MOE_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.dn[1], dec_dn_kernel<true, kDnD_FP8, kDnW>, kDnW * 64, 0));
    for (int i = 0; i < 2; ++i) {
      if (o.gu[i] < 1) o.gu[i] = 1;
      if (o.dn[i] < 1) o.dn[i] = 1;
    }
    o.cus = cus > 0 ? cus : 1;
  }
  *out = o;
  return MOE_OK;
}

struct PfWs {
  size_t cnt, off, nt, tslot, tm0, sp, pp, h, o, total;
  int max_tiles;
};
static PfWs pf_ws(int T_max, int k, int H, int I, int n_slots) {
  PfWs w{};
  size_t P = (size_t)T_max * k;
  w.max_tiles = (int)((P + kBM - 1) / kBM) + n_slots;
  size_t off = 0;
  w.cnt = off; off = align256(off + 4 * (size_t)n_slots);
  w.off = off; off = align256(off + 4 * (size_t)n_slots);
  w.nt = off; off = align256(off + 4);
  w.tslot = off; off = align256(off + 4 * (size_t)w.max_tiles);
  w.tm0 = off; off = align256(off + 4 * (size_t)w.max_tiles);
  w.sp = off; off = align256(off + 4 * P);
  w.pp = off; off = align256(off + 4 * P);
  w.h = off; off = align256(off + 2 * P * I);
  w.o = off; off = align256(off + 4 * P * H);
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
  if (mode == MOE_FWD_DECODE) {
    if (T_max > kDecTok || T_max * k > kDecPmax)
      MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T_max <= %d and T_max*k <= %d", kDecTok, kDecPmax);
    *bytes = dec_ws(T_max, k, H, I, n_slots).total;
  } else if (mode == MOE_FWD_PREFILL) {
    if (n_slots > 4096) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs n_slots <= 4096");
    *bytes = pf_ws(T_max, k, H, I, n_slots).total;
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

extern "C" moe_status moe_expert_forward(const moe_slots* slots, const uint16_t* x, const int32_t* pick_slot,
                                         const float* w, int32_t T, int32_t k, float* y, void* ws, size_t ws_bytes,
                                         uint32_t mode, hipStream_t stream) {
  clear_error();
  moe_status st = check_slots(slots);
  if (st) return st;
  if (T < 0 || k < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad T=%d k=%d", T, k);
  if (T == 0) return MOE_OK;
  if (!x || !pick_slot || !w || !y || !ws) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(x) || !aligned16(y)) MOE_FAIL(MOE_ERR_ARG, "x and y must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) & 255) MOE_FAIL(MOE_ERR_ARG, "workspace must be 256-byte aligned");
  const bool fp8 = slots->wtype == MOE_W_FP8_B128;
  const int H = slots->H, I = slots->I;
  char* wsb = (char*)ws;

  if (mode == MOE_FWD_DECODE) {
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
    a.h = (uint16_t*)(wsb + L.h);
    a.G_max = T * k < slots->n_slots ? T * k : slots->n_slots;
    const int f = fp8 ? 1 : 0;
    const long gu_tasks = (long)a.G_max * (I / 8), dn_tasks = 2L * (H / 16);
    const unsigned g1 = (unsigned)std::min<long>(gu_tasks, (long)occ.cus * occ.gu[f]);
    const unsigned g2 = (unsigned)std::min<long>(dn_tasks, (long)occ.cus * occ.dn[f]);
    if (fp8) {
      dec_gu_kernel<true, kDecD_FP8, kGuW><<<g1, kGuW * 64, 0, stream>>>(a);
      dec_dn_kernel<true, kDnD_FP8, kDnW><<<g2, kDnW * 64, 0, stream>>>(a);
    } else {
      dec_gu_kernel<false, kDecD_BF16, kGuW><<<g1, kGuW * 64, 0, stream>>>(a);
      dec_dn_kernel<false, kDnD_BF16, kDnW><<<g2, kDnW * 64, 0, stream>>>(a);
    }
    MOE_LAUNCHED();
    return MOE_OK;
  }
  if (mode != MOE_FWD_PREFILL) MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  if (slots->n_slots > 4096) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs n_slots <= 4096");
  if (H % 128 || I % 64) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs H %% 128 == 0 and I %% 64 == 0");
  PfWs L = pf_ws(T, k, H, I, slots->n_slots);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  PfArgs a{};
  a.w_gu = slots->w_gate_up; a.w_down = slots->w_down;
  a.s_gate = slots->s_gate; a.s_up = slots->s_up; a.s_down = slots->s_down;
  a.H = H; a.I = I; a.n_slots = slots->n_slots; a.T = T; a.k = k; a.P = T * k;
  a.max_tiles = L.max_tiles;
  a.x = x; a.pick_slot = pick_slot; a.w = w; a.y = y;
  a.cnt = (int32_t*)(wsb + L.cnt);
  a.off = (int32_t*)(wsb + L.off);
  a.n_tiles = (int32_t*)(wsb + L.nt);
  a.tile_slot = (int32_t*)(wsb + L.tslot);
  a.tile_m0 = (int32_t*)(wsb + L.tm0);
  a.sorted_pair = (int32_t*)(wsb + L.sp);
  a.pair_pos = (int32_t*)(wsb + L.pp);
  a.h = (uint16_t*)(wsb + L.h);
  a.o = (float*)(wsb + L.o);
  pf_sort_kernel<<<1, 1024, 0, stream>>>(a);
  const size_t ncomb = ((size_t)T * (H / 4) + 255) / 256;
  if (fp8) {
    pf_gemm_kernel<true, true><<<dim3(L.max_tiles, I / 64), kPfThreads, 0, stream>>>(a);
    pf_gemm_kernel<true, false><<<dim3(L.max_tiles, H / 128), kPfThreads, 0, stream>>>(a);
  } else {
    pf_gemm_kernel<false, true><<<dim3(L.max_tiles, I / 64), kPfThreads, 0, stream>>>(a);
    pf_gemm_kernel<false, false><<<dim3(L.max_tiles, H / 128), kPfThreads, 0, stream>>>(a);
  }
  pf_combine_kernel<<<(unsigned)ncomb, 256, 0, stream>>>(a);
  MOE_LAUNCHED();
  return MOE_OK;
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
