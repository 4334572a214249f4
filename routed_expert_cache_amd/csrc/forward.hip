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
constexpr int kDecTok = 16;     // MFMA N: tokens of one decode call
constexpr int kDecPmax = 512;   // T * k picks

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
  const uint16_t* xb;        // B-operand source [T][H]: x (BF16) or x permuted even/odd (FP8)
  uint16_t* xperm;           // workspace [T][H] (FP8 only)
  uint16_t* h;               // workspace [G_max][16][I]
  int G_max;
  int kp2;                   // K-parts of the down projection per expert
};

// Group plan in LDS: groups are the distinct valid slots of pick_slot in
// order of first appearance.  s_gslot[g] = slot of group g; if s_gw is not
// NULL, s_gw[g*16 + t] = gate weight of token t's pick of group g (0 if
// none).  Returns the number of groups.  Contains barriers; all threads call.
template <int NT>
__device__ int plan_groups(const DecArgs& a, int* s_ps, int* s_first, int* s_gslot, float* s_gw, int* s_n) {
  const int P = a.T * a.k, tid = threadIdx.x;
  for (int p = tid; p < P; p += NT) {
    const int s = a.pick_slot[p];
    s_ps[p] = (s >= 0 && s < a.n_slots) ? s : -1;
  }
  if (s_gw)
    for (int i = tid; i < a.G_max * kDecTok; i += NT) s_gw[i] = 0.f;
  if (tid == 0) *s_n = 0;
  __syncthreads();
  for (int p = tid; p < P; p += NT) {
    const int s = s_ps[p];
    bool first = s >= 0;
    for (int q = 0; q < p && first; ++q) first = s_ps[q] != s;
    s_first[p] = first;
    if (first) atomicAdd(s_n, 1);
  }
  __syncthreads();
  for (int p = tid; p < P; p += NT) {
    const int s = s_ps[p];
    if (s < 0) continue;
    int fq = p;
    if (!s_first[p])
      for (int q = 0; q < p; ++q)
        if (s_ps[q] == s) { fq = q; break; }
    int g = 0;
    for (int q = 0; q < fq; ++q) g += s_first[q];
    if (fq == p) s_gslot[g] = s;
    if (s_gw) s_gw[g * kDecTok + p / a.k] = a.w[p];
  }
  __syncthreads();
  return *s_n;
}

// FP8 only: x -> x permuted even/odd inside each 16-group, 16 elements per thread
__global__ __launch_bounds__(256) void dec_xperm_kernel(DecArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int per_row = a.H / 16;
  if (c >= a.T * per_row) return;
  const int t = c / per_row, kc = (c % per_row) * 16;
  const u32x4 v0 = ld16(a.x + (size_t)t * a.H + kc);
  const u32x4 v1 = ld16(a.x + (size_t)t * a.H + kc + 8);
  u32x4 ev, od;
  split_even_odd(v0, v1, ev, od);
  uint16_t* dst = a.xperm + (size_t)t * a.H + kc;
  *reinterpret_cast<u32x4*>(dst) = ev;
  *reinterpret_cast<u32x4*>(dst + 8) = od;
}

// gate/up + SwiGLU.  One workgroup per (gate/up brick row t = 8 rows of I,
// group).  The brick's A rows 0..7 are gate rows and 8..15 the same up rows,
// so one fragment holds gate and up of the same outputs.  Waves split K and
// issue a batch of contiguous 1 KB brick loads (plus the matching x loads)
// before its MFMAs.  Workgroups of group 0 also zero y for the down launch.
template <bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) void dec_gateup_kernel(DecArgs a) {
  __shared__ int s_ps[kDecPmax], s_first[kDecPmax], s_gslot[kDecPmax];
  __shared__ int s_n;
  __shared__ f32x4 red[NW][64];
  if (blockIdx.y == 0)
    for (int i = blockIdx.x * NW * 64 + threadIdx.x; i < a.T * a.H; i += gridDim.x * NW * 64) a.y[i] = 0.f;
  const int nG = plan_groups<NW * 64>(a, s_ps, s_first, s_gslot, nullptr, &s_n);
  const int g = blockIdx.y;
  if (g >= nG) return;
  const int slot = s_gslot[g];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I;
  const bool tok = r < a.T;
  f32x4 acc = {0, 0, 0, 0};
  if (!FP8) {
    const int nkt = H / 32;
    const uint16_t* gu = (const uint16_t*)a.w_gu + (size_t)slot * 2 * I * H + (size_t)t * nkt * 512 + lane * 8;
    const uint16_t* xr = a.xb + (size_t)(tok ? r : 0) * H + j * 8;
    const int kb = wv * nkt / NW, ke = (wv + 1) * nkt / NW;
    constexpr int CH = 8;
    for (int k0 = kb; k0 < ke; k0 += CH) {
      u32x4 av[CH], bv[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (k0 + c < ke) av[c] = ld16_nt(gu + (size_t)(k0 + c) * 512);
#pragma unroll
      for (int c = 0; c < CH; ++c) bv[c] = (tok && k0 + c < ke) ? ld16(xr + (k0 + c) * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (k0 + c < ke) acc = mfma16x16x32(av[c], bv[c], acc);
    }
  } else {
    const int nkt = H / 64, nbk = H / 128;
    const uint8_t* gu = (const uint8_t*)a.w_gu + (size_t)slot * 2 * I * H + (size_t)t * nkt * 1024 + lane * 16;
    const uint16_t* xr = a.xb + (size_t)(tok ? r : 0) * H + j * 16;
    // C rows 4j+i: j < 2 are gate rows, j >= 2 up rows, each with its scale row
    const float* sc = (j < 2 ? a.s_gate : a.s_up) + ((size_t)slot * (I / 128) + (8 * t) / 128) * nbk;
    const int bb = wv * nbk / NW, be = (wv + 1) * nbk / NW;
    constexpr int CB = 4;   // 128-K blocks per batch: 8 brick loads in flight per lane
    for (int b0 = bb; b0 < be; b0 += CB) {
      u32x4 q[CB][2], xv[CB][4];
#pragma unroll
      for (int c = 0; c < CB; ++c)
        if (b0 + c < be) {
          q[c][0] = ld16_nt(gu + (size_t)(2 * (b0 + c)) * 1024);
          q[c][1] = ld16_nt(gu + (size_t)(2 * (b0 + c) + 1) * 1024);
        }
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          xv[c][v] = (tok && b0 + c < be) ? ld16(xr + (b0 + c) * 128 + (v >> 1) * 64 + (v & 1) * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        if (b0 + c >= be) break;
        f32x4 p = {0, 0, 0, 0};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 ae, ao;
          e4m3x16_to_bf16(q[c][hh], ae, ao);
          p = mfma16x16x32(ae, xv[c][2 * hh], p);
          p = mfma16x16x32(ao, xv[c][2 * hh + 1], p);
        }
        const float s = sc[b0 + c];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += s * p[i];
      }
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && j < 2) {
    f32x4 G = red[0][lane], U = red[0][lane + 32];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      G += red[w][lane];
      U += red[w][lane + 32];
    }
    if (tok) {
      uint16_t* hrow = a.h + ((size_t)g * kDecTok + r) * I;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 8 * t + 4 * j + i;
        const int pos = FP8 ? ((o & ~15) + perm16(o & 15)) : o;
        hrow[pos] = f32_to_bf16_rne(silu_f32(G[i]) * U[i]);
      }
    }
  }
}

// down projection + gate weights.  Workgroup (16-row brick row t of H, half):
// half 0 takes the even groups, half 1 the odd ones; its waves take
// (group, K-part) units round-robin, sums are added in wave order, and each
// half adds its 16 x T partial into the zeroed y once.  Two additions into 0
// commute exactly, so y is the same bits whichever half lands first.
template <bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) void dec_down_kernel(DecArgs a) {
  __shared__ int s_ps[kDecPmax], s_first[kDecPmax], s_gslot[kDecPmax];
  __shared__ float s_gw[kDecPmax * kDecTok];
  __shared__ int s_n;
  __shared__ f32x4 red[NW][64];
  const int nG = plan_groups<NW * 64>(a, s_ps, s_first, s_gslot, s_gw, &s_n);
  const int t = blockIdx.x, hf = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I;
  const bool tok = r < a.T;
  const int KP = a.kp2;
  const int ngh = (nG - hf + 1) / 2;
  f32x4 acc = {0, 0, 0, 0};
  for (int u = wv; u < ngh * KP; u += NW) {
    const int g = 2 * (u / KP) + hf, part = u % KP;
    const int slot = s_gslot[g];
    const float wgt = s_gw[g * kDecTok + r];
    f32x4 blk = {0, 0, 0, 0};
    if (!FP8) {
      const int nkt = I / 32;
      const int kb = part * nkt / KP, ke = (part + 1) * nkt / KP;
      const uint16_t* wd = (const uint16_t*)a.w_down + (size_t)slot * H * I + (size_t)t * nkt * 512 + lane * 8;
      const uint16_t* hr = a.h + ((size_t)g * kDecTok + (tok ? r : 0)) * I + j * 8;
      constexpr int CH = 12;
      for (int k0 = kb; k0 < ke; k0 += CH) {
        u32x4 av[CH], bv[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (k0 + c < ke) av[c] = ld16_nt(wd + (size_t)(k0 + c) * 512);
#pragma unroll
        for (int c = 0; c < CH; ++c) bv[c] = (tok && k0 + c < ke) ? ld16(hr + (k0 + c) * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (k0 + c < ke) blk = mfma16x16x32(av[c], bv[c], blk);
      }
    } else {
      const int nkt = I / 64, nbk = I / 128;
      const int bb = part * nbk / KP, be = (part + 1) * nbk / KP;
      const uint8_t* wd = (const uint8_t*)a.w_down + (size_t)slot * H * I + (size_t)t * nkt * 1024 + lane * 16;
      const uint16_t* hr = a.h + ((size_t)g * kDecTok + (tok ? r : 0)) * I + j * 16;
      const float* sc = a.s_down + ((size_t)slot * (H / 128) + (16 * t) / 128) * nbk;
      constexpr int CB = 4;
      for (int b0 = bb; b0 < be; b0 += CB) {
        u32x4 qv[CB][2], hv[CB][4];
#pragma unroll
        for (int c = 0; c < CB; ++c)
          if (b0 + c < be) {
            qv[c][0] = ld16_nt(wd + (size_t)(2 * (b0 + c)) * 1024);
            qv[c][1] = ld16_nt(wd + (size_t)(2 * (b0 + c) + 1) * 1024);
          }
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            hv[c][v] = (tok && b0 + c < be) ? ld16(hr + (b0 + c) * 128 + (v >> 1) * 64 + (v & 1) * 8)
                                             : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          if (b0 + c >= be) break;
          f32x4 p = {0, 0, 0, 0};
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            u32x4 de, dd;
            e4m3x16_to_bf16(qv[c][hh], de, dd);
            p = mfma16x16x32(de, hv[c][2 * hh], p);
            p = mfma16x16x32(dd, hv[c][2 * hh + 1], p);
          }
          const float s = sc[b0 + c];
#pragma unroll
          for (int i = 0; i < 4; ++i) blk[i] += s * p[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += wgt * blk[i];
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    f32x4 Y = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) Y += red[w][lane];
    if (tok) {
      float* yr = a.y + (size_t)r * H + 16 * t + 4 * j;
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(yr + i, Y[i]);
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
  u32x4 ev, od;
  e4m3x16_to_bf16(q, ev, od);
  for (int t = 0; t < 16; ++t) {
    if (i + t >= n) break;
    const uint32_t v = (t & 1) ? od[t >> 2] : ev[t >> 2];
    out[i + t] = (uint16_t)(((t >> 1) & 1) ? (v >> 16) : (v & 0xFFFFu));
  }
}

// ================================================================ workspace layouts
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecWs {
  size_t xperm, h, total;
};
static DecWs dec_ws(int T_max, int k, int H, int I, int n_slots) {
  DecWs w{};
  int G = T_max * k < n_slots ? T_max * k : n_slots;
  size_t off = 0;
  w.xperm = off; off = align256(off + 2 * (size_t)T_max * H);
  w.h = off; off = align256(off + 2 * (size_t)G * kDecTok * I);
  w.total = off;
  return w;
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
    if (T_max > kDecTok || T_max * k > 512)
      MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T_max <= %d and T_max*k <= 512", kDecTok);
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
      MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T <= 16 and T*k <= 512 (T=%d k=%d)", T, k);
    DecWs L = dec_ws(T, k, H, I, slots->n_slots);
    if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
    DecArgs a{};
    a.w_gu = slots->w_gate_up; a.w_down = slots->w_down;
    a.s_gate = slots->s_gate; a.s_up = slots->s_up; a.s_down = slots->s_down;
    a.H = H; a.I = I; a.n_slots = slots->n_slots; a.T = T; a.k = k;
    a.x = x; a.pick_slot = pick_slot; a.w = w; a.y = y;
    a.xperm = (uint16_t*)(wsb + L.xperm);
    a.h = (uint16_t*)(wsb + L.h);
    a.xb = fp8 ? a.xperm : x;
    a.G_max = T * k < slots->n_slots ? T * k : slots->n_slots;
    // K-parts of the down projection: a unit keeps >= 12 bricks (BF16) / 4 blocks (FP8) of loads in flight
    const int ksteps = fp8 ? I / 128 : I / 32;
    const int unit = fp8 ? 4 : 12;
    int kp2 = 1;
    while (kp2 < 8 && ksteps % (2 * kp2) == 0 && ksteps / (2 * kp2) >= unit) kp2 *= 2;
    a.kp2 = kp2;
    constexpr int NW = 8;
    const dim3 g1(I / 8, a.G_max), g2(H / 16, 2);
    if (fp8) {
      dec_xperm_kernel<<<(T * (H / 16) + 255) / 256, 256, 0, stream>>>(a);
      dec_gateup_kernel<true, NW><<<g1, NW * 64, 0, stream>>>(a);
      dec_down_kernel<true, NW><<<g2, NW * 64, 0, stream>>>(a);
    } else {
      dec_gateup_kernel<false, NW><<<g1, NW * 64, 0, stream>>>(a);
      dec_down_kernel<false, NW><<<g2, NW * 64, 0, stream>>>(a);
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
