// Grouped SwiGLU expert evaluation of G = H u F, and the partial-sum merge.
//
// [FT] section "执行顺序与工程细节": after the cache update and the copy of F the
// GPU evaluates all of G as one grouped computation.  [OSDI] section 4.3: an
// expert is gate, up and down projections, down reads SiLU(gate) * up.
// [OSDI] section 4.2: FP8 weights are kept as stored, expanded in registers,
// dotted first and multiplied by the shared block scale once per block
// (post-scaling: scale * sum(w x) = sum(scale * w * x)).
//
// Decode (T <= 16): every slot in G is streamed once from HBM.  The MFMA
// 16x16x32 BF16 tile takes 16 weight rows as A and the (up to 16) tokens as
// B, so one weight read serves every token of the batch; tokens that did not
// pick a slot carry gate weight 0 in the down projection.
//   plan kernel    : groups = distinct slots of pick_slot (ascending), per
//                    token gate weight of each group; x padded to 16 rows
//                    (for FP8: K permuted even/odd inside each 16-group to
//                    match the register expansion of the codes)
//   gate/up kernel : one workgroup per (16-row tile of I, group); waves split
//                    K; h = silu(gate) * up rounded to BF16
//   down kernel    : one workgroup per 16-row tile of H; loops over the
//                    groups in order (deterministic), weights each group's
//                    block by its per-token gate weight
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

// ================================================================ decode
constexpr int kDecTok = 16;

struct DecArgs {
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int H, I, n_slots, T, k;
  const uint16_t* x;         // [T][H]
  const int32_t* pick_slot;  // [T*k]
  const float* w;            // [T*k]
  float* y;                  // [T][H]
  // workspace
  int32_t* nG;               // [1]
  int32_t* gslot;            // [G_max]
  float* gw;                 // [G_max][16]
  uint16_t* xpad;            // [16][H]
  uint16_t* h;               // [G_max][16][I]
  int G_max;
};

template <bool FP8>
__global__ __launch_bounds__(256) void dec_plan_kernel(DecArgs a) {
  if (blockIdx.x == 0) {
    __shared__ int s_slot[512];
    __shared__ int s_first[512];
    __shared__ float s_gw[512 * kDecTok];
    __shared__ int s_n;
    const int P = a.T * a.k;
    for (int i = threadIdx.x; i < a.G_max * kDecTok; i += 256) s_gw[i] = 0.f;
    for (int p = threadIdx.x; p < P; p += 256) {
      int s = a.pick_slot[p];
      s_slot[p] = (s >= 0 && s < a.n_slots) ? s : -1;
    }
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += 256) {
      int s = s_slot[p];
      bool first = s >= 0;
      for (int q = 0; q < p && first; ++q) first = s_slot[q] != s;
      s_first[p] = first;
      if (first) atomicAdd(&s_n, 1);
    }
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += 256) {
      int s = s_slot[p];
      if (s < 0) continue;
      int rank = 0;
      for (int q = 0; q < P; ++q) rank += (s_first[q] && s_slot[q] < s);
      if (s_first[p]) a.gslot[rank] = s;
      s_gw[rank * kDecTok + p / a.k] = a.w[p];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.G_max * kDecTok; i += 256) a.gw[i] = s_gw[i];
    if (threadIdx.x == 0) *a.nG = s_n;
  } else {
    // x -> xpad [16][H], 16 elements per thread
    const int c = (blockIdx.x - 1) * 256 + threadIdx.x;
    const int per_row = a.H / 16;
    if (c >= kDecTok * per_row) return;
    const int t = c / per_row, kc = (c % per_row) * 16;
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (t < a.T) {
      v0 = ld16(a.x + (size_t)t * a.H + kc);
      v1 = ld16(a.x + (size_t)t * a.H + kc + 8);
    }
    uint16_t* dst = a.xpad + (size_t)t * a.H + kc;
    if (FP8) {
      u32x4 ev, od;
      split_even_odd(v0, v1, ev, od);
      *reinterpret_cast<u32x4*>(dst) = ev;
      *reinterpret_cast<u32x4*>(dst + 8) = od;
    } else {
      *reinterpret_cast<u32x4*>(dst) = v0;
      *reinterpret_cast<u32x4*>(dst + 8) = v1;
    }
  }
}

template <bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) void dec_gateup_kernel(DecArgs a) {
  const int g = blockIdx.y;
  if (g >= *a.nG) return;
  const int slot = a.gslot[g];
  const int row0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I;
  f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  if (!FP8) {
    const uint16_t* wg = (const uint16_t*)a.w_gate + ((size_t)slot * I + row0 + r) * H + j * 8;
    const uint16_t* wu = (const uint16_t*)a.w_up + ((size_t)slot * I + row0 + r) * H + j * 8;
    const uint16_t* xb = a.xpad + (size_t)r * H + j * 8;
    const int nk = H / 32;
    const int kb = wv * nk / NW, ke = (wv + 1) * nk / NW;
#pragma unroll 4
    for (int kk = kb; kk < ke; ++kk) {
      u32x4 ag = ld16_nt(wg + kk * 32);
      u32x4 au = ld16_nt(wu + kk * 32);
      u32x4 b = ld16(xb + kk * 32);
      accg = mfma16x16x32(ag, b, accg);
      accu = mfma16x16x32(au, b, accu);
    }
  } else {
    const uint8_t* wg = (const uint8_t*)a.w_gate + ((size_t)slot * I + row0 + r) * H + j * 16;
    const uint8_t* wu = (const uint8_t*)a.w_up + ((size_t)slot * I + row0 + r) * H + j * 16;
    const uint16_t* xb = a.xpad + (size_t)r * H + j * 16;
    const int nbk = H / 128;
    const float* sg = a.s_gate + ((size_t)slot * (I / 128) + row0 / 128) * nbk;
    const float* su = a.s_up + ((size_t)slot * (I / 128) + row0 / 128) * nbk;
    const int bb = wv * nbk / NW, be = (wv + 1) * nbk / NW;
#pragma unroll 2
    for (int kb = bb; kb < be; ++kb) {
      f32x4 pg = {0, 0, 0, 0}, pu = {0, 0, 0, 0};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ko = kb * 128 + hh * 64;
        u32x4 qg = ld16_nt(wg + ko);
        u32x4 qu = ld16_nt(wu + ko);
        u32x4 xe = ld16(xb + ko), xo = ld16(xb + ko + 8);
        u32x4 ge, go, ue, uo;
        e4m3x16_to_bf16(qg, ge, go);
        e4m3x16_to_bf16(qu, ue, uo);
        pg = mfma16x16x32(ge, xe, pg);
        pg = mfma16x16x32(go, xo, pg);
        pu = mfma16x16x32(ue, xe, pu);
        pu = mfma16x16x32(uo, xo, pu);
      }
      const float cg = sg[kb], cu = su[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[i] += cg * pg[i];
        accu[i] += cu * pu[i];
      }
    }
  }
  __shared__ f32x4 red[NW][2][64];
  red[wv][0][lane] = accg;
  red[wv][1][lane] = accu;
  __syncthreads();
  if (wv == 0) {
    f32x4 G = red[0][0][lane], U = red[0][1][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      G += red[w][0][lane];
      U += red[w][1][lane];
    }
    uint16_t* hrow = a.h + ((size_t)g * kDecTok + r) * I;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 4 * j + i;
      const float hv = silu_f32(G[i]) * U[i];
      const int pos = FP8 ? ((row & ~15) + perm16(row & 15)) : row;
      hrow[pos] = f32_to_bf16_rne(hv);
    }
  }
}

template <bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) void dec_down_kernel(DecArgs a) {
  const int row0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int H = a.H, I = a.I;
  const int nG = *a.nG;
  f32x4 acc = {0, 0, 0, 0};
  for (int g = 0; g < nG; ++g) {
    const int slot = a.gslot[g];
    const float wgt = a.gw[g * kDecTok + r];
    f32x4 blk = {0, 0, 0, 0};
    if (!FP8) {
      const uint16_t* wd = (const uint16_t*)a.w_down + ((size_t)slot * H + row0 + r) * I + j * 8;
      const uint16_t* hb = a.h + ((size_t)g * kDecTok + r) * I + j * 8;
      const int nk = I / 32;
      const int kb = wv * nk / NW, ke = (wv + 1) * nk / NW;
#pragma unroll 4
      for (int kk = kb; kk < ke; ++kk) blk = mfma16x16x32(ld16_nt(wd + kk * 32), ld16(hb + kk * 32), blk);
    } else {
      const uint8_t* wd = (const uint8_t*)a.w_down + ((size_t)slot * H + row0 + r) * I + j * 16;
      const uint16_t* hb = a.h + ((size_t)g * kDecTok + r) * I + j * 16;
      const int nbk = I / 128;
      const float* sd = a.s_down + ((size_t)slot * (H / 128) + row0 / 128) * nbk;
      const int bb = wv * nbk / NW, be = (wv + 1) * nbk / NW;
      for (int kb = bb; kb < be; ++kb) {
        f32x4 p = {0, 0, 0, 0};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ko = kb * 128 + hh * 64;
          u32x4 q = ld16_nt(wd + ko);
          u32x4 he = ld16(hb + ko), ho = ld16(hb + ko + 8);
          u32x4 de, dd;
          e4m3x16_to_bf16(q, de, dd);
          p = mfma16x16x32(de, he, p);
          p = mfma16x16x32(dd, ho, p);
        }
        const float c = sd[kb];
#pragma unroll
        for (int i = 0; i < 4; ++i) blk[i] += c * p[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += wgt * blk[i];
  }
  __shared__ f32x4 red[NW][64];
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    f32x4 Y = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) Y += red[w][lane];
    if (r < a.T) *reinterpret_cast<f32x4*>(a.y + (size_t)r * H + row0 + 4 * j) = Y;
  }
}

// ================================================================ prefill
constexpr int kBM = 128;          // rows (pairs) per tile
constexpr int kPfThreads = 256;   // 4 waves, 2 x 2

struct PfArgs {
  const void* w_gate;
  const void* w_up;
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

// Grouped GEMM tile: C[128 x 128] = A[128 x K] * B[128 x K]^T over one slot's
// segment.  GATEUP: A = gathered x rows, B rows 0..63 = W_gate rows n0..n0+63,
// rows 64..127 = W_up rows n0..n0+63, epilogue h = silu(g) * u (BF16).
// DOWN: A = h rows of the segment, B = W_down rows n0..n0+127, epilogue
// o = w_pair * acc (FP32).  FP8 B operands are expanded exactly to BF16 when
// read from LDS; their 128 x 128 scale multiplies the block partial once.
template <bool FP8, bool GATEUP>
__global__ __launch_bounds__(kPfThreads) void pf_gemm_kernel(PfArgs a) {
  constexpr int BK = FP8 ? 128 : 64;
  constexpr int ASTR = BK + 8;                 // LDS row stride, BF16 elements
  constexpr int BSTR = FP8 ? (BK + 16) : (BK + 8);   // bytes (FP8) or elements (BF16)
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * ASTR];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[FP8 ? (128 * BSTR / 2) : (128 * BSTR)];
  __shared__ int rowtok[kBM];

  const int tile = blockIdx.x;
  if (tile >= *a.n_tiles) return;
  const int slot = a.tile_slot[tile];
  const int m0 = a.tile_m0[tile];
  const int seg = a.off[slot];
  const int mrows = min(kBM, a.cnt[slot] - m0);
  const int K = GATEUP ? a.H : a.I;
  const int N = GATEUP ? a.I : a.H;
  const int n0 = blockIdx.y * (GATEUP ? 64 : 128);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;          // wave tile: rows wm*64.., cols wn*64..
  const int r = lane & 15, j = lane >> 4;

  if (tid < kBM) {
    int pr = -1;
    if (tid < mrows) {
      pr = a.sorted_pair[seg + m0 + tid];
      if (GATEUP) pr = pr / a.k;               // token row of x
      else pr = seg + m0 + tid;                // row of h
    }
    rowtok[tid] = pr;
  }

  // B source rows
  const char* bsrc[2];
  const float* bscale[2] = {nullptr, nullptr};
  const size_t el = FP8 ? 1 : 2;
  if (GATEUP) {
    bsrc[0] = (const char*)a.w_gate + ((size_t)slot * N + n0) * K * el;
    bsrc[1] = (const char*)a.w_up + ((size_t)slot * N + n0) * K * el;
    if (FP8) {
      bscale[0] = a.s_gate + ((size_t)slot * (N / 128) + n0 / 128) * (K / 128);
      bscale[1] = a.s_up + ((size_t)slot * (N / 128) + n0 / 128) * (K / 128);
    }
  } else {
    bsrc[0] = (const char*)a.w_down + ((size_t)slot * N + n0) * K * el;
    bsrc[1] = bsrc[0] + (size_t)64 * K * el;
    if (FP8) bscale[0] = bscale[1] = a.s_down + ((size_t)slot * (N / 128) + n0 / 128) * (K / 128);
  }
  __syncthreads();

  f32x4 acc[4][4];
  f32x4 part[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0, 0, 0, 0};

  const uint16_t* asrc = GATEUP ? a.x : a.h;
  const int arow_stride = GATEUP ? a.H : a.I;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // ---- A tile: 128 rows x BK bf16, 16-element chunks (FP8: even/odd permuted)
    constexpr int ACH = kBM * BK / 16;
    for (int c = tid; c < ACH; c += kPfThreads) {
      const int row = c / (BK / 16), kc = (c % (BK / 16)) * 16;
      const int src = rowtok[row];
      u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      if (src >= 0) {
        const uint16_t* p = asrc + (size_t)src * arow_stride + k0 + kc;
        v0 = ld16(p);
        v1 = ld16(p + 8);
      }
      uint16_t* d = As + row * ASTR + kc;
      if (FP8) {
        u32x4 ev, od;
        split_even_odd(v0, v1, ev, od);
        *reinterpret_cast<u32x4*>(d) = ev;
        *reinterpret_cast<u32x4*>(d + 8) = od;
      } else {
        *reinterpret_cast<u32x4*>(d) = v0;
        *reinterpret_cast<u32x4*>(d + 8) = v1;
      }
    }
    // ---- B tile: 128 rows x BK (raw codes or bf16)
    constexpr int BROWB = BK * (FP8 ? 1 : 2);   // bytes per row in global
    constexpr int BCH = 128 * BROWB / 16;
    for (int c = tid; c < BCH; c += kPfThreads) {
      const int row = c / (BROWB / 16), cb = (c % (BROWB / 16)) * 16;
      const char* p = bsrc[row >> 6] + ((size_t)(row & 63) * K + k0) * el + cb;
      u32x4 v = ld16_nt(p);
      char* d = (char*)Bs + (size_t)row * (FP8 ? BSTR : BSTR * 2) + cb;
      *reinterpret_cast<u32x4*>(d) = v;
    }
    __syncthreads();

    if (!FP8) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 32) {
        u32x4 af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *reinterpret_cast<const u32x4*>(As + (wm * 64 + mi * 16 + r) * ASTR + ks + j * 8);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          bfr[ni] = *reinterpret_cast<const u32x4*>(Bs + (wn * 64 + ni * 16 + r) * BSTR + ks + j * 8);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16x16x32(af[mi], bfr[ni], acc[mi][ni]);
      }
    } else {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) part[mi][ni] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ko = hh * 64 + j * 16;
        u32x4 ae[4], ao[4], be[4], bo[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const uint16_t* p = As + (wm * 64 + mi * 16 + r) * ASTR + ko;
          ae[mi] = *reinterpret_cast<const u32x4*>(p);
          ao[mi] = *reinterpret_cast<const u32x4*>(p + 8);
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const u32x4 q = *reinterpret_cast<const u32x4*>((const char*)Bs + (wn * 64 + ni * 16 + r) * BSTR + ko);
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
      const int kb = k0 / 128;
      const float sc = bscale[wn][kb];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mi][ni][i] += sc * part[mi][ni][i];
    }
    __syncthreads();
  }

  // ---- epilogue.  Lane holds C[row = 4j + i][col = r] of each 16x16 tile.
  if (GATEUP) {
    // wave (wm, 0) has gate cols 0..63 (B rows 0..63), wave (wm, 1) up cols 0..63
    __shared__ float ups[kBM * 65];
    if (wn == 1) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) ups[(wm * 64 + mi * 16 + 4 * j + i) * 65 + ni * 16 + r] = acc[mi][ni][i];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 64 + mi * 16 + 4 * j + i;
          if (row < mrows) {
            uint16_t* hrow = a.h + (size_t)(seg + m0 + row) * a.I + n0;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
              const float u = ups[row * 65 + ni * 16 + r];
              hrow[ni * 16 + r] = f32_to_bf16_rne(silu_f32(acc[mi][ni][i]) * u);
            }
          }
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
  size_t nG, gslot, gw, xpad, h, total;
};
static DecWs dec_ws(int T_max, int k, int H, int I, int n_slots) {
  DecWs w{};
  int G = T_max * k < n_slots ? T_max * k : n_slots;
  size_t off = 0;
  w.nG = off; off = align256(off + 4);
  w.gslot = off; off = align256(off + 4 * (size_t)G);
  w.gw = off; off = align256(off + 4 * (size_t)G * kDecTok);
  w.xpad = off; off = align256(off + 2 * (size_t)kDecTok * H);
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
    if (T > kDecTok || T * k > 512) MOE_FAIL(MOE_ERR_SHAPE, "decode mode needs T <= 16 and T*k <= 512 (T=%d k=%d)", T, k);
    DecWs L = dec_ws(T, k, H, I, slots->n_slots);
    if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
    DecArgs a{};
    a.w_gate = slots->w_gate; a.w_up = slots->w_up; a.w_down = slots->w_down;
    a.s_gate = slots->s_gate; a.s_up = slots->s_up; a.s_down = slots->s_down;
    a.H = H; a.I = I; a.n_slots = slots->n_slots; a.T = T; a.k = k;
    a.x = x; a.pick_slot = pick_slot; a.w = w; a.y = y;
    a.nG = (int32_t*)(wsb + L.nG);
    a.gslot = (int32_t*)(wsb + L.gslot);
    a.gw = (float*)(wsb + L.gw);
    a.xpad = (uint16_t*)(wsb + L.xpad);
    a.h = (uint16_t*)(wsb + L.h);
    a.G_max = T * k < slots->n_slots ? T * k : slots->n_slots;
    const int xblocks = (kDecTok * (H / 16) + 255) / 256;
    constexpr int NW = 8;
    if (fp8) {
      dec_plan_kernel<true><<<1 + xblocks, 256, 0, stream>>>(a);
      dec_gateup_kernel<true, NW><<<dim3(I / 16, a.G_max), NW * 64, 0, stream>>>(a);
      dec_down_kernel<true, NW><<<H / 16, NW * 64, 0, stream>>>(a);
    } else {
      dec_plan_kernel<false><<<1 + xblocks, 256, 0, stream>>>(a);
      dec_gateup_kernel<false, NW><<<dim3(I / 16, a.G_max), NW * 64, 0, stream>>>(a);
      dec_down_kernel<false, NW><<<H / 16, NW * 64, 0, stream>>>(a);
    }
    MOE_LAUNCHED();
    return MOE_OK;
  }
  if (mode != MOE_FWD_PREFILL) MOE_FAIL(MOE_ERR_ARG, "bad mode %u", mode);
  if (slots->n_slots > 4096) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs n_slots <= 4096");
  if (H % 128 || I % 64) MOE_FAIL(MOE_ERR_SHAPE, "prefill mode needs H % 128 == 0 and I % 64 == 0");
  PfWs L = pf_ws(T, k, H, I, slots->n_slots);
  if (ws_bytes < L.total) MOE_FAIL(MOE_ERR_NO_SPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  PfArgs a{};
  a.w_gate = slots->w_gate; a.w_up = slots->w_up; a.w_down = slots->w_down;
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
