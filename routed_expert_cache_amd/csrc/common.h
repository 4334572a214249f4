// Internal helpers shared by the library's translation units (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/moe.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace moe {

// ---------------------------------------------------------------- host-side errors
void set_error(const char* fmt, ...);
void clear_error();

#define MOE_FAIL(code, ...)            \
  do {                                 \
    ::moe::set_error(__VA_ARGS__);     \
    return (code);                     \
  } while (0)

#define MOE_HIP(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      MOE_FAIL(MOE_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
               __LINE__);                                                                  \
  } while (0)

#define MOE_LAUNCHED()                                                                     \
  do {                                                                                     \
    hipError_t e_ = hipGetLastError();                                                     \
    if (e_ != hipSuccess)                                                                  \
      MOE_FAIL(MOE_ERR_HIP, "kernel launch failed: %s (%s:%d)", hipGetErrorString(e_),      \
               __FILE__, __LINE__);                                                        \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of one slot in each bank, in moe_slots order: gate_up, down, s_gate,
// s_up, s_down (the scale banks only for FP8).
struct BankBytes {
  size_t b[5];
  int nb;
};
inline BankBytes bank_bytes(int wtype, int H, int I) {
  BankBytes r{};
  size_t el = (wtype == MOE_W_BF16) ? 2 : 1;
  r.b[0] = el * 2 * (size_t)I * H;
  r.b[1] = el * (size_t)H * I;
  if (wtype == MOE_W_FP8_B128) {
    r.b[2] = r.b[3] = r.b[4] = sizeof(float) * (size_t)(I / 128) * (H / 128);
    r.nb = 5;
  } else {
    r.nb = 2;
  }
  return r;
}

// Validates the shape of a slot pool for the forward path.
moe_status check_slots(const moe_slots* s);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? nan : r);
}

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// operations, not for its global stores (which __syncthreads would also
// wait for, a full memory round trip).  For code whose waves exchange data
// through LDS only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over [base, base + bytes): a load past the end returns
// zero without a memory access, so masked loads need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Exact E4M3FN -> BF16 expansion ([OSDI] section 4.2 expands FP8 weights to
// BF16 before the BF16 product and scales afterwards).  16 codes (one 128-bit
// load) -> 16 BF16 in their natural order: `lo` holds codes 0..7 and `hi`
// codes 8..15.  gfx950 converts two OCP E4M3 codes to two BF16 per
// instruction; with the scale operand 1.0 the result is the code's exact
// value (every finite E4M3 value is a BF16 value), NaN codes give NaN.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, HIGH));
}
__device__ __forceinline__ void e4m3x16_to_bf16_nat(const u32x4& q, u32x4& lo, u32x4& hi) {
  lo = u32x4{e4m3x2_to_bf16x2<false>(q[0]), e4m3x2_to_bf16x2<true>(q[0]), e4m3x2_to_bf16x2<false>(q[1]),
             e4m3x2_to_bf16x2<true>(q[1])};
  hi = u32x4{e4m3x2_to_bf16x2<false>(q[2]), e4m3x2_to_bf16x2<true>(q[2]), e4m3x2_to_bf16x2<false>(q[3]),
             e4m3x2_to_bf16x2<true>(q[3])};
}

// ---------------------------------------------------------------- wave top-k
// Router selection for one token per wavefront ([FTK] routing and GPU-router
// paragraphs: top-k of the logits, gate weights = softmax over the kept k).
// Lane l holds the logits of experts l, l+64, ... as 32-bit keys whose
// unsigned order is the float order (sign-magnitude folded, -0 ranks as +0).
// Each of the k rounds takes the wave-wide maximum key (DPP exchanges inside
// each row of 16 lanes, then the four row results through scalar registers),
// finds the lowest expert index holding it with one ballot per key column
// (ties go to the lower index), and retires that key.  Lane j < k ends with
// pick j (rank order) and its weight.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- 15-i within each 16

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v)));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Ordered key of a float32 logit's bits: unsigned order of keys is the order
// of the values, -0 ranks as +0.
__device__ __forceinline__ uint32_t topk_key_of(uint32_t u) {
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Load one token's logits (row: buffer over its E floats) as ordered keys;
// bit v of `alive` marks key[v] as a real expert (v*64 + lane < E).
// topk_load issues the loads, topk_keys_of turns them into keys: callers that
// want other loads issued in between call the two halves.
template <int VPL>
__device__ __forceinline__ void topk_load(__amdgpu_buffer_rsrc_t row, uint32_t (&raw)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < VPL; ++v) raw[v] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(row, 4 * (v * 64 + lane), 0, 0);
}
template <int VPL>
__device__ __forceinline__ void topk_keys_of(const uint32_t (&raw)[VPL], int E, uint32_t (&key)[VPL], uint32_t& alive) {
  const int lane = threadIdx.x & 63;
  alive = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = v * 64 + lane;
    key[v] = topk_key_of(raw[v]);                   // 0 past E
    alive |= (e < E ? 1u : 0u) << v;
  }
}
template <int VPL>
__device__ __forceinline__ void topk_keys(__amdgpu_buffer_rsrc_t row, int E, uint32_t (&key)[VPL], uint32_t& alive) {
  uint32_t raw[VPL];
  topk_load<VPL>(row, raw);
  topk_keys_of<VPL>(raw, E, key, alive);
}

// Logit value of an ordered key (the inverse of the map in topk_keys_of).
__device__ __forceinline__ float topk_key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Softmax over the k kept logits, lane j < k holding pick j (pick 0 the
// maximum); the weight of this lane's pick.
__device__ __forceinline__ float topk_softmax(float my_z, int k) {
  const int lane = threadIdx.x & 63;
  const float zmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_z), 0));
  const float ex = (lane < k) ? expf(my_z - zmax) : 0.f;
  return ex / wave_sum_f32(ex);
}

template <int VPL>
__device__ __forceinline__ void topk_pick(uint32_t (&key)[VPL], uint32_t alive, int k, int& my_id, float& my_w) {
  const int lane = threadIdx.x & 63;
  my_id = -1;
  float my_z = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) m = ((alive >> v) & 1u) ? max(m, key[v]) : m;
    const uint32_t best = wave_max_u32(m);
    int e = -1;
#pragma unroll
    for (int v = VPL - 1; v >= 0; --v) {   // the lowest column holding `best` wins
      const uint64_t b = __ballot(((alive >> v) & 1u) && key[v] == best);
      if (b) e = v * 64 + (int)__builtin_ctzll(b);
    }
    if ((e & 63) == lane) alive &= ~(1u << (e >> 6));
    if (lane == j) {
      my_id = e;
      my_z = topk_key_value(best);
    }
  }
  my_w = topk_softmax(my_z, k);
}

// Top-k through a threshold, the same picks and weights as topk_pick.  tau is
// the smallest of the maxima of the ceil(E/16) groups of 16 experts (one DPP
// row of one key column); each group's maximum reaches tau, so at least that
// many keys do, and with at least k groups every pick is a key >= tau (a
// candidate).  The candidates are compacted into this wave's LDS scratch
// (key, expert) and each ranks itself against the others (higher key, or
// the same key and a lower index, is ahead: the order of topk_pick); ranks
// below k are the picks.  Fewer than k groups or more than 64 candidates
// (heavy ties) take the k-round selection.  scratch: 96 uint2 of this wave,
// 16-byte aligned.
template <int VPL>
__device__ __forceinline__ void topk_pick_fast(uint32_t (&key)[VPL], uint32_t alive, int E, int k, uint2* scratch,
                                               int& my_id, float& my_w) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane >> 4;
  uint32_t tl = 0xFFFFFFFFu;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    uint32_t m = ((alive >> v) & 1u) ? key[v] : 0u;
    m = max(m, dpp_u32<kDppXor1>(m));
    m = max(m, dpp_u32<kDppXor2>(m));
    m = max(m, dpp_u32<kDppHalfMirror>(m));
    m = max(m, dpp_u32<kDppMirror>(m));   // every lane of the row: the row's maximum
    if (v * 64 + r16 * 16 < E) tl = min(tl, m);
  }
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)tl, 0), t1 = (uint32_t)__builtin_amdgcn_readlane((int)tl, 16);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)tl, 32), t3 = (uint32_t)__builtin_amdgcn_readlane((int)tl, 48);
  const uint32_t tau = min(min(t0, t1), min(t2, t3));
  uint64_t b[VPL];
  int c = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    b[v] = __ballot(((alive >> v) & 1u) && key[v] >= tau);
    c += __popcll(b[v]);
  }
  if (c > 64 || (E + 15) / 16 < k) {   // uniform
    topk_pick<VPL>(key, alive, k, my_id, my_w);
    return;
  }
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int base = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    if ((b[v] >> lane) & 1ull) scratch[base + __popcll(b[v] & lt)] = make_uint2(key[v], (uint32_t)(v * 64 + lane));
    base += __popcll(b[v]);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's LDS writes are done
  const uint2 mine = lane < c ? scratch[lane] : make_uint2(0u, 0u);
  // eight candidates per round, read together; entries past c are masked
  // (the 64-entry buffer holds every read)
  int rank = 0;
  const auto ahead = [&](uint32_t kj, uint32_t ej, int j) {
    return ((kj > mine.x) | ((kj == mine.x) & (ej < mine.y))) & (j < c);
  };
  for (int j = 0; j < c; j += 8) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = *reinterpret_cast<const uint4*>(scratch + j + 2 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) rank += ahead(q[u].x, q[u].y, j + 2 * u) + ahead(q[u].z, q[u].w, j + 2 * u + 1);
  }
  uint2* pk = scratch + 64;
  if (lane < c && rank < k) pk[rank] = mine;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const uint2 p = lane < k ? pk[lane] : make_uint2(0u, 0u);
  my_id = lane < k ? (int)p.y : -1;
  my_w = topk_softmax(lane < k ? topk_key_value(p.x) : 0.f, k);
}

// a * sigmoid(a); the reciprocal is the hardware one (about 1 ulp), far
// below the BF16 rounding that h receives next.
__device__ __forceinline__ float silu_f32(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

}  // namespace moe
