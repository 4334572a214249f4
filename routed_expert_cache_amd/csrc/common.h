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

// a * sigmoid(a); the reciprocal is the hardware one (about 1 ulp), far
// below the BF16 rounding that h receives next.
__device__ __forceinline__ float silu_f32(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

}  // namespace moe
