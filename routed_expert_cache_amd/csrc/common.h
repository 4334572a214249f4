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

// Exact E4M3FN -> BF16 expansion of the four codes of one dword by integer
// bit operations ([OSDI] section 4.2 moves the E4M3 exponent into BF16 by the
// bias difference 120 and zero-fills the mantissa; that holds for normal
// codes).  Outputs: `ev` = BF16 pair (code0, code2), `od` = (code1, code3),
// low half first.  Codes with a zero exponent field (zero and subnormals) and
// the NaN codes S.1111.111 are not normal; they are patched by e4m3x4_fix.
__device__ __forceinline__ void e4m3x4_to_bf16_normal(uint32_t d, uint32_t& ev, uint32_t& od) {
  od = (d & 0x80008000u) | (((d >> 4) & 0x07F007F0u) + 0x3C003C00u);
  ev = ((d << 8) & 0x80008000u) | (((d << 4) & 0x07F007F0u) + 0x3C003C00u);
}

// Per-byte flag (bit 7 of each byte) of the codes that are not normal:
// exponent field 0, or magnitude 0x7F (NaN).  Zero iff all four are normal.
__device__ __forceinline__ uint32_t e4m3x4_special(uint32_t d) {
  uint32_t t1 = (d & 0x7F7F7F7Fu) + 0x01010101u;   // per byte: magnitude + 1 (<= 0x80)
  uint32_t t2 = (t1 & 0x7F7F7F7Fu) + 0x77777777u;  // bit 7 clear iff (mag+1) mod 128 <= 8
  return ~t2 & 0x80808080u;
}

// Exact BF16 of one E4M3FN code whose exponent field is 0 or which is NaN.
__device__ __forceinline__ uint32_t e4m3_special_bf16(uint32_t c) {
  uint32_t s = (c & 0x80u) << 8;
  uint32_t mag = c & 0x7Fu;
  if (mag == 0x7Fu) return s | 0x7FC0u;             // NaN
  uint32_t m = c & 7u;                                // exponent field is 0 here
  if (m == 0) return s;                               // signed zero
  uint32_t p = 31u - __builtin_clz(m);                // m * 2^-9 = 1.f * 2^(p-9)
  return s | ((118u + p) << 7) | ((m << (7u - p)) & 0x7Fu);
}

// Re-expand one dword exactly when any of its codes is special.
__device__ __forceinline__ void e4m3x4_fix(uint32_t d, uint32_t& ev, uint32_t& od) {
  uint32_t sp = e4m3x4_special(d);
  if (sp == 0) return;
  uint32_t c0 = d & 0xFFu, c1 = (d >> 8) & 0xFFu, c2 = (d >> 16) & 0xFFu, c3 = d >> 24;
  if (sp & 0x00000080u) ev = (ev & 0xFFFF0000u) | e4m3_special_bf16(c0);
  if (sp & 0x00800000u) ev = (ev & 0x0000FFFFu) | (e4m3_special_bf16(c2) << 16);
  if (sp & 0x00008000u) od = (od & 0xFFFF0000u) | e4m3_special_bf16(c1);
  if (sp & 0x80000000u) od = (od & 0x0000FFFFu) | (e4m3_special_bf16(c3) << 16);
}

// 16 codes (one 128-bit load) -> two MFMA operands of 8 BF16:
// `ev` holds codes 0,2,4,...,14 and `od` codes 1,3,...,15 (in that order).
// The exact patch runs only when some lane's codes are not all normal.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4& q, u32x4& ev, u32x4& od) {
  uint32_t e0, e1, e2, e3, o0, o1, o2, o3;
  const uint32_t d0 = q[0], d1 = q[1], d2 = q[2], d3 = q[3];
  e4m3x4_to_bf16_normal(d0, e0, o0);
  e4m3x4_to_bf16_normal(d1, e1, o1);
  e4m3x4_to_bf16_normal(d2, e2, o2);
  e4m3x4_to_bf16_normal(d3, e3, o3);
  const uint32_t sp = e4m3x4_special(d0) | e4m3x4_special(d1) | e4m3x4_special(d2) | e4m3x4_special(d3);
  if (__builtin_expect(__any(sp != 0), 0)) {
    if (sp) {
      e4m3x4_fix(d0, e0, o0);
      e4m3x4_fix(d1, e1, o1);
      e4m3x4_fix(d2, e2, o2);
      e4m3x4_fix(d3, e3, o3);
    }
  }
  ev = u32x4{e0, e1, e2, e3};
  od = u32x4{o0, o1, o2, o3};
}

// 16 codes (one 128-bit load) -> 16 BF16 in their natural order: `lo` holds
// codes 0..7 and `hi` codes 8..15.  gfx950 converts two OCP E4M3 codes to two
// BF16 per instruction; with the scale operand 1.0 the result is the code's
// exact value (every finite E4M3 value is a BF16 value), NaN codes give NaN.
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
