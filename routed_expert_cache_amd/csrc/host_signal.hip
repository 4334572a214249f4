// Hand-over between a GPU stream and the host executor through words of
// pinned host memory, for the host branch of a decode step ([FT] section
// "q* 策略": the host computes the misses it keeps while the GPU fills and
// evaluates G; the two partial sums are then added).
//
// The stream writes a sequence number into `ready` once the step's inputs
// are in pinned memory (moe_host_signal); the executor's dispatcher thread,
// which waits for that number, evaluates the host set and then stores the
// number into `done` (moe_host_forward_signal); the merge waits for `done`
// before it adds y_host (moe_merge_partial_after).  Both waits are bounded:
// a GPU wait that times out sets an error word and merges whatever y_host
// holds; no stream ever waits on a host callback.
#include "common.h"

namespace moe {

constexpr uint32_t kHostPollLimit = 1u << 21;   // polls of `done`, about a microsecond apart

__global__ void signal_write_kernel(uint32_t* word, uint32_t seq) {
  __hip_atomic_store(word, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Thread 0 of each workgroup waits until done - seq >= 0 (serial numbers
// compared modulo 2^32), then every thread reads y_host at system scope.
__global__ __launch_bounds__(256) void merge_after_kernel(const float* __restrict__ yg, const float* yh, size_t n4,
                                                          size_t n, float* yo, uint16_t* yb, const uint32_t* done,
                                                          uint32_t seq, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t it = 0;
    while ((int32_t)(__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) - seq) < 0) {
      if (++it >= kHostPollLimit) {
        if (err) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
      __builtin_amdgcn_s_sleep(32);
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");   // system scope: y_host as the host wrote it
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    const f32x4 h = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yh + 4 * i));
    const f32x4 v = *reinterpret_cast<const f32x4*>(yg + 4 * i) + h;
    *reinterpret_cast<f32x4*>(yo + 4 * i) = v;
    if (yb) {
      const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<u32x2*>(yb + 4 * i) = u32x2{lo, hi};
    }
  }
  if (i == 0) {
    for (size_t t = 4 * n4; t < n; ++t) {
      const float v = yg[t] + yh[t];
      yo[t] = v;
      if (yb) yb[t] = f32_to_bf16_rne(v);
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_host_signal(uint32_t* word, uint32_t seq, hipStream_t stream) {
  clear_error();
  if (!word) MOE_FAIL(MOE_ERR_ARG, "word is NULL");
  signal_write_kernel<<<1, 1, 0, stream>>>(word, seq);
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_merge_partial_after(const float* y_gpu, const float* y_host, const uint32_t* done,
                                              uint32_t seq, int32_t T, int32_t H, float* y_out, uint16_t* y_out_bf16,
                                              uint32_t* err, hipStream_t stream) {
  clear_error();
  if (T < 0 || H < 1) MOE_FAIL(MOE_ERR_SHAPE, "bad T=%d H=%d", T, H);
  if (T == 0) return MOE_OK;
  if (!y_gpu || !y_host || !done || !y_out) MOE_FAIL(MOE_ERR_ARG, "null argument");
  if (!aligned16(y_gpu) || !aligned16(y_host) || !aligned16(y_out) || (y_out_bf16 && ((uintptr_t)y_out_bf16 & 7)))
    MOE_FAIL(MOE_ERR_ARG, "y_gpu, y_host, y_out must be 16-byte and y_out_bf16 8-byte aligned");
  const size_t n = (size_t)T * H, n4 = n / 4;
  const size_t blocks = (n4 + 255) / 256 > 0 ? (n4 + 255) / 256 : 1;
  merge_after_kernel<<<(unsigned)blocks, 256, 0, stream>>>(y_gpu, y_host, n4, n, y_out, y_out_bf16, done, seq, err);
  MOE_LAUNCHED();
  return MOE_OK;
}
