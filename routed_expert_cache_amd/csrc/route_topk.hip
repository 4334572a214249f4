// Top-k router: one wavefront per token.
//
// Each of the 64 lanes holds E/64 logits as 64-bit keys
//   (order-preserving bits of the float32 logit) << 32 | (0xFFFFFFFF - expert),
// so the wave-wide maximum key is the largest logit with ties going to the
// lower expert index.  k rounds of (lane max, 6-step butterfly max) pick the
// experts in rank order; the winner's lane retires it.  Lane j keeps pick j,
// and the gate weights are the softmax over the kept logits ([FTK] routing
// and GPU-router paragraphs).
#include "common.h"

namespace moe {

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    int e = v * 64 + lane;
    key[v] = 0;
    if (e < E) {
      float f = row[e];
      uint32_t u = __float_as_uint(f);
      if ((u & 0x7fffffffu) == 0) u = 0;                       // -0 ranks as +0
      uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[v] = ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
    }
  }

  int my_id = -1;
  float my_z = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) best = key[v] > best ? key[v] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const uint32_t ord = (uint32_t)(best >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (v * 64 + lane == e) key[v] = 0;
    if (lane == j) {
      my_id = e;
      my_z = __uint_as_float(u);
    }
  }
  // softmax over the k kept logits; pick 0 holds the maximum
  const float zmax = __shfl(my_z, 0, 64);
  float ex = (lane < k) ? expf(my_z - zmax) : 0.f;
  float s = ex;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = ex / s;
  }
}

}  // namespace moe

extern "C" moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                                     int32_t* ids, float* w, hipStream_t stream) {
  using namespace moe;
  clear_error();
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    MOE_FAIL(MOE_ERR_SHAPE, "moe_route_topk: need T>=0, 1<=E<=1024, 1<=k<=min(E,32) (T=%d E=%d k=%d)",
             T, E, k);
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !w) MOE_FAIL(MOE_ERR_ARG, "moe_route_topk: null pointer");
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  else
    route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w);
  MOE_LAUNCHED();
  return MOE_OK;
}
