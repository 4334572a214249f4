// Top-k router: one wavefront per token (the selection itself is
// topk_keys / topk_pick_fast in common.h, shared with the fused router +
// cache step).  [FTK] routing and GPU-router paragraphs.
#include "common.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  __shared__ __align__(16) uint2 scratch[4][96];
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));   // one token per wave
  if (t >= T) return;
  uint32_t key[VPL], alive;
  topk_keys<VPL>(make_rsrc(logits + (size_t)t * E, 4u * (uint32_t)E), E, key, alive);
  int my_id;
  float my_w;
  topk_pick_fast<VPL>(key, alive, E, k, scratch[threadIdx.x >> 6], my_id, my_w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = my_w;
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
