// Router of an MoE verify round over 3.25-bit experts.
//
// Hibana: Fast Agentic Inference on Unified-Memory Devices, "Adaptive
// speculation" / "Expert sharing": a verify round must read each expert chosen
// by at least one of its drafted tokens.  This kernel picks each token's top-k
// experts on the device; the expert-grouped product (q3_mfma.hip) then reads
// each picked expert once, without the list of picked experts ever coming back
// to the host.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

__device__ __forceinline__ bool ranks_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// One wave per token: every lane holds up to 16 logits; each round takes the
// wave-wide best (highest logit, then lowest index) among those not yet taken.
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ logits, int E, int topk,
                                                  int32_t* __restrict__ ids) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? logits[(int64_t)t * E + e] : 0.f;
  }
  uint32_t taken = 0u;
  for (int r = 0; r < topk; ++r) {
    float bv = -__builtin_inff();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !((taken >> q) & 1u) && ranks_before(v[q], e, bv, be)) {
        bv = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == 0) ids[(int64_t)t * topk + r] = be;
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
  }
}

}  // namespace

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)t), dim3(64), 0, s, logits, (int)e, (int)topk, ids);
  return hipGetLastError();
}

}  // namespace q3
