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

// One block per token, one thread per expert: the token's logits go to LDS and
// every thread counts the experts that rank before its own (higher logit, or
// an equal logit at a lower index).  That count is the expert's rank, unique
// per expert, so the threads with rank < topk write ids[rank] directly: no
// sorting and no cross-thread reduction.
__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ logits, int E, int topk,
                                                    int32_t* __restrict__ ids) {
  __shared__ float v[1024];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  const float mine = e < E ? logits[(int64_t)t * E + e] : 0.f;
  if (e < E) v[e] = mine;
  __syncthreads();
  if (e >= E) return;
  int rank = 0;
  for (int o = 0; o < E; ++o) rank += ranks_before(v[o], o, mine, e) ? 1 : 0;
  if (rank < topk) ids[(int64_t)t * topk + rank] = e;
}

}  // namespace

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids, hipStream_t s) {
  const unsigned threads = (unsigned)((e + 63) / 64 * 64);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)t), dim3(threads), 0, s, logits, (int)e, (int)topk, ids);
  return hipGetLastError();
}

}  // namespace q3
