// MoE verify round over 3.25-bit experts.
//
// Hibana: Fast Agentic Inference on Unified-Memory Devices, "Adaptive
// speculation" / "Expert sharing": verifying a round of drafted tokens reads
// every expert any of them picked.  The router kernel picks each token's top-k
// experts; the grouped kernel then reads each picked expert's packed weights
// exactly once and applies them to all (token, slot) pairs routed to it.  The
// grid covers every expert, and blocks of experts nobody picked return before
// touching weight memory, so no list of picked experts has to come back to the
// host.
#include "q3_gemv_body.h"

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

template <int M, bool kCached>
__device__ __forceinline__ void grouped_run(const PlaneView& pv, const int* pairs, int base,
                                            const uint16_t* x, int64_t ldx, int x_by_slot, int topk, float* y,
                                            int64_t ldy, int lg_tpr, int64_t row0) {
  TokenRows<M> tok;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int q = pairs[base + m];                 // q = token * topk + slot
    tok.x[m] = x + (int64_t)(x_by_slot ? q : q / topk) * ldx;
    tok.y[m] = y + (int64_t)q * ldy;
  }
  gemv_block<M, kCached>(pv, tok, lg_tpr, row0);
}

template <bool kCached>
__global__ __launch_bounds__(kGemvThreads) void grouped_kernel(ExpertView w, const uint16_t* __restrict__ x,
                                                               int64_t ldx, int x_by_slot,
                                                               const int32_t* __restrict__ ids, int pairs_total,
                                                               int topk, float* __restrict__ y, int64_t ldy,
                                                               int lg_tpr) {
  __shared__ int pairs[64];
  __shared__ int count;
  const int e = blockIdx.y;
  if (threadIdx.x < 64) {
    const int q = threadIdx.x;
    const bool match = q < pairs_total && ids[q] == e;
    const unsigned long long mask = __ballot(match);
    if (match) pairs[__popcll(mask & ((1ull << q) - 1ull))] = q;
    if (q == 0) count = __popcll(mask);
  }
  __syncthreads();
  const int c = count;
  if (c == 0) return;   // expert not picked this round: its weights are never read

  PlaneView pv = w.base;
  pv.code += (int64_t)e * w.code_stride;
  pv.scale += (int64_t)e * w.scale_stride;
  pv.cb += (int64_t)e * w.cb_stride;
  const int64_t row0 = (int64_t)blockIdx.x * (kGemvThreads >> lg_tpr) * kGemvPasses;
  for (int base = 0; base < c; base += 8) {
    switch (c - base < 8 ? c - base : 8) {
      case 1: grouped_run<1, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 2: grouped_run<2, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 3: grouped_run<3, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 4: grouped_run<4, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 5: grouped_run<5, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 6: grouped_run<6, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      case 7: grouped_run<7, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
      default: grouped_run<8, kCached>(pv, pairs, base, x, ldx, x_by_slot, topk, y, ldy, lg_tpr, row0); break;
    }
    __syncthreads();   // the reduction scratch is reused by the next slice
  }
}

}  // namespace

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)t), dim3(64), 0, s, logits, (int)e, (int)topk, ids);
  return hipGetLastError();
}

hipError_t launch_grouped(const ExpertView& w, const uint16_t* x, int64_t ldx, int32_t x_by_slot,
                          const int32_t* ids, int32_t t, int32_t topk, float* y, int64_t ldy, hipStream_t s) {
  if (w.base.n == 0) return hipSuccess;
  const int lg = gemv_lg_tpr(w.base.groups);
  const int64_t rows_per_block = (int64_t)(kGemvThreads >> lg) * kGemvPasses;
  const dim3 grid((unsigned)((w.base.n + rows_per_block - 1) / rows_per_block), (unsigned)w.num_experts);
  if (w.base.groups <= kGemvThreads)
    hipLaunchKernelGGL((grouped_kernel<true>), grid, dim3(kGemvThreads), 0, s, w, x, ldx, (int)x_by_slot, ids,
                       (int)(t * topk), (int)topk, y, ldy, lg);
  else
    hipLaunchKernelGGL((grouped_kernel<false>), grid, dim3(kGemvThreads), 0, s, w, x, ldx, (int)x_by_slot, ids,
                       (int)(t * topk), (int)topk, y, ldy, lg);
  return hipGetLastError();
}

}  // namespace q3
