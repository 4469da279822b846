// VALU decode GEMV for 1..8 tokens over the 3.25-bit codebook format (the
// kernel body and its design notes are in q3_gemv_body.h).
#include "q3_gemv_body.h"

namespace q3 {

template <int M, bool kCached>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(PlaneView w, const uint16_t* __restrict__ x,
                                                            int64_t ldx, float* __restrict__ y, int64_t ldy,
                                                            int lg_tpr) {
  TokenRows<M> tok;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    tok.x[m] = x + m * ldx;
    tok.y[m] = y + m * ldy;
  }
  const int RS = kGemvThreads >> lg_tpr;
  gemv_block<M, kCached>(w, tok, lg_tpr, (int64_t)blockIdx.x * RS * kGemvPasses);
}

namespace {

template <int M>
hipError_t launch_gemv_m(const PlaneView& w, const uint16_t* x, int64_t ldx, float* y, int64_t ldy,
                         hipStream_t s) {
  const int lg = gemv_lg_tpr(w.groups);
  const int64_t rows_per_block = (int64_t)(kGemvThreads >> lg) * kGemvPasses;
  const dim3 grid((unsigned)((w.n + rows_per_block - 1) / rows_per_block));
  if (w.groups <= kGemvThreads)
    hipLaunchKernelGGL((gemv_kernel<M, true>), grid, dim3(kGemvThreads), 0, s, w, x, ldx, y, ldy, lg);
  else
    hipLaunchKernelGGL((gemv_kernel<M, false>), grid, dim3(kGemvThreads), 0, s, w, x, ldx, y, ldy, lg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t s) {
  if (w.n == 0) return hipSuccess;
  switch (m) {
    case 1: return launch_gemv_m<1>(w, x, ldx, y, ldy, s);
    case 2: return launch_gemv_m<2>(w, x, ldx, y, ldy, s);
    case 3: return launch_gemv_m<3>(w, x, ldx, y, ldy, s);
    case 4: return launch_gemv_m<4>(w, x, ldx, y, ldy, s);
    case 5: return launch_gemv_m<5>(w, x, ldx, y, ldy, s);
    case 6: return launch_gemv_m<6>(w, x, ldx, y, ldy, s);
    case 7: return launch_gemv_m<7>(w, x, ldx, y, ldy, s);
    case 8: return launch_gemv_m<8>(w, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q3
