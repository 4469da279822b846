// Quantizer: per-group scale and nearest code of each weight under its row's
// FP8 codebook (Hibana page, "Model surgery": 3-bit indices into a per-row
// 8-entry FP8 codebook, one 8-bit scale per 32 weights).  The page does not
// give the rule; the one taken here:
//   scale: the smallest s in 0..254 with max |w| over the group <= max |cb| *
//          2^(s-127) (254 if none fits, 0 for an all-zero group);
//   code:  the index of the nearest cb[j] * 2^(s-127), equal distances to the
//          lower index.
// Both decisions are exact.  Candidates a, b are FP8 values times a power of
// two, so a + b and 2w are exact in fp32, and |w - b| < |w - a| exactly when
// (a - b) and 2w - (a + b) have opposite signs (the sign of a rounded
// difference is the sign of the exact one).
//
// One thread per 32 bytes of weights (8 weights, two 16-byte loads); the 4
// threads of a group (consecutive lanes) share its largest magnitude by two
// lane swaps.  Reads 4 bytes and writes 1 + 1/32 bytes per weight; the exact
// nearest-code search (7 exact comparisons per weight) makes it ALU-bound.
#include "q3_internal.h"

namespace q3 {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int group_scale(float amax, float cbmax) {
  if (amax == 0.f) return 0;
  if (cbmax == 0.f) return 254;
  int ea, ec;
  frexpf(amax, &ea);
  frexpf(cbmax, &ec);
  // amax / cbmax lies in (2^(ea-ec-1), 2^(ea-ec+1)): the answer is 127+ea-ec or one more.
  int s = 127 + ea - ec - 1;
  s = s < 0 ? 0 : (s > 254 ? 254 : s);
  while (s < 254 && !(amax <= ldexpf(cbmax, s - 127))) ++s;
  return s;
}

__device__ __forceinline__ uint32_t nearest_code(float w, const float (&v)[8]) {
  const float ww = 2.f * w;
  uint32_t best = 0;
  float a = v[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    const float b = v[j];
    const float t = ww - (a + b);
    const bool closer = ((a > b) & (t < 0.f)) | ((a < b) & (t > 0.f));   // |w - b| < |w - a|, no branch
    best = closer ? (uint32_t)j : best;
    a = closer ? b : a;
  }
  return best;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t ldw,
                                                       const uint8_t* __restrict__ cb, int64_t n, int64_t k,
                                                       uint8_t* __restrict__ codes, int64_t ldc,
                                                       uint8_t* __restrict__ scales, int64_t lds) {
  // Chunk q (32 bytes) of rows blockIdx.y, blockIdx.y + gridDim.y, ...  Rows
  // hold a multiple of 4 chunks, so a group's 4 lanes leave together.
  const int64_t cpr = k / 8;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= cpr) return;
  for (int64_t r = blockIdx.y; r < n; r += gridDim.y) {
    const float4* src = reinterpret_cast<const float4*>(w + r * ldw + 8 * q);
    const float4 x0 = src[0], x1 = src[1];
    const uint2 cw = *reinterpret_cast<const uint2*>(cb + r * 8);
    // The fp8 conversions of gfx950 take OCP E4M3FN and are exact.
    const f32x2 p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.x, false);
    const f32x2 p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.x, true);
    const f32x2 p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.y, false);
    const f32x2 p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.y, true);
    float v[8] = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    float cbmax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) cbmax = fmaxf(cbmax, fabsf(v[j]));
    float amax = fmaxf(fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))),
                       fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w))));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int s = group_scale(amax, cbmax);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ldexpf(v[j], s - 127);   // exact: 4 significant bits, >= 2^-136
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= nearest_code(xs[i], v) << (8 * i);
      hi |= nearest_code(xs[4 + i], v) << (8 * i);
    }
    *reinterpret_cast<uint2*>(codes + r * ldc + 8 * q) = uint2{lo, hi};
    if ((q & 3) == 0) scales[r * lds + q / 4] = (uint8_t)s;
  }
}

}  // namespace

hipError_t launch_quantize(const float* w, int64_t ldw, const uint8_t* cb, int64_t n, int64_t k, uint8_t* codes,
                           int64_t ldc, uint8_t* scales, int64_t lds, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t gx = (k / 8 + 255) / 256;
  int64_t gy = 8192 / gx;
  gy = gy < 1 ? 1 : (gy > n ? n : (gy > 65535 ? 65535 : gy));
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, w, ldw, cb, n, k, codes,
                     ldc, scales, lds);
  return hipGetLastError();
}

}  // namespace q3
