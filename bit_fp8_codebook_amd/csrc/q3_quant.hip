// Quantizer: per-group scale and nearest code of each weight under its row's
// FP8 codebook (Hibana page, "Model surgery": 3-bit indices into a per-row
// 8-entry FP8 codebook, one 8-bit scale per 32 weights).  The page does not
// give the rule; the one taken here:
//   scale: the smallest s in 0..254 with max |w| over the group <= max |cb| *
//          2^(s-127) (254 if none fits, 0 for an all-zero group);
//   code:  the index of the nearest cb[j] * 2^(s-127), equal distances to the
//          lower index.
// Both decisions are exact: candidates are FP8 values times a power of two, so
// sums of two of them and 2w are exact in fp32.
//
// The nearest code by a search over sorted midpoints.  Once per row the block
// sorts the 8 codebook values (equal values by index) and keeps, per sorted
// position p, the lowest index holding that value (lo[p]) and the exact sums
// m[p] = u[p] + u[p+1] of neighbouring sorted values.  Scaled by 2^(s-127)
// (exact), w is nearer u[p+1] than u[p] exactly when 2w > m[p]; at 2w == m[p]
// the two are equidistant and the lower of lo[p], lo[p+1] wins, so where the
// upper one wins the threshold is lowered to the next float below m[p]
// (2w >= m  <=>  2w > pred(m) for floats).  The count of thresholds below 2w
// is the sorted position of the nearest value, and lo[] of it its code: the
// lowest index among the nearest entries, the same result as comparing all 8
// candidates in index order.  Equal neighbours share a code, so their
// threshold does not matter.
//
// One thread per 32 bytes of weights (8 weights, two 16-byte loads); the 4
// threads of a group (consecutive lanes) share its largest magnitude by two
// lane swaps.  Reads 4 bytes and writes 1 + 1/32 bytes per weight.
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

__device__ __forceinline__ float below(float t) {   // the largest float < t (t finite)
  const uint32_t u = __builtin_bit_cast(uint32_t, t);
  if ((u & 0x7FFFFFFFu) == 0u) return __builtin_bit_cast(float, 0x80000001u);   // +-0 -> -2^-149
  return __builtin_bit_cast(float, (u & 0x80000000u) ? u + 1u : u - 1u);
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t ldw,
                                                       const uint8_t* __restrict__ cb, int64_t n, int64_t k,
                                                       uint8_t* __restrict__ codes, int64_t ldc,
                                                       uint8_t* __restrict__ scales, int64_t lds) {
  __shared__ float su[8];      // sorted codebook values
  __shared__ int slo[8];       // lowest index holding each sorted value
  __shared__ float sm[8];      // sums of sorted neighbours (7 used)
  __shared__ uint32_t supper;  // bit p: at an exact tie the upper neighbour wins
  __shared__ uint32_t stab;    // 3-bit code of each sorted position
  // Chunk q (32 bytes) of rows blockIdx.y, blockIdx.y + gridDim.y, ...  Rows
  // hold a multiple of 4 chunks, so a group's 4 lanes are all in or all out.
  const int tid = threadIdx.x;
  const int64_t cpr = k / 8;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + tid;
  const bool active = q < cpr;
  for (int64_t r = blockIdx.y; r < n; r += gridDim.y) {
    // The weights do not depend on the row's table: their loads go out first.
    float4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
    if (active) {
      const float4* src = reinterpret_cast<const float4*>(w + r * ldw + 8 * q);
      x0 = src[0];
      x1 = src[1];
    }
    if (tid < 8) {
      const uint2 cw = *reinterpret_cast<const uint2*>(cb + r * 8);
      // The fp8 conversions of gfx950 take OCP E4M3FN and are exact.
      const f32x2 p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.x, false);
      const f32x2 p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.x, true);
      const f32x2 p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.y, false);
      const f32x2 p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw.y, true);
      const float v[8] = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
      float mine = v[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mine = tid == j ? v[j] : mine;
      int rank = 0, lo = 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rank += (v[j] < mine || (v[j] == mine && j < tid)) ? 1 : 0;
        lo = (v[j] == mine && j < lo) ? j : lo;
      }
      su[rank] = mine;
      slo[rank] = lo;
    }
    __syncthreads();
    if (tid < 8) {
      const int lo_p = slo[tid];
      bool upper = false;
      if (tid < 7) {
        sm[tid] = su[tid] + su[tid + 1];   // exact: two E4M3 values
        upper = slo[tid + 1] < lo_p;
      }
      const unsigned long long up = __ballot(upper);
      uint32_t tab = (uint32_t)lo_p << (3 * tid);
      tab |= __shfl_xor(tab, 1, 64);
      tab |= __shfl_xor(tab, 2, 64);
      tab |= __shfl_xor(tab, 4, 64);
      if (tid == 0) {
        supper = (uint32_t)up;
        stab = tab;
      }
    }
    __syncthreads();
    if (active) {
      const float cbmax = fmaxf(fabsf(su[0]), fabsf(su[7]));
      float amax = fmaxf(fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))),
                         fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w))));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int s = group_scale(amax, cbmax);
      const uint32_t upper = supper, tab = stab;
      float t[7];
#pragma unroll
      for (int p = 0; p < 7; ++p) {
        // Exact: sm[p] (the sum of two E4M3 values) has at most 18 significant
        // bits, none below 2^-9, so the scaled midpoint keeps every bit: its
        // lowest stays at or above 2^-136 (fp32 subnormals reach 2^-149) and,
        // with |w| <= 2^64 bounding s, its magnitude below 2^84.
        const float m = ldexpf(sm[p], s - 127);
        t[p] = (upper >> p) & 1u ? below(m) : m;
      }
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ww = 2.f * xs[i];
        uint32_t pos = 0;
#pragma unroll
        for (int p = 0; p < 7; ++p) pos += ww > t[p] ? 1u : 0u;
        const uint32_t c = (tab >> (3u * pos)) & 7u;
        if (i < 4) lo |= c << (8 * i);
        else hi |= c << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(codes + r * ldc + 8 * q) = uint2{lo, hi};
      if ((q & 3) == 0) scales[r * lds + q / 4] = (uint8_t)s;
    }
    __syncthreads();   // the next row's table reuses the shared arrays
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
