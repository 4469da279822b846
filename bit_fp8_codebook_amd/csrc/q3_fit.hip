// Per-row codebook fitting: the 8 E4M3FN entries of each row's codebook from
// the row's fp32 weights (the step before the quantizer and packing).
//
// Hibana: Fast Agentic Inference on Unified-Memory Devices, "Model surgery" /
// "Three-bit weights": every weight is a 3-bit index into an 8-entry FP8
// codebook, which the page's illustration fits to the weights it serves.  The
// page gives no procedure; the one computed here (one codebook per output row,
// every decision exact, so the result is bit-identical to exact arithmetic):
//   1. per group of 32: e = the smallest integer with max|w| <= 2^e (0 for an
//      all-zero group);
//   2. q = round(w * 2^(12 - e)), ties to even: integers in [-4096, 4096];
//   3. 1-D k-means (Lloyd) with 8 centroids on the row's q: start at the values
//      of ranks floor((2i+1)K/16) of the sorted q; each q joins its nearest
//      centroid (equal distances: the lower index); each centroid with points
//      becomes their exact mean (a rational sum/count), one without keeps its
//      value; the centroids are re-sorted by value (stable); stop when no
//      centroid changes, or after 64 updates;
//   4. entry i = centroid i / 2^12 rounded to the nearest E4M3FN value (equal
//      distances: even significand), sign of the centroid (-0 for a negative
//      centroid that rounds to zero).
//
// One block per row.  The row's q go into a histogram of the 8193 grid values
// in LDS (integer atomics: exact counts), two block scans turn it into prefix
// counts and prefix sums, and since 1-D clusters are contiguous ranges of q
// between the midpoints of neighbouring distinct centroids, each update is a
// few exact integer operations on the prefix arrays (one lane), however long
// the row.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kGridBits = 12;
constexpr int kHalf = 1 << kGridBits;           // q in [-kHalf, kHalf]
constexpr int kBins = 2 * kHalf + 1;
constexpr int kFitThreads = 256;
constexpr int kChunk = (kBins + kFitThreads - 1) / kFitThreads;   // bins per thread in the scans
constexpr int kMaxUpdates = 64;

// floor(num / den) for den > 0, exact: a double estimate corrected by the
// exact integer comparisons (|num|, den < 2^53).
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den) {
  int64_t q = (int64_t)floor((double)num / (double)den);
  while ((q + 1) * den <= num) ++q;
  while (q * den > num) --q;
  return q;
}

// E4M3FN magnitude of byte b (0..0x7E) in units of 2^-9.
__device__ __forceinline__ int64_t e4m3_units(int b) {
  const int e = b >> 3, m = b & 7;
  return e == 0 ? m : (int64_t)(8 + m) << (e - 1);
}

// The E4M3FN byte nearest to s / (c * 2^12), equal distances to the even
// significand.  In units of 2^-9 the value is |s| / (8c); |value| <= 1.
__device__ uint8_t round_e4m3fn(int64_t s, int64_t c) {
  const int64_t a = s < 0 ? -s : s;
  const int64_t c8 = 8 * c;
  int lo = 0, hi = 0x7E;                        // largest byte with units*8c <= |s|
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (e4m3_units(mid) * c8 <= a) lo = mid;
    else hi = mid - 1;
  }
  int b = lo;
  if (b < 0x7E) {
    const int64_t twice = 2 * a, mid2 = (e4m3_units(b) + e4m3_units(b + 1)) * c8;
    if (twice > mid2 || (twice == mid2 && (b & 1))) b += 1;
  }
  return (uint8_t)(b | (s < 0 ? 0x80 : 0));
}

// Exclusive block scan of one int per thread (kFitThreads threads); returns
// this thread's prefix, *total gets the sum.  Uses `tmp` (kFitThreads ints).
__device__ int block_scan(int v, int* tmp, int* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int d = 1; d < kFitThreads; d <<= 1) {
    const int add = t >= d ? tmp[t - d] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int incl = tmp[t];
  *total = tmp[kFitThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kFitThreads) void fit_kernel(const float* __restrict__ w, int64_t ldw, int64_t k,
                                                          uint8_t* __restrict__ cb) {
  extern __shared__ __align__(16) int smem[];
  int* cnt = smem;                       // kBins + 1: counts, then prefix counts
  int* psum = smem + (kBins + 1);        // kBins + 1: prefix sums of q
  __shared__ int tmp[kFitThreads];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* wr = w + row * ldw;
  const int groups = (int)(k / 32);

  for (int b = t; b < kBins + 1; b += kFitThreads) cnt[b] = 0;
  __syncthreads();

  // 1-2: exponent of each group, grid values, histogram.
  for (int g = t; g < groups; g += kFitThreads) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4*>(wr + 32 * g + 4 * i);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    int e = 0;
    if (amax > 0.f) {
      int x;
      const float f = frexpf(amax, &x);        // amax = f * 2^x, f in [0.5, 1)
      e = f == 0.5f ? x - 1 : x;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // exact scaling by a power of two (|result| <= 4096; results below
        // 2^-126 round to zero either way), then round half to even
        const int q = (int)rintf(ldexpf(v[i][j], kGridBits - e));
        atomicAdd(&cnt[q + kHalf], 1);
      }
  }
  __syncthreads();

  // Prefix arrays: cnt[b] = #q < b - kHalf, psum[b] = sum of those q.
  {
    // each thread owns bins [b0, b0 + kChunk): it reads its counts, and reads
    // each again just before overwriting it with the prefix
    const int b0 = t * kChunk;
    int lc = 0, ls = 0;
    for (int i = 0; i < kChunk; ++i) {
      const int b = b0 + i;
      const int c = b < kBins ? cnt[b] : 0;
      lc += c;
      ls += c * (b - kHalf);
    }
    int tc, ts;
    const int pc = block_scan(lc, tmp, &tc);
    const int ps = block_scan(ls, tmp, &ts);
    int rc = pc, rs = ps;
    for (int i = 0; i < kChunk; ++i) {
      const int b = b0 + i;
      if (b < kBins) {
        const int c = cnt[b];
        cnt[b] = rc;
        psum[b] = rs;
        rc += c;
        rs += c * (b - kHalf);
      }
    }
    if (t == 0) {
      cnt[kBins] = tc;
      psum[kBins] = ts;
    }
  }
  __syncthreads();
  if (t != 0) return;

  // 3: Lloyd on the prefix arrays (one lane).  The centroids are held as
  // separate sum and count arrays indexed only by compile-time constants (fully
  // unrolled loops, selects), so they stay in registers.
  const int64_t K = cnt[kBins];
  int64_t cs[8], cc[8];                          // centroid a is cs[a] / cc[a]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // value of rank r (0-based) of the sorted q: the smallest b with
    // #q <= b - kHalf greater than r, by a fixed-length binary search
    const int64_t r = (2 * i + 1) * K / 16;
    int lo = 0, hi = kBins - 1;
#pragma unroll
    for (int step = 0; step < 14; ++step) {     // 2^14 > kBins
      const int mid = (lo + hi) >> 1;            // mid + 1 <= kBins: in bounds
      const bool open = lo < hi, up = cnt[mid + 1] <= r;
      lo = open && up ? mid + 1 : lo;
      hi = open && !up ? mid : hi;
    }
    cs[i] = lo - kHalf;
    cc[i] = 1;
  }
  for (int it = 0; it < kMaxUpdates; ++it) {
    // Runs of equal centroids: the first index of a run takes the q between
    // the midpoints to the neighbouring distinct values (a q on a midpoint
    // goes to the lower run); the others get none and keep their value.
    int64_t ns[8], nc[8];
    int lo_q = -kHalf - 1;                       // q of the current run lie above this
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      ns[a] = cs[a];
      nc[a] = cc[a];
      bool start = true;
      if (a > 0) start = cs[a] * cc[a - 1] != cs[a - 1] * cc[a];
      bool have = false;                         // the next distinct value after this run
      int64_t bs = cs[a], bc = cc[a];
#pragma unroll
      for (int b = 7; b > a; --b) {
        const bool d = cs[b] * cc[a] != cs[a] * cc[b];
        have = have || d;
        bs = d ? cs[b] : bs;                     // ends on the smallest such b
        bc = d ? cc[b] : bc;
      }
      if (start) {
        int hi_q = kHalf;
        if (have) {
          const int64_t m = floor_div(cs[a] * bc + bs * cc[a], 2 * cc[a] * bc);
          hi_q = (int)(m < -kHalf - 1 ? -kHalf - 1 : (m > kHalf ? kHalf : m));
        }
        hi_q = hi_q < lo_q ? lo_q : hi_q;
        const int64_t n_in = cnt[hi_q + kHalf + 1] - cnt[lo_q + kHalf + 1];
        const int64_t s_in = (int64_t)psum[hi_q + kHalf + 1] - psum[lo_q + kHalf + 1];
        ns[a] = n_in > 0 ? s_in : ns[a];
        nc[a] = n_in > 0 ? n_in : nc[a];
        lo_q = hi_q;
      }
    }
    // Sort by value with adjacent compare-exchanges (stable: equal values never swap).
#pragma unroll
    for (int pass = 0; pass < 7; ++pass)
#pragma unroll
      for (int a = 0; a < 7 - pass; ++a) {
        const bool sw = ns[a + 1] * nc[a] < ns[a] * nc[a + 1];
        const int64_t xs = ns[a], xc = nc[a], ys = ns[a + 1], yc = nc[a + 1];
        ns[a] = sw ? ys : xs;
        nc[a] = sw ? yc : xc;
        ns[a + 1] = sw ? xs : ys;
        nc[a + 1] = sw ? xc : yc;
      }
    bool same = true;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      same = same && ns[a] * cc[a] == cs[a] * nc[a];
      cs[a] = ns[a];
      cc[a] = nc[a];
    }
    if (same) break;
  }

  // 4: round to E4M3FN.
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int a = 0; a < 4; ++a) lo |= (uint32_t)round_e4m3fn(cs[a], cc[a]) << (8 * a);
#pragma unroll
  for (int a = 0; a < 4; ++a) hi |= (uint32_t)round_e4m3fn(cs[a + 4], cc[a + 4]) << (8 * a);
  *reinterpret_cast<u32x2*>(cb + row * 8) = u32x2{lo, hi};
}

}  // namespace

hipError_t launch_fit_codebook(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* cb, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t shm = 2 * (kBins + 1) * sizeof(int);
  static bool allowed = false;   // one attribute call; idempotent if it races
  if (!allowed) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fit_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    allowed = true;
  }
  hipLaunchKernelGGL(fit_kernel, dim3((unsigned)n), dim3(kFitThreads), shm, s, w, ldw, k, cb);
  return hipGetLastError();
}

}  // namespace q3
