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
// few exact operations on the prefix arrays, however long the row: eight lanes,
// one per centroid, with exact rationals in fp64.
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

// floor of the midpoint (as/ac + bs/bc) / 2 of two centroids, exact: every
// operand is an integer below 2^53 in magnitude (products < 2^49), so the
// double estimate is corrected by exact comparisons.
__device__ __forceinline__ int64_t floor_mid(double as, double ac, double bs, double bc) {
  const double num = as * bc + bs * ac, den = 2.0 * ac * bc;
  double q = floor(num / den);
  while ((q + 1.0) * den <= num) q += 1.0;
  while (q * den > num) q -= 1.0;
  return (int64_t)q;
}

__device__ __forceinline__ int clamp_q(int64_t m) {
  return (int)(m < -kHalf - 1 ? -kHalf - 1 : (m > kHalf ? kHalf : m));
}

// Lane l's value in every lane (two readlanes: lane l of the wave's first group,
// which holds what every group holds).
__device__ __forceinline__ double from_lane(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The next lower lane's value (DPP row_shr:1 on both halves; the first lane of
// each 16-lane row reads 0, the first lane of the second group of a row reads
// the last lane of the first: lane a = 0 of a group never uses the result).
__device__ __forceinline__ double from_lower_lane(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x111, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x111, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The value of this lane lands in lane `dst` (ds_permute: each lane pushes).
__device__ __forceinline__ double permute_to(int dst, double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
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

// kNarrow (rows shorter than 65536): the prefix counts fit 16 bits, so the
// histogram is counted in the prefix-sum array and the prefix counts take half
// the space (49 KB of LDS instead of 65 KB: three blocks per CU instead of two).
template <bool kNarrow>
__global__ __launch_bounds__(kFitThreads) void fit_kernel(const float* __restrict__ w, int64_t ldw, int64_t k,
                                                          uint8_t* __restrict__ cb) {
  extern __shared__ __align__(16) int smem[];
  int* psum = smem;                                                 // kBins + 1: prefix sums of q
  int* cnt32 = smem + (kBins + 1);                                  // kBins + 1 (wide rows)
  uint16_t* cnt16 = reinterpret_cast<uint16_t*>(smem + (kBins + 1));   // kBins + 1 (narrow rows)
  int* hist = kNarrow ? psum : cnt32;                               // counts before the scan
  auto cnt = [&](int b) -> int { return kNarrow ? (int)cnt16[b] : cnt32[b]; };   // #q < b - kHalf
  __shared__ int tmp[kFitThreads];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* wr = w + row * ldw;
  const int groups = (int)(k / 32);

  for (int b = t; b < kBins + 1; b += kFitThreads) hist[b] = 0;
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
        atomicAdd(&hist[q + kHalf], 1);
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
      const int c = b < kBins ? hist[b] : 0;
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
        const int c = hist[b];          // this thread's own bin: read before it is overwritten
        if constexpr (kNarrow) cnt16[b] = (uint16_t)rc;
        else cnt32[b] = rc;
        psum[b] = rs;
        rc += c;
        rs += c * (b - kHalf);
      }
    }
    if (t == 0) {
      if constexpr (kNarrow) cnt16[kBins] = (uint16_t)tc;
      else cnt32[kBins] = tc;
      psum[kBins] = ts;
    }
  }
  __syncthreads();
  if (t >= 64) return;

  // 3: Lloyd on the prefix arrays, one centroid per lane: lane a of every
  // group of eight lanes holds centroid a as an exact rational s/c (|s| <= 2^30,
  // 1 <= c <= 2^18) in two doubles, so every cross product (< 2^49) and every
  // sum of two of them is exact in fp64 and compares exactly.  The eight
  // groups of the wave compute the same thing; group 0's lanes are read.
  const int a = t & 7;
  const int g0 = t & ~7;                         // first lane of this group
  const int64_t K = cnt(kBins);
  double cs, cc;
  {
    // value of rank r (0-based) of the sorted q: the smallest b with
    // #q <= b - kHalf greater than r, by a fixed-length binary search
    const int64_t r = (2 * a + 1) * K / 16;
    int lo = 0, hi = kBins - 1;
#pragma unroll
    for (int step = 0; step < 14; ++step) {     // 2^14 > kBins
      const int mid = (lo + hi) >> 1;            // mid + 1 <= kBins: in bounds
      const bool open = lo < hi, up = cnt(mid + 1) <= r;
      lo = open && up ? mid + 1 : lo;
      hi = open && !up ? mid : hi;
    }
    cs = (double)(lo - kHalf);
    cc = 1.0;
  }
  for (int it = 0; it < kMaxUpdates; ++it) {
    // Runs of equal centroids (the centroids are sorted): the first lane of a
    // run takes the q between the midpoints to the neighbouring distinct values
    // (a q on a midpoint goes to the lower run); the others get none and keep
    // their value.
    const double ps = from_lower_lane(cs);
    const double pc = from_lower_lane(cc);
    const bool start = a == 0 || ps * cc != cs * pc;
    const uint32_t starts = (uint32_t)__ballot(start) & 0xFFu;    // group 0's lanes
    const uint32_t above = starts >> (a + 1);
    const int nb = above ? a + 1 + __builtin_ctz(above) : a;     // next run's first lane
    const double ns = __shfl(cs, g0 + nb, 64);
    const double nc = __shfl(cc, g0 + nb, 64);
    int hi_q = kHalf, lo_q = -kHalf - 1;
    if (above) hi_q = clamp_q(floor_mid(cs, cc, ns, nc));
    if (a > 0) lo_q = clamp_q(floor_mid(ps, pc, cs, cc));
    hi_q = hi_q < lo_q ? lo_q : hi_q;
    const int n_in = cnt(hi_q + kHalf + 1) - cnt(lo_q + kHalf + 1);
    const int s_in = psum[hi_q + kHalf + 1] - psum[lo_q + kHalf + 1];
    const bool take = start && n_in > 0;
    const double ts = take ? (double)s_in : cs;
    const double tc = take ? (double)n_in : cc;
    // Stable rank by value: centroids below, and equal ones at lower lanes.
    int rank = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const double bs = from_lane(ts, b), bc = from_lane(tc, b);
      const double l = bs * tc, r = ts * bc;
      rank += (l < r || (l == r && b < a)) ? 1 : 0;
    }
    // Lane g0 + rank receives this centroid.
    const double ss = permute_to(g0 + rank, ts);
    const double sc = permute_to(g0 + rank, tc);
    const bool same = ss * cc == cs * sc;
    cs = ss;
    cc = sc;
    if (((uint32_t)__ballot(same) & 0xFFu) == 0xFFu) break;
  }

  // 4: round to E4M3FN, one entry per lane.
  if (t < 8) cb[row * 8 + a] = round_e4m3fn((int64_t)cs, (int64_t)cc);
}

template <bool kNarrow>
hipError_t launch_fit(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* cb, hipStream_t s) {
  const size_t shm = (kBins + 1) * sizeof(int) + (kBins + 1) * (kNarrow ? sizeof(uint16_t) : sizeof(int));
  static LdsAllowance seen;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(fit_kernel<kNarrow>), shm, seen);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fit_kernel<kNarrow>, dim3((unsigned)n), dim3(kFitThreads), shm, s, w, ldw, k, cb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fit_codebook(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* cb, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return k < 65536 ? launch_fit<true>(w, ldw, n, k, cb, s) : launch_fit<false>(w, ldw, n, k, cb, s);
}

}  // namespace q3
