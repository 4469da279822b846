// VALU decode GEMV for 1..8 tokens over the 3.25-bit codebook format.
//
// What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices,
// "Model surgery" / "Three-bit weights"): y[m][n] = sum_k x[m][k] * w[n][k] with
// w = codebook[n][code] * 2^(scale-127).  Decoding reads every weight once per
// token, so the kernel is built around streaming the 13 payload bytes per group
// exactly once.
//
// Work mapping: a thread owns one group column g (32 consecutive k) and walks
// rows; its 32 activations per token stay in registers (16 bf16 pairs), loaded
// once per block and reused for every row the block visits.  The threads of a
// row are consecutive, so each of the three code-word loads of a row is one
// 64-byte run per superchunk and the scale loads are one contiguous run.  Per
// group and row: 17 ALU ops unpack the indices, 8 byte permutes look up E4M3
// bytes, 16 conversions widen them exactly to bf16 with the group scale folded
// in, and 16*M bf16 dot2 instructions accumulate in fp32.
//
// A block handles batches of RS*P rows (RS row slots x P passes) in a
// grid-stride loop; the loads of the next batch are issued before the current
// batch is computed, and every load is a buffer load whose out-of-range
// offsets read as zero, so there are no branches around memory operations.
// Partial sums of a batch are combined across the row's threads with a
// transposing butterfly and, when a row spans several waves, through LDS.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kThreads = 256;
constexpr int kPasses = 4;        // rows per thread per batch
constexpr int kMaxBlocks = 1024;  // grid-stride beyond this

template <int M>
constexpr int pow2_tokens() { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// Sum V values over an aligned segment of S lanes (S a power of two, S >= V).
// Each butterfly level halves the number of live values per lane: the lane
// keeps the half selected by its lane bit and receives its partner's copy of
// that half.  Afterwards lane l of the segment holds the total of value index
// (l mod S) >> (log2 S - log2 V).
template <int V>
__device__ __forceinline__ float transpose_reduce(float (&v)[V], int S) {
  const int lane = threadIdx.x & 63;
  int o = S >> 1;
#pragma unroll
  for (int h = V / 2; h >= 1; h >>= 1) {
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float keep = upper ? v[i + h] : v[i];
      const float send = upper ? v[i] : v[i + h];
      v[i] = keep + __shfl_xor(send, o, 64);
    }
    o >>= 1;
  }
  float r = v[0];
  for (; o >= 1; o >>= 1) r += __shfl_xor(r, o, 64);
  return r;
}

struct Batch {
  uint32_t d[kPasses][3];
  uint32_t sb[kPasses];
  uint32_t cbl[kPasses], cbh[kPasses];
};

struct GemvCtx {
  rsrc_t code, scale, cb, x;
  int64_t n;
  uint32_t code_pitch, scale_pitch, ldx_bytes;
  int G, gp, TPR, RS, tg, tr;
};

__device__ __forceinline__ void load_batch(const GemvCtx& c, int g, int64_t row0, Batch& b) {
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t row = row0 + (int64_t)p * c.RS + c.tr;
    const bool ok = row < c.n && g < c.G;
    const uint32_t rc = (uint32_t)row * c.code_pitch;
#pragma unroll
    for (int j = 0; j < 3; ++j) b.d[p][j] = bload32(c.code, ok ? rc + word_offset(g, j, c.gp) : kOob);
    b.sb[p] = bload8(c.scale, ok ? (uint32_t)row * c.scale_pitch + g : kOob);
    const u32x2 cb = bload64(c.cb, row < c.n ? (uint32_t)row * 8u : kOob);
    b.cbl[p] = cb.x;
    b.cbh[p] = cb.y;
  }
}

template <int M>
__device__ __forceinline__ void load_x(const GemvCtx& c, int g, uint32_t (&xr)[M][16]) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = bload128(c.x, g < c.G ? m * c.ldx_bytes + 64u * g + 16u * q : kOob);
      xr[m][4 * q + 0] = v.x;
      xr[m][4 * q + 1] = v.y;
      xr[m][4 * q + 2] = v.z;
      xr[m][4 * q + 3] = v.w;
    }
  }
}

template <int M>
__device__ __forceinline__ void accumulate(const Batch& b, const uint32_t (&xr)[M][16],
                                           float (&acc)[kPasses * pow2_tokens<M>()]) {
  constexpr int MP = pow2_tokens<M>();
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    bf16x2 wv[16];
    dequant_group_bf16(b.d[p][0], b.d[p][1], b.d[p][2], b.sb[p], b.cbl[p], b.cbh[p], wv);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = acc[p * MP + m];
#pragma unroll
      for (int q = 0; q < 16; ++q) a = __builtin_amdgcn_fdot2_f32_bf16(wv[q], as_bf16x2(xr[m][q]), a, false);
      acc[p * MP + m] = a;
    }
  }
}

// Combine a batch's partial sums across the row's threads and store them.
template <int M>
__device__ __forceinline__ void reduce_store(const GemvCtx& c, float (&acc)[kPasses * pow2_tokens<M>()],
                                             int64_t row0, float* __restrict__ y, int64_t ldy,
                                             float (*red)[kPasses * pow2_tokens<M>()]) {
  constexpr int MP = pow2_tokens<M>();
  constexpr int V = kPasses * MP;
  const int tid = threadIdx.x;
  const int S = c.TPR < 64 ? c.TPR : 64;
  const int lane = tid & 63;
  if (S >= V) {
    const float r = transpose_reduce<V>(acc, S);
    const int lgS = 31 - __builtin_clz(S);
    const int lgV = 31 - __builtin_clz(V);
    const int ls = lane & (S - 1);
    const int vi = ls >> (lgS - lgV);
    const bool writer = (ls & ((S >> lgV) - 1)) == 0;
    if (c.TPR <= 64) {
      const int p = vi / MP, m = vi % MP;
      const int64_t row = row0 + (int64_t)p * c.RS + c.tr;
      if (writer && m < M && row < c.n) y[m * ldy + row] = r;
    } else {
      if (writer) red[tid >> 6][vi] = r;
      __syncthreads();
      const int wps = c.TPR >> 6;   // waves per row slot
      if (tid < c.RS * V) {
        const int slot = tid / V, v = tid % V;
        float s = 0.f;
        for (int q = 0; q < wps; ++q) s += red[slot * wps + q][v];
        const int p = v / MP, m = v % MP;
        const int64_t row = row0 + (int64_t)p * c.RS + slot;
        if (m < M && row < c.n) y[m * ldy + row] = s;
      }
      __syncthreads();   // red is reused by the next batch
    }
  } else {
    // Narrow rows (fewer threads per row than values): plain butterfly per value.
#pragma unroll
    for (int i = 0; i < V; ++i)
      for (int o = S >> 1; o >= 1; o >>= 1) acc[i] += __shfl_xor(acc[i], o, 64);
    if ((lane & (S - 1)) == 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int p = i / MP, m = i % MP;
        const int64_t row = row0 + (int64_t)p * c.RS + c.tr;
        if (m < M && row < c.n) y[m * ldy + row] = acc[i];
      }
    }
  }
}

// kCached: every group of a row has its own thread (groups <= 256), so the
// activations are loaded once per block and the next batch is prefetched.
// Otherwise each thread loops over groups g, g+256, ... reloading activations.
template <int M, bool kCached>
__global__ __launch_bounds__(kThreads) void gemv_kernel(PlaneView w, const uint16_t* __restrict__ x,
                                                        int64_t ldx, float* __restrict__ y, int64_t ldy,
                                                        int lg_tpr, int num_batches) {
  constexpr int V = kPasses * pow2_tokens<M>();
  __shared__ float red[kThreads / 64][V];

  GemvCtx c;
  c.n = w.n;
  c.G = w.groups;
  c.gp = (w.groups + 3) & ~3;
  c.TPR = 1 << lg_tpr;
  c.RS = kThreads >> lg_tpr;
  c.tg = threadIdx.x & (c.TPR - 1);
  c.tr = threadIdx.x >> lg_tpr;
  c.code_pitch = (uint32_t)w.code_pitch;
  c.scale_pitch = (uint32_t)w.scale_pitch;
  c.ldx_bytes = (uint32_t)(ldx * 2);
  c.code = make_rsrc(w.code, (uint32_t)(w.n * w.code_pitch));
  c.scale = make_rsrc(w.scale, (uint32_t)(w.n * w.scale_pitch));
  c.cb = make_rsrc(w.cb, (uint32_t)(w.n * 8));
  c.x = make_rsrc(x, (uint32_t)((int64_t)(M - 1) * ldx * 2 + (int64_t)w.groups * 64));
  const int64_t rows_per_batch = (int64_t)c.RS * kPasses;

  float acc[V];
  if (kCached) {
    uint32_t xr[M][16];
    load_x<M>(c, c.tg, xr);
    Batch A, B;
    int b = blockIdx.x;
    load_batch(c, c.tg, b * rows_per_batch, A);
    while (true) {
      load_batch(c, c.tg, (int64_t)(b + (int)gridDim.x) * rows_per_batch, B);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      accumulate<M>(A, xr, acc);
      reduce_store<M>(c, acc, b * rows_per_batch, y, ldy, red);
      b += gridDim.x;
      if (b >= num_batches) break;
      load_batch(c, c.tg, (int64_t)(b + (int)gridDim.x) * rows_per_batch, A);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      accumulate<M>(B, xr, acc);
      reduce_store<M>(c, acc, b * rows_per_batch, y, ldy, red);
      b += gridDim.x;
      if (b >= num_batches) break;
    }
  } else {
    const int nj = (c.G + c.TPR - 1) / c.TPR;
    for (int b = blockIdx.x; b < num_batches; b += gridDim.x) {
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      for (int j = 0; j < nj; ++j) {
        const int g = c.tg + j * c.TPR;
        uint32_t xr[M][16];
        load_x<M>(c, g, xr);
        Batch A;
        load_batch(c, g, b * rows_per_batch, A);
        accumulate<M>(A, xr, acc);
      }
      reduce_store<M>(c, acc, b * rows_per_batch, y, ldy, red);
    }
  }
}

// log2 of the threads per row: the smallest power of two covering the row's
// groups, at most the whole block.
int gemv_lg_tpr(int groups) {
  int lg = 0;
  while ((1 << lg) < groups && lg < 8) ++lg;
  return lg;
}

template <int M>
hipError_t launch_gemv_m(const PlaneView& w, const uint16_t* x, int64_t ldx, float* y, int64_t ldy,
                         hipStream_t s) {
  const int lg = gemv_lg_tpr(w.groups);
  const int64_t rows_per_batch = (int64_t)(kThreads >> lg) * kPasses;
  const int64_t batches = (w.n + rows_per_batch - 1) / rows_per_batch;
  const unsigned grid = (unsigned)(batches < kMaxBlocks ? batches : kMaxBlocks);
  if (w.groups <= kThreads)
    hipLaunchKernelGGL((gemv_kernel<M, true>), dim3(grid), dim3(kThreads), 0, s, w, x, ldx, y, ldy, lg,
                       (int)batches);
  else
    hipLaunchKernelGGL((gemv_kernel<M, false>), dim3(grid), dim3(kThreads), 0, s, w, x, ldx, y, ldy, lg,
                       (int)batches);
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
