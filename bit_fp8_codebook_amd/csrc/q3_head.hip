// The two-bit draft head's shortlist and FP8 rescoring (Hibana: Fast Agentic
// Inference on Unified-Memory Devices, "Model surgery" / "Two-bit draft head":
// a 2-bit copy of the drafter's output head shortlists candidates, and only
// those are scored again with the FP8 head, which makes the decision).
//
// The 2-bit scores of every row come from the matrix-core product in
// q3_linear.hip.  Here:
//   * shortlist: per query the `size` (<= 16) largest scores, larger first,
//     equal scores to the lower row.  Pass 1 runs kShortlistChunks blocks per
//     query, each keeping the top 16 of its slice of rows (per-thread sorted
//     lists, then a pairwise merge tree in LDS); pass 2 merges the chunks'
//     lists with the same tree.  The order (score desc, row asc) is total, so
//     the result is unique and run-to-run identical.
//   * rescore: per query one block; each wave takes listed rows, streams the
//     row's MXFP8 elements (E4M3FN, one E8M0 scale per 32) and the query's
//     bf16 activations, widens the elements exactly to bf16 with the scale
//     folded into the conversion, and accumulates v_dot2 products in fp32; a
//     fixed-order lane reduction gives the score.  The block then picks the
//     listed row with the largest score (ties to the lower row).
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kList = kShortlistMax;   // entries kept per list
constexpr int kThreads1 = 256;         // pass-1 block size

// (a, ia) ranks before (b, ib): larger score, or equal score and lower row.
__device__ __forceinline__ bool before(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

// Insert (v, id) into a sorted register list (v[0] best).  The caller scans
// rows in increasing order, so an equal score never displaces a kept one.
__device__ __forceinline__ void list_insert(float (&lv)[kList], int (&li)[kList], float v, int id) {
  if (!(v > lv[kList - 1])) return;
  lv[kList - 1] = v;
  li[kList - 1] = id;
#pragma unroll
  for (int j = kList - 1; j > 0; --j) {
    if (before(lv[j], li[j], lv[j - 1], li[j - 1])) {
      const float tv = lv[j];
      lv[j] = lv[j - 1];
      lv[j - 1] = tv;
      const int ti = li[j];
      li[j] = li[j - 1];
      li[j - 1] = ti;
    }
  }
}

// Merge the sorted lists at LDS slots a and b into slot a (top kList kept).
__device__ __forceinline__ void merge_lists(float* sv, int* si, int a, int b) {
  float ov[kList];
  int oi[kList];
  int x = 0, y = 0;
#pragma unroll
  for (int o = 0; o < kList; ++o) {
    const float va = sv[a * kList + x], vb = sv[b * kList + y];
    const int ia = si[a * kList + x], ib = si[b * kList + y];
    const bool takea = before(va, ia, vb, ib);
    ov[o] = takea ? va : vb;
    oi[o] = takea ? ia : ib;
    x += takea ? 1 : 0;
    y += takea ? 0 : 1;
  }
#pragma unroll
  for (int o = 0; o < kList; ++o) {
    sv[a * kList + o] = ov[o];
    si[a * kList + o] = oi[o];
  }
}

// Tree-merge the `count` (a power of two) lists in LDS into slot 0.
__device__ __forceinline__ void merge_tree(float* sv, int* si, int count) {
  for (int stride = count / 2; stride > 0; stride /= 2) {
    __syncthreads();
    if ((int)threadIdx.x < stride) merge_lists(sv, si, threadIdx.x, threadIdx.x + stride);
  }
  __syncthreads();
}

struct Cand {
  float v;
  int id;
};

// Pass 1: block (c, q) keeps the top kList rows of chunk c of query q.
__global__ __launch_bounds__(kThreads1) void shortlist_chunks(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                              Cand* __restrict__ cand) {
  __shared__ float sv[kThreads1 * kList];
  __shared__ int si[kThreads1 * kList];
  const int q = blockIdx.y, c = blockIdx.x;
  const int64_t cs = (n + kShortlistChunks - 1) / kShortlistChunks;
  const int64_t r0 = (int64_t)c * cs;
  const int64_t r1 = r0 + cs < n ? r0 + cs : n;
  float lv[kList];
  int li[kList];
#pragma unroll
  for (int j = 0; j < kList; ++j) {
    lv[j] = -__builtin_inff();   // below every (finite) score
    li[j] = 0x7FFFFFFF;
  }
  const float* row = scores + (int64_t)q * ld;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kThreads1) list_insert(lv, li, row[r], (int)r);
#pragma unroll
  for (int j = 0; j < kList; ++j) {
    sv[threadIdx.x * kList + j] = lv[j];
    si[threadIdx.x * kList + j] = li[j];
  }
  merge_tree(sv, si, kThreads1);
  if (threadIdx.x < kList) {
    Cand* out = cand + ((int64_t)q * kShortlistChunks + c) * kList;
    out[threadIdx.x] = Cand{sv[threadIdx.x], si[threadIdx.x]};
  }
}

// Pass 2: block q merges the chunk lists of query q and writes the first `size`.
__global__ __launch_bounds__(kShortlistChunks) void shortlist_merge(const Cand* __restrict__ cand, int32_t size,
                                                                    int32_t* __restrict__ ids, float* __restrict__ vals) {
  __shared__ float sv[kShortlistChunks * kList];
  __shared__ int si[kShortlistChunks * kList];
  const int q = blockIdx.x;
  const Cand* in = cand + (int64_t)q * kShortlistChunks * kList;
#pragma unroll
  for (int j = 0; j < kList; ++j) {
    const Cand e = in[threadIdx.x * kList + j];
    sv[threadIdx.x * kList + j] = e.v;
    si[threadIdx.x * kList + j] = e.id;
  }
  merge_tree(sv, si, kShortlistChunks);
  if ((int)threadIdx.x < size) {
    ids[(int64_t)q * size + threadIdx.x] = si[threadIdx.x];
    if (vals) vals[(int64_t)q * size + threadIdx.x] = sv[threadIdx.x];
  }
}

// Rescore: block q scores the listed rows of query q with the MXFP8 head.
constexpr int kRescoreWaves = 4;
__global__ __launch_bounds__(64 * kRescoreWaves) void rescore_kernel(Mxfp8View h, const uint16_t* __restrict__ x,
                                                                     int64_t ldx, const int32_t* __restrict__ ids,
                                                                     int32_t size, float* __restrict__ y,
                                                                     int32_t* __restrict__ best) {
  __shared__ float sy[kList];
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const rsrc_t er = make_rsrc(h.e8, (uint32_t)(h.n * h.lde));
  const rsrc_t sr = make_rsrc(h.s8, (uint32_t)(h.n * h.lds));
  const rsrc_t xr = make_rsrc(x + (int64_t)q * ldx, (uint32_t)(h.k * 2));
  for (int j = wave; j < size; j += kRescoreWaves) {
    const int id = ids[(int64_t)q * size + j];
    const bool ok = id >= 0 && id < h.n;
    float acc = 0.f;
    // Lane l takes 8 consecutive elements per 512-element slice (one quarter
    // of a 32-element scale group).
    for (int64_t k0 = 8 * lane; k0 < h.k; k0 += 512) {
      const uint32_t eo = ok ? (uint32_t)(id * h.lde + k0) : kOob;
      const u32x2 e = bload64(er, eo);
      const uint32_t sb = bload8(sr, ok ? (uint32_t)(id * h.lds + k0 / 32) : kOob);
      const u32x4 xv = bload128(xr, (uint32_t)(2 * k0));
      const float sc = e8m0_to_f32(sb);
      acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(e.x, sc, false), as_bf16x2(xv.x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(e.x, sc, true), as_bf16x2(xv.y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(e.y, sc, false), as_bf16x2(xv.z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(e.y, sc, true), as_bf16x2(xv.w), acc, false);
    }
#pragma unroll
    for (int off = 32; off > 0; off /= 2) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
      sy[j] = acc;
      y[(int64_t)q * size + j] = acc;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int bj = 0;
    for (int j = 1; j < size; ++j)
      if (before(sy[j], ids[(int64_t)q * size + j], sy[bj], ids[(int64_t)q * size + bj])) bj = j;
    best[q] = ids[(int64_t)q * size + bj];
  }
}

}  // namespace

hipError_t launch_shortlist(const float* scores, int64_t m, int64_t n, int64_t ld, int32_t size, void* cand,
                            int32_t* ids, float* vals, hipStream_t s) {
  Cand* c = static_cast<Cand*>(cand);
  hipLaunchKernelGGL(shortlist_chunks, dim3(kShortlistChunks, (unsigned)m), dim3(kThreads1), 0, s, scores, n, ld, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(shortlist_merge, dim3((unsigned)m), dim3(kShortlistChunks), 0, s, c, size, ids, vals);
  return hipGetLastError();
}

hipError_t launch_rescore(const Mxfp8View& h, const uint16_t* x, int64_t m, int64_t ldx, const int32_t* ids,
                          int32_t size, float* y, int32_t* best, hipStream_t s) {
  hipLaunchKernelGGL(rescore_kernel, dim3((unsigned)m), dim3(64 * kRescoreWaves), 0, s, h, x, ldx, ids, size, y, best);
  return hipGetLastError();
}

}  // namespace q3
