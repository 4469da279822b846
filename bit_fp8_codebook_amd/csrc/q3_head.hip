// The two-bit draft head's shortlist and FP8 rescoring (Hibana: Fast Agentic
// Inference on Unified-Memory Devices, "Model surgery" / "Two-bit draft head":
// a 2-bit copy of the drafter's output head shortlists candidates, and only
// those are scored again with the FP8 head, which makes the decision).
//
// The 2-bit scores of every row come from the matrix-core product in
// q3_linear.hip.  Here:
//   * shortlist: per query the `size` (<= 16) largest scores, larger first,
//     equal scores to the lower row.  Pass 1 runs kShortlistChunks blocks per
//     query, each keeping the top 16 of its slice of rows: per-thread sorted
//     lists, then 16 rounds that each take the best head over a wave's lists
//     (DPP maximum of the key, then minimum of the row among equal keys),
//     first within each wave, then over the waves' lists; pass 2 merges the
//     chunks' lists the same way.  The order (score desc, row asc) is total,
//     so the result is unique and run-to-run identical.
//   * rescore: per query one block; each wave takes listed rows, streams the
//     row's MXFP8 elements (E4M3FN, one E8M0 scale per 32) and the query's
//     bf16 activations, widens the elements exactly to bf16 with the scale
//     folded into the conversion, and accumulates v_dot2 products in fp32; a
//     fixed-order lane reduction gives the score.  The block then picks the
//     listed row with the largest score (ties to the lower row) by the same
//     wave-wide maximum and minimum.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kList = kShortlistMax;   // entries kept per list
constexpr int kThreads1 = 1024;        // pass-1 block size

// Entries are (key, row): key = an order-preserving 32-bit image of the score
// (larger score, larger key; -0 folded into +0, which compares equal to it as
// a score), ranked by key desc, then row asc.  Key 0 (below every finite
// score's key) with row kNoRow marks an empty slot.
__device__ __forceinline__ uint32_t score_key(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int kNoRow = 0x7FFFFFFF;

template <int L>
__device__ __forceinline__ void empty_list(uint32_t (&lk)[L], int (&li)[L]) {
#pragma unroll
  for (int j = 0; j < L; ++j) {
    lk[j] = 0u;
    li[j] = kNoRow;
  }
}

// Insert (k, id) into a lane's sorted list, branch-free.  The caller scans
// rows in increasing order, so the new entry goes after every kept entry with
// an equal or larger key (and falls off the end if there are L of them).
template <int L>
__device__ __forceinline__ void list_insert(uint32_t (&lk)[L], int (&li)[L], uint32_t k, int id) {
  bool g[L];   // g[j]: entry j stays in front of the new one
#pragma unroll
  for (int j = 0; j < L; ++j) g[j] = lk[j] >= k;
#pragma unroll
  for (int j = L - 1; j >= 0; --j) {
    const bool gp = j == 0 ? true : g[j - 1];
    const uint32_t pk = j == 0 ? 0u : lk[j - 1];
    const int pi = j == 0 ? 0 : li[j - 1];
    lk[j] = g[j] ? lk[j] : (gp ? k : pk);
    li[j] = g[j] ? li[j] : (gp ? id : pi);
  }
}

// Wave-wide maximum (minimum) of an unsigned value: DPP exchanges within
// quads, half-rows and rows, then the row broadcasts that leave the wave's
// result in lane 63, which is read out (the same value in every lane).  Lanes
// a broadcast does not write see the identity (0 for the maximum, all ones
// for the minimum), so no copy of the value is needed for them.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_extreme(uint32_t v) {
  constexpr int kId = kMax ? 0 : -1;
  auto pick = [](uint32_t a, int b) {
    const uint32_t u = (uint32_t)b;
    return kMax ? (a > u ? a : u) : (a < u ? a : u);
  };
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast15
  v = pick(v, __builtin_amdgcn_update_dpp(kId, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The wave's kList best entries over the sorted lists (L entries each) held
// by its 64 lanes, best first (the same values in every lane).  Each round
// takes the largest head key over the wave, then the lowest row among the
// heads with that key (read from the one lane holding the key when there is
// only one, the common case); that is the best head (rows of real entries
// are distinct), and the lane holding it drops its head.  Several lanes can
// hold the empty entry (0, kNoRow) at once; they all drop it, and every
// later round then yields the same empty entry again.
template <int L>
__device__ __forceinline__ void wave_top(uint32_t (&lk)[L], int (&li)[L], uint32_t (&ok)[kList], int (&oi)[kList]) {
#pragma unroll
  for (int o = 0; o < kList; ++o) {
    const uint32_t bk = wave_extreme<true>(lk[0]);
    const uint64_t hold = __ballot(lk[0] == bk);
    const int bi = __builtin_popcountll(hold) == 1
                       ? __builtin_amdgcn_readlane(li[0], (int)__builtin_ctzll(hold))
                       : (int)wave_extreme<false>(lk[0] == bk ? (uint32_t)li[0] : (uint32_t)kNoRow);
    ok[o] = bk;
    oi[o] = bi;
    const bool mine = lk[0] == bk && li[0] == bi;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      lk[j] = mine ? lk[j + 1] : lk[j];
      li[j] = mine ? li[j + 1] : li[j];
    }
    lk[L - 1] = mine ? 0u : lk[L - 1];
    li[L - 1] = mine ? kNoRow : li[L - 1];
  }
}

struct Cand {
  uint32_t k;
  int id;
};

// Pass 1: block (c, q) keeps the top kList rows of chunk c of query q:
// per-lane lists, the top of each wave, then the top of the block's waves.
// A lane's rows of the chunk (two or three for a 151936-row head) are loaded
// in one batch of up to kBatch1 before any insertion.  A lane that meets at
// most L rows keeps them all in an L-entry list (L = 4 when every lane meets
// at most 4, else kList), which makes the insertions and the wave's rounds
// cheaper: 16 waves share the CU, so the pass is bound by instruction issue.
constexpr int kWaves1 = kThreads1 / 64;
constexpr int kBatch1 = 16;
constexpr int kShortRun = 4;
template <int L>
__global__ __launch_bounds__(kThreads1) void shortlist_chunks(const float* __restrict__ scores, int64_t n, int64_t ld,
                                                              Cand* __restrict__ cand) {
  __shared__ uint32_t sk[kWaves1 * kList];
  __shared__ int si[kWaves1 * kList];
  const int q = blockIdx.y, c = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cs = (n + kShortlistChunks - 1) / kShortlistChunks;
  const int64_t r0 = (int64_t)c * cs;
  const int64_t r1 = r0 + cs < n ? r0 + cs : n;
  uint32_t lk[L];
  int li[L];
  empty_list(lk, li);
  const float* row = scores + (int64_t)q * ld;
  for (int64_t base = r0 + threadIdx.x; base < r1; base += kBatch1 * kThreads1) {
    float v[kBatch1];
#pragma unroll
    for (int u = 0; u < kBatch1; ++u) {
      const int64_t r = base + (int64_t)u * kThreads1;
      v[u] = r < r1 ? row[r] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBatch1; ++u) {
      const int64_t r = base + (int64_t)u * kThreads1;
      if (r < r1) list_insert(lk, li, score_key(v[u]), (int)r);
    }
  }
  uint32_t ok[kList];
  int oi[kList];
  wave_top(lk, li, ok, oi);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kList; ++j) {
      sk[wave * kList + j] = ok[j];
      si[wave * kList + j] = oi[j];
    }
  }
  __syncthreads();
  if (wave == 0) {
    // Lane t holds entries 4(t%4) .. 4(t%4)+3 of wave t/4's list: a sorted
    // four-entry list per lane, the 16 waves' lists between them.
    static_assert(kWaves1 * kList == kShortRun * 64, "four entries per lane");
    uint32_t k4[kShortRun];
    int i4[kShortRun];
#pragma unroll
    for (int j = 0; j < kShortRun; ++j) {
      k4[j] = sk[kShortRun * lane + j];
      i4[j] = si[kShortRun * lane + j];
    }
    wave_top(k4, i4, ok, oi);
    Cand* out = cand + ((int64_t)q * kShortlistChunks + c) * kList;
#pragma unroll
    for (int j = 0; j < kList; ++j)
      if (lane == j) out[j] = Cand{ok[j], oi[j]};
  }
}

// Pass 2, one wave per query: lane c holds chunk c's sorted list.
static_assert(kShortlistChunks == 64, "one chunk list per lane");
__device__ __forceinline__ void merge_chunks(const Cand* __restrict__ in, uint32_t (&ok)[kList], int (&oi)[kList]) {
  const int lane = threadIdx.x & 63;
  uint32_t lk[kList];
  int li[kList];
#pragma unroll
  for (int j = 0; j < kList; ++j) {
    const Cand e = in[lane * kList + j];
    lk[j] = e.k;
    li[j] = e.id;
  }
  wave_top(lk, li, ok, oi);
}

__global__ __launch_bounds__(64) void shortlist_merge(const Cand* __restrict__ cand, int32_t size,
                                                      int32_t* __restrict__ ids, float* __restrict__ vals) {
  const int q = blockIdx.x;
  const int lane = threadIdx.x;
  uint32_t ok[kList];
  int oi[kList];
  merge_chunks(cand + (int64_t)q * kShortlistChunks * kList, ok, oi);
#pragma unroll
  for (int j = 0; j < kList; ++j)
    if (lane == j && j < size) {
      ids[(int64_t)q * size + j] = oi[j];
      if (vals) vals[(int64_t)q * size + j] = key_score(ok[j]);
    }
}

// Rescore: block q scores the listed rows of query q with the MXFP8 head, one
// wave per listed row.  Lane l takes elements 1024p + 16l .. +15 (p = 0..3) of
// each 4096-wide slice of K: four 16-byte element loads (each instruction
// reads 1 KB of the row contiguously), eight 16-byte activation loads and four
// scale bytes, all issued before any arithmetic.  With `cand` set the
// block first merges the query's chunk lists (pass 2 of the shortlist) and
// writes the list to ids.
constexpr int kRescoreWaves = kList;
__global__ __launch_bounds__(64 * kRescoreWaves) void rescore_kernel(Mxfp8View h, const uint16_t* __restrict__ x,
                                                                     int64_t ldx, const Cand* __restrict__ cand,
                                                                     int32_t* __restrict__ ids, int32_t size,
                                                                     float* __restrict__ y,
                                                                     int32_t* __restrict__ best) {
  __shared__ float sy[kList];
  __shared__ int sid[kList];
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (cand) {
    if (wave == 0) {
      uint32_t ok[kList];
      int oi[kList];
      merge_chunks(cand + (int64_t)q * kShortlistChunks * kList, ok, oi);
#pragma unroll
      for (int j = 0; j < kList; ++j)
        if (lane == j && j < size) {
          sid[j] = oi[j];
          ids[(int64_t)q * size + j] = oi[j];
        }
    }
  } else if ((int)threadIdx.x < size) {
    sid[threadIdx.x] = ids[(int64_t)q * size + threadIdx.x];
  }
  __syncthreads();
  const rsrc_t er = make_rsrc(h.e8, (uint32_t)(h.n * h.lde));
  const rsrc_t sr = make_rsrc(h.s8, (uint32_t)(h.n * h.lds));
  const rsrc_t xr = make_rsrc(x + (int64_t)q * ldx, (uint32_t)(h.k * 2));
  if (wave < size) {
    const int id = sid[wave];
    const bool ok = id >= 0 && id < h.n;
    float acc = 0.f;
    for (int64_t k0 = 0; k0 < h.k; k0 += 4096) {
      // Lane l takes elements k0 + 1024p + 16l .. +15 (p = 0..3): each element
      // load reads 1 KB of the row contiguously, and the activations and the
      // scale byte of those 16 elements follow the same positions.
      u32x4 e[4], xv[8];
      uint32_t sb[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int64_t kp = k0 + 1024 * p + 16 * lane;   // 16 elements, all in or all out (k % 32 == 0)
        const bool in = kp < h.k;
        e[p] = bload128(er, ok && in ? (uint32_t)(id * h.lde + kp) : kOob);
        xv[2 * p] = bload128(xr, in ? (uint32_t)(2 * kp) : kOob);
        xv[2 * p + 1] = bload128(xr, in ? (uint32_t)(2 * kp + 16) : kOob);
        sb[p] = bload8(sr, ok && in ? (uint32_t)(id * h.lds + kp / 32) : kOob);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float sc = e8m0_to_f32(sb[p]);
        const uint32_t wd[4] = {e[p].x, e[p].y, e[p].z, e[p].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x4 xx = xv[2 * p + d / 2];
          const uint32_t x0 = (d & 1) ? xx.z : xx.x, x1 = (d & 1) ? xx.w : xx.y;
          acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(wd[d], sc, false), as_bf16x2(x0), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(fp8x2_to_bf16x2(wd[d], sc, true), as_bf16x2(x1), acc, false);
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off /= 2) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
      sy[wave] = acc;
      y[(int64_t)q * size + wave] = acc;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // The listed row with the largest score, equal scores to the lower id
    // (signed: ids are the caller's when no list is given), across lanes.
    const bool live = lane < size;
    const uint32_t k = live ? score_key(sy[lane]) : 0u;
    const uint32_t id = live ? (uint32_t)sid[lane] ^ 0x80000000u : 0xFFFFFFFFu;
    const uint32_t bk = wave_extreme<true>(k);
    const uint32_t bi = wave_extreme<false>(live && k == bk ? id : 0xFFFFFFFFu);
    if (lane == 0) best[q] = (int)(bi ^ 0x80000000u);
  }
}

}  // namespace

hipError_t launch_shortlist(const float* scores, int64_t m, int64_t n, int64_t ld, int32_t size, void* cand,
                            int32_t* ids, float* vals, hipStream_t s) {
  Cand* c = static_cast<Cand*>(cand);
  const int64_t rows_per_lane = ((n + kShortlistChunks - 1) / kShortlistChunks + kThreads1 - 1) / kThreads1;
  if (rows_per_lane <= kShortRun)
    hipLaunchKernelGGL(shortlist_chunks<kShortRun>, dim3(kShortlistChunks, (unsigned)m), dim3(kThreads1), 0, s, scores,
                       n, ld, c);
  else
    hipLaunchKernelGGL(shortlist_chunks<kList>, dim3(kShortlistChunks, (unsigned)m), dim3(kThreads1), 0, s, scores, n,
                       ld, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !ids) return e;
  hipLaunchKernelGGL(shortlist_merge, dim3((unsigned)m), dim3(64), 0, s, c, size, ids, vals);
  return hipGetLastError();
}

hipError_t launch_rescore(const Mxfp8View& h, const uint16_t* x, int64_t m, int64_t ldx, const void* cand,
                          int32_t* ids, int32_t size, float* y, int32_t* best, hipStream_t s) {
  hipLaunchKernelGGL(rescore_kernel, dim3((unsigned)m), dim3(64 * kRescoreWaves), 0, s, h, x, ldx,
                     static_cast<const Cand*>(cand), ids, size, y, best);
  return hipGetLastError();
}

}  // namespace q3
