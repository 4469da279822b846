// Shared body of the VALU GEMV: used by the dense product (q3_gemv.hip) and the
// expert-grouped product (q3_moe.hip).
//
// What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices,
// "Model surgery" / "Three-bit weights"): y[m][n] = sum_k x[m][k] * w[n][k] with
// w = codebook[n][code] * 2^(scale-127).  Decoding reads every weight once per
// token, so the kernel is built around streaming the 13 payload bytes per group
// exactly once.
//
// Work mapping: a thread owns one group column g (32 consecutive k) and walks
// rows; its 32 activations per token stay in registers (16 bf16 pairs) and are
// reused for every row it visits.  The threads of one row slot are consecutive,
// so a row's codes (12 bytes per thread) and scales (1 byte per thread) are read
// with fully coalesced loads.  Per group and row: 17 ALU ops unpack the indices,
// 8 byte permutes look up E4M3 bytes, 16 conversions widen them exactly to bf16
// with the group scale folded in, and 16*M bf16 dot2 instructions accumulate in
// fp32.  Partial sums of the P rows a thread visits are combined across the
// row's threads with a transposing butterfly (one shuffle per value instead of
// one per value per level) and, when a row spans several waves, through LDS.
#pragma once

#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {

// Tokens are addressed through per-token row pointers so the same body serves
// the dense product and the expert-grouped one (gathered activations).
template <int M>
struct TokenRows {
  const uint16_t* x[M];
  float* y[M];
};

constexpr int kGemvThreads = 256;
constexpr int kGemvPasses = 4;   // rows visited per thread per block

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

// One block: RS row slots x TPR group lanes (RS*TPR = 256), P passes over rows.
// `cached` means every group of a row has its own thread (groups <= 256), so the
// activations are loaded once; otherwise each thread loops over groups
// g, g+256, ... and reloads activations per group (correct for any k).
template <int M, bool kCached>
__device__ __forceinline__ void gemv_block(const PlaneView& w, const TokenRows<M>& tok, int lg_tpr,
                                           int64_t row0) {
  constexpr int P = kGemvPasses;
  constexpr int MP = pow2_tokens<M>();
  constexpr int V = P * MP;
  __shared__ float red[kGemvThreads / 64][V];

  const int tid = threadIdx.x;
  const int TPR = 1 << lg_tpr;
  const int RS = kGemvThreads >> lg_tpr;
  const int tg = tid & (TPR - 1);
  const int tr = tid >> lg_tpr;
  const int G = w.groups;

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;

  const int nj = kCached ? 1 : (G + TPR - 1) / TPR;
  for (int j = 0; j < nj; ++j) {
    const int g = tg + j * TPR;
    const bool gvalid = g < G;

    uint32_t xr[M][16];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (gvalid) v = *reinterpret_cast<const uint4*>(tok.x[m] + (int64_t)kGroup * g + 8 * q);
        xr[m][4 * q + 0] = v.x;
        xr[m][4 * q + 1] = v.y;
        xr[m][4 * q + 2] = v.z;
        xr[m][4 * q + 3] = v.w;
      }
    }

    // Issue every pass's loads before any arithmetic.
    uint32_t d[P][3], sb[P], cbl[P], cbh[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t row = row0 + (int64_t)p * RS + tr;
      if (gvalid && row < w.n) {
        const uint32_t* c = reinterpret_cast<const uint32_t*>(w.code + row * w.code_pitch) + 3 * g;
        d[p][0] = c[0];
        d[p][1] = c[1];
        d[p][2] = c[2];
        sb[p] = w.scale[row * w.scale_pitch + g];
        const uint2 cb = *reinterpret_cast<const uint2*>(w.cb + 8 * row);
        cbl[p] = cb.x;
        cbh[p] = cb.y;
      } else {
        d[p][0] = d[p][1] = d[p][2] = 0u;
        sb[p] = 127u;
        cbl[p] = cbh[p] = 0u;   // zero codebook: the slot contributes exactly 0
      }
    }

#pragma unroll
    for (int p = 0; p < P; ++p) {
      bf16x2 wv[16];
      dequant_group_bf16(d[p][0], d[p][1], d[p][2], sb[p], cbl[p], cbh[p], wv);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = acc[p * MP + m];
#pragma unroll
        for (int q = 0; q < 16; ++q) a = __builtin_amdgcn_fdot2_f32_bf16(wv[q], as_bf16x2(xr[m][q]), a, false);
        acc[p * MP + m] = a;
      }
    }
  }

  // Combine the partial sums of a row's TPR threads.
  const int S = TPR < 64 ? TPR : 64;
  const int lane = tid & 63;
  if (S >= V) {
    const float r = transpose_reduce<V>(acc, S);
    const int lgS = 31 - __builtin_clz(S);
    const int lgV = 31 - __builtin_clz(V);
    const int ls = lane & (S - 1);
    const int vi = ls >> (lgS - lgV);
    const bool writer = (ls & ((S >> lgV) - 1)) == 0;
    if (TPR <= 64) {
      const int p = vi / MP, m = vi % MP;
      const int64_t row = row0 + (int64_t)p * RS + tr;
      if (writer && m < M && row < w.n) tok.y[m][row] = r;
    } else {
      if (writer) red[tid >> 6][vi] = r;
      __syncthreads();
      const int wps = TPR >> 6;                     // waves per row slot
      if (tid < RS * V) {
        const int slot = tid / V, v = tid % V;
        float s = 0.f;
        for (int q = 0; q < wps; ++q) s += red[slot * wps + q][v];
        const int p = v / MP, m = v % MP;
        const int64_t row = row0 + (int64_t)p * RS + slot;
        if (m < M && row < w.n) tok.y[m][row] = s;
      }
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
        const int64_t row = row0 + (int64_t)p * RS + tr;
        if (m < M && row < w.n) tok.y[m][row] = acc[i];
      }
    }
  }
}

// log2 of the threads per row: the smallest power of two covering the row's
// groups, at most the whole block.
inline int gemv_lg_tpr(int groups) {
  int lg = 0;
  while ((1 << lg) < groups && lg < 8) ++lg;
  return lg;
}

}  // namespace q3
