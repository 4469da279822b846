// Matrix-core decode product for 1..64 tokens over the 3.25-bit codebook format.
//
// What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices,
// "Model surgery" / "Three-bit weights"): y[m][n] = sum_k x[m][k] * w[n][k].  The
// page's own kernel looks the codes up and feeds the FP8 matrix units; here the
// looked-up E4M3 bytes are widened exactly to bf16 (group scale folded into the
// conversion) and fed to gfx950's v_mfma_f32_16x16x32_bf16, so every product is
// exact and only the fp32 accumulation rounds, whatever the activations are.
//
// Wave tile: 16 weight rows (MFMA A operand) x 16 tokens per column tile (MFMA
// B operand), fp32 accumulators in the MFMA C/D registers.  Lane l serves row
// l%16 and k-block l/16: per step it loads 48 contiguous bytes of codes (three
// 16-byte loads = 4 groups of its row) plus the 4 scale bytes of those groups,
// so a wave step covers 16 rows x 16 groups (512 k).  Each group is dequantised
// once into 16 bf16 pairs, i.e. the A operands of 4 MFMAs (8 k each per lane).
// The B operand of the same lane is the matching 8 activations of token
// 16c + l%16, so A and B agree on which k sits in which slot by construction.
// The four waves of a block split K when there are few rows (partial sums are
// added through LDS in a fixed order: no atomics, run-to-run identical) and take
// different row tiles otherwise.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 pack_bf16x8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
             __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

template <int MT>
__global__ __launch_bounds__(256) void mfma_kernel(PlaneView w, const uint16_t* __restrict__ x, int64_t ldx,
                                                   int m, float* __restrict__ y, int64_t ldy, int sk) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;    // A: weight row in the tile / B: token in the column tile
  const int kb = lane >> 4;   // k-block of the lane (0..3)
  const int rb = 4 / sk;      // row tiles per block
  const int rt = wave / sk;
  const int ks = wave - rt * sk;
  const int64_t row_base = ((int64_t)blockIdx.x * rb + rt) * 16;
  const int64_t row = row_base + i;
  const bool rvalid = row < w.n;
  const int G = w.groups;
  const int steps = (G + 15) / 16;
  const int s0 = (ks * steps) / sk;
  const int s1 = ((ks + 1) * steps) / sk;

  uint32_t cbl = 0u, cbh = 0u;
  if (rvalid) {
    const uint2 cb = *reinterpret_cast<const uint2*>(w.cb + 8 * row);
    cbl = cb.x;
    cbh = cb.y;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int c = 0; c < MT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = s0; s < s1; ++s) {
    const int gq = 16 * s + 4 * kb;   // first of the lane's 4 groups (chunk aligned)
    uint4 c0 = make_uint4(0u, 0u, 0u, 0u), c1 = c0, c2 = c0;
    uint32_t sc4 = 0u;
    if (rvalid && gq < G) {
      const uint4* p = reinterpret_cast<const uint4*>(w.code + row * w.code_pitch + 12 * gq);
      c0 = p[0];
      c1 = p[1];
      c2 = p[2];
      sc4 = *reinterpret_cast<const uint32_t*>(w.scale + row * w.scale_pitch + gq);
    }
    const uint32_t cw[12] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w, c2.x, c2.y, c2.z, c2.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int g = gq + t;
      const bool gvalid = g < G;
      const bool wvalid = rvalid && gvalid;
      bf16x2 wv[16];
      dequant_group_bf16(cw[3 * t], cw[3 * t + 1], cw[3 * t + 2], (sc4 >> (8 * t)) & 0xFFu, wvalid ? cbl : 0u,
                         wvalid ? cbh : 0u, wv);
      bf16x8 a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = pack_bf16x8(wv[4 * e], wv[4 * e + 1], wv[4 * e + 2], wv[4 * e + 3]);
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        const int tok = 16 * c + i;
        uint4 xb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xb[e] = make_uint4(0u, 0u, 0u, 0u);
        if (tok < m && gvalid) {
          const uint4* xp = reinterpret_cast<const uint4*>(x + tok * ldx + (int64_t)kGroup * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) xb[e] = xp[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[e], __builtin_bit_cast(bf16x8, xb[e]), acc[c], 0, 0, 0);
      }
    }
  }

  if (sk > 1) {
    __shared__ f32x4 red[4][MT][64];
#pragma unroll
    for (int c = 0; c < MT; ++c) red[wave][c][lane] = acc[c];
    __syncthreads();
    if (ks == 0) {
      for (int q = 1; q < sk; ++q) {
#pragma unroll
        for (int c = 0; c < MT; ++c) acc[c] += red[wave + q][c][lane];
      }
    }
  }
  if (ks == 0) {
    // D layout: lane l holds rows 4*(l/16)+v (v = 0..3) of the tile for token l%16.
#pragma unroll
    for (int c = 0; c < MT; ++c) {
      const int tok = 16 * c + i;
      if (tok < m) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t r = row_base + 4 * kb + v;
          if (r < w.n) y[tok * ldy + r] = acc[c][v];
        }
      }
    }
  }
}

// K-split factor: split K over the block's waves until there are enough blocks
// to occupy the chip, never more ways than there are 512-k steps.
int choose_split(int64_t n, int groups) {
  const int64_t tiles = (n + 15) / 16;
  const int steps = (groups + 15) / 16;
  int sk = 1;
  while (sk < 4 && (tiles + (4 / sk) - 1) / (4 / sk) < 1024 && sk * 2 <= steps) sk *= 2;
  return sk;
}

template <int MT>
hipError_t launch_mt(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                     hipStream_t s) {
  const int sk = choose_split(w.n, w.groups);
  const int64_t tiles = (w.n + 15) / 16;
  const int rb = 4 / sk;
  const dim3 grid((unsigned)((tiles + rb - 1) / rb));
  hipLaunchKernelGGL((mfma_kernel<MT>), grid, dim3(256), 0, s, w, x, ldx, (int)m, y, ldy, sk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_small_m(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                               int64_t ldy, hipStream_t s) {
  if (w.n == 0) return hipSuccess;
  if (m <= 16) return launch_mt<1>(w, x, m, ldx, y, ldy, s);
  if (m <= 32) return launch_mt<2>(w, x, m, ldx, y, ldy, s);
  if (m <= 48) return launch_mt<3>(w, x, m, ldx, y, ldy, s);
  return launch_mt<4>(w, x, m, ldx, y, ldy, s);
}

}  // namespace q3
