// Packing and unpacking of the 3.25-bit format (Hibana: Fast Agentic Inference
// on Unified-Memory Devices, "Model surgery" / "Three-bit weights": a 3-bit
// index per weight, one 8-bit scale per group of 32) and of the two-bit draft
// head's 2.25-bit copy ("Two-bit draft head"; 2-bit indices, same scales).
// One-time work, not on the decode path; written for clarity, one thread per
// group.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

// One thread per (row, group) of the padded tiles: every byte of both planes is
// written exactly once, padding rows and groups as zero.
template <int kBits>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t ldc,
                                                   const uint8_t* __restrict__ scales, int64_t lds, int64_t n,
                                                   int64_t groups, int64_t padded_groups, int64_t padded_rows,
                                                   uint8_t* __restrict__ code_plane, uint8_t* __restrict__ scale_plane) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= padded_rows * padded_groups) return;
  const int64_t r = idx / padded_groups, g = idx % padded_groups;
  const bool real = r < n && g < groups;
  constexpr int kWd = kBits == 2 ? 2 : 3;
  uint32_t w[3] = {0u, 0u, 0u};
  if (real) {
    const uint8_t* c = codes + r * ldc + (int64_t)kGroup * g;
    uint32_t v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = c[i] & (kBits == 2 ? 3u : 7u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if constexpr (kBits == 2) {
        // byte b of word j: code 16j+4q+b in bits 2q..2q+1
#pragma unroll
        for (int j = 0; j < 2; ++j)
          w[j] |= (v[16 * j + b] | (v[16 * j + 4 + b] << 2) | (v[16 * j + 8 + b] << 4) | (v[16 * j + 12 + b] << 6))
                  << (8 * b);
      } else {
        const uint32_t spill = v[24 + b] | (v[28 + b] << 3);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const uint32_t byte = v[8 * j + b] | (v[8 * j + 4 + b] << 3) | (((spill >> (2 * j)) & 3u) << 6);
          w[j] |= byte << (8 * b);
        }
      }
    }
  }
  const uint32_t gp = (uint32_t)padded_groups;
#pragma unroll
  for (int j = 0; j < kWd; ++j)
    *reinterpret_cast<uint32_t*>(code_plane + (kBits == 2 ? code_word_offset2(r, (uint32_t)g, (uint32_t)j, gp)
                                                          : code_word_offset(r, (uint32_t)g, (uint32_t)j, gp))) = w[j];
  scale_plane[scale_byte_offset(r, (uint32_t)g, gp)] = real ? scales[r * lds + g] : (uint8_t)0;
}

template <int kBits>
__global__ __launch_bounds__(256) void unpack_kernel(PlaneView w, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t G = w.groups;
  if (idx >= w.n * G) return;
  const int64_t r = idx / G, g = idx % G;
  const uint32_t gp = ((uint32_t)G + 3u) & ~3u;
  uint32_t d[3] = {0u, 0u, 0u};
  uint32_t sel[8];
  if constexpr (kBits == 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      d[j] = *reinterpret_cast<const uint32_t*>(w.code + code_word_offset2(r, (uint32_t)g, (uint32_t)j, gp));
    unpack_selectors2(d[0], d[1], sel);
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      d[j] = *reinterpret_cast<const uint32_t*>(w.code + code_word_offset(r, (uint32_t)g, (uint32_t)j, gp));
    unpack_selectors(d[0], d[1], d[2], sel);
  }
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + r * G * kGroup + g * kGroup);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = sel[i];   // selector bytes are the codes in K order
  scales[r * G + g] = w.scale[scale_byte_offset(r, (uint32_t)g, gp)];
}

inline unsigned blocks_for(int64_t items) { return (unsigned)((items + 255) / 256); }

}  // namespace

hipError_t launch_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int64_t n,
                       int64_t k, uint8_t* code_plane, uint8_t* scale_plane, hipStream_t s, int bits) {
  const int64_t groups = k / kGroup;
  const int64_t padded = (groups + 3) / 4 * 4;
  const int64_t padded_rows = (n + 15) / 16 * 16;
  if (n == 0) return hipSuccess;
  if (bits == 2)
    hipLaunchKernelGGL(pack_kernel<2>, dim3(blocks_for(padded_rows * padded)), dim3(256), 0, s, codes, ldc, scales,
                       lds, n, groups, padded, padded_rows, code_plane, scale_plane);
  else
    hipLaunchKernelGGL(pack_kernel<3>, dim3(blocks_for(padded_rows * padded)), dim3(256), 0, s, codes, ldc, scales,
                       lds, n, groups, padded, padded_rows, code_plane, scale_plane);
  return hipGetLastError();
}

hipError_t launch_unpack(const PlaneView& w, uint8_t* codes, uint8_t* scales, hipStream_t s, int bits) {
  if (w.n == 0) return hipSuccess;
  if (bits == 2)
    hipLaunchKernelGGL(unpack_kernel<2>, dim3(blocks_for(w.n * w.groups)), dim3(256), 0, s, w, codes, scales);
  else
    hipLaunchKernelGGL(unpack_kernel<3>, dim3(blocks_for(w.n * w.groups)), dim3(256), 0, s, w, codes, scales);
  return hipGetLastError();
}

}  // namespace q3
