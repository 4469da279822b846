// Packing and unpacking of the 3.25-bit format (Hibana: Fast Agentic Inference
// on Unified-Memory Devices, "Model surgery" / "Three-bit weights": a 3-bit
// index per weight, one 8-bit scale per group of 32).  One-time work, not on the
// decode path; written for clarity, one thread per group.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t ldc,
                                                         int64_t n, int64_t groups, int64_t padded_groups,
                                                         uint8_t* __restrict__ plane, int64_t pitch) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * padded_groups) return;
  const int64_t r = idx / padded_groups, g = idx % padded_groups;
  uint32_t w[3] = {0u, 0u, 0u};
  if (g < groups) {
    const uint8_t* c = codes + r * ldc + (int64_t)kGroup * g;
    uint32_t v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = c[i] & 7u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t spill = v[24 + b] | (v[28 + b] << 3);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const uint32_t byte = v[8 * j + b] | (v[8 * j + 4 + b] << 3) | (((spill >> (2 * j)) & 3u) << 6);
        w[j] |= byte << (8 * b);
      }
    }
  }
  uint8_t* row = plane + r * pitch;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    *reinterpret_cast<uint32_t*>(row + word_offset((uint32_t)g, (uint32_t)j, (uint32_t)padded_groups)) = w[j];
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ scales, int64_t lds,
                                                          int64_t n, int64_t groups, int64_t row_bytes,
                                                          uint8_t* __restrict__ plane, int64_t pitch) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * row_bytes) return;
  const int64_t r = idx / row_bytes, g = idx % row_bytes;
  plane[r * pitch + g] = g < groups ? scales[r * lds + g] : (uint8_t)0;
}

__global__ __launch_bounds__(256) void unpack_kernel(PlaneView w, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t G = w.groups;
  if (idx >= w.n * G) return;
  const int64_t r = idx / G, g = idx % G;
  const uint8_t* row = w.code + r * w.code_pitch;
  const uint32_t gp = ((uint32_t)G + 3u) & ~3u;
  uint32_t d[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) d[j] = *reinterpret_cast<const uint32_t*>(row + word_offset((uint32_t)g, j, gp));
  uint32_t sel[8];
  unpack_selectors(d[0], d[1], d[2], sel);
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + r * G * kGroup + g * kGroup);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = sel[i];   // selector bytes are the codes in K order
  scales[r * G + g] = w.scale[r * w.scale_pitch + g];
}

inline unsigned blocks_for(int64_t items) { return (unsigned)((items + 255) / 256); }

}  // namespace

hipError_t launch_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int64_t n,
                       int64_t k, uint8_t* code_plane, int64_t code_pitch, uint8_t* scale_plane,
                       int64_t scale_pitch, hipStream_t s) {
  const int64_t groups = k / kGroup;
  const int64_t chunks = (k + 127) / 128;
  const int64_t padded = chunks * 4;
  const int64_t scale_row = (padded + 15) / 16 * 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(n * padded)), dim3(256), 0, s, codes, ldc, n, groups,
                     padded, code_plane, code_pitch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(blocks_for(n * scale_row)), dim3(256), 0, s, scales, lds, n,
                     groups, scale_row, scale_plane, scale_pitch);
  return hipGetLastError();
}

hipError_t launch_unpack(const PlaneView& w, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (w.n == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks_for(w.n * w.groups)), dim3(256), 0, s, w, codes, scales);
  return hipGetLastError();
}

}  // namespace q3
