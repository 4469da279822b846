// Read-ceiling probes for the benchmark: what a launch that only streams a
// buffer from HBM achieves on this GPU, timed the same way as the packed-weight
// products (graph-replayed, back-to-back dependent launches over cold copies).
// The decode layer's premise (Hibana: Fast Agentic Inference on Unified-Memory
// Devices, "Model surgery": decoding one request is limited by memory
// bandwidth) makes this the achievable denominator next to the 8 TB/s peak.
//
// Measurement code only, not part of the q3 library.  Built by
// __graft_entry__.build() into libbench_ceiling.so beside bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The weight stream's load policy (non-temporal, work-group scope), so the
// probe and the products read HBM the same way.
constexpr int kPolicy = 3;

// Thread t of T reads 16-byte chunks t, t + T, t + 2T, ... (each wave
// instruction covers 1 KB contiguously), kUnroll of them in flight per loop
// trip.  Chunks past `bytes` read zero through the buffer resource.  The XOR
// of everything read is compared with a constant so the loads stay live; the
// store behind it practically never runs and stays inside sink[0..255].
template <int kUnroll>
__global__ __launch_bounds__(256) void read_kernel(const uint8_t* buf, uint32_t bytes, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0, (int)bytes, 0x00020000);
  const uint32_t T = gridDim.x * blockDim.x;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t chunks = (bytes + 15u) / 16u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t base = 0; base < chunks; base += kUnroll * T) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q)
      v[q] = __builtin_amdgcn_raw_buffer_load_b128(r, (base + q * T + gid) * 16u, 0, kPolicy);
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) acc ^= v[q];
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[gid & 255u] = x;
}

__global__ __launch_bounds__(256) void empty_kernel() {}

template <int U>
hipError_t launch(const void* buf, uint32_t bytes, int blocks, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel<U>, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(buf), bytes, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Stream `bytes` (1..1 GiB) of device memory `buf` once: `blocks` blocks of 256
// threads, `unroll` (1, 2, 4, 8 or 16) 16-byte loads in flight per thread and
// loop trip.  sink: device memory of 256 uint32 (practically never written).
// Returns a hipError_t value (0 on success); bad arguments give
// hipErrorInvalidValue before any launch.
__attribute__((visibility("default"))) int ceiling_read(const void* buf, int64_t bytes, int blocks, int unroll,
                                                        void* sink, void* stream) {
  if (!buf || !sink || bytes < 1 || bytes > (int64_t(1) << 30) || blocks < 1 || blocks > 65535)
    return hipErrorInvalidValue;
  // Every offset the kernel forms stays below 2^32: base + q*T + gid < chunks + unroll*T.
  const int64_t chunks = (bytes + 15) / 16, T = int64_t(blocks) * 256;
  if ((chunks + int64_t(unroll) * T) * 16 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* out = static_cast<uint32_t*>(sink);
  const uint32_t b = static_cast<uint32_t>(bytes);
  switch (unroll) {
    case 1: return launch<1>(buf, b, blocks, out, s);
    case 2: return launch<2>(buf, b, blocks, out, s);
    case 4: return launch<4>(buf, b, blocks, out, s);
    case 8: return launch<8>(buf, b, blocks, out, s);
    case 16: return launch<16>(buf, b, blocks, out, s);
    default: return hipErrorInvalidValue;
  }
}

// An empty kernel of `blocks` blocks: the cost of one dependent launch.
__attribute__((visibility("default"))) int ceiling_empty(int blocks, void* stream) {
  if (blocks < 1 || blocks > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError();
}

}  // extern "C"
