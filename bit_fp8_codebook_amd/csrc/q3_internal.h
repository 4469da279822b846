// Internal interface between the C ABI (q3_api.cpp) and the kernel launchers.
// Everything here is already validated by the caller; launchers only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

struct PlaneView {
  const uint8_t* code;    // code plane (tile-major, 192*Gp bytes per 16-row tile), 16-byte aligned
  const uint8_t* scale;   // scale plane (tile-major, 16*Gp bytes per tile), 4-byte aligned
  const uint8_t* cb;      // codebook [n][8], 8-byte aligned
  int64_t n;
  int32_t groups;         // k / 32
};

hipError_t launch_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int64_t n,
                       int64_t k, uint8_t* code_plane, uint8_t* scale_plane, hipStream_t s);
hipError_t launch_unpack(const PlaneView& w, uint8_t* codes, uint8_t* scales, hipStream_t s);

// VALU path, 1 <= m <= 8.
hipError_t launch_gemv(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t s);

// MFMA path, 1 <= m <= 64.
hipError_t launch_gemm_small_m(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                               int64_t ldy, hipStream_t s);

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids,
                           hipStream_t s);

struct ExpertView {
  PlaneView base;            // expert 0; n and groups are shared
  int64_t code_stride, scale_stride, cb_stride;   // bytes between experts
  int32_t num_experts;
};

hipError_t launch_grouped(const ExpertView& w, const uint16_t* x, int64_t ldx, int32_t x_by_slot,
                          const int32_t* ids, int32_t t, int32_t topk, float* y, int64_t ldy, hipStream_t s);

}  // namespace q3
