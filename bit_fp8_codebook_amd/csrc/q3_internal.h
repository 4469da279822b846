// Internal interface between the C ABI (q3_api.cpp) and the kernel launchers.
// Everything here is already validated by the caller; launchers only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace q3 {

struct PlaneView {
  const uint8_t* code;    // code plane (tile-major, 192*Gp bytes per 16-row tile), 16-byte aligned
  const uint8_t* scale;   // scale plane (tile-major, 16*Gp bytes per tile), 4-byte aligned
  const uint8_t* cb;      // codebook [n][8], 8-byte aligned
  int64_t n;
  int32_t groups;         // k / 32
};

// bits = 3 (the 3.25-bit layer) or 2 (the two-bit draft head).
hipError_t launch_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int64_t n,
                       int64_t k, uint8_t* code_plane, uint8_t* scale_plane, hipStream_t s, int bits);
hipError_t launch_unpack(const PlaneView& w, uint8_t* codes, uint8_t* scales, hipStream_t s, int bits);

// Quantizer: per-group scale and nearest code under the row's codebook.
hipError_t launch_quantize(const float* w, int64_t ldw, const uint8_t* cb, int64_t n, int64_t k, uint8_t* codes,
                           int64_t ldc, uint8_t* scales, int64_t lds, hipStream_t s);

// Split-K products on matrices with few row tiles (q3_splitk.hip): whether the
// kernel takes (n, groups, m) on the matrix cores (dot false, m <= 16) or the
// vector ALUs (dot true, m <= 8), and the launch.
bool splitk_applies(int64_t n, int groups, int64_t m, bool dot);
hipError_t launch_splitk(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                         bool dot, hipStream_t s);

// Codebook fitting: the 8 E4M3FN entries of each row's codebook from its fp32
// weights (q3_fit.hip), k <= 2^18.
hipError_t launch_fit_codebook(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* cb, hipStream_t s);

// VALU path, 1 <= m <= 8.
hipError_t launch_gemv(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t s);

// MFMA path, 1 <= m <= 64.  ws (nullable, 16-byte aligned) of at least
// gemm_small_m_workspace_bytes(n, k, m) bytes lets streamed activations split
// K over blocks; without it every block covers the whole K.
int64_t gemm_small_m_workspace_bytes(int64_t n, int64_t k, int64_t m);
hipError_t launch_gemm_small_m(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                               int64_t ldy, void* ws, int64_t ws_bytes, hipStream_t s);

// Two-bit draft head: scores of every row for 1 <= m <= 16 queries (matrix cores).
hipError_t launch_head2_scores(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                               hipStream_t s);

// Shortlist: per query the `size` largest of n fp32 scores (ties to the lower
// row), in two launches through `cand` (m * kShortlistChunks * kShortlistMax
// (score, row) pairs).  With ids == nullptr only the first pass runs (the
// rescoring launch then merges the chunk lists itself).
constexpr int kShortlistMax = 16;
constexpr int kShortlistChunks = 64;
hipError_t launch_shortlist(const float* scores, int64_t m, int64_t n, int64_t ld, int32_t size, void* cand,
                            int32_t* ids, float* vals, hipStream_t s);

// MXFP8 rows gathered by ids: y[i][j] = x[i] . w8[ids[i][j]]; best[i] = the
// listed row with the largest y (ties to the lower row).  With cand set (the
// shortlist's first-pass lists), the list is merged first and written to ids.
struct Mxfp8View {
  const uint8_t* e8;   // [n][lde] E4M3FN
  int64_t lde;
  const uint8_t* s8;   // [n][lds] E8M0, one per 32 elements
  int64_t lds;
  int64_t n, k;
};
hipError_t launch_rescore(const Mxfp8View& h, const uint16_t* x, int64_t m, int64_t ldx, const void* cand,
                          int32_t* ids, int32_t size, float* y, int32_t* best, hipStream_t s);

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids,
                           hipStream_t s);
// Expert-budget routing: the `budget` experts of largest routing mass, then each
// token's top-k inside them; experts (nullable) gets the kept set ascending.
hipError_t launch_moe_budget_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t budget,
                                  int32_t* ids, int32_t* experts, hipStream_t s);

struct ExpertView {
  PlaneView base;            // expert 0; n and groups are shared
  int64_t code_stride, scale_stride, cb_stride;   // bytes between experts
  int32_t num_experts;
};

hipError_t launch_grouped(const ExpertView& w, const uint16_t* x, int64_t ldx, int32_t x_by_slot,
                          const int32_t* ids, int32_t t, int32_t topk, float* y, int64_t ldy, hipStream_t s);

// Routing-weight combine: out[i][r] = sum_j p[i][j] * part[i*topk + j][r], p[i]
// the softmax of token i's routed (in-range) logits; slots in slot order.
hipError_t launch_moe_combine(const float* part, int64_t ldp, const int32_t* ids, int32_t t, int32_t topk,
                              int32_t num_experts, const float* logits, int64_t ld_logits, int64_t n, float* out,
                              int64_t ldo, hipStream_t s);

// Library-owned scratch (q3_noalloc.hip): kScratchBytes of device memory per
// GPU; scratch_address gives this device's copy (looked up once per device).
constexpr int64_t kScratchBytes = int64_t(4) << 20;
hipError_t scratch_address(void** out);

// Fused expert MLP of a verify round, three launches: gate/up with SwiGLU into
// h (bf16 [2*pairs][I], high and low term per pair), down into part (fp32
// [pairs][ldp]), then the combine.
hipError_t launch_moe_mlp(const ExpertView& gu, const ExpertView& dn, const uint16_t* x, int64_t ldx,
                          const int32_t* ids, int32_t t, int32_t topk, const float* logits, int64_t ld_logits,
                          uint16_t* h, float* part, int64_t ldp, float* out, int64_t ldo, hipStream_t s);

// Dynamic LDS above 64 KB must be allowed per kernel on each device.  One
// LdsAllowance per kernel (a zero-initialised static) remembers, per device,
// the largest size already allowed, so later launches cost one atomic load.
constexpr int kMaxDevices = 64;
struct LdsAllowance {
  std::atomic<size_t> bytes[kMaxDevices];
};
hipError_t allow_dynamic_lds(const void* kernel, size_t bytes, LdsAllowance& seen);

}  // namespace q3
