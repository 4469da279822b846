// C ABI of the q3 library: host-side validation, then one launch on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/q3.h"
#include "q3_internal.h"

namespace {

constexpr int64_t kGroup = 32;
constexpr int64_t kMaxPlaneBytes = (int64_t(1) << 31) - (int64_t(1) << 24);   // per plane, and for x

int64_t padded_groups(int64_t k) { return (k / kGroup + 3) / 4 * 4; }
int64_t tiles_of(int64_t n) { return (n + 15) / 16; }
int64_t code_plane_bytes(int64_t n, int64_t k) { return tiles_of(n) * 192 * padded_groups(k); }
int64_t scale_plane_bytes(int64_t n, int64_t k) { return tiles_of(n) * 16 * padded_groups(k); }
int64_t code_plane_bytes2(int64_t n, int64_t k) { return tiles_of(n) * 128 * padded_groups(k); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

q3_status check_shape(int64_t n, int64_t k) {
  if (n < 0) return Q3_ERR_INVALID_ARG;
  if (k <= 0 || k % kGroup != 0 || k > (int64_t(1) << 30)) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (n > (int64_t(1) << 31)) return Q3_ERR_UNSUPPORTED_SHAPE;
  return Q3_OK;
}

// Packed planes of one matrix: pointers present, aligned, addressable.
q3_status check_planes(int64_t n, int64_t k, const void* code, const void* scale, const void* cb) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (n > 0 && (!code || !scale || !cb)) return Q3_ERR_INVALID_ARG;
  if (!aligned(code, 16) || !aligned(scale, 4) || !aligned(cb, 8)) return Q3_ERR_MISALIGNED;
  // The kernels address each plane through a 32-bit buffer resource.
  if (code_plane_bytes(n, k) > kMaxPlaneBytes || n * 8 > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  return Q3_OK;
}

// The two-bit draft head's planes: 4-byte codebook rows.
q3_status check_planes2(int64_t n, int64_t k, const void* code, const void* scale, const void* cb) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (n > 0 && (!code || !scale || !cb)) return Q3_ERR_INVALID_ARG;
  if (!aligned(code, 16) || !aligned(scale, 4) || !aligned(cb, 4)) return Q3_ERR_MISALIGNED;
  if (code_plane_bytes2(n, k) > kMaxPlaneBytes || n * 4 > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  return Q3_OK;
}

q3_status check_mxfp8(const q3_mxfp8_matrix* h) {
  if (!h) return Q3_ERR_INVALID_ARG;
  q3_status st = check_shape(h->n, h->k);
  if (st != Q3_OK) return st;
  if (h->n < 1 || !h->elements || !h->scales) return Q3_ERR_INVALID_ARG;
  if (h->ld_elements < h->k || h->ld_scales < h->k / kGroup) return Q3_ERR_INVALID_ARG;
  if (h->ld_elements % 16 || !aligned(h->elements, 16)) return Q3_ERR_MISALIGNED;
  if (h->n * h->ld_elements > kMaxPlaneBytes || h->n * h->ld_scales > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  return Q3_OK;
}

constexpr int64_t kShortlistPairBytes = 8;   // (score, row)
int64_t shortlist_ws(int64_t m) { return m * q3::kShortlistChunks * q3::kShortlistMax * kShortlistPairBytes; }
int64_t align8(int64_t b) { return (b + 7) / 8 * 8; }

q3_status check_matrix(const q3_matrix* w) {
  if (!w) return Q3_ERR_INVALID_ARG;
  return check_planes(w->n, w->k, w->code_plane, w->scale_plane, w->codebook);
}

q3_status check_tokens(int64_t k, int64_t n, const uint16_t* x, int64_t m, int64_t ldx, const float* y,
                       int64_t ldy, int64_t m_max) {
  if (m < 1 || m > m_max) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!x || (!y && n > 0)) return Q3_ERR_INVALID_ARG;
  if (ldx < k || ldy < n) return Q3_ERR_INVALID_ARG;
  if (ldx % 8 || !aligned(x, 16) || !aligned(y, 4)) return Q3_ERR_MISALIGNED;
  if ((m - 1) * ldx * 2 + k * 2 > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  return Q3_OK;
}

// gfx950 check, once per device (the only global state of the library).
std::atomic<int> g_device_ok[64];

q3_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Q3_ERR_HIP;
  if (dev < 0 || dev >= 64) return Q3_ERR_UNSUPPORTED_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q3_ERR_HIP;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? Q3_OK : Q3_ERR_UNSUPPORTED_DEVICE;
}

q3_status from_hip(hipError_t e) { return e == hipSuccess ? Q3_OK : Q3_ERR_HIP; }

q3::PlaneView view_of(const q3_matrix* w) {
  q3::PlaneView v;
  v.code = static_cast<const uint8_t*>(w->code_plane);
  v.scale = static_cast<const uint8_t*>(w->scale_plane);
  v.cb = static_cast<const uint8_t*>(w->codebook);
  v.n = w->n;
  v.groups = static_cast<int32_t>(w->k / kGroup);
  return v;
}

}  // namespace

extern "C" {

Q3_API const char* q3_status_string(q3_status s) {
  switch (s) {
    case Q3_OK: return "ok";
    case Q3_ERR_INVALID_ARG: return "invalid argument";
    case Q3_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case Q3_ERR_MISALIGNED: return "misaligned pointer or stride";
    case Q3_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case Q3_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

Q3_API q3_status q3_layout(int64_t n, int64_t k, q3_layout_info* out) {
  if (!out) return Q3_ERR_INVALID_ARG;
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  out->n = n;
  out->k = k;
  out->groups = k / kGroup;
  out->padded_groups = padded_groups(k);
  out->tiles = tiles_of(n);
  out->code_tile_bytes = 192 * out->padded_groups;
  out->scale_tile_bytes = 16 * out->padded_groups;
  out->code_plane_bytes = code_plane_bytes(n, k);
  out->scale_plane_bytes = scale_plane_bytes(n, k);
  out->codebook_bytes = 8 * n;
  out->payload_bytes = n * (k / kGroup) * 13;
  return Q3_OK;
}

Q3_API q3_status q3_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scale_bytes, int64_t lds, int64_t n,
                         int64_t k, void* code_plane, void* scale_plane, void* stream) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (n > 0 && (!codes || !scale_bytes || !code_plane || !scale_plane)) return Q3_ERR_INVALID_ARG;
  if (ldc < k || lds < k / kGroup) return Q3_ERR_INVALID_ARG;
  if (!aligned(code_plane, 16) || !aligned(scale_plane, 4)) return Q3_ERR_MISALIGNED;
  if (code_plane_bytes(n, k) > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_pack(codes, ldc, scale_bytes, lds, n, k, static_cast<uint8_t*>(code_plane),
                                  static_cast<uint8_t*>(scale_plane), static_cast<hipStream_t>(stream), 3));
}

Q3_API q3_status q3_unpack(const q3_matrix* w, uint8_t* codes_out, uint8_t* scale_out, void* stream) {
  q3_status st = check_matrix(w);
  if (st != Q3_OK) return st;
  if (w->n > 0 && (!codes_out || !scale_out)) return Q3_ERR_INVALID_ARG;
  if (!aligned(codes_out, 4)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_unpack(view_of(w), codes_out, scale_out, static_cast<hipStream_t>(stream), 3));
}

Q3_API q3_status q3_quantize(const float* w, int64_t ldw, const uint8_t* codebook, int64_t n, int64_t k,
                             uint8_t* codes, int64_t ldc, uint8_t* scale_bytes, int64_t lds, void* stream) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (n > 0 && (!w || !codebook || !codes || !scale_bytes)) return Q3_ERR_INVALID_ARG;
  if (ldw < k || ldc < k || lds < k / kGroup) return Q3_ERR_INVALID_ARG;
  if (!aligned(w, 16) || ldw % 4 || !aligned(codebook, 8) || !aligned(codes, 8) || ldc % 8) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_quantize(w, ldw, codebook, n, k, codes, ldc, scale_bytes, lds,
                                      static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_fit_codebook(const float* w, int64_t ldw, int64_t n, int64_t k, uint8_t* codebook,
                                 void* stream) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (k > (int64_t(1) << 18) || n > 0x7FFFFFFF) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (n > 0 && (!w || !codebook)) return Q3_ERR_INVALID_ARG;
  if (ldw < k) return Q3_ERR_INVALID_ARG;
  if (!aligned(w, 16) || ldw % 4 || !aligned(codebook, 8)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_fit_codebook(w, ldw, n, k, codebook, static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_gemv(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                         void* stream) {
  q3_status st = check_matrix(w);
  if (st != Q3_OK) return st;
  if ((st = check_tokens(w->k, w->n, x, m, ldx, y, ldy, 8)) != Q3_OK) return st;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_gemv(view_of(w), x, m, ldx, y, ldy, static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_gemm_small_m(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                                 int64_t ldy, void* stream) {
  q3_status st = check_matrix(w);
  if (st != Q3_OK) return st;
  if ((st = check_tokens(w->k, w->n, x, m, ldx, y, ldy, 64)) != Q3_OK) return st;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(
      q3::launch_gemm_small_m(view_of(w), x, m, ldx, y, ldy, nullptr, 0, static_cast<hipStream_t>(stream)));
}

Q3_API int64_t q3_gemm_small_m_workspace_bytes(int64_t n, int64_t k, int64_t m) {
  if (n < 1 || k < 32 || k % 32 || m < 1 || m > 64) return 0;
  return q3::gemm_small_m_workspace_bytes(n, k, m);
}

Q3_API q3_status q3_gemm_small_m_ws(const q3_matrix* w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                                    int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream) {
  q3_status st = check_matrix(w);
  if (st != Q3_OK) return st;
  if ((st = check_tokens(w->k, w->n, x, m, ldx, y, ldy, 64)) != Q3_OK) return st;
  if (workspace && !aligned(workspace, 16)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_gemm_small_m(view_of(w), x, m, ldx, y, ldy, workspace, workspace ? workspace_bytes : 0,
                                          static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_moe_topk(const float* logits, int32_t t, int32_t num_experts, int32_t topk,
                             int32_t* topk_ids, void* stream) {
  if (!logits || !topk_ids) return Q3_ERR_INVALID_ARG;
  if (t < 1 || num_experts < 1 || num_experts > 1024 || topk < 1 || topk > num_experts)
    return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4)) return Q3_ERR_MISALIGNED;
  q3_status st = check_device();
  if (st != Q3_OK) return st;
  return from_hip(q3::launch_moe_topk(logits, t, num_experts, topk, topk_ids, static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_moe_budget_topk(const float* logits, int32_t t, int32_t num_experts, int32_t topk,
                                    int32_t budget, int32_t* topk_ids, int32_t* experts, void* stream) {
  if (!logits || !topk_ids) return Q3_ERR_INVALID_ARG;
  if (t < 1 || t > 1024 || num_experts < 1 || num_experts > 1024 || topk < 1 || budget < topk ||
      budget > num_experts)
    return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(experts, 4)) return Q3_ERR_MISALIGNED;
  q3_status st = check_device();
  if (st != Q3_OK) return st;
  return from_hip(q3::launch_moe_budget_topk(logits, t, num_experts, topk, budget, topk_ids, experts,
                                             static_cast<hipStream_t>(stream)));
}

namespace {

q3_status check_stack(const q3_expert_stack* w) {
  if (!w) return Q3_ERR_INVALID_ARG;
  if (w->num_experts < 1 || w->num_experts > 65535) return Q3_ERR_UNSUPPORTED_SHAPE;
  q3_status st = check_planes(w->n, w->k, w->code_plane, w->scale_plane, w->codebook);
  if (st != Q3_OK) return st;
  if (w->code_expert_stride < code_plane_bytes(w->n, w->k) || w->scale_expert_stride < scale_plane_bytes(w->n, w->k) ||
      w->codebook_expert_stride < 8 * w->n)
    return Q3_ERR_INVALID_ARG;
  if (w->code_expert_stride % 16 || w->scale_expert_stride % 4 || w->codebook_expert_stride % 8)
    return Q3_ERR_MISALIGNED;
  return Q3_OK;
}

q3::ExpertView view_of(const q3_expert_stack* w) {
  q3::ExpertView v;
  v.base.code = static_cast<const uint8_t*>(w->code_plane);
  v.base.scale = static_cast<const uint8_t*>(w->scale_plane);
  v.base.cb = static_cast<const uint8_t*>(w->codebook);
  v.base.n = w->n;
  v.base.groups = static_cast<int32_t>(w->k / kGroup);
  v.code_stride = w->code_expert_stride;
  v.scale_stride = w->scale_expert_stride;
  v.cb_stride = w->codebook_expert_stride;
  v.num_experts = static_cast<int32_t>(w->num_experts);
  return v;
}

// Fused MLP workspace: h (bf16 [2*pairs][I]) and part (fp32 [pairs][ldp]),
// each 256-byte aligned.
int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }
int64_t mlp_ldp(int64_t n_dn) { return (n_dn + 3) / 4 * 4; }
int64_t mlp_h_bytes(int64_t pairs, int64_t inter) { return align256(2 * pairs * inter * 2); }
int64_t mlp_part_bytes(int64_t pairs, int64_t n_dn) { return align256(pairs * mlp_ldp(n_dn) * 4); }

}  // namespace

Q3_API q3_status q3_grouped_expert_gemv(const q3_expert_stack* w, const uint16_t* x, int64_t ldx,
                                        int32_t x_by_slot, const int32_t* topk_ids, int32_t t, int32_t topk,
                                        float* y, int64_t ldy, void* stream) {
  q3_status st = check_stack(w);
  if (st != Q3_OK) return st;
  if (x_by_slot != 0 && x_by_slot != 1) return Q3_ERR_INVALID_ARG;
  if (!x || !topk_ids || !y) return Q3_ERR_INVALID_ARG;
  if (t < 1 || topk < 1 || int64_t(t) * topk > 64) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (ldx < w->k || ldy < w->n) return Q3_ERR_INVALID_ARG;
  if (ldx % 8 || !aligned(x, 16) || !aligned(y, 4) || !aligned(topk_ids, 4)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_grouped(view_of(w), x, ldx, x_by_slot, topk_ids, t, topk, y, ldy,
                                     static_cast<hipStream_t>(stream)));
}

Q3_API int64_t q3_moe_mlp_workspace_bytes(int64_t n_gu, int64_t n_dn, int32_t t, int32_t topk) {
  if (n_gu < 32 || n_gu % 64 || n_dn < 1 || t < 1 || topk < 1 || int64_t(t) * topk > 64) return 0;
  const int64_t pairs = int64_t(t) * topk;
  return mlp_h_bytes(pairs, n_gu / 2) + mlp_part_bytes(pairs, n_dn);
}

Q3_API q3_status q3_moe_mlp(const q3_expert_stack* gate_up, const q3_expert_stack* down, const uint16_t* x,
                            int64_t ldx, const int32_t* topk_ids, int32_t t, int32_t topk, const float* logits,
                            int64_t ld_logits, void* workspace, int64_t workspace_bytes, float* out, int64_t ldo,
                            void* stream) {
  q3_status st = check_stack(gate_up);
  if (st != Q3_OK) return st;
  if ((st = check_stack(down)) != Q3_OK) return st;
  if (gate_up->num_experts != down->num_experts) return Q3_ERR_INVALID_ARG;
  if (gate_up->n % 64 || down->k != gate_up->n / 2) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!x || !topk_ids || !logits || !workspace || !out) return Q3_ERR_INVALID_ARG;
  if (t < 1 || topk < 1 || int64_t(t) * topk > 64) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (ldx < gate_up->k || ldo < down->n || ld_logits < gate_up->num_experts) return Q3_ERR_INVALID_ARG;
  if (workspace_bytes < q3_moe_mlp_workspace_bytes(gate_up->n, down->n, t, topk)) return Q3_ERR_INVALID_ARG;
  if (ldx % 8 || !aligned(x, 16) || !aligned(out, 4) || !aligned(topk_ids, 4) || !aligned(logits, 4) ||
      !aligned(workspace, 256))
    return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  const int64_t pairs = int64_t(t) * topk;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + mlp_h_bytes(pairs, gate_up->n / 2));
  return from_hip(q3::launch_moe_mlp(view_of(gate_up), view_of(down), x, ldx, topk_ids, t, topk, logits, ld_logits,
                                     h, part, mlp_ldp(down->n), out, ldo, static_cast<hipStream_t>(stream)));
}

Q3_API int64_t q3_moe_mlp_noalloc_max_bytes(void) { return q3::kScratchBytes; }

Q3_API q3_status q3_moe_mlp_noalloc(const q3_expert_stack* gate_up, const q3_expert_stack* down, const uint16_t* x,
                                    int64_t ldx, const int32_t* topk_ids, int32_t t, int32_t topk,
                                    const float* logits, int64_t ld_logits, float* out, int64_t ldo, void* stream) {
  q3_status st = check_stack(gate_up);
  if (st != Q3_OK) return st;
  if ((st = check_stack(down)) != Q3_OK) return st;
  if (gate_up->num_experts != down->num_experts) return Q3_ERR_INVALID_ARG;
  if (gate_up->n % 64 || down->k != gate_up->n / 2) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!x || !topk_ids || !logits || !out) return Q3_ERR_INVALID_ARG;
  if (t < 1 || topk < 1 || int64_t(t) * topk > 64) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (ldx < gate_up->k || ldo < down->n || ld_logits < gate_up->num_experts) return Q3_ERR_INVALID_ARG;
  if (q3_moe_mlp_workspace_bytes(gate_up->n, down->n, t, topk) > q3::kScratchBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (ldx % 8 || !aligned(x, 16) || !aligned(out, 4) || !aligned(topk_ids, 4) || !aligned(logits, 4))
    return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  void* scratch = nullptr;
  if (q3::scratch_address(&scratch) != hipSuccess) return Q3_ERR_HIP;
  const int64_t pairs = int64_t(t) * topk;
  uint8_t* ws = static_cast<uint8_t*>(scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + mlp_h_bytes(pairs, gate_up->n / 2));
  return from_hip(q3::launch_moe_mlp(view_of(gate_up), view_of(down), x, ldx, topk_ids, t, topk, logits, ld_logits,
                                     h, part, mlp_ldp(down->n), out, ldo, static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_layout2(int64_t n, int64_t k, q3_layout_info* out) {
  if (!out) return Q3_ERR_INVALID_ARG;
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  out->n = n;
  out->k = k;
  out->groups = k / kGroup;
  out->padded_groups = padded_groups(k);
  out->tiles = tiles_of(n);
  out->code_tile_bytes = 128 * out->padded_groups;
  out->scale_tile_bytes = 16 * out->padded_groups;
  out->code_plane_bytes = code_plane_bytes2(n, k);
  out->scale_plane_bytes = scale_plane_bytes(n, k);
  out->codebook_bytes = 4 * n;
  out->payload_bytes = n * (k / kGroup) * 9;
  return Q3_OK;
}

Q3_API q3_status q3_pack2(const uint8_t* codes, int64_t ldc, const uint8_t* scale_bytes, int64_t lds, int64_t n,
                          int64_t k, void* code_plane, void* scale_plane, void* stream) {
  q3_status st = check_shape(n, k);
  if (st != Q3_OK) return st;
  if (n > 0 && (!codes || !scale_bytes || !code_plane || !scale_plane)) return Q3_ERR_INVALID_ARG;
  if (ldc < k || lds < k / kGroup) return Q3_ERR_INVALID_ARG;
  if (!aligned(code_plane, 16) || !aligned(scale_plane, 4)) return Q3_ERR_MISALIGNED;
  if (code_plane_bytes2(n, k) > kMaxPlaneBytes) return Q3_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_pack(codes, ldc, scale_bytes, lds, n, k, static_cast<uint8_t*>(code_plane),
                                  static_cast<uint8_t*>(scale_plane), static_cast<hipStream_t>(stream), 2));
}

Q3_API q3_status q3_unpack2(const q3_matrix* w, uint8_t* codes_out, uint8_t* scale_out, void* stream) {
  if (!w) return Q3_ERR_INVALID_ARG;
  q3_status st = check_planes2(w->n, w->k, w->code_plane, w->scale_plane, w->codebook);
  if (st != Q3_OK) return st;
  if (w->n > 0 && (!codes_out || !scale_out)) return Q3_ERR_INVALID_ARG;
  if (!aligned(codes_out, 4)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_unpack(view_of(w), codes_out, scale_out, static_cast<hipStream_t>(stream), 2));
}

Q3_API q3_status q3_head2_scores(const q3_matrix* w2, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                                 int64_t ldy, void* stream) {
  if (!w2) return Q3_ERR_INVALID_ARG;
  q3_status st = check_planes2(w2->n, w2->k, w2->code_plane, w2->scale_plane, w2->codebook);
  if (st != Q3_OK) return st;
  if ((st = check_tokens(w2->k, w2->n, x, m, ldx, y, ldy, 16)) != Q3_OK) return st;
  if ((st = check_device()) != Q3_OK) return st;
  return from_hip(q3::launch_head2_scores(view_of(w2), x, m, ldx, y, ldy, static_cast<hipStream_t>(stream)));
}

Q3_API int64_t q3_shortlist_workspace_bytes(int64_t m) { return m < 1 ? 0 : shortlist_ws(m); }

Q3_API q3_status q3_shortlist(const float* scores, int64_t m, int64_t n, int64_t ld, int32_t size, void* workspace,
                              int64_t workspace_bytes, int32_t* ids, float* vals, void* stream) {
  if (!scores || !workspace || !ids) return Q3_ERR_INVALID_ARG;
  if (m < 1 || m > 65535 || n < 1 || n > 0x7FFFFFFF || size < 1 || size > q3::kShortlistMax || size > n)
    return Q3_ERR_UNSUPPORTED_SHAPE;
  if (ld < n) return Q3_ERR_INVALID_ARG;
  if (workspace_bytes < shortlist_ws(m)) return Q3_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(workspace, 8) || !aligned(ids, 4) || !aligned(vals, 4)) return Q3_ERR_MISALIGNED;
  q3_status st = check_device();
  if (st != Q3_OK) return st;
  return from_hip(q3::launch_shortlist(scores, m, n, ld, size, workspace, ids, vals, static_cast<hipStream_t>(stream)));
}

Q3_API q3_status q3_rescore_fp8(const q3_mxfp8_matrix* w8, const uint16_t* x, int64_t m, int64_t ldx,
                                const int32_t* ids, int32_t size, float* y, int32_t* best, void* stream) {
  q3_status st = check_mxfp8(w8);
  if (st != Q3_OK) return st;
  if (m < 1 || m > 65535 || size < 1 || size > q3::kShortlistMax) return Q3_ERR_UNSUPPORTED_SHAPE;
  if (!x || !ids || !y || !best) return Q3_ERR_INVALID_ARG;
  if (ldx < w8->k) return Q3_ERR_INVALID_ARG;
  if (ldx % 8 || !aligned(x, 16) || !aligned(ids, 4) || !aligned(y, 4) || !aligned(best, 4)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  q3::Mxfp8View h{static_cast<const uint8_t*>(w8->elements), w8->ld_elements, static_cast<const uint8_t*>(w8->scales),
                  w8->ld_scales, w8->n, w8->k};
  return from_hip(q3::launch_rescore(h, x, m, ldx, nullptr, const_cast<int32_t*>(ids), size, y, best,
                                     static_cast<hipStream_t>(stream)));
}

Q3_API int64_t q3_draft_head_workspace_bytes(int64_t m, int64_t n) {
  return m < 1 || n < 1 ? 0 : align8(m * n * 4) + shortlist_ws(m);
}

Q3_API q3_status q3_draft_head(const q3_matrix* w2, const q3_mxfp8_matrix* w8, const uint16_t* x, int64_t m,
                               int64_t ldx, int32_t size, void* workspace, int64_t workspace_bytes, int32_t* ids,
                               float* y8, int32_t* best, void* stream) {
  if (!w2) return Q3_ERR_INVALID_ARG;
  q3_status st = check_planes2(w2->n, w2->k, w2->code_plane, w2->scale_plane, w2->codebook);
  if (st != Q3_OK) return st;
  if ((st = check_mxfp8(w8)) != Q3_OK) return st;
  if (w8->n != w2->n || w8->k != w2->k) return Q3_ERR_INVALID_ARG;
  if (!workspace || !ids || !y8 || !best) return Q3_ERR_INVALID_ARG;
  if (size < 1 || size > q3::kShortlistMax || size > w2->n || w2->n > 0x7FFFFFFF) return Q3_ERR_UNSUPPORTED_SHAPE;
  float* scores = static_cast<float*>(workspace);
  if ((st = check_tokens(w2->k, w2->n, x, m, ldx, scores, w2->n, 16)) != Q3_OK) return st;
  if (workspace_bytes < q3_draft_head_workspace_bytes(m, w2->n)) return Q3_ERR_INVALID_ARG;
  if (!aligned(workspace, 8) || !aligned(ids, 4) || !aligned(y8, 4) || !aligned(best, 4)) return Q3_ERR_MISALIGNED;
  if ((st = check_device()) != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = q3::launch_head2_scores(view_of(w2), x, m, ldx, scores, w2->n, s);
  void* cand = static_cast<uint8_t*>(workspace) + align8(m * w2->n * 4);
  if (e == hipSuccess) e = q3::launch_shortlist(scores, m, w2->n, w2->n, size, cand, nullptr, nullptr, s);
  q3::Mxfp8View h{static_cast<const uint8_t*>(w8->elements), w8->ld_elements, static_cast<const uint8_t*>(w8->scales),
                  w8->ld_scales, w8->n, w8->k};
  if (e == hipSuccess) e = q3::launch_rescore(h, x, m, ldx, cand, ids, size, y8, best, s);
  return from_hip(e);
}

}  // extern "C"
