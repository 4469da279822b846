// Device-side building blocks shared by the q3 kernels (gfx950 only).
//
// Format (Hibana: Fast Agentic Inference on Unified-Memory Devices, "Model
// surgery" / "Three-bit weights"): a group of 32 weights is 32 three-bit
// indices into the row's 8-entry E4M3FN codebook plus one E8M0 scale.  The 96
// code bits of a group sit in three 32-bit words in a byte-lane order chosen so
// that a per-byte mask yields four indices in K order, ready to be used as
// v_perm_b32 byte selectors into the 8-byte codebook:
//   byte b of word j: bits 0..2 = c[8j+b], bits 3..5 = c[8j+4+b],
//                     bits 6..7 = bits 2j..2j+1 of (c[24+b] | c[28+b] << 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 32;

// Three code words of a group -> eight selector words; selector i holds the
// indices of weights 4i..4i+3 (one per byte, values 0..7).  17 VALU ops.
__device__ __forceinline__ void unpack_selectors(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t (&s)[8]) {
  const uint32_t m3 = 0x07070707u;
  s[0] = d0 & m3;
  s[1] = (d0 >> 3) & m3;
  s[2] = d1 & m3;
  s[3] = (d1 >> 3) & m3;
  s[4] = d2 & m3;
  s[5] = (d2 >> 3) & m3;
  // Bits 6..7 of every byte of the three words carry the last eight indices,
  // two bits per word; gather them into bits 0..5 of each byte.
  const uint32_t sp = ((d0 >> 6) & 0x03030303u) | ((d1 >> 4) & 0x0C0C0C0Cu) | ((d2 >> 2) & 0x30303030u);
  s[6] = sp & m3;
  s[7] = (sp >> 3) & m3;
}

// Codebook lookup of four indices at once: v_perm_b32 picks byte sel[b] of the
// 8-byte table {cb_hi:cb_lo} (entries 0..3 in cb_lo, 4..7 in cb_hi).
__device__ __forceinline__ uint32_t lookup4(uint32_t cb_lo, uint32_t cb_hi, uint32_t sel) {
  return __builtin_amdgcn_perm(cb_hi, cb_lo, sel);
}

// The E8M0 scale byte as an fp32 power of two 2^(s-127) (exact for 1..254).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __builtin_bit_cast(float, s << 23);
}

// Two E4M3FN bytes (low or high half of q) -> two bf16 values times the scale.
// Exact: an E4M3FN value has 4 significant bits and the power-of-two scale
// keeps it inside bf16's range for scale bytes 16..240.
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t q, float scale, bool high) {
  return high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, scale, false);
}

// Dequantise one group to 16 bf16 pairs in K order (pair p = weights 2p, 2p+1).
__device__ __forceinline__ void dequant_group_bf16(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t sbyte,
                                                   uint32_t cb_lo, uint32_t cb_hi, bf16x2 (&w)[16]) {
  uint32_t sel[8];
  unpack_selectors(d0, d1, d2, sel);
  const float sc = e8m0_to_f32(sbyte);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = lookup4(cb_lo, cb_hi, sel[i]);
    w[2 * i] = fp8x2_to_bf16x2(q, sc, false);
    w[2 * i + 1] = fp8x2_to_bf16x2(q, sc, true);
  }
}

// Two-bit draft-head groups (the head's 2-bit copy, "Two-bit draft head"):
// 32 codes in two words, byte b of word j holding code 16j+4q+b in bits
// 2q..2q+1, looked up in the row's 4-entry codebook (one word, entry j in
// byte j).  Selector 4j+q = (word j >> 2q) & 0x03 per byte: the codes of
// weights 16j+4q .. 16j+4q+3.  7 ALU ops per word.
__device__ __forceinline__ void unpack_selectors2(uint32_t d0, uint32_t d1, uint32_t (&s)[8]) {
  const uint32_t m2 = 0x03030303u;
  s[0] = d0 & m2;
  s[1] = (d0 >> 2) & m2;
  s[2] = (d0 >> 4) & m2;
  s[3] = (d0 >> 6) & m2;
  s[4] = d1 & m2;
  s[5] = (d1 >> 2) & m2;
  s[6] = (d1 >> 4) & m2;
  s[7] = (d1 >> 6) & m2;
}

__device__ __forceinline__ void dequant_group2_bf16(uint32_t d0, uint32_t d1, uint32_t sbyte, uint32_t cb4,
                                                    bf16x2 (&w)[16]) {
  uint32_t sel[8];
  unpack_selectors2(d0, d1, sel);
  const float sc = e8m0_to_f32(sbyte);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = __builtin_amdgcn_perm(0u, cb4, sel[i]);   // selector bytes 0..3 pick bytes of cb4
    w[2 * i] = fp8x2_to_bf16x2(q, sc, false);
    w[2 * i + 1] = fp8x2_to_bf16x2(q, sc, true);
  }
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Tile-major placement of the planes (rows in tiles of 16, a row's groups in
// steps of 16): the code-plane byte of word j of group g of row r and the
// scale-plane byte of the scale of (r, g), for gp padded groups per row.  A
// step holds q = min(16, gp - 16s)/4 quads of 4 groups; inside it, 16-byte
// piece 16*(q*j + kb) + i holds word j of quad kb of the tile's row i.
__device__ __forceinline__ uint32_t step_quads(uint32_t s, uint32_t gp) {
  const uint32_t rest = gp - 16u * s;
  return (rest < 16u ? rest : 16u) / 4u;
}
__device__ __forceinline__ int64_t code_word_offset(int64_t r, uint32_t g, uint32_t j, uint32_t gp) {
  const uint32_t i = (uint32_t)(r & 15), s = g >> 4, kb = (g >> 2) & 3u, t = g & 3u;
  const uint32_t q = step_quads(s, gp);
  return (r >> 4) * (int64_t)(192u * gp) + 3072u * s + 16u * (16u * (q * j + kb) + i) + 4u * t;
}
// The 2-bit head's planes: two words per group, so a tile is 128*Gp bytes and
// a full step 2048; the piece rule inside a step is the same.
__device__ __forceinline__ int64_t code_word_offset2(int64_t r, uint32_t g, uint32_t j, uint32_t gp) {
  const uint32_t i = (uint32_t)(r & 15), s = g >> 4, kb = (g >> 2) & 3u, t = g & 3u;
  const uint32_t q = step_quads(s, gp);
  return (r >> 4) * (int64_t)(128u * gp) + 2048u * s + 16u * (16u * (q * j + kb) + i) + 4u * t;
}
__device__ __forceinline__ int64_t scale_byte_offset(int64_t r, uint32_t g, uint32_t gp) {
  const uint32_t i = (uint32_t)(r & 15), s = g >> 4, kb = (g >> 2) & 3u, t = g & 3u;
  return (r >> 4) * (int64_t)(16u * gp) + 256u * s + 4u * (16u * kb + i) + t;
}

// Raw buffer resources: loads whose byte offset lies past num_records return
// zero, which the kernels use instead of branches around out-of-range rows,
// groups and tokens.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// An offset past every buffer: planes are kept below 2 GiB - 16 MiB, so kOob
// plus any in-kernel advance inside one tile stays out of range without
// wrapping.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
// Weight-stream loads: each packed weight byte is read once per launch, so the
// loads carry the non-temporal hint (nt) at work-group scope (sc0): measured on
// MI355X, this shortens a 4096 x 4096 decode launch from 5.3 to 4.7 us and the
// K = 8192 streams by 4-7%, against the default policy.
#ifndef Q3_STREAM_POLICY
#define Q3_STREAM_POLICY 3
#endif
__device__ __forceinline__ u32x4 bload128_stream(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, Q3_STREAM_POLICY);
}
__device__ __forceinline__ uint32_t bload32_stream(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, Q3_STREAM_POLICY);
}

}  // namespace q3
