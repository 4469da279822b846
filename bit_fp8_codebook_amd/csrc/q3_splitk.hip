// Decode / verify products on matrices with few 16-row tiles (up to 16 tokens):
// each tile's K is dealt out to many waves so that a launch has all of its
// packed weights in flight at once.
//
// What it computes is the layer of q3_linear.hip (Hibana: Fast Agentic
// Inference on Unified-Memory Devices, "Model surgery" / "Three-bit weights"):
// y[m][n] = sum_k x[m][k] * w[n][k], w = E4M3FN(codebook[n][code]) *
// 2^(scale - 127), products exact, fp32 accumulation.
//
// Why a separate kernel: decoding one token is bound by memory bandwidth, and a
// 4096 x 4096 layer is only 6.8 MB, a couple of microseconds at HBM speed, so
// the launch is dominated by latency.  Measured on MI355X (graph-replayed
// dependent launches over cold copies): a plain read of 6.8 MB takes 2.45 us
// per launch when every byte is requested at once; a launch that stages the
// activations in LDS behind a block barrier, keeps one 512-k step in flight
// per wave and sums K splits through two more barriers took 4.54 us.
//
// Layout of the work: one block per row tile.  The tile's K is cut into
// half-steps -- groups 2h, 2h+1 of every quad of a 512-k step, so lane
// (row i, quad kb) holds two groups' three code words in 8 bytes per word --
// and half-step u goes to wave u % W (a 4096 x 4096 launch: 256 blocks of 16
// waves, one half-step each).  Every wave first issues all of its loads: the
// activations of its half-steps, into its own LDS region (through registers
// and one LDS store for 1..4 tokens, buffer-to-LDS loads above that; no block
// barrier), then its code words, scale bytes and the row codebook.  It waits only for its own activations,
// dequantises each group exactly to bf16 (codebook byte permute, then the
// scaled FP8 -> bf16 conversion with the group's E8M0 scale) and multiplies:
//   * matrix cores (1..16 tokens): the group's 16 bf16 pairs are the A
//     operands of four v_mfma_f32_16x16x32_bf16, B is token i's activations
//     in lane (i, kb) -- lanes past the tokens repeat the last one, whose
//     extra output columns are dropped -- so one instruction stream serves any
//     token count up to 16;
//   * vector ALUs (1..4 tokens): v_dot2_f32_bf16 per token, then the four
//     quads of a row are added with lane exchanges.
// The waves' partial sums meet after a single block barrier and are added in
// wave order, so results are run-to-run identical.  One token on the matrix
// cores with K from 3072 up takes whole 512-k steps per wave instead
// (splitk_full_kernel: 16-byte loads, half as many load instructions), on
// matrices of up to 1536 row tiles at K = 4096 and 8192.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kSplitMaxWaves = 16;
#ifdef Q3_SPLITK_MAX_TILES
constexpr int64_t kSplitMaxTiles = Q3_SPLITK_MAX_TILES;
#else
constexpr int64_t kSplitMaxTiles = 512;
#endif
constexpr int64_t kFullMaxTiles = 1536;        // one token on whole steps (K = 4096 or 8192)
constexpr uint32_t kHalfStepBytes = 512;   // activations of one token over one half-step (4 quads x 128 B)

struct SplitArgs {
  const uint8_t* code;
  const uint8_t* scale;
  const uint8_t* cb;
  int64_t n;
  int G;            // groups per row (k / 32)
  int m;            // tokens
  const uint16_t* x;
  int64_t ldx;
  float* y;
  int64_t ldy;
  int vec_y;        // y rows 16-byte aligned and ldy % 4 == 0
  int y_rsrc;       // y's extent ((m-1)*ldy + n floats) is below 2 GiB: stores go through one buffer resource
};

// Output stores through one buffer resource over y with the system-coherent
// (sc1) policy: measured ~1% faster per launch than plain stores here, the
// outputs being the last thing a launch writes.  Only when y's extent fits a
// 32-bit resource.
constexpr int kStorePolicy = 16;
__device__ __forceinline__ rsrc_t y_rsrc(float* y, int64_t ldy, int64_t n, int m) {
  return make_rsrc(y, (uint32_t)(((int64_t)(m - 1) * ldy + n) * 4));
}
__device__ __forceinline__ void store_y4(float* y, int64_t ldy, int64_t n, int m, int64_t o, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), y_rsrc(y, ldy, n, m), (uint32_t)(o * 4), 0,
                                         kStorePolicy);
}
__device__ __forceinline__ void store_y1(float* y, int64_t ldy, int64_t n, int m, int64_t o, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), y_rsrc(y, ldy, n, m), (uint32_t)(o * 4), 0,
                                        kStorePolicy);
}

// s_waitcnt immediate that waits until at most `n` vector-memory loads of this
// wave are outstanding and leaves the other counters alone.
constexpr int vmcnt_le(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

// kW waves, kHS half-steps per wave at most; matrix cores (kDot false: up to
// NT = 1, 2, 4, 8 or 16 tokens) or vector ALUs (kDot true: exactly NT tokens).
template <int kW, int kHS, bool kDot, int NT>
__global__ __launch_bounds__(64 * kW) void splitk_kernel(SplitArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int kTok = NT;                          // tokens the LDS layout holds per half-step
  constexpr int kPairs = (kTok + 1) / 2;            // 16-byte loads per lane and half-step (two tokens each)
  constexpr uint32_t kHsBytes = kTok == 1 ? kHalfStepBytes : 2u * kPairs * kHalfStepBytes;
  constexpr uint32_t kWaveBytes = kHS * kHsBytes;
  constexpr uint32_t kRed = kW * kWaveBytes;          // partial sums of the waves

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kb = lane >> 4;
  const int m = a.m;
  const uint32_t gp = (uint32_t)((a.G + 3) & ~3);
  const int steps = (int)((gp + 15) / 16);
  const int full_steps = (int)(gp / 16);
  const uint32_t q_last = (gp - 16u * (uint32_t)(steps - 1)) / 4u;   // quads in the last step
  const int hsteps = 2 * steps;
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t T = blockIdx.x;

  const rsrc_t cr = make_rsrc(a.code, (uint32_t)(tiles * 192 * gp));
  const rsrc_t sr = make_rsrc(a.scale, (uint32_t)(tiles * 16 * gp));
  const rsrc_t cbr = make_rsrc(a.cb, (uint32_t)(a.n * 8));
  const rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)(m - 1) * a.ldx * 2 + (int64_t)a.G * 64));
  const uint32_t ldx_bytes = (uint32_t)(a.ldx * 2);
  const uint32_t kbytes = (uint32_t)a.G * 64u;   // bytes of one token's activations
  uint8_t* const xw = lds + wave * kWaveBytes;

  // ---- activations: every half-step of this wave, two tokens per load ------
  // Lane l moves 16 bytes of token 2p + l/32, quad (l/8)%4, piece l%8, to LDS
  // at 16*l: the region of a half-step is [token][quad][128 B].
  // Few tokens: the activations go through registers and a plain LDS store
  // (measured slightly faster than buffer-to-LDS loads at 1-4 tokens, slightly
  // slower at 16); one token moves 8 bytes per lane (lane l: quad l/16, bytes
  // 8*(l%16) of its 128).
  constexpr bool kXReg = NT <= 4;
  u32x4 xreg[kXReg ? kHS : 1][kXReg ? kPairs : 1];
  u32x2 xone[kTok == 1 ? kHS : 1];
  if constexpr (kTok == 1) {
#pragma unroll
    for (int u = 0; u < kHS; ++u) {
      const int hs = wave + kW * u;
      const uint32_t kofs = 1024u * (uint32_t)(hs >> 1) + 256u * (lane >> 4) + 128u * (hs & 1) + 8u * (lane & 15);
      xone[u] = bload64(xr, hs < hsteps && kofs < kbytes ? kofs : kOob);
    }
  } else {
    const int tk = lane >> 5, quad = (lane >> 3) & 3, piece = lane & 7;
#pragma unroll
    for (int u = 0; u < kHS; ++u) {
      const int hs = wave + kW * u;
      const uint32_t kofs = 1024u * (uint32_t)(hs >> 1) + 256u * quad + 128u * (hs & 1) + 16u * piece;
      const bool kok = hs < hsteps && kofs < kbytes;
#pragma unroll
      for (int p = 0; p < kPairs; ++p) {
        const int tok = 2 * p + tk;
        const uint32_t off = kok && tok < m ? (uint32_t)tok * ldx_bytes + kofs : kOob;
        if constexpr (kXReg) {
          xreg[u][p] = bload128(xr, off);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (__attribute__((address_space(3))) void*)(xw + (uint32_t)u * kHsBytes + 1024u * p), 16, off, 0, 0, 0);
        }
      }
    }
  }
  // The wait below counts the weight loads issued after this point.
  __builtin_amdgcn_sched_barrier(0);

  // ---- weights: three 8-byte code words (groups 2h, 2h+1) and two scale bytes
  // per half-step; the last step may hold fewer than four quads.
  u32x2 w[kHS][3];
  uint32_t sc[kHS];
#pragma unroll
  for (int u = 0; u < kHS; ++u) {
    const int hs = wave + kW * u;
    const int s = hs >> 1, h = hs & 1;
    const bool full = s < full_steps;
    const bool live = hs < hsteps && (full || (uint32_t)kb < q_last);
    const uint32_t js = full ? 1024u : 256u * q_last;
    const uint32_t base = live ? (uint32_t)T * 192u * gp + 3072u * (uint32_t)s + 16u * lane + 8u * h : kOob;
#pragma unroll
    for (int j = 0; j < 3; ++j) w[u][j] = __builtin_amdgcn_raw_buffer_load_b64(cr, base + js * j, 0, Q3_STREAM_POLICY);
    sc[u] = __builtin_amdgcn_raw_buffer_load_b16(
        sr, live ? (uint32_t)T * 16u * gp + 256u * (uint32_t)s + 4u * lane + 2u * h : kOob, 0, Q3_STREAM_POLICY);
  }
  const int64_t row = T * 16 + i;
  const u32x2 cbv = bload64(cbr, row < a.n ? (uint32_t)row * 8u : kOob);

  // Activations have landed once at most the weight loads are outstanding
  // (loads complete in issue order).
  if constexpr (kTok == 1) {
#pragma unroll
    for (int u = 0; u < kHS; ++u) *reinterpret_cast<u32x2*>(xw + (uint32_t)u * kHsBytes + 8u * lane) = xone[u];
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order: its own stores are read next
  } else if constexpr (kXReg) {
#pragma unroll
    for (int u = 0; u < kHS; ++u)
#pragma unroll
      for (int p = 0; p < kPairs; ++p)
        *reinterpret_cast<u32x4*>(xw + (uint32_t)u * kHsBytes + 1024u * p + 16u * lane) = xreg[u][p];
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order: its own stores are read next
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_le(4 * kHS + 1));
    __builtin_amdgcn_sched_barrier(0);
  }

  float* const red = reinterpret_cast<float*>(lds + kRed);
  if constexpr (!kDot && NT == 1 && kHS == 1) {
    // One token, one half-step: the activations go to registers right away
    // (every lane reads its quad's 128 bytes), and the waves' sums meet as the
    // 16 row sums of each, stored straight from the four lanes that hold them.
    u32x4 xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = *reinterpret_cast<const u32x4*>(xw + 128u * kb + 16u * e);
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x2 wv[16];
      dequant_group_bf16(w[0][0][t], w[0][1][t], w[0][2][t], (sc[0] >> (8 * t)) & 0xFFu, cbv.x, cbv.y, wv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x4 au = {__builtin_bit_cast(uint32_t, wv[4 * e]), __builtin_bit_cast(uint32_t, wv[4 * e + 1]),
                          __builtin_bit_cast(uint32_t, wv[4 * e + 2]), __builtin_bit_cast(uint32_t, wv[4 * e + 3])};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au), __builtin_bit_cast(bf16x8, xv[4 * t + e]),
                                                    d, 0, 0, 0);
      }
    }
    // Column 0 of D: lane 16 q holds rows 4 q .. 4 q + 3, stored as they are
    // (no lane exchange: each permute is a round trip through the LDS pipe).
    if (i == 0) *reinterpret_cast<f32x4*>(red + wave * 16 + 4 * kb) = d;
    __syncthreads();
    if (wave == 0 && lane < 16) {
      float v = red[lane];
#pragma unroll
      for (int q = 1; q < kW; ++q) v += red[q * 16 + lane];
      if (row < a.n) {
        if (a.y_rsrc) store_y1(a.y, a.ldy, a.n, m, row, v);
        else a.y[row] = v;
      }
    }
  } else if constexpr (!kDot) {
    // Lanes of absent tokens read the last token's activations: their output
    // columns repeat it and are never stored.
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    const uint32_t bl = (uint32_t)(i < m ? i : m - 1) * kHalfStepBytes + 128u * kb;
#pragma unroll
    for (int u = 0; u < kHS; ++u) {
      const uint8_t* xb = xw + (uint32_t)u * kHsBytes + bl;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x2 wv[16];
        dequant_group_bf16(w[u][0][t], w[u][1][t], w[u][2][t], (sc[u] >> (8 * t)) & 0xFFu, cbv.x, cbv.y, wv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(xb + 64u * t + 16u * e);
          const u32x4 au = {__builtin_bit_cast(uint32_t, wv[4 * e]), __builtin_bit_cast(uint32_t, wv[4 * e + 1]),
                            __builtin_bit_cast(uint32_t, wv[4 * e + 2]), __builtin_bit_cast(uint32_t, wv[4 * e + 3])};
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au), b, d, 0, 0, 0);
        }
      }
    }
    // D layout: lane l holds rows 4*(l/16)+v of the tile for token l%16; only
    // the lanes of real tokens take part in the sum over the waves.
    if (i < m) *reinterpret_cast<f32x4*>(red + 4 * (wave * 64 + lane)) = d;
    __syncthreads();
    if (wave == 0 && i < m) {
      f32x4 v = *reinterpret_cast<const f32x4*>(red + 4 * lane);
#pragma unroll
      for (int q = 1; q < kW; ++q) v += *reinterpret_cast<const f32x4*>(red + 4 * (q * 64 + lane));
      const int64_t row0 = T * 16 + 4 * kb;
      const int64_t o = (int64_t)i * a.ldy + row0;
      if (a.vec_y && a.y_rsrc && row0 + 3 < a.n) {
        store_y4(a.y, a.ldy, a.n, m, o, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row0 + e < a.n) a.y[o + e] = v[e];
      }
    }
  } else if constexpr (kDot && NT == 1 && kHS == 1) {
    // One token, one half-step on the vector ALUs: activations to registers
    // first, then the dot products, the four quads of a row added by lane
    // exchanges, and the waves' 16 row sums after one barrier.
    u32x4 xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = *reinterpret_cast<const u32x4*>(xw + 128u * kb + 16u * e);
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x2 wv[16];
      dequant_group_bf16(w[0][0][t], w[0][1][t], w[0][2][t], (sc[0] >> (8 * t)) & 0xFFu, cbv.x, cbv.y, wv);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * e + q], as_bf16x2(xv[4 * t + e][q]), acc, false);
    }
    acc += __shfl_xor(acc, 32, 64);
    acc += __shfl_xor(acc, 16, 64);
    if (lane < 16) red[wave * 16 + lane] = acc;
    __syncthreads();
    if (wave == 0 && lane < 16) {
      float v = red[lane];
#pragma unroll
      for (int q = 1; q < kW; ++q) v += red[q * 16 + lane];
      if (row < a.n) {
        if (a.y_rsrc) store_y1(a.y, a.ldy, a.n, m, row, v);
        else a.y[row] = v;
      }
    }
  } else {
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int u = 0; u < kHS; ++u) {
      const uint8_t* xb = xw + (uint32_t)u * kHsBytes + 128u * kb;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x2 wv[16];
        dequant_group_bf16(w[u][0][t], w[u][1][t], w[u][2][t], (sc[u] >> (8 * t)) & 0xFFu, cbv.x, cbv.y, wv);
#pragma unroll
        for (int tk = 0; tk < NT; ++tk) {
          float s = acc[tk];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x4 xx = *reinterpret_cast<const u32x4*>(xb + kHalfStepBytes * tk + 64u * t + 16u * e);
#pragma unroll
            for (int q = 0; q < 4; ++q) s = __builtin_amdgcn_fdot2_f32_bf16(wv[4 * e + q], as_bf16x2(xx[q]), s, false);
          }
          acc[tk] = s;
        }
      }
    }
    // The four quads of a row sit in lanes i, i+16, i+32, i+48.
#pragma unroll
    for (int tk = 0; tk < NT; ++tk) {
      float v = acc[tk];
      v += __shfl_xor(v, 32, 64);
      v += __shfl_xor(v, 16, 64);
      if (lane < 16) red[(wave * NT + tk) * 16 + lane] = v;
    }
    __syncthreads();
    if (wave == 0) {
      for (int o = lane; o < 16 * m; o += 64) {
        float v = red[o];
#pragma unroll
        for (int q = 1; q < kW; ++q) v += red[q * NT * 16 + o];
        const int64_t r = T * 16 + (o & 15);
        if (r < a.n) {
          if (a.y_rsrc) store_y1(a.y, a.ldy, a.n, m, (int64_t)(o >> 4) * a.ldy + r, v);
          else a.y[(int64_t)(o >> 4) * a.ldy + r] = v;
        }
      }
    }
  }
}

// One token on the matrix cores, whole 512-k steps: wave w takes steps w,
// w + kW, ... (kSPW of them) of the block's tile, so every lane reads its
// three code words and four scale bytes per step with 16-byte and 4-byte loads
// (half as many load instructions as half-steps) and each step's 1 KB of
// activations with one 16-byte load per lane.  kW * kSPW covers the step count;
// steps past it load nothing and add zero.
template <int kW, int kSPW>
__global__ __launch_bounds__(64 * kW) void splitk_full_kernel(SplitArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];   // kW x kSPW KB activations, then kW x 16 partial sums
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, kb = lane >> 4;
  const uint32_t gp = (uint32_t)a.G;                // a multiple of 16 here
  const int steps = (int)(gp / 16);
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t T = blockIdx.x;
  const rsrc_t cr = make_rsrc(a.code, (uint32_t)(tiles * 192 * gp));
  const rsrc_t sr = make_rsrc(a.scale, (uint32_t)(tiles * 16 * gp));
  const rsrc_t cbr = make_rsrc(a.cb, (uint32_t)(a.n * 8));
  const rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)a.G * 64));
  uint8_t* const xw = lds + wave * (1024u * kSPW);

  // Activations first (lane l: bytes 16l..16l+15 of each of its steps), then the weights.
  u32x4 xin[kSPW];
#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    const int st = wave + kW * u;
    xin[u] = bload128(xr, st < steps ? 1024u * (uint32_t)st + 16u * lane : kOob);
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 w0[kSPW], w1[kSPW], w2[kSPW];
  uint32_t sc[kSPW];
#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    const int st = wave + kW * u;
    const uint32_t base = st < steps ? (uint32_t)T * 192u * gp + 3072u * (uint32_t)st + 16u * lane : kOob;
    w0[u] = bload128_stream(cr, base);
    w1[u] = bload128_stream(cr, base + 1024u);
    w2[u] = bload128_stream(cr, base + 2048u);
    sc[u] = bload32_stream(sr, st < steps ? (uint32_t)T * 16u * gp + 256u * (uint32_t)st + 4u * lane : kOob);
  }
  const int64_t row = T * 16 + i;
  const u32x2 cbv = bload64(cbr, row < a.n ? (uint32_t)row * 8u : kOob);
#pragma unroll
  for (int u = 0; u < kSPW; ++u) *reinterpret_cast<u32x4*>(xw + 1024u * u + 16u * lane) = xin[u];
  __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order: its own stores are read next

  // Lane (i, kb) holds group t of quad kb for row i; its activations sit at
  // 256 kb + 64 t of the step.  B is token 0's activations in every lane
  // (columns 1..15 repeat column 0 and are dropped).
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kSPW; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 xv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xv[e] = *reinterpret_cast<const u32x4*>(xw + 1024u * u + 256u * kb + 64u * t + 16u * e);
      bf16x2 wv[16];
      dequant_group_bf16(w0[u][t], w1[u][t], w2[u][t], (sc[u] >> (8 * t)) & 0xFFu, cbv.x, cbv.y, wv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x4 au = {__builtin_bit_cast(uint32_t, wv[4 * e]), __builtin_bit_cast(uint32_t, wv[4 * e + 1]),
                          __builtin_bit_cast(uint32_t, wv[4 * e + 2]), __builtin_bit_cast(uint32_t, wv[4 * e + 3])};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, au), __builtin_bit_cast(bf16x8, xv[e]),
                                                    d, 0, 0, 0);
      }
    }
  // Column 0 of D (lane 16 q holds rows 4 q .. 4 q + 3) goes to LDS as it is,
  // then the waves' sums are added in wave order.
  float* const red = reinterpret_cast<float*>(lds + kW * kSPW * 1024u);
  if (i == 0) *reinterpret_cast<f32x4*>(red + wave * 16 + 4 * kb) = d;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float v = red[lane];
#pragma unroll
    for (int q = 1; q < kW; ++q) v += red[q * 16 + lane];
    if (row < a.n) {
      if (a.y_rsrc) store_y1(a.y, a.ldy, a.n, 1, row, v);
      else a.y[row] = v;
    }
  }
}

template <int kW, int kSPW>
hipError_t launch_full(const SplitArgs& a, hipStream_t s) {
  const size_t shm = (size_t)kW * (1024 * kSPW + 64);
  const int64_t tiles = (a.n + 15) / 16;
  hipLaunchKernelGGL((splitk_full_kernel<kW, kSPW>), dim3((unsigned)tiles), dim3(64 * kW), shm, s, a);
  return hipGetLastError();
}

template <int kW, int kHS, bool kDot, int NT>
size_t splitk_lds() {
  constexpr int kTok = NT;
  constexpr uint32_t kHsBytes = kTok == 1 ? kHalfStepBytes : 2u * ((kTok + 1) / 2) * kHalfStepBytes;
  return (size_t)kW * kHS * kHsBytes + (kDot ? (size_t)kW * NT * 16 * 4 : (size_t)kW * 64 * 16);
}

template <int kW, int kHS, bool kDot, int NT>
hipError_t launch_one_split(const SplitArgs& a, hipStream_t s) {
  const size_t shm = splitk_lds<kW, kHS, kDot, NT>();
  static LdsAllowance seen;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(splitk_kernel<kW, kHS, kDot, NT>), shm, seen);
  if (e != hipSuccess) return e;
  const int64_t tiles = (a.n + 15) / 16;
  hipLaunchKernelGGL((splitk_kernel<kW, kHS, kDot, NT>), dim3((unsigned)tiles), dim3(64 * kW), shm, s, a);
  return hipGetLastError();
}

// Whole steps per wave for one token on the matrix cores where that measured
// faster than half-steps on MI355X (graph-replayed launches over cold copies):
// from K = 3072 up (K = 4096, N = 8192: 5.09 -> 4.65 us; K = 8192, N = 4096:
// 5.21 -> 4.76 us; K = 6144, N = 4096: 5.04 -> 4.58 us), except K = 4096 with
// 224..256 row tiles (one 16-wave half-step block per CU), where half-steps
// were as fast or 1% faster; at K <= 2048 half-steps were as fast or faster.
// Only matrices of whole steps (K % 512 == 0).
bool use_full_steps(int64_t n, int groups, int64_t m, bool dot) {
  if (dot || m != 1 || groups % 16 != 0) return false;
  const int steps = groups / 16;
  const int64_t tiles = (n + 15) / 16;
  if (steps <= 4 || steps > kSplitMaxWaves) return false;
  return !(steps == 8 && tiles >= 224 && tiles <= 256);
}

// Waves per block and half-steps per wave for a matrix of `groups` groups per
// row: up to 16 waves with one half-step each, then two half-steps each.
struct SplitShape {
  int w, hs;
};
SplitShape split_shape(int groups) {
  const int gp = (groups + 3) & ~3;
  const int hsteps = 2 * ((gp + 15) / 16);
  if (hsteps <= kSplitMaxWaves) {
    int w = 1;
    while (w < hsteps) w *= 2;
    return {w, 1};
  }
  return {kSplitMaxWaves, (hsteps + kSplitMaxWaves - 1) / kSplitMaxWaves};
}

template <int kW, int kHS>
hipError_t launch_split_w(const SplitArgs& a, bool dot, hipStream_t s) {
  if (!dot) {
    if (a.m == 1) return launch_one_split<kW, kHS, false, 1>(a, s);
    if (a.m <= 2) return launch_one_split<kW, kHS, false, 2>(a, s);
    if (a.m <= 4) return launch_one_split<kW, kHS, false, 4>(a, s);
    if (a.m <= 8) return launch_one_split<kW, kHS, false, 8>(a, s);
    if constexpr (kHS == 1) return launch_one_split<kW, kHS, false, 16>(a, s);
    return hipErrorInvalidValue;
  }
  if constexpr (kHS == 1) {
    switch (a.m) {
      case 1: return launch_one_split<kW, kHS, true, 1>(a, s);
      case 2: return launch_one_split<kW, kHS, true, 2>(a, s);
      case 3: return launch_one_split<kW, kHS, true, 3>(a, s);
      case 4: return launch_one_split<kW, kHS, true, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.m == 1) return launch_one_split<kW, kHS, true, 1>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

// The split-K kernel takes dense products of up to 16 tokens (up to 4 on the
// vector ALUs, on at most 256 row tiles past one) on matrices of at most 512 row tiles and K up to 16384 (at most
// two half-steps per wave, then at most 8 tokens: the activations of every
// half-step are staged at once), and one token on the matrix cores with whole
// steps on matrices of up to 1536 row tiles at K = 4096 or 8192.
bool splitk_applies(int64_t n, int groups, int64_t m, bool dot) {
  if (n < 1 || m < 1 || m > (dot ? 4 : 16)) return false;
  const int64_t tiles = (n + 15) / 16;
  if (dot && m > 1) {
    // 2..4 tokens on the vector ALUs, one half-step per wave, on matrices of
    // at most 256 row tiles, measured against the stream kernel: 4096 x 4096 at
    // 2 and 3 tokens 5.35 -> 4.15 and 6.02 -> 4.55 us, 2048 x 2048 at 4 tokens
    // 4.95 -> 3.81 us; at 512 tiles the stream kernel was as fast or faster,
    // and 4 tokens over 16 waves (K > 2048) spill registers (4096 x 4096: 7.11
    // vs 6.78 us).
    const SplitShape sh = split_shape(groups);
    return tiles <= 256 && sh.hs == 1 && (m <= 3 || sh.w <= 8);
  }
  if (tiles > kSplitMaxTiles) {
    // One token on whole steps also beats the tall kernel up to 1536 row tiles
    // when the steps fill the block's waves (K = 4096 or 8192), measured:
    // 11008 x 4096 6.97 -> 5.49 us, 16384 x 4096 10.27 -> 7.08 us, 24576 x 4096
    // 10.66 -> 9.84 us, 12288 x 8192 11.45 -> 10.12 us, 16384 x 8192 17.12 ->
    // 12.53 us; from 1792 tiles (28672 x 8192: 18.2 vs 18.8 us) it does not.
    const int steps = groups / 16;
    return tiles <= kFullMaxTiles && (steps == 8 || steps == 16) && use_full_steps(n, groups, m, dot);
  }
  const SplitShape sh = split_shape(groups);
  return sh.hs == 1 || (sh.hs == 2 && m <= 8);
}

hipError_t launch_splitk(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                         bool dot, hipStream_t s) {
  if (!splitk_applies(w.n, w.groups, m, dot)) return hipErrorInvalidValue;
  SplitArgs a{};
  a.code = w.code;
  a.scale = w.scale;
  a.cb = w.cb;
  a.n = w.n;
  a.G = w.groups;
  a.m = (int)m;
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.vec_y = ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  a.y_rsrc = ((m - 1) * ldy + w.n) * 4 < (int64_t(1) << 31);
  if (use_full_steps(w.n, w.groups, m, dot)) {
    const int steps = w.groups / 16;
    if (steps <= 8) return launch_full<8, 1>(a, s);
    // K = 8192 past 1024 row tiles: 8-wave blocks of two steps per wave (four
    // blocks per CU instead of two), measured 18.3 -> 17.0 us at 24576 x 8192
    // and 15.2 -> 14.7 us at 20480 x 8192; at 1024 tiles and fewer the 16-wave
    // blocks were faster.
    if ((w.n + 15) / 16 > 1024) return launch_full<8, 2>(a, s);
    return launch_full<16, 1>(a, s);
  }
  const SplitShape sh = split_shape(w.groups);
  if (sh.hs == 1) {
    switch (sh.w) {
      case 1: return launch_split_w<1, 1>(a, dot, s);
      case 2: return launch_split_w<2, 1>(a, dot, s);
      case 4: return launch_split_w<4, 1>(a, dot, s);
      case 8: return launch_split_w<8, 1>(a, dot, s);
      case 16: return launch_split_w<16, 1>(a, dot, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (sh.hs == 2) return launch_split_w<16, 2>(a, dot, s);
  return hipErrorInvalidValue;
}

}  // namespace q3
