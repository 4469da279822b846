// Decode / verify products over the 3.25-bit codebook format: dense on the
// matrix cores (1..64 tokens), dense on the vector ALUs (1..8 tokens), and
// expert-grouped on the matrix cores (MoE verify rounds).
//
// What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices,
// "Model surgery" / "Three-bit weights"): y[m][n] = sum_k x[m][k] * w[n][k] with
// w = E4M3FN(codebook[n][code]) * 2^(scale - 127).  The page's own kernel looks
// the codes up and feeds the FP8 matrix units; here the looked-up E4M3 bytes are
// widened exactly to bf16 (group scale folded into the conversion), so every
// product is exact and only the fp32 accumulation rounds, whatever the
// activations are.
//
// Work unit: a step = one 16-row tile x 512 k (16 groups per row).  The planes
// are tile-major, so a step's code words are one contiguous 3 KB block (three
// 1 KB runs, one per word index) and its scales one 256-byte run; lane l of a
// wave serves row l%16 and groups 4*(l/16)..+3 of the step and reads its three
// words and four scale bytes with one 16-byte and one 4-byte buffer load per
// run, so every load instruction of the wave covers one contiguous span.  Each
// group is dequantised once into 16 bf16 pairs:
//   * matrix-core mode: the pairs are the A operands of 4 MFMAs
//     (v_mfma_f32_16x16x32_bf16) per column tile of 16 tokens; the B operand of
//     the same lane is the matching 8 activations of token 16c + l%16, read from
//     LDS once per step and used by all R row tiles of the wave, so A and B
//     agree on which k sits in which slot by construction;
//   * vector-ALU mode: the pairs meet the activations (read from LDS, the same
//     address for the 16 lanes of a quad) in v_dot2_f32_bf16, one fp32 partial
//     per lane, row and token; the four quads of a row are summed with lane
//     shuffles at the end.
//
// Activations are staged in LDS once per block ("full-K" mode) or, when they do
// not fit, one 512-k step at a time into a double buffer ("stream" mode).  The
// next step's code words and scales are loaded before the current step is
// computed (in stream mode right behind that step's activations, which are
// requested first); all loads are buffer loads whose out-of-range offsets read as zero,
// so rows past n, padding groups and absent tokens need no branches.  In full-K
// mode the waves of a block may split K (few rows); partial sums are then
// added through LDS in a fixed order, so results are run-to-run identical.
//
// The grouped variant runs one grid row per expert the round picked (with up
// to 64 experts, row y takes the y-th smallest picked id, so blocks with work
// are dispatched first; past 64, row e is expert e).  Its block first collects
// the (token, slot) pairs routed to that expert; a row without one returns
// before reading any weight byte (Hibana page, "Adaptive speculation" /
// "Expert sharing": a verify round reads every picked expert once).
#include <atomic>
#include <type_traits>

#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

// LDS bytes for full-K activation staging: up to 136 KB, one block per CU
// (measured on MI355X: 4096 x 4096 at 16 tokens 12.1 us streamed, 7.1 us
// staged whole in 8-wave blocks with K split over the waves).
#ifdef Q3_FULLK_KB
constexpr int kFullKBudget = Q3_FULLK_KB * 1024;
#else
constexpr int kFullKBudget = 136 * 1024;
#endif

// How a block holds the activations.
enum Mode : int {
  kShared = 0,   // all of K for all tokens, staged once per block
  kStream = 1,   // one 512-k step at a time, double-buffered through registers
};
constexpr uint32_t kRowPad = 16;          // LDS row padding against bank conflicts

// Which rows and tokens a block takes.
enum Grouping : int {
  kDense = 0,         // every token against every row
  kExperts = 1,       // grid row e: the (token, slot) pairs routed to expert e
  kSwiGLU = 2,        // as kExperts on a gate/up matrix [gate I rows; up I rows]: a wave takes
                      // gate tile q and up tile q and writes h = silu(g) * u as two bf16 terms
  kDownTerms = 3,     // as kExperts with each pair's activation given as two bf16 rows (high
                      // and low term): the block adds the two products and stores one output
                      // row per pair
};

struct KArgs {
  const uint8_t* code;
  int64_t code_stride;    // bytes between experts
  const uint8_t* scale;
  int64_t scale_stride;
  const uint8_t* cb;
  int64_t cb_stride;
  int64_t n;
  int G;
  const uint16_t* x;
  int64_t ldx;
  int64_t x_rows;   // rows of x that may be read
  float* y;
  int64_t ldy;
  int64_t split_stride;   // streamed modes split over blockIdx.z: split z writes y + z * split_stride
  int m;          // dense: number of tokens
  int vec_y;      // y rows 16-byte aligned: four consecutive outputs go out as one store
  int sk;         // K split over the waves of a block (full-K mode)
  const int32_t* ids;
  int pairs_total, topk, x_by_slot;
  int slice_cap;   // expert passes in full-K mode: token rows the LDS staging holds (<= 16, even)
  int num_experts;
  // kSwiGLU: tiles in the gate half; output terms h[2*pair + term][I]
  int half_tiles;
  uint16_t* h;
  int64_t ldh;
  // kDownTerms: per-pair outputs
  float* part;
  int64_t ldp;
};

__device__ __forceinline__ bf16x8 pack_bf16x8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
             __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

// Wave-uniform geometry of one matrix's planes.
struct Planes {
  rsrc_t code, scale;
  int full_steps, steps;
  uint32_t q_last;   // quads of groups in the last step (1..4)
};

// Per-lane view of one row tile: byte offsets of the lane's piece in step 0
// (kOob for tiles past the plane); a step adds a wave-uniform amount that
// stays inside the tile.
struct RowTile {
  uint32_t vcode;     // tile*64*words*Gp + 16*lane (words = 3, or 2 for the 2-bit head)
  uint32_t vscale;    // tile*16*Gp + 4*lane
  uint32_t cbl, cbh;  // the lane's row codebook (zero past n; the 2-bit head's 4 entries in cbl)
};

// Code words and scales of one step of R row tiles, for one lane; kWd code
// words per group (3 for the 3-bit layer, 2 for the 2-bit draft head).
template <int R, int kWd = 3>
struct StepData {
  u32x4 w[R][kWd];   // w[r][j][t] = word j of the lane's group t in row tile r
  uint32_t sc[R];  // byte t = scale of group t
};

// Branch-free on purpose: loads issued under a condition make the wait-count
// insertion assume the worst case and drain every outstanding prefetch.  Steps
// at or past s_end re-read step s_end-1 (cached, never computed).  On a partial
// last step, lanes past its quads (last_ok false) read zeros for both codes
// and scales; a zero scale byte widens to a zero fp32 scale, so those lanes
// contribute exactly zero whatever activations they meet.
template <int R, int kWd>
__device__ __forceinline__ void load_step(const Planes& p, const RowTile (&rt)[R], bool last_ok, int s, int s_end,
                                          StepData<R, kWd>& d) {
  const int sc = s < s_end ? s : s_end - 1;
  const bool full = sc < p.full_steps;
  const bool live = full || last_ok;
  const uint32_t js = full ? 1024u : 256u * p.q_last;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t o = (live ? rt[r].vcode : kOob) + 1024u * kWd * sc;
#pragma unroll
    for (int j = 0; j < kWd; ++j) d.w[r][j] = bload128_stream(p.code, o + js * j);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) d.sc[r] = bload32_stream(p.scale, (live ? rt[r].vscale : kOob) + 256u * sc);
}

__device__ __forceinline__ void dequant(const u32x4 (&w)[3], uint32_t sc, int t, uint32_t cbl, uint32_t cbh,
                                        bf16x2 (&wv)[16]) {
  dequant_group_bf16(w[0][t], w[1][t], w[2][t], (sc >> (8 * t)) & 0xFFu, cbl, cbh, wv);
}
__device__ __forceinline__ void dequant(const u32x4 (&w)[2], uint32_t sc, int t, uint32_t cbl, uint32_t,
                                        bf16x2 (&wv)[16]) {
  dequant_group2_bf16(w[0][t], w[1][t], (sc >> (8 * t)) & 0xFFu, cbl, wv);
}

// Matrix-core step: dequantise the step's 4 groups of every row tile and run
// 4*4*MT*R MFMAs.  xb[c] is the lane's LDS byte address of its B operand for
// column tile c at this step (group 0, k 0).  With few column tiles the B
// operands of a group are held while the row tiles are dequantised one by one;
// with many, the row tiles' A operands are held while the B operands stream.
template <int MT, int R, int kWd>
__device__ __forceinline__ void mfma_step(const StepData<R, kWd>& d, const RowTile (&rt)[R], const uint32_t (&xb)[MT],
                                          const uint8_t* lds, f32x4 (&acc)[R][MT]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (MT <= R) {
      bf16x8 b[4][MT];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < MT; ++c) b[e][c] = *reinterpret_cast<const bf16x8*>(lds + xb[c] + 64u * t + 16u * e);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bf16x2 wv[16];
        dequant(d.w[r], d.sc[r], t, rt[r].cbl, rt[r].cbh, wv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x8 a = pack_bf16x8(wv[4 * e], wv[4 * e + 1], wv[4 * e + 2], wv[4 * e + 3]);
#pragma unroll
          for (int c = 0; c < MT; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[e][c], acc[r][c], 0, 0, 0);
        }
      }
    } else {
      bf16x2 wv[R][16];
#pragma unroll
      for (int r = 0; r < R; ++r) dequant(d.w[r], d.sc[r], t, rt[r].cbl, rt[r].cbh, wv[r]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int c = 0; c < MT; ++c) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(lds + xb[c] + 64u * t + 16u * e);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const bf16x8 a = pack_bf16x8(wv[r][4 * e], wv[r][4 * e + 1], wv[r][4 * e + 2], wv[r][4 * e + 3]);
            acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[r][c], 0, 0, 0);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < MT; ++c) asm volatile("" : "+v"(acc[r][c]));
}

// Matrix-core step for one wave per SIMD holding many row tiles, software
// pipelined: the step is a sequence of 4*R units (group t, row tile r), and
// the vector-ALU dequantisation of unit u+1 is interleaved with the MFMAs of
// unit u (one MFMA, then a few ALU instructions), so the matrix core does not
// wait for the conversion.  The B operands of group t are held across its R
// units; those of group t+1 are read from LDS during the last unit of group t,
// each right after the MFMAs that last read the registers it replaces.  The
// next step's kLoads memory loads are handed out a few per unit through
// issue(integral_constant<Q>): a wave that issues them all at once stalls
// until the memory pipeline has room, and with one wave per SIMD the matrix
// core would stall with it.
template <int Q, int Q1, typename Issue>
__device__ __forceinline__ void issue_range(Issue& issue) {
  if constexpr (Q < Q1) {
    issue(std::integral_constant<int, Q>{});
    issue_range<Q + 1, Q1>(issue);
  }
}

template <int U, int MT, int R, int kLoads, typename Issue>
__device__ __forceinline__ void pipe_unit(const StepData<R>& d, const RowTile (&rt)[R], const uint32_t (&xb)[MT],
                                          const uint8_t* lds, f32x4 (&acc)[R][MT], bf16x8 (&b)[4][MT],
                                          bf16x2 (&wv)[2][16], Issue& issue) {
  constexpr int kUnits = 4 * R;
  if constexpr (U < kUnits) {
    constexpr int t = U / R, r = U % R, cur = U & 1;
    constexpr int kMfma = 4 * MT;                     // MFMAs per unit
    constexpr int kValu = (48 + kMfma - 1) / kMfma;   // ALU instructions after each of them
    constexpr int q0 = U * kLoads / kUnits, q1 = (U + 1) * kLoads / kUnits;
    issue_range<q0, q1>(issue);
    if constexpr (U + 1 < kUnits) {
      constexpr int t1 = (U + 1) / R, r1 = (U + 1) % R;
      dequant(d.w[r1], d.sc[r1], t1, rt[r1].cbl, rt[r1].cbh, wv[cur ^ 1]);
    }
    constexpr bool refill = r == R - 1 && t < 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x8 a = pack_bf16x8(wv[cur][4 * e], wv[cur][4 * e + 1], wv[cur][4 * e + 2], wv[cur][4 * e + 3]);
#pragma unroll
      for (int c = 0; c < MT; ++c) acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[e][c], acc[r][c], 0, 0, 0);
      if constexpr (refill) {
#pragma unroll
        for (int c = 0; c < MT; ++c)
          b[e][c] = *reinterpret_cast<const bf16x8*>(lds + xb[c] + 64u * (t + 1) + 16u * e);
      }
    }
    if constexpr (q1 > q0) __builtin_amdgcn_sched_group_barrier(0x020, q1 - q0, 0);   // this unit's loads first
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);   // then vector ALU work
      }
      if constexpr (refill) __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);   // this e's B reads for t+1
    }
    __builtin_amdgcn_sched_barrier(0);
    pipe_unit<U + 1, MT, R, kLoads>(d, rt, xb, lds, acc, b, wv, issue);
  }
}

template <int MT, int R, int kLoads, typename Issue>
__device__ __forceinline__ void mfma_step_pipe(const StepData<R>& d, const RowTile (&rt)[R], const uint32_t (&xb)[MT],
                                               const uint8_t* lds, f32x4 (&acc)[R][MT], Issue&& issue) {
  bf16x8 b[4][MT];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int c = 0; c < MT; ++c) b[e][c] = *reinterpret_cast<const bf16x8*>(lds + xb[c] + 16u * e);
  bf16x2 wv[2][16];
  dequant(d.w[0], d.sc[0], 0, rt[0].cbl, rt[0].cbh, wv[0]);
  __builtin_amdgcn_sched_barrier(0);
  pipe_unit<0, MT, R, kLoads>(d, rt, xb, lds, acc, b, wv, issue);
}

// Vector-ALU step for M tokens: xa[m] is the LDS byte address of token m's
// activations at this step and the lane's quad (group 0, k 0).  The next
// token's activations are read while the current token's dot products run;
// the scheduling barriers stop the compiler from hoisting every token's reads
// to the top (64 registers per token).
template <int M, int R, int kWd>
__device__ __forceinline__ void dot_step(const StepData<R, kWd>& d, const RowTile (&rt)[R], const uint32_t (&xa)[M],
                                         const uint8_t* lds, float (&acc)[R][M]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x2 wv[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r) dequant(d.w[r], d.sc[r], t, rt[r].cbl, rt[r].cbh, wv[r]);
    u32x4 xv[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[0][e] = *reinterpret_cast<const u32x4*>(lds + xa[0] + 64u * t + 16u * e);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m + 1 < M) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xv[(m + 1) & 1][e] = *reinterpret_cast<const u32x4*>(lds + xa[m + 1] + 64u * t + 16u * e);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float a = acc[r][m];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          a = __builtin_amdgcn_fdot2_f32_bf16(wv[r][q], as_bf16x2(xv[m & 1][q >> 2][q & 3]), a, false);
        acc[r][m] = a;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Pin the accumulation here: otherwise the compiler may sink the whole
  // step's arithmetic past the caller's barrier and keep every activation
  // read so far live (spilled) until then.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) asm volatile("" : "+v"(acc[r][m]));
}

// Copy `count` 16-byte chunks from global memory (buffer resource) into LDS.
// All loads of a batch are issued before any store, so a batch costs one
// memory latency instead of one per chunk.  src(c) returns the chunk's byte
// offset in the resource (kOob for zeros), dst(c) its LDS byte address.
template <int kBatch, int kThreads, typename Src, typename Dst>
__device__ __forceinline__ void stage_chunks(rsrc_t r, int count, uint8_t* lds, Src src, Dst dst) {
  for (int base = threadIdx.x; base < count; base += kBatch * kThreads) {
    u32x4 v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int c = base + q * kThreads;
      v[q] = bload128(r, c < count ? src(c) : kOob);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int c = base + q * kThreads;
      if (c < count) *reinterpret_cast<u32x4*>(lds + dst(c)) = v[q];
    }
  }
}

// Waves per SIMD the register budget is held to (128 registers per lane for 4,
// 256 for 2): a decode launch wants every wave resident at once.
template <int NT, int R, bool kDot>
constexpr int min_waves_per_eu() {
  if (kDot) return R == 1 ? (NT <= 5 ? 4 : 3) : 2;
  return R == 1 && NT <= 2 ? 4 : 2;
}

// OR of a value over the 64 lanes of a wave (every lane active), returned as
// a wave-uniform value: DPP exchanges inside rows of 16 lanes, then the four
// rows' results by readlane.
__device__ __forceinline__ uint32_t wave_or32(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);   // row_mirror
  return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) | __builtin_amdgcn_readlane((int)v, 16) |
                    __builtin_amdgcn_readlane((int)v, 32) | __builtin_amdgcn_readlane((int)v, 48));
}

// NT: column tiles of 16 tokens (matrix-core mode) or tokens (vector-ALU mode).
// kBits: 3 for the 3-bit layer, 2 for the two-bit draft head (two code words
// per group, a 4-entry codebook per row).
template <int NT, int R, int kW, int kGrouped, int kMode, bool kDot, int kBits>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(min_waves_per_eu<NT, R, kDot>())))
void linear_kernel(KArgs a) {
  constexpr int kWd = kBits == 2 ? 2 : 3;          // code words per group
  constexpr uint32_t kCbBytes = kBits == 2 ? 4 : 8;   // codebook bytes per row
  constexpr int kThreads = 64 * kW;
  constexpr int kSlice = kDot ? NT : 16 * NT;   // tokens per slice
  extern __shared__ __align__(16) uint8_t lds[];
  // Expert passes: each wave keeps its own copy of the block's (token, slot)
  // pairs, written and read by that wave alone, so no block barrier stands
  // between the ids and the first loads.
  __shared__ int pairs_w[kGrouped ? kW : 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform from here on
  const int i = lane & 15;
  const int kb = lane >> 4;
  const int sk = kMode != kStream ? a.sk : 1;
  const int rb = kW / sk;
  const int rg = wave / sk;
  const int ks = wave - rg * sk;

  // ---- which expert / tokens -------------------------------------------------
  int expert = 0, npairs = 0;
  if (kGrouped) {
    // Every wave reads the round's ids and finds its block's expert and pairs
    // itself, so the planes' addresses and the first loads need no barrier.
    const int id = lane < a.pairs_total ? a.ids[lane] : -1;
    int e = blockIdx.y;
    if (a.num_experts <= 64) {
      // Grid row y takes the round's y-th smallest picked expert, so the
      // blocks with work come first in dispatch order and the rows past the
      // round's distinct experts (at most its 64 pairs) exit at once.
      const bool valid = id >= 0 && id < a.num_experts;
      const uint64_t bit = valid ? 1ull << id : 0ull;
      const uint64_t used = (uint64_t)wave_or32((uint32_t)bit) | (uint64_t)wave_or32((uint32_t)(bit >> 32)) << 32;
      const bool sel = ((used >> lane) & 1ull) != 0 && (int)__popcll(used & ((1ull << lane) - 1ull)) == (int)blockIdx.y;
      const uint64_t pick = __ballot(sel);
      e = pick != 0 ? __builtin_ctzll(pick) : -1;
    }
    expert = __builtin_amdgcn_readfirstlane(e);
    const bool match = expert >= 0 && id == expert;
    const unsigned long long mask = __ballot(match);
    if (match) pairs_w[kGrouped ? wave : 0][__popcll(mask & ((1ull << lane) - 1ull))] = lane;
    npairs = __popcll(mask);
    // Order this wave's writes of its pairs before its reads of them.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (npairs == 0) return;   // not picked this round: no weight byte is read
  }
  const int* const pairs = pairs_w[kGrouped ? wave : 0];
  const int total_tokens = kGrouped == kDownTerms ? 2 * npairs : (kGrouped ? npairs : a.m);

  const int G = a.G;
  const uint32_t gp = (uint32_t)((G + 3) & ~3);
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t tile0 = ((int64_t)blockIdx.x * rb + rg) * R;   // first row tile of this wave
  // Row tiles of this wave: R consecutive tiles, or gate tile q and up tile q.
  int64_t tix[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (kGrouped == kSwiGLU) {
      const int64_t q = (int64_t)blockIdx.x * rb + rg;
      tix[r] = q < a.half_tiles ? q + r * a.half_tiles : tiles;
    } else {
      tix[r] = tile0 + r;
    }
  }

  Planes p;
  p.code = make_rsrc(a.code + (int64_t)expert * a.code_stride, (uint32_t)(tiles * 64 * kWd * gp));
  p.scale = make_rsrc(a.scale + (int64_t)expert * a.scale_stride, (uint32_t)(tiles * 16 * gp));
  p.full_steps = (int)(gp / 16);
  p.steps = (int)((gp + 15) / 16);
  p.q_last = (gp - 16u * (uint32_t)(p.steps - 1)) / 4u;
  const bool last_ok = (uint32_t)kb < p.q_last;   // lane has groups in a partial last step
  const rsrc_t cbr = make_rsrc(a.cb + (int64_t)expert * a.cb_stride, (uint32_t)(a.n * kCbBytes));
  RowTile rt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t T = tix[r];
    const bool tile_ok = T < tiles;
    rt[r].vcode = tile_ok ? (uint32_t)T * (64u * kWd * gp) + 16u * lane : kOob;
    rt[r].vscale = tile_ok ? (uint32_t)T * (16u * gp) + 4u * lane : kOob;
  }

  // Full-K mode splits K over the waves of a block; stream mode over the
  // blocks of a grid column (blockIdx.z), each split writing its own partial
  // output plane.
  const int zs = blockIdx.z, nzs = gridDim.z;
  const int s0 = kMode != kStream ? (ks * p.steps) / sk : (zs * p.steps) / nzs;
  const int s1 = kMode != kStream ? ((ks + 1) * p.steps) / sk : ((zs + 1) * p.steps) / nzs;
  float* const ybase = a.y + (int64_t)zs * a.split_stride;

  StepData<R, kWd> A, B;
  const rsrc_t xr_rsrc = make_rsrc(a.x, (uint32_t)((a.x_rows - 1) * a.ldx * 2 + (int64_t)G * 64));
  const uint32_t ldx_bytes = (uint32_t)(a.ldx * 2);

  // Tokens per slice: the matrix-core width, or for the expert passes in
  // full-K mode the rows their LDS was sized for (an expert meets each token at
  // most once per round, so one slice normally covers it).
  const int cap = kGrouped && kMode == kShared ? a.slice_cap : kSlice;
  for (int slice = 0; slice < total_tokens; slice += cap) {
    const int cnt = total_tokens - slice < cap ? total_tokens - slice : cap;
    // Token slot j of this slice -> its x row and y row.
    auto xrow = [&](int j) -> int {
      if (kGrouped == kDownTerms) return 2 * pairs[(slice + j) >> 1] + ((slice + j) & 1);
      if (kGrouped) return a.x_by_slot ? pairs[slice + j] : pairs[slice + j] / a.topk;
      return slice + j;
    };
    auto yrow = [&](int j) -> int { return kGrouped ? pairs[slice + j] : slice + j; };
    f32x4 acc[R][kDot ? 1 : NT];
    float dacc[R][kDot ? NT : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int c = 0; c < (kDot ? 1 : NT); ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < (kDot ? NT : 1); ++c) dacc[r][c] = 0.f;
    }
    // The slice's first weight step (and, once, the codebooks) is requested
    // right after the activations it will meet.
    auto begin_slice = [&](int sl) {
      load_step(p, rt, last_ok, s0, s1, A);
      if (sl == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t row = tix[r] * 16 + i;
          if constexpr (kBits == 2) {
            rt[r].cbl = bload32(cbr, row < a.n ? (uint32_t)row * 4u : kOob);
            rt[r].cbh = 0u;
          } else {
            const u32x2 cb = bload64(cbr, row < a.n ? (uint32_t)row * 8u : kOob);
            rt[r].cbl = cb.x;
            rt[r].cbh = cb.y;
          }
        }
      }
    };
    // Lane addresses of token slots at the step's start in a row-per-token x
    // layout of the given row stride, for buffer base `base` (absent tokens of
    // matrix-core mode go to `zero`, a 1 KB zero block, and stay there).
    auto run = [&](const StepData<R, kWd>& d, uint32_t base, uint32_t rstride, uint32_t zero, uint32_t adv) {
      if constexpr (kDot) {
        uint32_t xa[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) xa[m] = (m < cnt ? base + m * rstride + adv : zero) + 256u * kb;
        dot_step<NT, R>(d, rt, xa, lds, dacc);
      } else {
        uint32_t xb[NT];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int j = 16 * c + i;
          xb[c] = (j < cnt ? base + j * rstride + adv : zero) + 256u * kb;
        }
        mfma_step<NT, R>(d, rt, xb, lds, acc);
      }
    };

    if constexpr (kMode == kShared) {
      // Stage all activations: row j holds token j's K values (zero past K,
      // including the row's 16-byte pad, which lanes past a partial last
      // step's quads read with a zero scale); a 1 KB zero block follows.  The
      // first batch of activation loads goes out before the weight loads:
      // loads complete in issue order, so activations queued behind a step of
      // weights would hold up every wave of the block at the barrier below.
      const uint32_t rstride = gp * 64u + kRowPad;
      const uint32_t zero_base = (uint32_t)cnt * rstride;
      const int cpr = (int)(rstride / 16);
      const int nchunk = cnt * cpr + 64;   // rows are contiguous, then the zero block
      auto src = [&](int c) {
        const int j = c / cpr, q = c - j * cpr;
        return j < cnt && q * 8 < G * 32 ? (uint32_t)xrow(j) * ldx_bytes + 16u * q : kOob;
      };
      constexpr int kFirst = 4;
      u32x4 xv[kFirst];
#pragma unroll
      for (int q = 0; q < kFirst; ++q) {
        const int c = tid + q * kThreads;
        xv[q] = bload128(xr_rsrc, c < nchunk ? src(c) : kOob);
      }
      begin_slice(slice);
#pragma unroll
      for (int q = 0; q < kFirst; ++q) {
        const int c = tid + q * kThreads;
        if (c < nchunk) *reinterpret_cast<u32x4*>(lds + 16u * c) = xv[q];
      }
      if (nchunk > kFirst * kThreads)
        stage_chunks<4, kThreads>(xr_rsrc, nchunk - kFirst * kThreads, lds + 16 * kFirst * kThreads,
                                  [&](int c) { return src(c + kFirst * kThreads); },
                                  [&](int c) { return 16u * c; });
      __syncthreads();
      // One step is in flight while another is computed (measured: issuing
      // more steps ahead is slower on this pattern).  The scheduling barriers
      // keep each refill where it is issued; without them the compiler sinks
      // the loads below the MFMAs or hoists the refill above the computation
      // that still reads the registers.
      for (int s = s0; s < s1; s += 2) {
        load_step(p, rt, last_ok, s + 1, s1, B);
        __builtin_amdgcn_sched_barrier(0);
        run(A, 0u, rstride, zero_base, 1024u * s);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 >= s1) break;
        load_step(p, rt, last_ok, s + 2, s1, A);
        __builtin_amdgcn_sched_barrier(0);
        run(B, 0u, rstride, zero_base, 1024u * (s + 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Stream the activations one 512-k step at a time through two buffers of
      // kSlice rows (rows of absent tokens stay zero) followed by a 1 KB zero
      // block.  Step s+1's activations are fetched into registers before step s
      // is computed and stored to LDS after it, into the buffer step s-1 used.
      constexpr int kChunks = (kSlice * 64 + kThreads - 1) / kThreads;   // per thread
      const uint32_t rstride = 1024u + kRowPad;
      const uint32_t buf_bytes = (uint32_t)kSlice * rstride;
      const uint32_t zero_base = 2u * buf_bytes;
      const int nchunk = kSlice * 64;   // 16-byte chunks per buffer
      auto fetch = [&](int s, u32x4 (&r)[kChunks]) {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
          const int idx = tid + q * kThreads;
          const int j = idx >> 6, c16 = idx & 63;
          const int k0 = s * 512 + c16 * 8;
          const bool ok = idx < nchunk && j < cnt && s < s1 && k0 < G * 32;
          r[q] = bload128(xr_rsrc, ok ? (uint32_t)xrow(j) * ldx_bytes + 2u * k0 : kOob);
        }
      };
      auto put = [&](int buf, const u32x4 (&r)[kChunks]) {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
          const int idx = tid + q * kThreads;
          const int j = idx >> 6, c16 = idx & 63;
          if (idx < nchunk) *reinterpret_cast<u32x4*>(lds + buf * buf_bytes + j * rstride + 16u * c16) = r[q];
        }
      };
      u32x4 xr[kChunks];
      fetch(s0, xr);
      begin_slice(slice);
      if (tid < 64) *reinterpret_cast<u32x4*>(lds + zero_base + 16u * tid) = u32x4{0u, 0u, 0u, 0u};
      put(0, xr);
      __syncthreads();
      // Each step's activations are requested before its weights: loads
      // complete in issue order, so the LDS store of the activations (and the
      // barrier behind it) then waits for them alone while the weights are
      // still in flight (measured: 28672 x 8192 at 16 tokens 23.6 -> 21.8 us,
      // K = 28672, N = 8192 at 16 tokens 49.7 -> 46.9 us in one pass and
      // 24.9 -> 22.9 us split over blocks).
      for (int s = s0; s < s1; s += 2) {
        fetch(s + 1, xr);
        load_step(p, rt, last_ok, s + 1, s1, B);
        __builtin_amdgcn_sched_barrier(0);
        run(A, 0u, rstride, zero_base, 0u);
        __builtin_amdgcn_sched_barrier(0);
        put(1, xr);   // buffer 1 was last read at step s-1
        __syncthreads();
        if (s + 1 >= s1) break;
        fetch(s + 2, xr);
        load_step(p, rt, last_ok, s + 2, s1, A);
        __builtin_amdgcn_sched_barrier(0);
        run(B, buf_bytes, rstride, zero_base, 0u);
        __builtin_amdgcn_sched_barrier(0);
        put(0, xr);
        __syncthreads();
      }
    }

    // ---- combine K splits and store --------------------------------------------
    if constexpr (kDot) {
      // The four quads of a row sit in lanes i, i+16, i+32, i+48.
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          float v = dacc[r][m];
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);
          dacc[r][m] = v;
        }
    }
    if (kMode != kStream && sk > 1) {
      __syncthreads();   // activations no longer needed: reuse LDS for partial sums
      constexpr int kVals = kDot ? NT : 4 * NT;   // floats per lane and row tile
      float* red = reinterpret_cast<float*>(lds);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < kVals; ++v)
          red[((wave * R + r) * kVals + v) * 64 + lane] = kDot ? dacc[r][v] : acc[r][v / 4][v % 4];
      __syncthreads();
      if (ks == 0) {
        for (int q = 1; q < sk; ++q) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int v = 0; v < kVals; ++v) {
              const float o = red[(((wave + q) * R + r) * kVals + v) * 64 + lane];
              if constexpr (kDot) dacc[r][v] += o;
              else acc[r][v / 4][v % 4] += o;
            }
        }
      }
    }
    if (ks == 0) {
      if constexpr (kDot) {
        if (kb == 0) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int64_t row = tix[r] * 16 + i;
            if (row < a.n) {
#pragma unroll
              for (int m = 0; m < NT; ++m)
                if (m < cnt) ybase[(int64_t)yrow(m) * a.ldy + row] = dacc[r][m];
            }
          }
        }
      } else if constexpr (kGrouped == kSwiGLU) {
        // D layout: lane l holds rows 4*(l/16)+v of the tile for token l%16; the
        // gate and up tiles share it, so h is elementwise.  h goes out as a high
        // bf16 term and the bf16 rounding of the remainder (exact in fp32).
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int j = 16 * c + i;
          if (j < cnt && tix[0] < a.half_tiles) {
            const int pair = pairs[slice + j];
            uint32_t hi[2], lo[2];
#pragma unroll
            for (int v = 0; v < 4; v += 2) {
              float hv[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float g = acc[0][c][v + e], u = acc[1][c][v + e];
                hv[e] = g / (1.0f + expf(-g)) * u;
              }
              const bf16x2 h2 = {static_cast<__bf16>(hv[0]), static_cast<__bf16>(hv[1])};
              const bf16x2 l2 = {static_cast<__bf16>(hv[0] - static_cast<float>(h2[0])),
                                 static_cast<__bf16>(hv[1] - static_cast<float>(h2[1]))};
              hi[v / 2] = __builtin_bit_cast(uint32_t, h2);
              lo[v / 2] = __builtin_bit_cast(uint32_t, l2);
            }
            const int64_t col = tix[0] * 16 + 4 * kb;
            uint16_t* hr = a.h + (int64_t)(2 * pair) * a.ldh + col;
            *reinterpret_cast<u32x2*>(hr) = u32x2{hi[0], hi[1]};
            *reinterpret_cast<u32x2*>(hr + a.ldh) = u32x2{lo[0], lo[1]};
          }
        }
      } else if constexpr (kGrouped == kDownTerms) {
        // Token columns 2p and 2p+1 are the two terms of pair p: add the
        // neighbouring column, then the even lanes store the pair's outputs.
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int j = 16 * c + i;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            f32x4 v = acc[r][c];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += __shfl_xor(v[e], 1, 64);
            const int64_t row0 = tix[r] * 16 + 4 * kb;
            if (j < cnt && (i & 1) == 0) {
              float* pr = a.part + (int64_t)pairs[(slice + j) >> 1] * a.ldp;
              if (row0 + 3 < a.n) {
                *reinterpret_cast<f32x4*>(pr + row0) = v;
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (row0 + e < a.n) pr[row0 + e] = v[e];
              }
            }
          }
        }
      } else {
        // D layout: lane l holds rows 4*(l/16)+v (v = 0..3) of the tile for token l%16.
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int j = 16 * c + i;
          if (j < cnt) {
            float* yr = ybase + (int64_t)yrow(j) * a.ldy;
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const int64_t row0 = tix[r] * 16 + 4 * kb;
              if (a.vec_y && row0 + 3 < a.n) {
                *reinterpret_cast<f32x4*>(yr + row0) = acc[r][c];
              } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  if (row0 + v < a.n) yr[row0 + v] = acc[r][c][v];
              }
            }
          }
        }
      }
    }
    __syncthreads();   // LDS is rewritten by the next slice
  }
}

// Wide products: dense, 17..64 tokens per slice (2..4 column tiles), whole
// 512-k steps.  One wave per SIMD (a block of 4 waves) owns kWideRows row
// tiles, so each activation element staged in LDS meets kWideRows weight tiles
// and a launch on a vocabulary-sized matrix has about one row group per SIMD
// per round.  Activations stream through two LDS buffers with direct-to-LDS
// loads (one load instruction moves one token's 1 KB step slice; lane l's 16
// bytes land at 16*l), weights through two register sets, and the step's
// matrix-core work is software-pipelined against the dequantisation.  Step
// advances ride in scalar offsets, so the loop does no vector address work.
#ifdef Q3_WIDE_MIN_NT
constexpr int kWideMinNT = Q3_WIDE_MIN_NT;
#else
constexpr int kWideMinNT = 2;
#endif
constexpr int kWideWaves = 4;

template <int NT, int R>
__global__ __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(1)))
void wide_kernel(KArgs a) {
  constexpr int kW = kWideWaves, kSlice = 16 * NT;
  constexpr uint32_t rstride = 1024u + kRowPad;
  constexpr uint32_t buf_bytes = (uint32_t)kSlice * rstride;
  constexpr uint32_t zero_base = 2u * buf_bytes;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kb = lane >> 4;

  const uint32_t gp = (uint32_t)a.G;   // a multiple of 16 here
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t tile0 = ((int64_t)blockIdx.x * kW + wave) * R;
  Planes p;
  p.code = make_rsrc(a.code, (uint32_t)(tiles * 192 * gp));
  p.scale = make_rsrc(a.scale, (uint32_t)(tiles * 16 * gp));
  p.full_steps = p.steps = (int)(gp / 16);
  p.q_last = 4;
  // Steps [s_begin, s_end) of this K split (blockIdx.z) and its output plane.
  const int s_begin = (int)(blockIdx.z * p.steps / gridDim.z);
  const int s_end = (int)((blockIdx.z + 1) * p.steps / gridDim.z);
  float* const ybase = a.y + (int64_t)blockIdx.z * a.split_stride;
  const rsrc_t cbr = make_rsrc(a.cb, (uint32_t)(a.n * 8));
  RowTile rt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t T = tile0 + r;
    const bool tile_ok = T < tiles;
    rt[r].vcode = tile_ok ? (uint32_t)T * (192u * gp) + 16u * lane : kOob;
    rt[r].vscale = tile_ok ? (uint32_t)T * (16u * gp) + 4u * lane : kOob;
    const int64_t row = T * 16 + i;
    const u32x2 cb = bload64(cbr, row < a.n ? (uint32_t)row * 8u : kOob);
    rt[r].cbl = cb.x;
    rt[r].cbh = cb.y;
  }
  const rsrc_t xr = make_rsrc(a.x, (uint32_t)((a.x_rows - 1) * a.ldx * 2 + (int64_t)a.G * 64));
  const uint32_t ldx_bytes = (uint32_t)(a.ldx * 2);
  const uint32_t lane16 = 16u * (uint32_t)lane;
  if (tid < 64) *reinterpret_cast<u32x4*>(lds + zero_base + 16u * tid) = u32x4{0u, 0u, 0u, 0u};

  for (int slice = 0; slice < a.m; slice += kSlice) {
    const int cnt = a.m - slice < kSlice ? a.m - slice : kSlice;
    uint32_t xb0[NT], xb1[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int j = 16 * c + i;
      xb0[c] = (j < cnt ? (uint32_t)j * rstride : zero_base) + 256u * kb;
      xb1[c] = (j < cnt ? buf_bytes + (uint32_t)j * rstride : zero_base) + 256u * kb;
    }
    f32x4 acc[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The loads of step sn: weights into dst, activations into the LDS buffer
    // at buf.  Every wave moves kSlice/kW activation rows per step; rows of
    // absent tokens, and every load when sn is past the last step, read out
    // of range (zeros, no memory traffic) and are never used.
    constexpr int kLoads = 4 * R + kSlice / kW;
    auto loads_of = [&](StepData<R>& dst, uint32_t buf, int sn) {
      const bool live = sn < s_end;
      const uint32_t sc = (uint32_t)(live ? sn : s_end - 1);
      return [&, buf, live, sc](auto q) {
        constexpr int Q = decltype(q)::value;
        if constexpr (Q < 3 * R) {
          constexpr int r = Q / 3, j = Q % 3;
          dst.w[r][j] = __builtin_amdgcn_raw_buffer_load_b128(p.code, live ? rt[r].vcode + 1024u * j : kOob, 3072u * sc,
                                                              Q3_STREAM_POLICY);
        } else if constexpr (Q < 4 * R) {
          constexpr int r = Q - 3 * R;
          dst.sc[r] = __builtin_amdgcn_raw_buffer_load_b32(p.scale, live ? rt[r].vscale : kOob, 256u * sc,
                                                           Q3_STREAM_POLICY);
        } else {
          const int j = wave + kW * (Q - 4 * R);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (__attribute__((address_space(3))) void*)(lds + buf + (uint32_t)j * rstride), 16,
              live && j < cnt ? lane16 : kOob, (uint32_t)(slice + (j < cnt ? j : 0)) * ldx_bytes + 1024u * sc, 0, 0);
        }
      };
    };
    // Pairs of steps (A/B register sets, LDS buffers 0/1); an odd last step
    // runs after the loop, so the loop has a single exit (an exit between the
    // halves doubles the accumulators' register footprint).
    StepData<R> A, B;
    {
      auto first = loads_of(A, 0u, s_begin);
      issue_range<0, kLoads>(first);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int s = s_begin;
    for (; s + 1 < s_end; s += 2) {
      mfma_step_pipe<NT, R, kLoads>(A, rt, xb0, lds, acc, loads_of(B, buf_bytes, s + 1));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      mfma_step_pipe<NT, R, kLoads>(B, rt, xb1, lds, acc, loads_of(A, 0u, s + 2));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (s < s_end) mfma_step_pipe<NT, R, 0>(A, rt, xb0, lds, acc, [](auto) {});

    // D layout: lane l holds rows 4*(l/16)+v (v = 0..3) of the tile for token l%16.
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int j = 16 * c + i;
      if (j < cnt) {
        float* yr = ybase + (int64_t)(slice + j) * a.ldy;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t row0 = (tile0 + r) * 16 + 4 * kb;
          if (a.vec_y && row0 + 3 < a.n) {
            *reinterpret_cast<f32x4*>(yr + row0) = acc[r][c];
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (row0 + v < a.n) yr[row0 + v] = acc[r][c][v];
          }
        }
      }
    }
  }
}

// Wide products at two waves per SIMD, in half-steps.  With one block per CU
// a wide launch is bound by its weight stream more than by its arithmetic
// (measured on a 64-token vocabulary projection with one 8-wave block per CU:
// its loads alone, with no dequantisation and no MFMA, took 95 of its 98 us),
// because the block drains all of its loads at every step's barrier.  Here a block's activations are staged half
// a step at a time (the first two groups of every quad, then the last two), so
// the double buffer takes 64 KB and two blocks share a CU: the two blocks'
// barriers fall at unrelated times, and while one waits for its loads the
// other computes.  Each wave keeps R row tiles for all of K.
//
// LDS layout of a half-step buffer: token t's 512 bytes (four 64-k runs, one
// per quad kb) are 32 chunks of 8 activations, chunk c = 8 kb + 4 tt + e
// (group 2h + tt of quad kb, k 8e..8e+7) stored at position c ^ (t & 15): the
// 16 tokens of a column tile then read one chunk from 16 different bank
// groups.  One direct-to-LDS load moves 1 KB, tokens 2q and 2q+1.
template <int R>
struct HalfStep {
  u32x2 w[R][3];     // w[r][j][tt] = word j of the lane's group 2h+tt of row tile r
  uint32_t sc[R];    // bytes 0, 1: the scales of those two groups (bytes 2, 3 of a first half-step: the second's)
};

// Selectors, codebook lookup and exact bf16 widening of weights 8e..8e+7 of
// one group (one MFMA's A operand); the same selector rule as the whole-group
// unpacking.
template <int E>
__device__ __forceinline__ bf16x8 dequant_chunk(uint32_t d0, uint32_t d1, uint32_t d2, float sc, uint32_t cbl,
                                                uint32_t cbh) {
  constexpr uint32_t m3 = 0x07070707u;
  uint32_t src;
  if constexpr (E == 0) src = d0;
  else if constexpr (E == 1) src = d1;
  else if constexpr (E == 2) src = d2;
  else src = ((d0 >> 6) & 0x03030303u) | ((d1 >> 4) & 0x0C0C0C0Cu) | ((d2 >> 2) & 0x30303030u);
  const uint32_t qa = lookup4(cbl, cbh, src & m3), qb = lookup4(cbl, cbh, (src >> 3) & m3);
  return pack_bf16x8(fp8x2_to_bf16x2(qa, sc, false), fp8x2_to_bf16x2(qa, sc, true), fp8x2_to_bf16x2(qb, sc, false),
                     fp8x2_to_bf16x2(qb, sc, true));
}

// The lane's row codebook of each of the wave's row tiles.
struct RowCb {
  uint32_t lo, hi;
};

constexpr uint32_t kHalfTokenBytes = 512;   // one token's activations of one half-step
constexpr int kKeepPolicy = 1;               // work-group scope (sc0), no non-temporal hint

// Chunk CH = 4 tt + e of a half-step: B operands of the NT column tiles, then
// the chunk's dequantisation and 4 MFMAs for each row tile.  xrow: the lane's
// token row in the buffer plus 16 * ((8 kb) ^ (i & 8)); i7 = i & 7.
template <int NT, int R, int kLoads, int CH, typename Issue>
__device__ __forceinline__ void wide_hs_chunk(const HalfStep<R>& d, const RowCb (&cb)[R], uint32_t xrow, uint32_t i7,
                                            const uint8_t* lds, f32x4 (&acc)[R][NT], Issue& issue) {
  if constexpr (CH < 8) {
    constexpr int tt = CH / 4, e = CH % 4;
    // The next half-step's loads go out an eighth per chunk (issued all at
    // once, or in the first half of the chunks, the wave stalls on them: 5-10%
    // slower), and stay in their chunk: left alone, the scheduler sinks them
    // to the end, where the closing wait exposes their whole latency.
    constexpr int q0 = CH * kLoads / 8, q1 = (CH + 1) * kLoads / 8;
    issue_range<q0, q1>(issue);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t xa = xrow + 16u * ((uint32_t)CH ^ i7);
    bf16x8 b[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c)
      b[c] = *reinterpret_cast<const bf16x8*>(lds + xa + (uint32_t)c * 16u * kHalfTokenBytes);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sc = e8m0_to_f32((d.sc[r] >> (8 * tt)) & 0xFFu);
      const bf16x8 a = dequant_chunk<e>(d.w[r][0][tt], d.w[r][1][tt], d.w[r][2][tt], sc, cb[r].lo, cb[r].hi);
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[c], acc[r][c], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    wide_hs_chunk<NT, R, kLoads, CH + 1>(d, cb, xrow, i7, lds, acc, issue);
  }
}

template <int NT, int R, int kLoads, typename Issue>
__device__ __forceinline__ void wide_hs_half(const HalfStep<R>& d, const RowCb (&cb)[R], uint32_t xrow, uint32_t i7,
                                           const uint8_t* lds, f32x4 (&acc)[R][NT], Issue&& issue) {
  wide_hs_chunk<NT, R, kLoads, 0>(d, cb, xrow, i7, lds, acc, issue);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NT; ++c) asm volatile("" : "+v"(acc[r][c]));
}

constexpr int kWideHsWaves = 4;

size_t wide_hs_bytes(int slice) { return 2u * (size_t)slice * kHalfTokenBytes; }

template <int NT, int R>
__global__ __launch_bounds__(64 * kWideHsWaves) __attribute__((amdgpu_waves_per_eu(2)))
void wide_hs_kernel(KArgs a) {
  constexpr int kW = kWideHsWaves, kSlice = 16 * NT;
  constexpr uint32_t buf_bytes = (uint32_t)kSlice * kHalfTokenBytes;
  static_assert(kSlice % (2 * kW) == 0, "two tokens per activation load, spread evenly over the waves");
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kb = lane >> 4;

  const uint32_t gp = (uint32_t)a.G;   // a multiple of 16 here
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t tile0 = ((int64_t)blockIdx.x * kW + wave) * R;
  const rsrc_t code = make_rsrc(a.code, (uint32_t)(tiles * 192 * gp));
  const rsrc_t scale = make_rsrc(a.scale, (uint32_t)(tiles * 16 * gp));
  const int steps = (int)(gp / 16);
  const int s_begin = (int)(blockIdx.z * steps / gridDim.z);
  const int s_end = (int)((blockIdx.z + 1) * steps / gridDim.z);
  float* const ybase = a.y + (int64_t)blockIdx.z * a.split_stride;
  const rsrc_t cbr = make_rsrc(a.cb, (uint32_t)(a.n * 8));
  // Row tiles past the matrix read the last tile again (their outputs are
  // never stored), so a tile's plane offsets stay wave-uniform (the loads'
  // scalar offsets) and the lane's part is shared by all of them.
  uint32_t tcode[R], tscale[R];
  RowCb cb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t T = tile0 + r < tiles ? tile0 + r : tiles - 1;
    tcode[r] = (uint32_t)T * (192u * gp);
    tscale[r] = (uint32_t)T * (16u * gp);
    const int64_t row = (tile0 + r) * 16 + i;
    const u32x2 c2 = bload64(cbr, row < a.n ? (uint32_t)row * 8u : kOob);
    cb[r].lo = c2.x;
    cb[r].hi = c2.y;
  }
  const uint32_t vcode = 16u * lane, vscale = 4u * lane;
  const rsrc_t xr = make_rsrc(a.x, (uint32_t)((a.x_rows - 1) * a.ldx * 2 + (int64_t)a.G * 64));
  const uint32_t ldx_bytes = (uint32_t)(a.ldx * 2);
  // Activation loads: this wave moves tokens 2q, 2q+1 for q = wave + kW*j;
  // lane l takes token 2q + l/32 and the chunk stored at position l%32.  The
  // position-to-chunk map depends on the token's low four bits, which for
  // this wave's loads take two values (j even, j odd).
  uint32_t xsrc[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t t = 2u * (uint32_t)(wave + kW * par) + (uint32_t)(lane >> 5);
    const uint32_t c = ((uint32_t)lane & 31u) ^ (t & 15u);
    xsrc[par] = (uint32_t)(lane >> 5) * ldx_bytes + 256u * (c >> 3) + 16u * (c & 7u);
  }
  const uint32_t i7 = (uint32_t)i & 7u;

  for (int slice = 0; slice < a.m; slice += kSlice) {
    const int cnt = a.m - slice < kSlice ? a.m - slice : kSlice;
    const uint32_t xrow0 = (uint32_t)i * kHalfTokenBytes + 16u * ((8u * (uint32_t)kb) ^ ((uint32_t)i & 8u));
    const uint32_t xrow1 = xrow0 + buf_bytes;
    f32x4 acc[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The loads of half-step (sn, H): this wave's code words and scales into
    // dst, and its share of the activation rows into the LDS buffer at buf.
    // A half-step past the last reads out of range (zeros, no traffic); rows
    // of absent tokens hold zeros and only reach output columns never stored.
    constexpr int kLoads = 4 * R + kSlice / (2 * kW);
    HalfStep<R> A, B;   // A: first half-steps, B: second half-steps
    auto loads_of = [&](HalfStep<R>& dst, uint32_t buf, int sn, auto hc) {
      const bool live = sn < s_end;
      const uint32_t sc = (uint32_t)(live ? sn : s_end - 1);
      const uint32_t vc = live ? vcode + 8u * decltype(hc)::value : kOob;
      const uint32_t vs = live ? vscale : kOob;
      using Half = decltype(hc);
      return [&, buf, live, sc, vc, vs](auto q) {
        constexpr uint32_t H = Half::value;
        // The first half-step reads the first 8 bytes of every 16-byte piece
        // and the second the rest, half a step later.  Non-temporal loads in
        // the first half let the lines go before the second half reads them
        // (twice the algorithmic bytes fetched, measured): only the second
        // half of a piece is read with the streaming policy.
        constexpr int kPol = H == 0 ? kKeepPolicy : Q3_STREAM_POLICY;
        constexpr int Q = decltype(q)::value;
        if constexpr (Q < 3 * R) {
          constexpr int r = Q / 3, j = Q % 3;
          dst.w[r][j] = __builtin_amdgcn_raw_buffer_load_b64(code, vc + 1024u * j, tcode[r] + 3072u * sc, kPol);
        } else if constexpr (Q < 4 * R) {
          constexpr int r = Q - 3 * R;
          // The four scale bytes of the lane's quad come in with the first
          // half-step; the second takes bytes 2 and 3 of the same word.
          if constexpr (H == 0) dst.sc[r] = __builtin_amdgcn_raw_buffer_load_b32(scale, vs, tscale[r] + 256u * sc, kPol);
          else {
            (void)vs;
            dst.sc[r] = A.sc[r] >> 16;
          }
        } else {
          constexpr int jq = Q - 4 * R;
          const int qi = wave + kW * jq;                 // this load moves tokens 2qi, 2qi+1
          const int t = 2 * qi + (lane >> 5);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (__attribute__((address_space(3))) void*)(lds + buf + (uint32_t)qi * 1024u), 16,
              live && t < cnt ? xsrc[jq & 1] + 128u * H : kOob,
              (uint32_t)(slice + (2 * qi < cnt ? 2 * qi : 0)) * ldx_bytes + 1024u * sc, 0, 0);
        }
      };
    };
    {
      auto first = loads_of(A, 0u, s_begin, std::integral_constant<uint32_t, 0>{});
      issue_range<0, kLoads>(first);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = s_begin; s < s_end; ++s) {
      wide_hs_half<NT, R, kLoads>(A, cb, xrow0, i7, lds, acc,
                                loads_of(B, buf_bytes, s, std::integral_constant<uint32_t, 1>{}));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      wide_hs_half<NT, R, kLoads>(B, cb, xrow1, i7, lds, acc,
                                loads_of(A, 0u, s + 1, std::integral_constant<uint32_t, 0>{}));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    // D layout: lane l holds rows 4*(l/16)+v (v = 0..3) of the tile for token l%16.
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int j = 16 * c + i;
      if (j < cnt) {
        float* yr = ybase + (int64_t)(slice + j) * a.ldy;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t row0 = (tile0 + r) * 16 + 4 * kb;
          if (a.vec_y && row0 + 3 < a.n) {
            *reinterpret_cast<f32x4*>(yr + row0) = acc[r][c];
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (row0 + v < a.n) yr[row0 + v] = acc[r][c][v];
          }
        }
      }
    }
  }
}

// ---- host side ------------------------------------------------------------------

size_t full_k_bytes(int tokens, int groups) {
  const size_t gp = (size_t)((groups + 3) & ~3);
  return (size_t)tokens * (gp * 64 + kRowPad) + 1024;
}

size_t stream_bytes(int slice) { return 2u * slice * (1024u + kRowPad) + 1024u; }

size_t reduce_bytes(int vals, int r, int w) { return (size_t)w * r * vals * 64 * 4; }

// Dynamic LDS above 64 KB must be allowed per kernel and device.
template <int NT, int R, int kW, int kGrouped, int kMode, bool kDot, int kBits>
hipError_t allow_lds(size_t bytes) {
  static LdsAllowance seen;   // per kernel instantiation
  return allow_dynamic_lds(reinterpret_cast<const void*>(linear_kernel<NT, R, kW, kGrouped, kMode, kDot, kBits>),
                           bytes, seen);
}

template <int NT, int R, int kW, int kGrouped, int kMode, bool kDot, int kBits>
hipError_t launch_one(const KArgs& a, size_t shm, unsigned grid_y, unsigned grid_z, hipStream_t s) {
  const int rb = kW / (kMode != kStream ? a.sk : 1);
  const int64_t tiles = (a.n + 15) / 16;
  const int64_t groups = (tiles + R - 1) / R;   // row groups of R tiles
  const dim3 grid((unsigned)((groups + rb - 1) / rb), grid_y, grid_z);
  hipError_t e = allow_lds<NT, R, kW, kGrouped, kMode, kDot, kBits>(shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((linear_kernel<NT, R, kW, kGrouped, kMode, kDot, kBits>), grid, dim3(64 * kW), shm, s, a);
  return hipGetLastError();
}

template <int NT, int R>
hipError_t launch_wide(const KArgs& a, unsigned splits, hipStream_t s) {
  constexpr int kRowsPerBlock = R * kWideWaves;
  const size_t shm = stream_bytes(16 * NT);
  static LdsAllowance seen;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(wide_kernel<NT, R>), shm, seen);
  if (e != hipSuccess) return e;
  const int64_t tiles = (a.n + 15) / 16;
  const dim3 grid((unsigned)((tiles + kRowsPerBlock - 1) / kRowsPerBlock), 1, splits);
  hipLaunchKernelGGL((wide_kernel<NT, R>), grid, dim3(64 * kWideWaves), shm, s, a);
  return hipGetLastError();
}

template <int NT, int R>
hipError_t launch_wide_hs(const KArgs& a, unsigned splits, hipStream_t s) {
  constexpr int kRowsPerBlock = R * kWideHsWaves;
  const size_t shm = wide_hs_bytes(16 * NT);
  static LdsAllowance seen;
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(wide_hs_kernel<NT, R>), shm, seen);
  if (e != hipSuccess) return e;
  const int64_t tiles = (a.n + 15) / 16;
  const dim3 grid((unsigned)((tiles + kRowsPerBlock - 1) / kRowsPerBlock), 1, splits);
  hipLaunchKernelGGL((wide_hs_kernel<NT, R>), grid, dim3(64 * kWideHsWaves), shm, s, a);
  return hipGetLastError();
}

// Sum of the K splits' partial planes in split order: y[r][c] = sum_z
// part[z][r][c] (part rows of n floats, planes m*n apart), for S splits (a
// power of two up to kMaxSplits).  Four columns per thread; every plane's
// values are loaded before the first add, so the splits cost one memory
// latency, not one each.
constexpr int kMaxSplits = 16;
template <int S>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* part, int64_t m, int64_t n, float* y,
                                                           int64_t ldy, int vec) {
  const int64_t nq = (n + 3) / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * nq) return;
  const int64_t r = e / nq, c = 4 * (e - r * nq);
  const int64_t plane = m * n;
  const float* src = part + r * n + c;
  float* dst = y + r * ldy + c;
  if (vec && c + 3 < n) {
    f32x4 v[S];
#pragma unroll
    for (int z = 0; z < S; ++z) v[z] = *reinterpret_cast<const f32x4*>(src + z * plane);
    f32x4 acc = v[0];
#pragma unroll
    for (int z = 1; z < S; ++z) acc += v[z];
    *reinterpret_cast<f32x4*>(dst) = acc;
  } else {
    const int qn = n - c < 4 ? (int)(n - c) : 4;   // columns of this thread
    float v[4][S];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int z = 0; z < S; ++z) v[q][z] = src[z * plane + (q < qn ? q : 0)];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float acc = v[q][0];
#pragma unroll
      for (int z = 1; z < S; ++z) acc += v[q][z];
      if (q < qn) dst[q] = acc;
    }
  }
}

// Launch shape: R row tiles per wave, W waves per block, K split sk (full-K
// only).  Measured on MI355X over the decode shapes: tall matrices stream best
// with one row tile per wave in 8-wave blocks on the matrix cores (K=8192
// N=28672: 19.5 -> 18.9 us, K=4096 N=151936: 44.5 -> 43.2 us against two row
// tiles per wave in 4-wave blocks) and in 4-wave blocks on the vector ALUs (a
// 4096 x 4096 launch already fills the chip with one row tile per wave and a
// 4-way K split); activations that do not fit in LDS stream through 8-wave
// blocks.
struct Shape {
  int r, w, sk;
};

Shape pick_shape(int64_t n, int groups, bool full_k, int tokens, bool dot) {
  const int64_t tiles = (n + 15) / 16;
  const int steps = (((groups + 3) & ~3) + 15) / 16;
#if defined(Q3_FORCE_R) && defined(Q3_FORCE_W) && defined(Q3_FORCE_SK)
  (void)tiles;
  (void)steps;
  (void)tokens;
  (void)dot;
  return Shape{Q3_FORCE_R, Q3_FORCE_W, full_k ? Q3_FORCE_SK : 1};
#else
  if (!full_k) return Shape{!dot && tokens > 32 && tiles >= 4096 ? 2 : 1, 8, 1};
  if (tiles >= 1024) return dot ? Shape{1, 4, 1} : Shape{1, 8, 1};
  // Small matrices: split K over the block's waves up to about 1024 waves
  // (2048 when each wave has several tokens to multiply).
  const int64_t target = tokens > 4 ? 2048 : 1024;
  int sk = 1;
  while (sk < 8 && sk * 2 <= steps && tiles * sk < target) sk *= 2;
  return Shape{1, sk > 4 ? 8 : 4, sk};
#endif
}

// Block shape of the expert passes: one 16-row tile (two for the SwiGLU pass)
// per wave, four waves, the whole K per wave.
#ifdef Q3_EXPERT_SK
constexpr int kExpertSplitK = Q3_EXPERT_SK;
#else
constexpr int kExpertSplitK = 1;
#endif
#ifdef Q3_EXPERT_W
constexpr int kExpertWaves = Q3_EXPERT_W;
#else
constexpr int kExpertWaves = 4;
#endif
#ifdef Q3_EXPERT_STREAM
constexpr bool kExpertStream = true;
#else
constexpr bool kExpertStream = false;
#endif

template <int NT, int R, int kGrouped, bool kDot, int kBits>
hipError_t launch_r(KArgs a, int w, int mode, size_t shm, unsigned grid_y, unsigned splits, hipStream_t s) {
  if constexpr (kGrouped != kDense) {   // expert passes: one block shape
    if (mode == kShared) return launch_one<NT, R, kExpertWaves, kGrouped, kShared, kDot, kBits>(a, shm, grid_y, 1, s);
    return launch_one<NT, R, kExpertWaves, kGrouped, kStream, kDot, kBits>(a, shm, grid_y, 1, s);
  } else {
    switch (mode) {
      case kShared:
        if (w == 8) return launch_one<NT, R, 8, kGrouped, kShared, kDot, kBits>(a, shm, grid_y, 1, s);
        return launch_one<NT, R, 4, kGrouped, kShared, kDot, kBits>(a, shm, grid_y, 1, s);
      default:
        if (w == 8) return launch_one<NT, R, 8, kGrouped, kStream, kDot, kBits>(a, shm, grid_y, splits, s);
        return launch_one<NT, R, 4, kGrouped, kStream, kDot, kBits>(a, shm, grid_y, splits, s);
    }
  }
}


// tokens_in_slice: tokens the LDS staging holds at once.  wide_rows, splits
// and halfstep (dense matrix-core products of streamed activations only): row
// tiles per wave of the wide kernel (5, 2 or 1), K splits over blocks, each
// writing the partial plane a.y + z * a.split_stride, and the half-step
// variant of the five-tile kernel (three or four column tiles).
template <int NT, int kGrouped, bool kDot, int kBits = 3>
hipError_t launch_cfg(KArgs a, int tokens_in_slice, unsigned grid_y, hipStream_t s, int wide_rows = 5,
                      unsigned splits = 1, bool halfstep = false) {
  constexpr int kSlice = kDot ? NT : 16 * NT;
  const size_t fk = full_k_bytes(tokens_in_slice, a.G);
  const bool full_k = fk <= (size_t)kFullKBudget && !(kGrouped && kExpertStream);
  const Shape sh = kGrouped ? Shape{kGrouped == kSwiGLU ? 2 : 1, kExpertWaves, kExpertSplitK}
                            : pick_shape(a.n, a.G, full_k, tokens_in_slice, kDot);
  a.sk = full_k ? sh.sk : 1;
  // Streamed activations in one pass on fewer than 1536 row tiles: 4-wave
  // blocks, twice as many as with 8 (measured: 8192 x 28672 at 16 tokens
  // 65.0 -> 49.7 us, 14336 x 8192 21.6 -> 16.9 us, 4096 x 8192 20.8 -> 15.9 us;
  // 28672 x 8192 the same either way).  Products split over blocks keep the
  // 8-wave blocks their split count was planned for.
  Shape shape = sh;
  if (!kGrouped && !full_k && splits == 1 && (a.n + 15) / 16 < 1536) shape.w = 4;
  const int steps = (((a.G + 3) & ~3) + 15) / 16;
  while (a.sk > 1 && a.sk > steps) a.sk /= 2;   // every wave gets at least one step
  if (a.sk < 1 || a.sk > shape.w || shape.w % a.sk != 0) return hipErrorInvalidValue;
  const int mode = full_k ? kShared : kStream;
#ifndef Q3_NO_WIDE
  // Two or more column tiles of streamed activations on whole steps: the wide
  // kernel (one wave per SIMD, many row tiles, activations loaded into LDS).
  if constexpr (!kGrouped && !kDot && kBits == 3 && NT >= kWideMinNT) {
    if (mode == kStream && a.G % 16 == 0) {
      if (wide_rows == 1) return launch_wide<NT, 1>(a, splits, s);
      if constexpr (NT >= 3) {
        if (halfstep && wide_rows == 5) return launch_wide_hs<NT, 5>(a, splits, s);
      }
      return wide_rows == 2 ? launch_wide<NT, 2>(a, splits, s) : launch_wide<NT, 5>(a, splits, s);
    }
  }
#endif
  if (mode == kShared) splits = 1;
  size_t shm = mode == kShared ? fk : stream_bytes(kSlice);
  if (mode != kStream && a.sk > 1) {
    const size_t red = reduce_bytes(kDot ? NT : 4 * NT, shape.r, shape.w);
    if (shm < red) shm = red;
  }
  if constexpr (kGrouped == kSwiGLU) {
    return launch_r<NT, 2, kGrouped, kDot, kBits>(a, shape.w, mode, shm, grid_y, 1, s);
  } else if constexpr (kGrouped || kDot) {
    return launch_r<NT, 1, kGrouped, kDot, kBits>(a, shape.w, mode, shm, grid_y, splits, s);
  } else {
    switch (shape.r) {
      case 1: return launch_r<NT, 1, kGrouped, kDot, kBits>(a, shape.w, mode, shm, grid_y, splits, s);
      case 2: return launch_r<NT, 2, kGrouped, kDot, kBits>(a, shape.w, mode, shm, grid_y, splits, s);
      default: return hipErrorInvalidValue;
    }
  }
}

// Token rows an expert block stages at once: with distinct experts per token
// (top-k routing) an expert has at most t pairs, so t rows (times the terms per
// pair) cover it; more pairs (repeated ids) take further slices.  Even and at
// most 16 (one matrix-core column tile).
// Grid rows of an expert pass: with at most 64 experts, row y takes the
// round's y-th distinct picked expert, so no more rows than pairs are needed;
// past 64 experts, row e is expert e.
unsigned expert_rows(int num_experts, int pairs) {
  return (unsigned)(num_experts <= 64 && pairs < num_experts ? pairs : num_experts);
}

int expert_slice(int t, int pairs, int terms) {
  int c = (t < pairs ? t : pairs) * terms;
  c = c < 16 ? c : 16;
  c = c < 2 ? 2 : c;
  return c + (c & 1);
}

KArgs base_args(const PlaneView& w) {
  KArgs a{};
  a.code = w.code;
  a.scale = w.scale;
  a.cb = w.cb;
  a.n = w.n;
  a.G = w.groups;
  return a;
}

// Launch plan of a dense matrix-core product (1..64 tokens).  Activations that
// fit in LDS whole are staged once per block and K is split over the waves of
// a block.  Streamed activations put whole row groups in a block: on a matrix
// with few of them the grid would leave most of the chip idle, so K is split
// over the blocks of a grid column as well (partial planes in a workspace,
// then a fixed-order sum), and the wide kernel may take two row tiles per
// wave instead of five.  Splits stop at 128 blocks (wide) or 192 (8-wave stream
// blocks) and at two steps per split: measured on MI355X, more splits cost
// more in partial planes and per-block start-up than they gain (N = 8192,
// K = 28672, 16 tokens: 65.7 us in one pass, 28.7 us in 4 splits; a grid of
// 224 blocks or more is faster unsplit).
#ifndef Q3_SPLIT_TARGET_WIDE
#define Q3_SPLIT_TARGET_WIDE 128
#endif
#ifndef Q3_SPLIT_TARGET_STREAM
#define Q3_SPLIT_TARGET_STREAM 192
#endif
#ifndef Q3_SPLIT_MIN_STEPS
#define Q3_SPLIT_MIN_STEPS 2
#endif
struct SmallMPlan {
  int wide_rows;   // row tiles per wave of the wide kernel (1, 2 or 5)
  int splits;      // K splits over blocks
  bool halfstep;   // five row tiles in half-steps, two blocks per CU
};

// Blocks of the five-tile wide kernel from which its half-step variant (two
// blocks per CU) is the faster one, at three or four column tiles.  Measured
// at 64 tokens and K = 4096: 151,936 rows (475 blocks) 94.2 -> 89.8 us,
// 131,072 rows (410) 90.4 -> 82.6 us; 65,536 rows (205) 43.7 -> 50.8 us, where
// most CUs run a single block and the half-step kernel's extra barriers and
// 8-byte loads are not repaid.
constexpr int64_t kHalfStepMinBlocks = 400;

SmallMPlan plan_small_m(int64_t n, int groups, int64_t m) {
  SmallMPlan pl{5, 1, false};
  if (n <= 0) return pl;
  const int nt = (int)((m + 15) / 16);
  if (full_k_bytes((int)m, groups) <= (size_t)kFullKBudget) return pl;   // staged whole: no split
  const int64_t tiles = (n + 15) / 16;
  const int steps = (((groups + 3) & ~3) + 15) / 16;
  int64_t blocks, target;
  if (nt >= kWideMinNT && groups % 16 == 0) {
    // Rounds of 256 blocks (one block per CU: the activation buffers take
    // 134 KB of LDS) times the block's time: a five-tile block costs about
    // 1.8x a two-tile one (measured at 64 tokens: 9 and 12.5 us per round
    // and row tile), so five row tiles win only where they do not add a
    // nearly empty round (N = 65536: 46 vs 50 us; N = 98304: 89 vs 74 us).
    const int64_t blocks5 = (tiles + 19) / 20;
    const bool hs = nt >= 3 && blocks5 >= kHalfStepMinBlocks;
    const int64_t slots5 = hs ? 512 : 256;
    const int64_t rounds5 = (blocks5 + slots5 - 1) / slots5, rounds2 = ((tiles + 7) / 8 + 255) / 256;
    if (rounds2 * 50 < rounds5 * 90) pl.wide_rows = 2;
    else pl.halfstep = hs;
    // 512..1535 row tiles at K <= 4096: one row tile per wave (a grid of 128
    // blocks and more) in one pass beats two tiles per wave split over blocks
    // (8192 x 4096 at 64 tokens: 17.7 -> 16.0 us; 12288 x 4096: 19.2 -> 16.4 us).
    // At K = 8192 the splits pay more (8192 x 8192: 25.4 us split, 27.0 in one pass).
    if (tiles >= 512 && tiles < 1536 && groups <= 128) {
      pl.wide_rows = 1;
      return pl;
    }
    blocks = (tiles + 4 * pl.wide_rows - 1) / (4 * pl.wide_rows);
    target = Q3_SPLIT_TARGET_WIDE;
  } else {
    const Shape sh = pick_shape(n, groups, false, (int)m, false);
    blocks = (tiles + (int64_t)sh.r * sh.w - 1) / ((int64_t)sh.r * sh.w);
    target = Q3_SPLIT_TARGET_STREAM;
  }
  while (pl.splits < 16 && blocks * pl.splits < target && steps >= 2 * pl.splits * Q3_SPLIT_MIN_STEPS) pl.splits *= 2;
  return pl;
}

}  // namespace

int64_t gemm_small_m_workspace_bytes(int64_t n, int64_t k, int64_t m) {
#ifndef Q3_NO_SPLITK
  if (splitk_applies(n, (int)(k / 32), m, false)) return 0;
#endif
  const SmallMPlan pl = plan_small_m(n, (int)(k / 32), m);
  return pl.splits > 1 ? (int64_t)pl.splits * m * n * 4 : 0;
}

hipError_t launch_gemm_small_m(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                               int64_t ldy, void* ws, int64_t ws_bytes, hipStream_t s) {
  if (w.n == 0) return hipSuccess;
#ifndef Q3_NO_SPLITK
  if (splitk_applies(w.n, w.groups, m, false)) return launch_splitk(w, x, m, ldx, y, ldy, false, s);
#endif
  KArgs a = base_args(w);
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.m = (int)m;
  a.x_rows = m;
  a.vec_y = ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  SmallMPlan pl = plan_small_m(w.n, w.groups, m);
  const int64_t need = pl.splits > 1 ? (int64_t)pl.splits * m * w.n * 4 : 0;
  if (pl.splits > 1 && (ws == nullptr || ws_bytes < need)) pl.splits = 1;   // no workspace: one pass
  // A wide product in one pass on fewer than 1536 row tiles: one row tile per
  // wave, twice the grid of two (4096 x 4096 at 64 tokens 20.9 -> 15.8 us, at
  // 32 tokens 14.8 -> 11.7 us; 4096 x 8192 at 64 tokens 36.4 -> 26.7 us; at
  // 1792 tiles two tiles per wave stay faster, 28672 x 8192: 39.8 vs 53.8 us).
  if (pl.splits == 1 && pl.wide_rows == 2 && (w.n + 15) / 16 < 1536) pl.wide_rows = 1;
  if (pl.splits > 1) {
    a.y = static_cast<float*>(ws);
    a.ldy = w.n;
    a.split_stride = m * w.n;
    a.vec_y = ((uintptr_t)ws % 16 == 0) && (w.n % 4 == 0);
  }
  hipError_t e;
  if (m <= 16) e = launch_cfg<1, kDense, false>(a, (int)m, 1, s, pl.wide_rows, pl.splits);
  else if (m <= 32) e = launch_cfg<2, kDense, false>(a, (int)m, 1, s, pl.wide_rows, pl.splits);
  else if (m <= 48) e = launch_cfg<3, kDense, false>(a, (int)m, 1, s, pl.wide_rows, pl.splits, pl.halfstep);
  else e = launch_cfg<4, kDense, false>(a, (int)m, 1, s, pl.wide_rows, pl.splits, pl.halfstep);
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t threads = m * ((w.n + 3) / 4);
  const int vec = ((uintptr_t)ws % 16 == 0) && (w.n % 4 == 0) && ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const float* part = static_cast<const float*>(ws);
  switch (pl.splits) {
    case 2: hipLaunchKernelGGL(split_reduce_kernel<2>, grid, dim3(256), 0, s, part, m, w.n, y, ldy, vec); break;
    case 4: hipLaunchKernelGGL(split_reduce_kernel<4>, grid, dim3(256), 0, s, part, m, w.n, y, ldy, vec); break;
    case 8: hipLaunchKernelGGL(split_reduce_kernel<8>, grid, dim3(256), 0, s, part, m, w.n, y, ldy, vec); break;
    case kMaxSplits:
      hipLaunchKernelGGL(split_reduce_kernel<kMaxSplits>, grid, dim3(256), 0, s, part, m, w.n, y, ldy, vec);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_head2_scores(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                               hipStream_t s) {
  if (w.n == 0) return hipSuccess;
  KArgs a = base_args(w);
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.m = (int)m;
  a.x_rows = m;
  a.vec_y = ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  return launch_cfg<1, kDense, false, 2>(a, (int)m, 1, s);
}

hipError_t launch_gemv(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t s) {
  if (w.n == 0) return hipSuccess;
#ifndef Q3_NO_SPLITK
  if (splitk_applies(w.n, w.groups, m, true)) return launch_splitk(w, x, m, ldx, y, ldy, true, s);
#endif
  KArgs a = base_args(w);
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.m = (int)m;
  a.x_rows = m;
  switch (m) {
    case 1: return launch_cfg<1, kDense, true>(a, 1, 1, s);
    case 2: return launch_cfg<2, kDense, true>(a, 2, 1, s);
    case 3: return launch_cfg<3, kDense, true>(a, 3, 1, s);
    case 4: return launch_cfg<4, kDense, true>(a, 4, 1, s);
    case 5: return launch_cfg<5, kDense, true>(a, 5, 1, s);
    case 6: return launch_cfg<6, kDense, true>(a, 6, 1, s);
    case 7: return launch_cfg<7, kDense, true>(a, 7, 1, s);
    case 8: return launch_cfg<8, kDense, true>(a, 8, 1, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_grouped(const ExpertView& w, const uint16_t* x, int64_t ldx, int32_t x_by_slot,
                          const int32_t* ids, int32_t t, int32_t topk, float* y, int64_t ldy, hipStream_t s) {
  if (w.base.n == 0) return hipSuccess;
  KArgs a = base_args(w.base);
  a.code_stride = w.code_stride;
  a.scale_stride = w.scale_stride;
  a.cb_stride = w.cb_stride;
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.ids = ids;
  a.pairs_total = t * topk;
  a.topk = topk;
  a.x_by_slot = x_by_slot;
  a.vec_y = ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  a.x_rows = x_by_slot ? (int64_t)t * topk : t;
  a.slice_cap = expert_slice(t, a.pairs_total, 1);
  a.num_experts = w.num_experts;
  return launch_cfg<1, kExperts, false>(a, a.slice_cap, expert_rows(w.num_experts, a.pairs_total), s);
}

hipError_t launch_moe_mlp(const ExpertView& gu, const ExpertView& dn, const uint16_t* x, int64_t ldx,
                          const int32_t* ids, int32_t t, int32_t topk, const float* logits, int64_t ld_logits,
                          uint16_t* h, float* part, int64_t ldp, float* out, int64_t ldo, hipStream_t s) {
  const int pairs = t * topk;
  const int64_t inter = gu.base.n / 2;
  KArgs a = base_args(gu.base);
  a.code_stride = gu.code_stride;
  a.scale_stride = gu.scale_stride;
  a.cb_stride = gu.cb_stride;
  a.x = x;
  a.ldx = ldx;
  a.x_rows = t;
  a.ids = ids;
  a.pairs_total = pairs;
  a.topk = topk;
  a.num_experts = gu.num_experts;
  a.half_tiles = (int)(inter / 16);
  a.h = h;
  a.ldh = inter;
  a.slice_cap = expert_slice(t, pairs, 1);
  hipError_t e = launch_cfg<1, kSwiGLU, false>(a, a.slice_cap, expert_rows(gu.num_experts, pairs), s);
  if (e != hipSuccess) return e;
  KArgs b = base_args(dn.base);
  b.code_stride = dn.code_stride;
  b.scale_stride = dn.scale_stride;
  b.cb_stride = dn.cb_stride;
  b.x = h;
  b.ldx = inter;
  b.x_rows = 2 * (int64_t)pairs;
  b.ids = ids;
  b.pairs_total = pairs;
  b.topk = topk;
  b.num_experts = dn.num_experts;
  b.part = part;
  b.ldp = ldp;
  b.slice_cap = expert_slice(t, pairs, 2);
  e = launch_cfg<1, kDownTerms, false>(b, b.slice_cap, expert_rows(dn.num_experts, pairs), s);
  if (e != hipSuccess) return e;
  return launch_moe_combine(part, ldp, ids, t, topk, dn.num_experts, logits, ld_logits, dn.base.n, out, ldo, s);
}

}  // namespace q3
