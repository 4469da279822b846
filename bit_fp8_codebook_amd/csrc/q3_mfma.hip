// Matrix-core decode product over the 3.25-bit codebook format, dense (1..64
// tokens) and expert-grouped (MoE verify rounds).
//
// What it computes (Hibana: Fast Agentic Inference on Unified-Memory Devices,
// "Model surgery" / "Three-bit weights"): y[m][n] = sum_k x[m][k] * w[n][k].  The
// page's own kernel looks the codes up and feeds the FP8 matrix units; here the
// looked-up E4M3 bytes are widened exactly to bf16 (group scale folded into the
// conversion) and fed to gfx950's v_mfma_f32_16x16x32_bf16, so every product is
// exact and only the fp32 accumulation rounds, whatever the activations are.
//
// Wave tile: 16 weight rows (MFMA A operand) x 16 tokens per column tile (B
// operand), fp32 accumulators in the MFMA C/D registers.  A step covers 512 k
// (one 16-group superchunk): lane l serves row l%16 and groups 4*(l/16)..+3 of
// the superchunk, whose code words arrive in three 16-byte buffer loads (word j
// of the 4 groups; the four lanes of a row read one contiguous 64-byte run per
// load) plus one 4-byte scale load.  Each group is dequantised once into 16
// bf16 pairs = the A operands of 4 MFMAs; the B operand of the same lane is the
// matching 8 activations of token 16c + l%16, read from LDS, so A and B agree
// on which k sits in which slot by construction.
//
// Activations are staged in LDS once per block ("full-K" mode) or, when they do
// not fit, one 512-k step at a time into a double buffer ("stream" mode).  The
// next step's code words are loaded before the current step is computed; all
// loads are buffer loads whose out-of-range offsets read as zero, so rows past
// n, padding groups and absent tokens need no branches.  In full-K mode the four
// waves of a block may split K (few rows); partial sums are then added through
// LDS in a fixed order, so results are run-to-run identical.
//
// The grouped variant runs one grid row per expert.  Its block first collects
// the (token, slot) pairs routed to that expert; an expert nobody picked
// returns before reading any weight byte (Hibana page, "Adaptive speculation" /
// "Expert sharing": a verify round reads every picked expert once).
#include <atomic>

#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

constexpr int kThreads = 256;
constexpr int kFullKBudget = 72 * 1024;   // LDS bytes for full-K activation staging
constexpr uint32_t kRowPad = 16;          // LDS row padding against bank conflicts

struct MfmaArgs {
  const uint8_t* code;
  int64_t code_pitch, code_stride;   // stride: bytes between experts
  const uint8_t* scale;
  int64_t scale_pitch, scale_stride;
  const uint8_t* cb;
  int64_t cb_stride;
  int64_t n;
  int G;
  const uint16_t* x;
  int64_t ldx;
  int64_t x_rows;   // rows of x that may be read
  float* y;
  int64_t ldy;
  int m;          // dense: number of tokens
  int sk;         // K split over the waves of a block (full-K mode)
  const int32_t* ids;
  int pairs_total, topk, x_by_slot;
};

__device__ __forceinline__ bf16x8 pack_bf16x8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
             __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, u);
}

// Code words and scales of one 512-k step of one row tile, for one lane.
struct WStep {
  u32x4 w[3];     // w[j][t] = word j of the lane's group t
};

// Per-lane view of one row tile's code plane.  vcode is the lane's byte offset
// of step 0 (kOob for rows past n); a step adds a wave-uniform amount, which
// keeps out-of-range lanes out of range because every plane is below 2 GiB and
// kOob is 2 GiB.
struct Tile {
  rsrc_t code;
  uint32_t vcode;        // step-0 offset: row*pitch + 16*kb
  uint32_t vcode_last;   // same for the last superchunk when it is partial
  int full_steps, steps;
  uint32_t p_last;       // groups in the last superchunk (4..16)
};

// Branch-free on purpose: loads issued under a condition make the wait-count
// insertion assume the worst case and drain every outstanding prefetch.  Steps
// past the end re-read the last step (cached, never computed).
__device__ __forceinline__ void load_step(const Tile& t, int s, WStep& ws) {
  const int sc = s < t.steps ? s : t.steps - 1;
  const bool full = sc < t.full_steps;
  const uint32_t o = (full ? t.vcode : t.vcode_last) + 192u * sc;
  const uint32_t js = full ? 64u : 4u * t.p_last;
#pragma unroll
  for (int j = 0; j < 3; ++j) ws.w[j] = bload128(t.code, o + js * j);
}

// Dequantise the step's 4 groups and run 4*4*MT MFMAs.  sc holds the 4 groups'
// scale bytes; xb[c] is the lane's LDS byte address of its B operand for column
// tile c at this step (group 0, k 0).
template <int MT>
__device__ __forceinline__ void compute_step(const WStep& ws, uint32_t sc, uint32_t cbl, uint32_t cbh,
                                             const uint32_t (&xb)[MT], const uint8_t* lds, f32x4 (&acc)[MT]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bf16x2 wv[16];
    dequant_group_bf16(ws.w[0][t], ws.w[1][t], ws.w[2][t], (sc >> (8 * t)) & 0xFFu, cbl, cbh, wv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x8 a = pack_bf16x8(wv[4 * e], wv[4 * e + 1], wv[4 * e + 2], wv[4 * e + 3]);
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(lds + xb[c] + 64u * t + 16u * e);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
      }
    }
  }
}

// Token slot j of the current slice -> x row and y row.
struct Tokens {
  int count;          // tokens in this slice (<= 16*MT)
  int xrow[64];
  int yrow[64];
};

// Copy `count` 16-byte chunks from global memory (buffer resource) into LDS.
// All loads of a batch are issued before any store, so a batch costs one
// memory latency instead of one per chunk.  src(c) returns the chunk's byte
// offset in the resource (kOob for zeros), dst(c) its LDS byte address.
template <int kBatch, typename Src, typename Dst>
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

// One-column-tile instances are held to 128 registers per lane, i.e. 4 waves
// per SIMD: a decode launch needs every wave resident at once.
template <int MT, bool kGrouped, bool kFullK>
__global__ __launch_bounds__(kThreads, MT == 1 ? 4 : 1) void mfma_kernel(MfmaArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Tokens tk;
  __shared__ int pairs[64];
  __shared__ int npairs;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform from here on
  const int i = lane & 15;
  const int kb = lane >> 4;
  const int sk = kFullK ? a.sk : 1;
  const int rb = 4 / sk;
  const int rt = wave / sk;
  const int ks = wave - rt * sk;

  // ---- which expert / tokens -------------------------------------------------
  int expert = 0;
  if (kGrouped) {
    expert = blockIdx.y;
    if (tid < 64) {
      const bool match = tid < a.pairs_total && a.ids[tid] == expert;
      const unsigned long long mask = __ballot(match);
      if (match) pairs[__popcll(mask & ((1ull << tid) - 1ull))] = tid;
      if (tid == 0) npairs = __popcll(mask);
    }
    __syncthreads();
    if (npairs == 0) return;   // not picked this round: no weight byte is read
  }
  const int total_tokens = kGrouped ? __builtin_amdgcn_readfirstlane(npairs) : a.m;

  const int G = a.G;
  const int gp = (G + 3) & ~3;
  const int64_t row_base = ((int64_t)blockIdx.x * rb + rt) * 16;
  const int64_t row = row_base + i;
  const bool row_ok = row < a.n;

  Tile t;
  t.code = make_rsrc(a.code + (int64_t)expert * a.code_stride, (uint32_t)(a.n * a.code_pitch));
  t.full_steps = gp / 16;
  t.steps = (gp + 15) / 16;
  t.p_last = (uint32_t)(gp - 16 * (t.steps - 1));
  const bool last_ok = 4u * kb < t.p_last;
  t.vcode = row_ok ? (uint32_t)row * (uint32_t)a.code_pitch + 16u * kb : kOob;
  t.vcode_last = last_ok ? t.vcode : kOob;
  const rsrc_t cbr = make_rsrc(a.cb + (int64_t)expert * a.cb_stride, (uint32_t)(a.n * 8));
  const u32x2 cb = bload64(cbr, row_ok ? (uint32_t)row * 8u : kOob);
  // Lanes past the last superchunk's groups dequantise with a zero codebook,
  // so they contribute exactly zero whatever activations they meet.
  const uint32_t cbl_last = last_ok ? cb.x : 0u, cbh_last = last_ok ? cb.y : 0u;

  const rsrc_t xr_rsrc = make_rsrc(a.x, (uint32_t)((a.x_rows - 1) * a.ldx * 2 + (int64_t)G * 64));
  const uint32_t ldx_bytes = (uint32_t)(a.ldx * 2);

  const int s0 = kFullK ? (ks * t.steps) / sk : 0;
  const int s1 = kFullK ? ((ks + 1) * t.steps) / sk : t.steps;

  // Issue the first step's code loads, then stage the block's scale rows in LDS
  // (one contiguous read per row instead of a 4-byte read per lane and step).
  // Rows past n stage zeros.  The row stride is padded so the 16 rows a wave
  // reads at once fall into different banks.
  WStep A, B;
  load_step(t, s0, A);
  load_step(t, s0 + 1, B);
  const uint32_t sstride = (((uint32_t)gp + 15u) & ~15u) + 16u;
  const int block_rows = 16 * rb;
  {
    const rsrc_t scr = make_rsrc(a.scale + (int64_t)expert * a.scale_stride, (uint32_t)(a.n * a.scale_pitch));
    const int64_t row0 = (int64_t)blockIdx.x * block_rows;
    const int cpr = (gp + 15) / 16;   // 16-byte chunks per scale row
    stage_chunks<4>(scr, block_rows * cpr, lds,
                    [&](int c) {
                      const int r = c / cpr, q = c - r * cpr;
                      return row0 + r < a.n ? (uint32_t)(row0 + r) * (uint32_t)a.scale_pitch + 16u * q : kOob;
                    },
                    [&](int c) {
                      const int r = c / cpr, q = c - r * cpr;
                      return (uint32_t)r * sstride + 16u * q;
                    });
  }
  uint8_t* const xlds = lds + block_rows * sstride;
  const uint32_t sc_lane = (uint32_t)(rt * 16 + i) * sstride + 4u * kb;

  for (int slice = 0; slice < total_tokens; slice += 16 * MT) {
    if (tid == 0) {
      const int cnt = total_tokens - slice < 16 * MT ? total_tokens - slice : 16 * MT;
      tk.count = cnt;
      for (int j = 0; j < 16 * MT; ++j) {
        if (j < cnt) {
          if (kGrouped) {
            const int q = pairs[slice + j];
            tk.xrow[j] = a.x_by_slot ? q : q / a.topk;
            tk.yrow[j] = q;
          } else {
            tk.xrow[j] = slice + j;
            tk.yrow[j] = slice + j;
          }
        } else {
          tk.xrow[j] = 0;
          tk.yrow[j] = 0;
        }
      }
    }
    __syncthreads();
    const int cnt = __builtin_amdgcn_readfirstlane(tk.count);
    if (slice > 0) {
      load_step(t, s0, A);
      load_step(t, s0 + 1, B);
    }

    f32x4 acc[MT];
#pragma unroll
    for (int c = 0; c < MT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kFullK) {
      // Stage all activations: row j holds token j's K values (zero past K,
      // including the row's 16-byte pad, which lanes past the last superchunk's
      // groups read with a zero codebook); a 1 KB zero block serves the lanes
      // of absent tokens.
      const uint32_t kp_bytes = (uint32_t)gp * 64u;
      const uint32_t rstride = kp_bytes + kRowPad;
      const uint32_t zero_base = (uint32_t)cnt * rstride;
      const int cpr = (int)(rstride / 16);
      stage_chunks<8>(xr_rsrc, cnt * cpr + 64, xlds,
                      [&](int c) {
                        const int j = c / cpr, q = c - j * cpr;
                        return j < cnt && q * 8 < G * 32 ? (uint32_t)tk.xrow[j] * ldx_bytes + 16u * q : kOob;
                      },
                      [&](int c) { return 16u * c; });   // rows are contiguous, then the zero block
      __syncthreads();

      // Lane address of step 0 and the per-step advance (0 for absent tokens,
      // which stay on the zero block).
      uint32_t xb0[MT], xstep[MT];
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        const int j = 16 * c + i;
        xb0[c] = (j < cnt ? j * rstride : zero_base) + 256u * kb;
        xstep[c] = j < cnt ? 1024u : 0u;
      }
      auto run = [&](const WStep& ws, int s) {
        uint32_t xb[MT];
#pragma unroll
        for (int c = 0; c < MT; ++c) xb[c] = xb0[c] + xstep[c] * s;
        const bool full = s < t.full_steps;
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(lds + sc_lane + 16u * s);
        compute_step<MT>(ws, sc, full ? cb.x : cbl_last, full ? cb.y : cbh_last, xb, xlds, acc);
      };
      // Two steps are in flight when the loop starts; each computed step's
      // registers are refilled with the step two ahead.  The scheduling
      // barriers keep each refill where it is issued; without them the
      // compiler sinks the loads below the MFMAs.
      for (int s = s0; s < s1; s += 2) {
        run(A, s);
        load_step(t, s + 2, A);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 >= s1) break;
        run(B, s + 1);
        load_step(t, s + 3, B);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Stream the activations one 512-k step at a time through two buffers of
      // 16*MT rows (rows of absent tokens stay zero).  Step s+1's activations
      // are fetched into registers during step s-1 and stored to LDS after
      // step s is computed, so the store never waits on a fresh load.
      const uint32_t rstride = 1024u + kRowPad;
      const uint32_t buf_bytes = 16u * MT * rstride;
      const int nchunk = 16 * MT * 64;   // 16-byte chunks per buffer
      auto fetch = [&](int s, u32x4 (&r)[MT * 4]) {
#pragma unroll
        for (int q = 0; q < MT * 4; ++q) {
          const int idx = tid + q * kThreads;
          const int j = idx >> 6, c16 = idx & 63;
          const int k0 = s * 512 + c16 * 8;
          const bool ok = idx < nchunk && j < cnt && k0 < G * 32;
          r[q] = bload128(xr_rsrc, ok ? (uint32_t)tk.xrow[j] * ldx_bytes + 2u * k0 : kOob);
        }
      };
      auto put = [&](int buf, const u32x4 (&r)[MT * 4]) {
#pragma unroll
        for (int q = 0; q < MT * 4; ++q) {
          const int idx = tid + q * kThreads;
          const int j = idx >> 6, c16 = idx & 63;
          if (idx < nchunk) *reinterpret_cast<u32x4*>(xlds + buf * buf_bytes + j * rstride + 16u * c16) = r[q];
        }
      };
      auto run = [&](const WStep& ws, int s) {
        const int buf = (s - s0) & 1;
        uint32_t xb[MT];
#pragma unroll
        for (int c = 0; c < MT; ++c) xb[c] = buf * buf_bytes + (16 * c + i) * rstride + 256u * kb;
        const bool full = s < t.full_steps;
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(lds + sc_lane + 16u * s);
        compute_step<MT>(ws, sc, full ? cb.x : cbl_last, full ? cb.y : cbh_last, xb, xlds, acc);
      };
      u32x4 xr[MT * 4];
      fetch(s0, xr);
      put(0, xr);
      fetch(s0 + 1, xr);
      __syncthreads();
      for (int s = s0; s < s1; s += 2) {
        run(A, s);
        load_step(t, s + 2, A);
        __builtin_amdgcn_sched_barrier(0);
        put((s + 1 - s0) & 1, xr);   // buffer last read at step s-1
        fetch(s + 2, xr);
        __syncthreads();
        if (s + 1 >= s1) break;
        run(B, s + 1);
        load_step(t, s + 3, B);
        __builtin_amdgcn_sched_barrier(0);
        put((s + 2 - s0) & 1, xr);
        fetch(s + 3, xr);
        __syncthreads();
      }
    }

    // ---- combine K splits and store --------------------------------------------
    if (kFullK && sk > 1) {
      __syncthreads();   // activations no longer needed: reuse LDS for partial sums
      f32x4* red = reinterpret_cast<f32x4*>(xlds);
#pragma unroll
      for (int c = 0; c < MT; ++c) red[(wave * MT + c) * 64 + lane] = acc[c];
      __syncthreads();
      if (ks == 0) {
        for (int q = 1; q < sk; ++q) {
#pragma unroll
          for (int c = 0; c < MT; ++c) acc[c] += red[((wave + q) * MT + c) * 64 + lane];
        }
      }
    }
    if (ks == 0) {
      // D layout: lane l holds rows 4*(l/16)+v (v = 0..3) of the tile for token l%16.
#pragma unroll
      for (int c = 0; c < MT; ++c) {
        const int j = 16 * c + i;
        if (j < cnt) {
          float* yr = a.y + (int64_t)tk.yrow[j] * a.ldy;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t r = row_base + 4 * kb + v;
            if (r < a.n) yr[r] = acc[c][v];
          }
        }
      }
    }
    __syncthreads();   // token table and LDS are rewritten by the next slice
  }
}

// K split over the block's waves (full-K mode): the largest split whose blocks
// are all resident at once (`capacity` blocks on the chip), so no second round
// of waves starts after the first drains; never more ways than there are
// 512-k steps.
int choose_split(int64_t n, int groups, int64_t capacity) {
  const int64_t tiles = (n + 15) / 16;
  const int steps = (((groups + 3) & ~3) + 15) / 16;
  int sk = 1;
  while (sk < 4 && (tiles * sk * 2 + 3) / 4 <= capacity && sk * 2 <= steps) sk *= 2;
  return sk;
}

// Blocks of a kernel instance that fit on the device at once.
template <int MT, bool kGrouped, bool kFullK>
int64_t resident_blocks(size_t shm) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mfma_kernel<MT, kGrouped, kFullK>, kThreads, shm) !=
          hipSuccess)
    return 1024;
  return (int64_t)cus * (per_cu > 0 ? per_cu : 1);
}

size_t scale_stage_bytes(int groups, int rb) {
  const size_t gp = (size_t)((groups + 3) & ~3);
  return (size_t)16 * rb * (((gp + 15) & ~(size_t)15) + 16);
}

size_t full_k_bytes(int tokens, int groups) {
  const size_t gp = (size_t)((groups + 3) & ~3);
  return (size_t)tokens * (gp * 64 + kRowPad) + 1024;
}

size_t stream_bytes(int mt) { return 2u * 16u * mt * (1024u + kRowPad); }

// Dynamic LDS above 64 KB must be allowed per kernel; raise each kernel's limit
// once to the largest size this file ever requests.
template <int MT, bool kGrouped, bool kFullK>
hipError_t allow_lds(size_t bytes) {
  static std::atomic<size_t> allowed{64 * 1024};   // per kernel instantiation
  if (bytes <= allowed.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_kernel<MT, kGrouped, kFullK>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) {
    size_t cur = allowed.load(std::memory_order_acquire);
    while (cur < bytes && !allowed.compare_exchange_weak(cur, bytes)) {
    }
  }
  return e;
}

template <int MT, bool kGrouped>
hipError_t launch_cfg(MfmaArgs a, int tokens_in_slice, unsigned grid_y, hipStream_t s) {
  const int64_t tiles = (a.n + 15) / 16;
  const size_t fk = full_k_bytes(tokens_in_slice, a.G);
  if (fk + scale_stage_bytes(a.G, 4) <= (size_t)kFullKBudget) {
    // LDS with the largest split's needs (the scale staging shrinks as rb does).
    size_t shm = fk;
    const size_t red = (size_t)4 * MT * 64 * 16;
    if (shm < red) shm = red;
    shm += scale_stage_bytes(a.G, 4);
    a.sk = kGrouped ? 1 : choose_split(a.n, a.G, resident_blocks<MT, kGrouped, true>(shm));
    const int rb = 4 / a.sk;
    const dim3 grid((unsigned)((tiles + rb - 1) / rb), grid_y);
    hipError_t e = allow_lds<MT, kGrouped, true>(shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mfma_kernel<MT, kGrouped, true>), grid, dim3(kThreads), shm, s, a);
  } else {
    a.sk = 1;
    const dim3 grid((unsigned)((tiles + 3) / 4), grid_y);
    const size_t shm = stream_bytes(MT) + scale_stage_bytes(a.G, 4);
    hipError_t e = allow_lds<MT, kGrouped, false>(shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mfma_kernel<MT, kGrouped, false>), grid, dim3(kThreads), shm, s, a);
  }
  return hipGetLastError();
}

MfmaArgs base_args(const PlaneView& w) {
  MfmaArgs a{};
  a.code = w.code;
  a.code_pitch = w.code_pitch;
  a.scale = w.scale;
  a.scale_pitch = w.scale_pitch;
  a.cb = w.cb;
  a.n = w.n;
  a.G = w.groups;
  return a;
}

}  // namespace

hipError_t launch_gemm_small_m(const PlaneView& w, const uint16_t* x, int64_t m, int64_t ldx, float* y,
                               int64_t ldy, hipStream_t s) {
  if (w.n == 0) return hipSuccess;
  MfmaArgs a = base_args(w);
  a.x = x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.m = (int)m;
  a.x_rows = m;
  if (m <= 16) return launch_cfg<1, false>(a, (int)m, 1, s);
  if (m <= 32) return launch_cfg<2, false>(a, (int)m, 1, s);
  if (m <= 48) return launch_cfg<3, false>(a, (int)m, 1, s);
  return launch_cfg<4, false>(a, (int)m, 1, s);
}

hipError_t launch_grouped(const ExpertView& w, const uint16_t* x, int64_t ldx, int32_t x_by_slot,
                          const int32_t* ids, int32_t t, int32_t topk, float* y, int64_t ldy, hipStream_t s) {
  if (w.base.n == 0) return hipSuccess;
  MfmaArgs a = base_args(w.base);
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
  a.x_rows = x_by_slot ? (int64_t)t * topk : t;
  const int slice = a.pairs_total < 16 ? a.pairs_total : 16;
  return launch_cfg<1, true>(a, slice, (unsigned)w.num_experts, s);
}

}  // namespace q3
