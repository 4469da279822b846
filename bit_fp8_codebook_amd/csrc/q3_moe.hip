// Router of an MoE verify round over 3.25-bit experts.
//
// Hibana: Fast Agentic Inference on Unified-Memory Devices, "Adaptive
// speculation" / "Expert sharing": checking several drafted tokens in one
// round costs the weights of every expert any of them routes to, and a budget
// of experts shared by the whole round caps that set.  These kernels pick each token's top-k
// experts on the device, without or with a budget; the expert-grouped product
// (q3_linear.hip) then reads each picked expert once, without the list of
// picked experts ever coming back to the host.
#include "q3_device.h"
#include "q3_internal.h"

namespace q3 {
namespace {

__device__ __forceinline__ bool ranks_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// One block per token, one thread per expert: the token's logits go to LDS and
// every thread counts the experts that rank before its own (higher logit, or
// an equal logit at a lower index).  That count is the expert's rank, unique
// per expert, so the threads with rank < topk write ids[rank] directly: no
// sorting and no cross-thread reduction.
__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ logits, int E, int topk,
                                                    int32_t* __restrict__ ids) {
  __shared__ float v[1024];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  const float mine = e < E ? logits[(int64_t)t * E + e] : 0.f;
  if (e < E) v[e] = mine;
  __syncthreads();
  if (e >= E) return;
  int rank = 0;
  for (int o = 0; o < E; ++o) rank += ranks_before(v[o], o, mine, e) ? 1 : 0;
  if (rank < topk) ids[(int64_t)t * topk + rank] = e;
}

// Expert-budget routing, one block per token, one thread per expert.  Every
// block first computes the round's routing mass per expert (sum over tokens
// of the token's softmax probability of that expert): each wave takes tokens
// and reduces their max and exp-sum over the experts in a fixed order (the
// wave reductions below), then each thread sums its expert's probabilities over the tokens
// in token order, so every block gets the same masses bit for bit.  The kept
// set is the `budget` experts of largest mass (equal mass: lower index), each
// found by counting the experts that rank before it; the block's token then
// ranks the kept experts by its logits the same way (with up to 64 experts, in
// registers of the one wave that holds them all).  Block 0 also writes the
// kept set in ascending order.  When the round's logits fit (T*E floats up to
// kStageFloats), the block first copies them all to LDS with every load issued
// before the first use, so the per-token passes cost one memory latency in all
// instead of one per token; the arithmetic and its order are the same either
// way.
// Wave-wide maximum and sum, the same value in every lane: DPP exchanges inside
// rows of 16 lanes (xor 1, xor 2, then the half-row and row mirrors), which
// leave each row's result in all its lanes, then the four rows' values read
// out and combined in row order (a fixed order: run-to-run identical).  Lane
// butterflies through LDS permutes cost a memory-pipe round trip per step.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

constexpr int kStageFloats = 8192;

__global__ __launch_bounds__(1024) void budget_topk_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                           int budget, int32_t* __restrict__ ids,
                                                           int32_t* __restrict__ experts, int staged) {
  __shared__ float mass[1024];
  __shared__ float tok[1024];
  __shared__ int kept[1024];
  extern __shared__ float dyn[];   // [T][2] max and exp-sum of each token's logits; then [T][E] logits if staged
  float* const stats = dyn;
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6, waves = blockDim.x >> 6;
  const float* src = logits;
  if (staged) {
    float* const lg = dyn + 2 * T;
    const int total = T * E;
    for (int base = e; base < total; base += 4 * (int)blockDim.x) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = base + q * (int)blockDim.x;
        v[q] = i < total ? logits[i] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = base + q * (int)blockDim.x;
        if (i < total) lg[i] = v[q];
      }
    }
    __syncthreads();
    src = lg;
  }
  for (int u = wave; u < T; u += waves) {
    const float* row = src + (int64_t)u * E;
    float mx = -__builtin_inff();
    for (int o = lane; o < E; o += 64) mx = fmaxf(mx, row[o]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int o = lane; o < E; o += 64) sm += expf(row[o] - mx);
    sm = wave_sum(sm);
    if (lane == 0) {
      stats[2 * u] = mx;
      stats[2 * u + 1] = sm;
    }
  }
  __syncthreads();
  if (E <= 64) {
    // Every expert sits in wave 0, one per lane: masses, the kept set and the
    // token's ranking stay in registers, each expert's value broadcast with
    // readlane (same arithmetic and order as below, no LDS round trip per
    // expert and no further barrier).
    if (wave != 0) return;
    const bool live = lane < E;
    float m = 0.f, tk = 0.f;
    if (live) {
      for (int u = 0; u < T; ++u) m += expf(src[(int64_t)u * E + lane] - stats[2 * u]) / stats[2 * u + 1];
      tk = src[(int64_t)t * E + lane];
    }
    int rank = 0;
    for (int o = 0; o < E; ++o) {
      const float mo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), o));
      rank += ranks_before(mo, o, m, lane) ? 1 : 0;
    }
    const bool in = live && rank < budget;
    const uint64_t keep = __ballot(in);
    int r = 0;
    for (uint64_t b = keep; b != 0; b &= b - 1) {
      const int o = __builtin_ctzll(b);
      const float to = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tk), o));
      r += ranks_before(to, o, tk, lane) ? 1 : 0;
    }
    if (in) {
      if (r < topk) ids[(int64_t)t * topk + r] = lane;
      if (t == 0 && experts) experts[__popcll(keep & ((1ull << lane) - 1ull))] = lane;
    }
    return;
  }
  if (e < E) {
    float m = 0.f;
    for (int u = 0; u < T; ++u) m += expf(src[(int64_t)u * E + e] - stats[2 * u]) / stats[2 * u + 1];
    mass[e] = m;
    tok[e] = src[(int64_t)t * E + e];
  }
  __syncthreads();
  bool in = false;
  if (e < E) {
    int rank = 0;
    for (int o = 0; o < E; ++o) rank += ranks_before(mass[o], o, mass[e], e) ? 1 : 0;
    in = rank < budget;
    kept[e] = in ? 1 : 0;
  }
  __syncthreads();
  if (in) {
    int rank = 0, below = 0;
    for (int o = 0; o < E; ++o) {
      if (!kept[o]) continue;
      rank += ranks_before(tok[o], o, tok[e], e) ? 1 : 0;
      below += o < e ? 1 : 0;
    }
    if (rank < topk) ids[(int64_t)t * topk + rank] = e;
    if (t == 0 && experts) experts[below] = e;
  }
}

// The same routing for rounds of at most 16 tokens over at most 64 experts:
// one block per token, expert e in lane e of each of its waves, and the whole
// round's logits in the first wave's registers, all loaded at once.  Measured
// with clock stamps, what costs is the length of dependent instruction chains
// (a lone wave issues at a fraction of its SIMD's rate), so:
//   * each token's maximum and exp-sum over the experts are reduced by a
//     group of 64/T lanes (T experts per lane, then DPP steps inside the
//     group) on the logits transposed through LDS, all tokens at once;
//   * ranks are counted on 64-bit keys (the value's order-preserving bits
//     above 63 - index, -0 taken as +0), so "ranks before" is one unsigned
//     comparison; the 64 comparisons of each expert are split over four
//     waves (one per SIMD) and their counts added in wave order.
// The mass is the sum over tokens, in token order, of exp(l - max) times the
// hardware reciprocal of the exp-sum.  Every block runs the same code on the
// same logits, so all of them find the same kept set.  (Per dependent launch
// of the budget router for 8 tokens and 64 experts: 6.8 us with readlane loops
// and lane butterflies in one wave, 3.3 us with the keys and DPP reductions,
// 2.8 us with the transposed statistics.)
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
  uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);
  b ^= (b >> 31) ? 0xFFFFFFFFu : 0x80000000u;
  return ((uint64_t)b << 6) | (uint64_t)(63 - idx);
}

// Maximum and sum over an aligned group of G = 4, 8 or 16 lanes (the same
// DPP steps as the wave reductions, stopped at the group's width), the result
// in every lane of the group.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f<0x141>(v);
  if constexpr (G >= 16) v += dpp_f<0x140>(v);
  return v;
}

// Ranking split over kRankWaves waves of a block: wave w counts, for every
// expert (lane), the keys kKeysPerWave*w .. +kKeysPerWave-1 above its own, and
// the partial counts are added in wave order.  A lone wave issues its
// comparisons at a fraction of the SIMD's rate, so four waves on four SIMDs
// cut the counting chain to a quarter.
constexpr int kRankWaves = 4, kKeysPerWave = 64 / kRankWaves;
__device__ __forceinline__ int count_above_part(const uint64_t* keys, int wave, uint64_t mine) {
  ulonglong2 k[kKeysPerWave / 2];
#pragma unroll
  for (int q = 0; q < kKeysPerWave / 2; ++q)
    k[q] = reinterpret_cast<const ulonglong2*>(keys + kKeysPerWave * wave)[q];
  int c[4] = {0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < kKeysPerWave / 2; ++q) {
    c[(2 * q) & 3] += k[q].x > mine ? 1 : 0;
    c[(2 * q + 1) & 3] += k[q].y > mine ? 1 : 0;
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}
__device__ __forceinline__ int sum_parts(const int (&part)[kRankWaves][64], int lane) {
  int r = 0;
#pragma unroll
  for (int w = 0; w < kRankWaves; ++w) r += part[w][lane];
  return r;
}

template <int kT>
__global__ __launch_bounds__(64 * kRankWaves) void budget_topk_wave_kernel(const float* __restrict__ logits, int T,
                                                                           int E, int topk, int budget,
                                                                           int32_t* __restrict__ ids,
                                                                           int32_t* __restrict__ experts) {
  // The softmax statistics are taken transposed by wave 0: the round's logits
  // go to LDS token by token, and each group of G = 64/kT lanes reduces one
  // token over its kT experts per lane (instead of a whole-wave reduction per
  // token); the normalised probabilities come back expert by expert.  The two
  // rankings are then counted by all the block's waves (lane = expert in each).
  constexpr int G = 64 / kT, C = kT;
  __shared__ __align__(16) uint64_t mkeys[64], tkeys[64];
  __shared__ __align__(16) float lg[kT * 64];   // lg[u][e], absent experts -inf
  __shared__ __align__(16) float pr[64 * kT];   // pr[e][u] = exp(l - max) / sum, 0 for u >= T
  __shared__ int part[kRankWaves][64];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool live = lane < E;
  const int le = live ? lane : E - 1;
  const float tk = logits[(int64_t)t * E + le];
  if (wave == 0) {
    float l[kT];
#pragma unroll
    for (int u = 0; u < kT; ++u) l[u] = logits[(int64_t)(u < T ? u : T - 1) * E + le];   // rows past T repeat the last
#pragma unroll
    for (int u = 0; u < kT; ++u) lg[u * 64 + lane] = live ? l[u] : -__builtin_inff();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
      const int u = lane / G, p = lane % G;   // token u, experts p*C .. p*C + C - 1
      float v[C];
#pragma unroll
      for (int q = 0; q < C / 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(lg + u * 64 + p * C + 4 * q);
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
      float mx = v[0];
#pragma unroll
      for (int j = 1; j < C; ++j) mx = fmaxf(mx, v[j]);
      mx = group_max<G>(mx);
      float ex[C], sm = 0.f;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        ex[j] = p * C + j < E ? expf(v[j] - mx) : 0.f;
        sm += ex[j];
      }
      sm = group_sum<G>(sm);
      const float r = __builtin_amdgcn_rcpf(sm);   // v_rcp_f32 (1 ulp) in place of a division
#pragma unroll
      for (int j = 0; j < C; ++j) pr[(p * C + j) * kT + u] = u < T ? ex[j] * r : 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // The expert's mass: its probabilities summed in token order.
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < kT / 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(pr + lane * kT + 4 * q);
      m += f.x;
      m += f.y;
      m += f.z;
      m += f.w;
    }
    mkeys[lane] = live ? rank_key(m, lane) : 0ull;   // absent lanes key 0, ranked last
  }
  __syncthreads();
  // Kept set: the budget experts whose mass ranks first.
  const uint64_t mkey = mkeys[lane];
  part[wave][lane] = count_above_part(mkeys, wave, mkey);
  __syncthreads();
  const bool in = live && sum_parts(part, lane) < budget;
  const uint64_t keep = __ballot(in);
  // The token's ranking inside the kept set (experts outside it key 0, below every kept key).
  const uint64_t tkey = in ? rank_key(tk, lane) + 1ull : 0ull;
  if (wave == 0) tkeys[lane] = tkey;
  __syncthreads();
  part[wave][lane] = count_above_part(tkeys, wave, tkey);
  __syncthreads();
  if (wave == 0 && in) {
    const int r = sum_parts(part, lane);
    if (r < topk) ids[(int64_t)t * topk + r] = lane;
    if (t == 0 && experts) experts[__popcll(keep & ((1ull << lane) - 1ull))] = lane;
  }
}

// Plain top-k for at most 64 experts: one wave per token, expert e in lane e,
// ranks counted on the same 64-bit keys as above (absent lanes key 0, below
// every expert's key + 1).
__global__ __launch_bounds__(64 * kRankWaves) void topk_wave_kernel(const float* __restrict__ logits, int E, int topk,
                                                                    int32_t* __restrict__ ids) {
  __shared__ __align__(16) uint64_t keys[64];
  __shared__ int part[kRankWaves][64];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool live = lane < E;
  const float v = logits[(int64_t)t * E + (live ? lane : E - 1)];
  const uint64_t k = live ? rank_key(v, lane) + 1ull : 0ull;
  if (wave == 0) keys[lane] = k;
  __syncthreads();
  part[wave][lane] = count_above_part(keys, wave, k);
  __syncthreads();
  if (wave == 0) {
    const int r = sum_parts(part, lane);
    if (live && r < topk) ids[(int64_t)t * topk + r] = lane;
  }
}

}  // namespace

hipError_t launch_moe_budget_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t budget,
                                  int32_t* ids, int32_t* experts, hipStream_t s) {
#ifndef Q3_NO_WAVE_ROUTER
  if (e <= 64 && t <= 16) {
    if (t <= 4) hipLaunchKernelGGL(budget_topk_wave_kernel<4>, dim3((unsigned)t), dim3(64 * kRankWaves), 0, s, logits, (int)t,
                                   (int)e, (int)topk, (int)budget, ids, experts);
    else if (t <= 8) hipLaunchKernelGGL(budget_topk_wave_kernel<8>, dim3((unsigned)t), dim3(64 * kRankWaves), 0, s, logits,
                                        (int)t, (int)e, (int)topk, (int)budget, ids, experts);
    else hipLaunchKernelGGL(budget_topk_wave_kernel<16>, dim3((unsigned)t), dim3(64 * kRankWaves), 0, s, logits, (int)t, (int)e,
                            (int)topk, (int)budget, ids, experts);
    return hipGetLastError();
  }
#endif
  // One thread per expert, at least four waves (the per-token passes are spread over the waves).
  unsigned threads = (unsigned)((e + 63) / 64 * 64);
  threads = threads < 256u ? 256u : threads;
  const int staged = (int64_t)t * e <= kStageFloats;
  const size_t shm = ((size_t)t * 2 + (staged ? (size_t)t * e : 0)) * sizeof(float);
  hipLaunchKernelGGL(budget_topk_kernel, dim3((unsigned)t), dim3(threads), shm, s, logits, (int)t, (int)e, (int)topk,
                     (int)budget, ids, experts, staged);
  return hipGetLastError();
}

hipError_t launch_moe_topk(const float* logits, int32_t t, int32_t e, int32_t topk, int32_t* ids, hipStream_t s) {
#ifndef Q3_NO_WAVE_ROUTER
  if (e <= 64) {
    hipLaunchKernelGGL(topk_wave_kernel, dim3((unsigned)t), dim3(64 * kRankWaves), 0, s, logits, (int)e, (int)topk,
                       ids);
    return hipGetLastError();
  }
#endif
  const unsigned threads = (unsigned)((e + 63) / 64 * 64);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)t), dim3(threads), 0, s, logits, (int)e, (int)topk, ids);
  return hipGetLastError();
}

namespace {

// One block per (token, 256 output rows): the token's routing weights go to
// LDS, then each thread sums its row over the token's slots in slot order.
// The first eight slots' rows do not depend on the weights: their loads go out
// before the ids and logits are read, so the two latencies overlap.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int64_t ldp,
                                                      const int32_t* __restrict__ ids, int topk, int E,
                                                      const float* __restrict__ logits, int64_t ld_logits,
                                                      int64_t n, float* __restrict__ out, int64_t ldo) {
  __shared__ float pw[64];
  const int tk = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * 256 + tid;
  const bool row_ok = row < n;
  float v0[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v0[j] = row_ok && j < topk ? part[(int64_t)(tk * topk + j) * ldp + row] : 0.f;
  if (tid < 64) {
    const int lane = tid;
    const int e = lane < topk ? ids[tk * topk + lane] : -1;
    const bool in = e >= 0 && e < E;
    const float l = in ? logits[(int64_t)tk * ld_logits + e] : -__builtin_inff();
    const float mx = wave_max(l);
    const float z = in ? expf(l - mx) : 0.f;
    const float den = wave_sum(z);
    pw[lane] = in ? z / den : 0.f;
  }
  __syncthreads();
  if (!row_ok) return;
  // The slots' rows are loaded eight at a time before any of them is added
  // (rows of slots without a routed expert lie in the same buffer and are
  // read but never added), then summed in slot order.
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < topk && pw[j] != 0.f) sum += pw[j] * v0[j];
  for (int q0 = 8; q0 < topk; q0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = q0 + j < topk ? part[(int64_t)(tk * topk + q0 + j) * ldp + row] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q0 + j < topk && pw[q0 + j] != 0.f) sum += pw[q0 + j] * v[j];
  }
  out[(int64_t)tk * ldo + row] = sum;
}

}  // namespace

hipError_t launch_moe_combine(const float* part, int64_t ldp, const int32_t* ids, int32_t t, int32_t topk,
                              int32_t num_experts, const float* logits, int64_t ld_logits, int64_t n, float* out,
                              int64_t ldo, hipStream_t s) {
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)t);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, part, ldp, ids, (int)topk, (int)num_experts, logits,
                     ld_logits, n, out, ldo);
  return hipGetLastError();
}

}  // namespace q3
