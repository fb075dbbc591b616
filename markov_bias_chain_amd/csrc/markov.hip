// libmarkov: the DSpark sequential Markov draft-sampling chain on MI355X
// (gfx950, CDNA4).  The C ABI is declared in include/markov.h.
//
// Source pages (cited by title and section):
//   [SM] vLLM API page "vllm.models.deepseek_v41.nvidia.specialized_decode.
//        sampling.sharded_markov": module docstring and per-call diagram,
//        DSparkShardedMarkovSampler (fork_noise, sample, _kernel).
//   [FM] vLLM API page "vllm.models.deepseek_v41.nvidia.ops.fused_markov":
//        module docstring, FusedMarkovSampler.
//   [MS] vLLM API page "vllm.models.muse_spark.nvidia.specialized_decode.
//        runtime.markov": module docstring, MarkovSampler, FusedMarkovParams.
//
// Design (one GPU):
//  * markov_noise_fill: one thread per 4 consecutive vocab ids, one 16-byte
//    store; the (seed, row, step) part of the hash is computed per thread.
//  * markov_chain_sample: ONE persistent cooperative launch runs all N
//    positions.  The vocabulary is cut into groups of 16384 / r head rows
//    (32 KiB of bf16 head each); a wavefront owns one group per chunk, and a
//    chunk is 8 consecutive groups (one per wave of a 512-thread workgroup).
//    The first chunk of every workgroup stays in VGPRs for the whole launch
//    (128 VGPRs per lane), so the head is read from HBM once per call when
//    the grid covers the vocabulary; further chunks are streamed every step.
//  * The bias GEMV is 64-wide wavefront work: each lane holds 16-byte head
//    vectors (8 bf16 of one row) and dots them with the matching 8 bf16 of
//    the embedding row with v_dot2_f32_bf16; a transposing butterfly then
//    leaves one finished row sum per lane, so the epilogue (logit, cache
//    store, score, key) is one vocab id per lane.
//  * Each step ends in a grid-wide exchange through the workspace: every
//    workgroup stores its candidate (a packed 64-bit (score, index) key) in
//    its own slot with a single agent-scope store, and every workgroup polls
//    all slots, so there is no contended atomic and no second flag.  A zero
//    slot means "not arrived"; real keys are never zero.  Alternate calls use
//    alternate halves of the workspace and each call clears the half the
//    next call will use, so no reset launch is needed.
//  * Mode 1 (inverse CDF) publishes per-chunk (max key, sum of exp) partials;
//    a leader workgroup per row locates the chunk holding u * S, the chunk's
//    owner scans it in vocabulary order and publishes the token.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "markov.h"

namespace {

constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kThreads = kWaves * 64;      // 512 threads, one workgroup per CU
constexpr int kSlots = 32;                 // 16-byte head vectors per lane per group
constexpr int kSub = 8;                    // slots per sub-batch of the butterfly
constexpr int kRowPass = 8;                // request rows per register pass
constexpr int kHeader = 256;               // workspace header bytes
constexpr int kMaxPollPerLane = 16;        // slots one lane polls (<= 1024 per row)
constexpr unsigned long long kTimeoutTicks = 200000000ull;  // 2 s at 100 MHz

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------- bf16 helpers --

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------- lane exchanges --
// xor-partner exchanges within a wave64, on the cheapest path for each
// distance: DPP quad permutes (1, 2), DPP row rotate by 8 (= xor 8 inside a
// 16-lane row), ds_swizzle bit-mask mode (4, 16), ds_bpermute (32).

__device__ __forceinline__ int xsh1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int xsh2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int xsh4(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x101F); }
__device__ __forceinline__ int xsh8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); }
__device__ __forceinline__ int xsh16(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }
__device__ __forceinline__ int xsh32(int v) { return __shfl_xor(v, 32); }

template <int M>
__device__ __forceinline__ float xshf(float x) {
  int v = __float_as_int(x);
  if constexpr (M == 1) v = xsh1(v);
  else if constexpr (M == 2) v = xsh2(v);
  else if constexpr (M == 4) v = xsh4(v);
  else if constexpr (M == 8) v = xsh8(v);
  else if constexpr (M == 16) v = xsh16(v);
  else v = xsh32(v);
  return __int_as_float(v);
}

template <int M>
__device__ __forceinline__ uint64_t xshk(uint64_t k) {
  int lo = (int)(uint32_t)k, hi = (int)(uint32_t)(k >> 32);
  if constexpr (M == 1) { lo = xsh1(lo); hi = xsh1(hi); }
  else if constexpr (M == 2) { lo = xsh2(lo); hi = xsh2(hi); }
  else if constexpr (M == 4) { lo = xsh4(lo); hi = xsh4(hi); }
  else if constexpr (M == 8) { lo = xsh8(lo); hi = xsh8(hi); }
  else if constexpr (M == 16) { lo = xsh16(lo); hi = xsh16(hi); }
  else { lo = xsh32(lo); hi = xsh32(hi); }
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = umax64(k, xshk<1>(k));
  k = umax64(k, xshk<2>(k));
  k = umax64(k, xshk<4>(k));
  k = umax64(k, xshk<8>(k));
  k = umax64(k, xshk<16>(k));
  k = umax64(k, xshk<32>(k));
  return k;
}

__device__ __forceinline__ float wave_sum(float x) {
  x += xshf<1>(x);
  x += xshf<2>(x);
  x += xshf<4>(x);
  x += xshf<8>(x);
  x += xshf<16>(x);
  x += xshf<32>(x);
  return x;
}

// ------------------------------------------------------ packed (score, id) --
// A total order on fp32 scores with NaN above everything ([MS] module
// docstring: the lowest NaN id wins, else the lowest id of the maximum); +0
// and -0 are made equal.  The low word is ~v, so among equal scores the lower
// id has the larger key.  Real keys are >= 0x007FFFFF << 32, so 0 can mean
// "empty slot" and 1 "no candidate".

constexpr uint64_t kNoCandidate = 1;

__device__ __forceinline__ uint32_t score_ord(float s) {
  uint32_t b = __float_as_uint(s);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFFFFFu;
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float ord_score(uint32_t o) {
  if (o == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float s, uint32_t v) {
  return ((uint64_t)score_ord(s) << 32) | (uint32_t)(0xFFFFFFFFu - v);
}

__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

// ------------------------------------------------------------ SplitMix64 --
// Steele, Lea and Flood (OOPSLA 2014): one output of the generator whose
// state is x is the finaliser applied to x + golden-ratio increment.

__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// (seed, row, step) prefix: the seed is mixed first, then each counter is
// absorbed as h <- splitmix64(h ^ counter).
__device__ __forceinline__ uint64_t noise_prefix(int64_t seed, int row, int step) {
  uint64_t h = splitmix64((uint64_t)seed);
  h = splitmix64(h ^ (uint64_t)(int64_t)row);
  return splitmix64(h ^ (uint64_t)(int64_t)step);
}

// The top 23 bits as (2k + 1) * 2^-24, exactly representable in fp32.
__device__ __forceinline__ float hash_uniform(uint64_t h) {
  return (float)(uint32_t)(2u * (uint32_t)(h >> 41) + 1u) * 0x1p-24f;
}

// ------------------------------------------------------------ agent scope --
// Cross-workgroup data goes through single agent-scope atomic loads and
// stores: each word is self-validating, so no ordering between words is
// needed and no cache maintenance is issued.

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// The correctly rounded fp32 natural log: fp64 log of the fp32 argument,
// rounded once (fp32 log libraries are only faithfully rounded).
__device__ __forceinline__ float log_f32_rn(float x) { return (float)log((double)x); }

// ============================================================== noise fill ==

__global__ __launch_bounds__(256) void noise_fill_kernel(float* __restrict__ gumbel,
                                                         const int64_t* __restrict__ seeds,
                                                         int steps, int V) {
  const int rs = blockIdx.y;  // row * steps + step
  const int row = rs / steps, step = rs - row * steps;
  const int v0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (v0 >= V) return;  // V is a multiple of 16: a thread's 4 ids are all valid
  const uint64_t prefix = noise_prefix(seeds[row], row, step);
  float out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float u = hash_uniform(splitmix64(prefix ^ (uint64_t)(v0 + j)));
    out[j] = -log_f32_rn(-log_f32_rn(u));
  }
  float4* dst = reinterpret_cast<float4*>(gumbel + (size_t)rs * V + v0);
  *dst = make_float4(out[0], out[1], out[2], out[3]);
}

// ============================================================ chain kernel ==

struct ChainParams {
  const uint16_t* base;
  long long base_rs, base_ss;
  const uint16_t* head;
  const uint16_t* embed;
  const int64_t* prev;
  const float* temp;
  const int64_t* seeds;
  const float* gumbel;
  const int64_t* state_idx;
  float mult, cap, inv_cap;
  int has_cap;
  int rows, N, V, NG, NC, G;
  int64_t* tokens;
  long long tok_rs;
  uint16_t* cache;
  long long cache_rs, cache_ss;
  long long cache_states;
  unsigned char* ws;
  unsigned long long ws_half;  // bytes per parity half
};

// Workspace half layout (slot arrays of one parity):
//   keys [N][rows][NC] u64     candidate keys (mode 0: one per workgroup,
//                               mode 1: one per chunk)
//   sums [N][rows][NC] u32     mode 1: sum of exp(z - chunk max), sign bit set
//   dec  [N][rows]     u64     mode 1: the leader's decision for the row
//   tok  [N][rows]     u64     mode 1: the owner's token for the row
struct HalfLayout {
  uint64_t* keys;
  uint32_t* sums;
  uint64_t* dec;
  uint64_t* tok;
};

__host__ __device__ inline size_t half_bytes_needed(int rows, int N, int NC, int mode) {
  size_t slots = (size_t)N * rows * NC;
  size_t b = slots * 8;
  if (mode == 1) b += slots * 4 + (size_t)N * rows * 16;
  return (b + 255) & ~(size_t)255;
}

__device__ inline HalfLayout half_layout(unsigned char* half, int rows, int N, int NC) {
  HalfLayout L;
  size_t slots = (size_t)N * rows * NC;
  L.keys = reinterpret_cast<uint64_t*>(half);
  L.sums = reinterpret_cast<uint32_t*>(half + slots * 8);
  L.dec = reinterpret_cast<uint64_t*>(half + slots * 12);
  L.tok = L.dec + (size_t)N * rows;
  return L;
}

// The lane's dot products for one group and up to kRowPass request rows,
// as one finished row sum per lane (the row given by row_in_group()).
//
// Lane layout of a group (32 slots of 16 bytes per lane = 32 KiB of head):
// slot s, lane l hold bf16 elements [8*kseg, 8*kseg + 8) of group row
// (64*s + l) / (r/8), kseg = (64*s + l) % (r/8).  One slot is 1 KiB of
// consecutive head bytes, so every load instruction is fully coalesced.
//
// Reduction: per sub-batch of 8 slots, a transposing butterfly over lane
// bits 0..2 halves the values at each level (the lane keeps one half and
// trades the other with its partner), leaving slot 8q + (l & 7) partially
// summed; plain xor-adds over the remaining k-segment bits finish the sum,
// and lanes with ((l >> 3) & 3) == q keep it.  So lane l ends with slot
// (l & 31): row 2 (l & 31) + (l >> 5) for r = 256, row (l & 31) for r = 512
// (lanes 32..63 then hold duplicates).  The summation order depends only on
// the lane layout, not on the grid, so the bias is grid-invariant.
template <int R>
__device__ __forceinline__ int row_in_group(int lane) {
  if constexpr (R == 256) return 2 * (lane & 31) + (lane >> 5);
  else return lane & 31;
}

template <int R>
__device__ __forceinline__ float butterfly8(const float (&a)[kSub], int lane, int q, float prev) {
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  float a1[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float keep = b0 ? a[2 * m + 1] : a[2 * m];
    float send = b0 ? a[2 * m] : a[2 * m + 1];
    a1[m] = keep + xshf<1>(send);
  }
  float a2[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float keep = b1 ? a1[2 * m + 1] : a1[2 * m];
    float send = b1 ? a1[2 * m] : a1[2 * m + 1];
    a2[m] = keep + xshf<2>(send);
  }
  float keep = b2 ? a2[1] : a2[0];
  float send = b2 ? a2[0] : a2[1];
  float x = keep + xshf<4>(send);
  x += xshf<8>(x);
  x += xshf<16>(x);
  if constexpr (R == 512) x += xshf<32>(x);
  return (((lane >> 3) & 3) == q) ? x : prev;
}

__device__ __forceinline__ float dot8(uint4 h, uint4 e, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h.x), __builtin_bit_cast(bf16x2_t, e.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h.y), __builtin_bit_cast(bf16x2_t, e.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h.z), __builtin_bit_cast(bf16x2_t, e.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h.w), __builtin_bit_cast(bf16x2_t, e.w), acc, false);
  return acc;
}

template <int R>
__device__ __forceinline__ uint4 load_head_slot(const uint16_t* __restrict__ head, int g, int s, int lane, int V) {
  constexpr int kseg_n = R / 8;
  const int c = s * 64 + lane;
  const int row = g * (16384 / R) + c / kseg_n;
  const int kseg = c % kseg_n;
  if (row >= V) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(head + (size_t)row * R + kseg * 8);
}

// Dot products of one group with the embeddings of rows [b0, b0 + nb).
// FROM_REGS: the group's head is `h` (resident); otherwise it is streamed
// from memory, 8 slots at a time, once per row pass.
template <int R, bool FROM_REGS, int NH>
__device__ __forceinline__ void group_dots(const uint4 (&h)[NH], const uint16_t* __restrict__ head,
                                           int g, int V, const uint4* __restrict__ s_e,
                                           const int* __restrict__ s_active, int b0, int nb,
                                           int lane, float (&val)[kRowPass]) {
  constexpr int kseg_n = R / 8;
  const int kseg = lane % kseg_n;
#pragma unroll
  for (int q = 0; q < kSlots / kSub; ++q) {
    uint4 hs[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) {
      if constexpr (FROM_REGS) hs[s] = h[q * kSub + s];
      else hs[s] = load_head_slot<R>(head, g, q * kSub + s, lane, V);
    }
#pragma unroll
    for (int bi = 0; bi < kRowPass; ++bi) {
      if (bi < nb && s_active[b0 + bi]) {
        const uint4 e = s_e[(b0 + bi) * kseg_n + kseg];
        float a[kSub];
#pragma unroll
        for (int s = 0; s < kSub; ++s) a[s] = dot8(hs[s], e, 0.0f);
        val[bi] = butterfly8<R>(a, lane, q, val[bi]);
      }
    }
  }
}

// RES: every workgroup owns exactly one chunk (G == NC) and keeps its head in
// VGPRs for the whole launch.  !RES: workgroups stride over the chunks and
// stream the head from memory at every step.
template <int R, int MODE, bool RES>
__global__ __launch_bounds__(kThreads, 1) void chain_kernel(ChainParams p) {
  constexpr int RPG = 16384 / R;       // head rows per group
  constexpr int CHUNK = kWaves * RPG;  // vocab ids per chunk
  constexpr int KSEG = R / 8;          // 16-byte segments per head row

  __shared__ int s_state[MARKOV_MAX_ROWS];
  __shared__ int s_active[MARKOV_MAX_ROWS];
  __shared__ float s_T[MARKOV_MAX_ROWS];
  __shared__ int s_tok[MARKOV_MAX_ROWS];
  __shared__ int s_need[MARKOV_MAX_ROWS];
  __shared__ uint64_t s_dec[MARKOV_MAX_ROWS];
  __shared__ uint64_t s_key[kWaves][MARKOV_MAX_ROWS];
  __shared__ float s_wsum[kWaves][MARKOV_MAX_ROWS];
  __shared__ int s_abort;
  __shared__ uint32_t s_parity;
  extern __shared__ uint4 s_e[];  // [rows][KSEG] 16-byte vectors of the current embeddings

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x;
  const int rows = p.rows, N = p.N, V = p.V, G = p.G, NC = p.NC, NG = p.NG;
  uint32_t* header = reinterpret_cast<uint32_t*>(p.ws);
  const uint64_t deadline = now_ticks() + kTimeoutTicks;

  // ---- prologue: rows, parity, the resident head into VGPRs.
  uint4 h[RES ? kSlots : 1];
  if constexpr (RES) {
    const int g0 = wg * kWaves + wave;  // this wave's group
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
      h[s] = g0 < NG ? load_head_slot<R>(p.head, g0, s, lane, V) : make_uint4(0, 0, 0, 0);
  }
  if (tid == 0) {
    s_parity = ld_agent32(header);
    s_abort = 0;
  }
  for (int b = tid; b < rows; b += kThreads) {
    const int64_t st = p.state_idx ? p.state_idx[b] : b;
    const int64_t tok = p.prev[b];
    int active = st >= 0;
    if (active && st >= p.cache_states) {
      active = 0;
      if (wg == 0)
        __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_BAD_STATE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (active && (tok < 0 || tok >= V)) {
      active = 0;
      if (wg == 0)
        __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_state[b] = (int)st;
    s_active[b] = active;
    s_T[b] = p.temp[b];
    s_tok[b] = active ? (int)tok : 0;
  }
  __syncthreads();
  const uint32_t parity = s_parity & 1u;
  unsigned char* half = p.ws + kHeader + parity * p.ws_half;
  {
    // Clear the other half for the next call (nobody reads it in this one).
    uint4* other = reinterpret_cast<uint4*>(p.ws + kHeader + (parity ^ 1u) * p.ws_half);
    const size_t n16 = p.ws_half / 16;
    for (size_t k = (size_t)wg * kThreads + tid; k < n16; k += (size_t)G * kThreads)
      other[k] = make_uint4(0, 0, 0, 0);
  }
  const HalfLayout L = half_layout(half, rows, N, NC);
  // Embeddings of the anchor tokens.
  for (int k = tid; k < rows * KSEG; k += kThreads) {
    const int b = k / KSEG, seg = k - b * KSEG;
    if (s_active[b])
      s_e[k] = *reinterpret_cast<const uint4*>(p.embed + (size_t)s_tok[b] * R + seg * 8);
  }
  __syncthreads();

  for (int i = 0; i < N; ++i) {
    // ---- local work: dots, epilogue, keys for every chunk of this workgroup.
    if (lane == 0)
      for (int b = 0; b < rows; ++b) s_key[wave][b] = kNoCandidate;
    for (int j = 0; wg + j * G < NC; ++j) {
      const int c = wg + j * G;
      const int g = c * kWaves + wave;
      const int v = g * RPG + row_in_group<R>(lane);
      const bool own = g < NG && v < V && (R == 256 || lane < 32);
      for (int b0 = 0; b0 < rows; b0 += kRowPass) {
        const int nb = rows - b0 < kRowPass ? rows - b0 : kRowPass;
        // Issue this pass's base and noise loads before the dot products.
        uint32_t bl[kRowPass];
        float gl[kRowPass];
#pragma unroll
        for (int bi = 0; bi < kRowPass; ++bi) {
          bl[bi] = 0;
          gl[bi] = 0.0f;
          if (bi < nb && s_active[b0 + bi] && own) {
            const int b = b0 + bi;
            bl[bi] = p.base[b * p.base_rs + i * p.base_ss + v];
            if (MODE == 0 && s_T[b] > 0.0f) gl[bi] = p.gumbel[((size_t)b * N + i) * V + v];
          }
        }
        float val[kRowPass];
#pragma unroll
        for (int bi = 0; bi < kRowPass; ++bi) val[bi] = 0.0f;
        group_dots<R, RES>(h, p.head, g, V, s_e, s_active, b0, nb, lane, val);
#pragma unroll
        for (int bi = 0; bi < kRowPass; ++bi) {
          const int b = b0 + bi;
          if (!(bi < nb && s_active[b])) continue;
          const float T = s_T[b];
          uint64_t key = kNoCandidate;
          float z = 0.0f;
          if (own) {
            const float bias = bf16_to_f32(f32_to_bf16(val[bi]));
            float x = __fadd_rn(bf16_to_f32(bl[bi]), bias);
            x = __fmul_rn(x, p.mult);
            if (p.has_cap) x = __fmul_rn(tanhf(__fmul_rn(x, p.inv_cap)), p.cap);
            const uint32_t cb = f32_to_bf16(x);
            p.cache[(long long)s_state[b] * p.cache_rs + (long long)i * p.cache_ss + v] = (uint16_t)cb;
            const float cf = bf16_to_f32(cb);
            if (T > 0.0f) {
              z = __fdiv_rn(cf, T);
              if (MODE == 0) z = __fadd_rn(z, gl[bi]);
            } else {
              z = cf;
            }
            key = make_key(z, (uint32_t)v);
          }
          const uint64_t wk = wave_max_key(key);
          if (MODE == 0) {
            if (lane == 0 && wk > s_key[wave][b]) s_key[wave][b] = wk;
          } else {
            // Per-wave softmax partial relative to the wave's own maximum.
            const float m = ord_score((uint32_t)(wk >> 32));
            float e = 0.0f;
            if (own && wk != kNoCandidate && isfinite(m) && !isnan(z)) e = expf(z - m);
            const float ws = wave_sum(e);
            if (lane == 0) {
              s_key[wave][b] = wk;
              s_wsum[wave][b] = ws;
            }
          }
        }
      }
      if (MODE == 1) {
        // Combine the chunk's 8 wave partials (fixed order) and publish them.
        __syncthreads();
        for (int b = tid; b < rows; b += kThreads) {
          if (!s_active[b]) continue;
          uint64_t K = kNoCandidate;
          for (int w = 0; w < kWaves; ++w) K = umax64(K, s_key[w][b]);
          float S = 0.0f;
          const float M = ord_score((uint32_t)(K >> 32));
          if (K != kNoCandidate && isfinite(M)) {
            for (int w = 0; w < kWaves; ++w) {
              const uint64_t kw = s_key[w][b];
              const float mw = ord_score((uint32_t)(kw >> 32));
              if (kw != kNoCandidate && isfinite(mw)) S += s_wsum[w][b] * expf(mw - M);
            }
          }
          const size_t slot = ((size_t)i * rows + b) * NC + c;
          st_agent32(L.sums + slot, __float_as_uint(S) | 0x80000000u);
          st_agent(L.keys + slot, K);
        }
        __syncthreads();
      }
    }
    if (MODE == 0) {
      __syncthreads();
      for (int b = tid; b < rows; b += kThreads) {
        if (!s_active[b]) continue;
        uint64_t K = kNoCandidate;
        for (int w = 0; w < kWaves; ++w) K = umax64(K, s_key[w][b]);
        st_agent(L.keys + ((size_t)i * rows + b) * NC + wg, K);
      }
    }

    // ---- grid-wide exchange.
    if (MODE == 0) {
      // Every workgroup reads every workgroup's key; wave w serves rows w, w+8, ...
      for (int b = wave; b < rows; b += kWaves) {
        if (!s_active[b]) continue;
        const uint64_t* slots = L.keys + ((size_t)i * rows + b) * NC;
        uint64_t best = kNoCandidate;
        for (;;) {
          bool all = true;
          best = kNoCandidate;
#pragma unroll
          for (int k = 0; k < kMaxPollPerLane; ++k) {
            const int idx = lane + 64 * k;
            if (idx < G) {
              const uint64_t x = ld_agent(slots + idx);
              all = all && (x != 0);
              best = umax64(best, x);
            }
          }
          if (__all(all)) break;
          if (now_ticks() > deadline) {
            if (lane == 0) {
              s_abort = 1;
              __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        best = wave_max_key(best);
        if (lane == 0) s_tok[b] = (int)key_id(best);
      }
    } else {
      // H2: the leader workgroup of each row (b % G) finds the chunk that
      // holds u * S and publishes it with the threshold in that chunk's
      // own scale, or the token itself for an argmax row.
      const int KPL = (NC + 63) / 64;  // chunks per lane, contiguous
      for (int b = wg; b < rows; b += G) {
        if (((b / G) % kWaves) != wave || !s_active[b]) continue;
        const uint64_t* kslots = L.keys + ((size_t)i * rows + b) * NC;
        const uint32_t* sslots = L.sums + ((size_t)i * rows + b) * NC;
        for (;;) {
          bool all = true;
          for (int k = 0; k < KPL; ++k) {
            const int c = lane * KPL + k;
            if (c < NC) all = all && ld_agent(kslots + c) != 0 && ld_agent32(sslots + c) != 0;
          }
          if (__all(all)) break;
          if (now_ticks() > deadline) {
            if (lane == 0) {
              s_abort = 1;
              __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        uint64_t K = kNoCandidate;
        for (int k = 0; k < KPL; ++k) {
          const int c = lane * KPL + k;
          if (c < NC) K = umax64(K, ld_agent(kslots + c));
        }
        K = wave_max_key(K);
        const float M = ord_score((uint32_t)(K >> 32));
        uint64_t dec;
        if (!(s_T[b] > 0.0f) || !isfinite(M)) {
          dec = (1ull << 63) | key_id(K);
        } else {
          // Weights of this lane's chunks and their running sum.
          float lsum = 0.0f;
          for (int k = 0; k < KPL; ++k) {
            const int c = lane * KPL + k;
            if (c < NC) {
              const uint64_t kc = ld_agent(kslots + c);
              const float mc = ord_score((uint32_t)(kc >> 32));
              const float sc = __uint_as_float(ld_agent32(sslots + c) & 0x7FFFFFFFu);
              if (kc != kNoCandidate && isfinite(mc)) lsum += sc * expf(mc - M);
            }
          }
          // Inclusive scan of the lane totals in lane order.
          float incl = lsum;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const float o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
          }
          const float total = __shfl(incl, 63);
          const float excl = incl - lsum;
          const float t = hash_uniform(noise_prefix(p.seeds[b], b, i)) * total;
          // First chunk whose inclusive prefix exceeds t.
          int found = -1;
          float before = 0.0f, wfound = 0.0f;
          float run = excl;
          int last_pos = -1;
          float last_before = 0.0f, last_w = 0.0f;
          for (int k = 0; k < KPL; ++k) {
            const int c = lane * KPL + k;
            if (c < NC) {
              const uint64_t kc = ld_agent(kslots + c);
              const float mc = ord_score((uint32_t)(kc >> 32));
              const float sc = __uint_as_float(ld_agent32(sslots + c) & 0x7FFFFFFFu);
              const float w = (kc != kNoCandidate && isfinite(mc)) ? sc * expf(mc - M) : 0.0f;
              if (found < 0 && run + w > t) {
                found = c;
                before = run;
                wfound = expf(mc - M);
              }
              if (w > 0.0f) {
                last_pos = c;
                last_before = run;
                last_w = expf(mc - M);
              }
              run += w;
            }
          }
          const uint64_t hit = __ballot(found >= 0);
          int o;
          float tl;
          if (hit) {
            const int src = __builtin_ctzll(hit);
            o = __shfl(found, src);
            const float bf = __shfl(before, src);
            const float sf = __shfl(wfound, src);
            tl = (t - bf) / sf;
          } else {
            // Rounding left no chunk above t: the last chunk with weight.
            const uint64_t any = __ballot(last_pos >= 0);
            const int src = 63 - __builtin_clzll(any);
            o = __shfl(last_pos, src);
            const float bf = __shfl(last_before, src);
            const float sf = __shfl(last_w, src);
            tl = (t - bf) / sf;
          }
          if (!(tl >= 0.0f)) tl = 0.0f;
          dec = ((uint64_t)(uint32_t)(o + 1) << 32) | __float_as_uint(tl);
        }
        if (lane == 0) st_agent(L.dec + (size_t)i * rows + b, dec);
      }
      // H3: every workgroup reads every row's decision.
      for (int b = wave; b < rows; b += kWaves) {
        if (!s_active[b]) continue;
        uint64_t d;
        for (;;) {
          d = ld_agent(L.dec + (size_t)i * rows + b);
          if (d != 0) break;
          if (now_ticks() > deadline) {
            if (lane == 0) {
              s_abort = 1;
              __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            d = 1ull << 63;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) {
          if (d >> 63) {
            s_tok[b] = (int)(uint32_t)d;
            s_need[b] = 0;
          } else {
            const int o = (int)(d >> 32) - 1;
            s_dec[b] = d;
            s_need[b] = (o % G == wg) ? 2 : 1;
          }
        }
      }
      __syncthreads();
      // The chunk's owner scans it in vocabulary order (its cache values were
      // stored by this workgroup in this step).
      for (int b = wave; b < rows; b += kWaves) {
        if (!s_active[b] || s_need[b] != 2) continue;
        const uint64_t d = s_dec[b];
        const int o = (int)(d >> 32) - 1;
        const float tl = __uint_as_float((uint32_t)d);
        const float T = s_T[b];
        constexpr int PER = CHUNK / 64;  // ids per lane
        const int v0 = o * CHUNK + lane * PER;
        const uint16_t* crow = p.cache + (long long)s_state[b] * p.cache_rs + (long long)i * p.cache_ss;
        float z[PER];
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int v = v0 + k;
          z[k] = v < V ? __fdiv_rn(bf16_to_f32(crow[v]), T) : -INFINITY;
          m = fmaxf(m, z[k]);
        }
        // chunk maximum
        {
          float mm = m;
          mm = fmaxf(mm, xshf<1>(mm));
          mm = fmaxf(mm, xshf<2>(mm));
          mm = fmaxf(mm, xshf<4>(mm));
          mm = fmaxf(mm, xshf<8>(mm));
          mm = fmaxf(mm, xshf<16>(mm));
          mm = fmaxf(mm, xshf<32>(mm));
          m = mm;
        }
        float w[PER];
        float lsum = 0.0f;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          w[k] = (v0 + k < V && z[k] > -INFINITY) ? expf(z[k] - m) : 0.0f;
          lsum += w[k];
        }
        float incl = lsum;
#pragma unroll
        for (int dd = 1; dd < 64; dd <<= 1) {
          const float ov = __shfl_up(incl, dd);
          if (lane >= dd) incl += ov;
        }
        float run = incl - lsum;
        int found = -1, lastv = -1;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          if (found < 0 && w[k] > 0.0f && run + w[k] > tl) found = v0 + k;
          if (w[k] > 0.0f) lastv = v0 + k;
          run += w[k];
        }
        const uint64_t hit = __ballot(found >= 0);
        int tok;
        if (hit) {
          tok = __shfl(found, __builtin_ctzll(hit));
        } else {
          const uint64_t any = __ballot(lastv >= 0);
          tok = any ? __shfl(lastv, 63 - __builtin_clzll(any)) : o * CHUNK;
        }
        if (lane == 0) {
          s_tok[b] = tok;
          st_agent(L.tok + (size_t)i * rows + b, (1ull << 63) | (uint32_t)tok);
        }
      }
      // H4: rows whose chunk another workgroup owns.
      for (int b = wave; b < rows; b += kWaves) {
        if (!s_active[b] || s_need[b] != 1) continue;
        uint64_t d;
        for (;;) {
          d = ld_agent(L.tok + (size_t)i * rows + b);
          if (d != 0) break;
          if (now_ticks() > deadline) {
            if (lane == 0) {
              s_abort = 1;
              __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            d = 1ull << 63;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) s_tok[b] = (int)(uint32_t)d;
      }
    }
    __syncthreads();
    if (s_abort) break;

    // ---- the winners: tokens out, next embeddings in.
    if (wg == 0)
      for (int b = tid; b < rows; b += kThreads)
        if (s_active[b]) p.tokens[(long long)b * p.tok_rs + i] = s_tok[b];
    if (i + 1 < N) {
      for (int k = tid; k < rows * KSEG; k += kThreads) {
        const int b = k / KSEG, seg = k - b * KSEG;
        if (s_active[b]) {
          // A winner is always a valid id; the clamp only keeps the gather in
          // bounds should that ever fail.
          const uint32_t t = (uint32_t)s_tok[b] < (uint32_t)V ? (uint32_t)s_tok[b] : 0u;
          s_e[k] = *reinterpret_cast<const uint4*>(p.embed + (size_t)t * R + seg * 8);
        }
      }
      __syncthreads();
    }
  }
  // Every workgroup has read the parity by now (all published the last step).
  if (wg == 0 && tid == 0 && !s_abort) st_agent32(header, parity ^ 1u);
}

// ================================================================= host ==

thread_local std::string g_last_error;
std::atomic<int> g_grid_override{0};

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int groups_per_rank(int rank) { return 16384 / rank; }

struct Shape {
  int NG, NC;
};

int check_shape(int rows, int steps, int vocab, int rank, int mode, Shape* sh) {
  if (rows < 1 || rows > MARKOV_MAX_ROWS)
    return fail(MARKOV_E_UNSUPPORTED, "rows=%d outside [1, %d]", rows, MARKOV_MAX_ROWS);
  if (steps < 1 || steps > MARKOV_MAX_STEPS)
    return fail(MARKOV_E_UNSUPPORTED, "steps=%d outside [1, %d]", steps, MARKOV_MAX_STEPS);
  if (vocab < 16 || vocab % 16 != 0 || vocab > MARKOV_MAX_VOCAB)
    return fail(MARKOV_E_UNSUPPORTED, "vocab=%d is not a positive multiple of 16 up to %d", vocab,
                MARKOV_MAX_VOCAB);
  if (rank != 256 && rank != 512)
    return fail(MARKOV_E_UNSUPPORTED, "rank=%d (this build takes 256 or 512)", rank);
  if (mode != MARKOV_MODE_GUMBEL && mode != MARKOV_MODE_INVCDF)
    return fail(MARKOV_E_UNSUPPORTED, "mode=%d", mode);
  const int rpg = groups_per_rank(rank);
  sh->NG = (vocab + rpg - 1) / rpg;
  sh->NC = (sh->NG + kWaves - 1) / kWaves;
  if (sh->NC > 64 * kMaxPollPerLane)
    return fail(MARKOV_E_UNSUPPORTED, "vocab=%d needs %d chunks (max %d)", vocab, sh->NC,
                64 * kMaxPollPerLane);
  return MARKOV_OK;
}

const void* kernel_for(int rank, int mode, bool res) {
  if (rank == 256) {
    if (mode == 0) return res ? (const void*)chain_kernel<256, 0, true> : (const void*)chain_kernel<256, 0, false>;
    return res ? (const void*)chain_kernel<256, 1, true> : (const void*)chain_kernel<256, 1, false>;
  }
  if (mode == 0) return res ? (const void*)chain_kernel<512, 0, true> : (const void*)chain_kernel<512, 0, false>;
  return res ? (const void*)chain_kernel<512, 1, true> : (const void*)chain_kernel<512, 1, false>;
}

// Dynamic LDS above the default per-launch limit is opted into once per
// process for every chain kernel (the embeddings take up to 64 KiB).
int prepare_kernels() {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    for (int rank : {256, 512})
      for (int mode : {0, 1})
        for (bool res : {false, true}) {
          hipError_t e = hipFuncSetAttribute(kernel_for(rank, mode, res),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             MARKOV_MAX_ROWS * 512 * 2);
          if (e != hipSuccess && err == hipSuccess) err = e;
        }
  });
  if (err != hipSuccess) return fail(MARKOV_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
  return MARKOV_OK;
}

// The grid: one workgroup per CU at most.  If the CUs cover every chunk the
// head is resident (G == NC); otherwise workgroups stream their chunks.
int pick_grid(int rows, int rank, int mode, const Shape& sh, int* grid, bool* res) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  const size_t shmem = (size_t)rows * rank * 2;
  long long g = cus;  // one workgroup per CU: the grid never exceeds the CUs
  if (g > sh.NC) g = sh.NC;
  const int ov = g_grid_override.load();
  if (ov > 0 && ov < g) g = ov;
  if (g > 64 * kMaxPollPerLane) g = 64 * kMaxPollPerLane;
  const bool resident = (g == sh.NC);
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel_for(rank, mode, resident), kThreads, shmem);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "occupancy query: %s", hipGetErrorString(e));
  if (per_cu < 1) return fail(MARKOV_E_HIP, "the chain kernel does not fit on a compute unit");
  *grid = (int)g;
  *res = resident;
  return MARKOV_OK;
}

}  // namespace

extern "C" {

size_t markov_workspace_bytes(int rows, int steps, int vocab, int rank, int mode) {
  Shape sh;
  if (check_shape(rows, steps, vocab, rank, mode, &sh) != MARKOV_OK) return 0;
  return kHeader + 2 * half_bytes_needed(rows, steps, sh.NC, mode);
}

int markov_noise_fill(float* gumbel, const int64_t* seeds, int rows, int steps, int vocab,
                      void* stream) {
  g_last_error.clear();
  if (!gumbel || !seeds) return fail(MARKOV_E_INVAL, "null gumbel or seeds");
  if (!aligned16(gumbel)) return fail(MARKOV_E_INVAL, "gumbel is not 16-byte aligned");
  if (rows < 1 || rows > MARKOV_MAX_ROWS || steps < 1 || steps > MARKOV_MAX_STEPS)
    return fail(MARKOV_E_UNSUPPORTED, "rows=%d steps=%d out of range", rows, steps);
  if (vocab < 16 || vocab % 16 != 0 || vocab > MARKOV_MAX_VOCAB)
    return fail(MARKOV_E_UNSUPPORTED, "vocab=%d is not a positive multiple of 16 up to %d", vocab,
                MARKOV_MAX_VOCAB);
  dim3 grid((vocab / 4 + 255) / 256, rows * steps);
  hipLaunchKernelGGL(noise_fill_kernel, grid, dim3(256), 0, (hipStream_t)stream, gumbel, seeds, steps,
                     vocab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "noise launch: %s", hipGetErrorString(e));
  return MARKOV_OK;
}

int markov_chain_sample(const uint16_t* base_logits, int64_t base_row_stride, int64_t base_step_stride,
                        const uint16_t* head, const uint16_t* embed, const int64_t* prev_tokens,
                        const float* temperature, const int64_t* seeds, const float* gumbel,
                        const int64_t* state_idx, float output_multiplier, float soft_cap, int rows,
                        int steps, int vocab, int rank, int mode, int64_t* draft_tokens,
                        int64_t tokens_row_stride, uint16_t* cache, int64_t cache_states,
                        int64_t cache_state_stride, int64_t cache_step_stride, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Shape sh;
  int rc = check_shape(rows, steps, vocab, rank, mode, &sh);
  if (rc != MARKOV_OK) return rc;
  if (!base_logits || !head || !embed || !prev_tokens || !temperature || !draft_tokens || !cache ||
      !workspace)
    return fail(MARKOV_E_INVAL, "a required pointer is null");
  if (mode == MARKOV_MODE_GUMBEL && !gumbel) return fail(MARKOV_E_INVAL, "mode 0 needs gumbel noise");
  if (mode == MARKOV_MODE_INVCDF && !seeds) return fail(MARKOV_E_INVAL, "mode 1 needs seeds");
  if (!aligned16(base_logits) || !aligned16(head) || !aligned16(embed) || !aligned16(cache) ||
      (gumbel && !aligned16(gumbel)))
    return fail(MARKOV_E_INVAL, "base_logits, head, embed, cache and gumbel must be 16-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0) return fail(MARKOV_E_INVAL, "workspace is not 256-byte aligned");
  if (base_step_stride < vocab || base_row_stride < 0 || base_step_stride % 8 || base_row_stride % 8)
    return fail(MARKOV_E_INVAL, "base strides (%lld, %lld) must be multiples of 8 with step stride >= vocab",
                (long long)base_row_stride, (long long)base_step_stride);
  if (cache_step_stride < vocab || cache_state_stride < 0 || cache_step_stride % 8 || cache_state_stride % 8)
    return fail(MARKOV_E_INVAL, "cache strides (%lld, %lld) must be multiples of 8 with step stride >= vocab",
                (long long)cache_state_stride, (long long)cache_step_stride);
  if (cache_states < 1 || (!state_idx && cache_states < rows))
    return fail(MARKOV_E_INVAL, "cache_states=%lld is too small", (long long)cache_states);
  if (tokens_row_stride < steps && rows > 1)
    return fail(MARKOV_E_INVAL, "tokens_row_stride=%lld < steps", (long long)tokens_row_stride);
  if (!isfinite(output_multiplier) || !isfinite(soft_cap) || soft_cap < 0.0f)
    return fail(MARKOV_E_INVAL, "output_multiplier must be finite and soft_cap finite and >= 0");
  const size_t need = kHeader + 2 * half_bytes_needed(rows, steps, sh.NC, mode);
  if (workspace_bytes < need)
    return fail(MARKOV_E_INVAL, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
  int G = 0;
  bool res = false;
  rc = pick_grid(rows, rank, mode, sh, &G, &res);
  if (rc != MARKOV_OK) return rc;

  ChainParams p;
  p.base = base_logits;
  p.base_rs = base_row_stride;
  p.base_ss = base_step_stride;
  p.head = head;
  p.embed = embed;
  p.prev = prev_tokens;
  p.temp = temperature;
  p.seeds = seeds;
  p.gumbel = gumbel;
  p.state_idx = state_idx;
  p.mult = output_multiplier;
  p.cap = soft_cap;
  p.inv_cap = soft_cap > 0.0f ? 1.0f / soft_cap : 1.0f;
  p.has_cap = soft_cap > 0.0f;
  p.rows = rows;
  p.N = steps;
  p.V = vocab;
  p.NG = sh.NG;
  p.NC = sh.NC;
  p.G = G;
  p.tokens = draft_tokens;
  p.tok_rs = tokens_row_stride;
  p.cache = cache;
  p.cache_rs = cache_state_stride;
  p.cache_ss = cache_step_stride;
  p.cache_states = cache_states;
  p.ws = (unsigned char*)workspace;
  p.ws_half = ((workspace_bytes - kHeader) / 2) & ~(size_t)255;

  void* args[] = {&p};
  const size_t shmem = (size_t)rows * rank * 2;
  const void* kern = kernel_for(rank, mode, res);
  rc = prepare_kernels();
  if (rc != MARKOV_OK) return rc;
  hipError_t e = hipLaunchCooperativeKernel(kern, dim3(G), dim3(kThreads), args, (unsigned)shmem,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "chain launch (grid %d): %s", G, hipGetErrorString(e));
  return MARKOV_OK;
}

int markov_status(void* workspace, void* stream) {
  g_last_error.clear();
  if (!workspace) return fail(MARKOV_E_INVAL, "null workspace");
  uint32_t hdr[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(hdr, workspace, sizeof hdr, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "status read: %s", hipGetErrorString(e));
  if (hdr[1] == 0) return MARKOV_OK;
  static const uint32_t zero = 0;
  e = hipMemcpyAsync((char*)workspace + 4, &zero, 4, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "status clear: %s", hipGetErrorString(e));
  return fail(MARKOV_E_DEVICE, "device error bits 0x%x:%s%s%s", hdr[1],
              (hdr[1] & MARKOV_DEVERR_BAD_TOKEN) ? " previous token outside [0, V);" : "",
              (hdr[1] & MARKOV_DEVERR_TIMEOUT) ? " cross-workgroup wait timed out;" : "",
              (hdr[1] & MARKOV_DEVERR_BAD_STATE) ? " state index beyond the cache;" : "");
}

const char* markov_last_error(void) { return g_last_error.c_str(); }

int markov_set_grid(int g) { return g_grid_override.exchange(g < 0 ? 0 : g); }

int markov_grid(int rows, int steps, int vocab, int rank, int mode) {
  g_last_error.clear();
  Shape sh;
  int rc = check_shape(rows, steps, vocab, rank, mode, &sh);
  if (rc != MARKOV_OK) return rc;
  int G = 0;
  bool res = false;
  rc = pick_grid(rows, rank, mode, sh, &G, &res);
  return rc != MARKOV_OK ? rc : G;
}

}  // extern "C"
