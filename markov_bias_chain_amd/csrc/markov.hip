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
//    Each fp32 log is the correctly rounded one, reached through a bucket
//    table, a short fp64 series and a rounding-interval check (the fp64
//    library log decides the rare undecided cases).
//  * With MARKOV_NOISE_INLINE the chain kernel draws the same noise itself:
//    for one row the waves that idle during the exchange draw the next
//    step's values, so the noise costs no launch and no memory traffic.
//  * markov_chain_sample: ONE persistent launch (at most one workgroup per
//    CU) runs all N positions.  The vocabulary is cut into groups of
//    16384 / r head rows (32 KiB of bf16 head each); a wavefront owns one
//    group per chunk, and a chunk is 8 consecutive groups (one per wave of a
//    512-thread workgroup).  When the grid covers every chunk, each wave's
//    group stays in VGPRs for the whole launch (128 VGPRs per lane), so the
//    head is read from HBM once per call; otherwise groups are streamed every
//    step.
//  * The bias GEMV: up to 16 request rows per v_mfma_f32_16x16x32_bf16 pass
//    (head tiles as A, the rows' embeddings from LDS as B), results through
//    a per-wave LDS tile; a single request row swaps the operands (its
//    embedding as A, the head tile as B), so that every lane ends with its
//    vocab id's sum in a register.
//  * The epilogue (bias -> bf16, + base logit, output transform, bf16 cache
//    store, score, per-row best key) handles batches of 8 request rows with
//    8 lanes per row and 8 (r = 256) or 4 (r = 512) consecutive ids per
//    lane, so logits, noise and cache move in 16-byte vectors; per-row
//    maxima are DPP reductions over 8 lanes.
//  * Each step ends in a grid-wide exchange through the workspace: every
//    workgroup stores its candidate (a packed 64-bit (score, index) key) in
//    its own slot with a single agent-scope store, and every workgroup polls
//    all slots, so there is no contended atomic and no second flag.  A zero
//    slot means "not arrived"; real keys are never zero.  Alternate calls use
//    alternate halves of the workspace and each call clears the half the
//    next call will use, so no reset launch is needed.  A single row (or up
//    to 8 rows on a streamed head) on more than 64 workgroups exchanges in
//    two levels: 4 reducer workgroups write their partials into 16 copies,
//    each polled by a sixteenth of the workgroups.  While polling, each wave
//    fetches the embedding of the best key seen so far.
//  * Mode 1 (inverse CDF) publishes per-chunk (max key, sum of exp) partials;
//    a leader workgroup per row locates the chunk holding u * S, scans that
//    chunk's cache values in vocabulary order (stored at agent scope before
//    the partials) and publishes the token in 16 copies, like the one-row
//    partials.

#include <hip/hip_runtime.h>

#include <math.h>
#include <limits.h>
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
constexpr int kAhead = 8;                  // request rows whose next-step inputs are prefetched
constexpr int kLaunchRows = 64;            // request rows of one chain launch
constexpr int kBatch = 8;                  // request rows per epilogue batch
constexpr int kLanesPerRow = 8;            // lanes per request row in a batch
static_assert(kAhead == kBatch, "prefetched rows form one epilogue batch");
constexpr int kHeader = 256;               // workspace header bytes
constexpr int kModeFlags = MARKOV_BASE_F32 | MARKOV_CACHE_F32 | MARKOV_NOISE_INLINE;  // flag bits of `mode`
constexpr int kMaxPollPerLane = 16;        // slots one lane polls (<= 1024 per row)
constexpr int kLeaderRegs = 4;             // inverse-CDF chunks per lane kept in registers by a leader
constexpr int kXCDs = 8;                   // XCDs of the device (workgroups are placed round robin)
constexpr int kPartCopies = 16;            // <= kWaves rows: copies of each step's reducer partials
constexpr int kPartStride = 64;            // u64 words from one copy to the next (512 bytes)
constexpr int kDecCopies = 16;             // inverse CDF: copies of each step's tokens
constexpr unsigned long long kTimeoutTicks = 200000000ull;  // 2 s at 100 MHz (the default wait limit)
constexpr long long kTicksPerUs = 100;                       // s_memrealtime runs at 100 MHz

// ----------------------------------------------------------- bf16 helpers --

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 with the gfx950 conversion instruction (v_cvt_pk_bf16_f32):
// round to nearest even, NaN stays NaN (the cache it writes is compared
// bit for bit with the oracle's software rounding by the parity tests).
__device__ __forceinline__ uint32_t f32_to_bf16_hw(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16_hw(f)); }
// Two fp32 values to two bf16 (a in the low half) with one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Reductions over a whole wave on the DPP/readlane path (no LDS-latency
// swizzles): fold within each 16-lane row with quad permutes and row
// mirrors, then combine the four rows' lanes 0, 16, 32, 48 through scalars.
// Each result is the same value in every lane.
__device__ __forceinline__ uint32_t row_fold_umax(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
  const uint32_t a = __builtin_amdgcn_readlane((int)x, 0), b = __builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = __builtin_amdgcn_readlane((int)x, 32), d = __builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}
// Maximum of a 64-bit value over the wave (high word first, then the low
// word among the lanes that hold the high maximum).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  const uint32_t hi = row_fold_umax((uint32_t)(k >> 32));
  const uint32_t lo = row_fold_umax((uint32_t)(k >> 32) == hi ? (uint32_t)k : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// A signed 32-bit key that orders non-NaN fp32 values as their values do
// (-0 just below +0), and its inverse.
__device__ __forceinline__ int order_key(float z) {
  const int b = __float_as_int(z);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float order_key_inv(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// Signed maximum over the wave on the DPP path only: folds within each
// 16-lane row, then row broadcasts (lane 15 into rows 1 and 3, lane 31 into
// rows 2 and 3) leave the wave maximum in lane 63.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xF, BOUND);
}
__device__ __forceinline__ int wave_imax(int x) {
  x = max(x, dpp_i<0xB1, 0xF, true>(0, x));    // quad_perm [1,0,3,2]
  x = max(x, dpp_i<0x4E, 0xF, true>(0, x));    // quad_perm [2,3,0,1]
  x = max(x, dpp_i<0x141, 0xF, true>(0, x));   // row_half_mirror
  x = max(x, dpp_i<0x140, 0xF, true>(0, x));   // row_mirror
  x = max(x, dpp_i<0x142, 0xA, false>(x, x));  // row_bcast:15
  x = max(x, dpp_i<0x143, 0xC, false>(x, x));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

// Reductions over each group of 8 consecutive lanes (xor 1, xor 2, then the
// mirror within 8); every lane of a group ends with the group's result.
__device__ __forceinline__ int group8_imax(int x) {
  x = max(x, dpp_i<0xB1, 0xF, true>(0, x));
  x = max(x, dpp_i<0x4E, 0xF, true>(0, x));
  x = max(x, dpp_i<0x141, 0xF, true>(0, x));
  return x;
}
__device__ __forceinline__ uint32_t group8_umin(uint32_t x) {
  x = min(x, (uint32_t)dpp_i<0xB1, 0xF, true>(0, (int)x));
  x = min(x, (uint32_t)dpp_i<0x4E, 0xF, true>(0, (int)x));
  x = min(x, (uint32_t)dpp_i<0x141, 0xF, true>(0, (int)x));
  return x;
}
// Inclusive prefix sum over the wave in lane order on the DPP path: shifts
// by 1, 2, 4, 8 within each 16-lane row (lanes shifted in from outside the
// row add 0), then the row broadcasts carry rows 0..2 into the rows above.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += __int_as_float(dpp_i<0x111, 0xF, true>(0, __float_as_int(x)));  // row_shr:1
  x += __int_as_float(dpp_i<0x112, 0xF, true>(0, __float_as_int(x)));  // row_shr:2
  x += __int_as_float(dpp_i<0x114, 0xF, true>(0, __float_as_int(x)));  // row_shr:4
  x += __int_as_float(dpp_i<0x118, 0xF, true>(0, __float_as_int(x)));  // row_shr:8
  x += __int_as_float(dpp_i<0x142, 0xA, false>(0, __float_as_int(x)));  // row_bcast:15
  x += __int_as_float(dpp_i<0x143, 0xC, false>(0, __float_as_int(x)));  // row_bcast:31
  return x;
}
__device__ __forceinline__ float group8_sum(float x) {
  x += __int_as_float(dpp_i<0xB1, 0xF, true>(0, __float_as_int(x)));
  x += __int_as_float(dpp_i<0x4E, 0xF, true>(0, __float_as_int(x)));
  x += __int_as_float(dpp_i<0x141, 0xF, true>(0, __float_as_int(x)));
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

// ---------------------------------------------------------------- tracing --
// Built with -DMARKOV_TRACE (a separate library; off by default), the chain
// and step kernels stamp the 100 MHz s_memrealtime clock at fixed points of
// every step, one thread (thread 0) per workgroup, into trace_buf
// [workgroup][step][phase]; markov_trace_read copies it to the host.  Chain
// kernel phases: 0 step start, 1 local work done (wave 0), 2 keys published,
// 3 reducer partials / inverse-CDF leader work published, 4 winner known
// (wave 0), 5 step end; step 0 also holds 6 kernel entry and 7 prologue
// done.  Inverse CDF, in addition: 8 this workgroup's leader work done (wave
// 0), and the latest of any wave's 9 token published as a row's leader, 10
// partials all seen as a row's leader, 11 chunk chosen.  Step kernel phases (per
// launch): 0 entry, 1 first block's inputs issued, 2 all blocks done, 3 the
// last workgroup's picks done (mode 1: in workgroup 0's entry, the latest
// pick-kernel wave done).
constexpr int kTraceWGs = 1024, kTraceSteps = 32, kTracePhases = 12;
#ifdef MARKOV_TRACE
__device__ unsigned long long trace_buf[kTraceWGs * kTraceSteps * kTracePhases];
#define TRACE_STAMP(wgi, step, ph)                                                            \
  do {                                                                                        \
    if (threadIdx.x == 0 && (step) < kTraceSteps && (wgi) < kTraceWGs)                        \
      trace_buf[((size_t)(wgi) * kTraceSteps + (step)) * kTracePhases + (ph)] = now_ticks(); \
  } while (0)
// From lane 0 of the calling wave; the latest stamp of the workgroup's waves.
#define TRACE_STAMP_MAX(wgi, step, ph)                                                              \
  do {                                                                                              \
    if ((threadIdx.x & 63) == 0 && (step) < kTraceSteps && (wgi) < kTraceWGs)                       \
      __hip_atomic_fetch_max(trace_buf + ((size_t)(wgi) * kTraceSteps + (step)) * kTracePhases + (ph), \
                             (unsigned long long)now_ticks(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
  } while (0)
#else
#define TRACE_STAMP(wgi, step, ph) \
  do {                             \
  } while (0)
#define TRACE_STAMP_MAX(wgi, step, ph) \
  do {                                 \
  } while (0)
#endif

// c / T correctly rounded to fp32 (the IEEE quotient), as c times rT, the
// fp64 reciprocal of T correctly rounded, rounded once to fp32.  For fp32 c
// and T > 0 the fp64 product is within 2^-52 of c / T relatively, and a
// quotient of two fp32 numbers is never within 2^-51 of its magnitude of an
// fp32 rounding midpoint (c 2^j - M T, with M the midpoint's odd 25-bit
// significand, is a nonzero integer), so both round the same way; T = +inf
// gives 0 (or NaN for an infinite c) as the quotient does.  Three fp64/fp32
// operations instead of the division's scale / reciprocal / fma / fixup.
__device__ __forceinline__ float div_by_recip(float c, double rT) { return (float)((double)c * rT); }

// The correctly rounded fp32 natural log: fp64 log of the fp32 argument,
// rounded once (fp32 log libraries are only faithfully rounded).
__device__ __noinline__ float log_f32_rn(float x) { return (float)log((double)x); }

// A faster route to the same correctly rounded fp32 log of a positive
// normal fp32 x.  x = m 2^e with m in [sqrt(1/2), sqrt(2)) (from the bit
// pattern: e = (bits(x) - bits(sqrt(1/2))) >> 23); with the bucket centre
// m_j = 1 + j/128 nearest m, c_j an fp32 value near 1/m_j and r = m c_j - 1
// (exact in fp64: 24-bit times 24-bit), |r| < 2^-7.49,
//   ln x = e ln2 - ln c_j + ln(1 + r),
//   ln(1 + r) = r + r^2 (-1/2 + r (1/3 + r (-1/4 + r/5))) + O(r^6)
// in fp64 (Horner).  The bucket index j + 38 is the integer that the fp32
// rounding of m 128 + 1.5 2^23 - 90 leaves in its low bits (ties to even,
// as a rounding of 128 (m - 1) would), and one 16-byte table entry holds
// c_j and -ln c_j.  The bucket of 1 has c = 1 and ln c = 0, so results near
// 0 keep their relative accuracy; elsewhere |ln m| <= ln2/2 cannot cancel
// e ln2.  The truncated series is within r^6/6 of ln(1 + r), so the fp64
// result y is within 2^11 of its ulps of ln x, the most (relatively) near the
// edges of the bucket of 1, where |r| is up to 2^-8 and |ln x| as small (an
// exhaustive host check over the noise's inputs saw at most 1361; the term
// in r^6 brought that to 5 but cost an fp64 FMA per log); when the 29
// bits of y below fp32 precision are more than 2^12 ulps away from the
// rounding midpoint, rounding y gives the correctly rounded log; otherwise
// (about 2^-16 of the inputs) the fp64 library log decides.
// The buckets j = -38 .. 53: g_log_tab[j + 38] = {c_j, -ln(c_j) correctly
// rounded to fp64} (written by gen_log_table.py).
#include "log_table.inc"
struct LogTable {
  LogEntry e[kLogTable];
};
// The fast part: sets ok = false (and returns garbage) when the library
// log must decide.
__device__ __forceinline__ float log_f32_try(float x, const LogTable& t, bool& ok) {
  const uint32_t b = __float_as_uint(x);
  const int e = (int)(b - 0x3F3504F3u) >> 23;
  const float m = __uint_as_float(b - ((uint32_t)e << 23));
  const float f = __fmaf_rn(m, 128.0f, 12582822.0f);  // 1.5 2^23 + 128 (m - 1) + 38
  const int k = __float_as_int(f) - 0x4B400000;
  const double c = t.e[k].c, nlc = t.e[k].nlc;  // (as scalars: a struct copy lands on the stack)
  const double r = fma((double)m, c, -1.0);
  double q = fma(r, 0.2, -0.25);
  q = fma(r, q, 1.0 / 3.0);
  q = fma(r, q, -0.5);
  const double lp = fma(r * r, q, r);                                   // ln(1 + r)
  const double y = fma((double)e, 0x1.62e42fefa39efp-1, nlc + lp);  // + e ln2
  const uint32_t low = (uint32_t)__double_as_longlong(y) & 0x1FFFFFFFu;
  ok = low - ((1u << 28) - (1u << 12)) > (1u << 13);  // more than 2^12 from the midpoint 2^28
  return (float)y;
}
__device__ __forceinline__ void log_table_load(LogTable& t, int tid, int nthreads) {
  for (int k = tid; k < kLogTable; k += nthreads) t.e[k] = g_log_tab[k];
}

// The uniforms of M consecutive vocabulary ids v0 .. v0 + M - 1 of one
// (seed, row, step) prefix.
template <int M>
__device__ __forceinline__ void noise_uniforms(uint64_t prefix, int v0, float* u) {
#pragma unroll
  for (int j = 0; j < M; ++j) u[j] = hash_uniform(splitmix64(prefix ^ (uint64_t)(uint32_t)(v0 + j)));
}

// Gumbel noise -log(-log u) of M uniforms, both logs correctly rounded.  The
// M evaluations are independent (their fast paths interleave); the rare
// library-log fallbacks run afterwards.
template <int M>
__device__ __forceinline__ void gumbel_from_uniforms(const float* u, const LogTable& t, float* g) {
  float x[M];
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    x[j] = u[j];
    bool ok;
    g[j] = log_f32_try(x[j], t, ok);
    bad |= (ok ? 0u : 1u) << j;
  }
  if (bad) {
#pragma unroll
    for (int j = 0; j < M; ++j)
      if ((bad >> j) & 1u) g[j] = log_f32_rn(x[j]);
  }
  bad = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    x[j] = -g[j];  // -log u, positive
    bool ok;
    g[j] = log_f32_try(x[j], t, ok);
    bad |= (ok ? 0u : 1u) << j;
  }
  if (bad) {
#pragma unroll
    for (int j = 0; j < M; ++j)
      if ((bad >> j) & 1u) g[j] = log_f32_rn(x[j]);
  }
#pragma unroll
  for (int j = 0; j < M; ++j) g[j] = -g[j];
}

// Gumbel noise of M consecutive vocabulary ids v0 .. v0 + M - 1 of one
// (seed, row, step) prefix.
template <int M>
__device__ __forceinline__ void gumbel_noise(uint64_t prefix, int v0, const LogTable& t, float* g) {
  float u[M];
  noise_uniforms<M>(prefix, v0, u);
  gumbel_from_uniforms<M>(u, t, g);
}

// ============================================================== noise fill ==

__global__ __launch_bounds__(256) void noise_fill_kernel(float* __restrict__ gumbel,
                                                         const int64_t* __restrict__ seeds,
                                                         int steps, int V) {
  const int step = blockIdx.y, row = blockIdx.z;
  const int rs = row * steps + step;
  __shared__ LogTable tab;
  log_table_load(tab, threadIdx.x, 256);
  // the hashes while the table's loads are in flight
  // two tiles of 1024 ids per block (one table load and barrier for both:
  // 256 rows 490.7 -> 482.1 us per fill)
  const int v0 = (blockIdx.x * 512 + threadIdx.x) * 4, v1 = v0 + 1024;
  const uint64_t pre = noise_prefix(seeds[row], row, step);
  float u[8];
  noise_uniforms<4>(pre, v0, u);
  noise_uniforms<4>(pre, v1, u + 4);
  __syncthreads();
  if (v0 >= V) return;  // V is a multiple of 16: a thread's 4 ids are all valid
  float out[4];
  gumbel_from_uniforms<4>(u, tab, out);
  *reinterpret_cast<float4*>(gumbel + (size_t)rs * V + v0) = make_float4(out[0], out[1], out[2], out[3]);
  if (v1 >= V) return;
  gumbel_from_uniforms<4>(u + 4, tab, out);
  *reinterpret_cast<float4*>(gumbel + (size_t)rs * V + v1) = make_float4(out[0], out[1], out[2], out[3]);
}

// ==================================================== allocation-free scratch ==
// markov_chain_sample_noalloc keeps the chain's workspace in this array
// instead of a caller's buffer: 8 MiB, enough for every shape whose
// markov_workspace_bytes is at most that (each device the library runs on
// holds its own copy until the process ends).  Host code never uses the name
// itself as an address: it takes the array's device address per device with
// hipGetSymbolAddress and passes that pointer.
constexpr size_t kScratchBytes = MARKOV_NOALLOC_MAX_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zeroes n16 16-byte words (a fill kernel rather than a memset, so that a
// call captured in a graph records a kernel node).
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t k = (size_t)blockIdx.x * 256 + threadIdx.x; k < n16; k += (size_t)gridDim.x * 256)
    p[k] = make_uint4(0, 0, 0, 0);
}

// ============================================================ chain kernel ==

struct ChainParams {
  const void* base;  // bf16 bits, or fp32 when base_f32
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
  int row_base;  // the call's row index of this launch's row 0
  int64_t* tokens;
  long long tok_rs;
  void* cache;  // bf16 bits, or fp32 when cache_f32
  long long cache_rs, cache_ss;
  int base_f32, cache_f32;
  long long cache_states;
  unsigned char* ws;
  unsigned long long ws_half;  // bytes per parity half
  unsigned long long clear_bytes;  // bytes of the other half each call clears (<= ws_half)
  unsigned long long wait_ticks;  // bound of every cross-workgroup wait (s_memrealtime ticks)
  int nres;  // streamed head: 0, or kParked<R>: chunk 1's tiles kept in LDS after step 0
};

// Streamed head: the tile slots per wave of a workgroup's chunk 1 kept in LDS
// across steps when they fit beside the kernel's static arrays and the
// embeddings (160 KiB of LDS: up to 13 rows at r = 512, 10 at r = 256).
template <int R>
constexpr int kParked = R == 512 ? 15 : 14;

// Workspace half layout (slot arrays of one parity; every slot is written at
// most once per call, and 0 means "not written yet"):
//   keys [N][rows][NC] u64     candidate keys (mode 0: one per workgroup,
//                               mode 1: one per chunk)
//   mode 0, more than kWaves rows:
//   part [N][rows][NR] u64     reducer r's maximum over slots 64 r .. 64 r + 63
//   mode 0, at most kWaves rows (when there are reducers):
//   part [N][rows][kPartCopies][kPartStride] u64   reducer r's maximum in
//                               word r of every copy; workgroup g polls copy
//                               g % kPartCopies
//   mode 1:
//   tok  [N][kDecCopies][rows] u64   the row leader's token for the row, in
//                               every copy; workgroup g polls copy g % kDecCopies
//   sums [N][rows][NC] u32     sum of exp(z - chunk max), sign bit set
// (64-bit arrays first, so that every array is aligned to its element size.)
struct HalfLayout {
  uint64_t* keys;
  uint64_t* part;
  uint64_t* tok;
  uint32_t* sums;
};

// Reducer workgroups of the two-level mode-0 exchange (slots per reducer: 64).
__host__ __device__ inline int reducers_for(int NC) { return (NC + 63) / 64; }

// The chunk held by workgroup wg of a G-workgroup launch whose workgroups
// each hold one chunk, such that the workgroups of one XCD (launched round
// robin, workgroup wg on XCD wg % kXCDs) hold one contiguous run of chunks:
// XCD x gets G / kXCDs workgroups, one more for x < G % kXCDs, in order.
// A bijection on [0, G) whatever the placement.  (Loading the 66 MB
// DeepSeek-sized head with 253 workgroups, the last workgroup is done after
// 9.7 us this way against 10.8-10.9 us with chunk wg: with chunk wg the odd
// XCDs, XCDs 5 and 7 the most, take up to 2.5 us longer than the even ones.
// Per call: one row 39.5 -> 38.1 us, 8 rows 58.9 -> 57.6 us, the r = 512
// streamed head 574 -> 532 us, 64-row inverse CDF 224.0 -> 222.9 us.)
__host__ __device__ inline int xcd_run_chunk(int wg, int G) {
  const int x = wg % kXCDs, k = wg / kXCDs, q = G / kXCDs, r = G % kXCDs;
  return x * q + (x < r ? x : r) + k;
}
// Whether the partials of a launch of `rows` rows are kept in copies.
__host__ __device__ inline bool copied_parts(int rows, int NC) { return rows <= kWaves && reducers_for(NC) > 1; }

__host__ __device__ inline size_t half_bytes_needed(int rows, int N, int NC, int mode) {
  const size_t slots = (size_t)N * rows * NC;
  size_t b = slots * 8;
  if (mode == 1) {
    b += (size_t)N * kDecCopies * rows * 8 + slots * 4;
  } else if (copied_parts(rows, NC)) {
    b += (size_t)N * rows * kPartCopies * kPartStride * 8;
  } else {
    b += (size_t)N * rows * reducers_for(NC) * 8;
  }
  return (b + 255) & ~(size_t)255;
}

// A call of more than kLaunchRows rows runs either as persistent launches of
// kLaunchRows rows and one of the rest, one after another in the same
// workspace, or as step-kernel launches per position over all its rows (any
// call, when the path knob asks for them): its half holds the larger of
// those layouts.
__host__ size_t step_half_bytes_host(int rows, int rank, int mode, int NC);
__host__ inline size_t call_half_bytes(int rows, int N, int NC, int mode, int rank) {
  const int full = rows < kLaunchRows ? rows : kLaunchRows;
  size_t b = half_bytes_needed(full, N, NC, mode);
  const int tail = rows % kLaunchRows;
  if (rows > kLaunchRows && tail != 0) {
    const size_t t = half_bytes_needed(tail, N, NC, mode);
    if (t > b) b = t;
  }
  const size_t t = step_half_bytes_host(rows, rank, mode, NC);
  if (t > b) b = t;
  return b;
}

__device__ inline HalfLayout half_layout(unsigned char* half, int rows, int N, int NC, int mode) {
  HalfLayout L = {};
  const size_t slots = (size_t)N * rows * NC;
  uint64_t* cur = reinterpret_cast<uint64_t*>(half);
  L.keys = cur;
  cur += slots;
  if (mode == 1) {
    L.tok = cur;
    L.sums = reinterpret_cast<uint32_t*>(L.tok + (size_t)N * kDecCopies * rows);
  } else {
    L.part = cur;
  }
  return L;
}

// ------------------------------------------------------------ bias GEMV --
// The bias of a group of RPG = 16384 / r head rows for up to 16 request rows
// is a [RPG x r] . [r x 16] product on the matrix cores:
// v_mfma_f32_16x16x32_bf16 computes D[16 x 16] += A[16 x 32] . B[32 x 16]
// with fp32 accumulation (products of bf16 are exact in fp32).  Operand
// layouts (lane l of the wave): A[i][k] in lane i + 16 (k / 8), element
// k % 8; B[k][j] in lane j + 16 (k / 8); D[i][j] in lane j + 16 (i / 4),
// element i % 4.
//
// A group is 32 tiles of 16 rows x 32 k (MT = RPG / 16 row tiles by
// KT = r / 32 k tiles); tile (t, kt) is slot t * KT + kt, 16 bytes per lane:
// lane l holds head[16 t + (l & 15)][32 kt + 8 (l >> 4) + 0..7], so every
// load instruction reads 16 rows x 64 contiguous bytes.  B for k tile kt is
// the request rows' embeddings at the same k offsets, read from LDS.  The
// sums depend only on the group's rows and the embeddings, never on the
// grid, so the bias is grid-invariant.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowPass = 16;  // request rows per MFMA pass (the N of the tile)

template <int R>
__device__ __forceinline__ uint4 load_head_tile(const uint16_t* __restrict__ head, int g, int s,
                                                int lane, int V) {
  constexpr int KT = R / 32;
  const int t = s / KT, kt = s - (s / KT) * KT;
  const int row = g * (16384 / R) + 16 * t + (lane & 15);
  if (row >= V) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(head + (size_t)row * R + 32 * kt + 8 * (lane >> 4));
}

// The same tile with rows at or beyond V read from row V - 1 instead of set
// to zero: one unconditional load, whose wait can be counted past later
// loads.  The sums of those rows are never used (every epilogue checks
// v < V), so their values do not matter.
template <int R>
__device__ __forceinline__ uint4 load_head_tile_clamped(const uint16_t* __restrict__ head, int g, int s,
                                                        int lane, int V) {
  constexpr int KT = R / 32;
  const int t = s / KT, kt = s - (s / KT) * KT;
  const int row = g * (16384 / R) + 16 * t + (lane & 15);
  const int rc = row < V ? row : V - 1;
  return *reinterpret_cast<const uint4*>(head + (size_t)rc * R + 32 * kt + 8 * (lane >> 4));
}

// Row stride (floats) of a wave's bias tile in LDS: RPG + 4 keeps the 16
// request rows' 16-byte writes on different banks.
template <int R>
constexpr int bias_stride() { return 16384 / R + 4; }

// Row stride (16-byte vectors) of the embeddings in LDS: r/8 + 1 keeps the
// 16 request rows' reads of one k tile on different banks.
template <int R>
constexpr int emb_stride() { return R / 8 + 1; }

// sb[j * bias_stride + row] = sum_k head[row][k] * embed_row(b0 + j)[k] for
// j < nb; rows beyond nb get nothing.  The embedding pieces of EB k tiles are
// read from LDS together, before their products, and the scheduler may not
// sink those reads between the products: KT / EB LDS round trips per pass.
// Left to itself the compiler waited for each k tile's read just before its
// products.  EB = 2 costs no registers in any kernel here; larger EB costs
// 4 (EB - 1) VGPRs beyond one, and spills in kernels that hold the head and
// two batches of inputs, so each caller picks the largest EB its registers
// allow.
template <int R, int EB>
__device__ __forceinline__ void group_bias(const uint4 (&h)[kSlots], const uint4* __restrict__ s_e,
                                           int b0, int nb, int lane, float* __restrict__ sb) {
  constexpr int KT = R / 32, MT = kSlots / KT, ES = emb_stride<R>();
  static_assert(KT % EB == 0, "EB divides the k tiles");
  const int j = lane & 15;
  const bool jv = j < nb;
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k0 = 0; k0 < KT; k0 += EB) {
    uint4 ea[EB];
#pragma unroll
    for (int k = 0; k < EB; ++k)
      ea[k] = jv ? s_e[(b0 + j) * ES + 4 * (k0 + k) + (lane >> 4)] : make_uint4(0, 0, 0, 0);
    if constexpr (EB > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < EB; ++k) {
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, ea[k]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, h[t * KT + k0 + k]), bv,
                                                          acc[t], 0, 0, 0);
    }
  }
  if (jv) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
      *reinterpret_cast<float4*>(sb + j * bias_stride<R>() + 16 * t + 4 * (lane >> 4)) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
}

// One request row on MFMA with the roles of group_bias swapped: the
// embedding is the A operand, the same in all 16 rows of the tile (lane l
// supplies k = 32 kt + 8 (l >> 4) .. + 7, as a B operand would), and the head
// tile is the B operand (lane l holds head row 16 t + (l & 15) at those k,
// which is also the B layout).  Every row of the 16 x 16 result is then the
// bias of the tile's 16 head rows, so lane l finds the bias of head row
// 16 t + (l & 15) in element 0 of tile t's accumulator and keeps tile
// t = l >> 4 (r = 256: four tiles, lane l gets group row l) or t = (l >> 4) & 1
// (r = 512: two tiles, lanes 0..31 get group rows 0..31).  No reduction
// across lanes is needed.  (Against v_dot2c_f32_bf16 with a reduce-scatter
// across the quarters: 40.5 -> 40.0 us per DeepSeek-sized one-row call with
// inline noise, 38.9 -> 38.3 us with the noise read; splitting the tiles
// between MFMA and dot2 was slower than either.)  e_row is the request row's
// embedding in LDS.
template <int R>
__device__ __forceinline__ float one_row_bias(const uint4 (&h)[kSlots], const uint4* __restrict__ e_row,
                                              int lane) {
  constexpr int KT = R / 32, MT = kSlots / KT;
  static_assert(MT == 2 || MT == 4, "r = 256 or 512");
  const int q = lane >> 4;
  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // All of the lane's embedding pieces are read before the first product,
  // and the scheduler may not sink the reads between the products: one LDS
  // round trip per call instead of one per k tile (one row: 40.3 -> 40.0 us
  // per call with inline noise).
  uint4 ea[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) ea[kt] = e_row[4 * kt + q];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const bf16x8_t ev = __builtin_bit_cast(bf16x8_t, ea[kt]);
#pragma unroll
    for (int t = 0; t < MT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ev, __builtin_bit_cast(bf16x8_t, h[t * KT + kt]), acc[t],
                                                        0, 0, 0);
  }
  const int tl = q & (MT - 1);
  float b = acc[0][0];
#pragma unroll
  for (int t = 1; t < MT; ++t) b = tl == t ? acc[t][0] : b;
  return b;
}

// A request row's constants for one call, in registers.
struct RowConsts {
  bool active;
  float T;
  double rT;
  int state;
};

// FL: the element-type flags of mode are read (fp32 base logits or cache);
// without it both are bf16.  RES: every
// workgroup owns exactly one chunk (G == NC) and keeps its head in VGPRs
// for the whole launch.  !RES: workgroups stride over the chunks and stream
// the head from memory at every step.  SMALL (with RES): at most kAhead
// request rows, whose next-step inputs are prefetched in registers during
// the exchange.  ONE (with SMALL, mode 0): a single request row, whose bias
// and epilogue stay in registers.  NZ (mode 0): the noise is drawn inline
// from the seeds instead of read from memory.
template <int R, int MODE, bool RES, bool SMALL, bool ONE, bool FL, bool NZ>
__global__ __launch_bounds__(kThreads, 1) void chain_kernel(ChainParams p) {
  // Only the FL variants read the flags (bf16, noise from memory otherwise).
  const bool base_f32 = FL && p.base_f32;
  const bool cache_f32 = FL && p.cache_f32;
  const bool nz_inline = MODE == 0 && NZ;
  constexpr int RPG = 16384 / R;       // head rows per group
  constexpr int CHUNK = kWaves * RPG;  // vocab ids per chunk
  constexpr int KSEG = R / 8;          // 16-byte segments per head row
  constexpr int ES = emb_stride<R>();  // LDS row stride of the embeddings
  constexpr int BS = bias_stride<R>(); // LDS row stride of a wave's bias tile

  __shared__ int s_state[kLaunchRows];
  __shared__ int s_active[kLaunchRows];
  __shared__ float s_T[kLaunchRows];
  __shared__ double s_rT[kLaunchRows];  // RN64(1 / T) of the rows with T > 0
  __shared__ int64_t s_seed[kLaunchRows];  // mode 1: the rows' seeds
  __shared__ int s_tok[kLaunchRows];
  __shared__ uint64_t s_key[kWaves][kLaunchRows];
  __shared__ float s_wsum[kWaves][kLaunchRows];
  __shared__ float s_bias[kWaves][kRowPass * BS];  // each wave's [16][RPG] bias tile
  // the next step's base logits of every batch (inverse CDF, resident head, > kAhead rows)
  __shared__ uint32_t s_pre[(MODE == 1 && RES && !SMALL) ? kWaves * (kLaunchRows / kBatch) * (RPG / 16) * 64 : 1];
  __shared__ LogTable s_log;   // the noise's log table (mode 0, inline noise)
  __shared__ float s_nz0[64];  // one row, inline noise: wave 0's next-step noise (reducers)
  __shared__ int s_abort;
  __shared__ uint32_t s_parity;
  // Dynamic LDS: [rows][ES] 16-byte vectors of the current embeddings, then
  // (streamed head) [kWaves][nres][64] head tiles of the workgroup's chunk 1.
  extern __shared__ uint4 s_e[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wg = blockIdx.x;
  const int rows = p.rows, N = p.N, V = p.V, G = p.G, NC = p.NC, NG = p.NG;
  uint32_t* header = reinterpret_cast<uint32_t*>(p.ws);
  const uint64_t deadline = now_ticks() + p.wait_ticks;
  TRACE_STAMP(wg, 0, 6);
  // This workgroup's first chunk, in the XCD-contiguous assignment; a
  // streamed head's workgroup takes every G-th chunk from there (chunks
  // wc + j G).  Key slots stay indexed by workgroup, keys carry vocabulary
  // ids and partials are indexed by chunk, so nothing else depends on
  // which workgroup holds which chunk.
  const int wc = xcd_run_chunk(wg, G);
  // Batches of 2 to 8 prefetched rows: wave 0 (whose first threads publish
  // every row's key) wins issue against its SIMD's other wave (8 rows with
  // inline noise 60.9 -> 60.3 us per call; for one row or 64 rows the
  // same priority was slower).
  if (MODE == 0 && SMALL && !ONE && wave == 0) __builtin_amdgcn_s_setprio(3);
  // In the epilogue lane l owns group row lr (r = 512 groups have 32 rows:
  // lanes 32..63 have none).
  const int lr = (R == 256) ? lane : (lane & 31);
  const bool lane_owns = (R == 256) || lane < 32;

  // ---- prologue: rows, parity, the resident head into VGPRs.
  // The rows' data, the call parity and the noise's log table are loaded
  // before the head: loads complete in order, so waiting for them does not
  // wait for the head, which streams in while the prologue goes on.
  // (Unconditional loads from clamped indices, so that the waits for them
  // are counted past the head's loads.)
  static_assert(kLaunchRows <= kThreads && kLogTable <= kThreads, "one prologue load per thread");
  const int b_row = tid;
  const bool row_thread = b_row < rows;
  const int b_ld = row_thread ? b_row : 0;
  const int64_t* st_src = p.state_idx ? p.state_idx : p.prev;
  const int64_t r_sti = st_src[b_ld];
  const int64_t r_tok = p.prev[b_ld];
  const float r_T = p.temp[b_ld];
  const int64_t r_seed = (MODE == 1 || nz_inline) ? p.seeds[b_ld] : 0;
  const bool tab_thread = MODE == 0 && nz_inline && tid < kLogTable;
  double t_c = 0.0, t_nlc = 0.0;  // (scalars: a struct here lands on the stack)
  if (MODE == 0 && nz_inline) {
    const int k = tid < kLogTable ? tid : 0;
    t_c = g_log_tab[k].c;
    t_nlc = g_log_tab[k].nlc;
  }
  const uint32_t par = ld_agent32(header);
  // One row: the step-0 base logit (bf16 bits) of this lane's vocabulary id;
  // its first use comes after the head is issued, so its wait does not wait
  // for the head.  (Shifted where it was loaded, it held the step-0 noise
  // draw back until the whole head had arrived.)
  uint32_t b0_bits = 0;
  if constexpr (ONE && !FL) {
    const int v = (wc * kWaves + wave) * RPG + lr;
    b0_bits = reinterpret_cast<const uint16_t*>(p.base)[v < V ? v : V - 1];
  }
  uint4 h[kSlots];
  if constexpr (RES) {
    const int g0 = wc * kWaves + wave;  // this wave's group
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
      h[s] = load_head_tile_clamped<R>(p.head, g0 < NG ? g0 : NG - 1, s, lane, V);
  }
  if (tid == 0) {
    s_parity = par;
    s_abort = 0;
  }
  if (tab_thread) {
    s_log.e[tid].c = t_c;
    s_log.e[tid].nlc = t_nlc;
  }
  if (row_thread) {
    const int b = b_row;
    const int64_t st = p.state_idx ? r_sti : p.row_base + b_row;
    const int64_t tok = r_tok;
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
    s_T[b] = r_T;
    s_rT[b] = r_T > 0.0f ? 1.0 / (double)r_T : 0.0;
    s_seed[b] = r_seed;
    s_tok[b] = active ? (int)tok : 0;
  }
  // An LDS-only barrier: the head's loads stay in flight.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const uint32_t parity = s_parity & 1u;
  unsigned char* half = p.ws + kHeader + parity * p.ws_half;
  {
    // Clear the other half for the next call (nobody reads it in this one).
    uint4* other = reinterpret_cast<uint4*>(p.ws + kHeader + (parity ^ 1u) * p.ws_half);
    const size_t n16 = p.clear_bytes / 16;
    for (size_t k = (size_t)wg * kThreads + tid; k < n16; k += (size_t)G * kThreads)
      other[k] = make_uint4(0, 0, 0, 0);
  }
  const HalfLayout L = half_layout(half, rows, N, NC, MODE);
  // ---- per-step inputs.
  // Single row (lane = vocab id): the base logit and noise of lane lr's id,
  // prefetched for the next step while the current step's exchange is in
  // flight (they do not depend on the winner).
  constexpr bool ahead = RES && SMALL;
  const int v_res = (wc * kWaves + wave) * RPG + lr;
  const bool own_res = (wc * kWaves + wave) < NG && v_res < V && lane_owns;
  uint32_t one_base = 0;
  float one_noise = 0.0f;
  // Inline noise: waves 1 .. 7 draw the next step's noise here, while wave
  // 0 alone waits for the exchange, and wave 1 also draws wave 0's values
  // (into s_nz0), so the polling wave draws nothing.  (Wave 0 drawing its
  // own inside its first poll, behind the poll's loads, kept the draw's
  // registers live in the poll loop: 47 SGPR spills against 20, and 42.7 ->
  // 41.6 us per call on the DeepSeek-sized row.)  Step 0's noise every wave
  // draws here.
  const bool one_nz = MODE == 0 && ONE && nz_inline;
  const bool w0_by_w1 = one_nz;
  auto draw_one = [&](int i) {
    if (s_active[0] && own_res && s_T[0] > 0.0f)
      gumbel_noise<1>(noise_prefix(s_seed[0], p.row_base, i), v_res, s_log, &one_noise);
  };
  auto prefetch_one = [&](int i) {
    one_base = 0;
    one_noise = 0.0f;
    if (s_active[0] && own_res) {
      // the base logit as fp32 bits (a bf16 value widened)
      const long long at = (long long)i * p.base_ss + v_res;
      if (!FL && i == 0)
        one_base = b0_bits << 16;
      else
        one_base = base_f32 ? reinterpret_cast<const uint32_t*>(p.base)[at]
                              : (uint32_t)reinterpret_cast<const uint16_t*>(p.base)[at] << 16;
      if (MODE == 0 && s_T[0] > 0.0f && !one_nz) one_noise = p.gumbel[(size_t)i * V + v_res];
    }
    if (one_nz && (wave != 0 || i == 0)) draw_one(i);
    if (w0_by_w1 && wave == 1 && i > 0 && s_active[0] && s_T[0] > 0.0f) {
      const int g0 = wc * kWaves;  // wave 0's group
      const int v = g0 * RPG + lr;
      if (g0 < NG && v < V && lane_owns) gumbel_noise<1>(noise_prefix(s_seed[0], p.row_base, i), v, s_log, &s_nz0[lane]);
    }
  };
  // Several rows: a batch of kBatch request rows is spread over the wave,
  // kLanesPerRow lanes per row; lane l serves row b0 + (l >> 3) and the IPL
  // consecutive vocab ids g * RPG + (l & 7) * IPL + 0 .. IPL - 1 of group g,
  // so its base logits, noise and cache values move in 16-byte vectors.
  // V is a multiple of 16, so a lane's ids are all valid or all not.
  constexpr int IPL = RPG / kLanesPerRow;  // vocab ids per lane: 8 (r = 256) or 4 (r = 512)
  static_assert(kBatch * kLanesPerRow == 64 && (IPL == 8 || IPL == 4), "batch layout");
  const int rr = lane >> 3;  // row of the batch
  const int q = lane & 7;    // vocab segment of the group
  struct LaneIn {
    uint32_t bw[IPL];  // base logits: two bf16 per word (words 0 .. IPL/2 - 1), or IPL fp32
    float nz[IPL];     // noise
  };
  auto load_rows = [&](int i, int b0, int g, LaneIn& in) {
#pragma unroll
    for (int e = 0; e < IPL; ++e) in.bw[e] = 0;
#pragma unroll
    for (int e = 0; e < IPL; ++e) in.nz[e] = 0.0f;
    int b = b0 + rr;
    // Opaque to the optimiser: otherwise it hoists every batch's 64-bit row
    // address out of the step loop and spills them.
    asm volatile("" : "+v"(b));
    const int v0 = g * RPG + q * IPL;
    if (b < rows && g < NG && v0 < V && s_active[b]) {
      const long long at = (long long)b * p.base_rs + (long long)i * p.base_ss + v0;
      if (base_f32) {
        const uint4* brow = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.base) + at);
#pragma unroll
        for (int e4 = 0; e4 < IPL / 4; ++e4) {
          const uint4 t = brow[e4];
          in.bw[4 * e4] = t.x, in.bw[4 * e4 + 1] = t.y, in.bw[4 * e4 + 2] = t.z, in.bw[4 * e4 + 3] = t.w;
        }
      } else {
        const uint16_t* brow = reinterpret_cast<const uint16_t*>(p.base) + at;
        if constexpr (IPL == 8) {
          const uint4 t = *reinterpret_cast<const uint4*>(brow);
          in.bw[0] = t.x, in.bw[1] = t.y, in.bw[2] = t.z, in.bw[3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(brow);
          in.bw[0] = t.x, in.bw[1] = t.y;
        }
      }
      if (MODE == 0 && s_T[b] > 0.0f) {
        if (nz_inline) {
          // Prefetched rows draw it here, four ids at a time (right after
          // the publication, before the exchange's polls); the others in the
          // epilogue (where fewer registers are live).
          if constexpr (SMALL) {
            const uint64_t pre = noise_prefix(s_seed[b], p.row_base + b, i);
#pragma unroll
            for (int e = 0; e < IPL; e += 4) gumbel_noise<4>(pre, v0 + e, s_log, in.nz + e);
          }
        } else {
          const float4* grow = reinterpret_cast<const float4*>(p.gumbel + ((size_t)b * N + i) * (size_t)V + v0);
#pragma unroll
          for (int e4 = 0; e4 < IPL / 4; ++e4) {
            const float4 t = grow[e4];
            in.nz[4 * e4] = t.x, in.nz[4 * e4 + 1] = t.y, in.nz[4 * e4 + 2] = t.z, in.nz[4 * e4 + 3] = t.w;
          }
        }
      }
    }
  };
  LaneIn pre;  // the resident SMALL kernel's prefetched batch
  auto prefetch = [&](int i) {
    if constexpr (ONE) prefetch_one(i);
    else load_rows(i, 0, wc * kWaves + wave, pre);
  };
  // Embeddings of the anchor tokens; the first pass's loads are in flight
  // during the step-0 prefetch (which may draw noise).
  {
    const int b = tid / KSEG, seg = tid - b * KSEG;
    const bool mine = tid < rows * KSEG && s_active[b];
    uint4 e = make_uint4(0, 0, 0, 0);
    if (mine) e = *reinterpret_cast<const uint4*>(p.embed + (size_t)s_tok[b] * R + seg * 8);
    if (ahead) prefetch(0);
    if (mine) s_e[b * ES + seg] = e;
  }
  for (int k = tid + kThreads; k < rows * KSEG; k += kThreads) {
    const int b = k / KSEG, seg = k - b * KSEG;
    if (s_active[b])
      s_e[b * ES + seg] = *reinterpret_cast<const uint4*>(p.embed + (size_t)s_tok[b] * R + seg * 8);
  }
  __syncthreads();
  // Inverse CDF with a resident head and more than kAhead rows: every
  // batch's base logits of the next step are loaded before the step's
  // exchange and parked in LDS (s_pre, each wave's own lanes), so the local
  // work reads no global memory.
  constexpr bool stage = MODE == 1 && RES && !SMALL;
  constexpr int kStageBatches = kLaunchRows / kBatch;
  uint32_t pst[stage ? kStageBatches : 1][IPL / 2];  // bf16 pairs of every batch
  auto stage_load = [&](int i) {
    const int nbat = (rows + kBatch - 1) / kBatch;
    const int g = wc * kWaves + wave;
    const int v0 = g * RPG + q * IPL;
#pragma unroll
    for (int t = 0; t < (stage ? kStageBatches : 1); ++t) {
#pragma unroll
      for (int e = 0; e < IPL / 2; ++e) pst[t][e] = 0;
      int b = t * kBatch + rr;
      asm volatile("" : "+v"(b));  // keeps the row addresses inside the step loop
      if (t < nbat && b < rows && g < NG && v0 < V && s_active[b]) {
        const uint16_t* brow = reinterpret_cast<const uint16_t*>(p.base) +
                               ((long long)b * p.base_rs + (long long)i * p.base_ss + v0);
        if constexpr (IPL == 8) {
          const uint4 w4 = *reinterpret_cast<const uint4*>(brow);
          pst[t][0] = w4.x, pst[t][1] = w4.y, pst[t][2] = w4.z, pst[t][3] = w4.w;
        } else {
          const uint2 w2 = *reinterpret_cast<const uint2*>(brow);
          pst[t][0] = w2.x, pst[t][1] = w2.y;
        }
      }
    }
  };
  auto stage_park = [&]() {
    const int nbat = (rows + kBatch - 1) / kBatch;
#pragma unroll
    for (int t = 0; t < (stage ? kStageBatches : 1); ++t)
      if (t < nbat) {
#pragma unroll
        for (int e = 0; e < IPL / 2; ++e) s_pre[((wave * kStageBatches + t) * (IPL / 2) + e) * 64 + lane] = pst[t][e];
      }
  };
  auto stage_fetch = [&](int t, LaneIn& in) {
#pragma unroll
    for (int e = 0; e < IPL / 2; ++e) in.bw[e] = s_pre[((wave * kStageBatches + t) * (IPL / 2) + e) * 64 + lane];
#pragma unroll
    for (int e = 0; e < IPL; ++e) in.nz[e] = 0.0f;
  };
  if (stage && !base_f32) {
    stage_load(0);
    stage_park();
  }

  // A row's constants for the call (written once in the prologue).  With
  // at most kAhead rows (one batch) they are read before the bias pass, so
  // that these LDS reads overlap the pass's embedding reads instead of
  // waiting one after another in the epilogue, and the compiler keeps them
  // in registers; larger batches read them in the epilogue (in registers
  // across the pass they cost those kernels spills).
  auto row_consts = [&](int b) {
    RowConsts c;
    c.active = s_active[b] != 0;
    c.T = s_T[b];
    c.rT = s_rT[b];
    c.state = s_state[b];
    return c;
  };

  // Epilogue of the batch of rows b0 .. b0 + nb - 1 in the layout above:
  // per vocab id, bias -> bf16, + base logit, output transform, bf16 cache
  // store (one vector per lane), score; then per row the best (score, id)
  // key of the wave's group and, in mode 1, the group's sum of exp(z - max).
  // sbt is the wave's bias tile row block of the batch (row rr at rr * BS);
  // with SMALL, rc0 holds the lane's row's constants (row_consts(b0 + rr)).
  auto epilogue_rows = [&](int i, int b0, int nb, int g, const float* sbt, const LaneIn& in, bool nz_ready,
                           const RowConsts& rc0) {
    const int b = b0 + rr;
    const int v0 = g * RPG + q * IPL;
    const bool ok = rr < nb && g < NG && v0 < V && (SMALL ? rc0.active : s_active[b] != 0);
    const float T = SMALL ? rc0.T : s_T[b];
    const double rT = SMALL ? rc0.rT : s_rT[b];
    float bsum[IPL];
#pragma unroll
    for (int e4 = 0; e4 < IPL / 4; ++e4) {
      const float4 t = *reinterpret_cast<const float4*>(sbt + rr * BS + q * IPL + 4 * e4);
      bsum[4 * e4] = t.x, bsum[4 * e4 + 1] = t.y, bsum[4 * e4 + 2] = t.z, bsum[4 * e4 + 3] = t.w;
    }
    float x[IPL];
#pragma unroll
    for (int e = 0; e < IPL; ++e) {
      const uint32_t w = in.bw[e / 2];
      const float base = base_f32 ? __uint_as_float(in.bw[e])
                                    : __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
      x[e] = __fmul_rn(__fadd_rn(base, bf16_round(bsum[e])), p.mult);
    }
    if (p.has_cap) {
#pragma unroll
      for (int e = 0; e < IPL; ++e) x[e] = __fmul_rn(tanhf(__fmul_rn(x[e], p.inv_cap)), p.cap);
    }
    // The cache value: x rounded to bf16, or x itself in an fp32 cache.
    uint32_t cw[IPL / 2];
    float z[IPL];
#pragma unroll
    for (int e = 0; e < IPL / 2; ++e) {
      cw[e] = f32x2_to_bf16x2(x[2 * e], x[2 * e + 1]);
      z[2 * e] = cache_f32 ? x[2 * e] : __uint_as_float(cw[e] << 16);
      z[2 * e + 1] = cache_f32 ? x[2 * e + 1] : __uint_as_float(cw[e] & 0xFFFF0000u);
    }
    if (ok && MODE == 1) {
      // Inverse CDF: agent-scope stores (written through to the device's
      // coherence point), because the leader workgroup of the row, perhaps
      // on another XCD, scans the chosen chunk's values in this step; each
      // wave waits for them before its chunk's partials are published.
      const long long at = (long long)(SMALL ? rc0.state : s_state[b]) * p.cache_rs + (long long)i * p.cache_ss + v0;
      if (cache_f32) {
        uint64_t* crow = reinterpret_cast<uint64_t*>(reinterpret_cast<float*>(p.cache) + at);
#pragma unroll
        for (int e2 = 0; e2 < IPL / 2; ++e2)
          st_agent(crow + e2, ((uint64_t)__float_as_uint(z[2 * e2 + 1]) << 32) | __float_as_uint(z[2 * e2]));
      } else {
        uint64_t* crow = reinterpret_cast<uint64_t*>(reinterpret_cast<uint16_t*>(p.cache) + at);
#pragma unroll
        for (int e2 = 0; e2 < IPL / 4; ++e2) st_agent(crow + e2, ((uint64_t)cw[2 * e2 + 1] << 32) | cw[2 * e2]);
      }
    } else if (ok) {
      // Streaming stores: the cache is not read again by this launch.
      const long long at = (long long)(SMALL ? rc0.state : s_state[b]) * p.cache_rs + (long long)i * p.cache_ss + v0;
      if (cache_f32) {
        u32x4_t* crow = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(p.cache) + at);
#pragma unroll
        for (int e4 = 0; e4 < IPL / 4; ++e4)
          __builtin_nontemporal_store((u32x4_t){__float_as_uint(z[4 * e4]), __float_as_uint(z[4 * e4 + 1]),
                                                __float_as_uint(z[4 * e4 + 2]), __float_as_uint(z[4 * e4 + 3])},
                                      crow + e4);
      } else {
        uint16_t* crow = reinterpret_cast<uint16_t*>(p.cache) + at;
        if constexpr (IPL == 8) __builtin_nontemporal_store((u32x4_t){cw[0], cw[1], cw[2], cw[3]}, reinterpret_cast<u32x4_t*>(crow));
        else __builtin_nontemporal_store((u32x2_t){cw[0], cw[1]}, reinterpret_cast<u32x2_t*>(crow));
      }
    }
    // Scores: T <= 0 is argmax; c / 1 is exact.
    if (T > 0.0f && T != 1.0f) {
#pragma unroll
      for (int e = 0; e < IPL; ++e) z[e] = div_by_recip(z[e], rT);
    }
    if (MODE == 0 && T > 0.0f) {
      if (!SMALL && nz_inline && ok && !nz_ready) {
        const uint64_t pre = noise_prefix(s_seed[b], p.row_base + b, i);
#pragma unroll
        for (int e = 0; e < IPL; e += 2) {
          float g2[2];
          gumbel_noise<2>(pre, v0 + e, s_log, g2);
          z[e] = __fadd_rn(z[e], g2[0]);
          z[e + 1] = __fadd_rn(z[e + 1], g2[1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < IPL; ++e) z[e] = __fadd_rn(z[e], in.nz[e]);
      }
    }
    // This lane's best: the first NaN, else the first maximum (order keys
    // of z + 0, which makes -0 equal to +0).
    int kbest = INT_MIN;
    uint32_t ebest = 0, enan = IPL;
#pragma unroll
    for (int e = 0; e < IPL; ++e) {
      const bool isn = isnan(z[e]);
      enan = (isn && enan == IPL) ? e : enan;
      const int k = isn ? INT_MIN : order_key(__fadd_rn(z[e], 0.0f));
      ebest = k > kbest ? e : ebest;
      kbest = k > kbest ? k : kbest;
    }
    if (!ok) kbest = INT_MIN, enan = IPL;
    // The row's best over its kLanesPerRow lanes.
    const int gmax = group8_imax(kbest);
    const uint32_t gid = group8_umin(kbest != INT_MIN && kbest == gmax ? (uint32_t)v0 + ebest : 0xFFFFFFFFu);
    const uint32_t gnan = group8_umin(enan < IPL ? (uint32_t)v0 + enan : 0xFFFFFFFFu);
    float wsum = 0.0f;
    if (MODE == 1) {
      // The same exponential as the leader's scan of the chosen chunk, so
      // that its chunk weights and its in-chunk CDF are
      // built from the same function (a cruder one here than there would
      // shift draws near a chunk's upper edge onto its last id).  Both use
      // the hardware exp2 form: the library expf on every element cost
      // 252.5 vs 234.0 us per call at 64 rows.
      const float m = order_key_inv(gmax);
      float s = 0.0f;
      if (ok && gmax != INT_MIN && isfinite(m)) {
#pragma unroll
        for (int e = 0; e < IPL; ++e) s += isnan(z[e]) ? 0.0f : __expf(z[e] - m);
      }
      wsum = group8_sum(s);
    }
    if (q == 0 && rr < nb && (SMALL ? rc0.active : s_active[b] != 0)) {
      const uint64_t key = gnan != 0xFFFFFFFFu ? ((0xFFFFFFFFull << 32) | (0xFFFFFFFFu - gnan))
                           : gmax != INT_MIN ? (((uint64_t)score_ord(order_key_inv(gmax)) << 32) | (0xFFFFFFFFu - gid))
                                             : kNoCandidate;
      if (MODE == 0) {
        if (key > s_key[wave][b]) s_key[wave][b] = key;
      } else {
        s_key[wave][b] = key;
        s_wsum[wave][b] = wsum;
      }
    }
  };

  float* sb = s_bias[wave];
  // Streamed head: the first nres tiles of each wave's group in chunk 1 are
  // written to LDS at step 0 and read from there at later steps, so those
  // bytes are streamed from memory once per launch instead of every step.
  constexpr int NP = kParked<R>;
  uint4* const s_hres = s_e + rows * ES + wave * NP * 64;
  auto park_tiles = [&](int i, int j) {
    if constexpr (!RES) {
      if (i == 0 && j == 1 && p.nres > 0) {
#pragma unroll
        for (int s2 = 0; s2 < NP; ++s2) s_hres[s2 * 64 + lane] = h[s2];
      }
    }
  };
  // Local work of step i: bias, epilogue, keys for every chunk of this
  // workgroup (mode 1 also publishes each chunk's partials).
  // Streamed head: a workgroup's chunks are visited in alternating order
  // (odd steps backwards), so every step after the first starts with the
  // chunk the previous step ended with, whose head tiles are still in h:
  // with k chunks per workgroup a step streams k - 1 of them.
  const int nch = RES ? 1 : (NC - wc + G - 1) / G;  // this workgroup's chunks
  auto local_work = [&](int i) {
    if (lane == 0)
      for (int b = 0; b < rows; ++b) s_key[wave][b] = kNoCandidate;
    for (int jj = 0; jj < nch; ++jj) {
      const int j = (!RES && (i & 1)) ? nch - 1 - jj : jj;
      const int c = wc + j * G;
      const int g = c * kWaves + wave;
      LaneIn cur, nxt;
      if constexpr (!RES) {
        // Stream this group's head (all 32 tiles in flight at once), with
        // the first batch's inputs, unless the tiles are still here from
        // the previous step.  (Issuing the next chunk's tiles during this
        // chunk's epilogue instead was slower: the epilogue's noise draw
        // then runs with h live.)
        if (jj > 0 || i == 0) {
          if (i > 0 && j == 1 && p.nres > 0) {
#pragma unroll
            for (int s2 = NP; s2 < kSlots; ++s2)
              h[s2] = g < NG ? load_head_tile<R>(p.head, g, s2, lane, V) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int s2 = 0; s2 < NP; ++s2) h[s2] = s_hres[s2 * 64 + lane];
          } else {
#pragma unroll
            for (int s2 = 0; s2 < kSlots; ++s2)
              h[s2] = g < NG ? load_head_tile<R>(p.head, g, s2, lane, V) : make_uint4(0, 0, 0, 0);
          }
        }
      }
      if constexpr (ONE) {
        // Lane lr's vocab id v: bias, cache value and score ordinal in
        // registers; one wave maximum and a ballot give the lowest id of the
        // maximum (or of the NaNs, which order first).
        const int v = g * RPG + lr;
        const bool own = g < NG && v < V && lane_owns;
        // The row's constants and the noise wave 1 drew for wave 0 (both
        // written before the barrier that ended the previous step) are read
        // before the bias, so that their LDS round trips overlap the
        // embedding reads instead of following one another in the epilogue.
        const bool act = s_active[0] != 0;
        const float T = s_T[0];
        const auto rT = s_rT[0];
        const int st = s_state[0];
        if (w0_by_w1 && wave == 0 && i > 0) one_noise = s_nz0[lane];
        const float bsum = one_row_bias<R>(h, s_e, lane);
        park_tiles(i, j);
        uint32_t ord = 0;
        if (act && own) {
          float x = __fadd_rn(__uint_as_float(one_base), bf16_round(bsum));
          x = __fmul_rn(x, p.mult);
          if (p.has_cap) x = __fmul_rn(tanhf(__fmul_rn(x, p.inv_cap)), p.cap);
          const long long at = (long long)st * p.cache_rs + (long long)i * p.cache_ss + v;
          float z;
          if (cache_f32) {
            reinterpret_cast<float*>(p.cache)[at] = x;
            z = x;
          } else {
            const uint32_t cb = f32_to_bf16_hw(x);
            reinterpret_cast<uint16_t*>(p.cache)[at] = (uint16_t)cb;
            z = bf16_to_f32(cb);
          }
          if (T > 0.0f) {
            if (T != 1.0f) z = div_by_recip(z, rT);  // c / 1 is exact
            z = __fadd_rn(z, one_noise);
          }
          ord = score_ord(z);
        }
        const uint32_t m = row_fold_umax(ord);
        const uint64_t hit = __ballot(m != 0 && ord == m);
        if (lane == 0)
          s_key[wave][0] = hit ? (((uint64_t)m << 32) | (0xFFFFFFFFu - (uint32_t)(g * RPG + __builtin_ctzll(hit))))
                               : kNoCandidate;
        continue;
      }
      // Batches of kBatch rows; a pass of kRowPass rows shares one MFMA
      // bias tile.  Without a prefetch, the next batch's inputs are loaded
      // before the current batch's epilogue.
      static_assert(kRowPass == 2 * kBatch, "a pass is two batches");
      const int nbat = (rows + kBatch - 1) / kBatch;
      // (staged base logits hold bf16 only; fp32 ones are loaded per batch)
      const bool staged = stage && !base_f32;
      if (!ahead && !staged) load_rows(i, 0, g, cur);
      // Streamed head, inline noise: the first batch's noise is drawn here,
      // while the group's head tiles are still arriving, not in the epilogue.
      bool nz0 = false;
      if constexpr (!RES && MODE == 0) {
        if (nz_inline) {
          const int b = rr, v0 = g * RPG + q * IPL;
          if (b < rows && g < NG && v0 < V && s_active[b] && s_T[b] > 0.0f) {
            const uint64_t pk = noise_prefix(s_seed[b], p.row_base + b, i);
#pragma unroll
            for (int e = 0; e < IPL; e += 4) gumbel_noise<4>(pk, v0 + e, s_log, cur.nz + e);
          }
          nz0 = true;
        }
      }
      for (int t = 0; t < nbat; ++t) {
        const int b0 = t * kBatch;
        const RowConsts rc = SMALL ? row_consts(b0 + rr) : RowConsts{};
        if ((t & 1) == 0) {
          const int np = rows - b0 < kRowPass ? rows - b0 : kRowPass;
          // (8 rows: 52.0 -> 49.8 us per call with the noise read, 60.3 ->
          // 59.3 us with inline noise; 64-row inverse CDF 226.5 -> 224.1 us)
          group_bias<R, (MODE == 0 && RES && SMALL) ? 8 : 2>(h, s_e, b0, np, lane, sb);
          if (t == 0) park_tiles(i, j);
        }
        const int nb = rows - b0 < kBatch ? rows - b0 : kBatch;
        if constexpr (ahead) {
          epilogue_rows(i, b0, nb, g, sb + (t & 1) * kBatch * BS, pre, false, rc);
        } else if (staged) {
          stage_fetch(t, cur);
          epilogue_rows(i, b0, nb, g, sb + (t & 1) * kBatch * BS, cur, false, rc);
        } else {
          if (t + 1 < nbat) load_rows(i, b0 + kBatch, g, nxt);
          epilogue_rows(i, b0, nb, g, sb + (t & 1) * kBatch * BS, cur, t == 0 && nz0, rc);
          cur = nxt;
        }
      }
      if (MODE == 1) {
        // Combine the chunk's 8 wave partials (fixed order) and publish them,
        // once every wave's cache stores of the chunk are complete (the
        // row's leader reads them when it sees the partials).
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
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
  };

  // Publication of the workgroup's best key per row (mode 0): row b by
  // thread b.
  auto row_key = [&](int b) {
    uint64_t K = kNoCandidate;
    for (int w = 0; w < kWaves; ++w) K = umax64(K, s_key[w][b]);
    return K;
  };
  auto publish = [&](int i) {
    for (int b = tid; b < rows; b += kThreads)
      if (s_active[b]) st_agent(L.keys + ((size_t)i * rows + b) * NC + wg, row_key(b));
  };
  auto slot_wait_abort = [&]() {
    if (lane == 0) {
      s_abort = 1;
      __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto write_tokens = [&](int i) {
    if (wg == 0)
      for (int b = tid; b < rows; b += kThreads)
        if (s_active[b]) p.tokens[(long long)b * p.tok_rs + i] = s_tok[b];
  };

  // Inverse CDF: the token of row b at step i, given the chosen chunk o and
  // the threshold tl in that chunk's scale: the first id whose inclusive
  // running weight exceeds tl, in vocabulary order (else the last id with
  // weight).  The chunk's cache values are read at agent scope: another
  // workgroup stored them in this step.  One wave.
  auto scan_chunk = [&](int i, int b, int o, float tl) -> int {
    const float T = s_T[b];
    const double rT = s_rT[b];
    constexpr int PER = CHUNK / 64;  // ids per lane
    static_assert(PER == 8 || PER == 4, "chunk slice");
    if ((unsigned)o >= (unsigned)NC) o = NC - 1;
    const int v0 = o * CHUNK + lane * PER;
    const long long at = (long long)s_state[b] * p.cache_rs + (long long)i * p.cache_ss + v0;
    // PER cache values per lane; V is a multiple of 16, so a lane's ids are
    // all valid or all not.
    uint32_t cw[PER];  // fp32 bits of the cache values
#pragma unroll
    for (int k = 0; k < PER; ++k) cw[k] = 0;
    if (v0 < V) {
      if (cache_f32) {
        const uint64_t* crow = reinterpret_cast<const uint64_t*>(reinterpret_cast<const float*>(p.cache) + at);
#pragma unroll
        for (int k2 = 0; k2 < PER / 2; ++k2) {
          const uint64_t t2 = ld_agent(crow + k2);
          cw[2 * k2] = (uint32_t)t2, cw[2 * k2 + 1] = (uint32_t)(t2 >> 32);
        }
      } else {
        const uint64_t* crow = reinterpret_cast<const uint64_t*>(reinterpret_cast<const uint16_t*>(p.cache) + at);
#pragma unroll
        for (int k4 = 0; k4 < PER / 4; ++k4) {
          const uint64_t t4 = ld_agent(crow + k4);
          const uint32_t lo = (uint32_t)t4, hi = (uint32_t)(t4 >> 32);
          cw[4 * k4] = lo << 16, cw[4 * k4 + 1] = lo & 0xFFFF0000u;
          cw[4 * k4 + 2] = hi << 16, cw[4 * k4 + 3] = hi & 0xFFFF0000u;
        }
      }
    }
    float z[PER];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const float c = __uint_as_float(cw[k]);
      z[k] = v0 < V ? (T != 1.0f ? div_by_recip(c, rT) : c) : -INFINITY;
      m = fmaxf(m, z[k]);
    }
    m = order_key_inv(wave_imax(order_key(m)));  // chunk maximum (no NaN: the decision excludes it)
    float w[PER];
    float lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      w[k] = (v0 + k < V && z[k] > -INFINITY) ? __expf(z[k] - m) : 0.0f;  // as the partial sums
      lsum += w[k];
    }
    float run = wave_incl_scan(lsum) - lsum;
    int found = -1, lastv = -1;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (found < 0 && w[k] > 0.0f && run + w[k] > tl) found = v0 + k;
      if (w[k] > 0.0f) lastv = v0 + k;
      run += w[k];
    }
    const uint64_t hit = __ballot(found >= 0);
    if (hit) return __shfl(found, __builtin_ctzll(hit));
    const uint64_t any = __ballot(lastv >= 0);
    return any ? __shfl(lastv, 63 - __builtin_clzll(any)) : o * CHUNK;
  };

  {
    // The step loop: local work, publication, then the exchange of the
    // step (its tail overlaps the fetch of the next embedding).
    // Inverse CDF: a workgroup that leads a row (H2 below) stages its next
    // base logits after its decisions, in every wave: the leader's polls
    // would otherwise queue behind its own wave's staging loads (loads
    // complete in order) and behind the other waves' in the CU's memory
    // pipeline (64 rows: 233.0 -> 225.3 us per call against deferring the
    // leader wave alone).
    bool leads = false;
    if constexpr (MODE == 1)
      for (int b = wg; b < rows; b += G) leads = leads || s_active[b];
    TRACE_STAMP(wg, 0, 7);
    for (int i = 0; i < N; ++i) {
      TRACE_STAMP(wg, i, 0);
      local_work(i);
      TRACE_STAMP(wg, i, 1);
      if (MODE == 1 && ahead && i + 1 < N) prefetch(i + 1);
      if (stage && !base_f32 && i + 1 < N && !leads) {
        // Parked at once: the wait for the loads overlaps the wait for the
        // other workgroups' partials.
        stage_load(i + 1);
        stage_park();
      }
      if (MODE == 0) {
        __syncthreads();
        publish(i);
        TRACE_STAMP(wg, i, 2);
        if (ahead && i + 1 < N) prefetch(i + 1);
      }
      // The last step, mode 0, at most kWaves rows: only workgroup 0 needs
      // the winners (it writes the tokens); it polls every slot itself and
      // the others are done.
      const bool last0 = MODE == 0 && i + 1 == N && (SMALL || rows <= kWaves);
      if (last0 && wg != 0) break;

      // ---- grid-wide exchange.
      if (MODE == 0) {
        // Every workgroup reads every workgroup's key; wave w serves rows w,
        // w+8, ...  While it polls, the wave fetches the embedding row of the
        // best key seen so far: that key is almost always the final winner
        // (unless the workgroup holding the winner is the last to publish), so
        // the next step's embedding is usually in flight before the exchange
        // ends.  The row goes straight into the LDS embedding buffer, which no
        // wave reads again in this step.
        // More than kWaves rows with more than 64 workgroups: a two-level
        // exchange whose waits cover all of a wave's rows at once (wave w
        // serves rows w + 8 j).  Reducer r (workgroup r < NR): lane l polls
        // slot 64 r + l of each of the wave's rows until every one has
        // arrived, then publishes each row's maximum.  Every workgroup: lane
        // j NRP + r polls reducer r's partial of the wave's row j, then takes
        // the maximum over its NRP lanes.  (Polling the rows one after
        // another cost a round trip per row.)
        const int NRm = reducers_for(G);
        const int NRSm = reducers_for(NC);
        const bool many = !SMALL && rows > kWaves && NRm > 1;
        if constexpr (!SMALL) if (many) {
          const int nrw = rows > wave ? (rows - wave + kWaves - 1) / kWaves : 0;  // <= 8
          constexpr int kMaxRW = kLaunchRows / kWaves;
          if (wg < NRm) {
            const int idx = wg * 64 + lane;
            uint64_t x[kMaxRW];
#pragma unroll
            for (int j = 0; j < kMaxRW; ++j) {
              const int b = wave + kWaves * j;
              x[j] = (j < nrw && s_active[b] && idx < G) ? 0 : kNoCandidate;
            }
            for (;;) {
              bool all = true;
#pragma unroll
              for (int j = 0; j < kMaxRW; ++j) {
                if (x[j] == 0) x[j] = ld_agent(L.keys + ((size_t)i * rows + wave + kWaves * j) * NC + idx);
                all = all && x[j] != 0;
              }
              if (__all(all)) break;
              if (now_ticks() > deadline) {
                slot_wait_abort();
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int j = 0; j < kMaxRW; ++j) {
              const int b = wave + kWaves * j;
              if (j < nrw && s_active[b]) {
                const uint64_t K = wave_max_u64(x[j] == 0 ? kNoCandidate : x[j]);
                if (lane == 0) st_agent(L.part + ((size_t)i * rows + b) * NRSm + wg, K);
              }
            }
          }
          // Followers: NRP lanes per row (NRP a power of two >= NR).
          int NRP = 1;
          while (NRP < NRm) NRP <<= 1;
          const int per_pass = 64 / NRP;
          for (int j0 = 0; j0 < nrw; j0 += per_pass) {
            const int j = j0 + lane / NRP, r = lane % NRP;
            const int b = wave + kWaves * j;
            const bool mine = j < nrw && r < NRm && s_active[b];
            uint64_t x = mine ? 0 : kNoCandidate;
            for (;;) {
              if (x == 0) x = ld_agent(L.part + ((size_t)i * rows + b) * NRSm + r);
              if (__all(x != 0)) break;
              if (now_ticks() > deadline) {
                slot_wait_abort();
                if (x == 0) x = kNoCandidate;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
            // maximum over the row's NRP lanes
            for (int d = 1; d < NRP; d <<= 1) x = umax64(x, (uint64_t)__shfl_xor((long long)x, d));
            uint32_t win = key_id(x);
            if (win >= (uint32_t)V) win = 0;  // only after a timeout
            // Each row's winner and, for the next step, its embedding: the
            // loads of all the pass's rows are issued before any is stored.
            const bool lead = r == 0 && j < nrw && s_active[b];
            if (lead) s_tok[b] = (int)win;
            if (i + 1 < N) {
              constexpr int kHalf = kMaxRW / 2;
#pragma unroll
              for (int k0 = 0; k0 < kMaxRW; k0 += kHalf) {
                uint4 ev[kHalf];
#pragma unroll
                for (int k = 0; k < kHalf; ++k) {
                  const int jk = j0 + k0 + k;
                  const int bk = wave + kWaves * jk;
                  const uint32_t wk = (uint32_t)__shfl((int)win, (k0 + k) * NRP);
                  ev[k] = make_uint4(0, 0, 0, 0);
                  if (k0 + k < per_pass && jk < nrw && s_active[bk] && lane < KSEG)
                    ev[k] = *reinterpret_cast<const uint4*>(p.embed + (size_t)wk * R + lane * 8);
                }
#pragma unroll
                for (int k = 0; k < kHalf; ++k) {
                  const int jk = j0 + k0 + k;
                  const int bk = wave + kWaves * jk;
                  if (k0 + k < per_pass && jk < nrw && s_active[bk] && lane < KSEG) s_e[bk * ES + lane] = ev[k];
                }
              }
            }
          }
        }
        // One row, or at most kWaves rows on a streamed head, with more than
        // 64 workgroups exchange in two levels: wave b of reducer r
        // (workgroup r < NR) waits for row b's slots 64 r .. 64 r + 63 and
        // publishes their maximum into every copy of the row's partials;
        // wave b of every workgroup then polls the NR partials of its own
        // copy instead of all G slots, which keeps the polled lines few and
        // each polled by G / kPartCopies workgroups.  (Measured per call: one
        // row 41.5 -> 40.0 us, r = 512 streamed with 8 rows 756 -> 741 us;
        // resident 8 rows 54.0 -> 57.6 us, so the resident kernels of 2 to 8
        // rows keep the all-to-all and do not compile this path.)
        const int NR = !last0 && (RES ? ONE : rows <= kWaves) ? reducers_for(G) : 1;
        if (!many && NR > 1 && wg < NR) {
          for (int b = wave; b < rows; b += kWaves) {
            if (!s_active[b]) continue;
            const uint64_t* slots = L.keys + ((size_t)i * rows + b) * NC;
            const int idx = wg * 64 + lane;
            uint64_t x = idx < G ? 0 : kNoCandidate;
            for (;;) {
              if (x == 0) x = ld_agent(slots + idx);
              if (__all(x != 0)) break;
              if (now_ticks() > deadline) {
                slot_wait_abort();
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
            const uint64_t K = wave_max_u64(x == 0 ? kNoCandidate : x);
            if (lane < kPartCopies)
              st_agent(L.part + (((size_t)i * rows + b) * kPartCopies + lane) * kPartStride + wg, K);
          }
        }
        TRACE_STAMP(wg, i, 3);
        for (int b = many ? rows : wave; b < rows; b += kWaves) {
          if (!s_active[b]) continue;
          const uint64_t* slots = NR > 1 ? L.part + (((size_t)i * rows + b) * kPartCopies + wg % kPartCopies) * kPartStride
                                         : L.keys + ((size_t)i * rows + b) * NC;
          const int n = NR > 1 ? NR : G;  // words polled: partials or slots
          const bool next = i + 1 < N;
          uint64_t best = kNoCandidate;
          uint32_t spec = 0xFFFFFFFFu;
          uint4 ev = make_uint4(0, 0, 0, 0);
          for (;;) {
            bool all = true;
            uint64_t mine = kNoCandidate;
            uint64_t xs[4];  // the first 256 words: 4 per lane
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int idx = lane + 64 * k;
              xs[k] = idx < n ? ld_agent(slots + idx) : kNoCandidate;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              all = all && (xs[k] != 0);
              mine = umax64(mine, xs[k]);
            }
            for (int k0 = 256; k0 < n; k0 += 256) {  // 4 more words per lane per batch
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const int idx = k0 + lane + 64 * k;
                if (idx < n) {
                  const uint64_t x = ld_agent(slots + idx);
                  all = all && (x != 0);
                  mine = umax64(mine, x);
                }
              }
            }
            best = wave_max_u64(mine);
            if (__all(all)) break;
            const uint32_t cand = key_id(best);
            if (next && best != kNoCandidate && cand != spec && cand < (uint32_t)V) {
              spec = cand;
              if (lane < KSEG) ev = *reinterpret_cast<const uint4*>(p.embed + (size_t)cand * R + lane * 8);
            }
            if (now_ticks() > deadline) {
              slot_wait_abort();
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          uint32_t win = key_id(best);
          if (win >= (uint32_t)V) win = 0;  // only after a timeout
          TRACE_STAMP(wg, i, 4);
          if (next) {
            if (win != spec && lane < KSEG) ev = *reinterpret_cast<const uint4*>(p.embed + (size_t)win * R + lane * 8);
            if (lane < KSEG) s_e[b * ES + lane] = ev;
          }
          if (lane == 0) s_tok[b] = (int)win;
        }
      } else {
        // H2: the leader workgroup of each row (b % G) finds the chunk that
        // holds u * S and publishes it with the threshold in that chunk's
        // own scale, or the token itself for an argmax row.  Each lane owns
        // KPL contiguous chunks.  With at most kLeaderRegs chunks per lane the
        // polled slots stay in registers (a slot once written is final, so
        // only missing ones are reloaded); otherwise they are read again.
        const int KPL = (NC + 63) / 64;
        for (int b = wg; b < rows; b += G) {
          if (((b / G) % kWaves) != wave || !s_active[b]) continue;
          const uint64_t* kslots = L.keys + ((size_t)i * rows + b) * NC;
          const uint32_t* sslots = L.sums + ((size_t)i * rows + b) * NC;
          const bool regs = KPL <= kLeaderRegs;
          uint64_t kc[kLeaderRegs];
          uint32_t sc[kLeaderRegs];
#pragma unroll
          for (int k = 0; k < kLeaderRegs; ++k) kc[k] = 0, sc[k] = 0;
          // The row's uniform depends on no partial: drawn before the wait.
          const float u = hash_uniform(noise_prefix(s_seed[b], p.row_base + b, i));
          // Slot k of this lane: (key, sum bits), 0 where the chunk does not exist.
          auto slot = [&](int k, uint64_t& key, uint32_t& sum) {
            const int c = lane * KPL + k;
            key = 0, sum = 0;
            if (c < NC) {
              if (regs) {
#pragma unroll
                for (int r2 = 0; r2 < kLeaderRegs; ++r2)
                  if (r2 == k) key = kc[r2], sum = sc[r2];
              } else {
                key = ld_agent(kslots + c);
                sum = ld_agent32(sslots + c);
              }
            }
          };
          for (;;) {
            bool all = true;
            if (regs) {
#pragma unroll
              for (int k = 0; k < kLeaderRegs; ++k) {
                const int c = lane * KPL + k;
                if (k < KPL && c < NC) {
                  if (kc[k] == 0) kc[k] = ld_agent(kslots + c);
                  if (sc[k] == 0) sc[k] = ld_agent32(sslots + c);
                  all = all && kc[k] != 0 && sc[k] != 0;
                }
              }
            } else {
              for (int k = 0; k < KPL; ++k) {
                const int c = lane * KPL + k;
                if (c < NC) all = all && ld_agent(kslots + c) != 0 && ld_agent32(sslots + c) != 0;
              }
            }
            if (__all(all)) break;
            if (now_ticks() > deadline) {
              slot_wait_abort();
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          TRACE_STAMP_MAX(wg, i, 10);
          uint64_t K = kNoCandidate;
          for (int k = 0; k < KPL; ++k) {
            uint64_t key;
            uint32_t sum;
            slot(k, key, sum);
            if (lane * KPL + k < NC) K = umax64(K, key);
          }
          K = wave_max_u64(K);
          const float M = ord_score((uint32_t)(K >> 32));
          uint64_t dec;
          if (!(s_T[b] > 0.0f) || !isfinite(M)) {
            dec = (1ull << 63) | key_id(K);
          } else {
            // Weight of chunk c: its sum of exp(z - m_c) rescaled by
            // exp(m_c - M); the lanes' totals are scanned in chunk order.
            auto weight = [&](int k, float& e) -> float {
              uint64_t key;
              uint32_t sum;
              slot(k, key, sum);
              e = 0.0f;
              if (lane * KPL + k >= NC) return 0.0f;
              const float mc = ord_score((uint32_t)(key >> 32));
              if (key == kNoCandidate || !isfinite(mc)) return 0.0f;
              e = expf(mc - M);
              return __uint_as_float(sum & 0x7FFFFFFFu) * e;
            };
            // (With the slots in registers the weights are kept for the
            // search below instead of being computed twice.)
            float wk[kLeaderRegs], ek[kLeaderRegs];
            float lsum = 0.0f;
            if (regs) {
#pragma unroll
              for (int k = 0; k < kLeaderRegs; ++k) {
                ek[k] = 0.0f;
                wk[k] = k < KPL ? weight(k, ek[k]) : 0.0f;
                if (k < KPL) lsum += wk[k];
              }
            } else {
              for (int k = 0; k < KPL; ++k) {
                float e;
                lsum += weight(k, e);
              }
            }
            const float incl = wave_incl_scan(lsum);
            const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
            const float t = u * total;
            // First chunk with weight whose inclusive prefix exceeds t (else
            // the last chunk with weight, when rounding left none above t).
            // The weight test matters: a lane past the last chunk, or a
            // chunk of -inf logits, starts at a running sum that rounding
            // may put above t, and must never be chosen.
            int found = -1, last_pos = -1;
            float before = 0.0f, wfound = 0.0f, last_before = 0.0f, last_w = 0.0f;
            float run = incl - lsum;
            for (int k = 0; k < KPL; ++k) {
              float e, w;
              if (regs) {
#pragma unroll
                for (int r2 = 0; r2 < kLeaderRegs; ++r2)
                  if (r2 == k) w = wk[r2], e = ek[r2];
              } else {
                w = weight(k, e);
              }
              const int c = lane * KPL + k;
              if (found < 0 && w > 0.0f && run + w > t) {
                found = c;
                before = run;
                wfound = e;
              }
              if (w > 0.0f) {
                last_pos = c;
                last_before = run;
                last_w = e;
              }
              run += w;
            }
            const uint64_t hit = __ballot(found >= 0);
            int o;
            float tl;
            if (hit) {
              const int src = __builtin_ctzll(hit);
              o = __shfl(found, src);
              tl = (t - __shfl(before, src)) / __shfl(wfound, src);
            } else {
              const uint64_t any = __ballot(last_pos >= 0);
              const int src = 63 - __builtin_clzll(any);
              o = __shfl(last_pos, src);
              tl = (t - __shfl(last_before, src)) / __shfl(last_w, src);
            }
            if (!(tl >= 0.0f)) tl = 0.0f;
            // (Every chosen chunk has weight, hence exists; the clamp only
            // keeps the chunk's reads inside the vocabulary should that fail.)
            if ((unsigned)o >= (unsigned)NC) o = NC - 1;
            dec = ((uint64_t)(uint32_t)(o + 1) << 32) | __float_as_uint(tl);
          }
          TRACE_STAMP_MAX(wg, i, 11);
          // The leader scans the chosen chunk itself: its values were stored
          // at agent scope and completed before the chunk's partials, which
          // the leader has seen.
          int tok;
          if (dec >> 63) {
            const uint32_t tk = (uint32_t)dec;
            tok = tk < (uint32_t)V ? (int)tk : 0;
          } else {
            tok = scan_chunk(i, b, (int)(dec >> 32) - 1, __uint_as_float((uint32_t)dec));
          }
          // Every copy gets it: each copy's lines are polled by G / kDecCopies
          // workgroups instead of all G (64 rows: 258 -> 241 us per call when
          // the decisions and tokens were first copied so).
          if (lane == 0) s_tok[b] = tok;
          if (lane < kDecCopies) st_agent(L.tok + ((size_t)i * kDecCopies + lane) * rows + b, (1ull << 63) | (uint32_t)tok);
          TRACE_STAMP_MAX(wg, i, 9);
        }
        TRACE_STAMP(wg, i, 3);
        if (stage && !base_f32 && i + 1 < N && leads) {
          __syncthreads();  // after this workgroup's decisions
          stage_load(i + 1);
          stage_park();
        }
        TRACE_STAMP(wg, i, 8);
        // H4: the tokens of the rows this workgroup does not lead, polled all
        // at once.
        {
          const int b = wave + kWaves * lane;
          const bool mine = lane < kLaunchRows / kWaves && b < rows && s_active[b] && b % G != wg;
          uint64_t d = 0;
          for (;;) {
            if (mine && d == 0) d = ld_agent(L.tok + ((size_t)i * kDecCopies + wg % kDecCopies) * rows + b);
            if (__all(!mine || d != 0)) break;
            if (now_ticks() > deadline) {
              slot_wait_abort();
              if (d == 0) d = 1ull << 63;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          if (mine) s_tok[b] = (uint32_t)d < (uint32_t)V ? (int)(uint32_t)d : 0;
        }
        TRACE_STAMP(wg, i, 4);
      }
      __syncthreads();
      TRACE_STAMP(wg, i, 5);
      if (s_abort) break;

      // ---- the winners: tokens out, next embeddings in.
      write_tokens(i);
      if (MODE == 1 && i + 1 < N) {
        // The next embeddings: every load of a batch is issued before any is
        // stored (one round trip per batch, not per row).
        constexpr int kEmbPer = kLaunchRows * (R / 8) / kThreads;  // 16-byte pieces per thread: 4 or 8
        constexpr int kEmbBatch = 2;
#pragma unroll 1
        for (int j0 = 0; j0 < kEmbPer; j0 += kEmbBatch) {
          uint4 ev[kEmbBatch];
#pragma unroll
          for (int j = 0; j < kEmbBatch; ++j) {
            const int k = tid + (j0 + j) * kThreads;
            const int b = k / KSEG, seg = k - b * KSEG;
            ev[j] = make_uint4(0, 0, 0, 0);
            if (k < rows * KSEG && s_active[b]) {
              // A winner is always a valid id; the clamp only keeps the
              // gather in bounds should that ever fail.
              const uint32_t t = (uint32_t)s_tok[b] < (uint32_t)V ? (uint32_t)s_tok[b] : 0u;
              ev[j] = *reinterpret_cast<const uint4*>(p.embed + (size_t)t * R + seg * 8);
            }
          }
#pragma unroll
          for (int j = 0; j < kEmbBatch; ++j) {
            const int k = tid + (j0 + j) * kThreads;
            const int b = k / KSEG, seg = k - b * KSEG;
            if (k < rows * KSEG && s_active[b]) s_e[b * ES + seg] = ev[j];
          }
        }
        __syncthreads();
      }
    }
  }
  // Every workgroup has read the parity by now (all published the last step).
  if (wg == 0 && tid == 0 && !s_abort) st_agent32(header, parity ^ 1u);
}

// ============================================================= step kernel ==
// Batches beyond one persistent launch (more than kLaunchRows rows): per
// draft position one step-kernel launch (mode 0), or a step kernel and a
// pick kernel (mode 1), as the pages' fused loop for large batches
// (fused_markov page, FusedMarkovSampler: the bias GEMM plus two kernels a
// step, drawing by inverse CDF; muse_spark markov page, MarkovSampler: the
// blocks of a row count their arrivals and the last one picks the winner).
// Here the bias GEMM is fused into the step kernel (the bias never goes to
// memory):
//  * workgroup c owns chunk c (8 groups of 16384 / r vocab ids, one per
//    wave); each wave loads its group's head into VGPRs once per step and
//    reuses it for every request row (v_mfma_f32_16x16x32_bf16 passes of 16
//    rows, embeddings from LDS);
//  * the epilogue (bias -> bf16, + base, transform, cache store, score)
//    runs in batches of 8 rows with 16-byte vectors, the next two batches'
//    base logits and noise in flight;
//  * mode 0: each workgroup folds its best key of every row into the row's
//    slot with an agent-scope atomic max (fire and forget), then counts
//    itself on the step's arrival counter; the workgroup that arrives last
//    writes the step's tokens, also into the workspace, from where every
//    workgroup of the next launch loads its rows' winner embeddings itself
//    (a gather of all rows by the last workgroup cost ~5.5 us per step at
//    256 rows);
//  * mode 1: each workgroup writes its chunk's partials of every row (the
//    best key and the sum of exp(z - chunk max), as the persistent kernel's
//    chunks publish them); the pick kernel that follows (one wave per row)
//    combines them in chunk order, draws the row's uniform, finds the chunk
//    holding u * S and scans that chunk's cache values in vocabulary order,
//    with the persistent kernel's arithmetic (so both paths draw the same
//    tokens), and writes the token.
// No workgroup ever waits for another, so the launches need no
// co-residency.
//
// Workspace half layout of this path (the parity protocol of the persistent
// kernel: a call uses half P and its step-0 launch clears the other half
// for the next call; the last launch flips P):
//   arrive[2] u32 (256 bytes)          arrival counters, by step parity
//   mode 0: best[2][rows][kBestStride] u64   each row's best key, by step
//                                      parity (one 128-byte line per row)
//   mode 1: keys[rows][NC] u64, sums[rows][NC] u32   the chunks' partials
//                                      (written, then read by the pick
//                                      kernel that follows)
//   tok[rows] i32                      the last step's tokens (-1: inert row)
// Mode 0: the last workgroup of step i zeroes arrive[i & 1] and best[i & 1]
// after reading them, so step i + 2 finds them zero.  Mode 1: the last
// wave of the last pick launch to arrive zeroes arrive[0] and flips P.

constexpr int kBestStride = 16;  // u64 words per row's best key (a 128-byte line)
constexpr int kPrefetch = 2;     // epilogue batches whose inputs are in flight (mode 0)

__host__ __device__ inline size_t step_slots_bytes(int rows, int mode, int NC) {
  return mode == 0 ? (size_t)2 * rows * kBestStride * 8 : (size_t)rows * NC * 12;
}
// The persistent mode-0 variant: an arrival counter per position u32,
// best[N][rows][kBestStride] u64, then the tokens as tagged words
// tags[rows] u64.
__host__ __device__ inline size_t pers_arrive_bytes(int N) { return ((size_t)N * 4 + 255) & ~(size_t)255; }
__host__ __device__ inline size_t pers_half_bytes(int rows, int N) {
  const size_t b = pers_arrive_bytes(N) + (size_t)N * rows * kBestStride * 8 + (size_t)rows * 8;
  return (b + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t step_half_bytes(int rows, int R, int mode, int NC) {
  (void)R;
  const size_t b = 256 + step_slots_bytes(rows, mode, NC) + (size_t)rows * 4;
  return (b + 255) & ~(size_t)255;
}

// PERS (mode 0): one persistent launch runs every position, the head staying
// in registers; the last workgroup of each position writes the tokens as
// tagged words ((position + 1) << 32 | token), and each workgroup's
// embedding loads of the next position wait (bounded) for the tags of the
// rows they need.  The grid must then be co-resident (one workgroup per CU
// at most); best keys and arrival counters are kept per position, so
// nothing is reset within a call.
// NZ (mode 0): the kernel draws the Gumbel noise of each element itself, in
// the epilogue, with the noise fill kernel's function (bit-identical
// values), instead of reading it from memory.
template <int R, bool FL, int MODE, bool PERS, bool NZ>
__global__ __launch_bounds__(kThreads, 1) void step_kernel(ChainParams p, int step_arg) {
  static_assert(!PERS || MODE == 0, "the persistent variant is mode 0");
  static_assert(!NZ || MODE == 0, "inline noise is mode 0's");
  constexpr int RPG = 16384 / R;
  constexpr int KSEG = R / 8;
  constexpr int ES = emb_stride<R>();
  constexpr int BS = bias_stride<R>();
  constexpr int IPL = RPG / kLanesPerRow;
  constexpr int kBlock = kLaunchRows;  // rows whose embeddings sit in LDS at once
  const bool base_f32 = FL && p.base_f32;
  const bool cache_f32 = FL && p.cache_f32;

  __shared__ int s_state[kBlock];
  __shared__ int s_active[kBlock];
  __shared__ float s_T[kBlock];
  __shared__ double s_rT[kBlock];
  __shared__ uint64_t s_key[kWaves][kBlock];
  __shared__ float s_wsum[kWaves][MODE == 1 ? kBlock : 1];
  __shared__ float s_bias[kWaves][kRowPass * BS];
  __shared__ int s_last;
  __shared__ uint32_t s_parity;
  __shared__ int s_toks[PERS ? MARKOV_MAX_ROWS : 1];  // PERS: the previous position's tokens
  __shared__ int64_t s_seed[NZ ? kBlock : 1];          // NZ: the block's rows' noise seeds
  __shared__ LogTable s_log;                           // NZ: the noise's log table
  extern __shared__ uint4 s_e[];  // [kBlock][ES]

  int tid = threadIdx.x;  // (PERS: made opaque at every position, see below)
  const int lane = tid & 63, wave = tid >> 6;
  // (Workgroup c holds chunk c: the XCD-contiguous assignment of the chain
  // kernel made no difference to the step kernels, whose streams of base
  // logits, noise and cache are row-major over all chunks.)
  const int c = blockIdx.x;
  const int rows = p.rows, V = p.V, NG = p.NG, G = p.G;
  uint32_t* header = reinterpret_cast<uint32_t*>(p.ws);
  const int rr = lane >> 3, q = lane & 7;
  const int g = c * kWaves + wave;  // this wave's group
  int v0 = g * RPG + q * IPL;  // this lane's first vocab id in the batch layout
  int step = PERS ? 0 : step_arg;
  const uint64_t deadline = now_ticks() + p.wait_ticks;  // (PERS: the token waits)
  TRACE_STAMP(c, step, 0);

  // NZ: the log table into LDS (as scalars: a struct copy lands on the stack)
  double t_c = 0.0, t_nlc = 0.0;
  if (NZ && tid < kLogTable) t_c = g_log_tab[tid].c, t_nlc = g_log_tab[tid].nlc;
  // The head of this wave's group, in flight while the rows are set up.
  uint4 h[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) h[s] = load_head_tile_clamped<R>(p.head, g < NG ? g : NG - 1, s, lane, V);
  if (tid == 0) s_parity = ld_agent32(header);
  if (NZ && tid < kLogTable) s_log.e[tid].c = t_c, s_log.e[tid].nlc = t_nlc;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const uint32_t parity = s_parity & 1u;
  unsigned char* half = p.ws + kHeader + parity * p.ws_half;
  uint32_t* arrive = reinterpret_cast<uint32_t*>(half);
  const size_t arrive_bytes = PERS ? pers_arrive_bytes(p.N) : 256;
  uint64_t* best = reinterpret_cast<uint64_t*>(half + arrive_bytes);
  int* tokbuf = reinterpret_cast<int*>(half + 256 + step_slots_bytes(rows, MODE, p.NC));
  uint64_t* tags = reinterpret_cast<uint64_t*>(half + arrive_bytes + (size_t)p.N * rows * kBestStride * 8);  // PERS
  uint32_t* sums = reinterpret_cast<uint32_t*>(best + (size_t)rows * p.NC);  // mode 1
  if (step == 0) {
    // Clear the other half for the next call (nobody reads it in this one).
    uint4* other = reinterpret_cast<uint4*>(p.ws + kHeader + (parity ^ 1u) * p.ws_half);
    const size_t n16 = p.clear_bytes / 16;
    for (size_t k = (size_t)c * kThreads + tid; k < n16; k += (size_t)G * kThreads) other[k] = make_uint4(0, 0, 0, 0);
  }
  float* sb = s_bias[wave];

  struct In {
    uint32_t bw[IPL];
    float nz[IPL];  // (unused with NZ)
  };
  // Batch inputs of rows b0 .. b0 + 7 of the current block (row rr of the
  // batch in this lane).  Every lane loads, so that no branch skips the
  // loads and the waits for a batch's inputs can count the loads issued
  // after them.  A lane whose row is inactive (this includes every row of a
  // batch past the block's end) or whose ids lie past the vocabulary reads
  // the arrays' first elements instead, as does a lane of a
  // zero-temperature row for the noise; the epilogue ignores these values.
  // The persistent variant instead reloads the block's last batch for a
  // batch past the block's end (lines still in the L2s): measured faster
  // there, and slower for the per-position launches.
  auto load_in = [&](int rb, int b0, In& in) {
    if constexpr (PERS) {
      const int nbr_in = rows - rb < kBlock ? rows - rb : kBlock;
      if (b0 >= nbr_in) b0 = (nbr_in - 1) / kBatch * kBatch;
    }
    const int bl = b0 + rr;
    int b = rb + bl;
    asm volatile("" : "+v"(b));
    const bool lok = bl < kBlock && b < rows && g < NG && v0 < V && s_active[bl];
    {
      const long long at = lok ? (long long)b * p.base_rs + (long long)step * p.base_ss + v0 : 0;
      if (base_f32) {
        const uint4* brow = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.base) + at);
#pragma unroll
        for (int e4 = 0; e4 < IPL / 4; ++e4) {
          const uint4 t = brow[e4];
          in.bw[4 * e4] = t.x, in.bw[4 * e4 + 1] = t.y, in.bw[4 * e4 + 2] = t.z, in.bw[4 * e4 + 3] = t.w;
        }
      } else {
        const uint16_t* brow = reinterpret_cast<const uint16_t*>(p.base) + at;
        if constexpr (IPL == 8) {
          const uint4 t = *reinterpret_cast<const uint4*>(brow);
          in.bw[0] = t.x, in.bw[1] = t.y, in.bw[2] = t.z, in.bw[3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(brow);
          in.bw[0] = t.x, in.bw[1] = t.y;
        }
      }
      if (MODE == 0 && !NZ) {
        const bool nok = lok && s_T[bl] > 0.0f;
        const float4* grow =
            reinterpret_cast<const float4*>(p.gumbel + (nok ? ((size_t)b * p.N + step) * (size_t)V + v0 : 0));
#pragma unroll
        for (int e4 = 0; e4 < IPL / 4; ++e4) {
          const float4 t = grow[e4];
          in.nz[4 * e4] = t.x, in.nz[4 * e4 + 1] = t.y, in.nz[4 * e4 + 2] = t.z, in.nz[4 * e4 + 3] = t.w;
        }
      }
    }
  };

  // The embeddings of a row block, kPieces 16-byte pieces per thread, loaded
  // into registers one block ahead: the embedding table's rows of the
  // anchors (step 0) or of the previous step's winners.
  constexpr int kPieces = kBlock * KSEG / kThreads;
  static_assert(kPieces * kThreads == kBlock * KSEG, "whole pieces per thread");
  uint4 ne[kPieces];
  auto emb_load = [&](int rb2) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int k = j * kThreads + tid;
      const int bl = k / KSEG, seg = k - bl * KSEG;
      const int b = rb2 + bl;
      ne[j] = make_uint4(0, 0, 0, 0);
      int64_t tok = -1;
      if (b < rows) {
        if (PERS && step > 0) {
          tok = s_toks[b];  // -1 for an inert row
        } else if (step == 0) {
          const int64_t st = p.state_idx ? p.state_idx[b] : (int64_t)b;
          if (st >= 0 && st < p.cache_states) tok = p.prev[b];
        } else {
          tok = tokbuf[b];  // -1 for an inert row
        }
      }
      if (b < rows && tok >= 0 && tok < V) ne[j] = *reinterpret_cast<const uint4*>(p.embed + (size_t)tok * R + seg * 8);
    }
  };
  for (;; ++step) {
  if constexpr (PERS) {
    // Opaque at every position: the per-lane addresses derived from them
    // are then formed inside the loop instead of being hoisted out of it
    // and spilled (the head holds 128 registers for the whole launch).
    asm volatile("" : "+v"(v0), "+v"(tid));
  }
  if (PERS && step > 0) {
    TRACE_STAMP(c, step, 0);
    // Every row's token of the previous position: thread t waits (bounded)
    // for the tags of rows t, t + 512, ...; the tokens go to LDS.
    for (int b = tid; b < rows; b += kThreads) {
      uint64_t t = ld_agent(tags + b);
      while ((uint32_t)(t >> 32) != (uint32_t)step) {
        if (now_ticks() > deadline) {
          __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          t = 0;  // token 0: the launch runs to its end
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        t = ld_agent(tags + b);
      }
      s_toks[b] = (int)(uint32_t)t;
    }
    __syncthreads();
  }
  uint64_t* best_i = best + (size_t)(PERS ? step : (step & 1)) * rows * kBestStride;
  emb_load(0);

  for (int rb = 0; rb < rows; rb += kBlock) {
    const int nbr = rows - rb < kBlock ? rows - rb : kBlock;
    // ---- the block's rows: state, activity, temperature; embeddings.
    if (tid < nbr) {
      const int b = rb + tid;
      const int64_t st = p.state_idx ? p.state_idx[b] : (int64_t)b;
      const int64_t tok = p.prev[b];
      const float T = p.temp[b];
      int active = st >= 0;
      if (active && st >= p.cache_states) {
        active = 0;
        if (c == 0 && step == 0)
          __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_BAD_STATE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (active && (tok < 0 || tok >= V)) {
        active = 0;
        if (c == 0 && step == 0)
          __hip_atomic_fetch_or(header + 1, MARKOV_DEVERR_BAD_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_state[tid] = (int)st;
      s_active[tid] = active;
      s_T[tid] = T;
      s_rT[tid] = T > 0.0f ? 1.0 / (double)T : 0.0;
      if constexpr (NZ) s_seed[tid] = p.seeds[b];
    }
    if (lane == 0)
      for (int k = 0; k < kBlock; ++k) s_key[wave][k] = kNoCandidate;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int k = j * kThreads + tid;
      const int bl = k / KSEG, seg = k - bl * KSEG;
      if (bl < nbr && s_active[bl]) s_e[bl * ES + seg] = ne[j];
    }
    // the first batches' inputs and the next block's embeddings, then the
    // embeddings visible to every wave
    const int nbat = (nbr + kBatch - 1) / kBatch;
    // kPf + 1 input sets in a fixed rotation: batch t reads set
    // t mod kSets and, before its epilogue, loads batch t + kPf into
    // the set batch t - 1 has finished with.  The batch loop is unrolled by
    // kSets so that every set keeps its registers across iterations: a
    // register copy at the loop's back edge would wait for the loads still
    // in flight and leave a single batch of epilogue to hide them.
    // Batches past the block's end load the dummy inputs too: with the same
    // loads on every path, the wait for a batch's inputs is not forced down
    // to the most recent load by a path that skipped the later ones.
    // The inverse CDF at rank 256 with bf16 types keeps three batches in
    // flight: its input sets hold no noise, so the fourth set fits without
    // spills (256 rows 654.7 -> 650.4 us per call); at rank 512 or with fp32
    // types it spills.  In mode 0 the fourth set spilled too (628 -> 706 us
    // with the noise read), and with inline noise the draw, not the memory
    // latency, sets the pace (1177 -> 1207 us).
    constexpr int kPf = (MODE == 1 && R == 256 && !FL) ? 3 : kPrefetch;
    constexpr int kSets = kPf + 1;
    In in[kSets];
#pragma unroll
    for (int k = 0; k < kPf; ++k) load_in(rb, k * kBatch, in[k]);
    if (rb + kBlock < rows) emb_load(rb + kBlock);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (rb == 0) TRACE_STAMP(c, step, 1);

    for (int t0 = 0; t0 < nbat; t0 += kSets) {
#pragma unroll
    for (int u = 0; u < kSets; ++u) {
      const int t = t0 + u;
      if (t >= nbat) break;
      const int b0 = t * kBatch;
      if ((t & 1) == 0) {
        const int np = nbr - b0 < kRowPass ? nbr - b0 : kRowPass;
        // (256 rows: persistent step kernel 631 -> 627 us per call, inverse
        // CDF 670 -> 656 us; EB = 4 in mode 0 was 629 us)
        group_bias<R, MODE == 1 ? 4 : 2>(h, s_e, b0, np, lane, sb);
      }
      const In& cur = in[u];
      load_in(rb, (t + kPf) * kBatch, in[(u + kPf) % kSets]);
      // ---- epilogue of the batch (row rr of the batch, IPL ids from v0)
      const int bl = b0 + rr;
      const bool ok = bl < nbr && g < NG && v0 < V && s_active[bl];
      const float T = s_T[bl < kBlock ? bl : 0];
      const double rT = s_rT[bl < kBlock ? bl : 0];
      const float* sbt = sb + (t & 1) * kBatch * BS;
      float bsum[IPL];
#pragma unroll
      for (int e4 = 0; e4 < IPL / 4; ++e4) {
        const float4 v4 = *reinterpret_cast<const float4*>(sbt + rr * BS + q * IPL + 4 * e4);
        bsum[4 * e4] = v4.x, bsum[4 * e4 + 1] = v4.y, bsum[4 * e4 + 2] = v4.z, bsum[4 * e4 + 3] = v4.w;
      }
      float x[IPL];
#pragma unroll
      for (int e = 0; e < IPL; ++e) {
        const uint32_t w = cur.bw[e / 2];
        const float base = base_f32 ? __uint_as_float(cur.bw[e])
                                    : __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        x[e] = __fmul_rn(__fadd_rn(base, bf16_round(bsum[e])), p.mult);
      }
      if (p.has_cap) {
#pragma unroll
        for (int e = 0; e < IPL; ++e) x[e] = __fmul_rn(tanhf(__fmul_rn(x[e], p.inv_cap)), p.cap);
      }
      uint32_t cw[IPL / 2];
      float z[IPL];
#pragma unroll
      for (int e = 0; e < IPL / 2; ++e) {
        cw[e] = f32x2_to_bf16x2(x[2 * e], x[2 * e + 1]);
        z[2 * e] = cache_f32 ? x[2 * e] : __uint_as_float(cw[e] << 16);
        z[2 * e + 1] = cache_f32 ? x[2 * e + 1] : __uint_as_float(cw[e] & 0xFFFF0000u);
      }
      if (ok) {
        const long long at = (long long)s_state[bl] * p.cache_rs + (long long)step * p.cache_ss + v0;
        if (cache_f32) {
          u32x4_t* crow = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(p.cache) + at);
#pragma unroll
          for (int e4 = 0; e4 < IPL / 4; ++e4)
            __builtin_nontemporal_store((u32x4_t){__float_as_uint(z[4 * e4]), __float_as_uint(z[4 * e4 + 1]),
                                                  __float_as_uint(z[4 * e4 + 2]), __float_as_uint(z[4 * e4 + 3])},
                                        crow + e4);
        } else {
          uint16_t* crow = reinterpret_cast<uint16_t*>(p.cache) + at;
          if constexpr (IPL == 8)
            __builtin_nontemporal_store((u32x4_t){cw[0], cw[1], cw[2], cw[3]}, reinterpret_cast<u32x4_t*>(crow));
          else
            __builtin_nontemporal_store((u32x2_t){cw[0], cw[1]}, reinterpret_cast<u32x2_t*>(crow));
        }
      }
      if (T > 0.0f) {
        if (T != 1.0f) {
#pragma unroll
          for (int e = 0; e < IPL; ++e) z[e] = div_by_recip(z[e], rT);
        }
        if constexpr (MODE == 0 && NZ) {
          if (ok) {
            const uint64_t pk = noise_prefix(s_seed[bl], rb + bl, step);
            // two ids at a time: four left more registers spilled (at 256
            // rows the persistent step kernel took 1177 vs 1138 us per call)
#pragma unroll
            for (int e = 0; e < IPL; e += 2) {
              float g2[2];
              gumbel_noise<2>(pk, v0 + e, s_log, g2);
#pragma unroll
              for (int k = 0; k < 2; ++k) z[e + k] = __fadd_rn(z[e + k], g2[k]);
            }
          }
        } else if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < IPL; ++e) z[e] = __fadd_rn(z[e], cur.nz[e]);
        }
      }
      // this lane's first NaN, else first maximum; then the row's over its 8 lanes
      int kbest = INT_MIN;
      uint32_t ebest = 0, enan = IPL;
#pragma unroll
      for (int e = 0; e < IPL; ++e) {
        const bool isn = isnan(z[e]);
        enan = (isn && enan == IPL) ? e : enan;
        const int k = isn ? INT_MIN : order_key(__fadd_rn(z[e], 0.0f));
        ebest = k > kbest ? e : ebest;
        kbest = k > kbest ? k : kbest;
      }
      if (!ok) kbest = INT_MIN, enan = IPL;
      const int gmax = group8_imax(kbest);
      const uint32_t gid = group8_umin(kbest != INT_MIN && kbest == gmax ? (uint32_t)v0 + ebest : 0xFFFFFFFFu);
      const uint32_t gnan = group8_umin(enan < IPL ? (uint32_t)v0 + enan : 0xFFFFFFFFu);
      float wsum = 0.0f;
      if (MODE == 1) {
        // the group's sum of exp(z - max), as the persistent kernel forms it
        const float m = order_key_inv(gmax);
        float sm = 0.0f;
        if (ok && gmax != INT_MIN && isfinite(m)) {
#pragma unroll
          for (int e = 0; e < IPL; ++e) sm += isnan(z[e]) ? 0.0f : __expf(z[e] - m);
        }
        wsum = group8_sum(sm);
      }
      if (q == 0 && ok) {
        s_key[wave][bl] = gnan != 0xFFFFFFFFu ? ((0xFFFFFFFFull << 32) | (0xFFFFFFFFu - gnan))
                          : gmax != INT_MIN ? (((uint64_t)score_ord(order_key_inv(gmax)) << 32) | (0xFFFFFFFFu - gid))
                                            : kNoCandidate;
        if (MODE == 1) s_wsum[wave][bl] = wsum;
      }
    }
    }
    // ---- the block's keys: the workgroup's best per row into the row's
    // slot (mode 0), or the chunk's partials of every row (mode 1: the 8
    // waves' partials combined in wave order, as the persistent kernel does).
    __syncthreads();
    if (tid < nbr && s_active[tid]) {
      uint64_t K = kNoCandidate;
      for (int w = 0; w < kWaves; ++w) K = umax64(K, s_key[w][tid]);
      if (MODE == 0) {
        if (K != kNoCandidate)
          __hip_atomic_fetch_max(best_i + (size_t)(rb + tid) * kBestStride, K, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      } else {
        float S = 0.0f;
        const float M = ord_score((uint32_t)(K >> 32));
        if (K != kNoCandidate && isfinite(M)) {
          for (int w = 0; w < kWaves; ++w) {
            const uint64_t kw = s_key[w][tid];
            const float mw = ord_score((uint32_t)(kw >> 32));
            if (kw != kNoCandidate && isfinite(mw)) S += s_wsum[w][tid] * expf(mw - M);
          }
        }
        const size_t slot = (size_t)(rb + tid) * p.NC + c;
        best[slot] = K;
        sums[slot] = __float_as_uint(S);
      }
    }
    __syncthreads();
  }
  if (MODE == 1) {
    TRACE_STAMP(c, step, 2);
    return;  // the pick kernel follows
  }

  // ---- arrival; the last workgroup of the step picks every row's winner.
  TRACE_STAMP(c, step, 2);
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(arrive + (PERS ? step : (step & 1)), 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)(G - 1);
  }
  __syncthreads();
  if (s_last) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int b = tid; b < rows; b += kThreads) {
      const int64_t st = p.state_idx ? p.state_idx[b] : (int64_t)b;
      const int64_t tok0 = p.prev[b];
      const bool active = st >= 0 && st < p.cache_states && tok0 >= 0 && tok0 < V;
      int tok = -1;
      if (active) {
        const uint64_t K = ld_agent(best_i + (size_t)b * kBestStride);
        const uint32_t win = key_id(K);
        tok = (K > kNoCandidate && win < (uint32_t)V) ? (int)win : 0;
        p.tokens[(long long)b * p.tok_rs + step] = tok;
        if (!PERS) st_agent(best_i + (size_t)b * kBestStride, 0);  // for step + 2
      }
      if (PERS)
        st_agent(tags + b, ((uint64_t)(step + 1) << 32) | (uint32_t)tok);
      else
        tokbuf[b] = tok;
    }
    if (tid == 0) {
      if (!PERS) st_agent32(arrive + (step & 1), 0u);
      // every workgroup of the call has read the parity by now
      if (step + 1 == p.N) st_agent32(header, parity ^ 1u);
    }
    __syncthreads();
    TRACE_STAMP(c, step, 3);
  }
  if (!PERS || step + 1 == p.N) return;
  }
}

// Mode 1, after the step kernel of each position: one wave per request row
// draws the row's token from the chunks' partials.  The arithmetic is the
// persistent kernel's, in the same order (its leader's combination of the
// chunks, search and scan of the chosen chunk), so both paths
// draw the same tokens.
template <int R, bool FL>
__global__ __launch_bounds__(64) void pick_kernel(ChainParams p, int step) {
  constexpr int RPG = 16384 / R;
  constexpr int CHUNK = kWaves * RPG;  // vocab ids per chunk
  constexpr int PER = CHUNK / 64;      // ids per lane in the chunk scan
  static_assert(PER == 8 || PER == 4, "chunk slice");
  const bool cache_f32 = FL && p.cache_f32;
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int rows = p.rows, V = p.V, NC = p.NC;
  uint32_t* header = reinterpret_cast<uint32_t*>(p.ws);
  const uint32_t parity = ld_agent32(header) & 1u;
  unsigned char* half = p.ws + kHeader + parity * p.ws_half;
  uint32_t* arrive = reinterpret_cast<uint32_t*>(half);
  const uint64_t* keys = reinterpret_cast<const uint64_t*>(half + 256) + (size_t)b * NC;
  const uint32_t* sums = reinterpret_cast<const uint32_t*>(half + 256 + (size_t)rows * NC * 8) + (size_t)b * NC;
  int* tokbuf = reinterpret_cast<int*>(half + 256 + step_slots_bytes(rows, 1, NC));
  const int64_t st = p.state_idx ? p.state_idx[b] : (int64_t)b;
  const int64_t tok0 = p.prev[b];
  const bool active = st >= 0 && st < p.cache_states && tok0 >= 0 && tok0 < V;
  int tok = -1;
  if (active) {
    const float T = p.temp[b];
    const int KPL = (NC + 63) / 64;  // contiguous chunks per lane
    uint64_t K = kNoCandidate;
    for (int k = 0; k < KPL; ++k) {
      const int c = lane * KPL + k;
      if (c < NC) K = umax64(K, keys[c]);
    }
    K = wave_max_u64(K);
    const float M = ord_score((uint32_t)(K >> 32));
    if (!(T > 0.0f) || !isfinite(M)) {
      const uint32_t tk = key_id(K);  // argmax: the lowest NaN id, or of the maximum
      tok = tk < (uint32_t)V ? (int)tk : 0;
    } else {
      const float u = hash_uniform(noise_prefix(p.seeds[b], b, step));
      // Chunk c's weight: its sum rescaled by exp(m_c - M); the lanes'
      // totals scanned in chunk order.
      auto weight = [&](int k, float& e) -> float {
        e = 0.0f;
        const int c = lane * KPL + k;
        if (c >= NC) return 0.0f;
        const uint64_t key = keys[c];
        const float mc = ord_score((uint32_t)(key >> 32));
        if (key == kNoCandidate || !isfinite(mc)) return 0.0f;
        e = expf(mc - M);
        return __uint_as_float(sums[c] & 0x7FFFFFFFu) * e;
      };
      float lsum = 0.0f;
      for (int k = 0; k < KPL; ++k) {
        float e;
        lsum += weight(k, e);
      }
      const float incl = wave_incl_scan(lsum);
      const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
      const float t = u * total;
      // the first chunk with weight whose inclusive prefix exceeds t, else
      // the last chunk with weight
      int found = -1, last_pos = -1;
      float before = 0.0f, wfound = 0.0f, last_before = 0.0f, last_w = 0.0f;
      float run = incl - lsum;
      for (int k = 0; k < KPL; ++k) {
        float e;
        const float w = weight(k, e);
        const int c = lane * KPL + k;
        if (found < 0 && w > 0.0f && run + w > t) {
          found = c;
          before = run;
          wfound = e;
        }
        if (w > 0.0f) {
          last_pos = c;
          last_before = run;
          last_w = e;
        }
        run += w;
      }
      const uint64_t hit = __ballot(found >= 0);
      int o;
      float tl;
      if (hit) {
        const int src = __builtin_ctzll(hit);
        o = __shfl(found, src);
        tl = (t - __shfl(before, src)) / __shfl(wfound, src);
      } else {
        const uint64_t any = __ballot(last_pos >= 0);
        const int src = 63 - __builtin_clzll(any);
        o = __shfl(last_pos, src);
        tl = (t - __shfl(last_before, src)) / __shfl(last_w, src);
      }
      if (!(tl >= 0.0f)) tl = 0.0f;
      if ((unsigned)o >= (unsigned)NC) o = NC - 1;
      // The chosen chunk's cache values in vocabulary order, PER per lane.
      const double rT = 1.0 / (double)T;
      const int v0 = o * CHUNK + lane * PER;
      const long long at = st * p.cache_rs + (long long)step * p.cache_ss + v0;
      uint32_t cw[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) cw[k] = 0;
      if (v0 < V) {
        if (cache_f32) {
          const uint4* crow = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.cache) + at);
#pragma unroll
          for (int k4 = 0; k4 < PER / 4; ++k4) {
            const uint4 t4 = crow[k4];
            cw[4 * k4] = t4.x, cw[4 * k4 + 1] = t4.y, cw[4 * k4 + 2] = t4.z, cw[4 * k4 + 3] = t4.w;
          }
        } else {
          const uint16_t* crow = reinterpret_cast<const uint16_t*>(p.cache) + at;
          uint32_t pk[PER / 2];
          if constexpr (PER == 8) {
            const uint4 t4 = *reinterpret_cast<const uint4*>(crow);
            pk[0] = t4.x, pk[1] = t4.y, pk[2] = t4.z, pk[3] = t4.w;
          } else {
            const uint2 t2 = *reinterpret_cast<const uint2*>(crow);
            pk[0] = t2.x, pk[1] = t2.y;
          }
#pragma unroll
          for (int k = 0; k < PER; ++k) cw[k] = (k & 1) ? (pk[k / 2] & 0xFFFF0000u) : (pk[k / 2] << 16);
        }
      }
      float z[PER];
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float cv = __uint_as_float(cw[k]);
        z[k] = v0 < V ? (T != 1.0f ? div_by_recip(cv, rT) : cv) : -INFINITY;
        m = fmaxf(m, z[k]);
      }
      m = order_key_inv(wave_imax(order_key(m)));  // the chunk's maximum (no NaN here)
      float w[PER];
      float csum = 0.0f;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        w[k] = (v0 + k < V && z[k] > -INFINITY) ? __expf(z[k] - m) : 0.0f;
        csum += w[k];
      }
      float crun = wave_incl_scan(csum) - csum;
      int fv = -1, lastv = -1;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if (fv < 0 && w[k] > 0.0f && crun + w[k] > tl) fv = v0 + k;
        if (w[k] > 0.0f) lastv = v0 + k;
        crun += w[k];
      }
      const uint64_t chit = __ballot(fv >= 0);
      if (chit) {
        tok = __shfl(fv, __builtin_ctzll(chit));
      } else {
        const uint64_t any = __ballot(lastv >= 0);
        tok = any ? __shfl(lastv, 63 - __builtin_clzll(any)) : o * CHUNK;
      }
    }
    if (lane == 0) p.tokens[(long long)b * p.tok_rs + step] = tok;
  }
  if (lane == 0) tokbuf[b] = tok;
  TRACE_STAMP_MAX(0, step, 3);  // the latest pick of the position
  // The last step: the last wave to arrive flips the call parity (every
  // pick wave of the call has read it by then, every step launch is done).
  if (step + 1 == p.N && lane == 0) {
    const uint32_t old = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)(rows - 1)) {
      st_agent32(arrive, 0u);
      st_agent32(header, parity ^ 1u);
    }
  }
}

__host__ size_t step_half_bytes_host(int rows, int rank, int mode, int NC) {
  return step_half_bytes(rows, rank, mode, NC);
}

template <bool FL, bool NZ>
const void* step_kernel_nz(int rank, bool pers) {
  if (pers)
    return rank == 256 ? (const void*)step_kernel<256, FL, 0, true, NZ> : (const void*)step_kernel<512, FL, 0, true, NZ>;
  return rank == 256 ? (const void*)step_kernel<256, FL, 0, false, NZ> : (const void*)step_kernel<512, FL, 0, false, NZ>;
}
template <bool FL>
const void* step_kernel_for(int rank, int mode, bool pers = false, bool nz = false) {
  if (mode == 1)
    return rank == 256 ? (const void*)step_kernel<256, FL, 1, false, false>
                       : (const void*)step_kernel<512, FL, 1, false, false>;
  return nz ? step_kernel_nz<FL, true>(rank, pers) : step_kernel_nz<FL, false>(rank, pers);
}
template <bool FL>
const void* pick_kernel_for(int rank) {
  return rank == 256 ? (const void*)pick_kernel<256, FL> : (const void*)pick_kernel<512, FL>;
}

// ================================================================= host ==

thread_local std::string g_last_error;
std::atomic<int> g_grid_override{0};
std::atomic<unsigned long long> g_wait_ticks{kTimeoutTicks};
std::atomic<int> g_batch_path{0};  // 0 auto, 1 persistent launches, 2 step kernels (mode 0)

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
    return fail(MARKOV_E_UNSUPPORTED, "rank=%d (the library is compiled for 256 or 512)", rank);
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

// Kernel kinds: 0 streamed head, 1 resident head, 2 resident with at most
// kAhead rows, 3 resident with one row (mode 0).
template <int R, int MODE, bool FL, bool NZ>
const void* kernel_variant(int kind) {
  switch (kind) {
    case 0: return (const void*)chain_kernel<R, MODE, false, false, false, FL, NZ>;
    case 1: return (const void*)chain_kernel<R, MODE, true, false, false, FL, NZ>;
    case 2: return (const void*)chain_kernel<R, MODE, true, true, false, FL, NZ>;
    default: return (const void*)chain_kernel<R, MODE, true, true, MODE == 0, FL, NZ>;
  }
}

// Kernel kinds: 0 streamed head; 1 resident, more than kAhead rows; 2
// resident, prefetched rows; 3 one row (mode 0).
int kernel_kind(int rows, int mode, bool res) {
  if (!res) return 0;
  if (rows == 1 && mode == 0) return 3;
  return rows <= kAhead ? 2 : 1;
}

template <bool FL, bool NZ>
const void* kernel_for_fl(int rank, int mode, int kind) {
  if (rank == 256) return mode == 0 ? kernel_variant<256, 0, FL, NZ>(kind) : kernel_variant<256, 1, FL, false>(kind);
  return mode == 0 ? kernel_variant<512, 0, FL, NZ>(kind) : kernel_variant<512, 1, FL, false>(kind);
}

// fl: fp32 base logits or cache (the kernels that read those flags); nz:
// inline noise (mode 0; ignored in mode 1).
const void* kernel_for(int rank, int mode, int kind, bool fl, bool nz) {
  if (fl) return nz ? kernel_for_fl<true, true>(rank, mode, kind) : kernel_for_fl<true, false>(rank, mode, kind);
  return nz ? kernel_for_fl<false, true>(rank, mode, kind) : kernel_for_fl<false, false>(rank, mode, kind);
}

// The LDS one workgroup may use on the current device, and a chain kernel's
// static LDS (its __shared__ arrays); the rest is the kernel's dynamic LDS:
// the embeddings and, on a streamed head, the tiles kept across steps.
int device_lds_bytes() {
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return lds;
}
int static_lds_bytes(const void* kern) {
  hipFuncAttributes a;
  if (hipFuncGetAttributes(&a, kern) != hipSuccess) return -1;
  return (int)a.sharedSizeBytes;
}

// Dynamic LDS above the default per-launch limit is opted into once per
// process for every kernel: all the LDS a workgroup may have beside the
// kernel's static arrays.
int prepare_kernels() {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    const int lds = device_lds_bytes();
    // (at least the embeddings of kLaunchRows rows)
    auto allow = [&](const void* kern, int rank) {
      const int st = static_lds_bytes(kern);
      const int emb = kLaunchRows * (rank / 8 + 1) * 16;
      hipError_t e = st < 0 ? hipErrorInvalidValue
                            : hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  lds - st > emb ? lds - st : emb);
      if (e != hipSuccess && err == hipSuccess) err = e;
    };
    for (int rank : {256, 512})
      for (int mode : {0, 1})
        for (int kind = 0; kind < 4; ++kind)
          for (int flags = 0; flags < 4; ++flags) allow(kernel_for(rank, mode, kind, flags & 1, flags & 2), rank);
    for (int rank : {256, 512})
      for (int fl = 0; fl < 2; ++fl)
        for (int k = 0; k < 5; ++k) {  // mode 0 per position, mode 1, mode 0 persistent; both with inline noise
          const int mode = k == 1;
          const bool pers = k == 2 || k == 4, nz = k >= 3;
          allow(fl ? step_kernel_for<true>(rank, mode, pers, nz) : step_kernel_for<false>(rank, mode, pers, nz), rank);
        }
  });
  if (err != hipSuccess) return fail(MARKOV_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
  return MARKOV_OK;
}

// Streamed head: kParked<R> when chunk 1's parked tiles fit in the LDS left
// beside the kernel's static arrays and the embeddings, else 0.
int parked_slots(const void* kern, int rank, size_t emb_bytes) {
  const int np = rank == 512 ? kParked<512> : kParked<256>;
  const int st = static_lds_bytes(kern);
  if (st < 0) return 0;
  const long long need = (long long)st + (long long)emb_bytes + (long long)kWaves * np * 64 * 16;
  return need <= device_lds_bytes() ? np : 0;
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
  const size_t shmem = (size_t)rows * (rank / 8 + 1) * 16;
  long long g = cus;  // one workgroup per CU: the grid never exceeds the CUs
  if (g > sh.NC) g = sh.NC;
  const int ov = g_grid_override.load();
  if (ov > 0 && ov < g) g = ov;
  if (g > 64 * kMaxPollPerLane) g = 64 * kMaxPollPerLane;
  const bool resident = (g == sh.NC);
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel_for(rank, mode, kernel_kind(rows, mode, resident), false, false),
                                                    kThreads, shmem);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "occupancy query: %s", hipGetErrorString(e));
  if (per_cu < 1) return fail(MARKOV_E_HIP, "the chain kernel does not fit on a compute unit");
  *grid = (int)g;
  *res = resident;
  return MARKOV_OK;
}

// The allocation-free entry point's per-device state: the scratch array's
// device address (from hipGetSymbolAddress, with that device current) and the
// largest workspace half any call on the device has needed so far.  Every
// byte of a half beyond that mark is still zero (the array is zeroed once,
// by the first call, and no call writes beyond its own need), so a call
// clears only that much of the other half for the next call.
constexpr int kMaxDevices = 64;
struct ScratchState {
  unsigned char* ptr = nullptr;
  size_t high_water = 0;
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kMaxDevices];

int launch_zero(void* p, size_t bytes, void* stream) {
  const size_t n16 = bytes / 16;
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<uint4*>(p), n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "scratch clearing launch: %s", hipGetErrorString(e));
  return MARKOV_OK;
}

// The current device's scratch for a call needing need_half bytes per half:
// its address, and how much of the other half the call must clear.  The
// first call on a device looks the address up and enqueues the zeroing of
// the whole array on `stream`, ahead of its chain kernel.
int static_scratch(size_t need_half, void* stream, void** ws, size_t* clear_bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MARKOV_E_UNSUPPORTED, "device %d (max %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& st = g_scratch[dev];
  if (!st.ptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MARKOV_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int rc = launch_zero(ptr, kScratchBytes, stream);
    if (rc != MARKOV_OK) return rc;
    st.ptr = static_cast<unsigned char*>(ptr);
  }
  if (need_half > st.high_water) st.high_water = need_half;
  *ws = st.ptr;
  *clear_bytes = st.high_water;
  return MARKOV_OK;
}

// Both chain entry points.  no_alloc: the workspace is the library's static
// scratch (workspace_bytes is its size; there is no caller's buffer to
// check), and each call clears the scratch's high-water mark of the other
// half instead of the whole half.
int chain_sample(const void* base_logits, int64_t base_row_stride, int64_t base_step_stride,
                 const uint16_t* head, const uint16_t* embed, const int64_t* prev_tokens,
                 const float* temperature, const int64_t* seeds, const float* gumbel,
                 const int64_t* state_idx, float output_multiplier, float soft_cap, int rows,
                 int steps, int vocab, int rank, int mode, int64_t* draft_tokens,
                 int64_t tokens_row_stride, void* cache, int64_t cache_states,
                 int64_t cache_state_stride, int64_t cache_step_stride, void* workspace,
                 size_t workspace_bytes, void* stream, bool no_alloc) {
  const int base_f32 = (mode & MARKOV_BASE_F32) != 0, cache_f32 = (mode & MARKOV_CACHE_F32) != 0;
  const int noise_inline = (mode & MARKOV_NOISE_INLINE) != 0;
  mode &= ~kModeFlags;
  Shape sh;
  int rc = check_shape(rows, steps, vocab, rank, mode, &sh);
  if (rc != MARKOV_OK) return rc;
  if (noise_inline && mode != MARKOV_MODE_GUMBEL)
    return fail(MARKOV_E_INVAL, "MARKOV_NOISE_INLINE applies to MARKOV_MODE_GUMBEL only");
  if (noise_inline && !seeds) return fail(MARKOV_E_INVAL, "MARKOV_NOISE_INLINE needs seeds");
  if (!base_logits || !head || !embed || !prev_tokens || !temperature || !draft_tokens || !cache ||
      (!no_alloc && !workspace))
    return fail(MARKOV_E_INVAL, "a required pointer is null");
  if (mode == MARKOV_MODE_GUMBEL && !noise_inline && !gumbel)
    return fail(MARKOV_E_INVAL, "mode 0 needs gumbel noise (or MARKOV_NOISE_INLINE)");
  if (mode == MARKOV_MODE_INVCDF && !seeds) return fail(MARKOV_E_INVAL, "mode 1 needs seeds");
  if (!aligned16(base_logits) || !aligned16(head) || !aligned16(embed) || !aligned16(cache) ||
      (gumbel && !aligned16(gumbel)))
    return fail(MARKOV_E_INVAL, "base_logits, head, embed, cache and gumbel must be 16-byte aligned");
  if (!no_alloc && ((uintptr_t)workspace & 255u) != 0)
    return fail(MARKOV_E_INVAL, "workspace is not 256-byte aligned");
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
  // Calls with more rows than one launch takes run as consecutive launches
  // of at most kLaunchRows rows on the stream (each reads the head once);
  // they use the workspace one after another.
  const size_t need_half = call_half_bytes(rows, steps, sh.NC, mode, rank);
  const size_t need = kHeader + 2 * need_half;
  if (no_alloc && need > kScratchBytes)
    return fail(MARKOV_E_UNSUPPORTED,
                "this call shape needs %zu bytes of workspace; the allocation-free entry point has %zu "
                "(use markov_chain_sample with a workspace of markov_workspace_bytes)",
                need, (size_t)kScratchBytes);
  if (workspace_bytes < need)
    return fail(MARKOV_E_INVAL, "workspace_bytes=%zu < %zu needed", workspace_bytes, need);
  rc = prepare_kernels();
  if (rc != MARKOV_OK) return rc;
  size_t clear_bytes = ((workspace_bytes - kHeader) / 2) & ~(size_t)255;
  if (no_alloc) {
    rc = static_scratch(need_half, stream, &workspace, &clear_bytes);
    if (rc != MARKOV_OK) return rc;
  }
  const size_t besz = base_f32 ? 4 : 2;
  // Batches beyond one persistent launch run per position over all rows: a
  // step kernel (mode 0, the noise read from memory or drawn inline), or a
  // step kernel and a pick kernel (mode 1); also any batch, when the knob
  // asks for that path.
  const int path = g_batch_path.load();
  const bool use_step = path >= 2 || (path == 0 && rows > kLaunchRows);
  const bool step_nz = mode == MARKOV_MODE_GUMBEL && noise_inline;
  if (use_step) {
    // Mode 0: one persistent step kernel for all positions when its grid
    // (one workgroup per chunk) fits on the compute units at once and the
    // workspace holds its layout; otherwise one launch per position.
    bool pers = false;
    if (mode == MARKOV_MODE_GUMBEL && path != 2) {
      int dev = 0, cus = 0, per_cu = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu,
            (base_f32 || cache_f32) ? step_kernel_for<true>(rank, 0, true, step_nz) : step_kernel_for<false>(rank, 0, true, step_nz),
            kThreads, (size_t)kLaunchRows * (rank / 8 + 1) * 16);
      if (e != hipSuccess) return fail(MARKOV_E_HIP, "step kernel occupancy query: %s", hipGetErrorString(e));
      const size_t avail = no_alloc ? (kScratchBytes - kHeader) / 2 : ((workspace_bytes - kHeader) / 2) & ~(size_t)255;
      pers = per_cu >= 1 && sh.NC <= cus && pers_half_bytes(rows, steps) <= avail;
    }
    const size_t step_half = pers ? pers_half_bytes(rows, steps) : step_half_bytes(rows, rank, mode, sh.NC);
    const size_t step_need = kHeader + 2 * step_half;
    if (no_alloc && step_need > kScratchBytes)
      return fail(MARKOV_E_UNSUPPORTED,
                  "this call shape needs %zu bytes of workspace; the allocation-free entry point has %zu "
                  "(use markov_chain_sample with a workspace of markov_workspace_bytes)",
                  step_need, (size_t)kScratchBytes);
    if (!no_alloc && workspace_bytes < step_need)
      return fail(MARKOV_E_INVAL, "workspace_bytes=%zu < %zu needed by the step-kernel path", workspace_bytes,
                  step_need);
    if (no_alloc && need_half < step_half) {
      size_t cb = 0;
      rc = static_scratch(step_half, stream, &workspace, &cb);
      if (rc != MARKOV_OK) return rc;
      clear_bytes = cb;
    }
    ChainParams p = {};
    p.base = base_logits;
    p.base_f32 = base_f32;
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
    p.row_base = 0;
    p.N = steps;
    p.V = vocab;
    p.NG = sh.NG;
    p.NC = sh.NC;
    p.G = sh.NC;  // one workgroup per chunk
    p.tokens = draft_tokens;
    p.tok_rs = tokens_row_stride;
    p.cache = cache;
    p.cache_f32 = cache_f32;
    p.cache_rs = cache_state_stride;
    p.cache_ss = cache_step_stride;
    p.cache_states = cache_states;
    p.ws = (unsigned char*)workspace;
    p.ws_half = ((workspace_bytes - kHeader) / 2) & ~(size_t)255;
    p.clear_bytes = clear_bytes;
    p.wait_ticks = pers ? g_wait_ticks.load() : 0;  // (only the persistent variant waits)
    p.nres = 0;
    const bool fl = base_f32 || cache_f32;
    const void* kern =
        fl ? step_kernel_for<true>(rank, mode, pers, step_nz) : step_kernel_for<false>(rank, mode, pers, step_nz);
    const void* pick = fl ? pick_kernel_for<true>(rank) : pick_kernel_for<false>(rank);
    const size_t shmem = (size_t)kLaunchRows * (rank / 8 + 1) * 16;
    if (pers) {
      // A regular launch of at most one workgroup per CU (checked above):
      // on an otherwise idle device every workgroup is resident at once;
      // the token waits are bounded (MARKOV_DEVERR_TIMEOUT otherwise).
      int step = 0;
      void* args[] = {&p, &step};
      hipError_t e = hipLaunchKernel(kern, dim3(sh.NC), dim3(kThreads), args, (unsigned)shmem, (hipStream_t)stream);
      if (e != hipSuccess) return fail(MARKOV_E_HIP, "persistent step kernel launch: %s", hipGetErrorString(e));
      return MARKOV_OK;
    }
    for (int i = 0; i < steps; ++i) {
      int step = i;
      void* args[] = {&p, &step};
      hipError_t e = hipLaunchKernel(kern, dim3(sh.NC), dim3(kThreads), args, (unsigned)shmem, (hipStream_t)stream);
      if (e != hipSuccess) return fail(MARKOV_E_HIP, "step kernel launch (step %d): %s", i, hipGetErrorString(e));
      if (mode == MARKOV_MODE_INVCDF) {
        e = hipLaunchKernel(pick, dim3(rows), dim3(64), args, 0, (hipStream_t)stream);
        if (e != hipSuccess) return fail(MARKOV_E_HIP, "pick kernel launch (step %d): %s", i, hipGetErrorString(e));
      }
    }
    return MARKOV_OK;
  }
  for (int r0 = 0; r0 < rows; r0 += kLaunchRows) {
    const int nr = rows - r0 < kLaunchRows ? rows - r0 : kLaunchRows;
    int G = 0;
    bool res = false;
    rc = pick_grid(nr, rank, mode, sh, &G, &res);
    if (rc != MARKOV_OK) return rc;

    ChainParams p;
    p.base = static_cast<const char*>(base_logits) + (size_t)r0 * (size_t)base_row_stride * besz;
    p.base_f32 = base_f32;
    p.base_rs = base_row_stride;
    p.base_ss = base_step_stride;
    p.head = head;
    p.embed = embed;
    p.prev = prev_tokens + r0;
    p.temp = temperature + r0;
    p.seeds = seeds ? seeds + r0 : nullptr;
    p.gumbel = gumbel ? gumbel + (size_t)r0 * steps * vocab : nullptr;
    p.state_idx = state_idx ? state_idx + r0 : nullptr;
    p.mult = output_multiplier;
    p.cap = soft_cap;
    p.inv_cap = soft_cap > 0.0f ? 1.0f / soft_cap : 1.0f;
    p.has_cap = soft_cap > 0.0f;
    p.rows = nr;
    p.row_base = r0;
    p.N = steps;
    p.V = vocab;
    p.NG = sh.NG;
    p.NC = sh.NC;
    p.G = G;
    p.tokens = draft_tokens + (size_t)r0 * tokens_row_stride;
    p.tok_rs = tokens_row_stride;
    p.cache = cache;
    p.cache_f32 = cache_f32;
    p.cache_rs = cache_state_stride;
    p.cache_ss = cache_step_stride;
    p.cache_states = cache_states;
    p.ws = (unsigned char*)workspace;
    p.ws_half = ((workspace_bytes - kHeader) / 2) & ~(size_t)255;
    p.clear_bytes = clear_bytes;
    p.wait_ticks = g_wait_ticks.load();

    const void* kern = kernel_for(rank, mode, kernel_kind(nr, mode, res), base_f32 || cache_f32, noise_inline);
    size_t shmem = (size_t)nr * (rank / 8 + 1) * 16;
    p.nres = res ? 0 : parked_slots(kern, rank, shmem);
    shmem += (size_t)kWaves * p.nres * 64 * 16;
    void* args[] = {&p};
    // A regular launch: the grid is at most one workgroup per CU and the
    // kernel's resources admit only one per CU, so on an otherwise idle
    // device every workgroup is resident at once; every cross-workgroup wait
    // is bounded, so a grid that is not co-resident ends with
    // MARKOV_DEVERR_TIMEOUT instead of hanging.
    hipError_t e = hipLaunchKernel(kern, dim3(G), dim3(kThreads), args, (unsigned)shmem,
                                   (hipStream_t)stream);
    if (e != hipSuccess)
      return fail(MARKOV_E_HIP, "chain launch (rows %d..%d, grid %d): %s", r0, r0 + nr - 1, G,
                  hipGetErrorString(e));
  }
  return MARKOV_OK;
}

}  // namespace

extern "C" {

size_t markov_workspace_bytes(int rows, int steps, int vocab, int rank, int mode) {
  mode &= ~kModeFlags;
  Shape sh;
  if (check_shape(rows, steps, vocab, rank, mode, &sh) != MARKOV_OK) return 0;
  size_t half = call_half_bytes(rows, steps, sh.NC, mode, rank);
  if (mode == MARKOV_MODE_GUMBEL && pers_half_bytes(rows, steps) > half) half = pers_half_bytes(rows, steps);
  return kHeader + 2 * half;
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
  dim3 grid((vocab / 4 + 511) / 512, steps, rows);
  hipLaunchKernelGGL(noise_fill_kernel, grid, dim3(256), 0, (hipStream_t)stream, gumbel, seeds, steps,
                     vocab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "noise launch: %s", hipGetErrorString(e));
  return MARKOV_OK;
}

int markov_chain_sample(const void* base_logits, int64_t base_row_stride, int64_t base_step_stride,
                        const uint16_t* head, const uint16_t* embed, const int64_t* prev_tokens,
                        const float* temperature, const int64_t* seeds, const float* gumbel,
                        const int64_t* state_idx, float output_multiplier, float soft_cap, int rows,
                        int steps, int vocab, int rank, int mode, int64_t* draft_tokens,
                        int64_t tokens_row_stride, void* cache, int64_t cache_states,
                        int64_t cache_state_stride, int64_t cache_step_stride, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return chain_sample(base_logits, base_row_stride, base_step_stride, head, embed, prev_tokens,
                      temperature, seeds, gumbel, state_idx, output_multiplier, soft_cap, rows, steps,
                      vocab, rank, mode, draft_tokens, tokens_row_stride, cache, cache_states,
                      cache_state_stride, cache_step_stride, workspace, workspace_bytes, stream, false);
}

int markov_chain_sample_noalloc(const void* base_logits, int64_t base_row_stride,
                                int64_t base_step_stride, const uint16_t* head, const uint16_t* embed,
                                const int64_t* prev_tokens, const float* temperature,
                                const int64_t* seeds, const float* gumbel, const int64_t* state_idx,
                                float output_multiplier, float soft_cap, int rows, int steps,
                                int vocab, int rank, int mode, int64_t* draft_tokens,
                                int64_t tokens_row_stride, void* cache, int64_t cache_states,
                                int64_t cache_state_stride, int64_t cache_step_stride, void* stream) {
  g_last_error.clear();
  return chain_sample(base_logits, base_row_stride, base_step_stride, head, embed, prev_tokens,
                      temperature, seeds, gumbel, state_idx, output_multiplier, soft_cap, rows, steps,
                      vocab, rank, mode, draft_tokens, tokens_row_stride, cache, cache_states,
                      cache_state_stride, cache_step_stride, nullptr, kScratchBytes, stream, true);
}

int markov_status(void* workspace, void* stream) {
  g_last_error.clear();
  const bool no_alloc = workspace == nullptr;
  if (no_alloc) {
    // the allocation-free entry point's scratch on the current device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MARKOV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MARKOV_E_UNSUPPORTED, "device %d (max %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    workspace = g_scratch[dev].ptr;
    if (!workspace) return MARKOV_OK;  // no allocation-free call has run on this device
  }
  uint32_t hdr[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(hdr, workspace, sizeof hdr, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "status read: %s", hipGetErrorString(e));
  if (hdr[1] == 0) return MARKOV_OK;
  if (no_alloc && (hdr[1] & MARKOV_DEVERR_TIMEOUT)) {
    // A wait gave up: the scratch may hold a half-used exchange.  Zero all
    // of it (the caller cannot), error word included.
    const int rc = launch_zero(workspace, kScratchBytes, stream);
    if (rc != MARKOV_OK) return rc;
    e = hipStreamSynchronize((hipStream_t)stream);
  } else {
    static const uint32_t zero = 0;
    e = hipMemcpyAsync((char*)workspace + 4, &zero, 4, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "status clear: %s", hipGetErrorString(e));
  return fail(MARKOV_E_DEVICE, "device error bits 0x%x:%s%s%s", hdr[1],
              (hdr[1] & MARKOV_DEVERR_BAD_TOKEN) ? " previous token outside [0, V);" : "",
              (hdr[1] & MARKOV_DEVERR_TIMEOUT) ? " cross-workgroup wait timed out;" : "",
              (hdr[1] & MARKOV_DEVERR_BAD_STATE) ? " state index beyond the cache;" : "");
}

const char* markov_last_error(void) { return g_last_error.c_str(); }

int markov_set_grid(int g) { return g_grid_override.exchange(g < 0 ? 0 : g); }

int markov_set_batch_path(int path) { return g_batch_path.exchange(path < 0 || path > 3 ? 0 : path); }

#ifdef MARKOV_TRACE
// Trace builds only: the exchange's floor.  `rounds` rounds of the one-row
// mode-0 exchange with no other work, on G workgroups of kThreads threads
// (one per CU): thread 0 of every workgroup publishes a nonzero key into its
// slot of the round; then either two levels as the chain kernel's one-row
// exchange (reducer workgroup r < reducers_for(G) has wave 0's lane l poll
// slot 64 r + l and writes the maximum into kPartCopies copies, kPartStride
// words apart; wave 0 of every workgroup polls the partials of copy
// wg % kPartCopies), or all-to-all (wave 0 of every workgroup polls all G
// slots, 4 per lane).  A workgroup starts the next round once it knows the
// maximum.  stamps[round][wg] = {publication, maximum known}, ticks of the
// 100 MHz clock; every wait gives up after wait_ticks.
__global__ __launch_bounds__(kThreads, 1) void exchange_probe_kernel(uint64_t* slots, uint64_t* part,
                                                                     uint64_t* stamps, int G, int rounds,
                                                                     int two_level, uint64_t wait_ticks) {
  const int wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t deadline = now_ticks() + wait_ticks;
  const int NR = reducers_for(G);
  for (int r = 0; r < rounds; ++r) {
    uint64_t* sl = slots + (size_t)r * G;
    uint64_t* pr = part + (size_t)r * kPartCopies * kPartStride;
    if (tid == 0) {
      const uint64_t h = splitmix64(((uint64_t)r << 32) | (uint32_t)wg);
      const uint64_t key = ((h >> 32) | 1ull) << 32 | (0xFFFFFFFFu - (uint32_t)wg);
      stamps[((size_t)r * G + wg) * 2] = now_ticks();
      st_agent(sl + wg, key);
    }
    if (wave == 0) {
      if (two_level && wg < NR) {
        const int idx = wg * 64 + lane;
        uint64_t x = idx < G ? 0 : kNoCandidate;
        for (;;) {
          if (x == 0) x = ld_agent(sl + idx);
          if (__all(x != 0) || now_ticks() > deadline) break;
          __builtin_amdgcn_s_sleep(1);
        }
        const uint64_t K = wave_max_u64(x == 0 ? kNoCandidate : x);
        if (lane < kPartCopies) st_agent(pr + lane * kPartStride + wg, K);
      }
      const uint64_t* src = two_level ? pr + (wg % kPartCopies) * kPartStride : sl;
      const int n = two_level ? NR : G;
      uint64_t xs[4] = {0, 0, 0, 0};
      for (;;) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = lane + 64 * k;
          if (idx >= n) xs[k] = kNoCandidate;
          else if (xs[k] == 0) xs[k] = ld_agent(src + idx);
          all = all && xs[k] != 0;
        }
        if (__all(all) || now_ticks() > deadline) break;
        __builtin_amdgcn_s_sleep(1);
      }
      uint64_t m = kNoCandidate;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = umax64(m, xs[k]);
      m = wave_max_u64(m);
      if (lane == 0) stamps[((size_t)r * G + wg) * 2 + 1] = m ? now_ticks() : 0;
    }
    __syncthreads();
  }
}

// Runs the probe above (G <= the device's CUs, rounds <= 4096) and copies
// the stamps, [rounds][G][2] u64, to host memory.  Synchronising.
int markov_trace_exchange_probe(int G, int rounds, int two_level, uint64_t* stamps_host) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "exchange probe: %s", hipGetErrorString(e));
  if (G < 1 || G > cus || G > 64 * 4 || rounds < 1 || rounds > 4096 || !stamps_host)
    return fail(MARKOV_E_UNSUPPORTED, "exchange probe: G=%d (at most %d and 256), rounds=%d", G, cus, rounds);
  const size_t sb = (size_t)rounds * G * 8, pb = (size_t)rounds * kPartCopies * kPartStride * 8,
               tb = (size_t)rounds * G * 16;
  void *slots = nullptr, *part = nullptr, *stamps = nullptr;
  e = hipMalloc(&slots, sb);
  if (e == hipSuccess) e = hipMalloc(&part, pb);
  if (e == hipSuccess) e = hipMalloc(&stamps, tb);
  if (e == hipSuccess) e = hipMemset(slots, 0, sb);
  if (e == hipSuccess) e = hipMemset(part, 0, pb);
  if (e == hipSuccess) e = hipMemset(stamps, 0, tb);
  if (e == hipSuccess) {
    uint64_t* a0 = (uint64_t*)slots;
    uint64_t* a1 = (uint64_t*)part;
    uint64_t* a2 = (uint64_t*)stamps;
    uint64_t wt = g_wait_ticks.load();
    void* args[] = {&a0, &a1, &a2, &G, &rounds, &two_level, &wt};
    e = hipLaunchKernel((const void*)exchange_probe_kernel, dim3(G), dim3(kThreads), args, 0, nullptr);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(stamps_host, stamps, tb, hipMemcpyDeviceToHost);
  hipFree(slots);
  hipFree(part);
  hipFree(stamps);
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "exchange probe: %s", hipGetErrorString(e));
  return MARKOV_OK;
}

// Trace builds only (not part of the ABI in markov.h): copies the first
// `bytes` of trace_buf ([1024 workgroups][32 steps][12 phases] u64 ticks of
// the 100 MHz clock) to host memory and clears it.  Synchronising.
int markov_trace_read(void* dst, size_t bytes) {
  const size_t all = sizeof(unsigned long long) * kTraceWGs * kTraceSteps * kTracePhases;
  if (bytes > all) bytes = all;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(trace_buf), bytes, 0, hipMemcpyDeviceToHost);
  void* ptr = nullptr;
  if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(trace_buf));
  if (e == hipSuccess) e = hipMemset(ptr, 0, all);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(MARKOV_E_HIP, "trace read: %s", hipGetErrorString(e));
  return MARKOV_OK;
}
#endif

long long markov_set_wait_limit(long long us) {
  const unsigned long long t = us < 0 ? kTimeoutTicks : (unsigned long long)us * kTicksPerUs;
  return (long long)(g_wait_ticks.exchange(t) / kTicksPerUs);
}

int markov_grid(int rows, int steps, int vocab, int rank, int mode) {
  g_last_error.clear();
  mode &= ~kModeFlags;
  Shape sh;
  int rc = check_shape(rows, steps, vocab, rank, mode, &sh);
  if (rc != MARKOV_OK) return rc;
  int G = 0;
  bool res = false;
  rc = pick_grid(rows < kLaunchRows ? rows : kLaunchRows, rank, mode, sh, &G, &res);
  return rc != MARKOV_OK ? rc : G;
}

}  // extern "C"
