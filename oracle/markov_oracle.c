/*
 * markov_oracle.c -- plain, slow, single-threaded CPU oracle of the DSpark
 * sequential Markov draft-sampling chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant generator with the HIP library: every formula below is written out
 * again from the pages' definitions, in the most direct form available.
 *
 * Source pages (cited by title and section):
 *   [SM]  vLLM API page "vllm.models.deepseek_v41.nvidia.specialized_decode.
 *         sampling.sharded_markov": module docstring (the per-call diagram and
 *         the sampling contract) and the class DSparkShardedMarkovSampler.
 *   [FM]  vLLM API page "vllm.models.deepseek_v41.nvidia.ops.fused_markov":
 *         module docstring (inverse-CDF sampling, temperature 0 is argmax).
 *   [MS]  vLLM API page "vllm.models.muse_spark.nvidia.specialized_decode.
 *         runtime.markov": module docstring (NaN and tie rule),
 *         FusedMarkovParams and fused_markov_params (output-logit transform).
 *
 * Precision: the bias dot product is summed exactly in fp64 (every product of
 * two bf16 values is exact in fp64) and rounded once to bf16.  Everything the
 * pages fix to fp32 (logit add, transform, temperature division, Gumbel noise)
 * is done in fp32 with IEEE round-to-nearest-even; the inverse CDF is built in
 * fp64.
 *
 * Parity unpinned: only the exact bit pattern of fp32 tanhf (host libm here,
 * the device library on the GPU; both are within a few fp32 ulps, which the
 * bf16 cache rounding hides except next to a rounding boundary).  The fp32
 * logarithms are pinned to a 50-digit decimal logarithm correctly rounded to
 * fp32; everything else has a pin in the tests too.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bfloat16: the upper 16 bits of an IEEE binary32 value.                    */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a real value (given exactly as a double) to the nearest bfloat16,
 * ties to even, in one step.  NaN becomes the quiet NaN 0x7FC0; values that
 * round beyond the largest finite bf16 become infinity. */
uint16_t orc_bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int e;
  frexp(a, &e);          /* a lies in [2^(e-1), 2^e) */
  int lead = e - 1;      /* exponent of the leading bit */
  if (lead < -126) lead = -126; /* subnormal bf16: the spacing stays 2^-133 */
  double spacing = ldexp(1.0, lead - 7); /* 7 stored fraction bits */
  double n = nearbyint(a / spacing);     /* a/spacing is exact; ties to even */
  double r = n * spacing;
  if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

void orc_bf16_round_f32_array(const float* in, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = orc_bf16_round((double)in[i]);
}

/* ------------------------------------------------------------------------ */
/* Counter-based noise.  [SM] (module docstring, per-call diagram): the      */
/* Gumbel noise of each (row, position, vocab id) depends on the seeds and   */
/* positions only, never on the chain, and is keyed by the global vocab id.  */
/* The generator is SplitMix64 (Steele, Lea and Flood, "Fast splittable      */
/* pseudorandom number generators", OOPSLA 2014): one output is the          */
/* finaliser applied to the state advanced by the golden-ratio increment.    */
/* ------------------------------------------------------------------------ */

uint64_t orc_splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* One SplitMix64 output for state x (x advanced once, then finalised). */
uint64_t orc_splitmix64(uint64_t x) {
  return orc_splitmix64_mix(x + 0x9E3779B97F4A7C15ULL);
}

/* The (seed, row, step) prefix.  The seed is hashed first, then each
 * counter is absorbed in turn as h <- splitmix64(h XOR counter), so that
 * distinct (seed, row) pairs do not meet in a plain XOR of the counters. */
uint64_t orc_hash_step(int64_t seed, int64_t row, int64_t step) {
  uint64_t h = orc_splitmix64((uint64_t)seed);
  h = orc_splitmix64(h ^ (uint64_t)row);
  return orc_splitmix64(h ^ (uint64_t)step);
}

/* The full (seed, row, step, v) hash with v the global vocab id. */
uint64_t orc_hash_vocab(uint64_t prefix, int64_t v) {
  return orc_splitmix64(prefix ^ (uint64_t)v);
}

/* The top 23 bits of h as the odd multiple (2k+1) * 2^-24: exact in fp32 and
 * strictly inside (0, 1). */
float orc_uniform(uint64_t h) {
  uint64_t k = h >> 41;
  return (float)(2 * k + 1) * 0x1p-24f;
}

/* Standard Gumbel draw -log(-log u) in fp32, as the pages' fp32 noise.
 * Each fp32 logarithm is the correctly rounded one: the natural log of the
 * fp32 argument taken in fp64 and rounded once to fp32 (libm logf is only
 * faithfully rounded, so two libms would disagree in the last bit). */
float orc_log_f32(float x) { return (float)log((double)x); }
float orc_gumbel(float u) { return -orc_log_f32(-orc_log_f32(u)); }

/* gumbel[row][step][v] for rows x steps x V (contiguous). */
void orc_noise_fill(float* gumbel, const int64_t* seeds, int rows, int steps,
                    int V) {
  for (int row = 0; row < rows; ++row)
    for (int i = 0; i < steps; ++i) {
      uint64_t prefix = orc_hash_step(seeds[row], row, i);
      float* out = gumbel + ((size_t)row * steps + i) * (size_t)V;
      for (int v = 0; v < V; ++v)
        out[v] = orc_gumbel(orc_uniform(orc_hash_vocab(prefix, v)));
    }
}

/* Uniforms of a contiguous range of vocab ids (for the statistical pins). */
void orc_uniform_range(float* out, int64_t seed, int64_t row, int64_t step,
                       int64_t v0, int64_t count) {
  uint64_t prefix = orc_hash_step(seed, row, step);
  for (int64_t j = 0; j < count; ++j)
    out[j] = orc_uniform(orc_hash_vocab(prefix, v0 + j));
}

/* ------------------------------------------------------------------------ */
/* One draft position of one request row.                                    */
/* ------------------------------------------------------------------------ */

/* diag (optional, 8 doubles):
 *   mode 0 / argmax: [0] best score, [1] best score among the other ids,
 *                    [2] that runner-up's id, [3] 1 if a NaN decided.
 *   mode 1:          [0] u*S, [1] S, [2] distance from u*S to the nearer
 *                    edge of the chosen bin divided by S, [3] 1 if a NaN or
 *                    an infinite maximum decided, [4] the id across that
 *                    nearer edge (-1 if none). */
enum { ORC_DIAG = 8 };

/* The lowest id of a NaN score if any, else the lowest id of the maximum
 * ([MS] module docstring; [SM] docstring: torch.argmax tie order).  +0 and
 * -0 compare equal, so the lower id wins between them. */
static int64_t orc_pick_max(const float* s, int V, double* diag) {
  int64_t best = -1, nan_at = -1;
  for (int v = 0; v < V; ++v) {
    if (isnan(s[v])) { nan_at = v; break; }
    if (best < 0 || s[v] > s[best]) best = v;
  }
  int64_t win = nan_at >= 0 ? nan_at : best;
  if (diag) {
    double second = -INFINITY;
    int64_t second_at = -1;
    for (int v = 0; v < V; ++v) {
      if (v == win || isnan(s[v])) continue;
      if (second_at < 0 || s[v] > second) { second = s[v]; second_at = v; }
    }
    diag[0] = s[win];
    diag[1] = second;
    diag[2] = (double)second_at;
    diag[3] = nan_at >= 0 ? 1.0 : 0.0;
  }
  return win;
}

/*
 * orc_step: the logits of one position given the previous token, their
 * rounding into the draft-logits cache, and the draw.
 *
 *   bias[v]  = bf16( sum_k head[v][k] * embed[prev][k] )      [SM] docstring
 *   x        = f32(base[v]) + f32(bias[v])                     ("cache_round(
 *   x        = x * mult ; if cap > 0: x = tanhf(x * inv_cap) * cap   base + bias)")
 *   cache[v] = bf16(x)                                         [MS] FusedMarkovParams
 *   mode 0:  s[v] = f32(cache[v]) / T + gumbel[v]  (T > 0), s = cache (T <= 0);
 *            token = lowest NaN id, else lowest id of max s    [SM], [MS]
 *   mode 1:  inverse CDF of softmax(cache / T) at u            [FM] docstring
 *
 * gumbel may be NULL in mode 1 (unused).  bias_out (optional, [V]) receives
 * the bf16 bias for diagnostics.  Returns the token.
 *
 * Element types ([SM] DSparkShardedMarkovSampler and _kernel: base logits
 * and the draft-logits cache are each bf16 or fp32; cache_round rounds to
 * the cache's type): base is bf16 bits, or fp32 values when base_f32;
 * cache is bf16 bits, or fp32 values when cache_f32, in which case the
 * cache value is x itself.
 */
int64_t orc_step_t(const void* base, int base_f32, const uint16_t* head,
                   const uint16_t* embed, int V, int r, int64_t prev, float T,
                   const float* gumbel, float u, float mult, float cap, int mode,
                   void* cache, int cache_f32, double* diag, uint16_t* bias_out) {
  double* e = (double*)malloc(sizeof(double) * (size_t)r);
  float* s = (float*)malloc(sizeof(float) * (size_t)V);
  for (int k = 0; k < r; ++k)
    e[k] = (double)orc_bf16_to_f32(embed[(size_t)prev * r + k]);
  float inv_cap = cap > 0.0f ? 1.0f / cap : 1.0f;

  for (int v = 0; v < V; ++v) {
    double dot = 0.0;
    const uint16_t* hv = head + (size_t)v * r;
    for (int k = 0; k < r; ++k) dot += (double)orc_bf16_to_f32(hv[k]) * e[k];
    uint16_t bias_bits = orc_bf16_round(dot);
    if (bias_out) bias_out[v] = bias_bits; /* diagnostic copy of the bias */
    float bias = orc_bf16_to_f32(bias_bits);
    float b = base_f32 ? ((const float*)base)[v] : orc_bf16_to_f32(((const uint16_t*)base)[v]);
    float x = b + bias;
    x = x * mult;
    if (cap > 0.0f) x = tanhf(x * inv_cap) * cap;
    float cf;
    if (cache_f32) {
      ((float*)cache)[v] = x;
      cf = x;
    } else {
      uint16_t c = orc_bf16_round((double)x);
      ((uint16_t*)cache)[v] = c;
      cf = orc_bf16_to_f32(c);
    }
    if (T > 0.0f) {
      s[v] = (mode == 0) ? cf / T + gumbel[v] : cf / T;
    } else {
      s[v] = cf;
    }
  }

  int64_t win;
  if (mode == 0 || !(T > 0.0f)) {
    win = orc_pick_max(s, V, diag);
  } else {
    /* Inverse CDF of softmax(z), z = cache / T, in vocab order: the
     * smallest k whose cumulative weight exceeds u times the total. */
    int64_t nan_at = -1;
    float M = -INFINITY;
    for (int v = 0; v < V; ++v) {
      if (isnan(s[v])) { nan_at = v; break; }
      if (s[v] > M) M = s[v];
    }
    if (nan_at >= 0 || isinf(M)) {
      /* A NaN, an infinite maximum, or all -inf: the argmax rule decides. */
      win = orc_pick_max(s, V, NULL);
      if (diag) {
        memset(diag, 0, sizeof(double) * ORC_DIAG);
        diag[3] = 1.0;
        diag[4] = -1.0;
      }
    } else {
      double* cdf = (double*)malloc(sizeof(double) * (size_t)V);
      double acc = 0.0;
      for (int v = 0; v < V; ++v) {
        acc += exp((double)s[v] - (double)M);
        cdf[v] = acc;
      }
      double S = cdf[V - 1];
      double t = (double)u * S;
      win = -1;
      for (int v = 0; v < V; ++v)
        if (cdf[v] > t) { win = v; break; }
      /* No bin exceeds t only if u = 1 (the hash's u is at most 1 - 2^-24,
       * which keeps t below S by far more than an fp64 rounding): the last
       * id with weight. */
      if (win < 0) {
        for (int v = V - 1; v >= 0; --v)
          if (cdf[v] > (v > 0 ? cdf[v - 1] : 0.0)) { win = v; break; }
        if (win < 0) win = V - 1;
      }
      if (diag) {
        double lo = win > 0 ? cdf[win - 1] : 0.0;
        double hi = cdf[win];
        double dlo = t - lo, dhi = hi - t;
        memset(diag, 0, sizeof(double) * ORC_DIAG);
        diag[0] = t;
        diag[1] = S;
        if (dlo <= dhi) {
          diag[2] = dlo / S;
          diag[4] = win > 0 ? (double)(win - 1) : -1.0;
        } else {
          diag[2] = dhi / S;
          diag[4] = win + 1 < V ? (double)(win + 1) : -1.0;
        }
      }
      free(cdf);
    }
  }
  free(s);
  free(e);
  return win;
}

/* orc_step with bf16 base logits and a bf16 cache. */
int64_t orc_step(const uint16_t* base, const uint16_t* head,
                 const uint16_t* embed, int V, int r, int64_t prev, float T,
                 const float* gumbel, float u, float mult, float cap, int mode,
                 uint16_t* cache, double* diag, uint16_t* bias_out) {
  return orc_step_t(base, 0, head, embed, V, r, prev, T, gumbel, u, mult, cap,
                    mode, cache, 0, diag, bias_out);
}

/* ------------------------------------------------------------------------ */
/* The chain: N positions in order, each draw the next position's previous   */
/* token ([SM] module docstring, "winner p = draft_tokens[i]").              */
/* ------------------------------------------------------------------------ */

/*
 * base[row*base_rs + i*base_ss + v] (bf16), head/embed [V][r] (bf16),
 * prev_tokens[rows], temperature[rows] (fp32), seeds[rows],
 * gumbel[rows][N][V] or NULL (then drawn here from seeds with the hash
 * above), state_idx[rows] or NULL (identity); a negative state makes the row
 * inert (no reads, no writes).  mult = 1 and cap = 0 mean no transform.
 * row_mask[rows] or NULL selects the rows to compute (the others are left
 * untouched), which lets a test sample rows of a large call.
 * tokens[row*N + i]; cache[state*cache_rs + i*cache_ss + v].  base and
 * cache are bf16 bits, or fp32 with base_f32 / cache_f32 (see orc_step_t).
 * Returns 0, or -1 if a computed row has a previous token outside [0, V).
 */
int orc_chain_t(const void* base, int base_f32, int64_t base_rs, int64_t base_ss,
                const uint16_t* head, const uint16_t* embed, int V, int r,
                const int64_t* prev_tokens, const float* temperature,
                const int64_t* seeds, const float* gumbel,
                const int64_t* state_idx, float mult, float cap, int rows,
                int N, int mode, const uint8_t* row_mask, int64_t* tokens,
                void* cache, int cache_f32, int64_t cache_rs, int64_t cache_ss) {
  const size_t bsz = base_f32 ? 4 : 2, csz = cache_f32 ? 4 : 2;
  float* g = (float*)malloc(sizeof(float) * (size_t)V);
  int status = 0;
  for (int row = 0; row < rows; ++row) {
    if (row_mask && !row_mask[row]) continue;
    int64_t state = state_idx ? state_idx[row] : row;
    if (state < 0) continue;
    int64_t p = prev_tokens[row];
    if (p < 0 || p >= V) { status = -1; continue; }
    for (int i = 0; i < N; ++i) {
      const float* gi = NULL;
      float u = 0.0f;
      if (mode == 0) {
        if (gumbel) {
          gi = gumbel + ((size_t)row * N + i) * (size_t)V;
        } else {
          uint64_t prefix = orc_hash_step(seeds[row], row, i);
          for (int v = 0; v < V; ++v)
            g[v] = orc_gumbel(orc_uniform(orc_hash_vocab(prefix, v)));
          gi = g;
        }
      } else {
        u = orc_uniform(orc_hash_step(seeds[row], row, i));
      }
      p = orc_step_t((const char*)base + (size_t)(row * base_rs + i * base_ss) * bsz, base_f32,
                     head, embed, V, r, p, temperature[row], gi, u, mult, cap, mode,
                     (char*)cache + (size_t)(state * cache_rs + i * cache_ss) * csz, cache_f32,
                     NULL, NULL);
      tokens[(size_t)row * N + i] = p;
    }
  }
  free(g);
  return status;
}

/* orc_chain with bf16 base logits and a bf16 cache. */
int orc_chain(const uint16_t* base, int64_t base_rs, int64_t base_ss,
              const uint16_t* head, const uint16_t* embed, int V, int r,
              const int64_t* prev_tokens, const float* temperature,
              const int64_t* seeds, const float* gumbel,
              const int64_t* state_idx, float mult, float cap, int rows,
              int N, int mode, const uint8_t* row_mask, int64_t* tokens,
              uint16_t* cache, int64_t cache_rs, int64_t cache_ss) {
  return orc_chain_t(base, 0, base_rs, base_ss, head, embed, V, r, prev_tokens,
                     temperature, seeds, gumbel, state_idx, mult, cap, rows, N,
                     mode, row_mask, tokens, cache, 0, cache_rs, cache_ss);
}
