/* Runs every entry point of the CPU oracle on small inputs, for a build with
 * -fsanitize=address,undefined (tests/test_oracle_sanitize_cpu.py): out of
 * bounds accesses, leaks and undefined behaviour abort the run.  The inputs
 * come from a small linear congruential generator (test data only).  Prints
 * a checksum of the outputs. */
#include "../oracle/markov_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 0x2545F4914F6CDD1DULL;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (uint32_t)(lcg_state >> 33);
}
static float unif(float lo, float hi) { return lo + (hi - lo) * (float)(lcg() & 0xFFFFFF) / 16777216.0f; }

int main(void) {
  enum { V = 1040, R = 32, ROWS = 3, N = 4 };
  uint16_t* head = malloc(sizeof(uint16_t) * V * R);
  uint16_t* embed = malloc(sizeof(uint16_t) * V * R);
  uint16_t* base = malloc(sizeof(uint16_t) * ROWS * N * V);
  float* basef = malloc(sizeof(float) * ROWS * N * V);
  float* gumbel = malloc(sizeof(float) * ROWS * N * V);
  for (int k = 0; k < V * R; ++k) {
    head[k] = orc_bf16_round((double)unif(-0.1f, 0.1f));
    embed[k] = orc_bf16_round((double)unif(-0.1f, 0.1f));
  }
  for (int k = 0; k < ROWS * N * V; ++k) {
    basef[k] = unif(-4.0f, 4.0f);
    base[k] = orc_bf16_round((double)basef[k]);
  }
  base[5] = 0x7FC0;                   /* a NaN logit */
  base[V + 7] = base[V + 9] = 0x4220; /* an exact tie (40.0) */
  int64_t prev[ROWS] = {1, 1039, 500};
  float temp[ROWS] = {1.0f, 0.0f, 0.7f};
  int64_t seeds[ROWS] = {-5, 0, 123456789};
  int64_t sidx[ROWS] = {1, -1, 0};
  uint8_t mask[ROWS] = {1, 1, 1};
  orc_noise_fill(gumbel, seeds, ROWS, N, V);
  float us[64];
  orc_uniform_range(us, 7, 1, 2, 3, 64);
  double check = 0.0;
  for (int mode = 0; mode < 2; ++mode)
    for (int f = 0; f < 4; ++f) {
      const int base_f32 = f & 1, cache_f32 = f >> 1;
      int64_t tokens[ROWS * N];
      void* cache = calloc((size_t)ROWS * N * V, cache_f32 ? 4 : 2);
      int rc = orc_chain_t(base_f32 ? (const void*)basef : (const void*)base, base_f32, (int64_t)N * V, V, head,
                           embed, V, R, prev, temp, seeds, mode == 0 ? gumbel : NULL, sidx, 0.5f,
                           mode == 0 ? 30.0f : 0.0f, ROWS, N, mode, mask, tokens, cache, cache_f32,
                           (int64_t)N * V, V);
      if (rc != 0) return 2;
      for (int k = 0; k < ROWS * N; ++k) check += (double)tokens[k] * (k + 1);
      free(cache);
    }
  /* the chain drawing its own noise, and one step with diagnostics */
  int64_t tokens[ROWS * N];
  uint16_t* cache = calloc((size_t)ROWS * N * V, 2);
  if (orc_chain(base, (int64_t)N * V, V, head, embed, V, R, prev, temp, seeds, NULL, NULL, 1.0f, 0.0f, ROWS, N, 0,
                NULL, tokens, cache, (int64_t)N * V, V) != 0)
    return 3;
  double diag[ORC_DIAG];
  uint16_t bias[V];
  for (int mode = 0; mode < 2; ++mode) {
    int64_t t = orc_step(base, head, embed, V, R, 3, 0.9f, gumbel, 0.999f, 1.0f, 0.0f, mode, cache, diag, bias);
    check += (double)t + (isfinite(diag[0]) ? diag[0] : 1.0) + (isfinite(diag[2]) ? diag[2] : 1.0);
  }
  /* a previous token outside [0, V) is reported */
  int64_t bad[ROWS] = {V, 0, 0};
  if (orc_chain(base, (int64_t)N * V, V, head, embed, V, R, bad, temp, seeds, gumbel, NULL, 1.0f, 0.0f, ROWS, N, 0,
                NULL, tokens, cache, (int64_t)N * V, V) != -1)
    return 4;
  check += orc_log_f32(3.0f) + orc_gumbel(0.25f) + (double)orc_hash_vocab(orc_hash_step(-1, 2, 3), 4);
  printf("ok %.6g\n", check);
  free(head);
  free(embed);
  free(base);
  free(basef);
  free(gumbel);
  free(cache);
  return 0;
}
