/*
 * markov.h -- C ABI of libmarkov, the MI355X (gfx950) DSpark sequential
 * Markov draft-sampling chain.
 *
 * The method (vLLM API page "vllm.models.deepseek_v41.nvidia.specialized_
 * decode.sampling.sharded_markov", module docstring and its per-call
 * diagram): the draft backbone first yields base logits for all N draft
 * positions; the tokens then follow sequentially.  For position i the
 * low-rank transition bias bf16(markov_head[V, r] . markov_embed[previous
 * token]) is added to that position's base logits, the sum is rounded into a
 * bf16 draft-logits cache, and a token is sampled from it, which in turn is
 * the previous token of position i + 1.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device pointers owned by the caller; the
 *    library never allocates, frees or retains device memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Calls only enqueue work on it and never synchronise the host (except
 *    markov_status), so they can be captured in a HIP graph.
 *  - bf16 tensors are passed as uint16_t bit patterns.  Strides are counted in
 *    elements.
 *  - Every call returns a markov_status_t.  On an error nothing is enqueued
 *    and markov_last_error() gives the reason (a thread-local string).
 */
#ifndef LIBMARKOV_MARKOV_H
#define LIBMARKOV_MARKOV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MARKOV_OK = 0,
  MARKOV_E_INVAL = -1,       /* a null pointer, bad size, stride or alignment */
  MARKOV_E_UNSUPPORTED = -2, /* a shape the kernels do not take (reason given) */
  MARKOV_E_HIP = -3,         /* a HIP runtime call failed (reason given) */
  MARKOV_E_DEVICE = -4       /* markov_status: the kernel set an error bit */
} markov_status_t;

/* Sampling modes. */
#define MARKOV_MODE_GUMBEL 0 /* max of logit / T + gumbel (sharded_markov page) */
#define MARKOV_MODE_INVCDF 1 /* inverse CDF of softmax(logit / T) (fused_markov page) */

/* Element types, OR-ed into `mode` (sharded_markov page, _kernel and
 * unsupported_reason: base logits and the draft-logits cache are each bf16 or
 * fp32).  Without a flag the tensor is bf16. */
#define MARKOV_BASE_F32 0x10  /* base_logits are fp32 */
#define MARKOV_CACHE_F32 0x20 /* the cache is fp32: cache_round keeps x unrounded */

/* Noise placement, OR-ed into MARKOV_MODE_GUMBEL (sharded_markov page,
 * fork_noise; fused_markov page, module docstring: Gumbel-max costs a hash
 * and two logs per logit).  With MARKOV_NOISE_INLINE the chain's kernels
 * (the persistent chain kernel and the step kernels) draw gumbel[b][i][v]
 * themselves, from seeds, bit-identical to what
 * markov_noise_fill writes; `gumbel` is then not read and may be NULL, and
 * `seeds` is required.  Without it the noise is read from `gumbel`. */
#define MARKOV_NOISE_INLINE 0x40

/* Limits of the library. */
#define MARKOV_MAX_ROWS 4096 /* one persistent launch takes 64; more run per position */
#define MARKOV_MAX_STEPS 256
#define MARKOV_MAX_VOCAB (1 << 24)

/* Device error bits reported by markov_status. */
#define MARKOV_DEVERR_BAD_TOKEN 1u /* a previous token outside [0, V): row made inert */
#define MARKOV_DEVERR_TIMEOUT 2u   /* a cross-workgroup wait exceeded its bound */
#define MARKOV_DEVERR_BAD_STATE 4u /* a state index >= cache_states: row made inert */

/*
 * markov_workspace_bytes: bytes of device workspace markov_chain_sample needs
 * for this call shape (rows request rows, `steps` positions, vocabulary
 * `vocab`, rank dim `rank`, sampling `mode`).  Returns 0 for an unsupported
 * shape.  Host only.
 *
 * The pages keep the chain's exchange state in persistent buffers allocated
 * once, before any graph capture, so that graphs keep their addresses
 * (sharded_markov page, DSparkShardedMarkovSampler: the zeroed mailbox and
 * staging buffer; muse_spark markov page, MarkovSampler.__init__: the per-call
 * buffers and the per-row arrival counters, zeroed per call).  Here that
 * state is this caller-owned workspace.
 *
 * The workspace holds the per-position exchange slots of the workgroups (two
 * halves used by alternate calls) and a small header (call parity, error
 * word).  The caller allocates it, zeroes it ONCE, and passes the same
 * pointer and the same workspace_bytes to every later call; the kernel
 * leaves it ready for the next call, so graph replays need no memset.  One
 * workspace serves one call at a time: calls that overlap in time (e.g. on
 * two streams) must use different workspaces.  A workspace may serve
 * several call shapes: size it as the largest markov_workspace_bytes of
 * those shapes.
 */
size_t markov_workspace_bytes(int rows, int steps, int vocab, int rank, int mode);

/*
 * markov_noise_fill: the chain's Gumbel noise, gumbel[row][i][v] =
 * -log(-log(u)) in fp32, u the uniform of a counter-based hash of
 * (seeds[row], row, i, v) with v the global vocabulary id.
 *
 * sharded_markov page, module docstring and fork_noise: the noise depends
 * on the seeds and positions only, never on the chain, so it is drawn on a
 * side stream while the draft LM head runs.  The hash is SplitMix64 (Steele,
 * Lea and Flood, OOPSLA 2014): h = sm(seed); h = sm(h ^ row); h = sm(h ^ i);
 * h = sm(h ^ v), where sm(x) is one SplitMix64 output for state x; the top
 * 23 bits k of h give u = (2k + 1) * 2^-24.
 *
 *   gumbel  device, fp32 [rows][steps][vocab], contiguous, 16-byte aligned,
 *           written.
 *   seeds   device, int64 [rows]; the int64 bits are used as uint64.
 *   rows in [1, MARKOV_MAX_ROWS], steps in [1, MARKOV_MAX_STEPS], vocab a
 *   positive multiple of 16 up to MARKOV_MAX_VOCAB.
 */
int markov_noise_fill(float* gumbel, const int64_t* seeds, int rows, int steps,
                      int vocab, void* stream);

/*
 * markov_chain_sample: the whole N-position chain for `rows` request rows.
 * Up to 64 rows run in one persistent launch (sharded_markov page, module
 * docstring: one kernel runs the whole chain and keeps the head in
 * registers, so it is read once).  Larger batches run per position over all
 * rows (fused_markov page, FusedMarkovSampler: the fused loop that serves
 * batches beyond the chain's rows): MARKOV_MODE_GUMBEL runs one persistent
 * step kernel for all positions (one workgroup per chunk of 8 * 16384 / rank
 * vocabulary ids, when they fit on the compute units at once and the
 * workspace holds its layout; otherwise one step kernel launch per
 * position), with the noise read from memory or, with MARKOV_NOISE_INLINE,
 * drawn by the step kernel itself (the same values); MARKOV_MODE_INVCDF runs
 * a step kernel and a pick kernel per position.  The per-position launches
 * never wait for one another's workgroups; the persistent kernels (chain and
 * step kernel) are subject to the co-residency condition below.
 *
 * Launch and co-residency: the launch is a regular one (not a cooperative
 * launch) of at most one 512-thread workgroup per compute unit, and the
 * kernel's registers admit only one workgroup per compute unit.  Its
 * workgroups wait for one another at every position, so they must all be
 * resident at once: THE CALLER MUST NOT RUN OTHER KERNELS CONCURRENTLY ON THE
 * SAME DEVICE (on other streams, or other processes) that could keep compute
 * units from the chain.  Nothing at launch time checks this.  Every
 * cross-workgroup wait is bounded instead (sharded_markov page,
 * DSparkShardedMarkovSampler: timeout_ms bounds every cross-rank wait), by 2 s
 * unless markov_set_wait_limit says otherwise; a wait that gives up sets
 * MARKOV_DEVERR_TIMEOUT, the call then writes unspecified tokens (possibly
 * none) and cache values, and THE WORKSPACE MUST BE ZEROED AGAIN before its
 * next use.  markov_status reports the condition.
 *
 * For each row b with state s = state_idx[b] >= 0, starting from
 * p = prev_tokens[b], for i = 0 .. steps-1 in order
 * (sharded_markov page, module docstring and per-call diagram;
 *  muse_spark markov page, FusedMarkovParams and fused_markov_params):
 *   bias[v]  = bf16( sum_k head[v][k] * embed[p][k] ), fp32 accumulation
 *   x[v]     = f32(base[b][i][v]) + f32(bias[v])
 *   x[v]     = x[v] * output_multiplier;
 *              if soft_cap > 0: x[v] = tanhf(x[v] * (1 / soft_cap)) * soft_cap
 *   cache[s][i][v] = c[v] = bf16(x[v])  (round to nearest even; c = x with
 *            MARKOV_CACHE_F32)
 *   MARKOV_MODE_GUMBEL: score[v] = f32(c[v]) / T[b] + gumbel[b][i][v] if
 *            T[b] > 0, else f32(c[v]); the token is the lowest v whose score
 *            is NaN if any, else the lowest v of the maximum score.
 *   MARKOV_MODE_INVCDF (fused_markov page, module docstring): with T[b] > 0,
 *            the token is drawn by inverse CDF of softmax(f32(c) / T[b]) in
 *            vocabulary order at u = uniform(hash(seeds[b], b, i)) (the hash
 *            above without the vocabulary id); NaN and +inf maxima and
 *            T[b] <= 0 fall back to the argmax rule above.
 *   draft_tokens[b][i] = token; p = token.
 * Rows with state_idx[b] < 0 are padding: nothing of theirs is read or
 * written (muse_spark/sharded_markov pages: padding rows are inert).
 *
 *   base_logits     device, bf16 (fp32 with MARKOV_BASE_F32)
 *                   [rows][steps][>= vocab] with row stride
 *                   base_row_stride and step stride base_step_stride
 *                   (elements, multiples of 8), 16-byte aligned, read.
 *   head, embed     device, bf16 [>= vocab][rank], contiguous, 16-byte
 *                   aligned, read.  head is the Markov w2 (the bias head),
 *                   embed the Markov w1 (the embedding of the previous token).
 *   prev_tokens     device, int64 [rows]: each row's anchor token.  A value
 *                   outside [0, vocab) sets MARKOV_DEVERR_BAD_TOKEN and makes
 *                   the row inert.
 *   temperature     device, fp32 [rows].
 *   seeds           device, int64 [rows]; read in MARKOV_MODE_INVCDF and
 *                   with MARKOV_NOISE_INLINE (may be NULL otherwise).
 *   gumbel          device, fp32 [rows][steps][vocab] contiguous, as
 *                   markov_noise_fill writes it; read in MARKOV_MODE_GUMBEL
 *                   without MARKOV_NOISE_INLINE only (may be NULL otherwise).
 *   state_idx       device, int64 [rows], or NULL for the identity; negative
 *                   marks a padding row.  Distinct non-negative entries.
 *   output_multiplier  fp32 multiplier (1.0f: none); finite.
 *   soft_cap        fp32 soft cap (0: none); finite, >= 0.
 *   rows in [1, MARKOV_MAX_ROWS] (more than 64 rows run as described above,
 *   in order on `stream`; row indices in the mode-1 hash and the identity
 *   state map stay the call's); steps in [1, MARKOV_MAX_STEPS]; vocab a
 *   positive multiple of 16 up to MARKOV_MAX_VOCAB; rank 256 or 512;
 *   mode MARKOV_MODE_GUMBEL or MARKOV_MODE_INVCDF, with the element-type
 *   flags above and, for MARKOV_MODE_GUMBEL, MARKOV_NOISE_INLINE
 *   (markov_workspace_bytes and markov_grid ignore the flags).
 *   draft_tokens    device, int64 [rows][>= steps], row stride
 *                   tokens_row_stride, written for non-padding rows.
 *   cache           device, bf16 (fp32 with MARKOV_CACHE_F32)
 *                   [cache_states][steps][>= vocab] with state
 *                   stride cache_state_stride and step stride
 *                   cache_step_stride (multiples of 8), 16-byte aligned,
 *                   written at cache[state_idx[b]][i][0 .. vocab).  A state
 *                   index >= cache_states sets MARKOV_DEVERR_BAD_STATE and
 *                   makes the row inert; without state_idx, cache_states must
 *                   be >= rows.
 *   workspace       device, markov_workspace_bytes(...) bytes or more,
 *                   256-byte aligned, zeroed once before the first call.
 *
 * Errors: MARKOV_E_INVAL / MARKOV_E_UNSUPPORTED for bad arguments (checked on
 * the host before anything is enqueued), MARKOV_E_HIP if a HIP query or the
 * launch itself fails.  Device-side conditions (bad anchor token or state
 * index, a wait that gave up) are reported by markov_status.
 */
int markov_chain_sample(const void* base_logits, int64_t base_row_stride,
                        int64_t base_step_stride, const uint16_t* head,
                        const uint16_t* embed, const int64_t* prev_tokens,
                        const float* temperature, const int64_t* seeds,
                        const float* gumbel, const int64_t* state_idx,
                        float output_multiplier, float soft_cap, int rows,
                        int steps, int vocab, int rank, int mode,
                        int64_t* draft_tokens, int64_t tokens_row_stride,
                        void* cache, int64_t cache_states,
                        int64_t cache_state_stride, int64_t cache_step_stride,
                        void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * markov_chain_sample_noalloc: markov_chain_sample without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture
 * that may not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation.  It takes the same arguments but workspace and
 * workspace_bytes, runs the same kernels and writes the same outputs; the
 * call allocates and frees nothing.  The chain's exchange state lives in a
 * static device array of MARKOV_NOALLOC_MAX_BYTES bytes inside the library,
 * one per device it runs on, held until the process ends.
 *
 * Limits and sharing:
 *  - a call shape whose markov_workspace_bytes exceeds
 *    MARKOV_NOALLOC_MAX_BYTES is refused with MARKOV_E_UNSUPPORTED;
 *  - every call on one device uses that device's one array, which keeps the
 *    last call's state: calls that overlap in time on one device (other
 *    streams or threads without ordering) race and give wrong results;
 *  - the first call on a device also enqueues on `stream` a one-time kernel
 *    that zeroes the array (made outside graph capture, it stays out of any
 *    graph);
 *  - device errors are read with markov_status(NULL, stream); after
 *    MARKOV_DEVERR_TIMEOUT that call zeroes the array again itself.
 */
#define MARKOV_NOALLOC_MAX_BYTES ((size_t)8 << 20)
int markov_chain_sample_noalloc(const void* base_logits, int64_t base_row_stride,
                                int64_t base_step_stride, const uint16_t* head,
                                const uint16_t* embed, const int64_t* prev_tokens,
                                const float* temperature, const int64_t* seeds,
                                const float* gumbel, const int64_t* state_idx,
                                float output_multiplier, float soft_cap, int rows,
                                int steps, int vocab, int rank, int mode,
                                int64_t* draft_tokens, int64_t tokens_row_stride,
                                void* cache, int64_t cache_states,
                                int64_t cache_state_stride,
                                int64_t cache_step_stride, void* stream);

/*
 * markov_status: synchronises `stream`, then reads and clears the device
 * error word of `workspace` (sharded_markov page, DSparkShardedMarkovSampler:
 * cross-workgroup waits are bounded and report instead of hanging).
 * Returns MARKOV_OK, or MARKOV_E_DEVICE with the error bits described by
 * markov_last_error().  After a MARKOV_DEVERR_TIMEOUT the workspace must be
 * zeroed again before the next call.  With workspace NULL it reads the
 * array of markov_chain_sample_noalloc on the current device (MARKOV_OK if
 * no such call has run there) and zeroes that array after a timeout.
 */
int markov_status(void* workspace, void* stream);

/* markov_last_error: the reason for the calling thread's last error ("" if
 * none), in the manner of the pages' reason strings for configurations a
 * sampler cannot serve (sharded_markov page, unsupported_reason; muse_spark
 * markov page, unsupported).  The pointer stays valid until the thread's
 * next libmarkov call. */
const char* markov_last_error(void);

/*
 * markov_set_grid: tuning and testing knob.  0 (the default) lets the library
 * pick the number of persistent workgroups; g > 0 asks for at most g (clamped
 * to what the device can hold co-resident and to the work available).  The
 * chain's outputs do not depend on it.  Process-wide; returns the previous
 * value.
 */
int markov_set_grid(int g);

/*
 * markov_set_batch_path: tuning and testing knob for markov_chain_sample's
 * choice of kernels.  0 (the default):
 * batches of at most 64 rows run as one persistent chain launch, larger
 * batches over all rows per draft position (fused_markov page,
 * FusedMarkovSampler: the fused loop that serves batches beyond the
 * persistent chain, the bias GEMM plus two kernels a position; muse_spark
 * markov page, MarkovSampler: per-row arrival counters whose last block
 * picks the winner), in MARKOV_MODE_GUMBEL by the persistent step kernel
 * where it fits.  1: always persistent chain launches of at most 64 rows,
 * one after another.  2: always one launch per position.  3: the
 * persistent step kernel where it fits (MARKOV_MODE_GUMBEL; otherwise as 2).
 * markov_workspace_bytes covers every path.  Outputs do not depend on it.
 * Process-wide; returns the previous value.
 */
int markov_set_batch_path(int path);

/*
 * markov_set_wait_limit: testing and debugging knob.  Sets the bound, in
 * microseconds, of every cross-workgroup wait of later markov_chain_sample
 * calls (sharded_markov page, DSparkShardedMarkovSampler: timeout_ms bounds
 * every cross-rank wait); a negative value restores the default of 2 s.  With
 * 0 a wait gives up as soon as one poll finds a slot still empty, so a test
 * can drive the timeout path from the host while every workgroup still
 * exits normally.  Process-wide; returns the previous bound in microseconds.
 */
long long markov_set_wait_limit(long long us);

/* markov_grid: the number of workgroups markov_chain_sample would launch for
 * this shape on the current device under the current markov_set_grid value,
 * or a negative markov_status_t.  Host only. */
int markov_grid(int rows, int steps, int vocab, int rank, int mode);

#ifdef __cplusplus
}
#endif

#endif /* LIBMARKOV_MARKOV_H */
