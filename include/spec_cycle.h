/*
 * spec_cycle.h -- C ABI of libspeccycle.so: one fused, batched speculation cycle of
 * confidence-scheduled speculative decoding on an MI355X (gfx950) GPU.
 *
 * The cycle (per request b, all requests in parallel):
 *   1. prefix cut: L_b = number of leading draft positions whose running fp64 product of
 *      confidences stays >= threshold, stopping at the first failure ("DSpark turns speculation
 *      into a scheduler", section "Confidence is a serving primitive": prefix survival is the
 *      product of the per-position confidences; "The Speed Claim Nobody's Really Questioning",
 *      section "The Real Innovation: Confidence-Scheduled Verification": an early-stopping rule
 *      keeps the schedule lossless);
 *   2. semi-autoregressive draft: for j < L_b, x_j is sampled from
 *      softmax((base_j + A[x_{j-1}] . W) / T_b), the low-rank Markov transition bias from the
 *      previous sampled token ("DSpark turns speculation into a scheduler", section "DSpark's
 *      semi-autoregressive compromise"; "The Speed Claim...", section "The Semi-Autoregressive
 *      Trick": rank-256 Markov head);
 *   3. lossless verification: x_j is accepted while u_j < p_j(x_j) / q_j(x_j); at the first
 *      rejection one correction token is drawn from norm(max(0, p_j - q_j)); if all L_b drafts
 *      survive one bonus token is drawn from p at position L_b ("DSpark turns speculation into a
 *      scheduler", opening section and "Caveats"; "The Speed Claim...", section "Speculative
 *      Decoding in Two Sentences").
 * All randomness is a SplitMix64 counter hash of (seed, global request id, position, stream,
 * index): the same noise on any device and under any batching.
 *
 * Conventions
 *   - Every array pointer is a DEVICE pointer on the current HIP device; the caller owns every
 *     buffer.  Row-major layouts, last index fastest.
 *   - The call validates on the host, enqueues kernels on `stream` and returns; results are valid
 *     once the caller synchronises the stream.  It allocates nothing and copies nothing between
 *     host and device; scratch memory is the caller's `workspace`.
 *   - Reentrant for distinct workspaces; two calls sharing one workspace must be ordered on one
 *     stream.
 *   - Errors are negative return codes (below); nothing is enqueued when the host checks fail.
 *   - Per-request bad inputs (temperature not finite or <= 0, x0 outside [-1, V), a non-finite
 *     log-normaliser in a row the request needs) mark that request: accepted_len = -1, tokens -1.
 */
#ifndef SPEC_CYCLE_H
#define SPEC_CYCLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* spec_stream_t; /* a hipStream_t; NULL = the default stream */

enum {
  SPEC_OK = 0,
  SPEC_E_INVAL = -1,     /* NULL required pointer or bad dimension                           */
  SPEC_E_DTYPE = -2,     /* unsupported dtype / noise scheme / dimension combination          */
  SPEC_E_WORKSPACE = -3, /* workspace NULL or smaller than spec_workspace_bytes()             */
  SPEC_E_ARCH = -4,      /* current device is not gfx950                                      */
  SPEC_E_HIP = -5,       /* a HIP runtime call or kernel launch failed                        */
  SPEC_E_SCRATCH = -6    /* spec_cycle_noalloc: the dims need more than SPEC_SCRATCH_BYTES    */
};

enum { SPEC_FP32 = 0, SPEC_BF16 = 1 };          /* element type of logits, A and W           */
enum { SPEC_NOISE_FLAT = 0, SPEC_NOISE_CHUNKED = 1 };

/*
 * Execution paths of one cycle; both give identical results for the same inputs.
 *   SPEC_PATH_STEPWISE  k_init, then per position s = 0..K one sweep and one merge kernel: W
 *                       streams from memory once per position that has work.
 *   SPEC_PATH_RESIDENT  the whole cycle as ONE persistent launch (one workgroup per compute unit,
 *                       launched cooperatively so that all are resident together): every workgroup
 *                       keeps its slice of W in registers and LDS for all positions, so W crosses
 *                       HBM once per cycle, and the positions are separated by grid barriers
 *                       instead of kernel boundaries.  Needs bf16 rows, chunked noise, whole
 *                       64-column chunks (V % 64 == 0), 16-byte aligned logits, B <= 4 x compute
 *                       units, at most 640 vocabulary columns per compute unit (V <= 163840 on a
 *                       256-CU gfx950), logit tensors of at most 4 GiB - 1 MiB (B (K + 1) V 2 bytes) and A below
 *                       2 GiB (V R 2 bytes): its loads use 32-bit byte offsets.  A grid barrier
 *                       that does not complete within about a second (only if the device cannot
 *                       keep the grid resident) marks every request invalid instead of hanging.
 *                       The limit is 10^8 ticks of the 100 MHz real-time counter, or the decimal
 *                       value of the environment variable SPEC_RESIDENT_WAIT_TICKS, read at every
 *                       launch (0 forces the timeout path; spec_accept_stats then returns NaN).
 *   SPEC_PATH_AUTO      (0) the resident path when the call qualifies, else the stepwise one.
 */
enum { SPEC_PATH_AUTO = 0, SPEC_PATH_STEPWISE = 1, SPEC_PATH_RESIDENT = 2 };

typedef struct spec_dims {
  int32_t B;      /* requests, 1..1024                                                      */
  int32_t K;      /* draft positions per request, 1..32                                     */
  int32_t V;      /* vocabulary size, >= 2                                                  */
  int32_t R;      /* Markov rank, 1..256; bf16 needs R % 16 == 0                            */
  int32_t dtype;  /* SPEC_FP32 or SPEC_BF16                                                 */
  int32_t noise;  /* SPEC_NOISE_FLAT: one Gumbel per vocabulary index;                      */
                  /* SPEC_NOISE_CHUNKED: exact two-level Gumbel-max over 64-wide chunks     */
  int32_t path;   /* SPEC_PATH_*: 0 (AUTO) picks; forcing RESIDENT on a call that does not  */
                  /* qualify returns SPEC_E_DTYPE (spec_accept_stats: see there).           */
} spec_dims;

typedef struct spec_diag {   /* optional per-position diagnostics; any field may be NULL     */
  int32_t* verify_len;       /* [B]   L_b (-1 for an invalid request)                        */
  int32_t* draft_tokens;     /* [B,K] x_j for j < L_b, else -1                               */
  float* logq;               /* [B,K] log q_j(x_j) for j < L_b, else NaN                     */
  float* logp;               /* [B,K] log p_j(x_j) for decided positions (j <= a_b, j < L_b), else NaN */
} spec_diag;

/* Bytes of device workspace spec_cycle needs for these dimensions (0 if dims are invalid); with
 * SPEC_PATH_AUTO enough for either path. */
size_t spec_workspace_bytes(const spec_dims* d);

/* The path (SPEC_PATH_STEPWISE or SPEC_PATH_RESIDENT) spec_cycle takes for these dims on the
 * current device with 16-byte aligned logits, or a negative SPEC_E_* code. */
int spec_cycle_path(const spec_dims* d);

/*
 * One speculation cycle.
 *   base_logits   [B, K, V]    draft backbone logits of each draft position
 *   target_logits [B, K+1, V]  target logits; row j = target distribution at draft position j,
 *                              row K holds the bonus row of a request with L_b = K
 *   A             [V, R]       Markov factor gathered by the previous token
 *   W             [V, R]       Markov output factor, vocabulary-major: row v holds column v of
 *                              the R x V factor, so bias_v = sum_r A[prev, r] * W[v, r]
 *   x0            [B] int32    last committed token per request (Markov bias at position 0);
 *                              -1 = none; NULL = none for every request
 *   conf          [B, K] fp32  confidence of each draft position
 *   temp          [B] fp32     sampling temperature per request (scales both p and q)
 *   threshold                  prefix-survival threshold of the cut
 *   seed                       noise seed
 *   request_offset             global id of local request 0 in the noise hash, so a batch split
 *                              across calls (or GPUs) draws exactly the noise of one big call
 *   accepted_len  [B] int32    out: accepted drafts a_b (emitted tokens = a_b + 1), -1 invalid
 *   tokens        [B, K+1]     out: x_0..x_{a_b-1}, then the correction or bonus, then -1
 *   diag                       host struct of optional device outputs, may be NULL
 *   workspace                  device scratch of at least spec_workspace_bytes(d) bytes,
 *                              256-byte aligned; contents need no initialisation
 * Returns SPEC_OK or a negative SPEC_E_* code.
 */
int spec_cycle(const spec_dims* d, const void* base_logits, const void* target_logits,
               const void* A, const void* W, const int32_t* x0, const float* conf,
               const float* temp, float threshold, uint64_t seed, int64_t request_offset,
               int32_t* accepted_len, int32_t* tokens, const spec_diag* diag, void* workspace,
               size_t workspace_bytes, spec_stream_t stream);

/*
 * The same cycle with per-request verify lengths chosen by a scheduler (spec_schedule, for
 * instance) in place of the static-threshold prefix cut: step 1 of the cycle takes
 * L_b = verify_len[b] ("DSpark turns speculation into a scheduler", section "Confidence is a
 * serving primitive": the scheduler, not a fixed confidence threshold, sets each request's
 * verification length).  Every other step, argument and convention is spec_cycle's.
 *   verify_len [B] int32 device  L_b in 0..K; any other value marks request b invalid
 *                               (accepted_len = -1, tokens -1)
 * There is no conf or threshold argument.  Returns SPEC_OK or a negative SPEC_E_* code.
 */
int spec_cycle_lengths(const spec_dims* d, const void* base_logits, const void* target_logits,
                       const void* A, const void* W, const int32_t* x0, const int32_t* verify_len,
                       const float* temp, uint64_t seed, int64_t request_offset, int32_t* accepted_len,
                       int32_t* tokens, const spec_diag* diag, void* workspace, size_t workspace_bytes,
                       spec_stream_t stream);

/*
 * Profiling variant of spec_cycle for benchmarks: identical work and results, and every kernel
 * of the cycle is launched with a start/stop hipEvent_t pair attached to its own dispatch (no
 * extra queue packets; on the resident path the pair is recorded around its one launch).  On the
 * stepwise path kernel i is: 0 = set-up and prefix cut; 1 + 3s = sweep of the Markov-biased
 * rows of step s, 2 + 3s = sweep of the plain target rows of step s, 3 + 3s = per-request merge of
 * step s, for s = 0..K.  With bf16 rows and V % 8 == 0 the plain rows of step s run inside kernel
 * 1 + 3s, and the event pair of slot 2 + 3s is recorded back to back (an empty interval).  `events` is a host array of
 * n_events >= 2 * spec_cycle_kernel_count(d) events created by the caller (hipEventCreate);
 * events[2i] / events[2i+1] bracket kernel i.  The caller reads hipEventElapsedTime after the
 * stream is synchronised.  Returns SPEC_E_INVAL when the array is missing or too short.
 */
int spec_cycle_timed(const spec_dims* d, const void* base_logits, const void* target_logits,
                     const void* A, const void* W, const int32_t* x0, const float* conf,
                     const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                     int32_t* accepted_len, int32_t* tokens, const spec_diag* diag, void* workspace,
                     size_t workspace_bytes, spec_stream_t stream, void* const* events, int n_events);

/*
 * spec_cycle for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Identical work, arguments and results, with no
 * workspace argument: the scratch memory is a static device array of SPEC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  Its address on the current
 * device is looked up once per device on the first call there; after that the call allocates
 * nothing and frees nothing.
 *   Limit: dims whose spec_workspace_bytes() exceeds SPEC_SCRATCH_BYTES are rejected with
 *   SPEC_E_SCRATCH before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's one array, so calls that overlap on one GPU
 *   (different streams or threads, not ordered against each other) race and corrupt each other's
 *   results; order them on one stream.  A call leaves its state in the array; the next call sets
 *   up everything it reads, so nothing needs clearing in between.
 * Returns SPEC_OK, SPEC_E_SCRATCH, SPEC_E_HIP (the symbol lookup failed) or spec_cycle's codes.
 */
#define SPEC_SCRATCH_BYTES ((size_t)64 << 20)
int spec_cycle_noalloc(const spec_dims* d, const void* base_logits, const void* target_logits,
                       const void* A, const void* W, const int32_t* x0, const float* conf,
                       const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                       int32_t* accepted_len, int32_t* tokens, const spec_diag* diag, spec_stream_t stream);

/* Number of kernel slots of one spec_cycle call: 1 on the resident path (the whole cycle is
 * slot 0), 1 + 3 (K + 1) on the stepwise path; 0 for invalid dims. */
int spec_cycle_kernel_count(const spec_dims* d);

/* Bytes of device workspace spec_accept_stats needs (0 if dims are invalid; dims.noise unused). */
size_t spec_stats_workspace_bytes(const spec_dims* d);

/*
 * Acceptance statistics of drafted positions: the analytical acceptance rate
 *   alpha_{b,j} = sum_v min(p_j(v), q_j(v)) = 1 - TV(p_j, q_j),
 * the probability that a draft token drawn from q_j passes the accept test given that position j
 * is reached.  The drafter is trained on this total variation distance and the confidence head is
 * supervised by this per-step rate ("The Speed Claim Nobody's Really Questioning", sections "The
 * Semi-Autoregressive Trick" and "The Real Innovation: Confidence-Scheduled Verification").
 *   q_j = softmax((base row j + A[prev] . W) / T_b), prev = x0[b] at j = 0 (none if x0 is NULL or
 *         -1), else draft_tokens[b, j-1];   p_j = softmax(target row j / T_b).
 *   base_logits, target_logits, A, W, x0, temp: as for spec_cycle (same dims, same layouts)
 *   draft_tokens [B, K] int32  the drafted tokens (-1 past the drafted prefix), e.g. the
 *                              draft_tokens diagnostic of a spec_cycle call
 *   alpha        [B, K] fp32   out: alpha at every drafted position j (draft_tokens[b, j] >= 0,
 *                              j = 0 or draft_tokens[b, j-1] in [0, V)), NaN elsewhere and at every
 *                              position of a request whose temperature or x0 is invalid
 *   lse_q, lse_p [B, K] fp32   out, may be NULL: log-normalisers of q_j and p_j (NaN where alpha is)
 *   workspace                  device scratch of spec_stats_workspace_bytes(d) bytes, 256-byte
 *                              aligned, no initialisation needed
 * d->path: SPEC_PATH_AUTO or SPEC_PATH_RESIDENT take one cooperative launch with W held on chip
 * (bf16, V a multiple of 64, R <= 256 and a multiple of 16, logit tensors of at most 4 GiB - 1 MiB, 16-byte
 * aligned logits; RESIDENT on other dims returns SPEC_E_DTYPE, AUTO falls back); the rows go in
 * batches whose logits stay in the Infinity Cache between the two passes.  SPEC_PATH_STEPWISE
 * takes the sweep kernels (two passes over the logits, any dtype and V).
 * Asynchronous on `stream`, allocates nothing.  Returns SPEC_OK or a negative SPEC_E_* code
 * (NULL required pointer, bad dims or misaligned A / W: SPEC_E_INVAL; workspace: SPEC_E_WORKSPACE).
 */
int spec_accept_stats(const spec_dims* d, const void* base_logits, const void* target_logits,
                      const void* A, const void* W, const int32_t* x0, const int32_t* draft_tokens,
                      const float* temp, float* alpha, float* lse_q, float* lse_p, void* workspace,
                      size_t workspace_bytes, spec_stream_t stream);

/*
 * Expected calibration error of the confidences read as prefix-survival probabilities, the
 * quantity sequential temperature scaling minimises ("DSpark turns speculation into a scheduler",
 * section "Confidence is a serving primitive"; "The Speed Claim...", section "The Real Innovation",
 * where the fit takes this error from several percent to around one percent).  One pair per verified position
 * j < verify_len[b] of every request with accepted_len[b] >= 0: prediction = fp64 running product
 * of conf[b, 0..j]; outcome = 1 if j < accepted_len[b] (the prefix through j survived).  nbins
 * equal-width bins on [0, 1] (1..1024); ECE = sum over bins of (pairs in bin / all pairs) *
 * |mean prediction - mean outcome|, 0 when there is no pair.
 *   conf [B, K] fp32, verify_len [B] int32, accepted_len [B] int32: device inputs (the cycle's
 *   diagnostics and outputs);  ece [1] fp64 and n_pairs [1] int64: device outputs.
 * Asynchronous on `stream`.  Returns SPEC_OK or SPEC_E_INVAL (NULL pointer, B outside 1..1024,
 * K outside 1..32, nbins outside 1..1024).
 */
int spec_calibration_error(const float* conf, const int32_t* verify_len, const int32_t* accepted_len,
                           int32_t B, int32_t K, int32_t nbins, double* ece, int64_t* n_pairs,
                           spec_stream_t stream);

/*
 * Hardware-aware prefix scheduler: per-request verify lengths for the current batch pressure.
 * The confidences are read as prefix-survival probabilities P_{b,j} = prod_{i<=j} conf[b, i];
 * verification positions are weighed against a profiled throughput curve of the target engine
 * ("DSpark turns speculation into a scheduler", section "Confidence is a serving primitive";
 * "The Speed Claim...", section "The Real Innovation": verify more when the engine is idle, fewer
 * when it is busy, an early-stopping rule keeps the schedule lossless).
 *   Position j of request b is kept at threshold g / nbins iff bin(M_{b,j}) >= g, where M is the
 *   fp64 running minimum of P (so a prefix ends at its first failing position) and
 *   bin(M) = min(floor(M * nbins), nbins).  For g = 1..nbins (and g = nbins + 1: keep nothing):
 *   n_g kept positions, expected emitted tokens E_g = B + sum of P over them, goodput
 *   E_g / step_time[n_g].  The largest goodput wins, ties to the larger g.
 *   conf       [B, K] fp32 device  confidences
 *   step_time  [B K + 1] fp64 device  seconds of one target verification step carrying n draft
 *              tokens, n = 0..B K (the profiled throughput curve), > 0
 *   nbins      threshold grid, 1..4096
 *   verify_len [B] int32 device out: each request's prefix length at the chosen threshold
 *   out        [4] fp64 device out: threshold g / nbins (> 1 when nothing is kept), kept positions,
 *              expected emitted tokens, goodput (tokens per second)
 * Asynchronous on `stream`; one workgroup.  Returns SPEC_OK or SPEC_E_INVAL (NULL pointer, B
 * outside 1..1024, K outside 1..32, nbins outside 1..4096).
 */
int spec_schedule(const float* conf, int32_t B, int32_t K, const double* step_time, int32_t nbins,
                  int32_t* verify_len, double* out, spec_stream_t stream);

/* Bytes of device workspace spec_temperature_scaling needs for N sequences and G grid entries
 * (0 if N is outside 1..2^24 or G outside 1..1024). */
size_t spec_temperature_scaling_workspace_bytes(int32_t N, int32_t G);

/*
 * Sequential temperature scaling of the confidence head: per-position temperatures fitted left to
 * right on held-out sequences so that the cumulative prefix probability is calibrated ("DSpark
 * turns speculation into a scheduler", section "Confidence is a serving primitive": with the
 * earlier positions fixed, the next position's temperature minimises the calibration error of the
 * cumulative prefix probability; "The Speed Claim...", section "The Real Innovation").
 *   z            [N, K] fp32 device  the head's raw logits, c_{n,k}(T) = 1 / (1 + exp(-z_{n,k} / T))
 *   verify_len   [N] int32 device    verified positions of each held-out sequence
 *   accepted_len [N] int32 device    accepted drafts (-1: sequence left out); the prefix through k
 *                                    survived iff k < accepted_len
 *   grid         [G] fp64 device     candidate temperatures, ascending, G in 1..1024
 *   nbins        bins of the calibration error, 1..64
 *   T            [K] fp64 device out fitted temperatures: T_k is the grid value with the smallest
 *                                    calibration error of prod_{i<=k} c_{n,i}(T_i) against survival
 *                                    over the sequences with k < verify_len (ties: earlier entry)
 *   ece_before, ece_after [K] fp64 device out (may be NULL): that error with every T = 1, and fitted
 *   workspace    spec_temperature_scaling_workspace_bytes(N, G) bytes, 256-byte aligned
 * Asynchronous on `stream` (3 K + 1 kernels).  Returns SPEC_OK, SPEC_E_INVAL (NULL pointer, N outside
 * 1..2^24, K outside 1..256, G or nbins out of range) or SPEC_E_WORKSPACE.
 */
int spec_temperature_scaling(const float* z, const int32_t* verify_len, const int32_t* accepted_len,
                             int32_t N, int32_t K, const double* grid, int32_t G, int32_t nbins, double* T,
                             double* ece_before, double* ece_after, void* workspace, size_t workspace_bytes,
                             spec_stream_t stream);

/*
 * Decode-loop glue: the next cycle's context.  For every request with accepted_len[b] in 0..K,
 * x0[b] becomes tokens[b, accepted_len[b]], the last token the cycle emitted (the correction or
 * bonus), and emitted[b] (may be NULL) grows by accepted_len[b] + 1; invalid requests keep their
 * x0 ("DSpark turns speculation into a scheduler", opening section: keep the accepted prefix and
 * continue from it).  tokens [B, K+1], accepted_len [B]: a spec_cycle call's outputs; x0 [B]
 * int32 in/out; emitted [B] int64 in/out.  Asynchronous on `stream`.  Returns SPEC_OK or
 * SPEC_E_INVAL (NULL pointer, B outside 1..1024, K outside 1..32).
 */
int spec_advance(const int32_t* tokens, const int32_t* accepted_len, int32_t B, int32_t K, int32_t* x0,
                 int64_t* emitted, spec_stream_t stream);

/* Static description of an error code (never NULL). */
const char* spec_error_string(int code);

/* Library version: major * 10000 + minor * 100 + patch. */
int spec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_CYCLE_H */
