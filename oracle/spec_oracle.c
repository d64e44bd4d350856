/*
 * spec_oracle.c -- plain fp64 CPU oracle for one confidence-scheduled speculation cycle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or constant generator
 * with the HIP library: the counter hash below is written here from its published definition,
 * and the GPU side writes its own copy from the same definition.
 *
 * What it computes, per request b (sources: the three DSpark pages):
 *   1. prefix cut      -- verify length L_b = number of leading draft positions whose fp64
 *                         running product of confidences stays >= threshold; stop at the first
 *                         failure ("DSpark turns speculation into a scheduler", section
 *                         "Confidence is a serving primitive": prefix-survival product of the
 *                         per-position confidences; "The Speed Claim Nobody's Really
 *                         Questioning", section "The Real Innovation: Confidence-Scheduled
 *                         Verification": an early-stopping rule keeps the scheduler lossless).
 *   2. draft           -- for j < L_b: logits = base row j + Markov transition bias
 *                         A[x_{j-1}] . W (rank R), divided by the request temperature, sampled
 *                         with Gumbel-max ("DSpark turns speculation into a scheduler", section
 *                         "DSpark's semi-autoregressive compromise": low-rank transition signal
 *                         from the previous sampled token; "The Speed Claim...", section "The
 *                         Semi-Autoregressive Trick": Markov head of rank 256 adds a
 *                         prefix-dependent bias before each token is sampled).
 *   3. verify          -- accept x_j while u_j < p_j(x_j)/q_j(x_j); stop at the first reject
 *                         ("DSpark turns speculation into a scheduler", opening section and
 *                         "Caveats": with this accept/reject rule the emitted tokens follow
 *                         the target model's own distribution; "The Speed Claim...", section "Speculative Decoding in
 *                         Two Sentences": accept the longest valid prefix).
 *   4. correct / bonus -- on reject at position a: one token from norm(max(0, p_a - q_a));
 *                         when the whole prefix survives: one bonus token from p at position
 *                         L_b ("The Speed Claim...", section "Speculative Decoding in Two
 *                         Sentences": appending one bonus token).
 *
 * Readings taken where the pages are silent (all listed in the design notes):
 *   - temperature T_b scales both p and q (the user's sampling temperature defines the
 *     distribution the lossless rule preserves);
 *   - the Markov bias at position 0 uses the last committed token x0[b] (-1 = no bias);
 *   - the accept test is strict (u < p/q); argmax ties go to the smallest index;
 *   - when max(0, p - q) has no positive entry in fp64 the correction is drawn from p;
 *   - randomness: SplitMix64 counter hash keyed by (seed, request, position, stream, index),
 *     32-bit uniforms, Gumbel noise -log(-log1p(-U)); two noise schemes: FLAT (one Gumbel per
 *     vocabulary index) and CHUNKED (an exact two-level Gumbel-max: a Gumbel per 64-wide
 *     vocabulary chunk on the chunk log-mass, then a Gumbel per index inside the winning chunk).
 *
 * Everything is fp64; inputs are fp32 or bf16 (bf16 converts exactly).  Plain loops in the
 * order the method states them; OpenMP only splits independent requests across threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------------------
 * SplitMix64 (Steele, Lea, Flood 2014, "Fast splittable pseudorandom number generators";
 * public-domain reference splitmix64.c).  state += golden gamma; output = mix(state).
 * --------------------------------------------------------------------------------------- */
static const uint64_t SM_GAMMA = 0x9E3779B97F4A7C15ULL;

static uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* one SplitMix64 step: advance the state, return the output */
uint64_t oracle_splitmix64_next(uint64_t* state) {
  *state += SM_GAMMA;
  return sm_mix(*state);
}

/* first output of a SplitMix64 generator seeded with x */
static uint64_t sm_first(uint64_t x) {
  uint64_t s = x;
  return oracle_splitmix64_next(&s);
}

/* stream identifiers */
enum { ST_DRAFT = 1, ST_ACCEPT = 2, ST_RESIDUAL = 3, ST_BONUS = 4,
       ST_DRAFT_C = 5, ST_RESIDUAL_C = 7, ST_BONUS_C = 8 };

/* key of one noise row: chained SplitMix64 first outputs over (seed, request, position, stream) */
uint64_t oracle_rowkey(uint64_t seed, uint64_t request, uint64_t pos, uint64_t stream) {
  uint64_t k = sm_first(seed);
  k = sm_first(k ^ request);
  k = sm_first(k ^ pos);
  k = sm_first(k ^ stream);
  return k;
}

/* 32 random bits for index i of the row with key `key`: the (i/2+1)-th output of a SplitMix64
 * generator whose state starts at `key`; even i takes the high half, odd i the low half */
uint32_t oracle_bits32(uint64_t key, uint64_t i) {
  /* the n-th output from state `key` is mix(key + n * gamma) (mod 2^64), n = i/2 + 1 */
  uint64_t n = i / 2 + 1;
  uint64_t w = sm_mix(key + n * SM_GAMMA);
  return (i % 2 == 0) ? (uint32_t)(w >> 32) : (uint32_t)(w & 0xFFFFFFFFULL);
}

/* uniform in (0,1): (bits + 1/2) * 2^-32, exact in fp64 */
double oracle_uniform(uint64_t key, uint64_t i) {
  return ((double)oracle_bits32(key, i) + 0.5) * 0x1p-32;
}

/* standard Gumbel: G = -log(E), E = -log(1 - U) computed as -log1p(-U) */
double oracle_gumbel(uint64_t key, uint64_t i) {
  double u = oracle_uniform(key, i);
  double e = -log1p(-u);
  return -log(e);
}

/* ---------------------------------------------------------------------------------------
 * input element access: dtype 0 = fp32, 1 = bf16 stored as uint16 (exact widening)
 * --------------------------------------------------------------------------------------- */
static double load_elem(const void* p, int dtype, size_t idx) {
  if (dtype == 0) return (double)((const float*)p)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------------------------
 * small numerical helpers
 * --------------------------------------------------------------------------------------- */

/* log(sum_i exp(x_i)) over n entries, -inf entries allowed; NaN/+inf propagate */
double oracle_lse(const double* x, int64_t n) {
  double m = -INFINITY;
  for (int64_t i = 0; i < n; i++) {
    if (isnan(x[i])) return NAN;
    if (x[i] > m) m = x[i];
  }
  if (m == -INFINITY) return -INFINITY;
  if (m == INFINITY) return INFINITY;
  double s = 0.0;
  for (int64_t i = 0; i < n; i++) s += exp(x[i] - m);
  return m + log(s);
}

/* prefix cut: leading positions whose running product of confidences stays >= threshold */
int32_t oracle_cut(const float* conf, int32_t K, float threshold) {
  double P = 1.0;
  int32_t L = 0;
  for (int32_t j = 0; j < K; j++) {
    P *= (double)conf[j];
    if (!(P >= (double)threshold)) break;   /* first failure ends the prefix; NaN fails */
    L = j + 1;
  }
  return L;
}

/* Markov transition bias for previous token prev: bias[v] = sum_r A[prev][r] * W[v][r].
 * A and W are both stored vocabulary-major [V][R] (W row v is column v of the R x V factor). */
void oracle_bias(const void* A, const void* W, int dtype, int32_t V, int32_t R, int32_t prev, double* bias) {
  for (int32_t v = 0; v < V; v++) {
    double acc = 0.0;
    if (prev >= 0) {
      for (int32_t r = 0; r < R; r++)
        acc += load_elem(A, dtype, (size_t)prev * R + r) * load_elem(W, dtype, (size_t)v * R + r);
    }
    bias[v] = acc;
  }
}

/* ---------------------------------------------------------------------------------------
 * Gumbel-max samplers.  score[v] = -inf marks an excluded index.
 * Returns the chosen index (smallest index on exact ties) or -1 if every score is -inf.
 * margin outputs: best minus second-best perturbed score (+inf if one candidate).
 * --------------------------------------------------------------------------------------- */
static int32_t argmax_perturbed(const double* score, int64_t lo, int64_t hi, uint64_t key,
                                int64_t key_index_base, double* margin) {
  int32_t best = -1;
  double b1 = -INFINITY, b2 = -INFINITY;
  for (int64_t v = lo; v < hi; v++) {
    if (score[v] == -INFINITY) continue;
    double z = score[v] + oracle_gumbel(key, (uint64_t)(v - key_index_base));
    if (best < 0 || z > b1) {
      b2 = b1;
      b1 = z;
      best = (int32_t)v;
    } else if (z > b2) {
      b2 = z;
    }
  }
  if (margin) *margin = (best < 0) ? NAN : (b1 - b2);
  return best;
}

#define CHUNK 64

/* FLAT: argmax_v (score_v + G(key2, v)) */
static int32_t sample_flat(const double* score, int32_t V, uint64_t key2, double* m1) {
  return argmax_perturbed(score, 0, V, key2, 0, m1);
}

/* CHUNKED: chunk c = [64c, 64c+64) clipped to V; log-mass Lc = log sum_{v in c} exp(score_v);
 * c* = argmax_c (Lc + G(key1, c)); then argmax_{v in c*} (score_v + G(key2, v)).
 * Exact: P(c*) = mass_c / total, P(v | c*) = exp(score_v) / mass_c. */
static int32_t sample_chunked(const double* score, int32_t V, uint64_t key1, uint64_t key2,
                              double* m1, double* m2, double* scratch_chunks) {
  int32_t nch = (V + CHUNK - 1) / CHUNK;
  for (int32_t c = 0; c < nch; c++) {
    int64_t lo = (int64_t)c * CHUNK, hi = lo + CHUNK;
    if (hi > V) hi = V;
    scratch_chunks[c] = oracle_lse(score + lo, hi - lo);
  }
  int32_t cstar = argmax_perturbed(scratch_chunks, 0, nch, key1, 0, m1);
  if (cstar < 0) {
    if (m2) *m2 = NAN;
    return -1;
  }
  int64_t lo = (int64_t)cstar * CHUNK, hi = lo + CHUNK;
  if (hi > V) hi = V;
  /* level-2 noise is keyed by the vocabulary index itself */
  return argmax_perturbed(score, lo, hi, key2, 0, m2);
}

static int32_t sample(int noise, const double* score, int32_t V, uint64_t key1, uint64_t key2,
                      double* m1, double* m2, double* scratch_chunks) {
  if (noise == 0) {
    if (m2) *m2 = NAN;
    return sample_flat(score, V, key2, m1);
  }
  return sample_chunked(score, V, key1, key2, m1, m2, scratch_chunks);
}

/* ---------------------------------------------------------------------------------------
 * the cycle
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int32_t B, K, V, R;
  int32_t dtype; /* 0 = fp32, 1 = bf16 */
  int32_t noise; /* 0 = FLAT, 1 = CHUNKED */
} oracle_dims;

typedef struct {            /* every pointer may be NULL except accepted_len and tokens */
  int32_t* accepted_len;    /* [B]     accepted drafts, -1 for an invalid request        */
  int32_t* tokens;          /* [B,K+1] accepted drafts, then correction/bonus, -1 padded  */
  int32_t* verify_len;      /* [B]     L_b                                               */
  int32_t* draft_tokens;    /* [B,K]   x_j for j < L_b, else -1                          */
  int32_t* final_kind;      /* [B]     0 residual, 1 bonus, 2 residual fell back to p, -1 invalid */
  double* logq;             /* [B,K]   log q_j(x_j) for j < L_b                          */
  double* logp;             /* [B,K]   log p_j(x_j) for decided positions                */
  double* lse_q;            /* [B,K]   log-normaliser of the scaled draft row            */
  double* lse_p;            /* [B,K+1] log-normaliser of the scaled target row (rows read) */
  double* u;                /* [B,K]   accept uniform of each decided position           */
  double* ratio;            /* [B,K]   p/q at each decided position                      */
  double* draft_margin1;    /* [B,K]   FLAT margin, or CHUNKED level-1 margin            */
  double* draft_margin2;    /* [B,K]   CHUNKED level-2 margin (NaN for FLAT)             */
  double* final_margin1;    /* [B]     margin of the correction/bonus draw (level 1)     */
  double* final_margin2;    /* [B]     level-2 margin of that draw (NaN for FLAT)        */
} oracle_out;

/* where the target row for (request, position, accepted prefix) comes from */
typedef const void* (*target_row_fn)(const void* ctx, int32_t b, int32_t j, const int32_t* prefix);

typedef struct {
  const void* target;       /* [B, K+1, V] */
  int32_t K, V, dtype;
} array_ctx;

static const void* target_from_array(const void* ctx, int32_t b, int32_t j, const int32_t* prefix) {
  const array_ctx* a = (const array_ctx*)ctx;
  (void)prefix;
  size_t elem = (a->dtype == 0) ? 4 : 2;
  return (const char*)a->target + (((size_t)b * (a->K + 1) + j) * a->V) * elem;
}

typedef struct {
  const void* table;        /* [n_prefix, V]: row for every prefix of length 0..K */
  int32_t K, V, dtype;
} table_ctx;

/* prefix (y_0..y_{n-1}) -> row (V^n - 1)/(V - 1) + sum_i y_i V^(n-1-i) */
static const void* target_from_table(const void* ctx, int32_t b, int32_t j, const int32_t* prefix) {
  const table_ctx* t = (const table_ctx*)ctx;
  (void)b;
  int64_t off = 0, pw = 1;
  for (int32_t i = 0; i < j; i++) {
    off += pw;
    pw *= t->V;
  }
  int64_t id = 0;
  for (int32_t i = 0; i < j; i++) id = id * t->V + prefix[i];
  size_t elem = (t->dtype == 0) ? 4 : 2;
  return (const char*)t->table + (size_t)(off + id) * t->V * elem;
}

typedef struct {
  int32_t K, V, R, dtype, noise;
  const void* base_req;     /* [K, V] rows of this request */
  const void* A;
  const void* W;
  int32_t x0;               /* -1 = no bias at position 0 */
  const float* conf;        /* [K] */
  float temp, threshold;
  int32_t has_L, L_given;   /* has_L: the verify length is given (the scheduler's), not cut */
  uint64_t seed, gid;       /* gid = global request id used in the hash */
  target_row_fn target_row;
  const void* target_ctx;
  int32_t b;                /* local request index handed to target_row */
} req_in;

typedef struct {
  int32_t accepted_len, L, final_kind;
  int32_t* tokens;          /* [K+1] */
  int32_t* draft;           /* [K]   */
  double *logq, *logp, *lse_q, *lse_p, *u, *ratio, *dm1, *dm2;   /* [K] / lse_p [K+1] */
  double fm1, fm2;
} req_out;

static void set_invalid(const req_in* in, req_out* o) {
  o->accepted_len = -1;
  o->final_kind = -1;
  o->L = -1;
  for (int32_t j = 0; j <= in->K; j++) o->tokens[j] = -1;
  for (int32_t j = 0; j < in->K; j++) o->draft[j] = -1;
}

/* one request through the whole cycle; work buffers: s_rows [K*V], tmp [V], chunks [V/64+1] */
static void cycle_one(const req_in* in, req_out* o, double* s_rows, double* tmp, double* chunks) {
  const int32_t K = in->K, V = in->V;
  const double T = (double)in->temp;
  for (int32_t j = 0; j <= K; j++) o->tokens[j] = -1;
  for (int32_t j = 0; j < K; j++) {
    o->draft[j] = -1;
    o->logq[j] = o->logp[j] = o->lse_q[j] = o->u[j] = o->ratio[j] = o->dm1[j] = o->dm2[j] = NAN;
  }
  for (int32_t j = 0; j <= K; j++) o->lse_p[j] = NAN;
  o->fm1 = o->fm2 = NAN;

  if (!(T > 0.0) || isinf(T) || in->x0 < -1 || in->x0 >= V) {
    set_invalid(in, o);
    return;
  }

  /* 1. prefix cut, or the verify length a scheduler chose (outside [0, K]: a bad request) */
  if (in->has_L && (in->L_given < 0 || in->L_given > K)) {
    set_invalid(in, o);
    return;
  }
  const int32_t L = in->has_L ? in->L_given : oracle_cut(in->conf, K, in->threshold);
  o->L = L;

  /* 2. semi-autoregressive draft: x_j ~ softmax((base_j + A[x_{j-1}] W) / T) */
  for (int32_t j = 0; j < L; j++) {
    int32_t prev = (j == 0) ? in->x0 : o->draft[j - 1];
    double* s = s_rows + (size_t)j * V;
    oracle_bias(in->A, in->W, in->dtype, V, in->R, prev, tmp);
    for (int32_t v = 0; v < V; v++)
      s[v] = (load_elem(in->base_req, in->dtype, (size_t)j * V + v) + tmp[v]) / T;
    double lse = oracle_lse(s, V);
    o->lse_q[j] = lse;
    if (!isfinite(lse)) {
      set_invalid(in, o);
      return;
    }
    uint64_t k2 = oracle_rowkey(in->seed, in->gid, (uint64_t)j, ST_DRAFT);
    uint64_t k1 = oracle_rowkey(in->seed, in->gid, (uint64_t)j, ST_DRAFT_C);
    int32_t x = sample(in->noise, s, V, k1, k2, &o->dm1[j], &o->dm2[j], chunks);
    o->draft[j] = x;
    o->logq[j] = s[x] - lse;
  }

  /* 3. verification: accept while u_j < p_j(x_j) / q_j(x_j) */
  int32_t a = 0;
  for (int32_t j = 0; j < L; j++) {
    const void* trow = in->target_row(in->target_ctx, in->b, j, o->draft);
    for (int32_t v = 0; v < V; v++) tmp[v] = load_elem(trow, in->dtype, (size_t)v) / T;
    double lse = oracle_lse(tmp, V);
    o->lse_p[j] = lse;
    if (!isfinite(lse)) {
      set_invalid(in, o);
      return;
    }
    o->logp[j] = tmp[o->draft[j]] - lse;
    double ratio = exp(o->logp[j] - o->logq[j]);
    double u = oracle_uniform(oracle_rowkey(in->seed, in->gid, (uint64_t)j, ST_ACCEPT), 0);
    o->u[j] = u;
    o->ratio[j] = ratio;
    if (u < ratio) {
      a++;
    } else {
      break;
    }
  }

  /* 4. correction from norm(max(0, p - q)) at the rejected position, or bonus from p */
  int32_t y;
  if (a < L) {
    const int32_t j = a;
    const double* s = s_rows + (size_t)j * V;       /* scaled draft logits of row j */
    const void* trow = in->target_row(in->target_ctx, in->b, j, o->draft);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    int any = 0;
    for (int32_t v = 0; v < V; v++) {
      double lp = load_elem(trow, in->dtype, (size_t)v) / T - o->lse_p[j];
      double lq = s[v] - o->lse_q[j];
      if (lp > lq) {
        w[v] = lp + log(-expm1(lq - lp));           /* log(p_v - q_v) */
        any = 1;
      } else {
        w[v] = -INFINITY;
      }
    }
    uint64_t k2 = oracle_rowkey(in->seed, in->gid, (uint64_t)j, ST_RESIDUAL);
    uint64_t k1 = oracle_rowkey(in->seed, in->gid, (uint64_t)j, ST_RESIDUAL_C);
    if (any) {
      y = sample(in->noise, w, V, k1, k2, &o->fm1, &o->fm2, chunks);
      o->final_kind = 0;
    } else {
      for (int32_t v = 0; v < V; v++) w[v] = load_elem(trow, in->dtype, (size_t)v) / T;
      y = sample(in->noise, w, V, k1, k2, &o->fm1, &o->fm2, chunks);
      o->final_kind = 2;
    }
    free(w);
  } else {
    const void* trow = in->target_row(in->target_ctx, in->b, L, o->draft);
    for (int32_t v = 0; v < V; v++) tmp[v] = load_elem(trow, in->dtype, (size_t)v) / T;
    o->lse_p[L] = oracle_lse(tmp, V);
    if (!isfinite(o->lse_p[L])) {
      set_invalid(in, o);
      return;
    }
    uint64_t k2 = oracle_rowkey(in->seed, in->gid, (uint64_t)L, ST_BONUS);
    uint64_t k1 = oracle_rowkey(in->seed, in->gid, (uint64_t)L, ST_BONUS_C);
    y = sample(in->noise, tmp, V, k1, k2, &o->fm1, &o->fm2, chunks);
    o->final_kind = 1;
  }

  for (int32_t i = 0; i < a; i++) o->tokens[i] = o->draft[i];
  o->tokens[a] = y;
  o->accepted_len = a;
}

/* shared driver: runs requests [0, n) with per-request input/output views */
typedef struct {
  const oracle_dims* d;
  const void* base;         /* [nbase, K, V] */
  int64_t base_req_stride;  /* requests per base block: 1 = one block per request, 0 = shared */
  const void* A;
  const void* W;
  const int32_t* x0;        /* [n] or NULL */
  int64_t x0_stride;
  const float* conf;        /* [n, K] */
  int64_t conf_stride;
  const float* temp;        /* [n] */
  int64_t temp_stride;
  float threshold;
  const int32_t* L_in;      /* [n] given verify lengths, or NULL: the prefix cut */
  uint64_t seed;
  int64_t request_offset;
  target_row_fn target_row;
  const void* target_ctx;
  int32_t target_b_stride;  /* 1: request b reads target request b; 0: request 0 for all */
} driver_in;

static void run_driver(const driver_in* di, int64_t n, const oracle_out* out, int nthreads) {
  const oracle_dims* d = di->d;
  const int32_t K = d->K, V = d->V;
  const size_t elem = (d->dtype == 0) ? 4 : 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s_rows = (double*)malloc(sizeof(double) * ((size_t)K * V + 1));
    double* tmp = (double*)malloc(sizeof(double) * (size_t)V);
    double* chunks = (double*)malloc(sizeof(double) * ((size_t)V / CHUNK + 2));
    int32_t* toks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
    int32_t* draft = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    double* dbuf = (double*)malloc(sizeof(double) * (size_t)(8 * (K + 1)));
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < n; b++) {
      req_in in;
      in.K = K; in.V = V; in.R = d->R; in.dtype = d->dtype; in.noise = d->noise;
      in.base_req = (const char*)di->base + (size_t)(b * di->base_req_stride) * K * V * elem;
      in.A = di->A; in.W = di->W;
      in.x0 = di->x0 ? di->x0[b * di->x0_stride] : -1;
      in.conf = di->conf ? di->conf + b * di->conf_stride * K : NULL;
      in.has_L = di->L_in != NULL;
      in.L_given = di->L_in ? di->L_in[b] : 0;
      in.temp = di->temp[b * di->temp_stride];
      in.threshold = di->threshold;
      in.seed = di->seed;
      in.gid = (uint64_t)(di->request_offset + b);
      in.target_row = di->target_row;
      in.target_ctx = di->target_ctx;
      in.b = (int32_t)(b * di->target_b_stride);
      req_out o;
      o.tokens = toks; o.draft = draft;
      o.logq = dbuf; o.logp = dbuf + (K + 1); o.lse_q = dbuf + 2 * (K + 1);
      o.lse_p = dbuf + 3 * (K + 1); o.u = dbuf + 4 * (K + 1); o.ratio = dbuf + 5 * (K + 1);
      o.dm1 = dbuf + 6 * (K + 1); o.dm2 = dbuf + 7 * (K + 1);
      cycle_one(&in, &o, s_rows, tmp, chunks);

      out->accepted_len[b] = o.accepted_len;
      for (int32_t j = 0; j <= K; j++) out->tokens[b * (K + 1) + j] = toks[j];
      if (out->verify_len) out->verify_len[b] = o.L;
      if (out->final_kind) out->final_kind[b] = o.final_kind;
      for (int32_t j = 0; j < K; j++) {
        if (out->draft_tokens) out->draft_tokens[b * K + j] = draft[j];
        if (out->logq) out->logq[b * K + j] = o.logq[j];
        if (out->logp) out->logp[b * K + j] = o.logp[j];
        if (out->lse_q) out->lse_q[b * K + j] = o.lse_q[j];
        if (out->u) out->u[b * K + j] = o.u[j];
        if (out->ratio) out->ratio[b * K + j] = o.ratio[j];
        if (out->draft_margin1) out->draft_margin1[b * K + j] = o.dm1[j];
        if (out->draft_margin2) out->draft_margin2[b * K + j] = o.dm2[j];
      }
      if (out->lse_p)
        for (int32_t j = 0; j <= K; j++) out->lse_p[b * (K + 1) + j] = o.lse_p[j];
      if (out->final_margin1) out->final_margin1[b] = o.fm1;
      if (out->final_margin2) out->final_margin2[b] = o.fm2;
    }
    free(s_rows); free(tmp); free(chunks); free(toks); free(draft); free(dbuf);
  }
}

static int check_dims(const oracle_dims* d) {
  if (!d || d->B < 0 || d->K < 1 || d->V < 2 || d->R < 1) return -1;
  if (d->dtype != 0 && d->dtype != 1) return -2;
  if (d->noise != 0 && d->noise != 1) return -2;
  return 0;
}

/* The cycle over B requests; target_logits [B, K+1, V] (row j = target at draft position j,
 * row L_b = bonus row).  Host pointers.  Returns 0, or a negative code for bad arguments. */
int spec_cycle_ref(const oracle_dims* d, const void* base_logits, const void* target_logits,
                   const void* A, const void* W, const int32_t* x0, const float* conf,
                   const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                   const oracle_out* out, int nthreads) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!base_logits || !target_logits || !A || !W || !conf || !temp || !out || !out->accepted_len || !out->tokens)
    return -1;
  array_ctx ctx = {target_logits, d->K, d->V, d->dtype};
  driver_in di = {d, base_logits, 1, A, W, x0, 1, conf, 1, temp, 1, threshold, NULL, seed, request_offset,
                  target_from_array, &ctx, 1};
  run_driver(&di, d->B, out, nthreads);
  return 0;
}

/* The cycle with verify lengths given per request (a scheduler's, for instance) instead of the
 * prefix cut: verify_len [B] in 0..K (other values mark the request invalid).  Everything after
 * the cut is the same cycle. */
int spec_cycle_ref_lengths(const oracle_dims* d, const void* base_logits, const void* target_logits,
                           const void* A, const void* W, const int32_t* x0, const int32_t* verify_len,
                           const float* temp, uint64_t seed, int64_t request_offset, const oracle_out* out,
                           int nthreads) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!base_logits || !target_logits || !A || !W || !verify_len || !temp || !out || !out->accepted_len ||
      !out->tokens)
    return -1;
  array_ctx ctx = {target_logits, d->K, d->V, d->dtype};
  driver_in di = {d, base_logits, 1, A, W, x0, 1, NULL, 1, temp, 1, 0.0f, verify_len, seed, request_offset,
                  target_from_array, &ctx, 1};
  run_driver(&di, d->B, out, nthreads);
  return 0;
}

/* Same cycle with a prefix-dependent target: target_table [sum_{n=0..K} V^n, V], row of the
 * prefix (y_0..y_{n-1}) at (V^n - 1)/(V - 1) + base-V value of the prefix.  Used for the
 * brute-force losslessness check on tiny vocabularies. */
int spec_cycle_ref_table(const oracle_dims* d, const void* base_logits, const void* target_table,
                         const void* A, const void* W, const int32_t* x0, const float* conf,
                         const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                         const oracle_out* out, int nthreads) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!base_logits || !target_table || !A || !W || !conf || !temp || !out || !out->accepted_len || !out->tokens)
    return -1;
  table_ctx ctx = {target_table, d->K, d->V, d->dtype};
  driver_in di = {d, base_logits, 1, A, W, x0, 1, conf, 1, temp, 1, threshold, NULL, seed, request_offset,
                  target_from_table, &ctx, 1};
  run_driver(&di, d->B, out, nthreads);
  return 0;
}

/* Monte-Carlo driver: one request's inputs (B must be 1 in d, table target) repeated for
 * n_trials request ids request_offset .. request_offset + n_trials - 1.  out arrays sized by
 * n_trials. */
int spec_cycle_ref_mc(const oracle_dims* d, const void* base_logits, const void* target_table,
                      const void* A, const void* W, int32_t x0, const float* conf, float temp,
                      float threshold, uint64_t seed, int64_t request_offset, int64_t n_trials,
                      const oracle_out* out, int nthreads) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!base_logits || !target_table || !A || !W || !conf || !out || !out->accepted_len || !out->tokens)
    return -1;
  table_ctx ctx = {target_table, d->K, d->V, d->dtype};
  driver_in di = {d, base_logits, 0, A, W, &x0, 0, conf, 0, &temp, 0, threshold, NULL, seed, request_offset,
                  target_from_table, &ctx, 0};
  run_driver(&di, n_trials, out, nthreads);
  return 0;
}

/* number of OpenMP threads a parallel region would use (1 without OpenMP) */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------------------------
 * Acceptance statistics.
 *
 * alpha_{b,j} = sum_v min(p_j(v), q_j(v)) = 1 - TV(p_j, q_j): the probability that a draft
 * token drawn from q_j passes the accept test u < p/q, given that position j is reached.  The
 * pages name this quantity twice: the drafter is trained on the total variation distance because
 * it directly sets the acceptance rate, and the confidence head is supervised by this analytical
 * per-step acceptance rate ("The Speed Claim Nobody's Really Questioning", sections "The
 * Semi-Autoregressive Trick" and "The Real Innovation: Confidence-Scheduled Verification").
 *
 * Rows: every drafted position (draft_tokens[b][j] >= 0).  q_j = softmax((base row j + bias of
 * prev) / T_b) with prev = x0[b] at j = 0 (none if x0 is NULL or -1), else draft_tokens[b][j-1];
 * p_j = softmax(target row j / T_b).  Other positions, and every position of a request with a bad
 * temperature or x0, get NaN.  lse_q / lse_p (may be NULL) receive the two log-normalisers.
 * --------------------------------------------------------------------------------------- */
static void stats_row(const oracle_dims* d, const void* base_logits, const void* target_logits,
                      const void* A, const void* W, const int32_t* x0, const int32_t* draft_tokens,
                      const float* temp, int64_t row, double* s, double* t, double* out3) {
  const int32_t K = d->K, V = d->V, R = d->R;
  const int32_t b = (int32_t)(row / K), j = (int32_t)(row % K);
  out3[0] = out3[1] = out3[2] = NAN;
  if (draft_tokens[row] < 0) return;
  const double T = (double)temp[b];
  const int32_t xb = x0 ? x0[b] : -1;
  if (!(T > 0.0) || !isfinite(T) || xb < -1 || xb >= V) return;
  const int32_t prev = (j == 0) ? xb : draft_tokens[row - 1];
  if (j > 0 && prev < 0) return;
  oracle_bias(A, W, d->dtype, V, R, prev, s);
  for (int32_t v = 0; v < V; v++) {
    s[v] = (load_elem(base_logits, d->dtype, ((size_t)b * K + j) * V + v) + s[v]) / T;
    t[v] = load_elem(target_logits, d->dtype, ((size_t)b * (K + 1) + j) * V + v) / T;
  }
  const double lq = oracle_lse(s, V), lp = oracle_lse(t, V);
  double a = 0.0;
  for (int32_t v = 0; v < V; v++) {
    const double q = exp(s[v] - lq), p = exp(t[v] - lp);
    a += (p < q) ? p : q;
  }
  out3[0] = a;
  out3[1] = lq;
  out3[2] = lp;
}

int spec_accept_stats_ref(const oracle_dims* d, const void* base_logits, const void* target_logits,
                          const void* A, const void* W, const int32_t* x0, const int32_t* draft_tokens,
                          const float* temp, double* alpha, double* lse_q, double* lse_p, int nthreads) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!base_logits || !target_logits || !A || !W || !draft_tokens || !temp || !alpha) return -1;
  const int64_t n = (int64_t)d->B * d->K;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)d->V);
    double* t = (double*)malloc(sizeof(double) * (size_t)d->V);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t row = 0; row < n; row++) {
      double o[3];
      stats_row(d, base_logits, target_logits, A, W, x0, draft_tokens, temp, row, s, t, o);
      alpha[row] = o[0];
      if (lse_q) lse_q[row] = o[1];
      if (lse_p) lse_p[row] = o[2];
    }
    free(s);
    free(t);
  }
  (void)nthreads;
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Expected calibration error of the confidences as prefix-survival estimates.
 *
 * The scheduler reads the running product of the per-position confidences as the probability
 * that the draft prefix through position j survives verification, so it needs calibrated
 * magnitudes, and the calibration error of that cumulative prefix probability is what sequential
 * temperature scaling minimises ("DSpark turns speculation into a scheduler", section "Confidence
 * is a serving primitive"; "The Speed Claim...", section "The Real Innovation": the pages report
 * the calibration error falling from several percent to around one percent).
 *
 * Pairs: every verified position j < verify_len[b] of every valid request (accepted_len[b] >= 0).
 * Prediction P_{b,j} = prod_{i<=j} conf[b][i] (fp64, left to right); outcome y_{b,j} = 1 when the
 * prefix through j survived (j < accepted_len[b]), else 0.  nbins equal-width bins on [0, 1]:
 * bin = floor(P * nbins) clamped to [0, nbins - 1].  ECE = sum over bins of
 * (n_bin / N) * |mean P - mean y| over the bin's pairs; 0 when there is no pair.
 * --------------------------------------------------------------------------------------- */
double spec_calibration_error_ref(const float* conf, const int32_t* verify_len, const int32_t* accepted_len,
                                  int32_t B, int32_t K, int32_t nbins, int64_t* n_pairs) {
  if (nbins < 1) return NAN;
  double* sp = (double*)calloc((size_t)nbins, sizeof(double));
  double* sy = (double*)calloc((size_t)nbins, sizeof(double));
  int64_t* cnt = (int64_t*)calloc((size_t)nbins, sizeof(int64_t));
  int64_t N = 0;
  for (int32_t b = 0; b < B; b++) {
    if (accepted_len[b] < 0) continue;
    double P = 1.0;
    for (int32_t j = 0; j < verify_len[b] && j < K; j++) {
      P *= (double)conf[(size_t)b * K + j];
      int64_t m = (int64_t)floor(P * nbins);
      if (m < 0) m = 0;
      if (m > nbins - 1) m = nbins - 1;
      sp[m] += P;
      sy[m] += (j < accepted_len[b]) ? 1.0 : 0.0;
      cnt[m] += 1;
      N += 1;
    }
  }
  double ece = 0.0;
  for (int32_t m = 0; m < nbins; m++)
    if (cnt[m] > 0) ece += ((double)cnt[m] / (double)N) * fabs(sp[m] / cnt[m] - sy[m] / cnt[m]);
  if (n_pairs) *n_pairs = N;
  free(sp);
  free(sy);
  free(cnt);
  return N > 0 ? ece : 0.0;
}

/* ---------------------------------------------------------------------------------------
 * Hardware-aware prefix scheduler.
 *
 * The scheduler reads the confidences as prefix-survival probabilities P_{b,j} = prod_{i<=j}
 * c_{b,i}, weighs the expected accepted tokens of each verification position against a profiled
 * throughput curve of the target engine, and picks per-request prefix lengths under the current
 * batch pressure; an early-stopping rule (a request's prefix ends at its first position that
 * fails) keeps it lossless ("DSpark turns speculation into a scheduler", section "Confidence is a
 * serving primitive": which verification tokens have positive expected return given the batch
 * pressure; "The Speed Claim...", section "The Real Innovation": verify more when GPUs are idle,
 * fewer when they are busy, early stopping stays lossless).
 *
 * Reading written out here:
 *   M_{b,j} = min_{i<=j} P_{b,i} (fp64): position j is kept at threshold tau iff M_{b,j} >= tau,
 *     so every kept set is a prefix and a prefix ends at its first failing position;
 *   thresholds on a grid: g = 1..nbins with position j kept iff bin(M) >= g, where
 *     bin(M) = min(floor(fl(M * nbins)), nbins) (fp64 product), plus g = nbins + 1 = keep nothing;
 *   n_g = kept positions, S_g = sum of P over them; expected emitted tokens E_g = B + S_g (one
 *     correction or bonus token per request plus the expected accepted drafts);
 *   step_time[n] (n = 0..B K) = seconds of one target verification step with n draft tokens in
 *     the batch; goodput G_g = E_g / step_time[n_g];
 *   g* = argmax G_g, ties to the larger g (fewer tokens); verify_len[b] = number of leading
 *     positions with bin(M_{b,j}) >= g*.
 * out[0] = g* / nbins (the threshold; > 1 when nothing is kept), out[1] = n*, out[2] = E*,
 * out[3] = G*.  Returns 0, or -1 for bad arguments.
 * --------------------------------------------------------------------------------------- */
static int64_t sched_bin(double M, int32_t nbins) {
  double f = floor(M * (double)nbins);
  if (!(f >= 0.0)) return 0;                 /* NaN or negative: the lowest bin */
  if (f > (double)nbins) return nbins;
  return (int64_t)f;
}

int spec_schedule_ref(const float* conf, int32_t B, int32_t K, const double* step_time, int32_t nbins,
                      int32_t* verify_len, double* out) {
  if (!conf || !step_time || !verify_len || !out || B < 1 || K < 1 || nbins < 1) return -1;
  int64_t* bins = (int64_t*)malloc(sizeof(int64_t) * (size_t)B * K);
  double* P = (double*)malloc(sizeof(double) * (size_t)B * K);
  for (int32_t b = 0; b < B; b++) {
    double p = 1.0, m = INFINITY;
    for (int32_t j = 0; j < K; j++) {
      p *= (double)conf[(size_t)b * K + j];
      if (p < m || isnan(p)) m = p;          /* running minimum; a NaN stays */
      P[(size_t)b * K + j] = p;
      bins[(size_t)b * K + j] = sched_bin(m, nbins);
    }
  }
  int32_t best_g = nbins + 1;
  double best_G = (double)B / step_time[0], best_E = (double)B;
  int64_t best_n = 0;
  for (int32_t g = nbins; g >= 1; g--) {       /* larger g first: ties keep the larger g */
    int64_t n = 0;
    double S = 0.0;
    for (int64_t i = 0; i < (int64_t)B * K; i++)
      if (bins[i] >= g) {
        n++;
        S += P[i];
      }
    const double E = (double)B + S, G = E / step_time[n];
    if (G > best_G) {
      best_G = G;
      best_g = g;
      best_n = n;
      best_E = E;
    }
  }
  for (int32_t b = 0; b < B; b++) {
    int32_t L = 0;
    while (L < K && bins[(size_t)b * K + L] >= best_g) L++;
    verify_len[b] = L;
  }
  out[0] = (double)best_g / (double)nbins;
  out[1] = (double)best_n;
  out[2] = best_E;
  out[3] = best_G;
  free(bins);
  free(P);
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Sequential temperature scaling of the confidence head.
 *
 * The head's raw confidences come out too high.  A prefix survives with the product of its
 * positions' confidences, so the temperatures are fitted one position at a time, first to last:
 * each one is the grid temperature giving the smallest calibration error of the running product
 * on a held-out set, with the positions before it kept at their fitted values ("DSpark turns
 * speculation into a scheduler", section "Confidence is a serving primitive"; "The Speed
 * Claim...", section "The Real Innovation", which reports the error falling from several percent
 * to around one percent after this post-hoc fit).
 *
 * Reading written out here:
 *   z [N, K]: the head's raw logits, c_{n,k}(T) = 1 / (1 + exp(-z_{n,k} / T));
 *   pairs of position k: sequences n with k < verify_len[n] and accepted_len[n] >= 0; prediction
 *     P_{n,k} = prod_{i<=k} c_{n,i}(T_i) (fp64), outcome 1 if k < accepted_len[n];
 *   ECE_k(T) over those pairs with nbins equal-width bins (the calibration error defined above,
 *     restricted to position k);
 *   T_k = the grid value with the smallest ECE_k (ties to the earlier grid entry), grid ascending;
 *   out: T [K], ece_before [K] (all T = 1), ece_after [K] (fitted).
 * --------------------------------------------------------------------------------------- */
static double ece_of(const double* P, const int32_t* y, int64_t n, int32_t nbins, double* sp, double* sy,
                     int64_t* cnt) {
  for (int32_t m = 0; m < nbins; m++) {
    sp[m] = 0.0;
    sy[m] = 0.0;
    cnt[m] = 0;
  }
  for (int64_t i = 0; i < n; i++) {
    int64_t m = (int64_t)floor(P[i] * nbins);
    if (m < 0) m = 0;
    if (m > nbins - 1) m = nbins - 1;
    sp[m] += P[i];
    sy[m] += (double)y[i];
    cnt[m] += 1;
  }
  double e = 0.0;
  for (int32_t m = 0; m < nbins; m++)
    if (cnt[m] > 0) e += ((double)cnt[m] / (double)n) * fabs(sp[m] / cnt[m] - sy[m] / cnt[m]);
  return n > 0 ? e : 0.0;
}

int spec_temperature_scaling_ref(const float* z, const int32_t* verify_len, const int32_t* accepted_len,
                                 int32_t N, int32_t K, const double* grid, int32_t G, int32_t nbins, double* T,
                                 double* ece_before, double* ece_after) {
  if (!z || !verify_len || !accepted_len || !grid || !T || N < 1 || K < 1 || G < 1 || nbins < 1) return -1;
  double* run = (double*)malloc(sizeof(double) * (size_t)N);      /* fitted product through k - 1 */
  double* run1 = (double*)malloc(sizeof(double) * (size_t)N);     /* product with every T = 1 */
  double* P = (double*)malloc(sizeof(double) * (size_t)N);
  int32_t* y = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  double* sp = (double*)malloc(sizeof(double) * (size_t)nbins);
  double* sy = (double*)malloc(sizeof(double) * (size_t)nbins);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)nbins);
  for (int32_t n = 0; n < N; n++) run[n] = run1[n] = 1.0;
  for (int32_t k = 0; k < K; k++) {
    int64_t m = 0;
    for (int32_t n = 0; n < N; n++)
      if (accepted_len[n] >= 0 && k < verify_len[n]) {
        idx[m] = n;
        y[m] = (k < accepted_len[n]) ? 1 : 0;
        m++;
      }
    /* before: every temperature 1 */
    for (int64_t i = 0; i < m; i++) {
      const double zz = (double)z[(size_t)idx[i] * K + k];
      P[i] = run1[idx[i]] * (1.0 / (1.0 + exp(-zz)));
    }
    if (ece_before) ece_before[k] = ece_of(P, y, m, nbins, sp, sy, cnt);
    int32_t best = 0;
    double best_e = INFINITY;
    for (int32_t g = 0; g < G; g++) {
      for (int64_t i = 0; i < m; i++) {
        const double zz = (double)z[(size_t)idx[i] * K + k];
        P[i] = run[idx[i]] * (1.0 / (1.0 + exp(-zz / grid[g])));
      }
      const double e = ece_of(P, y, m, nbins, sp, sy, cnt);
      if (e < best_e) {
        best_e = e;
        best = g;
      }
    }
    T[k] = grid[best];
    if (ece_after) ece_after[k] = best_e;
    for (int32_t n = 0; n < N; n++) {
      const double zz = (double)z[(size_t)n * K + k];
      run[n] *= 1.0 / (1.0 + exp(-zz / grid[best]));
      run1[n] *= 1.0 / (1.0 + exp(-zz));
    }
  }
  free(run); free(run1); free(P); free(y); free(idx); free(sp); free(sy); free(cnt);
  return 0;
}
