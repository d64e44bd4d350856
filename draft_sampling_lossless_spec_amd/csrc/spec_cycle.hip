// spec_cycle.hip -- MI355X (gfx950) kernels and C ABI of one batched speculation cycle.
//
// Method (per request; sources named in include/spec_cycle.h): prefix cut on the fp64 running
// product of confidences; semi-autoregressive draft x_j ~ softmax((base_j + A[x_{j-1}] W)/T);
// accept while u_j < p_j(x_j)/q_j(x_j); correction from norm(max(0, p - q)) at the first
// rejection, or a bonus token from p when every verified draft survives.
//
// Device schedule.  The draft chain is sequential in the position (the bias of position s+1
// needs x_s), and every position needs a full pass over the Markov factor W, so the cycle runs
// as K+1 steps, two kernels each, all enqueued by one host call:
//   k_sweep(s)  one pass over the rows active at step s.  "Bias rows" (DRAFT rows of position
//               s and CORRECT rows of a position rejected at s-1) need A[prev] . W: a kind-A
//               work item owns 256 vocabulary columns, keeps their W fragments in VGPRs and
//               loops over up to 256 bias rows in sub-blocks of 32 (A rows staged in LDS),
//               computing the bias with v_mfma_f32_32x32x16_bf16 directly in the layout the
//               element-wise sweep consumes (bias never leaves registers).  "Plain rows"
//               (LSEP: the target row of the position being verified; BONUS) are streamed by
//               kind-B items of 16384 columns, 64 consecutive columns (one noise chunk) per
//               thread.  Every item writes one 16-byte partial per row: the log-normaliser of
//               its columns plus the best perturbed score and its index.
//   k_merge(s)  one workgroup per request: reduces its rows' partials, finishes the sampler
//               (CHUNKED: re-reads the winning 64-column chunk), takes the accept decision,
//               finalises tokens, and writes the request's roles for step s+1.
// Each sweep workgroup rebuilds the compact row lists of its step from the per-request role
// bytes with a block scan (cheap for B <= 8192), so no extra planning launch is needed.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "spec_cycle.h"
#include "device_common.h"

namespace spec {

enum : int { RO_DRAFT = 1, RO_CORRECT = 2, RO_LSEP = 4, RO_BONUS = 8 };
enum : int { PH_ALIVE = 0, PH_REJECTED = 1, PH_DONE = 2, PH_INVALID = 3 };

constexpr int NT = 256;             // threads per workgroup
constexpr int SUB = 32;             // bias rows per MFMA sub-block
constexpr int NSUB = 8;             // sub-blocks per kind-A item
constexpr int RB = SUB * NSUB;      // bias rows per kind-A item
constexpr int TILE_A = 256;         // vocabulary columns per kind-A item: 4 waves x 64
constexpr int TILE_B = NT * CHUNK;  // vocabulary columns per kind-B item
constexpr int MAX_B = 8192;
constexpr int MAX_K = 32;
constexpr int MAX_R = 256;
constexpr int A_PAD = 8;            // bf16 elements of LDS row padding (kills bank conflicts)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Params {
  int B, K, V, R, dtype, noise;
  const void* base;
  const void* target;
  const void* A;
  const void* W;
  const int32_t* x0;
  const float* conf;
  const float* temp;
  float threshold;
  uint64_t seed;
  int64_t req_off;
  int32_t* accepted_len;
  int32_t* tokens;
  int32_t* d_verify_len;
  int32_t* d_draft;
  float* d_logq;
  float* d_logp;
  // workspace
  int32_t* L;
  int32_t* acc;
  int32_t* phase;
  uint8_t* roles;      // [2][B], step parity
  int32_t* slots;      // [3][B]: bias slot of DRAFT row, bias slot of CORRECT row, plain slot
  int32_t* xs;         // [B][K]
  float* lse_q;        // [B][K]
  float* logq;         // [B][K]
  float* lse_p;        // [B][K+1]
  float* logp;         // [B][K]
  float4* part_bias;   // [2B][nrA]
  float4* part_bias2;  // [2B][nrA]  CORRECT rows: target-row fallback
  float4* part_plain;  // [B][nrB]
  int nrA, nrB, nrA_xcd, nrb, gridA;
};

// ------------------------------------------------------------------------------------------
// element loads
// ------------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float load1(const void* p, size_t i) {
  if (DT == SPEC_FP32) return ((const float*)p)[i];
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

// 16 consecutive elements starting at column v of a row; columns >= V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load16(const void* row, int v, int V, float (&x)[16]) {
  if (VEC && v + 16 <= V) {
    if (DT == SPEC_BF16) {
      const u32x4* q = (const u32x4*)((const uint16_t*)row + v);
      u32x4 a = __builtin_nontemporal_load(q);
      u32x4 b = __builtin_nontemporal_load(q + 1);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        x[2 * i] = bf16_lo(a[i]);
        x[2 * i + 1] = bf16_hi(a[i]);
        x[8 + 2 * i] = bf16_lo(b[i]);
        x[8 + 2 * i + 1] = bf16_hi(b[i]);
      }
    } else {
      const u32x4* q = (const u32x4*)((const float*)row + v);
#pragma unroll
      for (int k = 0; k < 4; k++) {
        u32x4 a = __builtin_nontemporal_load(q + k);
#pragma unroll
        for (int i = 0; i < 4; i++) x[4 * k + i] = __uint_as_float(a[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) x[i] = (v + i < V) ? load1<DT>(row, (size_t)(v + i)) : -INFINITY;
  }
}

// ------------------------------------------------------------------------------------------
// step-0 set-up: validation, prefix cut, state, output defaults
// ------------------------------------------------------------------------------------------
__global__ void k_init(Params p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  const int K = p.K;
  const float T = p.temp[b];
  const int x0 = p.x0 ? p.x0[b] : -1;
  const bool valid = (T > 0.0f) && isfinite(T) && x0 >= -1 && x0 < p.V;
  // prefix cut: keep position j while the fp64 running product of confidences is >= threshold
  double P = 1.0;
  int L = 0;
  for (int j = 0; j < K; j++) {
    P *= (double)p.conf[(size_t)b * K + j];
    if (!(P >= (double)p.threshold)) break;
    L = j + 1;
  }
  p.L[b] = L;
  p.acc[b] = 0;
  p.phase[b] = valid ? PH_ALIVE : PH_INVALID;
  p.roles[b] = valid ? (uint8_t)(L > 0 ? (RO_DRAFT | RO_LSEP) : RO_BONUS) : (uint8_t)0;
  p.roles[p.B + b] = 0;
  p.accepted_len[b] = -1;
  for (int j = 0; j <= K; j++) p.tokens[(size_t)b * (K + 1) + j] = -1;
  if (p.d_verify_len) p.d_verify_len[b] = valid ? L : -1;
  for (int j = 0; j < K; j++) {
    if (p.d_draft) p.d_draft[(size_t)b * K + j] = -1;
    if (p.d_logq) p.d_logq[(size_t)b * K + j] = NAN;
    if (p.d_logp) p.d_logp[(size_t)b * K + j] = NAN;
  }
}

// ------------------------------------------------------------------------------------------
// block-wide exclusive scan of packed counters (three 16-bit lanes in a uint64)
// ------------------------------------------------------------------------------------------
__device__ uint64_t block_excl_scan(uint64_t v, uint64_t* tmp, uint64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  uint64_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; i++) {
    uint64_t t = tmp[i];
    off += (i < w) ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return off + x - v;
}

struct RowMeta {       // one bias row of a sub-block, staged in LDS
  int b, j, role, prev, slot;
  float invT, lse_p, lse_q;
  uint64_t key1, key2;
};

struct Lists {
  int n_draft, n_correct, n_plain;
};

// Scan the role bytes of step s; fill `bias_req`/`bias_role` for bias slots [lo, lo+n) and
// `plain_req` for one plain slot; workgroup 0 also publishes every request's slots.
__device__ Lists build_lists(const Params& p, const uint8_t* roles, int bias_lo, int bias_n, int plain_slot,
                             int* bias_req, int* bias_role, int* plain_req, uint64_t* tmp) {
  const int per = (p.B + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  uint64_t cnt = 0;
  for (int i = 0; i < per; i++) {
    int b = b0 + i;
    if (b < p.B) {
      int r = roles[b];
      cnt += (uint64_t)((r & RO_DRAFT) ? 1 : 0) | ((uint64_t)((r & RO_CORRECT) ? 1 : 0) << 16) |
             ((uint64_t)((r & (RO_LSEP | RO_BONUS)) ? 1 : 0) << 32);
    }
  }
  uint64_t tot;
  uint64_t pre = block_excl_scan(cnt, tmp, &tot);
  Lists ls;
  ls.n_draft = (int)(tot & 0xFFFF);
  ls.n_correct = (int)((tot >> 16) & 0xFFFF);
  ls.n_plain = (int)((tot >> 32) & 0xFFFF);
  int d = (int)(pre & 0xFFFF), c = (int)((pre >> 16) & 0xFFFF), q = (int)((pre >> 32) & 0xFFFF);
  const bool publish = (blockIdx.x == 0);
  for (int i = 0; i < per; i++) {
    int b = b0 + i;
    if (b >= p.B) break;
    int r = roles[b];
    int sd = -1, sc = -1, sp = -1;
    if (r & RO_DRAFT) sd = d++;
    if (r & RO_CORRECT) sc = ls.n_draft + c++;
    if (r & (RO_LSEP | RO_BONUS)) sp = q++;
    if (sd >= bias_lo && sd < bias_lo + bias_n) { bias_req[sd - bias_lo] = b; bias_role[sd - bias_lo] = RO_DRAFT; }
    if (sc >= bias_lo && sc < bias_lo + bias_n) { bias_req[sc - bias_lo] = b; bias_role[sc - bias_lo] = RO_CORRECT; }
    if (sp >= 0 && sp == plain_slot) *plain_req = b;
    if (publish) {
      p.slots[b] = sd;
      p.slots[p.B + b] = sc;
      p.slots[2 * p.B + b] = sp;
    }
  }
  __syncthreads();
  return ls;
}

// ------------------------------------------------------------------------------------------
// kind A: bias rows (DRAFT / CORRECT) over 256 columns
// ------------------------------------------------------------------------------------------
struct WaveOut {        // one wave's result for one row over its 64 columns
  float4 a;             // {log-mass, best score, best index (bits), aux}
  float4 b;             // CORRECT: target-row fallback {lse, best score, best index, 0}
};

// Element-wise work of one lane on its 32 columns (16 per fragment, 2 fragments) of one row.
// z[i] = base + bias (unscaled), col(i) = v0 + 32*(i/16) + (i%16).  Returns the lane's
// contribution; the two lanes of a row (h = 0, 1) are merged by the caller.
template <int NOISE>
__device__ __forceinline__ void lane_bias_row(const RowMeta& rm, const float (&z)[32], const float (&t)[32], int v0,
                                              int V, int chunk, float4& oa, float4& ob) {
  const float invT = rm.invT;
  float s[32];
#pragma unroll
  for (int i = 0; i < 32; i++) {
    int v = v0 + 32 * (i >> 4) + (i & 15);
    s[i] = (v < V) ? z[i] * invT : -INFINITY;
  }
  if (rm.role == RO_DRAFT) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; i++) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.0f;
    if (mx != -INFINITY) {
      const float mo = mx * LOG2E;
#pragma unroll
      for (int i = 0; i < 32; i++) sum += exp2f(fmaf(s[i], LOG2E, -mo));
    } else {
#pragma unroll
      for (int i = 0; i < 32; i++) sum += s[i];   // every value -inf or NaN: keep a NaN visible
    }
    sum += __shfl_xor(sum, 32, 64);
    const float lse = (mx == -INFINITY) ? sum : mx + log2f(sum) * LN2;
    if (NOISE == SPEC_NOISE_CHUNKED) {
      float score = -INFINITY;
      if (lse != -INFINITY) score = lse + gumbel_bits(bits_at(rm.key1, (uint32_t)chunk));
      oa = make_float4(lse, score, __int_as_float(chunk), 0.0f);
    } else {
      float best = -INFINITY, bests = 0.0f;
      int bestv = -1;
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        int v = v0 + 32 * (i >> 4) + (i & 15);   // even column: one word serves v and v+1
        if (v >= V) continue;
        uint64_t w = pair_word(rm.key2, (uint32_t)v >> 1);
        uint32_t bb[2] = {(uint32_t)(w >> 32), (uint32_t)w};
#pragma unroll
        for (int e = 0; e < 2; e++) {
          float sv = s[i + e];
          if (v + e >= V || sv == -INFINITY) continue;
          if (sv + gumbel_bound(bb[e]) + 1e-3f < best) continue;
          float zz = sv + gumbel_bits(bb[e]);
          if (better(zz, v + e, best, bestv)) { best = zz; bestv = v + e; bests = sv; }
        }
      }
      float ob_ = __shfl_xor(best, 32, 64);
      int ov = __shfl_xor(bestv, 32, 64);
      float os = __shfl_xor(bests, 32, 64);
      if (ov >= 0 && (bestv < 0 || better(ob_, ov, best, bestv))) { best = ob_; bestv = ov; bests = os; }
      oa = make_float4(lse, best, __int_as_float(bestv), bests);
    }
    ob = make_float4(0, 0, 0, 0);
  } else {  // RO_CORRECT: residual norm(max(0, p - q)) and the target-row fallback
    float tt[32];
#pragma unroll
    for (int i = 0; i < 32; i++) {
      int v = v0 + 32 * (i >> 4) + (i & 15);
      tt[i] = (v < V) ? t[i] * invT : -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; i++) mt = fmaxf(mt, tt[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    float st = 0.0f, mass = 0.0f;
    const float mo = mt * LOG2E;
#pragma unroll
    for (int i = 0; i < 32; i++) {
      st += (mt != -INFINITY) ? exp2f(fmaf(tt[i], LOG2E, -mo)) : tt[i];
      float lp = tt[i] - rm.lse_p, lq = s[i] - rm.lse_q;
      if (lp > lq) mass += exp2f(lp * LOG2E) - exp2f(lq * LOG2E);
    }
    st += __shfl_xor(st, 32, 64);
    mass += __shfl_xor(mass, 32, 64);
    const float lse_t = (mt == -INFINITY) ? st : mt + log2f(st) * LN2;
    const float lmass = (mass > 0.0f) ? log2f(mass) * LN2 : -INFINITY;
    if (NOISE == SPEC_NOISE_CHUNKED) {
      float g = gumbel_bits(bits_at(rm.key1, (uint32_t)chunk));
      oa = make_float4(lmass, lmass == -INFINITY ? -INFINITY : lmass + g, __int_as_float(chunk), 0.0f);
      ob = make_float4(lse_t, lse_t == -INFINITY ? -INFINITY : lse_t + g, __int_as_float(chunk), 0.0f);
    } else {
      float br = -INFINITY, bp = -INFINITY;
      int vr = -1, vp = -1;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        int v = v0 + 32 * (i >> 4) + (i & 15);
        if (v >= V) continue;
        float g = gumbel_bits(bits_at(rm.key2, (uint32_t)v));
        float lp = tt[i] - rm.lse_p, lq = s[i] - rm.lse_q;
        if (lp > lq) {
          float sc = lp + logf(-expm1f(lq - lp)) + g;
          if (better(sc, v, br, vr)) { br = sc; vr = v; }
        }
        if (tt[i] != -INFINITY) {
          float sc = tt[i] + g;
          if (better(sc, v, bp, vp)) { bp = sc; vp = v; }
        }
      }
      float o1 = __shfl_xor(br, 32, 64);
      int i1 = __shfl_xor(vr, 32, 64);
      if (i1 >= 0 && (vr < 0 || better(o1, i1, br, vr))) { br = o1; vr = i1; }
      float o2 = __shfl_xor(bp, 32, 64);
      int i2 = __shfl_xor(vp, 32, 64);
      if (i2 >= 0 && (vp < 0 || better(o2, i2, bp, vp))) { bp = o2; vp = i2; }
      oa = make_float4(lmass, br, __int_as_float(vr), 0.0f);
      ob = make_float4(lse_t, bp, __int_as_float(vp), 0.0f);
    }
  }
}

// merge of two partial records {log-mass, best score, best index, aux}
__device__ __forceinline__ float4 merge_part(float4 x, float4 y) {
  float4 r;
  r.x = lse2(x.x, y.x);
  int ix = __float_as_int(x.z), iy = __float_as_int(y.z);
  bool take_y = (iy >= 0) && (ix < 0 || better(y.y, iy, x.y, ix));
  r.y = take_y ? y.y : x.y;
  r.z = take_y ? y.z : x.z;
  r.w = take_y ? y.w : x.w;
  return r;
}

template <int DT, int NOISE, bool VEC>
__device__ void kind_a(const Params& p, int s, const Lists& ls, int rb, int range, const int* bias_req,
                       const int* bias_role) {
  __shared__ __attribute__((aligned(16))) uint16_t sA16[SUB][MAX_R + A_PAD];
  __shared__ float sA32[DT == SPEC_FP32 ? SUB : 1][DT == SPEC_FP32 ? (MAX_R + 4) : 1];
  __shared__ RowMeta meta[SUB];
  __shared__ WaveOut red[NT / 64][SUB];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int V = p.V, R = p.R, K = p.K;
  const int vt0 = range * TILE_A;
  const int vw = vt0 + 64 * wave;          // this wave's 64 columns: one noise chunk
  const int chunk = vw / CHUNK;
  const int n_bias = ls.n_draft + ls.n_correct;
  const int row0 = rb * RB;
  const int nrows = min(RB, n_bias - row0);
  const int T16 = R / 16;                  // MFMA k-steps (bf16)

  // W fragments of this wave, resident for the whole item: the MFMA A-operand row i of
  // fragment f is column vw + 32f + perm(i), perm chosen so that accumulator q of lane l holds
  // column vw + 32f + 16*(l/32) + q.
  bf16x8 wf[2][16];
  if (DT == SPEC_BF16) {
    const int i = m;
    const int col_in = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const int kb = h * (R / 2);
#pragma unroll
    for (int f = 0; f < 2; f++) {
      const int v = vw + 32 * f + col_in;
#pragma unroll
      for (int t = 0; t < 16; t++) {
        if (t < T16) {
          if (v < V) {
            wf[f][t] = *(const bf16x8*)((const uint16_t*)p.W + (size_t)v * R + kb + 8 * t);
          } else {
            wf[f][t] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
      }
    }
  }

  for (int sb = 0; sb * SUB < nrows; sb++) {
    const int rows_here = min(SUB, nrows - sb * SUB);
    __syncthreads();
    // row metadata
    if (threadIdx.x < SUB) {
      RowMeta rm;
      const int r = threadIdx.x;
      if (r < rows_here) {
        const int b = bias_req[sb * SUB + r];
        const int role = bias_role[sb * SUB + r];
        const int j = (role == RO_DRAFT) ? s : p.acc[b];
        const int prev = (j == 0) ? (p.x0 ? p.x0[b] : -1) : p.xs[(size_t)b * K + j - 1];
        const uint64_t g = (uint64_t)(p.req_off + b);
        rm.b = b;
        rm.j = j;
        rm.role = role;
        rm.prev = prev;
        rm.slot = row0 + sb * SUB + r;
        rm.invT = 1.0f / p.temp[b];
        if (role == RO_DRAFT) {
          rm.key1 = row_key(p.seed, g, (uint64_t)j, ST_DRAFT_C);
          rm.key2 = row_key(p.seed, g, (uint64_t)j, ST_DRAFT);
          rm.lse_p = 0.0f;
          rm.lse_q = 0.0f;
        } else {
          rm.key1 = row_key(p.seed, g, (uint64_t)j, ST_RESIDUAL_C);
          rm.key2 = row_key(p.seed, g, (uint64_t)j, ST_RESIDUAL);
          rm.lse_p = p.lse_p[(size_t)b * (K + 1) + j];
          rm.lse_q = p.lse_q[(size_t)b * K + j];
        }
      } else {
        rm.b = -1;
        rm.j = 0;
        rm.role = 0;
        rm.prev = -1;
        rm.slot = -1;
        rm.invT = 1.0f;
        rm.key1 = rm.key2 = 0;
        rm.lse_p = rm.lse_q = 0.0f;
      }
      meta[r] = rm;
    }
    __syncthreads();
    // stage the gathered A rows of the sub-block (zeros for "no previous token")
    if (DT == SPEC_BF16) {
      const int segs = R / 8;   // 16-byte segments per row
      for (int e = threadIdx.x; e < SUB * segs; e += NT) {
        const int r = e / segs, sg = e % segs;
        const int prev = meta[r].prev;
        u32x4 val = {0, 0, 0, 0};
        if (prev >= 0) val = *(const u32x4*)((const uint16_t*)p.A + (size_t)prev * R + 8 * sg);
        *(u32x4*)&sA16[r][8 * sg] = val;
      }
    } else {
      for (int e = threadIdx.x; e < SUB * R; e += NT) {
        const int r = e / R, k = e % R;
        const int prev = meta[r].prev;
        sA32[r][k] = (prev >= 0) ? ((const float*)p.A)[(size_t)prev * R + k] : 0.0f;
      }
    }
    __syncthreads();

    const RowMeta rm = meta[m];
    const bool active = rm.role != 0;
    // element loads of this lane's row: 16 columns per fragment
    float z[32], tv[32];
    const size_t brow = (size_t)(active ? rm.b : 0) * K + rm.j;
    const void* base_row = (const char*)p.base + brow * (size_t)V * (DT == SPEC_FP32 ? 4 : 2);
    const size_t trow = (size_t)(active ? rm.b : 0) * (K + 1) + rm.j;
    const void* targ_row = (const char*)p.target + trow * (size_t)V * (DT == SPEC_FP32 ? 4 : 2);
    const int v0 = vw + 16 * h;
#pragma unroll
    for (int f = 0; f < 2; f++) {
      float x16[16];
      if (active) load16<DT, VEC>(base_row, v0 + 32 * f, V, x16);
#pragma unroll
      for (int q = 0; q < 16; q++) z[16 * f + q] = active ? x16[q] : -INFINITY;
    }
    const bool corr = rm.role == RO_CORRECT;
    if (corr) {
#pragma unroll
      for (int f = 0; f < 2; f++) {
        float x16[16];
        load16<DT, VEC>(targ_row, v0 + 32 * f, V, x16);
#pragma unroll
        for (int q = 0; q < 16; q++) tv[16 * f + q] = x16[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 32; q++) tv[q] = 0.0f;
    }

    // Markov bias for the lane's 32 columns
    if (DT == SPEC_BF16) {
#pragma unroll
      for (int f = 0; f < 2; f++) {
        f32x16 accv = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        const int kb = h * (R / 2);
#pragma unroll
        for (int t = 0; t < 16; t++) {
          if (t < T16) {
            bf16x8 bop = *(const bf16x8*)&sA16[m][kb + 8 * t];
            accv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[f][t], bop, accv, 0, 0, 0);
          }
        }
#pragma unroll
        for (int q = 0; q < 16; q++) z[16 * f + q] += accv[q];
      }
    } else {
#pragma unroll
      for (int f = 0; f < 2; f++) {
#pragma unroll
        for (int q = 0; q < 16; q++) {
          const int v = v0 + 32 * f + q;
          float a = 0.0f;
          if (v < V) {
            const float* wr = (const float*)p.W + (size_t)v * R;
            for (int k = 0; k < R; k++) a = fmaf(sA32[m][k], wr[k], a);
          }
          z[16 * f + q] += a;
        }
      }
    }

    float4 oa = make_float4(-INFINITY, -INFINITY, __int_as_float(-1), 0.0f), ob = oa;
    if (active) lane_bias_row<NOISE>(rm, z, tv, v0, V, chunk, oa, ob);
    if (h == 0) {
      red[wave][m].a = oa;
      red[wave][m].b = ob;
    }
    __syncthreads();
    if (threadIdx.x < SUB && threadIdx.x < rows_here) {
      const int r = threadIdx.x;
      float4 pa = red[0][r].a, pb = red[0][r].b;
#pragma unroll
      for (int w = 1; w < NT / 64; w++) {
        pa = merge_part(pa, red[w][r].a);
        pb = merge_part(pb, red[w][r].b);
      }
      const int slot = meta[r].slot;
      p.part_bias[(size_t)slot * p.nrA + range] = pa;
      if (meta[r].role == RO_CORRECT) p.part_bias2[(size_t)slot * p.nrA + range] = pb;
    }
  }
}

// ------------------------------------------------------------------------------------------
// kind B: plain target rows (LSEP / BONUS), 64 consecutive columns (one chunk) per thread
// ------------------------------------------------------------------------------------------
template <int DT, int NOISE, bool VEC>
__device__ void kind_b(const Params& p, int s, int b, int pslot, int range) {
  __shared__ float4 redb[NT / 64];
  const int K = p.K, V = p.V;
  const int role = p.roles[(s & 1) * p.B + b] & (RO_LSEP | RO_BONUS);
  const int j = s;   // LSEP verifies position s; BONUS reads row L_b == s
  const float invT = 1.0f / p.temp[b];
  const size_t trow = (size_t)b * (K + 1) + j;
  const void* row = (const char*)p.target + trow * (size_t)V * (DT == SPEC_FP32 ? 4 : 2);
  const int c = range * (TILE_B / CHUNK) + threadIdx.x;
  const int v0 = c * CHUNK;
  float x[64];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    float x16[16];
    load16<DT, VEC>(row, v0 + 16 * q, V, x16);
#pragma unroll
    for (int i = 0; i < 16; i++) x[16 * q + i] = x16[i] * invT;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 64; i++) mx = fmaxf(mx, x[i]);
  float lse = 0.0f;
  if (mx != -INFINITY) {
    float sum = 0.0f;
    const float mo = mx * LOG2E;
#pragma unroll
    for (int i = 0; i < 64; i++) sum += exp2f(fmaf(x[i], LOG2E, -mo));
    lse = mx + log2f(sum) * LN2;
  } else {
#pragma unroll
    for (int i = 0; i < 64; i++) lse += x[i];   // every value -inf or NaN: keep a NaN visible
  }
  float4 part = make_float4(lse, -INFINITY, __int_as_float(-1), 0.0f);
  if (role == RO_BONUS) {
    const uint64_t g = (uint64_t)(p.req_off + b);
    if (NOISE == SPEC_NOISE_CHUNKED) {
      if (lse != -INFINITY) {
        const uint64_t k1 = row_key(p.seed, g, (uint64_t)j, ST_BONUS_C);
        part.y = lse + gumbel_bits(bits_at(k1, (uint32_t)c));
        part.z = __int_as_float(c);
      }
    } else {
      const uint64_t k2 = row_key(p.seed, g, (uint64_t)j, ST_BONUS);
      float best = -INFINITY;
      int bv = -1;
      for (int i = 0; i < 64; i += 2) {
        const int v = v0 + i;
        if (v >= V) break;
        const uint64_t w = pair_word(k2, (uint32_t)v >> 1);
        const uint32_t bb[2] = {(uint32_t)(w >> 32), (uint32_t)w};
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const float sv = x[i + e];
          if (v + e >= V || sv == -INFINITY) continue;
          if (sv + gumbel_bound(bb[e]) + 1e-3f < best) continue;
          const float zz = sv + gumbel_bits(bb[e]);
          if (better(zz, v + e, best, bv)) { best = zz; bv = v + e; }
        }
      }
      part.y = best;
      part.z = __int_as_float(bv);
    }
  }
  // workgroup reduction
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float4 y;
    y.x = __shfl_xor(part.x, o, 64);
    y.y = __shfl_xor(part.y, o, 64);
    y.z = __shfl_xor(part.z, o, 64);
    y.w = __shfl_xor(part.w, o, 64);
    part = merge_part(part, y);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) redb[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 r = redb[0];
#pragma unroll
    for (int w = 1; w < NT / 64; w++) r = merge_part(r, redb[w]);
    p.part_plain[(size_t)pslot * p.nrB + range] = r;
  }
}

template <int DT, int NOISE, bool VEC>
__global__ __launch_bounds__(NT, 2) void k_sweep(Params p, int s) {
  __shared__ int bias_req[RB];
  __shared__ int bias_role[RB];
  __shared__ int plain_req;
  __shared__ uint64_t scan_tmp[NT / 64];
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;

  // which item is this workgroup?
  int kind, rb = 0, range = 0, pslot = -1;
  if ((int)blockIdx.x < p.gridA) {
    kind = 0;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int ri = local / p.nrb;
    rb = local % p.nrb;
    range = ri * 8 + xcd;   // all row-blocks of one column range run on one XCD, back to back
  } else {
    kind = 1;
    const int id = blockIdx.x - p.gridA;
    pslot = id / p.nrB;
    range = id % p.nrB;
  }
  if (threadIdx.x == 0) plain_req = -1;
  const Lists ls = build_lists(p, roles, kind == 0 ? rb * RB : 0, kind == 0 ? RB : 0, pslot, bias_req, bias_role,
                               &plain_req, scan_tmp);
  if (kind == 0) {
    if (range >= p.nrA || rb * RB >= ls.n_draft + ls.n_correct) return;
    kind_a<DT, NOISE, VEC>(p, s, ls, rb, range, bias_req, bias_role);
  } else {
    if (pslot >= ls.n_plain) return;
    const int b = plain_req;
    kind_b<DT, NOISE, VEC>(p, s, b, pslot, range);
  }
}


// ------------------------------------------------------------------------------------------
// merge: one workgroup per request
// ------------------------------------------------------------------------------------------

// reduce n partial records with the whole workgroup; every thread gets the result
__device__ float4 reduce_parts(const float4* parts, int n, float4* lds) {
  float4 a = make_float4(-INFINITY, -INFINITY, __int_as_float(-1), 0.0f);
  for (int i = threadIdx.x; i < n; i += NT) a = merge_part(a, parts[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float4 y;
    y.x = __shfl_xor(a.x, o, 64);
    y.y = __shfl_xor(a.y, o, 64);
    y.z = __shfl_xor(a.z, o, 64);
    y.w = __shfl_xor(a.w, o, 64);
    a = merge_part(a, y);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = a;
  __syncthreads();
  float4 r = lds[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) r = merge_part(r, lds[w]);
  return r;
}

// argmax over one wave (score, index), smallest index on ties; result in every lane
__device__ __forceinline__ void wave_argmax(float& sc, int& ix, float& aux) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float s2 = __shfl_xor(sc, o, 64);
    int i2 = __shfl_xor(ix, o, 64);
    float a2 = __shfl_xor(aux, o, 64);
    if (i2 >= 0 && (ix < 0 || better(s2, i2, sc, ix))) {
      sc = s2;
      ix = i2;
      aux = a2;
    }
  }
}

// scaled draft logit of column v: (base + A[prev] . W[v]) / T, bias accumulated in fp32
template <int DT>
__device__ float draft_logit(const Params& p, const void* base_row, int prev, int v, float invT) {
  float bias = 0.0f;
  if (prev >= 0) {
    const int R = p.R;
    for (int k = 0; k < R; k++)
      bias = fmaf(load1<DT>(p.A, (size_t)prev * R + k), load1<DT>(p.W, (size_t)v * R + k), bias);
  }
  return (load1<DT>(base_row, (size_t)v) + bias) * invT;
}

enum { L2_DRAFT = 0, L2_TARGET = 1, L2_RESIDUAL = 2 };

// Level two of the CHUNKED sampler, run by wave 0: argmax over the columns of chunk c of
// (score_v + G(key2, v)).  Returns the column and (in aux) its scaled draft logit for DRAFT.
template <int DT>
__device__ int level_two(const Params& p, int kind, int c, uint64_t key2, const void* base_row,
                         const void* targ_row, int prev, float invT, float lse_p, float lse_q, float* aux_out) {
  const int lane = threadIdx.x & 63;
  const int v = c * CHUNK + lane;
  float sc = -INFINITY, aux = 0.0f;
  int ix = -1;
  if (c >= 0 && v < p.V) {
    const float g = gumbel_bits(bits_at(key2, (uint32_t)v));
    if (kind == L2_DRAFT) {
      const float sv = draft_logit<DT>(p, base_row, prev, v, invT);
      if (sv != -INFINITY) {
        sc = sv + g;
        ix = v;
        aux = sv;
      }
    } else if (kind == L2_TARGET) {
      const float tv = load1<DT>(targ_row, (size_t)v) * invT;
      if (tv != -INFINITY) {
        sc = tv + g;
        ix = v;
      }
    } else {
      const float sv = draft_logit<DT>(p, base_row, prev, v, invT);
      const float tv = load1<DT>(targ_row, (size_t)v) * invT;
      const float lp = tv - lse_p, lq = sv - lse_q;
      if (lp > lq) {
        sc = lp + logf(-expm1f(lq - lp)) + g;
        ix = v;
      }
    }
  }
  wave_argmax(sc, ix, aux);
  if (aux_out) *aux_out = aux;
  return ix;
}

template <int DT, int NOISE>
__global__ __launch_bounds__(NT) void k_merge(Params p, int s) {
  __shared__ float4 red[NT / 64];
  __shared__ int sh_tok;
  __shared__ float sh_aux;
  const int b = blockIdx.x;
  const int B = p.B, K = p.K, V = p.V;
  const int roles = p.roles[(size_t)(s & 1) * B + b];
  uint8_t* roles_next = p.roles + (size_t)((s + 1) & 1) * B;
  if (roles == 0) {
    if (threadIdx.x == 0) roles_next[b] = 0;
    return;
  }
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const float invT = 1.0f / p.temp[b];
  const uint64_t g = (uint64_t)(p.req_off + b);
  const int x0 = p.x0 ? p.x0[b] : -1;
  const int L = p.L[b];
  int phase = p.phase[b];
  int acc = p.acc[b];
  bool invalid = false, rejected_now = false;
  int final_tok = -1;
  float logq_s = NAN;
  int x_s = -1;

  if (roles & RO_DRAFT) {
    const int slot = p.slots[b];
    const float4 tot = reduce_parts(p.part_bias + (size_t)slot * p.nrA, p.nrA, red);
    const float lse_q = tot.x;
    if (!isfinite(lse_q)) {
      invalid = true;
    } else {
      float sx;
      if (NOISE == SPEC_NOISE_CHUNKED) {
        const int prev = (s == 0) ? x0 : p.xs[(size_t)b * K + s - 1];
        const void* base_row = (const char*)p.base + ((size_t)b * K + s) * V * esz;
        const uint64_t key2 = row_key(p.seed, g, (uint64_t)s, ST_DRAFT);
        if (threadIdx.x < 64) {
          float aux;
          const int x = level_two<DT>(p, L2_DRAFT, __float_as_int(tot.z), key2, base_row, nullptr, prev, invT, 0.f,
                                      0.f, &aux);
          if (threadIdx.x == 0) {
            sh_tok = x;
            sh_aux = aux;
          }
        }
        __syncthreads();
        x_s = sh_tok;
        sx = sh_aux;
      } else {
        x_s = __float_as_int(tot.z);
        sx = tot.w;
      }
      if (x_s < 0) {
        invalid = true;
      } else {
        logq_s = sx - lse_q;
        if (threadIdx.x == 0) {
          p.xs[(size_t)b * K + s] = x_s;
          p.lse_q[(size_t)b * K + s] = lse_q;
          p.logq[(size_t)b * K + s] = logq_s;
          if (p.d_draft) p.d_draft[(size_t)b * K + s] = x_s;
          if (p.d_logq) p.d_logq[(size_t)b * K + s] = logq_s;
        }
      }
    }
  }

  if (!invalid && (roles & RO_LSEP)) {
    const int slot = p.slots[2 * B + b];
    const float4 tot = reduce_parts(p.part_plain + (size_t)slot * p.nrB, p.nrB, red);
    const float lse_p = tot.x;
    if (!isfinite(lse_p) || x_s < 0) {
      invalid = true;
    } else {
      const void* targ_row = (const char*)p.target + ((size_t)b * (K + 1) + s) * V * esz;
      const float logp_s = load1<DT>(targ_row, (size_t)x_s) * invT - lse_p;
      const uint32_t ub = bits_at(row_key(p.seed, g, (uint64_t)s, ST_ACCEPT), 0);
      const double u = ((double)ub + 0.5) * 0x1p-32;
      const double ratio = exp((double)logp_s - (double)logq_s);
      if (u < ratio) {
        acc = s + 1;
      } else {
        phase = PH_REJECTED;
        rejected_now = true;
      }
      if (threadIdx.x == 0) {
        p.lse_p[(size_t)b * (K + 1) + s] = lse_p;
        p.logp[(size_t)b * K + s] = logp_s;
        if (p.d_logp) p.d_logp[(size_t)b * K + s] = logp_s;
      }
    }
  }

  if (!invalid && (roles & RO_BONUS)) {
    const int slot = p.slots[2 * B + b];
    const float4 tot = reduce_parts(p.part_plain + (size_t)slot * p.nrB, p.nrB, red);
    if (!isfinite(tot.x)) {
      invalid = true;
    } else {
      if (NOISE == SPEC_NOISE_CHUNKED) {
        const void* targ_row = (const char*)p.target + ((size_t)b * (K + 1) + s) * V * esz;
        const uint64_t key2 = row_key(p.seed, g, (uint64_t)s, ST_BONUS);
        if (threadIdx.x < 64) {
          const int y = level_two<DT>(p, L2_TARGET, __float_as_int(tot.z), key2, nullptr, targ_row, -1, invT, 0.f,
                                      0.f, nullptr);
          if (threadIdx.x == 0) sh_tok = y;
        }
        __syncthreads();
        final_tok = sh_tok;
      } else {
        final_tok = __float_as_int(tot.z);
      }
      if (final_tok < 0) invalid = true;
    }
  }

  if (!invalid && (roles & RO_CORRECT)) {
    const int j = acc;   // rejected position
    const int slot = p.slots[B + b];
    const float4 prim = reduce_parts(p.part_bias + (size_t)slot * p.nrA, p.nrA, red);
    const float4 sec = reduce_parts(p.part_bias2 + (size_t)slot * p.nrA, p.nrA, red);
    const bool residual = prim.x > -INFINITY;
    if (NOISE == SPEC_NOISE_CHUNKED) {
      const int prev = (j == 0) ? x0 : p.xs[(size_t)b * K + j - 1];
      const void* base_row = (const char*)p.base + ((size_t)b * K + j) * V * esz;
      const void* targ_row = (const char*)p.target + ((size_t)b * (K + 1) + j) * V * esz;
      const uint64_t key2 = row_key(p.seed, g, (uint64_t)j, ST_RESIDUAL);
      const float lse_p = p.lse_p[(size_t)b * (K + 1) + j];
      const float lse_q = p.lse_q[(size_t)b * K + j];
      if (threadIdx.x < 64) {
        const int y = residual ? level_two<DT>(p, L2_RESIDUAL, __float_as_int(prim.z), key2, base_row, targ_row, prev,
                                               invT, lse_p, lse_q, nullptr)
                               : level_two<DT>(p, L2_TARGET, __float_as_int(sec.z), key2, nullptr, targ_row, -1, invT,
                                               0.f, 0.f, nullptr);
        if (threadIdx.x == 0) sh_tok = y;
      }
      __syncthreads();
      final_tok = sh_tok;
    } else {
      final_tok = __float_as_int(residual ? prim.z : sec.z);
    }
    if (final_tok < 0) invalid = true;
  }

  if (threadIdx.x == 0) {
    int nr = 0;
    if (invalid) {
      phase = PH_INVALID;
      p.accepted_len[b] = -1;
      for (int i = 0; i <= K; i++) p.tokens[(size_t)b * (K + 1) + i] = -1;
      if (p.d_verify_len) p.d_verify_len[b] = -1;
      for (int i = 0; i < K; i++) {
        if (p.d_draft) p.d_draft[(size_t)b * K + i] = -1;
        if (p.d_logq) p.d_logq[(size_t)b * K + i] = NAN;
        if (p.d_logp) p.d_logp[(size_t)b * K + i] = NAN;
      }
    } else {
      if (final_tok >= 0) {
        for (int i = 0; i < acc; i++) p.tokens[(size_t)b * (K + 1) + i] = p.xs[(size_t)b * K + i];
        p.tokens[(size_t)b * (K + 1) + acc] = final_tok;
        p.accepted_len[b] = acc;
        phase = PH_DONE;
      }
      if (s + 1 < L) nr |= RO_DRAFT;
      if (phase == PH_ALIVE && acc == s + 1) nr |= (s + 1 < L) ? RO_LSEP : RO_BONUS;
      if (rejected_now) nr |= RO_CORRECT;
    }
    p.phase[b] = phase;
    p.acc[b] = acc;
    roles_next[b] = (uint8_t)nr;
  }
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
struct Layout {
  size_t off_L, off_acc, off_phase, off_roles, off_slots, off_xs, off_lse_q, off_logq, off_lse_p, off_logp,
      off_pbias, off_pbias2, off_pplain, total;
  int nrA, nrB, nrA_xcd, nrb, gridA, gridB;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool dims_ok(const spec_dims* d) {
  if (!d) return false;
  if (d->B < 1 || d->B > MAX_B || d->K < 1 || d->K > MAX_K || d->V < 2 || d->R < 1 || d->R > MAX_R) return false;
  return true;
}

static int dtype_ok(const spec_dims* d) {
  if (d->dtype != SPEC_FP32 && d->dtype != SPEC_BF16) return 0;
  if (d->noise != SPEC_NOISE_FLAT && d->noise != SPEC_NOISE_CHUNKED) return 0;
  if (d->dtype == SPEC_BF16 && (d->R % 16) != 0) return 0;
  return 1;
}

static Layout layout(const spec_dims* d) {
  Layout l;
  const size_t B = (size_t)d->B, K = (size_t)d->K;
  l.nrA = (d->V + TILE_A - 1) / TILE_A;
  l.nrB = (d->V + TILE_B - 1) / TILE_B;
  l.nrA_xcd = (l.nrA + 7) / 8;
  l.nrb = (int)((2 * B + RB - 1) / RB);
  l.gridA = 8 * l.nrA_xcd * l.nrb;
  l.gridB = (int)B * l.nrB;
  size_t o = 0;
  l.off_L = o; o = align256(o + 4 * B);
  l.off_acc = o; o = align256(o + 4 * B);
  l.off_phase = o; o = align256(o + 4 * B);
  l.off_roles = o; o = align256(o + 2 * B);
  l.off_slots = o; o = align256(o + 12 * B);
  l.off_xs = o; o = align256(o + 4 * B * K);
  l.off_lse_q = o; o = align256(o + 4 * B * K);
  l.off_logq = o; o = align256(o + 4 * B * K);
  l.off_lse_p = o; o = align256(o + 4 * B * (K + 1));
  l.off_logp = o; o = align256(o + 4 * B * K);
  l.off_pbias = o; o = align256(o + 16 * 2 * B * (size_t)l.nrA);
  l.off_pbias2 = o; o = align256(o + 16 * 2 * B * (size_t)l.nrA);
  l.off_pplain = o; o = align256(o + 16 * B * (size_t)l.nrB);
  l.total = o;
  return l;
}

static int arch_ok() {
  static int cache[64] = {0};   // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  if (dev >= 0 && dev < 64 && cache[dev] != 0) return cache[dev] > 0 ? SPEC_OK : SPEC_E_ARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SPEC_E_HIP;
  const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  if (dev >= 0 && dev < 64) cache[dev] = ok;
  return ok > 0 ? SPEC_OK : SPEC_E_ARCH;
}

// Kernel i of a cycle (0 = init, 1 + 2s = sweep of step s, 2 + 2s = merge of step s) may carry
// a start/stop event pair, attached to its own dispatch packet.
struct Timing {
  hipEvent_t* ev;
  int n;
  hipEvent_t start(int i) const { return (ev && 2 * i + 1 < n) ? ev[2 * i] : nullptr; }
  hipEvent_t stop(int i) const { return (ev && 2 * i + 1 < n) ? ev[2 * i + 1] : nullptr; }
};

template <int DT, int NOISE, bool VEC>
static void launch_steps(const Params& p, const Layout& l, hipStream_t st, const Timing& tm) {
  for (int s = 0; s <= p.K; s++) {
    const int ks = 1 + 2 * s, km = 2 + 2 * s;
    hipExtLaunchKernelGGL((k_sweep<DT, NOISE, VEC>), dim3(l.gridA + l.gridB), dim3(NT), 0, st, tm.start(ks),
                          tm.stop(ks), 0, p, s);
    hipExtLaunchKernelGGL((k_merge<DT, NOISE>), dim3(p.B), dim3(NT), 0, st, tm.start(km), tm.stop(km), 0, p, s);
  }
}

template <int DT>
static void launch_all(const Params& p, const Layout& l, bool vec, hipStream_t st, const Timing& tm) {
  if (p.noise == SPEC_NOISE_CHUNKED) {
    if (vec) launch_steps<DT, SPEC_NOISE_CHUNKED, true>(p, l, st, tm);
    else launch_steps<DT, SPEC_NOISE_CHUNKED, false>(p, l, st, tm);
  } else {
    if (vec) launch_steps<DT, SPEC_NOISE_FLAT, true>(p, l, st, tm);
    else launch_steps<DT, SPEC_NOISE_FLAT, false>(p, l, st, tm);
  }
}

}  // namespace spec

using namespace spec;

extern "C" size_t spec_workspace_bytes(const spec_dims* d) {
  if (!dims_ok(d) || !dtype_ok(d)) return 0;
  return layout(d).total;
}

extern "C" const char* spec_error_string(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_E_INVAL: return "invalid argument (NULL pointer, misaligned pointer or bad dimension)";
    case SPEC_E_DTYPE: return "unsupported dtype, noise scheme or rank for this dtype";
    case SPEC_E_WORKSPACE: return "workspace missing, misaligned or smaller than spec_workspace_bytes()";
    case SPEC_E_ARCH: return "current HIP device is not gfx950";
    case SPEC_E_HIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

extern "C" int spec_version(void) { return 100; }

static int cycle_impl(const spec_dims* d, const void* base_logits, const void* target_logits, const void* A,
                      const void* W, const int32_t* x0, const float* conf, const float* temp, float threshold,
                      uint64_t seed, int64_t request_offset, int32_t* accepted_len, int32_t* tokens,
                      const spec_diag* diag, void* workspace, size_t workspace_bytes, spec_stream_t stream,
                      const Timing& tm) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!dtype_ok(d)) return SPEC_E_DTYPE;
  if (!base_logits || !target_logits || !A || !W || !conf || !temp || !accepted_len || !tokens) return SPEC_E_INVAL;
  if ((((uintptr_t)A) | ((uintptr_t)W)) & 15) return SPEC_E_INVAL;
  const Layout l = layout(d);
  if (!workspace || workspace_bytes < l.total || (((uintptr_t)workspace) & 255)) return SPEC_E_WORKSPACE;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;

  char* ws = (char*)workspace;
  Params p;
  p.B = d->B;
  p.K = d->K;
  p.V = d->V;
  p.R = d->R;
  p.dtype = d->dtype;
  p.noise = d->noise;
  p.base = base_logits;
  p.target = target_logits;
  p.A = A;
  p.W = W;
  p.x0 = x0;
  p.conf = conf;
  p.temp = temp;
  p.threshold = threshold;
  p.seed = seed;
  p.req_off = request_offset;
  p.accepted_len = accepted_len;
  p.tokens = tokens;
  p.d_verify_len = diag ? diag->verify_len : nullptr;
  p.d_draft = diag ? diag->draft_tokens : nullptr;
  p.d_logq = diag ? diag->logq : nullptr;
  p.d_logp = diag ? diag->logp : nullptr;
  p.L = (int32_t*)(ws + l.off_L);
  p.acc = (int32_t*)(ws + l.off_acc);
  p.phase = (int32_t*)(ws + l.off_phase);
  p.roles = (uint8_t*)(ws + l.off_roles);
  p.slots = (int32_t*)(ws + l.off_slots);
  p.xs = (int32_t*)(ws + l.off_xs);
  p.lse_q = (float*)(ws + l.off_lse_q);
  p.logq = (float*)(ws + l.off_logq);
  p.lse_p = (float*)(ws + l.off_lse_p);
  p.logp = (float*)(ws + l.off_logp);
  p.part_bias = (float4*)(ws + l.off_pbias);
  p.part_bias2 = (float4*)(ws + l.off_pbias2);
  p.part_plain = (float4*)(ws + l.off_pplain);
  p.nrA = l.nrA;
  p.nrB = l.nrB;
  p.nrA_xcd = l.nrA_xcd;
  p.nrb = l.nrb;
  p.gridA = l.gridA;

  // vector loads need 16-byte aligned rows
  const size_t esz = d->dtype == SPEC_FP32 ? 4 : 2;
  const bool vec = ((d->V * esz) % 16 == 0) && ((((uintptr_t)base_logits) | ((uintptr_t)target_logits)) & 15) == 0;

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipExtLaunchKernelGGL(k_init, dim3((d->B + NT - 1) / NT), dim3(NT), 0, st, tm.start(0), tm.stop(0), 0, p);
  if (d->dtype == SPEC_BF16) launch_all<SPEC_BF16>(p, l, vec, st, tm);
  else launch_all<SPEC_FP32>(p, l, vec, st, tm);
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

extern "C" int spec_cycle(const spec_dims* d, const void* base_logits, const void* target_logits, const void* A,
                          const void* W, const int32_t* x0, const float* conf, const float* temp, float threshold,
                          uint64_t seed, int64_t request_offset, int32_t* accepted_len, int32_t* tokens,
                          const spec_diag* diag, void* workspace, size_t workspace_bytes, spec_stream_t stream) {
  const Timing tm = {nullptr, 0};
  return cycle_impl(d, base_logits, target_logits, A, W, x0, conf, temp, threshold, seed, request_offset,
                    accepted_len, tokens, diag, workspace, workspace_bytes, stream, tm);
}

extern "C" int spec_cycle_kernel_count(const spec_dims* d) {
  if (!dims_ok(d)) return 0;
  return 1 + 2 * (d->K + 1);
}

extern "C" int spec_cycle_timed(const spec_dims* d, const void* base_logits, const void* target_logits,
                                const void* A, const void* W, const int32_t* x0, const float* conf,
                                const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                                int32_t* accepted_len, int32_t* tokens, const spec_diag* diag, void* workspace,
                                size_t workspace_bytes, spec_stream_t stream, void* const* events, int n_events) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!events || n_events < 2 * spec_cycle_kernel_count(d)) return SPEC_E_INVAL;
  const Timing tm = {(hipEvent_t*)events, n_events};
  return cycle_impl(d, base_logits, target_logits, A, W, x0, conf, temp, threshold, seed, request_offset,
                    accepted_len, tokens, diag, workspace, workspace_bytes, stream, tm);
}
