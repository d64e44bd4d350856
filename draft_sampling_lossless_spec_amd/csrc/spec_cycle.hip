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
constexpr int TILE_B = NT * 2 * CHUNK;  // vocabulary columns per kind-B item: two chunks per thread
constexpr int MAX_B = 1024;
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
  uint64_t* kreq;      // [B] noise-key prefix of each request: first(first(seed) ^ global id)
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
  p.kreq[b] = sm_first(sm_first(p.seed) ^ (uint64_t)(p.req_off + b));
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

struct RowMeta {       // one bias row of a kind-A item, staged in LDS
  int b, j, role, prev;
  float invT, lse_p, lse_q, pad;
  uint64_t key1, key2;
};

struct Lists {
  int n_draft, n_correct, n_plain;
};

// Scan the role bytes of step s into the compact row lists of this step, in LDS:
//   bias_list[i]  = (request << 1) | (1 if CORRECT)  for bias slot i (DRAFT rows first, then CORRECT)
//   plain_list[i] = request                          for plain slot i (LSEP or BONUS)
// Workgroup 0 also publishes every request's slots for the merge kernel.
__device__ Lists build_lists(const Params& p, const uint8_t* roles, uint16_t* bias_list, uint16_t* plain_list,
                             uint64_t* tmp, bool publish_slots = false) {
  const int per = (p.B + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  uint64_t cnt = 0;
  for (int i = 0; i < per; i++) {
    const int b = b0 + i;
    if (b < p.B) {
      const int r = roles[b];
      cnt += (uint64_t)((r & RO_DRAFT) ? 1 : 0) | ((uint64_t)((r & RO_CORRECT) ? 1 : 0) << 16) |
             ((uint64_t)((r & (RO_LSEP | RO_BONUS)) ? 1 : 0) << 32);
    }
  }
  uint64_t tot;
  const uint64_t pre = block_excl_scan(cnt, tmp, &tot);
  Lists ls;
  ls.n_draft = (int)(tot & 0xFFFF);
  ls.n_correct = (int)((tot >> 16) & 0xFFFF);
  ls.n_plain = (int)((tot >> 32) & 0xFFFF);
  int d = (int)(pre & 0xFFFF), c = (int)((pre >> 16) & 0xFFFF), q = (int)((pre >> 32) & 0xFFFF);
  const bool publish = (blockIdx.x == 0) && publish_slots;
  for (int i = 0; i < per; i++) {
    const int b = b0 + i;
    if (b >= p.B) break;
    const int r = roles[b];
    int sd = -1, sc = -1, sp = -1;
    if (r & RO_DRAFT) { sd = d++; bias_list[sd] = (uint16_t)(b << 1); }
    if (r & RO_CORRECT) { sc = ls.n_draft + c++; bias_list[sc] = (uint16_t)((b << 1) | 1); }
    if (r & (RO_LSEP | RO_BONUS)) { sp = q++; plain_list[sp] = (uint16_t)b; }
    if (publish) {
      p.slots[b] = sd;
      p.slots[p.B + b] = sc;
      p.slots[2 * p.B + b] = sp;
    }
  }
  __syncthreads();
  return ls;
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

__device__ __forceinline__ float4 empty_part() { return make_float4(-INFINITY, -INFINITY, __int_as_float(-1), 0.0f); }

// log-sum-exp of n values held by a lane and its partner lane (lane ^ 32); NaN-preserving
template <int N>
__device__ __forceinline__ float pair_lse(const float* x) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; i++) mx = fmaxf(mx, x[i]);
  mx = fmaxf(mx, xor32f(mx));
  float sum = 0.0f;
  if (mx != -INFINITY) {
    const float mo = mx * LOG2E;
#pragma unroll
    for (int i = 0; i < N; i++) sum += ex2(fmaf(x[i], LOG2E, -mo));
  } else {
#pragma unroll
    for (int i = 0; i < N; i++) sum += x[i];   // every value -inf or NaN: keep a NaN visible
  }
  sum += xor32f(sum);
  return (mx == -INFINITY) ? sum : mx + lg2(sum) * LN2;
}

// best (score, index, aux) of a lane and its partner lane
__device__ __forceinline__ void pair_best(float& sc, int& ix, float& aux) {
  const float s2 = xor32f(sc);
  const int i2 = xor32i(ix);
  const float a2 = xor32f(aux);
  if (i2 >= 0 && (ix < 0 || better(s2, i2, sc, ix))) {
    sc = s2;
    ix = i2;
    aux = a2;
  }
}

// 16 consecutive bf16 / fp32 values of a row as raw words (bf16: 8 words, fp32: 16 words)
template <int DT>
struct Raw16 {
  u32x4 w[DT == SPEC_BF16 ? 2 : 4];
};

// 16 columns of one row per lane; the lanes of one load instruction span 32 rows, so these are
// ordinary (temporal) loads: the other pieces of each cache line arrive from neighbouring
// instructions through the caches
template <int DT>
__device__ __forceinline__ void raw_load(const void* row, int v, Raw16<DT>& r) {
  const u32x4* q = (const u32x4*)((const char*)row + (size_t)v * (DT == SPEC_BF16 ? 2 : 4));
#pragma unroll
  for (int k = 0; k < (DT == SPEC_BF16 ? 2 : 4); k++) r.w[k] = q[k];
}

// as raw_load, for rows whose 16-byte pieces are each wholly inside or wholly past column V
// (aligned rows, V % 8 == 0 for bf16, V % 4 == 0 for fp32): the pieces past V read as -inf
template <int DT>
__device__ __forceinline__ void raw_load_pred(const void* row, int v, int V, Raw16<DT>& r) {
  const u32x4* q = (const u32x4*)((const char*)row + (size_t)v * (DT == SPEC_BF16 ? 2 : 4));
  const uint32_t ninf = (DT == SPEC_BF16) ? 0xFF80FF80u : 0xFF800000u;
  constexpr int per = (DT == SPEC_BF16) ? 8 : 4;
#pragma unroll
  for (int k = 0; k < (DT == SPEC_BF16 ? 2 : 4); k++) {
    if (v + per * k < V) r.w[k] = q[k];
    else r.w[k] = (u32x4){ninf, ninf, ninf, ninf};
  }
}

template <int DT>
__device__ __forceinline__ float raw_at(const Raw16<DT>& r, int i) {
  if (DT == SPEC_BF16) {
    const uint32_t w = r.w[i >> 3][(i >> 1) & 3];
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  return __uint_as_float(r.w[i >> 2][i & 3]);
}

// ------------------------------------------------------------------------------------------
// kind A: bias rows (DRAFT / CORRECT) over 256 columns, up to 256 rows
// ------------------------------------------------------------------------------------------
struct WaveOut {        // one wave's result for one row over its 64 columns
  float4 a;             // {log-mass, best score, best index (bits), aux}
  float4 b;             // CORRECT: target-row fallback {lse, best score, best index, 0}
};


// FLAT draft: best (s_v + G(key2, v)) over the lane's 32 columns, s in place in x[]
__device__ __forceinline__ void flat_best32(const float* x, int v0, int V, uint64_t key2, float& best, int& bestv,
                                            float& bests) {
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const int v = v0 + 32 * (i >> 4) + (i & 15);
    if (v >= V) continue;
    const uint64_t w = pair_word(key2, (uint32_t)v >> 1);
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const float sv = x[i + e];
      const uint32_t bb = e ? (uint32_t)w : (uint32_t)(w >> 32);
      if (v + e >= V || !(sv > -INFINITY)) continue;
      if (sv + gumbel_bound(bb) + 1e-3f < best) continue;
      const float zz = sv + gumbel_bits(bb);
      if (better(zz, v + e, best, bestv)) {
        best = zz;
        bestv = v + e;
        bests = sv;
      }
    }
  }
}

// fp32 factors: Markov bias of the lane's columns by VALU dot products (small vocabularies)
__device__ __forceinline__ void fp32_bias16(const Params& p, const RowMeta& rm, int vstart, int V, bool active,
                                            float* x) {
  const int R = p.R;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const int v = vstart + q;
    float a = 0.0f;
    if (active && rm.prev >= 0 && v < V) {
      const float* wr = (const float*)p.W + (size_t)v * R;
      const float* ar = (const float*)p.A + (size_t)rm.prev * R;
      for (int k = 0; k < R; k++) a = fmaf(ar[k], wr[k], a);
    }
    x[q] = a;
  }
}

// ------------------------------------------------------------------------------------------
// bias-row sweep, unit by unit.  A unit is (column range of 256, sub-block of 32 bias rows); the
// units of a step are split evenly over the resident workgroups in range-major order, so a
// workgroup reloads its W fragments only when it crosses into the next column range.
// ------------------------------------------------------------------------------------------
struct BiasLds {
  uint16_t sA[SUB][MAX_R + A_PAD];   // gathered A rows of the current unit (bf16)
  uint16_t sX[SUB][TILE_A + 8];      // draft logits of the current unit, 32 rows x 256 columns (bf16)
  WaveOut red[NT / 64][SUB];         // per-wave results of the current unit
};

__device__ __forceinline__ uint64_t key_of(const Params& p, int b, int pos, uint64_t stream) {
  return sm_first(sm_first(p.kreq[b] ^ (uint64_t)pos) ^ stream);
}

// metadata of every bias row of the step (rows past n_bias up to a whole sub-block are inactive)
__device__ void fill_all_meta(const Params& p, int s, const Lists& ls, const uint16_t* bias_list, RowMeta* meta) {
  const int n_bias = ls.n_draft + ls.n_correct;
  const int n_rows = (n_bias + SUB - 1) / SUB * SUB;
  for (int slot = threadIdx.x; slot < n_rows; slot += NT) {
    RowMeta rm;
    if (slot < n_bias) {
      const int e = bias_list[slot];
      const int b = e >> 1;
      const int role = (e & 1) ? RO_CORRECT : RO_DRAFT;
      const int j = (role == RO_DRAFT) ? s : p.acc[b];
      rm.b = b;
      rm.j = j;
      rm.role = role;
      rm.prev = (j == 0) ? (p.x0 ? p.x0[b] : -1) : p.xs[(size_t)b * p.K + j - 1];
      rm.invT = 1.0f / p.temp[b];
      rm.pad = 0.0f;
      if (role == RO_DRAFT) {
        rm.key1 = key_of(p, b, j, ST_DRAFT_C);
        rm.key2 = key_of(p, b, j, ST_DRAFT);
        rm.lse_p = rm.lse_q = 0.0f;
      } else {
        rm.key1 = key_of(p, b, j, ST_RESIDUAL_C);
        rm.key2 = key_of(p, b, j, ST_RESIDUAL);
        rm.lse_p = p.lse_p[(size_t)b * (p.K + 1) + j];
        rm.lse_q = p.lse_q[(size_t)b * p.K + j];
      }
    } else {
      rm.b = 0;
      rm.j = 0;
      rm.role = 0;
      rm.prev = -1;
      rm.invT = 1.0f;
      rm.lse_p = rm.lse_q = rm.pad = 0.0f;
      rm.key1 = rm.key2 = 0;
    }
    meta[slot] = rm;
  }
}

// register prefetch of one unit: A rows (bf16) and, for the tiled path, the 32 x 256 draft-logit
// tile, read with coalesced 16-byte loads (each wave instruction covers two 512-byte row pieces)
struct UnitPrefetch {
  u32x4 a[4];
  u32x4 x[4];
};

template <bool TILE>
__device__ __forceinline__ void unit_fetch(const Params& p, const RowMeta* meta, int range, UnitPrefetch& up) {
  const int R = p.R, segs = R / 8;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = threadIdx.x + NT * i;
    u32x4 val = {0, 0, 0, 0};
    if (e < SUB * segs) {
      const int prev = meta[e / segs].prev;
      if (prev >= 0) val = *(const u32x4*)((const uint16_t*)p.A + (size_t)prev * R + 8 * (e % segs));
    }
    up.a[i] = val;
  }
  if (TILE) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = range * TILE_A + 8 * (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 8 * i + 2 * wave + (lane >> 5);
      const RowMeta& rm = meta[r];
      u32x4 val = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};   // -inf past the row / no row
      if (rm.role != 0 && col < p.V)
        val = *(const u32x4*)((const uint16_t*)p.base + ((size_t)rm.b * p.K + rm.j) * (size_t)p.V + col);
      up.x[i] = val;
    }
  }
}

template <bool TILE>
__device__ __forceinline__ void unit_store(const Params& p, const UnitPrefetch& up, BiasLds& L) {
  const int segs = p.R / 8;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = threadIdx.x + NT * i;
    if (e < SUB * segs) *(u32x4*)&L.sA[e / segs][8 * (e % segs)] = up.a[i];
  }
  if (TILE) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 8 * i + 2 * wave + (lane >> 5);
      *(u32x4*)&L.sX[r][8 * (lane & 31)] = up.x[i];
    }
  }
}

// partials of one finished unit from red (threads 0..31)
__device__ __forceinline__ void unit_flush(const Params& p, const Lists& ls, const BiasLds& L, int slot0, int range) {
  if (threadIdx.x < SUB) {
    const int r = threadIdx.x, slot = slot0 + r;
    if (slot < ls.n_draft + ls.n_correct) {
      float4 pa = L.red[0][r].a;
#pragma unroll
      for (int w = 1; w < NT / 64; w++) pa = merge_part(pa, L.red[w][r].a);
      p.part_bias[(size_t)slot * p.nrA + range] = pa;
      if (slot >= ls.n_draft) {
        float4 pb = L.red[0][r].b;
#pragma unroll
        for (int w = 1; w < NT / 64; w++) pb = merge_part(pb, L.red[w][r].b);
        p.part_bias2[(size_t)slot * p.nrA + range] = pb;
      }
    }
  }
}

template <int DT, int NOISE, bool VEC>
__device__ void bias_sweep(const Params& p, int s, const Lists& ls, const RowMeta* meta, BiasLds& L) {
  constexpr bool TILE = (DT == SPEC_BF16) && VEC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int V = p.V, R = p.R, K = p.K;
  const int T16 = R / 16;
  const int kb = h * (R / 2);
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const int n_bias = ls.n_draft + ls.n_correct;
  const int nsb = (n_bias + SUB - 1) / SUB;
  const long long units = (long long)p.nrA * nsb;
  const int u0 = (int)(units * blockIdx.x / gridDim.x);
  const int u1 = (int)(units * (blockIdx.x + 1) / gridDim.x);
  if (u0 >= u1) return;

  bf16x8 wf[2][16];
  int w_range = -1;
  UnitPrefetch up;
  unit_fetch<TILE>(p, meta + (u0 % nsb) * SUB, u0 / nsb, up);

  for (int u = u0; u < u1; u++) {
    const int range = u / nsb, sb = u % nsb;
    __syncthreads();   // waves are done with the previous unit's LDS tiles and red
    if (DT == SPEC_BF16) unit_store<TILE>(p, up, L);
    if (u > u0) unit_flush(p, ls, L, ((u - 1) % nsb) * SUB, (u - 1) / nsb);
    __syncthreads();   // this unit's tiles are in LDS; red is free
    if (range != w_range && DT == SPEC_BF16) {
      // W fragments: MFMA A-operand row i of fragment f is column vw + 32f + perm(i), perm chosen
      // so that accumulator q of lane l holds column vw + 32f + 16*(l/32) + q; lane half l/32
      // covers k in [R/2 * (l/32), R/2 * (l/32 + 1))
      const int col_in = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
      const int vw = range * TILE_A + 64 * wave;
#pragma unroll
      for (int f = 0; f < 2; f++) {
        const int v = vw + 32 * f + col_in;
#pragma unroll
        for (int t = 0; t < 16; t++) {
          if (t < T16) {
            if (v < V) wf[f][t] = *(const bf16x8*)((const uint16_t*)p.W + (size_t)v * R + kb + 8 * t);
            else wf[f][t] = (bf16x8){0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
      }
    }
    w_range = range;
    if (u + 1 < u1) unit_fetch<TILE>(p, meta + ((u + 1) % nsb) * SUB, (u + 1) / nsb, up);

    const int vw = range * TILE_A + 64 * wave;   // this wave's 64 columns: one noise chunk
    const int chunk = vw / CHUNK;
    const int v0 = vw + 16 * h;                  // lane's first column in fragment 0
    const int slot0 = sb * SUB;
    const bool any_correct = slot0 + SUB > ls.n_draft && slot0 < n_bias;   // uniform
    const RowMeta& rm = meta[slot0 + m];
    const int role = rm.role;
    const float invT = rm.invT;
    const void* base_row = (const char*)p.base + ((size_t)rm.b * K + rm.j) * (size_t)V * esz;

    // Markov bias of the lane's 32 columns
    float x[32];
    if (DT == SPEC_BF16) {
      f32x16 acc0 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      f32x16 acc1 = acc0;
#pragma unroll
      for (int t = 0; t < 16; t++) {
        if (t < T16) {
          const bf16x8 bop = *(const bf16x8*)&L.sA[m][kb + 8 * t];
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][t], bop, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][t], bop, acc1, 0, 0, 0);
        }
      }
#pragma unroll
      for (int q = 0; q < 16; q++) {
        x[q] = acc0[q];
        x[16 + q] = acc1[q];
      }
    } else {
      fp32_bias16(p, rm, v0, V, role != 0, x);
      fp32_bias16(p, rm, v0 + 32, V, role != 0, x + 16);
    }
    // draft logits s = (base + bias) / T
    if (TILE) {
      const uint16_t* xr = &L.sX[m][64 * wave + 16 * h];
      const u32x4 a0 = *(const u32x4*)xr, a1 = *(const u32x4*)(xr + 8);
      const u32x4 c0 = *(const u32x4*)(xr + 32), c1 = *(const u32x4*)(xr + 40);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        x[2 * i] = (bf16_lo(a0[i]) + x[2 * i]) * invT;
        x[2 * i + 1] = (bf16_hi(a0[i]) + x[2 * i + 1]) * invT;
        x[8 + 2 * i] = (bf16_lo(a1[i]) + x[8 + 2 * i]) * invT;
        x[8 + 2 * i + 1] = (bf16_hi(a1[i]) + x[8 + 2 * i + 1]) * invT;
        x[16 + 2 * i] = (bf16_lo(c0[i]) + x[16 + 2 * i]) * invT;
        x[16 + 2 * i + 1] = (bf16_hi(c0[i]) + x[16 + 2 * i + 1]) * invT;
        x[24 + 2 * i] = (bf16_lo(c1[i]) + x[24 + 2 * i]) * invT;
        x[24 + 2 * i + 1] = (bf16_hi(c1[i]) + x[24 + 2 * i + 1]) * invT;
      }
    } else if (VEC) {
      Raw16<DT> r0, r1;
      if (role) {
        raw_load_pred<DT>(base_row, v0, V, r0);
        raw_load_pred<DT>(base_row, v0 + 32, V, r1);
      }
#pragma unroll
      for (int q = 0; q < 16; q++) {
        x[q] = role ? (raw_at<DT>(r0, q) + x[q]) * invT : -INFINITY;
        x[16 + q] = role ? (raw_at<DT>(r1, q) + x[16 + q]) * invT : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; i++) {
        const int v = v0 + 32 * (i >> 4) + (i & 15);
        x[i] = (role && v < V) ? (load1<DT>(base_row, (size_t)v) + x[i]) * invT : -INFINITY;
      }
    }

    float4 oa = empty_part(), ob = empty_part();
    if (!any_correct) {
      // ---- DRAFT rows only
      const float lse = pair_lse<32>(x);
      if (role) {
        if (NOISE == SPEC_NOISE_CHUNKED) {
          const float score = (lse > -INFINITY) ? lse + gumbel_bits(bits_at(rm.key1, (uint32_t)chunk)) : lse;
          oa = make_float4(lse, score, __int_as_float(chunk), 0.0f);
        } else {
          float best = -INFINITY, bests = 0.0f;
          int bestv = -1;
          flat_best32(x, v0, V, rm.key2, best, bestv, bests);
          pair_best(best, bestv, bests);
          oa = make_float4(lse, best, __int_as_float(bestv), bests);
        }
      }
    } else {
      // ---- unit holding CORRECT rows: residual norm(max(0, p - q)) and its target-row fallback,
      //      the target row streamed one 16-column fragment at a time with online reductions
      const bool corr = role == RO_CORRECT;
      const float lse_x = pair_lse<32>(x);   // draft log-mass (used by DRAFT lanes)
      const void* targ_row = (const char*)p.target + ((size_t)rm.b * (K + 1) + rm.j) * (size_t)V * esz;
      float mt = -INFINITY, st = 0.0f, mass = 0.0f;
      float br = -INFINITY, bp = -INFINITY, bd = -INFINITY, bds = 0.0f;
      int vr = -1, vp = -1, vd = -1;
      if (NOISE == SPEC_NOISE_FLAT && role == RO_DRAFT) flat_best32(x, v0, V, rm.key2, bd, vd, bds);
#pragma unroll
      for (int f = 0; f < 2; f++) {
        float t[16];
        if (VEC) {
          Raw16<DT> r0;
          if (corr) raw_load_pred<DT>(targ_row, v0 + 32 * f, V, r0);
#pragma unroll
          for (int q = 0; q < 16; q++) t[q] = corr ? raw_at<DT>(r0, q) * invT : -INFINITY;
        } else {
#pragma unroll
          for (int q = 0; q < 16; q++) {
            const int v = v0 + 32 * f + q;
            t[q] = (corr && v < V) ? load1<DT>(targ_row, (size_t)v) * invT : -INFINITY;
          }
        }
        if (corr) {
          float fm = -INFINITY;
#pragma unroll
          for (int q = 0; q < 16; q++) fm = fmaxf(fm, t[q]);
          const float nm = fmaxf(mt, fm);
          if (nm > -INFINITY) {
            float acc_s = (mt > -INFINITY) ? st * ex2((mt - nm) * LOG2E) : (st != st ? st : 0.0f);
#pragma unroll
            for (int q = 0; q < 16; q++) acc_s += ex2((t[q] - nm) * LOG2E);
            st = acc_s;
            mt = nm;
          } else {
#pragma unroll
            for (int q = 0; q < 16; q++) st += (t[q] != t[q]) ? t[q] : 0.0f;   // NaN stays visible
          }
#pragma unroll
          for (int q = 0; q < 16; q++) {
            const float lp = t[q] - rm.lse_p, lq = x[16 * f + q] - rm.lse_q;
            if (lp > lq) mass += ex2(lp * LOG2E) - ex2(lq * LOG2E);
          }
          if (NOISE == SPEC_NOISE_FLAT) {
#pragma unroll
            for (int q = 0; q < 16; q++) {
              const int v = v0 + 32 * f + q;
              if (v >= V) continue;
              const float g = gumbel_bits(bits_at(rm.key2, (uint32_t)v));
              const float lp = t[q] - rm.lse_p, lq = x[16 * f + q] - rm.lse_q;
              if (lp > lq) {
                const float sc = lp + logf(-expm1f(lq - lp)) + g;
                if (better(sc, v, br, vr)) { br = sc; vr = v; }
              }
              if (t[q] > -INFINITY && better(t[q] + g, v, bp, vp)) { bp = t[q] + g; vp = v; }
            }
          }
        }
      }
      // pair-combine (lane ^ 32 holds the other 16 columns of each fragment of the same row)
      const float m2 = xor32f(mt), s2 = xor32f(st);
      const float nm = fmaxf(mt, m2);
      float lse_t;
      if (nm > -INFINITY) {
        const float a = (mt > -INFINITY) ? st * ex2((mt - nm) * LOG2E) : (st != st ? st : 0.0f);
        const float c = (m2 > -INFINITY) ? s2 * ex2((m2 - nm) * LOG2E) : (s2 != s2 ? s2 : 0.0f);
        lse_t = nm + lg2(a + c) * LN2;
      } else {
        lse_t = (st != st || s2 != s2) ? NAN : -INFINITY;
      }
      mass += xor32f(mass);
      float dummy = 0.0f;
      pair_best(br, vr, dummy);
      pair_best(bp, vp, dummy);
      pair_best(bd, vd, bds);
      if (role == RO_DRAFT) {
        if (NOISE == SPEC_NOISE_CHUNKED) {
          const float score = (lse_x > -INFINITY) ? lse_x + gumbel_bits(bits_at(rm.key1, (uint32_t)chunk)) : lse_x;
          oa = make_float4(lse_x, score, __int_as_float(chunk), 0.0f);
        } else {
          oa = make_float4(lse_x, bd, __int_as_float(vd), bds);
        }
      } else if (corr) {
        const float lmass = (mass > 0.0f) ? lg2(mass) * LN2 : -INFINITY;
        if (NOISE == SPEC_NOISE_CHUNKED) {
          const float g = gumbel_bits(bits_at(rm.key1, (uint32_t)chunk));
          oa = make_float4(lmass, lmass > -INFINITY ? lmass + g : -INFINITY, __int_as_float(chunk), 0.0f);
          ob = make_float4(lse_t, lse_t > -INFINITY ? lse_t + g : -INFINITY, __int_as_float(chunk), 0.0f);
        } else {
          oa = make_float4(lmass, br, __int_as_float(vr), 0.0f);
          ob = make_float4(lse_t, bp, __int_as_float(vp), 0.0f);
        }
      }
    }
    if (h == 0) {
      L.red[wave][m].a = oa;
      L.red[wave][m].b = ob;
    }
  }
  __syncthreads();
  unit_flush(p, ls, L, ((u1 - 1) % nsb) * SUB, (u1 - 1) / nsb);
}

// ------------------------------------------------------------------------------------------
// kind B: plain target rows (LSEP / BONUS), 128 consecutive columns (two chunks) per thread,
// every load of the item issued before any arithmetic
// ------------------------------------------------------------------------------------------
// kind B layout: load k (0..15) of a thread covers 8 columns at 2048 k + 8 t of the item, so every
// load instruction of a wave reads 1 KiB of contiguous memory; the 64 columns of a noise chunk
// are the 8 values of 8 neighbouring lanes.
template <int DT>
struct Raw8 {
  u32x4 w[DT == SPEC_BF16 ? 1 : 2];
};

template <int DT>
__device__ __forceinline__ float raw8_at(const Raw8<DT>& r, int i) {
  if (DT == SPEC_BF16) {
    const uint32_t w = r.w[0][i >> 1];
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  return __uint_as_float(r.w[i >> 2][i & 3]);
}


constexpr int KB_LOADS = 16;   // loads of 8 columns per thread per kind-B item

template <int DT, int NOISE, bool VEC>
__device__ void kind_b(const Params& p, int s, int b, int pslot, int range, float4* redb) {
  const int K = p.K, V = p.V;
  const int role = p.roles[(size_t)(s & 1) * p.B + b] & (RO_LSEP | RO_BONUS);
  const int j = s;   // LSEP verifies position s; BONUS reads row L_b == s
  const float invT = 1.0f / p.temp[b];
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const void* row = (const char*)p.target + ((size_t)b * (K + 1) + j) * (size_t)V * esz;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vbase = range * TILE_B;
  const int vt = vbase + 8 * threadIdx.x;           // + 2048 k
  Raw8<DT> r[KB_LOADS];
  if (VEC) {
    // rows are 16-byte aligned and V % 8 == 0 (bf16) / V % 4 == 0 (fp32), so each 16-byte load
    // is wholly inside or wholly past the row end: predicate the loads, pad with -inf
    const uint32_t ninf = (DT == SPEC_BF16) ? 0xFF80FF80u : 0xFF800000u;
#pragma unroll
    for (int k = 0; k < KB_LOADS; k++) {
      const u32x4* q = (const u32x4*)((const char*)row + (size_t)(vt + 2048 * k) * esz);
#pragma unroll
      for (int u = 0; u < (DT == SPEC_BF16 ? 1 : 2); u++) {
        const int vv = vt + 2048 * k + 4 * u;
        if (vv < V) r[k].w[u] = __builtin_nontemporal_load(q + u);
        else r[k].w[u] = (u32x4){ninf, ninf, ninf, ninf};
      }
    }
  } else {
    // unaligned rows: the same layout filled element by element, -inf past the row end
#pragma unroll 1
    for (int k = 0; k < KB_LOADS; k++) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int v = vt + 2048 * k + i;
        const float x = (v < V) ? load1<DT>(row, (size_t)v) : -INFINITY;
        if (DT == SPEC_BF16) {
          const uint32_t hb = __float_as_uint(x) >> 16;   // exact: the value came from a bf16
          const uint32_t w = r[k].w[0][i >> 1];
          r[k].w[0][i >> 1] = (i & 1) ? ((w & 0xFFFFu) | (hb << 16)) : ((w & 0xFFFF0000u) | hb);
        } else {
          r[k].w[i >> 2][i & 3] = __float_as_uint(x);
        }
      }
    }
  }
  const uint64_t g = (uint64_t)(p.req_off + b);
  const float sc2 = invT * LOG2E;
  // log-mass of each 64-column chunk (8 lanes x 8 values); the rounds are independent and every
  // lane keeps the two chunks it owns: rounds k = lane % 8 and lane % 8 + 8
  float own0 = -INFINITY, own1 = -INFINITY;
#pragma unroll
  for (int k = 0; k < KB_LOADS; k++) {
    float mx = raw8_at<DT>(r[k], 0);
#pragma unroll
    for (int i = 1; i < 8; i++) mx = fmaxf(mx, raw8_at<DT>(r[k], i));
    mx = max8(mx);
    float sum = 0.0f;
    if (mx != -INFINITY) {
      const float mo = mx * sc2;
#pragma unroll
      for (int i = 0; i < 8; i++) sum += ex2(fmaf(raw8_at<DT>(r[k], i), sc2, -mo));
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) sum += raw8_at<DT>(r[k], i);   // every value -inf or NaN: keep a NaN visible
    }
    sum = sum8(sum);
    const float lse = (mx == -INFINITY) ? sum : mx * invT + lg2(sum) * LN2;
    if ((lane & 7) == (k & 7)) {
      if (k < 8) own0 = lse;
      else own1 = lse;
    }
  }
  float4 part = make_float4(lse2(own0, own1), -INFINITY, __int_as_float(-1), 0.0f);
  if (role == RO_BONUS) {
    if (NOISE == SPEC_NOISE_CHUNKED) {
      const uint64_t k1 = row_key(p.seed, g, (uint64_t)j, ST_BONUS_C);
#pragma unroll
      for (int o = 0; o < 2; o++) {
        const float lse = o ? own1 : own0;
        const int k = (lane & 7) + 8 * o;
        const int c = (vbase + 2048 * k) / CHUNK + (lane >> 3) + 8 * wave;
        if (lse > -INFINITY) {
          const float sc = lse + gumbel_bits(bits_at(k1, (uint32_t)c));
          if (better(sc, c, part.y, __float_as_int(part.z))) {
            part.y = sc;
            part.z = __int_as_float(c);
          }
        }
      }
    } else {
      const uint64_t k2 = row_key(p.seed, g, (uint64_t)j, ST_BONUS);
      float best = -INFINITY;
      int bv = -1;
#pragma unroll 1
      for (int k = 0; k < KB_LOADS; k++) {
        const int v0 = vt + 2048 * k;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int v = v0 + i;
          const uint64_t w = pair_word(k2, (uint32_t)v >> 1);
#pragma unroll
          for (int e = 0; e < 2; e++) {
            const float sv = raw8_at<DT>(r[k], i + e) * invT;
            const uint32_t bb = e ? (uint32_t)w : (uint32_t)(w >> 32);
            if (v + e >= V || !(sv > -INFINITY)) continue;
            if (sv + gumbel_bound(bb) + 1e-3f < best) continue;
            const float zz = sv + gumbel_bits(bb);
            if (better(zz, v + e, best, bv)) {
              best = zz;
              bv = v + e;
            }
          }
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
  __syncthreads();
  if (lane == 0) redb[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 rr = redb[0];
#pragma unroll
    for (int w = 1; w < NT / 64; w++) rr = merge_part(rr, redb[w]);
    p.part_plain[(size_t)pslot * p.nrB + range] = rr;
  }
}

// Row sweeps of one step.  Every workgroup rebuilds the step's row lists from the role bytes,
// then takes work items grid-stride.  k_bias takes the bias rows (MFMA, W fragments resident, two
// workgroups per CU); k_plain streams the target rows of LSEP / BONUS roles at high occupancy.
// For k_bias, items i and i + 8 run on one XCD, and consecutive items on an XCD are the
// row-blocks of one column range, so its W tile is shared in that XCD's L2.
// dynamic LDS of k_bias: row metadata of up to 2B bias rows (rounded to a sub-block), then the
// bias list [2B] and plain list [B]
__host__ __device__ constexpr size_t bias_meta_bytes(int B) { return (size_t)(2 * B + SUB) * sizeof(RowMeta); }

template <int DT, int NOISE, bool VEC>
__global__ __launch_bounds__(NT, 1) void k_bias(Params p, int s) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_bias[];
  __shared__ uint64_t scan_tmp[NT / 64];
  __shared__ BiasLds lds_a;
  RowMeta* meta = (RowMeta*)dyn_bias;
  uint16_t* bias_list = (uint16_t*)(dyn_bias + bias_meta_bytes(p.B));
  uint16_t* plain_list = bias_list + 2 * p.B;
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;
  const Lists ls = build_lists(p, roles, bias_list, plain_list, scan_tmp, true);
  if (ls.n_draft + ls.n_correct == 0) return;
  fill_all_meta(p, s, ls, bias_list, meta);
  __syncthreads();
  bias_sweep<DT, NOISE, VEC>(p, s, ls, meta, lds_a);
}

template <int DT, int NOISE, bool VEC>
__global__ __launch_bounds__(NT, 3) void k_plain(Params p, int s) {
  extern __shared__ uint16_t dyn_lists[];
  __shared__ uint64_t scan_tmp[NT / 64];
  __shared__ float4 redb[NT / 64];
  uint16_t* bias_list = dyn_lists;
  uint16_t* plain_list = dyn_lists + 2 * p.B;
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;
  const Lists ls = build_lists(p, roles, bias_list, plain_list, scan_tmp);
  const int n_items = ls.n_plain * p.nrB;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int pslot = it / p.nrB, range = it % p.nrB;
    kind_b<DT, NOISE, VEC>(p, s, plain_list[pslot], pslot, range, redb);
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

// Markov bias of column v, the share of thread quarter q = 0..3 of the rank (fp32 accumulate)
template <int DT>
__device__ float bias_quarter(const Params& p, int prev, int v, int q) {
  float a = 0.0f;
  const int R = p.R;
  if (prev < 0) return a;
  if (DT == SPEC_BF16) {
    const uint16_t* ar = (const uint16_t*)p.A + (size_t)prev * R;
    const uint16_t* wr = (const uint16_t*)p.W + (size_t)v * R;
    for (int k = 8 * q; k < R; k += 32) {
      const u32x4 aw = *(const u32x4*)(ar + k);
      const u32x4 ww = *(const u32x4*)(wr + k);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        a = fmaf(bf16_lo(aw[i]), bf16_lo(ww[i]), a);
        a = fmaf(bf16_hi(aw[i]), bf16_hi(ww[i]), a);
      }
    }
  } else {
    const float* ar = (const float*)p.A + (size_t)prev * R;
    const float* wr = (const float*)p.W + (size_t)v * R;
    for (int k = q; k < R; k += 4) a = fmaf(ar[k], wr[k], a);
  }
  return a;
}

enum { L2_DRAFT = 0, L2_TARGET = 1, L2_RESIDUAL = 2 };

// Level two of the CHUNKED sampler over chunk c, whole workgroup: argmax over the chunk's
// columns of (score_v + G(key2, v)); thread t works on column 64c + t/4 with a quarter of the
// rank.  Returns the column (-1 if none) and, for DRAFT, its scaled draft logit in *aux_out.
template <int DT>
__device__ int level_two(const Params& p, int kind, int c, uint64_t key2, const void* base_row,
                         const void* targ_row, int prev, float invT, float lse_p, float lse_q, float* aux_out,
                         float4* lds) {
  const int q = threadIdx.x & 3;
  const int v = c * CHUNK + (threadIdx.x >> 2);
  const bool in = c >= 0 && v < p.V;
  float bias = 0.0f;
  if (in && kind != L2_TARGET) bias = bias_quarter<DT>(p, prev, v, q);
  bias += __shfl_xor(bias, 1, 64);
  bias += __shfl_xor(bias, 2, 64);
  float sc = -INFINITY, aux = 0.0f;
  int ix = -1;
  if (in && q == 0) {
    const float g = gumbel_bits(bits_at(key2, (uint32_t)v));
    if (kind == L2_DRAFT) {
      const float sv = (load1<DT>(base_row, (size_t)v) + bias) * invT;
      if (sv > -INFINITY) {
        sc = sv + g;
        ix = v;
        aux = sv;
      }
    } else if (kind == L2_TARGET) {
      const float tv = load1<DT>(targ_row, (size_t)v) * invT;
      if (tv > -INFINITY) {
        sc = tv + g;
        ix = v;
      }
    } else {
      const float sv = (load1<DT>(base_row, (size_t)v) + bias) * invT;
      const float tv = load1<DT>(targ_row, (size_t)v) * invT;
      const float lp = tv - lse_p, lq = sv - lse_q;
      if (lp > lq) {
        sc = lp + logf(-expm1f(lq - lp)) + g;
        ix = v;
      }
    }
  }
  wave_argmax(sc, ix, aux);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = make_float4(sc, aux, __int_as_float(ix), 0.0f);
  __syncthreads();
  float bs = lds[0].x, ba = lds[0].y;
  int bi = __float_as_int(lds[0].z);
#pragma unroll
  for (int w = 1; w < NT / 64; w++) {
    const int i2 = __float_as_int(lds[w].z);
    if (i2 >= 0 && (bi < 0 || better(lds[w].x, i2, bs, bi))) {
      bs = lds[w].x;
      bi = i2;
      ba = lds[w].y;
    }
  }
  if (aux_out) *aux_out = ba;
  return bi;
}

template <int DT, int NOISE>
__global__ __launch_bounds__(NT) void k_merge(Params p, int s) {
  __shared__ float4 red[NT / 64];
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
        x_s = level_two<DT>(p, L2_DRAFT, __float_as_int(tot.z), key2, base_row, nullptr, prev, invT, 0.f, 0.f, &sx,
                            red);
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
        final_tok = level_two<DT>(p, L2_TARGET, __float_as_int(tot.z), key2, nullptr, targ_row, -1, invT, 0.f, 0.f,
                                  nullptr, red);
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
      final_tok = residual ? level_two<DT>(p, L2_RESIDUAL, __float_as_int(prim.z), key2, base_row, targ_row, prev,
                                           invT, lse_p, lse_q, nullptr, red)
                           : level_two<DT>(p, L2_TARGET, __float_as_int(sec.z), key2, nullptr, targ_row, -1, invT,
                                           0.f, 0.f, nullptr, red);
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
  size_t off_L, off_acc, off_phase, off_roles, off_slots, off_xs, off_kreq, off_lse_q, off_logq, off_lse_p, off_logp,
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
  l.off_kreq = o; o = align256(o + 8 * B);
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

static int cu_count() {
  static int ncu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int n = (dev >= 0 && dev < 64) ? ncu[dev] : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < 64) ncu[dev] = n;
  }
  return n;
}

// resident grids: k_bias holds two 256-thread workgroups per CU, k_plain three
static int grid_for(int max_items, int per_cu) {
  const int resident = per_cu * cu_count();
  return max_items < resident ? max_items : resident;
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

// Kernel i of a cycle (0 = init; 1 + 3s, 2 + 3s, 3 + 3s = bias sweep, plain sweep, merge of step s)
// may carry a start/stop event pair, attached to its own dispatch.
struct Timing {
  hipEvent_t* ev;
  int n;
  hipEvent_t start(int i) const { return (ev && 2 * i + 1 < n) ? ev[2 * i] : nullptr; }
  hipEvent_t stop(int i) const { return (ev && 2 * i + 1 < n) ? ev[2 * i + 1] : nullptr; }
};

template <int DT, int NOISE, bool VEC>
static void launch_steps(const Params& p, const Layout& l, hipStream_t st, const Timing& tm) {
  const size_t lists = (size_t)6 * p.B;
  for (int s = 0; s <= p.K; s++) {
    const int k0 = 1 + 3 * s;
    hipExtLaunchKernelGGL((k_bias<DT, NOISE, VEC>), dim3(cu_count()), dim3(NT), bias_meta_bytes(p.B) + lists, st,
                          tm.start(k0),
                          tm.stop(k0), 0, p, s);
    hipExtLaunchKernelGGL((k_plain<DT, NOISE, VEC>), dim3(grid_for(l.gridB, 3)), dim3(NT), lists, st,
                          tm.start(k0 + 1), tm.stop(k0 + 1), 0, p, s);
    hipExtLaunchKernelGGL((k_merge<DT, NOISE>), dim3(p.B), dim3(NT), 0, st, tm.start(k0 + 2), tm.stop(k0 + 2), 0, p,
                          s);
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
  p.kreq = (uint64_t*)(ws + l.off_kreq);
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
  return 1 + 3 * (d->K + 1);
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
