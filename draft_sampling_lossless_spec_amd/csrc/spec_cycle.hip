// spec_cycle.hip -- MI355X (gfx950) kernels and C ABI of one batched speculation cycle.
//
// Method (per request; sources named in include/spec_cycle.h): prefix cut on the fp64 running
// product of confidences; semi-autoregressive draft x_j ~ softmax((base_j + A[x_{j-1}] W)/T);
// accept while u_j < p_j(x_j)/q_j(x_j); correction from norm(max(0, p - q)) at the first
// rejection, or a bonus token from p when every verified draft survives.
//
// Device schedule.  The draft chain is sequential in the position (the bias of position s+1
// needs x_s), and every position needs a full pass over the Markov factor W, so the cycle runs
// as k_init and then K+1 steps, all enqueued by one host call.  Per step:
//   sweep       one pass over the rows active at step s.  "Bias rows" (DRAFT rows of position s
//               and CORRECT rows of a position rejected at s-1) need A[prev] . W.  On the bf16
//               fast path (k_sweep_fast, V % 8 == 0) the gathered A rows of up to 256 bias slots
//               are staged in LDS once per step; then every wave runs on its own over units of
//               one 64-column noise chunk x one 32-slot sub-block, keeping the chunk's W
//               fragments in the accumulation registers and computing the bias with
//               v_mfma_f32_32x32x16_bf16 directly in the layout the element-wise part consumes
//               (the bias never leaves registers); each unit writes one record per row (8 bytes
//               {log-mass, score} for chunked noise).  The general path (k_bias: fp32 factors or
//               unaligned rows) uses 32-slot x 256-column units with 16-byte records.  "Plain
//               rows" (LSEP: the target row of the position being verified; BONUS) are streamed
//               in 4096-column items, one wave each (inside k_sweep_fast, or k_plain).
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

#include <atomic>

#include "spec_cycle.h"
#include "device_common.h"
#include "resident.h"

namespace spec {

enum : int { RO_DRAFT = 1, RO_CORRECT = 2, RO_LSEP = 4, RO_BONUS = 8 };
enum : int { PH_ALIVE = 0, PH_REJECTED = 1, PH_DONE = 2, PH_INVALID = 3 };

constexpr int NT = 256;             // threads per workgroup
constexpr int SUB = 32;             // bias slots per MFMA sub-block
constexpr int TILE_A = 256;         // vocabulary columns per bias-row unit: 4 waves x 64
constexpr int KB_LOADS = 8;                 // 16-byte loads per lane per plain-row item
constexpr int TILE_B = KB_LOADS * 64 * 8;   // vocabulary columns per plain-row item (4096): one wave
constexpr int MAX_B = 1024;
constexpr int MAX_K = 32;
constexpr int MAX_R = 256;
constexpr int MAX_BINS = 1024;      // calibration-error bins
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
  const int32_t* L_in;   // [B] given verify lengths (a scheduler's), or null: the prefix cut
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
  int32_t* live;       // [K + 2]: nonzero when some request has a row at step s (step 0 always; later
                       // steps set by the merge of the step before); the step kernels of a step with
                       // none return at once, and its stale role bytes are never read
  int32_t* slots;      // [3][B]: bias slot of DRAFT row, bias slot of CORRECT row, plain slot
  int32_t* xs;         // [B][K]
  uint64_t* kreq;      // [B] noise-key prefix of each request: first(first(seed) ^ global id)
  float* lse_q;        // [B][K]
  float* logq;         // [B][K]
  float* lse_p;        // [B][K+1]
  float* logp;         // [B][K]
  float4* part_bias;   // [bias slots][nrA]
  float4* part_bias2;  // [bias slots][nrA]  CORRECT rows: target-row fallback
  // bias-row partials of the chunked fast sweep: 8-byte {log-mass, score} records (the record's
  // index is its noise chunk), same row stride nrA, in the same buffers
  int part8;
  float4* part_plain;  // [B][nrB]
  const u32x4* konst;  // [2]: 16 zero bytes, then 8 bf16 -inf (stand-in source of masked tile loads)
  int nrA, nrB;
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
  if (blockIdx.x == 0 && threadIdx.x < 2) {
    const uint32_t w = threadIdx.x ? 0xFF80FF80u : 0u;
    ((u32x4*)p.konst)[threadIdx.x] = (u32x4){w, w, w, w};
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < p.K + 2) p.live[threadIdx.x] = (threadIdx.x == 0) ? 1 : 0;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  const int K = p.K;
  const float T = p.temp[b];
  const int x0 = p.x0 ? p.x0[b] : -1;
  bool valid = (T > 0.0f) && isfinite(T) && x0 >= -1 && x0 < p.V;
  int L = 0;
  if (p.L_in) {
    // verify length chosen by a scheduler: outside 0..K marks the request invalid
    L = p.L_in[b];
    if (L < 0 || L > K) {
      valid = false;
      L = 0;
    }
  } else {
    // prefix cut: keep position j while the fp64 running product of confidences is >= threshold
    double P = 1.0;
    for (int j = 0; j < K; j++) {
      P *= (double)p.conf[(size_t)b * K + j];
      if (!(P >= (double)p.threshold)) break;   // the first failure ends the prefix; NaN fails
      L = j + 1;
    }
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
template <int NTH>
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
  for (int i = 0; i < NTH / 64; i++) {
    uint64_t t = tmp[i];
    off += (i < w) ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return off + x - v;
}

struct Lists {
  int n_draft, n_correct, n_plain;
  int c0;     // first CORRECT slot: n_draft rounded up to a whole sub-block, so no sub-block mixes roles
  int n_sb;   // bias sub-blocks of SUB slots
};

constexpr uint16_t NO_ROW = 0xFFFF;   // bias slot without a row (alignment gap or tail)

// bias-list capacity: 2B rows plus the two alignment gaps
__host__ __device__ constexpr int bias_slots_max(int B) { return 2 * B + 2 * SUB; }

// One request's bias-row inputs at step s, staged in LDS by every bias-sweep workgroup.  A DRAFT
// row is position s; a CORRECT row is position s - 1 (the position rejected at step s - 1).  Every
// field is a plain load indexed by (b, s), so all of them are issued at once.
struct ReqMeta {
  int prev_d;        // token before position s (x0 at s = 0); -1 = no Markov bias
  int prev_c;        // token before position s - 1
  float invT;
  float lse_p_c;     // log-normalisers of the target and draft rows at position s - 1
  float lse_q_c;
  uint32_t key_d[2]; // sweep noise key of the DRAFT row (chunk stream for CHUNKED, index stream for
                     // FLAT), low word first
  uint32_t key_c[2]; // sweep noise key of the CORRECT row
};

__device__ __forceinline__ void put_key(uint32_t (&k)[2], uint64_t v) {
  k[0] = (uint32_t)v;
  k[1] = (uint32_t)(v >> 32);
}
__device__ __forceinline__ uint64_t get_key(const uint32_t (&k)[2]) { return (uint64_t)k[0] | ((uint64_t)k[1] << 32); }

__device__ __forceinline__ uint64_t key_from(uint64_t kreq, int pos, uint64_t stream) {
  return sm_first(sm_first(kreq ^ (uint64_t)pos) ^ stream);
}

// Scan the role bytes of step s into the compact row lists of this step, in LDS:
//   bias_list[i]  = (request << 1) | (1 if CORRECT): DRAFT rows in [0, n_draft), CORRECT rows in
//                   [c0, c0 + n_correct), NO_ROW in the gap and the tail up to n_sb * SUB
//   plain_list[i] = request, for plain slot i (LSEP or BONUS)
// With `req`, every request's bias-row inputs are staged too; their loads go out with the role
// loads, so the prologue costs one memory latency.  Workgroup 0 of a publishing kernel also writes
// every request's slots for the merge kernel.
template <int NOISE, int NTH>
__device__ Lists build_lists(const Params& p, int s, const uint8_t* roles, uint16_t* bias_list, uint16_t* plain_list,
                             uint64_t* tmp, ReqMeta* req, bool publish_slots) {
  const int per = (p.B + NTH - 1) / NTH;
  const int b0 = threadIdx.x * per;
  uint64_t cnt = 0;
  for (int i = 0; i < per; i++) {
    const int b = b0 + i;
    if (b < p.B) {
      const int r = roles[b];
      cnt += (uint64_t)((r & RO_DRAFT) ? 1 : 0) | ((uint64_t)((r & RO_CORRECT) ? 1 : 0) << 16) |
             ((uint64_t)((r & (RO_LSEP | RO_BONUS)) ? 1 : 0) << 32);
      if (req) {
        // read whether or not the request has a bias row this step (the values are then unused)
        const int x0 = p.x0 ? p.x0[b] : -1;
        const int32_t* xr = p.xs + (size_t)b * p.K;
        const int jc = s > 0 ? s - 1 : 0;
        ReqMeta m;
        m.prev_d = (s == 0) ? x0 : xr[s - 1];
        m.prev_c = (s <= 1) ? x0 : xr[s - 2];
        m.invT = 1.0f / p.temp[b];
        m.lse_p_c = p.lse_p[(size_t)b * (p.K + 1) + jc];
        m.lse_q_c = p.lse_q[(size_t)b * p.K + jc];
        const uint64_t kr = p.kreq[b];
        put_key(m.key_d, key_from(kr, s, NOISE == SPEC_NOISE_CHUNKED ? ST_DRAFT_C : ST_DRAFT));
        put_key(m.key_c, key_from(kr, jc, NOISE == SPEC_NOISE_CHUNKED ? ST_RESIDUAL_C : ST_RESIDUAL));
        req[b] = m;
      }
    }
  }
  uint64_t tot;
  const uint64_t pre = block_excl_scan<NTH>(cnt, tmp, &tot);
  Lists ls;
  ls.n_draft = (int)(tot & 0xFFFF);
  ls.n_correct = (int)((tot >> 16) & 0xFFFF);
  ls.n_plain = (int)((tot >> 32) & 0xFFFF);
  ls.c0 = (ls.n_draft + SUB - 1) / SUB * SUB;
  ls.n_sb = (ls.c0 + ls.n_correct + SUB - 1) / SUB;
  int d = (int)(pre & 0xFFFF), c = (int)((pre >> 16) & 0xFFFF), q = (int)((pre >> 32) & 0xFFFF);
  const bool publish = (blockIdx.x == 0) && publish_slots;
  for (int i = 0; i < per; i++) {
    const int b = b0 + i;
    if (b >= p.B) break;
    const int r = roles[b];
    int sd = -1, sc = -1, sp = -1;
    if (r & RO_DRAFT) { sd = d++; bias_list[sd] = (uint16_t)(b << 1); }
    if (r & RO_CORRECT) { sc = ls.c0 + c++; bias_list[sc] = (uint16_t)((b << 1) | 1); }
    if (r & (RO_LSEP | RO_BONUS)) { sp = q++; plain_list[sp] = (uint16_t)b; }
    if (publish) {
      p.slots[b] = sd;
      p.slots[p.B + b] = sc;
      p.slots[2 * p.B + b] = sp;
    }
  }
  if (threadIdx.x < SUB) {
    const int g = ls.n_draft + threadIdx.x;
    if (g < ls.c0) bias_list[g] = NO_ROW;
    const int t = ls.c0 + ls.n_correct + threadIdx.x;
    if (t < ls.n_sb * SUB) bias_list[t] = NO_ROW;
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


// log-sum-exp of invT * y over n values held by a lane and its partner lane (lane ^ 32), invT > 0:
// the scale is folded into the exponent argument, max(invT y) = invT max(y).  Branch-free, so that
// it schedules with independent work: every value -inf gives -inf, a NaN gives NaN.
template <int N>
__device__ __forceinline__ float pair_lse_scaled(const float* y, float invT) {
  // two max chains and four sum chains: independent partial results keep the pipeline busy
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    m0 = fmaxf(m0, y[i]);
    m1 = fmaxf(m1, y[i + 1]);
  }
  float mx = fmaxf(m0, m1);
  mx = fmaxf(mx, xor32f(mx));
  // with no finite maximum the offset is 0: the terms are 0 (-inf) or NaN
  const float c = invT * LOG2E, mo = (mx == -INFINITY) ? 0.0f : mx * c;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    s0 += ex2(fmaf(y[i], c, -mo));
    s1 += ex2(fmaf(y[i + 1], c, -mo));
    s2 += ex2(fmaf(y[i + 2], c, -mo));
    s3 += ex2(fmaf(y[i + 3], c, -mo));
  }
  float sum = (s0 + s1) + (s2 + s3);
  sum += xor32f(sum);
  return (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
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

// ------------------------------------------------------------------------------------------
// bias rows (DRAFT / CORRECT): the Markov bias A[prev] . W of every column, never written out,
// plus the element-wise work of the row; a 32-slot sub-block holds one role only.  General path
// (k_bias: fp32 factors or unaligned rows): a unit is (column range of 256, sub-block), the units of
// a step are split evenly over one workgroup per CU in range-major order, so a workgroup reloads its
// W fragments only when it crosses into the next column range.  The bf16 fast path follows below.
// ------------------------------------------------------------------------------------------
struct WaveOut {        // one wave's result for one row over its 64 columns (one noise chunk)
  float4 a;             // {log-mass, best score, best index (bits), aux}
  float4 b;             // CORRECT: target-row fallback {lse, best score, best index, 0}
};

// the bias row of one slot, resolved from the lists and the per-request table
struct RowMeta {
  int b, j, prev;
  bool active, corr;
  float invT, lse_p, lse_q;
  uint64_t key;
};

__device__ __forceinline__ RowMeta row_meta(const uint16_t* bias_list, const ReqMeta* req, int s, int slot) {
  RowMeta rm;
  const uint16_t e = bias_list[slot];
  rm.active = e != NO_ROW;
  rm.corr = rm.active && (e & 1);
  rm.b = rm.active ? (e >> 1) : 0;
  rm.j = rm.corr ? s - 1 : s;
  const ReqMeta& m = req[rm.b];
  rm.prev = !rm.active ? -1 : (rm.corr ? m.prev_c : m.prev_d);
  rm.invT = rm.active ? m.invT : 1.0f;
  rm.lse_p = rm.corr ? m.lse_p_c : 0.0f;
  rm.lse_q = rm.corr ? m.lse_q_c : 0.0f;
  rm.key = rm.corr ? get_key(m.key_c) : get_key(m.key_d);
  return rm;
}

// FLAT draft: best (s_v + G(key, v)) over the lane's 32 columns (element i is column
// v0 + 32 (i / 16) + i % 16), s = invT y with y in y[]
__device__ __forceinline__ void flat_best32(const float* y, float invT, int v0, int V, uint64_t key, float& best,
                                            int& bestv, float& bests) {
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const int v = v0 + 32 * (i >> 4) + (i & 15);
    if (v >= V) continue;
    const uint64_t w = pair_word(key, (uint32_t)v >> 1);
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const float sv = y[i + e] * invT;
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

// DRAFT row over the 64 columns of a lane pair (lanes l and l ^ 32): y = draft logits of the lane's 32
// columns, before the temperature (the row's logits are invT y).  Every lane runs the cross-lane
// steps; inactive rows return an empty part.
template <int NOISE>
__device__ __forceinline__ float4 draft_part(const float (&y)[32], const RowMeta& rm, int chunk, int v0, int V) {
  float4 o = empty_part();
  if (NOISE == SPEC_NOISE_CHUNKED) {
    // the chunk's noise does not depend on the logits: computed first, it overlaps the log-sum-exp
    const float g = gumbel_bits(bits_at(rm.key, (uint32_t)chunk));
    const float lse = pair_lse_scaled<32>(y, rm.invT);
    const float score = (lse > -INFINITY) ? lse + g : lse;
    o = rm.active ? make_float4(lse, score, __int_as_float(chunk), 0.0f) : o;
    return o;
  }
  const float lse = pair_lse_scaled<32>(y, rm.invT);
  float best = -INFINITY, bests = 0.0f;
  int bestv = -1;
  if (rm.active) flat_best32(y, rm.invT, v0, V, rm.key, best, bestv, bests);
  pair_best(best, bestv, bests);
  if (rm.active) o = make_float4(lse, best, __int_as_float(bestv), bests);
  return o;
}

// CORRECT row at the rejected position: residual norm(max(0, p - q)) and, for a residual with no
// mass, the target row itself.  y = draft logits, t = target logits of the lane's 32 columns, both
// before the temperature.  Log-probabilities are formed in base 2 with one fused multiply-add each.
template <int NOISE>
__device__ __forceinline__ void correct_part(const float (&y)[32], const float (&t)[32], const RowMeta& rm, int chunk,
                                             int v0, int V, float4& oa, float4& ob) {
  const float lse_t = pair_lse_scaled<32>(t, rm.invT);
  const float c = rm.invT * LOG2E, op = -rm.lse_p * LOG2E, oq = -rm.lse_q * LOG2E;
  float mass = 0.0f;
  float br = -INFINITY, bp = -INFINITY, dummy = 0.0f;
  int vr = -1, vp = -1;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const float lp2 = fmaf(t[i], c, op), lq2 = fmaf(y[i], c, oq);
    if (lp2 > lq2) mass += ex2(lp2) - ex2(lq2);
  }
  if (NOISE == SPEC_NOISE_FLAT && rm.active) {
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const int v = v0 + 32 * (i >> 4) + (i & 15);
      if (v >= V) continue;
      const float g = gumbel_bits(bits_at(rm.key, (uint32_t)v));
      const float ts = t[i] * rm.invT;
      const float lp = ts - rm.lse_p, lq = y[i] * rm.invT - rm.lse_q;
      if (lp > lq) {
        const float sc = lp + logf(-expm1f(lq - lp)) + g;
        if (better(sc, v, br, vr)) { br = sc; vr = v; }
      }
      if (ts > -INFINITY && better(ts + g, v, bp, vp)) { bp = ts + g; vp = v; }
    }
  }
  mass += xor32f(mass);
  pair_best(br, vr, dummy);
  pair_best(bp, vp, dummy);
  oa = empty_part();
  ob = empty_part();
  if (!rm.active) return;
  const float lmass = (mass > 0.0f) ? lg2(mass) * LN2 : -INFINITY;
  if (NOISE == SPEC_NOISE_CHUNKED) {
    const float g = gumbel_bits(bits_at(rm.key, (uint32_t)chunk));
    oa = make_float4(lmass, lmass > -INFINITY ? lmass + g : -INFINITY, __int_as_float(chunk), 0.0f);
    ob = make_float4(lse_t, lse_t > -INFINITY ? lse_t + g : -INFINITY, __int_as_float(chunk), 0.0f);
  } else {
    oa = make_float4(lmass, br, __int_as_float(vr), 0.0f);
    ob = make_float4(lse_t, bp, __int_as_float(vp), 0.0f);
  }
}

// partials of one finished unit from red (threads 0..31)
__device__ __forceinline__ void unit_flush(const Params& p, const uint16_t* bias_list, const WaveOut (*red)[SUB],
                                           int slot0, int range) {
  if (threadIdx.x < SUB) {
    const int r = threadIdx.x, slot = slot0 + r;
    const uint16_t e = bias_list[slot];
    if (e != NO_ROW) {
      float4 pa = red[0][r].a;
#pragma unroll
      for (int w = 1; w < NT / 64; w++) pa = merge_part(pa, red[w][r].a);
      p.part_bias[(size_t)slot * p.nrA + range] = pa;
      if (e & 1) {
        float4 pb = red[0][r].b;
#pragma unroll
        for (int w = 1; w < NT / 64; w++) pb = merge_part(pb, red[w][r].b);
        p.part_bias2[(size_t)slot * p.nrA + range] = pb;
      }
    }
  }
}

// W fragments of column range `range`: MFMA A-operand row i of fragment f is column
// vw + 32 f + perm(i), perm chosen so that accumulator q of lane l holds column vw + 32 f +
// 16 (l / 32) + q; lane half l / 32 covers k in [R/2 (l/32), R/2 (l/32 + 1))
__device__ __forceinline__ void load_w(const Params& p, int range, bf16x8 (&wf)[2][16]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int R = p.R, T16 = R >> 4, kb = h * (R >> 1);
  const int col_in = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int vw = range * TILE_A + 64 * wave;
  // Fragments past V or past the rank are zero.  They are read from the 16-byte zero constant
  // rather than selected after the load, which would wait for it.
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int v = vw + 32 * f + col_in;
    const bool in = v < p.V;
    const uint16_t* wr = (const uint16_t*)p.W + (size_t)v * R + kb;
#pragma unroll
    for (int t = 0; t < 16; t++)
      wf[f][t] = *((in && t < T16) ? (const bf16x8*)(wr + 8 * t) : (const bf16x8*)p.konst);
  }
  // the fragments live in accumulation registers (the MFMA reads its A operand from there), which
  // leaves the vector registers to the logit tiles and the B operands
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int t = 0; t < 16; t++) asm volatile("" : "+a"(wf[f][t]));
}

// Markov bias of the lane's 32 columns (element i: column v0 + 32 (i / 16) + i % 16) for row
// m = lane % 32 of the sub-block whose A rows sit in sA
__device__ __forceinline__ void mfma_bias(const bf16x8 (&wf)[2][16], const uint16_t (*sA)[MAX_R + A_PAD], int R,
                                          float (&x)[32]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
  const int T16 = R >> 4, kb = h * (R >> 1);
  f32x16 acc0 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  f32x16 acc1 = acc0;
  // every B operand is read before the first MFMA, so the LDS latency is paid once
  bf16x8 bop[16];
#pragma unroll
  for (int t = 0; t < 16; t++) bop[t] = *(const bf16x8*)&sA[m][kb + 8 * (t < T16 ? t : 0)];
  __builtin_amdgcn_sched_barrier(0);   // keep all reads ahead of the MFMA chain
#pragma unroll
  for (int t = 0; t < 16; t++) {
    // for t >= R/16 both operands are zero (zero W fragments; sA zero past the rank)
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][t], bop[t], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][t], bop[t], acc1, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 16; q++) {
    x[q] = acc0[q];
    x[16 + q] = acc1[q];
  }
}

// ---- generic sweep: fp32 factors, or bf16 rows that are not 16-byte aligned / V % 8 != 0 ----

// fp32 factors: Markov bias of 16 consecutive columns by VALU dot products (small vocabularies)
__device__ __forceinline__ void fp32_bias16(const Params& p, int prev, int vstart, float* x) {
  const int R = p.R;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const int v = vstart + q;
    float a = 0.0f;
    if (prev >= 0 && v < p.V) {
      const float* wr = (const float*)p.W + (size_t)v * R;
      const float* ar = (const float*)p.A + (size_t)prev * R;
      for (int k = 0; k < R; k++) a = fmaf(ar[k], wr[k], a);
    }
    x[q] = a;
  }
}

struct GenericLds {
  uint16_t sA[SUB][MAX_R + A_PAD];   // A rows of the current unit (bf16)
  WaveOut red[NT / 64][SUB];
};

template <int DT, int NOISE, bool VEC>
__device__ void bias_sweep_generic(const Params& p, int s, const Lists& ls, const uint16_t* bias_list,
                                   const ReqMeta* req, GenericLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int V = p.V, R = p.R, K = p.K;
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const int nsb = ls.n_sb;
  const long long units = (long long)p.nrA * nsb;
  const int u0 = (int)(units * blockIdx.x / gridDim.x);
  const int u1 = (int)(units * (blockIdx.x + 1) / gridDim.x);
  if (u0 >= u1) return;
  bf16x8 wf[2][16];
  int w_range = -1;
  for (int u = u0; u < u1; u++) {
    const int range = u / nsb, slot0 = (u % nsb) * SUB;
    const bool corr_unit = slot0 >= ls.c0;
    __syncthreads();   // the previous unit is done with sA and red
    if (u > u0) unit_flush(p, bias_list, L.red, ((u - 1) % nsb) * SUB, (u - 1) / nsb);
    if (DT == SPEC_BF16) {
      const int segs = R >> 3;
      for (int e = threadIdx.x; e < SUB * segs; e += NT) {
        const int row = e / segs, sg = e - row * segs;
        const RowMeta rr = row_meta(bias_list, req, s, slot0 + row);
        u32x4 val = {0, 0, 0, 0};
        if (rr.prev >= 0) val = *(const u32x4*)((const uint16_t*)p.A + (size_t)rr.prev * R + 8 * sg);
        *(u32x4*)&L.sA[row][8 * sg] = val;
      }
    }
    __syncthreads();   // sA holds this unit's A rows; red is free
    if (DT == SPEC_BF16 && range != w_range) load_w(p, range, wf);
    w_range = range;

    const int vw = range * TILE_A + 64 * wave;   // this wave's 64 columns: one noise chunk
    const int chunk = vw / CHUNK;
    const int v0 = vw + 16 * h;
    const RowMeta rm = row_meta(bias_list, req, s, slot0 + m);
    float x[32];
    if (DT == SPEC_BF16) {
      mfma_bias(wf, L.sA, R, x);
    } else {
      fp32_bias16(p, rm.prev, v0, x);
      fp32_bias16(p, rm.prev, v0 + 32, x + 16);
    }
    {
      float bx[32];
#pragma unroll
      for (int i = 0; i < 32; i++) bx[i] = -INFINITY;
      const void* base_row = (const char*)p.base + ((size_t)rm.b * K + rm.j) * (size_t)V * esz;
      if (rm.active) {
        load16<DT, VEC>(base_row, v0, V, *(float(*)[16])bx);
        load16<DT, VEC>(base_row, v0 + 32, V, *(float(*)[16])(bx + 16));
      }
#pragma unroll
      for (int i = 0; i < 32; i++) x[i] = rm.active ? bx[i] + x[i] : -INFINITY;
    }
    WaveOut o;
    if (!corr_unit) {
      o.a = draft_part<NOISE>(x, rm, chunk, v0, V);
      o.b = empty_part();
    } else {
      float t[32];
#pragma unroll
      for (int i = 0; i < 32; i++) t[i] = -INFINITY;
      const void* targ_row = (const char*)p.target + ((size_t)rm.b * (K + 1) + rm.j) * (size_t)V * esz;
      if (rm.active) {
        load16<DT, VEC>(targ_row, v0, V, *(float(*)[16])t);
        load16<DT, VEC>(targ_row, v0 + 32, V, *(float(*)[16])(t + 16));
      }
#pragma unroll
      for (int i = 0; i < 32; i++) t[i] = rm.active ? t[i] : -INFINITY;
      correct_part<NOISE>(x, t, rm, chunk, v0, V, o.a, o.b);
    }
    if (h == 0) L.red[wave][m] = o;
  }
  __syncthreads();
  unit_flush(p, bias_list, L.red, ((u1 - 1) % nsb) * SUB, (u1 - 1) / nsb);
}

// ---- fast sweep: bf16, 16-byte aligned rows, V % 8 == 0 ----
// One workgroup of 4 waves per CU (one wave per SIMD, the full register file each).  The gathered
// A rows of the first bias slots (up to 288, as many as LDS holds) are staged in LDS once per step,
// then one barrier; after that every wave runs on its own: a unit is (noise chunk of 64 columns,
// sub-block of 32 slots), the wave holds the chunk's W fragments in accumulation registers (128 of
// them for R = 256), reads the sub-block's B operands from LDS (from the A table for sub-blocks past
// the staged ones), loads the draft / target logits straight into registers in the accumulator
// layout two units ahead, and writes the chunk record of each row directly to the partials.  All
// units of the step are split evenly over all waves of the grid in chunk-major order, so W streams
// once per step, a wave reloads W only when it crosses into the next chunk, and it issues that
// reload right after the last MFMA chain on the old fragments.

// dynamic LDS of the bias-row sweeps: per-request table [B], then the bias and plain lists
__host__ __device__ constexpr size_t bias_dyn_bytes(int B) {
  return (size_t)B * sizeof(ReqMeta) + (size_t)(bias_slots_max(B) + B) * sizeof(uint16_t);
}
constexpr int SA_STRIDE = MAX_R + A_PAD;   // bf16 elements per staged A row
// dynamic LDS of k_sweep_fast with the A rows of g slots staged
__host__ __device__ constexpr size_t fast_dyn_bytes(int B, int g) {
  return (bias_dyn_bytes(B) + 15) / 16 * 16 + (size_t)g * SA_STRIDE * sizeof(uint16_t);
}

// draft-logit tiles are prefetched FAST_DEPTH units ahead (two measured faster than three to six)
constexpr int FAST_DEPTH = 2;
struct TileRegs {
  u32x4 x[4];   // logits of the lane's 32 columns of one row (two pieces per MFMA tile)
};

// W fragments of noise chunk c: MFMA A-operand row i of fragment f is column 64 c + 32 f + perm(i),
// perm chosen so that accumulator q of lane l holds column 64 c + 32 f + 16 (l / 32) + q; lane half
// l / 32 covers k in [R/2 (l/32), R/2 (l/32 + 1)).  Columns past V read row 0 of W (finite values
// whose products land in columns whose logits are -inf); fragments past the rank are zero.
__device__ __forceinline__ void load_w_chunk(const Params& p, int c, bf16x8 (&wf)[2][16]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
  const int R = p.R, T16 = R >> 4, kb = h * (R >> 1);
  const int col_in = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int v = CHUNK * c + 32 * f + col_in;
    const bf16x8* wr = (const bf16x8*)((const uint16_t*)p.W + (size_t)(v < p.V ? v : 0) * R + kb);
    if (T16 == 16) {
#pragma unroll
      for (int t = 0; t < 16; t++) wf[f][t] = wr[t];
    } else {
#pragma unroll
      for (int t = 0; t < 16; t++) wf[f][t] = *(t < T16 ? wr + t : (const bf16x8*)p.konst);
    }
  }
}

// A rows of bias slots g0 .. g0 + rows - 1 into sA (every thread; rows without a Markov bias and
// the alignment gaps read zeros), STAGE_BATCH loads per thread in flight (32, one round for a full
// group, measured no faster)
constexpr int STAGE_BATCH = 8;
__device__ __forceinline__ void stage_a(const Params& p, const uint16_t* bias_list, const ReqMeta* req, int g0, int rows,
                                        uint16_t* sA) {
  const int segs = p.R >> 3, n = rows * segs;
  for (int e0 = 0; e0 < n; e0 += STAGE_BATCH * NT) {
    u32x4 v[STAGE_BATCH];
#pragma unroll
    for (int i = 0; i < STAGE_BATCH; i++) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      int prev = -1, sg = 0;
      if (e < n) {
        const int row = e / segs;
        sg = e - row * segs;
        const uint16_t ent = bias_list[g0 + row];
        if (ent != NO_ROW) prev = (ent & 1) ? req[ent >> 1].prev_c : req[ent >> 1].prev_d;
      }
      v[i] = *((prev >= 0) ? (const u32x4*)((const uint16_t*)p.A + (size_t)prev * p.R + 8 * sg) : p.konst);
    }
#pragma unroll
    for (int i = 0; i < STAGE_BATCH; i++) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      if (e < n) {
        const int row = e / segs;
        *(u32x4*)&sA[row * SA_STRIDE + 8 * (e - row * segs)] = v[i];
      }
    }
  }
}

// A unit's place in the wave's span: index, noise chunk, sub-block (all wave-uniform)
struct UPos {
  int u, c, k;
};

// the unit after q, or q itself at the end of the span
__device__ __forceinline__ UPos upos_next(UPos q, int nsbg, int u1) {
  if (q.u + 1 < u1) {
    q.u++;
    if (++q.k == nsbg) {
      q.k = 0;
      q.c++;
    }
  }
  return q;
}

// Logit tiles of unit q (sub-block q.k of the group starting at slot g0, chunk q.c): the draft row
// (target = false) or the target row (target = true, CORRECT units).  A slot without a row loads
// request 0's row (its results are never stored); columns past V (a partial last chunk only) read
// the 16-byte -inf constant instead.
__device__ __forceinline__ void tile_issue(const Params& p, int s, const uint16_t* bias_list, int g0, UPos q,
                                           bool target, TileRegs& T) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
  const uint16_t ent = bias_list[g0 + q.k * SUB + m];
  // a slot without a row (NO_ROW has its low bit set too) reads row 0 of request 0: always in bounds
  const bool has = ent != NO_ROW;
  const int b = has ? (ent >> 1) : 0;
  const int j = !has ? 0 : ((ent & 1) ? s - 1 : s);   // CORRECT rows (s >= 1): position s - 1
  const int v0 = CHUNK * q.c + 16 * h;   // + 32 (i / 2) + 8 (i % 2)
  const u32x4* row = target ? (const u32x4*)((const uint16_t*)p.target + (size_t)(b * (p.K + 1) + j) * p.V + v0)
                            : (const u32x4*)((const uint16_t*)p.base + (size_t)(b * p.K + j) * p.V + v0);
  if (CHUNK * (q.c + 1) <= p.V) {
#pragma unroll
    for (int i = 0; i < 4; i++) T.x[i] = row[4 * (i >> 1) + (i & 1)];
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int col = v0 + 32 * (i >> 1) + 8 * (i & 1);
      T.x[i] = *(col < p.V ? row + 4 * (i >> 1) + (i & 1) : p.konst + 1);
    }
  }
}

// bf16 pieces of the lane's 32 columns -> floats (element i: column v0 + 32 (i / 16) + i % 16)
__device__ __forceinline__ void unpack32(const u32x4 (&w)[4], float (&o)[32]) {
#pragma unroll
  for (int k = 0; k < 4; k++) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      o[8 * k + 2 * i] = bf16_lo(w[k][i]);
      o[8 * k + 2 * i + 1] = bf16_hi(w[k][i]);
    }
  }
}

// B operands of sub-block k at constant offsets: for t >= R/16 they read the zeroed columns
// [R, MAX_R) of the row
__device__ __forceinline__ void read_bop(const Params& p, const uint16_t* sA, int k, bf16x8 (&bop)[16]) {
  const int lane = threadIdx.x & 63;
  const uint16_t* arow = sA + (k * SUB + (lane & 31)) * SA_STRIDE + (lane >> 5) * (p.R >> 1);
#pragma unroll
  for (int t = 0; t < 16; t++) bop[t] = *(const bf16x8*)(arow + 8 * t);
}
// the same B operands for a sub-block past the staged ones, straight from the A table (its rows are
// hot in L2: every workgroup reads them); prev < 0 and the columns past the rank read zeros
__device__ __forceinline__ void read_bop_global(const Params& p, int prev, bf16x8 (&bop)[16]) {
  const int lane = threadIdx.x & 63;
  const int T16 = p.R >> 4;
  const uint16_t* ar = (const uint16_t*)p.A + (size_t)(prev >= 0 ? prev : 0) * p.R + (lane >> 5) * (p.R >> 1);
#pragma unroll
  for (int t = 0; t < 16; t++)
    bop[t] = *((prev >= 0 && t < T16) ? (const bf16x8*)(ar + 8 * t) : (const bf16x8*)p.konst);
}

// One unit cur of the wave's span (nx = the unit after it, is = the unit FAST_DEPTH after it, both
// clamped to the span) over nsbg sub-blocks starting at slot g0, the first kst of them staged in LDS.
// Tcur holds cur's draft tiles and receives is's; Tt holds cur's target tiles if cur is a CORRECT
// unit and receives nx's if that one is; rm holds cur's row meta and leaves with nx's.  Order: B
// operands (from LDS, or from the A table past the staged sub-blocks) and the next row meta, the
// draft tile unpacked into the accumulators (while those reads land); the MFMA chain; the next
// chunk's W fragments if the chunk changes; the element-wise part; the records; the next loads.
template <int NOISE>
__device__ __forceinline__ void fast_unit(const Params& p, int s, const Lists& ls, const uint16_t* bias_list,
                                          const ReqMeta* req, const uint16_t* sA, int kst, int g0, UPos cur, UPos nx,
                                          UPos is, bool last, bf16x8 (&wf)[2][16], TileRegs& Tcur, TileRegs& Tt,
                                          RowMeta& rm) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
  const int c = cur.c;
  const int slot0 = g0 + cur.k * SUB;
  bf16x8 bop[16];
  if (cur.k < kst) read_bop(p, sA, cur.k, bop);
  else read_bop_global(p, rm.prev, bop);
  const RowMeta rn = row_meta(bias_list, req, s, g0 + nx.k * SUB + m);
  __builtin_amdgcn_sched_barrier(0);   // keep all reads ahead of the MFMA chain
  // the W fragments live in accumulation registers (the MFMA reads its A operand from there), which
  // leaves the vector registers to the logit tiles and the B operands
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int t = 0; t < 16; t++) asm volatile("" : "+a"(wf[f][t]));
  float y[32];
  {
    // the accumulators start from the draft logits, so the chain leaves base + bias (its unpack runs
    // while the B operands arrive from LDS)
    float bx[32];
    unpack32(Tcur.x, bx);
    f32x16 acc0, acc1;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      acc0[q] = bx[q];
      acc1[q] = bx[16 + q];
    }
#pragma unroll
    for (int t = 0; t < 16; t++) {
      // for t >= R/16 both operands are zero (zero W fragments; zeroed A columns)
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][t], bop[t], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][t], bop[t], acc1, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 16; q++) {
      y[q] = acc0[q];
      y[16 + q] = acc1[q];
    }
  }
  // the next unit's chunk: its W fragments load while this unit's element-wise part runs
  if (!last && nx.c != c) load_w_chunk(p, nx.c, wf);
  const int v0 = CHUNK * c + 16 * h;
  float4 oa, ob;
  if (slot0 < ls.c0) {
    oa = draft_part<NOISE>(y, rm, c, v0, p.V);
    ob = empty_part();
  } else {
    float t[32];
    unpack32(Tt.x, t);
    correct_part<NOISE>(y, t, rm, c, v0, p.V, oa, ob);
  }
  if (h == 0 && rm.active) {
    const size_t i = (size_t)(slot0 + m) * p.nrA + c;
    if (NOISE == SPEC_NOISE_CHUNKED) {
      // the chunk index is the record's place in the row
      ((float2*)p.part_bias)[i] = make_float2(oa.x, oa.y);
      if (rm.corr) ((float2*)p.part_bias2)[i] = make_float2(ob.x, ob.y);
    } else {
      p.part_bias[i] = oa;
      if (rm.corr) p.part_bias2[i] = ob;
    }
  }
  rm = rn;
  tile_issue(p, s, bias_list, g0, is, false, Tcur);
  if (!last && g0 + nx.k * SUB >= ls.c0) tile_issue(p, s, bias_list, g0, nx, true, Tt);
}

// `between` runs after every FAST_DEPTH units of a wave (the fused kernel puts one plain item there)
template <int NOISE, typename Between>
__device__ void bias_sweep_fast(const Params& p, int s, const Lists& ls, const uint16_t* bias_list, const ReqMeta* req,
                                uint16_t* sA, int G, Between& between) {
  const int nslots = ls.n_sb * SUB;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
  if (p.R < MAX_R) {
    // the MFMA chain always runs over the full rank: A columns [R, MAX_R) of every staged row read
    // as zero (stage_a writes only the first R)
    const int zc = (MAX_R - p.R) / 8;
    for (int e = threadIdx.x; e < G * zc; e += NT)
      *(u32x4*)&sA[(e / zc) * SA_STRIDE + p.R + 8 * (e % zc)] = (u32x4){0u, 0u, 0u, 0u};
  }
  const int gw = blockIdx.x * (NT / 64) + wave, nw = gridDim.x * (NT / 64);
  // one pass over every sub-block, so W streams once per step: the A rows of the first G slots are
  // staged in LDS, the sub-blocks past them read their B operands from the A table
  {
    const int g0 = 0, nsbg = ls.n_sb, kst = min(G, nslots) / SUB;
    stage_a(p, bias_list, req, g0, kst * SUB, sA);
    __syncthreads();
    const long long units = (long long)p.nrA * nsbg;
    const int u0 = (int)(units * gw / nw), u1 = (int)(units * (gw + 1) / nw);
    if (u0 < u1) {
      bf16x8 wf[2][16];
      TileRegs T[FAST_DEPTH], Tt;
      UPos cur = {u0, u0 / nsbg, u0 % nsbg};
      UPos is = cur;
      load_w_chunk(p, cur.c, wf);
#pragma unroll
      for (int d = 0; d < FAST_DEPTH; d++) {
        tile_issue(p, s, bias_list, g0, is, false, T[d]);
        is = upos_next(is, nsbg, u1);
      }
      if (g0 + cur.k * SUB >= ls.c0) tile_issue(p, s, bias_list, g0, cur, true, Tt);
      RowMeta rm = row_meta(bias_list, req, s, g0 + cur.k * SUB + (threadIdx.x & 31));
      for (int u = u0; u < u1; u += FAST_DEPTH) {
#pragma unroll
        for (int d = 0; d < FAST_DEPTH; d++) {
          if (u + d < u1) {
            const UPos nx = upos_next(cur, nsbg, u1);
            fast_unit<NOISE>(p, s, ls, bias_list, req, sA, kst, g0, cur, nx, is, u + d + 1 == u1, wf, T[d], Tt, rm);
            cur = nx;
            is = upos_next(is, nsbg, u1);
          }
        }
        between();
      }
    }
  }
}

// Wave-wide reductions (every lane gets the result): DPP within each 16-lane row (xor 1, xor 2, half-
// row mirror, row mirror), one lane shuffle across rows (xor 16), one lane swap across halves (xor 32).
__device__ __forceinline__ float wave_max64(float x) {
  x = max8(x);
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, xor32f(x));
}
__device__ __forceinline__ float wave_sum64(float x) {
  x = sum8(x);
  x += dpp<0x140>(x);
  x += __shfl_xor(x, 16, 64);
  return x + xor32f(x);
}

// one all-reduce step of the winner (larger score, smaller index on ties, index < 0 = none) with the
// partner values sc2, ix2, aux2
__device__ __forceinline__ void argmax_take(float& sc, int& ix, float& aux, float sc2, int ix2, float aux2) {
  const bool take = (ix2 >= 0) & ((ix < 0) | (sc2 > sc) | ((sc2 == sc) & ((unsigned)ix2 < (unsigned)ix)));
  sc = take ? sc2 : sc;
  ix = take ? ix2 : ix;
  aux = take ? aux2 : aux;
}

template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& sc, int& ix, float& aux) {
  argmax_take(sc, ix, aux, dpp<CTRL>(sc), __builtin_amdgcn_update_dpp(0, ix, CTRL, 0xF, 0xF, false), dpp<CTRL>(aux));
}

__device__ __forceinline__ void wave_argmax64(float& sc, int& ix, float& aux) {
  argmax_dpp<0xB1>(sc, ix, aux);
  argmax_dpp<0x4E>(sc, ix, aux);
  argmax_dpp<0x141>(sc, ix, aux);
  argmax_dpp<0x140>(sc, ix, aux);
  argmax_take(sc, ix, aux, __shfl_xor(sc, 16, 64), __shfl_xor(ix, 16, 64), __shfl_xor(aux, 16, 64));
  argmax_take(sc, ix, aux, xor32f(sc), xor32i(ix), xor32f(aux));
}

// ------------------------------------------------------------------------------------------
// plain target rows (LSEP / BONUS): items of TILE_B columns, one wave each, no barrier; every load
// of the item is issued before any arithmetic
// ------------------------------------------------------------------------------------------
// layout: load k (0 .. KB_LOADS - 1) of lane l covers 8 columns at 512 k + 8 l of the item, so
// every load instruction reads 1 KiB of contiguous memory; the 64 columns of a noise chunk are the
// 8 values of 8 neighbouring lanes, and lane l keeps the chunk of round l % 8.
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

// The target-row pieces of one plain item: load k of lane l covers columns 512 k + 8 l of the item.
template <int DT>
struct PlainRaw {
  Raw8<DT> r[KB_LOADS];
  int role;     // the request's role byte at this step and its temperature, loaded with the pieces
  float temp;   // (used right after they land, they would otherwise cost a memory round per item)
};

template <int DT, bool VEC>
__device__ __forceinline__ void plain_load(const Params& p, int s, int b, int range, PlainRaw<DT>& R) {
  const int K = p.K, V = p.V;
  const int lane = threadIdx.x & 63;
  const int j = s;   // LSEP verifies position s; BONUS reads row L_b == s
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const void* row = (const char*)p.target + ((size_t)b * (K + 1) + j) * (size_t)V * esz;
  const int vt = range * TILE_B + 8 * lane;   // + 512 k
  Raw8<DT>* r = R.r;
  R.role = p.roles[(size_t)(s & 1) * p.B + b];
  R.temp = p.temp[b];
  if (VEC) {
    // rows are 16-byte aligned and V % 8 == 0 (bf16) / V % 4 == 0 (fp32), so each 16-byte load
    // is wholly inside or wholly past the row end: predicate the loads, pad with -inf
    const uint32_t ninf = (DT == SPEC_BF16) ? 0xFF80FF80u : 0xFF800000u;
#pragma unroll
    for (int k = 0; k < KB_LOADS; k++) {
      const u32x4* q = (const u32x4*)((const char*)row + (size_t)(vt + 512 * k) * esz);
#pragma unroll
      for (int u = 0; u < (DT == SPEC_BF16 ? 1 : 2); u++) {
        const int vv = vt + 512 * k + 4 * u;
        if (vv < V) r[k].w[u] = q[u];   // ordinary loads: non-temporal ones stream at about half the rate
        else r[k].w[u] = (u32x4){ninf, ninf, ninf, ninf};
      }
    }
  } else {
    // unaligned rows: the same layout filled element by element, -inf past the row end
#pragma unroll 1
    for (int k = 0; k < KB_LOADS; k++) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int v = vt + 512 * k + i;
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
}

// the log-mass (and for a BONUS row the Gumbel winner) of one plain item from its loaded pieces.
// DIRECT: an LSEP item's log-mass in one pass over the item instead of chunk by chunk (fewer
// instructions, more live registers: only where the register file allows it)
template <int DT, int NOISE, bool DIRECT = false>
__device__ __forceinline__ void plain_finish(const Params& p, int s, int b, int pslot, int range,
                                             const PlainRaw<DT>& R) {
  const int V = p.V;
  const int lane = threadIdx.x & 63;
  const int role = R.role & (RO_LSEP | RO_BONUS);
  const int j = s;
  const float invT = 1.0f / R.temp;
  const int vbase = range * TILE_B;
  const int vt = vbase + 8 * lane;   // + 512 k
  const Raw8<DT>* r = R.r;
  const uint64_t g = (uint64_t)(p.req_off + b);
  const float sc2 = invT * LOG2E;
  if (DIRECT && role != RO_BONUS) {
    // LSEP: only the item's log-mass is needed, as one maximum and one scaled sum over the lane's 64
    // values and then over the wave (with a finite maximum the plain scaled sum; every value -inf
    // gives -inf, a NaN gives NaN)
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB_LOADS; k++)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        m0 = fmaxf(m0, raw8_at<DT>(r[k], i));
        m1 = fmaxf(m1, raw8_at<DT>(r[k], i + 1));
      }
    const float mx = wave_max64(fmaxf(m0, m1));
    const float mo = (mx == -INFINITY) ? 0.0f : mx * sc2;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int k = 0; k < KB_LOADS; k++)
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        s0 += ex2(fmaf(raw8_at<DT>(r[k], i), sc2, -mo));
        s1 += ex2(fmaf(raw8_at<DT>(r[k], i + 1), sc2, -mo));
        s2 += ex2(fmaf(raw8_at<DT>(r[k], i + 2), sc2, -mo));
        s3 += ex2(fmaf(raw8_at<DT>(r[k], i + 3), sc2, -mo));
      }
    const float sum = wave_sum64((s0 + s1) + (s2 + s3));
    const float lse = (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
    if (lane == 0) p.part_plain[(size_t)pslot * p.nrB + range] = make_float4(lse, -INFINITY, __int_as_float(-1), 0.0f);
    return;
  }
  // log-mass of each 64-column chunk (8 lanes x 8 values).  The rounds are independent and written
  // without branches, so that they interleave: with a finite maximum the arithmetic is the plain
  // scaled sum; every value -inf gives -inf, and a NaN among -inf values gives NaN.
  float own = -INFINITY;
#pragma unroll
  for (int k = 0; k < KB_LOADS; k++) {
    float mx = raw8_at<DT>(r[k], 0);
#pragma unroll
    for (int i = 1; i < 8; i++) mx = fmaxf(mx, raw8_at<DT>(r[k], i));
    mx = max8(mx);
    const float mo = (mx == -INFINITY) ? 0.0f : mx * sc2;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      s0 += ex2(fmaf(raw8_at<DT>(r[k], i), sc2, -mo));
      s1 += ex2(fmaf(raw8_at<DT>(r[k], i + 1), sc2, -mo));
    }
    const float sum = sum8(s0 + s1);
    const float lse = (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
    own = ((lane & 7) == k) ? lse : own;
  }
  float4 part = make_float4(own, -INFINITY, __int_as_float(-1), 0.0f);
  if (role == RO_BONUS) {
    if (NOISE == SPEC_NOISE_CHUNKED) {
      const uint64_t k1 = row_key(p.seed, g, (uint64_t)j, ST_BONUS_C);
      const int c = (vbase + 512 * (lane & 7)) / CHUNK + (lane >> 3);
      if (own > -INFINITY) {
        part.y = own + gumbel_bits(bits_at(k1, (uint32_t)c));
        part.z = __int_as_float(c);
      }
    } else {
      const uint64_t k2 = row_key(p.seed, g, (uint64_t)j, ST_BONUS);
      float best = -INFINITY;
      int bv = -1;
#pragma unroll 1
      for (int k = 0; k < KB_LOADS; k++) {
        const int v0 = vt + 512 * k;
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
  // wave reduction: the log-mass as one maximum and one scaled sum over the 64 lanes (every value
  // -inf gives -inf, a NaN gives NaN); for a BONUS row also the winner (the role is the same for the
  // whole wave)
  {
    const float mx = wave_max64(part.x);
    const float mo = (mx == -INFINITY) ? 0.0f : mx * LOG2E;
    const float sum = wave_sum64(ex2(fmaf(part.x, LOG2E, -mo)));
    part.x = (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx + lg2(sum) * LN2;
  }
  if (role == RO_BONUS) {
    float sc = part.y, aux = part.w;
    int ix = __float_as_int(part.z);
    wave_argmax64(sc, ix, aux);
    part.y = sc;
    part.z = __int_as_float(ix);
    part.w = aux;
  }
  if (lane == 0) p.part_plain[(size_t)pslot * p.nrB + range] = part;
}

template <int DT, int NOISE, bool VEC>
__device__ __forceinline__ void plain_item(const Params& p, int s, int b, int pslot, int range) {
  PlainRaw<DT> R;
  plain_load<DT, VEC>(p, s, b, range, R);
  plain_finish<DT, NOISE>(p, s, b, pslot, range, R);
}

// Row sweeps of one step.  Every workgroup rebuilds the step's row lists from the role bytes;
// the bias-row sweep also stages each request's bias-row inputs.  The bias sweeps run one
// workgroup per CU (the W fragments fill the register file); k_plain streams the target rows of
// LSEP / BONUS roles, one wave per item, six workgroups per CU.
// dynamic LDS of the plain-row sweep: bias and plain lists
__host__ __device__ constexpr size_t plain_dyn_bytes(int B) { return (size_t)(bias_slots_max(B) + B) * sizeof(uint16_t); }

// bf16 fast path: bias rows and plain rows of a step in one launch.  Every wave first sweeps its
// share of the bias units, then its workgroup's share of the plain items (one wave per item), so the
// plain rows fill the time the bias rows leave and the step costs one dispatch less.  Dynamic LDS:
// the per-request table, the lists, then the A rows of G bias slots.
template <int NOISE>
__global__ __launch_bounds__(NT, 1) void k_sweep_fast(Params p, int s, int G) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_bias[];
  __shared__ uint64_t scan_tmp[NT / 64];
  if (p.live[s] == 0) return;
  ReqMeta* req = (ReqMeta*)dyn_bias;
  uint16_t* bias_list = (uint16_t*)(dyn_bias + (size_t)p.B * sizeof(ReqMeta));
  uint16_t* plain_list = bias_list + bias_slots_max(p.B);
  uint16_t* sA = (uint16_t*)(dyn_bias + (bias_dyn_bytes(p.B) + 15) / 16 * 16);
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;
  const Lists ls = build_lists<NOISE, NT>(p, s, roles, bias_list, plain_list, scan_tmp, req, true);
  // Plain items of this workgroup, wave w taking items i0 + w, i0 + w + 4, ...: one after every pair of
  // bias units (its row loads issued a pair of units earlier, so their latency passes under the bias
  // work), the rest afterwards with PLAIN_DEPTH items' loads in flight.  Item positions (plain slot,
  // 4096-column range) are wave-uniform and stepped without division.
  const long long n_items = (long long)ls.n_plain * p.nrB;
  const int i0 = (int)(n_items * blockIdx.x / gridDim.x), i1 = (int)(n_items * (blockIdx.x + 1) / gridDim.x);
  constexpr int PLAIN_DEPTH = 2, STRIDE = NT / 64;   // 2 measured as fast as 1, 3 and 4 slower
  const int nrB = p.nrB;
  auto advance = [nrB](int& sl, int& rg, int by) {
    rg += by;
    while (rg >= nrB) {
      rg -= nrB;
      sl++;
    }
  };
  int pit = i0 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  int psl = pit / nrB, prg = pit - (pit / nrB) * nrB;
  PlainRaw<SPEC_BF16> pb;
  if (pit < i1) plain_load<SPEC_BF16, true>(p, s, plain_list[psl], prg, pb);
  auto between = [&]() {
    if (pit < i1) {
      plain_finish<SPEC_BF16, NOISE, true>(p, s, plain_list[psl], psl, prg, pb);
      pit += STRIDE;
      advance(psl, prg, STRIDE);
      if (pit < i1) plain_load<SPEC_BF16, true>(p, s, plain_list[psl], prg, pb);
    }
  };
  if (ls.n_draft + ls.n_correct > 0) bias_sweep_fast<NOISE>(p, s, ls, bias_list, req, sA, G, between);
  PlainRaw<SPEC_BF16> R[PLAIN_DEPTH];
  int slot[PLAIN_DEPTH], rng[PLAIN_DEPTH];
  R[0] = pb;
  slot[0] = psl;
  rng[0] = prg;
  {
    int sl = psl, rg = prg;
#pragma unroll
    for (int d = 1; d < PLAIN_DEPTH; d++) {
      advance(sl, rg, STRIDE);
      slot[d] = sl;
      rng[d] = rg;
      if (pit + STRIDE * d < i1) plain_load<SPEC_BF16, true>(p, s, plain_list[sl], rg, R[d]);
    }
  }
  for (int it0 = pit; it0 < i1; it0 += STRIDE * PLAIN_DEPTH) {
#pragma unroll
    for (int d = 0; d < PLAIN_DEPTH; d++) {
      const int it = it0 + STRIDE * d;
      if (it < i1) {
        plain_finish<SPEC_BF16, NOISE, true>(p, s, plain_list[slot[d]], slot[d], rng[d], R[d]);
        advance(slot[d], rng[d], STRIDE * PLAIN_DEPTH);
        if (it + STRIDE * PLAIN_DEPTH < i1) plain_load<SPEC_BF16, true>(p, s, plain_list[slot[d]], rng[d], R[d]);
      }
    }
  }
}

template <int DT, int NOISE, bool VEC>
__global__ __launch_bounds__(NT, 1) void k_bias(Params p, int s) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_bias[];
  __shared__ uint64_t scan_tmp[NT / 64];
  __shared__ GenericLds lds_g;
  if (p.live[s] == 0) return;
  ReqMeta* req = (ReqMeta*)dyn_bias;
  uint16_t* bias_list = (uint16_t*)(dyn_bias + (size_t)p.B * sizeof(ReqMeta));
  uint16_t* plain_list = bias_list + bias_slots_max(p.B);
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;
  const Lists ls = build_lists<NOISE, NT>(p, s, roles, bias_list, plain_list, scan_tmp, req, true);
  if (ls.n_draft + ls.n_correct == 0) return;
  bias_sweep_generic<DT, NOISE, VEC>(p, s, ls, bias_list, req, lds_g);
}

template <int DT, int NOISE, bool VEC>
__global__ __launch_bounds__(NT, 6) void k_plain(Params p, int s) {
  extern __shared__ uint16_t dyn_lists[];
  __shared__ uint64_t scan_tmp[NT / 64];
  if (p.live[s] == 0) return;
  uint16_t* bias_list = dyn_lists;
  uint16_t* plain_list = dyn_lists + bias_slots_max(p.B);
  const uint8_t* roles = p.roles + (size_t)(s & 1) * p.B;
  const Lists ls = build_lists<NOISE, NT>(p, s, roles, bias_list, plain_list, scan_tmp, nullptr, false);
  const int n_items = ls.n_plain * p.nrB;
  const int nw = gridDim.x * (NT / 64);
  for (int it = blockIdx.x * (NT / 64) + (threadIdx.x >> 6); it < n_items; it += nw) {
    const int pslot = it / p.nrB, range = it % p.nrB;
    plain_item<DT, NOISE, VEC>(p, s, plain_list[pslot], pslot, range);
  }
}

// ------------------------------------------------------------------------------------------
// merge: one workgroup per request, three dependent memory rounds
//   1. the partials of every row the request has this step, all loaded together and reduced;
//   2. level two of the chunked sampler for the DRAFT row (threads 0..127) and for the CORRECT /
//      BONUS row (threads 128..255) side by side: 64 columns x 2 threads each, every thread half
//      of the Markov-bias dot product; the DRAFT half also reads the target values of its chunk,
//      so the accept test needs no further load;
//   3. decision, outputs and the roles of step s + 1.
// ------------------------------------------------------------------------------------------

// Running reduction of partial records {log-mass, best score, best index, aux}: the log-mass is
// kept as m + log(s) (one exponential per record instead of a full log-sum-exp), a NaN anywhere
// is remembered in `nan`; the winner follows `better`.
struct PartAcc {
  float m, s, sc, aux;
  int ix, nan;
};

__device__ __forceinline__ void pacc_init(PartAcc& a) {
  a.m = -INFINITY;
  a.s = 0.0f;
  a.sc = -INFINITY;
  a.aux = 0.0f;
  a.ix = -1;
  a.nan = 0;
}

__device__ __forceinline__ void pacc_mass(PartAcc& a, float m, float s, int nan) {
  a.nan |= nan;
  if (m > a.m) {
    a.s = s + a.s * ex2((a.m - m) * LOG2E);   // a.m = -inf: the old sum is 0
    a.m = m;
  } else if (m > -INFINITY) {
    a.s += s * ex2((m - a.m) * LOG2E);
  }
}

__device__ __forceinline__ void pacc_best(PartAcc& a, float sc, int ix, float aux) {
  if (ix >= 0 && (a.ix < 0 || better(sc, ix, a.sc, a.ix))) {
    a.sc = sc;
    a.ix = ix;
    a.aux = aux;
  }
}


__device__ __forceinline__ float4 pacc_final(const PartAcc& a) {
  const float lse = a.nan ? NAN : (a.m == -INFINITY ? -INFINITY : a.m + lg2(a.s) * LN2);
  return make_float4(lse, a.sc, __int_as_float(a.ix), a.aux);
}

// running record of every lane of a wave merged into every lane.  The mass as one wave maximum, each
// lane's sum rescaled to it (a lane at the maximum adds its sum as it is, a lane at -inf adds
// nothing) and one wave sum; the NaN flag by ballot; the winner by the DPP argmax (the same take
// rule as pacc_best).
__device__ __forceinline__ void wave_reduce_acc(PartAcc& a) {
  const float M = wave_max64(a.m);
  const float sl = (a.m == M) ? a.s : ((a.m == -INFINITY) ? 0.0f : a.s * ex2((a.m - M) * LOG2E));
  a.s = wave_sum64(sl);
  a.m = M;
  a.nan = __ballot(a.nan != 0) != 0ull;
  wave_argmax64(a.sc, a.ix, a.aux);
}

// records per row and thread in one round of the merge's partial reduction
constexpr int MERGE_BATCH = 10;

// records i0 + NT k + thread (k < MERGE_BATCH) of a row's n partials, empty past n; 8-byte
// records {log-mass, score} take their index from their place
__device__ __forceinline__ void load_parts(const char* parts, int rec8, int n, int i0, float4 (&b)[MERGE_BATCH]) {
#pragma unroll
  for (int k = 0; k < MERGE_BATCH; k++) {
    const int i = i0 + NT * k + (int)threadIdx.x;
    if (rec8) {
      const float2 r = (i < n) ? ((const float2*)parts)[i] : make_float2(-INFINITY, -INFINITY);
      b[k] = make_float4(r.x, r.y, __int_as_float(i < n ? i : -1), 0.0f);
    } else {
      b[k] = (i < n) ? ((const float4*)parts)[i] : empty_part();
    }
  }
}

// a batch of records into a running record: the batch's maximum first, then one scaled sum of
// exponentials, merged once; the winner by branch-free selects (smaller index on equal scores)
__device__ __forceinline__ void add_parts(PartAcc& a, const float4 (&b)[MERGE_BATCH]) {
  float mx = -INFINITY;
  int nan = 0;
#pragma unroll
  for (int k = 0; k < MERGE_BATCH; k++) {
    nan |= (b[k].x != b[k].x);
    mx = fmaxf(mx, b[k].x);
  }
  float sum = 0.0f;
  const float mo = (mx == -INFINITY) ? 0.0f : mx * LOG2E;
#pragma unroll
  for (int k = 0; k < MERGE_BATCH; k++) sum += ex2(fmaf(b[k].x, LOG2E, -mo));   // -inf: 0; NaN: flagged
  pacc_mass(a, mx, nan ? 0.0f : sum, nan);
#pragma unroll
  for (int k = 0; k < MERGE_BATCH; k++) {
    const int ix = __float_as_int(b[k].z);
    const bool take = (ix >= 0) & ((a.ix < 0) | (b[k].y > a.sc) | ((b[k].y == a.sc) & ((unsigned)ix < (unsigned)a.ix)));
    a.sc = take ? b[k].y : a.sc;
    a.aux = take ? b[k].w : a.aux;
    a.ix = take ? ix : a.ix;
  }
}

// half of the Markov-bias dot product A[prev] . W[v] (k in [hh R/2, (hh + 1) R/2)), fp32 accumulate
template <int DT>
__device__ __forceinline__ float bias_half(const Params& p, int prev, int v, int hh) {
  float a = 0.0f;
  const int R = p.R, k0 = hh * (R >> 1), k1 = k0 + (R >> 1);
  if (prev < 0 || v < 0 || v >= p.V) return a;
  if (DT == SPEC_BF16) {
    const uint16_t* ar = (const uint16_t*)p.A + (size_t)prev * R;
    const uint16_t* wr = (const uint16_t*)p.W + (size_t)v * R;
    if ((R & 15) == 0) {
      // fully unrolled to the largest rank, so every load is in flight before the first FMA
      u32x4 aw[MAX_R / 16], ww[MAX_R / 16];
#pragma unroll
      for (int i = 0; i < MAX_R / 16; i++) {
        const int k = k0 + 8 * i;
        aw[i] = (k < k1) ? *(const u32x4*)(ar + k) : (u32x4){0, 0, 0, 0};
        ww[i] = (k < k1) ? *(const u32x4*)(wr + k) : (u32x4){0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < MAX_R / 16; i++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          a = fmaf(bf16_lo(aw[i][q]), bf16_lo(ww[i][q]), a);
          a = fmaf(bf16_hi(aw[i][q]), bf16_hi(ww[i][q]), a);
        }
      }
    } else {
      for (int k = k0; k < k1; k++) a = fmaf(bf16_to_f32(ar[k]), bf16_to_f32(wr[k]), a);
    }
  } else {
    const float* ar = (const float*)p.A + (size_t)prev * R;
    const float* wr = (const float*)p.W + (size_t)v * R;
    for (int k = k0; k < k1; k++) a = fmaf(ar[k], wr[k], a);
  }
  return a;
}

enum { L2_NONE = 0, L2_DRAFT = 1, L2_TARGET = 2, L2_RESIDUAL = 3 };

struct L2Job {       // one level-two selection of a thread group
  int kind;          // L2_*
  int chunk;         // chunk of the winner of level one
  int prev;          // previous token (Markov bias), -1 = none
  uint64_t key;      // per-index noise key of the row
  const void* base_row;
  const void* targ_row;
  float invT, lse_p, lse_q;
  bool want_target;  // DRAFT: also return the target logit of the winner
};

struct L2Result {
  int v;             // winning column, -1 = none
  float sx;          // DRAFT: scaled draft logit of the winner
  float tx;          // target logit (unscaled) of the winner, when asked for
};

// Level two over the 64 columns of one chunk by a group of 128 threads (2 waves); thread t of the
// group takes column 64 c + t / 2 and half t % 2 of the rank.  Result in every thread of the group.
template <int DT>
__device__ L2Result level_two(const Params& p, const L2Job& jb, int gt, float4* lds2) {
  const int hh = gt & 1;
  const int v = jb.chunk * CHUNK + (gt >> 1);
  const bool in = jb.kind != L2_NONE && jb.chunk >= 0 && v < p.V;
  // the row values first (independent of the bias), then the bias dot product
  const bool need_base = in && (jb.kind == L2_DRAFT || jb.kind == L2_RESIDUAL);
  const bool need_targ = in && (jb.kind != L2_DRAFT || jb.want_target);
  const float bv = need_base ? load1<DT>(jb.base_row, (size_t)v) : 0.0f;
  const float tvr = need_targ ? load1<DT>(jb.targ_row, (size_t)v) : 0.0f;
  float bias = 0.0f;
  if (in && jb.kind != L2_TARGET) bias = bias_half<DT>(p, jb.prev, v, hh);
  bias += dpp<0xB1>(bias);   // the partner lane (xor 1) holds the other half
  float sc = -INFINITY, sx = 0.0f, tx = 0.0f;
  int ix = -1;
  if (in && hh == 0) {
    const float g = gumbel_bits(bits_at(jb.key, (uint32_t)v));
    if (jb.kind == L2_DRAFT) {
      const float sv = (bv + bias) * jb.invT;
      if (jb.want_target) tx = tvr;
      if (sv > -INFINITY) {
        sc = sv + g;
        ix = v;
        sx = sv;
      }
    } else if (jb.kind == L2_TARGET) {
      const float tv = tvr * jb.invT;
      if (tv > -INFINITY) {
        sc = tv + g;
        ix = v;
      }
    } else {
      const float sv = (bv + bias) * jb.invT;
      const float tv = tvr * jb.invT;
      const float lp = tv - jb.lse_p, lq = sv - jb.lse_q;
      if (lp > lq) {
        sc = lp + logf(-expm1f(lq - lp)) + g;
        ix = v;
      }
    }
  }
  // argmax over the wave by DPP (larger score, smallest index on ties), sx riding along; tx is read
  // from the winner's lane, the only one holding that column
  const int ix0 = ix;
  const float tx0 = tx;
  wave_argmax64(sc, ix, sx);
  {
    const unsigned long long wm = __ballot(ix >= 0 && ix0 == ix);
    tx = __shfl(tx0, wm ? __ffsll(wm) - 1 : 0, 64);
  }
  const int wv = (gt >> 6) & 1;
  if ((gt & 63) == 0) lds2[wv] = make_float4(sc, sx, __int_as_float(ix), tx);
  __syncthreads();
  L2Result r;
  float4 a = lds2[0], c = lds2[1];
  const int ia = __float_as_int(a.z), ic = __float_as_int(c.z);
  if (ic >= 0 && (ia < 0 || better(c.x, ic, a.x, ia))) a = c;
  r.v = __float_as_int(a.z);
  r.sx = a.y;
  r.tx = a.w;
  return r;
}

template <int DT, int NOISE>
__global__ __launch_bounds__(NT) void k_merge(Params p, int s) {
  __shared__ float4 red[4][NT / 64];
  __shared__ PartAcc racc[4][NT / 64];
  __shared__ float4 lds2[2][2];
  const int b = blockIdx.x;
  const int B = p.B, K = p.K, V = p.V;
  if (p.live[s] == 0) return;
  // round 0: every per-request value that depends only on (b, s), loaded together with the roles
  const int roles = p.roles[(size_t)(s & 1) * B + b];
  const float invT = 1.0f / p.temp[b];
  const int x0 = p.x0 ? p.x0[b] : -1;
  const int L = p.L[b];
  int phase = p.phase[b];
  int acc = p.acc[b];
  const uint64_t kreq = p.kreq[b];
  const int slot_d = p.slots[b], slot_c = p.slots[B + b], slot_p = p.slots[2 * B + b];
  const int32_t* xr = p.xs + (size_t)b * K;
  const int prev_d = (s == 0) ? x0 : xr[s - 1];                // token before position s
  const int prev_c = (s <= 1) ? x0 : xr[s - 2];                // token before position s - 1
  const int x_t = (threadIdx.x < K) ? xr[threadIdx.x] : -1;   // drafted tokens, for the output
  const int jc0 = s > 0 ? s - 1 : 0;
  const float lse_p_c = p.lse_p[(size_t)b * (K + 1) + jc0];    // read whether or not used
  const float lse_q_c = p.lse_q[(size_t)b * K + jc0];
  uint8_t* roles_next = p.roles + (size_t)((s + 1) & 1) * B;
  if (roles == 0) {
    if (threadIdx.x == 0) roles_next[b] = 0;
    return;
  }
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const bool hasD = roles & RO_DRAFT, hasC = roles & RO_CORRECT, hasP = roles & (RO_LSEP | RO_BONUS);

  // ---- round 1: partials of every row (DRAFT, CORRECT, its fallback, plain), each row's records
  // split over the whole workgroup: every thread keeps one running record per row and issues its
  // loads of all rows together (MERGE_BATCH per row and round), then the wave and the workgroup
  // reduce them
  {
    const int esz = p.part8 ? 8 : 16;
    const char* pd = (const char*)p.part_bias + (size_t)(hasD ? slot_d : 0) * p.nrA * esz;
    const char* pc = (const char*)p.part_bias + (size_t)(hasC ? slot_c : 0) * p.nrA * esz;
    const char* pc2 = (const char*)p.part_bias2 + (size_t)(hasC ? slot_c : 0) * p.nrA * esz;
    const char* pp = (const char*)(p.part_plain + (size_t)(hasP ? slot_p : 0) * p.nrB);
    const int nD = hasD ? p.nrA : 0, nC = hasC ? p.nrA : 0, nP = hasP ? p.nrB : 0;
    const int nmax = max(max(nD, nC), nP);
    PartAcc ad, ac, ac2, ap;
    pacc_init(ad);
    pacc_init(ac);
    pacc_init(ac2);
    pacc_init(ap);
    // the row kinds are uniform over the workgroup: absent rows cost neither loads nor arithmetic
    for (int i0 = 0; i0 < nmax; i0 += MERGE_BATCH * NT) {
      float4 bd[MERGE_BATCH], bc[MERGE_BATCH], bc2[MERGE_BATCH], bp[MERGE_BATCH];
      if (hasD) load_parts(pd, p.part8, nD, i0, bd);
      if (hasC) {
        load_parts(pc, p.part8, nC, i0, bc);
        load_parts(pc2, p.part8, nC, i0, bc2);
      }
      if (hasP) load_parts(pp, 0, nP, i0, bp);
      if (hasD) add_parts(ad, bd);
      if (hasC) {
        add_parts(ac, bc);
        add_parts(ac2, bc2);
      }
      if (hasP) add_parts(ap, bp);
    }
    if (hasD) wave_reduce_acc(ad);
    if (hasC) {
      wave_reduce_acc(ac);
      wave_reduce_acc(ac2);
    }
    if (hasP) wave_reduce_acc(ap);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      racc[0][w] = ad;
      racc[1][w] = ac;
      racc[2][w] = ac2;
      racc[3][w] = ap;
    }
    __syncthreads();
    if (threadIdx.x < 4) {
      PartAcc a = racc[threadIdx.x][0];
#pragma unroll
      for (int v = 1; v < NT / 64; v++) {
        const PartAcc& o = racc[threadIdx.x][v];
        pacc_mass(a, o.m, o.s, o.nan);
        pacc_best(a, o.sc, o.ix, o.aux);
      }
      red[0][threadIdx.x] = pacc_final(a);
    }
  }
  __syncthreads();
  const float4 tot_d = red[0][0], tot_c = red[0][1], tot_c2 = red[0][2], tot_p = red[0][3];

  // ---- round 2: level two (CHUNKED) or the single target value the accept test needs (FLAT)
  const int j_c = s - 1;   // a CORRECT row is the position rejected at step s - 1
  const bool residual = tot_c.x > -INFINITY;
  L2Result rd = {-1, 0.0f, 0.0f}, rf = {-1, 0.0f, 0.0f};
  const void* targ_s = (const char*)p.target + ((size_t)b * (K + 1) + s) * V * esz;
  if (NOISE == SPEC_NOISE_CHUNKED) {
    const int g = threadIdx.x >> 7, gt = threadIdx.x & 127;
    L2Job jb;
    jb.kind = L2_NONE;
    jb.chunk = -1;
    jb.prev = -1;
    jb.key = 0;
    jb.base_row = nullptr;
    jb.targ_row = nullptr;
    jb.invT = invT;
    jb.lse_p = 0.0f;
    jb.lse_q = 0.0f;
    jb.want_target = false;
    if (g == 0) {
      if (hasD && isfinite(tot_d.x)) {
        jb.kind = L2_DRAFT;
        jb.chunk = __float_as_int(tot_d.z);
        jb.prev = prev_d;
        jb.key = key_from(kreq, s, ST_DRAFT);
        jb.base_row = (const char*)p.base + ((size_t)b * K + s) * V * esz;
        jb.targ_row = targ_s;
        jb.want_target = (roles & RO_LSEP) != 0;
      }
    } else if (hasC) {
      jb.chunk = __float_as_int(residual ? tot_c.z : tot_c2.z);
      jb.key = key_from(kreq, j_c, ST_RESIDUAL);
      jb.targ_row = (const char*)p.target + ((size_t)b * (K + 1) + j_c) * V * esz;
      if (residual) {
        jb.kind = L2_RESIDUAL;
        jb.prev = prev_c;
        jb.base_row = (const char*)p.base + ((size_t)b * K + j_c) * V * esz;
        jb.lse_p = lse_p_c;
        jb.lse_q = lse_q_c;
      } else {
        jb.kind = L2_TARGET;
      }
    } else if ((roles & RO_BONUS) && isfinite(tot_p.x)) {
      jb.kind = L2_TARGET;
      jb.chunk = __float_as_int(tot_p.z);
      jb.key = key_from(kreq, s, ST_BONUS);
      jb.targ_row = targ_s;
    }
    const L2Result r = level_two<DT>(p, jb, gt, lds2[g]);
    // results of the other group through LDS
    __shared__ L2Result res[2];
    if (gt == 0) res[g] = r;
    __syncthreads();
    rd = res[0];
    rf = res[1];
  } else {
    rd.v = hasD ? __float_as_int(tot_d.z) : -1;
    rd.sx = tot_d.w;
    if ((roles & RO_LSEP) && rd.v >= 0 && rd.v < V) rd.tx = load1<DT>(targ_s, (size_t)rd.v);
    rf.v = hasC ? __float_as_int(residual ? tot_c.z : tot_c2.z) : ((roles & RO_BONUS) ? __float_as_int(tot_p.z) : -1);
  }

  // ---- round 3: decision and outputs (uniform across the workgroup; thread 0 writes scalars)
  bool invalid = false, rejected_now = false;
  int final_tok = -1;
  float logq_s = NAN;
  int x_s = -1;
  if (hasD) {
    const float lse_q = tot_d.x;
    if (!isfinite(lse_q) || rd.v < 0) {
      invalid = true;
    } else {
      x_s = rd.v;
      logq_s = rd.sx - lse_q;
      if (threadIdx.x == 0) {
        p.xs[(size_t)b * K + s] = x_s;
        p.lse_q[(size_t)b * K + s] = lse_q;
        p.logq[(size_t)b * K + s] = logq_s;
        if (p.d_draft) p.d_draft[(size_t)b * K + s] = x_s;
        if (p.d_logq) p.d_logq[(size_t)b * K + s] = logq_s;
      }
    }
  }
  if (!invalid && (roles & RO_LSEP)) {
    const float lse_p = tot_p.x;
    if (!isfinite(lse_p) || x_s < 0) {
      invalid = true;
    } else {
      const float logp_s = rd.tx * invT - lse_p;
      // accept when u = (ub + 1/2) 2^-32 < p / q = exp(logp - logq): the ratio in fp32 (its relative
      // error, about 1e-7, is below that of the fp32 log-probabilities it comes from), compared
      // exactly with u in fp64 as (ub + 1/2) < ratio 2^32
      const uint32_t ub = bits_at(key_from(kreq, s, ST_ACCEPT), 0);
      const float ratio32 = __builtin_amdgcn_ldexpf(ex2((logp_s - logq_s) * LOG2E), 32);
      if ((double)ub + 0.5 < (double)ratio32) {
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
    if (!isfinite(tot_p.x)) invalid = true;
    else final_tok = rf.v;
    if (final_tok < 0) invalid = true;
  }
  if (!invalid && hasC) {
    final_tok = rf.v;
    if (final_tok < 0) invalid = true;
  }

  const int t = threadIdx.x;
  if (invalid) {
    if (t <= K) p.tokens[(size_t)b * (K + 1) + t] = -1;
    if (t < K) {
      if (p.d_draft) p.d_draft[(size_t)b * K + t] = -1;
      if (p.d_logq) p.d_logq[(size_t)b * K + t] = NAN;
      if (p.d_logp) p.d_logp[(size_t)b * K + t] = NAN;
    }
    if (t == 0) {
      p.accepted_len[b] = -1;
      if (p.d_verify_len) p.d_verify_len[b] = -1;
      p.phase[b] = PH_INVALID;
      p.acc[b] = acc;
      roles_next[b] = 0;
    }
    return;
  }
  if (final_tok >= 0) {
    phase = PH_DONE;
    if (t < acc) p.tokens[(size_t)b * (K + 1) + t] = x_t;   // t < acc <= s: drafted before this step
    if (t == acc) p.tokens[(size_t)b * (K + 1) + t] = final_tok;
    if (t == 0) p.accepted_len[b] = acc;
  }
  if (t == 0) {
    int nr = 0;
    if (s + 1 < L) nr |= RO_DRAFT;
    if (phase == PH_ALIVE && acc == s + 1) nr |= (s + 1 < L) ? RO_LSEP : RO_BONUS;
    if (rejected_now) nr |= RO_CORRECT;
    p.phase[b] = phase;
    p.acc[b] = acc;
    roles_next[b] = (uint8_t)nr;
    if (nr) p.live[s + 1] = 1;
  }
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
// ==========================================================================================
// Acceptance statistics: alpha_{b,j} = sum_v min(p_j(v), q_j(v)) = 1 - TV(p_j, q_j), the
// analytical acceptance rate of every drafted position ("The Speed Claim Nobody's Really
// Questioning", sections "The Semi-Autoregressive Trick" and "The Real Innovation:
// Confidence-Scheduled Verification"), and the calibration error of the confidences' prefix
// product ("DSpark turns speculation into a scheduler", section "Confidence is a serving
// primitive").
//   k_stats_prep       one workgroup: compact list of the drafted positions, their previous
//                      token, NaN-filled outputs
//   k_stats_sweep<1>   the (draft, target) row pairs in units of 32 rows x 256 columns with the
//                      Markov bias on MFMA (bf16) or VALU dot products (fp32): per-range
//                      log-normalisers of q and p
//   k_stats_merge<1>   one wave per row: LSE_q, LSE_p
//   k_stats_sweep<2>   same sweep: per-range sum of min(p, q) = exp2 of the smaller log2-probability
//   k_stats_merge<2>   one wave per row: alpha
// ==========================================================================================
struct StatsParams {
  Params c;                // dims, logits, factors, konst: what the shared sweep helpers read
  const int32_t* draft;    // [B, K] drafted tokens, -1 past the drafted prefix
  float* alpha;            // [B, K] out
  float* o_lse_q;          // [B, K] out, may be null
  float* o_lse_p;          // [B, K] out, may be null
  int32_t* n_rows;         // [1] number of listed rows
  int32_t* rows;           // [B K] listed row ids b K + j
  int32_t* prev;           // [B K] previous token of each listed row (-1: none)
  float* lse_q;            // [B K] per listed row
  float* lse_p;            // [B K]
  float2* part;            // [slots][nrA] per-range partials
};

// drafted position j of request b needs a valid temperature and x0, and a drafted token at j - 1.
// Thread t takes requests t per .. t per + per - 1 (per <= MAX_B / NT), every load of a request
// issued before any is used; the listed rows keep the order b K + j.
__global__ __launch_bounds__(NT) void k_stats_prep(StatsParams sp) {
  const Params& p = sp.c;
  if (threadIdx.x < 2) {
    const uint32_t w = threadIdx.x ? 0xFF80FF80u : 0u;
    ((u32x4*)p.konst)[threadIdx.x] = (u32x4){w, w, w, w};
  }
  const int B = p.B, K = p.K;
  const int per = (B + NT - 1) / NT, b0 = threadIdx.x * per;
  constexpr int MAXPER = (MAX_B + NT - 1) / NT;
  uint32_t okm[MAXPER];
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < MAXPER; r++) {
    okm[r] = 0u;
    const int b = b0 + r;
    if (r >= per || b >= B) continue;
    const float T = p.temp[b];
    const int x0 = p.x0 ? p.x0[b] : -1;
    const bool valid = (T > 0.0f) && isfinite(T) && x0 >= -1 && x0 < p.V;
    int d[MAX_K];
#pragma unroll
    for (int j = 0; j < MAX_K; j++) d[j] = j < K ? sp.draft[(size_t)b * K + j] : -1;
#pragma unroll
    for (int j = 0; j < MAX_K; j++) {
      if (j >= K) break;
      const bool ok = valid && d[j] >= 0 && (j == 0 || (d[j - 1] >= 0 && d[j - 1] < p.V));
      okm[r] |= ok ? (1u << j) : 0u;
      const size_t i = (size_t)b * K + j;
      sp.alpha[i] = NAN;
      if (sp.o_lse_q) sp.o_lse_q[i] = NAN;
      if (sp.o_lse_p) sp.o_lse_p[i] = NAN;
    }
    cnt += __popc(okm[r]);
  }
  // exclusive scan of the per-thread counts: within each wave by shuffles, then over the waves
  __shared__ int wsum_s[NT / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    inc += lane >= o ? y : 0;
  }
  if (lane == 63) wsum_s[wv] = inc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; w++) {
    base += w < wv ? wsum_s[w] : 0;
    total += wsum_s[w];
  }
  if (threadIdx.x == 0) sp.n_rows[0] = total;
  int k = base + inc - cnt;
  // the listed rows of the thread's requests in order, previous tokens from the request's drafted
  // tokens (loaded again, all at once)
#pragma unroll
  for (int r = 0; r < MAXPER; r++) {
    const int b = b0 + r;
    uint32_t m = okm[r];
    if (m == 0u) continue;
    int d[MAX_K];
#pragma unroll
    for (int j = 0; j < MAX_K; j++) d[j] = j < K ? sp.draft[(size_t)b * K + j] : -1;
    const int x0 = p.x0 ? p.x0[b] : -1;
#pragma unroll
    for (int j = 0; j < MAX_K; j++) {
      if ((m >> j) & 1u) {
        sp.rows[k] = b * K + j;
        sp.prev[k] = j == 0 ? x0 : d[j - 1];
        k++;
      }
    }
  }
}

struct StatsLds {
  uint16_t sA[SUB][MAX_R + A_PAD];   // A rows of the current unit (bf16)
  float2 red[NT / 64][SUB];          // per-wave chunk results of the current unit
};

// per-range partials of one finished unit (threads 0..31): merge the four waves' chunk results
template <int PASS>
__device__ __forceinline__ void stats_flush(const StatsParams& sp, const float2 (*red)[SUB], int slot0, int range,
                                            int n_rows) {
  if (threadIdx.x < SUB && slot0 + (int)threadIdx.x < n_rows) {
    const int r = threadIdx.x;
    float2 a = red[0][r];
#pragma unroll
    for (int w = 1; w < NT / 64; w++) {
      const float2 o = red[w][r];
      if (PASS == 1) {
        a.x = lse2(a.x, o.x);
        a.y = lse2(a.y, o.y);
      } else {
        a.x += o.x;
      }
    }
    sp.part[(size_t)(slot0 + r) * sp.c.nrA + range] = a;
  }
}

template <int DT, int PASS, bool VEC>
__global__ __launch_bounds__(NT, 1) void k_stats_sweep(StatsParams sp) {
  __shared__ StatsLds L;
  const Params& p = sp.c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, h = lane >> 5;
  const int V = p.V, R = p.R, K = p.K;
  const size_t esz = (DT == SPEC_FP32) ? 4 : 2;
  const int n_rows = sp.n_rows[0];
  const int nsb = (n_rows + SUB - 1) / SUB;
  const long long units = (long long)p.nrA * nsb;
  const int u0 = (int)(units * blockIdx.x / gridDim.x);
  const int u1 = (int)(units * (blockIdx.x + 1) / gridDim.x);
  if (u0 >= u1) return;
  if (DT == SPEC_BF16 && R < MAX_R) {
    // the MFMA loop runs over the full rank: A columns past R read as zero
    uint32_t* z = (uint32_t*)&L.sA[0][0];
    for (int i = threadIdx.x; i < (int)(sizeof(L.sA) / 4); i += NT) z[i] = 0u;
  }
  bf16x8 wf[2][16];
  int w_range = -1;
  for (int u = u0; u < u1; u++) {
    const int range = u / nsb, slot0 = (u % nsb) * SUB;
    __syncthreads();   // the previous unit is done with sA and red
    if (u > u0) stats_flush<PASS>(sp, L.red, ((u - 1) % nsb) * SUB, (u - 1) / nsb, n_rows);
    if (DT == SPEC_BF16) {
      const int segs = R >> 3;
      for (int e = threadIdx.x; e < SUB * segs; e += NT) {
        const int row = e / segs, sg = e - row * segs;
        const int slot = slot0 + row;
        const int pv = slot < n_rows ? sp.prev[slot] : -1;
        u32x4 val = {0, 0, 0, 0};
        if (pv >= 0) val = *(const u32x4*)((const uint16_t*)p.A + (size_t)pv * R + 8 * sg);
        *(u32x4*)&L.sA[row][8 * sg] = val;
      }
    }
    __syncthreads();   // sA holds this unit's A rows; red is free
    if (DT == SPEC_BF16 && range != w_range) load_w(p, range, wf);
    w_range = range;

    const int vw = range * TILE_A + 64 * wave;   // this wave's 64 columns
    const int v0 = vw + 16 * h;
    const int slot = slot0 + m;
    const bool active = slot < n_rows;
    const int rid = active ? sp.rows[slot] : 0;
    const int b = rid / K, j = rid - b * K;
    const int pv = active ? sp.prev[slot] : -1;
    const float invT = active ? 1.0f / p.temp[b] : 1.0f;
    float y[32], t[32];
    if (DT == SPEC_BF16) {
      mfma_bias(wf, L.sA, R, y);
    } else {
      fp32_bias16(p, pv, v0, y);
      fp32_bias16(p, pv, v0 + 32, y + 16);
    }
    {
      float bx[32];
#pragma unroll
      for (int i = 0; i < 32; i++) bx[i] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 32; i++) t[i] = -INFINITY;
      const void* base_row = (const char*)p.base + ((size_t)b * K + j) * (size_t)V * esz;
      const void* targ_row = (const char*)p.target + ((size_t)b * (K + 1) + j) * (size_t)V * esz;
      if (active) {
        load16<DT, VEC>(base_row, v0, V, *(float(*)[16])bx);
        load16<DT, VEC>(base_row, v0 + 32, V, *(float(*)[16])(bx + 16));
        load16<DT, VEC>(targ_row, v0, V, *(float(*)[16])t);
        load16<DT, VEC>(targ_row, v0 + 32, V, *(float(*)[16])(t + 16));
      }
#pragma unroll
      for (int i = 0; i < 32; i++) y[i] = active ? bx[i] + y[i] : -INFINITY;
    }
    float2 o;
    if (PASS == 1) {
      o.x = pair_lse_scaled<32>(y, invT);
      o.y = pair_lse_scaled<32>(t, invT);
    } else {
      // sum of min(p, q) over the lane pair's 64 columns: exp2 of the smaller base-2 log-probability
      const float c = invT * LOG2E;
      const float oq = active ? -sp.lse_q[slot] * LOG2E : 0.0f, op = active ? -sp.lse_p[slot] * LOG2E : 0.0f;
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        a0 += ex2(fminf(fmaf(t[i], c, op), fmaf(y[i], c, oq)));
        a1 += ex2(fminf(fmaf(t[i + 1], c, op), fmaf(y[i + 1], c, oq)));
      }
      o.x = a0 + a1;
      o.x += xor32f(o.x);
      o.y = 0.0f;
    }
    if (h == 0) L.red[wave][m] = o;
  }
  __syncthreads();
  stats_flush<PASS>(sp, L.red, ((u1 - 1) % nsb) * SUB, (u1 - 1) / nsb, n_rows);
}

// one wave per listed row: reduce the row's per-range partials
template <int PASS>
__global__ __launch_bounds__(NT) void k_stats_merge(StatsParams sp) {
  const int n_rows = sp.n_rows[0];
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * (NT / 64);
  const int nrA = sp.c.nrA;
  for (int slot = blockIdx.x * (NT / 64) + (threadIdx.x >> 6); slot < n_rows; slot += nw) {
    const float2* pr = sp.part + (size_t)slot * nrA;
    if (PASS == 1) {
      // running {max, scaled sum} of both log-normalisers; a NaN anywhere stays visible
      float mq = -INFINITY, sq = 0.0f, mp = -INFINITY, s_p = 0.0f;
      for (int r = lane; r < nrA; r += 64) {
        const float2 v = pr[r];
        if (v.x > mq) { sq = sq * ex2((mq - v.x) * LOG2E) + 1.0f; mq = v.x; }
        else if (v.x > -INFINITY) sq += ex2((v.x - mq) * LOG2E);
        else if (isnan(v.x)) sq = NAN;
        if (v.y > mp) { s_p = s_p * ex2((mp - v.y) * LOG2E) + 1.0f; mp = v.y; }
        else if (v.y > -INFINITY) s_p += ex2((v.y - mp) * LOG2E);
        else if (isnan(v.y)) s_p = NAN;
      }
      float lq = mq > -INFINITY ? mq + lg2(sq) * LN2 : (isnan(sq) ? NAN : -INFINITY);
      float lp = mp > -INFINITY ? mp + lg2(s_p) * LN2 : (isnan(s_p) ? NAN : -INFINITY);
      for (int o = 32; o > 0; o >>= 1) {
        lq = lse2(lq, __shfl_xor(lq, o, 64));
        lp = lse2(lp, __shfl_xor(lp, o, 64));
      }
      if (lane == 0) {
        sp.lse_q[slot] = lq;
        sp.lse_p[slot] = lp;
        const int rid = sp.rows[slot];
        if (sp.o_lse_q) sp.o_lse_q[rid] = lq;
        if (sp.o_lse_p) sp.o_lse_p[rid] = lp;
      }
    } else {
      float a = 0.0f;
      for (int r = lane; r < nrA; r += 64) a += pr[r].x;
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
      if (lane == 0) sp.alpha[sp.rows[slot]] = a;
    }
  }
}

// Order-independent fp64 bin sums.  A value x is split into two integer limbs on the grids 2^-24
// and 2^-64 (h = floor(x 2^24), l = floor(frac(x 2^24) 2^40): exact for |x| < 2^16 down to 2^-64,
// the bits below truncated), the limbs are added with 64-bit integer LDS atomics, and the sum is
// rebuilt once from them.  Integer addition is associative, so the result is the same whatever
// order the threads add in (bit-identical from run to run), and it differs from an exact sum by
// at most 2^-64 per term.  Up to 2^20 terms per bin fit the limbs.  A term that is not finite
// makes the bin's sum NaN.
struct FxBin {
  long long hi, lo;
  int bad;
};

__device__ __forceinline__ void fx_clear(FxBin& f) {
  f.hi = 0;
  f.lo = 0;
  f.bad = 0;
}

__device__ __forceinline__ void fx_add(FxBin& f, double x) {
  if (!isfinite(x)) {
    atomicAdd(&f.bad, 1);
    return;
  }
  const double y = x * 0x1p24;
  const double h = floor(y);
  const double l = floor((y - h) * 0x1p40);   // y - h in [0, 1) is exact
  atomicAdd((unsigned long long*)&f.hi, (unsigned long long)(long long)h);
  atomicAdd((unsigned long long*)&f.lo, (unsigned long long)(long long)l);
}

__device__ __forceinline__ double fx_value(const FxBin& f) {
  return f.bad ? (double)NAN : (double)f.hi * 0x1p-24 + (double)f.lo * 0x1p-64;
}

// Expected calibration error of the prefix product of the confidences against realised
// survival: one workgroup; every verified position j < L_b of a valid request is one pair
// (prediction: fp64 running product through j; outcome: j < a_b); nbins equal-width bins.
__global__ __launch_bounds__(NT) void k_calibration(const float* conf, const int32_t* verify_len,
                                                   const int32_t* accepted_len, int B, int K, int nbins,
                                                   double* ece, int64_t* n_pairs) {
  // per bin: the predictions' sum (order-independent limbs), survivals and pairs (integers)
  __shared__ FxBin sp_[MAX_BINS];
  __shared__ int sy_[MAX_BINS];
  __shared__ int cnt_[MAX_BINS];
  for (int m = threadIdx.x; m < nbins; m += NT) {
    fx_clear(sp_[m]);
    sy_[m] = 0;
    cnt_[m] = 0;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += NT) {
    const int a = accepted_len[b];
    if (a < 0) continue;
    const int L = min(verify_len[b], K);
    double P = 1.0;
    for (int j = 0; j < L; j++) {
      P *= (double)conf[(size_t)b * K + j];
      int m = (int)floor(P * nbins);
      m = m < 0 ? 0 : (m > nbins - 1 ? nbins - 1 : m);
      fx_add(sp_[m], P);
      if (j < a) atomicAdd(&sy_[m], 1);
      atomicAdd(&cnt_[m], 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long N = 0;
    for (int m = 0; m < nbins; m++) N += cnt_[m];
    double e = 0.0;
    for (int m = 0; m < nbins; m++)
      if (cnt_[m] > 0) e += ((double)cnt_[m] / (double)N) * fabs(fx_value(sp_[m]) / cnt_[m] - (double)sy_[m] / cnt_[m]);
    ece[0] = N > 0 ? e : 0.0;
    n_pairs[0] = N;
  }
}

// ==========================================================================================
// Hardware-aware prefix scheduler ("DSpark turns speculation into a scheduler", section
// "Confidence is a serving primitive": per-request prefix lengths from prefix survival and a
// profiled throughput curve, verification tokens with positive expected return under the batch
// pressure; "The Speed Claim Nobody's Really Questioning", section "The Real Innovation": verify
// more when the engine is idle, fewer when it is busy, early stopping keeps it lossless).
// One workgroup: every position's running minimum of prefix survival is binned on a threshold
// grid (counts and order-independent survival sums in LDS), suffix sums over the bins give the kept count n_g
// and expected emitted tokens E_g = B + S_g of every threshold g / nbins, goodput
// E_g / step_time[n_g] is maximised (ties to the larger g; g = nbins + 1 keeps nothing), and each
// request's verify length is the length of its prefix at the chosen threshold.
// ==========================================================================================
constexpr int SCHED_NT = 1024;   // >= MAX_B: one request per thread
constexpr int MAX_SCHED_BINS = 4096;

__device__ __forceinline__ int sched_bin(double M, int nbins) {
  const double f = floor(M * (double)nbins);
  if (!(f >= 0.0)) return 0;   // NaN or negative: the lowest bin
  return f > (double)nbins ? nbins : (int)f;
}

__global__ __launch_bounds__(SCHED_NT) void k_schedule(const float* conf, int B, int K, const double* step_time,
                                                     int nbins, int32_t* verify_len, double* out) {
  __shared__ int cnt[MAX_SCHED_BINS + 1];
  __shared__ FxBin ssum[MAX_SCHED_BINS + 1];   // survival sums, order-independent limbs
  __shared__ int tn[SCHED_NT];
  __shared__ double ts[SCHED_NT];
  __shared__ double bestG[SCHED_NT / 64];
  __shared__ int bestg[SCHED_NT / 64];
  __shared__ int bestn[SCHED_NT / 64];
  __shared__ double bestS[SCHED_NT / 64];
  __shared__ int g_star;
  const int tid = threadIdx.x;
  for (int i = tid; i <= nbins; i += SCHED_NT) {
    cnt[i] = 0;
    fx_clear(ssum[i]);
  }
  __syncthreads();
  // one request per thread (B <= 1024): its confidences loaded at once, its bins kept in registers
  const int b = tid;
  int mb[MAX_K];
  {
    float c[MAX_K];
#pragma unroll
    for (int j = 0; j < MAX_K; j++) c[j] = (b < B && j < K) ? conf[(size_t)b * K + j] : 1.0f;
    double P = 1.0, M = INFINITY;
#pragma unroll
    for (int j = 0; j < MAX_K; j++) {
      mb[j] = -1;
      if (b < B && j < K) {
        P *= (double)c[j];
        if (P < M || isnan(P)) M = P;
        mb[j] = sched_bin(M, nbins);
        atomicAdd(&cnt[mb[j]], 1);
        fx_add(ssum[mb[j]], P);
      }
    }
  }
  __syncthreads();
  // suffix sums over bins 1..nbins: thread t owns a contiguous chunk of bins
  const int nb = nbins + 1, chunk = (nb + SCHED_NT - 1) / SCHED_NT;
  const int lo = tid * chunk, hi = min(lo + chunk, nb);
  int cn = 0;
  double cs = 0.0;
  for (int k = lo; k < hi; k++) {
    cn += cnt[k];
    cs += fx_value(ssum[k]);
  }
  tn[tid] = cn;
  ts[tid] = cs;
  __syncthreads();
  // inclusive scan from the top (Hillis-Steele): tn[t] = sum over threads t' >= t
  for (int o = 1; o < SCHED_NT; o <<= 1) {
    const int an = tid + o < SCHED_NT ? tn[tid + o] : 0;
    const double as = tid + o < SCHED_NT ? ts[tid + o] : 0.0;
    __syncthreads();
    tn[tid] += an;
    ts[tid] += as;
    __syncthreads();
  }
  // candidates of this chunk, top down; the suffix above the chunk is the next thread's total
  int n = tid + 1 < SCHED_NT ? tn[tid + 1] : 0;
  double S = tid + 1 < SCHED_NT ? ts[tid + 1] : 0.0;
  double best = -INFINITY, bS = 0.0;
  int bg = nbins + 1, bn = 0;
  if (tid == 0) best = (double)B / step_time[0];   // keep nothing
  for (int k = hi - 1; k >= lo; k--) {
    n += cnt[k];
    S += fx_value(ssum[k]);
    if (k >= 1) {
      const double G = ((double)B + S) / step_time[n];
      if (G > best) {   // top down: an equal goodput keeps the larger g found first
        best = G;
        bg = k;
        bn = n;
        bS = S;
      }
    }
  }
  // block argmax, ties to the larger g (nbins + 1 = keep nothing counts as the largest)
  for (int o = 32; o > 0; o >>= 1) {
    const double G2 = __shfl_xor(best, o, 64), S2 = __shfl_xor(bS, o, 64);
    const int g2 = __shfl_xor(bg, o, 64), n2 = __shfl_xor(bn, o, 64);
    if (G2 > best || (G2 == best && g2 > bg)) {
      best = G2;
      bg = g2;
      bn = n2;
      bS = S2;
    }
  }
  if ((tid & 63) == 0) {
    bestG[tid >> 6] = best;
    bestg[tid >> 6] = bg;
    bestn[tid >> 6] = bn;
    bestS[tid >> 6] = bS;
  }
  __syncthreads();
  if (tid == 0) {
    int w0 = 0;
    for (int w = 1; w < SCHED_NT / 64; w++)
      if (bestG[w] > bestG[w0] || (bestG[w] == bestG[w0] && bestg[w] > bestg[w0])) w0 = w;
    g_star = bestg[w0];
    out[0] = (double)bestg[w0] / (double)nbins;
    out[1] = (double)bestn[w0];
    out[2] = (double)B + bestS[w0];
    out[3] = bestG[w0];
  }
  __syncthreads();
  const int gs = g_star;
  if (b < B) {
    int L = 0;
    bool go = true;
#pragma unroll
    for (int j = 0; j < MAX_K; j++) {
      go = go && j < K && mb[j] >= gs;   // bins are non-increasing along j: the prefix ends at its first failure
      L += go ? 1 : 0;
    }
    verify_len[b] = L;
  }
}

// ==========================================================================================
// Sequential temperature scaling of the confidence head ("DSpark turns speculation into a
// scheduler", section "Confidence is a serving primitive": left to right, each position's
// temperature minimises the calibration error of the cumulative prefix probability with the
// earlier positions fixed; "The Speed Claim...", section "The Real Innovation").  Per position k:
//   k_sts_eval  workgroups per (grid temperature or unit temperatures, slice of sequences): bin sums for
//               the calibration error of prod_{i<k} c_i(T_i) * sigmoid(z_k / T) over the sequences that
//               verify position k, order-independent bin sums in LDS
//   k_sts_reduce the error of every grid entry from its slices' bin sums
//   k_sts_pick  the smallest error (ties to the earlier grid entry), then every sequence's running
//               products advanced with the chosen and with the unit temperature
// ==========================================================================================
constexpr int STS_NT = 256;
constexpr int STS_MAX_BINS = 64;
constexpr int STS_MAX_GRID = 1024;
constexpr int STS_MAX_K = 256;

__device__ __forceinline__ double sigmoid64(double x) { return 1.0 / (1.0 + exp(-x)); }

__global__ __launch_bounds__(STS_NT) void k_sts_init(int N, double* run, double* run1) {
  for (int n = blockIdx.x * STS_NT + threadIdx.x; n < N; n += gridDim.x * STS_NT) {
    run[n] = 1.0;
    run1[n] = 1.0;
  }
}

// bin sums of grid entry g = blockIdx.x over slice blockIdx.y of the sequences -> part[g][slice][bin]
__global__ __launch_bounds__(STS_NT) void k_sts_eval(const float* z, const int32_t* verify_len,
                                                   const int32_t* accepted_len, int N, int K, int k,
                                                   const double* grid, int G, int nbins, const double* run,
                                                   const double* run1, double* part) {
  __shared__ FxBin sp[STS_MAX_BINS];   // prediction sums, order-independent limbs
  __shared__ int sy[STS_MAX_BINS];
  __shared__ int cnt[STS_MAX_BINS];
  const int tid = threadIdx.x, g = blockIdx.x, sl = blockIdx.y, ns = gridDim.y;
  for (int m = tid; m < nbins; m += STS_NT) {
    fx_clear(sp[m]);
    sy[m] = 0;
    cnt[m] = 0;
  }
  __syncthreads();
  const bool unit = g == G;
  const double T = unit ? 1.0 : grid[g];
  const double* r = unit ? run1 : run;
  const int n0 = (int)((long long)N * sl / ns), n1 = (int)((long long)N * (sl + 1) / ns);
  for (int n = n0 + tid; n < n1; n += STS_NT) {
    const int a = accepted_len[n];
    if (a < 0 || k >= verify_len[n]) continue;
    const double P = r[n] * sigmoid64((double)z[(size_t)n * K + k] / T);
    int m = (int)floor(P * nbins);
    m = m < 0 ? 0 : (m > nbins - 1 ? nbins - 1 : m);
    fx_add(sp[m], P);
    if (k < a) atomicAdd(&sy[m], 1);
    atomicAdd(&cnt[m], 1);
  }
  __syncthreads();
  double* o = part + ((size_t)g * ns + sl) * 3 * STS_MAX_BINS;
  for (int m = tid; m < nbins; m += STS_NT) {
    o[m] = fx_value(sp[m]);
    o[STS_MAX_BINS + m] = (double)sy[m];
    o[2 * STS_MAX_BINS + m] = (double)cnt[m];
  }
}

// calibration error of every grid entry from its slices' bin sums (one thread per entry)
__global__ __launch_bounds__(STS_NT) void k_sts_reduce(int G, int ns, int nbins, const double* part, double* ece) {
  const int g = blockIdx.x * STS_NT + threadIdx.x;
  if (g > G) return;
  double sp[STS_MAX_BINS], sy[STS_MAX_BINS], cn[STS_MAX_BINS];
  for (int m = 0; m < nbins; m++) sp[m] = sy[m] = cn[m] = 0.0;
  for (int sl = 0; sl < ns; sl++) {
    const double* o = part + ((size_t)g * ns + sl) * 3 * STS_MAX_BINS;
    for (int m = 0; m < nbins; m++) {
      sp[m] += o[m];
      sy[m] += o[STS_MAX_BINS + m];
      cn[m] += o[2 * STS_MAX_BINS + m];
    }
  }
  double tot = 0.0, e = 0.0;
  for (int m = 0; m < nbins; m++) tot += cn[m];
  for (int m = 0; m < nbins; m++)
    if (cn[m] > 0.0) e += (cn[m] / tot) * fabs(sp[m] / cn[m] - sy[m] / cn[m]);
  ece[g] = tot > 0.0 ? e : 0.0;
}

__global__ __launch_bounds__(STS_NT) void k_sts_pick(const float* z, int N, int K, int k, const double* grid, int G,
                                                   double* run, double* run1, const double* ece, double* T,
                                                   double* ece_before, double* ece_after) {
  __shared__ int best;
  if (threadIdx.x == 0) {
    int b = 0;
    for (int g = 1; g < G; g++)
      if (ece[g] < ece[b]) b = g;
    best = b;
    if (blockIdx.x == 0) {
      T[k] = grid[b];
      if (ece_after) ece_after[k] = ece[b];
      if (ece_before) ece_before[k] = ece[G];
    }
  }
  __syncthreads();
  const double Tb = grid[best];
  for (int n = blockIdx.x * STS_NT + threadIdx.x; n < N; n += gridDim.x * STS_NT) {
    const double zz = (double)z[(size_t)n * K + k];
    run[n] *= sigmoid64(zz / Tb);
    run1[n] *= sigmoid64(zz);
  }
}

// ==========================================================================================
// Decode loop glue: the context of the next cycle.  The cycle emits tokens[b, 0..a_b] (the
// accepted drafts, then the correction or bonus), so the next cycle's Markov bias at position 0
// starts from tokens[b, a_b], the last token emitted ("DSpark turns speculation into a scheduler",
// opening section: draft, verify, keep the accepted prefix and continue from there).
// ==========================================================================================
__global__ __launch_bounds__(NT) void k_advance(const int32_t* tokens, const int32_t* accepted_len, int B, int K,
                                                int32_t* x0, int64_t* emitted) {
  const int b = blockIdx.x * NT + threadIdx.x;
  if (b >= B) return;
  const int a = accepted_len[b];
  if (a < 0 || a > K) return;   // invalid request: its context stays
  x0[b] = tokens[(size_t)b * (K + 1) + a];
  if (emitted) emitted[b] += a + 1;
}

struct Layout {
  size_t off_L, off_acc, off_phase, off_roles, off_slots, off_xs, off_kreq, off_lse_q, off_logq, off_lse_p, off_logp,
      off_pbias, off_pbias2, off_pplain, off_konst, off_live, total;
  int nrA, nrB, gridB;
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
  // partial records per bias row: room for the fast sweep's one record per noise chunk (the general
  // path's TILE_A-column ranges need fewer)
  l.nrA = (d->V + CHUNK - 1) / CHUNK;
  l.nrB = (d->V + TILE_B - 1) / TILE_B;
  l.gridB = (int)((B * l.nrB + NT / 64 - 1) / (NT / 64));
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
  const size_t nslots = (size_t)bias_slots_max(d->B);
  l.off_pbias = o; o = align256(o + 16 * nslots * (size_t)l.nrA);
  l.off_pbias2 = o; o = align256(o + 16 * nslots * (size_t)l.nrA);
  l.off_pplain = o; o = align256(o + 16 * B * (size_t)l.nrB);
  l.off_konst = o; o = align256(o + 32);
  l.off_live = o; o = align256(o + 4 * (K + 2));
  l.total = o;
  return l;
}

// Per-device caches of device properties.  Each slot is an atomic written with the value the
// runtime reports, so concurrent first calls on one device store the same value and a reader
// sees either 0 (unknown yet) or that value.
constexpr int MAX_DEV = 64;

static int cu_count() {
  static std::atomic<int> ncu[MAX_DEV];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int n = (dev >= 0 && dev < MAX_DEV) ? ncu[dev].load(std::memory_order_relaxed) : 0;
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < MAX_DEV) ncu[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// resident grid of a kernel with per_cu workgroups per CU
static int grid_for(int max_items, int per_cu) {
  const int resident = per_cu * cu_count();
  return max_items < resident ? max_items : resident;
}

static int arch_ok() {
  static std::atomic<int> cache[MAX_DEV];   // 0 unknown, 1 gfx950, -1 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  const int c = (dev >= 0 && dev < MAX_DEV) ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c != 0) return c > 0 ? SPEC_OK : SPEC_E_ARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SPEC_E_HIP;
  const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  if (dev >= 0 && dev < MAX_DEV) cache[dev].store(ok, std::memory_order_relaxed);
  return ok > 0 ? SPEC_OK : SPEC_E_ARCH;
}

// Cooperative launches on the current device (the resident path needs its whole grid resident).
static bool coop_ok() {
  static std::atomic<int> cache[MAX_DEV];   // 0 unknown, 1 supported, -1 not
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  int c = (dev >= 0 && dev < MAX_DEV) ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c == 0) {
    int v = 0;
    c = (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && v != 0) ? 1 : -1;
    if (dev >= 0 && dev < MAX_DEV) cache[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0;
}

// The path a call takes: SPEC_PATH_STEPWISE, SPEC_PATH_RESIDENT, or a negative error code.
// `aligned`: the logit rows allow 16-byte vector loads.
static int resolve_path(const spec_dims* d, bool aligned) {
  if (d->path == SPEC_PATH_STEPWISE) return SPEC_PATH_STEPWISE;
  const bool fits = aligned && res::eligible(d->B, d->K, d->V, d->R, d->dtype, d->noise, cu_count()) && coop_ok();
  if (d->path == SPEC_PATH_RESIDENT) return fits ? SPEC_PATH_RESIDENT : SPEC_E_DTYPE;
  if (d->path != SPEC_PATH_AUTO) return SPEC_E_INVAL;
  // The automatic choice: the resident cycle whenever the call qualifies.  At four requests per
  // compute unit (B = 1024) its workgroups merge their requests one after another, and it is still
  // faster than the stepwise kernels (high-concurrency workload: 1221 against 1566 us per cycle).
  return fits ? SPEC_PATH_RESIDENT : SPEC_PATH_STEPWISE;
}

// Workspace of a call on `path` (SPEC_PATH_AUTO: enough for either path).
static size_t need_bytes(const spec_dims* d, int path) {
  const size_t st = layout(d).total, rs = res::workspace_bytes(d->B, d->K);
  if (path == SPEC_PATH_STEPWISE) return st;
  if (path == SPEC_PATH_RESIDENT) return rs;
  return st > rs ? st : rs;
}

// k_sweep_fast: bias slots whose A rows are staged in LDS, the largest whole number of sub-blocks
// that fits next to the per-request table in the 160 KiB of a workgroup (nine at B <= 256)
// dynamic LDS ceiling of k_sweep_fast: the 160 KiB of a workgroup less its static scan buffer
constexpr size_t FAST_LDS_CAP = (size_t)160 * 1024 - sizeof(uint64_t) * (NT / 64);

static int sweep_fast_group(int B) {
  const size_t cap = FAST_LDS_CAP;
  int g = 16 * SUB;
  while (g > SUB && fast_dyn_bytes(B, g) > cap) g -= SUB;
  return g;
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
  const int G = sweep_fast_group(p.B);
  if (DT == SPEC_BF16 && VEC) {
    // the largest dynamic LDS any call can ask for, set once per device (the attribute is per device)
    static std::atomic<int> set[MAX_DEV];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= MAX_DEV || set[dev].load(std::memory_order_acquire) == 0) {
      (void)hipFuncSetAttribute((const void*)k_sweep_fast<NOISE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)FAST_LDS_CAP);
      if (dev >= 0 && dev < MAX_DEV) set[dev].store(1, std::memory_order_release);
    }
  }
  for (int s = 0; s <= p.K; s++) {
    const int k0 = 1 + 3 * s;
    if (DT == SPEC_BF16 && VEC) {
      hipExtLaunchKernelGGL((k_sweep_fast<NOISE>), dim3(cu_count()), dim3(NT), fast_dyn_bytes(p.B, G), st, tm.start(k0),
                            tm.stop(k0), 0, p, s, G);
      // the plain rows ran inside the sweep: an empty interval keeps the timing slots in place
      if (tm.start(k0 + 1)) {
        (void)hipEventRecord(tm.start(k0 + 1), st);
        (void)hipEventRecord(tm.stop(k0 + 1), st);
      }
    } else {
      hipExtLaunchKernelGGL((k_bias<DT, NOISE, VEC>), dim3(cu_count()), dim3(NT), bias_dyn_bytes(p.B), st,
                            tm.start(k0), tm.stop(k0), 0, p, s);
      hipExtLaunchKernelGGL((k_plain<DT, NOISE, VEC>), dim3(grid_for(l.gridB, 6)), dim3(NT), plain_dyn_bytes(p.B), st,
                            tm.start(k0 + 1), tm.stop(k0 + 1), 0, p, s);
    }
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
  if (d->path != SPEC_PATH_AUTO && d->path != SPEC_PATH_STEPWISE && d->path != SPEC_PATH_RESIDENT) return 0;
  return need_bytes(d, d->path);
}

extern "C" int spec_cycle_path(const spec_dims* d) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!dtype_ok(d)) return SPEC_E_DTYPE;
  return resolve_path(d, true);
}

extern "C" const char* spec_error_string(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_E_INVAL: return "invalid argument (NULL pointer, misaligned pointer or bad dimension)";
    case SPEC_E_DTYPE: return "unsupported dtype, noise scheme or rank for this dtype";
    case SPEC_E_WORKSPACE: return "workspace missing, misaligned or smaller than spec_workspace_bytes()";
    case SPEC_E_ARCH: return "current HIP device is not gfx950";
    case SPEC_E_HIP: return "HIP runtime error";
    case SPEC_E_SCRATCH: return "dimensions need more scratch than the static array of spec_cycle_noalloc holds";
    default: return "unknown error code";
  }
}

extern "C" int spec_version(void) { return 100; }

static int cycle_impl(const spec_dims* d, const void* base_logits, const void* target_logits, const void* A,
                      const void* W, const int32_t* x0, const float* conf, const int32_t* L_in, const float* temp,
                      float threshold, uint64_t seed, int64_t request_offset, int32_t* accepted_len,
                      int32_t* tokens, const spec_diag* diag, void* workspace, size_t workspace_bytes,
                      spec_stream_t stream, const Timing& tm) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!dtype_ok(d)) return SPEC_E_DTYPE;
  if (!base_logits || !target_logits || !A || !W || !(conf || L_in) || !temp || !accepted_len || !tokens)
    return SPEC_E_INVAL;
  if ((((uintptr_t)A) | ((uintptr_t)W)) & 15) return SPEC_E_INVAL;
  const Layout l = layout(d);
  // vector loads need 16-byte aligned rows
  const size_t esz = d->dtype == SPEC_FP32 ? 4 : 2;
  const bool vec = ((d->V * esz) % 16 == 0) && ((((uintptr_t)base_logits) | ((uintptr_t)target_logits)) & 15) == 0;
  if (d->path != SPEC_PATH_AUTO && d->path != SPEC_PATH_STEPWISE && d->path != SPEC_PATH_RESIDENT)
    return SPEC_E_INVAL;
  // the workspace the caller sized for the path it asked for (AUTO: either path)
  if (!workspace || workspace_bytes < need_bytes(d, d->path) || (((uintptr_t)workspace) & 255))
    return SPEC_E_WORKSPACE;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  const int path = resolve_path(d, vec);
  if (path < 0) return path;
  hipStream_t st = (hipStream_t)stream;
  if (path == SPEC_PATH_RESIDENT) {
    res::Args a;
    a.B = d->B;
    a.K = d->K;
    a.V = d->V;
    a.R = d->R;
    a.base = base_logits;
    a.target = target_logits;
    a.A = A;
    a.W = W;
    a.x0 = x0;
    a.conf = conf;
    a.temp = temp;
    a.L_in = L_in;
    a.threshold = threshold;
    a.seed = seed;
    a.req_off = request_offset;
    a.accepted_len = accepted_len;
    a.tokens = tokens;
    a.d_verify_len = diag ? diag->verify_len : nullptr;
    a.d_draft = diag ? diag->draft_tokens : nullptr;
    a.d_logq = diag ? diag->logq : nullptr;
    a.d_logp = diag ? diag->logp : nullptr;
    a.ws = (char*)workspace;
    a.nonce = 0;
    a.G = cu_count();
    (void)hipGetLastError();
    return res::launch(a, st, tm.start(0), tm.stop(0));
  }

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
  p.L_in = L_in;
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
  p.live = (int32_t*)(ws + l.off_live);
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
  p.konst = (const u32x4*)(ws + l.off_konst);
  p.nrB = l.nrB;

  // column ranges of the bias-row partials: one noise chunk on the bf16 fast sweep, TILE_A on the general path
  p.nrA = (d->dtype == SPEC_BF16 && vec) ? (d->V + CHUNK - 1) / CHUNK : (d->V + TILE_A - 1) / TILE_A;
  p.part8 = (d->dtype == SPEC_BF16 && vec && d->noise == SPEC_NOISE_CHUNKED) ? 1 : 0;

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
  return cycle_impl(d, base_logits, target_logits, A, W, x0, conf, nullptr, temp, threshold, seed, request_offset,
                    accepted_len, tokens, diag, workspace, workspace_bytes, stream, tm);
}

extern "C" int spec_cycle_lengths(const spec_dims* d, const void* base_logits, const void* target_logits,
                                  const void* A, const void* W, const int32_t* x0, const int32_t* verify_len,
                                  const float* temp, uint64_t seed, int64_t request_offset, int32_t* accepted_len,
                                  int32_t* tokens, const spec_diag* diag, void* workspace, size_t workspace_bytes,
                                  spec_stream_t stream) {
  if (!verify_len) return SPEC_E_INVAL;
  const Timing tm = {nullptr, 0};
  return cycle_impl(d, base_logits, target_logits, A, W, x0, nullptr, verify_len, temp, 0.0f, seed, request_offset,
                    accepted_len, tokens, diag, workspace, workspace_bytes, stream, tm);
}

// ------------------------------------------------------------------------------------------
// allocation-free variant: the workspace is a static device array, one per GPU
// ------------------------------------------------------------------------------------------
namespace spec {
static __device__ __align__(256) char scratch[SPEC_SCRATCH_BYTES];

// Device address of this device's copy of `scratch`, looked up once per device with that device
// current.  The array's name in host code is only a handle for the lookup, never an address.
static void* scratch_address(int dev) {
  static std::atomic<void*> addr[MAX_DEV];
  if (dev < 0 || dev >= MAX_DEV) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  addr[dev].store(q, std::memory_order_release);
  return q;
}
}  // namespace spec

extern "C" int spec_cycle_noalloc(const spec_dims* d, const void* base_logits, const void* target_logits,
                                  const void* A, const void* W, const int32_t* x0, const float* conf,
                                  const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                                  int32_t* accepted_len, int32_t* tokens, const spec_diag* diag,
                                  spec_stream_t stream) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!dtype_ok(d)) return SPEC_E_DTYPE;
  if (d->path != SPEC_PATH_AUTO && d->path != SPEC_PATH_STEPWISE && d->path != SPEC_PATH_RESIDENT)
    return SPEC_E_INVAL;
  const size_t need = need_bytes(d, d->path);
  if (need > SPEC_SCRATCH_BYTES) return SPEC_E_SCRATCH;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return SPEC_E_HIP;
  const Timing tm = {nullptr, 0};
  return cycle_impl(d, base_logits, target_logits, A, W, x0, conf, nullptr, temp, threshold, seed, request_offset,
                    accepted_len, tokens, diag, ws, SPEC_SCRATCH_BYTES, stream, tm);
}

extern "C" int spec_cycle_kernel_count(const spec_dims* d) {
  if (!dims_ok(d) || !dtype_ok(d)) return 0;
  const int path = resolve_path(d, true);
  if (path < 0) return 0;
  return path == SPEC_PATH_RESIDENT ? 1 : 1 + 3 * (d->K + 1);
}

extern "C" int spec_cycle_timed(const spec_dims* d, const void* base_logits, const void* target_logits,
                                const void* A, const void* W, const int32_t* x0, const float* conf,
                                const float* temp, float threshold, uint64_t seed, int64_t request_offset,
                                int32_t* accepted_len, int32_t* tokens, const spec_diag* diag, void* workspace,
                                size_t workspace_bytes, spec_stream_t stream, void* const* events, int n_events) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!events || n_events < 2 * spec_cycle_kernel_count(d)) return SPEC_E_INVAL;
  const Timing tm = {(hipEvent_t*)events, n_events};
  return cycle_impl(d, base_logits, target_logits, A, W, x0, conf, nullptr, temp, threshold, seed, request_offset,
                    accepted_len, tokens, diag, workspace, workspace_bytes, stream, tm);
}

// ------------------------------------------------------------------------------------------
// acceptance statistics: host side
// ------------------------------------------------------------------------------------------
struct StatsLayout {
  size_t off_konst, off_n, off_rows, off_prev, off_lq, off_lp, off_part, off_res, total;
  int nrA;
};

static StatsLayout stats_layout(const spec_dims* d) {
  StatsLayout l;
  const size_t n = (size_t)d->B * d->K;
  const size_t slots = (n + SUB - 1) / SUB * SUB;
  l.nrA = (d->V + TILE_A - 1) / TILE_A;
  size_t o = 0;
  l.off_konst = o; o = align256(o + 32);
  l.off_n = o; o = align256(o + 4);
  l.off_rows = o; o = align256(o + 4 * n);
  l.off_prev = o; o = align256(o + 4 * n);
  l.off_lq = o; o = align256(o + 4 * n);
  l.off_lp = o; o = align256(o + 4 * n);
  l.off_part = o; o = align256(o + 8 * slots * (size_t)l.nrA);
  // the W-resident statistics kernel's batch arrays and barrier flags (bf16 only)
  l.off_res = o;
  if (d->dtype == SPEC_BF16) o = align256(o + res::stats_layout(d->V, (int)n).total);
  l.total = o;
  return l;
}

extern "C" size_t spec_stats_workspace_bytes(const spec_dims* d) {
  if (!dims_ok(d) || !dtype_ok(d)) return 0;
  return stats_layout(d).total;
}

template <int DT, bool VEC>
static void launch_stats(const StatsParams& sp, hipStream_t st) {
  const int cu = cu_count();
  const int n = sp.c.B * sp.c.K;
  const int merge_grid = (n + NT / 64 - 1) / (NT / 64);
  hipLaunchKernelGGL(k_stats_prep, dim3(1), dim3(NT), 0, st, sp);
  hipLaunchKernelGGL((k_stats_sweep<DT, 1, VEC>), dim3(cu), dim3(NT), 0, st, sp);
  hipLaunchKernelGGL((k_stats_merge<1>), dim3(merge_grid), dim3(NT), 0, st, sp);
  hipLaunchKernelGGL((k_stats_sweep<DT, 2, VEC>), dim3(cu), dim3(NT), 0, st, sp);
  hipLaunchKernelGGL((k_stats_merge<2>), dim3(merge_grid), dim3(NT), 0, st, sp);
}

extern "C" int spec_accept_stats(const spec_dims* d, const void* base_logits, const void* target_logits,
                                 const void* A, const void* W, const int32_t* x0, const int32_t* draft_tokens,
                                 const float* temp, float* alpha, float* lse_q, float* lse_p, void* workspace,
                                 size_t workspace_bytes, spec_stream_t stream) {
  if (!dims_ok(d)) return SPEC_E_INVAL;
  if (!dtype_ok(d)) return SPEC_E_DTYPE;
  if (!base_logits || !target_logits || !A || !W || !draft_tokens || !temp || !alpha) return SPEC_E_INVAL;
  if ((((uintptr_t)A) | ((uintptr_t)W)) & 15) return SPEC_E_INVAL;
  const StatsLayout l = stats_layout(d);
  if (!workspace || workspace_bytes < l.total || (((uintptr_t)workspace) & 255)) return SPEC_E_WORKSPACE;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  char* ws = (char*)workspace;
  StatsParams sp;
  memset(&sp.c, 0, sizeof(sp.c));
  sp.c.B = d->B;
  sp.c.K = d->K;
  sp.c.V = d->V;
  sp.c.R = d->R;
  sp.c.dtype = d->dtype;
  sp.c.noise = d->noise;
  sp.c.base = base_logits;
  sp.c.target = target_logits;
  sp.c.A = A;
  sp.c.W = W;
  sp.c.x0 = x0;
  sp.c.temp = temp;
  sp.c.konst = (const u32x4*)(ws + l.off_konst);
  sp.c.nrA = l.nrA;
  sp.draft = draft_tokens;
  sp.alpha = alpha;
  sp.o_lse_q = lse_q;
  sp.o_lse_p = lse_p;
  sp.n_rows = (int32_t*)(ws + l.off_n);
  sp.rows = (int32_t*)(ws + l.off_rows);
  sp.prev = (int32_t*)(ws + l.off_prev);
  sp.lse_q = (float*)(ws + l.off_lq);
  sp.lse_p = (float*)(ws + l.off_lp);
  sp.part = (float2*)(ws + l.off_part);
  const size_t esz = d->dtype == SPEC_FP32 ? 4 : 2;
  const bool vec = ((d->V * esz) % 16 == 0) && ((((uintptr_t)base_logits) | ((uintptr_t)target_logits)) & 15) == 0;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  // the W-resident kernel where the shape allows it (d->path: AUTO or RESIDENT picks it, STEPWISE
  // the sweep kernels; RESIDENT on a shape that does not qualify is SPEC_E_DTYPE)
  const int G = cu_count() < res::MAX_G ? cu_count() : res::MAX_G;
  const bool res_ok = vec && res::stats_eligible(d->B, d->K, d->V, d->R, d->dtype, G) && coop_ok();
  if (d->path == SPEC_PATH_RESIDENT && !res_ok) return SPEC_E_DTYPE;
  if (d->path != SPEC_PATH_AUTO && d->path != SPEC_PATH_RESIDENT && d->path != SPEC_PATH_STEPWISE) return SPEC_E_INVAL;
  if (res_ok && d->path != SPEC_PATH_STEPWISE) {
    hipLaunchKernelGGL(k_stats_prep, dim3(1), dim3(NT), 0, st, sp);
    if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
    res::StatsArgs a;
    a.B = d->B;
    a.K = d->K;
    a.V = d->V;
    a.R = d->R;
    a.G = G;
    a.base = base_logits;
    a.target = target_logits;
    a.A = A;
    a.W = W;
    a.temp = temp;
    a.n_rows = sp.n_rows;
    a.rows = sp.rows;
    a.prev = sp.prev;
    a.alpha = alpha;
    a.o_lse_q = lse_q;
    a.o_lse_p = lse_p;
    a.ws = ws + l.off_res;
    return res::launch_stats(a, st);
  }
  if (d->dtype == SPEC_BF16) {
    if (vec) launch_stats<SPEC_BF16, true>(sp, st);
    else launch_stats<SPEC_BF16, false>(sp, st);
  } else {
    if (vec) launch_stats<SPEC_FP32, true>(sp, st);
    else launch_stats<SPEC_FP32, false>(sp, st);
  }
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

extern "C" int spec_calibration_error(const float* conf, const int32_t* verify_len, const int32_t* accepted_len,
                                      int32_t B, int32_t K, int32_t nbins, double* ece, int64_t* n_pairs,
                                      spec_stream_t stream) {
  if (!conf || !verify_len || !accepted_len || !ece || !n_pairs) return SPEC_E_INVAL;
  if (B < 1 || B > MAX_B || K < 1 || K > MAX_K || nbins < 1 || nbins > MAX_BINS) return SPEC_E_INVAL;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_calibration, dim3(1), dim3(NT), 0, (hipStream_t)stream, conf, verify_len, accepted_len, B, K,
                     nbins, ece, n_pairs);
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

extern "C" int spec_schedule(const float* conf, int32_t B, int32_t K, const double* step_time, int32_t nbins,
                             int32_t* verify_len, double* out, spec_stream_t stream) {
  if (!conf || !step_time || !verify_len || !out) return SPEC_E_INVAL;
  if (B < 1 || B > MAX_B || K < 1 || K > MAX_K || nbins < 1 || nbins > MAX_SCHED_BINS) return SPEC_E_INVAL;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(SCHED_NT), 0, (hipStream_t)stream, conf, B, K, step_time, nbins,
                     verify_len, out);
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

constexpr int STS_SLICES = 8;   // sequence slices per grid entry: (G + 1) x 8 workgroups fill the chip

extern "C" size_t spec_temperature_scaling_workspace_bytes(int32_t N, int32_t G) {
  if (N < 1 || N > (1 << 24) || G < 1 || G > STS_MAX_GRID) return 0;
  return align256(8 * (size_t)N) * 2 + align256(8 * ((size_t)G + 1)) +
         align256(8 * (size_t)(G + 1) * STS_SLICES * 3 * STS_MAX_BINS);
}

extern "C" int spec_temperature_scaling(const float* z, const int32_t* verify_len, const int32_t* accepted_len,
                                        int32_t N, int32_t K, const double* grid, int32_t G, int32_t nbins,
                                        double* T, double* ece_before, double* ece_after, void* workspace,
                                        size_t workspace_bytes, spec_stream_t stream) {
  if (!z || !verify_len || !accepted_len || !grid || !T) return SPEC_E_INVAL;
  if (N < 1 || N > (1 << 24) || K < 1 || K > STS_MAX_K || G < 1 || G > STS_MAX_GRID || nbins < 1 ||
      nbins > STS_MAX_BINS)
    return SPEC_E_INVAL;
  const size_t need = spec_temperature_scaling_workspace_bytes(N, G);
  if (!workspace || workspace_bytes < need || (((uintptr_t)workspace) & 255)) return SPEC_E_WORKSPACE;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  char* ws = (char*)workspace;
  double* run = (double*)ws;
  double* run1 = (double*)(ws + align256(8 * (size_t)N));
  double* ece = (double*)(ws + 2 * align256(8 * (size_t)N));
  double* part = (double*)(ws + 2 * align256(8 * (size_t)N) + align256(8 * ((size_t)G + 1)));
  hipStream_t st = (hipStream_t)stream;
  const int blocks = min((N + STS_NT - 1) / STS_NT, 4 * cu_count());
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_sts_init, dim3(blocks), dim3(STS_NT), 0, st, N, run, run1);
  for (int k = 0; k < K; k++) {
    hipLaunchKernelGGL(k_sts_eval, dim3(G + 1, STS_SLICES), dim3(STS_NT), 0, st, z, verify_len, accepted_len, N, K,
                       k, grid, G, nbins, run, run1, part);
    hipLaunchKernelGGL(k_sts_reduce, dim3((G + 1 + STS_NT - 1) / STS_NT), dim3(STS_NT), 0, st, G, STS_SLICES, nbins,
                       part, ece);
    hipLaunchKernelGGL(k_sts_pick, dim3(blocks), dim3(STS_NT), 0, st, z, N, K, k, grid, G, run, run1, ece, T,
                       ece_before, ece_after);
  }
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

extern "C" int spec_advance(const int32_t* tokens, const int32_t* accepted_len, int32_t B, int32_t K, int32_t* x0,
                            int64_t* emitted, spec_stream_t stream) {
  if (!tokens || !accepted_len || !x0) return SPEC_E_INVAL;
  if (B < 1 || B > MAX_B || K < 1 || K > MAX_K) return SPEC_E_INVAL;
  const int ac = arch_ok();
  if (ac != SPEC_OK) return ac;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_advance, dim3((B + NT - 1) / NT), dim3(NT), 0, (hipStream_t)stream, tokens, accepted_len, B, K,
                     x0, emitted);
  if (hipGetLastError() != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}
