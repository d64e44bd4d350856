// cycle_resident.hip -- the speculation cycle as ONE persistent launch with the Markov output
// factor W resident on chip (gfx950, bf16 rows, chunked noise).
//
// The cycle is sequential in the draft position (the Markov bias of position s + 1 needs the token
// drawn at s), and every position needs the whole of W (bias_v = A[prev] . W[v] for every v).
// Instead of streaming W from memory once per step, every workgroup owns a fixed slice of the
// vocabulary (at most ten 64-column chunks, see resident.h) and keeps that slice of W in its
// accumulation registers and LDS for the whole cycle: W crosses HBM once per cycle.  The grid is
// one workgroup per CU, launched cooperatively so that all of them are resident together.
//
// One step s (s = 0 .. K) of the cycle:
//   1. every workgroup rebuilds the step's row lists from the per-request roles (a block scan):
//      bias rows (DRAFT: position s of a request with s < L_b; CORRECT: the position rejected at
//      step s - 1) in 32-row sub-blocks, and plain rows (LSEP: the target row of the position
//      verified at step s; BONUS: the target row L_b of a request whose drafts all survived);
//   2. bias sub-blocks: the gathered A rows of the sub-block are staged in LDS (the MFMA B
//      operands), each wave runs v_mfma_f32_32x32x16_bf16 chains over its W tiles with the
//      accumulators seeded by the draft logits, so the chain leaves base + bias in registers;
//      the element-wise part gives, per row and 64-column chunk, the chunk log-mass and its
//      Gumbel score (DRAFT), or the residual mass sum max(0, p - q) and the target chunk log-mass
//      (CORRECT); the four waves' results are merged into ONE record per (row, workgroup);
//   3. plain rows: each workgroup streams its slice of every plain row: the row log-mass, and for
//      BONUS rows the chunk scores too; one record per (row, workgroup);
//   4. grid barrier;
//   5. merge: request b is finished by workgroup b % G (its requests one after another): it reduces the G
//      records of each of its rows, draws level two of the chunked sampler inside the winning
//      chunk (re-reading that chunk's 64 columns and W rows), takes the accept decision, writes
//      the outputs and publishes the request's roles of step s + 1 in tagged words (see publish),
//      which the lists of step s + 1 poll: no second grid barrier.
// The step loop ends when no request has a role left; every workgroup sees the same roles, so
// they all leave together.
//
// Grid barrier: once every wave's stores of the phase have completed, every workgroup stores a
// 64-bit token (a per-call nonce plus the barrier's index) into its own flag word, then one wave
// polls all G flags until each is within [token, token + 2^16) (a workgroup can be at most one
// barrier ahead).  Everything exchanged across workgroups goes through device-coherent loads and
// stores (see st_u64 / ld_u64 below), so the barrier needs no cache write-back or invalidation.  Flags left from
// earlier calls never fall in that window (the nonce differs), so nothing is cleared between
// calls.  A wait that has not finished after about a second sets the workspace's error word and
// gives up; every later barrier then passes at once and the merges mark every request invalid, so
// a synchronisation fault ends the kernel with invalid outputs instead of hanging the GPU.  The
// lists' wait for the published words has the same limit and the same error word.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <stdlib.h>
#include <time.h>
#include <unistd.h>

#include <atomic>

#include "device_common.h"
#include "resident.h"
#include "spec_cycle.h"

namespace spec {
namespace res {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Masked 16-byte loads are still issued, at an address clamped inside their tensor (or, for
// buffer loads, past its end, which reads zeros), so that every load is unconditional with nothing
// waiting on it until its value is used.  Where the value matters it is replaced at its use by one
// of these (eight bf16 -inf, or zeros).  Tiles of a slot without a row, or of a chunk the
// workgroup does not own, are computed on whatever their loads return and their results are
// discarded.
constexpr u32x4 kNegInf = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
constexpr u32x4 kZero = {0u, 0u, 0u, 0u};

enum : int { RO_DRAFT = 1, RO_CORRECT = 2, RO_LSEP = 4, RO_BONUS = 8 };
enum : int { PH_ALIVE = 0, PH_REJECTED = 1, PH_DONE = 2, PH_INVALID = 3 };
enum : int { ST_L = 0, ST_ACC = 1, ST_PHASE = 2, ST_ROLES = 3 /* and 4: two step parities */ };
// A bias-slot entry: bit 0 CORRECT, bits 1..10 the request, bits 11.. the previous token + 1 (0 =
// no Markov bias); a slot without a row holds NO_ENT.
constexpr uint32_t NO_ENT = 0xFFFFFFFFu;
__device__ __forceinline__ uint32_t ent_make(int b, bool corr, int prev) {
  return ((uint32_t)(prev + 1) << 11) | ((uint32_t)b << 1) | (corr ? 1u : 0u);
}
__device__ __forceinline__ int ent_req(uint32_t e) { return (int)((e >> 1) & 1023u); }
__device__ __forceinline__ int ent_prev(uint32_t e) { return (int)(e >> 11) - 1; }
constexpr uint64_t TOKEN_WINDOW = 1ull << 16;

constexpr uint64_t WAIT_TICKS = 100000000ull;   // default wait limit; s_memrealtime runs at 100 MHz: one second

// per-request inputs of the step's bias rows, rebuilt by every workgroup at every step
struct ReqMeta {
  int prev_d;        // token before position s (x0 at s = 0); -1 = no Markov bias
  int prev_c;        // token before position s - 1
  float invT;
  float lse_p_c;     // log-normalisers of the target and draft rows at position s - 1
  float lse_q_c;
  uint32_t key_d[2]; // DRAFT_C noise key of position s
  uint32_t key_c[2]; // RESIDUAL_C noise key of position s - 1
  uint32_t key_r[2]; // the request's noise key (set-up)
};

struct Lists {
  int n_draft, n_correct, n_plain, c0, n_sb;
};

// per-wave result of one bias row over the wave's tiles (LDS, merged by the workgroup)
struct WaveRec {
  float4 a;   // DRAFT: {log-mass of the wave's chunks, best chunk score, best chunk, half-tile log-mass}
              // CORRECT: {log residual mass, best score, best chunk, half-tile residual mass (linear)}
  float4 t;   // CORRECT: {target log-mass, best score, best chunk, half-tile target log-mass}
};

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t key_of(const uint32_t (&k)[2]) { return (uint64_t)k[0] | ((uint64_t)k[1] << 32); }
__device__ __forceinline__ void put_key(uint32_t (&k)[2], uint64_t v) {
  k[0] = (uint32_t)v;
  k[1] = (uint32_t)(v >> 32);
}
__device__ __forceinline__ uint64_t req_key(uint64_t seed, int64_t gid) { return sm_first(sm_first(seed) ^ (uint64_t)gid); }
__device__ __forceinline__ uint64_t pos_key(uint64_t kreq, int pos, uint64_t stream) {
  return sm_first(sm_first(kreq ^ (uint64_t)pos) ^ stream);
}

// threadIdx.x behind an opaque copy: values derived from it are rebuilt where they are used
// instead of being hoisted out of the (long) step loop and kept in registers
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Gumbel noise from 32 random bits without branches: the same three cases and the same
// arithmetic as gumbel_bits (series for u < 1/64, -log(1 - u) below 1/2, the exact complement
// above), with the logarithm's argument selected instead of the code path, so the results are
// identical and the whole element-wise part stays straight-line code.
__device__ __forceinline__ float gumbel_bf(uint32_t b) {
  const bool lo = b < 0x80000000u;
  const float u = ((float)b + 0.5f) * 0x1p-32f;
  const float c = (float)(~b) + 0.5f;
  float series = u * fmaf(u, fmaf(u, fmaf(u, fmaf(u, 0.2f, 0.25f), 0.33333334f), 0.5f), 1.0f);
  const float lg = lg2(lo ? 1.0f - u : c);
  float e_lo = -lg * LN2, e_hi = (32.0f - lg) * LN2;
  // every candidate is computed on every lane, so the selects below stay selects (no exec-masked
  // blocks, which would split the scheduling region this runs in)
  asm volatile("" : "+v"(series), "+v"(e_lo), "+v"(e_hi));
  const float e = lo ? (u < 0.015625f ? series : e_lo) : e_hi;
  return -lg2(e) * LN2;
}

// 16-byte load of global memory at `p` (the cast keeps it a global load when `p` itself was read
// from memory, where the compiler no longer knows its address space)
__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4*)p;
}

// log(exp(a) + exp(b)), -inf aware, NaN propagating
__device__ __forceinline__ float lse_add(float a, float b) { return lse2(a, b); }

// argmax take rule: larger score, smaller chunk / index on ties, index < 0 = none
__device__ __forceinline__ bool takes(float s2, int i2, float s1, int i1) {
  return i2 >= 0 && (i1 < 0 || s2 > s1 || (s2 == s1 && (unsigned)i2 < (unsigned)i1));
}

// Lane exchanges without address registers: DPP within 16-lane rows, a swizzle across the two
// rows of each 32-lane half (lane ^ 16), a permlane swap across the halves (lane ^ 32).
__device__ __forceinline__ int xor16i(int x) { return __builtin_amdgcn_ds_swizzle(x, 0x401F); }
__device__ __forceinline__ float xor16f(float x) { return __int_as_float(xor16i(__float_as_int(x))); }
// Maximum that propagates NaN (v_maximum3_f32 on gfx950).  Unlike fmaxf it needs no quieting of
// operands the compiler cannot prove canonical (accumulators, unpacked bf16), which would cost one
// more instruction per operand; where the maxima below are taken, a NaN in the values makes the
// result NaN either way (it reaches the sum of exponentials).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// A value and its partner lane's (lane ^ 32) from one v_permlane32_swap: .x holds the value of the
// lower lane of the pair, .y that of the upper, in both lanes (so reductions need no select).
__device__ __forceinline__ float2 pair32(float x) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return make_float2(__int_as_float((int)r[0]), __int_as_float((int)r[1]));
}
__device__ __forceinline__ float pmax32(float x) {
  const float2 r = pair32(x);
  return vmax(r.x, r.y);
}
__device__ __forceinline__ float psum32(float x) {
  const float2 r = pair32(x);
  return r.x + r.y;
}
template <int CTRL>
__device__ __forceinline__ int dppi(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// wave-wide reductions (every lane gets the result): xor 1, xor 2, half-row mirror, row mirror,
// then xor 16 and xor 32
__device__ __forceinline__ float wmax(float x) {
  x = vmax(x, dpp<0xB1>(x));
  x = vmax(x, dpp<0x4E>(x));
  x = vmax(x, dpp<0x141>(x));
  x = vmax(x, dpp<0x140>(x));
  x = vmax(x, xor16f(x));
  return pmax32(x);
}
__device__ __forceinline__ float wsum(float x) {
  x = sum8(x);
  x += dpp<0x140>(x);
  x += xor16f(x);
  return psum32(x);
}

// one argmax step against the partner values
__device__ __forceinline__ void am_take(float& sc, int& ix, float& aux, float s2, int i2, float a2) {
  const bool t = takes(s2, i2, sc, ix);
  sc = t ? s2 : sc;
  ix = t ? i2 : ix;
  aux = t ? a2 : aux;
}
template <int CTRL>
__device__ __forceinline__ void am_dpp(float& sc, int& ix, float& aux) {
  am_take(sc, ix, aux, dpp<CTRL>(sc), dppi<CTRL>(ix), dpp<CTRL>(aux));
}
// wave argmax of (score, index) with a float payload; every lane gets the winner (the take rule
// is commutative, so the mirror steps reduce like the xor steps)
__device__ __forceinline__ void wargmax(float& sc, int& ix, float& aux) {
  am_dpp<0xB1>(sc, ix, aux);    // xor 1
  am_dpp<0x4E>(sc, ix, aux);    // xor 2
  am_dpp<0x141>(sc, ix, aux);   // half-row mirror
  am_dpp<0x140>(sc, ix, aux);   // row mirror
  am_take(sc, ix, aux, xor16f(sc), xor16i(ix), xor16f(aux));
  am_take(sc, ix, aux, xor32f(sc), xor32i(ix), xor32f(aux));
}

// log-sum-exp of invT * y over N values of a lane and its partner lane (lane ^ 32): every -inf
// gives -inf, a NaN gives NaN
template <int N>
__device__ __forceinline__ float pair_lse(const float* y, float invT) {
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    m0 = vmax(m0, y[i]);
    m1 = vmax(m1, y[i + 1]);
  }
  float mx = vmax(m0, m1);
  mx = pmax32(mx);
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
  sum = psum32(sum);
  return (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
}

// log-sum-exp of invT * x over the values of NT tiles (16 per lane each) of a lane and its
// partner lane, read straight from the accumulators
template <int NTL>
__device__ __forceinline__ float tiles_lse(const f32x16* a, float invT) {
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int t = 0; t < NTL; t++)
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      m0 = vmax(m0, a[t][q]);
      m1 = vmax(m1, a[t][q + 1]);
    }
  float mx = vmax(m0, m1);
  mx = pmax32(mx);
  const float c = invT * LOG2E, mo = (mx == -INFINITY) ? 0.0f : mx * c;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int t = 0; t < NTL; t++)
#pragma unroll
    for (int q = 0; q < 16; q += 4) {
      s0 += ex2(fmaf(a[t][q], c, -mo));
      s1 += ex2(fmaf(a[t][q + 1], c, -mo));
      s2 += ex2(fmaf(a[t][q + 2], c, -mo));
      s3 += ex2(fmaf(a[t][q + 3], c, -mo));
    }
  float sum = (s0 + s1) + (s2 + s3);
  sum = psum32(sum);
  return (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
}

// log-sum-exp of invT * x over the 32 values of two accumulator tiles of a lane and its partner
// lane (lane ^ 32); -inf everywhere gives -inf, a NaN gives NaN
__device__ __forceinline__ float lse_two(const f32x16& x, const f32x16& y, float invT) {
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int q = 0; q < 16; q += 2) {
    m0 = vmax(m0, vmax(x[q], y[q]));
    m1 = vmax(m1, vmax(x[q + 1], y[q + 1]));
  }
  const float mx = pmax32(vmax(m0, m1));
  const float c = invT * LOG2E, mo = (mx == -INFINITY) ? 0.0f : mx * c;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; q += 2) {
    s0 += ex2(fmaf(x[q], c, -mo));
    s1 += ex2(fmaf(x[q + 1], c, -mo));
    s2 += ex2(fmaf(y[q], c, -mo));
    s3 += ex2(fmaf(y[q + 1], c, -mo));
  }
  const float sum = psum32((s0 + s1) + (s2 + s3));
  return (mx == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sum) * LN2;
}

// Scheduling helpers.  vfence(x) is an empty statement with side effects that reads and redefines
// x: work that produces x stays before it, work that consumes it after it.  interleave<M, D, V>()
// asks the scheduler for 16 groups of (M MFMAs, D LDS reads, V VALU instructions) in the current
// region, the shape of one 16-k-step chain with its shadow work.
template <class T>
__device__ __forceinline__ void vfence(T& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void vfence(u32x4 (&x)[2]) {
  asm volatile("" : "+v"(x[0]));
  asm volatile("" : "+v"(x[1]));
}
template <int M, int D, int V>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int t = 0; t < KSTEPS; t++) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);   // LDS read
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // VALU
  }
}


// The element-wise work of a bias sub-block, cut into slices that run one per k-step of an MFMA
// chain.  Each slice's state is fenced at the k-step boundary (fence_*), which pins the slice to its
// k-step: its inputs are defined at the step's start and its outputs consumed at its end.
//
// Log-sum-exp of invT * x over the 32 values of two accumulator tiles (x, y) of a lane and its
// partner lane: the maximum in steps 0..3 (8 values each), the exchange in step 4, the scaled
// exponential sums in steps 5..12 (4 values each), the result in step 13.  -inf everywhere gives
// -inf, a NaN gives NaN.
struct Lse2 {
  float m0, m1, m2, m3, mo;   // running maxima, then the maximum (m0) and its scaled value
  float f0, f1, f2, f3;       // scaled exponents of the group in flight
  float e0, e1, e2, e3;       // their exponentials
  float s0, s1, s2, s3;       // running sums
  float r;                    // the result
};
__device__ __forceinline__ void lse2_init(Lse2& st) {
  st.m0 = st.m1 = st.m2 = st.m3 = -INFINITY;
  st.mo = st.f0 = st.f1 = st.f2 = st.f3 = st.e0 = st.e1 = st.e2 = st.e3 = 0.0f;
  st.s0 = st.s1 = st.s2 = st.s3 = st.r = 0.0f;
}
// Software-pipelined exponential sums: in one slice the scaled exponents of group g, the
// exponentials of group g - 1 and the additions of group g - 2, so that no instruction of a slice
// waits on another of the same slice (one wave per SIMD has no other wave to hide that latency).
// v(g, i): value i (0..3) of group g.
template <class VF>
__device__ __forceinline__ void lse_pipe(Lse2& st, int g, int ng, VF v, float c) {
  if (g >= 2 && g - 2 < ng) {
    st.s0 += st.e0;
    st.s1 += st.e1;
    st.s2 += st.e2;
    st.s3 += st.e3;
  }
  if (g >= 1 && g - 1 < ng) {
    st.e0 = ex2(st.f0);
    st.e1 = ex2(st.f1);
    st.e2 = ex2(st.f2);
    st.e3 = ex2(st.f3);
  }
  if (g < ng) {
    st.f0 = fmaf(v(g, 0), c, -st.mo);
    st.f1 = fmaf(v(g, 1), c, -st.mo);
    st.f2 = fmaf(v(g, 2), c, -st.mo);
    st.f3 = fmaf(v(g, 3), c, -st.mo);
  }
}
__device__ __forceinline__ void lse_pipe_fence(Lse2& st, int g, int ng) {
  if (g >= 2 && g - 2 < ng) {
    vfence(st.s0);
    vfence(st.s1);
    vfence(st.s2);
    vfence(st.s3);
  }
  if (g >= 1 && g - 1 < ng) {
    vfence(st.e0);
    vfence(st.e1);
    vfence(st.e2);
    vfence(st.e3);
  }
  if (g < ng) {
    vfence(st.f0);
    vfence(st.f1);
    vfence(st.f2);
    vfence(st.f3);
  }
}
__device__ __forceinline__ void lse_fold_max(Lse2& st, float c) {
  st.m0 = pmax32(vmax(vmax(st.m0, st.m1), vmax(st.m2, st.m3)));
  st.mo = (st.m0 == -INFINITY) ? 0.0f : st.m0 * c;
}
__device__ __forceinline__ void lse_result(Lse2& st, float invT) {
  const float sum = psum32((st.s0 + st.s1) + (st.s2 + st.s3));
  st.r = (st.m0 == -INFINITY) ? (sum == 0.0f ? -INFINITY : NAN) : st.m0 * invT + lg2(sum) * LN2;
}

// Log-sum-exp of invT * x over the 32 values of two accumulator tiles (x, y) of a lane and its
// partner lane, in 16 slices: the maximum in slices 0..3 (8 values each, four chains), the
// exchange with the partner in slice 4, the pipelined exponential sums (eight groups of four) in
// slices 5..14, the result in slice 15.  -inf everywhere gives -inf, a NaN gives NaN.
__device__ __forceinline__ void lse2_step(Lse2& st, int t, const f32x16& x, const f32x16& y, float c, float invT) {
  if (t < 4) {
    const int q = 4 * t;
    st.m0 = vmax(st.m0, vmax(x[q], y[q]));
    st.m1 = vmax(st.m1, vmax(x[q + 1], y[q + 1]));
    st.m2 = vmax(st.m2, vmax(x[q + 2], y[q + 2]));
    st.m3 = vmax(st.m3, vmax(x[q + 3], y[q + 3]));
  } else if (t == 4) {
    lse_fold_max(st, c);
  } else if (t < 15) {
    lse_pipe(st, t - 5, 8, [&](int g, int i) { return (i < 2) ? x[2 * g + i] : y[2 * g + i - 2]; }, c);
  } else {
    lse_result(st, invT);
  }
}
__device__ __forceinline__ void lse2_fence(Lse2& st, int t) {
  if (t < 4) {
    vfence(st.m0);
    vfence(st.m1);
    vfence(st.m2);
    vfence(st.m3);
  } else if (t == 4) {
    vfence(st.m0);
    vfence(st.mo);
  } else if (t < 15) {
    lse_pipe_fence(st, t - 5, 8);
  } else {
    vfence(st.r);
  }
}

// The same for the 16 values of one tile, in 9 slices: the maximum in slices 0 and 1 (and the
// exchange in 1), the exponential sums (four groups) in slices 2..7, the result in slice 8.
__device__ __forceinline__ void lse1_step(Lse2& st, int t, const f32x16& x, float c, float invT) {
  if (t < 2) {
    const int q = 8 * t;
    st.m0 = vmax(st.m0, vmax(x[q], x[q + 4]));
    st.m1 = vmax(st.m1, vmax(x[q + 1], x[q + 5]));
    st.m2 = vmax(st.m2, vmax(x[q + 2], x[q + 6]));
    st.m3 = vmax(st.m3, vmax(x[q + 3], x[q + 7]));
    if (t == 1) lse_fold_max(st, c);
  } else if (t < 8) {
    lse_pipe(st, t - 2, 4, [&](int g, int i) { return x[4 * g + i]; }, c);
  } else if (t == 8) {
    lse_result(st, invT);
  }
}
__device__ __forceinline__ void lse1_fence(Lse2& st, int t) {
  if (t < 2) {
    vfence(st.m0);
    vfence(st.m1);
    vfence(st.m2);
    vfence(st.m3);
    if (t == 1) vfence(st.mo);
  } else if (t < 8) {
    lse_pipe_fence(st, t - 2, 4);
  } else if (t == 8) {
    vfence(st.r);
  }
}

// Gumbel noise of index i of a noise row (the same arithmetic as gumbel_bf(bits_at(key, i))) in
// four slices: the two SplitMix64 rounds, the uniform and the logarithm's argument, the result.
struct GumbelStage {
  uint32_t lo, hi;
  float u, lg, series, r;
};
__device__ __forceinline__ void gumbel_step(GumbelStage& g, int t, uint64_t key, uint32_t i) {
  if (t == 0) {
    uint64_t z = key + (uint64_t)((i >> 1) + 1u) * SM_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    g.lo = (uint32_t)z;
    g.hi = (uint32_t)(z >> 32);
  } else if (t == 1) {
    uint64_t z = (uint64_t)g.lo | ((uint64_t)g.hi << 32);
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    g.lo = (i & 1u) ? (uint32_t)z : (uint32_t)(z >> 32);   // the index's 32 bits
  } else if (t == 2) {
    const uint32_t b = g.lo;
    const bool lo = b < 0x80000000u;
    g.u = ((float)b + 0.5f) * 0x1p-32f;
    const float c = (float)(~b) + 0.5f;
    g.series = g.u * fmaf(g.u, fmaf(g.u, fmaf(g.u, fmaf(g.u, 0.2f, 0.25f), 0.33333334f), 0.5f), 1.0f);
    g.lg = lg2(lo ? 1.0f - g.u : c);
  } else if (t == 3) {
    const bool lo = g.lo < 0x80000000u;
    const float e = lo ? (g.u < 0.015625f ? g.series : -g.lg * LN2) : (32.0f - g.lg) * LN2;
    g.r = -lg2(e) * LN2;
  }
}
__device__ __forceinline__ void gumbel_fence(GumbelStage& g, int t) {
  if (t == 0) {
    vfence(g.lo);
    vfence(g.hi);
  } else if (t == 1) {
    vfence(g.lo);
  } else if (t == 2) {
    vfence(g.u);
    vfence(g.lg);
    vfence(g.series);
  } else if (t == 3) {
    vfence(g.r);
  }
}

// residual mass sum max(0, p - q) over N values of a lane and its partner lane; t = target logits,
// y = draft logits (before the temperature), lse_p / lse_q the rows' log-normalisers
template <int N>
__device__ __forceinline__ float pair_residual(const float* t, const float* y, float invT, float lse_p, float lse_q) {
  const float c = invT * LOG2E, op = -lse_p * LOG2E, oq = -lse_q * LOG2E;
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const float a2 = fmaf(t[i], c, op), b2 = fmaf(y[i], c, oq);
    const float a3 = fmaf(t[i + 1], c, op), b3 = fmaf(y[i + 1], c, oq);
    if (a2 > b2) m0 += ex2(a2) - ex2(b2);
    if (a3 > b3) m1 += ex2(a3) - ex2(b3);
  }
  float m = m0 + m1;
  return psum32(m);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// bf16 logits of one 16-byte piece into half `hf` of a tile's 16 accumulator values
__device__ __forceinline__ void seed_piece(f32x16& a, const u32x4& w, int hf) {
#pragma unroll
  for (int e = 0; e < 4; e++) {
    a[8 * hf + 2 * e] = bf_lo(w[e]);
    a[8 * hf + 2 * e + 1] = bf_hi(w[e]);
  }
}


// bf16 value i (0..8NP-1) of NP packed 16-byte pieces
template <int NP>
__device__ __forceinline__ float pk(const u32x4* t, int i) {
  const uint32_t w = t[i >> 3][(i >> 1) & 3];
  return (i & 1) ? bf_hi(w) : bf_lo(w);
}

// draft value i (0..31) of a chunk held in two accumulator tiles
__device__ __forceinline__ float acc2(const f32x16& a0, const f32x16& a1, int i) { return i < 16 ? a0[i] : a1[i - 16]; }
// target value i (0..31) of a chunk held in four packed pieces (two per tile)
__device__ __forceinline__ float tgt4(const u32x4& t0, const u32x4& t1, const u32x4& t2, const u32x4& t3, int i) {
  const u32x4& t = i < 8 ? t0 : (i < 16 ? t1 : (i < 24 ? t2 : t3));
  const uint32_t w = t[(i >> 1) & 3];
  return (i & 1) ? bf_hi(w) : bf_lo(w);
}

// CORRECT element-wise slice: values i0, i0 + 1 of a chunk held in two accumulator tiles (x, y:
// draft logits with the Markov bias) and four packed target pieces.  With p = exp2(t c + op) and
// q = exp2(x c + oq) the normalised target and draft probabilities (op, oq: minus the rows'
// log-normalisers in base 2), it adds max(p - q, 0) to the residual sums and p to the target sums.
struct Corr2 {
  float r0, r1, p0, p1;
};
__device__ __forceinline__ void corr_step(Corr2& st, int i0, const f32x16& x, const f32x16& y, const u32x4& t0,
                                          const u32x4& t1, const u32x4& t2, const u32x4& t3, float c, float op,
                                          float oq) {
#pragma unroll
  for (int i = i0; i < i0 + 2; i++) {
    const float ep = ex2(fmaf(tgt4(t0, t1, t2, t3, i), c, op));
    const float eq = ex2(fmaf(acc2(x, y, i), c, oq));
    // max(p - q, 0) as the subtraction's result clamped to [0, 1] (p and q lie in [0, 1]; a NaN
    // clamps to 0, as the maximum with 0 would give)
    const float r = __builtin_amdgcn_fmed3f(ep - eq, 0.0f, 1.0f);
    if (i & 1) {
      st.r1 += r;
      st.p1 += ep;
    } else {
      st.r0 += r;
      st.p0 += ep;
    }
  }
}
__device__ __forceinline__ void corr_fence(Corr2& st) {
  vfence(st.r0);
  vfence(st.r1);
  vfence(st.p0);
  vfence(st.p1);
}
// residual mass (linear) and target log-mass of a lane pair's sums; lse_p: the target row's
// log-normaliser (natural units)
__device__ __forceinline__ void corr_end(const Corr2& st, float lse_p, float& mass, float& tlse) {
  mass = psum32(st.r0 + st.r1);
  const float sp = psum32(st.p0 + st.p1);
  tlse = sp > 0.0f ? lse_p + lg2(sp) * LN2 : (sp == 0.0f ? -INFINITY : NAN);
}

// CORRECT element-wise part of one chunk (two tiles) of a lane and its partner lane: the residual
// mass sum max(0, p - q) (linear) and the target log-mass, straight from the accumulators and the
// packed target logits
__device__ __forceinline__ void chunk_correct(const f32x16& a0, const f32x16& a1, const u32x4& t0, const u32x4& t1,
                                              const u32x4& t2, const u32x4& t3, float invT, float lse_p, float lse_q,
                                              float& mass, float& tlse) {
  const float c = invT * LOG2E, op = -lse_p * LOG2E, oq = -lse_q * LOG2E;
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 32; i++) tm = fmaxf(tm, tgt4(t0, t1, t2, t3, i));
  tm = pmax32(tm);
  const float mo = (tm == -INFINITY) ? 0.0f : tm * c;
  float m0 = 0.0f, m1 = 0.0f, s0 = 0.0f, s1 = 0.0f;
  // in groups of eight values, each group scheduled on its own: the register peak stays small
#pragma unroll
  for (int g8 = 0; g8 < 32; g8 += 8) {
#pragma unroll
    for (int i = g8; i < g8 + 8; i += 2) {
      const float ta = tgt4(t0, t1, t2, t3, i), tb = tgt4(t0, t1, t2, t3, i + 1);
      const float pa = fmaf(ta, c, op), qa = fmaf(acc2(a0, a1, i), c, oq);
      const float pb = fmaf(tb, c, op), qb = fmaf(acc2(a0, a1, i + 1), c, oq);
      if (pa > qa) m0 += ex2(pa) - ex2(qa);
      if (pb > qb) m1 += ex2(pb) - ex2(qb);
      s0 += ex2(fmaf(ta, c, -mo));
      s1 += ex2(fmaf(tb, c, -mo));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  float m = m0 + m1, sm = s0 + s1;
  mass = psum32(m);
  sm = psum32(sm);
  tlse = (tm == -INFINITY) ? (sm == 0.0f ? -INFINITY : NAN) : tm * invT + lg2(sm) * LN2;
}

// CORRECT element-wise part over 8 NP values of a lane and its partner lane, the target values
// unpacked on the fly from NP 16-byte pieces: the residual mass sum max(0, p - q) (linear) and the
// target log-mass
template <int NP>
__device__ __forceinline__ void pair_correct(const float* y, const u32x4* tp, float invT, float lse_p, float lse_q,
                                             float& mass, float& tlse) {
  constexpr int N = 8 * NP;
  const float c = invT * LOG2E, op = -lse_p * LOG2E, oq = -lse_q * LOG2E;
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; i++) tm = fmaxf(tm, pk<NP>(tp, i));
  tm = pmax32(tm);
  const float mo = (tm == -INFINITY) ? 0.0f : tm * c;
  float m0 = 0.0f, m1 = 0.0f, s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const float t0 = pk<NP>(tp, i), t1 = pk<NP>(tp, i + 1);
    const float a0 = fmaf(t0, c, op), b0 = fmaf(y[i], c, oq);
    const float a1 = fmaf(t1, c, op), b1 = fmaf(y[i + 1], c, oq);
    if (a0 > b0) m0 += ex2(a0) - ex2(b0);
    if (a1 > b1) m1 += ex2(a1) - ex2(b1);
    s0 += ex2(fmaf(t0, c, -mo));
    s1 += ex2(fmaf(t1, c, -mo));
  }
  float m = m0 + m1, sm = s0 + s1;
  mass = psum32(m);
  sm = psum32(sm);
  tlse = (tm == -INFINITY) ? (sm == 0.0f ? -INFINITY : NAN) : tm * invT + lg2(sm) * LN2;
}

// 16 logits of a lane (two 16-byte pieces) -> floats
__device__ __forceinline__ void unpack16(u32x4 a, u32x4 b, float* o) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[2 * i] = bf_lo(a[i]);
    o[2 * i + 1] = bf_hi(a[i]);
    o[8 + 2 * i] = bf_lo(b[i]);
    o[8 + 2 * i + 1] = bf_hi(b[i]);
  }
}

// ------------------------------------------------------------------------------------------
// Data exchanged between workgroups (records, roles, drafted tokens, log-normalisers) is written
// and read only through these device-coherent accessors: relaxed agent-scope atomics, which the
// gfx950 code generator emits as sc1 loads and stores that are coherent across the XCDs without
// any cache write-back or invalidation.  The grid barrier then only has to order them (each wave
// waits for its own stores to complete before its workgroup announces arrival).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void st_u64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64(const void* p) {
  return __hip_atomic_load((uint64_t*)const_cast<void*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_i32(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_i32(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f32(float* p, float v) { st_i32((int32_t*)p, __float_as_int(v)); }
__device__ __forceinline__ float ld_f32(const float* p) { return __int_as_float(ld_i32((const int32_t*)p)); }
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
// Records (16 bytes) move through buffer loads and stores with the device-scope cache policy
// (sc1): the same coherence as the atomics above, one 16-byte access per lane, and lanes that read
// consecutive records coalesce.  The descriptor covers one record area (out-of-range offsets read
// zero and drop writes).
constexpr int CPOL_SC1 = 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void rec_store(__amdgpu_buffer_rsrc_t r, size_t idx, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)(idx * 16), 0, CPOL_SC1);
}
__device__ __forceinline__ float4 rec_load(__amdgpu_buffer_rsrc_t r, size_t idx) {
  const f32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(idx * 16), 0, CPOL_SC1);
  return make_float4(x[0], x[1], x[2], x[3]);
}

// Read-only operand loads (logits, A rows) through a descriptor over a whole tensor of `bytes`
// bytes (< 4 GiB): ordinary cache policy; offsets at or past `bytes` read zeros.
constexpr uint32_t OOB_OFF = 0x80000000u;   // past the end of A (the resident cycle takes A below 2 GiB)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ld_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ldb16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// ------------------------------------------------------------------------------------------
// grid barrier on per-workgroup flags (see the file header)
// ------------------------------------------------------------------------------------------
// the error word holds the nonce of a call whose barrier timed out (any other value: no error)
__device__ __forceinline__ bool failed(const uint64_t* err, uint64_t nonce) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nonce;
}

__device__ void grid_barrier(uint64_t* flags, uint64_t* err, uint64_t nonce, int G, uint64_t token, uint64_t wait_ticks) {
  // every wave's coherent stores of this phase have completed before its workgroup announces
  // arrival (the clobber keeps the compiler from moving memory operations across the wait)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int tid = opaque_tid();
  if (tid < 64) {
    const int lane = tid;
    if (lane == 0)
      __hip_atomic_store(&flags[(size_t)blockIdx.x * FLAG_STRIDE], token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      bool ok = true;
      for (int i = lane; i < G; i += 64) {
        const uint64_t f = __hip_atomic_load(&flags[(size_t)i * FLAG_STRIDE], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = ok && (f - token) < TOKEN_WINDOW;
      }
      if (__all(ok)) break;
      if (failed(err, nonce)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) {
        if (lane == 0) __hip_atomic_store(err, nonce, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  // the coherent loads of the next phase are issued after every workgroup has arrived
  __syncthreads();
}

// ------------------------------------------------------------------------------------------
// LDS of the resident kernel (dynamic; carved in this order)
// ------------------------------------------------------------------------------------------
struct Smem {
  bf16x8* wl;        // [4 tiles][KSTEPS][64]: W tiles of the workgroup's LDS chunks (MFMA A operands)
  bf16x8* sA;        // [2][KSTEPS][64]: B operands (gathered A rows) of the current / next sub-block
  ReqMeta* req;      // [B]
  uint8_t* role;     // [B] roles of the step
  uint8_t* Lq;       // [B] verify lengths
  uint16_t* slot;    // [3][B]: DRAFT bias slot, CORRECT bias slot, plain slot (0xFFFF = none)
  uint32_t* blist;   // [max bias slots]: entries (ent_make), NO_ENT in gaps
  uint16_t* plist;   // [B]
  int4* wcnt;        // [NW] per-wave row counts of a list-building round
};

__host__ __device__ inline size_t smem_bytes(int B) {
  size_t o = 0;
  o += (size_t)4 * KSTEPS * 64 * 16;                 // wl
  o += (size_t)2 * KSTEPS * 64 * 16;                 // sA
  o += (size_t)B * sizeof(ReqMeta);                  // req
  o += (size_t)B * 2;                                // role, Lq
  o += (size_t)3 * B * 2;                            // slot
  o += (size_t)max_bias_slots(B) * 4 + (size_t)B * 2; // blist, plist
  o = (o + 15) & ~(size_t)15;
  o += NW * 16;                                      // wcnt
  return o;
}

__device__ inline Smem carve(char* base, int B) {
  Smem m;
  char* p = base;
  m.wl = (bf16x8*)p; p += (size_t)4 * KSTEPS * 64 * 16;
  m.sA = (bf16x8*)p; p += (size_t)2 * KSTEPS * 64 * 16;
  m.req = (ReqMeta*)p; p += (size_t)B * sizeof(ReqMeta);
  m.role = (uint8_t*)p; p += B;
  m.Lq = (uint8_t*)p; p += B;
  m.slot = (uint16_t*)p; p += (size_t)3 * B * 2;
  m.blist = (uint32_t*)p; p += (size_t)max_bias_slots(B) * 4;
  m.plist = (uint16_t*)p; p += (size_t)B * 2;
  p = (char*)(((uintptr_t)p + 15) & ~(uintptr_t)15);
  m.wcnt = (int4*)p;
  return m;
}

// ------------------------------------------------------------------------------------------
// kernel parameters (device view of the workspace)
// ------------------------------------------------------------------------------------------
struct KP {
  Args a;
  int32_t* st;        // [6][B]
  int32_t* xs;        // [B][K]
  float* lse_q;       // [B][K]
  float* logq;        // [B][K]
  float* lse_p;       // [B][K+1]
  float* logp;        // [B][K]
  float4* rec_d;      // [slots][NW][MAX_G]: per-wave records of bias rows
  float4* rec_c;      // [CORRECT slot - c0][NW][MAX_G]: CORRECT rows' target-row records
  float4* rec_p;      // [B][MAX_G]: records of the plain rows' items (ceil(V / TP) <= MAX_G per row)
  uint64_t* flags;    // [G][FLAG_STRIDE]
  uint64_t* err;
  uint64_t* pub;      // [2][B][PUB_WORDS]: per-request words of the next step (see publish)
};

// What the merge of request b at step s hands to the lists of step s + 1, as three 64-bit words
// whose high halves hold the tag s + 1 and whose low halves hold (roles of step s + 1) << 28 |
// (token drafted at s) + 1, the draft row's log-normaliser at s, and the target row's (the last two
// matter only to a CORRECT row of step s + 1, which needs both).  Each word is stored and loaded
// whole (agent-scope 64-bit atomics), so a reader that finds tag s + 1 in a word holds that word's
// value of step s; the lists poll the words of every request until all carry the step's tag, which
// also orders the step: a merge publishes only after it has read its records, so no workgroup
// overwrites records that a merge still reads.  Words of both step parities are cleared (tag 0) at
// set-up, before the first grid barrier, so words of an earlier call never carry a live tag, and a
// parity's word of step s - 2 carries tag s - 1.  Tokens fit the 28 bits (V < 2^26: A below 2 GiB).
__device__ __forceinline__ uint64_t* pub_of(const KP& p, int parity, int b) {
  return p.pub + ((size_t)parity * p.a.B + b) * PUB_WORDS;
}
__device__ __forceinline__ void publish(const KP& p, int s, int b, int roles, int x, float lse_q, float lse_p) {
  uint64_t* w = pub_of(p, (s + 1) & 1, b);
  const uint64_t tag = (uint64_t)(uint32_t)(s + 1) << 32;
  st_u64(&w[0], tag | ((uint32_t)roles << 28) | (uint32_t)(x + 1));
  st_u64(&w[1], tag | __float_as_uint(lse_q));
  st_u64(&w[2], tag | __float_as_uint(lse_p));
}

// W fragment f (tile f of a chunk: 32 columns) at k-step t for lane l: row i = l % 32 of the MFMA
// A operand is column 64 c + 32 f + perm(i), perm chosen so that accumulator q of lane l holds
// column 64 c + 32 f + 16 (l / 32) + q; lane half l / 32 covers k in [R/2 (l/32), R/2 (l/32 + 1)).
// Columns past V and k-steps past the rank read zeros.
__device__ __forceinline__ bf16x8 w_frag(const KP& p, int c, int f, int t) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
  const int R = p.a.R;
  const int col_in = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int v = CH * c + 32 * f + col_in;
  const bool in = c >= 0 && v < p.a.V && t < (R >> 4);
  // out of range: read row 0 and zero the value (no branch around the load)
  const u32x4 x = *(const u32x4*)((const uint16_t*)p.a.W + (in ? (size_t)v * R + h * (R >> 1) + 8 * t : 0));
  const u32x4 z = in ? x : (u32x4){0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// ------------------------------------------------------------------------------------------
// merge of one request by one wave
// ------------------------------------------------------------------------------------------
// running reduction of records {log-mass, best score, best chunk}: the mass kept as m + log(s)
struct PAcc {
  float m, s, sc;
  int ix, nan;
};

// a lane's running record of N records at once: the largest log-mass first, then N independent
// exponentials (a NaN log-mass marks the record NaN)
template <int N>
__device__ __forceinline__ void pacc_of(PAcc& a, const float4 (&r)[N]) {
  float m = r[0].x;
#pragma unroll
  for (int i = 1; i < N; i++) m = vmax(m, r[i].x);
  a.nan = m != m;
  a.m = a.nan ? -INFINITY : m;
  a.s = 0.0f;
  if (a.m > -INFINITY) {
#pragma unroll
    for (int i = 0; i < N; i++) a.s += ex2((r[i].x - a.m) * LOG2E);
  }
  a.sc = -INFINITY;
  a.ix = -1;
#pragma unroll
  for (int i = 0; i < N; i++) {
    const int ix = __float_as_int(r[i].z);
    if (takes(r[i].y, ix, a.sc, a.ix)) {
      a.sc = r[i].y;
      a.ix = ix;
    }
  }
}

enum { L2_NONE = 0, L2_DRAFT = 1, L2_TARGET = 2, L2_RESIDUAL = 3 };

struct Job {
  int kind;              // L2_*
  int chunk;             // winning chunk of level one
  int prev;              // previous token of the Markov bias, -1 = none
  uint64_t key;          // per-index noise key of the row
  const uint16_t* base;  // draft row
  const uint16_t* targ;  // target row
  float lse_p, lse_q;
  bool want_target;      // DRAFT: also return the target logit of the winner
};

struct L2Out {
  int v;      // winning column, -1 = none
  float sx;   // DRAFT: scaled draft logit of the winner
  float tx;   // target logit (unscaled) of the winner, when asked for
};

// LDS scratch of the merge phase (it lives in the B-operand buffers, idle between the barriers)
struct MergeLds {
  uint16_t arow[2][256];   // A rows of the two level-two jobs
  float4 part[4][NT];      // per-workgroup records of the request's four row kinds (thread t: workgroup t)
  float4 rec[4][NW];       // the four kinds' totals (entry [r][0])
  float4 win[2][NW];       // per-wave level-two winners {score, index, scaled draft logit, target logit}
};

// Level two of the chunked sampler for two jobs at once by the whole workgroup, the 256-rank dot
// products on the matrix cores: waves 2q and 2q + 1 take job q, lane l its columns
// 64 chunk + 32 (w & 1) + l % 32.  Each 16 ranks are one v_mfma_f32_32x32x16_bf16 whose first
// operand is the job's A row on all 32 rows and whose second is the 32 columns' W rows, so every
// row of the product is the columns' bias and each lane holds its column's bias in every
// accumulator (two chains over alternate k-steps).  Lane half h feeds ranks 16 t + 8 h .. + 7 of
// k-step t.  The lower half's lanes score their columns, the winner is found per wave, then per
// job.  Result uniform.
template <class Between>
__device__ __forceinline__ void level_two(const KP& p, const Job (&jb)[2], float invT, MergeLds* ml, L2Out (&out)[2],
                                          Between&& between) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int V = p.a.V, R = p.a.R;
  const int qj = wave >> 1, hk = lane >> 5;
  // this wave's job, field by field (a select of whole structs goes through scratch memory)
  const bool j1 = qj != 0;
  const int kind = j1 ? jb[1].kind : jb[0].kind;
  const int chunk = j1 ? jb[1].chunk : jb[0].chunk;
  const int prev = j1 ? jb[1].prev : jb[0].prev;
  const uint64_t key = j1 ? jb[1].key : jb[0].key;
  const uint16_t* base = j1 ? jb[1].base : jb[0].base;
  const uint16_t* targ = j1 ? jb[1].targ : jb[0].targ;
  const float lse_p = j1 ? jb[1].lse_p : jb[0].lse_p, lse_q = j1 ? jb[1].lse_q : jb[0].lse_q;
  const bool want_target = j1 ? jb[1].want_target : jb[0].want_target;
  const int v = chunk * CH + 32 * (wave & 1) + (lane & 31);
  // (a chunk index past the vocabulary comes only from records a timed-out wait left incomplete)
  const bool in = kind != L2_NONE && chunk >= 0 && chunk < n_chunks(V) && v < V;
  const bool need_base = in && (kind == L2_DRAFT || kind == L2_RESIDUAL);
  const bool need_targ = in && (kind != L2_DRAFT || want_target);
  const bool need_bias = in && kind != L2_TARGET && prev >= 0;
  // every global load is issued before any is waited for: the W rows (buffer loads; k-steps past
  // the rank and columns without a bias read past the end of W: zeros) and the two logits of the
  // column; the A row's pieces come from LDS at the products (entries past R are zeros there)
  const __amdgpu_buffer_rsrc_t rsW = ld_rsrc(p.a.W, (uint32_t)V * (uint32_t)R * 2u);
  const int KS = R >> 4;
  u32x4 wv[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; t++) {
    const uint32_t vo = (need_bias && t < KS) ? 2u * (uint32_t)(v * R + 16 * t + 8 * hk) : OOB_OFF;
    wv[t] = ldb16(rsW, vo, 0u);
  }
  const uint16_t bvr = *(need_base ? base + v : (const uint16_t*)p.a.base);
  const uint16_t tvr = *(need_targ ? targ + v : (const uint16_t*)p.a.target);
  __builtin_amdgcn_sched_barrier(0);   // every load is in flight before any is used
  const float gg = gumbel_bf(bits_at(key, (uint32_t)v));   // the column's noise meanwhile
  __builtin_amdgcn_sched_barrier(0);
  between();   // the caller's work that needs none of these loads
  __builtin_amdgcn_sched_barrier(0);
  f32x16 c0 = {}, c1 = {};
#pragma unroll
  for (int t = 0; t < KSTEPS; t += 2) {
    const u32x4 a0 = *(const u32x4*)&ml->arow[qj][16 * t + 8 * hk];
    const u32x4 a1 = *(const u32x4*)&ml->arow[qj][16 * t + 16 + 8 * hk];
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, wv[t]), c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, wv[t + 1]), c1, 0, 0, 0);
  }
  const float bias = c0[0] + c1[0];
  const float bv = need_base ? bf16_to_f32(bvr) : 0.0f, tv = need_targ ? bf16_to_f32(tvr) : 0.0f;
  float sc = -INFINITY, sx = 0.0f, tx = 0.0f;
  int ix = -1;
  if (in && hk == 0) {
    if (kind == L2_DRAFT) {
      const float sv = (bv + bias) * invT;
      if (want_target) tx = tv;
      if (sv > -INFINITY) {
        sc = sv + gg;
        ix = v;
        sx = sv;
      }
    } else if (kind == L2_TARGET) {
      const float t = tv * invT;
      if (t > -INFINITY) {
        sc = t + gg;
        ix = v;
      }
    } else {
      const float sv = (bv + bias) * invT, t = tv * invT;
      const float lp = t - lse_p, lq = sv - lse_q;
      if (lp > lq) {
        sc = lp + logf(-expm1f(lq - lp)) + gg;
        ix = v;
      }
    }
  }
  // the winner's target logit rides along: the winning lane is found by ballot after the argmax
  const int ix0 = ix;
  const float tx0 = tx;
  wargmax(sc, ix, sx);
  const unsigned long long wm = __ballot(ix >= 0 && ix0 == ix);
  const int src = __builtin_amdgcn_readfirstlane(wm ? __ffsll(wm) - 1 : 0);
  tx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tx0), src));
  if (lane == 0) ml->win[qj][wave & 1] = make_float4(sc, __int_as_float(ix), sx, tx);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; q++) {
    float4 bw = ml->win[q][0];
    const float4 c = ml->win[q][1];
    if (takes(c.x, __float_as_int(c.y), bw.x, __float_as_int(bw.y))) bw = c;
    out[q].v = __float_as_int(bw.y);
    out[q].sx = bw.z;
    out[q].tx = bw.w;
  }
}

// The four wave records of one workgroup (cb: its first chunk, nl: its LDS chunks) for one bias
// row, combined into that workgroup's {log-mass, best chunk score, best chunk}.  A wave record
// holds the log-mass of the wave's register chunks, their best score and chunk, and the log-mass
// of the wave's half of an LDS chunk; the halves of LDS chunk i are in waves 2i and 2i + 1, and
// the chunk's Gumbel score is formed here from the whole chunk.
// log-sum-exp of N terms with the largest subtracted first: N independent exponentials and one
// logarithm (a chain of pairwise log-additions costs one exponential and one logarithm per term
// in sequence).  -inf terms add nothing; a NaN term makes the result NaN (v_maximum propagates it).
template <int N>
__device__ __forceinline__ float lse_of(const float (&x)[N]) {
  float M = x[0];
#pragma unroll
  for (int i = 1; i < N; i++) M = vmax(M, x[i]);
  if (M == -INFINITY) return -INFINITY;
  float S = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i++) S += ex2((x[i] - M) * LOG2E);
  return M + lg2(S) * LN2;
}

__device__ __forceinline__ float4 wg_draft(const float4 (&a)[NW], int cb, int nl, const float (&gl)[LDS_CHUNKS]) {
  float bs = -INFINITY;
  int bc = -1;
  // the log-mass over the register chunks' wave sums and the LDS chunks' halves
  float x[NW + 2 * LDS_CHUNKS];
#pragma unroll
  for (int w = 0; w < NW; w++) {
    x[w] = a[w].x;
    if (takes(a[w].y, __float_as_int(a[w].z), bs, bc)) {
      bs = a[w].y;
      bc = __float_as_int(a[w].z);
    }
  }
  // constant indices (the bound is the largest LDS chunk count) keep the records in registers
#pragma unroll
  for (int i = 0; i < LDS_CHUNKS; i++) {
    x[NW + 2 * i] = i < nl ? a[2 * i].w : -INFINITY;
    x[NW + 2 * i + 1] = i < nl ? a[2 * i + 1].w : -INFINITY;
  }
  const float lse = lse_of(x);
#pragma unroll
  for (int i = 0; i < LDS_CHUNKS; i++) {
    const float hc = i < nl ? lse2(a[2 * i].w, a[2 * i + 1].w) : -INFINITY;
    const int cgl = cb + NW * AG_CHUNKS + i;
    const float sc = hc > -INFINITY ? hc + gl[i] : -INFINITY;
    if (hc > -INFINITY && takes(sc, cgl, bs, bc)) {
      bs = sc;
      bc = cgl;
    }
  }
  return make_float4(lse, bs, __int_as_float(bc), 0.0f);
}

// The same for a CORRECT row: the residual records a (log residual mass of the register chunks,
// best score, best chunk, LINEAR residual mass of the LDS half) and the target records t (target
// log-mass, best score, best chunk, target log-mass of the LDS half); both draws use `key`.
__device__ __forceinline__ void wg_correct(const float4 (&a)[NW], const float4 (&t)[NW], int cb, int nl,
                                           const float (&gl)[LDS_CHUNKS], float4& rd, float4& rt) {
  float ms = 0.0f, bs = -INFINITY, bt = -INFINITY;
  int bc = -1, btc = -1;
  float x[NW + 2 * LDS_CHUNKS];
#pragma unroll
  for (int w = 0; w < NW; w++) {
    ms += a[w].x > -INFINITY ? ex2(a[w].x * LOG2E) : 0.0f;
    if (takes(a[w].y, __float_as_int(a[w].z), bs, bc)) {
      bs = a[w].y;
      bc = __float_as_int(a[w].z);
    }
    x[w] = t[w].x;
    if (takes(t[w].y, __float_as_int(t[w].z), bt, btc)) {
      bt = t[w].y;
      btc = __float_as_int(t[w].z);
    }
  }
#pragma unroll
  for (int i = 0; i < LDS_CHUNKS; i++) {
    x[NW + 2 * i] = i < nl ? t[2 * i].w : -INFINITY;
    x[NW + 2 * i + 1] = i < nl ? t[2 * i + 1].w : -INFINITY;
  }
  const float lt = lse_of(x);
#pragma unroll
  for (int i = 0; i < LDS_CHUNKS; i++) {
    const int cgl = cb + NW * AG_CHUNKS + i;
    const float gg = gl[i];
    const float mc = i < nl ? a[2 * i].w + a[2 * i + 1].w : 0.0f;
    ms += mc;
    const float lmc = mc > 0.0f ? lg2(mc) * LN2 : -INFINITY;
    if (lmc > -INFINITY && takes(lmc + gg, cgl, bs, bc)) {
      bs = lmc + gg;
      bc = cgl;
    }
    const float tc = i < nl ? lse2(t[2 * i].w, t[2 * i + 1].w) : -INFINITY;
    if (tc > -INFINITY && takes(tc + gg, cgl, bt, btc)) {
      bt = tc + gg;
      btc = cgl;
    }
  }
  rd = make_float4(ms > 0.0f ? lg2(ms) * LN2 : -INFINITY, bs, __int_as_float(bc), 0.0f);
  rt = make_float4(lt, bt, __int_as_float(btc), 0.0f);
}

// Request b at step s, by the whole workgroup: reduce its rows' records, level two, accept
// decision, outputs, roles of step s + 1.  The request's state is touched by this workgroup only.
__device__ void merge_request(const KP& p, const Smem& S, int b, int s, int c0) {
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int B = p.a.B, K = p.a.K, V = p.a.V, G = p.a.G;
  MergeLds* ml = (MergeLds*)S.sA;
  const int roles = S.role[b];
  __syncthreads();   // the scratch of the previous request's merge is no longer read
  if (roles == 0) {
    if (tid == 0) publish(p, s, b, 0, -1, 0.0f, 0.0f);
    return;
  }
  const ReqMeta rm = S.req[b];
  const float invT = rm.invT;
  const int L = S.Lq[b];
  int phase = p.st[ST_PHASE * B + b];
  int acc = p.st[ST_ACC * B + b];
  const uint64_t kreq = req_key(p.a.seed, p.a.req_off + b);
  const bool hasD = roles & RO_DRAFT, hasC = roles & RO_CORRECT, hasP = roles & (RO_LSEP | RO_BONUS);
  const int sd = S.slot[b], sc_ = S.slot[B + b], sp = S.slot[2 * B + b];
  const int x_t = tid < K ? p.xs[(size_t)b * K + tid] : -1;   // drafted tokens, for the output
  // ---- records of every row of the request: thread t combines workgroup t's wave records of
  //      each row kind (G <= NT) and takes plain item t (ceil(V / TP) <= NT); the combined records
  //      go to LDS, where wave r reduces kind r (DRAFT, CORRECT residual, CORRECT target, plain) ----
  // A rows of the two level-two jobs (DRAFT: the token before position s; CORRECT: the token before
  // s - 1), loaded now so that their latency hides behind the records'; thread t < 128 takes four
  // entries of job t / 64 (a job without a previous token reads past the end of A: zeros)
  uint2 arow_v;
  {
    const int qa = (tid >> 6) & 1, la = tid & 63;
    const int prev = qa == 0 ? (hasD ? rm.prev_d : -1) : (hasC ? rm.prev_c : -1);
    const __amdgpu_buffer_rsrc_t rsA = ld_rsrc(p.a.A, (uint32_t)V * (uint32_t)p.a.R * 2u);
    const bool in = tid < 128 && prev >= 0 && 4 * la < p.a.R;
    const uint32_t vo = in ? 2u * (uint32_t)(prev * p.a.R + 4 * la) : OOB_OFF;
    arow_v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsA, (int)vo, 0, 0));
  }
  // wave r's running record of row kind r (DRAFT, CORRECT residual, CORRECT target, plain)
  const bool kind_on = wave == 0 ? hasD : (wave == 3 ? hasP : hasC);   // wave-uniform
  PAcc pa;
  pa.m = -INFINITY;
  pa.s = 0.0f;
  pa.sc = -INFINITY;
  pa.ix = -1;
  pa.nan = 0;
  uint64_t key_l2d, key_l2r, key_l2b, key_acc;   // per-index noise keys of the level-two rows and the accept draw
  {
    const uint64_t key_d = key_of(rm.key_d), key_c = key_of(rm.key_c);
    const int nrP = (V + TP - 1) / TP;
    const int gi = tid < G ? tid : 0;
    const int cb = chunk_begin(gi, G, V), ncw = chunks_of(gi, G, V);
    const int nl = ncw > NW * AG_CHUNKS ? ncw - NW * AG_CHUNKS : 0;
    const float4 none = make_float4(-INFINITY, -INFINITY, __int_as_float(-1), 0.0f);
    // every load of the request's records is issued before any is used (a kind the request does
    // not have reads row 0 and is ignored)
    const auto rs_d = rec_rsrc(p.rec_d, rec_d_bytes(B)), rs_p = rec_rsrc(p.rec_p, rec_p_bytes(B)),
               rs_c = rec_rsrc(p.rec_c, rec_c_bytes(B));
    const size_t rd_base = (size_t)(hasD ? sd : 0) * NW * MAX_G + gi;
    // (a request without a CORRECT row reads past the record areas: zeros, no memory access)
    const size_t REC_PAST = (size_t)1 << 26;
    const size_t rc_base = hasC ? (size_t)sc_ * NW * MAX_G + gi : REC_PAST;
    const size_t rt_base = hasC ? (size_t)(sc_ - c0) * NW * MAX_G + gi : REC_PAST;
    float4 ad[NW], ac[NW], at[NW];
#pragma unroll
    for (int w = 0; w < NW; w++) ad[w] = rec_load(rs_d, rd_base + (size_t)w * MAX_G);
    const float4 ap = rec_load(rs_p, (size_t)(hasP ? sp : 0) * MAX_G + (tid < nrP ? tid : 0));
#pragma unroll
    for (int w = 0; w < NW; w++) {
      ac[w] = rec_load(rs_d, rc_base + (size_t)w * MAX_G);
      at[w] = rec_load(rs_c, rt_base + (size_t)w * MAX_G);
    }
    key_l2d = pos_key(kreq, s, ST_DRAFT);
    key_l2r = pos_key(kreq, s > 0 ? s - 1 : 0, ST_RESIDUAL);
    key_l2b = pos_key(kreq, s, ST_BONUS);
    key_acc = pos_key(kreq, s, ST_ACCEPT);
    // the Gumbel noise of workgroup gi's LDS chunks for both row kinds, while the loads are in flight
    float gld[LDS_CHUNKS], glc[LDS_CHUNKS];
#pragma unroll
    for (int i = 0; i < LDS_CHUNKS; i++) {
      const uint32_t cgl = (uint32_t)(cb + NW * AG_CHUNKS + i);
      gld[i] = gumbel_bf(bits_at(key_d, cgl));
      glc[i] = gumbel_bf(bits_at(key_c, cgl));
    }
    __builtin_amdgcn_sched_barrier(0);   // the loads are in flight before any is used
    // (component-wise selects: a select of whole structs goes through scratch memory)
    auto sel4 = [](bool c, float4 a, float4 b) {
      return make_float4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
    };
    // the A rows of the level-two jobs into LDS (read there after the barriers below; a job without a
    // previous token, or rank entries past R, hold zeros, and a job without a bias multiplies zero W)
    if (tid < 128) *(uint2*)&ml->arow[(tid >> 6) & 1][4 * (tid & 63)] = arow_v;
    ml->part[0][tid] = sel4(hasD && tid < G, wg_draft(ad, cb, nl, gld), none);
    ml->part[3][tid] = sel4(hasP && tid < nrP, ap, none);
    if (hasC) {
      float4 rd = none, rt = none;
      if (tid < G) wg_correct(ac, at, cb, nl, glc, rd, rt);
      ml->part[1][tid] = rd;
      ml->part[2][tid] = rt;
    }
    __syncthreads();
    // wave r reduces row kind r: the winning chunk first (level two's loads need only that), the
    // log-mass while those loads are in flight (below)
    if (kind_on) {
      float4 r4[NT / 64];
#pragma unroll
      for (int i = 0; i < NT / 64; i++) r4[i] = ml->part[wave][64 * i + lane];
      pacc_of(pa, r4);
      float aux = 0.0f;
      wargmax(pa.sc, pa.ix, aux);
      if (lane == 0) ml->rec[wave][1] = make_float4(pa.sc, __int_as_float(pa.ix), 0.0f, 0.0f);
    } else if (lane == 0) {
      ml->rec[wave][1] = make_float4(-INFINITY, __int_as_float(-1), 0.0f, 0.0f);
    }
  }
  __syncthreads();
  int cz[4];   // each row kind's winning chunk (-1: none)
#pragma unroll
  for (int r = 0; r < 4; r++) cz[r] = __float_as_int(ml->rec[r][1].y);

  // ---- level two: the DRAFT row and the CORRECT / BONUS row side by side ----
  // A row kind has a winning chunk exactly when its log-mass is above -inf (a chunk competes only
  // with a positive mass); where the log-mass is not finite the decision below marks the request
  // invalid whatever level two drew.
  const int j_c = s - 1;
  const bool residual = cz[1] >= 0;
  const uint16_t* targ_s = (const uint16_t*)p.a.target + ((size_t)b * (K + 1) + s) * V;
  Job jb[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    jb[q].kind = L2_NONE;
    jb[q].chunk = -1;
    jb[q].prev = -1;
    jb[q].key = 0;
    jb[q].base = nullptr;
    jb[q].targ = nullptr;
    jb[q].lse_p = 0.0f;
    jb[q].lse_q = 0.0f;
    jb[q].want_target = false;
  }
  if (hasD && cz[0] >= 0) {
    jb[0].kind = L2_DRAFT;
    jb[0].chunk = cz[0];
    jb[0].prev = rm.prev_d;
    jb[0].key = key_l2d;
    jb[0].base = (const uint16_t*)p.a.base + ((size_t)b * K + s) * V;
    jb[0].targ = targ_s;
    jb[0].want_target = (roles & RO_LSEP) != 0;
  }
  if (hasC) {
    jb[1].chunk = residual ? cz[1] : cz[2];
    jb[1].key = key_l2r;
    jb[1].targ = (const uint16_t*)p.a.target + ((size_t)b * (K + 1) + j_c) * V;
    if (residual) {
      jb[1].kind = L2_RESIDUAL;
      jb[1].prev = rm.prev_c;
      jb[1].base = (const uint16_t*)p.a.base + ((size_t)b * K + j_c) * V;
      jb[1].lse_p = rm.lse_p_c;
      jb[1].lse_q = rm.lse_q_c;
    } else {
      jb[1].kind = L2_TARGET;
    }
  } else if ((roles & RO_BONUS) && cz[3] >= 0) {
    jb[1].kind = L2_TARGET;
    jb[1].chunk = cz[3];
    jb[1].key = key_l2b;
    jb[1].targ = targ_s;
  }
  L2Out r2[2];
  level_two(p, jb, invT, ml, r2, [&]() {
    // wave r's row-kind log-mass (read after level two's last barrier)
    if (kind_on) {
      const float M = wmax(pa.m);
      const float sl = (pa.m == -INFINITY) ? 0.0f : pa.s * ex2((pa.m - M) * LOG2E);
      const float S_ = wsum(sl);
      const int nan = __ballot(pa.nan != 0) != 0ull;
      const float lse = nan ? NAN : (M == -INFINITY ? -INFINITY : M + lg2(S_) * LN2);
      if (lane == 0) ml->rec[wave][0] = make_float4(lse, pa.sc, __int_as_float(pa.ix), 0.0f);
    } else if (lane == 0) {
      ml->rec[wave][0] = make_float4(-INFINITY, -INFINITY, __int_as_float(-1), 0.0f);
    }
  });
  const L2Out rd = r2[0], rf = r2[1];
  float4 tot[4];
#pragma unroll
  for (int r = 0; r < 4; r++) tot[r] = ml->rec[r][0];
  const float4 tot_d = tot[0], tot_c = tot[1], tot_p = tot[3];

  // ---- decision and outputs (uniform over the workgroup; thread 0 writes scalars) ----
  bool invalid = false, rejected_now = false;
  int final_tok = -1, x_s = -1;
  float logq_s = NAN, pub_q = 0.0f, pub_p = 0.0f;
  if (hasD) {
    const float lse_q = tot_d.x;
    pub_q = lse_q;
    if (!isfinite(lse_q) || rd.v < 0) {
      invalid = true;
    } else {
      x_s = rd.v;
      logq_s = rd.sx - lse_q;
      if (tid == 0) {
        st_i32(&p.xs[(size_t)b * K + s], x_s);
        if (p.a.d_draft) p.a.d_draft[(size_t)b * K + s] = x_s;
        if (p.a.d_logq) p.a.d_logq[(size_t)b * K + s] = logq_s;
      }
    }
  }
  if (!invalid && (roles & RO_LSEP)) {
    const float lse_p = tot_p.x;
    pub_p = lse_p;
    if (!isfinite(lse_p) || x_s < 0) {
      invalid = true;
    } else {
      const float logp_s = rd.tx * invT - lse_p;
      // accept when u = (ub + 1/2) 2^-32 < p / q = exp(logp - logq): the ratio in fp32 (its relative
      // error, about 1e-7, is below that of the fp32 log-probabilities it comes from), compared
      // exactly with u in fp64 as (ub + 1/2) < ratio 2^32
      const uint32_t ub = bits_at(key_acc, 0);
      const float ratio32 = __builtin_amdgcn_ldexpf(ex2((logp_s - logq_s) * LOG2E), 32);
      if ((double)ub + 0.5 < (double)ratio32) {
        acc = s + 1;
      } else {
        phase = PH_REJECTED;
        rejected_now = true;
      }
      if (tid == 0 && p.a.d_logp) p.a.d_logp[(size_t)b * K + s] = logp_s;
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
  if (invalid) {
    if (tid <= K) p.a.tokens[(size_t)b * (K + 1) + tid] = -1;
    if (tid < K) {
      if (p.a.d_draft) p.a.d_draft[(size_t)b * K + tid] = -1;
      if (p.a.d_logq) p.a.d_logq[(size_t)b * K + tid] = NAN;
      if (p.a.d_logp) p.a.d_logp[(size_t)b * K + tid] = NAN;
    }
    if (tid == 0) {
      p.a.accepted_len[b] = -1;
      if (p.a.d_verify_len) p.a.d_verify_len[b] = -1;
      p.st[ST_PHASE * B + b] = PH_INVALID;
      p.st[ST_ACC * B + b] = acc;
      publish(p, s, b, 0, -1, 0.0f, 0.0f);
    }
    return;
  }
  if (final_tok >= 0) {
    phase = PH_DONE;
    if (tid < acc) p.a.tokens[(size_t)b * (K + 1) + tid] = x_t;   // tid < acc <= s: drafted before this step
    if (tid == acc) p.a.tokens[(size_t)b * (K + 1) + tid] = final_tok;
    if (tid == 0) p.a.accepted_len[b] = acc;
  }
  if (tid == 0) {
    int nr = 0;
    if (s + 1 < L) nr |= RO_DRAFT;
    if (phase == PH_ALIVE && acc == s + 1) nr |= (s + 1 < L) ? RO_LSEP : RO_BONUS;
    if (rejected_now) nr |= RO_CORRECT;
    p.st[ST_PHASE * B + b] = phase;
    p.st[ST_ACC * B + b] = acc;
    publish(p, s, b, nr, x_s, pub_q, pub_p);
  }
}

// ------------------------------------------------------------------------------------------
// the kernel
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(NT, 1) void k_resident(KP p) {
  extern __shared__ __align__(16) char smem_raw[];
  const int B = p.a.B, K = p.a.K, V = p.a.V, G = p.a.G;
  Smem S = carve(smem_raw, B);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = blockIdx.x;
  const int cbeg = chunk_begin(g, G, V), nch = chunks_of(g, G, V);
  const int n_lds = nch > NW * AG_CHUNKS ? nch - NW * AG_CHUNKS : 0;   // 0..2 LDS chunks

  // ---- W slice on chip: this wave's two register chunks, and the workgroup's LDS tiles ----
  bf16x8 wf[4][KSTEPS];   // [tile: chunk 2 wave + tile / 2, half tile % 2][k-step]
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int cl = AG_CHUNKS * wave + (i >> 1);
    const int c = cl < nch ? cbeg + cl : -1;
#pragma unroll
    for (int t = 0; t < KSTEPS; t++) wf[i][t] = w_frag(p, c, i & 1, t);
  }
  // LDS tile u = 2 (local chunk - 8) + half, processed by wave u: all of a thread's loads issued
  // before any is stored (out of range: read row 0 and store zeros)
  {
    constexpr int NE = 4 * KSTEPS * 64 / NT;
    u32x4 z[NE];
#pragma unroll
    for (int q = 0; q < NE; q++) {
      const int e = (int)threadIdx.x + NT * q;
      const int u = e / (KSTEPS * 64), t = (e / 64) % KSTEPS, l = e % 64;
      const int cl = NW * AG_CHUNKS + (u >> 1);
      const int c = cl < nch ? cbeg + cl : -1;
      // the fragment of lane l: same mapping as w_frag, computed for lane l
      const int mm = l & 31, hh = l >> 5;
      const int col_in = 16 * ((mm >> 2) & 1) + 4 * (mm >> 3) + (mm & 3);
      const int v = CH * c + 32 * (u & 1) + col_in;
      const bool in = c >= 0 && v < V && t < (p.a.R >> 4);
      const u32x4 x = *(const u32x4*)((const uint16_t*)p.a.W + (in ? (size_t)v * p.a.R + hh * (p.a.R >> 1) + 8 * t : 0));
      z[q] = in ? x : kZero;
    }
#pragma unroll
    for (int q = 0; q < NE; q++) ((u32x4*)S.wl)[threadIdx.x + NT * q] = z[q];
  }

  // ---- set-up: verify lengths and validity of every request (every workgroup, redundantly);
  // the merge wave of a request initialises its outputs ----
  const uint64_t seed = p.a.seed;
  for (int b = threadIdx.x; b < B; b += NT) {
    const float T = p.a.temp[b];
    const int x0 = p.a.x0 ? p.a.x0[b] : -1;
    bool valid = (T > 0.0f) && isfinite(T) && x0 >= -1 && x0 < V;
    int L = 0;
    if (p.a.L_in) {
      L = p.a.L_in[b];
      if (L < 0 || L > K) {
        valid = false;
        L = 0;
      }
    } else {
      // the running fp64 product of the confidences, stopping at the first that falls below the
      // threshold; every confidence of the request is loaded first (one round trip)
      float cf[MAX_K];
#pragma unroll
      for (int j = 0; j < MAX_K; j++) cf[j] = j < K ? p.a.conf[(size_t)b * K + j] : 0.0f;
      double P = 1.0;
      bool run = true;
#pragma unroll
      for (int j = 0; j < MAX_K; j++) {
        if (j < K && run) {
          P *= (double)cf[j];
          run = P >= (double)p.a.threshold;
          L = run ? j + 1 : L;
        }
      }
    }
    S.Lq[b] = (uint8_t)L;
    S.role[b] = valid ? (uint8_t)(L > 0 ? (RO_DRAFT | RO_LSEP) : RO_BONUS) : (uint8_t)0;
    // the request's table entries that every step keeps: 1/T, the request's noise key, and x0 as
    // the token before position 0 (used only while the request is valid)
    S.req[b].invT = 1.0f / T;
    S.req[b].prev_d = x0;
    put_key(S.req[b].key_r, req_key(seed, p.a.req_off + b));
  }
  __syncthreads();
  // outputs and state of the requests this workgroup merges (request b: workgroup b % G, wave b / G)
  for (int i = threadIdx.x; i < NW * (K + 1); i += NT) {
    const int w = i / (K + 1), j = i % (K + 1);
    const int b = g + G * w;
    if (b >= B) continue;
    p.a.tokens[(size_t)b * (K + 1) + j] = -1;
    if (j < K) {
      if (p.a.d_draft) p.a.d_draft[(size_t)b * K + j] = -1;
      if (p.a.d_logq) p.a.d_logq[(size_t)b * K + j] = NAN;
      if (p.a.d_logp) p.a.d_logp[(size_t)b * K + j] = NAN;
    }
    if (j == 0) {
      const bool valid = S.role[b] != 0;
      p.a.accepted_len[b] = -1;
      if (p.a.d_verify_len) p.a.d_verify_len[b] = valid ? (int)S.Lq[b] : -1;
      p.st[ST_ACC * B + b] = 0;
      p.st[ST_PHASE * B + b] = valid ? PH_ALIVE : PH_INVALID;
    }
  }
  // their published words of both step parities: tag 0 (see publish)
  for (int i = threadIdx.x; i < NW * 2 * PUB_WORDS; i += NT) {
    const int b = g + G * (i / (2 * PUB_WORDS)), j = i % (2 * PUB_WORDS);
    if (b < B) st_u64(&pub_of(p, j / PUB_WORDS, b)[j % PUB_WORDS], 0ull);
  }

  uint64_t token = p.a.nonce;
  for (int s = 0; s <= K; s++) {
    // lane-derived values are redefined opaquely at every step, so that addresses built from them
    // are computed where they are used instead of being kept in registers across the whole loop
    int tid = opaque_tid();
#define lane (tid & 63)
#define m32 (tid & 31)
#define h ((tid >> 5) & 1)
    // ---- 1. roles of step s -> lists and the per-request table ----
    Lists ls;
    {
      // requests in rounds of NT (request i NT + tid in round i); within a round every wave counts
      // its rows with ballots, the waves' counts are combined in LDS; slots follow the order
      // (round, wave, lane).  CORRECT slots are taken relative first and moved behind the DRAFT
      // rows once their number is known.
      int nd = 0, nc = 0, np = 0;
      const int rounds = (B + NT - 1) / NT;
      for (int i = 0; i < rounds; i++) {
        const int b = i * NT + tid;
        // the request's role and its table row: at s = 0 the set-up's roles; after that the words
        // published by the request's merge of step s - 1, polled until all three carry tag s (a
        // request without a role does not use the rest)
        int r = 0, xd = -1, xc = -1;
        float lpc = 0.0f, lqc = 0.0f;
        uint64_t kd = 0, kc = 0;
        const int jc = s > 0 ? s - 1 : 0;
        if (b < B) {
          // the step's noise keys before the wait (the asm keeps them from being moved past it)
          kd = pos_key(key_of(S.req[b].key_r), s, ST_DRAFT_C);
          kc = pos_key(key_of(S.req[b].key_r), jc, ST_RESIDUAL_C);
          asm volatile("" : "+v"(kd), "+v"(kc));
          // at s = 0 the token before the position is x0, which the set-up left in prev_d; after
          // that prev_d holds the previous step's token before its position
          xc = S.req[b].prev_d;
          if (s == 0) {
            r = S.role[b];
            xd = xc;
          } else {
            const uint64_t* w = pub_of(p, s & 1, b);
            uint64_t w0, w1, w2;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (true) {
              w0 = ld_u64(&w[0]);
              w1 = ld_u64(&w[1]);
              w2 = ld_u64(&w[2]);
              if ((uint32_t)(w0 >> 32) == (uint32_t)s && (uint32_t)(w1 >> 32) == (uint32_t)s &&
                  (uint32_t)(w2 >> 32) == (uint32_t)s)
                break;
              // a wait that does not end within the barrier's limit fails the call like a barrier
              // (the request then has no role; the merges mark every request invalid)
              if (failed(p.err, p.a.nonce) || __builtin_amdgcn_s_memrealtime() - t0 > p.a.wait_ticks) {
                __hip_atomic_store(p.err, p.a.nonce, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w0 = 0;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
            r = (int)((uint32_t)w0 >> 28);
            xd = (int)((uint32_t)w0 & 0x0FFFFFFFu) - 1;
            lqc = __uint_as_float((uint32_t)w1);
            lpc = __uint_as_float((uint32_t)w2);
            // xc, the token before position s - 1, is the previous step's prev_d: in the table while
            // the request had a role there (which a CORRECT row at s implies), x0 from the set-up at s = 1
            S.role[b] = (uint8_t)r;
          }
        }
        const uint64_t md = __ballot((r & RO_DRAFT) != 0), mc = __ballot((r & RO_CORRECT) != 0),
                       mp = __ballot((r & (RO_LSEP | RO_BONUS)) != 0);
        auto below = [&](uint64_t m) {   // set bits of m in lanes below this one
          return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        };
        if (lane == 0) S.wcnt[wave] = make_int4(__popcll(md), __popcll(mc), __popcll(mp), 0);
        __syncthreads();
        int od = nd, oc = nc, op = np;
#pragma unroll
        for (int w = 0; w < NW; w++) {
          const int4 c = S.wcnt[w];
          if (w < wave) {
            od += c.x;
            oc += c.y;
            op += c.z;
          }
          nd += c.x;
          nc += c.y;
          np += c.z;
        }
        if (b < B) {
          uint16_t sd = 0xFFFF, sc = 0xFFFF, sp = 0xFFFF;
          if (r & RO_DRAFT) sd = (uint16_t)(od + below(md));
          if (r & RO_CORRECT) sc = (uint16_t)(oc + below(mc));   // relative to the first CORRECT slot
          if (r & (RO_LSEP | RO_BONUS)) {
            sp = (uint16_t)(op + below(mp));
            S.plist[sp] = (uint16_t)b;
          }
          S.slot[b] = sd;
          S.slot[B + b] = sc;
          S.slot[2 * B + b] = sp;
          if (r) {
            ReqMeta m = S.req[b];   // invT and key_r are kept from the set-up
            m.prev_d = xd;
            m.prev_c = xc;
            m.lse_p_c = lpc;
            m.lse_q_c = lqc;
            put_key(m.key_d, kd);
            put_key(m.key_c, kc);
            S.req[b] = m;
            if (r & RO_DRAFT) S.blist[sd] = ent_make(b, false, m.prev_d);
          }
        }
        __syncthreads();   // the wave counts are read before the next round writes them
      }
      // the counts are uniform over the workgroup (every wave read the same LDS words)
      ls.n_draft = nd;
      ls.n_correct = nc;
      ls.n_plain = np;
      ls.c0 = (nd + SUB - 1) / SUB * SUB;
      ls.n_sb = (ls.c0 + nc + SUB - 1) / SUB;
      for (int b = tid; b < B; b += NT) {
        const uint16_t rc = S.slot[B + b];
        if (rc != 0xFFFF) {
          S.slot[B + b] = (uint16_t)(ls.c0 + rc);
          S.blist[ls.c0 + rc] = ent_make(b, true, S.req[b].prev_c);
        }
      }
      if (tid < SUB) {
        const int gi = ls.n_draft + tid;
        if (gi < ls.c0) S.blist[gi] = NO_ENT;
        const int ti = ls.c0 + ls.n_correct + tid;
        if (ti < ls.n_sb * SUB) S.blist[ti] = NO_ENT;
      }
      __syncthreads();
    }
    if (ls.n_sb == 0 && ls.n_plain == 0) break;   // uniform over the grid: every workgroup read the same roles

    // ---- 2. bias sub-blocks ----
    // row of sub-block k for this lane, and its tile loads
    auto row_of = [&](int k, int& b, int& j, bool& corr) {
      const uint32_t e = S.blist[k * SUB + m32];
      const bool has = e != NO_ENT;
      b = has ? ent_req(e) : -1;
      corr = has && (e & 1u);
      j = corr ? s - 1 : s;
    };
    // Operand loads are buffer loads over whole tensors (each smaller than 4 GiB, so a 32-bit byte
    // offset reaches all of it): an offset past the end reads zeros instead of faulting, so no
    // address is clamped and no value selected where the value is not used.
    //
    // B operands of sub-block k into sA[k & 1]: lane l of k-step t takes rank entries
    // (l >> 5) R/2 + 8 t ... + 7 of the A row of its slot (l & 31); wave w stages k-steps w, w + 4,
    // w + 8, w + 12 that lie below the rank (the rest hold zeros, written at the step's start).  A
    // slot without a previous token reads past the end of A, i.e. zeros.
    const int nks = p.a.R >> 4;
    auto stage_issue_ent = [&](uint32_t ent, u32x4 (&v)[4]) {
      const __amdgpu_buffer_rsrc_t rsA = ld_rsrc(p.a.A, (uint32_t)V * (uint32_t)p.a.R * 2u);
      const int prev = ent == NO_ENT ? -1 : ent_prev(ent);
      const uint32_t vo = prev >= 0 ? 2u * (uint32_t)(prev * p.a.R + h * (p.a.R >> 1) + 8 * wave) : OOB_OFF;
#pragma unroll
      for (int i = 0; i < 4; i++) v[i] = ldb16(rsA, vo + 64u * i, 0u);
    };
    auto stage_issue = [&](int k, u32x4 (&v)[4]) {
      stage_issue_ent((k < ls.n_sb) ? S.blist[k * SUB + m32] : NO_ENT, v);
    };
    auto stage_store = [&](int k, const u32x4 (&v)[4]) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (4 * i + wave < nks) ((u32x4*)S.sA)[(k & 1) * KSTEPS * 64 + (4 * i + wave) * 64 + lane] = v[i];
    };
    // The lane's logits of tile i (0..3: register chunks of this wave; 4: its LDS tile) in a row
    // are the 16 columns from 64 c + 32 f + 16 h, two 16-byte pieces.  V is a multiple of the
    // chunk width, so no piece crosses V; tiles of chunks the workgroup does not own read whatever
    // lies there (zeros past the tensor) and their results are discarded.  row_off is the byte
    // offset of the lane's first register-tile piece in row j of request b (rows of nrow
    // positions); the LDS tile lies a wave-uniform distance dlds further.
    const uint32_t Vb = 2u * (uint32_t)V;
    const uint32_t dlds = 2u * (uint32_t)(CH * (NW * AG_CHUNKS - AG_CHUNKS * wave + (wave >> 1)) + 32 * (wave & 1));
    auto row_off = [&](int b, int j, int nrow) -> uint32_t {
      return b >= 0 ? (uint32_t)(b * nrow + j) * Vb + 2u * (uint32_t)(CH * (cbeg + AG_CHUNKS * wave) + 16 * h)
                    : PAST_END;   // an empty slot reads zeros, without a memory access
    };
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo, int i, u32x4 (&T)[2]) {
      const uint32_t off = i < 4 ? (uint32_t)((i >> 1) * 2 * CH + (i & 1) * 64) : dlds;
      T[0] = ldb16(rs, vo + off, 0u);
      T[1] = ldb16(rs, vo + off + 16u, 0u);
    };
    const __amdgpu_buffer_rsrc_t rs_base = ld_rsrc(p.a.base, (uint32_t)B * (uint32_t)K * Vb);
    const __amdgpu_buffer_rsrc_t rs_tgt = ld_rsrc(p.a.target, (uint32_t)B * (uint32_t)(K + 1) * Vb);
    auto seed_acc = [&](const u32x4 (&tt)[2], int i) -> f32x16 {
      float x[16];
      unpack16(tt[0], tt[1], x);
      f32x16 a;
#pragma unroll
      for (int q = 0; q < 16; q++) a[q] = x[q];
      return a;
    };

    // Per sub-block, three MFMA passes in turn: register chunk 0 (tiles 0, 1), register chunk 1
    // (tiles 2, 3), the LDS half chunk (tile 4; waves without one run it on zero W and -inf
    // logits, which costs no time: the workgroup waits for the waves that have one).  The
    // element-wise part of each pass follows the next pass's MFMA chain in straight-line code, so
    // the two can overlap; only 2 or 3 tiles of accumulators are live at a time.  DRAFT and
    // CORRECT sub-blocks (the latter after all the former) run in separate loops.
    const bool wave_lds = 2 * n_lds > wave;     // this wave has an LDS tile (wave-uniform)
    const int cg0 = cbeg + AG_CHUNKS * wave;   // global chunk of this wave's register chunk 0
    const bool has0 = AG_CHUNKS * wave < nch, has1 = AG_CHUNKS * wave + 1 < nch;
    const bf16x8* wlw = S.wl + (size_t)wave * KSTEPS * 64;
    const int n_dsb = ls.c0 / SUB;             // DRAFT sub-blocks [0, n_dsb), CORRECT [n_dsb, n_sb)
    auto chain_reg = [&](f32x16& x, f32x16& y, const bf16x8 (&w0)[KSTEPS], const bf16x8 (&w1)[KSTEPS],
                         const bf16x8* sAk) {
      bf16x8 bop = sAk[lane], bop1 = sAk[64 + lane];
#pragma unroll
      for (int t = 0; t < KSTEPS; t++) {
        const bf16x8 bop2 = (t + 2 < KSTEPS) ? sAk[(t + 2) * 64 + lane] : bop;
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0[t], bop, x, 0, 0, 0);
        y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1[t], bop, y, 0, 0, 0);
        bop = bop1;
        bop1 = bop2;
      }
    };
    auto chain_lds = [&](f32x16& x, const bf16x8* sAk) {
      bf16x8 bop = sAk[lane], wl = wlw[lane], bop1 = sAk[64 + lane], wl1 = wlw[64 + lane];
#pragma unroll
      for (int t = 0; t < KSTEPS; t++) {
        const bf16x8 bop2 = (t + 2 < KSTEPS) ? sAk[(t + 2) * 64 + lane] : bop;
        const bf16x8 wl2 = (t + 2 < KSTEPS) ? wlw[(t + 2) * 64 + lane] : wl;
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl, bop, x, 0, 0, 0);
        bop = bop1;
        bop1 = bop2;
        wl = wl1;
        wl1 = wl2;
      }
    };
    auto pin_w = [&]() {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) asm volatile("" : "+a"(wf[i][t]));
    };
    auto store_records = [&](int k, bool corr_sb, int b, const WaveRec& wr) {
      if (h == 0 && b >= 0) {
        const size_t ri = ((size_t)(k * SUB + m32) * NW + wave) * MAX_G + g;
        rec_store(rec_rsrc(p.rec_d, rec_d_bytes(B)), ri, wr.a);
        if (corr_sb) {
          const size_t rc = ((size_t)(k * SUB + m32 - ls.c0) * NW + wave) * MAX_G + g;
          rec_store(rec_rsrc(p.rec_c, rec_c_bytes(B)), rc, wr.t);
        }
      }
    };
    u32x4 Tc[5][2];                            // draft logits of the current sub-block
    if (ls.n_sb > 0) {
      // k-steps past the rank read zeros (the merges reuse this LDS, so they are rewritten here)
      if (nks < KSTEPS)
        for (int e = tid; e < 2 * KSTEPS * 64; e += NT)
          if (((e >> 6) & (KSTEPS - 1)) >= nks) ((u32x4*)S.sA)[e] = kZero;
      u32x4 sv[4];
      stage_issue(0, sv);
      int b, j;
      bool corr;
      row_of(0, b, j, corr);
      const uint32_t vo = row_off(b, j, K);
#pragma unroll
      for (int i = 0; i < 5; i++) load_tile(rs_base, vo, i, Tc[i]);
      stage_store(0, sv);
    }
    __syncthreads();

    // DRAFT sub-blocks: chunk log-masses and Gumbel scores of position s.  The last part of a
    // sub-block (its LDS tile's log-mass and its records) runs in the next sub-block's first chain,
    // which has VALU issue slots to spare; the state of that part is carried over.
    // record of DRAFT sub-block kk from its scalars and LDS-tile log-mass
    auto draft_record = [&](int kk, int bb, float l0, float l1, float gm, float hl) __attribute__((always_inline)) {
      const float2 gp = pair32(gm);
      const float g0 = gp.x, g1 = gp.y;
      l0 = has0 ? l0 : -INFINITY;
      l1 = has1 ? l1 : -INFINITY;
      hl = wave_lds ? hl : -INFINITY;
      const float s0 = (l0 > -INFINITY) ? l0 + g0 : -INFINITY;
      const float s1 = (l1 > -INFINITY) ? l1 + g1 : -INFINITY;
      // best of the two register chunks: larger score, the smaller chunk on ties, a NaN log-mass
      // never wins (it makes the row invalid through the log-mass)
      const bool t0 = has0 && !(l0 != l0);
      float bs = t0 ? s0 : -INFINITY;
      int bc = t0 ? cg0 : -1;
      const bool t1 = has1 && takes(s1, cg0 + 1, bs, bc);
      bs = t1 ? s1 : bs;
      bc = t1 ? cg0 + 1 : bc;
      WaveRec wr;
      wr.a = make_float4(lse_add(l0, l1), bs, __int_as_float(bc), hl);
      wr.t = make_float4(-INFINITY, -INFINITY, __int_as_float(-1), -INFINITY);
      store_records(kk, false, bb, wr);
    };
    f32x16 a4p = {};                     // the previous sub-block's LDS-tile accumulators
    float l0p = 0.0f, l1p = 0.0f, gmp = 0.0f, invTp = 1.0f;
    int bp = -1;                         // its row (-1: none, or no previous sub-block)
    // the row of the lane's slot in the next sub-block, with its temperature and noise key (read
    // one sub-block ahead, so that no sub-block waits on its own)
    int bn, jn;
    {
      bool cn;
      row_of(0, bn, jn, cn);
    }
    float invTn = S.req[bn >= 0 ? bn : 0].invT;
    uint32_t kn0 = S.req[bn >= 0 ? bn : 0].key_d[0], kn1 = S.req[bn >= 0 ? bn : 0].key_d[1];
    for (int k = 0; k < n_dsb; k++) {
      tid = opaque_tid();
      const int b = bn, j = jn;
      const float invT = b >= 0 ? invTn : 1.0f;
      const uint64_t key = (uint64_t)kn0 | ((uint64_t)kn1 << 32);
      const bf16x8* sAk = S.sA + (size_t)(k & 1) * KSTEPS * 64;
      // in flight during this sub-block: the next sub-block's B operands, and its draft logits,
      // each tile loaded into the registers its predecessor leaves when it seeds its pass
      const uint32_t ent2 = (k + 1 < ls.n_sb) ? S.blist[(k + 1) * SUB + m32] : NO_ENT;
      u32x4 sv[4];
      stage_issue_ent(ent2, sv);
      const int b2 = ent2 == NO_ENT ? -1 : ent_req(ent2);
      const int j2 = (ent2 != NO_ENT && (ent2 & 1u)) ? s - 1 : s;
      const uint32_t vo2 = row_off(b2, j2, K);
      {
        const ReqMeta& rq = S.req[b2 >= 0 ? b2 : 0];
        invTn = rq.invT;
        kn0 = rq.key_d[0];
        kn1 = rq.key_d[1];
      }
      bn = b2;
      jn = j2;
      f32x16 a0 = seed_acc(Tc[0], 0), a1 = seed_acc(Tc[1], 1);
      load_tile(rs_base, vo2, 0, Tc[0]);
      load_tile(rs_base, vo2, 1, Tc[1]);
      const float lc = invT * LOG2E;
      __builtin_amdgcn_sched_barrier(0);
      // Three MFMA chains, each k-step a scheduling region of its own: the chain's MFMAs, the LDS
      // read two k-steps ahead, and one slice of element-wise work that does not depend on the
      // chain, so that the VALU issues while the matrix core runs.
      // chain 0: register chunk 0; slices: the seeds of chain 1, the noise of chunk cg0 + h, the
      // previous sub-block's LDS-tile log-mass and records
      pin_w();
      vfence(a0);
      vfence(a1);
      vfence(Tc[2]);
      vfence(Tc[3]);
      vfence(a4p);
      f32x16 a2, a3;
      GumbelStage gs;
      Lse2 stp;
      lse2_init(stp);
      {
        bf16x8 bq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) bq[u] = sAk[u * 64 + lane];
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) bq[t + 4] = sAk[(t + 4) * 64 + lane];
          const bf16x8 bop = bq[t];
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][t], bop, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][t], bop, a1, 0, 0, 0);
          if (t < 2) { vfence(Tc[2][t]); seed_piece(a2, Tc[2][t], t); }
          else if (t < 4) { vfence(Tc[3][t - 2]); seed_piece(a3, Tc[3][t - 2], t - 2); }
          if (t < 4) {
            gumbel_step(gs, t, key, (uint32_t)(cg0 + h));
            gumbel_fence(gs, t);
          } else if (t < 13) {
            lse1_step(stp, t - 4, a4p, invTp * LOG2E, invTp);
            lse1_fence(stp, t - 4);
          } else if (t == 13) {
            draft_record(k - 1, bp, l0p, l1p, gmp, stp.r);   // stores nothing for bp < 0
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float gm = gs.r;
      load_tile(rs_base, vo2, 2, Tc[2]);
      load_tile(rs_base, vo2, 3, Tc[3]);
      __builtin_amdgcn_sched_barrier(0);
      // chain 1: register chunk 1; slices: chunk 0's log-mass, the seed of the LDS chain
      vfence(a0);
      vfence(a1);
      vfence(Tc[4]);
      f32x16 a4;
      Lse2 st0;
      lse2_init(st0);
      {
        bf16x8 bq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) bq[u] = sAk[u * 64 + lane];
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) bq[t + 4] = sAk[(t + 4) * 64 + lane];
          const bf16x8 bop = bq[t];
          a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[2][t], bop, a2, 0, 0, 0);
          a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[3][t], bop, a3, 0, 0, 0);
          lse2_step(st0, t, a0, a1, lc, invT);
          lse2_fence(st0, t);
          if (t >= 14) {
            vfence(Tc[4][t - 14]);
            seed_piece(a4, Tc[4][t - 14], t - 14);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float l0 = st0.r;
      load_tile(rs_base, vo2, 4, Tc[4]);
      __builtin_amdgcn_sched_barrier(0);
      // chain L: the LDS half chunk; slices: chunk 1's log-mass
      vfence(a2);
      vfence(a3);
      Lse2 st1;
      lse2_init(st1);
      {
        bf16x8 bq[KSTEPS], wq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) { bq[u] = sAk[u * 64 + lane]; wq[u] = wlw[u * 64 + lane]; }
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) bq[t + 4] = sAk[(t + 4) * 64 + lane];
          const bf16x8 bop = bq[t];
          if (t + 4 < KSTEPS) wq[t + 4] = wlw[(t + 4) * 64 + lane];
          const bf16x8 wl = wq[t];
          a4 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl, bop, a4, 0, 0, 0);
          lse2_step(st1, t, a2, a3, lc, invT);
          lse2_fence(st1, t);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float l1 = st1.r;
      a4p = a4;
      l0p = l0;
      l1p = l1;
      gmp = gm;
      invTp = invT;
      bp = b;
      stage_store(k + 1, sv);
      __syncthreads();
    }
    if (bp >= 0) draft_record(n_dsb - 1, bp, l0p, l1p, gmp, tiles_lse<1>(&a4p, invTp));

    for (int k = n_dsb; k < ls.n_sb; k++) {
      tid = opaque_tid();
      int b, j;
      bool corr;
      row_of(k, b, j, corr);
      const ReqMeta rm = S.req[b >= 0 ? b : 0];
      const float invT = b >= 0 ? rm.invT : 1.0f;
      const uint64_t key = key_of(rm.key_c);
      const bf16x8* sAk = S.sA + (size_t)(k & 1) * KSTEPS * 64;
      u32x4 sv[4];
      stage_issue(k + 1, sv);
      int b2 = -1, j2 = 0;
      bool c2 = false;
      if (k + 1 < ls.n_sb) row_of(k + 1, b2, j2, c2);
      const uint32_t vo2 = row_off(b2, j2, K);
      u32x4 Tt[5][2];
      const uint32_t vot = row_off(b, j, K + 1);
      load_tile(rs_tgt, vot, 0, Tt[0]);
      load_tile(rs_tgt, vot, 1, Tt[1]);
      f32x16 a0 = seed_acc(Tc[0], 0), a1 = seed_acc(Tc[1], 1);
      load_tile(rs_base, vo2, 0, Tc[0]);
      load_tile(rs_base, vo2, 1, Tc[1]);
      const float lp = rm.lse_p_c;
      const float c = invT * LOG2E, op = -rm.lse_p_c * LOG2E, oq = -rm.lse_q_c * LOG2E;
      __builtin_amdgcn_sched_barrier(0);
      // chain 0: register chunk 0; slices: the seeds of chain 1, the noise of chunk cg0 + h
      pin_w();
      vfence(a0);
      vfence(a1);
      f32x16 a2, a3;
      GumbelStage gs;
      {
        bf16x8 bq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) bq[u] = sAk[u * 64 + lane];
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) bq[t + 4] = sAk[(t + 4) * 64 + lane];
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][t], bq[t], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][t], bq[t], a1, 0, 0, 0);
          if (t < 2) {
            vfence(Tc[2][t]);
            seed_piece(a2, Tc[2][t], t);
          } else if (t < 4) {
            vfence(Tc[3][t - 2]);
            seed_piece(a3, Tc[3][t - 2], t - 2);
          } else if (t < 8) {
            gumbel_step(gs, t - 4, key, (uint32_t)(cg0 + h));
            gumbel_fence(gs, t - 4);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float gm = gs.r;
      load_tile(rs_base, vo2, 2, Tc[2]);
      load_tile(rs_base, vo2, 3, Tc[3]);
      load_tile(rs_tgt, vot, 2, Tt[2]);
      load_tile(rs_tgt, vot, 3, Tt[3]);
      __builtin_amdgcn_sched_barrier(0);
      // chain 1: register chunk 1; slices: chunk 0's residual and target sums, the LDS seed
      vfence(a0);
      vfence(a1);
      f32x16 a4;
      Corr2 c0s = {0.0f, 0.0f, 0.0f, 0.0f};
      {
        bf16x8 bq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) bq[u] = sAk[u * 64 + lane];
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) bq[t + 4] = sAk[(t + 4) * 64 + lane];
          a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[2][t], bq[t], a2, 0, 0, 0);
          a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[3][t], bq[t], a3, 0, 0, 0);
          corr_step(c0s, 2 * t, a0, a1, Tt[0][0], Tt[0][1], Tt[1][0], Tt[1][1], c, op, oq);
          corr_fence(c0s);
          if (t >= 14) {
            vfence(Tc[4][t - 14]);
            seed_piece(a4, Tc[4][t - 14], t - 14);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      load_tile(rs_base, vo2, 4, Tc[4]);
      load_tile(rs_tgt, vot, 4, Tt[4]);
      __builtin_amdgcn_sched_barrier(0);
      // chain L: the LDS half chunk; slices: chunk 1's residual and target sums
      vfence(a2);
      vfence(a3);
      Corr2 c1s = {0.0f, 0.0f, 0.0f, 0.0f};
      {
        bf16x8 bq[KSTEPS], wq[KSTEPS];
#pragma unroll
        for (int u = 0; u < 4; u++) {
          bq[u] = sAk[u * 64 + lane];
          wq[u] = wlw[u * 64 + lane];
        }
#pragma unroll
        for (int t = 0; t < KSTEPS; t++) {
          if (t + 4 < KSTEPS) {
            bq[t + 4] = sAk[(t + 4) * 64 + lane];
            wq[t + 4] = wlw[(t + 4) * 64 + lane];
          }
          a4 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wq[t], bq[t], a4, 0, 0, 0);
          corr_step(c1s, 2 * t, a2, a3, Tt[2][0], Tt[2][1], Tt[3][0], Tt[3][1], c, op, oq);
          corr_fence(c1s);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      const float2 gp = pair32(gm);
      const float g0 = gp.x, g1 = gp.y;
      float m0, t0, m1, t1, mh, th;
      corr_end(c0s, lp, m0, t0);
      corr_end(c1s, lp, m1, t1);
      {
        // the LDS half tile: 16 values against two target pieces
        Corr2 hs = {0.0f, 0.0f, 0.0f, 0.0f};
        const f32x16 zero = {};
#pragma unroll
        for (int i = 0; i < 16; i += 2)
          corr_step(hs, i, a4, zero, Tt[4][0], Tt[4][1], Tt[4][0], Tt[4][1], c, op, oq);
        corr_end(hs, lp, mh, th);
      }

      m0 = has0 ? m0 : 0.0f;
      t0 = has0 ? t0 : -INFINITY;
      m1 = has1 ? m1 : 0.0f;
      t1 = has1 ? t1 : -INFINITY;
      mh = wave_lds ? mh : 0.0f;
      th = wave_lds ? th : -INFINITY;
      const float lm0 = m0 > 0.0f ? lg2(m0) * LN2 : -INFINITY;
      const float lm1 = m1 > 0.0f ? lg2(m1) * LN2 : -INFINITY;
      float bs = -INFINITY, bt = -INFINITY;
      int bc = -1, btc = -1;
      if (lm0 > -INFINITY) { bs = lm0 + g0; bc = cg0; }
      if (lm1 > -INFINITY && takes(lm1 + g1, cg0 + 1, bs, bc)) { bs = lm1 + g1; bc = cg0 + 1; }
      if (has0 && t0 > -INFINITY) { bt = t0 + g0; btc = cg0; }
      if (has1 && t1 > -INFINITY && takes(t1 + g1, cg0 + 1, bt, btc)) { bt = t1 + g1; btc = cg0 + 1; }
      const float msum = m0 + m1;
      WaveRec wr;
      wr.a = make_float4(msum > 0.0f ? lg2(msum) * LN2 : -INFINITY, bs, __int_as_float(bc), mh);
      wr.t = make_float4(lse_add(t0, t1), bt, __int_as_float(btc), th);
      stage_store(k + 1, sv);
      store_records(k, true, b, wr);
      __syncthreads();
    }

    // ---- 3. plain rows: every LSEP / BONUS target row in contiguous items of TP columns, the
    //         items of all plain rows spread over all waves of the grid (target rows need no W,
    //         so they are not tied to a workgroup's vocabulary slice) ----
    {
      // Wave w takes items w, w + GW, w + 2 GW, ... (GW: all waves of the grid).  Every piece of
      // an item is used once (LSEP: a running lane maximum with a rescaled sum; BONUS: per-chunk
      // masses), and the piece of the wave's next item is loaded into its registers right after,
      // so that one item's loads are in flight during the whole of the previous item's arithmetic.
      tid = opaque_tid();
      const int nrP = (V + TP - 1) / TP;
      const int n_items = ls.n_plain * nrP;
      const int GW = G * NW;
      constexpr int NP = TP / 512;   // 16-byte pieces per lane
      struct PItem {
        int ps, t, rb, xin;          // plain slot, item of the row, request (-1: none), pieces inside V
      };
      auto item_of = [&](int it) {
        PItem q;
        q.ps = it < n_items ? it / nrP : -1;
        q.t = q.ps >= 0 ? it - q.ps * nrP : 0;
        q.rb = q.ps >= 0 ? __builtin_amdgcn_readfirstlane((int)S.plist[q.ps]) : -1;
        q.xin = 0;
#pragma unroll
        for (int i = 0; i < NP; i++) q.xin |= (q.t * TP + (i * 64 + lane) * 8 < V) ? (1 << i) : 0;
        return q;
      };
      // the lane's piece i of item q; a piece past V, or of no item, is read at an offset past the
      // tensor (zeros, no memory access) and its results are masked
      const uint32_t tgt_bytes = (uint32_t)B * (uint32_t)(K + 1) * Vb;
      auto load_piece = [&](const PItem& q, int i) -> u32x4 {
        const uint32_t off = (q.rb >= 0 && ((q.xin >> i) & 1))
                                 ? (uint32_t)(q.rb * (K + 1) + s) * Vb + 2u * (uint32_t)(q.t * TP + (i * 64 + lane) * 8)
                                 : tgt_bytes;
        return ldb16(rs_tgt, off, 0u);
      };
      int it = g * NW + wave;
      PItem cur = item_of(it);
      u32x4 x[NP];
      if (cur.rb >= 0) {   // wave-uniform conditions throughout
#pragma unroll
        for (int i = 0; i < NP; i++) x[i] = load_piece(cur, i);
      }
      while (cur.rb >= 0) {
        const PItem nxt = item_of(it + GW);
        const int rr = __builtin_amdgcn_readfirstlane((int)S.role[cur.rb]);
        const float invT = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, S.req[cur.rb].invT)));
        const float c = invT * LOG2E;
        float4 rec;
        if (rr & RO_LSEP) {
          // the item's log-mass: per lane a running maximum m and the sum of exp(c (v - m)),
          // rescaled whenever m grows; then the wave maximum and the rescaled lane sums
          float m = -INFINITY, s0 = 0.0f, s1 = 0.0f;
#pragma unroll
          for (int i = 0; i < NP; i++) {
            // piece i of the next item replaces this one as soon as it is read (unconditionally,
            // so that every wait counts the same loads); the pieces are pinned in order
            const u32x4 w = x[i];
            x[i] = load_piece(nxt, i);
            const bool in = (cur.xin >> i) & 1;
            float pm = vmax(bf_lo(w[0]), bf_hi(w[0]));
#pragma unroll
            for (int e = 1; e < 4; e++) pm = vmax(pm, vmax(bf_lo(w[e]), bf_hi(w[e])));
            const float mn = vmax(m, in ? pm : -INFINITY);
            const float mo = (mn == -INFINITY) ? 0.0f : mn * c;
            const float sc = (m == -INFINITY) ? 0.0f : ex2(fmaf(m, c, -mo));
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; e++) {
              a0 += ex2(fmaf(bf_lo(w[e]), c, -mo));
              a1 += ex2(fmaf(bf_hi(w[e]), c, -mo));
            }
            s0 = fmaf(s0, sc, in ? a0 : 0.0f);
            s1 = fmaf(s1, sc, in ? a1 : 0.0f);
            m = mn;
            __builtin_amdgcn_sched_barrier(0);
          }
          const float mx = wmax(m);
          const float Mo = (mx == -INFINITY) ? 0.0f : mx * c;
          const float sm = wsum(m == -INFINITY ? 0.0f : (s0 + s1) * ex2(fmaf(m, c, -Mo)));
          const float lse = (mx == -INFINITY) ? (sm == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sm) * LN2;
          rec = make_float4(lse, -INFINITY, __int_as_float(-1), 0.0f);
        } else {
          // BONUS: the log-mass of each 64-column chunk (8 lanes per chunk in every piece, all
          // eight holding it after the group reductions); then lane l takes chunk
          // 8 (l mod 8) + l / 8 of the item, i.e. piece l mod 8 of its lane group, for the
          // item's log-mass, the chunk's Gumbel score and the best chunk
          float lcs[NP];
#pragma unroll
          for (int i = 0; i < NP; i++) {
            const u32x4 w = x[i];
            x[i] = load_piece(nxt, i);
            float mx = vmax(bf_lo(w[0]), bf_hi(w[0]));
#pragma unroll
            for (int e = 1; e < 4; e++) mx = vmax(mx, vmax(bf_lo(w[e]), bf_hi(w[e])));
            mx = vmax(mx, dpp<0xB1>(mx));   // over the 8 lanes of the chunk
            mx = vmax(mx, dpp<0x4E>(mx));
            mx = vmax(mx, dpp<0x141>(mx));
            const float mo = (mx == -INFINITY) ? 0.0f : mx * c;
            float sm = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; e++) sm += ex2(fmaf(bf_lo(w[e]), c, -mo)) + ex2(fmaf(bf_hi(w[e]), c, -mo));
            sm = sum8(sm);
            lcs[i] = (mx == -INFINITY) ? (sm == 0.0f ? -INFINITY : NAN) : mx * invT + lg2(sm) * LN2;
            lcs[i] = ((cur.xin >> i) & 1) ? lcs[i] : -INFINITY;
            __builtin_amdgcn_sched_barrier(0);
          }
          float lc = lcs[0];
#pragma unroll
          for (int i = 1; i < NP; i++) lc = ((lane & 7) == i) ? lcs[i] : lc;
          const int cg = cur.t * (TP / CH) + 8 * (lane & 7) + (lane >> 3);   // global chunk of the lane
          lc = cg * CH < V ? lc : -INFINITY;
          // wave log-sum-exp of the chunk masses
          const float M = wmax(lc);
          const float e = (lc == -INFINITY) ? 0.0f : ex2((lc - (M == -INFINITY ? 0.0f : M)) * LOG2E);
          const int nan = __ballot(lc != lc) != 0ull;
          const float S_ = wsum(e);
          const float lse_tot = nan ? NAN : (M == -INFINITY ? -INFINITY : M + lg2(S_) * LN2);
          // the chunk's score and the wave argmax
          const uint64_t key = pos_key(req_key(seed, p.a.req_off + cur.rb), s, ST_BONUS_C);
          const float gn = gumbel_bits(bits_at(key, (uint32_t)cg));
          float bs = lc > -INFINITY ? lc + gn : -INFINITY, dummy = 0.0f;
          int bc = lc > -INFINITY ? cg : -1;
          wargmax(bs, bc, dummy);
          rec = make_float4(lse_tot, bs, __int_as_float(bc), 0.0f);
        }
        if (lane == 0) rec_store(rec_rsrc(p.rec_p, rec_p_bytes(B)), (size_t)cur.ps * MAX_G + cur.t, rec);
        cur = nxt;
        it += GW;
      }
    }

    // ---- 4. grid barrier: every record of step s is written ----
    grid_barrier(p.flags, p.err, p.a.nonce, G, token++, p.a.wait_ticks);

    // ---- 5. merges: this workgroup's requests b = g, g + G, ... one after another; each publishes
    //         its request's roles, drafted token and log-normalisers for step s + 1 ----
    for (int r = 0; r < NW; r++) {
      const int b = g + G * r;
      if (b >= B) break;
      merge_request(p, S, b, s, ls.c0);
    }
    __syncthreads();   // the merges' reads of the tables are done before the next lists rewrite them
  }
#undef lane
#undef m32
#undef h
  // a synchronisation fault: every request this workgroup merges is marked invalid
  if (failed(p.err, p.a.nonce)) {
    for (int i = threadIdx.x; i < NW * (K + 1); i += NT) {
      const int w = i / (K + 1), j = i % (K + 1);
      const int b = g + G * w;
      if (b >= B) continue;
      p.a.tokens[(size_t)b * (K + 1) + j] = -1;
      if (j == 0) p.a.accepted_len[b] = -1;
    }
  }
}


// ==========================================================================================
// Acceptance statistics with W on chip: alpha_{b,j} = sum_v min(p_j(v), q_j(v)) of every listed
// drafted position ("The Speed Claim Nobody's Really Questioning", sections "The Semi-Autoregressive
// Trick" and "The Real Innovation: Confidence-Scheduled Verification").  One cooperative launch
// with the vocabulary partition and W layout of k_resident.  The listed rows go in batches of
// nbr rows (a multiple of SUB, their logits sized to stay in the Infinity Cache), each in four
// phases:
//   1. every workgroup, every sub-block of 32 rows: q = base + A[prev] . W (MFMA) and p over its
//      slice -> per-workgroup log-normalisers of q and p;
//   2. (grid barrier) one wave per row: the rows' log-normalisers;
//   3. (grid barrier) every workgroup again: sum over its slice of min(p, q), the smaller of the two
//      probabilities taken in the log domain;
//   4. one wave per row: alpha, summed over the workgroups in a fixed order.  It runs after the
//      next batch's first barrier, beside that batch's phase 2 (after a last barrier for the last
//      batch): phases 1 and 2 of a batch touch other arrays than phase 4 of the one before.
// ==========================================================================================
struct StatsKP {
  int B, K, V, R, G, nbr;
  const void* base;
  const void* target;
  const void* A;
  const void* W;
  const float* temp;
  const int32_t* n_rows;   // [1] listed rows
  const int32_t* rows;     // [n] row id b K + j of each listed row
  const int32_t* prev;     // [n] its previous token (-1: none)
  float* alpha;            // [B, K] out
  float* o_lse_q;          // [B, K] out, may be null
  float* o_lse_p;          // [B, K] out, may be null
  float* lq;               // [nbr] log-normalisers of the batch's rows
  float* lp;               // [nbr]
  float2* part1;           // [nbr][MAX_G] per-workgroup log-normalisers
  float* part2;            // [nbr][MAX_G] per-workgroup sums of min(p, q)
  uint64_t* flags;         // [MAX_G][FLAG_STRIDE]
  uint64_t* err;
  uint64_t nonce;
  uint64_t wait_ticks;     // limit of every bounded wait, s_memrealtime ticks
};

__host__ __device__ inline size_t stats_smem_bytes() {
  return (size_t)4 * KSTEPS * 64 * 16 + (size_t)2 * KSTEPS * 64 * 16 + (size_t)2 * NW * SUB * 8;
}

__global__ __launch_bounds__(NT, 1) void k_stats_res(StatsKP p) {
  extern __shared__ __align__(16) char smem_raw[];
  bf16x8* wl = (bf16x8*)smem_raw;                             // [4][KSTEPS][64] W tiles of the LDS chunks
  bf16x8* sA = wl + 4 * KSTEPS * 64;                          // [2][KSTEPS][64] B operands
  float2* red = (float2*)(sA + 2 * KSTEPS * 64);              // [2][NW][SUB] wave results
  const int K = p.K, V = p.V, R = p.R, G = p.G;
  const int tid = threadIdx.x, lane = tid & 63, m32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;
  const int cbeg = chunk_begin(g, G, V), nch = chunks_of(g, G, V);
  const int n_lds = nch > NW * AG_CHUNKS ? nch - NW * AG_CHUNKS : 0;
  const int nks = R >> 4;

  // ---- W slice on chip (the layout of k_resident): register chunks 2 wave, 2 wave + 1 and the
  //      LDS tiles of local chunks 8 and 9 ----
  bf16x8 wf[4][KSTEPS];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int cl = AG_CHUNKS * wave + (i >> 1);
    const int c = cl < nch ? cbeg + cl : -1;
    const int col_in = 16 * ((m32 >> 2) & 1) + 4 * (m32 >> 3) + (m32 & 3);
    const int v = CH * c + 32 * (i & 1) + col_in;
#pragma unroll
    for (int t = 0; t < KSTEPS; t++) {
      const bool in = c >= 0 && v < V && t < nks;
      const u32x4 x = *(const u32x4*)((const uint16_t*)p.W + (in ? (size_t)v * R + h * (R >> 1) + 8 * t : 0));
      wf[i][t] = __builtin_bit_cast(bf16x8, in ? x : kZero);
    }
  }
  {
    constexpr int NE = 4 * KSTEPS * 64 / NT;   // every load of the thread before any store
    u32x4 z[NE];
#pragma unroll
    for (int q = 0; q < NE; q++) {
      const int e = tid + NT * q;
      const int u = e / (KSTEPS * 64), t = (e / 64) % KSTEPS, l = e % 64;
      const int cl = NW * AG_CHUNKS + (u >> 1);
      const int c = cl < nch ? cbeg + cl : -1;
      const int mm = l & 31, hh = l >> 5;
      const int col_in = 16 * ((mm >> 2) & 1) + 4 * (mm >> 3) + (mm & 3);
      const int v = CH * c + 32 * (u & 1) + col_in;
      const bool in = c >= 0 && v < V && t < nks;
      const u32x4 x = *(const u32x4*)((const uint16_t*)p.W + (in ? (size_t)v * R + hh * (R >> 1) + 8 * t : 0));
      z[q] = in ? x : kZero;
    }
#pragma unroll
    for (int q = 0; q < NE; q++) ((u32x4*)wl)[tid + NT * q] = z[q];
  }
  // k-steps past the rank read zeros
  for (int e = tid; e < 2 * KSTEPS * 64; e += NT)
    if (((e >> 6) & (KSTEPS - 1)) >= nks) ((u32x4*)sA)[e] = kZero;

  const int n = p.n_rows[0];
  const int nbr = p.nbr;
  const uint32_t Vb = 2u * (uint32_t)V;
  const __amdgpu_buffer_rsrc_t rs_base = ld_rsrc(p.base, (uint32_t)p.B * (uint32_t)K * Vb);
  const __amdgpu_buffer_rsrc_t rs_tgt = ld_rsrc(p.target, (uint32_t)p.B * (uint32_t)(K + 1) * Vb);
  const __amdgpu_buffer_rsrc_t rsA = ld_rsrc(p.A, (uint32_t)V * (uint32_t)R * 2u);
  const uint32_t dlds = 2u * (uint32_t)(CH * (NW * AG_CHUNKS - AG_CHUNKS * wave + (wave >> 1)) + 32 * (wave & 1));
  const uint32_t col0 = 2u * (uint32_t)(CH * (cbeg + AG_CHUNKS * wave) + 16 * h);
  // tile i of this wave (0..3: register chunks; 4: its LDS tile) exists in the workgroup's slice
  const bool has0 = AG_CHUNKS * wave < nch, has1 = AG_CHUNKS * wave + 1 < nch, wave_lds = 2 * n_lds > wave;
  auto tile_on = [&](int i) { return i < 2 ? has0 : (i < 4 ? has1 : wave_lds); };
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo, int i, u32x4 (&T)[2]) {
    const uint32_t off = i < 4 ? (uint32_t)((i >> 1) * 2 * CH + (i & 1) * 64) : dlds;
    T[0] = ldb16(rs, vo + off, 0u);
    T[1] = ldb16(rs, vo + off + 16u, 0u);
  };
  auto load_tiles = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo, u32x4 (&T)[5][2]) {
#pragma unroll
    for (int i = 0; i < 5; i++) load_tile(rs, vo, i, T[i]);
  };
  // the listed row of the lane's slot in sub-block k of the batch from r0
  struct RowIn {
    int lr, rid, prev;
    float invT;
    uint32_t vb, vt;   // byte offsets of the lane's first piece in the base and target rows
  };
  auto row_in = [&](int r0, int nb, int k) {
    RowIn r;
    r.lr = k * SUB + m32;
    const bool act = r.lr < nb;
    r.rid = act ? p.rows[r0 + r.lr] : -1;
    r.prev = act ? p.prev[r0 + r.lr] : -1;
    const int b = act ? r.rid / K : 0, j = act ? r.rid - b * K : 0;
    r.invT = act ? 1.0f / p.temp[b] : 1.0f;
    r.vb = act ? (uint32_t)(b * K + j) * Vb + col0 : PAST_END;   // inactive: past both tensors
    r.vt = act ? (uint32_t)(b * (K + 1) + j) * Vb + col0 : PAST_END;
    return r;
  };
  auto stage_issue = [&](int prev, u32x4 (&v)[4]) {
    const uint32_t vo = prev >= 0 ? 2u * (uint32_t)(prev * R + h * (R >> 1) + 8 * wave) : OOB_OFF;
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = ldb16(rsA, vo + 64u * i, 0u);
  };
  auto stage_store = [&](int k, const u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (4 * i + wave < nks) ((u32x4*)sA)[(k & 1) * KSTEPS * 64 + (4 * i + wave) * 64 + lane] = v[i];
  };
  // MFMA chains of register chunk ci (tiles 2 ci, 2 ci + 1) and of the LDS tile over the rank,
  // LDS operands read two k-steps ahead
  auto chain_reg = [&](f32x16& x, f32x16& y, int ci, const bf16x8* sAk) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int t = 0; t < KSTEPS; t++) asm volatile("" : "+a"(wf[i][t]));
    bf16x8 bop = sAk[lane], bop1 = sAk[64 + lane];
#pragma unroll
    for (int t = 0; t < KSTEPS; t++) {
      const bf16x8 bop2 = (t + 2 < KSTEPS) ? sAk[(t + 2) * 64 + lane] : bop;
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ci == 0 ? wf[0][t] : wf[2][t], bop, x, 0, 0, 0);
      y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ci == 0 ? wf[1][t] : wf[3][t], bop, y, 0, 0, 0);
      bop = bop1;
      bop1 = bop2;
    }
  };
  auto chain_lds = [&](f32x16& x, const bf16x8* sAk) {
    const bf16x8* wlw = wl + (size_t)wave * KSTEPS * 64;
    bf16x8 bop = sAk[lane], bop1 = sAk[64 + lane], wv = wlw[lane], wv1 = wlw[64 + lane];
#pragma unroll
    for (int t = 0; t < KSTEPS; t++) {
      const bf16x8 bop2 = (t + 2 < KSTEPS) ? sAk[(t + 2) * 64 + lane] : bop;
      const bf16x8 wv2 = (t + 2 < KSTEPS) ? wlw[(t + 2) * 64 + lane] : wv;
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, bop, x, 0, 0, 0);
      bop = bop1;
      bop1 = bop2;
      wv = wv1;
      wv1 = wv2;
    }
  };
  // accumulators seeded with the draft logits of tile i; a tile outside the workgroup's slice
  // starts at -inf, so that its values drop out of every sum below without a test there
  auto seed = [&](const u32x4 (&T)[2], int i) {
    float x[16];
    unpack16(T[0], T[1], x);
    const bool on = tile_on(i);
    f32x16 a;
#pragma unroll
    for (int q = 0; q < 16; q++) a[q] = on ? x[q] : -INFINITY;
    return a;
  };
  // word e (two target logits) of tile i; -inf outside the slice
  auto tword = [&](const u32x4 (&Tt)[5][2], int i, int e) -> uint32_t {
    return tile_on(i) ? Tt[i][e >> 2][e & 3] : 0xFF80FF80u;
  };

  // One pass over the batch's sub-blocks.  Per sub-block three MFMA groups in turn (register
  // chunk 0, register chunk 1, the LDS tile), each followed by its element-wise part:
  // EW(row, x, y, i0, two, Tt, aux) -> float2 over tiles i0 (x) and i0 + 1 (y, if two) of the
  // lane's row, CB(a, b) combines two groups' results, FL(k, row) the four waves' results of
  // sub-block k (wave 0, lanes below SUB).  AUX(row) -> float2 is loaded a sub-block ahead and
  // handed to EW.  Every tile is reloaded with the next sub-block's logits as soon as it has been
  // used (draft logits: when seeded; target logits: after their element-wise part), so that each
  // load has a whole sub-block to arrive; scheduling barriers keep the loads in place.
  // PRE(row, Tt) -> float runs beside the first MFMA chain on the target logits alone; with
  // pre_all it uses all five target tiles, which are then reloaded right after it.
  auto pass = [&](int r0, int nb, auto EW, auto CB, auto FL, auto AUX, auto PRE, bool pre_all) __attribute__((always_inline)) {
    const int nsb = (nb + SUB - 1) / SUB;
    u32x4 Tb[5][2], Tt[5][2], sv[4];
    RowIn rw = row_in(r0, nb, 0);
    stage_issue(rw.prev, sv);
    load_tiles(rs_base, rw.vb, Tb);
    load_tiles(rs_tgt, rw.vt, Tt);
    float2 ax = AUX(rw);
    stage_store(0, sv);
    __syncthreads();
    for (int k = 0; k < nsb; k++) {
      const bf16x8* sAk = sA + (size_t)(k & 1) * KSTEPS * 64;
      const RowIn rn = row_in(r0, nb, k + 1);   // rows past the batch read past both tensors
      const float2 axn = AUX(rn);
      f32x16 a0 = seed(Tb[0], 0), a1 = seed(Tb[1], 1);
      load_tile(rs_base, rn.vb, 0, Tb[0]);
      load_tile(rs_base, rn.vb, 1, Tb[1]);
      stage_issue(rn.prev, sv);
      __builtin_amdgcn_sched_barrier(0);
      chain_reg(a0, a1, 0, sAk);
      const float pre = PRE(rw, Tt);
      if (pre_all) load_tiles(rs_tgt, rn.vt, Tt);
      f32x16 a2 = seed(Tb[2], 2), a3 = seed(Tb[3], 3), a4 = seed(Tb[4], 4);
      load_tile(rs_base, rn.vb, 2, Tb[2]);
      load_tile(rs_base, rn.vb, 3, Tb[3]);
      load_tile(rs_base, rn.vb, 4, Tb[4]);
      __builtin_amdgcn_sched_barrier(0);
      // each group's element-wise part shares a scheduling region with the next group's MFMA chain
      chain_reg(a2, a3, 1, sAk);
      float2 o = EW(rw, a0, a1, 0, true, Tt, ax);
      if (!pre_all) {
        load_tile(rs_tgt, rn.vt, 0, Tt[0]);
        load_tile(rs_tgt, rn.vt, 1, Tt[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      chain_lds(a4, sAk);
      o = CB(o, EW(rw, a2, a3, 2, true, Tt, ax));
      if (!pre_all) {
        load_tile(rs_tgt, rn.vt, 2, Tt[2]);
        load_tile(rs_tgt, rn.vt, 3, Tt[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
      o = CB(o, EW(rw, a4, a4, 4, false, Tt, ax));
      if (!pre_all) load_tile(rs_tgt, rn.vt, 4, Tt[4]);
      o.y = pre_all ? pre : o.y;
      if (h == 0) red[((k & 1) * NW + wave) * SUB + m32] = o;
      if (k + 1 < nsb) stage_store(k + 1, sv);
      __syncthreads();
      if (wave == 0 && lane < SUB) FL(k, rw);
      rw = rn;
      ax = axn;
    }
    // nothing of the last (empty) prefetch is left in flight past the pass
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  uint64_t token = p.nonce;
  const int GW = G * NW;
  // alpha of the nb rows of the batch from r0: one wave per row, the workgroups' sums in a fixed
  // order (phase 4 of a batch runs in phase 2 of the next, which reads other arrays)
  auto merge2 = [&](int r0, int nb) {
    for (int lr = g * NW + wave; lr < nb; lr += GW) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < MAX_G / 64; i++) {
        const int w = lane + 64 * i;
        a += w < G ? ld_f32(&p.part2[(size_t)lr * MAX_G + w]) : 0.0f;
      }
      a = wsum(a);
      if (lane == 0) p.alpha[p.rows[r0 + lr]] = failed(p.err, p.nonce) ? NAN : a;
    }
  };
  for (int r0 = 0; r0 < n; r0 += nbr) {
    const int nb = min(nbr, n - r0);
    // ---- 1. per-workgroup log-normalisers of q (per MFMA group) and p (beside the first chain) ----
    pass(r0, nb,
         [&](const RowIn& rw, const f32x16& x, const f32x16& y, int, bool two, const u32x4 (&)[5][2], float2) -> float2 {
           const float c = rw.invT * LOG2E;
           float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
           for (int q = 0; q < 16; q += 2) {
             m0 = vmax(m0, vmax(x[q], x[q + 1]));
             if (two) m1 = vmax(m1, vmax(y[q], y[q + 1]));
           }
           const float mq = pmax32(vmax(m0, m1));
           const float oq = (mq == -INFINITY) ? 0.0f : mq * c;
           float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
           for (int q = 0; q < 16; q += 2) {
             s0 += ex2(fmaf(x[q], c, -oq));
             s1 += ex2(fmaf(x[q + 1], c, -oq));
             if (two) {
               s2 += ex2(fmaf(y[q], c, -oq));
               s3 += ex2(fmaf(y[q + 1], c, -oq));
             }
           }
           const float sq = psum32((s0 + s1) + (s2 + s3));
           const float lq = (mq == -INFINITY) ? (sq == 0.0f ? -INFINITY : NAN) : mq * rw.invT + lg2(sq) * LN2;
           return make_float2(lq, 0.0f);
         },
         [](float2 a, float2 b) { return make_float2(lse2(a.x, b.x), 0.0f); },
         [&](int k, const RowIn& rw) {
           if (rw.lr >= nb) return;
           float2 a = red[((k & 1) * NW + 0) * SUB + m32];
#pragma unroll
           for (int w = 1; w < NW; w++) {
             const float2 o = red[((k & 1) * NW + w) * SUB + m32];
             a.x = lse2(a.x, o.x);
             a.y = lse2(a.y, o.y);
           }
           float* pr = (float*)&p.part1[(size_t)rw.lr * MAX_G + g];
           st_f32(pr, a.x);
           st_f32(pr + 1, a.y);
         },
         [](const RowIn&) { return make_float2(0.0f, 0.0f); },
         [&](const RowIn& rw, const u32x4 (&Tt)[5][2]) -> float {
           const float c = rw.invT * LOG2E;
           float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
           for (int i = 0; i < 5; i++)
#pragma unroll
             for (int e = 0; e < 8; e += 2) {
               const uint32_t t0 = tword(Tt, i, e), t1 = tword(Tt, i, e + 1);
               m0 = vmax(m0, vmax(bf_lo(t0), bf_hi(t0)));
               m1 = vmax(m1, vmax(bf_lo(t1), bf_hi(t1)));
             }
           const float mp = pmax32(vmax(m0, m1));
           const float op = (mp == -INFINITY) ? 0.0f : mp * c;
           float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
           for (int i = 0; i < 5; i++)
#pragma unroll
             for (int e = 0; e < 8; e += 2) {
               const uint32_t t0 = tword(Tt, i, e), t1 = tword(Tt, i, e + 1);
               s0 += ex2(fmaf(bf_lo(t0), c, -op));
               s1 += ex2(fmaf(bf_hi(t0), c, -op));
               s2 += ex2(fmaf(bf_lo(t1), c, -op));
               s3 += ex2(fmaf(bf_hi(t1), c, -op));
             }
           const float sp = psum32((s0 + s1) + (s2 + s3));
           return (mp == -INFINITY) ? (sp == 0.0f ? -INFINITY : NAN) : mp * rw.invT + lg2(sp) * LN2;
         },
         true);
    grid_barrier(p.flags, p.err, p.nonce, G, token++, p.wait_ticks);
    // ---- 2. the rows' log-normalisers: one wave per row (and phase 4 of the previous batch) ----
    if (r0 > 0) merge2(r0 - nbr, nbr);
    for (int lr = g * NW + wave; lr < nb; lr += GW) {
      float mq = -INFINITY, mp = -INFINITY;
      float2 v[MAX_G / 64];
#pragma unroll
      for (int i = 0; i < MAX_G / 64; i++) {
        const int w = lane + 64 * i;
        const float* pr = (const float*)&p.part1[(size_t)lr * MAX_G + (w < G ? w : 0)];
        v[i] = w < G ? make_float2(ld_f32(pr), ld_f32(pr + 1)) : make_float2(-INFINITY, -INFINITY);
        mq = vmax(mq, v[i].x);
        mp = vmax(mp, v[i].y);
      }
      const float Mq = wmax(mq), Mp = wmax(mp);
      const float bq = Mq == -INFINITY ? 0.0f : Mq, bp = Mp == -INFINITY ? 0.0f : Mp;
      float sq = 0.0f, sp = 0.0f;
#pragma unroll
      for (int i = 0; i < MAX_G / 64; i++) {
        sq += ex2((v[i].x - bq) * LOG2E);
        sp += ex2((v[i].y - bp) * LOG2E);
      }
      sq = wsum(sq);
      sp = wsum(sp);
      const float lq = (Mq == -INFINITY) ? -INFINITY : Mq + lg2(sq) * LN2;
      const float lpv = (Mp == -INFINITY) ? -INFINITY : Mp + lg2(sp) * LN2;
      if (lane == 0) {
        st_f32(&p.lq[lr], lq);
        st_f32(&p.lp[lr], lpv);
        const int rid = p.rows[r0 + lr];
        if (p.o_lse_q) p.o_lse_q[rid] = lq;
        if (p.o_lse_p) p.o_lse_p[rid] = lpv;
      }
    }
    grid_barrier(p.flags, p.err, p.nonce, G, token++, p.wait_ticks);
    // ---- 3. per-workgroup sums of min(p, q) ----
    pass(r0, nb,
         [&](const RowIn& rw, const f32x16& x, const f32x16& y, int i0, bool two, const u32x4 (&Tt)[5][2], float2 ax) -> float2 {
           // min(p, q) as the smaller base-2 log-probability: p if p < q, else q
           const float c = rw.invT * LOG2E;
           const float oq = -ax.x * LOG2E, op = -ax.y * LOG2E;
           auto lmin = [](float lp2, float lq2) { return lp2 < lq2 ? lp2 : lq2; };
           float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
           for (int e = 0; e < 8; e++) {
             const uint32_t tw = tword(Tt, i0, e);
             a0 += ex2(lmin(fmaf(bf_lo(tw), c, op), fmaf(x[2 * e], c, oq)));
             a1 += ex2(lmin(fmaf(bf_hi(tw), c, op), fmaf(x[2 * e + 1], c, oq)));
             if (two) {
               const uint32_t tv = tword(Tt, i0 + 1, e);
               a0 += ex2(lmin(fmaf(bf_lo(tv), c, op), fmaf(y[2 * e], c, oq)));
               a1 += ex2(lmin(fmaf(bf_hi(tv), c, op), fmaf(y[2 * e + 1], c, oq)));
             }
           }
           return make_float2(psum32(a0 + a1), 0.0f);
         },
         [](float2 a, float2 b) { return make_float2(a.x + b.x, 0.0f); },
         [&](int k, const RowIn& rw) {
           if (rw.lr >= nb) return;
           float a = red[((k & 1) * NW + 0) * SUB + m32].x;
#pragma unroll
           for (int w = 1; w < NW; w++) a += red[((k & 1) * NW + w) * SUB + m32].x;
           st_f32(&p.part2[(size_t)rw.lr * MAX_G + g], a);
         },
         [&](const RowIn& rw) {   // the row's log-normalisers (written before the last barrier)
           const bool act = rw.lr < nb;
           return make_float2(act ? ld_f32(&p.lq[rw.lr]) : 0.0f, act ? ld_f32(&p.lp[rw.lr]) : 0.0f);
         },
         [](const RowIn&, const u32x4 (&)[5][2]) { return 0.0f; }, false);
  }
  // ---- 4. alpha of the last batch ----
  grid_barrier(p.flags, p.err, p.nonce, G, token++, p.wait_ticks);
  if (n > 0) merge2((n - 1) / nbr * nbr, n - (n - 1) / nbr * nbr);
}

}  // namespace res
}  // namespace spec

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
namespace spec {
namespace res {

// Barrier tokens of one call are nonce + i (i < 2^16).  Nonces are distinct across the calls of a
// process (a counter) and across processes (the counter starts from a hash of the time, the
// process id and an address), with the low 16 bits zero.
static uint64_t next_nonce() {
  static std::atomic<uint64_t> ctr{0};
  static const uint64_t salt = [] {
    uint64_t x = (uint64_t)time(nullptr) * 0x9E3779B97F4A7C15ull;
    x ^= (uint64_t)getpid() << 32;
    x ^= (uint64_t)(uintptr_t)&ctr;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
  }();
  uint64_t z = salt + (ctr.fetch_add(1, std::memory_order_relaxed) + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z & ~(TOKEN_WINDOW - 1);
}

// Limit of the kernels' bounded waits in s_memrealtime ticks: one second, or the decimal value of
// the environment variable SPEC_RESIDENT_WAIT_TICKS, read at every launch (a test sets 0 to force
// the timeout path: the call then ends with every request invalid instead of waiting).
static uint64_t wait_limit() {
  const char* e = getenv("SPEC_RESIDENT_WAIT_TICKS");
  if (!e || !*e) return WAIT_TICKS;
  char* end = nullptr;
  const unsigned long long v = strtoull(e, &end, 10);
  return (end && *end == 0) ? (uint64_t)v : WAIT_TICKS;
}

int launch(const Args& a_in, void* stream, void* ev_start, void* ev_stop) {
  Args a = a_in;
  a.nonce = next_nonce();
  a.wait_ticks = wait_limit();
  const Layout l = layout(a.B, a.K);
  KP p{};
  p.a = a;
  char* ws = a.ws;
  p.st = (int32_t*)(ws + l.off_state);
  p.xs = (int32_t*)(ws + l.off_xs);
  float* f = (float*)(ws + l.off_f);
  const size_t nf = (size_t)a.B * (a.K + 1);
  p.lse_q = f;
  p.logq = f + nf;
  p.lse_p = f + 2 * nf;
  p.logp = f + 3 * nf;
  p.rec_d = (float4*)(ws + l.off_rec_d);
  p.rec_c = (float4*)(ws + l.off_rec_c);
  p.rec_p = (float4*)(ws + l.off_rec_p);
  p.flags = (uint64_t*)(ws + l.off_flags);
  p.err = p.flags + (size_t)MAX_G * FLAG_STRIDE;
  p.pub = (uint64_t*)(ws + l.off_pub);
  // every workspace pointer of the kernel lies inside the workspace (a field left unset is null)
  {
    const void* wp[] = {p.st, p.xs, p.lse_q, p.logq, p.lse_p, p.logp, p.rec_d, p.rec_c, p.rec_p, p.flags, p.err, p.pub};
    for (const void* q : wp)
      if ((const char*)q < ws || (const char*)q >= ws + l.total) return SPEC_E_WORKSPACE;
  }
  const size_t lds = smem_bytes(a.B);
  // the dynamic LDS ceiling, once per device
  static std::atomic<int> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  if (dev < 0 || dev >= 64 || attr_set[dev].load(std::memory_order_acquire) == 0) {
    if (hipFuncSetAttribute((const void*)k_resident, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem_bytes(MAX_B)) != hipSuccess)
      return SPEC_E_HIP;
    if (dev >= 0 && dev < 64) attr_set[dev].store(1, std::memory_order_release);
  }
  hipStream_t st = (hipStream_t)stream;
  if (ev_start && hipEventRecord((hipEvent_t)ev_start, st) != hipSuccess) return SPEC_E_HIP;
  void* args[] = {&p};
  if (hipLaunchCooperativeKernel((const void*)k_resident, dim3(a.G), dim3(NT), args, (unsigned)lds, st) != hipSuccess)
    return SPEC_E_HIP;
  if (ev_stop && hipEventRecord((hipEvent_t)ev_stop, st) != hipSuccess) return SPEC_E_HIP;
  return SPEC_OK;
}

int launch_stats(const StatsArgs& a, void* stream) {
  const StatsLayout l = stats_layout(a.V, a.B * a.K);
  StatsKP p{};
  p.B = a.B;
  p.K = a.K;
  p.V = a.V;
  p.R = a.R;
  p.G = a.G;
  p.nbr = l.nbr;
  p.base = a.base;
  p.target = a.target;
  p.A = a.A;
  p.W = a.W;
  p.temp = a.temp;
  p.n_rows = a.n_rows;
  p.rows = a.rows;
  p.prev = a.prev;
  p.alpha = a.alpha;
  p.o_lse_q = a.o_lse_q;
  p.o_lse_p = a.o_lse_p;
  p.lq = (float*)(a.ws + l.off_lq);
  p.lp = (float*)(a.ws + l.off_lp);
  p.part1 = (float2*)(a.ws + l.off_part1);
  p.part2 = (float*)(a.ws + l.off_part2);
  p.flags = (uint64_t*)(a.ws + l.off_flags);
  p.err = p.flags + (size_t)MAX_G * FLAG_STRIDE;
  p.nonce = next_nonce();
  p.wait_ticks = wait_limit();
  static std::atomic<int> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_HIP;
  if (dev < 0 || dev >= 64 || attr_set[dev].load(std::memory_order_acquire) == 0) {
    if (hipFuncSetAttribute((const void*)k_stats_res, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)stats_smem_bytes()) != hipSuccess)
      return SPEC_E_HIP;
    if (dev >= 0 && dev < 64) attr_set[dev].store(1, std::memory_order_release);
  }
  void* args[] = {&p};
  if (hipLaunchCooperativeKernel((const void*)k_stats_res, dim3(a.G), dim3(NT), args, (unsigned)stats_smem_bytes(),
                                 (hipStream_t)stream) != hipSuccess)
    return SPEC_E_HIP;
  return SPEC_OK;
}


}  // namespace res
}  // namespace spec
