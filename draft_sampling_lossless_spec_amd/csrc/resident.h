// resident.h -- the W-resident speculation cycle: one persistent launch per cycle in which every
// workgroup keeps its slice of the Markov output factor W on chip (accumulation registers and
// LDS) for all steps of the cycle.  Shared by the kernel source and the host dispatch.
//
// Vocabulary partition.  The vocabulary is cut into 64-column noise chunks; workgroup g of a grid
// of G owns chunks [cbeg(g), cbeg(g) + nch(g)), the first (nchunks % G) workgroups one more than
// the rest.  Within a workgroup, wave w keeps workgroup-local chunks 2w and 2w + 1 in its
// accumulation registers (MFMA A operands), and local chunks 8 and 9 live in LDS as four 32-column
// tiles, tile u processed by wave u.  So a workgroup holds at most RES_MAX_CHUNKS chunks.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "spec_cycle.h"

namespace spec {
namespace res {

constexpr int NT = 256;                 // threads per workgroup: 4 waves, one per SIMD
constexpr int NW = NT / 64;
constexpr int CH = 64;                  // noise chunk width (columns)
constexpr int AG_CHUNKS = 2;            // chunks per wave in accumulation registers
constexpr int LDS_CHUNKS = 2;           // chunks per workgroup in LDS
constexpr int MAX_CHUNKS = NW * AG_CHUNKS + LDS_CHUNKS;   // 10
constexpr int SUB = 32;                 // rows per MFMA sub-block
constexpr int TP = 4096;                // columns of a plain-row item (one wave: 8 loads of 1 KiB)
constexpr int KSTEPS = 16;              // k-steps of 16 in the rank (R <= 256)
constexpr int MAX_G = 256;              // workgroups (one per CU of a gfx950)
constexpr int MAX_B = 1024;
constexpr int MAX_K = 32;
constexpr int FLAG_STRIDE = 2;          // uint64 words between two workgroups' barrier flags
constexpr int PUB_WORDS = 4;            // uint64 words a merge publishes per request and step (3 used)

__host__ __device__ constexpr int n_chunks(int V) { return (V + CH - 1) / CH; }
__host__ __device__ constexpr int chunks_of(int g, int G, int V) {
  return n_chunks(V) / G + (g < n_chunks(V) % G ? 1 : 0);
}
__host__ __device__ constexpr int chunk_begin(int g, int G, int V) {
  return g * (n_chunks(V) / G) + (g < n_chunks(V) % G ? g : n_chunks(V) % G);
}
// bias slots: DRAFT rows from 0, CORRECT rows from the next multiple of SUB (no sub-block mixes)
__host__ __device__ constexpr int max_bias_slots(int B) { return 2 * B + 2 * SUB; }

// record areas (bytes)
__host__ __device__ constexpr size_t rec_d_bytes(int B) { return 16 * (size_t)max_bias_slots(B) * NW * MAX_G; }
__host__ __device__ constexpr size_t rec_c_bytes(int B) { return 16 * (size_t)(B + SUB) * NW * MAX_G; }
__host__ __device__ constexpr size_t rec_p_bytes(int B) { return 16 * (size_t)B * MAX_G; }

// Workspace of the resident cycle (offsets in bytes from the workspace base, 256-byte aligned).
struct Layout {
  size_t off_state;    // per-request int32 [6][B]: L, acc, phase, roles (two step parities), valid
  size_t off_xs;       // int32 [B][K]: drafted tokens
  size_t off_f;        // fp32 [4][B][K+1]: lse_q, logq, lse_p, logp
  size_t off_rec_d;    // float4 [bias slots][NW][MAX_G]: per-wave records of bias rows
  size_t off_rec_c;    // float4 [B + SUB][NW][MAX_G]: CORRECT rows' target-row records, indexed
                       // from the first CORRECT slot
  size_t off_rec_p;    // float4 [B][MAX_G]: plain-row item records (ceil(V / TP) <= MAX_G items)
  size_t off_flags;    // uint64 [G][FLAG_STRIDE]: grid-barrier flags; uint64 [2]: error word
  size_t off_pub;      // uint64 [2][B][PUB_WORDS]: what each request's merge hands to the next
                       // step (two step parities)
  size_t total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline Layout layout(int B, int K) {
  Layout l;
  size_t o = 0;
  l.off_state = o; o = align256(o + 4 * (size_t)6 * B);
  l.off_xs = o; o = align256(o + 4 * (size_t)B * K);
  l.off_f = o; o = align256(o + 4 * (size_t)4 * B * (K + 1));
  l.off_rec_d = o; o = align256(o + rec_d_bytes(B));
  l.off_rec_c = o; o = align256(o + rec_c_bytes(B));
  l.off_rec_p = o; o = align256(o + rec_p_bytes(B));
  l.off_flags = o; o = align256(o + 8 * (size_t)(MAX_G * FLAG_STRIDE + 2));
  l.off_pub = o; o = align256(o + 8 * (size_t)2 * B * PUB_WORDS);
  l.total = o;
  return l;
}

// Arguments of one resident cycle (device pointers; see spec_cycle in spec_cycle.h).
struct Args {
  int B, K, V, R;
  const void* base;
  const void* target;
  const void* A;
  const void* W;
  const int32_t* x0;
  const float* conf;
  const float* temp;
  const int32_t* L_in;     // verify lengths from a scheduler, or null: the prefix cut
  float threshold;
  uint64_t seed;
  int64_t req_off;
  int32_t* accepted_len;
  int32_t* tokens;
  int32_t* d_verify_len;
  int32_t* d_draft;
  float* d_logq;
  float* d_logp;
  char* ws;
  uint64_t nonce;          // per-call value: barrier tokens are nonce + i, unique across calls
  uint64_t wait_ticks;     // limit of every bounded wait, s_memrealtime ticks (100 MHz)
  int G;                   // workgroups
};

// A byte offset past every logit tensor the resident kernels take (they take tensors of at most
// this many bytes): buffer loads there read zeros without a memory access, and the largest tile
// offset added to it stays below 2^32.
constexpr uint32_t PAST_END = 0xFFF00000u;

// Does the resident cycle take these dimensions on a device with G compute units?
__host__ __device__ inline bool eligible(int B, int K, int V, int R, int dtype, int noise, int G) {
  if (dtype != SPEC_BF16 || noise != SPEC_NOISE_CHUNKED) return false;
  if (V % CH != 0 || R % 16 != 0 || R > 256 || G < 1 || G > MAX_G) return false;
  if (B < 1 || B > NW * G || B > MAX_B || K < 1 || K > MAX_K) return false;
  // logit tensors up to PAST_END bytes and A below 2 GiB: their loads use 32-bit byte offsets
  if ((size_t)B * (K + 1) * V * 2 > (size_t)PAST_END || (size_t)V * R * 2 >= ((size_t)1 << 31)) return false;
  return (n_chunks(V) + G - 1) / G <= MAX_CHUNKS && (V + TP - 1) / TP <= MAX_G;
}

// ---- acceptance statistics with W on chip ----
// Listed rows go in batches whose base and target logits (4 V bytes a row) fit in this many bytes
// of the Infinity Cache, so that the second pass over a batch finds them there.
constexpr size_t STATS_BATCH_BYTES = (size_t)160 << 20;

__host__ __device__ inline bool stats_eligible(int B, int K, int V, int R, int dtype, int G) {
  if (dtype != SPEC_BF16 || V % CH != 0 || R % 16 != 0 || R > 256 || G < 1 || G > MAX_G) return false;
  if (B < 1 || K < 1) return false;
  if ((size_t)B * (K + 1) * V * 2 > (size_t)PAST_END || (size_t)V * R * 2 >= ((size_t)1 << 31)) return false;
  return (n_chunks(V) + G - 1) / G <= MAX_CHUNKS;
}

// workspace of the statistics kernel (offsets from its base, 256-byte aligned); n: B K rows
struct StatsLayout {
  int nbr;             // listed rows per batch (a multiple of SUB)
  size_t off_lq, off_lp, off_part1, off_part2, off_flags, total;
};
__host__ __device__ inline StatsLayout stats_layout(int V, int n) {
  StatsLayout l;
  const size_t per = STATS_BATCH_BYTES / ((size_t)4 * (size_t)(V > 0 ? V : 1));
  size_t nbr = per / SUB * SUB;
  const size_t cap = ((size_t)(n > 0 ? n : 1) + SUB - 1) / SUB * SUB;
  if (nbr < SUB) nbr = SUB;
  if (nbr > cap) nbr = cap;
  l.nbr = (int)nbr;
  size_t o = 0;
  l.off_lq = o; o = align256(o + 4 * nbr);
  l.off_lp = o; o = align256(o + 4 * nbr);
  l.off_part1 = o; o = align256(o + 8 * nbr * MAX_G);
  l.off_part2 = o; o = align256(o + 4 * nbr * MAX_G);
  l.off_flags = o; o = align256(o + 8 * (size_t)(MAX_G * FLAG_STRIDE + 2));
  l.total = o;
  return l;
}

// Arguments of one statistics launch (device pointers; see spec_accept_stats in spec_cycle.h).
// n_rows, rows and prev are the listed drafted positions (written by the list kernel before).
struct StatsArgs {
  int B, K, V, R, G;
  const void* base;
  const void* target;
  const void* A;
  const void* W;
  const float* temp;
  const int32_t* n_rows;
  const int32_t* rows;
  const int32_t* prev;
  float* alpha;
  float* o_lse_q;
  float* o_lse_p;
  char* ws;                // stats_layout(V, B K).total bytes
};

}  // namespace res
}  // namespace spec

// Host side of the resident cycle (launch is defined in cycle_resident.hip).
namespace spec {
namespace res {
// Enqueue one resident cycle on `stream` (a hipStream_t); ev_start / ev_stop (hipEvent_t, may be
// null) are recorded around the launch.  Returns SPEC_OK or SPEC_E_HIP.
int launch(const Args& a, void* stream, void* ev_start, void* ev_stop);
// Enqueue the statistics of the listed rows (one cooperative launch of G workgroups).  Returns
// SPEC_OK or SPEC_E_HIP.
int launch_stats(const StatsArgs& a, void* stream);
inline size_t workspace_bytes(int B, int K) { return layout(B, K).total; }
}  // namespace res
}  // namespace spec
