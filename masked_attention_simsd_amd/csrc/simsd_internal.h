// simsd_internal.h -- device helpers and launcher declarations shared by the
// gfx950 kernels of libsimsd. Internal to the library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace simsd {

constexpr int kWave = 64;
constexpr int kMaxSeqCounters = 65536;  // counter words at the start of a workspace

// Device status bits (the same values as SIMSD_DEV_* in simsd.h).
constexpr int kDevBadTau = 1;
constexpr int kDevZeroResidual = 2;
constexpr int kDevQZero = 4;
constexpr int kDevBadToken = 8;
constexpr int kDevBadPrefix = 16;
constexpr int kDevSyncTimeout = 32;
constexpr int kDevCommitOverflow = 64;

// bf16 <-> fp32. bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays NaN (quiet). Branch-free (selects), so
// it costs the same in every lane.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = (u >> 16) | 0x40u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? qnan : rne);
}

// fp64 -> bf16 with a single rounding (nearest even). The double is first
// narrowed to fp32 with round-to-odd, which keeps enough information for the
// second, nearest-even narrowing to equal a direct one (fp32 carries 16 more
// significand bits than bf16). Branch-free.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const float f = static_cast<float>(x);  // nearest even
  const double back = static_cast<double>(f);
  const uint32_t u = __float_as_uint(f);
  // inexact, finite result: step toward zero if nearest-even overshot in
  // magnitude, then force the last bit to 1 (round to odd)
  const bool adjust = back != x && !__builtin_isnan(x) && !__builtin_isinf(f);
  const uint32_t down = __builtin_fabs(back) > __builtin_fabs(x) ? 1u : 0u;
  const uint32_t odd = (u - down) | 1u;
  return f32_to_bf16(__uint_as_float(adjust ? odd : u));
}

// RoPE arithmetic shared by the RoPE-copy kernel and the attention kernel's
// fused prologue, so both round identically: the frequencies base^(-2i/d)
// come from the host (fp64, once per call), the angle is pos * frequency,
// cos/sin and the pair rotation are fp64 (explicit fma, no contraction left
// to the compiler), and each output is rounded to bf16 once.
constexpr int kMaxRopeFreqs = 64;  // d/2 for d <= 128
__device__ __forceinline__ void rope_rotate(uint16_t xa, uint16_t xb, double co, double si,
                                            uint16_t* ra, uint16_t* rb) {
  const double a = bf16_to_f32(xa), b = bf16_to_f32(xb);
  *ra = f64_to_bf16(__builtin_fma(a, co, -(b * si)));
  *rb = f64_to_bf16(__builtin_fma(b, co, a * si));
}

struct RopeArgs {
  uint16_t* q;
  uint16_t* k;
  const int32_t* start_pos;  // [b] (pair k at start_pos[s] + k), or [b][B] positions
  int b, B, Hq, Hkv, d;
  int interleaved, no_copy;
  int positions;  // 1: start_pos holds one position per pair ([b][B])
  double inv_freq[kMaxRopeFreqs];  // base^(-2i/d), i < d/2
};

struct AttnArgs {
  const uint16_t* q_blk;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_pre;
  const uint16_t* v_pre;
  const int32_t* offsets;
  const int32_t* tau;
  void* out;
  float* lse;
  int32_t* status;
  float* part_o;      // [unit_slice][split][wave][qb][dblk][lane] x 4 floats
  float* part_ml;     // [unit_slice][split][row] x (m, l)
  int32_t* counters;  // [unit_slice]
  int b, B, Hq, Hkv, G, d;
  int row0, nrows;    // block rows computed: [row0, row0 + nrows)
  int M;              // query rows per (sequence, KV head) = nrows * G
  int row_slices;     // ceil(M / rows per workgroup)
  int chunk;          // prefix keys per split (multiple of the key tile)
  int shift;          // split 0 runs chunk - shift keys, split k >= 1 starts at k * chunk - shift (-1: the launch picks)
  int nsplit;         // splits per (sequence, KV head, row slice)
  int max_prefix;
  int total_real;     // b * Hkv * row_slices * nsplit
  int total_grid;     // total_real rounded up to a multiple of 8
  float scale_log2;   // softmax scale * log2(e)
  int data_rule;      // 0 causal, 1 bidirectional, 2 skip data rows
  int out_f32;
  int xcd_remap;      // 1: workgroup ids remapped so a unit's splits share an XCD
  int rotate;         // 1: each unit starts its prefix walk at its own tile
  int lpt;            // 1: unsplit launch, workgroups dispatched first take the longest sequences
  int kv_head_major;  // prefix cache layout: 0 [sum P][Hkv][d], 1 [Hkv][sum P][d]
  int kv_pair;        // 2 with the paired layout (key and value rows adjacent), else 1
  // RoPE-copy fused into the prologue (rope != 0): query rows and block key
  // rows are rotated on the fly; the rotated block keys go to k_rot if set
  int rope;
  const int32_t* start_pos;  // [b], or [b][B] positions with rope_positions
  int rope_interleaved, rope_no_copy, rope_positions;
  uint16_t* k_rot;
  double rope_inv_freq[kMaxRopeFreqs];  // base^(-2i/d), i < d/2
  // explicit block mask (mask_mode): bit c of word c/64 of row r's
  // mask_words words says whether row r sees block key c; no tau
  int mask_mode;
  int nblk;  // block rows (and keys) per sequence: R (2B without a mask)
  const uint64_t* block_mask;  // [b][nblk][mask_words]
  int mask_words;
  // rows in use of each region [offsets[s], offsets[s+1]): prefix_lens[s], or,
  // with prefix_lens_are_ends (prefix_lens = offsets + 1, a packed cache),
  // prefix_lens[s] - offsets[s]
  const int32_t* prefix_lens;
  int prefix_lens_are_ends;
};

struct CommitArgs {
  const uint16_t* k_blk;  // [b][2B][Hkv][d]
  const uint16_t* v_blk;
  const int32_t* tau;         // [b][B]
  const int32_t* accept_len;  // [b]
  uint16_t* k_cache;          // [C][Hkv][d] or [Hkv][C][d], C = offsets[b]
  uint16_t* v_cache;
  const int32_t* offsets;  // [b+1] region bounds
  int32_t* lens;           // [b] used rows, updated in place
  const int32_t* pos;      // [b][B] positions of this round's pairs (with next_pos)
  int32_t* next_pos;       // [b][B] positions of the next round, or null
  int32_t* status;
  int b, B, Hkv, d;
  int head_major;
  int pair;  // 2 with the paired layout (key and value rows adjacent), else 1
};

struct AttnPlan {
  int nwc, qb;        // compute waves and 16-row query blocks per wave
  int pipe;           // key-tile pipeline variant (keys per tile x ring stages)
  int xcd_remap;
  int rotate;
  int lpt;
  int rows_per_wg;
  int row_slices;
  int chunk, nsplit, shift;
  size_t counters_bytes, ml_bytes, o_bytes, total_bytes;
};

struct AcceptArgs {
  const float* p;
  const float* q;
  const int32_t* draft;
  const int32_t* tau;
  const float* u;
  int b, B, V;
  int32_t* accept_len;
  int32_t* correction;
  int32_t* status;
  int32_t* counters;  // [b], zero between calls
  double* seg_sum;    // [b][segments] published residual mass words (ready bit), zero between calls
  // Logits input (simsd_accept_logits): p and q are the row softmaxes of zt
  // and zd at temperature 1 / inv_t, evaluated where needed from the row
  // statistics (max, sum of exp) the row-statistics pass leaves in row_stats.
  const float* zt;
  const float* zd;
  double* row_stats;              // [2][b][B] x (max, 1 / sum, logit at the draft token, 0): target rows, then draft rows
  double inv_t;
  int32_t* row_counters;          // [2 b B], zero between calls
  unsigned long long* row_words;  // [2 b B][nseg1] x (max, sum) with ready bits, zero between calls
  int nseg1;                      // vocabulary segments per row of the statistics pass
};

int accept_segments(int V);

constexpr int kMaxAcceptVocab = 1 << 21;  // vocabulary entries per row the acceptance kernel takes

constexpr int kAttnTileKeys = 64;  // keys staged per tile
constexpr int kMaxPrefix = 1 << 30; // largest max_prefix (key counts stay far from int overflow)
constexpr long kMaxRopeTableBytes = 64 * 1024;  // fused RoPE cos/sin table (LDS beside the key ring)
constexpr int kAttnMaxUnits = kMaxSeqCounters;  // (sequence, KV head, row slice) units per call

// Tuning overrides set through simsd_set_tuning (process-wide, default -1 =
// the plan's own choice). Keys are the SIMSD_TUNE_* values of simsd.h.
int tuning(int key);

AttnPlan plan_attention(int b, int B, int Hq, int Hkv, int d, int max_prefix, int data_rule);
// the same for `nrows` computed query rows per sequence (explicit-mask calls)
AttnPlan plan_attention_rows(int b, int nrows, int Hq, int Hkv, int d, int max_prefix);

hipError_t launch_rope_copy(const RopeArgs& a, hipStream_t stream);
hipError_t launch_verify_attention(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);
hipError_t launch_commit_kv(const CommitArgs& a, hipStream_t stream);
// acceptance from logits: the row-statistics pass, then the acceptance kernel
// in logits mode (same stream)
hipError_t launch_accept_logits(const AcceptArgs& a, hipStream_t stream);
constexpr int kRowStatSeg = 4096;  // smallest statistics segment (sizes the workspace)
// rows x segments of one statistics pass: its grid of 256-thread workgroups
// must stay below 2^32 work-items, the dispatch's limit per dimension
constexpr long kMaxRowStatUnits = (1L << 24) - 1;

}  // namespace simsd
