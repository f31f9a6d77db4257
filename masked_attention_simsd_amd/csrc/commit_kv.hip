// commit_kv.hip -- append the accepted drafts' key/value rows to the KV cache.
//
// SimSD pages ([nl]/[fr] Methodologie 4, Acceptance / Acceptation): the
// longest prefix accepted along the draft's temporal order is committed and
// the round repeats. Sequence s accepted the data tokens D_k with
// tau(k) <= L_s; their (already rotated) key and value rows go, in temporal
// order, to the end of the sequence's cache region, and its used length grows
// by L_s.
//
// Pure data movement (a few KB per sequence): one workgroup per (sequence,
// temporal step) copies one block row of every KV head with 16-byte loads and
// stores; the used lengths are updated by a second launch on the same stream,
// so every copy has read the old length before it changes, and the length
// array can be updated in place. Both launches check tau and the sizes the
// same way, so a sequence they reject is left untouched by both.
#include "simsd_internal.h"

namespace simsd {

namespace {

constexpr int kCommitThreads = 256;

// What both launches decide for sequence s, from the same inputs.
struct CommitPlan {
  bool ok;       // commit this sequence
  int bits;      // status bits when not
  int L, len;    // accepted drafts, used rows before the commit
  int row0;      // first cache row written (region start + len)
};

// One wave evaluates tau[s] (lane j holds tau(j+1)); `t1` is the temporal
// label whose position the caller wants (returned in *k_out, -1 if none).
__device__ __forceinline__ CommitPlan commit_plan(const CommitArgs& a, int s, int lane, int t1, int* k_out) {
  const int B = a.B;
  const int tv = lane < B ? a.tau[static_cast<size_t>(s) * B + lane] : 0;
  const bool in_range = tv >= 1 && tv <= B;
  // a permutation of 1..B: every value in range and all B bits present
  unsigned long long bits = (lane < B && in_range) ? (1ull << (tv - 1)) : 0ull;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) bits |= __shfl_xor(bits, o);
  const unsigned long long full = B == 64 ? ~0ull : ((1ull << B) - 1ull);
  const bool perm = __ballot(lane < B && !in_range) == 0ull && bits == full;
  const unsigned long long hit = __ballot(lane < B && tv == t1);
  *k_out = hit ? __builtin_ctzll(hit) : -1;

  CommitPlan p{};
  p.L = a.accept_len[s];
  p.len = a.lens[s];
  const int o0 = a.offsets[s], o1 = a.offsets[s + 1];
  const int cap = o1 - o0;
  // the region must lie inside the cache, and L more rows must fit after len
  const bool region = o0 >= 0 && o1 >= o0 && o1 <= a.offsets[a.b];
  const bool fits = region && p.L >= 0 && p.L <= B && p.len >= 0 && p.len <= cap && p.L <= cap - p.len;
  p.ok = perm && fits;
  p.bits = !perm ? kDevBadTau : (!fits ? kDevCommitOverflow : 0);
  p.row0 = o0 + p.len;
  return p;
}

// Grid (b, B): workgroup (s, t) copies the draft with temporal label t + 1,
// if it was accepted.
__global__ __launch_bounds__(kCommitThreads) void commit_rows_kernel(CommitArgs a) {
  const int s = blockIdx.x, t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  int k;
  const CommitPlan p = commit_plan(a, s, lane, t + 1, &k);
  if (!p.ok || t >= p.L) return;

  // one block row of every KV head, K then V, in 16-byte pieces
  const int per_head = a.d / 8;
  const int per_tensor = a.Hkv * per_head;
  const size_t C = static_cast<size_t>(a.offsets[a.b]);
  const size_t dst_row = static_cast<size_t>(p.row0) + t;
  for (int i = threadIdx.x; i < 2 * per_tensor; i += kCommitThreads) {
    const int tensor = i >= per_tensor;
    const int c = i - tensor * per_tensor;
    const int h = c / per_head, piece = c % per_head;
    const uint16_t* src = (tensor ? a.v_blk : a.k_blk) +
                          ((static_cast<size_t>(s) * 2 * a.B + k) * a.Hkv + h) * a.d + piece * 8;
    uint16_t* dst = (tensor ? a.v_cache : a.k_cache) +
                    (a.head_major ? (static_cast<size_t>(h) * C + dst_row) * a.d
                                  : (dst_row * a.Hkv + h) * a.d) +
                    piece * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// One wave per sequence: the new used length, and the status bits.
__global__ __launch_bounds__(kCommitThreads) void commit_lens_kernel(CommitArgs a) {
  const int s = blockIdx.x * (kCommitThreads / 64) + (threadIdx.x >> 6);
  if (s >= a.b) return;
  const int lane = threadIdx.x & 63;
  int k;
  const CommitPlan p = commit_plan(a, s, lane, 0, &k);
  if (lane == 0) {
    if (p.ok) a.lens[s] = p.len + p.L;
    if (a.status && p.bits) atomicOr(&a.status[s], p.bits);
  }
}

}  // namespace

hipError_t launch_commit_kv(const CommitArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(commit_rows_kernel, dim3(static_cast<unsigned>(a.b), static_cast<unsigned>(a.B)),
                     dim3(kCommitThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned waves_per_wg = kCommitThreads / 64;
  hipLaunchKernelGGL(commit_lens_kernel, dim3((static_cast<unsigned>(a.b) + waves_per_wg - 1) / waves_per_wg),
                     dim3(kCommitThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace simsd
