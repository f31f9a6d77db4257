// commit_kv.hip -- append the accepted drafts' key/value rows to the KV cache.
//
// SimSD pages ([nl]/[fr] Methodologie 4, Acceptance / Acceptation): the
// longest prefix accepted along the draft's temporal order is committed and
// the round repeats. Sequence s accepted the data tokens D_k with
// tau(k) <= L_s; their (already rotated) key and value rows go, in temporal
// order, to the end of the sequence's cache region, and its used length grows
// by L_s.
//
// The same launch writes the positions the next round verifies (the block's
// still-open positions, the rejected one first, then fresh ones), so a round
// loop runs on the device without a host round trip.
//
// Pure data movement (a few KB per sequence, latency bound): one workgroup
// per sequence. Wave 0 checks tau, inverts it in LDS and decides whether the
// sequence can be committed; then every thread copies its 16-byte pieces of
// the accepted rows (all K and V heads of a row are contiguous), up to eight
// rows' loads in flight before their stores, and the workgroup advances the
// used length. Only this workgroup reads or writes the sequence's length, so
// the length array can be updated in place within the one launch.
#include "simsd_internal.h"

#include <climits>

namespace simsd {

namespace {

constexpr int kCommitThreads = 256;
constexpr int kRowsInFlight = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte piece

__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(CommitArgs a) {
  __shared__ int inv[64];  // inv[t] = 0-based position with temporal label t + 1
  __shared__ int sh_L, sh_len, sh_row0, sh_bits;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.B;

  if (tid < 64) {
    const bool valid = lane < B;
    const int tv = valid ? a.tau[static_cast<size_t>(s) * B + lane] : 0;
    const int pv = (a.next_pos && valid) ? a.pos[static_cast<size_t>(s) * B + lane] : 0;
    const bool in_range = tv >= 1 && tv <= B;
    // a permutation of 1..B: every label in range and all B label bits present
    // (the lanes' labels read with readlane in a uniform loop: B <= 64 scalar
    // reads, no LDS permutes)
    unsigned long long bits = 0ull;
    for (int t = 0; t < B; ++t) {
      const int lt = __builtin_amdgcn_readlane(tv, t);
      bits |= (lt >= 1 && lt <= B) ? (1ull << (lt - 1)) : 0ull;
    }
    const unsigned long long full = B == 64 ? ~0ull : ((1ull << B) - 1ull);
    const bool perm = __ballot(valid && !in_range) == 0ull && bits == full;
    if (perm && valid) inv[tv - 1] = lane;
    // the same values in every lane (one address each)
    const int L = a.accept_len[s], len = a.lens[s];
    const int o0 = a.offsets[s], o1 = a.offsets[s + 1];
    const int cap = o1 - o0;
    // the region must lie inside the cache, and L more rows must fit after len
    const bool region = o0 >= 0 && o1 >= o0 && o1 <= a.offsets[a.b];
    const bool fits = region && L >= 0 && L <= B && len >= 0 && len <= cap && L <= cap - len;
    const int fail = !perm ? kDevBadTau : (!fits ? kDevCommitOverflow : 0);
    if (lane == 0) sh_bits = fail, sh_L = L, sh_len = len, sh_row0 = o0 + len;
    if (a.next_pos) {
      // The next round's positions: the B smallest not in the cache. When L <
      // B the rejected step's position comes first (its correction token is
      // committed but has no key/value row yet), then the other open
      // positions (label > L + 1) in increasing order (ties by pair index),
      // then L positions following the block's largest. A sequence that
      // commits nothing keeps its block.
      int* nx = a.next_pos + static_cast<size_t>(s) * B;
      int pmax = INT_MIN;
      int rank = 0;
      for (int t = 0; t < B; ++t) {
        const int pt = __builtin_amdgcn_readlane(pv, t), tt = __builtin_amdgcn_readlane(tv, t);
        pmax = max(pmax, pt);
        rank += (tt > L + 1 && (pt < pv || (pt == pv && t < lane))) ? 1 : 0;
      }
      const bool corr = valid && tv == L + 1;
      const bool open = valid && tv > L + 1;
      if (valid) {
        if (fail) {
          nx[lane] = pv;
        } else {
          if (corr) nx[0] = pv;
          if (open) nx[(L < B ? 1 : 0) + rank] = pv;
          if (lane < L) nx[B - L + lane] = pmax + 1 + lane;
        }
      }
    }
  }
  __syncthreads();
  if (sh_bits) {
    if (tid == 0 && a.status) atomicOr(&a.status[s], sh_bits);
    return;  // nothing of this sequence is written, its length is kept
  }
  const int L = sh_L;

  // pieces of one block row: K then V, every head, 16 bytes each
  const int per_head = a.d / 8;
  const int per_tensor = a.Hkv * per_head;
  const int pieces = 2 * per_tensor;
  const size_t C = static_cast<size_t>(a.offsets[a.b]);
  for (int i = tid; i < pieces; i += kCommitThreads) {
    const int tensor = i >= per_tensor;
    const int c = i - tensor * per_tensor;
    const int h = c / per_head, piece = c % per_head;
    const uint16_t* src = (tensor ? a.v_blk : a.k_blk) +
                          (static_cast<size_t>(s) * 2 * B * a.Hkv + h) * a.d + piece * 8;
    // cache row `row` of head h: token-major (row Hkv + h) d, head-major (h C + row) d,
    // both times 2 with the paired layout (key and value rows adjacent)
    const size_t rstride = static_cast<size_t>(a.pair) *
                           (a.head_major ? static_cast<size_t>(a.d) : static_cast<size_t>(a.Hkv) * a.d);
    uint16_t* dst = (tensor ? a.v_cache : a.k_cache) +
                    static_cast<size_t>(a.pair) *
                        (a.head_major ? static_cast<size_t>(h) * C * a.d : static_cast<size_t>(h) * a.d) +
                    piece * 8;
    for (int t0 = 0; t0 < L; t0 += kRowsInFlight) {
      // Slots past L repeat the last accepted row: they load it and store the
      // same bytes to its own place again (same thread, same value), so both
      // loops are branch-free and the batch stays in registers.
      u32x4 v[kRowsInFlight];
#pragma unroll
      for (int r = 0; r < kRowsInFlight; ++r) {
        const int t = min(t0 + r, L - 1);
        v[r] = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(inv[t]) * a.Hkv * a.d);
      }
#pragma unroll
      for (int r = 0; r < kRowsInFlight; ++r) {
        const size_t row = static_cast<size_t>(sh_row0) + min(t0 + r, L - 1);
        *reinterpret_cast<u32x4*>(dst + row * rstride) = v[r];
      }
    }
  }
  if (tid == 0) a.lens[s] = sh_len + L;
}

}  // namespace

hipError_t launch_commit_kv(const CommitArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kv_kernel, dim3(static_cast<unsigned>(a.b)), dim3(kCommitThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace simsd
