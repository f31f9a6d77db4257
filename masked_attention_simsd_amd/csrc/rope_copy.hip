// rope_copy.hip -- RoPE over the paired block with the copy rule.
//
// SimSD pages ([nl] "Technische Samenvatting: SimSD - Simple Speculative
// Decoding in Diffusion Language Models" and [fr] "SimSD: Simple Speculative
// Decoding in Diffusion Language Models", Methodologie 3): the mask slot D~_k
// takes the rotary position of its paired data token D_k. The pair's
// position is start + k, or given per pair (a later round of a block
// re-verifies the positions still open, wherever they lie). The kernel makes
// that literal: a workgroup owns response position k of one sequence (and a
// chunk of heads), evaluates the d/2 rotation angles of that position once,
// and applies the same angles to the rows of both D_k and D~_k, for query and
// KV heads.
//
// The kernel is bound by latency and HBM traffic (one read + one write of the
// block's Q and K); the head dimension of the grid gives every thread a single
// rotation. fp64 is used for angles, cos/sin and the rotation, and each output
// is rounded to bf16 once (the frequencies base^(-2i/d) are computed on the
// host in fp64 and passed in the arguments).
#include "simsd_internal.h"

#include <algorithm>

namespace simsd {

namespace {

constexpr int kRopeThreads = 256;
typedef __attribute__((address_space(1))) uint16_t gu16;  // global memory
constexpr int kMaxHalf = 64;  // d <= 128

// One thread rotates 4 consecutive pairs of one head row: rotate-half pairs
// (i, i + half) come as two 8-byte pieces, interleaved pairs (2i, 2i+1) as one
// 16-byte piece. The row is loaded first (before the angles are known) so the
// memory latency overlaps the fp64 angle evaluation.
struct Pairs4 {
  uint32_t w[4];
};

__device__ __forceinline__ Pairs4 load4(const uint16_t* row, int i0, int half, bool interleaved) {
  // two 8-byte pieces in either layout (rotate-half: elements i0.. and
  // half+i0..; interleaved: the 16 contiguous bytes from 2 i0), so the number
  // of loads does not depend on the layout and the angle inputs loaded before
  // them can be waited for alone
  const int o0 = interleaved ? 2 * i0 : i0;
  const int o1 = interleaved ? 2 * i0 + 4 : half + i0;
  const uint2 lo = *reinterpret_cast<const uint2*>(row + o0);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + o1);
  Pairs4 v;
  v.w[0] = lo.x, v.w[1] = lo.y, v.w[2] = hi.x, v.w[3] = hi.y;
  return v;
}

__device__ __forceinline__ uint16_t lo16(uint32_t w) { return static_cast<uint16_t>(w); }
__device__ __forceinline__ uint16_t hi16(uint32_t w) { return static_cast<uint16_t>(w >> 16); }

__device__ __forceinline__ void rotate_store4(uint16_t* row, int i0, int half, bool interleaved,
                                              const Pairs4& v, const double* cs, const double* sn) {
  if (!interleaved) {
    // element j of the first half pairs with element j of the second half
    const uint16_t a[4] = {lo16(v.w[0]), hi16(v.w[0]), lo16(v.w[1]), hi16(v.w[1])};
    const uint16_t c[4] = {lo16(v.w[2]), hi16(v.w[2]), lo16(v.w[3]), hi16(v.w[3])};
    uint16_t ra[4], rc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rope_rotate(a[j], c[j], cs[i0 + j], sn[i0 + j], &ra[j], &rc[j]);
    *reinterpret_cast<uint2*>(row + i0) = make_uint2(ra[0] | (static_cast<uint32_t>(ra[1]) << 16),
                                                     ra[2] | (static_cast<uint32_t>(ra[3]) << 16));
    *reinterpret_cast<uint2*>(row + half + i0) = make_uint2(rc[0] | (static_cast<uint32_t>(rc[1]) << 16),
                                                            rc[2] | (static_cast<uint32_t>(rc[3]) << 16));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint16_t r0, r1;
      rope_rotate(lo16(v.w[j]), hi16(v.w[j]), cs[i0 + j], sn[i0 + j], &r0, &r1);
      w[j] = r0 | (static_cast<uint32_t>(r1) << 16);
    }
    *reinterpret_cast<uint4*>(row + 2 * i0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Grid: (sequence, position k) x head chunks. Threads of a workgroup each own
// one group of 4 pairs of one row (D_k or D~_k) of one head, so every thread
// does a single independent load / rotate / store.
__global__ __launch_bounds__(kRopeThreads) void rope_copy_kernel(RopeArgs a, int heads_per_wg) {
  __shared__ double cs_d[kMaxHalf], sn_d[kMaxHalf];  // angles of D_k
  __shared__ double cs_t[kMaxHalf], sn_t[kMaxHalf];  // angles of D~_k (only with no_copy)
  const int s = blockIdx.x / a.B;
  const int k = blockIdx.x % a.B;  // 0-based response position
  const int half = a.d / 2;
  const int tid = threadIdx.x;
  // this thread's item: (row slot, head in this chunk, group of 4 pairs)
  const int groups = half / 4;
  const int heads = a.Hq + a.Hkv;
  const int h0 = blockIdx.y * heads_per_wg;
  const int nh = min(heads_per_wg, heads - h0);
  const int items = 2 * nh * groups;
  const bool active = tid < items;  // heads_per_wg is chosen so items <= blockDim
  // threads past the items load item 0's row (never stored): every load is
  // unconditional, so the wait for the angle inputs can leave the rows in flight
  const int it = active ? tid : 0;
  const int grp = it % groups;
  const int hh = h0 + (it / groups) % nh;
  const int slot = it / (groups * nh);  // 0: D_k, 1: D~_k
  const int r = k + slot * a.B;
  // The angle inputs (this thread's frequency, the sequence's start position)
  // are requested before the row, so that waiting for them does not also wait
  // for the row (loads complete in issue order) and the fp64 angle evaluation
  // overlaps the row's latency.
  const double inv_freq = a.inv_freq[min(tid, half - 1)];
  // the pair's position: start + k, or its own entry of a [b][B] position array
  const int pidx = a.positions ? s * a.B + k : s;
  const long pos_d = static_cast<long>(a.start_pos[pidx]) + (a.positions ? 0 : k);
  // The two base pointers are pinned to scalar registers before the per-lane
  // select: selecting between the two argument slots instead would turn into a
  // per-lane load of the pointer itself, a full memory round trip before the
  // row load can be issued.
  gu16* qbase = (gu16*)a.q;
  gu16* kbase = (gu16*)a.k;
  asm volatile("" : "+s"(qbase), "+s"(kbase));
  gu16* grow = hh < a.Hq ? qbase + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hq + hh) * a.d
                         : kbase + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hkv + (hh - a.Hq)) * a.d;
  uint16_t* row = (uint16_t*)grow;
  const Pairs4 v = load4(row, grp * 4, half, a.interleaved != 0);

  if (tid < half) {
    double ang = static_cast<double>(pos_d) * inv_freq;
    sincos(ang, &sn_d[tid], &cs_d[tid]);
    if (a.no_copy) {
      ang = static_cast<double>(pos_d + a.B) * inv_freq;
      sincos(ang, &sn_t[tid], &cs_t[tid]);
    }
  }
  __syncthreads();
  if (active) {
    const bool use_t = slot && a.no_copy;
    rotate_store4(row, grp * 4, half, a.interleaved != 0, v, use_t ? cs_t : cs_d, use_t ? sn_t : sn_d);
  }
}

}  // namespace

hipError_t launch_rope_copy(const RopeArgs& a, hipStream_t stream) {
  // one thread per (row slot, head, 4-pair group): 2 * groups items per head,
  // at most kRopeThreads items per workgroup
  const int groups = a.d / 8;
  const int heads_per_wg = std::max(1, kRopeThreads / (2 * groups));
  static_assert(kRopeThreads % 32 == 0, "items per head divide the workgroup");
  const int heads = a.Hq + a.Hkv;
  dim3 grid(static_cast<unsigned>(a.b) * static_cast<unsigned>(a.B),
            static_cast<unsigned>((heads + heads_per_wg - 1) / heads_per_wg));
  hipLaunchKernelGGL(rope_copy_kernel, grid, dim3(kRopeThreads), 0, stream, a, heads_per_wg);
  return hipGetLastError();
}

}  // namespace simsd
