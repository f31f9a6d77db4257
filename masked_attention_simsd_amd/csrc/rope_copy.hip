// rope_copy.hip -- RoPE over the paired block with the copy rule.
//
// SimSD pages ([nl] "Technische Samenvatting: SimSD - Simple Speculative
// Decoding in Diffusion Language Models" and [fr] "SimSD: Simple Speculative
// Decoding in Diffusion Language Models", Methodologie 3): the mask slot D~_k
// takes the rotary position of its paired data token D_k. The kernel makes
// that literal: a workgroup owns response position k of one sequence (and a
// chunk of heads), evaluates the d/2 rotation angles of that position once,
// and applies the same angles to the rows of both D_k and D~_k, for query and
// KV heads.
//
// The kernel is bound by latency and HBM traffic (one read + one write of the
// block's Q and K); the head dimension of the grid gives every thread a single
// rotation. fp64 is used for angles, cos/sin and the rotation, and each output
// is rounded to bf16 once.
#include "simsd_internal.h"

#include <algorithm>

namespace simsd {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kMaxHalf = 64;  // d <= 128

// One thread rotates 4 consecutive pairs of one head row.
__device__ __forceinline__ void rotate4(uint16_t* row, int i0, int half, bool interleaved,
                                        const double* cs, const double* sn) {
  if (!interleaved) {
    // pairs (i, i + half) for i = i0 .. i0+3: two 8-byte loads
    uint2 lo = *reinterpret_cast<const uint2*>(row + i0);
    uint2 hi = *reinterpret_cast<const uint2*>(row + half + i0);
    uint16_t a[4] = {static_cast<uint16_t>(lo.x), static_cast<uint16_t>(lo.x >> 16),
                     static_cast<uint16_t>(lo.y), static_cast<uint16_t>(lo.y >> 16)};
    uint16_t c[4] = {static_cast<uint16_t>(hi.x), static_cast<uint16_t>(hi.x >> 16),
                     static_cast<uint16_t>(hi.y), static_cast<uint16_t>(hi.y >> 16)};
    uint16_t ra[4], rc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      double xa = bf16_to_f32(a[j]), xb = bf16_to_f32(c[j]);
      double co = cs[i0 + j], si = sn[i0 + j];
      ra[j] = f64_to_bf16(xa * co - xb * si);
      rc[j] = f64_to_bf16(xb * co + xa * si);
    }
    lo.x = ra[0] | (static_cast<uint32_t>(ra[1]) << 16);
    lo.y = ra[2] | (static_cast<uint32_t>(ra[3]) << 16);
    hi.x = rc[0] | (static_cast<uint32_t>(rc[1]) << 16);
    hi.y = rc[2] | (static_cast<uint32_t>(rc[3]) << 16);
    *reinterpret_cast<uint2*>(row + i0) = lo;
    *reinterpret_cast<uint2*>(row + half + i0) = hi;
  } else {
    // pairs (2i, 2i+1) for i = i0 .. i0+3: one 16-byte load
    uint4 v = *reinterpret_cast<const uint4*>(row + 2 * i0);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      double xa = bf16_to_f32(static_cast<uint16_t>(w[j]));
      double xb = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
      double co = cs[i0 + j], si = sn[i0 + j];
      uint16_t ra = f64_to_bf16(xa * co - xb * si);
      uint16_t rb = f64_to_bf16(xb * co + xa * si);
      w[j] = ra | (static_cast<uint32_t>(rb) << 16);
    }
    *reinterpret_cast<uint4*>(row + 2 * i0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Grid: (sequence, position k) x head chunks. Threads of a workgroup each own
// one group of 4 pairs of one row (D_k or D~_k) of one head, so every thread
// does a single independent load / rotate / store.
__global__ __launch_bounds__(kRopeThreads) void rope_copy_kernel(RopeArgs a, int heads_per_wg) {
  __shared__ double cs_d[kMaxHalf], sn_d[kMaxHalf];  // angles of D_k
  __shared__ double cs_t[kMaxHalf], sn_t[kMaxHalf];  // angles of D~_k (same unless no_copy)
  const int s = blockIdx.x / a.B;
  const int k = blockIdx.x % a.B;  // 0-based response position
  const int half = a.d / 2;
  const int tid = threadIdx.x;
  const long pos_d = static_cast<long>(a.start_pos[s]) + k;
  const long pos_t = a.no_copy ? pos_d + a.B : pos_d;
  if (tid < half) {
    const double inv_freq = pow(a.base, -2.0 * tid / a.d);
    double ang = static_cast<double>(pos_d) * inv_freq;
    sincos(ang, &sn_d[tid], &cs_d[tid]);
    if (a.no_copy) {
      ang = static_cast<double>(pos_t) * inv_freq;
      sincos(ang, &sn_t[tid], &cs_t[tid]);
    }
  }
  __syncthreads();
  const double* cs = cs_d;
  const double* sn = sn_d;
  // items of this workgroup: (row slot, head in this chunk, group of 4 pairs)
  const int groups = half / 4;
  const int heads = a.Hq + a.Hkv;
  const int h0 = blockIdx.y * heads_per_wg;
  const int nh = min(heads_per_wg, heads - h0);
  const int items = 2 * nh * groups;
  for (int it = tid; it < items; it += kRopeThreads) {
    const int grp = it % groups;
    const int hh = h0 + (it / groups) % nh;
    const int slot = it / (groups * nh);  // 0: D_k, 1: D~_k
    const int r = k + slot * a.B;
    uint16_t* row;
    if (hh < a.Hq) {
      row = a.q + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hq + hh) * a.d;
    } else {
      row = a.k + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hkv + (hh - a.Hq)) * a.d;
    }
    const bool use_t = slot && a.no_copy;
    rotate4(row, grp * 4, half, a.interleaved != 0, use_t ? cs_t : cs, use_t ? sn_t : sn);
  }
}

}  // namespace

hipError_t launch_rope_copy(const RopeArgs& a, hipStream_t stream) {
  // one thread per (row slot, head, 4-pair group): 2 * groups items per head
  const int groups = a.d / 8;
  const int heads_per_wg = std::max(1, kRopeThreads / (2 * groups));
  const int heads = a.Hq + a.Hkv;
  dim3 grid(static_cast<unsigned>(a.b) * static_cast<unsigned>(a.B),
            static_cast<unsigned>((heads + heads_per_wg - 1) / heads_per_wg));
  hipLaunchKernelGGL(rope_copy_kernel, grid, dim3(kRopeThreads), 0, stream, a, heads_per_wg);
  return hipGetLastError();
}

}  // namespace simsd
