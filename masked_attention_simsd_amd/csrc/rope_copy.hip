// rope_copy.hip -- RoPE over the paired block with the copy rule.
//
// SimSD pages ([nl] "Technische Samenvatting: SimSD - Simple Speculative
// Decoding in Diffusion Language Models" and [fr] "SimSD: Simple Speculative
// Decoding in Diffusion Language Models", Methodologie 3): the mask slot D~_k
// takes the rotary position of its paired data token D_k. The kernel makes
// that literal: one workgroup owns response position k of one sequence,
// evaluates the d/2 rotation angles of that position once, and applies them
// to the rows of both D_k and D~_k, for the query heads and the KV heads.
//
// Work per workgroup is tiny (2 rows x (Hq + Hkv) heads x d elements), so the
// kernel is bound by HBM traffic (read + write of Q and K of the block); fp64
// is used for angles, cos/sin and the rotation, and each output is rounded to
// bf16 once.
#include "simsd_internal.h"

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

__global__ __launch_bounds__(kRopeThreads) void rope_copy_kernel(RopeArgs a) {
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
    ang = static_cast<double>(pos_t) * inv_freq;
    sincos(ang, &sn_t[tid], &cs_t[tid]);
  }
  __syncthreads();
  // Work items: (row in {D_k, D~_k}) x (head in Q then K) x (groups of 4 pairs)
  const int groups = half / 4;
  const int heads = a.Hq + a.Hkv;
  const int items = 2 * heads * groups;
  for (int it = tid; it < items; it += kRopeThreads) {
    const int grp = it % groups;
    const int hh = (it / groups) % heads;
    const int slot = it / (groups * heads);  // 0: D_k, 1: D~_k
    const int r = k + slot * a.B;
    uint16_t* row;
    if (hh < a.Hq) {
      row = a.q + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hq + hh) * a.d;
    } else {
      row = a.k + ((static_cast<size_t>(s) * 2 * a.B + r) * a.Hkv + (hh - a.Hq)) * a.d;
    }
    rotate4(row, grp * 4, half, a.interleaved != 0, slot ? cs_t : cs_d, slot ? sn_t : sn_d);
  }
}

}  // namespace

hipError_t launch_rope_copy(const RopeArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.b) * static_cast<unsigned>(a.B));
  hipLaunchKernelGGL(rope_copy_kernel, grid, dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace simsd
