// accept.hip -- rejection-sampling acceptance along the draft's temporal order.
//
// SimSD pages ([nl] "Technische Samenvatting: SimSD - Simple Speculative
// Decoding in Diffusion Language Models" and [fr] "SimSD: Simple Speculative
// Decoding in Diffusion Language Models", Methodologie 4, acceptance):
// standard rejection sampling is applied in the temporal order the draft
// induced, and the longest accepted prefix is committed.
//
// The step is latency bound, and one CU cannot keep enough misses in flight to
// stream a 32K-151K vocabulary row quickly, so each sequence is spread over
// ceil(V / 4096) workgroups of 256 threads (grid: segments x sequences).
//   Phase 1 (wave 0 of every workgroup, one lane per temporal step t): tau and
//   the draft ids are read together, tau is inverted in LDS, p[k][x] and
//   q[k][x] are gathered at k = tau^-1(t), the IEEE fp32 ratio is compared
//   with u_t, and one ballot gives the first rejected step L. Every workgroup
//   of a sequence repeats this (a few gathers) so none waits for another.
//   Phase 2 (only if L < B): each workgroup reads its 4096-entry segment of
//   the rows p[k*], q[k*] (k* = tau^-1(L+1)), 16 contiguous entries per
//   thread, and publishes the segment's fp64 residual mass max(0, p - q) with
//   device-coherent stores. The last workgroup of the sequence (agent-scope
//   counter) fetches all segment masses at once, forms Z in segment order,
//   finds the segment holding T = u_{B+1} * Z and rescans it with a
//   workgroup-wide prefix sum for the first token whose running mass exceeds T.
// Traffic: 2 V fp32 per rejecting sequence plus one segment re-read.
#include "simsd_internal.h"

namespace simsd {

namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kPerThread = 16;                  // contiguous entries per thread
constexpr int kSeg = kAccThreads * kPerThread;  // entries per segment / workgroup

// Masses of entries y0 .. y0+15 of one row: the residual max(0, p - q) in
// fp32, or p itself for the zero-residual fallback; entries at or past V are 0.
__device__ __forceinline__ void load_masses(const float* prow, const float* qrow, int y0, int V,
                                            bool vec, bool use_p, float w[kPerThread]) {
  float pv[kPerThread], qv[kPerThread];
  if (vec && y0 + kPerThread <= V) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const float4 a = *reinterpret_cast<const float4*>(prow + y0 + 4 * j);
      pv[4 * j] = a.x, pv[4 * j + 1] = a.y, pv[4 * j + 2] = a.z, pv[4 * j + 3] = a.w;
      const float4 b = use_p ? a : *reinterpret_cast<const float4*>(qrow + y0 + 4 * j);
      qv[4 * j] = b.x, qv[4 * j + 1] = b.y, qv[4 * j + 2] = b.z, qv[4 * j + 3] = b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const bool in = y0 + e < V;
      pv[e] = in ? prow[y0 + e] : 0.0f;
      qv[e] = (in && !use_p) ? qrow[y0 + e] : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const float r = use_p ? pv[e] : pv[e] - qv[e];
    w[e] = r > 0.0f ? r : 0.0f;
  }
}

// Exclusive prefix sum (thread order) of one fp64 value per thread and the
// workgroup total, which is computed as last exclusive prefix + last value so
// that a rescan's running sums end exactly at the segment mass.
__device__ double block_excl_scan(double v, double* total) {
  __shared__ double sh_wave[kAccWaves];
  __shared__ double sh_total;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  double incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  if (lane == kWave - 1) sh_wave[wave] = incl;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += sh_wave[w];
  excl += base;
  if (tid == kAccThreads - 1) sh_total = excl + v;
  __syncthreads();
  *total = sh_total;
  __syncthreads();  // the shared slots may be reused after this
  return excl;
}

__device__ __forceinline__ double thread_sum(const float w[kPerThread]) {
  double ls = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) ls += static_cast<double>(w[e]);
  return ls;
}

__global__ __launch_bounds__(kAccThreads) void accept_kernel(AcceptArgs a) {
  __shared__ int inv_s[64];
  __shared__ int sh_L, sh_stat, sh_last, sh_pick, sh_seg;
  __shared__ double sh_mass[kMaxAcceptVocab / kSeg];
  __shared__ double sh_T, sh_base;

  const int seg = blockIdx.x, nseg = gridDim.x;
  const int s = blockIdx.y;
  const int B = a.B, V = a.V;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float u_corr = a.u[static_cast<size_t>(s) * (B + 1) + B];  // requested early

  if (wave == 0) {
    const int t_k = lane < B ? a.tau[static_cast<size_t>(s) * B + lane] : 0;  // tau(lane+1)
    const int x_k = lane < B ? a.draft[static_cast<size_t>(s) * B + lane] : 0;
    if (lane < B) inv_s[lane] = -1;
    // invert: position k = lane writes itself at slot tau(k) - 1; a duplicate or
    // out-of-range label makes tau invalid
    const bool in_range = lane < B && t_k >= 1 && t_k <= B;
    if (in_range) inv_s[t_k - 1] = lane;
    int cnt = 0;
    for (int k = 0; k < B; ++k) cnt += __shfl(t_k, k, kWave) == lane + 1;
    const bool bad = __ballot(lane < B && (cnt != 1 || !in_range)) != 0ull;
    if (bad) {
      if (lane == 0) {
        sh_L = -1;
        sh_stat = kDevBadTau;
      }
    } else {
      const int kk = lane < B ? inv_s[lane] : 0;  // position with label lane + 1
      const int x = __shfl(x_k, kk, kWave);
      bool acc = true;
      int stat = 0;
      if (lane < B) {
        float r;
        if (x < 0 || x >= V) {
          stat |= kDevBadToken;
          r = 0.0f;
        } else {
          const size_t at = (static_cast<size_t>(s) * B + kk) * V + x;
          const float pa = a.p[at], qa = a.q[at];
          if (qa > 0.0f) {
            r = pa / qa;  // IEEE-rounded fp32 division (no fast-math in this library)
            r = r > 1.0f ? 1.0f : r;
          } else {
            stat |= kDevQZero;
            r = pa > 0.0f ? 1.0f : 0.0f;
          }
        }
        acc = a.u[static_cast<size_t>(s) * (B + 1) + lane] < r;
      }
      const unsigned long long rej = __ballot(lane < B && !acc);
      const int L = rej ? __ffsll(static_cast<long long>(rej)) - 1 : B;
      // status bits only from the steps that were examined (1 .. L+1)
      const bool seen = lane < B && lane <= L;
      int st = 0;
      if (__ballot(seen && (stat & kDevBadToken))) st |= kDevBadToken;
      if (__ballot(seen && (stat & kDevQZero))) st |= kDevQZero;
      if (lane == 0) {
        sh_L = L;
        sh_stat = st;
      }
    }
  }
  __syncthreads();
  const int L = sh_L;
  if (L < 0 || L == B) {
    if (seg == 0 && tid == 0) {
      a.accept_len[s] = L < 0 ? 0 : B;
      a.correction[s] = -1;
      if (a.status && sh_stat) atomicOr(&a.status[s], sh_stat);
    }
    return;
  }

  const int kstar = inv_s[L];
  const float* prow = a.p + (static_cast<size_t>(s) * B + kstar) * V;
  const float* qrow = a.q + (static_cast<size_t>(s) * B + kstar) * V;
  const bool vec = (V % 4) == 0;

  // ---- every workgroup: residual mass of its segment, published coherently ----
  float w[kPerThread];
  load_masses(prow, qrow, seg * kSeg + kPerThread * tid, V, vec, false, w);
  double mine;
  block_excl_scan(thread_sum(w), &mine);
  double* segsum = a.seg_sum + static_cast<size_t>(s) * nseg;
  if (tid == 0)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(segsum + seg),
                       static_cast<unsigned long long>(__double_as_longlong(mine)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);  // the store is acknowledged before the counter moves
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&a.counters[s], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == nseg - 1;
  }
  __syncthreads();
  if (!sh_last) return;

  // ---- last workgroup: all masses at once, threshold, segment, rescan ----
  bool use_p = false;
  for (int mode = 0; mode < 2; ++mode) {
    use_p = mode == 1;
    if (!use_p) {
      for (int j = tid; j < nseg; j += kAccThreads)
        sh_mass[j] = __longlong_as_double(static_cast<long long>(__hip_atomic_load(
            reinterpret_cast<unsigned long long*>(segsum + j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    } else {  // zero residual: the (rare) fallback draws from p; masses of p, all segments here
      for (int j = 0; j < nseg; ++j) {
        float wp[kPerThread];
        load_masses(prow, qrow, j * kSeg + kPerThread * tid, V, vec, true, wp);
        double m;
        block_excl_scan(thread_sum(wp), &m);
        if (tid == 0) sh_mass[j] = m;
      }
    }
    __syncthreads();
    if (tid == 0) {
      double Z = 0.0;
      for (int j = 0; j < nseg; ++j) Z += sh_mass[j];
      if (Z > 0.0) {
        const double T = static_cast<double>(u_corr) * Z;
        double cum = 0.0, cum_last = 0.0;
        int pick = -1, lastpos = -1;
        for (int j = 0; j < nseg; ++j) {
          const double m = sh_mass[j];
          if (m > 0.0) lastpos = j, cum_last = cum;
          if (cum + m > T) {
            pick = j;
            break;
          }
          cum += m;
        }
        if (pick < 0) {  // rounding left T at or past the total
          pick = lastpos;
          cum = cum_last;
        }
        sh_seg = pick;
        sh_base = cum;
        sh_T = T;
      } else {
        sh_seg = -2;
        if (mode == 0) sh_stat |= kDevZeroResidual;
      }
    }
    __syncthreads();
    if (sh_seg != -2) break;
  }

  if (tid == 0) sh_pick = 0x7fffffff;
  __syncthreads();
  const int j = sh_seg;  // < 0: no mass anywhere
  if (j >= 0) {
    const int y0 = j * kSeg + kPerThread * tid;
    if (j != seg || use_p) load_masses(prow, qrow, y0, V, vec, use_p, w);
    double total;
    const double excl = block_excl_scan(thread_sum(w), &total);
    const double T = sh_T, base = sh_base;
    int hit = -1, lastpos = -1;
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      run += static_cast<double>(w[e]);
      if (w[e] > 0.0f) {
        lastpos = y0 + e;
        if (hit < 0 && base + (excl + run) > T) hit = y0 + e;
      }
    }
    if (hit >= 0) atomicMin(&sh_pick, hit);
    __syncthreads();
    const bool none = sh_pick == 0x7fffffff;
    __syncthreads();
    if (none) {  // rounding: no crossing inside the segment; take its last positive entry
      if (tid == 0) sh_pick = -1;
      __syncthreads();
      if (lastpos >= 0) atomicMax(&sh_pick, lastpos);
    }
  } else if (tid == 0) {
    sh_pick = -1;  // no mass at all: nothing can be drawn
  }
  __syncthreads();
  if (tid == 0) {
    a.accept_len[s] = L;
    a.correction[s] = sh_pick;
    if (a.status && sh_stat) atomicOr(&a.status[s], sh_stat);
    __hip_atomic_store(&a.counters[s], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int accept_segments(int V) { return (V + kSeg - 1) / kSeg; }

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(accept_segments(a.V)), static_cast<unsigned>(a.b));
  hipLaunchKernelGGL(accept_kernel, grid, dim3(kAccThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace simsd
