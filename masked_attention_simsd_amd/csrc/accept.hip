// accept.hip -- rejection-sampling acceptance along the draft's temporal order.
//
// SimSD pages ([nl] "Technische Samenvatting: SimSD - Simple Speculative
// Decoding in Diffusion Language Models" and [fr] "SimSD: Simple Speculative
// Decoding in Diffusion Language Models", Methodologie 4, acceptance):
// standard rejection sampling is applied in the temporal order the draft
// induced, and the longest accepted prefix is committed.
//
// One workgroup (16 waves) per sequence.
//   Phase 1 (wave 0, one lane per temporal step t): invert tau, gather
//   p[k][x] and q[k][x] at k = tau^-1(t), take the fp32 ratio, compare with
//   u_t, and find the first rejected step with one ballot.
//   Phase 2 (all waves, only if a step was rejected): stream the vocabulary
//   row of p and q at k* = tau^-1(L+1) once to get each wave's residual mass
//   max(0, p - q) over a contiguous vocabulary segment (fp64 sums), pick the
//   segment holding u_{B+1} * Z, and let its wave rescan that segment with a
//   wave-wide prefix sum to find the first token whose running mass exceeds
//   the threshold.
// The vocabulary stream is the only sizeable traffic (2 V fp32 per rejecting
// sequence), so the kernel is HBM/latency bound; the second read of the
// chosen segment is served from L2.
#include "simsd_internal.h"

namespace simsd {

namespace {

constexpr int kAccThreads = 1024;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kIter = kWave * 4;  // vocabulary entries per wave iteration

__device__ __forceinline__ float4 load4(const float* row, int y, int V, bool vec) {
  if (vec && y + 3 < V) return *reinterpret_cast<const float4*>(row + y);
  float4 r;
  r.x = y < V ? row[y] : 0.0f;
  r.y = y + 1 < V ? row[y + 1] : 0.0f;
  r.z = y + 2 < V ? row[y + 2] : 0.0f;
  r.w = y + 3 < V ? row[y + 3] : 0.0f;
  return r;
}

// Mass of the four entries y .. y+3: the residual max(0, p - q) (fp32), or p
// itself when the residual is empty.
__device__ __forceinline__ void masses(const float* prow, const float* qrow, int y, int V,
                                       bool vec, bool use_p, float w[4]) {
  float4 pv = load4(prow, y, V, vec);
  float pa[4] = {pv.x, pv.y, pv.z, pv.w};
  if (use_p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pa[j] > 0.0f ? pa[j] : 0.0f;
    return;
  }
  float4 qv = load4(qrow, y, V, vec);
  float qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r = pa[j] - qa[j];
    w[j] = r > 0.0f ? r : 0.0f;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (fp64).
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__global__ __launch_bounds__(kAccThreads) void accept_kernel(AcceptArgs a) {
  __shared__ int inv_s[64];
  __shared__ int sh_L, sh_stat, sh_done, sh_wstar, sh_pick;
  __shared__ double seg_sum[kAccWaves];
  __shared__ double sh_T, sh_base;

  const int s = blockIdx.x;
  const int B = a.B, V = a.V;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  if (wave == 0) {
    // Invert tau: lane t looks for the unique k with tau(k) = t + 1.
    int cnt = 0, kk = -1;
    if (lane < B) {
      for (int k = 0; k < B; ++k) {
        if (a.tau[static_cast<size_t>(s) * B + k] == lane + 1) {
          ++cnt;
          kk = k;
        }
      }
    }
    const bool bad = __ballot(lane < B && cnt != 1) != 0ull;
    if (lane < B) inv_s[lane] = kk;
    if (bad) {
      if (lane == 0) {
        sh_L = -1;
        sh_stat = kDevBadTau;
      }
    } else {
      bool acc = true;
      int stat = 0;
      if (lane < B) {
        const int x = a.draft[static_cast<size_t>(s) * B + kk];
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
    if (tid == 0) {
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
  const int per_wave = ((V + kAccWaves * kIter - 1) / (kAccWaves * kIter)) * kIter;
  const int seg_lo = wave * per_wave;
  const int seg_hi = min(V, seg_lo + per_wave);
  const float u_corr = a.u[static_cast<size_t>(s) * (B + 1) + B];

  bool use_p = false;
  for (int mode = 0; mode < 2; ++mode) {
    use_p = mode == 1;
    // Pass 1: residual mass of this wave's contiguous segment.
    double running = 0.0;
    for (int base = seg_lo; base < seg_hi; base += kIter) {
      const int y = base + 4 * lane;
      float w[4] = {0.f, 0.f, 0.f, 0.f};
      if (y < seg_hi) masses(prow, qrow, y, seg_hi, vec, use_p, w);
      const double ls = ((static_cast<double>(w[0]) + w[1]) + w[2]) + w[3];
      const double incl = wave_incl_scan(ls, lane);
      running += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) seg_sum[wave] = running;
    __syncthreads();
    if (tid == 0) {
      double Z = 0.0;
      for (int w = 0; w < kAccWaves; ++w) Z += seg_sum[w];
      sh_done = Z > 0.0;
      if (Z > 0.0) {
        const double T = static_cast<double>(u_corr) * Z;
        double cum = 0.0;
        int wstar = -1, lastpos = -1;
        for (int w = 0; w < kAccWaves; ++w) {
          if (seg_sum[w] > 0.0) lastpos = w;
          if (wstar < 0 && cum + seg_sum[w] > T) {
            wstar = w;
            break;
          }
          cum += seg_sum[w];
        }
        if (wstar < 0) {  // rounding left T at or past the total
          wstar = lastpos;
          cum = 0.0;
          for (int w = 0; w < wstar; ++w) cum += seg_sum[w];
        }
        sh_wstar = wstar;
        sh_T = T;
        sh_base = cum;
      }
      if (mode == 0 && !(Z > 0.0)) sh_stat |= kDevZeroResidual;
    }
    __syncthreads();
    if (sh_done) break;
  }
  if (!sh_done) {  // no mass at all: nothing can be drawn
    if (tid == 0) {
      a.accept_len[s] = L;
      a.correction[s] = -1;
      if (a.status && sh_stat) atomicOr(&a.status[s], sh_stat);
    }
    return;
  }

  // Pass 2: the chosen wave rescans its segment for the first y with
  // running mass > T (zero-mass tokens are never drawn).
  if (wave == sh_wstar) {
    const double T = sh_T;
    double running = sh_base;
    int pick = -1, lastpos = -1;
    for (int base = seg_lo; base < seg_hi && pick < 0; base += kIter) {
      const int y = base + 4 * lane;
      float w[4] = {0.f, 0.f, 0.f, 0.f};
      if (y < seg_hi) masses(prow, qrow, y, seg_hi, vec, use_p, w);
      const double ls = ((static_cast<double>(w[0]) + w[1]) + w[2]) + w[3];
      const double incl = wave_incl_scan(ls, lane);
      double excl = __shfl_up(incl, 1, kWave);
      if (lane == 0) excl = 0.0;
      int hit = -1, lp = -1;
      double c = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c += w[j];
        if (w[j] > 0.0f) {
          lp = y + j;
          if (hit < 0 && running + (excl + c) > T) hit = y + j;
        }
      }
      const unsigned long long hits = __ballot(hit >= 0);
      if (hits) {
        const int first = __ffsll(static_cast<long long>(hits)) - 1;
        pick = __shfl(hit, first, kWave);
      }
      const unsigned long long lps = __ballot(lp >= 0);
      if (lps) {
        const int lastl = 63 - __clzll(static_cast<long long>(lps));
        lastpos = __shfl(lp, lastl, kWave);
      }
      running += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) sh_pick = pick >= 0 ? pick : lastpos;
  }
  __syncthreads();
  if (tid == 0) {
    a.accept_len[s] = L;
    a.correction[s] = sh_pick;
    if (a.status && sh_stat) atomicOr(&a.status[s], sh_stat);
  }
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(a.b), dim3(kAccThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace simsd
