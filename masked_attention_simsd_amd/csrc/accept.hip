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
// ceil(V / (256 PER)) workgroups of 256 threads (grid: segments x sequences,
// PER contiguous entries per thread).
//   Phase 1 (wave 0 of every workgroup, one lane per temporal step t): tau and
//   the draft ids are read together, tau is inverted in LDS, p[k][x] and
//   q[k][x] are gathered at k = tau^-1(t), the IEEE fp32 ratio is compared
//   with u_t, and one ballot gives the first rejected step L. Every workgroup
//   of a sequence repeats this (a few gathers) so none waits for another.
//   Phase 2 (only if L < B): each workgroup reads its segment of the rows
//   p[k*], q[k*] (k* = tau^-1(L+1)), forms the segment's fp64 residual mass
//   max(0, p - q) and publishes it with a ready bit, then bumps the sequence's
//   agent-scope arrival counter without waiting for the publish to land. The
//   last arrival polls the ready bits (every publish was issued before its
//   counter bump, so each poll ends), clears the words for the next call,
//   forms Z, finds the segment holding T = u_{B+1} * Z with a one-wave prefix
//   scan over the segment masses, and rescans that segment with a
//   workgroup-wide prefix sum for the first token whose running mass exceeds T.
// Traffic: 2 V fp32 per rejecting sequence plus one segment re-read.
//
// From logits (simsd_accept_logits) a row-statistics pass first reduces every
// target and draft row to its maximum and sum of exponentials and publishes
// them, with the logit at the row's draft token, as ready-bit words; phase 1
// then reads a position's ratio inputs from those words instead of gathering,
// and phase 2 evaluates p and q from the logits of the rejected rows. Large
// batches run the pass and the acceptance in one grid (accept_logits_kernel).
#include "simsd.h"
#include "simsd_internal.h"

#include <stdlib.h>

namespace simsd {

namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / kWave;
constexpr int kMinPer = 4;  // smallest entries-per-thread variant (sizes the workspace)
// A published segment mass carries this bit (masses are +0 or positive, so
// the sign bit is free); a cleared word (0) means "not yet published".
constexpr unsigned long long kReady = 1ull << 63;
constexpr int kPollLimit = 1 << 16;  // bound on the polls of one mass word

// Arrival counters of different sequences sit 128 bytes apart (their own
// cache lines, as far as the fixed counter region allows): every workgroup of
// a launch bumps one, and counters sharing a line serialise each other's
// atomics.
__device__ __forceinline__ int* seq_counter(const AcceptArgs& a, int s) {
  const int stride = min(32, kMaxSeqCounters / a.b);
  return a.counters + static_cast<size_t>(s) * stride;
}
// The row-statistics counters (2 b B rows) likewise, 128 bytes apart for up to
// 2048 rows; the workspace size reserves the padded region by the same rule.
__device__ __forceinline__ int* row_counter(const AcceptArgs& a, int row) {
  const int rows = 2 * a.b * a.B;
  return a.row_counters + static_cast<size_t>(row) * (rows <= 2048 ? 32 : 1);
}

// 2^(j/256), j = 0..255, each the fp64 value nearest the exact one (computed
// in 80-digit decimal arithmetic; a CPU test recomputes and compares every
// entry).
__constant__ double kExp2Frac[256] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0,
};

// exp(x) for x <= 0 in fp64 by table (Tang's method), for the statistics
// pass where it runs once per logit and its instruction count sets the pass's
// speed: x = (256 n + j) ln2/256 + r with |r| <= ln2/512 (k = 256 n + j from
// a round-to-nearest shifter), e^x = 2^n T[j] (1 + p(r)) with T[j] =
// 2^(j/256) from `tab` and p the Taylor series of e^r - 1 to degree 4
// (truncation < 4e-17), scaled by 2^n with ldexp. The reduction
// uses ln2/256 as one double: r is off by at most |x| 2^-53, so a term e^x
// carries a relative error of about |x| 1.1e-16 on top of a few 1e-16, and
// its share of a row sum's error, e^x |x| 1.1e-16 <= 0.37 * 1.1e-16 per unit
// of the sum, stays at the rounding level of the sum itself. With TWO_PART
// the reduction takes ln2/256 in two parts (one more fma) and the error is a
// few 1e-16 at every x, for probabilities evaluated one by one. x is first
// clamped to [-708, 0] (NaN as well): below that the true value is under
// 3.4e-308 and the result, 3.3e-308, is equally invisible in a row sum of at
// least 1 (it keeps n >= -1022 with T[j](1 + p) >= 1, so the scaled result
// stays normal); a probability that small rounds to 0 in fp32 either way.
template <bool TWO_PART = false>
__device__ __forceinline__ double exp_nonpos_tab(double x, const double* tab) {
  x = fmax(x, -708.0);
  constexpr double kShift = 6755399441055744.0;  // 1.5 * 2^52: k lands in the low word
  const double kt = __builtin_fma(x, 369.3299304675746, kShift);  // x * 256 / ln2 + shift
  const int k = __double2loint(kt);
  const double kd = kt - kShift;
  double r = __builtin_fma(-kd, 0x1.62e42fefa39efp-9, x);  // ln2/256 (its high part with TWO_PART)
  if constexpr (TWO_PART) r = __builtin_fma(-kd, 0x1.abc9e3b39803fp-64, r);  // ln2/256, low part
  double p = 1.0 / 24.0;
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p *= r;
  const double t = tab[k & 255];
  return __builtin_amdgcn_ldexp(__builtin_fma(t, p, t), k >> 8);  // arithmetic shift: floor(k / 256)
}

// Softmax probability of logit z in a row with statistics (max m, sum of
// exp s, passed as 1/s) at inverse temperature inv_t: exp((z - m) inv_t) / s
// in fp64 (table exponential with the two-part reduction), rounded once to
// fp32 (the precision the decisions are taken in).
__device__ __forceinline__ float softmax_prob_tab(float z, double m, double inv_s, double inv_t,
                                                  const double* tab) {
  return static_cast<float>(exp_nonpos_tab<true>((static_cast<double>(z) - m) * inv_t, tab) * inv_s);
}

// Row statistics of the target and draft rows (s, k): (max, 1 / sum of exp).
struct RowStats {
  double mt, st, md, sd;  // st, sd: reciprocal row sums
};
// The statistics pass publishes kRowStatWords 64-bit words per row, each
// with the ready bit: the row maximum (float bits), 1 / sum (a positive
// double, so its sign bit is free), the row's logit at position k's draft
// token (float bits; never written when that token lies outside the
// vocabulary) and an unused word. Readers poll them, so they may run in the
// same launch as the pass.
constexpr int kRowStatWords = 4;
__device__ __forceinline__ unsigned long long* row_stat_words(const AcceptArgs& a, size_t row) {
  return reinterpret_cast<unsigned long long*>(a.row_stats) + kRowStatWords * row;
}
__device__ __forceinline__ void publish_word(unsigned long long* w, unsigned long long bits) {
  __hip_atomic_store(w, bits | kReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Statistics of position k of sequence s (target and draft rows) and, when the
// draft token is in the vocabulary, its two logits; waits (bounded) until they
// are published. Returns false if a wait ran out.
__device__ __forceinline__ bool row_stats_of(const AcceptArgs& a, int s, int k, bool with_logits, RowStats* rs,
                                             double* zt_x, double* zd_x) {
  const size_t rt = static_cast<size_t>(s) * a.B + k, rd = rt + static_cast<size_t>(a.b) * a.B;
  const unsigned long long* t = row_stat_words(a, rt);
  const unsigned long long* d = row_stat_words(a, rd);
  unsigned long long w[6];
  bool ok = false;
  int polls = 0;
  do {
    w[0] = __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[1] = __hip_atomic_load(t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[2] = __hip_atomic_load(t + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[3] = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[4] = __hip_atomic_load(d + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[5] = __hip_atomic_load(d + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = (w[0] & w[1] & w[3] & w[4] & kReady) && (!with_logits || (w[2] & w[5] & kReady));
    if (ok) break;
    __builtin_amdgcn_s_sleep(2);
  } while (++polls < kPollLimit);
  *rs = RowStats{static_cast<double>(__uint_as_float(static_cast<uint32_t>(w[0]))),
                 __longlong_as_double(static_cast<long long>(w[1] & ~kReady)),
                 static_cast<double>(__uint_as_float(static_cast<uint32_t>(w[3]))),
                 __longlong_as_double(static_cast<long long>(w[4] & ~kReady))};
  *zt_x = static_cast<double>(__uint_as_float(static_cast<uint32_t>(w[2])));
  *zd_x = static_cast<double>(__uint_as_float(static_cast<uint32_t>(w[5])));
  return ok;
}

// Zero the statistics of sequence s's 2 B rows once every workgroup of the
// sequence has read them, so a call leaves the whole workspace zero and a
// workspace can be reused at any other sizes.
__device__ __forceinline__ void clear_row_stats(const AcceptArgs& a, int s, int tid) {
  const int n = kRowStatWords * a.B;  // words of the sequence's rows in one half
  unsigned long long* w = row_stat_words(a, 0);
  for (int i = tid; i < 2 * n; i += kAccThreads) {
    const size_t half = i < n ? 0 : static_cast<size_t>(a.b) * a.B * kRowStatWords;
    __hip_atomic_store(w + half + static_cast<size_t>(s) * n + i % n, 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// 16 bytes with the non-temporal hint, for the logits the statistics pass
// reads once (bench runs rotating 640 MB of logits copies, single launches:
// b8 24.4 -> 23.9 us, b16 53.7 -> 52.7, ragged 48.2 -> 47.2; the same hint
// on the acceptance pass's rows gained nothing).
__device__ __forceinline__ float4 load_nt4(const float* p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f x = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(x.x, x.y, x.z, x.w);
}

// Masses of entries y0 .. y0+PER-1 of one row: the residual max(0, p - q) in
// fp32, or p itself for the zero-residual fallback; entries at or past V are 0.
// LOGITS: prow / qrow are logits rows and p, q their softmax (row stats rs).
template <int PER, bool LOGITS>
__device__ __forceinline__ void load_masses(const float* prow, const float* qrow, int y0, int V,
                                            bool vec, bool use_p, const RowStats& rs, double inv_t,
                                            const double* tab, float (&w)[PER]) {
  float pv[PER], qv[PER];
  if (vec && y0 + PER <= V) {
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const float4 a = *reinterpret_cast<const float4*>(prow + y0 + 4 * j);
      pv[4 * j] = a.x, pv[4 * j + 1] = a.y, pv[4 * j + 2] = a.z, pv[4 * j + 3] = a.w;
      const float4 b = use_p ? a : *reinterpret_cast<const float4*>(qrow + y0 + 4 * j);
      qv[4 * j] = b.x, qv[4 * j + 1] = b.y, qv[4 * j + 2] = b.z, qv[4 * j + 3] = b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool in = y0 + e < V;
      pv[e] = in ? prow[y0 + e] : (LOGITS ? -INFINITY : 0.0f);
      qv[e] = (in && !use_p) ? qrow[y0 + e] : (LOGITS ? -INFINITY : 0.0f);
    }
  }
  if constexpr (LOGITS) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      pv[e] = softmax_prob_tab(pv[e], rs.mt, rs.st, inv_t, tab);
      qv[e] = use_p ? 0.0f : softmax_prob_tab(qv[e], rs.md, rs.sd, inv_t, tab);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float r = use_p ? pv[e] : pv[e] - qv[e];
    w[e] = r > 0.0f ? r : 0.0f;
  }
}

// Wave-level scans by DPP (row shifts and row broadcasts move data between
// lanes inside the VALU; the lane shuffles they replace went through LDS, two
// permutes per fp64 step). An fp64 value moves as its two 32-bit halves;
// lanes whose source lies outside the row (bound_ctrl) or whose row the row
// mask leaves out read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xf, true);
  return __hiloint2double(hi, lo);
}
// Inclusive prefix sum over the 64 lanes in lane order: shifts by 1, 2, 4, 8
// inside each row of 16, then the last lane of row 0 / 2 into rows 1 / 3
// (row_bcast:15) and the last lane of row 1 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_f64<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f64<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f64<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f64<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31
  return x;
}
// The inclusive scan shifted up by one lane (lane 0: 0), i.e. the exclusive scan.
__device__ __forceinline__ double wave_shift_up1(double incl) { return dpp_f64<0x138, 0xf>(incl); }  // wave_shr:1
__device__ __forceinline__ double wave_last(double v) {  // lane 63's value, in every lane
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), kWave - 1),
                          __builtin_amdgcn_readlane(__double2loint(v), kWave - 1));
}

// Maximum over the 64 lanes, in every lane: the same row shifts and row
// broadcasts, with lanes that have no source keeping -inf (bound_ctrl off).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_src(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_max_src<0x111, 0xf>(x));
  x = fmaxf(x, dpp_max_src<0x112, 0xf>(x));
  x = fmaxf(x, dpp_max_src<0x114, 0xf>(x));
  x = fmaxf(x, dpp_max_src<0x118, 0xf>(x));
  x = fmaxf(x, dpp_max_src<0x142, 0xa>(x));
  x = fmaxf(x, dpp_max_src<0x143, 0xc>(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

// Exclusive prefix sum (thread order) of one fp64 value per thread, and the
// workgroup total (last exclusive prefix + last value).
__device__ double block_excl_scan(double v, double* total) {
  __shared__ double sh_wave[kAccWaves];
  __shared__ double sh_total;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const double incl = wave_incl_scan(v);
  double excl = wave_shift_up1(incl);
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

// Sum of one fp64 value per thread over the workgroup (fixed order); the
// result is valid in thread 0.
__device__ double block_sum(double v) {
  __shared__ double sh_wave[kAccWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  v = wave_incl_scan(v);
  if (lane == kWave - 1) sh_wave[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (tid == 0)
    for (int w = 0; w < kAccWaves; ++w) t += sh_wave[w];
  __syncthreads();
  return t;
}

template <int PER>
__device__ __forceinline__ double thread_sum(const float (&w)[PER]) {
  double ls = 0.0;
#pragma unroll
  for (int e = 0; e < PER; ++e) ls += static_cast<double>(w[e]);
  return ls;
}

// One wave over the segment masses m[0..nseg): Z = their sum (lanes own
// contiguous runs of segments; run sums are combined by a lane scan). For
// Z > 0 it picks the first segment j with m_j > 0 whose running sum passes
// T = u * Z (rounding fallback: the last segment with positive mass) and
// returns 1 with the running sum before it in *base; Z == 0 returns 0.
__device__ int locate_segment(const double* m, int nseg, float u, int* seg_out, double* base_out,
                              double* T_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (nseg + kWave - 1) / kWave;
  const int j0 = min(lane * per, nseg), j1 = min(j0 + per, nseg);
  double loc = 0.0;
  for (int j = j0; j < j1; ++j) loc += m[j];
  const double incl = wave_incl_scan(loc);
  const double excl = wave_shift_up1(incl);
  const double Z = wave_last(incl);
  if (!(Z > 0.0)) return 0;
  const double T = static_cast<double>(u) * Z;
  int hit = -1, lastpos = -1;
  double hit_base = 0.0, last_base = 0.0, run = excl;
  for (int j = j0; j < j1; ++j) {
    const double mj = m[j];
    if (mj > 0.0) {
      lastpos = j, last_base = run;
      if (hit < 0 && run + mj > T) hit = j, hit_base = run;
    }
    run += mj;
  }
  const unsigned long long hits = __ballot(hit >= 0);
  int src;
  if (hits) {
    src = __ffsll(static_cast<long long>(hits)) - 1;
  } else {  // rounding left T at or past the total
    const unsigned long long pos = __ballot(lastpos >= 0);
    src = 63 - __clzll(static_cast<long long>(pos));
    hit = lastpos, hit_base = last_base;
  }
  // src is uniform: read the lane's registers directly (no LDS permute)
  *seg_out = __builtin_amdgcn_readlane(hit, src);
  *base_out = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(hit_base), src),
                               __builtin_amdgcn_readlane(__double2loint(hit_base), src));
  *T_out = T;
  return 1;
}

template <int PER, bool LOGITS>
__device__ __forceinline__ void accept_body(const AcceptArgs& a, const int seg, const int nseg, const int s,
                                            double* sh_mass) {
  constexpr int kSeg = kAccThreads * PER;  // entries per segment / workgroup
  __shared__ int inv_s[64];
  __shared__ int sh_L, sh_stat, sh_last, sh_pick, sh_seg;
  __shared__ int sh_wave_hit[kAccWaves], sh_wave_last[kAccWaves];
  __shared__ double sh_T, sh_base;
  __shared__ double sh_rs[4];  // LOGITS: row statistics of the rejected step's rows
  __shared__ double exp_tab[LOGITS ? 256 : 1];  // LOGITS: 2^(j/256) for the residual rows

  const int B = a.B, V = a.V;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float u_corr = a.u[static_cast<size_t>(s) * (B + 1) + B];  // requested early
  if (wave == 0) {
    // LOGITS: wave 0 stages the exponential's table (its own ratios read it
    // before the first barrier, the other waves after it); requested first,
    // written to LDS once the loads below are in flight
    double tab_v[LOGITS ? 256 / kWave : 1];
    if constexpr (LOGITS)
#pragma unroll
      for (int j = 0; j < 256 / kWave; ++j) tab_v[j] = kExp2Frac[lane + j * kWave];
    const int t_k = lane < B ? a.tau[static_cast<size_t>(s) * B + lane] : 0;  // tau(lane+1)
    const int x_k = lane < B ? a.draft[static_cast<size_t>(s) * B + lane] : 0;
    // u_t of temporal step t = lane + 1, requested with tau and the drafts so
    // that its latency is not paid after the gathers
    const float u_t = lane < B ? a.u[static_cast<size_t>(s) * (B + 1) + lane] : 0.0f;
    // LOGITS: position lane's row statistics and draft-token logits, requested
    // with tau (none of them depends on it)
    RowStats rs{};
    double zt_x = 0.0, zd_x = 0.0;
    bool stats_ok = true;
    if constexpr (LOGITS) {
      if (lane < B) stats_ok = row_stats_of(a, s, lane, x_k >= 0 && x_k < V, &rs, &zt_x, &zd_x);
#pragma unroll
      for (int j = 0; j < 256 / kWave; ++j) exp_tab[lane + j * kWave] = tab_v[j];
    }
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
      // acceptance ratio min(1, p/q) at a draft token x of a row pair, and its
      // status bits
      auto ratio = [&](float pa, float qa, int& stat) {
        if (qa > 0.0f) {
          const float r = pa / qa;  // IEEE-rounded fp32 division (no fast-math in this library)
          return r > 1.0f ? 1.0f : r;
        }
        stat |= kDevQZero;
        return pa > 0.0f ? 1.0f : 0.0f;
      };
      bool acc = true;
      int stat = 0;
      if constexpr (LOGITS) {
        // position lane's ratio from its own statistics, then each step takes
        // the ratio of its position
        int stat_k = 0;
        float r_k = 0.0f;
        if (x_k < 0 || x_k >= V) {
          stat_k = kDevBadToken;
        } else {
          const float pa = softmax_prob_tab(static_cast<float>(zt_x), rs.mt, rs.st, a.inv_t, exp_tab);
          const float qa = softmax_prob_tab(static_cast<float>(zd_x), rs.md, rs.sd, a.inv_t, exp_tab);
          r_k = ratio(pa, qa, stat_k);
        }
        const float r = __shfl(r_k, kk, kWave);
        stat = __shfl(stat_k, kk, kWave);
        if (lane < B) acc = u_t < r;
      } else {
        const int x = __shfl(x_k, kk, kWave);
        if (lane < B) {
          float r = 0.0f;
          if (x < 0 || x >= V) {
            stat |= kDevBadToken;
          } else {
            const size_t at = (static_cast<size_t>(s) * B + kk) * V + x;
            r = ratio(a.p[at], a.q[at], stat);
          }
          acc = u_t < r;
        }
      }
      const unsigned long long rej = __ballot(lane < B && !acc);
      const int L = rej ? __ffsll(static_cast<long long>(rej)) - 1 : B;
      // status bits only from the steps that were examined (1 .. L+1)
      const bool seen = lane < B && lane <= L;
      int st = 0;
      if (__ballot(seen && (stat & kDevBadToken))) st |= kDevBadToken;
      if (__ballot(seen && (stat & kDevQZero))) st |= kDevQZero;
      if (__ballot(!stats_ok)) st |= kDevSyncTimeout;
      if (lane == 0) {
        sh_L = L;
        sh_stat = st;
      }
      if constexpr (LOGITS) {
        // the rejected step's statistics (its position's lane), for the residual pass
        if (L < B && lane == inv_s[L]) {
          sh_rs[0] = rs.mt, sh_rs[1] = rs.st, sh_rs[2] = rs.md, sh_rs[3] = rs.sd;
        }
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
    if constexpr (LOGITS) {
      // the sequence's last workgroup past its reads of the row statistics
      // clears them (every workgroup of s takes this branch: L is the same)
      if (tid == 0) {
        const int prev = __hip_atomic_fetch_add(seq_counter(a, s), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_last = prev == nseg - 1;
      }
      __syncthreads();
      if (sh_last) {
        clear_row_stats(a, s, tid);
        if (tid == 0) __hip_atomic_store(seq_counter(a, s), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  const int kstar = inv_s[L];
  const float* prow = (LOGITS ? a.zt : a.p) + (static_cast<size_t>(s) * B + kstar) * V;
  const float* qrow = (LOGITS ? a.zd : a.q) + (static_cast<size_t>(s) * B + kstar) * V;
  const bool vec = (V % 4) == 0;
  RowStats rs{};
  if constexpr (LOGITS) rs = RowStats{sh_rs[0], sh_rs[1], sh_rs[2], sh_rs[3]};

  // ---- every workgroup: residual mass of its segment, published with the
  // ready bit; the arrival counter moves without waiting for the publish ----
  float w[PER];
  load_masses<PER, LOGITS>(prow, qrow, seg * kSeg + PER * tid, V, vec, false, rs, a.inv_t, exp_tab, w);
  const double mine = block_sum(thread_sum<PER>(w));
  unsigned long long* words = reinterpret_cast<unsigned long long*>(a.seg_sum) +
                              static_cast<size_t>(s) * nseg;
  if (tid == 0) {
    __hip_atomic_store(words + seg, static_cast<unsigned long long>(__double_as_longlong(mine)) | kReady,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int prev = __hip_atomic_fetch_add(seq_counter(a, s), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == nseg - 1;
  }
  __syncthreads();
  if (!sh_last) return;
  // every workgroup of s has read its row statistics (before its arrival)
  if constexpr (LOGITS) clear_row_stats(a, s, tid);

  // ---- last workgroup: collect the masses, clear the words, locate ----
  bool timed_out = false;
  for (int j = tid; j < nseg; j += kAccThreads) {
    if (j == seg) continue;  // own mass: thread 0 below
    unsigned long long v;
    int polls = 0;
    do {
      v = __hip_atomic_load(words + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v & kReady) break;
      __builtin_amdgcn_s_sleep(1);
    } while (++polls < kPollLimit);
    timed_out |= !(v & kReady);
    sh_mass[j] = __longlong_as_double(static_cast<long long>(v & ~kReady));
    // cleared by the thread that read it: the clear lands after the publish
    __hip_atomic_store(words + j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) {
    sh_mass[seg] = mine;
    // own word: cleared by the thread that published it, after the publish
    __hip_atomic_store(words + seg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (timed_out) atomicOr(&sh_stat, kDevSyncTimeout);
  __syncthreads();

  bool use_p = false;
  for (int mode = 0; mode < 2; ++mode) {
    use_p = mode == 1;
    if (use_p) {  // zero residual: the (rare) fallback draws from p; masses of p, all segments here
      for (int j = 0; j < nseg; ++j) {
        float wp[PER];
        load_masses<PER, LOGITS>(prow, qrow, j * kSeg + PER * tid, V, vec, true, rs, a.inv_t, exp_tab, wp);
        const double m = block_sum(thread_sum<PER>(wp));
        if (tid == 0) sh_mass[j] = m;
      }
      __syncthreads();
    }
    if (wave == 0) {
      int jseg;
      double base, T;
      const int found = locate_segment(sh_mass, nseg, u_corr, &jseg, &base, &T);
      if (lane == 0) {
        if (found) {
          sh_seg = jseg;
          sh_base = base;
          sh_T = T;
        } else {
          sh_seg = -1;
          if (mode == 0) sh_stat |= kDevZeroResidual;
        }
      }
    }
    __syncthreads();
    if (sh_seg >= 0) break;
  }

  const int j = sh_seg;  // < 0: no mass anywhere
  if (j >= 0) {
    const int y0 = j * kSeg + PER * tid;
    if (j != seg || use_p) load_masses<PER, LOGITS>(prow, qrow, y0, V, vec, use_p, rs, a.inv_t, exp_tab, w);
    double total;
    const double excl = block_excl_scan(thread_sum<PER>(w), &total);
    const double T = sh_T, base = sh_base;
    int hit = -1, lastpos = -1;
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      run += static_cast<double>(w[e]);
      if (w[e] > 0.0f) {
        lastpos = y0 + e;
        if (hit < 0 && base + (excl + run) > T) hit = y0 + e;
      }
    }
    // Entries grow with the thread index, so each wave's candidate is the hit
    // of its lowest hitting lane (every thread past the crossing also hits)
    // and its fallback the last positive entry of its highest such lane; one
    // word per wave in LDS, one barrier, and thread 0 takes the first hit
    // over the waves (rounding fallback: the last positive entry).
    const unsigned long long hits = __ballot(hit >= 0);
    const unsigned long long pos = __ballot(lastpos >= 0);
    if (lane == 0) {
      sh_wave_hit[wave] = hits ? __builtin_amdgcn_readlane(hit, __ffsll(static_cast<long long>(hits)) - 1) : -1;
      sh_wave_last[wave] = pos ? __builtin_amdgcn_readlane(lastpos, 63 - __clzll(static_cast<long long>(pos))) : -1;
    }
    __syncthreads();
    if (tid == 0) {
      int pick = -1;
      for (int v = kAccWaves - 1; v >= 0; --v) pick = sh_wave_hit[v] >= 0 ? sh_wave_hit[v] : pick;
      if (pick < 0)
        for (int v = 0; v < kAccWaves; ++v) pick = sh_wave_last[v] >= 0 ? sh_wave_last[v] : pick;
      sh_pick = pick;
    }
  } else if (tid == 0) {
    sh_pick = -1;  // no mass at all: nothing can be drawn
  }
  // thread 0 set sh_pick itself and writes the result: no barrier needed
  if (tid == 0) {
    a.accept_len[s] = L;
    a.correction[s] = sh_pick;
    if (a.status && sh_stat) atomicOr(&a.status[s], sh_stat);
    __hip_atomic_store(seq_counter(a, s), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Maximum of one float per thread over the workgroup, returned to every thread.
__device__ float block_max_all(float v) {
  __shared__ float sh_wave[kAccWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  v = wave_max(v);
  if (lane == 0) sh_wave[wave] = v;
  __syncthreads();
  float m = sh_wave[0];
  for (int w = 1; w < kAccWaves; ++w) m = fmaxf(m, sh_wave[w]);
  __syncthreads();
  return m;
}

// Row statistics for acceptance from logits: for every target and draft row
// (2 b B rows of V logits) the maximum m and s = sum_y exp((z_y - m) / T).
// Grid: rows x segments of 256 PER1 entries (PER1 per thread). Each
// workgroup reduces its segment to (m_j, s_j) -- s_j relative to its own
// maximum -- and publishes both with ready bits; the row's last arrival
// collects them, folds S = sum_j s_j exp((m_j - M) / T) with M = max_j m_j in a
// fixed order, writes (M, S) and clears its words and counter.
template <int PER1, bool UNIT_T>
__device__ __forceinline__ void row_stats_body(const AcceptArgs& a, const long id) {
  constexpr int SEG1 = PER1 * kAccThreads;
  __shared__ int sh_last;
  __shared__ double tab[256];  // 2^(j/256)
  const int nrow_half = a.b * a.B;
  // rows in storage order: every target row, then every draft row, so a
  // sequence's statistics are complete once its draft rows are, through the
  // second half of the pass (taking each sequence's 2 B rows together made
  // the pass 0.8-2.5 us slower)
  const int row = static_cast<int>(id / a.nseg1), seg = static_cast<int>(id % a.nseg1);
  const int V = a.V, tid = threadIdx.x;
  const float* z = (row < nrow_half ? a.zt : a.zd) + static_cast<size_t>(row % nrow_half) * V;
  const int xdraft = a.draft[row % nrow_half];  // the draft token of the row's position
  // thread tid takes the 4-entry pieces seg SEG1 + 4 (tid + 256 j): each load
  // instruction of a wave reads 1 KB of contiguous logits
  const int y0 = seg * SEG1 + 4 * tid;
  float v[PER1];
#pragma unroll
  for (int j = 0; j < PER1 / 4; ++j) {
    const int y = y0 + j * 4 * kAccThreads;
    if ((V % 4) == 0) {
      float4 f = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (y < V) f = load_nt4(z + y);
      v[4 * j] = f.x, v[4 * j + 1] = f.y, v[4 * j + 2] = f.z, v[4 * j + 3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = y + e < V ? __builtin_nontemporal_load(z + y + e) : -INFINITY;
    }
  }
  tab[tid] = kExp2Frac[tid];  // visible after the barrier in block_max_all
  // The workgroup whose segment holds the draft token leaves the logit there
  // beside the row's statistics, so the acceptance pass reads it together
  // with them instead of gathering it.
  const int xoff = xdraft - seg * SEG1;
  if (xoff >= 0 && xoff < SEG1 && xdraft < V && tid == (xoff % (4 * kAccThreads)) / 4) {
    float zx = 0.0f;
#pragma unroll
    for (int e = 0; e < PER1; ++e)
      if ((e / 4) * 4 * kAccThreads + (e % 4) == xoff - 4 * tid) zx = v[e];
    publish_word(row_stat_words(a, row) + 2, __float_as_uint(zx));
  }
  float tm = -INFINITY;
#pragma unroll
  for (int e = 0; e < PER1; ++e) tm = fmaxf(tm, v[e]);
  const float m = block_max_all(tm);
  const double md = static_cast<double>(m), inv_t = a.inv_t;
  double ts;
#pragma unroll
  for (int e = 0; e < PER1; ++e) {
    const double x = static_cast<double>(v[e]) - md;  // exact
    const double t = exp_nonpos_tab(UNIT_T ? x : x * inv_t, tab);
    ts = e == 0 ? t : ts + t;
  }
  const double sum = block_sum(ts);

  unsigned long long* words = a.row_words + static_cast<size_t>(row) * a.nseg1 * 2;
  if (tid == 0) {
    __hip_atomic_store(words + 2 * seg, static_cast<unsigned long long>(__float_as_uint(m)) | kReady,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(words + 2 * seg + 1,
                       static_cast<unsigned long long>(__double_as_longlong(sum)) | kReady, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    const int prev = __hip_atomic_fetch_add(row_counter(a, row), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == a.nseg1 - 1;
  }
  __syncthreads();
  if (!sh_last) return;

  // last arrival: every thread collects its segments (in order), clearing the
  // words it read (its own were published by thread 0, which clears them)
  constexpr int kMaxSegPerThread = (kMaxAcceptVocab / SEG1 + kAccThreads - 1) / kAccThreads;
  float mj[kMaxSegPerThread];
  double sj[kMaxSegPerThread];
  float tmax = -INFINITY;
  bool timed_out = false;
#pragma unroll
  for (int i = 0; i < kMaxSegPerThread; ++i) {
    const int j = tid + i * kAccThreads;
    mj[i] = -INFINITY;
    sj[i] = 0.0;
    if (j >= a.nseg1) continue;
    if (j == seg) {
      mj[i] = m;
      sj[i] = sum;  // thread 0 holds the block sum; broadcast below
      continue;
    }
    unsigned long long wm = 0, ws = 0;
    int polls = 0;
    do {
      wm = __hip_atomic_load(words + 2 * j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ws = __hip_atomic_load(words + 2 * j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((wm & kReady) && (ws & kReady)) break;
      __builtin_amdgcn_s_sleep(1);
    } while (++polls < kPollLimit);
    timed_out |= !((wm & kReady) && (ws & kReady));
    mj[i] = __uint_as_float(static_cast<uint32_t>(wm));
    sj[i] = __longlong_as_double(static_cast<long long>(ws & ~kReady));
    __hip_atomic_store(words + 2 * j, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(words + 2 * j + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the own segment's sum lives in thread 0 (block_sum); hand it to its owner
  __shared__ double sh_own;
  if (tid == 0) {
    sh_own = sum;
    __hip_atomic_store(words + 2 * seg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(words + 2 * seg + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxSegPerThread; ++i) {
    if (tid + i * kAccThreads == seg) sj[i] = sh_own;
    tmax = fmaxf(tmax, mj[i]);
  }
  const float M = block_max_all(tmax);
  double part = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxSegPerThread; ++i)
    if (tid + i * kAccThreads < a.nseg1)
      part += sj[i] * exp_nonpos_tab<true>((static_cast<double>(mj[i]) - static_cast<double>(M)) * a.inv_t, tab);
  const double S = block_sum(part);
  if (timed_out && a.status) atomicOr(&a.status[(row % nrow_half) / a.B], kDevSyncTimeout);
  if (tid == 0) {
    publish_word(row_stat_words(a, row), __float_as_uint(M));
    publish_word(row_stat_words(a, row) + 1, static_cast<unsigned long long>(__double_as_longlong(1.0 / S)));
    __hip_atomic_store(row_counter(a, row), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int PER, bool LOGITS>
__global__ __launch_bounds__(kAccThreads) void accept_kernel(AcceptArgs a) {
  extern __shared__ double dyn_mass[];  // one mass per segment
  accept_body<PER, LOGITS>(a, blockIdx.x, gridDim.x, blockIdx.y, dyn_mass);
}

template <int PER1, bool UNIT_T>
__global__ __launch_bounds__(kAccThreads) void row_stats_kernel(AcceptArgs a) {
  row_stats_body<PER1, UNIT_T>(a, blockIdx.x);
}

// Acceptance from logits in one launch: the first `units` workgroups compute
// the row statistics, the rest (one per (sequence, segment)) run acceptance,
// each waiting (bounded) for its sequence's statistics. Workgroups are
// dispatched in id order, so every statistics workgroup has been dispatched
// before an acceptance workgroup can start waiting for it, and the waits end.
template <int PER1, bool UNIT_T, int PER>
__global__ __launch_bounds__(kAccThreads) void accept_logits_kernel(
    AcceptArgs a, long units, int nseg) {
  extern __shared__ double dyn_mass[];
  const long id = blockIdx.x;
  if (id < units) {
    row_stats_body<PER1, UNIT_T>(a, id);
    return;
  }
  const long k = id - units;
  accept_body<PER, true>(a, static_cast<int>(k % nseg), nseg, static_cast<int>(k / nseg), dyn_mass);
}

// Entries per thread (segment width / 256): 4 (1024-entry segments). With
// the arrival counters on their own cache lines, more and shorter segments
// win at every measured shape (one MI355X, back to back, 4 / 8 / 16:
// b = 16, V = 32768 -> 9.0 / 9.8 / 11.9 us; b = 64, V = 32768 -> 11.9 / 13.5 /
// 15.1 us; b = 8, V = 151936 -> 11.4 / 12.5 / 14.1 us). The tuning override
// SIMSD_TUNE_ACCEPT_PER = 4, 8 or 16 replaces it.
int accept_per(int b, int V) {
  const int forced = tuning(SIMSD_TUNE_ACCEPT_PER);
  if (forced == 4 || forced == 8 || forced == 16) return forced;
  (void)b, (void)V;
  return 4;
}

}  // namespace

int accept_segments(int V) { return (V + kAccThreads * kMinPer - 1) / (kAccThreads * kMinPer); }

template <bool LOGITS>
hipError_t launch_accept_mode(const AcceptArgs& a, hipStream_t stream) {
  const int per = accept_per(a.b, a.V);
  const int nseg = (a.V + kAccThreads * per - 1) / (kAccThreads * per);
  dim3 grid(static_cast<unsigned>(nseg), static_cast<unsigned>(a.b));
  const size_t dyn = static_cast<size_t>(nseg) * sizeof(double);
  if (per == 4)
    hipLaunchKernelGGL((accept_kernel<4, LOGITS>), grid, dim3(kAccThreads), dyn, stream, a);
  else if (per == 8)
    hipLaunchKernelGGL((accept_kernel<8, LOGITS>), grid, dim3(kAccThreads), dyn, stream, a);
  else
    hipLaunchKernelGGL((accept_kernel<16, LOGITS>), grid, dim3(kAccThreads), dyn, stream, a);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) { return launch_accept_mode<false>(a, stream); }

// Entries per thread of the row-statistics pass: 16 (4096-entry segments).
// The pass is bound by VALU issue (about 19 instructions per logit with the
// table exp, every one a 4-cycle wave issue) more than by HBM, so the shortest
// segments, whose workgroups (56 VGPRs, 8 waves per SIMD) overlap one
// another's loads and arithmetic best, win (one MI355X, kernel trace, 16 / 32
// / 64 per thread: V = 151936 with 256 rows -> 43.6 / 45.1 / 46.4 us; V =
// 32768 with 1024 rows -> 37.6 / 41.0 / 42.2 us; a variant streaming longer
// runs with prefetch measured 42.9 us on the first). The tuning override
// SIMSD_TUNE_ROWSTAT_PER = 16, 32 or 64 replaces the default.
// Statistics and acceptance go in one launch when the statistics grid takes
// at least two rounds of resident workgroups (MI355X: 256 CUs x 8), so that
// the acceptance of the sequences done early overlaps the rest of the
// statistics; a grid that fits one round gains no overlap, and the waiting
// acceptance workgroups cost it. Interleaved runs (event pairs, logits copies
// rotated past the MALL), two launches -> one: b = 64 B = 8 V = 32768
// 51.7 -> 47.7 us, b = 8 B = 16 V = 151936 53.7 -> 53.3 us; with the rows
// in sequence order (which slowed the pass itself) also b = 16 B = 16 V =
// 151936 91.4 -> 88.4, b = 32 B = 8 V = 32768 35.0 -> 32.8, b = 32 B = 4
// V = 65536 37.2 -> 32.6, b = 4 B = 16 V = 151936 37.1 -> 36.5, but b = 16
// B = 8 V = 32768 (2048 statistics workgroups, one round) 25.1 -> 26.4.
constexpr long kOneLaunchMinRowStatUnits = 2L * 256 * 8;
int row_stat_per() {
  const int forced = tuning(SIMSD_TUNE_ROWSTAT_PER);
  return (forced == 16 || forced == 32 || forced == 64) ? forced : 16;
}

hipError_t launch_accept_logits(const AcceptArgs& a0, hipStream_t stream) {
  AcceptArgs a = a0;
  const int per1 = row_stat_per();
  a.nseg1 = (a.V + kAccThreads * per1 - 1) / (kAccThreads * per1);
  const long units = 2L * a.b * a.B * a.nseg1;
  const dim3 grid(static_cast<unsigned>(units)), block(kAccThreads);
  // T = 1 (inverse temperature exactly 1) skips a multiply per logit
  const bool unit = a.inv_t == 1.0;
  const int per = accept_per(a.b, a.V);
  const int nseg = (a.V + kAccThreads * per - 1) / (kAccThreads * per);
  const long one_grid = units + static_cast<long>(nseg) * a.b;
  if (units >= kOneLaunchMinRowStatUnits && per1 == 16 && per == 4 && one_grid <= kMaxRowStatUnits) {
    // the default widths: statistics and acceptance in one launch (a grid as
    // large as one statistics pass may be)
    const dim3 g1(static_cast<unsigned>(one_grid));
    const size_t dyn = static_cast<size_t>(nseg) * sizeof(double);
    if (unit)
      hipLaunchKernelGGL((accept_logits_kernel<16, true, 4>), g1, block, dyn, stream, a, units, nseg);
    else
      hipLaunchKernelGGL((accept_logits_kernel<16, false, 4>), g1, block, dyn, stream, a, units, nseg);
    return hipGetLastError();
  }
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, a); };
  if (per1 == 16)
    unit ? go(row_stats_kernel<16, true>) : go(row_stats_kernel<16, false>);
  else if (per1 == 32)
    unit ? go(row_stats_kernel<32, true>) : go(row_stats_kernel<32, false>);
  else
    unit ? go(row_stats_kernel<64, true>) : go(row_stats_kernel<64, false>);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_accept_mode<true>(a, stream);
}

}  // namespace simsd
