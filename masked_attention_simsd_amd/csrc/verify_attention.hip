// verify_attention.hip -- one attention pass of SimSD verification on gfx950.
//
// What is computed (SimSD pages, [nl] "Technische Samenvatting: SimSD - Simple
// Speculative Decoding in Diffusion Language Models" and [fr] "SimSD: Simple
// Speculative Decoding in Diffusion Language Models", Methodologie 1, 2, 4):
// every query row of the paired block (data tokens D, mask slots D~) attends
// to the whole cached prompt prefix plus the block keys its temporal step
// allows; a mask slot D~_i sees D_j iff tau(j) < tau(i) and D~_j iff
// tau(j) >= tau(i). The data-row rule is a flag (causal / bidirectional /
// skip). Masked keys are excluded from the softmax, not biased.
//
// Design (MI355X-first):
//  * Work unit = (sequence, KV head, row slice). All G query heads of a KV
//    head and all block rows form M = G * rows query rows, so every K/V byte
//    fetched from HBM feeds M rows (grouped-query reuse). M is covered by up
//    to 4 compute waves of 1-2 MFMA row blocks of 16.
//  * The prefix is split into chunks of `chunk` keys (split-KV), one
//    workgroup per (unit, chunk), so a long prefix fills all 256 CUs. The
//    block keys (2B <= 128) are taken by the workgroup of chunk 0 after its
//    prefix keys, with the temporal mask generated from tau held in LDS.
//  * Key tiles of 64 keys are streamed HBM -> registers (16-byte loads, one
//    tile of prefetch ahead) -> LDS. K is stored row-major; V is stored
//    transposed with an XOR-swizzled key column so the PV operand is one
//    16-byte LDS read and the transposing writes do not collide on banks.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with fp32
//    accumulation. The S^T output layout puts 8 consecutive keys of one query
//    in each lane, which is exactly the P^T operand of the PV product, so the
//    softmax never leaves registers. Row maxima need two cross-lane steps;
//    row sums stay lane-local until the end.
//  * Split partials (m, l, unnormalised O) go to the workspace in register
//    order; the last workgroup of a unit to finish (agent-scope counter)
//    merges them with the log-sum-exp rule and writes the output, then resets
//    the counter. Workgroup ids are remapped so that the chunks of one unit
//    run on the same XCD (ids are dispatched round-robin over the 8 XCDs).
#include "simsd_internal.h"

#include <algorithm>
#include <cstdlib>

namespace simsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TK = kAttnTileKeys;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct AttnSmem {
  uint16_t k[TK][D + 8];   // key tile, row-major, 16-byte row pad
  uint16_t vt[D][TK + 8];  // value tile transposed; key column XOR (4 * (d / 8))
  int tau[64];
  int last;
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  union {
    uint4 u;
    bf16x8 b;
  } c;
  c.u = v;
  return c.b;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Temporal mask between block rows (query row qr with slot flag / label, key
// block row c). See the header comment for the rule.
__device__ __forceinline__ bool block_allowed(bool q_slot, int tau_q, int c, int B,
                                              const int* tau_s, int data_rule) {
  const bool k_slot = c >= B;
  const int tau_k = tau_s[k_slot ? c - B : c];
  if (q_slot) return k_slot ? (tau_k >= tau_q) : (tau_k < tau_q);
  if (k_slot) return false;
  return data_rule == 1 ? true : (tau_k <= tau_q);
}

template <int D, int NWC, int QB, bool OUT_F32>
__global__ __launch_bounds__(kAttnThreads) void verify_attn_kernel(AttnArgs a) {
  constexpr int KK = D / 32;                        // MFMA k-steps of Q.K
  constexpr int DB = D / 16;                        // 16-wide d blocks of P.V
  constexpr int CH = D / 8;                         // 16-byte chunks per row
  constexpr int CPT = TK * CH / kAttnThreads;       // chunks per thread per tensor
  constexpr int MWG = NWC * QB * 16;                // query rows per workgroup
  static_assert(CPT >= 1 && TK * CH % kAttnThreads == 0, "tile/thread mismatch");
  static_assert(NWC >= 1 && NWC <= 4, "compute waves");

  __shared__ AttnSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int a16 = lane >> 4, n16 = lane & 15;

  // ---- which (sequence, KV head, row slice, split) this workgroup owns ----
  const int wg = blockIdx.x;
  const int logical = (wg & 7) * (a.total_grid >> 3) + (wg >> 3);
  if (logical >= a.total_real) return;
  const int split = logical % a.nsplit;
  const int us = logical / a.nsplit;
  const int slice = us % a.row_slices;
  const int unit = us / a.row_slices;
  const int s = unit / a.Hkv, g = unit % a.Hkv;
  const int B = a.B, twoB = 2 * a.B;

  int P = a.offsets[s + 1] - a.offsets[s];
  const bool bad_prefix = P < 0 || P > a.max_prefix;
  P = P < 0 ? 0 : (P > a.max_prefix ? a.max_prefix : P);
  const int ns = P > 0 ? (P + a.chunk - 1) / a.chunk : 1;
  if (split >= ns) return;
  const int key_lo = split * a.chunk;
  const int key_hi = min(P, key_lo + a.chunk);
  const bool with_block = split == 0;

  if (tid < 64) sm.tau[tid] = tid < B ? a.tau[static_cast<size_t>(s) * B + tid] : 0;
  __syncthreads();

  if (a.status && split == 0 && slice == 0 && g == 0 && wave == 0) {
    int cnt = 0;
    if (lane < B)
      for (int k = 0; k < B; ++k) cnt += sm.tau[k] == lane + 1;
    const bool bad_tau = __ballot(lane < B && cnt != 1) != 0ull;
    if (lane == 0 && (bad_tau || bad_prefix))
      atomicOr(&a.status[s], (bad_tau ? kDevBadTau : 0) | (bad_prefix ? kDevBadPrefix : 0));
  }

  // ---- this lane's queries: one per 16-row block, row m of the unit ----
  const bool computes = wave < NWC;
  bf16x8 qreg[QB][KK];
  int tau_q[QB];
  bool slot_q[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = slice * MWG + (wave * QB + qb) * 16 + n16;
    const bool valid = computes && m < a.M;
    const int r = a.row0 + (valid ? m / a.G : 0);
    const int h = g * a.G + (valid ? m % a.G : 0);
    const uint16_t* qrow = a.q_blk + ((static_cast<size_t>(s) * twoB + r) * a.Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (valid) v = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * a16);
      qreg[qb][kk] = as_bf16x8(v);
    }
    slot_q[qb] = r >= B;
    tau_q[qb] = sm.tau[r >= B ? r - B : r];
  }

  f32x4 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tile schedule: prefix tiles of this chunk, then the block tiles ----
  const size_t row_stride = static_cast<size_t>(a.Hkv) * D;
  const uint16_t* kpre = a.k_pre + (static_cast<size_t>(a.offsets[s]) * a.Hkv + g) * D;
  const uint16_t* vpre = a.v_pre + (static_cast<size_t>(a.offsets[s]) * a.Hkv + g) * D;
  const uint16_t* kblk = a.k_blk + (static_cast<size_t>(s) * twoB * a.Hkv + g) * D;
  const uint16_t* vblk = a.v_blk + (static_cast<size_t>(s) * twoB * a.Hkv + g) * D;
  const int n_pre = (key_hi - key_lo + TK - 1) / TK;
  const int n_blk = with_block ? (twoB + TK - 1) / TK : 0;
  const int ntiles = n_pre + n_blk;

  uint4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int t) {
    const bool blk = t >= n_pre;
    const int r0 = blk ? (t - n_pre) * TK : key_lo + t * TK;
    const int nvalid = blk ? min(TK, twoB - r0) : min(TK, key_hi - r0);
    const uint16_t* kb = blk ? kblk : kpre;
    const uint16_t* vb = blk ? vblk : vpre;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kAttnThreads * i;
      const int j = c / CH, cc = c % CH;
      if (j < nvalid) {
        const size_t off = static_cast<size_t>(r0 + j) * row_stride + cc * 8;
        kreg[i] = *reinterpret_cast<const uint4*>(kb + off);
        vreg[i] = *reinterpret_cast<const uint4*>(vb + off);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);  // zero keys/values: no NaN from stale LDS
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kAttnThreads * i;
      const int j = c / CH, cc = c % CH;
      *reinterpret_cast<uint4*>(&sm.k[j][cc * 8]) = kreg[i];
      const int jp = j ^ (4 * cc);
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.vt[cc * 8 + 2 * e][jp] = static_cast<uint16_t>(w[e]);
        sm.vt[cc * 8 + 2 * e + 1][jp] = static_cast<uint16_t>(w[e] >> 16);
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);
    if (!computes) continue;

    const bool blk = t >= n_pre;
    const int r0 = blk ? (t - n_pre) * TK : key_lo + t * TK;
    const int nvalid = blk ? min(TK, twoB - r0) : min(TK, key_hi - r0);
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      if (32 * ks >= nvalid) break;
      // S^T block kb: MFMA row mr -> key 32ks + 8(mr/4) + 4kb + mr%4
      f32x4 sacc[QB][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key_m = 32 * ks + 8 * (n16 >> 2) + 4 * kb + (n16 & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ak = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.k[key_m][32 * kk + 8 * a16]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qreg[qb][kk], sacc[qb][kb], 0, 0, 0);
        }
      }
      // lane holds keys 32ks + 8*a16 + (4kb + i) of query n16
      bf16x8 pop[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float sv[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kl = 32 * ks + 8 * a16 + 4 * kb + i;
            bool ok = kl < nvalid;
            if (blk && ok) ok = block_allowed(slot_q[qb], tau_q[qb], r0 + kl, B, sm.tau, a.data_rule);
            sv[4 * kb + i] = ok ? sacc[qb][kb][i] * a.scale_log2 : -INFINITY;
          }
        float mx = sv[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
        m_run[qb] = m_new;
        uint32_t pk[4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(sv[2 * j] - m_use);
          const float p1 = __builtin_amdgcn_exp2f(sv[2 * j + 1] - m_use);
          pk[j] = pack_bf16x2(p0, p1);
          psum += bf16_to_f32(static_cast<uint16_t>(pk[j])) + bf16_to_f32(static_cast<uint16_t>(pk[j] >> 16));
        }
        l_run[qb] = l_run[qb] * alpha + psum;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
        pop[qb] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
      // O^T += V^T P^T: operand = 8 consecutive keys of column d
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + n16;
        const int pb = (4 * ks + a16) ^ db;
        uint4 raw = *reinterpret_cast<const uint4*>(&sm.vt[d][8 * pb]);
        if (n16 & 8) raw = make_uint4(raw.z, raw.w, raw.x, raw.y);  // halves swapped by the swizzle
        const bf16x8 av = as_bf16x8(raw);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pop[qb], oacc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- finish: full row sums, then either write or hand off to the merge ----
  float l_tot[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    l_tot[qb] = l;
  }

  if (ns > 1) {
    const size_t part = static_cast<size_t>(us) * a.nsplit + split;
    if (computes) {
      f32x4* po = reinterpret_cast<f32x4*>(a.part_o) + part * (NWC * QB * DB * 64);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) po[((wave * QB + qb) * DB + db) * 64 + lane] = oacc[qb][db];
      if (a16 == 0) {
        float2* pml = reinterpret_cast<float2*>(a.part_ml) + part * MWG;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) pml[(wave * QB + qb) * 16 + n16] = make_float2(m_run[qb], l_tot[qb]);
      }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = __hip_atomic_fetch_add(&a.counters[us], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      sm.last = prev == ns - 1;
    }
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
    if (computes) {
      const size_t part0 = static_cast<size_t>(us) * a.nsplit;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = (wave * QB + qb) * 16 + n16;
        float mmax = -INFINITY;
        for (int k = 0; k < ns; ++k) {
          const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[(part0 + k) * MWG + row];
          mmax = fmaxf(mmax, ml.x);
        }
        const float m_use = mmax == -INFINITY ? 0.0f : mmax;
        float lsum = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < ns; ++k) {
          const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[(part0 + k) * MWG + row];
          const float w = __builtin_amdgcn_exp2f(ml.x - m_use);
          lsum += w * ml.y;
          const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o) + (part0 + k) * (NWC * QB * DB * 64);
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[qb][db] += w * po[((wave * QB + qb) * DB + db) * 64 + lane];
        }
        m_run[qb] = mmax;
        l_tot[qb] = lsum;
      }
    }
    if (tid == 0) __hip_atomic_store(&a.counters[us], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!computes) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = slice * MWG + (wave * QB + qb) * 16 + n16;
    if (m >= a.M) continue;
    const int r = a.row0 + m / a.G;
    const int h = g * a.G + m % a.G;
    const size_t orow = (static_cast<size_t>(s) * twoB + r) * a.Hq + h;
    const float inv_l = 1.0f / l_tot[qb];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const f32x4 o = oacc[qb][db] * inv_l;
      const int d0 = 16 * db + 4 * a16;
      if (OUT_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow * D + d0) = o;
      } else {
        uint2 v;
        v.x = pack_bf16x2(o[0], o[1]);
        v.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow * D + d0) = v;
      }
    }
    if (a.lse && a16 == 0) a.lse[orow] = (m_run[qb] + __log2f(l_tot[qb])) * kLn2;
  }
}

template <int D, int NWC, int QB>
hipError_t launch_variant(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.total_grid)), block(kAttnThreads);
  if (a.out_f32)
    hipLaunchKernelGGL((verify_attn_kernel<D, NWC, QB, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((verify_attn_kernel<D, NWC, QB, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if (p.nwc == 1) return launch_variant<D, 1, 1>(a, stream);
  if (p.nwc == 2) return launch_variant<D, 2, 1>(a, stream);
  if (p.qb == 1) return launch_variant<D, 4, 1>(a, stream);
  return launch_variant<D, 4, 2>(a, stream);
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

}  // namespace

// Launch plan: rows per workgroup from M = G * rows, then the number of
// prefix splits so that about `target` workgroups cover the prefix, with
// chunks no longer than `chunk_max` keys (keeps ragged batches balanced).
// Tuning overrides: SIMSD_ATTN_TARGET_WG, SIMSD_ATTN_CHUNK_MAX.
AttnPlan plan_attention(int b, int B, int Hq, int Hkv, int d, int max_prefix, int data_rule) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int nrows = data_rule == 2 ? B : 2 * B;
  const int M = nrows * G;
  if (M <= 16) {
    p.nwc = 1, p.qb = 1;
  } else if (M <= 32) {
    p.nwc = 2, p.qb = 1;
  } else if (M <= 64) {
    p.nwc = 4, p.qb = 1;
  } else {
    p.nwc = 4, p.qb = 2;
  }
  p.rows_per_wg = p.nwc * p.qb * 16;
  p.row_slices = (M + p.rows_per_wg - 1) / p.rows_per_wg;
  const int target = std::max(1, env_int("SIMSD_ATTN_TARGET_WG", 512));
  const int chunk_max = std::max(TK, env_int("SIMSD_ATTN_CHUNK_MAX", 2048) / TK * TK);
  const long units = static_cast<long>(b) * Hkv * p.row_slices;
  const int max_tiles = std::max(1, (max_prefix + TK - 1) / TK);
  int nsplit = static_cast<int>(std::min<long>(max_tiles, std::max<long>(1, (target + units - 1) / units)));
  int chunk = ((max_prefix + nsplit - 1) / nsplit + TK - 1) / TK * TK;
  chunk = std::max(TK, std::min(chunk, chunk_max));
  nsplit = std::max(1, (max_prefix + chunk - 1) / chunk);
  p.chunk = chunk;
  p.nsplit = nsplit;
  const size_t us = static_cast<size_t>(units);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  // The counter words sit in a region of fixed size at the start of every
  // workspace, so calls of different shapes never write partials over
  // another shape's counters (which must stay zero between calls).
  p.counters_bytes = static_cast<size_t>(kAttnMaxUnits) * sizeof(int32_t);
  p.ml_bytes = nsplit > 1 ? up(us * nsplit * p.rows_per_wg * 2 * sizeof(float)) : 0;
  p.o_bytes = nsplit > 1 ? up(us * nsplit * p.rows_per_wg * static_cast<size_t>(d) * sizeof(float)) : 0;
  p.total_bytes = p.counters_bytes + p.ml_bytes + p.o_bytes;
  return p;
}

hipError_t launch_verify_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, p, stream);
  return launch_d<128>(a, p, stream);
}

}  // namespace simsd
