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
//  * The prefix is split into chunks (split-KV), about one workgroup per CU,
//    so a long prefix fills all 256 CUs. The block keys (2B <= 128) are taken
//    by the workgroup of chunk 0 after its prefix keys, with the temporal mask
//    generated from tau held in LDS.
//  * Key tiles stream HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging) into a ring of NS tiles; NS - 1 tiles are in flight while one is
//    consumed, with one barrier per tile. K and V stay row-major in LDS with
//    XOR-swizzled 16-byte chunks so that the K operand reads and the
//    transposing V reads (ds_read_b64_tr_b16, which yields the V^T operand
//    from row-major V) hit distinct banks.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with fp32
//    accumulation. The S^T output layout puts 8 consecutive keys of one query
//    in each lane, which is exactly the P^T operand of the PV product, so the
//    softmax never leaves registers. Row maxima and sums over the 4 lanes of a
//    query use lane swaps; O is rescaled only when a row maximum moved.
//  * Split partials (m, l, unnormalised O) are handed to the last workgroup
//    of the unit to finish through device-coherent 16-byte stores / loads and
//    an agent-scope counter (no cache-wide fences); it merges them with the
//    log-sum-exp rule, writes the output and resets the counter. Workgroup ids
//    are remapped so the chunks of one unit run on the same XCD (ids are
//    dispatched round-robin over the 8 XCDs).
#include "simsd.h"
#include "simsd_internal.h"

#include <algorithm>

namespace simsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define SIMSD_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.6931471805599453f;
// block-key rule of a kernel instance (its MODE template argument)
constexpr int kModeTau = 0, kModeTauRope = 1, kModeMask = 2;
constexpr int TK = kAttnTileKeys;  // chunk granularity of the split plan

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  union {
    uint4 u;
    bf16x8 b;
  } c;
  c.u = v;
  return c.b;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  union {
    bf16x2 b;
    uint32_t u;
  } c;
  c.b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);  // v_cvt_pk_bf16_f32, nearest even
  return c.u;
}

// 16 bytes HBM -> LDS without passing through registers (global_load_lds_dwordx4,
// scalar-base form): lane l reads sbase + voff and its bytes land at LDS byte
// address m0 + 16 * l; `sbase` and `lds` are wave-uniform. Issued as inline asm
// so that the compiler does not add its own (conservative) wait before later
// LDS reads; the kernel waits explicitly with vmcnt.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

// The same with the non-temporal hint, for the key/value stream, which each
// launch reads once: streaming-read probes (256 workgroups, 1 MiB runs, a
// four-stage 16 KB ring) reach 6.9 TB/s with it against 6.1 without.
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

// 4 bytes HBM -> LDS (global_load_lds_dword): lane l reads sbase + voff and
// its word lands at LDS byte address m0 + 4 * l.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer descriptor over [base, base + bytes) for device-coherent (sc1) 8- and
// 16-byte accesses: partials written by one workgroup are read by another,
// possibly on another XCD, without cache-wide writeback or invalidation.
constexpr int kCoherent = 16;  // cache-policy bit selecting sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

// Max / sum of x over lanes l, l^16, l^32, l^48 (the four lanes holding one
// query row) with the VALU lane-swap instructions instead of LDS permutes.
__device__ __forceinline__ float max_over_row_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_row_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most n vector-memory loads of this wave are outstanding.
// Wait until tile t has landed when `ahead` younger tiles (DPW DMA instructions
// each) may stay in flight: vmcnt(ahead * DPW), with ahead <= A.
template <int DPW, int A>
__device__ __forceinline__ void wait_tile(int ahead);

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0) only
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int DPW, int A>
__device__ __forceinline__ void wait_tile(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) wait_vmcnt<A * DPW>();
    else wait_tile<DPW, A - 1>(ahead);
  }
}

// XOR swizzles of the 16-byte chunks inside a key row of a staged tile. A K
// operand read (16 lanes, rows 8(n/4) + n%4, one chunk column) and a V operand
// transposing read (32 lanes, 8 rows x 32 bytes) then touch distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return (row & 3) | (((row >> 3) & 3) << 2);
  else return ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return ((row & 3) | (((row >> 3) & 1) << 2)) << 1;
  else return (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) << 1;
}

// Temporal mask between block rows, branch-free: query with slot flag / label,
// key block row with slot flag / label (a data token D_j or mask slot D~_j,
// label tau(j)).
__device__ __forceinline__ bool block_allowed(bool q_slot, int tau_q, bool k_slot, int tau_k, int data_rule) {
  const bool slot_row = k_slot ? (tau_k >= tau_q) : (tau_k < tau_q);
  const bool data_row = !k_slot && (data_rule == 1 || tau_k <= tau_q);
  return q_slot ? slot_row : data_row;
}

// Doubles per row of the fused-RoPE cos/sin table: D/2 (cos, sin) pairs plus
// one pad pair, so that rows a bank period apart (D * 8 bytes) do not map to
// the same LDS banks when lanes of different rows read the same frequency.
template <int D>
__host__ __device__ constexpr int rope_row_doubles() {
  return D + 2;
}

// RoPE-copy table row of block row r: data row D_{r+1} and (with the copy
// rule) mask slot D~_{r-B+1} share position r resp. r - B; without the copy
// rule the slot keeps its own row r (position start + r).
__device__ __forceinline__ int rope_pos_row(int r, int B, int no_copy) {
  return r < B ? r : (no_copy ? r : r - B);
}

// Rotate one query or key row held as this lane's KK chunks of 8 elements:
// chunk kk holds elements 32 kk + 8 a16 + j. Rotate-half pairs element e with
// e + D/2 (chunk kk + KK/2, same lane); interleaved pairs 2i with 2i + 1
// (neighbours in one chunk). Table row `pr` holds (cos, sin) per frequency.
template <int D, int KK>
__device__ __forceinline__ void rope_rows(bf16x8 (&x)[KK], int pr, int a16, int interleaved,
                                          const double* tab) {
  const double* t = tab + static_cast<size_t>(pr) * rope_row_doubles<D>();  // D/2 (cos, sin) pairs
  union U {
    bf16x8 b;
    uint16_t h[8];
  };
  if (!interleaved) {
#pragma unroll
    for (int kk = 0; kk < KK / 2; ++kk) {
      U lo, hi;
      lo.b = x[kk];
      hi.b = x[kk + KK / 2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * kk + 8 * a16 + j;
        rope_rotate(lo.h[j], hi.h[j], t[2 * i], t[2 * i + 1], &lo.h[j], &hi.h[j]);
      }
      x[kk] = lo.b;
      x[kk + KK / 2] = hi.b;
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      U v;
      v.b = x[kk];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int i = (32 * kk + 8 * a16 + j) / 2;
        rope_rotate(v.h[j], v.h[j + 1], t[2 * i], t[2 * i + 1], &v.h[j], &v.h[j + 1]);
      }
      x[kk] = v.b;
    }
  }
}

// D head dim; NW waves per workgroup (all issue the DMA), of which NWC x KS
// compute: NWC row groups of QB 16-row query blocks, and KS waves per row
// group that take disjoint slices of every key tile (KS = 2 puts two
// independent waves on each SIMD, so one's MFMA work overlaps the other's
// softmax; their states are merged through LDS at the end); TK keys per staged
// tile; NS tiles in the LDS ring (NS - 1 in flight while one is consumed).
// MODE selects the block-key rule and is fixed at compile time, so the
// temporal-mask kernels carry none of the other modes' code:
//   kModeTau     the temporal mask from tau;
//   kModeTauRope the same with RoPE-copy fused into the prologue -- the query
//                rows and the block key rows are rotated on the fly from a
//                per-workgroup cos/sin table (dynamic LDS);
//   kModeMask    an explicit block mask (bit words per block row), no tau.
template <int D, int NW, int NWC, int QB, int TKEYS, int NS, int KS, int MODE, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) void verify_attn_kernel(AttnArgs a) {
  constexpr bool ROPE = MODE == kModeTauRope;
  constexpr bool MASK = MODE == kModeMask;
  constexpr int TK = TKEYS;         // keys per staged tile
  constexpr int KK = D / 32;          // MFMA k-steps of Q.K
  constexpr int DB = D / 16;          // 16-wide d blocks of P.V
  constexpr int CH = D / 8;           // 16-byte chunks per key row
  constexpr int ROW_B = D * 2;        // bytes per key row
  constexpr int RPI = 1024 / ROW_B;   // key rows per DMA wave instruction
  constexpr int IPW = TK / RPI / NW;  // DMA instructions per wave per tensor per tile
  constexpr int DPW = 2 * IPW;        // ... for K and V together
  constexpr int TENSOR_B = TK * ROW_B;
  constexpr int STAGE_B = 2 * TENSOR_B;
  constexpr int TKW = TK / KS;        // keys of a tile per computing wave
  constexpr int NSUB = TKW / 32;      // 32-key PV steps per tile and wave
  constexpr int NKB = TKW / 16;       // 16-key S^T blocks per tile and wave
  constexpr int MWG = NWC * QB * 16;  // query rows per workgroup
  static_assert(IPW >= 1 && (TK / RPI) % NW == 0 && NWC * KS <= NW, "tile / wave mismatch");
  static_assert(TKW % 32 == 0 && (KS == 1 || KS == 2), "key slice per wave");
  static_assert(KS == 1 || NWC * QB * (D / 16) * 64 * 16 <= NS * STAGE_B, "state exchange fits the ring");
  static_assert(NS >= 2 && (NS - 1) * DPW < 64, "pipeline depth");
  static_assert(NS * STAGE_B <= 150 * 1024, "LDS ring");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE_B];
  __shared__ float xml[KS == 2 ? NWC * QB * 64 * 2 : 1];  // (m, l) handed between key slices
  __shared__ int tau_s[64];
  __shared__ int pos_s[ROPE ? 64 : 1];  // fused RoPE with a position per pair
  __shared__ int vbad_s;                // a block V row held a non-finite value (split 0)
  __shared__ int last_s;
  extern __shared__ double rope_tab[];  // ROPE: [position][d/2] x (cos, sin), rows padded

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps DMA math scalar
  const int a16 = lane >> 4, n16 = lane & 15;

  // ---- which (sequence, KV head, row slice, split) this workgroup owns ----
  const int wg = blockIdx.x;
  const int logical = a.lpt ? wg : (a.xcd_remap ? (wg & 7) * (a.total_grid >> 3) + (wg >> 3) : wg);
  if (logical >= a.total_real) return;
  const int split = logical % a.nsplit;
  const int us = logical / a.nsplit;
  const int slice = us % a.row_slices;
  const int unit = us / a.row_slices;
  int s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  if (a.lpt) {
    // Longest first (unsplit launches of at most 64 sequences whose
    // workgroups do not all fit at once): workgroups are dispatched in id
    // order, so the k-th group of Hkv ids takes the k-th longest sequence and
    // the short ones fill the CUs that free up at the end. Wave 0 ranks the
    // sequences by prefix length (ties by index), identically in every
    // workgroup, and picks the one of rank s.
    __shared__ int lpt_seq;
    if (wave == 0) {
      const int sl = lane < a.b ? lane : 0;
      int pl = a.prefix_lens[sl] - (a.prefix_lens_are_ends ? a.offsets[sl] : 0);
      pl = lane < a.b ? max(pl, 0) : -1;
      int rank = 0;
      for (int t = 0; t < kWave; ++t) {
        const int pt = __shfl(pl, t, kWave);
        rank += (pt > pl || (pt == pl && t < lane)) ? 1 : 0;
      }
      const unsigned long long hit = __ballot(lane < a.b && rank == s);
      if (lane == 0) lpt_seq = __ffsll(static_cast<long long>(hit)) - 1;
    }
    __syncthreads();
    s = lpt_seq;
  }
  // block keys: the 2B rows of the paired block, or the R rows of an
  // explicit-mask call (no tau, B = 0)
  const int B = a.B, twoB = MASK ? a.nblk : 2 * a.B;

  // the prefix: the first P rows of the region [offsets[s], offsets[s+1]):
  // P = prefix_ends[s] - offsets[s] with prefix_ends = offsets + 1 (the whole
  // region), or P = prefix_lens[s] for a cache with room to grow. Three
  // independent scalar loads either way, no branch before the first DMA.
  const int o0 = a.offsets[s];
  const int cap = a.offsets[s + 1] - o0;
  int P = a.prefix_lens[s] - (a.prefix_lens_are_ends ? o0 : 0);
  // read before the first DMA is issued, so it can be a scalar load (the DMA
  // asm clobbers memory as far as the compiler knows)
  // (with a position per pair the table reads them from LDS, staged below;
  // this then loads the sequence's first one, unused)
  const long pos0 = ROPE ? static_cast<long>(a.start_pos[a.rope_positions ? s * a.B : s]) : 0;
  const int rows_total = a.offsets[a.b];  // rows of a head-major cache per KV head

  // ---- tau, the workgroup's query rows (and the RoPE frequencies) ----
  // Staged into LDS by DMA at kernel entry when the rows fit one ring stage
  // (every default plan): tau into tau_s, the MWG query rows into ring slot
  // NS - 1, which the ring first fills at the first pipeline step, and with
  // fused RoPE the frequencies (kernel arguments) behind the cos/sin table.
  // Their addresses need no loaded value, so they are requested before the
  // prefix bounds arrive; loads complete in issue order, so the later wait
  // for them leaves the first key tiles in flight, and the work between that
  // wait and the first tile (table, query rotation, mask bits) overlaps the
  // ring fill. (Plain loads would need a compiler wait for every outstanding
  // load, the ring DMA included.) Rows past the unit's M rows take a copy of
  // its last row: their results are never stored. Query rows sit row-major in
  // LDS with their 16-byte chunks XOR-swizzled by row, so the 16 rows one read
  // instruction touches hit distinct banks.
  const bool computes = wave < NWC * KS;
  const int rw = wave % NWC;   // row group
  const int kh = wave / NWC;   // key slice of every tile (KS = 2)
  const bool owner = computes && kh == 0;  // finishes the rows after the loop
  const int kw0 = kh * TKW;                // first key of this wave's slice of a tile
  constexpr bool QDMA = MWG * ROW_B <= STAGE_B;
  static_assert(QDMA || !ROPE, "fused RoPE stages its query rows by DMA");
  constexpr int NQI = MWG * ROW_B / 1024;  // DMA instructions for the query rows
  constexpr int QPW = (NQI + NW - 1) / NW;  // ... per wave (the last one repeated to even them out)
  SIMSD_LDS uint8_t* const ring_l = (SIMSD_LDS uint8_t*)ring;
  const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring_l));
  SIMSD_LDS uint8_t* const q_st = ring_l + (NS - 1) * STAGE_B;
  // fused RoPE: the table's (cos, sin) pairs, then the staged frequencies
  const int rope_npos = ROPE ? (a.rope_no_copy ? twoB : B) : 0;
  double* const rope_freq = rope_tab + static_cast<size_t>(rope_npos) * rope_row_doubles<D>();
  bf16x8 qreg[QB][KK];
  int r_q[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = min(slice * MWG + (rw * QB + qb) * 16 + n16, a.M - 1);
    r_q[qb] = a.row0 + m / a.G;
  }
  int tau_ld = 0;
  if constexpr (QDMA) {
    if (wave == 0) {
      if constexpr (ROPE) {
        // the D/2 fp64 frequencies: 16 bytes per lane, lanes past them repeat the last piece
        const char* kargs = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
        dma16(kargs + offsetof(AttnArgs, rope_inv_freq), 16u * static_cast<uint32_t>(min(lane, D / 4 - 1)),
              static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIMSD_LDS double*)rope_freq)));
      }
      if constexpr (!MASK) {
        const int* tau_row = a.tau + static_cast<size_t>(s) * B;
        dma4(tau_row, 4u * static_cast<uint32_t>(min(lane, B - 1)),
             static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIMSD_LDS int*)tau_s)));
      }
      if constexpr (ROPE) {
        if (a.rope_positions) {
          const int* pos_row = a.start_pos + static_cast<size_t>(s) * B;
          dma4(pos_row, 4u * static_cast<uint32_t>(min(lane, B - 1)),
               static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIMSD_LDS int*)pos_s)));
        }
      }
    }
    const uint16_t* q_seq = a.q_blk + static_cast<size_t>(s) * twoB * a.Hq * D;
    const uint32_t q_lds = ring_base + static_cast<uint32_t>((NS - 1) * STAGE_B);
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int gi = min(i * NW + wave, NQI - 1);
      const int row = gi * RPI + lane / CH;  // query row of the workgroup
      const int p = lane % CH;               // LDS chunk slot this lane fills
      const int m = min(slice * MWG + row, a.M - 1);
      const int r = a.row0 + m / a.G;
      const int h = g * a.G + m % a.G;
      const uint32_t src = static_cast<uint32_t>((r * a.Hq + h) * D) * 2u +
                           16u * static_cast<uint32_t>(p ^ (row & (CH - 1)));
      dma16(q_seq, src, q_lds + static_cast<uint32_t>(gi * 1024));
    }
  }

  const int lim = min(a.max_prefix, max(cap, 0));
  const bool bad_prefix = P < 0 || P > lim;
  P = P < 0 ? 0 : (P > lim ? lim : P);
  const int ns = P > 0 ? (P + a.chunk - 1) / a.chunk : 1;
  if (split >= ns) {
    if constexpr (QDMA) wait_vmcnt<0>();  // no DMA may land in LDS after the workgroup ends
    return;
  }
  // split 0 also takes the block tiles, so its prefix run is `shift` keys
  // shorter and every later boundary moves down by as much; the last split
  // runs to the end of the prefix
  const int key_lo = split == 0 ? 0 : split * a.chunk - a.shift;
  const int key_hi = split == ns - 1 ? P : (split + 1) * a.chunk - a.shift;

  // ---- tile schedule: (split 0) the block tiles, then the prefix tiles of this chunk ----
  // prefix rows of (s, g): token-major [sum P][Hkv][d] or head-major [Hkv][sum P][d];
  // with the paired layout every (token, head) slot holds the key row then
  // the value row ([..][2][d]), so rows are kv_pair times as far apart
  const uint32_t rsb = static_cast<uint32_t>(a.kv_pair) *
                       (a.kv_head_major ? ROW_B : static_cast<uint32_t>(a.Hkv) * ROW_B);  // bytes between rows
  const size_t pre0 = static_cast<size_t>(a.kv_pair) *
                      (a.kv_head_major ? (static_cast<size_t>(g) * rows_total + o0) * D
                                       : (static_cast<size_t>(o0) * a.Hkv + g) * D);
  const char* kpre = reinterpret_cast<const char*>(a.k_pre + pre0);
  const char* vpre = reinterpret_cast<const char*>(a.v_pre + pre0);
  const uint32_t rsb_blk = static_cast<uint32_t>(a.Hkv) * ROW_B;  // block rows are [2B][Hkv][d]
  const char* kblk = reinterpret_cast<const char*>(a.k_blk + (static_cast<size_t>(s) * twoB * a.Hkv + g) * D);
  const char* vblk = reinterpret_cast<const char*>(a.v_blk + (static_cast<size_t>(s) * twoB * a.Hkv + g) * D);
  // split 0 takes the block tiles first: their rows live apart from the
  // prefix strip, so their first-touch latency overlaps the prefix DMA
  const int n_blk = split == 0 ? (twoB + TK - 1) / TK : 0;
  const int n_pre = (key_hi - key_lo + TK - 1) / TK;
  const int ntiles = n_blk + n_pre;
  // Prefix tiles are visited from a per-unit starting tile (wrapping around),
  // so that the many workgroups whose strips start at equally aligned
  // addresses do not walk the same HBM channels in lockstep.
  const int rot = (a.rotate && n_pre > 1) ? static_cast<int>((static_cast<unsigned>(us) * 2654435761u) >> 8) % n_pre : 0;
  auto pre_tile = [&](int t) {  // prefix tile index of schedule slot t >= n_blk
    const int j = t - n_blk + rot;
    return j >= n_pre ? j - n_pre : j;
  };
  // Per-lane byte offsets of the DMA of a full prefix tile: instruction i of
  // this wave fills LDS rows gi*RPI .. gi*RPI+RPI-1 (gi = NW i + wave); lane l
  // supplies the chunk that the swizzle places in LDS slot l % CH of its row.
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (i * NW + wave) * RPI + lane / CH;
    const int p = lane % CH;
    koff[i] = static_cast<uint32_t>(row) * rsb + 16u * static_cast<uint32_t>(p ^ swz_k<D>(row));
    voff[i] = static_cast<uint32_t>(row) * rsb + 16u * static_cast<uint32_t>(p ^ swz_v<D>(row));
  }

  // Issue the DMA of tile t into ring slot t % NS. In a partial tile, rows past
  // the valid end re-read the last valid row (in bounds; those keys are masked).
  auto issue = [&](int t) {
    const bool blk = t < n_blk;
    const int r0 = blk ? t * TK : key_lo + pre_tile(t) * TK;
    const int nvalid = blk ? min(TK, twoB - r0) : min(TK, key_hi - r0);
    const uint32_t stride = blk ? rsb_blk : rsb;
    const char* kb = (blk ? kblk : kpre) + static_cast<size_t>(r0) * stride;
    const char* vb = (blk ? vblk : vpre) + static_cast<size_t>(r0) * stride;
    const uint32_t stage = ring_base + static_cast<uint32_t>((t % NS) * STAGE_B);
    if (nvalid == TK && !blk) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const uint32_t lds = stage + static_cast<uint32_t>((i * NW + wave) * 1024);
        dma16_nt(kb, koff[i], lds);
        dma16_nt(vb, voff[i], lds + TENSOR_B);
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int row = (i * NW + wave) * RPI + lane / CH;
        const int p = lane % CH;
        const uint32_t src = static_cast<uint32_t>(min(row, nvalid - 1)) * stride;
        const uint32_t lds = stage + static_cast<uint32_t>((i * NW + wave) * 1024);
        dma16_nt(kb, src + 16u * static_cast<uint32_t>(p ^ swz_k<D>(row)), lds);
        dma16_nt(vb, src + 16u * static_cast<uint32_t>(p ^ swz_v<D>(row)), lds + TENSOR_B);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) issue(t);

  if constexpr (!QDMA) {
    // Plain loads, requested right behind the first tiles (the compiler's
    // wait for them also waits for those tiles).
    tau_ld = (!MASK && tid < B) ? a.tau[static_cast<size_t>(s) * B + tid] : 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int m = min(slice * MWG + (rw * QB + qb) * 16 + n16, a.M - 1);
      const int h = g * a.G + m % a.G;
      const uint16_t* qrow = a.q_blk + ((static_cast<size_t>(s) * twoB + r_q[qb]) * a.Hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qreg[qb][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * a16));
    }
  }

  // explicit mask: this lane's rows' mask words (<= 128 block keys), requested
  // with the queries (split 0 only: it takes the block tiles)
  // (two arrays, not one of pairs: a pair selected by a runtime condition
  // would be folded into an indexed access, which moves it to scratch)
  uint64_t mlo[QB], mhi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mlo[qb] = mhi[qb] = 0;
    if (MASK && split == 0) {
      const uint64_t* mrow = a.block_mask + (static_cast<size_t>(s) * twoB + r_q[qb]) * a.mask_words;
      mlo[qb] = mrow[0];
      if (a.mask_words > 1) mhi[qb] = mrow[1];
    }
  }

  if constexpr (QDMA) {
    // tau and the query rows have landed; the first tiles may stay in flight
    wait_tile<DPW, NS - 1>(min(NS - 1, ntiles));
  } else {
    if (tid < 64) tau_s[tid] = tau_ld;
  }
  if (tid == 0) vbad_s = 0;
  wait_lgkm0();
  block_barrier();  // tau_s, the query rows (and the RoPE frequencies) visible
  if constexpr (QDMA) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = (rw * QB + qb) * 16 + n16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        union {
          u32x4 u;
          bf16x8 b;
        } qv;
        qv.u = *reinterpret_cast<SIMSD_LDS const u32x4*>(q_st + row * ROW_B + 16 * ((4 * kk + a16) ^ (row & (CH - 1))));
        qreg[qb][kk] = qv.b;
      }
    }
    // complete before the first pipeline step refills this slot
    wait_lgkm0();
  }
  if constexpr (ROPE) {
    // cos/sin of every (block position, frequency) this workgroup needs,
    // computed while the first tiles are in flight. Row p of the table is
    // position start + p (or pair p's own position): the B data positions,
    // then (without the copy rule) the B positions after them that the mask
    // slots take instead. Entry e of
    // the table has frequency e % (D/2) = lane % (D/2), read from the staged
    // frequencies.
    const double inv_l = rope_freq[lane % (D / 2)];
    static_assert((NW * 64) % (D / 2) == 0, "table entries keep the lane's frequency");
    for (int e = tid; e < rope_npos * (D / 2); e += NW * 64) {
      const int pi = e / (D / 2);
      const long pos = a.rope_positions ? static_cast<long>(pos_s[pi]) : pos0 + pi;
      const double ang = static_cast<double>(pos) * inv_l;
      double sn, cs;
      sincos(ang, &sn, &cs);
      const int f = e - pi * (D / 2);  // frequency index
      rope_tab[pi * rope_row_doubles<D>() + 2 * f] = cs;
      rope_tab[pi * rope_row_doubles<D>() + 2 * f + 1] = sn;
    }
    wait_lgkm0();
    block_barrier();  // the table visible
  }
  if (a.status && split == 0 && slice == 0 && g == 0 && wave == 0) {
    // tau is a permutation of 1..B iff every label is in range and the OR of
    // the label bits over the B lanes has all B bits set (a duplicate leaves
    // one unset); one LDS read and a wave OR, no loop over the labels
    const int t = lane < B ? tau_s[lane] : 1;
    const bool in_range = t >= 1 && t <= B;
    uint64_t bit = (lane < B && in_range) ? (1ull << (t - 1)) : 0ull;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bit |= __shfl_xor(bit, off, kWave);
    const uint64_t full = B >= 64 ? ~0ull : ((1ull << B) - 1ull);
    const bool bad_tau = (__ballot(!in_range) != 0ull) || bit != full;
    if (lane == 0 && (bad_tau || bad_prefix))
      atomicOr(&a.status[s], (bad_tau ? kDevBadTau : 0) | (bad_prefix ? kDevBadPrefix : 0));
  }

  int tau_q[QB];
  bool slot_q[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = r_q[qb];
    slot_q[qb] = r >= B;
    tau_q[qb] = MASK ? 0 : tau_s[r >= B ? r - B : r];
    if constexpr (ROPE) rope_rows<D, KK>(qreg[qb], rope_pos_row(r, B, a.rope_no_copy), a16, a.rope_interleaved, rope_tab);
  }
  // Temporal mask of this lane's keys in the block tiles, evaluated once here
  // (while the first tiles are in flight): bit (bt * NKB * 4 + kb * 4 + i) is
  // key kw0 + 32(kb/2) + 8 a16 + 4(kb%2) + i of block tile bt, set if allowed.
  static_assert(((128 + TK - 1) / TK) * NKB * 4 <= 64, "block mask bits");
  // Per block tile, the labels of this lane's keys are read from LDS together
  // (clamped indices, no branch around the reads, so one wait covers them),
  // then every query block takes its bits from them.
  uint64_t blk_bits[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) blk_bits[qb] = 0;
  if (split == 0 && computes) {
    const int nbt = (twoB + TK - 1) / TK;
    for (int bt = 0; bt < nbt; ++bt) {
      int tau_k[NKB][4];
      if constexpr (!MASK) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = min(bt * TK + kw0 + 32 * (kb >> 1) + 8 * a16 + 4 * (kb & 1) + i, twoB - 1);
            tau_k[kb][i] = tau_s[c >= B ? c - B : c];
          }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // this tile's bits at fixed positions, then one shift into place (a
        // per-key variable 64-bit shift compiled into a chain of branches)
        uint32_t w = 0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = bt * TK + kw0 + 32 * (kb >> 1) + 8 * a16 + 4 * (kb & 1) + i;
            bool ok;
            if constexpr (MASK)
              ok = c < twoB && (((c >= 64 ? mhi[qb] : mlo[qb]) >> (c & 63)) & 1ull) != 0;
            else
              ok = c < twoB && block_allowed(slot_q[qb], tau_q[qb], c >= B, tau_k[kb][i], a.data_rule);
            w |= ok ? (1u << (kb * 4 + i)) : 0u;
          }
        blk_bits[qb] |= static_cast<uint64_t>(w) << ((bt * NKB * 4) & 63);
      }
    }
  }

  // Make the compiler complete the Q loads here, not at their first use inside
  // the tile loop (a wait there would also drain the DMA ring every tile).
  if constexpr (!QDMA) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qreg[qb][kk]));
  }

  const float c2 = a.scale_log2;  // softmax scale * log2(e)
  f32x4 oacc[QB][DB];
  float m_run[QB], l_run[QB];  // running max of raw scores, lane-partial sums
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile's work for a computing wave: S^T, mask, online softmax, P.V.
  auto compute_tile = [&](int t) {
    const bool blk = t < n_blk;
    const int r0 = blk ? t * TK : key_lo + pre_tile(t) * TK;
    const int nvalid = blk ? min(TK, twoB - r0) : min(TK, key_hi - r0);
    SIMSD_LDS uint8_t* const kst_p = ring_l + (t % NS) * STAGE_B;
    SIMSD_LDS uint8_t* const vst_p = kst_p + TENSOR_B;

    // S^T blocks: block kb covers keys 32(kb/2) + 8(m/4) + 4(kb%2) + m%4 for MFMA row m
    // (relative to this wave's key slice kw0), so lane (a16, n16) ends up with keys
    // kw0 + 32ks + 8*a16 + 0..7 of query n16.
    f32x4 sacc[QB][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = kw0 + 32 * (kb >> 1) + 8 * (n16 >> 2) + 4 * (kb & 1) + (n16 & 3);
      const int sw = swz_k<D>(row);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        union {
          u32x4 u;
          bf16x8 b;
        } ak;
        ak.u = *reinterpret_cast<SIMSD_LDS const u32x4*>(kst_p + row * ROW_B + 16 * ((4 * kk + a16) ^ sw));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak.b, qreg[qb][kk], sacc[qb][kb], 0, 0, 0);
      }
    }

    const bool need_mask = blk || nvalid < TK;
    bf16x8 pop[QB][NSUB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (need_mask) {
        // Branch-free inside: this tile's block bits in one word (block
        // tiles) or the valid-key bound (a partial prefix tile), then a
        // select per key. Its inputs pass through an empty volatile asm so
        // that none of this work is hoisted above the branch onto every
        // full tile (hoisted compares cost b16 about 4 us).
        uint32_t bw = static_cast<uint32_t>(blk_bits[qb] >> ((t * NKB * 4) & 63));
        int lim = nvalid - (kw0 + 8 * a16);  // this lane's keys at offsets below lim are valid
        int isblk = blk ? 1 : 0;
        asm volatile("" : "+v"(bw), "+v"(lim), "+v"(isblk));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int off = 32 * (kb >> 1) + 4 * (kb & 1) + i;
            const bool ok = isblk ? ((bw >> (kb * 4 + i)) & 1u) != 0u : off < lim;
            sacc[qb][kb][i] = ok ? sacc[qb][kb][i] : -INFINITY;
          }
      }
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[qb][kb][i]);
      mx = max_over_row_lanes(mx);
      const float m_new = fmaxf(m_run[qb], mx);
      const bool grew = m_new > m_run[qb];
      if (__ballot(grew) != 0ull) {  // rescale only when some row max moved
        const float alpha = grew ? __builtin_amdgcn_exp2f((m_run[qb] - m_new) * c2) : 1.0f;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
        m_run[qb] = m_new;
      }
      const float nmc = m_new == -INFINITY ? 0.0f : -m_new * c2;
      float psum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NSUB; ++ks) {
        uint32_t pk[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const f32x4 sv = sacc[qb][2 * ks + kb2];
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[0], c2, nmc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[1], c2, nmc));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2], c2, nmc));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[3], c2, nmc));
          psum += (p0 + p1) + (p2 + p3);
          pk[2 * kb2] = pack_bf16x2(p0, p1);
          pk[2 * kb2 + 1] = pack_bf16x2(p2, p3);
        }
        pop[qb][ks] = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
      l_run[qb] += psum;
    }

    // O^T += V^T P^T; the V^T operand (8 consecutive keys of one d column) comes
    // from two transposing LDS reads of the row-major, swizzled V tile.
#pragma unroll
    for (int ks = 0; ks < NSUB; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i16x4 part[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = kw0 + 32 * ks + 8 * a16 + 4 * hh + (n16 >> 2);
          const int c = 2 * db + ((n16 & 3) >> 1);
          part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<SIMSD_LDS i16x4*>(
              vst_p + row * ROW_B + 16 * (c ^ swz_v<D>(row)) + 8 * (n16 & 1)));
        }
        union {
          i16x4 h[2];
          bf16x8 b;
        } av;
        av.h[0] = part[0];
        av.h[1] = part[1];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.b, pop[qb][ks], oacc[qb][db], 0, 0, 0);
      }
  };

  // Pipeline step of tile t: wait until it has landed (tiles t+1 .. t+NS-2
  // may still be in flight), one barrier (every wave's share of tile t is in
  // LDS and tile t-1 is consumed), then refill the slot tile t-1 used.
  auto advance = [&](int t) {
    wait_tile<DPW, NS - 2>(min(NS - 2, ntiles - 1 - t));
    if (t < n_blk) {
      // A block tile: every lane zeroes the non-finite values of the 16-byte
      // V pieces it brought in itself (landed with this wave's wait), before
      // the barrier publishes the tile. A hidden key's zero weight then never
      // meets a NaN or Inf in the product (0 * NaN would be NaN); the terms of
      // visible keys are added back after the loop.
      const uint32_t vstage = static_cast<uint32_t>((t % NS) * STAGE_B + TENSOR_B);
      bool found = false;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        SIMSD_LDS u32x4* pc =
            reinterpret_cast<SIMSD_LDS u32x4*>(ring_l + vstage + (i * NW + wave) * 1024 + 16 * lane);
        const u32x4 x = *pc;
        u32x4 y;
        bool bad = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = x[w] & 0xffffu, hi = x[w] >> 16;
          const bool bl = (lo & 0x7f80u) == 0x7f80u, bh = (hi & 0x7f80u) == 0x7f80u;
          y[w] = (bl ? 0u : lo) | (bh ? 0u : (hi << 16));
          bad = bad || bl || bh;
        }
        if (bad) *pc = y;
        found = found || bad;
      }
      if (found) vbad_s = 1;
      wait_lgkm0();
    }
    block_barrier();
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
  };

  // Fused RoPE-copy: rotate the block key rows of a landed block tile in
  // place in LDS, once per workgroup (every thread takes (row, pair-of-chunks)
  // items), and write the rotated rows out for the cache if asked.
  auto rotate_block_tile = [&](int t) {
    const int r0 = t * TK;
    SIMSD_LDS uint8_t* const kst_p = ring_l + (t % NS) * STAGE_B;
    const bool write = a.k_rot != nullptr && split == 0 && slice == 0;
    constexpr int HALF_CH = CH / 2;
    // items of 8 bytes (half a 16-byte chunk: 4 pairs of the split halves, 2
    // of the interleaved form), over the tile's valid rows only, so that
    // every thread of a b8 workgroup takes one (with 16-byte items over all
    // rows, half of them had nothing to do and the others eight rotations)
    const int per_row = 2 * (a.rope_interleaved ? CH : HALF_CH);
    const int nrow = min(TK, twoB - r0);
    for (int it = tid; it < nrow * per_row; it += NW * 64) {
      const int row = it / per_row, cc = (it % per_row) >> 1, hf = it & 1;
      const int c = r0 + row;
      const int sw = swz_k<D>(row);
      const double* tr = rope_tab + static_cast<size_t>(rope_pos_row(c, B, a.rope_no_copy)) * rope_row_doubles<D>();
      union U {
        u32x2 u;
        uint16_t h[4];
      };
      SIMSD_LDS u32x2* pa = reinterpret_cast<SIMSD_LDS u32x2*>(kst_p + row * ROW_B + 16 * (cc ^ sw) + 8 * hf);
      uint16_t* const dst = write ? a.k_rot + ((static_cast<size_t>(s) * twoB + c) * a.Hkv + g) * D : nullptr;
      U x;
      x.u = *pa;
      if (a.rope_interleaved) {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const int i = (8 * cc + 4 * hf + j) / 2;
          rope_rotate(x.h[j], x.h[j + 1], tr[2 * i], tr[2 * i + 1], &x.h[j], &x.h[j + 1]);
        }
        *pa = x.u;
      } else {
        SIMSD_LDS u32x2* pb =
            reinterpret_cast<SIMSD_LDS u32x2*>(kst_p + row * ROW_B + 16 * ((cc + HALF_CH) ^ sw) + 8 * hf);
        U y;
        y.u = *pb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * cc + 4 * hf + j;
          rope_rotate(x.h[j], y.h[j], tr[2 * i], tr[2 * i + 1], &x.h[j], &y.h[j]);
        }
        *pa = x.u;
        *pb = y.u;
        if (write) *reinterpret_cast<u32x2*>(dst + 8 * (cc + HALF_CH) + 4 * hf) = y.u;
      }
      if (write) *reinterpret_cast<u32x2*>(dst + 8 * cc + 4 * hf) = x.u;
    }
    wait_lgkm0();
    block_barrier();  // rotated rows visible to every wave
  };

  for (int t = 0; t < ntiles; ++t) {
    advance(t);
    if constexpr (ROPE) {
      if (t < n_blk) rotate_block_tile(t);
    }
    if (computes) compute_tile(t);
  }

  if constexpr (KS == 2) {
    // Fold the second key slice into the first: the slice-1 waves leave
    // (m, lane-partial l, O) in LDS (the ring is free once every wave has
    // left the loop), the slice-0 waves merge them with the log-sum-exp rule.
    wait_lgkm0();
    block_barrier();
    float* xo = reinterpret_cast<float*>(ring);
    if (computes && kh == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int slot = (rw * QB + qb) * 64 + lane;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4*>(xo + ((rw * QB + qb) * DB + db) * 256 + 4 * lane) = oacc[qb][db];
        xml[2 * slot] = m_run[qb];
        xml[2 * slot + 1] = l_run[qb];
      }
    }
    wait_lgkm0();
    block_barrier();
    if (owner) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int slot = (rw * QB + qb) * 64 + lane;
        const float m1 = xml[2 * slot], l1 = xml[2 * slot + 1];
        const float m_new = fmaxf(m_run[qb], m1);
        const float base = m_new == -INFINITY ? 0.0f : m_new;
        const float wa = __builtin_amdgcn_exp2f((m_run[qb] - base) * c2);
        const float wb = __builtin_amdgcn_exp2f((m1 - base) * c2);
        l_run[qb] = l_run[qb] * wa + l1 * wb;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[qb][db] = oacc[qb][db] * wa +
                         *reinterpret_cast<const f32x4*>(xo + ((rw * QB + qb) * DB + db) * 256 + 4 * lane) * wb;
        m_run[qb] = m_new;
      }
    }
  }

  // ---- split 0: the non-finite block values its rows see ----
  // Rare (only when a block V row held a NaN or Inf; uniform): for every
  // block key its query sees, each owner lane folds the non-finite values at
  // its d columns into the IEEE sum they form (NaN, +Inf or -Inf) and adds it
  // to its unnormalised output, as the plain softmax over the allowed keys
  // would (every allowed key has a positive weight there).
  if (split == 0 && owner && __builtin_amdgcn_readfirstlane(vbad_s)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      uint32_t pos_inf[DB], neg_inf[DB], nan_bits[DB];  // bit i: column 16 db + 4 a16 + i
#pragma unroll
      for (int db = 0; db < DB; ++db) pos_inf[db] = neg_inf[db] = nan_bits[db] = 0u;
#pragma unroll 1
      for (int c = 0; c < twoB; ++c) {
        bool ok;
        if constexpr (MASK)
          ok = (((c >= 64 ? mhi[qb] : mlo[qb]) >> (c & 63)) & 1ull) != 0;
        else
          ok = block_allowed(slot_q[qb], tau_q[qb], c >= B, tau_s[c >= B ? c - B : c], a.data_rule);
        if (!ok) continue;
        const char* vr = vblk + static_cast<size_t>(c) * rsb_blk + 8 * a16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint2 v4 = *reinterpret_cast<const uint2*>(vr + 32 * db);
          const uint32_t e[4] = {v4.x & 0xffffu, v4.x >> 16, v4.y & 0xffffu, v4.y >> 16};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool inf = (e[i] & 0x7fffu) == 0x7f80u, nan = (e[i] & 0x7fffu) > 0x7f80u;
            pos_inf[db] |= (inf && !(e[i] & 0x8000u)) ? (1u << i) : 0u;
            neg_inf[db] |= (inf && (e[i] & 0x8000u)) ? (1u << i) : 0u;
            nan_bits[db] |= nan ? (1u << i) : 0u;
          }
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool pi = (pos_inf[db] >> i) & 1u, ni = (neg_inf[db] >> i) & 1u, na = (nan_bits[db] >> i) & 1u;
          if (na || (pi && ni)) oacc[qb][db][i] = __builtin_nanf("");
          else if (pi) oacc[qb][db][i] += INFINITY;
          else if (ni) oacc[qb][db][i] -= INFINITY;
        }
    }
  }

  // ---- finish: full row sums, then either write or hand off to the merge ----
  float l_tot[QB], m_sc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_tot[qb] = sum_over_row_lanes(l_run[qb]);
    m_sc[qb] = m_run[qb] * c2;  // log2 units
  }

  if (ns > 1) {
    // Hand the split's partial (m, l, unnormalised O) to the last workgroup of
    // the unit. Partials are written and read with device-coherent (agent
    // scope) accesses, so no cache-wide writeback/invalidate is needed; the
    // barrier waits for this workgroup's stores to be acknowledged before the
    // counter is bumped, and the last workgroup reads only after its bump
    // returned.
    // With a bf16 output the unnormalised O partials travel as bf16 (one more
    // rounding of relative size 2^-9, below the output's own), halving the
    // hand-off and merge bytes; with an fp32 output they stay fp32.
    constexpr bool PBF = !OUT_F32;
    constexpr int EB = PBF ? 8 : 16;                    // bytes per lane and (row block, d block)
    constexpr int PART_O_B = NWC * QB * DB * 64 * EB;   // bytes of one split's O partial
    constexpr int PART_ML_B = MWG * 8;                  // bytes of one split's (m, l) pairs
    const size_t part = static_cast<size_t>(us) * a.nsplit + split;
    if (owner) {
      const auto ro = coherent_rsrc(reinterpret_cast<char*>(a.part_o) + part * PART_O_B, PART_O_B);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (((rw * QB + qb) * DB + db) * 64 + lane) * EB;
          if constexpr (PBF)
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{pack_bf16x2(oacc[qb][db][0], oacc[qb][db][1]), pack_bf16x2(oacc[qb][db][2], oacc[qb][db][3])},
                ro, off, 0, kCoherent);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oacc[qb][db]), ro, off, 0, kCoherent);
        }
      if (a16 == 0) {
        const auto rml = coherent_rsrc(reinterpret_cast<char*>(a.part_ml) + part * PART_ML_B, PART_ML_B);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(u32x2, f32x2{m_sc[qb], l_tot[qb]}), rml, ((rw * QB + qb) * 16 + n16) * 8, 0,
              kCoherent);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    __syncthreads();
    if (tid == 0) {
      const int prev = __hip_atomic_fetch_add(&a.counters[us], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_s = prev == ns - 1;
    }
    __syncthreads();
    if (!last_s) return;
    if (owner) {
      // Online log-sum-exp merge of the ns partials in split order (fixed, so
      // the result does not depend on which workgroup came last). The loads of
      // MB partials are issued together: one memory round trip per MB splits.
      constexpr int MB = (QB == 1 || PBF) ? 4 : 2;
      const size_t part0 = static_cast<size_t>(us) * a.nsplit;
      const auto ro = coherent_rsrc(reinterpret_cast<char*>(a.part_o) + part0 * PART_O_B, ns * PART_O_B);
      const auto rml = coherent_rsrc(reinterpret_cast<char*>(a.part_ml) + part0 * PART_ML_B, ns * PART_ML_B);
      float m_acc[QB], l_acc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        m_acc[qb] = -INFINITY;
        l_acc[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int k0 = 0; k0 < ns; k0 += MB) {
        f32x2 ml[MB][QB];
        f32x4 po[MB][QB][DB];
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          const int k = min(k0 + j, ns - 1);  // past the end: re-read the last one (ignored)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int row = (rw * QB + qb) * 16 + n16;
            ml[j][qb] = __builtin_bit_cast(
                f32x2, __builtin_amdgcn_raw_buffer_load_b64(rml, k * PART_ML_B + row * 8, 0, kCoherent));
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int off = k * PART_O_B + (((rw * QB + qb) * DB + db) * 64 + lane) * EB;
              if constexpr (PBF) {
                const u32x2 h = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(ro, off, 0, kCoherent));
                po[j][qb][db] = f32x4{__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xffff0000u),
                                      __uint_as_float(h[1] << 16), __uint_as_float(h[1] & 0xffff0000u)};
              } else {
                po[j][qb][db] =
                    __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, kCoherent));
              }
            }
          }
        }
#pragma unroll
        for (int j = 0; j < MB; ++j) {
          if (k0 + j >= ns) break;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float mk = ml[j][qb][0];
            const float m_new = fmaxf(m_acc[qb], mk);
            const float base = m_new == -INFINITY ? 0.0f : m_new;  // all empty so far: weights 0
            const float wa = __builtin_amdgcn_exp2f(m_acc[qb] - base);
            const float wb = __builtin_amdgcn_exp2f(mk - base);
            l_acc[qb] = l_acc[qb] * wa + ml[j][qb][1] * wb;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[qb][db] = oacc[qb][db] * wa + po[j][qb][db] * wb;
            m_acc[qb] = m_new;
          }
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        m_sc[qb] = m_acc[qb];
        l_tot[qb] = l_acc[qb];
      }
    }
    if (tid == 0) __hip_atomic_store(&a.counters[us], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!owner) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = slice * MWG + (rw * QB + qb) * 16 + n16;
    if (m >= a.M) continue;
    const int r = a.row0 + m / a.G;
    const int h = g * a.G + m % a.G;
    const size_t orow = (static_cast<size_t>(s) * twoB + r) * a.Hq + h;
    // a row that sees no key at all (explicit mask, empty prefix) gives 0;
    // under tau every row sees at least itself or its data partner
    const float inv_l = (!MASK || l_tot[qb] > 0.0f) ? 1.0f / l_tot[qb] : 0.0f;
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
    if (a.lse && a16 == 0) a.lse[orow] = (m_sc[qb] + __log2f(l_tot[qb])) * kLn2;
  }
}

// Dynamic LDS of the fused RoPE path: the (cos, sin) fp64 table per
// (position, frequency) and the staged frequencies.
inline size_t rope_table_bytes(const AttnArgs& a) {
  if (!a.rope) return 0;
  const int npos = a.rope_no_copy ? 2 * a.B : a.B;
  // the table (padded rows), then 1 KB where one wave's DMA stages the frequencies
  const int row = a.d == 64 ? rope_row_doubles<64>() : rope_row_doubles<128>();
  return static_cast<size_t>(npos) * row * sizeof(double) + 1024;
}

template <int D, int NWC, int QB, int TK, int NS, int NW = 4, int KS = 1, int MODE = kModeTau>
hipError_t launch_variant(const AttnArgs& a0, hipStream_t stream) {
  AttnArgs a = a0;
  if (a.shift < 0) {
    // Split 0 also streams the block tiles, so by default it gives up one
    // tile's worth of prefix keys per block tile of this variant (capped at
    // half a chunk), which evens out the splits' finish times (one MI355X,
    // interleaved runs: b8 54.9 -> 54.3 us, b16 108.4 -> 107.2 us, b = 1
    // prefix 1024 17.0 -> 16.2 us; larger shifts measured slower on b8).
    const int blk_tiles = (a.nblk + TK - 1) / TK;
    a.shift = a.nsplit > 1 ? std::min(a.chunk / 2, blk_tiles * TK) : 0;
  }
  dim3 grid(static_cast<unsigned>(a.total_grid)), block(NW * 64);
  const size_t dyn = MODE == kModeTauRope ? rope_table_bytes(a) : 0;
  if (a.out_f32)
    hipLaunchKernelGGL((verify_attn_kernel<D, NW, NWC, QB, TK, NS, KS, MODE, true>), grid, block, dyn, stream, a);
  else
    hipLaunchKernelGGL((verify_attn_kernel<D, NW, NWC, QB, TK, NS, KS, MODE, false>), grid, block, dyn, stream,
                       a);
  return hipGetLastError();
}

// The fused-RoPE and explicit-mask paths instantiate only the variants the
// plan picks by default (the same ones as the tau path, so the three agree bit
// for bit where their rules coincide).
// LDS a workgroup may use on gfx950 (static and dynamic together).
constexpr size_t kLdsPerWorkgroup = 160 * 1024;

// Whether an instance's static LDS plus `dyn` bytes of dynamic LDS fit a workgroup.
template <int D, int NWC, int QB, int TK, int NS, int NW, int KS, int MODE>
bool lds_fits(size_t dyn) {
  static size_t static_bytes = [] {
    hipFuncAttributes attr{};
    const void* f = reinterpret_cast<const void*>(&verify_attn_kernel<D, NW, NWC, QB, TK, NS, KS, MODE, false>);
    return hipFuncGetAttributes(&attr, f) == hipSuccess ? attr.sharedSizeBytes : kLdsPerWorkgroup;
  }();
  return static_bytes + dyn <= kLdsPerWorkgroup;
}

template <int D, int MODE>
hipError_t launch_d_default(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if (p.nwc == 1) return launch_variant<D, 1, 1, 64, 2, 4, 1, MODE>(a, stream);
  if (p.nwc == 2) return launch_variant<D, 2, 1, 64, 2, 4, 1, MODE>(a, stream);
  if (p.qb == 2) {
    if constexpr (D == 128) {
      // the 128-key ring leaves ~28 KB: a larger fused RoPE table (more than
      // 26 positions, with the staged frequencies) takes the 64-key form of
      // the same two-wave layout
      const size_t dyn = MODE == kModeTauRope ? rope_table_bytes(a) : 0;
      if (p.pipe == 9 && lds_fits<D, 4, 2, 128, 2, 8, 2, MODE>(dyn))
        return launch_variant<D, 4, 2, 128, 2, 8, 2, MODE>(a, stream);
      if (p.pipe == 7 || p.pipe == 9) return launch_variant<D, 4, 2, 64, 2, 8, 2, MODE>(a, stream);
    }
    return launch_variant<D, 4, 2, 64, 2, 4, 1, MODE>(a, stream);
  }
  if constexpr (D == 128) {
    if (p.pipe == 6) {
      // the longest-first ring of large ragged batches, if the RoPE table fits beside it
      const size_t dyn = MODE == kModeTauRope ? rope_table_bytes(a) : 0;
      if (lds_fits<D, 4, 1, 64, 4, 4, 1, MODE>(dyn)) return launch_variant<D, 4, 1, 64, 4, 4, 1, MODE>(a, stream);
      return launch_variant<D, 4, 1, 64, 2, 4, 1, MODE>(a, stream);
    }
    if (p.pipe == 2) {
      // the 64 x 3 ring if the RoPE table fits beside it, else 64 x 2: the
      // depth of the ring changes no arithmetic, so both agree bit for bit
      // with a two-launch sequence on the 64 x 3 ring
      const size_t dyn = MODE == kModeTauRope ? rope_table_bytes(a) : 0;
      if (lds_fits<D, 4, 1, 64, 3, 4, 1, MODE>(dyn)) return launch_variant<D, 4, 1, 64, 3, 4, 1, MODE>(a, stream);
      return launch_variant<D, 4, 1, 64, 2, 4, 1, MODE>(a, stream);
    }
    if (p.pipe != 1) return launch_variant<D, 4, 1, 32, 4, 4, 1, MODE>(a, stream);
  }
  return launch_variant<D, 4, 1, 64, 2, 4, 1, MODE>(a, stream);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if (p.nwc == 1) return launch_variant<D, 1, 1, 64, 2>(a, stream);
  if (p.nwc == 2) return launch_variant<D, 2, 1, 64, 2>(a, stream);
  if (p.qb == 2 || p.nwc == 8) {
    // 128 rows: 4 waves x 2 row blocks, or 8 waves x 1
    if constexpr (D == 128) {
      switch (p.pipe) {
        case 1: return launch_variant<D, 4, 2, 32, 4>(a, stream);
        case 2: return launch_variant<D, 4, 2, 64, 3>(a, stream);
        case 3: return launch_variant<D, 8, 1, 32, 4, 8>(a, stream);
        case 4: return launch_variant<D, 8, 1, 64, 2, 8>(a, stream);
        case 5: return launch_variant<D, 8, 1, 32, 6, 8>(a, stream);
        case 6: return launch_variant<D, 8, 1, 64, 3, 8>(a, stream);
        case 7: return launch_variant<D, 4, 2, 64, 2, 8, 2>(a, stream);
        case 8: return launch_variant<D, 4, 2, 64, 3, 8, 2>(a, stream);
        case 9: return launch_variant<D, 4, 2, 128, 2, 8, 2>(a, stream);
        default: return launch_variant<D, 4, 2, 64, 2>(a, stream);
      }
    }
    return launch_variant<D, 4, 2, 64, 2>(a, stream);
  }
  if constexpr (D == 128) {
    switch (p.pipe) {
      case 1: return launch_variant<D, 4, 1, 64, 2>(a, stream);
      case 2: return launch_variant<D, 4, 1, 64, 3>(a, stream);
      case 3: return launch_variant<D, 4, 1, 32, 3>(a, stream);
      case 4: return launch_variant<D, 4, 1, 32, 6>(a, stream);
      case 5: return launch_variant<D, 4, 1, 32, 8>(a, stream);
      case 6: return launch_variant<D, 4, 1, 64, 4>(a, stream);
      case 7: return launch_variant<D, 4, 1, 64, 2, 8, 2>(a, stream);
      case 8: return launch_variant<D, 4, 1, 64, 3, 8, 2>(a, stream);
      case 9: return launch_variant<D, 4, 1, 64, 4, 8, 2>(a, stream);
      default: return launch_variant<D, 4, 1, 32, 4>(a, stream);
    }
  }
  return launch_variant<D, 4, 1, 64, 2>(a, stream);
}

// A tuning override if one is set, else the plan's own value.
int tuned(int key, int dflt) {
  const int v = tuning(key);
  return v < 0 ? dflt : v;
}

}  // namespace

// Launch plan: rows per workgroup from M = G * rows, then the number of
// prefix splits. Measured on MI355X: a workgroup streams fastest when it owns
// one long contiguous run of keys, and every split adds a pipeline fill plus a
// partial hand-off (fp32 O of all its rows written and read back), so the plan
// splits only as far as needed to give each of the 256 CUs a workgroup:
// units >= 256 run unsplit (a ragged batch then has all its workgroups
// resident at once, two per CU), fewer units get ceil(256 / units) splits.
// Tuning overrides (simsd_set_tuning): SIMSD_TUNE_ATTN_TARGET_WG, _CHUNK_MAX, _PIPE, ...
AttnPlan plan_attention(int b, int B, int Hq, int Hkv, int d, int max_prefix, int data_rule) {
  return plan_attention_rows(b, data_rule == 2 ? B : 2 * B, Hq, Hkv, d, max_prefix);
}

AttnPlan plan_attention_rows(int b, int nrows, int Hq, int Hkv, int d, int max_prefix) {
  AttnPlan p{};
  const int G = Hq / Hkv;
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
  p.xcd_remap = tuned(SIMSD_TUNE_ATTN_XCD_REMAP, 1) != 0;  // tuning: keep a unit's splits on one XCD
  p.rotate = tuned(SIMSD_TUNE_ATTN_ROTATE, 1) != 0; // tuning: per-unit starting prefix tile
  p.row_slices = (M + p.rows_per_wg - 1) / p.rows_per_wg;
  const int target = std::max(1, tuned(SIMSD_TUNE_ATTN_TARGET_WG, 256));
  const int chunk_max = std::max(TK, tuned(SIMSD_TUNE_ATTN_CHUNK_MAX, 1 << 30) / TK * TK);
  const long units = static_cast<long>(b) * Hkv * p.row_slices;
  // A split shorter than a few tiles costs more in hand-off and merge than it
  // saves (b = 1, prefix 1024: 16 one-tile splits 19 us, 4 four-tile splits
  // 14 us), so every split gets at least kMinSplitTiles key tiles.
  constexpr int kMinSplitTiles = 4;
  const int max_tiles = std::max(1, (max_prefix + TK - 1) / TK);
  const int max_splits = std::max(1, max_tiles / kMinSplitTiles);
  int nsplit = static_cast<int>(std::min<long>(max_splits, std::max<long>(1, (target + units - 1) / units)));
  int chunk = ((max_prefix + nsplit - 1) / nsplit + TK - 1) / TK * TK;
  chunk = std::max(TK, std::min(chunk, chunk_max));
  nsplit = std::max(1, (max_prefix + chunk - 1) / chunk);
  // Key-tile ring (keys per tile x stages), for d = 128. 64 rows: 0 = 32x4,
  // 1 = 64x2, 2 = 64x3, 3 = 32x3, 4 = 32x6, 5 = 32x8, 6 = 64x4, 7-9 = 64x2,
  // 64x3, 64x4 with two waves per row group. 128 rows: 0 = 4 waves x 2 row
  // blocks 64x2, 1 = 4x2 32x4, 2 = 4x2 64x3, 3 = 8 waves x 1 32x4, 4 = 8x1
  // 64x2, 5 = 8x1 32x6, 6 = 8x1 64x3, 7 = 4x2 64x2 with two waves per row
  // group, 8 = the same 64x3, 9 = the same 128x2. With one 64-row workgroup
  // per CU the 64x3 ring keeps two 32 KB tiles in flight and takes half the
  // barriers of 32-key tiles (b8 with the non-temporal stream: 51.1 us
  // against 53.8 for 32x4 and 51.5 for 64x4); with two per CU the other
  // workgroup covers the latency and 64x2 suffices. A 128-row workgroup carries twice the MFMA and softmax work per
  // byte; alone on its CU it runs best with two waves per row group on every
  // SIMD, each taking half of every key tile, so one wave's MFMA work overlaps
  // the other's softmax, and with 128-key tiles, which halve the barriers per
  // byte (b16, interleaved runs: 110.5 us vs 114.1 with 64-key tiles and
  // 116-119 with one wave per row group).
  // An unsplit launch of more than 256 workgroups (a large ragged batch) is
  // ended by its longest sequences, each streamed by one workgroup. With 64
  // rows, d = 128 and at most 64 sequences it runs longest first (ids in
  // descending order of prefix length) on a 64 x 4 ring that keeps one
  // workgroup per CU with three tiles in flight: the long sequences start
  // first at the higher per-workgroup rate and the short ones fill the CUs
  // as they free up (ragged, 64 x U[512, 8192]: 222-224 us against 240.5 us
  // for all 512 workgroups resident two per CU on the 64 x 2 ring; without
  // the order the 64 x 4 ring takes 289 us).
  const long wgs = units * nsplit;
  const bool lpt_ok = nsplit == 1 && p.row_slices == 1 && b <= 64;
  const bool lpt_ring = p.qb == 1 && wgs > 256 && lpt_ok && d == 128;
  const int pipe_default = p.qb == 1 ? (wgs > 256 ? (lpt_ring ? 6 : 1) : 2) : (wgs <= 256 ? 9 : 0);
  p.pipe = tuned(SIMSD_TUNE_ATTN_PIPE, pipe_default);
  p.chunk = chunk;
  p.nsplit = nsplit;
  // tuning: SIMSD_TUNE_ATTN_LPT = 0 / 1 forces the longest-first order off / on
  p.lpt = (tuned(SIMSD_TUNE_ATTN_LPT, lpt_ring ? 1 : 0) != 0 && lpt_ok) ? 1 : 0;
  // prefix keys moved off split 0, which also takes the block tiles: -1
  // (default) lets the launch take one tile's worth per block tile of the
  // variant it runs; SIMSD_TUNE_ATTN_SHIFT >= 0 fixes it
  const int shift_set = tuned(SIMSD_TUNE_ATTN_SHIFT, -1);
  p.shift = shift_set < 0 ? -1 : std::min(chunk / 2, shift_set);
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
  if (a.rope)
    return a.d == 64 ? launch_d_default<64, kModeTauRope>(a, p, stream) : launch_d_default<128, kModeTauRope>(a, p, stream);
  if (a.mask_mode)
    return a.d == 64 ? launch_d_default<64, kModeMask>(a, p, stream) : launch_d_default<128, kModeMask>(a, p, stream);
  if (a.d == 64) return launch_d<64>(a, p, stream);
  return launch_d<128>(a, p, stream);
}

}  // namespace simsd
