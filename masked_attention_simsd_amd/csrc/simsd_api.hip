// simsd_api.hip -- the C ABI of libsimsd (declared in include/simsd.h).
//
// Host-side argument checks happen here, before anything is enqueued; the
// kernels live in rope_copy.hip, verify_attention.hip and accept.hip. No entry
// point allocates, frees or synchronises.
#include "simsd.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "simsd_internal.h"

namespace {

// Tuning overrides (simsd_set_tuning); -1 = the plan's own choice.
std::atomic<int> g_tuning[SIMSD_TUNE_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1};

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The paired K/V layout needs the value half to start d elements after the
// key half of the same buffer (no prefix pointers: nothing to check).
bool paired_ok(uint32_t flags, const void* k, const void* v, int d) {
  if (!(flags & SIMSD_KV_PAIRED) || !k || !v) return true;
  return reinterpret_cast<uintptr_t>(v) == reinterpret_cast<uintptr_t>(k) + static_cast<uintptr_t>(d) * 2u;
}

int launch_status(hipError_t e) {
  if (e == hipSuccess) return SIMSD_OK;
  g_last_hip_error = static_cast<int>(e);
  return SIMSD_ERR_LAUNCH;
}

// RoPE frequencies base^(-2i/d), i < d/2, in fp64 (the same expression the
// rotary embedding is defined by; computed once per call on the host).
void fill_inv_freq(double* out, float base, int d) {
  for (int i = 0; i < d / 2; ++i) out[i] = std::pow(static_cast<double>(base), -2.0 * i / d);
}

// RoPE flags: known bits only; explicit positions exclude the no-copy
// ablation (which numbers the mask slots after a consecutive data section).
bool rope_flags_ok(uint32_t f) {
  if (f & ~(SIMSD_ROPE_INTERLEAVED | SIMSD_ROPE_NO_COPY | SIMSD_ROPE_POSITIONS)) return false;
  return !((f & SIMSD_ROPE_NO_COPY) && (f & SIMSD_ROPE_POSITIONS));
}

int check_common(int b, int B, int Hq, int Hkv, int d) {
  if (b < 1 || B < 1 || B > 64 || Hq < 1 || Hkv < 1) return SIMSD_ERR_SIZE;
  if (Hq % Hkv != 0) return SIMSD_ERR_HEADS;
  if (d != 64 && d != 128) return SIMSD_ERR_HEAD_DIM;
  return SIMSD_OK;
}

// Shared by simsd_verify_attention and simsd_verify_attention_rope (rope
// points at the fused-RoPE arguments, or is NULL).
struct RopeIn {
  const int32_t* start_pos;
  float base;
  uint32_t flags;
  void* k_rot;
};

int verify_attention_impl(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pre,
                          const void* v_pre, const int32_t* prefix_offsets, const int32_t* tau,
                          void* out, float* lse, int b, int B, int Hq, int Hkv, int d, int max_prefix,
                          float scale, uint32_t flags, int32_t* status, void* workspace,
                          size_t ws_bytes, void* stream, const RopeIn* rope, bool check_only = false) {
  if (!q_blk || !k_blk || !v_blk || !prefix_offsets || !tau || !out) return SIMSD_ERR_NULL;
  if (max_prefix > 0 && (!k_pre || !v_pre)) return SIMSD_ERR_NULL;
  int rc = check_common(b, B, Hq, Hkv, d);
  if (rc) return rc;
  if (max_prefix < 0 || max_prefix > simsd::kMaxPrefix) return SIMSD_ERR_SIZE;
  const uint32_t rule = flags & 3u;
  if (rule == 3u || (flags & ~(3u | SIMSD_OUT_F32 | SIMSD_KV_HEAD_MAJOR | SIMSD_PREFIX_LENS | SIMSD_KV_PAIRED)))
    return SIMSD_ERR_FLAGS;
  if (!paired_ok(flags, k_pre, v_pre, d)) return SIMSD_ERR_FLAGS;
  if (!std::isfinite(scale)) return SIMSD_ERR_SCALE;
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out) ||
      (k_pre && !aligned16(k_pre)) || (v_pre && !aligned16(v_pre)))
    return SIMSD_ERR_ALIGN;
  if (rope) {
    if (!rope->start_pos) return SIMSD_ERR_NULL;
    if (!rope_flags_ok(rope->flags)) return SIMSD_ERR_FLAGS;
    if (!(rope->base > 0.0f) || !std::isfinite(rope->base)) return SIMSD_ERR_SCALE;
    // the cos/sin table lives in LDS beside the key ring
    const long npos = (rope->flags & SIMSD_ROPE_NO_COPY) ? 2L * B : B;
    if (npos * d * 8 > simsd::kMaxRopeTableBytes) return SIMSD_ERR_SIZE;
    if (rope->k_rot) {
      if (!aligned16(rope->k_rot)) return SIMSD_ERR_ALIGN;
      const uintptr_t r0 = reinterpret_cast<uintptr_t>(rope->k_rot), k0 = reinterpret_cast<uintptr_t>(k_blk);
      const uintptr_t n = static_cast<uintptr_t>(b) * 2 * B * Hkv * d * 2;
      if (r0 < k0 + n && k0 < r0 + n) return SIMSD_ERR_ALIAS;
    }
  }
  const simsd::AttnPlan plan = simsd::plan_attention(b, B, Hq, Hkv, d, max_prefix, static_cast<int>(rule));
  if (static_cast<long>(b) * Hkv * plan.row_slices > simsd::kAttnMaxUnits ||
      static_cast<long>(b) * Hkv * plan.row_slices * plan.nsplit > (1L << 30))
    return SIMSD_ERR_SIZE;
  if (check_only || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || ws_bytes < plan.total_bytes)
    return SIMSD_ERR_WORKSPACE;

  simsd::AttnArgs a{};
  a.q_blk = static_cast<const uint16_t*>(q_blk);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.k_pre = static_cast<const uint16_t*>(k_pre);
  a.v_pre = static_cast<const uint16_t*>(v_pre);
  a.offsets = prefix_offsets;
  a.tau = tau;
  a.out = out;
  a.lse = lse;
  a.status = status;
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + plan.counters_bytes);
  a.part_o = reinterpret_cast<float*>(ws + plan.counters_bytes + plan.ml_bytes);
  a.b = b, a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv, a.d = d;
  a.nblk = 2 * B;
  a.row0 = rule == SIMSD_DATA_SKIP ? B : 0;
  a.nrows = rule == SIMSD_DATA_SKIP ? B : 2 * B;
  a.M = a.nrows * a.G;
  a.row_slices = plan.row_slices;
  a.chunk = plan.chunk;
  a.nsplit = plan.nsplit;
  a.shift = plan.shift;
  a.max_prefix = max_prefix;
  if (static_cast<long>(b) * Hkv * plan.row_slices > simsd::kAttnMaxUnits) return SIMSD_ERR_SIZE;
  const long total = static_cast<long>(b) * Hkv * plan.row_slices * plan.nsplit;
  if (total > (1L << 30)) return SIMSD_ERR_SIZE;
  a.total_real = static_cast<int>(total);
  a.total_grid = static_cast<int>((total + 7) / 8 * 8);
  const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt(static_cast<float>(d));
  a.scale_log2 = sc * 1.4426950408889634f;
  a.data_rule = static_cast<int>(rule);
  a.out_f32 = (flags & SIMSD_OUT_F32) ? 1 : 0;
  a.kv_head_major = (flags & SIMSD_KV_HEAD_MAJOR) ? 1 : 0;
  a.kv_pair = (flags & SIMSD_KV_PAIRED) ? 2 : 1;
  const bool lens = (flags & SIMSD_PREFIX_LENS) != 0;
  a.prefix_lens = lens ? prefix_offsets + b + 1 : prefix_offsets + 1;
  a.prefix_lens_are_ends = lens ? 0 : 1;
  a.xcd_remap = plan.xcd_remap;
  a.rotate = plan.rotate;
  a.lpt = plan.lpt;
  if (rope) {
    a.rope = 1;
    a.start_pos = rope->start_pos;
    fill_inv_freq(a.rope_inv_freq, rope->base, d);
    a.rope_interleaved = (rope->flags & SIMSD_ROPE_INTERLEAVED) ? 1 : 0;
    a.rope_no_copy = (rope->flags & SIMSD_ROPE_NO_COPY) ? 1 : 0;
    a.rope_positions = (rope->flags & SIMSD_ROPE_POSITIONS) ? 1 : 0;
    a.k_rot = static_cast<uint16_t*>(rope->k_rot);
  }
  return launch_status(simsd::launch_verify_attention(a, plan, static_cast<hipStream_t>(stream)));
}

// ---- the allocation-free attention entry point ----
// One fixed device buffer, of this size, stands in for the caller's workspace
// (every GPU the library runs on holds its own copy until the process ends).
constexpr size_t kScratchBytes = static_cast<size_t>(SIMSD_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= static_cast<size_t>(simsd::kAttnMaxUnits) * 4,
              "the scratch holds at least the counter region");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};  // the device address of `scratch` on each device, once known

__global__ void zero_words_kernel(uint4* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The address of the current device's scratch array. On the first call on a
// device it is looked up (hipGetSymbolAddress, with that device current) and
// the counter region at its start is cleared by a fill kernel on `stream`,
// ahead of the kernels the call then enqueues there; every attention call
// leaves that region zero again.
int scratch_of_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SIMSD_ERR_SIZE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launch_status(e);
    if (!p) return launch_status(hipErrorInvalidSymbol);
    const int n = simsd::kAttnMaxUnits * 4 / 16;  // counter words, 16 bytes per thread
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint4*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_status(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SIMSD_OK;
}

}  // namespace

namespace simsd {
int tuning(int key) {
  return key >= 0 && key < SIMSD_TUNE_COUNT ? g_tuning[key].load(std::memory_order_relaxed) : -1;
}
}  // namespace simsd

extern "C" {

int simsd_set_tuning(int key, int value) {
  if (key < 0 || key >= SIMSD_TUNE_COUNT || value < -1) return SIMSD_ERR_SIZE;
  g_tuning[key].store(value, std::memory_order_relaxed);
  return SIMSD_OK;
}

int simsd_rope_copy(void* q_blk, void* k_blk, const int32_t* start_pos, int b, int B, int Hq,
                    int Hkv, int d, float rope_base, uint32_t flags, void* stream) {
  if (!q_blk || !k_blk || !start_pos) return SIMSD_ERR_NULL;
  int rc = check_common(b, B, Hq, Hkv, d);
  if (rc) return rc;
  if (!rope_flags_ok(flags)) return SIMSD_ERR_FLAGS;
  if (!(rope_base > 0.0f) || !std::isfinite(rope_base)) return SIMSD_ERR_SCALE;
  if (!aligned16(q_blk) || !aligned16(k_blk)) return SIMSD_ERR_ALIGN;
  simsd::RopeArgs a{};
  a.q = static_cast<uint16_t*>(q_blk);
  a.k = static_cast<uint16_t*>(k_blk);
  a.start_pos = start_pos;
  a.b = b, a.B = B, a.Hq = Hq, a.Hkv = Hkv, a.d = d;
  fill_inv_freq(a.inv_freq, rope_base, d);
  a.interleaved = (flags & SIMSD_ROPE_INTERLEAVED) ? 1 : 0;
  a.no_copy = (flags & SIMSD_ROPE_NO_COPY) ? 1 : 0;
  a.positions = (flags & SIMSD_ROPE_POSITIONS) ? 1 : 0;
  return launch_status(simsd::launch_rope_copy(a, static_cast<hipStream_t>(stream)));
}

size_t simsd_verify_attention_workspace(int b, int B, int Hq, int Hkv, int d, int max_prefix) {
  if (check_common(b, B, Hq, Hkv, d) || max_prefix < 0 || max_prefix > simsd::kMaxPrefix) return 0;
  if (static_cast<long>(b) * Hkv * ((2L * B * (Hq / Hkv) + 127) / 128) > simsd::kAttnMaxUnits) return 0;
  // The data-row rule changes the row count and so the plan: size for both.
  const size_t all_rows = simsd::plan_attention(b, B, Hq, Hkv, d, max_prefix, 0).total_bytes;
  const size_t slots_only = simsd::plan_attention(b, B, Hq, Hkv, d, max_prefix, 2).total_bytes;
  return all_rows > slots_only ? all_rows : slots_only;
}

int simsd_verify_attention(const void* q_blk, const void* k_blk, const void* v_blk,
                           const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                           const int32_t* tau, void* out, float* lse, int b, int B, int Hq,
                           int Hkv, int d, int max_prefix, float scale, uint32_t flags,
                           int32_t* status, void* workspace, size_t ws_bytes, void* stream) {
  return verify_attention_impl(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse, b, B, Hq,
                               Hkv, d, max_prefix, scale, flags, status, workspace, ws_bytes, stream,
                               nullptr);
}

int simsd_verify_attention_rope(const void* q_blk, const void* k_blk, const void* v_blk,
                                const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                                const int32_t* tau, const int32_t* start_pos, float rope_base,
                                uint32_t rope_flags, void* k_rot, void* out, float* lse, int b, int B,
                                int Hq, int Hkv, int d, int max_prefix, float scale, uint32_t flags,
                                int32_t* status, void* workspace, size_t ws_bytes, void* stream) {
  const RopeIn rope{start_pos, rope_base, rope_flags, k_rot};
  return verify_attention_impl(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse, b, B, Hq,
                               Hkv, d, max_prefix, scale, flags, status, workspace, ws_bytes, stream,
                               &rope);
}

int simsd_verify_attention_noalloc(const void* q_blk, const void* k_blk, const void* v_blk,
                                   const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                                   const int32_t* tau, void* out, float* lse, int b, int B, int Hq, int Hkv,
                                   int d, int max_prefix, float scale, uint32_t flags, int32_t* status,
                                   void* stream) {
  // sizes and arguments first (nothing touched on a bad call), then the
  // scratch size the plan needs against the fixed buffer
  const size_t need = simsd_verify_attention_workspace(b, B, Hq, Hkv, d, max_prefix);
  int rc = verify_attention_impl(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse, b, B, Hq,
                                 Hkv, d, max_prefix, scale, flags, status, nullptr, 0, stream, nullptr,
                                 /*check_only=*/true);
  if (rc != SIMSD_ERR_WORKSPACE) return rc;  // an argument error, reported as for simsd_verify_attention
  if (need == 0 || need > kScratchBytes) return SIMSD_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  return verify_attention_impl(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau, out, lse, b, B, Hq, Hkv,
                               d, max_prefix, scale, flags, status, ws, kScratchBytes, stream, nullptr);
}

size_t simsd_verify_attention_mask_workspace(int b, int R, int Hq, int Hkv, int d, int max_prefix) {
  if (R < 1 || R > 128 || check_common(b, 1, Hq, Hkv, d) || max_prefix < 0 || max_prefix > simsd::kMaxPrefix)
    return 0;
  const simsd::AttnPlan plan = simsd::plan_attention_rows(b, R, Hq, Hkv, d, max_prefix);
  if (static_cast<long>(b) * Hkv * plan.row_slices > simsd::kAttnMaxUnits) return 0;
  return plan.total_bytes;
}

int simsd_verify_attention_mask(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pre,
                                const void* v_pre, const int32_t* prefix_offsets, const uint64_t* block_mask,
                                void* out, float* lse, int b, int R, int Hq, int Hkv, int d, int max_prefix,
                                float scale, uint32_t flags, int32_t* status, void* workspace,
                                size_t ws_bytes, void* stream) {
  if (!q_blk || !k_blk || !v_blk || !prefix_offsets || !block_mask || !out) return SIMSD_ERR_NULL;
  if (max_prefix > 0 && (!k_pre || !v_pre)) return SIMSD_ERR_NULL;
  if (R < 1 || R > 128) return SIMSD_ERR_SIZE;
  int rc = check_common(b, 1, Hq, Hkv, d);
  if (rc) return rc;
  if (max_prefix < 0 || max_prefix > simsd::kMaxPrefix) return SIMSD_ERR_SIZE;
  if (flags & ~(SIMSD_OUT_F32 | SIMSD_KV_HEAD_MAJOR | SIMSD_PREFIX_LENS | SIMSD_KV_PAIRED)) return SIMSD_ERR_FLAGS;
  if (!paired_ok(flags, k_pre, v_pre, d)) return SIMSD_ERR_FLAGS;
  if (!std::isfinite(scale)) return SIMSD_ERR_SCALE;
  if (!aligned16(q_blk) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out) ||
      (k_pre && !aligned16(k_pre)) || (v_pre && !aligned16(v_pre)) ||
      (reinterpret_cast<uintptr_t>(block_mask) & 7u))
    return SIMSD_ERR_ALIGN;
  const simsd::AttnPlan plan = simsd::plan_attention_rows(b, R, Hq, Hkv, d, max_prefix);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || ws_bytes < plan.total_bytes)
    return SIMSD_ERR_WORKSPACE;
  simsd::AttnArgs a{};
  a.q_blk = static_cast<const uint16_t*>(q_blk);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.k_pre = static_cast<const uint16_t*>(k_pre);
  a.v_pre = static_cast<const uint16_t*>(v_pre);
  a.offsets = prefix_offsets;
  a.tau = nullptr;
  a.out = out;
  a.lse = lse;
  a.status = status;
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + plan.counters_bytes);
  a.part_o = reinterpret_cast<float*>(ws + plan.counters_bytes + plan.ml_bytes);
  a.b = b, a.B = 0, a.Hq = Hq, a.Hkv = Hkv, a.G = Hq / Hkv, a.d = d;
  a.nblk = R;
  a.row0 = 0;
  a.nrows = R;
  a.M = R * a.G;
  a.row_slices = plan.row_slices;
  a.chunk = plan.chunk;
  a.nsplit = plan.nsplit;
  a.shift = plan.shift;
  a.max_prefix = max_prefix;
  if (static_cast<long>(b) * Hkv * plan.row_slices > simsd::kAttnMaxUnits) return SIMSD_ERR_SIZE;
  const long total = static_cast<long>(b) * Hkv * plan.row_slices * plan.nsplit;
  if (total > (1L << 30)) return SIMSD_ERR_SIZE;
  a.total_real = static_cast<int>(total);
  a.total_grid = static_cast<int>((total + 7) / 8 * 8);
  const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt(static_cast<float>(d));
  a.scale_log2 = sc * 1.4426950408889634f;
  a.data_rule = 0;
  a.out_f32 = (flags & SIMSD_OUT_F32) ? 1 : 0;
  a.kv_head_major = (flags & SIMSD_KV_HEAD_MAJOR) ? 1 : 0;
  a.kv_pair = (flags & SIMSD_KV_PAIRED) ? 2 : 1;
  const bool lens = (flags & SIMSD_PREFIX_LENS) != 0;
  a.prefix_lens = lens ? prefix_offsets + b + 1 : prefix_offsets + 1;
  a.prefix_lens_are_ends = lens ? 0 : 1;
  a.xcd_remap = plan.xcd_remap;
  a.rotate = plan.rotate;
  a.lpt = plan.lpt;
  a.mask_mode = 1;
  a.block_mask = block_mask;
  a.mask_words = (R + 63) / 64;
  return launch_status(simsd::launch_verify_attention(a, plan, static_cast<hipStream_t>(stream)));
}

size_t simsd_accept_workspace(int b, int B, int V) {
  if (b < 1 || b > simsd::kMaxSeqCounters || B < 1 || B > 64 || V < 1 || V > simsd::kMaxAcceptVocab)
    return 0;
  const size_t seg = static_cast<size_t>(b) * simsd::accept_segments(V) * sizeof(double);
  return static_cast<size_t>(simsd::kMaxSeqCounters) * sizeof(int32_t) + (seg + 255) / 256 * 256;
}

int simsd_accept(const float* p, const float* q, const int32_t* draft_tokens, const int32_t* tau,
                 const float* uniforms, int b, int B, int V, int32_t* accept_len,
                 int32_t* correction_token, int32_t* status, void* workspace, size_t ws_bytes,
                 void* stream) {
  if (!p || !q || !draft_tokens || !tau || !uniforms || !accept_len || !correction_token)
    return SIMSD_ERR_NULL;
  if (b < 1 || b > simsd::kMaxSeqCounters || B < 1 || B > 64 || V < 1 || V > simsd::kMaxAcceptVocab)
    return SIMSD_ERR_SIZE;
  if (!aligned16(p) || !aligned16(q)) return SIMSD_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      ws_bytes < simsd_accept_workspace(b, B, V))
    return SIMSD_ERR_WORKSPACE;
  simsd::AcceptArgs a{};
  a.p = p, a.q = q, a.draft = draft_tokens, a.tau = tau, a.u = uniforms;
  a.b = b, a.B = B, a.V = V;
  a.accept_len = accept_len, a.correction = correction_token, a.status = status;
  a.counters = static_cast<int32_t*>(workspace);
  a.seg_sum = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                        static_cast<size_t>(simsd::kMaxSeqCounters) * sizeof(int32_t));
  return launch_status(simsd::launch_accept(a, static_cast<hipStream_t>(stream)));
}

size_t simsd_accept_logits_workspace(int b, int B, int V) {
  const size_t base = simsd_accept_workspace(b, B, V);
  if (!base) return 0;
  const long rows = 2L * b * B;
  const long nseg1 = (V + simsd::kRowStatSeg - 1) / simsd::kRowStatSeg;
  if (rows * nseg1 > simsd::kMaxRowStatUnits) return 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  // row counters 128 bytes apart for up to 2048 rows (the row-statistics
  // kernel indexes them with the same rule), packed beyond that
  const long row_stride = rows <= 2048 ? 32 : 1;
  // per row: (max, 1 / sum, logit at the draft token, unused)
  return base + up(rows * row_stride * sizeof(int32_t)) + up(rows * nseg1 * 2 * sizeof(uint64_t)) +
         up(rows * 4 * sizeof(double));
}

int simsd_accept_logits(const float* target_logits, const float* draft_logits, float temperature,
                        const int32_t* draft_tokens, const int32_t* tau, const float* uniforms, int b,
                        int B, int V, int32_t* accept_len, int32_t* correction_token, int32_t* status,
                        void* workspace, size_t ws_bytes, void* stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !tau || !uniforms || !accept_len ||
      !correction_token)
    return SIMSD_ERR_NULL;
  if (b < 1 || b > simsd::kMaxSeqCounters || B < 1 || B > 64 || V < 1 || V > simsd::kMaxAcceptVocab)
    return SIMSD_ERR_SIZE;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SIMSD_ERR_SCALE;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return SIMSD_ERR_ALIGN;
  const size_t need = simsd_accept_logits_workspace(b, B, V);
  if (!need) return SIMSD_ERR_SIZE;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || ws_bytes < need)
    return SIMSD_ERR_WORKSPACE;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const long rows = 2L * b * B;
  const int nseg1 = (V + simsd::kRowStatSeg - 1) / simsd::kRowStatSeg;
  char* ws = static_cast<char*>(workspace);
  const size_t acc_bytes = simsd_accept_workspace(b, B, V);
  simsd::AcceptArgs a{};
  a.zt = target_logits, a.zd = draft_logits, a.draft = draft_tokens, a.tau = tau, a.u = uniforms;
  a.b = b, a.B = B, a.V = V;
  a.accept_len = accept_len, a.correction = correction_token, a.status = status;
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.seg_sum = reinterpret_cast<double*>(ws + static_cast<size_t>(simsd::kMaxSeqCounters) * sizeof(int32_t));
  size_t off = acc_bytes;
  a.row_counters = reinterpret_cast<int32_t*>(ws + off);
  off += up(rows * (rows <= 2048 ? 32 : 1) * sizeof(int32_t));  // padded as in the workspace size
  a.row_words = reinterpret_cast<unsigned long long*>(ws + off);
  off += up(rows * nseg1 * 2 * sizeof(uint64_t));
  a.row_stats = reinterpret_cast<double*>(ws + off);
  a.nseg1 = nseg1;
  a.inv_t = 1.0 / static_cast<double>(temperature);
  return launch_status(simsd::launch_accept_logits(a, static_cast<hipStream_t>(stream)));
}

int simsd_commit_kv(const void* k_blk, const void* v_blk, const int32_t* tau, const int32_t* accept_len,
                    void* k_cache, void* v_cache, const int32_t* cache_offsets, int32_t* cache_lens,
                    const int32_t* pos, int32_t* next_pos, int b, int B, int Hkv, int d, uint32_t flags,
                    int32_t* status, void* stream) {
  if (!k_blk || !v_blk || !tau || !accept_len || !k_cache || !v_cache || !cache_offsets || !cache_lens)
    return SIMSD_ERR_NULL;
  if (next_pos && !pos) return SIMSD_ERR_NULL;
  int rc = check_common(b, B, Hkv, Hkv, d);
  if (rc) return rc;
  if (flags & ~(SIMSD_KV_HEAD_MAJOR | SIMSD_KV_PAIRED)) return SIMSD_ERR_FLAGS;
  if (!paired_ok(flags, k_cache, v_cache, d)) return SIMSD_ERR_FLAGS;
  // each workgroup rewrites its sequence's length after reading its inputs:
  // the lengths must not be one of the inputs another workgroup reads (the
  // cache and the block are the caller's to keep apart)
  auto overlap = [](const void* x, size_t nx, const void* y, size_t ny) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x), b0 = reinterpret_cast<uintptr_t>(y);
    return a0 < b0 + ny && b0 < a0 + nx;
  };
  const size_t nl = static_cast<size_t>(b) * 4;
  if (overlap(cache_lens, nl, tau, nl * B) || overlap(cache_lens, nl, accept_len, nl) ||
      overlap(cache_lens, nl, cache_offsets, nl + 4))
    return SIMSD_ERR_ALIAS;
  // next_pos is written by the workgroup of its sequence after that workgroup
  // read the sequence's inputs: it may be pos itself, but no other input
  if (next_pos) {
    const size_t np = nl * B;
    if ((next_pos != pos && overlap(next_pos, np, pos, np)) || overlap(next_pos, np, tau, np) ||
        overlap(next_pos, np, accept_len, nl) || overlap(next_pos, np, cache_offsets, nl + 4) ||
        overlap(next_pos, np, cache_lens, nl))
      return SIMSD_ERR_ALIAS;
  }
  if (!aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) || !aligned16(v_cache))
    return SIMSD_ERR_ALIGN;
  simsd::CommitArgs a{};
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.tau = tau;
  a.accept_len = accept_len;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.offsets = cache_offsets;
  a.lens = cache_lens;
  a.pos = pos;
  a.next_pos = next_pos;
  a.status = status;
  a.b = b, a.B = B, a.Hkv = Hkv, a.d = d;
  a.head_major = (flags & SIMSD_KV_HEAD_MAJOR) ? 1 : 0;
  a.pair = (flags & SIMSD_KV_PAIRED) ? 2 : 1;
  return launch_status(simsd::launch_commit_kv(a, static_cast<hipStream_t>(stream)));
}

const char* simsd_status_string(int code) {
  switch (code) {
    case SIMSD_OK: return "ok";
    case SIMSD_ERR_NULL: return "a required pointer is NULL";
    case SIMSD_ERR_SIZE: return "a size argument is out of range";
    case SIMSD_ERR_HEADS: return "Hq is not a multiple of Hkv";
    case SIMSD_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case SIMSD_ERR_FLAGS: return "unknown or conflicting flags";
    case SIMSD_ERR_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case SIMSD_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SIMSD_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case SIMSD_ERR_SCALE: return "rope_base or scale out of range";
    case SIMSD_ERR_ALIAS: return "an output overlaps an input it must not overlap";
    case SIMSD_ERR_SCRATCH: return "the sizes need more scratch than the fixed device buffer holds";
    default: return "unknown status";
  }
}

int simsd_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
