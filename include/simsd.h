/*
 * simsd.h -- C ABI of libsimsd, the MI355X (gfx950) verification hot path of
 * SimSD (simple speculative decoding for diffusion language models).
 *
 * Sources, cited by page title and section (second-hand summaries of the
 * SimSD paper, arXiv 2606.02544):
 *   [nl] "Technische Samenvatting: SimSD - Simple Speculative Decoding in
 *        Diffusion Language Models" (gist.science/nl/paper/2606.02544)
 *   [fr] "SimSD: Simple Speculative Decoding in Diffusion Language Models",
 *        part "Resume Technique" (gist.science/fr/paper/2606.02544)
 *
 * The verification step of one speculative round (see [nl]/[fr] Methodologie
 * 4): the target model reads the cached prompt, a data section D of B draft
 * tokens and a mask section D~ of B [MASK] slots (Methodologie 1), rotates the
 * block's queries and keys with the RoPE copy rule (Methodologie 3), runs one
 * attention pass under the temporal mask (Methodologie 2), and finally the
 * drafts are accepted or rejected along the draft's temporal order. The entry
 * points below are the attention-layer and acceptance parts of that step
 * (RoPE-copy, attention, acceptance), and their extensions (RoPE-copy fused
 * into attention, attention under an explicit mask, acceptance from logits);
 * projections, MLP and LM head are outside this library.
 *
 * Conventions common to every entry point
 *   - Every tensor argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or synchronises; each call enqueues its
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     returns at once.
 *   - The return value is a host-detected error code (simsd_status_t). On any
 *     nonzero return nothing has been launched and no memory was touched.
 *   - Data-dependent problems are reported per sequence in the optional device
 *     array `status` (int32 [b]): each call ORs its SIMSD_DEV_* bits into it
 *     and never clears it, so one zeroed array can collect a whole chain.
 *   - bf16 is the IEEE-754 binary32 upper half (bfloat16), stored as uint16.
 *   - Block rows of a sequence are numbered r = 0..2B-1: r < B is the data
 *     token D_{r+1}, r >= B the mask slot D~_{r-B+1}.
 *   - tau[s][k-1] is the temporal step label tau(k) in 1..B of response
 *     position k (the step map of Methodologie 2; the pages call the map mu and
 *     its values tau). D_k and D~_k share tau(k).
 *   - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 */
#ifndef SIMSD_H
#define SIMSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SIMSD_OK = 0,
  SIMSD_ERR_NULL = 1,      /* a required pointer is NULL */
  SIMSD_ERR_SIZE = 2,      /* b < 1, B outside 1..64, Hq/Hkv < 1, V < 1, max_prefix < 0, ... */
  SIMSD_ERR_HEADS = 3,     /* Hq is not a multiple of Hkv */
  SIMSD_ERR_HEAD_DIM = 4,  /* d is not 64 or 128 */
  SIMSD_ERR_FLAGS = 5,     /* unknown or conflicting flag bits */
  SIMSD_ERR_WORKSPACE = 6, /* workspace NULL, too small or not 256-byte aligned */
  SIMSD_ERR_ALIGN = 7,     /* a tensor pointer is not 16-byte aligned */
  SIMSD_ERR_LAUNCH = 8,    /* the HIP runtime refused a launch (see simsd_last_hip_error) */
  SIMSD_ERR_SCALE = 9,     /* rope_base <= 0 or a non-finite scale */
  SIMSD_ERR_ALIAS = 10,    /* an output overlaps an input it must not overlap */
  SIMSD_ERR_SCRATCH = 11   /* simsd_verify_attention_noalloc: the sizes need more than the fixed
                              scratch buffer holds */
} simsd_status_t;

/* Device status bits (int32 per sequence, OR-ed in). */
#define SIMSD_DEV_BAD_TAU 1       /* tau[s] is not a permutation of 1..B */
#define SIMSD_DEV_ZERO_RESIDUAL 2 /* acceptance: residual mass 0, correction drawn from p */
#define SIMSD_DEV_Q_ZERO 4        /* acceptance: q(x) == 0 met (accepted iff p(x) > 0) */
#define SIMSD_DEV_BAD_TOKEN 8     /* acceptance: a draft id outside [0, V) (step rejected) */
#define SIMSD_DEV_BAD_PREFIX 16   /* attention: P_s < 0 or P_s > max_prefix (P_s clamped into range) */
#define SIMSD_DEV_SYNC_TIMEOUT 32 /* acceptance: a segment mass of this sequence was not seen within
                                     the poll bound; the correction is unspecified and the workspace
                                     must be zeroed again before reuse (not expected to occur) */
#define SIMSD_DEV_COMMIT_OVERFLOW 64 /* KV commit: accept_len outside 0..B, a negative used length, or
                                        a cache region too small; nothing of the sequence written */

/* simsd_rope_copy flags */
#define SIMSD_ROPE_HALF 0u        /* rotate-half pairing (i, i + d/2) (default) */
#define SIMSD_ROPE_INTERLEAVED 1u /* pairing (2i, 2i+1) */
#define SIMSD_ROPE_NO_COPY 2u     /* ablation: D~_k at start + B + k - 1 instead of start + k - 1 */
#define SIMSD_ROPE_POSITIONS 4u   /* start_pos holds one position per pair, int32 [b][B]: D_k and D~_k
                                     at start_pos[s][k-1] (a later round of a block; not with NO_COPY) */

/* simsd_verify_attention flags: data-row rule (2 bits) | output dtype | cache layout */
#define SIMSD_DATA_CAUSAL 0u /* D_i sees the prefix and D_j with tau(j) <= tau(i) (default) */
#define SIMSD_DATA_BIDIR 1u  /* D_i sees the prefix and every D_j */
#define SIMSD_DATA_SKIP 2u   /* data rows are not computed; their out/lse rows are untouched */
#define SIMSD_OUT_F32 4u     /* out is fp32 instead of bf16 */
#define SIMSD_KV_HEAD_MAJOR 8u /* k_pre / v_pre are [Hkv][sum P][d] instead of [sum P][Hkv][d] */
#define SIMSD_PREFIX_LENS 16u  /* prefix_offsets holds 2b+1 int32: b+1 region bounds, then b used
                                  lengths (a cache with room to grow; see simsd_commit_kv) */
#define SIMSD_KV_PAIRED 32u    /* k_pre / v_pre (k_cache / v_cache for simsd_commit_kv) are the two
                                  halves of one buffer whose innermost dims are [2][d], the key
                                  row then the value row of each (token, KV head): [sum P][Hkv][2][d],
                                  or [Hkv][sum P][2][d] with SIMSD_KV_HEAD_MAJOR. v_pre must equal
                                  k_pre + d elements (else SIMSD_ERR_FLAGS). One tile's keys and
                                  values are then one contiguous run (b16: ~5% faster streaming) */

/*
 * simsd_rope_copy -- rotary position embedding of the block's queries and
 * keys with the copy rule ([nl]/[fr] Methodologie 3: each mask slot D~_k reuses
 * the RoPE index of its paired data token D_k).
 *
 *   q_blk      bf16 [b][2B][Hq][d], rotated in place
 *   k_blk      bf16 [b][2B][Hkv][d], rotated in place
 *   start_pos  int32 [b]: position of D_1 of each sequence (normally its
 *              prefix length P_s). D_k and D~_k both sit at start_pos + k - 1;
 *              with SIMSD_ROPE_NO_COPY, D~_k sits at start_pos + B + k - 1.
 *              With SIMSD_ROPE_POSITIONS it is int32 [b][B] instead, one
 *              position per pair (each pair is one response position,
 *              Methodologie 1): D_k and D~_k both sit at start_pos[s][k-1].
 *              A later round of a block verifies the positions still open,
 *              wherever they lie; simsd_commit_kv writes them.
 *   rope_base  base of the frequencies: frequency i = 0..d/2-1 turns by
 *              pos * rope_base^(-2i/d) radians. Angles, cos/sin and the
 *              rotation are evaluated in fp64; each result is rounded to bf16
 *              once (round to nearest even).
 *   flags      SIMSD_ROPE_* bits.
 * The cached prefix keys are not touched (they were rotated when cached).
 * Errors: SIMSD_ERR_NULL, _SIZE (b<1, B not in 1..64, heads<1), _HEAD_DIM,
 * _FLAGS (unknown bits, or NO_COPY with POSITIONS), _SCALE (rope_base <= 0 or
 * not finite), _ALIGN, _LAUNCH.
 */
int simsd_rope_copy(void* q_blk, void* k_blk, const int32_t* start_pos, int b, int B, int Hq,
                    int Hkv, int d, float rope_base, uint32_t flags, void* stream);

/*
 * simsd_verify_attention -- one attention pass of the verification forward
 * over the cached prefix plus the paired block, under the temporal mask
 * ([nl]/[fr] Methodologie 2 and 4; the prefix comes from the KV cache,
 * [nl] Belangrijkste Bijdragen 3 / [fr] Principales Contributions).
 *
 * Allowed keys of a query in block row r of sequence s:
 *   - every cached prefix position of the sequence;
 *   - mask slot D~_i: data tokens D_j with tau(j) < tau(i) and mask slots D~_j
 *     with tau(j) >= tau(i) (itself included);
 *   - data token D_i (the pages give no rule; chosen by flags):
 *     SIMSD_DATA_CAUSAL: D_j with tau(j) <= tau(i); SIMSD_DATA_BIDIR: every
 *     D_j; never a mask slot. SIMSD_DATA_SKIP: the row is not computed.
 * out = softmax over the allowed keys only (masked keys enter neither the
 * maximum nor the sum) of scale * q.k, applied to the values.
 *
 *   q_blk, k_blk, v_blk  bf16 [b][2B][Hq|Hkv|Hkv][d] (post-RoPE)
 *   k_pre, v_pre         bf16 packed prefix cache, token-major [sum_s P_s][Hkv][d]
 *                        (default) or, with SIMSD_KV_HEAD_MAJOR, head-major
 *                        [Hkv][sum_s P_s][d]; rows prefix_offsets[s] ..
 *                        prefix_offsets[s+1]-1 belong to sequence s. Head-major
 *                        lets each KV head's keys stream contiguously (faster
 *                        on long prefixes); sum_s P_s is read from
 *                        prefix_offsets[b].
 *   prefix_offsets       int32 [b+1], non-decreasing, offsets[0] = 0. With
 *                        SIMSD_PREFIX_LENS it holds 2b+1 values: the b+1
 *                        bounds of each sequence's cache region, followed by
 *                        the b used lengths P_s; the prefix of sequence s is
 *                        then the first P_s rows of its region (rows
 *                        offsets[s] .. offsets[s] + P_s - 1; the head-major
 *                        stride is offsets[b]), and P_s larger than the region
 *                        is clamped to it and flagged SIMSD_DEV_BAD_PREFIX.
 *   tau                  int32 [b][B]
 *   out                  [b][2B][Hq][d], bf16 (or fp32 with SIMSD_OUT_F32)
 *   lse                  optional fp32 [b][2B][Hq]: natural-log sum of exp of
 *                        the allowed scores (NULL to skip)
 *   max_prefix           host int >= every P_s, at most 2^30; it sizes the launch. A
 *                        sequence with P_s > max_prefix (or P_s < 0) is
 *                        computed with P_s clamped into [0, max_prefix] and
 *                        flagged SIMSD_DEV_BAD_PREFIX.
 *   scale                softmax scale; <= 0 selects 1/sqrt(d)
 *   status               optional int32 [b]; SIMSD_DEV_BAD_TAU (output of
 *                        that sequence is then unspecified), _BAD_PREFIX
 *   workspace, ws_bytes  device scratch of at least
 *                        simsd_verify_attention_workspace(...) bytes, 256-byte
 *                        aligned. Its first 256 KiB hold one counter word per
 *                        (sequence, KV head, row slice); the rest holds
 *                        per-split partial results. The first 256 KiB must be
 *                        ZERO before the first call that uses the buffer;
 *                        every call, whatever its sizes, leaves them zero
 *                        again. Calls that share a workspace must not run
 *                        concurrently. b * Hkv * ceil(2B * Hq/Hkv / 128) must
 *                        not exceed 65536 (else SIMSD_ERR_SIZE).
 * Numerics: bf16 inputs, fp32 MFMA accumulation and fp32 softmax.
 * Errors: SIMSD_ERR_NULL, _SIZE, _HEADS, _HEAD_DIM, _FLAGS, _WORKSPACE,
 * _ALIGN, _SCALE, _LAUNCH.
 */
int simsd_verify_attention(const void* q_blk, const void* k_blk, const void* v_blk,
                           const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                           const int32_t* tau, void* out, float* lse, int b, int B, int Hq,
                           int Hkv, int d, int max_prefix, float scale, uint32_t flags,
                           int32_t* status, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes simsd_verify_attention (and simsd_verify_attention_rope)
 * needs for these sizes (0 on bad sizes). */
size_t simsd_verify_attention_workspace(int b, int B, int Hq, int Hkv, int d, int max_prefix);

/*
 * simsd_verify_attention_noalloc -- simsd_verify_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and bit-identical results. The workspace is a
 * fixed device array inside the library, SIMSD_NOALLOC_SCRATCH_BYTES per GPU,
 * held by each GPU the library runs on until the process ends. Nothing is
 * allocated or freed by the call.
 *   - Sizes whose simsd_verify_attention_workspace exceeds
 *     SIMSD_NOALLOC_SCRATCH_BYTES are refused with SIMSD_ERR_SCRATCH (the
 *     headline shapes need at most 16.5 MiB: 8 sequences of 16384 cached
 *     tokens with B = 16 and 32/8 heads of 128).
 *   - The stream must belong to the current device. The first call on a
 *     device looks up that device's copy of the array and enqueues, ahead of
 *     its own kernels, a fill kernel that clears the counter region at its
 *     start; every call leaves that region zero again.
 *   - Every call on a GPU shares that GPU's array: calls that may overlap in
 *     time on one GPU (other streams, other threads, concurrent replays of
 *     captured graphs) race and must be serialised by the caller.
 * Errors: those of simsd_verify_attention except _WORKSPACE, and
 * SIMSD_ERR_SCRATCH.
 */
#define SIMSD_NOALLOC_SCRATCH_BYTES (32u << 20)
int simsd_verify_attention_noalloc(const void* q_blk, const void* k_blk, const void* v_blk,
                                   const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                                   const int32_t* tau, void* out, float* lse, int b, int B, int Hq, int Hkv,
                                   int d, int max_prefix, float scale, uint32_t flags, int32_t* status,
                                   void* stream);

/*
 * simsd_verify_attention_mask -- the same attention pass with the block mask
 * given explicitly instead of generated from tau: the generalisation that
 * verifies several drafts or a draft graph against one cached prefix (the
 * Spiffy page's draft graphs; the tau rule of [nl]/[fr] Methodologie 2 is the
 * special case). Every block row sees the whole cached prefix of its sequence
 * and the block keys its mask allows; the softmax runs over those keys only.
 * A row that sees no key (empty prefix, empty mask row) gets out = 0 and
 * lse = -inf.
 *
 *   q_blk, k_blk, v_blk  bf16 [b][R][Hq|Hkv|Hkv][d], R block rows (1..128)
 *   block_mask   uint64 [b][R][ceil(R/64)], 8-byte aligned: bit (c % 64) of
 *                word c / 64 of row r set = row r sees block key c
 *   flags        SIMSD_OUT_F32 | SIMSD_KV_HEAD_MAJOR | SIMSD_PREFIX_LENS only
 *   status       optional int32 [b]; SIMSD_DEV_BAD_PREFIX
 *   other arguments as for simsd_verify_attention; the workspace size comes
 *   from simsd_verify_attention_mask_workspace.
 * Errors: SIMSD_ERR_NULL, _SIZE (R outside 1..128, ...), _HEADS, _HEAD_DIM,
 * _FLAGS, _WORKSPACE, _ALIGN, _SCALE, _LAUNCH.
 */
int simsd_verify_attention_mask(const void* q_blk, const void* k_blk, const void* v_blk, const void* k_pre,
                                const void* v_pre, const int32_t* prefix_offsets, const uint64_t* block_mask,
                                void* out, float* lse, int b, int R, int Hq, int Hkv, int d, int max_prefix,
                                float scale, uint32_t flags, int32_t* status, void* workspace,
                                size_t ws_bytes, void* stream);

/* Workspace bytes simsd_verify_attention_mask needs (0 on bad sizes). */
size_t simsd_verify_attention_mask_workspace(int b, int R, int Hq, int Hkv, int d, int max_prefix);

/*
 * simsd_verify_attention_rope -- the RoPE copy rule ([nl]/[fr] Methodologie
 * 3: a mask slot D~_k takes the rotary position of its data token D_k) fused
 * into the attention pass: the same result as simsd_rope_copy on q_blk and
 * k_blk followed by simsd_verify_attention, in one launch, without modifying
 * q_blk or k_blk. The query rows and the block key rows are rotated in
 * registers with exactly the arithmetic of simsd_rope_copy (fp64 angles,
 * cos/sin and rotation, one rounding to bf16), so out and lse are
 * bit-identical to the two-call sequence.
 *
 *   q_blk, k_blk   bf16 [b][2B][Hq|Hkv][d] BEFORE RoPE (read only)
 *   start_pos, rope_base, rope_flags  as for simsd_rope_copy (with
 *                  SIMSD_ROPE_POSITIONS, one position per pair, [b][B])
 *   k_rot          optional bf16 [b][2B][Hkv][d] output: the rotated block
 *                  keys (what simsd_rope_copy would leave in k_blk; the rows a
 *                  KV-cache commit appends). Must not overlap k_blk. NULL to
 *                  skip.
 *   all other arguments as for simsd_verify_attention (the same workspace).
 * The cos/sin table of the block positions lives in LDS:
 * (NO_COPY ? 2B : B) * d <= 8192 (only d = 128 with SIMSD_ROPE_NO_COPY and
 * B > 32 is refused, SIMSD_ERR_SIZE).
 * Errors: those of simsd_verify_attention and simsd_rope_copy, and
 * SIMSD_ERR_ALIAS (k_rot overlaps k_blk).
 */
int simsd_verify_attention_rope(const void* q_blk, const void* k_blk, const void* v_blk,
                                const void* k_pre, const void* v_pre, const int32_t* prefix_offsets,
                                const int32_t* tau, const int32_t* start_pos, float rope_base,
                                uint32_t rope_flags, void* k_rot, void* out, float* lse, int b, int B,
                                int Hq, int Hkv, int d, int max_prefix, float scale, uint32_t flags,
                                int32_t* status, void* workspace, size_t ws_bytes, void* stream);

/*
 * simsd_accept -- rejection-sampling acceptance along the draft's temporal
 * order ([nl]/[fr] Methodologie 4: standard rejection sampling in the order
 * the draft induced; the longest accepted prefix is committed).
 *
 *   p, q          fp32 [b][B][V]: target and draft probabilities at the B
 *                 response positions, in natural position order
 *   draft_tokens  int32 [b][B]: draft token id at each position
 *   tau           int32 [b][B]
 *   uniforms      fp32 [b][B+1] in [0,1): u_t (t = 1..B) decides temporal
 *                 step t, u_{B+1} draws the correction
 *   accept_len    int32 [b] out: L = number of leading accepted steps (0..B)
 *   correction_token int32 [b] out: -1 when L == B (no bonus slot), else the
 *                 token drawn for position tau^-1(L+1)
 * Per sequence: for t = 1..B with k = tau^-1(t) and x = draft[k], step t is
 * accepted iff u_t < min(1, p[k][x] / q[k][x]) (IEEE fp32 division; if
 * q[k][x] == 0 the step is accepted iff p[k][x] > 0). On the first rejection
 * the correction is the smallest y whose running sum of the residual
 * max(0, p[k][y] - q[k][y]) (fp32 terms, fp64 sums) exceeds u_{B+1} * Z, Z
 * the total residual. If Z == 0 the same draw is made from p[k]
 * (SIMSD_DEV_ZERO_RESIDUAL). Decisions are bit-reproducible; the drawn token
 * can differ from a sequential-sum reference only when u_{B+1} * Z lies within
 * rounding of a CDF step.
 *   status        optional int32 [b]: SIMSD_DEV_BAD_TAU (then L = 0,
 *                 correction -1), _ZERO_RESIDUAL, _Q_ZERO, _BAD_TOKEN,
 *                 _SYNC_TIMEOUT
 *   workspace, ws_bytes  device scratch of at least simsd_accept_workspace()
 *                 bytes, 256-byte aligned, ALL ZERO before the first call that
 *                 uses it (every call leaves it zero again): the first 256 KiB
 *                 hold one arrival counter per sequence, the rest the
 *                 per-segment residual masses the workgroups of a sequence
 *                 publish to each other. Calls sharing a workspace must not
 *                 run concurrently.
 * Errors: SIMSD_ERR_NULL, _SIZE (b<1 or b>65536, B not in 1..64, V<1 or
 * V>2^21), _ALIGN, _WORKSPACE, _LAUNCH.
 */
int simsd_accept(const float* p, const float* q, const int32_t* draft_tokens, const int32_t* tau,
                 const float* uniforms, int b, int B, int V, int32_t* accept_len,
                 int32_t* correction_token, int32_t* status, void* workspace, size_t ws_bytes,
                 void* stream);

/* Workspace bytes simsd_accept needs for these sizes (0 on bad sizes). */
size_t simsd_accept_workspace(int b, int B, int V);

/*
 * simsd_accept_logits -- acceptance from the verification logits ([nl]/[fr]
 * Methodologie 4: the single verification pass yields the target's logits
 * for every drafted position; the draft model's logits give q). The same
 * decisions as simsd_accept on p = softmax(target_logits / T) and
 * q = softmax(draft_logits / T), row-wise over the vocabulary, with the
 * softmax evaluated where it is needed instead of materialised: one pass
 * over all 2 b B rows finds each row's maximum and sum of exponentials
 * (fp64), then the acceptance step evaluates p and q at the draft tokens
 * and over the rejected position's row (fp64 exp, one rounding to fp32).
 * Large batches run both in one launch (each sequence's acceptance starts
 * once its rows' statistics are published), small ones in two.
 * The temperature is this library's reading (the pages do not define one for
 * SimSD); T = 1 gives the plain softmax.
 *
 *   target_logits, draft_logits  fp32 [b][B][V], natural position order,
 *                 16-byte aligned
 *   temperature   T > 0, finite (else SIMSD_ERR_SCALE)
 *   other arguments as for simsd_accept
 *   workspace, ws_bytes  at least simsd_accept_logits_workspace() bytes,
 *                 256-byte aligned, ALL ZERO before the first call that uses
 *                 it. Every call leaves all of it zero again (counters, ready
 *                 words and the row statistics, which the acceptance pass
 *                 clears once the last reader of a sequence is done), so one
 *                 buffer serves later calls at any sizes it is large enough
 *                 for. Calls sharing a workspace must not run concurrently.
 * Decisions agree with simsd_accept on the fp32-rounded softmax except where
 * a uniform lies within a few fp32 ulps of its step's ratio, or u_{B+1} * Z
 * within rounding of a CDF step (the exponentials are evaluated in another
 * order than a sequential softmax).
 * Errors: SIMSD_ERR_NULL, _SIZE (as simsd_accept; also 2 b B ceil(V/4096) >=
 * 2^24), _SCALE, _ALIGN, _WORKSPACE, _LAUNCH.
 */
int simsd_accept_logits(const float* target_logits, const float* draft_logits, float temperature,
                        const int32_t* draft_tokens, const int32_t* tau, const float* uniforms, int b,
                        int B, int V, int32_t* accept_len, int32_t* correction_token, int32_t* status,
                        void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes simsd_accept_logits needs (0 on bad sizes). */
size_t simsd_accept_logits_workspace(int b, int B, int V);

/*
 * simsd_commit_kv -- commit the accepted drafts of a verification round to the
 * KV cache and name the positions the next round verifies ([nl]/[fr]
 * Methodologie 4, Acceptance / Acceptation: the longest prefix accepted along
 * the temporal order is committed and the round repeats; each pair (D_k, D~_k)
 * is one response position, Methodologie 1; compatibility with a KV cache,
 * [nl] Belangrijkste Bijdragen 3 / [fr] Principales Contributions).
 *
 * Sequence s accepted its first L = accept_len[s] drafts in temporal order,
 * the data tokens D_k with tau(k) <= L. Their key and value rows (block rows
 * k - 1 of k_blk / v_blk, already rotated at their own positions) are written
 * in temporal order t = 1..L (k = tau^-1(t)) to rows cache_lens[s] + t - 1 of
 * the sequence's cache region, and cache_lens[s] grows by L. Under the
 * default data-row rule (SIMSD_DATA_CAUSAL) each of these rows was computed
 * from exactly the context a token-by-token decode in temporal order gives it.
 * The order of rows inside a region does not matter to attention (each row
 * carries its position in its rotated key).
 *
 * The round loop (this library's reading of "the process repeats"): the next
 * round verifies the B smallest positions not in the cache. When L < B, the
 * first of them is the rejected step's position tau^-1(L+1): its correction
 * token is committed but has no key/value row yet, so the caller places it as
 * that round's data token at temporal step 1, with the draft probability of
 * that position equal to the target's (standard rejection sampling then
 * accepts it with probability one), and the next commit appends its row.
 * Then come the other open positions (labels > L + 1) in increasing order,
 * then L positions following this block's largest.
 *
 *   k_blk, v_blk     bf16 [b][2B][Hkv][d] (rows 0..B-1 are D_1..D_B)
 *   tau              int32 [b][B]
 *   accept_len       int32 [b] (the output of simsd_accept)
 *   k_cache, v_cache bf16 cache, token-major [C][Hkv][d] or, with
 *                    SIMSD_KV_HEAD_MAJOR, head-major [Hkv][C][d], C =
 *                    cache_offsets[b]; sequence s owns rows cache_offsets[s]
 *                    .. cache_offsets[s+1]-1, of which the first
 *                    cache_lens[s] are in use. Only the appended rows are
 *                    written.
 *   cache_offsets    int32 [b+1], non-decreasing, region bounds
 *   cache_lens       int32 [b], updated in place (each sequence's length is
 *                    read and advanced by the one workgroup that copies its
 *                    rows). Laid out right after the region bounds
 *                    (cache_lens = cache_offsets + b + 1), the same array
 *                    serves as the prefix_offsets of simsd_verify_attention
 *                    with SIMSD_PREFIX_LENS.
 *   pos              int32 [b][B]: the positions of this round's pairs (what
 *                    simsd_rope_copy took); required with next_pos, else
 *                    unused and may be NULL
 *   next_pos         optional int32 [b][B] out: the next round's positions
 *                    as above (pass it to simsd_rope_copy /
 *                    simsd_verify_attention_rope with SIMSD_ROPE_POSITIONS).
 *                    It may be pos itself (updated in place). A sequence with
 *                    a status bit from this call keeps its block (next_pos =
 *                    pos). Positions stay below 2^31 - B.
 *   flags            SIMSD_KV_HEAD_MAJOR | SIMSD_KV_PAIRED or 0
 *   status           optional int32 [b]; SIMSD_DEV_BAD_TAU or
 *                    SIMSD_DEV_COMMIT_OVERFLOW (L outside 0..B, a negative
 *                    length, or L more rows do not fit the region): nothing of
 *                    that sequence is written and its length is kept.
 * The cache must not overlap k_blk / v_blk; cache_lens must not overlap tau,
 * accept_len or cache_offsets, and next_pos no input other than pos itself
 * (SIMSD_ERR_ALIAS).
 * Errors: SIMSD_ERR_NULL (next_pos without pos, ...), _SIZE (b<1, B not in
 * 1..64, Hkv<1), _HEAD_DIM, _FLAGS, _ALIGN (bf16 tensors 16-byte aligned),
 * _ALIAS, _LAUNCH.
 */
int simsd_commit_kv(const void* k_blk, const void* v_blk, const int32_t* tau, const int32_t* accept_len,
                    void* k_cache, void* v_cache, const int32_t* cache_offsets, int32_t* cache_lens,
                    const int32_t* pos, int32_t* next_pos, int b, int B, int Hkv, int d, uint32_t flags,
                    int32_t* status, void* stream);

/*
 * simsd_set_tuning -- override one choice of the kernel plans, process-wide,
 * for measurement and for tests that check every kernel variant against a
 * reference. The plans read only these explicit settings (never the
 * environment), so a call's plan and workspace size depend on its arguments
 * and on the settings in force when it is made; change settings only while no
 * call is being issued from another thread, and query workspace sizes after
 * setting them. value -1 restores the plan's own choice for that key.
 *   SIMSD_TUNE_ATTN_PIPE       attention key-tile ring / wave layout variant
 *   SIMSD_TUNE_ATTN_TARGET_WG  workgroups the split plan aims for (>= 1)
 *   SIMSD_TUNE_ATTN_CHUNK_MAX  cap on prefix keys per split (>= 64)
 *   SIMSD_TUNE_ATTN_XCD_REMAP  0/1: keep a unit's splits on one XCD
 *   SIMSD_TUNE_ATTN_ROTATE     0/1: per-unit starting prefix tile
 *   SIMSD_TUNE_ATTN_LPT        0/1: longest-first order of unsplit launches
 *   SIMSD_TUNE_ATTN_SHIFT      prefix keys moved off split 0 (>= 0; default: one key
 *                              tile per block tile of the variant launched)
 *   SIMSD_TUNE_ACCEPT_PER      acceptance entries per thread: 4, 8 or 16
 *   SIMSD_TUNE_ROWSTAT_PER     row-statistics entries per thread: 16, 32 or 64
 * Returns SIMSD_OK, or SIMSD_ERR_SIZE for an unknown key or a value below -1.
 */
#define SIMSD_TUNE_ATTN_PIPE 0
#define SIMSD_TUNE_ATTN_TARGET_WG 1
#define SIMSD_TUNE_ATTN_CHUNK_MAX 2
#define SIMSD_TUNE_ATTN_XCD_REMAP 3
#define SIMSD_TUNE_ATTN_ROTATE 4
#define SIMSD_TUNE_ATTN_LPT 5
#define SIMSD_TUNE_ATTN_SHIFT 6
#define SIMSD_TUNE_ACCEPT_PER 7
#define SIMSD_TUNE_ROWSTAT_PER 8
#define SIMSD_TUNE_COUNT 9
int simsd_set_tuning(int key, int value);

/* Static text for a simsd_status_t value. */
const char* simsd_status_string(int code);

/* The hipError_t of the last failed launch in this thread (0 if none). */
int simsd_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SIMSD_H */
