/*
 * simsd_oracle.c -- plain, slow CPU oracle for the SimSD verification path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this file; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it. It shares no source with the HIP kernels.
 *
 * Sources (cited by page title and section; the pages are second-hand
 * summaries of the SimSD paper, arXiv 2606.02544):
 *   [nl] "Technische Samenvatting: SimSD - Simple Speculative Decoding in
 *        Diffusion Language Models" (gist.science/nl/paper/2606.02544)
 *   [fr] "SimSD: Simple Speculative Decoding in Diffusion Language Models",
 *        part "Resume Technique" (gist.science/fr/paper/2606.02544)
 *
 * Precision: attention and RoPE in fp64 on the exact (bf16-valued) inputs.
 * The acceptance test takes its accept/reject decisions in fp32, the
 * precision the GPU path decides in, so that integer results can be compared
 * bit for bit; its residual mass is summed in fp64 in vocabulary order.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Data-row rules (the pages define only mask-slot rows; see
 * simsd_oracle_allowed). Numeric values match the public flag bits. */
#define ORACLE_DATA_CAUSAL 0
#define ORACLE_DATA_BIDIR 1
#define ORACLE_DATA_SKIP 2

/* Step map. [nl] Methodologie 2 / [fr] Methodologie 2: a permutation gives each
 * response position k (1..B) a temporal step label tau(k) in 1..B. Writes the
 * inverse (inv[t-1] = the 0-based position whose label is t). Returns 0 if tau
 * is a permutation of 1..B, 1 otherwise (inv is then filled with -1 where
 * undefined). */
int simsd_oracle_tau_inverse(const int32_t* tau, int B, int32_t* inv) {
  int bad = 0;
  for (int t = 0; t < B; ++t) inv[t] = -1;
  for (int k = 0; k < B; ++k) {
    int t = tau[k];
    if (t < 1 || t > B || inv[t - 1] != -1) {
      bad = 1;
      continue;
    }
    inv[t - 1] = k;
  }
  return bad;
}

/* The temporal attention mask A_ij between the 2B block rows.
 * Block row numbering: row r < B is the data token D_{r+1}; row r >= B is the
 * mask slot D~_{r-B+1} ([nl]/[fr] Methodologie 1, input layout with a data
 * section and a mask section of length B each).
 *
 * [nl]/[fr] Methodologie 2 (mask logic), for a mask-slot query D~_i:
 *   - it may look at data token D_j exactly when tau(j) < tau(i);
 *   - it may look at mask slot D~_j exactly when tau(j) >= tau(i) (so also at
 *     itself);
 *   - nothing else in the block (data tokens from the current or later steps
 *     stay hidden).
 * For a data-token query D_i the pages give no rule. Reading used here:
 *   DATA_CAUSAL: D_i sees D_j with tau(j) <= tau(i), and no mask slot;
 *   DATA_BIDIR : D_i sees every D_j, and no mask slot.
 * (DATA_SKIP rows are not computed, so they have no mask.)
 * The cached prompt prefix is visible to every block row and is not part of
 * this function. Returns 1 if query row qr may attend to key row kr. */
int simsd_oracle_allowed(int B, const int32_t* tau, int data_rule, int qr, int kr) {
  int q_is_slot = qr >= B, k_is_slot = kr >= B;
  int ti = tau[q_is_slot ? qr - B : qr];
  int tj = tau[k_is_slot ? kr - B : kr];
  if (q_is_slot) {
    if (!k_is_slot) return tj < ti;
    return tj >= ti;
  }
  if (k_is_slot) return 0;
  if (data_rule == ORACLE_DATA_BIDIR) return 1;
  return tj <= ti;
}

/* One query row of verify attention, plain masked softmax attention over the
 * explicit allowed key set (masked keys are excluded: they enter neither the
 * maximum nor the sum).
 *   q      : [d]            the query (block row qr of its sequence, head h)
 *   k_pre  : [P][Hkv][d]    cached prefix keys of this sequence (already rotated)
 *   v_pre  : [P][Hkv][d]
 *   k_blk  : [2B][Hkv][d]   keys of the paired block of this sequence
 *   v_blk  : [2B][Hkv][d]
 *   g      : the KV head this query head reads (grouped-query attention)
 * Writes out[d] and *lse = log(sum_j exp(s_j)) with s_j = scale * <q, k_j>.
 * Key order: prefix positions 0..P-1, then block rows 0..2B-1. */
void simsd_oracle_attention_row(const double* q, const double* k_pre, const double* v_pre, int P,
                                const double* k_blk, const double* v_blk, const int32_t* tau,
                                int B, int Hkv, int d, int g, int qr, double scale, int data_rule,
                                double* out, double* lse) {
  int nkeys = P + 2 * B;
  double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
  char* ok = (char*)malloc((size_t)nkeys);
  double m = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    const double* kj;
    if (j < P) {
      ok[j] = 1; /* the whole cached prefix is visible */
      kj = k_pre + ((size_t)j * Hkv + g) * d;
    } else {
      ok[j] = (char)simsd_oracle_allowed(B, tau, data_rule, qr, j - P);
      kj = k_blk + ((size_t)(j - P) * Hkv + g) * d;
    }
    if (!ok[j]) continue;
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += q[e] * kj[e];
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  double denom = 0.0;
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    if (!ok[j]) continue;
    double w = exp(s[j] - m);
    denom += w;
    const double* vj = j < P ? v_pre + ((size_t)j * Hkv + g) * d
                             : v_blk + ((size_t)(j - P) * Hkv + g) * d;
    for (int e = 0; e < d; ++e) out[e] += w * vj[e];
  }
  for (int e = 0; e < d; ++e) out[e] /= denom;
  *lse = m + log(denom);
  free(s);
  free(ok);
}

/* Verify attention over a batch of sequences ([nl]/[fr] Methodologie 4,
 * verification: one forward over prompt + data section + mask section under
 * the temporal mask; the prompt comes from the KV cache, [nl] Belangrijkste
 * Bijdragen 3 / [fr] Principales Contributions, compatibility with KV cache).
 *   q_blk [b][2B][Hq][d], k_blk/v_blk [b][2B][Hkv][d]
 *   k_pre/v_pre [sum P][Hkv][d] packed, sequence s at rows
 *   prefix_offsets[s] .. prefix_offsets[s+1]-1; tau [b][B] (1-based labels)
 *   out [b][2B][Hq][d], lse [b][2B][Hq]
 * Query head h reads KV head h / (Hq/Hkv). DATA_SKIP leaves data rows of out
 * and lse untouched. Returns the number of sequences whose tau is not a
 * permutation (those are skipped). */
int simsd_oracle_verify_attention(const double* q_blk, const double* k_blk, const double* v_blk,
                                  const double* k_pre, const double* v_pre,
                                  const int32_t* prefix_offsets, const int32_t* tau, int b, int B,
                                  int Hq, int Hkv, int d, double scale, int data_rule, double* out,
                                  double* lse) {
  int G = Hq / Hkv, bad = 0;
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  for (int s = 0; s < b; ++s) {
    const int32_t* ts = tau + (size_t)s * B;
    if (simsd_oracle_tau_inverse(ts, B, inv)) {
      ++bad;
      continue;
    }
    int P = prefix_offsets[s + 1] - prefix_offsets[s];
    const double* kp = k_pre + (size_t)prefix_offsets[s] * Hkv * d;
    const double* vp = v_pre + (size_t)prefix_offsets[s] * Hkv * d;
    const double* kb = k_blk + (size_t)s * 2 * B * Hkv * d;
    const double* vb = v_blk + (size_t)s * 2 * B * Hkv * d;
    for (int r = 0; r < 2 * B; ++r) {
      if (data_rule == ORACLE_DATA_SKIP && r < B) continue;
      for (int h = 0; h < Hq; ++h) {
        size_t row = ((size_t)s * 2 * B + r) * Hq + h;
        simsd_oracle_attention_row(q_blk + row * d, kp, vp, P, kb, vb, ts, B, Hkv, d, h / G, r,
                                   scale, data_rule, out + row * d, lse + row);
      }
    }
  }
  free(inv);
  return bad;
}

/* RoPE with the copy rule ([nl]/[fr] Methodologie 3, position-encoding
 * alignment: each mask slot D~_k takes the RoPE index of its paired data
 * token D_k).
 * Positions: D_k and D~_k (k = 1..B) both sit at start_pos[s] + k - 1, or,
 * when `positions` is given ([b][B]), both at positions[s][k-1] (each pair is
 * one response position, Methodologie 1; a later round of the same block
 * re-verifies the positions still open, wherever they lie). With no_copy set
 * (an ablation the pages report but do not define; only with consecutive
 * positions), D~_k instead sits at start_pos[s] + B + k - 1, i.e. the mask
 * section is numbered after the data section as a plain concatenation would.
 * Rotation (standard rotary embedding, fp64): frequency i = 0..d/2-1 has
 * inv_freq_i = base^(-2i/d) and angle = pos * inv_freq_i. Rotate-half pairs
 * element i with element i + d/2; interleaved pairs 2i with 2i+1. Each pair
 * (x, y) becomes (x cos - y sin, y cos + x sin).
 *   x [b][2B][H][d] rotated in place (used for Q with H = Hq and for K with
 *   H = Hkv). */
void simsd_oracle_rope_copy(double* x, const int32_t* start_pos, const int32_t* positions, int b, int B,
                            int H, int d, double base, int interleaved, int no_copy) {
  int half = d / 2;
  for (int s = 0; s < b; ++s) {
    for (int r = 0; r < 2 * B; ++r) {
      int k = r < B ? r : r - B; /* 0-based response position of this row */
      long pos = positions ? (long)positions[(size_t)s * B + k] : (long)start_pos[s] + k;
      if (no_copy && r >= B) pos += B;
      for (int h = 0; h < H; ++h) {
        double* v = x + (((size_t)s * 2 * B + r) * H + h) * d;
        for (int i = 0; i < half; ++i) {
          double inv_freq = pow(base, -2.0 * i / d);
          double ang = (double)pos * inv_freq;
          double c = cos(ang), sn = sin(ang);
          int a = interleaved ? 2 * i : i;
          int bb = interleaved ? 2 * i + 1 : i + half;
          double xa = v[a], xb = v[bb];
          v[a] = xa * c - xb * sn;
          v[bb] = xb * c + xa * sn;
        }
      }
    }
  }
}

/* Rejection-sampling acceptance along the draft's temporal order
 * ([nl]/[fr] Methodologie 4, acceptance: standard rejection sampling is run
 * in the temporal order the draft induced, and the longest accepted prefix is
 * committed).
 * Inputs per sequence s (positions k = 0..B-1 in natural order):
 *   p [b][B][V] target probabilities at the mask slots, q [b][B][V] draft
 *   probabilities, draft [b][B] draft token ids, tau [b][B] step labels,
 *   u [b][B+1] uniforms in [0,1): u[t-1] decides step t, u[B] the correction.
 * Steps:
 *   1. For t = 1..B: k = tau^-1(t), x = draft[k]; ratio r = min(1, p/q) in
 *      IEEE fp32 (r = 1 if p > 0 = q, r = 0 if p = q = 0; status bit 4).
 *      Step t is accepted iff u_t < r. L = number of leading accepted steps.
 *   2. L == B: nothing to correct (no bonus slot exists), correction = -1.
 *   3. Otherwise k* = tau^-1(L+1); residual rho_y = max(0, p - q) in fp32;
 *      Z = sum_y rho_y in fp64 in index order; T = u_{B+1} * Z; the
 *      correction is the smallest y whose running sum C_y exceeds T (largest
 *      y with rho_y > 0 if rounding leaves none). If Z == 0 the same draw is
 *      made from p[k*] instead and status bit 2 is set.
 * Outputs: accept_len[s], correction[s], status[s] (1: tau not a
 * permutation; 2: Z == 0 fallback; 4: q(x) == 0 met; 8: a draft id outside
 * [0,V)), boundary[s] = 1 when T lies within 1e-6 * Z of the drawn token's
 * CDF interval ends (a differently ordered sum may pick the neighbour).
 * For a bad tau the outputs are accept_len 0, correction -1. */
void simsd_oracle_accept(const float* p, const float* q, const int32_t* draft, const int32_t* tau,
                         const float* u, int b, int B, int V, int32_t* accept_len,
                         int32_t* correction, int32_t* status, int32_t* boundary) {
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  for (int s = 0; s < b; ++s) {
    const float* ps = p + (size_t)s * B * V;
    const float* qs = q + (size_t)s * B * V;
    const float* us = u + (size_t)s * (B + 1);
    status[s] = 0;
    boundary[s] = 0;
    accept_len[s] = 0;
    correction[s] = -1;
    if (simsd_oracle_tau_inverse(tau + (size_t)s * B, B, inv)) {
      status[s] |= 1;
      continue;
    }
    int L = B;
    for (int t = 1; t <= B; ++t) {
      int k = inv[t - 1];
      int x = draft[(size_t)s * B + k];
      float r;
      if (x < 0 || x >= V) {
        status[s] |= 8;
        r = 0.0f;
      } else {
        float a = ps[(size_t)k * V + x], c = qs[(size_t)k * V + x];
        if (c > 0.0f) {
          r = a / c;
          if (r > 1.0f) r = 1.0f;
        } else {
          status[s] |= 4;
          r = a > 0.0f ? 1.0f : 0.0f;
        }
      }
      if (!(us[t - 1] < r)) {
        L = t - 1;
        break;
      }
    }
    accept_len[s] = L;
    if (L == B) continue;
    int kstar = inv[L];
    const float* pk = ps + (size_t)kstar * V;
    const float* qk = qs + (size_t)kstar * V;
    double Z = 0.0;
    for (int y = 0; y < V; ++y) {
      float rho = pk[y] - qk[y];
      if (rho < 0.0f) rho = 0.0f;
      Z += (double)rho;
    }
    int use_p = 0;
    if (!(Z > 0.0)) {
      status[s] |= 2;
      use_p = 1;
      Z = 0.0;
      for (int y = 0; y < V; ++y) Z += (double)(pk[y] > 0.0f ? pk[y] : 0.0f);
      if (!(Z > 0.0)) continue; /* no mass anywhere: correction stays -1 */
    }
    double T = (double)us[B] * Z, C = 0.0, Cprev = 0.0;
    int pick = -1, last_pos = -1;
    for (int y = 0; y < V; ++y) {
      float w;
      if (use_p) {
        w = pk[y] > 0.0f ? pk[y] : 0.0f;
      } else {
        w = pk[y] - qk[y];
        if (w < 0.0f) w = 0.0f;
      }
      if (w > 0.0f) last_pos = y;
      Cprev = C;
      C += (double)w;
      if (pick < 0 && C > T) {
        pick = y;
        if (fabs(T - Cprev) < 1e-6 * Z || fabs(T - C) < 1e-6 * Z) boundary[s] = 1;
        break;
      }
    }
    if (pick < 0) {
      pick = last_pos;
      boundary[s] = 1;
    }
    correction[s] = pick;
  }
  free(inv);
}

/* Softmax of each row of logits at a sampling temperature, the distribution
 * the target (and the draft) assign to each response position from the
 * logits of its verification pass ([nl] Methodologie 4, Verificatie; [fr]
 * Methodologie 4: the single forward pass yields the logits of every
 * candidate). The temperature is this build's reading: the pages sample at
 * temperature but do not define it for SimSD; p = softmax(z / T).
 * Plain definition in fp64: m = max_y z_y (subtracting it changes nothing
 * mathematically), s = sum_y exp((z_y - m) / T) in index order, and each
 * output is exp((z_y - m) / T) / s rounded once to fp32 (the precision the
 * acceptance decisions are taken in). */
void simsd_oracle_softmax_rows(const float* z, int rows, int V, double temperature, float* out) {
  for (int r = 0; r < rows; ++r) {
    const float* zr = z + (size_t)r * V;
    float* o = out + (size_t)r * V;
    double m = -INFINITY;
    for (int y = 0; y < V; ++y)
      if ((double)zr[y] > m) m = (double)zr[y];
    double s = 0.0;
    for (int y = 0; y < V; ++y) s += exp(((double)zr[y] - m) / temperature);
    for (int y = 0; y < V; ++y) o[y] = (float)(exp(((double)zr[y] - m) / temperature) / s);
  }
}

/* Attention of block rows under an explicit block mask instead of the
 * temporal rule: the "next" generalisation the SimSD pages point to for
 * verifying several drafts or a draft graph against one cached prefix
 * (Spiffy page, draft graphs; [nl]/[fr] Methodologie 2 is the special case
 * the tau rule produces). Every row sees the whole cached prefix of its
 * sequence and the block keys c with allowed[s][r][c] != 0; the softmax runs
 * over those keys only (fp64, keys in order prefix 0..P-1 then block rows
 * 0..R-1, exactly as simsd_oracle_attention_row). A row with no visible key
 * (empty prefix and no allowed block key) has out = 0 and lse = -inf.
 *   q_blk [b][R][Hq][d], k_blk/v_blk [b][R][Hkv][d], allowed [b][R][R] bytes,
 *   k_pre/v_pre packed [sum P][Hkv][d] with prefix_offsets[b+1];
 *   out [b][R][Hq][d], lse [b][R][Hq]. */
void simsd_oracle_attention_masked(const double* q_blk, const double* k_blk, const double* v_blk,
                                   const double* k_pre, const double* v_pre,
                                   const int32_t* prefix_offsets, const uint8_t* allowed, int b, int R,
                                   int Hq, int Hkv, int d, double scale, double* out, double* lse) {
  int G = Hq / Hkv;
  for (int s = 0; s < b; ++s) {
    int P = prefix_offsets[s + 1] - prefix_offsets[s];
    const double* kp = k_pre + (size_t)prefix_offsets[s] * Hkv * d;
    const double* vp = v_pre + (size_t)prefix_offsets[s] * Hkv * d;
    const double* kb = k_blk + (size_t)s * R * Hkv * d;
    const double* vb = v_blk + (size_t)s * R * Hkv * d;
    int nkeys = P + R;
    double* sc = (double*)malloc(sizeof(double) * (size_t)nkeys);
    char* ok = (char*)malloc((size_t)nkeys);
    for (int r = 0; r < R; ++r) {
      const uint8_t* arow = allowed + ((size_t)s * R + r) * R;
      for (int h = 0; h < Hq; ++h) {
        size_t row = ((size_t)s * R + r) * Hq + h;
        const double* q = q_blk + row * d;
        int g = h / G;
        double m = -INFINITY;
        for (int j = 0; j < nkeys; ++j) {
          const double* kj;
          if (j < P) {
            ok[j] = 1;
            kj = kp + ((size_t)j * Hkv + g) * d;
          } else {
            ok[j] = (char)(arow[j - P] != 0);
            kj = kb + ((size_t)(j - P) * Hkv + g) * d;
          }
          if (!ok[j]) continue;
          double dot = 0.0;
          for (int e = 0; e < d; ++e) dot += q[e] * kj[e];
          sc[j] = dot * scale;
          if (sc[j] > m) m = sc[j];
        }
        double* o = out + row * d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        if (m == -INFINITY) {
          lse[row] = -INFINITY;
          continue;
        }
        double denom = 0.0;
        for (int j = 0; j < nkeys; ++j) {
          if (!ok[j]) continue;
          double w = exp(sc[j] - m);
          denom += w;
          const double* vj = j < P ? vp + ((size_t)j * Hkv + g) * d : vb + ((size_t)(j - P) * Hkv + g) * d;
          for (int e = 0; e < d; ++e) o[e] += w * vj[e];
        }
        for (int e = 0; e < d; ++e) o[e] /= denom;
        lse[row] = m + log(denom);
      }
    }
    free(sc);
    free(ok);
  }
}
