/*
 * pa_oracle.c — plain, slow, fp64 CPU oracle for paged causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes (sources are the two web pages the method is described
 * on; "Triton deep dive" is "vLLM Triton Attention Backend Deep Dive",
 * "ROCm backends" is "vLLM AMD ROCm Attention Backend Optimization"):
 *
 *   - Paged attention (Triton deep dive, section "Technical implementation of
 *     paged attention"): the KV cache is cut into fixed-size pages; for each
 *     query token and each query head the scores against the cached keys of
 *     the matching KV head are formed by walking the pages.  Paging changes
 *     where a key lives, never what is computed, so the oracle first gathers
 *     the pages of a request into a dense array and then runs textbook
 *     softmax(scale * q k^T) v on it.
 *   - GQA (Triton deep dive, section "Q-block optimization"): several query
 *     heads share one KV head; query head h reads KV head h / (Hq / Hkv).
 *   - Continuous batch of prefill / extend / decode requests (ROCm backends,
 *     section "The challenge of mixed inference workloads"): request b holds
 *     q_b new tokens on top of c_b = L_b - q_b cached ones.  Causality is
 *     aligned to the end of the sequence: new token j sits at position
 *     c_b + j and sees keys 0 .. c_b + j.
 *   - Masks other than causal (Triton deep dive, section on the backend's
 *     use cases: encoder / decoder attention and multimodal prefix
 *     attention, named there without formulas).  ORC_MASK_FULL: every new
 *     token of a request sees all L_b keys (encoder self-attention, or
 *     cross-attention onto a cached encoder output).  ORC_MASK_PREFIX: the
 *     first prefix_lens[b] key positions form a bidirectional prefix, the
 *     rest stays causal; the token at position p sees keys
 *     0 .. max(p, prefix_lens[b] - 1), at most L_b - 1.
 *   - Sink tokens (Triton deep dive, same list of use cases; named there
 *     for GPT-OSS without a formula): a per-query-head logit sinks[h] joins
 *     the softmax of every row of head h as one more key whose value is
 *     zero, so it only adds e^{sinks[h]} to the denominator.
 *   - ALiBi and its square-root variant (Triton deep dive, same list of use
 *     cases: "ALiBi sqrt", used by a StepFun audio model; no formula there).
 *     Reading: ALiBi as published by Press et al. ("Train Short, Test Long",
 *     2022) adds -m_h * (p - t) to the logit of the query at position p and
 *     the key at position t, with a fixed slope m_h per query head; the sqrt
 *     variant adds -m_h * sqrt(p - t).  |p - t| is used, so that keys after
 *     the query (full and prefix masks) are penalised by their distance too.
 *     The slopes are an input (alibi_slopes[Hq]).
 *   - Split-KV partials and their log-sum-exp merge (Triton deep dive,
 *     section "Parallel tiled softmax (3D kernel)"; ROCm backends, bullet
 *     "Chunked context processing"): the key range is cut into contiguous
 *     pieces, each piece yields a normalised partial output and its LSE, and
 *     the pieces are combined with weights exp(lse_s - max lse).
 *   - Absorbed MLA decode (ROCm backends, sections "AITER MLA backend" and
 *     "Hybrid processing strategy"): one shared 576-wide latent row per token
 *     serves as the key (all 576 columns) and as the value (its first 512
 *     columns).
 *
 * All arithmetic is fp64.  Inputs are bf16 or fp32 values; they are widened
 * exactly (a bf16 is the top half of an fp32).  The scale arrives as an fp32
 * and is widened too.
 *
 * Cache layouts (the element at page p, slot s, KV head h, column d):
 *   ORC_LAYOUT_MHA  key  : k[((p * Hkv + h) * P + s) * Dqk + d]
 *                   value: v[((p * Hkv + h) * Dv + d) * P + s]
 *   ORC_LAYOUT_MLA  key  : c[(p * P + s) * Dqk + d]          (Hkv == 1)
 *                   value: c[(p * P + s) * Dqk + d], d < Dv  (same buffer)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_LAYOUT_MHA = 0, ORC_LAYOUT_MLA = 1 };
enum { ORC_MASK_CAUSAL = 0, ORC_MASK_FULL = 1, ORC_MASK_PREFIX = 2 };
enum { ORC_ALIBI_NONE = 0, ORC_ALIBI_LINEAR = 1, ORC_ALIBI_SQRT = 2 };
enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_DATA = 2, ORC_ERR_NOMEM = 3 };

/* Read element idx of an array of the given dtype, widened to double. */
static double load_elem(const void* base, int dtype, size_t idx) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t key_index(int layout, int64_t page, int slot, int head, int d,
                        int Hkv, int P, int Dqk) {
  if (layout == ORC_LAYOUT_MLA) return ((size_t)page * P + slot) * Dqk + d;
  return (((size_t)page * Hkv + head) * P + slot) * Dqk + d;
}

static size_t value_index(int layout, int64_t page, int slot, int head, int d,
                          int Hkv, int P, int Dqk, int Dv) {
  if (layout == ORC_LAYOUT_MLA) return ((size_t)page * P + slot) * Dqk + d;
  return (((size_t)page * Hkv + head) * Dv + d) * P + slot;
}

/*
 * Dense gather of keys [0, n) of request b, KV head h, into Kd[n][Dqk] and
 * Vd[n][Dv].  Token t lives in logical page t / P at slot t % P; the block
 * table row of the request maps the logical page to a physical one.
 * Returns ORC_ERR_DATA if a needed table entry is outside [0, num_pages).
 */
static int gather(const void* kc, const void* vc, int dtype, int layout,
                  const int32_t* bt_row, int num_pages, int n, int h, int Hkv,
                  int P, int Dqk, int Dv, double* Kd, double* Vd) {
  for (int t = 0; t < n; ++t) {
    int64_t page = bt_row[t / P];
    int slot = t % P;
    if (page < 0 || page >= num_pages) return ORC_ERR_DATA;
    for (int d = 0; d < Dqk; ++d)
      Kd[(size_t)t * Dqk + d] =
          load_elem(kc, dtype, key_index(layout, page, slot, h, d, Hkv, P, Dqk));
    for (int d = 0; d < Dv; ++d)
      Vd[(size_t)t * Dv + d] = load_elem(
          vc, dtype, value_index(layout, page, slot, h, d, Hkv, P, Dqk, Dv));
  }
  return ORC_OK;
}

/*
 * ALiBi bias of the key at position t for the query at position pos:
 * -slope * |pos - t| (linear) or -slope * sqrt(|pos - t|) (sqrt); 0 without.
 */
static double alibi_bias(int mode, double slope, int pos, int t) {
  const double dist = fabs((double)pos - (double)t);
  if (mode == ORC_ALIBI_LINEAR) return -slope * dist;
  if (mode == ORC_ALIBI_SQRT) return -slope * sqrt(dist);
  return 0.0;
}

/*
 * Textbook attention of one query row over dense keys [t0, t1):
 *   s_t = sigma * q . k_t + bias_t,  m = max s_t,  l = sum exp(s_t - m),
 *   out = sum exp(s_t - m) v_t / l,  lse = m + ln l,
 * with bias_t = alibi_bias(alibi_mode, slope, pos, t).
 * An empty range gives out = 0 and lse = -inf.  `s` is scratch of size t1.
 */
static void attend_biased(const double* qrow, const double* Kd, const double* Vd,
                          int t0, int t1, int Dqk, int Dv, double sigma,
                          int alibi_mode, double slope, int pos, double* s,
                          double* out, double* lse) {
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  if (t1 <= t0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int t = t0; t < t1; ++t) {
    double dot = 0.0;
    for (int d = 0; d < Dqk; ++d) dot += qrow[d] * Kd[(size_t)t * Dqk + d];
    s[t] = sigma * dot + alibi_bias(alibi_mode, slope, pos, t);
    if (s[t] > m) m = s[t];
  }
  double l = 0.0;
  for (int t = t0; t < t1; ++t) {
    double w = exp(s[t] - m);
    l += w;
    for (int d = 0; d < Dv; ++d) out[d] += w * Vd[(size_t)t * Dv + d];
  }
  for (int d = 0; d < Dv; ++d) out[d] /= l;
  *lse = m + log(l);
}

/* attend_biased without a bias. */
static void attend(const double* qrow, const double* Kd, const double* Vd,
                   int t0, int t1, int Dqk, int Dv, double sigma, double* s,
                   double* out, double* lse) {
  attend_biased(qrow, Kd, Vd, t0, t1, Dqk, Dv, sigma, ORC_ALIBI_NONE, 0.0, 0, s, out, lse);
}

static int check_common(int B, int Hq, int Hkv, int Dqk, int Dv, int P,
                        int max_pages, int layout) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Dqk <= 0 || Dv <= 0 || P <= 0 ||
      max_pages < 0)
    return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_ARG;
  if (layout != ORC_LAYOUT_MHA && layout != ORC_LAYOUT_MLA) return ORC_ERR_ARG;
  if (layout == ORC_LAYOUT_MLA && (Hkv != 1 || Dv > Dqk)) return ORC_ERR_ARG;
  return ORC_OK;
}

/*
 * Paged attention over a varlen continuous batch, causal or with one of the
 * other masks above (mask; prefix_lens [B] is read for ORC_MASK_PREFIX only),
 * with optional sink logits (sinks [Hq] or NULL) and an optional ALiBi bias
 * (alibi_mode ORC_ALIBI_LINEAR / ORC_ALIBI_SQRT with alibi_slopes [Hq]).
 *   q        [T, Hq, Dqk] (dtype), T = qsl[B]
 *   out      [T, Hq, Dv] double;  lse [T, Hq] double (may be NULL)
 *   row_sel  optional [T * Hq] bytes; when given, only rows with a nonzero
 *            byte are computed (the others are left untouched).
 * Returns ORC_OK, ORC_ERR_ARG (bad sizes) or ORC_ERR_DATA (a request with
 * seq_len < q_len, a negative count, or a table entry out of range).
 */
int orc_attention_masked(const void* q, const void* kc, const void* vc, int dtype,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* qsl, int B, int Hq, int Hkv, int Dqk, int Dv,
                         int P, int num_pages, int max_pages, int layout, float scale,
                         int mask, const int32_t* prefix_lens, const float* sinks,
                         const float* alibi_slopes, int alibi_mode,
                         const uint8_t* row_sel, double* out, double* lse,
                         int nthreads) {
  int rc = check_common(B, Hq, Hkv, Dqk, Dv, P, max_pages, layout);
  if (rc) return rc;
  if (mask != ORC_MASK_CAUSAL && mask != ORC_MASK_FULL && mask != ORC_MASK_PREFIX)
    return ORC_ERR_ARG;
  if (mask == ORC_MASK_PREFIX && !prefix_lens) return ORC_ERR_ARG;
  if (alibi_mode != ORC_ALIBI_NONE && alibi_mode != ORC_ALIBI_LINEAR &&
      alibi_mode != ORC_ALIBI_SQRT)
    return ORC_ERR_ARG;
  if (alibi_mode != ORC_ALIBI_NONE && !alibi_slopes) return ORC_ERR_ARG;
  const int g = Hq / Hkv;
  const double sigma = (double)scale;
  int err = ORC_OK;
  if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t job = 0; job < (int64_t)B * Hkv; ++job) {
    const int b = (int)(job / Hkv), h = (int)(job % Hkv);
    const int i0 = qsl[b], nq = qsl[b + 1] - qsl[b], L = seq_lens[b];
    if (nq <= 0) {
      if (nq < 0) {
#pragma omp atomic write
        err = ORC_ERR_DATA;
      }
      continue;
    }
    if (L < nq || (L + P - 1) / P > max_pages) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
      continue;
    }
    int any = 1;
    if (row_sel) {
      any = 0;
      for (int j = 0; j < nq && !any; ++j)
        for (int hh = h * g; hh < (h + 1) * g; ++hh)
          if (row_sel[(size_t)(i0 + j) * Hq + hh]) any = 1;
    }
    if (!any) continue;
    const int c = L - nq;
    double* Kd = malloc(sizeof(double) * (size_t)L * Dqk);
    double* Vd = malloc(sizeof(double) * (size_t)L * Dv);
    double* qrow = malloc(sizeof(double) * (size_t)Dqk);
    double* s = malloc(sizeof(double) * (size_t)L);
    if (!Kd || !Vd || !qrow || !s) {
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      free(Kd); free(Vd); free(qrow); free(s);
      continue;
    }
    if (gather(kc, vc, dtype, layout, block_table + (size_t)b * max_pages,
               num_pages, L, h, Hkv, P, Dqk, Dv, Kd, Vd)) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
    } else {
      for (int j = 0; j < nq; ++j) {
        const int i = i0 + j, pos = c + j;
        for (int hh = h * g; hh < (h + 1) * g; ++hh) {
          if (row_sel && !row_sel[(size_t)i * Hq + hh]) continue;
          for (int d = 0; d < Dqk; ++d)
            qrow[d] = load_elem(q, dtype, ((size_t)i * Hq + hh) * Dqk + d);
          /* keys [0, end) are visible: causal end = pos + 1 */
          int end = pos + 1;
          if (mask == ORC_MASK_FULL) end = L;
          if (mask == ORC_MASK_PREFIX && prefix_lens[b] > end)
            end = prefix_lens[b] < L ? prefix_lens[b] : L;
          double l_out;
          attend_biased(qrow, Kd, Vd, 0, end, Dqk, Dv, sigma, alibi_mode,
                        alibi_mode ? (double)alibi_slopes[hh] : 0.0, pos, s,
                        out + ((size_t)i * Hq + hh) * Dv, &l_out);
          if (sinks) {
            /* one more logit, sinks[hh], with a zero value: the row's weights
               shrink by e^{lse} / (e^{lse} + e^{sink}) */
            const double sk = (double)sinks[hh];
            const double mx = l_out > sk ? l_out : sk;
            if (mx > -INFINITY) {
              const double wr = exp(l_out - mx), ws = exp(sk - mx);
              double* o = out + ((size_t)i * Hq + hh) * Dv;
              for (int d = 0; d < Dv; ++d) o[d] *= wr / (wr + ws);
              l_out = mx + log(wr + ws);
            }
          }
          if (lse) lse[(size_t)i * Hq + hh] = l_out;
        }
      }
    }
    free(Kd); free(Vd); free(qrow); free(s);
  }
  return err;
}

/* Causal paged attention (orc_attention_masked with ORC_MASK_CAUSAL). */
int orc_attention(const void* q, const void* kc, const void* vc, int dtype,
                  const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* qsl, int B, int Hq, int Hkv, int Dqk, int Dv,
                  int P, int num_pages, int max_pages, int layout, float scale,
                  const uint8_t* row_sel, double* out, double* lse,
                  int nthreads) {
  return orc_attention_masked(q, kc, vc, dtype, block_table, seq_lens, qsl, B,
                              Hq, Hkv, Dqk, Dv, P, num_pages, max_pages,
                              layout, scale, ORC_MASK_CAUSAL, NULL, NULL, NULL,
                              ORC_ALIBI_NONE, row_sel, out, lse, nthreads);
}

/*
 * Key range of partition s out of S for a sequence of L keys: contiguous,
 * page aligned, T_s = P * ceil(ceil(L / P) / S) keys each, the last ones
 * possibly short or empty.
 */
void orc_split_range(int L, int P, int S, int s, int* t0, int* t1) {
  int pages = (L + P - 1) / P;
  int per = P * ((pages + S - 1) / S);
  long a = (long)s * per, e = a + per;
  if (a > L) a = L;
  if (e > L) e = L;
  *t0 = (int)a;
  *t1 = (int)e;
}

/*
 * Split-KV decode partials: every request has exactly one query token
 * (q is [B, Hq, Dqk]); partition s of request b gives the normalised partial
 * part_out[b, h, s, :] and its LSE part_lse[b, h, s] (-inf and zeros when
 * the partition is empty).
 */
int orc_decode_split(const void* q, const void* kc, const void* vc, int dtype,
                     const int32_t* block_table, const int32_t* seq_lens,
                     int B, int Hq, int Hkv, int Dqk, int Dv, int P,
                     int num_pages, int max_pages, int layout, float scale,
                     int S, double* part_out, double* part_lse, int nthreads) {
  int rc = check_common(B, Hq, Hkv, Dqk, Dv, P, max_pages, layout);
  if (rc) return rc;
  if (S <= 0) return ORC_ERR_ARG;
  const int g = Hq / Hkv;
  const double sigma = (double)scale;
  int err = ORC_OK;
  if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t job = 0; job < (int64_t)B * Hkv; ++job) {
    const int b = (int)(job / Hkv), h = (int)(job % Hkv);
    const int L = seq_lens[b];
    if (L < 1 || (L + P - 1) / P > max_pages) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
      continue;
    }
    double* Kd = malloc(sizeof(double) * (size_t)L * Dqk);
    double* Vd = malloc(sizeof(double) * (size_t)L * Dv);
    double* qrow = malloc(sizeof(double) * (size_t)Dqk);
    double* s = malloc(sizeof(double) * (size_t)L);
    if (!Kd || !Vd || !qrow || !s) {
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      free(Kd); free(Vd); free(qrow); free(s);
      continue;
    }
    if (gather(kc, vc, dtype, layout, block_table + (size_t)b * max_pages,
               num_pages, L, h, Hkv, P, Dqk, Dv, Kd, Vd)) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
    } else {
      for (int hh = h * g; hh < (h + 1) * g; ++hh) {
        for (int d = 0; d < Dqk; ++d)
          qrow[d] = load_elem(q, dtype, ((size_t)b * Hq + hh) * Dqk + d);
        for (int sp = 0; sp < S; ++sp) {
          int t0, t1;
          orc_split_range(L, P, S, sp, &t0, &t1);
          size_t row = ((size_t)b * Hq + hh) * S + sp;
          attend(qrow, Kd, Vd, t0, t1, Dqk, Dv, sigma, s, part_out + row * Dv,
                 part_lse + row);
        }
      }
    }
    free(Kd); free(Vd); free(qrow); free(s);
  }
  return err;
}

/*
 * Chunked-context partials (ROCm backends, bullet "Chunked context
 * processing": the context is processed a fixed number of keys at a time and
 * the pieces are combined by their log-sum-exp).  The keys of every request
 * are cut into chunks of C keys, chunk s covering [s C, (s + 1) C).  For new
 * token j of request b (position c_b + j, as in orc_attention) and query head
 * h, part_out[i, h, s, :] and part_lse[i, h, s] (i = qsl[b] + j) are plain
 * attention over the keys of chunk s that the token sees:
 *   [s C, min((s + 1) C, c_b + j + 1)).
 * A chunk holding none of them gives zeros and -inf, so orc_merge_lse over
 * the S chunks of a row gives that row of orc_attention.  With mask /
 * prefix_lens (as in orc_attention_masked) a token sees the chunk's keys
 * below its visible end instead.
 *   part_out [T, Hq, S, Dv], part_lse [T, Hq, S], both double.
 */
int orc_chunked_partials_masked(const void* q, const void* kc, const void* vc,
                                int dtype, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* qsl, int B,
                                int Hq, int Hkv, int Dqk, int Dv, int P, int num_pages,
                                int max_pages, int layout, float scale, int C, int S,
                                int mask, const int32_t* prefix_lens,
                                double* part_out, double* part_lse, int nthreads) {
  int rc = check_common(B, Hq, Hkv, Dqk, Dv, P, max_pages, layout);
  if (rc) return rc;
  if (C <= 0 || S <= 0) return ORC_ERR_ARG;
  if (mask != ORC_MASK_CAUSAL && mask != ORC_MASK_FULL && mask != ORC_MASK_PREFIX)
    return ORC_ERR_ARG;
  if (mask == ORC_MASK_PREFIX && !prefix_lens) return ORC_ERR_ARG;
  const int g = Hq / Hkv;
  const double sigma = (double)scale;
  int err = ORC_OK;
  if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t job = 0; job < (int64_t)B * Hkv; ++job) {
    const int b = (int)(job / Hkv), h = (int)(job % Hkv);
    const int i0 = qsl[b], nq = qsl[b + 1] - qsl[b], L = seq_lens[b];
    if (nq <= 0) {
      if (nq < 0) {
#pragma omp atomic write
        err = ORC_ERR_DATA;
      }
      continue;
    }
    if (L < nq || (L + P - 1) / P > max_pages) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
      continue;
    }
    const int c = L - nq;
    double* Kd = malloc(sizeof(double) * (size_t)L * Dqk);
    double* Vd = malloc(sizeof(double) * (size_t)L * Dv);
    double* qrow = malloc(sizeof(double) * (size_t)Dqk);
    double* s = malloc(sizeof(double) * (size_t)L);
    if (!Kd || !Vd || !qrow || !s) {
#pragma omp atomic write
      err = ORC_ERR_NOMEM;
      free(Kd); free(Vd); free(qrow); free(s);
      continue;
    }
    if (gather(kc, vc, dtype, layout, block_table + (size_t)b * max_pages,
               num_pages, L, h, Hkv, P, Dqk, Dv, Kd, Vd)) {
#pragma omp atomic write
      err = ORC_ERR_DATA;
    } else {
      for (int j = 0; j < nq; ++j) {
        const int i = i0 + j;
        long seen = (long)c + j + 1;  /* keys 0 .. c + j under the causal mask */
        if (mask == ORC_MASK_FULL) seen = L;
        if (mask == ORC_MASK_PREFIX && prefix_lens[b] > seen)
          seen = prefix_lens[b] < L ? prefix_lens[b] : L;
        for (int hh = h * g; hh < (h + 1) * g; ++hh) {
          for (int d = 0; d < Dqk; ++d)
            qrow[d] = load_elem(q, dtype, ((size_t)i * Hq + hh) * Dqk + d);
          for (int sp = 0; sp < S; ++sp) {
            long t0 = (long)sp * C, t1 = t0 + C;
            if (t1 > seen) t1 = seen;
            if (t0 > t1) t0 = t1;
            size_t row = ((size_t)i * Hq + hh) * S + sp;
            attend(qrow, Kd, Vd, (int)t0, (int)t1, Dqk, Dv, sigma, s,
                   part_out + row * Dv, part_lse + row);
          }
        }
      }
    }
    free(Kd); free(Vd); free(qrow); free(s);
  }
  return err;
}

/* Causal chunk partials (orc_chunked_partials_masked with ORC_MASK_CAUSAL). */
int orc_chunked_partials(const void* q, const void* kc, const void* vc, int dtype,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* qsl, int B, int Hq, int Hkv, int Dqk,
                         int Dv, int P, int num_pages, int max_pages, int layout,
                         float scale, int C, int S, double* part_out,
                         double* part_lse, int nthreads) {
  return orc_chunked_partials_masked(q, kc, vc, dtype, block_table, seq_lens, qsl,
                                     B, Hq, Hkv, Dqk, Dv, P, num_pages, max_pages,
                                     layout, scale, C, S, ORC_MASK_CAUSAL, NULL,
                                     part_out, part_lse, nthreads);
}

/*
 * Log-sum-exp merge of S partials per row (rows are independent):
 *   M = max_s lse_s;  w_s = exp(lse_s - M) (0 when lse_s = -inf);
 *   out = sum w_s o_s / sum w_s;  lse = M + ln sum w_s.
 * A row whose partials are all empty gives out = 0 and lse = -inf.
 * part_out [rows, S, Dv], part_lse [rows, S]; lse may be NULL.
 */
int orc_merge_lse(const double* part_out, const double* part_lse, int rows,
                  int S, int Dv, double* out, double* lse) {
  if (rows < 0 || S <= 0 || Dv <= 0) return ORC_ERR_ARG;
  for (int r = 0; r < rows; ++r) {
    const double* ls = part_lse + (size_t)r * S;
    const double* os = part_out + (size_t)r * S * Dv;
    double* o = out + (size_t)r * Dv;
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (ls[s] > M) M = ls[s];
    for (int d = 0; d < Dv; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      if (lse) lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int s = 0; s < S; ++s) {
      if (ls[s] == -INFINITY) continue;
      double w = exp(ls[s] - M);
      wsum += w;
      for (int d = 0; d < Dv; ++d) o[d] += w * os[(size_t)s * Dv + d];
    }
    for (int d = 0; d < Dv; ++d) o[d] /= wsum;
    if (lse) lse[r] = M + log(wsum);
  }
  return ORC_OK;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
