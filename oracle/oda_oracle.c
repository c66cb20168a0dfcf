/*
 * oda_oracle.c -- CPU fp64 oracle for the On-Demand Attention (ODA) decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the HIP path is checked against.  Only tests/, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or helper with the HIP library; neither includes or
 * links the other.
 *
 * What it follows (page "On-Demand Attention ... summary" on picx.dev):
 *   - section "Local-First Decoding", the access-set equation:
 *       S^F_t = {1..t},  S^L_t = {1..min(s,t)} U {max(1,t-w+1)..t}
 *   - same section, the Local pass and recall score, and the gate: if the
 *     recall score exceeds theta the step is recomputed with Full, otherwise
 *     the Local result is accepted (theta = 0 by default);
 *   - section "Computational Savings", the per-step savings
 *       dF(n,rho) = (1-rho) F_Full(n) - F_Local - F_Recall.
 * Hybrid layers and the focus region follow the Declarative Attention pages
 * (zhichai.net and kongchang.com, "Three Attention Modes"): a focus read covers
 * one contiguous region of the cache; sliding-window layers keep a fixed
 * recent window in both access modes.
 *
 * FP8 KV: quantising the stored cache is the complementary technique of the
 * kongchang.com page, section "The KV Cache Compression Technology Ecosystem".
 * K/V may be FP8 E4M3 codes (the OCP OFP8 encoding) with one dequantisation
 * scale per tensor; the queries stay bf16.
 *
 * Arithmetic: every value (bf16, fp32 or E4M3 input) is widened exactly to double;
 * dot products, exp and log are plain fp64 libm calls.  Attention is the
 * textbook softmax: z_p = scale * <q, K_p>, m = max z, Z = sum exp(z - m),
 * O = sum (exp(z_p - m)/Z) V_p, lse = m + log Z.  No splitting, blocking or
 * reordering; OpenMP only distributes independent (layer, request, head)
 * outputs over threads.
 *
 * Parity-pinned by tests/test_oracle_pins.py (brute-force sets, closed forms,
 * torch scaled_dot_product_attention in float64, special cases, hand-worked
 * fixtures in tests/golden/, the E4M3 code table against torch.float8_e4m3fn).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_F32 = 1, OR_FP8 = 2 };
enum { OR_GATED = 0, OR_SLIDING = 1 };
enum { OR_LOCAL = 0, OR_FULL = 1 };
enum { OR_ACCT_STEPS = 0, OR_ACCT_FULL_CALLS, OR_ACCT_F_LOCAL, OR_ACCT_F_FULL_TAKEN,
       OR_ACCT_F_FULL_ALWAYS, OR_ACCT_DELTA_F, OR_ACCT_KV_BYTES, OR_ACCT_F_RECALL,
       OR_ACCT_N };

typedef struct {
  int32_t num_layers, num_q_heads, num_kv_heads, head_dim;
  int32_t sink, window;        /* s, w of gated layers                          */
  int32_t sw_window;           /* window of sliding-window layers (no sinks)     */
  int32_t dtype;               /* K/V: OR_BF16 (16-bit words), OR_F32, or OR_FP8
                                  (e4m3 bytes; queries are then bf16 words)      */
  int32_t focus;               /* 0: a fired gated layer reads S^F_t;
                                  1: it reads S^L_t U [a, b)                     */
  int32_t pad_;
  double  scale;               /* softmax scale; 0 means 1/sqrt(head_dim)        */
  int64_t recall_flops;        /* F_Recall charged per request per step          */
  double  k_scale, v_scale;    /* dequantisation: K = k_scale * code value, V likewise;
                                  0 means 1                                       */
  const uint8_t* layer_kind;   /* [num_layers], OR_GATED / OR_SLIDING; NULL: all gated */
} oracle_cfg;

/* FP8 E4M3 (the "fn" variant: no infinities): sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals m/8 * 2^-6;
 * exponent 15 with mantissa 7 is NaN; every other code is (1 + m/8) * 2^(e-7). */
double oracle_fp8_e4m3(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

static double widen(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == OR_F32) return (double)((const float*)base)[idx];
  if (dtype == OR_FP8) return oracle_fp8_e4m3(((const uint8_t*)base)[idx]);
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Queries are bf16 when K/V are FP8. */
static int32_t q_dtype(int32_t dtype) { return dtype == OR_FP8 ? OR_BF16 : dtype; }

static int64_t esize(int32_t dtype) { return dtype == OR_F32 ? 4 : (dtype == OR_FP8 ? 1 : 2); }

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

static int layer_kind(const oracle_cfg* c, int32_t l) {
  return c->layer_kind ? c->layer_kind[l] : OR_GATED;
}

/* Membership of position p (1-based) in the access set used at decode
 * position t.  Gated layers: the equation of "Local-First Decoding" written
 * as two closed ranges; Full is {1..t}; the focus variant adds [fa, fb).
 * Sliding-window layers: {max(1, t-W+1)..t} in both modes. */
int oracle_in_set(const oracle_cfg* c, int32_t kind, int32_t mode, int64_t t, int64_t p,
                  int64_t fa, int64_t fb) {
  if (kind == OR_SLIDING) {
    return p >= max64(1, t - c->sw_window + 1) && p <= t;
  }
  int in_sink = p >= 1 && p <= min64(c->sink, t);
  int in_window = p >= max64(1, t - c->window + 1) && p <= t;
  int local = in_sink || in_window;
  if (mode == OR_LOCAL) return local;
  if (c->focus) return local || (p >= fa && p < fb && p >= 1 && p <= t);
  return p >= 1 && p <= t;
}

/* Enumerates the access set by testing every position 1..t; writes the
 * members in ascending order to out (may be NULL) and returns their number. */
int64_t oracle_access_set(const oracle_cfg* c, int32_t kind, int32_t mode, int64_t t,
                          int64_t fa, int64_t fb, int64_t* out) {
  int64_t n = 0;
  for (int64_t p = 1; p <= t; ++p) {
    if (oracle_in_set(c, kind, mode, t, p, fa, fb)) {
      if (out) out[n] = p;
      ++n;
    }
  }
  return n;
}

/* Softmax attention of one query vector over the positions pos[0..n).
 *   q   : head_dim values (dtype)
 *   kv_k, kv_v : one request's sequence, rows [T][num_kv_heads][head_dim];
 *                position p lives in row p-1
 *   g   : the KV head this query head reads
 *   z   : caller scratch of n doubles
 * Writes out[head_dim] and returns lse = m + log Z. */
double oracle_attention(const void* q, const void* kv_k, const void* kv_v, int32_t num_kv_heads,
                        int32_t head_dim, int32_t g, int32_t dtype, double scale, double k_scale,
                        double v_scale, const int64_t* pos, int64_t n, double* out, double* z) {
  const int64_t d = head_dim;
  const int32_t qt = q_dtype(dtype);
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t row = ((pos[i] - 1) * num_kv_heads + g) * d;
    double dot = 0.0;
    for (int64_t j = 0; j < d; ++j) dot += widen(q, qt, j) * (k_scale * widen(kv_k, dtype, row + j));
    z[i] = scale * dot;
    if (z[i] > m) m = z[i];
  }
  double Z = 0.0;
  for (int64_t i = 0; i < n; ++i) Z += exp(z[i] - m);
  for (int64_t j = 0; j < d; ++j) out[j] = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double wgt = exp(z[i] - m) / Z;
    const int64_t row = ((pos[i] - 1) * num_kv_heads + g) * d;
    for (int64_t j = 0; j < d; ++j) out[j] += wgt * (v_scale * widen(kv_v, dtype, row + j));
  }
  return m + log(Z);
}

/* The gate of "Local-First Decoding": Full iff the recall score exceeds theta.
 * Both are fp32 inputs compared exactly in double; NaN compares false. */
int oracle_gate(float score, float theta) { return (double)score > (double)theta; }

/* Per-step accounting for one request, following "Computational Savings":
 *   n_L(l), n_F(l) are the sizes of the Local and Full access sets of layer l;
 *   F_Local = sum_l 4*Hq*d*n_L(l), F_Full = sum_l 4*Hq*d*n_F(l)
 *   (a multiply-add is 2 FLOPs, and both q.K and p.V are contractions over
 *   head_dim for each attended position and query head);
 *   dF = (1-a) F_Full - F_Local - F_Recall;
 *   KV bytes = sum_l Hkv*d*2*esize*(n_L(l) + a*n_F(l)).
 * Set sizes are counted by enumeration, not by formula. */
void oracle_step_accounting(const oracle_cfg* c, int64_t t, int32_t fired, int64_t fa, int64_t fb,
                            int64_t* acct) {
  const int64_t per_pos = 4LL * c->num_q_heads * c->head_dim;
  const int64_t bytes_per_pos = (int64_t)c->num_kv_heads * c->head_dim * 2 * esize(c->dtype);
  int64_t f_local = 0, f_full = 0, bytes = 0;
  for (int32_t l = 0; l < c->num_layers; ++l) {
    const int32_t kind = layer_kind(c, l);
    const int64_t nl = oracle_access_set(c, kind, OR_LOCAL, t, fa, fb, NULL);
    const int64_t nf = oracle_access_set(c, kind, OR_FULL, t, fa, fb, NULL);
    f_local += per_pos * nl;
    f_full += per_pos * nf;
    bytes += bytes_per_pos * (nl + (fired ? nf : 0));
  }
  acct[OR_ACCT_STEPS] += 1;
  acct[OR_ACCT_FULL_CALLS] += fired ? 1 : 0;
  acct[OR_ACCT_F_LOCAL] += f_local;
  acct[OR_ACCT_F_FULL_TAKEN] += fired ? f_full : 0;
  acct[OR_ACCT_F_FULL_ALWAYS] += f_full;
  acct[OR_ACCT_DELTA_F] += (fired ? 0 : f_full) - f_local - c->recall_flops;
  acct[OR_ACCT_KV_BYTES] += bytes;
  acct[OR_ACCT_F_RECALL] += c->recall_flops;
}

/*
 * A whole decode run, step by step, as the "Local-First Decoding" section
 * describes it: at every step each active request attends its Local set in
 * every layer; the gate then decides per request; a fired request recomputes
 * every layer over its Full set and that result is accepted, otherwise the
 * Local result is accepted.  The new token's K/V are part of the sequence
 * arrays (position t = prefill_b + k at step k = 1..K), so "commit" is that
 * position becoming visible to later steps.
 *
 *   kseq, vseq : [L][B][T][Hkv][d]   (T rows per request; rows >= prefill_b + K unused)
 *   q_local    : [K][L][B][Hq][d] (bf16 words when K/V are FP8); q_full: same shape,
 *                NULL = reuse q_local
 *   score      : [K][B] fp32;        focus: [B][2] (a, b) or NULL
 *   active     : [B] or NULL (all active); inactive requests are skipped
 * Outputs (any may be NULL except out):
 *   out [K][L][B][Hq][d] double, lse [K][L][B][Hq], fire [K][B],
 *   call_list [K][B] (ascending, padded with -1), call_count [K],
 *   full_calls [B] (accumulated), acct [B][OR_ACCT_N] (accumulated).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_decode_run(const oracle_cfg* c, int32_t B, int32_t K, const int64_t* prefill, int64_t T,
                      const void* kseq, const void* vseq, const void* q_local, const void* q_full,
                      const float* score, float theta, const int64_t* focus, const uint8_t* active,
                      double* out, double* lse, uint8_t* fire, int32_t* call_list,
                      int32_t* call_count, int64_t* full_calls, int64_t* acct) {
  const int32_t L = c->num_layers, Hq = c->num_q_heads, Hkv = c->num_kv_heads, d = c->head_dim;
  if (L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0 || B < 0 || K < 0 || !out) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (prefill[b] < 0 || prefill[b] + K > T) return -1;
  const double scale = c->scale > 0.0 ? c->scale : 1.0 / sqrt((double)d);
  const double ks = c->k_scale > 0.0 ? c->k_scale : 1.0, vs = c->v_scale > 0.0 ? c->v_scale : 1.0;
  const int32_t group = Hq / Hkv;
  const int64_t es = esize(c->dtype), qes = esize(q_dtype(c->dtype));
  const int64_t seq_stride = T * Hkv * d;  /* elements per (layer, request) sequence */
  const void* qf_base = q_full ? q_full : q_local;
  uint8_t* fired = (uint8_t*)calloc((size_t)(B > 0 ? B : 1), 1);
  if (!fired) return -1;

  for (int32_t k = 1; k <= K; ++k) {
    /* The gate needs only the step's scores; deciding it first does not
     * change what either pass reads. */
    int32_t count = 0;
    for (int32_t b = 0; b < B; ++b) {
      const int is_active = active ? active[b] != 0 : 1;
      fired[b] = is_active && oracle_gate(score[(int64_t)(k - 1) * B + b], theta);
      if (fire) fire[(int64_t)(k - 1) * B + b] = fired[b];
      if (call_list) call_list[(int64_t)(k - 1) * B + b] = -1;
    }
    for (int32_t b = 0; b < B; ++b) {
      if (fired[b]) {
        if (call_list) call_list[(int64_t)(k - 1) * B + count] = b;
        ++count;
      }
    }
    if (call_count) call_count[k - 1] = count;

#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int32_t l = 0; l < L; ++l) {
      for (int32_t b = 0; b < B; ++b) {
        for (int32_t h = 0; h < Hq; ++h) {
          if (active && !active[b]) continue;
          const int64_t t = prefill[b] + k;
          const int32_t kind = layer_kind(c, l);
          const int64_t fa = focus ? focus[2 * b] : 0, fb = focus ? focus[2 * b + 1] : 0;
          int64_t* pos = (int64_t*)malloc((size_t)t * sizeof(int64_t));
          double* z = (double*)malloc((size_t)t * sizeof(double));
          const char* kb = (const char*)kseq + ((int64_t)l * B + b) * seq_stride * es;
          const char* vb = (const char*)vseq + ((int64_t)l * B + b) * seq_stride * es;
          const int64_t qoff = ((((int64_t)(k - 1) * L + l) * B + b) * Hq + h) * d;
          const int64_t ooff = qoff;
          const int64_t loff = (((int64_t)(k - 1) * L + l) * B + b) * Hq + h;
          const int32_t mode = fired[b] ? OR_FULL : OR_LOCAL;
          const void* qb = (const char*)(fired[b] ? qf_base : q_local) + qoff * qes;
          /* The Local attempt is always computed; a fired request then
           * recomputes over its Full set and that result is the one kept. */
          const int64_t nl = oracle_access_set(c, kind, OR_LOCAL, t, fa, fb, pos);
          double l_lse = oracle_attention((const char*)q_local + qoff * qes, kb, vb, Hkv, d,
                                          h / group, c->dtype, scale, ks, vs, pos, nl, out + ooff, z);
          if (mode == OR_FULL) {
            const int64_t nf = oracle_access_set(c, kind, OR_FULL, t, fa, fb, pos);
            l_lse = oracle_attention(qb, kb, vb, Hkv, d, h / group, c->dtype, scale, ks, vs, pos, nf,
                                     out + ooff, z);
          }
          if (lse) lse[loff] = l_lse;
          free(pos);
          free(z);
        }
      }
    }

    for (int32_t b = 0; b < B; ++b) {
      if (active && !active[b]) continue;
      if (full_calls) full_calls[b] += fired[b];
      if (acct) {
        const int64_t fa = focus ? focus[2 * b] : 0, fb = focus ? focus[2 * b + 1] : 0;
        oracle_step_accounting(c, prefill[b] + k, fired[b], fa, fb, acct + (int64_t)b * OR_ACCT_N);
      }
    }
  }
  free(fired);
  return 0;
}

/* Recall score of the recall head, q_t = R_psi(h_{t-1}, E(x_t), h^L_t) of
 * "Local-First Decoding" (picx.dev summary).  The pages fix the inputs and the
 * size of R_psi but not its layers; the stand-in is one hidden layer with
 * ReLU: x = [h_{t-1}; E(x_t); h^L_t] (in_dim values), u = W1 x + b1
 * (hidden values), q = w2 . max(u, 0) + b2.
 *   w1 : bf16 words [hidden][in_dim];  b1, w2 : f32 [hidden];  b2 : f32
 *   x  : bf16 words [batch][in_dim];   q  : double [batch]
 * Plain fp64 loops; OpenMP only over independent requests. */
void oracle_recall_head(int32_t in_dim, int32_t hidden, const uint16_t* w1, const float* b1,
                        const float* w2, float b2, const uint16_t* x, int32_t batch, double* q) {
#pragma omp parallel for schedule(static)
  for (int32_t b = 0; b < batch; ++b) {
    const uint16_t* xb = x + (int64_t)b * in_dim;
    double acc = (double)b2;
    for (int32_t j = 0; j < hidden; ++j) {
      const uint16_t* row = w1 + (int64_t)j * in_dim;
      double u = (double)b1[j];
      for (int32_t i = 0; i < in_dim; ++i) u += widen(row, OR_BF16, i) * widen(xb, OR_BF16, i);
      if (u > 0.0) acc += (double)w2[j] * u;
    }
    q[b] = acc;
  }
}

void oracle_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t oracle_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
