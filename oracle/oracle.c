/*
 * CPU ORACLE -- test infrastructure only.
 *
 * A plain, slow, fp64 decoder that states what the persistent decode path
 * must compute.  Only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg load it; the GPU path shares no code with it.
 *
 * Sources (web pages on Mirage Persistent Kernel, "MPK"):
 *   P1  "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference into One
 *        Kernel Launch" (hysenlabs.com, English review)
 *   P3  gokawiil.com blog excerpt on MPK, section "Why MPK?" and Figure 1
 *   P4  "Mirage Persistent Kernel：把 LLM 推理压进单个 GPU 内核" (hysenlabs.com, Chinese review)
 *   P5  "Mirage Persistent Kernel kompiliert LLM-Inferenz in einen Persistent
 *        Kernel" (hysenlabs.com, German review)
 *
 * What the pages fix: decoding is autoregressive over a token tensor
 * tokens[num_requests, seq_length] holding prompt and generated ids, with an
 * integer step per request advanced after every iteration (P1 "How MPK Works";
 * P5 "Betrieb und Konfiguration"); the model is a Qwen3-8B decoder built from
 * normalisation, linear and attention operators (P1 "The Problem" and "Getting
 * Started"; P4 "它解决什么"), with RMSNorm fused into the following linear layer
 * (P1 "The API"; P5 "Grenzen der README-Aussagen").  The pages are silent on
 * the layer's arithmetic; every reading taken here (eps, QK-norm, RoPE, GQA
 * grouping, KV-cache precision, argmax ties, prompt handling) is listed with
 * its reason in the design notes, and each function below says which reading
 * it follows.  Arithmetic is fp64 throughout; bf16 weights are widened
 * exactly; the KV cache is stored as bf16 (round to nearest even from the
 * fp32 value, the GPU's own precision at that point).
 *
 * Parity pins (tests/test_oracle_pins.py) tie each function to closed forms,
 * invariants and brute force.  The composed 36-layer decoder has no pin beyond
 * its pinned parts: for the full model, parity is unpinned beyond this file.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 <-> floating point (exact widening; RNE narrowing) ---------------- */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---- RMSNorm --------------------------------------------------------------
 * y_i = g_i * x_i / sqrt(mean_j x_j^2 + eps).  Reading: eps inside the root,
 * the gain multiplies the normalised value (no 1+g form).  The operator is
 * named by P1 "The API" (rmsnorm_linear_layer) and P4 "它解决什么". */
void orc_rmsnorm(int32_t n, const double* x, const uint16_t* gain, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = orc_bf16_to_f64(gain[i]) * (x[i] * inv);
}

/* ---- Linear layer ----------------------------------------------------------
 * y[o] = sum_i W[o][i] * x[i], W row-major [rows][cols] bf16.  Each row is one
 * sequential fp64 sum, so results do not depend on the thread count. */
void orc_linear(int32_t rows, int32_t cols, const uint16_t* W, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int32_t o = 0; o < rows; ++o) {
    const uint16_t* w = W + (int64_t)o * cols;
    double acc = 0.0;
    for (int32_t i = 0; i < cols; ++i) acc += orc_bf16_to_f64(w[i]) * x[i];
    y[o] = acc;
  }
}

/* ---- Rotary position embedding --------------------------------------------
 * Reading (pages silent): pairs (i, i + d/2) for i < d/2, angle
 * pos * theta^(-2i/d), rotation by +angle:
 *   (a, b) -> (a cos - b sin, b cos + a sin). */
void orc_rope(int32_t d, double theta, int64_t pos, double* x) {
  int32_t half = d / 2;
  for (int32_t i = 0; i < half; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    double c = cos(ang), s = sin(ang);
    double a = x[i], b = x[i + half];
    x[i] = a * c - b * s;
    x[i + half] = b * c + a * s;
  }
}

/* ---- Softmax --------------------------------------------------------------*/
void orc_softmax(int32_t n, const double* s, double* w) {
  double m = -INFINITY;
  for (int32_t i = 0; i < n; ++i) m = s[i] > m ? s[i] : m;
  double z = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    w[i] = exp(s[i] - m);
    z += w[i];
  }
  for (int32_t i = 0; i < n; ++i) w[i] /= z;
}

/* ---- One attention head over a bf16 K/V history ---------------------------
 * out = sum_t softmax_t(q . K[t] / sqrt(d)) V[t], t = 0..n-1 (all positions up
 * to and including the current one: causal decode).  K, V: [n][d] bf16. */
void orc_attention_head(int32_t d, int32_t n, const double* q, const uint16_t* K,
                        const uint16_t* V, double* out) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)d);
  for (int32_t t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int32_t i = 0; i < d; ++i) acc += q[i] * orc_bf16_to_f64(K[(int64_t)t * d + i]);
    s[t] = acc * scale;
  }
  orc_softmax(n, s, s);
  for (int32_t i = 0; i < d; ++i) out[i] = 0.0;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t i = 0; i < d; ++i) out[i] += s[t] * orc_bf16_to_f64(V[(int64_t)t * d + i]);
  free(s);
}

/* ---- Grouped-query attention ----------------------------------------------
 * Reading: q head h reads kv head floor(h / (n_q / n_kv)) (contiguous groups).
 * q: [n_q][d]; K, V: [n_kv][stride][d] bf16 of which the first n positions are
 * attended; out: [n_q][d]. */
void orc_gqa_attention(int32_t n_q, int32_t n_kv, int32_t d, int32_t n, int64_t stride,
                       const double* q, const uint16_t* K, const uint16_t* V, double* out) {
  int32_t group = n_q / n_kv;
  for (int32_t h = 0; h < n_q; ++h) {
    int32_t j = h / group;
    orc_attention_head(d, n, q + (int64_t)h * d, K + (int64_t)j * stride * d,
                       V + (int64_t)j * stride * d, out + (int64_t)h * d);
  }
}

/* ---- SiLU ------------------------------------------------------------------*/
double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* ---- Argmax: lowest index among equal maxima; also the top-2 margin ---------*/
int32_t orc_argmax(int32_t n, const double* v, double* margin) {
  int32_t best = 0;
  for (int32_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  double second = -INFINITY;
  for (int32_t i = 0; i < n; ++i)
    if (i != best && v[i] > second) second = v[i];
  if (margin) *margin = v[best] - second;
  return best;
}

/* ---- Model ---------------------------------------------------------------- */
typedef struct {
  int32_t layers, hidden, n_q, n_kv, head_dim, ffn, vocab;
  double rms_eps, rope_theta;
  const uint16_t* E;          /* [vocab][hidden]: embedding and tied LM head */
  const uint16_t* final_norm; /* [hidden] */
  const uint16_t* const* attn_norm; /* per layer [hidden] */
  const uint16_t* const* wq;        /* [n_q*d][hidden] */
  const uint16_t* const* wk;        /* [n_kv*d][hidden] */
  const uint16_t* const* wv;        /* [n_kv*d][hidden] */
  const uint16_t* const* q_norm;    /* [d] */
  const uint16_t* const* k_norm;    /* [d] */
  const uint16_t* const* wo;        /* [hidden][n_q*d] */
  const uint16_t* const* ffn_norm;  /* [hidden] */
  const uint16_t* const* wg;        /* [ffn][hidden] */
  const uint16_t* const* wu;        /* [ffn][hidden] */
  const uint16_t* const* wd;        /* [hidden][ffn] */
} orc_model;

typedef struct {
  int32_t batch, tokens_width, max_seq;
  int32_t* tokens;           /* [batch][tokens_width] */
  int32_t* step;             /* [batch] */
  const int32_t* prompt_len; /* [batch] */
  uint16_t* kcache;          /* [layers][batch][n_kv][max_seq][d] bf16 */
  uint16_t* vcache;
} orc_state;

static int64_t kv_off(const orc_model* m, const orc_state* st, int32_t l, int32_t r) {
  return (((int64_t)l * st->batch + r) * m->n_kv) * (int64_t)st->max_seq * m->head_dim;
}

/* One decoder layer for request r at position pos; h [hidden] updated in
 * place; K/V of this position written to the cache.  Order (reading S1, S4):
 *   a = RMSNorm(h; attn_norm); q = Wq a, k = Wk a, v = Wv a;
 *   per head q_h = RoPE(RMSNorm(q_h; q_norm)), k_j = RoPE(RMSNorm(k_j; k_norm));
 *   K[pos] = bf16(k), V[pos] = bf16(v); o = GQA attention over positions 0..pos;
 *   h += Wo o; b = RMSNorm(h; ffn_norm); h += Wd (silu(Wg b) * (Wu b)). */
void orc_layer(const orc_model* m, int32_t l, orc_state* st, int32_t r, int32_t pos, double* h) {
  const int32_t H = m->hidden, d = m->head_dim, nq = m->n_q, nkv = m->n_kv, F = m->ffn;
  double* a = (double*)malloc(sizeof(double) * H);
  double* q = (double*)malloc(sizeof(double) * nq * d);
  double* k = (double*)malloc(sizeof(double) * nkv * d);
  double* v = (double*)malloc(sizeof(double) * nkv * d);
  double* o = (double*)malloc(sizeof(double) * nq * d);
  double* t = (double*)malloc(sizeof(double) * (H > F ? H : F));
  double* g = (double*)malloc(sizeof(double) * F);
  double* u = (double*)malloc(sizeof(double) * F);

  orc_rmsnorm(H, h, m->attn_norm[l], m->rms_eps, a);
  orc_linear(nq * d, H, m->wq[l], a, q);
  orc_linear(nkv * d, H, m->wk[l], a, k);
  orc_linear(nkv * d, H, m->wv[l], a, v);
  for (int32_t hh = 0; hh < nq; ++hh) {
    orc_rmsnorm(d, q + (int64_t)hh * d, m->q_norm[l], m->rms_eps, t);
    memcpy(q + (int64_t)hh * d, t, sizeof(double) * d);
    orc_rope(d, m->rope_theta, pos, q + (int64_t)hh * d);
  }
  uint16_t* Kc = st->kcache + kv_off(m, st, l, r);
  uint16_t* Vc = st->vcache + kv_off(m, st, l, r);
  for (int32_t j = 0; j < nkv; ++j) {
    orc_rmsnorm(d, k + (int64_t)j * d, m->k_norm[l], m->rms_eps, t);
    memcpy(k + (int64_t)j * d, t, sizeof(double) * d);
    orc_rope(d, m->rope_theta, pos, k + (int64_t)j * d);
    for (int32_t i = 0; i < d; ++i) {
      int64_t at = ((int64_t)j * st->max_seq + pos) * d + i;
      Kc[at] = orc_f32_to_bf16((float)k[(int64_t)j * d + i]);
      Vc[at] = orc_f32_to_bf16((float)v[(int64_t)j * d + i]);
    }
  }
  orc_gqa_attention(nq, nkv, d, pos + 1, st->max_seq, q, Kc, Vc, o);
  orc_linear(H, nq * d, m->wo[l], o, t);
  for (int32_t i = 0; i < H; ++i) h[i] += t[i];

  orc_rmsnorm(H, h, m->ffn_norm[l], m->rms_eps, a);
  orc_linear(F, H, m->wg[l], a, g);
  orc_linear(F, H, m->wu[l], a, u);
  for (int32_t i = 0; i < F; ++i) g[i] = orc_silu(g[i]) * u[i];
  orc_linear(H, F, m->wd[l], g, t);
  for (int32_t i = 0; i < H; ++i) h[i] += t[i];

  free(a); free(q); free(k); free(v); free(o); free(t); free(g); free(u);
}

/* Final RMSNorm and tied LM head: logits = E . RMSNorm(h; final_norm). */
void orc_lm_head(const orc_model* m, const double* h, double* logits) {
  double* z = (double*)malloc(sizeof(double) * m->hidden);
  orc_rmsnorm(m->hidden, h, m->final_norm, m->rms_eps, z);
  orc_linear(m->vocab, m->hidden, m->E, z, logits);
  free(z);
}

/* Greedy decoding, n_iter iterations over every request (P1 "How MPK Works":
 * the runtime advances step after each decoding iteration).  Iteration for
 * request r at p = step[r]: consume tokens[r][p], run all layers, take the
 * argmax of the logits; when p + 1 >= prompt_len[r] the argmax becomes
 * tokens[r][p + 1] (otherwise position p + 1 already holds a prompt id that is
 * kept); then step[r] = p + 1.  Requests are independent.  Optional outputs per
 * iteration and request: logits [n_iter][batch][vocab], argmax and top-2
 * margin [n_iter][batch].  Returns 0, or -1 if a position would leave the
 * token tensor or the KV cache. */
int32_t orc_decode(const orc_model* m, orc_state* st, int32_t n_iter, double* logits_out,
                   int32_t* argmax_out, double* margin_out) {
  const int32_t H = m->hidden, V = m->vocab;
  double* h = (double*)malloc(sizeof(double) * H);
  double* logits = (double*)malloc(sizeof(double) * V);
  for (int32_t s = 0; s < n_iter; ++s) {
    for (int32_t r = 0; r < st->batch; ++r) {
      int32_t p = st->step[r];
      if (p + 1 >= st->tokens_width || p >= st->max_seq) {
        free(h);
        free(logits);
        return -1;
      }
      int32_t tok = st->tokens[(int64_t)r * st->tokens_width + p];
      const uint16_t* e = m->E + (int64_t)tok * H;
      for (int32_t i = 0; i < H; ++i) h[i] = orc_bf16_to_f64(e[i]);
      for (int32_t l = 0; l < m->layers; ++l) orc_layer(m, l, st, r, p, h);
      orc_lm_head(m, h, logits);
      double margin;
      int32_t next = orc_argmax(V, logits, &margin);
      if (logits_out) memcpy(logits_out + ((int64_t)s * st->batch + r) * V, logits, sizeof(double) * V);
      if (argmax_out) argmax_out[(int64_t)s * st->batch + r] = next;
      if (margin_out) margin_out[(int64_t)s * st->batch + r] = margin;
      if (p + 1 >= st->prompt_len[r]) st->tokens[(int64_t)r * st->tokens_width + p + 1] = next;
      st->step[r] = p + 1;
    }
  }
  free(h);
  free(logits);
  return 0;
}
