/* orthrus_oracle.c -- the CPU oracle for the Orthrus dual-view decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only tests/, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * What it computes (source: "Orthrus: Memory-Efficient Parallel Token
 * Generation via Dual-View Diffusion", as summarised on the HN item page
 * "Idea" paragraph, the atlas.scime.ai page "Approach" section and the
 * arXiv abstract on the opentrain.ai page):
 *   - a frozen autoregressive (AR) Transformer view that builds the KV cache
 *     (prefill) and verifies drafts causally;
 *   - a trainable diffusion-attention path in every layer (its own Q/K/V/O
 *     projections) that projects K mask positions in ONE forward pass over
 *     the same cache, bidirectionally inside the block, writing nothing to
 *     the cache;
 *   - greedy argmax over the shared LM head, longest-matching-prefix
 *     acceptance plus the AR bonus token, and commit of only the accepted
 *     KV entries (openai-hub.net page, "KV Cache Overhead" section).
 *
 * Arithmetic: float64 everywhere, sums in increasing index order.  For bf16
 * models the oracle rounds to bf16 exactly where the model stores bf16
 * (weights as given; GEMM input activations; q and k after QK-norm + RoPE;
 * cached K/V; attention output), taking each value to fp32 first and then to
 * bf16 with round-to-nearest-even.  fp32 models round nothing.
 *
 * Layer definition (Qwen3-style, see the function comments): RMSNorm ->
 * Q,K,V projections -> per-head QK RMSNorm -> rotate-half RoPE -> grouped
 * query attention -> O projection + residual -> RMSNorm -> SwiGLU FFN +
 * residual; final RMSNorm; untied LM head.
 *
 * The canonical weight buffer is a concatenation of tensors in a fixed
 * order (oc_weight_layout); each tensor starts at a multiple of 256
 * elements; matrices are row-major [out][in].
 *
 * The bf16 rounding points are pinned by numpy compositions of one and two
 * bf16 layers (frozen rows and mask rows) that agree to 1e-9, and by
 * mutation: removing any one rounding statement makes a composition fail.
 *
 * The diffusion view's values (mask-row logits, hence the drafts) have no
 * printed worked example on the pages, so no pin by value: they are marked
 * "parity unpinned" below.  Their structure is pinned (block
 * bidirectionality, no cache writes, reduction to the AR view under tied
 * weights and a causal block), and so is their wiring (compositions of the
 * pinned primitives with numpy matmuls, gains away from 1, fp32 and bf16).
 *
 * Per-layer entry points (oc_ar_layer, oc_draft_layer, oc_final,
 * oc_seq_load_kv) run the same arithmetic one layer at a time from given
 * inputs, so a test can hold another implementation to the oracle layer by
 * layer from that implementation's own layer inputs and cache.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t L, d, hq, hkv, hd, F, V, K;
  double theta, eps;
  int32_t bf16;   /* 1: bf16 weights (uint16 bit patterns) and bf16 storage points */
} oc_cfg;

enum {
  T_EMBED = 0, T_LMHEAD = 1, T_FNORM = 2, T_MASK = 3, T_GLOBAL = 4,
  /* per layer, offset from 4 + 17*l */
  T_ANORM = 0, T_FFNNORM = 1, T_WQ = 2, T_WK = 3, T_WV = 4, T_WO = 5, T_QN = 6, T_KN = 7,
  T_DQ = 8, T_DK = 9, T_DV = 10, T_DO = 11, T_DQN = 12, T_DKN = 13,
  T_WG = 14, T_WU = 15, T_WD = 16, T_PER_LAYER = 17
};

/* numel of canonical tensor t (global index) */
static size_t tensor_numel(const oc_cfg* c, int t) {
  size_t d = c->d, qd = (size_t)c->hq * c->hd, kd = (size_t)c->hkv * c->hd;
  if (t == T_EMBED || t == T_LMHEAD) return (size_t)c->V * d;
  if (t == T_FNORM || t == T_MASK) return d;
  int r = (t - T_GLOBAL) % T_PER_LAYER;
  switch (r) {
    case T_ANORM: case T_FFNNORM: return d;
    case T_WQ: case T_DQ: return qd * d;
    case T_WK: case T_WV: case T_DK: case T_DV: return kd * d;
    case T_WO: case T_DO: return d * qd;
    case T_QN: case T_KN: case T_DQN: case T_DKN: return (size_t)c->hd;
    case T_WG: case T_WU: return (size_t)c->F * d;
    case T_WD: return d * (size_t)c->F;
  }
  return 0;
}

int oc_num_tensors(const oc_cfg* c) { return T_GLOBAL + T_PER_LAYER * c->L; }

/* Offset (elements) and numel of tensor t; t == -1 gives the total numel. */
int oc_weight_layout(const oc_cfg* c, int t, size_t* off, size_t* numel) {
  int nt = oc_num_tensors(c);
  if (t < -1 || t >= nt) return -1;
  size_t o = 0;
  for (int i = 0; i < nt; ++i) {
    if (i == t) { *off = o; *numel = tensor_numel(c, i); return 0; }
    o += (tensor_numel(c, i) + 255) / 256 * 256;
  }
  *off = 0; *numel = o;
  return 0;
}

/* ---------------------------------------------------------------- rounding */
double oc_round_bf16(double x) {
  union { float f; uint32_t u; } v;
  v.f = (float)x;                         /* to fp32, nearest-even */
  uint32_t rnd = ((v.u >> 16) & 1u) + 0x7FFFu;
  v.u = ((v.u + rnd) >> 16) << 16;        /* to bf16, nearest-even */
  return (double)v.f;
}

static double bf16_bits_to_double(uint16_t b) {
  union { float f; uint32_t u; } v; v.u = (uint32_t)b << 16; return (double)v.f;
}

/* ------------------------------------------------------------ primitives */
/* RMSNorm: y_i = x_i / sqrt(mean(x^2) + eps) * g_i. */
void oc_rmsnorm(const double* x, const double* g, int n, double eps, double* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * r * (g ? g[i] : 1.0);
}

/* Rotate-half RoPE at absolute position pos: the pair (i, i + hd/2) is
 * rotated by the angle pos * theta^(-2i/hd). */
void oc_rope(double* v, int hd, long pos, double theta) {
  int h = hd / 2;
  for (int i = 0; i < h; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * i / hd);
    double cs = cos(ang), sn = sin(ang);
    double x1 = v[i], x2 = v[i + h];
    v[i] = x1 * cs - x2 * sn;
    v[i + h] = x2 * cs + x1 * sn;
  }
}

/* Scaled dot-product attention of one query over n keys:
 * out = sum_j softmax_j(q.k_j / sqrt(hd)) v_j.  Keys/values are rows of
 * stride hd.  Two passes (max, then sums) in float64. */
void oc_attention(const double* q, const double* const* keys, const double* const* vals, int n,
                  int hd, double* out) {
  double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)hd);
  double m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int t = 0; t < hd; ++t) acc += q[t] * keys[j][t];
    s[j] = acc * scale;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - m); l += s[j]; }
  for (int t = 0; t < hd; ++t) out[t] = 0.0;
  for (int j = 0; j < n; ++j)
    for (int t = 0; t < hd; ++t) out[t] += s[j] * vals[j][t];
  for (int t = 0; t < hd; ++t) out[t] /= l;
  free(s);
}

/* Contiguous-array wrapper of oc_attention for the tests. */
void oc_attention_dense(const double* q, const double* K, const double* V, int n, int hd,
                        double* out) {
  const double** kp = (const double**)malloc(sizeof(void*) * (n > 0 ? n : 1));
  const double** vp = (const double**)malloc(sizeof(void*) * (n > 0 ? n : 1));
  for (int j = 0; j < n; ++j) { kp[j] = K + (size_t)j * hd; vp[j] = V + (size_t)j * hd; }
  oc_attention(q, kp, vp, n, hd, out);
  free(kp); free(vp);
}

/* oc_attention of nq queries over the same n keys (one call per query,
 * queries in parallel; each result is exactly the single-query one). */
void oc_attention_many(const double* q, const double* K, const double* V, int nq, int n, int hd,
                       double* out) {
  const double** kp = (const double**)malloc(sizeof(void*) * (n > 0 ? n : 1));
  const double** vp = (const double**)malloc(sizeof(void*) * (n > 0 ? n : 1));
  for (int j = 0; j < n; ++j) { kp[j] = K + (size_t)j * hd; vp[j] = V + (size_t)j * hd; }
#pragma omp parallel for schedule(dynamic)
  for (int i = 0; i < nq; ++i) oc_attention(q + (size_t)i * hd, kp, vp, n, hd, out + (size_t)i * hd);
  free(kp); free(vp);
}

double oc_silu(double x) { return x / (1.0 + exp(-x)); }

/* Greedy choice: the largest value, lowest index on exact ties; -1 on NaN. */
int oc_argmax(const double* x, int n) {
  int best = 0;
  for (int i = 0; i < n; ++i) {
    if (x[i] != x[i]) return -1;
    if (x[i] > x[best]) best = i;
  }
  return n > 0 ? best : -1;
}

/* Longest-matching-prefix acceptance: d[0..K) are the drafts d_1..d_K,
 * a[0..K] the AR tokens a_0..a_K (a_i = AR argmax after d_1..d_i).  Returns
 * m = the largest j <= K with d_i == a_{i-1} for every i <= j. */
int oc_accept(const int32_t* d, const int32_t* a, int K) {
  int m = 0;
  while (m < K && d[m] == a[m]) ++m;
  return m;
}

/* ------------------------------------------------------------------ model */
typedef struct {
  oc_cfg c;
  const void* w;
  size_t* off;         /* per tensor offset (elements) */
  double* attn_tap;    /* optional: [L][rows][hq*hd] attention outputs of the last call */
  int attn_tap_rows;
} oc_model;

typedef struct {
  const oc_model* m;
  int cap, len;
  double* k;   /* [L][hkv][cap][hd] */
  double* v;
} oc_seq;

oc_model* oc_model_new(const oc_cfg* c, const void* weights) {
  oc_model* m = (oc_model*)calloc(1, sizeof(oc_model));
  m->c = *c;
  m->w = weights;
  int nt = oc_num_tensors(c);
  m->off = (size_t*)malloc(sizeof(size_t) * nt);
  for (int t = 0; t < nt; ++t) { size_t n; oc_weight_layout(c, t, &m->off[t], &n); }
  return m;
}

void oc_model_free(oc_model* m) { if (m) { free(m->off); free(m); } }

void oc_model_set_attn_tap(oc_model* m, double* tap, int rows) {
  m->attn_tap = tap; m->attn_tap_rows = rows;
}

static inline double wget(const oc_model* m, int t, size_t i) {
  size_t o = m->off[t] + i;
  if (m->c.bf16) return bf16_bits_to_double(((const uint16_t*)m->w)[o]);
  return (double)((const float*)m->w)[o];
}

static int lt(int l, int r) { return T_GLOBAL + T_PER_LAYER * l + r; }

static void load_vec(const oc_model* m, int t, int n, double* out) {
  for (int i = 0; i < n; ++i) out[i] = wget(m, t, (size_t)i);
}

static void store_round(const oc_model* m, double* x, size_t n) {
  if (!m->c.bf16) return;
  for (size_t i = 0; i < n; ++i) x[i] = oc_round_bf16(x[i]);
}

/* y[r][o] = sum_k x[r][k] * W[o][k] for R rows; W = tensor t, [out][in]. */
static void linear(const oc_model* m, int t, const double* x, int R, int in, int out, double* y) {
#pragma omp parallel
  {
    double* wrow = (double*)malloc(sizeof(double) * in);
#pragma omp for schedule(static)
    for (int o = 0; o < out; ++o) {
      for (int k = 0; k < in; ++k) wrow[k] = wget(m, t, (size_t)o * in + k);
      for (int r = 0; r < R; ++r) {
        const double* xr = x + (size_t)r * in;
        double acc = 0.0;
        for (int k = 0; k < in; ++k) acc += xr[k] * wrow[k];
        y[(size_t)r * out + o] = acc;
      }
    }
    free(wrow);
  }
}

oc_seq* oc_seq_new(const oc_model* m, int cap) {
  oc_seq* s = (oc_seq*)calloc(1, sizeof(oc_seq));
  s->m = m; s->cap = cap; s->len = 0;
  size_t n = (size_t)m->c.L * m->c.hkv * cap * m->c.hd;
  s->k = (double*)calloc(n, sizeof(double));
  s->v = (double*)calloc(n, sizeof(double));
  return s;
}

void oc_seq_free(oc_seq* s) { if (s) { free(s->k); free(s->v); free(s); } }
int oc_seq_len(const oc_seq* s) { return s->len; }
void oc_seq_set_len(oc_seq* s, int len) { s->len = len; }

static double* kslot(const oc_seq* s, int l, int g, int p) {
  const oc_cfg* c = &s->m->c;
  return s->k + (((size_t)l * c->hkv + g) * s->cap + p) * c->hd;
}
static double* vslot(const oc_seq* s, int l, int g, int p) {
  const oc_cfg* c = &s->m->c;
  return s->v + (((size_t)l * c->hkv + g) * s->cap + p) * c->hd;
}

/* Sum of every cached K/V value in slots [0, upto) -- the tests use it to
 * show that the draft pass leaves the committed cache untouched. */
double oc_seq_checksum(const oc_seq* s, int upto) {
  const oc_cfg* c = &s->m->c;
  double acc = 0.0;
  for (int l = 0; l < c->L; ++l)
    for (int g = 0; g < c->hkv; ++g)
      for (int p = 0; p < upto; ++p)
        for (int t = 0; t < c->hd; ++t)
          acc += kslot(s, l, g, p)[t] * (1.0 + 1e-3 * t) + vslot(s, l, g, p)[t] * (2.0 - 1e-3 * t);
  return acc;
}

/* The rest of a layer after attention: O projection + residual, then the
 * SwiGLU FFN + residual (frozen FFN, shared by both views). */
static void layer_tail(const oc_model* m, int l, int to, double* h, double* o, int R) {
  const oc_cfg* c = &m->c;
  int d = c->d, qd = c->hq * c->hd, F = c->F;
  double* y = (double*)malloc(sizeof(double) * (size_t)R * (d > 2 * F ? d : 2 * F));
  store_round(m, o, (size_t)R * qd);
  linear(m, to, o, R, qd, d, y);
  for (size_t i = 0; i < (size_t)R * d; ++i) h[i] += y[i];
  double* g = (double*)malloc(sizeof(double) * d);
  double* u = (double*)malloc(sizeof(double) * (size_t)R * d);
  load_vec(m, lt(l, T_FFNNORM), d, g);
  for (int r = 0; r < R; ++r) oc_rmsnorm(h + (size_t)r * d, g, d, c->eps, u + (size_t)r * d);
  store_round(m, u, (size_t)R * d);
  double* gate = (double*)malloc(sizeof(double) * (size_t)R * F);
  double* up = (double*)malloc(sizeof(double) * (size_t)R * F);
  linear(m, lt(l, T_WG), u, R, d, F, gate);
  linear(m, lt(l, T_WU), u, R, d, F, up);
  for (size_t i = 0; i < (size_t)R * F; ++i) gate[i] = oc_silu(gate[i]) * up[i];
  store_round(m, gate, (size_t)R * F);
  linear(m, lt(l, T_WD), gate, R, F, d, y);
  for (size_t i = 0; i < (size_t)R * d; ++i) h[i] += y[i];
  free(y); free(g); free(u); free(gate); free(up);
}

/* Q/K/V projections of R normalised rows with the given tensors, then
 * per-head QK RMSNorm and RoPE at pos[r]; q, k, v come back rounded to the
 * storage precision. */
static void qkv_proj(const oc_model* m, int l, int tq, int tk, int tv, int tqn, int tkn,
                     const double* h, int R, const long* pos, double* q, double* k, double* v) {
  const oc_cfg* c = &m->c;
  int d = c->d, hd = c->hd, qd = c->hq * hd, kd = c->hkv * hd;
  double* g = (double*)malloc(sizeof(double) * d);
  double* u = (double*)malloc(sizeof(double) * (size_t)R * d);
  load_vec(m, lt(l, T_ANORM), d, g);
  for (int r = 0; r < R; ++r) oc_rmsnorm(h + (size_t)r * d, g, d, c->eps, u + (size_t)r * d);
  store_round(m, u, (size_t)R * d);
  linear(m, tq, u, R, d, qd, q);
  linear(m, tk, u, R, d, kd, k);
  linear(m, tv, u, R, d, kd, v);
  double* qn = (double*)malloc(sizeof(double) * hd);
  double* kn = (double*)malloc(sizeof(double) * hd);
  load_vec(m, tqn, hd, qn);
  load_vec(m, tkn, hd, kn);
  for (int r = 0; r < R; ++r) {
    for (int hh = 0; hh < c->hq; ++hh) {
      double* x = q + (size_t)r * qd + (size_t)hh * hd;
      oc_rmsnorm(x, qn, hd, c->eps, x);
      oc_rope(x, hd, pos[r], c->theta);
    }
    for (int gg = 0; gg < c->hkv; ++gg) {
      double* x = k + (size_t)r * kd + (size_t)gg * hd;
      oc_rmsnorm(x, kn, hd, c->eps, x);
      oc_rope(x, hd, pos[r], c->theta);
    }
  }
  store_round(m, q, (size_t)R * qd);
  store_round(m, k, (size_t)R * kd);
  store_round(m, v, (size_t)R * kd);
  free(g); free(u); free(qn); free(kn);
}

static void final_logits(const oc_model* m, const double* h, int R, double* logits,
                         int32_t* amax) {
  const oc_cfg* c = &m->c;
  int d = c->d, V = c->V;
  double* g = (double*)malloc(sizeof(double) * d);
  double* z = (double*)malloc(sizeof(double) * (size_t)R * d);
  load_vec(m, T_FNORM, d, g);
  for (int r = 0; r < R; ++r) oc_rmsnorm(h + (size_t)r * d, g, d, c->eps, z + (size_t)r * d);
  store_round(m, z, (size_t)R * d);
  double* lg = logits ? logits : (double*)malloc(sizeof(double) * (size_t)R * V);
  linear(m, T_LMHEAD, z, R, d, V, lg);
  if (amax)
    for (int r = 0; r < R; ++r) amax[r] = oc_argmax(lg + (size_t)r * V, V);
  if (!logits) free(lg);
  free(g); free(z);
}

/* Cache slots [0, n) of layer l from K and V rows laid out [hkv][n][hd]
 * (test infrastructure: lets a test hold the oracle to another
 * implementation's cache state, layer by layer). */
int oc_seq_load_kv(oc_seq* s, int l, const double* k, const double* v, int n) {
  const oc_cfg* c = &s->m->c;
  if (l < 0 || l >= c->L || n < 0 || n > s->cap) return -2;
  for (int g = 0; g < c->hkv; ++g)
    for (int p = 0; p < n; ++p) {
      memcpy(kslot(s, l, g, p), k + ((size_t)g * n + p) * c->hd, sizeof(double) * c->hd);
      memcpy(vslot(s, l, g, p), v + ((size_t)g * n + p) * c->hd, sizeof(double) * c->hd);
    }
  return 0;
}

/* The inverse of oc_seq_load_kv: cache slots [0, n) of layer l into K and V
 * rows [hkv][n][hd]. */
int oc_seq_read_kv(const oc_seq* s, int l, double* k, double* v, int n) {
  const oc_cfg* c = &s->m->c;
  if (l < 0 || l >= c->L || n < 0 || n > s->cap) return -2;
  for (int g = 0; g < c->hkv; ++g)
    for (int p = 0; p < n; ++p) {
      memcpy(k + ((size_t)g * n + p) * c->hd, kslot(s, l, g, p), sizeof(double) * c->hd);
      memcpy(v + ((size_t)g * n + p) * c->hd, vslot(s, l, g, p), sizeof(double) * c->hd);
    }
  return 0;
}

/* One layer of the frozen AR view for R consecutive rows at positions
 * pos0..pos0+R-1 whose layer inputs are h[R][d] (overwritten with the layer
 * outputs).  Row r's K/V are written to cache slot pos0+r of layer l, then
 * row r attends causally to slots [0, pos0+r].  o_raw (optional, [R][hq*hd])
 * receives the attention output before its bf16 rounding. */
int oc_ar_layer(const oc_model* m, oc_seq* s, int l, double* h, int R, int pos0, double* o_raw) {
  const oc_cfg* c = &m->c;
  if (l < 0 || l >= c->L || pos0 < 0 || pos0 + R > s->cap) return -2;
  int hd = c->hd, qd = c->hq * hd, kd = c->hkv * hd, grp = c->hq / c->hkv;
  long* pos = (long*)malloc(sizeof(long) * R);
  for (int r = 0; r < R; ++r) pos[r] = pos0 + r;
  double* q = (double*)malloc(sizeof(double) * (size_t)R * qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)R * kd);
  double* v = (double*)malloc(sizeof(double) * (size_t)R * kd);
  double* o = (double*)malloc(sizeof(double) * (size_t)R * qd);
  qkv_proj(m, l, lt(l, T_WQ), lt(l, T_WK), lt(l, T_WV), lt(l, T_QN), lt(l, T_KN), h, R, pos, q, k,
           v);
  for (int r = 0; r < R; ++r)
    for (int g = 0; g < c->hkv; ++g) {
      memcpy(kslot(s, l, g, pos0 + r), k + (size_t)r * kd + (size_t)g * hd, sizeof(double) * hd);
      memcpy(vslot(s, l, g, pos0 + r), v + (size_t)r * kd + (size_t)g * hd, sizeof(double) * hd);
    }
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < R; ++r)
    for (int hh = 0; hh < c->hq; ++hh) {
      int g = hh / grp, n = pos0 + r + 1;
      const double** kp = (const double**)malloc(sizeof(void*) * n);
      const double** vp = (const double**)malloc(sizeof(void*) * n);
      for (int j = 0; j < n; ++j) { kp[j] = kslot(s, l, g, j); vp[j] = vslot(s, l, g, j); }
      oc_attention(q + (size_t)r * qd + (size_t)hh * hd, kp, vp, n, hd,
                   o + (size_t)r * qd + (size_t)hh * hd);
      free(kp); free(vp);
    }
  if (o_raw) memcpy(o_raw, o, sizeof(double) * (size_t)R * qd);
  if (m->attn_tap && R <= m->attn_tap_rows) {
    double* tap = m->attn_tap + (size_t)l * m->attn_tap_rows * qd;
    memcpy(tap, o, sizeof(double) * (size_t)R * qd);
    store_round(m, tap, (size_t)R * qd);
  }
  layer_tail(m, l, lt(l, T_WO), h, o, R);
  free(pos); free(q); free(k); free(v); free(o);
  return 0;
}

/* The rest of layer l after attention (O projection + residual, FFN +
 * residual) for R rows with inputs h[R][d] (overwritten with the layer
 * outputs) and attention outputs o[R][hq*hd] (rounded to the model's
 * storage precision first, as in every layer): the diffusion view's O
 * projection if diffusion != 0, else the frozen one. */
int oc_layer_tail(const oc_model* m, int l, int diffusion, double* h, const double* o, int R) {
  const oc_cfg* c = &m->c;
  if (l < 0 || l >= c->L || R < 1) return -2;
  size_t n = (size_t)R * c->hq * c->hd;
  double* oc = (double*)malloc(sizeof(double) * n);
  memcpy(oc, o, sizeof(double) * n);
  layer_tail(m, l, lt(l, diffusion ? T_DO : T_WO), h, oc, R);
  free(oc);
  return 0;
}

/* Final RMSNorm and LM head of R rows: logits [R][V] and argmax tokens [R]
 * (each optional). */
void oc_final(const oc_model* m, const double* h, int R, double* logits, int32_t* amax) {
  final_logits(m, h, R, logits, amax);
}

/* Frozen AR view over R consecutive tokens at positions pos0..pos0+R-1:
 * the embeddings, then every layer (oc_ar_layer), then the final norm and LM
 * head.  This single routine is prefill (R = prompt), plain greedy decoding
 * (R = 1), the draft pass's anchor row (R = 1 at position len) and the
 * verify pass (R = K at len+1).  Logits [R][V] (optional) and argmax tokens
 * [R] are returned.  The sequence length is not changed (callers commit). */
int oc_ar_rows(const oc_model* m, oc_seq* s, const int32_t* tokens, int R, int pos0,
               double* logits, int32_t* amax) {
  const oc_cfg* c = &m->c;
  if (pos0 < 0 || pos0 + R > s->cap) return -2;
  int d = c->d;
  for (int r = 0; r < R; ++r)
    if (tokens[r] < 0 || tokens[r] >= c->V) return -1;
  double* h = (double*)malloc(sizeof(double) * (size_t)R * d);
  for (int r = 0; r < R; ++r)
    for (int i = 0; i < d; ++i) h[(size_t)r * d + i] = wget(m, T_EMBED, (size_t)tokens[r] * d + i);
  for (int l = 0; l < c->L; ++l) oc_ar_layer(m, s, l, h, R, pos0, NULL);
  final_logits(m, h, R, logits, amax);
  free(h);
  return 0;
}

/* One layer of the diffusion view for the block of K mask positions
 * n+1..n+K (n = len) whose layer inputs are h[K][d] (overwritten with the
 * layer outputs): the diffusion Q/K/V/O projections and QK-norm gains, the
 * shared norms and FFN; every row attends to the cache slots [0, n] plus
 * all K block rows of this layer (bidirectional; causal = 1 restricts row i
 * to block rows 0..i, for the structural test).  Block K/V stay in local
 * scratch: nothing is written to the cache.  o_raw (optional, [K][hq*hd])
 * receives the attention output before its bf16 rounding. */
int oc_draft_layer(const oc_model* m, const oc_seq* s, int l, double* h, int n, int K, int causal,
                   double* o_raw) {
  const oc_cfg* c = &m->c;
  if (l < 0 || l >= c->L || n < 0 || n >= s->cap || K <= 0) return -2;
  int hd = c->hd, qd = c->hq * hd, kd = c->hkv * hd, grp = c->hq / c->hkv;
  long* pos = (long*)malloc(sizeof(long) * K);
  for (int r = 0; r < K; ++r) pos[r] = n + 1 + r;
  double* q = (double*)malloc(sizeof(double) * (size_t)K * qd);
  double* bk = (double*)malloc(sizeof(double) * (size_t)K * kd);
  double* bv = (double*)malloc(sizeof(double) * (size_t)K * kd);
  double* o = (double*)malloc(sizeof(double) * (size_t)K * qd);
  qkv_proj(m, l, lt(l, T_DQ), lt(l, T_DK), lt(l, T_DV), lt(l, T_DQN), lt(l, T_DKN), h, K, pos, q,
           bk, bv);
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < K; ++r)
    for (int hh = 0; hh < c->hq; ++hh) {
      int g = hh / grp, nb = causal ? r + 1 : K, nk = n + 1 + nb;
      const double** kp = (const double**)malloc(sizeof(void*) * nk);
      const double** vp = (const double**)malloc(sizeof(void*) * nk);
      for (int j = 0; j <= n; ++j) { kp[j] = kslot(s, l, g, j); vp[j] = vslot(s, l, g, j); }
      for (int j = 0; j < nb; ++j) {
        kp[n + 1 + j] = bk + (size_t)j * kd + (size_t)g * hd;
        vp[n + 1 + j] = bv + (size_t)j * kd + (size_t)g * hd;
      }
      oc_attention(q + (size_t)r * qd + (size_t)hh * hd, kp, vp, nk, hd,
                   o + (size_t)r * qd + (size_t)hh * hd);
      free(kp); free(vp);
    }
  if (o_raw) memcpy(o_raw, o, sizeof(double) * (size_t)K * qd);
  if (m->attn_tap && K <= m->attn_tap_rows) {
    double* tap = m->attn_tap + (size_t)l * m->attn_tap_rows * qd;
    memcpy(tap, o, sizeof(double) * (size_t)K * qd);
    store_round(m, tap, (size_t)K * qd);
  }
  layer_tail(m, l, lt(l, T_DO), h, o, K);
  free(pos); free(q); free(bk); free(bv); free(o);
  return 0;
}

/* Diffusion view over the block of K mask positions n+1..n+K in one
 * forward pass: every row starts from the mask embedding (or, for the
 * structural test only, from the embeddings of given tokens), then every
 * layer (oc_draft_layer), then the shared final norm and LM head.  Parity
 * unpinned (values): see the file header. */
int oc_draft_rows(const oc_model* m, const oc_seq* s, int n, int K, const int32_t* in_tokens,
                  int causal, double* logits, int32_t* amax) {
  const oc_cfg* c = &m->c;
  if (n < 0 || n >= s->cap || K <= 0) return -2;
  int d = c->d;
  double* h = (double*)malloc(sizeof(double) * (size_t)K * d);
  for (int r = 0; r < K; ++r)
    for (int i = 0; i < d; ++i)
      h[(size_t)r * d + i] = in_tokens ? wget(m, T_EMBED, (size_t)in_tokens[r] * d + i)
                                       : wget(m, T_MASK, (size_t)i);
  for (int l = 0; l < c->L; ++l) oc_draft_layer(m, s, l, h, n, K, causal, NULL);
  final_logits(m, h, K, logits, amax);
  free(h);
  return 0;
}

/* Prefill: the AR view over the whole prompt; len <- P; returns the first
 * generated token (argmax of the last prompt row) or < 0 on error. */
int oc_prefill(const oc_model* m, oc_seq* s, const int32_t* prompt, int P, double* last_logits) {
  if (P <= 0 || P > s->cap) return -2;
  int32_t* am = (int32_t*)malloc(sizeof(int32_t) * P);
  double* lg = (double*)malloc(sizeof(double) * (size_t)P * m->c.V);
  int rc = oc_ar_rows(m, s, prompt, P, 0, lg, am);
  int tok = rc ? rc : am[P - 1];
  if (!rc) {
    s->len = P;
    if (last_logits) memcpy(last_logits, lg + (size_t)(P - 1) * m->c.V, sizeof(double) * m->c.V);
  }
  free(am); free(lg);
  return tok;
}

/* One draft -> verify -> accept -> commit step with block size K, as
 * described by the pages: pass 1 runs the AR view on the pending token at
 * position n (its argmax a_0; its K/V staged at slot n) and the diffusion
 * view on K mask positions n+1..n+K (drafts d_1..d_K, nothing cached);
 * pass 2 runs the AR view causally over d_1..d_K at n+1..n+K (a_1..a_K,
 * K/V staged); m = the longest prefix with d_i == a_{i-1}; the step emits
 * d_1..d_m and the bonus a_m; only slots n..n+m become committed.
 * K == 0 is plain greedy decoding (one AR row, emits a_0).
 * planted (optional) replaces the drafts after pass 1.
 * Outputs: drafts[K], ar[K+1], logits_anchor[V], logits_draft[K][V],
 * logits_verify[K][V] (each optional), emitted[K+1]; returns m or < 0. */
int oc_step(const oc_model* m, oc_seq* s, int32_t pending, int K, const int32_t* planted,
            int32_t* drafts, int32_t* ar, double* logits_anchor, double* logits_draft,
            double* logits_verify, int32_t* emitted, int32_t* new_pending) {
  int n = s->len;
  if (n + K + 1 > s->cap) return -2;
  int32_t a0;
  int rc = oc_ar_rows(m, s, &pending, 1, n, logits_anchor, &a0);
  if (rc) return rc;
  ar[0] = a0;
  if (K == 0) {
    emitted[0] = a0;
    s->len = n + 1;
    *new_pending = a0;
    return 0;
  }
  int32_t* d = (int32_t*)malloc(sizeof(int32_t) * K);
  rc = oc_draft_rows(m, s, n, K, NULL, 0, logits_draft, d);
  if (rc) { free(d); return rc; }
  if (planted) memcpy(d, planted, sizeof(int32_t) * K);
  for (int i = 0; i < K; ++i) if (d[i] < 0) { free(d); return -1; }
  rc = oc_ar_rows(m, s, d, K, n + 1, logits_verify, ar + 1);
  if (rc) { free(d); return rc; }
  int acc = oc_accept(d, ar, K);
  for (int i = 0; i < acc; ++i) emitted[i] = d[i];
  emitted[acc] = ar[acc];
  if (drafts) memcpy(drafts, d, sizeof(int32_t) * K);
  s->len = n + 1 + acc;
  *new_pending = ar[acc];
  free(d);
  return acc;
}

/* Plain greedy AR decoding: prefill, then one row at a time.  Writes the
 * first n_new generated tokens (token 1 = argmax of the last prompt row). */
int oc_ar_generate(const oc_model* m, const int32_t* prompt, int P, int n_new, int32_t* out) {
  oc_seq* s = oc_seq_new(m, P + n_new + 1);
  int tok = oc_prefill(m, s, prompt, P, NULL);
  if (tok < 0) { oc_seq_free(s); return tok; }
  for (int t = 0; t < n_new; ++t) {
    out[t] = tok;
    if (t + 1 == n_new) break;
    int32_t nx;
    int rc = oc_ar_rows(m, s, &tok, 1, s->len, NULL, &nx);
    if (rc) { oc_seq_free(s); return rc; }
    s->len += 1;
    tok = nx;
  }
  oc_seq_free(s);
  return 0;
}

/* Orthrus generation: prefill, then draft/verify/accept/commit steps until
 * n_new tokens exist (the step that crosses n_new is truncated).  planted:
 * optional [max_steps][K] table used instead of the drafts.  Per-step
 * accept lengths go to accept_out[max_steps] (optional) and the cache length
 * before each step to len_out; returns the number of steps or < 0. */
int oc_generate(const oc_model* m, const int32_t* prompt, int P, int n_new, int K,
                const int32_t* planted, int max_steps, int32_t* out, int32_t* accept_out,
                int32_t* len_out) {
  oc_seq* s = oc_seq_new(m, P + n_new + K + 2);
  int tok = oc_prefill(m, s, prompt, P, NULL);
  if (tok < 0) { oc_seq_free(s); return tok; }
  int have = 0;
  out[have++] = tok;
  int32_t* em = (int32_t*)malloc(sizeof(int32_t) * (K + 1));
  int32_t* ar = (int32_t*)malloc(sizeof(int32_t) * (K + 1));
  int steps = 0;
  while (have < n_new) {
    if (steps >= max_steps) break;
    if (len_out) len_out[steps] = s->len;
    int32_t np;
    int acc = oc_step(m, s, tok, K, planted ? planted + (size_t)steps * K : NULL, NULL, ar, NULL,
                      NULL, NULL, em, &np);
    if (acc < 0) { steps = acc; break; }
    if (accept_out) accept_out[steps] = acc;
    for (int i = 0; i <= acc && have < n_new; ++i) out[have++] = em[i];
    tok = np;
    ++steps;
  }
  free(em); free(ar);
  oc_seq_free(s);
  return steps;
}

/* ------------------------------------------------------ sampling at T > 0
 * The pages say only that T > 0 relies on rejection sampling (HN item page
 * and atlas.scime.ai page, "Limitations").  The rule followed is the
 * standard speculative-sampling one: drafts are draws of the draft
 * distribution q; draft i is accepted with probability
 * min(1, p_{i-1}(d_i) / q_i(d_i)); at the first rejection the final token is
 * a draw of max(0, p - q) renormalised, after K acceptances a draw of p_K.
 * Distributions are softmax(z / T) of the logits. */

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11): ten rounds on the 128-bit counter, the key
 * bumped by the Weyl constants between rounds. */
void oc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform in [0, 1) a draw of (purpose, index) of sequence seq at step
 * uses: counter (index, seq, step, purpose) under key seed; 24 bits of the
 * first output word. */
double oc_uniform(uint64_t seed, uint32_t step, uint32_t purpose, uint32_t index, uint32_t seq) {
  uint32_t ctr[4] = {index, seq, step, purpose}, key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oc_philox4x32_10(ctr, key, out);
  return (double)(out[0] >> 8) / 16777216.0;
}

/* softmax(z / T) of n logits into prob (float64, index-order sum). */
void oc_softmax_t(const double* z, int n, double T, double* prob) {
  double m = -INFINITY, s = 0.0;
  for (int j = 0; j < n; ++j) if (z[j] > m) m = z[j];
  for (int j = 0; j < n; ++j) { prob[j] = exp((z[j] - m) / T); s += prob[j]; }
  for (int j = 0; j < n; ++j) prob[j] /= s;
}

/* A draw of the (unnormalised) weights w[0..n) with uniform u: the first j
 * whose running sum in index order exceeds u * sum(w); -1 if all are 0. */
int oc_draw(const double* w, int n, double u) {
  double s = 0.0;
  for (int j = 0; j < n; ++j) s += w[j];
  if (!(s > 0.0)) return -1;
  double t = u * s, acc = 0.0;
  int last = -1;
  for (int j = 0; j < n; ++j) {
    if (!(w[j] > 0.0)) continue;
    last = j;
    acc += w[j];
    if (acc > t) return j;
  }
  return last;
}

/* A draw of softmax(z / T) with uniform u. */
int oc_sample_logits(const double* z, int n, double T, double u) {
  double* p = (double*)malloc(sizeof(double) * n);
  oc_softmax_t(z, n, T, p);
  int j = oc_draw(p, n, u);
  free(p);
  return j;
}

/* Acceptance of one sequence's K drafts and its final token.  pz: the AR
 * logits [K+1][V] (p_0 from the anchor row, p_i from verify row i); qz:
 * the draft logits [K][V] (q_1..q_K); d: the drafts; ua[i]: the uniform of
 * draft i+1's test; uf: the final token's.  Returns m; *tok = the final
 * token. */
int oc_spec_accept(const double* pz, const double* qz, const int32_t* d, int K, int V, double T,
                   const double* ua, double uf, int32_t* tok) {
  double* p = (double*)malloc(sizeof(double) * V);
  double* q = (double*)malloc(sizeof(double) * V);
  int m = 0;
  for (; m < K; ++m) {
    if (d[m] < 0 || d[m] >= V) break;
    oc_softmax_t(pz + (size_t)m * V, V, T, p);
    oc_softmax_t(qz + (size_t)m * V, V, T, q);
    if (!(ua[m] < p[d[m]] / q[d[m]])) break;
  }
  oc_softmax_t(pz + (size_t)m * V, V, T, p);
  if (m < K) {
    oc_softmax_t(qz + (size_t)m * V, V, T, q);
    for (int j = 0; j < V; ++j) q[j] = p[j] > q[j] ? p[j] - q[j] : 0.0;
    int j = oc_draw(q, V, uf);
    *tok = j >= 0 ? j : oc_draw(p, V, uf);
  } else {
    *tok = oc_draw(p, V, uf);
  }
  free(p); free(q);
  return m;
}
