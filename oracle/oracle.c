/* oracle.c -- plain CPU oracle of the Llama-family decode step (test infrastructure only).
 *
 * Written for clarity, not speed: every step is the textbook definition in IEEE double,
 * in the order the pages give it.  The only concession to run time is an OpenMP
 * `parallel for` over independent output rows (each row is one thread's plain loop, so
 * the result does not depend on the thread count) and over independent heads.
 * See oracle.h for the storage rounding points and the sources.
 */
#include "oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* scalar encodings (IEEE 754 definitions written out)                                  */
/* ------------------------------------------------------------------------------------ */

double orc_bf16_to_double(uint16_t b) {
  /* bf16 is the top half of an IEEE binary32 */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round |a| > 0 to a binary format with `mbits` stored mantissa bits and minimum normal
 * exponent `emin`, round to nearest even.  Returns the rounded magnitude. */
static double round_to_format(double a, int mbits, int emin) {
  int e;
  frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;             /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin;    /* subnormal range: fixed spacing */
  double ulp = ldexp(1.0, E - mbits);
  return nearbyint(a / ulp) * ulp;   /* a/ulp is exact; nearbyint rounds half to even */
}

uint16_t orc_double_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  double r = round_to_format(a, 7, -126);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: at most 8 significant bits, within binary32 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

double orc_fp16_to_double(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

uint16_t orc_double_to_fp16(double x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  double r = round_to_format(a, 10, -14);
  if (r > 65504.0) return (uint16_t)(sign | 0x7C00);
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  int e;
  frexp(r, &e);
  int E = e - 1;
  int mant = (int)(r / ldexp(1.0, E - 10)) - 1024;
  return (uint16_t)(sign | ((E + 15) << 10) | mant);
}

double orc_round_act(double x, int32_t act) {
  if (act == ORC_ACT_BF16) return orc_bf16_to_double(orc_double_to_bf16(x));
  return (double)(float)x; /* binary32, round to nearest even */
}

void orc_round_act_n(const double* x, int32_t n, int32_t act, double* out) {
  for (int32_t i = 0; i < n; i++) out[i] = orc_round_act(x[i], act);
}

/* ------------------------------------------------------------------------------------ */
/* single operations                                                                    */
/* ------------------------------------------------------------------------------------ */

void orc_rmsnorm(const double* x, const float* g, int32_t n, double eps, double* out) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; i++) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; i++) out[i] = x[i] * r * (double)g[i];
}

/* Q4_0 ("Go 语言原本" 20.2.4, quantization: tensors back to bytes): blocks of 32 columns,
 * 16 bytes of 4-bit codes and one fp16 scale d per block; the low 4 bits of a block's byte j
 * belong to column j of the block, the high 4 bits to column j + 16; a code q stands for
 * (q - 8) * d.  Codes are stored [rows][cols/2] bytes, scales [rows][cols/32]. */
static int32_t q4_0_code(const void* w, int32_t cols, int32_t r, int32_t c) {
  const uint8_t* row = (const uint8_t*)w + (size_t)r * (cols / 2);
  const int32_t blk = c / 32, j = c % 32;
  const uint8_t byte = row[blk * 16 + (j % 16)];
  return (int32_t)(j < 16 ? (byte & 15) : (byte >> 4)) - 8;
}

static double q4_0_scale(const void* s, int32_t cols, int32_t r, int32_t c) {
  return orc_fp16_to_double(((const uint16_t*)s)[(size_t)r * (cols / 32) + c / 32]);
}

void orc_dequant_row(int32_t wfmt, const void* w, const void* s, int32_t cols, int32_t r,
                     float* out) {
  if (wfmt == ORC_W_INT8_ROW) {
    const int8_t* q = (const int8_t*)w + (size_t)r * cols;
    float sc = ((const float*)s)[r];
    for (int32_t c = 0; c < cols; c++) out[c] = (float)q[c] * sc;
  } else if (wfmt == ORC_W_Q8_0) {
    const int8_t* q = (const int8_t*)w + (size_t)r * cols;
    const uint16_t* d = (const uint16_t*)s + (size_t)r * (cols / 32);
    for (int32_t c = 0; c < cols; c++) out[c] = (float)q[c] * (float)orc_fp16_to_double(d[c / 32]);
  } else if (wfmt == ORC_W_Q4_0) {
    for (int32_t c = 0; c < cols; c++) out[c] = (float)q4_0_code(w, cols, r, c) * (float)q4_0_scale(s, cols, r, c);
  } else {
    const uint16_t* b = (const uint16_t*)w + (size_t)r * cols;
    for (int32_t c = 0; c < cols; c++) out[c] = (float)orc_bf16_to_double(b[c]);
  }
}

static double row_dot(int32_t wfmt, const void* w, const void* s, int32_t cols, int32_t r,
                      const double* x) {
  if (wfmt == ORC_W_INT8_ROW) {
    const int8_t* q = (const int8_t*)w + (size_t)r * cols;
    double acc = 0.0;
    for (int32_t c = 0; c < cols; c++) acc += (double)q[c] * x[c];
    return (double)((const float*)s)[r] * acc; /* scale applied after the dot */
  }
  if (wfmt == ORC_W_Q8_0) {
    const int8_t* q = (const int8_t*)w + (size_t)r * cols;
    const uint16_t* d = (const uint16_t*)s + (size_t)r * (cols / 32);
    double acc = 0.0;
    for (int32_t b = 0; b < cols / 32; b++) {
      double part = 0.0;
      for (int32_t c = b * 32; c < b * 32 + 32; c++) part += (double)q[c] * x[c];
      acc += orc_fp16_to_double(d[b]) * part;
    }
    return acc;
  }
  if (wfmt == ORC_W_Q4_0) {
    double acc = 0.0;
    for (int32_t b = 0; b < cols / 32; b++) {
      double part = 0.0;
      for (int32_t c = b * 32; c < b * 32 + 32; c++) part += (double)q4_0_code(w, cols, r, c) * x[c];
      acc += q4_0_scale(s, cols, r, b * 32) * part;
    }
    return acc;
  }
  const uint16_t* bw = (const uint16_t*)w + (size_t)r * cols;
  double acc = 0.0;
  for (int32_t c = 0; c < cols; c++) acc += orc_bf16_to_double(bw[c]) * x[c];
  return acc;
}

void orc_gemv(int32_t wfmt, const void* w, const void* s, int32_t rows, int32_t cols,
              const double* x, double* out) {
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < rows; r++) out[r] = row_dot(wfmt, w, s, cols, r, x);
}

void orc_rope(double* v, int32_t d, int32_t pos, double theta) {
  int32_t half = d / 2;
  for (int32_t i = 0; i < half; i++) {
    double f = pow(theta, -2.0 * (double)i / (double)d);
    double a = (double)pos * f;
    double c = cos(a), sn = sin(a);
    double u = v[i], w = v[i + half];
    v[i] = u * c - w * sn;
    v[i + half] = u * sn + w * c;
  }
}

void orc_attention(const double* q, int32_t hq, int32_t hkv, int32_t d, int32_t n_pos,
                   const double* K, const double* V, double* out) {
  int32_t G = hq / hkv;
  double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
  for (int32_t h = 0; h < hq; h++) {
    int32_t j = h / G;
    double* sc = (double*)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
    double m = -INFINITY;
    for (int32_t t = 0; t < n_pos; t++) {
      const double* k = K + ((size_t)t * hkv + j) * d;
      double dot = 0.0;
      for (int32_t i = 0; i < d; i++) dot += q[(size_t)h * d + i] * k[i];
      sc[t] = dot * scale;
      if (sc[t] > m) m = sc[t];
    }
    double sum = 0.0;
    for (int32_t t = 0; t < n_pos; t++) {
      sc[t] = exp(sc[t] - m);
      sum += sc[t];
    }
    for (int32_t i = 0; i < d; i++) {
      double o = 0.0;
      for (int32_t t = 0; t < n_pos; t++) o += (sc[t] / sum) * V[((size_t)t * hkv + j) * d + i];
      out[(size_t)h * d + i] = o;
    }
    free(sc);
  }
}

/* attention over the positions t < n_pos with keep[t] != 0; prob (may be NULL) gets each
 * attended position's softmax probability added, summed over the query heads */
void orc_attention_kept(const double* q, int32_t hq, int32_t hkv, int32_t d, int32_t n_pos,
                        const double* K, const double* V, const uint8_t* keep, double* out,
                        double* prob) {
  int32_t G = hq / hkv;
  double scale = 1.0 / sqrt((double)d);
  double* p = (double*)malloc(sizeof(double) * (size_t)hq * (size_t)(n_pos > 0 ? n_pos : 1));
#pragma omp parallel for schedule(static)
  for (int32_t h = 0; h < hq; h++) {
    int32_t j = h / G;
    double* sc = p + (size_t)h * n_pos;
    double m = -INFINITY;
    for (int32_t t = 0; t < n_pos; t++) {
      if (!keep[t]) continue;
      const double* k = K + ((size_t)t * hkv + j) * d;
      double dot = 0.0;
      for (int32_t i = 0; i < d; i++) dot += q[(size_t)h * d + i] * k[i];
      sc[t] = dot * scale;
      if (sc[t] > m) m = sc[t];
    }
    double sum = 0.0;
    for (int32_t t = 0; t < n_pos; t++) {
      sc[t] = keep[t] ? exp(sc[t] - m) : 0.0;
      sum += sc[t];
    }
    for (int32_t t = 0; t < n_pos; t++) sc[t] /= sum;
    for (int32_t i = 0; i < d; i++) {
      double o = 0.0;
      for (int32_t t = 0; t < n_pos; t++)
        if (keep[t]) o += sc[t] * V[((size_t)t * hkv + j) * d + i];
      out[(size_t)h * d + i] = o;
    }
  }
  if (prob)
    for (int32_t h = 0; h < hq; h++)
      for (int32_t t = 0; t < n_pos; t++) prob[t] += p[(size_t)h * n_pos + t];
  free(p);
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

int32_t orc_argmax_f32(const float* v, int32_t n) {
  if (n <= 0) return -1;
  int32_t best = 0;
  for (int32_t i = 0; i < n; i++) {
    if (isnan(v[i])) return -2;
    if (v[i] > v[best]) best = i;
  }
  return best;
}

void orc_kv_quant_i8(const double* x, int32_t d, int8_t* q, uint16_t* s16) {
  double amax = 0.0;
  for (int32_t i = 0; i < d; i++)
    if (fabs(x[i]) > amax) amax = fabs(x[i]);
  uint16_t h = orc_double_to_fp16(amax / 127.0);
  double s = orc_fp16_to_double(h);
  for (int32_t i = 0; i < d; i++) {
    double c = (s == 0.0) ? 0.0 : nearbyint(x[i] / s);
    if (c > 127.0) c = 127.0;
    if (c < -127.0) c = -127.0;
    q[i] = (int8_t)c;
  }
  *s16 = h;
}

/* ------------------------------------------------------------------------------------ */
/* model                                                                                */
/* ------------------------------------------------------------------------------------ */

typedef struct { const void* w; const void* s; int32_t rows, cols; } mat_t;

typedef struct {
  mat_t wq, wk, wv, wo, w_gate, w_up, w_down;
  const float *attn_norm, *ffn_norm;
} layer_t;

typedef struct {
  void* k;        /* [L][max_ctx][hkv][d] native encoding */
  void* v;
  uint16_t* ks;   /* [L][max_ctx][hkv] for int8 */
  uint16_t* vs;
} kv_t;

struct orc_model {
  orc_cfg c;
  layer_t* layers;
  mat_t tok_emb, lm_head;
  const float* final_norm;
  kv_t* kv; /* [max_seqs], allocated on first use */
};

static size_t kv_elem_size(int32_t kvfmt) {
  return kvfmt == ORC_KV_F32 ? 4 : (kvfmt == ORC_KV_BF16 ? 2 : 1);
}

orc_model* orc_create(const orc_cfg* cfg) {
  const orc_cfg* c = cfg;
  if (c->dim <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->head_dim > 1024 || (c->head_dim % 2) || c->ffn_dim <= 0 || c->vocab <= 0 ||
      (c->n_q_heads % c->n_kv_heads) || c->max_ctx <= 0 || c->max_seqs <= 0)
    return NULL;
  if ((c->wfmt == ORC_W_Q8_0 || c->wfmt == ORC_W_Q4_0) && ((c->dim % 32) || (c->ffn_dim % 32) ||
                                ((c->n_q_heads * c->head_dim) % 32)))
    return NULL;
  orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
  m->c = *cfg;
  m->layers = (layer_t*)calloc((size_t)c->n_layers, sizeof(layer_t));
  m->kv = (kv_t*)calloc((size_t)c->max_seqs, sizeof(kv_t));
  return m;
}

void orc_destroy(orc_model* m) {
  if (!m) return;
  for (int32_t s = 0; s < m->c.max_seqs; s++) {
    free(m->kv[s].k); free(m->kv[s].v); free(m->kv[s].ks); free(m->kv[s].vs);
  }
  free(m->kv);
  free(m->layers);
  free(m);
}

int32_t orc_set_tensor(orc_model* m, const char* name, const void* p0, const void* p1) {
  const orc_cfg* c = &m->c;
  int32_t qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  mat_t mt = {p0, p1, 0, 0};
  if (!strcmp(name, "tok_emb")) { mt.rows = c->vocab; mt.cols = c->dim; m->tok_emb = mt; return 0; }
  if (!strcmp(name, "lm_head")) { mt.rows = c->vocab; mt.cols = c->dim; m->lm_head = mt; return 0; }
  if (!strcmp(name, "final_norm")) { m->final_norm = (const float*)p0; return 0; }
  int li = -1, n = 0;
  char field[32];
  if (sscanf(name, "L%d.%31s%n", &li, field, &n) != 2 || li < 0 || li >= c->n_layers) return -1;
  layer_t* L = &m->layers[li];
  if (!strcmp(field, "attn_norm")) { L->attn_norm = (const float*)p0; return 0; }
  if (!strcmp(field, "ffn_norm")) { L->ffn_norm = (const float*)p0; return 0; }
  if (!strcmp(field, "wq")) { mt.rows = qd; mt.cols = c->dim; L->wq = mt; return 0; }
  if (!strcmp(field, "wk")) { mt.rows = kvd; mt.cols = c->dim; L->wk = mt; return 0; }
  if (!strcmp(field, "wv")) { mt.rows = kvd; mt.cols = c->dim; L->wv = mt; return 0; }
  if (!strcmp(field, "wo")) { mt.rows = c->dim; mt.cols = qd; L->wo = mt; return 0; }
  if (!strcmp(field, "w_gate")) { mt.rows = c->ffn_dim; mt.cols = c->dim; L->w_gate = mt; return 0; }
  if (!strcmp(field, "w_up")) { mt.rows = c->ffn_dim; mt.cols = c->dim; L->w_up = mt; return 0; }
  if (!strcmp(field, "w_down")) { mt.rows = c->dim; mt.cols = c->ffn_dim; L->w_down = mt; return 0; }
  return -1;
}

static int mat_ok(const mat_t* t, int32_t wfmt) {
  return t->w && (wfmt == ORC_W_BF16 || t->s) && t->rows > 0;
}

int32_t orc_ready(const orc_model* m) {
  int32_t f = m->c.wfmt;
  if (!mat_ok(&m->tok_emb, f) || !m->final_norm) return 0;
  if (!m->c.tied && !mat_ok(&m->lm_head, f)) return 0;
  for (int32_t l = 0; l < m->c.n_layers; l++) {
    const layer_t* L = &m->layers[l];
    if (!L->attn_norm || !L->ffn_norm || !mat_ok(&L->wq, f) || !mat_ok(&L->wk, f) ||
        !mat_ok(&L->wv, f) || !mat_ok(&L->wo, f) || !mat_ok(&L->w_gate, f) ||
        !mat_ok(&L->w_up, f) || !mat_ok(&L->w_down, f))
      return 0;
  }
  return 1;
}

static int kv_alloc(orc_model* m, int32_t seq) {
  kv_t* kv = &m->kv[seq];
  if (kv->k) return 0;
  const orc_cfg* c = &m->c;
  size_t per = (size_t)c->n_layers * c->max_ctx * c->n_kv_heads * c->head_dim;
  size_t es = kv_elem_size(c->kvfmt);
  kv->k = calloc(per, es);
  kv->v = calloc(per, es);
  if (c->kvfmt == ORC_KV_I8) {
    size_t ns = (size_t)c->n_layers * c->max_ctx * c->n_kv_heads;
    kv->ks = (uint16_t*)calloc(ns, 2);
    kv->vs = (uint16_t*)calloc(ns, 2);
  }
  return (kv->k && kv->v && (c->kvfmt != ORC_KV_I8 || (kv->ks && kv->vs))) ? 0 : -1;
}

/* element offset of (layer, pos, head, 0) in a sequence's cache */
static size_t kv_off(const orc_cfg* c, int32_t layer, int32_t pos, int32_t head) {
  return (((size_t)layer * c->max_ctx + pos) * c->n_kv_heads + head) * c->head_dim;
}
static size_t ks_off(const orc_cfg* c, int32_t layer, int32_t pos, int32_t head) {
  return ((size_t)layer * c->max_ctx + pos) * c->n_kv_heads + head;
}

/* store one position's k or v (double, [hkv][d]) with the cache's rounding */
static void kv_store(const orc_cfg* c, void* base, uint16_t* sbase, int32_t layer, int32_t pos,
                     const double* x) {
  for (int32_t h = 0; h < c->n_kv_heads; h++) {
    const double* xh = x + (size_t)h * c->head_dim;
    size_t o = kv_off(c, layer, pos, h);
    if (c->kvfmt == ORC_KV_F32) {
      for (int32_t i = 0; i < c->head_dim; i++) ((float*)base)[o + i] = (float)xh[i];
    } else if (c->kvfmt == ORC_KV_BF16) {
      for (int32_t i = 0; i < c->head_dim; i++) ((uint16_t*)base)[o + i] = orc_double_to_bf16(xh[i]);
    } else {
      orc_kv_quant_i8(xh, c->head_dim, (int8_t*)base + o, sbase + ks_off(c, layer, pos, h));
    }
  }
}

/* decode stored positions [0, n) of one layer into doubles [n][hkv][d] */
static void kv_load(const orc_cfg* c, const void* base, const uint16_t* sbase, int32_t layer,
                    int32_t pos0, int32_t n, double* out) {
  int32_t hd = c->head_dim;
  for (int32_t t = 0; t < n; t++)
    for (int32_t h = 0; h < c->n_kv_heads; h++) {
      size_t o = kv_off(c, layer, pos0 + t, h);
      double* dst = out + ((size_t)t * c->n_kv_heads + h) * hd;
      if (c->kvfmt == ORC_KV_F32) {
        for (int32_t i = 0; i < hd; i++) dst[i] = (double)((const float*)base)[o + i];
      } else if (c->kvfmt == ORC_KV_BF16) {
        for (int32_t i = 0; i < hd; i++) dst[i] = orc_bf16_to_double(((const uint16_t*)base)[o + i]);
      } else {
        double s = orc_fp16_to_double(sbase[ks_off(c, layer, pos0 + t, h)]);
        for (int32_t i = 0; i < hd; i++) dst[i] = (double)((const int8_t*)base)[o + i] * s;
      }
    }
}

static void embed_row(const orc_model* m, int32_t token, double* x) {
  float* row = (float*)malloc(sizeof(float) * (size_t)m->c.dim);
  orc_dequant_row(m->c.wfmt, m->tok_emb.w, m->tok_emb.s, m->c.dim, token, row);
  for (int32_t i = 0; i < m->c.dim; i++) x[i] = (double)row[i];
  free(row);
}

static void gemv_mat(const orc_model* m, const mat_t* t, const double* x, double* out) {
  orc_gemv(m->c.wfmt, t->w, t->s, t->rows, t->cols, x, out);
}

static void round_vec(double* v, int32_t n, int32_t act) {
  for (int32_t i = 0; i < n; i++) v[i] = orc_round_act(v[i], act);
}

typedef struct { double *xn, *q, *k, *v, *o, *tmp, *a, *b, *h; } scratch_t;

static void scratch_init(scratch_t* s, const orc_cfg* c) {
  int32_t qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  int32_t big = c->dim > c->ffn_dim ? c->dim : c->ffn_dim;
  if (c->vocab > big) big = c->vocab;
  s->xn = (double*)calloc((size_t)c->dim, 8);
  s->q = (double*)calloc((size_t)qd, 8);
  s->k = (double*)calloc((size_t)kvd, 8);
  s->v = (double*)calloc((size_t)kvd, 8);
  s->o = (double*)calloc((size_t)qd, 8);
  s->tmp = (double*)calloc((size_t)big, 8);
  s->a = (double*)calloc((size_t)c->ffn_dim, 8);
  s->b = (double*)calloc((size_t)c->ffn_dim, 8);
  s->h = (double*)calloc((size_t)c->ffn_dim, 8);
}

static void scratch_free(scratch_t* s) {
  free(s->xn); free(s->q); free(s->k); free(s->v); free(s->o); free(s->tmp);
  free(s->a); free(s->b); free(s->h);
}

/* logits of the residual stream x: final RMSNorm, rounding, LM head (tok_emb when tied) */
static int32_t head_logits(const orc_model* m, const double* x, scratch_t* s, float* logits) {
  const orc_cfg* c = &m->c;
  orc_rmsnorm(x, m->final_norm, c->dim, c->rms_eps, s->xn);
  round_vec(s->xn, c->dim, c->act);
  const mat_t* head = c->tied ? &m->tok_emb : &m->lm_head;
  double* lg = (double*)malloc(sizeof(double) * (size_t)c->vocab);
  gemv_mat(m, head, s->xn, lg);
  float* l32 = logits ? logits : (float*)malloc(sizeof(float) * (size_t)c->vocab);
  for (int32_t i = 0; i < c->vocab; i++) l32[i] = (float)lg[i];
  int32_t next = orc_argmax_f32(l32, c->vocab);
  if (!logits) free(l32);
  free(lg);
  return next;
}

/* the feed-forward half of a layer: x += W_down (silu(W_gate xn) * (W_up xn));
 * xn2_pre / h_pre (may be NULL) receive the values before activation rounding */
static void ffn_half(const orc_model* m, const layer_t* L, double* x, scratch_t* s,
                     double* xn2_pre, double* h_pre) {
  const orc_cfg* c = &m->c;
  orc_rmsnorm(x, L->ffn_norm, c->dim, c->rms_eps, s->xn);
  if (xn2_pre) memcpy(xn2_pre, s->xn, sizeof(double) * (size_t)c->dim);
  round_vec(s->xn, c->dim, c->act);
  gemv_mat(m, &L->w_gate, s->xn, s->a);
  gemv_mat(m, &L->w_up, s->xn, s->b);
  for (int32_t i = 0; i < c->ffn_dim; i++) {
    const double hv = orc_silu(s->a[i]) * s->b[i];
    if (h_pre) h_pre[i] = hv;
    s->h[i] = orc_round_act(hv, c->act);
  }
  gemv_mat(m, &L->w_down, s->h, s->tmp);
  for (int32_t i = 0; i < c->dim; i++) x[i] += s->tmp[i];
}

int32_t orc_trace_len(const orc_model* m) {
  const orc_cfg* c = &m->c;
  const int32_t qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  return 5 * c->dim + 2 * qd + 2 * kvd + c->ffn_dim;
}

/* xn -> q, k, v with RoPE applied to every q and k head at position pos */
static void qkv_rope(const orc_model* m, const layer_t* L, int32_t pos, scratch_t* s) {
  const orc_cfg* c = &m->c;
  gemv_mat(m, &L->wq, s->xn, s->q);
  gemv_mat(m, &L->wk, s->xn, s->k);
  gemv_mat(m, &L->wv, s->xn, s->v);
  for (int32_t h = 0; h < c->n_q_heads; h++) orc_rope(s->q + (size_t)h * c->head_dim, c->head_dim, pos, c->rope_theta);
  for (int32_t h = 0; h < c->n_kv_heads; h++) orc_rope(s->k + (size_t)h * c->head_dim, c->head_dim, pos, c->rope_theta);
}

static int32_t step_impl(orc_model* m, int32_t seq, int32_t token, int32_t pos, float* logits,
                         double* hidden, double* trace, const uint8_t* keep, int32_t score_layers,
                         double* scores);

int32_t orc_step(orc_model* m, int32_t seq, int32_t token, int32_t pos, float* logits,
                 double* hidden, double* trace) {
  return step_impl(m, seq, token, pos, logits, hidden, trace, NULL, 0, NULL);
}

int32_t orc_step_kept(orc_model* m, int32_t seq, int32_t token, int32_t pos, const uint8_t* keep,
                      int32_t score_layers, double* scores, float* logits) {
  if (!keep || pos < 0 || !keep[pos]) return -15;
  return step_impl(m, seq, token, pos, logits, NULL, NULL, keep, score_layers, scores);
}

static int32_t step_impl(orc_model* m, int32_t seq, int32_t token, int32_t pos, float* logits,
                         double* hidden, double* trace, const uint8_t* keep, int32_t score_layers,
                         double* scores) {
  const orc_cfg* c = &m->c;
  if (!orc_ready(m)) return -10;
  if (seq < 0 || seq >= c->max_seqs) return -11;
  if (pos < 0 || pos >= c->max_ctx) return -12;
  if (token < 0 || token >= c->vocab) return -13;
  if (kv_alloc(m, seq)) return -14;
  kv_t* kv = &m->kv[seq];
  int32_t qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  double* x = (double*)malloc(sizeof(double) * (size_t)c->dim);
  double* Kd = (double*)malloc(sizeof(double) * (size_t)(pos + 1) * kvd);
  double* Vd = (double*)malloc(sizeof(double) * (size_t)(pos + 1) * kvd);
  scratch_t s;
  scratch_init(&s, c);

  embed_row(m, token, x);
  if (hidden) memcpy(hidden, x, sizeof(double) * (size_t)c->dim);
  const int32_t D = c->dim;
  const size_t dsz = sizeof(double);
  for (int32_t l = 0; l < c->n_layers; l++) {
    const layer_t* L = &m->layers[l];
    /* trace record fields of this layer (NULL when not tracing) */
    double* t_x_in = trace ? trace + (size_t)l * orc_trace_len(m) : NULL;
    double* t_xn = trace ? t_x_in + D : NULL;
    double* t_q = trace ? t_xn + D : NULL;
    double* t_k = trace ? t_q + qd : NULL;
    double* t_v = trace ? t_k + kvd : NULL;
    double* t_o = trace ? t_v + kvd : NULL;
    double* t_xmid = trace ? t_o + qd : NULL;
    double* t_xn2 = trace ? t_xmid + D : NULL;
    double* t_h = trace ? t_xn2 + D : NULL;
    double* t_xout = trace ? t_h + c->ffn_dim : NULL;
    if (trace) memcpy(t_x_in, x, dsz * D);
    orc_rmsnorm(x, L->attn_norm, c->dim, c->rms_eps, s.xn);
    if (trace) memcpy(t_xn, s.xn, dsz * D);
    round_vec(s.xn, c->dim, c->act);
    qkv_rope(m, L, pos, &s);
    if (trace) {
      memcpy(t_q, s.q, dsz * qd);
      memcpy(t_k, s.k, dsz * kvd);
      memcpy(t_v, s.v, dsz * kvd);
    }
    kv_store(c, kv->k, kv->ks, l, pos, s.k);
    kv_store(c, kv->v, kv->vs, l, pos, s.v);
    kv_load(c, kv->k, kv->ks, l, 0, pos + 1, Kd);
    kv_load(c, kv->v, kv->vs, l, 0, pos + 1, Vd);
    if (keep)
      orc_attention_kept(s.q, c->n_q_heads, c->n_kv_heads, c->head_dim, pos + 1, Kd, Vd, keep, s.o,
                     l >= c->n_layers - score_layers ? scores : NULL);
    else
      orc_attention(s.q, c->n_q_heads, c->n_kv_heads, c->head_dim, pos + 1, Kd, Vd, s.o);
    if (trace) memcpy(t_o, s.o, dsz * qd);
    round_vec(s.o, qd, c->act);
    gemv_mat(m, &L->wo, s.o, s.tmp);
    for (int32_t i = 0; i < c->dim; i++) x[i] += s.tmp[i];
    if (trace) memcpy(t_xmid, x, dsz * D);
    ffn_half(m, L, x, &s, t_xn2, t_h);
    if (trace) memcpy(t_xout, x, dsz * D);
    if (hidden) memcpy(hidden + (size_t)(l + 1) * c->dim, x, sizeof(double) * (size_t)c->dim);
  }
  int32_t next = head_logits(m, x, &s, logits);
  scratch_free(&s);
  free(x); free(Kd); free(Vd);
  return next;
}

int32_t orc_kv_write(orc_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                     const void* k, const void* v, const uint16_t* ks, const uint16_t* vs) {
  const orc_cfg* c = &m->c;
  if (seq < 0 || seq >= c->max_seqs || layer < 0 || layer >= c->n_layers || pos0 < 0 || n < 0 ||
      pos0 + n > c->max_ctx)
    return -1;
  if (c->kvfmt == ORC_KV_I8 && (!ks || !vs)) return -1;
  if (kv_alloc(m, seq)) return -2;
  kv_t* kv = &m->kv[seq];
  size_t es = kv_elem_size(c->kvfmt);
  size_t row = (size_t)c->n_kv_heads * c->head_dim;
  for (int32_t t = 0; t < n; t++) {
    size_t o = kv_off(c, layer, pos0 + t, 0);
    memcpy((char*)kv->k + o * es, (const char*)k + (size_t)t * row * es, row * es);
    memcpy((char*)kv->v + o * es, (const char*)v + (size_t)t * row * es, row * es);
    if (c->kvfmt == ORC_KV_I8) {
      size_t so = ks_off(c, layer, pos0 + t, 0);
      memcpy(kv->ks + so, ks + (size_t)t * c->n_kv_heads, 2 * (size_t)c->n_kv_heads);
      memcpy(kv->vs + so, vs + (size_t)t * c->n_kv_heads, 2 * (size_t)c->n_kv_heads);
    }
  }
  return 0;
}

int32_t orc_kv_read(const orc_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                    double* k, double* v) {
  const orc_cfg* c = &m->c;
  if (seq < 0 || seq >= c->max_seqs || layer < 0 || layer >= c->n_layers || pos0 < 0 || n < 0 ||
      pos0 + n > c->max_ctx || !m->kv[seq].k)
    return -1;
  kv_load(c, m->kv[seq].k, m->kv[seq].ks, layer, pos0, n, k);
  kv_load(c, m->kv[seq].v, m->kv[seq].vs, layer, pos0, n, v);
  return 0;
}

int32_t orc_kv_read_raw(const orc_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                        void* k, void* v, uint16_t* ks, uint16_t* vs) {
  const orc_cfg* c = &m->c;
  if (seq < 0 || seq >= c->max_seqs || layer < 0 || layer >= c->n_layers || pos0 < 0 || n < 0 ||
      pos0 + n > c->max_ctx || !m->kv[seq].k)
    return -1;
  const kv_t* kv = &m->kv[seq];
  size_t es = kv_elem_size(c->kvfmt);
  size_t row = (size_t)c->n_kv_heads * c->head_dim;
  for (int32_t t = 0; t < n; t++) {
    size_t o = kv_off(c, layer, pos0 + t, 0);
    memcpy((char*)k + (size_t)t * row * es, (const char*)kv->k + o * es, row * es);
    memcpy((char*)v + (size_t)t * row * es, (const char*)kv->v + o * es, row * es);
    if (c->kvfmt == ORC_KV_I8 && ks && vs) {
      size_t so = ks_off(c, layer, pos0 + t, 0);
      memcpy(ks + (size_t)t * c->n_kv_heads, kv->ks + so, 2 * (size_t)c->n_kv_heads);
      memcpy(vs + (size_t)t * c->n_kv_heads, kv->vs + so, 2 * (size_t)c->n_kv_heads);
    }
  }
  return 0;
}

int32_t orc_full_forward(orc_model* m, const int32_t* tokens, int32_t n, float* logits,
                         double* hidden) {
  const orc_cfg* c = &m->c;
  if (!orc_ready(m)) return -10;
  if (n <= 0 || n > c->max_ctx) return -12;
  for (int32_t t = 0; t < n; t++)
    if (tokens[t] < 0 || tokens[t] >= c->vocab) return -13;
  int32_t D = c->dim, hd = c->head_dim, hkv = c->n_kv_heads;
  int32_t qd = c->n_q_heads * hd, kvd = hkv * hd;
  double* X = (double*)malloc(sizeof(double) * (size_t)n * D);   /* residual, every position */
  double* Q = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* K = (double*)malloc(sizeof(double) * (size_t)n * kvd); /* rounded as stored */
  double* V = (double*)malloc(sizeof(double) * (size_t)n * kvd);
  scratch_t s;
  scratch_init(&s, c);
  for (int32_t t = 0; t < n; t++) embed_row(m, tokens[t], X + (size_t)t * D);
  if (hidden) memcpy(hidden, X + (size_t)(n - 1) * D, sizeof(double) * (size_t)D);
  for (int32_t l = 0; l < c->n_layers; l++) {
    const layer_t* L = &m->layers[l];
    for (int32_t t = 0; t < n; t++) {
      orc_rmsnorm(X + (size_t)t * D, L->attn_norm, D, c->rms_eps, s.xn);
      round_vec(s.xn, D, c->act);
      qkv_rope(m, L, t, &s);
      memcpy(Q + (size_t)t * qd, s.q, sizeof(double) * (size_t)qd);
      for (int32_t h = 0; h < hkv; h++) {
        const double* kh = s.k + (size_t)h * hd;
        const double* vh = s.v + (size_t)h * hd;
        double* kd = K + (size_t)t * kvd + (size_t)h * hd;
        double* vd = V + (size_t)t * kvd + (size_t)h * hd;
        if (c->kvfmt == ORC_KV_I8) {
          int8_t qb[1024];
          uint16_t sc;
          orc_kv_quant_i8(kh, hd, qb, &sc);
          for (int32_t i = 0; i < hd; i++) kd[i] = (double)qb[i] * orc_fp16_to_double(sc);
          orc_kv_quant_i8(vh, hd, qb, &sc);
          for (int32_t i = 0; i < hd; i++) vd[i] = (double)qb[i] * orc_fp16_to_double(sc);
        } else {
          int32_t a = (c->kvfmt == ORC_KV_BF16) ? ORC_ACT_BF16 : ORC_ACT_F32;
          for (int32_t i = 0; i < hd; i++) {
            kd[i] = orc_round_act(kh[i], a);
            vd[i] = orc_round_act(vh[i], a);
          }
        }
      }
    }
    for (int32_t t = 0; t < n; t++) {
      double* x = X + (size_t)t * D;
      orc_attention(Q + (size_t)t * qd, c->n_q_heads, hkv, hd, t + 1, K, V, s.o); /* causal */
      round_vec(s.o, qd, c->act);
      gemv_mat(m, &L->wo, s.o, s.tmp);
      for (int32_t i = 0; i < D; i++) x[i] += s.tmp[i];
      ffn_half(m, L, x, &s, NULL, NULL);
    }
    if (hidden) memcpy(hidden + (size_t)(l + 1) * D, X + (size_t)(n - 1) * D, sizeof(double) * (size_t)D);
  }
  int32_t next = head_logits(m, X + (size_t)(n - 1) * D, &s, logits);
  scratch_free(&s);
  free(X); free(Q); free(K); free(V);
  return next;
}

void orc_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
