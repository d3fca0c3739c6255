/* oracle.h -- plain CPU oracle of the Llama-family per-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may call it.  It shares no code, header or table with the GPU library and
 * never calls it.
 *
 * Every quantity is computed in IEEE double, except at the storage points a model
 * configuration fixes:
 *   - weights are read in their stored encodings (int8 + fp32 row scale, Q8_0, bf16);
 *   - activations rounded to the model's activation type (fp32 or bf16, round to nearest
 *     even) at: each RMSNorm output, the attention output, the SwiGLU output;
 *   - keys/values rounded to the KV type when written to the cache (fp32, bf16, or int8
 *     with one fp16 scale per token and KV head);
 *   - logits stored as fp32; greedy argmax taken on the fp32 logits, lowest index on ties.
 * The residual stream, post-RoPE queries, scores, softmax and all sums stay in double.
 *
 * Sources ("page" = the web page, then its section):
 *   - "从 smollm3.go 看 LLM inference": layer structure (Transformer block), Q/K/V
 *     projections and attention over positions [0, pos] (self-attention), GQA head map
 *     kvHead = h / kvMul (multi-head attention), logits projection and greedy sampling
 *     (sampling), KV cache layout [layer][position][kvDim] (KV cache), int8 row scales
 *     (int8 weight-only quantization).
 *   - "扔掉 vLLM！從零構建 Qwen3-8B 推理引擎": 4.2.2 pre-norm layer, 4.4.2 GQA decode with
 *     1/sqrt(d_head) scaling, 4.3.1 paged blocks.
 *   - "Go 语言原本" 20.2.3 row-major layout, 20.2.4 Q8_0 (one f16 scale per 32 int8).
 *   - nxmr.cn C17 engine article: 4.3 prefill/decode and tied LM head, 4.4 half-split RoPE
 *     and GQA, 4.5 SwiGLU with SiLU, 4.6 greedy sampling.
 */
#ifndef ORC_ORACLE_H
#define ORC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_W_INT8_ROW 0
#define ORC_W_Q8_0     1
#define ORC_W_BF16     2
#define ORC_W_Q4_0     3
#define ORC_ACT_F32    0
#define ORC_ACT_BF16   1
#define ORC_KV_F32     0
#define ORC_KV_BF16    1
#define ORC_KV_I8      2

typedef struct {
  int32_t dim, n_layers, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  double  rms_eps, rope_theta;
  int32_t tied, wfmt, act, kvfmt, max_ctx, max_seqs;
} orc_cfg;

typedef struct orc_model orc_model;

/* ---- scalar encodings ---- */
double   orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double x);      /* round to nearest even */
double   orc_fp16_to_double(uint16_t h);
uint16_t orc_double_to_fp16(double x);      /* round to nearest even */
double   orc_round_act(double x, int32_t act);
void     orc_round_act_n(const double* x, int32_t n, int32_t act, double* out);

/* ---- single operations on plain arrays ---- */
/* out[i] = x[i] / sqrt(mean(x^2) + eps) * g[i] */
void    orc_rmsnorm(const double* x, const float* g, int32_t n, double eps, double* out);
/* fp32 value of one stored weight row: int8-row q*s, Q8_0 q*d (one fp32 product each),
 * bf16 widened.  w/s as for orc_gemv. */
void    orc_dequant_row(int32_t wfmt, const void* w, const void* s, int32_t cols,
                        int32_t r, float* out);
/* out[r] = sum_c W[r,c] x[c] in the stored encoding: int8-row s_r * sum q x;
 * Q8_0 sum_b d_b sum_{c in b} q x; bf16 sum w x. */
void    orc_gemv(int32_t wfmt, const void* w, const void* s, int32_t rows, int32_t cols,
                 const double* x, double* out);
/* half-split rotation of one head vector of length d at position pos */
void    orc_rope(double* v, int32_t d, int32_t pos, double theta);
/* q [hq][d]; K, V [n_pos][hkv][d]; out [hq][d]; q head h reads kv head h / (hq/hkv) */
void    orc_attention(const double* q, int32_t hq, int32_t hkv, int32_t d, int32_t n_pos,
                      const double* K, const double* V, double* out);
/* orc_attention over the positions t < n_pos with keep[t] != 0 only; prob (may be NULL,
 * double [n_pos]) gets each attended position's softmax probability added, summed over the
 * query heads */
void    orc_attention_kept(const double* q, int32_t hq, int32_t hkv, int32_t d, int32_t n_pos,
                           const double* K, const double* V, const uint8_t* keep, double* out,
                           double* prob);
double  orc_silu(double z);
/* first index of the maximum; -1 if n <= 0, -2 if any value is NaN */
int32_t orc_argmax_f32(const float* v, int32_t n);
/* symmetric int8 code of one (token, head) vector: s = fp16(max|x|/127),
 * q = clamp(rint(x / s), -127, 127), s == 0 gives q == 0 */
void    orc_kv_quant_i8(const double* x, int32_t d, int8_t* q, uint16_t* s16);

/* ---- whole model ---- */
orc_model* orc_create(const orc_cfg* cfg);
void       orc_destroy(orc_model* m);
/* Binds a tensor by name (the caller keeps the memory alive).  Matrices: p0 = int8 codes or
 * bf16 bits, p1 = fp32 row scales (int8-row), fp16 block scales [rows][cols/32] (Q8_0) or
 * NULL (bf16).  Norm gains ("*_norm"): p0 = fp32 [dim]. */
int32_t    orc_set_tensor(orc_model* m, const char* name, const void* p0, const void* p1);
int32_t    orc_ready(const orc_model* m);
/* One decode step of sequence `seq` for `token` at position `pos`: writes K/V at pos,
 * attends over [0, pos].  logits (fp32 [vocab]) and hidden (double [(L+1)*dim]: the
 * residual stream after the embedding and after each layer) may be NULL.
 * trace (may be NULL) receives, per layer, the record
 *   x_in [D] | xn [D] | q [q_dim] | k [kv_dim] | v [kv_dim] | o [q_dim] | x_mid [D] |
 *   xn2 [D] | h [F] | x_out [D]
 * where xn, o, xn2 and h are the values before their activation rounding, q and k are
 * after RoPE, and k, v are before the KV rounding (orc_trace_len() doubles per layer).
 * Returns the greedy next token, or < 0 on error. */
int32_t    orc_step(orc_model* m, int32_t seq, int32_t token, int32_t pos,
                    float* logits, double* hidden, double* trace);
int32_t    orc_trace_len(const orc_model* m);
/* orc_step with a kept set (the Initial-Key KV cache of the C17 engine article, 5.3): the
 * token at `pos` attends only to the positions t <= pos with keep[t] != 0 (keep [pos + 1];
 * the new position is always attended).  In each of the last score_layers layers, the
 * softmax probability every attended position receives is added, summed over the query
 * heads, to scores[t] (double [pos + 1]; may be NULL).  Returns as orc_step. */
int32_t    orc_step_kept(orc_model* m, int32_t seq, int32_t token, int32_t pos, const uint8_t* keep,
                         int32_t score_layers, double* scores, float* logits);
/* Writes n positions of stored K/V (native encoding, [n][hkv][d]; scales [n][hkv] fp16
 * for int8) at pos0..pos0+n-1 of (seq, layer). */
int32_t    orc_kv_write(orc_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                        const void* k, const void* v, const uint16_t* ks, const uint16_t* vs);
/* Reads back stored K/V as decoded doubles [n][hkv][d]. */
int32_t    orc_kv_read(const orc_model* m, int32_t seq, int32_t layer, int32_t pos0, int32_t n,
                       double* k, double* v);
/* Reads stored K/V in the native encoding (same layout as orc_kv_write). */
int32_t    orc_kv_read_raw(const orc_model* m, int32_t seq, int32_t layer, int32_t pos0,
                           int32_t n, void* k, void* v, uint16_t* ks, uint16_t* vs);
/* Same arithmetic with no cache: every position's K/V recomputed from tokens[0..n-1]
 * layer by layer, causal attention; logits and hidden of the last position. */
int32_t    orc_full_forward(orc_model* m, const int32_t* tokens, int32_t n,
                            float* logits, double* hidden);
int32_t    orc_num_threads(void);
/* Sets the OpenMP thread count of later calls (n > 0). */
void       orc_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
