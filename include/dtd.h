/* dtd.h -- C ABI of libdtd.so, the MI355X (gfx950) decode step of a Llama-family
 * decoder-only transformer.
 *
 * What one decode step computes, per sequence (the pre-norm block described by
 * "从 smollm3.go 看 LLM inference", Transformer block and self-attention sections, and by
 * the Qwen3-8B engine article, 4.2.2):
 *   x = embed(token); for every layer: x += Wo . attn(rope(Wq . rmsnorm(x)), K, V);
 *   x += Wdown . (silu(Wgate . rmsnorm(x)) * (Wup . rmsnorm(x)));
 *   logits = Whead . rmsnorm(x); next = argmax(logits)  (greedy, lowest index on ties).
 * The interface mirrors the Qwen3-8B engine article's inner service (4.1.2: Prefill,
 * DecodeStep, ResetSeq, token ids only, the engine owns each seq_id's KV) and
 * smollm3.go's Forward(token, pos) / Prefill(tokens, startPos) (Prefill and Decode).
 *
 * Conventions for every entry point:
 *   - Returns dtd_status: 0 on success, < 0 on error.  Never throws, never aborts.
 *   - Everything is validated on the host before any work is enqueued; on error nothing
 *     changes and dtd_last_error() describes the problem.
 *   - `*_dev` pointers are device memory owned by the caller; they must stay valid until
 *     the enqueued work completes, which the caller observes by synchronising the stream
 *     given to dtd_create (the ownership rule of cgo-style boundaries, "Go 语言原本" 20.2.3:
 *     memory handed across may only be kept while the caller keeps it alive).
 *   - Host pointers are read during the call only.
 *   - The engine owns its copies of the weights, the KV block pool, block tables and
 *     work buffers.  One engine is driven from one host thread and one stream.
 *   - A HIP runtime failure returns DTD_E_HIP and leaves the engine unusable (destroy it).
 */
#ifndef DTD_H
#define DTD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DTD_ABI_VERSION 1

typedef enum {
  DTD_OK = 0,
  DTD_E_ARG = -1,          /* bad argument, shape, size, name or token id */
  DTD_E_STATE = -2,        /* call not valid in this state (e.g. no weights loaded) */
  DTD_E_NOSEQ = -3,        /* unknown seq_id */
  DTD_E_CTX = -4,          /* sequence would exceed max_ctx */
  DTD_E_KVFULL = -5,       /* no free KV block or sequence slot */
  DTD_E_OOM = -6,          /* device allocation failed */
  DTD_E_HIP = -7,          /* HIP runtime error; engine unusable */
  DTD_E_UNSUPPORTED = -8   /* configuration outside what the kernels implement */
} dtd_status;

/* weight storage (the offline export formats):
 *   INT8_ROW: int8 codes [rows][cols] + one fp32 scale per row; W[r][c] = q[r][c]*s[r]
 *             ("从 smollm3.go 看 LLM inference", int8 weight-only quantization);
 *   Q8_0:     int8 codes [rows][cols] + one fp16 scale per run of 32 columns
 *             [rows][cols/32] ("Go 语言原本" 20.2.4);
 *   BF16:     bf16 bit patterns [rows][cols];
 *   Q4_0:     4-bit codes in blocks of 32 columns, 16 bytes per block [rows][cols/2] (byte j
 *             of a block: column j in the low 4 bits, column j+16 in the high 4 bits), plus
 *             one fp16 scale per block [rows][cols/32]; W = (q - 8) * d ("Go 语言原本" 20.2.4). */
enum { DTD_W_INT8_ROW = 0, DTD_W_Q8_0 = 1, DTD_W_BF16 = 2, DTD_W_Q4_0 = 3 };
/* activation storage type at the rounding points: each RMSNorm output, the attention
 * output and the SwiGLU output.  The residual stream, queries, scores, softmax,
 * accumulators and logits are fp32 in every configuration. */
enum { DTD_ACT_F32 = 0, DTD_ACT_BF16 = 1 };
/* KV cache storage: fp32, bf16, or int8 codes with one fp16 scale per (token, KV head),
 * s = fp16(max|x|/127), q = clamp(rint(x/s), -127, 127). */
enum { DTD_KV_F32 = 0, DTD_KV_BF16 = 1, DTD_KV_I8 = 2 };

typedef struct {
  int32_t abi_version;        /* DTD_ABI_VERSION */
  int32_t dim;                /* model width D */
  int32_t n_layers;
  int32_t n_q_heads;          /* Hq; q_dim = Hq * head_dim <= 16384 */
  int32_t n_kv_heads;         /* Hkv, divides Hq; q head h reads kv head h / (Hq/Hkv) */
  int32_t head_dim;           /* d: a multiple of 4 in [8, 128] */
  int32_t ffn_dim;            /* F */
  int32_t vocab;              /* V */
  float   rms_eps;            /* added inside the square root */
  float   rope_theta;         /* half-split RoPE base: pair (i, i+d/2) turns by pos*theta^(-2i/d) */
  int32_t tied_embeddings;    /* 1: the LM head reuses tok_emb */
  int32_t wfmt;               /* DTD_W_* */
  int32_t act;                /* DTD_ACT_* */
  int32_t kvfmt;              /* DTD_KV_* */
  int32_t kv_block_size;      /* tokens per KV block (paged KV, Qwen3-8B engine article 4.3.1) */
  int32_t kv_num_blocks;      /* blocks in the pool, shared by all sequences and layers */
  int32_t max_seqs;           /* live sequences at once */
  int32_t max_ctx;            /* positions per sequence */
  int32_t max_batch;          /* sequences per decode_step call, <= 64 */
} dtd_config;

/* One named weight part for dtd_load_weights.  Names: "tok_emb", "lm_head" (absent when
 * tied), "final_norm", and per layer i "L{i}.attn_norm", "L{i}.wq", "L{i}.wk", "L{i}.wv",
 * "L{i}.wo", "L{i}.ffn_norm", "L{i}.w_gate", "L{i}.w_up", "L{i}.w_down", each followed by
 * a part suffix: ".q" int8 codes and ".s" scales (INT8_ROW, Q8_0), ".w" bf16 bits (BF16),
 * ".g" fp32 gains (norms).  Matrices are row-major [out][in]: wq [Hq*d][D],
 * wk/wv [Hkv*d][D], wo [D][Hq*d], w_gate/w_up [F][D], w_down [D][F], tok_emb/lm_head
 * [V][D].  nbytes must equal the exact size of the part. */
typedef struct {
  const char* name;
  const void* data;
  int64_t     nbytes;
  int32_t     on_device;      /* 0: host memory, 1: device memory */
} dtd_tensor;

/* Expected weight part, as reported by dtd_expected_tensors. */
typedef struct {
  char    name[48];
  int64_t nbytes;
  int32_t rows, cols;         /* matrix shape, or [1][D] for gains */
  int32_t elem;               /* bytes per element of this part: 1, 2 or 4 */
} dtd_tensor_spec;

typedef struct dtd_engine dtd_engine;

/* ---- host-only queries (no GPU needed) ------------------------------------------- */

/* Checks a configuration against what the kernels implement.  msg (may be NULL) gets a
 * NUL-terminated reason of at most msg_len bytes. */
dtd_status dtd_validate_config(const dtd_config* cfg, char* msg, int32_t msg_len);

/* Lists the weight parts dtd_load_weights expects for cfg.  Returns the count (and fills
 * at most cap entries of out, which may be NULL), or a dtd_status < 0 if cfg is invalid. */
int32_t dtd_expected_tensors(const dtd_config* cfg, dtd_tensor_spec* out, int32_t cap);

/* ---- lifecycle ---------------------------------------------------------------------- */

/* Creates an engine on the current HIP device: the KV block pool (fixed-size blocks shared
 * by all sequences, handed out from a free list: the paged KV cache of the Qwen3-8B engine
 * article, 4.3.1), per-sequence block tables, the RoPE tables and work buffers.  hip_stream
 * is a hipStream_t (NULL = the null stream); all work is enqueued on it.  The engine keeps
 * its own copy of *cfg.  Errors: DTD_E_ARG / DTD_E_UNSUPPORTED for a configuration
 * dtd_validate_config rejects, DTD_E_OOM when device memory runs out, DTD_E_HIP for another
 * HIP failure; *out is then NULL and dtd_last_error(NULL) has the reason. */
dtd_status dtd_create(const dtd_config* cfg, void* hip_stream, dtd_engine** out);

/* Copies every weight part into engine-owned device memory (repacked for the kernels).
 * All parts must be given in one call.  Loading fails closed, like the hardened model
 * loader of the nxmr.cn C17 engine article (4.1): a missing, unknown, duplicate or wrongly
 * sized part is rejected (DTD_E_ARG) before anything is copied, and the engine then holds
 * no weights (later steps fail with DTD_E_STATE).  t[i].data is host memory or, with
 * on_device = 1, device memory; nbytes is the part's exact size (dtd_expected_tensors).
 * Synchronous: the caller may free its buffers when it returns. */
dtd_status dtd_load_weights(dtd_engine* e, const dtd_tensor* t, int32_t n);

/* Appends n tokens (device int32 [n], each in [0, V)) to sequence seq_id, creating the
 * sequence if it is new, and writes the greedy next token after the last one to
 * next_token_dev (int32 [1]) and, if logits_dev is not NULL, its fp32 logits [V].  The
 * result is that of running the tokens through the decode step one position after the
 * other (smollm3.go's Prefill(tokens, startPos); the C17 engine article, 4.3).  It runs as
 * batched steps over chunks of up to 64 positions: the projections of a chunk as one GEMM
 * (matrix cores with bf16 activations and int8-row or bf16 weights), every position's K/V
 * appended to the cache before the chunk's attention, each position attending causally to
 * [0, its position] (the Qwen3-8B engine article's batched prefill, 4.4.1).  One position
 * per step instead when n = 1, when hidden-state capture is on, or with the persistent-
 * only schedule (dtd_debug_set_path 2). */
dtd_status dtd_prefill(dtd_engine* e, int64_t seq_id, const int32_t* tokens_dev, int32_t n,
                       int32_t* next_token_dev, float* logits_dev);

/* One decode step for `batch` distinct existing sequences: token b (tokens_dev[b], device
 * int32) goes at position len(seq_ids_host[b]) of its sequence, whose KV grows by one.
 * Writes next_tokens_dev[b] (int32 [batch]) and, if logits_dev is not NULL, fp32 logits
 * [batch][V].  next_tokens_dev may equal tokens_dev (greedy loop without a host round
 * trip). */
dtd_status dtd_decode_step(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                           const int32_t* tokens_dev, int32_t* next_tokens_dev,
                           float* logits_dev);

/* dtd_decode_step for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): same arguments, semantics and errors,
 * but the call allocates nothing, on the device or the host.  It runs the one-kernel-per-
 * sub-step schedule at every batch size, with its work memory -- the split-K attention
 * partials (batch x Hq x nch x (head_dim + 2) fp32, nch = ceil(max_ctx / chunk)) and, for
 * batched matrix-core projections, their split-K sums (splits x batch x rows fp32) -- in a
 * static device array of 32 MiB that the library holds on each GPU until the process ends;
 * a call that would need more returns DTD_E_UNSUPPORTED before anything is enqueued.  Every
 * call on one GPU shares that array, and each call writes every value it reads there before
 * reading it: calls that overlap on one GPU (other streams, other engines, other threads)
 * race and must be serialised by the caller.  Kernel-timing hooks are not applied to it. */
dtd_status dtd_decode_step_noalloc(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                                   const int32_t* tokens_dev, int32_t* next_tokens_dev,
                                   float* logits_dev);

/* ---- sampling ----------------------------------------------------------------------- */

/* Sampler settings: the sampler of the nxmr.cn C17 engine article (4.6) and of smollm3.go's
 * walkthrough ("sampling: from logits to the next token").
 *   temperature  0 = greedy: the largest logit, the lowest index among equal ones.  Above 0
 *                the logits are divided by it and soft-maxed.
 *   top_k        > 0 keeps the top_k most probable tokens (0 = off).
 *   top_p        < 1 keeps the shortest run of most probable tokens whose probability
 *                reaches top_p (1 = off); range (0, 1].
 *   min_p        > 0 keeps the tokens whose probability is at least min_p (0 = off); the
 *                most probable token always stays; range [0, 1].
 *   seed         key of the draws.
 * The filters apply in that order, each to the renormalised distribution the one before it
 * left; "most probable" orders by logit, then by index.  One token is then drawn by inverse
 * transform sampling in vocabulary order: the first kept token whose cumulative
 * probability exceeds u, with u = the top 53 bits of the first word of the Philox4x64-10
 * block (Salmon et al., SC 2011) at counter (c, 0, 0, 0) and key (seed, 0), times 2^-53.
 * The same (seed, c) always gives the same u.  Probabilities are computed as exact integer
 * sums of weights exp((l - max) / T) in 2^-44 fixed point: tokens with a weight below
 * 2^-44 of the largest are never drawn.  NaN logits are never drawn. */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
  float min_p;
  uint64_t seed;
} dtd_sampler;

/* Samples one token per row: rows b < batch of logits_dev (fp32, row b at
 * logits_dev + b * row_stride, vocab columns) with samplers_host[b] and draw counter
 * counters_host[b] (host arrays [batch]) -> tokens_dev[b] (device int32 [batch]).  Needs no
 * engine and allocates nothing; enqueued on hip_stream (a hipStream_t, NULL = the null
 * stream), asynchronous.  DTD_E_ARG for a null pointer, batch outside [1, 64], vocab
 * outside [1, 2^19], row_stride < vocab or settings outside their ranges (the message is
 * then what dtd_last_error(NULL) returns); DTD_E_HIP if the launch fails. */
dtd_status dtd_sample(const float* logits_dev, int64_t row_stride, int32_t batch, int32_t vocab,
                      const dtd_sampler* samplers_host, const int64_t* counters_host, int32_t* tokens_dev,
                      void* hip_stream);

/* Sets how sequence seq_id picks its next tokens from then on: every later dtd_prefill and
 * decode step of it draws with *s instead of taking the greedy token, with counter = the
 * position whose logits are sampled (the last prompt position for a prefill), so a
 * sequence's draws do not depend on the batch it shares.  s = NULL or temperature 0
 * restores greedy.  The sequence need not exist yet; dtd_reset_seq forgets the setting.
 * Host only.  DTD_E_ARG for settings outside their ranges, DTD_E_UNSUPPORTED when the
 * model's vocabulary exceeds 2^19. */
dtd_status dtd_set_sampler(dtd_engine* e, int64_t seq_id, const dtd_sampler* s);

/* ---- prefix cache --------------------------------------------------------------------- */

/* The automatic prefix cache of the Qwen3-8B engine article (4.4.4).  With max_entries > 0,
 * every dtd_prefill that starts a new sequence first looks for the longest cached prefix of
 * its tokens (the whole token list first, then ever shorter prefixes, matched by a hash of
 * the prefix and then token by token) and takes those positions' KV instead of computing
 * them: whole KV blocks are shared, a partly filled last block is copied.  The last prompt
 * position always runs, for its logits.  After the prefill, the sequence's prompt is recorded
 * as an entry (when the host knows all of its tokens: prefills only, no decode steps before).
 * Entries hold references to their KV blocks; the least recently used entries are dropped
 * when more than max_entries exist or when a call needs free blocks.  With the cache on,
 * dtd_prefill reads its tokens to the host first (it synchronises the stream).  max_entries
 * 0 turns the cache off and drops every entry.  Host only.  DTD_E_ARG if max_entries < 0. */
dtd_status dtd_set_prefix_cache(dtd_engine* e, int32_t max_entries);

/* Records positions [0, n) of sequence seq_id as a prefix-cache entry whose tokens are
 * tokens_host[0, n) (the caller vouches that those are the tokens the positions hold, e.g. a
 * prompt and the tokens decoded after it).  Host only.  DTD_E_NOSEQ for an unknown seq_id,
 * DTD_E_ARG for n outside [1, its length], DTD_E_STATE when the cache is off. */
dtd_status dtd_prefix_cache_add(dtd_engine* e, int64_t seq_id, const int32_t* tokens_host, int32_t n);

/* ---- KV budget ------------------------------------------------------------------------- */

/* The Initial-Key cache of the nxmr.cn C17 engine article (5.3): from now on, whenever
 * sequence seq_id holds more than `budget` KV entries after a prefill or decode step, its
 * cache keeps only the entries of its first n_initial positions (where attention pools), its
 * last n_recent entries, and, of the others, those with the largest sums of the attention
 * they received (softmax probability, summed over the query heads and over the last
 * score_layers layers, added at every decode step and, for a prefill, by its last position's
 * query; the earlier entry wins equal sums); the rest are evicted and the kept entries are
 * compacted, in order, into fresh KV blocks (synchronous: the host reads the sums).  Kept
 * keys keep their RoPE rotation and new tokens are rotated by their true position, so a
 * sequence's positions still end at max_ctx (the RoPE table); the budget bounds the KV blocks
 * it holds.  With budget >= its length nothing is evicted and the outputs are the full
 * cache's.  A budgeted sequence decoding alone runs the batch-1 step kernel (which keeps
 * the scored layers' queries and softmax statistics for the score sums that follow it); in
 * a batch or a prefill chunk it runs the per-sub-step kernels.  Budgeted sequences are never
 * reused from or recorded in the prefix cache, and are refused by dtd_decode_step_noalloc.  budget 0 turns
 * the budget off (entries already evicted stay evicted).  The sequence need not exist yet;
 * dtd_reset_seq drops the setting.  DTD_E_ARG for budget < n_initial + n_recent + 1,
 * n_recent < 1, budget > max_ctx or score_layers outside [1, n_layers]; DTD_E_STATE when
 * setting a budget on a sequence whose entries were evicted before. */
dtd_status dtd_set_kv_budget(dtd_engine* e, int64_t seq_id, int32_t budget, int32_t n_initial, int32_t n_recent,
                             int32_t score_layers);

/* ---- continuous batching ----------------------------------------------------------------- */

/* A scheduler runs requests through one engine as continuous batches: the scheduling loop of
 * the Qwen3-8B engine article (4.3.2).  A request is a prompt (host int32 tokens) and a token
 * budget.  It is admitted, in arrival order, when the KV pool can hold its whole run and the
 * batch (at most max_batch) has room; its prompt is then prefilled.  Every scheduling step
 * runs one decode step for all admitted requests together, each at its own position; a
 * request that has max_new_tokens tokens, or produced stop_token (>= 0), leaves and frees its
 * KV (recorded in the prefix cache first when that is on), and the next ones join.  Requests
 * use engine sequence ids below 0; the scheduler assumes it has the engine's sequences and KV
 * pool to itself.  prompt_budget caps the prompt tokens admitted per step (0 = 4096; at least
 * one request is admitted).  dtd_sched_destroy first stops the loop and drops unfinished
 * requests. */
typedef struct dtd_sched dtd_sched;
dtd_status dtd_sched_create(dtd_engine* e, int32_t prompt_budget, dtd_sched** out);
void       dtd_sched_destroy(dtd_sched* s);

/* Queues a request; *id_out gets its id.  sampler NULL = greedy.  Thread-safe.  DTD_E_ARG for
 * a bad argument or token id, DTD_E_CTX when n + max_new_tokens - 1 positions exceed max_ctx,
 * DTD_E_KVFULL when the whole pool could not hold the run. */
dtd_status dtd_sched_submit(dtd_sched* s, const int32_t* prompt_host, int32_t n, int32_t max_new_tokens,
                            int32_t stop_token, const dtd_sampler* sampler, int64_t* id_out);

/* One scheduling step on the calling thread (admissions, one batched decode step,
 * departures); *pending (may be NULL) gets the number of queued and running requests after
 * it.  Returns the first engine error of the step (the requests it hit fail; the others go on;
 * dtd_sched_last_error has the message).  DTD_E_STATE while the background loop runs. */
dtd_status dtd_sched_step(dtd_sched* s, int32_t* pending);

/* Runs scheduling steps on a thread of the scheduler's own whenever requests are queued or
 * running, until dtd_sched_stop.  While it runs, make no other calls on the engine. */
dtd_status dtd_sched_start(dtd_sched* s);
dtd_status dtd_sched_stop(dtd_sched* s);

/* Blocks until request id is done or timeout_ms passes (< 0: no limit).  Returns the
 * request's status (DTD_OK, or the engine error it failed with), DTD_E_STATE on time-out,
 * DTD_E_NOSEQ for an unknown id.  Thread-safe. */
dtd_status dtd_sched_wait(dtd_sched* s, int64_t id, int32_t timeout_ms);

/* Copies up to cap of request id's generated tokens to tokens_host; returns how many it has
 * (or the status it failed with, < 0); *done (may be NULL) = 1 once it has left.  Thread-safe. */
int32_t dtd_sched_result(dtd_sched* s, int64_t id, int32_t* tokens_host, int32_t cap, int32_t* done);

/* Forgets a finished request.  DTD_E_STATE if it has not finished. */
dtd_status dtd_sched_release(dtd_sched* s, int64_t id);

/* Message of the scheduler's first failed step (empty if none). */
const char* dtd_sched_last_error(const dtd_sched* s);

/* Forgets a sequence, as the Qwen3-8B engine article's ResetSeq call does (4.1.2): its KV
 * blocks and its slot return to the free lists, its sampler setting is dropped, and the
 * seq_id may be used again for a new sequence.  Host only (nothing is enqueued; the
 * blocks' contents are not cleared).  DTD_E_NOSEQ for an unknown seq_id. */
dtd_status dtd_reset_seq(dtd_engine* e, int64_t seq_id);

/* Current length (positions written) of a sequence, or a dtd_status < 0. */
int32_t dtd_seq_len(const dtd_engine* e, int64_t seq_id);

/* The engine's configuration (its copy of what dtd_create got) and its HIP stream. */
dtd_status dtd_get_config(const dtd_engine* e, dtd_config* out);
void*      dtd_get_stream(const dtd_engine* e);

/* Reports what the device flagged since the last check, and synchronises the stream:
 *   - DTD_E_ARG: an earlier prefill or decode step read a token id outside [0, V) (it used
 *     id 0 instead); the flag is cleared, the engine stays usable;
 *   - DTD_E_HIP: a wait of the batch-1 step kernel for another workgroup timed out (every
 *     workgroup then gave up, so the outputs of that step and of any later one are not
 *     valid); the engine is unusable from then on, destroy it;
 *   - DTD_OK otherwise. */
dtd_status dtd_check_device_errors(dtd_engine* e);

void        dtd_destroy(dtd_engine* e);
/* Message of the engine's last failed call.  With e == NULL: the message of this thread's
 * last dtd_create if it failed, else "null engine".  The string is owned by the library
 * and valid until the next call on the same engine (or thread, for e == NULL). */
const char* dtd_last_error(const dtd_engine* e);

/* ---- debug and measurement entry points (tests and benchmarks) -------------------- */

/* Dequantises stored rows [r0, r0+nrows) of one matrix (name as in load_weights without
 * the part suffix, e.g. "L3.w_down") to fp32 out_dev [nrows][cols], with the same
 * per-element product the kernels use (q * s in fp32, or bf16 widened). */
dtd_status dtd_debug_dequant_rows(dtd_engine* e, const char* matrix, int32_t r0, int32_t nrows,
                                  float* out_dev);

/* While enabled, each later prefill token or decode step copies the fp32 residual stream
 * after the embedding and after every layer to out_dev [(L+1)][batch][D] (the buffer is
 * overwritten by every step).  enable = 0 turns it off. */
dtd_status dtd_debug_capture_hidden(dtd_engine* e, int32_t enable, float* out_dev);

/* A decode step like dtd_decode_step in which every kernel reads its input from an inject
 * record and its output is copied to a capture record, so that each kernel can be checked
 * against the reference operation on identical inputs.  Both buffers hold one record per
 * layer; a record is these fields in order, each [batch][n] (f32 = fp32, act = the
 * activation type), of dtd_debug_probe_record_bytes() bytes in total:
 *   x_in f32 [D] | xn act [D] | q f32 [q_dim] | k f32 [kv_dim] | v f32 [kv_dim] |
 *   o act [q_dim] | x_mid f32 [D] | xn2 act [D] | h act [F] | x_out f32 [D]
 * Per layer: xn = RMSNorm(inject.x_in); (q, k, v) = QKV+RoPE(inject.xn);
 * o = attention(inject.q, cache + inject k/v appended at the new position);
 * x_mid = inject.x_in + Wo.inject.o; xn2 = RMSNorm(inject.x_mid);
 * h = SwiGLU(inject.xn2); x_out = inject.x_mid + Wdown.inject.h.  The final norm and LM
 * head read the last layer's inject.x_out.  Unlike dtd_decode_step, a seq_id not seen
 * before starts a new sequence at position 0. */
dtd_status dtd_debug_decode_probe(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                                  const int32_t* tokens_dev, const void* inject_dev,
                                  void* capture_dev, int32_t* next_tokens_dev, float* logits_dev);

/* Bytes of one probe record for cfg and batch (host only), or a dtd_status < 0. */
int64_t dtd_debug_probe_record_bytes(const dtd_config* cfg, int32_t batch);

/* Writes stored KV of positions [pos0, pos0+n) of one layer from host memory, native
 * encoding [n][Hkv][d] (fp32 / bf16 bits / int8 codes) plus fp16 scales [n][Hkv] for
 * int8 (k_scale, v_scale NULL otherwise).  Creates the sequence if new, allocates its
 * blocks and extends its length to at least pos0+n (positions must be written before
 * they are attended).  Synchronous. */
dtd_status dtd_debug_kv_write(dtd_engine* e, int64_t seq_id, int32_t layer, int32_t pos0,
                              int32_t n, const void* k, const void* v, const void* k_scale,
                              const void* v_scale);

/* Reads stored KV of positions [pos0, pos0+n) through the block table into host memory
 * in the layout dtd_debug_kv_write takes.  Synchronous. */
dtd_status dtd_debug_kv_read(dtd_engine* e, int64_t seq_id, int32_t layer, int32_t pos0,
                             int32_t n, void* k, void* v, void* k_scale, void* v_scale);

/* Sets a sequence's length to len (creating it if new) with synthetic KV in every layer;
 * for timing long contexts only.  Element i of KV head j at position t of layer l, for K
 * (w = 0) and V (w = 1): h = m(seed ^ m(l<<40 ^ t<<20 ^ j<<12 ^ i<<1 ^ w)) with m the
 * splitmix64 finaliser, u = (h>>40) * 2^-23 - 1 in [-1, 1), and the value u * a with
 * a = 0.02 * sqrt(D) * 1.7320508 in fp32 (uniform with the standard deviation
 * 0.02 * sqrt(D)); bf16 stores it rounded to nearest even; int8 stores rint(127 u) with
 * the fp16 scale a / 127.  Positions below len of a longer sequence are overwritten and
 * its length is kept.  Errors: DTD_E_ARG for len outside [1, max_ctx], DTD_E_KVFULL
 * when the sequence slots or KV blocks run out. */
dtd_status dtd_debug_kv_fill(dtd_engine* e, int64_t seq_id, int32_t len, uint64_t seed);

/* Kernel timing.  kind: 0 = the gate/up projection, 1 = the down projection, 2 = the
 * QKV projection, 3 = the output projection, 4 = attention, 5 = LM head (per-kernel
 * schedule), 6 = the persistent step kernel (whole batch-1 step).  While enabled,
 * HIP events bracket every launch of that kernel on the engine's stream; *total_ms
 * and *count return the summed duration and number of launches since enabling and
 * reset them.  Synchronises the stream when reading. */
dtd_status dtd_debug_kernel_timing(dtd_engine* e, int32_t kind, int32_t enable,
                                   double* total_ms, int64_t* count);

/* Streaming-read ceiling of the device: reads `bytes` (rounded down to 16) of device memory
 * buf_dev once untimed, then `reps` times, with 16-byte nontemporal loads spread over every
 * compute unit, on hip_stream; *gbs gets the timed passes' bytes per second / 1e9.  Needs no
 * engine; on error the message is what dtd_last_error(NULL) returns.  Synchronous. */
dtd_status dtd_debug_stream_read(const void* buf_dev, int64_t bytes, int32_t reps, void* hip_stream, double* gbs);

/* Positions the last dtd_prefill of seq_id took from the prefix cache (0 for none), free KV
 * blocks, and prefix-cache entries; or a dtd_status < 0. */
int32_t dtd_debug_prefix_reused(const dtd_engine* e, int64_t seq_id);
int32_t dtd_debug_kv_blocks_free(const dtd_engine* e);
int32_t dtd_debug_prefix_entries(const dtd_engine* e);

/* A sequence's cache entries in order: their token positions (out_host [cap]; -1 where
 * unknown) or their attention-score sums (synchronous).  Returns the entry count, or a
 * dtd_status < 0. */
int32_t dtd_debug_kv_positions(const dtd_engine* e, int64_t seq_id, int32_t* out_host, int32_t cap);
int32_t dtd_debug_kv_scores(dtd_engine* e, int64_t seq_id, float* out_host, int32_t cap);

/* Schedule selection.  path 0 (default): batch-1 steps run as one persistent kernel per
 * step (every phase in one cooperative launch) when the device allows it, other batches
 * and hidden-state capture as one kernel per sub-step; 1: always one kernel per sub-step;
 * 2: persistent only (calls it cannot serve fail with DTD_E_UNSUPPORTED). */
dtd_status dtd_debug_set_path(dtd_engine* e, int32_t path);

/* 1 if a decode step of this batch size would run the persistent kernel now, else 0. */
int32_t dtd_debug_uses_persistent(const dtd_engine* e, int32_t batch);

/* The head size the batch-1 step kernel of this engine has fixed at compile time: 128 when
 * the model has head size 128, 4 query heads per KV head and KV blocks of 16 positions, 64
 * for head size 64 with the same group and block sizes and bf16 activations (the
 * instantiations built for those shapes, whose probe variants dtd_debug_decode_probe then
 * runs too), or 0 when the kernel reads the shape at run time or the engine has no step kernel
 * (a device without cooperative launches, or a shape outside the kernel's limits).  A
 * dtd_status < 0 for a null engine. */
int32_t dtd_debug_step_kernel_shape(const dtd_engine* e);

/* The batched decode attention's split-K plan (host only, no device call), as the engine
 * makes it each step for the one-wave-per-chunk kernel: batch contexts pos[b] + 1 (1 <=
 * batch <= 64), n_kv_heads waves per chunk, at most max_chunks chunks per sequence and
 * `slots` resident waves.  Sequence b is cut into chunks of ct[b] positions (a multiple of
 * 16, at most 2048); cend[b] is the number of chunks of sequences 0..b.  Returns the batch's
 * chunk count, or DTD_E_ARG for out-of-range arguments (a context above max_chunks x 2048
 * included).  Split-K of attention over the context is the Qwen3-8B engine article's
 * decode attention (4.4.2); the chunk sizing is this library's. */
int32_t dtd_debug_plan_attention_chunks(int32_t batch, const int32_t* pos, int32_t n_kv_heads, int32_t max_chunks,
                                        int32_t slots, int32_t* ct, int32_t* cend);

#ifdef __cplusplus
}
#endif
#endif /* DTD_H */
