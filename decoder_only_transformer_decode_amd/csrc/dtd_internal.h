// dtd_internal.h -- types shared by the host engine (dtd_engine.cpp) and the gfx950
// kernels (dtd_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtd {

constexpr int kMaxBatch = 64;
constexpr int kMaxUpdates = 64;
constexpr int kPrefillChunk = 64;   // prompt positions per batched prefill step
constexpr int kMaxSampleVocab = 1 << 19;   // fixed-point token weights: V * 2^44 < 2^64
constexpr int kAttnTile = 64;      // positions per LDS tile in decode attention (one per lane)
constexpr int kPersistWaves = 8;   // waves per workgroup of the persistent step kernel
constexpr int kErrToken = 1;       // device error bits: token id out of range
constexpr int kErrBarrier = 2;     //                    a cross-workgroup wait timed out

enum WFmt { W_INT8_ROW = 0, W_Q8_0 = 1, W_BF16 = 2, W_Q4_0 = 3 };
enum Act { ACT_F32 = 0, ACT_BF16 = 1 };
enum KvFmt { KV_F32 = 0, KV_BF16 = 1, KV_I8 = 2 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Per-step descriptor, copied host -> device once per step.  Kernels read the batch's
// positions, sequence slots and I/O pointers from it, so launch arguments stay fixed.
struct StepDesc {
  int32_t batch;
  int32_t do_head;                   // run final norm + LM head + argmax
  int32_t n_updates;                 // block-table entries to set before the step
  int32_t n_chunks;                  // decode attention chunks with work, over the batch
  const int32_t* tokens;             // [batch] token ids (caller memory)
  int32_t* next_tokens;              // [batch] greedy outputs (caller memory)
  float* logits_out;                 // [batch][V] or null (caller memory)
  int32_t pos[kMaxBatch];            // position the new token takes
  int32_t slot[kMaxBatch];           // sequence slot (block-table row)
  int32_t pos_block[kMaxBatch];      // physical KV block of the new position
  int32_t upd[kMaxUpdates][3];       // (slot, logical block, physical block)
  // KV budget: a sequence's token position (for RoPE) can run ahead of its cache index `pos`
  // once entries have been evicted; attention-score sums are added, from layer score_from[b]
  // on (L: none), to the sequence slot's row of the score buffer
  int32_t rpos[kMaxBatch];
  int32_t score_from[kMaxBatch];
  // Split-K of the decode attention: sequence b's context in chunks of ct[b] positions (a
  // multiple of 16); its chunks are entries cend[b-1] .. cend[b]-1 of one list over the batch
  // (cend[-1] = 0), which the one-wave-per-chunk kernel walks
  int32_t ct[kMaxBatch];
  int32_t cend[kMaxBatch];
};

struct Dims {
  int D, L, Hq, Hkv, hd, F, V;
  int G;            // Hq / Hkv
  int q_dim, kv_dim, qkv_rows;
  int bs;           // KV block size
  int max_blocks;   // block-table row length = ceil(max_ctx / bs)
  int max_ctx;
  int ct;           // attention chunk length (positions per split)
  int nch;          // chunks per sequence at max_ctx
  float eps;
  int wfmt, act, kvfmt;
};

// A weight matrix in device memory: codes or bf16 bits [rows][cols] and scales
// (fp32 [rows] for int8-row, fp16 [rows][cols/32] for Q8_0, null for bf16).
struct MatDev {
  const void* w;
  const void* s;
  int rows, cols;
};

// KV pool of one layer: K and V [n_blocks][Hkv][bs][hd] in the KV encoding, plus fp16
// scales [n_blocks][Hkv][bs] for int8.
struct KvLayer {
  void* k;
  void* v;
  uint16_t* ks;
  uint16_t* vs;
};

struct EpiArgs {
  const StepDesc* desc;
  // EPI_QKV
  float* q;            // [B][q_dim] post-RoPE
  float* knew;         // [B][kv_dim] post-RoPE, not yet rounded to the KV type
  float* vnew;         // [B][kv_dim]
  const float* rope_cos;  // [max_ctx][hd/2]
  const float* rope_sin;
  // EPI_RESID
  float* x;            // [B][D] residual stream, += result
  // EPI_SWIGLU
  void* h;             // [B][F] activation type
  // EPI_LOGITS
  float* logits;       // [B][V] engine buffer
};

// Byte offsets of the fields of one layer's probe record (see dtd_debug_decode_probe).
struct ProbeLayout {
  size_t x_in, xn, q, k, v, o, x_mid, xn2, h, x_out, record;
};

// One layer's weights and KV pool, as the persistent kernel reads them (device table).
struct PLayer {
  MatDev qkv, o, gu, down;
  const float* attn_norm;
  const float* ffn_norm;
  KvLayer kv;
};

// Arguments of the persistent batch-1 step kernel (dtd_persistent.hip).  Vectors that
// pass between workgroups live in "tagged" buffers: 64-bit words (epoch << 32 | fp32 bits)
// written with device-scope stores; a reader polls a word until it carries the epoch of
// the phase it wants, so the data and its readiness arrive in one memory round trip.
struct PersistArgs {
  Dims d;
  const PLayer* layers;     // [L] in device memory
  MatDev emb, head;
  const float* final_norm;
  const StepDesc* desc;
  int32_t* bt;
  const float* rope_cos;
  const float* rope_sin;
  uint64_t* t_q;            // tagged [q_dim] post-RoPE queries
  uint64_t* t_k;            // tagged [kv_dim] post-RoPE new key
  uint64_t* t_v;            // tagged [kv_dim] new value
  uint64_t* t_o;            // tagged [q_dim] attention output (rounded to the activation type)
  uint64_t* t_xm;           // tagged [D] residual stream after attention
  uint64_t* t_h;            // tagged [F] SwiGLU output (rounded)
  uint64_t* t_xo;           // tagged [D] residual stream after the feed-forward block
  uint64_t* t_part;         // tagged [Hq][nch][hd+2] attention chunk partials (acc, m, l)
  uint64_t* t_am;           // tagged [nwg][2] per-workgroup argmax (value, index)
  uint32_t epoch;           // tag of this launch's first phase (6 per layer, 1 for the head)
  float* logits;            // [V]
  int32_t* err;
  int ct;                   // attention chunk length of this step
  int nch;                  // chunk stride of partials
  int xs_floats;            // LDS floats before the residual-stream copy
  const uint8_t* inject;    // probe records (null: normal step)
  uint8_t* capture;
  ProbeLayout po;
  // layers from the descriptor's score_from[0] on (a KV budget's scored layers): each one's
  // post-RoPE queries [L][q_dim] and per-head softmax (max, sum) [L][Hq][2], for the score
  // sums computed after the step
  float* score_q;
  float* score_stat;
};

// Packed hand-off of the SwiGLU output with bf16 activations: each workgroup of the step
// kernel writes this many words (three values each) of its F-row share, pads included.
__host__ __device__ inline int h_words_per_wg(int F, int nwg) { return ((F + nwg - 1) / nwg + 2) / 3; }
// words of the SwiGLU output's hand-off buffer (either layout)
inline size_t h_buffer_words(int F, int nwg) {
  const size_t packed = (size_t)nwg * h_words_per_wg(F, nwg);
  return packed > (size_t)F ? packed : (size_t)F;
}

// Sampler settings of one row (dtd_sample.hip): temperature 0 = greedy; top_k 0, top_p 1
// and min_p 0 turn those filters off.  counter picks the draw (the position whose logits
// the row holds).
struct SampleRow {
  float temperature;
  int32_t top_k;
  float top_p;
  float min_p;
  uint64_t seed;
  int64_t counter;
};

// Arguments of the sampling kernel, passed by value: rows b < B of logits (row stride
// `stride` floats, V columns) -> out[b].
struct SampleArgs {
  const float* logits;
  int64_t stride;
  int32_t V;
  int32_t B;
  int32_t* out;
  SampleRow row[kMaxBatch];
};

// ---- launchers (dtd_kernels.hip, dtd_persistent.hip) ----
size_t persistent_smem_bytes(const Dims& d, int nch, int nwg);
size_t persistent_xs_floats(const Dims& d, int nch);
int persistent_tags_per_step(const Dims& d);
bool persistent_supports(const Dims& d);   // shapes the persistent step kernel handles
// the head size the step kernel fixes at compile time for this shape (128; 64 with bf16
// activations; with G 4 and KV blocks of 16), or 0 (the shape read at run time)
int persistent_fixed_hd(const Dims& d);
hipError_t persistent_prepare(const Dims& d, size_t smem, int* blocks_per_cu);
hipError_t launch_persistent(const PersistArgs& a, int nwg, size_t smem, hipStream_t st);
hipError_t launch_embed(const Dims& d, const MatDev& emb, const StepDesc* desc, int B,
                        int32_t* block_table, float* x, int32_t* err, hipStream_t st);
hipError_t launch_rmsnorm(const Dims& d, const float* x, const float* g, void* xn, int B,
                          hipStream_t st);
hipError_t launch_gemv(const Dims& d, const MatDev& m, const void* xin, int B, int epi,
                       const EpiArgs& ea, hipStream_t st);
// batch > 1 projections on the matrix cores (bf16 activations; int8-row or bf16 weights)
bool gemm_eligible(const Dims& d, int B);
int gemm_splits(int N, int K, int cus);                 // K splits of an N x K matrix
size_t gemm_partial_bytes(const Dims& d, int B, int cus);   // work buffer of the split-K sums
// a residual projection (O or down) on the matrix cores, its residual add into ea.x and the
// RMSNorm of the result with gain g into xn (one launch for the split-K sums, the add and
// the norm when K is split)
hipError_t launch_gemm_resid_norm(const Dims& d, const MatDev& m, const void* xin, int B, const EpiArgs& ea,
                                  float* partials, int cus, const float* g, void* xn, hipStream_t st);
hipError_t launch_gemm(const Dims& d, const MatDev& m, const void* xin, int B, int epi, const EpiArgs& ea,
                       float* partials, int cus, hipStream_t st);
// whether the decode attention of these dimensions runs one wave per chunk (k_attn_w), which
// takes the descriptor's per-sequence chunks; the other shapes split at d.ct
bool attn_w_shape(const Dims& d);
// n_chunks: the descriptor's chunk count (k_attn_w shapes)
hipError_t launch_attention(const Dims& d, const StepDesc* desc, int B, int n_chunks, const float* q,
                            const float* knew, const float* vnew, const KvLayer& kv,
                            const int32_t* block_table, float* partials, hipStream_t st);
hipError_t launch_kv_append(const Dims& d, const StepDesc* desc, int B, const float* knew, const float* vnew,
                            const KvLayer& kv, hipStream_t st);
hipError_t launch_kv_copy_block(const Dims& d, const PLayer* layers, int src, int dst, hipStream_t st);
hipError_t launch_combine(const Dims& d, const StepDesc* desc, int B, const float* partials,
                          void* o, hipStream_t st, float* stat = nullptr);
// causal attention of a prefill chunk: n consecutive positions from desc->pos[0] (the last
// one last_pos) of the sequence in desc->slot[0], all appended; leaves launch_attention's
// partials [n][Hq][nch][hd+2] for launch_combine
hipError_t launch_attn_prefill(const Dims& d, const StepDesc* desc, int n, int last_pos, const float* q,
                               const KvLayer& kv, const int32_t* bt, float* partials, hipStream_t st);
// KV budget score sums of layers layer0 .. layer0 + nl - 1 (their queries, K pools and
// statistics q_ls floats, k_ls / s_ls bytes and st_ls floats apart), added in layer order
hipError_t launch_score(const Dims& d, const StepDesc* desc, int B, int max_pos, int layer0, int nl, const float* q,
                        size_t q_ls, const KvLayer& kv, size_t k_ls, size_t s_ls, const int32_t* bt, const float* stat,
                        size_t st_ls, float* scores, hipStream_t st);
// KV budget, one eviction on the device (n = budget + 1 entries): picks the entry, closes
// the gap in the score and position rows, writes the n - 1 kept indices to keep, and puts
// the nb new blocks (fresh) in the sequence's block-table row
hipError_t launch_evict_one(float* scores, int32_t* kvpos, int n, int n_init, int rec0, int new_pos, int32_t* keep,
                            const int32_t* fresh, int nb, int32_t* bt_row, hipStream_t st);
hipError_t launch_kv_gather(const Dims& d, const PLayer* layers, const int32_t* old_blocks, const int32_t* new_blocks,
                            const int32_t* keep, int n, hipStream_t st);
hipError_t launch_argmax(const Dims& d, const StepDesc* desc, int B, const float* logits,
                         hipStream_t st);
hipError_t launch_dequant_rows(const Dims& d, const MatDev& m, const int32_t* rows, int nrows,
                               float* out, hipStream_t st);
hipError_t launch_sample(const SampleArgs& a, hipStream_t st);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int cus, hipStream_t st);
hipError_t launch_kv_fill(const Dims& d, const KvLayer& kv, const int32_t* blocks, int nblk_used,
                          int len, int layer, uint64_t seed, hipStream_t st);

}  // namespace dtd
