// dtd_internal.h -- types shared by the host engine (dtd_engine.cpp) and the gfx950
// kernels (dtd_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtd {

constexpr int kMaxBatch = 64;
constexpr int kMaxUpdates = 64;
constexpr int kAttnTile = 64;      // positions per LDS tile in decode attention (one per lane)

enum WFmt { W_INT8_ROW = 0, W_Q8_0 = 1, W_BF16 = 2 };
enum Act { ACT_F32 = 0, ACT_BF16 = 1 };
enum KvFmt { KV_F32 = 0, KV_BF16 = 1, KV_I8 = 2 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Per-step descriptor, copied host -> device once per step.  Kernels read the batch's
// positions, sequence slots and I/O pointers from it, so launch arguments stay fixed.
struct StepDesc {
  int32_t batch;
  int32_t do_head;                   // run final norm + LM head + argmax
  int32_t n_updates;                 // block-table entries to set before the step
  int32_t pad_;
  const int32_t* tokens;             // [batch] token ids (caller memory)
  int32_t* next_tokens;              // [batch] greedy outputs (caller memory)
  float* logits_out;                 // [batch][V] or null (caller memory)
  int32_t pos[kMaxBatch];            // position the new token takes
  int32_t slot[kMaxBatch];           // sequence slot (block-table row)
  int32_t upd[kMaxUpdates][3];       // (slot, logical block, physical block)
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

// ---- launchers (dtd_kernels.hip) ----
hipError_t launch_embed(const Dims& d, const MatDev& emb, const StepDesc* desc, int B,
                        int32_t* block_table, float* x, int32_t* err, hipStream_t st);
hipError_t launch_rmsnorm(const Dims& d, const float* x, const float* g, void* xn, int B,
                          hipStream_t st);
hipError_t launch_gemv(const Dims& d, const MatDev& m, const void* xin, int B, int epi,
                       const EpiArgs& ea, hipStream_t st);
hipError_t launch_attention(const Dims& d, const StepDesc* desc, int B, const float* q,
                            const float* knew, const float* vnew, const KvLayer& kv,
                            const int32_t* block_table, float* partials, hipStream_t st);
hipError_t launch_combine(const Dims& d, const StepDesc* desc, int B, const float* partials,
                          void* o, hipStream_t st);
hipError_t launch_argmax(const Dims& d, const StepDesc* desc, int B, const float* logits,
                         hipStream_t st);
hipError_t launch_dequant_rows(const Dims& d, const MatDev& m, const int32_t* rows, int nrows,
                               float* out, hipStream_t st);
hipError_t launch_kv_fill(const Dims& d, const KvLayer& kv, const int32_t* blocks, int nblk_used,
                          int len, int layer, uint64_t seed, hipStream_t st);

}  // namespace dtd
