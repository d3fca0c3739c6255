// dtd_engine.cpp -- host side of libdtd.so: the C ABI of include/dtd.h, configuration and
// weight validation (fail-closed, in the spirit of the hardened loader of the nxmr.cn C17
// engine article, 4.1), weight repacking, the paged KV block pool with per-sequence block
// tables (Qwen3-8B engine article, 4.3.1: fixed-size blocks, O(1) allocation from a free
// pool, one block list per sequence id), and the per-step launch sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/dtd.h"
#include "dtd_internal.h"

using namespace dtd;

namespace {

constexpr int kRing = 64;   // pinned step-descriptor slots in flight
constexpr int kEvictRing = 8;   // pinned block-list slots of device-side evictions in flight

struct LayerW {
  MatDev qkv, o, gu, down;
  float* attn_norm = nullptr;
  float* ffn_norm = nullptr;
};

struct Seq {
  int slot = -1;
  int len = 0;
  std::vector<int32_t> blocks;
  // token ids of positions [0, len) when the host knows them all (prefill inputs with the
  // prefix cache on); decode steps append ids only the device holds
  std::vector<int32_t> tokens;
  bool tokens_known = true;
  int reused = 0;   // positions the last prefill took from the prefix cache
  // KV budget: tokens run so far (the next token's RoPE position) and the true position of
  // each cache entry (kept in step only while a budget is set)
  int rpos = 0;
  std::vector<int32_t> kv_pos;
  // the positions live in the device's row (kvpos_dev) instead: after an eviction decided on
  // the device, until the host needs them again
  bool pos_on_dev = false;
};

// Initial-Key KV budget of one sequence (the C17 engine article, 5.3)
struct KvBudget {
  int budget = 0, n_initial = 0, n_recent = 0, score_layers = 0;
};

// Per-row extras of a step: RoPE positions and the first scored layer (null: none)
struct StepExtra {
  const int* rpos = nullptr;
  const int* score_from = nullptr;
};

// A prefix-cache entry: the KV of a token sequence's positions [0, tokens.size()), held as
// references to the blocks that store it.
struct PrefixEntry {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  uint64_t used = 0;   // LRU clock of the last hit or insert
};

struct TimerPair {
  hipEvent_t a, b;
};

}  // namespace

struct dtd_engine {
  dtd_config cfg{};
  Dims d{};
  hipStream_t stream = nullptr;
  int device = 0;
  bool broken = false;
  bool loaded = false;
  std::string err;

  std::vector<LayerW> layers;
  MatDev emb{}, head{};
  float* final_norm = nullptr;
  std::vector<void*> weight_allocs;

  float* rope_cos = nullptr;
  float* rope_sin = nullptr;

  void* kpool = nullptr;
  void* vpool = nullptr;
  uint16_t* kspool = nullptr;
  uint16_t* vspool = nullptr;
  size_t kv_layer_elems = 0;    // elements of K (or V) per layer
  size_t kv_layer_scales = 0;   // fp16 scales of K (or V) per layer
  int32_t* bt_dev = nullptr;

  float* x = nullptr;
  void* xn = nullptr;
  float* q = nullptr;
  float* knew = nullptr;
  float* vnew = nullptr;
  float* partials = nullptr;
  float* gemm_partials = nullptr;   // split-K sums of the batched matrix-core projections
  int32_t* tok_scratch = nullptr;   // greedy tokens of a prefill chunk [mb]
  int mb = 0;                       // rows of the work buffers (max batch or prefill chunk)
  int cus = 0;                      // compute units of the device
  void* o = nullptr;
  void* h = nullptr;
  float* logits = nullptr;
  int32_t* err_dev = nullptr;
  StepDesc* desc_dev = nullptr;
  int32_t* rows_dev = nullptr;  // scratch for debug row lists
  int rows_cap = 0;

  StepDesc* desc_host = nullptr;  // pinned [kRing]
  hipEvent_t desc_ev[kRing];
  bool desc_ev_used[kRing];
  int ring = 0;
  int32_t* err_host = nullptr;    // pinned

  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, dtd_sampler> samplers;   // sequences that do not decode greedily
  std::vector<int> free_slots;
  std::vector<int32_t> free_blocks;
  std::vector<int32_t> blk_ref;   // holders of each KV block: sequences and prefix-cache entries
  std::unordered_map<int64_t, KvBudget> budgets;   // sequences under a KV budget
  float* scores_dev = nullptr;    // [max_seqs][max_ctx] attention-score sums of budgeted sequences
  float* attn_stat = nullptr;     // [mb][Hq][2] merged softmax max and normaliser of a scored layer
  float* p_score_q = nullptr;     // step kernel: [L][q_dim] queries of the scored layers
  float* p_score_stat = nullptr;  // step kernel: [L][Hq][2] their softmax max and normaliser
  int32_t* evict_dev = nullptr;   // [3][max_ctx] eviction lists (old blocks, new blocks, kept entries)
  int32_t* kvpos_dev = nullptr;   // [max_seqs][max_ctx] entry positions of budgeted sequences (device-side evictions)
  int32_t* evict_host = nullptr;  // pinned [kEvictRing][2][max_blocks] block lists for device-side evictions
  hipEvent_t evict_ev[kEvictRing];
  bool evict_ev_used[kEvictRing];
  int evict_ring = 0;
  int step_score_min = 1 << 30;   // first scored layer of the step being run
  int step_max_pos = 0;
  int step_chunks = 0;           // decode attention chunks of the current step (k_attn_w shapes)

  // prefix cache: entries by id, and every prefix of every entry by its hash
  int pcache_cap = 0;             // 0: off
  int64_t pcache_next = 0;
  uint64_t pcache_clock = 0;
  std::unordered_map<int64_t, PrefixEntry> pcache;
  std::unordered_multimap<uint64_t, std::pair<int64_t, int32_t>> pindex;   // hash -> (entry, length)

  float* capture = nullptr;

  // persistent batch-1 step kernel
  bool persist_ok = false;
  int nwg = 0;                   // workgroups (one per compute unit)
  size_t p_smem = 0;
  int p_nch = 0;                 // chunk stride of partials for the persistent path
  PLayer* players = nullptr;     // [L] device table
  uint64_t* tags = nullptr;      // tagged hand-off buffers of the step kernel (one allocation)
  size_t tags_words = 0;
  uint32_t epoch = 1;            // tag of the next launch's first phase (0 never used)
  int path = 0;                  // 0 auto, 1 per-kernel, 2 persistent

  void* scratch_dev = nullptr;   // this device's copy of the allocation-free entry point's scratch
  int timing_kind = -1;
  std::vector<TimerPair> timers;
  size_t timers_used = 0;
};

static thread_local std::string g_create_err;   // message of this thread's last failed dtd_create

// Work memory of dtd_decode_step_noalloc: a file-scope device array, one copy on every GPU
// the library runs on, held until the process ends.  Host code never uses the array's
// name as an address (on the host it names a stand-in, not device memory): each device's
// copy is looked up once with hipGetSymbolAddress, when the first engine is created on
// that device, and kept in g_scratch_dev.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

// The address of this device's scratch copy (the device is current); nullptr on failure.
static void* scratch_on_current_device(int device, hipError_t* err) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *err = hipSuccess;
  if (device < 0 || device >= kMaxDevices) { *err = hipErrorInvalidDevice; return nullptr; }
  if (!g_scratch_dev[device]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_dev[device] = p;
  }
  return g_scratch_dev[device];
}

// ---------------------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------------------

static dtd_status fail(dtd_engine* e, dtd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (e) e->err = buf;
  return st;
}

#define HIP_OK(e, call)                                                               \
  do {                                                                                \
    hipError_t _r = (call);                                                           \
    if (_r != hipSuccess) {                                                           \
      (e)->broken = true;                                                             \
      return fail((e), DTD_E_HIP, "%s failed: %s", #call, hipGetErrorString(_r));     \
    }                                                                                 \
  } while (0)

static int vec_elems(int wfmt) { return wfmt == DTD_W_BF16 ? 8 : (wfmt == DTD_W_Q4_0 ? 32 : 16); }

static dtd_status check_config(const dtd_config* c, char* msg, int32_t msg_len) {
  auto bad = [&](dtd_status st, const char* fmt, auto... args) {
    if (msg && msg_len > 0) snprintf(msg, (size_t)msg_len, fmt, args...);
    return st;
  };
  if (!c) return bad(DTD_E_ARG, "%s", "null config");
  if (c->abi_version != DTD_ABI_VERSION) return bad(DTD_E_ARG, "abi_version %d, library has %d", c->abi_version, DTD_ABI_VERSION);
  if (c->dim <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->ffn_dim <= 0 || c->vocab <= 0)
    return bad(DTD_E_ARG, "%s", "dimensions must be positive");
  if (c->n_q_heads % c->n_kv_heads) return bad(DTD_E_ARG, "n_kv_heads %d does not divide n_q_heads %d", c->n_kv_heads, c->n_q_heads);
  if (c->wfmt < 0 || c->wfmt > 3 || c->act < 0 || c->act > 1 || c->kvfmt < 0 || c->kvfmt > 2)
    return bad(DTD_E_ARG, "%s", "unknown weight, activation or KV format");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return bad(DTD_E_ARG, "%s", "rms_eps must be >= 0 and rope_theta > 0");
  if (c->kv_block_size <= 0 || c->kv_block_size > 4096 || c->kv_num_blocks <= 0 || c->max_seqs <= 0 ||
      c->max_ctx <= 0 || c->max_batch <= 0)
    return bad(DTD_E_ARG, "%s", "KV pool, sequence and batch limits must be positive");
  if (c->max_batch > kMaxBatch) return bad(DTD_E_UNSUPPORTED, "max_batch %d > %d", c->max_batch, kMaxBatch);
  if (c->head_dim % 4 || c->head_dim < 8 || c->head_dim > 128)
    return bad(DTD_E_UNSUPPORTED, "head_dim %d (a multiple of 4 in [8, 128] supported)", c->head_dim);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G * c->head_dim > 2048) return bad(DTD_E_UNSUPPORTED, "query group size x head_dim = %d > 2048", G * c->head_dim);
  const int qd = c->n_q_heads * c->head_dim;
  if (qd > 16384) return bad(DTD_E_UNSUPPORTED, "n_q_heads x head_dim = %d > 16384", qd);
  const int v = vec_elems(c->wfmt);
  if (c->dim % v || c->ffn_dim % v || qd % v)
    return bad(DTD_E_UNSUPPORTED, "dim, ffn_dim and n_q_heads*head_dim must be multiples of %d", v);
  if ((c->wfmt == DTD_W_Q8_0 || c->wfmt == DTD_W_Q4_0) && (c->dim % 32 || c->ffn_dim % 32 || qd % 32))
    return bad(DTD_E_ARG, "%s", "Q8_0 and Q4_0 need every matrix width to be a multiple of 32");
  if ((int64_t)c->max_ctx * c->kv_block_size > (int64_t)1 << 40) return bad(DTD_E_ARG, "%s", "max_ctx too large");
  if (msg && msg_len > 0) msg[0] = 0;
  return DTD_OK;
}

// expected weight parts, in a fixed order
static std::vector<dtd_tensor_spec> expected_parts(const dtd_config* c) {
  std::vector<dtd_tensor_spec> out;
  const int D = c->dim, F = c->ffn_dim, V = c->vocab;
  const int qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  auto add = [&](const std::string& name, int rows, int cols, int elem, int64_t nbytes) {
    dtd_tensor_spec s{};
    snprintf(s.name, sizeof(s.name), "%s", name.c_str());
    s.rows = rows; s.cols = cols; s.elem = elem; s.nbytes = nbytes;
    out.push_back(s);
  };
  auto mat = [&](const std::string& base, int rows, int cols) {
    if (c->wfmt == DTD_W_BF16) {
      add(base + ".w", rows, cols, 2, (int64_t)rows * cols * 2);
    } else {
      add(base + ".q", rows, cols, 1, (int64_t)rows * cols / (c->wfmt == DTD_W_Q4_0 ? 2 : 1));
      if (c->wfmt == DTD_W_INT8_ROW) add(base + ".s", rows, 1, 4, (int64_t)rows * 4);
      else add(base + ".s", rows, cols / 32, 2, (int64_t)rows * (cols / 32) * 2);
    }
  };
  auto gain = [&](const std::string& base) { add(base + ".g", 1, D, 4, (int64_t)D * 4); };
  mat("tok_emb", V, D);
  for (int i = 0; i < c->n_layers; i++) {
    const std::string L = "L" + std::to_string(i);
    gain(L + ".attn_norm");
    mat(L + ".wq", qd, D);
    mat(L + ".wk", kvd, D);
    mat(L + ".wv", kvd, D);
    mat(L + ".wo", D, qd);
    gain(L + ".ffn_norm");
    mat(L + ".w_gate", F, D);
    mat(L + ".w_up", F, D);
    mat(L + ".w_down", D, F);
  }
  gain("final_norm");
  if (!c->tied_embeddings) mat("lm_head", V, D);
  return out;
}

static Dims make_dims(const dtd_config* c) {
  Dims d{};
  d.D = c->dim; d.L = c->n_layers; d.Hq = c->n_q_heads; d.Hkv = c->n_kv_heads; d.hd = c->head_dim;
  d.F = c->ffn_dim; d.V = c->vocab;
  d.G = d.Hq / d.Hkv;
  d.q_dim = d.Hq * d.hd; d.kv_dim = d.Hkv * d.hd; d.qkv_rows = d.q_dim + 2 * d.kv_dim;
  d.bs = c->kv_block_size;
  d.max_blocks = (c->max_ctx + d.bs - 1) / d.bs;
  d.max_ctx = c->max_ctx;
  // Split the context so that a full batch at full context gives ~4096 work items (one
  // wave each in the common-shape attention kernel: several per compute unit).
  const int64_t work = (int64_t)c->max_batch * d.Hkv * c->max_ctx;
  int ct = kAttnTile;
  while (ct < 2048 && (int64_t)ct * 4096 < work) ct <<= 1;
  d.ct = ct;
  d.nch = (c->max_ctx + ct - 1) / ct;
  d.eps = c->rms_eps;
  d.wfmt = c->wfmt; d.act = c->act; d.kvfmt = c->kvfmt;
  return d;
}

static size_t act_bytes(int act) { return act == DTD_ACT_BF16 ? 2 : 4; }
static size_t kv_elem_bytes(int kvfmt) { return kvfmt == DTD_KV_F32 ? 4 : (kvfmt == DTD_KV_BF16 ? 2 : 1); }

// stored row of logical row r within the fused QKV matrix (q/k heads pair rows (i, i+hd/2))
static int qkv_stored_row(const Dims& d, int part, int r) {
  if (part == 2) return d.q_dim + d.kv_dim + r;
  const int h = r / d.hd, i = r % d.hd, half = d.hd / 2;
  const int p = i < half ? 2 * i : 2 * (i - half) + 1;
  return (part == 0 ? 0 : d.q_dim) + h * d.hd + p;
}

static void release_weights(dtd_engine* e) {
  for (void* p : e->weight_allocs) (void)hipFree(p);
  e->weight_allocs.clear();
  e->layers.clear();
  e->loaded = false;
}

// ---------------------------------------------------------------------------------------
// host-only queries
// ---------------------------------------------------------------------------------------

extern "C" dtd_status dtd_validate_config(const dtd_config* cfg, char* msg, int32_t msg_len) {
  return check_config(cfg, msg, msg_len);
}

extern "C" int32_t dtd_expected_tensors(const dtd_config* cfg, dtd_tensor_spec* out, int32_t cap) {
  const dtd_status st = check_config(cfg, nullptr, 0);
  if (st != DTD_OK) return st;
  const auto v = expected_parts(cfg);
  if (out)
    for (int32_t i = 0; i < cap && i < (int32_t)v.size(); i++) out[i] = v[(size_t)i];
  return (int32_t)v.size();
}

// ---------------------------------------------------------------------------------------
// lifecycle
// ---------------------------------------------------------------------------------------

template <typename T>
static dtd_status dev_alloc(dtd_engine* e, T** p, size_t bytes) {
  void* q = nullptr;
  if (bytes == 0) bytes = 16;
  hipError_t r = hipMalloc(&q, bytes);
  if (r != hipSuccess) {
    (void)hipGetLastError();
    return fail(e, DTD_E_OOM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(r));
  }
  *p = (T*)q;
  return DTD_OK;
}

static void free_all(dtd_engine* e) {
  release_weights(e);
  void* ps[] = {e->rope_cos, e->rope_sin, e->kpool, e->vpool, e->kspool, e->vspool, e->bt_dev,
                e->x, e->xn, e->q, e->knew, e->vnew, e->partials, e->gemm_partials, e->o, e->h, e->logits,
                e->err_dev, e->desc_dev, e->rows_dev, e->players, e->tags, e->tok_scratch,
                e->scores_dev, e->attn_stat, e->evict_dev, e->p_score_q, e->p_score_stat, e->kvpos_dev};
  for (void* p : ps)
    if (p) (void)hipFree(p);
  if (e->desc_host) (void)hipHostFree(e->desc_host);
  if (e->evict_host) (void)hipHostFree(e->evict_host);
  for (int i = 0; i < kEvictRing; i++)
    if (e->evict_ev[i]) (void)hipEventDestroy(e->evict_ev[i]);
  if (e->err_host) (void)hipHostFree(e->err_host);
  for (int i = 0; i < kRing; i++)
    if (e->desc_ev[i]) (void)hipEventDestroy(e->desc_ev[i]);
  for (auto& t : e->timers) { (void)hipEventDestroy(t.a); (void)hipEventDestroy(t.b); }
}

extern "C" dtd_status dtd_create(const dtd_config* cfg, void* hip_stream, dtd_engine** out) {
  g_create_err.clear();
  if (!out) { g_create_err = "dtd_create: out is null"; return DTD_E_ARG; }
  *out = nullptr;
  char vmsg[256] = {0};
  const dtd_status vs = check_config(cfg, vmsg, (int32_t)sizeof(vmsg));
  if (vs != DTD_OK) {
    g_create_err = std::string("dtd_create: ") + vmsg;
    return vs;
  }
  dtd_engine* e = new dtd_engine();
  for (int i = 0; i < kRing; i++) { e->desc_ev[i] = nullptr; e->desc_ev_used[i] = false; }
  for (int i = 0; i < kEvictRing; i++) { e->evict_ev[i] = nullptr; e->evict_ev_used[i] = false; }
  e->cfg = *cfg;
  e->d = make_dims(cfg);
  e->stream = (hipStream_t)hip_stream;
  const Dims& d = e->d;
  // a failed create leaves its message for dtd_last_error(NULL) on this thread
  auto cleanup = [&](dtd_status st) {
    g_create_err = e->err.empty() ? "dtd_create: a HIP call failed: " + std::string(hipGetErrorString(hipGetLastError()))
                                  : "dtd_create: " + e->err;
    free_all(e);
    delete e;
    return st;
  };
  if (hipGetDevice(&e->device) != hipSuccess) { e->err = "hipGetDevice failed"; return cleanup(DTD_E_HIP); }
  {
    hipError_t r;
    e->scratch_dev = scratch_on_current_device(e->device, &r);
    if (!e->scratch_dev) {
      e->err = std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(r);
      return cleanup(DTD_E_HIP);
    }
  }

  // RoPE tables: angle pos * theta^(-2i/d) in double, cos/sin stored as fp32
  const int half = d.hd / 2;
  std::vector<float> cs((size_t)cfg->max_ctx * half), sn((size_t)cfg->max_ctx * half);
  for (int p = 0; p < cfg->max_ctx; p++)
    for (int i = 0; i < half; i++) {
      const double f = std::pow((double)cfg->rope_theta, -2.0 * i / d.hd);
      const double a = (double)p * f;
      cs[(size_t)p * half + i] = (float)std::cos(a);
      sn[(size_t)p * half + i] = (float)std::sin(a);
    }
  dtd_status st;
  if ((st = dev_alloc(e, &e->rope_cos, cs.size() * 4)) || (st = dev_alloc(e, &e->rope_sin, sn.size() * 4)))
    return cleanup(st);
  if (hipMemcpy(e->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(e->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
    return cleanup(DTD_E_HIP);

  // KV pool: per layer K, V [n_blocks][Hkv][bs][hd] (+ fp16 scales [n_blocks][Hkv][bs])
  e->kv_layer_elems = (size_t)cfg->kv_num_blocks * d.Hkv * d.bs * d.hd;
  e->kv_layer_scales = (size_t)cfg->kv_num_blocks * d.Hkv * d.bs;
  const size_t kvb = e->kv_layer_elems * kv_elem_bytes(cfg->kvfmt) * d.L;
  if ((st = dev_alloc(e, &e->kpool, kvb)) || (st = dev_alloc(e, &e->vpool, kvb))) return cleanup(st);
  if (cfg->kvfmt == DTD_KV_I8) {
    if ((st = dev_alloc(e, &e->kspool, e->kv_layer_scales * 2 * d.L)) ||
        (st = dev_alloc(e, &e->vspool, e->kv_layer_scales * 2 * d.L)))
      return cleanup(st);
  }
  const size_t bt_bytes = (size_t)cfg->max_seqs * d.max_blocks * 4;
  if ((st = dev_alloc(e, &e->bt_dev, bt_bytes))) return cleanup(st);
  if (hipMemset(e->bt_dev, 0, bt_bytes) != hipSuccess) return cleanup(DTD_E_HIP);

  // work buffers hold a decode batch or a prefill chunk, whichever is larger
  const int MB = std::max(cfg->max_batch, kPrefillChunk);
  e->mb = MB;
  const size_t ab = act_bytes(cfg->act);
  if ((st = dev_alloc(e, &e->x, (size_t)MB * d.D * 4)) ||
      (st = dev_alloc(e, &e->xn, (size_t)MB * d.D * ab)) ||
      (st = dev_alloc(e, &e->q, (size_t)MB * d.q_dim * 4)) ||
      (st = dev_alloc(e, &e->knew, (size_t)MB * d.kv_dim * 4)) ||
      (st = dev_alloc(e, &e->vnew, (size_t)MB * d.kv_dim * 4)) ||
      (st = dev_alloc(e, &e->partials, std::max((size_t)MB * d.nch, (size_t)(cfg->max_ctx + kAttnTile - 1) / kAttnTile) *
                                              d.Hq * (d.hd + 2) * 4)) ||
      (st = dev_alloc(e, &e->o, (size_t)MB * d.q_dim * ab)) ||
      (st = dev_alloc(e, &e->h, (size_t)MB * d.F * ab)) ||
      (st = dev_alloc(e, &e->logits, (size_t)MB * d.V * 4)) ||
      (st = dev_alloc(e, &e->err_dev, 16)) || (st = dev_alloc(e, &e->desc_dev, sizeof(StepDesc))) ||
      (st = dev_alloc(e, &e->tok_scratch, (size_t)MB * 4)) ||
      (st = dev_alloc(e, &e->scores_dev, (size_t)cfg->max_seqs * cfg->max_ctx * 4)) ||
      (st = dev_alloc(e, &e->attn_stat, (size_t)MB * d.Hq * 2 * 4)) ||
      (st = dev_alloc(e, &e->p_score_q, (size_t)d.L * d.q_dim * 4)) ||
      (st = dev_alloc(e, &e->p_score_stat, (size_t)d.L * d.Hq * 2 * 4)) ||
      (st = dev_alloc(e, &e->evict_dev, (size_t)3 * cfg->max_ctx * 4)) ||
      (st = dev_alloc(e, &e->kvpos_dev, (size_t)cfg->max_seqs * cfg->max_ctx * 4)))
    return cleanup(st);
  if (hipMemset(e->err_dev, 0, 16) != hipSuccess) return cleanup(DTD_E_HIP);

  // persistent batch-1 step kernel: one workgroup per compute unit, all resident
  {
    int cus = 0, coop = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, e->device) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, e->device) != hipSuccess)
      return cleanup(DTD_E_HIP);
    e->cus = cus > 0 ? cus : 1;
    // split-K sums of the matrix-core projections (batched steps)
    if (MB >= 2 && gemm_eligible(d, MB)) {
      if ((st = dev_alloc(e, &e->gemm_partials, gemm_partial_bytes(d, MB, e->cus)))) return cleanup(st);
    }
    e->p_nch = (cfg->max_ctx + kAttnTile - 1) / kAttnTile;
    e->p_smem = persistent_smem_bytes(d, e->p_nch, cus > 0 ? cus : 1);
    if (coop && cus > 0 && persistent_supports(d) && persistent_prepare(d, e->p_smem, &per_cu) == hipSuccess &&
        per_cu >= 1) {
      e->persist_ok = true;
      e->nwg = cus;
    }
    (void)hipGetLastError();
    const int nw = e->nwg > 0 ? e->nwg : 1;
    // tagged buffers: q, k, v, o, x_mid, h, x_out, chunk partials, per-workgroup argmax
    e->tags_words = (size_t)2 * d.q_dim + 2 * (size_t)d.kv_dim + 2 * (size_t)d.D + h_buffer_words(d.F, nw) +
                    (size_t)d.Hq * e->p_nch * (d.hd + 2) + 2 * (size_t)nw;
    if ((st = dev_alloc(e, &e->players, sizeof(PLayer) * (size_t)d.L)) ||
        (st = dev_alloc(e, &e->tags, sizeof(uint64_t) * e->tags_words)))
      return cleanup(st);
    if (hipMemset(e->tags, 0, sizeof(uint64_t) * e->tags_words) != hipSuccess) return cleanup(DTD_E_HIP);
  }
  if (hipHostMalloc((void**)&e->desc_host, sizeof(StepDesc) * kRing, 0) != hipSuccess ||
      hipHostMalloc((void**)&e->err_host, 16, 0) != hipSuccess ||
      hipHostMalloc((void**)&e->evict_host, sizeof(int32_t) * kEvictRing * 2 * d.max_blocks, 0) != hipSuccess)
    return cleanup(DTD_E_OOM);
  memset(e->err_host, 0, 16);
  for (int i = 0; i < kRing; i++)
    if (hipEventCreateWithFlags(&e->desc_ev[i], hipEventDisableTiming) != hipSuccess) return cleanup(DTD_E_HIP);
  for (int i = 0; i < kEvictRing; i++)
    if (hipEventCreateWithFlags(&e->evict_ev[i], hipEventDisableTiming) != hipSuccess) return cleanup(DTD_E_HIP);

  // free lists: slots in order; blocks in a fixed shuffled order so that block tables are
  // never the identity (the paged path is exercised even for one sequence)
  for (int s = cfg->max_seqs - 1; s >= 0; s--) e->free_slots.push_back(s);
  e->free_blocks.resize((size_t)cfg->kv_num_blocks);
  for (int i = 0; i < cfg->kv_num_blocks; i++) e->free_blocks[(size_t)i] = i;
  e->blk_ref.assign((size_t)cfg->kv_num_blocks, 0);
  uint64_t lcg = 0x9E3779B97F4A7C15ull;
  for (int i = cfg->kv_num_blocks - 1; i > 0; i--) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    const int j = (int)((lcg >> 33) % (uint64_t)(i + 1));
    std::swap(e->free_blocks[(size_t)i], e->free_blocks[(size_t)j]);
  }
  *out = e;
  return DTD_OK;
}

extern "C" void dtd_destroy(dtd_engine* e) {
  if (!e) return;
  (void)hipSetDevice(e->device);
  (void)hipStreamSynchronize(e->stream);
  free_all(e);
  delete e;
}

extern "C" const char* dtd_last_error(const dtd_engine* e) {
  if (e) return e->err.c_str();
  return g_create_err.empty() ? "null engine" : g_create_err.c_str();
}

// ---------------------------------------------------------------------------------------
// weights
// ---------------------------------------------------------------------------------------

namespace {

struct SrcPart {
  const uint8_t* host = nullptr;  // host copy of the caller's part
  std::vector<uint8_t> own;       // staging if the caller's part lives on the device
  int64_t nbytes = 0;
};

// one logical matrix: codes/bits (part "q" or "w") and scales (part "s")
struct SrcMat {
  const SrcPart* w = nullptr;
  const SrcPart* s = nullptr;
  int rows = 0, cols = 0;
};

}  // namespace

// Packs several logical matrices stacked (or interleaved) by a row map into one device
// matrix: stored row `r` takes row srcrow[r] of matrix srcmat[r].
static dtd_status upload_packed(dtd_engine* e, const std::vector<SrcMat>& mats,
                                const std::vector<std::pair<int, int>>& rowmap, int cols, MatDev* out) {
  const int wfmt = e->cfg.wfmt;
  const int rows = (int)rowmap.size();
  const size_t eb = wfmt == DTD_W_BF16 ? 2 : 1;
  const size_t wrow = wfmt == DTD_W_Q4_0 ? (size_t)cols / 2 : (size_t)cols * eb;
  const size_t srow = wfmt == DTD_W_INT8_ROW ? 4 : (wfmt == DTD_W_BF16 ? 0 : (size_t)(cols / 32) * 2);
  std::vector<uint8_t> wbuf((size_t)rows * wrow), sbuf((size_t)rows * srow);
  for (int r = 0; r < rows; r++) {
    const SrcMat& m = mats[(size_t)rowmap[(size_t)r].first];
    const int sr = rowmap[(size_t)r].second;
    memcpy(wbuf.data() + (size_t)r * wrow, m.w->host + (size_t)sr * wrow, wrow);
    if (srow) memcpy(sbuf.data() + (size_t)r * srow, m.s->host + (size_t)sr * srow, srow);
  }
  void* wd = nullptr;
  void* sd = nullptr;
  dtd_status st;
  if ((st = dev_alloc(e, &wd, wbuf.size()))) return st;
  e->weight_allocs.push_back(wd);
  HIP_OK(e, hipMemcpy(wd, wbuf.data(), wbuf.size(), hipMemcpyHostToDevice));
  if (srow) {
    if ((st = dev_alloc(e, &sd, sbuf.size()))) return st;
    e->weight_allocs.push_back(sd);
    HIP_OK(e, hipMemcpy(sd, sbuf.data(), sbuf.size(), hipMemcpyHostToDevice));
  }
  out->w = wd;
  out->s = sd;
  out->rows = rows;
  out->cols = cols;
  return DTD_OK;
}

extern "C" dtd_status dtd_load_weights(dtd_engine* e, const dtd_tensor* t, int32_t n) {
  if (!e) return DTD_E_ARG;
  if (e->broken) return fail(e, DTD_E_STATE, "engine unusable after a HIP error");
  if (!t || n <= 0) return fail(e, DTD_E_ARG, "no tensors");
  HIP_OK(e, hipSetDevice(e->device));
  const auto spec = expected_parts(&e->cfg);
  std::unordered_map<std::string, size_t> idx;
  for (size_t i = 0; i < spec.size(); i++) idx[spec[i].name] = i;
  std::vector<SrcPart> parts(spec.size());
  std::vector<bool> seen(spec.size(), false);
  for (int32_t i = 0; i < n; i++) {
    if (!t[i].name || !t[i].data) return fail(e, DTD_E_ARG, "tensor %d: null name or data", i);
    auto it = idx.find(t[i].name);
    if (it == idx.end()) return fail(e, DTD_E_ARG, "unknown tensor '%s'", t[i].name);
    if (seen[it->second]) return fail(e, DTD_E_ARG, "duplicate tensor '%s'", t[i].name);
    if (t[i].nbytes != spec[it->second].nbytes)
      return fail(e, DTD_E_ARG, "tensor '%s': %lld bytes, expected %lld", t[i].name,
                  (long long)t[i].nbytes, (long long)spec[it->second].nbytes);
    seen[it->second] = true;
  }
  for (size_t i = 0; i < spec.size(); i++)
    if (!seen[i]) return fail(e, DTD_E_ARG, "missing tensor '%s'", spec[i].name);
  // all parts validated: only now touch engine state
  for (int32_t i = 0; i < n; i++) {
    SrcPart& p = parts[idx[t[i].name]];
    p.nbytes = t[i].nbytes;
    if (t[i].on_device) {
      p.own.resize((size_t)t[i].nbytes);
      HIP_OK(e, hipMemcpy(p.own.data(), t[i].data, (size_t)t[i].nbytes, hipMemcpyDeviceToHost));
      p.host = p.own.data();
    } else {
      p.host = (const uint8_t*)t[i].data;
    }
  }
  auto part = [&](const std::string& name) -> const SrcPart* { return &parts[idx[name]]; };
  const bool bf = e->cfg.wfmt == DTD_W_BF16;
  auto srcmat = [&](const std::string& base, int rows, int cols) {
    SrcMat m;
    m.w = part(base + (bf ? ".w" : ".q"));
    m.s = bf ? nullptr : part(base + ".s");
    m.rows = rows; m.cols = cols;
    return m;
  };
  auto gain = [&](const std::string& name, float** dst) -> dtd_status {
    dtd_status st = dev_alloc(e, dst, (size_t)e->d.D * 4);
    if (st) return st;
    e->weight_allocs.push_back(*dst);
    HIP_OK(e, hipMemcpy(*dst, part(name + ".g")->host, (size_t)e->d.D * 4, hipMemcpyHostToDevice));
    return DTD_OK;
  };

  release_weights(e);
  const Dims& d = e->d;
  dtd_status st;
  auto identity = [](int src, int rows) {
    std::vector<std::pair<int, int>> m((size_t)rows);
    for (int r = 0; r < rows; r++) m[(size_t)r] = {src, r};
    return m;
  };
  if ((st = upload_packed(e, {srcmat("tok_emb", d.V, d.D)}, identity(0, d.V), d.D, &e->emb))) goto bad;
  e->layers.resize((size_t)d.L);
  for (int l = 0; l < d.L; l++) {
    const std::string L = "L" + std::to_string(l);
    LayerW& W = e->layers[(size_t)l];
    if ((st = gain(L + ".attn_norm", &W.attn_norm)) || (st = gain(L + ".ffn_norm", &W.ffn_norm))) goto bad;
    {
      std::vector<SrcMat> m = {srcmat(L + ".wq", d.q_dim, d.D), srcmat(L + ".wk", d.kv_dim, d.D),
                               srcmat(L + ".wv", d.kv_dim, d.D)};
      std::vector<std::pair<int, int>> map((size_t)d.qkv_rows);
      for (int part_i = 0; part_i < 3; part_i++) {
        const int rows = part_i == 0 ? d.q_dim : d.kv_dim;
        for (int r = 0; r < rows; r++) map[(size_t)qkv_stored_row(d, part_i, r)] = {part_i, r};
      }
      if ((st = upload_packed(e, m, map, d.D, &W.qkv))) goto bad;
    }
    if ((st = upload_packed(e, {srcmat(L + ".wo", d.D, d.q_dim)}, identity(0, d.D), d.q_dim, &W.o))) goto bad;
    {
      std::vector<SrcMat> m = {srcmat(L + ".w_gate", d.F, d.D), srcmat(L + ".w_up", d.F, d.D)};
      std::vector<std::pair<int, int>> map((size_t)2 * d.F);
      for (int f = 0; f < d.F; f++) { map[(size_t)2 * f] = {0, f}; map[(size_t)2 * f + 1] = {1, f}; }
      if ((st = upload_packed(e, m, map, d.D, &W.gu))) goto bad;
    }
    if ((st = upload_packed(e, {srcmat(L + ".w_down", d.D, d.F)}, identity(0, d.D), d.F, &W.down))) goto bad;
  }
  if ((st = gain("final_norm", &e->final_norm))) goto bad;
  if (e->cfg.tied_embeddings) e->head = e->emb;
  else if ((st = upload_packed(e, {srcmat("lm_head", d.V, d.D)}, identity(0, d.V), d.D, &e->head))) goto bad;
  {
    std::vector<PLayer> tab((size_t)d.L);
    const size_t kvb = kv_elem_bytes(e->cfg.kvfmt);
    for (int l = 0; l < d.L; l++) {
      const LayerW& W = e->layers[(size_t)l];
      PLayer& P = tab[(size_t)l];
      P.qkv = W.qkv; P.o = W.o; P.gu = W.gu; P.down = W.down;
      P.attn_norm = W.attn_norm; P.ffn_norm = W.ffn_norm;
      P.kv.k = (uint8_t*)e->kpool + (size_t)l * e->kv_layer_elems * kvb;
      P.kv.v = (uint8_t*)e->vpool + (size_t)l * e->kv_layer_elems * kvb;
      P.kv.ks = e->kspool ? e->kspool + (size_t)l * e->kv_layer_scales : nullptr;
      P.kv.vs = e->vspool ? e->vspool + (size_t)l * e->kv_layer_scales : nullptr;
    }
    HIP_OK(e, hipMemcpy(e->players, tab.data(), sizeof(PLayer) * tab.size(), hipMemcpyHostToDevice));
  }
  e->loaded = true;
  return DTD_OK;
bad:
  release_weights(e);
  return st;
}

// ---------------------------------------------------------------------------------------
// the step
// ---------------------------------------------------------------------------------------

static hipError_t timed_begin(dtd_engine* e, int kind, TimerPair** tp) {
  *tp = nullptr;
  if (e->timing_kind != kind) return hipSuccess;
  if (e->timers_used == e->timers.size()) {
    TimerPair p;
    hipError_t r = hipEventCreate(&p.a);
    if (r != hipSuccess) return r;
    r = hipEventCreate(&p.b);
    if (r != hipSuccess) return r;
    e->timers.push_back(p);
  }
  *tp = &e->timers[e->timers_used++];
  return hipEventRecord((*tp)->a, e->stream);
}

static hipError_t timed_end(dtd_engine* e, TimerPair* tp) {
  return tp ? hipEventRecord(tp->b, e->stream) : hipSuccess;
}

#define TIMED(kind, call)                                   \
  do {                                                      \
    TimerPair* _tp;                                         \
    HIP_OK(e, timed_begin(e, (kind), &_tp));                \
    HIP_OK(e, (call));                                      \
    HIP_OK(e, timed_end(e, _tp));                           \
  } while (0)

struct Update { int slot, lblock, pblock; };

// Probe records of dtd_debug_decode_probe: per layer, fields [B][n] in this order.
static ProbeLayout probe_layout(const Dims& d, int B, size_t ab) {
  ProbeLayout p{};
  size_t off = 0;
  auto field = [&](size_t n, size_t eb) { const size_t o = off; off += (size_t)B * n * eb; return o; };
  p.x_in = field(d.D, 4);
  p.xn = field(d.D, ab);
  p.q = field(d.q_dim, 4);
  p.k = field(d.kv_dim, 4);
  p.v = field(d.kv_dim, 4);
  p.o = field(d.q_dim, ab);
  p.x_mid = field(d.D, 4);
  p.xn2 = field(d.D, ab);
  p.h = field(d.F, ab);
  p.x_out = field(d.D, 4);
  p.record = off;
  return p;
}

// With inject/capture (debug probe): every kernel of every layer reads its input from the
// inject record and its output is copied to the capture record, so each kernel can be
// compared with the reference operation on identical inputs.
static dtd_status run_sub_steps(dtd_engine* e, int B, bool do_head, const uint8_t* inject, uint8_t* capture,
                                float* partials, float* gemm_partials, bool append_first);

// partials: the split-K attention partials of the per-sub-step schedule (the engine's buffer,
// or the allocation-free entry point's static scratch).  force_per_kernel: run that schedule
// even at batch 1; no_timing: leave the kernel-timing hooks (which may create events) out.
// Split-K of the decode attention for the one-wave-per-chunk kernel: each context (len_b =
// pos_b + 1) cut into equal chunks of ct_b positions (a multiple of 16) of at most T, with T
// the shortest length (from 64, at most 2048, and at least len_b / nch for every b) for which
// the whole batch's chunks, one wave each per KV head, fit in `slots` resident waves.  With
// one fixed chunk length instead, mixed contexts leave short last chunks and more waves than
// slots, and the last ones run alone.  Writes ct[b] and the running chunk count cend[b];
// returns the batch's chunk count.
static int plan_chunks(int B, const int* poss, int Hkv, int nch, int64_t slots, int32_t* ct, int32_t* cend) {
  auto r16 = [](int64_t x) { return (int)((x + 15) / 16 * 16); };
  int64_t tot = 0;
  int maxlen = 1;
  for (int b = 0; b < B; b++) {
    tot += poss[b] + 1;
    maxlen = std::max(maxlen, poss[b] + 1);
  }
  auto chunks = [&](int T, bool write) {
    int n = 0;
    for (int b = 0; b < B; b++) {
      const int len = poss[b] + 1, n0 = (len + T - 1) / T;
      const int c = r16((len + n0 - 1) / n0);
      n += (len + c - 1) / c;
      if (write) {
        ct[b] = c;
        cend[b] = n;
      }
    }
    return n;
  };
  int T = std::max(64, std::max(r16((tot * Hkv + slots - 1) / slots), r16((maxlen + nch - 1) / nch)));
  T = std::min(T, 2048);
  while (T < 2048 && (int64_t)chunks(T, false) * Hkv > slots) T += 16;
  return chunks(T, true);
}

// The descriptor's attention chunks: planned (8 resident waves per compute unit, two per
// SIMD) for the one-wave-per-chunk kernel, else every context split at d.ct.
static void plan_attention_chunks(dtd_engine* e, StepDesc* hd, int B, const int* poss, bool wplan) {
  const Dims& d = e->d;
  e->step_chunks = 0;
  hd->n_chunks = 0;
  if (!wplan) {
    for (int b = 0; b < B; b++) hd->ct[b] = d.ct;
    return;
  }
  hd->n_chunks = plan_chunks(B, poss, d.Hkv, d.nch, (int64_t)e->cus * 8, hd->ct, hd->cend);
  e->step_chunks = hd->n_chunks;
}

static dtd_status run_step(dtd_engine* e, int B, const int* slots, const int* poss, const int* pblks,
                           const int32_t* tokens, int32_t* next, float* logits_out, bool do_head,
                           const Update* upd, int n_upd, const uint8_t* inject = nullptr,
                           uint8_t* capture = nullptr, float* partials = nullptr, float* gemm_partials = nullptr,
                           bool force_per_kernel = false, bool no_timing = false, bool append_first = false,
                           const StepExtra* extra = nullptr) {
  if (!partials) partials = e->partials;
  if (!gemm_partials) gemm_partials = e->gemm_partials;
  const Dims& d = e->d;
  hipStream_t st = e->stream;
  // descriptor into the next pinned ring slot, then one host->device copy
  StepDesc* hd = &e->desc_host[e->ring];
  if (e->desc_ev_used[e->ring]) HIP_OK(e, hipEventSynchronize(e->desc_ev[e->ring]));
  memset(hd, 0, sizeof(StepDesc));
  hd->batch = B;
  hd->do_head = do_head ? 1 : 0;
  hd->n_updates = (int32_t)n_upd;
  hd->tokens = tokens;
  hd->next_tokens = next;
  hd->logits_out = logits_out;
  e->step_score_min = 1 << 30;
  e->step_max_pos = 0;
  for (int b = 0; b < B; b++) {
    hd->pos[b] = poss[b]; hd->slot[b] = slots[b]; hd->pos_block[b] = pblks[b];
    hd->rpos[b] = extra && extra->rpos ? extra->rpos[b] : poss[b];
    hd->score_from[b] = extra && extra->score_from ? extra->score_from[b] : d.L;
    e->step_score_min = std::min(e->step_score_min, hd->score_from[b]);
    e->step_max_pos = std::max(e->step_max_pos, poss[b]);
  }
  plan_attention_chunks(e, hd, B, poss, attn_w_shape(d) && !(append_first && B >= 2));
  for (int u = 0; u < n_upd; u++) {
    hd->upd[u][0] = upd[u].slot; hd->upd[u][1] = upd[u].lblock; hd->upd[u][2] = upd[u].pblock;
  }
  HIP_OK(e, hipMemcpyAsync(e->desc_dev, hd, sizeof(StepDesc), hipMemcpyHostToDevice, st));
  HIP_OK(e, hipEventRecord(e->desc_ev[e->ring], st));
  e->desc_ev_used[e->ring] = true;
  e->ring = (e->ring + 1) % kRing;

  if (e->persist_ok && B == 1 && !e->capture && e->path != 1 && !force_per_kernel) {
    PersistArgs a{};
    a.d = d;
    a.layers = e->players;
    a.emb = e->emb;
    a.head = e->head;
    a.final_norm = e->final_norm;
    a.desc = e->desc_dev;
    a.bt = e->bt_dev;
    a.rope_cos = e->rope_cos;
    a.rope_sin = e->rope_sin;
    {
      uint64_t* t = e->tags;
      a.t_q = t; t += d.q_dim;
      a.t_k = t; t += d.kv_dim;
      a.t_v = t; t += d.kv_dim;
      a.t_o = t; t += d.q_dim;
      a.t_xm = t; t += d.D;
      a.t_h = t; t += h_buffer_words(d.F, e->nwg);
      a.t_xo = t; t += d.D;
      a.t_part = t; t += (size_t)d.Hq * e->p_nch * (d.hd + 2);
      a.t_am = t;
    }
    // tags are 32-bit: before they would wrap, clear the buffers and start again at 1
    const uint32_t ntag = (uint32_t)persistent_tags_per_step(d);
    if (e->epoch > 0xffffffffu - ntag) {
      HIP_OK(e, hipMemsetAsync(e->tags, 0, sizeof(uint64_t) * e->tags_words, st));
      e->epoch = 1;
    }
    a.epoch = e->epoch;
    a.logits = e->logits;
    a.err = e->err_dev;
    // attention split: about one (kv head, chunk) item per workgroup, chunks of >= 64
    const int64_t T = poss[0] + 1;
    int ct = (int)((T * d.Hkv + e->nwg - 1) / e->nwg);
    ct = std::max(kAttnTile, (ct + kAttnTile - 1) / kAttnTile * kAttnTile);
    a.ct = ct;
    a.nch = e->p_nch;
    a.xs_floats = (int)persistent_xs_floats(d, e->p_nch);
    a.inject = inject;
    a.capture = capture;
    a.po = probe_layout(d, 1, act_bytes(e->cfg.act));
    a.score_q = e->p_score_q;
    a.score_stat = e->p_score_stat;
    TIMED(6, launch_persistent(a, e->nwg, e->p_smem, st));
    e->epoch += ntag;
    // a KV budget's score sums over the scored layers, from the queries and softmax
    // statistics the step kernel kept (the new entry is in the cache by now)
    // (one launch for all of them)
    const size_t kvb = kv_elem_bytes(e->cfg.kvfmt);
    const int l0 = std::max(e->step_score_min, 0);
    if (l0 < d.L) {
      KvLayer kv;
      kv.k = (uint8_t*)e->kpool + (size_t)l0 * e->kv_layer_elems * kvb;
      kv.v = (uint8_t*)e->vpool + (size_t)l0 * e->kv_layer_elems * kvb;
      kv.ks = e->kspool ? e->kspool + (size_t)l0 * e->kv_layer_scales : nullptr;
      kv.vs = e->vspool ? e->vspool + (size_t)l0 * e->kv_layer_scales : nullptr;
      HIP_OK(e, launch_score(d, e->desc_dev, 1, e->step_max_pos, l0, d.L - l0, e->p_score_q + (size_t)l0 * d.q_dim,
                             d.q_dim, kv, e->kv_layer_elems * kvb, e->kv_layer_scales * 2, e->bt_dev,
                             e->p_score_stat + (size_t)l0 * d.Hq * 2, (size_t)d.Hq * 2, e->scores_dev, st));
    }
    return DTD_OK;
  }
  if (e->path == 2 && !force_per_kernel)
    return fail(e, DTD_E_UNSUPPORTED, "persistent step kernel unavailable for this call");
  const int timing_saved = e->timing_kind;
  if (no_timing) e->timing_kind = -1;
  const dtd_status rs = run_sub_steps(e, B, do_head, inject, capture, partials, gemm_partials, append_first);
  e->timing_kind = timing_saved;
  return rs;
}

// The per-sub-step schedule of one step (the descriptor is already on the device).
static dtd_status run_sub_steps(dtd_engine* e, int B, bool do_head, const uint8_t* inject, uint8_t* capture,
                                float* partials, float* gemm_partials, bool append_first) {
  const Dims& d = e->d;
  hipStream_t st = e->stream;
  // a projection: on the matrix cores when the batch makes it a real GEMM, else the
  // weight-streaming GEMV
  const bool mfma = gemm_eligible(d, B);
  auto proj = [&](const MatDev& m, const void* xin, int epi, const EpiArgs& ea) {
    return mfma ? launch_gemm(d, m, xin, B, epi, ea, gemm_partials, e->cus, st) : launch_gemv(d, m, xin, B, epi, ea, st);
  };

  HIP_OK(e, launch_embed(d, e->emb, e->desc_dev, B, e->bt_dev, e->x, e->err_dev, st));
  const size_t ab = act_bytes(e->cfg.act);
  const ProbeLayout pl = probe_layout(d, B, ab);
  const bool probe = inject && capture;
  auto cp = [&](void* dst, const void* src, size_t n) {
    return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, st);
  };
  if (e->capture)
    HIP_OK(e, hipMemcpyAsync(e->capture, e->x, (size_t)B * d.D * 4, hipMemcpyDeviceToDevice, st));
  const size_t kvb = kv_elem_bytes(e->cfg.kvfmt);
  EpiArgs ea{};
  ea.desc = e->desc_dev;
  ea.q = e->q; ea.knew = e->knew; ea.vnew = e->vnew;
  ea.rope_cos = e->rope_cos; ea.rope_sin = e->rope_sin;
  ea.x = e->x; ea.h = e->h; ea.logits = e->logits;
  const size_t fx = (size_t)B * d.D * 4, fxn = (size_t)B * d.D * ab, fq = (size_t)B * d.q_dim * 4;
  const size_t fkv = (size_t)B * d.kv_dim * 4, fo = (size_t)B * d.q_dim * ab, fh = (size_t)B * d.F * ab;
  // On the matrix-core path (no probe records), a residual projection's split-K sums, the
  // residual add and the RMSNorm after it run as one launch: xn_ready says the norm of the
  // next block's input is already in xn.
  const bool fuse_norm = mfma && !probe;
  bool xn_ready = false;
  for (int l = 0; l < d.L; l++) {
    const LayerW& W = e->layers[(size_t)l];
    KvLayer kv;
    kv.k = (uint8_t*)e->kpool + (size_t)l * e->kv_layer_elems * kvb;
    kv.v = (uint8_t*)e->vpool + (size_t)l * e->kv_layer_elems * kvb;
    kv.ks = e->kspool ? e->kspool + (size_t)l * e->kv_layer_scales : nullptr;
    kv.vs = e->vspool ? e->vspool + (size_t)l * e->kv_layer_scales : nullptr;
    const uint8_t* in = probe ? inject + (size_t)l * pl.record : nullptr;
    uint8_t* out = probe ? capture + (size_t)l * pl.record : nullptr;
    if (probe) {
      HIP_OK(e, cp(e->x, in + pl.x_in, fx));
      HIP_OK(e, cp(out + pl.x_in, in + pl.x_in, fx));
    }
    if (!xn_ready) HIP_OK(e, launch_rmsnorm(d, e->x, W.attn_norm, e->xn, B, st));
    xn_ready = false;
    if (probe) {
      HIP_OK(e, cp(out + pl.xn, e->xn, fxn));
      HIP_OK(e, cp(e->xn, in + pl.xn, fxn));
    }
    TIMED(2, proj(W.qkv, e->xn, EPI_QKV, ea));
    if (probe) {
      HIP_OK(e, cp(out + pl.q, e->q, fq));
      HIP_OK(e, cp(out + pl.k, e->knew, fkv));
      HIP_OK(e, cp(out + pl.v, e->vnew, fkv));
      HIP_OK(e, cp(e->q, in + pl.q, fq));
      HIP_OK(e, cp(e->knew, in + pl.k, fkv));
      HIP_OK(e, cp(e->vnew, in + pl.v, fkv));
    }
    if (append_first) HIP_OK(e, launch_kv_append(d, e->desc_dev, B, e->knew, e->vnew, kv, st));
    const bool scored = l >= e->step_score_min;
    if (append_first && B >= 2) {
      // a prefill chunk (consecutive positions of one sequence, their K/V appended above):
      // blocked causal attention over the cache
      TIMED(4, launch_attn_prefill(d, e->desc_dev, B, e->step_max_pos, e->q, kv, e->bt_dev, partials, st));
    } else {
      TIMED(4, launch_attention(d, e->desc_dev, B, e->step_chunks, e->q, e->knew, e->vnew, kv, e->bt_dev, partials,
                                st));
    }
    HIP_OK(e, launch_combine(d, e->desc_dev, B, partials, e->o, st, scored ? e->attn_stat : nullptr));
    if (scored)
      HIP_OK(e, launch_score(d, e->desc_dev, B, e->step_max_pos, l, 1, e->q, 0, kv, 0, 0, e->bt_dev, e->attn_stat, 0,
                             e->scores_dev, st));
    if (probe) {
      HIP_OK(e, cp(out + pl.o, e->o, fo));
      HIP_OK(e, cp(e->o, in + pl.o, fo));
      HIP_OK(e, cp(e->x, in + pl.x_in, fx));
    }
    if (fuse_norm) {
      TIMED(3, launch_gemm_resid_norm(d, W.o, e->o, B, ea, gemm_partials, e->cus, W.ffn_norm, e->xn, st));
    } else {
      TIMED(3, proj(W.o, e->o, EPI_RESID, ea));
      if (probe) {
        HIP_OK(e, cp(out + pl.x_mid, e->x, fx));
        HIP_OK(e, cp(e->x, in + pl.x_mid, fx));
      }
      HIP_OK(e, launch_rmsnorm(d, e->x, W.ffn_norm, e->xn, B, st));
    }
    if (probe) {
      HIP_OK(e, cp(out + pl.xn2, e->xn, fxn));
      HIP_OK(e, cp(e->xn, in + pl.xn2, fxn));
    }
    TIMED(0, proj(W.gu, e->xn, EPI_SWIGLU, ea));
    if (probe) {
      HIP_OK(e, cp(out + pl.h, e->h, fh));
      HIP_OK(e, cp(e->h, in + pl.h, fh));
    }
    // the next norm: the next layer's attention norm, or the final norm before the head
    const float* next_g = l + 1 < d.L ? e->layers[(size_t)l + 1].attn_norm : (do_head ? e->final_norm : nullptr);
    if (fuse_norm && next_g) {
      TIMED(1, launch_gemm_resid_norm(d, W.down, e->h, B, ea, gemm_partials, e->cus, next_g, e->xn, st));
      xn_ready = true;
    } else {
      TIMED(1, proj(W.down, e->h, EPI_RESID, ea));
    }
    if (probe) HIP_OK(e, cp(out + pl.x_out, e->x, fx));
    if (e->capture)
      HIP_OK(e, hipMemcpyAsync(e->capture + (size_t)(l + 1) * B * d.D, e->x, (size_t)B * d.D * 4,
                               hipMemcpyDeviceToDevice, st));
  }
  if (probe) HIP_OK(e, cp(e->x, inject + (size_t)(d.L - 1) * pl.record + pl.x_out, fx));
  if (do_head) {
    if (!xn_ready) HIP_OK(e, launch_rmsnorm(d, e->x, e->final_norm, e->xn, B, st));
    TIMED(5, proj(e->head, e->xn, EPI_LOGITS, ea));
    HIP_OK(e, launch_argmax(d, e->desc_dev, B, e->logits, st));
  }
  return DTD_OK;
}

static dtd_status ready(dtd_engine* e) {
  if (!e) return DTD_E_ARG;
  if (e->broken) return fail(e, DTD_E_STATE, "engine unusable after a HIP error");
  if (!e->loaded) return fail(e, DTD_E_STATE, "weights not loaded");
  HIP_OK(e, hipSetDevice(e->device));
  return DTD_OK;
}

static bool sampler_valid(const dtd_sampler& s) {
  return std::isfinite(s.temperature) && s.temperature >= 0.f && s.top_k >= 0 && s.top_p > 0.f && s.top_p <= 1.f &&
         s.min_p >= 0.f && s.min_p <= 1.f;
}

static SampleRow sample_row(const dtd_sampler& s, int64_t counter) {
  return SampleRow{s.temperature, s.top_k, s.top_p, s.min_p, s.seed, counter};
}

// Replaces the greedy tokens of a step's rows whose sequences have a sampler with a
// temperature above 0: rows b < B of `logits` (V floats apart), drawing with counter =
// the position whose logits the row holds.
static dtd_status sample_rows(dtd_engine* e, int B, const int64_t* seq_ids, const int* poss, const float* logits,
                              int32_t* out) {
  if (e->samplers.empty()) return DTD_OK;
  SampleArgs a;
  bool any = false;
  for (int b = 0; b < B; b++) {
    auto it = e->samplers.find(seq_ids[b]);
    const dtd_sampler g{0.f, 0, 1.f, 0.f, 0};
    a.row[b] = sample_row(it == e->samplers.end() ? g : it->second, poss[b]);
    any = any || a.row[b].temperature > 0.f;
  }
  if (!any) return DTD_OK;
  a.logits = logits;
  a.stride = e->d.V;
  a.V = e->d.V;
  a.B = B;
  a.out = out;
  HIP_OK(e, launch_sample(a, e->stream));
  return DTD_OK;
}

static int blocks_needed(const dtd_engine* e, int len) { return (len + e->d.bs - 1) / e->d.bs; }

// ---- KV blocks: a free list plus a holder count per block, so that sequences and prefix-cache
// entries can share blocks (the Qwen3-8B engine article's paged KV block manager, 4.3.1: fixed
// blocks, O(1) allocation and release, free blocks reused)
static int32_t take_block(dtd_engine* e) {
  const int32_t b = e->free_blocks.back();
  e->free_blocks.pop_back();
  e->blk_ref[(size_t)b] = 1;
  return b;
}

static void drop_block(dtd_engine* e, int32_t b) {
  if (--e->blk_ref[(size_t)b] == 0) e->free_blocks.push_back(b);
}

// ---- prefix cache (the Qwen3-8B engine article's automatic prefix cache, 4.4.4): KV of token
// sequences already run, found by a hash of the token prefix, the whole sequence first and then
// ever shorter prefixes; a hit skips prefilling the matched positions.

// FNV-1a over the token ids, one hash per prefix length: h[L] covers tokens [0, L)
static void prefix_hashes(const int32_t* t, int n, std::vector<uint64_t>& h) {
  h.resize((size_t)n + 1);
  uint64_t x = 0xcbf29ce484222325ull;
  h[0] = x;
  for (int i = 0; i < n; i++) {
    const uint32_t v = (uint32_t)t[i];
    for (int k = 0; k < 4; k++) {
      x ^= (v >> (8 * k)) & 0xffu;
      x *= 0x100000001b3ull;
    }
    h[(size_t)i + 1] = x;
  }
}

static void pcache_drop(dtd_engine* e, int64_t id) {
  auto it = e->pcache.find(id);
  if (it == e->pcache.end()) return;
  const PrefixEntry& pe = it->second;
  std::vector<uint64_t> h;
  prefix_hashes(pe.tokens.data(), (int)pe.tokens.size(), h);
  for (size_t L = 1; L < h.size(); L++) {
    auto r = e->pindex.equal_range(h[L]);
    for (auto j = r.first; j != r.second;) {
      if (j->second.first == id) j = e->pindex.erase(j);
      else ++j;
    }
  }
  for (int32_t b : pe.blocks) drop_block(e, b);
  e->pcache.erase(it);
}

// evicts least recently used entries (never `keep`) until `need` blocks are free or no other
// entry is left
static bool make_room(dtd_engine* e, int need, int64_t keep = -1) {
  while ((int)e->free_blocks.size() < need) {
    auto lru = e->pcache.end();
    for (auto it = e->pcache.begin(); it != e->pcache.end(); ++it)
      if (it->first != keep && (lru == e->pcache.end() || it->second.used < lru->second.used)) lru = it;
    if (lru == e->pcache.end()) break;
    pcache_drop(e, lru->first);
  }
  return (int)e->free_blocks.size() >= need;
}

// the longest cached prefix of t[0, n) shorter than n (the last position is always run, for
// its logits); 0 if none.  *entry gets the entry holding it.
static int pcache_lookup(dtd_engine* e, const int32_t* t, int n, int64_t* entry) {
  if (e->pcache.empty() || n < 2) return 0;
  std::vector<uint64_t> h;
  prefix_hashes(t, n, h);
  for (int L = n - 1; L >= 1; L--) {
    auto r = e->pindex.equal_range(h[(size_t)L]);
    for (auto j = r.first; j != r.second; ++j) {
      const PrefixEntry& pe = e->pcache.at(j->second.first);
      if (j->second.second == L && (int)pe.tokens.size() >= L && std::equal(t, t + L, pe.tokens.begin())) {
        *entry = j->second.first;
        return L;
      }
    }
  }
  return 0;
}

// records positions [0, n) of sequence s, holding tokens t, as an entry
static void pcache_insert(dtd_engine* e, const Seq& s, const int32_t* t, int n) {
  if (e->pcache_cap <= 0 || n < 1 || n > s.len) return;
  std::vector<uint64_t> h;
  prefix_hashes(t, n, h);
  auto r = e->pindex.equal_range(h[(size_t)n]);
  for (auto j = r.first; j != r.second; ++j) {
    PrefixEntry& pe = e->pcache.at(j->second.first);
    if (j->second.second == n && (int)pe.tokens.size() == n && std::equal(t, t + n, pe.tokens.begin())) {
      pe.used = ++e->pcache_clock;             // already cached
      return;
    }
  }
  while ((int)e->pcache.size() >= e->pcache_cap) {
    auto lru = e->pcache.begin();
    for (auto it = e->pcache.begin(); it != e->pcache.end(); ++it)
      if (it->second.used < lru->second.used) lru = it;
    pcache_drop(e, lru->first);
  }
  const int64_t id = e->pcache_next++;
  PrefixEntry pe;
  pe.tokens.assign(t, t + n);
  pe.blocks.assign(s.blocks.begin(), s.blocks.begin() + blocks_needed(e, n));
  for (int32_t b : pe.blocks) e->blk_ref[(size_t)b]++;
  pe.used = ++e->pcache_clock;
  e->pcache.emplace(id, std::move(pe));
  for (int L = 1; L <= n; L++) e->pindex.emplace(h[(size_t)L], std::make_pair(id, L));
}

// copies every layer's K and V (and int8 scales) of block src to block dst, on the stream
static dtd_status copy_block(dtd_engine* e, int32_t src, int32_t dst) {
  HIP_OK(e, launch_kv_copy_block(e->d, e->players, src, dst, e->stream));
  return DTD_OK;
}

// ---- KV budget (the Initial-Key cache of the C17 engine article, 5.3) ----------------------

static const KvBudget* budget_of(const dtd_engine* e, int64_t seq_id) {
  auto it = e->budgets.find(seq_id);
  return it == e->budgets.end() ? nullptr : &it->second;
}

// a new sequence under a budget starts with a clear score row
static dtd_status budget_seq_created(dtd_engine* e, int64_t seq_id, Seq& s) {
  if (!budget_of(e, seq_id)) return DTD_OK;
  s.kv_pos.reserve((size_t)e->cfg.max_ctx);
  HIP_OK(e, hipMemsetAsync(e->scores_dev + (size_t)s.slot * e->cfg.max_ctx, 0, (size_t)e->cfg.max_ctx * 4, e->stream));
  return DTD_OK;
}

// Brings the host's entry positions of a budgeted sequence up to date when they live on the
// device: its first `known` entries from the device row (synchronous).
static dtd_status pull_kv_pos(dtd_engine* e, Seq& s, int known) {
  if (!s.pos_on_dev) return DTD_OK;
  s.kv_pos.resize((size_t)known);
  HIP_OK(e, hipStreamSynchronize(e->stream));
  if (known > 0)
    HIP_OK(e, hipMemcpy(s.kv_pos.data(), e->kvpos_dev + (size_t)s.slot * e->cfg.max_ctx, (size_t)known * 4,
                        hipMemcpyDeviceToHost));
  s.pos_on_dev = false;
  return DTD_OK;
}

// Brings a sequence back to its budget when it holds more entries: the entries of its first
// n_initial positions, its last n_recent entries, and the highest attention-score sums of the
// others (the earlier entry on equal sums) stay, in order, copied into fresh blocks; the rest
// are dropped with their scores.  new_pos: the token position of the entry the last step
// appended (entry n - 1).
//  - One entry over the budget (a decode step): decided and carried out on the device, with
//    no host round trip; the positions then live in the device's row.
//  - Otherwise (a prefill): synchronous, the host reads the scores.
static dtd_status kv_evict(dtd_engine* e, Seq& s, const KvBudget& kb, int new_pos) {
  const int n = s.len;
  const int mc = e->cfg.max_ctx;
  if (n == kb.budget + 1 && n > kb.n_initial + kb.n_recent) {
    // entries [0, n_initial) hold positions 0 .. n_initial - 1 (never evicted)
    if (!s.pos_on_dev) {
      HIP_OK(e, hipMemcpy(e->kvpos_dev + (size_t)s.slot * mc, s.kv_pos.data(), (size_t)(n - 1) * 4,
                          hipMemcpyHostToDevice));
      s.pos_on_dev = true;
    }
    const int m = n - 1, nb = blocks_needed(e, m);
    if (!make_room(e, nb))
      return fail(e, DTD_E_KVFULL, "KV budget: %d blocks for the kept entries, %zu free", nb, e->free_blocks.size());
    const int ring = e->evict_ring;
    int32_t* hs = e->evict_host + (size_t)ring * 2 * e->d.max_blocks;
    if (e->evict_ev_used[ring]) HIP_OK(e, hipEventSynchronize(e->evict_ev[ring]));
    std::copy(s.blocks.begin(), s.blocks.end(), hs);
    std::vector<int32_t> fresh;
    for (int i = 0; i < nb; i++) fresh.push_back(take_block(e));
    std::copy(fresh.begin(), fresh.end(), hs + e->d.max_blocks);
    // one copy of both lists (old blocks at 0, new ones at max_blocks, the kept entries after
    // them); the eviction kernel also writes the new blocks into the block table
    hipStream_t st = e->stream;
    const size_t mb = (size_t)e->d.max_blocks;
    HIP_OK(e, hipMemcpyAsync(e->evict_dev, hs, (mb + (size_t)nb) * 4, hipMemcpyHostToDevice, st));
    HIP_OK(e, launch_evict_one(e->scores_dev + (size_t)s.slot * mc, e->kvpos_dev + (size_t)s.slot * mc, n,
                               kb.n_initial, n - kb.n_recent, new_pos, e->evict_dev + 2 * mb, e->evict_dev + mb, nb,
                               e->bt_dev + (size_t)s.slot * mb, st));
    HIP_OK(e, launch_kv_gather(e->d, e->players, e->evict_dev, e->evict_dev + mb, e->evict_dev + 2 * mb, m, st));
    HIP_OK(e, hipEventRecord(e->evict_ev[ring], st));
    e->evict_ev_used[ring] = true;
    e->evict_ring = (ring + 1) % kEvictRing;
    for (int32_t b : s.blocks) drop_block(e, b);   // reused only by work queued after the gather
    s.blocks.assign(fresh.begin(), fresh.end());
    s.len = m;
    s.tokens_known = false;
    return DTD_OK;
  }
  if (s.pos_on_dev) {
    dtd_status ps = pull_kv_pos(e, s, n - 1);
    if (ps) return ps;
    s.kv_pos.push_back(new_pos);
  }
  if (n <= kb.budget) return DTD_OK;
  std::vector<float> sc((size_t)n);
  HIP_OK(e, hipStreamSynchronize(e->stream));
  HIP_OK(e, hipMemcpy(sc.data(), e->scores_dev + (size_t)s.slot * mc, (size_t)n * 4, hipMemcpyDeviceToHost));
  int n_init = 0;
  while (n_init < n && s.kv_pos[(size_t)n_init] < kb.n_initial) n_init++;
  const int rec0 = std::max(n_init, n - kb.n_recent);
  std::vector<int32_t> middle;
  for (int i = n_init; i < rec0; i++) middle.push_back(i);
  std::stable_sort(middle.begin(), middle.end(), [&](int a, int b) { return sc[(size_t)a] > sc[(size_t)b]; });
  const int take = std::max(0, kb.budget - n_init - (n - rec0));
  if ((int)middle.size() > take) middle.resize((size_t)take);
  std::vector<int32_t> keep;
  for (int i = 0; i < n_init; i++) keep.push_back(i);
  keep.insert(keep.end(), middle.begin(), middle.end());
  for (int i = rec0; i < n; i++) keep.push_back(i);
  std::sort(keep.begin(), keep.end());
  const int m = (int)keep.size();
  const int nb = blocks_needed(e, m);
  if (!make_room(e, nb))
    return fail(e, DTD_E_KVFULL, "KV budget: %d blocks for the kept entries, %zu free", nb, e->free_blocks.size());
  std::vector<int32_t> fresh;
  for (int i = 0; i < nb; i++) fresh.push_back(take_block(e));
  HIP_OK(e, hipMemcpy(e->evict_dev, s.blocks.data(), s.blocks.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(e, hipMemcpy(e->evict_dev + mc, fresh.data(), fresh.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(e, hipMemcpy(e->evict_dev + 2 * (size_t)mc, keep.data(), keep.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(e, launch_kv_gather(e->d, e->players, e->evict_dev, e->evict_dev + mc, e->evict_dev + 2 * (size_t)mc, m,
                             e->stream));
  std::vector<float> nsc((size_t)mc, 0.f);
  std::vector<int32_t> npos((size_t)m);
  for (int i = 0; i < m; i++) {
    nsc[(size_t)i] = sc[(size_t)keep[(size_t)i]];
    npos[(size_t)i] = s.kv_pos[(size_t)keep[(size_t)i]];
  }
  HIP_OK(e, hipStreamSynchronize(e->stream));
  HIP_OK(e, hipMemcpy(e->scores_dev + (size_t)s.slot * mc, nsc.data(), (size_t)mc * 4, hipMemcpyHostToDevice));
  for (int32_t b : s.blocks) drop_block(e, b);
  s.blocks.assign(fresh.begin(), fresh.end());
  HIP_OK(e, hipMemcpy(e->bt_dev + (size_t)s.slot * e->d.max_blocks, s.blocks.data(), s.blocks.size() * 4,
                      hipMemcpyHostToDevice));
  s.kv_pos.assign(npos.begin(), npos.end());
  s.len = m;
  s.tokens_known = false;
  return DTD_OK;
}

static dtd_status prefill_run(dtd_engine* e, int64_t seq_id, Seq& s, const int32_t* tokens_dev, int n,
                              int32_t* next_token_dev, float* logits_dev);

extern "C" dtd_status dtd_prefill(dtd_engine* e, int64_t seq_id, const int32_t* tokens_dev, int32_t n,
                                  int32_t* next_token_dev, float* logits_dev) {
  dtd_status st = ready(e);
  if (st) return st;
  if (!tokens_dev || !next_token_dev || n <= 0) return fail(e, DTD_E_ARG, "prefill: null pointer or n <= 0");
  auto it = e->seqs.find(seq_id);
  const bool is_new = it == e->seqs.end();
  const int len0 = is_new ? 0 : it->second.len;
  if ((int64_t)len0 + n > e->cfg.max_ctx)
    return fail(e, DTD_E_CTX, "prefill: %d + %d positions exceed max_ctx %d", len0, n, e->cfg.max_ctx);
  if (is_new && e->free_slots.empty()) return fail(e, DTD_E_KVFULL, "prefill: no free sequence slot");
  // with the prefix cache on, the host reads the tokens: to look up a new sequence's longest
  // cached prefix, and to record the prompt afterwards
  const bool pc = e->pcache_cap > 0;
  std::vector<int32_t> host;
  if (pc) {
    host.resize((size_t)n);
    HIP_OK(e, hipStreamSynchronize(e->stream));
    HIP_OK(e, hipMemcpy(host.data(), tokens_dev, (size_t)n * 4, hipMemcpyDeviceToHost));
  }
  int64_t hit = -1;
  const KvBudget* kb = budget_of(e, seq_id);
  const int reuse = (pc && is_new && !kb) ? pcache_lookup(e, host.data(), n, &hit) : 0;
  const int shared = reuse / e->d.bs;       // whole blocks taken over from the entry
  const int have = is_new ? 0 : (int)it->second.blocks.size();
  const int need = blocks_needed(e, len0 + n) - have - shared;
  if (!make_room(e, need, hit))
    return fail(e, DTD_E_KVFULL, "prefill: needs %d KV blocks, %zu free", need, e->free_blocks.size());
  if (is_new) {
    Seq s;
    s.blocks.reserve((size_t)e->d.max_blocks);
    s.slot = e->free_slots.back();
    e->free_slots.pop_back();
    it = e->seqs.emplace(seq_id, s).first;
    if ((st = budget_seq_created(e, seq_id, it->second))) return st;
  }
  Seq& s = it->second;
  if (!pc) s.tokens_known = false;
  s.reused = reuse;
  if (reuse > 0) {
    // positions [0, reuse) from the entry: its whole blocks shared, a partial last one copied
    PrefixEntry& pe = e->pcache.at(hit);
    pe.used = ++e->pcache_clock;
    for (int j = 0; j < shared; j++) {
      s.blocks.push_back(pe.blocks[(size_t)j]);
      e->blk_ref[(size_t)pe.blocks[(size_t)j]]++;
    }
    if (reuse % e->d.bs) {
      const int32_t nb = take_block(e);
      if ((st = copy_block(e, pe.blocks[(size_t)shared], nb))) return st;
      s.blocks.push_back(nb);
    }
    HIP_OK(e, hipStreamSynchronize(e->stream));
    HIP_OK(e, hipMemcpy(e->bt_dev + (size_t)s.slot * e->d.max_blocks, s.blocks.data(), s.blocks.size() * 4,
                        hipMemcpyHostToDevice));
    s.len = reuse;
    s.rpos = reuse;
    s.tokens.assign(host.begin(), host.begin() + reuse);
    tokens_dev += reuse;
    n -= reuse;
  }
  if (pc && s.tokens_known) s.tokens.insert(s.tokens.end(), host.begin() + reuse, host.end());
  st = prefill_run(e, seq_id, s, tokens_dev, n, next_token_dev, logits_dev);
  if (st) return st;
  if (kb) return kv_evict(e, s, *kb, s.rpos - 1);
  if (pc && s.tokens_known && (int)s.tokens.size() == s.len) pcache_insert(e, s, s.tokens.data(), s.len);
  return DTD_OK;
}

// Runs n tokens of an existing sequence (its blocks for the positions before are in place).
static dtd_status prefill_run(dtd_engine* e, int64_t seq_id, Seq& s, const int32_t* tokens_dev, int n,
                              int32_t* next_token_dev, float* logits_dev) {
  dtd_status st = DTD_OK;
  // under a KV budget (or after one evicted entries) the steps carry RoPE positions, and the
  // last prompt position's attention adds to the scores
  const KvBudget* kb = budget_of(e, seq_id);
  const bool extra_on = kb || s.rpos != s.len;
  const int sfrom = kb ? e->d.L - kb->score_layers : e->d.L;
  if (kb && (st = pull_kv_pos(e, s, s.len))) return st;   // positions are appended on the host below
  // Batched prefill: the prompt in chunks of up to kPrefillChunk positions, each chunk one
  // step of the per-sub-step schedule with the chunk's positions as its batch (projections on
  // the matrix cores where the formats allow); every position's K/V is appended before the
  // chunk's attention, so that each position attends to the ones before it.  With the
  // persistent-only schedule selected, or hidden-state capture on (its buffer holds one
  // step's batch), positions go one per step.
  if (n >= 2 && e->path != 2 && !e->capture) {
    for (int c0 = 0; c0 < n; c0 += kPrefillChunk) {
      const int B = std::min(kPrefillChunk, n - c0);
      const bool last = c0 + B == n;
      int slots[kPrefillChunk], poss[kPrefillChunk], pblks[kPrefillChunk];
      Update upd[kPrefillChunk];
      int n_upd = 0;
      for (int b = 0; b < B; b++) {
        const int pos = s.len + b;
        if (pos / e->d.bs >= (int)s.blocks.size()) {
          const int32_t blk = take_block(e);
          s.blocks.push_back(blk);
          upd[n_upd++] = {s.slot, (int)s.blocks.size() - 1, blk};
        }
        slots[b] = s.slot;
        poss[b] = pos;
        pblks[b] = s.blocks[(size_t)(pos / e->d.bs)];
      }
      int rps[kPrefillChunk], sfs[kPrefillChunk];
      for (int b = 0; b < B; b++) {
        rps[b] = s.rpos + b;
        sfs[b] = (last && b == B - 1) ? sfrom : e->d.L;
      }
      const StepExtra ex{rps, sfs};
      st = run_step(e, B, slots, poss, pblks, tokens_dev + c0, e->tok_scratch, nullptr, last, upd, n_upd,
                    nullptr, nullptr, nullptr, nullptr, true, false, true, extra_on ? &ex : nullptr);
      if (st) return st;
      if (kb)
        for (int b = 0; b < B; b++) s.kv_pos.push_back(s.rpos + b);
      s.len += B;
      s.rpos += B;
      if (last) {
        HIP_OK(e, hipMemcpyAsync(next_token_dev, e->tok_scratch + (B - 1), 4, hipMemcpyDeviceToDevice, e->stream));
        if (logits_dev)
          HIP_OK(e, hipMemcpyAsync(logits_dev, e->logits + (size_t)(B - 1) * e->d.V, (size_t)e->d.V * 4,
                                   hipMemcpyDeviceToDevice, e->stream));
        const int lastpos = s.rpos - 1;
        return sample_rows(e, 1, &seq_id, &lastpos, e->logits + (size_t)(B - 1) * e->d.V, next_token_dev);
      }
    }
    return DTD_OK;
  }
  for (int i = 0; i < n; i++) {
    const int pos = s.len;
    Update upd[1];
    int n_upd = 0;
    if (pos / e->d.bs >= (int)s.blocks.size()) {
      const int32_t b = take_block(e);
      s.blocks.push_back(b);
      upd[n_upd++] = {s.slot, (int)s.blocks.size() - 1, b};
    }
    const bool last = i == n - 1;
    const int pblk = s.blocks[(size_t)(pos / e->d.bs)];
    const int rp = s.rpos, sf = last ? sfrom : e->d.L;
    const StepExtra ex{&rp, &sf};
    st = run_step(e, 1, &s.slot, &pos, &pblk, tokens_dev + i, next_token_dev, last ? logits_dev : nullptr, last,
                  upd, n_upd, nullptr, nullptr, nullptr, nullptr, false, false, false, extra_on ? &ex : nullptr);
    if (st) return st;
    if (kb) s.kv_pos.push_back(s.rpos);
    s.len++;
    s.rpos++;
  }
  const int lastpos = s.rpos - 1;
  return sample_rows(e, 1, &seq_id, &lastpos, e->logits, next_token_dev);
}

// Sequence lookups, block allocation and the step launch of a decode call.  Uses fixed-size
// arrays only (no heap allocation): a sequence's block list has its full capacity reserved
// when the sequence is created.
static dtd_status decode_impl(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                              const int32_t* tokens_dev, int32_t* next_tokens_dev, float* logits_dev,
                              const uint8_t* inject, uint8_t* capture, bool create_missing,
                              float* partials = nullptr, float* gemm_partials = nullptr, bool no_alloc = false) {
  dtd_status st = ready(e);
  if (st) return st;
  if (batch <= 0 || batch > e->cfg.max_batch)
    return fail(e, DTD_E_ARG, "decode_step: batch %d outside [1, %d]", batch, e->cfg.max_batch);
  if (!seq_ids_host || !tokens_dev || !next_tokens_dev) return fail(e, DTD_E_ARG, "decode_step: null pointer");
  int need = 0;
  Seq* ss[kMaxBatch];
  int missing = 0;
  for (int b = 0; b < batch; b++) {
    for (int c = 0; c < b; c++)
      if (seq_ids_host[c] == seq_ids_host[b])
        return fail(e, DTD_E_ARG, "decode_step: seq_id %lld repeated in the batch", (long long)seq_ids_host[b]);
    if (create_missing && e->seqs.find(seq_ids_host[b]) == e->seqs.end()) missing++;
  }
  if (missing > (int)e->free_slots.size()) return fail(e, DTD_E_KVFULL, "decode_step: no free sequence slot");
  if (!make_room(e, missing)) return fail(e, DTD_E_KVFULL, "decode_step: no free KV block");
  for (int b = 0; b < batch; b++) {
    auto it = e->seqs.find(seq_ids_host[b]);
    if (it == e->seqs.end() && !create_missing)
      return fail(e, DTD_E_NOSEQ, "decode_step: unknown seq_id %lld", (long long)seq_ids_host[b]);
    if (it != e->seqs.end()) {
      const Seq& s = it->second;
      if (s.len + 1 > e->cfg.max_ctx || s.rpos + 1 > e->cfg.max_ctx)
        return fail(e, DTD_E_CTX, "decode_step: seq_id %lld is at max_ctx %d", (long long)seq_ids_host[b], e->cfg.max_ctx);
      if (s.len / e->d.bs >= (int)s.blocks.size()) need++;
    } else {
      need++;
    }
  }
  if (!make_room(e, need))
    return fail(e, DTD_E_KVFULL, "decode_step: needs %d KV blocks, %zu free", need, e->free_blocks.size());
  // validated: only now change engine state
  for (int b = 0; b < batch && missing; b++)
    if (e->seqs.find(seq_ids_host[b]) == e->seqs.end()) {
      Seq s;
      s.slot = e->free_slots.back();
      s.blocks.reserve((size_t)e->d.max_blocks);
      e->free_slots.pop_back();
      auto nit = e->seqs.emplace(seq_ids_host[b], std::move(s)).first;
      if ((st = budget_seq_created(e, seq_ids_host[b], nit->second))) return st;
    }
  for (int b = 0; b < batch; b++) ss[b] = &e->seqs.find(seq_ids_host[b])->second;
  int slots[kMaxBatch], poss[kMaxBatch], pblks[kMaxBatch];
  Update upd[kMaxBatch];
  int n_upd = 0;
  for (int b = 0; b < batch; b++) {
    Seq& s = *ss[b];
    if (s.len / e->d.bs >= (int)s.blocks.size()) {
      const int32_t blk = take_block(e);
      s.blocks.push_back(blk);
      upd[n_upd++] = {s.slot, (int)s.blocks.size() - 1, blk};
    }
    slots[b] = s.slot;
    poss[b] = s.len;
    pblks[b] = s.blocks[(size_t)(s.len / e->d.bs)];
  }
  // KV budgets (and sequences whose entries were evicted): RoPE positions and score sums
  int rps[kMaxBatch], sfs[kMaxBatch];
  bool extra_on = false;
  const KvBudget* kbs[kMaxBatch];
  for (int b = 0; b < batch; b++) {
    kbs[b] = budget_of(e, seq_ids_host[b]);
    rps[b] = ss[b]->rpos;
    sfs[b] = kbs[b] ? e->d.L - kbs[b]->score_layers : e->d.L;
    extra_on = extra_on || kbs[b] || ss[b]->rpos != ss[b]->len;
  }
  const StepExtra ex{rps, sfs};
  st = run_step(e, batch, slots, poss, pblks, tokens_dev, next_tokens_dev, logits_dev, true, upd, n_upd,
                inject, capture, partials, gemm_partials, no_alloc, no_alloc, false, extra_on ? &ex : nullptr);
  if (st) return st;
  st = sample_rows(e, batch, seq_ids_host, rps, e->logits, next_tokens_dev);
  if (st) return st;
  for (int b = 0; b < batch; b++) {
    if (kbs[b] && !ss[b]->pos_on_dev) ss[b]->kv_pos.push_back(ss[b]->rpos);
    ss[b]->len++;
    ss[b]->rpos++;
    ss[b]->tokens_known = false;   // the token ids of a decode step stay on the device
  }
  for (int b = 0; b < batch; b++)
    if (kbs[b] && (st = kv_evict(e, *ss[b], *kbs[b], ss[b]->rpos - 1))) return st;
  return DTD_OK;
}

extern "C" dtd_status dtd_decode_step(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                                      const int32_t* tokens_dev, int32_t* next_tokens_dev,
                                      float* logits_dev) {
  return decode_impl(e, batch, seq_ids_host, tokens_dev, next_tokens_dev, logits_dev, nullptr, nullptr, false);
}

extern "C" dtd_status dtd_decode_step_noalloc(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                                              const int32_t* tokens_dev, int32_t* next_tokens_dev,
                                              float* logits_dev) {
  if (!e) return DTD_E_ARG;
  if (batch <= 0 || batch > e->cfg.max_batch)
    return fail(e, DTD_E_ARG, "decode_step_noalloc: batch %d outside [1, %d]", batch, e->cfg.max_batch);
  // The static scratch holds the split-K attention partials [batch][Hq][nch][hd + 2] fp32,
  // then (batched matrix-core projections) the split-K sums of the projections.
  const Dims& d = e->d;
  const size_t attn = ((size_t)batch * d.Hq * d.nch * (d.hd + 2) * sizeof(float) + 255) / 256 * 256;
  const size_t gemm = gemm_eligible(d, batch) ? gemm_partial_bytes(d, batch, e->cus) : 0;
  if (attn + gemm > kNoAllocScratchBytes)
    return fail(e, DTD_E_UNSUPPORTED,
                "decode_step_noalloc: %zu bytes of attention partials and %zu of projection partial sums for "
                "batch %d exceed the %zu-byte static scratch (fewer sequences per call, or a shorter max_ctx, fit)",
                attn, gemm, batch, kNoAllocScratchBytes);
  for (int b = 0; b < batch && seq_ids_host; b++) {
    auto it = e->seqs.find(seq_ids_host[b]);
    if (budget_of(e, seq_ids_host[b]) || (it != e->seqs.end() && it->second.rpos != it->second.len))
      return fail(e, DTD_E_UNSUPPORTED, "decode_step_noalloc: seq_id %lld is under a KV budget",
                  (long long)seq_ids_host[b]);
  }
  float* base = (float*)e->scratch_dev;
  return decode_impl(e, batch, seq_ids_host, tokens_dev, next_tokens_dev, logits_dev, nullptr, nullptr, false,
                     base, (float*)((uint8_t*)base + attn), true);
}

extern "C" dtd_status dtd_debug_decode_probe(dtd_engine* e, int32_t batch, const int64_t* seq_ids_host,
                                             const int32_t* tokens_dev, const void* inject_dev,
                                             void* capture_dev, int32_t* next_tokens_dev,
                                             float* logits_dev) {
  if (e && (!inject_dev || !capture_dev)) return fail(e, DTD_E_ARG, "decode_probe: null buffer");
  return decode_impl(e, batch, seq_ids_host, tokens_dev, next_tokens_dev, logits_dev,
                     (const uint8_t*)inject_dev, (uint8_t*)capture_dev, true);
}

extern "C" int64_t dtd_debug_probe_record_bytes(const dtd_config* cfg, int32_t batch) {
  const dtd_status st = check_config(cfg, nullptr, 0);
  if (st != DTD_OK) return st;
  if (batch <= 0) return DTD_E_ARG;
  const Dims d = make_dims(cfg);
  return (int64_t)probe_layout(d, batch, act_bytes(cfg->act)).record;
}

extern "C" dtd_status dtd_reset_seq(dtd_engine* e, int64_t seq_id) {
  if (!e) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  if (it == e->seqs.end()) return fail(e, DTD_E_NOSEQ, "reset_seq: unknown seq_id %lld", (long long)seq_id);
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) drop_block(e, *b);
  e->free_slots.push_back(it->second.slot);
  e->seqs.erase(it);
  e->samplers.erase(seq_id);
  e->budgets.erase(seq_id);
  return DTD_OK;
}

extern "C" dtd_status dtd_set_sampler(dtd_engine* e, int64_t seq_id, const dtd_sampler* s) {
  if (!e) return DTD_E_ARG;
  if (!s || s->temperature == 0.f) {
    if (s && !sampler_valid(*s)) return fail(e, DTD_E_ARG, "set_sampler: invalid settings");
    e->samplers.erase(seq_id);
    return DTD_OK;
  }
  if (e->d.V > kMaxSampleVocab)
    return fail(e, DTD_E_UNSUPPORTED, "set_sampler: vocabulary %d above %d", e->d.V, kMaxSampleVocab);
  if (!sampler_valid(*s))
    return fail(e, DTD_E_ARG, "set_sampler: temperature %g, top_k %d, top_p %g, min_p %g outside their ranges",
                (double)s->temperature, s->top_k, (double)s->top_p, (double)s->min_p);
  e->samplers[seq_id] = *s;
  return DTD_OK;
}

extern "C" dtd_status dtd_set_prefix_cache(dtd_engine* e, int32_t max_entries) {
  if (!e) return DTD_E_ARG;
  if (max_entries < 0) return fail(e, DTD_E_ARG, "set_prefix_cache: max_entries %d < 0", max_entries);
  e->pcache_cap = max_entries;
  while ((int)e->pcache.size() > max_entries) {
    auto lru = e->pcache.begin();
    for (auto it = e->pcache.begin(); it != e->pcache.end(); ++it)
      if (it->second.used < lru->second.used) lru = it;
    pcache_drop(e, lru->first);
  }
  return DTD_OK;
}

extern "C" dtd_status dtd_prefix_cache_add(dtd_engine* e, int64_t seq_id, const int32_t* tokens_host, int32_t n) {
  if (!e) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  if (it == e->seqs.end()) return fail(e, DTD_E_NOSEQ, "prefix_cache_add: unknown seq_id %lld", (long long)seq_id);
  if (!tokens_host || n < 1 || n > it->second.len)
    return fail(e, DTD_E_ARG, "prefix_cache_add: n %d outside [1, %d] or null tokens", n, it->second.len);
  if (e->pcache_cap <= 0) return fail(e, DTD_E_STATE, "prefix_cache_add: the prefix cache is off");
  pcache_insert(e, it->second, tokens_host, n);
  return DTD_OK;
}

extern "C" dtd_status dtd_set_kv_budget(dtd_engine* e, int64_t seq_id, int32_t budget, int32_t n_initial,
                                        int32_t n_recent, int32_t score_layers) {
  if (!e) return DTD_E_ARG;
  if (budget == 0) {
    e->budgets.erase(seq_id);
    return DTD_OK;
  }
  if (budget < 0 || n_initial < 0 || n_recent < 1 || budget < n_initial + n_recent + 1 || budget > e->cfg.max_ctx ||
      score_layers < 1 || score_layers > e->d.L)
    return fail(e, DTD_E_ARG, "set_kv_budget: budget %d, n_initial %d, n_recent %d, score_layers %d out of range",
                budget, n_initial, n_recent, score_layers);
  auto it = e->seqs.find(seq_id);
  const bool had = budget_of(e, seq_id) != nullptr;
  e->budgets[seq_id] = KvBudget{budget, n_initial, n_recent, score_layers};
  if (it != e->seqs.end() && !had) {
    Seq& s = it->second;
    if (s.rpos != s.len) return fail(e, DTD_E_STATE, "set_kv_budget: the sequence has evicted entries");
    dtd_status st = budget_seq_created(e, seq_id, s);
    if (st) return st;
    s.kv_pos.clear();
    for (int p = 0; p < s.len; p++) s.kv_pos.push_back(p);
  }
  return DTD_OK;
}

extern "C" int32_t dtd_debug_kv_positions(const dtd_engine* e, int64_t seq_id, int32_t* out_host, int32_t cap) {
  if (!e || (cap > 0 && !out_host)) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  if (it == e->seqs.end()) return DTD_E_NOSEQ;
  const Seq& s = it->second;
  const int n = std::min(s.len, cap);
  if (s.pos_on_dev) {   // after evictions decided on the device
    if (n > 0 && (hipStreamSynchronize(e->stream) != hipSuccess ||
                  hipMemcpy(out_host, e->kvpos_dev + (size_t)s.slot * e->cfg.max_ctx, (size_t)n * 4,
                            hipMemcpyDeviceToHost) != hipSuccess))
      return DTD_E_HIP;
    return s.len;
  }
  for (int i = 0; i < n; i++)
    out_host[i] = budget_of(e, seq_id) ? s.kv_pos[(size_t)i] : (s.rpos == s.len ? i : -1);
  return s.len;
}

extern "C" int32_t dtd_debug_kv_scores(dtd_engine* e, int64_t seq_id, float* out_host, int32_t cap) {
  if (!e || (cap > 0 && !out_host)) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  if (it == e->seqs.end()) return DTD_E_NOSEQ;
  const int n = std::min(it->second.len, cap);
  if (n > 0) {
    HIP_OK(e, hipStreamSynchronize(e->stream));
    HIP_OK(e, hipMemcpy(out_host, e->scores_dev + (size_t)it->second.slot * e->cfg.max_ctx, (size_t)n * 4,
                        hipMemcpyDeviceToHost));
  }
  return it->second.len;
}

extern "C" dtd_status dtd_get_config(const dtd_engine* e, dtd_config* out) {
  if (!e || !out) return DTD_E_ARG;
  *out = e->cfg;
  return DTD_OK;
}

extern "C" void* dtd_get_stream(const dtd_engine* e) { return e ? (void*)e->stream : nullptr; }

extern "C" int32_t dtd_debug_prefix_reused(const dtd_engine* e, int64_t seq_id) {
  if (!e) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  return it == e->seqs.end() ? DTD_E_NOSEQ : it->second.reused;
}

extern "C" int32_t dtd_debug_kv_blocks_free(const dtd_engine* e) {
  if (!e) return DTD_E_ARG;
  return (int32_t)e->free_blocks.size();
}

extern "C" int32_t dtd_debug_prefix_entries(const dtd_engine* e) {
  if (!e) return DTD_E_ARG;
  return (int32_t)e->pcache.size();
}

extern "C" dtd_status dtd_sample(const float* logits_dev, int64_t row_stride, int32_t batch, int32_t vocab,
                                 const dtd_sampler* samplers_host, const int64_t* counters_host, int32_t* tokens_dev,
                                 void* hip_stream) {
  if (!logits_dev || !samplers_host || !counters_host || !tokens_dev || batch < 1 || batch > kMaxBatch ||
      vocab < 1 || vocab > kMaxSampleVocab || row_stride < vocab) {
    g_create_err = "sample: null pointer, batch outside [1, 64], vocab outside [1, 2^19] or row_stride < vocab";
    return DTD_E_ARG;
  }
  SampleArgs a;
  for (int b = 0; b < batch; b++) {
    if (!sampler_valid(samplers_host[b])) {
      g_create_err = "sample: sampler settings outside their ranges";
      return DTD_E_ARG;
    }
    a.row[b] = sample_row(samplers_host[b], counters_host[b]);
  }
  a.logits = logits_dev;
  a.stride = row_stride;
  a.V = vocab;
  a.B = batch;
  a.out = tokens_dev;
  const hipError_t r = launch_sample(a, (hipStream_t)hip_stream);
  if (r != hipSuccess) {
    g_create_err = std::string("sample: ") + hipGetErrorString(r);
    return DTD_E_HIP;
  }
  return DTD_OK;
}

extern "C" int32_t dtd_seq_len(const dtd_engine* e, int64_t seq_id) {
  if (!e) return DTD_E_ARG;
  auto it = e->seqs.find(seq_id);
  return it == e->seqs.end() ? DTD_E_NOSEQ : it->second.len;
}

extern "C" dtd_status dtd_check_device_errors(dtd_engine* e) {
  if (!e) return DTD_E_ARG;
  if (e->broken) return fail(e, DTD_E_STATE, "engine unusable after a HIP error");
  HIP_OK(e, hipSetDevice(e->device));
  HIP_OK(e, hipStreamSynchronize(e->stream));
  // the device's error bits stay set until cleared here; read them now (not after every step)
  HIP_OK(e, hipMemcpy(e->err_host, e->err_dev, 4, hipMemcpyDeviceToHost));
  const int32_t flags = *e->err_host;
  if (flags & kErrBarrier) {
    e->broken = true;
    return fail(e, DTD_E_HIP, "persistent step kernel: a wait for another workgroup timed out; engine unusable");
  }
  if (flags) {
    *e->err_host = 0;
    HIP_OK(e, hipMemsetAsync(e->err_dev, 0, 4, e->stream));
    HIP_OK(e, hipStreamSynchronize(e->stream));
    return fail(e, DTD_E_ARG, "a token id outside [0, %d) was read on the device (used as id 0)", e->d.V);
  }
  return DTD_OK;
}

// ---------------------------------------------------------------------------------------
// debug / measurement
// ---------------------------------------------------------------------------------------

extern "C" dtd_status dtd_debug_dequant_rows(dtd_engine* e, const char* matrix, int32_t r0, int32_t nrows,
                                             float* out_dev) {
  dtd_status st = ready(e);
  if (st) return st;
  if (!matrix || !out_dev || nrows <= 0 || r0 < 0) return fail(e, DTD_E_ARG, "dequant_rows: bad arguments");
  const Dims& d = e->d;
  const std::string name = matrix;
  const MatDev* m = nullptr;
  int rows = 0;
  std::vector<int32_t> map;
  int li = -1;
  char field[32] = {0};
  if (name == "tok_emb" || (name == "lm_head" && !e->cfg.tied_embeddings)) {
    m = name == "tok_emb" ? &e->emb : &e->head;
    rows = d.V;
    for (int r = r0; r < r0 + nrows && r < rows; r++) map.push_back(r);
  } else if (sscanf(name.c_str(), "L%d.%31s", &li, field) == 2 && li >= 0 && li < d.L) {
    const LayerW& W = e->layers[(size_t)li];
    const std::string f = field;
    if (f == "wq" || f == "wk" || f == "wv") {
      const int part = f == "wq" ? 0 : (f == "wk" ? 1 : 2);
      rows = part == 0 ? d.q_dim : d.kv_dim;
      m = &W.qkv;
      for (int r = r0; r < r0 + nrows && r < rows; r++) map.push_back(qkv_stored_row(d, part, r));
    } else if (f == "w_gate" || f == "w_up") {
      rows = d.F;
      m = &W.gu;
      for (int r = r0; r < r0 + nrows && r < rows; r++) map.push_back(2 * r + (f == "w_up"));
    } else if (f == "wo" || f == "w_down") {
      rows = d.D;
      m = f == "wo" ? &W.o : &W.down;
      for (int r = r0; r < r0 + nrows && r < rows; r++) map.push_back(r);
    }
  }
  if (!m) return fail(e, DTD_E_ARG, "dequant_rows: unknown matrix '%s'", matrix);
  if ((int)map.size() != nrows) return fail(e, DTD_E_ARG, "dequant_rows: rows [%d, %d) outside [0, %d)", r0, r0 + nrows, rows);
  if (e->rows_cap < nrows) {
    if (e->rows_dev) HIP_OK(e, hipFree(e->rows_dev));
    e->rows_dev = nullptr;
    e->rows_cap = 0;
    if ((st = dev_alloc(e, &e->rows_dev, (size_t)nrows * 4))) return st;
    e->rows_cap = nrows;
  }
  HIP_OK(e, hipStreamSynchronize(e->stream));
  HIP_OK(e, hipMemcpy(e->rows_dev, map.data(), (size_t)nrows * 4, hipMemcpyHostToDevice));
  HIP_OK(e, launch_dequant_rows(d, *m, e->rows_dev, nrows, out_dev, e->stream));
  HIP_OK(e, hipStreamSynchronize(e->stream));
  return DTD_OK;
}

extern "C" dtd_status dtd_debug_capture_hidden(dtd_engine* e, int32_t enable, float* out_dev) {
  if (!e) return DTD_E_ARG;
  if (enable && !out_dev) return fail(e, DTD_E_ARG, "capture_hidden: null buffer");
  e->capture = enable ? out_dev : nullptr;
  return DTD_OK;
}

// a debug write that extends a sequence to `len` positions: they are its token positions too
// (unless entries were evicted before)
static void grow_debug_len(dtd_engine* e, int64_t seq_id, Seq& s, int len) {
  if (s.rpos == s.len) {
    if (budget_of(e, seq_id))
      for (int p = s.len; p < len; p++) s.kv_pos.push_back(p);
    s.rpos = len;
  }
  s.len = len;
}

// make sure a sequence exists with blocks for [0, len); new block-table entries are written
// synchronously (the debug entry points are synchronous)
static dtd_status ensure_seq_blocks(dtd_engine* e, int64_t seq_id, int len, Seq** out) {
  auto it = e->seqs.find(seq_id);
  if (it == e->seqs.end()) {
    if (e->free_slots.empty()) return fail(e, DTD_E_KVFULL, "no free sequence slot");
    Seq s;
    s.blocks.reserve((size_t)e->d.max_blocks);
    s.slot = e->free_slots.back();
    e->free_slots.pop_back();
    it = e->seqs.emplace(seq_id, s).first;
    dtd_status st = budget_seq_created(e, seq_id, it->second);
    if (st) return st;
  }
  Seq& s = it->second;
  const int need = blocks_needed(e, len) - (int)s.blocks.size();
  if (!make_room(e, need)) return fail(e, DTD_E_KVFULL, "needs %d KV blocks, %zu free", need, e->free_blocks.size());
  s.tokens_known = false;
  if (need > 0) {
    for (int i = 0; i < need; i++) s.blocks.push_back(take_block(e));
    HIP_OK(e, hipStreamSynchronize(e->stream));
    HIP_OK(e, hipMemcpy(e->bt_dev + (size_t)s.slot * e->d.max_blocks, s.blocks.data(), s.blocks.size() * 4,
                        hipMemcpyHostToDevice));
  }
  *out = &s;
  return DTD_OK;
}

static dtd_status kv_copy(dtd_engine* e, int64_t seq_id, int32_t layer, int32_t pos0, int32_t n,
                          void* k, void* v, void* ks, void* vs, bool write) {
  dtd_status st = ready(e);
  if (st) return st;
  const Dims& d = e->d;
  if (layer < 0 || layer >= d.L || pos0 < 0 || n <= 0 || (int64_t)pos0 + n > e->cfg.max_ctx || !k || !v)
    return fail(e, DTD_E_ARG, "kv copy: bad layer/range/pointer");
  const bool i8 = e->cfg.kvfmt == DTD_KV_I8;
  if (i8 && (!ks || !vs)) return fail(e, DTD_E_ARG, "kv copy: int8 KV needs scale buffers");
  Seq* s = nullptr;
  if (write) {
    if ((st = ensure_seq_blocks(e, seq_id, pos0 + n, &s))) return st;
  } else {
    auto it = e->seqs.find(seq_id);
    if (it == e->seqs.end()) return fail(e, DTD_E_NOSEQ, "kv read: unknown seq_id");
    s = &it->second;
    if (pos0 + n > (int)s->blocks.size() * d.bs) return fail(e, DTD_E_ARG, "kv read: positions not allocated");
  }
  HIP_OK(e, hipStreamSynchronize(e->stream));
  // one block of one layer is [Hkv][bs][hd] (+ scales [Hkv][bs]): copy it whole, patch the
  // touched positions on the host, copy it back
  const size_t eb = kv_elem_bytes(e->cfg.kvfmt);
  const size_t rowb = (size_t)d.hd * eb;
  const size_t blkb = (size_t)d.Hkv * d.bs * rowb;
  const size_t blks = (size_t)d.Hkv * d.bs;
  uint8_t* kb = (uint8_t*)e->kpool + (size_t)layer * e->kv_layer_elems * eb;
  uint8_t* vb = (uint8_t*)e->vpool + (size_t)layer * e->kv_layer_elems * eb;
  uint16_t* ksb = i8 ? e->kspool + (size_t)layer * e->kv_layer_scales : nullptr;
  uint16_t* vsb = i8 ? e->vspool + (size_t)layer * e->kv_layer_scales : nullptr;
  std::vector<uint8_t> img(blkb);
  std::vector<uint16_t> simg(blks);
  for (int which = 0; which < 2; which++) {
    uint8_t* pool = which ? vb : kb;
    uint16_t* spool = which ? vsb : ksb;
    uint8_t* host = (uint8_t*)(which ? v : k);
    uint16_t* hsc = (uint16_t*)(which ? vs : ks);
    for (int lb = pos0 / d.bs; lb <= (pos0 + n - 1) / d.bs; lb++) {
      const size_t blk = (size_t)s->blocks[(size_t)lb];
      const int t_lo = std::max(pos0, lb * d.bs), t_hi = std::min(pos0 + n, (lb + 1) * d.bs);
      HIP_OK(e, hipMemcpy(img.data(), pool + blk * blkb, blkb, hipMemcpyDeviceToHost));
      if (i8) HIP_OK(e, hipMemcpy(simg.data(), spool + blk * blks, blks * 2, hipMemcpyDeviceToHost));
      for (int pos = t_lo; pos < t_hi; pos++) {
        const int off = pos - lb * d.bs, t = pos - pos0;
        for (int j = 0; j < d.Hkv; j++) {
          uint8_t* dev_row = img.data() + ((size_t)j * d.bs + off) * rowb;
          uint8_t* host_row = host + ((size_t)t * d.Hkv + j) * rowb;
          uint16_t* dev_s = simg.data() + (size_t)j * d.bs + off;
          uint16_t* host_s = i8 ? hsc + (size_t)t * d.Hkv + j : nullptr;
          if (write) {
            memcpy(dev_row, host_row, rowb);
            if (i8) *dev_s = *host_s;
          } else {
            memcpy(host_row, dev_row, rowb);
            if (i8) *host_s = *dev_s;
          }
        }
      }
      if (write) {
        HIP_OK(e, hipMemcpy(pool + blk * blkb, img.data(), blkb, hipMemcpyHostToDevice));
        if (i8) HIP_OK(e, hipMemcpy(spool + blk * blks, simg.data(), blks * 2, hipMemcpyHostToDevice));
      }
    }
  }
  if (write && pos0 + n > s->len) grow_debug_len(e, seq_id, *s, pos0 + n);
  return DTD_OK;
}

extern "C" dtd_status dtd_debug_kv_write(dtd_engine* e, int64_t seq_id, int32_t layer, int32_t pos0,
                                         int32_t n, const void* k, const void* v, const void* k_scale,
                                         const void* v_scale) {
  return kv_copy(e, seq_id, layer, pos0, n, (void*)k, (void*)v, (void*)k_scale, (void*)v_scale, true);
}

extern "C" dtd_status dtd_debug_kv_read(dtd_engine* e, int64_t seq_id, int32_t layer, int32_t pos0,
                                        int32_t n, void* k, void* v, void* k_scale, void* v_scale) {
  return kv_copy(e, seq_id, layer, pos0, n, k, v, k_scale, v_scale, false);
}

extern "C" dtd_status dtd_debug_kv_fill(dtd_engine* e, int64_t seq_id, int32_t len, uint64_t seed) {
  dtd_status st = ready(e);
  if (st) return st;
  if (len <= 0 || len > e->cfg.max_ctx) return fail(e, DTD_E_ARG, "kv_fill: len %d outside [1, max_ctx]", len);
  Seq* s = nullptr;
  if ((st = ensure_seq_blocks(e, seq_id, len, &s))) return st;
  const Dims& d = e->d;
  const int nblk = blocks_needed(e, len);
  int32_t* blocks_dev = nullptr;
  if ((st = dev_alloc(e, &blocks_dev, (size_t)nblk * 4))) return st;
  hipError_t r = hipMemcpy(blocks_dev, s->blocks.data(), (size_t)nblk * 4, hipMemcpyHostToDevice);
  const size_t eb = kv_elem_bytes(e->cfg.kvfmt);
  for (int l = 0; l < d.L && r == hipSuccess; l++) {
    KvLayer kv;
    kv.k = (uint8_t*)e->kpool + (size_t)l * e->kv_layer_elems * eb;
    kv.v = (uint8_t*)e->vpool + (size_t)l * e->kv_layer_elems * eb;
    kv.ks = e->kspool ? e->kspool + (size_t)l * e->kv_layer_scales : nullptr;
    kv.vs = e->vspool ? e->vspool + (size_t)l * e->kv_layer_scales : nullptr;
    r = launch_kv_fill(d, kv, blocks_dev, nblk, len, l, seed, e->stream);
  }
  if (r == hipSuccess) r = hipStreamSynchronize(e->stream);
  (void)hipFree(blocks_dev);
  if (r != hipSuccess) {
    e->broken = true;
    return fail(e, DTD_E_HIP, "kv_fill: %s", hipGetErrorString(r));
  }
  if (len > s->len) grow_debug_len(e, seq_id, *s, len);
  return DTD_OK;
}

extern "C" dtd_status dtd_debug_kernel_timing(dtd_engine* e, int32_t kind, int32_t enable, double* total_ms,
                                              int64_t* count) {
  if (!e) return DTD_E_ARG;
  if (kind < 0 || kind > 6) return fail(e, DTD_E_ARG, "kernel_timing: kind %d outside [0, 6]", kind);
  HIP_OK(e, hipSetDevice(e->device));
  double total = 0.0;
  int64_t cnt = 0;
  if (e->timing_kind == kind && e->timers_used) {
    HIP_OK(e, hipStreamSynchronize(e->stream));
    for (size_t i = 0; i < e->timers_used; i++) {
      float ms = 0.f;
      HIP_OK(e, hipEventElapsedTime(&ms, e->timers[i].a, e->timers[i].b));
      total += ms;
      cnt++;
    }
  }
  e->timers_used = 0;
  e->timing_kind = enable ? kind : (e->timing_kind == kind ? -1 : e->timing_kind);
  if (total_ms) *total_ms = total;
  if (count) *count = cnt;
  return DTD_OK;
}

extern "C" dtd_status dtd_debug_set_path(dtd_engine* e, int32_t path) {
  if (!e) return DTD_E_ARG;
  if (path < 0 || path > 2) return fail(e, DTD_E_ARG, "set_path: path %d outside [0, 2]", path);
  if (path == 2 && !e->persist_ok) return fail(e, DTD_E_UNSUPPORTED, "persistent step kernel unavailable on this device");
  e->path = path;
  return DTD_OK;
}

extern "C" int32_t dtd_debug_uses_persistent(const dtd_engine* e, int32_t batch) {
  if (!e) return DTD_E_ARG;
  return e->persist_ok && batch == 1 && !e->capture && e->path != 1 ? 1 : 0;
}

extern "C" int32_t dtd_debug_plan_attention_chunks(int32_t batch, const int32_t* pos, int32_t n_kv_heads, int32_t max_chunks,
                                        int32_t slots, int32_t* ct, int32_t* cend) {
  if (batch < 1 || batch > kMaxBatch || !pos || !ct || !cend || n_kv_heads < 1 || max_chunks < 1 || slots < 1)
    return DTD_E_ARG;
  for (int b = 0; b < batch; b++)
    if (pos[b] < 0 || (int64_t)pos[b] + 1 > (int64_t)max_chunks * 2048) return DTD_E_ARG;
  std::vector<int> p(pos, pos + batch);
  return plan_chunks(batch, p.data(), n_kv_heads, max_chunks, slots, ct, cend);
}

extern "C" int32_t dtd_debug_step_kernel_shape(const dtd_engine* e) {
  if (!e) return DTD_E_ARG;
  return e->persist_ok ? persistent_fixed_hd(e->d) : 0;
}

extern "C" dtd_status dtd_debug_stream_read(const void* buf_dev, int64_t bytes, int32_t reps, void* hip_stream,
                                            double* gbs) {
  if (!buf_dev || bytes < 16 || reps <= 0 || !gbs) {
    g_create_err = "stream_read: null buffer or output, bytes < 16 or reps <= 0";
    return DTD_E_ARG;
  }
  hipStream_t st = (hipStream_t)hip_stream;
  int dev = 0, cus = 0;
  uint32_t* sink = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t r = hipGetDevice(&dev);
  if (r == hipSuccess) r = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (r == hipSuccess) r = hipMalloc((void**)&sink, 256);
  if (r == hipSuccess) r = hipEventCreate(&a);
  if (r == hipSuccess) r = hipEventCreate(&b);
  if (r == hipSuccess) r = launch_stream_read(buf_dev, (size_t)bytes, sink, cus, st);   // untimed first pass
  if (r == hipSuccess) r = hipEventRecord(a, st);
  for (int i = 0; i < reps && r == hipSuccess; i++) r = launch_stream_read(buf_dev, (size_t)bytes, sink, cus, st);
  if (r == hipSuccess) r = hipEventRecord(b, st);
  if (r == hipSuccess) r = hipEventSynchronize(b);
  float ms = 0.f;
  if (r == hipSuccess) r = hipEventElapsedTime(&ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (sink) (void)hipFree(sink);
  if (r != hipSuccess) {
    g_create_err = std::string("stream_read: ") + hipGetErrorString(r);
    return DTD_E_HIP;
  }
  *gbs = (double)(bytes / 16 * 16) * reps / (ms * 1e-3) / 1e9;
  return DTD_OK;
}
