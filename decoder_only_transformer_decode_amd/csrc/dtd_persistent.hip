// dtd_persistent.hip -- the whole batch-1 decode step as one persistent gfx950 kernel.
//
// One workgroup per compute unit (all resident: the launch is cooperative) runs every
// phase of the step:
//   per layer: [RMSNorm -> QKV GEMV + RoPE] | [KV append + split-K GQA attention; the
//   workgroup that ran a kv head's last chunk merges that head's chunks] | [O GEMV +
//   residual] | [RMSNorm -> gate/up GEMV + SwiGLU] | [down GEMV + residual]; then
//   [final RMSNorm -> LM head GEMV + greedy argmax].
//
// Hand-off between workgroups, without grid barriers or cache maintenance.  Every value
// that one workgroup passes to another is stored as a 64-bit word (tag << 32 | fp32 bits)
// with a device-scope store, which is written through to memory; the tag names the launch
// and the phase.  A consumer loads the words it needs with device-scope loads and re-polls
// a word until it carries the tag it expects.  Value and readiness sit in one naturally
// aligned word, so stores need no ordering among themselves (an agent-scope release or
// acquire would write back or invalidate a whole L2, costing far more than the data), and
// a workgroup waits only for what it reads: an attention item waits for its own head
// group's q/k/v, not for the whole QKV projection.  A buffer is only rewritten after a
// chain of such waits through every reader of its previous contents, so a reader never
// meets a later phase's word in place of the one it waits for.
//
// Weight streaming: each projection's rows are split into contiguous row-pair ranges per
// workgroup; within a workgroup, wave w owns pairs w, w+PW, ...  A wave walks its rows in
// 1 KB lines (16 bytes per lane, coalesced) in groups of GRP lines, double buffered in
// registers: while one group is multiplied against the input vector (held in LDS with a
// bank-conflict-free swizzle), the next is in flight.  At the end of a projection each wave
// issues the first group of the NEXT projection before it waits for that projection's input,
// so weights keep streaming from HBM while the dependency resolves.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "dtd_device.h"
#include "dtd_internal.h"

namespace dtd {
namespace {

using namespace dev;

constexpr int PW = kPersistWaves;   // waves per workgroup
constexpr int PT = PW * 64;         // threads per workgroup
constexpr int GRP = 8;              // lines per lane in one prefetch group
constexpr unsigned kSpinLimit = 1u << 20;

// tags of one layer's hand-offs: tag = epoch + layer * kTagsPerLayer + kind; the head's
// argmax words take epoch + L * kTagsPerLayer
enum { TG_QKV = 0, TG_PART = 1, TG_O = 2, TG_XM = 3, TG_H = 4, TG_XO = 5, kTagsPerLayer = 6 };

#ifdef DTD_PHASE_TRACE
// Phase timeline, in a profiling build only: wave 0 of each workgroup records the 100 MHz
// real-time counter at every phase boundary (1 + 11 per layer + 3 events).
constexpr int kTraceWG = 256, kTraceEv = 512;
__device__ uint64_t g_phase_trace[kTraceWG * kTraceEv];
#define PTRACE(ev)                                                                          \
  do {                                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < kTraceWG && (ev) < kTraceEv)                       \
      g_phase_trace[blockIdx.x * kTraceEv + (ev)] = __builtin_amdgcn_s_memrealtime();       \
  } while (0)
#else
#define PTRACE(ev) \
  do {             \
  } while (0)
#endif

template <int WFMT> struct PVec { static constexpr int VEC = 16; };   // elements per 16 B
template <> struct PVec<W_BF16> { static constexpr int VEC = 8; };

// ---------------------------------------------------------------------------------------
// tagged words
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ void put_tag(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Re-polls p until it carries tag.  Gives up (raising kErrBarrier and the workgroup's LDS
// fail flag) after kSpinLimit polls, or as soon as another thread or workgroup has given up,
// so every wait ends.
__device__ __noinline__ float wait_slow(const uint64_t* p, uint32_t tag, int32_t* err, int* fail) {
  unsigned spins = 0;
  for (;;) {
    if (*(volatile int*)fail) return 0.f;
    __builtin_amdgcn_s_sleep(2);
    const uint64_t w = get_word(p);
    if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
    ++spins;
    if (spins > kSpinLimit ||
        ((spins & 255) == 0 &&
         (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrBarrier))) {
      __hip_atomic_fetch_or(err, kErrBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *(volatile int*)fail = 1;
      return 0.f;
    }
  }
}

// value of word p (first loaded as w) once it carries tag
__device__ __forceinline__ float tag_value(const uint64_t* p, uint64_t w, uint32_t tag, int32_t* err, int* fail) {
  if ((uint32_t)(w >> 32) == tag) return __uint_as_float((uint32_t)w);
  return wait_slow(p, tag, err, fail);
}

// Reads n tagged words, word i at src(i), handing each value to put(i, v).  Every thread
// of the workgroup takes part with up to 8 loads in flight before it checks any tag.  The
// caller synchronises the workgroup and then tests the fail flag.
template <typename Src, typename Put>
__device__ __forceinline__ void gather(int n, uint32_t tag, int32_t* err, int* fail, Src src, Put put) {
  constexpr int B = 8;
  for (int i0 = 0; i0 < n; i0 += B * PT) {
    uint64_t w[B];
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int i = i0 + k * PT + (int)threadIdx.x;
      w[k] = i < n ? get_word(src(i)) : 0;
    }
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int i = i0 + k * PT + (int)threadIdx.x;
      if (i < n) put(i, tag_value(src(i), w[k], tag, err, fail));
    }
  }
}

// ---------------------------------------------------------------------------------------
// weight streaming
// ---------------------------------------------------------------------------------------

// LDS position of input element i, for lines of 64 lanes x VEC elements: the q-th float4 of
// lane l in line j sits at float4 index (j*VEC/4 + q)*64 + l.
template <int VEC>
__device__ __forceinline__ int swz(int i) {
  constexpr int KSTEP = 64 * VEC;
  const int st = i / KSTEP, r = i - st * KSTEP, ln = r / VEC, e = r - ln * VEC;
  return st * KSTEP + (e >> 2) * 256 + ln * 4 + (e & 3);
}

// one weight-streaming phase of this workgroup
struct PPhase {
  const uint8_t* w;
  const uint8_t* s;
  int N;     // matrix rows
  int Kb;    // bytes per row
  int K;     // elements per row
  int cpr;   // 1 KB lines per row
  int p0;    // first row pair owned by this workgroup
  int np;    // row pairs owned by this workgroup
};

template <int WFMT>
__device__ __forceinline__ PPhase make_phase(const MatDev& m, int g, int nwg) {
  PPhase p;
  p.w = (const uint8_t*)m.w;
  p.s = (const uint8_t*)m.s;
  p.N = m.rows;
  p.K = m.cols;
  p.Kb = m.cols * (WFMT == W_BF16 ? 2 : 1);
  p.cpr = (p.Kb + 1023) >> 10;
  const int pairs = (m.rows + 1) >> 1;
  p.p0 = (int)((long long)pairs * g / nwg);
  p.np = (int)((long long)pairs * (g + 1) / nwg) - p.p0;
  return p;
}

__device__ __forceinline__ PPhase empty_phase() {
  PPhase p{};
  p.cpr = 1;
  return p;
}

// pairs of this wave in the phase
__device__ __forceinline__ int wave_pairs(const PPhase& p, int wave) {
  return p.np > wave ? (p.np - wave + PW - 1) / PW : 0;
}

// Issues the loads of lines [c0, c0 + GRP) of this wave's stream in phase p.
template <int WFMT>
__device__ __forceinline__ void issue_group(const PPhase& p, int c0, uint4 (&buf)[GRP], float (&sc)[GRP]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int total = wave_pairs(p, wave) * 2 * p.cpr;
  int k = 0, rs = 0, j = 0;
  if (c0 < total) {
    const int per = 2 * p.cpr;
    k = c0 / per;
    const int rem = c0 - k * per;
    rs = rem >= p.cpr;
    j = rem - rs * p.cpr;
  }
#pragma unroll
  for (int s = 0; s < GRP; s++) {
    buf[s] = make_uint4(0u, 0u, 0u, 0u);
    sc[s] = 0.f;
    if (c0 + s < total) {
      const int row = 2 * (p.p0 + wave + PW * k) + rs;
      const int cb = (j * 64 + lane) * 16;
      if (row < p.N && cb < p.Kb) {
        buf[s] = *(const uint4*)(p.w + (size_t)row * p.Kb + cb);
        if constexpr (WFMT == W_Q8_0)
          sc[s] = f16_to_f32(*(const uint16_t*)(p.s + ((size_t)row * (p.K >> 5) + (cb >> 5)) * 2));
      }
      if (++j == p.cpr) {
        j = 0;
        if (++rs == 2) { rs = 0; ++k; }
      }
    }
  }
}

// Epilogue destinations of one phase: tagged words, and in a probe step (the c* pointers
// set) also plain values in the capture record.
struct PEpi {
  uint32_t tag;
  // QKV
  uint64_t* tq;
  uint64_t* tk;
  uint64_t* tv;
  float* cq;
  float* ck;
  float* cv;
  int pos;
  const float* rope_cos;
  const float* rope_sin;
  // residual: out[r] = xf[r] + value
  const float* xf;
  uint64_t* tout;
  float* cout;
  // SwiGLU
  uint64_t* th;
  void* ch;
  // logits
  float* logits;
  float* logits_out;
  float best;     // running argmax (lane 0)
  int best_idx;
};

__device__ __forceinline__ void emit(uint64_t* t, float* c, uint32_t tag, int i, float v) {
  if (c) c[i] = v;
  put_tag(t + i, tag, v);
}

template <int WFMT, int EPI>
__device__ __forceinline__ void pair_epilogue(const Dims& d, const PPhase& p, int pair, float v0, float v1,
                                              PEpi& e) {
  const int r0 = 2 * pair, r1 = r0 + 1;
  if constexpr (WFMT == W_INT8_ROW) {  // per-row scale after the dot
    v0 *= ((const float*)p.s)[r0];
    if (r1 < p.N) v1 *= ((const float*)p.s)[r1];
  }
  if constexpr (EPI == EPI_QKV) {
    // stored QKV rows: q and k heads hold the RoPE pairs (i, i + hd/2) as rows (2i, 2i+1)
    const int half = d.hd >> 1;
    if (r0 < d.q_dim + d.kv_dim) {
      const bool isq = r0 < d.q_dim;
      const int nn = isq ? r0 : r0 - d.q_dim;
      const int h = nn / d.hd, i = (nn - h * d.hd) >> 1;
      const float c = e.rope_cos[(size_t)e.pos * half + i];
      const float s = e.rope_sin[(size_t)e.pos * half + i];
      uint64_t* t = isq ? e.tq : e.tk;
      float* cp = isq ? e.cq : e.ck;
      emit(t, cp, e.tag, h * d.hd + i, v0 * c - v1 * s);
      emit(t, cp, e.tag, h * d.hd + i + half, v0 * s + v1 * c);
    } else {
      const int nn = r0 - d.q_dim - d.kv_dim;
      emit(e.tv, e.cv, e.tag, nn, v0);
      emit(e.tv, e.cv, e.tag, nn + 1, v1);
    }
  } else if constexpr (EPI == EPI_RESID) {
    emit(e.tout, e.cout, e.tag, r0, e.xf[r0] + v0);
    if (r1 < p.N) emit(e.tout, e.cout, e.tag, r1, e.xf[r1] + v1);
  } else if constexpr (EPI == EPI_SWIGLU) {
    const float hv = v0 / (1.0f + expf(-v0)) * v1;   // rows (2f, 2f+1) = (gate f, up f)
    if (e.ch) store_act(e.ch, pair, hv, d.act);
    put_tag(e.th + pair, e.tag, round_act(hv, d.act));
  } else {
    e.logits[r0] = v0;
    if (e.logits_out) e.logits_out[r0] = v0;
    if (v0 > e.best || (e.best_idx == INT_MAX && !isnan(v0))) { e.best = v0; e.best_idx = r0; }
    if (r1 < p.N) {
      e.logits[r1] = v1;
      if (e.logits_out) e.logits_out[r1] = v1;
      if (v1 > e.best) { e.best = v1; e.best_idx = r1; }
    }
  }
}

// Streams this wave's rows of phase p against the input vector in LDS (xs).  On entry pre
// holds this phase's first group (already issued); on exit it holds the first group of
// phase nx, issued before returning and still in flight.
template <int WFMT, int EPI>
__device__ __forceinline__ void gemv_phase(const Dims& d, const PPhase& p, const PPhase& nx, uint4 (&pre)[GRP],
                                           float (&psc)[GRP], const float* xs, PEpi& e) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int total = wave_pairs(p, wave) * 2 * p.cpr;
  const float4* x4 = (const float4*)xs;
  uint4 cur[GRP];
  float csc[GRP];
#pragma unroll
  for (int s = 0; s < GRP; s++) { cur[s] = pre[s]; csc[s] = psc[s]; }
  float acc0 = 0.f, acc1 = 0.f;
  int k = 0, rs = 0, j = 0;   // consume cursor
  for (int c0 = 0; c0 < total || c0 == 0; c0 += GRP) {
    if (c0 + GRP < total) issue_group<WFMT>(p, c0 + GRP, pre, psc);
    else issue_group<WFMT>(nx, 0, pre, psc);   // first group of the next phase
#pragma unroll
    for (int s = 0; s < GRP; s++) {
      if (c0 + s < total) {
        const uint4 w = cur[s];
        float part = 0.f;
        if constexpr (WFMT == W_BF16) {
          const float4 xa = x4[(j * 2 + 0) * 64 + lane], xb = x4[(j * 2 + 1) * 64 + lane];
          part = __uint_as_float(w.x << 16) * xa.x + __uint_as_float(w.x & 0xffff0000u) * xa.y +
                 __uint_as_float(w.y << 16) * xa.z + __uint_as_float(w.y & 0xffff0000u) * xa.w +
                 __uint_as_float(w.z << 16) * xb.x + __uint_as_float(w.z & 0xffff0000u) * xb.y +
                 __uint_as_float(w.w << 16) * xb.z + __uint_as_float(w.w & 0xffff0000u) * xb.w;
        } else {
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const float4 xv = x4[(j * 4 + q) * 64 + lane];
            part += sext8(u[q], 0) * xv.x + sext8(u[q], 1) * xv.y + sext8(u[q], 2) * xv.z +
                    sext8(u[q], 3) * xv.w;
          }
          if constexpr (WFMT == W_Q8_0) part *= csc[s];
        }
        if (rs) acc1 += part;
        else acc0 += part;
        if (++j == p.cpr) {
          j = 0;
          if (++rs == 2) {
            rs = 0;
            const float v0 = wave_sum(acc0), v1 = wave_sum(acc1);
            acc0 = acc1 = 0.f;
            if (lane == 0) pair_epilogue<WFMT, EPI>(d, p, p.p0 + wave + PW * k, v0, v1, e);
            ++k;
          }
        }
      }
    }
    // after the last group, pre holds the next phase's loads still in flight: copying them
    // here would wait for them, so they are left for the next phase to pick up
    if (c0 + GRP >= total) break;
#pragma unroll
    for (int s = 0; s < GRP; s++) { cur[s] = pre[s]; csc[s] = psc[s]; }
  }
}

// ---------------------------------------------------------------------------------------
// input staging
// ---------------------------------------------------------------------------------------

template <int VEC>
__device__ __forceinline__ void zero_tail(int K, float* xs) {
  constexpr int KSTEP = 64 * VEC;
  const int Kp = (K + KSTEP - 1) / KSTEP * KSTEP;
  for (int i = K + (int)threadIdx.x; i < Kp; i += PT) xs[swz<VEC>(i)] = 0.f;
}

// activation vector in plain storage (fp32 or bf16) into LDS, swizzled
template <int VEC>
__device__ __forceinline__ void stage_plain(const void* src, int act, int K, float* xs) {
  zero_tail<VEC>(K, xs);
  for (int i = threadIdx.x; i < K; i += PT) xs[swz<VEC>(i)] = load_act(src, i, act);
}

// tagged vector into LDS, swizzled
template <int VEC>
__device__ __forceinline__ void stage_tagged(const uint64_t* src, uint32_t tag, int K, float* xs, int32_t* err,
                                             int* fail) {
  zero_tail<VEC>(K, xs);
  gather(K, tag, err, fail, [&](int i) { return src + i; }, [&](int i, float v) { xs[swz<VEC>(i)] = v; });
}

// xs = round_act(xf / sqrt(mean(xf^2) + eps) * gain), xf in LDS (complete: the caller has
// synchronised); cap: optional copy in activation storage
template <int VEC>
__device__ __forceinline__ void norm_lds(const float* xf, const float* gain, int D, float eps, int act, float* xs,
                                         void* cap, float* red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += PT) ss += xf[i] * xf[i];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  zero_tail<VEC>(D, xs);
  for (int i = threadIdx.x; i < D; i += PT) {
    const float v = round_act(xf[i] * r * gain[i], act);
    if (cap) store_act(cap, i, v, act);
    xs[swz<VEC>(i)] = v;
  }
}

__device__ __forceinline__ void load_plain_f32(const void* src, int n, float* dst) {
  for (int i = threadIdx.x; i < n; i += PT) dst[i] = ((const float*)src)[i];
}

// ---------------------------------------------------------------------------------------
// the step kernel
// ---------------------------------------------------------------------------------------

template <int WFMT, int KVFMT>
__global__ __launch_bounds__(PT) void k_step(PersistArgs a) {
  constexpr int VEC = PVec<WFMT>::VEC;
  extern __shared__ float smem[];
  __shared__ float red[PW];
  __shared__ int sfail;
  __shared__ float wbest[PW];
  __shared__ int widx[PW];
  const Dims& d = a.d;
  const int g = blockIdx.x, nwg = gridDim.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const bool probe = a.inject != nullptr;
  const StepDesc* desc = a.desc;
  int32_t* err = a.err;
  float* xs = smem;                   // swizzled input vector of the current projection
  float* xf = smem + a.xs_floats;     // residual stream [D], plain order
  const int G = d.G, hd = d.hd, cs = hd + 2;
  auto T = [&](int l, int kind) { return a.epoch + (uint32_t)(l * kTagsPerLayer + kind); };
  auto inj = [&](int l, size_t off) { return (const void*)(a.inject + (size_t)l * a.po.record + off); };
  auto cap = [&](int l, size_t off) { return (void*)(a.capture + (size_t)l * a.po.record + off); };

  PTRACE(0);
  if (tid == 0) sfail = 0;
  // this step's block-table entries: every workgroup writes them (identical values), so its
  // own attention reads see them without a hand-off
  for (int u = tid; u < desc->n_updates; u += PT)
    a.bt[(size_t)desc->upd[u][0] * d.max_blocks + desc->upd[u][1]] = desc->upd[u][2];
  int tok = desc->tokens[0];
  if (tok < 0 || tok >= d.V) {
    if (tid == 0) __hip_atomic_fetch_or(err, kErrToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = 0;
  }
  const int pos = desc->pos[0], slot = desc->slot[0], pos_blk = desc->pos_block[0];

  uint4 pre[GRP];
  float psc[GRP];
  PPhase ph = make_phase<WFMT>(a.layers[0].qkv, g, nwg);
  issue_group<WFMT>(ph, 0, pre, psc);
  // layer-0 input: the token's embedding row, dequantised by every workgroup
  if (!probe)
    for (int i = tid; i < d.D; i += PT) xf[i] = deq_elem(a.emb, d.wfmt, tok, i);
  __syncthreads();

  PEpi e{};
  e.pos = pos;
  e.rope_cos = a.rope_cos;
  e.rope_sin = a.rope_sin;
  e.xf = xf;
  for (int l = 0; l < d.L; l++) {
    const PLayer& Ly = a.layers[l];
    const int tb = 1 + l * 11;
    PTRACE(tb);
    // ---- RMSNorm -> QKV GEMV + RoPE ----
    // A probe step takes every wait of a normal step (the waits are what order the reuse of
    // the hand-off buffers), then replaces the input it received with the injected one.
    if (l > 0) {
      gather(d.D, T(l - 1, TG_XO), err, &sfail, [&](int i) { return a.t_xo + i; },
             [&](int i, float v) { xf[i] = v; });
      __syncthreads();
      if (sfail) return;
    }
    if (probe) {
      load_plain_f32(inj(l, a.po.x_in), d.D, xf);
      __syncthreads();
      if (g == 0) {
        norm_lds<VEC>(xf, Ly.attn_norm, d.D, d.eps, d.act, xs, cap(l, a.po.xn), red);
        __syncthreads();
      }
      stage_plain<VEC>(inj(l, a.po.xn), d.act, d.D, xs);
    } else {
      norm_lds<VEC>(xf, Ly.attn_norm, d.D, d.eps, d.act, xs, nullptr, red);
    }
    __syncthreads();
    e.tag = T(l, TG_QKV);
    e.tq = a.t_q;
    e.tk = a.t_k;
    e.tv = a.t_v;
    e.cq = probe ? (float*)cap(l, a.po.q) : nullptr;
    e.ck = probe ? (float*)cap(l, a.po.k) : nullptr;
    e.cv = probe ? (float*)cap(l, a.po.v) : nullptr;
    PPhase nx = make_phase<WFMT>(Ly.o, g, nwg);   // the prefetch skips attention
    PTRACE(tb + 1);
    gemv_phase<WFMT, EPI_QKV>(d, ph, nx, pre, psc, xs, e);
    PTRACE(tb + 2);

    // ---- KV append + split-K attention ----
    const int nv = (pos + a.ct) / a.ct;
    const int items = d.Hkv * nv;
    const uint32_t tpart = T(l, TG_PART);
    {
      AttnCtx ac{};
      ac.d = d;
      ac.kv = Ly.kv;
      ac.bt = a.bt;
      ac.ct = a.ct;
      ac.nch = a.nch;
      float* ain = smem + attn_smem_floats(G, hd);   // [G*hd] q group | [hd] k | [hd] v
      const int nin = G * hd + 2 * hd;
      for (int it = g; it < items; it += nwg) {
        const int j = it / nv, c = it - j * nv;
        __syncthreads();
        gather(nin, T(l, TG_QKV), err, &sfail,
               [&](int t) {
                 return t < G * hd ? a.t_q + j * G * hd + t
                                   : t < G * hd + hd ? a.t_k + j * hd + (t - G * hd)
                                                     : a.t_v + j * hd + (t - G * hd - hd);
               },
               [&](int t, float v) { ain[t] = v; });
        if (probe) {
          const float* qi = (const float*)inj(l, a.po.q);
          const float* ki = (const float*)inj(l, a.po.k);
          const float* vi = (const float*)inj(l, a.po.v);
          for (int t = tid; t < nin; t += PT)
            ain[t] = t < G * hd ? qi[j * G * hd + t] : t < G * hd + hd ? ki[j * hd + t - G * hd]
                                                                       : vi[j * hd + t - G * hd - hd];
        }
        __syncthreads();
        if (sfail) return;
        uint64_t* tp = a.t_part;
        attn_item<KVFMT>(ac, 0, j, c, pos, slot, pos_blk, ain, ain + G * hd, ain + G * hd + hd, smem,
                         [tp, tpart](size_t i, float v) { put_tag(tp + i, tpart, v); });
      }
      PTRACE(tb + 3);
      // Merge: the workgroup that ran a head group's last chunk combines its chunks, after all
      // of its own items (so no workgroup waits on one that is itself waiting).
      for (int it = g; it < items; it += nwg) {
        const int j = it / nv, c = it - j * nv;
        if (c != nv - 1) continue;
        float* ml = smem;                 // [G][nv][2]: (m, l), then (weight, l)
        float* Ls = smem + 2 * G * nv;    // [G] sum of weighted l
        __syncthreads();
        gather(G * nv * 2, tpart, err, &sfail,
               [&](int t) {
                 const int gg = t / (2 * nv), r = t - gg * 2 * nv;
                 return a.t_part + ((size_t)(j * G + gg) * a.nch + (r >> 1)) * cs + hd + (r & 1);
               },
               [&](int t, float v) { ml[t] = v; });
        __syncthreads();
        if (sfail) return;
        for (int gg = wave; gg < G; gg += PW) {   // weights e^(m_c - M) and their l sum
          float M = -INFINITY;
          for (int cc = lane; cc < nv; cc += 64) M = fmaxf(M, ml[(gg * nv + cc) * 2]);
          M = wave_max(M);
          float L = 0.f;
          for (int cc = lane; cc < nv; cc += 64) {
            const float w = expf(ml[(gg * nv + cc) * 2] - M);
            ml[(gg * nv + cc) * 2] = w;
            L += w * ml[(gg * nv + cc) * 2 + 1];
          }
          L = wave_sum(L);
          if (lane == 0) Ls[gg] = L;
        }
        __syncthreads();
        for (int oi = tid; oi < G * hd; oi += PT) {
          const int gg = oi / hd, i = oi - gg * hd, h = j * G + gg;
          const uint64_t* P = a.t_part + (size_t)h * a.nch * cs + i;
          float acc = 0.f;
          for (int c0 = 0; c0 < nv; c0 += 8) {
            uint64_t w[8];
#pragma unroll
            for (int k = 0; k < 8; k++) w[k] = c0 + k < nv ? get_word(P + (size_t)(c0 + k) * cs) : 0;
#pragma unroll
            for (int k = 0; k < 8; k++)
              if (c0 + k < nv)
                acc += ml[(gg * nv + c0 + k) * 2] * tag_value(P + (size_t)(c0 + k) * cs, w[k], tpart, err, &sfail);
          }
          const float o = acc / Ls[gg];
          if (probe) store_act(cap(l, a.po.o), (size_t)h * hd + i, o, d.act);
          put_tag(a.t_o + h * hd + i, T(l, TG_O), round_act(o, d.act));
        }
        __syncthreads();
        if (sfail) return;
      }
    }

    PTRACE(tb + 4);
    // ---- O GEMV + residual ----
    __syncthreads();
    stage_tagged<VEC>(a.t_o, T(l, TG_O), d.q_dim, xs, err, &sfail);
    __syncthreads();
    if (sfail) return;
    if (probe) {
      stage_plain<VEC>(inj(l, a.po.o), d.act, d.q_dim, xs);
      __syncthreads();
    }
    e.tag = T(l, TG_XM);
    e.tout = a.t_xm;
    e.cout = probe ? (float*)cap(l, a.po.x_mid) : nullptr;
    ph = nx;
    nx = make_phase<WFMT>(Ly.gu, g, nwg);
    PTRACE(tb + 5);
    gemv_phase<WFMT, EPI_RESID>(d, ph, nx, pre, psc, xs, e);
    PTRACE(tb + 6);

    // ---- RMSNorm -> gate/up GEMV + SwiGLU ----
    __syncthreads();
    gather(d.D, T(l, TG_XM), err, &sfail, [&](int i) { return a.t_xm + i; }, [&](int i, float v) { xf[i] = v; });
    __syncthreads();
    if (sfail) return;
    if (probe) {
      load_plain_f32(inj(l, a.po.x_mid), d.D, xf);
      __syncthreads();
      if (g == 0) {
        norm_lds<VEC>(xf, Ly.ffn_norm, d.D, d.eps, d.act, xs, cap(l, a.po.xn2), red);
        __syncthreads();
      }
      stage_plain<VEC>(inj(l, a.po.xn2), d.act, d.D, xs);
    } else {
      norm_lds<VEC>(xf, Ly.ffn_norm, d.D, d.eps, d.act, xs, nullptr, red);
    }
    __syncthreads();
    e.tag = T(l, TG_H);
    e.th = a.t_h;
    e.ch = probe ? cap(l, a.po.h) : nullptr;
    ph = nx;
    nx = make_phase<WFMT>(Ly.down, g, nwg);
    PTRACE(tb + 7);
    gemv_phase<WFMT, EPI_SWIGLU>(d, ph, nx, pre, psc, xs, e);
    PTRACE(tb + 8);

    // ---- down GEMV + residual ----
    __syncthreads();
    stage_tagged<VEC>(a.t_h, T(l, TG_H), d.F, xs, err, &sfail);
    __syncthreads();
    if (sfail) return;
    if (probe) {
      stage_plain<VEC>(inj(l, a.po.h), d.act, d.F, xs);
      __syncthreads();
    }
    e.tag = T(l, TG_XO);
    e.tout = a.t_xo;
    e.cout = probe ? (float*)cap(l, a.po.x_out) : nullptr;
    ph = nx;
    nx = l + 1 < d.L ? make_phase<WFMT>(a.layers[l + 1].qkv, g, nwg)
                     : (desc->do_head ? make_phase<WFMT>(a.head, g, nwg) : empty_phase());
    PTRACE(tb + 9);
    gemv_phase<WFMT, EPI_RESID>(d, ph, nx, pre, psc, xs, e);
    PTRACE(tb + 10);
    ph = nx;
    __syncthreads();
  }
  if (!desc->do_head) return;

  // ---- final RMSNorm -> LM head + greedy argmax ----
  gather(d.D, T(d.L - 1, TG_XO), err, &sfail, [&](int i) { return a.t_xo + i; },
         [&](int i, float v) { xf[i] = v; });
  __syncthreads();
  if (sfail) return;
  if (probe) {
    load_plain_f32(inj(d.L - 1, a.po.x_out), d.D, xf);
    __syncthreads();
  }
  norm_lds<VEC>(xf, a.final_norm, d.D, d.eps, d.act, xs, nullptr, red);
  __syncthreads();
  e.logits = a.logits;
  e.logits_out = desc->logits_out;
  e.best = -INFINITY;
  e.best_idx = INT_MAX;
  PTRACE(1 + d.L * 11);
  gemv_phase<WFMT, EPI_LOGITS>(d, ph, empty_phase(), pre, psc, xs, e);
  PTRACE(2 + d.L * 11);
  if (lane == 0) { wbest[wave] = e.best; widx[wave] = e.best_idx; }
  __syncthreads();
  const uint32_t thead = T(d.L, 0);
  if (tid == 0) {
    float b = wbest[0];
    int bi = widx[0];
    for (int w = 1; w < PW; w++)
      if (wbest[w] > b || (wbest[w] == b && widx[w] < bi)) { b = wbest[w]; bi = widx[w]; }
    put_tag(a.t_am + 2 * g, thead, b);
    put_tag(a.t_am + 2 * g + 1, thead, __int_as_float(bi));
  }
  if (g != 0) return;
  // workgroup 0 reduces the per-workgroup winners (first index among equal maxima)
  gather(2 * nwg, thead, err, &sfail, [&](int t) { return a.t_am + t; }, [&](int t, float v) { xs[t] = v; });
  __syncthreads();
  if (sfail || wave != 0) return;
  float b = -INFINITY;
  int bi = INT_MAX;
  for (int w = lane; w < nwg; w += 64) {
    const float v = xs[2 * w];
    const int vi = __float_as_int(xs[2 * w + 1]);
    if (v > b || (v == b && vi < bi)) { b = v; bi = vi; }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(b, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (ov > b || (ov == b && oi < bi)) { b = ov; bi = oi; }
  }
  if (lane == 0) desc->next_tokens[0] = bi == INT_MAX ? 0 : bi;
  PTRACE(3 + d.L * 11);
}

template <int WFMT, int KVFMT>
const void* step_kernel() {
  return (const void*)k_step<WFMT, KVFMT>;
}

const void* pick(int wfmt, int kvfmt) {
  if (wfmt == W_INT8_ROW) {
    if (kvfmt == KV_F32) return step_kernel<W_INT8_ROW, KV_F32>();
    if (kvfmt == KV_BF16) return step_kernel<W_INT8_ROW, KV_BF16>();
    return step_kernel<W_INT8_ROW, KV_I8>();
  }
  if (wfmt == W_Q8_0) {
    if (kvfmt == KV_F32) return step_kernel<W_Q8_0, KV_F32>();
    if (kvfmt == KV_BF16) return step_kernel<W_Q8_0, KV_BF16>();
    return step_kernel<W_Q8_0, KV_I8>();
  }
  if (kvfmt == KV_F32) return step_kernel<W_BF16, KV_F32>();
  if (kvfmt == KV_BF16) return step_kernel<W_BF16, KV_BF16>();
  return step_kernel<W_BF16, KV_I8>();
}

}  // namespace

size_t persistent_xs_floats(const Dims& d, int nch) {
  const int vec = d.wfmt == W_BF16 ? 8 : 16, kstep = 64 * vec;
  int kmax = d.D > d.F ? d.D : d.F;
  if (d.q_dim > kmax) kmax = d.q_dim;
  size_t need = (size_t)(kmax + kstep - 1) / kstep * kstep;                             // projection input
  const size_t at = dev::attn_smem_floats(d.G, d.hd) + (size_t)d.G * d.hd + 2 * (size_t)d.hd;  // attention
  const size_t mg = 2 * (size_t)d.G * nch + (size_t)d.G;                                // chunk merge
  if (at > need) need = at;
  if (mg > need) need = mg;
  return (need + 3) / 4 * 4;
}

size_t persistent_smem_bytes(const Dims& d, int nch) {
  return (persistent_xs_floats(d, nch) + (size_t)d.D) * sizeof(float);
}

int persistent_tags_per_step(const Dims& d) { return d.L * kTagsPerLayer + 1; }

hipError_t persistent_prepare(const Dims& d, size_t smem, int* blocks_per_cu) {
  const void* f = pick(d.wfmt, d.kvfmt);
  hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (r != hipSuccess) return r;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, PT, smem);
}

hipError_t launch_persistent(const PersistArgs& a, int nwg, size_t smem, hipStream_t st) {
  void* args[] = {(void*)&a};
  return hipLaunchCooperativeKernel(pick(a.d.wfmt, a.d.kvfmt), dim3(nwg), dim3(PT), args, (unsigned)smem, st);
}

}  // namespace dtd

#ifdef DTD_PHASE_TRACE
// copies the phase timeline of the last launch ([256][512] uint64) to host memory
extern "C" int dtd_phase_trace_dump(void* host, size_t bytes) {
  if (bytes > sizeof(dtd::g_phase_trace)) bytes = sizeof(dtd::g_phase_trace);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(dtd::g_phase_trace), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : 1;
}
#endif
