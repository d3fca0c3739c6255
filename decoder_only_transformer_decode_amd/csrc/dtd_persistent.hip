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
// Weight streaming: each projection's row pairs are dealt out to the workgroups; within a
// workgroup, wave w owns pairs w, w+PW, ... (with fewer pairs than waves, several waves share
// a pair, each with part of its lines).  A wave walks its rows in
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
constexpr int kLogPW = __builtin_ctz(PW);
constexpr int kFixedG = 4, kFixedBs = 16;   // the common attention shape (with head size 128)
static_assert((PW & (PW - 1)) == 0, "waves per workgroup: a power of two");
constexpr int PT = PW * 64;         // threads per workgroup
constexpr int GRP = 2;              // lines per lane in one prefetch group
constexpr unsigned kSpinLimit = 1u << 20;

// tags of one layer's hand-offs: tag = epoch + layer * kTagsPerLayer + kind; the head's
// argmax words take epoch + L * kTagsPerLayer
enum { TG_QKV = 0, TG_PART = 1, TG_O = 2, TG_XM = 3, TG_H = 4, TG_XO = 5, kTagsPerLayer = 6 };

template <int WFMT> struct PVec { static constexpr int VEC = 16; };   // elements per 16 B
template <> struct PVec<W_BF16> { static constexpr int VEC = 8; };
template <> struct PVec<W_Q4_0> { static constexpr int VEC = 32; };   // one Q4_0 block

// ---------------------------------------------------------------------------------------
// tagged words
// ---------------------------------------------------------------------------------------

typedef __attribute__((address_space(1))) uint64_t gword;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Reads a register that a load may have written, unconditionally.  The compiler tracks loads
// in flight per register; a load whose register is read only under a branch some wave can
// skip counts as possibly pending after that branch, and the next wait for a weight group
// then drains every load in flight instead of waiting for that group alone.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

__device__ __forceinline__ void settle(const v4u& v) {
  settle(v.x);
  settle(v.y);
  settle(v.z);
  settle(v.w);
}

__device__ __forceinline__ void settle(const float4& v) {
  settle(v.x);
  settle(v.y);
  settle(v.z);
  settle(v.w);
}

__device__ __forceinline__ void settle(const uint4& v) {
  settle(v.x);
  settle(v.y);
  settle(v.z);
  settle(v.w);
}

__device__ __forceinline__ void put_tag(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store((gword*)p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_word(uint64_t* p, uint64_t w) {
  __hip_atomic_store((gword*)p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load((gword*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until all B words w[k] carry tag, re-loading the stale ones together (load(k))
// once per round, so that a batch costs one memory round trip per round rather than one per
// stale word.  Words a thread does not hold start out carrying the tag.  Gives up (raising
// kErrBarrier and the workgroup's LDS fail flag) after kSpinLimit rounds, or as soon as
// another thread or workgroup has given up, so every wait ends; the caller synchronises the
// workgroup and then tests the fail flag.
//
// SHIFT is the position of the tag in a word: 32 (value in the low half), or 48 for words
// that carry three bf16 values under a 16-bit tag.
template <int B, int SHIFT = 32, typename Load>
__device__ __forceinline__ void await_tags(uint64_t (&w)[B], uint32_t tag, int32_t* err, int* fail, Load load) {
  unsigned spins = 0;
  for (;;) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < B; k++) all = all && (uint32_t)(w[k] >> SHIFT) == tag;
    if (all || *(volatile int*)fail) return;
    ++spins;
    if (spins > kSpinLimit ||
        ((spins & 255) == 0 &&
         (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrBarrier))) {
      __hip_atomic_fetch_or(err, kErrBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *(volatile int*)fail = 1;
      return;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int k = 0; k < B; k++)
      if ((uint32_t)(w[k] >> SHIFT) != tag) w[k] = load(k);
  }
}

// Reads n tagged words, word i at src(i), handing each value to put(i, v).  Every thread
// of the workgroup takes part with up to B loads in flight.  The caller synchronises the
// workgroup and then tests the fail flag.
// Reads n tagged words, word i at src(i), handing each whole word to put(i, w).  Every
// thread of the workgroup takes part with up to B loads in flight.  The caller synchronises
// the workgroup and then tests the fail flag.
template <int B, int SHIFT, typename Src, typename Put>
__device__ __forceinline__ void gather_words(int n, uint32_t tag, int32_t* err, int* fail, Src src, Put put) {
  for (int i0 = 0; i0 < n; i0 += B * PT) {
    uint64_t w[B];
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int i = i0 + k * PT + (int)threadIdx.x;
      w[k] = i < n ? get_word(src(i)) : (uint64_t)tag << SHIFT;
    }
    await_tags<B, SHIFT>(w, tag, err, fail, [&](int k) { return get_word(src(i0 + k * PT + (int)threadIdx.x)); });
#pragma unroll
    for (int k = 0; k < B; k++) {
      const int i = i0 + k * PT + (int)threadIdx.x;
      if (i < n) put(i, w[k]);
    }
#pragma unroll
    for (int k = 0; k < B; k++) settle(w[k]);
  }
}

// the same, handing each word's value (low 32 bits) as a float
template <int B = 8, typename Src, typename Put>
__device__ __forceinline__ void gather(int n, uint32_t tag, int32_t* err, int* fail, Src src, Put put) {
  gather_words<B, 32>(n, tag, err, fail, src, [&](int i, uint64_t w) { put(i, __uint_as_float((uint32_t)w)); });
}

// ---------------------------------------------------------------------------------------
// weight streaming
// ---------------------------------------------------------------------------------------

// LDS position of input element i, for lines of 64 lanes x VEC elements: the q-th float4 of
// lane l in line j sits at float4 index (j*VEC/4 + q)*64 + l.
// (i >= 0; unsigned, the divisions are plain shifts)
template <int VEC>
__device__ __forceinline__ int swz(int i) {
  constexpr unsigned KSTEP = 64 * VEC;
  const unsigned u = (unsigned)i, st = u / KSTEP, r = u % KSTEP, ln = r / VEC, e = r % VEC;
  return (int)(st * KSTEP + (e >> 2) * 256 + ln * 4 + (e & 3));
}

// this thread's wave, as a value the compiler knows is wave-uniform (branches on it become
// scalar branches, and both arms of an if/else are never laid out as one masked sequence)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// one weight-streaming phase of this workgroup, with the share of the calling wave
struct PPhase {
  const uint8_t* w;
  const uint8_t* s;
  int N;       // matrix rows
  int Kb;      // bytes per row
  int K;       // elements per row
  int p0;      // first row pair owned by this workgroup
  int ps;      // stride between the row pairs it owns
  int np;      // row pairs owned by this workgroup
  int sp;      // waves sharing each pair, each with a contiguous range of its lines
  // this wave's share: pairs pb, pb + pst, ...; lines [jb, je) of each; 2 * pairs * (je - jb)
  // lines in all; the results of its k-th pair go to LDS slots ob + ost * k (+1)
  int pb, pst, jb, je, total, ob, ost;
};

template <int WFMT>
__device__ __forceinline__ PPhase make_phase(const MatDev& m, int g, int nwg) {
  PPhase p;
  p.w = (const uint8_t*)m.w;
  p.s = (const uint8_t*)m.s;
  p.N = m.rows;
  p.K = m.cols;
  p.Kb = WFMT == W_BF16 ? m.cols * 2 : (WFMT == W_Q4_0 ? m.cols >> 1 : m.cols);
  const int cpr = (p.Kb + 1023) >> 10;   // 1 KB lines per row
  // Row pairs are dealt out round-robin (workgroup g owns pairs g, g + nwg, ...), not in one
  // contiguous slice per workgroup: every hand-off lines all workgroups up at the start of a
  // projection, and with contiguous slices they would then all read the same offset of
  // slices a fixed stride apart, which piles the requests onto a few HBM channels; dealt
  // out, they read neighbouring rows of one region.
  const int pairs = (m.rows + 1) >> 1;
  p.p0 = g;
  p.ps = nwg;
  p.np = g < pairs ? (pairs - 1 - g) / nwg + 1 : 0;
  // With fewer pairs than waves, sp waves share each pair, each taking a contiguous range of
  // its lines, so that every wave keeps loads in flight; their partial results meet in the
  // epilogue.
  // (sp and ws are powers of two: their divisions are shifts)
  int sp = 1, lsp = 0;
  while (2 * sp <= PW && 2 * sp * p.np <= PW && 2 * sp <= cpr) sp *= 2, lsp++;
  p.sp = sp;
  const int lws = kLogPW - lsp, ws = PW >> lsp, wave = wave_id();
  const int part = wave >> lws, wl = wave & (ws - 1);
  const int ch = (cpr + sp - 1) >> lsp;
  p.jb = min(cpr, part * ch);
  p.je = min(cpr, p.jb + ch);
  const int npw = p.np > wl ? (p.np - wl + ws - 1) >> lws : 0;
  p.total = 2 * npw * (p.je - p.jb);
  p.pb = g + nwg * wl;
  p.pst = nwg * ws;
  p.ob = 2 * (part * p.np + wl);
  p.ost = 2 * ws;
  return p;
}

// a phase with no rows; its (unused) loads read `any`, a readable global address
__device__ __forceinline__ PPhase empty_phase(const void* any) {
  PPhase p{};
  p.ps = 1;
  p.sp = 1;
  p.je = 1;
  p.pst = 1;
  p.ost = 2;
  p.w = p.s = (const uint8_t*)any;
  return p;
}


// The weight stream's loads are issued so that the compiler's wait insertion can count
// them exactly: every group issues the same loads unconditionally, each buffer has one
// issue site per loop, and branches depend only on wave-uniform values.  Otherwise it
// falls back to a full drain (vmcnt(0)) before each group, leaving one group in flight
// per wave instead of two.

template <int WFMT> struct Grp {
  static constexpr int SC = WFMT == W_BF16 ? 0 : GRP;   // scale loads per group
};

struct WBuf {
  v4u w[GRP];
  uint32_t sc[GRP];   // Q8_0, Q4_0: fp16 block scale bits; int8-row: fp32 row scale bits
};

// A wave's stream in one phase: its row pairs in turn, each pair as 2*cpr lines that
// interleave the two rows, (row 0, line 0), (row 1, line 0), (row 0, line 1), ... so a line's
// row is the parity of its index, and both rows of a line step share one input chunk.  A
// pair's line count is even and GRP is even, so every group starts on row 0.
//
// Position of the next line step a wave issues: line count c, pair k (of the wave) and line j
// of the rows.  Kept across calls so that no division is needed per group.
struct ICur {
  int c, k, j;
};

// Issues the next GRP lines of this wave's stream in phase p, with their scales (Q8_0: the
// block scale of the lane's 16 columns; Q4_0: the scale of the lane's whole block of 32;
// int8-row: the row scale), and advances the cursor.  Every call issues
// the same loads whatever the phase: a line (or a lane's part of one) outside the matrix reads
// offset 0 of the matrix instead, and its value is never used (whole lines are skipped by the
// consumer; a lane's part past the row end meets the input vector's zero padding).  Addresses
// are a uniform base plus a 32-bit offset (a matrix is below 4 GiB).
template <int WFMT>
__device__ __forceinline__ void issue_group(const PPhase& p, ICur& ic, WBuf& b) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < GRP; s++) {
    const int row = 2 * (p.pb + p.pst * ic.k) + (s & 1);
    const int cb = (ic.j * 64 + lane) * 16;
    const bool rok = ic.c + s < p.total && row < p.N;
    const bool ok = rok && cb < p.Kb;
    b.w[s] = gload_stream<v4u>(p.w + (ok ? (uint32_t)row * (uint32_t)p.Kb + (uint32_t)cb : 0u));
    if constexpr (WFMT == W_Q8_0)
      b.sc[s] = gload<uint16_t>(p.s + (ok ? ((uint32_t)row * (uint32_t)(p.K >> 5) + (uint32_t)(cb >> 5)) * 2u : 0u));
    else if constexpr (WFMT == W_Q4_0)
      b.sc[s] = gload<uint16_t>(p.s + (ok ? ((uint32_t)row * (uint32_t)(p.K >> 5) + (uint32_t)(cb >> 4)) * 2u : 0u));
    else if constexpr (WFMT == W_INT8_ROW)
      b.sc[s] = gload<uint32_t>(p.s + (rok ? (uint32_t)row * 4u : 0u));
    if (s & 1) {
      if (++ic.j == p.je) { ic.j = p.jb; ++ic.k; }
    }
  }
  ic.c += GRP;
}

// Epilogue destinations of one phase: tagged words, and in a probe step (the c* pointers
// set) also plain values in the capture record.
struct PEpi {
  uint32_t tag;
  int act;        // activation type (a constant in the step kernels that fix it)
  // QKV
  uint64_t* tq;
  uint64_t* tk;
  uint64_t* tv;
  float* cq;
  float* ck;
  float* cv;
  const float* rope;   // LDS: cos | sin of this step's position, hd/2 each
  // residual: out[r] = xf[r] + value
  const float* xf;
  uint64_t* tout;
  float* cout;
  // SwiGLU
  uint64_t* th;
  void* ch;
  int hs;         // bf16 activations: packed words of h per workgroup
  // logits
  float* logits;
  float* logits_out;
  float best;     // this thread's argmax over its rows
  int best_idx;
};

__device__ __forceinline__ void emit(uint64_t* t, float* c, uint32_t tag, int i, float v) {
  if (c) c[i] = v;
  put_tag(t + i, tag, v);
}

// Result of row r (0 or 1) of local pair t (global pair p.p0 + p.ps*t) of a finished
// projection: the parts of the waves that shared the pair, added in a fixed order.
__device__ __forceinline__ float pair_result(const PPhase& p, const float* ores, int t, int r) {
  float v = ores[2 * t + r];
  for (int part = 1; part < p.sp; part++) v += ores[2 * (part * p.np + t) + r];
  return v;
}

// The epilogue of one projection, run by the whole workgroup after its rows are done (their
// results in ores, LDS, read through pair_result).
// Stores happen only here, never inside the streaming loop: gfx950 counts loads and stores
// on one counter, so a store pending there would make every wait for a weight group also
// wait for the store's acknowledgement and for the group issued after it.
template <int EPI>
__device__ __forceinline__ void phase_epilogue(const Dims& d, const PPhase& p, const float* ores, PEpi& e) {
  if constexpr (EPI == EPI_QKV) {
    // stored QKV rows: q and k heads hold the RoPE pairs (i, i + hd/2) as rows (2i, 2i+1)
    const int half = d.hd >> 1;
    for (int t = threadIdx.x; t < p.np; t += PT) {
      const int r = 2 * (p.p0 + p.ps * t);
      const float v0 = pair_result(p, ores, t, 0), v1 = pair_result(p, ores, t, 1);
      if (r < d.q_dim + d.kv_dim) {
        const bool isq = r < d.q_dim;
        const int nn = isq ? r : r - d.q_dim;
        const int h = nn / d.hd, i = (nn - h * d.hd) >> 1;
        const float c = e.rope[i], sn = e.rope[half + i];
        uint64_t* tt = isq ? e.tq : e.tk;
        float* cp = isq ? e.cq : e.ck;
        emit(tt, cp, e.tag, h * d.hd + i, v0 * c - v1 * sn);
        emit(tt, cp, e.tag, h * d.hd + i + half, v0 * sn + v1 * c);
      } else {
        const int nn = r - d.q_dim - d.kv_dim;
        emit(e.tv, e.cv, e.tag, nn, v0);
        emit(e.tv, e.cv, e.tag, nn + 1, v1);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    for (int u = threadIdx.x; u < 2 * p.np; u += PT) {
      const int r = 2 * (p.p0 + p.ps * (u >> 1)) + (u & 1);
      if (r < p.N) emit(e.tout, e.cout, e.tag, r, e.xf[r] + pair_result(p, ores, u >> 1, u & 1));
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (e.act == ACT_BF16) {
      // three outputs per word under a 16-bit tag: word u of this workgroup carries its local
      // pairs 3u, 3u + 1, 3u + 2 in bits 0-15, 16-31, 32-47.  Every one of its hs words is
      // written in every layer, pads as zero, so a stale word is never more than one layer's
      // tags behind and a 16-bit tag cannot be mistaken.
      // One output per lane, the three of word u in lanes 4u .. 4u+2 of a quad (16 words per
      // wave and pass), so that a lane computes one SiLU, not three in a row; the quad's first
      // lane collects the other two by DPP and stores the word.
      const int lane = threadIdx.x & 63;
      for (int u0 = 16 * wave_id(); u0 < e.hs; u0 += 16 * PW) {   // wave-uniform
        const int u = u0 + (lane >> 2), hh = lane & 3, t = 3 * u + hh;
        uint32_t b = 0;
        if (hh < 3 && t < p.np) {   // rows (2f, 2f+1) = (gate f, up f)
          const float v0 = pair_result(p, ores, t, 0), v1 = pair_result(p, ores, t, 1);
          const float hv = v0 / (1.0f + expf(-v0)) * v1;
          if (e.ch) store_act(e.ch, p.p0 + p.ps * t, hv, e.act);
          b = f32_to_bf16(hv);
        }
        // quad_perm [1,1,1,1] and [2,2,2,2]: every lane of the quad reads lane 1, lane 2
        const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x55, 0xf, 0xf, false);
        const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xaa, 0xf, 0xf, false);
        if (hh == 0 && u < e.hs)
          put_word(e.th + (size_t)p.p0 * e.hs + u,
                   (uint64_t)(e.tag & 0xffffu) << 48 | (uint64_t)b2 << 32 | (uint64_t)b1 << 16 | b);
      }
    } else {
      for (int t = threadIdx.x; t < p.np; t += PT) {   // rows (2f, 2f+1) = (gate f, up f)
        const int f = p.p0 + p.ps * t;
        const float v0 = pair_result(p, ores, t, 0), v1 = pair_result(p, ores, t, 1);
        const float hv = v0 / (1.0f + expf(-v0)) * v1;
        if (e.ch) store_act(e.ch, f, hv, e.act);
        put_tag(e.th + f, e.tag, hv);
      }
    }
  } else {
    for (int u = threadIdx.x; u < 2 * p.np; u += PT) {   // rows visited in increasing order
      const int r = 2 * (p.p0 + p.ps * (u >> 1)) + (u & 1);
      if (r >= p.N) continue;
      const float v = pair_result(p, ores, u >> 1, u & 1);
      gstore<float>(e.logits + r, v);
      if (e.logits_out) gstore<float>(e.logits_out + r, v);
      if (v > e.best || (e.best_idx == INT_MAX && !isnan(v))) { e.best = v; e.best_idx = r; }
    }
  }
}

// Sum over the 64 lanes of a wave with DPP moves only (no LDS round trips): quad swaps,
// then half-row and row mirrors give every lane its 16-lane row sum, two row broadcasts
// fold rows 0+1 into row 1 / rows 2+3 into row 3 and then row 1 into row 3; lane 63 holds
// the total, returned as a wave-uniform value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0xb1, 0xf>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4e, 0xf>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xf>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);   // row_mirror
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over the workgroup: DPP within each wave, then the PW wave totals through LDS (red,
// 16-byte aligned) read back as two float4, added in a fixed order.  Uses the compile-time
// wave count: reading blockDim would be a scalar memory load on the critical path.
__device__ __forceinline__ float wg_sum(float v, float* red) {
  static_assert(PW == 8, "two float4 of wave totals");
  const float t = wave_total(v);
  __syncthreads();   // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  const float4 a = *(const float4*)red, b = *(const float4*)(red + 4);
  return ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
}

// the same shape of reduction for the maximum (rows left out by a broadcast keep -inf)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp((int)0xff800000, __float_as_int(v), CTRL, ROW_MASK,
                                                             0xf, false)));
}

__device__ __forceinline__ float wave_top(float v) {
  v = dpp_max<0xb1, 0xf>(v);
  v = dpp_max<0x4e, 0xf>(v);
  v = dpp_max<0x141, 0xf>(v);
  v = dpp_max<0x140, 0xf>(v);
  v = dpp_max<0x142, 0xa>(v);
  v = dpp_max<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// consume cursor of one wave's stream: line step j of pair k, and the running dot products
// of the pair's two rows
struct Cursor {
  int k, j;
  float acc0, acc1;
  float rsc0, rsc1;   // int8-row: scales of the pair's rows
};

// Q4_0 nibble k (0..7) of v as (q - 8) / 16, where v holds the codes with bit 3 of every
// nibble flipped: a nibble q ^ 8 read as a signed 4-bit integer is q - 8, and
// v_cvt_off_f32_i4 converts the low 4 bits of its operand to that integer / 16.  The
// operand's byte comes straight out of the register (an SDWA byte select), so an even nibble
// costs one instruction and the odd ones share one shift per dword.
template <int SEL>
__device__ __forceinline__ float q4_byte(uint32_t v) {
  float r;
  if constexpr (SEL == 0)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(v));
  else if constexpr (SEL == 1)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(v));
  else if constexpr (SEL == 2)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(v));
  else
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(v));
  return r;
}

// dot product of one line (16 bytes per lane) with this lane's input chunk; Q4_0 lines give
// it / 16 (the scale carries the factor 16)
template <int WFMT>
__device__ __forceinline__ float line_dot(const v4u& v, const float4 (&x)[PVec<WFMT>::VEC / 4]) {
  float part = 0.f;
  if constexpr (WFMT == W_Q4_0) {
    // the lane's 16 bytes are one block of 32 columns: byte b holds column b in its low 4
    // bits and column b + 16 in its high 4 bits (the Q4_0 block of "Go 语言原本" 20.2.4)
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint32_t lo = u[q] ^ 0x88888888u, hi = lo >> 4;
      part = fmaf(q4_byte<0>(lo), x[q].x, part);
      part = fmaf(q4_byte<1>(lo), x[q].y, part);
      part = fmaf(q4_byte<2>(lo), x[q].z, part);
      part = fmaf(q4_byte<3>(lo), x[q].w, part);
      part = fmaf(q4_byte<0>(hi), x[4 + q].x, part);
      part = fmaf(q4_byte<1>(hi), x[4 + q].y, part);
      part = fmaf(q4_byte<2>(hi), x[4 + q].z, part);
      part = fmaf(q4_byte<3>(hi), x[4 + q].w, part);
    }
  } else if constexpr (WFMT == W_BF16) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 xq = x[q >> 1];
      const float x0 = q & 1 ? xq.z : xq.x, x1 = q & 1 ? xq.w : xq.y;
      part = fmaf(__uint_as_float(u[q] << 16), x0, part);
      part = fmaf(__uint_as_float(u[q] & 0xffff0000u), x1, part);
    }
  } else {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      part = fmaf(sext8(u[q], 0), x[q].x, part);
      part = fmaf(sext8(u[q], 1), x[q].y, part);
      part = fmaf(sext8(u[q], 2), x[q].z, part);
      part = fmaf(sext8(u[q], 3), x[q].w, part);
    }
  }
  return part;
}

// Multiplies lines [c0, c0 + GRP) of buffer b against the input vector: two line steps, each
// one line of row 0 and one of row 1 of a pair at the same input chunk.  A finished pair's
// dot products go to ores (LDS, local pair index).  Every line's registers are read whether
// or not the line is real (a pad step's products are dropped by a select): a load whose value
// is never read is still pending when its register is reissued, and the compiler then waits
// for every load in flight, not just that one.
template <int WFMT>
__device__ __forceinline__ void consume_group(const PPhase& p, int c0, int total, const WBuf& b, const float4* x4,
                                              Cursor& cu, float* ores) {
  const int lane = threadIdx.x & 63;
  if (c0 >= total) {   // a pad group (wave-uniform): its registers are read, nothing else
    // (the scales in the form the products use, so that no conversion of them is placed
    // next to their loads)
#pragma unroll
    for (int s = 0; s < GRP; s++) {
      settle(b.w[s]);
      if constexpr (WFMT == W_Q8_0 || WFMT == W_Q4_0) settle(f16_to_f32((uint16_t)b.sc[s]));
      else if constexpr (WFMT == W_INT8_ROW) settle(__uint_as_float(b.sc[s]));
    }
    return;
  }
  constexpr int XQ = PVec<WFMT>::VEC / 4;      // float4 of input per lane and line
  constexpr int NS = GRP / 2;                  // line steps in a group
  // all steps' input chunks first, so their LDS round trips overlap (a pad step reads some
  // chunk below cpr)
  float4 xc[NS][XQ];
  int jj = cu.j;
#pragma unroll
  for (int st = 0; st < NS; st++) {
#pragma unroll
    for (int q = 0; q < XQ; q++) xc[st][q] = x4[(jj * XQ + q) * 64 + lane];
    jj = jj + 1 == p.je ? p.jb : jj + 1;
  }
  float part[GRP];
#pragma unroll
  for (int st = 0; st < NS; st++) {
    part[2 * st] = line_dot<WFMT>(b.w[2 * st], xc[st]);
    part[2 * st + 1] = line_dot<WFMT>(b.w[2 * st + 1], xc[st]);
  }
  if constexpr (WFMT == W_Q8_0) {
#pragma unroll
    for (int s = 0; s < GRP; s++) part[s] *= f16_to_f32((uint16_t)b.sc[s]);
  } else if constexpr (WFMT == W_Q4_0) {   // (q - 8) / 16 above: the factor 16 goes with d
#pragma unroll
    for (int s = 0; s < GRP; s++) part[s] *= 16.f * f16_to_f32((uint16_t)b.sc[s]);
  }
#pragma unroll
  for (int st = 0; st < GRP / 2; st++) {
    const bool valid = c0 + 2 * st < total;   // wave-uniform; both lines of a step together
    cu.acc0 += valid ? part[2 * st] : 0.f;
    cu.acc1 += valid ? part[2 * st + 1] : 0.f;
    if constexpr (WFMT == W_INT8_ROW) {   // every line of a row carries the row's scale
      cu.rsc0 = valid ? __uint_as_float(b.sc[2 * st]) : cu.rsc0;
      cu.rsc1 = valid ? __uint_as_float(b.sc[2 * st + 1]) : cu.rsc1;
    }
    if (valid && ++cu.j == p.je) {
      cu.j = p.jb;
      // int8-row: per-row scale after the dot
      const float v0 = wave_total(cu.acc0) * cu.rsc0, v1 = wave_total(cu.acc1) * cu.rsc1;
      cu.acc0 = cu.acc1 = 0.f;
      if (lane == 0) {
        const int o = p.ob + p.ost * cu.k;
        ores[o] = v0;
        ores[o + 1] = v1;
      }
      ++cu.k;
    }
  }
}

// Issues the next group of phase p into b (past the wave's last line: pad loads, see
// issue_group).  Nothing of the following consume may be scheduled above these loads: a
// product of the group issued just before would then wait for that group before this one is
// on its way.
template <int WFMT>
__device__ __forceinline__ void issue_next(const PPhase& p, WBuf& b, ICur& ic) {
  issue_group<WFMT>(p, ic, b);
  __builtin_amdgcn_sched_barrier(0);
}

// Streams this wave's rows of phase p against the input vector in LDS (xs), leaving each
// finished dot product in ores.  Two register buffers alternate, A with the even groups and
// B with the odd ones (no copies between them, so nothing waits on a load in flight): on
// entry A and B hold groups 0 and 1 of this phase (issued before the wait for its input); on
// exit they hold pad loads, whose values are not used (the caller issues the next phase's
// first groups after its epilogue).  The group count is padded to an even number >= 2 so
// the roles line up.  A wave's share of one projection is only a few groups, so without
// loads in flight across the wait between phases every phase would cost whole round trips
// to HBM.
template <int WFMT>
__device__ __forceinline__ void gemv_phase(const PPhase& p, WBuf& A, WBuf& B, const float* xs, float* ores,
                                           ICur& ic) {
  const int wave = wave_id();
  const int total = p.total;
  int ng2 = ((total + GRP - 1) / GRP + 1) & ~1;
  if (ng2 < 2) ng2 = 2;
  const float4* x4 = (const float4*)xs;
  Cursor cu{0, p.jb, 0.f, 0.f, 1.f, 1.f};
  // The two waves sharing a SIMD (w and w + 4) take turns at the higher issue priority, one
  // group each; otherwise the older wave wins every tie and the younger one finishes its
  // share of the phase well after it.
  const bool young = wave >= PW / 2;
  for (int gi = 0; gi < ng2; gi += 2) {
    if (young) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    consume_group<WFMT>(p, gi * GRP, total, A, x4, cu, ores);       // B stays in flight
    issue_next<WFMT>(p, A, ic);
    if (young) __builtin_amdgcn_s_setprio(0);
    else __builtin_amdgcn_s_setprio(1);
    consume_group<WFMT>(p, (gi + 1) * GRP, total, B, x4, cu, ores); // A stays in flight
    issue_next<WFMT>(p, B, ic);
  }
  __builtin_amdgcn_s_setprio(0);
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

// tagged words carrying two bf16 values each (low half, high half) into LDS, swizzled;
// pos(w, i0, i1) gives the two element indices of word w (-1: none)
template <int VEC, int B = 8, typename Pos>
__device__ __forceinline__ void stage_tagged_pairs(const uint64_t* src, uint32_t tag, int nwords, int K, float* xs,
                                                   int32_t* err, int* fail, Pos pos) {
  zero_tail<VEC>(K, xs);
  gather<B>(nwords, tag, err, fail, [&](int w) { return src + w; }, [&](int w, float v) {
    const uint32_t b = __float_as_uint(v);
    int i0, i1;
    pos(w, i0, i1);
    if (i0 >= 0) xs[swz<VEC>(i0)] = __uint_as_float(b << 16);
    if (i1 >= 0) xs[swz<VEC>(i1)] = __uint_as_float(b & 0xffff0000u);
  });
}

// tagged vector into LDS, swizzled
template <int VEC>
__device__ __forceinline__ void stage_tagged(const uint64_t* src, uint32_t tag, int K, float* xs, int32_t* err,
                                             int* fail) {
  zero_tail<VEC>(K, xs);
  gather(K, tag, err, fail, [&](int i) { return src + i; }, [&](int i, float v) { xs[swz<VEC>(i)] = v; });
}

// RMSNorm gains of this thread's elements (i = tid + k*PT), loaded ahead of the wait for
// the vector they scale
constexpr int kNormPer = 8;             // model width up to 8 * PT
constexpr int kNormV = kNormPer / 4;    // passes of 4 consecutive elements per thread

// this thread's gains: elements 4(tid + k PT) .. +4 of pass k (0 past D; D is a multiple of 4)
__device__ __forceinline__ void gain_issue(const float* gain, int D, float4 (&gn)[kNormV]) {
#pragma unroll
  for (int k = 0; k < kNormV; k++) {
    const int i = 4 * ((int)threadIdx.x + k * PT);
    gn[k] = i < D ? gload<float4>(gain + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// xs = round_act(xf / sqrt(mean(xf^2) + eps) * gain), xf in LDS (complete: the caller has
// synchronised); cap: optional copy in activation storage.  A thread takes 4 consecutive
// elements per pass, which are 4 consecutive floats of the swizzled input too, so the reads,
// the gains and the writes are float4 and the serial chain stays short.
template <int VEC>
__device__ __forceinline__ void norm_lds(const float* xf, const float4 (&gn)[kNormV], int D, float eps, int act,
                                         float* xs, void* cap, float* red) {
  float4 xv[kNormV];
#pragma unroll
  for (int k = 0; k < kNormV; k++) {   // all reads first, unconditionally (a clamped index)
    const int i = 4 * ((int)threadIdx.x + k * PT);
    xv[k] = *(const float4*)(xf + (i < D ? i : 0));
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormV; k++) {
    const float4 v = xv[k];
    const float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    ss += 4 * ((int)threadIdx.x + k * PT) < D ? q : 0.f;
  }
  ss = wg_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  zero_tail<VEC>(D, xs);
#pragma unroll
  for (int k = 0; k < kNormV; k++) {
    const int i = 4 * ((int)threadIdx.x + k * PT);
    if (i < D) {
      const float4 g = gn[k], x = xv[k];
      const float4 v = make_float4(round_act(x.x * r * g.x, act), round_act(x.y * r * g.y, act),
                                   round_act(x.z * r * g.z, act), round_act(x.w * r * g.w, act));
      if (cap) {
        store_act(cap, i, v.x, act);
        store_act(cap, i + 1, v.y, act);
        store_act(cap, i + 2, v.z, act);
        store_act(cap, i + 3, v.w, act);
      }
      *(float4*)(xs + swz<VEC>(i)) = v;
    }
  }
  // the gains were read above only where i < D; this unconditional read ends their loads on
  // every path (see settle())
#pragma unroll
  for (int k = 0; k < kNormV; k++) settle(gn[k]);
}

__device__ __forceinline__ void load_plain_f32(const void* src, int n, float* dst) {
  for (int i = threadIdx.x; i < n; i += PT) dst[i] = ((const float*)src)[i];
}

// ---------------------------------------------------------------------------------------
// split-K GQA attention items
//
// An item (kv head j, chunk c) attends the G query heads that share kv head j to
// positions [c*ct, min((c+1)*ct, pos+1)) in 64-position tiles, with an online softmax
// across tiles, and leaves an unnormalised partial (acc, running max m, running sum l) per
// head (the GQA decode rule of the Qwen3-8B engine article, 4.4.2: each K/V row is read
// once for the whole query group).  A tile's K and V rows are loaded into registers ahead
// of use, 16-byte vectors spread over the workgroup: an item's first tile before the wait
// for its q, each later tile while the previous one is computed.  The block-table row sits
// in LDS, so no KV load waits on another load.
// ---------------------------------------------------------------------------------------

template <int KVFMT> struct KvEB { static constexpr int EB = KVFMT == KV_F32 ? 4 : (KVFMT == KV_BF16 ? 2 : 1); };
constexpr int kAttnOut = 4;    // outputs per thread: G*hd <= 2048 over PT threads

// One tile (64 rows x hd*EB bytes, hd <= 128) of K and of V in registers: EB 16-byte
// vectors per thread and matrix.
template <int KVFMT>
struct KvRegs {
  static constexpr int NV = KvEB<KVFMT>::EB * 64 * 128 / 16 / PT;
  uint4 k[NV];
  uint4 v[NV];
  float ks, vs;   // int8: scales of tile row threadIdx.x
};

__device__ __forceinline__ size_t kv_row(const Dims& d, const int* bt_s, int j, int t) {
  const int lb = t / d.bs;
  return ((size_t)bt_s[lb] * d.Hkv + j) * d.bs + (t - lb * d.bs);
}

// issues the loads of tile rows [t0, t0 + n) of kv head j
template <int KVFMT>
__device__ __forceinline__ void kv_issue(const Dims& d, const KvLayer& kv, const int* bt_s, int j, int t0, int n,
                                         KvRegs<KVFMT>& r) {
  constexpr int EB = KvEB<KVFMT>::EB;
  const int vpr = d.hd * EB / 16;
#pragma unroll
  for (int k = 0; k < KvRegs<KVFMT>::NV; k++) {
    const int v = (int)threadIdx.x + k * PT;
    r.k[k] = r.v[k] = make_uint4(0u, 0u, 0u, 0u);
    if (v < n * vpr) {
      const int tl = v / vpr, cc = v - tl * vpr;
      const size_t off = kv_row(d, bt_s, j, t0 + tl) * d.hd * EB + (size_t)cc * 16;
      r.k[k] = gload<uint4>((const uint8_t*)kv.k + off);
      r.v[k] = gload<uint4>((const uint8_t*)kv.v + off);
    }
  }
  if constexpr (KVFMT == KV_I8) {
    r.ks = r.vs = 0.f;
    if ((int)threadIdx.x < n) {
      const size_t row = kv_row(d, bt_s, j, t0 + threadIdx.x);
      r.ks = f16_to_f32(gload<uint16_t>(kv.ks + row));
      r.vs = f16_to_f32(gload<uint16_t>(kv.vs + row));
    }
  }
}

// KV tile rows in LDS are padded to hd + 4 floats: lane t reading row t as float4s then
// touches every bank once per 16 lanes.
__host__ __device__ inline int kv_ld(int hd) { return hd + 4; }

// Decodes the registers of tile rows [t0, t0 + n) into LDS tiles tk, tv [64][hd+4]; row pos
// (the new position) comes from new_s [2][hd] instead; rows [n, 64) of tv are zeroed (their
// probabilities are 0, and 0 times a stale non-finite value would not be).  int8: row
// scales in ks_s, vs_s.
template <int KVFMT>
__device__ __forceinline__ void kv_store(const Dims& d, const KvRegs<KVFMT>& r, int t0, int n, int pos,
                                         const float* new_s, const float* ks_s, const float* vs_s, float* tk,
                                         float* tv) {
  constexpr int EB = KvEB<KVFMT>::EB;
  constexpr int PER = 16 / EB;   // elements per vector
  const int hd = d.hd, ldk = kv_ld(hd), vpr = hd * EB / 16;
#pragma unroll
  for (int k = 0; k < KvRegs<KVFMT>::NV; k++) {
    const int v = (int)threadIdx.x + k * PT;
    if (v < kAttnTile * vpr) {
      const int tl = v / vpr, e0 = (v - tl * vpr) * PER;
      float4* dk = (float4*)(tk + tl * ldk + e0);
      float4* dv = (float4*)(tv + tl * ldk + e0);
      float fk[PER], fv[PER];
      if (tl >= n) {
#pragma unroll
        for (int e = 0; e < PER; e++) fk[e] = fv[e] = 0.f;
      } else if (t0 + tl == pos) {
#pragma unroll
        for (int e = 0; e < PER; e++) { fk[e] = new_s[e0 + e]; fv[e] = new_s[hd + e0 + e]; }
      } else {
        const uint32_t uk[4] = {r.k[k].x, r.k[k].y, r.k[k].z, r.k[k].w};
        const uint32_t uv[4] = {r.v[k].x, r.v[k].y, r.v[k].z, r.v[k].w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          if constexpr (KVFMT == KV_F32) {
            fk[q] = __uint_as_float(uk[q]);
            fv[q] = __uint_as_float(uv[q]);
          } else if constexpr (KVFMT == KV_BF16) {
            fk[2 * q] = __uint_as_float(uk[q] << 16);
            fk[2 * q + 1] = __uint_as_float(uk[q] & 0xffff0000u);
            fv[2 * q] = __uint_as_float(uv[q] << 16);
            fv[2 * q + 1] = __uint_as_float(uv[q] & 0xffff0000u);
          } else {
            const float sk = ks_s[tl], sv = vs_s[tl];
#pragma unroll
            for (int b = 0; b < 4; b++) {
              fk[4 * q + b] = sext8(uk[q], b) * sk;
              fv[4 * q + b] = sext8(uv[q], b) * sv;
            }
          }
        }
      }
#pragma unroll
      for (int e = 0; e < PER / 4; e++) {
        dk[e] = make_float4(fk[4 * e], fk[4 * e + 1], fk[4 * e + 2], fk[4 * e + 3]);
        dv[e] = make_float4(fv[4 * e], fv[4 * e + 1], fv[4 * e + 2], fv[4 * e + 3]);
      }
    }
  }
  // the tile's loads were read above only for rows below n
#pragma unroll
  for (int k = 0; k < KvRegs<KVFMT>::NV; k++) {
    settle(r.k[k]);
    settle(r.v[k]);
  }
  if constexpr (KVFMT == KV_I8) {
    settle(r.ks);
    settle(r.vs);
  }
}

// partial products of the MFMA tile, per group of 4 heads: scores [8 waves][64 lanes][4],
// then P V [4 row quarters][2 halves][64][4]
__host__ __device__ inline size_t attn_red_floats(int G) { return (size_t)(G + 3) / 4 * (4 * 2 * 64 * 4); }

__host__ __device__ inline size_t attn_p_floats(int G, int hd) {
  return (size_t)G * hd + 2 * (size_t)kAttnTile * kv_ld(hd) + (size_t)G * kAttnTile + (size_t)G * 4 +
         2 * (size_t)hd + 2 * (size_t)kAttnTile + PW + attn_red_floats(G);
}

// One item; all threads call it.  kr holds the item's first tile (issued by the caller).
// qg, kn, vn: the group's queries and head j's new key/value (LDS); sm: attn_p_floats of LDS.
template <int KVFMT, typename Put>
__device__ __forceinline__ void attn_item_p(const Dims& d, const KvLayer& kv, const int* bt_s, int j, int c,
                                            int ct, int nch, int pos, int pos_blk, const float* qg, const float* kn,
                                            const float* vn, float* sm, KvRegs<KVFMT>& kr, Put put) {
  const int hd = d.hd, G = d.G, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_begin = c * ct, t_end = min(pos + 1, t_begin + ct), ldk = kv_ld(hd);
  float* q_s = sm;                          // [G][hd], pre-scaled by 1/sqrt(hd)
  float* tk = q_s + G * hd;                 // [64][hd+4]
  float* tv = tk + kAttnTile * ldk;         // [64][hd+4]
  float* p_s = tv + kAttnTile * ldk;        // [G][64]: scores, then probabilities
  float* st_s = p_s + G * kAttnTile;        // [G][4]: running max, running sum, rescale
  float* new_s = st_s + G * 4;              // [2][hd]: stored (decoded) new k, v
  float* ks_s = new_s + 2 * hd;             // [64] int8 row scales of K
  float* vs_s = ks_s + kAttnTile;           // [64] and of V
  float* red = vs_s + kAttnTile;            // [PW]
  float* mred = red + PW;                   // [attn_red_floats(G)] MFMA partials

  const float scale = 1.0f / sqrtf((float)hd);
  for (int e = tid; e < G * hd; e += PT) q_s[e] = qg[e] * scale;
  for (int g = tid; g < G; g += PT) { st_s[g * 4] = -INFINITY; st_s[g * 4 + 1] = 0.f; }
  if (pos >= t_begin && pos < t_end) {   // this item appends the new token of head j
    const int off = pos - (pos / d.bs) * d.bs;
    kv_append<KVFMT>(kv, ((size_t)pos_blk * d.Hkv + j) * d.bs + off, hd, kn, vn, new_s, red);
  }
  float acc[kAttnOut];
#pragma unroll
  for (int k = 0; k < kAttnOut; k++) acc[k] = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += kAttnTile) {
    const int n = min(kAttnTile, t_end - t0);
    if constexpr (KVFMT == KV_I8) {
      if (tid < n) { ks_s[tid] = kr.ks; vs_s[tid] = kr.vs; }
    }
    __syncthreads();   // new_s, q_s, scales; the previous tile's readers are done
    kv_store<KVFMT>(d, kr, t0, n, pos, new_s, ks_s, vs_s, tk, tv);
    if (t0 + kAttnTile < t_end) kv_issue<KVFMT>(d, kv, bt_s, j, t0 + kAttnTile, min(kAttnTile, t_end - t0 - kAttnTile), kr);
    __syncthreads();
    // Scores on the matrix cores, heads in groups of 4: one v_mfma_f32_4x4x1f32 multiplies,
    // for one head dimension d, the 64 tile rows (A: lane t holds k[t][d]) by 4 queries (B:
    // lane t holds q[4 hg + t % 4][d], 0 past the last head); lane t then holds
    // S[4(t/4) + r][4 hg + t % 4] in its r-th result.  The waves each run a share of the head
    // dimensions; their partial results meet in LDS.
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int nhg = (G + 3) >> 2;
    // the head dimensions split over all 8 waves (4 when hd is not a multiple of 32), which
    // halves each wave's chain of dependent products
    const int sw = hd % 32 == 0 ? PW : 4;
    if (wave < sw) {
      const int d0 = wave * (hd / sw), d1 = d0 + hd / sw;
      const float* kr_ = tk + lane * ldk;
      for (int hg = 0; hg < nhg; hg++) {
        const int gq = 4 * hg + (lane & 3);
        const bool qok = gq < G;
        const float* qr_ = q_s + (qok ? gq : 0) * hd;
        f4v sacc = {0.f, 0.f, 0.f, 0.f};
        for (int dd = d0; dd < d1; dd += 4) {
          const float4 ka = *(const float4*)(kr_ + dd);
          const float4 q4 = *(const float4*)(qr_ + dd);
          const float4 qa = qok ? q4 : make_float4(0.f, 0.f, 0.f, 0.f);
          sacc = __builtin_amdgcn_mfma_f32_4x4x1f32(ka.x, qa.x, sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_4x4x1f32(ka.y, qa.y, sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_4x4x1f32(ka.z, qa.z, sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_4x4x1f32(ka.w, qa.w, sacc, 0, 0, 0);
        }
        *(float4*)(mred + ((hg * PW + wave) * 64 + lane) * 4) = make_float4(sacc[0], sacc[1], sacc[2], sacc[3]);
      }
    }
    __syncthreads();
    // softmax: wave w takes heads w, w + PW, ...; lane t is tile row t, its score the sum of
    // the 4 partials
    for (int g = wave; g < G; g += PW) {
      const float* mr = mred + (g >> 2) * (PW * 256);
      const int src = (4 * (lane >> 2) + (g & 3)) * 4 + (lane & 3);
      float raw = ((mr[src] + mr[256 + src]) + (mr[512 + src] + mr[768 + src]));
      if (sw == PW) raw += (mr[1024 + src] + mr[1280 + src]) + (mr[1536 + src] + mr[1792 + src]);
      const float sc = lane < n ? raw : -INFINITY;
      const float mt = wave_top(sc);
      const float mo = st_s[g * 4], lo = st_s[g * 4 + 1];
      const float mn = fmaxf(mo, mt);
      const float pr = lane < n ? expf(sc - mn) : 0.f;
      const float ps = wave_total(pr);
      p_s[g * kAttnTile + lane] = pr;
      if (lane == 0) {
        const float al = expf(mo - mn);
        st_s[g * 4] = mn;
        st_s[g * 4 + 1] = lo * al + ps;
        st_s[g * 4 + 2] = al;
      }
    }
    __syncthreads();
    // P V on the matrix cores, per group of 4 heads: one MFMA per tile row t multiplies 64
    // head dimensions (A: lane holds v[t][64 half + lane]) by 4 probabilities (B: lane holds
    // p[4 hg + lane % 4][t]); lane l then holds O[64 half + 4(l/4) + r][4 hg + l % 4].  Wave w
    // takes half w % 2 and rows 16 (w/2) .. +16; the 4 row quarters meet in LDS.
    {
      const int half = wave & 1, qt = wave >> 1;
      const int col = 64 * half + lane;
      const bool in = col < hd;
      for (int hg = 0; hg < nhg; hg++) {
        const int gp = 4 * hg + (lane & 3);
        const bool pok = gp < G;
        f4v oacc = {0.f, 0.f, 0.f, 0.f};
        if (64 * half < hd) {
          const float* pq = p_s + (pok ? gp : 0) * kAttnTile + 16 * qt;
          for (int t4 = 0; t4 < 16; t4 += 4) {
            const float4 p4 = *(const float4*)(pq + t4);
            const float4 pp = pok ? p4 : make_float4(0.f, 0.f, 0.f, 0.f);
            const float* vr = tv + (16 * qt + t4) * ldk + (in ? col : 0);
            oacc = __builtin_amdgcn_mfma_f32_4x4x1f32(in ? vr[0] : 0.f, pp.x, oacc, 0, 0, 0);
            oacc = __builtin_amdgcn_mfma_f32_4x4x1f32(in ? vr[ldk] : 0.f, pp.y, oacc, 0, 0, 0);
            oacc = __builtin_amdgcn_mfma_f32_4x4x1f32(in ? vr[2 * ldk] : 0.f, pp.z, oacc, 0, 0, 0);
            oacc = __builtin_amdgcn_mfma_f32_4x4x1f32(in ? vr[3 * ldk] : 0.f, pp.w, oacc, 0, 0, 0);
          }
        }
        if (hg == 0) __syncthreads();   // the score partials are no longer read
        *(float4*)(mred + (hg * 2048) + ((qt * 2 + half) * 64 + lane) * 4) =
            make_float4(oacc[0], oacc[1], oacc[2], oacc[3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kAttnOut; k++) {
      const int oi = tid + k * PT;
      if (oi < G * hd) {
        const int g = oi / hd, i = oi - g * hd;
        const int hf = i >> 6, ii = i & 63;
        const float* mr = mred + (g >> 2) * 2048;
        const int src = (hf * 64 + 4 * (ii >> 2) + (g & 3)) * 4 + (ii & 3);
        const float sum = mr[src] + mr[512 + src] + mr[1024 + src] + mr[1536 + src];
        acc[k] = acc[k] * st_s[g * 4 + 2] + sum;
      }
    }
  }
  __syncthreads();
  const int cs = hd + 2;
#pragma unroll
  for (int k = 0; k < kAttnOut; k++) {
    const int oi = tid + k * PT;
    if (oi < G * hd) {
      const int g = oi / hd, i = oi - g * hd;
      put(((size_t)(j * G + g) * nch + c) * cs + i, acc[k]);   // partial layout [Hq][nch][hd+2]
    }
  }
  for (int g = tid; g < G; g += PT) {
    const size_t P = ((size_t)(j * G + g) * nch + c) * cs;
    put(P + hd, st_s[g * 4]);
    put(P + hd + 1, st_s[g * 4 + 1]);
  }
}

// ---------------------------------------------------------------------------------------
// the step kernel
// ---------------------------------------------------------------------------------------

// The layer table is read through the constant address space: the host writes it before the
// launch and the kernel never does, so its (wave-uniform) fields come in by scalar loads,
// which wait on their own counter.  Read by vector loads they would be the youngest loads in
// flight when a projection starts, and waiting for them there would drain the weight groups
// issued before them.
typedef const __attribute__((address_space(4))) PLayer CPLayer;
typedef const __attribute__((address_space(4))) MatDev CMatDev;

__device__ __forceinline__ MatDev cmat(CMatDev* m) {
  MatDev r;
  r.w = m->w;
  r.s = m->s;
  r.rows = m->rows;
  r.cols = m->cols;
  return r;
}

__device__ __forceinline__ KvLayer ckv(CPLayer* t) {
  KvLayer r;
  r.k = t->kv.k;
  r.v = t->kv.v;
  r.ks = t->kv.ks;
  r.vs = t->kv.vs;
  return r;
}

// Phases of the flat loop: four per layer, then the LM head.
enum { PH_QKV = 0, PH_O = 1, PH_GU = 2, PH_DOWN = 3, PH_HEAD = 4 };

// The step as one flat loop over phases, so that the weight streaming, the input staging,
// the epilogues and the attention each exist once in the binary: the loop body is executed
// every layer, and a body larger than the instruction cache (64 KB) is refetched from L2
// every layer, which stalls the weight stream far more than the fetch itself costs.
// PROBE: the debug-probe variant (every projection's input from the inject record, outputs
// copied to the capture record).  A separate instantiation, so that the normal step kernel
// carries none of that code.
// ACTT: the activation type as a constant (ACT_F32, ACT_BF16), or -1 to read it from the
// dimensions (the probe variants).
template <int WFMT, int KVFMT, bool PROBE, int ACTT, int HD>
__global__ __launch_bounds__(PT) void k_step(PersistArgs a) {
  constexpr int VEC = PVec<WFMT>::VEC;
  // Dynamic LDS is placed after the static variables below; without the alignment it would
  // start at their (unaligned) end, and every float4 access to it would be split.
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ __attribute__((aligned(16))) float red[PW];
  __shared__ int sfail;
  __shared__ float wbest[PW];
  __shared__ int widx[PW];
  __shared__ float rope_s[128];       // cos | sin of this step's token position (hd <= 128)
  // The common attention shape as constants where the instantiation names it (HD > 0: head
  // size HD, 4 query heads per KV head, KV blocks of 16 positions): the attention item's and
  // the merge's divisions, strides, loop and split counts by them then fold away.
  Dims dv = a.d;
  if constexpr (HD > 0) {
    dv.hd = HD;
    dv.G = kFixedG;
    dv.bs = kFixedBs;
  }
  const Dims& d = dv;
  const int g = blockIdx.x, nwg = gridDim.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  constexpr bool probe = PROBE;
  const int act = ACTT >= 0 ? ACTT : a.d.act;
  const StepDesc* desc = a.desc;
  int32_t* err = a.err;
  float* xs = smem;                   // swizzled input vector of the current projection
  float* xf = smem + a.xs_floats;     // residual stream [D], plain order
  int* bt_s = (int*)(xf + d.D);       // the sequence's block-table row [max_blocks]
  float* ores = (float*)(bt_s + d.max_blocks);   // finished dot products of this workgroup's rows
  const int G = d.G, hd = d.hd, cs = hd + 2;
  auto T = [&](int l, int kind) { return a.epoch + (uint32_t)(l * kTagsPerLayer + kind); };
  auto inj = [&](int l, size_t off) { return (const void*)(a.inject + (size_t)l * a.po.record + off); };
  auto cap = [&](int l, size_t off) { return (void*)(a.capture + (size_t)l * a.po.record + off); };

  if (tid == 0) sfail = 0;
  int tok = desc->tokens[0];
  if (tok < 0 || tok >= d.V) {
    if (tid == 0) __hip_atomic_fetch_or(err, kErrToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = 0;
  }
  // pos: the new entry's cache index (attention covers entries 0..pos); rpos: the token's
  // position in the text, which RoPE rotates by (they differ once a KV budget has evicted)
  const int pos = desc->pos[0], slot = desc->slot[0], pos_blk = desc->pos_block[0], rpos = desc->rpos[0];
  const int score_from = desc->score_from[0];
  const bool do_head = desc->do_head != 0;

  WBuf pre, preb;   // weight groups in flight (A, B of gemv_phase)
  float4 gn[kNormV];
  CPLayer* layers = (CPLayer*)a.layers;
  const void* dummy = layers[0].qkv.w;
  PPhase ph = make_phase<WFMT>(cmat(&layers[0].qkv), g, nwg);
  ICur ic{0, 0, ph.jb};   // issue cursor of phase ph (then of the phase after it)
  issue_group<WFMT>(ph, ic, pre);
  issue_group<WFMT>(ph, ic, preb);
  // the sequence's block-table row in LDS with this step's entries applied; workgroup 0
  // also stores those entries in the table for later steps
  {
    const int32_t* btrow = a.bt + (size_t)slot * d.max_blocks;
    for (int b = tid; b < d.max_blocks; b += PT) {
      int v = btrow[b];
      for (int u = 0; u < desc->n_updates; u++)
        if (desc->upd[u][0] == slot && desc->upd[u][1] == b) v = desc->upd[u][2];
      bt_s[b] = v;
    }
    if (g == 0)
      for (int u = tid; u < desc->n_updates; u += PT)
        a.bt[(size_t)desc->upd[u][0] * d.max_blocks + desc->upd[u][1]] = desc->upd[u][2];
  }
  for (int i = tid; i < (hd >> 1); i += PT) {
    rope_s[i] = gload<float>(a.rope_cos + (size_t)rpos * (hd >> 1) + i);
    rope_s[(hd >> 1) + i] = gload<float>(a.rope_sin + (size_t)rpos * (hd >> 1) + i);
  }
  // layer-0 input: the token's embedding row, dequantised by every workgroup
  if (!probe)
    for (int i = tid; i < d.D; i += PT) xf[i] = deq_elem(a.emb, d.wfmt, tok, i);
  __syncthreads();

  PEpi e{};
  e.rope = rope_s;
  e.xf = xf;
  e.logits = a.logits;
  e.logits_out = desc->logits_out;
  e.best = -INFINITY;
  e.best_idx = INT_MAX;
  e.act = act;
  const int nph = 4 * d.L + (do_head ? 1 : 0);
#pragma clang loop unroll(disable)
  for (int q = 0; q < nph; q++) {
    const int l = q >> 2;                        // layer (d.L for the head)
    const int k = q == 4 * d.L ? PH_HEAD : (q & 3);
    CPLayer* Ly = layers + (l < d.L ? l : d.L - 1);

    // The phase after this one (its first weight groups are issued at the end of this
    // projection; after QKV none: the O projection's weights are issued after attention,
    // since otherwise their registers would stay live across the attention items).  Worked
    // out here, while the input below is still on its way, not between the input and the
    // projection.
    PPhase nx;
    {
      // the matrix is picked first, so that the descriptor's arithmetic has one copy
      MatDev nm;
      bool has = true;
      if (k == PH_O) nm = cmat(&Ly->gu);
      else if (k == PH_GU) nm = cmat(&Ly->down);
      else if (k == PH_DOWN && l + 1 < d.L) nm = cmat(&layers[l + 1].qkv);
      else if (k == PH_DOWN && do_head) nm = a.head;
      else has = false;
      nx = has ? make_phase<WFMT>(nm, g, nwg) : empty_phase(dummy);
    }

    // ---- input of the projection ----
    // A probe step takes every wait of a normal step (the waits are what order the reuse of
    // the hand-off buffers), then replaces the input it received with the injected one.
    if (k == PH_QKV || k == PH_GU || k == PH_HEAD) {
      // RMSNorm of the residual stream: layer 0's QKV input is the embedding row (in xf)
      gain_issue(k == PH_QKV ? Ly->attn_norm : (k == PH_GU ? Ly->ffn_norm : a.final_norm), d.D, gn);
      if (q > 0) {
        const uint64_t* src = k == PH_GU ? a.t_xm : a.t_xo;
        gather(d.D, k == PH_GU ? T(l, TG_XM) : T(l - 1, TG_XO), err, &sfail, [&](int i) { return src + i; },
               [&](int i, float v) { xf[i] = v; });
        __syncthreads();
        if (sfail) return;
      }
      // Every path reads the gains (gn): a load whose register is never read stays pending
      // into the projection below, and waiting for it there would also wait for the weight
      // groups in flight.
      if (probe) {
        const int lp = k == PH_HEAD ? d.L - 1 : l;
        load_plain_f32(inj(lp, k == PH_QKV ? a.po.x_in : (k == PH_GU ? a.po.x_mid : a.po.x_out)), d.D, xf);
        __syncthreads();
        const bool keep = k != PH_HEAD && g == 0;   // workgroup 0 records the normalised input
        norm_lds<VEC>(xf, gn, d.D, d.eps, act, xs, keep ? cap(l, k == PH_QKV ? a.po.xn : a.po.xn2) : nullptr,
                      red);
        if (k != PH_HEAD) {
          __syncthreads();
          stage_plain<VEC>(inj(l, k == PH_QKV ? a.po.xn : a.po.xn2), act, d.D, xs);
        }
      } else {
        norm_lds<VEC>(xf, gn, d.D, d.eps, act, xs, nullptr, red);
      }
    } else {
      // the attention output (O) or the SwiGLU output (down), as produced
      const bool is_o = k == PH_O;
      if (act == ACT_BF16) {   // two values per word
        if (is_o) {
          // (4 words per thread: one round up to q_dim 4096)
          stage_tagged_pairs<VEC, 4>(a.t_o, T(l, TG_O), d.q_dim >> 1, d.q_dim, xs, err, &sfail,
                                  [](int w, int& i0, int& i1) { i0 = 2 * w; i1 = 2 * w + 1; });
        } else {   // three values per word, 16-bit tag
          const int hs = h_words_per_wg(d.F, nwg);
          // Word w comes from workgroup w / hs, found by a multiply with 2^32 / hs rounded up
          // (64-bit: it is 2^32 for hs = 1; exact while w * hs < 2^32), and workgroup gp owns
          // fq + (gp < fr) SwiGLU outputs: no integer division per word on the way in.
          const uint64_t hs_inv = 0xffffffffull / (uint64_t)hs + 1ull;
          const int fq = d.F / nwg, fr = d.F - fq * nwg;
          zero_tail<VEC>(d.F, xs);
          gather_words<8, 48>(nwg * hs, T(l, TG_H) & 0xffffu, err, &sfail, [&](int w) { return a.t_h + w; },
                              [&](int w, uint64_t word) {
                                const int gp = (int)(((uint64_t)(uint32_t)w * hs_inv) >> 32), u = w - gp * hs;
                                const int np = fq + (gp < fr ? 1 : 0);
#pragma unroll
                                for (int hh = 0; hh < 3; hh++) {
                                  const int t = 3 * u + hh;
                                  if (t < np)
                                    xs[swz<VEC>(gp + nwg * t)] = __uint_as_float((uint32_t)(word >> (16 * hh)) << 16);
                                }
                              });
        }
      } else {
        stage_tagged<VEC>(is_o ? a.t_o : a.t_h, T(l, is_o ? TG_O : TG_H), is_o ? d.q_dim : d.F, xs, err, &sfail);
      }
      __syncthreads();
      if (sfail) return;
      if (probe) stage_plain<VEC>(inj(l, is_o ? a.po.o : a.po.h), act, is_o ? d.q_dim : d.F, xs);
    }
    __syncthreads();

    // ---- the projection; the next one's first weight groups are issued at its end ----
#pragma unroll
    for (int i = 0; i < kNormV; i++) settle(gn[i]);   // no gain load may reach the stream
    // The loop ends with loads of nothing (pad groups) in A and B; the next phase's first
    // groups are issued after the epilogue below.  A CU's memory instructions issue in order,
    // so issued before the epilogue they would hold up its stores, which publish what every
    // other workgroup waits for, until their own data had come in.
    gemv_phase<WFMT>(ph, pre, preb, xs, ores, ic);
    __syncthreads();

    // ---- epilogue ----
    if (k == PH_QKV) {
      e.tag = T(l, TG_QKV);
      e.tq = a.t_q;
      e.tk = a.t_k;
      e.tv = a.t_v;
      e.cq = probe ? (float*)cap(l, a.po.q) : nullptr;
      e.ck = probe ? (float*)cap(l, a.po.k) : nullptr;
      e.cv = probe ? (float*)cap(l, a.po.v) : nullptr;
      phase_epilogue<EPI_QKV>(d, ph, ores, e);
    } else if (k == PH_O || k == PH_DOWN) {
      const bool is_o = k == PH_O;
      e.tag = T(l, is_o ? TG_XM : TG_XO);
      e.tout = is_o ? a.t_xm : a.t_xo;
      e.cout = probe ? (float*)cap(l, is_o ? a.po.x_mid : a.po.x_out) : nullptr;
      phase_epilogue<EPI_RESID>(d, ph, ores, e);
    } else if (k == PH_GU) {
      e.tag = T(l, TG_H);
      e.th = a.t_h;
      e.hs = h_words_per_wg(d.F, nwg);
      e.ch = probe ? cap(l, a.po.h) : nullptr;
      phase_epilogue<EPI_SWIGLU>(d, ph, ores, e);
    } else {
      phase_epilogue<EPI_LOGITS>(d, ph, ores, e);
    }
    // the next phase's first weight groups (none after QKV, see above)
    if (k != PH_QKV && k != PH_HEAD) {
      ic = ICur{0, 0, nx.jb};
      issue_group<WFMT>(nx, ic, pre);
      issue_group<WFMT>(nx, ic, preb);
    }

    if (k == PH_QKV) {
      // ---- KV append + split-K attention ----
      const int nv = (pos + a.ct) / a.ct;
      const int items = d.Hkv * nv;
      const uint32_t tpart = T(l, TG_PART);
      float* ain = smem + attn_p_floats(G, hd);   // [G*hd] q group | [hd] k | [hd] v
      const int nin = G * hd + 2 * hd;
      KvRegs<KVFMT> kr;
      const KvLayer lkv = ckv(Ly);
      for (int it = g; it < items; it += nwg) {
        const int j = it / nv, c = it - j * nv, t0 = c * a.ct;
        // the item's first KV tile is on its way while q, k, v are awaited
        kv_issue<KVFMT>(d, lkv, bt_s, j, t0, min(kAttnTile, min(pos + 1, t0 + a.ct) - t0), kr);
        __syncthreads();
        gather<2>(nin, T(l, TG_QKV), err, &sfail,
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
        // a scored layer keeps its queries for the score sums (the head group's first chunk)
        if (l >= score_from && c == 0)
          for (int t = tid; t < G * hd; t += PT) a.score_q[(size_t)l * d.q_dim + j * G * hd + t] = ain[t];
        uint64_t* tp = a.t_part;
        attn_item_p<KVFMT>(d, lkv, bt_s, j, c, a.ct, a.nch, pos, pos_blk, ain, ain + G * hd, ain + G * hd + hd,
                           smem, kr, [tp, tpart](size_t i, float v) { put_tag(tp + i, tpart, v); });
      }
      // the O projection's first weight groups, on their way during the merge (a merging
      // workgroup would otherwise be the last to start O, and every workgroup waits for its rows)
      nx = make_phase<WFMT>(cmat(&Ly->o), g, nwg);
      ic = ICur{0, 0, nx.jb};
      issue_group<WFMT>(nx, ic, pre);
      issue_group<WFMT>(nx, ic, preb);
      // Merge: q head h = j G + gh is combined by the workgroup that ran chunk
      // nv - 1 - (gh mod nv) of head group j, after all of its own items (so no workgroup waits
      // on one that is itself waiting), and the G heads of a group merge in parallel.  Output
      // dimension i gets PT / hd threads, each over every (PT / hd)-th chunk.
      for (int it = g; it < items; it += nwg) {
        const int j = it / nv, c = it - j * nv;
        for (int gh = nv - 1 - c; gh < G; gh += nv) {
          const int h = j * G + gh;
          const uint64_t* PH = a.t_part + (size_t)h * a.nch * cs;   // chunk cc at PH + cc cs
          const int NP = PT / hd, i = tid % hd, part = tid / hd;
          float* ml = smem;                   // [nv][2]: (m, l), then (weight, l)
          float* psum = smem + 2 * nv;        // [NP][hd] partial sums
          float* Lsum = psum + NP * hd;       // [1]
          constexpr int MB = 8;
          __syncthreads();
          gather<1>(2 * nv, tpart, err, &sfail, [&](int t) { return PH + (size_t)(t >> 1) * cs + hd + (t & 1); },
                 [&](int t, float v) { ml[t] = v; });
          __syncthreads();
          if (sfail) return;
          if (wave == 0) {   // weights e^(m_c - M) and their l sum
            float M = -INFINITY;
            for (int cc = lane; cc < nv; cc += 64) M = fmaxf(M, ml[cc * 2]);
            M = wave_top(M);
            float L = 0.f;
            for (int cc = lane; cc < nv; cc += 64) {
              const float wt = expf(ml[cc * 2] - M);
              ml[cc * 2] = wt;
              L += wt * ml[cc * 2 + 1];
            }
            L = wave_total(L);
            if (lane == 0) {
              Lsum[0] = L;
              if (l >= score_from) {   // a scored layer: the head's softmax max and sum
                a.score_stat[((size_t)l * d.Hq + h) * 2] = M;
                a.score_stat[((size_t)l * d.Hq + h) * 2 + 1] = L;
              }
            }
          }
          __syncthreads();
          float acc = 0.f;
          for (int c0 = 0; c0 < nv; c0 += MB * NP) {
            uint64_t w[MB];
#pragma unroll
            for (int u = 0; u < MB; u++) {
              const int cc = c0 + part + u * NP;
              w[u] = part < NP && cc < nv ? get_word(PH + (size_t)cc * cs + i) : (uint64_t)tpart << 32;
            }
            await_tags<MB>(w, tpart, err, &sfail,
                           [&](int u) { return get_word(PH + (size_t)(c0 + part + u * NP) * cs + i); });
#pragma unroll
            for (int u = 0; u < MB; u++) {
              const int cc = c0 + part + u * NP;
              if (part < NP && cc < nv) acc += ml[cc * 2] * __uint_as_float((uint32_t)w[u]);
            }
#pragma unroll
            for (int u = 0; u < MB; u++) settle(w[u]);
          }
          if (part < NP) psum[part * hd + i] = acc;
          __syncthreads();
          if (sfail) return;
          if (tid < hd) {
            float sum = 0.f;
            for (int pp = 0; pp < NP; pp++) sum += psum[pp * hd + tid];
            const float o = sum / Lsum[0];
            if (probe) store_act(cap(l, a.po.o), (size_t)h * hd + tid, o, act);
            if (act == ACT_BF16) {   // outputs 2w, 2w + 1 share word w (hd is even)
              const uint32_t mine = f32_to_bf16(o);
              const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1, 64);
              if ((tid & 1) == 0) put_tag(a.t_o + ((h * hd + tid) >> 1), T(l, TG_O), __uint_as_float(mine | (other << 16)));
            } else {
              put_tag(a.t_o + h * hd + tid, T(l, TG_O), o);
            }
          }
          __syncthreads();
        }
      }
      __syncthreads();
    }
    ph = nx;
  }
  if (!do_head) return;

  // ---- greedy argmax over the logits: this workgroup's winner, then workgroup 0 reduces ----
  {   // first index among equal maxima
    float b = e.best;
    int bi = e.best_idx;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(b, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > b || (ov == b && oi < bi)) { b = ov; bi = oi; }
    }
    if (lane == 0) { wbest[wave] = b; widx[wave] = bi; }
  }
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
  gather<1>(2 * nwg, thead, err, &sfail, [&](int t) { return a.t_am + t; }, [&](int t, float v) { xs[t] = v; });
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
}

// The normal step per activation type, with the attention shape of the target models fixed
// (4 query heads per KV head, KV blocks of 16, and head size 128 with either activation type
// or head size 64 with bf16 activations) or read at run time; and its probe variant: with a
// fixed shape, the same instantiation parameters as the normal step (so a probe at that
// shape checks the code the normal step runs), otherwise one variant that reads the
// activation type at run time.
template <int WFMT, int KVFMT>
const void* step_kernel(bool probe, int act, int fixed_hd) {
  if (fixed_hd == 64)
    return probe ? (const void*)k_step<WFMT, KVFMT, true, ACT_BF16, 64>
                 : (const void*)k_step<WFMT, KVFMT, false, ACT_BF16, 64>;
  const bool fixed = fixed_hd == 128;
  if (probe) {
    if (fixed)
      return act == ACT_BF16 ? (const void*)k_step<WFMT, KVFMT, true, ACT_BF16, 128>
                             : (const void*)k_step<WFMT, KVFMT, true, ACT_F32, 128>;
    return (const void*)k_step<WFMT, KVFMT, true, -1, 0>;
  }
  if (fixed)
    return act == ACT_BF16 ? (const void*)k_step<WFMT, KVFMT, false, ACT_BF16, 128>
                           : (const void*)k_step<WFMT, KVFMT, false, ACT_F32, 128>;
  return act == ACT_BF16 ? (const void*)k_step<WFMT, KVFMT, false, ACT_BF16, 0>
                         : (const void*)k_step<WFMT, KVFMT, false, ACT_F32, 0>;
}

const void* pick(const Dims& d, bool probe) {
  const int wfmt = d.wfmt, kvfmt = d.kvfmt, act = d.act;
  const int fixed = persistent_fixed_hd(d);
  if (wfmt == W_INT8_ROW) {
    if (kvfmt == KV_F32) return step_kernel<W_INT8_ROW, KV_F32>(probe, act, fixed);
    if (kvfmt == KV_BF16) return step_kernel<W_INT8_ROW, KV_BF16>(probe, act, fixed);
    return step_kernel<W_INT8_ROW, KV_I8>(probe, act, fixed);
  }
  if (wfmt == W_Q8_0) {
    if (kvfmt == KV_F32) return step_kernel<W_Q8_0, KV_F32>(probe, act, fixed);
    if (kvfmt == KV_BF16) return step_kernel<W_Q8_0, KV_BF16>(probe, act, fixed);
    return step_kernel<W_Q8_0, KV_I8>(probe, act, fixed);
  }
  if (wfmt == W_Q4_0) {
    if (kvfmt == KV_F32) return step_kernel<W_Q4_0, KV_F32>(probe, act, fixed);
    if (kvfmt == KV_BF16) return step_kernel<W_Q4_0, KV_BF16>(probe, act, fixed);
    return step_kernel<W_Q4_0, KV_I8>(probe, act, fixed);
  }
  if (kvfmt == KV_F32) return step_kernel<W_BF16, KV_F32>(probe, act, fixed);
  if (kvfmt == KV_BF16) return step_kernel<W_BF16, KV_BF16>(probe, act, fixed);
  return step_kernel<W_BF16, KV_I8>(probe, act, fixed);
}

}  // namespace

int persistent_fixed_hd(const Dims& d) {
  if (d.G != kFixedG || d.bs != kFixedBs) return 0;
  if (d.hd == 128) return 128;
  return d.hd == 64 && d.act == ACT_BF16 ? 64 : 0;
}

size_t persistent_xs_floats(const Dims& d, int nch) {
  const int vec = d.wfmt == W_BF16 ? 8 : (d.wfmt == W_Q4_0 ? 32 : 16), kstep = 64 * vec;
  int kmax = d.D > d.F ? d.D : d.F;
  if (d.q_dim > kmax) kmax = d.q_dim;
  size_t need = (size_t)(kmax + kstep - 1) / kstep * kstep;                             // projection input
  const size_t at = attn_p_floats(d.G, d.hd) + (size_t)d.G * d.hd + 2 * (size_t)d.hd;  // attention
  const size_t mg = 2 * (size_t)d.G * nch + (size_t)d.G;                                // chunk merge
  if (at > need) need = at;
  if (mg > need) need = mg;
  return (need + 3) / 4 * 4;
}

// rows one workgroup owns in the largest projection
static size_t rows_per_wg(const Dims& d, int nwg) {
  int nmax = d.qkv_rows;
  if (d.D > nmax) nmax = d.D;
  if (2 * d.F > nmax) nmax = 2 * d.F;
  if (d.V > nmax) nmax = d.V;
  const size_t pairs = ((size_t)nmax + 1) / 2;
  return 2 * ((pairs + nwg - 1) / nwg);
}

size_t persistent_smem_bytes(const Dims& d, int nch, int nwg) {
  // result slots: a projection's rows, or 2 per wave when waves share pairs
  const size_t res = rows_per_wg(d, nwg) > 2 * (size_t)PW ? rows_per_wg(d, nwg) : 2 * (size_t)PW;
  return (persistent_xs_floats(d, nch) + (size_t)d.D + (size_t)d.max_blocks + res) * sizeof(float);
}

bool persistent_supports(const Dims& d) {
  const int eb = d.kvfmt == KV_F32 ? 4 : (d.kvfmt == KV_BF16 ? 2 : 1);
  return d.D <= kNormPer * PT && d.D % 4 == 0 && d.hd <= 128 && (d.hd * eb) % 16 == 0 && d.hd % 16 == 0 &&
         (size_t)d.G * d.hd <= (size_t)kAttnOut * PT;
}

int persistent_tags_per_step(const Dims& d) { return d.L * kTagsPerLayer + 1; }

hipError_t persistent_prepare(const Dims& d, size_t smem, int* blocks_per_cu) {
  for (const bool probe : {true, false}) {
    hipError_t r = hipFuncSetAttribute(pick(d, probe),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (r != hipSuccess) return r;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, pick(d, false), PT, smem);
}

hipError_t launch_persistent(const PersistArgs& a, int nwg, size_t smem, hipStream_t st) {
  void* args[] = {(void*)&a};
  return hipLaunchCooperativeKernel(pick(a.d, a.inject != nullptr), dim3(nwg), dim3(PT),
                                    args, (unsigned)smem, st);
}

}  // namespace dtd

