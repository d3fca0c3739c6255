// dtd_sample.hip -- stochastic next-token sampling over fp32 logits on gfx950.
//
// The sampler of the pages (the nxmr.cn C17 engine article, 4.6; the smollm3.go walkthrough,
// "sampling: from logits to the next token"): temperature (0 = greedy), top-k, top-p (the
// shortest run of most probable tokens whose probability reaches p) and min-p (a probability
// floor), each on the renormalised distribution the one before it left, then a draw from a
// seeded counter-based generator.  "Most probable" orders tokens by logit, then by index.
//
// One workgroup of 1024 threads samples one row.  Nothing is sorted: every filter keeps a
// prefix of the (logit descending, index ascending) order, and such a prefix is found by a
// radix select over a 32-bit key that orders logits that way, counting tokens (top-k) or
// summing their weights (top-p) per 8-bit digit, four passes from the top digit down; ties
// at the boundary key are cut by index.  Weights are exp((l - max) / T) in fixed point
// (2^44 = the largest logit's weight), so every sum is an exact integer sum: the kept set
// and the drawn token do not depend on the order the threads add in.  The draw is inverse
// transform sampling in vocabulary order: the first kept token whose running weight exceeds
// u times the kept total, u from Philox4x64-10.
#include <math.h>
#include <stdint.h>
#include <limits.h>

#include "dtd_internal.h"

namespace dtd {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr float kFixOne = 17592186044416.0f;          // 2^44: weight of the largest logit

// ---- Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1,
// 2, 3", SC 2011): ten rounds of two 64x64->128-bit products, with the key bumped by two
// Weyl constants between rounds.  Only the first output word is used.
__device__ uint64_t philox_word0(uint64_t seed, uint64_t counter) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = counter, x1 = 0, x2 = 0, x3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    const uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
  }
  return x0;
}

// NaN logits take part as -inf (never drawn)
__device__ __forceinline__ float clean(float l) { return isnan(l) ? -INFINITY : l; }

// 32-bit key, ascending = logit descending; -0 and +0 share a key
__device__ __forceinline__ uint32_t key_of(float l) {
  uint32_t u = __float_as_uint(l);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? u : (u ^ 0x7fffffffu);
}
__device__ __forceinline__ float logit_of(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? k : (k ^ 0x7fffffffu));
}

struct Weigher {
  float m;   // the row's largest logit
  float c;   // log2(e) / T
  // fixed-point exp((l - m) / T), truncated: 2^44 at l = m, 0 below 2^-44 (e * 2^44 is exact
  // in fp32, and the conversion truncates)
  __device__ __forceinline__ uint64_t operator()(float l) const {
    const float dl = l - m;
    if (dl == 0.f) return 1ull << 44;
    if (!(dl > -INFINITY)) return 0;
    const float x = dl * c;
    if (!(x > -45.f)) return 0;
    return (uint64_t)(__builtin_amdgcn_exp2f(x) * kFixOne);
  }
};

// the kept set: keys below k, and index < i among the keys equal to k (k = 0xffffffff with
// i = INT_MAX keeps every token: cleaned keys never reach 0xffffffff)
struct Kept {
  uint32_t k;
  int i;
  __device__ __forceinline__ bool has(uint32_t key, int idx) const {
    return key < k || (key == k && idx < i);
  }
};

// ---- row iteration ------------------------------------------------------------------------
// f(x, i) for every logit x = L[i] of the row (raw: NaN included), i < V.  Each thread takes
// the row in 16-byte pieces, strided by the block, four pieces in flight; rows that are not
// 16-byte aligned go element by element, four in flight.  Each thread sees its indices in
// increasing order.
template <typename F>
__device__ __forceinline__ void for_each_logit(const float* L, int V, bool vec4, F&& f) {
  const int t = threadIdx.x;
  if (vec4) {
    const float4* L4 = reinterpret_cast<const float4*>(L);
    const int n4 = V >> 2;
    int j = t;
    for (; j + 3 * kThreads < n4; j += 4 * kThreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) v[u] = L4[j + u * kThreads];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int i = 4 * (j + u * kThreads);
        f(v[u].x, i); f(v[u].y, i + 1); f(v[u].z, i + 2); f(v[u].w, i + 3);
      }
    }
    for (; j < n4; j += kThreads) {
      const float4 v = L4[j];
      f(v.x, 4 * j); f(v.y, 4 * j + 1); f(v.z, 4 * j + 2); f(v.w, 4 * j + 3);
    }
    for (int i = 4 * n4 + t; i < V; i += kThreads) f(L[i], i);
  } else {
    int i = t;
    for (; i + 3 * kThreads < V; i += 4 * kThreads) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) v[u] = L[i + u * kThreads];
#pragma unroll
      for (int u = 0; u < 4; u++) f(v[u], i + u * kThreads);
    }
    for (; i < V; i += kThreads) f(L[i], i);
  }
}

// f(x, i) for the logits of [s0, s1) by one wave (s0 a multiple of 4 unless the segment is
// empty): 16-byte pieces strided by the wave, four in flight per lane.
template <typename F>
__device__ __forceinline__ void for_each_in_segment(const float* L, int s0, int s1, bool vec4, F&& f) {
  const int lane = threadIdx.x & 63;
  if (s0 >= s1) return;
  if (vec4) {
    const float4* L4 = reinterpret_cast<const float4*>(L);
    const int j0 = s0 >> 2, j1 = s1 >> 2;
    int j = j0 + lane;
    for (; j + 3 * 64 < j1; j += 4 * 64) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) v[u] = L4[j + u * 64];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int i = 4 * (j + u * 64);
        f(v[u].x, i); f(v[u].y, i + 1); f(v[u].z, i + 2); f(v[u].w, i + 3);
      }
    }
    for (; j < j1; j += 64) {
      const float4 v = L4[j];
      f(v.x, 4 * j); f(v.y, 4 * j + 1); f(v.z, 4 * j + 2); f(v.w, 4 * j + 3);
    }
    for (int i = 4 * j1 + lane; i < s1; i += 64) f(L[i], i);
  } else {
    for (int i = s0 + lane; i < s1; i += 64) f(L[i], i);
  }
}

// ---- block-wide helpers (1024 threads) --------------------------------------------------

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// exclusive prefix of v over the block's threads; *total gets the block sum
__device__ uint64_t block_excl_scan(uint64_t v, uint64_t* red, uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t inc = wave_incl_scan<unsigned long long>(v);
  __syncthreads();
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (int w = 0; w < kWaves; w++) {
    const uint64_t s = red[w];
    if (w < wave) before += s;
    all += s;
  }
  *total = all;
  return before + inc - v;
}

constexpr int kMaxDigit = 4096;   // buckets of the widest radix digit (12 bits)

struct Shared {
  uint32_t cnt[kMaxDigit];
  uint64_t mass[kMaxDigit];
  uint64_t red[kWaves];
  float redf[kWaves];
  int redi[kWaves];
  // results one thread finds and the block reads back
  int digit;
  uint32_t cnt_before, cnt_in;
  uint64_t mass_before, mass_in;
  int found;
  uint64_t seg_before, target, total;
  int seg;
};

// Weighted draw in vocabulary order: with T the total of w(x, i) over the row, the first index
// at which the running sum of w exceeds target(T) (target(T) < T; *total gets T).  Two
// levels: one segment per wave (a multiple of 256 long) summed with coalesced loads, then the
// segment holding the crossing split into one short run per thread.
template <typename W, typename G>
__device__ int first_crossing(const float* L, int V, bool vec4, const W& w, const G& target_of, Shared& sh,
                              uint64_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int seg_len = ((V + kWaves - 1) / kWaves + 255) / 256 * 256;
  {
    const int s0 = min(V, wave * seg_len), s1 = min(V, s0 + seg_len);
    uint64_t s = 0;
    for_each_in_segment(L, s0, s1, vec4, [&](float x, int i) { s += w(clean(x), i); });
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor((unsigned long long)s, m, 64);
    __syncthreads();
    if (lane == 0) sh.red[wave] = s;
    __syncthreads();
    if (t == 0) {
      uint64_t all = 0;
      for (int k = 0; k < kWaves; k++) all += sh.red[k];
      const uint64_t target = all ? target_of(all) : 0;
      uint64_t acc = 0;
      int g = kWaves - 1;
      for (int k = 0; k < kWaves; k++) {
        if (acc + sh.red[k] > target) { g = k; break; }
        acc += sh.red[k];
      }
      sh.seg = g;
      sh.seg_before = acc;
      sh.target = target;
      sh.total = all;
      sh.found = V - 1;
    }
    __syncthreads();
  }
  *total = sh.total;
  if (sh.total == 0) return -1;
  const int g = sh.seg;
  const uint64_t base = sh.seg_before, target = sh.target;
  const int s0 = min(V, g * seg_len), s1 = min(V, s0 + seg_len);
  const int run = (seg_len + kThreads - 1) / kThreads;
  const int r0 = min(s1, s0 + t * run), r1 = min(s1, r0 + run);
  uint64_t mine = 0;
  for (int i = r0; i < r1; i++) mine += w(clean(L[i]), i);
  uint64_t tot;
  const uint64_t before = base + block_excl_scan(mine, sh.red, &tot);
  if (mine > 0 && before <= target && target < before + mine) {
    uint64_t acc = before;
    for (int i = r0; i < r1; i++) {
      acc += w(clean(L[i]), i);
      if (acc > target) { sh.found = i; break; }
    }
  }
  __syncthreads();
  return sh.found;
}

// Radix select: the shortest prefix of the kept set (key order, then index) whose token count
// (by_mass false) or weight (true) reaches need = need_of(the kept set's total count or
// weight), 1 <= need <= that total.  Three passes over the row, digits of 12, 10 and 10 bits
// from the top: the wide first digit spreads a row's keys over many buckets (sign, exponent
// and three mantissa bits), so few lanes of a wave hit one bucket at a time.  A thread merges
// consecutive tokens of one bucket before adding them to it (a row of many equal logits then
// costs few atomics).  Count passes compute no weights.  Returns the new kept set; *mass
// gets the prefix's weight (by_mass only).
template <typename N>
__device__ Kept select_prefix(const float* L, int V, bool vec4, const Weigher& wt, Kept kept, bool by_mass,
                              const N& need_of, Shared& sh, uint64_t* mass_out) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  uint64_t lt_mass = 0, ties = 0, need = 0;
  int shift = 32;
  for (int pass = 0; pass < 3; pass++) {
    const int width = pass == 0 ? 12 : 10;
    shift -= width;
    const int nb = 1 << width;
    for (int q = t; q < nb; q += kThreads) { sh.cnt[q] = 0; sh.mass[q] = 0; }
    __syncthreads();
    int cur = -1;
    uint32_t cc = 0;
    uint64_t cm = 0;
    auto flush = [&]() {
      if (cur >= 0) {
        atomicAdd(&sh.cnt[cur], cc);
        if (cm) atomicAdd((unsigned long long*)&sh.mass[cur], (unsigned long long)cm);
      }
    };
    for_each_logit(L, V, vec4, [&](float x, int i) {
      const float l = clean(x);
      const uint32_t k = key_of(l);
      if ((k & pmask) != prefix || !kept.has(k, i)) return;
      uint64_t e = 0;
      if (by_mass) {
        e = wt(l);
        if (e == 0) return;            // weightless tokens sit after every weighted one
      }
      const int dg = (int)((k >> shift) & (uint32_t)(nb - 1));
      if (dg != cur) {
        flush();
        cur = dg;
        cc = 0;
        cm = 0;
      }
      cc++;
      cm += e;
    });
    flush();
    __syncthreads();
    // per-thread runs of q = nb / 1024 consecutive buckets (at least one), block prefix sums
    // of counts and weights, then the bucket where the running total reaches need
    const int q = nb >= kThreads ? nb / kThreads : 1;
    const int b0 = t * q;
    uint64_t tc = 0, tm = 0;
    for (int u = 0; u < q && b0 + u < nb; u++) { tc += sh.cnt[b0 + u]; tm += sh.mass[b0 + u]; }
    uint64_t call, mall;
    uint64_t cb = block_excl_scan(tc, sh.red, &call);
    __syncthreads();
    uint64_t mb = block_excl_scan(tm, sh.red, &mall);
    if (pass == 0) need = need_of(by_mass ? mall : call);
    for (int u = 0; u < q && b0 + u < nb; u++) {
      const uint64_t c = sh.cnt[b0 + u], m = sh.mass[b0 + u];
      const uint64_t before = by_mass ? mb : cb, v = by_mass ? m : c;
      if (v > 0 && before < need && need <= before + v) {
        sh.digit = b0 + u;
        sh.cnt_in = (uint32_t)c;
        sh.mass_before = mb;
        sh.cnt_before = (uint32_t)cb;
      }
      cb += c;
      mb += m;
    }
    __syncthreads();
    const int d = sh.digit;
    prefix |= (uint32_t)d << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    lt_mass += sh.mass_before;
    need -= by_mass ? sh.mass_before : (uint64_t)sh.cnt_before;
    ties = sh.cnt_in;
    __syncthreads();
  }
  // every kept token with key == prefix has the same logit and so the same weight
  const uint64_t e_tie = wt(logit_of(prefix));
  uint64_t r = need;                                   // ties to keep
  if (by_mass) r = (need + e_tie - 1) / e_tie;
  if (r > ties) r = ties;
  Kept out{prefix, 0};
  if (r == ties) {
    out.i = prefix == kept.k ? kept.i : V;
  } else {
    // the r-th kept tie in index order; the cut is just after it
    const uint32_t kk = prefix;
    auto is_tie = [&](float l, int i) -> uint64_t { return (key_of(l) == kk && kept.has(kk, i)) ? 1 : 0; };
    uint64_t tot;
    out.i = first_crossing(L, V, vec4, is_tie, [&](uint64_t) { return r - 1; }, sh, &tot) + 1;
  }
  *mass_out = lt_mass + r * e_tie;
  return out;
}

__global__ __launch_bounds__(kThreads) void k_sample(SampleArgs a) {
  __shared__ Shared sh;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const SampleRow P = a.row[b];
  const float* L = a.logits + (size_t)b * a.stride;
  const int V = a.V;
  const bool vec4 = (reinterpret_cast<uintptr_t>(L) & 15) == 0;

  // largest logit, lowest index among equal ones (NaN skipped)
  float best = -INFINITY;
  int idx = INT_MAX;
  for_each_logit(L, V, vec4, [&](float x, int i) {
    if (x > best || (idx == INT_MAX && !isnan(x))) { best = x; idx = i; }
  });
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(idx, m, 64);
    if (ob > best || (ob == best && oi < idx)) { best = ob; idx = oi; }
  }
  if (lane == 0) { sh.redf[wave] = best; sh.redi[wave] = idx; }
  __syncthreads();
  best = sh.redf[0];
  idx = sh.redi[0];
  for (int w = 1; w < kWaves; w++)
    if (sh.redf[w] > best || (sh.redf[w] == best && sh.redi[w] < idx)) { best = sh.redf[w]; idx = sh.redi[w]; }
  const int top = idx == INT_MAX ? 0 : idx;
  __syncthreads();
  // greedy; also when no logit is finite, or one is +inf (it then holds all the probability)
  if (P.temperature == 0.f || !(best > -INFINITY) || best == INFINITY) {
    if (t == 0) a.out[b] = top;
    return;
  }

  const Weigher wt{best, 1.4426950408889634f / P.temperature};
  Kept kept{0xffffffffu, INT_MAX};
  uint64_t kept_mass = 0;
  bool have_mass = false;
  if (P.top_k > 0 && P.top_k < V) {
    const uint64_t k = (uint64_t)P.top_k;
    kept = select_prefix(L, V, vec4, wt, kept, false, [&](uint64_t) { return k; }, sh, &kept_mass);
  }
  if (P.top_p < 1.f) {
    // the weight to reach comes from the kept set's total, which the first pass measures
    const double p = P.top_p;
    auto need_of = [&](uint64_t tot) -> uint64_t {
      const double want = ceil(p * (double)tot);
      const uint64_t n = want < 1.0 ? 1 : (uint64_t)want;
      return n > tot ? tot : n;
    };
    kept = select_prefix(L, V, vec4, wt, kept, true, need_of, sh, &kept_mass);
    have_mass = true;
  }
  uint64_t floor_w = 0;                                   // min-p: weight floor of the kept set
  if (P.min_p > 0.f) {
    if (!have_mass) {                                     // the kept set's weight
      uint64_t s = 0;
      for_each_logit(L, V, vec4, [&](float x, int i) {
        const float l = clean(x);
        if (kept.has(key_of(l), i)) s += wt(l);
      });
      uint64_t tot;
      block_excl_scan(s, sh.red, &tot);
      kept_mass = tot;
      __syncthreads();
    }
    const double f = ceil((double)P.min_p * (double)kept_mass);
    floor_w = f >= 18446744073709551615.0 ? ~0ull : (uint64_t)f;
  }
  auto wfinal = [&](float l, int i) -> uint64_t {
    if (!kept.has(key_of(l), i)) return 0;
    const uint64_t e = wt(l);
    return e >= floor_w ? e : 0;
  };
  // u from (seed, counter); the draw is the first kept token whose running weight exceeds
  // floor(u * total): x with its low 11 bits cleared times total, high 64 bits
  const uint64_t x = philox_word0(P.seed, (uint64_t)P.counter) & ~0x7ffull;
  uint64_t total;
  const int tok = first_crossing(L, V, vec4, wfinal, [&](uint64_t tot) { return __umul64hi(x, tot); }, sh, &total);
  if (t == 0) a.out[b] = total == 0 ? top : tok;          // min-p left nothing: the top token
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_sample, dim3(a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dtd
