// dtd_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the Llama-family decode step.
//
// Decode at small batch is bound by HBM traffic: every weight byte is read once per
// step and used for B multiply-adds ("从 smollm3.go 看 LLM inference", int8 weight-only
// quantization section: the int8 path exists to cut weight-memory traffic).  The kernels
// are therefore shaped around streaming weights with 16-byte coalesced loads per lane,
// dequantising in registers, keeping activations in LDS, and reducing across the 64-wide
// wavefront with cross-lane shuffles.  Everything that does not move weight or KV bytes
// (RMSNorm scaling, RoPE, KV append, SwiGLU, residual adds, argmax) rides in the
// prologues and epilogues of those kernels.
#include <algorithm>
#include <type_traits>
#include <math.h>
#include <stdint.h>
#include <limits.h>

#include "dtd_device.h"
#include "dtd_internal.h"

namespace dtd {
namespace {

using namespace dev;
using std::max;

// ---------------------------------------------------------------------------------------
// S0 embedding (+ block-table updates of this step)
// ---------------------------------------------------------------------------------------

// one workgroup of 1024 threads per sequence (a few elements per thread in flight)
__global__ __launch_bounds__(1024) void k_embed(Dims d, MatDev emb, const StepDesc* desc,
                                                int32_t* bt, float* x, int32_t* err) {
  const int b = blockIdx.x;
  if (b == 0) {
    for (int u = threadIdx.x; u < desc->n_updates; u += blockDim.x)
      bt[(size_t)desc->upd[u][0] * d.max_blocks + desc->upd[u][1]] = desc->upd[u][2];
  }
  int t = desc->tokens[b];
  if (t < 0 || t >= d.V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    t = 0;
  }
  float* xb = x + (size_t)b * d.D;
  for (int i = threadIdx.x; i < d.D; i += blockDim.x) xb[i] = deq_elem(emb, d.wfmt, t, i);
}

// ---------------------------------------------------------------------------------------
// S1 / S7 / S10 RMSNorm: xn = round_act(x / sqrt(mean(x^2) + eps) * g)
// ---------------------------------------------------------------------------------------

// One workgroup of kNormThreads per row (many loads in flight: a row is a few KB and the
// batch is a few dozen rows).
constexpr int kNormThreads = 1024;
constexpr int kNormPieces = 2;            // 16-byte pieces per thread: rows up to 8192
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const float* x, const float* g, void* xn, int D,
                                                          float eps, int act) {
  __shared__ float red[kNormThreads / 64];
  const int b = blockIdx.x;
  const float* xb = x + (size_t)b * D;
  if ((D & 3) == 0 && D <= kNormPieces * 4 * kNormThreads) {
    // the row in 16-byte pieces, kept in registers
    constexpr int NP = kNormPieces;
    float4 v[NP];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const int i = 4 * ((int)threadIdx.x + kNormThreads * k);
      v[k] = i < D ? *(const float4*)(xb + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const int i = 4 * ((int)threadIdx.x + kNormThreads * k);
      if (i >= D) continue;
      const float4 gg = *(const float4*)(g + i);
      const float y0 = v[k].x * r * gg.x, y1 = v[k].y * r * gg.y, y2 = v[k].z * r * gg.z, y3 = v[k].w * r * gg.w;
      if (act == ACT_BF16) {
        const uint32_t lo = f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
        const uint32_t hi = f32_to_bf16(y2) | ((uint32_t)f32_to_bf16(y3) << 16);
        *(uint2*)((uint16_t*)xn + (size_t)b * D + i) = make_uint2(lo, hi);
      } else {
        *(float4*)((float*)xn + (size_t)b * D + i) = make_float4(y0, y1, y2, y3);
      }
    }
    return;
  }
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += kNormThreads) ss += xb[i] * xb[i];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (act == ACT_BF16) {
    uint16_t* o = (uint16_t*)xn + (size_t)b * D;
    for (int i = threadIdx.x; i < D; i += kNormThreads) o[i] = f32_to_bf16(xb[i] * r * g[i]);
  } else {
    float* o = (float*)xn + (size_t)b * D;
    for (int i = threadIdx.x; i < D; i += kNormThreads) o[i] = xb[i] * r * g[i];
  }
}

// ---------------------------------------------------------------------------------------
// S2 / S6 / S8 / S9 / S10 weight-streaming GEMV with fused epilogues
//
// A 256-thread block = 4 waves; each wave owns ROWS consecutive stored rows and all NB
// batch columns of its grid.y slice.  Per K step each lane loads one 16-byte vector of
// each row (16 int8 codes or 8 bf16), reads the matching activations from LDS, and
// accumulates in fp32.  The activation chunk is staged into LDS in a swizzled order so
// that lane l's j-th float4 of a K step sits at float4 index (j*64 + l): the wave's
// ds_read_b128 then covers consecutive addresses and is free of bank conflicts.
// ---------------------------------------------------------------------------------------

struct GemvArgs {
  Dims d;
  MatDev m;
  const void* xin;   // [B][K] activations (fp32 or bf16)
  int B;
  int act_in;
  int kc;            // activation chunk length staged in LDS (multiple of the K step)
  EpiArgs ea;
};

template <int WFMT> struct WVec { static constexpr int VEC = 16; static constexpr int EB = 1; };
template <> struct WVec<W_BF16> { static constexpr int VEC = 8; static constexpr int EB = 2; };
// Q4_0: one 16-byte piece is one whole 32-column block (addressed in bytes as k / 2)
template <> struct WVec<W_Q4_0> { static constexpr int VEC = 32; static constexpr int EB = 1; };

template <int EPI, int ROWS>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, int b, int row0, const float* v) {
  const int N = a.m.rows;
  const Dims& d = a.d;
  if constexpr (EPI == EPI_QKV) {
    // Stored QKV rows: q and k heads hold the RoPE pairs (i, i + hd/2) as adjacent rows
    // (2i, 2i+1); v rows are in natural order.  The rotation is by the token's position,
    // which runs ahead of its cache index once a KV budget has evicted entries.
    const int pos = a.ea.desc->rpos[b];
    const int half = d.hd >> 1;
#pragma unroll
    for (int i = 0; i < ROWS; i += 2) {
      const int n = row0 + i;
      if (n >= N) break;
      const float u = v[i], w = v[i + 1];
      if (n < d.q_dim + d.kv_dim) {
        const bool isq = n < d.q_dim;
        const int nn = isq ? n : n - d.q_dim;
        const int h = nn / d.hd, p = (nn - h * d.hd) >> 1;
        const float c = a.ea.rope_cos[(size_t)pos * half + p];
        const float s = a.ea.rope_sin[(size_t)pos * half + p];
        float* dst = isq ? a.ea.q + (size_t)b * d.q_dim : a.ea.knew + (size_t)b * d.kv_dim;
        dst[h * d.hd + p] = u * c - w * s;
        dst[h * d.hd + p + half] = u * s + w * c;
      } else {
        const int nn = n - d.q_dim - d.kv_dim;
        a.ea.vnew[(size_t)b * d.kv_dim + nn] = u;
        a.ea.vnew[(size_t)b * d.kv_dim + nn + 1] = w;
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < ROWS; i++)
      if (row0 + i < N) a.ea.x[(size_t)b * N + row0 + i] += v[i];
  } else if constexpr (EPI == EPI_SWIGLU) {
    // stored rows (2f, 2f+1) = (gate f, up f)
#pragma unroll
    for (int i = 0; i < ROWS; i += 2) {
      const int n = row0 + i;
      if (n >= N) break;
      const int f = n >> 1;
      const float gt = v[i], up = v[i + 1];
      const float hv = gt / (1.0f + expf(-gt)) * up;
      if (d.act == ACT_BF16)
        ((uint16_t*)a.ea.h)[(size_t)b * d.F + f] = f32_to_bf16(hv);
      else
        ((float*)a.ea.h)[(size_t)b * d.F + f] = hv;
    }
  } else {  // EPI_LOGITS
    float* out = a.ea.desc->logits_out;
#pragma unroll
    for (int i = 0; i < ROWS; i++) {
      const int r = row0 + i;
      if (r < N) {
        a.ea.logits[(size_t)b * N + r] = v[i];
        if (out) out[(size_t)b * N + r] = v[i];
      }
    }
  }
}

template <int WFMT, int EPI, int NB, int ROWS>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  constexpr int VEC = WVec<WFMT>::VEC;
  constexpr int EB = WVec<WFMT>::EB;
  constexpr int KSTEP = 64 * VEC;
  extern __shared__ __attribute__((aligned(16))) float xs[];   // read as float4
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = a.m.rows, K = a.m.cols;
  const int row0 = (blockIdx.x * 4 + wave) * ROWS;
  const int b0 = blockIdx.y * NB;
  const int nb = min(NB, a.B - b0);
  const int KCP = a.kc;
  const uint8_t* wbase = (const uint8_t*)a.m.w;
  const size_t row_bytes = WFMT == W_Q4_0 ? (size_t)K / 2 : (size_t)K * EB;

  float acc[ROWS][NB];
#pragma unroll
  for (int i = 0; i < ROWS; i++)
#pragma unroll
    for (int bb = 0; bb < NB; bb++) acc[i][bb] = 0.f;

  // one k-step's weights: ROWS 16-byte pieces per lane (and their Q8_0 / Q4_0 block scales)
  auto load_w = [&](uint4 (&wv)[ROWS], float (&qs)[ROWS], int kc0, int kcn, int ks) {
    const int kl = ks + lane * VEC;
    const bool kvalid = kl < kcn;
    const int k = kc0 + kl;
#pragma unroll
    for (int i = 0; i < ROWS; i++) {
      const int r = row0 + i;
      const bool ok = kvalid && r < N;
      wv[i] = ok ? *(const uint4*)(wbase + (size_t)r * row_bytes + (WFMT == W_Q4_0 ? (size_t)k / 2 : (size_t)k * EB))
                 : make_uint4(0u, 0u, 0u, 0u);
      qs[i] = 0.f;
      if constexpr (WFMT == W_Q8_0 || WFMT == W_Q4_0)
        qs[i] = ok ? f16_to_f32(((const uint16_t*)a.m.s)[(size_t)r * (K / 32) + (k >> 5)]) : 0.f;
    }
  };
  // one k-step's multiply-adds against the staged activations
  auto dot_w = [&](const uint4 (&wv)[ROWS], const float (&qs)[ROWS], int ks) {
#pragma unroll
    for (int bb = 0; bb < NB; bb++) {
      float xv[VEC];
      const float4* xp = (const float4*)(xs + bb * KCP + ks) + lane;
#pragma unroll
      for (int jj = 0; jj < VEC / 4; jj++) {
        const float4 t = xp[jj * 64];
        xv[4 * jj + 0] = t.x; xv[4 * jj + 1] = t.y; xv[4 * jj + 2] = t.z; xv[4 * jj + 3] = t.w;
      }
#pragma unroll
      for (int i = 0; i < ROWS; i++) {
        const uint32_t u[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
        if constexpr (WFMT == W_BF16) {
          float s = acc[i][bb];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            s += __uint_as_float(u[q] << 16) * xv[2 * q];
            s += __uint_as_float(u[q] & 0xffff0000u) * xv[2 * q + 1];
          }
          acc[i][bb] = s;
        } else if constexpr (WFMT == W_Q4_0) {
          // byte b of the block: column b in the low 4 bits, column b + 16 in the high 4
          float s = 0.f;
#pragma unroll
          for (int q = 0; q < 4; q++)
#pragma unroll
            for (int by = 0; by < 4; by++) {
              const uint32_t byte = (u[q] >> (8 * by)) & 0xffu;
              s += (float)((int)(byte & 15u) - 8) * xv[4 * q + by];
              s += (float)((int)(byte >> 4) - 8) * xv[16 + 4 * q + by];
            }
          acc[i][bb] += qs[i] * s;
        } else {
          float s = 0.f;
#pragma unroll
          for (int q = 0; q < 4; q++)
#pragma unroll
            for (int by = 0; by < 4; by++) s += sext8(u[q], by) * xv[4 * q + by];
          if constexpr (WFMT == W_Q8_0) acc[i][bb] += qs[i] * s;
          else acc[i][bb] += s;
        }
      }
    }
  };

  uint4 wa[ROWS], wb[ROWS];
  float qa[ROWS], qb[ROWS];
  for (int kc0 = 0; kc0 < K; kc0 += KCP) {
    const int kcn = min(KCP, K - kc0);
    const int kcpad = (kcn + KSTEP - 1) / KSTEP * KSTEP;
    if (kc0) __syncthreads();
    load_w(wa, qa, kc0, kcn, 0);     // the chunk's first weights are in flight while x is staged
    // x staged 4 columns per access (K and every chunk are multiples of 4), four accesses in
    // flight per thread: the staging is a few load latencies, not one per column
    const int n4 = NB * kcpad / 4;
    for (int base = threadIdx.x; base < n4; base += 256 * 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int idx = (base + u * 256) * 4, bb = idx / kcpad, kk = idx - bb * kcpad;
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (base + u * 256 < n4 && bb < nb && kk < kcn) {
          const size_t gi = (size_t)(b0 + bb) * K + kc0 + kk;
          if (a.act_in == ACT_BF16) {
            const uint2 r = *(const uint2*)((const uint16_t*)a.xin + gi);
            v[u] = make_float4(bf16_to_f32(r.x & 0xffffu), bf16_to_f32(r.x >> 16), bf16_to_f32(r.y & 0xffffu),
                               bf16_to_f32(r.y >> 16));
          } else {
            v[u] = *(const float4*)((const float*)a.xin + gi);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        if (base + u * 256 >= n4) break;
        const int idx = (base + u * 256) * 4, bb = idx / kcpad, kk = idx - bb * kcpad;
        const int st = kk / KSTEP, r = kk - st * KSTEP, ln = r / VEC, j = r - ln * VEC;
        *(float4*)&xs[bb * KCP + st * KSTEP + (j >> 2) * 256 + ln * 4] = v[u];
      }
    }
    __syncthreads();

    // two k-steps per trip, the next step's weights always one step ahead
    for (int ks = 0; ks < kcn; ks += 2 * KSTEP) {
      if (ks + KSTEP < kcn) load_w(wb, qb, kc0, kcn, ks + KSTEP);
      dot_w(wa, qa, ks);
      if (ks + KSTEP >= kcn) break;
      if (ks + 2 * KSTEP < kcn) load_w(wa, qa, kc0, kcn, ks + 2 * KSTEP);
      dot_w(wb, qb, ks + KSTEP);
    }
  }

#pragma unroll
  for (int i = 0; i < ROWS; i++)
#pragma unroll
    for (int bb = 0; bb < NB; bb++) acc[i][bb] = wave_sum(acc[i][bb]);

  if (lane == 0) {
    for (int bb = 0; bb < nb; bb++) {
      float v[ROWS];
#pragma unroll
      for (int i = 0; i < ROWS; i++) {
        v[i] = acc[i][bb];
        if constexpr (WFMT == W_INT8_ROW)
          if (row0 + i < N) v[i] *= ((const float*)a.m.s)[row0 + i];  // scale after the dot
      }
      gemv_epilogue<EPI, ROWS>(a, b0 + bb, row0, v);
    }
  }
}

// ---------------------------------------------------------------------------------------
// S2 / S6 / S8 / S9 / S10 at batch > 1: weight-streaming GEMM on the matrix cores
//
// With several sequences a projection is a real (small-M) GEMM: every weight element is
// used once per sequence, and streaming the weights at HBM speed takes more multiply-adds
// than the vector units deliver.  C[n][b] = sum_k W[n][k] X[b][k] runs as
// v_mfma_f32_16x16x32_bf16 tiles: A = 16 weight rows x 32 k (int8-row codes are exact in
// bf16, their row scale is applied to the fp32 sum, after the dot, as in the int8
// weight-only scheme of "从 smollm3.go 看 LLM inference"), B = 32 k x 16 sequences of the
// bf16 activations, fp32 accumulation.
//
// A workgroup (4 waves) owns 64 weight rows, each wave 16; each lane streams its row's 16-byte
// pieces straight from HBM into MFMA operand registers (nontemporal loads), one K chunk of
// 256 columns ahead of use.  The activation chunk [16*NBB sequences][256] is staged in LDS,
// double buffered, and read as the B operands by all four waves.  When a matrix has fewer
// row tiles than compute units, its K range is split over S workgroups (blockIdx.y); their
// fp32 partial sums go to a work buffer and k_gemm_reduce adds them in a fixed order and
// runs the epilogue, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmRows = 64;                 // weight rows per workgroup (4 waves x 16)
constexpr int kGemmKC = 256;                  // K columns per staged activation chunk
constexpr int kGemmLd = kGemmKC * 2 + 16;     // LDS bytes per staged sequence row (16 B pad)

struct GemmArgs {
  GemvArgs g;        // dims, matrix, bf16 input [B][K], batch, epilogue destinations
  float* partials;   // [S][B][N] fp32 when S > 1
  int S;             // K splits
  int nchunk;        // K chunks of kGemmKC columns
};

// k covered by one 16-byte piece per lane: 8 bf16 or 16 int8 per lane, 4 lanes per row
template <int WFMT> struct GemmW {
  static constexpr int EB = WFMT == W_BF16 ? 2 : 1;
  static constexpr int KSTEP = 64 / EB;            // k per load step of a 16-row tile
  static constexpr int LPC = kGemmKC / KSTEP;       // load steps per chunk: bf16 8, int8 4
};

// two int8 codes (bytes b, b + 1 of u) as a packed pair of bf16 (exact: |q| <= 127)
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t u, int b) {
  const uint32_t lo = __float_as_uint(sext8(u, b)), hi = __float_as_uint(sext8(u, b + 1));
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);   // upper halves: lo's, then hi's
}

// x = hi + mid + lo as three bf16 bit patterns (each rounded to nearest even; the
// differences are exact in fp32)
__device__ __forceinline__ void split3(float x, uint32_t (&t)[3]) {
  t[0] = f32_to_bf16(x);
  const float r1 = x - bf16_to_f32(t[0]);
  t[1] = f32_to_bf16(r1);
  t[2] = f32_to_bf16(r1 - bf16_to_f32(t[1]));
}

// 8 fp32 values as the three bf16x8 operand terms
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 (&out)[3]) {
  u32x4 w[3];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    uint32_t a[3], b[3];
    split3(x[2 * u], a);
    split3(x[2 * u + 1], b);
#pragma unroll
    for (int s = 0; s < 3; s++) w[s][u] = a[s] | (b[s] << 16);
  }
#pragma unroll
  for (int s = 0; s < 3; s++) out[s] = __builtin_bit_cast(bf16x8, w[s]);
}

// acc += A B for operands given as NA and NB bf16 terms (1: exact in bf16, 3: an fp32 value
// split by split3): the term products whose weights add to at least 2^-24, smaller first
template <int NA, int NB>
__device__ __forceinline__ f32x4 mfma_terms(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x4 acc) {
  if constexpr (NA == 3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b[0], acc, 0, 0, 0);
  if constexpr (NB == 3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[2], acc, 0, 0, 0);
  if constexpr (NA == 3 && NB == 3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[1], acc, 0, 0, 0);
  if constexpr (NA == 3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b[0], acc, 0, 0, 0);
  if constexpr (NB == 3) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[0], acc, 0, 0, 0);
  return acc;
}

template <int WFMT, int EPI, int NBB>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];   // [2][16*NBB][kGemmLd]
  constexpr int EB = GemmW<WFMT>::EB, KSTEP = GemmW<WFMT>::KSTEP, LPC = GemmW<WFMT>::LPC;
  constexpr int XROWS = 16 * NBB, XV = XROWS * kGemmKC / 8 / 256;   // 16-byte X pieces per thread
  constexpr int BUF = XROWS * kGemmLd;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.g.m.rows, K = a.g.m.cols, B = a.g.B;
  const int n0 = blockIdx.x * kGemmRows;
  const int sp = blockIdx.y, S = a.S;
  const int c_lo = sp * a.nchunk / S, c_hi = (sp + 1) * a.nchunk / S;
  // this lane's weight row, and the k offset of its 16 bytes within a load step
  const int row = n0 + 16 * wave + (lane & 15);
  const bool row_ok = row < N;
  const uint8_t* wbase = (const uint8_t*)a.g.m.w;
  const uint8_t* wrow = wbase + (size_t)(row_ok ? row : 0) * (size_t)K * EB;
  const int kl = (lane >> 4) * (16 / EB);
  const uint8_t* xg = (const uint8_t*)a.g.xin;

  // Loads outside the matrix (past K, or chunks past this split) read the matrix's first 16
  // bytes: every such lane of a wave hits one line, and each buffer keeps one issue site.
  auto issue_w = [&](int c, u32x4 (&w)[LPC]) {
#pragma unroll
    for (int i = 0; i < LPC; i++) {
      const int k = c * kGemmKC + i * KSTEP + kl;
      const bool ok = row_ok && c < c_hi && k < K;
      w[i] = gload_stream<u32x4>(ok ? wrow + (size_t)k * EB : wbase);
    }
  };
  auto x_piece = [&](int c, int v, int& r, int& k) {
    const int idx = tid + 256 * v;
    constexpr int PPR = kGemmKC / 8;                // 16-byte pieces per row
    r = idx / PPR;
    k = c * kGemmKC + (idx % PPR) * 8;
  };
  auto issue_x = [&](int c, uint4 (&x)[XV]) {
#pragma unroll
    for (int v = 0; v < XV; v++) {
      int r, k;
      x_piece(c, v, r, k);
      const bool ok = r < B && k < K && c < c_hi;
      x[v] = gload<uint4>(ok ? xg + ((size_t)r * K + k) * 2 : xg);
    }
  };
  auto store_x = [&](int c, const uint4 (&x)[XV], int buf) {
#pragma unroll
    for (int v = 0; v < XV; v++) {
      int r, k;
      x_piece(c, v, r, k);
      const bool ok = r < B && k < K;
      *(uint4*)(xl + buf * BUF + r * kGemmLd + (k - c * kGemmKC) * 2) = ok ? x[v] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  f32x4 acc[NBB];
#pragma unroll
  for (int j = 0; j < NBB; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const u32x4 (&w)[LPC], int buf) {
    const uint8_t* xb = xl + buf * BUF + (lane & 15) * kGemmLd;
#pragma unroll
    for (int i = 0; i < LPC; i++) {
      const int kc = (i * KSTEP + kl) * 2;         // byte column of the lane's first k in the chunk
      if constexpr (WFMT == W_BF16) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, w[i]);
#pragma unroll
        for (int j = 0; j < NBB; j++) {
          const bf16x8 Bv = *(const bf16x8*)(xb + j * 16 * kGemmLd + kc);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv, acc[j], 0, 0, 0);
        }
      } else {
        // the lane's 16 codes are k .. k+15: the first 8 feed one product, the last 8 the next
        const u32x4 lo = {i8x2_to_bf16x2(w[i].x, 0), i8x2_to_bf16x2(w[i].x, 2), i8x2_to_bf16x2(w[i].y, 0),
                          i8x2_to_bf16x2(w[i].y, 2)};
        const u32x4 hi = {i8x2_to_bf16x2(w[i].z, 0), i8x2_to_bf16x2(w[i].z, 2), i8x2_to_bf16x2(w[i].w, 0),
                          i8x2_to_bf16x2(w[i].w, 2)};
        const bf16x8 A0 = __builtin_bit_cast(bf16x8, lo), A1 = __builtin_bit_cast(bf16x8, hi);
#pragma unroll
        for (int j = 0; j < NBB; j++) {
          const bf16x8 B0 = *(const bf16x8*)(xb + j * 16 * kGemmLd + kc);
          const bf16x8 B1 = *(const bf16x8*)(xb + j * 16 * kGemmLd + kc + 16);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B1, acc[j], 0, 0, 0);
        }
      }
    }
  };

  // Chunk c is multiplied from LDS buffer c & 1 with weight registers WA (even steps) or WB
  // (odd steps) while chunk c + 1's activations and chunk c + 2's weights are on their way.
  u32x4 WA[LPC], WB[LPC];
  uint4 xr[XV];
  issue_x(c_lo, xr);
  issue_w(c_lo, WA);
  issue_w(c_lo + 1, WB);
  store_x(c_lo, xr, 0);
  __syncthreads();
  for (int c = c_lo; c < c_hi; c += 2) {
    issue_x(c + 1, xr);
    consume(WA, 0);
    issue_w(c + 2, WA);
    store_x(c + 1, xr, 1);
    __syncthreads();
    if (c + 1 >= c_hi) break;                     // (uniform)
    issue_x(c + 2, xr);
    consume(WB, 1);
    issue_w(c + 3, WB);
    store_x(c + 2, xr, 0);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < LPC; i++) { (void)WA[i]; (void)WB[i]; }

  // lane l holds rows 4(l/16) .. +3 of the wave's 16, for sequence 16 j + l % 16
  const int r0 = n0 + 16 * wave + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < NBB; j++) {
    const int b = 16 * j + (lane & 15);
    if (b >= B) continue;
    if (S == 1) {
      float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      if constexpr (WFMT == W_INT8_ROW) {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (r0 + r < N) v[r] *= ((const float*)a.g.m.s)[r0 + r];   // row scale after the dot
      }
      gemv_epilogue<EPI, 4>(a.g, b, r0, v);
    } else {
      float* P = a.partials + ((size_t)sp * B + b) * N;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (r0 + r < N) P[r0 + r] = acc[j][r];
    }
  }
}

// the S partial sums of 4 consecutive rows of one sequence, added in split order, then the
// epilogue
template <int WFMT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmArgs a) {
  const int N = a.g.m.rows, B = a.g.B;
  const int nq = (N + 3) / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nq * B) return;
  const int b = idx / nq, r0 = (idx - b * nq) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.S; sp++) {
    const float* P = a.partials + ((size_t)sp * B + b) * N;
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (r0 + r < N) v[r] += P[r0 + r];
  }
  if constexpr (WFMT == W_INT8_ROW) {
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (r0 + r < N) v[r] *= ((const float*)a.g.m.s)[r0 + r];
  }
  gemv_epilogue<EPI, 4>(a.g, b, r0, v);
}

// The split-K sums of a residual projection (O or down: N = D rows), the residual add, and
// the RMSNorm that follows it (of the next block), in one launch: one workgroup per
// sequence.  Thread t takes rows 4 (t + kNormThreads k), the rows k_rmsnorm's vector path
// gives it, and runs k_gemm_reduce's and k_rmsnorm's operations in their order.  D a
// multiple of 4, at most 8192.
template <int WFMT>
__global__ __launch_bounds__(kNormThreads) void k_gemm_reduce_norm(GemmArgs a, const float* g, void* xn) {
  __shared__ float red[kNormThreads / 64];
  constexpr int NP = kNormPieces;
  const int D = a.g.m.rows, B = a.g.B, b = blockIdx.x;
  float* xb = a.g.ea.x + (size_t)b * D;
  float4 v[NP];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NP; k++) {
    const int i = 4 * ((int)threadIdx.x + kNormThreads * k);
    v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i >= D) continue;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.S; sp++) {
      const float4 p = *(const float4*)(a.partials + ((size_t)sp * B + b) * D + i);
      s[0] += p.x; s[1] += p.y; s[2] += p.z; s[3] += p.w;
    }
    if constexpr (WFMT == W_INT8_ROW) {
      const float4 sc = *(const float4*)((const float*)a.g.m.s + i);
      s[0] *= sc.x; s[1] *= sc.y; s[2] *= sc.z; s[3] *= sc.w;
    }
    float4 x = *(const float4*)(xb + i);
    x.x += s[0]; x.y += s[1]; x.z += s[2]; x.w += s[3];
    *(float4*)(xb + i) = x;
    v[k] = x;
    ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + a.g.d.eps);
  const int act = a.g.d.act;
#pragma unroll
  for (int k = 0; k < NP; k++) {
    const int i = 4 * ((int)threadIdx.x + kNormThreads * k);
    if (i >= D) continue;
    const float4 gg = *(const float4*)(g + i);
    const float y0 = v[k].x * r * gg.x, y1 = v[k].y * r * gg.y, y2 = v[k].z * r * gg.z, y3 = v[k].w * r * gg.w;
    if (act == ACT_BF16) {
      const uint32_t lo = f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
      const uint32_t hi = f32_to_bf16(y2) | ((uint32_t)f32_to_bf16(y3) << 16);
      *(uint2*)((uint16_t*)xn + (size_t)b * D + i) = make_uint2(lo, hi);
    } else {
      *(float4*)((float*)xn + (size_t)b * D + i) = make_float4(y0, y1, y2, y3);
    }
  }
}

// ---------------------------------------------------------------------------------------
// S4 + S5 split-K GQA decode attention (work item in dtd_device.h) and the chunk merge
// ---------------------------------------------------------------------------------------

template <int KVFMT>
__global__ __launch_bounds__(256) void k_attn(AttnCtx a, const StepDesc* desc, float* partials) {
  extern __shared__ __attribute__((aligned(16))) float sm[];   // read as float4
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int pos = desc->pos[b];
  if (c * a.ct > pos) return;               // chunk beyond this sequence's length
  const int G = a.d.G, hd = a.d.hd;
  attn_item<KVFMT>(a, b, j, c, pos, desc->slot[b], desc->pos_block[b],
                   a.q + (size_t)b * a.d.q_dim + (size_t)j * G * hd,
                   a.knew + (size_t)b * a.d.kv_dim + (size_t)j * hd,
                   a.vnew + (size_t)b * a.d.kv_dim + (size_t)j * hd, sm,
                   [partials](size_t i, float v) { partials[i] = v; });
}

// ---------------------------------------------------------------------------------------
// S4 + S5 for the common shapes (KV blocks of 16 positions; head size 128 or 64 with 4 query
// heads per KV head, or 32 with 5): one wave per (sequence b, KV head j, chunk c)
//
// The wave walks its chunk one paged block (16 positions) at a time; the block ids of the
// chunk sit in two registers and are broadcast with readlane, and the loads of the next two
// blocks are in flight while one is being used.  K and V are read once for the G heads (the
// GQA decode rule of the Qwen3-8B engine article, 4.4.2), with no workgroup barrier.
//  - Scores on the matrix cores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16, rows the block's
//    16 positions, columns the group's heads (G <= 16; the other columns are zero).  Lane
//    (quad, r16) loads its A operand straight from the pool, 8 elements of position r16 per
//    32-wide slice of the head; bf16 and int8 keys are exact in bf16 (int8 scales multiply
//    the score rows), fp32 keys and the queries enter as three bf16 terms, so the products
//    keep fp32 accuracy.
//  - The online softmax runs on the score layout (a head's 16 scores on 4 lanes), and each
//    block's P and rescale factors go to the P V layout through 1 KB of the wave's LDS.
//  - P V on the vector units: one wave-wide load of PB bytes per lane reads whole V rows,
//    lane l holding elements [e0, e0 + ELEM) of one position (LPP lanes per position), and
//    the G heads' accumulators stay in registers until the cross-group sum at the end.
// The wave leaves an unnormalised partial (acc, m, l) per head in the same layout as k_attn;
// k_combine merges the chunks.
// ---------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// sum / max over aligned groups of L consecutive lanes; every lane of a group gets its result
template <int L>
__device__ __forceinline__ float grp_sum(float v) {
  if constexpr (L >= 2) v += dppf<0xb1>(v);    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dppf<0x4e>(v);    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dppf<0x141>(v);   // row_half_mirror
  if constexpr (L >= 16) v += dppf<0x140>(v);  // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int L>
__device__ __forceinline__ float grp_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dppf<0xb1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dppf<0x4e>(v));
  if constexpr (L >= 8) v = fmaxf(v, dppf<0x141>(v));
  if constexpr (L >= 16) v = fmaxf(v, dppf<0x140>(v));
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (L >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// sum / max over the lanes l, l ^ S, l ^ 2S, ... (one lane of every group of S)
template <int S>
__device__ __forceinline__ float xgrp_sum(float v) {
#pragma unroll
  for (int m = S; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int S>
__device__ __forceinline__ float xgrp_max(float v) {
#pragma unroll
  for (int m = S; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Layout of one wave-wide load of a block's rows: PB bytes per lane (16; 8 for int8, so that
// a lane holds 8 elements in every format and the registers stay within two waves per SIMD).
template <int KVFMT, int HD>
struct WaveKv {
  static constexpr int EB = KVFMT == KV_F32 ? 4 : (KVFMT == KV_BF16 ? 2 : 1);
  static constexpr int PB = KVFMT == KV_I8 ? 8 : 16;
  static constexpr int RB = HD * EB;         // bytes of one position's row (one KV head)
  static constexpr int LPP = RB / PB;        // lanes per position in one wave-wide load
  static constexpr int PPI = 64 / LPP;       // positions per wave-wide load
  static constexpr int ELEM = PB / EB;       // elements per lane per load
  static constexpr int NI = 16 / PPI;        // loads per 16-position block
  static constexpr int LOADB = 64 * PB;      // bytes per wave-wide load
  static_assert(16 * RB >= LOADB && PPI <= 16, "a block must fill at least one wave-wide load");
};

template <int PB> struct Piece;
template <> struct Piece<16> { typedef uint4 T; };
template <> struct Piece<8> { typedef uint2 T; };

// the floats of one piece of a stored row (int8: the codes, unscaled)
template <int KVFMT, int ELEM>
__device__ __forceinline__ void decode_piece(const uint2& u, float (&f)[ELEM]) {
  static_assert(KVFMT == KV_I8 && ELEM == 8, "8-byte pieces: int8");
  const uint32_t w[2] = {u.x, u.y};
#pragma unroll
  for (int q = 0; q < 2; q++)
#pragma unroll
    for (int b = 0; b < 4; b++) f[4 * q + b] = sext8(w[q], b);
}

template <int KVFMT, int ELEM>
__device__ __forceinline__ void decode_piece(const uint4& u, float (&f)[ELEM]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if constexpr (KVFMT == KV_F32) {
      f[q] = __uint_as_float(w[q]);
    } else if constexpr (KVFMT == KV_BF16) {
      f[2 * q] = __uint_as_float(w[q] << 16);
      f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    } else {
#pragma unroll
      for (int b = 0; b < 4; b++) f[4 * q + b] = sext8(w[q], b);
    }
  }
}

template <int KVFMT, int HD, int G>
__global__ __launch_bounds__(256) void k_attn_w(AttnCtx a, const StepDesc* desc, float* partials) {
  using W = WaveKv<KVFMT, HD>;
  constexpr int RB = W::RB, LPP = W::LPP, PPI = W::PPI, ELEM = W::ELEM, NI = W::NI, PB = W::PB;
  constexpr int NS = HD / 32;                    // 32-wide slices of the head dimension
  constexpr int NTK = KVFMT == KV_F32 ? 3 : 1;   // bf16 terms of a stored key element
  constexpr int KPC = 8 * W::EB / PB;            // pieces of a lane's 8 key elements in one slice
  static_assert(HD % 32 == 0 && G <= 16, "head size a multiple of 32, at most 16 query heads per KV head");
  typedef typename Piece<PB>::T PieceT;
  // per wave: this block's P [16 positions][G] and alpha [G] on their way from the score
  // layout to the P V layout; the new position's key row as stored
  __shared__ float pl_s[4][17 * G];
  __shared__ __attribute__((aligned(16))) uint8_t nrow_s[4][RB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, quad = lane >> 4;
  const int w = blockIdx.x * 4 + wave, j = blockIdx.y;
  const Dims& d = a.d;
  if (w >= desc->n_chunks) return;                      // (wave-uniform) past the chunk list
  // chunk w of the list: sequence b = the number of sequences whose chunks end at or before
  // w, chunk c of its context
  const int ce = lane < desc->batch ? desc->cend[lane] : INT_MAX;
  const int b = __popcll(__ballot(ce <= w));
  const int c = w - (b > 0 ? __builtin_amdgcn_readlane(ce, b - 1) : 0);
  const int ct = desc->ct[b];
  const int pos = desc->pos[b];
  const int t_begin = c * ct;
  if (c >= a.nch || t_begin > pos) return;              // (wave-uniform) chunk past the sequence
  const int t_end = min(pos + 1, t_begin + ct);
  const int pg = lane / LPP, e0 = (lane % LPP) * ELEM;
  const int Hkv = d.Hkv;
  float* pl = pl_s[wave];
  uint8_t* nrow = nrow_s[wave];

  // The query group as the B operand of S^T = K Q^T on the matrix cores: lane (quad, r16)
  // holds head r16 (zero past G), elements 32 s + 8 quad .. +7 of slice s, scaled by
  // log2(e)/sqrt(hd) so that scores are in base-2 units (every exponential is one v_exp_f32),
  // as three bf16 terms (fp32 accuracy)
  bf16x8 qb[NS][3];
  {
    const float sc = 1.4426950408889634f / sqrtf((float)HD);
    const float* qh = a.q + (size_t)b * d.q_dim + (size_t)(j * G + (r16 < G ? r16 : 0)) * HD + 8 * quad;
#pragma unroll
    for (int s = 0; s < NS; s++) {
      const float4 u0 = gload<float4>(qh + 32 * s), u1 = gload<float4>(qh + 32 * s + 4);
      const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float y[8];
#pragma unroll
      for (int u = 0; u < 8; u++) y[u] = r16 < G ? x[u] * sc : 0.f;
      split8(y, qb[s]);
    }
  }
  // block ids of the chunk's blocks (at most 128)
  const int lb0 = t_begin >> 4, nb = (t_end - t_begin + 15) >> 4;
  const int32_t* btrow = a.bt + (size_t)desc->slot[b] * d.max_blocks;
  const int bt_lo = lane < nb ? gload<int32_t>(btrow + lb0 + lane) : 0;
  const int bt_hi = lane + 64 < nb ? gload<int32_t>(btrow + lb0 + lane + 64) : 0;

  float new_ks = 1.f;   // int8: the new position's key scale
  // The new position: rounded to the KV encoding and appended through the block table by the
  // wave whose chunk holds it; its stored (decoded) values replace the block's row there.
  const bool has_new = pos >= t_begin && pos < t_end;
  float nk[ELEM], nv[ELEM];
#pragma unroll
  for (int e = 0; e < ELEM; e++) nk[e] = nv[e] = 0.f;
  if (has_new) {
    const size_t row = ((size_t)desc->pos_block[b] * Hkv + j) * 16 + (pos & 15);
#pragma unroll
    for (int which = 0; which < 2; which++) {
      const float* src = (which ? a.vnew : a.knew) + (size_t)b * d.kv_dim + (size_t)j * HD + e0;
      float x[ELEM];
#pragma unroll
      for (int e = 0; e < ELEM; e += 4) {
        const float4 v = gload<float4>(src + e);
        x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
      }
      float dec[ELEM];
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if constexpr (KVFMT == KV_F32) {
#pragma unroll
        for (int e = 0; e < ELEM; e++) dec[e] = x[e];
#pragma unroll
        for (int qd = 0; qd < 4; qd++) w[qd] = __float_as_uint(x[qd]);
      } else if constexpr (KVFMT == KV_BF16) {
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
          const uint32_t lo = f32_to_bf16(x[2 * qd]), hi = f32_to_bf16(x[2 * qd + 1]);
          w[qd] = lo | hi << 16;
          dec[2 * qd] = bf16_to_f32(lo);
          dec[2 * qd + 1] = bf16_to_f32(hi);
        }
      } else {
        // s = fp16(max|x| / 127) over the head's hd values (the LPP lanes of a position hold
        // them all), q = clamp(rint(x / s), -127, 127), s = 0 gives q = 0
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < ELEM; e++) mx = fmaxf(mx, fabsf(x[e]));
        mx = grp_max<LPP>(mx);
        const uint16_t s16 = f32_to_f16(mx / 127.0f);
        const float sc = f16_to_f32(s16);
#pragma unroll
        for (int qd = 0; qd < ELEM / 4; qd++) {
          uint32_t packed = 0;
#pragma unroll
          for (int bb = 0; bb < 4; bb++) {
            const int e = 4 * qd + bb;
            const float code = sc != 0.f ? fminf(fmaxf(rintf(x[e] / sc), -127.f), 127.f) : 0.f;
            dec[e] = code * sc;
            packed |= ((uint32_t)(int32_t)code & 0xffu) << (8 * bb);
          }
          w[qd] = packed;
        }
        if (lane == 0) gstore<uint16_t>((which ? a.kv.vs : a.kv.ks) + row, s16);
        if (which == 0) new_ks = sc;
      }
      uint8_t* dst = (uint8_t*)(which ? a.kv.v : a.kv.k) + row * RB + (size_t)e0 * W::EB;
      if (pg == 0) {
        if constexpr (PB == 16) gstore<uint4>(dst, make_uint4(w[0], w[1], w[2], w[3]));
        else gstore<uint64_t>(dst, (uint64_t)w[1] << 32 | w[0]);
        // the key row as stored, for the score of the new position (its block's loads may
        // have been issued before the store)
        if (which == 0) {
          if constexpr (PB == 16) *(uint4*)(nrow + e0 * W::EB) = make_uint4(w[0], w[1], w[2], w[3]);
          else *(uint2*)(nrow + e0 * W::EB) = make_uint2(w[0], w[1]);
        }
      }
#pragma unroll
      for (int e = 0; e < ELEM; e++) (which ? nv : nk)[e] = dec[e];
    }
  }

  struct Tile {
    PieceT kq[NS * KPC];   // key r16 of the block, elements 32 s + 8 quad .. +7 of each slice
    PieceT v[NI];          // V in the P V layout: position PPI i + pg, elements e0 ..
    uint2 ks4;             // int8: key scales of positions 4 quad .. +3
    float vs[NI];          // int8: value scales of the P V positions
  };
  // Issues block t of the chunk (past the last block: one line at the pool's start, unused).
  auto issue = [&](int t, Tile& T) {
    const bool real = t < nb;
    const int blk = t < 64 ? __builtin_amdgcn_readlane(bt_lo, t & 63) : __builtin_amdgcn_readlane(bt_hi, t & 63);
    const size_t rowbase = ((size_t)(real ? blk : 0) * Hkv + j) * 16;
    const uint8_t* kb = (const uint8_t*)a.kv.k + (real ? (rowbase + r16) * RB + (size_t)8 * quad * W::EB : 0);
    const uint8_t* vb = (const uint8_t*)a.kv.v + (real ? rowbase * RB + lane * PB : 0);
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int u = 0; u < KPC; u++) T.kq[s * KPC + u] = gload<PieceT>(kb + (real ? 32 * s * W::EB + u * PB : 0));
#pragma unroll
    for (int i = 0; i < NI; i++) T.v[i] = gload<PieceT>(vb + (real ? i * W::LOADB : 0));
    if constexpr (KVFMT == KV_I8) {
      T.ks4 = gload<uint2>(a.kv.ks + (real ? rowbase + 4 * quad : 0));
#pragma unroll
      for (int i = 0; i < NI; i++) T.vs[i] = f16_to_f32(gload<uint16_t>(a.kv.vs + (real ? rowbase + PPI * i + pg : 0)));
    }
  };

  // running max and sum of head r16 (the score layout's column), and the P V accumulators
  float mc = -INFINITY, lc = 0.f, acc[G][ELEM];
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int e = 0; e < ELEM; e++) acc[h][e] = 0.f;
  // EDGE: the chunk's last block, the only one that can end inside the block or hold the new
  // position (the selects for those cases are left out of every other block)
  auto consume = [&](int t, const Tile& T, auto edge) {
    constexpr bool EDGE = decltype(edge)::value;
    const int p0 = t_begin + 16 * t;
    const int kn = pos - p0;                       // the new position's row in this block
    // ---- S^T = K Q^T: rows the block's 16 positions, columns the group's heads ----
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; s++) {
      PieceT pc[KPC];
#pragma unroll
      for (int u = 0; u < KPC; u++) pc[u] = T.kq[s * KPC + u];
      if (EDGE && has_new && r16 == kn) {
#pragma unroll
        for (int u = 0; u < KPC; u++) pc[u] = *(const PieceT*)(nrow + (32 * s + 8 * quad) * W::EB + u * PB);
      }
      bf16x8 ka[3];
      if constexpr (KVFMT == KV_BF16) {
        ka[0] = __builtin_bit_cast(bf16x8, pc[0]);
      } else if constexpr (KVFMT == KV_I8) {
        const u32x4 w4 = {i8x2_to_bf16x2(pc[0].x, 0), i8x2_to_bf16x2(pc[0].x, 2), i8x2_to_bf16x2(pc[0].y, 0),
                          i8x2_to_bf16x2(pc[0].y, 2)};
        ka[0] = __builtin_bit_cast(bf16x8, w4);
      } else {
        const float x[8] = {__uint_as_float(pc[0].x), __uint_as_float(pc[0].y), __uint_as_float(pc[0].z),
                            __uint_as_float(pc[0].w), __uint_as_float(pc[1].x), __uint_as_float(pc[1].y),
                            __uint_as_float(pc[1].z), __uint_as_float(pc[1].w)};
        split8(x, ka);
      }
      sacc = mfma_terms<NTK, 3>(ka, qb[s], sacc);
    }
    // lane (quad, r16): positions p0 + 4 quad + i, head r16
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int key = 4 * quad + i;
      float v = sacc[i];
      if constexpr (KVFMT == KV_I8) {
        const uint32_t hw = i < 2 ? T.ks4.x : T.ks4.y;
        float ksc = f16_to_f32((uint16_t)((i & 1) ? hw >> 16 : hw & 0xffffu));
        if (EDGE && has_new && key == kn) ksc = new_ks;
        v *= ksc;
      }
      sv[i] = (!EDGE || p0 + key < t_end) ? v : -INFINITY;   // a stale row past the end is dropped
    }
    // the online softmax of head r16 over the block's 16 positions (4 lanes of the column)
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(mc, mx);                // finite: the chunk's first position is in range
    const float al = __builtin_amdgcn_exp2f(mc - mn);   // 2^(-inf) = 0 on the first block
    float pr[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      pr[i] = __builtin_amdgcn_exp2f(sv[i] - mn);
      ps += pr[i];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lc = lc * al + ps;
    mc = mn;
    // P and alpha to the P V layout through this wave's LDS (a wave's LDS accesses complete
    // in order; the empty asm keeps the compiler from moving them across each other)
    if (r16 < G) {
#pragma unroll
      for (int i = 0; i < 4; i++) pl[(4 * quad + i) * G + r16] = pr[i];
      if (quad == 0) pl[16 * G + r16] = al;
    }
    asm volatile("" ::: "memory");
    float alpha[G], p_[NI][G];
#pragma unroll
    for (int h = 0; h < G; h++) alpha[h] = pl[16 * G + h];
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
      for (int h = 0; h < G; h++) p_[i][h] = pl[(PPI * i + pg) * G + h];
    asm volatile("" ::: "memory");
    // ---- O = O * alpha + P V ----
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
      for (int e = 0; e < ELEM; e++) acc[h][e] *= alpha[h];
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const int p = p0 + PPI * i + pg;
      const bool isnew = EDGE && has_new && p == pos;
      const bool valid = !EDGE || p < t_end;   // rows past the chunk's end (last block) are never attended
      float vf[ELEM];
      decode_piece<KVFMT, ELEM>(T.v[i], vf);
      // a stale row past the end holds anything, and 0 times a non-finite value is not 0
#pragma unroll
      for (int e = 0; e < ELEM; e++) vf[e] = isnew ? nv[e] : (valid ? vf[e] : 0.f);
#pragma unroll
      for (int h = 0; h < G; h++) {
        float pv = p_[i][h];
        if constexpr (KVFMT == KV_I8) pv = valid ? pv * (isnew ? 1.f : T.vs[i]) : 0.f;   // V's row scale into p
#pragma unroll
        for (int e = 0; e < ELEM; e++) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
      }
    }
  };

  Tile TA, TB;
  issue(0, TA);
  issue(1, TB);
  using Mid = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  for (int t = 0; t < nb; t += 2) {
    if (t == nb - 1) consume(t, TA, Last{});
    else consume(t, TA, Mid{});
    issue(t + 2, TA);
    if (t + 1 >= nb) break;
    if (t + 1 == nb - 1) consume(t + 1, TB, Last{});
    else consume(t + 1, TB, Mid{});
    issue(t + 3, TB);
  }

  // the position groups' accumulators, each head's max and sum (from its column's lanes),
  // then the partial in k_attn's layout
#pragma unroll
  for (int h = 0; h < G; h++)
#pragma unroll
    for (int e = 0; e < ELEM; e++) acc[h][e] = xgrp_sum<LPP>(acc[h][e]);
  float mh[G], lh[G];
#pragma unroll
  for (int h = 0; h < G; h++) {
    mh[h] = __shfl(mc, h, 64);
    lh[h] = __shfl(lc, h, 64);
  }
  const int cs = HD + 2;
  if (pg == 0) {
#pragma unroll
    for (int h = 0; h < G; h++) {
      float* P = partials + (((size_t)b * d.Hq + (size_t)j * G + h) * a.nch + c) * cs;
#pragma unroll
      for (int e = 0; e < ELEM; e++) gstore<float>(P + e0 + e, acc[h][e]);   // (rows of hd + 2: no 16-B alignment)
      if (lane == 0) {
        P[HD] = mh[h] * 0.6931471805599453f;   // base-2 running max back to natural units
        P[HD + 1] = lh[h];
      }
    }
  }
}

// KV append of every new position of a step, before its attention: one workgroup per
// (position b, KV head j).  A prefill chunk puts several positions of one sequence in one
// step, and each attends to the ones before it, which must then be in the cache already.
// The attention kernels append their own new position again, with identical bytes.
template <int KVFMT>
__global__ __launch_bounds__(128) void k_kv_append(Dims d, KvLayer kv, const StepDesc* desc, const float* knew,
                                                   const float* vnew) {
  __shared__ float new_s[256];
  __shared__ float red[4];
  const int b = blockIdx.x, j = blockIdx.y;
  const int pos = desc->pos[b];
  const size_t row = ((size_t)desc->pos_block[b] * d.Hkv + j) * d.bs + (pos % d.bs);
  kv_append<KVFMT>(kv, row, d.hd, knew + (size_t)b * d.kv_dim + (size_t)j * d.hd,
                   vnew + (size_t)b * d.kv_dim + (size_t)j * d.hd, new_s, red);
}

// Prefix reuse: copies KV block src to block dst in every layer (grid: layer x {K, V, K
// scales, V scales}); `elem` = bytes of one stored element, 16-byte pieces, tail bytes alone.
__global__ __launch_bounds__(256) void k_kv_copy_block(const PLayer* layers, int Hkv, int bs, int hd, int elem,
                                                       int src, int dst) {
  const KvLayer kv = layers[blockIdx.x].kv;
  const int which = blockIdx.y;
  const bool scales = which >= 2;
  uint8_t* pool = (uint8_t*)(which == 0 ? kv.k : which == 1 ? kv.v : which == 2 ? (void*)kv.ks : (void*)kv.vs);
  if (!pool) return;
  const size_t n = scales ? (size_t)Hkv * bs * 2 : (size_t)Hkv * bs * hd * elem;
  const uint8_t* a = pool + (size_t)src * n;
  uint8_t* b = pool + (size_t)dst * n;
  const size_t n16 = n % 16 == 0 ? n / 16 : 0;    // 16-byte pieces only when every block starts aligned
  for (size_t i = threadIdx.x; i < n16; i += 256) ((uint4*)b)[i] = ((const uint4*)a)[i];
  for (size_t i = n16 * 16 + threadIdx.x; i < n; i += 256) b[i] = a[i];
}

// one (head, sequence), a block of max(hd, 64) threads: o = merge of its chunk partials,
// rounded to the activation type; with stat, also the softmax's max M and normaliser L
// (natural-log units) per (sequence, head).  Each chunk's weight e^(m_c - M) is worked out
// once, into LDS; the sums over chunks have a fixed order.
__global__ __launch_bounds__(256) void k_combine(Dims d, const StepDesc* desc, const float* partials,
                                                 void* o, float* stat) {
  extern __shared__ float w_s[];         // [nch] chunk weights
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x, nt = blockDim.x;
  const int ct = desc->ct[b];
  const int nv = (desc->pos[b] + ct) / ct;
  const int cs = d.hd + 2;
  const float* P = partials + ((size_t)b * d.Hq + h) * d.nch * cs;
  float mx = -INFINITY;
  for (int c = i; c < nv; c += nt) mx = fmaxf(mx, P[c * cs + d.hd]);
  const float M = block_max(mx, red);
  float ls = 0.f;
  for (int c = i; c < nv; c += nt) {
    const float w = expf(P[c * cs + d.hd] - M);
    w_s[c] = w;
    ls += w * P[c * cs + d.hd + 1];
  }
  const float L = block_sum(ls, red);   // (its barriers also publish w_s)
  if (i < d.hd) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 4 <= nv; c += 4) {
#pragma unroll
      for (int u = 0; u < 4; u++) acc[u] += w_s[c + u] * P[(c + u) * cs + i];
    }
    for (; c < nv; c++) acc[0] += w_s[c] * P[c * cs + i];
    store_act(o, (size_t)b * d.q_dim + (size_t)h * d.hd + i, ((acc[0] + acc[1]) + (acc[2] + acc[3])) / L, d.act);
  }
  if (stat && i == 0) {
    stat[((size_t)b * d.Hq + h) * 2] = M;
    stat[((size_t)b * d.Hq + h) * 2 + 1] = L;
  }
}

// KV budget scores (the Initial-Key cache of the C17 engine article, 5.3): the softmax
// probability each cache entry t <= pos of sequence b gets from this step's queries, summed
// over the query heads, added to scores[slot][t].  Grid (B, groups of 4 entries), four
// waves: wave w takes entry 4 * group + w, and the row's queries are staged in LDS.  The
// wave recomputes every q_h . k_t / sqrt(d) from the stored key, the heads side by side
// (P lanes per head, each with a slice of the head dimension), and adds
// exp(s - M_h) / L_h with the merged attention statistics in head order, so every entry's
// sum has one fixed order.  Layers layer0 .. layer0 + nl - 1 in one launch (those from the row's score_from on):
// layer l's queries, keys, scales and statistics sit l strides past layer0's, and each
// layer's sum is added to the entry in layer order by the wave that owns the entry.
struct ScoreLayers {
  int layer0, nl;
  const float* q;      // layer0's [B][q_dim]
  size_t q_ls;         // floats between layers
  KvLayer kv;          // layer0's pools
  size_t k_ls, s_ls;   // bytes of K, fp16 scales between layers
  const float* stat;   // layer0's [B][Hq][2]
  size_t st_ls;        // floats between layers
};
template <int KVFMT>
__global__ __launch_bounds__(256) void k_score(Dims d, const StepDesc* desc, ScoreLayers a, const int32_t* bt,
                                               float* scores) {
  extern __shared__ __attribute__((aligned(16))) float qb[];   // [q_dim] this row's queries of one layer (read as float4)
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.y * 4 + wave;
  const int pos = desc->pos[b], slot = desc->slot[b];
  const bool mine = t <= pos;          // (wave-uniform; waves past the row still take the barriers)
  const float scale = 1.f / sqrtf((float)d.hd);
  int P = 1;                           // lanes per head: a power of 2, P heads' worth fit 64 lanes
  while (2 * P * d.Hq <= 64 && d.hd % (8 * P) == 0) P *= 2;
  const int blk = mine ? bt[(size_t)slot * d.max_blocks + t / d.bs] : 0;
  for (int l = 0; l < a.nl; l++) {
    if (a.layer0 + l < desc->score_from[b]) continue;   // block-uniform
    __syncthreads();                                     // the previous layer's readers are done
    const float* q = a.q + (size_t)l * a.q_ls;
    for (int i = threadIdx.x; i < d.q_dim; i += 256) qb[i] = q[(size_t)b * d.q_dim + i];
    __syncthreads();
    if (!mine) continue;
    const uint8_t* kl = (const uint8_t*)a.kv.k + (size_t)l * a.k_ls;
    const uint16_t* ksl = KVFMT == KV_I8 ? (const uint16_t*)((const uint8_t*)a.kv.ks + (size_t)l * a.s_ls) : nullptr;
    const float* stat = a.stat + (size_t)l * a.st_ls;
    // lane (head h, part) takes dims [part dl, (part + 1) dl) of q_h . k_{h / G}, the P lanes
    // of a head add their parts, and the heads' terms are added in head order
    const int dl = d.hd / P;
    float sum = 0.f;
    for (int h0 = 0; h0 < d.Hq; h0 += 64 / P) {
      const int h = h0 + lane / P, part = lane & (P - 1);
      float p = 0.f;
      if (h < d.Hq) {
        const size_t row = ((size_t)blk * d.Hkv + h / d.G) * d.bs + (t % d.bs);
        const float* qh = qb + (size_t)h * d.hd + part * dl;
        const size_t e0 = row * d.hd + (size_t)part * dl;
        for (int i = 0; i < dl; i += 4) {
          float k4[4];
          if constexpr (KVFMT == KV_F32) {
            const float4 v = *(const float4*)((const float*)kl + e0 + i);
            k4[0] = v.x; k4[1] = v.y; k4[2] = v.z; k4[3] = v.w;
          } else if constexpr (KVFMT == KV_BF16) {
            const uint2 v = *(const uint2*)((const uint16_t*)kl + e0 + i);
            k4[0] = __uint_as_float(v.x << 16); k4[1] = __uint_as_float(v.x & 0xffff0000u);
            k4[2] = __uint_as_float(v.y << 16); k4[3] = __uint_as_float(v.y & 0xffff0000u);
          } else {
            const uint32_t v = *(const uint32_t*)((const int8_t*)kl + e0 + i);
            const float ks = f16_to_f32(ksl[row]);
#pragma unroll
            for (int u = 0; u < 4; u++) k4[u] = sext8(v, u) * ks;
          }
          const float4 q4 = *(const float4*)(qh + i);
          p += q4.x * k4[0] + q4.y * k4[1] + q4.z * k4[2] + q4.w * k4[3];
        }
      }
      for (int m = 1; m < P; m <<= 1) p += __shfl_xor(p, m, 64);
      float e = 0.f;
      if (h < d.Hq) {
        const float M = stat[((size_t)b * d.Hq + h) * 2], L = stat[((size_t)b * d.Hq + h) * 2 + 1];
        e = expf(p * scale - M) / L;
      }
      for (int u = 0; u < 64 / P && h0 + u < d.Hq; u++) sum += __shfl(e, u * P, 64);
    }
    if (lane == 0) scores[(size_t)slot * d.max_ctx + t] += sum;
  }
}

// KV budget eviction in the steady state of decoding (the Initial-Key cache of the C17 engine
// article, 5.3): a step left n = budget + 1 entries, so one goes.  The entry is the middle one
// (index in [n_init, rec0)) with the lowest score sum, the later one among equal sums (the
// earlier entry wins ties).  The kernel records new_pos as the position of entry n - 1 (the
// one the step appended), closes the gap in the score and position rows (entries after it
// move down one place; the freed last score starts again at 0) and writes the kept indices,
// in order, for k_kv_gather.  One block of 1024 threads, no host round trip.
__global__ __launch_bounds__(1024) void k_evict_one(float* scores, int32_t* kvpos, int n, int n_init, int rec0,
                                                    int new_pos, int32_t* keep, const int32_t* fresh, int nb,
                                                    int32_t* bt_row) {
  __shared__ float wbest[16];
  __shared__ int widx[16];
  __shared__ int ev;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t == 0) kvpos[n - 1] = new_pos;
  for (int i = t; i < nb; i += 1024) bt_row[i] = fresh[i];   // the sequence's new blocks
  float best = INFINITY;
  int bi = -1;
  for (int i = n_init + t; i < rec0; i += 1024) {
    const float s = scores[i];
    if (s < best || (s == best && i > bi)) { best = s; bi = i; }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (ob < best || (ob == best && oi > bi)) { best = ob; bi = oi; }
  }
  if (lane == 0) { wbest[wave] = best; widx[wave] = bi; }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < 16; w++)
      if (wbest[w] < best || (wbest[w] == best && widx[w] > bi)) { best = wbest[w]; bi = widx[w]; }
    ev = bi;
  }
  __syncthreads();
  const int e = ev;   // >= n_init: the middle range is never empty at n = budget + 1
  // entries e+1 .. n-1 move down one place, 1024 at a time: every chunk reads its sources
  // before any of them is overwritten by the next chunk
  for (int base = e; base < n - 1; base += 1024) {
    const int i = base + t;
    float sv = 0.f;
    int pv = 0;
    if (i < n - 1) { sv = scores[i + 1]; pv = kvpos[i + 1]; }
    __syncthreads();
    if (i < n - 1) { scores[i] = sv; kvpos[i] = pv; }
    __syncthreads();
  }
  if (t == 0) scores[n - 1] = 0.f;
  for (int i = t; i < n - 1; i += 1024) keep[i] = i < e ? i : i + 1;
}

// KV budget eviction: copies cache entries keep[i] (i < n, through the old block list) to
// entry i (through the new block list) in every layer: K and V rows and int8 scales.  Grid
// (layers, n); one block per (layer, entry).
__global__ __launch_bounds__(128) void k_kv_gather(const PLayer* layers, int Hkv, int bs, int hd, int elem,
                                                   const int32_t* old_blocks, const int32_t* new_blocks,
                                                   const int32_t* keep) {
  const KvLayer kv = layers[blockIdx.x].kv;
  const int i = blockIdx.y, t = keep[i];
  const int ob = old_blocks[t / bs], nb = new_blocks[i / bs];
  const size_t rowb = (size_t)hd * elem;
  const bool wide = rowb % 16 == 0;          // rows of 16-byte pieces (every row starts aligned)
  const size_t pieces = wide ? rowb / 16 : rowb;
  for (size_t x = threadIdx.x; x < (size_t)Hkv * pieces; x += 128) {
    const int j = (int)(x / pieces);
    const size_t p = x - (size_t)j * pieces;
    const size_t src = ((size_t)ob * Hkv + j) * bs + (t % bs), dst = ((size_t)nb * Hkv + j) * bs + (i % bs);
    if (wide) {
      ((uint4*)kv.k)[dst * pieces + p] = ((const uint4*)kv.k)[src * pieces + p];
      ((uint4*)kv.v)[dst * pieces + p] = ((const uint4*)kv.v)[src * pieces + p];
    } else {
      ((uint8_t*)kv.k)[dst * rowb + p] = ((const uint8_t*)kv.k)[src * rowb + p];
      ((uint8_t*)kv.v)[dst * rowb + p] = ((const uint8_t*)kv.v)[src * rowb + p];
    }
    if (kv.ks && p == 0) {
      kv.ks[dst] = kv.ks[src];
      kv.vs[dst] = kv.vs[src];
    }
  }
}

// S11 greedy argmax over the fp32 logits, lowest index among equal maxima
__global__ __launch_bounds__(1024) void k_argmax(const float* logits, int V, const StepDesc* desc) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int b = blockIdx.x;
  const float* L = logits + (size_t)b * V;
  float best = -INFINITY;
  int idx = INT_MAX;
  auto take = [&](float x, int v) {
    if (x > best || (idx == INT_MAX && !isnan(x))) { best = x; idx = v; }
  };
  // a thread's entries in ascending order: 16-byte pieces t, t + 1024, ... (four loads in
  // flight), then the tail past the last whole piece
  const int nq = (V & 3) == 0 ? V >> 2 : 0;
  for (int q0 = threadIdx.x; q0 < nq; q0 += 4 * 1024) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int q = q0 + u * 1024;
      x[u] = q < nq ? *(const float4*)(L + 4 * (size_t)q) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int q = q0 + u * 1024;
      if (q < nq) {
        take(x[u].x, 4 * q);
        take(x[u].y, 4 * q + 1);
        take(x[u].z, 4 * q + 2);
        take(x[u].w, 4 * q + 3);
      }
    }
  }
  for (int v = 4 * nq + (int)threadIdx.x; v < V; v += 1024) take(L[v], v);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(idx, m, 64);
    if (ob > best || (ob == best && oi < idx)) { best = ob; idx = oi; }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { bv[wave] = best; bi[wave] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; w++)
      if (bv[w] > best || (bv[w] == best && bi[w] < idx)) { best = bv[w]; idx = bi[w]; }
    desc->next_tokens[b] = idx == INT_MAX ? 0 : idx;
  }
}

__global__ __launch_bounds__(256) void k_dequant_rows(Dims d, MatDev m, const int32_t* rows,
                                                      float* out) {
  const int r = blockIdx.x, sr = rows[r];
  for (int c = threadIdx.x; c < m.cols; c += 256)
    out[(size_t)r * m.cols + c] = deq_elem(m, d.wfmt, sr, c);
}

// Streaming-read ceiling probe: reads n 16-byte vectors with nontemporal loads, four in
// flight per thread, grid-stride, and folds them by XOR.  The fold is stored only when it
// equals `never` (a value the caller picks), so the loads cannot be dropped.
__global__ __launch_bounds__(256) void k_stream_read(const uint4* p, size_t n, uint32_t never, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = gload_stream<uint4>(p + i), b = gload_stream<uint4>(p + i + stride);
    const uint4 c = gload_stream<uint4>(p + i + 2 * stride), d = gload_stream<uint4>(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const uint4 a = gload_stream<uint4>(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) sink[0] = acc;
}

// counter-based hash (splitmix64 finaliser) for synthetic KV contents
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void k_kv_fill(Dims d, KvLayer kv, const int32_t* blocks, int len,
                                                 int layer, uint64_t seed) {
  const int bi = blockIdx.x, j = blockIdx.y;
  const int blk = blocks[bi];
  const float amp = 0.02f * sqrtf((float)d.D) * 1.7320508f;  // uniform(-amp, amp) has sd 0.02*sqrt(D)
  for (int e = threadIdx.x; e < d.bs * d.hd; e += 256) {
    const int off = e / d.hd, i = e - off * d.hd, t = bi * d.bs + off;
    if (t >= len) continue;
    const size_t row = ((size_t)blk * d.Hkv + j) * d.bs + off;
    for (int which = 0; which < 2; which++) {
      const uint64_t h = mix64(seed ^ mix64(((uint64_t)layer << 40) ^ ((uint64_t)t << 20) ^
                                            ((uint64_t)j << 12) ^ ((uint64_t)i << 1) ^ (uint64_t)which));
      const float u = (float)(h >> 40) * (1.0f / 16777216.0f) * 2.f - 1.f;
      void* pool = which ? kv.v : kv.k;
      if (d.kvfmt == KV_F32) ((float*)pool)[row * d.hd + i] = u * amp;
      else if (d.kvfmt == KV_BF16) ((uint16_t*)pool)[row * d.hd + i] = f32_to_bf16(u * amp);
      else {
        ((int8_t*)pool)[row * d.hd + i] = (int8_t)rintf(u * 127.f);
        if (i == 0) (which ? kv.vs : kv.ks)[row] = f32_to_f16(amp / 127.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Prefill attention: the causal attention of a chunk of n consecutive positions p0 .. p0+n-1
// of one sequence, every one of whose K/V entries is already in the cache.  Blocked with an
// online softmax, FlashAttention-2 style (the Qwen3-8B engine article, 4.4.1; lightLLM's
// context_flashattention_nopad): a workgroup takes 16 query positions, up to 4 query heads
// of one KV head (one head per wave) and one chunk of the keys (the decode attention's chunk
// length, a multiple of 64), and walks the chunk's keys up to its last position in tiles of
// 64 staged once in LDS for all its waves, so each K/V row is read once per 16 positions
// rather than once per position.  Each (position, head, chunk) leaves an unnormalised partial
// (O, max, sum) in the decode attention's layout, and k_combine merges a position's chunks
// exactly as it does after a decode step.
//
// Both products run on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) at
// fp32 accuracy: an fp32 operand x enters as three bf16 terms, hi = bf16(x),
// mid = bf16(x - hi), lo = bf16(x - hi - mid), which carry x to 2^-24 relative, and every
// product of terms whose weights add to at least 2^-24 is taken (hi hi, hi mid, mid hi,
// hi lo, mid mid, lo hi).  bf16 or int8 K/V is exact in bf16 (one term), so S = Q K^T
// takes three products and O += P V three.  int8 K/V keep their per-entry scales outside
// the products: the K scale multiplies its score column, the V scale its probability
// column.  The scores of a tile leave the MFMA with a row's keys spread over 16 lanes; P goes
// through LDS to reach the operand layout of the second product.
// ---------------------------------------------------------------------------------------

constexpr int kPfQ = 16;   // query positions per workgroup
constexpr int kPfT = 64;   // keys per staged tile

struct PfLayout {
  int hdp, kld, vld, pld;                    // head size padded to 32; LDS row pitches
  size_t k[3], v[3], ksc, vsc, p, bytes;     // terms of K (hi, mid, lo) and of V
};

// K tile [64][kld] bf16 and V tile transposed [hdp][vld] bf16, three terms each for fp32
// K/V and one otherwise; int8 scales [64] each; each wave's P [16][pld] fp32
__host__ __device__ inline PfLayout pf_layout(int hd, int kvfmt) {
  PfLayout L;
  L.hdp = (hd + 31) / 32 * 32;
  L.kld = L.hdp + 8;
  L.vld = kPfT + 8;
  L.pld = kPfT + 4;
  const int terms = kvfmt == KV_F32 ? 3 : 1;
  size_t o = 0;
  for (int u = 0; u < 3; u++) { L.k[u] = o; if (u < terms) o += (size_t)kPfT * L.kld * 2; }
  for (int u = 0; u < 3; u++) { L.v[u] = o; if (u < terms) o += (size_t)L.hdp * L.vld * 2; }
  L.ksc = o; o += kPfT * 4;
  L.vsc = o; o += kPfT * 4;
  L.p = o; o += (size_t)4 * kPfQ * L.pld * 4;
  L.bytes = o;
  return L;
}

// sum or max over the 16 lanes of a lane's row group (lanes l ^ 1, 2, 4, 8): every lane of
// the group gets the same result
__device__ __forceinline__ float grp16_sum(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float grp16_max(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// K/V element e of a pool, as fp32 (int8: the code; its scale is applied apart)
template <int KVFMT>
__device__ __forceinline__ float kv_raw(const void* pool, size_t e) {
  if constexpr (KVFMT == KV_F32) return ((const float*)pool)[e];
  else if constexpr (KVFMT == KV_BF16) return bf16_to_f32(((const uint16_t*)pool)[e]);
  else return (float)((const int8_t*)pool)[e];
}

// 8 consecutive elements from e (a multiple-of-8 head size: aligned vector loads)
template <int KVFMT>
__device__ __forceinline__ void kv_raw8(const void* pool, size_t e, float (&x)[8]) {
  if constexpr (KVFMT == KV_F32) {
    const float4 a = *(const float4*)((const float*)pool + e), b = *(const float4*)((const float*)pool + e + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else if constexpr (KVFMT == KV_BF16) {
    const uint4 a = *(const uint4*)((const uint16_t*)pool + e);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int u = 0; u < 4; u++) { x[2 * u] = bf16_to_f32(w[u] & 0xffffu); x[2 * u + 1] = bf16_to_f32(w[u] >> 16); }
  } else {
    const uint2 a = *(const uint2*)((const int8_t*)pool + e);
#pragma unroll
    for (int u = 0; u < 4; u++) { x[u] = sext8(a.x, u); x[4 + u] = sext8(a.y, u); }
  }
}

template <int KVFMT>
__global__ __launch_bounds__(256) void k_attn_prefill(Dims d, const StepDesc* desc, int n, const float* q,
                                                      KvLayer kv, const int32_t* bt, float* partials) {
  extern __shared__ __attribute__((aligned(16))) uint8_t pf_sm[];
  constexpr int NT = KVFMT == KV_F32 ? 3 : 1;   // bf16 terms of a K/V element
  const PfLayout Ly = pf_layout(d.hd, KVFMT);
  uint16_t* kt[3];
  uint16_t* vt[3];
#pragma unroll
  for (int u = 0; u < 3; u++) { kt[u] = (uint16_t*)(pf_sm + Ly.k[u]); vt[u] = (uint16_t*)(pf_sm + Ly.v[u]); }
  float* ksc = (float*)(pf_sm + Ly.ksc);
  float* vsc = (float*)(pf_sm + Ly.vsc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* pw = (float*)(pf_sm + Ly.p) + (size_t)wave * kPfQ * Ly.pld;
  const int hd = d.hd, HDP = Ly.hdp, G = d.G;
  const int ngz = (G + 3) / 4;
  const int j = blockIdx.x / ngz, g = (blockIdx.x - j * ngz) * 4 + wave;
  const bool active = g < G;                 // wave-uniform
  const int h = j * G + (active ? g : 0);
  const int c = blockIdx.y, i0 = blockIdx.z * kPfQ;
  const int p0 = desc->pos[0], slot = desc->slot[0];
  const int last = p0 + min(n, i0 + kPfQ) - 1;   // the last key any row of this block attends
  const int k_lo = c * d.ct, k_hi = min(last + 1, k_lo + d.ct);   // this block's keys
  if (k_lo > last) return;                       // (block-uniform) a chunk past every row
  const int* btrow = bt + (size_t)slot * d.max_blocks;
  const int r16 = lane & 15, quad = lane >> 4;

  // this wave's queries / sqrt(d) as A operands: row r16 (position i0 + r16; rows past the
  // chunk repeat its last query and are never stored), k = 32 s + 8 quad + u
  bf16x8 qa[4][3];
  {
    const float inv = 1.f / sqrtf((float)hd);
    const float* qr = q + (size_t)min(i0 + r16, n - 1) * d.q_dim + (size_t)h * hd;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int dd = 32 * s + 8 * quad + u;
        x[u] = dd < hd ? qr[dd] * inv : 0.f;
      }
      split8(x, qa[s]);
    }
  }
  f32x4 oacc[8];   // O: d-blocks of 16 (head size <= 128)
#pragma unroll
  for (int db = 0; db < 8; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[4], l[4];   // running max and sum of rows 4 quad + i
#pragma unroll
  for (int i = 0; i < 4; i++) { m[i] = -INFINITY; l[i] = 0.f; }

  const int pieces = HDP / 8;
  for (int t0 = k_lo; t0 < k_hi; t0 += kPfT) {
    __syncthreads();   // every wave is done with the previous tile and its P
    // ---- stage keys t0 .. t0+63 of KV head j; zeros past `last` and past the head size ----
    for (int idx = tid; idx < kPfT * pieces; idx += 256) {
      const int kr = idx / pieces, d0 = (idx - kr * pieces) * 8, t = t0 + kr;
      float kx[8], vx[8];
#pragma unroll
      for (int u = 0; u < 8; u++) { kx[u] = 0.f; vx[u] = 0.f; }
      float ks = 0.f, vs = 0.f;
      if (t < k_hi && d0 < hd) {
        const int blk = btrow[t / d.bs];
        const size_t row = ((size_t)blk * d.Hkv + j) * d.bs + (t % d.bs);
        if ((hd & 7) == 0) {
          kv_raw8<KVFMT>(kv.k, row * hd + d0, kx);
          kv_raw8<KVFMT>(kv.v, row * hd + d0, vx);
        } else {
#pragma unroll
          for (int u = 0; u < 8; u++)
            if (d0 + u < hd) {
              kx[u] = kv_raw<KVFMT>(kv.k, row * hd + d0 + u);
              vx[u] = kv_raw<KVFMT>(kv.v, row * hd + d0 + u);
            }
        }
        if constexpr (KVFMT == KV_I8) {
          ks = f16_to_f32(kv.ks[row]);
          vs = f16_to_f32(kv.vs[row]);
        }
      }
      if constexpr (KVFMT == KV_I8) {
        if (d0 == 0) { ksc[kr] = ks; vsc[kr] = vs; }
      }
      bf16x8 kb8[3];
      split8(kx, kb8);
#pragma unroll
      for (int s = 0; s < NT; s++) *(bf16x8*)(kt[s] + (size_t)kr * Ly.kld + d0) = kb8[s];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        uint32_t vv[3];
        split3(vx[u], vv);
#pragma unroll
        for (int s = 0; s < NT; s++) vt[s][(size_t)(d0 + u) * Ly.vld + kr] = (uint16_t)vv[s];
      }
    }
    __syncthreads();
    // ---- S = Q K^T, the online softmax, P to LDS ----
    float al[4];
    if (active) {
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; kb++) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; s++) {
        if (32 * s >= HDP) break;
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
          const size_t at = (size_t)(16 * kb + r16) * Ly.kld + 32 * s + 8 * quad;
          bf16x8 kb8[3];
#pragma unroll
          for (int u = 0; u < NT; u++) kb8[u] = *(const bf16x8*)(kt[u] + at);
          sacc[kb] = mfma_terms<3, NT>(qa[s], kb8, sacc[kb]);
        }
      }
      // lane: rows 4 quad + i, key t0 + 16 kb + r16
      float mx[4];
#pragma unroll
      for (int i = 0; i < 4; i++) mx[i] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        const int key = t0 + 16 * kb + r16;
        const float kscale = KVFMT == KV_I8 ? ksc[16 * kb + r16] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int pos = p0 + i0 + 4 * quad + i;
          const float s = sacc[kb][i] * kscale;
          sacc[kb][i] = (key <= pos && key < k_hi) ? s : -INFINITY;
          mx[i] = fmaxf(mx[i], sacc[kb][i]);
        }
      }
      // a row none of whose keys so far is in range keeps max -inf; its terms use 0 in its
      // place (every exponential is then of -inf: 0), and its partial is never read
      float ps[4], base[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float mn = fmaxf(m[i], grp16_max(mx[i]));
        base[i] = mn == -INFINITY ? 0.f : mn;
        al[i] = expf(m[i] - base[i]);
        m[i] = mn;
        ps[i] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        const float vscale = KVFMT == KV_I8 ? vsc[16 * kb + r16] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float p = expf(sacc[kb][i] - base[i]);
          ps[i] += p;
          pw[(4 * quad + i) * Ly.pld + 16 * kb + r16] = p * vscale;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; i++) l[i] = l[i] * al[i] + grp16_sum(ps[i]);
    }
    __syncthreads();   // P is in LDS (the barrier also orders the wave's own writes and reads)
    // ---- O = O * alpha + P V ----
    if (active) {
#pragma unroll
      for (int db = 0; db < 8; db++)
#pragma unroll
        for (int i = 0; i < 4; i++) oacc[db][i] *= al[i];
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const float* pr = pw + r16 * Ly.pld + 32 * ks + 8 * quad;
        const float4 a0 = *(const float4*)pr, a1 = *(const float4*)(pr + 4);
        const float px[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bf16x8 pa[3];
        split8(px, pa);
#pragma unroll
        for (int db = 0; db < 8; db++) {
          if (16 * db >= HDP) break;
          const size_t at = (size_t)(16 * db + r16) * Ly.vld + 32 * ks + 8 * quad;
          bf16x8 vb8[3];
#pragma unroll
          for (int u = 0; u < NT; u++) vb8[u] = *(const bf16x8*)(vt[u] + at);
          oacc[db] = mfma_terms<3, NT>(pa, vb8, oacc[db]);
        }
      }
    }
  }
  if (!active) return;
  // ---- the partial (O, max, sum) of every row whose position reaches this chunk ----
  const int cs = hd + 2;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int b = i0 + 4 * quad + i;
    if (b >= n || p0 + b < k_lo) continue;
    float* P = partials + (((size_t)b * d.Hq + h) * d.nch + c) * cs;
#pragma unroll
    for (int db = 0; db < 8; db++) {
      const int dd = 16 * db + r16;
      if (dd < hd) P[dd] = oacc[db][i];
    }
    if (r16 == 0) {
      P[hd] = m[i];
      P[hd + 1] = l[i];
    }
  }
}

// ---------------------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------------------

template <int WFMT, int EPI>
hipError_t gemv_dispatch(const GemvArgs& a, int NB, int ROWS, dim3 grid, size_t smem, hipStream_t st) {
  if constexpr (WFMT == W_Q4_0) {
    // one 16-byte load covers 32 columns: eight rows per wave keep enough bytes in flight
    if (NB == 1 && ROWS == 8) {
      hipLaunchKernelGGL((k_gemv<WFMT, EPI, 1, 8>), grid, dim3(256), smem, st, a);
      return hipGetLastError();
    }
  }
  if (NB == 1 && ROWS == 2) hipLaunchKernelGGL((k_gemv<WFMT, EPI, 1, 2>), grid, dim3(256), smem, st, a);
  else if (NB == 1 && ROWS == 4) hipLaunchKernelGGL((k_gemv<WFMT, EPI, 1, 4>), grid, dim3(256), smem, st, a);
  else if (NB == 4 && ROWS == 2) hipLaunchKernelGGL((k_gemv<WFMT, EPI, 4, 2>), grid, dim3(256), smem, st, a);
  else hipLaunchKernelGGL((k_gemv<WFMT, EPI, 4, 4>), grid, dim3(256), smem, st, a);
  return hipGetLastError();
}

template <int WFMT>
hipError_t gemv_epi(const GemvArgs& a, int epi, int NB, int ROWS, dim3 grid, size_t smem, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return gemv_dispatch<WFMT, EPI_QKV>(a, NB, ROWS, grid, smem, st);
    case EPI_RESID: return gemv_dispatch<WFMT, EPI_RESID>(a, NB, ROWS, grid, smem, st);
    case EPI_SWIGLU: return gemv_dispatch<WFMT, EPI_SWIGLU>(a, NB, ROWS, grid, smem, st);
    default: return gemv_dispatch<WFMT, EPI_LOGITS>(a, NB, ROWS, grid, smem, st);
  }
}


// Lets an instantiation use more than the default 64 KB of dynamic LDS (once per kernel).
template <int WFMT, int EPI, int NBB>
hipError_t gemm_lds_limit(size_t smem) {
  static const hipError_t r = hipFuncSetAttribute((const void*)k_gemm<WFMT, EPI, NBB>,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  return r;
}

template <int WFMT, int EPI>
hipError_t gemm_dispatch(const GemmArgs& a, int nbb, dim3 grid, size_t smem, hipStream_t st, bool reduce = true) {
  hipError_t r = hipSuccess;
  switch (nbb) {
    case 1: hipLaunchKernelGGL((k_gemm<WFMT, EPI, 1>), grid, dim3(256), smem, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<WFMT, EPI, 2>), grid, dim3(256), smem, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<WFMT, EPI, 3>), grid, dim3(256), smem, st, a); break;
    default:
      if ((r = gemm_lds_limit<WFMT, EPI, 4>(smem)) != hipSuccess) return r;
      hipLaunchKernelGGL((k_gemm<WFMT, EPI, 4>), grid, dim3(256), smem, st, a);
      break;
  }
  r = hipGetLastError();
  if (r != hipSuccess || a.S == 1 || !reduce) return r;
  const int threads = (a.g.m.rows + 3) / 4 * a.g.B;
  hipLaunchKernelGGL((k_gemm_reduce<WFMT, EPI>), dim3((threads + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int WFMT>
hipError_t gemm_epi(const GemmArgs& a, int epi, int nbb, dim3 grid, size_t smem, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return gemm_dispatch<WFMT, EPI_QKV>(a, nbb, grid, smem, st);
    case EPI_RESID: return gemm_dispatch<WFMT, EPI_RESID>(a, nbb, grid, smem, st);
    case EPI_SWIGLU: return gemm_dispatch<WFMT, EPI_SWIGLU>(a, nbb, grid, smem, st);
    default: return gemm_dispatch<WFMT, EPI_LOGITS>(a, nbb, grid, smem, st);
  }
}

}  // namespace

bool gemm_eligible(const Dims& d, int B) {
  return B >= 2 && B <= kMaxBatch && d.act == ACT_BF16 && (d.wfmt == W_INT8_ROW || d.wfmt == W_BF16);
}

// K splits: about one workgroup per compute unit; where that leaves some compute units with
// two workgroups and the rest with one, as many as give every compute unit two.  (Two per
// compute unit everywhere measured slower: the larger partial sums cost more than they
// gained; the uneven count, 288 workgroups of the Qwen3-8B QKV matrix, cost 1.6%.)
int gemm_splits(int N, int K, int cus) {
  const int tiles = (N + kGemmRows - 1) / kGemmRows;
  const int nchunk = (K + kGemmKC - 1) / kGemmKC;
  if (tiles >= cus) return 1;
  int S = (cus + tiles - 1) / tiles;
  if (tiles * S > cus) S = 2 * cus / tiles;
  return S < nchunk ? S : nchunk;
}

size_t gemm_partial_bytes(const Dims& d, int B, int cus) {
  size_t m = 0;
  const int shapes[5][2] = {{d.qkv_rows, d.D}, {d.D, d.q_dim}, {2 * d.F, d.D}, {d.D, d.F}, {d.V, d.D}};
  for (const auto& sh : shapes) {
    const int S = gemm_splits(sh[0], sh[1], cus);
    if (S > 1) m = std::max(m, (size_t)S * B * sh[0] * sizeof(float));
  }
  return m;
}

hipError_t launch_gemm(const Dims& d, const MatDev& m, const void* xin, int B, int epi, const EpiArgs& ea,
                       float* partials, int cus, hipStream_t st) {
  GemmArgs a;
  a.g.d = d;
  a.g.m = m;
  a.g.xin = xin;
  a.g.B = B;
  a.g.act_in = d.act;
  a.g.kc = 0;
  a.g.ea = ea;
  a.partials = partials;
  a.S = gemm_splits(m.rows, m.cols, cus);
  a.nchunk = (m.cols + kGemmKC - 1) / kGemmKC;
  const int nbb = (B + 15) / 16;
  const dim3 grid((m.rows + kGemmRows - 1) / kGemmRows, a.S);
  const size_t smem = 2 * (size_t)16 * nbb * kGemmLd;
  if (d.wfmt == W_INT8_ROW) return gemm_epi<W_INT8_ROW>(a, epi, nbb, grid, smem, st);
  return gemm_epi<W_BF16>(a, epi, nbb, grid, smem, st);
}

hipError_t launch_gemm_resid_norm(const Dims& d, const MatDev& m, const void* xin, int B, const EpiArgs& ea,
                                  float* partials, int cus, const float* g, void* xn, hipStream_t st) {
  const int S = gemm_splits(m.rows, m.cols, cus);
  if (S == 1 || m.rows != d.D || d.D % 4 || d.D > kNormPieces * 4 * kNormThreads) {
    const hipError_t r = launch_gemm(d, m, xin, B, EPI_RESID, ea, partials, cus, st);
    return r != hipSuccess ? r : launch_rmsnorm(d, ea.x, g, xn, B, st);
  }
  GemmArgs a;
  a.g.d = d;
  a.g.m = m;
  a.g.xin = xin;
  a.g.B = B;
  a.g.act_in = d.act;
  a.g.kc = 0;
  a.g.ea = ea;
  a.partials = partials;
  a.S = S;
  a.nchunk = (m.cols + kGemmKC - 1) / kGemmKC;
  const int nbb = (B + 15) / 16;
  const dim3 grid((m.rows + kGemmRows - 1) / kGemmRows, a.S);
  const size_t smem = 2 * (size_t)16 * nbb * kGemmLd;
  // the GEMM with its split-K partial sums only (the reduce below runs the epilogue)
  hipError_t r;
  if (d.wfmt == W_INT8_ROW) {
    r = gemm_dispatch<W_INT8_ROW, EPI_RESID>(a, nbb, grid, smem, st, false);
    if (r == hipSuccess) hipLaunchKernelGGL(k_gemm_reduce_norm<W_INT8_ROW>, dim3(B), dim3(kNormThreads), 0, st, a, g, xn);
  } else {
    r = gemm_dispatch<W_BF16, EPI_RESID>(a, nbb, grid, smem, st, false);
    if (r == hipSuccess) hipLaunchKernelGGL(k_gemm_reduce_norm<W_BF16>, dim3(B), dim3(kNormThreads), 0, st, a, g, xn);
  }
  return r != hipSuccess ? r : hipGetLastError();
}

hipError_t launch_embed(const Dims& d, const MatDev& emb, const StepDesc* desc, int B,
                        int32_t* block_table, float* x, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(B), dim3(1024), 0, st, d, emb, desc, block_table, x, err);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const Dims& d, const float* x, const float* g, void* xn, int B,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kNormThreads), 0, st, x, g, xn, d.D, d.eps, d.act);
  return hipGetLastError();
}

hipError_t launch_gemv(const Dims& d, const MatDev& m, const void* xin, int B, int epi,
                       const EpiArgs& ea, hipStream_t st) {
  GemvArgs a;
  a.d = d;
  a.m = m;
  a.xin = xin;
  a.B = B;
  a.act_in = d.act;
  a.ea = ea;
  const int NB = B == 1 ? 1 : 4;
  const int ROWS = (d.wfmt == W_Q4_0 && B == 1 && m.rows >= 8 * 4 * 256) ? 8 : (m.rows >= 4 * 16 * 256 ? 4 : 2);
  const int VEC = d.wfmt == W_BF16 ? 8 : (d.wfmt == W_Q4_0 ? 32 : 16), KSTEP = 64 * VEC;
  const int budget_floats = 16384;  // 64 KiB of LDS
  int kc = (budget_floats / NB) / KSTEP * KSTEP;
  const int kpad = (m.cols + KSTEP - 1) / KSTEP * KSTEP;
  if (kc > kpad) kc = kpad;
  a.kc = kc;
  const dim3 grid((m.rows + 4 * ROWS - 1) / (4 * ROWS), (B + NB - 1) / NB);
  const size_t smem = sizeof(float) * (size_t)NB * kc;
  switch (d.wfmt) {
    case W_INT8_ROW: return gemv_epi<W_INT8_ROW>(a, epi, NB, ROWS, grid, smem, st);
    case W_Q8_0: return gemv_epi<W_Q8_0>(a, epi, NB, ROWS, grid, smem, st);
    case W_Q4_0: return gemv_epi<W_Q4_0>(a, epi, NB, ROWS, grid, smem, st);
    default: return gemv_epi<W_BF16>(a, epi, NB, ROWS, grid, smem, st);
  }
}

bool attn_w_shape(const Dims& d) {
  // the instantiations launch_attention dispatches to k_attn_w
  if (d.bs != 16) return false;
  if (d.hd == 128 || d.hd == 64) return d.G == 4;
  return d.hd == 32 && d.G == 5 && d.kvfmt != KV_I8;
}

hipError_t launch_attention(const Dims& d, const StepDesc* desc, int B, int n_chunks, const float* q,
                            const float* knew, const float* vnew, const KvLayer& kv,
                            const int32_t* block_table, float* partials, hipStream_t st) {
  AttnCtx a;
  a.d = d;
  a.q = q;
  a.knew = knew;
  a.vnew = vnew;
  a.kv = kv;
  a.bt = block_table;
  a.ct = d.ct;
  a.nch = d.nch;
  if (attn_w_shape(d)) {
    if (n_chunks <= 0) return hipSuccess;
    const dim3 gw((n_chunks + 3) / 4, d.Hkv, 1);
#define DTD_ATTN_W(KV, HDv, Gv)                                                                   \
  if (d.kvfmt == KV && d.hd == HDv && d.G == Gv) {                                                \
    hipLaunchKernelGGL((k_attn_w<KV, HDv, Gv>), gw, dim3(256), 0, st, a, desc, partials);         \
    return hipGetLastError();                                                                     \
  }
    DTD_ATTN_W(KV_BF16, 128, 4)
    DTD_ATTN_W(KV_I8, 128, 4)
    DTD_ATTN_W(KV_F32, 128, 4)
    DTD_ATTN_W(KV_BF16, 64, 4)
    DTD_ATTN_W(KV_I8, 64, 4)
    DTD_ATTN_W(KV_F32, 64, 4)
    DTD_ATTN_W(KV_BF16, 32, 5)
    DTD_ATTN_W(KV_F32, 32, 5)
#undef DTD_ATTN_W
  }
  const dim3 grid(d.nch, d.Hkv, B);
  const size_t smem = sizeof(float) * attn_smem_floats(d.G, d.hd);
  if (d.kvfmt == KV_F32) hipLaunchKernelGGL(k_attn<KV_F32>, grid, dim3(256), smem, st, a, desc, partials);
  else if (d.kvfmt == KV_BF16) hipLaunchKernelGGL(k_attn<KV_BF16>, grid, dim3(256), smem, st, a, desc, partials);
  else hipLaunchKernelGGL(k_attn<KV_I8>, grid, dim3(256), smem, st, a, desc, partials);
  return hipGetLastError();
}

hipError_t launch_kv_append(const Dims& d, const StepDesc* desc, int B, const float* knew, const float* vnew,
                            const KvLayer& kv, hipStream_t st) {
  const dim3 grid(B, d.Hkv);
  if (d.kvfmt == KV_F32) hipLaunchKernelGGL(k_kv_append<KV_F32>, grid, dim3(128), 0, st, d, kv, desc, knew, vnew);
  else if (d.kvfmt == KV_BF16) hipLaunchKernelGGL(k_kv_append<KV_BF16>, grid, dim3(128), 0, st, d, kv, desc, knew, vnew);
  else hipLaunchKernelGGL(k_kv_append<KV_I8>, grid, dim3(128), 0, st, d, kv, desc, knew, vnew);
  return hipGetLastError();
}

hipError_t launch_kv_copy_block(const Dims& d, const PLayer* layers, int src, int dst, hipStream_t st) {
  const int elem = d.kvfmt == KV_F32 ? 4 : (d.kvfmt == KV_BF16 ? 2 : 1);
  hipLaunchKernelGGL(k_kv_copy_block, dim3(d.L, 4), dim3(256), 0, st, layers, d.Hkv, d.bs, d.hd, elem, src, dst);
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const StepDesc* desc, int B, const float* partials,
                          void* o, hipStream_t st, float* stat) {
  const int nt = (d.hd + 63) / 64 * 64;
  hipLaunchKernelGGL(k_combine, dim3(d.Hq, B), dim3(nt), (size_t)d.nch * 4, st, d, desc, partials, o, stat);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const Dims& d, const StepDesc* desc, int n, int last_pos, const float* q,
                               const KvLayer& kv, const int32_t* bt, float* partials, hipStream_t st) {
  const PfLayout L = pf_layout(d.hd, d.kvfmt);
  const dim3 grid(d.Hkv * ((d.G + 3) / 4), last_pos / d.ct + 1, (n + kPfQ - 1) / kPfQ);
  const void* fn = d.kvfmt == KV_F32 ? (const void*)k_attn_prefill<KV_F32>
                   : d.kvfmt == KV_BF16 ? (const void*)k_attn_prefill<KV_BF16> : (const void*)k_attn_prefill<KV_I8>;
  // above 64 KB of LDS a kernel needs the attribute (fp32 K/V at head size 128: about 125 KB)
  static bool raised[3] = {false, false, false};
  if (L.bytes > 65536 && !raised[d.kvfmt]) {
    const hipError_t r = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.bytes);
    if (r != hipSuccess) return r;
    raised[d.kvfmt] = true;
  }
  if (d.kvfmt == KV_F32) hipLaunchKernelGGL(k_attn_prefill<KV_F32>, grid, dim3(256), L.bytes, st, d, desc, n, q, kv, bt, partials);
  else if (d.kvfmt == KV_BF16) hipLaunchKernelGGL(k_attn_prefill<KV_BF16>, grid, dim3(256), L.bytes, st, d, desc, n, q, kv, bt, partials);
  else hipLaunchKernelGGL(k_attn_prefill<KV_I8>, grid, dim3(256), L.bytes, st, d, desc, n, q, kv, bt, partials);
  return hipGetLastError();
}

hipError_t launch_score(const Dims& d, const StepDesc* desc, int B, int max_pos, int layer0, int nl, const float* q,
                        size_t q_ls, const KvLayer& kv, size_t k_ls, size_t s_ls, const int32_t* bt, const float* stat,
                        size_t st_ls, float* scores, hipStream_t st) {
  if (nl <= 0) return hipSuccess;
  ScoreLayers a{layer0, nl, q, q_ls, kv, k_ls, s_ls, stat, st_ls};
  const dim3 grid(B, (max_pos + 1 + 3) / 4);
  const size_t smem = (size_t)d.q_dim * 4;
  if (d.kvfmt == KV_F32) hipLaunchKernelGGL(k_score<KV_F32>, grid, dim3(256), smem, st, d, desc, a, bt, scores);
  else if (d.kvfmt == KV_BF16) hipLaunchKernelGGL(k_score<KV_BF16>, grid, dim3(256), smem, st, d, desc, a, bt, scores);
  else hipLaunchKernelGGL(k_score<KV_I8>, grid, dim3(256), smem, st, d, desc, a, bt, scores);
  return hipGetLastError();
}

hipError_t launch_evict_one(float* scores, int32_t* kvpos, int n, int n_init, int rec0, int new_pos, int32_t* keep,
                            const int32_t* fresh, int nb, int32_t* bt_row, hipStream_t st) {
  hipLaunchKernelGGL(k_evict_one, dim3(1), dim3(1024), 0, st, scores, kvpos, n, n_init, rec0, new_pos, keep, fresh,
                     nb, bt_row);
  return hipGetLastError();
}

hipError_t launch_kv_gather(const Dims& d, const PLayer* layers, const int32_t* old_blocks, const int32_t* new_blocks,
                            const int32_t* keep, int n, hipStream_t st) {
  const int elem = d.kvfmt == KV_F32 ? 4 : (d.kvfmt == KV_BF16 ? 2 : 1);
  hipLaunchKernelGGL(k_kv_gather, dim3(d.L, n), dim3(128), 0, st, layers, d.Hkv, d.bs, d.hd, elem, old_blocks,
                     new_blocks, keep);
  return hipGetLastError();
}

hipError_t launch_argmax(const Dims& d, const StepDesc* desc, int B, const float* logits,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(B), dim3(1024), 0, st, logits, d.V, desc);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const Dims& d, const MatDev& m, const int32_t* rows, int nrows,
                               float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_dequant_rows, dim3(nrows), dim3(256), 0, st, d, m, rows, out);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int cus, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(cus * 16), dim3(256), 0, st, (const uint4*)buf, bytes / 16,
                     0xA5C3E1F7u, sink);
  return hipGetLastError();
}

hipError_t launch_kv_fill(const Dims& d, const KvLayer& kv, const int32_t* blocks, int nblk_used,
                          int len, int layer, uint64_t seed, hipStream_t st) {
  hipLaunchKernelGGL(k_kv_fill, dim3(nblk_used, d.Hkv), dim3(256), 0, st, d, kv, blocks, len, layer,
                     seed);
  return hipGetLastError();
}

}  // namespace dtd
