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

__global__ __launch_bounds__(256) void k_embed(Dims d, MatDev emb, const StepDesc* desc,
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

__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, const float* g, void* xn, int D,
                                                 float eps, int act) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const float* xb = x + (size_t)b * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) ss += xb[i] * xb[i];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (act == ACT_BF16) {
    uint16_t* o = (uint16_t*)xn + (size_t)b * D;
    for (int i = threadIdx.x; i < D; i += 256) o[i] = f32_to_bf16(xb[i] * r * g[i]);
  } else {
    float* o = (float*)xn + (size_t)b * D;
    for (int i = threadIdx.x; i < D; i += 256) o[i] = xb[i] * r * g[i];
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

template <int EPI, int ROWS>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, int b, int row0, const float* v) {
  const int N = a.m.rows;
  const Dims& d = a.d;
  if constexpr (EPI == EPI_QKV) {
    // Stored QKV rows: q and k heads hold the RoPE pairs (i, i + hd/2) as adjacent rows
    // (2i, 2i+1); v rows are in natural order.
    const int pos = a.ea.desc->pos[b];
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
  const size_t row_bytes = (size_t)K * EB;

  float acc[ROWS][NB];
#pragma unroll
  for (int i = 0; i < ROWS; i++)
#pragma unroll
    for (int bb = 0; bb < NB; bb++) acc[i][bb] = 0.f;

  for (int kc0 = 0; kc0 < K; kc0 += KCP) {
    const int kcn = min(KCP, K - kc0);
    const int kcpad = (kcn + KSTEP - 1) / KSTEP * KSTEP;
    if (kc0) __syncthreads();
    for (int idx = threadIdx.x; idx < NB * kcpad; idx += 256) {
      const int bb = idx / kcpad, kk = idx - bb * kcpad;
      float v = 0.f;
      if (bb < nb && kk < kcn) {
        const size_t gi = (size_t)(b0 + bb) * K + kc0 + kk;
        v = a.act_in == ACT_BF16 ? bf16_to_f32(((const uint16_t*)a.xin)[gi])
                                 : ((const float*)a.xin)[gi];
      }
      const int st = kk / KSTEP, r = kk - st * KSTEP, ln = r / VEC, j = r - ln * VEC;
      xs[bb * KCP + st * KSTEP + (j >> 2) * 256 + ln * 4 + (j & 3)] = v;
    }
    __syncthreads();

    for (int ks = 0; ks < kcn; ks += KSTEP) {
      const int kl = ks + lane * VEC;
      const bool kvalid = kl < kcn;
      const int k = kc0 + kl;
      uint4 wv[ROWS];
      float qs[ROWS];
#pragma unroll
      for (int i = 0; i < ROWS; i++) {
        const int r = row0 + i;
        const bool ok = kvalid && r < N;
        wv[i] = ok ? *(const uint4*)(wbase + (size_t)r * row_bytes + (size_t)k * EB)
                   : make_uint4(0u, 0u, 0u, 0u);
        if constexpr (WFMT == W_Q8_0)
          qs[i] = ok ? f16_to_f32(((const uint16_t*)a.m.s)[(size_t)r * (K / 32) + (k >> 5)]) : 0.f;
      }
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
    r = idx >> 5;                                   // kGemmKC / 8 = 32 pieces per row
    k = c * kGemmKC + (idx & 31) * 8;
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

// one (head, sequence): o = merge of its chunk partials, rounded to the activation type
__global__ __launch_bounds__(256) void k_combine(Dims d, const StepDesc* desc, const float* partials,
                                                 void* o) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int nv = (desc->pos[b] + d.ct) / d.ct;
  const float* P = partials + ((size_t)b * d.Hq + h) * d.nch * (d.hd + 2);
  if (i < d.hd) store_act(o, (size_t)b * d.q_dim + (size_t)h * d.hd + i, combine_one(P, nv, d.hd, i), d.act);
}

// S11 greedy argmax over the fp32 logits, lowest index among equal maxima
__global__ __launch_bounds__(1024) void k_argmax(const float* logits, int V, const StepDesc* desc) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int b = blockIdx.x;
  const float* L = logits + (size_t)b * V;
  float best = -INFINITY;
  int idx = INT_MAX;
  for (int v = threadIdx.x; v < V; v += 1024) {
    const float x = L[v];
    if (x > best || (idx == INT_MAX && !isnan(x))) { best = x; idx = v; }
  }
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
// launch helpers
// ---------------------------------------------------------------------------------------

template <int WFMT, int EPI>
hipError_t gemv_dispatch(const GemvArgs& a, int NB, int ROWS, dim3 grid, size_t smem, hipStream_t st) {
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
hipError_t gemm_dispatch(const GemmArgs& a, int nbb, dim3 grid, size_t smem, hipStream_t st) {
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
  if (r != hipSuccess || a.S == 1) return r;
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

int gemm_splits(int N, int K, int cus) {
  const int tiles = (N + kGemmRows - 1) / kGemmRows;
  const int nchunk = (K + kGemmKC - 1) / kGemmKC;
  if (tiles >= cus) return 1;
  const int S = (cus + tiles - 1) / tiles;
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

hipError_t launch_embed(const Dims& d, const MatDev& emb, const StepDesc* desc, int B,
                        int32_t* block_table, float* x, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(B), dim3(256), 0, st, d, emb, desc, block_table, x, err);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const Dims& d, const float* x, const float* g, void* xn, int B,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(256), 0, st, x, g, xn, d.D, d.eps, d.act);
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
  const int ROWS = m.rows >= 4 * 16 * 256 ? 4 : 2;
  const int VEC = d.wfmt == W_BF16 ? 8 : 16, KSTEP = 64 * VEC;
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
    default: return gemv_epi<W_BF16>(a, epi, NB, ROWS, grid, smem, st);
  }
}

hipError_t launch_attention(const Dims& d, const StepDesc* desc, int B, const float* q,
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
  const dim3 grid(d.nch, d.Hkv, B);
  const size_t smem = sizeof(float) * attn_smem_floats(d.G, d.hd);
  if (d.kvfmt == KV_F32) hipLaunchKernelGGL(k_attn<KV_F32>, grid, dim3(256), smem, st, a, desc, partials);
  else if (d.kvfmt == KV_BF16) hipLaunchKernelGGL(k_attn<KV_BF16>, grid, dim3(256), smem, st, a, desc, partials);
  else hipLaunchKernelGGL(k_attn<KV_I8>, grid, dim3(256), smem, st, a, desc, partials);
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const StepDesc* desc, int B, const float* partials,
                          void* o, hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3(d.Hq, B), dim3(d.hd), 0, st, d, desc, partials, o);
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
