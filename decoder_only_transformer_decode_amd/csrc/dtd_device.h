// dtd_device.h -- device helpers shared by the per-kernel path (dtd_kernels.hip) and the
// persistent step kernel (dtd_persistent.hip): number formats, wavefront reductions,
// weight dequantisation, and the split-K GQA decode-attention work item.
#pragma once

#include <math.h>
#include <stdint.h>

#include "dtd_internal.h"

namespace dtd {
namespace dev {

// ---------------------------------------------------------------------------------------
// global-memory access through pointers the compiler cannot prove global (read from a table
// or a struct): without the address-space cast it emits FLAT instructions, which count
// against the LDS counter too, so every later LDS access would wait for them, in-flight
// weight prefetches included
// ---------------------------------------------------------------------------------------

typedef unsigned int gv4u __attribute__((ext_vector_type(4)));
typedef unsigned int gv2u __attribute__((ext_vector_type(2)));

// 8- and 16-byte types load through native vectors: a copy of HIP's vector structs is
// split into 32-bit pieces that lose the address space
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  if constexpr (sizeof(T) == 16) {
    const gv4u v = *(const __attribute__((address_space(1))) gv4u*)p;
    return __builtin_bit_cast(T, v);
  } else if constexpr (sizeof(T) == 8) {
    const gv2u v = *(const __attribute__((address_space(1))) gv2u*)p;
    return __builtin_bit_cast(T, v);
  } else {
    return *(const __attribute__((address_space(1))) T*)p;
  }
}

// the same for data read once per step (weights): the nontemporal hint streams the lines
// through the caches instead of keeping them, which sustains a higher HBM read rate
template <typename T>
__device__ __forceinline__ T gload_stream(const void* p) {
  if constexpr (sizeof(T) == 16) {
    const gv4u v = __builtin_nontemporal_load((const __attribute__((address_space(1))) gv4u*)p);
    return __builtin_bit_cast(T, v);
  } else {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)p);
  }
}

template <typename T>
__device__ __forceinline__ void gstore(void* p, T v) {
  if constexpr (sizeof(T) == 16) {
    *(__attribute__((address_space(1))) gv4u*)p = __builtin_bit_cast(gv4u, v);
  } else if constexpr (sizeof(T) == 8) {
    *(__attribute__((address_space(1))) gv2u*)p = __builtin_bit_cast(gv2u, v);
  } else {
    *(__attribute__((address_space(1))) T*)p = v;
  }
}

// ---------------------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16, round to nearest even (NaN kept quiet); written as a select rather than an
// early return so that it compiles without a branch
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? nan : rne);
}

__device__ __forceinline__ float round_act(float v, int act) {
  return act == ACT_BF16 ? bf16_to_f32(f32_to_bf16(v)) : v;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {  // hardware convert, RNE
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// signed byte `byte` of u as float (one v_cvt_f32_i32 with a byte-select operand)
__device__ __forceinline__ float sext8(uint32_t u, int byte) {
  return (float)((int32_t)(u << (24 - 8 * byte)) >> 24);
}

// store v into activation storage of type act at element i
__device__ __forceinline__ void store_act(void* p, size_t i, float v, int act) {
  if (act == ACT_BF16) ((uint16_t*)p)[i] = f32_to_bf16(v);
  else ((float*)p)[i] = v;
}

__device__ __forceinline__ float load_act(const void* p, size_t i, int act) {
  return act == ACT_BF16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// ---------------------------------------------------------------------------------------
// reductions (wave64 butterflies; block versions for any multiple of 64 threads)
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// red: >= blockDim.x/64 floats of LDS; every thread gets the result
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < nw; w++) s += red[w];
  return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = red[0];
  for (int w = 1; w < nw; w++) s = fmaxf(s, red[w]);
  return s;
}

// one stored weight element as fp32: int8-row q*s, Q8_0 q*d, Q4_0 (q-8)*d (one fp32 product;
// a Q4_0 block's byte j holds column j in its low 4 bits and column j+16 in its high 4 bits),
// bf16 widen
__device__ __forceinline__ float deq_elem(const MatDev& m, int wfmt, int r, int c) {
  const size_t e = (size_t)r * m.cols + c;
  if (wfmt == W_Q4_0) {
    const uint8_t byte = ((const uint8_t*)m.w)[(size_t)r * (m.cols / 2) + (c / 32) * 16 + (c % 16)];
    const int q = (c % 32) < 16 ? (byte & 15) : (byte >> 4);
    return (float)(q - 8) * f16_to_f32(((const uint16_t*)m.s)[(size_t)r * (m.cols / 32) + c / 32]);
  }
  if (wfmt == W_INT8_ROW) return (float)((const int8_t*)m.w)[e] * ((const float*)m.s)[r];
  if (wfmt == W_Q8_0)
    return (float)((const int8_t*)m.w)[e] *
           f16_to_f32(((const uint16_t*)m.s)[(size_t)r * (m.cols / 32) + c / 32]);
  return bf16_to_f32(((const uint16_t*)m.w)[e]);
}

// ---------------------------------------------------------------------------------------
// split-K GQA decode attention, one work item = (sequence b, kv head j, chunk c)
//
// The item streams positions [c*ct, min((c+1)*ct, pos+1)) of kv head j through LDS in
// 64-position tiles; the G query heads that share kv head j all use each staged K/V row,
// so K/V is read once per query group (the GQA decode rule of the Qwen3-8B engine
// article, 4.4.2).  Softmax is online across tiles (running max, running sum, rescaled
// accumulators); the item leaves an unnormalised partial (acc, m, l) per head, merged by
// k_combine.  The item whose chunk holds the new position rounds the new k/v to the KV
// encoding, writes it through the block table and attends to the stored value.
// ---------------------------------------------------------------------------------------

struct AttnCtx {
  Dims d;
  const float* q;        // [B][q_dim] post-RoPE
  const float* knew;     // [B][kv_dim] post-RoPE, not yet rounded to the KV type
  const float* vnew;     // [B][kv_dim]
  KvLayer kv;
  const int32_t* bt;     // block table [max_seqs][max_blocks]
  int ct;                // chunk length
  int nch;               // chunk stride of partials
};

constexpr int kMaxOutPerThread = 8;   // G*hd <= 2048 outputs over >= 256 threads

// LDS floats an item needs
__host__ __device__ inline size_t attn_smem_floats(int G, int hd) {
  return (size_t)G * hd + (size_t)kAttnTile * (hd + 1) + (size_t)G * kAttnTile + (size_t)G * 4 +
         2 * (size_t)hd + 32;
}

template <int KVFMT>
__device__ __forceinline__ void stage_tile(const Dims& d, const void* pool, const uint16_t* spool,
                                           const int32_t* btrow, int j, int t0, int n, int pos,
                                           const float* newv, float* t_s, int ldk) {
  const int hd = d.hd, per = hd >> 2;
  for (int e = threadIdx.x; e < n * per; e += blockDim.x) {
    const int tl = e / per, i = (e - tl * per) * 4, t = t0 + tl;
    float v0, v1, v2, v3;
    if (t == pos) {
      v0 = newv[i]; v1 = newv[i + 1]; v2 = newv[i + 2]; v3 = newv[i + 3];
    } else {
      const int blk = gload<int32_t>(btrow + t / d.bs), off = t - (t / d.bs) * d.bs;
      const size_t row = ((size_t)blk * d.Hkv + j) * d.bs + off;
      const size_t base = row * hd + i;
      if constexpr (KVFMT == KV_F32) {
        const float4 f = gload<float4>((const float*)pool + base);
        v0 = f.x; v1 = f.y; v2 = f.z; v3 = f.w;
      } else if constexpr (KVFMT == KV_BF16) {
        const uint2 u = gload<uint2>((const uint16_t*)pool + base);
        v0 = __uint_as_float(u.x << 16); v1 = __uint_as_float(u.x & 0xffff0000u);
        v2 = __uint_as_float(u.y << 16); v3 = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const uint32_t u = gload<uint32_t>((const int8_t*)pool + base);
        const float s = f16_to_f32(gload<uint16_t>(spool + row));
        v0 = sext8(u, 0) * s; v1 = sext8(u, 1) * s; v2 = sext8(u, 2) * s; v3 = sext8(u, 3) * s;
      }
    }
    float* dst = t_s + tl * ldk + i;
    dst[0] = v0; dst[1] = v1; dst[2] = v2; dst[3] = v3;
  }
}

// Rounds the new position's key and value (kn, vn: hd fp32 each) to the KV encoding,
// writes them to pool row `row` of kv head j's layout, and leaves the stored (decoded)
// values in new_s [2][hd].  All threads of the block must call this: the int8 scale is a
// block-wide max.  red: reduction scratch (>= one float per wave).
template <int KVFMT>
__device__ __forceinline__ void kv_append(const KvLayer& kv, size_t row, int hd, const float* kn, const float* vn,
                                          float* new_s, float* red) {
  const int tid = threadIdx.x;
  for (int which = 0; which < 2; which++) {
    const float* src = which ? vn : kn;
    void* pool = which ? kv.v : kv.k;
    const float xv = tid < hd ? src[tid] : 0.f;
    if constexpr (KVFMT == KV_F32) {
      if (tid < hd) { gstore<float>((float*)pool + row * hd + tid, xv); new_s[which * hd + tid] = xv; }
    } else if constexpr (KVFMT == KV_BF16) {
      if (tid < hd) {
        const uint16_t bits = f32_to_bf16(xv);
        gstore<uint16_t>((uint16_t*)pool + row * hd + tid, bits);
        new_s[which * hd + tid] = bf16_to_f32(bits);
      }
    } else {
      const float amax = block_max(fabsf(xv), red);
      const uint16_t s16 = f32_to_f16(amax / 127.0f);
      const float s = f16_to_f32(s16);
      float qv = 0.f;
      if (s != 0.f) qv = fminf(fmaxf(rintf(xv / s), -127.f), 127.f);
      if (tid < hd) {
        gstore<int8_t>((int8_t*)pool + row * hd + tid, (int8_t)qv);
        new_s[which * hd + tid] = qv * s;
      }
      if (tid == 0) gstore<uint16_t>((which ? kv.vs : kv.ks) + row, s16);
    }
  }
}

// All threads of the block must call this (it synchronises the block).  sm: LDS of
// attn_smem_floats(G, hd) floats.  qg: the G query vectors of head group j; kn, vn: head
// j's new key and value (not yet rounded); pos_blk: physical block of position pos.
// The partial (acc[hd], m, l) of head h goes out through put(index, value), index =
// ((b*Hq + h)*nch + c)*(hd+2) + field.
template <int KVFMT, typename Put>
__device__ __forceinline__ void attn_item(const AttnCtx& a, int b, int j, int c, int pos, int slot,
                                          int pos_blk, const float* qg, const float* kn, const float* vn,
                                          float* sm, Put put) {
  const Dims& d = a.d;
  const int len = pos + 1;
  const int t_begin = c * a.ct;
  const int t_end = min(len, t_begin + a.ct);
  const int hd = d.hd, G = d.G, tid = threadIdx.x, NT = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, NW = NT >> 6;
  const int ldk = hd + 1;
  const int32_t* btrow = a.bt + (size_t)slot * d.max_blocks;

  float* q_s = sm;                          // [G][hd], pre-scaled by 1/sqrt(hd)
  float* t_s = q_s + G * hd;                // [64][hd+1]: K tile, then V tile
  float* p_s = t_s + kAttnTile * ldk;       // [G][64]: scores, then probabilities
  float* st_s = p_s + G * kAttnTile;        // [G][4]: running max, running sum, rescale
  float* new_s = st_s + G * 4;              // [2][hd]: stored (decoded) new k, v
  float* red = new_s + 2 * hd;              // [32] reduction scratch

  const float scale = 1.0f / sqrtf((float)hd);
  for (int e = tid; e < G * hd; e += NT) q_s[e] = qg[e] * scale;
  for (int g = tid; g < G; g += NT) { st_s[g * 4] = -INFINITY; st_s[g * 4 + 1] = 0.f; }

  if (pos >= t_begin && pos < t_end) {  // this item appends the new token of head j
    const int off = pos - (pos / d.bs) * d.bs;
    kv_append<KVFMT>(a.kv, ((size_t)pos_blk * d.Hkv + j) * d.bs + off, hd, kn, vn, new_s, red);
  }
  __syncthreads();

  float acc[kMaxOutPerThread];
#pragma unroll
  for (int k = 0; k < kMaxOutPerThread; k++) acc[k] = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += kAttnTile) {
    const int n = min(kAttnTile, t_end - t0);
    stage_tile<KVFMT>(d, a.kv.k, a.kv.ks, btrow, j, t0, n, pos, new_s, t_s, ldk);
    __syncthreads();
    for (int sidx = tid; sidx < G * kAttnTile; sidx += NT) {
      const int g = sidx / kAttnTile, tl = sidx - g * kAttnTile;
      float s = -INFINITY;
      if (tl < n) {
        s = 0.f;
        const float* qg = q_s + g * hd;
        const float* kr = t_s + tl * ldk;
        for (int i = 0; i < hd; i++) s += qg[i] * kr[i];
      }
      p_s[sidx] = s;
    }
    __syncthreads();
    for (int g = wave; g < G; g += NW) {
      const float s = p_s[g * kAttnTile + lane];
      const float mt = wave_max(s);
      const float mo = st_s[g * 4], lo = st_s[g * 4 + 1];
      const float mn = fmaxf(mo, mt);
      const float p = lane < n ? expf(s - mn) : 0.f;
      const float ps = wave_sum(p);
      p_s[g * kAttnTile + lane] = p;
      if (lane == 0) {
        const float al = expf(mo - mn);
        st_s[g * 4] = mn;
        st_s[g * 4 + 1] = lo * al + ps;
        st_s[g * 4 + 2] = al;
      }
    }
    __syncthreads();
    stage_tile<KVFMT>(d, a.kv.v, a.kv.vs, btrow, j, t0, n, pos, new_s + hd, t_s, ldk);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxOutPerThread; k++) {
      const int oi = tid + k * NT;
      if (oi < G * hd) {
        const int g = oi / hd, i = oi - g * hd;
        const float* pg = p_s + g * kAttnTile;
        float sum = 0.f;
        for (int tl = 0; tl < n; tl++) sum += pg[tl] * t_s[tl * ldk + i];
        acc[k] = acc[k] * st_s[g * 4 + 2] + sum;
      }
    }
    __syncthreads();
  }

  const int cs = hd + 2;
#pragma unroll
  for (int k = 0; k < kMaxOutPerThread; k++) {
    const int oi = tid + k * NT;
    if (oi < G * hd) {
      const int g = oi / hd, i = oi - g * hd, h = j * G + g;
      put((((size_t)b * d.Hq + h) * a.nch + c) * cs + i, acc[k]);
    }
  }
  for (int g = tid; g < G; g += NT) {
    const int h = j * G + g;
    const size_t P = (((size_t)b * d.Hq + h) * a.nch + c) * cs;
    put(P + hd, st_s[g * 4]);
    put(P + hd + 1, st_s[g * 4 + 1]);
  }
}

}  // namespace dev
}  // namespace dtd
