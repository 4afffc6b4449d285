// Decode-step kernels of libwq for gfx950: the work of a Llama-style decode step around its
// weight-only-quantized linears (the linears themselves are wq_kernels.hip).
//
// The pages name this loop without defining it: the gpt-fast write-up (m.greenbasetech.com,
// part on torch.compile) runs a whole decode step as one captured region, and the speed-up
// strategies page (sharktoolz.top, section 6) keeps a key/value cache shared by groups of query
// heads. The definitions followed are the Llama decoder layer's (include/wq_decode.h states each).
//
// gfx950 design:
//  * Every kernel reads the decode position and the token ids from device memory, so a step is
//    captured once as a HIP graph and replayed for step after step; wq_argmax_next advances them.
//  * Attention of one new token, caches of up to 4096 positions: one workgroup of 16 waves per
//    (query head, sequence) over all positions, a running softmax per wave and the waves combined
//    in LDS: one launch and no workspace (rope_attention_wide_kernel). Longer caches, flash-decoding
//    style: the positions 0..pos are cut into
//    chunks of 64, one workgroup per (chunk, query head, sequence), so that even a short context
//    spreads over the CUs (Llama-2-7B at 512 positions: 256 workgroups; chunks of 128 left half
//    the CUs idle). A workgroup first issues the loads of all its key and value rows (16
//    lanes per position, a 16-byte slice each: 256-byte coalesced reads), then rotates its query
//    (and, in the last chunk, the new key), scores its positions with a 16-lane DPP sum, takes
//    the softmax of its chunk in LDS and sums the weighted value slices. Chunks meet in a workspace:
//    each writes (max, sum, weighted values), and a second launch combines them in chunk order
//    (deterministic). A single launch in which the last chunk to finish combines (an atomic counter
//    per head) needs device-scope fences, which write back and invalidate L2 on every XCD, and was
//    an order of magnitude slower.
//  * RMSNorm, embedding, silu*up and argmax stream 16 bytes per lane; reductions run in a fixed
//    order (DPP within 16-lane rows, shuffles across the rows of a wave, then waves in order), so
//    every result is deterministic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "wq_device.h"
#include "wq_internal.h"
#include "../../include/wq_decode.h"

namespace {

constexpr int DEC_THREADS = 256;
constexpr int ATT_CHUNK = 64;    // positions per attention workgroup of the chunked kernel
constexpr int ATT_WIDE_THREADS = 1024;   // the single-workgroup kernel: 16 waves per (query head, sequence)
constexpr int ATT_WIDE_MAX = 4096;       // longest cache (positions) it serves; longer ones take the chunks
constexpr int ATT_WIDE_PPL = 32 * 16;    // positions x dimensions per 16-lane group and step (a register budget:
                                         // 4 positions per lane group at head size 128, 8 at 64)

__device__ __forceinline__ float f16v(uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); }
__device__ __forceinline__ uint32_t to_f16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float lo16(uint32_t w) { return f16v(w & 0xFFFFu); }
__device__ __forceinline__ float hi16(uint32_t w) { return f16v(w >> 16); }

// Sum over each row of 16 lanes, left in every lane of the row: four DPP adds (lane ^ 1, lane ^ 2,
// the other half of each 8 lanes, the other half of the 16), no LDS traffic (a __shfl_xor tree
// compiled to ds_bpermute, an LDS round trip per step).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141, 0xF>(v);   // row_half_mirror
  v += dpp<0x140, 0xF>(v);   // row_mirror
  return v;
}

// The same for the maximum.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0xB1, 0xF>(v));
  v = fmaxf(v, dpp<0x4E, 0xF>(v));
  v = fmaxf(v, dpp<0x141, 0xF>(v));
  v = fmaxf(v, dpp<0x140, 0xF>(v));
  return v;
}

// Sum / max over the workgroup in a fixed order: DPP within each 16-lane row, the four rows of a
// wave by two shuffles, then the waves in order. Every thread gets the result. `red` holds one
// float per wave.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = row_max16(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, red[i]);
  return t;
}

// ---------------------------------------------------------------- embedding
__global__ __launch_bounds__(DEC_THREADS) void embed_kernel(const uint16_t* __restrict__ table,
                                                            const int32_t* __restrict__ tokens, float* __restrict__ x,
                                                            int d, int vocab) {
  const int m = blockIdx.x;
  int t = tokens[m];
  t = t < 0 ? 0 : t >= vocab ? vocab - 1 : t;
  const uint4* src = reinterpret_cast<const uint4*>(table + (size_t)t * d);
  float4* dst = reinterpret_cast<float4*>(x + (size_t)m * d);
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const uint4 v = src[c];
    dst[2 * c] = make_float4(lo16(v.x), hi16(v.x), lo16(v.y), hi16(v.y));
    dst[2 * c + 1] = make_float4(lo16(v.z), hi16(v.z), lo16(v.w), hi16(v.w));
  }
}

// ---------------------------------------------------------------- residual add + RMSNorm
// One workgroup per row. Rows of up to RN_CHUNKS * 8 * 256 values stay in registers between the
// sum of squares and the scaling (every load issued up front: the workgroup waits for memory once);
// longer rows are read again.
constexpr int RN_CHUNKS = 4;

__device__ __forceinline__ void add_delta(float4& a, float4& b, const uint4& t) {
  a.x += lo16(t.x); a.y += hi16(t.x); a.z += lo16(t.y); a.w += hi16(t.y);
  b.x += lo16(t.z); b.y += hi16(t.z); b.z += lo16(t.w); b.w += hi16(t.w);
}
__device__ __forceinline__ float sumsq(const float4& a, const float4& b) {
  return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
}
__device__ __forceinline__ uint4 scaled(const float4& a, const float4& b, const uint4& w, float r) {
  uint4 o;
  o.x = to_f16(a.x * r * lo16(w.x)) | (to_f16(a.y * r * hi16(w.x)) << 16);
  o.y = to_f16(a.z * r * lo16(w.y)) | (to_f16(a.w * r * hi16(w.y)) << 16);
  o.z = to_f16(b.x * r * lo16(w.z)) | (to_f16(b.y * r * hi16(w.z)) << 16);
  o.w = to_f16(b.z * r * lo16(w.w)) | (to_f16(b.w * r * hi16(w.w)) << 16);
  return o;
}

__global__ __launch_bounds__(DEC_THREADS) void add_rmsnorm_kernel(float* __restrict__ x, const uint16_t* __restrict__ delta,
                                                                  const uint16_t* __restrict__ g, float eps,
                                                                  uint16_t* __restrict__ out, int d) {
  __shared__ float red[DEC_THREADS / 64];
  const int m = blockIdx.x, C = d / 8;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)m * d);
  const uint4* dr = delta ? reinterpret_cast<const uint4*>(delta + (size_t)m * d) : nullptr;
  const uint4* gr = reinterpret_cast<const uint4*>(g);
  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)m * d);
  float ss = 0.0f;
  if (C <= RN_CHUNKS * DEC_THREADS) {
    float4 xa[RN_CHUNKS], xb[RN_CHUNKS];
    uint4 dt[RN_CHUNKS], gw[RN_CHUNKS];
#pragma unroll
    for (int i = 0; i < RN_CHUNKS; ++i) {
      const int c = min((int)threadIdx.x + i * DEC_THREADS, C - 1);   // past the row end: a valid chunk, unused
      xa[i] = xr[2 * c];
      xb[i] = xr[2 * c + 1];
      dt[i] = dr ? dr[c] : make_uint4(0u, 0u, 0u, 0u);
      gw[i] = gr[c];
    }
#pragma unroll
    for (int i = 0; i < RN_CHUNKS; ++i) {
      const int c = (int)threadIdx.x + i * DEC_THREADS;
      if (c < C) {
        if (dr) {
          add_delta(xa[i], xb[i], dt[i]);
          xr[2 * c] = xa[i];
          xr[2 * c + 1] = xb[i];
        }
        ss += sumsq(xa[i], xb[i]);
      }
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < RN_CHUNKS; ++i) {
      const int c = (int)threadIdx.x + i * DEC_THREADS;
      if (c < C) orow[c] = scaled(xa[i], xb[i], gw[i], r);
    }
    return;
  }
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float4 a = xr[2 * c], b = xr[2 * c + 1];
    if (dr) {
      add_delta(a, b, dr[c]);
      xr[2 * c] = a;
      xr[2 * c + 1] = b;
    }
    ss += sumsq(a, b);
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = threadIdx.x; c < C; c += blockDim.x) orow[c] = scaled(xr[2 * c], xr[2 * c + 1], gr[c], r);
}

// ---------------------------------------------------------------- silu(gate) * up
__global__ __launch_bounds__(DEC_THREADS) void silu_mul_kernel(const uint16_t* __restrict__ gate,
                                                               const uint16_t* __restrict__ up, uint16_t* __restrict__ out,
                                                               int n8) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n8) return;
  const uint4 g = reinterpret_cast<const uint4*>(gate)[c], u = reinterpret_cast<const uint4*>(up)[c];
  auto f = [](uint32_t gw, uint32_t uw) {   // both fp16 halves of a word
    return (uint32_t)silu_mul_f16(gw & 0xFFFFu, uw & 0xFFFFu) | ((uint32_t)silu_mul_f16(gw >> 16, uw >> 16) << 16);
  };
  uint4 o;
  o.x = f(g.x, u.x);
  o.y = f(g.y, u.y);
  o.z = f(g.z, u.z);
  o.w = f(g.w, u.w);
  reinterpret_cast<uint4*>(out)[c] = o;
}

// ---------------------------------------------------------------- argmax and step advance
__global__ __launch_bounds__(DEC_THREADS) void argmax_kernel(const uint16_t* __restrict__ logits, int vocab,
                                                             int32_t* __restrict__ tokens, int32_t* __restrict__ pos) {
  __shared__ float bv[DEC_THREADS / 64];
  __shared__ int bi[DEC_THREADS / 64];
  const int m = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(logits + (size_t)m * vocab);
  float best = -INFINITY;
  int idx = 0x7FFFFFFF;
  auto take = [&](float v, int i) {   // larger, or equal at a lower index; NaN never wins
    if (v > best || (v == best && i < idx)) { best = v; idx = i; }
  };
  for (int c = threadIdx.x; c < vocab / 8; c += blockDim.x) {
    const uint4 w = row[c];
    take(lo16(w.x), 8 * c); take(hi16(w.x), 8 * c + 1); take(lo16(w.y), 8 * c + 2); take(hi16(w.y), 8 * c + 3);
    take(lo16(w.z), 8 * c + 4); take(hi16(w.z), 8 * c + 5); take(lo16(w.w), 8 * c + 6); take(hi16(w.w), 8 * c + 7);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) take(__shfl_xor(best, o), __shfl_xor(idx, o));
  if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) take(bv[i], bi[i]);
    tokens[m] = idx == 0x7FFFFFFF ? 0 : idx;
    if (m == 0) *pos += 1;
  }
}

// ---------------------------------------------------------------- rotary embedding + cache append + attention
// Workgroup (chunk c, query head h, sequence m); HD = head size (64 or 128). Lane (lg = tid / 16,
// j = tid % 16) owns dimensions j*HD/16 .. of the positions t0 + lg + 16 i (i < ATT_CHUNK / 16), and
// issues the loads of all its key and value slices first, so that a workgroup waits for memory once.
template <int HD>
__global__ __launch_bounds__(DEC_THREADS) void rope_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ cache_k, uint16_t* __restrict__ cache_v, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, const int32_t* __restrict__ posp, uint16_t* __restrict__ out, int H, int Hkv,
    int S, float* __restrict__ part, int nsplit_max) {
  constexpr int P2 = HD / 2;               // rotated pairs of a head
  constexpr int DPL = HD / 16;             // dimensions per lane
  constexpr int WPL = DPL / 2;             // their 32-bit words
  constexpr int PPT = ATT_CHUNK / 16;      // positions per lane
  __shared__ float qs[HD], kn[HD], vn[HD], sc[ATT_CHUNK], acc[16][HD], red[DEC_THREADS / 64];
  const int c = blockIdx.x, h = blockIdx.y, m = blockIdx.z, tid = threadIdx.x;
  int p = *posp;
  p = p < 0 ? 0 : p >= S ? S - 1 : p;
  const int nsplit = (p + ATT_CHUNK) / ATT_CHUNK;          // chunks covering positions 0..p
  if (c >= nsplit) return;                                  // (whole workgroup: uniform)
  const int t0 = c * ATT_CHUNK, t1 = min(p + 1, t0 + ATT_CHUNK);
  const int group = H / Hkv, kh = h / group;
  const bool has_p = c == nsplit - 1;
  const size_t kvrow = (size_t)Hkv * HD;                    // elements of one cache position
  const int lg = tid >> 4, j = tid & 15;

  // this lane's key and value slices (positions past the chunk end read its last position; the
  // new position p is read too but replaced by the values computed below)
  uint32_t kw[PPT][WPL], vw[PPT][WPL];
  {
    const uint16_t* ckm = cache_k + (size_t)m * S * kvrow + (size_t)kh * HD + j * DPL;
    const uint16_t* cvm = cache_v + (size_t)m * S * kvrow + (size_t)kh * HD + j * DPL;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const size_t t = (size_t)min(t0 + lg + 16 * i, t1 - 1);
      if constexpr (WPL == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(ckm + t * kvrow);
        const uint4 b = *reinterpret_cast<const uint4*>(cvm + t * kvrow);
        kw[i][0] = a.x; kw[i][1] = a.y; kw[i][2] = a.z; kw[i][3] = a.w;
        vw[i][0] = b.x; vw[i][1] = b.y; vw[i][2] = b.z; vw[i][3] = b.w;
      } else {
        const uint2 a = *reinterpret_cast<const uint2*>(ckm + t * kvrow);
        const uint2 b = *reinterpret_cast<const uint2*>(cvm + t * kvrow);
        kw[i][0] = a.x; kw[i][1] = a.y;
        vw[i][0] = b.x; vw[i][1] = b.y;
      }
    }
  }

  if (tid < P2) {   // rotate pair tid of the query (kept in float32, scaled), and of the new key
    const float co = rope_cos[(size_t)p * P2 + tid], si = rope_sin[(size_t)p * P2 + tid];
    const float scale = 1.0f / sqrtf((float)HD);
    const uint32_t qq = *reinterpret_cast<const uint32_t*>(q + ((size_t)m * H + h) * HD + 2 * tid);
    qs[2 * tid] = (lo16(qq) * co - hi16(qq) * si) * scale;
    qs[2 * tid + 1] = (lo16(qq) * si + hi16(qq) * co) * scale;
    if (has_p) {
      const uint32_t kk = *reinterpret_cast<const uint32_t*>(k + ((size_t)m * Hkv + kh) * HD + 2 * tid);
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(v + ((size_t)m * Hkv + kh) * HD + 2 * tid);
      const uint32_t kr = to_f16(lo16(kk) * co - hi16(kk) * si) | (to_f16(lo16(kk) * si + hi16(kk) * co) << 16);
      kn[2 * tid] = lo16(kr);
      kn[2 * tid + 1] = hi16(kr);
      vn[2 * tid] = lo16(vv);
      vn[2 * tid + 1] = hi16(vv);
      if (h % group == 0) {   // one query head of the group writes the cache; the others use kn, vn
        *reinterpret_cast<uint32_t*>(cache_k + ((size_t)m * S + p) * kvrow + (size_t)kh * HD + 2 * tid) = kr;
        *reinterpret_cast<uint32_t*>(cache_v + ((size_t)m * S + p) * kvrow + (size_t)kh * HD + 2 * tid) = vv;
      }
    }
  }
  __syncthreads();

  float qv[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) qv[d] = qs[j * DPL + d];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {   // scores: a 16-lane shuffle sum per position
    const int t = t0 + lg + 16 * i;
    float s = 0.0f;
    if (t == p) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) s += qv[d] * kn[j * DPL + d];
    } else {
#pragma unroll
      for (int w = 0; w < WPL; ++w) s += qv[2 * w] * lo16(kw[i][w]) + qv[2 * w + 1] * hi16(kw[i][w]);
    }
    s = row_sum16(s);
    if (j == 0 && t < t1) sc[t - t0] = s;
  }
  __syncthreads();

  const int n = t1 - t0;   // softmax of the chunk (n <= ATT_CHUNK < DEC_THREADS)
  const float mx = block_max(tid < n ? sc[tid] : -INFINITY, red);
  const float e = tid < n ? expf(sc[tid] - mx) : 0.0f;
  const float l = block_sum(e, red);   // its barriers also order the reads of sc above
  if (tid < n) sc[tid] = e;
  __syncthreads();

  float ar[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) ar[d] = 0.0f;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {   // weighted values of this lane's positions
    const int t = t0 + lg + 16 * i;
    if (t < t1) {
      const float pt = sc[t - t0];
      if (t == p) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) ar[d] += pt * vn[j * DPL + d];
      } else {
#pragma unroll
        for (int w = 0; w < WPL; ++w) {
          ar[2 * w] += pt * lo16(vw[i][w]);
          ar[2 * w + 1] += pt * hi16(vw[i][w]);
        }
      }
    }
  }
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[lg][j * DPL + d] = ar[d];
  __syncthreads();
  float a = 0.0f;
  if (tid < HD)
    for (int g = 0; g < 16; ++g) a += acc[g][tid];   // position groups in order

  uint16_t* orow = out + ((size_t)m * H + h) * HD;
  if (nsplit == 1) {
    if (tid < HD) orow[tid] = (uint16_t)to_f16(a / l);
    return;
  }
  // several chunks: this one's (max, sum, weighted values) for attention_combine_kernel
  float* pr = part + (((size_t)m * H + h) * nsplit_max + c) * (HD + 2);
  if (tid < HD) pr[2 + tid] = a;
  if (tid == 0) { pr[0] = mx; pr[1] = l; }
}

// One workgroup of 16 waves per (query head h, sequence m) over all positions 0..p, for caches of
// up to ATT_WIDE_MAX positions: no partial result leaves the workgroup, so there is no workspace
// and no combine launch (a launch costs a few microseconds whatever it does, and the chunked
// kernel's combine was one per layer). Wave w takes the steps of STEP positions (16 at head size
// 128, 32 at 64) that start at STEP w, STEP (w + 16), ...; lane (lg = lane / 16, j = lane % 16)
// holds dimensions j*HD/16.. of positions step + lg + 4 i (i < STEP / 4), as a 16-byte (8-byte)
// slice of each key and value row. Each wave keeps
// a running softmax over its steps (its maximum M_w, sum L_w and weighted values A_w, rescaled by
// e^(old max - new max) when the maximum grows); the 16 waves then meet in LDS and thread d < HD
// combines them in wave order: out = sum_w e^(M_w - M) A_w / sum_w e^(M_w - M) L_w (deterministic).
// The query (float32, scaled by 1/sqrt(HD)) and the new key at p are rotated as in the chunked
// kernel; one query head of each key/value group writes the cache row at p, and every head selects
// the rotated key and the value at p (from LDS) in place of that cache row's words. Scores sum over
// a position's 16 lanes with DPP; the exponentials are __expf (exp2 of x log2 e).
template <int HD>
__global__ __launch_bounds__(ATT_WIDE_THREADS) void rope_attention_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ cache_k, uint16_t* __restrict__ cache_v, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, const int32_t* __restrict__ posp, uint16_t* __restrict__ out, int H, int Hkv,
    int S) {
  constexpr int P2 = HD / 2;               // rotated pairs of a head
  constexpr int DPL = HD / 16;             // dimensions per lane
  constexpr int WPL = DPL / 2;             // their 32-bit words
  constexpr int NW = ATT_WIDE_THREADS / 64;
  constexpr int PPL = ATT_WIDE_PPL / HD;   // positions of a lane group per step
  constexpr int STEP = 4 * PPL;            // positions of one wave step
  __shared__ float qs[HD], wm[NW], wl[NW], wacc[NW][HD];
  __shared__ uint32_t knp[P2], vnp[P2];   // the rotated new key and the new value at p, fp16 pairs
  const int h = blockIdx.x, m = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lg = (tid >> 4) & 3, j = tid & 15;
  int p = *posp;
  p = p < 0 ? 0 : p >= S ? S - 1 : p;
  const int group = H / Hkv, kh = h / group;
  const size_t kvrow = (size_t)Hkv * HD;   // elements of one cache position
  const uint16_t* ckm = cache_k + (size_t)m * S * kvrow + (size_t)kh * HD + j * DPL;
  const uint16_t* cvm = cache_v + (size_t)m * S * kvrow + (size_t)kh * HD + j * DPL;

  uint32_t kw[PPL][WPL], vw[PPL][WPL];
  auto load = [&](int t0) {   // positions past p read position p (its row is not used: kn, vn replace it)
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const size_t t = (size_t)min(t0 + lg + 4 * i, p);
      if constexpr (WPL == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(ckm + t * kvrow);
        const uint4 b = *reinterpret_cast<const uint4*>(cvm + t * kvrow);
        kw[i][0] = a.x; kw[i][1] = a.y; kw[i][2] = a.z; kw[i][3] = a.w;
        vw[i][0] = b.x; vw[i][1] = b.y; vw[i][2] = b.z; vw[i][3] = b.w;
      } else {
        const uint2 a = *reinterpret_cast<const uint2*>(ckm + t * kvrow);
        const uint2 b = *reinterpret_cast<const uint2*>(cvm + t * kvrow);
        kw[i][0] = a.x; kw[i][1] = a.y;
        vw[i][0] = b.x; vw[i][1] = b.y;
      }
    }
  };
  const int first = wave * STEP;
  if (first <= p) load(first);   // wave-uniform: the first step's loads before the rotation

  if (tid < P2) {   // rotate pair tid of the query (kept in float32, scaled), and of the new key
    const float co = rope_cos[(size_t)p * P2 + tid], si = rope_sin[(size_t)p * P2 + tid];
    const float scale = 1.0f / sqrtf((float)HD);
    const uint32_t qq = *reinterpret_cast<const uint32_t*>(q + ((size_t)m * H + h) * HD + 2 * tid);
    qs[2 * tid] = (lo16(qq) * co - hi16(qq) * si) * scale;
    qs[2 * tid + 1] = (lo16(qq) * si + hi16(qq) * co) * scale;
    const uint32_t kk = *reinterpret_cast<const uint32_t*>(k + ((size_t)m * Hkv + kh) * HD + 2 * tid);
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(v + ((size_t)m * Hkv + kh) * HD + 2 * tid);
    const uint32_t kr = to_f16(lo16(kk) * co - hi16(kk) * si) | (to_f16(lo16(kk) * si + hi16(kk) * co) << 16);
    knp[tid] = kr;
    vnp[tid] = vv;
    if (h % group == 0) {   // one query head of the group writes the cache; the others use knp, vnp
      *reinterpret_cast<uint32_t*>(cache_k + ((size_t)m * S + p) * kvrow + (size_t)kh * HD + 2 * tid) = kr;
      *reinterpret_cast<uint32_t*>(cache_v + ((size_t)m * S + p) * kvrow + (size_t)kh * HD + 2 * tid) = vv;
    }
  }
  __syncthreads();

  float qv[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) qv[d] = qs[j * DPL + d];
  uint32_t knw[WPL], vnw[WPL];   // this lane's words of the key and value at p: selected, not branched to
#pragma unroll
  for (int w = 0; w < WPL; ++w) {
    knw[w] = knp[j * WPL + w];
    vnw[w] = vnp[j * WPL + w];
  }
  float mx = -INFINITY, l = 0.0f, acc[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[d] = 0.0f;
  for (int t0 = first; t0 <= p; t0 += NW * STEP) {   // wave-uniform loop
    if (t0 != first) load(t0);
    float sc[PPL];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < PPL; ++i) {   // scores: a DPP sum over the 16 lanes of a position
      const int t = t0 + lg + 4 * i;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        const uint32_t kwd = t == p ? knw[w] : kw[i][w];
        s += qv[2 * w] * lo16(kwd) + qv[2 * w + 1] * hi16(kwd);
      }
      s = row_sum16(s);
      sc[i] = t <= p ? s : -INFINITY;
      bm = fmaxf(bm, sc[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));   // the step's maximum over the wave: finite (t0 <= p)
    const float nm = fmaxf(mx, bm);
    const float so = __expf(mx - nm);     // 0 on the wave's first step
    l *= so;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[d] *= so;
#pragma unroll
    for (int i = 0; i < PPL; ++i) {       // weighted values of this lane's positions
      const int t = t0 + lg + 4 * i;
      const float e = __expf(sc[i] - nm); // 0 past p
      l += e;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        const uint32_t vwd = t == p ? vnw[w] : vw[i][w];
        acc[2 * w] += e * lo16(vwd);
        acc[2 * w + 1] += e * hi16(vwd);
      }
    }
    mx = nm;
  }
  // the wave's 4 lane groups share its maximum: add their sums (a fixed xor tree), then the waves
  // meet in LDS (a wave with no positions brings M = -inf, L = 0, A = 0)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    acc[d] += __shfl_xor(acc[d], 16);
    acc[d] += __shfl_xor(acc[d], 32);
  }
  if (lg == 0) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) wacc[wave][j * DPL + d] = acc[d];
    if (j == 0) {
      wm[wave] = mx;
      wl[wave] = l;
    }
  }
  __syncthreads();
  if (tid < HD) {
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w]);   // finite: wave 0 holds position 0
    float L = 0.0f, A = 0.0f;
    for (int w = 0; w < NW; ++w) {   // waves in order: deterministic
      const float c = __expf(wm[w] - M);
      L += c * wl[w];
      A += c * wacc[w][tid];
    }
    out[((size_t)m * H + h) * HD + tid] = (uint16_t)to_f16(A / L);
  }
}

// The chunks of one (query head, sequence) combined in chunk order (deterministic), as a running
// softmax: M the largest maximum so far, L = sum_c e^(max_c - M) sum_c, A = sum_c e^(max_c - M)
// acc_c; out = A / L. A separate launch, so that every chunk's partial result is visible to it
// without fences. The partial results of every possible chunk are loaded before the position is
// known (those past the last chunk are ignored), so that the launch waits for memory once.
template <int HD>
__global__ __launch_bounds__(HD) void attention_combine_kernel(const int32_t* __restrict__ posp, const float* __restrict__ part,
                                                               uint16_t* __restrict__ out, int H, int S, int nsplit_max) {
  const size_t head = (size_t)blockIdx.y * H + blockIdx.x;
  const float* pb = part + head * nsplit_max * (HD + 2);
  const int tid = threadIdx.x;
  int p = *posp;
  float M = -INFINITY, L = 0.0f, A = 0.0f;
  constexpr int BATCH = 8;
  for (int c0 = 0; c0 < nsplit_max; c0 += BATCH) {
    float mc[BATCH], lc[BATCH], ac[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int cc = min(c0 + b, nsplit_max - 1);
      mc[b] = pb[cc * (HD + 2)];
      lc[b] = pb[cc * (HD + 2) + 1];
      ac[b] = pb[cc * (HD + 2) + 2 + tid];
    }
    p = p < 0 ? 0 : p >= S ? S - 1 : p;
    const int nsplit = (p + ATT_CHUNK) / ATT_CHUNK;
    if (nsplit == 1) return;   // the attention kernel wrote the output itself
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (c0 + b >= nsplit) break;
      const float nm = fmaxf(M, mc[b]);
      const float wo = expf(M - nm), wn = expf(mc[b] - nm);
      L = L * wo + lc[b] * wn;
      A = A * wo + ac[b] * wn;
      M = nm;
    }
    if (c0 + BATCH >= nsplit) break;
  }
  out[head * HD + tid] = (uint16_t)to_f16(A / L);
}

// The workspace of wq_rope_attention_noalloc: device memory the library holds, one copy per GPU,
// for callers that cannot allocate. In host code `scratch` names a host-side stand-in: its device
// address, found per device, is what kernels receive.
static __device__ __align__(256) unsigned char scratch[WQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device, looked up on the first call there.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return wq::device_status(e);
  if (dev < 0 || dev >= MAX_DEVICES) return wq::device_status(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return wq::device_status(e);
    if (!p) return wq::device_status(hipErrorInvalidSymbol);
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return WQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int64_t att_splits(int64_t max_seq) { return (max_seq + ATT_CHUNK - 1) / ATT_CHUNK; }

size_t att_part_bytes(int64_t M, int64_t H, int64_t hd, int64_t max_seq) {
  const size_t b = (size_t)M * H * att_splits(max_seq) * (hd + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
}

}  // namespace

extern "C" {

int wq_rope_table(double theta, int64_t head_dim, int64_t positions, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out || !(theta > 0.0)) return WQ_ERR_ARG;
  if (head_dim < 2 || head_dim % 2 || positions < 1) return WQ_ERR_SHAPE;
  const int64_t P2 = head_dim / 2;
  for (int64_t i = 0; i < P2; ++i) {
    const double f = std::pow(theta, -2.0 * (double)i / (double)head_dim);
    for (int64_t p = 0; p < positions; ++p) {
      const double a = (double)p * f;
      cos_out[p * P2 + i] = (float)std::cos(a);
      sin_out[p * P2 + i] = (float)std::sin(a);
    }
  }
  return WQ_OK;
}

int wq_embed(const uint16_t* table, const int32_t* tokens, float* x, int64_t M, int64_t d, int64_t vocab, void* stream) {
  if (!table || !tokens || !x || M < 0 || d < 0 || vocab < 0) return WQ_ERR_ARG;
  if (M < 1 || M > 65535 || d < 8 || d % 8 || vocab < 1 || vocab > INT32_MAX || d > (1 << 24)) return WQ_ERR_SHAPE;
  if (!aligned16(table) || !aligned16(x)) return WQ_ERR_ALIGN;
  return wq::device_status(launch(embed_kernel, dim3((unsigned)M), dim3(DEC_THREADS), 0, static_cast<hipStream_t>(stream),
                                  table, tokens, x, (int)d, (int)vocab));
}

int wq_add_rmsnorm(float* x, const uint16_t* delta, const uint16_t* g, float eps, uint16_t* out, int64_t M, int64_t d,
                   void* stream) {
  if (!x || !g || !out || M < 0 || d < 0 || !(eps >= 0.0f)) return WQ_ERR_ARG;
  if (M < 1 || M > 65535 || d < 8 || d % 8 || d > (1 << 24)) return WQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(g) || !aligned16(out) || (delta && !aligned16(delta))) return WQ_ERR_ALIGN;
  return wq::device_status(launch(add_rmsnorm_kernel, dim3((unsigned)M), dim3(DEC_THREADS), 0,
                                  static_cast<hipStream_t>(stream), x, delta, g, eps, out, (int)d));
}

size_t wq_attention_workspace_bytes(int64_t M, int64_t n_heads, int64_t head_dim, int64_t max_seq) {
  if (M < 1 || n_heads < 1 || head_dim < 1 || max_seq < 1) return 0;
  if (max_seq <= ATT_WIDE_MAX) return 0;   // one workgroup per head: no partial results leave it
  return att_part_bytes(M, n_heads, head_dim, max_seq);
}

namespace {
// The argument checks of wq_rope_attention that do not concern its workspace.
int check_attention_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* cache_k,
                         const uint16_t* cache_v, const float* rope_cos, const float* rope_sin, const int32_t* pos,
                         const uint16_t* out, int64_t M, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                         int64_t max_seq) {
  if (!q || !k || !v || !cache_k || !cache_v || !rope_cos || !rope_sin || !pos || !out) return WQ_ERR_ARG;
  if (M < 0 || n_heads < 0 || n_kv_heads < 0 || head_dim < 0 || max_seq < 0) return WQ_ERR_ARG;
  if (M < 1 || M > 65535 || n_heads < 1 || n_heads > 65535 || n_kv_heads < 1 || n_heads % n_kv_heads ||
      (head_dim != 64 && head_dim != 128) || max_seq < 1 || max_seq > (1 << 24) ||
      (double)M * max_seq * n_kv_heads * head_dim > 9.0e15)
    return WQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cache_k) || !aligned16(cache_v) ||
      !aligned16(out) || !aligned16(rope_cos) || !aligned16(rope_sin))
    return WQ_ERR_ALIGN;
  return WQ_OK;
}
}  // namespace

int wq_rope_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* cache_k, uint16_t* cache_v,
                      const float* rope_cos, const float* rope_sin, const int32_t* pos, uint16_t* out, int64_t M,
                      int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t max_seq, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const int st = check_attention_args(q, k, v, cache_k, cache_v, rope_cos, rope_sin, pos, out, M, n_heads, n_kv_heads,
                                      head_dim, max_seq);
  if (st != WQ_OK) return st;
  const size_t need = wq_attention_workspace_bytes(M, n_heads, head_dim, max_seq);
  if (need && (!workspace || workspace_bytes < need)) return WQ_ERR_ARG;
  if (need && !aligned16(workspace)) return WQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_seq <= ATT_WIDE_MAX) {   // one workgroup per (query head, sequence), one launch
    const dim3 gw((unsigned)n_heads, (unsigned)M);
    return wq::device_status(
        head_dim == 128
            ? launch(rope_attention_wide_kernel<128>, gw, dim3(ATT_WIDE_THREADS), 0, s, q, k, v, cache_k, cache_v,
                     rope_cos, rope_sin, pos, out, (int)n_heads, (int)n_kv_heads, (int)max_seq)
            : launch(rope_attention_wide_kernel<64>, gw, dim3(ATT_WIDE_THREADS), 0, s, q, k, v, cache_k, cache_v,
                     rope_cos, rope_sin, pos, out, (int)n_heads, (int)n_kv_heads, (int)max_seq));
  }
  const int splits = (int)att_splits(max_seq);
  float* part = static_cast<float*>(workspace);
  const dim3 grid((unsigned)splits, (unsigned)n_heads, (unsigned)M);
  hipError_t e =
      head_dim == 128
          ? launch(rope_attention_kernel<128>, grid, dim3(DEC_THREADS), 0, s, q, k, v, cache_k, cache_v, rope_cos, rope_sin,
                   pos, out, (int)n_heads, (int)n_kv_heads, (int)max_seq, part, splits)
          : launch(rope_attention_kernel<64>, grid, dim3(DEC_THREADS), 0, s, q, k, v, cache_k, cache_v, rope_cos, rope_sin,
                   pos, out, (int)n_heads, (int)n_kv_heads, (int)max_seq, part, splits);
  if (e == hipSuccess && splits > 1) {   // a cache of more than one chunk: the combine launch
    const dim3 g2((unsigned)n_heads, (unsigned)M);
    e = head_dim == 128
            ? launch(attention_combine_kernel<128>, g2, dim3(128), 0, s, pos, (const float*)part, out, (int)n_heads,
                     (int)max_seq, splits)
            : launch(attention_combine_kernel<64>, g2, dim3(64), 0, s, pos, (const float*)part, out, (int)n_heads,
                     (int)max_seq, splits);
  }
  return wq::device_status(e);
}

int wq_rope_attention_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* cache_k,
                              uint16_t* cache_v, const float* rope_cos, const float* rope_sin, const int32_t* pos,
                              uint16_t* out, int64_t M, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                              int64_t max_seq, void* stream) {
  const int st = check_attention_args(q, k, v, cache_k, cache_v, rope_cos, rope_sin, pos, out, M, n_heads, n_kv_heads,
                                      head_dim, max_seq);
  if (st != WQ_OK) return st;
  const size_t need = wq_attention_workspace_bytes(M, n_heads, head_dim, max_seq);
  if (need > WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERR_SCRATCH;
  void* ws = nullptr;
  if (need) {
    const int s2 = scratch_on_current_device(&ws);
    if (s2 != WQ_OK) return s2;
  }
  return wq_rope_attention(q, k, v, cache_k, cache_v, rope_cos, rope_sin, pos, out, M, n_heads, n_kv_heads, head_dim,
                           max_seq, ws, need ? (size_t)WQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int wq_silu_mul(const uint16_t* gate, const uint16_t* up, uint16_t* out, int64_t n, void* stream) {
  if (!gate || !up || !out || n < 0) return WQ_ERR_ARG;
  if (n < 8 || n % 8 || n / 8 > INT32_MAX) return WQ_ERR_SHAPE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(out)) return WQ_ERR_ALIGN;
  const int64_t n8 = n / 8;
  return wq::device_status(launch(silu_mul_kernel, dim3((unsigned)((n8 + DEC_THREADS - 1) / DEC_THREADS)),
                                  dim3(DEC_THREADS), 0, static_cast<hipStream_t>(stream), gate, up, out, (int)n8));
}

int wq_argmax_next(const uint16_t* logits, int64_t M, int64_t vocab, int32_t* tokens, int32_t* pos, void* stream) {
  if (!logits || !tokens || !pos || M < 0 || vocab < 0) return WQ_ERR_ARG;
  if (M < 1 || M > 65535 || vocab < 8 || vocab % 8 || vocab > INT32_MAX) return WQ_ERR_SHAPE;
  if (!aligned16(logits)) return WQ_ERR_ALIGN;
  return wq::device_status(launch(argmax_kernel, dim3((unsigned)M), dim3(DEC_THREADS), 0, static_cast<hipStream_t>(stream),
                                  logits, (int)vocab, tokens, pos));
}

}  // extern "C"
