// Device half of libwq: fused dequant + linear kernels for gfx950 (CDNA4), and wq_dequant.
//
// The FP6-LLM news page (m.zhengruan.com), section "重新设计内核方案", describes the
// computation these kernels perform. Low-bit weights are re-packed offline into aligned
// blocks, loaded, turned into fp16 values in registers, and fed to the matrix units,
// with dequantization and the product in ONE kernel, so that no fp16 weight tensor is
// ever written to memory. The gpt-fast write-up (m.greenbasetech.com) explains why this
// is the decode lever: the layer is bound by memory bandwidth, and the bytes per
// parameter set the speed.
//
// gfx950 design:
//  * Layout: row-major, 32-code units (32/16/24/16/64 bytes for W8/W4/W6/FP4/F16). Lane l of a
//    wave reads unit l of a 64-unit "chunk" of one row, so one wave-load covers 1-4 KB
//    contiguously.
//  * Decode in VGPRs, exact:
//      W8  offset-binary byte u = q+128 -> fp16 (1024+u) by v_perm_b32 against 0x64,
//          then -1152 (v_pk_add_f16).
//      W4  nibble pairs -> fp16 (1024+q) / (1024+16q) by one v_and_or_b32, then one
//          v_pk_fma_f16 gives q-z.
//      W6  the 192-bit unit goes through gfx950's v_cvt_scalef32_pk32_f16_bf6 at scale 1.0,
//          which yields the 32 e3m2 values as exact fp16.
//      FP4 each byte (two e2m1 codes) goes through gfx950's v_cvt_scalef32_pk_f16_fp4 at
//          scale 1.0: two exact fp16 values per instruction.
//  * M <= GEMV_MAX_M: VALU GEMV. v_dot2_f32_f16 accumulates in fp32, lanes run along K,
//    and each row's sum finishes with a DPP + cross-row shuffle wave reduction; waves of a
//    workgroup split K and add their partials through LDS in a fixed order.
//  * Larger M: v_mfma_f32_16x16x32_f16. Lane (n = l%16, q = l/16) decodes a unit into the B
//    fragment; the A fragment is x at the same K positions, since any permutation of K
//    applied to both operands leaves the product unchanged. W6, FP4 and W4 (K % 256 == 0)
//    read their weights row-contiguously into per-wave LDS first (lm_kernel); W8, F16 and
//    the other W4 shapes load fragments straight from HBM (mfma_kernel).
//  * bfloat16 activations (WQ_ACT_BF16 in the format code) run the same kernels with
//    v_dot2_f32_bf16 and v_mfma_f32_16x16x32_bf16: the decode yields bfloat16 pairs (gfx950's
//    bf6 and fp4 converts have bf16 forms; W4 (128 + q) by the same nibble placement against
//    128.0; W8 through byte-to-float converts), and y is rounded once to bfloat16.
//  * A grouped call runs several linears in one launch with one of these kernel families.
//  * No atomics anywhere, so every result is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <numeric>
#include <cstdint>
#include <cstdio>

#include "wq_device.h"
#include "wq_internal.h"

namespace {

constexpr int GEMV_MAX_M = 4;   // largest M served by the VALU GEMV; above it the MFMA kernel runs
constexpr int MFMA_M = 16;      // rows of x per MFMA launch
constexpr int GEMV_WAVES = 4;   // waves per workgroup of the GEMV (row blocks x split of K)
constexpr int MFMA_MAX_WAVES = 8;   // waves per workgroup of the MFMA kernel

// The waves that split K (WK) are a power of two (1, 2, 4 or 8; the planner picks no other),
// so a wave's share of the work is found with shifts and masks on its wave-uniform index.
__device__ __forceinline__ int wk_log2(int WK) { return __builtin_ctz((unsigned)WK); }

// ---------------------------------------------------------------- GEMV (M <= GEMV_MAX_M)
// Lanes run along K. Lane l of a wave owns one "segment" of SEG consecutive K of a row
// and reads its weight bytes with one 16-byte load (W6: a 16-byte and an 8-byte load),
// so every load instruction of a wave reads one contiguous block:
//   W4: SEG = 32 (one unit = one zero-point group)   W6: SEG = 32 (one unit, two planes)
//   FP4: SEG = 32 (one unit)    W8: SEG = 16 (half a unit)    F16: SEG = 8
// A wave covers a chunk of 64 segments of B rows. A workgroup of 4 waves holds 4 / WK row
// blocks of B rows; the WK waves of a block take the chunks c = wave, wave + WK, ... and
// double-buffer them: while chunk i is decoded, the loads of chunk i+1 (x first, then the
// B rows) are in flight.
//
// The decode skips the per-weight bias and zero-point subtraction. A lane dots x with
// the biased fp16 values it forms in one v_and_or_b32 / v_perm_b32:
//   W8: (1152 + q)                         -> sum - 1152 X
//   W4: (1024 + q) from nibbles 0 and 2 (fp16 exponent of 1024: mantissa step 1),
//       (64 + q)   from nibbles 1 and 3 (exponent of 64, so the nibble's 16 q is q)
//                                          -> one dot2 chain that starts at
//                                             -(1024 X_lo + 64 X_hi + z (X_lo + X_hi))
// where X, X_lo, X_hi are sums of x over the segment, shared by all rows of the wave.
// Every product is exact in fp32; one-hot inputs give exact results.
template <int FMT> constexpr int seg_codes() { return wfmt(FMT) == WQ_FMT_W8 ? 16 : wfmt(FMT) == WQ_FMT_F16 ? 8 : 32; }

template <int FMT> struct Seg { uint4 a; };
template <> struct Seg<WQ_FMT_W6E3M2> { uint4 a; uint2 b; };
template <> struct Seg<WQ_FMT_W6E3M2_P24> { uint4 a; uint2 b; };
template <> struct Seg<WQ_FMT_W5E2M2> { uint4 a; uint32_t b; };   // W3: Seg's .x .y .z hold its 12 bytes

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int FMT, int M, int B>
struct GemvStage {
  h2 x[M][seg_codes<FMT>() / 2];
  Seg<wfmt(FMT)> w[B];
  // W4, W3: the group's fp16 scale (.x) and zero point (.y) in one register: the zero lands in
  // the high half straight from its load (a d16_hi load), so a stage in flight holds one register
  // per row for its metadata
  u16x2 sz[group_meta(FMT) ? B : 1];
};

// Base pointers are a kernel argument plus a wave-uniform offset (uniform() keeps it in
// SGPRs), so the loads take the SGPR-base + 32-bit lane offset form.
template <int FMT, int M, int B>
__device__ __forceinline__ void gemv_load(GemvStage<FMT, M, B>& st, const uint16_t* __restrict__ x,
                                          const uint8_t* __restrict__ w, const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ zeros, int row0, int N, int K, int c, int lane) {
  constexpr int L = seg_codes<FMT>();
  const int S = K / L;                         // segments per row
  const uint32_t sg = (uint32_t)min(c * 64 + lane, S - 1);   // lanes past the row end read a valid segment, masked later
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint8_t* xr = reinterpret_cast<const uint8_t*>(x) + uniform((size_t)m * K * 2);
    const uint4* xp = reinterpret_cast<const uint4*>(xr + 2u * L * sg);
#pragma unroll
    for (int i = 0; i < L / 8; ++i) {
      const uint4 v = xp[i];
      st.x[m][4 * i] = as_h2(v.x); st.x[m][4 * i + 1] = as_h2(v.y);
      st.x[m][4 * i + 2] = as_h2(v.z); st.x[m][4 * i + 3] = as_h2(v.w);
    }
  }
  const size_t row_bytes = (size_t)K * unit_bytes<FMT>() / 32;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int n = min(row0 + b, N - 1);
    const uint8_t* row = w + uniform((size_t)n * row_bytes);
    if constexpr (w6_geom(FMT)) {
      uint32_t lo, hi;
      w6_homes(sg, S, lo, hi);
      st.w[b].a = ld_nt16(row + lo);
      st.w[b].b = ld_nt8(row + hi);
    } else if constexpr (wfmt(FMT) == WQ_FMT_W3G32) {
      st.w[b].a = ld_nt12(row + 12u * sg);
    } else if constexpr (wfmt(FMT) == WQ_FMT_W5E2M2) {
      uint32_t lo, hi;
      w5_homes(sg, S, lo, hi);
      st.w[b].a = ld_nt16(row + lo);
      st.w[b].b = ld_nt4(row + hi);
    } else {
      st.w[b].a = ld_nt16(row + 16u * sg);
    }
    if constexpr (group_meta(FMT)) {
      // one 32-bit offset serves the scale and the zero (each array holds N*K/16 < 2^32 bytes, as
      // N*K/32 < 2^31), so both loads take the kernel-argument base in SGPRs plus this lane offset
      // (with a 64-bit wave-uniform row offset the compiler formed a 64-bit address per load on the
      // VALU; int3 at M = 1 12.67 -> 12.44 us, W4 13.22 -> 13.16)
      const uint32_t mo = (uint32_t)n * (uint32_t)(2 * S) + 2u * sg;
      st.sz[b].x = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(scales) + mo);
      st.sz[b].y = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(zeros) + mo);
    }
  }
}

// bfloat16 activations: W4 (128 + q) in one v_and_or_b32 per pair (against 128.0, whose bfloat16
// mantissa step is 1), the chain starting at -(128 + z) X; W8 (128 + q) through byte-to-float
// converts, the sum starting at -128 X; W6 and FP4 through the bf16 forms of the converts.
template <int FMT, int M, int B>
__device__ __forceinline__ void gemv_compute_bf16(const GemvStage<FMT, M, B>& st, float (&acc)[B][M]) {
  constexpr int F = wfmt(FMT);
  constexpr int P = seg_codes<FMT>() / 2;   // pairs per segment
  const h2 ones = as_h2(0x3F803F80u);       // bfloat16 (1, 1)
  const auto& xp = st.x;
  float sx[M];
  if constexpr (F == WQ_FMT_W4G32 || F == WQ_FMT_W8) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int p = 0; p < P; p += 2) {
        a = dot2_bf16(xp[m][p], ones, a);
        c = dot2_bf16(xp[m][p + 1], ones, c);
      }
      sx[m] = a + c;
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) {
    h2 v[P];
    if constexpr (F == WQ_FMT_W4G32) {
      const uint32_t m0 = in_vgpr(0x000F000Fu), mag = in_vgpr(0x43004300u);
      const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // pair t of word i: codes 8i+2t (nibble t), 8i+2t+1 (nibble t+4)
        v[4 * i] = as_h2((wd[i] & m0) | mag);
        v[4 * i + 1] = as_h2(((wd[i] >> 4) & m0) | mag);
        v[4 * i + 2] = as_h2(((wd[i] >> 8) & m0) | mag);
        v[4 * i + 3] = as_h2(((wd[i] >> 12) & m0) | mag);
      }
      const float s = f16_to_f32(st.sz[b].x), z = f16_to_f32(st.sz[b].y);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float t = -(128.0f + z) * sx[m];
#pragma unroll
        for (int p = 0; p < 16; ++p) t = dot2_bf16(v[p], xp[m][p], t);
        acc[b][m] = __builtin_fmaf(s, t, acc[b][m]);
      }
      continue;
    } else if constexpr (F == WQ_FMT_W8) {
      const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // offset-binary bytes u = q + 128, exact in bfloat16
        v[2 * i] = pack_bf16((float)(wd[i] & 0xFFu), (float)((wd[i] >> 8) & 0xFFu));
        v[2 * i + 1] = pack_bf16((float)((wd[i] >> 16) & 0xFFu), (float)(wd[i] >> 24));
      }
    } else if constexpr (F == WQ_FMT_W6E3M2) {
      u32x6 u;
      u[0] = st.w[b].a.x; u[1] = st.w[b].a.y; u[2] = st.w[b].a.z; u[3] = st.w[b].a.w;
      u[4] = st.w[b].b.x; u[5] = st.w[b].b.y;
      const u32x16 h = __builtin_bit_cast(u32x16, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(u, 1.0f));
#pragma unroll
      for (int p = 0; p < 16; ++p) v[p] = as_h2(h[p]);
    } else if constexpr (F == WQ_FMT_W5E2M2) {
      h2 h[16];   // e2m2(code) * 2^-14 as fp16, then as bfloat16 (exact)
      decode_fp5(st.w[b].a, st.w[b].b, h);
#pragma unroll
      for (int p = 0; p < 16; ++p) v[p] = pack_bf16((float)h[p][0], (float)h[p][1]);
    } else if constexpr (F == WQ_FMT_W4E2M1) {
      const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[4 * i] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[i], 1.0f, 0));
        v[4 * i + 1] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[i], 1.0f, 1));
        v[4 * i + 2] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[i], 1.0f, 2));
        v[4 * i + 3] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[i], 1.0f, 3));
      }
    } else {   // BF16 weights
      v[0] = as_h2(st.w[b].a.x); v[1] = as_h2(st.w[b].a.y); v[2] = as_h2(st.w[b].a.z); v[3] = as_h2(st.w[b].a.w);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f, c = 0.f;
      if constexpr (F == WQ_FMT_W8) a = -128.0f * sx[m];
#pragma unroll
      for (int p = 0; p < P; p += 2) {
        a = dot2_bf16(v[p], xp[m][p], a);
        c = dot2_bf16(v[p + 1], xp[m][p + 1], c);
      }
      acc[b][m] += a + c;
    }
  }
}

template <int FMT, int M, int B>
__device__ __forceinline__ void gemv_compute(const GemvStage<FMT, M, B>& st, float (&acc)[B][M], bool active) {
  if (!active) return;
  if constexpr (bf16_act(FMT)) {
    gemv_compute_bf16<FMT, M, B>(st, acc);
    return;
  }
  constexpr int P = seg_codes<FMT>() / 2;   // fp16 pairs per segment
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  const auto& xp = st.x;
  if constexpr (wfmt(FMT) == WQ_FMT_W4G32) {
    const uint32_t m0 = in_vgpr(0x000F000Fu), m1 = in_vgpr(0x00F000F0u);
    const uint32_t mag_lo = in_vgpr(0x64006400u), mag_hi = in_vgpr(0x54005400u);
    float cx[M], sx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float xl = 0.f, xh = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xl = __builtin_amdgcn_fdot2(xp[m][4 * i], ones, xl, false);
        xh = __builtin_amdgcn_fdot2(xp[m][4 * i + 1], ones, xh, false);
        xl = __builtin_amdgcn_fdot2(xp[m][4 * i + 2], ones, xl, false);
        xh = __builtin_amdgcn_fdot2(xp[m][4 * i + 3], ones, xh, false);
      }
      cx[m] = __builtin_fmaf(1024.0f, xl, 64.0f * xh);
      sx[m] = xl + xh;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
      h2 v[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = wd[i], e = d >> 8;
        v[4 * i] = as_h2((d & m0) | mag_lo);       // codes 8i+0, 8i+1: 1024 + q
        v[4 * i + 1] = as_h2((d & m1) | mag_hi);   // codes 8i+2, 8i+3: 64 + q
        v[4 * i + 2] = as_h2((e & m0) | mag_lo);   // codes 8i+4, 8i+5
        v[4 * i + 3] = as_h2((e & m1) | mag_hi);   // codes 8i+6, 8i+7
      }
      const float s = f16_to_f32(st.sz[b].x), z = f16_to_f32(st.sz[b].y);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float t = -__builtin_fmaf(z, sx[m], cx[m]);
#pragma unroll
        for (int p = 0; p < 16; ++p) t = __builtin_amdgcn_fdot2(v[p], xp[m][p], t, false);
        acc[b][m] = __builtin_fmaf(s, t, acc[b][m]);
      }
    }
  } else if constexpr (wfmt(FMT) == WQ_FMT_W3G32) {
    // biased pairs 1024 + q, 128 + q, 16 + q by class (w3_class); the chain starts at
    // -(1024 X0 + 128 X1 + 16 X2 + z X) with Xc the sum of x over the pairs of class c
    const W3Masks w3m = w3_masks();
    float cx[M], sx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float xc[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 16; ++p) xc[w3_class(p)] = __builtin_amdgcn_fdot2(xp[m][p], ones, xc[w3_class(p)], false);
      cx[m] = __builtin_fmaf(1024.0f, xc[0], __builtin_fmaf(128.0f, xc[1], 16.0f * xc[2]));
      sx[m] = xc[0] + xc[1] + xc[2];
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      h2 v[16];
      decode_w3_biased(st.w[b].a, w3m, v);
      const float s = f16_to_f32(st.sz[b].x), z = f16_to_f32(st.sz[b].y);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float t = -__builtin_fmaf(z, sx[m], cx[m]);
#pragma unroll
        for (int p = 0; p < 16; ++p) t = __builtin_amdgcn_fdot2(v[p], xp[m][p], t, false);
        acc[b][m] = __builtin_fmaf(s, t, acc[b][m]);
      }
    }
  } else if constexpr (wfmt(FMT) == WQ_FMT_W8) {
    const uint32_t mag = in_vgpr(0x64646464u);
    float sx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int p = 0; p < P; p += 2) {
        a = __builtin_amdgcn_fdot2(xp[m][p], ones, a, false);
        c = __builtin_amdgcn_fdot2(xp[m][p + 1], ones, c, false);
      }
      sx[m] = -1152.0f * (a + c);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
      h2 v[P];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = as_h2(__builtin_amdgcn_perm(mag, wd[i], 0x04010400u));       // (1024+u0, 1024+u1)
        v[2 * i + 1] = as_h2(__builtin_amdgcn_perm(mag, wd[i], 0x04030402u));   // (1024+u2, 1024+u3)
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = sx[m], c = 0.f;
#pragma unroll
        for (int p = 0; p < P; p += 2) {
          a = __builtin_amdgcn_fdot2(v[p], xp[m][p], a, false);
          c = __builtin_amdgcn_fdot2(v[p + 1], xp[m][p + 1], c, false);
        }
        acc[b][m] += a + c;
      }
    }
  } else {
    [[maybe_unused]] const P24Masks p24m = wfmt(FMT) == WQ_FMT_W6E3M2_P24 ? p24_masks() : P24Masks{};
#pragma unroll
    for (int b = 0; b < B; ++b) {
      h2 v[P];
      if constexpr (wfmt(FMT) == WQ_FMT_W6E3M2) {
        u32x6 u;
        u[0] = st.w[b].a.x; u[1] = st.w[b].a.y; u[2] = st.w[b].a.z; u[3] = st.w[b].a.w;
        u[4] = st.w[b].b.x; u[5] = st.w[b].b.y;
        const h32 h = __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(u, 1.0f);
#pragma unroll
        for (int p = 0; p < 16; ++p) { v[p][0] = h[2 * p]; v[p][1] = h[2 * p + 1]; }
      } else if constexpr (wfmt(FMT) == WQ_FMT_W4E2M1) {
        const uint32_t wd[4] = {st.w[b].a.x, st.w[b].a.y, st.w[b].a.z, st.w[b].a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) decode_fp4_word(wd[i], v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      } else if constexpr (wfmt(FMT) == WQ_FMT_W5E2M2) {
        decode_fp5(st.w[b].a, st.w[b].b, v);
      } else if constexpr (wfmt(FMT) == WQ_FMT_W6E3M2_P24) {
        decode_p24(st.w[b].a, st.w[b].b, p24m, v);
      } else {
        v[0] = as_h2(st.w[b].a.x); v[1] = as_h2(st.w[b].a.y); v[2] = as_h2(st.w[b].a.z); v[3] = as_h2(st.w[b].a.w);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int p = 0; p < P; p += 2) {
          a = __builtin_amdgcn_fdot2(v[p], xp[m][p], a, false);
          c = __builtin_amdgcn_fdot2(v[p + 1], xp[m][p + 1], c, false);
        }
        acc[b][m] += a + c;
      }
    }
  }
}

// One workgroup's work: R = 4 / WK row blocks of B rows of one linear; the WK waves of
// each block split K. SILU (B even): rows 2i and 2i+1 are a gate row and an up row, and the
// output is silu(gate) * up of each pair (act [M, N / 2]), formed from the two rows' fp16
// results exactly as wq_silu_mul forms it.
template <int FMT, int M, int B, bool SILU = false>
__device__ __forceinline__ void gemv_body(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                          const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
                                          uint16_t* __restrict__ y, int N, int K, int block, int WK) {
  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar arithmetic
  const int lwk = wk_log2(WK);
  const int R = (blockDim.x >> 6) >> lwk;
  const int sub = wave_id >> lwk, wave = wave_id & (WK - 1);
  const int S = K / seg_codes<FMT>(), C = (S + 63) >> 6;
  const int row0 = (block * R + sub) * B;
  const int NI = wave < C ? (C - wave + WK - 1) >> lwk : 0;   // chunks of this wave (wave-uniform)
  float acc[B][M];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[b][m] = 0.0f;

  // Double-buffered chunk stream. No load sits under a branch that the compute of the
  // other buffer waits behind, so the wait before each compute covers only its own loads.
  GemvStage<FMT, M, B> A, Bf;
  auto chunk = [&](int i) { return wave + i * WK; };
  auto act = [&](int i) { return chunk(i) * 64 + lane < S; };
  if (NI > 0) {
    gemv_load<FMT, M, B>(A, x, w, scales, zeros, row0, N, K, chunk(0), lane);
    int i = 0;
    for (; i + 2 < NI; i += 2) {
      gemv_load<FMT, M, B>(Bf, x, w, scales, zeros, row0, N, K, chunk(i + 1), lane);
      gemv_compute<FMT, M, B>(A, acc, act(i));
      gemv_load<FMT, M, B>(A, x, w, scales, zeros, row0, N, K, chunk(i + 2), lane);
      gemv_compute<FMT, M, B>(Bf, acc, act(i + 1));
    }
    if (i + 1 < NI) {
      gemv_load<FMT, M, B>(Bf, x, w, scales, zeros, row0, N, K, chunk(i + 1), lane);
      gemv_compute<FMT, M, B>(A, acc, act(i));
      gemv_compute<FMT, M, B>(Bf, acc, act(i + 1));
    } else {
      gemv_compute<FMT, M, B>(A, acc, act(i));
    }
  }

  if (WK == 1) {   // each wave is its own row block: no cross-wave step
    [[maybe_unused]] uint16_t o16[B][M];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float t = wave_sum_to_lane63(acc[b][m]);
        const int n = row0 + b;
        if constexpr (SILU) {
          if constexpr (row_scaled<FMT>()) t *= f16_to_f32(scales[min(n, N - 1)]) * code_scale<FMT>();
          o16[b][m] = out16<FMT>(t);
        } else if (lane == 63 && n < N) {
          if constexpr (row_scaled<FMT>()) t *= f16_to_f32(scales[n]) * code_scale<FMT>();
          y[(size_t)m * N + n] = out16<FMT>(t);
        }
      }
    if constexpr (SILU) {
      static_assert(B % 2 == 0, "gate/up pairs need an even row count per wave");
      if (lane == 63)
#pragma unroll
        for (int b = 0; b < B; b += 2)
          if (row0 + b < N)
#pragma unroll
            for (int m = 0; m < M; ++m) y[(size_t)m * (N / 2) + (row0 + b) / 2] = silu_mul_f16(o16[b][m], o16[b + 1][m]);
    }
    return;
  }
  __shared__ float red[GEMV_WAVES][B * M];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float t = wave_sum_to_lane63(acc[b][m]);
      if (lane == 63) red[wave_id][b * M + m] = t;
    }
  __syncthreads();
  if constexpr (SILU) {
    if (wave == 0) {   // lane b * M + m holds (b, m); its pair partner (b + 1, m) is M lanes up
      const int b = lane / M, m = lane % M, n = row0 + b;
      const bool mine = lane < B * M && n < N;
      float t = 0.0f;
      if (lane < B * M)
        for (int i = 0; i < WK; ++i) t += red[sub * WK + i][lane];   // fixed order: deterministic
      if constexpr (row_scaled<FMT>()) t *= mine ? f16_to_f32(scales[n]) * code_scale<FMT>() : 1.0f;
      const uint16_t o = out16<FMT>(t);
      const uint16_t ou = (uint16_t)__shfl_down((int)o, M, 64);
      if (mine && (b & 1) == 0) y[(size_t)m * (N / 2) + n / 2] = silu_mul_f16(o, ou);
    }
    return;
  }
  if (wave == 0 && lane < B * M) {
    const int b = lane / M, m = lane % M, n = row0 + b;
    float t = 0.0f;
    for (int i = 0; i < WK; ++i) t += red[sub * WK + i][lane];   // fixed order: deterministic
    if (n < N) {
      if constexpr (row_scaled<FMT>()) t *= f16_to_f32(scales[n]) * code_scale<FMT>();
      y[(size_t)m * N + n] = out16<FMT>(t);
    }
  }
}

template <int FMT, int M, int B>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_kernel(const uint16_t* __restrict__ x,
                                                                   const uint8_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint16_t* __restrict__ zeros,
                                                                   uint16_t* __restrict__ y, int N, int K, int WK) {
  gemv_body<FMT, M, B>(x, w, scales, zeros, y, N, K, blockIdx.x, WK);
}

// gemv_kernel whose N rows are gate/up pairs: act [M, N / 2] = silu(gate) * up (see gemv_body).
template <int FMT, int M, int B>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_silu_kernel(const uint16_t* __restrict__ x,
                                                                   const uint8_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint16_t* __restrict__ zeros,
                                                                   uint16_t* __restrict__ act, int N, int K, int WK) {
  gemv_body<FMT, M, B, true>(x, w, scales, zeros, act, N, K, blockIdx.x, WK);
}

// Several independent linears of one format and one M in a single launch: the grid is the
// concatenation of their workgroups, so the machine ramps up and drains once for all of them.
// A wave finds its item without a dependent chain of scalar loads: the item boundaries are
// read at once and compared branch-free, and an item's fields sit in one 64-byte record that
// a single round of scalar loads brings in (the first loads of a launch miss every cache, so
// each dependent round before the first weight load adds to the launch's ramp-up).
constexpr int MAX_GROUP = 16;
struct GroupItem {
  const uint16_t* x;
  const uint8_t* w;
  const uint16_t* scales;
  const uint16_t* zeros;
  uint16_t* y;
  int N, K, WK, first_block;
  int pad[2];
};
static_assert(sizeof(GroupItem) == 64, "one item is one 64-byte record");
struct GemvGroup {
  int count;
  int first_block[MAX_GROUP];   // first workgroup of each item (prefix sums); INT_MAX past count
  GroupItem item[MAX_GROUP];
};

// The item of this workgroup: the number of later items whose first workgroup it has reached
// (b >= first_block[i] exactly when first_block[i] - b - 1 is negative: no overflow for
// 0 <= b, first_block[i] <= INT_MAX), counted in scalar arithmetic.
__device__ __forceinline__ const GroupItem& group_item(const GemvGroup& g) {
  const int b = blockIdx.x;
  int j = 0;
#pragma unroll
  for (int i = 1; i < MAX_GROUP; ++i) j += (int)((unsigned)(g.first_block[i] - b - 1) >> 31);
  return g.item[j];
}

template <int FMT, int M, int B>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_grouped_kernel(const GemvGroup g) {
  const GroupItem& it = group_item(g);
  gemv_body<FMT, M, B>(it.x, it.w, it.scales, it.zeros, it.y, it.N, it.K, blockIdx.x - it.first_block, it.WK);
}

// ---------------------------------------------------------------- MFMA, fragment loads (W8, F16, W4 with K % 256 != 0)
// v_mfma_f32_16x16x32_f16 with the weights as the B operand: lane (nl = l%16, q = l/16)
// decodes unit u = 4t+q of row nl of a 16-row block straight into its B fragment (8 K per
// MFMA step), and holds x[m = nl][the same K] as the A fragment (rows m >= M are zero).
// Any permutation of K applied to both operands leaves the product unchanged, so the
// unit order inside a 128-wide K tile is free. A wave covers RB row blocks, which share its
// x fragments; a workgroup holds R row groups x WK waves that take the K tiles t = kw,
// kw + WK, ..., double-buffered like the GEMV, and add their partials through LDS in a
// fixed order. Loads take a wave-uniform base plus a 32-bit lane offset.
template <int FMT, int RB>
struct MfmaStage {
  h8 xa[4];
  Raw<wfmt(FMT)> w[RB];
  uint16_t s[group_meta(FMT) ? RB : 1], z[group_meta(FMT) ? RB : 1];
};

template <int FMT, int RB>
__device__ __forceinline__ void mfma_load(MfmaStage<FMT, RB>& st, const uint16_t* __restrict__ x,
                                           const uint8_t* __restrict__ w, const uint16_t* __restrict__ scales,
                                           const uint16_t* __restrict__ zeros, int n0, int M, int N, int K, int t,
                                           int nl, int q) {
  constexpr int UB = unit_bytes<FMT>();
  const int U = K >> 5;
  const uint32_t u = (uint32_t)min(4 * t + q, U - 1);   // past the row end: a valid unit, masked later
  const uint32_t xo = (uint32_t)min(nl, M - 1) * (uint32_t)K * 2u + 64u * u;
  const uint4* xp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(x) + xo);
#pragma unroll
  for (int i = 0; i < 4; ++i) st.xa[i] = __builtin_bit_cast(h8, xp[i]);
  const uint32_t row_bytes = (uint32_t)U * UB;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int nb = min(n0 + 16 * r, N - 1);                        // wave-uniform
    const uint32_t nn = (uint32_t)(min(n0 + 16 * r + nl, N - 1) - nb);   // 0..15
    const uint8_t* rowb = w + uniform((size_t)nb * row_bytes);
    static_assert(!w6_geom(FMT) && wfmt(FMT) != WQ_FMT_W4E2M1 && wfmt(FMT) != WQ_FMT_W5E2M2,
                  "W6 (both layouts), FP4 and FP5 on the matrix cores take lm_kernel");
    const uint8_t* p = rowb + nn * row_bytes + UB * u;
    if constexpr (wfmt(FMT) == WQ_FMT_W3G32) st.w[r].a = ld_nt12(p);
    else st.w[r].a = ld_nt16(p);
    if constexpr (wfmt(FMT) == WQ_FMT_W8 || wfmt(FMT) == WQ_FMT_F16) st.w[r].b = ld_nt16(p + 16);
    if constexpr (wfmt(FMT) == WQ_FMT_F16) { st.w[r].c = ld_nt16(p + 32); st.w[r].d = ld_nt16(p + 48); }
    if constexpr (group_meta(FMT)) {
      const size_t mb = uniform((size_t)nb * U);
      st.s[r] = (scales + mb)[nn * U + u];
      st.z[r] = (zeros + mb)[nn * U + u];
    }
  }
}

template <int FMT, int RB>
__device__ __forceinline__ void mfma_compute(const MfmaStage<FMT, RB>& st, f4 (&acc)[RB], bool xrow, bool unit_ok) {
  const h8 zero8 = {};
  h8 xa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xa[i] = (xrow && unit_ok) ? st.xa[i] : zero8;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    h2 wv[16];
    if constexpr (bf16_act(FMT)) {
      if constexpr (wfmt(FMT) == WQ_FMT_W4G32) decode_bf16<FMT>(st.w[r], st.s[r], st.z[r], wv);
      else decode_bf16<FMT>(st.w[r], 0, 0, wv);
    } else {
      h2 zc1 = {}, zc2 = {};
      if constexpr (group_meta(FMT)) group_consts<FMT>(st.z[r], zc1, zc2);
      decode<FMT>(st.w[r], zc1, zc2, wv);
      if constexpr (group_meta(FMT)) {
        const _Float16 sv = __builtin_bit_cast(_Float16, st.s[r]);
        const h2 s2 = {sv, sv};
#pragma unroll
        for (int p = 0; p < 16; ++p) wv[p] = wv[p] * s2;   // fp16((q-z)*s): one rounding of an exact product
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r] = mfma16<FMT>(xa[i], frag_of(wv, i), acc[r]);
  }
}

template <int FMT, int RB, bool SILU = false>
__device__ __forceinline__ void mfma_body(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                           const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
                                           uint16_t* __restrict__ y, int M, int N, int K, int block, int WK) {
  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lwk = wk_log2(WK);
  const int R = (blockDim.x >> 6) >> lwk;
  const int sub = wave_id >> lwk, kw = wave_id & (WK - 1);
  const int nl = lane & 15, q = lane >> 4;
  const int U = K >> 5, T = (U + 3) >> 2;
  const int n0 = (block * R + sub) * 16 * RB;
  const int NI = kw < T ? (T - kw + WK - 1) >> lwk : 0;
  const bool xrow = nl < M;
  f4 acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  MfmaStage<FMT, RB> A, Bs;
  auto tile = [&](int i) { return kw + i * WK; };
  auto ok = [&](int i) { return 4 * tile(i) + q < U; };
  if (NI > 0) {
    mfma_load<FMT, RB>(A, x, w, scales, zeros, n0, M, N, K, tile(0), nl, q);
    __builtin_amdgcn_sched_barrier(0);   // keep the stage's loads ahead of the compute
    int i = 0;
    for (; i + 2 < NI; i += 2) {
      mfma_load<FMT, RB>(Bs, x, w, scales, zeros, n0, M, N, K, tile(i + 1), nl, q);
      __builtin_amdgcn_sched_barrier(0);   // keep the stage's loads ahead of the compute
      mfma_compute<FMT, RB>(A, acc, xrow, ok(i));
      mfma_load<FMT, RB>(A, x, w, scales, zeros, n0, M, N, K, tile(i + 2), nl, q);
      __builtin_amdgcn_sched_barrier(0);   // keep the stage's loads ahead of the compute
      mfma_compute<FMT, RB>(Bs, acc, xrow, ok(i + 1));
    }
    if (i + 1 < NI) {
      mfma_load<FMT, RB>(Bs, x, w, scales, zeros, n0, M, N, K, tile(i + 1), nl, q);
      __builtin_amdgcn_sched_barrier(0);   // keep the stage's loads ahead of the compute
      mfma_compute<FMT, RB>(A, acc, xrow, ok(i));
      mfma_compute<FMT, RB>(Bs, acc, xrow, ok(i + 1));
    } else {
      mfma_compute<FMT, RB>(A, acc, xrow, ok(i));
    }
  }

  // D[m][n] sits in lane (n + 16*(m/4)), register m%4. Row block r of this group is finished
  // by the group's wave r % WK, which adds the WK partials in a fixed order.
  auto store = [&](int r, const f4& t) {
    const int n = n0 + 16 * r + nl;
    if constexpr (SILU) {   // rows n, n ^ 1 (a gate/up pair) sit in lanes l, l ^ 1 (wave-uniform call)
      float sc = 1.0f;
      if constexpr (row_scaled<FMT>()) sc = f16_to_f32(scales[min(n, N - 1)]) * code_scale<FMT>();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const uint16_t o = out16<FMT>(t[i] * sc);
        const uint16_t ou = (uint16_t)__builtin_amdgcn_update_dpp(0, (int)o, 0xB1, 0xF, 0xF, false);   // lane ^ 1
        if (m < M && n < N && (nl & 1) == 0) y[(size_t)m * (N / 2) + n / 2] = silu_mul_f16(o, ou);
      }
      return;
    }
    if (n >= N) return;
    float sc = 1.0f;
    if constexpr (row_scaled<FMT>()) sc = f16_to_f32(scales[n]) * code_scale<FMT>();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      if (m < M) y[(size_t)m * N + n] = out16<FMT>(t[i] * sc);
    }
  };
  if (WK == 1) {
#pragma unroll
    for (int r = 0; r < RB; ++r) store(r, acc[r]);
    return;
  }
  __shared__ f4 red[MFMA_MAX_WAVES][RB][64];
#pragma unroll
  for (int r = 0; r < RB; ++r) red[wave_id][r][lane] = acc[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if ((r & (WK - 1)) != kw) continue;
    f4 t = red[sub * WK][r][lane];
    for (int i = 1; i < WK; ++i) t += red[sub * WK + i][r][lane];   // fixed order: deterministic
    store(r, t);
  }
}

template <int FMT, int RB>
__global__ __launch_bounds__(64 * MFMA_MAX_WAVES) void mfma_kernel(const uint16_t* __restrict__ x,
                                                                     const uint8_t* __restrict__ w,
                                                                     const uint16_t* __restrict__ scales,
                                                                     const uint16_t* __restrict__ zeros,
                                                                     uint16_t* __restrict__ y, int M, int N, int K,
                                                                     int WK) {
  mfma_body<FMT, RB>(x, w, scales, zeros, y, M, N, K, blockIdx.x, WK);
}

// mfma_kernel whose N rows are gate/up pairs: act [M, N / 2] = silu(gate) * up.
template <int FMT, int RB>
__global__ __launch_bounds__(64 * MFMA_MAX_WAVES) void mfma_silu_kernel(const uint16_t* __restrict__ x,
                                                                          const uint8_t* __restrict__ w,
                                                                          const uint16_t* __restrict__ scales,
                                                                          const uint16_t* __restrict__ zeros,
                                                                          uint16_t* __restrict__ act, int M, int N, int K,
                                                                          int WK) {
  mfma_body<FMT, RB, true>(x, w, scales, zeros, act, M, N, K, blockIdx.x, WK);
}

// Several linears of one format and one M in a single launch (see GemvGroup); each item keeps
// its own K split, and a workgroup holds blockDim / 64 / WK of its row groups.
template <int FMT, int RB>
__global__ __launch_bounds__(64 * MFMA_MAX_WAVES) void mfma_grouped_kernel(const GemvGroup g, int M) {
  const GroupItem& it = group_item(g);
  mfma_body<FMT, RB>(it.x, it.w, it.scales, it.zeros, it.y, M, it.N, it.K, blockIdx.x - it.first_block, it.WK);
}

// ---------------------------------------------------------------- W4 / W6 / FP4 on the matrix cores through LDS
// The fragment-shaped loads of mfma_kernel read, per wave instruction, 16 rows x 16 bytes
// (W4) or 16 rows x 64 + 32 bytes (W6), a pattern that HBM serves far below the rate of
// contiguous reads (16-byte row pieces at about a fifth). Here each wave reads its rows
// contiguously instead, 32 units (a "stage") of each of the 16 rows of a row block at a
// time, parks them in its own LDS region, and reads the MFMA B fragments from there. No
// barriers: the region belongs to one wave, and LDS operations of a wave complete in order.
//   W4: one wave instruction reads 2 rows x 512 B; the stage's scales and zeros (16 rows x
//       32 groups) come straight into registers, lane (n, q) holding groups 8q..8q+7 of
//       row n, which are exactly the groups its fragments need.
//   W6: the lo slices as 2 rows x 512 B per instruction, the hi slices as 4 rows x 256 B.
//   FP4: as W4 (16-byte units), with no metadata.
//   FP5: the 16-byte magnitude slices as W4, and one 4-byte sign word per unit and row.
// LDS image of one 16-row block (XOR swizzles put the 16 rows of a fragment read in
// different banks; gfx950 serves a 16-byte read in four groups of 16 lanes, and with the
// swizzle u ^ r instead of u ^ (r & 7) every fragment read lost 4 cycles to conflicts):
//   W4, FP4: unit u (0..31) of row r at 512 r + 16 (u ^ (r & 7))                         8 KB
//   W6: lo slice of unit u at 512 r + 16 (u ^ (r & 7)),
//       hi slice at 8192 + 256 r + 8 (u ^ (2r & 31))                                       12 KB
//   FP5: magnitude slice of unit u as W4, sign word at 8192 + 128 r + 4 (u ^ ((r >> 1) & 7))
//       (a 4-byte read serves 64 lanes over 64 banks: rows 2p and 2p+1 take either half)   10 KB
// K tile j (0..7) of a stage is 4 units, one per lane quad q: unit 4j + q, so that the 4 quads of a
// row read adjacent units of x (a wave's x load touches half as many cache lines as with unit 8q + j,
// which cost up to a fifth of the time at M = 16). W4 and W3 park the stage's group scales and zeros
// (loaded as 8 groups per lane) in the wave's LDS region too, and read each unit's pair from there:
//   W4, W3 metadata: scale of group g of row r at 8192 + 64 r + 2 (g ^ (((r >> 2) & 3) << 3)),
//       zero 1024 bytes further (the XOR spreads the 16 rows of a read over the banks)      +2 KB
// Its x fragments
// sit in a register ring of lm_xring slots and are loaded lm_xring - 1 tiles ahead (W4 keeps
// the ring at 2 so that its two-block kernel fits 256 VGPRs: two waves per SIMD).
template <int FMT> constexpr bool lm_w6() { return w6_geom(FMT); }   // two plane slices per unit (both FP6 layouts)
template <int FMT> constexpr bool lm_w5() { return wfmt(FMT) == WQ_FMT_W5E2M2; }   // 16-byte slice + sign word
template <int FMT> constexpr int lm_block() {
  return lm_w6<FMT>() ? 16 * 512 + 16 * 256 : lm_w5<FMT>() ? 16 * 512 + 16 * 128 : group_meta(FMT) ? 16 * 512 + 2048
                                                                                                 : 16 * 512;
}
template <int FMT> constexpr int lm_loads() { return lm_w6<FMT>() ? 12 : 8; }
template <int FMT, int MT> constexpr int lm_xring() { return group_meta(FMT) || MT > 1 ? 2 : 4; }
__device__ __forceinline__ int lm_unit(int q, int j) { return 4 * j + q; }
// byte offset, within a row block's LDS image, of the scale of group g (0..31) of row r (W4, W3)
__device__ __forceinline__ uint32_t lm_meta_off(int r, int g) { return 8192u + 64u * r + 2u * (g ^ (((r >> 2) & 3) << 3)); }
constexpr int LM_MAX_MT = 4;   // 16-row tiles of x per launch (M up to 64 reads the weights once)
constexpr int LM_WAVES = 4;   // waves per workgroup

template <int FMT, int RB>
struct LmStage {
  uint4 v[RB][lm_loads<FMT>()];
  uint4 s[group_meta(FMT) ? RB : 1], z[group_meta(FMT) ? RB : 1];   // W4, W3: 8 groups' fp16 scales / zeros
  uint32_t sg[lm_w5<FMT>() ? RB : 1][lm_w5<FMT>() ? 8 : 1];   // FP5: the sign words
};

// Global loads of stage h (units 32h .. 32h+31 of each row) of RB row blocks.
template <int FMT, int RB>
__device__ __forceinline__ void lm_load(LmStage<FMT, RB>& st, const uint8_t* __restrict__ w,
                                        const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int n0,
                                        int N, int K, int h, int lane) {
  const int U = K >> 5;
  const uint32_t row_bytes = (uint32_t)U * unit_bytes<FMT>();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int nb = min(n0 + 16 * r, N - 1);
    const uint8_t* rowb = w + uniform((size_t)nb * row_bytes);
    if constexpr (lm_w5<FMT>()) {
      const int c = h >> 1, half = h & 1;                  // 64-unit chunk and which half of it
      const int uc = min(64, U - 64 * c);                   // units in the chunk
      const uint32_t cbase = 64u * 20 * c;
      const int j = min(32 * half + (lane & 31), uc - 1);  // past the chunk end: a valid unit, masked later
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // lane l -> row 2i + l/32, unit l%32: its 16-byte slice and sign word
        const uint32_t nn = (uint32_t)(min(n0 + 16 * r + 2 * i + (lane >> 5), N - 1) - nb);
        st.v[r][i] = ld_nt16(rowb + nn * row_bytes + cbase + 16u * j);
        st.sg[r][i] = ld_nt4(rowb + nn * row_bytes + cbase + 16u * uc + 4u * j);
      }
    } else if constexpr (!lm_w6<FMT>()) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // lane l -> row 2i + l/32, unit l%32
        const uint32_t nn = (uint32_t)(min(n0 + 16 * r + 2 * i + (lane >> 5), N - 1) - nb);
        const uint32_t j = (uint32_t)min(32 * h + (lane & 31), U - 1);   // past the row end: a valid unit, masked later
        if constexpr (wfmt(FMT) == WQ_FMT_W3G32) st.v[r][i] = ld_nt12(rowb + nn * row_bytes + 12u * j);
        else st.v[r][i] = ld_nt16(rowb + nn * row_bytes + 16u * j);
      }
    }
    if constexpr (group_meta(FMT)) {
      // lane (n, q): groups 32h + 8q .. +7 of row n (U is a multiple of 8, so a group of 8 lies
      // wholly inside the row or wholly past its end; one past the end reads the row's last 8)
      const uint32_t nn = (uint32_t)(min(n0 + 16 * r + (lane & 15), N - 1) - nb);
      const int g0 = min(32 * h + 8 * (lane >> 4), U - 8);
      const size_t mb = uniform((size_t)nb * U * 2);
      const uint32_t mo = 2u * (nn * (uint32_t)U + (uint32_t)g0);
      st.s[r] = ld_nt16(reinterpret_cast<const uint8_t*>(scales) + mb + mo);
      st.z[r] = ld_nt16(reinterpret_cast<const uint8_t*>(zeros) + mb + mo);
    }
    if constexpr (lm_w6<FMT>()) {
      const int c = h >> 1, half = h & 1;                  // 64-unit chunk and which half of it
      const int uc = min(64, U - 64 * c);                   // units in the chunk
      const uint32_t cbase = 64u * 24 * c;
#pragma unroll
      for (int i = 0; i < 8; ++i) {   // lo: lane l -> row 2i + l/32, unit l%32
        const uint32_t nn = (uint32_t)(min(n0 + 16 * r + 2 * i + (lane >> 5), N - 1) - nb);
        const int j = min(32 * half + (lane & 31), uc - 1);   // past the chunk end: a valid unit, masked later
        st.v[r][i] = ld_nt16(rowb + nn * row_bytes + cbase + 16u * j);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // hi: lane l -> row 4i + l/16, units 2(l%16), 2(l%16)+1
        const uint32_t nn = (uint32_t)(min(n0 + 16 * r + 4 * i + (lane >> 4), N - 1) - nb);
        // when j0 is the chunk's last unit (odd uc), read the 16 bytes that end with its slice and
        // keep the second half: units j0-1, j0, or for a one-unit chunk (the last of a row of
        // 64c + 1 units) the end of the lo plane and the one slice. No branch: a branch between
        // the loads of a stage would make the compiler wait for them at the join.
        const int j0 = min(32 * half + 2 * (lane & 15), uc - 1);
        const uint32_t sh = (j0 + 1 >= uc) ? 8u : 0u;
        const uint4 v = ld_nt16(rowb + (nn * row_bytes + cbase + 16u * uc + 8u * j0 - sh));
        st.v[r][8 + i] = sh ? make_uint4(v.z, v.w, v.z, v.w) : v;
      }
    }
  }
}

// The ragged last stage of a row (nv < 32 valid units): units nv..31 were loaded from clamped
// addresses and must contribute nothing. W4 and W3 zero their group scales ((q - z) * 0 = 0); the
// other formats zero their bytes, whose code 0 is the value +0.
template <int FMT, int RB>
__device__ __forceinline__ void lm_zero_past_row(LmStage<FMT, RB>& st, int nv, int lane) {
  auto keep = [](uint4 v, bool ok) { return ok ? v : make_uint4(0u, 0u, 0u, 0u); };
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if constexpr (group_meta(FMT)) {
      // lane (n, q) holds the scales of units 8q .. 8q+7 of the stage, two per dword
      const int v = nv - 8 * (lane >> 4);
      const uint32_t m[4] = {(v > 0 ? 0xFFFFu : 0u) | (v > 1 ? 0xFFFF0000u : 0u),
                             (v > 2 ? 0xFFFFu : 0u) | (v > 3 ? 0xFFFF0000u : 0u),
                             (v > 4 ? 0xFFFFu : 0u) | (v > 5 ? 0xFFFF0000u : 0u),
                             (v > 6 ? 0xFFFFu : 0u) | (v > 7 ? 0xFFFF0000u : 0u)};
      st.s[r] = make_uint4(st.s[r].x & m[0], st.s[r].y & m[1], st.s[r].z & m[2], st.s[r].w & m[3]);
    } else {
      // lo slices (and FP4 units, FP5 magnitudes): lane l holds unit l % 32 of its rows
      const bool ok = (lane & 31) < nv;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.v[r][i] = keep(st.v[r][i], ok);
      if constexpr (lm_w5<FMT>()) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st.sg[r][i] = ok ? st.sg[r][i] : 0u;
      }
      if constexpr (lm_w6<FMT>()) {   // hi slices: lane l holds units 2(l % 16) and 2(l % 16) + 1
        const int u0 = 2 * (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = st.v[r][8 + i];
          st.v[r][8 + i] = make_uint4(u0 < nv ? v.x : 0u, u0 < nv ? v.y : 0u, u0 + 1 < nv ? v.z : 0u,
                                      u0 + 1 < nv ? v.w : 0u);
        }
      }
    }
  }
}

template <int FMT, int RB>
__device__ __forceinline__ void lm_store(const LmStage<FMT, RB>& st, uint8_t* lds, int lane) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    uint8_t* base = lds + r * lm_block<FMT>();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 2 * i + (lane >> 5), u = lane & 31;
      *reinterpret_cast<uint4*>(base + 512 * rr + 16 * (u ^ (rr & 7))) = st.v[r][i];
    }
    if constexpr (group_meta(FMT)) {   // lane (rr, qq) holds the scales and zeros of groups 8qq .. 8qq+7 of row rr
      const int rr = lane & 15, qq = lane >> 4;
      *reinterpret_cast<uint4*>(base + lm_meta_off(rr, 8 * qq)) = st.s[r];
      *reinterpret_cast<uint4*>(base + 1024 + lm_meta_off(rr, 8 * qq)) = st.z[r];
    }
    if constexpr (lm_w5<FMT>()) {   // sign word of unit u of row rr at 8192 + 128 rr + 4 (u ^ ((rr >> 1) & 7))
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 2 * i + (lane >> 5), u = lane & 31;
        *reinterpret_cast<uint32_t*>(base + 8192 + 128 * rr + 4 * (u ^ ((rr >> 1) & 7))) = st.sg[r][i];
      }
    }
    if constexpr (lm_w6<FMT>()) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * i + (lane >> 4), u = 2 * (lane & 15), sw = (2 * rr) & 31;
        *reinterpret_cast<uint2*>(base + 8192 + 256 * rr + 8 * (u ^ sw)) = make_uint2(st.v[r][8 + i].x, st.v[r][8 + i].y);
        *reinterpret_cast<uint2*>(base + 8192 + 256 * rr + 8 * ((u + 1) ^ sw)) = make_uint2(st.v[r][8 + i].z, st.v[r][8 + i].w);
      }
    }
  }
}

// A workgroup of LM_WAVES waves holds R = LM_WAVES / WK row groups of 16 RB rows; the WK
// waves of a group take the stages h = kw, kw + WK, ...
template <int FMT, int RB, int MT, bool SILU = false>
__device__ __forceinline__ void lm_body(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                        const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
                                        uint16_t* __restrict__ y, int M, int N, int K, int block, int WK) {
  extern __shared__ uint4 lm_lds[];
  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lwk = wk_log2(WK);
  const int R = LM_WAVES >> lwk;
  const int sub = wave_id >> lwk, kw = wave_id & (WK - 1);
  const int nl = lane & 15, q = lane >> 4;
  const int U = K >> 5, H = (U + 31) >> 5;
  const int n0 = (block * R + sub) * 16 * RB;
  const int NI = kw < H ? (H - kw + WK - 1) >> lwk : 0;
  uint8_t* lds = reinterpret_cast<uint8_t*>(lm_lds) + wave_id * RB * lm_block<FMT>();
  f4 acc[RB][MT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[r][mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  LmStage<FMT, RB> st;
  constexpr int XR = lm_xring<FMT, MT>();
  [[maybe_unused]] const W4Masks w4m = wfmt(FMT) == WQ_FMT_W4G32 && !bf16_act(FMT) ? w4_masks() : W4Masks{};
  [[maybe_unused]] const W3Masks w3m = wfmt(FMT) == WQ_FMT_W3G32 ? w3_masks() : W3Masks{};
  [[maybe_unused]] const P24Masks p24m = wfmt(FMT) == WQ_FMT_W6E3M2_P24 ? p24_masks() : P24Masks{};
  // x fragments. Row m of the product depends only on row m of x, so the lanes of rows past M load
  // row M - 1 again and their outputs are not stored (loading nothing there, under an exec mask,
  // was slower). Units past the row end (the ragged last stage) contribute nothing because their
  // weights are zeroed when the stage is parked.
  h8 xr[XR][MT][4];
  auto xload = [&](int t) {   // x[m = 16 mt + nl][unit 32h + lm_unit(q, j)] of K tile t = 8i + j
    const int h = kw + (t >> 3) * WK, j = t & 7;
    const uint32_t u = (uint32_t)min(32 * h + lm_unit(q, j), U - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* xp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(x) +
                                                       (uint32_t)min(16 * mt + nl, M - 1) * (uint32_t)K * 2u + 64u * u);
#pragma unroll
      for (int k = 0; k < 4; ++k) xr[t % XR][mt][k] = __builtin_bit_cast(h8, xp[k]);
    }
  };
  auto park = [&](int h) {   // the loaded stage h -> LDS (W4 and W3: with its metadata)
    if (32 * h + 32 > U) lm_zero_past_row<FMT, RB>(st, U - 32 * h, lane);   // wave-uniform: the ragged last stage
    lm_store<FMT, RB>(st, lds, lane);
  };
  if (NI > 0) {
#pragma unroll
    for (int t = 0; t + 1 < XR; ++t) xload(t);
    lm_load<FMT, RB>(st, w, scales, zeros, n0, N, K, kw, lane);
    park(kw);
  }
  for (int i = 0; i < NI; ++i) {
    const int h = kw + i * WK;
    if (i + 1 < NI) lm_load<FMT, RB>(st, w, scales, zeros, n0, N, K, h + WK, lane);
    __builtin_amdgcn_sched_barrier(0);   // keep the next stage's loads ahead of the compute
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 8 * i + j;
      if (j + XR - 1 < 8 || i + 1 < NI) xload(t + XR - 1);
      const int u = lm_unit(q, j);   // unit within the stage
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const uint8_t* base = lds + r * lm_block<FMT>();
        Raw<wfmt(FMT)> raw;
        raw.a = *reinterpret_cast<const uint4*>(base + 512 * nl + 16 * (u ^ (nl & 7)));
        if constexpr (w6_geom(FMT))
          raw.b = *reinterpret_cast<const uint2*>(base + 8192 + 256 * nl + 8 * (u ^ ((2 * nl) & 31)));
        if constexpr (lm_w5<FMT>())
          raw.b = *reinterpret_cast<const uint32_t*>(base + 8192 + 128 * nl + 4 * (u ^ ((nl >> 1) & 7)));
        [[maybe_unused]] uint16_t sb = 0, zb = 0;   // W4, W3: this unit's group scale and zero
        if constexpr (group_meta(FMT)) {
          sb = *reinterpret_cast<const uint16_t*>(base + lm_meta_off(nl, u));
          zb = *reinterpret_cast<const uint16_t*>(base + 1024 + lm_meta_off(nl, u));
        }
        h2 wv[16];
        if constexpr (bf16_act(FMT)) {
          if constexpr (wfmt(FMT) == WQ_FMT_W4G32) decode_bf16<FMT>(raw, sb, zb, wv);
          else decode_bf16<FMT>(raw, 0, 0, wv);
        } else {
          if constexpr (wfmt(FMT) == WQ_FMT_W4G32) {
            h2 zc1, zc2;
            w4_consts(zb, zc1, zc2);
            decode_w4_unit(raw.a, zc1, zc2, w4m, wv);
            const _Float16 sv = __builtin_bit_cast(_Float16, sb);
            const h2 s2 = {sv, sv};
#pragma unroll
            for (int p = 0; p < 16; ++p) wv[p] = wv[p] * s2;   // fp16((q-z)*s): one rounding of an exact product
          } else if constexpr (wfmt(FMT) == WQ_FMT_W3G32) {
            h2 zc[3];
            w3_consts(zb, zc);
            decode_w3_unit(raw.a, zc, w3m, wv);
            const _Float16 sv = __builtin_bit_cast(_Float16, sb);
            const h2 s2 = {sv, sv};
#pragma unroll
            for (int p = 0; p < 16; ++p) wv[p] = wv[p] * s2;   // fp16((q-z)*s): one rounding of an exact product
          } else if constexpr (wfmt(FMT) == WQ_FMT_W6E3M2_P24) {
            decode_p24(raw.a, raw.b, p24m, wv);
          } else {
            decode<FMT>(raw, h2{}, h2{}, wv);
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const h8 b = frag_of(wv, k);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[r][mt] = mfma16<FMT>(xr[t % XR][mt][k], b, acc[r][mt]);
        }
      }
    }
    if (i + 1 < NI) park(h + WK);
  }

  // WK partials through LDS (every wave is done with its region after the barrier), fixed
  // order; D[m][n] of x tile mt sits in lane (n + 16*(m/4)), register m%4
  __syncthreads();
  f4* red = reinterpret_cast<f4*>(lm_lds);
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[((wave_id * RB + r) * MT + mt) * 64 + lane] = acc[r][mt];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if ((r & (WK - 1)) != kw) continue;
    const int n = n0 + 16 * r + nl;
    const float sc = row_scaled<FMT>() && n < N ? f16_to_f32(scales[n]) * code_scale<FMT>() : 1.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f4 t = red[(((sub * WK) * RB + r) * MT + mt) * 64 + lane];
      for (int k = 1; k < WK; ++k) t += red[(((sub * WK + k) * RB + r) * MT + mt) * 64 + lane];
      if constexpr (SILU) {   // rows n, n ^ 1 (a gate/up pair) sit in lanes l, l ^ 1
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int m = 16 * mt + 4 * q + k;
          const uint16_t o = out16<FMT>(t[k] * sc);
          const uint16_t ou = (uint16_t)__builtin_amdgcn_update_dpp(0, (int)o, 0xB1, 0xF, 0xF, false);   // lane ^ 1
          if (m < M && n < N && (nl & 1) == 0) y[(size_t)m * (N / 2) + n / 2] = silu_mul_f16(o, ou);
        }
        continue;
      }
      if (n < N) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int m = 16 * mt + 4 * q + k;
          if (m < M) y[(size_t)m * N + n] = out16<FMT>(t[k] * sc);
        }
      }
    }
  }
}

// MT 16-row tiles of x (M <= 16 MT) share each decoded weight fragment, so the weights are
// read once for up to 64 rows of x.
template <int FMT, int RB, int MT>
__global__ __launch_bounds__(64 * LM_WAVES) void lm_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                          int M, int N, int K, int WK) {
  lm_body<FMT, RB, MT>(x, w, scales, zeros, y, M, N, K, blockIdx.x, WK);
}

// lm_kernel whose N rows are gate/up pairs: act [M, N / 2] = silu(gate) * up.
template <int FMT, int RB, int MT>
__global__ __launch_bounds__(64 * LM_WAVES) void lm_silu_kernel(const uint16_t* __restrict__ x,
                                                               const uint8_t* __restrict__ w,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint16_t* __restrict__ zeros,
                                                               uint16_t* __restrict__ act, int M, int N, int K, int WK) {
  lm_body<FMT, RB, MT, true>(x, w, scales, zeros, act, M, N, K, blockIdx.x, WK);
}

// Several linears in a single launch (see GemvGroup), each with its own K split.
template <int FMT, int RB, int MT>
__global__ __launch_bounds__(64 * LM_WAVES) void lm_grouped_kernel(const GemvGroup g, int M) {
  const GroupItem& it = group_item(g);
  lm_body<FMT, RB, MT>(it.x, it.w, it.scales, it.zeros, it.y, M, it.N, it.K, blockIdx.x - it.first_block, it.WK);
}

// ---------------------------------------------------------------- dequant
// One thread per unit: decode exactly, multiply by the scale in fp32 (exact), round once.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros, uint16_t* __restrict__ out,
                                                      int N, int K) {
  const int U = K >> 5;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)N * U) return;
  const int n = (int)(gid / U), u = (int)(gid % U);
  Raw<wfmt(FMT)> raw;
  load_unit<FMT>(w, n, u, U, raw);
  h2 zc1 = {}, zc2 = {};
  float s = 1.0f;
  if constexpr (group_meta(FMT)) {
    group_consts<FMT>(zeros[gid], zc1, zc2);
    s = f16_to_f32(scales[gid]);
  } else if constexpr (row_scaled<FMT>()) {
    s = f16_to_f32(scales[n]) * code_scale<FMT>();
  }
  h2 wv[16];
  decode<FMT>(raw, zc1, zc2, wv);
  uint32_t o[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    if constexpr (wfmt(FMT) == WQ_FMT_F16) {
      o[p] = as_u32(wv[p]);   // F16 and BF16 weights: a copy
    } else if constexpr (bf16_act(FMT)) {
      o[p] = as_u32(pack_bf16((float)wv[p][0] * s, (float)wv[p][1] * s));
    } else {
      const _Float16 a = (_Float16)((float)wv[p][0] * s), b = (_Float16)((float)wv[p][1] * s);
      o[p] = as_u32(h2{a, b});
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(out + (size_t)n * K + 32 * u);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

// ---------------------------------------------------------------- host-side planning
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool valid_fmt(int code) {
  switch (code) {
#define WQ_CASE(C) case C:
    WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
    return true;
    default: return false;
  }
}

// The planner below decides by weight layout (wfmt of a kernel code): the activation type
// changes the decode, not the bytes or the shape of the work.

struct GemvPlan {
  int B;      // rows per wave
  int WK;     // waves splitting K for one row block
  int R;      // row blocks per workgroup
  int grid;   // workgroups
};

// Waves splitting K: the fewest that give enough waves over the row blocks (W4, with the
// most decode work per byte, runs best at ~4 waves per CU, W8 at ~32 (Llama-7B linears at
// M = 1: 18.9 -> 18.6 us against ~16; ~4 and ~8 were slower), the others at ~16), then,
// among the splits with the same chunks per wave, the smallest (even work). Only powers
// of two, so that workgroups hold a multiple of 4 waves and spread evenly over a CU's
// four SIMDs (a 6-wave workgroup puts two waves on two SIMDs and one on the others).
// int3, whose decode takes the most instructions per byte, also splits until a wave has
// at most 2 chunks (Llama-7B linears at M = 1: 13.4 us against 14.3 us; W4 lost 3% so).
int gemv_waves_for(int fmt, int64_t N, int64_t K, int B) {
  const int64_t L = fmt == WQ_FMT_W8 ? 16 : fmt == WQ_FMT_F16 ? 8 : 32;
  const int64_t C = (K / L + 63) / 64, blocks = (N + B - 1) / B;
  const int64_t target = fmt == WQ_FMT_W4G32 || fmt == WQ_FMT_W4E2M1 || fmt == WQ_FMT_W3G32 ? 1024
                         : fmt == WQ_FMT_W8 ? 8192 : 4096;
  static const int cand[] = {1, 2, 4};
  int WK = 1;
  for (int w : cand) {
    if (w > C) break;
    WK = w;
    if (blocks * w >= target) break;
  }
  if (fmt == WQ_FMT_W3G32)
    while (WK < 4 && 2 * WK <= C && (C + WK - 1) / WK > 2) WK *= 2;
  const int64_t per = (C + WK - 1) / WK;
  for (int w : cand)
    if (w <= WK && (C + w - 1) / w == per) { WK = w; break; }
  return WK;
}

// Rows per wave: 4, halved while the launch would have fewer than 1024 waves. F16 rows of
// 10240 or more outputs take one row per wave (the weight stream needs more waves in flight
// when nothing is decoded).
int gemv_rows_per_wave(int fmt, int64_t N, int64_t K) {
  if (fmt == WQ_FMT_F16 && N >= 10240) return 1;
  int B = 4;
  while (B > 1 && ((N + B - 1) / B) * gemv_waves_for(fmt, N, K, B) < 1024) B >>= 1;
  return B;
}

GemvPlan plan_gemv(int fmt, int64_t N, int64_t K) {
  const int B = gemv_rows_per_wave(fmt, N, K), WK = gemv_waves_for(fmt, N, K, B);
  const int R = GEMV_WAVES / WK;
  const int64_t blocks = (N + B - 1) / B;
  return {B, WK, R, static_cast<int>((blocks + R - 1) / R)};
}

struct MfmaPlan {
  int RB;     // 16-row blocks per wave
  int WK;     // waves per workgroup, splitting K
  int grid;   // workgroups
};

// The matrix cores serve M >= 5, and M = 4 for N >= 2048 (W6) / 4096 (W8) and larger W4,
// where they beat the VALU GEMV (which then spends four dot products per weight pair):
// lm_kernel for W6 and for W4 with K a multiple of 256 (see use_lm), mfma_kernel for the rest.
bool use_mfma(int fmt, int64_t M, int64_t N) {
  if (M > GEMV_MAX_M) return true;
  return M == GEMV_MAX_M && ((fmt == WQ_FMT_W6E3M2 && N >= 2048) || (fmt == WQ_FMT_W8 && N >= 4096));
}

// RB: as many row blocks per wave as keeps >= 256 row groups (W4 and F16, whose decode
// is heavier per byte, take one or two). WK: doubled up to 8 until ~2048 waves.
int mfma_rows(int fmt, int64_t N) {
  if (fmt == WQ_FMT_W6E3M2 || fmt == WQ_FMT_W8) return N >= 16384 ? 4 : N >= 8192 ? 2 : 1;
  return fmt == WQ_FMT_F16 && N >= 8192 ? 2 : 1;
}

int mfma_waves_for(int64_t N, int64_t K, int RB) {
  const int64_t T = (K / 32 + 3) / 4;
  const int64_t groups = (N + 16 * RB - 1) / (16 * RB);
  int WK = 1;
  while (WK < MFMA_MAX_WAVES && WK < T && groups * WK < 2048) WK *= 2;
  return WK;
}

MfmaPlan plan_mfma(int fmt, int64_t N, int64_t K) {
  const int RB = mfma_rows(fmt, N);
  return {RB, mfma_waves_for(N, K, RB), static_cast<int>((N + 16 * RB - 1) / (16 * RB))};
}

struct LmPlan {
  int RB;     // 16-row blocks per wave
  int WK;     // waves of a row group splitting K (1, 2 or 4)
  int grid;   // workgroups
};

// The LDS-staged kernel serves W6 (both layouts: fmt is the planning layout, pfmt) wherever the
// matrix cores run for it, and W4, W3, FP4 and FP5 from M = 5 on and at M = 4 from N*K = 2^24 on,
// where it beats the VALU GEMV (W4 and W3 only when K is a multiple of 256, so that a lane's 8
// groups of metadata are one aligned 16-byte load).
// The LDS-staged kernel (code: a format code, with or without WQ_ACT_BF16): every M above
// GEMV_MAX_M (W6 also at M = 4 from N = 2048), and on large matrices (N*K >= 2^24) from 3 rows of
// x, 2 for FP4 and FP5: the GEMV's work grows with every row of x, this kernel's hardly (Llama-7B
// linears at M = 3: W4 22.2 -> 20.6 us, W6 30.1 -> 24.9, FP4 19.6 -> 15.8, int3 22.4 -> 19.9, FP5
// 26.4 -> 20.4; at M = 2 FP4 17.7 -> 15.2, while W4, int3 and W6 stay faster on the GEMV there).
// With bfloat16 x only W6 moves to 3 rows (Llama-70B linears 102.4 -> 85.3 us); W4, which scales
// every weight in fp32 there, stays on the GEMV up to 3 rows (22.2 us against 28.1).
bool use_lm(int code, int64_t M, int64_t N, int64_t K) {
  const int fmt = pfmt(code);
  if (group_meta(fmt) && K % 256) return false;
  if (!group_meta(fmt) && fmt != WQ_FMT_W4E2M1 && fmt != WQ_FMT_W5E2M2 && fmt != WQ_FMT_W6E3M2) return false;
  if (use_mfma(fmt, M, N)) return true;   // W6 takes no other matrix-core kernel
  const int64_t from = bf16_act(code) ? (fmt == WQ_FMT_W6E3M2 ? 3 : 4)
                                      : (fmt == WQ_FMT_W4E2M1 || fmt == WQ_FMT_W5E2M2 ? 2 : 3);
  return M >= from && N * K >= (int64_t(1) << 24);
}

// Two row blocks per wave from 8192 rows. WK doubled until ~1024 waves for W6 (one wave per
// SIMD at two row blocks) and ~2048 for W4 and FP4 (two waves per SIMD fit): on the Llama-70B
// gate/up pair at M = 8, W4 ran 88.5 us at 1024 and 83.5 us at 2048, W6 gained nothing.
int lm_rows(int64_t N) { return N >= 8192 ? 2 : 1; }

int lm_waves_for(int fmt, int64_t N, int64_t K, int RB) {
  const int64_t H = (K / 32 + 31) / 32;
  const int64_t groups = (N + 16 * RB - 1) / (16 * RB);
  const int64_t target = fmt == WQ_FMT_W6E3M2 ? 1024 : 2048;
  int WK = 1;
  while (WK < LM_WAVES && WK < H && groups * WK < target) WK *= 2;
  return WK;
}

LmPlan plan_lm(int fmt, int64_t N, int64_t K) {
  const int RB = lm_rows(N), WK = lm_waves_for(fmt, N, K, RB);
  const int64_t groups = (N + 16 * RB - 1) / (16 * RB);
  const int R = LM_WAVES / WK;
  return {RB, WK, static_cast<int>((groups + R - 1) / R)};
}

// 16-row tiles of x one LDS-staged launch takes (1, 2 or 4)
int lm_tiles(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

// Rows of x per launch: 64 where the LDS-staged kernel serves the shape (W6, FP4; W4 with K
// a multiple of 256), else 16. The kernels address x with 32-bit lane offsets (row * 2K + 64 u),
// which hold 64 rows only while K <= 2^25; longer rows take 16-row slabs.
int64_t slab_rows(int fmt, int64_t K) {
  const bool lm = fmt == WQ_FMT_W6E3M2 || fmt == WQ_FMT_W4E2M1 || fmt == WQ_FMT_W5E2M2 ||
                  (group_meta(fmt) && K % 256 == 0);
  return lm && K <= (int64_t(1) << 25) ? 16 * LM_MAX_MT : MFMA_M;
}

template <int FMT, int M>
hipError_t launch_gemv_m(const GemvPlan& p, hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc,
                         const uint16_t* z, uint16_t* y, int N, int K) {
  const dim3 grid(p.grid), block(64 * p.WK * p.R);
  switch (p.B) {
    case 4: return launch(gemv_kernel<FMT, M, 4>, grid, block, 0, s, x, w, sc, z, y, N, K, p.WK);
    case 2: return launch(gemv_kernel<FMT, M, 2>, grid, block, 0, s, x, w, sc, z, y, N, K, p.WK);
    default: return launch(gemv_kernel<FMT, M, 1>, grid, block, 0, s, x, w, sc, z, y, N, K, p.WK);
  }
}

// The LDS-staged kernel for (RB, MT) as template arguments: one launch, or (GemvGroup) a
// grouped one.
template <int FMT, int RB, int MT>
hipError_t lm_launch(dim3 grid, size_t shm, hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc,
                     const uint16_t* z, uint16_t* y, int M, int N, int K, int WK, const GemvGroup* g) {
  if (g) return launch(lm_grouped_kernel<FMT, RB, MT>, grid, dim3(64 * LM_WAVES), shm, s, *g, M);
  return launch(lm_kernel<FMT, RB, MT>, grid, dim3(64 * LM_WAVES), shm, s, x, w, sc, z, y, M, N, K, WK);
}

template <int FMT>
hipError_t launch_lm(int RB, int M, dim3 grid, hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc,
                     const uint16_t* z, uint16_t* y, int N, int K, int WK, const GemvGroup* g) {
  if constexpr (group_meta(FMT) || w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2) {
    const size_t shm = (size_t)LM_WAVES * RB * lm_block<FMT>();
    const int MT = lm_tiles(M);
    if (RB == 2) {
      if (MT == 1) return lm_launch<FMT, 2, 1>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
      if (MT == 2) return lm_launch<FMT, 2, 2>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
      return lm_launch<FMT, 2, 4>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
    }
    if (MT == 1) return lm_launch<FMT, 1, 1>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
    if (MT == 2) return lm_launch<FMT, 1, 2>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
    return lm_launch<FMT, 1, 4>(grid, shm, s, x, w, sc, z, y, M, N, K, WK, g);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_linear_fmt(hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc, const uint16_t* z,
                             uint16_t* y, int M, int N, int K) {
  if (use_lm(FMT, M, N, K)) {
    const LmPlan p = plan_lm(pfmt(FMT), N, K);
    return launch_lm<FMT>(p.RB, M, dim3(p.grid), s, x, w, sc, z, y, N, K, p.WK, nullptr);
  }
  if (!use_mfma(pfmt(FMT), M, N)) {
    const GemvPlan p = plan_gemv(pfmt(FMT), N, K);
    switch (M) {
      case 1: return launch_gemv_m<FMT, 1>(p, s, x, w, sc, z, y, N, K);
      case 2: return launch_gemv_m<FMT, 2>(p, s, x, w, sc, z, y, N, K);
      case 3: return launch_gemv_m<FMT, 3>(p, s, x, w, sc, z, y, N, K);
      default: return launch_gemv_m<FMT, 4>(p, s, x, w, sc, z, y, N, K);
    }
  }
  if constexpr (w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2) {
    return hipErrorInvalidValue;   // W6, FP4 and FP5 on the matrix cores always take lm_kernel (use_lm)
  } else {
    const MfmaPlan p = plan_mfma(pfmt(FMT), N, K);
    const dim3 grid(p.grid), block(64 * p.WK);
    switch (p.RB) {
      case 4: return launch(mfma_kernel<FMT, 4>, grid, block, 0, s, x, w, sc, z, y, M, N, K, p.WK);
      case 2: return launch(mfma_kernel<FMT, 2>, grid, block, 0, s, x, w, sc, z, y, M, N, K, p.WK);
      default: return launch(mfma_kernel<FMT, 1>, grid, block, 0, s, x, w, sc, z, y, M, N, K, p.WK);
    }
  }
}

// wq_linear_silu: the decode kernels of wq_linear's plan for the [N, K] matrix of gate/up row
// pairs, with the pair epilogue; the GEMV takes at least 2 rows per wave (a row's sum does not
// depend on the rows per wave, only on the K split, which stays the plan's). Never the tiled
// prefill kernel: prefill-sized M runs as slabs of the decode kernels.
template <int FMT>
hipError_t launch_linear_silu_fmt(hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc,
                                  const uint16_t* z, uint16_t* act, int M, int N, int K) {
  if constexpr (bf16_act(FMT)) {
    return hipErrorInvalidValue;   // fp16 activations only (the entry point rejects the flag)
  } else {
    const int pf = pfmt(FMT);
    if (use_lm(pf, M, N, K)) {
      if constexpr (group_meta(FMT) || w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2) {
        const LmPlan p = plan_lm(pf, N, K);
        const size_t shm = (size_t)LM_WAVES * p.RB * lm_block<FMT>();
        const dim3 grid(p.grid), block(64 * LM_WAVES);
        const int MT = lm_tiles(M);
        if (p.RB == 2) {
          if (MT == 1) return launch(lm_silu_kernel<FMT, 2, 1>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
          if (MT == 2) return launch(lm_silu_kernel<FMT, 2, 2>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
          return launch(lm_silu_kernel<FMT, 2, 4>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
        }
        if (MT == 1) return launch(lm_silu_kernel<FMT, 1, 1>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
        if (MT == 2) return launch(lm_silu_kernel<FMT, 1, 2>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
        return launch(lm_silu_kernel<FMT, 1, 4>, grid, block, shm, s, x, w, sc, z, act, M, N, K, p.WK);
      }
      return hipErrorInvalidValue;
    }
    if (!use_mfma(pf, M, N)) {
      const GemvPlan p = plan_gemv(pf, N, K);
      const int B = p.B < 2 ? 2 : p.B;
      const int64_t blocks = ((int64_t)N + B - 1) / B;
      const dim3 grid((unsigned)((blocks + p.R - 1) / p.R)), block(64 * p.WK * p.R);
      auto go = [&](auto kb2, auto kb4) {
        return B == 4 ? launch(kb4, grid, block, 0, s, x, w, sc, z, act, N, K, p.WK)
                      : launch(kb2, grid, block, 0, s, x, w, sc, z, act, N, K, p.WK);
      };
      switch (M) {
        case 1: return go(gemv_silu_kernel<FMT, 1, 2>, gemv_silu_kernel<FMT, 1, 4>);
        case 2: return go(gemv_silu_kernel<FMT, 2, 2>, gemv_silu_kernel<FMT, 2, 4>);
        case 3: return go(gemv_silu_kernel<FMT, 3, 2>, gemv_silu_kernel<FMT, 3, 4>);
        default: return go(gemv_silu_kernel<FMT, 4, 2>, gemv_silu_kernel<FMT, 4, 4>);
      }
    }
    if constexpr (w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2) {
      return hipErrorInvalidValue;   // these take lm_kernel wherever the matrix cores run (use_lm)
    } else {
      const MfmaPlan p = plan_mfma(pf, N, K);
      const dim3 grid(p.grid), block(64 * p.WK);
      switch (p.RB) {
        case 4: return launch(mfma_silu_kernel<FMT, 4>, grid, block, 0, s, x, w, sc, z, act, M, N, K, p.WK);
        case 2: return launch(mfma_silu_kernel<FMT, 2>, grid, block, 0, s, x, w, sc, z, act, M, N, K, p.WK);
        default: return launch(mfma_silu_kernel<FMT, 1>, grid, block, 0, s, x, w, sc, z, act, M, N, K, p.WK);
      }
    }
  }
}

template <int FMT, int M>
hipError_t launch_grouped_m(const GemvGroup& g, int B, int block_waves, int grid, hipStream_t s) {
  switch (B) {
    case 4: return launch(gemv_grouped_kernel<FMT, M, 4>, dim3(grid), dim3(64 * block_waves), 0, s, g);
    case 2: return launch(gemv_grouped_kernel<FMT, M, 2>, dim3(grid), dim3(64 * block_waves), 0, s, g);
    default: return launch(gemv_grouped_kernel<FMT, M, 1>, dim3(grid), dim3(64 * block_waves), 0, s, g);
  }
}

template <int FMT>
hipError_t launch_grouped_fmt(const GemvGroup& g, int M, int B, int block_waves, int grid, hipStream_t s) {
  switch (M) {
    case 1: return launch_grouped_m<FMT, 1>(g, B, block_waves, grid, s);
    case 2: return launch_grouped_m<FMT, 2>(g, B, block_waves, grid, s);
    case 3: return launch_grouped_m<FMT, 3>(g, B, block_waves, grid, s);
    default: return launch_grouped_m<FMT, 4>(g, B, block_waves, grid, s);
  }
}

// Launch order of a grouped call: the items with the longest rows (most chunks per wave)
// first, so that the waves that finish last are the short ones. Ties keep the caller's order.
void grouped_order(const wq_linear_item* items, int count, int (&order)[MAX_GROUP]) {
  for (int i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order, order + count, [&](int a, int b) { return items[a].K > items[b].K; });
}

// Which kernel family runs a linear of M <= 16 rows, and which runs a grouped call: the
// largest item's (by N*K), except that W4 on the LDS path needs every K a multiple of 256
// and otherwise takes the fragment-load kernel. Every family computes any shape correctly.
enum Family { FAM_GEMV, FAM_LM, FAM_MFMA };

Family family_of(int code, int64_t M, int64_t N, int64_t K) {
  if (use_lm(code, M, N, K)) return FAM_LM;
  return use_mfma(pfmt(code), M, N) ? FAM_MFMA : FAM_GEMV;
}

int largest_item(const int64_t* N, const int64_t* K, int count) {
  int big = 0;
  for (int i = 1; i < count; ++i)
    if (N[i] * K[i] > N[big] * K[big]) big = i;
  return big;
}

Family group_family(int code, int64_t M, const int64_t* N, const int64_t* K, int count) {
  const int big = largest_item(N, K, count);
  const int fmt = pfmt(code);
  Family f = family_of(code, M, N[big], K[big]);
  if (f == FAM_LM && group_meta(fmt))
    for (int i = 0; i < count; ++i)
      if (K[i] % 256) f = FAM_MFMA;
  return f;
}

// rows per wave (GEMV) or 16-row blocks per wave (matrix cores) of a grouped launch. The
// LDS-staged kernel takes two row blocks if any item has the rows for them: picking the largest
// item's made equal-size items (11008x4096 and 4096x11008) decide by their order, and one row
// block cost up to a third (the Llama-70B TP8 shard group at M = 16: 43 us against 33 us).
int group_rows(Family f, int fmt, const int64_t* N, const int64_t* K, int count) {
  if (f == FAM_LM) {
    int rb = 1;
    for (int i = 0; i < count; ++i) rb = std::max(rb, lm_rows(N[i]));
    return rb;
  }
  const int big = largest_item(N, K, count);
  return f == FAM_GEMV ? gemv_rows_per_wave(fmt, N[big], K[big]) : mfma_rows(fmt, N[big]);
}

// rows of x one grouped launch of this family takes for every item
int64_t group_launch_rows(Family f, int fmt, const int64_t* K, int count) {
  if (f != FAM_LM) return MFMA_M;
  int64_t rows = 16 * LM_MAX_MT;
  for (int i = 0; i < count; ++i) rows = std::min(rows, slab_rows(fmt, K[i]));
  return rows;
}

int check_linear_args(const uint16_t* x, const void* w, const uint16_t* sc, const uint16_t* z, const uint16_t* y,
                      int64_t M, int64_t N, int64_t K, int fmt) {
  if (!valid_fmt(fmt)) return WQ_ERR_FMT;
  if (!x || !w || !y || M < 0 || N < 0 || K < 0) return WQ_ERR_ARG;
  if (wfmt(fmt) != WQ_FMT_F16 && !sc) return WQ_ERR_ARG;
  if (group_meta(fmt) && !z) return WQ_ERR_ARG;
  if (M < 1 || N < 1 || K < 32 || K % 32) return WQ_ERR_SHAPE;
  if (N > INT32_MAX / 2 || K > (int64_t(1) << 26) || (N * (K / 32)) > INT32_MAX) return WQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (sc && !aligned16(sc)) || (z && !aligned16(z))) return WQ_ERR_ALIGN;
  return WQ_OK;
}

template <int FMT>
hipError_t launch_grouped_mc(Family f, const GemvGroup& g, int M, int RB, int block_waves, int grid, hipStream_t s) {
  if (f == FAM_LM) return launch_lm<FMT>(RB, M, dim3(grid), s, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, &g);
  if constexpr (w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2) {
    return hipErrorInvalidValue;   // W6, FP4 and FP5 groups on the matrix cores are always FAM_LM
  } else {
    switch (RB) {
      case 4: return launch(mfma_grouped_kernel<FMT, 4>, dim3(grid), dim3(64 * block_waves), 0, s, g, M);
      case 2: return launch(mfma_grouped_kernel<FMT, 2>, dim3(grid), dim3(64 * block_waves), 0, s, g, M);
      default: return launch(mfma_grouped_kernel<FMT, 1>, dim3(grid), dim3(64 * block_waves), 0, s, g, M);
    }
  }
}

thread_local int last_device_error = hipSuccess;

}  // namespace

namespace wq {
int device_status(int hip_error) {
  if (hip_error == hipSuccess) return WQ_OK;
  last_device_error = hip_error;
  return WQ_ERR_DEVICE;
}
}  // namespace wq

extern "C" {

const char* wq_last_device_error(void) {
  return last_device_error == hipSuccess ? "none" : hipGetErrorName(static_cast<hipError_t>(last_device_error));
}

int wq_linear(const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros, uint16_t* y,
              int64_t M, int64_t N, int64_t K, int fmt, void* stream) {
  const int st = check_linear_args(x, packed_w, scales, zeros, y, M, N, K, fmt);
  if (st != WQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* w = static_cast<const uint8_t*>(packed_w);
  if (wq::pf_takes(fmt, M, &N, &K, 1))   // prefill-sized M: one tiled launch for all rows
    return wq::pf_launch(fmt, x, w, scales, zeros, y, M, N, K, stream);
  const int64_t slab = slab_rows(pfmt(fmt), K);
  for (int64_t m0 = 0; m0 < M; m0 += slab) {
    const int mm = static_cast<int>(M - m0 < slab ? M - m0 : slab);
    const uint16_t* xs = x + m0 * K;
    uint16_t* ys = y + m0 * N;
    hipError_t e = hipSuccess;
    switch (fmt) {
#define WQ_CASE(C) case C: e = launch_linear_fmt<C>(s, xs, w, scales, zeros, ys, mm, (int)N, (int)K); break;
      WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
      default: return WQ_ERR_FMT;
    }
    if (e != hipSuccess) return wq::device_status(e);
  }
  return WQ_OK;
}

int wq_linear_silu(const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros,
                   uint16_t* act, int64_t M, int64_t F, int64_t K, int fmt, void* stream) {
  if (!valid_fmt(fmt) || bf16_act(fmt)) return WQ_ERR_FMT;
  if (F < 0) return WQ_ERR_ARG;
  if (F < 1 || F > INT32_MAX / 4) return WQ_ERR_SHAPE;
  const int64_t N = 2 * F;
  const int st = check_linear_args(x, packed_w, scales, zeros, act, M, N, K, fmt);
  if (st != WQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* w = static_cast<const uint8_t*>(packed_w);
  const int64_t slab = slab_rows(pfmt(fmt), K);
  for (int64_t m0 = 0; m0 < M; m0 += slab) {
    const int mm = static_cast<int>(M - m0 < slab ? M - m0 : slab);
    const uint16_t* xs = x + m0 * K;
    uint16_t* as = act + m0 * F;
    hipError_t e = hipSuccess;
    switch (fmt) {
#define WQ_CASE(C) case C: e = launch_linear_silu_fmt<C>(s, xs, w, scales, zeros, as, mm, (int)N, (int)K); break;
      WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
      default: return WQ_ERR_FMT;
    }
    if (e != hipSuccess) return wq::device_status(e);
  }
  return WQ_OK;
}

int wq_dequant(int fmt, const void* packed, const uint16_t* scales, const uint16_t* zeros, uint16_t* w_out, int64_t N,
               int64_t K, void* stream) {
  if (!valid_fmt(fmt)) return WQ_ERR_FMT;
  if (!packed || !w_out || N < 0 || K < 0) return WQ_ERR_ARG;
  if (wfmt(fmt) != WQ_FMT_F16 && !scales) return WQ_ERR_ARG;
  if (group_meta(fmt) && !zeros) return WQ_ERR_ARG;
  if (N < 1 || K < 32 || K % 32) return WQ_ERR_SHAPE;
  if (N * (K / 32) > INT32_MAX) return WQ_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(w_out) || (scales && !aligned16(scales)) || (zeros && !aligned16(zeros)))
    return WQ_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* w = static_cast<const uint8_t*>(packed);
  const int64_t units = N * (K / 32);
  const dim3 grid(static_cast<unsigned>((units + 255) / 256)), block(256);
  hipError_t e = hipSuccess;
  switch (fmt) {
#define WQ_CASE(C) \
  case C: e = launch(dequant_kernel<C>, grid, block, 0, s, w, scales, zeros, w_out, (int)N, (int)K); break;
    WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
    default: return WQ_ERR_FMT;
  }
  return wq::device_status(e);
}

int wq_linear_grouped(const wq_linear_item* items, int count, int64_t M, int fmt, void* stream) {
  if (!valid_fmt(fmt)) return WQ_ERR_FMT;
  if (!items || count < 0 || count > MAX_GROUP) return WQ_ERR_ARG;
  if (count == 0) return WQ_OK;
  for (int i = 0; i < count; ++i) {
    const wq_linear_item& it = items[i];
    const int st = check_linear_args(it.x, it.packed_w, it.scales, it.zeros, it.y, M, it.N, it.K, fmt);
    if (st != WQ_OK) return st;
  }
  int64_t Ns[MAX_GROUP], Ks[MAX_GROUP];
  for (int i = 0; i < count; ++i) { Ns[i] = items[i].N; Ks[i] = items[i].K; }
  // one family and one rows-per-wave (B or RB) for the whole launch: the largest item's (the
  // small items alone would pick fewer rows per wave to get enough waves, which the launch
  // has anyway); each item keeps the K split its own plan gives for that B / RB
  if (count > 1 && wq::pf_takes(fmt, M, Ns, Ks, count))   // prefill-sized M: all items' tiles in one launch
    return wq::pf_launch_grouped(fmt, items, count, M, stream);
  const int pf = pfmt(fmt);
  const Family fam = group_family(fmt, M, Ns, Ks, count);
  if (M > group_launch_rows(fam, pf, Ks, count)) {   // several slabs: one wq_linear per item
    for (int i = 0; i < count; ++i) {
      const wq_linear_item& it = items[i];
      const int st = wq_linear(it.x, it.packed_w, it.scales, it.zeros, it.y, M, it.N, it.K, fmt, stream);
      if (st != WQ_OK) return st;
    }
    return WQ_OK;
  }
  const int B = group_rows(fam, pf, Ns, Ks, count);
  int order[MAX_GROUP];
  grouped_order(items, count, order);
  GemvGroup g = {};
  g.count = count;
  int WKs[MAX_GROUP];
  int block_waves = fam == FAM_GEMV ? GEMV_WAVES : fam == FAM_LM ? LM_WAVES : 1;
  for (int i = 0; i < count; ++i) {
    const int64_t n = items[order[i]].N, k = items[order[i]].K;
    WKs[i] = fam == FAM_GEMV ? gemv_waves_for(pf, n, k, B) : fam == FAM_LM ? lm_waves_for(pf, n, k, B) : mfma_waves_for(n, k, B);
    if (fam == FAM_MFMA) block_waves = std::max(block_waves, WKs[i]);   // powers of two up to MFMA_MAX_WAVES
  }
  const int rows_per_block = fam == FAM_GEMV ? B : 16 * B;
  int grid = 0;
  for (int i = 0; i < MAX_GROUP; ++i) g.first_block[i] = INT_MAX;
  for (int i = 0; i < count; ++i) {
    const wq_linear_item& it = items[order[i]];
    const int R = block_waves / WKs[i];
    GroupItem& gi = g.item[i];
    g.first_block[i] = gi.first_block = grid;
    gi.x = it.x;
    gi.w = static_cast<const uint8_t*>(it.packed_w);
    gi.scales = it.scales;
    gi.zeros = it.zeros;
    gi.y = it.y;
    gi.N = static_cast<int>(it.N);
    gi.K = static_cast<int>(it.K);
    gi.WK = WKs[i];
    grid += static_cast<int>(((it.N + rows_per_block - 1) / rows_per_block + R - 1) / R);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fam == FAM_GEMV) {
    switch (fmt) {
#define WQ_CASE(C) case C: e = launch_grouped_fmt<C>(g, (int)M, B, block_waves, grid, s); break;
      WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
      default: return WQ_ERR_FMT;
    }
  } else {
    switch (fmt) {
#define WQ_CASE(C) case C: e = launch_grouped_mc<C>(fam, g, (int)M, B, block_waves, grid, s); break;
      WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
      default: return WQ_ERR_FMT;
    }
  }
  return wq::device_status(e);
}

const char* wq_linear_kernel_name(int fmt, int64_t M, int64_t N, int64_t K) {
  static thread_local char buf[96];
  if (!valid_fmt(fmt) || M < 1 || N < 1 || K < 32 || K % 32) return "";
  const int pf = pfmt(fmt);
  if (wq::pf_takes(fmt, M, &N, &K, 1)) {
    snprintf(buf, sizeof(buf), "pf_kernel<%d>", fmt);
    return buf;
  }
  const int64_t mm = M < slab_rows(pf, K) ? M : slab_rows(pf, K);   // the first launch's rows
  if (use_lm(fmt, mm, N, K)) {
    snprintf(buf, sizeof(buf), "lm_kernel<%d, %d, %d>", fmt, plan_lm(pf, N, K).RB, lm_tiles(mm));
  } else if (!use_mfma(pf, mm, N)) {
    const GemvPlan p = plan_gemv(pf, N, K);
    snprintf(buf, sizeof(buf), "gemv_kernel<%d, %d, %d>", fmt, static_cast<int>(mm), p.B);
  } else {
    snprintf(buf, sizeof(buf), "mfma_kernel<%d, %d>", fmt, plan_mfma(pf, N, K).RB);
  }
  return buf;
}

const char* wq_linear_grouped_kernel_name(int fmt, int64_t M, const int64_t* N, const int64_t* K, int count) {
  static thread_local char buf[96];
  if (!valid_fmt(fmt) || M < 1 || !N || !K || count < 1 || count > MAX_GROUP) return "";
  for (int i = 0; i < count; ++i)
    if (N[i] < 1 || K[i] < 32 || K[i] % 32) return "";
  if (count > 1 && wq::pf_takes(fmt, M, N, K, count)) {
    snprintf(buf, sizeof(buf), "pf_grouped_kernel<%d>", fmt);
    return buf;
  }
  const int big = largest_item(N, K, count);
  const int pf = pfmt(fmt);
  const Family fam = group_family(fmt, M, N, K, count);
  if (M > group_launch_rows(fam, pf, K, count))
    return wq_linear_kernel_name(fmt, M, N[big], K[big]);   // separate launches: the largest item's
  const int B = group_rows(fam, pf, N, K, count);
  if (fam == FAM_GEMV) snprintf(buf, sizeof(buf), "gemv_grouped_kernel<%d, %d, %d>", fmt, static_cast<int>(M), B);
  else if (fam == FAM_LM) snprintf(buf, sizeof(buf), "lm_grouped_kernel<%d, %d, %d>", fmt, B, lm_tiles(M));
  else snprintf(buf, sizeof(buf), "mfma_grouped_kernel<%d, %d>", fmt, B);
  return buf;
}

}  // extern "C"
