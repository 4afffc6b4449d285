// Device helpers shared by the kernel translation units of libwq (gfx950): vector types,
// the format code, the exact decoders of every weight format, the fragment and output
// conversions of both activation types, and the wave reduction.
#ifndef WQ_DEVICE_H_
#define WQ_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "wq_internal.h"

namespace {

// Launch kernel k and return the launch's own status. hipLaunchKernel reports what this launch
// met; the thread's last-error slot, which may hold an error another library left pending, is
// neither read nor cleared. The arguments are converted to the kernel's parameter types first.
template <typename... P, size_t... I>
hipError_t launch_tuple(void (*k)(P...), dim3 grid, dim3 block, size_t shm, hipStream_t s, std::tuple<P...>& t,
                        std::index_sequence<I...>) {
  void* args[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, shm, s);
}
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t shm, hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(a...);
  return launch_tuple(k, grid, block, shm, s, t, std::index_sequence_for<P...>{});
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h32 __attribute__((ext_vector_type(32)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b32 __attribute__((ext_vector_type(32)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x6 __attribute__((ext_vector_type(6)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));


// A constant kept in a VGPR. gfx950 VALU ops take at most one SGPR or literal and VOP3
// ops take no literal, so masks used by v_and_or_b32 / v_perm_b32 must sit in VGPRs.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
  asm volatile("" : "+v"(c));
  return c;
}

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// A kernel's format code: the weight format in the low byte, WQ_ACT_BF16 for bfloat16
// activations. Registers hold 16-bit pairs as h2 whatever their type; only the dot products,
// the matrix instructions and the output conversion look at the type. wfmt() is the weight
// layout (BF16 weights are laid out and loaded as F16 ones).
constexpr int wfmt(int c) { return (c & 0xFF) == WQ_FMT_BF16 ? WQ_FMT_F16 : (c & 0xFF); }
constexpr bool bf16_act(int c) { return (c & WQ_ACT_BF16) != 0; }
// The two FP6 layouts share W6's geometry (a 16-byte and an 8-byte slice per unit, in planes);
// int4 and int3 carry a scale and a zero point per group of 32 K.
constexpr bool w6_geom(int c) { return wfmt(c) == WQ_FMT_W6E3M2 || wfmt(c) == WQ_FMT_W6E3M2_P24; }
constexpr bool group_meta(int c) { return wfmt(c) == WQ_FMT_W4G32 || wfmt(c) == WQ_FMT_W3G32; }
// The layout the launch planner sizes work by: the 2+4 FP6 layout moves the same bytes in the
// same slices as W6 and is planned as W6.
constexpr int pfmt(int c) { return w6_geom(c) ? WQ_FMT_W6E3M2 : wfmt(c); }

__device__ __forceinline__ float dot2_bf16(h2 a, h2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
}
// Pairs 4k .. 4k+3 of a decoded unit as one 8-element MFMA fragment (32-bit moves only).
__device__ __forceinline__ h8 frag_of(const h2 (&wv)[16], int k) {
  return __builtin_bit_cast(h8, make_uint4(as_u32(wv[4 * k]), as_u32(wv[4 * k + 1]), as_u32(wv[4 * k + 2]),
                                           as_u32(wv[4 * k + 3])));
}

__device__ __forceinline__ h2 pack_bf16(float lo, float hi) {   // two values rounded to nearest even
  const b2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(h2, v);
}

template <int FMT>
__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {   // 16x16x32 product of the activation type
  if constexpr (bf16_act(FMT))
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int FMT>
__device__ __forceinline__ uint16_t out16(float v) {   // y: rounded once to the activation type
  if constexpr (bf16_act(FMT)) return __builtin_bit_cast(uint16_t, (__bf16)v);
  else return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// ---------------------------------------------------------------- raw units and loads
// A 32-code unit in registers. W6 keeps its two plane slices (16 + 8 bytes), which read in
// order are the unit's 192-bit little-endian stream.
template <int FMT> struct Raw;
template <> struct Raw<WQ_FMT_W8> { uint4 a, b; };
template <> struct Raw<WQ_FMT_W4G32> { uint4 a; };
template <> struct Raw<WQ_FMT_W6E3M2> { uint4 a; uint2 b; };
template <> struct Raw<WQ_FMT_W4E2M1> { uint4 a; };
template <> struct Raw<WQ_FMT_W5E2M2> { uint4 a; uint32_t b; };   // magnitude nibbles, sign word
template <> struct Raw<WQ_FMT_W3G32> { uint4 a; };                  // the 12 bytes in .x .y .z (.w unused)
template <> struct Raw<WQ_FMT_W6E3M2_P24> { uint4 a; uint2 b; };    // low nibbles; bit-4 word, sign word
template <> struct Raw<WQ_FMT_F16> { uint4 a, b, c, d; };

template <int FMT> constexpr int unit_bytes() {
  constexpr int f = wfmt(FMT);
  return f == WQ_FMT_W8 ? 32 : f == WQ_FMT_W4G32 || f == WQ_FMT_W4E2M1 ? 16 : f == WQ_FMT_W3G32 ? 12
       : w6_geom(f) ? 24 : f == WQ_FMT_W5E2M2 ? 20 : 64;
}

// Formats with one fp16 scale per output row, applied to the finished fp32 sum.
template <int FMT> constexpr bool row_scaled() {
  return wfmt(FMT) == WQ_FMT_W8 || w6_geom(FMT) || wfmt(FMT) == WQ_FMT_W4E2M1 || wfmt(FMT) == WQ_FMT_W5E2M2;
}

// The decoders hand FP5 values over as e2m2(code) * 2^-14 and the 2+4 FP6 values as
// e3m2(code) * 2^-12 (exact fp16 bit placements); the row scale that multiplies the finished
// sum carries the power of two (exact in fp32).
template <int FMT> constexpr float code_scale() {
  return wfmt(FMT) == WQ_FMT_W5E2M2 ? 16384.0f : wfmt(FMT) == WQ_FMT_W6E3M2_P24 ? 4096.0f : 1.0f;
}

// 12 bytes at a 4-byte aligned address, as one dwordx3 load (the type's alignment is lowered to
// 4 so that the load is never widened past the 12 bytes).
typedef unsigned int u32x3a __attribute__((ext_vector_type(3), aligned(4)));
__device__ __forceinline__ uint4 ld12(const uint8_t* p) {
  const u32x3a t = *reinterpret_cast<const u32x3a*>(p);
  return make_uint4(t[0], t[1], t[2], 0u);
}
__device__ __forceinline__ uint4 ld_nt12(const uint8_t* p) {
  const u32x3a t = __builtin_nontemporal_load(reinterpret_cast<const u32x3a*>(p));
  return make_uint4(t[0], t[1], t[2], 0u);
}

// Byte offsets, from the start of row n, of the two plane slices of W6 unit u (U units per row).
__device__ __forceinline__ void w6_homes(int u, int U, uint32_t& lo, uint32_t& hi) {
  const int c = u >> 6, j = u & 63, uc = min(64, U - 64 * c);
  lo = (uint32_t)(64 * c * 24 + 16 * j);
  hi = (uint32_t)(64 * c * 24 + 16 * uc + 8 * j);
}

// FP5: the same chunks of 64 units, 16 bytes of magnitude nibbles and then a 4-byte sign word per unit.
__device__ __forceinline__ void w5_homes(int u, int U, uint32_t& lo, uint32_t& hi) {
  const int c = u >> 6, j = u & 63, uc = min(64, U - 64 * c);
  lo = (uint32_t)(64 * c * 20 + 16 * j);
  hi = (uint32_t)(64 * c * 20 + 16 * uc + 4 * j);
}

// Unit u of row n (used by the MFMA and dequant kernels, where a lane owns a whole unit).
template <int FMT>
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ w, int n, int u, int U, Raw<wfmt(FMT)>& r) {
  constexpr int UB = unit_bytes<FMT>();
  const uint8_t* row = w + (size_t)n * U * UB;
  if constexpr (wfmt(FMT) == WQ_FMT_W8) {
    const uint4* q = reinterpret_cast<const uint4*>(row + (size_t)u * UB);
    r.a = q[0]; r.b = q[1];
  } else if constexpr (wfmt(FMT) == WQ_FMT_W4G32 || wfmt(FMT) == WQ_FMT_W4E2M1) {
    r.a = *reinterpret_cast<const uint4*>(row + (size_t)u * UB);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W3G32) {
    r.a = ld12(row + (size_t)u * UB);
  } else if constexpr (w6_geom(FMT)) {
    uint32_t lo, hi;
    w6_homes(u, U, lo, hi);
    r.a = *reinterpret_cast<const uint4*>(row + lo);
    r.b = *reinterpret_cast<const uint2*>(row + hi);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W5E2M2) {
    uint32_t lo, hi;
    w5_homes(u, U, lo, hi);
    r.a = *reinterpret_cast<const uint4*>(row + lo);
    r.b = *reinterpret_cast<const uint32_t*>(row + hi);
  } else {
    const uint4* q = reinterpret_cast<const uint4*>(row + (size_t)u * UB);
    r.a = q[0]; r.b = q[1]; r.c = q[2]; r.d = q[3];
  }
}

// ---------------------------------------------------------------- exact decode to fp16 pairs
// out[p] holds the values of codes 2p and 2p+1 of the unit:
//   W8: q      W4: q - z      W6: e3m2(code)      FP4: e2m1(code)      F16: the weights
// zc1 = -(1024 + z), zc2 = -(64 + z) as fp16 pairs (W4 only; exact small integers).
__device__ __forceinline__ void decode_w8_word(uint32_t d, h2& lo, h2& hi) {
  const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04010400u)) + bias;
  hi = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04030402u)) + bias;
}

__device__ __forceinline__ void decode_w4_word(uint32_t d, h2 zc1, h2 zc2, h2& o0, h2& o1, h2& o2, h2& o3) {
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t d8 = d >> 8;
  o0 = as_h2((d & 0x000F000Fu) | 0x64006400u) + zc1;                       // codes 0,1: 1024+q
  o1 = __builtin_elementwise_fma(as_h2((d & 0x00F000F0u) | 0x64006400u), sixteenth, zc2);   // 1024+16q
  o2 = as_h2((d8 & 0x000F000Fu) | 0x64006400u) + zc1;
  o3 = __builtin_elementwise_fma(as_h2((d8 & 0x00F000F0u) | 0x64006400u), sixteenth, zc2);
}

// FP5 e2m2: the pair of codes 2p, 2p+1 (p = 4d + t: nibbles t and t+4 of magnitude word d, sign
// bits p and 16+p of the sign word) as fp16 bits s.ee.mm at 15 and 11..8, i.e. e2m2(code) * 2^-14
// exactly (fp16's exponent bias 15 is e2m2's bias 1 + 14; the subnormal codes land on fp16
// subnormals). A shift and an AND for the magnitudes, a shift and an AND for the signs, an OR.
__device__ __forceinline__ void decode_fp5(const uint4& mag, uint32_t sgn, h2 (&out)[16]) {
  const uint32_t w[4] = {mag.x, mag.y, mag.z, mag.w};
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p = 4 * d + t;
      const uint32_t m = (t < 2 ? w[d] << (8 - 4 * t) : w[d] >> (4 * t - 8)) & 0x0F000F00u;
      out[p] = as_h2(m | ((sgn << (15 - p)) & 0x80008000u));
    }
}

// FP6 e3m2 in the 2+4 split layout: pair p = 4d + t takes its two low nibbles from word d as FP5
// does (to fp16 bits 11..8 and 27..24), bit 4 from bits p and 16+p of the bit-4 word (to fp16
// bits 12 and 28) and the signs from the sign word (to bits 15 and 31): fp16 bits s.eee.mm at
// 15 and 12..8, i.e. e3m2(code) * 2^-12 exactly (fp16's exponent bias 15 is e3m2's bias 3 + 12;
// the subnormal codes land on fp16 subnormals). Three shifts, an AND and two AND-ORs per pair,
// with the masks in VGPRs.
struct P24Masks { uint32_t nib, e2, sg; };
__device__ __forceinline__ P24Masks p24_masks() {
  return {in_vgpr(0x0F000F00u), in_vgpr(0x10001000u), in_vgpr(0x80008000u)};
}
__device__ __forceinline__ void decode_p24(const uint4& mag, const uint2& hi, const P24Masks& k, h2 (&out)[16]) {
  const uint32_t w[4] = {mag.x, mag.y, mag.z, mag.w};
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p = 4 * d + t;
      const uint32_t m = t < 2 ? w[d] << (8 - 4 * t) : w[d] >> (4 * t - 8);
      const uint32_t e = p <= 12 ? hi.x << (12 - p) : hi.x >> (p - 12);
      const uint32_t sg = (hi.y << (15 - p)) & k.sg;
      out[p] = as_h2((m & k.nib) | ((e & k.e2) | sg));
    }
}

// int3 (W3 layout): in each word, the pairs at offsets 0, 3 and 6 of both halves are placed in
// the mantissas of 1024.0 (step 1), 128.0 (step 1/8) and 16.0 (step 1/64), so the masked field
// reads 1024 + q, 128 + q or 16 + q; the word shifted right by 10 brings offsets 10 and 13 to 0
// and 3. The last pair is gathered from bits 9 and 25 of the three words. One AND-OR per pair
// (the last takes three), with the masks in VGPRs. w3_class(p) names the bias of pair p:
// 0 -> 1024, 1 -> 128, 2 -> 16.
constexpr int w3_class(int p) { return p == 15 ? 0 : (p % 5 == 2 ? 2 : (p % 5 == 1 || p % 5 == 4) ? 1 : 0); }
struct W3Masks { uint32_t f0, f1, f2, mag0, mag1, mag2, b0, b1, b2; };
__device__ __forceinline__ W3Masks w3_masks() {
  return {in_vgpr(0x00070007u), in_vgpr(0x00380038u), in_vgpr(0x01C001C0u), in_vgpr(0x64006400u),
          in_vgpr(0x58005800u), in_vgpr(0x4C004C00u), in_vgpr(0x00010001u), in_vgpr(0x00020002u),
          in_vgpr(0x00040004u)};
}
__device__ __forceinline__ void decode_w3_biased(const uint4& r, const W3Masks& k, h2 (&out)[16]) {
  const uint32_t w[3] = {r.x, r.y, r.z};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t d = w[i], e = d >> 10;
    out[5 * i] = as_h2((d & k.f0) | k.mag0);
    out[5 * i + 1] = as_h2((d & k.f1) | k.mag1);
    out[5 * i + 2] = as_h2((d & k.f2) | k.mag2);
    out[5 * i + 3] = as_h2((e & k.f0) | k.mag0);
    out[5 * i + 4] = as_h2((e & k.f1) | k.mag1);
  }
  out[15] = as_h2(((r.x >> 9) & k.b0) | (((r.y >> 8) & k.b1) | (((r.z >> 7) & k.b2) | k.mag0)));
}
// q - z exactly: the biased values plus zc[class] = -(1024 + z), -(128 + z), -(16 + z).
__device__ __forceinline__ void decode_w3_unit(const uint4& r, const h2 (&zc)[3], const W3Masks& k, h2 (&out)[16]) {
  decode_w3_biased(r, k, out);
#pragma unroll
  for (int p = 0; p < 16; ++p) out[p] += zc[w3_class(p)];
}
__device__ __forceinline__ void w3_consts(uint16_t zbits, h2 (&zc)[3]) {
  const _Float16 z = __builtin_bit_cast(_Float16, zbits);
  const _Float16 c0 = (_Float16)-1024.0f - z, c1 = (_Float16)-128.0f - z, c2 = (_Float16)-16.0f - z;   // exact
  zc[0] = h2{c0, c0};
  zc[1] = h2{c1, c1};
  zc[2] = h2{c2, c2};
}

// Byte b of d holds codes 2b (low nibble) and 2b+1 (high nibble); the convert takes the
// byte index as an immediate and returns them in that order.
__device__ __forceinline__ void decode_fp4_word(uint32_t d, h2& o0, h2& o1, h2& o2, h2& o3) {
  o0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
  o1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
  o2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
  o3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
}

template <int FMT>
__device__ __forceinline__ void decode(const Raw<wfmt(FMT)>& r, h2 zc1, h2 zc2, h2 (&out)[16]) {
  if constexpr (wfmt(FMT) == WQ_FMT_W8) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) decode_w8_word(w[i], out[2 * i], out[2 * i + 1]);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W4G32) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_w4_word(w[i], zc1, zc2, out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W6E3M2) {
    u32x6 v;
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w; v[4] = r.b.x; v[5] = r.b.y;
    const h32 h = __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(v, 1.0f);
#pragma unroll
    for (int p = 0; p < 16; ++p) { out[p][0] = h[2 * p]; out[p][1] = h[2 * p + 1]; }
  } else if constexpr (wfmt(FMT) == WQ_FMT_W4E2M1) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_fp4_word(w[i], out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W5E2M2) {
    decode_fp5(r.a, r.b, out);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W6E3M2_P24) {
    decode_p24(r.a, r.b, P24Masks{0x0F000F00u, 0x10001000u, 0x80008000u}, out);
  } else if constexpr (wfmt(FMT) == WQ_FMT_W3G32) {
    // zc1 = -(1024 + z), zc2 = -(128 + z) (w3_consts); -(16 + z) = zc2 + 112 exactly
    const h2 zc[3] = {zc1, zc2, zc2 + h2{(_Float16)112.0f, (_Float16)112.0f}};
    decode_w3_unit(r.a, zc, W3Masks{0x00070007u, 0x00380038u, 0x01C001C0u, 0x64006400u, 0x58005800u, 0x4C004C00u,
                                    0x00010001u, 0x00020002u, 0x00040004u}, out);
  } else {
    const uint32_t w[16] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w,
                            r.c.x, r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w};
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = as_h2(w[p]);
  }
}

// The zero-point constants decode<FMT> takes for a group's zero point z: W4 -(1024 + z) and
// -(64 + z), W3 -(1024 + z) and -(128 + z); zero for the other formats.
template <int FMT>
__device__ __forceinline__ void group_consts(uint16_t zbits, h2& zc1, h2& zc2) {
  if constexpr (wfmt(FMT) == WQ_FMT_W4G32 || wfmt(FMT) == WQ_FMT_W3G32) {
    const _Float16 z = __builtin_bit_cast(_Float16, zbits);
    const _Float16 c1 = (_Float16)-1024.0f - z;
    const _Float16 c2 = (wfmt(FMT) == WQ_FMT_W4G32 ? (_Float16)-64.0f : (_Float16)-128.0f) - z;   // exact integers
    zc1 = h2{c1, c1};
    zc2 = h2{c2, c2};
  } else {
    zc1 = h2{};
    zc2 = h2{};
  }
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// The feed-forward's gate: silu(g) * u = g / (1 + e^-g) * u for fp16 g and u, in float32, rounded
// once to fp16. One definition for the stand-alone kernel and the fused linear epilogue, so that
// both give the same bits.
__device__ __forceinline__ uint16_t silu_mul_f16(uint16_t g, uint16_t u) {
  const float gv = f16_to_f32(g), uv = f16_to_f32(u);
  return __builtin_bit_cast(uint16_t, (_Float16)(gv / (1.0f + expf(-gv)) * uv));
}

// The weights of a unit as bfloat16 pairs for bfloat16 activations (same pair order as
// decode): W8 q, W6 e3m2(code), FP4 e2m1(code), BF16 the weights, all exact, with the row
// scale applied after the sum; W4 (q - z) s rounded once to bfloat16, since its scale changes
// along K. For W4, the nibble placed at bit 16 of 128.0f gives (128 + q) in fp32, and one fma
// with s and c = -(128 + z) s gives (q - z) s exactly (every product is exact in fp32).
template <int FMT>
__device__ __forceinline__ void decode_bf16(const Raw<wfmt(FMT)>& r, uint16_t sbits, uint16_t zbits, h2 (&out)[16]) {
  constexpr int F = wfmt(FMT);
  if constexpr (F == WQ_FMT_W8) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      out[2 * i] = pack_bf16((float)(w[i] & 0xFFu) - 128.0f, (float)((w[i] >> 8) & 0xFFu) - 128.0f);
      out[2 * i + 1] = pack_bf16((float)((w[i] >> 16) & 0xFFu) - 128.0f, (float)(w[i] >> 24) - 128.0f);
    }
  } else if constexpr (F == WQ_FMT_W4G32) {
    const float s = f16_to_f32(sbits);
    const float c = -(128.0f + f16_to_f32(zbits)) * s;
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {   // codes 8i+2t (nibble t) and 8i+2t+1 (nibble t+4)
        const float lo = __builtin_bit_cast(float, ((w[i] << (16 - 4 * t)) & 0x000F0000u) | 0x43000000u);
        const float hi = __builtin_bit_cast(float, ((w[i] >> (4 * t)) & 0x000F0000u) | 0x43000000u);
        out[4 * i + t] = pack_bf16(__builtin_fmaf(lo, s, c), __builtin_fmaf(hi, s, c));
      }
    }
  } else if constexpr (F == WQ_FMT_W6E3M2) {
    u32x6 v;
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w; v[4] = r.b.x; v[5] = r.b.y;
    const u32x16 h = __builtin_bit_cast(u32x16, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(v, 1.0f));
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = as_h2(h[p]);
  } else if constexpr (F == WQ_FMT_W5E2M2) {
    h2 h[16];   // e2m2(code) * 2^-14 as fp16, then as bfloat16 (exact: at most 3 significant bits)
    decode_fp5(r.a, r.b, h);
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = pack_bf16((float)h[p][0], (float)h[p][1]);
  } else if constexpr (F == WQ_FMT_W4E2M1) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[4 * i] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 0));
      out[4 * i + 1] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 1));
      out[4 * i + 2] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 2));
      out[4 * i + 3] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 3));
    }
  } else {
    const uint32_t w[16] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w,
                            r.c.x, r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w};
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = as_h2(w[p]);
  }
}

// zero-point constants of one W4 group
__device__ __forceinline__ void w4_consts(uint16_t zbits, h2& zc1, h2& zc2) {
  const _Float16 z = __builtin_bit_cast(_Float16, zbits);
  const _Float16 c1 = (_Float16)-1024.0f - z, c2 = (_Float16)-64.0f - z;   // exact integers
  zc1 = h2{c1, c1};
  zc2 = h2{c2, c2};
}

// ---------------------------------------------------------------- wave reduction
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes with DPP only (no LDS): the total lands in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp<0x141, 0xF>(v);   // row_half_mirror: adds the other quad of each 8 lanes
  v += dpp<0x140, 0xF>(v);   // row_mirror: adds the other half of each 16-lane row
  v += dpp<0x142, 0xA>(v);   // row_bcast15: rows 1 and 3 add the last lane of rows 0 and 2
  v += dpp<0x143, 0xC>(v);   // row_bcast31: rows 2 and 3 add lane 31
  return v;
}


// A wave-uniform byte offset held in SGPRs. Adding it to a kernel-argument pointer keeps
// the global address space and lets loads take the SGPR-base + 32-bit VGPR offset form
// instead of a per-lane 64-bit address computed on the VALU.
__device__ __forceinline__ size_t uniform(size_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<size_t>(hi) << 32) | lo;
}

// The W4 decode of the matrix-core kernels with its masks in VGPRs, so that each pair takes one
// v_and_or_b32 (with literal masks the compiler emits an AND and an OR). The masks are made once,
// outside the loops. Nibbles 0 and 2 of a byte pair, placed in the mantissa of 1024.0 (step 1),
// give 1024 + q; nibbles 1 and 3, placed in that of 64.0 (step 1/16, where the nibble weighs 16),
// give 64 + q; adding zc1 = -(1024 + z) or zc2 = -(64 + z) gives q - z exactly.
struct W4Masks { uint32_t lo, hi, mag_lo, mag_hi; };
__device__ __forceinline__ W4Masks w4_masks() {
  return {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u), in_vgpr(0x54005400u)};
}
__device__ __forceinline__ void decode_w4_unit(const uint4& r, h2 zc1, h2 zc2, const W4Masks& k, h2 (&out)[16]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // word i: codes 8i..8i+7, pair t = codes 8i+2t (nibble t), 8i+2t+1 (nibble t+4)
    const uint32_t d = w[i], e = d >> 8;
    out[4 * i] = as_h2((d & k.lo) | k.mag_lo) + zc1;
    out[4 * i + 1] = as_h2((d & k.hi) | k.mag_hi) + zc2;
    out[4 * i + 2] = as_h2((e & k.lo) | k.mag_lo) + zc1;
    out[4 * i + 3] = as_h2((e & k.hi) | k.mag_hi) + zc2;
  }
}

__device__ __forceinline__ uint4 ld_nt16(const uint8_t* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint32_t ld_nt4(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint2 ld_nt8(const uint8_t* p) {
  const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(t[0], t[1]);
}

}  // namespace

// Every kernel code: the weight formats with fp16 activations, and (all but F16, W3G32 and
// W6E3M2_P24) with bfloat16 ones.
#define WQ_KERNEL_CODES(X)                                                                              \
  X(WQ_FMT_F16) X(WQ_FMT_W8) X(WQ_FMT_W4G32) X(WQ_FMT_W6E3M2) X(WQ_FMT_W4E2M1)                          \
  X(WQ_FMT_W8 | WQ_ACT_BF16) X(WQ_FMT_W4G32 | WQ_ACT_BF16) X(WQ_FMT_W6E3M2 | WQ_ACT_BF16)              \
  X(WQ_FMT_W4E2M1 | WQ_ACT_BF16) X(WQ_FMT_BF16 | WQ_ACT_BF16) X(WQ_FMT_W5E2M2) X(WQ_FMT_W5E2M2 | WQ_ACT_BF16) \
  X(WQ_FMT_W3G32) X(WQ_FMT_W6E3M2_P24)

#endif  // WQ_DEVICE_H_
