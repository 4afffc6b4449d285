// Host half of libwq: argument checks, sizes, and the offline quantize + pack step.
//
// The FP6-LLM news page (m.zhengruan.com), section "重新设计内核方案", re-packs the
// low-bit weights before inference so that the kernel reads aligned 32/64-bit blocks.
// Here that step runs on the host in float64, row-parallel over std::thread workers,
// and writes the layout declared in include/wq.h.
//
// Scale and code rules (readings; the pages give names, not formulas):
//   int8  per row:       s = fp16(max|w| / 127),      q = clamp(rint(w/s), -127, 127)
//   int4  per 32 along K: s = fp16((hi - lo) / 15), z = clamp(rint(-lo/s), 0, 15),
//                        q = clamp(rint(w/s) + z, 0, 15), lo/hi widened to include 0
//   int3  per 32 along K: the same with 7 in place of 15
//   fp6   per row:       s = fp16(max|w| / 28),       code = e3m2 nearest to w/s (two layouts)
//   fp4   per row:       s = fp16(max|w| / 6),        code = e2m1 nearest to w/s
//   fp5   per row:       s = fp16(max|w| / 7),        code = e2m2 nearest to w/s
// Every quotient is one IEEE float64 operation; every rounding is to nearest even.

#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace wq {

// float64 -> fp16 bits, round to nearest even, written from the fp16 definition:
// normal values (1 + n/1024) 2^E for E in [-14, 15], subnormals n 2^-24.
uint16_t f64_to_f16_bits(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (std::isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // rounds past 65504 (or is infinite)
  if (a < 0x1p-14) {
    // subnormal range: spacing 2^-24; a * 2^24 is exact, rint rounds half to even
    const double n = std::nearbyint(a * 0x1p24);
    return sign | static_cast<uint16_t>(n);  // n == 1024 encodes 2^-14, the smallest normal
  }
  int e2 = 0;
  (void)std::frexp(a, &e2);  // a = f 2^e2, f in [0.5, 1)
  int E = e2 - 1;            // 2^E <= a < 2^(E+1)
  const double frac = std::ldexp(a, -E) - 1.0;  // exact, in [0, 1)
  double n = std::nearbyint(frac * 1024.0);     // exact product, rounded half to even
  if (n == 1024.0) { n = 0.0; ++E; }
  if (E > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((E + 15) << 10) | static_cast<int>(n));
}

double f16_bits_to_f64(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

// e3m2 code of a finite float64 t: sign from t's sign bit, magnitude rounded to the
// nearest e3m2 value with ties to the even code, saturating at 28. Written from the
// format's structure: below 0.25 the values are multiples of 1/16 (codes 0..4, code 4
// being 0.25); from 0.25 up, exponent E in [-2, 4] and two mantissa bits.
uint8_t e3m2_encode(double t) {
  const uint8_t sign = std::signbit(t) ? 0x20 : 0;
  const double a = std::fabs(t);
  if (a >= 28.0) return sign | 31;
  if (a < 0.25) {
    const double n = std::nearbyint(a * 16.0);  // exact product; 0..4
    return sign | static_cast<uint8_t>(n);
  }
  int e2 = 0;
  (void)std::frexp(a, &e2);
  const int E = e2 - 1;                               // -2 .. 4
  const double m = std::nearbyint((std::ldexp(a, -E) - 1.0) * 4.0);  // 0..4, ties to even
  int code = 4 * (E + 3) + static_cast<int>(m);       // m == 4 carries into the next binade
  if (code > 31) code = 31;
  return sign | static_cast<uint8_t>(code);
}

// e2m1 code of a finite float64 t, by the same rules as e3m2_encode (sign kept, ties to the
// even code, saturating at 6). Below 1 the values are multiples of 1/2 (codes 0..2, code 2
// being 1); from 1 up, exponent E in [0, 2] and one mantissa bit.
uint8_t e2m1_encode(double t) {
  const uint8_t sign = std::signbit(t) ? 0x8 : 0;
  const double a = std::fabs(t);
  if (a >= 6.0) return sign | 7;
  if (a < 1.0) return sign | static_cast<uint8_t>(std::nearbyint(a * 2.0));   // exact product; 0..2
  int e2 = 0;
  (void)std::frexp(a, &e2);
  const int E = e2 - 1;                                                 // 0 .. 2
  const double m = std::nearbyint((std::ldexp(a, -E) - 1.0) * 2.0);     // 0..2, ties to even
  int code = 2 * (E + 1) + static_cast<int>(m);                         // m == 2 carries into the next binade
  if (code > 7) code = 7;
  return sign | static_cast<uint8_t>(code);
}

// e2m2 code of a finite float64 t, by the same rules (sign kept, ties to the even code,
// saturating at 7). Below 1 the values are multiples of 1/4 (codes 0..4, code 4 being 1); from
// 1 up, exponent E in [0, 2] and two mantissa bits.
uint8_t e2m2_encode(double t) {
  const uint8_t sign = std::signbit(t) ? 0x10 : 0;
  const double a = std::fabs(t);
  if (a >= 7.0) return sign | 15;
  if (a < 1.0) return sign | static_cast<uint8_t>(std::nearbyint(a * 4.0));   // exact product; 0..4
  int e2 = 0;
  (void)std::frexp(a, &e2);
  const int E = e2 - 1;                                                 // 0 .. 2
  const double m = std::nearbyint((std::ldexp(a, -E) - 1.0) * 4.0);     // 0..4, ties to even
  int code = 4 * (E + 1) + static_cast<int>(m);                         // m == 4 carries into the next binade
  if (code > 15) code = 15;
  return sign | static_cast<uint8_t>(code);
}

namespace {

bool shape_ok(int64_t N, int64_t K) { return N >= 1 && K >= 32 && K % 32 == 0; }

int fmt_bits(int fmt) {
  switch (fmt) {
    case WQ_FMT_F16: return 16;
    case WQ_FMT_W8: return 8;
    case WQ_FMT_W4G32: return 4;
    case WQ_FMT_W6E3M2: return 6;
    case WQ_FMT_W4E2M1: return 4;
    case WQ_FMT_BF16: return 16;
    case WQ_FMT_W5E2M2: return 5;
    case WQ_FMT_W3G32: return 3;
    case WQ_FMT_W6E3M2_P24: return 6;
    default: return 0;
  }
}

// The size calls take a format code with or without the activation flag.
int weight_fmt(int fmt) { return (fmt & ~0xFF) == WQ_ACT_BF16 ? (fmt & 0xFF) : fmt; }

// Run f(row_begin, row_end) over [0, N) on up to hardware_concurrency threads and return the
// first non-OK status.
template <class F>
int parallel_rows(int64_t N, int64_t work_per_row, F f) {
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int64_t total = N * work_per_row;
  unsigned nt = static_cast<unsigned>(std::min<int64_t>(hw, std::max<int64_t>(1, total / (1 << 20))));
  nt = std::max(1u, std::min<unsigned>(nt, static_cast<unsigned>(N)));
  if (nt == 1) return f(0, N);
  std::vector<std::thread> ts;
  std::vector<int> st(nt, WQ_OK);
  int64_t per = (N + nt - 1) / nt;
  for (unsigned i = 0; i < nt; ++i) {
    int64_t b = i * per, e = std::min<int64_t>(N, b + per);
    if (b >= e) break;
    ts.emplace_back([&, i, b, e] { st[i] = f(b, e); });
  }
  for (auto& t : ts) t.join();
  for (int s : st)
    if (s != WQ_OK) return s;
  return WQ_OK;
}

// ---- layout writers (one 32-code unit at a time) ----
void put_unit_w8(uint8_t* dst, const int8_t* q) {
  for (int j = 0; j < 32; ++j) dst[j] = static_cast<uint8_t>(q[j] + 128);
}
void put_unit_w4(uint8_t* dst, const uint8_t* q) {
  for (int d = 0; d < 4; ++d) {
    uint32_t word = 0;
    for (int t = 0; t < 4; ++t) {
      word |= static_cast<uint32_t>(q[8 * d + 2 * t] & 15) << (4 * t);
      word |= static_cast<uint32_t>(q[8 * d + 2 * t + 1] & 15) << (4 * (t + 4));
    }
    for (int b = 0; b < 4; ++b) dst[4 * d + b] = static_cast<uint8_t>(word >> (8 * b));
  }
}
void put_unit_w6(uint8_t* dst, const uint8_t* c) {
  // 32 codes x 6 bits = 192 bits, low code first; assembled in three 64-bit words
  uint64_t w[3] = {0, 0, 0};
  for (int j = 0; j < 32; ++j) {
    const int bit = 6 * j, word = bit >> 6, off = bit & 63;
    w[word] |= static_cast<uint64_t>(c[j] & 63) << off;
    if (off > 58) w[word + 1] |= static_cast<uint64_t>(c[j] & 63) >> (64 - off);
  }
  for (int i = 0; i < 24; ++i) dst[i] = static_cast<uint8_t>(w[i >> 3] >> (8 * (i & 7)));
}

// W6 units are stored split by planes, 64 units ("chunk") at a time: bytes 0..15 of the
// chunk's Uc units first, then bytes 16..23 of the same units. Returns where the two
// slices of unit u of row r live.
template <class P>
void w6_unit_homes(P base, int64_t r, int64_t u, int64_t U, P& lo, P& hi) {
  const int64_t c = u / 64, j = u % 64, uc = std::min<int64_t>(64, U - 64 * c);
  P chunk = base + (r * U + 64 * c) * 24;
  lo = chunk + 16 * j;
  hi = chunk + 16 * uc + 8 * j;
}

// FP5: the same chunks of 64 units; 16 bytes of magnitude nibbles per unit, then 4 bytes of signs.
template <class P>
void w5_unit_homes(P base, int64_t r, int64_t u, int64_t U, P& lo, P& hi) {
  const int64_t c = u / 64, j = u % 64, uc = std::min<int64_t>(64, U - 64 * c);
  P chunk = base + (r * U + 64 * c) * 20;
  lo = chunk + 16 * j;
  hi = chunk + 16 * uc + 4 * j;
}

// A word of one bit of every code of a unit: bit `bit` of code 2p in bit p, of code 2p+1 in bit
// 16+p (the FP5 sign word: bit 4; the P24 bit-4 and sign words: bits 4 and 5).
uint32_t bit_word(const uint8_t* c, int bit) {
  uint32_t s = 0;
  for (int p = 0; p < 16; ++p) s |= static_cast<uint32_t>((c[2 * p] >> bit) & 1) << p |
                                   static_cast<uint32_t>((c[2 * p + 1] >> bit) & 1) << (16 + p);
  return s;
}

// W3: pair p = codes (2p, 2p+1); pairs 0..14 in word p / 5 at these offsets (even code in the
// low half, odd code 16 bits up); bit b of the last pair in bits 9 and 25 of word b.
constexpr int kW3Offset[5] = {0, 3, 6, 10, 13};

void put_unit_w3(uint8_t* dst, const uint8_t* q) {
  uint32_t w[3] = {0, 0, 0};
  for (int p = 0; p < 15; ++p) {
    const int o = kW3Offset[p % 5];
    w[p / 5] |= static_cast<uint32_t>(q[2 * p] & 7) << o | static_cast<uint32_t>(q[2 * p + 1] & 7) << (16 + o);
  }
  for (int b = 0; b < 3; ++b)
    w[b] |= static_cast<uint32_t>((q[30] >> b) & 1) << 9 | static_cast<uint32_t>((q[31] >> b) & 1) << 25;
  for (int i = 0; i < 12; ++i) dst[i] = static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3)));
}

void get_unit_w3(const uint8_t* src, uint8_t* q) {
  uint32_t w[3];
  for (int i = 0; i < 3; ++i)
    w[i] = src[4 * i] | (src[4 * i + 1] << 8) | (src[4 * i + 2] << 16) | (static_cast<uint32_t>(src[4 * i + 3]) << 24);
  for (int p = 0; p < 15; ++p) {
    const int o = kW3Offset[p % 5];
    q[2 * p] = (w[p / 5] >> o) & 7;
    q[2 * p + 1] = (w[p / 5] >> (16 + o)) & 7;
  }
  q[30] = q[31] = 0;
  for (int b = 0; b < 3; ++b) {
    q[30] |= static_cast<uint8_t>(((w[b] >> 9) & 1) << b);
    q[31] |= static_cast<uint8_t>(((w[b] >> 25) & 1) << b);
  }
}

int check_weights(const float* w, int64_t K, int64_t r) {
  for (int64_t k = 0; k < K; ++k)
    if (!std::isfinite(w[r * K + k])) return WQ_ERR_NONFINITE;
  return WQ_OK;
}

}  // namespace
}  // namespace wq

using namespace wq;

extern "C" {

int wq_version(void) { return (1 << 16) | 0; }

const char* wq_status_string(int s) {
  switch (s) {
    case WQ_OK: return "ok";
    case WQ_ERR_ARG: return "invalid argument (NULL pointer or negative size)";
    case WQ_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 32, N >= 1, M >= 1)";
    case WQ_ERR_FMT: return "unknown weight format";
    case WQ_ERR_NONFINITE: return "non-finite weight";
    case WQ_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case WQ_ERR_DEVICE: return "HIP runtime error at launch";
    case WQ_ERR_RANGE: return "scale overflows fp16";
    case WQ_ERR_SCRATCH: return "sizes exceed the scratch buffer of a no-allocation call";
    default: return "unknown status";
  }
}

size_t wq_packed_bytes(int fmt, int64_t N, int64_t K) {
  fmt = weight_fmt(fmt);
  int b = fmt_bits(fmt);
  if (!b || !shape_ok(N, K)) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) * b / 8;
}

size_t wq_scales_bytes(int fmt, int64_t N, int64_t K) {
  fmt = weight_fmt(fmt);
  if (!fmt_bits(fmt) || !shape_ok(N, K) || fmt == WQ_FMT_F16 || fmt == WQ_FMT_BF16) return 0;
  const bool grouped = fmt == WQ_FMT_W4G32 || fmt == WQ_FMT_W3G32;
  return grouped ? static_cast<size_t>(N) * (K / 32) * 2 : static_cast<size_t>(N) * 2;
}

size_t wq_zeros_bytes(int fmt, int64_t N, int64_t K) {
  fmt = weight_fmt(fmt);
  if ((fmt != WQ_FMT_W4G32 && fmt != WQ_FMT_W3G32) || !shape_ok(N, K)) return 0;
  return static_cast<size_t>(N) * (K / 32) * 2;
}

int wq_pack_int8(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales) {
  if (!w || !packed || !scales || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  return parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    std::vector<int8_t> q(K);
    for (int64_t r = r0; r < r1; ++r) {
      if (check_weights(w, K, r)) return static_cast<int>(WQ_ERR_NONFINITE);
      const float* row = w + r * K;
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs(row[k]));
      const uint16_t sb = f64_to_f16_bits(static_cast<double>(amax) / 127.0);
      if ((sb & 0x7FFF) == 0x7C00) return static_cast<int>(WQ_ERR_RANGE);
      const double s = f16_bits_to_f64(sb);
      scales[r] = sb;
      for (int64_t k = 0; k < K; ++k) {
        double v = s > 0 ? std::nearbyint(static_cast<double>(row[k]) / s) : 0.0;
        q[k] = static_cast<int8_t>(std::min(127.0, std::max(-127.0, v)));
      }
      for (int64_t u = 0; u < K / 32; ++u) put_unit_w8(out + (r * K + 32 * u), q.data() + 32 * u);
    }
    return static_cast<int>(WQ_OK);
  });
}

}  // extern "C"

namespace {

// int4 / int3: codes 0..top with an fp16 scale and an integer zero point per group of 32 K;
// put writes one unit of UB bytes.
template <int UB, class Put>
int pack_asymmetric_g32(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, uint16_t* zeros,
                        double top, Put put) {
  if (!w || !packed || !scales || !zeros || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t G = K / 32;
  return parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    uint8_t q[32];
    for (int64_t r = r0; r < r1; ++r) {
      if (check_weights(w, K, r)) return static_cast<int>(WQ_ERR_NONFINITE);
      for (int64_t g = 0; g < G; ++g) {
        const float* grp = w + r * K + 32 * g;
        double lo = 0.0, hi = 0.0;
        for (int j = 0; j < 32; ++j) {
          lo = std::min(lo, static_cast<double>(grp[j]));
          hi = std::max(hi, static_cast<double>(grp[j]));
        }
        const uint16_t sb = f64_to_f16_bits((hi - lo) / top);
        if ((sb & 0x7FFF) == 0x7C00) return static_cast<int>(WQ_ERR_RANGE);
        const double s = f16_bits_to_f64(sb);
        double z = 0.0;
        if (s > 0) {
          z = std::min(top, std::max(0.0, std::nearbyint(-lo / s)));
          for (int j = 0; j < 32; ++j) {
            double v = std::nearbyint(static_cast<double>(grp[j]) / s) + z;
            q[j] = static_cast<uint8_t>(std::min(top, std::max(0.0, v)));
          }
        } else {
          std::memset(q, 0, sizeof(q));
        }
        scales[r * G + g] = sb;
        zeros[r * G + g] = static_cast<uint16_t>(f64_to_f16_bits(z) & 0x7FFF);  // integer zero point: +0 never -0
        put(out + (r * G + g) * UB, q);
      }
    }
    return static_cast<int>(WQ_OK);
  });
}

}  // namespace

extern "C" {

int wq_pack_int4(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, uint16_t* zeros) {
  return pack_asymmetric_g32<16>(w, N, K, packed, scales, zeros, 15.0, put_unit_w4);
}

int wq_pack_int3(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, uint16_t* zeros) {
  return pack_asymmetric_g32<12>(w, N, K, packed, scales, zeros, 7.0, put_unit_w3);
}

}  // extern "C"

namespace {

// FP6 e3m2 per row, in the bf6-convert layout (p24 false) or the 2+4 split (p24 true); both
// store a unit as a 16-byte and an 8-byte slice in W6's planes.
int pack_fp6_rows(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, bool p24) {
  if (!w || !packed || !scales || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t U = K / 32;
  return parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    std::vector<uint8_t> c(K);
    for (int64_t r = r0; r < r1; ++r) {
      if (check_weights(w, K, r)) return static_cast<int>(WQ_ERR_NONFINITE);
      const float* row = w + r * K;
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs(row[k]));
      const uint16_t sb = f64_to_f16_bits(static_cast<double>(amax) / 28.0);
      if ((sb & 0x7FFF) == 0x7C00) return static_cast<int>(WQ_ERR_RANGE);
      const double s = f16_bits_to_f64(sb);
      scales[r] = sb;
      for (int64_t k = 0; k < K; ++k) c[k] = s > 0 ? e3m2_encode(static_cast<double>(row[k]) / s) : 0;
      for (int64_t u = 0; u < U; ++u) {
        const uint8_t* cu = c.data() + 32 * u;
        uint8_t unit[24];
        if (p24) {
          put_unit_w4(unit, cu);   // the low four bits, placed as W4 codes
          const uint32_t e2 = bit_word(cu, 4), sg = bit_word(cu, 5);
          for (int b = 0; b < 4; ++b) {
            unit[16 + b] = static_cast<uint8_t>(e2 >> (8 * b));
            unit[20 + b] = static_cast<uint8_t>(sg >> (8 * b));
          }
        } else {
          put_unit_w6(unit, cu);
        }
        uint8_t* lo;
        uint8_t* hi;
        w6_unit_homes(out, r, u, U, lo, hi);
        std::memcpy(lo, unit, 16);
        std::memcpy(hi, unit + 16, 8);
      }
    }
    return static_cast<int>(WQ_OK);
  });
}

}  // namespace

extern "C" {

int wq_pack_fp6(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales) {
  return pack_fp6_rows(w, N, K, packed, scales, false);
}

int wq_pack_fp6_p24(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales) {
  return pack_fp6_rows(w, N, K, packed, scales, true);
}

int wq_pack_fp4(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales) {
  if (!w || !packed || !scales || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  return parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) {
      if (check_weights(w, K, r)) return static_cast<int>(WQ_ERR_NONFINITE);
      const float* row = w + r * K;
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs(row[k]));
      const uint16_t sb = f64_to_f16_bits(static_cast<double>(amax) / 6.0);
      if ((sb & 0x7FFF) == 0x7C00) return static_cast<int>(WQ_ERR_RANGE);
      const double s = f16_bits_to_f64(sb);
      scales[r] = sb;
      // byte p of the row holds code 2p in its low nibble and code 2p+1 in its high nibble
      for (int64_t k = 0; k < K; k += 2) {
        const uint8_t lo = s > 0 ? e2m1_encode(static_cast<double>(row[k]) / s) : 0;
        const uint8_t hi = s > 0 ? e2m1_encode(static_cast<double>(row[k + 1]) / s) : 0;
        out[(r * K + k) / 2] = static_cast<uint8_t>(lo | (hi << 4));
      }
    }
    return static_cast<int>(WQ_OK);
  });
}

int wq_pack_fp5(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales) {
  if (!w || !packed || !scales || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t U = K / 32;
  return parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
    std::vector<uint8_t> c(K);
    for (int64_t r = r0; r < r1; ++r) {
      if (check_weights(w, K, r)) return static_cast<int>(WQ_ERR_NONFINITE);
      const float* row = w + r * K;
      float amax = 0.0f;
      for (int64_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs(row[k]));
      const uint16_t sb = f64_to_f16_bits(static_cast<double>(amax) / 7.0);
      if ((sb & 0x7FFF) == 0x7C00) return static_cast<int>(WQ_ERR_RANGE);
      const double s = f16_bits_to_f64(sb);
      scales[r] = sb;
      for (int64_t k = 0; k < K; ++k) c[k] = s > 0 ? e2m2_encode(static_cast<double>(row[k]) / s) : 0;
      for (int64_t u = 0; u < U; ++u) {
        uint8_t* lo;
        uint8_t* hi;
        w5_unit_homes(out, r, u, U, lo, hi);
        put_unit_w4(lo, c.data() + 32 * u);   // the low four bits, placed as W4 codes
        const uint32_t sw = bit_word(c.data() + 32 * u, 4);
        for (int b = 0; b < 4; ++b) hi[b] = static_cast<uint8_t>(sw >> (8 * b));
      }
    }
    return static_cast<int>(WQ_OK);
  });
}

int wq_unpack(int fmt, const void* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
              void* codes, uint16_t* scales_out, uint16_t* zeros_out) {
  if (!fmt_bits(fmt)) return WQ_ERR_FMT;
  if (!packed || !codes || N < 0 || K < 0) return WQ_ERR_ARG;
  if (!shape_ok(N, K)) return WQ_ERR_SHAPE;
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  const int64_t U = K / 32;
  if (fmt == WQ_FMT_W8) {
    int8_t* o = static_cast<int8_t*>(codes);
    for (int64_t i = 0; i < N * K; ++i) o[i] = static_cast<int8_t>(static_cast<int>(in[i]) - 128);
  } else if (fmt == WQ_FMT_W4G32) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t r = 0; r < N; ++r)
      for (int64_t u = 0; u < U; ++u)
        for (int d = 0; d < 4; ++d) {
          const uint8_t* p = in + (r * U + u) * 16 + 4 * d;
          const uint32_t word = p[0] | (p[1] << 8) | (p[2] << 16) | (static_cast<uint32_t>(p[3]) << 24);
          for (int t = 0; t < 4; ++t) {
            o[r * K + 32 * u + 8 * d + 2 * t] = (word >> (4 * t)) & 15;
            o[r * K + 32 * u + 8 * d + 2 * t + 1] = (word >> (4 * (t + 4))) & 15;
          }
        }
  } else if (fmt == WQ_FMT_W6E3M2) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t r = 0; r < N; ++r)
      for (int64_t u = 0; u < U; ++u) {
        const uint8_t* lo;
        const uint8_t* hi;
        w6_unit_homes(in, r, u, U, lo, hi);
        uint8_t p[24];
        std::memcpy(p, lo, 16);
        std::memcpy(p + 16, hi, 8);
        for (int j = 0; j < 32; ++j) {
          int v = 0;
          for (int b = 0; b < 6; ++b) {
            const int bit = 6 * j + b;
            v |= ((p[bit >> 3] >> (bit & 7)) & 1) << b;
          }
          o[r * K + 32 * u + j] = static_cast<uint8_t>(v);
        }
      }
  } else if (fmt == WQ_FMT_W3G32) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t i = 0; i < N * U; ++i) get_unit_w3(in + 12 * i, o + 32 * i);
  } else if (fmt == WQ_FMT_W6E3M2_P24) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t r = 0; r < N; ++r)
      for (int64_t u = 0; u < U; ++u) {
        const uint8_t* lo;
        const uint8_t* hi;
        w6_unit_homes(in, r, u, U, lo, hi);
        uint8_t* cu = o + r * K + 32 * u;
        for (int d = 0; d < 4; ++d) {
          const uint32_t word = lo[4 * d] | (lo[4 * d + 1] << 8) | (lo[4 * d + 2] << 16) |
                                (static_cast<uint32_t>(lo[4 * d + 3]) << 24);
          for (int t = 0; t < 4; ++t) {
            cu[8 * d + 2 * t] = (word >> (4 * t)) & 15;
            cu[8 * d + 2 * t + 1] = (word >> (4 * (t + 4))) & 15;
          }
        }
        for (int b = 0; b < 2; ++b) {
          const uint8_t* h = hi + 4 * b;
          const uint32_t bw = h[0] | (h[1] << 8) | (h[2] << 16) | (static_cast<uint32_t>(h[3]) << 24);
          for (int p = 0; p < 16; ++p) {
            cu[2 * p] |= static_cast<uint8_t>(((bw >> p) & 1) << (4 + b));
            cu[2 * p + 1] |= static_cast<uint8_t>(((bw >> (16 + p)) & 1) << (4 + b));
          }
        }
      }
  } else if (fmt == WQ_FMT_W4E2M1) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t i = 0; i < N * K / 2; ++i) {
      o[2 * i] = in[i] & 15;
      o[2 * i + 1] = in[i] >> 4;
    }
  } else if (fmt == WQ_FMT_W5E2M2) {
    uint8_t* o = static_cast<uint8_t*>(codes);
    for (int64_t r = 0; r < N; ++r)
      for (int64_t u = 0; u < U; ++u) {
        const uint8_t* lo;
        const uint8_t* hi;
        w5_unit_homes(in, r, u, U, lo, hi);
        uint8_t* cu = o + r * K + 32 * u;
        for (int d = 0; d < 4; ++d) {
          const uint32_t word = lo[4 * d] | (lo[4 * d + 1] << 8) | (lo[4 * d + 2] << 16) |
                                (static_cast<uint32_t>(lo[4 * d + 3]) << 24);
          for (int t = 0; t < 4; ++t) {
            cu[8 * d + 2 * t] = (word >> (4 * t)) & 15;
            cu[8 * d + 2 * t + 1] = (word >> (4 * (t + 4))) & 15;
          }
        }
        const uint32_t sw = hi[0] | (hi[1] << 8) | (hi[2] << 16) | (static_cast<uint32_t>(hi[3]) << 24);
        for (int p = 0; p < 16; ++p) {
          cu[2 * p] |= static_cast<uint8_t>(((sw >> p) & 1) << 4);
          cu[2 * p + 1] |= static_cast<uint8_t>(((sw >> (16 + p)) & 1) << 4);
        }
      }
  } else {
    std::memcpy(codes, packed, static_cast<size_t>(N) * K * 2);
  }
  if (scales_out && scales) std::memcpy(scales_out, scales, wq_scales_bytes(fmt, N, K));
  if (zeros_out && zeros) std::memcpy(zeros_out, zeros, wq_zeros_bytes(fmt, N, K));
  return WQ_OK;
}

}  // extern "C"
