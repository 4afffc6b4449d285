/*
 * wq.h -- C ABI of libwq: weight-only-quantized linear layers on AMD MI355X (gfx950).
 *
 * The operation is the linear layer of LLM decode with low-bit weights and fp16
 * activations:  y[M,N] = x[M,K] . dequant(Wq)[N,K]^T  (fp16 in and out, fp32 sums).
 *   - gpt-fast write-up (m.greenbasetech.com): decode is bound by memory bandwidth; the
 *     lever is fewer bytes per parameter, first int8, then groupwise int4 weights.
 *   - gpt-fast guide (www.jsqmd.com), section "量化技术深度解析": int4, group size 32.
 *   - FP6-LLM news (m.zhengruan.com), section "重新设计内核方案": FP6 weights with fp16
 *     activations; dequantization fused with the matrix product in one kernel, and the
 *     weights re-packed offline into aligned 32/64-bit blocks; one kernel design for
 *     weights of several bit widths.
 *
 * Formats (the pages give names, not bit formats; these are this library's readings):
 *   WQ_FMT_W8      int8, symmetric, one fp16 scale per output row: s = fp16(max|w|/127),
 *                  q = clamp(rint(w/s), -127, 127), w^ = q*s.
 *   WQ_FMT_W4G32   int4, asymmetric, groups of 32 consecutive K: s = fp16((hi-lo)/15) with
 *                  lo = min(min w, 0), hi = max(max w, 0); integer zero point
 *                  z = clamp(rint(-lo/s), 0, 15) stored as fp16; q = clamp(rint(w/s)+z, 0, 15);
 *                  w^ = (q-z)*s.
 *   WQ_FMT_W6E3M2  FP6 e3m2 (sign, 3 exponent bits with bias 3, 2 mantissa bits, subnormals,
 *                  no inf/NaN, max 28), one fp16 scale per row: s = fp16(max|w|/28), code =
 *                  nearest e3m2 to w/s (ties to even code, saturating); w^ = e3m2(code)*s.
 *   WQ_FMT_W4E2M1  FP4 e2m1 (sign, 2 exponent bits with bias 1, 1 mantissa bit, a subnormal,
 *                  no inf/NaN, max 6), one fp16 scale per row: s = fp16(max|w|/6), code =
 *                  nearest e2m1 to w/s (ties to even code, saturating); w^ = e2m1(code)*s.
 *                  A further bit width through the same kernels; the pages name none.
 *   WQ_FMT_W5E2M2  FP5 e2m2 (sign, 2 exponent bits with bias 1, 2 mantissa bits, subnormals,
 *                  no inf/NaN, max 7), one fp16 scale per row: s = fp16(max|w|/7), code =
 *                  nearest e2m2 to w/s (ties to even code, saturating); w^ = e2m2(code)*s.
 *                  Another further bit width (the FP6-LLM news page, section "重新设计内核方案",
 *                  describes one kernel design for several bit widths and names none besides 6).
 *   WQ_FMT_W3G32   int3, asymmetric, groups of 32 consecutive K: int4's rule with 7 in place of
 *                  15 (s = fp16((hi-lo)/7), z = clamp(rint(-lo/s), 0, 7), q = clamp(rint(w/s)+z,
 *                  0, 7)); w^ = (q-z)*s. A further bit width, as for FP4 and FP5.
 *   WQ_FMT_W6E3M2_P24  the FP6 e3m2 codes and scales of WQ_FMT_W6E3M2 in a second layout, each
 *                  code split into a 4-bit and a 2-bit part (the "6 = 2 + 4" split of the
 *                  FP6-LLM news page, section "重新设计内核方案"), stitched back together with
 *                  bit operations instead of gfx950's bf6 convert: the two FP6 layouts side by side.
 *   WQ_FMT_F16     plain fp16 weights W[N,K] (the unquantized baseline); no metadata.
 *   WQ_FMT_BF16    plain bfloat16 weights W[N,K], the unquantized baseline for bfloat16
 *                  activations (WQ_ACT_BF16 below); no metadata.
 *   Quotients are IEEE float64 operations; rint and fp16 conversion round to nearest even.
 *   A scale that rounds to 0 makes the codes of its row or group 0 (and z = 0).
 *
 * Packed layout (identical for host and device): rows one after another; row n holds
 * K codes cut into units of 32 consecutive K, stored in order with no padding:
 *   W8  32 B: byte j = q_j + 128.
 *   W4  16 B: four little-endian u32; word d holds codes 8d..8d+7, code 8d+2t in nibble t,
 *             code 8d+2t+1 in nibble t+4.
 *   W6  24 B: code j in bits 6j..6j+5 of the unit read as a 192-bit little-endian number,
 *       stored split by planes: a row's units are taken 64 at a time (a chunk; the last
 *       chunk of a row may hold fewer, Uc), and in a chunk bytes 0..15 of its Uc units
 *       come first, unit after unit, then bytes 16..23 of the same units.
 *   FP4 16 B: code j in bits 4j..4j+3 of the unit read as a little-endian number (byte p:
 *       code 2p in the low nibble, code 2p+1 in the high nibble).
 *   FP5 20 B: bytes 0..15 hold the low four bits of the codes placed as W4 codes; bytes 16..19
 *       a little-endian u32 of signs, the sign of code 2p in bit p and of code 2p+1 in bit
 *       16+p. Stored split by planes in chunks of 64 units as W6 (bytes 0..15 of the chunk's
 *       units, then bytes 16..19 of the same units).
 *   W3  12 B: three little-endian u32. Codes 2p, 2p+1 form pair p; the even code sits in the low
 *       half of a word and the odd one in the high half at the same offset. Pair p < 15 is in
 *       word p / 5 at offset o = 0, 3, 6, 10, 13 for p % 5 = 0..4 (code 2p in bits o..o+2,
 *       code 2p+1 in bits 16+o..18+o); bit b of code 30 is bit 9 and bit b of code 31 bit 25
 *       of word b. Units stored whole.
 *   P24 24 B: bytes 0..15 hold the low four bits of the codes placed as W4 codes; bytes 16..19 a
 *       little-endian u32 with bit 4 of code 2p in bit p and of code 2p+1 in bit 16+p; bytes
 *       20..23 the same for bit 5 (the sign). Stored split by planes as W6.
 *   F16 64 B: fp16 weight j at bytes 2j..2j+1 (so F16 is the plain row-major matrix); BF16 the same
 *       with bfloat16 bits.
 * So packed_w is exactly N*K*bits/8 bytes. scales: W8/W6/P24/FP4/FP5 [N]; W4 and W3 [N][K/32]
 * row-major. zeros: W4 and W3 [N][K/32] row-major; otherwise unused (may be NULL). fp16 values are passed
 * as uint16_t bit patterns.
 *
 * Activations: by default x, y and dequantized weights are fp16. OR-ing WQ_ACT_BF16 into the
 * fmt argument of wq_dequant, wq_linear, wq_linear_grouped and the kernel-name calls makes them
 * bfloat16 (named besides fp16 by the gpt-fast guide, www.jsqmd.com, section "混合精度训练与推理",
 * and the speed-up strategies page, sharktoolz.top, section 4). The packed weights and their fp16 metadata are the same for both;
 * the product still accumulates in fp32, and the dequantized value of a weight is its exact
 * value rounded once to bfloat16. Valid codes with the flag: W8, W4G32, W6E3M2, W4E2M1, W5E2M2, BF16;
 * F16, W3G32 and W6E3M2_P24 weights take fp16 activations only and BF16 weights bfloat16 ones
 * (else WQ_ERR_FMT).
 * The size calls ignore the flag.
 *
 * Conventions for every call:
 *   - K must be a positive multiple of 32 and at most 2^26; N >= 1; M >= 1; N*K/32 must fit
 *     in an int32. Otherwise WQ_ERR_SHAPE.
 *   - Every error is returned synchronously, before anything is launched. The device
 *     calls never synchronize; a fault in a kernel shows up at the caller's next sync.
 *   - Memory is owned by the caller. The library allocates no device memory and may be called
 *     from several host threads at once. The only state it keeps between calls is, per host
 *     thread, the HIP error behind that thread's latest WQ_ERR_DEVICE (wq_last_device_error).
 *   - stream is a hipStream_t (NULL = the legacy default stream).
 */
#ifndef WQ_H_
#define WQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_FMT_F16 = 0, WQ_FMT_W8 = 1, WQ_FMT_W4G32 = 2, WQ_FMT_W6E3M2 = 3, WQ_FMT_W4E2M1 = 4, WQ_FMT_BF16 = 5,
  WQ_FMT_W5E2M2 = 6, WQ_FMT_W3G32 = 7, WQ_FMT_W6E3M2_P24 = 8
} wq_fmt;

/* Activation-type flag, OR-ed into a format code: bfloat16 x and y instead of fp16. */
typedef enum { WQ_ACT_F16 = 0, WQ_ACT_BF16 = 0x100 } wq_act;

typedef enum {
  WQ_OK = 0,
  WQ_ERR_ARG = -1,        /* NULL pointer or a negative size                        */
  WQ_ERR_SHAPE = -2,      /* K not a positive multiple of 32, N < 1 or M < 1         */
  WQ_ERR_FMT = -3,        /* unknown format code                                     */
  WQ_ERR_NONFINITE = -4,  /* a weight given to a packer is NaN or infinite           */
  WQ_ERR_ALIGN = -5,      /* a device pointer is not 16-byte aligned                 */
  WQ_ERR_DEVICE = -6,     /* the HIP runtime refused the launch                      */
  WQ_ERR_RANGE = -7,      /* a scale would overflow fp16 (max|w| too large)          */
  WQ_ERR_SCRATCH = -8     /* the sizes need more than a no-allocation call's scratch */
} wq_status;
/* WQ_ERR_DEVICE reflects only the call's own launches: the status of each launch is the value
 * that the launch call itself returns (hipLaunchKernel). An error that an earlier HIP runtime
 * call on the calling thread left pending, from this library or any other, is neither read
 * nor cleared by this library. */

/* Library version, (major << 16) | minor. */
int wq_version(void);

/* Human-readable text for a status code (static storage; never NULL). */
const char* wq_status_string(int status);

/* The name of the HIP runtime error (hipGetErrorName) behind the calling thread's most recent
 * WQ_ERR_DEVICE, or "none" if it has had none. Static storage; never NULL; no device call. */
const char* wq_last_device_error(void);

/* Sizes in bytes of packed_w, scales and zeros for (fmt, N, K); 0 for an invalid
 * combination (unknown fmt, N < 1, K not a positive multiple of 32) or, for zeros, a
 * format without zero points. Host only. */
size_t wq_packed_bytes(int fmt, int64_t N, int64_t K);
size_t wq_scales_bytes(int fmt, int64_t N, int64_t K);
size_t wq_zeros_bytes(int fmt, int64_t N, int64_t K);

/* Offline quantize + pack, on the host (the FP6-LLM page re-packs weights before
 * inference). w: host fp32 W[N,K], row-major. packed, scales, zeros: host buffers of
 * the sizes above, written completely. Rows are processed in parallel on host threads.
 * Errors: WQ_ERR_ARG, WQ_ERR_SHAPE, WQ_ERR_NONFINITE, WQ_ERR_RANGE; on error the output
 * buffers hold unspecified bytes. */
int wq_pack_int8(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales);
int wq_pack_int4(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, uint16_t* zeros);
int wq_pack_fp6(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales);
int wq_pack_fp4(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales);
int wq_pack_fp5(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales);
int wq_pack_int3(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales, uint16_t* zeros);
int wq_pack_fp6_p24(const float* w, int64_t N, int64_t K, void* packed, uint16_t* scales);

/* Inverse of the packers' layout step, on the host: packed -> logical codes [N,K]
 * (int8 for W8; 0..15 for W4 and FP4; 0..63 for W6; 0..31 for FP5, one byte each; uint16 fp16 bits for F16) and
 * a copy of the metadata in logical order (scales_out/zeros_out may be NULL to skip).
 * BF16: uint16 bfloat16 bits. A test hook. Errors: WQ_ERR_ARG, WQ_ERR_SHAPE, WQ_ERR_FMT. */
int wq_unpack(int fmt, const void* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
              void* codes, uint16_t* scales_out, uint16_t* zeros_out);

/* On the device: the dequantization step on its own. The FP6-LLM news page (m.zhengruan.com),
 * section "重新设计内核方案", describes turning the low-bit weights back into fp16 values, which the
 * fused kernels below do in registers; this call writes them out, as the separate dequant kernel of
 * the two-kernel approach that page contrasts with does (a test hook, and for callers that want the
 * dense weights). Dequantize packed weights to fp16 W^[N,K] row-major, w_out[n*K+k] =
 * fp16(w^[n,k]) rounded once to nearest even (bit-exact by construction: each product
 * is exact in fp32); with WQ_ACT_BF16 in fmt, bfloat16 rounded once to nearest even. All
 * pointers are device pointers, 16-byte aligned; zeros only for W4. Asynchronous on
 * stream. Errors: WQ_ERR_ARG, WQ_ERR_SHAPE, WQ_ERR_FMT, WQ_ERR_ALIGN, WQ_ERR_DEVICE. */
int wq_dequant(int fmt, const void* packed, const uint16_t* scales, const uint16_t* zeros, uint16_t* w_out,
               int64_t N, int64_t K, void* stream);

/* On the device: the fused weight-only-quantized linear layer. The FP6-LLM news page
 * (m.zhengruan.com), section "重新设计内核方案", fuses the dequantization and the matrix product
 * into one kernel that turns the packed weights into fp16 values on chip and feeds them to the
 * product; the gpt-fast write-up (m.greenbasetech.com, part on GPU quantization) explains why:
 * decode is bound by memory bandwidth, so the bytes per weight set its speed.
 * y[M,N] = x[M,K] . dequant(packed_w)[N,K]^T with fp16 x and y (bfloat16 with WQ_ACT_BF16 in
 * fmt; row-major, row strides K and N) and fp32 accumulation; the kernel reads every packed byte
 * once and never writes dequantized weights to memory. All pointers are device pointers, 16-byte
 * aligned; zeros only for W4 and W3 (else may be NULL). y must not overlap the inputs.
 * M of any size. The decode kernels take up to 64 rows of x per launch for W6, FP4, FP5 and W4
 * with K a multiple of 256, up to 16 for W8, fp16/bf16 weights and other W4 shapes, and more rows
 * run as several such launches. The tiled prefill kernel takes all rows in one launch from 193
 * rows on, and from fewer rows where its chain of K steps is short against its tile count: W8
 * and fp16/bf16 weights from 17 rows, W4, W6 and FP4 from 65, FP5 from 81.
 * Up to 4 rows the VALU GEMV runs, except on large matrices (N*K >= 2^24) where the LDS-staged
 * matrix-core kernel takes W4 and W3 (K a multiple of 256) and W6 from 3 rows, FP4 and FP5 from
 * 2, and W6 at 4 rows from N = 2048; W8 takes the fragment-load matrix-core kernel at 4 rows from
 * N = 4096. wq_linear_kernel_name names the kernel that runs for a shape.
 * Asynchronous on stream. Errors: WQ_ERR_ARG, WQ_ERR_SHAPE, WQ_ERR_FMT, WQ_ERR_ALIGN,
 * WQ_ERR_DEVICE. */
int wq_linear(const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros, uint16_t* y,
              int64_t M, int64_t N, int64_t K, int fmt, void* stream);

/* One independent linear of a grouped call: device pointers as for wq_linear. */
typedef struct {
  const uint16_t* x;       /* [M,K] fp16 */
  const void* packed_w;    /* packed weights of fmt */
  const uint16_t* scales;  /* as for wq_linear */
  const uint16_t* zeros;   /* W4 and W3 only, else NULL */
  uint16_t* y;             /* [M,N] fp16 output */
  int64_t N, K;
} wq_linear_item;

/* On the device: several linears in one launch. The gpt-fast write-up (m.greenbasetech.com,
 * part on torch.compile) finds decode held back because the CPU cannot issue work fast enough,
 * and hands the GPU bigger pieces of work at a time; a grouped call is that at the level of one
 * launch. count (0..16) independent linears of one format and one M in a single
 * launch, each computing exactly what wq_linear computes for it (same decode; the fp32
 * sum may run in another order when the items' sizes differ a lot). One launch
 * instead of count means the GPU ramps up and drains once; in a decode step this fits
 * q/k/v or gate/up, and any set of linears whose inputs are ready. Items must not write
 * into one another's inputs. The launch uses the kernel wq_linear would use for the
 * largest item (by N*K) for every item. When M is more than that kernel takes in one
 * launch (see wq_linear), every item runs as its own wq_linear call instead. Errors: as wq_linear, per item, all checked before any launch; WQ_ERR_ARG
 * also for count outside 0..16 or items == NULL. */
int wq_linear_grouped(const wq_linear_item* items, int count, int64_t M, int fmt, void* stream);

/* On the device: the first half of a Llama feed-forward in one launch, act = silu(gate) * up
 * (silu(g) = g / (1 + e^-g)), with the gate and up projections as one weight matrix of 2F rows:
 * row 2i is the gate projection's row i and row 2i+1 the up projection's row i (quantize and
 * pack the interleaved fp32 matrix [2F, K] with any wq_pack_*: every format's metadata is per row
 * or per group within a row, so the codes are those of the two matrices packed apart). The
 * speed-up strategies page (sharktoolz.top, section 6) and the gpt-fast write-up (part on
 * torch.compile) motivate the decode step this serves: fewer, larger launches per token.
 * act[m, i] = fp16(g / (1 + exp(-g)) * u) in float32, where g and u are rows 2i and 2i+1 of
 * y = x . dequant(packed_w)^T as wq_linear computes them with its decode kernels (rounded to
 * fp16 each); that is, the result equals wq_linear on the [2F, K] matrix followed by
 * wq_silu_mul (wq_decode.h) on its even and odd columns, bit for bit, wherever wq_linear takes
 * a decode kernel for the shape (wq_linear_kernel_name not "pf_kernel..."), without the 2F
 * outputs ever reaching memory. Prefill-sized M runs as several decode-kernel launches (never
 * the tiled prefill kernel). x [M, K] fp16; act [M, F] fp16; F >= 1; fp16 activations only
 * (WQ_ACT_BF16 in fmt: WQ_ERR_FMT). Other arguments and errors as wq_linear with N = 2F. */
int wq_linear_silu(const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros,
                   uint16_t* act, int64_t M, int64_t F, int64_t K, int fmt, void* stream);

/* Name of the kernel wq_linear launches for (fmt, M, N, K) (for profiles), or "" if the
 * arguments are invalid. Host only; static storage. */
const char* wq_linear_kernel_name(int fmt, int64_t M, int64_t N, int64_t K);

/* Name of the kernel wq_linear_grouped launches for count items of sizes N[i] x K[i] (with
 * separate launches: the largest item's kernel), or "". */
const char* wq_linear_grouped_kernel_name(int fmt, int64_t M, const int64_t* N, const int64_t* K, int count);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H_ */
