// Prefill half of libwq: the fused dequant + linear for many rows of x (gfx950, CDNA4).
//
// The FP6-LLM news page (m.zhengruan.com), section "重新设计内核方案", describes the fused
// kernel: weights re-packed offline, turned into fp16 values on chip and fed to the matrix
// units in the same kernel. Its batch range (the same page, on FP6-LLM's throughput across
// batch sizes) and gpt-fast's prefill compile option (the gpt-fast guide, www.jsqmd.com, section
// 高级优化技巧 -> 编译优化技巧) are the workloads where M reaches hundreds of rows. There the product
// (2 M N K flops) costs more than the weight stream, so this kernel tiles y and reuses each
// decoded weight for 128 rows of x.
//
// This translation unit is compiled with the MFMA accumulators in VGPRs (-mllvm
// -amdgpu-mfma-vgpr-form): with them in AGPRs the loop rotated all 64 accumulator registers
// through copies every iteration, and the kernel needed more than 256 registers per lane,
// i.e. one wave per SIMD. In VGPRs it needs under 256, so two workgroups share a CU.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "wq_device.h"
#include "wq_internal.h"

namespace {

// Past 64 rows of x the weight stream stops being the only cost: the product itself, 2 M N K
// flops, grows with M. Here a workgroup computes a 128 (x rows) x 128 (weight rows) tile of y.
// Per K step of 64 (two 32-code units of each weight row) it parks the x tile and the weight
// tile in LDS, the weights decoded once into 16-bit values of the activation type (the exact
// decode of the other kernels; W4 as fp16((q - z) s), the other formats as exact code values
// with their row scale applied to the result), and its four waves (2 x 2, 64 x 64 each) run 32
// MFMAs from there, so each decoded weight serves 128 rows of x and each x value 128 weight
// rows. Double-buffered LDS with one barrier per step; the global loads of the next two steps
// are in flight while a step is multiplied. A step is short (32 MFMAs per wave), so the time of
// a tile is the chain of its K steps: wq_linear takes this kernel from 193 rows of x on, where
// it beats launches of 64 rows that reread the weights. 64 or 72 KB of LDS and under 256 registers
// per lane let two workgroups share a CU. LDS rows are 128 B with the 16-byte chunks of each row
// XOR-swizzled by the row (the weight tile of W4 with fp16 activations: 144-byte padded rows).

constexpr int PF_MIN_M = 193;      // M from which the tiled kernel always runs
constexpr int PF_MIN_M_ANY = 65;   // below: the decode kernels (up to 64 rows in one launch)
constexpr int PF_BM = 128, PF_BN = 128;       // tile of y

// The LDS layout of a tile row (64 K of 16-bit values, 16-byte chunks c = 0..7): 128 bytes with
// chunk c at 16 (c ^ (row & 7)), see below; the weight tile of W4 with fp16 activations keeps
// 144-byte rows with chunks in order: its decode needs more registers, and the swizzled weight
// addresses took it past the 256 that two workgroups per CU allow (spills in the loop).
template <int FMT, bool W> constexpr bool pf_xor() { return !W || FMT != WQ_FMT_W4G32; }   // W: weight tile
template <int FMT, bool W> constexpr int pf_row() { return pf_xor<FMT, W>() ? 128 : 144; }   // bytes per row
template <int FMT> constexpr int pf_x_bytes() { return 128 * pf_row<FMT, false>(); }      // the x tile
template <int FMT> constexpr int pf_buf_bytes() { return pf_x_bytes<FMT>() + 128 * pf_row<FMT, true>(); }
template <int FMT> constexpr int pf_lds_bytes() { return 2 * pf_buf_bytes<FMT>(); }     // two buffers
template <int FMT, bool W> __device__ __forceinline__ int pf_off(int row, int c) {   // chunk c of a tile row
  return row * pf_row<FMT, W>() + ((pf_xor<FMT, W>() ? c ^ (row & 7) : c) << 4);
}

// Swizzled rows: chunk c (K 8c .. 8c+7) of LDS row `row` sits at 128 row + 16 (c ^ (row & 7)).
// A fragment read (16 consecutive rows, one chunk) then spreads over the banks without
// conflicts, and so does a park store (8 lanes per x row, or 4 weight rows x 2 halves). With
// 144-byte padded rows every fragment read loses 4 cycles to bank conflicts (measured), and the
// swizzle made W6, FP4 and F16 prefill 9-14% faster.

template <int FMT>
struct PfStage {
  uint4 x[4];               // 16 B of each of 4 x rows
  Raw<wfmt(FMT)> w;         // one unit of one weight row
  uint32_t sw, zw;          // W4, W3: the aligned 32-bit words holding that unit's group scale and zero
};

// x: load i of wave v covers x rows 32 v + 8 i .. +7 of the tile, 8 lanes per row, so every
// load reads whole 128-B lines (the step's 64 values of 8 rows). Weights: thread t stages row
// t/2 of the weight tile, unit (2 step + t%2) of the row.
__device__ __forceinline__ int pf_xrow(int t, int i) { return 32 * (t >> 6) + 8 * i + ((t & 63) >> 3); }
__device__ __forceinline__ int pf_xunit(int t, int step) { return 2 * step + ((t & 7) >> 2); }

template <int FMT>
__device__ __forceinline__ void pf_load(PfStage<FMT>& st, const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                        const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int m0,
                                        int n0, int M, int N, int K, int step, int r, int h) {
  const int U = K >> 5, t = threadIdx.x;
  const int u = min(2 * step + h, U - 1);   // past the row end: a valid unit, zeroed when parked
  const int nr = min(n0 + r, N - 1);
  const uint32_t xo = 64u * (uint32_t)min(pf_xunit(t, step), U - 1) + 16u * (t & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mr = min(m0 + pf_xrow(t, i), M - 1);
    st.x[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(x) + (size_t)mr * K * 2 + xo);
  }
  load_unit<FMT>(w, nr, u, U, st.w);
  if constexpr (group_meta(FMT)) {   // the aligned 32-bit word holding each (no 16-bit loads,
    const size_t gi = (size_t)nr * U + u;       // whose partial register writes make the compiler wait for
    st.sw = reinterpret_cast<const uint32_t*>(scales)[gi >> 1];   // every load in flight); the halves
    st.zw = reinterpret_cast<const uint32_t*>(zeros)[gi >> 1];    // are taken when the stage is parked
  }
}

template <int FMT>
__device__ __forceinline__ void pf_park(const PfStage<FMT>& st, uint8_t* xs, uint8_t* ws, int n0, int N, int step, int U,
                                        int r, int h) {
  const bool unit_ok = 2 * step + h < U;   // this thread's weight unit
  const int t = threadIdx.x;
  const bool xunit_ok = pf_xunit(t, step) < U;
  uint16_t sb = 0, zb = 0;
  if constexpr (group_meta(FMT)) {   // the unit's half of each metadata word
    const int sh = 16 * (int)(((size_t)min(n0 + r, N - 1) * U + min(2 * step + h, U - 1)) & 1);
    sb = (uint16_t)(st.sw >> sh);
    zb = (uint16_t)(st.zw >> sh);
  }
  h2 wv[16];
  if constexpr (bf16_act(FMT)) {
    decode_bf16<FMT>(st.w, sb, zb, wv);
  } else {
    h2 zc1 = {}, zc2 = {};
    if constexpr (group_meta(FMT)) group_consts<FMT>(zb, zc1, zc2);
    decode<FMT>(st.w, zc1, zc2, wv);
    if constexpr (group_meta(FMT)) {
      const _Float16 sv = __builtin_bit_cast(_Float16, sb);
      const h2 s2 = {sv, sv};
#pragma unroll
      for (int p = 0; p < 16; ++p) wv[p] = wv[p] * s2;   // fp16((q-z)*s): one rounding of an exact product
    }
  }
  // zeroing by masks, not selects: the stores stay unconditional and branch-free, so the wait
  // before them covers only this stage's loads
  const uint32_t xm = xunit_ok ? ~0u : 0u, wm = unit_ok ? ~0u : 0u;
  // x row pf_xrow(t, i) has low bits (t >> 3) & 7 for every i; weight chunk 4h + i of row r is
  // chunk (4h ^ (r & 4)) + (i ^ (r & 3)) after the swizzle

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 xv = st.x[i];
    *reinterpret_cast<uint4*>(xs + pf_off<FMT, false>(pf_xrow(t, i), t & 7)) =
        make_uint4(xv.x & xm, xv.y & xm, xv.z & xm, xv.w & xm);
    *reinterpret_cast<uint4*>(ws + pf_off<FMT, true>(r, 4 * h + i)) =
        make_uint4(as_u32(wv[4 * i]) & wm, as_u32(wv[4 * i + 1]) & wm, as_u32(wv[4 * i + 2]) & wm,
                   as_u32(wv[4 * i + 3]) & wm);
  }
}

// One 128 x 128 tile of y: tile b of the linear's grid.
template <int FMT>
__device__ __forceinline__ void pf_tile(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                        const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
                                        uint16_t* __restrict__ y, int M, int N, int K, int b) {
  extern __shared__ uint4 pf_lds[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(pf_lds);
  // Tiles in chunks of 8 weight-row tiles: every x-row tile of one weight tile gets the same
  // block id modulo 8, i.e. the same XCD, so the weight tile's bytes are shared through its L2.
  const int tiles_m = (M + PF_BM - 1) / PF_BM, tiles_n = (N + PF_BN - 1) / PF_BN;
  const int chunk = b / (8 * tiles_m), rem = b - chunk * 8 * tiles_m;
  const int nx = min(8, tiles_n - 8 * chunk);
  const int mt = rem / nx, nt = 8 * chunk + rem % nx;
  const int m0 = mt * PF_BM, n0 = nt * PF_BN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), wm = wave >> 1, wn = wave & 1;
  const int r = t >> 1, h = t & 1;
  const int i16 = lane & 15, q = lane >> 4;
  const int U = K >> 5, steps = ((U + 3) >> 2) << 1;   // an even count: an odd last step multiplies zeros
  f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // Two register stages, no branches around loads or parks (past the last step they reread
  // the last unit and park into the idle buffer), so the wait before each park covers only the
  // older stage: while step s is multiplied, steps s+1 and s+2 are in flight.
  PfStage<FMT> R0, R1;
  pf_load<FMT>(R0, x, w, scales, zeros, m0, n0, M, N, K, 0, r, h);
  pf_load<FMT>(R1, x, w, scales, zeros, m0, n0, M, N, K, 1, r, h);
  constexpr int BUF = pf_buf_bytes<FMT>(), XT = pf_x_bytes<FMT>();
  pf_park<FMT>(R0, lds, lds + XT, n0, N, 0, U, r, h);
  pf_load<FMT>(R0, x, w, scales, zeros, m0, n0, M, N, K, 2, r, h);
  __syncthreads();
  auto mul = [&](int s) {
    const uint8_t* xs = lds + (s & 1) * BUF;
    const uint8_t* ws = xs + XT;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {   // the two units of the step; lane quad q takes K 8q .. 8q+7 of each
      h8 a[4], bf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        a[mi] = *reinterpret_cast<const h8*>(xs + pf_off<FMT, false>(64 * wm + 16 * mi + i16, 4 * kh + q));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bf[ni] = *reinterpret_cast<const h8*>(ws + pf_off<FMT, true>(64 * wn + 16 * ni + i16, 4 * kh + q));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16<FMT>(a[mi], bf[ni], acc[mi][ni]);
    }
  };
  for (int s = 0; s < steps; s += 2) {   // R1 holds step s+1, R0 step s+2
    mul(s);
    pf_park<FMT>(R1, lds + ((s + 1) & 1) * BUF, lds + ((s + 1) & 1) * BUF + XT, n0, N, s + 1, U, r, h);
    pf_load<FMT>(R1, x, w, scales, zeros, m0, n0, M, N, K, s + 3, r, h);
    __syncthreads();
    mul(s + 1);
    pf_park<FMT>(R0, lds + (s & 1) * BUF, lds + (s & 1) * BUF + XT, n0, N, s + 2, U, r, h);
    pf_load<FMT>(R0, x, w, scales, zeros, m0, n0, M, N, K, s + 4, r, h);
    __syncthreads();
  }
  // D[m][n] of a 16 x 16 tile sits in lane (n + 16 (m / 4)), register m % 4
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = n0 + 64 * wn + 16 * ni + i16;
    if (n >= N) continue;
    const float sc = row_scaled<FMT>() ? f16_to_f32(scales[n]) * code_scale<FMT>() : 1.0f;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m = m0 + 64 * wm + 16 * mi + 4 * q + k;
        if (m < M) y[(size_t)m * N + n] = out16<FMT>(acc[mi][ni][k] * sc);
      }
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 2) void pf_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ zeros, uint16_t* __restrict__ y, int M,
                                                    int N, int K) {
  pf_tile<FMT>(x, w, scales, zeros, y, M, N, K, blockIdx.x);
}

// Several linears of one format at the same M in one launch: the grid is the concatenation of
// their tiles (items with the longest K first, so the longest tiles start first).
constexpr int PF_MAX_GROUP = 16;
struct PfGroup {
  int count;
  int first_tile[PF_MAX_GROUP + 1];   // prefix sums of the per-linear tile counts
  const uint16_t* x[PF_MAX_GROUP];
  const uint8_t* w[PF_MAX_GROUP];
  const uint16_t* scales[PF_MAX_GROUP];
  const uint16_t* zeros[PF_MAX_GROUP];
  uint16_t* y[PF_MAX_GROUP];
  int N[PF_MAX_GROUP], K[PF_MAX_GROUP];
};

template <int FMT>
__global__ __launch_bounds__(256, 2) void pf_grouped_kernel(const PfGroup g, int M) {
  int j = 0;
  while (j + 1 < g.count && (int)blockIdx.x >= g.first_tile[j + 1]) ++j;   // workgroup-uniform
  pf_tile<FMT>(g.x[j], g.w[j], g.scales[j], g.zeros[j], g.y[j], M, g.N[j], g.K[j], blockIdx.x - g.first_tile[j]);
}

int64_t pf_tiles(int64_t M, int64_t N) { return ((M + PF_BM - 1) / PF_BM) * ((N + PF_BN - 1) / PF_BN); }

template <int FMT>
hipError_t launch_pf(hipStream_t s, const uint16_t* x, const uint8_t* w, const uint16_t* sc, const uint16_t* z,
                     uint16_t* y, int M, int N, int K) {
  return launch(pf_kernel<FMT>, dim3((unsigned)pf_tiles(M, N)), dim3(256), pf_lds_bytes<FMT>(), s, x, w, sc, z, y, M, N,
                K);
}

template <int FMT>
hipError_t launch_pf_grouped(hipStream_t s, const PfGroup& g, int M) {
  return launch(pf_grouped_kernel<FMT>, dim3((unsigned)g.first_tile[g.count]), dim3(256), pf_lds_bytes<FMT>(), s, g, M);
}

}  // namespace

namespace wq {

// The tiled kernel's time is about its longest chain of K steps (one per 64 K) while its tiles
// fit the CUs, else its tile-steps over the CUs; the decode kernels cost about one weight
// stream per 64 rows of x (W4, W6, FP4, FP5) or per 16 rows (W8, fp16 and bf16 weights). Which one
// runs below 193 rows (from 193 always the tiled kernel) was fitted to crossovers measured on
// the Llama-7B and 70B shapes at M = 20..192:
//  * W8, fp16/bf16 weights, from 17 rows: the tiled kernel when max(chain, tile-steps / 256)
//    times 1.58 (W8) or 2.1 (16-bit) us is at most the 16-row launches' weight megabytes;
//  * W4, W6, FP4, from 65 rows, and FP5 from 81 (its tiled kernel is the slowest of the 4- to
//    6-bit ones; on the 7B linears it took 154 / 156 / 158 us at 65 / 96 / 128 rows, the
//    decode kernels' 64-row slabs 130 / 174 / 216 us): when the chain is at most 2x (W4, the
//    heaviest decode) or 4x the tile count. (Past 64 rows a group that the tiled kernel does
//    not take runs one call per linear, so the tiles of all its linears count.)
// So the down projections (K = 11008, 28672; 32 to 128 tiles) keep the decode kernels.
bool pf_takes(int code, int64_t M, const int64_t* N, const int64_t* K, int count) {
  const int w = pfmt(code);
  const bool rows16 = w == WQ_FMT_F16 || w == WQ_FMT_W8;
  if (M < (rows16 ? 17 : w == WQ_FMT_W5E2M2 ? PF_MIN_M_ANY + 16 : PF_MIN_M_ANY) || M > INT32_MAX) return false;
  int64_t tiles = 0, kmax = 0, tile_steps = 0;
  double mbytes = 0.0;
  for (int i = 0; i < count; ++i) {
    const int64_t t = pf_tiles(M, N[i]);
    tiles += t;
    tile_steps += t * ((K[i] + 63) / 64);
    mbytes += (double)N[i] * (double)K[i] * (w == WQ_FMT_F16 ? 2.0 : 1.0) * 1e-6;
    kmax = K[i] > kmax ? K[i] : kmax;
  }
  if (tiles > INT32_MAX) return false;
  if (M >= PF_MIN_M) return true;
  const int64_t chain = (kmax + 63) / 64;
  if (rows16) {
    const double steps = chain > tile_steps / 256.0 ? (double)chain : tile_steps / 256.0;
    return steps * (w == WQ_FMT_F16 ? 2.1 : 1.58) <= (double)((M + 15) / 16) * mbytes;
  }
  return chain <= (group_meta(w) ? 2 : 4) * tiles;
}

int pf_launch(int code, const uint16_t* x, const void* packed_w, const uint16_t* scales, const uint16_t* zeros,
              uint16_t* y, int64_t M, int64_t N, int64_t K, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* w = static_cast<const uint8_t*>(packed_w);
  hipError_t e = hipSuccess;
  switch (code) {
#define WQ_CASE(C) case C: e = launch_pf<C>(s, x, w, scales, zeros, y, (int)M, (int)N, (int)K); break;
    WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
    default: return WQ_ERR_FMT;
  }
  return device_status(e);
}

int pf_launch_grouped(int code, const wq_linear_item* items, int count, int64_t M, void* stream) {
  if (count < 1 || count > PF_MAX_GROUP) return WQ_ERR_ARG;
  int order[PF_MAX_GROUP];
  for (int i = 0; i < count; ++i) order[i] = i;
  for (int i = 1; i < count; ++i)   // stable, by K descending
    for (int j = i; j > 0 && items[order[j]].K > items[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
  PfGroup g = {};
  g.count = count;
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    const wq_linear_item& it = items[order[i]];
    g.first_tile[i] = (int)tiles;
    g.x[i] = it.x;
    g.w[i] = static_cast<const uint8_t*>(it.packed_w);
    g.scales[i] = it.scales;
    g.zeros[i] = it.zeros;
    g.y[i] = it.y;
    g.N[i] = (int)it.N;
    g.K[i] = (int)it.K;
    tiles += pf_tiles(M, it.N);
    if (tiles > INT32_MAX) return WQ_ERR_SHAPE;
  }
  g.first_tile[count] = (int)tiles;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  switch (code) {
#define WQ_CASE(C) case C: e = launch_pf_grouped<C>(s, g, (int)M); break;
    WQ_KERNEL_CODES(WQ_CASE)
#undef WQ_CASE
    default: return WQ_ERR_FMT;
  }
  return device_status(e);
}

}  // namespace wq
