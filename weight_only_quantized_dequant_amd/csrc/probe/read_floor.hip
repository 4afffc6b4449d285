// Plain-read probe (measurement only, not part of libwq's interface): how fast a kernel that
// does nothing but stream a buffer from HBM reads it on this GPU. The gpt-fast write-up
// (m.greenbasetech.com) treats decode as bound by memory bandwidth; the rate a bare read
// reaches for a given byte count is the practical ceiling of a weight-streaming kernel of
// that size, so the benchmark reports it beside the 8 TB/s peak.
//
// Each wave reads one contiguous span of the buffer with UNR 16-byte loads in flight per lane
// (a wave instruction reads 1 KB contiguous) and folds the words into one value, which is
// stored only when it equals a constant, so that the loads cannot be dropped. Built into its
// own library (libwq_probe.so), loaded by bench.py only.

#include <hip/hip_runtime.h>
#include <cstdint>

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

namespace {

template <int UNR>
__global__ __launch_bounds__(256) void read_span_kernel(const probe_u32x4* __restrict__ p, uint64_t n16,
                                                        uint64_t per16, uint32_t* __restrict__ sink) {
  const uint64_t wave = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t b = wave * per16;
  const uint64_t e = b + per16 < n16 ? b + per16 : n16;
  uint32_t acc = 0;
  uint64_t i = b + lane;
  for (; i + (UNR - 1) * 64 < e; i += UNR * 64) {   // all UNR loads of the step lie below e
    probe_u32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 64);
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < e; i += 64) {
    const probe_u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// A kernel that does nothing: launched back to back, what every launch costs whatever its work.
__global__ __launch_bounds__(256) void empty_kernel(uint32_t* __restrict__ sink, uint32_t never) {
  if (threadIdx.x == never) sink[0] = never;   // never == 0xFFFFFFFF: no thread stores
}

}  // namespace

extern "C" {

// Launch `workgroups` workgroups of 256 threads of a kernel that does nothing (sink: any device
// buffer of 4 bytes or more, never written). Returns 0, -1 for bad arguments (nothing launched),
// or the HIP error code of the launch.
int wq_probe_empty(int workgroups, uint32_t* sink, void* stream) {
  if (!sink || workgroups < 1) return -1;
  uint32_t never = 0xFFFFFFFFu;
  void* args[] = {&sink, &never};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(empty_kernel), dim3(workgroups), dim3(256), args, 0,
                              static_cast<hipStream_t>(stream));
}

// Read `bytes` (a multiple of 16) of the device buffer `buf` (16-byte aligned) with `waves`
// waves (a multiple of 4) and `unroll` (2 or 4) loads in flight per lane. `sink` is a device
// buffer of at least waves / 4 words that the kernel may write. Returns 0, or -1 for bad
// arguments (nothing launched), or the HIP error code of the launch.
int wq_probe_read(const void* buf, int64_t bytes, int waves, int unroll, uint32_t* sink, int64_t sink_words,
                  void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 || waves < 4 || waves % 4 || waves / 4 > sink_words ||
      (unroll != 2 && unroll != 4) || reinterpret_cast<uintptr_t>(buf) % 16)
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16, per16 = (n16 + waves - 1) / waves;
  const dim3 grid(waves / 4), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const probe_u32x4* p = static_cast<const probe_u32x4*>(buf);
  void* args[] = {&p, const_cast<uint64_t*>(&n16), const_cast<uint64_t*>(&per16), &sink};
  const void* k = unroll == 2 ? reinterpret_cast<const void*>(read_span_kernel<2>)
                              : reinterpret_cast<const void*>(read_span_kernel<4>);
  return (int)hipLaunchKernel(k, grid, block, args, 0, s);   // the launch's own status
}

}  // extern "C"
