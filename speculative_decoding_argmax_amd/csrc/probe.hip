// Streaming-read reference: one plain read of a buffer, the practical ceiling
// that the HBM-bound draft and verify calls are compared with (the published
// 8 TB/s is a signalling rate; a real read stream reaches less).

#include "launch.hpp"

namespace mtp {

typedef unsigned int u32x4_probe_t __attribute__((ext_vector_type(4)));

// Each wave reads LOADS KiB at a time, contiguous (lane l takes the l-th
// 16-byte element of each KiB), with non-temporal loads; waves step through
// the buffer grid-strided. Each wave XORs what it read into one sink word
// (its global wave index), so the loads cannot be dropped. On MI355X, 4 KiB
// per wave and 2 workgroups per CU read 6.86 TB/s over 268 MB and 6.92 TB/s
// over 1 GB (a sweep of 4-16 KiB and 2-16 workgroups per CU); a grid-stride
// pattern with the loads of one thread 8 MB apart reached only 4.6-5.7 TB/s.
template <int LOADS>
__global__ void __launch_bounds__(256)
    stream_read(const u32x4_probe_t *__restrict__ p, int64_t n, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t step = (int64_t)gridDim.x * 4 * LOADS * kWave;
  u32x4_probe_t acc = {0u, 0u, 0u, 0u};
  for (int64_t base = gw * LOADS * kWave; base < n; base += step) {
    if (base + LOADS * kWave <= n) {
      u32x4_probe_t v[LOADS];
#pragma unroll
      for (int i = 0; i < LOADS; ++i) v[i] = __builtin_nontemporal_load(p + base + i * kWave + lane);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) acc ^= v[i];
    } else {
      for (int i = 0; i < LOADS; ++i) {
        const int64_t e = base + i * kWave + lane;
        if (e < n) acc ^= __builtin_nontemporal_load(p + e);
      }
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d, kWave);
  if (lane == 0) sink[gw] = x;
}

// Atomic round-trip reference: the latency of one dependent agent-scope
// atomic, the step that the cross-workgroup finish of every call repeats
// three or four times at the call's end. Lane 0 of workgroup b runs a chain
// of `iters` fetch-and-adds on word 64 b (or word 0 when `same`), each
// address taken from the previous return (always the same word, but the
// compiler cannot know it), so every atomic waits for the one before. The
// chain's duration in ticks of the 100 MHz real-time counter goes to
// ticks[b].
__global__ void __launch_bounds__(64)
    atomic_chain(uint32_t *words, int iters, int same, unsigned long long *ticks) {
  if (threadIdx.x != 0) return;
  uint32_t *w = words + (same ? 0 : 64 * (int64_t)blockIdx.x);
  uint32_t v = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i)
    v = __hip_atomic_fetch_add(&w[(v >> 31) & 1u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the last return must have arrived before the clock is read
  asm volatile("" : : "v"(v) : "memory");
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  ticks[blockIdx.x] = (t1 - t0) | ((unsigned long long)(v >> 31) << 63);  // v keeps the chain live
}

hipError_t launch_atomic_chain(uint32_t *words, int wgs, int iters, int same,
                               unsigned long long *ticks, hipStream_t stream) {
  hipLaunchKernelGGL(atomic_chain, dim3(wgs), dim3(64), 0, stream, words, iters, same, ticks);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int cus,
                              hipStream_t stream) {
  // two 4-wave workgroups per CU, at most one sink word per wave
  int blocks = 2 * cus;
  if (blocks > kStreamSinkWords / 4) blocks = kStreamSinkWords / 4;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_read<4>, dim3(blocks), dim3(256), 0, stream,
                     (const u32x4_probe_t *)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace mtp
