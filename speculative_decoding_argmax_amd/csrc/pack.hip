// One-time set-up kernels: candidate sub-table packing and workspace clearing.

#include "launch.hpp"

namespace mtp {

// table[i][:] = head[ids[i]][:], one 16-byte chunk per thread per step; a row
// whose id falls outside [0, V) is written as zeros instead of read.
__global__ void __launch_bounds__(256)
    pack_rows(const uint4 *__restrict__ head, int64_t V, int nch, const int32_t *__restrict__ ids,
              int64_t C, uint4 *__restrict__ table) {
  const int64_t total = C * nch;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
    const int64_t row = e / nch;
    const int64_t c = e - row * nch;
    const int64_t id = ids[row];
    table[e] = (id >= 0 && id < V) ? head[id * nch + c] : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Tiled layout (see gemm_dma.hip): output 16-byte element o is lane o % 64 of
// fragment f = o / 64 = (t * S + s) * 4 + rb, i.e. source row
// 64 t + 16 rb + (lane % 16) (ids[row] if ids is given), 16-byte column
// 4 s + lane / 16. Rows past C, columns past the row end and out-of-range ids
// are zero.
__global__ void __launch_bounds__(256)
    pack_tiled(const uint4 *__restrict__ head, int64_t V, int nch, const int32_t *__restrict__ ids,
               int64_t C, int S, uint4 *__restrict__ tiled, int64_t total) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total; o += step) {
    const int lane = (int)(o & 63);
    const int64_t f = o >> 6;
    const int rb = (int)(f & 3);
    const int64_t ts = f >> 2;
    const int64_t t = ts / S;
    const int s = (int)(ts - t * S);
    const int64_t row = t * 64 + rb * 16 + (lane & 15);
    const int col = 4 * s + (lane >> 4);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < C && col < nch) {
      const int64_t id = ids ? (int64_t)ids[row] : row;
      if (id >= 0 && id < V) v = head[id * nch + col];
    }
    tiled[o] = v;
  }
}

__global__ void __launch_bounds__(256) fill_zero_u64(unsigned long long *p, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += step) p[e] = 0ull;
}

hipError_t launch_pack(const void *head, int64_t V, int nch, const int32_t *ids, int64_t C,
                       void *table, int num_cus, hipStream_t stream) {
  const int64_t total = C * nch;
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_rows, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4 *)head,
                     V, nch, ids, C, (uint4 *)table);
  return hipGetLastError();
}

hipError_t launch_pack_tiled(const void *head, int64_t V, int nch, const int32_t *ids,
                             int64_t C, int S, void *tiled, int num_cus, hipStream_t stream) {
  const int64_t total = tiled_rows(C) / 64 * S * 4 * 64;
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_tiled, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4 *)head, V, nch, ids, C, S, (uint4 *)tiled, total);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_u64, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (unsigned long long *)ws, n);
  return hipGetLastError();
}

}  // namespace mtp
