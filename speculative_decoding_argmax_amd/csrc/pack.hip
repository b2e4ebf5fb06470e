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
