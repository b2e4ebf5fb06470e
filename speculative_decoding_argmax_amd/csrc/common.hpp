// Device-side building blocks shared by the draft / verify kernels (gfx950).
//
//  * bf16 dot products on v_dot2c_f32_bf16 (two bf16 products + fp32 add),
//  * wave64 sums on DPP and lane reads (every lane ends with the same,
//    bit-identical total),
//  * the (score, row) order used by every argmax: larger score first, equal
//    scores to the lower row (rows are ascending in token id, so the lower
//    row is the lower id), packed into one 64-bit key so a single unsigned
//    atomic max merges workgroups,
//  * the cross-workgroup finish: each workgroup merges its per-row winners
//    into the workspace keys, and the last workgroup to arrive (ticket)
//    decodes them, writes the outputs, runs greedy acceptance for verify,
//    and clears the workspace for the next call. Launches whose workgroups
//    reach the finish together spread its keys and counters over
//    kFinishGroups regions of the workspace (grouped finish).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Workspace layout: [0, 256) ticket (uint32 at offset 0), then one 64-bit key
// per hidden row. The grouped finish uses instead kFinishGroups regions of
// finish_group_stride(M) bytes from offset kWsHeader on: region g holds group
// g's counter (uint32 at its offset 0) and, from offset 64, its M keys.
constexpr size_t kWsHeader = 256;
constexpr int kFinishGroups = 8;

// Bytes per group region: the counter's 64 bytes and M keys, rounded up to
// 256 so that every group's counter and keys lie in lines of their own.
__host__ __device__ constexpr size_t finish_group_stride(int64_t M) {
  return ((64 + (size_t)M * 8 + 255) / 256) * 256;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// acc + sum of the 8 products of two 16-byte bf16 chunks, in element order.
__device__ __forceinline__ float dot8_bf16(const uint4 &w, const uint4 &h, float acc) {
  acc = dot2_bf16(w.x, h.x, acc);
  acc = dot2_bf16(w.y, h.y, acc);
  acc = dot2_bf16(w.z, h.z, acc);
  acc = dot2_bf16(w.w, h.w, acc);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane returns the same bits. Within each 16-lane
// row a DPP butterfly leaves the row's sum in all its lanes; the four row sums
// are then read out (v_readlane) and added as (r0 + r1) + (r2 + r3). The
// pairing never changes, so identical inputs give identical totals.
// (The gfx950 permlane16/32 swaps are not used here: with both operands the
// same value, the compiler folds the two swap results into one.)
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f32<0x141>(v);  // row_half_mirror: quad 0 <-> quad 1 of each 8
  v += dpp_f32<0x140>(v);  // row_mirror: half 0 <-> half 1 of each 16
  const int u = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
  return (r0 + r1) + (r2 + r3);
}

// True if (v, i) beats (bv, bi): larger score, or equal score and lower row.
// bi < 0 marks "no candidate yet".
__device__ __forceinline__ bool better(float v, int64_t i, float bv, int64_t bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

// Monotone map of a finite float to uint32 (-0.0 folded onto +0.0).
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unorder_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, u);
}

// Key: score order in the high word, complemented row in the low word, so the
// unsigned maximum is the best (score, lowest row). 0 means "empty".
__device__ __forceinline__ unsigned long long make_key(float v, uint32_t row) {
  return ((unsigned long long)order_bits(v) << 32) | (unsigned long long)(~row);
}

// A kernel argument of every row kernel: its size is kept at 80 bytes (the
// group count sits in the padding after k), since some kernels already use
// every scalar register and a larger argument made the compiler reload
// arguments and drain the loads in flight inside their main loop.
struct RowSink {
  uint32_t *ticket;          // workspace + 0
  unsigned long long *keys;  // workspace + kWsHeader, one per hidden row
  const int32_t *ids;        // row -> token id, or nullptr for identity
  int32_t *out_ids;          // [M]
  float *out_logit;          // [M] or nullptr
  int M;
  // verify only (k < 0 for draft)
  int B, k;
  int groups;                // 1, or kFinishGroups for the grouped finish
  const int32_t *draft;      // [B][k]
  int32_t *out_accept;       // [B]
  int32_t *out_tokens;       // [B][k+1]
};
static_assert(sizeof(RowSink) == 80, "kept at 80 bytes (see above)");

// The last workgroup, once every key is final: hidden row m's id and logit
// from its key (0: no candidate seen, id -1 and NaN).
__device__ __forceinline__ void finish_outputs(const RowSink &s, int m,
                                               unsigned long long key) {
  int32_t id = -1;
  float val = __builtin_nanf("");
  if (key != 0ull) {
    const uint32_t row = ~(uint32_t)(key & 0xFFFFFFFFull);
    val = unorder_bits((uint32_t)(key >> 32));
    id = s.ids ? s.ids[row] : (int32_t)row;
  }
  s.out_ids[m] = id;
  if (s.out_logit) s.out_logit[m] = val;
}

// The last workgroup, after finish_outputs for every row: for verify, greedy
// acceptance of each sequence's drafts against the target ids just written;
// then the call's ticket goes back to zero for the next call.
__device__ __forceinline__ void finish_accept(const RowSink &s) {
  if (s.k >= 0) {
    __syncthreads();  // out_ids (the target argmax) written by this workgroup
    const int k = s.k;
    for (int b = threadIdx.x; b < s.B; b += blockDim.x) {
      const int32_t *t = s.out_ids + (int64_t)b * (k + 1);
      int n = 0;
      while (n < k && s.draft[(int64_t)b * k + n] == t[n]) ++n;
      s.out_accept[b] = n;
      for (int p = 0; p <= k; ++p) s.out_tokens[(int64_t)b * (k + 1) + p] = p <= n ? t[p] : -1;
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_exchange(s.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The grouped finish (see finish_rows). The group count is a constant, so
// the last workgroup issues its G key reads per row back to back.
__device__ __forceinline__ void finish_rows_grouped(const RowSink &s, const float *wg_val,
                                                 const int64_t *wg_row, int m_begin,
                                                 int m_count) {
  __shared__ int s_last;
  __shared__ int s_seen;
  constexpr uint32_t G = kFinishGroups;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const uint32_t bid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const uint32_t g = bid % G;
  const size_t gstride = finish_group_stride(s.M);
  char *const groups = reinterpret_cast<char *>(s.ticket) + kWsHeader;
  unsigned long long *const keys =
      reinterpret_cast<unsigned long long *>(groups + (size_t)g * gstride + 64);
  if (tid == 0) s_seen = 0;
  __syncthreads();
  for (int t = tid; t < m_count; t += nthreads) {
    if (wg_row[t] >= 0) {
      const unsigned long long key = make_key(wg_val[t], (uint32_t)wg_row[t]);
      const unsigned long long old = __hip_atomic_fetch_max(&keys[m_begin + t], key,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
      if (old >= key) s_seen = 1;  // consumes the returned value
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t nblocks = gridDim.x * gridDim.y * gridDim.z;
    uint32_t *const gt = reinterpret_cast<uint32_t *>(groups + (size_t)g * gstride);
    const uint32_t gsize = nblocks / G + (g < nblocks % G ? 1u : 0u);
    const uint32_t ngroups = nblocks < G ? nblocks : G;
    const uint32_t pg = __hip_atomic_fetch_add(gt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = 0;
    if (pg == gsize - 1) {
      // every workgroup of the group has counted: reset its counter
      __hip_atomic_exchange(gt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t prev =
          __hip_atomic_fetch_add(s.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == ngroups - 1;
    }
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  for (int m = tid; m < s.M; m += nthreads) {
    unsigned long long key = 0ull;
#pragma unroll
    for (uint32_t q = 0; q < G; ++q) {
      unsigned long long *const kq =
          reinterpret_cast<unsigned long long *>(groups + (size_t)q * gstride + 64);
      const unsigned long long v =
          __hip_atomic_exchange(&kq[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      key = v > key ? v : key;
    }
    finish_outputs(s, m, key);
  }
  finish_accept(s);
}

// Called by every thread of every workgroup after the workgroup's per-row
// winners for rows [m_begin, m_begin + m_count) sit in wg_val / wg_row
// (wg_row < 0: the workgroup saw no row). Must be reached by all threads.
//
// All cross-workgroup traffic goes through atomic read-modify-writes, which
// the hardware performs at the memory's coherence point, so no agent-scope
// fence is needed (on a multi-XCD gfx950 such a fence writes back and
// invalidates the whole L2 of the XCD, once per workgroup). Ordering: every
// key update returns its old value before the workgroup's barrier (the
// returned value feeds an LDS write), and only then does one thread take a
// ticket; the last ticket holder reads the keys with atomic exchanges, which
// also clear them for the next call.
//
// Grouped finish (s.groups > 1): workgroup b updates the keys of group
// b mod G and takes that group's ticket; the last workgroup of each group
// takes the call's ticket, and the last of those reads every group's keys.
// Same-address atomics are performed one after another, so when hundreds of
// workgroups arrive together the single ticket and key queue up; G groups in
// separate lines split the queue at the cost of one more dependent round
// trip. It is a function of its own so that the one-level path keeps its
// code (reading the grid size where it did, inside the ticket branch).
__device__ __forceinline__ void finish_rows(const RowSink &s, const float *wg_val,
                                            const int64_t *wg_row, int m_begin, int m_count) {
  if (s.groups > 1) {
    finish_rows_grouped(s, wg_val, wg_row, m_begin, m_count);
    return;
  }
  __shared__ int s_last;
  __shared__ int s_seen;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  if (tid == 0) s_seen = 0;
  __syncthreads();
  for (int t = tid; t < m_count; t += nthreads) {
    if (wg_row[t] >= 0) {
      const unsigned long long key = make_key(wg_val[t], (uint32_t)wg_row[t]);
      const unsigned long long old = __hip_atomic_fetch_max(&s.keys[m_begin + t], key,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
      if (old >= key) s_seen = 1;  // consumes the returned value
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t nblocks = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t prev =
        __hip_atomic_fetch_add(s.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == nblocks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  for (int m = tid; m < s.M; m += nthreads)
    finish_outputs(
        s, m, __hip_atomic_exchange(&s.keys[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  finish_accept(s);
}

}  // namespace mtp
