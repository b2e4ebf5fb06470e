// Row-streaming GEMV + argmax on the vector ALUs (small numbers of hidden rows).
//
// Each wave owns blocks of RB consecutive table rows, strided over all waves of
// the grid so that concurrently running waves read neighbouring memory. A row is
// split over the 64 lanes in 16-byte chunks (lane l reads chunks l, l+64, ...),
// so every load instruction of a wave reads 1 KiB of one row, fully coalesced.
// The lanes' slices of the MR hidden rows sit in registers for the whole kernel.
// Per (row, hidden row) a lane accumulates its chunks with v_dot2c_f32_bf16 in
// chunk order, then the wave sums the 64 partials (wave_sum); every lane holds
// the total, so the running (best score, best row) is wave-uniform. Waves merge
// through LDS, workgroups through the workspace keys (finish_rows).
//
// The summation order of a row's score depends only on the column index, never
// on where the row sits in the grid, so duplicated rows score bit-identically
// and ties resolve to the lower row.

#include "common.hpp"
#include "launch.hpp"

namespace mtp {

constexpr int kValuThreads = 256;
constexpr int kValuWaves = kValuThreads / kWave;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Weight rows are read exactly once per call: non-temporal loads keep them
// from displacing the hidden vector and the workspace in the caches.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Where the candidate rows live. Packed: row i of the table is candidate i.
// Gathered: candidate i is head row ids[i] (any order, repeats allowed); an
// id outside [0, V) is no candidate, and its row is never read.
struct RowSource {
  const int32_t *ids;  // gathered rows: ids[N]; nullptr for a packed table
  int64_t V;           // rows of the head (gathered rows only)
};

// Table row of candidate i (< 0: not a candidate). Packed: i itself;
// gathered: ids[i] if it names a head row.
template <bool GATHER>
__device__ __forceinline__ int32_t source_row(const RowSource &src, int64_t i) {
  if (!GATHER) return (int32_t)i;
  const int32_t id = src.ids[i];
  return (id >= 0 && id < src.V) ? id : -1;
}

// Loads RB rows x NCL chunks of this lane's slice, row i at base + i * nch.
// COLS_OK says every chunk is inside the row, so no column predication.
template <int RB, int NCL, bool COLS_OK>
__device__ __forceinline__ void load_consecutive(uint4 (&w)[RB][NCL],
                                                 const uint4 *__restrict__ base, int nch,
                                                 int lane) {
#pragma unroll
  for (int i = 0; i < RB; ++i) {
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const bool ok = COLS_OK || lane + kWave * c < nch;
      w[i][c] = ok ? load_stream(base + (int64_t)i * nch + kWave * c)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Loads the rows of candidates r0 .. r0 + RB - 1 and sets rows[i] to each
// one's table row (-1: past N or not a candidate). A full block of a packed
// table is consecutive rows addressed straight from r0. Otherwise every row
// is looked up; a non-candidate loads table row 0 instead, so no load needs
// a row predicate (the argmax skips it).
template <int RB, int NCL, bool COLS_OK, bool GATHER>
__device__ __forceinline__ void load_rows(uint4 (&w)[RB][NCL], int32_t (&rows)[RB],
                                          const uint4 *__restrict__ W, const RowSource &src,
                                          int64_t r0, int64_t N, int nch, int lane) {
  if (!GATHER && r0 + RB <= N) {
#pragma unroll
    for (int i = 0; i < RB; ++i) rows[i] = (int32_t)(r0 + i);
    load_consecutive<RB, NCL, COLS_OK>(w, W + r0 * nch + lane, nch, lane);
    return;
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    rows[i] = r0 + i < N ? source_row<GATHER>(src, r0 + i) : -1;
    const uint4 *row = W + (int64_t)(rows[i] >= 0 ? rows[i] : 0) * nch + lane;
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const bool ok = COLS_OK || lane + kWave * c < nch;
      w[i][c] = ok ? load_stream(row + kWave * c) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// MR hidden rows, NCL 16-byte chunks per lane and row, RB table rows per wave
// iteration; PF: the next iteration's rows are loaded before this one's are
// reduced; EXACT: H == NCL * 512 (no column predication).
template <int MR, int NCL, int RB, bool PF, bool EXACT, bool GATHER>
__global__ void __launch_bounds__(kValuThreads)
    gemv_argmax_valu(const uint4 *__restrict__ X, const uint4 *__restrict__ W, int M, int64_t N,
                     int nch, RowSource src, RowSink sink) {
  __shared__ float s_val[kValuWaves][MR];
  __shared__ int64_t s_row[kValuWaves][MR];
  __shared__ float f_val[MR];
  __shared__ int64_t f_row[MR];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * MR;

  uint4 h[MR][NCL];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const int col = lane + kWave * c;
      h[r][c] = (m0 + r < M && (EXACT || col < nch)) ? X[(int64_t)(m0 + r) * nch + col]
                                                     : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  float bv[MR];
  int64_t bi[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    bv[r] = 0.0f;
    bi[r] = -1;
  }

  const int64_t stride = (int64_t)gridDim.x * kValuWaves * RB;
  // wave-uniform row cursor, kept in scalar registers
  int64_t r0 = ((int64_t)blockIdx.x * kValuWaves + __builtin_amdgcn_readfirstlane(wave)) * RB;
  uint4 nxt[RB][NCL];
  int32_t rows_nxt[RB];
  if (PF && r0 < N) load_rows<RB, NCL, EXACT, GATHER>(nxt, rows_nxt, W, src, r0, N, nch, lane);
  for (; r0 < N; r0 += stride) {
    uint4 w[RB][NCL];
    int32_t rows[RB];
    if (PF) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        rows[i] = rows_nxt[i];
#pragma unroll
        for (int c = 0; c < NCL; ++c) w[i][c] = nxt[i][c];
      }
      if (r0 + stride < N)
        load_rows<RB, NCL, EXACT, GATHER>(nxt, rows_nxt, W, src, r0 + stride, N, nch, lane);
    } else {
      load_rows<RB, NCL, EXACT, GATHER>(w, rows, W, src, r0, N, nch, lane);
    }
    float acc[MR][RB];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[r][i] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCL; ++c)
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r][i] = dot8_bf16(w[i][c], h[r][c], acc[r][i]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float s = wave_sum(acc[r][i]);
        // argmax index: the position in a packed table, the id when gathered
        // (for a packed table the test is written on r0 so that it stays a
        // vector compare inside one basic block, as the scheduler needs to
        // interleave the reductions with the next row's products)
        const int64_t key = GATHER ? (int64_t)rows[i] : r0 + i;
        const bool cand = GATHER ? rows[i] >= 0 : r0 + i < N;
        if (cand && better(s, key, bv[r], bi[r])) {
          bv[r] = s;
          bi[r] = key;
        }
      }
    }
  }

  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      s_val[wave][r] = bv[r];
      s_row[wave][r] = bi[r];
    }
  }
  __syncthreads();
  if (threadIdx.x < MR) {
    const int r = threadIdx.x;
    float v = s_val[0][r];
    int64_t ix = s_row[0][r];
    for (int q = 1; q < kValuWaves; ++q) {
      if (s_row[q][r] >= 0 && better(s_val[q][r], s_row[q][r], v, ix)) {
        v = s_val[q][r];
        ix = s_row[q][r];
      }
    }
    f_val[r] = v;
    f_row[r] = ix;
  }
  __syncthreads();
  finish_rows(sink, f_val, f_row, m0, min(MR, M - m0));
}

// Two instantiated variants per (MR, NCL): RB rows per iteration with no
// prefetch (about 16 chunk loads in flight per wave), and the default: one or
// two rows per iteration with the next iteration's rows already in flight
// (measured on MI355X: 41 us for 65,536 x 2,048 and 144 us for the
// 248,320 x 2,048 verify with 4 hidden rows, at one workgroup per CU).
template <int NCL>
constexpr int valu_rb_plain() {
  return NCL >= 16 ? 1 : (16 / NCL > 4 ? 4 : 16 / NCL);
}
template <int NCL>
constexpr int valu_rb_prefetch() {
  return NCL <= 5 ? 2 : 1;
}

template <int MR, int NCL, int RB, bool PF>
static hipError_t launch_variant(const ValuLaunch &L) {
  const int64_t row_blocks = (L.N + RB - 1) / RB;
  const int64_t want = (row_blocks + kValuWaves - 1) / kValuWaves;
  const int gx = (int)(want < L.max_blocks_x ? want : L.max_blocks_x);
  const int gy = (L.M + MR - 1) / MR;
  const RowSource src{L.gather_ids, L.gather_V};
  const bool exact = L.nch == NCL * kWave;
  hipError_t e;
  if (L.gather_ids) {
    if (exact)
      e = launch_call_kernel((gemv_argmax_valu<MR, NCL, RB, PF, true, true>), dim3(gx, gy),
                             dim3(kValuThreads), L.stream, true, true, (const uint4 *)L.X, (const uint4 *)L.W,
                         L.M, L.N, L.nch, src, L.sink);
    else
      e = launch_call_kernel((gemv_argmax_valu<MR, NCL, RB, PF, false, true>), dim3(gx, gy),
                             dim3(kValuThreads), L.stream, true, true, (const uint4 *)L.X, (const uint4 *)L.W,
                         L.M, L.N, L.nch, src, L.sink);
  } else if (exact) {
    e = launch_call_kernel((gemv_argmax_valu<MR, NCL, RB, PF, true, false>), dim3(gx, gy),
                           dim3(kValuThreads), L.stream, true, true, (const uint4 *)L.X, (const uint4 *)L.W,
                       L.M, L.N, L.nch, src, L.sink);
  } else {
    e = launch_call_kernel((gemv_argmax_valu<MR, NCL, RB, PF, false, false>), dim3(gx, gy),
                           dim3(kValuThreads), L.stream, true, true, (const uint4 *)L.X, (const uint4 *)L.W,
                       L.M, L.N, L.nch, src, L.sink);
  }
  return e;
}

template <int MR, int NCL>
static hipError_t launch_mr_ncl(const ValuLaunch &L) {
  if (L.prefetch)
    return launch_variant<MR, NCL, valu_rb_prefetch<NCL>(), true>(L);
  return launch_variant<MR, NCL, valu_rb_plain<NCL>(), false>(L);
}

// Chunks per lane that have an instantiation; a request rounds up to the next.
static const int kNclSteps[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32};

int valu_ncl_for(int nch) {
  const int need = (nch + kWave - 1) / kWave;
  for (int n : kNclSteps)
    if (n >= need) return n;
  return 0;
}

int valu_rows_for(int M, int ncl) {
  // hidden slices stay in registers: MR * NCL chunks of 4 VGPRs each, <= 128 VGPRs
  int mr = 1;
  while (mr < 8 && mr < M && (2 * mr) * ncl <= 32) mr *= 2;
  return mr;
}

template <int MR>
static hipError_t dispatch_ncl(int ncl, const ValuLaunch &L) {
  switch (ncl) {
#define MTP_NCL_CASE(n) \
  case n:               \
    if constexpr (MR * n <= 32) return launch_mr_ncl<MR, n>(L); \
    break;
    MTP_NCL_CASE(1)
    MTP_NCL_CASE(2)
    MTP_NCL_CASE(3)
    MTP_NCL_CASE(4)
    MTP_NCL_CASE(5)
    MTP_NCL_CASE(6)
    MTP_NCL_CASE(8)
    MTP_NCL_CASE(10)
    MTP_NCL_CASE(12)
    MTP_NCL_CASE(16)
    MTP_NCL_CASE(20)
    MTP_NCL_CASE(24)
    MTP_NCL_CASE(32)
#undef MTP_NCL_CASE
    default:
      break;
  }
  return hipErrorInvalidValue;
}

int valu_total_blocks(const ValuLaunch &L, int mr, int ncl) {
  const int rb = L.prefetch ? (ncl <= 5 ? 2 : 1) : (ncl >= 16 ? 1 : (16 / ncl > 4 ? 4 : 16 / ncl));
  const int64_t row_blocks = (L.N + rb - 1) / rb;
  const int64_t want = (row_blocks + kValuWaves - 1) / kValuWaves;
  const int gx = (int)(want < L.max_blocks_x ? want : L.max_blocks_x);
  return gx * ((L.M + mr - 1) / mr);
}

hipError_t launch_valu(const ValuLaunch &L, int mr, int ncl) {
  switch (mr) {
    case 1: return dispatch_ncl<1>(ncl, L);
    case 2: return dispatch_ncl<2>(ncl, L);
    case 4: return dispatch_ncl<4>(ncl, L);
    case 8: return dispatch_ncl<8>(ncl, L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
