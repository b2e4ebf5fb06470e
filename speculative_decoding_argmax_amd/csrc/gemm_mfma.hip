// Skinny GEMM + per-row argmax on the matrix cores (many hidden rows).
//
// When a call scores tens or hundreds of hidden rows against the same table
// rows, each weight byte feeds that many multiply-adds and the dot products
// become a real contraction: v_mfma_f32_16x16x32_bf16 computes a 16 x 16 tile
// of logits from 16 table rows x 32 columns (operand A, streamed from HBM) and
// 16 hidden rows x 32 columns (operand B).
//
// Layout of one 16x16x32 step, lane l = j + 16 g (j < 16, g < 4):
//   A: table row (v0 + j), columns [8g, 8g + 8) of the 32-column step: one
//      16-byte load, so a load instruction reads 64 contiguous bytes of each
//      of 16 rows;
//   B: hidden row (m0 + j), the same columns, read from LDS;
//   D: logits of table rows v0 + 4g + {0,1,2,3} for hidden row m0 + j.
//
// A workgroup (4 waves) owns tiles of 4 * RW * 16 table rows, grid-strided over
// the table; each wave owns RW row blocks of 16 and all NB column blocks of 16
// hidden rows. The hidden rows are staged into LDS one K chunk (KS steps of 32
// columns) at a time, double buffered, in fragment order (the 64 lanes' B
// operands of one step stored contiguously, so each B read is one
// conflict-free ds_read_b128). Each wave's weight loads run PFD chunks ahead
// of its MFMAs through a register ring, so that much of its stream is always in
// flight. Each lane tracks, per column block, the best (logit, row) of its
// hidden row over the rows it saw; the workgroup then merges lanes and waves
// through LDS and finish_rows merges workgroups.
//
// Every logit sums its columns in the same order (K chunks ascending, 32-column
// steps ascending, the MFMA's fixed in-step order), whatever the row's tile or
// position, so duplicated rows score bit-identically and ties go to the lower
// row.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mtp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 256;
constexpr int kMfmaWaves = kMfmaThreads / kWave;

__device__ __forceinline__ uint4 load_nt16(const uint4 *p) {
  const u32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ bool better32(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

// NB: column blocks of 16 hidden rows; RW: 16-row blocks of the table per wave;
// KS: 32-column steps per K chunk; PFD: how many chunks ahead each wave's
// weight fragments are loaded.
template <int NB, int RW, int KS, int PFD>
__global__ void __launch_bounds__(kMfmaThreads)
    gemm_argmax_mfma(const uint4 *__restrict__ X, const uint4 *__restrict__ W, int M, int N,
                     int nch, RowSink sink) {
  constexpr int CPR = KS * 4;                  // 16-byte chunks of a row per K chunk
  constexpr int TILE = kMfmaWaves * RW * 16;   // table rows per workgroup tile
  constexpr int SLOTS = KS * NB * kWave;       // 16-byte B fragments per K chunk
  constexpr int SPT = (SLOTS + kMfmaThreads - 1) / kMfmaThreads;
  __shared__ uint4 xs[2][SLOTS];               // hidden chunk, fragment order
  __shared__ float f_val[NB * 16];
  __shared__ int64_t f_row[NB * 16];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int m0 = blockIdx.y * NB * 16;
  const int nchunks = (nch + CPR - 1) / CPR;
  const int ntiles = (N + TILE - 1) / TILE;
  const int my_tiles = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int total = my_tiles * nchunks;

  // Hidden staging. Slot (s, nb, l) of a chunk holds the B operand of lane l
  // for step s and column block nb: hidden row m0 + 16 nb + (l % 16), 16-byte
  // column c*CPR + 4 s + l / 16. Thread t owns slots t, t + 256, ... so the LDS
  // writes are contiguous. Rows past M and columns past the row end read a
  // clamped, valid address: extra hidden columns are never reported, and past
  // the row end the matching weights are zero.
  uint4 st[SPT];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int slot = tid + kMfmaThreads * k;
      if (SLOTS % kMfmaThreads == 0 || slot < SLOTS) {
        const int f = slot / kWave;
        const int l = slot % kWave;
        const int s = f / NB;
        const int nb = f - s * NB;
        const int m = min(m0 + nb * 16 + (l & 15), M - 1);
        const int col = min(c * CPR + 4 * s + (l >> 4), nch - 1);
        st[k] = X[(int64_t)m * nch + col];
      }
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int slot = tid + kMfmaThreads * k;
      if (SLOTS % kMfmaThreads == 0 || slot < SLOTS) xs[buf][slot] = st[k];
    }
  };

  // Weight fragments of iteration `it` (tile it / nchunks, chunk it % nchunks).
  auto load_a = [&](uint4 (&a)[KS][RW], int it) {
    const int tile = blockIdx.x + (it / nchunks) * gridDim.x;
    const int c = it % nchunks;
    const int vbase = tile * TILE + wave * RW * 16 + j;
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) {
      const int v = vbase + rw * 16;
      const uint4 *row = W + (int64_t)v * nch + c * CPR + g;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bool ok = v < N && c * CPR + 4 * s + g < nch;
        a[s][rw] = ok ? load_nt16(row + 4 * s) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  f32x4_t acc[RW][NB];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rw][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float bv[NB];
  int bi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = 0.f;
    bi[nb] = -1;
  }

  // Weight fragments rotate through a ring of PFD + 1 register sets: set
  // it % NSLOT holds iteration it, and the loads for iteration it + PFD go into
  // the set freed by iteration it - 1. The loop is unrolled by NSLOT so every
  // set index is a compile-time constant (no register copies, which would make
  // the wave wait for loads it has only just issued).
  constexpr int NSLOT = PFD + 1;
  uint4 a[NSLOT][KS][RW];
  if (total > 0) {
    stage_load(0);
    stage_store(0);
#pragma unroll
    for (int p = 0; p < PFD; ++p)
      if (p < total) load_a(a[p], p);
  }
  __syncthreads();

  auto body = [&](auto slot_tag, int it) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr int LOAD_SLOT = (SLOT + PFD) % NSLOT;
    const int buf = it & 1;
    const int c = it % nchunks;
    if (it + 1 < total) stage_load((it + 1) % nchunks);
    if (it + PFD < total) load_a(a[LOAD_SLOT], it + PFD);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 b = xs[buf][(s * NB + nb) * kWave + lane];
#pragma unroll
        for (int rw = 0; rw < RW; ++rw) acc[rw][nb] = mfma16(a[SLOT][s][rw], b, acc[rw][nb]);
      }
    }
    if (c == nchunks - 1) {
      const int tile = blockIdx.x + (it / nchunks) * gridDim.x;
      const int vbase = tile * TILE + wave * RW * 16 + 4 * g;
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = vbase + rw * 16 + r;
            const float z = acc[rw][nb][r];
            if (v < N && better32(z, v, bv[nb], bi[nb])) {
              bv[nb] = z;
              bi[nb] = v;
            }
          }
          acc[rw][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (it + 1 < total) stage_store(buf ^ 1);
    __syncthreads();
  };

  for (int it = 0; it < total; it += NSLOT) {
    body(std::integral_constant<int, 0>{}, it);
    if constexpr (NSLOT > 1) {
      if (it + 1 < total) body(std::integral_constant<int, 1 % NSLOT>{}, it + 1);
    }
    if constexpr (NSLOT > 2) {
      if (it + 2 < total) body(std::integral_constant<int, 2 % NSLOT>{}, it + 2);
    }
    if constexpr (NSLOT > 3) {
      if (it + 3 < total) body(std::integral_constant<int, 3 % NSLOT>{}, it + 3);
    }
  }
  static_assert(NSLOT <= 4, "ring of at most four weight sets");

  // Merge the 16 candidates of each hidden row (4 lane groups x 4 waves).
  // The staging buffer is free now: reuse it for the candidates.
  float *red_v = reinterpret_cast<float *>(&xs[0][0]);
  int *red_i = reinterpret_cast<int *>(red_v + kMfmaWaves * NB * kWave);
  static_assert(sizeof(xs) >= (size_t)kMfmaWaves * NB * kWave * 8, "reduction scratch");
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    red_v[(wave * NB + nb) * kWave + lane] = bv[nb];
    red_i[(wave * NB + nb) * kWave + lane] = bi[nb];
  }
  __syncthreads();
  if (tid < NB * 16) {
    const int nb = tid >> 4;
    const int jj = tid & 15;
    float v = 0.f;
    int ix = -1;
    for (int w = 0; w < kMfmaWaves; ++w) {
      for (int gg = 0; gg < 4; ++gg) {
        const int o = (w * NB + nb) * kWave + jj + 16 * gg;
        if (red_i[o] >= 0 && better32(red_v[o], red_i[o], v, ix)) {
          v = red_v[o];
          ix = red_i[o];
        }
      }
    }
    f_val[tid] = v;
    f_row[tid] = ix;
  }
  __syncthreads();
  const int mcount = M - m0 < NB * 16 ? M - m0 : NB * 16;
  finish_rows(sink, f_val, f_row, m0, mcount);
}

// Column blocks with an instantiation; M rounds up to the next (up to 160 rows
// per pass; more rows take several passes over the table).
static const int kNbSteps[] = {1, 2, 3, 4, 6, 8, 10};

int mfma_nb_for(int M) {
  const int need = (M + 15) / 16;
  for (int n : kNbSteps)
    if (n >= need) return n;
  return 10;
}

template <int NB, int RW, int KS, int PFD>
static hipError_t launch_nb(const MfmaLaunch &L) {
  constexpr int TILE = kMfmaWaves * RW * 16;
  const int64_t ntiles = (L.N + TILE - 1) / TILE;
  const int gx = (int)(ntiles < L.max_blocks_x ? ntiles : L.max_blocks_x);
  const int gy = (L.M + NB * 16 - 1) / (NB * 16);
  return launch_call_kernel((gemm_argmax_mfma<NB, RW, KS, PFD>), dim3(gx, gy),
                            dim3(kMfmaThreads), L.stream, true, true, (const uint4 *)L.X,
                            (const uint4 *)L.W, L.M, (int)L.N, L.nch, L.sink);
}

// Instantiated shapes (measured on MI355X; none spills registers).
hipError_t launch_mfma(const MfmaLaunch &L, int nb) {
  switch (nb) {
    case 1: return launch_nb<1, 2, 4, 1>(L);
    case 2: return launch_nb<2, 4, 4, 2>(L);
    case 3: return launch_nb<3, 2, 4, 2>(L);
    case 4: return launch_nb<4, 2, 4, 2>(L);
    case 6: return launch_nb<6, 2, 4, 2>(L);
    case 8: return launch_nb<8, 2, 4, 2>(L);
    case 10: return launch_nb<10, 4, 2, 3>(L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
