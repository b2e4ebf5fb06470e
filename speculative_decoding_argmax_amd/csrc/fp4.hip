// MXFP4 candidate table: quantising pack and the draft GEMV + argmax over it
// (mtp.h, "MXFP4 candidate table").
//
// Format: OCP microscaling MXFP4. Elements are E2M1 (sign, 2 exponent bits
// with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6); each
// block of 32 consecutive elements of a row shares one E8M0 scale 2^e (code
// e + 127), e = floor(log2(max |w| over the block)) - 2 clamped to
// [-127, 127], -127 for an all-zero block. Element j is the E2M1 value
// nearest to w[j] * 2^-e, ties to the even code, magnitudes past 6 saturating
// to 6; a negative value keeps its sign bit when it rounds to zero. Two codes
// share a byte, element 2i in the low nibble; a row is H/2 code bytes and H/32
// scale bytes.
//
// A second scale reading (fit rule, selected per pack call): the smallest e
// with max |w| <= 6 * 2^e, so that no element of the block saturates; it is
// one larger than the OCP exponent in blocks whose maximum exceeds 1.5 times
// its power of two, and the same elsewhere.
//
// The pack computes e from the bf16 bits of the block maximum and the code by
// counting the rounding midpoints below |w| * 2^-e (the ones whose tie goes
// up, at 0.75, 1.75 and 3.5, counted with >=), in fp32, where the scaling is
// exact wherever the result can reach a midpoint.
//
// The draft streams one block (16 code bytes, 32 columns) per lane and load;
// v_cvt_scalef32_pk_bf16_fp4 (scale 1.0) turns each code byte into a bf16
// pair exactly (low nibble first), v_dot2c_f32_bf16 accumulates the block
// against the hidden columns in order, and the block's partial sum is
// multiplied by its scale (a power of two: exact) and added to the row's sum.
// Rows per wave, prefetch, argmax and the cross-workgroup finish follow the
// fp8 kernel.

#include "common.hpp"
#include "launch.hpp"

namespace mtp {

typedef __bf16 bf16x2_fp4_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_fp4_t __attribute__((ext_vector_type(4)));

// ---- quantising pack ------------------------------------------------------

// Scale exponent of a block from the bf16 bits of its largest magnitude
// (0: all-zero block). With amax = sig * 2^(fl - 7), sig the 8-bit
// significand in [128, 255]: the OCP rule takes fl - 2; the fit rule takes
// fl - 2 when 6 * 2^(fl - 2) = 1.5 * 2^fl covers amax (sig <= 192), else fl - 1.
__device__ __forceinline__ int mx_exponent(uint32_t mx, bool fit) {
  if (mx == 0) return -127;
  const int E = (int)(mx >> 7);
  // normal: 2^(E-127) <= amax; subnormal m * 2^-133: highest set bit of m
  const int hb = 31 - __builtin_clz((mx & 0x7Fu) | 1u);
  const int fl = E > 0 ? E - 127 : hb - 133;
  const int sig = E > 0 ? (int)(0x80u | (mx & 0x7Fu)) : (int)((mx & 0x7Fu) << (7 - hb));
  int e = fl - 2 + (fit && sig > 192 ? 1 : 0);
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// E2M1 code of the bf16 value `bits` scaled by 2^-e.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t bits, int e) {
  const float y = ldexpf(__uint_as_float((bits & 0x7FFFu) << 16), -e);
  uint32_t c = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) + (y > 2.5f) +
               (y >= 3.5f) + (y > 5.0f);
  if ((bits & 0x8000u) && (bits & 0x7FFFu)) c |= 8u;
  return c;
}

// One wave per candidate row (grid-strided), one block of 32 elements per
// lane and step. ids NULL: row i is head row i. A row whose id is outside
// [0, V) is written as zero codes with scale code 0.
__global__ void __launch_bounds__(256)
    pack_mxfp4(const uint4 *__restrict__ head, int64_t V, int H, const int32_t *__restrict__ ids,
               int64_t C, uint4 *__restrict__ q, uint8_t *__restrict__ scales, int fit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int nblk = H / 32;
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < C;
       row += waves) {
    const int64_t id = ids ? (int64_t)ids[row] : row;
    const bool valid = id >= 0 && id < V;
    const uint4 *src = head + (valid ? id : 0) * (int64_t)(H / 8);
    for (int b = lane; b < nblk; b += kWave) {
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 v = src[4 * b + k];
        w[4 * k] = v.x;
        w[4 * k + 1] = v.y;
        w[4 * k + 2] = v.z;
        w[4 * k + 3] = v.w;
      }
      uint32_t mx = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
        mx = lo > mx ? lo : mx;
        mx = hi > mx ? hi : mx;
      }
      const int e = valid ? mx_exponent(mx, fit != 0) : -127;
      uint32_t out[4] = {0u, 0u, 0u, 0u};
      if (valid) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          // word k holds elements 2k (low half) and 2k + 1: one code byte
          const uint32_t byte = e2m1_code(w[k] & 0xFFFFu, e) | (e2m1_code(w[k] >> 16, e) << 4);
          out[k >> 2] |= byte << (8 * (k & 3));
        }
      }
      q[row * nblk + b] = make_uint4(out[0], out[1], out[2], out[3]);
      scales[row * nblk + b] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_pack_mxfp4(const void *head, int64_t V, int H, const int32_t *ids, int64_t C,
                             void *q, uint8_t *scales, int rule, int num_cus,
                             hipStream_t stream) {
  const int64_t waves_per_block = 4;
  int64_t blocks = (C + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_mxfp4, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4 *)head, V, H, ids, C, (uint4 *)q, scales, rule);
  return hipGetLastError();
}

// MXFP4 tiled layout (batched draft rows on the matrix cores): rows in tiles
// of 64 (zero rows pad the last), columns padded with zeros to a multiple of
// 256 and grouped in fours of 32-column steps. Code fragment (t, p, rb), 1 KiB,
// ordered (t, p, rb): lane j + 16g holds, for u = 0..3, 4 bytes (8 codes, the
// even element in the low nibble) of row 64t + 16rb + j at columns
// 32(4p + u) + 8g .. 32(4p + u) + 8g + 7. Scale group (t, p), 256 bytes: byte
// rb * 64 + j * 4 + u is the E8M0 code of that row's block 4p + u. One wave
// per row (padding rows included), one 32-element block per lane and step;
// padding blocks get zero codes and scale code 0.
__global__ void __launch_bounds__(256)
    pack_tiled_mxfp4(const uint4 *__restrict__ head, int64_t V, int H,
                     const int32_t *__restrict__ ids, int64_t C, int64_t Cp, int Hp,
                     uint8_t *__restrict__ tiled, uint8_t *__restrict__ tscales, int fit) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int nblk = H / 32;
  const int nblkp = Hp / 32;
  const int SP = Hp / 128;
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < Cp;
       row += waves) {
    const int64_t id = row < C ? (ids ? (int64_t)ids[row] : row) : -1;
    const bool valid = id >= 0 && id < V;
    const uint4 *src = head + (valid ? id : 0) * (int64_t)(H / 8);
    const int64_t t = row / 64;
    const int rb = (int)((row % 64) / 16);
    const int j = (int)(row % 16);
    for (int b = lane; b < nblkp; b += kWave) {
      uint32_t words[4] = {0u, 0u, 0u, 0u};
      int e = -127;
      if (valid && b < nblk) {
        uint32_t w[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 v = src[4 * b + k];
          w[4 * k] = v.x;
          w[4 * k + 1] = v.y;
          w[4 * k + 2] = v.z;
          w[4 * k + 3] = v.w;
        }
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
          mx = lo > mx ? lo : mx;
          mx = hi > mx ? hi : mx;
        }
        e = mx_exponent(mx, fit != 0);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t byte = e2m1_code(w[k] & 0xFFFFu, e) | (e2m1_code(w[k] >> 16, e) << 4);
          words[k >> 2] |= byte << (8 * (k & 3));
        }
      }
      const int p = b / 4;
      const int u = b % 4;
      const int64_t frag = (t * SP + p) * 4 + rb;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint32_t *>(tiled + (frag * kWave + j + 16 * g) * 16 + 4 * u) = words[g];
      tscales[(t * SP + p) * 256 + rb * 64 + j * 4 + u] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_pack_tiled_mxfp4(const void *head, int64_t V, int H, const int32_t *ids,
                                   int64_t C, void *tiled, uint8_t *tscales, int rule,
                                   int num_cus, hipStream_t stream) {
  const int64_t Cp = (C + 63) / 64 * 64;
  const int Hp = (H + 255) / 256 * 256;
  const int64_t waves_per_block = 4;
  int64_t blocks = (Cp + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_tiled_mxfp4, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4 *)head, V, H, ids, C, Cp, Hp, (uint8_t *)tiled, tscales, rule);
  return hipGetLastError();
}

// ---- draft GEMV + argmax ---------------------------------------------------

constexpr int kFp4Threads = 256;
constexpr int kFp4Waves = kFp4Threads / kWave;

__device__ __forceinline__ uint4 load_stream_fp4(const uint4 *p) {
  const u32x4_fp4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_fp4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The scale 2^(code - 127) as a float (code 0: 2^-127, a subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t code) {
  return __uint_as_float(code ? code << 23 : 0x00400000u);
}

// Sum over one block's 32 columns of value(code) * hidden, in column order:
// code word k (8 elements) against hidden chunk h[k].
__device__ __forceinline__ float dot32_fp4(const uint4 &c, const uint4 (&h)[4]) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t hw[4] = {h[k].x, h[k].y, h[k].z, h[k].w};
    const bf16x2_fp4_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[k], 1.0f, 0);
    const bf16x2_fp4_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[k], 1.0f, 1);
    const bf16x2_fp4_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[k], 1.0f, 2);
    const bf16x2_fp4_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[k], 1.0f, 3);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p0, __builtin_bit_cast(bf16x2_fp4_t, hw[0]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p1, __builtin_bit_cast(bf16x2_fp4_t, hw[1]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p2, __builtin_bit_cast(bf16x2_fp4_t, hw[2]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(p3, __builtin_bit_cast(bf16x2_fp4_t, hw[3]), acc, false);
  }
  return acc;
}

// MR hidden rows, NCL blocks per lane and row, RB table rows per wave
// iteration, next iteration's rows in flight; EXACT: H is NCL * 2048 (no
// block predication). GATHER: candidate i is head row gids[i] of a head of
// gV rows (any order, repeats allowed) and its argmax key is that id, so
// ties go to the lowest id; an id outside [0, gV) is no candidate (its loads
// read row 0 and it is never reported). Otherwise candidate i is row i.
template <int MR, int NCL, int RB, bool EXACT, bool GATHER>
__global__ void __launch_bounds__(kFp4Threads)
    gemv_argmax_mxfp4(const uint4 *__restrict__ X, const uint4 *__restrict__ Q,
                      const uint8_t *__restrict__ S, int M, int64_t N, int nblk,
                      const int32_t *__restrict__ gids, int64_t gV, RowSink sink) {
  __shared__ float s_val[kFp4Waves][MR];
  __shared__ int64_t s_row[kFp4Waves][MR];
  __shared__ float f_val[MR];
  __shared__ int64_t f_row[MR];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * MR;
  const int nch = 4 * nblk;  // hidden row: 16-byte chunks of 8 bf16

  uint4 h[MR][NCL][4];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const int blk = lane + kWave * c;
      const bool ok = m0 + r < M && (EXACT || blk < nblk);
      const uint4 *xr = X + (int64_t)(m0 + r) * nch + 4 * blk;
#pragma unroll
      for (int k = 0; k < 4; ++k) h[r][c][k] = ok ? xr[k] : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  float bv[MR];
  int64_t bi[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    bv[r] = 0.0f;
    bi[r] = -1;
  }

  // key[i] (gathered candidates only): the id of candidate r0 + i, -1 when
  // it is past N or not a candidate
  auto load = [&](uint4(&w)[RB][NCL], uint32_t(&s)[RB][NCL], int32_t(&key)[RB], int64_t r0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      // rows past N and non-candidates read row 0 (never reported); a packed
      // table keeps no keys, its row is a wave-uniform expression of r0
      int64_t row;
      if constexpr (GATHER) {
        int32_t k = -1;
        if (r0 + i < N) {
          const int32_t id = gids[r0 + i];
          k = (id >= 0 && id < gV) ? id : -1;
        }
        key[i] = k;
        row = k >= 0 ? k : 0;
      } else {
        row = r0 + i < N ? r0 + i : 0;
      }
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        const int blk = lane + kWave * c;
        const bool ok = EXACT || blk < nblk;
        w[i][c] = ok ? load_stream_fp4(Q + row * nblk + blk) : make_uint4(0u, 0u, 0u, 0u);
        s[i][c] = ok ? (uint32_t)S[row * nblk + blk] : 0u;
      }
    }
  };

  const int64_t stride = (int64_t)gridDim.x * kFp4Waves * RB;
  int64_t r0 = ((int64_t)blockIdx.x * kFp4Waves + __builtin_amdgcn_readfirstlane(wave)) * RB;
  uint4 nxt[RB][NCL];
  uint32_t snxt[RB][NCL];
  int32_t knxt[RB];
  if (r0 < N) load(nxt, snxt, knxt, r0);
  for (; r0 < N; r0 += stride) {
    uint4 w[RB][NCL];
    uint32_t sc[RB][NCL];
    int32_t key[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if constexpr (GATHER) key[i] = knxt[i];
#pragma unroll
      for (int c = 0; c < NCL; ++c) {
        w[i][c] = nxt[i][c];
        sc[i][c] = snxt[i][c];
      }
    }
    if (r0 + stride < N) load(nxt, snxt, knxt, r0 + stride);
    float acc[MR][RB];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[r][i] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCL; ++c)
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const float scale = e8m0_value(sc[i][c]);
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r][i] += dot32_fp4(w[i][c], h[r][c]) * scale;
      }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float s = wave_sum(acc[r][i]);
        // a packed table's candidate is row r0 + i; a gathered one its id
        if constexpr (GATHER) {
          if (key[i] >= 0 && better(s, key[i], bv[r], bi[r])) {
            bv[r] = s;
            bi[r] = key[i];
          }
        } else if (r0 + i < N && better(s, r0 + i, bv[r], bi[r])) {
          bv[r] = s;
          bi[r] = r0 + i;
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
    for (int q = 1; q < kFp4Waves; ++q) {
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

// Rows per iteration: about 8 KiB of codes in flight per wave. A packed
// table with one block per lane (H up to 2,048) runs 4 rows per iteration,
// and 2 once a pass holds 4 or more hidden rows (sweep on MI355X at
// 65,536 x 2,048: 18.6 against 19.3 us at M = 1, 31.9 against 35.1 us at
// M = 4). Gathered rows keep 8: each row waits on its id first, and 4 rows
// per iteration were slower there (22.2 against 21.2 us at M = 1).
template <int MR, int NCL, bool GATHER>
constexpr int fp4_rb() {
  if (NCL == 1 && !GATHER) return MR >= 4 ? 2 : 4;
  return NCL >= 8 ? 1 : 8 / NCL;
}

template <int MR, int NCL, bool GATHER>
static hipError_t launch_fp4_shape(const Fp4Launch &L) {
  constexpr int RB = fp4_rb<MR, NCL, GATHER>();
  const int64_t row_blocks = (L.N + RB - 1) / RB;
  const int64_t want = (row_blocks + kFp4Waves - 1) / kFp4Waves;
  const int gx = (int)(want < L.max_blocks_x ? want : L.max_blocks_x);
  const int gy = (L.M + MR - 1) / MR;
  const dim3 grid(gx, gy), block(kFp4Threads);
  const uint4 *X = (const uint4 *)L.X, *Q = (const uint4 *)L.Q;
  const int32_t *gids = GATHER ? L.gather_ids : nullptr;
  const int64_t gV = GATHER ? L.gather_V : 0;
  if (L.nblk == NCL * kWave)
    return launch_call_kernel((gemv_argmax_mxfp4<MR, NCL, RB, true, GATHER>), grid, block,
                              L.stream, true, true, X, Q, L.scales, L.M, L.N, L.nblk, gids, gV,
                              L.sink);
  return launch_call_kernel((gemv_argmax_mxfp4<MR, NCL, RB, false, GATHER>), grid, block,
                            L.stream, true, true, X, Q, L.scales, L.M, L.N, L.nblk, gids, gV,
                            L.sink);
}

template <int MR, int NCL>
static hipError_t launch_fp4_cfg(const Fp4Launch &L) {
  // the hidden slices take 16 registers per (row, block): MR * NCL <= 8
  if constexpr (MR * NCL > 8) {
    return hipErrorInvalidValue;
  } else {
    return L.gather_ids ? launch_fp4_shape<MR, NCL, true>(L)
                        : launch_fp4_shape<MR, NCL, false>(L);
  }
}

template <int MR>
static hipError_t launch_fp4_mr(const Fp4Launch &L, int ncl) {
  switch (ncl) {
    case 1: return launch_fp4_cfg<MR, 1>(L);
    case 2: return launch_fp4_cfg<MR, 2>(L);
    case 3: return launch_fp4_cfg<MR, 3>(L);
    case 4: return launch_fp4_cfg<MR, 4>(L);
    case 6: return launch_fp4_cfg<MR, 6>(L);
    case 8: return launch_fp4_cfg<MR, 8>(L);
    default: return hipErrorInvalidValue;
  }
}

// Blocks per lane that have an instantiation (a request rounds up).
static const int kFp4NclSteps[] = {1, 2, 3, 4, 6, 8};

int fp4_ncl_for(int nblk) {
  const int need = (nblk + kWave - 1) / kWave;
  for (int n : kFp4NclSteps)
    if (n >= need) return n;
  return 0;
}

// Hidden rows per pass: the smallest power of two >= M, at most 8 and with
// MR * NCL <= 8 (more rows take several passes over the table).
int fp4_rows_for(int M, int ncl) {
  int mr = 1;
  while (mr < M && mr < 8 && 2 * mr * ncl <= 8) mr *= 2;
  return mr;
}

hipError_t launch_fp4(const Fp4Launch &L, int mr, int ncl) {
  switch (mr) {
    case 1: return launch_fp4_mr<1>(L, ncl);
    case 2: return launch_fp4_mr<2>(L, ncl);
    case 4: return launch_fp4_mr<4>(L, ncl);
    case 8: return launch_fp4_mr<8>(L, ncl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
