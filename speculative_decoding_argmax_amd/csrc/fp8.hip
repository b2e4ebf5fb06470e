// FP8 (E4M3) candidate table: quantising pack and the draft GEMV + argmax
// over it (mtp.h, "FP8 candidate table").
//
// Format: OCP 8-bit float E4M3 (sign, 4 exponent bits with bias 7, 3
// mantissa bits, subnormals m * 2^-9, no infinities, S.1111.111 NaN, largest
// magnitude 448). Each row has one scale 2^e, the smallest power of two with
// max|w| <= 448 * 2^e (e = 0 for an all-zero row); element j is the E4M3
// code nearest to w[j] * 2^-e, ties to the even code. The pack works on the
// integer fields of the bf16 encoding only: a bf16 value is an 8-bit
// significand times a power of two, the scale shifts that power, and the
// E4M3 code is the significand shifted right to 3 fraction bits (or to the
// 2^-9 subnormal step) with round-half-to-even on the dropped bits, the carry
// running into the exponent field. No floating-point arithmetic is involved.
//
// The draft kernel streams 16 codes (16 bytes) per lane and load, converts
// them to bf16 pairs with v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3
// value is a bf16 value) and accumulates with v_dot2c_f32_bf16 against the
// hidden row, in column order; the wave sum is multiplied by the row's scale
// (a power of two: exact). Rows per wave, prefetch, argmax and the
// cross-workgroup finish follow the bf16 vector-ALU kernel.

#include "common.hpp"
#include "launch.hpp"

namespace mtp {

typedef __bf16 bf16x2_fp8_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_fp8_t __attribute__((ext_vector_type(4)));

// ---- quantising pack ------------------------------------------------------

// A finite nonzero bf16 magnitude (15 bits, sign dropped) as sig * 2^ex with
// an 8-bit significand sig in [128, 255]; subnormal bf16 values are shifted
// up to that form. Zero gives sig = 0.
__device__ __forceinline__ void bf16_sig_exp(uint32_t mag, int &sig, int &ex) {
  const int E = (int)(mag >> 7);
  const int f = (int)(mag & 0x7Fu);
  if (E != 0) {
    sig = 128 | f;
    ex = E - 134;
  } else if (f != 0) {
    const int sh = __clz(f) - 24;  // moves the highest set bit to bit 7
    sig = f << sh;
    ex = -133 - sh;
  } else {
    sig = 0;
    ex = 0;
  }
}

// x >> sh rounded to nearest, ties to even (x < 2^16, sh >= 1).
__device__ __forceinline__ uint32_t shr_round_even(uint32_t x, int sh) {
  if (sh > 20) return 0u;  // x / 2^sh < 1/2
  const uint32_t q = x >> sh;
  const uint32_t rem = x & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

// Row scale exponent from the row's largest bf16 magnitude: the smallest e
// with sig * 2^ex <= 448 * 2^e = 7 * 2^(6 + e). With sig in [128, 255] the
// bound 7 * 2^d first covers sig at d = 5 (224) when sig <= 224, else at
// d = 6 (448), and e = ex + d - 6. A zero row keeps e = 0.
__device__ __forceinline__ int fp8_row_exp(uint32_t max_mag) {
  int sig, ex;
  bf16_sig_exp(max_mag, sig, ex);
  if (sig == 0) return 0;
  return sig <= 224 ? ex - 1 : ex;
}

// 2^e as an fp32 bit pattern (e in [-149, 127]; the pack's range is
// [-141, 120]).
__device__ __forceinline__ float pow2_f32(int e) {
  return __uint_as_float(e >= -126 ? (uint32_t)(e + 127) << 23 : 1u << (e + 149));
}

// E4M3 code of the bf16 value `bits` times 2^-e: nearest code, ties to the
// even code, magnitudes past 448 saturating to 448 (code 0x7E), the sign bit
// kept also when the magnitude rounds to zero.
__device__ __forceinline__ uint32_t e4m3_of_bf16(uint32_t bits, int e) {
  const uint32_t sign = (bits >> 8) & 0x80u;
  int sig, ex;
  bf16_sig_exp(bits & 0x7FFFu, sig, ex);
  if (sig == 0) return sign;
  // y = sig * 2^(ex - e) lies in [2^u, 2^(u+1)) with u = ex - e + 7; its
  // E4M3 exponent field would be be = u + 7
  const int be = ex - e + 14;
  uint32_t c;
  if (be >= 1) {
    // normal code: exponent field and the 7 fraction bits of sig, rounded
    // to 3 fraction bits; a carry out of the fraction bumps the exponent
    c = shr_round_even(((uint32_t)be << 7) | (uint32_t)(sig & 0x7F), 4);
  } else {
    // subnormal code: y in steps of 2^-9 is sig * 2^(be - 5); a count of 8
    // is code 0x08, the smallest normal value 2^-6
    c = shr_round_even((uint32_t)sig, 5 - be);
  }
  return sign | (c > 0x7Eu ? 0x7Eu : c);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// One wave per candidate row (grid-strided). ids NULL: row i is head row i.
// A row whose id is outside [0, V) is written as zero codes with scale 1.
__global__ void __launch_bounds__(256)
    pack_fp8(const uint4 *__restrict__ head, int64_t V, int H, const int32_t *__restrict__ ids,
             int64_t C, uint2 *__restrict__ q, float *__restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int nch = H / 8;  // 16-byte chunks of 8 bf16
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < C;
       row += waves) {
    const int64_t id = ids ? (int64_t)ids[row] : row;
    const bool valid = id >= 0 && id < V;
    const uint4 *src = head + (valid ? id : 0) * nch;
    uint32_t mx = 0;
    for (int c = lane; c < nch; c += kWave) {
      const uint4 v = src[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
        mx = lo > mx ? lo : mx;
        mx = hi > mx ? hi : mx;
      }
    }
    mx = valid ? wave_max_u32(mx) : 0u;
    // a row holding Inf or NaN is outside the contract: it keeps e = 0
    const int e = mx < 0x7F80u ? fp8_row_exp(mx) : 0;
    uint2 *dst = q + row * (int64_t)(H / 8);
    for (int c = lane; c < nch; c += kWave) {
      uint32_t b[2] = {0u, 0u};
      if (valid) {
        const uint4 v = src[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t bits = (k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu);
          const uint32_t code = e4m3_of_bf16(bits, e);
          b[k >> 2] |= code << (8 * (k & 3));
        }
      }
      dst[c] = make_uint2(b[0], b[1]);
    }
    if (lane == 0) scales[row] = valid ? pow2_f32(e) : 1.0f;
  }
}

hipError_t launch_pack_fp8(const void *head, int64_t V, int H, const int32_t *ids, int64_t C,
                           void *q, float *scales, int num_cus, hipStream_t stream) {
  const int64_t waves_per_block = 4;
  int64_t blocks = (C + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint4 *)head,
                     V, H, ids, C, (uint2 *)q, scales);
  return hipGetLastError();
}

// FP8 tiled layout (the fp8 form of the 64-row tiled layout): rows in tiles
// of 64, columns padded to a multiple of 128 and grouped in pairs of 32-column
// steps. Fragment (t, p, rb), 1 KiB, ordered (t, p, rb): lane j + 16g holds
// the 8 codes of row 64t + 16rb + j, columns 64p + 8g .. 64p + 8g + 7, then
// the 8 codes of columns 64p + 32 + 8g .. 64p + 32 + 8g + 7. One wave per
// row (padding rows included, written as zeros); rows quantised as pack_fp8.
__global__ void __launch_bounds__(256)
    pack_tiled_fp8(const uint4 *__restrict__ head, int64_t V, int H, const int32_t *__restrict__ ids,
                   int64_t C, int64_t Cp, int Hp, uint8_t *__restrict__ tiled,
                   float *__restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int nch = H / 8;
  const int SP = Hp / 64;
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < Cp;
       row += waves) {
    const int64_t id = row < C ? (ids ? (int64_t)ids[row] : row) : -1;
    const bool valid = id >= 0 && id < V;
    const uint4 *src = head + (valid ? id : 0) * nch;
    uint32_t mx = 0;
    if (valid) {
      for (int c = lane; c < nch; c += kWave) {
        const uint4 v = src[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
          mx = lo > mx ? lo : mx;
          mx = hi > mx ? hi : mx;
        }
      }
    }
    mx = wave_max_u32(mx);
    const int e = mx < 0x7F80u ? fp8_row_exp(mx) : 0;
    const int64_t t = row / 64;
    const int rb = (int)(row % 64) / 16;
    const int jj = (int)(row % 16);
    for (int c8 = lane; c8 < Hp / 8; c8 += kWave) {
      uint32_t b[2] = {0u, 0u};
      if (valid && c8 < nch) {
        const uint4 v = src[c8];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t bits = (k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFFu);
          const uint32_t code = e4m3_of_bf16(bits, e);
          b[k >> 2] |= code << (8 * (k & 3));
        }
      }
      const int s = c8 / 4, g = c8 % 4;
      const int64_t off = ((((t * SP + s / 2) * 4 + rb) * kWave + jj + 16 * g) * 16) + (s & 1) * 8;
      *reinterpret_cast<uint2 *>(tiled + off) = make_uint2(b[0], b[1]);
    }
    if (lane == 0 && row < C) scales[row] = valid ? pow2_f32(e) : 1.0f;
  }
}

hipError_t launch_pack_tiled_fp8(const void *head, int64_t V, int H, const int32_t *ids,
                                 int64_t C, void *tiled, float *scales, int num_cus,
                                 hipStream_t stream) {
  const int64_t Cp = tiled_rows(C);
  const int Hp = tiled_cols(H);
  const int64_t waves_per_block = 4;
  int64_t blocks = (Cp + waves_per_block - 1) / waves_per_block;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(pack_tiled_fp8, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint4 *)head, V, H, ids, C, Cp, Hp, (uint8_t *)tiled, scales);
  return hipGetLastError();
}

// ---- draft GEMV + argmax ---------------------------------------------------

constexpr int kFp8Threads = 256;
constexpr int kFp8Waves = kFp8Threads / kWave;

__device__ __forceinline__ uint4 load_stream_fp8(const uint4 *p) {
  const u32x4_fp8_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_fp8_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// acc + sum over 16 columns of value(code) * hidden: codes c (16 bytes),
// hidden h0 (columns 0..7), h1 (columns 8..15), in column order.
__device__ __forceinline__ float dot16_fp8(const uint4 &c, const uint4 &h0, const uint4 &h1,
                                           float acc) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2_fp8_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cw[k], 1.0f, false);
    const bf16x2_fp8_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)cw[k], 1.0f, true);
    acc = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2_fp8_t, hw[2 * k]), acc,
                                          false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2_fp8_t, hw[2 * k + 1]),
                                          acc, false);
  }
  return acc;
}

// MR hidden rows, NCL code chunks (16 columns) per lane and row, RB table
// rows per wave iteration, next iteration's rows in flight; EXACT: H is
// NCL * 1024 (no column predication). GATHER: candidate i is head row
// gids[i] of a head of gV rows (any order, repeats allowed), keyed by that
// id, so ties go to the lowest id; an id outside [0, gV) is no candidate
// (its loads read row 0 and it is never reported). Otherwise candidate i is
// row i.
template <int MR, int NCL, int RB, bool EXACT, bool GATHER>
__global__ void __launch_bounds__(kFp8Threads)
    gemv_argmax_fp8(const uint4 *__restrict__ X, const uint4 *__restrict__ Q,
                    const float *__restrict__ scales, int M, int64_t N, int ncq,
                    const int32_t *__restrict__ gids, int64_t gV, RowSink sink) {
  __shared__ float s_val[kFp8Waves][MR];
  __shared__ int64_t s_row[kFp8Waves][MR];
  __shared__ float f_val[MR];
  __shared__ int64_t f_row[MR];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int m0 = blockIdx.y * MR;
  const int nch = 2 * ncq;  // hidden row: 16-byte chunks of 8 bf16

  uint4 h[MR][NCL][2];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
#pragma unroll
    for (int c = 0; c < NCL; ++c) {
      const int col = lane + kWave * c;
      const bool ok = m0 + r < M && (EXACT || col < ncq);
      const uint4 *xr = X + (int64_t)(m0 + r) * nch + 2 * col;
      h[r][c][0] = ok ? xr[0] : make_uint4(0u, 0u, 0u, 0u);
      h[r][c][1] = ok ? xr[1] : make_uint4(0u, 0u, 0u, 0u);
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
  auto load = [&](uint4(&w)[RB][NCL], int32_t(&key)[RB], int64_t r0) {
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
      const uint4 *p = Q + row * ncq + lane;
#pragma unroll
      for (int c = 0; c < NCL; ++c)
        w[i][c] = (EXACT || lane + kWave * c < ncq) ? load_stream_fp8(p + kWave * c)
                                                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  const int64_t stride = (int64_t)gridDim.x * kFp8Waves * RB;
  int64_t r0 = ((int64_t)blockIdx.x * kFp8Waves + __builtin_amdgcn_readfirstlane(wave)) * RB;
  uint4 nxt[RB][NCL];
  int32_t knxt[RB];
  if (r0 < N) load(nxt, knxt, r0);
  for (; r0 < N; r0 += stride) {
    uint4 w[RB][NCL];
    int32_t key[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if constexpr (GATHER) key[i] = knxt[i];
#pragma unroll
      for (int c = 0; c < NCL; ++c) w[i][c] = nxt[i][c];
    }
    if (r0 + stride < N) load(nxt, knxt, r0 + stride);
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
        for (int r = 0; r < MR; ++r)
          acc[r][i] = dot16_fp8(w[i][c], h[r][c][0], h[r][c][1], acc[r][i]);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      // a packed table's candidate is row r0 + i (wave-uniform); a gathered
      // one is keyed by its id
      float scale;
      if constexpr (GATHER)
        scale = key[i] >= 0 ? scales[key[i]] : 0.0f;
      else
        scale = r0 + i < N ? scales[r0 + i] : 0.0f;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float s = wave_sum(acc[r][i]) * scale;
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
    for (int q = 1; q < kFp8Waves; ++q) {
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
// table with two chunks per lane (H up to 2,048) runs 2 rows per iteration
// once a pass holds 4 or more hidden rows (sweep on MI355X at
// 65,536 x 2,048: 32.9 against 34.9 us at M = 4; at M = 1, 4 rows stay
// best). Gathered rows keep the general rule (each row waits on its id).
template <int MR, int NCL, bool GATHER>
constexpr int fp8_rb() {
  if (NCL == 2 && MR >= 4 && !GATHER) return 2;
  return NCL >= 8 ? 1 : (8 / NCL > 4 ? 4 : 8 / NCL);
}

template <int MR, int NCL, bool GATHER>
static hipError_t launch_fp8_shape(const Fp8Launch &L) {
  constexpr int RB = fp8_rb<MR, NCL, GATHER>();
  const int64_t row_blocks = (L.N + RB - 1) / RB;
  const int64_t want = (row_blocks + kFp8Waves - 1) / kFp8Waves;
  const int gx = (int)(want < L.max_blocks_x ? want : L.max_blocks_x);
  const int gy = (L.M + MR - 1) / MR;
  const dim3 grid(gx, gy), block(kFp8Threads);
  const uint4 *X = (const uint4 *)L.X, *Q = (const uint4 *)L.Q;
  const int32_t *gids = GATHER ? L.gather_ids : nullptr;
  const int64_t gV = GATHER ? L.gather_V : 0;
  if (L.ncq == NCL * kWave)
    return launch_call_kernel((gemv_argmax_fp8<MR, NCL, RB, true, GATHER>), grid, block,
                              L.stream, true, true, X, Q, L.scales, L.M, L.N, L.ncq, gids, gV,
                              L.sink);
  return launch_call_kernel((gemv_argmax_fp8<MR, NCL, RB, false, GATHER>), grid, block, L.stream,
                            true, true, X, Q, L.scales, L.M, L.N, L.ncq, gids, gV, L.sink);
}

template <int MR, int NCL>
static hipError_t launch_fp8_cfg(const Fp8Launch &L) {
  // the hidden slices take 8 registers per (row, chunk): MR * NCL <= 16
  if constexpr (MR * NCL > 16) {
    return hipErrorInvalidValue;
  } else {
    return L.gather_ids ? launch_fp8_shape<MR, NCL, true>(L)
                        : launch_fp8_shape<MR, NCL, false>(L);
  }
}

template <int MR>
static hipError_t launch_fp8_mr(const Fp8Launch &L, int ncl) {
  switch (ncl) {
    case 1: return launch_fp8_cfg<MR, 1>(L);
    case 2: return launch_fp8_cfg<MR, 2>(L);
    case 3: return launch_fp8_cfg<MR, 3>(L);
    case 4: return launch_fp8_cfg<MR, 4>(L);
    case 5: return launch_fp8_cfg<MR, 5>(L);
    case 6: return launch_fp8_cfg<MR, 6>(L);
    case 8: return launch_fp8_cfg<MR, 8>(L);
    case 10: return launch_fp8_cfg<MR, 10>(L);
    case 12: return launch_fp8_cfg<MR, 12>(L);
    case 16: return launch_fp8_cfg<MR, 16>(L);
    default: return hipErrorInvalidValue;
  }
}

// Code chunks per lane that have an instantiation (a request rounds up).
static const int kFp8NclSteps[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};

int fp8_ncl_for(int ncq) {
  const int need = (ncq + kWave - 1) / kWave;
  for (int n : kFp8NclSteps)
    if (n >= need) return n;
  return 0;
}

// Hidden rows per pass: the smallest power of two >= M, at most 8 and with
// MR * NCL <= 16 (more rows take several passes over the table).
int fp8_rows_for(int M, int ncl) {
  int mr = 1;
  while (mr < M && mr < 8 && 2 * mr * ncl <= 16) mr *= 2;
  return mr;
}

hipError_t launch_fp8(const Fp8Launch &L, int mr, int ncl) {
  switch (mr) {
    case 1: return launch_fp8_mr<1>(L, ncl);
    case 2: return launch_fp8_mr<2>(L, ncl);
    case 4: return launch_fp8_mr<4>(L, ncl);
    case 8: return launch_fp8_mr<8>(L, ncl);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
