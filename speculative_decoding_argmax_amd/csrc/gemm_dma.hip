// Skinny GEMM + per-row argmax on the matrix cores, fed by LDS DMA from a
// table stored in the 64-row tiled layout (mtp.h, "Tiled tables").
//
// Tiled layout: rows are grouped in tiles of 64 (zero rows pad the last tile),
// columns in steps of 32 (zero columns pad H to a multiple of 128). Tile t,
// step s holds four 1 KiB fragments, one per 16-row block rb, and fragment
// (t, s, rb) is exactly the A operand of v_mfma_f32_16x16x32_bf16 for table
// rows 64t + 16rb + [0, 16) and columns 32s + [0, 32): lane l = j + 16g holds
// row 64t + 16rb + j, columns 32s + 8g + [0, 8). Fragments are ordered
// (t, s, rb), so a 64-row tile is one contiguous stream and every K chunk of it
// is one contiguous block.
//
// A workgroup of WV waves owns tiles of WV * RW * 16 table rows, grid-strided
// over the table. Each K chunk (KS steps of 32 columns) of a tile is copied
// into LDS by global_load_lds_dwordx4 (one 1 KiB fragment per instruction,
// straight from HBM, no registers): the RBT * KS weight fragments and, gathered
// from the row-major hidden block, the KS * NB hidden fragments (operand B,
// 16 hidden rows x 32 columns each). Chunks rotate through NBUF LDS slots: the
// copy of chunk it + NBUF - 1 is in flight while chunk it is multiplied. Each
// wave owns RW 16-row blocks and all NB 16-row blocks of hidden rows; lanes
// keep the best (logit, row) of their hidden row, then lanes and waves merge
// through LDS and finish_rows merges workgroups.
//
// Synchronisation: each slot is its own __shared__ array and the loop is
// unrolled by NBUF, so the compiler can see that reads of slot it do not alias
// the copies into other slots and leaves those copies in flight. Before
// reading a slot, every wave waits (s_waitcnt vmcnt) until its own copies into
// that slot have landed (all waves issue the same number of fragment copies
// per chunk, so the count of younger copies is a constant; scale copies are
// left out of it and only make their waves wait longer), then all waves meet at a
// plain s_barrier (no fence, which would wait for every copy in flight). The
// barrier also orders the next copy into a slot after every wave's reads of
// that slot's previous chunk.
//
// Every logit sums its columns in one order (chunks, then steps, ascending;
// the MFMA's fixed in-step order), whatever the row's tile or position, so
// duplicated rows score bit-identically and ties go to the lower row.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mtp {

typedef __bf16 bf16x8_dma_t __attribute__((ext_vector_type(8)));
typedef float f32x4_dma_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_ring_t __attribute__((ext_vector_type(4)));

#define MTP_LDS(p) ((__attribute__((address_space(3))) void *)(p))

__device__ __forceinline__ f32x4_dma_t mfma16_dma(const uint4 &a, const uint4 &b,
                                                  f32x4_dma_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_dma_t, a),
                                                 __builtin_bit_cast(bf16x8_dma_t, b), c, 0, 0,
                                                 0);
}

__device__ __forceinline__ bool better_row(float v, int i, float bv, int bi) {
  return bi < 0 || v > bv || (v == bv && i < bi);
}

// The better of two (logit, row) candidates, kept in (v, i): a row >= 0
// beats none (-1), a higher logit beats a lower one, and equal logits go to
// the lower row. This is a total order on the candidates, so every
// reduction order picks the same winner.
__device__ __forceinline__ void pick_better(float &v, int &i, float v2, int i2) {
  const bool take = i2 >= 0 && (i < 0 || v2 > v || (v2 == v && i2 < i));
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Merge the 4 * WV candidates that the lanes hold for each of the NB * 16
// hidden rows (entry (w * NB + nb) * 64 + j + 16 g of red_v / red_i: wave w,
// lane j + 16 g, hidden row 16 nb + j) into f_val / f_row. Thread t < NB * 16
// takes row t: it reads all of the row's candidates first, so that the LDS
// reads overlap, then reduces them pairwise (a chain of log2(4 WV) picks
// instead of 4 WV reads and compares one after another).
template <int NB, int WV>
__device__ __forceinline__ void merge_candidates(const float *red_v, const int *red_i, int tid,
                                                 float *f_val, int64_t *f_row) {
  constexpr int Q = 4 * WV;
  static_assert((Q & (Q - 1)) == 0, "a power-of-two candidate count");
  if (tid < NB * 16) {
    const int nb = tid >> 4;
    const int jj = tid & 15;
    float cv[Q];
    int ci[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int o = ((q >> 2) * NB + nb) * kWave + jj + 16 * (q & 3);
      cv[q] = red_v[o];
      ci[q] = red_i[o];
    }
#pragma unroll
    for (int w = 1; w < Q; w <<= 1)
#pragma unroll
      for (int q = 0; q < Q; q += 2 * w) pick_better(cv[q], ci[q], cv[q + w], ci[q + w]);
    f_val[tid] = cv[0];
    f_row[tid] = ci[0];
  }
}

// Workgroup barrier without a memory fence (a fence would wait for every copy
// in flight). The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Piece swizzle of row-major weight chunks in LDS (RW16 16-byte pieces per
// row, rows stored one after another). An MFMA read has lanes j = 0..15 (and
// g) on rows 16 b + j at one piece index q; the row's piece q sits at
// position q ^ rm_swizzle(row). With 8 pieces per row (128-byte rows) the
// value (j + j / 8) mod 8 puts every 8 consecutive lanes, and every 16, on
// distinct 16-byte bank groups; with 16 or more pieces j itself does.
template <int RW16>
__device__ __forceinline__ int rm_swizzle(int trow) {
  const int j = trow & 15;
  if constexpr (RW16 == 8) return (j + (j >> 3)) & 7;
  else return j & (RW16 - 1);
}

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// NB: 16-row blocks of hidden rows; RW: 16-row table blocks per wave; KS:
// 32-column steps per chunk; NBUF: LDS slots (3 or 4); WV: waves per group;
// CP: cache-policy bits of the weight copies (2 = nt: the table is streamed
// once per call, so its lines should not displace the hidden rows in L2).
// FP8: the table holds E4M3 codes in the fp8 tiled layout (one 1 KiB
// fragment carries two 32-column steps of a 16-row block: lane j + 16g holds
// the 8 codes of step 2p, columns 8g..8g+7, then those of step 2p + 1), and
// scales[row] multiplies each finished logit.
// FP4: the table holds MXFP4 codes in the MXFP4 tiled layout (one 1 KiB
// fragment carries four steps: lane j + 16g holds 4 bytes, 8 codes, per step)
// and `scales` points at its scale groups (256 bytes per 64 rows and four
// steps); each step's codes are converted with their block's scale into the
// bf16 operand (exact), so no scale touches the logit.
template <int NB, int RW, int KS, int NBUF, int WV, int CP, bool FP8 = false, bool FP4 = false,
          bool RM = false, int PS = 1>
__global__ void __launch_bounds__(WV * 64)
    gemm_argmax_dma(const uint4 *__restrict__ X, const uint4 *__restrict__ WT, int M, int N,
                    int nch, int S, RowSink sink, const float *__restrict__ scales, int nphase) {
  constexpr int RBT = WV * RW;                 // 16-row blocks per workgroup tile
  constexpr int TV = RBT * 16;                 // table rows per workgroup tile
  // row-major weights: 16-byte pieces per row per chunk, rows per copy
  constexpr int RW16 = 4 * KS;
  constexpr int RPC = 64 / RW16;
  static_assert(!RM || (KS == 2 && !FP8 && !FP4),
                "row-major chunks: two steps, i.e. whole 128-byte lines of bf16 rows");
  static_assert(!FP8 || KS % 2 == 0, "fp8 chunks hold whole step pairs");
  static_assert(!FP4 || KS % 4 == 0, "fp4 chunks hold whole step groups");
  static_assert(!(FP8 && FP4), "one table format");
  static_assert(!FP4 || (RBT / 4) * (KS / 4) <= WV, "one wave per scale piece");
  // weight fragments per chunk
  constexpr int AF = FP4 ? RBT * KS / 4 : FP8 ? RBT * KS / 2 : RBT * KS;
  constexpr int FR = AF + KS * NB;             // fragments per chunk
  constexpr int PER_WAVE = (FR + WV - 1) / WV; // copies per wave per chunk
  static_assert(NBUF >= 3 && NBUF <= 4, "three or four slots");
  static_assert(RBT % 4 == 0, "workgroup tiles are whole 64-row tiles");
  static_assert(FR * 64 * 16 >= WV * NB * 64 * 4, "merge scratch fits a slot");
  __shared__ uint4 slot0[FR * 64];
  __shared__ uint4 slot1[FR * 64];
  __shared__ uint4 slot2[FR * 64];
  __shared__ uint4 slot3[NBUF > 3 ? FR * 64 : 1];
  __shared__ float f_val[NB * 16];
  __shared__ int64_t f_row[NB * 16];
  // fp8: the row scales of a tile, copied with the tile's last chunk into
  // the slot's scale array (one array per slot, like the fragments)
  constexpr int SCN = FP8 ? TV : 1;
  __shared__ float scale0[SCN];
  __shared__ float scale1[SCN];
  __shared__ float scale2[SCN];
  __shared__ float scale3[NBUF > 3 ? SCN : 1];
  // fp4: the scale groups of a chunk, one 256-byte piece per 64-row tile and
  // step group, copied with the chunk into the slot's array
  constexpr int NPC = FP4 ? (RBT / 4) * (KS / 4) : 0;   // pieces per chunk
  constexpr int SC4 = FP4 ? NPC * 64 : 1;               // 32-bit words per slot
  __shared__ uint32_t s4_0[SC4];
  __shared__ uint32_t s4_1[SC4];
  __shared__ uint32_t s4_2[SC4];
  __shared__ uint32_t s4_3[NBUF > 3 ? SC4 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index as a scalar: copy addresses and LDS offsets are then
  // computed on the scalar unit, not per lane
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane & 15;
  const int g = lane >> 4;
  const int m0 = blockIdx.y * NB * 16;
  // grid size and position held in registers: the barrier's compiler fence
  // would otherwise make every chunk reload gridDim from the dispatch packet
  const int gdx = gridDim.x;
  const int bx = blockIdx.x;
  const int nchunks = S / KS;                  // S is a multiple of 4
  const int ntiles = (N + TV - 1) / TV;
  const int my_tiles = bx < ntiles ? (ntiles - 1 - bx) / gdx + 1 : 0;
  const int total = my_tiles * nchunks;
  const int nrb = ((N + 63) / 64) * 4;         // 16-row blocks stored (padded)

  auto slot = [&](auto tag) -> uint4 * {
    constexpr int SL = decltype(tag)::value;
    if constexpr (SL == 0) return slot0;
    else if constexpr (SL == 1) return slot1;
    else if constexpr (SL == 2) return slot2;
    else return slot3;
  };
  auto scl4 = [&](auto tag) -> uint32_t * {
    constexpr int SL = decltype(tag)::value;
    if constexpr (SL == 0) return s4_0;
    else if constexpr (SL == 1) return s4_1;
    else if constexpr (SL == 2) return s4_2;
    else return s4_3;
  };
  auto scl = [&](auto tag) -> float * {
    constexpr int SL = decltype(tag)::value;
    if constexpr (SL == 0) return scale0;
    else if constexpr (SL == 1) return scale1;
    else if constexpr (SL == 2) return scale2;
    else return scale3;
  };

  // row-major weights: lane offsets of a copy within its RPC row segments,
  // one for copies whose rows start at an even multiple of 8 (f even) and
  // one for odd ones (the swizzle depends on the row modulo 16)
  const int rowbytes = nch * 16;
  int rm_voff[2] = {0, 0};
  if constexpr (RM) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int trow = par * RPC + lane / RW16;
      rm_voff[par] = (lane / RW16) * rowbytes + 16 * ((lane % RW16) ^ rm_swizzle<RW16>(trow));
    }
  }

  // Row-major chunk order. With a row pitch that is a multiple of 4 KiB, every
  // workgroup reading chunk c of its tile at the same moment puts all
  // concurrent reads on the same low address bits, and the HBM channels they
  // map to limit the stream (5.0-5.5 TB/s on MI355X against 6.7-7.0 with an
  // unaligned pitch or with workgroups at different column offsets). With PS
  // > 1 the columns of a row form PS contiguous segments of nchunks / PS
  // chunks, and workgroup b starts every tile at segment
  // p = (b / 8) % PS (so that every XCD holds every phase) and wraps around:
  // segments p, p + 1, ..., PS - 1, 0, ..., p - 1. Each segment is summed on
  // its own, its chunks in ascending order from zero; at the end of a tile the
  // segment sums are put back in segment order and added in one fixed order.
  // Every logit is thus the same sum of the same segment sums whatever the
  // workgroup's phase, and duplicated rows still score bit-identically.
  static_assert(PS == 1 || (RM && (PS == 2 || PS == 4 || PS == 8)), "segments: row-major, 2/4/8");
  const int seglen = nchunks / PS;
  int rot = 0;  // the workgroup's phase p
  if constexpr (PS > 1) rot = (bx >> 3) % PS;
  const int c0 = rot * seglen;
  // next chunk to copy: tile and position within the tile's rotated order
  int rm_iss_t = bx, rm_iss_pos = 0;

  // Copy the next chunk (tile iss_t, K chunk iss_c) into a slot, then step
  // the position. Fragment f < AF: weights, step f / RBT of the chunk,
  // 16-row block f % RBT of the tile; f >= AF: hidden fragment for step
  // (f - AF) / NB, hidden block (f - AF) % NB. Every wave issues PER_WAVE
  // copies; surplus ones repeat the last fragment (same bytes, same place).
  int iss_t = bx, iss_c = 0;
  auto issue = [&](auto tag) {
    uint4 *base = slot(tag);
    int tile, c;
    if constexpr (RM) {
      tile = rm_iss_t;
      c = rm_iss_pos + c0;
      c = c < nchunks ? c : c - nchunks;
      if (++rm_iss_pos == nchunks) {
        rm_iss_pos = 0;
        rm_iss_t += gdx;
      }
    } else {
      tile = iss_t;
      c = iss_c;
      if (++iss_c == nchunks) {
        iss_c = 0;
        iss_t += gdx;
      }
    }
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      int f = wave + WV * q;
      f = f < FR ? f : FR - 1;
      if (f < AF && RM) {
        // row-major weights: copy f holds RPC whole row segments of the chunk
        // (RW16 pieces of 16 bytes each, at least one 128-byte line per row);
        // the piece at LDS position (row, q) is the row's piece
        // q ^ rm_swizzle(row), so the MFMA-order reads below hit distinct
        // banks. A buffer load from a per-copy descriptor (scalar: the copy's
        // first row and chunk) plus a loop-invariant lane offset keeps no
        // per-copy address register alive; rows past the table fall outside
        // the descriptor's range and read zeros (never reported).
        const int64_t row0 = (int64_t)tile * TV + f * RPC;
        const int64_t left = ((int64_t)N - row0) * rowbytes;
        const int nrec = left <= 0 ? 0 : left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left;
        __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(reinterpret_cast<const char *>(WT) + row0 * rowbytes + c * (RW16 * 16)),
            (short)0, nrec, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MTP_LDS(base + f * kWave), 16,
                                                 rm_voff[f & 1], 0, 0, CP);
      } else if (f < AF) {
        const int s = f / RBT;  // step (bf16), step pair (fp8) or step group (fp4) of the chunk
        int rb = tile * RBT + f % RBT;
        rb = rb < nrb ? rb : nrb - 1;          // past the table: valid, never reported
        const uint4 *src =
            FP4   ? WT + (((int64_t)(rb >> 2) * (S / 4) + c * (KS / 4) + s) * 4 + (rb & 3)) * kWave + lane
            : FP8 ? WT + (((int64_t)(rb >> 2) * (S / 2) + c * (KS / 2) + s) * 4 + (rb & 3)) * kWave + lane
                  : WT + (((int64_t)(rb >> 2) * S + c * KS + s) * 4 + (rb & 3)) * kWave + lane;
        __builtin_amdgcn_global_load_lds((const void *)src, MTP_LDS(base + f * kWave), 16, 0, CP);
      } else {
        const int fb = f - AF;
        const int s = fb / NB;
        const int nb = fb - s * NB;
        // hidden rows past M and columns past H read valid addresses: the
        // extra hidden columns are never reported, and past H the weights
        // are zero
        const int m = min(m0 + nb * 16 + j, M - 1);
        const int col = min((c * KS + s) * 4 + g, nch - 1);
        const uint4 *src = X + (int64_t)m * nch + col;
        __builtin_amdgcn_global_load_lds((const void *)src, MTP_LDS(base + f * kWave), 16, 0, 0);
      }
    }
    if constexpr (FP4) {
      // every chunk brings its scale groups: wave w < NPC copies piece w
      // (64-row tile w / (KS/4) of the workgroup tile, step group w % (KS/4));
      // issued after the chunk's fragments, so the chunk's wait covers it
      if (wave < NPC) {
        int t64 = tile * (RBT / 4) + wave / (KS / 4);
        t64 = t64 < nrb / 4 ? t64 : nrb / 4 - 1;  // past the table: valid, never reported
        const uint32_t *src = reinterpret_cast<const uint32_t *>(scales) +
                              ((int64_t)t64 * (S / 4) + c * (KS / 4) + wave % (KS / 4)) * kWave + lane;
        __builtin_amdgcn_global_load_lds((const void *)src, MTP_LDS(scl4(tag) + wave * 64), 4, 0, 0);
      }
    }
    if constexpr (FP8) {
      // the tile's last chunk also brings its row scales: wave w copies those
      // of 64-row block w (issued after the chunk's fragments, so the waits
      // for the chunk cover it; rows past N read row N - 1, never reported)
      if (c == nchunks - 1 && wave < RBT / 4) {
        const int row = min(tile * TV + wave * 64 + lane, N - 1);
        __builtin_amdgcn_global_load_lds((const void *)(scales + row),
                                         MTP_LDS(scl(tag) + wave * 64), 4, 0, 0);
      }
    }
  };

  f32x4_dma_t acc[RW][NB];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
  float bv[NB];
  int bi[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    bv[nb] = 0.f;
    bi[nb] = -1;
  }

  if (0 < total) issue(std::integral_constant<int, 0>{});
  if (1 < total) issue(std::integral_constant<int, 1>{});
  if constexpr (NBUF > 3) {
    if (2 < total) issue(std::integral_constant<int, 2>{});
  }
  int cur_t = bx, cur_c = 0;  // position of the chunk being multiplied
  // row-major: position of the chunk being multiplied within its tile's
  // rotated order, and the sums of the tile's finished segments, newest first
  int rm_pos = 0;
  constexpr int SPS = PS > 1 ? PS : 1, SRW = PS > 1 ? RW : 1, SNB = PS > 1 ? NB : 1;
  f32x4_dma_t seg[SPS][SRW][SNB];

  auto body = [&](auto tag, int it) {
    constexpr int SL = decltype(tag)::value;
    // copies younger than this chunk's: chunks it+1 .. it+NBUF-2, PER_WAVE
    // each. The scale copies are not counted (fp4: one per chunk from waves
    // below NPC; fp8: one per tile-last chunk from waves below RBT / 4), so
    // those waves also wait for the oldest younger copy; an exact count,
    // chosen per wave by a scalar branch, measured no faster on MI355X.
    if (it + NBUF - 2 < total)
      wait_vmcnt<(NBUF - 2) * PER_WAVE>();
    else
      wait_vmcnt<0>();
    barrier_no_fence();
    if (it + NBUF - 1 < total) issue(std::integral_constant<int, (SL + NBUF - 1) % NBUF>{});
    const uint4 *A = slot(tag);
    const uint4 *Bf = A + AF * kWave;
    uint4 raw[RW];
    uint32_t sc4[RW];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 a[RW];
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        if constexpr (FP4) {
          // one fragment and one scale word per step group; each step's 4
          // code bytes become that step's bf16 operand, scaled by its block's
          // 2^e inside the conversion (exact)
          const int blk = wave * RW + rw;
          if (s % 4 == 0) {
            raw[rw] = A[((s / 4) * RBT + blk) * kWave + lane];
            sc4[rw] = scl4(tag)[((blk / 4) * (KS / 4) + s / 4) * 64 + (blk % 4) * 16 + j];
          }
          const uint32_t cw = s % 4 == 0 ? raw[rw].x : s % 4 == 1 ? raw[rw].y : s % 4 == 2 ? raw[rw].z : raw[rw].w;
          const uint32_t code = (sc4[rw] >> (8 * (s % 4))) & 0xFFu;
          const float sf = __uint_as_float(code ? code << 23 : 0x00400000u);
          a[rw] = make_uint4(
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 0)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 1)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 2)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sf, 3)));
        } else if constexpr (FP8) {
          // one read per step pair; each half converts to that step's
          // bf16 operand (E4M3 -> bf16 is exact)
          if (s % 2 == 0) raw[rw] = A[((s / 2) * RBT + wave * RW + rw) * kWave + lane];
          const uint32_t w0 = s % 2 ? raw[rw].z : raw[rw].x;
          const uint32_t w1 = s % 2 ? raw[rw].w : raw[rw].y;
          a[rw] = make_uint4(
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true)));
        } else if constexpr (RM) {
          // row j of 16-row block blk, piece 4s + g of the chunk
          const int trow = (wave * RW + rw) * 16 + j;
          a[rw] = A[trow * RW16 + ((4 * s + g) ^ rm_swizzle<RW16>(trow))];
        } else {
          a[rw] = A[(s * RBT + wave * RW + rw) * kWave + lane];
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 b = Bf[(s * NB + nb) * kWave + lane];
#pragma unroll
        for (int rw = 0; rw < RW; ++rw) acc[rw][nb] = mfma16_dma(a[rw], b, acc[rw][nb]);
      }
    }
    bool tile_done;
    int tile;
    if constexpr (RM) {
      tile = cur_t;
      ++rm_pos;
      if constexpr (PS > 1) {
        if (rm_pos % seglen == 0) {
          // segment done: shift it into the finished sums, start the next
#pragma unroll
          for (int rw = 0; rw < RW; ++rw)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
              for (int q = PS - 1; q > 0; --q) seg[q][rw][nb] = seg[q - 1][rw][nb];
              seg[0][rw][nb] = acc[rw][nb];
              acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
      tile_done = rm_pos == nchunks;
      if (tile_done) {
        rm_pos = 0;
        cur_t += gdx;
        if constexpr (PS > 1) {
          // seg[PS - 1 - q] holds the segment finished q-th, i.e. segment
          // (q + rot) % PS: reverse, then rotate right by rot, which leaves
          // segment s at index s; then add them in a fixed pairwise order
#pragma unroll
          for (int rw = 0; rw < RW; ++rw)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              f32x4_dma_t r[PS];
#pragma unroll
              for (int q = 0; q < PS; ++q) r[q] = seg[PS - 1 - q][rw][nb];
#pragma unroll
              for (int bit = 1; bit < PS; bit <<= 1) {
                if (rot & bit) {
                  f32x4_dma_t t2[PS];
#pragma unroll
                  for (int q = 0; q < PS; ++q) t2[q] = r[(q - bit + PS) % PS];
#pragma unroll
                  for (int q = 0; q < PS; ++q) r[q] = t2[q];
                }
              }
#pragma unroll
              for (int w = 1; w < PS; w <<= 1)
#pragma unroll
                for (int q = 0; q < PS; q += 2 * w) r[q] = r[q] + r[q + w];
              acc[rw][nb] = r[0];
            }
        }
      }
    } else {
      tile = cur_t;
      tile_done = ++cur_c == nchunks;
      if (tile_done) {
        cur_c = 0;
        cur_t += gdx;
      }
    }
    if (tile_done) {
      const int vbase = tile * TV + wave * RW * 16 + 4 * g;
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = vbase + rw * 16 + r;
            float z = acc[rw][nb][r];
            if constexpr (FP8) z *= scl(tag)[(wave * RW + rw) * 16 + 4 * g + r];
            if (v < N && better_row(z, v, bv[nb], bi[nb])) {
              bv[nb] = z;
              bi[nb] = v;
            }
          }
          acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  };

  for (int it = 0; it < total; it += NBUF) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < total) body(std::integral_constant<int, 1>{}, it + 1);
    if (it + 2 < total) body(std::integral_constant<int, 2>{}, it + 2);
    if constexpr (NBUF > 3) {
      if (it + 3 < total) body(std::integral_constant<int, 3>{}, it + 3);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Merge the 4 * WV candidates of each hidden row (slots are free now).
  float *red_v = reinterpret_cast<float *>(slot0);
  int *red_i = reinterpret_cast<int *>(slot1);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    red_v[(wave * NB + nb) * kWave + lane] = bv[nb];
    red_i[(wave * NB + nb) * kWave + lane] = bi[nb];
  }
  __syncthreads();
  merge_candidates<NB, WV>(red_v, red_i, tid, f_val, f_row);
  __syncthreads();
  const int mcount = M - m0 < NB * 16 ? M - m0 : NB * 16;
  finish_rows(sink, f_val, f_row, m0, mcount);
}


// ---------------------------------------------------------------------------
// Wide verify blocks (more than 128 hidden rows per call): weights through a
// per-wave register ring, hidden fragments through LDS.
//
// With 160 hidden rows the kernel above spends its LDS on three slots of
// 42 KiB (32 KiB of weights, 10 KiB of hidden fragments), so only two chunks
// of weights are in flight per CU, too few to cover the memory latency at
// this chunk rate. But each wave multiplies only its own 16-row blocks: the
// weight fragments need no sharing, so each wave streams them straight into
// registers (one coalesced 1 KiB non-temporal load per fragment), D - 1
// chunks ahead, and the LDS holds only the hidden fragments that all waves
// read. The hidden block is first packed into fragment order by
// pack_hidden_frags (zero rows past M, zero columns past H), so that each
// hidden copy is one contiguous 1 KiB buffer load with a loop-invariant lane
// offset. Per chunk each wave issues RW * KS weight loads, then waits until
// chunk it's hidden fragments have landed (a fixed count of younger loads),
// meets the other waves at the barrier, and issues the hidden copies of
// chunk it + D - 1 into the slot freed by chunk it - 1.
//
// The hand-counted wait assumes the issue order A(it + D - 1), barrier,
// B(it + D - 1) in every body: the compiler fences after each group keep
// it, and the weight pointer is not __restrict__, because loads through a
// restrict pointer count as invariant and may move across the fences. The
// loop always runs whole trips of D bodies (a body skipped on some path would
// make the compiler's own register waits as strict as that path's count):
// the up to D - 1 chunks past the end are multiplied into a tile that is
// never evaluated. Summation order per logit is that of the kernel above
// (steps ascending, MFMA in-step order), so results are bit-identical to it.
//
// Row-major heads (RM, H % 64 == 0): a chunk is two steps, i.e. one 128-byte
// segment of every row. A 16-row block of it takes two buffer loads, each
// covering 8 whole row segments (a load shaped like the MFMA operand, 16 rows
// x 64 bytes, streams at about half the rate): in load h, lane l holds row
// 8h + (l mod 8) of the block, 16-byte piece l / 16 + 4 ((l / 8) mod 2) of the
// segment. The operands of the chunk's two steps are then one DPP exchange of
// half rows away: lanes 8..15 of each 16-lane row of load 0 swap with lanes
// 0..7 of load 1 (row_ror:8 with a bank mask, one v_mov_b32_dpp per dword),
// after which load 0 holds step 0 (lane j + 16g: row j, piece g) and load 1
// step 1 (row j, piece 4 + g), exactly the tiled fragments. Rows past the
// table fall outside the load's descriptor range and read zeros. Two chunks
// of registers (D = 2) keep as many weight bytes in flight per wave as three
// one-step chunks do, and the running best of each lane lives in the LDS
// reduction arrays (read and written only when a tile ends), so the wave
// stays within the 256 registers of two waves per SIMD.

// hidden [M][nch] (16-byte chunks) -> fragments (st, b), 1 KiB each, ordered
// st * nbt + b: lane j + 16 g holds hidden row 16 b + j, chunk 4 st + g.
__global__ void __launch_bounds__(256)
    pack_hidden_frags(const uint4 *__restrict__ X, int M, int nch, int S, int nbt,
                      uint4 *__restrict__ out) {
  const int64_t total = (int64_t)S * nbt * kWave;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += step) {
    const int lane = (int)(e & (kWave - 1));
    const int64_t fr = e / kWave;
    const int b = (int)(fr % nbt);
    const int st = (int)(fr / nbt);
    const int row = b * 16 + (lane & 15);
    const int col = st * 4 + (lane >> 4);
    out[e] = (row < M && col < nch) ? X[(int64_t)row * nch + col] : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int NB, int RW, int KS, int D, int WV, int CP, bool RM = false>
__global__ void __launch_bounds__(WV * 64)
    gemm_argmax_ring(const uint4 *__restrict__ XP, const uint4 *WT, int M, int N, int S,
                     int nbt, int nch, RowSink sink) {
  constexpr int RBT = WV * RW;
  constexpr int TV = RBT * 16;
  constexpr int BF = KS * NB;                   // hidden fragments per chunk
  constexpr int PWB = (BF + WV - 1) / WV;       // hidden copies per wave per chunk
  constexpr int AL = RW * KS;                   // weight loads per wave per chunk
  static_assert(RM ? (KS == 2 && D >= 2 && D <= 4) : (D >= 3 && D <= 4), "ring depth");
  static_assert(RBT % 4 == 0, "whole 64-row tiles");
  __shared__ uint4 bs0[BF * 64];
  __shared__ uint4 bs1[BF * 64];
  __shared__ uint4 bs2[D > 2 ? BF * 64 : 1];
  __shared__ uint4 bs3[D > 3 ? BF * 64 : 1];
  __shared__ float red_v[WV * NB * 64];
  __shared__ int red_i[WV * NB * 64];
  __shared__ float f_val[NB * 16];
  __shared__ int64_t f_row[NB * 16];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4;
  const int m0 = blockIdx.y * NB * 16;
  const int gdx = gridDim.x;
  const int bx = blockIdx.x;
  const int by = blockIdx.y;
  const int nchunks = S / KS;
  const int ntiles = (N + TV - 1) / TV;
  const int my_tiles = bx < ntiles ? (ntiles - 1 - bx) / gdx + 1 : 0;
  const int total = my_tiles * nchunks;
  const int nrb = ((N + 63) / 64) * 4;

  auto bslot = [&](auto tag) __attribute__((always_inline)) -> uint4 * {
    constexpr int SL = decltype(tag)::value;
    if constexpr (SL == 0) return bs0;
    else if constexpr (SL == 1) return bs1;
    else if constexpr (SL == 2) return bs2;
    else return bs3;
  };

  uint4 ar[D][KS][RW];
  int a_t = bx, a_c = 0;
  // row-major: one descriptor per tile (rows past the table lie outside its
  // range and read zeros), the chunk's column offset as the scalar offset,
  // and per load the lane's offset within the tile: row 8h + (l mod 8) of
  // the wave's block rw, piece l / 16 + 4 ((l / 8) mod 2) of the segment.
  // These stay in registers for the whole kernel, so a chunk's loads cost
  // no per-load address arithmetic.
  const int64_t rowbytes = (int64_t)nch * 16;
  int rm_voff[2][RM ? RW : 1];
  if constexpr (RM) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rw = 0; rw < RW; ++rw)
        rm_voff[h][rw] = (int)(((wave * RW + rw) * 16 + 8 * h + (lane & 7)) * rowbytes) +
                         16 * ((lane >> 4) + 4 * ((lane >> 3) & 1));
  }
  auto rm_rsrc = [&](int tile) __attribute__((always_inline)) {
    const int64_t row0 = (int64_t)tile * TV;
    const int64_t left = ((int64_t)N - row0) * rowbytes;
    const int nrec = left <= 0 ? 0 : left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const char *>(WT) + row0 * rowbytes), (short)0, nrec,
        0x00020000);
  };
  __amdgpu_buffer_rsrc_t a_rs = rm_rsrc(bx);
  // tiled: one descriptor per tile over this wave's 64-row groups (groups
  // past the table read zeros, never reported); a chunk's fragments sit at
  // the chunk's scalar offset (c * KS + s) * 4 KiB plus a fixed lane offset,
  // so the loads need no per-load address arithmetic (the tiled ring ran
  // about 3% faster than with 64-bit addresses per load, same-box A/B)
  auto t_rsrc = [&](int tile) __attribute__((always_inline)) {
    const int64_t g0 = (int64_t)tile * (RBT / 4) + wave * (RW / 4);
    const int64_t left = ((int64_t)(nrb / 4) - g0) * S * 4096;
    const int64_t span = (int64_t)((RW + 3) / 4) * S * 4096;
    const int64_t n = left < span ? left : span;
    const int nrec = n <= 0 ? 0 : n > 0x7FFFFFFF ? 0x7FFFFFFF : (int)n;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const char *>(WT) + g0 * S * 4096), (short)0, nrec, 0x00020000);
  };
  __amdgpu_buffer_rsrc_t t_rs = t_rsrc(bx);
  // keep `own` in lanes 0..7 (swap_hi) or 8..15 (swap_lo) of each 16-lane
  // row and take the other half from `other` rotated by 8 lanes (row_ror:8)
  auto swap_hi = [](uint32_t own, uint32_t other) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)own, (int)other, 0x128, 0xF, 0xC, false);
  };
  auto swap_lo = [](uint32_t own, uint32_t other) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)own, (int)other, 0x128, 0xF, 0x3, false);
  };
  auto issue_a = [&](auto tag) __attribute__((always_inline)) {
    constexpr int SL = decltype(tag)::value;
    const int c = a_c;
    if constexpr (RM) {
      const __amdgpu_buffer_rsrc_t r = a_rs;
      if (++a_c == nchunks) {
        a_c = 0;
        a_t += gdx;
        a_rs = rm_rsrc(a_t);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int rw = 0; rw < RW; ++rw) {
          const u32x4_ring_t v = __builtin_amdgcn_raw_buffer_load_b128(r, rm_voff[h][rw], c * 128, CP);
          ar[SL][h][rw] = make_uint4(v.x, v.y, v.z, v.w);
        }
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t r = t_rs;
    if (++a_c == nchunks) {
      a_c = 0;
      a_t += gdx;
      t_rs = t_rsrc(a_t);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const u32x4_ring_t v = __builtin_amdgcn_raw_buffer_load_b128(
            r, lane * 16 + (rw / 4) * S * 4096 + (rw % 4) * 1024, (c * KS + s) * 4096, CP);
        ar[SL][s][rw] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
  };
  // hidden copies: one descriptor per chunk (its first fragment of this
  // pass), and per copy a scalar offset to fragment (s, nb) of the chunk,
  // which depends only on the wave (computed outside the loop)
  int b_c = 0;
  auto issue_b = [&](auto tag) __attribute__((always_inline)) {
    uint4 *base = bslot(tag);
    const int c = b_c;
    if (++b_c == nchunks) b_c = 0;
    const uint4 *fr = XP + ((int64_t)c * KS * nbt + by * NB) * kWave;
    __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)fr, (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int q = 0; q < PWB; ++q) {
      int f = wave + WV * q;
      f = f < BF ? f : BF - 1;                   // surplus copies repeat the last fragment
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, MTP_LDS(base + f * kWave), 16, lane * 16,
                                               ((f / NB) * nbt + f % NB) * 1024, 0, 0);
    }
  };

  f32x4_dma_t acc[RW][NB];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
  // running best (logit, row) of each lane's hidden row: registers, or for
  // row-major heads this lane's entries of the reduction arrays
  constexpr int NBR = RM ? 1 : NB;
  float bv[NBR];
  int bi[NBR];
#pragma unroll
  for (int nb = 0; nb < NBR; ++nb) {
    bv[nb] = 0.f;
    bi[nb] = -1;
  }
  if constexpr (RM) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      red_v[(wave * NB + nb) * kWave + lane] = 0.f;
      red_i[(wave * NB + nb) * kWave + lane] = -1;
    }
  }

  // prologue: chunks 0 .. D - 2, in the order A B A B ...
  issue_a(std::integral_constant<int, 0>{});
  asm volatile("" ::: "memory");
  issue_b(std::integral_constant<int, 0>{});
  asm volatile("" ::: "memory");
  if constexpr (D > 2) {
    issue_a(std::integral_constant<int, 1>{});
    asm volatile("" ::: "memory");
    issue_b(std::integral_constant<int, 1>{});
    asm volatile("" ::: "memory");
  }
  if constexpr (D > 3) {
    issue_a(std::integral_constant<int, 2>{});
    asm volatile("" ::: "memory");
    issue_b(std::integral_constant<int, 2>{});
    asm volatile("" ::: "memory");
  }
  int cur_t = bx, cur_c = 0;

  auto body = [&](auto tag) __attribute__((always_inline)) {
    constexpr int SL = decltype(tag)::value;
    constexpr int NX = (SL + D - 1) % D;
    issue_a(std::integral_constant<int, NX>{});
    asm volatile("" ::: "memory");
    // younger than chunk it's hidden copies: D - 2 whole chunks, then this
    // body's weight loads (the weights of chunk it are older still)
    wait_vmcnt<(D - 2) * (AL + PWB) + AL>();
    barrier_no_fence();
    issue_b(std::integral_constant<int, NX>{});
    asm volatile("" ::: "memory");
    if constexpr (RM) {
      // half-row exchange: loads 0 and 1 of each block become the operands
      // of steps 0 and 1 (row_ror:8 is its own inverse; the bank mask keeps
      // the other half of each 16-lane row)
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const uint4 l0 = ar[SL][0][rw], l1 = ar[SL][1][rw];
        ar[SL][0][rw] = make_uint4(swap_hi(l0.x, l1.x), swap_hi(l0.y, l1.y),
                                   swap_hi(l0.z, l1.z), swap_hi(l0.w, l1.w));
        ar[SL][1][rw] = make_uint4(swap_lo(l1.x, l0.x), swap_lo(l1.y, l0.y),
                                   swap_lo(l1.z, l0.z), swap_lo(l1.w, l0.w));
      }
    }
    const uint4 *Bf = bslot(tag);
    if constexpr (RM) {
      // operand B one fragment ahead: the LDS read of fragment f + 1 is in
      // flight while the MFMAs of fragment f run
      uint4 bnext = Bf[lane];
#pragma unroll
      for (int f = 0; f < KS * NB; ++f) {
        const uint4 b = bnext;
        if (f + 1 < KS * NB) bnext = Bf[(f + 1) * kWave + lane];
#pragma unroll
        for (int rw = 0; rw < RW; ++rw)
          acc[rw][f % NB] = mfma16_dma(ar[SL][f / NB][rw], b, acc[rw][f % NB]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 b = Bf[(s * NB + nb) * kWave + lane];
#pragma unroll
          for (int rw = 0; rw < RW; ++rw) acc[rw][nb] = mfma16_dma(ar[SL][s][rw], b, acc[rw][nb]);
        }
      }
    }
    if (++cur_c == nchunks) {
      const int tile = cur_t;
      cur_c = 0;
      cur_t += gdx;
      const int vbase = tile * TV + wave * RW * 16 + 4 * g;
      if constexpr (RM) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float cv = red_v[(wave * NB + nb) * kWave + lane];
          int ci = red_i[(wave * NB + nb) * kWave + lane];
#pragma unroll
          for (int rw = 0; rw < RW; ++rw) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = vbase + rw * 16 + r;
              const float z = acc[rw][nb][r];
              if (v < N && better_row(z, v, cv, ci)) {
                cv = z;
                ci = v;
              }
            }
            acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
          }
          red_v[(wave * NB + nb) * kWave + lane] = cv;
          red_i[(wave * NB + nb) * kWave + lane] = ci;
        }
      } else {
#pragma unroll
        for (int rw = 0; rw < RW; ++rw) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = vbase + rw * 16 + r;
              const float z = acc[rw][nb][r];
              if (v < N && better_row(z, v, bv[nb], bi[nb])) {
                bv[nb] = z;
                bi[nb] = v;
              }
            }
            acc[rw][nb] = f32x4_dma_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
  };

  for (int it = 0; it < total; it += D) {
    body(std::integral_constant<int, 0>{});
    body(std::integral_constant<int, 1>{});
    if constexpr (D > 2) body(std::integral_constant<int, 2>{});
    if constexpr (D > 3) body(std::integral_constant<int, 3>{});
  }
  wait_vmcnt<0>();
  __syncthreads();

  if constexpr (!RM) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      red_v[(wave * NB + nb) * kWave + lane] = bv[nb];
      red_i[(wave * NB + nb) * kWave + lane] = bi[nb];
    }
  }
  __syncthreads();
  merge_candidates<NB, WV>(red_v, red_i, tid, f_val, f_row);
  __syncthreads();
  const int mcount = M - m0 < NB * 16 ? M - m0 : NB * 16;
  finish_rows(sink, f_val, f_row, m0, mcount);
}

// Padded sizes of the tiled layout.
int64_t tiled_rows(int64_t rows) { return (rows + 63) / 64 * 64; }
int tiled_cols(int H) { return (H + 127) / 128 * 128; }

template <int NB, int RW, int KS, int NBUF, int WV, int CP, bool FP8 = false, bool FP4 = false,
          bool RM = false, int PS = 1>
static hipError_t launch_dma_cfg(const DmaLaunch &L) {
  constexpr int TV = WV * RW * 16;
  const int64_t ntiles = (L.N + TV - 1) / TV;
  const int gx = (int)(ntiles < L.max_blocks_x ? ntiles : L.max_blocks_x);
  const int gy = (L.M + NB * 16 - 1) / (NB * 16);
  return launch_call_kernel((gemm_argmax_dma<NB, RW, KS, NBUF, WV, CP, FP8, FP4, RM, PS>),
                            dim3(gx, gy), dim3(WV * 64), L.stream, true, true,
                            (const uint4 *)L.X, (const uint4 *)L.WT, L.M, (int)L.N, L.nch, L.S,
                            L.sink, L.scales, L.nphase);
}

// Hidden-row blocks per pass: M rounds up to an instantiated count (at most
// 160 rows per pass; more rows take several passes over the table).
static const int kDmaNbSteps[] = {1, 2, 3, 4, 6, 8, 10};

int dma_nb_for(int M) {
  const int need = (M + 15) / 16;
  for (int n : kDmaNbSteps)
    if (n >= need) return n;
  return 10;
}

// Instantiated shapes (measured on MI355X at the workload shapes; none spills
// registers, every one fits the 160 KiB LDS). Non-temporal weight copies
// (CP = 2) stream 6.7 TB/s where default-policy copies reach 6.0 TB/s.
template <int NB, int RW, int KS, int D, int WV, int CP, bool RM = false>
static hipError_t launch_ring_cfg(const DmaLaunch &L) {
  constexpr int TV = WV * RW * 16;
  const int64_t ntiles = (L.N + TV - 1) / TV;
  const int gx = (int)(ntiles < L.max_blocks_x ? ntiles : L.max_blocks_x);
  const int gy = (L.M + NB * 16 - 1) / (NB * 16);
  const int nbt = gy * NB;
  const int64_t elems = (int64_t)L.S * nbt * kWave;
  const int pblocks = (int)(elems / 256 + 1 < 1024 ? elems / 256 + 1 : 1024);
  hipError_t e = launch_call_kernel(pack_hidden_frags, dim3(pblocks), dim3(256), L.stream, true,
                                    false, (const uint4 *)L.X, L.M, L.nch, L.S, nbt,
                                    (uint4 *)L.stage);
  if (e != hipSuccess) return e;
  return launch_call_kernel((gemm_argmax_ring<NB, RW, KS, D, WV, CP, RM>), dim3(gx, gy),
                            dim3(WV * 64), L.stream, false, true, (const uint4 *)L.stage,
                            (const uint4 *)L.WT, L.M, (int)L.N, L.S, nbt, L.nch, L.sink);
}

// Staging bytes of the wide passes (the packed hidden block), 0 for M <= 128.
size_t ring_stage_bytes(int M, int H) {
  if (dma_nb_for(M) != 10) return 0;
  const size_t nbt = (size_t)10 * ((M + 159) / 160);
  return (size_t)(tiled_cols(H) / 32) * nbt * 1024;
}

hipError_t launch_dma(const DmaLaunch &L, int nb) {
  constexpr int NT = 2;
  // wide passes: the register-ring kernel (M = 160 at H = 5,120 on MI355X:
  // 415 us against 489 us, bit-identical results) when staging is given
  if (nb == 10 && L.stage) return launch_ring_cfg<10, 4, 1, 3, 8, NT>(L);
  switch (nb) {
    case 1: return launch_dma_cfg<1, 1, 2, 3, 8, NT>(L);  // 3 slots: 80.3 against 82.3 us
    case 2: return launch_dma_cfg<2, 2, 2, 4, 8, NT>(L);
    case 3: return launch_dma_cfg<3, 2, 2, 3, 8, NT>(L);
    case 4: return launch_dma_cfg<4, 2, 2, 3, 8, NT>(L);
    case 6: return launch_dma_cfg<6, 4, 1, 3, 8, NT>(L);
    case 8: return launch_dma_cfg<8, 4, 1, 3, 8, NT>(L);
    case 10: return launch_dma_cfg<10, 4, 1, 3, 8, NT>(L);
    default: return hipErrorInvalidValue;
  }
}

// Row-major tables and heads (H % 64 == 0): the same kernel with each weight
// copy holding 8 whole 128-byte row segments (two 32-column steps per chunk).
// A row-major copy of 16 rows x 64 bytes, the MFMA operand's own shape, streams
// at half the rate on MI355X (3.8 against 7.1 TB/s for copy-only loops over
// 248,320 x 5,120), so every shape takes two-step chunks; 96 to 160 hidden rows
// use 256-row tiles to fit their two-step chunks in three LDS slots.
bool dma_rm_ok(int H) { return H % 64 == 0; }

// PSMAX: column segments (workgroup phases) this pass takes on rows a multiple
// of 4 KiB apart; the segment sums cost RW * NB * 4 registers each.
template <int NB, int RW, int NBUF, int PSMAX>
static hipError_t launch_rm(const DmaLaunch &L) {
  constexpr int NT = 2;
  if constexpr (PSMAX > 1) {
    if (L.nphase > 1) return launch_dma_cfg<NB, RW, 2, NBUF, 8, NT, false, false, true, PSMAX>(L);
  }
  return launch_dma_cfg<NB, RW, 2, NBUF, 8, NT, false, false, true, 1>(L);
}

hipError_t launch_dma_rm(const DmaLaunch &L, int nb) {
  // wide passes with staging: the register ring on row-major rows
  if (nb == 10 && L.stage) return launch_ring_cfg<10, 4, 2, 2, 8, 2, true>(L);
  switch (nb) {
    case 1: return launch_rm<1, 1, 3, 8>(L);
    case 2: return launch_rm<2, 2, 4, 4>(L);
    case 3: return launch_rm<3, 2, 3, 4>(L);
    case 4: return launch_rm<4, 2, 3, 2>(L);
    case 6: return launch_rm<6, 2, 3, 2>(L);
    case 8: return launch_rm<8, 2, 3, 1>(L);
    case 10: return launch_rm<10, 2, 3, 1>(L);
    default: return hipErrorInvalidValue;
  }
}

// FP8 tables: hidden-row blocks per pass 1..4 (up to 64 rows; more rows take
// further passes). A 16-row pass copies chunks of two step pairs (KS = 4):
// fp8 fragments carry half the bytes of bf16 ones, and one-pair chunks keep
// too few bytes in flight per CU to stream the table (45 us against 48 us for
// a 65,536 x 4,096 table on MI355X); wider passes keep one-pair chunks.
int dma_nb_for_fp8(int M) {
  const int need = (M + 15) / 16;
  return need < 4 ? need : 4;
}

// MXFP4 tiled tables (columns padded to a multiple of 256): hidden-row blocks
// per pass 1..4. With a quarter of the bf16 bytes per step, chunks hold one
// or two step groups (4 or 8 steps). Shapes from a sweep on MI355X (65,536
// rows; all bit-identical): 16 rows at H = 4,096 run 29.9 us with 128-row
// tiles, 8-step chunks and two workgroups per CU, against 31.8 us with
// 256-row tiles; 32 rows at H = 5,120 run 40.0 us with 4-step chunks in four
// slots, against 41.0 us with 8-step chunks in three.
int dma_nb_for_fp4(int M) {
  const int need = (M + 15) / 16;
  return need < 4 ? need : 4;
}

int tiled_cols_fp4(int H) { return (H + 255) / 256 * 256; }

hipError_t launch_dma_fp4(const DmaLaunch &L, int nb) {
  constexpr int NT = 2;
  switch (nb) {
    case 1: return launch_dma_cfg<1, 1, 8, 3, 8, NT, false, true>(L);
    case 2: return launch_dma_cfg<2, 2, 4, 4, 8, NT, false, true>(L);
    case 3: return launch_dma_cfg<3, 4, 4, 3, 8, NT, false, true>(L);
    case 4: return launch_dma_cfg<4, 4, 4, 3, 8, NT, false, true>(L);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dma_fp8(const DmaLaunch &L, int nb) {
  constexpr int NT = 2;
  switch (nb) {
    case 1: return launch_dma_cfg<1, 1, 4, 3, 8, NT, true>(L);
    case 2: return launch_dma_cfg<2, 2, 2, 4, 8, NT, true>(L);
    case 3: return launch_dma_cfg<3, 2, 2, 4, 8, NT, true>(L);
    case 4: return launch_dma_cfg<4, 2, 2, 4, 8, NT, true>(L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
