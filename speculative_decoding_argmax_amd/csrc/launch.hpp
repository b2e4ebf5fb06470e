// Internal launchers of the HIP kernels (host side). Not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mtp {

// Timing of one call (a measurement aid, mtp_time_next_call): when set, the
// next draft or verify call of this thread launches its first kernel with
// `start` and its last with `stop` through hipExtLaunchKernel, which stamps
// the events with the dispatches' own start and end times (no marker packets
// in the stream). The request is cleared by the launch that takes `stop`.
struct CallTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
CallTiming &call_timing();

// Launch a draft / verify kernel; `first` / `last`: the call's first / last
// kernel (for the timing request above).
template <typename K, typename... Args>
hipError_t launch_call_kernel(K kernel, dim3 grid, dim3 block, hipStream_t stream, bool first,
                              bool last, Args... args) {
  CallTiming &t = call_timing();
  if (t.start || t.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, first ? t.start : nullptr,
                          last ? t.stop : nullptr, 0, args...);
    if (last) t = CallTiming{};
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  }
  return hipGetLastError();
}

struct ValuLaunch {
  const void *X;     // hidden [M][H] bf16
  const void *W;     // table / head [N][H] bf16
  int M;
  int64_t N;
  int nch;           // H / 8 (16-byte chunks per row)
  int max_blocks_x;  // cap on workgroups along the row dimension
  bool prefetch;     // prefetching variant (fewer rows per iteration)
  RowSink sink;
  hipStream_t stream;
  // gathered candidates: row i is head row gather_ids[i] of gather_V rows
  // (W is then the head); nullptr for a packed table
  const int32_t *gather_ids = nullptr;
  int64_t gather_V = 0;
};

// Chunks-per-lane instantiation covering nch 16-byte chunks (0: too wide).
int valu_ncl_for(int nch);
// Hidden rows per workgroup for M rows at that width.
int valu_rows_for(int M, int ncl);
// Workgroups a launch will use (the ticket counts them).
int valu_total_blocks(const ValuLaunch &L, int mr, int ncl);
hipError_t launch_valu(const ValuLaunch &L, int mr, int ncl);

struct MfmaLaunch {
  const void *X;     // hidden [M][H] bf16
  const void *W;     // table / head [N][H] bf16
  int M;
  int64_t N;
  int nch;           // H / 8
  int max_blocks_x;  // cap on workgroups along the table
  RowSink sink;
  hipStream_t stream;
};

// Column blocks of 16 hidden rows per pass for M rows.
int mfma_nb_for(int M);
hipError_t launch_mfma(const MfmaLaunch &L, int nb);

struct DmaLaunch {
  const void *X;     // hidden [M][H] bf16, row-major
  const void *WT;    // table in the 64-row tiled layout (row-major for launch_dma_rm)
  int M;
  int64_t N;         // table rows (before padding)
  int nch;           // H / 8
  int S;             // 32-column steps per padded row (tiled_cols(H) / 32; H / 32 row-major)
  int max_blocks_x;
  RowSink sink;
  hipStream_t stream;
  const float *scales = nullptr;  // fp8 tables: row scales [N]
  void *stage = nullptr;          // wide passes: packed hidden block (ring_stage_bytes)
  int nphase = 1;                 // row-major: workgroup chunk phases (1: none)
};

int64_t tiled_rows(int64_t rows);
int tiled_cols(int H);
int dma_nb_for(int M);
hipError_t launch_dma(const DmaLaunch &L, int nb);
size_t ring_stage_bytes(int M, int H);
// Row-major tables and heads through the same kernel (H % 64 == 0).
bool dma_rm_ok(int H);
hipError_t launch_dma_rm(const DmaLaunch &L, int nb);
int dma_nb_for_fp8(int M);
hipError_t launch_dma_fp8(const DmaLaunch &L, int nb);
int dma_nb_for_fp4(int M);
int tiled_cols_fp4(int H);
hipError_t launch_dma_fp4(const DmaLaunch &L, int nb);
hipError_t launch_pack_tiled_mxfp4(const void *head, int64_t V, int H, const int32_t *ids,
                                   int64_t C, void *tiled, uint8_t *tscales, int rule,
                                   int num_cus, hipStream_t stream);
hipError_t launch_pack_tiled_fp8(const void *head, int64_t V, int H, const int32_t *ids,
                                 int64_t C, void *tiled, float *scales, int num_cus,
                                 hipStream_t stream);
hipError_t launch_pack_tiled(const void *head, int64_t V, int nch, const int32_t *ids,
                             int64_t C, int S, void *tiled, int num_cus, hipStream_t stream);

hipError_t launch_pack(const void *head, int64_t V, int nch, const int32_t *ids, int64_t C,
                       void *table, int num_cus, hipStream_t stream);

struct Fp8Launch {
  const void *X;        // hidden [M][H] bf16
  const void *Q;        // E4M3 codes [N][H]
  const float *scales;  // [N] row scales (powers of two)
  int M;
  int64_t N;
  int ncq;              // H / 16 (16-byte code chunks per row)
  int max_blocks_x;
  RowSink sink;
  hipStream_t stream;
  // gathered candidates: candidate i is row gather_ids[i] of a head of
  // gather_V rows (Q and scales are then the head's); nullptr for a table
  const int32_t *gather_ids = nullptr;
  int64_t gather_V = 0;
};

// Code chunks per lane that have an instantiation (0: too wide).
int fp8_ncl_for(int ncq);
int fp8_rows_for(int M, int ncl);
hipError_t launch_fp8(const Fp8Launch &L, int mr, int ncl);
hipError_t launch_pack_fp8(const void *head, int64_t V, int H, const int32_t *ids, int64_t C,
                           void *q, float *scales, int num_cus, hipStream_t stream);
hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t stream);

struct Fp4Launch {
  const void *X;          // hidden [M][H] bf16
  const void *Q;          // MXFP4 codes [N][H/2]
  const uint8_t *scales;  // [N][H/32] E8M0 block scales
  int M;
  int64_t N;
  int nblk;               // H / 32 (blocks per row)
  int max_blocks_x;
  RowSink sink;
  hipStream_t stream;
  // gathered candidates: candidate i is row gather_ids[i] of a head of
  // gather_V rows (Q and scales are then the head's); nullptr for a table
  const int32_t *gather_ids = nullptr;
  int64_t gather_V = 0;
};

// Blocks per lane that have an instantiation (0: too wide).
int fp4_ncl_for(int nblk);
int fp4_rows_for(int M, int ncl);
hipError_t launch_fp4(const Fp4Launch &L, int mr, int ncl);
hipError_t launch_pack_mxfp4(const void *head, int64_t V, int H, const int32_t *ids, int64_t C,
                             void *q, uint8_t *scales, int rule, int num_cus,
                             hipStream_t stream);

// Streaming-read reference (probe.hip): sink words written per call, at most.
constexpr int kStreamSinkWords = 8192;
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int cus,
                              hipStream_t stream);
// Atomic round-trip reference (probe.hip).
hipError_t launch_atomic_chain(uint32_t *words, int wgs, int iters, int same,
                               unsigned long long *ticks, hipStream_t stream);

}  // namespace mtp
