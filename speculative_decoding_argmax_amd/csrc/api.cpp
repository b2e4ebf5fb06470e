// C ABI of the MTP draft / verify library: argument checks, path selection and
// launch. Every check that can fail runs before anything is enqueued.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <new>
#include <cstdint>
#include <cstring>

#include "launch.hpp"
#include "mtp.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local mtp::CallTiming g_call_timing;

mtp_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MTP_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device (cached per device).
hipError_t current_cus(int *cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *cus = v;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) n = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return hipSuccess;
}

// Workspace of a call with M hidden rows: the ticket header and the regions
// of the grouped finish (which also hold the one-level finish's M keys).
size_t rows_workspace_bytes(int64_t M) {
  return mtp::kWsHeader + (size_t)mtp::kFinishGroups * mtp::finish_group_stride(M);
}

// The least a call accepts: the ticket header and M keys (one-level finish).
size_t min_rows_workspace_bytes(int64_t M) {
  const size_t keys = (size_t)M * 8;
  return mtp::kWsHeader + ((keys + 255) / 256) * 256;
}

// The grouped finish, when the workspace holds its regions and each
// workgroup of the launch streams less than kGroupedFinishBytes of the table:
// such workgroups reach the finish within a few microseconds of each other,
// and hundreds of same-address atomics then queue (measured on MI355X,
// same-box A/B: MXFP4 M = 1 drafts at 32,768 and 65,536 x 2,048 rows 13.9 ->
// 10.4 and 18.2 -> 15.6 us, bf16 at 16,384 rows 14.7 -> 13.7 us, fp8 at
// 32,768 rows 15.3 -> 14.5 us, bf16 at 24,576 rows (384 KiB per workgroup)
// 18.8 -> 18.4 us; at 512 KiB the two finishes time the same, bf16 at
// 32,768 rows 23.0 us; beyond that the extra round trip costs 0.3-0.7 us,
// e.g. 27.7 -> 28.2 us at 32,768 x 2,560 and 40.6 -> 41.3 us for the bf16
// 65,536-row draft).
constexpr double kGroupedFinishBytes = 448.0 * 1024.0;

void choose_finish(mtp::RowSink &s, size_t ws_bytes, double table_bytes, int64_t workgroups) {
  if (ws_bytes >= rows_workspace_bytes(s.M) && workgroups > 0 &&
      table_bytes / (double)workgroups < kGroupedFinishBytes) {
    s.groups = mtp::kFinishGroups;
  }
}

// Tiled calls with more than 128 hidden rows also stage the packed hidden
// block in the workspace. It starts past the largest counter region any call
// can use (MTP_MAX_ROWS keys), so the scratch it leaves behind never lies
// where another call on the same workspace expects zeroed keys; the start is
// rounded up to 256 bytes (the workspace itself is only 8-byte aligned,
// hence the slack).
size_t stage_offset() { return rows_workspace_bytes(MTP_MAX_ROWS); }

size_t call_workspace_bytes(int64_t M, int H) {
  const size_t b = mtp::ring_stage_bytes((int)M, H);
  return b ? stage_offset() + b + 256 : rows_workspace_bytes(M);
}

void *stage_ptr(void *ws) {
  const uintptr_t p = (uintptr_t)ws + stage_offset();
  return (void *)((p + 255) & ~(uintptr_t)255);
}

// Row-major calls with more than 128 hidden rows use the staging area when
// the workspace holds it (the size queries include it), and otherwise run
// without it on the LDS-fed kernel.
void *rows_stage(void *ws, size_t ws_bytes, int64_t M, int H) {
  if (mtp::ring_stage_bytes((int)M, H) == 0 || ws_bytes < call_workspace_bytes(M, H))
    return nullptr;
  return stage_ptr(ws);
}

bool shape_ok(int64_t M, int64_t N, int64_t H) {
  return M >= 1 && M <= MTP_MAX_ROWS && N >= 1 && N <= INT32_MAX && H >= 8 &&
         H <= MTP_MAX_HIDDEN && H % 8 == 0;
}

mtp_status check_cfg(const mtp_config *cfg) {
  if (!cfg) return MTP_OK;
  if (cfg->path < MTP_PATH_AUTO || cfg->path > MTP_PATH_MFMA) return MTP_ERR_INVALID_ARG;
  if (cfg->blocks_per_cu < 0 || cfg->blocks_per_cu > 16) return MTP_ERR_INVALID_ARG;
  for (int r : cfg->reserved)
    if (r != 0) return MTP_ERR_INVALID_ARG;
  return MTP_OK;
}

// Score M hidden rows against N table rows and finish through `sink`.
// Path: the vector-ALU kernel while one pass keeps every hidden row's slice in
// registers (few rows), the matrix cores beyond: fed by LDS DMA from the rows
// when H % 64 == 0, else by the register-staged kernel.
// Gathered candidates (gather_ids != nullptr: candidate i is head row
// gather_ids[i]) run on the vector-ALU kernel only.
mtp_status run_rows(const mtp_bf16 *X, int M, int H, const mtp_bf16 *W, int64_t N,
                    mtp::RowSink sink, size_t ws_bytes, hipStream_t stream,
                    const mtp_config *cfg, void *stage, const int32_t *gather_ids = nullptr,
                    int64_t gather_V = 0) {
  const double table_bytes = (double)N * H * 2;
  const int nch = H / 8;
  const int ncl = mtp::valu_ncl_for(nch);
  int path = cfg ? cfg->path : MTP_PATH_AUTO;
  if (gather_ids) {
    if (path == MTP_PATH_MFMA) return MTP_ERR_UNSUPPORTED;
    path = MTP_PATH_VALU;
  }
  if (path == MTP_PATH_AUTO)
    path = (ncl != 0 && mtp::valu_rows_for(M, ncl) >= M) ? MTP_PATH_VALU : MTP_PATH_MFMA;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  if (path == MTP_PATH_VALU) {
    if (ncl == 0) return MTP_ERR_UNSUPPORTED;
    // Resident workgroups per CU, from a same-box sweep of 1-4 on MI355X
    // (65,536 rows, M = 1, 2, 4, 8, H = 1,024 .. 4,096, and checks at 5,120
    // and 8,192): one for rows of 3 to 8 chunks per lane (H 2,048 .. 4,096;
    // at 4,096 one beats two, 83.1 -> 78.3 us at M = 1), two when a pass holds
    // 8 hidden rows there (H = 2,048, M = 8: 69.0 -> 53.3 us). Short rows (at
    // most 2 chunks, H <= 1,024) keep too little in flight with one: two, four
    // with 8 rows per pass (29.0 -> 23.0 us at M = 1, 59.8 -> 36.1 us at
    // M = 8). Wider rows than 8 chunks take two (H = 8,192: 83.0 against
    // 85.4 us with one; even at 5,120).
    const int mr_v = mtp::valu_rows_for(M, ncl);
    const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu
                       : ncl <= 2                    ? (mr_v >= 8 ? 4 : 2)
                       : ncl <= 8                    ? (mr_v >= 8 ? 2 : 1)
                                                     : 2;
    choose_finish(sink, ws_bytes, table_bytes, (int64_t)per_cu * cus);
    mtp::ValuLaunch L;
    L.X = X;
    L.W = W;
    L.M = M;
    L.N = N;
    L.nch = nch;
    L.max_blocks_x = per_cu * cus;
    L.prefetch = true;
    L.sink = sink;
    L.stream = stream;
    L.gather_ids = gather_ids;
    L.gather_V = gather_V;
    e = mtp::launch_valu(L, mtp::valu_rows_for(M, ncl), ncl);
  } else if (mtp::dma_rm_ok(H)) {
    // matrix cores fed by LDS DMA straight from the row-major rows
    const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu : 1;
    choose_finish(sink, ws_bytes, table_bytes, (int64_t)per_cu * cus);
    mtp::DmaLaunch L;
    L.X = X;
    L.WT = W;
    L.M = M;
    L.N = N;
    L.nch = nch;
    L.S = H / 32;
    L.max_blocks_x = per_cu * cus;
    L.sink = sink;
    L.stream = stream;
    L.stage = stage;
    // rows a multiple of 4 KiB apart: stagger the workgroups over 8 chunk
    // phases (the arithmetic of every logit is the same either way)
    L.nphase = ((int64_t)H * 2) % 4096 == 0 ? 8 : 1;
    e = mtp::launch_dma_rm(L, mtp::dma_nb_for(M));
  } else {
    // widths that are not a multiple of 64: register-staged matrix-core kernel
    const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu : 2;
    choose_finish(sink, ws_bytes, table_bytes, (int64_t)per_cu * cus);
    mtp::MfmaLaunch L;
    L.X = X;
    L.W = W;
    L.M = M;
    L.N = N;
    L.nch = nch;
    L.max_blocks_x = per_cu * cus;
    L.sink = sink;
    L.stream = stream;
    e = mtp::launch_mfma(L, mtp::mfma_nb_for(M));
  }
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

// Score M hidden rows against N rows of a tiled table.
mtp_status run_rows_tiled(const mtp_bf16 *X, int M, int H, const void *WT, int64_t N,
                          mtp::RowSink sink, void *ws, size_t ws_bytes, hipStream_t stream,
                          const mtp_config *cfg) {
  if (cfg && cfg->path == MTP_PATH_VALU) return MTP_ERR_UNSUPPORTED;
  const bool stage = mtp::ring_stage_bytes(M, H) != 0;
  if (ws_bytes < (stage ? call_workspace_bytes(M, H) : min_rows_workspace_bytes(M)))
    return MTP_ERR_WORKSPACE;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu : 1;
  choose_finish(sink, ws_bytes, (double)mtp::tiled_rows(N) * mtp::tiled_cols(H) * 2,
                (int64_t)per_cu * cus);
  mtp::DmaLaunch L;
  L.X = X;
  L.WT = WT;
  L.M = M;
  L.N = N;
  L.nch = H / 8;
  L.S = mtp::tiled_cols(H) / 32;
  L.max_blocks_x = per_cu * cus;
  L.sink = sink;
  L.stream = stream;
  L.stage = stage ? stage_ptr(ws) : nullptr;
  e = mtp::launch_dma(L, mtp::dma_nb_for(M));
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

size_t tiled_bytes_of(int64_t rows, int H) {
  if (rows < 1 || rows > INT32_MAX || H < 8 || H > MTP_MAX_HIDDEN || H % 8 != 0) return 0;
  return (size_t)mtp::tiled_rows(rows) * (size_t)mtp::tiled_cols(H) * 2;
}

mtp_status check_draft_args(const mtp_bf16 *hidden, int M, int H, const void *table,
                            const int32_t *ids, int64_t C, const int32_t *out_ids,
                            const float *out_logit, const void *ws, size_t ws_bytes,
                            const mtp_config *cfg) {
  if (!hidden || !table || !out_ids) return MTP_ERR_INVALID_ARG;
  if (!shape_ok(M, C, H)) return MTP_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(table, 16) || !aligned(out_ids, 4) ||
      (ids && !aligned(ids, 4)) || (out_logit && !aligned(out_logit, 4)))
    return MTP_ERR_INVALID_ARG;
  mtp_status st = check_cfg(cfg);
  if (st != MTP_OK) return st;
  if (!ws || !aligned(ws, 8)) return MTP_ERR_WORKSPACE;
  if (ws_bytes < min_rows_workspace_bytes(M)) return MTP_ERR_WORKSPACE;
  return MTP_OK;
}

mtp::RowSink draft_sink(void *ws, const int32_t *ids, int32_t *out_ids, float *out_logit, int M) {
  mtp::RowSink s;
  std::memset(&s, 0, sizeof s);
  s.ticket = (uint32_t *)ws;
  s.keys = (unsigned long long *)((char *)ws + mtp::kWsHeader);
  s.groups = 1;
  s.ids = ids;
  s.out_ids = out_ids;
  s.out_logit = out_logit;
  s.M = M;
  s.B = 0;
  s.k = -1;
  return s;
}

// Verify arguments other than the workspace.
mtp_status check_verify_io(const mtp_bf16 *hidden, int B, int k, int H, const void *head,
                           int64_t V, const int32_t *draft, const int32_t *out_argmax,
                           const float *out_logit, const int32_t *out_accept,
                           const int32_t *out_tokens) {
  if (!hidden || !head || !out_argmax || !out_accept || !out_tokens) return MTP_ERR_INVALID_ARG;
  if (B < 1 || k < 0 || k > MTP_MAX_K) return MTP_ERR_INVALID_ARG;
  if (k > 0 && !draft) return MTP_ERR_INVALID_ARG;
  const int64_t M = (int64_t)B * (k + 1);
  if (!shape_ok(M, V, H)) return MTP_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(head, 16) || !aligned(out_argmax, 4) ||
      !aligned(out_accept, 4) || !aligned(out_tokens, 4) || (draft && !aligned(draft, 4)) ||
      (out_logit && !aligned(out_logit, 4)))
    return MTP_ERR_INVALID_ARG;
  return MTP_OK;
}

mtp_status check_verify_args(const mtp_bf16 *hidden, int B, int k, int H, const void *head,
                             int64_t V, const int32_t *draft, const int32_t *out_argmax,
                             const float *out_logit, const int32_t *out_accept,
                             const int32_t *out_tokens, const void *ws, size_t ws_bytes,
                             const mtp_config *cfg) {
  mtp_status st = check_verify_io(hidden, B, k, H, head, V, draft, out_argmax, out_logit,
                                  out_accept, out_tokens);
  if (st != MTP_OK) return st;
  const int64_t M = (int64_t)B * (k + 1);
  st = check_cfg(cfg);
  if (st != MTP_OK) return st;
  if (!ws || !aligned(ws, 8)) return MTP_ERR_WORKSPACE;
  if (ws_bytes < min_rows_workspace_bytes(M)) return MTP_ERR_WORKSPACE;
  return MTP_OK;
}

mtp::RowSink verify_sink(void *ws, int B, int k, const int32_t *draft, int32_t *out_argmax,
                         float *out_logit, int32_t *out_accept, int32_t *out_tokens) {
  mtp::RowSink s;
  std::memset(&s, 0, sizeof s);
  s.ticket = (uint32_t *)ws;
  s.keys = (unsigned long long *)((char *)ws + mtp::kWsHeader);
  s.groups = 1;
  s.ids = nullptr;
  s.out_ids = out_argmax;
  s.out_logit = out_logit;
  s.M = B * (k + 1);
  s.B = B;
  s.k = k;
  s.draft = draft;
  s.out_accept = out_accept;
  s.out_tokens = out_tokens;
  return s;
}

// ---- Scratch of the allocation-free verify ---------------------------------
//
// mtp_verify_accept_noalloc keeps its workspace (ticket header + one 64-bit key
// per hidden row, the layout mtp_verify_accept uses) in this file-scope device
// array instead of a caller-provided buffer. Every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address is taken once per device with hipGetSymbolAddress (that device
// current) and only that address is passed to kernels.
constexpr size_t kScratchBytes =
    mtp::kWsHeader + (((size_t)MTP_NOALLOC_MAX_ROWS * 8 + 255) / 256) * 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_dev[kMaxDevices];

// Device address of the current device's scratch (looked up on first use).
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

static_assert(kScratchBytes == 8448, "the size mtp.h states for the scratch array");

}  // namespace

mtp::CallTiming &mtp::call_timing() { return g_call_timing; }

extern "C" {

const char *mtp_status_string(mtp_status status) {
  switch (status) {
    case MTP_OK: return "MTP_OK";
    case MTP_ERR_INVALID_ARG: return "MTP_ERR_INVALID_ARG: null pointer, size out of range or misaligned pointer";
    case MTP_ERR_UNSUPPORTED: return "MTP_ERR_UNSUPPORTED: shape or configuration not handled";
    case MTP_ERR_WORKSPACE: return "MTP_ERR_WORKSPACE: workspace missing or too small";
    case MTP_ERR_IDS: return "MTP_ERR_IDS: candidate ids not strictly ascending in [0, V)";
    case MTP_ERR_HIP: return "MTP_ERR_HIP: HIP call or kernel launch failed";
  }
  return "unknown mtp_status";
}

int mtp_last_hip_error(void) { return g_last_hip_error; }

void mtp_time_next_call(hipEvent_t start, hipEvent_t stop) {
  g_call_timing.start = start;
  g_call_timing.stop = stop;
}

int mtp_version(void) { return 100; }

mtp_status mtp_validate_ids(const int32_t *ids_host, int64_t C, int64_t V) {
  if (!ids_host || C <= 0 || V <= 0) return MTP_ERR_INVALID_ARG;
  for (int64_t i = 0; i < C; ++i) {
    if (ids_host[i] < 0 || ids_host[i] >= V) return MTP_ERR_IDS;
    if (i > 0 && ids_host[i] <= ids_host[i - 1]) return MTP_ERR_IDS;
  }
  return MTP_OK;
}

size_t mtp_draft_workspace_bytes(int M, int64_t C, int H) {
  if (!shape_ok(M, C, H)) return 0;
  return call_workspace_bytes(M, H);
}

size_t mtp_verify_workspace_bytes(int B, int k, int64_t V, int H) {
  if (B < 1 || k < 0 || k > MTP_MAX_K) return 0;
  const int64_t M = (int64_t)B * (k + 1);
  if (!shape_ok(M, V, H)) return 0;
  return call_workspace_bytes(M, H);
}

mtp_status mtp_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || ws_bytes == 0 || ws_bytes % 8 != 0 || !aligned(ws, 8)) return MTP_ERR_INVALID_ARG;
  hipError_t e = mtp::launch_fill_zero(ws, ws_bytes, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_pack_candidates(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                               int64_t C, mtp_bf16 *table, hipStream_t stream) {
  if (!head || !ids || !table) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || C < 1 || C > INT32_MAX || H < 8 || H > MTP_MAX_HIDDEN ||
      H % 8 != 0)
    return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(table, 16) || !aligned(ids, 4)) return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack(head, V, H / 8, ids, C, table, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_cfg(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *table,
                                const int32_t *ids, int64_t C, int32_t *out_ids,
                                float *out_logit, void *ws, size_t ws_bytes, hipStream_t stream,
                                const mtp_config *cfg) {
  mtp_status st =
      check_draft_args(hidden, M, H, table, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  return run_rows(hidden, M, H, table, C, draft_sink(ws, ids, out_ids, out_logit, M), ws_bytes,
                  stream, cfg, rows_stage(ws, ws_bytes, M, H));
}

mtp_status mtp_draft_argmax(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *table,
                            const int32_t *ids, int64_t C, int32_t *out_ids, float *out_logit,
                            void *ws, size_t ws_bytes, hipStream_t stream) {
  return mtp_draft_argmax_cfg(hidden, M, H, table, ids, C, out_ids, out_logit, ws, ws_bytes,
                              stream, nullptr);
}

mtp_status mtp_verify_accept_cfg(const mtp_bf16 *hidden, int B, int k, int H,
                                 const mtp_bf16 *head, int64_t V, const int32_t *draft,
                                 int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                 int32_t *out_tokens, void *ws, size_t ws_bytes,
                                 hipStream_t stream, const mtp_config *cfg) {
  mtp_status st = check_verify_args(hidden, B, k, H, head, V, draft, out_argmax, out_logit,
                                    out_accept, out_tokens, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  return run_rows(hidden, B * (k + 1), H, head, V,
                  verify_sink(ws, B, k, draft, out_argmax, out_logit, out_accept, out_tokens),
                  ws_bytes, stream, cfg, rows_stage(ws, ws_bytes, (int64_t)B * (k + 1), H));
}

mtp_status mtp_verify_accept(const mtp_bf16 *hidden, int B, int k, int H, const mtp_bf16 *head,
                             int64_t V, const int32_t *draft, int32_t *out_argmax,
                             float *out_logit, int32_t *out_accept, int32_t *out_tokens,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
  return mtp_verify_accept_cfg(hidden, B, k, H, head, V, draft, out_argmax, out_logit,
                               out_accept, out_tokens, ws, ws_bytes, stream, nullptr);
}

mtp_status mtp_verify_accept_noalloc(const mtp_bf16 *hidden, int B, int k, int H,
                                     const mtp_bf16 *head, int64_t V, const int32_t *draft,
                                     int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                     int32_t *out_tokens, hipStream_t stream) {
  mtp_status st = check_verify_io(hidden, B, k, H, head, V, draft, out_argmax, out_logit,
                                  out_accept, out_tokens);
  if (st != MTP_OK) return st;
  const int64_t M = (int64_t)B * (k + 1);
  if (M > MTP_NOALLOC_MAX_ROWS) return MTP_ERR_WORKSPACE;
  void *ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  // The array keeps whatever the last call on this device left in it: clear
  // the ticket and this call's keys first (a kernel, stream-ordered before
  // the verify kernels; no hipMemsetAsync).
  const size_t used = min_rows_workspace_bytes(M);
  e = mtp::launch_fill_zero(ws, used, stream);
  if (e != hipSuccess) return hip_fail(e);
  // one-level finish (no workspace size given): the array holds the ticket
  // and the keys only
  return run_rows(hidden, B * (k + 1), H, head, V,
                  verify_sink(ws, B, k, draft, out_argmax, out_logit, out_accept, out_tokens), 0,
                  stream, nullptr, nullptr);
}

size_t mtp_tiled_bytes(int64_t rows, int H) { return tiled_bytes_of(rows, H); }

mtp_status mtp_pack_tiled(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids, int64_t C,
                          void *tiled, size_t tiled_bytes, hipStream_t stream) {
  if (!head || !tiled) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || C < 1 || C > INT32_MAX || (!ids && C > V)) return MTP_ERR_INVALID_ARG;
  const size_t need = tiled_bytes_of(C, H);
  if (need == 0) return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(tiled, 16) || (ids && !aligned(ids, 4)))
    return MTP_ERR_INVALID_ARG;
  if (tiled_bytes < need) return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack_tiled(head, V, H / 8, ids, C, mtp::tiled_cols(H) / 32, tiled, cus,
                             stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_tiled_cfg(const mtp_bf16 *hidden, int M, int H,
                                      const void *table_tiled, const int32_t *ids, int64_t C,
                                      int32_t *out_ids, float *out_logit, void *ws,
                                      size_t ws_bytes, hipStream_t stream,
                                      const mtp_config *cfg) {
  mtp_status st = check_draft_args(hidden, M, H, table_tiled, ids, C, out_ids, out_logit, ws,
                                   ws_bytes, cfg);
  if (st != MTP_OK) return st;
  return run_rows_tiled(hidden, M, H, table_tiled, C, draft_sink(ws, ids, out_ids, out_logit, M),
                        ws, ws_bytes, stream, cfg);
}

mtp_status mtp_draft_argmax_tiled(const mtp_bf16 *hidden, int M, int H, const void *table_tiled,
                                  const int32_t *ids, int64_t C, int32_t *out_ids,
                                  float *out_logit, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return mtp_draft_argmax_tiled_cfg(hidden, M, H, table_tiled, ids, C, out_ids, out_logit, ws,
                                    ws_bytes, stream, nullptr);
}

mtp_status mtp_verify_accept_tiled_cfg(const mtp_bf16 *hidden, int B, int k, int H,
                                       const void *head_tiled, int64_t V, const int32_t *draft,
                                       int32_t *out_argmax, float *out_logit,
                                       int32_t *out_accept, int32_t *out_tokens, void *ws,
                                       size_t ws_bytes, hipStream_t stream,
                                       const mtp_config *cfg) {
  mtp_status st = check_verify_args(hidden, B, k, H, head_tiled, V, draft, out_argmax, out_logit,
                                    out_accept, out_tokens, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  return run_rows_tiled(
      hidden, B * (k + 1), H, head_tiled, V,
      verify_sink(ws, B, k, draft, out_argmax, out_logit, out_accept, out_tokens), ws, ws_bytes,
      stream, cfg);
}

mtp_status mtp_verify_accept_tiled(const mtp_bf16 *hidden, int B, int k, int H,
                                   const void *head_tiled, int64_t V, const int32_t *draft,
                                   int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                   int32_t *out_tokens, void *ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return mtp_verify_accept_tiled_cfg(hidden, B, k, H, head_tiled, V, draft, out_argmax,
                                     out_logit, out_accept, out_tokens, ws, ws_bytes, stream,
                                     nullptr);
}

mtp_status mtp_draft_argmax_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                       const mtp_bf16 *head, int64_t V, const int32_t *ids,
                                       int64_t C, int32_t *out_ids, float *out_logit, void *ws,
                                       size_t ws_bytes, hipStream_t stream,
                                       const mtp_config *cfg) {
  if (!ids) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX) return MTP_ERR_INVALID_ARG;
  mtp_status st =
      check_draft_args(hidden, M, H, head, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  // the key of a gathered candidate is its id, so the finish needs no id map
  return run_rows(hidden, M, H, head, C, draft_sink(ws, nullptr, out_ids, out_logit, M), ws_bytes,
                  stream, cfg, nullptr, ids, V);
}

mtp_status mtp_draft_argmax_gather(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *head,
                                   int64_t V, const int32_t *ids, int64_t C, int32_t *out_ids,
                                   float *out_logit, void *ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return mtp_draft_argmax_gather_cfg(hidden, M, H, head, V, ids, C, out_ids, out_logit, ws,
                                     ws_bytes, stream, nullptr);
}

size_t mtp_fp8_table_bytes(int64_t C, int H) {
  if (C < 1 || C > INT32_MAX || H < 16 || H > MTP_MAX_HIDDEN || H % 16 != 0) return 0;
  return (size_t)C * (size_t)H;
}

mtp_status mtp_pack_candidates_fp8(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                   int64_t C, uint8_t *table_q, float *scales,
                                   hipStream_t stream) {
  if (!head || !table_q || !scales) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || mtp_fp8_table_bytes(C, H) == 0) return MTP_ERR_INVALID_ARG;
  if (!ids && C > V) return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(table_q, 16) || !aligned(scales, 4) ||
      (ids && !aligned(ids, 4)))
    return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack_fp8(head, V, H, ids, C, table_q, scales, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

// fp8 draft over C candidates: table rows 0..C-1, or (gather_ids) head rows
// gather_ids[i] of a head of gather_V rows, keyed by id.
static mtp_status run_fp8(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                          const float *scales, const int32_t *ids, int64_t C, int32_t *out_ids,
                          float *out_logit, void *ws, size_t ws_bytes, hipStream_t stream,
                          const mtp_config *cfg, const int32_t *gather_ids, int64_t gather_V) {
  if (!scales || !aligned(scales, 4)) return MTP_ERR_INVALID_ARG;
  if (H % 16 != 0) return MTP_ERR_INVALID_ARG;
  mtp_status st =
      check_draft_args(hidden, M, H, table_q, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  if (cfg && cfg->path == MTP_PATH_MFMA) return MTP_ERR_UNSUPPORTED;
  const int ncq = H / 16;
  const int ncl = mtp::fp8_ncl_for(ncq);
  if (ncl == 0) return MTP_ERR_UNSUPPORTED;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const int mr = mtp::fp8_rows_for(M, ncl);
  // two workgroups per CU when one pass covers every hidden row with enough
  // arithmetic per byte (MR * NCL >= 8) to be ALU-limited; one otherwise
  // (measured on MI355X at H = 2,048 .. 5,120, M = 1 .. 8). Short rows (at
  // most two chunks per lane, H <= 2,048) with 2 to 4 hidden rows in one
  // pass take four: a same-box sweep of 1-4 workgroups per CU at 65,536 x
  // 2,048 gave 29.9 -> 26.3 us at M = 2, 31.9 -> 30.4 at M = 3 and 32.2 ->
  // 30.4 at M = 4, while every other cell measured kept its count.
  const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu
                     : (ncl <= 2 && mr >= 2 && mr <= 4 && mr >= M) ? 4
                     : (ncl == 1 && M == 1) ? 2  // H <= 1,024: 18.9 -> 15.0 us
                     : ((mr >= M && mr * ncl >= 8) ? 2 : 1);
  mtp::Fp8Launch L;
  L.X = hidden;
  L.Q = table_q;
  L.scales = scales;
  L.M = M;
  L.N = C;
  L.ncq = ncq;
  L.max_blocks_x = per_cu * cus;
  // gathered candidates are keyed by id: the finish needs no id map
  L.sink = draft_sink(ws, gather_ids ? nullptr : ids, out_ids, out_logit, M);
  choose_finish(L.sink, ws_bytes, (double)C * (H + 4), (int64_t)per_cu * cus);
  L.stream = stream;
  L.gather_ids = gather_ids;
  L.gather_V = gather_V;
  e = mtp::launch_fp8(L, mr, ncl);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_fp8_cfg(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                    const float *scales, const int32_t *ids, int64_t C,
                                    int32_t *out_ids, float *out_logit, void *ws,
                                    size_t ws_bytes, hipStream_t stream,
                                    const mtp_config *cfg) {
  return run_fp8(hidden, M, H, table_q, scales, ids, C, out_ids, out_logit, ws, ws_bytes, stream,
                 cfg, nullptr, 0);
}

mtp_status mtp_draft_argmax_fp8_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                           const uint8_t *head_q, const float *head_scales,
                                           int64_t V, const int32_t *ids, int64_t C,
                                           int32_t *out_ids, float *out_logit, void *ws,
                                           size_t ws_bytes, hipStream_t stream,
                                           const mtp_config *cfg) {
  if (!ids) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX) return MTP_ERR_INVALID_ARG;
  return run_fp8(hidden, M, H, head_q, head_scales, ids, C, out_ids, out_logit, ws, ws_bytes,
                 stream, cfg, ids, V);
}

mtp_status mtp_draft_argmax_fp8_gather(const mtp_bf16 *hidden, int M, int H,
                                       const uint8_t *head_q, const float *head_scales,
                                       int64_t V, const int32_t *ids, int64_t C, int32_t *out_ids,
                                       float *out_logit, void *ws, size_t ws_bytes,
                                       hipStream_t stream) {
  return mtp_draft_argmax_fp8_gather_cfg(hidden, M, H, head_q, head_scales, V, ids, C, out_ids,
                                         out_logit, ws, ws_bytes, stream, nullptr);
}

mtp_status mtp_draft_argmax_fp8(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                const float *scales, const int32_t *ids, int64_t C,
                                int32_t *out_ids, float *out_logit, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
  return mtp_draft_argmax_fp8_cfg(hidden, M, H, table_q, scales, ids, C, out_ids, out_logit, ws,
                                  ws_bytes, stream, nullptr);
}

size_t mtp_mxfp4_table_bytes(int64_t C, int H) {
  if (C < 1 || C > INT32_MAX || H < 32 || H > MTP_MAX_HIDDEN || H % 32 != 0) return 0;
  return (size_t)C * (size_t)(H / 2);
}

size_t mtp_mxfp4_scale_bytes(int64_t C, int H) {
  if (mtp_mxfp4_table_bytes(C, H) == 0) return 0;
  return (size_t)C * (size_t)(H / 32);
}

mtp_status mtp_pack_candidates_mxfp4_rule(const mtp_bf16 *head, int64_t V, int H,
                                          const int32_t *ids, int64_t C, uint8_t *table_q,
                                          uint8_t *scales, int rule, hipStream_t stream) {
  if (!head || !table_q || !scales) return MTP_ERR_INVALID_ARG;
  if (rule != MTP_MX_SCALE_OCP && rule != MTP_MX_SCALE_FIT) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || mtp_mxfp4_table_bytes(C, H) == 0) return MTP_ERR_INVALID_ARG;
  if (!ids && C > V) return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(table_q, 16) || (ids && !aligned(ids, 4)))
    return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack_mxfp4(head, V, H, ids, C, table_q, scales, rule, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_pack_candidates_mxfp4(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                     int64_t C, uint8_t *table_q, uint8_t *scales,
                                     hipStream_t stream) {
  return mtp_pack_candidates_mxfp4_rule(head, V, H, ids, C, table_q, scales, MTP_MX_SCALE_OCP,
                                        stream);
}

// MXFP4 draft over C candidates: table rows 0..C-1, or (gather_ids) head rows
// gather_ids[i] of a head of gather_V rows, keyed by id.
static mtp_status run_mxfp4(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                     const uint8_t *scales, const int32_t *ids, int64_t C, int32_t *out_ids,
                     float *out_logit, void *ws, size_t ws_bytes, hipStream_t stream,
                     const mtp_config *cfg, const int32_t *gather_ids, int64_t gather_V) {
  if (!scales || H % 32 != 0) return MTP_ERR_INVALID_ARG;
  mtp_status st =
      check_draft_args(hidden, M, H, table_q, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  if (cfg && cfg->path == MTP_PATH_MFMA) return MTP_ERR_UNSUPPORTED;
  const int nblk = H / 32;
  const int ncl = mtp::fp4_ncl_for(nblk);
  if (ncl == 0) return MTP_ERR_UNSUPPORTED;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const int mr = mtp::fp4_rows_for(M, ncl);
  // two workgroups per CU: a row is only H/2 bytes, so one workgroup per CU
  // keeps too little in flight (measured on MI355X, 65,536 rows at H = 2,048:
  // 19.3 us against 21.4 us at M = 1, 35.7 against 45.8 us at M = 4). With
  // one block per lane (H <= 2,048) and 2 to 4 hidden rows per pass the
  // kernel is bound by its arithmetic, and four workgroups per CU hide more
  // of it (same-box A/B at 65,536 x 2,048: 21.7 -> 21.0 us at M = 2, 30.9 ->
  // 28.3 us at M = 4; at M = 1 and 8, and at H = 4,096, two stay faster).
  const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu
                                                      : (ncl == 1 && mr >= 2 && mr <= 4 ? 4 : 2);
  mtp::Fp4Launch L;
  L.X = hidden;
  L.Q = table_q;
  L.scales = scales;
  L.M = M;
  L.N = C;
  L.nblk = nblk;
  L.max_blocks_x = per_cu * cus;
  // gathered candidates are keyed by id: the finish needs no id map
  L.sink = draft_sink(ws, gather_ids ? nullptr : ids, out_ids, out_logit, M);
  choose_finish(L.sink, ws_bytes, (double)C * (H / 2 + H / 32), (int64_t)per_cu * cus);
  L.stream = stream;
  L.gather_ids = gather_ids;
  L.gather_V = gather_V;
  e = mtp::launch_fp4(L, mr, ncl);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_mxfp4_cfg(const mtp_bf16 *hidden, int M, int H,
                                      const uint8_t *table_q, const uint8_t *scales,
                                      const int32_t *ids, int64_t C, int32_t *out_ids,
                                      float *out_logit, void *ws, size_t ws_bytes,
                                      hipStream_t stream, const mtp_config *cfg) {
  return run_mxfp4(hidden, M, H, table_q, scales, ids, C, out_ids, out_logit, ws, ws_bytes,
                   stream, cfg, nullptr, 0);
}

mtp_status mtp_draft_argmax_mxfp4_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                             const uint8_t *head_q, const uint8_t *head_scales,
                                             int64_t V, const int32_t *ids, int64_t C,
                                             int32_t *out_ids, float *out_logit, void *ws,
                                             size_t ws_bytes, hipStream_t stream,
                                             const mtp_config *cfg) {
  if (!ids) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX) return MTP_ERR_INVALID_ARG;
  return run_mxfp4(hidden, M, H, head_q, head_scales, ids, C, out_ids, out_logit, ws, ws_bytes,
                   stream, cfg, ids, V);
}

mtp_status mtp_draft_argmax_mxfp4_gather(const mtp_bf16 *hidden, int M, int H,
                                         const uint8_t *head_q, const uint8_t *head_scales,
                                         int64_t V, const int32_t *ids, int64_t C,
                                         int32_t *out_ids, float *out_logit, void *ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return mtp_draft_argmax_mxfp4_gather_cfg(hidden, M, H, head_q, head_scales, V, ids, C, out_ids,
                                           out_logit, ws, ws_bytes, stream, nullptr);
}

mtp_status mtp_draft_argmax_mxfp4(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                  const uint8_t *scales, const int32_t *ids, int64_t C,
                                  int32_t *out_ids, float *out_logit, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return mtp_draft_argmax_mxfp4_cfg(hidden, M, H, table_q, scales, ids, C, out_ids, out_logit, ws,
                                    ws_bytes, stream, nullptr);
}

size_t mtp_tiled_mxfp4_bytes(int64_t rows, int H) {
  if (rows < 1 || rows > INT32_MAX || H < 32 || H > MTP_MAX_HIDDEN || H % 32 != 0) return 0;
  return (size_t)mtp::tiled_rows(rows) * (size_t)(mtp::tiled_cols_fp4(H) / 2);
}

size_t mtp_tiled_mxfp4_scale_bytes(int64_t rows, int H) {
  if (mtp_tiled_mxfp4_bytes(rows, H) == 0) return 0;
  return (size_t)mtp::tiled_rows(rows) * (size_t)(mtp::tiled_cols_fp4(H) / 32);
}

mtp_status mtp_pack_tiled_mxfp4_rule(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                     int64_t C, void *tiled_q, size_t q_bytes,
                                     uint8_t *tiled_scales, size_t scale_bytes, int rule,
                                     hipStream_t stream) {
  if (!head || !tiled_q || !tiled_scales) return MTP_ERR_INVALID_ARG;
  if (rule != MTP_MX_SCALE_OCP && rule != MTP_MX_SCALE_FIT) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || (!ids && C > V)) return MTP_ERR_INVALID_ARG;
  const size_t need = mtp_tiled_mxfp4_bytes(C, H);
  if (need == 0 || q_bytes < need || scale_bytes < mtp_tiled_mxfp4_scale_bytes(C, H))
    return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(tiled_q, 16) || !aligned(tiled_scales, 4) ||
      (ids && !aligned(ids, 4)))
    return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack_tiled_mxfp4(head, V, H, ids, C, tiled_q, tiled_scales, rule, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_pack_tiled_mxfp4(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                int64_t C, void *tiled_q, size_t q_bytes, uint8_t *tiled_scales,
                                size_t scale_bytes, hipStream_t stream) {
  return mtp_pack_tiled_mxfp4_rule(head, V, H, ids, C, tiled_q, q_bytes, tiled_scales,
                                   scale_bytes, MTP_MX_SCALE_OCP, stream);
}

mtp_status mtp_draft_argmax_tiled_mxfp4_cfg(const mtp_bf16 *hidden, int M, int H,
                                            const void *table_q, const uint8_t *tiled_scales,
                                            const int32_t *ids, int64_t C, int32_t *out_ids,
                                            float *out_logit, void *ws, size_t ws_bytes,
                                            hipStream_t stream, const mtp_config *cfg) {
  if (!tiled_scales || !aligned(tiled_scales, 4) || H % 32 != 0) return MTP_ERR_INVALID_ARG;
  mtp_status st =
      check_draft_args(hidden, M, H, table_q, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  if (cfg && cfg->path == MTP_PATH_VALU) return MTP_ERR_UNSUPPORTED;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const int nb = mtp::dma_nb_for_fp4(M);
  // 16-row passes: two workgroups per CU (their 128-row tiles fit twice)
  const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu : (nb == 1 ? 2 : 1);
  mtp::DmaLaunch L;
  L.X = hidden;
  L.WT = table_q;
  L.M = M;
  L.N = C;
  L.nch = H / 8;
  L.S = mtp::tiled_cols_fp4(H) / 32;
  L.max_blocks_x = per_cu * cus;
  L.sink = draft_sink(ws, ids, out_ids, out_logit, M);
  choose_finish(L.sink, ws_bytes, (double)C * (H / 2 + H / 32), (int64_t)per_cu * cus);
  L.stream = stream;
  L.scales = reinterpret_cast<const float *>(tiled_scales);
  e = mtp::launch_dma_fp4(L, nb);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_tiled_mxfp4(const mtp_bf16 *hidden, int M, int H,
                                        const void *table_q, const uint8_t *tiled_scales,
                                        const int32_t *ids, int64_t C, int32_t *out_ids,
                                        float *out_logit, void *ws, size_t ws_bytes,
                                        hipStream_t stream) {
  return mtp_draft_argmax_tiled_mxfp4_cfg(hidden, M, H, table_q, tiled_scales, ids, C, out_ids,
                                          out_logit, ws, ws_bytes, stream, nullptr);
}

size_t mtp_tiled_fp8_bytes(int64_t rows, int H) {
  if (rows < 1 || rows > INT32_MAX || H < 16 || H > MTP_MAX_HIDDEN || H % 16 != 0) return 0;
  return (size_t)mtp::tiled_rows(rows) * (size_t)mtp::tiled_cols(H);
}

mtp_status mtp_pack_tiled_fp8(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                              int64_t C, void *tiled_q, size_t tiled_bytes, float *scales,
                              hipStream_t stream) {
  if (!head || !tiled_q || !scales) return MTP_ERR_INVALID_ARG;
  if (V < 1 || V > INT32_MAX || (!ids && C > V)) return MTP_ERR_INVALID_ARG;
  const size_t need = mtp_tiled_fp8_bytes(C, H);
  if (need == 0 || tiled_bytes < need) return MTP_ERR_INVALID_ARG;
  if (!aligned(head, 16) || !aligned(tiled_q, 16) || !aligned(scales, 4) ||
      (ids && !aligned(ids, 4)))
    return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_pack_tiled_fp8(head, V, H, ids, C, tiled_q, scales, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_tiled_fp8_cfg(const mtp_bf16 *hidden, int M, int H,
                                          const void *table_q, const float *scales,
                                          const int32_t *ids, int64_t C, int32_t *out_ids,
                                          float *out_logit, void *ws, size_t ws_bytes,
                                          hipStream_t stream, const mtp_config *cfg) {
  if (!scales || !aligned(scales, 4) || H % 16 != 0) return MTP_ERR_INVALID_ARG;
  mtp_status st =
      check_draft_args(hidden, M, H, table_q, ids, C, out_ids, out_logit, ws, ws_bytes, cfg);
  if (st != MTP_OK) return st;
  if (cfg && cfg->path == MTP_PATH_VALU) return MTP_ERR_UNSUPPORTED;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const int per_cu = (cfg && cfg->blocks_per_cu > 0) ? cfg->blocks_per_cu : 1;
  mtp::DmaLaunch L;
  L.X = hidden;
  L.WT = table_q;
  L.M = M;
  L.N = C;
  L.nch = H / 8;
  L.S = mtp::tiled_cols(H) / 32;
  L.max_blocks_x = per_cu * cus;
  L.sink = draft_sink(ws, ids, out_ids, out_logit, M);
  choose_finish(L.sink, ws_bytes, (double)C * (H + 4), (int64_t)per_cu * cus);
  L.stream = stream;
  L.scales = scales;
  e = mtp::launch_dma_fp8(L, mtp::dma_nb_for_fp8(M));
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_draft_argmax_tiled_fp8(const mtp_bf16 *hidden, int M, int H, const void *table_q,
                                      const float *scales, const int32_t *ids, int64_t C,
                                      int32_t *out_ids, float *out_logit, void *ws,
                                      size_t ws_bytes, hipStream_t stream) {
  return mtp_draft_argmax_tiled_fp8_cfg(hidden, M, H, table_q, scales, ids, C, out_ids, out_logit,
                                        ws, ws_bytes, stream, nullptr);
}

static_assert(MTP_STREAM_SINK_WORDS == mtp::kStreamSinkWords, "sink size");

mtp_status mtp_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0) return MTP_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return MTP_ERR_INVALID_ARG;
  int cus = 0;
  hipError_t e = current_cus(&cus);
  if (e != hipSuccess) return hip_fail(e);
  e = mtp::launch_stream_read(buf, bytes, sink, cus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_probe_atomic(uint32_t *words, int wgs, int iters, int same,
                            unsigned long long *ticks, hipStream_t stream) {
  if (!words || !ticks || wgs < 1 || wgs > MTP_PROBE_MAX_WGS || iters < 1 ||
      iters > MTP_PROBE_MAX_ITERS || (same != 0 && same != 1))
    return MTP_ERR_INVALID_ARG;
  if (!aligned(words, 4) || !aligned(ticks, 8)) return MTP_ERR_INVALID_ARG;
  hipError_t e = mtp::launch_atomic_chain(words, wgs, iters, same, ticks, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

struct mtp_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

mtp_status mtp_graph_begin(hipStream_t stream) {
  if (!stream) return MTP_ERR_INVALID_ARG;
  const hipError_t e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

mtp_status mtp_graph_end(hipStream_t stream, mtp_graph **out) {
  if (!out) return MTP_ERR_INVALID_ARG;
  *out = nullptr;
  if (!stream) return MTP_ERR_INVALID_ARG;
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(stream, &graph);
  if (e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return hip_fail(e);
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return hip_fail(e);
  }
  mtp_graph *g = new (std::nothrow) mtp_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return hip_fail(hipErrorOutOfMemory);
  }
  *out = g;
  return MTP_OK;
}

mtp_status mtp_graph_launch(const mtp_graph *g, hipStream_t stream) {
  if (!g) return MTP_ERR_INVALID_ARG;
  const hipError_t e = hipGraphLaunch(g->exec, stream);
  if (e != hipSuccess) return hip_fail(e);
  return MTP_OK;
}

void mtp_graph_destroy(mtp_graph *g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
