/*
 * mtp.h -- C ABI of the MI355X (gfx950) MTP draft / verify LM-head library.
 *
 * The library runs the decode-side hot path of MTP speculative decoding with
 * greedy (argmax) acceptance, as hand-written HIP kernels:
 *
 *   draft   score hidden rows against a packed candidate sub-table of the
 *           output head and return, per row, the global token id of the
 *           highest-scoring candidate.
 *           [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big
 *           table" (少读一张大表): the draft path reads a 65,536-row table
 *           picked from the 248,320-row vocabulary; each rank finds the maximum
 *           over its candidates and exchanges the maximum score together with
 *           its global token id.]
 *   verify  score the k+1 verify positions of every sequence against the full
 *           head, take each position's argmax, and accept the longest prefix
 *           of drafts that agrees with it, plus the target's own next token.
 *           [same section: the main model keeps verifying with the full
 *           vocabulary; edge-inference runtime blog, section 2.1, and
 *           long-context blog, section 5: target verification accepts several
 *           drafted tokens per step.]
 *
 * Conventions shared by every entry point
 *   - bfloat16 values are passed as their 16-bit patterns (mtp_bf16), rows
 *     dense and row-major: element (r, j) of a [R][H] matrix is at r*H + j.
 *   - Scores are sums of bf16*bf16 products accumulated in fp32. The argmax
 *     picks the largest score; equal scores go to the lowest token id.
 *   - Device pointers point to memory on the current HIP device. The caller
 *     owns every buffer; the library allocates, frees and retains nothing.
 *   - Calls are asynchronous on `stream` (NULL = the default stream): they
 *     return once the kernels are enqueued, with no host synchronisation and
 *     no allocation, so they can be recorded into a HIP graph.
 *   - Argument errors are returned synchronously, before anything is
 *     enqueued. MTP_ERR_HIP reports a failed launch; mtp_last_hip_error()
 *     then gives the hipError_t (per thread). Device data is not validated
 *     per call: candidate ids must satisfy mtp_validate_ids(), draft ids may
 *     be any int32.
 *   - Workspace: a caller-owned device buffer of at least the queried size,
 *     8-byte aligned, zeroed once with mtp_workspace_init(). Every call
 *     leaves its counters zeroed again, so it needs no per-call clearing.
 *     With more than 128 hidden rows the query also covers a staging area
 *     past the counters of the largest call (MTP_MAX_ROWS rows), where the
 *     tiled calls pack the hidden block in fragment order: each such call
 *     writes it before reading it and leaves it as scratch, and no call
 *     keeps counters there. Calls that share a workspace must be ordered on one stream;
 *     calls with distinct workspaces may run concurrently from any threads.
 *   - Outputs are bit-identical for identical inputs, whatever the launch
 *     configuration.
 */
#ifndef MTP_H
#define MTP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t mtp_bf16; /* bfloat16 bit pattern */

typedef enum {
  MTP_OK = 0,
  MTP_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misaligned pointer */
  MTP_ERR_UNSUPPORTED = 2, /* a shape or configuration the kernels do not handle */
  MTP_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query says */
  MTP_ERR_IDS = 4,         /* candidate ids not strictly ascending or outside [0, V) */
  MTP_ERR_HIP = 5          /* a HIP call or kernel launch failed */
} mtp_status;

/* Limits checked by every entry point. */
#define MTP_MAX_K 15          /* drafts per sequence */
#define MTP_MAX_ROWS 4096     /* hidden rows per call (draft M, verify B*(k+1)) */
#define MTP_MAX_HIDDEN 16384  /* H; H must also be a multiple of 8 */

/* Launch selection for the *_cfg variants (tuning, tests). Zero fields mean
 * "choose automatically"; the plain entry points use all zeros. */
typedef enum { MTP_PATH_AUTO = 0, MTP_PATH_VALU = 1, MTP_PATH_MFMA = 2 } mtp_path;
/* (Row-major tables: AUTO picks the vector-ALU kernel for few hidden rows and
 * the matrix-core kernel beyond. Tiled tables always use the matrix cores.) */
typedef struct {
  int path;          /* mtp_path */
  int blocks_per_cu; /* workgroups per compute unit of the row-streaming grid (1..16) */
  int reserved[6];   /* must be zero */
} mtp_config;

/* Human-readable name of a status code (static storage). */
const char *mtp_status_string(mtp_status status);

/*
 * Measurement aid, not a step of the method: time the next draft or verify
 * call made by this thread. Its first kernel is launched with `start` and its
 * last with `stop` (hipExtLaunchKernel), so hipEventElapsedTime(start, stop)
 * gives the call's time on the GPU from the first dispatch's start to the last
 * one's end, with no marker packets between the calls of a stream. Either
 * event may be NULL. The request stays pending until a call launches (calls
 * that fail their argument checks launch nothing) and applies to one call.
 * Events must be created with timing enabled on the call's device; not for
 * use inside a graph capture.
 */
void mtp_time_next_call(hipEvent_t start, hipEvent_t stop);

/* hipError_t of the calling thread's last MTP_ERR_HIP (0 if none). */
int mtp_last_hip_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int mtp_version(void);

/* Host check of a candidate id list: strictly ascending, every id in [0, V).
 * ids_host: host array of C int32. Returns MTP_OK or MTP_ERR_IDS
 * (MTP_ERR_INVALID_ARG for a null pointer or C, V <= 0). */
mtp_status mtp_validate_ids(const int32_t *ids_host, int64_t C, int64_t V);

/* Bytes of workspace needed by mtp_draft_argmax for M hidden rows, and by
 * mtp_verify_accept for B sequences with k drafts each (the same sizes serve
 * every variant of these calls). 0 for arguments out of range.
 *   - Counters: 256 bytes of header and 8 regions of 64 + 8*M bytes, each
 *     rounded up to 256 (2,304 bytes at M = 1). Launches whose workgroups
 *     each stream less than 448 KiB of the table spread the cross-workgroup
 *     finish over the 8 regions (a grouped finish: 8 group tickets and key
 *     sets, so that hundreds of workgroups arriving together do not queue
 *     on one address). Every call accepts the counters' least size, 256 +
 *     8*M bytes rounded up to 256, and then runs the one-level finish; the
 *     winner is the same either way.
 *   - With M or B*(k+1) above 128 the size includes a staging area of about
 *     M*H*2 bytes for the packed hidden block, placed past the counters of
 *     the largest call (MTP_MAX_ROWS rows, 264,448 bytes). A tiled call with
 *     more than 128 hidden rows returns MTP_ERR_WORKSPACE when given less. A
 *     row-major call given the full size runs its passes of more than 128
 *     rows (H % 64 == 0) on the register-ring matrix-core kernel, given less
 *     on the LDS-fed one; both sum every logit in the same order, so the
 *     results are the same bits. */
size_t mtp_draft_workspace_bytes(int M, int64_t C, int H);
size_t mtp_verify_workspace_bytes(int B, int k, int64_t V, int H);

/* Zero `ws_bytes` bytes of a workspace on `stream` (a fill kernel, so it may
 * be captured into a graph). ws must be 8-byte aligned, ws_bytes a multiple
 * of 8. */
mtp_status mtp_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Pack the candidate sub-table (one-time set-up, not per call):
 *   table[i][:] = head[ids[i]][:]  for i < C.
 * head  device [V][H] bf16;  ids device int32 [C], strictly ascending in
 * [0, V) (check them with mtp_validate_ids first);  table device [C][H]
 * bf16, written. A row whose id is out of range is filled with zeros.
 * head and table 16-byte aligned, H a multiple of 8.
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * the full head stays resident and a smaller table serves the draft path,
 * about 160 MiB per machine = 32,768 rows x 2,560 x 2 bytes, i.e. dense
 * unpadded bf16 rows.]
 */
mtp_status mtp_pack_candidates(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                               int64_t C, mtp_bf16 *table, hipStream_t stream);

/*
 * Draft step: for each hidden row m < M,
 *   z[m][i]       = sum_j hidden[m][j] * table[i][j]     (fp32 accumulate)
 *   i*            = lowest i with z[m][i] = max_i z[m][i]
 *   out_ids[m]    = ids[i*]          (ids NULL: i* itself)
 *   out_logit[m]  = z[m][i*]         (skipped if out_logit is NULL)
 * hidden device [M][H] bf16 (16-byte aligned); table device [C][H] bf16
 * (16-byte aligned); ids device int32 [C] ascending, or NULL for the
 * identity map; out_ids device int32 [M]; out_logit device float [M] or
 * NULL; ws/ws_bytes the workspace (mtp_draft_workspace_bytes(M, C, H)).
 * 1 <= M <= MTP_MAX_ROWS, 1 <= C < 2^31, 8 <= H <= MTP_MAX_HIDDEN, H % 8 == 0.
 * Rows of a batch are independent: the result equals M separate calls.
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table".]
 */
mtp_status mtp_draft_argmax(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *table,
                            const int32_t *ids, int64_t C, int32_t *out_ids, float *out_logit,
                            void *ws, size_t ws_bytes, hipStream_t stream);

mtp_status mtp_draft_argmax_cfg(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *table,
                                const int32_t *ids, int64_t C, int32_t *out_ids,
                                float *out_logit, void *ws, size_t ws_bytes, hipStream_t stream,
                                const mtp_config *cfg);

/*
 * Verify step with greedy acceptance, for B sequences of k drafts each.
 *   hidden      device [B*(k+1)][H] bf16; row b*(k+1)+p is the target's
 *               hidden state that predicts slot p of sequence b (p = 0..k).
 *   head        device [V][H] bf16, the full output head.
 *   draft       device int32 [B][k], the drafted tokens (unused if k == 0).
 *   out_argmax  device int32 [B][k+1]: t[b][p] = lowest v maximising
 *               sum_j hidden[b*(k+1)+p][j] * head[v][j] (fp32 accumulate).
 *   out_logit   device float [B][k+1] (that maximum) or NULL.
 *   out_accept  device int32 [B]: n_b = lowest p < k with draft[b][p] !=
 *               t[b][p], or k if every draft agrees.
 *   out_tokens  device int32 [B][k+1]: t[b][0..n_b] (the accepted drafts,
 *               equal to t there, then the bonus token t[b][n_b]); slots
 *               after n_b are -1.
 *   ws/ws_bytes workspace (mtp_verify_workspace_bytes(B, k, V, H)).
 * 1 <= B, 0 <= k <= MTP_MAX_K, B*(k+1) <= MTP_MAX_ROWS, 1 <= V < 2^31.
 * k == 0 is plain greedy decoding: n_b = 0, tokens[b][0] = t[b][0].
 * [edge-inference runtime blog, section 2.1: verification in parallel
 * accepts more tokens than steps executed; long-context blog, section 5;
 * Qwen3.8 Flash dual-Spark tuning log, sections "MTP guesses one more step"
 * (k = 3 and k = 4) and "read one fewer big table" (full-vocabulary
 * verification).]
 */
mtp_status mtp_verify_accept(const mtp_bf16 *hidden, int B, int k, int H, const mtp_bf16 *head,
                             int64_t V, const int32_t *draft, int32_t *out_argmax,
                             float *out_logit, int32_t *out_accept, int32_t *out_tokens,
                             void *ws, size_t ws_bytes, hipStream_t stream);

mtp_status mtp_verify_accept_cfg(const mtp_bf16 *hidden, int B, int k, int H,
                                 const mtp_bf16 *head, int64_t V, const int32_t *draft,
                                 int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                 int32_t *out_tokens, void *ws, size_t ws_bytes,
                                 hipStream_t stream, const mtp_config *cfg);

/*
 * Allocation-free verify, for callers that cannot allocate device memory or
 * hold a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and results as
 * mtp_verify_accept (row-major head), without ws / ws_bytes. The ticket and
 * the per-row keys live in a static device array of the library, 8,448 bytes
 * (header + MTP_NOALLOC_MAX_ROWS keys), which every GPU the library runs on
 * holds from its first such call until the process ends; this array is the
 * one exception to "the library allocates nothing".
 *   - B*(k+1) <= MTP_NOALLOC_MAX_ROWS; a larger call returns
 *     MTP_ERR_WORKSPACE with nothing enqueued. Other argument errors are those
 *     of mtp_verify_accept.
 *   - The array keeps what the last call left in it. Each call first clears
 *     the part it uses (one small kernel on `stream`, no hipMemsetAsync).
 *   - All calls on one GPU share its array: calls that may overlap (other
 *     streams, or threads without ordering between them) race and give
 *     undefined results. Order them on one stream, or use mtp_verify_accept
 *     with one workspace per stream.
 *   - No hipMalloc, hipFree or allocating library routine is called. The first
 *     call on a device looks up the array's device address
 *     (hipGetSymbolAddress); a failure there returns MTP_ERR_HIP.
 */
#define MTP_NOALLOC_MAX_ROWS 1024
mtp_status mtp_verify_accept_noalloc(const mtp_bf16 *hidden, int B, int k, int H,
                                     const mtp_bf16 *head, int64_t V, const int32_t *draft,
                                     int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                     int32_t *out_tokens, hipStream_t stream);

/*
 * Tiled tables (batched rows).
 *
 * When one call scores many hidden rows (a batch of sequences), the table
 * rows feed the matrix cores, whose operand is 16 table rows x 32 columns. The
 * tiled layout stores a table so that each such operand is 1 KiB contiguous
 * and every 64-row tile is one contiguous stream:
 *   rows are padded with zero rows to Rp = ceil(R / 64) * 64, columns with
 *   zeros to Hp = ceil(H / 128) * 128; S = Hp / 32;
 *   16-byte element e of the buffer (lane = e % 64, f = e / 64, rb = f % 4,
 *   s = (f / 4) % S, t = f / (4 S)) holds the 8 bf16 values of row
 *   64 t + 16 rb + lane % 16, columns 32 s + 8 (lane / 16) .. + 8.
 * The values are the row-major table's; only their order differs. A tiled
 * call computes the same sums as the row-major call on the same table (up to
 * fp32 summation order, which can move a pick only inside a near tie). Size:
 * mtp_tiled_bytes(R, H) = Rp * Hp * 2 bytes (0 if out of range).
 * Like the packed candidate table, the tiled form is built once (the full
 * head for verification, the candidate table for drafting) and stays
 * resident. [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big
 * table": both the full head and the small draft table are kept in memory.]
 */
size_t mtp_tiled_bytes(int64_t rows, int H);

/* Build a tiled table from the row-major head [V][H] (device): rows ids[i]
 * (ids device int32 [C], strictly ascending in [0, V)), or, with ids NULL,
 * the first C rows (C <= V; C == V tiles the whole head). tiled: device,
 * 16-byte aligned, tiled_bytes >= mtp_tiled_bytes(C, H); written. Rows
 * whose id is out of range are zero. */
mtp_status mtp_pack_tiled(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids, int64_t C,
                          void *tiled, size_t tiled_bytes, hipStream_t stream);

/* mtp_draft_argmax on a tiled candidate table (C rows, built by
 * mtp_pack_tiled); arguments and results as mtp_draft_argmax. */
mtp_status mtp_draft_argmax_tiled(const mtp_bf16 *hidden, int M, int H, const void *table_tiled,
                                  const int32_t *ids, int64_t C, int32_t *out_ids,
                                  float *out_logit, void *ws, size_t ws_bytes,
                                  hipStream_t stream);
mtp_status mtp_draft_argmax_tiled_cfg(const mtp_bf16 *hidden, int M, int H,
                                      const void *table_tiled, const int32_t *ids, int64_t C,
                                      int32_t *out_ids, float *out_logit, void *ws,
                                      size_t ws_bytes, hipStream_t stream,
                                      const mtp_config *cfg);

/* mtp_verify_accept on a tiled head (V rows, built by mtp_pack_tiled with
 * ids NULL and C == V); arguments and results as mtp_verify_accept. */
mtp_status mtp_verify_accept_tiled(const mtp_bf16 *hidden, int B, int k, int H,
                                   const void *head_tiled, int64_t V, const int32_t *draft,
                                   int32_t *out_argmax, float *out_logit, int32_t *out_accept,
                                   int32_t *out_tokens, void *ws, size_t ws_bytes,
                                   hipStream_t stream);
mtp_status mtp_verify_accept_tiled_cfg(const mtp_bf16 *hidden, int B, int k, int H,
                                       const void *head_tiled, int64_t V, const int32_t *draft,
                                       int32_t *out_argmax, float *out_logit,
                                       int32_t *out_accept, int32_t *out_tokens, void *ws,
                                       size_t ws_bytes, hipStream_t stream,
                                       const mtp_config *cfg);

/*
 * Draft over gathered candidates (no packed table):
 *   out_ids[m] = argmax over i < C of  hidden[m] . head[ids[i]]   (an id)
 * The candidate list may change every call: a fixed set plus rows chosen for
 * this step, in any order, repeats allowed. Ties go to the lowest id,
 * whatever the order of the list; an id outside [0, V) is not a candidate
 * (its row is never read); with no valid id, out_ids[m] = -1 and
 * out_logit[m] = NaN. Reads C head rows of H bf16 each, in list order, so
 * the cost per call is that of a packed table of C rows, without the packing.
 * hidden device [M][H] bf16; head device [V][H] bf16; ids device int32 [C];
 * out_ids / out_logit / ws as mtp_draft_argmax (workspace size
 * mtp_draft_workspace_bytes(M, C, H)). Runs on the vector-ALU kernel (any M;
 * more than its per-pass row count re-reads the rows); cfg->path must be
 * MTP_PATH_AUTO or MTP_PATH_VALU (MTP_ERR_UNSUPPORTED otherwise), and H must
 * be at most 16,384.
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * the upstream work on the same bottleneck drafts over a fixed candidate set
 * plus rows picked per step; reading rows through the id list makes a
 * per-step set cost no repacking.]
 */
mtp_status mtp_draft_argmax_gather(const mtp_bf16 *hidden, int M, int H, const mtp_bf16 *head,
                                   int64_t V, const int32_t *ids, int64_t C, int32_t *out_ids,
                                   float *out_logit, void *ws, size_t ws_bytes,
                                   hipStream_t stream);
mtp_status mtp_draft_argmax_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                       const mtp_bf16 *head, int64_t V, const int32_t *ids,
                                       int64_t C, int32_t *out_ids, float *out_logit, void *ws,
                                       size_t ws_bytes, hipStream_t stream,
                                       const mtp_config *cfg);

/*
 * FP8 candidate table.
 *
 * The draft reads its candidate rows as 8-bit floats instead of bf16: half
 * the bytes of the call that dominates the draft path.
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * the upstream work on this bottleneck stores the candidate rows in a
 * low-precision float format and reports a further gain over bf16 rows.]
 *
 * Format: OCP 8-bit float E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; subnormals m * 2^-9; no infinities; S.1111.111 is NaN; largest
 * magnitude 448). Row i has one scale s_i = 2^e_i, the smallest power of two
 * with max_j |w_i[j]| <= 448 * s_i (s_i = 1 for an all-zero row), and stores
 * q_i[j] = the E4M3 code nearest to w_i[j] / s_i, ties to the even code.
 * The draft's logit of row i is s_i * sum_j hidden[j] * value(q_i[j]),
 * accumulated in fp32; its argmax follows mtp_draft_argmax (lowest id on
 * ties). This is an approximation of the bf16 draft: each weight carries a
 * relative error up to 2^-4 (the verify still scores the full bf16 head).
 *
 * mtp_fp8_table_bytes(C, H) = C * H (the codes; the scales are C floats);
 * 0 when out of range. H must be a multiple of 16 (16-byte code chunks).
 */
size_t mtp_fp8_table_bytes(int64_t C, int H);

/* Quantise the candidate rows (one-time set-up): table_q[i][:] and
 * scales[i] from head[ids[i]][:] as above (ids NULL: head rows 0..C-1,
 * C <= V). head device [V][H] bf16, 16-byte aligned; ids device int32 [C]
 * (check with mtp_validate_ids; an out-of-range id gives a zero row with
 * scale 1); table_q device [C][H] bytes, 16-byte aligned, written; scales
 * device float [C], written. The codes are exactly the format's rounding of
 * the bf16 values (bit-identical to any correct implementation). */
mtp_status mtp_pack_candidates_fp8(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                   int64_t C, uint8_t *table_q, float *scales,
                                   hipStream_t stream);

/* Draft over an fp8 candidate table: out_ids[m] = ids[argmax_i logit_i]
 * (ids NULL: i). hidden device [M][H] bf16; table_q, scales as written by
 * mtp_pack_candidates_fp8; out_ids / out_logit / ws as mtp_draft_argmax
 * (workspace size mtp_draft_workspace_bytes(M, C, H)). Runs on the
 * vector-ALU kernel: 1, 2, 4 or 8 hidden rows per pass (at most 16 / NCL,
 * NCL = ceil(H / 1024)); more rows take further passes over the table.
 * cfg->path MTP_PATH_MFMA gives MTP_ERR_UNSUPPORTED. */
mtp_status mtp_draft_argmax_fp8(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                const float *scales, const int32_t *ids, int64_t C,
                                int32_t *out_ids, float *out_logit, void *ws, size_t ws_bytes,
                                hipStream_t stream);
mtp_status mtp_draft_argmax_fp8_cfg(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                    const float *scales, const int32_t *ids, int64_t C,
                                    int32_t *out_ids, float *out_logit, void *ws,
                                    size_t ws_bytes, hipStream_t stream,
                                    const mtp_config *cfg);

/*
 * Draft over gathered candidates on an fp8 head (no packed table): the
 * dynamic candidate list of mtp_draft_argmax_gather, read from a head whose
 * every row was quantised once by mtp_pack_candidates_fp8 (ids NULL, C = V):
 *   out_ids[m] = argmax over i < C of  hidden[m] . fp8(head row ids[i])
 * with the fp8 logit of mtp_draft_argmax_fp8. Ties go to the lowest id,
 * whatever the order of the list; an id outside [0, V) is not a candidate;
 * with no valid id, out_ids[m] = -1 and out_logit[m] = NaN. Reads C rows of
 * H code bytes and one row scale each, in list order.
 * hidden device [M][H] bf16; head_q device [V][H] E4M3 codes (16-byte
 * aligned); head_scales device float [V]; ids device int32 [C]; H % 16 == 0;
 * out_ids / out_logit / ws as mtp_draft_argmax (workspace size
 * mtp_draft_workspace_bytes(M, C, H)). Runs on the vector-ALU kernel;
 * cfg->path must be MTP_PATH_AUTO or MTP_PATH_VALU (MTP_ERR_UNSUPPORTED
 * otherwise).
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * a fixed candidate set plus rows picked per step, in a low-precision float
 * format.]
 */
mtp_status mtp_draft_argmax_fp8_gather(const mtp_bf16 *hidden, int M, int H,
                                       const uint8_t *head_q, const float *head_scales,
                                       int64_t V, const int32_t *ids, int64_t C, int32_t *out_ids,
                                       float *out_logit, void *ws, size_t ws_bytes,
                                       hipStream_t stream);
mtp_status mtp_draft_argmax_fp8_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                           const uint8_t *head_q, const float *head_scales,
                                           int64_t V, const int32_t *ids, int64_t C,
                                           int32_t *out_ids, float *out_logit, void *ws,
                                           size_t ws_bytes, hipStream_t stream,
                                           const mtp_config *cfg);

/*
 * MXFP4 candidate table (4-bit rows; draft calls only).
 *
 * The candidate rows in the OCP microscaling 4-bit format, a quarter of the
 * bf16 bytes: elements E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
 * bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and one E8M0 scale 2^e per
 * block of 32 consecutive elements of a row, e = floor(log2(max |w| over the
 * block)) - 2 clamped to [-127, 127] (-127 for an all-zero block). Element j
 * is the E2M1 value nearest to w[j] * 2^-e (ties to the even code; past 6 it
 * saturates; a negative value keeps its sign bit when it rounds to zero).
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * the upstream work stores the candidate rows in a 4-bit float format and
 * reports a further gain over bf16 rows; the pages fix no block size or
 * scale format, and MXFP4 is the 4-bit block format gfx950 converts in
 * hardware.] The verify keeps the bf16 head.
 *
 * Layout: table_q [C][H/2] bytes, row-major, byte j/2 of a row holding
 * element j in its low nibble when j is even and in its high nibble when j is
 * odd; scales [C][H/32] bytes, the code e + 127 of block b = j/32. H must be
 * a multiple of 32. A row's logit is sum_j x[j] * 2^e(j/32) * value(q[j]),
 * accumulated in fp32 (each block's partial sum is scaled, exactly, by its
 * power of two); argmax and ids as mtp_draft_argmax.
 *
 * mtp_mxfp4_table_bytes / mtp_mxfp4_scale_bytes: C*H/2 and C*H/32 (0 if out
 * of range). mtp_pack_candidates_mxfp4 quantises head rows ids[i] (ids NULL:
 * the first C rows); an id outside [0, V) gives a zero row (scale code 0).
 * mtp_draft_argmax_mxfp4 runs on the vector-ALU kernel (any M; more than a
 * few hidden rows take several passes); cfg->path MTP_PATH_MFMA gives
 * MTP_ERR_UNSUPPORTED. Workspace as mtp_draft_argmax.
 */
size_t mtp_mxfp4_table_bytes(int64_t C, int H);
size_t mtp_mxfp4_scale_bytes(int64_t C, int H);
mtp_status mtp_pack_candidates_mxfp4(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                     int64_t C, uint8_t *table_q, uint8_t *scales,
                                     hipStream_t stream);

/* Block scale readings for the MXFP4 packs. The pages fix no scale format
 * (same section as above); the OCP rule above is the default. The fit rule
 * takes the smallest e with max |w| <= 6 * 2^e over the block (same clamp,
 * -127 for an all-zero block), so no element saturates: e is one larger than
 * the OCP exponent in blocks whose maximum lies above 6 * 2^(e_ocp), and the
 * same elsewhere. The stored format is unchanged, so every MXFP4 draft entry
 * point (packed, gathered, tiled) reads tables of either rule. */
#define MTP_MX_SCALE_OCP 0
#define MTP_MX_SCALE_FIT 1

/* mtp_pack_candidates_mxfp4 with the block scale rule `rule`
 * (MTP_MX_SCALE_OCP or MTP_MX_SCALE_FIT; anything else gives
 * MTP_ERR_INVALID_ARG before anything is enqueued). */
mtp_status mtp_pack_candidates_mxfp4_rule(const mtp_bf16 *head, int64_t V, int H,
                                          const int32_t *ids, int64_t C, uint8_t *table_q,
                                          uint8_t *scales, int rule, hipStream_t stream);
mtp_status mtp_draft_argmax_mxfp4(const mtp_bf16 *hidden, int M, int H, const uint8_t *table_q,
                                  const uint8_t *scales, const int32_t *ids, int64_t C,
                                  int32_t *out_ids, float *out_logit, void *ws, size_t ws_bytes,
                                  hipStream_t stream);
mtp_status mtp_draft_argmax_mxfp4_cfg(const mtp_bf16 *hidden, int M, int H,
                                      const uint8_t *table_q, const uint8_t *scales,
                                      const int32_t *ids, int64_t C, int32_t *out_ids,
                                      float *out_logit, void *ws, size_t ws_bytes,
                                      hipStream_t stream, const mtp_config *cfg);

/*
 * Draft over gathered candidates on an MXFP4 head (no packed table): the
 * dynamic candidate list of mtp_draft_argmax_gather, read from a head whose
 * every row was quantised once by mtp_pack_candidates_mxfp4 (ids NULL,
 * C = V):
 *   out_ids[m] = argmax over i < C of  hidden[m] . mxfp4(head row ids[i])
 * with the MXFP4 logit of mtp_draft_argmax_mxfp4. Ties go to the lowest id,
 * whatever the order of the list; an id outside [0, V) is not a candidate;
 * with no valid id, out_ids[m] = -1 and out_logit[m] = NaN. Reads C rows of
 * H/2 code bytes and H/32 scale bytes in list order.
 * hidden device [M][H] bf16; head_q device [V][H/2] codes (16-byte aligned);
 * head_scales device [V][H/32] E8M0 scales; ids device int32 [C]; H % 32 == 0;
 * out_ids / out_logit / ws as mtp_draft_argmax (workspace size
 * mtp_draft_workspace_bytes(M, C, H)). Runs on the vector-ALU kernel;
 * cfg->path must be MTP_PATH_AUTO or MTP_PATH_VALU (MTP_ERR_UNSUPPORTED
 * otherwise).
 * [Qwen3.8 Flash dual-Spark tuning log, section "read one fewer big table":
 * the upstream work drafts over a fixed candidate set plus rows picked per
 * step, with the candidate rows in a 4-bit float format.]
 */
mtp_status mtp_draft_argmax_mxfp4_gather(const mtp_bf16 *hidden, int M, int H,
                                         const uint8_t *head_q, const uint8_t *head_scales,
                                         int64_t V, const int32_t *ids, int64_t C,
                                         int32_t *out_ids, float *out_logit, void *ws,
                                         size_t ws_bytes, hipStream_t stream);
mtp_status mtp_draft_argmax_mxfp4_gather_cfg(const mtp_bf16 *hidden, int M, int H,
                                             const uint8_t *head_q, const uint8_t *head_scales,
                                             int64_t V, const int32_t *ids, int64_t C,
                                             int32_t *out_ids, float *out_logit, void *ws,
                                             size_t ws_bytes, hipStream_t stream,
                                             const mtp_config *cfg);

/*
 * MXFP4 candidate table in the tiled layout (batched draft rows: the
 * matrix-core kernel). Same codes and scales as mtp_pack_candidates_mxfp4,
 * stored for the 64-row tiled kernel: rows in tiles of 64 (zero rows pad the
 * last), columns padded with zeros to a multiple of 256 and grouped in fours
 * of 32-column steps.
 *   - codes: fragment (t, p, rb), 1 KiB, ordered (t, p, rb); lane j + 16g
 *     holds, for u = 0..3, 4 bytes (8 codes, the even element in the low
 *     nibble) of row 64t + 16rb + j at columns 32(4p + u) + 8g .. + 7;
 *   - scales: group (t, p), 256 bytes, ordered (t, p); byte rb*64 + j*4 + u
 *     is the E8M0 code of row 64t + 16rb + j, block 4p + u. Padding blocks
 *     have zero codes and scale code 0.
 * The kernel converts each step's codes with their block's scale into the
 * bf16 operand of one v_mfma_f32_16x16x32_bf16 step (exact), so the logits
 * are those of the bf16 tiled kernel over the dequantised rows.
 * mtp_tiled_mxfp4_bytes(R, H) = ceil64(R) * ceil256(H) / 2 and
 * mtp_tiled_mxfp4_scale_bytes(R, H) = ceil64(R) * ceil256(H) / 32 (0 if out
 * of range; H a multiple of 32). The draft takes up to 64 hidden rows per
 * pass (more take further passes); cfg->path MTP_PATH_VALU gives
 * MTP_ERR_UNSUPPORTED.
 */
size_t mtp_tiled_mxfp4_bytes(int64_t rows, int H);
size_t mtp_tiled_mxfp4_scale_bytes(int64_t rows, int H);
mtp_status mtp_pack_tiled_mxfp4(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                int64_t C, void *tiled_q, size_t q_bytes, uint8_t *tiled_scales,
                                size_t scale_bytes, hipStream_t stream);
/* mtp_pack_tiled_mxfp4 with the block scale rule `rule` (MTP_MX_SCALE_OCP or
 * MTP_MX_SCALE_FIT; anything else gives MTP_ERR_INVALID_ARG). */
mtp_status mtp_pack_tiled_mxfp4_rule(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                                     int64_t C, void *tiled_q, size_t q_bytes,
                                     uint8_t *tiled_scales, size_t scale_bytes, int rule,
                                     hipStream_t stream);
mtp_status mtp_draft_argmax_tiled_mxfp4(const mtp_bf16 *hidden, int M, int H,
                                        const void *table_q, const uint8_t *tiled_scales,
                                        const int32_t *ids, int64_t C, int32_t *out_ids,
                                        float *out_logit, void *ws, size_t ws_bytes,
                                        hipStream_t stream);
mtp_status mtp_draft_argmax_tiled_mxfp4_cfg(const mtp_bf16 *hidden, int M, int H,
                                            const void *table_q, const uint8_t *tiled_scales,
                                            const int32_t *ids, int64_t C, int32_t *out_ids,
                                            float *out_logit, void *ws, size_t ws_bytes,
                                            hipStream_t stream, const mtp_config *cfg);

/*
 * FP8 candidate table in the tiled layout (batched draft rows: the
 * matrix-core kernel). Same codes and scales as mtp_pack_candidates_fp8,
 * stored as the fp8 form of the 64-row tiled layout: rows in tiles of 64
 * (zero rows pad the last), columns padded with zeros to a multiple of 128
 * and grouped in pairs of 32-column steps; fragment (t, p, rb), 1 KiB,
 * ordered (t, p, rb), lane j + 16g holding the 8 codes of row
 * 64t + 16rb + j at columns 64p + 8g .. 64p + 8g + 7 followed by those at
 * columns 64p + 32 + 8g .. 64p + 32 + 8g + 7. The kernel converts each half to
 * the bf16 operand of one v_mfma_f32_16x16x32_bf16 step (exact) and
 * multiplies each finished logit by its row's scale.
 * mtp_tiled_fp8_bytes(R, H) = ceil64(R) * ceil128(H) (0 if out of range; H a
 * multiple of 16). scales: float [C], written by the pack.
 */
size_t mtp_tiled_fp8_bytes(int64_t rows, int H);
mtp_status mtp_pack_tiled_fp8(const mtp_bf16 *head, int64_t V, int H, const int32_t *ids,
                              int64_t C, void *tiled_q, size_t tiled_bytes, float *scales,
                              hipStream_t stream);
/* mtp_draft_argmax_fp8 on the tiled fp8 table: up to 64 hidden rows per
 * pass (more take further passes); cfg->path MTP_PATH_VALU gives
 * MTP_ERR_UNSUPPORTED. */
mtp_status mtp_draft_argmax_tiled_fp8(const mtp_bf16 *hidden, int M, int H, const void *table_q,
                                      const float *scales, const int32_t *ids, int64_t C,
                                      int32_t *out_ids, float *out_logit, void *ws,
                                      size_t ws_bytes, hipStream_t stream);
mtp_status mtp_draft_argmax_tiled_fp8_cfg(const mtp_bf16 *hidden, int M, int H,
                                          const void *table_q, const float *scales,
                                          const int32_t *ids, int64_t C, int32_t *out_ids,
                                          float *out_logit, void *ws, size_t ws_bytes,
                                          hipStream_t stream, const mtp_config *cfg);

/*
 * Graph-captured MTP step.
 *
 * Records the library calls a caller makes on `stream` between
 * mtp_graph_begin and mtp_graph_end into one HIP graph, so that a whole MTP
 * round (k draft calls, then verify with acceptance) is submitted with one
 * launch and replayed without per-kernel launch cost. Every call of this
 * library only enqueues kernels (no allocation, no host synchronisation, no
 * memset; the workspaces reset themselves), which is what capture requires.
 * [edge-inference runtime blog, section 3 (CUDA Graph), subsections 3.2 and
 * 3.3: capture once, replay every decode step; nothing inside the capture
 * may allocate or branch on device data. Production-inference page on vLLM,
 * section 5: decode repeats many small launches, so the replayed graph
 * removes their submission cost.]
 *
 * Usage: mtp_graph_begin(s); <calls on s>; mtp_graph_end(s, &g); then
 * mtp_graph_launch(g, s) any number of times. A replay reads the device
 * buffers whose pointers were passed during capture: write new inputs into
 * those buffers (stream-ordered before the launch) and read outputs from the
 * captured output buffers after it. The buffers must stay allocated until
 * mtp_graph_destroy. Replays of one graph, and any other use of the
 * workspaces it captured, must be stream-ordered.
 *
 * stream must be a created stream (the null stream cannot be captured).
 * Capture mode is thread-local: other threads may keep using HIP. An error
 * inside the capture (an argument error of a captured call) leaves the stream
 * capturing; mtp_graph_end then ends the capture and returns the error of
 * ending it, and the caller discards the graph.
 * mtp_graph_end and mtp_graph_destroy create and free HIP graph objects
 * (host-side set-up work); mtp_graph_launch allocates nothing.
 */
typedef struct mtp_graph mtp_graph;

mtp_status mtp_graph_begin(hipStream_t stream);
/* Ends the capture on `stream` and instantiates it; *graph receives the
 * handle (NULL on error). */
mtp_status mtp_graph_end(hipStream_t stream, mtp_graph **graph);
/* Enqueues one replay of the captured step on `stream`. */
mtp_status mtp_graph_launch(const mtp_graph *graph, hipStream_t stream);
/* Frees the graph (NULL is ignored). Call after its last replay finished. */
void mtp_graph_destroy(mtp_graph *graph);

/*
 * Streaming-read reference (a measurement aid, not a step of the method).
 *
 * Reads `bytes` bytes at `buf` once, as a plain stream of non-temporal 16-byte
 * loads, and writes one XOR word per wave into `sink` (at most
 * MTP_STREAM_SINK_WORDS words; their values carry no meaning). Timing it
 * over a buffer of a call's size gives the read rate this device actually
 * reaches: the practical ceiling of the draft and verify calls, whose cost is
 * the bytes of the rows they read. [Qwen3.8 Flash dual-Spark tuning log,
 * section "read one fewer big table": the draft's time follows the size of
 * the table it reads.]
 *
 * buf: device, 16-byte aligned; bytes: > 0, a multiple of 16. sink: device
 * uint32 [MTP_STREAM_SINK_WORDS], 4-byte aligned. Errors: MTP_ERR_INVALID_ARG
 * for a null pointer, misalignment or a bad size; MTP_ERR_HIP for a launch
 * failure. Asynchronous on `stream`; allocates nothing.
 */
#define MTP_STREAM_SINK_WORDS 8192
mtp_status mtp_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Atomic round-trip reference (a probe, like mtp_stream_read).
 *
 * Every call merges its workgroups' winners through device-scope atomics at
 * its end: each workgroup updates its keys and takes a ticket, and the last
 * one reads the merged keys, a few dependent round trips to the memory's
 * coherence point. [Qwen3.8 Flash dual-Spark tuning log, section "read one
 * fewer big table": the draft finds the maximum within its candidates and
 * exchanges (max score, global token id).] This probe times that round trip:
 * in each of `wgs` workgroups one lane runs `iters` agent-scope
 * fetch-and-adds, each waiting for the one before, on its own word
 * (words[64 b], 256 bytes apart; same == 0) or all on words[0] (same == 1),
 * and writes the chain's duration in ticks of the 100 MHz real-time counter
 * to ticks[b] (the top bit carries no meaning; mask it off).
 *
 * words: device uint32 [64 * wgs] (same == 0) or [2] (same == 1), 4-byte
 * aligned, any contents (they are incremented). ticks: device uint64 [wgs],
 * 8-byte aligned. 1 <= wgs <= MTP_PROBE_MAX_WGS, 1 <= iters <=
 * MTP_PROBE_MAX_ITERS. Errors: MTP_ERR_INVALID_ARG for a null pointer,
 * misalignment or a value out of range; MTP_ERR_HIP for a launch failure.
 * Asynchronous on `stream`; allocates nothing.
 */
#define MTP_PROBE_MAX_WGS 4096
#define MTP_PROBE_MAX_ITERS 1024
mtp_status mtp_probe_atomic(uint32_t *words, int wgs, int iters, int same,
                            unsigned long long *ticks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MTP_H */
