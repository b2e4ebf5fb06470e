// Host driver for the sanitizer build of the C ABI (test infrastructure).
// The library's sources are compiled for the host only, with
// AddressSanitizer and UndefinedBehaviorSanitizer, and linked into this
// program. Every call below carries at least one argument that the library
// rejects before any HIP call (null, misaligned, out-of-range size, short
// workspace or bad configuration), so nothing is ever launched and no device
// is needed. It also runs the pure host functions (size queries, id
// validation, status strings) over their edge cases.
#include <cstdint>
#include <cstdio>

#include "mtp.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

int main() {
  // never dereferenced: every call that takes them is rejected first
  const uint16_t *F = reinterpret_cast<const uint16_t *>(uintptr_t(0x10000));
  const uint16_t *ODD = reinterpret_cast<const uint16_t *>(uintptr_t(0x10002));
  const int32_t *FI = reinterpret_cast<const int32_t *>(uintptr_t(0x10000));
  int32_t *FO = reinterpret_cast<int32_t *>(uintptr_t(0x10000));
  float *FL = reinterpret_cast<float *>(uintptr_t(0x10000));
  void *WS = reinterpret_cast<void *>(uintptr_t(0x10000));
  uint8_t *FQ = reinterpret_cast<uint8_t *>(uintptr_t(0x10000));
  const mtp_status INV = MTP_ERR_INVALID_ARG, WSE = MTP_ERR_WORKSPACE;

  for (int s = 0; s <= 7; ++s) EXPECT(mtp_status_string((mtp_status)s) != nullptr);
  EXPECT(mtp_version() >= 100);
  EXPECT(mtp_last_hip_error() == 0);

  // size queries at their limits
  EXPECT(mtp_draft_workspace_bytes(1, 65536, 2048) == 2304);
  EXPECT(mtp_draft_workspace_bytes(MTP_MAX_ROWS, 1, 8) > 0);
  EXPECT(mtp_draft_workspace_bytes(MTP_MAX_ROWS + 1, 1, 8) == 0);
  EXPECT(mtp_draft_workspace_bytes(1, INT64_MAX, 8) == 0);
  EXPECT(mtp_draft_workspace_bytes(1, 1, MTP_MAX_HIDDEN) > 0);
  EXPECT(mtp_draft_workspace_bytes(MTP_MAX_ROWS, 1, MTP_MAX_HIDDEN) > 0);
  EXPECT(mtp_draft_workspace_bytes(-5, 1, 8) == 0);
  EXPECT(mtp_verify_workspace_bytes(256, 15, 248320, MTP_MAX_HIDDEN) > 0);
  EXPECT(mtp_verify_workspace_bytes(257, 15, 10, 8) == 0);
  EXPECT(mtp_verify_workspace_bytes(1 << 30, 15, 10, 8) == 0);
  EXPECT(mtp_tiled_bytes(INT32_MAX, 8) > 0 && mtp_tiled_bytes(INT64_MAX, 8) == 0);
  EXPECT(mtp_tiled_fp8_bytes(1, 15) == 0 && mtp_tiled_mxfp4_bytes(1, 48) == 0);
  EXPECT(mtp_fp8_table_bytes(3, 16) == 48 && mtp_mxfp4_table_bytes(3, 64) == 96);
  EXPECT(mtp_mxfp4_scale_bytes(3, 64) == 6 && mtp_tiled_mxfp4_scale_bytes(0, 64) == 0);

  // id validation
  const int32_t good[3] = {0, 4, 9}, dup[3] = {0, 4, 4}, neg[2] = {-1, 3}, big[2] = {1, 10};
  EXPECT(mtp_validate_ids(good, 3, 10) == MTP_OK);
  EXPECT(mtp_validate_ids(dup, 3, 10) == MTP_ERR_IDS);
  EXPECT(mtp_validate_ids(neg, 2, 10) == MTP_ERR_IDS);
  EXPECT(mtp_validate_ids(big, 2, 10) == MTP_ERR_IDS);
  EXPECT(mtp_validate_ids(nullptr, 3, 10) == INV);
  EXPECT(mtp_validate_ids(good, 0, 10) == INV);

  // draft / verify, row-major and tiled, gathered, fp8, mxfp4: rejected calls
  EXPECT(mtp_draft_argmax(nullptr, 1, 64, F, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax(ODD, 1, 64, F, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax(F, 0, 64, F, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax(F, 1, 60, F, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax(F, 1, 64, F, FI, 100, FO, FL, WS, 8, nullptr) == WSE);
  EXPECT(mtp_draft_argmax(F, 1, 64, F, FI, 100, FO, FL, nullptr, 4096, nullptr) == WSE);
  mtp_config bad_cfg{};
  bad_cfg.path = 7;
  EXPECT(mtp_draft_argmax_cfg(F, 1, 64, F, FI, 100, FO, FL, WS, 4096, nullptr, &bad_cfg) == INV);
  bad_cfg.path = 0;
  bad_cfg.blocks_per_cu = 17;
  EXPECT(mtp_draft_argmax_cfg(F, 1, 64, F, FI, 100, FO, FL, WS, 4096, nullptr, &bad_cfg) == INV);
  bad_cfg.blocks_per_cu = 0;
  bad_cfg.reserved[5] = 1;
  EXPECT(mtp_draft_argmax_cfg(F, 1, 64, F, FI, 100, FO, FL, WS, 4096, nullptr, &bad_cfg) == INV);
  EXPECT(mtp_verify_accept(F, 1, 16, 64, F, 100, FI, FO, FL, FO, FO, WS, 4096, nullptr) == INV);
  EXPECT(mtp_verify_accept(F, 1, 3, 64, F, 100, nullptr, FO, FL, FO, FO, WS, 4096, nullptr) == INV);
  EXPECT(mtp_verify_accept(F, 0, 3, 64, F, 100, FI, FO, FL, FO, FO, WS, 4096, nullptr) == INV);
  EXPECT(mtp_verify_accept(F, 1, 3, 64, F, 100, FI, FO, FL, FO, FO, WS, 16, nullptr) == WSE);
  EXPECT(mtp_verify_accept_tiled(F, 1, 3, 64, F, 0, FI, FO, FL, FO, FO, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_tiled(F, 1, 64, nullptr, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_gather(F, 1, 64, F, 100, nullptr, 10, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_gather(F, 1, 64, F, 0, FI, 10, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_fp8(F, 1, 64, FQ, nullptr, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_fp8(F, 1, 40, FQ, FL, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_mxfp4(F, 1, 48, FQ, FQ, FI, 100, FO, FL, WS, 4096, nullptr) == INV);
  EXPECT(mtp_draft_argmax_fp8_gather(F, 1, 64, FQ, FL, 100, nullptr, 10, FO, FL, WS, 4096,
                                     nullptr) == INV);
  EXPECT(mtp_draft_argmax_fp8_gather(F, 1, 40, FQ, FL, 100, FI, 10, FO, FL, WS, 4096,
                                     nullptr) == INV);
  EXPECT(mtp_draft_argmax_mxfp4_gather(F, 1, 64, FQ, FQ, 100, nullptr, 10, FO, FL, WS, 4096,
                                       nullptr) == INV);
  EXPECT(mtp_draft_argmax_mxfp4_gather(F, 1, 48, FQ, FQ, 100, FI, 10, FO, FL, WS, 4096,
                                       nullptr) == INV);
  EXPECT(mtp_draft_argmax_tiled_fp8(F, 1, 64, FQ, nullptr, FI, 100, FO, FL, WS, 4096, nullptr) ==
         INV);
  EXPECT(mtp_draft_argmax_tiled_mxfp4(F, 1, 64, FQ, nullptr, FI, 100, FO, FL, WS, 4096,
                                      nullptr) == INV);

  // packs, workspace init, streaming read, graphs: rejected calls
  EXPECT(mtp_pack_candidates(F, 0, 64, FI, 10, reinterpret_cast<mtp_bf16 *>(FO), nullptr) == INV);
  EXPECT(mtp_pack_tiled(F, 10, 64, nullptr, 11, WS, 1 << 20, nullptr) == INV);
  EXPECT(mtp_pack_tiled(F, 10, 64, nullptr, 10, WS, 16, nullptr) == INV);
  EXPECT(mtp_pack_candidates_fp8(F, 10, 24, FI, 5, FQ, FL, nullptr) == INV);
  EXPECT(mtp_pack_candidates_mxfp4(F, 10, 40, FI, 5, FQ, FQ, nullptr) == INV);
  EXPECT(mtp_pack_tiled_fp8(F, 10, 64, nullptr, 10, WS, 8, FL, nullptr) == INV);
  EXPECT(mtp_pack_tiled_mxfp4(F, 10, 64, nullptr, 10, WS, 1 << 20, FQ, 1, nullptr) == INV);
  EXPECT(mtp_pack_candidates_mxfp4_rule(F, 10, 64, FI, 5, FQ, FQ, 2, nullptr) == INV);
  EXPECT(mtp_pack_tiled_mxfp4_rule(F, 10, 64, nullptr, 10, WS, 1 << 20, FQ, 1,
                                   MTP_MX_SCALE_FIT, nullptr) == INV);
  EXPECT(mtp_workspace_init(WS, 12, nullptr) == INV);
  EXPECT(mtp_workspace_init(nullptr, 64, nullptr) == INV);
  uint32_t *SINK = reinterpret_cast<uint32_t *>(uintptr_t(0x10000));
  EXPECT(mtp_stream_read(F, 24, SINK, nullptr) == INV);
  EXPECT(mtp_stream_read(F, 0, SINK, nullptr) == INV);
  mtp_graph *g = reinterpret_cast<mtp_graph *>(uintptr_t(1));
  EXPECT(mtp_graph_begin(nullptr) == INV);
  EXPECT(mtp_graph_end(nullptr, &g) == INV && g == nullptr);
  EXPECT(mtp_graph_end(nullptr, nullptr) == INV);
  EXPECT(mtp_graph_launch(nullptr, nullptr) == INV);
  mtp_graph_destroy(nullptr);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("sanitized C ABI run ok\n");
  return 0;
}
