// Argument checks of every C-ABI entry point, run against the launch stubs
// under the host address and undefined-behaviour sanitizers (test
// infrastructure). Each case states the status it expects and whether the
// call must reach a launch; extreme sizes exercise the 64-bit size arithmetic.
#include <cstdint>
#include <cstdio>

#include "moe_finalize.h"

namespace moef {
extern int g_launches;
}

static int failures = 0;

static void check(const char* what, int got, int want, bool launched_expected) {
  static int last = 0;
  const bool launched = moef::g_launches != last;
  last = moef::g_launches;
  if (got != want || launched != launched_expected) {
    std::fprintf(stderr, "FAIL %s: status %d (want %d), launched %d (want %d)\n", what, got, want,
                 (int)launched, (int)launched_expected);
    ++failures;
  }
}

template <typename T>
static T* at(uint64_t a) { return reinterpret_cast<T*>(a); }

int main() {
  const uint64_t G2 = 0x100000000ull, IDX = 0x200000000000ull, W = 0x300000000000ull,
                 PK = 0x400000000000ull, SH = 0x500000000000ull, OUT = 0x600000000000ull,
                 RES = 0x700000000000ull, GAM = 0x7100000000ull, RO = 0x720000000000ull,
                 NM = 0x730000000000ull, Q = 0x740000000000ull, S = 0x750000000000ull;
  // moe_finalize
  check("finalize ok", moe_finalize(at<uint16_t>(G2), 4096, at<int32_t>(IDX), at<float>(W),
                                    nullptr, at<uint16_t>(SH), 2.5f, at<uint16_t>(OUT), 256,
                                    7168, 8, nullptr, nullptr), MOEF_OK, true);
  check("finalize packed ok", moe_finalize(at<uint16_t>(G2), 4096, at<int32_t>(IDX), nullptr,
                                           at<int32_t>(PK), nullptr, 1.0f, at<uint16_t>(OUT), 1,
                                           8, 1, nullptr, nullptr), MOEF_OK, true);
  // largest accepted sizes: gemm2_out spans 2^31 rows of 2 MiB (4.5e15 bytes),
  // so the other buffers sit below it, apart from each other; 32767 tokens of
  // 2048 chunks are the most whole tokens of 2^20 columns MOEF_MAX_UNITS allows
  check("finalize largest sizes", moe_finalize(at<uint16_t>(0x10000000000000ull), INT32_MAX,
                                               at<int32_t>(0x30000000000ull),
                                               at<float>(0x40000000000ull), nullptr, nullptr, 1.0f,
                                               at<uint16_t>(0x1000), 32767, 1 << 20, 16,
                                               nullptr, nullptr),
        MOEF_OK, true);
  check("finalize 32768 tokens of 2^20 columns", moe_finalize(
      at<uint16_t>(0x10000000000000ull), INT32_MAX, at<int32_t>(0x30000000000ull),
      at<float>(0x40000000000ull), nullptr, nullptr, 1.0f, at<uint16_t>(0x1000), 32768, 1 << 20,
      16, nullptr, nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("finalize MOEF_MAX_UNITS one-chunk tokens", moe_finalize(
      at<uint16_t>(G2), 1, at<int32_t>(IDX), at<float>(W), nullptr, nullptr, 1.0f,
      at<uint16_t>(0x7f0000000000ull), MOEF_MAX_UNITS, 512, 1, nullptr, nullptr), MOEF_OK, true);
  check("finalize one unit beyond MOEF_MAX_UNITS", moe_finalize(
      at<uint16_t>(G2), 1, at<int32_t>(IDX), at<float>(W), nullptr, nullptr, 1.0f,
      at<uint16_t>(0x7f0000000000ull), MOEF_MAX_UNITS + 1, 512, 1, nullptr, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("finalize units beyond 2^31", moe_finalize(at<uint16_t>(G2), 1, at<int32_t>(IDX),
                                                   at<float>(W), nullptr, nullptr, 1.0f,
                                                   at<uint16_t>(OUT), INT32_MAX, 1 << 20, 1,
                                                   nullptr, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("finalize T=0", moe_finalize(nullptr, 0, nullptr, nullptr, nullptr, nullptr, 1.0f, nullptr,
                                     0, 4096, 8, nullptr, nullptr), MOEF_OK, false);
  check("finalize T<0", moe_finalize(at<uint16_t>(G2), 1, at<int32_t>(IDX), at<float>(W), nullptr,
                                     nullptr, 1.0f, at<uint16_t>(OUT), -5, 4096, 8, nullptr,
                                     nullptr), MOEF_ERR_BAD_SHAPE, false);
  check("finalize T huge", moe_finalize(at<uint16_t>(G2), 1, at<int32_t>(IDX), at<float>(W),
                                        nullptr, nullptr, 1.0f, at<uint16_t>(OUT), INT64_MAX, 8, 1,
                                        nullptr, nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("finalize H huge", moe_finalize(at<uint16_t>(G2), 1, at<int32_t>(IDX), at<float>(W),
                                        nullptr, nullptr, 1.0f, at<uint16_t>(OUT), 1,
                                        INT64_MAX - 7, 1, nullptr, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("finalize P huge", moe_finalize(at<uint16_t>(G2), INT64_MAX, at<int32_t>(IDX),
                                        at<float>(W), nullptr, nullptr, 1.0f, at<uint16_t>(OUT), 1,
                                        8, 1, nullptr, nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("finalize both formats", moe_finalize(at<uint16_t>(G2), 8, at<int32_t>(IDX), at<float>(W),
                                              at<int32_t>(PK), nullptr, 1.0f, at<uint16_t>(OUT), 2,
                                              8, 1, nullptr, nullptr), MOEF_ERR_BAD_FORMAT, false);
  check("finalize out overlaps gemm2_out", moe_finalize(at<uint16_t>(G2), 8, at<int32_t>(IDX),
                                                        at<float>(W), nullptr, nullptr, 1.0f,
                                                        at<uint16_t>(G2 + 16), 2, 8, 1, nullptr,
                                                        nullptr), MOEF_ERR_BAD_ALIAS, false);
  check("finalize with a separate err_flag", moe_finalize(at<uint16_t>(G2), 8, at<int32_t>(IDX),
                                                         at<float>(W), nullptr, nullptr, 1.0f,
                                                         at<uint16_t>(OUT), 2, 8, 1,
                                                         at<int32_t>(S), nullptr),
        MOEF_OK, true);
  check("finalize err_flag inside the index map", moe_finalize(at<uint16_t>(G2), 8,
                                                               at<int32_t>(IDX), at<float>(W),
                                                               nullptr, nullptr, 1.0f,
                                                               at<uint16_t>(OUT), 2, 8, 1,
                                                               at<int32_t>(IDX + 4), nullptr),
        MOEF_ERR_BAD_ALIAS, false);
  // residual + RMSNorm
  check("rmsnorm ok", moe_finalize_residual_rmsnorm(
      at<uint16_t>(G2), 4096, at<int32_t>(IDX), at<float>(W), nullptr, at<uint16_t>(SH), 2.5f,
      at<uint16_t>(RES), at<uint16_t>(GAM), 1e-6f, at<uint16_t>(RO), at<uint16_t>(NM), 1024,
      7168, 8, nullptr, nullptr), MOEF_OK, true);
  check("rmsnorm in place", moe_finalize_residual_rmsnorm(
      at<uint16_t>(G2), 4096, at<int32_t>(IDX), at<float>(W), nullptr, nullptr, 2.5f,
      at<uint16_t>(RES), at<uint16_t>(GAM), 1e-6f, at<uint16_t>(RES), at<uint16_t>(NM), 16,
      16384, 8, nullptr, nullptr), MOEF_OK, true);
  check("rmsnorm H too large", moe_finalize_residual_rmsnorm(
      at<uint16_t>(G2), 4096, at<int32_t>(IDX), at<float>(W), nullptr, nullptr, 2.5f,
      at<uint16_t>(RES), at<uint16_t>(GAM), 1e-6f, at<uint16_t>(RO), at<uint16_t>(NM), 16,
      16392, 8, nullptr, nullptr), MOEF_ERR_UNSUPPORTED, false);
  // quant
  check("quant ok", moe_finalize_quant_ue8m0(at<uint16_t>(G2), 81536, at<int32_t>(IDX),
                                             at<float>(W), nullptr, at<uint16_t>(SH), 2.5f,
                                             at<uint8_t>(Q), at<uint8_t>(S), 8192, 7168, 8, nullptr,
                                             nullptr), MOEF_OK, true);
  check("quant scales overlap codes", moe_finalize_quant_ue8m0(
      at<uint16_t>(G2), 8, at<int32_t>(IDX), at<float>(W), nullptr, nullptr, 1.0f, at<uint8_t>(Q),
      at<uint8_t>(Q + 100), 2, 128, 1, nullptr, nullptr), MOEF_ERR_BAD_ALIAS, false);
  // decode, gate, act quant, EP combine
  check("decode ok", moe_topk_packed_decode(at<int32_t>(PK), 65536, at<int32_t>(IDX),
                                            at<float>(W), nullptr), MOEF_OK, true);
  check("decode n huge", moe_topk_packed_decode(at<int32_t>(PK), INT64_MAX, at<int32_t>(IDX),
                                                at<float>(W), nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("decode MOEF_MAX_ITEMS", moe_topk_packed_decode(at<int32_t>(PK), MOEF_MAX_ITEMS,
                                                        at<int32_t>(IDX), at<float>(W), nullptr),
        MOEF_OK, true);
  check("decode MOEF_MAX_ITEMS + 1", moe_topk_packed_decode(at<int32_t>(PK), MOEF_MAX_ITEMS + 1,
                                                            at<int32_t>(IDX), at<float>(W),
                                                            nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("gate ok", moe_topk_sigmoid_gate(at<float>(G2), 8192, 256, 8, at<int32_t>(IDX),
                                         at<float>(W), at<int32_t>(PK), nullptr), MOEF_OK, true);
  check("gate T huge", moe_topk_sigmoid_gate(at<float>(G2), INT64_MAX, 256, 8, at<int32_t>(IDX),
                                             nullptr, nullptr, nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("gate MOEF_MAX_UNITS tokens", moe_topk_sigmoid_gate(at<float>(G2), MOEF_MAX_UNITS, 1, 1,
                                                            at<int32_t>(IDX), nullptr, nullptr,
                                                            nullptr), MOEF_OK, true);
  check("gate MOEF_MAX_UNITS + 1 tokens", moe_topk_sigmoid_gate(
      at<float>(G2), MOEF_MAX_UNITS + 1, 1, 1, at<int32_t>(IDX), nullptr, nullptr, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("act quant ue8m0 ok", moe_act_quant_fp8_ue8m0(at<uint16_t>(G2), 8192, 7168, at<uint8_t>(Q),
                                                      at<uint8_t>(S), nullptr), MOEF_OK, true);
  check("act quant amax ok", moe_act_quant_fp8_amax(at<uint16_t>(G2), 8192, 7168, at<uint8_t>(Q),
                                                    at<float>(S), nullptr), MOEF_OK, true);
  check("act quant H huge", moe_act_quant_fp8_amax(at<uint16_t>(G2), 1, INT64_MAX - 127,
                                                   at<uint8_t>(Q), at<float>(S), nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("act quant MOEF_MAX_UNITS chunks", moe_act_quant_fp8_ue8m0(
      at<uint16_t>(0x100000000000ull), MOEF_MAX_UNITS, 512, at<uint8_t>(0x300000000000ull),
      at<uint8_t>(0x400000000000ull), nullptr), MOEF_OK, true);
  check("act quant MOEF_MAX_UNITS + 1 chunks", moe_act_quant_fp8_ue8m0(
      at<uint16_t>(0x100000000000ull), MOEF_MAX_UNITS + 1, 512, at<uint8_t>(0x300000000000ull),
      at<uint8_t>(0x400000000000ull), nullptr), MOEF_ERR_UNSUPPORTED, false);
  check("ep combine ok", moe_finalize_ep_combine(at<uint16_t>(G2), 4, at<uint16_t>(SH),
                                                 at<uint16_t>(OUT), 8192, 7168, nullptr),
        MOEF_OK, true);
  check("ep combine T huge", moe_finalize_ep_combine(at<uint16_t>(G2), 4, nullptr,
                                                     at<uint16_t>(OUT), INT64_MAX, 8, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
  check("ep combine MOEF_MAX_ITEMS vectors", moe_finalize_ep_combine(
      at<uint16_t>(0x100000000000ull), 2, nullptr, at<uint16_t>(0x300000000000ull),
      MOEF_MAX_ITEMS / 16, 128, nullptr), MOEF_OK, true);
  check("ep combine MOEF_MAX_ITEMS + 16 vectors", moe_finalize_ep_combine(
      at<uint16_t>(0x100000000000ull), 2, nullptr, at<uint16_t>(0x300000000000ull),
      MOEF_MAX_ITEMS / 16 + 1, 128, nullptr), MOEF_ERR_UNSUPPORTED, false);
  // all-reduce + residual + RMSNorm: rank buffers 2^46 bytes apart hold the
  // largest accepted size (MOEF_MAX_UNITS / 32 tokens of 16384 columns)
  {
    const uint16_t* ranks[MOEF_MAX_AR_RANKS + 1];
    for (int r = 0; r <= MOEF_MAX_AR_RANKS; ++r)
      ranks[r] = at<uint16_t>(0x1000000000000ull + (uint64_t)r * 0x400000000000ull);
    const uint64_t top = 0x1000000000000ull + 0x400000000000ull * (MOEF_MAX_AR_RANKS + 1);
    uint16_t* res = at<uint16_t>(top);
    uint16_t* ro = at<uint16_t>(top + 0x400000000000ull);
    uint16_t* nm = at<uint16_t>(top + 0x800000000000ull);
    const uint16_t* gam = at<uint16_t>(0x1000);
    check("allreduce ok", moe_allreduce_residual_rmsnorm(ranks, 8, res, gam, 1e-6f, ro, nm, 256,
                                                         7168, nullptr), MOEF_OK, true);
    check("allreduce largest sizes", moe_allreduce_residual_rmsnorm(
        ranks, MOEF_MAX_AR_RANKS, res, gam, 1e-6f, ro, nm, MOEF_MAX_UNITS / 32, 16384, nullptr),
        MOEF_OK, true);
    check("allreduce one token beyond", moe_allreduce_residual_rmsnorm(
        ranks, 2, res, gam, 1e-6f, ro, nm, MOEF_MAX_UNITS / 32 + 1, 16384, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
    check("allreduce in place", moe_allreduce_residual_rmsnorm(ranks, 3, res, gam, 1e-6f, res, nm,
                                                               16, 7168, nullptr), MOEF_OK, true);
    check("allreduce T beyond 2^31 - 1", moe_allreduce_residual_rmsnorm(
        ranks, 2, res, gam, 1e-6f, ro, nm, (int64_t)INT32_MAX + 1, 8, nullptr),
        MOEF_ERR_UNSUPPORTED, false);
    check("allreduce no ranks", moe_allreduce_residual_rmsnorm(ranks, 0, res, gam, 1e-6f, ro, nm,
                                                               16, 7168, nullptr),
          MOEF_ERR_BAD_SHAPE, false);
    check("allreduce too many ranks", moe_allreduce_residual_rmsnorm(
        ranks, MOEF_MAX_AR_RANKS + 1, res, gam, 1e-6f, ro, nm, 16, 7168, nullptr),
        MOEF_ERR_BAD_SHAPE, false);
    check("allreduce T=0", moe_allreduce_residual_rmsnorm(nullptr, 4, nullptr, nullptr, 1e-6f,
                                                          nullptr, nullptr, 0, 7168, nullptr),
          MOEF_OK, false);
    const uint16_t* with_null[3] = {ranks[0], nullptr, ranks[2]};
    check("allreduce NULL rank", moe_allreduce_residual_rmsnorm(with_null, 3, res, gam, 1e-6f, ro,
                                                                nm, 16, 7168, nullptr),
          MOEF_ERR_NULL_POINTER, false);
    const uint16_t* odd[2] = {ranks[0], at<uint16_t>(0x1000000000000ull + 0x400000000000ull + 8)};
    check("allreduce misaligned rank", moe_allreduce_residual_rmsnorm(odd, 2, res, gam, 1e-6f, ro,
                                                                      nm, 16, 7168, nullptr),
          MOEF_ERR_MISALIGNED, false);
    check("allreduce normed overlaps a rank", moe_allreduce_residual_rmsnorm(
        ranks, 4, res, gam, 1e-6f, ro, at<uint16_t>(0x1000000000000ull + 3 * 0x400000000000ull + 64),
        16, 7168, nullptr), MOEF_ERR_BAD_ALIAS, false);
    check("allreduce residual_out overlaps residual", moe_allreduce_residual_rmsnorm(
        ranks, 4, res, gam, 1e-6f, res + 8, nm, 16, 7168, nullptr), MOEF_ERR_BAD_ALIAS, false);
    check("allreduce H too large", moe_allreduce_residual_rmsnorm(ranks, 4, res, gam, 1e-6f, ro, nm,
                                                                  16, 16392, nullptr),
          MOEF_ERR_UNSUPPORTED, false);
  }
  if (failures) {
    std::fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  std::printf("host_checks: ok\n");
  return 0;
}
