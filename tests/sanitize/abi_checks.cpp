// Host-only exercise of libgsa's argument checks, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py).
// Every call either fails validation or, on a host without a GPU, stops at the
// device check; no pointer handed to the library is ever dereferenced.  Sizes
// reach the int64 extremes so that the checks' own arithmetic (products of
// sizes) is exercised where it could overflow.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "gsa.h"

namespace {
int g_fail = 0;
bool g_gpu = false;
void* const P = reinterpret_cast<void*>(0x100000);       // 16-byte aligned, never dereferenced
void* const P2 = reinterpret_cast<void*>(0x40000000);    // another, far from P
void* const MIS = reinterpret_cast<void*>(0x100004);
float* const F = static_cast<float*>(P);
constexpr int64_t BIG = INT64_MAX;
constexpr int64_t HUGE2 = (int64_t)1 << 40;

void expect(const char* what, int got, std::initializer_list<int> want) {
  for (int w : want)
    if (got == w) return;
  std::fprintf(stderr, "FAIL %s: status %d (%s): %s\n", what, got, gsa_status_string(got), gsa_last_error_message());
  ++g_fail;
}
// a call with valid arguments: GSA_ERR_NO_DEVICE on a host without a GPU (with
// a GPU it would launch, so it is skipped there)
#define VALID(what, call) \
  do {                    \
    if (!g_gpu) expect(what, (call), {GSA_ERR_NO_DEVICE}); \
  } while (0)
}  // namespace

int main() {
  int n = 0;
  g_gpu = hipGetDeviceCount(&n) == hipSuccess && n > 0;
  (void)hipGetLastError();
  const int INV = GSA_ERR_INVALID_ARG, UNS = GSA_ERR_UNSUPPORTED, MISA = GSA_ERR_MISALIGNED, WS = GSA_ERR_WORKSPACE;

  // status strings and version
  for (int s = -1; s <= 8; ++s) expect("status string", gsa_status_string(s)[0] == 'G', {1});
  expect("version", gsa_version() > 0, {1});

  // gate logits
  expect("gate null", gsa_gate_logits(nullptr, P, F, 8, 64, 8, 1, 1, nullptr), {INV});
  expect("gate sizes", gsa_gate_logits(P, P, F, 0, 64, 8, 1, 1, nullptr), {INV});
  expect("gate act", gsa_gate_logits(P, P, F, 8, 64, 8, 1, 7, nullptr), {INV});
  expect("gate dm", gsa_gate_logits(P, P, F, 8, 60, 8, 1, 1, nullptr), {UNS});
  expect("gate huge", gsa_gate_logits(P, P, F, BIG, BIG, BIG, 1, 1, nullptr), {UNS, INV});
  expect("gate mis", gsa_gate_logits(P, MIS, F, 8, 64, 8, 1, 1, nullptr), {MISA});
  VALID("gate ok", gsa_gate_logits(P, P, F, 8, 64, 8, 1, 1, nullptr));

  // forward / forward_lse
  expect("fwd null", gsa_forward(nullptr, P, P, F, P, 1, 8, 4, 2, 128, 1, 1, nullptr), {INV});
  expect("fwd heads", gsa_forward(P, P, P, F, P, 1, 8, 4, 3, 128, 1, 1, nullptr), {INV});
  expect("fwd mode", gsa_forward(P, P, P, F, P, 1, 8, 4, 2, 128, 9, 1, nullptr), {INV});
  expect("fwd gate", gsa_forward(P, P, P, nullptr, P, 1, 8, 4, 2, 128, 1, 1, nullptr), {INV});
  expect("fwd D", gsa_forward(P, P, P, F, P, 1, 8, 4, 2, 96, 1, 1, nullptr), {UNS});
  expect("fwd huge BS", gsa_forward(P, P, P, F, P, BIG, BIG, 4, 2, 128, 1, 1, nullptr), {UNS});
  expect("fwd huge B", gsa_forward(P, P, P, F, P, HUGE2, HUGE2, 4, 2, 128, 1, 1, nullptr), {UNS});
  expect("fwd huge H", gsa_forward(P, P, P, F, P, 1, 8, BIG, 1, 128, 1, 1, nullptr), {UNS});
  expect("fwd huge S", gsa_forward(P, P, P, F, P, 1, BIG / 2, 4, 2, 128, 1, 1, nullptr), {UNS});
  expect("fwd mis", gsa_forward(P, P, MIS, F, P, 1, 8, 4, 2, 128, 1, 1, nullptr), {MISA});
  expect("lse null", gsa_forward_lse(P, P, P, F, P, nullptr, 1, 8, 4, 2, 128, 1, 1, nullptr), {INV});
  VALID("fwd ok", gsa_forward(P, P, P, F, P, 2, 100, 8, 2, 128, 1, 1, nullptr));
  VALID("lse ok", gsa_forward_lse(P, P, P, F, P, F, 2, 100, 8, 2, 64, 2, 1, nullptr));

  // decode, its size queries and the no-allocation variant
  expect("splits bad", (int)gsa_decode_num_splits(0, 10, 4, 2, 128, 0), {0});
  expect("splits huge", gsa_decode_num_splits(BIG, BIG, BIG, 1, 128, 0) >= 0, {1});
  expect("ws huge", gsa_decode_workspace_bytes(BIG, BIG, BIG, 1, 128, 0) >= 0, {1});
  expect("dec null", gsa_decode(nullptr, P, P, F, P, 2, 100, 8, 2, 128, 1, 1, 0, P2, 1 << 30, nullptr), {INV});
  expect("dec ns", gsa_decode(P, P, P, F, P, 2, 100, 8, 2, 128, 1, 1, -1, P2, 1 << 30, nullptr), {INV});
  expect("dec ws", gsa_decode(P, P, P, F, P, 2, 100, 8, 2, 128, 1, 1, 0, P2, 16, nullptr), {WS});
  expect("dec huge", gsa_decode(P, P, P, F, P, BIG, BIG, 8, 2, 128, 1, 1, 0, P2, 1 << 30, nullptr), {UNS});
  expect("dec huge2", gsa_decode(P, P, P, F, P, HUGE2, HUGE2, 8, 2, 128, 1, 1, 0, P2, 1 << 30, nullptr), {UNS});
  VALID("dec ok", gsa_decode(P, P, P, F, P, 2, 100, 8, 2, 128, 1, 1, 0, P2, 1 << 30, nullptr));
  expect("noalloc scratch", gsa_noalloc_scratch_bytes() == GSA_NOALLOC_SCRATCH_BYTES, {1});
  expect("noalloc big", gsa_decode_noalloc(P, P, P, F, P, 64, 16384, 32, 8, 128, 1, 1, 8, nullptr), {WS});
  expect("noalloc huge", gsa_decode_noalloc(P, P, P, F, P, BIG, BIG, 32, 8, 128, 1, 1, 0, nullptr), {UNS});
  VALID("noalloc ok", gsa_decode_noalloc(P, P, P, F, P, 64, 16384, 32, 8, 128, 1, 1, 0, nullptr));
  expect("gdec ws huge", gsa_gated_decode_workspace_bytes(BIG, BIG, BIG, 1, 128, BIG, 1, 1, 0) >= 0, {1});
  expect("gdec ws huge2", gsa_gated_decode_workspace_bytes(HUGE2, 2, 4096, 1, 4096, HUGE2, 1, 1, 0) == 0, {1});
  const size_t gws = gsa_gated_decode_workspace_bytes(64, 16384, 32, 8, 128, 4096, 1, 1, 0);
  expect("gdec ws", gws > 0, {1});
  expect("gdec null", gsa_gated_decode(nullptr, P, P, P, P, P, 64, 16384, 32, 8, 128, 4096, 1, 1, 0, P2, gws,
                                       nullptr), {INV});
  expect("gdec ws small", gsa_gated_decode(P, P, P, P, P, P, 64, 16384, 32, 8, 128, 4096, 1, 1, 0, P2, 16,
                                           nullptr), {WS});
  expect("gdec huge", gsa_gated_decode(P, P, P, P, P, P, BIG, BIG, 32, 8, 128, 4096, 1, 1, 0, P2, gws, nullptr),
         {UNS});
  expect("gdec huge dm", gsa_gated_decode(P, P, P, P, P, P, 64, 16, 32, 8, 128, HUGE2, 1, 1, 0, P2, gws, nullptr),
         {UNS, INV});
  VALID("gdec ok", gsa_gated_decode(P, P, P, P, P, P, 64, 16384, 32, 8, 128, 4096, 1, 1, 0, P2, gws, nullptr));
  VALID("gdec none", gsa_gated_decode(nullptr, nullptr, P, P, P, P, 2, 100, 8, 2, 128, 0, 0, 1, 0, P2, 1 << 30,
                                      nullptr));
  expect("dvar layout", gsa_decode_variant(P, P, P, F, P, 2, 100, 8, 2, 128, 5, 0, 0, 1, 0, P2, 1 << 30, nullptr),
         {INV});
  VALID("dvar ok", gsa_decode_variant(P, P, P, F, P, 2, 100, 8, 2, 128, 3, 1, 1, 1, 0, P2, 1 << 30, nullptr));

  // backward and its workspace query
  expect("bws huge", gsa_backward_workspace_bytes(BIG, BIG, BIG, 1, 128, BIG, 1) == 0, {1});
  expect("bws huge2", gsa_backward_workspace_bytes(HUGE2, HUGE2, 8, 1, 128, HUGE2, 1) == 0, {1});
  const size_t bws = gsa_backward_workspace_bytes(1, 64, 4, 2, 128, 64, 1);
  expect("bws ok", bws > 0, {1});
  expect("bwd null", gsa_backward(P, P, F, P, P, P, P, F, nullptr, P, F, P, P, P, 1, 64, 4, 2, 128, 64, 1, 1, P2,
                                  bws, nullptr), {INV});
  expect("bwd fp32", gsa_backward(P, P, F, P, P, P, P, F, P, P, F, P, P, P, 1, 64, 4, 2, 128, 64, 1, 0, P2, bws,
                                  nullptr), {UNS});
  expect("bwd ws", gsa_backward(P, P, F, P, P, P, P, F, P, P, F, P, P, P, 1, 64, 4, 2, 128, 64, 1, 1, P2, 16,
                                nullptr), {WS});
  expect("bwd huge", gsa_backward(P, P, F, P, P, P, P, F, P, P, F, P, P, P, 1, 64, 4, 2, 128, BIG, 1, 1, P2, bws,
                                  nullptr), {UNS, INV});
  VALID("bwd ok", gsa_backward(P, P, F, P, P, P, P, F, P, P, F, P, P, P, 1, 64, 4, 2, 128, 64, 1, 1, P2, bws,
                               nullptr));

  // variants, projection, value gate, head mean, first-token share
  expect("fvar combine", gsa_forward_variant(P, P, P, F, P, nullptr, 1, 8, 4, 2, 128, 1, 5, 0, 1, nullptr), {INV});
  VALID("fvar ok", gsa_forward_variant(P, P, P, F, P, nullptr, 1, 8, 4, 2, 128, 3, 1, 1, 1, nullptr));
  expect("proj huge", gsa_project_qkvg(P, P, P, P, P, F, BIG, BIG, 4, 2, 128, 512, 1, nullptr), {UNS, INV});
  expect("proj huge2", gsa_project_qkvg(P, P, P, P, P, F, HUGE2, HUGE2, 4, 2, 128, 512, 1, nullptr), {UNS});
  expect("proj gate", gsa_project_qkvg(P, P, P, P, P, nullptr, 64, 64, 4, 2, 128, 512, 1, nullptr), {INV});
  VALID("proj ok", gsa_project_qkvg(P, P, P, P, P, F, 64, 64, 4, 2, 128, 512, 1, nullptr));
  expect("vg layout", gsa_value_gate(P, F, P2, 1, 8, 2, 128, 3, 1, nullptr), {INV});
  expect("vg huge", gsa_value_gate(P, F, P2, BIG, BIG, 2, 128, 1, 1, nullptr), {UNS});
  VALID("vg ok", gsa_value_gate(P, F, P2, 1, 8, 2, 128, 1, 1, nullptr));
  expect("hm overlap", gsa_gate_head_mean(F, F + 4, 8, 4, 64, nullptr), {INV});
  expect("hm huge", gsa_gate_head_mean(F, static_cast<float*>(P2), BIG, 4, 64, nullptr), {UNS});
  expect("hm huge2", gsa_gate_head_mean(F, static_cast<float*>(P2), HUGE2, 4096, 4096, nullptr), {UNS});
  VALID("hm ok", gsa_gate_head_mean(F, static_cast<float*>(P2), 8, 4, 64, nullptr));
  expect("ft null", gsa_first_token_attention(P, P, nullptr, F, nullptr, 1, 8, 4, 2, 128, 1, nullptr), {INV});
  VALID("ft ok", gsa_first_token_attention(P, P, F, static_cast<float*>(P2), nullptr, 1, 8, 4, 2, 128, 1, nullptr));

  // the per-thread message is a valid C string
  expect("message", (int)(std::strlen(gsa_last_error_message()) < 4096), {1});
  std::printf("abi checks: %s (%d failures, gpu visible: %d)\n", g_fail ? "FAIL" : "ok", g_fail, (int)g_gpu);
  return g_fail ? 1 : 0;
}
