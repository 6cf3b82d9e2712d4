// Host-side checks of the C ABI (no GPU needed), built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code of every library source:
// every entry point's argument validation, the size queries and the trace
// calls that launch nothing. Exit status 0 when every status matches.
#include <cstdint>
#include <cstdio>

#include "gmla.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, gmla_last_error());
    ++failures;
  }
}

int main() {
  void* A = (void*)0x100000;  // aligned, never dereferenced: every call below fails validation first
  const int64_t* S = (const int64_t*)A;
  const int32_t* N = (const int32_t*)A;
  const size_t big = (size_t)1 << 40;
  // decode
  expect(gmla_decode(nullptr, A, S, N, A, nullptr, A, big, 4, 64, 512, 0, 1e4f, 0.1f, 0, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "decode null q");
  expect(gmla_decode(A, (char*)A + 8, S, N, A, nullptr, A, big, 4, 64, 512, 0, 1e4f, 0.1f, 0, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "decode misaligned cache");
  expect(gmla_decode(A, A, S, N, A, nullptr, A, big, 4, 64, 512, 3, 1e4f, 0.1f, 0, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "decode odd d_r");
  expect(gmla_decode(A, A, S, N, A, nullptr, A, big, 4, 64, 96, 0, 1e4f, 0.1f, 0, GMLA_BF16, nullptr),
         GMLA_ERR_UNSUPPORTED, "decode d_c 96");
  expect(gmla_decode(A, A, S, N, A, nullptr, A, 16, 4, 64, 512, 0, 1e4f, 0.1f, 0, GMLA_BF16, nullptr),
         GMLA_ERR_WORKSPACE, "decode workspace");
  expect(gmla_decode(A, A, S, N, A, nullptr, A, big, 4, 64, 512, 0, 1e4f, 0.1f, -1, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "decode splits");
  expect(gmla_decode_noalloc(A, A, S, N, A, nullptr, 64, 128, 512, 64, 1e4f, 0.1f, 65535, GMLA_BF16, nullptr),
         GMLA_ERR_UNSUPPORTED, "decode_noalloc scratch");
  // prefill
  expect(gmla_prefill(A, A, nullptr, nullptr, nullptr, nullptr, A, A, A, A, A, big, 1, 16, 256, 2, 128, 0, 128, 0, 128,
                      0.1f, 0.f, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "prefill null W_q");
  expect(gmla_prefill(A, A, nullptr, A, nullptr, nullptr, A, A, A, A, A, big, 1, 16, 100, 2, 128, 0, 128, 0, 128, 0.1f,
                      0.f, GMLA_BF16, nullptr),
         GMLA_ERR_UNSUPPORTED, "prefill d_model");
  expect(gmla_prefill(A, A, nullptr, A, nullptr, nullptr, A, A, A, A, A, big, 2, 1 << 30, 64, 1, 64, 0, 64, 0, 64, 0.1f,
                      0.f, GMLA_F32, nullptr),
         GMLA_ERR_UNSUPPORTED, "prefill B*L past INT_MAX");
  expect(gmla_prefill(A, A, nullptr, A, nullptr, nullptr, A, A, A, A, A, 100, 1, 16, 256, 2, 128, 0, 128, 0, 128, 0.1f,
                      0.f, GMLA_BF16, nullptr),
         GMLA_ERR_WORKSPACE, "prefill workspace");
  // decode-step projections
  expect(gmla_decode_prepare(A, A, A, nullptr, A, A, A, A, S, N, A, A, big, 4, 256, 16, 512, 0, 128, 64, 1e4f,
                             GMLA_F32, nullptr),
         GMLA_ERR_UNSUPPORTED, "prepare fp32");
  expect(gmla_decode_prepare(A, A, A, nullptr, A, A, A, A, S, N, A, A, big, 4, 256, 16, 512, 0, 136, 64, 1e4f,
                             GMLA_BF16, nullptr),
         GMLA_ERR_UNSUPPORTED, "prepare d_k");
  // gate and output
  expect(gmla_gate_out(A, A, nullptr, A, A, nullptr, A, big, 4, 256, 2, 0, 128, GMLA_BF16, nullptr),
         GMLA_ERR_INVALID_ARG, "gate_out null y");
  expect(gmla_gate_out(A, A, nullptr, A, A, A, A, big, 4, 100, 2, 0, 128, GMLA_BF16, nullptr), GMLA_ERR_UNSUPPORTED,
         "gate_out d_model");
  expect(gmla_head_gate_out(A, A, nullptr, A, nullptr, A, A, A, big, 4, 256, 3, 0, 128, GMLA_BF16, nullptr),
         GMLA_ERR_UNSUPPORTED, "head_gate_out H");
  // size queries
  if (gmla_decode_workspace_size(0, 64, 512, 0, GMLA_BF16) != 0) ++failures;
  if (gmla_decode_workspace_size(4, 64, 256, 8, GMLA_BF16) != 0) ++failures;
  if (gmla_prefill_workspace_size(1, 16, 2, 0, 128, 0, 128, GMLA_BF16) == 0) ++failures;
  if (gmla_gate_out_workspace_size(32, 7168, 64, 512, 128, 1, GMLA_BF16) == 0) ++failures;
  // diagnostics and the trace, without launches
  if (gmla_version() < 10000) ++failures;
  expect(gmla_trace_begin(0), GMLA_ERR_INVALID_ARG, "trace_begin 0");
  int count = -1;
  double ms = -1.0;
  expect(gmla_trace_summary(nullptr, &count, &ms), GMLA_ERR_INVALID_ARG, "trace_summary null");
  gmla_trace_reset();
  std::printf("abi_check: %s (%s)\n", failures ? "FAILED" : "ok", gmla_status_string(GMLA_ERR_WORKSPACE));
  return failures ? 1 : 0;
}
