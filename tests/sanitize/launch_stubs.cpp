// Host-only stand-ins for the kernel launchers of libtq, so that the host code
// (tq_host.cpp) can be built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer with g++ and no GPU.  Each stub checks the
// argument block the host code built and counts the launch.
#include <cstdio>
#include <cstdlib>

#include "tq_common.h"

namespace tq {

int g_launches = 0;

static void expect(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "stub check failed: %s\n", what);
    std::abort();
  }
}

int launch_quantize(int d, const QuantArgs &a, hipStream_t) {
  expect(d == 64 || d == 128 || d == 256, "quantize d");
  expect(a.t.x != nullptr && a.t.idx != nullptr && a.t.scl != nullptr, "quantize tensor pointers");
  expect(a.batch > 0 && a.n_new > 0 && a.H > 0, "quantize sizes");
  ++g_launches;
  return 0;
}

int launch_quantize_fast(int d, const QuantArgs &a, hipStream_t s) {
  expect(a.n_tensor == 1 || a.n_tensor == 2, "quantize tensor count");
  if (a.n_tensor == 2) expect(a.t2.x != nullptr && a.t2.bq == a.t.bq, "second tensor");
  return launch_quantize(d, a, s);
}

int launch_decode(int d, const DecodeArgs &a, hipStream_t) {
  expect(d == 64 || d == 128 || d == 256, "decode d");
  expect(a.part != nullptr && a.out != nullptr && a.n_split >= 1, "decode workspace");
  expect(a.split_tokens > 0 && a.split_tokens % 256 == 0, "split length");
  ++g_launches;
  return 0;
}

int launch_decode_fast(int d, int rb, const DecodeArgs &a, hipStream_t s, bool) {
  expect(rb == 1 || rb == 2, "row blocks");
  expect(a.qop != nullptr && a.qscale != nullptr, "query operands");
  return launch_decode(d, a, s);
}

int launch_score_fast(int d, const DecodeArgs &a, hipStream_t) {
  expect(d == 128 || d == 256, "score d");
  expect(a.scores != nullptr && a.score_dummy != nullptr && a.kv_fixed >= 0, "score arguments");
  ++g_launches;
  return 0;
}

}  // namespace tq
