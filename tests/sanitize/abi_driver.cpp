// Drives the C ABI's host paths (include/ll_attn.h) without a GPU: every
// validation error of every entry point, the workspace and state size
// queries, calls that pass validation and reach a (stubbed, failing) launch,
// and kernel timing switched on and off from one thread while another thread
// makes calls.  Built twice by tests/test_sanitize.py, with AddressSanitizer +
// UndefinedBehaviorSanitizer and with ThreadSanitizer, on the host code only.
// Exit status 0 = every call returned the expected status.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <thread>

#include "ll_attn.h"

static int failures = 0;
static void expect(ll_status got, ll_status want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, ll_last_error());
    failures++;
  }
}

int main() {
  void* d = reinterpret_cast<void*>(0x1000);  // never dereferenced on the host
  const float* f = static_cast<const float*>(d);
  float* fw = static_cast<float*>(d);
  ll_problem p = {2, 16384, 16, 64, 64, 15, 64, LL_BF16, LL_MAMBA2};
  size_t bytes = 0;
  expect(ll_attn_fwd_workspace_bytes(&p, &bytes), LL_OK, "workspace bytes");
  expect(ll_attn_fwd_workspace_bytes(nullptr, &bytes), LL_ERR_NULL, "workspace bytes of NULL");
  ll_problem bad = p;
  bad.C = 48;
  expect(ll_attn_fwd(&bad, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_SHAPE, "C = 48");
  bad = p;
  bad.L = 3;
  expect(ll_attn_fwd(&bad, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_SHAPE, "too few levels");
  bad = p;
  bad.io = static_cast<ll_dtype>(7);
  expect(ll_attn_fwd(&bad, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_DTYPE, "io dtype");
  expect(ll_attn_fwd(&p, d, nullptr, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_NULL, "NULL k");
  expect(ll_attn_fwd(&p, d, d, d, f, f, nullptr, d, nullptr, d, bytes - 1, nullptr), LL_ERR_WORKSPACE,
         "short workspace");
  // passes validation; the stubbed launch fails
  expect(ll_attn_fwd(&p, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_HIP, "stubbed launch");
  ll_problem big = p;
  big.B = 16;  // 16 x 16 heads x 16384 tokens: 100 MB of block states and nodes
  expect(ll_attn_fwd_noalloc(&big, d, d, d, f, f, nullptr, d, nullptr, nullptr), LL_ERR_WORKSPACE,
         "noalloc beyond the scratch");
  expect(ll_attn_fwd_from_state(&p, 3, f, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr), LL_ERR_POSITION,
         "from_state with T > lowbit(pos0)");
  expect(ll_decode_step(64, 16, 64, 64, 17, LL_BF16, LL_MAMBA2, 1 << 16, d, d, d, f, f, nullptr, d, d, nullptr),
         LL_ERR_POSITION, "decode position beyond the levels");
  expect(ll_decode_step(64, 16, 64, 64, 17, LL_BF16, LL_GATED_DELTANET, 5, d, d, d, f, f, nullptr, d, d, nullptr),
         LL_ERR_NULL, "decode without beta");
  expect(ll_decode_step_ragged(64, 16, 64, 64, 17, LL_BF16, LL_MAMBA2, nullptr, d, d, d, f, f, nullptr, d, d,
                               nullptr),
         LL_ERR_NULL, "ragged decode without positions");
  expect(ll_lambda_mlp(10, 33, 8, f, f, f, f, fw, nullptr), LL_ERR_UNSUPPORTED, "MLP with 33 levels");
  expect(ll_lambda_mlp(0, 15, 30, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), LL_OK, "MLP of no rows");
  size_t cb = 0;
  expect(ll_ccq_query_workspace_bytes(2, 16384, 16, 64, LL_BF16, &cb), LL_OK, "ccq workspace");
  expect(ll_ccq_query(2, 16384, 16, 64, LL_BF16, d, d, f, f, d, d, cb - 1, nullptr), LL_ERR_WORKSPACE, "ccq short");
  size_t bb = 0;
  ll_problem q = {4, 2048, 16, 64, 64, 12, 64, LL_BF16, LL_MAMBA2};
  expect(ll_attn_bwd_workspace_bytes(&q, &bb), LL_OK, "bwd workspace");
  expect(ll_attn_bwd(&q, d, d, d, f, f, d, nullptr, d, d, d, fw, fw, d, bb, nullptr), LL_ERR_NULL, "bwd NULL dO");
  size_t sb = 0;
  expect(ll_decode_state_bytes(64, 16, 64, 64, 17, &sb), LL_OK, "state bytes");
  if (sb != (size_t)64 * 16 * 17 * (64 * 64 + 1) * 4) failures++;

  // kernel timing toggled while another thread calls through the timed launch path
  std::atomic<bool> stop{false};
  std::thread caller([&] {
    for (int i = 0; i < 2000; ++i) {
      if (ll_attn_fwd(&p, d, d, d, f, f, nullptr, d, nullptr, d, bytes, nullptr) != LL_ERR_HIP) failures++;
    }
    stop = true;
  });
  while (!stop) {
    ll_kernel_timing_enable(1);
    ll_kernel_timing_enable(0);
  }
  caller.join();
  const char* names[16];
  double ms[16];
  int launches[16], count = 0;
  expect(ll_kernel_timing_read(names, ms, launches, 16, &count), LL_OK, "timing read");
  if (failures) fprintf(stderr, "%d failures\n", failures);
  else printf("abi driver: all calls returned as expected\n");
  return failures ? 1 : 0;
}
