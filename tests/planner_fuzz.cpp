// Host-only fuzz driver for the attention library's host planner (layout and
// batch checks, launch classification, workspace sizing, launch-table fill),
// built with the address and undefined-behaviour sanitizers on the host side
// by tests/test_planner_sanitize.py.  Random layouts and batches, well formed
// and malformed, go through attention_workspace_bytes, kv_append_quant and
// mixed_attention_fwd with placeholder device addresses.
//
// The placeholder addresses are never dereferenced on the host.  The calls
// that would enqueue kernels run only when no device is visible (the launch
// then fails with MAB_ERR_HIP and nothing runs); with a device present, only
// the calls that return before any launch are made.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "mab.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static const uintptr_t kFakeDev = 0x7F0000000000ull;  // 256-byte aligned, never dereferenced

static int run(uint64_t seed, bool may_launch) {
  std::mt19937_64 rng(seed);
  auto uni = [&](int64_t lo, int64_t hi) { return (int64_t)(lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1))); };
  const int fmts[3] = {MAB_KV_Q8, MAB_KV_Q4, MAB_KV_F16};
  mab_kv_layout L;
  L.num_kv_heads = (int32_t)uni(1, 8);
  L.num_q_heads = L.num_kv_heads * (int32_t)uni(1, 9);  // groups up to 9: 9 is unsupported
  L.head_dim = uni(0, 9) == 0 ? (int32_t)uni(1, 300) : (uni(0, 1) ? 64 : 128);
  L.page_size = uni(0, 9) == 0 ? (int32_t)uni(-3, 70) : 16 * (int32_t)uni(1, 20);
  L.num_pages = (int32_t)uni(0, 1 << 20);
  L.k_format = fmts[uni(0, 2)];
  L.v_format = uni(0, 3) == 0 ? fmts[uni(0, 2)] : L.k_format;
  L.reserved = uni(0, 30) == 0 ? 1 : 0;

  const int num_seqs = (int)uni(0, 300);
  std::vector<int32_t> q_start(num_seqs + 1), prefix(num_seqs > 0 ? num_seqs : 1);
  q_start[0] = 0;
  const int kind = (int)uni(0, 3);  // 0: decode rows only, 1: verify rows, 2: chunks, 3: a mix
  for (int s = 0; s < num_seqs; ++s) {
    int q_len = 1;
    if (kind == 1) q_len = (int)uni(1, 16);
    if (kind == 2) q_len = (int)uni(17, 3000);
    if (kind == 3) q_len = uni(0, 4) == 0 ? (int)uni(2, 2500) : 1;
    if (uni(0, 200) == 0) q_len = (int)uni(-2, 0);  // malformed
    q_start[s + 1] = q_start[s] + q_len;
    prefix[s] = (int32_t)uni(0, 300000);
    if (uni(0, 300) == 0) prefix[s] = (int32_t)uni(-5, -1);  // malformed
  }
  int64_t max_ctx = 1;
  for (int s = 0; s < num_seqs; ++s) max_ctx = std::max<int64_t>(max_ctx, (int64_t)prefix[s] + q_start[s + 1] - q_start[s]);
  mab_batch B;
  B.num_seqs = num_seqs;
  B.num_rows = q_start[num_seqs] + (uni(0, 100) == 0 ? 1 : 0);  // sometimes inconsistent
  const int64_t ps = L.page_size > 0 ? L.page_size : 16;
  B.max_pages_per_seq = (int32_t)std::min<int64_t>(1 << 30, (max_ctx + ps - 1) / ps + (uni(0, 50) == 0 ? -1 : 0));
  B.flags = uni(0, 1) ? MAB_BATCH_INVARIANT : 0;
  if (uni(0, 100) == 0) B.flags = (int32_t)uni(2, 9);  // unknown flag bits: refused
  B.q_start = (const int32_t*)kFakeDev;
  B.prefix_len = (const int32_t*)kFakeDev;
  B.block_table = (const int32_t*)kFakeDev;
  B.q_start_host = q_start.data();
  B.prefix_len_host = prefix.data();

  const int64_t ws = attention_workspace_bytes(&L, &B);
  CHECK(ws >= -8);
  const int64_t ws2 = attention_workspace_bytes(&L, &B);
  CHECK(ws == ws2);  // a pure function of the layout and the batch (and the device)
  if (ws < 0) {
    // the entry points return the same error before anything is enqueued
    void* d = (void*)kFakeDev;
    CHECK(mixed_attention_fwd(&L, &B, d, d, d, 0.125f, (float*)d, d, 1 << 20, nullptr) == (int32_t)-ws);
    return 0;
  }
  if (L.reserved == 0) {
    CHECK(kv_pool_bytes(&L, L.k_format) > 0);
  }
  void* d = (void*)kFakeDev;
  // workspace one byte short: refused before any launch
  if (ws > 0 && B.num_rows > 0) CHECK(mixed_attention_fwd(&L, &B, d, d, d, 0.125f, (float*)d, d, ws - 1, nullptr) == MAB_ERR_WORKSPACE);
  // a bad softmax scale: refused before any launch
  CHECK(mixed_attention_fwd(&L, &B, d, d, d, -1.f, (float*)d, d, ws, nullptr) == MAB_ERR_UNSUPPORTED);
  if (may_launch) {
    // no device: the launch itself fails, after the launch tables are filled
    const int32_t st = mixed_attention_fwd(&L, &B, d, d, d, 0.125f, (float*)d, d, ws, nullptr);
    CHECK(st == MAB_OK || st == MAB_ERR_HIP);
    const int32_t st2 = kv_append_quant(&L, &B, d, d, d, d, nullptr);
    CHECK(st2 == MAB_OK || st2 == MAB_ERR_HIP);
    // the no-allocation call finds no device to take its array from
    CHECK(mixed_attention_fwd_noalloc(&L, &B, d, d, d, 0.125f, (float*)d, nullptr) == MAB_ERR_HIP);
  }
  return 0;
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 200;
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess) devices = 0;
  const bool may_launch = devices == 0;
  for (int i = 0; i < n; ++i) {
    if (run(0x9E3779B97F4A7C15ull * (uint64_t)(i + 1), may_launch)) {
      fprintf(stderr, "case %d failed\n", i);
      return 1;
    }
  }
  printf("ok %d%s\n", n, may_launch ? "" : " (device present: launching calls skipped)");
  return 0;
}
