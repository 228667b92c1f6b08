// Host-only fuzz driver for the planner and validator (test infrastructure).
// Built with g++ and AddressSanitizer/UBSan by tests/test_host_sanitize.py:
// any out-of-bounds access, overflow or misuse aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "hda.h"

static int fail(const char* what, int iter) {
  fprintf(stderr, "FAIL %s at iteration %d\n", what, iter);
  return 1;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  for (int it = 0; it < iters; ++it) {
    const int B = 1 + (int)(rng() % 300);
    const int hi = (int)(rng() % 4 == 0 ? 3 : rng() % 2 ? 2000 : 200000);
    std::vector<int32_t> lens(B);
    for (auto& L : lens) L = 1 + (int32_t)(rng() % hi);
    const bool dyn = rng() % 2;
    const int32_t tl = 1 + (int32_t)(rng() % 600), W = 1 + (int32_t)(rng() % 2000);
    const int32_t S = 1 + (int32_t)(rng() % 80);
    int64_t need = 0;
    int st = dyn ? hda_plan(lens.data(), B, tl, W, nullptr, 0, &need)
                 : hda_plan_static(lens.data(), B, S, nullptr, 0, &need);
    if (st != HDA_ERR_CAPACITY || need <= HDA_PLAN_HEADER_INTS) return fail("size query", it);
    if (need > hda_plan_capacity(B, dyn ? W : B * S)) return fail("capacity bound", it);
    // exact-size buffer: heap allocation of exactly `need` ints, so ASan sees
    // any write past the end
    std::vector<int32_t> plan((size_t)need);
    int64_t got = 0;
    st = dyn ? hda_plan(lens.data(), B, tl, W, plan.data(), need, &got)
             : hda_plan_static(lens.data(), B, S, plan.data(), need, &got);
    if (st != HDA_OK || got != need) return fail("plan", it);
    if (hda_plan_validate(plan.data(), need, lens.data(), B) != HDA_OK) return fail("validate", it);
    if (hda_workspace_bytes(plan.data(), need, 8, 2, 128) <= 0) return fail("workspace", it);
    // one int short
    if (need > 1) {
      std::vector<int32_t> small((size_t)need - 1);
      st = dyn ? hda_plan(lens.data(), B, tl, W, small.data(), need - 1, &got)
               : hda_plan_static(lens.data(), B, S, small.data(), need - 1, &got);
      if (st != HDA_ERR_CAPACITY) return fail("short buffer", it);
    }
    // random corruption: the validator must answer with a status, never crash
    for (int c = 0; c < 4; ++c) {
      std::vector<int32_t> bad = plan;
      const size_t k = rng() % bad.size();
      bad[k] = (int32_t)(rng() % 7 == 0 ? rng() : (int64_t)bad[k] + (int64_t)(rng() % 5) - 2);
      st = hda_plan_validate(bad.data(), (int64_t)bad.size(), lens.data(), B);
      if (st != HDA_OK && st != HDA_ERR_BAD_PLAN && st != HDA_ERR_PLAN_MISMATCH &&
          st != HDA_ERR_INVALID_ARG)
        return fail("validate status", it);
      (void)hda_workspace_bytes(bad.data(), (int64_t)bad.size(), 8, 2, 128);
    }
    // truncated plan
    st = hda_plan_validate(plan.data(), need - 1 - (int64_t)(rng() % need), lens.data(), B);
    if (st == HDA_OK) return fail("truncated accepted", it);
  }
  // prefill row blocks: exact-size buffers, then one row short
  for (int it = 0; it < iters / 4; ++it) {
    const int B = 1 + (int)(rng() % 60);
    std::vector<int32_t> kv(B), ql(B);
    for (int b = 0; b < B; ++b) {
      kv[b] = 1 + (int32_t)(rng() % (rng() % 2 ? 100 : 100000));
      ql[b] = 1 + (int32_t)(rng() % kv[b]);
    }
    const int32_t qb = 1 + (int32_t)(rng() % 16);
    int64_t n = 0;
    if (hda_prefill_rows(ql.data(), kv.data(), B, qb, nullptr, nullptr, 0, &n) != HDA_ERR_CAPACITY)
      return fail("prefill size query", it);
    std::vector<int32_t> rows((size_t)n * 4), lens((size_t)n);
    if (hda_prefill_rows(ql.data(), kv.data(), B, qb, rows.data(), lens.data(), n, &n) != HDA_OK)
      return fail("prefill rows", it);
    std::vector<int32_t> plan(1 << 16);
    int64_t got = 0;
    const int st = hda_plan(lens.data(), (int32_t)n, 1 + (int32_t)(rng() % 300),
                            1 + (int32_t)(rng() % 300), plan.data(), (int64_t)plan.size(), &got);
    if (st == HDA_OK && hda_plan_validate(plan.data(), got, lens.data(), (int32_t)n) != HDA_OK)
      return fail("prefill plan validate", it);
    if (n > 1) {
      std::vector<int32_t> r2((size_t)(n - 1) * 4), l2((size_t)(n - 1));
      if (hda_prefill_rows(ql.data(), kv.data(), B, qb, r2.data(), l2.data(), n - 1, &n) !=
          HDA_ERR_CAPACITY)
        return fail("prefill short buffer", it);
    }
  }
  printf("plan_fuzz: %d iterations clean\n", iters);
  return 0;
}
