// Host planner, plan validator and workspace sizing for libhda.
//
// Pure host C++ (no HIP headers): it builds into libhda.so and, on its own,
// into a sanitizer-instrumented test driver.
//
// The tile plan follows the planner the pages describe (page "Tencent HPC
// llega a SGLang y desafía a los kernels de inferencia predeterminados",
// section "Por qué Tencent HPC importa para el serving de modelos en línea":
// uniform tiles, assigned to thread blocks by the current workload and
// rebuilt as request lengths change; arex-research page, Dynamic Attention
// paragraphs: tiles allocated per decode step by the actual KV length).  The
// pages do not say how tiles map to blocks; this planner takes a contiguous
// balanced split of the request-major tile sequence, so each workgroup's
// share differs from any other's by at most one tile and consecutive tiles of
// one request collapse into a single work item.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "hda.h"

namespace {

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Tile-to-workgroup arithmetic of the balanced contiguous split: T tiles over
// W workgroups, the first r = T mod W taking q + 1 = T / W + 1 tiles.
struct Split {
  int64_t q, r;
  int64_t first_tile(int64_t w) const { return w * q + std::min<int64_t>(w, r); }
  int64_t owner(int64_t t) const {
    const int64_t big = r * (q + 1);
    return t < big ? t / (q + 1) : r + (t - big) / q;
  }
};

inline int64_t tiles_of(int32_t len, int32_t tile_len) {
  return ((int64_t)len + tile_len - 1) / tile_len;
}

int check_lens(const int32_t* seq_lens, int32_t batch) {
  if (!seq_lens || batch < 1) return HDA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < batch; ++b)
    if (seq_lens[b] < 1) return HDA_ERR_INVALID_ARG;
  return HDA_OK;
}

inline int64_t plan_len_for(int64_t W, int64_t N, int64_t B) {
  return HDA_PLAN_HEADER_INTS + (W + 1) + 4 * N + (B + 1);
}

}  // namespace

extern "C" {

int64_t hda_plan_capacity(int32_t batch, int32_t n_workgroups) {
  if (batch < 1 || n_workgroups < 1) return -1;
  return plan_len_for(n_workgroups, (int64_t)n_workgroups + batch - 1, batch);
}

int hda_plan(const int32_t* seq_lens, int32_t batch, int32_t tile_len,
             int32_t n_workgroups, int32_t* plan, int64_t capacity,
             int64_t* plan_len) {
  if (!plan_len || tile_len < 1 || n_workgroups < 1) return HDA_ERR_INVALID_ARG;
  int st = check_lens(seq_lens, batch);
  if (st != HDA_OK) return st;
  if ((int64_t)n_workgroups + batch > kI32Max) return HDA_ERR_INVALID_ARG;
  const int64_t W = n_workgroups, B = batch;

  int64_t T = 0;
  for (int64_t b = 0; b < B; ++b) T += tiles_of(seq_lens[b], tile_len);
  if (T > kI32Max) return HDA_ERR_INVALID_ARG;
  const Split sp{T / W, T % W};

  // Items per request: the number of workgroups its tile range touches.
  auto items_of = [&](int64_t first, int64_t n) {
    return sp.owner(first + n - 1) - sp.owner(first) + 1;
  };
  int64_t N = 0, P = 0;
  {
    int64_t first = 0;
    for (int64_t b = 0; b < B; ++b) {
      const int64_t n = tiles_of(seq_lens[b], tile_len);
      const int64_t k = items_of(first, n);
      N += k;
      if (k > 1) P += k;
      first += n;
    }
  }
  const int64_t need = plan_len_for(W, N, B);
  *plan_len = need;
  if (capacity < need) return HDA_ERR_CAPACITY;
  if (!plan) return HDA_ERR_INVALID_ARG;

  int32_t* hdr = plan;
  int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  int32_t* items = wg_ptr + (W + 1);
  int32_t* rpp = items + 4 * N;
  hdr[0] = HDA_PLAN_VERSION;
  hdr[1] = (int32_t)B;
  hdr[2] = tile_len;
  hdr[3] = (int32_t)W;
  hdr[4] = (int32_t)T;
  hdr[5] = (int32_t)N;
  hdr[6] = (int32_t)P;
  hdr[7] = 0;

  // Walk the workgroups; a request cursor (b, its first tile) advances
  // through the request-major tile sequence.
  int64_t n_items = 0, next_slot = 0;
  int64_t b = 0, b_first = 0, b_tiles = tiles_of(seq_lens[0], tile_len);
  for (int64_t w = 0; w < W; ++w) {
    wg_ptr[w] = (int32_t)n_items;
    int64_t t0 = sp.first_tile(w);
    const int64_t t1 = sp.first_tile(w + 1);
    while (t0 < t1) {
      while (t0 >= b_first + b_tiles) {  // move to the request holding t0
        b_first += b_tiles;
        ++b;
        b_tiles = tiles_of(seq_lens[b], tile_len);
      }
      const int64_t hi = std::min(t1, b_first + b_tiles);
      const int64_t k0 = (t0 - b_first) * tile_len;
      const int64_t k1 = std::min<int64_t>((hi - b_first) * tile_len, seq_lens[b]);
      const bool split = items_of(b_first, b_tiles) > 1;
      int32_t* it = items + 4 * n_items;
      it[0] = (int32_t)b;
      it[1] = (int32_t)k0;
      it[2] = (int32_t)k1;
      it[3] = split ? (int32_t)next_slot++ : -1;
      ++n_items;
      t0 = hi;
    }
  }
  wg_ptr[W] = (int32_t)n_items;

  rpp[0] = 0;
  {
    int64_t first = 0;
    for (int64_t r = 0; r < B; ++r) {
      const int64_t n = tiles_of(seq_lens[r], tile_len);
      const int64_t k = items_of(first, n);
      rpp[r + 1] = rpp[r] + (int32_t)(k > 1 ? k : 0);
      first += n;
    }
  }
  return HDA_OK;
}

int hda_plan_static(const int32_t* seq_lens, int32_t batch, int32_t n_splits,
                    int32_t* plan, int64_t capacity, int64_t* plan_len) {
  if (!plan_len || n_splits < 1) return HDA_ERR_INVALID_ARG;
  int st = check_lens(seq_lens, batch);
  if (st != HDA_OK) return st;
  const int64_t B = batch, S = n_splits, W = B * S;
  if (W + B > kI32Max) return HDA_ERR_INVALID_ARG;
  // chunk c of a request of length L is empty iff floor(cL/S) == floor((c+1)L/S);
  // exactly min(L, S) chunks are non-empty.
  int64_t N = 0, P = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t k = std::min<int64_t>(seq_lens[b], S);
    N += k;
    if (k > 1) P += k;
  }
  const int64_t need = plan_len_for(W, N, B);
  *plan_len = need;
  if (capacity < need) return HDA_ERR_CAPACITY;
  if (!plan) return HDA_ERR_INVALID_ARG;

  int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  int32_t* items = wg_ptr + (W + 1);
  int32_t* rpp = items + 4 * N;
  plan[0] = HDA_PLAN_VERSION;
  plan[1] = (int32_t)B;
  plan[2] = 0;
  plan[3] = (int32_t)W;
  plan[4] = (int32_t)N;
  plan[5] = (int32_t)N;
  plan[6] = (int32_t)P;
  plan[7] = 0;
  int64_t n_items = 0, next_slot = 0;
  rpp[0] = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t L = seq_lens[b];
    const bool split = std::min<int64_t>(L, S) > 1;
    for (int64_t c = 0; c < S; ++c) {
      wg_ptr[b * S + c] = (int32_t)n_items;
      const int64_t k0 = c * L / S, k1 = (c + 1) * L / S;
      if (k1 == k0) continue;
      int32_t* it = items + 4 * n_items++;
      it[0] = (int32_t)b;
      it[1] = (int32_t)k0;
      it[2] = (int32_t)k1;
      it[3] = split ? (int32_t)next_slot++ : -1;
    }
    rpp[b + 1] = (int32_t)next_slot;
  }
  wg_ptr[W] = (int32_t)n_items;
  return HDA_OK;
}

int hda_plan_validate(const int32_t* plan, int64_t plan_len,
                      const int32_t* seq_lens, int32_t batch) {
  if (!plan || plan_len < HDA_PLAN_HEADER_INTS) return HDA_ERR_INVALID_ARG;
  int st = check_lens(seq_lens, batch);
  if (st != HDA_OK) return st;
  if (plan[0] != HDA_PLAN_VERSION) return HDA_ERR_BAD_PLAN;
  if (plan[1] != batch) return HDA_ERR_PLAN_MISMATCH;
  const int64_t B = plan[1], tile_len = plan[2], W = plan[3], T = plan[4],
                N = plan[5], P = plan[6];
  if (tile_len < 0 || W < 1 || T < 0 || N < B || P < 0 || plan[7] != 0)
    return HDA_ERR_BAD_PLAN;
  if (plan_len != plan_len_for(W, N, B)) return HDA_ERR_BAD_PLAN;
  const int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  const int32_t* items = wg_ptr + (W + 1);
  const int32_t* rpp = items + 4 * N;
  if (wg_ptr[0] != 0 || wg_ptr[W] != N) return HDA_ERR_BAD_PLAN;
  for (int64_t w = 0; w < W; ++w)
    if (wg_ptr[w + 1] < wg_ptr[w]) return HDA_ERR_BAD_PLAN;

  // Items of each request must tile [0, len_b) in token order; the lengths
  // they cover decide whether the plan matches these seq_lens.
  std::vector<int64_t> next(B, 0), count(B, 0);
  bool mismatch = false;
  for (int64_t i = 0; i < N; ++i) {
    const int32_t* it = items + 4 * i;
    const int64_t b = it[0], k0 = it[1], k1 = it[2];
    if (b < 0 || b >= B || k0 < 0 || k1 <= k0) return HDA_ERR_BAD_PLAN;
    if (k0 != next[b]) return HDA_ERR_BAD_PLAN;
    if (k1 > seq_lens[b]) mismatch = true;
    next[b] = k1;
    ++count[b];
  }
  for (int64_t b = 0; b < B; ++b)
    if (next[b] != seq_lens[b]) mismatch = true;
  if (mismatch) return HDA_ERR_PLAN_MISMATCH;

  // Slots: -1 for single-item requests, else numbered in item order and
  // matching req_part_ptr.
  if (rpp[0] != 0) return HDA_ERR_BAD_PLAN;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t want = count[b] > 1 ? count[b] : 0;
    if ((int64_t)rpp[b + 1] - rpp[b] != want) return HDA_ERR_BAD_PLAN;
  }
  if (rpp[B] != P) return HDA_ERR_BAD_PLAN;
  std::vector<int64_t> seen(B, 0);
  int64_t expect_slot = 0;
  for (int64_t i = 0; i < N; ++i) {
    const int32_t* it = items + 4 * i;
    const int64_t b = it[0];
    if (count[b] == 1) {
      if (it[3] != -1) return HDA_ERR_BAD_PLAN;
    } else {
      if (it[3] != expect_slot || it[3] != rpp[b] + seen[b]) return HDA_ERR_BAD_PLAN;
      ++expect_slot;
      ++seen[b];
    }
  }
  if (tile_len > 0) {  // dynamic plan: the tile count must match the lengths
    int64_t t = 0;
    for (int64_t b = 0; b < B; ++b) t += tiles_of(seq_lens[b], (int32_t)tile_len);
    if (t != T) return HDA_ERR_PLAN_MISMATCH;
  }
  return HDA_OK;
}

// Launch width for a step.  The tile kernel streams K/V, so a step lasts
// about as long as its busiest compute unit: with W x Hkv workgroups spread
// over n_cu units (at most wg_per_cu each), that unit holds
// ceil(W Hkv / n_cu) workgroups of ceil(T / W) tiles.  A width between one
// and two workgroups per unit leaves some units with two and the others
// with one, and the step waits for the doubly loaded ones (measured: 1 x
// 131072 + 31 x 4096 tokens in tiles of 128 over 8 kv heads takes 161 us at
// W = 32 or 63, 220 us at W = 40).  So: the widths with the fewest tiles on
// the busiest unit, within 1/32 of the least; among them the fewest partial
// slots (each costs a write by the tile kernel and a read by the merge, and
// P = 0 skips the merge); then the widest.  Extreme mix: 63 (one split
// request); 32 x 4096 tokens: 32 (one request per workgroup, no merge).
int hda_launch_config(const int32_t* seq_lens, int32_t batch, int32_t n_kv_heads, int32_t n_cu,
                      int32_t wg_per_cu, int32_t tile_len, int32_t* n_workgroups) {
  if (!n_workgroups || n_kv_heads < 1 || n_cu < 1 || wg_per_cu < 1 || tile_len < 1)
    return HDA_ERR_INVALID_ARG;
  int st = check_lens(seq_lens, batch);
  if (st != HDA_OK) return st;
  int64_t T = 0;
  for (int32_t b = 0; b < batch; ++b) T += tiles_of(seq_lens[b], tile_len);
  if (T > kI32Max) return HDA_ERR_INVALID_ARG;
  const int64_t w_max =
      std::max<int64_t>(1, std::min<int64_t>(T, (int64_t)n_cu * wg_per_cu / n_kv_heads));
  auto unit_tiles = [&](int64_t W) {
    return ((W * n_kv_heads + n_cu - 1) / n_cu) * ((T + W - 1) / W);
  };
  int64_t least = unit_tiles(w_max);
  for (int64_t W = w_max - 1; W >= 1; --W) least = std::min(least, unit_tiles(W));
  int64_t best_w = -1, best_p = -1;
  for (int64_t W = w_max; W >= 1; --W) {
    if (unit_tiles(W) * 32 > least * 33) continue;
    const Split sp{T / W, T % W};
    int64_t P = 0, first = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = tiles_of(seq_lens[b], tile_len);
      const int64_t k = sp.owner(first + n - 1) - sp.owner(first) + 1;
      if (k > 1) P += k;
      first += n;
    }
    if (best_p < 0 || P < best_p) {
      best_p = P;
      best_w = W;
    }
  }
  *n_workgroups = (int32_t)best_w;
  return HDA_OK;
}

int64_t hda_workspace_bytes(const int32_t* plan, int64_t plan_len,
                            int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim) {
  if (!plan || plan_len < HDA_PLAN_HEADER_INTS || n_q_heads < 1 ||
      n_kv_heads < 1 || head_dim < 1)
    return -1;
  if (plan[0] != HDA_PLAN_VERSION || plan[1] < 1 || plan[3] < 1 || plan[6] < 0) return -1;
  const int64_t B = plan[1], W = plan[3], P = plan[6];
  return round_up(W * n_kv_heads * 4, 256) + round_up(P * n_q_heads * head_dim * 4, 256) +
         round_up(P * n_q_heads * 4, 256) + round_up(B * n_q_heads * head_dim * 2, 256) +
         round_up(B * 8, 256);
}

int32_t hda_prefill_rows_per_block(int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads) return -1;
  const int32_t g = n_q_heads / n_kv_heads;
  return g <= 16 ? 16 / g : -1;
}

// Block size for a batch: tiles of 16/g rows, as many as the mean query run
// fills, rounded up to a power of two (1, 2, 4, 8 or 16 tiles; the kernel
// shapes).  A longer block lets more query rows share each K/V load; one
// longer than most requests' runs leaves tiles idle.
int32_t hda_prefill_block_rows(const int32_t* q_lens, int32_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads) {
  const int32_t unit = hda_prefill_rows_per_block(n_q_heads, n_kv_heads);
  if (!q_lens || batch < 1 || unit < 1) return -1;
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (q_lens[b] < 1) return -1;
    total += q_lens[b];
  }
  const int64_t per_tile = (int64_t)unit * batch;              // mean / unit, rounded up
  const int64_t need = (total + per_tile - 1) / per_tile;
  int32_t tiles = 1;
  while (tiles < HDA_PREFILL_MAX_TILES && tiles < need) tiles *= 2;
  return tiles * unit;
}

// Row blocks of a multi-token batch: the query rows of each request, in
// order, grouped into blocks of rows_per_block (the last shorter).  Row r of
// request b sits at position kv_len - q_len + r; a block needs cache tokens
// [0, position of its last row + 1), its length for hda_plan.
int hda_prefill_rows(const int32_t* q_lens, const int32_t* kv_lens, int32_t batch,
                     int32_t rows_per_block, int32_t* rows, int32_t* row_lens,
                     int64_t capacity, int64_t* n_rows) {
  if (!q_lens || !kv_lens || !n_rows || batch < 1 || rows_per_block < 1)
    return HDA_ERR_INVALID_ARG;
  int64_t R = 0, total_q = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (q_lens[b] < 1 || kv_lens[b] < 1 || q_lens[b] > kv_lens[b]) return HDA_ERR_INVALID_ARG;
    R += ((int64_t)q_lens[b] + rows_per_block - 1) / rows_per_block;
    total_q += q_lens[b];
  }
  if (R > kI32Max || total_q > kI32Max) return HDA_ERR_INVALID_ARG;
  *n_rows = R;
  if (!rows || !row_lens || capacity < R) return HDA_ERR_CAPACITY;
  int64_t k = 0, q_start = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = q_lens[b], ctx = kv_lens[b] - q_lens[b];
    for (int32_t q0 = 0; q0 < n; q0 += rows_per_block, ++k) {
      const int32_t nq = std::min(rows_per_block, n - q0);
      rows[4 * k] = b;
      rows[4 * k + 1] = (int32_t)(q_start + q0);
      rows[4 * k + 2] = nq;
      rows[4 * k + 3] = ctx + q0;
      row_lens[k] = ctx + q0 + nq;
    }
    q_start += n;
  }
  return HDA_OK;
}

int64_t hda_prefill_workspace_bytes(const int32_t* plan, int64_t plan_len, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim,
                                    int32_t rows_per_block) {
  if (!plan || plan_len < HDA_PLAN_HEADER_INTS || n_q_heads < 1 || n_kv_heads < 1 ||
      head_dim < 1)
    return -1;
  const int32_t unit = hda_prefill_rows_per_block(n_q_heads, n_kv_heads);
  const int32_t qb = rows_per_block;
  if (unit < 1 || qb < 1 || qb > HDA_PREFILL_MAX_TILES * unit || plan[0] != HDA_PLAN_VERSION || plan[1] < 1 ||
      plan[3] < 1 || plan[6] < 0)
    return -1;
  const int64_t W = plan[3], P = plan[6];
  return round_up(W * n_kv_heads * 4, 256) + round_up(P * qb * n_q_heads * head_dim * 4, 256) +
         round_up(P * qb * n_q_heads * 4, 256);
}

const char* hda_status_string(int status) {
  switch (status) {
    case HDA_OK: return "ok";
    case HDA_ERR_INVALID_ARG: return "invalid argument";
    case HDA_ERR_CAPACITY: return "plan buffer too small";
    case HDA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HDA_ERR_PLAN_MISMATCH: return "plan does not match batch or lengths";
    case HDA_ERR_HIP: return "HIP runtime error";
    case HDA_ERR_WORKSPACE: return "workspace missing or too small";
    case HDA_ERR_BAD_PLAN: return "malformed plan";
    default: return "unknown status";
  }
}

int hda_version(void) { return HDA_VERSION; }

int64_t hda_params_bytes(void) { return (int64_t)sizeof(hda_params); }

}  // extern "C"
