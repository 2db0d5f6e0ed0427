// CPU check of the prefill schedule (host code only).  For random batches
// (query counts up to kv_len, so chunked prefills too), windows, GQA groups
// and both head dims:
//   * each item's first query token is a multiple of the plan's tile_q
//     inside its request, and the items of a request cover every one of its
//     query tiles exactly once;
//   * each item's key range is exactly what its tokens may see: from the
//     window start of its first token (0 without a window) to the position
//     of its last token, so every token's visible keys lie inside it;
//   * items are sorted by KV tiles visited, heaviest first, and total_tiles
//     is their sum;
//   * check_prefill_items accepts the schedule and rejects planted mistakes.
// Prints "ok <cases>" or the first failing case.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "psw_host.hpp"

void psw_mirror_free(psw_device_mirror*, psw_stream_t) {}  // the device mirror is not linked here

using namespace psw;

static int64_t window_lo(int64_t pos, int64_t wl) { return wl >= 0 ? std::max<int64_t>(0, pos - wl) : 0; }

static int check_case(const PlanState& st, int64_t wl, int kv_tile, const PrefillSchedule& ps) {
  if (ps.items.size() % 4) return 1;
  const int n = static_cast<int>(ps.items.size() / 4);
  std::vector<std::vector<int32_t>> starts(st.batch);
  int64_t total = 0, prev_cost = INT64_MAX;
  for (int i = 0; i < n; ++i) {
    const int32_t b = ps.items[4 * i], t0 = ps.items[4 * i + 1];
    const int64_t k0 = ps.items[4 * i + 2], k1 = ps.items[4 * i + 3];
    if (b < 0 || b >= st.batch) return 2;
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int64_t start = int64_t(st.kv_len[b]) - qo;
    if (t0 < 0 || t0 >= qo || t0 % st.tile_q) return 3;
    const int32_t t1 = std::min(t0 + st.tile_q, qo) - 1;  // last token of the item
    if (k0 != window_lo(start + t0, wl) || k1 != start + t1) return 4;
    for (int32_t t : {t0, t1, (t0 + t1) / 2}) {
      const int64_t pos = start + t;
      if (window_lo(pos, wl) < k0 || pos > k1) return 5;
    }
    const int64_t cost = k1 / kv_tile - k0 / kv_tile + 1;
    if (cost > prev_cost) return 6;
    prev_cost = cost;
    total += cost;
    starts[b].push_back(t0);
  }
  for (int32_t b = 0; b < st.batch; ++b) {
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    std::sort(starts[b].begin(), starts[b].end());
    if (int64_t(starts[b].size()) != (qo + st.tile_q - 1) / st.tile_q) return 7;
    for (size_t k = 0; k < starts[b].size(); ++k)
      if (starts[b][k] != int32_t(k) * st.tile_q) return 7;
  }
  if (total != ps.total_tiles) return 8;
  return 0;
}

int main() {
  std::mt19937 rng(3);
  const int groups[] = {1, 2, 4, 8, 16, 32};
  int cases = 0;
  for (int it = 0; it < 3000; ++it) {
    PlanState st{};
    st.head_dim = (rng() & 1) ? 256 : 512;
    st.num_kv_heads = st.head_dim == 256 ? 8 : 1;
    st.group = groups[rng() % 6];
    st.num_qo_heads = st.num_kv_heads * st.group;
    if (derive_tile_q(st.group, st.head_dim, &st.tile_q) != PSW_OK) {
      std::printf("fail: no tile for group %d head_dim %d\n", int(st.group), int(st.head_dim));
      return 1;
    }
    st.batch = 1 + rng() % (rng() % 4 == 0 ? 100 : 12);
    st.qo_indptr.assign(1, 0);
    st.kv_len.resize(st.batch);
    for (int32_t b = 0; b < st.batch; ++b) {
      const int32_t kv = 1 + rng() % ((rng() % 4 == 0) ? 9000 : 1500);
      const int32_t qo = rng() % 3 == 0 ? kv : 1 + int32_t(rng() % kv);
      st.kv_len[b] = kv;
      st.qo_indptr.push_back(st.qo_indptr.back() + qo);
      st.max_kv_len = std::max(st.max_kv_len, kv);
      st.max_qo_len = std::max(st.max_qo_len, qo);
    }
    st.total_qo = st.qo_indptr.back();
    const int64_t wl_in = (rng() % 3 == 0) ? -1 : int64_t(rng() % 3000);
    const int64_t wl = effective_window(st, wl_in);
    const int kv_tile = kv_tile_for(st.head_dim);
    PrefillSchedule ps;
    build_prefill_schedule(st, wl, kv_tile, &ps);
    ++cases;
    const int rc = check_case(st, wl, kv_tile, ps);
    if (rc) {
      std::printf("fail %d: head_dim %d group %d batch %d window %lld\n", rc, int(st.head_dim),
                  int(st.group), int(st.batch), (long long)wl_in);
      return 1;
    }
    if (check_prefill_items(st, ps) != PSW_OK) {
      std::printf("fail: check_prefill_items rejected a built schedule: %s\n", psw_last_error());
      return 1;
    }
    // planted mistakes: each one alone must be rejected
    const size_t k = 4 * (rng() % (ps.items.size() / 4));
    const int32_t b = ps.items[k];
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    std::vector<std::pair<size_t, int32_t>> plants = {
        {k, st.batch},                 // request out of range
        {k + 1, qo},                   // first token past the request
        {k + 3, st.kv_len[b]},         // last key past kv_len
        {k + 2, ps.items[k + 3] + 1},  // first key after the last
    };
    if (st.tile_q > 1 && ps.items[k + 1] + 1 < qo) plants.push_back({k + 1, ps.items[k + 1] + 1});
    for (const auto& pl : plants) {
      PrefillSchedule bad = ps;
      bad.items[pl.first] = pl.second;
      if (check_prefill_items(st, bad) == PSW_OK) {
        std::printf("fail: a planted mistake at field %zu passed the check\n", pl.first % 4);
        return 1;
      }
    }
  }
  std::printf("ok %d\n", cases);
  return 0;
}
