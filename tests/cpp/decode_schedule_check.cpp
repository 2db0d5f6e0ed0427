// CPU check of the decode schedule (host code only): for random batches,
// window widths, GQA groups and forms, every request's visible key range is
// covered by its items exactly once, items stay inside their request, cut
// pieces start on 64-key boundaries and own consecutive partial slots, whole
// requests are written directly only by the decode kernel, and the split
// form's work-groups stream equal shares.  Prints "ok <cases>" or the first
// failing case.
#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

#include "psw_host.hpp"

void psw_mirror_free(psw_device_mirror*, psw_stream_t) {}  // the device mirror is not linked here

using namespace psw;

static int check_case(const PlanState& st, int64_t wl, int32_t mode, const DecodeSchedule& ds) {
  const bool dk = st.group <= kDecodeKernelMaxGroup;
  const int n_items = static_cast<int>(ds.items.size() / 4);
  std::vector<std::vector<std::pair<int64_t, int64_t>>> cover(st.batch);
  std::vector<int> pieces(st.batch, 0);
  if (static_cast<int>(ds.wg_items.size()) != (dk ? ds.num_wgs + 1 : int(ds.wg_items.size())))
    return 1;
  for (int i = 0; i < n_items; ++i) {
    const int b = ds.items[4 * i], sl = ds.items[4 * i + 1];
    const int64_t k0 = ds.items[4 * i + 2], k1 = ds.items[4 * i + 3];
    if (b < 0 || b >= st.batch || k0 > k1) return 2;
    const int64_t p = st.kv_len[b] - 1, lo = wl >= 0 ? std::max<int64_t>(0, p - wl) : 0;
    if (k0 < lo || k1 > p) return 3;
    if (sl >= ds.num_partials) return 4;
    if (sl < 0 && (!dk || k0 != lo || k1 != p)) return 5;
    if (sl >= 0) {
      const int f = ds.req_splits[2 * b], c = ds.req_splits[2 * b + 1];
      if (sl < f || sl >= f + c) return 6;
      ++pieces[b];
      if (k0 != lo && k0 % kDecodeSplitUnit) return 7;
    }
    cover[b].push_back({k0, k1});
  }
  for (int b = 0; b < st.batch; ++b) {
    const int64_t p = st.kv_len[b] - 1, lo = wl >= 0 ? std::max<int64_t>(0, p - wl) : 0;
    std::sort(cover[b].begin(), cover[b].end());
    int64_t next = lo;
    for (const auto& r : cover[b]) {
      if (r.first != next) return 8;
      next = r.second + 1;
    }
    if (next != p + 1) return 9;
    if (pieces[b] != ds.req_splits[2 * b + 1]) return 10;
  }
  if (ds.direct != (ds.num_partials == 0)) return 11;
  if (dk) {
    if (ds.wg_items.front() != 0 || ds.wg_items.back() != n_items) return 12;
    for (int g = 0; g < ds.num_wgs; ++g)
      if (ds.wg_items[g] >= ds.wg_items[g + 1]) return 13;  // every work-group has an item
    if (!ds.direct || mode == PSW_DECODE_SPLIT) {
      // split form: at most kDecodeResidentWaves' worth of work-groups,
      // shares within one unit
      if (int64_t(ds.num_wgs) * (st.head_dim / 128) * st.num_kv_heads >
          std::max<int64_t>(kDecodeResidentWaves, (st.head_dim / 128) * st.num_kv_heads))
        return 14;
      int64_t mn = INT64_MAX, mx = 0;
      for (int g = 0; g < ds.num_wgs; ++g) {
        int64_t units = 0;
        for (int i = ds.wg_items[g]; i < ds.wg_items[g + 1]; ++i) {
          const int64_t k0 = ds.items[4 * i + 2], k1 = ds.items[4 * i + 3];
          units += k1 / kDecodeSplitUnit - k0 / kDecodeSplitUnit + 1;
        }
        mn = std::min(mn, units);
        mx = std::max(mx, units);
      }
      if (ds.num_wgs > 0 && mx - mn > 1) return 15;
    }
  }
  return 0;
}

int main() {
  std::mt19937 rng(1);
  const int groups[] = {1, 2, 4, 8, 16, 32};
  int cases = 0;
  for (int it = 0; it < 3000; ++it) {
    PlanState st{};
    st.head_dim = (rng() & 1) ? 256 : 512;
    st.num_kv_heads = st.head_dim == 256 && (rng() & 1) ? 8 : 1;
    st.group = groups[rng() % 6];
    st.num_qo_heads = st.num_kv_heads * st.group;
    st.batch = 1 + rng() % (rng() % 3 == 0 ? 300 : 20);
    st.kv_len.resize(st.batch);
    for (auto& k : st.kv_len) k = 1 + rng() % ((rng() % 4 == 0) ? 40000 : 3000);
    const int64_t wl = (rng() % 3 == 0) ? -1 : int64_t(rng() % 2000);
    const int32_t mode = rng() % 3;
    DecodeSchedule ds;
    build_decode_schedule(st, wl, effective_decode_mode(st, mode), &ds);
    const int rc = check_case(st, wl, effective_decode_mode(st, mode), ds);
    ++cases;
    if (rc) {
      std::printf("fail %d: head_dim %d kv heads %d group %d batch %d window %lld mode %d\n", rc,
                  int(st.head_dim), int(st.num_kv_heads), int(st.group), int(st.batch),
                  (long long)wl, int(mode));
      return 1;
    }
  }
  std::printf("ok %d\n", cases);
  return 0;
}
