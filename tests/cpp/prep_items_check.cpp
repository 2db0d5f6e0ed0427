// CPU check of the prep work items (host code only).  For random plans --
// batches of requests at random start positions, page sizes 8..64, resident
// windows whose pages wrap as a ring -- that the prep entries' host checks
// accept, every item built by build_prep_items must
//   * hold 1..16 tokens, all inside one page (first slot + tokens <= page size,
//     first slot = position mod page size),
//   * take its page id from its own request's table, the page that holds its
//     position (ring or not), and no page outside the pool,
//   * stay below kv_len (hence inside the RoPE table the entry checked) and at
//     or after the request's first new token,
//   * name the token of its position in the query rows;
// the items of a request cover its new tokens exactly once, no (page, slot)
// is written twice in the call, and check_prep_items accepts the items.
// Items that break a rule (planted here, on the host) are rejected.
// Prints "ok <cases>" or the first failing case.
#include <algorithm>
#include <cstdio>
#include <random>
#include <set>
#include <vector>

#include "psw_host.hpp"

void psw_mirror_free(psw_device_mirror*, psw_stream_t) {}  // the device mirror is not linked here

using namespace psw;

static int check_case(const PlanState& st, const std::vector<int32_t>& it) {
  if (it.size() % 6) return 1;
  std::vector<std::vector<int>> seen(st.batch);
  std::set<std::pair<int, int>> written;
  for (size_t i = 0; i < it.size() / 6; ++i) {
    const int b = it[6 * i], tok0 = it[6 * i + 1], n = it[6 * i + 2];
    const int page = it[6 * i + 3], slot = it[6 * i + 4], pos = it[6 * i + 5];
    if (b < 0 || b >= st.batch) return 2;
    if (n < 1 || n > 16) return 3;
    if (slot != pos % st.page_size || slot + n > st.page_size) return 4;
    const int qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int start = st.kv_len[b] - qo;
    if (pos < start || pos + n > st.kv_len[b]) return 5;
    if (tok0 != st.qo_indptr[b] + pos - start) return 6;
    // the page of the position, from the request's own list
    const int np = st.n_pages(b);
    const int own = st.kv_page_indices[st.kv_page_indptr[b] + (pos / st.page_size) % np];
    if (page != own || page < 0 || page >= st.num_pages) return 7;
    for (int t = 0; t < n; ++t) {
      seen[b].push_back(pos + t);
      if (!written.insert({page, slot + t}).second) return 8;
    }
  }
  for (int b = 0; b < st.batch; ++b) {
    const int qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int start = st.kv_len[b] - qo;
    std::sort(seen[b].begin(), seen[b].end());
    if (int(seen[b].size()) != qo) return 9;
    for (int t = 0; t < qo; ++t)
      if (seen[b][t] != start + t) return 10;
  }
  return 0;
}

int main() {
  std::mt19937 rng(7);
  int cases = 0, accepted = 0;
  for (int iter = 0; iter < 4000; ++iter) {
    const int P = 8 << (rng() % 4);  // 8, 16, 32, 64
    const int B = 1 + rng() % 12;
    std::vector<int32_t> qo_indptr{0}, kv_indptr{0}, last, kv_len, ids;
    int next_page = 0;
    for (int b = 0; b < B; ++b) {
      const int qo = 1 + rng() % (rng() % 4 == 0 ? 600 : 40);
      const int start = rng() % 3 == 0 ? 0 : int(rng() % 3000);
      const int kv = start + qo;
      int need = (kv + P - 1) / P;
      if (rng() % 3 == 0) {
        // resident window: a ring that still holds the new tokens
        const int ring = std::min(need, (qo + P - 1) / P + 1 + int(rng() % 8));
        need = ring;
      }
      qo_indptr.push_back(qo_indptr.back() + qo);
      kv_indptr.push_back(kv_indptr.back() + need);
      last.push_back((kv - 1) % P + 1);
      kv_len.push_back(kv);
      for (int i = 0; i < need; ++i) ids.push_back(next_page++);
    }
    const int num_pages = next_page + int(rng() % 5);
    // a random permutation of the pool's pages for the tables
    std::vector<int32_t> perm(num_pages);
    for (int i = 0; i < num_pages; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    for (auto& id : ids) id = perm[id];
    psw_plan_desc d{};
    d.batch = B;
    d.qo_indptr = qo_indptr.data();
    d.kv_page_indptr = kv_indptr.data();
    d.kv_page_indices = ids.data();
    d.kv_last_page_len = last.data();
    d.kv_len = kv_len.data();
    d.num_qo_heads = 16;
    d.num_kv_heads = 8;
    d.head_dim = 256;
    d.page_size = P;
    d.num_pages = num_pages;
    PlanState st;
    if (build_state(&d, &st) != PSW_OK) {
      std::printf("fail: build_state rejected a valid plan: %s\n", psw_last_error());
      return 1;
    }
    ++cases;
    psw_plan plan;
    plan.st = st;
    psw_pool pool{};
    pool.base = reinterpret_cast<void*>(0x1000);
    pool.num_layers = 1;
    pool.num_pages = num_pages;
    pool.page_size = P;
    pool.num_kv_heads = 8;
    pool.head_dim = 256;
    pool.numel = int64_t(num_pages) * 2 * 8 * P * 256;
    const float tab = 0.0f;
    const int64_t rope = st.max_kv_len + int(rng() % 3);
    // the entry's own checks first: only plans they accept reach the items
    if (check_prep_call(&plan, &pool, 0, 256, &tab, &tab, rope, rope * 128, rope * 128, 1e-6f,
                        nullptr) != PSW_OK)
      continue;
    ++accepted;
    std::vector<int32_t> items;
    build_prep_items(st, &items);
    const int rc = check_case(st, items);
    if (rc) {
      std::printf("fail %d: iteration %d, page size %d, batch %d\n", rc, iter, P, B);
      return 1;
    }
    if (check_prep_items(st, items) != PSW_OK) {
      std::printf("fail: check_prep_items rejected built items: %s\n", psw_last_error());
      return 1;
    }
    // planted mistakes are rejected
    const size_t k = 6 * (rng() % (items.size() / 6));
    const int field = rng() % 5;
    std::vector<int32_t> bad = items;
    switch (field) {
      case 0: bad[k + 3] = (bad[k + 3] + 1) % num_pages == bad[k + 3] ? -1 : (bad[k + 3] + 1) % num_pages; break;
      case 1: bad[k + 2] = 17; break;
      case 2: bad[k + 4] = P - bad[k + 2] + 1; break;
      case 3: bad[k + 5] += 1; break;
      default: bad[k + 0] = B; break;
    }
    if (check_prep_items(st, bad) == PSW_OK) {
      std::printf("fail: a planted mistake in field %d was accepted (iteration %d)\n", field, iter);
      return 1;
    }
  }
  if (accepted < cases / 2) {
    std::printf("fail: only %d of %d random plans were accepted\n", accepted, cases);
    return 1;
  }
  std::printf("ok %d\n", accepted);
  return 0;
}
