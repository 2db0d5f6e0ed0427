// Host-side page accounting of the two KV families a two-family model serves
// from: each family has its own page pool, each request its own state in
// both, and a step is admitted for both families or for neither (PR "feat(gemma4): paged KV serving
// across both attention families", Description; its review thread for
// committing the frontier once the step has succeeded).  No HIP API is used
// here; everything runs, and is tested, on the CPU.
//
// Model.  A request has one frontier F (its KV length, the same in both
// families) and holds exactly ceil(F / P_f) pages of family f.  A step of n
// new tokens needs ceil((F + n) / P_f) - held_f more pages of family f.
// Admission checks every precondition first, then reserves the pages of both
// families; if the second reservation is refused, the first is handed back in
// the order it was taken, so both free lists (not only their sizes) are what
// they were.  The reservation stays pending (the caller builds its plans from
// it and runs the step) until commit, which appends the pages and moves the
// frontier, or abort, which returns the pages.  Nothing moves the frontier
// before the step has succeeded.
#include <algorithm>
#include <memory>
#include <string>
#include <unordered_set>
#include <vector>

#include "psw_host.hpp"

namespace {

// Page ids of one pool: a stack of free ids (initially 0..n-1, id 0 handed
// out first).
struct PagePool {
  int64_t page_size = 0;
  std::vector<int32_t> free_ids;

  void init(int64_t n, int64_t p) {
    page_size = p;
    free_ids.resize(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) free_ids[static_cast<size_t>(i)] = static_cast<int32_t>(n - 1 - i);
  }
  // takes k ids or none
  bool take(int64_t k, std::vector<int32_t>* out) {
    if (k > static_cast<int64_t>(free_ids.size())) return false;
    for (int64_t i = 0; i < k; ++i) {
      out->push_back(free_ids.back());
      free_ids.pop_back();
    }
    return true;
  }
  // gives ids back so that the next take returns them in the same order
  void give_back(const std::vector<int32_t>& ids) {
    for (auto it = ids.rbegin(); it != ids.rend(); ++it) free_ids.push_back(*it);
  }
};

}  // namespace

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct psw_kv_server {
  PagePool pool[2];  // PSW_KV_LOCAL, PSW_KV_GLOBAL
  int64_t window_left = -1;
  int64_t rope_positions = 0;
  int64_t ring_pages = 0;  // local family: 0 = no ring
  int64_t live_requests = 0;

  // pages family f holds at frontier F
  int64_t pages_at(int f, int64_t F) const {
    const int64_t full = ceil_div(F, pool[f].page_size);
    return f == PSW_KV_LOCAL && ring_pages > 0 ? std::min(full, ring_pages) : full;
  }
};

struct psw_kv_request {
  const psw_kv_server* owner = nullptr;
  int64_t frontier = 0;
  std::vector<int32_t> held[2];
  bool pending = false;
  int64_t pending_n = 0;
  std::vector<int32_t> reserved[2];
};

namespace {

using psw::fail;

int check_pair(const psw_kv_server* s, const psw_kv_request* r) {
  if (!s) return fail(PSW_E_NULL, "server is NULL");
  if (!r) return fail(PSW_E_NULL, "request is NULL");
  // a page id is meaningful only for the pool it came from
  if (r->owner != s) return fail(PSW_E_PLAN, "request belongs to another server");
  return PSW_OK;
}

int check_family(int32_t family) {
  if (family != PSW_KV_LOCAL && family != PSW_KV_GLOBAL)
    return fail(PSW_E_SHAPE, "family must be PSW_KV_LOCAL (0) or PSW_KV_GLOBAL (1)");
  return PSW_OK;
}

}  // namespace

extern "C" {

int psw_kv_server_create(const psw_kv_server_desc* d, psw_kv_server** out) {
  psw::clear_error();
  if (!d || !out) return fail(PSW_E_NULL, "descriptor or output is NULL");
  *out = nullptr;
  if (d->local_pages < 1 || d->global_pages < 1)
    return fail(PSW_E_SHAPE, "each pool needs at least one page");
  if (d->local_page_size < 1 || d->global_page_size < 1)
    return fail(PSW_E_SHAPE, "page sizes must be >= 1");
  if (!psw::fits_i32(d->local_pages) || !psw::fits_i32(d->global_pages) ||
      !psw::fits_i32(d->local_page_size) || !psw::fits_i32(d->global_page_size) ||
      !psw::fits_i32(d->rope_positions))
    return fail(PSW_E_OVERFLOW, "a pool extent or rope_positions is past INT32_MAX");
  if (d->window_left < -1) return fail(PSW_E_RANGE, "window_left must be >= -1");
  if (d->rope_positions < 1) return fail(PSW_E_SHAPE, "rope_positions must be >= 1");
  if (d->local_ring_pages < 0 || !psw::fits_i32(d->local_ring_pages))
    return fail(PSW_E_RANGE, "local_ring_pages must be in [0, INT32_MAX]");
  if (d->local_ring_pages > 0 && d->window_left < 0)
    return fail(PSW_E_RANGE, "a local ring needs a window (window_left >= 0)");
  auto s = std::make_unique<psw_kv_server>();
  s->pool[PSW_KV_LOCAL].init(d->local_pages, d->local_page_size);
  s->pool[PSW_KV_GLOBAL].init(d->global_pages, d->global_page_size);
  s->window_left = d->window_left;
  s->rope_positions = d->rope_positions;
  s->ring_pages = d->local_ring_pages;
  *out = s.release();
  return PSW_OK;
}

int psw_kv_server_destroy(psw_kv_server* s) {
  psw::clear_error();
  if (!s) return PSW_OK;
  if (s->live_requests != 0)
    return fail(PSW_E_PLAN, std::to_string(s->live_requests) +
                                " request(s) still hold state in this server; release them first");
  delete s;
  return PSW_OK;
}

int psw_kv_server_free_pages(const psw_kv_server* s, int64_t* local_free, int64_t* global_free) {
  psw::clear_error();
  if (!s || !local_free || !global_free) return fail(PSW_E_NULL, "server or output is NULL");
  *local_free = static_cast<int64_t>(s->pool[PSW_KV_LOCAL].free_ids.size());
  *global_free = static_cast<int64_t>(s->pool[PSW_KV_GLOBAL].free_ids.size());
  return PSW_OK;
}

int psw_kv_request_create(psw_kv_server* s, psw_kv_request** out) {
  psw::clear_error();
  if (!s || !out) return fail(PSW_E_NULL, "server or output is NULL");
  auto r = std::make_unique<psw_kv_request>();
  r->owner = s;
  *out = r.release();
  ++s->live_requests;
  return PSW_OK;
}

int psw_kv_request_release(psw_kv_server* s, psw_kv_request* r) {
  psw::clear_error();
  int rc = check_pair(s, r);
  if (rc) return rc;
  for (int f = 0; f < 2; ++f) {
    s->pool[f].give_back(r->reserved[f]);
    s->pool[f].give_back(r->held[f]);
  }
  --s->live_requests;
  delete r;
  return PSW_OK;
}

int psw_kv_request_info(const psw_kv_request* r, psw_kv_request_state* st) {
  psw::clear_error();
  if (!r || !st) return fail(PSW_E_NULL, "request or output is NULL");
  st->frontier = r->frontier;
  st->local_held = static_cast<int64_t>(r->held[PSW_KV_LOCAL].size());
  st->global_held = static_cast<int64_t>(r->held[PSW_KV_GLOBAL].size());
  st->pending = r->pending ? 1 : 0;
  st->pending_tokens = r->pending ? r->pending_n : 0;
  st->local_reserved = static_cast<int64_t>(r->reserved[PSW_KV_LOCAL].size());
  st->global_reserved = static_cast<int64_t>(r->reserved[PSW_KV_GLOBAL].size());
  return PSW_OK;
}

int psw_kv_admit(psw_kv_server* s, psw_kv_request* r, int64_t n_new) {
  psw::clear_error();
  int rc = check_pair(s, r);
  if (rc) return rc;
  // every precondition before any state changes
  if (r->pending) return fail(PSW_E_PLAN, "the request already has a step pending");
  if (n_new < 1) return fail(PSW_E_SHAPE, "a step needs at least one new token");
  const int64_t post = r->frontier + n_new;
  if (!psw::fits_i32(post)) return fail(PSW_E_OVERFLOW, "KV length after the step is past INT32_MAX");
  for (int f = 0; f < 2; ++f) {
    if (static_cast<int64_t>(r->held[f].size()) != s->pages_at(f, r->frontier))
      return fail(PSW_E_SHAPE, std::string(f == PSW_KV_LOCAL ? "local" : "global") +
                                   " pages held do not match the frontier");
  }
  if (post > s->rope_positions)
    return fail(PSW_E_RANGE, "position " + std::to_string(post - 1) + " is past the " +
                                 std::to_string(s->rope_positions) + " RoPE positions");
  if (s->ring_pages > 0) {
    // once the ring wraps it must hold every key the step's queries see
    const int64_t ring = s->ring_pages * s->pool[PSW_KV_LOCAL].page_size;
    if (post > ring && ring < s->window_left + n_new)
      return fail(PSW_E_RANGE, "a step of " + std::to_string(n_new) +
                                   " tokens does not fit the local ring with window " +
                                   std::to_string(s->window_left));
  } else if (s->window_left >= 0 && post > s->window_left + 1) {
    // without a ring, cache slots equal absolute positions only while no query
    // can lose a key to the window; a step past it is refused
    return fail(PSW_E_RANGE, "KV length " + std::to_string(post) +
                                 " would cross the local window of " +
                                 std::to_string(s->window_left + 1) + " keys");
  }
  int64_t need[2];
  for (int f = 0; f < 2; ++f)
    need[f] = s->pages_at(f, post) - static_cast<int64_t>(r->held[f].size());
  // take both sides first; if the second side is short, hand the first back
  std::vector<int32_t> got[2];
  if (!s->pool[PSW_KV_LOCAL].take(need[PSW_KV_LOCAL], &got[PSW_KV_LOCAL]))
    return fail(PSW_E_RANGE, "local pool has " +
                                 std::to_string(s->pool[PSW_KV_LOCAL].free_ids.size()) +
                                 " free pages, the step needs " + std::to_string(need[PSW_KV_LOCAL]));
  if (!s->pool[PSW_KV_GLOBAL].take(need[PSW_KV_GLOBAL], &got[PSW_KV_GLOBAL])) {
    s->pool[PSW_KV_LOCAL].give_back(got[PSW_KV_LOCAL]);
    return fail(PSW_E_RANGE, "global pool has " +
                                 std::to_string(s->pool[PSW_KV_GLOBAL].free_ids.size()) +
                                 " free pages, the step needs " +
                                 std::to_string(need[PSW_KV_GLOBAL]) +
                                 "; the local reservation was returned");
  }
  for (int f = 0; f < 2; ++f) r->reserved[f] = std::move(got[f]);
  r->pending = true;
  r->pending_n = n_new;
  return PSW_OK;
}

int psw_kv_commit(psw_kv_server* s, psw_kv_request* r) {
  psw::clear_error();
  int rc = check_pair(s, r);
  if (rc) return rc;
  if (!r->pending) return fail(PSW_E_PLAN, "no step is pending");
  for (int f = 0; f < 2; ++f) {
    r->held[f].insert(r->held[f].end(), r->reserved[f].begin(), r->reserved[f].end());
    r->reserved[f].clear();
  }
  r->frontier += r->pending_n;
  r->pending = false;
  r->pending_n = 0;
  return PSW_OK;
}

int psw_kv_abort(psw_kv_server* s, psw_kv_request* r) {
  psw::clear_error();
  int rc = check_pair(s, r);
  if (rc) return rc;
  if (!r->pending) return fail(PSW_E_PLAN, "no step is pending");
  for (int f = 0; f < 2; ++f) {
    s->pool[f].give_back(r->reserved[f]);
    r->reserved[f].clear();
  }
  r->pending = false;
  r->pending_n = 0;
  return PSW_OK;
}

int psw_kv_step_tables(const psw_kv_server* s, psw_kv_request* const* reqs, int64_t n_reqs,
                       int32_t family, int32_t* qo_indptr, int32_t* kv_page_indptr,
                       int32_t* kv_page_indices, int64_t indices_cap,
                       int32_t* kv_last_page_len, int32_t* kv_len) {
  psw::clear_error();
  if (!s || !reqs || !qo_indptr || !kv_page_indptr || !kv_page_indices || !kv_last_page_len ||
      !kv_len)
    return fail(PSW_E_NULL, "a server, request list or output array is NULL");
  int rc = check_family(family);
  if (rc) return rc;
  if (n_reqs < 1) return fail(PSW_E_SHAPE, "at least one request");
  std::unordered_set<const psw_kv_request*> seen;
  int64_t qo = 0, pages = 0;
  for (int64_t b = 0; b < n_reqs; ++b) {
    const psw_kv_request* r = reqs[b];
    rc = check_pair(s, r);
    if (rc) return rc;
    if (!seen.insert(r).second) return fail(PSW_E_SHAPE, "a request appears twice in the batch");
    if (!r->pending) return fail(PSW_E_PLAN, "request " + std::to_string(b) + " has no step pending");
    qo += r->pending_n;
    pages += static_cast<int64_t>(r->held[family].size() + r->reserved[family].size());
  }
  if (!psw::fits_i32(qo) || !psw::fits_i32(pages))
    return fail(PSW_E_OVERFLOW, "batch totals past INT32_MAX");
  if (pages > indices_cap)
    return fail(PSW_E_SHAPE, "kv_page_indices holds " + std::to_string(indices_cap) +
                                 " entries, the batch needs " + std::to_string(pages));
  // the step's tables: queries are the new tokens, KV is everything after it
  const int64_t psz = s->pool[family].page_size;
  qo_indptr[0] = 0;
  kv_page_indptr[0] = 0;
  int64_t pi = 0;
  for (int64_t b = 0; b < n_reqs; ++b) {
    const psw_kv_request* r = reqs[b];
    for (int32_t id : r->held[family]) kv_page_indices[pi++] = id;
    for (int32_t id : r->reserved[family]) kv_page_indices[pi++] = id;
    const int64_t kv = r->frontier + r->pending_n;
    qo_indptr[b + 1] = static_cast<int32_t>(qo_indptr[b] + r->pending_n);
    kv_page_indptr[b + 1] = static_cast<int32_t>(pi);
    kv_last_page_len[b] = static_cast<int32_t>((kv - 1) % psz + 1);
    kv_len[b] = static_cast<int32_t>(kv);
  }
  return PSW_OK;
}

}  // extern "C"
