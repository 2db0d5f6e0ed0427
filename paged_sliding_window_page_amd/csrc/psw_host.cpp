// Host-side validation, plan construction and work scheduling.  No HIP API is
// used in this file: everything here runs, and can be tested, without a GPU.
//
// Contracts implemented (see psw.h for the public statement):
//   [P1] PR "feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
//        Description: one overflow-checked geometry check for the prep and
//        attention entries, checked i32 narrowing, the plan keeps the largest
//        page id and final-page length and replaces them only when an update
//        succeeds as a whole, query/KV heads are validated before any
//        division, and the plan's tile must equal the kernel's own.
//   [P1] Verification: out-of-pool page ids, final-page lengths above the
//        page size, i32 overflow and a zero KV-head count are errors raised
//        before any launch.
//   [P2] Proposed Plan: the prep checks the layer index, that the pool holds
//        whole pages, that the request's pages cover every written position,
//        that positions stay inside the RoPE tables, and the table sizes.
#include "psw_host.hpp"

#include <cstdint>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <numeric>
#include <unordered_set>

namespace psw {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

bool fits_i32(int64_t v) {
  return v >= std::numeric_limits<int32_t>::min() && v <= std::numeric_limits<int32_t>::max();
}

bool checked_mul(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *out = a * b;
  return true;
}

static bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_pool(const psw_pool* p, bool need_base) {
  if (!p) return fail(PSW_E_NULL, "pool descriptor is NULL");
  if (need_base && !p->base) return fail(PSW_E_NULL, "pool base pointer is NULL");
  if (p->num_layers < 1 || p->num_pages < 1 || p->num_kv_heads < 0 || p->head_dim < 1 ||
      p->page_size < 1)
    return fail(p->num_kv_heads == 0 ? PSW_E_HEADS : PSW_E_SHAPE,
                "pool geometry has a non-positive extent");
  if (p->num_kv_heads == 0) return fail(PSW_E_HEADS, "pool has zero KV heads");
  if (!fits_i32(p->num_layers) || !fits_i32(p->num_pages) || !fits_i32(p->num_kv_heads) ||
      !fits_i32(p->head_dim) || !fits_i32(p->page_size))
    return fail(PSW_E_OVERFLOW, "pool extent past INT32_MAX");
  if (!is_pow2(p->page_size) || p->page_size > 1024)
    return fail(PSW_E_SHAPE, "page_size must be a power of two in [1, 1024]");
  // re-derive the whole-page element count with overflow-checked multiplies
  int64_t n = 1;
  const int64_t dims[6] = {p->num_layers, p->num_pages, 2, p->num_kv_heads, p->page_size,
                           p->head_dim};
  for (int64_t dim : dims)
    if (!checked_mul(n, dim, &n)) return fail(PSW_E_OVERFLOW, "pool size overflows int64");
  int64_t bytes;
  if (!checked_mul(n, 2, &bytes)) return fail(PSW_E_OVERFLOW, "pool byte size overflows int64");
  if (p->numel != n)
    return fail(PSW_E_SHAPE, "pool numel " + std::to_string(p->numel) +
                                 " != layers*pages*2*kv_heads*page_size*head_dim = " +
                                 std::to_string(n));
  // the kernels form a page's byte offset as a 32-bit page id times a 32-bit
  // page size
  if (2 * p->num_kv_heads * p->page_size * p->head_dim * 2 > int64_t(UINT32_MAX))
    return fail(PSW_E_UNSUPPORTED, "a pool page (K and V blocks) is 4 GiB or more");
  return PSW_OK;
}

int derive_tile_q(int64_t group, int64_t head_dim, int32_t* tile_q) {
  if (!tile_q) return fail(PSW_E_NULL, "tile_q output pointer is NULL");
  if (!fits_i32(group) || !fits_i32(head_dim))
    return fail(PSW_E_OVERFLOW, "tile query argument past INT32_MAX");
  // positivity is checked after narrowing, in the i32 domain
  const int32_t g = static_cast<int32_t>(group), d = static_cast<int32_t>(head_dim);
  if (g <= 0 || d <= 0) return fail(PSW_E_HEADS, "tile query needs a positive group and head_dim");
  if (d != 256 && d != 512) return fail(PSW_E_UNSUPPORTED, "no prefill kernel for this head_dim");
  if (!is_pow2(g) || g > kMaxGroup)
    return fail(PSW_E_UNSUPPORTED, "GQA group must be a power of two <= 32");
  *tile_q = (d == 512 ? kPrefillRows512 : kPrefillRows) / g;
  return PSW_OK;
}

static uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

int build_state(const psw_plan_desc* d, PlanState* out) {
  if (!d) return fail(PSW_E_NULL, "plan description is NULL");
  // settle the head relation first: nothing below divides before this passes
  if (d->num_kv_heads == 0) return fail(PSW_E_HEADS, "num_kv_heads is zero");
  if (d->num_kv_heads < 0 || d->num_qo_heads <= 0)
    return fail(PSW_E_HEADS, "head counts must be positive");
  if (!fits_i32(d->num_kv_heads) || !fits_i32(d->num_qo_heads))
    return fail(PSW_E_OVERFLOW, "head count past INT32_MAX");
  if (d->num_qo_heads % d->num_kv_heads != 0)
    return fail(PSW_E_HEADS, "num_qo_heads is not a multiple of num_kv_heads");
  if (d->batch < 1) return fail(PSW_E_SHAPE, "batch must be >= 1");
  if (!fits_i32(d->batch) || !fits_i32(d->batch + 1))
    return fail(PSW_E_OVERFLOW, "batch past INT32_MAX");
  if (d->head_dim < 1 || d->page_size < 1 || d->num_pages < 1)
    return fail(PSW_E_SHAPE, "head_dim, page_size and num_pages must be positive");
  if (!fits_i32(d->head_dim) || !fits_i32(d->page_size) || !fits_i32(d->num_pages))
    return fail(PSW_E_OVERFLOW, "geometry past INT32_MAX");
  if (!is_pow2(d->page_size) || d->page_size > 1024)
    return fail(PSW_E_SHAPE, "page_size must be a power of two in [1, 1024]");
  if (!d->qo_indptr || !d->kv_page_indptr || !d->kv_last_page_len ||
      (!d->kv_page_indices && d->kv_page_indptr[d->batch] > 0))
    return fail(PSW_E_NULL, "a plan metadata array is NULL");
  if (d->tile_q_override < 0 || !fits_i32(d->tile_q_override))
    return fail(PSW_E_OVERFLOW, "tile_q_override must be in [0, INT32_MAX]");

  PlanState s;
  const int32_t B = static_cast<int32_t>(d->batch);
  s.batch = B;
  s.num_qo_heads = static_cast<int32_t>(d->num_qo_heads);
  s.num_kv_heads = static_cast<int32_t>(d->num_kv_heads);
  s.group = s.num_qo_heads / s.num_kv_heads;
  s.head_dim = static_cast<int32_t>(d->head_dim);
  s.page_size = static_cast<int32_t>(d->page_size);
  s.num_pages = static_cast<int32_t>(d->num_pages);

  if (d->qo_indptr[0] != 0) return fail(PSW_E_SHAPE, "qo_indptr[0] must be 0");
  if (d->kv_page_indptr[0] != 0) return fail(PSW_E_SHAPE, "kv_page_indptr[0] must be 0");
  s.qo_indptr.assign(d->qo_indptr, d->qo_indptr + B + 1);
  s.kv_page_indptr.assign(d->kv_page_indptr, d->kv_page_indptr + B + 1);
  s.last_page_len.assign(d->kv_last_page_len, d->kv_last_page_len + B);
  for (int32_t b = 0; b < B; ++b) {
    if (s.qo_indptr[b + 1] <= s.qo_indptr[b])
      return fail(PSW_E_SHAPE, "qo_indptr must be strictly increasing (qo_len >= 1), request " +
                                   std::to_string(b));
    if (s.kv_page_indptr[b + 1] <= s.kv_page_indptr[b])
      return fail(PSW_E_SHAPE, "kv_page_indptr must be strictly increasing (>= 1 page), request " +
                                   std::to_string(b));
  }
  s.total_qo = s.qo_indptr[B];
  s.total_pages = s.kv_page_indptr[B];
  s.kv_page_indices.assign(d->kv_page_indices, d->kv_page_indices + s.total_pages);
  for (int32_t i = 0; i < s.total_pages; ++i) {
    const int32_t id = s.kv_page_indices[i];
    if (id < 0 || id >= s.num_pages)
      return fail(PSW_E_RANGE, "page id " + std::to_string(id) + " at position " +
                                   std::to_string(i) + " is outside the pool of " +
                                   std::to_string(s.num_pages) + " pages");
    s.max_page_id = std::max(s.max_page_id, id);
  }
  s.kv_len.resize(B);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t last = s.last_page_len[b];
    if (last < 1 || last > s.page_size)
      return fail(PSW_E_RANGE, "last_page_len " + std::to_string(last) + " of request " +
                                   std::to_string(b) + " is outside [1, page_size]");
    const int64_t n_pages = int64_t(s.kv_page_indptr[b + 1]) - s.kv_page_indptr[b];
    int64_t kv = (n_pages - 1) * int64_t(s.page_size) + last;
    if (!fits_i32(kv))
      return fail(PSW_E_OVERFLOW, "kv_len of request " + std::to_string(b) + " is past INT32_MAX");
    if (d->kv_len) {
      // absolute length: equal to the derived one unless the pages wrap
      const int64_t given = d->kv_len[b];
      if (given <= n_pages * s.page_size) {
        if (given != kv)
          return fail(PSW_E_SHAPE, "kv_len of request " + std::to_string(b) +
                                       " disagrees with its pages and last_page_len");
      } else if (last != (given - 1) % s.page_size + 1) {
        return fail(PSW_E_SHAPE, "last_page_len of wrapped request " + std::to_string(b) +
                                     " must be (kv_len - 1) % page_size + 1");
      }
      kv = given;
      s.any_ring = s.any_ring || given > n_pages * s.page_size;
    }
    const int32_t qo = s.qo_indptr[b + 1] - s.qo_indptr[b];
    if (kv < qo)
      return fail(PSW_E_SHAPE, "request " + std::to_string(b) + " has kv_len < qo_len");
    s.kv_len[b] = static_cast<int32_t>(kv);
    s.max_last_page_len = std::max(s.max_last_page_len, last);
    s.max_kv_len = std::max(s.max_kv_len, s.kv_len[b]);
    s.max_qo_len = std::max(s.max_qo_len, qo);
  }
  int32_t derived = 0;
  if (derive_tile_q(s.group, s.head_dim, &derived) != PSW_OK) derived = 0;  // no kernel: entries reject
  clear_error();
  if (d->tile_q_override > 0) {
    s.tile_q = static_cast<int32_t>(d->tile_q_override);
    s.tile_overridden = true;
  } else {
    s.tile_q = derived;
  }
  uint64_t h = 1469598103934665603ull;
  const int32_t scalars[] = {s.batch, s.num_qo_heads, s.num_kv_heads, s.head_dim, s.page_size,
                             s.num_pages, s.tile_q, s.max_page_id, s.max_last_page_len};
  h = fnv1a(h, scalars, sizeof(scalars));
  for (const auto* v :
       {&s.qo_indptr, &s.kv_page_indptr, &s.kv_page_indices, &s.last_page_len, &s.kv_len})
    h = fnv1a(h, v->data(), v->size() * sizeof(int32_t));
  s.digest = h;
  *out = std::move(s);
  return PSW_OK;
}

int64_t effective_window(const PlanState& st, int64_t window_left) {
  // a window at least max_kv_len - 1 wide excludes nothing: run the causal path
  if (window_left < 0 || window_left >= int64_t(st.max_kv_len) - 1) return -1;
  return window_left;
}

void build_prefill_schedule(const PlanState& st, int64_t wl, int32_t kv_tile, PrefillSchedule* out) {
  struct Item { int32_t b, t0, lo, hi; int64_t cost; };
  std::vector<Item> items;
  int64_t total = 0;
  for (int32_t b = 0; b < st.batch; ++b) {
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int32_t start = st.kv_len[b] - qo;
    for (int32_t t0 = 0; t0 < qo; t0 += st.tile_q) {
      const int64_t p0 = int64_t(start) + t0;
      const int64_t p1 = int64_t(start) + std::min(t0 + st.tile_q, qo) - 1;
      const int64_t lo = wl >= 0 ? std::max<int64_t>(0, p0 - wl) : 0;
      const int64_t cost = p1 / kv_tile - lo / kv_tile + 1;
      items.push_back({b, t0, int32_t(lo), int32_t(p1), cost});
      total += cost;
    }
  }
  // longest first, so the tail of the grid is made of short items
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& c) { return a.cost > c.cost; });
  out->items.resize(items.size() * 4);
  for (size_t i = 0; i < items.size(); ++i) {
    out->items[4 * i + 0] = items[i].b;
    out->items[4 * i + 1] = items[i].t0;
    out->items[4 * i + 2] = items[i].lo;
    out->items[4 * i + 3] = items[i].hi;
  }
  out->window_left = wl;
  out->kv_tile = kv_tile;
  out->tile_q = st.tile_q;
  out->total_tiles = total;
}

int32_t effective_decode_mode(const PlanState& st, int32_t mode) {
  return st.group > kDecodeKernelMaxGroup ? int32_t(PSW_DECODE_SPLIT) : mode;
}

void build_decode_schedule(const PlanState& st, int64_t wl, int32_t mode, DecodeSchedule* out) {
  // keys each request must read: the window (or everything) ending at p = kv_len - 1
  std::vector<int64_t> lo(st.batch), n(st.batch);
  int64_t n_max = 0;
  for (int32_t b = 0; b < st.batch; ++b) {
    const int64_t p = int64_t(st.kv_len[b]) - 1;
    lo[b] = wl >= 0 ? std::max<int64_t>(0, p - wl) : 0;
    n[b] = p - lo[b] + 1;
    n_max = std::max(n_max, n[b]);
  }
  // The decode kernel runs a list of items per work-group and writes whole
  // requests itself; the attention kernel (wider groups) runs one item per
  // work-group and always writes partials.
  const bool decode_kernel = st.group <= kDecodeKernelMaxGroup;
  // Direct form: one work-group per (request, KV head) reads all of the
  // request's keys and writes O (no partials, no merge launch).
  const bool full_grid = int64_t(st.batch) * st.num_kv_heads >= kDecodeFullGrid;
  const int64_t direct_keys = full_grid ? kDecodeDirectKeysFull
                              : st.head_dim == 256 ? kDecodeDirectKeys256
                                                   : kDecodeDirectKeys512;
  const bool direct = decode_kernel && (mode == PSW_DECODE_DIRECT ||
                                        (mode == PSW_DECODE_AUTO && n_max <= direct_keys));
  out->items.clear();
  out->wg_items.clear();
  out->req_splits.assign(2 * st.batch, 0);
  int32_t slot = 0;
  if (direct) {
    // longest first, so the short requests fill in behind the long ones
    std::vector<int32_t> order(st.batch);
    for (int32_t b = 0; b < st.batch; ++b) order[b] = b;
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return n[x] > n[y]; });
    for (int32_t b : order) {
      out->wg_items.push_back(static_cast<int32_t>(out->items.size() / 4));
      out->items.insert(out->items.end(), {b, -1, int32_t(lo[b]), int32_t(lo[b] + n[b] - 1)});
    }
  } else {
    // Split form.  The requests' keys, in units of kDecodeSplitUnit keys at
    // absolute multiples (so no decode tile is read by two pieces), are laid
    // end to end in request order and cut into equal contiguous shares, one
    // per work-group, at most kDecodeResidentWaves' worth of work-groups (all
    // of them run at once): every work-group streams the same amount and the
    // launch ends together.
    // A share covers pieces of one or more requests; a piece that is a whole
    // request is written directly, the others get a partial slot each, and
    // the pieces of a request are consecutive, so its slots are too.
    const int64_t unit = kDecodeSplitUnit;
    std::vector<int64_t> u0(st.batch), start(st.batch + 1, 0);
    for (int32_t b = 0; b < st.batch; ++b) {
      u0[b] = lo[b] / unit;
      start[b + 1] = start[b] + (lo[b] + n[b] - 1) / unit - u0[b] + 1;
    }
    const int64_t total = start[st.batch];
    // A piece writes group x head_dim fp32 partials that the merge reads back,
    // against 4 x head_dim bytes of K and V per key: shares of at least
    // 16 x group keys keep that traffic under 1/16 of the K/V stream.
    const int64_t min_units = std::max<int64_t>(1, (16 * int64_t(st.group) + unit - 1) / unit);
    const int64_t waves = st.head_dim / 128;
    const int64_t resident =
        std::max<int64_t>(1, kDecodeResidentWaves / waves / st.num_kv_heads);
    // at least one work-group per request (up to the resident count): a
    // work-group runs its items one after another, each paying the latency of
    // its first loads, so short requests are not stacked several deep
    const int64_t groups = std::min(
        resident, std::max<int64_t>({1, (total + min_units - 1) / min_units, int64_t(st.batch)}));
    int32_t b = 0;
    for (int64_t g = 0; g < groups; ++g) {
      int64_t s0 = total * g / groups;
      const int64_t s1 = total * (g + 1) / groups;
      out->wg_items.push_back(static_cast<int32_t>(out->items.size() / 4));
      while (s0 < s1) {
        while (start[b + 1] <= s0) ++b;
        const int64_t a = s0 - start[b];
        const int64_t e = std::min(s1, start[b + 1]) - start[b];
        const int64_t k0 = std::max(lo[b], (u0[b] + a) * unit);
        const int64_t k1 = std::min(lo[b] + n[b] - 1, (u0[b] + e) * unit - 1);
        const bool whole = a == 0 && start[b] + e == start[b + 1];
        int32_t sl = -1;
        if (!(whole && decode_kernel)) {
          if (out->req_splits[2 * b + 1] == 0) out->req_splits[2 * b] = slot;
          ++out->req_splits[2 * b + 1];
          sl = slot++;
        }
        out->items.insert(out->items.end(), {b, sl, int32_t(k0), int32_t(k1)});
        s0 = start[b] + e;
      }
    }
  }
  out->wg_items.push_back(static_cast<int32_t>(out->items.size() / 4));
  out->num_partials = slot;
  out->num_wgs = decode_kernel ? static_cast<int32_t>(out->wg_items.size() - 1)
                               : static_cast<int32_t>(out->items.size() / 4);
  out->window_left = wl;
  out->mode = mode;
  out->direct = slot == 0;
}

void build_prep_items(const PlanState& st, std::vector<int32_t>* out) {
  out->clear();
  for (int32_t b = 0; b < st.batch; ++b) {
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int32_t start = st.kv_len[b] - qo;
    int32_t t = 0;
    while (t < qo) {
      const int32_t pos = start + t;
      const int32_t slot = pos & (st.page_size - 1);
      const int32_t n = std::min({qo - t, st.page_size - slot, 16});
      const int32_t page = st.page_of(b, pos);
      out->insert(out->end(), {b, st.qo_indptr[b] + t, n, page, slot, pos});
      t += n;
    }
  }
}

static int bad_item(const char* what, size_t i, const std::string& why) {
  return fail(PSW_E_PLAN, std::string(what) + " item " + std::to_string(i) + ": " + why);
}

int check_prefill_items(const PlanState& st, const PrefillSchedule& ps) {
  if (ps.items.size() % 4) return fail(PSW_E_PLAN, "prefill schedule is not made of quads");
  for (size_t i = 0; i < ps.items.size() / 4; ++i) {
    const int32_t b = ps.items[4 * i], t0 = ps.items[4 * i + 1];
    const int32_t k0 = ps.items[4 * i + 2], k1 = ps.items[4 * i + 3];
    if (b < 0 || b >= st.batch) return bad_item("prefill", i, "request out of range");
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    if (t0 < 0 || t0 >= qo || t0 % ps.tile_q)
      return bad_item("prefill", i, "first query token outside the request or off the tile");
    if (k0 < 0 || k0 > k1 || k1 >= st.kv_len[b])
      return bad_item("prefill", i, "key range outside the request's keys");
  }
  return PSW_OK;
}

int check_decode_items(const PlanState& st, const DecodeSchedule& ds, bool split_kernel) {
  if (ds.items.size() % 4) return fail(PSW_E_PLAN, "decode schedule is not made of quads");
  const size_t n = ds.items.size() / 4;
  if (ds.req_splits.size() != size_t(2) * st.batch)
    return fail(PSW_E_PLAN, "decode schedule has no split list per request");
  for (size_t i = 0; i < n; ++i) {
    const int32_t b = ds.items[4 * i], sl = ds.items[4 * i + 1];
    const int32_t k0 = ds.items[4 * i + 2], k1 = ds.items[4 * i + 3];
    if (b < 0 || b >= st.batch) return bad_item("decode", i, "request out of range");
    if (k0 < 0 || k0 > k1 || k1 >= st.kv_len[b])
      return bad_item("decode", i, "key range outside the request's keys");
    if (sl >= ds.num_partials || sl < -1)
      return bad_item("decode", i, "partial slot outside the workspace");
    if (sl < 0 && split_kernel)
      return bad_item("decode", i, "the split attention kernel writes a partial for every item");
  }
  for (int32_t b = 0; b < st.batch; ++b) {
    const int64_t f = ds.req_splits[2 * b], c = ds.req_splits[2 * b + 1];
    if (c < 0 || (c > 0 && (f < 0 || f + c > ds.num_partials)))
      return fail(PSW_E_PLAN, "decode split list of request " + std::to_string(b) +
                                  " points outside the workspace");
  }
  if (!split_kernel) {
    if (ds.wg_items.size() != size_t(ds.num_wgs) + 1 || ds.wg_items.front() != 0 ||
        ds.wg_items.back() != int32_t(n))
      return fail(PSW_E_PLAN, "decode work-group item lists do not cover the items");
    for (int32_t g = 0; g < ds.num_wgs; ++g)
      if (ds.wg_items[g] > ds.wg_items[g + 1])
        return fail(PSW_E_PLAN, "decode work-group item lists are not in order");
  } else if (int64_t(ds.num_wgs) != int64_t(n)) {
    return fail(PSW_E_PLAN, "the split attention kernel runs one item per work-group");
  }
  return PSW_OK;
}

int check_prep_items(const PlanState& st, const std::vector<int32_t>& items) {
  constexpr size_t kInts = 6, kMaxTokens = 16;
  if (items.size() % kInts) return fail(PSW_E_PLAN, "prep items are not made of sextuples");
  for (size_t i = 0; i < items.size() / kInts; ++i) {
    const int32_t* it = items.data() + kInts * i;
    const int32_t b = it[0], tok0 = it[1], n = it[2], page = it[3], slot = it[4], pos = it[5];
    if (b < 0 || b >= st.batch) return bad_item("prep", i, "request out of range");
    const int32_t qo = st.qo_indptr[b + 1] - st.qo_indptr[b];
    const int64_t start = int64_t(st.kv_len[b]) - qo;
    if (n < 1 || size_t(n) > kMaxTokens) return bad_item("prep", i, "token count outside [1, 16]");
    if (pos < start || int64_t(pos) + n > st.kv_len[b])
      return bad_item("prep", i, "positions outside the request's new tokens");
    if (tok0 != st.qo_indptr[b] + (pos - start))
      return bad_item("prep", i, "first token does not match its position");
    if (slot != pos % st.page_size || slot + n > st.page_size)
      return bad_item("prep", i, "slots leave the page");
    if (page < 0 || page >= st.num_pages || page != st.page_of(b, pos))
      return bad_item("prep", i, "page is not the request's page for its position");
  }
  return PSW_OK;
}

static int check_plan_vs_pool(const psw_plan* plan, const psw_pool* pool, int64_t layer,
                              psw_stream_t stream, int64_t want_head_dim) {
  if (!plan) return fail(PSW_E_NULL, "plan is NULL");
  int rc = check_pool(pool, true);
  if (rc != PSW_OK) return rc;
  const PlanState& s = plan->st;
  if (stream != plan->stream)
    return fail(PSW_E_PLAN, "stream differs from the stream the plan was created on");
  if (s.head_dim != want_head_dim || pool->head_dim != want_head_dim)
    return fail(PSW_E_PLAN, "entry is for head_dim " + std::to_string(want_head_dim) +
                                ", plan has " + std::to_string(s.head_dim) + ", pool has " +
                                std::to_string(pool->head_dim));
  if (s.num_kv_heads != pool->num_kv_heads)
    return fail(PSW_E_PLAN, "plan and pool disagree on num_kv_heads");
  if (s.page_size != pool->page_size)
    return fail(PSW_E_PLAN, "plan and pool disagree on page_size");
  if (s.max_page_id >= pool->num_pages)
    return fail(PSW_E_RANGE, "plan page id " + std::to_string(s.max_page_id) +
                                 " is past the pool's " + std::to_string(pool->num_pages) +
                                 " pages");
  if (s.max_last_page_len > pool->page_size)
    return fail(PSW_E_RANGE, "plan last_page_len past the pool's page_size");
  if (layer < 0 || layer >= pool->num_layers)
    return fail(PSW_E_RANGE, "layer " + std::to_string(layer) + " outside [0, " +
                                 std::to_string(pool->num_layers) + ")");
  return PSW_OK;
}

int check_attention_call(const psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                         float sm_scale, int64_t window_left, const void* o, int32_t o_dtype,
                         psw_stream_t stream, int64_t want_head_dim) {
  int rc = check_plan_vs_pool(plan, pool, layer, stream, want_head_dim);
  if (rc != PSW_OK) return rc;
  if (!q || !o) return fail(PSW_E_NULL, "q or o is NULL");
  if (!std::isfinite(sm_scale)) return fail(PSW_E_SCALE, "sm_scale is not finite");
  if (window_left < -1) return fail(PSW_E_RANGE, "window_left must be >= -1");
  if (o_dtype != 0 && o_dtype != 1) return fail(PSW_E_SHAPE, "o_dtype must be 0 (fp32) or 1 (bf16)");
  const PlanState& s = plan->st;
  int32_t tile = 0;
  rc = derive_tile_q(s.group, s.head_dim, &tile);
  if (rc != PSW_OK) return rc;
  if (s.tile_q != tile)
    return fail(PSW_E_PLAN, "plan records tile_q " + std::to_string(s.tile_q) +
                                " but the kernel is compiled for " + std::to_string(tile));
  int64_t rows;
  if (!checked_mul(int64_t(s.total_qo), s.num_qo_heads, &rows) ||
      !checked_mul(rows, s.head_dim, &rows))
    return fail(PSW_E_OVERFLOW, "q/o size overflows int64");
  // a wrapped ring holds the last n_pages * page_size positions: every key a
  // query of the call sees must be among them
  if (s.any_ring) {
    for (int32_t b = 0; b < s.batch; ++b) {
      if (!s.wraps(b)) continue;
      const int64_t ring = int64_t(s.n_pages(b)) * s.page_size;
      const int64_t qo = s.qo_indptr[b + 1] - s.qo_indptr[b];
      if (window_left < 0 || ring < window_left + qo)
        return fail(PSW_E_RANGE, "request " + std::to_string(b) + " has a ring of " +
                                     std::to_string(ring) + " slots, too few for " +
                                     (window_left < 0 ? std::string("attention without a window")
                                                      : "window " + std::to_string(window_left) +
                                                            " and " + std::to_string(qo) +
                                                            " queries"));
    }
  }
  return PSW_OK;
}

// RoPE tables, eps and the positions the plan writes (shared by the preps).
static int check_rope_eps(const PlanState& s, int64_t want_head_dim, const float* rope_cos,
                          const float* rope_sin, int64_t rope_positions, int64_t rope_cos_numel,
                          int64_t rope_sin_numel, float eps) {
  if (!rope_cos || !rope_sin) return fail(PSW_E_NULL, "RoPE table pointer is NULL");
  if (rope_positions < 1) return fail(PSW_E_SHAPE, "rope_positions must be >= 1");
  if (!fits_i32(rope_positions)) return fail(PSW_E_OVERFLOW, "rope_positions past INT32_MAX");
  int64_t want;
  if (!checked_mul(rope_positions, want_head_dim / 2, &want))
    return fail(PSW_E_OVERFLOW, "RoPE table size overflows int64");
  if (rope_cos_numel != want || rope_sin_numel != want)
    return fail(PSW_E_SHAPE, "RoPE tables must hold rope_positions * head_dim/2 = " +
                                 std::to_string(want) + " floats each");
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(PSW_E_SCALE, "eps must be finite and > 0");
  // positions written are start_pos .. kv_len-1; the last one must index the tables
  if (int64_t(s.max_kv_len) - 1 >= rope_positions)
    return fail(PSW_E_RANGE, "position " + std::to_string(s.max_kv_len - 1) +
                                 " is past the RoPE table of " + std::to_string(rope_positions) +
                                 " positions");
  return PSW_OK;
}

int check_prep_call(const psw_plan* plan, const psw_pool* pool, int64_t layer,
                    int64_t want_head_dim, const float* rope_cos, const float* rope_sin,
                    int64_t rope_positions, int64_t rope_cos_numel, int64_t rope_sin_numel,
                    float eps, psw_stream_t stream) {
  int rc = check_plan_vs_pool(plan, pool, layer, stream, want_head_dim);
  if (rc != PSW_OK) return rc;
  const PlanState& s = plan->st;
  rc = check_rope_eps(s, want_head_dim, rope_cos, rope_sin, rope_positions, rope_cos_numel,
                      rope_sin_numel, eps);
  if (rc != PSW_OK) return rc;
  // every written position has a page, and no page is written twice
  std::unordered_set<int32_t> written;
  for (int32_t b = 0; b < s.batch; ++b) {
    const int32_t qo = s.qo_indptr[b + 1] - s.qo_indptr[b];
    const int64_t start = int64_t(s.kv_len[b]) - qo;
    const int64_t n_pages = int64_t(s.kv_page_indptr[b + 1]) - s.kv_page_indptr[b];
    if (!s.wraps(b) && n_pages * s.page_size < start + qo)
      return fail(PSW_E_RANGE, "pages of request " + std::to_string(b) +
                                   " do not cover its positions");
    if (qo > n_pages * s.page_size)
      return fail(PSW_E_RANGE, "request " + std::to_string(b) + " writes " + std::to_string(qo) +
                                   " positions into a ring of " +
                                   std::to_string(n_pages * s.page_size) + " slots");
    for (int64_t pg = start / s.page_size; pg <= (start + qo - 1) / s.page_size; ++pg) {
      const int32_t id = s.page_of(b, pg * s.page_size);
      if (!written.insert(id).second)
        return fail(PSW_E_SHAPE, "page " + std::to_string(id) +
                                     " would be written twice by this prep call");
    }
  }
  return PSW_OK;
}

int check_q_prep_call(const psw_plan* plan, int64_t want_head_dim, const void* q_in,
                      const void* q_norm_w, const float* rope_cos, const float* rope_sin,
                      int64_t rope_positions, int64_t rope_cos_numel, int64_t rope_sin_numel,
                      float eps, const void* q_out, psw_stream_t stream) {
  if (!plan) return fail(PSW_E_NULL, "plan is NULL");
  const PlanState& s = plan->st;
  if (stream != plan->stream)
    return fail(PSW_E_PLAN, "stream differs from the stream the plan was created on");
  if (s.head_dim != want_head_dim)
    return fail(PSW_E_PLAN, "entry is for head_dim " + std::to_string(want_head_dim) +
                                ", plan has " + std::to_string(s.head_dim));
  if (!q_in || !q_norm_w || !q_out) return fail(PSW_E_NULL, "q_in, q_norm_w or q_out is NULL");
  return check_rope_eps(s, want_head_dim, rope_cos, rope_sin, rope_positions, rope_cos_numel,
                        rope_sin_numel, eps);
}

}  // namespace psw

// ------------------------------------------------------------ C ABI (host) --

extern "C" {

const char* psw_last_error(void) { return psw::g_last_error.c_str(); }

const char* psw_version(void) { return "psw 0.1.0 gfx950"; }

int psw_check_pool(const psw_pool* pool) {
  psw::clear_error();
  return psw::check_pool(pool, false);
}

int psw_plan_decode_form(const psw_plan* plan, int64_t window_left, int32_t* direct,
                         int64_t* work_groups) {
  psw::clear_error();
  if (!plan || !direct || !work_groups) return psw::fail(PSW_E_NULL, "plan or output is NULL");
  const psw::PlanState& st = plan->st;
  if (st.max_qo_len != 1) return psw::fail(PSW_E_SHAPE, "the plan is not a decode batch");
  if (window_left < -1) return psw::fail(PSW_E_RANGE, "window_left must be >= -1");
  psw::DecodeSchedule ds;
  psw::build_decode_schedule(st, psw::effective_window(st, window_left),
                             psw::effective_decode_mode(st, plan->decode_mode), &ds);
  *direct = ds.direct ? 1 : 0;
  *work_groups = int64_t(ds.num_wgs) * st.num_kv_heads;
  return PSW_OK;
}

int psw_plan_set_decode_mode(psw_plan* plan, int32_t mode) {
  psw::clear_error();
  if (!plan) return psw::fail(PSW_E_NULL, "plan is NULL");
  if (mode != PSW_DECODE_AUTO && mode != PSW_DECODE_SPLIT && mode != PSW_DECODE_DIRECT)
    return psw::fail(PSW_E_SHAPE, "decode mode must be PSW_DECODE_AUTO, _SPLIT or _DIRECT");
  plan->decode_mode = mode;
  plan->decode.window_left = -2;  // rebuilt by the next decode call
  return PSW_OK;
}

int psw_prefill_tile_q(int64_t group, int64_t head_dim, int32_t* tile_q) {
  psw::clear_error();
  return psw::derive_tile_q(group, head_dim, tile_q);
}

int psw_plan_create(const psw_plan_desc* desc, psw_stream_t stream, psw_plan** out) {
  psw::clear_error();
  if (!out) return psw::fail(PSW_E_NULL, "plan output pointer is NULL");
  psw::PlanState st;
  int rc = psw::build_state(desc, &st);
  if (rc != PSW_OK) return rc;
  psw_plan* p = new psw_plan();
  p->stream = stream;
  p->st = std::move(st);
  p->generation = 1;
  *out = p;
  return PSW_OK;
}

int psw_plan_update(psw_plan* plan, const psw_plan_desc* desc) {
  psw::clear_error();
  if (!plan) return psw::fail(PSW_E_NULL, "plan is NULL");
  psw::PlanState st;
  int rc = psw::build_state(desc, &st);  // builds the whole new state off to the side
  if (rc != PSW_OK) return rc;           // ... and leaves the plan untouched on failure
  plan->st = std::move(st);              // commit
  plan->generation += 1;
  plan->prefill = psw::PrefillSchedule();
  plan->decode = psw::DecodeSchedule();
  plan->prep_items.clear();
  plan->prep_built = false;
  return PSW_OK;
}

void psw_plan_destroy(psw_plan* plan) {
  if (!plan) return;
  if (plan->mirror) psw_mirror_free(plan->mirror, plan->stream);
  delete plan;
}

int psw_plan_get_info(const psw_plan* plan, psw_plan_info* info) {
  psw::clear_error();
  if (!plan || !info) return psw::fail(PSW_E_NULL, "plan or info is NULL");
  const psw::PlanState& s = plan->st;
  info->batch = s.batch;
  info->total_qo = s.total_qo;
  info->total_pages = s.total_pages;
  info->max_qo_len = s.max_qo_len;
  info->max_kv_len = s.max_kv_len;
  info->max_page_id = s.max_page_id;
  info->max_last_page_len = s.max_last_page_len;
  info->num_qo_heads = s.num_qo_heads;
  info->num_kv_heads = s.num_kv_heads;
  info->head_dim = s.head_dim;
  info->page_size = s.page_size;
  info->num_pages = s.num_pages;
  info->group = s.group;
  info->tile_q = s.tile_q;
  info->generation = plan->generation;
  info->digest = s.digest;
  return PSW_OK;
}

}  // extern "C"
