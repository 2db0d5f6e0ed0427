// One-token decode at head_dim 512 that allocates no memory: the plan's
// metadata, the decode schedule and the split-KV partials live in a
// file-scope device array (`scratch`) instead of the plan's device mirror.
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// Each GPU holds its own copy of `scratch` until the process ends.  In host
// code the array's name is only a host-side stand-in: its device address is
// looked up once per device (hipGetSymbolAddress, on the first call with that
// device current) and only that address is used for copies and kernel
// arguments.  Every call on a GPU shares the GPU's copy and leaves its
// contents behind; two calls that overlap on one GPU (other streams, other
// threads) race on it.  The layout is rebuilt by every call: nothing needs to
// start at zero (every partial slot a merge reads is written by the decode
// launch before it).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "psw_device.hpp"
#include "psw_host.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
// what the device's copy holds: the plan state (digest), window and mode
struct Held {
  bool valid = false;
  uint64_t digest = 0, generation = 0;
  const void* plan = nullptr;
  int64_t wl = -3;
  int32_t mode = -1;
};
Held g_held[kMaxDevices];

using psw::fail;

int hip_fail(hipError_t e, const char* what) {
  return fail(PSW_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Device address of this GPU's scratch array (looked up once per device).
int scratch_of(int dev, char** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PSW_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_ptr[dev]);
  return PSW_OK;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

extern "C" int paged_decode_hd512_noalloc(psw_plan* plan, const psw_pool* pool, int64_t layer,
                                          const void* q, float sm_scale, void* o,
                                          int32_t o_dtype, psw_stream_t stream) {
  psw::clear_error();
  constexpr int D = 512;
  int rc = psw::check_attention_call(plan, pool, layer, q, sm_scale, -1, o, o_dtype, stream, D);
  if (rc) return rc;
  const psw::PlanState& st = plan->st;
  if (st.max_qo_len != 1)
    return fail(PSW_E_SHAPE, "decode entries take one query token per request");
  if (st.page_size < 8) return fail(PSW_E_UNSUPPORTED, "the decode kernel needs page_size >= 8");
  if (st.group > psw_dev::kDecodeMaxGroup)
    return fail(PSW_E_UNSUPPORTED, "the allocation-free decode runs GQA groups of at most 16");
  const int64_t wle = psw::effective_window(st, -1);
  const int32_t dmode = psw::effective_decode_mode(st, plan->decode_mode);
  if (plan->decode.window_left != wle || plan->decode.mode != dmode)
    psw::build_decode_schedule(st, wle, dmode, &plan->decode);
  const psw::DecodeSchedule& ds = plan->decode;
  rc = psw::check_decode_items(st, ds, false);
  if (rc) return rc;

  // layout: qo_indptr | kv_page_indptr | kv_page_indices | kv_len | items |
  // wg_items | partial O | partial (max, sum), 256-byte aligned
  const size_t B = size_t(st.batch);
  size_t off = 0;
  const size_t o_qo = off;
  off = align256(off + (B + 1) * 4);
  const size_t o_kvp = off;
  off = align256(off + (B + 1) * 4);
  const size_t o_idx = off;
  off = align256(off + st.kv_page_indices.size() * 4);
  const size_t o_len = off;
  off = align256(off + B * 4);
  const size_t o_items = off;
  off = align256(off + (ds.items.size() + ds.wg_items.size()) * 4);
  const size_t o_part = off;
  const size_t n_part = size_t(ds.num_partials) * st.num_qo_heads;
  off = align256(off + n_part * D * 4);
  const size_t o_ml = off;
  off = align256(off + n_part * 2 * 4);
  if (off > kScratchBytes)
    return fail(PSW_E_RANGE, "the batch needs " + std::to_string(off) +
                                 " bytes of workspace; the allocation-free decode holds " +
                                 std::to_string(kScratchBytes));

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PSW_E_UNSUPPORTED, "device index out of range");
  char* base = nullptr;
  rc = scratch_of(dev, &base);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);

  // Upload the metadata and schedule unless this GPU's copy already holds
  // them (same plan state, window and mode).  The sources are pageable host
  // memory owned by the plan, which HIP copies synchronously with respect to
  // the host, so they may change as soon as a copy returns.
  {
    std::lock_guard<std::mutex> lock(g_mu);
    Held& h = g_held[dev];
    const bool same = h.valid && h.digest == st.digest && h.plan == plan &&
                      h.generation == plan->generation && h.wl == wle && h.mode == dmode;
    if (!same) {
      h.valid = false;
      struct Part { size_t off; const std::vector<int32_t>* v; };
      const Part parts[] = {{o_qo, &st.qo_indptr}, {o_kvp, &st.kv_page_indptr},
                            {o_idx, &st.kv_page_indices}, {o_len, &st.kv_len},
                            {o_items, &ds.items},
                            {o_items + ds.items.size() * 4, &ds.wg_items}};
      for (const Part& pt : parts) {
        if (pt.v->empty()) continue;
        e = hipMemcpyAsync(base + pt.off, pt.v->data(), pt.v->size() * 4,
                           hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync to the scratch array");
      }
      h.valid = true;
      h.digest = st.digest;
      h.plan = plan;
      h.generation = plan->generation;
      h.wl = wle;
      h.mode = dmode;
    }
  }

  psw_dev::AttnParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.o = o;
  p.pool = static_cast<const __bf16*>(pool->base);
  p.qo_indptr = reinterpret_cast<const int32_t*>(base + o_qo);
  p.kv_page_indptr = reinterpret_cast<const int32_t*>(base + o_kvp);
  p.kv_page_indices = reinterpret_cast<const int32_t*>(base + o_idx);
  p.kv_len = reinterpret_cast<const int32_t*>(base + o_len);
  p.items = reinterpret_cast<const int32_t*>(base + o_items);
  p.wg_items = p.items + ds.items.size();
  if (ds.num_partials > 0) {
    p.part_o = reinterpret_cast<float*>(base + o_part);
    p.part_ml = reinterpret_cast<float*>(base + o_ml);
  }
  p.ps.head = pool->page_size * pool->head_dim;
  p.ps.kv = pool->num_kv_heads * p.ps.head;
  p.ps.page = 2 * p.ps.kv;
  p.ps.layer = pool->num_pages * p.ps.page;
  int shift = 0;
  while ((int64_t(1) << shift) < pool->page_size) ++shift;
  p.ps.page_shift = shift;
  p.ps.page_size = static_cast<int32_t>(pool->page_size);
  p.layer_off = layer * p.ps.layer;
  p.num_qo_heads = st.num_qo_heads;
  p.num_kv_heads = st.num_kv_heads;
  int gs = 0;
  while ((1 << gs) < st.group) ++gs;
  p.group_shift = gs;
  p.window_left = -1;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.out_bf16 = o_dtype == 1;
  e = psw_dev::launch_decode(D, p, ds.num_wgs * st.num_kv_heads, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (ds.num_partials > 0) {
    psw_dev::MergeParams mp{};
    mp.part_o = p.part_o;
    mp.part_ml = p.part_ml;
    mp.o = o;
    mp.num_qo_heads = st.num_qo_heads;
    e = psw_dev::launch_merge_d512(o_dtype == 1, mp, ds.req_splits.data(), st.qo_indptr.data(),
                                   st.batch, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return PSW_OK;
}
