// C-ABI entry points that launch work, and the plan's device mirror.
//
// Every entry runs the host checks of psw_host.cpp first and returns before any
// HIP call when they fail (PR "feat(kernels): Rust wrapper for the hd256
// windowed paged prefill", Verification).  All uploads and launches go to the
// stream the plan was created on (PR "feat(gemma4): paged KV serving across both
// attention families", review thread: one construction stream keeps pool
// initialisation and KV writes ordered).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "psw_device.hpp"
#include "psw_host.hpp"

// Pinned host staging of one metadata upload.  A copy from pinned memory is
// asynchronous, so an entry never waits on the host for its uploads; a slot
// is refilled only once the event recorded behind its copy has completed.
struct psw_stage_slot {
  int32_t* host = nullptr;
  size_t cap = 0;  // bytes
  hipEvent_t ev = nullptr;
  bool busy = false;
};

struct psw_device_mirror {
  int device = -1;
  // metadata: qo_indptr[B+1] | kv_page_indptr[B+1] | kv_page_indices[nnz] | kv_len[B]
  int32_t* meta = nullptr;
  size_t meta_cap = 0;
  uint64_t meta_gen = 0;
  size_t off_kvp = 0, off_idx = 0, off_kvlen = 0;
  int32_t* pf_items = nullptr;
  size_t pf_cap = 0;
  uint64_t pf_gen = 0;
  int64_t pf_wl = -3;
  int32_t* dc_items = nullptr;
  size_t dc_cap = 0;
  uint64_t dc_gen = 0;
  int64_t dc_wl = -3;
  int32_t dc_mode = -1;
  int32_t* prep = nullptr;
  size_t prep_cap = 0;
  uint64_t prep_gen = 0;
  float* part = nullptr;
  size_t part_cap = 0;
  int32_t* err = nullptr;  // [4]: flag, page, position, spare
  std::vector<psw_stage_slot> slots;
  std::vector<int32_t*> retired;  // outgrown pinned buffers, freed with the mirror
};

namespace {

using psw::fail;

int hip_fail(hipError_t e, const char* what) {
  return fail(PSW_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define PSW_HIP(call)                                  \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #call);  \
  } while (0)

// Most uploads that may be in flight at once before an upload waits for the
// oldest (a serving loop has one or two: the previous step's and its own).
constexpr size_t kMaxStageSlots = 16;

// A staging slot of at least `bytes` whose previous copy has completed.
int acquire_slot(psw_device_mirror* m, size_t bytes, psw_stage_slot** out) {
  psw_stage_slot* pick = nullptr;
  for (psw_stage_slot& sl : m->slots) {
    if (sl.busy) {
      const hipError_t q = hipEventQuery(sl.ev);
      if (q == hipSuccess) sl.busy = false;
      else if (q != hipErrorNotReady) return hip_fail(q, "hipEventQuery");
    }
    if (!sl.busy && (!pick || sl.cap >= bytes)) pick = &sl;
  }
  if (!pick && m->slots.size() < kMaxStageSlots) {
    psw_stage_slot sl;
    PSW_HIP(hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming));
    m->slots.push_back(sl);
    pick = &m->slots.back();
  }
  if (!pick) {
    // every slot still in flight: the only wait, on the oldest upload
    pick = &m->slots.front();
    PSW_HIP(hipEventSynchronize(pick->ev));
    pick->busy = false;
  }
  if (pick->cap < bytes) {
    if (pick->host) m->retired.push_back(pick->host);  // its last copy has completed
    pick->host = nullptr;
    pick->cap = 0;
    const size_t want = bytes < 4096 ? 4096 : bytes + bytes / 2;
    PSW_HIP(hipHostMalloc(reinterpret_cast<void**>(&pick->host), want, hipHostMallocDefault));
    pick->cap = want;
  }
  *out = pick;
  return PSW_OK;
}

// Device buffer of at least `bytes`.  Growth is stream-ordered: the old
// buffer is released after the work already queued on the stream, the new one
// allocated in stream order, and the host never waits.
template <typename T>
int ensure(T** p, size_t* cap, size_t bytes, hipStream_t s) {
  if (bytes <= *cap && *p) return PSW_OK;
  if (*p) {
    PSW_HIP(hipFreeAsync(*p, s));
    *p = nullptr;
    *cap = 0;
  }
  const size_t want = bytes < 256 ? 256 : bytes;
  PSW_HIP(hipMallocAsync(reinterpret_cast<void**>(p), want, s));
  *cap = want;
  return PSW_OK;
}

int upload(psw_device_mirror* m, int32_t** dptr, size_t* cap, const std::vector<int32_t>& src,
           hipStream_t s) {
  const size_t bytes = (src.empty() ? 1 : src.size()) * sizeof(int32_t);
  int rc = ensure(dptr, cap, bytes, s);
  if (rc) return rc;
  psw_stage_slot* sl = nullptr;
  rc = acquire_slot(m, bytes, &sl);
  if (rc) return rc;
  if (src.empty()) sl->host[0] = 0;
  else std::memcpy(sl->host, src.data(), bytes);
  PSW_HIP(hipMemcpyAsync(*dptr, sl->host, bytes, hipMemcpyHostToDevice, s));
  PSW_HIP(hipEventRecord(sl->ev, s));
  sl->busy = true;
  return PSW_OK;
}

int ensure_mirror(psw_plan* plan) {
  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);
  int dev = -1;
  PSW_HIP(hipGetDevice(&dev));
  if (!plan->mirror) {
    psw_device_mirror* m = psw_mirror_new();
    m->device = dev;
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&m->err), 4 * sizeof(int32_t), s);
    if (e == hipSuccess) e = hipMemsetAsync(m->err, 0, 4 * sizeof(int32_t), s);
    if (e != hipSuccess) {
      psw_mirror_free(m, plan->stream);
      return hip_fail(e, "device error word");
    }
    plan->mirror = m;
  } else if (plan->mirror->device != dev) {
    return fail(PSW_E_PLAN, "the current device differs from the device the plan's mirror lives on");
  }
  psw_device_mirror* m = plan->mirror;
  if (m->meta_gen != plan->generation) {
    const psw::PlanState& st = plan->st;
    std::vector<int32_t> meta;
    meta.reserve(st.qo_indptr.size() * 2 + st.kv_page_indices.size() + st.kv_len.size());
    meta.insert(meta.end(), st.qo_indptr.begin(), st.qo_indptr.end());
    m->off_kvp = meta.size();
    meta.insert(meta.end(), st.kv_page_indptr.begin(), st.kv_page_indptr.end());
    m->off_idx = meta.size();
    meta.insert(meta.end(), st.kv_page_indices.begin(), st.kv_page_indices.end());
    m->off_kvlen = meta.size();
    meta.insert(meta.end(), st.kv_len.begin(), st.kv_len.end());
    int rc = upload(m, &m->meta, &m->meta_cap, meta, s);
    if (rc) return rc;
    m->meta_gen = plan->generation;
  }
  return PSW_OK;
}

psw_dev::PoolStrides strides_of(const psw_pool* pool) {
  psw_dev::PoolStrides ps;
  ps.head = pool->page_size * pool->head_dim;
  ps.kv = pool->num_kv_heads * ps.head;
  ps.page = 2 * ps.kv;
  ps.layer = pool->num_pages * ps.page;
  int shift = 0;
  while ((int64_t(1) << shift) < pool->page_size) ++shift;
  ps.page_shift = shift;
  ps.page_size = static_cast<int32_t>(pool->page_size);
  return ps;
}

int group_shift_of(int32_t group) {
  int s = 0;
  while ((1 << s) < group) ++s;
  return s;
}

int run_attention(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                  float sm_scale, int64_t window_left, void* o, int32_t o_dtype,
                  psw_stream_t stream, int head_dim) {
  psw::clear_error();
  int rc = psw::check_attention_call(plan, pool, layer, q, sm_scale, window_left, o, o_dtype,
                                     stream, head_dim);
  if (rc) return rc;
  const psw::PlanState& st = plan->st;
  if (st.page_size < 8)
    return fail(PSW_E_UNSUPPORTED, "the attention kernels need page_size >= 8");
  const int64_t wle = psw::effective_window(st, window_left);
  const bool decode = st.max_qo_len == 1;
  const int kv_tile = psw::kv_tile_for(head_dim);
  // the group-32 decode runs in the split mode of the attention kernel
  static_assert(psw::kDecodeKernelMaxGroup == psw_dev::kDecodeMaxGroup, "decode group bound");
  const int32_t dmode = psw::effective_decode_mode(st, plan->decode_mode);
  if (decode) {
    if (plan->decode.window_left != wle || plan->decode.mode != dmode)
      psw::build_decode_schedule(st, wle, dmode, &plan->decode);
  } else {
    if (plan->prefill.window_left != wle)
      psw::build_prefill_schedule(st, wle, kv_tile, &plan->prefill);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);
  rc = ensure_mirror(plan);
  if (rc) return rc;
  psw_device_mirror* m = plan->mirror;
  psw_dev::AttnParams p{};
  int n_items = 0;
  // the group-32 decode runs the split mode of the attention kernel, whose
  // every work item writes a partial
  const bool split_kernel = decode && st.group > psw_dev::kDecodeMaxGroup;
  if (decode) {
    if (m->dc_gen != plan->generation || m->dc_wl != wle || m->dc_mode != dmode) {
      rc = psw::check_decode_items(st, plan->decode, split_kernel);
      if (rc) return rc;
      // items, then the work-groups' item offsets
      std::vector<int32_t> table(plan->decode.items);
      table.insert(table.end(), plan->decode.wg_items.begin(), plan->decode.wg_items.end());
      rc = upload(m, &m->dc_items, &m->dc_cap, table, s);
      if (rc) return rc;
      m->dc_gen = plan->generation;
      m->dc_wl = wle;
      m->dc_mode = dmode;
    }
    p.items = m->dc_items;
    p.wg_items = m->dc_items + plan->decode.items.size();
    p.out_bf16 = o_dtype == 1;
    n_items = static_cast<int>(plan->decode.items.size() / 4);
    if (plan->decode.num_partials > 0) {
      const size_t part_floats =
          size_t(plan->decode.num_partials) * st.num_qo_heads * (size_t(head_dim) + 2);
      rc = ensure(&m->part, &m->part_cap, part_floats * sizeof(float), s);
      if (rc) return rc;
      p.part_o = m->part;
      p.part_ml = m->part + size_t(plan->decode.num_partials) * st.num_qo_heads * head_dim;
    }
  } else {
    if (m->pf_gen != plan->generation || m->pf_wl != wle) {
      rc = psw::check_prefill_items(st, plan->prefill);
      if (rc) return rc;
      rc = upload(m, &m->pf_items, &m->pf_cap, plan->prefill.items, s);
      if (rc) return rc;
      m->pf_gen = plan->generation;
      m->pf_wl = wle;
    }
    p.items = m->pf_items;
    n_items = static_cast<int>(plan->prefill.items.size() / 4);
  }
  p.q = static_cast<const __bf16*>(q);
  p.o = o;
  p.pool = static_cast<const __bf16*>(pool->base);
  p.qo_indptr = m->meta;
  p.kv_page_indptr = m->meta + m->off_kvp;
  p.kv_page_indices = m->meta + m->off_idx;
  p.kv_len = m->meta + m->off_kvlen;
  p.ps = strides_of(pool);
  p.layer_off = layer * p.ps.layer;
  p.num_qo_heads = st.num_qo_heads;
  p.num_kv_heads = st.num_kv_heads;
  p.group_shift = group_shift_of(st.group);
  p.window_left = static_cast<int32_t>(wle);
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  if ((split_kernel || (decode && plan->decode.num_partials > 0)) && !p.part_o)
    return fail(PSW_E_PLAN, "the schedule writes partials but no workspace backs them");
  hipError_t e;
  if (decode && !split_kernel)
    e = psw_dev::launch_decode(head_dim, p, plan->decode.num_wgs * st.num_kv_heads, s);
  else
    e = head_dim == 256 ? psw_dev::launch_attention_d256(decode, o_dtype == 1, p, n_items, s)
                        : psw_dev::launch_attention_d512(decode, o_dtype == 1, p, n_items, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (decode && plan->decode.num_partials > 0) {
    psw_dev::MergeParams mp{};
    mp.part_o = p.part_o;
    mp.part_ml = p.part_ml;
    mp.o = o;
    mp.num_qo_heads = st.num_qo_heads;
    const int32_t* rs = plan->decode.req_splits.data();
    e = head_dim == 256
            ? psw_dev::launch_merge_d256(o_dtype == 1, mp, rs, st.qo_indptr.data(), st.batch, s)
            : psw_dev::launch_merge_d512(o_dtype == 1, mp, rs, st.qo_indptr.data(), st.batch, s);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return PSW_OK;
}

int prepare_prep(psw_plan* plan, const psw_pool* pool, int64_t layer, const float* rope_cos,
                 const float* rope_sin, int64_t rope_positions, float eps,
                 psw_dev::PrepParams* p) {
  if (!plan->prep_built) {
    psw::build_prep_items(plan->st, &plan->prep_items);
    int rc = psw::check_prep_items(plan->st, plan->prep_items);
    if (rc) return rc;
    plan->prep_built = true;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);
  int rc = ensure_mirror(plan);
  if (rc) return rc;
  psw_device_mirror* m = plan->mirror;
  if (m->prep_gen != plan->generation) {
    rc = upload(m, &m->prep, &m->prep_cap, plan->prep_items, s);
    if (rc) return rc;
    m->prep_gen = plan->generation;
  }
  p->cos = rope_cos;
  p->sin = rope_sin;
  p->pool = static_cast<__bf16*>(pool->base);
  p->err = m->err;
  p->items = m->prep;
  p->ps = strides_of(pool);
  p->layer_off = layer * p->ps.layer;
  p->num_qo_heads = plan->st.num_qo_heads;
  p->num_kv_heads = plan->st.num_kv_heads;
  p->num_pages = static_cast<int32_t>(pool->num_pages);
  p->rope_positions = static_cast<int32_t>(rope_positions);
  p->eps = eps;
  return PSW_OK;
}

}  // namespace

psw_device_mirror* psw_mirror_new() { return new psw_device_mirror(); }

void psw_mirror_free(psw_device_mirror* m, psw_stream_t stream) {
  if (!m) return;
  // the plan's work is ordered on its stream: once it has drained, no kernel
  // or copy uses the buffers below
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipStreamSynchronize(s);
  for (void* p : {(void*)m->meta, (void*)m->pf_items, (void*)m->dc_items,
                  (void*)m->prep, (void*)m->part, (void*)m->err})
    if (p) (void)hipFreeAsync(p, s);
  for (psw_stage_slot& sl : m->slots) {
    if (sl.host) (void)hipHostFree(sl.host);
    if (sl.ev) (void)hipEventDestroy(sl.ev);
  }
  for (int32_t* h : m->retired) (void)hipHostFree(h);
  delete m;
}

extern "C" {

int paged_prefill_window_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                               float sm_scale, int64_t window_left, void* o, int32_t o_dtype,
                               psw_stream_t stream) {
  return run_attention(plan, pool, layer, q, sm_scale, window_left, o, o_dtype, stream, 256);
}

int paged_prefill_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                        float sm_scale, void* o, int32_t o_dtype, psw_stream_t stream) {
  return run_attention(plan, pool, layer, q, sm_scale, -1, o, o_dtype, stream, 512);
}

int paged_decode_window_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                              float sm_scale, int64_t window_left, void* o, int32_t o_dtype,
                              psw_stream_t stream) {
  psw::clear_error();
  if (plan && plan->st.max_qo_len != 1)
    return fail(PSW_E_SHAPE, "decode entries take one query token per request");
  return run_attention(plan, pool, layer, q, sm_scale, window_left, o, o_dtype, stream, 256);
}

int paged_decode_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                       float sm_scale, void* o, int32_t o_dtype, psw_stream_t stream) {
  psw::clear_error();
  if (plan && plan->st.max_qo_len != 1)
    return fail(PSW_E_SHAPE, "decode entries take one query token per request");
  return run_attention(plan, pool, layer, q, sm_scale, -1, o, o_dtype, stream, 512);
}

int qkv_norm_rope_paged_prefill_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer,
                                      const void* q_in, const void* k_in, const void* v_in,
                                      const void* q_norm_w, const void* k_norm_w,
                                      const float* rope_cos, const float* rope_sin,
                                      int64_t rope_positions, int64_t rope_cos_numel,
                                      int64_t rope_sin_numel, float eps, void* q_out,
                                      psw_stream_t stream) {
  psw::clear_error();
  int rc = psw::check_prep_call(plan, pool, layer, 256, rope_cos, rope_sin, rope_positions,
                                rope_cos_numel, rope_sin_numel, eps, stream);
  if (rc) return rc;
  if (!q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !q_out)
    return fail(PSW_E_NULL, "a prep input/output pointer is NULL");
  psw_dev::PrepParams p{};
  rc = prepare_prep(plan, pool, layer, rope_cos, rope_sin, rope_positions, eps, &p);
  if (rc) return rc;
  p.q_in = static_cast<const __bf16*>(q_in);
  p.k_in = static_cast<const __bf16*>(k_in);
  p.v_in = static_cast<const __bf16*>(v_in);
  p.q_w = static_cast<const __bf16*>(q_norm_w);
  p.k_w = static_cast<const __bf16*>(k_norm_w);
  p.q_out = static_cast<__bf16*>(q_out);
  const int n = static_cast<int>(plan->prep_items.size() / psw_dev::kPrepItemInts);
  hipError_t e = psw_dev::launch_prep_hd256(p, n, reinterpret_cast<hipStream_t>(plan->stream));
  if (e != hipSuccess) return hip_fail(e, "prep launch");
  return PSW_OK;
}

int k_v_norm_rope_paged_prefill_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer,
                                      const void* k_in, const void* k_norm_w,
                                      const float* rope_cos, const float* rope_sin,
                                      int64_t rope_positions, int64_t rope_cos_numel,
                                      int64_t rope_sin_numel, float eps, psw_stream_t stream) {
  psw::clear_error();
  int rc = psw::check_prep_call(plan, pool, layer, 512, rope_cos, rope_sin, rope_positions,
                                rope_cos_numel, rope_sin_numel, eps, stream);
  if (rc) return rc;
  if (!k_in || !k_norm_w) return fail(PSW_E_NULL, "k_in or k_norm_w is NULL");
  psw_dev::PrepParams p{};
  rc = prepare_prep(plan, pool, layer, rope_cos, rope_sin, rope_positions, eps, &p);
  if (rc) return rc;
  p.k_in = static_cast<const __bf16*>(k_in);
  p.k_w = static_cast<const __bf16*>(k_norm_w);
  const int n = static_cast<int>(plan->prep_items.size() / psw_dev::kPrepItemInts);
  hipError_t e = psw_dev::launch_prep_hd512(p, n, reinterpret_cast<hipStream_t>(plan->stream));
  if (e != hipSuccess) return hip_fail(e, "prep launch");
  return PSW_OK;
}

int q_norm_rope_prefill_hd512(psw_plan* plan, const void* q_in, const void* q_norm_w,
                              const float* rope_cos, const float* rope_sin, int64_t rope_positions,
                              int64_t rope_cos_numel, int64_t rope_sin_numel, float eps,
                              void* q_out, psw_stream_t stream) {
  psw::clear_error();
  int rc = psw::check_q_prep_call(plan, 512, q_in, q_norm_w, rope_cos, rope_sin, rope_positions,
                                  rope_cos_numel, rope_sin_numel, eps, q_out, stream);
  if (rc) return rc;
  if (!plan->prep_built) {
    psw::build_prep_items(plan->st, &plan->prep_items);
    rc = psw::check_prep_items(plan->st, plan->prep_items);
    if (rc) return rc;
    plan->prep_built = true;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);
  rc = ensure_mirror(plan);
  if (rc) return rc;
  psw_device_mirror* m = plan->mirror;
  if (m->prep_gen != plan->generation) {
    rc = upload(m, &m->prep, &m->prep_cap, plan->prep_items, s);
    if (rc) return rc;
    m->prep_gen = plan->generation;
  }
  psw_dev::PrepParams p{};
  p.cos = rope_cos;
  p.sin = rope_sin;
  p.err = m->err;
  p.items = m->prep;
  p.num_qo_heads = plan->st.num_qo_heads;
  p.num_kv_heads = plan->st.num_kv_heads;
  p.rope_positions = static_cast<int32_t>(rope_positions);
  p.eps = eps;
  p.q_in = static_cast<const __bf16*>(q_in);
  p.q_w = static_cast<const __bf16*>(q_norm_w);
  p.q_out = static_cast<__bf16*>(q_out);
  const int n = static_cast<int>(plan->prep_items.size() / psw_dev::kPrepItemInts);
  hipError_t e = psw_dev::launch_prep_q_hd512(p, n, s);
  if (e != hipSuccess) return hip_fail(e, "prep launch");
  return PSW_OK;
}

int psw_rope_tables(float* cos_out, float* sin_out, int64_t positions, int64_t head_dim,
                    double theta, psw_stream_t stream) {
  psw::clear_error();
  if (!cos_out || !sin_out) return fail(PSW_E_NULL, "cos/sin output is NULL");
  if (positions < 1 || head_dim < 2 || head_dim % 2 != 0)
    return fail(PSW_E_SHAPE, "positions must be >= 1 and head_dim even and >= 2");
  if (!psw::fits_i32(positions) || !psw::fits_i32(head_dim))
    return fail(PSW_E_OVERFLOW, "positions or head_dim past INT32_MAX");
  int64_t n;
  if (!psw::checked_mul(positions, head_dim / 2, &n) || n > (int64_t(1) << 40))
    return fail(PSW_E_OVERFLOW, "table too large");
  if (!std::isfinite(theta) || !(theta > 0.0)) return fail(PSW_E_SCALE, "theta must be finite and > 0");
  hipError_t e = psw_dev::launch_rope_tables(cos_out, sin_out, positions, head_dim / 2, theta,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return PSW_OK;
}

int psw_plan_device_errors(psw_plan* plan) {
  psw::clear_error();
  if (!plan) return fail(PSW_E_NULL, "plan is NULL");
  if (!plan->mirror) return PSW_OK;
  psw_device_mirror* m = plan->mirror;
  hipStream_t s = reinterpret_cast<hipStream_t>(plan->stream);
  PSW_HIP(hipStreamSynchronize(s));
  int32_t w[4] = {0, 0, 0, 0};
  PSW_HIP(hipMemcpy(w, m->err, sizeof(w), hipMemcpyDeviceToHost));
  if (w[0] == 0) return PSW_OK;
  static const int32_t zeros[4] = {0, 0, 0, 0};
  PSW_HIP(hipMemcpy(m->err, zeros, sizeof(zeros), hipMemcpyHostToDevice));
  return fail(PSW_E_RANGE, "a prep kernel skipped an item: page " + std::to_string(w[1]) +
                               ", last position " + std::to_string(w[2]));
}

}  // extern "C"
