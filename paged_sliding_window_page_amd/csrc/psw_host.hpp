// Internal host-side declarations: validation, the plan and its schedules.
// This header and psw_host.cpp use no HIP API, so every host check can be
// exercised on a machine without a GPU.  Sources:
//   [P1] PR "feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
//        Description, Verification.
//   [P2] issue "gemma4: serving prep needs pool-write forms -- hd256 QKV in one
//        pass, hd512 V alongside K", Proposed Plan.
//   [P3] PR "feat(gemma4): paged KV serving across both attention families",
//        Description and review thread.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "psw.h"

namespace psw {

// ----------------------------------------------------------------- errors --

// Records a thread-local message and returns `code` (for `return fail(...)`).
int fail(int code, const std::string& msg);
void clear_error();

// Checked narrowing to int32 ([P1] Description: every 64-bit to 32-bit
// conversion is checked; an overflowing length is an error, never a wrapped
// value that happens to look legal).
bool fits_i32(int64_t v);
// a * b without int64 overflow; false on overflow or negative operands.
bool checked_mul(int64_t a, int64_t b, int64_t* out);

// ------------------------------------------------------------------- pool --

int check_pool(const psw_pool* pool, bool need_base);

// ------------------------------------------------------------------- plan --

// Tiling decisions, shared by the plan (which records them) and the device
// code (which was compiled for them).
constexpr int kPrefillRows = 256;          // query rows (token x head) per work-group (head_dim 256)
constexpr int kPrefillRows512 = 128;       // the same at head_dim 512 (four waves of 32 rows)
constexpr int kKvTile256 = 64;             // keys per prefill tile at head_dim 256
constexpr int kKvTile512 = 32;             // keys per prefill tile at head_dim 512
// Decode pieces start and end at multiples of this key index: one decode
// tile, so no tile is read by two pieces and shares come out equal to within
// one tile (64 measured ~2% slower on the global-family batch).
constexpr int kDecodeSplitUnit = 32;
// Waves the split decode spreads over the GPU: four per CU (256 CUs).  The
// kernel could keep eight per CU resident, but the equal-share launch streams
// K/V faster with four (measured: global-family batch 116 -> 104 us).
constexpr int kDecodeResidentWaves = 1024;
// Automatic decode form (measured on MI355X, split vs direct over batch x KV
// length): the direct form wins while its longest work-group loop stays
// shorter than the split form's extra merge launch -- up to about 160 keys at
// head_dim 256 and 256 at head_dim 512 -- or, once the direct grid alone
// fills the 256 CUs, up to 1024 keys.
constexpr int kDecodeDirectKeys256 = 160;
constexpr int kDecodeDirectKeys512 = 256;
constexpr int kDecodeDirectKeysFull = 1024;
constexpr int kDecodeFullGrid = 256;
constexpr int kDecodeKernelMaxGroup = 16;  // widest GQA group of the decode kernel
constexpr int kMaxGroup = 32;

int derive_tile_q(int64_t group, int64_t head_dim, int32_t* tile_q);
inline int kv_tile_for(int64_t head_dim) { return head_dim == 512 ? kKvTile512 : kKvTile256; }

struct PlanState {
  int32_t batch = 0;
  int32_t num_qo_heads = 0, num_kv_heads = 0, head_dim = 0, page_size = 0, num_pages = 0;
  int32_t group = 0;
  int32_t tile_q = 0;
  bool tile_overridden = false;
  int32_t total_qo = 0, total_pages = 0;
  int32_t max_qo_len = 0, max_kv_len = 0;
  int32_t max_page_id = -1, max_last_page_len = 0;
  std::vector<int32_t> qo_indptr, kv_page_indptr, kv_page_indices, last_page_len, kv_len;
  bool any_ring = false;  // some request's pages wrap (resident window)
  uint64_t digest = 0;

  int32_t n_pages(int32_t b) const { return kv_page_indptr[b + 1] - kv_page_indptr[b]; }
  bool wraps(int32_t b) const { return int64_t(kv_len[b]) > int64_t(n_pages(b)) * page_size; }
  // page id holding absolute position p of request b (ring or not)
  int32_t page_of(int32_t b, int64_t p) const {
    return kv_page_indices[kv_page_indptr[b] + (p / page_size) % n_pages(b)];
  }
};

// Builds and validates a complete PlanState from a description; *out is only
// written on success.
int build_state(const psw_plan_desc* d, PlanState* out);

// Attention work item: quads (request, first query token, first key, last key
// inclusive).  Prefill: one item per (request, query tile), heaviest first.
struct PrefillSchedule {
  int64_t window_left = -2;   // key the schedule was built for (-2 = none)
  int32_t kv_tile = 0;
  int32_t tile_q = 0;
  std::vector<int32_t> items;  // quads
  int64_t total_tiles = 0;     // sum over items of KV tiles visited
};
void build_prefill_schedule(const PlanState& st, int64_t window_left, int32_t kv_tile,
                            PrefillSchedule* out);

// Decode (qo_len == 1 everywhere) split-KV schedule.  Items are quads
// (request, partial slot, first key, last key), longest first; the slots of a
// request are consecutive, in key order.
struct DecodeSchedule {
  int64_t window_left = -2;
  int32_t mode = -1;                 // PSW_DECODE_* the schedule was built for
  bool direct = false;               // every item a whole request: no partials, no merge launch
  // quads (request, partial slot or -1 for a whole request written by the
  // decode kernel, first key, last key)
  std::vector<int32_t> items;
  std::vector<int32_t> wg_items;     // decode kernel: work-group g runs items [wg_items[g], wg_items[g+1])
  std::vector<int32_t> req_splits;   // pairs (first partial slot, number of pieces) per request
  int32_t num_partials = 0;
  int32_t num_wgs = 0;               // work-groups per KV head of the decode launch
};
void build_decode_schedule(const PlanState& st, int64_t window_left, int32_t mode,
                           DecodeSchedule* out);
// The decode form a plan's mode resolves to: wider groups than the decode
// kernel's run through the split mode of the attention kernel.
int32_t effective_decode_mode(const PlanState& st, int32_t mode);

// Prep work items: up to 16 consecutive positions of one request inside one
// page, as (request, first global token, tokens, page id, first slot, first
// position).
void build_prep_items(const PlanState& st, std::vector<int32_t>* out);

// Consistency of a schedule before its first launch: the kernels trust their
// items (request, keys, slots, pages), so every field is checked here against
// the plan.  PSW_OK, or PSW_E_PLAN with a message naming the item.
int check_prefill_items(const PlanState& st, const PrefillSchedule& ps);
// split_kernel: the schedule feeds the split mode of the attention kernel,
// where every item writes a partial slot.
int check_decode_items(const PlanState& st, const DecodeSchedule& ds, bool split_kernel);
int check_prep_items(const PlanState& st, const std::vector<int32_t>& items);

// Window normalisation: -1 when the window cannot exclude any key.
int64_t effective_window(const PlanState& st, int64_t window_left);

// Checks shared by the attention entries before any HIP call.
int check_attention_call(const psw_plan* plan, const psw_pool* pool, int64_t layer,
                         const void* q, float sm_scale, int64_t window_left, const void* o,
                         int32_t o_dtype, psw_stream_t stream, int64_t want_head_dim);

// Checks shared by the prep entries before any HIP call.
int check_prep_call(const psw_plan* plan, const psw_pool* pool, int64_t layer,
                    int64_t want_head_dim, const float* rope_cos, const float* rope_sin,
                    int64_t rope_positions, int64_t rope_cos_numel, int64_t rope_sin_numel,
                    float eps, psw_stream_t stream);

// Checks of the query-only prep entry (no pool) before any HIP call.
int check_q_prep_call(const psw_plan* plan, int64_t want_head_dim, const void* q_in,
                      const void* q_norm_w, const float* rope_cos, const float* rope_sin,
                      int64_t rope_positions, int64_t rope_cos_numel, int64_t rope_sin_numel,
                      float eps, const void* q_out, psw_stream_t stream);

}  // namespace psw

// Device mirror (defined in the HIP translation unit; opaque here).
struct psw_device_mirror;
psw_device_mirror* psw_mirror_new();
// Releases the mirror after the work queued on the plan's stream.
void psw_mirror_free(psw_device_mirror* m, psw_stream_t stream);

struct psw_plan {
  psw_stream_t stream = nullptr;
  psw::PlanState st;
  uint64_t generation = 0;
  psw::PrefillSchedule prefill;
  psw::DecodeSchedule decode;
  int32_t decode_mode = PSW_DECODE_AUTO;
  std::vector<int32_t> prep_items;
  bool prep_built = false;
  psw_device_mirror* mirror = nullptr;  // created by the first launch
};
