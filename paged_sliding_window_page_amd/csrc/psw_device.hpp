// Device-side types, pool addressing and launcher declarations shared by the
// HIP translation units of the library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psw_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pool addressing (element strides, 64-bit).  Per layer and page there is a K
// block [kv_head][slot][dim] followed by a V block stored dim-major,
// [kv_head][dim][slot]: V is the operand contracted over keys, so keeping keys
// contiguous lets the attention kernels fetch it with the same 16-byte loads as
// K, without a transpose anywhere on the read path.
struct PoolStrides {
  int64_t layer;      // num_pages * 2 * H_kv * P * D
  int64_t page;       // 2 * H_kv * P * D
  int64_t kv;         // H_kv * P * D   (K block -> V block)
  int64_t head;       // P * D
  int32_t page_shift; // log2(P)
  int32_t page_size;
};

// Work item of the attention kernels: (request, first query token, first key,
// last key inclusive).  In split-KV mode the item index is the partial slot.
struct AttnParams {
  const __bf16* q;
  void* o;
  float* part_o;       // split mode: [n_partials][H_q][D] unnormalised
  float* part_ml;      // split mode: [n_partials][H_q][2] (running max in log2 units, sum)
  const __bf16* pool;
  const int32_t* qo_indptr;
  const int32_t* kv_page_indptr;
  const int32_t* kv_page_indices;
  const int32_t* kv_len;
  const int32_t* items;
  const int32_t* wg_items;  // decode kernel: items of work-group g are [wg_items[g], wg_items[g+1])
  PoolStrides ps;
  int64_t layer_off;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group_shift;  // log2(H_q / H_kv)
  int32_t window_left;  // -1: none
  float scale_log2;     // sm_scale * log2(e)
  int32_t out_bf16;     // decode kernel: O element type of whole-request items (else fp32)
};

// Page list index of an absolute page index a = key / page_size of one
// request.  The list holds n pages; when kv_len exceeds them it is a ring that
// keeps the last n * page_size positions, page a at index a % n.  Indices are
// first clamped into the resident span [lo, hi] (loads past either end read
// some resident page; the caller masks those keys), then mapped without a
// division: base is the multiple of n at or below hi.
struct PageRing {
  int n, lo, hi, base;
  __device__ __forceinline__ int operator()(int a) const {
    const int c = min(max(a, lo), hi);
    return c - base + (c < base ? n : 0);
  }
};
__device__ __forceinline__ PageRing page_ring(int n_pages, int kv_len, int page_shift) {
  PageRing r;
  r.n = n_pages;
  r.hi = (kv_len - 1) >> page_shift;
  r.lo = max(0, kv_len - (n_pages << page_shift)) >> page_shift;
  r.base = (r.hi / n_pages) * n_pages;
  return r;
}

// Split-KV merge launch: up to kMergeReqsPerLaunch requests, whose split lists
// travel in the launch's own arguments (a work-group reads them with its first
// loads instead of a dependent load from memory).
constexpr int kMergeReqsPerLaunch = 256;
struct MergeParams {
  const float* part_o;
  const float* part_ml;
  void* o;
  int32_t num_qo_heads;
  // per request of the launch: first partial slot, number of pieces (0: the
  // decode kernel wrote its O), output row
  int32_t req[3 * kMergeReqsPerLaunch];
};

// Prep work item: (request, first global token, tokens (<= 16), page id,
// first slot, first position).  Every item lies inside one page.
struct PrepParams {
  const __bf16* q_in;
  const __bf16* k_in;
  const __bf16* v_in;
  const __bf16* q_w;
  const __bf16* k_w;
  const float* cos;
  const float* sin;
  __bf16* q_out;
  __bf16* pool;
  int32_t* err;
  const int32_t* items;
  PoolStrides ps;
  int64_t layer_off;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t num_pages;
  int32_t rope_positions;
  float eps;
  int32_t n_items;  // set by the launchers that pad the grid
};

constexpr int kPrepItemInts = 6;
constexpr int kPrepMaxTokens = 16;

// Launchers (return the hipError_t of the launch).
hipError_t launch_attention_d256(bool split, bool out_bf16, const AttnParams& p, int n_items,
                                 hipStream_t s);
hipError_t launch_attention_d512(bool split, bool out_bf16, const AttnParams& p, int n_items,
                                 hipStream_t s);
// head_dim-512 prefill: 128 query rows per work-group, all 512 dims per wave
hipError_t launch_prefill512(bool out_bf16, const AttnParams& p, int n_items, hipStream_t s);
// One-token decode kernel: n_wgs = work-groups x KV heads, each work-group
// running its items (whole requests write O, pieces write the same partials
// as the split attention kernels).  Needs H_q / H_kv <= kDecodeMaxGroup.
constexpr int kDecodeMaxGroup = 16;
hipError_t launch_decode(int head_dim, const AttnParams& p, int n_wgs, hipStream_t s);
// Merges the partials of every request of a batch that has pieces: p holds
// the pointers and head count; req_splits (pairs: first slot, count) and
// qo_indptr are the batch's host arrays, sent kMergeReqsPerLaunch requests per
// launch (launches with no pieces to merge are skipped).
hipError_t launch_merge_d256(bool out_bf16, MergeParams p, const int32_t* req_splits,
                             const int32_t* qo_indptr, int batch, hipStream_t s);
hipError_t launch_merge_d512(bool out_bf16, MergeParams p, const int32_t* req_splits,
                             const int32_t* qo_indptr, int batch, hipStream_t s);
hipError_t launch_prep_hd256(const PrepParams& p, int n_items, hipStream_t s);
hipError_t launch_prep_hd512(const PrepParams& p, int n_items, hipStream_t s);
hipError_t launch_prep_q_hd512(const PrepParams& p, int n_items, hipStream_t s);
hipError_t launch_rope_tables(float* c, float* s, int64_t positions, int64_t half, double theta,
                              hipStream_t st);

}  // namespace psw_dev
