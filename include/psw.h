/*
 * psw.h -- C ABI of the MI355X (gfx950) paged sliding-window attention library.
 *
 * Operations (all on one GPU, all on one ordered HIP stream):
 *
 *   paged_prefill_window_hd256          attention read through a page table,
 *                                       head_dim 256, GQA, sliding window
 *   paged_prefill_hd512                 the same at head_dim 512, full causal
 *   qkv_norm_rope_paged_prefill_hd256   fused prep: Q norm+RoPE to a contiguous
 *                                       buffer, K norm+RoPE and V weightless norm
 *                                       scattered into the layer's pool pages
 *   k_v_norm_rope_paged_prefill_hd512   fused prep: K norm+RoPE, and V = the raw K
 *                                       normalised without weight (K's inv_rms)
 *   q_norm_rope_prefill_hd512           the global family's Q norm+RoPE to a
 *                                       contiguous buffer
 *
 * Sources (the pages this library implements):
 *   [P1] PR "feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
 *        Description and Verification.
 *   [P2] issue "gemma4: serving prep needs pool-write forms -- hd256 QKV in one
 *        pass, hd512 V alongside K", Description, Proposed Plan, Acceptance
 *        Criteria.
 *   [P3] PR "feat(gemma4): paged KV serving across both attention families",
 *        Description and the review thread (stream ordering, commit after
 *        success).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Return value: PSW_OK (0) or a negative psw_status.  On any failure nothing
 * has been launched and no device memory has been written; psw_last_error()
 * returns a thread-local message naming the offending argument.  Every check
 * runs on the host before any launch ([P1] Verification: inconsistent layouts,
 * bad layer indices, page metadata outside the pool, non-finite scales, i32
 * overflow and a zero KV-head count are all errors raised before launching).
 *
 * Pointers: "device" pointers are HIP device allocations owned by the caller
 * (for example torch tensors); "host" pointers are read during the call only.
 * The library never frees or retains caller memory.
 *
 * Pool layout (a whole-page, layer-indexed pool per KV family, bf16):
 *     K block: pool[layer][page][0][kv_head][slot][dim]
 *     V block: pool[layer][page][1][kv_head][dim][slot]   (dim-major)
 * i.e. numel == num_layers * num_pages * 2 * num_kv_heads * page_size * head_dim
 * exactly; device offsets are 64-bit, so pools larger than 2 GiB are fine.
 *
 * Page table: CSR.  Request b owns kv_page_indices[kv_page_indptr[b] ..
 * kv_page_indptr[b+1]) (at least one page) and its KV length is
 * (n_pages - 1) * page_size + kv_last_page_len[b].  Its qo_len =
 * qo_indptr[b+1] - qo_indptr[b] >= 1 queries are the last qo_len tokens of the
 * KV: token t sits at position start_pos + t with start_pos = kv_len - qo_len
 * ([P2] Proposed Plan: a token's cache slot is its absolute position).
 *
 * Ordering: a plan records the stream it was created with; every entry point
 * rejects any other stream with PSW_E_PLAN, which keeps pool setup, prep and
 * attention in order without events ([P3] review thread: a fresh
 * stream on the same device races earlier KV writes).
 */
#ifndef PSW_H
#define PSW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without including HIP headers (identical type). */
typedef struct ihipStream_t* psw_stream_t;

typedef enum {
  PSW_OK = 0,
  PSW_E_NULL = -1,      /* a required pointer is NULL                              */
  PSW_E_SHAPE = -2,     /* malformed metadata: indptr not monotone, qo_len < 1,
                           kv_len < qo_len, head_dim / page_size / batch invalid  */
  PSW_E_RANGE = -3,     /* page id outside the pool, last_page_len outside
                           [1, page_size], layer outside the pool, position past
                           the RoPE table, window_left < -1, pages not covering   */
  PSW_E_OVERFLOW = -4,  /* a length or total past INT32_MAX, or a size product
                           that overflows int64                                   */
  PSW_E_HEADS = -5,     /* zero KV heads, or query heads not a multiple of them    */
  PSW_E_SCALE = -6,     /* non-finite sm_scale, or eps not finite and positive     */
  PSW_E_PLAN = -7,      /* plan disagrees with the pool, the entry, its compiled
                           tile, or the stream it was created on                  */
  PSW_E_HIP = -8,       /* a HIP runtime call failed (message has the HIP error)   */
  PSW_E_UNSUPPORTED = -9 /* a geometry the library has no kernel for              */
} psw_status;

/* Thread-local description of the last failure on this thread ("" if none). */
const char* psw_last_error(void);

/* Library version as a static string. */
const char* psw_version(void);

/* Diagnostic, off the hot path: the shader clock in MHz while every CU issues
 * bf16 MFMAs (eight waves per CU of back-to-back v_mfma_f32_32x32x16_bf16, the
 * prefill kernels' occupancy), from the shader-clock and constant-rate
 * counters of each work-group.  The MFMA peak scales with this clock, so a
 * benchmark can report its fraction of the clock-adjusted peak next to the
 * nominal one.  Runs two short launches on `stream` (~1 ms each), allocates
 * and frees a small device buffer, and waits for the stream.  PSW_E_NULL for
 * a NULL `mhz`, PSW_E_HIP when the device or a launch fails. */
int psw_measure_mfma_clock(psw_stream_t stream, double* mhz);

/* ---------------------------------------------------------------- pool ---- */

/* A caller-owned bf16 pool in the layout above.  Geometry is re-derived with
 * overflow-checked multiplies and must match numel exactly (whole pages); a
 * page (its K and V blocks) must stay under 4 GiB (PSW_E_UNSUPPORTED). */
typedef struct {
  void* base;            /* device, bf16, numel elements                        */
  int64_t numel;
  int64_t num_layers;
  int64_t num_pages;
  int64_t page_size;     /* power of two, 1 .. 1024                             */
  int64_t num_kv_heads;
  int64_t head_dim;
} psw_pool;

/* Host-only check of a pool descriptor (one overflow-checked geometry check
 * used by the prep and attention entries alike, [P1] Description).  base may
 * be NULL here; entry points additionally require it non-NULL. */
int psw_check_pool(const psw_pool* pool);

/* ---------------------------------------------------------------- plan ---- */

/* Host description of one batch.  All arrays are HOST memory, int32, copied by
 * psw_plan_create / psw_plan_update. */
typedef struct {
  int64_t batch;                    /* >= 1                                      */
  const int32_t* qo_indptr;         /* [batch+1], [0] = 0, strictly increasing   */
  const int32_t* kv_page_indptr;    /* [batch+1], [0] = 0, strictly increasing   */
  const int32_t* kv_page_indices;   /* [kv_page_indptr[batch]]                   */
  const int32_t* kv_last_page_len;  /* [batch], each in [1, page_size]           */
  int64_t num_qo_heads;
  int64_t num_kv_heads;             /* >= 1; num_qo_heads % num_kv_heads == 0    */
  int64_t head_dim;
  int64_t page_size;
  int64_t num_pages;                /* pool size the page ids are checked against */
  int64_t tile_q_override;          /* 0: derive tile_q; else the plan records
                                       this value and prefill entries whose
                                       compiled tile differs reject the plan     */
  const int32_t* kv_len;            /* optional [batch]: absolute KV lengths, for
                                       resident windows (below); NULL: each is
                                       (n_pages - 1) * page_size + last_page_len */
} psw_plan_desc;

/* Resident windows (a ring of pages per request).  With kv_len given, a
 * request whose kv_len exceeds n_pages * page_size keeps only its last
 * R = n_pages * page_size positions: position p lives in page
 * kv_page_indices[kv_page_indptr[b] + (p / page_size) % n_pages], slot
 * p % page_size: once the ring has wrapped, a position and its cache slot
 * differ ([P2] Proposed Plan: callers past the window need a slot map).
 * Positions, masks and RoPE stay absolute.  kv_last_page_len must then be
 * (kv_len - 1) % page_size + 1, and a request that does not wrap must have
 * exactly its derived kv_len.  Attention rejects (PSW_E_RANGE) a wrapped
 * request whose ring could miss a key its queries see: no window, or
 * R < window_left + qo_len; the prep rejects a step longer than its ring. */

/* Opaque plan: validated host copy of the metadata, the recorded bounds
 * (max page id, max last-page length), the tile decision and work lists, and a
 * device mirror uploaded lazily, on the plan's stream, by the first launch that
 * needs it.  ([P1] Description: the bounds are taken from the host metadata,
 * and the query/KV head relation is validated before any division uses it.) */
typedef struct psw_plan psw_plan;

/* Creates a plan bound to `stream`.  Pure host work: no HIP call is made here,
 * so every reject can be exercised on a host without a GPU.  On failure *out is
 * left untouched. */
int psw_plan_create(const psw_plan_desc* desc, psw_stream_t stream, psw_plan** out);

/* Replaces the plan's batch in place.  All or nothing: the new description is
 * validated and the new state built completely before it is committed; on any
 * failure the plan is unchanged ([P1] Description: bounds are committed only
 * after an in-place update fully succeeds).  Head count, head_dim and
 * page_size may change; the stream may not. */
int psw_plan_update(psw_plan* plan, const psw_plan_desc* desc);

/* Frees the plan and its device mirror (synchronises the plan's stream first
 * if a mirror exists).  NULL is a no-op. */
void psw_plan_destroy(psw_plan* plan);

/* Read-only view of what a plan recorded. */
typedef struct {
  int64_t batch;
  int64_t total_qo;          /* sum of qo_len                                    */
  int64_t total_pages;       /* kv_page_indptr[batch]                            */
  int64_t max_qo_len;
  int64_t max_kv_len;
  int64_t max_page_id;       /* recorded bound, checked against the pool         */
  int64_t max_last_page_len; /* recorded bound, checked against page_size        */
  int64_t num_qo_heads, num_kv_heads, head_dim, page_size, num_pages;
  int64_t group;             /* num_qo_heads / num_kv_heads                      */
  int64_t tile_q;            /* query tokens per prefill work-group              */
  uint64_t generation;       /* bumped by every successful update                */
  uint64_t digest;           /* FNV-1a over the recorded metadata                */
} psw_plan_info;

int psw_plan_get_info(const psw_plan* plan, psw_plan_info* info);

/* Tile-size query ([P1] Description: a plan tiled differently from what the
 * kernel derives for itself is refused rather than misread).  Query tokens per prefill
 * work-group for a GQA group and head_dim: 256 / group at head_dim 256 and
 * 128 / group at head_dim 512 (query rows are tokens x the group's heads);
 * positivity is checked in the i32 domain. */
int psw_prefill_tile_q(int64_t group, int64_t head_dim, int32_t* tile_q);

/* ----------------------------------------------------------- attention ---- */

/* Windowed paged prefill at head_dim 256 ([P1] Description).  Attention only:
 * reads K/V of `layer` through the plan's page table, never writes the pool.
 *   q:   device bf16 [total_qo][num_qo_heads][256], contiguous
 *   o:   device [total_qo][num_qo_heads][256], fp32 (o_dtype 0) or bf16 (1)
 *   sm_scale:    multiplies q.k before the softmax; must be finite (1.0 for the
 *                unscaled attention the model runs)
 *   window_left: key j is visible to the query at position p iff
 *                0 <= p - j <= window_left (inclusive distance); -1 = no window
 * qo_len == 1 for every request selects the decode kernels, otherwise
 * the MFMA prefill kernel runs ([P3] Description: the serving loop's decode
 * step is a call of this entry with one query token per request). */
int paged_prefill_window_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer,
                               const void* q, float sm_scale, int64_t window_left,
                               void* o, int32_t o_dtype, psw_stream_t stream);

/* Full causal paged prefill at head_dim 512 (the global family: 16 query heads
 * over 1 KV head in the serving geometry), same contract without a window. */
int paged_prefill_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer,
                        const void* q, float sm_scale, void* o, int32_t o_dtype,
                        psw_stream_t stream);

/* --------------------------------------------------------------- decode ---- */

/* Decode is the prefill contract at qo_len 1 ([P3] Description: one-token
 * decode is served by the prefill entry, and a dedicated form is left to
 * measurement).
 * The prefill entries take it as well; these two require qo_len == 1 for
 * every request (PSW_E_SHAPE otherwise) and are otherwise identical to
 * paged_prefill_window_hd256 / paged_prefill_hd512.
 * Two forms, chosen per call by the plan's decode mode:
 *   PSW_DECODE_SPLIT   the batch's keys (32-key units) laid end to end and
 *                      cut into equal shares, one per work-group (at most
 *                      four waves' worth per CU, at least one per request, at
 *                      most one per unit); a request inside one share is
 *                      written directly, the pieces of a request cut between
 *                      shares write fp32 partials to the plan's workspace and
 *                      a merge launch combines them;
 *   PSW_DECODE_DIRECT  one work-group per (request, KV head) over all of its
 *                      keys, writing O itself: no workspace, no merge;
 *   PSW_DECODE_AUTO    DIRECT while every request reads at most 160 keys
 *                      (head_dim 256) or 256 keys (head_dim 512), or at most
 *                      1024 keys once batch x KV heads >= 256 work-groups
 *                      fill the GPU; SPLIT otherwise (crossovers measured on
 *                      MI355X: `bench.py --decode-sweep`).
 * A GQA group of 32 always takes SPLIT. */
enum { PSW_DECODE_AUTO = 0, PSW_DECODE_SPLIT = 1, PSW_DECODE_DIRECT = 2 };
int psw_plan_set_decode_mode(psw_plan* plan, int32_t mode);
/* What the next decode call with this window would launch: *direct = 1 when
 * it writes no partials (the direct form, or a split in which no request is
 * cut) and so has no merge launch, *work_groups = the decode launch's
 * work-groups (shares or requests, times KV heads).  PSW_E_SHAPE when the
 * plan has a request with qo_len > 1. */
int psw_plan_decode_form(const psw_plan* plan, int64_t window_left, int32_t* direct,
                         int64_t* work_groups);
int paged_decode_window_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer,
                              const void* q, float sm_scale, int64_t window_left, void* o,
                              int32_t o_dtype, psw_stream_t stream);
int paged_decode_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer, const void* q,
                       float sm_scale, void* o, int32_t o_dtype, psw_stream_t stream);

/* paged_decode_hd512 for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks, kernels and results as paged_decode_hd512, but the
 * plan's metadata, the decode schedule and the split-KV partials go to a
 * static device array of 32 MiB per GPU (held until the process ends) instead
 * of the plan's device buffers: no hipMalloc, hipFree or other allocation.
 * A batch whose metadata, schedule and partials need more than 32 MiB is
 * rejected with PSW_E_RANGE; GQA groups above 16 with PSW_E_UNSUPPORTED.
 * The metadata is copied from the plan's host memory (synchronously with
 * respect to the host) whenever the GPU's array does not already hold this
 * plan's state, window and mode.  Every call on one GPU shares that array and
 * keeps the last call's contents: calls that overlap on one GPU (from other
 * streams or threads) race and must be ordered by the caller. */
int paged_decode_hd512_noalloc(psw_plan* plan, const psw_pool* pool, int64_t layer,
                               const void* q, float sm_scale, void* o, int32_t o_dtype,
                               psw_stream_t stream);

/* ----------------------------------------------------------------- prep ---- */

/* hd256 fused prep ([P2] Proposed Plan), one pass per token:
 *   q_out[t][h] = rope(rms(q_in[t][h]) * q_norm_w, p)           (contiguous)
 *   K block     = rope(rms(k_in[t][g]) * k_norm_w, p)           (pool, layer)
 *   V block     = v_in[t][g] * inv_rms(v_in[t][g])              (pool, layer)
 * with rms(x) = x / sqrt(mean(x^2) + eps), p = start_pos + t, slot p in page
 * ids[p / page_size].  RoPE rotates pairs (i, i + 128) by the angle whose cos
 * and sin are rope_cos/rope_sin[p][i].  Math in fp32, one bf16 RNE store.
 *   q_in: device bf16 [total_qo][num_qo_heads][256]; k_in, v_in: device bf16
 *   [total_qo][num_kv_heads][256]; q_norm_w, k_norm_w: device bf16 [256];
 *   rope_cos, rope_sin: device fp32 [rope_positions][128], with numel passed
 *   for the length check; q_out: device bf16 [total_qo][num_qo_heads][256].
 * Rejects: positions past rope_positions, table lengths that disagree, eps not
 * finite and > 0, pages that do not cover [start_pos, start_pos + qo_len), and
 * a page written by two requests. */
int qkv_norm_rope_paged_prefill_hd256(psw_plan* plan, const psw_pool* pool, int64_t layer,
                                      const void* q_in, const void* k_in, const void* v_in,
                                      const void* q_norm_w, const void* k_norm_w,
                                      const float* rope_cos, const float* rope_sin,
                                      int64_t rope_positions, int64_t rope_cos_numel,
                                      int64_t rope_sin_numel, float eps, void* q_out,
                                      psw_stream_t stream);

/* hd512 fused prep ([P2] Description and Proposed Plan): from the raw k_proj
 * output alone,
 *   inv     = 1 / sqrt(mean(k^2) + eps)
 *   K block = rope(k * inv * k_norm_w, p)
 *   V block = k * inv        (same inv, never rotated)
 *   k_in: device bf16 [total_qo][num_kv_heads][512]; k_norm_w: device bf16 [512];
 *   rope tables fp32 [rope_positions][256].  Same rejects as the hd256 prep. */
int k_v_norm_rope_paged_prefill_hd512(psw_plan* plan, const psw_pool* pool, int64_t layer,
                                      const void* k_in, const void* k_norm_w,
                                      const float* rope_cos, const float* rope_sin,
                                      int64_t rope_positions, int64_t rope_cos_numel,
                                      int64_t rope_sin_numel, float eps,
                                      psw_stream_t stream);

/* hd512 query prep, the global family's share of each layer's write side
 * next to k_v_norm_rope_paged_prefill_hd512 (same per-row rule as the query
 * part of the hd256 prep, [P2] Proposed Plan; [P3] Description for the
 * global family's geometry):
 *   q_out[t][h] = rope(rms(q_in[t][h]) * q_norm_w, p),  p = start_pos + t,
 * contiguous, RoPE pairs (i, i + 256).  No pool is read or written.
 *   q_in: device bf16 [total_qo][num_qo_heads][512]; q_norm_w: device bf16
 *   [512]; rope_cos, rope_sin: device fp32 [rope_positions][256];
 *   q_out: device bf16 [total_qo][num_qo_heads][512], caller-owned.
 * Rejects (before launch): NULL plan or pointers, another stream, a plan not
 * at head_dim 512, positions past rope_positions, table lengths that
 * disagree, eps not finite and > 0. */
int q_norm_rope_prefill_hd512(psw_plan* plan, const void* q_in, const void* q_norm_w,
                              const float* rope_cos, const float* rope_sin,
                              int64_t rope_positions, int64_t rope_cos_numel,
                              int64_t rope_sin_numel, float eps, void* q_out,
                              psw_stream_t stream);

/* RoPE tables for the prep entries: cos/sin[p][i] of p * theta^(-2i/head_dim),
 * i < head_dim/2, p < positions, angles formed and evaluated in fp64 on the
 * device, stored as fp32.  cos, sin: device fp32 [positions][head_dim/2]. */
int psw_rope_tables(float* cos_out, float* sin_out, int64_t positions, int64_t head_dim,
                    double theta, psw_stream_t stream);

/* --------------------------------------------- two-family page accounting ---- */

/* Host-side page accounting for serving from two KV families at once ([P3]
 * Description: each family has its own pool and each request its own state
 * in both, and admitting a step must leave the two pools in agreement; [P3]
 * review thread: the KV frontier moves once the step has succeeded).  No device memory is involved: the server
 * hands out page ids of the two caller-owned pools (psw_pool), and
 * psw_kv_step_tables turns a batch of admitted steps into the CSR metadata of
 * psw_plan_desc.  Not thread-safe: one host thread drives a server.
 *
 * A request has one frontier F (its KV length, the same in both families) and
 * holds exactly ceil(F / page_size_f) pages of family f.  A step of n tokens:
 *   psw_kv_admit   checks, before any state changes: the request belongs to
 *                  this server, no step is pending, the held pages match F,
 *                  F + n <= rope_positions, and F + n <= window_left + 1 when
 *                  window_left >= 0 (slots equal absolute positions only
 *                  until the window starts dropping keys, so a step that
 *                  would go past the window is refused).  Then it reserves ceil((F+n)/P_f) - held_f
 *                  pages of both families; if either pool is short, nothing
 *                  is kept: both pools end exactly as they were (the same free
 *                  ids in the same order) and PSW_E_RANGE is returned.
 *   psw_kv_commit  after the step succeeded: the reserved pages join the held
 *                  ones and F += n.
 *   psw_kv_abort   after a failed step: the reserved pages go back, F stays.
 * Page ids are handed out lowest first from a fresh pool, and a pool's free
 * list is last-in first-out.
 * With local_ring_pages = R_p > 0 the local family instead keeps at most R_p
 * pages per request (a resident window, see psw_plan_desc.kv_len): it holds
 * min(ceil(F / P), R_p) pages; a step that ends past R_p * P positions needs
 * R_p * P >= window_left + n (window_left >= 0), and its tokens overwrite the
 * oldest slots of the same pages; the window bound above then no longer
 * applies. */
enum { PSW_KV_LOCAL = 0, PSW_KV_GLOBAL = 1 };

typedef struct {
  int64_t local_pages, global_pages;            /* pool sizes (page ids 0..n-1)   */
  int64_t local_page_size, global_page_size;    /* slots per page                 */
  int64_t window_left;                          /* local window (inclusive), -1 */
  int64_t rope_positions;                       /* positions the RoPE tables hold */
  int64_t local_ring_pages;                     /* 0: no ring (refuse to pass the
                                                   window); else the local family
                                                   keeps at most this many pages
                                                   per request, as a ring       */
} psw_kv_server_desc;

typedef struct psw_kv_server psw_kv_server;     /* opaque: the two pools         */
typedef struct psw_kv_request psw_kv_request;   /* opaque: one request's state   */

typedef struct {
  int64_t frontier;                             /* committed KV length            */
  int64_t local_held, global_held;              /* committed pages per family     */
  int32_t pending;                              /* 1 while a step is admitted     */
  int64_t pending_tokens;                       /* its token count                */
  int64_t local_reserved, global_reserved;      /* its reserved pages             */
} psw_kv_request_state;

/* Rejects: NULL pointers, pools or page sizes < 1, window_left < -1,
 * rope_positions < 1, extents past INT32_MAX. */
int psw_kv_server_create(const psw_kv_server_desc* desc, psw_kv_server** out);
/* PSW_E_PLAN while requests of this server are not released (nothing freed). */
int psw_kv_server_destroy(psw_kv_server* server);
int psw_kv_server_free_pages(const psw_kv_server* server, int64_t* local_free,
                             int64_t* global_free);
/* A request with F = 0 and no pages. */
int psw_kv_request_create(psw_kv_server* server, psw_kv_request** out);
/* Returns every held and reserved page to the pools and frees the state;
 * PSW_E_PLAN for a request of another server. */
int psw_kv_request_release(psw_kv_server* server, psw_kv_request* request);
int psw_kv_request_info(const psw_kv_request* request, psw_kv_request_state* out);
int psw_kv_admit(psw_kv_server* server, psw_kv_request* request, int64_t n_new);
int psw_kv_commit(psw_kv_server* server, psw_kv_request* request);
int psw_kv_abort(psw_kv_server* server, psw_kv_request* request);
/* CSR tables of one family for a batch of requests that each have a step
 * pending: request b's queries are its n_b new tokens, its pages the held then
 * the reserved ones (a ring's order once it wraps), its KV length F_b + n_b.
 * Host arrays: qo_indptr and kv_page_indptr [n_reqs + 1], kv_last_page_len
 * and kv_len [n_reqs] (the plan's optional absolute lengths, needed once a
 * ring wraps), kv_page_indices of indices_cap entries (PSW_E_SHAPE when too
 * small).  Also rejects a request listed twice, one without a pending step,
 * and one of another server. */
int psw_kv_step_tables(const psw_kv_server* server, psw_kv_request* const* requests,
                       int64_t n_reqs, int32_t family, int32_t* qo_indptr,
                       int32_t* kv_page_indptr, int32_t* kv_page_indices,
                       int64_t indices_cap, int32_t* kv_last_page_len, int32_t* kv_len);

/* ----------------------------------------------------------- device check ---- */

/* Second line of defence inside the prep kernels ([P2] Proposed Plan): a
 * position beyond the RoPE tables or a page id outside the pool makes it skip
 * that row's writes and record the first offending value in a per-plan device
 * word instead of trapping.  This call synchronises the plan's stream, returns
 * 0 when nothing was recorded and PSW_E_RANGE otherwise (the word is cleared). */
int psw_plan_device_errors(psw_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* PSW_H */
