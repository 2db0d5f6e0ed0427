// Full paged prefill at head_dim 512 (PR "feat(gemma4): paged KV serving
// across both attention families", Description: the global family has one KV
// head of 512 dims and attends to every earlier key; PR "feat(kernels): Rust
// wrapper for the hd256 windowed paged prefill", Description: explicit
// sm_scale, keys found through the page table and the final page's length).
//
// Work-group: 4 waves x 32 query rows = 128 rows = (128 / group) tokens x the
// group's heads of one KV head, one work-group per CU.  Each wave owns all 512
// dims of its rows: O^T (32 rows x 512 dims, fp32) fills the 256 accumulator
// registers, Q (32 rows x 512 dims, bf16) 128 vector registers, so every
// score feeds 64 MFMAs of its own wave and the softmax runs once per row.
// Keys come in tiles of 32: K [32][512] and V^T [32 keys][512 dims], 32 KiB
// each, in two K buffers and three V buffers (all 160 KiB of LDS), shared by
// the 128 rows.
//
// Per wave and tile step t (between two work-group barriers):
//   O^T  += V^T(t-1) P^T(t-1)     32 x v_mfma_f32_32x32x16_bf16
//   S^T(t+1) = K(t+1) Q^T          32 x v_mfma_f32_32x32x16_bf16
// with the LDS operand reads running three MFMAs ahead through one register
// ring, and, interleaved with the 64 MFMAs, the softmax of S(t) into P(t)
// (row max, lazily raised running max, exponentials, row sums) and this
// wave's share of the loads of K(t+2) and V(t+1) (global_load_lds_dwordx4,
// 16 bytes per lane straight into LDS).  A step ends by waiting for its own
// loads, zeroing V keys past kv_len, reading the first operands of the next
// step (V(t), published a step earlier) and the barrier; the V ring is three
// deep so that those reads can precede the barrier and the matrix unit finds
// its first operands ready after it.
//
// Operand layouts are those of the other attention kernels: K rows
// XOR-swizzled on the 16-byte chunk index and read in the kperm order, so each
// lane's S^T accumulators are exactly the 8 consecutive keys its P^T operand
// needs; V^T dim-major chunks of 8 keys.
#pragma once
#include "psw_attention.hpp"

namespace psw_dev {
namespace {

// The QK MFMAs as inline assembly with their accumulators in VGPRs, so that
// the 256 accumulator registers hold O (the PV MFMAs, left to the compiler,
// take the accumulator-register form) and the scores stay where the softmax
// reads them.  The compiler does not see these as MFMAs, so the kernel keeps
// the hardware's wait states itself: a dependent accumulation into the same
// registers needs none, the chain's sources come from LDS reads (ordered by
// lgkmcnt) or from registers written long before, the first k-step takes a
// literal zero accumulator, and the chain's last MFMA carries the wait states
// before anything may read its result (the count the compiler inserts after
// this MFMA before a dependent read on gfx950).  tests/test_isa_hazards_cpu.py
// checks the compiled code for any read of a chain's result, or write of its
// sources, inside the wait states.
__device__ __forceinline__ f32x16 mfma_qk_first(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The chain's last MFMA, followed by the wait states in the same statement, so
// that even a register copy the compiler places right after it is safe.
__device__ __forceinline__ void mfma_qk_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 11" : "+v"(d) : "v"(a), "v"(b));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// v_max3_f32 as one instruction: fmaxf on values the compiler cannot prove
// canonical costs two extra quieting instructions per operand.  The scores
// are finite or -inf here, never NaN.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool OUT_BF16, bool PAGE16>
__global__ __launch_bounds__(256, 1) void prefill512_kernel(AttnParams P) {
  constexpr int D = 512;
  constexpr int KT = 32;            // keys per tile
  constexpr int NCH = D / 8;        // 16-byte chunks per K row (64)
  constexpr int KS = D / 16;        // QK k-steps (32)
  constexpr int DB = D / 32;        // O^T 32-dim blocks (16)
  constexpr int NT = KT / 16;       // PV k-steps per tile (2)
  constexpr int NV = NT * DB;       // PV MFMAs per tile (32)
  constexpr int TILE = KT * D * 2;  // 32 KiB
  constexpr int AH = 3;             // LDS operand reads in flight ahead of the MFMAs
  // O and the row sums are rescaled only when a row's maximum rises by more
  // than kSlack (log2 units) over the one they are scaled to: P stays below
  // 2^16 and the rescale (256 accumulators) is rare.
  constexpr float kSlack = 16.0f;

  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb2[TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int hkv = P.num_kv_heads;
  const int item = blockIdx.x / hkv;
  const int kvh = blockIdx.x - item * hkv;
  const int b = ldu(P.items + 4 * item + 0);
  const int t0 = ldu(P.items + 4 * item + 1);
  const int k_lo = ldu(P.items + 4 * item + 2);
  const int k_hi = ldu(P.items + 4 * item + 3);
  const int q_beg = ldu(P.qo_indptr + b);
  const int qo_len = ldu(P.qo_indptr + b + 1) - q_beg;
  const int kvl = ldu(P.kv_len + b);
  const int start = kvl - qo_len;
  const int pg0 = ldu(P.kv_page_indptr + b);
  const int32_t* pages = P.kv_page_indices + pg0;
  const int last_page = ldu(P.kv_page_indptr + b + 1) - pg0 - 1;
  const int gs = P.group_shift;
  const int tok_w = 32 >> gs;  // tokens per wave
  const int wl = P.window_left;

  // this lane's query row: token t0 + tl, head kvh * group + hh
  const int tl = w * tok_w + (n >> gs);
  const int hh = n & ((1 << gs) - 1);
  const int tok = t0 + tl;
  const bool row_valid = tok < qo_len;
  const int pos = start + tok;
  const int head = (kvh << gs) + hh;
  const int hi_n = row_valid ? min(k_hi, pos) : -1;
  const int lo_n = max(k_lo, wl >= 0 ? pos - wl : 0);
  const int wt0 = t0 + w * tok_w;
  const int w_pmin = start + wt0;
  const int w_pmax = start + min(wt0 + tok_w, qo_len) - 1;
  const bool wave_live = wt0 < qo_len;

  const char* kbase_g =
      reinterpret_cast<const char*>(P.pool + P.layer_off + (int64_t)kvh * P.ps.head);
  const char* vbase_g = kbase_g + P.ps.kv * 2;
  const int pshift = PAGE16 ? 4 : P.ps.page_shift;
  const int psize = PAGE16 ? 16 : P.ps.page_size;
  const int64_t page_bytes = P.ps.page * 2;
  const uint32_t pb32 = (uint32_t)page_bytes;  // one page is below 4 GiB (host check)
  const int jt0 = k_lo / KT;
  const int ntiles = k_hi / KT - jt0 + 1;
  const PageRing ring = page_ring(last_page + 1, kvl, pshift);

  // ---- Q of this lane's row, B operands of the QK MFMAs ----
  // lane (n, h), k-step ks: dims 16 ks + 8 h .. + 7 of row n; loaded in the
  // prologue through LDS
  bf16x8 qf[KS];

  // ---- tile loads (16 instructions of 1 KiB per K or V^T tile) ----
  // K: wave w loads keys 4 w .. 4 w + 3 of each of the tile's two 16-key
  // halves, one 1 KiB row per instruction, lane l reading chunk l ^ kswz(key)
  // so that LDS position l holds it.  The four rows of a half lie in one page
  // (pages hold at least 8 keys) in consecutive slots and in consecutive LDS
  // rows, so they share one scalar base and one M0 and step by the
  // instruction offset, which the load applies to both addresses.  V^T:
  // wave w loads the chunks of k8 = w (keys 8 w .. 8 w + 7, one page) for
  // dims 64 j .. 64 j + 63, j < 8: one scalar base, the lane's offset
  // 2 P (64 j + lane) held in a register.  So each wave needs three page ids
  // per tile step (its two K halves, its V keys), fetched with one vector
  // load a step ahead (lanes 0-2) and read back with readlane.
  // kvo[j]: the K lanes' chunk offsets (the swizzle depends on the key only
  // through w and j); vvo[j]: the V lanes' offsets.  Loop-invariant.
  uint32_t kvo[4], vvo[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) kvo[j] = (uint32_t)((lane ^ kswz(4 * w + j)) << 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) vvo[j] = (uint32_t)((64 * j + lane) * 2 * psize);
  // the keys whose pages a wave loads for a tile starting at key j0
  auto k_key = [&](int j0, int half) __attribute__((always_inline)) { return j0 + 16 * half + 4 * w; };
  auto v_key = [&](int j0) __attribute__((always_inline)) { return j0 + 8 * w; };
  // page id of a key (keys past the request's pages read a resident page;
  // they are masked and their V zeroed)
  auto page_of = [&](int key) __attribute__((always_inline)) { return pages[ring(key >> pshift)]; };
  // lanes 0-1: the pages of the K halves of tile tk, lanes 2-63: the page of
  // the V keys of tile tv (one load instruction, no branch)
  auto fetch_pids = [&](int tk, int tv) __attribute__((always_inline)) {
    const int jk = (jt0 + tk) * KT, jv = (jt0 + tv) * KT;
    return page_of(lane < 2 ? k_key(jk, lane) : v_key(jv));
  };
  auto settled = [](int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
  };
  // byte offset of a page (64-bit: a pool may pass 4 GiB) plus a slot offset
  auto page_off = [&](int page) __attribute__((always_inline)) {
    return (uint64_t)(uint32_t)page * pb32;
  };
  // byte offsets, inside the pool's K and V blocks, of what a wave loads for
  // a tile starting at key j0: K halves (first key's row), V (first key's slot)
  auto k_off = [&](int page, int j0, int half) __attribute__((always_inline)) {
    return page_off(page) + (uint32_t)((k_key(j0, half) & (psize - 1)) * (D * 2));
  };
  auto v_off = [&](int page, int j0) __attribute__((always_inline)) {
    return page_off(page) + (uint32_t)((v_key(j0) & (psize - 1)) * 2);
  };
  // rows 2 p and 2 p + 1 (p = 0, 1) of the wave's four rows of one K half
  // (m0 clobbered: see the tile-load helpers in psw_attention.hpp)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto k_load_pair = [&](char* kl, uint64_t koff, int half, int p) __attribute__((always_inline)) {
    const char* base = kbase_g + koff;
    const uint32_t m0 =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(kl + (16 * half + 4 * w) * 1024);
    if (p == 0)
      asm volatile(
          "s_mov_b32 m0, %2\n\t"
          "global_load_lds_dwordx4 %0, %3\n\t"
          "global_load_lds_dwordx4 %1, %3 offset:1024"
          :
          : "v"(kvo[0]), "v"(kvo[1]), "s"(m0), "s"(base)
          : "memory", "m0");
    else
      asm volatile(
          "s_mov_b32 m0, %2\n\t"
          "global_load_lds_dwordx4 %0, %3 offset:2048\n\t"
          "global_load_lds_dwordx4 %1, %3 offset:3072"
          :
          : "v"(kvo[2]), "v"(kvo[3]), "s"(m0), "s"(base)
          : "memory", "m0");
  };
#pragma clang diagnostic pop
  auto k_load_half = [&](char* kl, uint64_t koff, int half) __attribute__((always_inline)) {
    k_load_pair(kl, koff, half, 0);
    k_load_pair(kl, koff, half, 1);
  };
  auto v_load = [&](char* vl, uint64_t voff, int j) __attribute__((always_inline)) {
    lds_dma16_s(vbase_g + voff, vvo[j], vl + (8 * w + j) * 1024);
  };
  // Zero, in the V^T chunks this wave loaded (keys 8 w .. 8 w + 7), the keys
  // at or past kv_len (their pool slots may hold anything, NaN included, and
  // 0 * NaN would reach O).
  auto v_sanitize = [&](char* vl, int j0) __attribute__((always_inline)) {
    const int jc = v_key(j0);
    if (jc + 8 <= kvl) return;
    rare_path();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8* cp = reinterpret_cast<bf16x8*>(vl + (8 * w + j) * 1024 + lane * 16);
      bf16x8 v = *cp;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (jc + e >= kvl) ? (__bf16)0.0f : v[e];
      *cp = v;
    }
    // the step's last LDS operations before its barrier: the lgkmcnt(3) wait
    // there leaves the last three in flight, which would be these writes
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  };

  // ---- LDS operand addresses ----
  const int krow = kperm(n);
  const int ksw = kswz(krow);
  const int kaddr0 = krow * NCH * 16 + 16 * (h ^ (ksw & 1)) + 32 * (ksw >> 1);
  const int vaddr0 = (h * D + n) * 16;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.0f;
  const float c2 = P.scale_log2;
  f32x16 sbuf[2] = {};  // S(t) and S(t+1), alternating by step parity
  bf16x8 pb[NT];      // P(t-1), the B operands of the current step's PV
#pragma unroll
  for (int t = 0; t < NT; ++t) pb[t] = bf16x8{};
  bf16x8 ra[AH + 1];  // A operands: V^T chunks (PV ops), then K chunks (QK ops)

  // Tiles inside every row's keys (no element mask): starts in [full_lo, full_hi].
  const int full_lo = wave_live ? max(k_lo, wl >= 0 ? w_pmax - wl : k_lo) : 0x7fffffff;
  const int full_hi = min(k_hi, w_pmin) - (KT - 1);

  // operand read of op i of a step (PV ops first when the step has them)
  // ka, va: opaque copies of kaddr0, vaddr0 made once per step, so that the
  // compiler forms each op's address from them instead of holding 64
  // precomputed addresses in registers across the loop
  auto load_op = [&](int i, auto pv_c, const char* vl, const char* kl, int ka, int va)
                     __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_c)::value;
    if (PV && i < NV) {
      const int db = i / NT, t = i % NT;  // O block db takes its NT MFMAs back to back
      ra[i % (AH + 1)] = *reinterpret_cast<const bf16x8*>(vl + va + (2 * t * D + 32 * db) * 16);
    } else {
      const int ks = PV ? i - NV : i;
      ra[i % (AH + 1)] =
          *reinterpret_cast<const bf16x8*>(kl + (ka ^ ((ks & 7) << 5)) + (ks >> 3) * 256);
    }
  };

  // K buffer roles: Kr holds K(t+1) (read by this step's QK), Kw the buffer
  // K(t+2) is loaded into.  V buffer roles: Vp holds V(t-1) (read by this
  // step's PV), Vc holds V(t) (read by the next step), Vn receives V(t+1).
  char* Kr = kb1;
  char* Kw = kb0;
  char* Vp = vb2;
  char* Vc = vb0;
  char* Vn = vb1;
  int pid = 0;        // page ids of this step's loads (lanes 0-2)

  // ---- prologue: Q, then K(0), K(1), V(0) resident, S(0) = K(0) Q^T ----
  {
    // Q through LDS: wave w's 32 rows into a 32 KiB buffer of its own, one
    // 1 KiB row per load instruction (lane l brings chunk l ^ (r % 16) of
    // row r, so that the operand reads below, 32 rows at one chunk, hit
    // distinct banks), then read back in the operand layout.  Loaded straight
    // into registers, each load instruction touched 32 rows at 32 bytes and
    // the loads took ~12 k cycles to issue.  A row past qo_len takes the
    // request's first query (its output is never written).
    char* const qst = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? vb0 : vb1;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int tk = t0 + w * tok_w + (r >> gs);
      const int hd = (kvh << gs) + (r & ((1 << gs) - 1));
      const __bf16* row = P.q + ((int64_t)(q_beg + (tk < qo_len ? tk : 0)) * P.num_qo_heads + hd) * D;
      lds_dma16_s(row, (uint32_t)((lane ^ (r & 15)) << 4), qst + r * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's rows landed
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qst + n * 1024 + (((2 * ks + h) ^ (n & 15)) << 4));
    // every wave has its Q before the tiles overwrite the buffers
    lds_barrier();
    const int j0 = jt0 * KT;
    const int pk0 = ldu(pages + ring(k_key(j0, 0) >> pshift));
    const int pk1 = ldu(pages + ring(k_key(j0, 1) >> pshift));
    const int pv0 = ldu(pages + ring(v_key(j0) >> pshift));
    k_load_half(kb0, k_off(pk0, j0, 0), 0);
    k_load_half(kb0, k_off(pk1, j0, 1), 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) v_load(vb0, v_off(pv0, j0), j);
    if (ntiles > 1) {
      const int pk2 = ldu(pages + ring(k_key(j0 + KT, 0) >> pshift));
      const int pk3 = ldu(pages + ring(k_key(j0 + KT, 1) >> pshift));
      k_load_half(kb1, k_off(pk2, j0 + KT, 0), 0);
      k_load_half(kb1, k_off(pk3, j0 + KT, 1), 1);
    }
    pid = fetch_pids(2, 1);  // step 0 loads K(2) and V(1)
    __builtin_amdgcn_s_waitcnt(0);
    v_sanitize(vb0, j0);
    lds_barrier();
    pid = settled(pid);
    const int ka = kaddr0;
#pragma unroll
    for (int i = 0; i < AH; ++i) load_op(i, std::false_type{}, nullptr, kb0, ka, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if (i + AH < KS) load_op(i + AH, std::false_type{}, nullptr, kb0, ka, 0);
      if (i == 0) sbuf[0] = mfma_qk_first(ra[0], qf[0]);
      else if (i < KS - 1) mfma_qk(sbuf[0], ra[i % (AH + 1)], qf[i]);
      else mfma_qk_last(sbuf[0], ra[i % (AH + 1)], qf[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave is done with K(0) before step 0 loads K(2) over it
    lds_barrier();
  }

  // One step t.  PV: O += P(t-1) V(t-1); QK: S(t+1) = K(t+1) Q^T; SM: the
  // softmax of S(t); LK / LV: loads of K(t+2) / V(t+1).  The flags are
  // compile-time so that no MFMA or load of a step sits behind a branch.
  // The scores alternate between two register sets: S(t) is read from
  // sbuf[PAR] while the QK chain writes S(t+1) into sbuf[PAR ^ 1], so the
  // softmax spreads over all 64 MFMAs of the step.
  // PAR 2 + x: "same-set" step on sbuf[x]: S(t+1) overwrites S(t) in the QK
  // half, so the softmax runs in the PV half (the steps after the pairs).
  auto step = [&](int t, auto par_c, auto pv_c, auto qk_c, auto sm_c, auto lk_c, auto lv_c)
                  __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value & 1;
    constexpr bool SAME = decltype(par_c)::value >= 2;
    constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
    constexpr bool SM = decltype(sm_c)::value;
    constexpr bool LK = decltype(lk_c)::value, LV = decltype(lv_c)::value;
    constexpr int NOP = (PV ? NV : 0) + (QK ? KS : 0);
    static_assert(!SAME || PV || !QK, "a same-set step overwrites S(t) only after its PV half");
    f32x16& sc = sbuf[PAR];                // S(t)
    f32x16& sn = sbuf[SAME ? PAR : PAR ^ 1];  // S(t+1)
    const int j0 = (jt0 + t) * KT;  // first key of tile t
    // The step's set-up runs after its first MFMA is issued, in that MFMA's
    // shadow (before, ~40 instructions of it stood between the barrier and
    // the first MFMA): the page ids of the next step's loads (K(t+3) in
    // lanes 0-1, V(t+2) in lane 2) are fetched at the first QK op, the load
    // offsets of this step and the tile mask after op 0.
    int pid_next = 0;
    uint64_t kp[2] = {0, 0}, vp = 0;
    bool plain = true;
    float cmul = c2;
    auto setup = [&]() __attribute__((always_inline)) {
      if (LK) {
        kp[0] = k_off(__builtin_amdgcn_readlane(pid, 0), j0 + 2 * KT, 0);
        kp[1] = k_off(__builtin_amdgcn_readlane(pid, 1), j0 + 2 * KT, 1);
      }
      if (LV) vp = v_off(__builtin_amdgcn_readlane(pid, 2), j0 + KT);
      // masked tiles (and a negative scale) scale and mask the scores up
      // front; the exponentials below then use them as they are
      if (SM) {
        plain = j0 >= full_lo && j0 <= full_hi && c2 >= 0.0f;
        if (!plain) {
          rare_path();
          // register r holds key j0 + 16 (r / 8) + 8 h + r % 8
          const int kb0_ = j0 + 8 * h - lo_n;
          const unsigned span = (unsigned)(hi_n - lo_n);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned rel = (unsigned)(kb0_ + 16 * (r >> 3) + (r & 7));
            sc[r] = rel <= span ? sc[r] * c2 : -__builtin_inff();
          }
        }
        cmul = plain ? c2 : 1.0f;
      }
    };
    float mx = -__builtin_inff(), m_use = m_run, m_new = m_run;
    bool need = false;
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t pnu[8];    // P(t) as bf16 pairs (keys 2j, 2j + 1 of the lane)
    const int ka = opaque(kaddr0), va = opaque(vaddr0);
    if (!PV) {
#pragma unroll
      for (int i = 0; i < AH; ++i) load_op(i, std::false_type{}, Vp, Kr, ka, va);
    }
    // softmax schedule over the step's ops: the row max at ops 1-8, its
    // reduction at op 9, the 16 exponentials from op 10 on, ES ops apart;
    // parts a short step has no op for run after its MFMAs
    constexpr int ES = NOP >= 64 && !SAME ? 3 : 1;
    constexpr int SM_END = 10 + 16 * ES;
    static_assert(!SAME || !QK || SM_END <= NV, "a same-set step's softmax ends in its PV half");
    auto sm_at = [&](int i) __attribute__((always_inline)) {
      if (i >= 1 && i <= 8) mx = max3(mx, sc[2 * i - 2], sc[2 * i - 1]);
      if (i == 9) {
        mx = max_with_partner_half(mx * cmul);
        m_new = fmaxf(m_run, mx);
        need = __any(m_new > m_run + kSlack);
        m_use = need ? m_new : m_run;
      }
      if (i >= 10 && (i - 10) % ES == 0 && (i - 10) / ES < 16) {
        // P(t) in place of S(t); every second exponential rounds the pair to
        // bf16 (the PV operand) and adds the rounded values to the row sum,
        // so that O is normalised by the sum of the weights it was built
        // from (a row dominated by one key then returns that key's V as it
        // is, instead of off by the key's rounding)
        const int e = (i - 10) / ES;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], cmul, -m_use));
        sc[e] = p;
        if (e & 1) {
          const bf16x2 pk = {(__bf16)sc[e - 1], (__bf16)p};
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          ls[(e >> 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(pk, one, ls[(e >> 1) & 3], false);
          pnu[e >> 1] = __builtin_bit_cast(uint32_t, pk);
          pin(__builtin_bit_cast(float, pnu[e >> 1]));
        }
      }
    };
    constexpr int FOP = (PV && QK) ? NV : 8;  // op that fetches the next step's page ids
    static_assert(!(LK || LV) || NOP > FOP, "a step with loads has an op to fetch page ids at");
    auto op = [&](int i) __attribute__((always_inline)) {
      if (i + AH < NOP) load_op(i + AH, pv_c, Vp, Kr, ka, va);
      // the next step's first PV operands (V(t), published a step ago) in
      // the last ops: their ring slots continue this step's
      else if (SM) load_op(i + AH - NOP, std::true_type{}, Vc, Kw, 0, va);
      if (PV && i < NV) {
        oacc[i / NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i % (AH + 1)], pb[i % NT],
                                                                oacc[i / NT], 0, 0, 0);
      } else {
        const int ks = PV ? i - NV : i;
        if (ks == 0) sn = mfma_qk_first(ra[i % (AH + 1)], qf[0]);
        else if (ks < KS - 1) mfma_qk(sn, ra[i % (AH + 1)], qf[ks]);
        else mfma_qk_last(sn, ra[i % (AH + 1)], qf[ks]);
      }
      if ((LK || LV) && i == FOP) pid_next = fetch_pids(t + 3, t + 2);
      // loads: K(t+2) two rows at a time at ops 2, 6, 10 and 14 of the PV
      // half (four at ops 2 and 4: 1.2% slower), V(t+1) at the first even
      // ops of the QK half (ops 6.. in a step without one), so that the tile
      // writes into LDS split between the halves
      constexpr int LB = (PV && QK) ? NV : 6;
      if (LK && i >= 2 && i <= 14 && i % 4 == 2) k_load_pair(Kw, kp[i >= 10], i >= 10, (i >> 2) & 1);
      if (LV && i >= LB && i <= LB + 14 && i % 2 == 0) v_load(Vn, vp, (i - LB) / 2);
      if (SM) sm_at(i);
      __builtin_amdgcn_sched_barrier(0);
    };
    // op 0, the set-up in its MFMA's shadow, then the other ops (a step of
    // one tile's softmax alone has none)
    if constexpr (NOP > 0) op(0);
    setup();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < NOP; ++i) op(i);
    if (SM) {
#pragma unroll
      for (int i = NOP; i < SM_END; ++i) sm_at(i);
    }
    static_assert(!(LV || LK) || NOP >= 32, "a step with loads has at least 32 ops");
    // the loads of this step landed: publish V(t+1) (zeroed past kv_len) and
    // K(t+2).  vmcnt(0) only: the next step's first operand reads stay in flight.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    if (LV) v_sanitize(Vn, j0 + KT);
    if (SM) {
      if (need) {
        rare_path();
        // O was accumulated against m_run (the last PV of it issued at the
        // start of this step); nothing to rescale before the first tile
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        if (m_run > 0.5f * kNegBig) {
          // one block at a time: read into VGPRs, scale, write back (the
          // scheduler would otherwise read all 256 accumulators first)
#pragma unroll
          for (int i = 0; i < DB; ++i) {
            // pinned to the accumulator registers on both sides, so that the
            // block is scaled in place (otherwise the allocator moves all
            // 256 accumulators around the branch)
            asm volatile("" : "+a"(oacc[i]));
            f32x16 tt = oacc[i];
#pragma unroll
            for (int e = 0; e < 16; ++e) tt[e] *= alpha;
            oacc[i] = tt;
            asm volatile("" : "+a"(oacc[i]));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        l_run *= alpha;
        m_run = m_new;
      }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    if (LK || LV) pid = settled(pid_next);
    if (SM) {
      // P(t), the B operands of the next step's PV (register r of half h:
      // key 16 (r / 8) + 8 h + r % 8)
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const u32x4 v = {pnu[4 * q], pnu[4 * q + 1], pnu[4 * q + 2], pnu[4 * q + 3]};
        pb[q] = __builtin_bit_cast(bf16x8, v);
      }
    }
    if constexpr (NOP == 0) {
      // no ops to issue them in: the next step's first operands here
      if (SM) {
#pragma unroll
        for (int i = 0; i < AH; ++i) load_op(i, std::true_type{}, Vc, Kw, 0, va);
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc37f);  // lgkmcnt(3): all but the three operand reads
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    char* const kt = Kr;
    Kr = Kw;
    Kw = kt;
    char* const vt = Vp;
    Vp = Vc;
    Vc = Vn;
    Vn = vt;
  };

  using T = std::true_type;
  using F = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using S1 = std::integral_constant<int, 3>;  // same-set steps on sbuf[1]
  // step 0 (no PV, S(0) in sbuf[0]), then full steps in pairs (S(t) in
  // sbuf[t % 2]); after the pairs t is odd, S(t) is in sbuf[1], and the
  // remaining steps keep it there (same-set steps)
  if (ntiles >= 3) step(0, P0{}, F{}, T{}, T{}, T{}, T{});
  else if (ntiles == 2) step(0, P0{}, F{}, T{}, T{}, F{}, T{});
  else step(0, P0{}, F{}, F{}, T{}, F{}, F{});
  int t = 1;
  for (; t + 3 < ntiles; t += 2) {
    step(t, P1{}, T{}, T{}, T{}, T{}, T{});
    step(t + 1, P0{}, T{}, T{}, T{}, T{}, T{});
  }
  if (t + 2 < ntiles) {  // one more full step
    step(t, S1{}, T{}, T{}, T{}, T{}, T{});
    ++t;
  }
  if (t + 1 < ntiles) {  // t == ntiles - 2 >= 1
    step(t, S1{}, T{}, T{}, T{}, F{}, T{});
    ++t;
  }
  if (t < ntiles) {      // t == ntiles - 1 >= 1
    step(t, S1{}, T{}, F{}, T{}, F{}, F{});
    ++t;
  }
  step(t, S1{}, T{}, F{}, F{}, F{}, F{});  // PV(ntiles - 1)

  // every wave is done reading its last tiles: LDS is free
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  // lane (n, h), O^T block db, register r holds dim 32 db + 8 (r / 4) + 4 h + r % 4
  if constexpr (OUT_BF16) {
    // O rows of this wave through 32 KiB of LDS: [row n][64 chunks of 16 B],
    // chunk c of row n at position c ^ n; then one whole row per store
    char* const stg = w == 0 ? kb0 : w == 1 ? kb1 : w == 2 ? vb0 : vb1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v = {(__bf16)(oacc[db][4 * g] * inv), (__bf16)(oacc[db][4 * g + 1] * inv),
                    (__bf16)(oacc[db][4 * g + 2] * inv), (__bf16)(oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<bf16x4*>(stg + n * 1024 + (((4 * db + g) ^ n) << 4) + 8 * h) = v;
      }
    // LDS operations of one wave complete in order: no wait between the
    // writes above and the reads below, only no compiler reordering
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + r * 1024 + ((lane ^ r) << 4));
      const int tt = t0 + w * tok_w + (r >> gs);
      if (tt < qo_len) {
        const int hd = (kvh << gs) + (r & ((1 << gs) - 1));
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(P.o) +
                                   ((int64_t)(q_beg + tt) * P.num_qo_heads + hd) * D + lane * 8) = v;
      }
    }
  } else {
    if (!row_valid) return;
    const int64_t orow = ((int64_t)(q_beg + tok) * P.num_qo_heads + head) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = 32 * db + 8 * g;
        f32x4 v = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                   oacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(P.o) + orow + off) = v;
      }
  }
}

}  // namespace
}  // namespace psw_dev
