// Windowed paged prefill at head_dim 256, two wave groups in ping-pong (PR
// "feat(kernels): Rust wrapper for the hd256 windowed paged prefill",
// Description: explicit sm_scale, inclusive window, keys through the page
// table).
//
// Work-group: 8 waves x 32 query rows = 256 rows = (256 / group) tokens x the
// group's heads of one KV head.  Keys come in tiles of 32 (K [32][256] and
// V^T [32 keys][256 dims], 16 KiB each, three buffers each in LDS), shared by
// all 256 rows.  Each wave keeps Q dims 0..127 of its rows in registers and
// dims 128..255 in LDS (64 KiB), which leaves room for two waves per SIMD.
// Q arrives through LDS (whole rows per load instruction, then read back in
// the MFMA operand layout) and O leaves through LDS (whole rows per store).
//
// A wave alternates two kinds of phase:
//   MFMA phase u:  O += P(u-1) V(u-1);  S(u) = K(u) Q^T         (32 MFMAs)
//   ALU phase u:   softmax of S(u) -> P(u) (row max, running max, lazy O
//                  rescale, exponentials, row sums)
// Waves 0-3 (group 0) start with an MFMA phase and waves 4-7 (group 1) with
// an empty ALU phase, and every phase ends at a work-group barrier, so on each
// SIMD one wave keeps the matrix unit busy while the other runs its softmax.
// The matrix operands come from LDS as in attention_kernel (XOR-swizzled K
// rows read in the kperm order, dim-major V^T chunks), so P^T feeds the PV
// MFMAs straight from the S^T accumulators.
//
// Loads are split between the groups, four load instructions per wave each
// time: group 0 loads K(u+2) at the end of its MFMA phase u (while it waits
// for group 1's softmax) into the buffer K(u-1) left, group 1 loads V(j+2)
// in its ALU phase j into the buffer of V(j-1); each ALU phase waits for all
// but the latest four loads of its wave (vmcnt(4)), group 1 zeroes the keys
// past kv_len of the V tile that just landed, and the barrier that follows
// publishes the tile, at least one phase before its first reader.
#pragma once
#include "psw_attention.hpp"

namespace psw_dev {
namespace {

template <bool OUT_BF16, bool PAGE16>
__global__ __launch_bounds__(512, 1) void prefill256_pp_kernel(AttnParams P) {
  constexpr int D = 256;
  constexpr int KT = 32;           // keys per tile
  constexpr int NCH = D / 8;       // 16-byte chunks per K row
  constexpr int NT = KT / 16;      // PV k-steps per tile
  constexpr int DB = D / 32;       // O^T 32-row blocks
  constexpr int KS = D / 16;       // QK k-steps
  constexpr int TILE = KT * D * 2; // 16 KiB
  constexpr int NW = 8;
  constexpr int AH = 3;            // LDS operand reads in flight ahead of the MFMAs
  // O and the row sums are rescaled only when a row's maximum rises by more
  // than kSlack (log2 units) over the one they are scaled to: P then stays
  // below 2^20, far inside the range of bf16 and of the fp32 sums, and the
  // rescale (128 multiplies per lane) is rare.
  constexpr float kSlack = 20.0f;

  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char kb2[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb2[TILE];
  // Q dims 128..255 of every wave's rows (the first 128 dims stay in
  // registers): [wave][k-step 8..15][lane] chunks of 16 bytes
  constexpr int KSR = KS / 2;     // QK k-steps whose Q operand is in registers
  __shared__ __attribute__((aligned(1024))) char qlds[NW * (KS - KSR) * 1024];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w >> 2;   // 0: MFMA first, 1: ALU first
  const int wg = w & 3;
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

  // this lane's query row: token t0 + tl, head kvh*group + hh
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

  // Q rows of this wave in LDS, in halves of 128 dims: [row n][16 chunks of
  // 16 B], chunk c of row n stored at position c ^ (n % 16), so that the 16
  // rows a ds_read_b128 serves together fall in distinct banks.  Dims
  // 128..255 stay in qlds; dims 0..127 pass through a tile buffer that is not
  // in use yet on their way to registers.
  bf16x8 qf[KSR];
  char* const qhi = qlds + w * 8192;
  char* const qlo = ((w >> 1) == 0 ? kb2 : (w >> 1) == 1 ? vb0 : (w >> 1) == 2 ? vb1 : vb2) +
                    (w & 1) * 8192;
  const int qrd = n * 256 + ((h ^ (n & 15)) << 4);  // k-step ks of the half: qrd ^ (ks << 5)

  const char* kbase_g =
      reinterpret_cast<const char*>(P.pool + P.layer_off + (int64_t)kvh * P.ps.head);
  const char* vbase_g = kbase_g + P.ps.kv * 2;
  const int pshift = PAGE16 ? 4 : P.ps.page_shift;
  const int psize = PAGE16 ? 16 : P.ps.page_size;
  const int64_t page_bytes = P.ps.page * 2;
  const int jt0 = k_lo / KT;
  const int ntiles = k_hi / KT - jt0 + 1;

  // ---- tile loads ----
  // A tile is 16 load instructions of 1 KiB; instruction `ins` covers K keys
  // 2 ins, 2 ins + 1 and V^T chunks (k8 = ins / 4, d = 64 (ins % 4) + lane).
  // Wave wg of the loading group issues instructions 4 r + wg, r < 4.
  const PageRing ring = page_ring(last_page + 1, kvl, PAGE16 ? 4 : P.ps.page_shift);
  auto page_id = [&](int idx) __attribute__((always_inline)) { return ldu(pages + ring(idx)); };

  // ---- LDS operand addresses (as in attention_kernel, 32-key tiles) ----
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
  f32x16 s = {};          // S(t) from the last MFMA phase
  bf16x8 pb[NT];          // P(t) from the last ALU phase
#pragma unroll
  for (int t = 0; t < NT; ++t) pb[t] = bf16x8{};

  // MFMA phase: PV of the previous tile (ops 0..NV-1, if any), then QK of
  // this one (if any), as one sequence of ops whose LDS operand reads run AH
  // ops ahead through a ring of registers.  The first AH reads are issued at
  // the end of the phase before (preload), so the phase opens with an MFMA.
  // The swizzled offsets are formed from opaque copies where they are used,
  // not kept in registers across the loop.
  constexpr int NV = NT * DB;
  bf16x8 ra[AH + 1];  // A operands: V^T chunks (PV ops), K chunks (QK ops)
  bf16x8 rq[AH + 1];  // B operands of the QK ops whose Q part sits in LDS
  auto load_op = [&](int i, auto pv_c, auto qk_c, const char* vl, const char* kl, int ka, int qb)
                     __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_c)::value;
    if (PV && i < NV) {
      const int t = i % NT, db = i / NT;  // O block db takes its NT MFMAs back to back
      ra[i % (AH + 1)] = *reinterpret_cast<const bf16x8*>(vl + vaddr0 + (2 * t * D + 32 * db) * 16);
    } else {
      const int ks = PV ? i - NV : i;
      if (ks >= KSR)
        rq[i % (AH + 1)] = *reinterpret_cast<const bf16x8*>(qhi + (qb ^ ((ks - KSR) << 5)));
      ra[i % (AH + 1)] =
          *reinterpret_cast<const bf16x8*>(kl + (ka ^ ((ks & 7) << 5)) + (ks >> 3) * 256);
    }
  };
  auto preload = [&](auto pv_c, const char* vl, const char* kl) __attribute__((always_inline)) {
    const int ka = opaque(kaddr0), qb = opaque(qrd);
#pragma unroll
    for (int i = 0; i < AH; ++i) load_op(i, pv_c, std::true_type{}, vl, kl, ka, qb);
  };
  auto mfma_seq = [&](auto pv_c, auto qk_c, const char* vl, const char* kl) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
    constexpr int NOP = (PV ? NV : 0) + (QK ? KS : 0);
    const int ka = opaque(kaddr0), qb = opaque(qrd);
    // the preloaded operands and P pass through an empty statement that stays
    // after the barrier, so no MFMA of this phase is hoisted above it
#pragma unroll
    for (int i = 0; i < AH; ++i) asm volatile("" : "+v"(ra[i]));
    if (PV) asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
    if (QK) s = f32x16{};
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i + AH < NOP) load_op(i + AH, pv_c, qk_c, vl, kl, ka, qb);
      if (PV && i < NV) {
        oacc[i / NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i % (AH + 1)], pb[i % NT],
                                                                oacc[i / NT], 0, 0, 0);
      } else {
        const int ks = PV ? i - NV : i;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[i % (AH + 1)],
                                                    ks < KSR ? qf[ks] : rq[i % (AH + 1)], s, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax of S(t) (tile starting at key j0) into P(t); rescales O if the
  // running max rose past the slack.
  // Tiles inside every row's keys and window (no element mask): tile starts
  // j0 in [full_lo, full_hi], worked out once.
  const int full_lo = wave_live ? max(k_lo, wl >= 0 ? w_pmax - wl : k_lo) : 0x7fffffff;
  const int full_hi = min(k_hi, w_pmin) - (KT - 1);
  auto softmax = [&](int j0) __attribute__((always_inline)) {
    const bool full = j0 >= full_lo && j0 <= full_hi;
    float mx = -__builtin_inff();
    if (full) {
      // max of s * c2: c2 times the max of s, or of the min for a negative c2
      float e = s[0];
      if (c2 >= 0.0f) {
#pragma unroll
        for (int r = 1; r < 16; ++r) e = fmaxf(e, s[r]);
      } else {
        rare_path();
#pragma unroll
        for (int r = 1; r < 16; ++r) e = fminf(e, s[r]);
      }
      mx = e * c2;
    } else {
      rare_path();
      // register r holds key j0 + 16 (r / 8) + 8 h + r % 8
      const int kb0 = j0 + 8 * h - lo_n;
      const unsigned span = (unsigned)(hi_n - lo_n);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned rel = (unsigned)(kb0 + 16 * (r >> 3) + (r & 7));
        const float v = rel <= span ? s[r] * c2 : -__builtin_inff();
        s[r] = v;   // masked tiles keep scaled scores
        mx = fmaxf(mx, v);
      }
    }
    mx = max_with_partner_half(mx);
    const float m_new = fmaxf(m_run, mx);
    const bool need = __any(m_new > m_run + kSlack);
    const float m_use = need ? m_new : m_run;
    const float cmul = full ? c2 : 1.0f;
    // four partial row sums: a short dependency chain
    float ls[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], cmul, -m_use));
      ls[r & 3] = r < 4 ? p : ls[r & 3] + p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    if (need) {
      rare_path();
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    }
    l_run += lsum;
    // P(t) and the row sum complete here, inside the ALU phase: keep the
    // compiler from sinking the exponentials or the additions into the next
    // MFMA phase
    asm volatile("" : "+v"(l_run) : "v"(pb[0]), "v"(pb[1]));
  };

  // Tile loads: group 0 loads K(u+2) at the end of its MFMA(u), group 1
  // V(j+2) in its ALU(j) (ALU(-1) of group 1 also V(0)), four instructions
  // per wave; each group's ALU phase waits for all but its latest four
  // loads, and group 1 zeroes the keys past kv_len of V(j+1).  With 16-slot
  // pages the page ids of a tile are read through the scalar cache in the ALU
  // phase before its loads.
  // 16-slot pages: a tile is two pages; tp holds their byte offsets in the
  // pool (page id x page bytes, from 32-bit halves: a page of this geometry
  // is far below 4 GiB).
  const uint32_t pb32 = (uint32_t)page_bytes;
  int64_t tpid[2] = {0, 0};  // page byte offsets of this wave's next tile
  auto fetch_pids = [&](int tile, int64_t* tp) __attribute__((always_inline)) {
    if constexpr (PAGE16) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
        tp[p] = (int64_t)((uint64_t)(uint32_t)page_id(((jt0 + tile) * KT >> 4) + p) * pb32);
    }
  };
  // The loop's fetches walk the page list one tile (two entries) at a time
  // as a byte offset modulo the list length, instead of clamping and mapping
  // every index: tiles past the last page then read other pages of the
  // request, whose keys are masked and whose V is zeroed like any key past
  // kv_len.  pl4: byte offset of the next fetched tile's first entry.
  const int n_list = last_page + 1;
  const uint32_t n4 = 4u * (uint32_t)n_list;
  uint32_t pl4 = 4u * (uint32_t)((2 * (jt0 + (grp == 0 ? 3 : 2))) % n_list);
  auto list_at = [&](uint32_t off) __attribute__((always_inline)) {
    return ldu(reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(pages) + off));
  };
  auto fetch_next = [&](int64_t* tp) __attribute__((always_inline)) {
    if constexpr (PAGE16) {
      uint32_t p1 = pl4 + 4u;
      if (p1 >= n4) p1 -= n4;
      tp[0] = (int64_t)((uint64_t)(uint32_t)list_at(pl4) * pb32);
      tp[1] = (int64_t)((uint64_t)(uint32_t)list_at(p1) * pb32);
      pl4 += 8u;
      if (pl4 >= n4) pl4 -= n4;
      if (pl4 >= n4) pl4 -= n4;
    }
  };
  // One load instruction r (0..3) of wave wg of the loading group: K rows
  // and V^T chunks of instruction 4 r + wg of the tile (16 instructions of
  // 1 KiB per tile).  kp / vp: the tile's two page ids (16-slot pages).
  auto k_load = [&](char* kl, int jj, const int64_t* kp, int r) __attribute__((always_inline)) {
    if constexpr (PAGE16) {
      // key 8 r + 2 wg + h of the tile (page r / 2), chunk n ^ kswz(key)
      const int key = 8 * (r & 1) + 2 * wg + h;
      const uint32_t off = key * D * 2 + ((n ^ kswz(key)) << 4);
      lds_dma16_s(kbase_g + kp[r >> 1], off, kl + (4 * r + wg) * 1024);
    } else {
      const int ins = 4 * r + wg;
      const int u = ins * 64 + lane;
      const int key = u / NCH;
      const int c = (u % NCH) ^ kswz(key);
      const int keyg = jj + key;
      const int64_t pg = page_id(keyg >> pshift);
      lds_dma16(kbase_g + pg * page_bytes + (int64_t)(keyg & (psize - 1)) * D * 2 + c * 16,
                kl + ins * 1024);
    }
  };
  auto v_load = [&](char* vl, int jj, const int64_t* vp, int r) __attribute__((always_inline)) {
    if constexpr (PAGE16) {
      // keys 8 r .. 8 r + 7 of the tile (page r / 2), dim 64 wg + lane
      lds_dma16_s(vbase_g + vp[r >> 1] + 16 * (r & 1), (64 * wg + lane) * 32,
                  vl + (4 * r + wg) * 1024);
    } else {
      const int ins = 4 * r + wg;
      const int keyg = jj + 8 * (ins >> 2);
      const int d = 64 * (ins & 3) + lane;
      const int64_t pg = page_id(keyg >> pshift);
      lds_dma16(vbase_g + pg * page_bytes + (int64_t)d * psize * 2 + (keyg & (psize - 1)) * 2,
                vl + ins * 1024);
    }
  };
  auto v_tile_sanitize = [&](char* vl, int jj) __attribute__((always_inline)) {
    if (jj + KT <= kvl) return;
    rare_path();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ins = 4 * r + wg;
      const int jc = jj + 8 * (ins >> 2);
      if (jc + 8 > kvl) {
        bf16x8* cp = reinterpret_cast<bf16x8*>(vl + ins * 1024 + lane * 16);
        bf16x8 v = *cp;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (jc + e >= kvl) ? (__bf16)0.0f : v[e];
        *cp = v;
      }
    }
  };

  // ---- prologue: K(0) (group 0) and K(1) (group 1), then Q ----
  {
    int64_t p0[2] = {0, 0};
    fetch_pids(grp, p0);
#pragma unroll
    for (int r = 0; r < 4; ++r) k_load(grp == 0 ? kb0 : kb1, (jt0 + grp) * KT, p0, r);
    // 8 instructions per half, each 4 whole half-rows (16 lanes per row);
    // rows past qo_len read the last row of the request (never stored)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      const int t = min(t0 + w * tok_w + (row >> gs), qo_len - 1);
      const int hd = (kvh << gs) + (row & ((1 << gs) - 1));
      const char* g = reinterpret_cast<const char*>(
                          P.q + ((int64_t)(q_beg + t) * P.num_qo_heads + hd) * D) + c * 16;
      lds_dma16(g, qlo + i * 1024);
      lds_dma16(g + 256, qhi + i * 1024);
    }
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < KSR; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qlo + (qrd ^ (ks << 5)));
    // K(0), K(1) and every wave's Q landed; the Q scratch halves are read
    lds_barrier();
  }

  // The three K and three V tile buffers by role, rotated at the end of every
  // MFMA phase so that no phase computes a buffer index: during MFMA(u), K0,
  // K1, K2 hold K(u), K(u+1), K(u+2) and V0, V1, V2 hold V(u-1), V(u),
  // V(u+1); during ALU(j), which follows MFMA(j), K0 holds K(j+1) and V0, V1,
  // V2 hold V(j), V(j+1), V(j+2).
  char* K0 = kb0;
  char* K1 = kb1;
  char* K2 = kb2;
  char* V0 = vb2;
  char* V1 = vb0;
  char* V2 = vb1;
  // ALU(j): this group's loads, softmax of S(j) (if j is a tile), barrier.
  auto alu_phase = [&](int j) __attribute__((always_inline)) {
    int64_t tn[2] = {0, 0};
    fetch_next(tn);   // tile j + 3
    if (grp == 1) {
      if (j < 0) {
        rare_path();
        int64_t p0[2] = {0, 0};
        fetch_pids(0, p0);
#pragma unroll
        for (int r = 0; r < 4; ++r) v_load(V1, jt0 * KT, p0, r);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) v_load(V2, (jt0 + j + 2) * KT, tpid, r);
    }
    if (j >= 0 && j < ntiles) softmax((jt0 + j) * KT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(4 | 0x70 | 0xF00);  // vmcnt(4): the loads before the last landed
    asm volatile("" ::: "memory");
    if (grp == 1) v_tile_sanitize(V1, (jt0 + j + 1) * KT);
#pragma unroll
    for (int p = 0; p < 2; ++p) tpid[p] = tn[p];
    // first operands of MFMA(j+1): V(j) (resident since the end of slot
    // 2j), or K(0) before the first phase
    if (j >= 0) preload(std::true_type{}, V0, K0);
    else preload(std::false_type{}, V1, K0);
    // barrier with those three operand reads still in flight (lgkmcnt(3)):
    // LDS accesses complete in order, so every earlier one (the V zeroing
    // above) is done, and the buffers they read, V(j) and K(j+1), are not
    // refilled in the next slot.  Nor does the barrier wait for the scalar
    // page-id loads of this phase.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc37f);  // lgkmcnt(3); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // MFMA(u): PV(u-1) from V(u-1) (if u >= 1), QK(u) from K(u) (if u <
  // ntiles), operands preloaded.  Group 0 then loads K(u+2) into the buffer
  // of K(u-1), which both groups finished reading in the slot before, while
  // it waits at the barrier for group 1's softmax.
  auto mfma_phase = [&](int u, auto pv_c, auto qk_c) __attribute__((always_inline)) {
    // the wave in its MFMA phase takes issue priority over the softmax wave
    // on the same SIMD, so the matrix unit is not left waiting on VALU issue
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_seq(pv_c, qk_c, V0, K0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (decltype(qk_c)::value && grp == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) k_load(K2, (jt0 + u + 2) * KT, tpid, r);
    }
    lds_barrier();
    // the next tile's view of the rings
    char* const kt = K0;
    K0 = K1;
    K1 = K2;
    K2 = kt;
    char* const vt = V0;
    V0 = V1;
    V1 = V2;
    V2 = vt;
  };

  fetch_pids(grp == 0 ? 2 : 1, tpid);
  // group 1 starts with ALU(-1) (no softmax, the first V loads); group 0
  // with MFMA(0)
  // the first MFMA phase (QK only) and the last (PV only) are peeled off
  if (grp == 0) preload(std::false_type{}, V1, K0);
  else alu_phase(-1);
  mfma_phase(0, std::false_type{}, std::true_type{});
  for (int u = 1; u < ntiles; ++u) {
    alu_phase(u - 1);
    mfma_phase(u, std::true_type{}, std::true_type{});
  }
  alu_phase(ntiles - 1);
  mfma_phase(ntiles, std::true_type{}, std::false_type{});
  // tail: group 0 matches group 1's extra lead-in barrier
  if (grp == 0) lds_barrier();
  // every wave's tile loads landed: all of LDS is free
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if constexpr (OUT_BF16) {
    // O rows of this wave through 16 KiB of LDS: [row n][32 chunks of 16 B],
    // chunk c of row n at position c ^ n; then two whole rows per store
    char* const stg = w < 6 ? ((w >> 1) == 0 ? (w & 1 ? kb1 : kb0)
                               : (w >> 1) == 1 ? (w & 1 ? vb0 : kb2) : (w & 1 ? vb2 : vb1))
                            : qlds + (w - 6) * 16384;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v = {(__bf16)(oacc[db][4 * g] * inv), (__bf16)(oacc[db][4 * g + 1] * inv),
                    (__bf16)(oacc[db][4 * g + 2] * inv), (__bf16)(oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<bf16x4*>(stg + n * 512 + (((4 * db + g) ^ n) << 4) + 8 * h) = v;
      }
    // LDS operations of one wave complete in order: no wait between the
    // writes above and the reads below, only no compiler reordering
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    const int c = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 2 * i + (lane >> 5);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + r * 512 + ((c ^ r) << 4));
      const int t = t0 + w * tok_w + (r >> gs);
      if (t < qo_len) {
        const int hd = (kvh << gs) + (r & ((1 << gs) - 1));
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(P.o) +
                                   ((int64_t)(q_beg + t) * P.num_qo_heads + hd) * D + c * 8) = v;
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
