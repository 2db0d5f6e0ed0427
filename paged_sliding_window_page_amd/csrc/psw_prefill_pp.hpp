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
// Loads: group 0's ALU phase u loads K(u+2) and V(u+1) whole (8 load
// instructions per wave) into the buffers K(u-1) and V(u-2) left, waits for
// the loads of its previous ALU phase (vmcnt(8)), zeroes V(u)'s keys past
// kv_len in the chunks it loaded, and the barrier that follows publishes
// them: every tile is resident one full phase before its first reader.
#pragma once
#include "psw_attention.hpp"

namespace psw_dev {
namespace {

// global_load_lds_dwordx4 issued as inline assembly: 16 bytes per lane from
// gsrc into LDS at lds_base + 16 * lane.  The tile buffers are picked at run
// time, so the compiler could not tell these writes from the MFMA operand
// reads of other buffers and would wait for every one of them before each
// read; the kernel orders them itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void lds_dma16(const void* gsrc, const char* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory", "m0");
}

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
  constexpr int LPW = 2;           // load instructions per wave per tile half (K, and V)
  constexpr int AH = 2;            // LDS operand reads in flight ahead of the MFMAs

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
  auto kbuf = [&](int i) __attribute__((always_inline)) -> char* {
    i %= 3;
    return i == 0 ? kb0 : (i == 1 ? kb1 : kb2);
  };
  auto vbuf = [&](int i) __attribute__((always_inline)) -> char* {
    i %= 3;
    return i == 0 ? vb0 : (i == 1 ? vb1 : vb2);
  };

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

  bf16x8 qf[KSR];
  char* const qw = qlds + w * (KS - KSR) * 1024 + lane * 16;  // this lane's Q chunks in LDS
  {
    const __bf16* qrow =
        P.q + ((int64_t)(q_beg + (row_valid ? tok : 0)) * P.num_qo_heads + head) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      v = row_valid ? v : bf16x8{};
      if (ks < KSR) qf[ks] = v;
      else *reinterpret_cast<bf16x8*>(qw + (ks - KSR) * 1024) = v;
    }
  }

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
  // Group g loads instructions 8 g .. 8 g + 7 (keys 16 g .. 16 g + 15), wave
  // wg of the group instructions 8 g + 4 r + wg, r < LPW.
  auto page_id = [&](int idx) __attribute__((always_inline)) { return ldu(pages + min(idx, last_page)); };




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

  // MFMA phase: PV of the previous tile (if any), then QK of this one (if any);
  // LDS operand reads run AH MFMAs ahead.
  auto mfma_phase = [&](const char* vl, bool do_pv, const char* kl, bool do_qk) __attribute__((always_inline)) {
    if (do_pv) {
      constexpr int NV = NT * DB;
      bf16x8 a[AH + 1];
      // O block db takes its NT MFMAs back to back
      auto ld = [&](int i) __attribute__((always_inline)) {
        const int t = i % NT, db = i / NT;
        return *reinterpret_cast<const bf16x8*>(vl + vaddr0 + (2 * t * D + 32 * db) * 16);
      };
#pragma unroll
      for (int i = 0; i < AH; ++i) a[i] = ld(i);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i + AH < NV) a[(i + AH) % (AH + 1)] = ld(i + AH);
        oacc[i / NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % (AH + 1)], pb[i % NT],
                                                                oacc[i / NT], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_qk) {
      // K operands AH k-steps ahead; Q operands of the upper k-steps from LDS
      // on the same schedule
      bf16x8 a[AH + 1], qa[AH + 1];
      auto ld = [&](int ks) __attribute__((always_inline)) {
        if (ks >= KSR) qa[ks % (AH + 1)] = *reinterpret_cast<const bf16x8*>(qw + (ks - KSR) * 1024);
        a[ks % (AH + 1)] =
            *reinterpret_cast<const bf16x8*>(kl + (kaddr0 ^ ((ks & 7) << 5)) + (ks >> 3) * 256);
      };
#pragma unroll
      for (int i = 0; i < AH; ++i) ld(i);
      s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + AH < KS) ld(ks + AH);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % (AH + 1)],
                                                    ks < KSR ? qf[ks] : qa[ks % (AH + 1)], s, 0,
                                                    0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Softmax of S(t) (tile starting at key j0) into P(t); rescales O if the
  // running max rose past the slack.
  auto softmax = [&](int j0) __attribute__((always_inline)) {
    const bool full = wave_live && j0 >= k_lo && j0 + KT - 1 <= k_hi && j0 + KT - 1 <= w_pmin &&
                      (wl < 0 || w_pmax - j0 <= wl);
    float mx = -__builtin_inff();
    if (full) {
      float hi = -__builtin_inff(), lo = __builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hi = fmaxf(hi, s[r]);
        lo = fminf(lo, s[r]);
      }
      mx = c2 >= 0.0f ? hi * c2 : lo * c2;
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
    const bool need = __any(m_new > m_run + kRescaleSlack);
    const float m_use = need ? m_new : m_run;
    const float cmul = full ? c2 : 1.0f;
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], cmul, -m_use));
      lsum += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    if (need) {
      rare_path();
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    }
    l_run += lsum;
  };

  // ---- prologue: K(0), K(1), V(0) resident ----
  {
    const int j0 = jt0 * KT;
    // all 16 instructions of each tile, two per wave
    auto all_k = [&](char* kl, int jj) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < LPW; ++r) {
        const int ins = 2 * w + r;  // 0..15
        const int u = ins * 64 + lane;
        const int key = u / NCH;
        const int c = (u % NCH) ^ kswz(key);
        const int keyg = jj + key;
        const int64_t pg = page_id(keyg >> pshift);
        lds_dma16(kbase_g + pg * page_bytes + (int64_t)(keyg & (psize - 1)) * D * 2 + c * 16,
                   kl + ins * 1024);
      }
    };
    auto all_v = [&](char* vl, int jj) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < LPW; ++r) {
        const int ins = 2 * w + r;
        const int keyg = jj + 8 * (ins >> 2);
        const int d = 64 * (ins & 3) + lane;
        const int64_t pg = page_id(keyg >> pshift);
        lds_dma16(vbase_g + pg * page_bytes + (int64_t)d * psize * 2 + (keyg & (psize - 1)) * 2,
                   vl + ins * 1024);
      }
    };
    all_k(kb0, j0);
    all_k(kb1, j0 + KT);
    all_v(vb0, j0);
    __builtin_amdgcn_s_waitcnt(0);
    // zero V(0)'s keys past kv_len in the chunks this wave loaded
    if (j0 + KT > kvl) {
      rare_path();
#pragma unroll
      for (int r = 0; r < LPW; ++r) {
        const int ins = 2 * w + r;
        const int jc = j0 + 8 * (ins >> 2);
        if (jc + 8 > kvl) {
          bf16x8* cp = reinterpret_cast<bf16x8*>(vb0 + ins * 1024 + lane * 16);
          bf16x8 v = *cp;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (jc + e >= kvl) ? (__bf16)0.0f : v[e];
          *cp = v;
        }
      }
    }
    __syncthreads();
  }

  // Tile loads are issued by group 0 only, in its ALU phases: ALU(j) loads
  // K(j+2) and V(j+1) whole (8 instructions per wave), waits for the loads
  // of ALU(j-1) and zeroes V(j) past kv_len.  The page ids are read through
  // the scalar cache at the start of the ALU phase before.
  int64_t kpid[2] = {0, 0}, vpid[2] = {0, 0};
  auto fetch_pids = [&](int k_tile, int v_tile, int64_t* kp, int64_t* vp)
                        __attribute__((always_inline)) {
    if constexpr (PAGE16) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        kp[p] = page_id(((jt0 + k_tile) * KT >> 4) + p);
        vp[p] = page_id(((jt0 + v_tile) * KT >> 4) + p);
      }
    }
  };
  // the 16 instructions of a tile, four per wave of group 0
  auto k_tile_load = [&](char* kl, int jj, const int64_t* kp) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ins = 4 * r + wg;
      const int u = ins * 64 + lane;
      const int key = u / NCH;
      const int c = (u % NCH) ^ kswz(key);
      const int keyg = jj + key;
      const int64_t pg = PAGE16 ? kp[ins >> 3] : page_id(keyg >> pshift);
      lds_dma16(kbase_g + pg * page_bytes + (int64_t)(keyg & (psize - 1)) * D * 2 + c * 16,
                 kl + ins * 1024);
    }
  };
  auto v_tile_load = [&](char* vl, int jj, const int64_t* vp) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ins = 4 * r + wg;
      const int keyg = jj + 8 * (ins >> 2);
      const int d = 64 * (ins & 3) + lane;
      const int64_t pg = PAGE16 ? vp[ins >> 3] : page_id(keyg >> pshift);
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

  // ALU(j): softmax of S(j) (if j is a tile), group 0's loads, barrier.
  // KB/VB: buffers of K(j+2), V(j+1); VP: buffer of V(j).
  auto alu_phase = [&](int j, int KB, int VB, int VP) __attribute__((always_inline)) {
    int64_t kn[2] = {0, 0}, vn[2] = {0, 0};
    if (grp == 0) {
      fetch_pids(j + 3, j + 2, kn, vn);
      k_tile_load(kbuf(KB), (jt0 + j + 2) * KT, kpid);
      v_tile_load(vbuf(VB), (jt0 + j + 1) * KT, vpid);
    }
    if (j >= 0 && j < ntiles) softmax((jt0 + j) * KT);
    if (grp == 0) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(8 | 0x70 | 0xF00);  // vmcnt(8): ALU(j-1)'s loads landed
      asm volatile("" ::: "memory");
      v_tile_sanitize(vbuf(VP), (jt0 + j) * KT);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        kpid[p] = kn[p];
        vpid[p] = vn[p];
      }
    }
    lds_barrier();
  };
  // MFMA(u): PV(u-1) from V(u-1), QK(u) from K(u)
  auto mfma_phase_t = [&](int u, int KB, int VBP) __attribute__((always_inline)) {
    mfma_phase(vbuf(VBP), u >= 1, kbuf(KB), u < ntiles);
    lds_barrier();
  };
  // loop body u >= 1 (compile-time u % 3 picks the buffers)

  fetch_pids(2, 1, kpid, vpid);
  // group 1 runs an empty ALU(-1) first; group 0 starts with MFMA(0)
  for (int u = 0; u <= ntiles; ++u) {
    if (grp == 1 || u > 0) alu_phase(u - 1, u + 1, u, u + 2);
    mfma_phase_t(u, u, u + 2);
  }
  // tail: group 0 matches group 1's extra lead-in barrier
  if (grp == 0) lds_barrier();
  // no tile loads in flight past this point
  __builtin_amdgcn_s_waitcnt(0);

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_valid) return;
  const float inv = 1.0f / l_tot;
  const int64_t orow = ((int64_t)(q_beg + tok) * P.num_qo_heads + head) * D + 4 * h;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int off = 32 * db + 8 * g;
      if constexpr (OUT_BF16) {
        bf16x4 v = {(__bf16)(oacc[db][4 * g] * inv), (__bf16)(oacc[db][4 * g + 1] * inv),
                    (__bf16)(oacc[db][4 * g + 2] * inv), (__bf16)(oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.o) + orow + off) = v;
      } else {
        f32x4 v = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                   oacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(P.o) + orow + off) = v;
      }
    }
}

}  // namespace
}  // namespace psw_dev
