// Paged attention for gfx950: bf16 MFMA, online softmax, K/V gathered through
// a page table.  This kernel template serves the split-KV form of one-token
// decode when a GQA group is wider than the decode kernel's 16 query heads per
// KV head (PR "feat(gemma4): paged KV serving across both attention
// families", Description: serving decodes through the prefill entry), at head
// dim 256 and 512; the pieces write partial results that merge_kernel
// combines.  (The prefills have kernels of their own: psw_prefill_pp.hpp at
// head_dim 256, psw_prefill512.hpp at head_dim 512; the template's non-split
// form is not instantiated.)
//
// Work-group: 4 waves of 32 query rows (at head_dim 512 two waves share a row
// group, each with half the dims: 64 rows), rows = tokens x the group's heads
// of one KV head, so the group's heads share every K/V tile.  Per KV tile (64
// keys at D=256, 32 at D=512):
//   S^T[key][row] = K Q^T     v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in
//                             registers (B)
//   P = exp2(S*scale*log2e - m) with a lazily raised running max m
//   O^T[d][row]  += V^T P^T   V^T from LDS (A), P^T straight from the S^T
//                             accumulators (B), O^T in accumulator registers
// The K rows feeding S^T are read in a permuted order (kperm below) chosen so
// that the keys a lane holds in its S^T accumulators are exactly the 8
// consecutive keys its P^T operand needs; no data moves between the two MFMAs.
//
// Tiles are fetched with global_load_lds_dwordx4 (16 B per lane straight into
// LDS, no VGPR staging) into a double buffer; the next tile's loads are in
// flight while the current one is multiplied.  LDS tiles are XOR-swizzled so
// that the MFMA operand reads (ds_read_b128) hit distinct banks.  Only tiles
// that intersect a row's window are visited; whole tiles inside every row's
// window skip the element mask.
#pragma once
#include <type_traits>

#include "psw_device.hpp"

namespace psw_dev {
namespace {

constexpr float kNegBig = -1.0e30f;     // finite "minus infinity" for running maxima
constexpr float kRescaleSlack = 8.0f;   // log2 units: rescale O only past a 256x rise
constexpr int kQkAhead = 2;  // K operand reads in flight ahead of the QK MFMAs (k-steps)
constexpr int kPvAhead = 2;  // V^T operand reads in flight ahead of the PV MFMAs

__device__ __forceinline__ int kperm(int m) {
  // S^T row m (0..31) -> key within the 32-key block.  With the 32x32 MFMA
  // accumulator layout (lane half h, register r holds row 8*(r/4) + 4*h + r%4)
  // this puts key 16*(r/8) + 8*h + (r%8) in register r of half h.
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// XOR swizzle of the 16-byte chunk index inside a K row (bank spread).
__device__ __forceinline__ int kswz(int key) {
  return (key & 3) | ((key >> 1) & 4) | ((key << 1) & 8);
}

// The tile loads below write m0 and name it among their clobbers; clang
// treats m0 as reserved and warns that it may not be preserved across the
// statement, which is what the clobber says.  The warning is silenced here
// only.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// global_load_lds_dwordx4 issued as inline assembly: 16 bytes per lane from
// gsrc into LDS at lds_base + 16 * lane.  The compiler does not track these
// loads: a kernel that uses them orders them itself, with explicit vmcnt
// waits and barriers, against the LDS reads of the buffers they fill (the
// compiler would otherwise wait for every load in flight before unrelated
// LDS reads, and rebuild a 64-bit vector address for every load).
__device__ __forceinline__ void lds_dma16(const void* gsrc, const char* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory", "m0");
}

// The same with a wave-uniform 64-bit base and a 32-bit per-lane offset (the
// saddr form), which keeps one VGPR per address instead of two.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, const char* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void lds_load16(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

// Wave-uniform read of read-only metadata through the scalar data cache
// (constant address space), so it never waits behind vector memory traffic.
template <typename T>
__device__ __forceinline__ T ldu(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<const __attribute__((address_space(4))) char*>(
          (const __attribute__((address_space(4))) char*)p));
}

// Pin the computation of v before this point (an empty volatile use), so
// later passes cannot sink it out of the block it is interleaved into.
__device__ __forceinline__ void pin(float v) { asm volatile("" ::"v"(v)); }

// Work-group barrier over LDS traffic only: waits for this wave's own LDS
// reads and writes (lgkmcnt) but not for tile loads still in flight into LDS
// (a workgroup fence would also wait for those, vmcnt).  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The value of lane l ^ 32 (the other half of the wave), through
// v_permlane32_swap (a VALU lane swap, no LDS round trip).  Swapping x with
// itself leaves the low half of x in both halves of one register and the high
// half in both halves of the other, so their max is the max over l and l ^ 32.
__device__ __forceinline__ float max_with_partner_half(float x) {
  float lo = x, hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
  return fmaxf(lo, hi);
}

// A copy of v the compiler cannot see through (values derived from it are
// recomputed where they are used instead of being held in registers).
__device__ __forceinline__ int opaque(int v) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// Keep the compiler from if-converting a rare branch into straight-line code.
__device__ __forceinline__ void rare_path() { asm volatile("" ::: "memory"); }

// PAGE16: the serving page size (16 slots), for which the page of every load
// instruction is a compile-time function of the tile; otherwise page_size is a
// runtime power of two >= 8.
template <int D, bool SPLIT, bool OUT_BF16, bool PAGE16>
__global__ __launch_bounds__(256, 1) void attention_kernel(AttnParams P) {
  // Four waves of 32 query rows.  At head_dim 512 the dims are split between
  // the two waves of a row group (each keeps O^T and Q for 256 dims, which
  // leaves room in its registers) and the pair's partial scores are summed
  // through LDS: 2 row groups x 2 dim halves, 64 rows per work-group.
  constexpr int DH = D == 512 ? 2 : 1;    // dim halves
  constexpr int DW = D / DH;              // dims per wave
  constexpr int NW = 4;                   // waves per work-group
  constexpr int RG = NW / DH;             // row groups
  constexpr int KT = D == 256 ? 64 : 32;  // keys per tile
  constexpr int NCH = D / 8;              // 16-B chunks per K row
  constexpr int KBLK = KT / 32;           // S^T 32-key blocks per tile
  constexpr int NT = KT / 16;             // PV steps (16 keys each) per tile
  constexpr int DB = DW / 32;             // O^T 32-row blocks per wave
  constexpr int KS = DW / 16;             // QK k-steps per wave
  constexpr int TILE = KT * D * 2;        // bytes of one K (or V^T) tile: 32 KiB
  constexpr int ROUNDS = TILE / (NW * 64 * 16);
  constexpr int KEYS_PER_LOAD = 1024 / (D * 2);  // keys one K load instruction covers
  static_assert((NW * KEYS_PER_LOAD) % 16 == 0 || 16 % (NW * KEYS_PER_LOAD) == 0, "");

  // K and V^T tiles have separate double buffers: K[t+1] must be resident
  // while V[t-1] is still being read (see the pipeline below).
  // Four distinct arrays (not one indexed array) so that the compiler can
  // tell the stage being read from the stage the in-flight DMA is writing.
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE];
  // partial S^T of each wave, [step parity][wave][register quad][lane]
  // (conflict-free); two copies, so that a wave writes the next tile's while
  // its partner may still be reading the previous step's, with no barrier
  // between them
  __shared__ f32x4 xs[2][DH > 1 ? NW : 1][4 * KBLK][64];

  const int lane = threadIdx.x & 63;
  // wave index, explicitly wave-uniform so that per-wave address math is scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = w & (RG - 1);  // row group
  const int dh = w / RG;        // dim half (0 unless D == 512)
  const int n = lane & 31;
  const int h = lane >> 5;
  const int hkv = P.num_kv_heads;
  const int item = blockIdx.x / hkv;
  const int kvh = blockIdx.x - item * hkv;
  const int b = ldu(P.items + 4 * item + 0);
  // split mode (one query per request): field 1 is the partial slot, t0 = 0
  const int t0 = SPLIT ? 0 : ldu(P.items + 4 * item + 1);
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
  const int tok_w = 32 >> gs;            // tokens per wave
  const int wl = P.window_left;

  // this lane's query row: token t0 + tl, head kvh*group + hh
  const int tl = rg * tok_w + (n >> gs);
  const int hh = n & ((1 << gs) - 1);
  const int tok = t0 + tl;
  const bool row_valid = tok < qo_len;
  const int pos = start + tok;
  const int head = (kvh << gs) + hh;
  // keys this lane's row may see: [lo_n, hi_n] (empty for padding rows)
  const int hi_n = row_valid ? min(k_hi, pos) : -1;
  const int lo_n = max(k_lo, wl >= 0 ? pos - wl : 0);
  // the same range, over every row of this wave (for whole-tile decisions)
  const int wt0 = t0 + rg * tok_w;
  const int w_pmin = start + wt0;
  const int w_pmax = start + min(wt0 + tok_w, qo_len) - 1;
  const bool wave_live = wt0 < qo_len;

  bf16x8 qf[KS];
  {
    const __bf16* qrow = P.q + ((int64_t)(q_beg + (row_valid ? tok : 0)) * P.num_qo_heads + head) * D +
                         DW * dh + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      qf[ks] = row_valid ? v : bf16x8{};
    }
  }

  const char* kbase_g = reinterpret_cast<const char*>(P.pool + P.layer_off + (int64_t)kvh * P.ps.head);
  const char* vbase_g = kbase_g + P.ps.kv * 2;
  const int pshift = PAGE16 ? 4 : P.ps.page_shift;
  const int psize = PAGE16 ? 16 : P.ps.page_size;
  const int64_t page_bytes = P.ps.page * 2;

  const int jt0 = k_lo / KT;
  const int jt1 = k_hi / KT;
  const int ntiles = jt1 - jt0 + 1;

  // ---- tile loads: every load instruction reads from one page ----
  // K tile in LDS: [key][chunk ^ kswz(key)] of 16-byte chunks (D/8 per key).
  // V^T tile in LDS: [k8][d] of 16-byte chunks, chunk (k8, d) holding the 8
  // keys 8*k8 .. 8*k8+7 of dim d.  Eight lanes reading consecutive d at one k8
  // touch consecutive 16-byte chunks, so no swizzle is needed.
  // Load instruction r of wave w covers K keys (r*4+w)*KEYS_PER_LOAD.. and the
  // V^T chunks k8 = (r*4+w)*64 / D, d = ((r*4+w)*64) % D + lane: one page each.
  int koff[ROUNDS], voff[ROUNDS];   // per-lane byte offsets inside the page
  int kpg[ROUNDS], vpg[ROUNDS];     // page of the tile (wave-uniform)
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int ins = r * NW + w;
    const int u = ins * 64 + lane;
    const int key = u / NCH;
    const int c = (u % NCH) ^ kswz(key);
    kpg[r] = (ins * KEYS_PER_LOAD) >> pshift;
    koff[r] = (key & (psize - 1)) * D * 2 + c * 16;
    const int k8 = (ins * 64) / D;
    const int d = (ins * 64) % D + lane;
    vpg[r] = (8 * k8) >> pshift;
    voff[r] = d * psize * 2 + ((8 * k8) & (psize - 1)) * 2;
  }
  // Page ids of a tile: pages are clamped to the request's last page (keys past
  // kv_len are masked, and their V values zeroed after landing).  With 16-slot
  // pages the pipeline fetches the ids one step ahead with a vector load
  // (lanes [0, NPG): the V tile's pages, lanes [NPG, 2 NPG): the K tile's)
  // and reads them back with readlane, so issuing a tile never waits on the
  // page table.  Other page sizes read the ids per load, through the scalar
  // cache.
  constexpr int NPG = KT / 8;  // most pages a tile can touch (page_size >= 8)
  constexpr int NPP = PAGE16 ? KT / 16 : 1;
  const PageRing ring = page_ring(last_page + 1, kvl, pshift);
  auto page_id = [&](int j0, int p) { return ldu(pages + ring((j0 >> pshift) + p)); };
  auto load_pids = [&](int tv, int tk) {  // tile indices of the V and K tiles
    int r = 0;
    if (lane < 2 * NPG) {
      const int jt = (jt0 + (lane < NPG ? tv : tk)) * KT;
      r = pages[ring((jt >> pshift) + (lane & (NPG - 1)))];
    }
    return r;
  };
  // One load instruction (round r) of a K or V^T tile.  PAGE16: pp holds the
  // base pointer of each of the tile's pages; otherwise the page is looked up
  // per round.
  auto k_round = [&](char* kl, const char* const* pp, auto pg, int j0, int r) {
    if constexpr (PAGE16) {
      lds_dma16_s(pp[(r * NW * KEYS_PER_LOAD) >> 4], (uint32_t)koff[r], kl + (r * NW + w) * 1024);
    } else {
      const char* src = kbase_g + (int64_t)pg(kpg[r]) * page_bytes +
                        (KT < psize ? (j0 & (psize - 1)) * D * 2 : 0);
      lds_load16(src + koff[r], kl + (r * NW + w) * 1024);
    }
  };
  auto v_round = [&](char* vl, const char* const* pp, auto pg, int j0, int r) {
    if constexpr (PAGE16) {
      lds_dma16_s(pp[(8 * ((r * NW * 64) / D)) >> 4], (uint32_t)voff[r], vl + (r * NW + w) * 1024);
    } else {
      const char* src =
          vbase_g + (int64_t)pg(vpg[r]) * page_bytes + (KT < psize ? (j0 & (psize - 1)) * 2 : 0);
      lds_load16(src + voff[r], vl + (r * NW + w) * 1024);
    }
  };
  // Copy of v made by an opaque move, issued where v's load is known to have
  // landed: later readlanes of the copy need no wait (the compiler cannot
  // track the load's completion across loop iterations and would otherwise
  // wait for every load in flight).
  auto settled = [](int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
  };
  auto tile_pages = [&](const char* base, auto pg, const char** pp) {
    if constexpr (PAGE16) {
#pragma unroll
      for (int p = 0; p < NPP; ++p)  // 32-bit factors: pages are below 4 GiB
        pp[p] = base + (uint64_t)(uint32_t)pg(p) * (uint32_t)page_bytes;
    }
  };
  auto issue_k = [&](char* kl, int j0, auto pg) {
    const char* pp[NPP];
    tile_pages(kbase_g, pg, pp);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) k_round(kl, pp, pg, j0, r);
  };
  // Zero, in the V^T chunks this lane loaded itself, the keys at or past
  // kv_len (their pool slots may hold anything, NaN included, and 0 * NaN would
  // leak into O).  Called after this wave's loads have landed.
  auto sanitize = [&](char* vl, int j0) {
    if (j0 + KT <= kvl) return;
    rare_path();
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int jc = j0 + 8 * (((r * NW + w) * 64) / D);
      if (jc + 8 > kvl) {
        bf16x8* cp = reinterpret_cast<bf16x8*>(vl + (r * NW + w) * 1024 + lane * 16);
        bf16x8 v = *cp;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (jc + e >= kvl) ? (__bf16)0.0f : v[e];
        *cp = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- per-lane LDS operand addresses ----
  // K row of S^T row n in block kb: key 32*kb + kperm(n); its 16-B chunk 2*ks+h
  // sits at position (2*ks+h) ^ kswz(key).  Writing sw = kswz(key), that is
  // 2*(ks ^ (sw>>1)) + (h ^ (sw&1)) for ks < 8, so the byte offset is
  // kaddr0 ^ (ks << 5), plus 256 for every further 8 k-steps.
  const int krow = kperm(n);
  const int ksw = kswz(krow);
  const int kaddr0 = krow * NCH * 16 + 16 * (h ^ (ksw & 1)) + 32 * (ksw >> 1);
  // this wave's dims start DW * dh into the row: whole 256-byte swizzle groups
  const int kdh = DW * 2 * dh;
  // V^T operand of PV step t, O^T block db: row d = 32*db + n, keys
  // 16t + 8h .. +7, i.e. chunk (k8 = 2t + h, d).
  const int vaddr0 = (h * D + DW * dh + n) * 16;
  auto vaddr = [&](int t, int db) { return vaddr0 + (2 * t * D + 32 * db) * 16; };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.0f;
  bf16x8 pprev[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) pprev[t] = bf16x8{};
  // scores enter the softmax as s * sm_scale * log2(e); the running max is
  // kept in those units.  A negative scale flips which raw score is largest.
  const float c2 = P.scale_log2;

  // O^T += V^T P^T for one tile (V^T operands read two steps ahead).
  auto pv = [&](const char* vl, const bf16x8* pb, auto extra) {
    constexpr int NSTEP = NT * DB;
    constexpr int RA = kPvAhead + 1;
    bf16x8 a[RA];
    auto ld = [&](int i) { return *reinterpret_cast<const bf16x8*>(vl + vaddr(i / DB, i % DB)); };
#pragma unroll
    for (int i = 0; i < kPvAhead; ++i) a[i] = ld(i);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + kPvAhead < NSTEP) a[(i + kPvAhead) % RA] = ld(i + kPvAhead);
      oacc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % RA], pb[i / DB], oacc[i % DB],
                                                              0, 0, 0);
      extra(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Row max of raw scores in softmax units, with or without the element mask.
  // Register r of block kb holds key j0 + 32*kb + 16*(r/8) + 8*h + r%8.
  auto tile_max = [&](f32x16* s, bool masked, int j0) {
    float mx = -__builtin_inff();
    if (!masked) {
      // max of s * c2: c2 times the max of s, or of the min for a negative c2
      float e = s[0][0];
      if (c2 >= 0.0f) {
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) e = fmaxf(e, s[kb][r]);
      } else {
        rare_path();
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) e = fminf(e, s[kb][r]);
      }
      mx = e * c2;
    } else {
      rare_path();
      const int kb0 = j0 + 8 * h - lo_n;
      const unsigned span = (unsigned)(hi_n - lo_n);
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned rel = (unsigned)(kb0 + 32 * kb + 16 * (r >> 3) + (r & 7));
          const float v = rel <= span ? s[kb][r] * c2 : -__builtin_inff();
          s[kb][r] = v;   // masked tiles keep scaled scores
          mx = fmaxf(mx, v);
        }
    }
    return max_with_partner_half(mx);
  };

  // ---- pipeline ----
  // Scores run one tile ahead of the softmax: step t computes the softmax of
  // tile t interleaved with the QK MFMAs of tile t+1 (the VALU and the matrix
  // unit work side by side), then O += P(t) V(t).  Tile t's K sits in K buffer
  // t % 2 and its V^T in V buffer t % 2; the loads of K[t+2] and V[t+1] go
  // into the buffers that K[t] and V[t-1] left, spread over the QK MFMAs, and
  // every wave waits for its own loads at the end of the step, before the
  // barrier that makes them visible.
  auto qk_mfma = [&](f32x16* sacc, int ks, bf16x8 (*a)[KBLK]) {
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb)
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % (kQkAhead + 1)][kb], qf[ks],
                                                         sacc[kb], 0, 0, 0);
  };
  auto qk_ld = [&](const char* kl, int ks, bf16x8* dst) {
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb)
      dst[kb] = *reinterpret_cast<const bf16x8*>(
          kl + (kaddr0 ^ ((ks & 7) << 5)) + (ks >> 3) * 256 + kb * 32 * NCH * 16 + kdh);
  };
  // partial scores of the other dim half (head_dim 512): write, barrier, add
  auto xs_put = [&](const f32x16* sacc, int xb) {
    if constexpr (DH > 1) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xs[xb][w][4 * kb + c][lane] = f32x4{sacc[kb][4 * c], sacc[kb][4 * c + 1],
                                              sacc[kb][4 * c + 2], sacc[kb][4 * c + 3]};
    }
  };
  auto xs_add = [&](f32x16* sacc, int xb) {
    // a + b is the same float in both waves of a pair, so both run identical
    // softmaxes
    if constexpr (DH > 1) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 o = xs[xb][w ^ RG][4 * kb + c][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[kb][4 * c + i] += o[i];
        }
    }
  };

  f32x16 s[KBLK];   // scores of the tile whose softmax runs next
  int pid = 0;      // page ids of the loads of the coming step (16-slot pages)
  {
    // prologue: K[0], V[0], K[1] resident, S(0) computed
    const int j0 = jt0 * KT;
    if constexpr (PAGE16) pid = load_pids(1, 2);
    issue_k(k_lds0, j0, [&](int p) { return page_id(j0, p); });
    {
      const char* pp[NPP];
      tile_pages(vbase_g, [&](int p) { return page_id(j0, p); }, pp);
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r)
        v_round(v_lds0, pp, [&](int p) { return page_id(j0, p); }, j0, r);
    }
    if (ntiles > 1) issue_k(k_lds1, j0 + KT, [&](int p) { return page_id(j0 + KT, p); });
    __builtin_amdgcn_s_waitcnt(0);
    sanitize(v_lds0, j0);
    __syncthreads();
    if constexpr (PAGE16) pid = settled(pid);
    bf16x8 a[kQkAhead + 1][KBLK];
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kQkAhead; ++ks) qk_ld(k_lds0, ks, a[ks]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + kQkAhead < KS) qk_ld(k_lds0, ks + kQkAhead, a[(ks + kQkAhead) % (kQkAhead + 1)]);
      qk_mfma(s, ks, a);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DH > 1) {
      xs_put(s, 1);
      lds_barrier();
      xs_add(s, 1);
    }
  }

  // FULL: a step with a next tile and loads of V[t+1] and K[t+2], known at
  // compile time, so that no MFMA or load of the step sits behind a branch
  // (with run-time conditions the compiler also gave up tracking the LDS
  // reads and waited for all of them before every MFMA)
  auto step = [&](auto ST, int it, auto FULL) {
    constexpr int st = decltype(ST)::value;
    constexpr bool full_c = decltype(FULL)::value;
    char* kfree = st ? k_lds1 : k_lds0;   // K[t] (used) -> K[t+2]
    char* knext = st ? k_lds0 : k_lds1;   // K[t+1]
    char* vcur = st ? v_lds1 : v_lds0;    // V[t]
    char* vfree = st ? v_lds0 : v_lds1;   // V[t-1] (used) -> V[t+1]
    const int j0 = (jt0 + it) * KT;
    const bool has_next = full_c || it + 1 < ntiles;
    const bool load_v = full_c || it + 1 < ntiles;
    const bool load_k = full_c || it + 2 < ntiles;
    // page ids of V[t+2] and K[t+3] for the next step (16-slot pages)
    const int pid_next = PAGE16 ? load_pids(it + 2, it + 3) : 0;
    auto pg_v = [&](int p) { return page_id(j0 + KT, p); };
    auto pg_k = [&](int p) { return page_id(j0 + 2 * KT, p); };
    const char* vpp[NPP];
    const char* kpp[NPP];
    tile_pages(vbase_g, [&](int p) { return __builtin_amdgcn_readlane(pid, p); }, vpp);
    tile_pages(kbase_g, [&](int p) { return __builtin_amdgcn_readlane(pid, NPG + p); }, kpp);

    f32x16 s2[KBLK];   // scores of tile t+1
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) s2[kb] = f32x16{};
    bf16x8 a[kQkAhead + 1][KBLK];
    if (has_next) {
#pragma unroll
      for (int ks = 0; ks < kQkAhead; ++ks) qk_ld(knext, ks, a[ks]);
    }
    // the first MFMAs of QK(t+1) go out before the row max of tile t is
    // reduced, so the matrix unit has work while the VALU does it
    constexpr int KS0 = 4;
    auto qk_step = [&](int ks) {
      if (has_next) {
        if (ks + kQkAhead < KS)
          qk_ld(knext, ks + kQkAhead, a[(ks + kQkAhead) % (kQkAhead + 1)]);
        qk_mfma(s2, ks, a);
      }
    };
    // the loads of V[t+1] go out over the QK MFMAs, those of K[t+2] over the
    // PV MFMAs, so the per-CU load path is busy for the whole step
    auto load_round = [&](int ks) {
      constexpr int PER = KS / ROUNDS;
      if (ks % PER == 0 && load_v) v_round(vfree, vpp, pg_v, j0 + KT, ks / PER);
    };
#pragma unroll
    for (int ks = 0; ks < KS0; ++ks) {
      qk_step(ks);
      load_round(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    // softmax of tile t: row max, running max, exponentials (spread over the
    // remaining QK MFMAs)
    const bool full = wave_live && j0 >= k_lo && j0 + KT - 1 <= k_hi && j0 + KT - 1 <= w_pmin &&
                      (wl < 0 || w_pmax - j0 <= wl);
    const float tmax = tile_max(s, !full, j0);
    const float m_new = fmaxf(m_run, tmax);
    const bool need = __any(m_new > m_run + kRescaleSlack);
    const float m_use = need ? m_new : m_run;
    const float cmul = full ? c2 : 1.0f;
    float lsum = 0.0f;
    constexpr int NE = KBLK * 16;  // exponentials per lane
#pragma unroll
    for (int ks = KS0; ks < KS; ++ks) {
      qk_step(ks);
      load_round(ks);
#pragma unroll
      for (int e = (ks - KS0) * NE / (KS - KS0); e < (ks - KS0 + 1) * NE / (KS - KS0); ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 4][e & 15], cmul, -m_use));
        s[e >> 4][e & 15] = p;
        lsum += p;
        pin(p);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[t][i] = (__bf16)s[t >> 1][8 * (t & 1) + i];
    pin(lsum);
    if (need) {
      rare_path();
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    }
    l_run += lsum;
    // O += P(t) V(t)
    pv(vcur, pb, [&](int i) {
      constexpr int PER = NT * DB / ROUNDS;
      if (i % PER == 0 && load_k) k_round(kfree, kpp, pg_k, j0 + 2 * KT, i / PER);
    });
    // hand over: tile t+1's partial scores to the partner wave (the copy of
    // this step's parity: the partner read it two steps back, before the
    // last barrier), this wave's loads landed and zeroed past kv_len, then
    // the barrier
    xs_put(s2, st);
    __builtin_amdgcn_s_waitcnt(0);
    if (load_v) sanitize(vfree, j0 + KT);
    __syncthreads();
    xs_add(s2, st);
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) s[kb] = s2[kb];
    if constexpr (PAGE16) pid = settled(pid_next);
  };
  // steps with two more tiles after them in pairs (buffer parity is a
  // template argument), then the last one to three tiles
  int it = 0;
  for (; it + 3 < ntiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it, std::true_type{});
    step(std::integral_constant<int, 1>{}, it + 1, std::true_type{});
  }
  if (it < ntiles) step(std::integral_constant<int, 0>{}, it, std::false_type{});
  if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1, std::false_type{});
  if (it + 2 < ntiles) step(std::integral_constant<int, 0>{}, it + 2, std::false_type{});

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_valid) return;
  // lane (n, h), O^T block db, register r holds d = 32*db + 8*(r/4) + 4*h + r%4
  if constexpr (SPLIT) {
    const int slot = ldu(P.items + 4 * item + 1);
    const int64_t base = ((int64_t)slot * P.num_qo_heads + head);
    float* po = P.part_o + base * D + DW * dh + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * g) = v;
      }
    if (h == 0 && dh == 0) {
      P.part_ml[base * 2 + 0] = m_run;
      P.part_ml[base * 2 + 1] = l_tot;
    }
  } else {
    const float inv = 1.0f / l_tot;
    const int64_t orow = ((int64_t)(q_beg + tok) * P.num_qo_heads + head) * D + DW * dh + 4 * h;
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
}

// Combines the split-KV partials of one (request, head): with per-split running
// max m_s (log2 units), sum l_s and unnormalised o_s,
//   O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D / 4) void merge_kernel(MergeParams P) {
  const int b = blockIdx.y;  // request of this launch
  const int head = blockIdx.x;
  const int first = P.req[3 * b];
  const int ns = P.req[3 * b + 1];
  const int qrow = P.req[3 * b + 2];
  const int nh = P.num_qo_heads;
  const float* const part_o = P.part_o;
  const float* const part_ml = P.part_ml;
  // every argument read in one round of loads, before the branch below
  asm volatile("" ::"s"(first), "s"(ns), "s"(qrow), "s"(nh), "s"(part_o), "s"(part_ml));
  if (ns == 0) return;  // the decode kernel wrote this request's O itself
  // One pass with a running maximum: 16 splits at a time, all of their loads
  // issued first, so a request with up to 16 splits costs one memory round
  // trip after the launch arguments.
  constexpr int U = 16;
  const float* ml = part_ml + ((int64_t)first * nh + head) * 2;
  const int64_t ml_stride = 2 * (int64_t)nh;
  const int d = 4 * threadIdx.x;
  const float* po = part_o + ((int64_t)first * nh + head) * D + d;
  const int64_t po_stride = (int64_t)nh * D;
  float M = kNegBig, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < ns; s0 += U) {
    float m[U], l[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, ns - 1);  // past the end: repeat the last split (weight 0 below)
      m[u] = ml[sp * ml_stride];
      l[u] = ml[sp * ml_stride + 1];
      v[u] = *reinterpret_cast<const f32x4*>(po + sp * po_stride);
    }
    float mx = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = s0 + u < ns ? fmaxf(mx, m[u]) : mx;
    const float r = __builtin_amdgcn_exp2f(M - mx);  // rescale what is summed so far
    L *= r;
    acc *= r;
    M = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = s0 + u < ns ? __builtin_amdgcn_exp2f(m[u] - M) : 0.0f;
      L += wgt * l[u];
      acc += wgt * v[u];
    }
  }
  const float inv = 1.0f / L;
  const int64_t orow = ((int64_t)qrow * nh + head) * D + d;
  if constexpr (OUT_BF16) {
    bf16x4 v = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                (__bf16)(acc[3] * inv)};
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.o) + orow) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(P.o) + orow) = acc * inv;
  }
}

}  // namespace
}  // namespace psw_dev
