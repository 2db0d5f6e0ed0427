// One-token decode through the paged prefill entries (PR "feat(gemma4): paged KV
// serving across both attention families", Description: serving decodes by
// calling the prefill entry with one query per request).
//
// Work: each work-group (one KV head) runs a short list of items, each a
// (request, key range) piece.  A piece that is a whole request writes O
// itself; the pieces of a request cut between work-groups write an
// unnormalised partial (o, running max in log2 units, sum) to their slot and
// merge_kernel combines them.  The host cuts the batch's keys into equal
// contiguous shares, one per work-group and at most four waves' worth per CU
// (all of them resident at once), so every work-group streams the same number
// of tiles and the launch ends together.
//
// Decode streams every K/V byte once and uses it for at most 16 query rows,
// so the kernel is laid out for the memory stream, not for the matrix cores:
//   * head_dim is split across the waves of the work-group, 128 dims each
//     (2 waves at 256, 4 at 512), so per-wave state stays small (O^T 32
//     registers, Q 16, one K/V tile part 64) and two waves fit per SIMD;
//   * tiles of 32 keys go straight from HBM into MFMA operand registers,
//     double-buffered: the next tile's loads (and the page ids of the one
//     after) are in flight while the current one is multiplied.  No LDS
//     staging of K or V;
//   * V pages are dim-major ([dim][slot]), so a lane's V^T operand (one dim, 8
//     consecutive keys) is a single 16-byte load;
//   * S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys x rows) is computed as two
//     16-key blocks whose K rows are read in the order that leaves each lane
//     holding 8 consecutive keys, which is exactly the P^T operand of
//     O^T += V^T P^T (the same instruction).  With several waves, the partial
//     S^T of each wave's dims are summed through LDS in a fixed order, so
//     every wave sees bit-identical scores and softmax state.
// Query rows beyond the GQA group are zero padding of the 16-column MFMA.
#include <type_traits>

#include "psw_device.hpp"

namespace psw_dev {
namespace {

constexpr float kNegBigD = -1.0e30f;
constexpr float kSlackD = 8.0f;  // log2 units: rescale O only past a 256x rise
constexpr int kTK = 32;          // keys per tile
constexpr int kDW = 128;         // head dims per wave
constexpr int kNST = 2;          // register stages of the K/V tile pipeline (the loop assumes 2)

template <typename T>
__device__ __forceinline__ T ldu(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      (const __attribute__((address_space(4))) char*)p);
}

// Streaming 16-byte load: every K/V byte is read once, so the loads carry the
// non-temporal hint (plain loads that allocate in the caches sustain markedly
// less HBM read bandwidth on this part).
__device__ __forceinline__ bf16x8 ld_stream(const char* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// PMODE: 0 = pages smaller than 16 slots (per-lane page ids), 1 = 16-slot
// pages (two wave-uniform page ids per tile), 2 = pages of 32 slots or more
// (one wave-uniform page id per tile).
template <int D, int PMODE>
__global__ __launch_bounds__(64 * (D / kDW)) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(AttnParams P) {
  constexpr int W = D / kDW;   // waves; wave w owns dims [kDW w, kDW (w + 1))
  constexpr int KS = kDW / 32; // 32-dim k-steps of the per-wave QK
  constexpr int DB = kDW / 16; // 16-dim blocks of the per-wave O^T
  __shared__ f32x4 sx[2][W][2][64];  // partial S^T exchange [buffer][wave][block][lane]

  const int lane = threadIdx.x & 63;
  const int w = W > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int n = lane & 15;   // query row (head within the group); K row; V^T dim
  const int q4 = lane >> 4;  // lane quarter
  const int hkv = P.num_kv_heads;
  const int wg = blockIdx.x / hkv;
  const int kvh = blockIdx.x - wg * hkv;
  const int group = 1 << P.group_shift;
  const bool row_valid = n < group;
  const int head = kvh * group + (row_valid ? n : 0);
  const int dim0 = kDW * w;
  const char* kbase =
      reinterpret_cast<const char*>(P.pool + P.layer_off + (int64_t)kvh * P.ps.head);
  const char* vbase = kbase + P.ps.kv * 2;
  const int64_t page_bytes = P.ps.page * 2;
  const int pshift = P.ps.page_shift;
  const int pmask = P.ps.page_size - 1;
  const int psize = P.ps.page_size;
  // Tile-relative key of the K row this lane feeds into S^T block sb: block sb,
  // output row 4 q + r holds key 8 q + 4 sb + r, so the lane of row n reads key
  // 8 (n / 4) + 4 sb + n % 4.  Its V^T operand covers keys 8 q4 .. 8 q4 + 7.
  const int kkey0 = 8 * (n >> 2) + (n & 3);
  const int kdim_off = (dim0 + 8 * q4) * 2;
  const int vdim_off = (dim0 + n) * psize * 2;
  const float c2 = P.scale_log2;

  // The S^T exchange alternates between two LDS buffers tile by tile; the
  // parity carries over from one item to the next, so a buffer is never
  // rewritten before the barrier that follows every wave's last read of it.
  int xpar = 0;
  const int item_end = ldu(P.wg_items + wg + 1);
  for (int item = ldu(P.wg_items + wg); item < item_end; ++item) {
  const int b = ldu(P.items + 4 * item + 0);
  const int slot = ldu(P.items + 4 * item + 1);  // partial slot; < 0: the whole request
  const int k_lo = ldu(P.items + 4 * item + 2);
  const int k_hi = ldu(P.items + 4 * item + 3);
  const int q_row = ldu(P.qo_indptr + b);  // qo_len == 1
  const int32_t* pages = P.kv_page_indices + ldu(P.kv_page_indptr + b);

  // Q^T operand (B of S^T = K Q^T): lane (row n, quarter q4) holds
  // Q[n][dim0 + 32 ks + 8 q4 .. +8]
  bf16x8 qf[KS];
  {
    const __bf16* qrow = P.q + ((int64_t)q_row * P.num_qo_heads + head) * D + dim0 + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
      qf[ks] = row_valid ? v : bf16x8{};
    }
  }
  // page list index of an absolute page (resident windows wrap the list)
  const PageRing ring = page_ring(ldu(P.kv_page_indptr + b + 1) - ldu(P.kv_page_indptr + b),
                                  ldu(P.kv_len + b), pshift);
  const int jt0 = k_lo / kTK;

  // Page ids of tile t, fetched one step before that tile's K/V loads are
  // issued, so no load waits on a page id.  Every lane loads (the index
  // depends on the lane, which keeps this a vector load in the same in-order
  // stream as K and V); 16-slot pages: lanes 0 / 1 end up with the ids of the
  // tile's two pages; 32 slots or more: lane 0 with its one page; smaller
  // pages: each lane with the pages of its own two K rows and V^T chunk.
  struct TilePids { int a, b, c; };
  auto pid_load = [&](int t) {
    const int j0 = (jt0 + t) * kTK;
    TilePids r;
    if constexpr (PMODE == 0) {
      const int k0 = j0 + kkey0;
      r.a = pages[ring(k0 >> pshift)];
      r.b = pages[ring((k0 + 4) >> pshift)];
      r.c = pages[ring((j0 + 8 * q4) >> pshift)];
    } else {
      r.a = pages[ring((j0 >> pshift) + (lane & 1))];
      r.b = r.c = 0;
    }
    return r;
  };
  // byte addresses of one tile's K rows (block 0 / 1) and this lane's V^T chunk
  auto tile_addr = [&](int j0, const TilePids& pid, const char** kp0, const char** kp1,
                       const char** vp) {
    if constexpr (PMODE == 2) {
      const int64_t pg = (int64_t)__builtin_amdgcn_readlane(pid.a, 0) * page_bytes;
      const int in_page = j0 & pmask;
      *kp0 = kbase + pg + (int64_t)(in_page + kkey0) * D * 2 + kdim_off;
      *kp1 = *kp0 + 4 * D * 2;
      *vp = vbase + pg + (in_page + 8 * q4) * 2 + vdim_off;
    } else if constexpr (PMODE == 1) {
      const int64_t pa = (int64_t)__builtin_amdgcn_readlane(pid.a, 0) * page_bytes;
      const int64_t pb = (int64_t)__builtin_amdgcn_readlane(pid.a, 1) * page_bytes;
      // keys 0..15 of the tile sit in page a, 16..31 in page b
      const int64_t kpg = kkey0 < 16 ? pa : pb;
      *kp0 = kbase + kpg + (int64_t)(kkey0 & 15) * D * 2 + kdim_off;
      *kp1 = *kp0 + 4 * D * 2;
      *vp = vbase + (q4 < 2 ? pa : pb) + ((8 * q4) & 15) * 2 + vdim_off;
    } else {
      const int k0 = j0 + kkey0, k1 = k0 + 4, kv = j0 + 8 * q4;
      *kp0 = kbase + (int64_t)pid.a * page_bytes + (int64_t)(k0 & pmask) * D * 2 + kdim_off;
      *kp1 = kbase + (int64_t)pid.b * page_bytes + (int64_t)(k1 & pmask) * D * 2 + kdim_off;
      *vp = vbase + (int64_t)pid.c * page_bytes + (kv & pmask) * 2 + vdim_off;
    }
  };
  auto load = [&](int j0, const TilePids& pid, bf16x8 (*kr)[KS], bf16x8* vr) {
    const char *kp0, *kp1, *vp;
    tile_addr(j0, pid, &kp0, &kp1, &vp);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[0][ks] = ld_stream(kp0 + 64 * ks);
      kr[1][ks] = ld_stream(kp1 + 64 * ks);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vr[db] = ld_stream(vp + (int64_t)db * 16 * psize * 2);
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBigD, l_run = 0.0f;

  const int ntiles = k_hi / kTK - jt0 + 1;
  bf16x8 kr[kNST][2][KS];
  bf16x8 vr[kNST][DB];
  TilePids pr[kNST];
  // prologue: page ids of tiles 0 and 1, tile 0 in flight (ids past the last
  // tile are clamped by the ring to a page of the request: harmless reads)
  pr[0] = pid_load(0);
  pr[1] = pid_load(1);
  load(jt0 * kTK, pr[0], kr[0], vr[0]);

  // One tile: with LOAD, first the page ids of tile it + 2 (into this stage's
  // id registers, whose tile is now in flight) and then tile it + 1's K/V.
  // LOAD is a constant, so the loop below never joins paths that differ in
  // the number of loads in flight (the wait counts stay those of the steady
  // state instead of draining every tile).
  auto step = [&](auto STAGE, int it, auto LOAD) {
    constexpr int cb = decltype(STAGE)::value;  // == it % 2
    constexpr int nb = 1 - cb;                  // stage of tile it + 1
    const int j0 = (jt0 + it) * kTK;
    if constexpr (decltype(LOAD)::value) {
      const TilePids ids = pid_load(it + 2);
      load(j0 + kTK, pr[nb], kr[nb], vr[nb]);
      pr[cb] = ids;
    }
    f32x4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[cb][0][ks], qf[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[cb][1][ks], qf[ks], s[1], 0, 0, 0);
    }
    if constexpr (W > 1) {
      // two exchange buffers alternate by tile parity: a wave rewrites one
      // only after the next barrier, which every wave reaches after reading it
      const int xb = (it + xpar) & 1;
      sx[xb][w][0][lane] = s[0];
      sx[xb][w][1][lane] = s[1];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      s[0] = sx[xb][0][0][lane];
      s[1] = sx[xb][0][1][lane];
#pragma unroll
      for (int v = 1; v < W; ++v) {
        s[0] += sx[xb][v][0][lane];
        s[1] += sx[xb][v][1][lane];
      }
    }
    // lane (row n, q4): s[sb][r] is the score of key j0 + 8 q4 + 4 sb + r
    const int key0 = j0 + 8 * q4;
    float x[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key0 + e;
      x[e] = (key >= k_lo && key <= k_hi) ? s[e >> 2][e & 3] * c2 : -__builtin_inff();
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run + kSlackD)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
    }
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(x[e] - m_run);
      l_run += p;
      pb[e] = (__bf16)p;
    }
    // Keys outside the split (before the window, past the end of the last
    // page) may hold anything, NaN included: their V must be exactly zero,
    // not multiplied by a zero weight.
    if (j0 < k_lo || j0 + kTK - 1 > k_hi) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool out = key0 + e < k_lo || key0 + e > k_hi;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          if (out) vr[cb][db][e] = (__bf16)0.0f;
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[cb][db], pb, oacc[db], 0, 0, 0);
  };
  // steady state two tiles at a time, every step loading; then the last one
  // or two tiles, the final one without a load
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using LD = std::true_type;
  using NL = std::false_type;
  int it = 0;
  for (; it + 2 < ntiles; it += 2) {
    step(I0{}, it, LD{});
    step(I1{}, it + 1, LD{});
  }
  if (it + 1 < ntiles) {
    step(I0{}, it, LD{});
    step(I1{}, it + 1, NL{});
  } else {
    step(I0{}, it, NL{});
  }

  xpar ^= ntiles & 1;

  // row sums: each lane holds the part over its keys; add the four quarters
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // lane (n, q4), O^T block db, register r: dim dim0 + 16 db + 4 q4 + r of row n
  if (row_valid && slot < 0) {
    // the piece is the whole request: normalise and write O
    const float inv = 1.0f / l_tot;
    const int64_t orow = ((int64_t)q_row * P.num_qo_heads + head) * D + dim0 + 4 * q4;
    if (P.out_bf16) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 v = {(__bf16)(oacc[db][0] * inv), (__bf16)(oacc[db][1] * inv),
                    (__bf16)(oacc[db][2] * inv), (__bf16)(oacc[db][3] * inv)};
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.o) + orow + 16 * db) = v;
      }
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(static_cast<float*>(P.o) + orow + 16 * db) = oacc[db] * inv;
    }
  } else if (row_valid) {
    const int64_t base = (int64_t)slot * P.num_qo_heads + head;
    float* po = P.part_o + base * D + dim0 + 4 * q4;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = oacc[db];
    if (w == 0 && q4 == 0) {
      P.part_ml[base * 2 + 0] = m_run;
      P.part_ml[base * 2 + 1] = l_tot;
    }
  }
  }  // items
}

template <int D>
hipError_t launch_d(const AttnParams& p, int n_wgs, hipStream_t s) {
  const dim3 grid(n_wgs), block(64 * (D / kDW));
  if (p.ps.page_size >= 32)
    hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, s, p);
  else if (p.ps.page_size == 16)
    hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<D, 0>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int head_dim, const AttnParams& p, int n_wgs, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  return head_dim == 256 ? launch_d<256>(p, n_wgs, s) : launch_d<512>(p, n_wgs, s);
}

}  // namespace psw_dev
