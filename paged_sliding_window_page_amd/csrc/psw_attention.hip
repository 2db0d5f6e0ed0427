// Paged prefill attention for gfx950: bf16 MFMA, online softmax, K/V gathered
// through a page table.  One kernel template serves
//   * windowed paged prefill at head_dim 256 (PR "feat(kernels): Rust wrapper
//     for the hd256 windowed paged prefill", Description: explicit sm_scale,
//     window_left an inclusive distance, addresses from page ids and the
//     last-page length),
//   * full paged prefill at head_dim 512 (PR "feat(gemma4): paged KV serving
//     across both attention families", Description: global layers are full
//     attention at head_dim 512 with one KV head),
//   * the split-KV form that one-token decode runs through the same entry
//     (same PR, Description: decode runs the prefill entry at seq_len 1), whose
//     partial results are combined by merge_kernel.
//
// Work-group: 4 waves, 128 query rows = (128 / group) tokens x group heads of
// one KV head, so the group's heads share every K/V tile.  Each wave owns 32
// rows.  Per KV tile (64 keys at D=256, 32 at D=512):
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
#include "psw_device.hpp"

namespace psw_dev {
namespace {

constexpr float kNegBig = -1.0e30f;     // finite "minus infinity" for running maxima
constexpr float kRescaleSlack = 8.0f;   // log2 units: rescale O only past a 256x rise

__device__ __forceinline__ int kperm(int m) {
  // S^T row m (0..31) -> key within the 32-key block.  With the 32x32 MFMA
  // accumulator layout (lane half h, register r holds row 8*(r/4) + 4*h + r%4)
  // this puts key 16*(r/8) + 8*h + (r%8) in register r of half h.
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// XOR swizzles of the 16-byte chunk index inside a K row / V^T row.
__device__ __forceinline__ int kswz(int key) {
  return (key & 3) | ((key >> 1) & 4) | ((key << 1) & 8);
}

template <int D>
__device__ __forceinline__ int vswz(int d) {
  if constexpr (D == 256) {  // 8 chunks per V^T row (64 keys)
    return (d & 6) | ((d ^ (d >> 3)) & 1);
  } else {                   // 4 chunks per V^T row (32 keys)
    return (((d >> 3) ^ (d >> 1)) & 1) | (((d >> 2) & 1) << 1);
  }
}

__device__ __forceinline__ void lds_load16(const void* gsrc, void* ldst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

template <int D, bool SPLIT, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void attention_kernel(AttnParams P) {
  constexpr int KT = D == 256 ? 64 : 32;  // keys per tile
  constexpr int NCH = D / 8;              // 16-B chunks per K row
  constexpr int VCH = KT / 8;             // 16-B chunks per V^T row
  constexpr int KBLK = KT / 32;           // S^T 32-key blocks per tile
  constexpr int NT = KT / 16;             // PV steps (16 keys each) per tile
  constexpr int DB = D / 32;              // O^T 32-row blocks
  constexpr int KS = D / 16;              // QK k-steps
  constexpr int TILE = KT * D * 2;        // bytes of one K (or V^T) tile: 32 KiB
  constexpr int ROUNDS = TILE / (256 * 16);

  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int hkv = P.num_kv_heads;
  const int item = blockIdx.x / hkv;
  const int kvh = blockIdx.x - item * hkv;
  const int b = P.items[4 * item + 0];
  const int t0 = P.items[4 * item + 1];
  const int k_lo = P.items[4 * item + 2];
  const int k_hi = P.items[4 * item + 3];
  const int q_beg = P.qo_indptr[b];
  const int qo_len = P.qo_indptr[b + 1] - q_beg;
  const int kvl = P.kv_len[b];
  const int start = kvl - qo_len;
  const int32_t* __restrict__ pages = P.kv_page_indices + P.kv_page_indptr[b];
  const int gs = P.group_shift;
  const int tok_w = 32 >> gs;            // tokens per wave
  const int wl = P.window_left;

  // this lane's query row: token t0 + tl, head kvh*group + hh
  const int tl = w * tok_w + (n >> gs);
  const int hh = n & ((1 << gs) - 1);
  const int tok = t0 + tl;
  const bool row_valid = tok < qo_len;
  const int pos = start + tok;
  const int head = (kvh << gs) + hh;

  const int wt0 = t0 + w * tok_w;        // first token of this wave
  const bool wave_live = wt0 < qo_len;
  const int p_min_w = start + wt0;
  const int p_max_w = start + min(wt0 + tok_w, qo_len) - 1;

  bf16x8 qf[KS];
  {
    const __bf16* qrow = P.q + ((int64_t)(q_beg + (row_valid ? tok : 0)) * P.num_qo_heads + head) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      qf[ks] = row_valid ? v : bf16x8{};
    }
  }

  const __bf16* kbase_g = P.pool + P.layer_off + (int64_t)kvh * P.ps.head;
  const __bf16* vbase_g = kbase_g + P.ps.kv;
  const int pshift = P.ps.page_shift;
  const int pmask = P.ps.page_size - 1;
  const int psize = P.ps.page_size;

  // Issue the direct-to-LDS loads of tile j0 into stage st.  Keys at or past
  // kv_len are clamped to a valid address inside the request's pages; their
  // scores are masked and their V values zeroed after the load lands.
  auto issue = [&](int st, int j0) {
    char* kl = smem[st][0];
    char* vl = smem[st][1];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int u = (r * 4 + w) * 64 + lane;
      const int key = u / NCH;
      const int c = (u % NCH) ^ kswz(key);
      const int j = min(j0 + key, kvl - 1);
      const int64_t page = pages[j >> pshift];
      const __bf16* src = kbase_g + page * P.ps.page + (int64_t)(j & pmask) * D + c * 8;
      lds_load16(src, kl + (r * 4 + w) * 1024);
    }
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int u = (r * 4 + w) * 64 + lane;
      const int d = u / VCH;
      const int k8 = (u % VCH) ^ vswz<D>(d);
      int jc = j0 + 8 * k8;
      if (jc > kvl - 1) jc = (kvl - 1) & ~7;
      const int64_t page = pages[jc >> pshift];
      const __bf16* src = vbase_g + page * P.ps.page + (int64_t)d * psize + (jc & pmask);
      lds_load16(src, vl + (r * 4 + w) * 1024);
    }
  };

  // Zero, in the V^T chunks this lane loaded itself, the keys at or past
  // kv_len (their pool slots may hold anything, NaN included, and 0 * NaN would
  // leak into O).  Called after this wave's loads have landed.
  auto sanitize = [&](int st, int j0) {
    if (j0 + KT <= kvl) return;
    char* vl = smem[st][1];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int u = (r * 4 + w) * 64 + lane;
      const int d = u / VCH;
      const int k8 = (u % VCH) ^ vswz<D>(d);
      const int jc = j0 + 8 * k8;
      if (jc + 8 > kvl) {
        bf16x8* cp = reinterpret_cast<bf16x8*>(vl + (r * 4 + w) * 1024 + lane * 16);
        bf16x8 v = *cp;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (jc + e >= kvl) v[e] = (__bf16)0.0f;
        *cp = v;
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.0f;

  const int jt0 = k_lo / KT;
  const int jt1 = k_hi / KT;
  const int ntiles = jt1 - jt0 + 1;

  issue(0, jt0 * KT);
  __builtin_amdgcn_s_waitcnt(0);
  sanitize(0, jt0 * KT);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int j0 = (jt0 + it) * KT;
    if (it + 1 < ntiles) issue(st ^ 1, j0 + KT);

    // does this wave have any (row, key) pair in this tile?
    bool active = wave_live && j0 <= p_max_w;
    if (wl >= 0) active = active && (j0 + KT - 1 >= p_min_w - wl);
    if (active) {
      const char* kl = smem[st][0];
      const char* vl = smem[st][1];
      f32x16 s[KBLK];
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        s[kb] = f32x16{};
        const int key = 32 * kb + kperm(n);
        const char* krow = kl + key * (NCH * 16);
        const int sw = kswz(key);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + h) ^ sw) << 4));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
        }
      }
      // scale, mask, tile max.  Register r of block kb holds key
      // j0 + 32*kb + 16*(r/8) + 8*h + r%8 for this lane's row.
      const bool full = j0 >= k_lo && j0 + KT - 1 <= k_hi && j0 + KT - 1 <= p_min_w &&
                        (wl < 0 || p_max_w - j0 <= wl);
      float tmax = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[kb][r] * P.scale_log2;
          if (!full) {
            const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * h + (r & 7);
            bool ok = key >= k_lo && key <= k_hi && key <= pos && row_valid;
            if (wl >= 0) ok = ok && (pos - key <= wl);
            v = ok ? v : -__builtin_inff();
          }
          s[kb][r] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      if (__any(m_new > m_run + kRescaleSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      }
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_run);
          s[kb][r] = p;
          lsum += p;
        }
      }
      l_run += lsum;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[t >> 1][8 * (t & 1) + i];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = 32 * db + n;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              vl + (d * VCH + ((2 * t + h) ^ vswz<D>(d))) * 16);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
        }
      }
    }
    if (it + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);
      sanitize(st ^ 1, j0 + KT);
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_valid) return;
  // lane (n, h), O^T block db, register r holds d = 32*db + 8*(r/4) + 4*h + r%4
  if constexpr (SPLIT) {
    const int64_t base = ((int64_t)item * P.num_qo_heads + head);
    float* po = P.part_o + base * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * g) = v;
      }
    if (h == 0) {
      P.part_ml[base * 2 + 0] = m_run;
      P.part_ml[base * 2 + 1] = l_tot;
    }
  } else {
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
}

// Combines the split-KV partials of one (request, head): with per-split running
// max m_s (log2 units), sum l_s and unnormalised o_s,
//   O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D / 4) void merge_kernel(MergeParams P) {
  const int b = blockIdx.x / P.num_qo_heads;
  const int head = blockIdx.x - b * P.num_qo_heads;
  const int first = P.req_splits[2 * b];
  const int ns = P.req_splits[2 * b + 1];
  float M = kNegBig;
  for (int s = 0; s < ns; ++s)
    M = fmaxf(M, P.part_ml[((int64_t)(first + s) * P.num_qo_heads + head) * 2]);
  float L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int d = 4 * threadIdx.x;
  for (int s = 0; s < ns; ++s) {
    const int64_t base = (int64_t)(first + s) * P.num_qo_heads + head;
    const float wgt = __builtin_amdgcn_exp2f(P.part_ml[base * 2] - M);
    L += wgt * P.part_ml[base * 2 + 1];
    const f32x4 v = *reinterpret_cast<const f32x4*>(P.part_o + base * D + d);
    acc += wgt * v;
  }
  const float inv = 1.0f / L;
  const int64_t orow = ((int64_t)P.qo_indptr[b] * P.num_qo_heads + head) * D + d;
  if constexpr (OUT_BF16) {
    bf16x4 v = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                (__bf16)(acc[3] * inv)};
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.o) + orow) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(P.o) + orow) = acc * inv;
  }
}

template <int D, bool SPLIT, bool OB>
hipError_t launch_one(const AttnParams& p, int n_items, hipStream_t s) {
  hipLaunchKernelGGL((attention_kernel<D, SPLIT, OB>), dim3(n_items * p.num_kv_heads), dim3(256),
                     0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int head_dim, bool split, bool out_bf16, const AttnParams& p,
                            int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (head_dim == 256) {
    if (split) return out_bf16 ? launch_one<256, true, true>(p, n_items, s)
                               : launch_one<256, true, false>(p, n_items, s);
    return out_bf16 ? launch_one<256, false, true>(p, n_items, s)
                    : launch_one<256, false, false>(p, n_items, s);
  }
  if (split) return out_bf16 ? launch_one<512, true, true>(p, n_items, s)
                             : launch_one<512, true, false>(p, n_items, s);
  return out_bf16 ? launch_one<512, false, true>(p, n_items, s)
                  : launch_one<512, false, false>(p, n_items, s);
}

hipError_t launch_merge(int head_dim, bool out_bf16, const MergeParams& p, int batch,
                        hipStream_t s) {
  const dim3 grid(batch * p.num_qo_heads);
  if (head_dim == 256) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<256, true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<256, false>), grid, dim3(64), 0, s, p);
  } else {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<512, true>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<512, false>), grid, dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace psw_dev
