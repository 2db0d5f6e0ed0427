// Fused pool-write prep for gfx950 (issue "gemma4: serving prep needs
// pool-write forms -- hd256 QKV in one pass, hd512 V alongside K", Description
// and Proposed Plan), plus the RoPE table builder.
//
//   hd256: Q rows  -> rope(rms(q) * w_q, p)  to the contiguous q_out
//          K rows  -> rope(rms(k) * w_k, p)  to the layer's K block
//          V rows  -> v * inv_rms(v)         to the layer's V block (never rotated)
//   hd512: K rows  -> rope(k * inv * w_k, p) to the K block and
//          V rows  -> k * inv                to the V block, inv = inv_rms(k) shared
//
// rms(x) = x / sqrt(mean(x^2) + eps); RoPE rotates pairs (i, i + D/2) with the
// caller's fp32 cos/sin tables; p = start_pos + token.  Math is fp32, each
// output rounded once to bf16 (RNE).
//
// A work item is up to 16 consecutive positions of one request that fall in one
// page.  A row (one token, one head) is handled by D/16 lanes; lane i holds
// elements [8i, 8i+8) and [D/2 + 8i, D/2 + 8i + 8), so both members of each
// rotated pair sit in the same lane and every load and store is a 16-byte
// vector.  V goes to the dim-major V block (keys contiguous per dim) through an
// LDS transpose, so its stores are runs of consecutive slots.
//
// Second line of defence behind the host checks: a position past the RoPE
// table or a page id outside the pool makes the item write nothing and record
// the offending value in the plan's device error word (no trap).
#include "psw_device.hpp"

namespace psw_dev {
namespace {

// Sum over the LPR lanes that share a row (aligned groups of LPR lanes).
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void load8(const __bf16* p, float* f) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}

__device__ __forceinline__ void store8(__bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
  *reinterpret_cast<bf16x8*>(p) = v;
}

__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
}

struct Item {
  int b, tok0, ntok, page, slot0, pos0;
};

__device__ __forceinline__ Item read_item(const int32_t* it) {
  return Item{it[0], it[1], it[2], it[3], it[4], it[5]};
}

// Device-side bounds check of an item; on failure record and skip.
__device__ __forceinline__ bool item_ok(const PrepParams& P, const Item& it) {
  const bool ok = it.page >= 0 && it.page < P.num_pages && it.pos0 >= 0 &&
                  it.pos0 + it.ntok <= P.rope_positions && it.ntok >= 1 &&
                  it.ntok <= kPrepMaxTokens && it.slot0 >= 0 &&
                  it.slot0 + it.ntok <= P.ps.page_size;
  if (!ok && threadIdx.x == 0) {
    // first offending value wins; a plain vector store is enough for a flag
    P.err[0] = 1;
    P.err[1] = it.page;
    P.err[2] = it.pos0 + it.ntok - 1;
  }
  return ok;
}

// Normalise (+ weight) and rotate one row held as two 8-element halves.
template <int D, bool WEIGHT, bool ROTATE>
__device__ __forceinline__ void norm_rope(float* x1, float* x2, const float* w1, const float* w2,
                                          const float* c, const float* s, float inv) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = x1[e] * inv, bb = x2[e] * inv;
    if constexpr (WEIGHT) {
      a *= w1[e];
      bb *= w2[e];
    }
    if constexpr (ROTATE) {
      x1[e] = a * c[e] - bb * s[e];
      x2[e] = bb * c[e] + a * s[e];
    } else {
      x1[e] = a;
      x2[e] = bb;
    }
  }
}

// hd256: blockIdx.y selects the row kind and a group of up to 8 heads:
// y < nqg -> Q heads 8y.., y < nqg + nkg -> K heads, else V heads.
__global__ __launch_bounds__(256) void prep_hd256_kernel(PrepParams P) {
  constexpr int D = 256, LPR = 16, RPP = 256 / LPR;  // rows per pass
  constexpr int HALF = D / 2;
  constexpr int VSUB = 2;                            // V heads staged at a time
  const Item it = read_item(P.items + kPrepItemInts * blockIdx.x);
  if (!item_ok(P, it)) return;
  const int nqg = (P.num_qo_heads + 7) / 8;
  const int nkg = (P.num_kv_heads + 7) / 8;
  const int y = blockIdx.y;
  const int kind = y < nqg ? 0 : (y < nqg + nkg ? 1 : 2);
  const int hg = kind == 0 ? y : (kind == 1 ? y - nqg : y - nqg - nkg);
  const int heads = kind == 0 ? P.num_qo_heads : P.num_kv_heads;
  const int h0 = 8 * hg;
  const int hcount = min(8, heads - h0);
  const int li = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  const int64_t page_off = P.layer_off + (int64_t)it.page * P.ps.page;

  if (kind < 2) {
    float w1[8], w2[8];
    const __bf16* wp = kind == 0 ? P.q_w : P.k_w;
    load8(wp + 8 * li, w1);
    load8(wp + HALF + 8 * li, w2);
    const int nrows = it.ntok * hcount;
    for (int row = rsub; row < nrows; row += RPP) {
      const int tt = row / hcount;
      const int hd = h0 + row - tt * hcount;
      const int tok = it.tok0 + tt;
      const int pos = it.pos0 + tt;
      const __bf16* src = kind == 0 ? P.q_in + ((int64_t)tok * P.num_qo_heads + hd) * D
                                    : P.k_in + ((int64_t)tok * P.num_kv_heads + hd) * D;
      float x1[8], x2[8], c[8], s[8];
      load8(src + 8 * li, x1);
      load8(src + HALF + 8 * li, x2);
      load8f(P.cos + (int64_t)pos * HALF + 8 * li, c);
      load8f(P.sin + (int64_t)pos * HALF + 8 * li, s);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
      ss = row_sum<LPR>(ss);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + P.eps);
      norm_rope<D, true, true>(x1, x2, w1, w2, c, s, inv);
      __bf16* dst = kind == 0 ? P.q_out + ((int64_t)tok * P.num_qo_heads + hd) * D
                              : P.pool + page_off + (int64_t)hd * P.ps.head +
                                    (int64_t)(it.slot0 + tt) * D;
      store8(dst + 8 * li, x1);
      store8(dst + HALF + 8 * li, x2);
    }
    return;
  }

  // V: weightless norm, staged per VSUB heads for the transpose into the
  // dim-major V block.  vstage: [VSUB][token][D + 2] bf16
  __shared__ __bf16 vstage[VSUB * kPrepMaxTokens * (D + 2)];
  for (int hs = 0; hs < hcount; hs += VSUB) {
    const int hn = min(VSUB, hcount - hs);
    const int nrows = it.ntok * hn;
    for (int row = rsub; row < nrows; row += RPP) {
      const int tt = row / hn;
      const int hl = row - tt * hn;
      const int tok = it.tok0 + tt;
      const __bf16* src = P.v_in + ((int64_t)tok * P.num_kv_heads + h0 + hs + hl) * D;
      float x1[8], x2[8];
      load8(src + 8 * li, x1);
      load8(src + HALF + 8 * li, x2);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
      ss = row_sum<LPR>(ss);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + P.eps);
      __bf16* vs = vstage + (hl * kPrepMaxTokens + tt) * (D + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vs[8 * li + e] = (__bf16)(x1[e] * inv);
        vs[HALF + 8 * li + e] = (__bf16)(x2[e] * inv);
      }
    }
    __syncthreads();
    // consecutive threads take consecutive slots of one (head, dim) row
    const int total = hn * D * it.ntok;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
      const int tt = idx % it.ntok;
      const int rest = idx / it.ntok;
      const int d = rest % D;
      const int hl = rest / D;
      P.pool[page_off + P.ps.kv + (int64_t)(h0 + hs + hl) * P.ps.head +
             (int64_t)d * P.ps.page_size + it.slot0 + tt] =
          vstage[(hl * kPrepMaxTokens + tt) * (D + 2) + d];
    }
    __syncthreads();
  }
}

// hd512: one raw K row per (token, KV head) yields the K row (weighted norm +
// rope) and the V row (weightless norm, same inv, no rope).
__global__ __launch_bounds__(256) void prep_hd512_kernel(PrepParams P) {
  constexpr int D = 512, LPR = 32, RPP = 256 / LPR;
  constexpr int HALF = D / 2;
  const Item it = read_item(P.items + kPrepItemInts * blockIdx.x);
  if (!item_ok(P, it)) return;
  const int li = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  const int heads = P.num_kv_heads;
  const int64_t page_off = P.layer_off + (int64_t)it.page * P.ps.page;
  float w1[8], w2[8];
  load8(P.k_w + 8 * li, w1);
  load8(P.k_w + HALF + 8 * li, w2);

  __shared__ __bf16 vstage[kPrepMaxTokens * (D + 2)];

  for (int hd0 = 0; hd0 < heads; ++hd0) {
    for (int tt = rsub; tt < it.ntok; tt += RPP) {
      const int tok = it.tok0 + tt;
      const int pos = it.pos0 + tt;
      const __bf16* src = P.k_in + ((int64_t)tok * heads + hd0) * D;
      float x1[8], x2[8];
      load8(src + 8 * li, x1);
      load8(src + HALF + 8 * li, x2);
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
      ss = row_sum<LPR>(ss);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + P.eps);
      float v1[8], v2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v1[e] = x1[e];
        v2[e] = x2[e];
      }
      float c[8], s[8];
      load8f(P.cos + (int64_t)pos * HALF + 8 * li, c);
      load8f(P.sin + (int64_t)pos * HALF + 8 * li, s);
      norm_rope<D, true, true>(x1, x2, w1, w2, c, s, inv);
      __bf16* dst = P.pool + page_off + (int64_t)hd0 * P.ps.head + (int64_t)(it.slot0 + tt) * D;
      store8(dst + 8 * li, x1);
      store8(dst + HALF + 8 * li, x2);
      norm_rope<D, false, false>(v1, v2, nullptr, nullptr, nullptr, nullptr, inv);
      __bf16* vs = vstage + tt * (D + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vs[8 * li + e] = (__bf16)v1[e];
        vs[HALF + 8 * li + e] = (__bf16)v2[e];
      }
    }
    __syncthreads();
    const int total = D * it.ntok;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
      const int tt = idx % it.ntok;
      const int d = idx / it.ntok;
      P.pool[page_off + P.ps.kv + (int64_t)hd0 * P.ps.head + (int64_t)d * P.ps.page_size +
             it.slot0 + tt] = vstage[tt * (D + 2) + d];
    }
    __syncthreads();
  }
}

// cos/sin[p][i] = cos/sin(p * theta^(-2i/D)), formed and evaluated in fp64.
__global__ void rope_table_kernel(float* __restrict__ c, float* __restrict__ s, int64_t positions,
                                  int64_t half, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= positions * half) return;
  const int64_t p = idx / half;
  const int64_t i = idx - p * half;
  const double inv_freq = pow(theta, -(double)(2 * i) / (double)(2 * half));
  const double ang = (double)p * inv_freq;
  c[idx] = (float)cos(ang);
  s[idx] = (float)sin(ang);
}

}  // namespace

hipError_t launch_prep_hd256(const PrepParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const int groups = (p.num_qo_heads + 7) / 8 + 2 * ((p.num_kv_heads + 7) / 8);
  hipLaunchKernelGGL(prep_hd256_kernel, dim3(n_items, groups), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prep_hd512(const PrepParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(prep_hd512_kernel, dim3(n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rope_tables(float* c, float* s, int64_t positions, int64_t half, double theta,
                              hipStream_t st) {
  const int64_t n = positions * half;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, s, positions,
                     half, theta);
  return hipGetLastError();
}

}  // namespace psw_dev
