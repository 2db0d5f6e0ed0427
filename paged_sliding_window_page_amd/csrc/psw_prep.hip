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
template <bool WEIGHT, bool ROTATE>
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Inputs are read once and outputs written once: streaming (non-temporal)
// 16-byte accesses, which keep them from displacing the reused RoPE tables
// and sustain more HBM bandwidth than cache-allocating ones.
__device__ __forceinline__ bf16x8 load8_stream(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ void widen8(bf16x8 v, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}

__device__ __forceinline__ void store8_stream(__bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (__bf16)f[e];
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

// 1 / sqrt(mean(x^2) + eps) over a row spread across LPR lanes
template <int LPR>
__device__ __forceinline__ float inv_rms(const float* x1, const float* x2, float inv_d, float eps) {
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
  ss = row_sum<LPR>(ss);
  return 1.0f / sqrtf(ss * inv_d + eps);
}

// Writes the staged V rows of `nh` heads to their dim-major V blocks: the
// element for (head h, token t, dim d) goes to slot slot0 + t of row d.
// vstage layout: [head][token][D + 8] bf16.  With slot0 and ntok multiples of
// 8, each thread stores 8 consecutive slots as one 16-byte vector, and
// consecutive threads cover consecutive 16-byte pieces of the block.
template <int D, int THREADS>
__device__ __forceinline__ void store_v_transposed(const PrepParams& P, const __bf16* vstage,
                                                   const Item& it, int64_t vblock0, int nh) {
  constexpr int RS = D + 8;
  if ((it.slot0 & 7) == 0 && (it.ntok & 7) == 0) {
    const int nch = it.ntok >> 3;
    const int total = nh * D * nch;
    for (int idx = threadIdx.x; idx < total; idx += THREADS) {
      const int ch = idx % nch;
      const int rest = idx / nch;
      const int d = rest % D;
      const int h = rest / D;
      const __bf16* src = vstage + (h * kPrepMaxTokens + 8 * ch) * RS + d;
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = src[e * RS];
      __bf16* dst = P.pool + vblock0 + (int64_t)h * P.ps.head + (int64_t)d * P.ps.page_size +
                    it.slot0 + 8 * ch;
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
    }
  } else {
    const int total = nh * D * it.ntok;
    for (int idx = threadIdx.x; idx < total; idx += THREADS) {
      const int tt = idx % it.ntok;
      const int rest = idx / it.ntok;
      const int d = rest % D;
      const int h = rest / D;
      P.pool[vblock0 + (int64_t)h * P.ps.head + (int64_t)d * P.ps.page_size + it.slot0 + tt] =
          vstage[(h * kPrepMaxTokens + tt) * RS + d];
    }
  }
}

// Heads of one row kind per hd256 work-group: 2 rather than 8 gives 4x the
// work-groups, each with a quarter of the registers and LDS, so more of them
// are resident and their load / compute / store phases overlap.
constexpr int kPrepHeads256 = 2;

// Work-groups are dispatched to the 8 XCDs in turn (block x to XCD x % 8),
// each XCD with its own L2.  The prep grids give an item's head groups blocks
// x that are equal mod 8, so they all run on one XCD and the item's RoPE rows
// come into that L2 once (-4.5% on the 8192-token hd256 prep): block x is
// head group (x / 8) % g of item 8 ((x / 8) / g) + x % 8, for g head groups
// per item and a grid padded to a multiple of 8 items.
__device__ __forceinline__ void xcd_item_group(int g, int* item, int* group) {
  const int k = blockIdx.x >> 3;
  const int r = k / g;
  *item = 8 * r + (blockIdx.x & 7);
  *group = k - r * g;
}

// hd256.  A work-group takes one item and one group of up to kPrepHeads256
// heads of one row kind; of the g = nqg + 2 nkg groups of an item, group
// y < nqg -> Q heads, y < nqg + nkg -> K heads, else V heads.  The kinds
// interleave in dispatch order, so the V work-groups (a transpose through
// LDS, slower per byte) spread over the launch instead of all running at its
// end (-9% on 8192 tokens, with the smaller head groups).  Lane group tt (16
// lanes) owns token tt of the item and all the group's heads, so the RoPE
// rows of its position are loaded once, and every input row of the lane group
// is requested before the first one is used.
__global__ __launch_bounds__(256) void prep_hd256_kernel(PrepParams P) {
  constexpr int D = 256, LPR = 16, HALF = D / 2, HG = kPrepHeads256;
  const int nqg = (P.num_qo_heads + HG - 1) / HG;
  const int nkg = (P.num_kv_heads + HG - 1) / HG;
  int itx, y;
  xcd_item_group(nqg + 2 * nkg, &itx, &y);
  if (itx >= P.n_items) return;
  const Item it = read_item(P.items + kPrepItemInts * itx);
  if (!item_ok(P, it)) return;
  const int kind = y < nqg ? 0 : (y < nqg + nkg ? 1 : 2);
  const int hg = kind == 0 ? y : (kind == 1 ? y - nqg : y - nqg - nkg);
  const int heads = kind == 0 ? P.num_qo_heads : P.num_kv_heads;
  const int h0 = HG * hg;
  const int hcount = min(HG, heads - h0);
  const int li = threadIdx.x % LPR;
  const int tt = threadIdx.x / LPR;
  const bool live = tt < it.ntok;
  const int tok = it.tok0 + tt;
  const int pos = it.pos0 + tt;
  const int64_t page_off = P.layer_off + (int64_t)it.page * P.ps.page;

  constexpr int VST = HG;  // V heads staged per round (LDS: VST * 16 rows * 528 B)
  __shared__ __attribute__((aligned(16))) __bf16 vstage[VST * kPrepMaxTokens * (D + 8)];

  const __bf16* src = kind == 0 ? P.q_in + ((int64_t)tok * P.num_qo_heads + h0) * D
                    : kind == 1 ? P.k_in + ((int64_t)tok * P.num_kv_heads + h0) * D
                                : P.v_in + ((int64_t)tok * P.num_kv_heads + h0) * D;
  bf16x8 r1[HG], r2[HG];   // raw rows, widened when used
  if (live) {
#pragma unroll
    for (int h = 0; h < HG; ++h)
      if (h < hcount) {
        r1[h] = load8_stream(src + h * D + 8 * li);
        r2[h] = load8_stream(src + h * D + HALF + 8 * li);
      }
  }
  if (kind < 2) {
    float w1[8], w2[8], c[8], sn[8];
    const __bf16* wp = kind == 0 ? P.q_w : P.k_w;
    load8(wp + 8 * li, w1);
    load8(wp + HALF + 8 * li, w2);
    if (!live) return;
    load8f(P.cos + (int64_t)pos * HALF + 8 * li, c);
    load8f(P.sin + (int64_t)pos * HALF + 8 * li, sn);
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      if (h >= hcount) break;
      float x1[8], x2[8];
      widen8(r1[h], x1);
      widen8(r2[h], x2);
      const float inv = inv_rms<LPR>(x1, x2, 1.0f / D, P.eps);
      norm_rope<true, true>(x1, x2, w1, w2, c, sn, inv);
      __bf16* dst = kind == 0 ? P.q_out + ((int64_t)tok * P.num_qo_heads + h0 + h) * D
                              : P.pool + page_off + (int64_t)(h0 + h) * P.ps.head +
                                    (int64_t)(it.slot0 + tt) * D;
      store8_stream(dst + 8 * li, x1);
      store8_stream(dst + HALF + 8 * li, x2);
    }
    return;
  }

  // V: weightless norm, staged (VST heads per round) for the transpose into
  // the dim-major V block
#pragma unroll
  for (int r = 0; r < HG / VST; ++r) {
    if (VST * r >= hcount) break;
    if (live) {
#pragma unroll
      for (int j = 0; j < VST; ++j) {
        const int h = VST * r + j;
        if (h >= hcount) break;
        float x1[8], x2[8];
        widen8(r1[h], x1);
        widen8(r2[h], x2);
        const float inv = inv_rms<LPR>(x1, x2, 1.0f / D, P.eps);
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[e] = (__bf16)(x1[e] * inv);
          b[e] = (__bf16)(x2[e] * inv);
        }
        __bf16* vs = vstage + (j * kPrepMaxTokens + tt) * (D + 8);
        *reinterpret_cast<bf16x8*>(vs + 8 * li) = a;
        *reinterpret_cast<bf16x8*>(vs + HALF + 8 * li) = b;
      }
    }
    __syncthreads();
    store_v_transposed<D, 256>(P, vstage, it,
                               page_off + P.ps.kv + (int64_t)(h0 + VST * r) * P.ps.head,
                               min(VST, hcount - VST * r));
    __syncthreads();
  }
}

// hd512: one raw K row per (token, KV head) yields the K row (weighted norm +
// rope) and the V row (weightless norm, same inv, no rope).  Lane group g (32
// lanes) owns tokens g and g + 8 of the item.
__global__ __launch_bounds__(256) void prep_hd512_kernel(PrepParams P) {
  constexpr int D = 512, LPR = 32, HALF = D / 2, NG = 256 / LPR;
  constexpr int TPG = kPrepMaxTokens / NG;  // tokens per lane group
  const Item it = read_item(P.items + kPrepItemInts * blockIdx.x);
  if (!item_ok(P, it)) return;
  const int li = threadIdx.x % LPR;
  const int g = threadIdx.x / LPR;
  const int heads = P.num_kv_heads;
  const int64_t page_off = P.layer_off + (int64_t)it.page * P.ps.page;
  float w1[8], w2[8];
  load8(P.k_w + 8 * li, w1);
  load8(P.k_w + HALF + 8 * li, w2);

  __shared__ __attribute__((aligned(16))) __bf16 vstage[kPrepMaxTokens * (D + 8)];

  // the rotation rows of this lane group's tokens, loaded once, alongside
  // the first head's rows
  float c[TPG][8], sn[TPG][8];
#pragma unroll
  for (int k = 0; k < TPG; ++k) {
    const int tt = g + NG * k;
    const int pos = it.pos0 + min(tt, it.ntok - 1);
    load8f(P.cos + (int64_t)pos * HALF + 8 * li, c[k]);
    load8f(P.sin + (int64_t)pos * HALF + 8 * li, sn[k]);
  }
  for (int hd = 0; hd < heads; ++hd) {
    bf16x8 r1[TPG], r2[TPG];
#pragma unroll
    for (int k = 0; k < TPG; ++k) {
      const int tt = g + NG * k;
      if (tt < it.ntok) {
        const __bf16* src = P.k_in + ((int64_t)(it.tok0 + tt) * heads + hd) * D;
        r1[k] = load8_stream(src + 8 * li);
        r2[k] = load8_stream(src + HALF + 8 * li);
      }
    }
#pragma unroll
    for (int k = 0; k < TPG; ++k) {
      const int tt = g + NG * k;
      if (tt >= it.ntok) break;
      float x1[8], x2[8];
      widen8(r1[k], x1);
      widen8(r2[k], x2);
      const float inv = inv_rms<LPR>(x1, x2, 1.0f / D, P.eps);
      bf16x8 a, b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(x1[e] * inv);
        b[e] = (__bf16)(x2[e] * inv);
      }
      __bf16* vs = vstage + tt * (D + 8);
      *reinterpret_cast<bf16x8*>(vs + 8 * li) = a;
      *reinterpret_cast<bf16x8*>(vs + HALF + 8 * li) = b;
      norm_rope<true, true>(x1, x2, w1, w2, c[k], sn[k], inv);
      __bf16* dst = P.pool + page_off + (int64_t)hd * P.ps.head + (int64_t)(it.slot0 + tt) * D;
      store8_stream(dst + 8 * li, x1);
      store8_stream(dst + HALF + 8 * li, x2);
    }
    __syncthreads();
    store_v_transposed<D, 256>(P, vstage, it, page_off + P.ps.kv + (int64_t)hd * P.ps.head, 1);
    __syncthreads();
  }
}

// hd512 query prep: q_out row = rope(rms(q_in row) * q_norm_w, p), written
// contiguously.  Work-group: one item (<= 16 consecutive positions of one
// request) x kQHeads heads; lane group g (32 lanes) owns tokens g and g + 8 of
// the item, all of the work-group's heads, so a token's rotation rows are read
// once.  Only positions are checked on the device (no pool is touched).
constexpr int kQHeads = 2;  // 2: 8% faster than 4 on 8192 tokens x 16 heads
__global__ __launch_bounds__(256) void prep_q_hd512_kernel(PrepParams P) {
  constexpr int D = 512, LPR = 32, HALF = D / 2, NG = 256 / LPR, HG = kQHeads;
  constexpr int TPG = kPrepMaxTokens / NG;  // tokens per lane group
  int itx, hgi;
  xcd_item_group((P.num_qo_heads + HG - 1) / HG, &itx, &hgi);
  if (itx >= P.n_items) return;
  const Item it = read_item(P.items + kPrepItemInts * itx);
  const bool ok = it.pos0 >= 0 && it.ntok >= 1 && it.ntok <= kPrepMaxTokens &&
                  it.pos0 + it.ntok <= P.rope_positions;
  if (!ok) {
    if (threadIdx.x == 0) {
      P.err[0] = 1;
      P.err[1] = -1;
      P.err[2] = it.pos0 + it.ntok - 1;
    }
    return;
  }
  const int li = threadIdx.x % LPR;
  const int g = threadIdx.x / LPR;
  const int h0 = HG * hgi;
  const int hcount = min(HG, P.num_qo_heads - h0);
  float w1[8], w2[8];
  load8(P.q_w + 8 * li, w1);
  load8(P.q_w + HALF + 8 * li, w2);
  // every load of the lane group first: rows and rotation rows in flight together
  float c[TPG][8], sn[TPG][8];
  bf16x8 r1[TPG][HG], r2[TPG][HG];
#pragma unroll
  for (int k = 0; k < TPG; ++k) {
    const int tt = g + NG * k;
    if (tt >= it.ntok) break;
    const int pos = it.pos0 + tt;
    load8f(P.cos + (int64_t)pos * HALF + 8 * li, c[k]);
    load8f(P.sin + (int64_t)pos * HALF + 8 * li, sn[k]);
    const __bf16* src = P.q_in + ((int64_t)(it.tok0 + tt) * P.num_qo_heads + h0) * D;
#pragma unroll
    for (int h = 0; h < HG; ++h)
      if (h < hcount) {
        r1[k][h] = load8_stream(src + h * D + 8 * li);
        r2[k][h] = load8_stream(src + h * D + HALF + 8 * li);
      }
  }
#pragma unroll
  for (int k = 0; k < TPG; ++k) {
    const int tt = g + NG * k;
    if (tt >= it.ntok) break;
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      if (h >= hcount) break;
      float x1[8], x2[8];
      widen8(r1[k][h], x1);
      widen8(r2[k][h], x2);
      const float inv = inv_rms<LPR>(x1, x2, 1.0f / D, P.eps);
      norm_rope<true, true>(x1, x2, w1, w2, c[k], sn[k], inv);
      __bf16* dst = P.q_out + ((int64_t)(it.tok0 + tt) * P.num_qo_heads + h0 + h) * D;
      store8_stream(dst + 8 * li, x1);
      store8_stream(dst + HALF + 8 * li, x2);
    }
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
  const int64_t groups = (p.num_qo_heads + kPrepHeads256 - 1) / kPrepHeads256 +
                         2 * ((p.num_kv_heads + kPrepHeads256 - 1) / kPrepHeads256);
  const int64_t blocks = (((int64_t)n_items + 7) / 8) * 8 * groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  PrepParams q = p;
  q.n_items = n_items;
  hipLaunchKernelGGL(prep_hd256_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_prep_hd512(const PrepParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(prep_hd512_kernel, dim3(n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prep_q_hd512(const PrepParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const int64_t groups = (p.num_qo_heads + kQHeads - 1) / kQHeads;
  const int64_t blocks = (((int64_t)n_items + 7) / 8) * 8 * groups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  PrepParams q = p;
  q.n_items = n_items;
  hipLaunchKernelGGL(prep_q_hd512_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q);
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
