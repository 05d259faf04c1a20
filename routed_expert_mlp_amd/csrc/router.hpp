// Sigmoid router top-k of the GLM-5.3-Flash routed MLP ("Module glm5next_mlp",
// sections "The stack this layer runs" and "Traps this module exists to
// hold", Constants KERNEL_MAX_TOP_K).  fp32 logits from the router weight; the
// correction bias only changes which experts are chosen; a chosen expert's
// weight is its plain sigmoid score over the sum of the chosen plain scores
// (full expert count), times routed_scaling_factor; K <= 16.
//
// Logits are fp32 with a blocked accumulation order (short sequential runs,
// then a tree or a sum of partials) so the emitted weights stay within 1e-6
// relative of an fp64 evaluation.
#pragma once

#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Logits for few tokens (decode): one workgroup per expert, threads stride
// over H in float4 chunks, tokens processed in groups of TG.
// ---------------------------------------------------------------------------
constexpr int LOGIT_TG = 8;

__global__ __launch_bounds__(256) void k_logits_gemv(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ wr,
                                                     float* __restrict__ logits, int T, int H, int E) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nchunk = H >> 2;                    // float4 chunks per row
  const float4* wrow = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H);
  __shared__ float red[4][LOGIT_TG];
  for (int t0 = 0; t0 < T; t0 += LOGIT_TG) {
    const int nt = min(LOGIT_TG, T - t0);
    float acc[LOGIT_TG];
#pragma unroll
    for (int t = 0; t < LOGIT_TG; ++t) acc[t] = 0.0f;
    for (int c = tid; c < nchunk; c += 256) {
      const float4 w4 = wrow[c];
#pragma unroll
      for (int t = 0; t < LOGIT_TG; ++t) {
        if (t < nt) {
          const uint2 xb = *reinterpret_cast<const uint2*>(x + static_cast<int64_t>(t0 + t) * H + 4 * c);
          float a = acc[t];
          a = fmaf(__uint_as_float(xb.x << 16), w4.x, a);
          a = fmaf(__uint_as_float(xb.x & 0xffff0000u), w4.y, a);
          a = fmaf(__uint_as_float(xb.y << 16), w4.z, a);
          a = fmaf(__uint_as_float(xb.y & 0xffff0000u), w4.w, a);
          acc[t] = a;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < LOGIT_TG; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) red[wv][t] = s;
    }
    __syncthreads();
    if (tid < nt) {
      const float s = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
      logits[static_cast<int64_t>(t0 + tid) * E + e] = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Logits for up to a few hundred tokens, H a multiple of 8 up to 2048 CPT:
// workgroup (b, g) takes experts NE b .. NE b + NE - 1 and tokens LOGIT_TG g ..
// + LOGIT_TG - 1.  Thread tid keeps the experts' weights at columns
// 8 (tid + 256 i) .. + 7 (i < CPT) in registers and reads each token's
// matching 16 bytes once for all NE experts, every load issued before the
// first product.  grid.x is a multiple of 8, so all token groups of an expert
// block run on one XCD (blocks go to the XCDs round-robin) and read its
// weight rows from that XCD's L2.  Per logit: a sequential fmaf run over the
// thread's columns, a wave tree, then the four waves' sums.
// ---------------------------------------------------------------------------
template <int CPT, int NE>
__global__ __launch_bounds__(256) void k_logits_rows(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     float* __restrict__ logits, int T, int H, int E) {
  const int e0 = blockIdx.x * NE;
  if (e0 >= E) return;
  const int t0 = blockIdx.y * LOGIT_TG;
  const int nt = min(LOGIT_TG, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n8 = H >> 3;
  float4 w[NE][CPT][2];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    const float4* row = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(min(e0 + n, E - 1)) * H);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      w[n][i][0] = c < n8 ? row[2 * c] : make_float4(0.f, 0.f, 0.f, 0.f);
      w[n][i][1] = c < n8 ? row[2 * c + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // tokens past T read token T - 1 again (their sums are dropped)
  uint4 xv[LOGIT_TG][CPT];
#pragma unroll
  for (int t = 0; t < LOGIT_TG; ++t) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(min(t0 + t, T - 1)) * H);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      xv[t][i] = c < n8 ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __shared__ float red[4][NE * LOGIT_TG];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
#pragma unroll
    for (int t = 0; t < LOGIT_TG; ++t) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const uint4 v = xv[t][i];
        const float4 wa = w[n][i][0], wb = w[n][i][1];
        a = fmaf(__uint_as_float(v.x << 16), wa.x, a);
        a = fmaf(__uint_as_float(v.x & 0xffff0000u), wa.y, a);
        a = fmaf(__uint_as_float(v.y << 16), wa.z, a);
        a = fmaf(__uint_as_float(v.y & 0xffff0000u), wa.w, a);
        a = fmaf(__uint_as_float(v.z << 16), wb.x, a);
        a = fmaf(__uint_as_float(v.z & 0xffff0000u), wb.y, a);
        a = fmaf(__uint_as_float(v.w << 16), wb.z, a);
        a = fmaf(__uint_as_float(v.w & 0xffff0000u), wb.w, a);
      }
      const float s = wave_sum(a);
      if (lane == 0) red[wv][n * LOGIT_TG + t] = s;
    }
  }
  __syncthreads();
  if (tid < NE * LOGIT_TG) {
    const int n = tid / LOGIT_TG, t = tid - n * LOGIT_TG;
    if (e0 + n < E && t < nt)
      logits[static_cast<int64_t>(t0 + t) * E + e0 + n] =
          (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
  }
}

// ---------------------------------------------------------------------------
// Logits for many tokens (prefill): fp32 tiled GEMM on the vector ALUs,
// 64 tokens x 64 experts per workgroup, each thread 4 x 4 outputs.  Every
// 32-wide k tile is summed into a fresh partial before joining the total.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_gemm(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ wr,
                                                     float* __restrict__ logits, int T, int H, int E) {
  constexpr int BT = 64, BE = 64, BKk = 32;
  __shared__ float xs[BKk][BT + 4];
  __shared__ float ws[BKk][BE + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;   // x: token tiles, y: expert tiles
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4], part[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  // loaders: x tile 64 x 32 bf16 -> each thread 8 bf16; w tile 64 x 32 fp32 -> each thread 8 fp32
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  for (int k0 = 0; k0 < H; k0 += BKk) {
    {
      const int t = t0 + lr;
      uint4 xv = make_uint4(0, 0, 0, 0);
      if (t < T) xv = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H + k0 + lk);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[lk + 2 * q][lr] = __uint_as_float(xw[q] << 16);
        xs[lk + 2 * q + 1][lr] = __uint_as_float(xw[q] & 0xffff0000u);
      }
      const int e = e0 + lr;
      float4 w0 = make_float4(0, 0, 0, 0), w1 = w0;
      if (e < E) {
        const float4* p = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H + k0 + lk);
        w0 = p[0];
        w1 = p[1];
      }
      ws[lk + 0][lr] = w0.x; ws[lk + 1][lr] = w0.y; ws[lk + 2][lr] = w0.z; ws[lk + 3][lr] = w0.w;
      ws[lk + 4][lr] = w1.x; ws[lk + 5][lr] = w1.y; ws[lk + 6][lr] = w1.z; ws[lk + 7][lr] = w1.w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[i][j] = 0.0f;
#pragma unroll 8
    for (int k = 0; k < BKk; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[static_cast<int64_t>(t) * E + e] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token by one wavefront.  Candidate e's key is
//     (order-preserving bits of its biased score) << 32 | (0xFFFFFFFF - e),
// so a larger key is a larger score and, between equal scores, the lower id
// (keys are distinct).  Each lane sorts its NJ keys (experts lane + 64 j,
// E <= 64 * NJ) descending once; a round finds the largest of the lanes'
// first keys and the owning lane drops its first key.  The round reduces the
// 32-bit score halves only (DPP max within rows of 16, then the 4 row
// winners) and takes the id half into account only when several lanes hold
// the top score, which keeps the dependent chain short: the wavefront sits on
// the decode critical path.  Returns the id in slot `want`.  With ids != null all K rounds run
// and ids/wts (and ids2/wts2 when not null) are written: the weight of slot k
// is its unbiased sigmoid score over the sum of the K chosen scores (added in
// slot order) times rsf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_order_bits(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);   // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t u64_of(uint32_t lo, uint32_t hi) {
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(dpp_mov<CTRL>(static_cast<int>(v)));
  return o > v ? o : v;
}

// Wave-wide max of a 32-bit value (wave-uniform result).  All lanes active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<DPP_QUAD_1032>(v);
  v = dpp_max_u32<DPP_QUAD_2301>(v);
  v = dpp_max_u32<DPP_ROW_HALF_MIRROR>(v);
  v = dpp_max_u32<DPP_ROW_MIRROR>(v);
  const uint32_t a = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const uint32_t b = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const uint32_t c = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const uint32_t d = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return max(max(a, b), max(c, d));
}

// Logit e of a row: one fp32 value, or (planes == 3, the split-weight router
// GEMM) the sum of the three partial logits against the hi, mid and lo bf16
// parts of the router weight, added as (lo + mid) + hi.  With splits > 1 the
// GEMM's reduction was cut into that many parts whose rows sit sstride floats
// apart; their sums are added in part order.
__device__ __forceinline__ float logit_of(const float* __restrict__ lrow, int E, int planes, int e, int splits = 1,
                                          int64_t sstride = 0) {
  float v = planes == 3 ? (lrow[2 * E + e] + lrow[E + e]) + lrow[e] : lrow[e];
  for (int q = 1; q < splits; ++q) {
    const float* l = lrow + q * sstride;
    v += planes == 3 ? (l[2 * E + e] + l[E + e]) + l[e] : l[e];
  }
  return v;
}

// Sort key of expert e with router logit l and correction bias b (the biased
// sigmoid score decides, then the lower id).  Every top-k path builds its
// keys with this one expression, so they rank the experts bit for bit alike.
__device__ __forceinline__ uint64_t topk_key(float l, float b, int e) {
  return u64_of(0xFFFFFFFFu - static_cast<uint32_t>(e), f32_order_bits(1.0f / (1.0f + expf(-l)) + b));
}

// The rounds of topk_wave over this lane's NJ keys (experts lane + 64 j;
// 0 for none), the winners' weights from their logits (lrow, planes, splits
// as in logit_of).
template <int NJ>
__device__ __forceinline__ int topk_rounds(uint64_t (&key)[NJ], const float* __restrict__ lrow, int E, int K,
                                           float rsf, int want, int32_t* ids, float* wts, int32_t* ids2,
                                           float* wts2, int planes, int splits, int64_t sstride) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NJ - 1; ++i)
#pragma unroll
    for (int j = 0; j < NJ - 1 - i; ++j) {
      const uint64_t a = key[j], b = key[j + 1];
      const bool sw = b > a;
      key[j] = sw ? b : a;
      key[j + 1] = sw ? a : b;
    }
  // Each round takes the largest head key.  The score half decides first (a
  // 32-bit wave max); only when several lanes hold that score does the id half
  // (larger ~id = smaller id) decide, in a second 32-bit max over those lanes.
  uint32_t kh[NJ], kl[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    kh[j] = static_cast<uint32_t>(key[j] >> 32);
    kl[j] = static_cast<uint32_t>(key[j]);
  }
  const int nr = ids ? K : want + 1;
  int want_id = 0, my_id = 0;
  for (int k = 0; k < nr; ++k) {
    const uint32_t m = wave_max_u32(kh[0]);
    uint64_t top = __builtin_amdgcn_ballot_w64(kh[0] == m);
    if (__popcll(top) > 1) {
      const uint32_t c = wave_max_u32(kh[0] == m ? kl[0] : 0u);
      top = __builtin_amdgcn_ballot_w64(kh[0] == m && kl[0] == c);
    }
    const int win = static_cast<int>(__builtin_ctzll(top));
    const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(kl[0]), win)));
    if (lane == win) {
#pragma unroll
      for (int j = 0; j < NJ - 1; ++j) {
        kh[j] = kh[j + 1];
        kl[j] = kl[j + 1];
      }
      kh[NJ - 1] = 0;
      kl[NJ - 1] = 0;
    }
    if (k == want) want_id = id;
    if (lane == k) my_id = id;
  }
  if (ids) {
    // the same expression as in topk_key on the same logit: the same bits
    const float my_s = lane < K ? 1.0f / (1.0f + expf(-logit_of(lrow, E, planes, my_id, splits, sstride))) : 0.0f;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    if (lane < K) {
      const float w = my_s / sum * rsf;
      ids[lane] = my_id;
      wts[lane] = w;
      if (ids2) ids2[lane] = my_id;
      if (wts2) wts2[lane] = w;
    }
  }
  return want_id;
}

template <int NJ>
__device__ __forceinline__ int topk_wave(const float* __restrict__ lrow, const float* __restrict__ bias, int E,
                                         int K, float rsf, int want, int32_t* ids, float* wts, int32_t* ids2,
                                         float* wts2, int planes = 1, int splits = 1, int64_t sstride = 0) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? topk_key(logit_of(lrow, E, planes, e, splits, sstride), bias[e], e) : 0;   // 0: below every real key
  }
  return topk_rounds<NJ>(key, lrow, E, K, rsf, want, ids, wts, ids2, wts2, planes, splits, sstride);
}

// topk_wave on keys the logits kernel already built with topk_key (one
// fp32 logit per expert, no planes or parts).
template <int NJ>
__device__ __forceinline__ int topk_wave_keys(const uint64_t* __restrict__ keys, const float* __restrict__ lrow,
                                              int E, int K, float rsf, int want, int32_t* ids, float* wts,
                                              int32_t* ids2, float* wts2) {
  const int lane = threadIdx.x & 63;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? keys[e] : 0;
  }
  return topk_rounds<NJ>(key, lrow, E, K, rsf, want, ids, wts, ids2, wts2, 1, 1, 0);
}

template <int NJ>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int K, float rsf, int32_t* __restrict__ ids,
                                              float* __restrict__ wts, int32_t* ids_out, float* w_out,
                                              int planes, int splits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t o = static_cast<int64_t>(t) * K;
  topk_wave<NJ>(logits + static_cast<int64_t>(t) * E * planes, bias, E, K, rsf, 0, ids + o, wts + o,
                ids_out ? ids_out + o : nullptr, w_out ? w_out + o : nullptr, planes, splits,
                static_cast<int64_t>(T) * E * planes);
}

// ---------------------------------------------------------------------------
// Router weight for the matrix cores: each fp32 w splits exactly into three
// bf16 parts, hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each
// difference is exact in fp32 and the last part has at most 8 significant
// bits left), so x . w = x . hi + x . mid + x . lo with every bf16 x bf16
// product exact in fp32.  Planes [3][n] (hi, mid, lo); 8 values per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_split_bf16x3(const float* __restrict__ w, uint16_t* __restrict__ planes,
                                                      int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const float4 a = *reinterpret_cast<const float4*>(w + i);
  const float4 b = *reinterpret_cast<const float4*>(w + i + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r0[2], r1[2], r2[2];
    uint16_t h[2], m[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      r0[u] = v[2 * q + u];
      h[u] = f32_to_bf16(r0[u]);
      r1[u] = r0[u] - bf16_to_f32(h[u]);
      m[u] = f32_to_bf16(r1[u]);
      r2[u] = r1[u] - bf16_to_f32(m[u]);
    }
    hi[q] = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
    mid[q] = static_cast<uint32_t>(m[0]) | (static_cast<uint32_t>(m[1]) << 16);
    lo[q] = pack_bf16x2(r2[0], r2[1]);
  }
  *reinterpret_cast<uint4*>(planes + i) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4*>(planes + n + i) = make_uint4(mid[0], mid[1], mid[2], mid[3]);
  *reinterpret_cast<uint4*>(planes + 2 * n + i) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ---------------------------------------------------------------------------
// Decode: top-k for every token plus the per-expert token lists, in one
// workgroup of 1024 threads (T * K <= 4096 slots).  Groups are the touched
// experts in ascending id order; a group's slot list order is unspecified
// (each slot's result does not depend on it).
// ---------------------------------------------------------------------------
struct Groups {
  int32_t* n_groups;   // [1]
  int32_t* expert;     // [E]
  int32_t* count;      // [E]
  int32_t* offset;     // [E]
  int32_t* slots;      // [T*K]
};

template <int NJ>
__global__ __launch_bounds__(1024) void k_topk_bucket(const float* __restrict__ logits,
                                                      const float* __restrict__ bias, int T, int E, int K,
                                                      float rsf, int32_t* __restrict__ ids,
                                                      float* __restrict__ wts, int32_t* ids_out,
                                                      float* w_out, Groups g) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_off[1024];
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  for (int t = wv; t < T; t += 16) {
    const int64_t o = static_cast<int64_t>(t) * K;
    topk_wave<NJ>(logits + static_cast<int64_t>(t) * E, bias, E, K, rsf, 0, ids + o, wts + o,
                  ids_out ? ids_out + o : nullptr, w_out ? w_out + o : nullptr);
  }
  __threadfence_block();
  __syncthreads();
  const int nslot = T * K;
  for (int i = tid; i < nslot; i += 1024) atomicAdd(&s_cnt[ids[i]], 1);
  __syncthreads();
  // exclusive scans over experts of (count) and (count > 0): one element per thread
  const int c = tid < E ? s_cnt[tid] : 0;
  const int flag = c > 0 ? 1 : 0;
  int inc_c = c, inc_f = flag;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int a = __shfl_up(inc_c, m, 64);
    const int b = __shfl_up(inc_f, m, 64);
    if (lane >= m) {
      inc_c += a;
      inc_f += b;
    }
  }
  if (lane == 63) s_wsum[wv] = (inc_c & 0xffff) | (inc_f << 16);
  __syncthreads();
  int base_c = 0, base_f = 0;
  for (int w = 0; w < wv; ++w) {
    base_c += s_wsum[w] & 0xffff;
    base_f += s_wsum[w] >> 16;
  }
  const int off = base_c + inc_c - c;
  const int grp = base_f + inc_f - flag;
  if (tid < E) {
    s_off[tid] = off;
    if (flag) {
      g.expert[grp] = tid;
      g.count[grp] = c;
      g.offset[grp] = off;
    }
    if (tid == E - 1) *g.n_groups = grp + flag;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < nslot; i += 1024) {
    const int e = ids[i];
    const int pos = s_off[e] + atomicAdd(&s_cnt[e], 1);
    g.slots[pos] = i;
  }
}

}  // namespace moe
