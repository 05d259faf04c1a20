// One-token decode ("Module glm5next_mlp", modules: forward -- the GLM MLP
// decode forward, one token).  Three launches stream every weight byte once:
//
//   1. k_dec_logits_shared: router logits (fp32 rows of gate.weight) and the
//      BF16 shared expert's gate/up + clamped SwiGLU, both of which only need
//      x, in one grid;
//   2. k_dec_gateup: its first blocks stream the shared expert's BF16 down
//      rows (ys = W2s hs, fp32), which need nothing from the router, while
//      the other blocks first redo the router top-k from the E logits
//      (router.hpp topk_wave; "Traps": bias steers selection only, weights
//      are the renormalised unbiased scores times rsf) to learn which expert
//      they serve, then stream its NVFP4 gate/up rows + clamped SwiGLU -> h
//      (bf16).  One wavefront also writes ids and weights.  The shared rows
//      keep HBM busy while the selection runs, and redoing the selection
//      (~1 KB of logits per wavefront) is cheaper than a launch of its own;
//   3. k_dec_down_combine: routed NVFP4 down rows of all K experts and the
//      combine out = bf16(ys + sum_k w_k y_k) for a block of output rows
//      (fixed k order).
//
// Each wavefront issues all loads of its rows before using any of them, so a
// wavefront has its whole share of the weight stream in flight at once.
#pragma once

#include "common.hpp"
#include "gemv.hpp"
#include "router.hpp"

namespace moe {

// Lane l of a wavefront covers chunks l, l+64, ..., of a row (one coalesced
// 1 KB load per instruction); a chunk is 16 bytes.

// -------------------------------------------------------------------------
// 1. logits + shared gate/up.  Blocks [0, n_logit_blocks) take 4 router rows
// each (one per wavefront), the rest take 4 shared (gate, up) row pairs.
//   NR: float4 chunks per lane of a router row (>= H / 256)
//   NS: 8-bf16 chunks per lane of a shared row (>= H / 512)
// -------------------------------------------------------------------------
template <int NR, int NS>
__global__ __launch_bounds__(256) void k_dec_logits_shared(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr, float* __restrict__ logits,
                                                           int E, int H, const uint16_t* __restrict__ sw13, int Is,
                                                           uint16_t* __restrict__ hs, float L, int n_logit_blocks) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) < n_logit_blocks) {
    const int e = blockIdx.x * 4 + wv;
    if (e >= E) return;
    const float4* row = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H);
    const uint2* xv = reinterpret_cast<const uint2*>(x);
    float4 w[NR];
    uint2 xs[NR];
    const int nch = H >> 2;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = lane + 64 * i;
      w[i] = c < nch ? row[c] : make_float4(0, 0, 0, 0);
      xs[i] = c < nch ? xv[c] : make_uint2(0, 0);
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      acc = fmaf(__uint_as_float(xs[i].x << 16), w[i].x, acc);
      acc = fmaf(__uint_as_float(xs[i].x & 0xffff0000u), w[i].y, acc);
      acc = fmaf(__uint_as_float(xs[i].y << 16), w[i].z, acc);
      acc = fmaf(__uint_as_float(xs[i].y & 0xffff0000u), w[i].w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[e] = acc;
  } else {
    const int j = (blockIdx.x - n_logit_blocks) * 4 + wv;
    if (j >= Is) return;
    const uint4* g = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(j) * H);
    const uint4* u = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(Is + j) * H);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    const int nch = H >> 3;
    uint4 wg[NS], wu[NS], xs[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch;
      wg[i] = ok ? g[c] : make_uint4(0, 0, 0, 0);
      wu[i] = ok ? u[c] : make_uint4(0, 0, 0, 0);
      xs[i] = ok ? xv[c] : make_uint4(0, 0, 0, 0);
    }
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint32_t xp[4] = {xs[i].x, xs[i].y, xs[i].z, xs[i].w};
      ag = dot2_bf16(wg[i].x, xp[0], ag); ag = dot2_bf16(wg[i].y, xp[1], ag);
      ag = dot2_bf16(wg[i].z, xp[2], ag); ag = dot2_bf16(wg[i].w, xp[3], ag);
      au = dot2_bf16(wu[i].x, xp[0], au); au = dot2_bf16(wu[i].y, xp[1], au);
      au = dot2_bf16(wu[i].z, xp[2], au); au = dot2_bf16(wu[i].w, xp[3], au);
    }
    ag = wave_sum(ag);
    au = wave_sum(au);
    if (lane == 0) hs[j] = f32_to_bf16(swiglu_clamped(ag, au, L));
  }
}

// -------------------------------------------------------------------------
// 1'. The same grid for T <= 16 tokens (general decode): each wavefront
// loads its router row (or shared gate/up row pair) once, then runs every
// token's dot product against it; x rows are re-read per token (they stay in
// the caches).  Per token the arithmetic and reduction order are those of
// k_dec_logits_shared.  Writes logits [T][E] and hs [T][Is].
// -------------------------------------------------------------------------
template <int NR, int NS>
__global__ __launch_bounds__(256) void k_dec_logits_shared_t(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             float* __restrict__ logits, int E, int H,
                                                             const uint16_t* __restrict__ sw13, int Is,
                                                             uint16_t* __restrict__ hs, float L, int n_logit_blocks,
                                                             int T) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) < n_logit_blocks) {
    const int e = blockIdx.x * 4 + wv;
    if (e >= E) return;
    const float4* row = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H);
    float4 w[NR];
    const int nch = H >> 2;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = lane + 64 * i;
      w[i] = c < nch ? row[c] : make_float4(0, 0, 0, 0);
    }
    for (int t = 0; t < T; ++t) {
      const uint2* xv = reinterpret_cast<const uint2*>(x + static_cast<int64_t>(t) * H);
      uint2 xs[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int c = lane + 64 * i;
        xs[i] = c < nch ? xv[c] : make_uint2(0, 0);
      }
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        acc = fmaf(__uint_as_float(xs[i].x << 16), w[i].x, acc);
        acc = fmaf(__uint_as_float(xs[i].x & 0xffff0000u), w[i].y, acc);
        acc = fmaf(__uint_as_float(xs[i].y << 16), w[i].z, acc);
        acc = fmaf(__uint_as_float(xs[i].y & 0xffff0000u), w[i].w, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) logits[static_cast<int64_t>(t) * E + e] = acc;
    }
  } else {
    const int j = (blockIdx.x - n_logit_blocks) * 4 + wv;
    if (j >= Is) return;
    const uint4* g = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(j) * H);
    const uint4* u = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(Is + j) * H);
    const int nch = H >> 3;
    uint4 wg[NS], wu[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch;
      wg[i] = ok ? g[c] : make_uint4(0, 0, 0, 0);
      wu[i] = ok ? u[c] : make_uint4(0, 0, 0, 0);
    }
    for (int t = 0; t < T; ++t) {
      const uint4* xv = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * H);
      float ag = 0.0f, au = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int c = lane + 64 * i;
        const uint4 xs = c < nch ? xv[c] : make_uint4(0, 0, 0, 0);
        const uint32_t xp[4] = {xs.x, xs.y, xs.z, xs.w};
        ag = dot2_bf16(wg[i].x, xp[0], ag); ag = dot2_bf16(wg[i].y, xp[1], ag);
        ag = dot2_bf16(wg[i].z, xp[2], ag); ag = dot2_bf16(wg[i].w, xp[3], ag);
        au = dot2_bf16(wu[i].x, xp[0], au); au = dot2_bf16(wu[i].y, xp[1], au);
        au = dot2_bf16(wu[i].z, xp[2], au); au = dot2_bf16(wu[i].w, xp[3], au);
      }
      ag = wave_sum(ag);
      au = wave_sum(au);
      if (lane == 0) hs[static_cast<int64_t>(t) * Is + j] = f32_to_bf16(swiglu_clamped(ag, au, L));
    }
  }
}

// -------------------------------------------------------------------------
// 2. shared down + top-k + routed gate/up for one token.  1-D grid:
//  * blocks [0, n_sd): shared down rows r = (b*4 + wave)*RS .. +RS,
//    ys[r] = sum_j W2s[r, j] hs[j] in fp32 (lane l takes the 16-byte chunks
//    l, l+64, ... of each row, NSC of them);
//  * blocks n_sd + a: slot k = a / njb finds its expert (topk_wave,
//    NJ >= E / 64) and runs gate rows j = ((a % njb)*4 + wave)*RJ .. +RJ and
//    up rows I + j, njb = ceil(I / (4 RJ)).  Lane l covers the 16-byte chunks
//    l, l+64, ... (NC of them) of each row, so every load instruction reads
//    1 KB contiguous.  Wavefront 0 of the first gate/up block runs all K
//    rounds and writes ids/wts (and ids_out/w_out when not null).
// -------------------------------------------------------------------------
template <int RJ, int NC, int NJ, int RS, int NSC>
__global__ __launch_bounds__(256) void k_dec_gateup(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q13,
                                                    const uint8_t* __restrict__ s13, const float* __restrict__ g13,
                                                    const float* __restrict__ logits, const float* __restrict__ bias,
                                                    int K, float rsf, int32_t* __restrict__ ids,
                                                    float* __restrict__ wts, int32_t* ids_out, float* w_out, int E,
                                                    int H, int I, float L, uint16_t* __restrict__ h,
                                                    const uint16_t* __restrict__ sw2, const uint16_t* __restrict__ hs,
                                                    int Is, float* __restrict__ ys, int n_sd, int T) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) < n_sd) {
    const int r0 = (blockIdx.x * 4 + wv) * RS;
    if (r0 >= H) return;
    const int nsc = Is >> 3;                     // 8-bf16 chunks per row
    uint4 w[RS][NSC];
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const uint4* row = reinterpret_cast<const uint4*>(sw2 + static_cast<int64_t>(min(r0 + r, H - 1)) * Is);
#pragma unroll
      for (int i = 0; i < NSC; ++i) {
        const int c = lane + 64 * i;
        w[r][i] = c < nsc ? row[c] : make_uint4(0, 0, 0, 0);
      }
    }
    for (int t = 0; t < T; ++t) {
      uint32_t hv[NSC][4];
#pragma unroll
      for (int i = 0; i < NSC; ++i) {
        const int c = lane + 64 * i;
        const uint4 v = c < nsc ? reinterpret_cast<const uint4*>(hs + static_cast<int64_t>(t) * Is)[c]
                                : make_uint4(0, 0, 0, 0);
        hv[i][0] = v.x; hv[i][1] = v.y; hv[i][2] = v.z; hv[i][3] = v.w;
      }
      float acc[RS];
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        acc[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < NSC; ++i) acc[r] = bf16_chunk_dot(w[r][i], hv[i], acc[r]);
        acc[r] = wave_sum(acc[r]);
      }
      if (lane < RS) {
        float v = acc[0];
#pragma unroll
        for (int r = 1; r < RS; ++r)
          if (lane == r) v = acc[r];
        if (r0 + lane < H) ys[static_cast<int64_t>(t) * H + r0 + lane] = v;
      }
    }
    return;
  }
  const int a = blockIdx.x - n_sd;
  const int njb = static_cast<int>(cdiv(I, 4 * RJ));
  const int slot = a / njb;                          // t * K + k
  const int t = slot / K, k = slot - t * K;
  const int jb = a - slot * njb;
  const int j0 = (jb * 4 + wv) * RJ;
  if (j0 >= I) return;
  const bool writer = jb == 0 && k == 0 && wv == 0;
  const int64_t o = static_cast<int64_t>(t) * K;
  const int sel = topk_wave<NJ>(logits + static_cast<int64_t>(t) * E, bias, E, K, rsf, k, writer ? ids + o : nullptr,
                                wts + o, ids_out ? ids_out + o : nullptr, w_out ? w_out + o : nullptr);
  x += static_cast<int64_t>(t) * H;
  const int e = min(max(sel, 0), E - 1);
  const int64_t rq = H >> 1, rs = H >> 4;                 // code / scale bytes per row
  const uint8_t* qe = q13 + static_cast<int64_t>(e) * 2 * I * rq;
  const uint8_t* se = s13 + static_cast<int64_t>(e) * 2 * I * rs;
  const int nch = H >> 5;
  uint4 cg[RJ][NC], cu[RJ][NC];
  uint32_t sg[RJ][NC], su[RJ][NC];
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    const int j = min(j0 + r, I - 1);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch;
      cg[r][i] = ok ? *reinterpret_cast<const uint4*>(qe + j * rq + 16 * c) : make_uint4(0, 0, 0, 0);
      cu[r][i] = ok ? *reinterpret_cast<const uint4*>(qe + (I + j) * rq + 16 * c) : make_uint4(0, 0, 0, 0);
      sg[r][i] = ok ? *reinterpret_cast<const uint16_t*>(se + j * rs + 2 * c) : 0u;
      su[r][i] = ok ? *reinterpret_cast<const uint16_t*>(se + (I + j) * rs + 2 * c) : 0u;
    }
  }
  float ag[RJ], au[RJ];
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    ag[r] = 0.0f;
    au[r] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    uint32_t xp[16];
    const uint4* xv = reinterpret_cast<const uint4*>(x + 32 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = c < nch ? xv[q] : make_uint4(0, 0, 0, 0);
      xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < RJ; ++r) {
      ag[r] = nvfp4_chunk_dot(cg[r][i], sg[r][i], xp, ag[r]);
      au[r] = nvfp4_chunk_dot(cu[r][i], su[r][i], xp, au[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    ag[r] = wave_sum(ag[r]);
    au[r] = wave_sum(au[r]);
  }
  if (lane < RJ) {
    float gg = ag[0], uu = au[0];
#pragma unroll
    for (int r = 1; r < RJ; ++r)
      if (lane == r) {
        gg = ag[r];
        uu = au[r];
      }
    const int j = j0 + lane;
    if (j < I)
      h[static_cast<int64_t>(slot) * I + j] =
          f32_to_bf16(swiglu_clamped(g13[2 * e] * gg, g13[2 * e + 1] * uu, L));
  }
}

// -------------------------------------------------------------------------
// 3. routed down + combine for T tokens (T*K slots, slot = t*K + k).  Block
// b owns output rows r0 = b*R .. +R and has KW wavefronts; wavefront w
// streams those R rows of expert ids[s]'s NVFP4 down projection against h_s
// for its slots s = w, w + KW, ... (NP of them; one 16-byte chunk per lane,
// lanes < I/32, the h_s chunk in registers), every load issued before any
// arithmetic.  Per-(slot, row) partials meet in LDS and thread (t, r) writes
// out[t][r0+r] = bf16(ys[t] + sum_k (w_{tK+k} g2) acc_{tK+k}), k in order
// (ys = 0 without a shared expert).
// -------------------------------------------------------------------------
template <int R, int KW, int NP>
__global__ __launch_bounds__(KW * 64) void k_dec_down_combine(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ q2, const uint8_t* __restrict__ s2,
    const float* __restrict__ g2, const float* __restrict__ ys, const int32_t* __restrict__ ids,
    const float* __restrict__ wts, int E, int K, int H, int I, uint16_t* __restrict__ out, int T) {
  __shared__ float part[KW * NP][R];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r0 = blockIdx.x * R;
  const int S = T * K;
  const int64_t rq = I >> 1, rs = I >> 4;
  int e[NP];
  bool act[NP];
  uint4 cw[NP][R];
  uint32_t sc[NP][R];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = wv + KW * p;
    const bool routed = sl < S;
    e[p] = routed ? min(max(ids[sl], 0), E - 1) : 0;
    act[p] = routed && lane < (I >> 5);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t base = static_cast<int64_t>(e[p]) * H + min(r0 + r, H - 1);
      cw[p][r] = act[p] ? *reinterpret_cast<const uint4*>(q2 + base * rq + 16 * lane) : make_uint4(0, 0, 0, 0);
      sc[p][r] = act[p] ? *reinterpret_cast<const uint16_t*>(s2 + base * rs + 2 * lane) : 0u;
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = wv + KW * p;
    uint32_t xp[16];
    const uint4* hp = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(sl) * I + 32 * lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = act[p] ? hp[q] : make_uint4(0, 0, 0, 0);
      xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = fmaf(e2m1x16_dot(cw[p][r].x, cw[p][r].y, xp), e4m3_to_f32<0>(sc[p][r]), 0.0f);
      acc[r] = fmaf(e2m1x16_dot(cw[p][r].z, cw[p][r].w, xp + 8), e4m3_to_f32<1>(sc[p][r]), acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
      const float wk = sl < S ? wts[sl] * g2[e[p]] : 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) part[sl][r] = wk * acc[r];
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < T * R) {
    const int t = tid / R, r = tid - t * R;
    if (r0 + r < H) {
      const int64_t oi = static_cast<int64_t>(t) * H + r0 + r;
      float o = ys ? ys[oi] : 0.0f;
      for (int k = 0; k < K; ++k) o += part[t * K + k][r];
      out[oi] = f32_to_bf16(o);
    }
  }
}

}  // namespace moe
