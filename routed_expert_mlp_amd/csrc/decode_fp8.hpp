// One-token decode of a layer whose routed experts are FP8 block-scaled
// (E4M3 "fn" bytes [out, in] row-major, one fp32 scale per 128 x 128 block,
// multiplied: the FP8 checkpoint named on the TensorRT-LLM page "Add
// GLM-5.3-Flash (glm5_next) support"; activations stay bf16, W8A16).  The
// launches are those of decode1.hpp: launch 1 (router logits + BF16 shared
// gate/up) is shared; launches 2 and 3 here stream FP8 rows instead of NVFP4
// ones.
//
// A lane reads 16-byte chunks (16 weights) of a row, so every load
// instruction is 1 KB contiguous; a chunk lies inside one 128-column scale
// block, so its 16 products (E4M3 x bf16, exact in fp32) are summed first
// and then multiplied by the block's scale.
#pragma once

#include "common.hpp"
#include "decode1.hpp"
#include "router.hpp"

namespace moe {

constexpr int F8_BLOCK = 128;

// Bytes 2W and 2W+1 of a word (two E4M3 values, lower byte = lower element)
// -> bf16 pair; exact (E4M3 values fit bf16).
template <int W>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, W == 1);
}

// One 16-byte chunk of E4M3 weights times 16 bf16 activations (8 packed
// pairs), accumulated in fp32 from 0.
__device__ __forceinline__ float e4m3x16_dot(uint4 c, const uint32_t* xp) {
  float s = 0.0f;
  s = dot2_bf16(e4m3x2_to_bf16<0>(c.x), xp[0], s);
  s = dot2_bf16(e4m3x2_to_bf16<1>(c.x), xp[1], s);
  s = dot2_bf16(e4m3x2_to_bf16<0>(c.y), xp[2], s);
  s = dot2_bf16(e4m3x2_to_bf16<1>(c.y), xp[3], s);
  s = dot2_bf16(e4m3x2_to_bf16<0>(c.z), xp[4], s);
  s = dot2_bf16(e4m3x2_to_bf16<1>(c.z), xp[5], s);
  s = dot2_bf16(e4m3x2_to_bf16<0>(c.w), xp[6], s);
  return dot2_bf16(e4m3x2_to_bf16<1>(c.w), xp[7], s);
}

// -------------------------------------------------------------------------
// 2 (FP8). top-k + routed gate/up for T tokens (slot = t*K + k), the grid
// and selection of k_dec_gateup: block a serves slot a / njb, njb =
// ceil(I / (4 RJ)); wavefront 0 selects the expert and hands it over through
// LDS; wavefront w runs gate rows j = ((a % njb)*4 + w)*RJ .. +RJ and up rows
// I + j (RJ divides 128, so they share one row block of scales).  Lane l
// covers chunks l, l+64, ... (NC of them; EXACT: H == 1024 NC).
//   s13: [E][2I/128][H/128] fp32 block scales.
// -------------------------------------------------------------------------
template <int RJ, int NC, bool EXACT, int NJ, class G>
__global__ __launch_bounds__(256) void k_dec_gateup_f8(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q13,
                                                       const float* __restrict__ s13, const float* __restrict__ logits,
                                                       const float* __restrict__ bias, int K_, float rsf,
                                                       int32_t* __restrict__ ids, float* __restrict__ wts,
                                                       int32_t* ids_out, float* w_out, int E_, int H_, int I_, float L,
                                                       uint16_t* __restrict__ h) {
  static_assert(F8_BLOCK % RJ == 0, "a wavefront's rows share one scale row block");
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  __shared__ int s_sel;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int a = blockIdx.x;
  const int njb = static_cast<int>(cdiv(I, 4 * RJ));
  const int slot = a / njb;
  const int t = slot / K, k = slot - t * K;
  const int jb = a - slot * njb;
  const int j0 = (jb * 4 + wv) * RJ;
  const int nch = H >> 4;                                   // 16-byte chunks per row
  x += static_cast<int64_t>(t) * H;
  if (wv == 0) {
    const bool writer = jb == 0 && k == 0;
    const int64_t o = static_cast<int64_t>(t) * K;
    const int sel = topk_wave<NJ>(logits + static_cast<int64_t>(t) * E, bias, E, K, rsf, k,
                                  writer ? ids + o : nullptr, wts + o, ids_out ? ids_out + o : nullptr,
                                  w_out ? w_out + o : nullptr);
    if (lane == 0) s_sel = sel;
  }
  __syncthreads();
  if (j0 >= I) return;
  const int e = min(max(s_sel, 0), E - 1);
  const int nsb = H / F8_BLOCK;                              // scale blocks per row
  const uint8_t* qe = q13 + static_cast<int64_t>(e) * 2 * I * H;
  const float* se = s13 + static_cast<int64_t>(e) * (2 * I / F8_BLOCK) * nsb;
  const float* sgr = se + (j0 / F8_BLOCK) * nsb;
  const float* sur = se + ((I + j0) / F8_BLOCK) * nsb;
  uint4 cg[RJ][NC], cu[RJ][NC];
  float sg[NC], su[NC];
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    const int j = min(j0 + r, I - 1);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = EXACT ? lane + 64 * i : min(lane + 64 * i, nch - 1);
      cg[r][i] = *reinterpret_cast<const uint4*>(qe + static_cast<int64_t>(j) * H + 16 * c);
      cu[r][i] = *reinterpret_cast<const uint4*>(qe + static_cast<int64_t>(I + j) * H + 16 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = EXACT ? lane + 64 * i : min(lane + 64 * i, nch - 1);
    sg[i] = sgr[c >> 3];
    su[i] = sur[c >> 3];
  }
  float ag[RJ], au[RJ];
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    ag[r] = 0.0f;
    au[r] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = EXACT ? lane + 64 * i : min(lane + 64 * i, nch - 1);
    const bool ok = EXACT || lane + 64 * i < nch;
    uint32_t xp[8];
    const uint4* xv = reinterpret_cast<const uint4*>(x + 16 * c);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 v = xv[q];
      xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < RJ; ++r) {
      const uint4 g = ok ? cg[r][i] : make_uint4(0, 0, 0, 0), u = ok ? cu[r][i] : make_uint4(0, 0, 0, 0);
      ag[r] = fmaf(e4m3x16_dot(g, xp), sg[i], ag[r]);
      au[r] = fmaf(e4m3x16_dot(u, xp), su[i], au[r]);
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
    if (j < I) h[static_cast<int64_t>(slot) * I + j] = f32_to_bf16(swiglu_clamped(gg, uu, L));
  }
}

// -------------------------------------------------------------------------
// 3 (FP8). shared down + routed down + combine for T <= 4 tokens, the
// structure of k_dec_down_combine: block b owns output rows r0 = b*R .. +R
// (R divides 128: one scale row block) and NW >= R wavefronts; each asks for
// its slots' ids and weights first, then loads its shared down row (w < R),
// the first token's hs chunks and its slots' h chunks, then the R rows of
// each slot's FP8 down projection (lane l its chunks l, l+64, ..., ND of them,
// below I/16) and their block scales.
//   s2: [E][H/128][I/128] fp32 block scales.
// -------------------------------------------------------------------------
template <int R, int NW, int NP, int NSC, int ND, class G>
__global__ __launch_bounds__(NW * 64) void k_dec_down_combine_f8(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ q2, const float* __restrict__ s2,
    const uint16_t* __restrict__ sw2, const uint16_t* __restrict__ hs, int Is_, const int32_t* __restrict__ ids,
    const float* __restrict__ wts, int E_, int K_, int H_, int I_, uint16_t* __restrict__ out, int T) {
  static_assert(R <= NW, "one wavefront per shared down row");
  static_assert(F8_BLOCK % R == 0, "a block's rows share one scale row block");
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  const int Is = G::IS >= 0 ? G::IS : Is_;
  __shared__ float part[NW * NP][R];
  __shared__ float ysp[DEC_MAX_T][R];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r0 = blockIdx.x * R;
  const int S = T * K;
  const int nd = I >> 4;                                // 16-byte chunks per routed down row
  const int nsb = I / F8_BLOCK;                         // scale blocks per routed down row
  // 1. ids and weights of this wavefront's slots
  int idv[NP];
  float wsl[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = min(wv + NW * p, S - 1);
    idv[p] = ids[sl];
    wsl[p] = wts[sl];
  }
  // 2. loads that do not depend on the ids
  const bool shared_row = Is > 0 && wv < R;
  const int nsc = Is >> 3;
  uint4 sw[NSC];
  uint32_t hs0[NSC][4];
  if (shared_row) {
    const uint4* row = reinterpret_cast<const uint4*>(sw2 + static_cast<int64_t>(min(r0 + wv, H - 1)) * Is);
#pragma unroll
    for (int i = 0; i < NSC; ++i) sw[i] = row[min(lane + 64 * i, nsc - 1)];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(hs)[min(lane + 64 * i, nsc - 1)];
      hs0[i][0] = v.x; hs0[i][1] = v.y; hs0[i][2] = v.z; hs0[i][3] = v.w;
    }
  }
  uint32_t xp[NP][ND][8];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = min(wv + NW * p, S - 1);
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int c = min(lane + 64 * i, nd - 1);
      const uint4* hp = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(sl) * I + 16 * c);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = hp[q];
        xp[p][i][4 * q] = v.x; xp[p][i][4 * q + 1] = v.y; xp[p][i][4 * q + 2] = v.z; xp[p][i][4 * q + 3] = v.w;
      }
    }
  }
  // 3. the routed down rows and block scales of this wavefront's slots
  uint4 cw[NP][R][ND];
  float sc[NP][ND];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e = min(max(idv[p], 0), E - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = static_cast<int64_t>(e) * H + min(r0 + r, H - 1);
#pragma unroll
      for (int i = 0; i < ND; ++i)
        cw[p][r][i] = *reinterpret_cast<const uint4*>(q2 + row * I + 16 * min(lane + 64 * i, nd - 1));
    }
    const float* srow = s2 + (static_cast<int64_t>(e) * (H / F8_BLOCK) + min(r0, H - 1) / F8_BLOCK) * nsb;
#pragma unroll
    for (int i = 0; i < ND; ++i) sc[p][i] = srow[min(lane + 64 * i, nd - 1) >> 3];
  }
  __builtin_amdgcn_sched_barrier(0);
  if (shared_row) {
#pragma unroll
    for (int i = 0; i < NSC; ++i)
      if (lane + 64 * i >= nsc) sw[i] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const bool live = wv + NW * p < S;
#pragma unroll
    for (int i = 0; i < ND; ++i)
      if (!live || lane + 64 * i >= nd) {
        sc[p][i] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) cw[p][r][i] = make_uint4(0, 0, 0, 0);
      }
  }
  if (shared_row) {
    for (int t = 0; t < T; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < NSC; ++i) {
        uint32_t hv[4] = {hs0[i][0], hs0[i][1], hs0[i][2], hs0[i][3]};
        if (t > 0) {
          const int c = lane + 64 * i;
          const uint4 v = c < nsc ? reinterpret_cast<const uint4*>(hs + static_cast<int64_t>(t) * Is)[c]
                                  : make_uint4(0, 0, 0, 0);
          hv[0] = v.x; hv[1] = v.y; hv[2] = v.z; hv[3] = v.w;
        }
        acc = bf16_chunk_dot(sw[i], hv, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) ysp[t][wv] = acc;
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = wv + NW * p;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < ND; ++i) acc[r] = fmaf(e4m3x16_dot(cw[p][r][i], xp[p][i]), sc[p][i], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0 && sl < S) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[sl][r] = wsl[p] * acc[r];
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < T * R) {
    const int t = tid / R, r = tid - t * R;
    if (r0 + r < H) {
      float o = Is > 0 ? ysp[t][r] : 0.0f;
      for (int k = 0; k < K; ++k) o += part[t * K + k][r];
      out[static_cast<int64_t>(t) * H + r0 + r] = f32_to_bf16(o);
    }
  }
}

// -------------------------------------------------------------------------
// 3' (FP8). The same step with R output rows per block and a grid row per
// token (blockIdx.y = t: token t's K slots, shared vector and output row),
// in the layout of k_dec_down_combine1: wavefront k < K takes slot t*K + k
// (its R FP8 down rows, lane l its chunks l, l+64, ..., ND of them, and the
// slot's h chunks, read once for all R rows), wavefronts K..K+NSW-1 take R/NSW
// shared down rows each.  Per (slot, row) and per shared row the products
// and their orders, and the combine order, are those of
// k_dec_down_combine_f8, so the two kernels agree bit for bit.
//   requires K + NSW <= 16; R divides 128 (the block's rows share one scale
//   row block); I <= 1024 ND
// -------------------------------------------------------------------------
template <int R, int NSW, int NSC, int ND, class G>
__global__ __launch_bounds__(1024) void k_dec_down_combine1_f8(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ q2, const float* __restrict__ s2,
    const uint16_t* __restrict__ sw2, const uint16_t* __restrict__ hs, int Is_, const int32_t* __restrict__ ids,
    const float* __restrict__ wts, int E_, int K_, int H_, int I_, uint16_t* __restrict__ out) {
  static_assert(R % NSW == 0, "whole shared rows per wavefront");
  static_assert(F8_BLOCK % R == 0, "a block's rows share one scale row block");
  constexpr int SR = R / NSW;
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  const int Is = G::IS >= 0 ? G::IS : Is_;
  __shared__ float part[16][R];
  __shared__ float ysp[R];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  {
    const int t = blockIdx.y;
    ids += t * K;
    wts += t * K;
    h += static_cast<int64_t>(t) * K * I;
    hs += static_cast<int64_t>(t) * Is;
    out += static_cast<int64_t>(t) * H;
  }
  const int r0 = blockIdx.x * R;
  if (wv < K) {
    // routed slot wv: ids first; then h_k (independent of the ids); then the R down rows
    const int nd = I >> 4;                      // 16-byte chunks per routed down row
    const int nsb = I / F8_BLOCK;
    const int idv = ids[wv];
    const float wsl = wts[wv];
    uint32_t xp[ND][8];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int c = min(lane + 64 * i, nd - 1);
      const uint4* hp = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(wv) * I + 16 * c);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = hp[q];
        xp[i][4 * q] = v.x; xp[i][4 * q + 1] = v.y; xp[i][4 * q + 2] = v.z; xp[i][4 * q + 3] = v.w;
      }
    }
    const int e = min(max(idv, 0), E - 1);
    uint4 cw[R][ND];
    float sc[ND];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = static_cast<int64_t>(e) * H + min(r0 + r, H - 1);
#pragma unroll
      for (int i = 0; i < ND; ++i)
        cw[r][i] = *reinterpret_cast<const uint4*>(q2 + row * I + 16 * min(lane + 64 * i, nd - 1));
    }
    const float* srow = s2 + (static_cast<int64_t>(e) * (H / F8_BLOCK) + min(r0, H - 1) / F8_BLOCK) * nsb;
#pragma unroll
    for (int i = 0; i < ND; ++i) sc[i] = srow[min(lane + 64 * i, nd - 1) >> 3];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < ND; ++i)
      if (lane + 64 * i >= nd) {
        sc[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) cw[r][i] = make_uint4(0, 0, 0, 0);
      }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < ND; ++i) acc[r] = fmaf(e4m3x16_dot(cw[r][i], xp[i]), sc[i], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[wv][r] = wsl * acc[r];
    }
  } else if (wv < K + NSW && Is > 0) {
    // shared rows r0 + sr0 .. + SR - 1 against hs
    const int sr0 = (wv - K) * SR;
    const int nsc = Is >> 3;
    uint4 sw[SR][NSC];
    uint32_t hv[NSC][4];
#pragma unroll
    for (int i = 0; i < SR; ++i) {
      const uint4* row = reinterpret_cast<const uint4*>(sw2 + static_cast<int64_t>(min(r0 + sr0 + i, H - 1)) * Is);
#pragma unroll
      for (int c = 0; c < NSC; ++c) sw[i][c] = row[min(lane + 64 * c, nsc - 1)];
    }
#pragma unroll
    for (int c = 0; c < NSC; ++c) {
      const uint4 v = reinterpret_cast<const uint4*>(hs)[min(lane + 64 * c, nsc - 1)];
      hv[c][0] = v.x; hv[c][1] = v.y; hv[c][2] = v.z; hv[c][3] = v.w;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NSC; ++c)
      if (lane + 64 * c >= nsc) {
#pragma unroll
        for (int i = 0; i < SR; ++i) sw[i][c] = make_uint4(0, 0, 0, 0);
      }
    float acc[SR];
#pragma unroll
    for (int i = 0; i < SR; ++i) {
      acc[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < NSC; ++c) acc[i] = bf16_chunk_dot(sw[i][c], hv[c], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < SR; ++i) acc[i] = wave_sum(acc[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < SR; ++i) ysp[sr0 + i] = acc[i];
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < R && r0 + tid < H) {
    float o = Is > 0 ? ysp[tid] : 0.0f;
    for (int k = 0; k < K; ++k) o += part[k][tid];
    out[r0 + tid] = f32_to_bf16(o);
  }
}

}  // namespace moe
