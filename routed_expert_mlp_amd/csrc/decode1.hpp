// One-token decode ("Module glm5next_mlp", modules: forward -- the GLM MLP
// decode forward, one token).  Three launches stream every weight byte once:
//
//   1. k_dec_logits_shared: router logits (fp32 rows of gate.weight) and the
//      BF16 shared expert's gate/up + clamped SwiGLU, both of which only need
//      x, in one grid;
//   2. k_dec_gateup: wavefront 0 of every block redoes the router top-k from
//      the E logits (router.hpp topk_wave; "Traps": bias steers selection
//      only, weights are the renormalised unbiased scores times rsf) and hands
//      the block's expert to the other wavefronts through LDS; the block then
//      streams its NVFP4 gate/up rows + clamped SwiGLU -> h (bf16).  One block
//      also writes ids and weights.  Redoing the selection per block (~2 KB of
//      logits and bias) is cheaper than a launch of its own;
//   3. k_dec_down_combine (k_dec_down_combine1 for one token): for a block of
//      output rows, the shared expert's BF16 down rows (they need nothing
//      from the router, so they stream while the expert ids arrive), the
//      routed NVFP4 down rows of all K experts, and the combine
//      out = bf16(ys + sum_k w_k y_k) (fixed k order) from the block's own
//      partial sums.
//
// Each wavefront issues all loads of its rows before using any of them, so a
// wavefront has its whole share of the weight stream in flight at once.
//
// CT (template flag of the NVFP4 kernels): the routed codes are read from the
// tile layout of moe_nvfp4_tile_pack instead of the row-major array
// (nvfp4_code_off); a lane still reads the same 16-byte chunk of the same
// row, so nothing after the load changes.  The scales stay row-major.
#pragma once

#include "common.hpp"
#include "gemv.hpp"
#include "router.hpp"

namespace moe {

// Lane l of a wavefront covers chunks l, l+64, ..., of a row (one coalesced
// 1 KB load per instruction); a chunk is 16 bytes.

// Layer geometry of the decode kernels: compile-time constants (a kernel
// instance for one layer shape; the selection and index arithmetic fold) or
// 0 = taken from the kernel arguments (IS: -1).
template <int H_, int I_, int E_, int K_, int IS_>
struct DecGeo {
  static constexpr int H = H_, I = I_, E = E_, K = K_, IS = IS_;
};
using DecGeoAny = DecGeo<0, 0, 0, 0, -1>;


// -------------------------------------------------------------------------
// 1. logits + shared gate/up.  Blocks [0, n_logit_blocks) take 4 router rows
// each (one per wavefront), the rest take 4 shared (gate, up) row pairs.
//   NR: float4 chunks per lane of a router row (>= H / 256)
//   NS: 8-bf16 chunks per lane of a shared row (>= H / 512)
// -------------------------------------------------------------------------
// keys (may be null): also the top-k sort key of each expert (router.hpp
// topk_key of its logit and correction bias), so that the routed gate/up
// launch starts its selection from the keys.
template <int NR, int NS, class G>
__global__ __launch_bounds__(256) void k_dec_logits_shared(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr, float* __restrict__ logits,
                                                           int E_, int H_, const uint16_t* __restrict__ sw13, int Is_,
                                                           uint16_t* __restrict__ hs, float L, int n_logit_blocks,
                                                           const float* __restrict__ bias = nullptr,
                                                           uint64_t* __restrict__ keys = nullptr) {
  const int E = G::E ? G::E : E_, H = G::H ? G::H : H_;
  const int Is = G::IS >= 0 ? G::IS : Is_;
  // with the geometry compiled in and rows of exactly 64 NR float4 / 64 NS
  // 8-bf16 chunks, no load needs a lane guard
  constexpr bool EXACT_R = G::H == 256 * NR, EXACT_S = G::H == 512 * NS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (static_cast<int>(blockIdx.x) < n_logit_blocks) {
    const int e = blockIdx.x * 4 + wv;
    if (e >= E) return;
    const float4* row = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H);
    const uint2* xv = reinterpret_cast<const uint2*>(x);
    const float be = keys ? bias[e] : 0.0f;
    float4 w[NR];
    uint2 xs[NR];
    const int nch = H >> 2;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = lane + 64 * i;
      w[i] = (EXACT_R || c < nch) ? row[c] : make_float4(0, 0, 0, 0);
      xs[i] = (EXACT_R || c < nch) ? xv[c] : make_uint2(0, 0);
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
    if (lane == 0) {
      logits[e] = acc;
      if (keys) keys[e] = topk_key(acc, be, e);
    }
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
      const bool ok = EXACT_S || c < nch;
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
// 1'. The same grid for T <= 16 tokens (general decode), with the tokens in
// groups of DEC_TG over grid.y: each wavefront loads its router row (or
// shared gate/up row pair) once, then runs the dot products of its group's
// tokens against it; x rows are re-read per token (they stay in the caches).
// With gridDim.x a multiple of 8 every group of a row block runs on the same
// XCD (blocks go to the XCDs round-robin), so the groups after the first read
// the rows from that XCD's L2.  Per token the arithmetic and reduction order
// are those of k_dec_logits_shared.  Writes logits [T][E] and hs [T][Is].
// -------------------------------------------------------------------------
constexpr int DEC_TG = 4;
constexpr int DEC_MAX_H = 4096;   // the decode kernels' largest hidden size

template <int NR, int NS>
__global__ __launch_bounds__(256) void k_dec_logits_shared_t(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             float* __restrict__ logits, int E, int H,
                                                             const uint16_t* __restrict__ sw13, int Is,
                                                             uint16_t* __restrict__ hs, float L, int n_logit_blocks,
                                                             int T, const float* __restrict__ bias = nullptr,
                                                             uint64_t* __restrict__ keys = nullptr) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ta = blockIdx.y * DEC_TG, tb = min(T, ta + DEC_TG);
  // the group's x rows, staged once per block in LDS (after the weight loads
  // are issued): each wavefront then reads them at LDS latency, token after token
  __shared__ uint4 xl[DEC_TG * (DEC_MAX_H / 8)];
  const int nx = H >> 3;
  auto stage_x = [&] {
    const uint4* xg = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(ta) * H);
    for (int q = threadIdx.x; q < (tb - ta) * nx; q += 256) xl[q] = xg[q];
    __syncthreads();
  };
  if (static_cast<int>(blockIdx.x) < n_logit_blocks) {
    const int e = blockIdx.x * 4 + wv;
    const float4* row = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(min(e, E - 1)) * H);
    const float be = keys ? bias[min(e, E - 1)] : 0.0f;
    float4 w[NR];
    const int nch = H >> 2;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = lane + 64 * i;
      w[i] = c < nch ? row[c] : make_float4(0, 0, 0, 0);
    }
    stage_x();
    if (e >= E) return;
    for (int t = ta; t < tb; ++t) {
      const uint2* xv = reinterpret_cast<const uint2*>(xl + (t - ta) * nx);
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
      if (lane == 0) {
        logits[static_cast<int64_t>(t) * E + e] = acc;
        if (keys) keys[static_cast<int64_t>(t) * E + e] = topk_key(acc, be, e);
      }
    }
  } else {
    const int j = (blockIdx.x - n_logit_blocks) * 4 + wv;
    const int jj = min(j, max(Is - 1, 0));
    const uint4* g = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(jj) * H);
    const uint4* u = reinterpret_cast<const uint4*>(sw13 + static_cast<int64_t>(Is + jj) * H);
    const int nch = H >> 3;
    uint4 wg[NS], wu[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < nch && Is > 0;
      wg[i] = ok ? g[c] : make_uint4(0, 0, 0, 0);
      wu[i] = ok ? u[c] : make_uint4(0, 0, 0, 0);
    }
    stage_x();
    if (j >= Is) return;
    for (int t = ta; t < tb; ++t) {
      const uint4* xv = xl + (t - ta) * nx;
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
// 2. top-k + routed gate/up for T tokens (T*K slots, slot = t*K + k).  1-D
// grid; block a serves slot a / njb, njb = ceil(I / (4 RJ)): its wavefront 0
// finds the slot's expert (topk_wave, NJ >= E / 64) and hands it to the
// other wavefronts through LDS (one selection per block: a selection costs
// a few hundred instructions, too many to repeat in every wavefront), and
// wavefront w runs gate rows j = ((a % njb)*4 + w)*RJ .. +RJ and up rows
// I + j.  Lane l covers the 16-byte chunks l, l+64, ... (NC of them; EXACT:
// every lane has all NC, i.e. H == 2048 NC) of each row, so every load
// instruction reads 1 KB contiguous.
// Wavefront 0 of the first block of each token's slot 0 runs all K rounds
// and writes ids/wts (and ids_out / w_out when not null).
// -------------------------------------------------------------------------
template <int RJ, int NC, bool EXACT, int NJ, class G, bool CT = false>
__global__ __launch_bounds__(256) void k_dec_gateup(const uint16_t* __restrict__ x, const uint8_t* __restrict__ q13,
                                                    const uint8_t* __restrict__ s13, const float* __restrict__ g13,
                                                    const float* __restrict__ logits, const float* __restrict__ bias,
                                                    int K_, float rsf, int32_t* __restrict__ ids,
                                                    float* __restrict__ wts, int32_t* ids_out, float* w_out, int E_,
                                                    int H_, int I_, float L, uint16_t* __restrict__ h,
                                                    const uint64_t* __restrict__ keys = nullptr) {
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  __shared__ int s_sel;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int a = blockIdx.x;
  const int njb = static_cast<int>(cdiv(I, 4 * RJ));
  const int slot = a / njb;                          // t * K + k
  const int t = slot / K, k = slot - t * K;
  const int jb = a - slot * njb;
  const int j0 = (jb * 4 + wv) * RJ;
  const int nch = H >> 5;
  x += static_cast<int64_t>(t) * H;
  if (wv == 0) {
    const bool writer = jb == 0 && k == 0;
    const int64_t o = static_cast<int64_t>(t) * K;
    // from the launch-1 sort keys when given (the same keys, built by the same expression)
    const int sel = keys ? topk_wave_keys<NJ>(keys + static_cast<int64_t>(t) * E, logits + static_cast<int64_t>(t) * E,
                                              E, K, rsf, k, writer ? ids + o : nullptr, wts + o,
                                              ids_out ? ids_out + o : nullptr, w_out ? w_out + o : nullptr)
                         : topk_wave<NJ>(logits + static_cast<int64_t>(t) * E, bias, E, K, rsf, k,
                                         writer ? ids + o : nullptr, wts + o, ids_out ? ids_out + o : nullptr,
                                         w_out ? w_out + o : nullptr);
    if (lane == 0) s_sel = sel;
  }
  __syncthreads();
  if (j0 >= I) return;
  const int e = min(max(s_sel, 0), E - 1);
  const int64_t rq = H >> 1, rs = H >> 4;                 // code / scale bytes per row
  const uint8_t* qe = q13 + static_cast<int64_t>(e) * 2 * I * rq;
  const uint8_t* se = s13 + static_cast<int64_t>(e) * 2 * I * rs;
  uint4 cg[RJ][NC], cu[RJ][NC];
  uint32_t sg[RJ][NC], su[RJ][NC];
#pragma unroll
  for (int r = 0; r < RJ; ++r) {
    const int j = min(j0 + r, I - 1);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = EXACT || c < nch;
      cg[r][i] = ok ? *reinterpret_cast<const uint4*>(qe + nvfp4_code_off<CT>(j, c, H)) : make_uint4(0, 0, 0, 0);
      cu[r][i] = ok ? *reinterpret_cast<const uint4*>(qe + nvfp4_code_off<CT>(I + j, c, H)) : make_uint4(0, 0, 0, 0);
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
      const uint4 v = (EXACT || c < nch) ? xv[q] : make_uint4(0, 0, 0, 0);
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
// 3. shared down + routed down + combine for T <= 4 tokens (T*K slots, slot
// = t*K + k).  Block b owns output rows r0 = b*R .. +R and NW >= R
// wavefronts.  Every wavefront first asks for the ids and weights of its
// slots s = w + NW p (p < NP), then (w < R) its shared down row r0 + w
// (BF16, lane l its 16-byte chunks l, l+64, ..., NSC of them) and the first
// token's hs chunks, and the h_s chunks of its slots -- none of which depend
// on the ids, so they stream while the ids arrive -- and finally the R rows
// of each slot's NVFP4 down projection (lane l its 16-byte chunk l, lanes <
// I/32).  ys[t][r] = W2s[r] . hs[t] and the per-(slot, row) products
// (w_s g2) acc_s meet in LDS, and thread (t, r) writes
// out[t][r0+r] = bf16(ys + sum_k (w_{tK+k} g2) acc_{tK+k}), k in order
// (ys = 0 without a shared expert).
// -------------------------------------------------------------------------
constexpr int DEC_MAX_T = 4;

template <int R, int NW, int NP, int NSC, class G, bool CT = false>
__global__ __launch_bounds__(NW * 64) void k_dec_down_combine(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ q2, const uint8_t* __restrict__ s2,
    const float* __restrict__ g2, const uint16_t* __restrict__ sw2, const uint16_t* __restrict__ hs, int Is_,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int E_, int K_, int H_, int I_,
    uint16_t* __restrict__ out, int T) {
  static_assert(R <= NW, "one wavefront per shared down row");
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  const int Is = G::IS >= 0 ? G::IS : Is_;
  __shared__ float part[NW * NP][R];
  __shared__ float ysp[DEC_MAX_T][R];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r0 = blockIdx.x * R;
  const int S = T * K;
  // Every load is issued unconditionally from an in-bounds address (lanes and
  // slots past the end re-read a valid element and are zeroed afterwards), so
  // no load sits behind a branch and the waits before the arithmetic can be
  // exact.
  const int nd = I >> 5;                               // routed down chunks per row
  const bool dlane = lane < nd;
  const int dl = dlane ? lane : nd - 1;
  // 1. ids and weights of this wavefront's slots
  int idv[NP];
  float wsl[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = min(wv + NW * p, S - 1);
    idv[p] = ids[sl];
    wsl[p] = wts[sl];
  }
  // 2. loads that do not depend on the ids: the shared down row, hs of token 0, h of each slot
  const bool shared_row = Is > 0 && wv < R;
  const int nsc = Is >> 3;                               // 8-bf16 chunks per shared row
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
  uint32_t xp[NP][16];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int sl = min(wv + NW * p, S - 1);
    const uint4* hp = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(sl) * I + 32 * dl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = hp[q];
      xp[p][4 * q] = v.x; xp[p][4 * q + 1] = v.y; xp[p][4 * q + 2] = v.z; xp[p][4 * q + 3] = v.w;
    }
  }
  // 3. the routed down rows of this wavefront's slots
  const int64_t rq = I >> 1, rs = I >> 4;
  int e[NP];
  uint4 cw[NP][R];
  uint32_t sc[NP][R];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    e[p] = min(max(idv[p], 0), E - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t base = static_cast<int64_t>(e[p]) * H + min(r0 + r, H - 1);
      cw[p][r] = *reinterpret_cast<const uint4*>(q2 + static_cast<int64_t>(e[p]) * H * rq +
                                                 nvfp4_code_off<CT>(min(r0 + r, H - 1), dl, I));
      sc[p][r] = *reinterpret_cast<const uint16_t*>(s2 + base * rs + 2 * dl);
    }
  }
  float gk[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) gk[p] = g2[e[p]];
  __builtin_amdgcn_sched_barrier(0);
  if (shared_row) {
#pragma unroll
    for (int i = 0; i < NSC; ++i)
      if (lane + 64 * i >= nsc) sw[i] = make_uint4(0, 0, 0, 0);
  }
  bool act[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    act[p] = wv + NW * p < S && dlane;
    if (!act[p]) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cw[p][r] = make_uint4(0, 0, 0, 0);
        sc[p][r] = 0u;
      }
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
      acc[r] = fmaf(e2m1x16_dot(cw[p][r].x, cw[p][r].y, xp[p]), e4m3_to_f32<0>(sc[p][r]), 0.0f);
      acc[r] = fmaf(e2m1x16_dot(cw[p][r].z, cw[p][r].w, xp[p] + 8), e4m3_to_f32<1>(sc[p][r]), acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0 && sl < S) {
      const float wk = wsl[p] * gk[p];
#pragma unroll
      for (int r = 0; r < R; ++r) part[sl][r] = wk * acc[r];
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
// 3'. The same layer output for one token with R output rows per block and
// the work split by kind: wavefronts 0..K-1 each take one routed slot's R
// down rows (lane l: the 16-byte chunk l of every row, as above), wavefronts
// K..K+NSW-1 each take R/NSW shared down rows.  Each wavefront reads its
// input vector (h_k, or hs) once for all of its rows, so the vectors cost a
// quarter of the cache traffic of 4-row blocks.  Per (slot, row) and per
// shared row the products, their order and the combine order are those of
// k_dec_down_combine, so the two kernels agree bit for bit.
//   requires K + NSW <= 16, I <= 2048 (one chunk per lane and row)
// -------------------------------------------------------------------------
template <int R, int NSW, int NSC, class G, bool CT = false>
__global__ __launch_bounds__(1024) void k_dec_down_combine1(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ q2, const uint8_t* __restrict__ s2,
    const float* __restrict__ g2, const uint16_t* __restrict__ sw2, const uint16_t* __restrict__ hs, int Is_,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int E_, int K_, int H_, int I_,
    uint16_t* __restrict__ out) {
  static_assert(R % NSW == 0, "whole shared rows per wavefront");
  constexpr int SR = R / NSW;
  const int K = G::K ? G::K : K_, E = G::E ? G::E : E_, H = G::H ? G::H : H_, I = G::I ? G::I : I_;
  const int Is = G::IS >= 0 ? G::IS : Is_;
  __shared__ float part[16][R];
  __shared__ float ysp[R];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  {
    // grid.y = token (decode of a few tokens): token t's K slots, its shared
    // vector and its output row
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
    const int nd = I >> 5;
    const bool dlane = lane < nd;
    const int dl = dlane ? lane : nd - 1;
    const int idv = ids[wv];
    const float wsl = wts[wv];
    uint32_t xp[16];
    const uint4* hp = reinterpret_cast<const uint4*>(h + static_cast<int64_t>(wv) * I + 32 * dl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = hp[q];
      xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
    const int64_t rq = I >> 1, rs = I >> 4;
    const int e = min(max(idv, 0), E - 1);
    uint4 cw[R];
    uint32_t sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t base = static_cast<int64_t>(e) * H + min(r0 + r, H - 1);
      cw[r] = *reinterpret_cast<const uint4*>(q2 + static_cast<int64_t>(e) * H * rq +
                                              nvfp4_code_off<CT>(min(r0 + r, H - 1), dl, I));
      sc[r] = *reinterpret_cast<const uint16_t*>(s2 + base * rs + 2 * dl);
    }
    const float gk = g2[e];
    __builtin_amdgcn_sched_barrier(0);
    if (!dlane) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cw[r] = make_uint4(0, 0, 0, 0);
        sc[r] = 0u;
      }
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = fmaf(e2m1x16_dot(cw[r].x, cw[r].y, xp), e4m3_to_f32<0>(sc[r]), 0.0f);
      acc[r] = fmaf(e2m1x16_dot(cw[r].z, cw[r].w, xp + 8), e4m3_to_f32<1>(sc[r]), acc[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
      const float wk = wsl * gk;
#pragma unroll
      for (int r = 0; r < R; ++r) part[wv][r] = wk * acc[r];
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
