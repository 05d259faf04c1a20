// Grouped GEMM for FP8 block-scaled routed experts (E4M3 "fn" bytes [out, in],
// one fp32 scale per 128 x 128 block), the forward_prefill_gemm step of
// "Module glm5next_mlp" with the W8A16 weights of the FP8 checkpoint named on
// the TensorRT-LLM page "Add GLM-5.3-Flash (glm5_next) support".
//
// The structure of k_gemm_nvfp4 (gemm_fp4.hpp) with the FP8 operand:
//   * one workgroup of 8 wavefronts per CU, tile = 128 rows x 256 weight rows
//     (gate/up: 128 gate + the matching 128 up rows; down: 256 output
//     columns); wavefront w owns rows 64 (w & 1) .. +63 and weight rows
//     64 (w >> 1) .. +63 (gate/up: 32 gate + their 32 up rows), 2 x 2
//     v_mfma_f32_32x32x16_bf16 tiles, so every activation fragment read from
//     LDS feeds 2 MFMAs (as in k_gemm_nvfp4) and every weight is converted
//     by the two wavefronts of its column quarter (E4M3 -> bf16 is one
//     instruction per two weights, exact);
//   * activations and codes reach LDS by DMA in whole-line shapes (8 lanes
//     per 128-byte activation row piece, 4 lanes per 64-byte code piece),
//     with the XOR swizzles of k_gemm_nvfp4 applied on the global side; rings
//     of 4 stages of 64 columns (16 KB of activations + 16 KB of codes each,
//     128 KB), three stages in flight, a fixed issue schedule and
//     compile-time waits;
//   * a 128-column k block is two stages and lies in one scale block for
//     every 32-row n-tile, so its MFMAs accumulate into a fresh tile that is
//     then added to the running sum times the block's scale: every weight x
//     activation product is exact and each block sum is scaled once.
// Rows past a tile's end and weight rows past the matrix edge reload row 0
// (outputs dropped).  Requires kdim % 128 == 0 and kdim <= 8192.
#pragma once

#include "common.hpp"
#include "decode_fp8.hpp"
#include "gemm.hpp"
#include "gemm_fp4.hpp"

#include <type_traits>

namespace moe {

constexpr int F8D_WROWS = 256;     // weight rows per workgroup
constexpr int F8D_THREADS = 512;   // 8 wavefronts

struct F8dLds {
  uint4* a[4];
  uint4* c[4];
};

// NV: valid 32-row m-tiles of this wavefront's two (0..2).
template <int MODE, int NV>
__device__ __forceinline__ void f8d_mainloop(const F8dLds& L, const uint8_t* abase, const uint32_t (&ao)[2],
                                             const uint8_t* cbase, const uint32_t (&co)[2], float sreg0,
                                             float sreg1, int wv, int lane, int kdim,
                                             f32x16 (&acc)[2][2]) {
  const int g = lane >> 5, ln = lane & 31;
  const int nkb = kdim >> 6;                   // stages of 64 columns (even)
  const int mh = wv & 1, nq = wv >> 1;

  auto issue = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(abase + (ao[i] + 128u * k)),
                                       (void __attribute__((address_space(3)))*)(L.a[SL] + wv * 128 + i * 64),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(cbase + (co[i] + 64u * k)),
                                       (void __attribute__((address_space(3)))*)(L.c[SL] + wv * 128 + i * 64),
                                       16, 0, 0);
  };

  // consumer offsets: n-tile nt = weight rows p(nt) .. +31 of the workgroup
  int cidx[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int p = (MODE == GEMM_GATEUP ? 128 * nt + 32 * nq : 64 * nq + 32 * nt) + ln;
    const int sc = f4_swz_c(p);
#pragma unroll
    for (int h = 0; h < 2; ++h) cidx[nt][h] = p * 4 + ((2 * g + h) ^ sc);
  }
  const int sa = f4_swz_a(ln);
  int aidx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aidx[s] = ln * 8 + ((4 * g + s) ^ sa);

  f32x16 part[2][2];
  // stage k: wait for its DMA (VM instructions may stay in flight), barrier,
  // issue stage k + 3, then 4 k-steps; an even stage opens a 128-column k
  // block (fresh tiles), an odd one closes it (running sum += scale x tile)
  auto stage = [&](int k, auto slot_c, auto vm_c, bool more) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int VM = decltype(vm_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (more) issue(k + 3, std::integral_constant<int, (SL + 3) & 3>{});
    const uint4* As = L.a[SL];
    const uint4* Cs = L.c[SL];
    uint4 cw[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) cw[nt][h] = Cs[cidx[nt][h]];
    const bool open = (k & 1) == 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint4 c = cw[nt][s >> 1];
        const uint32_t w0 = (s & 1) ? c.z : c.x, w1 = (s & 1) ? c.w : c.y;
        const bf16x2 p0 = e4m3x2_to_bf16<0>(w0), p1 = e4m3x2_to_bf16<1>(w0);
        const bf16x2 p2 = e4m3x2_to_bf16<0>(w1), p3 = e4m3x2_to_bf16<1>(w1);
        bf[nt] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m < NV) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, As[aidx[s] + (2 * mh + m) * 256]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            if (open && s == 0)
              part[m][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[nt], f32x16{}, 0, 0, 0);
            else
              part[m][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[nt], part[m][nt], 0, 0, 0);
          }
        }
      }
    }
    if (!open) {
      // the k block's scales from the lanes that hold them (no memory access
      // here: a load would wait behind the stages already in flight)
      const int kb = k >> 1;
      const float s0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sreg0), kb));
      const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sreg1), kb));
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (m < NV)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            acc[m][0][j] = fmaf(s0, part[m][0][j], acc[m][0][j]);
            acc[m][1][j] = fmaf(s1, part[m][1][j], acc[m][1][j]);
          }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using V0 = std::integral_constant<int, 0>;
  using V4 = std::integral_constant<int, 4>;
  using V8 = std::integral_constant<int, 8>;

  // prologue: stages 0, 1, 2 (4 DMA instructions each per wavefront)
  issue(0, S0{});
  if (nkb > 1) issue(1, S1{});
  if (nkb > 2) issue(2, S2{});
  // steady stages wait with 8 instructions (the next two stages) in flight;
  // stage nkb - 2 with 4, the last with none
  int k = 0;
  for (; k + 4 <= nkb - 2; k += 4) {
    stage(k, S0{}, V8{}, k + 3 < nkb);
    stage(k + 1, S1{}, V8{}, k + 4 < nkb);
    stage(k + 2, S2{}, V8{}, k + 5 < nkb);
    stage(k + 3, S3{}, V8{}, k + 6 < nkb);
  }
  // the last 4 or 2 stages (nkb even), slots continuing from k % 4 == 0
  if (nkb - k == 4) {
    stage(k, S0{}, V8{}, true);
    stage(k + 1, S1{}, V8{}, false);
    stage(k + 2, S2{}, V4{}, false);
    stage(k + 3, S3{}, V0{}, false);
  } else {
    stage(k, S0{}, V4{}, false);
    stage(k + 1, S1{}, V0{}, false);
  }
}

// Grid: 1-D, XCD-aware as in k_gemm_nvfp4.  n_blocks = column blocks of
// F8D_WROWS weight rows (gate/up: 128 gate columns each).
template <int MODE>
__global__ __launch_bounds__(F8D_THREADS, 1) void k_gemm_f8d(GemmArgs a) {
  const int nbn = a.n_blocks;
  const int ntl = *a.n_tiles;
  const int total = ntl * nbn, chunk = (total + 7) >> 3;
  const int kk = blockIdx.x >> 3;
  if (kk >= chunk) return;
  const int w = (blockIdx.x & 7) * chunk + kk;
  if (w >= total) return;
  const int tile = w / nbn, nblk = w - tile * nbn;
  const int e = a.tile_expert[tile];
  const int m0 = a.tile_m0[tile];
  const int valid = min(GM_BM, a.count[e] - m0);
  const int p0 = a.offset[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;

  // activation DMA: instruction i of wave wv covers tile rows 16 wv + 8 i .. +7,
  // 8 lanes per row, lane -> 16-byte chunk (lane & 7) ^ swizzle
  uint32_t ao[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wv + 8 * i + (lane >> 3);
    const int rr = r < valid ? r : 0;
    const int64_t row = (MODE == GEMM_GATEUP) ? a.perm[p0 + rr] / a.K : p0 + rr;
    ao[i] = static_cast<uint32_t>((row * kdim + 8 * ((lane & 7) ^ f4_swz_a(r))) * 2);
  }
  // weight row of workgroup row p (0..255); rows past the edge reload row 0
  auto wrow = [&](int p) -> int64_t {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 128 + (p & 127);
      return j < a.half_n ? (p < 128 ? j : a.half_n + j) : 0;
    } else {
      const int n = nblk * F8D_WROWS + p;
      return n < a.half_n ? n : 0;
    }
  };
  // code DMA: instruction i of wave wv covers workgroup rows 16 (2 wv + i) .. +15,
  // 4 lanes per row, lane -> 16-byte piece q = (lane & 3) ^ swizzle of the
  // row's 64 bytes of the stage
  const uint8_t* cbase = a.bq + e * a.stride_q;
  uint32_t co[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 16 * (2 * wv + i) + (lane >> 2);
    const int q = (lane & 3) ^ f4_swz_c(p);
    co[i] = static_cast<uint32_t>(wrow(p) * kdim + 16 * q);
  }
  // block-scale rows of this wavefront's two n-tiles (one 128-row block each)
  const int nq = wv >> 1, nkb128 = kdim >> 7;
  const float* bsf = a.bsf + e * a.stride_s;
  int64_t sr0, sr1;
  if (MODE == GEMM_GATEUP) {
    sr0 = wrow(32 * nq) >> 7;
    sr1 = wrow(128 + 32 * nq) >> 7;
  } else {
    sr0 = wrow(64 * nq) >> 7;
    sr1 = wrow(64 * nq + 32) >> 7;
  }
  // lane l holds the scales of k block l (kdim <= 8192), loaded before any DMA
  const float sreg0 = bsf[sr0 * nkb128 + min(lane, nkb128 - 1)];
  const float sreg1 = bsf[sr1 * nkb128 + min(lane, nkb128 - 1)];
  // down: this wavefront's output rows (lane l: tile row 64 (wv % 2) + l), read
  // before the main loop (a read per row in the epilogue waits for every store before it)
  int orow_l = 0;
  if constexpr (MODE != GEMM_GATEUP) {
    const int r = 64 * (wv & 1) + lane;
    orow_l = a.perm[p0 + (r < valid ? r : 0)];
  }

  __shared__ uint4 la0[1024], la1[1024], la2[1024], la3[1024];   // activation ring (16 KB each)
  __shared__ uint4 lc0[1024], lc1[1024], lc2[1024], lc3[1024];   // code ring (16 KB each)
  const F8dLds L{{la0, la1, la2, la3}, {lc0, lc1, lc2, lc3}};
  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][nt][j] = 0.0f;
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(a.a);
  // this wavefront's valid m-tiles among 2 mh, 2 mh + 1 (it still moves its
  // share of every stage's DMA and meets every barrier)
  switch (min(2, max(0, ((valid + 31) >> 5) - 2 * (wv & 1)))) {
    case 0: f8d_mainloop<MODE, 0>(L, abase, ao, cbase, co, sreg0, sreg1, wv, lane, kdim, acc); break;
    case 1: f8d_mainloop<MODE, 1>(L, abase, ao, cbase, co, sreg0, sreg1, wv, lane, kdim, acc); break;
    default: f8d_mainloop<MODE, 2>(L, abase, ao, cbase, co, sreg0, sreg1, wv, lane, kdim, acc); break;
  }

  // epilogue: lane holds rows (2 mh + m) * 32 + c32_row(lane, j), column ln of each n-tile
  const int mh = wv & 1, ln = lane & 31;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = (2 * mh + m) * 32 + c32_row(lane, j);
      int orow_i = 0;
      if constexpr (MODE != GEMM_GATEUP) orow_i = __shfl(orow_l, row & 63);
      if (row >= valid) continue;
      if (MODE == GEMM_GATEUP) {
        const int jc = nblk * 128 + 32 * nq + ln;
        if (jc >= a.half_n) continue;
        static_cast<uint16_t*>(a.out)[static_cast<int64_t>(p0 + row) * a.ldo + jc] =
            f32_to_bf16(swiglu_clamped(acc[m][0][j], acc[m][1][j], a.limit));
      } else {
        const int64_t orow = orow_i;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = nblk * F8D_WROWS + 64 * nq + 32 * nt + ln;
          if (n < a.half_n) static_cast<float*>(a.out)[orow * a.ldo + n] = acc[m][nt][j];
        }
      }
    }
  }
}

}  // namespace moe
