// Routed NVFP4 grouped GEMM, gate/up + clamped SwiGLU, for tiles of at most
// 32 rows (decode with up to a few hundred tokens, where an expert holds a
// handful of rows): the products, their order and the outputs of
// k_gemm_nvfp4, with the LDS spent on the weight stream.
//
// A tile of at most 32 rows runs a single 32-row MFMA slice per weight
// fragment, so the kernel is a weight stream: the data in flight per CU sets
// its rate.  k_gemm_nvfp4 spends 64 KB of its rings on 128 activation rows
// and keeps one 32 KB code unit in flight.  Here the activation ring holds 32
// rows (4 stages x 4 KB) and the code ring four units (4 x 32 KB), with unit
// u + 3 issued as unit u starts: three units (96 KB) in flight.  Scales keep
// two groups of four stages (2 x 8 KB).  160 KB of LDS, one workgroup per CU.
//
// Same workgroup shape as k_gemm_nvfp4 (8 wavefronts, 512 weight rows; gate/
// up: 256 gate + the matching 256 up rows), so the DMA layouts, swizzles,
// consumer offsets, k order and dequantisation are k_gemm_nvfp4's, for both
// weight layouts.  The 32 activation rows of a stage are one DMA instruction
// for each of wavefronts 0-3 (8 rows each); wavefronts 4-7 issue none, so
// their wait counts are their own (a template parameter).
//
// Issue schedule (A(k): activation stage k into slot k % 4; C(u): code unit u
// = stages 2u, 2u+1 into slot u % 4; S(v): scale group v = stages 4v..4v+3
// into slot v % 2).  Prologue: S0 C0 A0 C1 A1 C2 A2.  After the barrier of
// stage k: S(k/4 + 1) when k % 4 == 0, C(k/2 + 3) when k is even, A(k + 3);
// each only while it exists.  Every slot written was last read in an earlier
// stage, which every wavefront has left at the barrier.  The wait before
// stage k lets stay in flight exactly the DMA instructions issued after the
// last one stage k needs (A(k), C(k/2), S(k/4)); counted per block of four
// stages, the counts depend on the block's position (first, full, second to
// last, last) and on whether the wavefront issues activations.
//
// Requires kdim % 256 == 0 and kdim >= 512; rows past the tile's valid count
// and weight rows past the matrix edge load row 0 again (outputs dropped).
#pragma once

#include "common.hpp"
#include "gemm.hpp"
#include "gemm_fp4.hpp"

#include <type_traits>

namespace moe {

constexpr int F4M_ROWS = 32;   // activation rows per tile (at most)

struct F4MLds {
  uint4* a[4];
  uint4* c[4];
  uint8_t* s[2];
};

enum F4MBlock { F4M_FULL = 0, F4M_PENULT = 1, F4M_LAST = 2 };

// DMA instructions a wavefront (NA = its activation instructions per stage)
// may leave in flight before stage r of a block
template <int NA, int KIND, bool FIRST, int R>
constexpr int f4m_wait() {
  if (KIND == F4M_LAST) return R == 0 ? 2 * NA : R == 1 ? 2 * NA : R == 2 ? NA : 0;
  if (R == 0) return FIRST ? 8 + 2 * NA : 4 + 2 * NA;
  if (R == 1) return FIRST ? 9 + 2 * NA : 5 + 2 * NA;
  if (R == 2) return 5 + 2 * NA;
  return KIND == F4M_PENULT ? 2 * NA : 4 + 2 * NA;
}

template <int MODE, bool TILED, int NA>
__device__ __forceinline__ void f4m_mainloop(const F4MLds& L, const F4Src& src, int wv, int lane, int kdim,
                                             f32x16 (&acc)[2]) {
  constexpr int NT_ROWS = 256;                 // gate row -> its up row
  const int g = lane >> 5, ln = lane & 31;
  const int nblk4 = kdim >> 8;                 // blocks of four stages, at least 2

  auto issue_a = [&](int k, auto slot_c) {
    if constexpr (NA > 0) {
      constexpr int SL = decltype(slot_c)::value;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.a + (src.ao[0] + 128u * k)),
                                       (void __attribute__((address_space(3)))*)(L.a[SL] + wv * 64), 16, 0, 0);
    }
  };
  constexpr uint32_t C_STEP = TILED ? 1024u : 64u;
  constexpr uint32_t S_STEP = TILED ? 512u : 16u;
  auto issue_c = [&](int u, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.c + (src.co[i] + C_STEP * u)),
                                       (void __attribute__((address_space(3)))*)(L.c[SL] + wv * 256 + i * 64),
                                       16, 0, 0);
  };
  auto issue_s = [&](int v, auto slot_c) {
    constexpr int SSL = decltype(slot_c)::value;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.s + (src.so + S_STEP * v)),
                                     (void __attribute__((address_space(3)))*)(L.s[SSL] + wv * 1024), 16, 0, 0);
  };

  const int prow = 32 * wv + ln;               // this lane's gate row within the workgroup
  const int sc = f4_swz_c(prow), sa = f4_swz_a(ln);
  constexpr int S_STAGE = TILED ? 128 : 4;
  int aidx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aidx[s] = ln * 8 + ((4 * g + s) ^ sa);
  int cidx[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) cidx[t] = prow * 4 + ((2 * t + g) ^ sc);
  const int soff = (TILED ? (prow >> 5) * 512 + 4 * (prow & 31) : prow * 16) >> 2;

  // stage r of a block of parity P (code slots 2P, 2P + 1; scale slot P)
  auto stage = [&](auto r_c, auto p_c, auto vm_c, auto issue) {
    constexpr int R = decltype(r_c)::value;
    constexpr int P = decltype(p_c)::value;
    constexpr int VM = decltype(vm_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint4* As = L.a[R];
    const uint4* Cs = L.c[2 * P + (R >> 1)];
    uint32_t sw[2];
    {
      const uint32_t* Ss = reinterpret_cast<const uint32_t*>(L.s[P]);
      sw[0] = Ss[soff + (S_STAGE >> 2) * R];
      sw[1] = Ss[soff + (S_STAGE >> 2) * R + NT_ROWS * 4];
    }
    uint4 cw[2];
    cw[0] = Cs[cidx[R & 1]];
    cw[1] = Cs[cidx[R & 1] + NT_ROWS * 4];
    const uint32_t s0 = sw[0] >> (16 * g), s1 = sw[1] >> (16 * g);
    bf16x8 af = __builtin_bit_cast(bf16x8, As[aidx[0]]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bfrag[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint4 c = cw[nt];
        const uint32_t word = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
        const uint32_t sb = nt == 0 ? s0 : s1;
        const float scale = (s < 2) ? e4m3_to_f32<0>(sb) : e4m3_to_f32<1>(sb);
        uint32_t o[4];
        e2m1x8_scaled_bf16(word, scale, o);
        bfrag[nt] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfrag[nt], acc[nt], 0, 0, 0);
      if (s < 3) af = __builtin_bit_cast(bf16x8, As[aidx[s + 1]]);
      if (s == 0) issue();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // block j (parity P = j % 2) of kind KIND
  auto block = [&](int j, auto p_c, auto kind_c, auto first_c) {
    constexpr int P = decltype(p_c)::value;
    constexpr int KIND = decltype(kind_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    using SN = std::integral_constant<int, P ^ 1>;            // scale slot of group j + 1
    using C3 = std::integral_constant<int, P ? 1 : 3>;       // code slot of unit 2j + 3
    using C4 = std::integral_constant<int, P ? 2 : 0>;       // code slot of unit 2j + 4
    using W0 = std::integral_constant<int, f4m_wait<NA, KIND, FIRST, 0>()>;
    using W1 = std::integral_constant<int, f4m_wait<NA, KIND, FIRST, 1>()>;
    using W2 = std::integral_constant<int, f4m_wait<NA, KIND, FIRST, 2>()>;
    using W3 = std::integral_constant<int, f4m_wait<NA, KIND, FIRST, 3>()>;
    const int k = 4 * j;
    if constexpr (KIND == F4M_LAST) {
      stage(I0{}, p_c, W0{}, [&] { issue_a(k + 3, I3{}); });
      stage(I1{}, p_c, W1{}, [] {});
      stage(I2{}, p_c, W2{}, [] {});
      stage(I3{}, p_c, W3{}, [] {});
    } else {
      stage(I0{}, p_c, W0{}, [&] { issue_s(j + 1, SN{}); issue_c(2 * j + 3, C3{}); issue_a(k + 3, I3{}); });
      stage(I1{}, p_c, W1{}, [&] { issue_a(k + 4, I0{}); });
      stage(I2{}, p_c, W2{}, [&] {
        if constexpr (KIND == F4M_FULL) issue_c(2 * j + 4, C4{});
        issue_a(k + 5, I1{});
      });
      stage(I3{}, p_c, W3{}, [&] { issue_a(k + 6, I2{}); });
    }
  };
  using KF = std::integral_constant<int, F4M_FULL>;
  using KP = std::integral_constant<int, F4M_PENULT>;
  using KL = std::integral_constant<int, F4M_LAST>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  issue_s(0, I0{});
  issue_c(0, I0{});
  issue_a(0, I0{});
  issue_c(1, I1{});
  issue_a(1, I1{});
  issue_c(2, I2{});
  issue_a(2, I2{});
  if (nblk4 == 2) {
    block(0, P0{}, KP{}, T_{});
    block(1, P1{}, KL{}, F_{});
    return;
  }
  block(0, P0{}, KF{}, T_{});
  // full blocks 1 .. nblk4 - 3 in pairs (parities 1, 0), then the second to
  // last and the last block
  const int jfull = nblk4 - 3;
  for (int j = 1; j + 1 <= jfull; j += 2) {
    block(j, P1{}, KF{}, F_{});
    block(j + 1, P0{}, KF{}, F_{});
  }
  if (nblk4 & 1) {
    block(nblk4 - 2, P1{}, KP{}, F_{});
    block(nblk4 - 1, P0{}, KL{}, F_{});
  } else {
    block(nblk4 - 3, P1{}, KF{}, F_{});
    block(nblk4 - 2, P0{}, KP{}, F_{});
    block(nblk4 - 1, P1{}, KL{}, F_{});
  }
}

// Work mapping as k_gemm_nvfp4 (same n_blocks).  With skip_rows (the
// scheduler lists the tiles of more than skip_rows rows first, for
// k_gemm_nvfp4) it takes the tiles after the first n_tiles[1], each of at
// most 32 rows; without, every tile, in passes of 32 rows that each stream
// the tile's weights again (for few tokens, where a tile of more than 32 rows
// is rare and an extra launch of k_gemm_nvfp4 for it would cost more).  With
// split_pass = S the passes of those first n_tiles[1] tiles go to workgroups
// of their own: the first blocks of the grid take (tile, column block, pass)
// with the pass varying fastest inside each XCD's share, so the S passes over
// the same weight rows run side by side in one L2, and the remaining blocks
// take the tiles of at most 32 rows, each XCD a contiguous share.
template <int MODE, bool TILED>
__global__ __launch_bounds__(F4_THREADS, 1) void k_gemm_nvfp4_m32(GemmArgs a) {
  // gate/up only: the down projection stays on k_gemm_nvfp4 (its short
  // reduction did not pay for this kernel's deeper ring: 3% slower, measured)
  static_assert(MODE == GEMM_GATEUP, "k_gemm_nvfp4_m32 computes the gate/up projection");
  const int nbn = a.n_blocks;
  const int nbig = (a.skip_rows || a.split_pass) ? a.n_tiles[1] : 0;
  const int ntl = a.n_tiles[0] - nbig;
  const int total = ntl * nbn, chunk = (total + 7) >> 3;
  const int S = a.split_pass;
  const int htotal = nbig * nbn * S, hchunk = (htotal + 7) >> 3;   // 0 without split_pass
  int kk = blockIdx.x >> 3;
  int tile, nblk, mp0 = 0, mp1 = GM_BM;
  if (kk < hchunk) {
    const int w = (blockIdx.x & 7) * hchunk + kk;
    if (w >= htotal) return;
    const int q = w / S;
    tile = q / nbn;
    nblk = q - tile * nbn;
    mp0 = F4M_ROWS * (w - q * S);
    mp1 = mp0 + F4M_ROWS;
  } else {
    kk -= hchunk;
    if (kk >= chunk) return;
    const int w = (blockIdx.x & 7) * chunk + kk;
    if (w >= total) return;
    tile = nbig + w / nbn;
    nblk = w - (w / nbn) * nbn;
  }
  const int e = a.tile_expert[tile];
  const int m0 = a.tile_m0[tile];
  const int valid = min(mp1, min(GM_BM, a.count[e] - m0));
  if (mp0 >= valid) return;
  if (a.skip_rows && valid > F4M_ROWS) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;

  F4Src src;
  src.a = reinterpret_cast<const uint8_t*>(a.a);
  src.ao[1] = 0;
  // weight row of workgroup row p (0..511: 256 gate rows, then the matching up rows)
  auto wrow = [&](int p) -> int64_t {
    const int j = nblk * 256 + (p & 255);
    return j < a.half_n ? (p < 256 ? j : a.half_n + j) : 0;
  };
  src.c = (TILED ? a.bq_t : a.bq) + e * a.stride_q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 16 * (4 * wv + i) + (lane >> 2);
    const int q = (lane & 3) ^ f4_swz_c(p);
    const int64_t R = wrow(p);
    src.co[i] = TILED ? static_cast<uint32_t>((R >> 4) * (kdim >> 7) * 1024 +
                                              16 * (4 * (R & 15) + (q ^ f4_swz_c(static_cast<int>(R & 15)))))
                      : static_cast<uint32_t>(R * (kdim >> 1) + 16 * q);
  }
  src.s = (TILED ? a.bs_t : a.bs) + e * a.stride_s;
  if (TILED) {
    const int64_t R0 = wrow(64 * wv + 32 * (lane >> 5));
    src.so = static_cast<uint32_t>((R0 >> 5) * (kdim >> 8) * 512 + 16 * (lane & 31));
  } else {
    src.so = static_cast<uint32_t>(wrow(64 * wv + lane) * (kdim >> 4));
  }
  const float g0 = a.gscale ? a.gscale[2 * e] : 1.0f;
  const float g1 = a.gscale ? a.gscale[2 * e + 1] : 1.0f;

  __shared__ uint4 la0[256], la1[256], la2[256], la3[256];       // activation ring (4 KB each)
  __shared__ uint4 lc0[2048], lc1[2048], lc2[2048], lc3[2048];   // code ring (32 KB each)
  __shared__ __attribute__((aligned(16))) uint8_t ls0[F4_WROWS * 16], ls1[F4_WROWS * 16];   // scale ring
  const F4MLds L{{la0, la1, la2, la3}, {lc0, lc1, lc2, lc3}, {ls0, ls1}};
  const int ln = lane & 31;

  for (int mp = mp0; mp < valid; mp += F4M_ROWS) {
    const int pv = min(F4M_ROWS, valid - mp);   // rows of this pass
    const int p0 = a.offset[e] + m0 + mp;
    // every wavefront has left the previous pass's last stage before its rings refill
    if (mp > mp0) __syncthreads();
    // activation DMA (wavefronts 0-3): pass rows 8 wv .. +7, 8 lanes per row
    {
      const int r = 8 * (wv & 3) + (lane >> 3);
      const int rr = r < pv ? r : 0;
      const int64_t row = a.perm[p0 + rr] / a.K;   // the slot's token
      src.ao[0] = static_cast<uint32_t>((row * kdim + 8 * ((lane & 7) ^ f4_swz_a(r))) * 2);
    }
    f32x16 acc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[nt][j] = 0.0f;
    if (wv < 4)
      f4m_mainloop<MODE, TILED, 1>(L, src, wv, lane, kdim, acc);
    else
      f4m_mainloop<MODE, TILED, 0>(L, src, wv, lane, kdim, acc);

    // lane holds rows c32_row(lane, j) of gate column jc (acc[0]) and up column jc (acc[1])
    const int jc = nblk * 256 + 32 * wv + ln;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = c32_row(lane, j);
      if (row >= pv || jc >= a.half_n) continue;
      static_cast<uint16_t*>(a.out)[static_cast<int64_t>(p0 + row) * a.ldo + jc] =
          f32_to_bf16(swiglu_clamped(g0 * acc[0][j], g1 * acc[1][j], a.limit));
    }
  }
}

}  // namespace moe
