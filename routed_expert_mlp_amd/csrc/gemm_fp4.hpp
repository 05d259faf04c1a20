// Routed NVFP4 grouped GEMM for prefill (gate/up with the clamped SwiGLU, and
// down), v_mfma_f32_32x32x16_bf16 with the weights dequantised in registers.
//
// "Module glm5next_mlp", forward_prefill_gemm / MOE_GROUPED_MODULE: every
// expert's sorted rows run through one W4A16 GEMM against that expert's NVFP4
// weights (E2M1 codes, one E4M3 scale per 16 columns of a row, an fp32 global
// per expert and projection applied after the sum).
//
// Why this kernel looks the way it does (measured on gfx950):
//   * A global->LDS DMA instruction costs the texture path about two cycles
//     per distinct 128-byte line its 64 lanes touch.  Loads where each lane
//     reads 16 bytes of a different weight or activation row therefore run at
//     a quarter (or less) of the rate of loads where eight lanes cover one
//     128-byte line.  Every DMA here is laid out for whole lines: activations
//     8 lanes per row (one 64-column stage = 128 bytes), codes 4 lanes per
//     row (two stages = 64 bytes), scales one lane per row (four stages = 16
//     bytes, the scale array being the smallest stream).
//   * The lane -> (row, 16-byte piece) assignment of each DMA is free (the
//     LDS side is always lane-contiguous), so the XOR swizzle that keeps the
//     MFMA operand reads free of bank conflicts is applied on the global side.
//   * One workgroup of 8 wavefronts per CU, tile = 128 rows x 512 weight rows
//     (gate/up: 256 gate + the matching 256 up rows; down: 512 output
//     columns).  Each wavefront owns all 128 rows x 64 weight rows (4 x 2
//     MFMA tiles), so every weight element is dequantised once per tile and
//     each activation stage in LDS feeds 512 output columns.
//   * LDS rings: activations 4 stages (16 KB each), codes 2 units of two
//     stages (32 KB each), scales 2 groups of four stages (8 KB each): 144 KB.
//     The DMA schedule is static (a prologue, a first, middle and last block
//     of four stages), so every wait is a compile-time count; activation and
//     code and scale slots are separate LDS arrays whose reads the compiler
//     schedules (the next k-step's activation fragments are read during the
//     current k-step's MFMAs).  The scale slot alternates per block of four
//     stages, so the middle blocks run in pairs and the parity of the block
//     count is a template parameter: every slot is a compile-time array (an
//     asm read from a run-time slot had to wait on itself at every stage;
//     measured 3% slower).
//
//   * Weight layout.  In the row-major layout a code instruction reads 64
//     bytes of each of 16 rows (16 half lines) and a scale instruction 16
//     bytes of each of 64 rows (64 lines).  The tile layout
//     (k_nvfp4_tile_pack) stores exactly the bytes of one instruction
//     contiguously, in the order its lanes deliver them to LDS (the LDS
//     swizzle included): 1 KB of codes, two 512-byte runs of scales.  The
//     scale runs are stage-major (the 32 rows' words of one stage side by
//     side), so that a stage's scale read touches 32 consecutive words: in
//     the row-major layout's LDS image the rows are 16 bytes apart and rows
//     16 apart share a bank (measured: those reads were every LDS bank
//     conflict of the kernel).  Codes in LDS, and all arithmetic, are the
//     same for both layouts.
//
// Rows past the tile's valid count load row 0 again (outputs dropped); weight
// rows past the matrix edge load row 0 again (outputs not stored).  Requires
// kdim % 256 == 0 and kdim >= 512.
#pragma once

#include "common.hpp"
#include "gemm.hpp"

#include <type_traits>

namespace moe {

constexpr int F4_WROWS = 512;      // weight rows per workgroup
constexpr int F4_THREADS = 512;    // 8 wavefronts

// 16-byte position of activation chunk c (0..7) of tile row r: c ^ f4_swz_a(r).
// Conflict-free MFMA operand reads whether a ds_read_b128 phase serves 8 or 16
// lanes (rows r..r+7 get distinct positions, and so do the even and the odd
// rows among r..r+15).
__device__ __forceinline__ int f4_swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// (f4_swz_c, the code-piece swizzle, is in common.hpp: the decode kernels read the tile layout too.)

// LDS of one workgroup: every ring slot is an array of its own (activations
// four, codes two, scales two), so that the compiler's wait insertion can tell
// a read of one slot from the DMA into another.
struct F4Lds {
  uint4* a[4];
  uint4* c[2];
  uint8_t* s[2];
};

// DMA sources: wave-uniform bases and this lane's 32-bit byte offsets
// (activations: its two rows' first chunk; codes: its four rows' first piece;
// scales: its row).  The host keeps every offset below 2^31.
struct F4Src {
  const uint8_t* a;
  uint32_t ao[2];
  const uint8_t* c;
  uint32_t co[4];
  const uint8_t* s;
  uint32_t so;
};

template <int MODE, int MTV, bool TILED, bool ODD>
__device__ __forceinline__ void f4_mainloop(const F4Lds& L, const F4Src& src, int wv, int lane, int kdim,
                                            f32x16 (&acc)[4][2]) {
  // weight-row stride between this lane's two n-tiles
  constexpr int NT_ROWS = MODE == GEMM_GATEUP ? 256 : 32;
  const int g = lane >> 5, ln = lane & 31;
  const int nkb = kdim >> 6;                   // stages; a multiple of 4, at least 8
  const int nblk4 = nkb >> 2;                  // blocks of four stages

  // ---- DMA issue (per wave: A = 2, C = 4, S = 1 instructions)
  auto issue_a = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src.a + (src.ao[i] + 128u * k)),
                                       (void __attribute__((address_space(3)))*)(L.a[SL] + wv * 128 + i * 64),
                                       16, 0, 0);
  };
  // code unit u (two stages) and scale group v (four stages) advance by 64
  // and 16 bytes along a row in the row-major layout, by a 1 KB and a 512-byte
  // block in the tile layout
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
                                     (void __attribute__((address_space(3)))*)(L.s[SSL] + wv * 1024),
                                     16, 0, 0);
  };

  // ---- consumer offsets (uint4 units within a ring entry)
  const int prow = (MODE == GEMM_GATEUP ? 32 * wv : 64 * wv) + ln;   // weight row of n-tile 0
  const int sc = f4_swz_c(prow), sa = f4_swz_a(ln);
  // scale word of (row, stage) in a scale slot: row-major image: row * 16 +
  // 4 stage; tile layout (stage-major per 32-row group): (row / 32) * 512 +
  // 128 stage + 4 (row % 32)
  constexpr int S_STAGE = TILED ? 128 : 4;
  int aidx[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aidx[s] = ln * 8 + ((4 * g + s) ^ sa);
  int cidx[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) cidx[t] = prow * 4 + ((2 * t + g) ^ sc);
  const int soff = (TILED ? (prow >> 5) * 512 + 4 * (prow & 31) : prow * 16) >> 2;   // in words

  // ---- one stage: wait for its data (VM = DMA instructions allowed to stay in
  // flight), barrier, then 4 k-steps of 8 MFMAs with the next k-step's
  // activation fragments read during the current one; the next loads are
  // issued after the first k-step
  auto stage = [&](int k, auto slot_c, auto ss_c, auto vm_c, auto issue) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int SS = decltype(ss_c)::value;
    constexpr int VM = decltype(vm_c)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint4* As = L.a[SL];
    const uint4* Cs = L.c[SL >> 1];
    uint32_t sw[2];
    {
      const uint32_t* Ss = reinterpret_cast<const uint32_t*>(L.s[SS]);
      sw[0] = Ss[soff + (S_STAGE >> 2) * SL];
      sw[1] = Ss[soff + (S_STAGE >> 2) * SL + NT_ROWS * 4];
    }
    uint4 cw[2];
    cw[0] = Cs[cidx[SL & 1]];
    cw[1] = Cs[cidx[SL & 1] + NT_ROWS * 4];
    // this lane's two scale bytes (its 32 columns = two 16-blocks) sit at bytes 2g, 2g+1
    const uint32_t s0 = sw[0] >> (16 * g), s1 = sw[1] >> (16 * g);
    // activation fragments: each is re-read for the next k-step right after
    // its last MFMA of this one, so the reads overlap the remaining MFMAs
    bf16x8 af[MTV];
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt) af[mt] = __builtin_bit_cast(bf16x8, As[aidx[0] + mt * 256]);
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
      for (int mt = 0; mt < MTV; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfrag[nt], acc[mt][nt], 0, 0, 0);
        if (s < 3) af[mt] = __builtin_bit_cast(bf16x8, As[aidx[(s + 1) & 3] + mt * 256]);
      }
      // the next loads go out after the first k-step's MFMAs, not in the burst
      // of LDS reads that follows the barrier (measured: a few percent)
      if (s == 0) issue();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Issue schedule (A(k) = activation stage k into slot k%4, C(u) = code unit u
  // into slot u%2, S(v) = scale group v into slot v%2).  Prologue: S0 C0 A0 C1
  // A1 A2 S1.  Stage k of a middle block issues, after its barrier:
  //   k%4 == 0: S(k/4+1) C(k/2+1) A(k+3); 1: A(k+3); 2: C(k/2+1) A(k+3); 3: A(k+3)
  // The first block skips S and C at k = 0; the last block issues only
  // C(k/2+1) A(k+3) at its first stage.  Counting the DMA instructions issued
  // after the last one each stage needs gives the waits below.
  issue_s(0, I0{});
  issue_c(0, I0{});
  issue_a(0, I0{});
  issue_c(1, I1{});
  issue_a(1, I1{});
  issue_a(2, I2{});
  issue_s(1, I1{});
  using V0 = std::integral_constant<int, 0>;
  using V2 = std::integral_constant<int, 2>;
  using V4 = std::integral_constant<int, 4>;
  using V5 = std::integral_constant<int, 5>;
  using V8 = std::integral_constant<int, 8>;
  using V9 = std::integral_constant<int, 9>;
  // first block (scale slot 0)
  stage(0, I0{}, I0{}, V9{}, [&] { issue_a(3, I3{}); });
  stage(1, I1{}, I0{}, V5{}, [&] { issue_a(4, I0{}); });
  stage(2, I2{}, I0{}, V5{}, [&] { issue_c(2, I0{}); issue_a(5, I1{}); });
  stage(3, I3{}, I0{}, V8{}, [&] { issue_a(6, I2{}); });
  // middle block j reads scale slot j % 2 and loads group j + 1 into the other
  auto middle = [&](int j, auto ss_c) {
    using NS = std::integral_constant<int, decltype(ss_c)::value ^ 1>;
    const int k = 4 * j;
    stage(k, I0{}, ss_c, V4{}, [&] { issue_s(j + 1, NS{}); issue_c(2 * j + 1, I1{}); issue_a(k + 3, I3{}); });
    stage(k + 1, I1{}, ss_c, V9{}, [&] { issue_a(k + 4, I0{}); });
    stage(k + 2, I2{}, ss_c, V4{}, [&] { issue_c(2 * j + 2, I0{}); issue_a(k + 5, I1{}); });
    stage(k + 3, I3{}, ss_c, V8{}, [&] { issue_a(k + 6, I2{}); });
  };
  auto last = [&](auto ss_c) {
    const int j = nblk4 - 1, k = 4 * j;
    stage(k, I0{}, ss_c, V4{}, [&] { issue_c(2 * j + 1, I1{}); issue_a(k + 3, I3{}); });
    stage(k + 1, I1{}, ss_c, V8{}, [] {});
    stage(k + 2, I2{}, ss_c, V2{}, [] {});
    stage(k + 3, I3{}, ss_c, V0{}, [] {});
  };
  // middle blocks in pairs (slots 1, 0), so every slot is a compile-time
  // array; ODD = an odd number of blocks of four stages (one unpaired middle
  // block, and the last block then reads slot 0)
  const int jend = nblk4 - 1 - (ODD ? 1 : 0);
  for (int j = 1; j < jend; j += 2) {
    middle(j, I1{});
    middle(j + 1, I0{});
  }
  if constexpr (ODD) {
    middle(nblk4 - 2, I1{});
    last(I0{});
  } else {
    last(I1{});
  }
}

// Grid: 1-D, XCD-aware as in k_gemm_fast (block b runs on XCD b % 8; each XCD
// takes a contiguous run of (tile, column block) work, column blocks of a
// tile back to back).  n_blocks = column blocks of F4_WROWS weight rows
// (gate/up: 256 gate columns each).  TILED: codes and scales in the tile
// layout (a.bq_t, a.bs_t).
template <int MODE, bool TILED>
__global__ __launch_bounds__(F4_THREADS, 1) void k_gemm_nvfp4(GemmArgs a) {
  const int nbn = a.n_blocks;
  // with skip_rows, the tiles of more than skip_rows rows (the scheduler puts them first)
  const int ntl = a.skip_rows ? a.n_tiles[1] : a.n_tiles[0];
  const int total = ntl * nbn, chunk = (total + 7) >> 3;
  const int kk = blockIdx.x >> 3;
  if (kk >= chunk) return;
  const int w = (blockIdx.x & 7) * chunk + kk;
  if (w >= total) return;
  const int tile = w / nbn, nblk = w - tile * nbn;
  const int e = a.tile_expert[tile];
  const int m0 = a.tile_m0[tile];
  const int valid = min(GM_BM, a.count[e] - m0);
  if (valid <= a.skip_rows) return;
  const int p0 = a.offset[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;

  // activation DMA: instruction i of wave wv covers tile rows 16 wv + 8 i .. +7,
  // 8 lanes per row, lane -> 16-byte chunk (lane & 7) ^ swizzle
  F4Src src;
  src.a = reinterpret_cast<const uint8_t*>(a.a);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * wv + 8 * i + (lane >> 3);
    const int rr = r < valid ? r : 0;
    const int64_t row = (MODE == GEMM_GATEUP) ? a.perm[p0 + rr] / a.K : p0 + rr;
    src.ao[i] = static_cast<uint32_t>((row * kdim + 8 * ((lane & 7) ^ f4_swz_a(r))) * 2);
  }
  // weight row of workgroup row p (0..511); rows past the edge reload row 0
  auto wrow = [&](int p) -> int64_t {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 256 + (p & 255);
      return j < a.half_n ? (p < 256 ? j : a.half_n + j) : 0;
    } else {
      const int n = nblk * F4_WROWS + p;
      return n < a.half_n ? n : 0;
    }
  };
  // code DMA: instruction i of wave wv covers workgroup rows 16 (4 wv + i) .. +15,
  // 4 lanes per row, lane -> 16-byte piece q = (lane & 3) ^ swizzle of a 64-byte
  // unit.  Tile layout: row R's piece q sits at 16 (4 (R % 16) + (q ^ z(R % 16)))
  // of its 16-row group's block, i.e. at 16 lane when the rows are in the matrix
  // (z = the same swizzle, which depends on R % 16 only).
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
  // scale DMA, row-major: workgroup row 64 wv + lane, 16 bytes (four stages)
  // per group.  Tile layout: lanes 32 G .. 32 G + 31 take the 512-byte block
  // of the 32-row group that starts at workgroup row 64 wv + 32 G (a block is
  // stage-major, so lane l's 16 bytes are stage l / 8, rows 4 (l % 8) .. +3).
  src.s = (TILED ? a.bs_t : a.bs) + e * a.stride_s;
  if (TILED) {
    const int64_t R0 = wrow(64 * wv + 32 * (lane >> 5));
    src.so = static_cast<uint32_t>((R0 >> 5) * (kdim >> 8) * 512 + 16 * (lane & 31));
  } else {
    src.so = static_cast<uint32_t>(wrow(64 * wv + lane) * (kdim >> 4));
  }

  __shared__ uint4 la0[1024], la1[1024], la2[1024], la3[1024];   // activation ring (16 KB each)
  __shared__ uint4 lc0[2048], lc1[2048];                          // code ring (32 KB each)
  __shared__ __attribute__((aligned(16))) uint8_t ls0[F4_WROWS * 16], ls1[F4_WROWS * 16];   // scale ring
  const F4Lds L{{la0, la1, la2, la3}, {lc0, lc1}, {ls0, ls1}};
  // down: the tile's output rows, lane l holding rows l and 64 + l, read before
  // the main loop (a read per row in the epilogue waits for every store before it)
  int orow_l[2] = {0, 0};
  if constexpr (MODE != GEMM_GATEUP) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * i + lane;
      orow_l[i] = a.perm[p0 + (r < valid ? r : 0)];
    }
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;
  if ((kdim >> 8) & 1) {
    switch ((valid + 31) >> 5) {
      case 1: f4_mainloop<MODE, 1, TILED, true>(L, src, wv, lane, kdim, acc); break;
      case 2: f4_mainloop<MODE, 2, TILED, true>(L, src, wv, lane, kdim, acc); break;
      case 3: f4_mainloop<MODE, 3, TILED, true>(L, src, wv, lane, kdim, acc); break;
      default: f4_mainloop<MODE, 4, TILED, true>(L, src, wv, lane, kdim, acc); break;
    }
  } else {
    switch ((valid + 31) >> 5) {
      case 1: f4_mainloop<MODE, 1, TILED, false>(L, src, wv, lane, kdim, acc); break;
      case 2: f4_mainloop<MODE, 2, TILED, false>(L, src, wv, lane, kdim, acc); break;
      case 3: f4_mainloop<MODE, 3, TILED, false>(L, src, wv, lane, kdim, acc); break;
      default: f4_mainloop<MODE, 4, TILED, false>(L, src, wv, lane, kdim, acc); break;
    }
  }

  const int mt_valid = (valid + 31) >> 5;
  const int ln = lane & 31;
  float g0, g1 = 1.0f;
  if (MODE == GEMM_GATEUP) {
    g0 = a.gscale ? a.gscale[2 * e] : 1.0f;
    g1 = a.gscale ? a.gscale[2 * e + 1] : 1.0f;
  } else {
    g0 = a.gscale ? a.gscale[e] : 1.0f;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt >= mt_valid) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = mt * 32 + c32_row(lane, j);
      int orow_i = 0;
      if constexpr (MODE != GEMM_GATEUP) orow_i = __shfl(orow_l[mt >> 1], row & 63);
      if (row >= valid) continue;
      if (MODE == GEMM_GATEUP) {
        const int jc = nblk * 256 + 32 * wv + ln;
        if (jc >= a.half_n) continue;
        static_cast<uint16_t*>(a.out)[static_cast<int64_t>(p0 + row) * a.ldo + jc] =
            f32_to_bf16(swiglu_clamped(g0 * acc[mt][0][j], g1 * acc[mt][1][j], a.limit));
      } else {
        const int64_t orow = orow_i;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int n = nblk * F4_WROWS + 64 * wv + 32 * nt + ln;
          if (n < a.half_n) static_cast<float*>(a.out)[orow * a.ldo + n] = g0 * acc[mt][nt][j];
        }
      }
    }
  }
}

// Row-major NVFP4 codes / scales -> the tile layout (moe_nvfp4_tile_pack):
// one thread per 16-byte piece, codes first (mats * rows * cols/32 pieces),
// then scales (mats * rows * cols/256 pieces).  rows % 32 == 0, cols % 256 == 0.
__global__ __launch_bounds__(256) void k_nvfp4_tile_pack(const uint8_t* __restrict__ q,
                                                         const uint8_t* __restrict__ s, int64_t mats, int64_t rows,
                                                         int64_t cols, uint8_t* __restrict__ qt,
                                                         uint8_t* __restrict__ st) {
  const int64_t nq = mats * rows * (cols >> 5), ns = mats * rows * (cols >> 8);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < nq) {
    const int L = static_cast<int>(idx & 63);
    const int64_t blk = idx >> 6, units = cols >> 7, groups = rows >> 4;
    const int64_t u = blk % units, r = (blk / units) % groups, m = blk / units / groups;
    const int64_t row = m * rows + 16 * r + (L >> 2);
    const int piece = (L & 3) ^ f4_swz_c(L >> 2);
    reinterpret_cast<uint4*>(qt)[idx] =
        *reinterpret_cast<const uint4*>(q + row * (cols >> 1) + 64 * u + 16 * piece);
  } else if (idx < nq + ns) {
    // piece P of a scale block: stage P / 8, rows 4 (P % 8) .. +3 of the group
    const int64_t j = idx - nq;
    const int P = static_cast<int>(j & 31);
    const int64_t blk = j >> 5, units = cols >> 8, groups = rows >> 5;
    const int64_t v = blk % units, r = (blk / units) % groups, m = blk / units / groups;
    const int64_t row = m * rows + 32 * r + 4 * (P & 7);
    const int64_t col = 16 * v + 4 * (P >> 3);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const uint32_t*>(s + (row + i) * (cols >> 4) + col);
    reinterpret_cast<uint4*>(st)[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace moe
