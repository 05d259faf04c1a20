// Prefill projections on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// "Module glm5next_mlp", forward_prefill_gemm / MOE_GROUPED_MODULE: routed
// prefill runs each expert's sorted rows through a grouped W4A16 GEMM.  The
// same kernel, with BF16 weights and identity rows, runs the shared expert and
// the dense FFN (the page's DENSE layer: BF16 gate/up, clamped SwiGLU, down).
//
// Tiling (one workgroup = 4 wavefronts, 128 rows of A):
//   * A (activations, bf16) is staged through LDS in MFMA-fragment order, two
//     stages of 128 x 128; every wavefront reads all 128 rows from LDS.
//   * B (weights) goes straight from HBM into each wavefront's registers:
//     wavefront w owns 64 output columns (4 MFMA n-tiles).  For NVFP4 a lane
//     loads 16 bytes = 32 codes of one weight row and their two E4M3 scales,
//     and turns them into four bf16x8 MFMA operands (exact: e2m1 x e4m3 fits
//     bf16); the per-expert fp32 global scale is applied in the epilogue.
//   * The reduction order inside a 128-wide k block is permuted identically
//     for A and B (lane group g covers k0+32g..k0+32g+31 and k-step s its
//     elements 8s..8s+7), which leaves the dot products unchanged.
//   * Gate/up: a wavefront's n-tiles are gate columns j..j+31 and the up
//     columns I+j..I+j+31, so the clamped SwiGLU pairs accumulators held by
//     the same lane.
//   * Rows past the tile's valid count are zero in A, their MFMAs skipped
//     (16-row granularity) and their outputs not stored.
#pragma once

#include "common.hpp"

#include <type_traits>

namespace moe {

constexpr int GM_BM = 128;
constexpr int GM_BK = 128;

enum GemmMode {
  GEMM_GATEUP = 0,          // h[row][j] = bf16(swiglu(G0*gate, G1*up))
  GEMM_DOWN_SLOT_F32 = 1,   // y[perm(row)][n] = G2*acc (routed down, un-permuted)
  GEMM_DOWN_BF16 = 2,       // out[row][n] = bf16(acc) (dense down)
  GEMM_DOWN_F32 = 3,        // ys[row][n] = acc (shared down)
};

struct GemmArgs {
  const uint16_t* a;         // activations, row length kdim
  int kdim;                  // reduction length (multiple of 32)
  const uint8_t* bq;         // NVFP4 codes [E][rows][kdim/2]
  const uint8_t* bs;         // NVFP4 scales [E][rows][kdim/16]
  const uint16_t* bb;        // BF16 weights [rows][kdim]
  const uint8_t* bq_t;       // NVFP4 codes and scales in the tile layout (tile
  const uint8_t* bs_t;       //   kernel only; null = read bq / bs)
  const float* bsf;          // FP8 experts: fp32 128 x 128 block scales [E][rows/128][kdim/128]
                             //   (bq then holds E4M3 bytes [E][rows][kdim])
  int64_t stride_q, stride_s;
  const float* gscale;       // routed globals (gate/up: [E,2]; down: [E]); null = 1
  int half_n;                // gate/up: I (gate rows, up rows = I + j); down: output columns
  // routed tiles
  const int32_t* n_tiles;
  const int32_t* tile_expert;
  const int32_t* tile_m0;
  const int32_t* count;
  const int32_t* offset;
  const int32_t* perm;
  int T;                     // dense rows (routed NVFP4 GEMM: activation rows)
  int K;                     // slot -> token = slot / K (routed gate/up gather)
  void* out;
  int ldo;
  float limit;
  int n_blocks;              // output-column blocks (fast kernel's 1-D work mapping)
  // BF16 fast kernel only: row strides of A and B (0 = kdim), and a split of
  // the reduction into ksplit parts of kdim each (A and B columns advance by
  // kdim per part, part q writes its fp32 result split_out elements after part
  // q-1; GEMM_DOWN_F32 only)
  int lda, ldb;
  int ksplit;
  int64_t split_out;
  // routed NVFP4 kernel only: tiles of at most skip_rows rows are left to
  // k_gemm_nvfp4_m32 (0 = none)
  int skip_rows;
  // k_gemm_nvfp4_m32 only: with split_pass > 0 each of the first n_tiles[1]
  // tiles (those of more than 32 rows) is taken by split_pass workgroups, one
  // 32-row pass each, ahead of the other tiles (0 = passes in one workgroup)
  int split_pass;
};

template <bool NVFP4, int MODE, bool ROUTED>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  __shared__ uint4 lds[2][8 * 4 * 64];   // 2 stages x (8 m-tiles x 4 k-steps x 64 lanes x 16 B)
  const int tile = blockIdx.x, nblk = blockIdx.y;   // x: M tiles, y: N blocks
  int e = 0, m0, valid, p0;
  if (ROUTED) {
    if (tile >= *a.n_tiles) return;
    e = a.tile_expert[tile];
    m0 = a.tile_m0[tile];
    valid = min(GM_BM, a.count[e] - m0);
    p0 = a.offset[e] + m0;
  } else {
    m0 = tile * GM_BM;
    if (m0 >= a.T) return;
    valid = min(GM_BM, a.T - m0);
    p0 = m0;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kdim = a.kdim;
  const int mt_valid = static_cast<int>(cdiv(valid, 16));

  // ---- A loader: thread owns row r, half h (64 columns of a 128 block)
  const int ar = tid >> 1, ah = tid & 1;
  const uint16_t* arow = nullptr;
  if (ar < valid) {
    if (ROUTED && MODE == GEMM_GATEUP) {
      const int slot = a.perm[p0 + ar];
      arow = a.a + static_cast<int64_t>(slot / a.K) * kdim;
    } else {
      arow = a.a + static_cast<int64_t>(p0 + ar) * kdim;
    }
  }

  // ---- B rows of this wavefront's 4 n-tiles
  const int g = lane >> 4, ln = lane & 15;
  int brow[4];
  bool bvalid[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 128 + wv * 32 + (nt & 1) * 16 + ln;
      bvalid[nt] = j < a.half_n;
      const int jj = bvalid[nt] ? j : 0;
      brow[nt] = nt < 2 ? jj : a.half_n + jj;
    } else {
      const int n = nblk * 256 + wv * 64 + nt * 16 + ln;
      bvalid[nt] = n < a.half_n;
      brow[nt] = bvalid[nt] ? n : 0;
    }
  }
  const uint8_t* bq = nullptr;
  const uint8_t* bs = nullptr;
  if (NVFP4) {
    bq = a.bq + e * a.stride_q;
    bs = a.bs + e * a.stride_s;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  uint4 av[8];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int col = k0 + 64 * ah + 8 * q;
      av[q] = (arow && col < kdim) ? *reinterpret_cast<const uint4*>(arow + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int gg = 2 * ah + (q >> 2), ks = q & 3;
      lds[buf][((ar >> 4) * 4 + ks) * 64 + (ar & 15) + 16 * gg] = av[q];
    }
  };

  const int nkb = static_cast<int>(cdiv(kdim, GM_BK));
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * GM_BK;
    const int buf = kb & 1;
    const int kg = k0 + 32 * g;              // first k of this lane's group
    const bool kvalid = kg < kdim;
    // B for this k block
    uint4 bcode[4];
    uint32_t bscale[4];
    if (NVFP4) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (kvalid) {
          bcode[nt] = *reinterpret_cast<const uint4*>(bq + static_cast<int64_t>(brow[nt]) * (kdim >> 1) + (kg >> 1));
          bscale[nt] = *reinterpret_cast<const uint16_t*>(bs + static_cast<int64_t>(brow[nt]) * (kdim >> 4) + (kg >> 4));
        } else {
          bcode[nt] = make_uint4(0, 0, 0, 0);
          bscale[nt] = 0;
        }
      }
    }
    if (kb + 1 < nkb) load_a(k0 + GM_BK);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bfrag[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        uint4 v;
        if (NVFP4) {
          const uint32_t cw = ks == 0 ? bcode[nt].x : ks == 1 ? bcode[nt].y : ks == 2 ? bcode[nt].z : bcode[nt].w;
          const float s = (ks < 2) ? e4m3_to_f32<0>(bscale[nt]) : e4m3_to_f32<1>(bscale[nt]);
          uint32_t o[4];
          e2m1x8_scaled_bf16(cw, s, o);
          v = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          v = kvalid ? *reinterpret_cast<const uint4*>(a.bb + static_cast<int64_t>(brow[nt]) * kdim + kg + 8 * ks)
                     : make_uint4(0, 0, 0, 0);
        }
        bfrag[nt] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (mt < mt_valid) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, lds[buf][(mt * 4 + ks) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfrag[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows mt*16 + 4*(lane>>4) + i, column ln of each n-tile
  float g0 = 1.0f, g1 = 1.0f;
  if (ROUTED && a.gscale) {
    if (MODE == GEMM_GATEUP) {
      g0 = a.gscale[2 * e];
      g1 = a.gscale[2 * e + 1];
    } else {
      g0 = a.gscale[e];
    }
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt >= mt_valid) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * (lane >> 4) + i;
      if (row >= valid) continue;
      if (MODE == GEMM_GATEUP) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + static_cast<int64_t>(p0 + row) * a.ldo;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if (!bvalid[nt]) continue;
          const int j = nblk * 128 + wv * 32 + nt * 16 + ln;
          o[j] = f32_to_bf16(swiglu_clamped(g0 * acc[mt][nt][i], g1 * acc[mt][nt + 2][i], a.limit));
        }
      } else {
        int64_t orow;
        if (MODE == GEMM_DOWN_SLOT_F32) orow = a.perm[p0 + row];
        else orow = p0 + row;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (!bvalid[nt]) continue;
          const int n = nblk * 256 + wv * 64 + nt * 16 + ln;
          if (MODE == GEMM_DOWN_BF16)
            static_cast<uint16_t*>(a.out)[orow * a.ldo + n] = f32_to_bf16(acc[mt][nt][i]);
          else
            static_cast<float*>(a.out)[orow * a.ldo + n] = g0 * acc[mt][nt][i];
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fast grouped / dense GEMM (kdim % 64 == 0): v_mfma_f32_32x32x16_bf16.
//   * workgroup tile 128 rows x 256 output columns (gate/up: 128 gate + the
//     matching 128 up columns), 4 wavefronts of 128 x 64 (4 x 2 MFMA tiles);
//   * A goes global -> LDS directly (global_load_lds_dwordx4) into an NST-deep
//     ring in MFMA-fragment order: lane l of wavefront w loads 64 contiguous
//     bytes of row 32w + l%32 at k0 + 32*(l/32);
//   * B (NVFP4 16-byte code chunks + their 2 E4M3 scale bytes, or BF16) goes
//     into an NST-deep register ring and is turned into bf16 operands per
//     k-step;
//   * the main loop is instantiated per valid 32-row m-tile count, so it has
//     no branches;
//   * 1-D grid, XCD-aware: block b runs on XCD b % 8, and each XCD takes a
//     contiguous chunk of (tile, column-block) work with the column blocks of
//     a tile back to back, so the tile's A rows stay in that XCD's L2.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16 output: lane l, element j -> row (j/4)*8 + (l/32)*4 + j%4, column l%32.
__device__ __forceinline__ int c32_row(int lane, int j) { return (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3); }

template <bool NVFP4, int NST>
struct BRing {
  static constexpr int BW = NVFP4 ? 1 : 4;
  uint4 b[NST][2][BW];
  uint32_t s[NST][2];
};

template <bool NVFP4, int NST, int MTV>
__device__ __forceinline__ void gemm_fast_mainloop(const GemmArgs& a, uint4 (&L0)[1024], uint4 (&L1)[1024],
                                                   uint4 (&L2)[1024], uint4 (&L3)[1024], const uint16_t* arow,
                                                   const uint8_t* bq, const uint8_t* bs, const int (&brow)[2],
                                                   int wv, int lane, int g, int kdim, f32x16 (&acc)[4][2]) {
  constexpr int BK = 64;
  constexpr int BW = NVFP4 ? 1 : 4;
  constexpr int LOADS = 4 + (NVFP4 ? 4 : 8);      // vector memory instructions per stage per lane
  const int nkb = kdim / BK;
  BRing<NVFP4, NST> r;
  auto slot_lds = [&](auto slot_c) -> uint4* {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL == 0) return L0;
    else if constexpr (SL == 1) return L1;
    else if constexpr (SL == 2) return L2;
    else return L3;
  };
  const int64_t ldb = a.ldb ? a.ldb : kdim;
  auto issue = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const int kg = k * BK + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(arow + kg + 8 * s),
                                       (void __attribute__((address_space(3)))*)&slot_lds(slot_c)[(wv * 4 + s) * 64],
                                       16, 0, 0);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (NVFP4) {
        r.b[SL][nt][0] = *reinterpret_cast<const uint4*>(bq + static_cast<int64_t>(brow[nt]) * (kdim >> 1) + (kg >> 1));
        r.s[SL][nt] = *reinterpret_cast<const uint16_t*>(bs + static_cast<int64_t>(brow[nt]) * (kdim >> 4) + (kg >> 4));
      } else {
#pragma unroll
        for (int q = 0; q < BW; ++q)
          r.b[SL][nt][q] = *reinterpret_cast<const uint4*>(a.bb + static_cast<int64_t>(brow[nt]) * ldb + kg + 8 * q);
      }
    }
  };
  auto compute = [&](auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[MTV];
#pragma unroll
      for (int mt = 0; mt < MTV; ++mt) af[mt] = __builtin_bit_cast(bf16x8, slot_lds(slot_c)[(mt * 4 + s) * 64 + lane]);
      bf16x8 bfrag[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint4 v;
        if (NVFP4) {
          const uint4 c = r.b[SL][nt][0];
          const uint32_t cw = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
          const float scale = (s < 2) ? e4m3_to_f32<0>(r.s[SL][nt]) : e4m3_to_f32<1>(r.s[SL][nt]);
          uint32_t o[4];
          e2m1x8_scaled_bf16(cw, scale, o);
          v = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          v = r.b[SL][nt][s];
        }
        bfrag[nt] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfrag[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  if (0 < nkb) issue(0, std::integral_constant<int, 0>{});
  if (NST > 2 && 1 < nkb) issue(1, std::integral_constant<int, 1 % NST>{});
  if (NST > 3 && 2 < nkb) issue(2, std::integral_constant<int, 2 % NST>{});
  auto step = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if (k >= nkb) return;
    const int ahead = min(nkb - 1 - k, NST - 2);   // stages issued after k still allowed in flight
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (k + NST - 1 < nkb) issue(k + NST - 1, std::integral_constant<int, (SL + NST - 1) % NST>{});
    compute(slot_c);
  };
  for (int k = 0; k < nkb; k += NST) {
    step(k, std::integral_constant<int, 0>{});
    step(k + 1, std::integral_constant<int, 1 % NST>{});
    step(k + 2, std::integral_constant<int, 2 % NST>{});
    if (NST == 4) step(k + 3, std::integral_constant<int, 3 % NST>{});
  }
}

// The MTV A fragments of one k-step from LDS: ds_read_b128 at base +
// mt * 4096 bytes, in one asm statement that also waits for them, so the
// compiler adds no wait of its own for LDS DMA (see gemm_dma_mainloop).
// Early-clobber outputs: every read of the block uses the address register.
template <int MTV>
__device__ __forceinline__ void lds_a_frags(uint32_t base, bf16x8 (&af)[MTV]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v0, v1, v2, v3;
  if constexpr (MTV == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v0) : "v"(base) : "memory");
  } else if constexpr (MTV == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:4096\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1) : "v"(base) : "memory");
  } else if constexpr (MTV == 3) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:4096\n\tds_read_b128 %2, %3 offset:8192\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2) : "v"(base) : "memory");
  } else {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:4096\n\tds_read_b128 %2, %4 offset:8192\n\t"
                 "ds_read_b128 %3, %4 offset:12288\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3) : "v"(base) : "memory");
  }
  af[0] = __builtin_bit_cast(bf16x8, v0);
  if constexpr (MTV > 1) af[1] = __builtin_bit_cast(bf16x8, v1);
  if constexpr (MTV > 2) af[2] = __builtin_bit_cast(bf16x8, v2);
  if constexpr (MTV > 3) af[3] = __builtin_bit_cast(bf16x8, v3);
}

// This lane's NVFP4 operand of one stage from LDS: the 16-byte code chunks of
// its two columns (n-tile stride 4096 bytes) and the E4M3 scale words (stride
// 1024 bytes), in one asm statement that waits for them.
__device__ __forceinline__ void lds_b_stage(uint32_t cbase, uint32_t sbase, uint4 (&c)[2], uint32_t (&sc)[2]) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 c0, c1;
  uint32_t s0, s1;
  asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:4096\n\tds_read_b32 %2, %5\n\t"
               "ds_read_b32 %3, %5 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(c0), "=&v"(c1), "=&v"(s0), "=&v"(s1) : "v"(cbase), "v"(sbase) : "memory");
  c[0] = make_uint4(c0.x, c0.y, c0.z, c0.w);
  c[1] = make_uint4(c1.x, c1.y, c1.z, c1.w);
  sc[0] = s0;
  sc[1] = s1;
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T*)p));
}

// NVFP4 main loop with every operand staged by LDS DMA (global_load_lds):
// per 64-wide k stage a lane issues 4 x 16 B of A (as above), the 16-byte
// code chunk of each of its two weight rows, and the 4-byte scale word of
// each row that holds both of its 16-column blocks' E4M3 scales.  The only
// vector memory operations in flight in the loop are these DMAs, which
// complete in issue order, so the explicit vmcnt waits (at most one later
// stage in flight) plus a bare barrier order each stage, and the compiler
// adds no wait for all outstanding loads (see compute() for which LDS reads
// are asm statements).  Three-stage ring, 26 KB per stage.
template <int MTV>
__device__ __forceinline__ void gemm_dma_mainloop(uint4 (&A0)[1024], uint4 (&A1)[1024], uint4 (&A2)[1024],
                                                  uint4 (&C0)[512], uint4 (&C1)[512], uint4 (&C2)[512],
                                                  uint32_t (&S0)[512], uint32_t (&S1)[512], uint32_t (&S2)[512],
                                                  const uint16_t* arow, const uint8_t* bq, const uint8_t* bs,
                                                  const int (&brow)[2], int wv, int lane, int g, int kdim,
                                                  f32x16 (&acc)[4][2]) {
  constexpr int BK = 64, LOADS = 8;
  const int nkb = kdim / BK;
  const uint8_t* qrow[2];
  const uint8_t* srow[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    qrow[nt] = bq + static_cast<int64_t>(brow[nt]) * (kdim >> 1);
    srow[nt] = bs + static_cast<int64_t>(brow[nt]) * (kdim >> 4);
  }
  auto slotA = [&](auto c) -> uint4* {
    constexpr int SL = decltype(c)::value;
    if constexpr (SL == 0) return A0; else if constexpr (SL == 1) return A1; else return A2;
  };
  auto slotC = [&](auto c) -> uint4* {
    constexpr int SL = decltype(c)::value;
    if constexpr (SL == 0) return C0; else if constexpr (SL == 1) return C1; else return C2;
  };
  auto slotS = [&](auto c) -> uint32_t* {
    constexpr int SL = decltype(c)::value;
    if constexpr (SL == 0) return S0; else if constexpr (SL == 1) return S1; else return S2;
  };
  auto issue = [&](int k, auto slot_c) {
    const int kg = k * BK + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(arow + kg + 8 * s),
                                       (void __attribute__((address_space(3)))*)&slotA(slot_c)[(wv * 4 + s) * 64],
                                       16, 0, 0);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(qrow[nt] + (kg >> 1)),
                                       (void __attribute__((address_space(3)))*)&slotC(slot_c)[(nt * 4 + wv) * 64],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(srow[nt] + 4 * k),
                                       (void __attribute__((address_space(3)))*)&slotS(slot_c)[(nt * 4 + wv) * 64],
                                       4, 0, 0);
    }
  };
  auto compute = [&](auto slot_c) {
    // Slot 0 is read first after the loop back-edge, where the compiler
    // cannot tell which ring slots still have DMA in flight and would wait
    // for all of them: its reads are asm.  Slots 1 and 2 use plain LDS reads,
    // which the compiler interleaves with the MFMAs.
    constexpr bool ASM_READS = decltype(slot_c)::value == 0;
    uint4 cw[2];
    uint32_t sw[2];
    if constexpr (ASM_READS) {
      lds_b_stage(lds_addr(&slotC(slot_c)[wv * 64 + lane]), lds_addr(&slotS(slot_c)[wv * 64 + lane]), cw, sw);
    } else {
      cw[0] = slotC(slot_c)[wv * 64 + lane];
      cw[1] = slotC(slot_c)[256 + wv * 64 + lane];
      sw[0] = slotS(slot_c)[wv * 64 + lane];
      sw[1] = slotS(slot_c)[256 + wv * 64 + lane];
    }
    // this lane's two scale bytes (its 32 columns = two 16-blocks) sit at bytes 2g, 2g+1
    const uint32_t s0 = sw[0] >> (16 * g), s1 = sw[1] >> (16 * g);
    const uint32_t abase = lds_addr(&slotA(slot_c)[lane]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[MTV];
      if constexpr (ASM_READS) {
        lds_a_frags<MTV>(abase + s * 1024, af);
      } else {
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt) af[mt] = __builtin_bit_cast(bf16x8, slotA(slot_c)[(mt * 4 + s) * 64 + lane]);
      }
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
      for (int mt = 0; mt < MTV; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfrag[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  issue(0, std::integral_constant<int, 0>{});
  if (1 < nkb) issue(1, std::integral_constant<int, 1>{});
  auto step = [&](int k, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if (k >= nkb) return;
    if (k + 1 < nkb) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LOADS));   // stage k+1 may stay in flight
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (k + 2 < nkb) issue(k + 2, std::integral_constant<int, (SL + 2) % 3>{});
    compute(slot_c);
  };
  for (int k = 0; k < nkb; k += 3) {
    step(k, std::integral_constant<int, 0>{});
    step(k + 1, std::integral_constant<int, 1>{});
    step(k + 2, std::integral_constant<int, 2>{});
  }
}

template <bool NVFP4, int MODE, bool ROUTED, int NST>
__global__ __launch_bounds__(256, 2) void k_gemm_fast(GemmArgs a) {
  // work item -> (tile, column block), XCD-aware (see above)
  const int nbn = a.n_blocks;
  const int ntl = ROUTED ? *a.n_tiles : static_cast<int>(cdiv(a.T, GM_BM));
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  const int total = ntl * nbn * ks, chunk = (total + 7) >> 3;
  const int kk = blockIdx.x >> 3;
  if (kk >= chunk) return;
  const int w0 = (blockIdx.x & 7) * chunk + kk;
  if (w0 >= total) return;
  const int split = w0 % ks, w = w0 / ks;
  const int tile = w / nbn, nblk = w - tile * nbn;
  int e = 0, valid, p0;
  if (ROUTED) {
    e = a.tile_expert[tile];
    const int m0 = a.tile_m0[tile];
    valid = min(GM_BM, a.count[e] - m0);
    p0 = a.offset[e] + m0;
  } else {
    p0 = tile * GM_BM;
    valid = min(GM_BM, a.T - p0);
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, ln = lane & 31;
  const int kdim = a.kdim;
  const int mt_valid = (valid + 31) >> 5;
  const uint16_t* arow;
  {
    const int64_t lda = a.lda ? a.lda : kdim;
    const int r0 = wv * 32 + ln;
    const int rr = r0 < valid ? r0 : 0;                  // rows past the tile reload row 0 (outputs dropped)
    if (ROUTED && MODE == GEMM_GATEUP) arow = a.a + static_cast<int64_t>(a.perm[p0 + rr] / a.K) * lda;
    else arow = a.a + static_cast<int64_t>(p0 + rr) * lda;
    arow += static_cast<int64_t>(split) * kdim;
  }
  int brow[2];
  bool bvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (MODE == GEMM_GATEUP) {
      const int j = nblk * 128 + wv * 32 + ln;
      bvalid[nt] = j < a.half_n;
      const int jj = bvalid[nt] ? j : 0;
      brow[nt] = nt == 0 ? jj : a.half_n + jj;
    } else {
      const int n = nblk * 256 + wv * 64 + nt * 32 + ln;
      bvalid[nt] = n < a.half_n;
      brow[nt] = bvalid[nt] ? n : 0;
    }
  }
  const uint8_t* bq = NVFP4 ? a.bq + e * a.stride_q : nullptr;
  const uint8_t* bs = NVFP4 ? a.bs + e * a.stride_s : nullptr;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mt][nt][j] = 0.0f;
  if constexpr (NVFP4) {
    __shared__ uint4 A0[1024], A1[1024], A2[1024];
    __shared__ uint4 C0[512], C1[512], C2[512];
    __shared__ uint32_t S0[512], S1[512], S2[512];
    switch (mt_valid) {
      case 1: gemm_dma_mainloop<1>(A0, A1, A2, C0, C1, C2, S0, S1, S2, arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
      case 2: gemm_dma_mainloop<2>(A0, A1, A2, C0, C1, C2, S0, S1, S2, arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
      case 3: gemm_dma_mainloop<3>(A0, A1, A2, C0, C1, C2, S0, S1, S2, arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
      default: gemm_dma_mainloop<4>(A0, A1, A2, C0, C1, C2, S0, S1, S2, arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
    }
  } else {
  GemmArgs as = a;
  as.bb += static_cast<int64_t>(split) * kdim;
  __shared__ uint4 L0[1024];
  __shared__ uint4 L1[1024];
  __shared__ uint4 L2[NST > 2 ? 1024 : 1];
  __shared__ uint4 L3[NST > 3 ? 1024 : 1];
  switch (mt_valid) {
    case 1: gemm_fast_mainloop<NVFP4, NST, 1>(as, L0, L1, *reinterpret_cast<uint4(*)[1024]>(&L2[0]), *reinterpret_cast<uint4(*)[1024]>(&L3[0]), arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
    case 2: gemm_fast_mainloop<NVFP4, NST, 2>(as, L0, L1, *reinterpret_cast<uint4(*)[1024]>(&L2[0]), *reinterpret_cast<uint4(*)[1024]>(&L3[0]), arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
    case 3: gemm_fast_mainloop<NVFP4, NST, 3>(as, L0, L1, *reinterpret_cast<uint4(*)[1024]>(&L2[0]), *reinterpret_cast<uint4(*)[1024]>(&L3[0]), arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
    default: gemm_fast_mainloop<NVFP4, NST, 4>(as, L0, L1, *reinterpret_cast<uint4(*)[1024]>(&L2[0]), *reinterpret_cast<uint4(*)[1024]>(&L3[0]), arow, bq, bs, brow, wv, lane, g, kdim, acc); break;
  }
  }
  float g0 = 1.0f, g1 = 1.0f;
  if (ROUTED && a.gscale) {
    if (MODE == GEMM_GATEUP) {
      g0 = a.gscale[2 * e];
      g1 = a.gscale[2 * e + 1];
    } else {
      g0 = a.gscale[e];
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt >= mt_valid) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = mt * 32 + c32_row(lane, j);
      if (row >= valid) continue;
      if (MODE == GEMM_GATEUP) {
        if (!bvalid[0]) continue;
        const int jc = nblk * 128 + wv * 32 + ln;
        static_cast<uint16_t*>(a.out)[static_cast<int64_t>(p0 + row) * a.ldo + jc] =
            f32_to_bf16(swiglu_clamped(g0 * acc[mt][0][j], g1 * acc[mt][1][j], a.limit));
      } else {
        const int64_t orow = (MODE == GEMM_DOWN_SLOT_F32) ? static_cast<int64_t>(a.perm[p0 + row])
                                                          : static_cast<int64_t>(p0 + row);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if (!bvalid[nt]) continue;
          const int n = nblk * 256 + wv * 64 + nt * 32 + ln;
          if (MODE == GEMM_DOWN_BF16)
            static_cast<uint16_t*>(a.out)[orow * a.ldo + n] = f32_to_bf16(acc[mt][nt][j]);
          else
            static_cast<float*>(a.out)[split * a.split_out + orow * a.ldo + n] = g0 * acc[mt][nt][j];
        }
      }
    }
  }
}

// NVFP4 -> fp32 / bf16 dequantisation, through the same device routines as
// the GEMV and GEMM: one thread per 32 columns of a row.
__global__ __launch_bounds__(256) void k_nvfp4_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                       float global, int64_t rows, int cols,
                                                       float* out_f32, uint16_t* out_bf16) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int nch = cols >> 5;
  if (idx >= rows * nch) return;
  const int64_t r = idx / nch;
  const int c = static_cast<int>(idx - r * nch);
  const uint4 cw = *reinterpret_cast<const uint4*>(q + r * (cols >> 1) + 16 * c);
  const uint32_t sc = *reinterpret_cast<const uint16_t*>(s + r * (cols >> 4) + 2 * c);
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float scale = (w < 2 ? e4m3_to_f32<0>(sc) : e4m3_to_f32<1>(sc)) * global;
    const int64_t o = r * cols + 32 * c + 8 * w;
    if (out_bf16) {
      uint32_t p[4];
      e2m1x8_scaled_bf16(words[w], scale, p);
      *reinterpret_cast<uint4*>(out_bf16 + o) = make_uint4(p[0], p[1], p[2], p[3]);
    }
    if (out_f32) {
      const f32x2 v0 = e2m1x2_to_f32<0>(words[w]), v1 = e2m1x2_to_f32<1>(words[w]);
      const f32x2 v2 = e2m1x2_to_f32<2>(words[w]), v3 = e2m1x2_to_f32<3>(words[w]);
      float4* of = reinterpret_cast<float4*>(out_f32 + o);
      of[0] = make_float4(v0.x * scale, v0.y * scale, v1.x * scale, v1.y * scale);
      of[1] = make_float4(v2.x * scale, v2.y * scale, v3.x * scale, v3.y * scale);
    }
  }
}

}  // namespace moe
