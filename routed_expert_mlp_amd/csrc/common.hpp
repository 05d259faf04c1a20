// Device helpers shared by the routed MoE MLP kernels (gfx950 / CDNA4).
//
// Number formats follow the OCP Microscaling Formats v1.0 (FP4 E2M1) and OCP
// OFP8 (E4M3 "fn") specifications; NVFP4 = E2M1 codes with one E4M3 scale per
// 16 consecutive elements of a row.
//
// gfx950 facts the dequantisation relies on (checked on the device against
// the OCP definitions):
//   * v_cvt_scalef32_pk_{f32,bf16}_fp4 decode two E2M1 codes of one byte
//     exactly; its fp32 scale operand contributes only its exponent, so the
//     E4M3 block scale (which has a mantissa) is applied by a separate fp32
//     multiply or fma.
//   * v_cvt_f32_fp8 decodes OCP E4M3 ("fn": 0x7E = 448, 0x7F = NaN,
//     subnormals), so it decodes the block scales directly.
//   * e2m1 (<= 2 significant bits) x e4m3 (<= 4) has <= 6 significant bits,
//     so a dequantised weight is exact in fp32 and in bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed bf16x2 bits (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3 byte `sel` (0..3) of a 32-bit word -> fp32.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), SEL);
}

// Byte SEL of `codes` (two E2M1 codes: low nibble = even element) -> bf16 pair.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, SEL);
}

// Byte SEL of `codes` -> fp32 pair (exact E2M1 values).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum of 16 E2M1 codes (two 32-bit words, element order = nibble order) times
// 16 bf16 activations (8 packed pairs), accumulated in fp32 from 0.
__device__ __forceinline__ float e2m1x16_dot(uint32_t c0, uint32_t c1, const uint32_t* xp) {
  float s = 0.0f;
  s = dot2_bf16(e2m1x2_to_bf16<0>(c0), xp[0], s);
  s = dot2_bf16(e2m1x2_to_bf16<1>(c0), xp[1], s);
  s = dot2_bf16(e2m1x2_to_bf16<2>(c0), xp[2], s);
  s = dot2_bf16(e2m1x2_to_bf16<3>(c0), xp[3], s);
  s = dot2_bf16(e2m1x2_to_bf16<0>(c1), xp[4], s);
  s = dot2_bf16(e2m1x2_to_bf16<1>(c1), xp[5], s);
  s = dot2_bf16(e2m1x2_to_bf16<2>(c1), xp[6], s);
  s = dot2_bf16(e2m1x2_to_bf16<3>(c1), xp[7], s);
  return s;
}

// Eight E2M1 codes (one 32-bit word) times one fp32 scale -> 8 bf16 packed
// in 4 words, element order kept.  Exact (see the header comment).
__device__ __forceinline__ void e2m1x8_scaled_bf16(uint32_t codes, float scale, uint32_t* out4) {
  f32x2 a = e2m1x2_to_f32<0>(codes);
  f32x2 b = e2m1x2_to_f32<1>(codes);
  f32x2 c = e2m1x2_to_f32<2>(codes);
  f32x2 d = e2m1x2_to_f32<3>(codes);
  out4[0] = pack_bf16x2(a.x * scale, a.y * scale);
  out4[1] = pack_bf16x2(b.x * scale, b.y * scale);
  out4[2] = pack_bf16x2(c.x * scale, c.y * scale);
  out4[3] = pack_bf16x2(d.x * scale, d.y * scale);
}

// Lane permutes within rows of 16 lanes (DPP): a few cycles each, unlike
// __shfl_xor, which goes through the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_QUAD_1032 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// Keep (v, i, a) of the larger v; on equal v the smaller i.
__device__ __forceinline__ void argmax_take(float& v, int& i, float& a, float ov, int oi, float oa) {
  const bool take = (ov > v) || (ov == v && oi < i);
  v = take ? ov : v;
  i = take ? oi : i;
  a = take ? oa : a;
}

template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(float& v, int& i, float& a) {
  const float ov = __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
  const int oi = dpp_mov<CTRL>(i);
  const float oa = __int_as_float(dpp_mov<CTRL>(__float_as_int(a)));
  argmax_take(v, i, a, ov, oi, oa);
}

// Wave-wide argmax of (v, i) (larger v, then smaller i), carrying a; every
// lane returns the winner.  All 64 lanes must be active.
__device__ __forceinline__ void wave_argmax(float& v, int& i, float& a) {
  argmax_dpp_step<DPP_QUAD_1032>(v, i, a);
  argmax_dpp_step<DPP_QUAD_2301>(v, i, a);
  argmax_dpp_step<DPP_ROW_HALF_MIRROR>(v, i, a);
  argmax_dpp_step<DPP_ROW_MIRROR>(v, i, a);      // every lane now holds its row's winner
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
  float ba = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0));
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int oi = __builtin_amdgcn_readlane(i, 16 * r);
    const float oa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16 * r));
    argmax_take(bv, bi, ba, ov, oi, oa);
  }
  v = bv;
  i = bi;
  a = ba;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
}

// Sum over the 64 lanes; every lane returns the same bits (each step adds a
// commutative pair).  All 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<DPP_QUAD_1032>(v);
  v = dpp_add<DPP_QUAD_2301>(v);
  v = dpp_add<DPP_ROW_HALF_MIRROR>(v);
  v = dpp_add<DPP_ROW_MIRROR>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// SiLU(min(g, L)) * clamp(u, -L, L): the asymmetric clamped SwiGLU.
__device__ __forceinline__ float swiglu_clamped(float g, float u, float L) {
  g = fminf(g, L);
  u = fminf(fmaxf(u, -L), L);
  return g / (1.0f + expf(-g)) * u;
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained).
// 16-byte position of code piece q (0..3) of weight row p inside a 64-byte
// row unit of the NVFP4 tile layout: q ^ f4_swz_c(p).
__host__ __device__ __forceinline__ int f4_swz_c(int p) { return ((p >> 1) & 3) ^ ((p >> 3) & 1); }

// Byte offset of 16-byte code chunk c (columns 32c .. 32c+31) of row R of an
// NVFP4 code matrix with `cols` columns.  Row-major: R * cols/2 + 16 c.  Tile
// layout (moe_nvfp4_tile_pack; rows % 32 == 0, cols % 256 == 0): 1 KB blocks
// of 16 rows x 128 columns, row-group major; inside a block row r's four
// pieces sit at 16 (4 r + (q ^ f4_swz_c(r))).
template <bool TILED>
__device__ __forceinline__ int64_t nvfp4_code_off(int64_t R, int c, int cols) {
  if (TILED)
    return ((R >> 4) * (cols >> 7) + (c >> 2)) * 1024 +
           16 * (4 * static_cast<int>(R & 15) + ((c & 3) ^ f4_swz_c(static_cast<int>(R & 15))));
  return R * (cols >> 1) + 16 * static_cast<int64_t>(c);
}

__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14);
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
