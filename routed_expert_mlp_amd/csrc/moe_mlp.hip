// C ABI of the routed MoE MLP library (declarations and contract in
// include/moe_mlp.h).  Host code: argument validation (before anything is
// enqueued), workspace layout, and the launch sequences of the decode and
// prefill forms.  The library allocates nothing, never synchronises, and
// keeps no state between calls.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "../../include/moe_mlp.h"
#include "common.hpp"
#include "decode1.hpp"
#include "gemm.hpp"
#include "gemm_bf16.hpp"
#include "gemm_fp4.hpp"
#include "gemv.hpp"
#include "permute.hpp"
#include "router.hpp"

static_assert(MOE_MLP_MAX_EXPERTS <= moe::PERM_MAX_E, "k_perm_hist keeps one LDS counter per expert");

namespace {

using namespace moe;

constexpr int64_t kMaxDim = 65536;

bool finite_pos(float v) { return std::isfinite(v) && v > 0.0f; }
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool bad_dim(int64_t d) { return d <= 0 || d % 32 != 0 || d > kMaxDim; }

int validate_cfg(const moe_mlp_config* c, int64_t T, int prefill) {
  if (!c) return MOE_MLP_ERR_NULL_ARG;
  if (c->kind != MOE_MLP_KIND_ROUTED && c->kind != MOE_MLP_KIND_DENSE) return MOE_MLP_ERR_BAD_VALUE;
  if (T < 0 || (!prefill && T > MOE_MLP_DECODE_MAX_T)) return MOE_MLP_ERR_BAD_SHAPE;
  if (bad_dim(c->hidden)) return MOE_MLP_ERR_BAD_SHAPE;
  if (!finite_pos(c->swiglu_limit)) return MOE_MLP_ERR_BAD_VALUE;
  if (c->kind == MOE_MLP_KIND_DENSE) {
    if (bad_dim(c->dense_intermediate)) return MOE_MLP_ERR_BAD_SHAPE;
    return MOE_MLP_OK;
  }
  if (bad_dim(c->moe_intermediate)) return MOE_MLP_ERR_BAD_SHAPE;
  if (c->n_shared_experts != 0 && c->n_shared_experts != 1) return MOE_MLP_ERR_BAD_VALUE;
  if (c->n_shared_experts == 1 && bad_dim(c->shared_intermediate)) return MOE_MLP_ERR_BAD_SHAPE;
  if (c->num_experts < 1 || c->num_experts > MOE_MLP_MAX_EXPERTS) return MOE_MLP_ERR_BAD_VALUE;
  if (!finite_pos(c->routed_scaling_factor)) return MOE_MLP_ERR_BAD_VALUE;
  if (c->top_k < 1 || c->top_k > MOE_MLP_MAX_TOP_K || c->top_k > c->num_experts) return MOE_MLP_ERR_BAD_TOPK;
  if (T * c->top_k >= (int64_t(1) << 31)) return MOE_MLP_ERR_BAD_SHAPE;
  return MOE_MLP_OK;
}

// Workspace regions, each 256-byte aligned.
struct Plan {
  size_t logits = 0, ids = 0, wts = 0;
  size_t g_n = 0, g_expert = 0, g_count = 0, g_offset = 0, g_slots = 0;          // decode groups
  size_t count = 0, offset = 0, perm = 0, n_tiles = 0, tile_e = 0, tile_m0 = 0;  // prefill permutation
  size_t phist = 0, pbase = 0, prank = 0;                                        // permutation scratch
  size_t h = 0, hs = 0, y = 0, ys = 0;
  size_t wsplit = 0;                                                             // router weight, 3 bf16 planes
  int logit_planes = 1;
  int logit_splits = 1;       // reduction parts of the split-weight logits GEMM
  size_t total = 0;
  int64_t max_tiles = 0;
};

struct Alloc {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t off = cur;
    cur += (bytes + 255) & ~size_t(255);
    return off;
  }
};

// The grouped-GEMM form runs prefill, and decode from this many tokens on
// (measured: the expert GEMVs re-stream each touched expert's rows once per
// pass of 4 of its tokens; the GEMM streams them once per 128-row tile and
// overtakes the GEMVs from T = 64, by 2.2x at T = 256).
constexpr int64_t kDecodeGemmMinT = 64;

int gemm_form(const moe_mlp_config* c, int64_t T, int prefill) {
  return (prefill || T >= kDecodeGemmMinT) ? 1 : 0;
}

// Prefill router logits on the matrix cores (split fp32 weight, see router.hpp)
// when there are enough tokens and the reduction length suits the fast GEMM.
bool mfma_logits(const moe_mlp_config* c, int64_t T, int prefill) {
  return prefill && T >= 64 && c->hidden % 64 == 0;
}

Plan make_plan(const moe_mlp_config* c, int64_t T, int prefill) {
  Plan p;
  Alloc a;
  if (c->kind == MOE_MLP_KIND_DENSE) {
    p.h = a.take(size_t(T) * c->dense_intermediate * 2);
    p.total = a.cur;
    return p;
  }
  const int64_t E = c->num_experts, K = c->top_k, H = c->hidden, I = c->moe_intermediate;
  const int64_t Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const int64_t S = T * K;
  if (mfma_logits(c, T, prefill)) {
    p.logit_planes = 3;
    p.wsplit = a.take(size_t(3 * E * H) * 2);
    // the logits GEMM has only ceil(T/128) x ceil(3E/256) output tiles: cut
    // its reduction into 4 parts when H allows, for 4x the workgroups
    if (H % 256 == 0) p.logit_splits = 4;
  }
  p.logits = a.take(size_t(T * E * p.logit_planes * p.logit_splits) * 4);
  p.ids = a.take(size_t(S) * 4);
  p.wts = a.take(size_t(S) * 4);
  if (prefill) {
    p.max_tiles = cdiv(S, GM_BM) + E;
    p.count = a.take(size_t(E) * 4);
    p.offset = a.take(size_t(E + 1) * 4);
    p.perm = a.take(size_t(S) * 4);
    p.n_tiles = a.take(4);
    p.tile_e = a.take(size_t(p.max_tiles) * 4);
    p.tile_m0 = a.take(size_t(p.max_tiles) * 4);
    p.phist = a.take(size_t(cdiv(S, PERM_CHUNK)) * E * 4);
    p.pbase = a.take(size_t(cdiv(S, PERM_CHUNK)) * E * 4);
    p.prank = a.take(size_t(S) * 4);
  } else {
    p.g_n = a.take(4);
    p.g_expert = a.take(size_t(E) * 4);
    p.g_count = a.take(size_t(E) * 4);
    p.g_offset = a.take(size_t(E) * 4);
    p.g_slots = a.take(size_t(S) * 4);
  }
  p.h = a.take(size_t(S * I) * 2);
  if (Is) {
    p.hs = a.take(size_t(T * Is) * 2);
    p.ys = a.take(size_t(T * H) * 4);
  }
  p.y = a.take(size_t(S * H) * 4);
  p.total = a.cur;
  return p;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

int validate_weights(const moe_mlp_config* c, const moe_mlp_weights* w) {
  if (!w) return MOE_MLP_ERR_NULL_ARG;
  const void* need[12];
  int n = 0;
  if (c->kind == MOE_MLP_KIND_DENSE) {
    need[n++] = w->dense_w13;
    need[n++] = w->dense_w2;
  } else {
    need[n++] = w->router_w;
    need[n++] = w->router_bias;
    need[n++] = w->w13_q;
    need[n++] = w->w13_s;
    need[n++] = w->w13_g;
    need[n++] = w->w2_q;
    need[n++] = w->w2_s;
    need[n++] = w->w2_g;
    if (c->n_shared_experts) {
      need[n++] = w->shared_w13;
      need[n++] = w->shared_w2;
    }
  }
  for (int i = 0; i < n; ++i)
    if (!need[i]) return MOE_MLP_ERR_KIND_MISMATCH;
  for (int i = 0; i < n; ++i)
    if (!aligned(need[i])) return MOE_MLP_ERR_MISALIGNED;
  if (c->kind == MOE_MLP_KIND_ROUTED) {   // the optional tile-layout copies
    const void* opt[4] = {w->w13_q_tiled, w->w13_s_tiled, w->w2_q_tiled, w->w2_s_tiled};
    for (const void* q : opt)
      if (q && !aligned(q)) return MOE_MLP_ERR_MISALIGNED;
  }
  return MOE_MLP_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_MLP_OK : MOE_MLP_ERR_HIP; }

// Stage timing: a stage's start event is attached to its first kernel's
// dispatch packet and its stop event to its last (hipExtLaunchKernelGGL), so
// the interval is the kernels' own execution, as a kernel trace reports it.
// Null events give an ordinary launch.
struct Ev {
  hipEvent_t a = nullptr, b = nullptr;
};

template <typename F, typename... Args>
void launch(F kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1, Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
}

// Calls f(std::integral_constant<int, NJ>) with the smallest supported NJ >= E / 64
// (the per-lane candidate count of the top-k wavefront).
template <typename F>
void with_nj(int E, F&& f) {
  switch (static_cast<int>(cdiv(E, 64))) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: case 8: f(std::integral_constant<int, 8>{}); break;
    case 9: case 10: case 11: case 12: f(std::integral_constant<int, 12>{}); break;
    default: f(std::integral_constant<int, 16>{}); break;
  }
}

void topk_bucket(int E, const float* logits, const float* bias, int T, int K, float rsf, int32_t* ids,
                 float* wts, int32_t* ids_out, float* w_out, Groups g, hipStream_t s, Ev ev) {
  with_nj(E, [&](auto nj) {
    launch(k_topk_bucket<decltype(nj)::value>, dim3(1), dim3(1024), s, ev.a, ev.b, logits, bias, T, E, K, rsf,
           ids, wts, ids_out, w_out, g);
  });
}

void topk_tokens(int E, const float* logits, const float* bias, int T, int K, float rsf, int32_t* ids,
                 float* wts, int32_t* ids_out, float* w_out, hipStream_t s, Ev ev, int planes = 1, int splits = 1) {
  with_nj(E, [&](auto nj) {
    launch(k_topk<decltype(nj)::value>, dim3(static_cast<unsigned>(cdiv(T, 4))), dim3(256), s, ev.a, ev.b, logits,
           bias, T, E, K, rsf, ids, wts, ids_out, w_out, planes, splits);
  });
}

void router_logits(const uint16_t* x, const float* wr, float* logits, int64_t T, int H, int E, hipStream_t s,
                   Ev ev) {
  // one workgroup per expert row up to the decode limit (the tile GEMM below
  // has only ceil(T/64) x ceil(E/64) workgroups, too few for small T)
  if (T <= MOE_MLP_DECODE_MAX_T) {
    launch(k_logits_gemv, dim3(E), dim3(256), s, ev.a, ev.b, x, wr, logits, static_cast<int>(T), H, E);
  } else {
    const dim3 grid(static_cast<unsigned>(cdiv(T, 64)), static_cast<unsigned>(cdiv(E, 64)));
    launch(k_logits_gemm, grid, dim3(256), s, ev.a, ev.b, x, wr, logits, static_cast<int>(T), H, E);
  }
}

// BF16 rows of up to 8 chunks per lane (the shared expert and dense FFN) take
// the all-loads-first kernel (NC = chunks per lane).  The routed NVFP4 GEMVs
// keep the looping kernel: they run thousands of blocks and hide latency by
// occupancy, and holding their chunks (with 16 activation words per chunk
// and token) costs more registers than it saves in waits (measured).
template <bool NVFP4, int MODE, int RW>
void gemv(const GemvArgs& a, int groups, hipStream_t s, Ev ev) {
  const dim3 grid(static_cast<unsigned>(cdiv(a.half_rows, 4 * RW)), static_cast<unsigned>(groups));
  const int nch = NVFP4 ? (a.cols >> 5) : (a.cols >> 3);
  if constexpr (NVFP4) {
    launch(k_gemv<NVFP4, MODE, RW, 0>, grid, dim3(256), s, ev.a, ev.b, a);
    return;
  } else {
  switch (static_cast<int>(cdiv(nch, 64))) {
    case 1: launch(k_gemv<NVFP4, MODE, RW, 1>, grid, dim3(256), s, ev.a, ev.b, a); break;
    case 2: launch(k_gemv<NVFP4, MODE, RW, 2>, grid, dim3(256), s, ev.a, ev.b, a); break;
    case 3: launch(k_gemv<NVFP4, MODE, RW, 3>, grid, dim3(256), s, ev.a, ev.b, a); break;
    case 4: launch(k_gemv<NVFP4, MODE, RW, 4>, grid, dim3(256), s, ev.a, ev.b, a); break;
    case 5: case 6: launch(k_gemv<NVFP4, MODE, RW, 6>, grid, dim3(256), s, ev.a, ev.b, a); break;
    case 7: case 8: launch(k_gemv<NVFP4, MODE, RW, 8>, grid, dim3(256), s, ev.a, ev.b, a); break;
    default: launch(k_gemv<NVFP4, MODE, RW, 0>, grid, dim3(256), s, ev.a, ev.b, a); break;
  }
  }
}

// Routed NVFP4 projections with a reduction length that is a multiple of 256
// and at least 512 take k_gemm_nvfp4, BF16 projections (shared expert, dense
// FFN, router logits) with a reduction length that is a multiple of 128 take
// k_gemm_bf16; other reduction lengths that are a multiple of 64 the
// 32x32x16-MFMA kernel (k_gemm_fast); the rest the general 16x16x32 kernel.
template <bool NVFP4, int MODE, bool ROUTED>
void gemm(const GemmArgs& a0, int64_t m_tiles, hipStream_t s, Ev ev) {
  GemmArgs a = a0;
  if constexpr (NVFP4 && ROUTED && (MODE == GEMM_GATEUP || MODE == GEMM_DOWN_SLOT_F32)) {
    // its DMA offsets are 32-bit: activation rows (T here) and weight rows
    // times the row length must stay below 2^31 bytes
    const int64_t w_rows = MODE == GEMM_GATEUP ? 2 * int64_t(a.half_n) : int64_t(a.half_n);
    if (a.kdim % 256 == 0 && a.kdim >= 512 && int64_t(a.T) * a.kdim * 2 < (int64_t(1) << 31) &&
        w_rows * a.kdim / 2 < (int64_t(1) << 31)) {
      a.n_blocks = static_cast<int>(cdiv(a.half_n, MODE == GEMM_GATEUP ? F4_WROWS / 2 : F4_WROWS));
      const dim3 grid(static_cast<unsigned>(8 * cdiv(m_tiles * a.n_blocks, 8)));
      if (a.bq_t && a.bs_t)
        launch(k_gemm_nvfp4<MODE, true>, grid, dim3(F4_THREADS), s, ev.a, ev.b, a);
      else
        launch(k_gemm_nvfp4<MODE, false>, grid, dim3(F4_THREADS), s, ev.a, ev.b, a);
      return;
    }
  }
  if constexpr (!NVFP4 && !ROUTED) {
    // 32-bit DMA offsets: rows times row stride (in bytes) below 2^31
    const int64_t lda = a.lda ? a.lda : a.kdim, ldb = a.ldb ? a.ldb : a.kdim;
    const int64_t w_rows = MODE == GEMM_GATEUP ? 2 * int64_t(a.half_n) : int64_t(a.half_n);
    if (a.kdim % 128 == 0 && int64_t(a.T) * lda * 2 < (int64_t(1) << 31) && w_rows * ldb * 2 < (int64_t(1) << 31)) {
      a.n_blocks = static_cast<int>(cdiv(a.half_n, MODE == GEMM_GATEUP ? B16_BN / 2 : B16_BN));
      const int64_t work = cdiv(a.T, B16_BM) * a.n_blocks * (a.ksplit > 1 ? a.ksplit : 1);
      launch(k_gemm_bf16<MODE>, dim3(static_cast<unsigned>(8 * cdiv(work, 8))), dim3(B16_THREADS), s, ev.a, ev.b, a);
      return;
    }
  }
  if (a.kdim % 64 == 0) {
    a.n_blocks = static_cast<int>(cdiv(a.half_n, MODE == GEMM_GATEUP ? 128 : 256));
    const int64_t work = m_tiles * a.n_blocks * (a.ksplit > 1 ? a.ksplit : 1);
    const dim3 grid(static_cast<unsigned>(8 * cdiv(work, 8)));
    constexpr int NST = NVFP4 ? 4 : 3;
    launch(k_gemm_fast<NVFP4, MODE, ROUTED, NST>, grid, dim3(256), s, ev.a, ev.b, a);
  } else {
    const int nb = MODE == GEMM_GATEUP ? 128 : 256;
    const dim3 grid(static_cast<unsigned>(m_tiles), static_cast<unsigned>(cdiv(a.half_n, nb)));
    launch(k_gemm<NVFP4, MODE, ROUTED>, grid, dim3(256), s, ev.a, ev.b, a);
  }
}

GemvArgs bf16_gemv_args(const uint16_t* w, int half_rows, int cols, int T, const uint16_t* in, void* out,
                        float limit) {
  GemvArgs a{};
  a.wb = w;
  a.half_rows = half_rows;
  a.cols = cols;
  a.T = T;
  a.K = 1;
  a.in = in;
  a.out = out;
  a.limit = limit;
  return a;
}

GemmArgs bf16_gemm_args(const uint16_t* act, int kdim, const uint16_t* w, int half_n, int T, void* out, int ldo,
                        float limit) {
  GemmArgs a{};
  a.a = act;
  a.kdim = kdim;
  a.bb = w;
  a.half_n = half_n;
  a.T = T;
  a.K = 1;
  a.out = out;
  a.ldo = ldo;
  a.limit = limit;
  return a;
}

// Router logits [T][3][E] against the three bf16 parts of the router weight
// (k_split_bf16x3 into the workspace, then the bf16 MFMA GEMM over the stacked
// [3E, H] parts); the top-k adds the parts.  Plain fp32 otherwise.
void router_logits_plan(const Plan& p, void* ws, const uint16_t* x, const float* wr, float* logits, int64_t T,
                        int H, int E, hipStream_t s, Ev ev) {
  if (p.logit_planes == 1) {
    router_logits(x, wr, logits, T, H, E, s, ev);
    return;
  }
  uint16_t* planes = at<uint16_t>(ws, p.wsplit);
  const int64_t n = static_cast<int64_t>(E) * H;
  launch(k_split_bf16x3, dim3(static_cast<unsigned>(cdiv(n / 8, 256))), dim3(256), s, ev.a, nullptr, wr, planes, n);
  GemmArgs ga = bf16_gemm_args(x, H / p.logit_splits, planes, 3 * E, static_cast<int>(T), logits, 3 * E, 1.0f);
  ga.lda = H;
  ga.ldb = H;
  ga.ksplit = p.logit_splits;
  ga.split_out = T * 3 * E;
  gemm<false, GEMM_DOWN_F32, false>(ga, cdiv(T, GM_BM), s, Ev{nullptr, ev.b});
}

const char* const kDecodeStages[] = {"router_logits", "topk_bucket", "shared_gateup", "routed_gateup",
                                    "shared_down", "routed_down", "combine"};
const char* const kDecode1Stages[] = {"logits_shared_gateup", "routed_gateup_shared_down",
                                       "routed_down_combine"};
const char* const kPrefillStages[] = {"router_logits", "topk", "permute", "routed_gateup", "routed_down",
                                     "shared_gateup", "shared_down", "combine"};
const char* const kDenseStages[] = {"dense_gateup", "dense_down"};

// The one-token decode kernels hold a row's chunks in registers: they take
// H <= 4096 and I, Is <= 2048.
constexpr int kDec1MaxH = 4096;

int dec1_kw(int K) { return K <= 4 ? 4 : K <= 8 ? 8 : 16; }

// The few-token decode kernels (decode1.hpp) take up to 4 tokens (the MTP
// verify shapes: one token plus up to three drafted ones), T*K <= 64 slots.
constexpr int64_t kDecFewMaxT = 4;

bool decode1_ok(const moe_mlp_config* c, int64_t T, int prefill) {
  if (prefill || T < 1 || T > kDecFewMaxT || c->kind != MOE_MLP_KIND_ROUTED) return false;
  if (T * c->top_k > 64) return false;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  return c->hidden <= kDec1MaxH && c->moe_intermediate <= 2048 && Is <= 2048;
}

int n_stages(const moe_mlp_config* c, int64_t T, int prefill) {
  if (c->kind == MOE_MLP_KIND_DENSE) return 2;
  if (decode1_ok(c, T, prefill)) return 3;
  return gemm_form(c, T, prefill) ? 8 : 7;
}

// Few-token decode (1..4 tokens): 3 launches (see decode1.hpp).
template <int NSC>
void dec_gateup(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, const float* logits,
                int32_t* ids, float* wts, int32_t* ids_out, float* w_out, uint16_t* h, const uint16_t* hs,
                float* ys, int T, hipStream_t s, Ev ev) {
  constexpr int RJ = 4, NC = 2, RS = 8;
  const int H = c->hidden, I = c->moe_intermediate, K = c->top_k;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const int n_sd = Is ? static_cast<int>(cdiv(H, 4 * RS)) : 0;
  const unsigned grid = static_cast<unsigned>(n_sd + T * K * cdiv(I, 4 * RJ));
  with_nj(c->num_experts, [&](auto nj) {
    launch(k_dec_gateup<RJ, NC, decltype(nj)::value, RS, NSC>, dim3(grid), dim3(256), s, ev.a, ev.b, x, w->w13_q,
           w->w13_s, w->w13_g, logits, w->router_bias, K, c->routed_scaling_factor, ids, wts, ids_out, w_out,
           c->num_experts, H, I, c->swiglu_limit, h, w->shared_w2, hs, Is, ys, n_sd, T);
  });
}

template <int KW, int NP>
void launch_down_combine(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* h, const float* ys,
                         const int32_t* ids, const float* wts, uint16_t* out, int T, hipStream_t s, Ev ev) {
  constexpr int R = 4;
  const int H = c->hidden;
  launch(k_dec_down_combine<R, KW, NP>, dim3(static_cast<unsigned>(cdiv(H, R))), dim3(KW * 64), s, ev.a, ev.b, h,
         w->w2_q, w->w2_s, w->w2_g, ys, ids, wts, c->num_experts, c->top_k, H, c->moe_intermediate, out, T);
}

void decode1(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, int T, uint16_t* out,
             int32_t* ids_out, float* w_out, float* logits, int32_t* ids, float* wts, uint16_t* h, uint16_t* hs,
             float* ys, hipStream_t s, Ev e0, Ev e1, Ev e2) {
  const int H = c->hidden, E = c->num_experts, K = c->top_k;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const int nlb = static_cast<int>(cdiv(E, 4)), nsb = static_cast<int>(cdiv(Is, 4));
  if (T == 1)
    launch(k_dec_logits_shared<16, 8>, dim3(nlb + nsb), dim3(256), s, e0.a, e0.b, x, w->router_w, logits, E, H,
           w->shared_w13, Is, hs, c->swiglu_limit, nlb);
  else
    launch(k_dec_logits_shared_t<16, 8>, dim3(nlb + nsb), dim3(256), s, e0.a, e0.b, x, w->router_w, logits, E, H,
           w->shared_w13, Is, hs, c->swiglu_limit, nlb, T);
  const int nsc = static_cast<int>(cdiv(Is / 8, 64));
  if (nsc <= 1) dec_gateup<1>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, ys, T, s, e1);
  else if (nsc == 2) dec_gateup<2>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, ys, T, s, e1);
  else if (nsc == 3) dec_gateup<3>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, ys, T, s, e1);
  else dec_gateup<4>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, ys, T, s, e1);
  const float* ysr = Is ? ys : nullptr;
  // one wavefront per slot at one token (K <= 16), else 16 wavefronts looping over the T*K slots
  const int S = T * K;
  if (T == 1 && dec1_kw(K) == 4) launch_down_combine<4, 1>(c, w, h, ysr, ids, wts, out, T, s, e2);
  else if (T == 1 && dec1_kw(K) == 8) launch_down_combine<8, 1>(c, w, h, ysr, ids, wts, out, T, s, e2);
  else if (S <= 16) launch_down_combine<16, 1>(c, w, h, ysr, ids, wts, out, T, s, e2);
  else if (S <= 32) launch_down_combine<16, 2>(c, w, h, ysr, ids, wts, out, T, s, e2);
  else if (S <= 48) launch_down_combine<16, 3>(c, w, h, ysr, ids, wts, out, T, s, e2);
  else launch_down_combine<16, 4>(c, w, h, ysr, ids, wts, out, T, s, e2);
}

int run_layer(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, int64_t T, uint16_t* out,
              int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes, void* stream, int prefill,
              void* const* events = nullptr, int n_events = 0) {
  int st = validate_cfg(c, T, prefill);
  if (st) return st;
  if (events && n_events < 2 * n_stages(c, T, prefill)) return MOE_MLP_ERR_BAD_VALUE;
  if (T == 0) return MOE_MLP_OK;
  if ((st = validate_weights(c, w))) return st;
  if (!x || !out || !ws) return MOE_MLP_ERR_NULL_ARG;
  if (!aligned(x) || !aligned(out) || !aligned(ws)) return MOE_MLP_ERR_MISALIGNED;
  if (c->kind == MOE_MLP_KIND_ROUTED && ((ids_out && !aligned(ids_out)) || (w_out && !aligned(w_out))))
    return MOE_MLP_ERR_MISALIGNED;
  if (!decode1_ok(c, T, prefill)) prefill = gemm_form(c, T, prefill);   // from here on: the form that runs
  const Plan p = make_plan(c, T, prefill);
  if (ws_bytes < p.total) return MOE_MLP_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = c->hidden;
  const float L = c->swiglu_limit;
  const int Ti = static_cast<int>(T);
  // Stage i's (start, stop) events, or none.
  auto ev = [&](int i) {
    Ev e;
    if (events) {
      e.a = static_cast<hipEvent_t>(events[2 * i]);
      e.b = static_cast<hipEvent_t>(events[2 * i + 1]);
    }
    return e;
  };
  auto empty_stage = [&](Ev e) {   // nothing to run: a zero-length interval
    if (e.a) {
      (void)hipEventRecord(e.a, s);
      (void)hipEventRecord(e.b, s);
    }
  };

  if (c->kind == MOE_MLP_KIND_DENSE) {
    const int Id = c->dense_intermediate;
    uint16_t* h = at<uint16_t>(ws, p.h);
    if (prefill) {
      const int64_t mt = cdiv(T, GM_BM);
      gemm<false, GEMM_GATEUP, false>(bf16_gemm_args(x, H, w->dense_w13, Id, Ti, h, Id, L), mt, s, ev(0));
      gemm<false, GEMM_DOWN_BF16, false>(bf16_gemm_args(h, Id, w->dense_w2, H, Ti, out, H, L), mt, s, ev(1));
    } else {
      gemv<false, GEMV_GATEUP, 2>(bf16_gemv_args(w->dense_w13, Id, H, Ti, x, h, L), 1, s, ev(0));
      gemv<false, GEMV_DOWN_BF16, 2>(bf16_gemv_args(w->dense_w2, H, Id, Ti, h, out, L), 1, s, ev(1));
    }
    return launch_status();
  }

  const int E = c->num_experts, K = c->top_k, I = c->moe_intermediate;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  float* logits = at<float>(ws, p.logits);
  int32_t* ids = at<int32_t>(ws, p.ids);
  float* wts = at<float>(ws, p.wts);
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* y = at<float>(ws, p.y);
  uint16_t* hs = Is ? at<uint16_t>(ws, p.hs) : nullptr;
  float* ys = Is ? at<float>(ws, p.ys) : nullptr;
  const int64_t S = T * K;
  const float rsf = c->routed_scaling_factor;

  if (decode1_ok(c, T, prefill)) {
    decode1(c, w, x, Ti, out, ids_out, w_out, logits, ids, wts, h, hs, ys, s, ev(0), ev(1), ev(2));
    return launch_status();
  }
  // decode of up to 16 tokens with H <= 4096: router logits and the shared
  // expert's gate/up share one launch (stage router_logits; shared_gateup
  // then records an empty stage)
  const bool fused_k1 = !prefill && T <= 16 && H <= kDec1MaxH && Is <= 2048;
  if (fused_k1) {
    const int nlb = static_cast<int>(cdiv(E, 4)), nsb = static_cast<int>(cdiv(Is, 4));
    launch(k_dec_logits_shared_t<16, 8>, dim3(nlb + nsb), dim3(256), s, ev(0).a, ev(0).b, x, w->router_w, logits,
           E, H, w->shared_w13, Is, hs, L, nlb, Ti);
  } else {
    router_logits_plan(p, ws, x, w->router_w, logits, T, H, E, s, ev(0));
  }
  if (prefill) {
    topk_tokens(E, logits, w->router_bias, Ti, K, rsf, ids, wts, ids_out, w_out, s, ev(1), p.logit_planes,
                p.logit_splits);
    Perm pm{at<int32_t>(ws, p.count), at<int32_t>(ws, p.offset), at<int32_t>(ws, p.perm),
            at<int32_t>(ws, p.n_tiles), at<int32_t>(ws, p.tile_e), at<int32_t>(ws, p.tile_m0)};
    const Ev pe = ev(2);
    const int nchunk = static_cast<int>(cdiv(S, PERM_CHUNK));
    int32_t* phist = at<int32_t>(ws, p.phist);
    int32_t* prank = at<int32_t>(ws, p.prank);
    launch(k_perm_hist, dim3(nchunk), dim3(PERM_CHUNK), s, pe.a, nullptr, ids, static_cast<int>(S), E, phist, prank);
    int32_t* pbase = at<int32_t>(ws, p.pbase);
    launch(k_perm_schedule, dim3(1), dim3(1024), s, nullptr, nullptr, E, nchunk, GM_BM, phist, pbase, pm);
    launch(k_perm_scatter, dim3(static_cast<unsigned>(cdiv(S, 256))), dim3(256), s, nullptr, pe.b, ids,
           static_cast<int>(S), E, pbase, prank, pm);
    GemmArgs g{};
    g.n_tiles = pm.n_tiles;
    g.tile_expert = pm.tile_expert;
    g.tile_m0 = pm.tile_m0;
    g.count = pm.count;
    g.offset = pm.offset;
    g.perm = pm.perm;
    g.K = K;
    g.limit = L;
    // routed gate/up + SwiGLU -> h (expert-sorted rows)
    GemmArgs gu = g;
    gu.a = x;
    gu.kdim = H;
    gu.bq = w->w13_q;
    gu.bs = w->w13_s;
    if (w->w13_q_tiled && w->w13_s_tiled) {
      gu.bq_t = w->w13_q_tiled;
      gu.bs_t = w->w13_s_tiled;
    }
    gu.stride_q = int64_t(2) * I * H / 2;
    gu.stride_s = int64_t(2) * I * H / 16;
    gu.gscale = w->w13_g;
    gu.half_n = I;
    gu.T = static_cast<int>(T);              // activation rows (tokens)
    gu.out = h;
    gu.ldo = I;
    gemm<true, GEMM_GATEUP, true>(gu, p.max_tiles, s, ev(3));
    // routed down -> y (slot rows)
    GemmArgs gd = g;
    gd.a = h;
    gd.kdim = I;
    gd.bq = w->w2_q;
    gd.bs = w->w2_s;
    if (w->w2_q_tiled && w->w2_s_tiled) {
      gd.bq_t = w->w2_q_tiled;
      gd.bs_t = w->w2_s_tiled;
    }
    gd.stride_q = int64_t(H) * I / 2;
    gd.stride_s = int64_t(H) * I / 16;
    gd.gscale = w->w2_g;
    gd.half_n = H;
    gd.T = static_cast<int>(S);              // activation rows (slots)
    gd.out = y;
    gd.ldo = H;
    gemm<true, GEMM_DOWN_SLOT_F32, true>(gd, p.max_tiles, s, ev(4));
    const int64_t mt = cdiv(T, GM_BM);
    if (Is) {
      gemm<false, GEMM_GATEUP, false>(bf16_gemm_args(x, H, w->shared_w13, Is, Ti, hs, Is, L), mt, s, ev(5));
      gemm<false, GEMM_DOWN_F32, false>(bf16_gemm_args(hs, Is, w->shared_w2, H, Ti, ys, H, L), mt, s, ev(6));
    } else {
      empty_stage(ev(5));
      empty_stage(ev(6));
    }
  } else {
    Groups gr{at<int32_t>(ws, p.g_n), at<int32_t>(ws, p.g_expert), at<int32_t>(ws, p.g_count),
              at<int32_t>(ws, p.g_offset), at<int32_t>(ws, p.g_slots)};
    topk_bucket(E, logits, w->router_bias, Ti, K, rsf, ids, wts, ids_out, w_out, gr, s, ev(1));
    const int groups = static_cast<int>(S < E ? S : E);
    if (Is && !fused_k1) gemv<false, GEMV_GATEUP, 1>(bf16_gemv_args(w->shared_w13, Is, H, Ti, x, hs, L), 1, s, ev(2));
    else empty_stage(ev(2));
    GemvArgs r{};
    r.n_groups = gr.n_groups;
    r.g_expert = gr.expert;
    r.g_count = gr.count;
    r.g_offset = gr.offset;
    r.g_slots = gr.slots;
    r.T = Ti;
    r.K = K;
    r.limit = L;
    GemvArgs gu = r;
    gu.wq = w->w13_q;
    gu.ws = w->w13_s;
    gu.stride_q = int64_t(2) * I * H / 2;
    gu.stride_s = int64_t(2) * I * H / 16;
    gu.gscale = w->w13_g;
    gu.half_rows = I;
    gu.cols = H;
    gu.in = x;
    gu.out = h;
    gemv<true, GEMV_GATEUP, 2>(gu, groups, s, ev(3));
    if (Is) gemv<false, GEMV_DOWN_F32, 2>(bf16_gemv_args(w->shared_w2, H, Is, Ti, hs, ys, L), 1, s, ev(4));
    else empty_stage(ev(4));
    GemvArgs gd = r;
    gd.wq = w->w2_q;
    gd.ws = w->w2_s;
    gd.stride_q = int64_t(H) * I / 2;
    gd.stride_s = int64_t(H) * I / 16;
    gd.gscale = w->w2_g;
    gd.half_rows = H;
    gd.cols = I;
    gd.in = h;
    gd.out = y;
    gemv<true, GEMV_DOWN_F32, 4>(gd, groups, s, ev(5));
  }
  const int64_t nq = T * (H / 4);
  const Ev ce = ev(prefill ? 7 : 6);
  const dim3 cgrid(static_cast<unsigned>(cdiv(nq, 256)));
  const float *yc = y, *ysc = ys, *wc = wts;
  if (K <= 4)
    launch(k_combine<4>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out);
  else if (K <= 8)
    launch(k_combine<8>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out);
  else
    launch(k_combine<MOE_MLP_MAX_TOP_K>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out);
  return launch_status();
}

}  // namespace

extern "C" {

int moe_mlp_workspace_size(const moe_mlp_config* cfg, int64_t T, int prefill, size_t* bytes) {
  const int st = validate_cfg(cfg, T, prefill);
  if (st) return st;
  if (!bytes) return MOE_MLP_ERR_NULL_ARG;
  *bytes = make_plan(cfg, T, gemm_form(cfg, T, prefill)).total;
  return MOE_MLP_OK;
}

int moe_mlp_decode(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x, int64_t T,
                   uint16_t* out, int32_t* ids_out, float* w_out, void* workspace, size_t ws_bytes,
                   void* stream) {
  return run_layer(cfg, w, x, T, out, ids_out, w_out, workspace, ws_bytes, stream, 0);
}

int moe_mlp_prefill(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x, int64_t T,
                    uint16_t* out, int32_t* ids_out, float* w_out, void* workspace, size_t ws_bytes,
                    void* stream) {
  return run_layer(cfg, w, x, T, out, ids_out, w_out, workspace, ws_bytes, stream, 1);
}

int moe_mlp_forward_profiled(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x, int64_t T,
                             uint16_t* out, int32_t* ids_out, float* w_out, void* workspace, size_t ws_bytes,
                             void* stream, int prefill, void* const* events, int n_events) {
  if (!events) return MOE_MLP_ERR_NULL_ARG;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return MOE_MLP_ERR_NULL_ARG;
  return run_layer(cfg, w, x, T, out, ids_out, w_out, workspace, ws_bytes, stream, prefill ? 1 : 0, events,
                   n_events);
}

const char* moe_mlp_stage_name(const moe_mlp_config* cfg, int64_t T, int prefill, int stage) {
  if (!cfg || stage < 0) return nullptr;
  if (cfg->kind == MOE_MLP_KIND_DENSE) return stage < 2 ? kDenseStages[stage] : nullptr;
  if (decode1_ok(cfg, T, prefill)) return stage < 3 ? kDecode1Stages[stage] : nullptr;
  if (gemm_form(cfg, T, prefill)) return stage < 8 ? kPrefillStages[stage] : nullptr;
  return stage < 7 ? kDecodeStages[stage] : nullptr;
}

int moe_router_topk(const moe_mlp_config* cfg, const float* router_w, const float* router_bias,
                    const uint16_t* x, int64_t T, int32_t* ids, float* w, void* workspace, size_t ws_bytes,
                    void* stream) {
  int st = validate_cfg(cfg, T, 1);
  if (st) return st;
  if (cfg->kind != MOE_MLP_KIND_ROUTED) return MOE_MLP_ERR_KIND_MISMATCH;
  if (T == 0) return MOE_MLP_OK;
  if (!router_w || !router_bias || !x || !ids || !w || !workspace) return MOE_MLP_ERR_NULL_ARG;
  if (!aligned(router_w) || !aligned(router_bias) || !aligned(x) || !aligned(ids) || !aligned(w) ||
      !aligned(workspace))
    return MOE_MLP_ERR_MISALIGNED;
  const Plan p = make_plan(cfg, T, 1);
  if (ws_bytes < p.total) return MOE_MLP_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(workspace, p.logits);
  router_logits_plan(p, workspace, x, router_w, logits, T, cfg->hidden, cfg->num_experts, s, Ev{});
  topk_tokens(cfg->num_experts, logits, router_bias, static_cast<int>(T), cfg->top_k,
              cfg->routed_scaling_factor, ids, w, nullptr, nullptr, s, Ev{}, p.logit_planes, p.logit_splits);
  return launch_status();
}

int moe_nvfp4_tile_pack(const uint8_t* q, const uint8_t* s, int64_t mats, int64_t rows, int64_t cols,
                        uint8_t* q_tiled, uint8_t* s_tiled, void* stream) {
  if (!q || !s || !q_tiled || !s_tiled) return MOE_MLP_ERR_NULL_ARG;
  if (mats < 0 || rows <= 0 || cols <= 0 || rows % 32 != 0 || cols % 256 != 0) return MOE_MLP_ERR_BAD_SHAPE;
  if (!aligned(q) || !aligned(s) || !aligned(q_tiled) || !aligned(s_tiled)) return MOE_MLP_ERR_MISALIGNED;
  const int64_t pieces = mats * rows * (cols / 32) + mats * rows * (cols / 256);
  if (pieces == 0) return MOE_MLP_OK;
  if (cdiv(pieces, 256) > int64_t(0x7FFFFFFF)) return MOE_MLP_ERR_BAD_SHAPE;
  k_nvfp4_tile_pack<<<static_cast<unsigned>(cdiv(pieces, 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      q, s, mats, rows, cols, q_tiled, s_tiled);
  return launch_status();
}

int moe_nvfp4_dequant(const uint8_t* q, const uint8_t* s, float global, int64_t rows, int64_t cols,
                      float* out_f32, uint16_t* out_bf16, void* stream) {
  if (!q || !s || (!out_f32 && !out_bf16)) return MOE_MLP_ERR_NULL_ARG;
  if (rows < 0 || bad_dim(cols)) return MOE_MLP_ERR_BAD_SHAPE;
  if (!std::isfinite(global)) return MOE_MLP_ERR_BAD_VALUE;
  if (!aligned(q) || (out_f32 && !aligned(out_f32)) || (out_bf16 && !aligned(out_bf16)))
    return MOE_MLP_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(s) & 1u) != 0) return MOE_MLP_ERR_MISALIGNED;
  if (rows == 0) return MOE_MLP_OK;
  const int64_t n = rows * (cols / 32);
  k_nvfp4_dequant<<<static_cast<unsigned>(cdiv(n, 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      q, s, global, rows, static_cast<int>(cols), out_f32, out_bf16);
  return launch_status();
}

const char* moe_mlp_status_string(int status) {
  switch (status) {
    case MOE_MLP_OK: return "MOE_MLP_OK";
    case MOE_MLP_ERR_NULL_ARG: return "MOE_MLP_ERR_NULL_ARG";
    case MOE_MLP_ERR_BAD_SHAPE: return "MOE_MLP_ERR_BAD_SHAPE";
    case MOE_MLP_ERR_BAD_TOPK: return "MOE_MLP_ERR_BAD_TOPK";
    case MOE_MLP_ERR_BAD_VALUE: return "MOE_MLP_ERR_BAD_VALUE";
    case MOE_MLP_ERR_MISALIGNED: return "MOE_MLP_ERR_MISALIGNED";
    case MOE_MLP_ERR_WORKSPACE_TOO_SMALL: return "MOE_MLP_ERR_WORKSPACE_TOO_SMALL";
    case MOE_MLP_ERR_KIND_MISMATCH: return "MOE_MLP_ERR_KIND_MISMATCH";
    case MOE_MLP_ERR_HIP: return "MOE_MLP_ERR_HIP";
    default: return "MOE_MLP_ERR_UNKNOWN";
  }
}

}  // extern "C"
