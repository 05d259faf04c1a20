// C ABI of the routed MoE MLP library (declarations and contract in
// include/moe_mlp.h).  Host code: argument validation (before anything is
// enqueued), workspace layout, and the launch sequences of the decode and
// prefill forms.  The library allocates nothing and never synchronises; the
// only state it keeps between calls is the per-device address of the
// scratch array of moe_mlp_decode_noalloc.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "../../include/moe_mlp.h"
#include "common.hpp"
#include "decode1.hpp"
#include "decode_fp8.hpp"
#include "gemm.hpp"
#include "gemm_bf16.hpp"
#include "gemm_fp4.hpp"
#include "gemm_fp4s.hpp"
#include "gemm_fp8.hpp"
#include "gemm_fp8d.hpp"
#include "gemm_skinny.hpp"
#include "gemv.hpp"
#include "permute.hpp"
#include "router.hpp"

static_assert(MOE_MLP_MAX_EXPERTS <= moe::PERM_MAX_E, "k_perm_hist keeps one LDS counter per expert");

// The workspace of moe_mlp_decode_noalloc: a device array in the library's
// code object, so every GPU the library runs on holds its own copy from the
// time the code object is loaded there until the process ends.  In host code
// `scratch` names a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device (scratch_on_device).
static __device__ __align__(256) unsigned char scratch[MOE_MLP_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace moe;

constexpr int64_t kMaxDim = 65536;

bool finite_pos(float v) { return std::isfinite(v) && v > 0.0f; }
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool bad_dim(int64_t d) { return d <= 0 || d % 32 != 0 || d > kMaxDim; }

bool is_fp8(const moe_mlp_config* c) { return c->kind == MOE_MLP_KIND_ROUTED_FP8; }
bool is_routed(const moe_mlp_config* c) { return c->kind == MOE_MLP_KIND_ROUTED || is_fp8(c); }

int validate_cfg(const moe_mlp_config* c, int64_t T, int prefill) {
  if (!c) return MOE_MLP_ERR_NULL_ARG;
  if (!is_routed(c) && c->kind != MOE_MLP_KIND_DENSE) return MOE_MLP_ERR_BAD_VALUE;
  if (T < 0 || (!prefill && T > MOE_MLP_DECODE_MAX_T)) return MOE_MLP_ERR_BAD_SHAPE;
  if (bad_dim(c->hidden)) return MOE_MLP_ERR_BAD_SHAPE;
  if (!finite_pos(c->swiglu_limit)) return MOE_MLP_ERR_BAD_VALUE;
  if (c->kind == MOE_MLP_KIND_DENSE) {
    if (bad_dim(c->dense_intermediate)) return MOE_MLP_ERR_BAD_SHAPE;
    return MOE_MLP_OK;
  }
  if (bad_dim(c->moe_intermediate)) return MOE_MLP_ERR_BAD_SHAPE;
  if (is_fp8(c) && (c->hidden % MOE_MLP_FP8_BLOCK != 0 || c->moe_intermediate % MOE_MLP_FP8_BLOCK != 0))
    return MOE_MLP_ERR_BAD_SHAPE;
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
  size_t keys = 0;                                                               // one-token decode: top-k sort keys
  size_t wsplit = 0;                                                             // router weight, 3 bf16 planes
  int logit_planes = 1;
  int logit_splits = 1;       // reduction parts of the split-weight logits GEMM
  // few-token grouped-GEMM form: the shared expert's GEMMs split their
  // reduction (gate/up into sgu_splits parts, down into sd_splits) so that
  // their few output tiles still fill the GPU; parts are fp32, added in order
  int sgu_splits = 1, sd_splits = 1;
  size_t sgu_parts = 0;
  // up to 64 tokens the shared expert's projections run on k_skinny_bf16
  // (fp32 parts of kr columns; gate/up then always through the parts)
  bool skinny = false;
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

// FP8 experts have no expert-GEMV decode path: past the few-token kernels
// their decode runs the grouped GEMM.
int gemm_form(const moe_mlp_config* c, int64_t T, int prefill) {
  return (prefill || T >= kDecodeGemmMinT || is_fp8(c)) ? 1 : 0;
}

// Prefill router logits on the matrix cores (split fp32 weight, see router.hpp)
// when there are enough tokens and the reduction length suits the fast GEMM.
bool mfma_logits(const moe_mlp_config* c, int64_t T, int prefill) {
  return prefill && T > MOE_MLP_DECODE_MAX_T && c->hidden % 64 == 0;
}

// k_skinny_bf16 takes up to 64 tokens and reductions that are a multiple of
// 512; its part length: 1024 up to 32 tokens when the reduction allows (the
// token columns of a part in LDS and the weights in registers stay within
// budget), else 512.
bool skinny_ok(int64_t T, int64_t K) { return T >= 1 && T <= 64 && K % 512 == 0; }
int skinny_kr(int64_t T, int64_t K) { return (T <= 32 && K % 1024 == 0) ? 1024 : 512; }

// Reduction parts for a BF16 GEMM with `tiles` output tiles over a reduction
// of kdim: the most parts (of at most 16) that keep tiles x parts within one
// workgroup per CU (256) and every part a multiple of 128 long; 1 when the
// tiles alone give half the CUs work.
int reduction_splits(int64_t tiles, int64_t kdim) {
  if (tiles >= 128) return 1;
  for (int s : {16, 12, 8, 6, 4, 3, 2})
    if (tiles * s <= 256 && kdim % (128 * s) == 0) return s;
  return 1;
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
    // the logits GEMM has only ceil(T/256) x ceil(3E/256) output tiles: cut
    // its reduction into 4 parts when H allows, for 4x the workgroups (more
    // parts made the few-token GEMM faster but the top-k, which adds 3 x
    // parts values per logit, slower by more: measured at 64 tokens)
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
    p.n_tiles = a.take(8);
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
  if (!prefill && T <= DEC_MAX_T && c->kind == MOE_MLP_KIND_ROUTED) p.keys = a.take(size_t(T * E) * 8);
  if (Is) {
    if (skinny_ok(T, H) && skinny_ok(T, Is)) {
      p.skinny = true;
      p.sgu_splits = static_cast<int>(H / skinny_kr(T, H));
      p.sd_splits = static_cast<int>(Is / skinny_kr(T, Is));
      p.sgu_parts = a.take(size_t(p.sgu_splits) * T * 2 * Is * 4);
    } else if (prefill) {
      p.sgu_splits = reduction_splits(cdiv(T, B16_BM) * cdiv(2 * Is, B16_BN), H);
      p.sd_splits = reduction_splits(cdiv(T, B16_BM) * cdiv(H, B16_BN), Is);
      if (p.sgu_splits > 1) p.sgu_parts = a.take(size_t(p.sgu_splits) * T * 2 * Is * 4);
    }
    p.hs = a.take(size_t(T * Is) * 2);
    p.ys = a.take(size_t(p.sd_splits) * T * H * 4);
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
  } else if (is_fp8(c)) {
    need[n++] = w->router_w;
    need[n++] = w->router_bias;
    need[n++] = w->w13_f8;
    need[n++] = w->w13_f8_scale;
    need[n++] = w->w2_f8;
    need[n++] = w->w2_f8_scale;
    if (c->n_shared_experts) {
      need[n++] = w->shared_w13;
      need[n++] = w->shared_w2;
    }
  } else {
    // a projection's codes: the row-major array, or the tile-layout codes and
    // scales (then every kernel reads the tile-layout codes; see codes13)
    need[n++] = w->router_w;
    need[n++] = w->router_bias;
    need[n++] = w->w13_q ? w->w13_q : (w->w13_s_tiled ? w->w13_q_tiled : nullptr);
    need[n++] = w->w13_s;
    need[n++] = w->w13_g;
    need[n++] = w->w2_q ? w->w2_q : (w->w2_s_tiled ? w->w2_q_tiled : nullptr);
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
    // tile-layout codes only: the shapes the tile layout and its grouped GEMM
    // take (a reduction of at least 512 and a multiple of 256)
    if ((!w->w13_q && (c->hidden % 256 != 0 || c->hidden < 512)) ||
        (!w->w2_q && (c->moe_intermediate % 256 != 0 || c->moe_intermediate < 512)))
      return MOE_MLP_ERR_BAD_SHAPE;
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

// Routed NVFP4 codes that the kernels read: the row-major array, or (when it
// is not given) the tile-layout copy; the kernels take the layout as a
// template flag (true = tile layout).
const uint8_t* codes13(const moe_mlp_weights* w) { return w->w13_q ? w->w13_q : w->w13_q_tiled; }
const uint8_t* codes2(const moe_mlp_weights* w) { return w->w2_q ? w->w2_q : w->w2_q_tiled; }

template <typename F>
void with_ct(bool tiled, F&& f) {
  if (tiled) f(std::true_type{});
  else f(std::false_type{});
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
  // up to the decode limit: k_logits_rows (H a multiple of 8 up to 8192),
  // else one workgroup per expert row (the tile GEMM below has only
  // ceil(T/64) x ceil(E/64) workgroups, too few for small T)
  if (T <= MOE_MLP_DECODE_MAX_T && H % 8 == 0 && H <= 8192) {
    const int cpt = static_cast<int>(cdiv(H / 8, 256));
    auto go = [&](auto kern, int ne) {
      const dim3 grid(static_cast<unsigned>(8 * cdiv(cdiv(E, ne), 8)), static_cast<unsigned>(cdiv(T, LOGIT_TG)));
      launch(kern, grid, dim3(256), s, ev.a, ev.b, x, wr, logits, static_cast<int>(T), H, E);
    };
    // two experts per workgroup up to 64 tokens, four beyond when H <= 4096
    // (each token row is then read from L2 by E / 4 workgroups; the weights
    // of four experts at larger H would not fit the registers); measured at
    // 32 and 64 tokens, two experts: 7.8 -> 7.3 us and 13.2 -> 11.0 us
    const bool ne4 = T > 64;
    switch (cpt) {
      case 1: ne4 ? go(k_logits_rows<1, 4>, 4) : go(k_logits_rows<1, 2>, 2); break;
      case 2: ne4 ? go(k_logits_rows<2, 4>, 4) : go(k_logits_rows<2, 2>, 2); break;
      case 3: go(k_logits_rows<3, 2>, 2); break;
      default: go(k_logits_rows<4, 2>, 2); break;
    }
  } else if (T <= MOE_MLP_DECODE_MAX_T) {
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
void gemv(const GemvArgs& a, int groups, hipStream_t s, Ev ev, bool tiled_codes = false) {
  // without expert groups the tokens go in groups of GEMV_TC over grid.y, and
  // grid.x is a multiple of 8: blocks go to the 8 XCDs round-robin, so every
  // token group of a row block runs on the same XCD and reads its rows from L2
  if (!a.n_groups) groups = static_cast<int>(cdiv(a.T, GEMV_TC));
  const int64_t nrb = cdiv(a.half_rows, 4 * RW);
  const dim3 grid(static_cast<unsigned>(a.n_groups ? nrb : cdiv(nrb, 8) * 8), static_cast<unsigned>(groups));
  const int nch = NVFP4 ? (a.cols >> 5) : (a.cols >> 3);
  if constexpr (NVFP4) {
    // up to 16 tokens an expert group holds at most 16 tokens (1.2 on average
    // at 16): one token per pass
    with_ct(tiled_codes, [&](auto ctc) {
      constexpr bool CT = decltype(ctc)::value;
      if (a.T <= 16)
        launch(k_gemv<NVFP4, MODE, RW, 0, 1, CT>, grid, dim3(256), s, ev.a, ev.b, a);
      else
        launch(k_gemv<NVFP4, MODE, RW, 0, GEMV_TC, CT>, grid, dim3(256), s, ev.a, ev.b, a);
    });
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

// Routed NVFP4 down projection of decode batches (up to MOE_MLP_DECODE_MAX_T
// tokens, a few per expert) on k_skinny_f4_down: reductions of 512, 1024,
// 1536 or 2048 columns and output rows a multiple of 64.
bool skinny_down_ok(const moe_mlp_config* c, int64_t T) {
  const int I = c->moe_intermediate;
  return c->kind == MOE_MLP_KIND_ROUTED && T <= MOE_MLP_DECODE_MAX_T && c->hidden % SF4_ROWS == 0 && I % 512 == 0 &&
         I <= 2048;
}

// groups = grid.y (the largest number of expert groups); tiled = the codes
// are the tile-layout copy.  12 activation rows of LDS per pass (37 KB) are
// the most that keep four workgroups on a CU; measured against 8 rows (the
// same at 16 and 64 tokens; 64 tokens top-16 with 8 hot experts 148.9 ->
// 135.0 us, 256 tokens 236.9 -> 220.0 us) and 16 rows (three workgroups on
// a CU: 64 tokens 158 -> 175 us).
void skinny_down(const SkinnyF4Args& a, int kdim, int groups, bool tiled, hipStream_t s, Ev ev) {
  const dim3 grid(static_cast<unsigned>(a.N / SF4_ROWS), static_cast<unsigned>(groups));
  with_ct(tiled, [&](auto ctc) {
    constexpr bool CT = decltype(ctc)::value;
    auto go = [&](auto nu) {
      constexpr int NU = decltype(nu)::value;
      launch(k_skinny_f4_down<NU, 12, CT>, grid, dim3(256), s, ev.a, ev.b, a);
    };
    switch (kdim / 128) {
      case 4: go(std::integral_constant<int, 4>{}); break;
      case 8: go(std::integral_constant<int, 8>{}); break;
      case 12: go(std::integral_constant<int, 12>{}); break;
      default: go(std::integral_constant<int, 16>{}); break;
    }
  });
}

// Routed FP8 projections: k_gemm_f8d (LDS DMA rings) when its 32-bit DMA
// offsets hold (activation rows and weight rows times the row length below
// 2^31) and the reduction is at most 8192; otherwise k_gemm_f8.
template <int MODE>
void gemm_fp8(const GemmArgs& a0, int64_t m_tiles, hipStream_t s, Ev ev) {
  GemmArgs a = a0;
  const int64_t w_rows = MODE == GEMM_GATEUP ? 2 * int64_t(a.half_n) : int64_t(a.half_n);
  if (a.kdim <= 8192 && int64_t(a.T) * a.kdim * 2 < (int64_t(1) << 31) && w_rows * a.kdim < (int64_t(1) << 31)) {
    a.n_blocks = static_cast<int>(cdiv(a.half_n, MODE == GEMM_GATEUP ? F8D_WROWS / 2 : F8D_WROWS));
    const dim3 grid(static_cast<unsigned>(8 * cdiv(m_tiles * a.n_blocks, 8)));
    launch(k_gemm_f8d<MODE>, grid, dim3(F8D_THREADS), s, ev.a, ev.b, a);
    return;
  }
  const dim3 grid(static_cast<unsigned>(m_tiles),
                  static_cast<unsigned>(cdiv(a.half_n, MODE == GEMM_GATEUP ? 128 : 256)));
  launch(k_gemm_f8<MODE>, grid, dim3(256), s, ev.a, ev.b, a);
}

// Tiles of at most this many rows go to k_gemm_nvfp4_m32 (the scheduler puts
// them after the others): up to MOE_MLP_DECODE_MAX_T tokens, in the gate/up
// projection.  With thousands of tokens the few short tiles cost more as a
// launch of their own, after the large ones, than inside k_gemm_nvfp4; the
// down projection (its reduction is the short one, I) ran 3% slower on the
// small-tile kernel at 64 tokens (both measured).
int small_tile_rows(int64_t T) { return T <= MOE_MLP_DECODE_MAX_T ? F4M_ROWS : 0; }

// Largest expert row count for which k_gemm_nvfp4_m32 splits the tiles of
// more than 32 rows into one workgroup per pass (instead of k_gemm_nvfp4).
constexpr int64_t SPLIT_PASS_MAX_ROWS = 2 * F4M_ROWS;

// Routed NVFP4 projections with a reduction length that is a multiple of 256
// and at least 512 take k_gemm_nvfp4; with small_rows (gate/up) it takes only
// the tiles of more than small_rows rows (at most slots / (small_rows + 1) of
// them) and k_gemm_nvfp4_m32 the rest (up to 64 rows an expert
// k_gemm_nvfp4_m32 takes the long tiles too, one workgroup per 32-row
// pass); max_count = the most rows an expert can
// hold (the token count): at most 64, k_gemm_nvfp4_m32 takes every tile and
// k_gemm_nvfp4 is not launched (its launch cost 4.4 us at 64 tokens, where no
// tile had more than 32 rows).  BF16
// projections (shared expert, dense FFN, router logits) with a reduction
// length that is a multiple of 128 take k_gemm_bf16; other reduction lengths
// that are a multiple of 64 the 32x32x16-MFMA kernel (k_gemm_fast); the rest
// the general 16x16x32 kernel.
template <bool NVFP4, int MODE, bool ROUTED>
void gemm(const GemmArgs& a0, int64_t m_tiles, hipStream_t s, Ev ev, int small_rows = 0, int64_t slots = 0,
          int64_t max_count = -1) {
  GemmArgs a = a0;
  if constexpr (NVFP4 && ROUTED && (MODE == GEMM_GATEUP || MODE == GEMM_DOWN_SLOT_F32)) {
    // its DMA offsets are 32-bit: activation rows (T here) and weight rows
    // times the row length must stay below 2^31 bytes
    const int64_t w_rows = MODE == GEMM_GATEUP ? 2 * int64_t(a.half_n) : int64_t(a.half_n);
    if (a.kdim % 256 == 0 && a.kdim >= 512 && int64_t(a.T) * a.kdim * 2 < (int64_t(1) << 31) &&
        w_rows * a.kdim / 2 < (int64_t(1) << 31)) {
      a.n_blocks = static_cast<int>(cdiv(a.half_n, MODE == GEMM_GATEUP ? F4_WROWS / 2 : F4_WROWS));
      const bool use_small = MODE == GEMM_GATEUP && small_rows == F4M_ROWS;
      // up to 64 tokens and 512 slots k_gemm_nvfp4_m32 takes every tile (a
      // tile of more than 32 rows in two passes; the 128-row kernel's launch
      // would mostly find nothing to do: 4.4 us at 64 tokens); with more
      // slots (top-16 at 64 tokens) the tiles of more than 32 rows go to the
      // 128-row kernel in one pass (64 tokens top-16 with 8 hot experts:
      // routed gate/up 283.6 -> 273.6 us)
      const bool small_only = use_small && max_count >= 0 && max_count <= 2 * F4M_ROWS && slots <= 512;
      const int64_t big_tiles = use_small ? std::min<int64_t>(m_tiles, slots / (F4M_ROWS + 1)) : m_tiles;
      // with more slots but still at most 64 rows an expert (top-16 at 64
      // tokens), the tiles of more than 32 rows are split into one workgroup
      // per 32-row pass inside k_gemm_nvfp4_m32, dispatched first, instead:
      // the few hot experts' tiles no longer hold a handful of CUs after the
      // rest of the chip has finished (64 tokens top-16 with 8 hot experts:
      // routed gate/up 269 -> 210 us, step 464 -> 421 us; 128 tokens, where
      // the split would take up to 4 passes, measured the same either way)
      const bool split = use_small && !small_only && max_count >= 0 && max_count <= SPLIT_PASS_MAX_ROWS;
      const int split_s = split ? static_cast<int>(cdiv(max_count, F4M_ROWS)) : 0;
      a.skip_rows = (use_small && !small_only && !split) ? F4M_ROWS : 0;
      a.split_pass = split_s;
      with_ct(a.bq_t && a.bs_t, [&](auto ctc) {
        constexpr bool CT = decltype(ctc)::value;
        if (!small_only && !split && big_tiles > 0)
          launch(k_gemm_nvfp4<MODE, CT>, dim3(static_cast<unsigned>(8 * cdiv(big_tiles * a.n_blocks, 8))),
                 dim3(F4_THREADS), s, ev.a, use_small ? nullptr : ev.b, a);
        if constexpr (MODE == GEMM_GATEUP) {
          if (use_small) {
            const int64_t blocks = 8 * (cdiv(big_tiles * a.n_blocks * split_s, 8) + cdiv(m_tiles * a.n_blocks, 8));
            launch(k_gemm_nvfp4_m32<MODE, CT>, dim3(static_cast<unsigned>(blocks)), dim3(F4_THREADS), s,
                   (small_only || split || big_tiles == 0) ? ev.a : nullptr, ev.b, a);
          }
        }
      });
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

// out[q][t][n] (q < K / kr parts, part stride T * N) = x[t] . w[n] over the
// part's kr columns, on k_skinny_bf16 (skinny_ok(T, K) holds).
void skinny_gemm(const uint16_t* x, const uint16_t* w, int N, int K, int T, float* out, hipStream_t s, Ev ev) {
  const int kr = skinny_kr(T, K), nparts = K / kr;
  const dim3 grid(static_cast<unsigned>(cdiv(N, F16S_ROWS) * nparts));
  const int64_t ps = int64_t(T) * N;
  auto go = [&](auto kern) { launch(kern, grid, dim3(256), s, ev.a, ev.b, x, K, w, K, N, T, nparts, out, ps); };
  const int tb = static_cast<int>(cdiv(T, 16));
  if (kr == 1024) {
    if (tb == 1) go(k_skinny_bf16<1, 1024>);
    else go(k_skinny_bf16<2, 1024>);
  } else {
    switch (tb) {
      case 1: go(k_skinny_bf16<1, 512>); break;
      case 2: go(k_skinny_bf16<2, 512>); break;
      case 3: go(k_skinny_bf16<3, 512>); break;
      default: go(k_skinny_bf16<4, 512>); break;
    }
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
const char* const kDecode1Stages[] = {"logits_shared_gateup", "routed_gateup", "shared_routed_down_combine"};
const char* const kPrefillStages[] = {"router_logits", "topk", "permute", "routed_gateup", "routed_down",
                                     "shared_gateup", "shared_down", "combine"};
const char* const kDenseStages[] = {"dense_gateup", "dense_down"};

// The one-token decode kernels hold a row's chunks in registers: they take
// H <= 4096 and I, Is <= 2048.
constexpr int kDec1MaxH = DEC_MAX_H;

// The few-token decode kernels (decode1.hpp) take up to 4 tokens (the MTP
// verify shapes: one token plus up to three drafted ones), T*K <= 64 slots.
constexpr int64_t kDecFewMaxT = 4;
static_assert(kDecFewMaxT <= DEC_MAX_T, "k_dec_down_combine keeps the shared rows' sums of DEC_MAX_T tokens");

bool decode1_ok(const moe_mlp_config* c, int64_t T, int prefill) {
  if (prefill || T < 1 || T > kDecFewMaxT || !is_routed(c)) return false;
  if (T * c->top_k > 64) return false;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  return c->hidden <= kDec1MaxH && c->moe_intermediate <= 2048 && Is <= 2048;
}

int n_stages(const moe_mlp_config* c, int64_t T, int prefill) {
  if (c->kind == MOE_MLP_KIND_DENSE) return 2;
  if (decode1_ok(c, T, prefill)) return 3;
  return gemm_form(c, T, prefill) ? 8 : 7;
}

// Few-token decode (1..4 tokens): 3 launches (see decode1.hpp).  The layer
// shape of GLM-5.3-Flash (H 4096, I and Is 1536, 288 experts, top-8) has
// kernel instances of its own with the geometry compiled in.
using DecGeoFlash = DecGeo<4096, 1536, 288, 8, 1536>;

bool flash_shape(const moe_mlp_config* c) {
  return c->hidden == DecGeoFlash::H && c->moe_intermediate == DecGeoFlash::I &&
         c->num_experts == DecGeoFlash::E && c->top_k == DecGeoFlash::K && c->n_shared_experts == 1 &&
         c->shared_intermediate == DecGeoFlash::IS;
}
bool glm_flash_geometry(const moe_mlp_config* c) { return c->kind == MOE_MLP_KIND_ROUTED && flash_shape(c); }
bool glm_flash_geometry_fp8(const moe_mlp_config* c) { return is_fp8(c) && flash_shape(c); }

// k_dec_logits_shared_t: row blocks (padded to a multiple of 8, the extra
// blocks exit) x token groups.
dim3 logits_shared_t_grid(int row_blocks, int64_t T) {
  return dim3(static_cast<unsigned>(cdiv(row_blocks, 8) * 8), static_cast<unsigned>(cdiv(T, DEC_TG)));
}

// Routed gate/up: RJ (gate, up) row pairs per wavefront (16 KB of codes at H = 4096).
constexpr int kDecRJ = 4;

void dec_gateup(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, const float* logits,
                int32_t* ids, float* wts, int32_t* ids_out, float* w_out, uint16_t* h, int T, hipStream_t s, Ev ev,
                const uint64_t* keys = nullptr) {
  constexpr int NC = 2;
  const int H = c->hidden, I = c->moe_intermediate, K = c->top_k;
  const unsigned grid = static_cast<unsigned>(T * K * cdiv(I, 4 * kDecRJ));
  const uint8_t* q13 = codes13(w);
  auto go = [&](auto kern) {
    launch(kern, dim3(grid), dim3(256), s, ev.a, ev.b, x, q13, w->w13_s, w->w13_g, logits, w->router_bias, K,
           c->routed_scaling_factor, ids, wts, ids_out, w_out, c->num_experts, H, I, c->swiglu_limit, h, keys);
  };
  with_ct(!w->w13_q, [&](auto ctc) {
    constexpr bool CT = decltype(ctc)::value;
    if (glm_flash_geometry(c)) {
      go(k_dec_gateup<kDecRJ, NC, true, 5, DecGeoFlash, CT>);
      return;
    }
    with_nj(c->num_experts, [&](auto nj) {
      constexpr int NJ = decltype(nj)::value;
      if (H == 64 * 32 * NC) go(k_dec_gateup<kDecRJ, NC, true, NJ, DecGeoAny, CT>);     // every lane holds NC chunks
      else go(k_dec_gateup<kDecRJ, NC, false, NJ, DecGeoAny, CT>);
    });
  });
}

// Shared + routed down + combine: 4 output rows per block; NW wavefronts with
// NP slots each (NW * NP >= T * K), NSC 16-byte chunks per lane of a shared row.
template <int NW, int NP>
void launch_down_combine(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* h, const uint16_t* hs,
                         const int32_t* ids, const float* wts, uint16_t* out, int T, hipStream_t s, Ev ev) {
  constexpr int R = 4;
  const int H = c->hidden;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const dim3 grid(static_cast<unsigned>(cdiv(H, R))), block(NW * 64);
  const uint8_t* q2 = codes2(w);
  auto go = [&](auto kern) {
    launch(kern, grid, block, s, ev.a, ev.b, h, q2, w->w2_s, w->w2_g, w->shared_w2, hs, Is, ids, wts,
           c->num_experts, c->top_k, H, c->moe_intermediate, out, T);
  };
  with_ct(!w->w2_q, [&](auto ctc) {
    constexpr bool CT = decltype(ctc)::value;
    if (glm_flash_geometry(c)) {
      go(k_dec_down_combine<R, NW, NP, 3, DecGeoFlash, CT>);
      return;
    }
    switch (static_cast<int>(cdiv(Is / 8, 64))) {
      case 0: case 1: go(k_dec_down_combine<R, NW, NP, 1, DecGeoAny, CT>); break;
      case 2: go(k_dec_down_combine<R, NW, NP, 2, DecGeoAny, CT>); break;
      case 3: go(k_dec_down_combine<R, NW, NP, 3, DecGeoAny, CT>); break;
      default: go(k_dec_down_combine<R, NW, NP, 4, DecGeoAny, CT>); break;
    }
  });
}

// Shared + routed down + combine of 1..4 tokens (k_dec_down_combine1): a
// wavefront per routed slot and 4 for the shared rows, a grid row per token;
// 16 output rows per block for one token, 8 for 2..4 tokens (more blocks,
// each with a token's whole slot set; measured against 16 rows: 2 tokens
// 17.8 -> 15.8 us, 4 tokens 31.7 -> 26.8 us, 1 token 9.6 against 9.7 us).
constexpr int kDown1Shared = 4;

template <int R>
void launch_down_combine1_r(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* h, const uint16_t* hs,
                            const int32_t* ids, const float* wts, uint16_t* out, int T, hipStream_t s, Ev ev) {
  constexpr int NSW = kDown1Shared;
  const int H = c->hidden, K = c->top_k;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const dim3 grid(static_cast<unsigned>(cdiv(H, R)), static_cast<unsigned>(T)),
      block(static_cast<unsigned>((K + NSW) * 64));
  const uint8_t* q2 = codes2(w);
  auto go = [&](auto kern) {
    launch(kern, grid, block, s, ev.a, ev.b, h, q2, w->w2_s, w->w2_g, w->shared_w2, hs, Is, ids, wts,
           c->num_experts, K, H, c->moe_intermediate, out);
  };
  with_ct(!w->w2_q, [&](auto ctc) {
    constexpr bool CT = decltype(ctc)::value;
    if (glm_flash_geometry(c)) {
      go(k_dec_down_combine1<R, NSW, 3, DecGeoFlash, CT>);
      return;
    }
    switch (static_cast<int>(cdiv(Is / 8, 64))) {
      case 0: case 1: go(k_dec_down_combine1<R, NSW, 1, DecGeoAny, CT>); break;
      case 2: go(k_dec_down_combine1<R, NSW, 2, DecGeoAny, CT>); break;
      case 3: go(k_dec_down_combine1<R, NSW, 3, DecGeoAny, CT>); break;
      default: go(k_dec_down_combine1<R, NSW, 4, DecGeoAny, CT>); break;
    }
  });
}

void launch_down_combine1(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* h, const uint16_t* hs,
                          const int32_t* ids, const float* wts, uint16_t* out, int T, hipStream_t s, Ev ev) {
  if (T == 1) launch_down_combine1_r<16>(c, w, h, hs, ids, wts, out, T, s, ev);
  else launch_down_combine1_r<8>(c, w, h, hs, ids, wts, out, T, s, ev);
}

// Few-token decode with FP8 experts: launches 2 and 3 of decode_fp8.hpp.
template <class G, int NJ, int NSC, int NW, int NP>
void dec_fp8_launch(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, const float* logits,
                    int32_t* ids, float* wts, int32_t* ids_out, float* w_out, uint16_t* h, const uint16_t* hs,
                    uint16_t* out, int T, hipStream_t s, Ev e1, Ev e2) {
  constexpr int RJ = 2, R = 4;
  const int H = c->hidden, I = c->moe_intermediate, K = c->top_k;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const unsigned grid = static_cast<unsigned>(T * K * cdiv(I, 4 * RJ));
  // H <= 4096: at most 4 chunks of 16 bytes per lane and row; H == 4096 fills them all
  if (H == 4096)
    launch(k_dec_gateup_f8<RJ, 4, true, NJ, G>, dim3(grid), dim3(256), s, e1.a, e1.b, x, w->w13_f8,
           w->w13_f8_scale, logits, w->router_bias, K, c->routed_scaling_factor, ids, wts, ids_out, w_out,
           c->num_experts, H, I, c->swiglu_limit, h);
  else
    launch(k_dec_gateup_f8<RJ, 4, false, NJ, G>, dim3(grid), dim3(256), s, e1.a, e1.b, x, w->w13_f8,
           w->w13_f8_scale, logits, w->router_bias, K, c->routed_scaling_factor, ids, wts, ids_out, w_out,
           c->num_experts, H, I, c->swiglu_limit, h);
  // I <= 2048: at most 2 chunks of 16 bytes per lane and down row.  More
  // than 16 slots (3 or 4 tokens at top-8): 8 rows per block, a wavefront per
  // slot and a grid row per token, so each h vector is read once per 8 rows
  // (measured, 4 tokens: 65.5 -> 42.9 us); up to 16 slots the 4-row blocks,
  // one slot per wavefront, are as fast (1 and 2 tokens: 13.6 / 13.4 us and
  // 23.3 / 24.2 us; 16-row blocks 20.9 us at 1 token).
  constexpr int R1 = 8, NSW1 = 4;
  if (K + NSW1 <= 16 && T * K > 16)
    launch(k_dec_down_combine1_f8<R1, NSW1, NSC, 2, G>,
           dim3(static_cast<unsigned>(cdiv(H, R1)), static_cast<unsigned>(T)),
           dim3(static_cast<unsigned>((K + NSW1) * 64)), s, e2.a, e2.b, h, w->w2_f8, w->w2_f8_scale, w->shared_w2,
           hs, Is, ids, wts, c->num_experts, K, H, I, out);
  else
    launch(k_dec_down_combine_f8<R, NW, NP, NSC, 2, G>, dim3(static_cast<unsigned>(cdiv(H, R))), dim3(NW * 64), s,
           e2.a, e2.b, h, w->w2_f8, w->w2_f8_scale, w->shared_w2, hs, Is, ids, wts, c->num_experts, K, H, I, out, T);
}

template <class G, int NJ, int NSC>
void dec_fp8_nw(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, const float* logits,
                int32_t* ids, float* wts, int32_t* ids_out, float* w_out, uint16_t* h, const uint16_t* hs,
                uint16_t* out, int T, hipStream_t s, Ev e1, Ev e2) {
  const int S = T * c->top_k;
  if (S <= 4) dec_fp8_launch<G, NJ, NSC, 4, 1>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
  else if (S <= 8) dec_fp8_launch<G, NJ, NSC, 8, 1>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
  else if (S <= 16) dec_fp8_launch<G, NJ, NSC, 16, 1>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
  else if (S <= 32) dec_fp8_launch<G, NJ, NSC, 16, 2>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
  else dec_fp8_launch<G, NJ, NSC, 16, 4>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
}

void dec_fp8(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, const float* logits, int32_t* ids,
             float* wts, int32_t* ids_out, float* w_out, uint16_t* h, const uint16_t* hs, uint16_t* out, int T,
             hipStream_t s, Ev e1, Ev e2) {
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  if (glm_flash_geometry_fp8(c)) {
    dec_fp8_nw<DecGeoFlash, 5, 3>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
    return;
  }
  with_nj(c->num_experts, [&](auto nj) {
    constexpr int NJ = decltype(nj)::value;
    switch (static_cast<int>(cdiv(Is / 8, 64))) {
      case 0: case 1: dec_fp8_nw<DecGeoAny, NJ, 1>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2); break;
      case 2: dec_fp8_nw<DecGeoAny, NJ, 2>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2); break;
      case 3: dec_fp8_nw<DecGeoAny, NJ, 3>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2); break;
      default: dec_fp8_nw<DecGeoAny, NJ, 4>(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2); break;
    }
  });
}

void decode1(const moe_mlp_config* c, const moe_mlp_weights* w, const uint16_t* x, int T, uint16_t* out,
             int32_t* ids_out, float* w_out, float* logits, int32_t* ids, float* wts, uint16_t* h, uint16_t* hs,
             hipStream_t s, Ev e0, Ev e1, Ev e2, uint64_t* keys) {
  const int H = c->hidden, E = c->num_experts, K = c->top_k;
  const int Is = c->n_shared_experts ? c->shared_intermediate : 0;
  const int nlb = static_cast<int>(cdiv(E, 4)), nsb = static_cast<int>(cdiv(Is, 4));
  // NVFP4 experts: launch 1 also writes the top-k sort keys
  if (is_fp8(c)) keys = nullptr;
  if (T == 1 && glm_flash_geometry(c))
    launch(k_dec_logits_shared<16, 8, DecGeoFlash>, dim3(nlb + nsb), dim3(256), s, e0.a, e0.b, x, w->router_w, logits,
           E, H, w->shared_w13, Is, hs, c->swiglu_limit, nlb, w->router_bias, keys);
  else if (T == 1)
    launch(k_dec_logits_shared<16, 8, DecGeoAny>, dim3(nlb + nsb), dim3(256), s, e0.a, e0.b, x, w->router_w, logits,
           E, H, w->shared_w13, Is, hs, c->swiglu_limit, nlb, w->router_bias, keys);
  else
    launch(k_dec_logits_shared_t<16, 8>, logits_shared_t_grid(nlb + nsb, T), dim3(256), s, e0.a, e0.b, x, w->router_w, logits, E, H,
           w->shared_w13, Is, hs, c->swiglu_limit, nlb, T, w->router_bias, keys);
  if (is_fp8(c)) {
    dec_fp8(c, w, x, logits, ids, wts, ids_out, w_out, h, hs, out, T, s, e1, e2);
    return;
  }
  dec_gateup(c, w, x, logits, ids, wts, ids_out, w_out, h, T, s, e1, keys);
  if (K + kDown1Shared <= 16) {
    launch_down_combine1(c, w, h, hs, ids, wts, out, T, s, e2);
    return;
  }
  // one slot per wavefront up to 8 slots (4 or 8 wavefronts), else 16 wavefronts with up to 4 slots each
  const int S = T * K;
  if (S <= 4) launch_down_combine<4, 1>(c, w, h, hs, ids, wts, out, T, s, e2);
  else if (S <= 8) launch_down_combine<8, 1>(c, w, h, hs, ids, wts, out, T, s, e2);
  else if (S <= 16) launch_down_combine<16, 1>(c, w, h, hs, ids, wts, out, T, s, e2);
  else if (S <= 32) launch_down_combine<16, 2>(c, w, h, hs, ids, wts, out, T, s, e2);
  else launch_down_combine<16, 4>(c, w, h, hs, ids, wts, out, T, s, e2);
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
  if (is_routed(c) && ((ids_out && !aligned(ids_out)) || (w_out && !aligned(w_out))))
    return MOE_MLP_ERR_MISALIGNED;
  if (!decode1_ok(c, T, prefill)) prefill = gemm_form(c, T, prefill);   // from here on: the form that runs
  // with tile-layout codes only, the grouped GEMM must take its tile kernel,
  // whose 32-bit DMA offsets bound the activation rows (tokens, slots) times
  // the reduction length
  if (prefill && c->kind == MOE_MLP_KIND_ROUTED &&
      ((!w->w13_q && T * c->hidden * 2 >= (int64_t(1) << 31)) ||
       (!w->w2_q && T * c->top_k * c->moe_intermediate * 2 >= (int64_t(1) << 31))))
    return MOE_MLP_ERR_BAD_SHAPE;
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
    decode1(c, w, x, Ti, out, ids_out, w_out, logits, ids, wts, h, hs, s, ev(0), ev(1), ev(2),
            p.keys ? at<uint64_t>(ws, p.keys) : nullptr);
    return launch_status();
  }
  // decode of up to 16 tokens with H <= 4096: router logits and the shared
  // expert's gate/up share one launch (stage router_logits; shared_gateup
  // then records an empty stage)
  const bool fused_k1 = !prefill && T <= 16 && H <= kDec1MaxH && Is <= 2048 && !p.skinny;
  if (fused_k1) {
    const int nlb = static_cast<int>(cdiv(E, 4)), nsb = static_cast<int>(cdiv(Is, 4));
    launch(k_dec_logits_shared_t<16, 8>, logits_shared_t_grid(nlb + nsb, Ti), dim3(256), s, ev(0).a, ev(0).b, x, w->router_w, logits,
           E, H, w->shared_w13, Is, hs, L, nlb, Ti, static_cast<const float*>(nullptr), static_cast<uint64_t*>(nullptr));
  } else {
    router_logits_plan(p, ws, x, w->router_w, logits, T, H, E, s, ev(0));
  }
  if (prefill) {
    topk_tokens(E, logits, w->router_bias, Ti, K, rsf, ids, wts, ids_out, w_out, s, ev(1), p.logit_planes,
                p.logit_splits);
    Perm pm{at<int32_t>(ws, p.count), at<int32_t>(ws, p.offset), at<int32_t>(ws, p.perm),
            at<int32_t>(ws, p.n_tiles), at<int32_t>(ws, p.tile_e), at<int32_t>(ws, p.tile_m0)};
    const Ev pe = ev(2);
    const int small_rows = small_tile_rows(T);
    if (S <= PERM_SMALL_MAX) {
      launch(k_perm_small, dim3(1), dim3(1024), s, pe.a, pe.b, ids, static_cast<int>(S), E, GM_BM, small_rows, pm);
    } else {
      const int nchunk = static_cast<int>(cdiv(S, PERM_CHUNK));
      int32_t* phist = at<int32_t>(ws, p.phist);
      int32_t* prank = at<int32_t>(ws, p.prank);
      launch(k_perm_hist, dim3(nchunk), dim3(PERM_CHUNK), s, pe.a, nullptr, ids, static_cast<int>(S), E, phist,
             prank);
      int32_t* pbase = at<int32_t>(ws, p.pbase);
      launch(k_perm_schedule, dim3(1), dim3(1024), s, nullptr, nullptr, E, nchunk, GM_BM, small_rows, phist, pbase,
             pm);
      launch(k_perm_scatter, dim3(static_cast<unsigned>(cdiv(S, 256))), dim3(256), s, nullptr, pe.b, ids,
             static_cast<int>(S), E, pbase, prank, pm);
    }
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
    if (is_fp8(c)) {
      gu.bq = w->w13_f8;
      gu.bs = nullptr;
      gu.bq_t = gu.bs_t = nullptr;
      gu.bsf = w->w13_f8_scale;
      gu.stride_q = int64_t(2) * I * H;
      gu.stride_s = int64_t(2) * (I / MOE_MLP_FP8_BLOCK) * (H / MOE_MLP_FP8_BLOCK);
      gu.gscale = nullptr;
      gemm_fp8<GEMM_GATEUP>(gu, p.max_tiles, s, ev(3));
    } else {
      gemm<true, GEMM_GATEUP, true>(gu, p.max_tiles, s, ev(3), small_rows, S, T);
    }
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
    if (is_fp8(c)) {
      gd.bq = w->w2_f8;
      gd.bs = nullptr;
      gd.bq_t = gd.bs_t = nullptr;
      gd.bsf = w->w2_f8_scale;
      gd.stride_q = int64_t(H) * I;
      gd.stride_s = int64_t(H / MOE_MLP_FP8_BLOCK) * (I / MOE_MLP_FP8_BLOCK);
      gd.gscale = nullptr;
      gemm_fp8<GEMM_DOWN_SLOT_F32>(gd, p.max_tiles, s, ev(4));
    } else if (skinny_down_ok(c, T)) {
      SkinnyF4Args sa{};
      const bool tiled = w->w2_q_tiled && (!w->w2_q || w->w2_s_tiled);
      sa.wq = tiled ? w->w2_q_tiled : w->w2_q;
      sa.ws = w->w2_s;
      sa.stride_q = int64_t(H) * I / 2;
      sa.stride_s = int64_t(H) * I / 16;
      sa.gscale = w->w2_g;
      sa.N = H;
      sa.offsets = pm.offset;
      if (small_rows && T <= GM_BM) {
        // experts in the scheduler's tile order (at most one tile each up to
        // 128 rows): those of more than 32 rows are dispatched first
        sa.n_groups = pm.n_tiles;
        sa.g_expert = pm.tile_expert;
      }
      sa.out_idx = pm.perm;
      sa.in = h;
      sa.out = y;
      skinny_down(sa, I, E, tiled, s, ev(4));
    } else {
      gemm<true, GEMM_DOWN_SLOT_F32, true>(gd, p.max_tiles, s, ev(4), small_rows, S, T);
    }
    const int64_t mt = cdiv(T, GM_BM);
    if (Is && p.skinny) {
      float* parts = at<float>(ws, p.sgu_parts);
      skinny_gemm(x, w->shared_w13, 2 * Is, H, Ti, parts, s, Ev{ev(5).a, nullptr});
      launch(k_swiglu_parts, dim3(static_cast<unsigned>(cdiv(T * Is, 256))), dim3(256), s, nullptr, ev(5).b,
             static_cast<const float*>(parts), p.sgu_splits, int64_t(T) * 2 * Is, Ti, Is, L, hs);
    } else if (Is && p.sgu_splits > 1) {
      // few tokens: gate and up rows as plain fp32 outputs in sgu_splits
      // reduction parts, then the SwiGLU over the parts added in order
      GemmArgs gs = bf16_gemm_args(x, H / p.sgu_splits, w->shared_w13, 2 * Is, Ti, at<float>(ws, p.sgu_parts),
                                   2 * Is, L);
      gs.lda = gs.ldb = H;
      gs.ksplit = p.sgu_splits;
      gs.split_out = int64_t(T) * 2 * Is;
      gemm<false, GEMM_DOWN_F32, false>(gs, mt, s, Ev{ev(5).a, nullptr});
      launch(k_swiglu_parts, dim3(static_cast<unsigned>(cdiv(T * Is, 256))), dim3(256), s, nullptr, ev(5).b,
             static_cast<const float*>(at<float>(ws, p.sgu_parts)), p.sgu_splits, gs.split_out, Ti, Is, L, hs);
    } else if (Is) {
      gemm<false, GEMM_GATEUP, false>(bf16_gemm_args(x, H, w->shared_w13, Is, Ti, hs, Is, L), mt, s, ev(5));
    }
    if (Is && p.skinny) {
      skinny_gemm(hs, w->shared_w2, H, Is, Ti, ys, s, ev(6));
    } else if (Is && p.sd_splits > 1) {
      // down in sd_splits reduction parts; the combine adds them in order
      GemmArgs gs = bf16_gemm_args(hs, Is / p.sd_splits, w->shared_w2, H, Ti, ys, H, L);
      gs.lda = gs.ldb = Is;
      gs.ksplit = p.sd_splits;
      gs.split_out = int64_t(T) * H;
      gemm<false, GEMM_DOWN_F32, false>(gs, mt, s, ev(6));
    } else if (Is) {
      gemm<false, GEMM_DOWN_F32, false>(bf16_gemm_args(hs, Is, w->shared_w2, H, Ti, ys, H, L), mt, s, ev(6));
    }
    if (!Is) {
      empty_stage(ev(5));
      empty_stage(ev(6));
    }
  } else {
    Groups gr{at<int32_t>(ws, p.g_n), at<int32_t>(ws, p.g_expert), at<int32_t>(ws, p.g_count),
              at<int32_t>(ws, p.g_offset), at<int32_t>(ws, p.g_slots)};
    topk_bucket(E, logits, w->router_bias, Ti, K, rsf, ids, wts, ids_out, w_out, gr, s, ev(1));
    const int groups = static_cast<int>(S < E ? S : E);
    if (Is && p.skinny) {
      float* parts = at<float>(ws, p.sgu_parts);
      skinny_gemm(x, w->shared_w13, 2 * Is, H, Ti, parts, s, Ev{ev(2).a, nullptr});
      launch(k_swiglu_parts, dim3(static_cast<unsigned>(cdiv(T * Is, 256))), dim3(256), s, nullptr, ev(2).b,
             static_cast<const float*>(parts), p.sgu_splits, int64_t(T) * 2 * Is, Ti, Is, L, hs);
    } else if (Is && !fused_k1) {
      gemv<false, GEMV_GATEUP, 1>(bf16_gemv_args(w->shared_w13, Is, H, Ti, x, hs, L), 1, s, ev(2));
    } else {
      empty_stage(ev(2));
    }
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
    gu.wq = codes13(w);
    gu.ws = w->w13_s;
    gu.stride_q = int64_t(2) * I * H / 2;
    gu.stride_s = int64_t(2) * I * H / 16;
    gu.gscale = w->w13_g;
    gu.half_rows = I;
    gu.cols = H;
    gu.in = x;
    gu.out = h;
    // with k_skinny_f4_down the h rows are in group order, else in slot
    // order for the down GEMV
    const bool sk_down = skinny_down_ok(c, T);
    gu.sorted_out = sk_down ? 1 : 0;
    gemv<true, GEMV_GATEUP, 2>(gu, groups, s, ev(3), !w->w13_q);
    if (Is && p.skinny) skinny_gemm(hs, w->shared_w2, H, Is, Ti, ys, s, ev(4));
    else if (Is) gemv<false, GEMV_DOWN_F32, 2>(bf16_gemv_args(w->shared_w2, H, Is, Ti, hs, ys, L), 1, s, ev(4));
    else empty_stage(ev(4));
    GemvArgs gd = r;
    gd.wq = codes2(w);
    gd.ws = w->w2_s;
    gd.stride_q = int64_t(H) * I / 2;
    gd.stride_s = int64_t(H) * I / 16;
    gd.gscale = w->w2_g;
    gd.half_rows = H;
    gd.cols = I;
    gd.in = h;
    gd.out = y;
    if (sk_down) {
      SkinnyF4Args sa{};
      const bool tiled = w->w2_q_tiled && (!w->w2_q || w->w2_s_tiled);
      sa.wq = tiled ? w->w2_q_tiled : w->w2_q;
      sa.ws = w->w2_s;
      sa.stride_q = gd.stride_q;
      sa.stride_s = gd.stride_s;
      sa.gscale = w->w2_g;
      sa.N = H;
      sa.n_groups = gr.n_groups;
      sa.g_expert = gr.expert;
      sa.g_count = gr.count;
      sa.g_offset = gr.offset;
      sa.out_idx = gr.slots;
      sa.in = h;
      sa.out = y;
      skinny_down(sa, I, groups, tiled, s, ev(5));
    } else {
      gemv<true, GEMV_DOWN_F32, 4>(gd, groups, s, ev(5), !w->w2_q);
    }
  }
  const int64_t nq = T * (H / 4);
  const Ev ce = ev(prefill ? 7 : 6);
  const dim3 cgrid(static_cast<unsigned>(cdiv(nq, 256)));
  const float *yc = y, *ysc = ys, *wc = wts;
  if (K <= 4)
    launch(k_combine<4>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out, p.sd_splits);
  else if (K <= 8)
    launch(k_combine<8>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out, p.sd_splits);
  else
    launch(k_combine<MOE_MLP_MAX_TOP_K>, cgrid, dim3(256), s, ce.a, ce.b, yc, ysc, wc, Ti, K, H, out, p.sd_splits);
  return launch_status();
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_MLP_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_MLP_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MOE_MLP_OK;
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

int moe_mlp_decode_noalloc(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x, int64_t T,
                           uint16_t* out, int32_t* ids_out, float* w_out, void* stream) {
  const int st = validate_cfg(cfg, T, 0);
  if (st) return st;
  if (T == 0) return run_layer(cfg, w, x, T, out, ids_out, w_out, nullptr, 0, stream, 0);
  if (make_plan(cfg, T, gemm_form(cfg, T, 0)).total > MOE_MLP_NOALLOC_SCRATCH_BYTES)
    return MOE_MLP_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int sp = scratch_on_device(&ws);
  if (sp) return sp;
  return run_layer(cfg, w, x, T, out, ids_out, w_out, ws, MOE_MLP_NOALLOC_SCRATCH_BYTES, stream, 0);
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
  if (!is_routed(cfg)) return MOE_MLP_ERR_KIND_MISMATCH;
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
    case MOE_MLP_ERR_SCRATCH_LIMIT: return "MOE_MLP_ERR_SCRATCH_LIMIT";
    default: return "MOE_MLP_ERR_UNKNOWN";
  }
}

}  // extern "C"
