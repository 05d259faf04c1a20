/*
 * moe_mlp.h -- C ABI of the MI355X (gfx950) routed MoE MLP library.
 *
 * The layer is the GLM-5.3-Flash MLP of the "Module glm5next_mlp" API page
 * (GLM-5.3-Flash MLP production surface), section "The stack this layer
 * runs".  In a ROUTED layer the token's hidden vector goes through an fp32
 * router projection; the top-k of the router scores picks K experts, each an
 * NVFP4 gate/up projection, clamped SwiGLU and NVFP4 down projection; a BF16
 * shared expert of the same shape runs for every token; the routed outputs,
 * weighted, and the shared output are summed.  A DENSE layer is a single BF16
 * gate/up, clamped SwiGLU, down FFN.
 *
 * The rules of that page's section "Traps this module exists to hold", as
 * implemented here: the SwiGLU clamp is asymmetric (the gate has only an
 * upper bound, the up projection both; the limit is swiglu_limit and is never
 * defaulted); the router's correction bias affects which experts are chosen
 * and nothing else, the weight of a chosen expert being its plain sigmoid
 * score divided by the sum of the chosen plain scores over the full expert
 * count, times routed_scaling_factor; routed_scaling_factor does not touch
 * the shared expert.  Section Constants, KERNEL_MAX_TOP_K: at most 16 experts
 * per token.  The page's "forward" (one-token decode) and
 * "forward_prefill_gemm" (grouped-GEMM prefill) are moe_mlp_decode and
 * moe_mlp_prefill here.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument except `stream` is a DEVICE pointer (HIP device
 *     memory of the current device), unless stated otherwise.  Config and
 *     weight-descriptor structs themselves are HOST memory.
 *   - All tensors are row-major, contiguous, 16-byte aligned.  bf16 values
 *     travel as uint16_t bit patterns.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates, frees or synchronises, keeps no pointer after return
 *     and holds no global state (except the per-device scratch array of
 *     moe_mlp_decode_noalloc); calls are reentrant.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns without waiting.  Device faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and the outputs are untouched.  T == 0 is a
 *     no-op returning MOE_MLP_OK.
 *   - Results are deterministic: the same inputs give the same bits on every
 *     call (no floating-point atomics; fixed summation orders).
 *
 * Storage formats (the page names the routed experts NVFP4 W4A16):
 *   - NVFP4 weight [rows, cols]: codes uint8 [rows, cols/2], the element in
 *     column c is the low nibble of byte c/2 when c is even, the high nibble
 *     when c is odd; each code is an FP4 E2M1 value (OCP Microscaling Formats
 *     v1.0).  Block scales uint8 [rows, cols/16]: one OCP OFP8 E4M3 ("fn")
 *     value per 16 consecutive columns of a row.  W[r][c] = e2m1 * e4m3.
 *     One fp32 global scale per (expert, projection) multiplies the dot
 *     product.
 *   - x, shared/dense weights, the SwiGLU output h and the layer output are
 *     bf16; h is rounded to bf16 (nearest even) before each down projection
 *     and the output once after an fp32 combine.  Router logits, scores and
 *     weights are fp32.
 */
#ifndef MOE_MLP_H
#define MOE_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (return values; 0 = success, negative = error) ---- */
#define MOE_MLP_OK                      0
#define MOE_MLP_ERR_NULL_ARG           -1  /* a required pointer is NULL */
#define MOE_MLP_ERR_BAD_SHAPE          -2  /* H, I, Is or Id not a positive multiple of 32; T < 0;
                                              T above the entry point's maximum */
#define MOE_MLP_ERR_BAD_TOPK           -3  /* top_k < 1, > MOE_MLP_MAX_TOP_K, or > num_experts */
#define MOE_MLP_ERR_BAD_VALUE          -4  /* limit / rsf not finite and > 0; bad kind; E out of range;
                                              n_shared_experts not 0 or 1 */
#define MOE_MLP_ERR_MISALIGNED         -5  /* a device pointer is not 16-byte aligned */
#define MOE_MLP_ERR_WORKSPACE_TOO_SMALL -6 /* ws_bytes below moe_mlp_workspace_size() */
#define MOE_MLP_ERR_KIND_MISMATCH      -7  /* weights missing for the config's kind */
#define MOE_MLP_ERR_HIP                -8  /* a kernel launch failed (hipGetLastError) */
#define MOE_MLP_ERR_SCRATCH_LIMIT      -9  /* moe_mlp_decode_noalloc: the call needs more than
                                              MOE_MLP_NOALLOC_SCRATCH_BYTES of scratch */

#define MOE_MLP_MAX_TOP_K      16    /* Module glm5next_mlp, Constants, KERNEL_MAX_TOP_K */
#define MOE_MLP_MAX_EXPERTS    1024  /* one wavefront holds at most 16 scores per lane */
#define MOE_MLP_DECODE_MAX_T   256   /* moe_mlp_decode handles up to this many tokens */
#define MOE_MLP_NOALLOC_SCRATCH_BYTES (64u << 20)   /* scratch of moe_mlp_decode_noalloc, per device */

#define MOE_MLP_KIND_ROUTED 0   /* router + routed NVFP4 experts + optional shared expert */
#define MOE_MLP_KIND_DENSE  1   /* dense BF16 FFN (layers before first_k_dense_replace) */
#define MOE_MLP_KIND_ROUTED_FP8 2 /* router + routed FP8 block-scaled experts + optional shared expert
                                     (H and I multiples of MOE_MLP_FP8_BLOCK) */
#define MOE_MLP_FP8_BLOCK   128 /* FP8 expert weights: one fp32 scale per 128 x 128 block */

/*
 * Layer geometry and constants.  Every field is read from the caller; none
 * has a default (Module glm5next_mlp, Structs: the config comes from the
 * checkpoint's own config and is never filled in by the library).
 */
typedef struct moe_mlp_config {
  int32_t kind;                  /* MOE_MLP_KIND_ROUTED, _DENSE or _ROUTED_FP8 */
  int32_t hidden;                /* H; multiple of 32 */
  int32_t moe_intermediate;      /* I, routed experts; multiple of 32 (ROUTED) */
  int32_t num_experts;           /* E, the FULL expert count; 1..MOE_MLP_MAX_EXPERTS (ROUTED) */
  int32_t top_k;                 /* K; 1..min(MOE_MLP_MAX_TOP_K, E) (ROUTED) */
  int32_t n_shared_experts;      /* 0 or 1 (ROUTED) */
  int32_t shared_intermediate;   /* Is; multiple of 32 when n_shared_experts == 1 */
  int32_t dense_intermediate;    /* Id; multiple of 32 (DENSE) */
  float   routed_scaling_factor; /* finite, > 0 (ROUTED); multiplies the top-k weights only */
  float   swiglu_limit;          /* L; finite, > 0 */
} moe_mlp_config;

/*
 * Weight contract for one layer (all device pointers, caller-owned).
 * Fields that the config's kind does not use may be NULL.
 */
typedef struct moe_mlp_weights {
  const float*    router_w;     /* [E, H] fp32 gate.weight */
  const float*    router_bias;  /* [E] fp32 correction bias (selection only) */
  const uint8_t*  w13_q;        /* [E, 2I, H/2] NVFP4 codes; rows [0,I) gate, [I,2I) up */
  const uint8_t*  w13_s;        /* [E, 2I, H/16] E4M3 block scales */
  const float*    w13_g;        /* [E, 2] fp32 global scales (gate, up) */
  const uint8_t*  w2_q;         /* [E, H, I/2] NVFP4 codes of the down projection */
  const uint8_t*  w2_s;         /* [E, H, I/16] E4M3 block scales */
  const float*    w2_g;         /* [E] fp32 global scale of the down projection */
  const uint16_t* shared_w13;   /* [2 Is, H] bf16: gate rows then up rows */
  const uint16_t* shared_w2;    /* [H, Is] bf16 */
  const uint16_t* dense_w13;    /* [2 Id, H] bf16: gate rows then up rows (DENSE) */
  const uint16_t* dense_w2;     /* [H, Id] bf16 (DENSE) */
  /* Optional (NULL = not given): the routed codes and scales again, in the
   * tile layout of moe_nvfp4_tile_pack (same sizes as the row-major arrays).
   * When a projection's codes AND scales are given, the grouped-GEMM form
   * (moe_mlp_prefill, decode from 64 tokens) reads them instead of the
   * row-major arrays wherever its NVFP4 tile kernel runs, and so does the
   * few-token MFMA down projection of decode batches (5..256 tokens); the
   * values and the arithmetic are the same, so the results are bitwise the
   * same.
   * One resident copy of the codes: a projection's row-major codes (w13_q,
   * w2_q) may be NULL when its tile-layout codes and scales are given; every
   * kernel then reads the tile-layout codes (the decode forms with the
   * row-major scales, which stay required), with bitwise the same results.
   * This takes a reduction length (H for gate/up, I for down) that is a
   * multiple of 256 and at least 512, and for the grouped-GEMM form T*H*2 and
   * T*K*I*2 below 2^31 (else MOE_MLP_ERR_BAD_SHAPE). */
  const uint8_t*  w13_q_tiled;  /* moe_nvfp4_tile_pack(w13_q, w13_s, E, 2I, H, ...) codes */
  const uint8_t*  w13_s_tiled;  /* ... and scales */
  const uint8_t*  w2_q_tiled;   /* moe_nvfp4_tile_pack(w2_q, w2_s, E, H, I, ...) codes */
  const uint8_t*  w2_s_tiled;   /* ... and scales */
  /* MOE_MLP_KIND_ROUTED_FP8 experts (the FP8 checkpoint named on the
   * TensorRT-LLM page "Add GLM-5.3-Flash (glm5_next) support"; NULL for the
   * other kinds): OCP E4M3 ("fn") bytes [out, in] row-major and one fp32
   * scale per 128 x 128 block, W = e4m3 * scale; no global scale (w13_g /
   * w2_g and the NVFP4 fields are not read). */
  const uint8_t*  w13_f8;       /* [E, 2I, H] E4M3; rows [0,I) gate, [I,2I) up */
  const float*    w13_f8_scale; /* [E, 2I/128, H/128] fp32 */
  const uint8_t*  w2_f8;        /* [E, H, I] E4M3 */
  const float*    w2_f8_scale;  /* [E, H/128, I/128] fp32 */
} moe_mlp_weights;

/*
 * Workspace bytes that moe_mlp_decode (prefill == 0) or moe_mlp_prefill
 * (prefill != 0) needs for T tokens.  `bytes` is a HOST pointer.  The
 * workspace holds logits, routing, expert-sorted indices and intermediate
 * activations; its contents need no initialisation and are garbage after a
 * call.  Validates cfg like the compute calls (T limit included).
 */
int moe_mlp_workspace_size(const moe_mlp_config* cfg, int64_t T, int prefill, size_t* bytes);

/*
 * Decode form ("forward": the page's one-token decode), for 1..MOE_MLP_DECODE_MAX_T
 * tokens.  Up to 63 tokens the routed experts stream the NVFP4 codes once
 * per touched expert: 1..4 tokens (the MTP verify shapes) in three fused
 * launches of W4A16 GEMVs; 5..63 tokens with W4A16 GEMVs for gate/up and,
 * when I is a multiple of 512 up to 2048 and H of 64, an MFMA down
 * projection that dequantises each weight once for all of an expert's
 * tokens.  From 64 tokens on, the call runs the kernels of moe_mlp_prefill
 * (faster there; up to 256 tokens with the same MFMA down projection; the
 * workspace size and stage list follow).
 *   x        [T, H] bf16 input.
 *   out      [T, H] bf16 output.
 *   ids_out  [T, K] int32 chosen expert ids, descending biased score
 *            (exact ties: lower id first); may be NULL.  ROUTED only.
 *   w_out    [T, K] fp32 routing weights, same order; may be NULL.
 *   workspace/ws_bytes: device scratch of at least moe_mlp_workspace_size(cfg, T, 0).
 *   stream   hipStream_t (NULL = default stream).
 */
int moe_mlp_decode(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x,
                   int64_t T, uint16_t* out, int32_t* ids_out, float* w_out,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_mlp_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a device array
 * of MOE_MLP_NOALLOC_SCRATCH_BYTES that the library's code object holds on
 * every GPU it runs on, from the first call there until the process ends
 * (its device address is looked up once per device, with that device
 * current).  The call itself allocates and frees nothing.  The caller still
 * passes x, out, ids_out, w_out (as moe_mlp_decode) and enqueues on `stream`
 * of the current device.  Returns MOE_MLP_ERR_SCRATCH_LIMIT, before anything
 * is enqueued, when moe_mlp_workspace_size(cfg, T, 0) exceeds the array
 * (at H=4096, I=Is=1536, E=288, K=8: up to about 100 tokens fit).  Every call
 * on one GPU uses that GPU's one array, which keeps the last call's contents
 * (the kernels never read scratch they have not written in the same call):
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.
 */
int moe_mlp_decode_noalloc(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x,
                           int64_t T, uint16_t* out, int32_t* ids_out, float* w_out, void* stream);

/*
 * Prefill form ("forward_prefill_gemm": the page's grouped-GEMM prefill),
 * any T >= 1 (bounded by INT32 index range: T * K < 2^31).  Tokens are
 * sorted by expert id, each expert's rows run through a grouped GEMM that
 * dequantises NVFP4 into bf16 MFMA operands, then are un-permuted and
 * combined with the shared expert.  Arguments as moe_mlp_decode, with the
 * workspace sized by moe_mlp_workspace_size(cfg, T, 1).
 */
int moe_mlp_prefill(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x,
                    int64_t T, uint16_t* out, int32_t* ids_out, float* w_out,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * Measurement entry: exactly the kernels of moe_mlp_decode (prefill == 0) or
 * moe_mlp_prefill (prefill != 0) on `stream`, with stage i's start event
 * events[2i] attached to the dispatch of the stage's first kernel and its
 * stop event events[2i+1] to the completion of its last kernel
 * (hipExtLaunchKernelGGL), so hipEventElapsedTime(events[2i], events[2i+1])
 * is the stage's kernel execution time as a kernel trace reports it.
 * `events` is a HOST array of n_events caller-created hipEvent_t handles
 * (none NULL); n_events >= 2 * n_stages, else MOE_MLP_ERR_BAD_VALUE.
 * Stages (moe_mlp_stage_name): ROUTED decode of 1..4 tokens (T*K <= 64,
 * H <= 4096, I and Is <= 2048) logits_shared_gateup, routed_gateup,
 * shared_routed_down_combine; other ROUTED decode below 64 tokens router_logits,
 * topk_bucket, shared_gateup, routed_gateup, shared_down, routed_down,
 * combine; ROUTED prefill (and decode from 64 tokens) router_logits, topk,
 * permute, routed_gateup, routed_down, shared_gateup, shared_down, combine;
 * DENSE dense_gateup, dense_down.  A stage with
 * nothing to run records both events back to back: no shared expert, or
 * (decode of T <= 16 tokens, H <= 4096, Is <= 2048) shared_gateup, whose
 * work runs inside router_logits.
 */
int moe_mlp_forward_profiled(const moe_mlp_config* cfg, const moe_mlp_weights* w, const uint16_t* x,
                             int64_t T, uint16_t* out, int32_t* ids_out, float* w_out, void* workspace,
                             size_t ws_bytes, void* stream, int prefill, void* const* events, int n_events);

/* Name of stage `stage` of the decode (prefill == 0) or prefill form for the
 * config and token count T (static string), or NULL past the last stage. */
const char* moe_mlp_stage_name(const moe_mlp_config* cfg, int64_t T, int prefill, int stage);

/*
 * Router alone (test entry; Module glm5next_mlp, "The stack this layer runs":
 * gate.weight -> fp32 logits -> router_topk -> ids[K], weights[K], with the
 * selection and weight rules of "Traps this module exists to hold"):
 * logits = x . router_w^T (fp32), sigmoid scores, top-K of score + bias,
 * weights = rsf * score / sum of chosen scores.
 * Uses the routed config fields hidden, num_experts, top_k and
 * routed_scaling_factor (kind ROUTED or ROUTED_FP8).  ids [T, K] int32, w [T, K] fp32 (both required).
 * Workspace: moe_mlp_workspace_size(cfg, T, 1) bytes (prefill sizing).
 */
int moe_router_topk(const moe_mlp_config* cfg, const float* router_w, const float* router_bias,
                     const uint16_t* x, int64_t T, int32_t* ids, float* w,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * NVFP4 dequantisation (test entry; Module glm5next_mlp, "The stack this
 * layer runs": the routed experts' NVFP4 gate/up and down weights; element
 * and scale formats of the OCP MX v1.0 and OFP8 specifications), the same
 * device routines the GEMV and grouped GEMM use:
 * out[r][c] = global * e2m1(code[r][c]) * e4m3(scale[r][c/16]).
 *   q [rows, cols/2], s [rows, cols/16]; cols a positive multiple of 32.
 *   out_f32 [rows, cols] fp32 and/or out_bf16 [rows, cols] bf16 (RNE); at
 *   least one non-NULL.  With global == 1 both outputs are exact.
 */
int moe_nvfp4_dequant(const uint8_t* q, const uint8_t* s, float global, int64_t rows,
                      int64_t cols, float* out_f32, uint16_t* out_bf16, void* stream);

/*
 * NVFP4 weights (Module glm5next_mlp, the NVFP4 expert weights: E2M1 codes and
 * one E4M3 scale per 16 columns of a row) copied from the row-major layout
 * into the tile layout that the grouped GEMM's loads read in whole 128-byte
 * lines: `mats` matrices of [rows, cols], codes q [mats, rows, cols/2] and
 * scales s [mats, rows, cols/16] -> q_tiled and s_tiled of the same sizes
 * (device pointers, 16-byte aligned, caller-owned; the inputs are only
 * read).  Done once when the weights are loaded.
 *   q_tiled: for matrix m, 16-row group r and 128-column unit u, a 1024-byte
 *     block at ((m * rows/16 + r) * cols/128 + u) * 1024 whose 16-byte piece
 *     L (0..63) is bytes 64u + 16 ((L % 4) ^ z(L / 4)) .. +15 of the codes of
 *     row 16r + L/4, with z(i) = ((i >> 1) & 3) ^ ((i >> 3) & 1) (the XOR
 *     swizzle of the kernel's LDS layout).
 *   s_tiled: for matrix m, 32-row group r and 256-column unit v, a 512-byte
 *     block at ((m * rows/32 + r) * cols/256 + v) * 512, stage-major: bytes
 *     128 t + 4 l .. +3 of the block are scale bytes 16v + 4t .. +3 of row
 *     32r + l (t = 0..3, the four 64-column stages of the unit; l = 0..31).
 * rows a multiple of 32, cols a multiple of 256 (BAD_SHAPE otherwise);
 * mats >= 0.  Stream-ordered; no allocation.
 */
int moe_nvfp4_tile_pack(const uint8_t* q, const uint8_t* s, int64_t mats, int64_t rows, int64_t cols,
                        uint8_t* q_tiled, uint8_t* s_tiled, void* stream);

/* Human-readable name of a status code (static string; never NULL). */
const char* moe_mlp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MLP_H */
