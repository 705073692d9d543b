/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 small-M decode projection.
 *
 * The operation (ReSET project page, "Core contribution -- the nvfp4r
 * CUDA-core kernel"): y = A . W^T for a small number M (1..8 on the pages;
 * up to 128 here) of active decode tokens, where both the activation A [M][K]
 * and the weight W [N][K]
 * are NVFP4 tensors (ReSET reading notes, section 2.1 and section 6.1):
 *
 *   - every element is a 4-bit E2M1 float, two per byte, element 2j in the
 *     low nibble of byte j;
 *   - each run of 16 consecutive elements of a row shares one FP8 E4M3
 *     block scale; scales are stored row-major [rows][K/16], not interleaved
 *     (reading notes, section 5.3 and its Table 3);
 *   - the tensor carries one FP32 global scale;
 *   - value = E2M1(code) * E4M3(block scale) * global scale.
 *
 * The activation is quantized on the fly, once per layer, by its own call
 * (the "Q" step, reading notes section 5.3); weights are packed once,
 * offline.  The quantization recipe (global scale amax / (6*448), block
 * scale RNE to E4M3 with saturation at 448, element RNE to E2M1 with
 * saturation at 6, ties to the even code) is fixed and bit-reproducible.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates and frees nothing.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  No call synchronizes, so every call
 *     can be captured into a hipGraph.
 *   - Arguments are validated on the host BEFORE any HIP call.  A negative
 *     status means nothing was launched and no output was touched.
 *   - Device pointers must be 16-byte aligned (NVFP4_ERR_ALIGN otherwise),
 *     except scalars (global scales, entropy/temperature outputs, flags)
 *     and the sampler's arrays (4 bytes).
 *   - Shapes: 1 <= M <= 128, N >= 1, 32 <= K <= 2^24, K % 32 == 0 (the
 *     sampler: 1 <= M <= 65535, 1 <= N < 2^24).
 *   - Outputs must not overlap inputs (NVFP4_ERR_ARG).
 *   - Non-finite inputs give undefined (but memory-safe) results.
 *   - Workspace `ws` is caller-owned device scratch of at least
 *     nvfp4_workspace_size(op, M, N, K) bytes; it must be zero-filled once
 *     after allocation (nvfp4_workspace_init does that with a kernel).
 *     It holds per-call intermediates, plus (the LM-head epilogue) one
 *     ticket counter per token at its start that every call leaves at zero,
 *     so graph replays are safe and no call needs the workspace cleared
 *     again.  Calls that share one workspace must be ordered on one stream;
 *     a call whose kernels did not run to completion can leave a ticket
 *     non-zero, and the workspace must then be zero-filled again.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,      /* a required pointer is NULL                     */
  NVFP4_ERR_SHAPE = -2,     /* M not in [1,128], N < 1, K outside [32, 2^24]
                               or K % 32 != 0 (K > 131072 for dynamic
                               per-token scales; M x K >= 2^30 for the
                               per-tensor quantization); with the LM-head epilogue also an
                               N whose workspace would pass 2 GB (N beyond
                               about 10^8); sampler sizes out of range        */
  NVFP4_ERR_ALIGN = -3,     /* a tensor pointer is not 16-byte aligned (the
                               sampler's: not 4-byte aligned)                 */
  NVFP4_ERR_WORKSPACE = -4, /* ws is NULL or ws_bytes is too small             */
  NVFP4_ERR_DEVICE = -5,    /* the current HIP device is not a gfx950         */
  NVFP4_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed     */
  NVFP4_ERR_ARG = -7        /* other bad argument: flags, epilogue parameters,
                               overlapping input/output buffers               */
} nvfp4_status_t;

/* nvfp4_quantize_act flags: one activation global scale per tensor, or one
   per token (row) */
enum { NVFP4_GS_DYNAMIC = 0, NVFP4_GS_STATIC = 1, NVFP4_GS_TOKEN_DYNAMIC = 2, NVFP4_GS_TOKEN_STATIC = 3 };

/* ops for nvfp4_workspace_size */
enum {
  NVFP4_OP_PACK = 0, NVFP4_OP_QUANT = 1, NVFP4_OP_GEMV = 2, NVFP4_OP_GEMV_LMHEAD = 3, NVFP4_OP_SAMPLE = 4,
  NVFP4_OP_QUANT_ROTATED = 5
};

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_str(int status);

/* Bytes of workspace the op needs for this shape (0 = none; M is ignored
 * for NVFP4_OP_PACK, where N x K is the weight; K is ignored for
 * NVFP4_OP_SAMPLE, where N is the vocabulary; for NVFP4_OP_QUANT_ROTATED, N
 * is the rotation size).  Pure host function. */
size_t nvfp4_workspace_size(int op, int M, int64_t N, int64_t K);

/* Zero-fill a workspace with a kernel on `stream` (graph-capturable; no
 * hipMemset).  ws must be 16-byte aligned; ws_bytes % 16 == 0. */
int nvfp4_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Offline weight packing: W fp32 [N][K] -> codes u8 [N][K/2], E4M3 block
 * scales u8 [N][K/16], global scale fp32 [1] (= amax(|W|) / 2688).
 * The packed bytes are bit-identical to the reference recipe.  Needs
 * nvfp4_workspace_size(NVFP4_OP_PACK, 0, N, K) bytes of ws.  1 <= N,
 * K >= 32, K % 32 == 0 (M limits do not apply).
 */
int nvfp4_pack_weights(const float* w, int64_t N, int64_t K,
                       uint8_t* codes, uint8_t* scales, float* gscale,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * On-the-fly activation quantization, the per-layer "Q" step (reading
 * notes, section 5.3): x bf16 [M][K] (raw bit patterns) -> codes u8
 * [M][K/2], scales u8 [M][K/16] and the global scale.
 *   flags = NVFP4_GS_DYNAMIC: *gscale (device) is WRITTEN with
 *           amax over all M x K elements / 2688 (one scale per tensor, so a
 *           row's codes depend on the other rows); M x K < 2^30;
 *   flags = NVFP4_GS_STATIC:  *gscale (device) is READ (a calibrated
 *           scale); rows are then independent; M x K < 2^30;
 *   flags = NVFP4_GS_TOKEN_DYNAMIC: gscale[M] (device) is WRITTEN, row m's
 *           scale being the amax over that row alone / 2688 (the recipe
 *           applied to each row as its own tensor; K <= 131072).  Rows are
 *           independent and the quantization is one launch at every M.
 *   flags = NVFP4_GS_TOKEN_STATIC: gscale[M] (device) is READ.
 *   Per-token scales go with nvfp4_gemv_smallm_token_scales.
 * Codes, scales and gscale are bit-identical to the reference recipe.
 * Workspace: nvfp4_workspace_size(NVFP4_OP_QUANT, M, 0, K) bytes (may be 0;
 * ws may then be NULL).
 */
int nvfp4_quantize_act(const uint16_t* x_bf16, int M, int64_t K,
                       uint8_t* codes, uint8_t* scales, float* gscale,
                       int flags, void* ws, size_t ws_bytes, void* stream);

/*
 * Rotation-fused activation quantization "Q+R", a comparison point (reading
 * notes, section 5.3 and Table 3: rotation-based NVFP4 pipelines rotate
 * each layer's activation before quantizing it, at about 2.3x the cost of
 * the plain Q step on the pages' GPU).  Each run of `rot` consecutive
 * elements of a row (rot = 16, 32, 64 or 128; K % rot == 0) is multiplied
 * by the normalized Walsh-Hadamard matrix H_rot / sqrt(rot) (Sylvester
 * order), computed in float32 by butterfly stages h = 1, 2, ..., rot/2, each
 * pair (i, i + h) becoming (a + b, a - b), then one multiply by the float32
 * nearest to 1/sqrt(rot); the rotated tensor is then quantized exactly as
 * nvfp4_quantize_act does (its amax sets the dynamic global scale).
 * flags: NVFP4_GS_DYNAMIC or NVFP4_GS_STATIC (per-token flags:
 * NVFP4_ERR_ARG).  A projection on such an activation needs weights rotated
 * the same way before packing: (A Q)(W Q)^T = A W^T for the orthogonal Q.
 * Same shapes (M x K < 2^30), outputs and errors as nvfp4_quantize_act;
 * workspace: nvfp4_workspace_size(NVFP4_OP_QUANT_ROTATED, M, rot, K) bytes
 * (may be 0; ws may then be NULL); rot not in {16, 32, 64, 128}: NVFP4_ERR_ARG;
 * K % rot != 0: NVFP4_ERR_SHAPE.  Codes, scales and gscale are
 * bit-identical to the oracle's rotation followed by the recipe.
 */
int nvfp4_quantize_act_rotated(const uint16_t* x_bf16, int M, int64_t K, int rot,
                               uint8_t* codes, uint8_t* scales, float* gscale,
                               int flags, void* ws, size_t ws_bytes, void* stream);

/*
 * ReSET per-sequence state, device resident (ReSET reading notes, sections
 * 4.1 and 4.2): running sum and count of all entropies so far, running sum
 * and length of the current reasoning step, and a ring of the last `window`
 * entropies.  Opaque; nvfp4_reset_state_size(window) bytes per sequence
 * (a multiple of 16), M sequences stored back to back.  1 <= window <= 1024.
 */
size_t nvfp4_reset_state_size(int window);
int nvfp4_reset_state_init(void* state, int M, int window, void* stream);

/*
 * Optional fused LM-head epilogue (ReSET project page, "Step-aware
 * temperature scaling"; reading notes sections 3.1, 4.1-4.3): after the
 * GEMV produced the logits y [M][N], compute per token the softmax entropy
 * H_t (natural log, temperature 1, all N logits) and the ReSET temperature:
 *   update the sequence state with H_t (a position flagged step_start[m]=1
 *   begins a new step; the first call after init always does);
 *   Hbar = mean of all entropies so far;
 *   Hstep = mean of the last min(window, count) entropies while the current
 *           step is at most `window` positions long, else the step's mean;
 *   tau   = Hstep if Hstep > Hbar (uncertain step) else tau0;
 *   T     = t_low if H_t < tau else t_high      (mode 0, ReSET)
 *   T     = t_base                              (mode 1, ReSET off)
 *   T     = t_low if H_t < tau0 else t_high     (mode 2, the fixed-threshold
 *           rule of the reading notes, section 3.1, formula (1): the
 *           token-level baseline ReSET improves on).
 * The state is updated in every mode, so a sequence may switch modes.
 * Any other mode is NVFP4_ERR_ARG.
 */
typedef struct {
  float tau0, t_low, t_high, t_base;
  int window;                 /* must equal the window the states were initialised with */
  int mode;                   /* 0 = ReSET, 1 = BASE, 2 = fixed threshold tau0           */
  const uint8_t* step_start;  /* [M] device: 1 = this position starts a new step          */
  void* state;                /* [M] device states (nvfp4_reset_state_size(window) each) */
  float* entropy;             /* [M] device out, nats                                    */
  float* temperature;         /* [M] device out                                          */
} nvfp4_lmhead_epilogue_t;

/*
 * y [M][N] fp32 = dequant(A) . dequant(W)^T, the small-M decode projection.
 * A is (a_codes [M][K/2], a_scales [M][K/16], *a_gscale), W is (w_codes
 * [N][K/2], w_scales [N][K/16], *w_gscale); both global scales are device
 * pointers.  Each weight byte is read from HBM once for all M tokens.
 * Result: within |y - y_exact| <= 1e-5 * sum_k |a_k w_k| of the exact real
 * dot product of the dequantized rows; repeated calls give identical bits.
 * Workspace: nvfp4_workspace_size(NVFP4_OP_GEMV, M, N, K) bytes for the
 *   plain projection (0 for shapes served without splitting K; ws may then
 *   be NULL) and nvfp4_workspace_size(NVFP4_OP_GEMV_LMHEAD, M, N, K) bytes
 *   with the epilogue, zero-filled once after allocation.
 * epi == NULL: plain projection.
 * epi != NULL: LM-head epilogue as above.
 */
int nvfp4_gemv_smallm(int M, int64_t N, int64_t K,
                      const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                      float* y, const nvfp4_lmhead_epilogue_t* epi,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_gemv_smallm for an activation quantized with one global scale per
 * token (NVFP4_GS_TOKEN_*): a_gscale points to M floats (device) and output
 * row m is scaled by a_gscale[m] * (*w_gscale).  This is one of the ways to
 * shorten the separate "Q" step (reading notes, section 5.3): no tensor-wide
 * amax has to finish before any row is quantized.  Everything else,
 * including the epilogue, workspace and error behaviour, is as for
 * nvfp4_gemv_smallm, with the same kernels.
 */
int nvfp4_gemv_smallm_token_scales(int M, int64_t N, int64_t K,
                                   const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                                   const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                                   float* y, const nvfp4_lmhead_epilogue_t* epi,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_gemv_smallm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same operation, kernels, arguments and errors, without a
 * workspace argument.  The workspace (the LM-head epilogue's partials, or
 * the partial sums of a projection whose K is split over workgroups; other
 * plain projections need none) lives in a static device array of
 * nvfp4_gemv_noalloc_scratch_bytes() = 16 MiB that each GPU the library runs
 * on holds until the process ends; nothing is allocated or freed by the
 * call.  Shapes whose workspace would exceed it (the LM-head epilogue at
 * about N * M > 10^7, e.g. M = 128 with N > 130000) return
 * NVFP4_ERR_WORKSPACE before any HIP call; a plain projection whose K split
 * would not fit is served by a kernel that needs no workspace (its outputs
 * may then differ from nvfp4_gemv_smallm's in rounding, within the same
 * tolerance).  Every call on one GPU shares
 * that GPU's array: calls that can overlap on one GPU (different streams
 * without ordering, or threads) race and give undefined results; calls on
 * one stream are ordered.  The array keeps the last call's contents; no
 * call depends on them (every partial is written before it is read) except
 * the epilogue's per-token ticket counters, which start at zero with the
 * array and which every completed call leaves at zero.
 */
int nvfp4_gemv_smallm_noalloc(int M, int64_t N, int64_t K,
                              const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                              float* y, const nvfp4_lmhead_epilogue_t* epi, void* stream);

/* Bytes of the static scratch array of nvfp4_gemv_smallm_noalloc. */
size_t nvfp4_gemv_noalloc_scratch_bytes(void);

/*
 * Name of the kernel variant nvfp4_gemv_smallm launches for this shape
 * (lmhead != 0: with the epilogue).  Static string; pure host function.
 * The launch table is chosen per (M, N, K) on the host, like the pages'
 * runtime dispatch (reading notes, section 5.2), and is fixed for the life
 * of the process, so a captured graph replays the same kernels.
 */
const char* nvfp4_gemv_variant(int M, int64_t N, int64_t K, int lmhead);

/*
 * Top-p (nucleus) sampling of one token per sequence from the logits
 * [M][N] fp32 (row-major, e.g. the y of an LM-head nvfp4_gemv_smallm), at
 * the per-sequence temperature temperature[M] (e.g. the epilogue's output).
 * The decode loop of the ReSET reading notes samples with top-p = 0.95
 * (section 6.1) at the temperature chosen per token (section 4.3); nucleus
 * sampling as published by Holtzman et al. (ICLR 2020):
 *   p = softmax(z / T); order = decreasing logit, equal logits by
 *   increasing index; the nucleus is the shortest prefix of the order whose
 *   mass is >= top_p; the token is the first of the order whose cumulative
 *   mass exceeds u * (nucleus mass), with u = uniforms[m] in [0, 1) drawn
 *   by the caller (values outside are clamped into it).
 * Out: tokens[M] int32; nucleus[M] int32 = nucleus size (may be NULL).
 * Probabilities are float32 exponentials summed in 2^-40 fixed point, so the
 * cut points agree with exact arithmetic to within a few 1e-6 of the row's
 * mass; repeated calls give identical tokens.  Logits must be finite; a row
 * whose temperature is not positive and finite gets token -1, nucleus 0.
 * Array pointers are device pointers, 4-byte aligned.  Workspace: ws (16-byte
 * aligned) of nvfp4_workspace_size(NVFP4_OP_SAMPLE, M, N, 0) bytes; it
 * needs no zero-fill (every call clears what it accumulates into) and holds
 * nothing between calls.  Outputs and ws must not overlap inputs or each
 * other.  Four launches on `stream`; a row whose nucleus lies among its
 * elements within 2^-20 of a chunk maximum's probability (a peaked
 * distribution) is drawn at the start of the second, and the rest of the
 * work is skipped for it.
 * Errors: NVFP4_ERR_SHAPE (M outside [1, 65535], N outside [1, 2^24 - 1]),
 * NVFP4_ERR_NULL, NVFP4_ERR_ALIGN, NVFP4_ERR_WORKSPACE, NVFP4_ERR_ARG
 * (top_p outside (0, 1], overlap), NVFP4_ERR_DEVICE, NVFP4_ERR_HIP.
 */
int nvfp4_sample_top_p(int M, int64_t N, const float* logits, const float* temperature, float top_p,
                       const float* uniforms, int32_t* tokens, int32_t* nucleus, void* ws, size_t ws_bytes,
                       void* stream);

/* Name of compiled kernel variant `index` (0-based), NULL past the end. */
const char* nvfp4_gemv_variant_name(int index);

/*
 * Tuning and test hook, process-wide: nvfp4_gemv_smallm (and
 * nvfp4_workspace_size, nvfp4_gemv_variant) use the compiled variant named
 * `variant` for every M its token count covers and every shape it fits
 * (NULL or "" = the launch table's choice).  balance = 1 (the default)
 * deals the rows of small-N shapes out evenly over the CUs in the MFMA tile
 * kernels; balance = 0 keeps whole tiles (16-, 8- or 4-row groups times the
 * kernel's group count).  Both change
 * workspace sizes, which must be queried again.  Not for use while another
 * thread launches GEMVs.  Errors: NVFP4_ERR_ARG (unknown name, balance not
 * 0 or 1; nothing changes).
 */
int nvfp4_gemv_tune(const char* variant, int balance);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
