// C-ABI entry points declared in include/nvfp4.h.
//
// Every entry point validates its arguments with plain host code first and
// returns a negative status without any HIP call when they are wrong (so
// these paths run, and are tested, without a GPU).  Then it checks that the
// current device is a gfx950 and enqueues kernels on the caller's stream.
// Nothing here allocates, frees or synchronizes.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

namespace {

using namespace nvfp4;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

bool shape_ok_k(int64_t K) { return K >= 32 && K % 32 == 0 && K <= ((int64_t)1 << 24); }
bool shape_ok(int M, int64_t N, int64_t K) {
  return M >= 1 && M <= kMaxTokens && N >= 1 && N <= ((int64_t)1 << 40) && shape_ok_k(K);
}

// Scratch of the entry point that allocates nothing
// (nvfp4_gemv_smallm_noalloc): a file-scope device array, one copy per GPU,
// held until the process ends.  In host code `scratch` is only a handle:
// its device address (per device) comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[64];

// Device address of this device's scratch array (the current device);
// NULL after a HIP error.
void* scratch_for(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Device check, cached per device ordinal (1 = gfx950, 2 = other).
std::atomic<int> g_arch_cache[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NVFP4_ERR_HIP;
  const int slot = dev < 64 ? dev : 63;
  int cached = dev < 64 ? g_arch_cache[slot].load(std::memory_order_relaxed) : 0;
  if (cached == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NVFP4_ERR_HIP;
    cached = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < 64) g_arch_cache[slot].store(cached, std::memory_order_relaxed);
  }
  return cached == 1 ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Largest tensor the rotation-fused quantization reduces in one launch
// (every workgroup rotating the whole tensor for the amax): 32768 elements
// at rot = 16, halved for each doubling of the rotation (graph-replayed
// timings of the decode shapes; above it the amax partials pass is faster).
int64_t rot_self_max_elems(int rot) { return (int64_t)32768 * 16 / rot; }

size_t quant_ws_bytes(int64_t elems, bool two_launch) {
  if (!two_launch) return 0;
  return ((size_t)amax_partial_count(elems) * sizeof(float) + 15) & ~(size_t)15;
}

}  // namespace

extern "C" {

const char* nvfp4_status_str(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE:
      return "NVFP4_ERR_SHAPE: a size is out of range (GEMV and quantization: 1<=M<=128, N>=1, 32<=K<=2^24, "
             "K%32==0, K<=131072 for dynamic per-token scales, M*K<2^30 for a per-tensor scale; sampler: "
             "1<=M<=65535, 1<=N<2^24)";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: a pointer is not aligned (16 bytes; 4 for the sampler)";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace missing or too small";
    case NVFP4_ERR_DEVICE: return "NVFP4_ERR_DEVICE: the current device is not a gfx950";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: a HIP call or kernel launch failed";
    case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG: invalid argument (flags, epilogue, overlapping buffers)";
  }
  return "NVFP4: unknown status";
}

int nvfp4_quantize_act_rotated(const uint16_t* x_bf16, int M, int64_t K, int rot, uint8_t* codes, uint8_t* scales,
                               float* gscale, int flags, void* ws, size_t ws_bytes, void* stream) {
  if (rot != 16 && rot != 32 && rot != 64 && rot != 128) return NVFP4_ERR_ARG;
  if (flags != NVFP4_GS_DYNAMIC && flags != NVFP4_GS_STATIC) return NVFP4_ERR_ARG;
  if (M < 1 || M > kMaxTokens || !shape_ok_k(K) || K % rot != 0) return NVFP4_ERR_SHAPE;
  if (!x_bf16 || !codes || !scales || !gscale) return NVFP4_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
  const int64_t elems = (int64_t)M * K;
  // the quantizer addresses the tensor through a buffer of 2-byte elements
  // with 32-bit byte offsets
  if (elems >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  const bool two = flags == NVFP4_GS_DYNAMIC && elems > rot_self_max_elems(rot);
  const size_t need = flags == NVFP4_GS_DYNAMIC ? quant_ws_bytes(elems, two) : 0;
  if (need > 0 && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return NVFP4_ERR_ALIGN;
  const size_t xb = (size_t)elems * 2, cb = (size_t)elems / 2, sb = (size_t)elems / 16;
  if (overlaps(x_bf16, xb, codes, cb) || overlaps(x_bf16, xb, scales, sb) || overlaps(x_bf16, xb, gscale, 4) ||
      overlaps(codes, cb, scales, sb) || overlaps(codes, cb, gscale, 4) || overlaps(scales, sb, gscale, 4) ||
      (need > 0 && (overlaps(ws, need, x_bf16, xb) || overlaps(ws, need, codes, cb) ||
                    overlaps(ws, need, scales, sb) || overlaps(ws, need, gscale, 4))))
    return NVFP4_ERR_ARG;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  const GsMode mode = flags == NVFP4_GS_STATIC ? GS_STATIC : two ? GS_FROM_PARTIALS : GS_SELF;
  return hip_status(launch_quantize_rotated(x_bf16, elems, rot, codes, scales, gscale, mode,
                                            two ? static_cast<float*>(ws) : nullptr,
                                            two ? amax_partial_count(elems) : 0, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_workspace_size(int op, int M, int64_t N, int64_t K) {
  switch (op) {
    case NVFP4_OP_PACK:
      if (N < 1 || !shape_ok_k(K)) return 0;
      return quant_ws_bytes(N * K, true);
    case NVFP4_OP_QUANT:
      if (M < 1 || M > kMaxTokens || !shape_ok_k(K)) return 0;
      return quant_ws_bytes((int64_t)M * K, (int64_t)M * K > kActSelfAmaxMaxElems);
    case NVFP4_OP_GEMV:
      if (!shape_ok(M, N, K)) return 0;
      return gemv_workspace_bytes(M, N, K, false);
    case NVFP4_OP_GEMV_LMHEAD:
      if (!shape_ok(M, N, K)) return 0;
      return gemv_workspace_bytes(M, N, K, true);
    case NVFP4_OP_QUANT_ROTATED:  // N = the rotation size
      if (M < 1 || M > kMaxTokens || !shape_ok_k(K) || (N != 16 && N != 32 && N != 64 && N != 128)) return 0;
      return quant_ws_bytes((int64_t)M * K, (int64_t)M * K > rot_self_max_elems((int)N));
    case NVFP4_OP_SAMPLE:
      if (M < 1 || M > kSampleMaxM || N < 1 || N > kSampleMaxN) return 0;
      return sample_workspace_bytes(M, N);
  }
  return 0;
}

int nvfp4_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return NVFP4_ERR_NULL;
  if (!aligned16(ws)) return NVFP4_ERR_ALIGN;
  if (ws_bytes % 16 != 0) return NVFP4_ERR_ARG;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  return hip_status(launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

int nvfp4_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                       float* gscale, void* ws, size_t ws_bytes, void* stream) {
  if (N < 1 || !shape_ok_k(K)) return NVFP4_ERR_SHAPE;
  if (!w || !codes || !scales || !gscale) return NVFP4_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_workspace_size(NVFP4_OP_PACK, 0, N, K);
  if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(ws)) return NVFP4_ERR_ALIGN;
  const size_t wb = (size_t)N * K * 4, cb = (size_t)N * K / 2, sb = (size_t)N * K / 16;
  if (overlaps(w, wb, codes, cb) || overlaps(w, wb, scales, sb) || overlaps(w, wb, gscale, 4) ||
      overlaps(codes, cb, scales, sb) || overlaps(codes, cb, gscale, 4) || overlaps(scales, sb, gscale, 4) ||
      overlaps(ws, ws_bytes, w, wb) || overlaps(ws, ws_bytes, codes, cb) || overlaps(ws, ws_bytes, scales, sb) ||
      overlaps(ws, ws_bytes, gscale, 4))
    return NVFP4_ERR_ARG;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  return hip_status(launch_quantize_f32(w, N, K, codes, scales, gscale, static_cast<float*>(ws),
                                        amax_partial_count(N * K), static_cast<hipStream_t>(stream)));
}

int nvfp4_quantize_act(const uint16_t* x_bf16, int M, int64_t K, uint8_t* codes, uint8_t* scales,
                       float* gscale, int flags, void* ws, size_t ws_bytes, void* stream) {
  if (M < 1 || M > kMaxTokens || !shape_ok_k(K)) return NVFP4_ERR_SHAPE;
  if (!x_bf16 || !codes || !scales || !gscale) return NVFP4_ERR_NULL;
  if (flags != NVFP4_GS_DYNAMIC && flags != NVFP4_GS_STATIC && flags != NVFP4_GS_TOKEN_DYNAMIC &&
      flags != NVFP4_GS_TOKEN_STATIC)
    return NVFP4_ERR_ARG;
  const bool per_token = flags == NVFP4_GS_TOKEN_DYNAMIC || flags == NVFP4_GS_TOKEN_STATIC;
  if (flags == NVFP4_GS_TOKEN_DYNAMIC && K > kTokenScaleMaxK) return NVFP4_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
  const int64_t elems = (int64_t)M * K;
  // the quantizer addresses a tensor (per-tensor scale) or a row (per-token)
  // through a buffer of 2-byte elements with 32-bit byte offsets
  if (!per_token && elems >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  const bool two = flags == NVFP4_GS_DYNAMIC && elems > kActSelfAmaxMaxElems;
  const size_t need = quant_ws_bytes(elems, two);
  if (need > 0 && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return NVFP4_ERR_ALIGN;
  const size_t xb = (size_t)elems * 2, cb = (size_t)elems / 2, sb = (size_t)elems / 16;
  const size_t gb = per_token ? (size_t)M * 4 : 4;
  if (overlaps(x_bf16, xb, codes, cb) || overlaps(x_bf16, xb, scales, sb) || overlaps(x_bf16, xb, gscale, gb) ||
      overlaps(codes, cb, scales, sb) || overlaps(codes, cb, gscale, gb) || overlaps(scales, sb, gscale, gb) ||
      (need > 0 && (overlaps(ws, need, x_bf16, xb) || overlaps(ws, need, codes, cb) ||
                    overlaps(ws, need, scales, sb) || overlaps(ws, need, gscale, gb))))
    return NVFP4_ERR_ARG;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  const GsMode mode = flags == NVFP4_GS_STATIC || flags == NVFP4_GS_TOKEN_STATIC ? GS_STATIC
                      : two                                                    ? GS_FROM_PARTIALS
                                                                               : GS_SELF;
  return hip_status(launch_quantize_bf16(x_bf16, M, K, codes, scales, gscale, mode,
                                         two ? static_cast<float*>(ws) : nullptr,
                                         two ? amax_partial_count(elems) : 0, per_token,
                                         static_cast<hipStream_t>(stream)));
}

size_t nvfp4_reset_state_size(int window) {
  if (window < 1 || window > kResetMaxWindow) return 0;
  return reset_state_bytes(window);
}

int nvfp4_reset_state_init(void* state, int M, int window, void* stream) {
  if (M < 1 || M > kMaxTokens) return NVFP4_ERR_SHAPE;
  if (window < 1 || window > kResetMaxWindow) return NVFP4_ERR_ARG;
  if (!state) return NVFP4_ERR_NULL;
  if (!aligned16(state)) return NVFP4_ERR_ALIGN;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  return hip_status(launch_reset_state_init(state, M, window, static_cast<hipStream_t>(stream)));
}

namespace {

// nvfp4_gemv_smallm and its per-token-scale form: a_gscale holds 1 or M floats
int gemv_entry(int M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
               const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
               float* y, const nvfp4_lmhead_epilogue_t* epi, void* ws, size_t ws_bytes, void* stream,
               bool per_token, int64_t ws_cap = kNoWsCap) {
  if (!shape_ok(M, N, K)) return NVFP4_ERR_SHAPE;
  if (!a_codes || !a_scales || !a_gscale || !w_codes || !w_scales || !w_gscale || !y) return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(y))
    return NVFP4_ERR_ALIGN;
  const size_t yb = (size_t)M * N * 4;
  const size_t acb = (size_t)M * K / 2, asb = (size_t)M * K / 16;
  const size_t wcb = (size_t)N * K / 2, wsb = (size_t)N * K / 16;
  const size_t agb = per_token ? (size_t)M * 4 : 4;
  if (overlaps(y, yb, a_codes, acb) || overlaps(y, yb, a_scales, asb) || overlaps(y, yb, a_gscale, agb) ||
      overlaps(y, yb, w_codes, wcb) || overlaps(y, yb, w_scales, wsb) || overlaps(y, yb, w_gscale, 4))
    return NVFP4_ERR_ARG;
  const GemvConfig cfg = choose_gemv_config(M, N, K, epi != nullptr, ws_cap);
  // the epilogue's merge addresses its partials (grid x mt x 16 bytes) with
  // 32-bit buffer offsets
  if (epi && cfg.ws_bytes > (int64_t)0x7FFFFF00) return NVFP4_ERR_SHAPE;
  const size_t need = (size_t)cfg.ws_bytes;
  if (need > 0 && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return NVFP4_ERR_ALIGN;
  if (need > 0 && (overlaps(ws, need, y, yb) || overlaps(ws, need, a_codes, acb) || overlaps(ws, need, a_scales, asb) ||
                   overlaps(ws, need, a_gscale, agb) || overlaps(ws, need, w_codes, wcb) ||
                   overlaps(ws, need, w_scales, wsb) || overlaps(ws, need, w_gscale, 4)))
    return NVFP4_ERR_ARG;
  EpilogueArgs ea{};
  if (epi) {
    if (!epi->step_start || !epi->state || !epi->entropy || !epi->temperature) return NVFP4_ERR_NULL;
    if (epi->window < 1 || epi->window > kResetMaxWindow || (epi->mode < 0 || epi->mode > 2))
      return NVFP4_ERR_ARG;
    if (!aligned16(epi->state)) return NVFP4_ERR_ALIGN;
    const size_t stb = (size_t)M * reset_state_bytes(epi->window);
    if (overlaps(ws, need, epi->state, stb) || overlaps(y, yb, epi->state, stb) ||
        overlaps(y, yb, epi->entropy, (size_t)M * 4) || overlaps(y, yb, epi->temperature, (size_t)M * 4) ||
        overlaps(epi->entropy, (size_t)M * 4, epi->temperature, (size_t)M * 4) ||
        overlaps(epi->state, stb, epi->entropy, (size_t)M * 4) ||
        overlaps(epi->state, stb, epi->temperature, (size_t)M * 4) ||
        overlaps(ws, need, epi->entropy, (size_t)M * 4) || overlaps(ws, need, epi->temperature, (size_t)M * 4))
      return NVFP4_ERR_ARG;
    ea.tau0 = epi->tau0;
    ea.t_low = epi->t_low;
    ea.t_high = epi->t_high;
    ea.t_base = epi->t_base;
    ea.window = epi->window;
    ea.mode = epi->mode;
    ea.step_start = epi->step_start;
    ea.state = epi->state;
    ea.entropy = epi->entropy;
    ea.temperature = epi->temperature;
  }
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  return hip_status(launch_gemv(cfg, M, N, K, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, y,
                                epi ? &ea : nullptr, ws, per_token, static_cast<hipStream_t>(stream)));
}

}  // namespace

int nvfp4_gemv_smallm(int M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                      const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                      const float* w_gscale, float* y, const nvfp4_lmhead_epilogue_t* epi, void* ws,
                      size_t ws_bytes, void* stream) {
  return gemv_entry(M, N, K, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, y, epi, ws, ws_bytes, stream,
                    false);
}

int nvfp4_gemv_smallm_token_scales(int M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                                   const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                                   const float* w_gscale, float* y, const nvfp4_lmhead_epilogue_t* epi, void* ws,
                                   size_t ws_bytes, void* stream) {
  return gemv_entry(M, N, K, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, y, epi, ws, ws_bytes, stream,
                    true);
}

int nvfp4_gemv_smallm_noalloc(int M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_gscale, float* y, const nvfp4_lmhead_epilogue_t* epi, void* stream) {
  // host checks first: shape, then the scratch this shape needs
  if (!shape_ok(M, N, K)) return NVFP4_ERR_SHAPE;
  if (gemv_workspace_bytes(M, N, K, epi != nullptr, kNoAllocScratchBytes) > kNoAllocScratchBytes)
    return NVFP4_ERR_WORKSPACE;
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  void* ws = scratch_for(dev);
  if (!ws) return NVFP4_ERR_HIP;
  return gemv_entry(M, N, K, a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, y, epi, ws,
                    kNoAllocScratchBytes, stream, false, kNoAllocScratchBytes);
}

size_t nvfp4_gemv_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

const char* nvfp4_gemv_variant(int M, int64_t N, int64_t K, int lmhead) {
  if (!shape_ok(M, N, K)) return "invalid shape";
  return gemv_variant_name(choose_gemv_config(M, N, K, lmhead != 0).variant);
}

const char* nvfp4_gemv_variant_name(int index) { return gemv_variant_by_index(index); }

int nvfp4_gemv_tune(const char* variant, int balance) {
  if (balance != 0 && balance != 1) return NVFP4_ERR_ARG;
  return set_gemv_tuning(variant, balance) == 0 ? NVFP4_OK : NVFP4_ERR_ARG;
}

int nvfp4_sample_top_p(int M, int64_t N, const float* logits, const float* temperature, float top_p,
                       const float* uniforms, int32_t* tokens, int32_t* nucleus, void* ws, size_t ws_bytes,
                       void* stream) {
  if (M < 1 || M > kSampleMaxM || N < 1 || N > kSampleMaxN) return NVFP4_ERR_SHAPE;
  if (!logits || !temperature || !uniforms || !tokens) return NVFP4_ERR_NULL;
  if (!aligned4(logits) || !aligned4(temperature) || !aligned4(uniforms) || !aligned4(tokens) ||
      (nucleus && !aligned4(nucleus)))
    return NVFP4_ERR_ALIGN;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return NVFP4_ERR_ARG;
  const size_t need = sample_workspace_bytes(M, N);
  if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(ws)) return NVFP4_ERR_ALIGN;
  const size_t lb = (size_t)M * (size_t)N * 4, vb = (size_t)M * 4;
  const void* outs[3] = {tokens, nucleus, ws};
  const size_t outb[3] = {vb, nucleus ? vb : 0, need};
  for (int k = 0; k < 3; ++k) {
    if (overlaps(outs[k], outb[k], logits, lb) || overlaps(outs[k], outb[k], temperature, vb) ||
        overlaps(outs[k], outb[k], uniforms, vb))
      return NVFP4_ERR_ARG;
    for (int l = k + 1; l < 3; ++l)
      if (overlaps(outs[k], outb[k], outs[l], outb[l])) return NVFP4_ERR_ARG;
  }
  const int d = check_device();
  if (d != NVFP4_OK) return d;
  return hip_status(launch_sample_top_p(M, N, logits, temperature, top_p, uniforms, tokens, nucleus, ws,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
