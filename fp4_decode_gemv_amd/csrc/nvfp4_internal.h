// Host-side declarations shared by the C-ABI layer and the kernel translation
// units.  No device code and no torch types here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// ---------------------------------------------------------------- quantize --

// How the global scale of a quantization is obtained.
enum GsMode : int {
  GS_FROM_PARTIALS = 0,  // reduce per-workgroup amax partials written by amax_partials
  GS_STATIC = 1,         // read *gscale
  GS_SELF = 2            // every workgroup reduces the whole (small) tensor itself
};

// Number of amax partials the two-launch path uses for `elems` elements.
int amax_partial_count(int64_t elems);

// Activation quantization takes one launch up to this many elements (every
// workgroup reduces the whole tensor for the global amax), two launches
// above it (parallel amax partials, then quantize).
constexpr int64_t kActSelfAmaxMaxElems = 131072;

// Launchers (no validation: the C-ABI layer has done it).
hipError_t launch_quantize_bf16(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                                uint8_t* scales, float* gscale, GsMode mode, float* partials,
                                int n_parts, bool per_token, hipStream_t stream);
// largest K of a per-token dynamic quantization (one launch, every
// workgroup of a row reads the whole row for its amax)
constexpr int64_t kTokenScaleMaxK = 131072;
// Rotation-fused quantization (one tensor of `elems` elements, rot = 16, 32,
// 64 or 128; modes GS_SELF up to kActSelfAmaxMaxElems, GS_STATIC,
// GS_FROM_PARTIALS with amax_partial_count(elems) partials)
hipError_t launch_quantize_rotated(const uint16_t* x, int64_t elems, int rot, uint8_t* codes, uint8_t* scales,
                                   float* gscale, GsMode mode, float* partials, int n_parts, hipStream_t stream);
hipError_t launch_quantize_f32(const float* x, int64_t rows, int64_t K, uint8_t* codes,
                               uint8_t* scales, float* gscale, float* partials, int n_parts,
                               hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// -------------------------------------------------------------------- gemv --

// Tokens (M) a GEMV, an activation quantization and a ReSET state set serve
// per call: 1..kMaxTokens.
constexpr int kMaxTokens = 128;

struct EpilogueArgs {
  float tau0, t_low, t_high, t_base;
  int window, mode;
  const uint8_t* step_start;
  void* state;
  float* entropy;
  float* temperature;
};

// Launch configuration of the small-M GEMV, chosen per (M, N, K) on the
// host and fixed for the life of a captured graph.
struct GemvConfig {
  int variant;     // index into the kernel variant table
  int mt;          // compiled token count (1, 2, 4 or 8) >= M
  int g;           // lanes per weight row
  int r;           // rows per lane
  int waves;       // waves per workgroup
  int kp;          // K elements per LDS phase
  int64_t rows_per_wg;
  int64_t grid;       // workgroups (row tiles)
  int64_t lds_bytes;  // dynamic LDS per workgroup
  // workspace layout (byte offset of the epilogue partials) and total size
  // (0 = none needed)
  int64_t ws_bytes;
  int ksplit;  // tiled GEMM: K splits summed by a second launch (1 = none)
};

// ws_cap: the largest workspace the caller can offer (a split-K choice that
// needs more falls back to kernels that need none)
constexpr int64_t kNoWsCap = INT64_MAX;
GemvConfig choose_gemv_config(int M, int64_t N, int64_t K, bool epi, int64_t ws_cap = kNoWsCap);
const char* gemv_variant_name(int variant);
// Tuning override: force a variant by name (NULL or "" = none) and choose
// the MFMA kernels' row mapping (balance 1 = even deal, 0 = whole tiles).
// Returns -1 for an unknown name (nothing changes), else 0.
int set_gemv_tuning(const char* variant, int balance);
const char* gemv_variant_by_index(int index);  // NULL past the end

// Workspace bytes the GEMV needs for this shape (with or without the
// LM-head epilogue); 0 = none.
size_t gemv_workspace_bytes(int M, int64_t N, int64_t K, bool epi, int64_t ws_cap = kNoWsCap);
size_t reset_state_bytes(int window);
constexpr int kResetMaxWindow = 1024;

hipError_t launch_gemv(const GemvConfig& cfg, int M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_gscale, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* w_gscale, float* y,
                       const EpilogueArgs* epi, void* ws, bool per_token, hipStream_t stream);

hipError_t launch_reset_state_init(void* state, int M, int window, hipStream_t stream);

// ----------------------------------------------------------------- sampler --

constexpr int64_t kSampleMaxN = ((int64_t)1 << 24) - 1;  // fixed-point mass sums fit 64 bits
constexpr int kSampleMaxM = 65535;
constexpr int64_t kSampleChunk = 4096;  // elements per workgroup of the wide launches

size_t sample_workspace_bytes(int M, int64_t N);
hipError_t launch_sample_top_p(int M, int64_t N, const float* logits, const float* temperature, float top_p,
                               const float* uniforms, int32_t* tokens, int32_t* nucleus, void* ws,
                               hipStream_t stream);

}  // namespace nvfp4
