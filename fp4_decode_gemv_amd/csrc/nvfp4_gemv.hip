// Small-M NVFP4 GEMV for gfx950 (CDNA4), y[M][N] = A[M][K] . W[N][K]^T.
//
// What the method asks for (ReSET project page, "Core contribution -- the
// nvfp4r CUDA-core kernel", C1-C3; reading notes section 5.2): every weight
// tile streamed from HBM once for all M tokens (C1), several independent
// accumulator chains per thread (C2), FP4 unpacked in registers and fed
// straight to the multiply-adds (C3).  The pages' design targets Blackwell
// CUDA cores; two CDNA4 forms of it live here, and the launch table picks
// one per (M, N, K) from measured latency, fixed for the life of a captured
// graph (reading notes section 5.2, runtime dispatch):
//
// Direct VALU kernel (gemv_direct_kernel), for M <= 2
//   * G consecutive lanes of a wave64 share one weight row; each lane loads
//     16 bytes (32 codes = 2 blocks) per step with one dwordx4 load; R rows
//     per lane give R*M independent accumulator chains; a P-deep register
//     ring keeps loads in flight.  No LDS and no barrier: every lane loads
//     the activation codes and scales of its own K positions straight from
//     L1/L2 (the activation is a few KB and shared by every workgroup) and
//     decodes them in registers once for its R rows.
//   * E2M1 codes become f16 with v_cvt_scalef32_pk_f16_fp4 (scale 1.0: the
//     instruction applies only the exponent of its scale operand).  Per
//     16-element block and token, 8 v_dot2c_f32_f16 give the exact block sum
//     of E2M1 x E2M1 products (multiples of 1/4, at most 576 in magnitude),
//     and one FMA applies sa*sw, the product of the two E4M3 block scales
//     (exact in f32), decoded with v_cvt_pk_f32_fp8 (OCP E4M3).
//
// LDS VALU kernel (gemv_valu_kernel), any M <= 8
//   * The same row mapping, but the activation of a K phase is decoded once
//     per workgroup into LDS as f16 values E2M1(q) * E4M3(s_b) (exact in
//     f16), so a block needs 8 v_dot2c per token and one FMA with sw.  Cost:
//     about 0.5 + 0.56*M VALU operations per weight element, so the VALU
//     issue rate, not HBM, bounds it from M of about 4 up.
//
// MFMA-assisted kernel (gemv_mfma_kernel), M <= 8
//   * The same in-register weight decode, then the weight block scale is
//     applied in f16 (E2M1 * E4M3 is exact in f16) and
//     v_mfma_f32_16x16x32_f16 does the multiply-adds: rows of W are the
//     16-row side of the instruction, tokens the 16-column side (columns
//     >= M are ignored).  Lane (i, kg) loads 32 bytes (64 codes) of row i at
//     element offset 64*kg of each 256-element step, so one wave
//     instruction covers 16 full 128-byte lines; its eight 32-bit words feed
//     eight MFMAs whose k index is permuted the same way on the activation
//     side.  The activation operand is decoded in registers the
//     same way (E2M1 * E4M3 of the activation, exact in f16) straight from
//     L1/L2, so nothing is staged in LDS.
//   * The waves of a workgroup share its 16*R rows and split K; their 16x16
//     partial tiles are added in LDS in a fixed order.  VALU work is about
//     (1 + 1/R) operations per weight element whatever M is.
//
// Every kernel multiplies by the two global scales once at the end.
//
// The register-staged MFMA kernel (gemv_lmfma_kernel) also has 16-token
// instantiations, for M = 9..16, where every token column of the MFMA tile
// is in use (two activation row groups staged per step), and 32-, 64- and
// 128-token ones, for M = 17..128, with 2, 4 or 8 16-token column tiles:
// each decoded weight operand feeds one MFMA per column tile, so the weight
// bytes and their decode are shared by all the tokens.  The MFMA tile kernels deal the rows
// of small-N shapes out evenly over the CUs (tile_rows_for).
//
// Optional LM-head epilogue (ReSET project page, "Step-aware temperature
// scaling"; reading notes sections 3.1, 4.1-4.3): each workgroup also
// writes per-token softmax partials (max, sum e^(z-max), sum e^(z-max)(z-max))
// of its logits to the workspace; a second launch with one workgroup per
// token merges them in a fixed order, computes the entropy and runs the
// ReSET update on the device-resident state.  No counters or atomics, so
// the pair replays in a graph as launched.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family buffer resource for raw byte-addressed loads.
constexpr int kBufferWord3 = 0x00020000;

struct GemvParams {
  int M;
  int64_t N, K;
  int kp;  // K elements per LDS phase (multiple of 128)
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gscale;
  int a_gs_stride;  // 0: one activation global scale; 1: one per token (a_gscale[M])
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_gscale;
  float* y;
  // LM-head epilogue (used only by the EPI instantiations)
  EpilogueArgs epi;
  float* partials;         // epilogue: [row tiles][MT][4] = {max, S, T, -}
  uint32_t* tickets;       // epilogue: [kMaxTokens] per-token counters, zero at rest
  int ksplit;              // tiled GEMM: K splits (1 = none); partials then hold [split][tile][M][128] sums
  size_t state_bytes;      // bytes per ReSET state
  // weight rows per workgroup of the MFMA kernels (<= 16 R): workgroup b
  // owns rows [b * tile_rows, (b + 1) * tile_rows); rows of its 16 R-row
  // tile past that range read as zeros and are never stored
  int tile_rows;
};

// Product of the two global scales for token t (< M): the activation's scale
// is shared by all tokens or, with per-token scales, the token's own.
__device__ __forceinline__ float token_scale(const GemvParams& p, int t) {
  return p.a_gscale[t * p.a_gs_stride] * (*p.w_gscale);
}


// ReSET per-sequence state (device).  Followed by float ring[window].
struct ResetState {
  double sum_all;    // sum of all entropies so far
  double step_sum;   // sum over the current step
  int64_t count;     // positions seen
  int32_t step_len;  // positions in the current step
  int32_t window;
};

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// two f32 -> packed f16 pair (round toward zero; callers only pass values
// that are exactly representable, so the rounding mode never matters)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

template <int B>
__device__ __forceinline__ half2_t fp4x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, B);
}

// Activation block-scale byte -> f32 (OCP E4M3, exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) { return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0]; }

// 8 activation elements (4 bytes of codes) -> 4 half2 of E2M1 * block scale.
__device__ __forceinline__ uint4 act_decode8(uint32_t word, float sa) {
  uint32_t out[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float2_t f;
    if (b == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    if (b == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
    if (b == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
    if (b == 3) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    // both products are exact and representable in f16, so the rounding
    // mode of the conversion does not matter
    out[b] = pack_f16x2(f[0] * sa, f[1] * sa);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// dot of 8 weight codes (one 32-bit word) with 8 f16 activation values,
// accumulated into t.
__device__ __forceinline__ float dot8(uint32_t wword, const uint4& a, float t) {
  t = __builtin_amdgcn_fdot2(fp4x2<0>(wword), as_half2(a.x), t, false);
  t = __builtin_amdgcn_fdot2(fp4x2<1>(wword), as_half2(a.y), t, false);
  t = __builtin_amdgcn_fdot2(fp4x2<2>(wword), as_half2(a.z), t, false);
  t = __builtin_amdgcn_fdot2(fp4x2<3>(wword), as_half2(a.w), t, false);
  return t;
}

// 8 weight codes times one block scale (f16 pair, both halves equal) -> half8.
// E2M1 * E4M3 is exact in f16, so the packed multiply is exact.
__device__ __forceinline__ half8_t wdecode8_scaled(uint32_t word, half2_t s) {
  const half2_t a = fp4x2<0>(word) * s, b = fp4x2<1>(word) * s;
  const half2_t c = fp4x2<2>(word) * s, d = fp4x2<3>(word) * s;
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// ----------------------------------------------------------------------------
// LM-head epilogue, shared by both kernels.  Every thread passes NV values
// with their token index and a validity flag.
// ----------------------------------------------------------------------------

// Cross-lane reductions over a wave64 with DPP (no LDS traffic): within each
// row of 16 lanes by rotations by 8 and 4 and quad permutations, then across
// the four rows through readlane in a fixed order, so every lane gets the
// same, reproducible result.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float rowsum4(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0x128>(x);  // row_ror:8
  x += dpp<0x124>(x);  // row_ror:4
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  return rowsum4(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  const float a = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16)));
  const float b = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48)));
  return fmaxf(a, b);
}

// Merge two softmax partials (m, S, T) with S = sum e^(z-m),
// T = sum e^(z-m) (z-m):  m = max, S = S_a e^(m_a-m) + S_b e^(m_b-m),
// T = e^(m_a-m) (T_a + (m_a-m) S_a) + e^(m_b-m) (T_b + (m_b-m) S_b).
__device__ __forceinline__ void merge_partial(float& m, float& S, float& T, float mb, float Sb, float Tb) {
  if (mb == -INFINITY) return;
  if (m == -INFINITY) {
    m = mb;
    S = Sb;
    T = Tb;
    return;
  }
  const float mn = fmaxf(m, mb);
  const float da = m - mn, db = mb - mn;
  const float fa = expf(da), fb = expf(db);
  T = __builtin_fmaf(fa, __builtin_fmaf(da, S, T), fb * __builtin_fmaf(db, Sb, Tb));
  S = __builtin_fmaf(S, fa, Sb * fb);
  m = mn;
}

// LM-head epilogue, part 1 (in the GEMV kernel): the softmax partials
// (max, S, T) of every token over this workgroup's ROWS rows.  Each thread
// passes NV logits with their token, their row within the tile and two
// flags: `own` (this thread owns the (token, row) slot: every slot of a
// token < M is owned by exactly one thread) and `ok` (the row exists).  The
// slots go through LDS (one barrier); wave w then reduces tokens w, w+NW, ...
// with DPP and writes {max, S, T, 0} to partials[tile][token].
template <int MT, int ROWS, int NV>
__device__ __forceinline__ void lmhead_partials(const GemvParams& p, const float (&val)[NV], const int (&tok)[NV],
                                                const int (&rowt)[NV], const bool (&own)[NV], const bool (&ok)[NV],
                                                int64_t tile) {
  static_assert(ROWS <= 64, "one logit per lane in the reduction");
  __shared__ float slot[MT][ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (own[i]) slot[tok[i]][rowt[i]] = ok[i] ? val[i] : -INFINITY;
  __syncthreads();
  for (int m = wave; m < p.M; m += nw) {
    const float x = lane < ROWS ? slot[m][lane] : -INFINITY;
    const float mx = wave_max(x);  // finite: a tile holds at least one row
    const float d = x - mx;
    const float e = x == -INFINITY ? 0.0f : expf(d);
    const float S = wave_sum(e);
    const float T = wave_sum(e == 0.0f ? 0.0f : e * d);
    if (lane == 0)
      *reinterpret_cast<float4*>(p.partials + (tile * MT + m) * 4) = make_float4(mx, S, T, 0.0f);
  }
}

// LM-head epilogue, part 2 (one launch after the GEMV): kMergeGroups
// workgroups per token each merge a contiguous slice of the token's row-tile
// partials in a fixed order and publish one slice partial; the token's last
// slice workgroup to finish merges the kMergeGroups slice partials in index
// order, computes H = log S - T/S (natural log) and runs the ReSET update of
// the token's sequence state.  "Last" comes from a per-token ticket counter
// that the last workgroup puts back to zero, so the counters need no clearing
// between calls (and no memset node in a captured graph).  The slice
// partials are written and read with device-scope atomic accesses (they go
// past the per-XCD L2s), and the ticket is taken only after the write has
// completed, so no release fence is needed (on gfx950 a release writes back
// the whole L2).
// Workspace: kEpiTicketBytes of tickets [kMaxTokens] spaced kTicketStride
// apart (zero at rest), the
// row-tile partials [ntiles][MT], then the slice partials [MT][kMergeGroups],
// all float4 {max, S, T, -}.
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = 64;
constexpr int kMergeLoads = 4;  // partials per thread and round, all loads in flight at once
// uint32 slots between two tokens' tickets: one 128-byte line each, so the
// tokens' device-scope ticket atomics do not contend for one line (with
// eight tokens packed into one line the merge took about 5 us longer)
constexpr int kTicketStride = 32;
constexpr int64_t kEpiTicketBytes = (4 * kTicketStride * kMaxTokens + 255) / 256 * 256;
static_assert(kMergeGroups <= 64, "one slice partial per lane of a wave");

// offset of the slice partials from the row-tile partials
__host__ __device__ constexpr int64_t merge_slices_offset(int64_t ntiles, int mt) {
  return (ntiles * mt * 16 + 255) / 256 * 256;
}

// The merged (m, S, T) of a wave's 64 partials, in every lane: DPP moves
// within each row of 16 lanes (rotations by 8 and 4, then the quad
// permutations), then the four rows in index order through readlane.  The
// order is fixed, so the result is reproducible.
__device__ __forceinline__ void wave_merge(float& m, float& S, float& T) {
  merge_partial(m, S, T, dpp<0x128>(m), dpp<0x128>(S), dpp<0x128>(T));  // row_ror:8
  merge_partial(m, S, T, dpp<0x124>(m), dpp<0x124>(S), dpp<0x124>(T));  // row_ror:4
  merge_partial(m, S, T, dpp<0xB1>(m), dpp<0xB1>(S), dpp<0xB1>(T));     // quad_perm [1,0,3,2]
  merge_partial(m, S, T, dpp<0x4E>(m), dpp<0x4E>(S), dpp<0x4E>(T));     // quad_perm [2,3,0,1]
  auto lane_f = [](float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  };
  float gm = lane_f(m, 0), gS = lane_f(S, 0), gT = lane_f(T, 0);
  merge_partial(gm, gS, gT, lane_f(m, 16), lane_f(S, 16), lane_f(T, 16));
  merge_partial(gm, gS, gT, lane_f(m, 32), lane_f(S, 32), lane_f(T, 32));
  merge_partial(gm, gS, gT, lane_f(m, 48), lane_f(S, 48), lane_f(T, 48));
  m = gm;
  S = gS;
  T = gT;
}

// The end of the LM-head epilogue for token m, run by one wave whose lanes
// hold partials (max, S, T) of disjoint parts of the row (empty partials
// where a lane has none): every lane loads the sequence state and a part of
// the ring of the last entropies in the same round trip (the state block
// holds p.epi.window of them), the lanes' partials are merged in a fixed
// order, and lane 0 computes H = log S - T/S and runs the ReSET update.
// sring: LDS for kResetMaxWindow floats.
__device__ __forceinline__ void lmhead_reset_tail(const GemvParams& p, int m, float gm, float Sm, float Tm, int lane,
                                                  float* sring) {
  ResetState* st = reinterpret_cast<ResetState*>(reinterpret_cast<char*>(p.epi.state) + (size_t)m * p.state_bytes);
  const float* ring = reinterpret_cast<const float*>(st + 1);
  const int64_t count0 = st->count;
  const int32_t st_window = st->window, len0 = st->step_len;
  const double sum_all0 = st->sum_all, step_sum0 = st->step_sum;
  const bool new_step = p.epi.step_start[m] != 0;
  const int wcap = p.epi.window < kResetMaxWindow ? p.epi.window : kResetMaxWindow;
  float rv[kResetMaxWindow / 64];
#pragma unroll
  for (int k = 0; k < kResetMaxWindow / 64; ++k) {
    const int i = lane + 64 * k;
    rv[k] = i < wcap ? ring[i] : 0.0f;
  }
  wave_merge(gm, Sm, Tm);
  const double Sd = Sm, Td = Tm;
  const float H = (float)(log(Sd) - Td / Sd);
  // ---- ReSET update: update with H first, then decide ----
  // the ring holds the window the state was initialised with; never index
  // past the smaller of that and the caller's window
  int w = st_window < p.epi.window ? st_window : p.epi.window;
  if (w < 1) w = 1;
  const int slot = (int)(count0 % w);
#pragma unroll
  for (int k = 0; k < kResetMaxWindow / 64; ++k) {
    const int i = lane + 64 * k;
    if (i < wcap) sring[i] = i == slot ? H : rv[k];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the wave's LDS writes before its reads
  if (lane != 0) return;
  const double h = (double)H;
  const bool reset = count0 == 0 || new_step;
  const int64_t count = count0 + 1;
  const double sum_all = sum_all0 + h;
  const double step_sum = (reset ? 0.0 : step_sum0) + h;
  const int32_t step_len = (reset ? 0 : len0) + 1;
  const int64_t nwin = count < w ? count : w;
  double wsum = 0.0;
  for (int64_t i = count - nwin; i < count; ++i) wsum += (double)sring[i % w];
  const double hbar = sum_all / (double)count;
  const double hstep = step_len <= w ? wsum / (double)nwin : step_sum / (double)step_len;
  const double tau = hstep > hbar ? hstep : (double)p.epi.tau0;
  float T_t;
  if (p.epi.mode == 1) T_t = p.epi.t_base;                                   // BASE
  else if (p.epi.mode == 2) T_t = h < (double)p.epi.tau0 ? p.epi.t_low : p.epi.t_high;  // fixed threshold
  else T_t = h < tau ? p.epi.t_low : p.epi.t_high;                           // ReSET
  float* ring_w = reinterpret_cast<float*>(st + 1);
  ring_w[slot] = H;
  st->count = count;
  st->sum_all = sum_all;
  st->step_sum = step_sum;
  st->step_len = step_len;
  p.epi.entropy[m] = H;
  p.epi.temperature[m] = T_t;
}


__global__ __launch_bounds__(kMergeThreads) void lmhead_slice_kernel(GemvParams p, int mt, int ntiles) {
  __shared__ float wm[kMergeThreads / 64], wS[kMergeThreads / 64], wt[kMergeThreads / 64];
  __shared__ float sring[kResetMaxWindow];
  __shared__ uint32_t is_last;
  const int m = blockIdx.x / kMergeGroups, grp = blockIdx.x % kMergeGroups;
  if (m >= p.M) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* slices = reinterpret_cast<float*>(reinterpret_cast<char*>(p.partials) + merge_slices_offset(ntiles, mt));
  // this workgroup's slice of tiles; thread t takes lo + t, lo + t + NT, ...
  const int per = (ntiles + kMergeGroups - 1) / kMergeGroups;
  const int lo = grp * per, hi = lo + per < ntiles ? lo + per : ntiles;
  // row-tile partials [ntiles][mt] through a buffer resource; tiles outside
  // the slice take the empty partial (-inf, 0, 0) and no load
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      p.partials, (short)0, (int)((int64_t)ntiles * mt * 16), kBufferWord3);
  float gm = -INFINITY, Sm = 0.0f, Tm = 0.0f;
  for (int base = lo; base < hi; base += kMergeThreads * kMergeLoads) {  // same trip count for every thread
    float4_t q[kMergeLoads];
#pragma unroll
    for (int j = 0; j < kMergeLoads; ++j) {
      const int idx = base + j * kMergeThreads + (int)threadIdx.x;
      const int off = idx < hi ? (int)(((int64_t)idx * mt + m) * 16) : (int)0x7FFFFFF0;
      q[j] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < kMergeLoads; ++j) {
      const bool in = base + j * kMergeThreads + (int)threadIdx.x < hi;
      merge_partial(gm, Sm, Tm, in ? q[j][0] : -INFINITY, q[j][1], q[j][2]);
    }
  }
  // across the wave, then across the waves through LDS in index order
  wave_merge(gm, Sm, Tm);
  if (lane == 0) {
    wm[wave] = gm;
    wS[wave] = Sm;
    wt[wave] = Tm;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kMergeThreads / 64; ++w) merge_partial(gm, Sm, Tm, wm[w], wS[w], wt[w]);
    float* sp = slices + ((int64_t)m * kMergeGroups + grp) * 4;
    __hip_atomic_store(sp, gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sp + 1, Sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sp + 2, Tm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the slice partial has landed
    uint32_t* ticket = p.tickets + (int64_t)m * kTicketStride;
    const uint32_t done = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = done == kMergeGroups - 1 ? 1u : 0u;
    if (done == kMergeGroups - 1) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (is_last == 0 || wave != 0) return;
  // the token's last slice workgroup, wave 0: lane g takes slice partial g
  const float* sp = slices + ((int64_t)m * kMergeGroups + (lane < kMergeGroups ? lane : 0)) * 4;
  gm = __hip_atomic_load(sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  Sm = __hip_atomic_load(sp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  Tm = __hip_atomic_load(sp + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane >= kMergeGroups) {  // no slice: the empty partial
    gm = -INFINITY;
    Sm = Tm = 0.0f;
  }
  lmhead_reset_tail(p, m, gm, Sm, Tm, lane, sring);
}

// ----------------------------------------------------------------------------
// VALU kernel
// ----------------------------------------------------------------------------

template <int MT, int G, int R, int NW, int P, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_valu_kernel(GemvParams p) {
  extern __shared__ uint4 lds[];  // activation phase [MT][4][C] of 16 bytes
  constexpr int RG = 64 / G;      // row-groups per wave
  constexpr int ROWS = R * NW * RG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane % G;
  const int rg = lane / G;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * ROWS;

  const uint8_t* wc[R];
  const uint8_t* ws[R];
  int64_t row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = tile0 + (int64_t)(r * NW + wave) * RG + rg;
    const int64_t rr = row[r] < N ? row[r] : N - 1;  // clamp: loads stay in bounds
    wc[r] = p.w_codes + rr * (K / 2);
    ws[r] = p.w_scales + rr * (K / 16);
  }

  float acc[R][MT][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m][0] = acc[r][m][1] = 0.0f;

  for (int64_t kb = 0; kb < K; kb += p.kp) {
    const int C = (int)((K - kb < p.kp ? K - kb : p.kp) / 32);  // 32-element chunks in this phase
    const int n = g < C ? (C - g + G - 1) / G : 0;              // chunks of this lane: g, g+G, ...
    const uint8_t* wcp[R];
    const uint8_t* wsp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wcp[r] = wc[r] + kb / 2;
      wsp[r] = ws[r] + kb / 16;
    }
    // the first P chunks go in flight before the activation is staged
    uint4 wb[P][R];
    uint32_t sbuf[P][R];
#pragma unroll
    for (int j = 0; j < P; ++j)
      if (j < n)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int c = g + j * G;
          wb[j][r] = *reinterpret_cast<const uint4*>(wcp[r] + c * 16);
          sbuf[j][r] = *reinterpret_cast<const uint16_t*>(wsp[r] + c * 2);
        }
    __syncthreads();  // the previous phase is done with the LDS tile
    for (int it = threadIdx.x; it < MT * 4 * C; it += NW * 64) {
      const int m = it / (4 * C);
      const int rem = it - m * 4 * C;
      const int q = rem / C;
      const int c = rem - q * C;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M) {
        const int64_t k = kb + (int64_t)c * 32 + q * 8;
        const uint32_t word = *reinterpret_cast<const uint32_t*>(p.a_codes + (int64_t)m * (K / 2) + k / 2);
        v = act_decode8(word, e4m3_to_f32(p.a_scales[(int64_t)m * (K / 16) + k / 16]));
      }
      lds[(m * 4 + q) * C + c] = v;
    }
    __syncthreads();

    for (int i0 = 0; i0 < n; i0 += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int i = i0 + j;
        if (i < n) {
          const int c = g + i * G;
          uint4 w[R];
          uint32_t s[R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            w[r] = wb[j][r];
            s[r] = sbuf[j][r];
          }
          if (i + P < n) {
            const int cn = c + P * G;
#pragma unroll
            for (int r = 0; r < R; ++r) {
              wb[j][r] = *reinterpret_cast<const uint4*>(wcp[r] + cn * 16);
              sbuf[j][r] = *reinterpret_cast<const uint16_t*>(wsp[r] + cn * 2);
            }
          }
          float t[R][MT][2];
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) t[r][m][0] = t[r][m][1] = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint4 a[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) a[m] = lds[(m * 4 + q) * C + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint32_t ww = word_of(w[r], q);
#pragma unroll
              for (int m = 0; m < MT; ++m) t[r][m][q >> 1] = dot8(ww, a[m], t[r][m][q >> 1]);
            }
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float2_t sw = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], false);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              acc[r][m][0] = __builtin_fmaf(t[r][m][0], sw[0], acc[r][m][0]);
              acc[r][m][1] = __builtin_fmaf(t[r][m][1], sw[1], acc[r][m][1]);
            }
          }
        }
      }
    }
  }

  // reduce the G lanes of each row-group
  float scale[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) scale[m] = token_scale(p, m < M ? m : 0);
  float out[R * MT];
  int tok[R * MT];
  bool ok[R * MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m][0] + acc[r][m][1];
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      out[r * MT + m] = v * scale[m];
      tok[r * MT + m] = m;
      ok[r * MT + m] = g == 0 && row[r] < N && m < M;
    }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (ok[r * MT + m]) p.y[(int64_t)m * N + row[r]] = out[r * MT + m];

  if constexpr (EPI) {
    int rowt[R * MT];
    bool own[R * MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        rowt[r * MT + m] = (int)(row[r] - tile0);
        own[r * MT + m] = g == 0 && m < M;
      }
    lmhead_partials<MT, R * NW * (64 / G), R * MT>(p, out, tok, rowt, own, ok, blockIdx.x);
  }
}

// ----------------------------------------------------------------------------
// Direct VALU kernel (M <= 2): no LDS, activation decoded in registers
// ----------------------------------------------------------------------------

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 as_uint4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }

template <bool NT>
__device__ __forceinline__ uint4 ld_w16(const uint8_t* ptr) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *reinterpret_cast<const uint4*>(ptr);
  }
}

template <int MT, int G, int R, int NW, int P, bool NT, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_direct_kernel(GemvParams p) {
  constexpr int RG = 64 / G;
  constexpr int ROWS = R * NW * RG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane % G;
  const int rg = lane / G;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * ROWS;

  const uint8_t* wc[R];
  const uint8_t* ws[R];
  int64_t row[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = tile0 + (int64_t)(r * NW + wave) * RG + rg;
    const int64_t rr = row[r] < N ? row[r] : N - 1;  // clamp: loads stay in bounds
    wc[r] = p.w_codes + rr * (K / 2);
    ws[r] = p.w_scales + rr * (K / 16);
  }
  const uint8_t* ac[MT];
  const uint8_t* as[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mm = m < M ? m : M - 1;  // tokens >= M reuse a valid row; their sums are never stored
    ac[m] = p.a_codes + (int64_t)mm * (K / 2);
    as[m] = p.a_scales + (int64_t)mm * (K / 16);
  }

  float acc[R][MT][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m][0] = acc[r][m][1] = 0.0f;

  const int C = (int)(K / 32);                    // 32-element chunks per row
  const int n = g < C ? (C - g + G - 1) / G : 0;  // chunks of this lane: g, g+G, ...
  uint4 wb[P][R], ab[P][MT];
  uint32_t sb[P][R], asb[P][MT];
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (j < n) {
      const int c = g + j * G;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wb[j][r] = ld_w16<NT>(wc[r] + c * 16);
        sb[j][r] = *reinterpret_cast<const uint16_t*>(ws[r] + c * 2);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        ab[j][m] = *reinterpret_cast<const uint4*>(ac[m] + c * 16);
        asb[j][m] = *reinterpret_cast<const uint16_t*>(as[m] + c * 2);
      }
    }
  for (int i0 = 0; i0 < n; i0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = i0 + j;
      if (i < n) {
        uint4 w[R], a[MT];
        uint32_t s[R], sa[MT];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          w[r] = wb[j][r];
          s[r] = sb[j][r];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          a[m] = ab[j][m];
          sa[m] = asb[j][m];
        }
        if (i + P < n) {
          const int cn = g + (i + P) * G;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            wb[j][r] = ld_w16<NT>(wc[r] + cn * 16);
            sb[j][r] = *reinterpret_cast<const uint16_t*>(ws[r] + cn * 2);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            ab[j][m] = *reinterpret_cast<const uint4*>(ac[m] + cn * 16);
            asb[j][m] = *reinterpret_cast<const uint16_t*>(as[m] + cn * 2);
          }
        }
        // activation: 32 E2M1 values as f16 pairs, and its two block scales
        half2_t ah[MT][16];
        float2_t saf[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = word_of(a[m], q);
            ah[m][4 * q + 0] = fp4x2<0>(word);
            ah[m][4 * q + 1] = fp4x2<1>(word);
            ah[m][4 * q + 2] = fp4x2<2>(word);
            ah[m][4 * q + 3] = fp4x2<3>(word);
          }
          saf[m] = __builtin_amdgcn_cvt_pk_f32_fp8(sa[m], false);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float2_t sw = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], false);
          half2_t wh[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = word_of(w[r], q);
            wh[4 * q + 0] = fp4x2<0>(word);
            wh[4 * q + 1] = fp4x2<1>(word);
            wh[4 * q + 2] = fp4x2<2>(word);
            wh[4 * q + 3] = fp4x2<3>(word);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              t0 = __builtin_amdgcn_fdot2(wh[k], ah[m][k], t0, false);
              t1 = __builtin_amdgcn_fdot2(wh[8 + k], ah[m][8 + k], t1, false);
            }
            acc[r][m][0] = __builtin_fmaf(t0, saf[m][0] * sw[0], acc[r][m][0]);
            acc[r][m][1] = __builtin_fmaf(t1, saf[m][1] * sw[1], acc[r][m][1]);
          }
        }
      }
    }
  }

  float scale[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) scale[m] = token_scale(p, m < M ? m : 0);
  float out[R * MT];
  int tok[R * MT];
  bool ok[R * MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m][0] + acc[r][m][1];
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      out[r * MT + m] = v * scale[m];
      tok[r * MT + m] = m;
      ok[r * MT + m] = g == 0 && row[r] < N && m < M;
    }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (ok[r * MT + m]) p.y[(int64_t)m * N + row[r]] = out[r * MT + m];

  if constexpr (EPI) {
    int rowt[R * MT];
    bool own[R * MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        rowt[r * MT + m] = (int)(row[r] - tile0);
        own[r * MT + m] = g == 0 && m < M;
      }
    lmhead_partials<MT, R * NW * (64 / G), R * MT>(p, out, tok, rowt, own, ok, blockIdx.x);
  }
}

// One 256-element step of the MFMA kernels.  Lane (li, kg) holds, for each
// of its R weight rows li (+16r) and for its activation row, the 64 codes of
// elements 64*kg .. 64*kg+63 of the step (two uint4) and their four block
// scales (one byte each).  Both sides are decoded to exact f16 values
// E2M1 * E4M3 and eight v_mfma_f32_16x16x32_f16 per row tile add the step
// into acc[r] (D layout: lane (li, kg) holds rows 4*kg + v, token li).
template <int R>
__device__ __forceinline__ void mfma_step(const uint4 (&w)[R][2], const uint32_t (&s)[R], const uint4& a0,
                                          const uint4& a1, uint32_t sa, float4_t (&acc)[R]) {
  // block scales as f16 pairs (both halves equal; E4M3 values are exact in f16)
  const float2_t sa01 = __builtin_amdgcn_cvt_pk_f32_fp8(sa, false);
  const float2_t sa23 = __builtin_amdgcn_cvt_pk_f32_fp8(sa, true);
  const half2_t ha[4] = {as_half2(pack_f16x2(sa01[0], sa01[0])), as_half2(pack_f16x2(sa01[1], sa01[1])),
                         as_half2(pack_f16x2(sa23[0], sa23[0])), as_half2(pack_f16x2(sa23[1], sa23[1]))};
  half2_t hw[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float2_t sw01 = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], false);
    const float2_t sw23 = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], true);
    hw[r][0] = as_half2(pack_f16x2(sw01[0], sw01[0]));
    hw[r][1] = as_half2(pack_f16x2(sw01[1], sw01[1]));
    hw[r][2] = as_half2(pack_f16x2(sw23[0], sw23[0]));
    hw[r][3] = as_half2(pack_f16x2(sw23[1], sw23[1]));
  }
  // word j of the lane's 64 codes: B operand decoded once, used by all R tiles
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t aw = word_of(j < 4 ? a0 : a1, j & 3);
    const half8_t b = wdecode8_scaled(aw, ha[j >> 1]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t ww = word_of(w[r][j >> 2], j & 3);
      acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wdecode8_scaled(ww, hw[r][j >> 1]), b, acc[r], 0, 0, 0);
    }
  }
}

// Add the NW waves' partial tiles in a fixed order (through LDS; every wave
// must have left its main loop), scale by the global scales, store y and run
// the optional epilogue.
// CT column tiles of 16 tokens each: acc[r * CT + ct] holds row tile r,
// tokens 16 ct .. 16 ct + 15.
template <int MT, int R, int NW, bool EPI, int CT = 1>
__device__ __forceinline__ void mfma_finish(const GemvParams& p, const float4_t (&acc)[R * CT], float* red,
                                            int64_t tile0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kg = lane >> 4;
  const int64_t N = p.N;
  const int M = p.M;
#pragma unroll
  for (int rc = 0; rc < R * CT; ++rc)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * R * CT + rc) * 4 + v) * 64 + lane] = acc[rc][v];
  __syncthreads();
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;  // rows this workgroup owns
  // wave w finalizes the (r, ct, v) register slots w, w + NW, ...; D layout:
  // lane (li, kg) holds rows 4*kg + v of each 16-row tile, token 16 ct + li
  constexpr int NV = (R * CT * 4 + NW - 1) / NW;
  // each output's global scale, every load issued before the first store (a
  // load between stores would wait for the stores before it)
  float tsc[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int t = 16 * (((wave + u * NW) >> 2) % CT) + li;
    tsc[u] = token_scale(p, t < M ? t : 0);
  }
  float out[NV];
  int tok[NV], rowt[NV];
  bool ok[NV], own[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int rv = wave + u * NW;
    out[u] = 0.0f;
    tok[u] = li < MT ? li : 0;
    rowt[u] = 0;
    ok[u] = own[u] = false;
    if (rv < R * CT * 4) {
      const int rc = rv >> 2, v = rv & 3;
      const int r = rc / CT, t = 16 * (rc % CT) + li;  // row tile, token
      float sum = 0.0f;
      for (int w = 0; w < NW; ++w) sum += red[((w * R * CT + rc) * 4 + v) * 64 + lane];
      const int64_t row = tile0 + 16 * r + 4 * kg + v;
      out[u] = sum * tsc[u];
      tok[u] = t < MT ? t : 0;
      rowt[u] = 16 * r + 4 * kg + v;
      own[u] = t < M;
      ok[u] = t < M && rowt[u] < rows;
      if (ok[u]) p.y[(int64_t)t * N + row] = out[u];
    }
  }
  if constexpr (EPI) lmhead_partials<MT, 16 * R, NV>(p, out, tok, rowt, own, ok, blockIdx.x);
}

// ----------------------------------------------------------------------------
// MFMA-assisted kernel
// ----------------------------------------------------------------------------

template <int MT, int R, int NW, int P, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_mfma_kernel(GemvParams p) {
  extern __shared__ uint4 lds4[];  // [NW][R][4][64] partial tiles at the end
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;   // row of the A operand / column (token) of B and D
  const int kg = lane >> 4;   // k group: elements 64*kg .. 64*kg+63 of a 256-step
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * (16 * R);
  const int nsteps = (int)((K + 255) / 256);
  const int n = wave < nsteps ? (nsteps - wave + NW - 1) / NW : 0;  // steps of this wave: wave, wave+NW, ...
  (void)MT;

  const uint8_t* wc[R];
  const uint8_t* ws[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t rr = tile0 + 16 * r + li;
    rr = rr < N ? rr : N - 1;  // clamp: loads stay in bounds
    wc[r] = p.w_codes + rr * (K / 2);
    ws[r] = p.w_scales + rr * (K / 16);
  }
  // activation row fed to B column li (columns >= M read a valid row; ignored)
  const int btok = li < M ? li : M - 1;
  const uint8_t* ac = p.a_codes + (int64_t)btok * (K / 2);
  const uint8_t* as = p.a_scales + (int64_t)btok * (K / 16);

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // one step = 256 elements of K: lane (li, kg) holds 64 codes (32 bytes, 4
  // blocks) of its weight rows and of its activation row
  uint4 wb[P][R][2], ab[P][2];
  uint32_t sbuf[P][R], asb[P];
  auto load = [&](int slot, int step) {
    const int64_t e = (int64_t)step * 256 + 64 * kg;  // first element of this lane
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t eh = e + 32 * h;  // K % 32 == 0: a 32-element half is all in or all out
      const bool in = eh < K;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wb[slot][r][h] = in ? *reinterpret_cast<const uint4*>(wc[r] + eh / 2) : make_uint4(0, 0, 0, 0);
      ab[slot][h] = in ? *reinterpret_cast<const uint4*>(ac + eh / 2) : make_uint4(0, 0, 0, 0);
    }
    // four block scales; the second pair only when the second half is inside
    const bool in0 = e < K, in1 = e + 32 < K;
#pragma unroll
    for (int r = 0; r < R; ++r)
      sbuf[slot][r] = in1 ? *reinterpret_cast<const uint32_t*>(ws[r] + e / 16)
                          : (in0 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ws[r] + e / 16) : 0u);
    asb[slot] = in1 ? *reinterpret_cast<const uint32_t*>(as + e / 16)
                    : (in0 ? (uint32_t)*reinterpret_cast<const uint16_t*>(as + e / 16) : 0u);
  };
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (j < n) load(j, wave + j * NW);

  for (int i0 = 0; i0 < n; i0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = i0 + j;
      if (i < n) {
        uint4 w[R][2];
        uint32_t s[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          w[r][0] = wb[j][r][0];
          w[r][1] = wb[j][r][1];
          s[r] = sbuf[j][r];
        }
        const uint4 a0 = ab[j][0], a1 = ab[j][1];
        const uint32_t sa = asb[j];
        if (i + P < n) load(j, wave + (i + P) * NW);
        mfma_step<R>(w, s, a0, a1, sa, acc);
      }
    }
  }

  mfma_finish<MT, R, NW, EPI>(p, acc, reinterpret_cast<float*>(lds4), tile0);
}

// ----------------------------------------------------------------------------
// LDS-staged MFMA kernel
// ----------------------------------------------------------------------------
// In the MFMA operand layout the 16 lanes of a row group hold 16 different
// rows, so a 16-byte load made straight into it sends every 4-lane group of
// the load to 4 different cache lines.  Here a wave loads each 256-element
// step with 8 consecutive lanes per 128-byte row of codes and 4 lanes per
// 16-byte row of scale bytes (whole lines per lane group), writes the step
// into its own LDS slot and reads it back in the operand layout.  Code rows
// sit 144 bytes apart in the slot, so the operand reads (16 rows x 16 bytes
// per lane group) hit 64 different banks.  A wave touches only its own slot,
// so no workgroup barrier is needed until the final reduction.
constexpr int kLdsCodeRow = 144;  // LDS bytes per 128-byte row of codes
constexpr int kLdsScaleRow = 20;  // LDS bytes per 16-byte row of scales

// activation rows in a slot: 8 for up to 8 tokens, else the token count
// (16, 32, 64 or 128)
template <int MT>
constexpr int lmfma_act_rows() {
  return MT > 8 ? MT : 8;
}

template <int R, int MT>
constexpr int lmfma_slot_bytes() {
  return (16 * R + lmfma_act_rows<MT>()) * (kLdsCodeRow + kLdsScaleRow);
}

template <int R>
struct LmfmaStep {
  uint4 w[R][2];    // weight codes: rows 8h + lane/8 of tile r, 16 bytes at 16*(lane%8)
  uint4 a[16];      // activation codes: rows 8 g + lane/8 (g < activation rows / 8), 16 bytes at 16*(lane%8)
  uint32_t ws[R];   // weight scales: row lane/4 of tile r, bytes 4*(lane%4) .. +3 (or +1)
  uint32_t wsh[R];  // bytes 4*(lane%4) + 2, +3 when the word is loaded in halves
  uint32_t as[8], ash[8];  // activation scales: rows 16 s + lane/4, the same bytes
};

// One 256-element step for CT column tiles of 16 tokens: as mfma_step, but
// each decoded weight operand feeds the CT tiles' MFMAs.  a0/a1/sa[ct] hold
// the lane's token 16 ct + li; acc[r * CT + ct].
template <int R, int CT>
__device__ __forceinline__ void mfma_step_ct(const uint4 (&w)[R][2], const uint32_t (&s)[R], const uint4 (&a0)[CT],
                                             const uint4 (&a1)[CT], const uint32_t (&sa)[CT], float4_t (&acc)[R * CT]) {
  half2_t ha[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float2_t sa01 = __builtin_amdgcn_cvt_pk_f32_fp8(sa[ct], false);
    const float2_t sa23 = __builtin_amdgcn_cvt_pk_f32_fp8(sa[ct], true);
    ha[ct][0] = as_half2(pack_f16x2(sa01[0], sa01[0]));
    ha[ct][1] = as_half2(pack_f16x2(sa01[1], sa01[1]));
    ha[ct][2] = as_half2(pack_f16x2(sa23[0], sa23[0]));
    ha[ct][3] = as_half2(pack_f16x2(sa23[1], sa23[1]));
  }
  half2_t hw[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float2_t sw01 = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], false);
    const float2_t sw23 = __builtin_amdgcn_cvt_pk_f32_fp8(s[r], true);
    hw[r][0] = as_half2(pack_f16x2(sw01[0], sw01[0]));
    hw[r][1] = as_half2(pack_f16x2(sw01[1], sw01[1]));
    hw[r][2] = as_half2(pack_f16x2(sw23[0], sw23[0]));
    hw[r][3] = as_half2(pack_f16x2(sw23[1], sw23[1]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (CT <= 2) {
      // activation operands first (CT of them live), then one weight
      // operand at a time
      half8_t b[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        b[ct] = wdecode8_scaled(word_of(j < 4 ? a0[ct] : a1[ct], j & 3), ha[ct][j >> 1]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const half8_t a = wdecode8_scaled(word_of(w[r][j >> 2], j & 3), hw[r][j >> 1]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[r * CT + ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[ct], acc[r * CT + ct], 0, 0, 0);
      }
    } else {
      // weight operands first (R of them live), then one column tile's
      // activation operand at a time, so the live registers grow with R,
      // not CT
      half8_t a[R];
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = wdecode8_scaled(word_of(w[r][j >> 2], j & 3), hw[r][j >> 1]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const half8_t b = wdecode8_scaled(word_of(j < 4 ? a0[ct] : a1[ct], j & 3), ha[ct][j >> 1]);
#pragma unroll
        for (int r = 0; r < R; ++r)
          acc[r * CT + ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], b, acc[r * CT + ct], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int MT, int R, int NW, int P, bool K64, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_lmfma_kernel(GemvParams p) {
  extern __shared__ uint4 lds4[];  // NW slots; reused by the final reduction
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kg = lane >> 4;  // operand layout
  const int lq = lane >> 3, lc = lane & 7;   // code loads: row, 16-byte chunk
  const int sq = lane >> 2, sp = lane & 3;   // scale loads: row, 4-byte part
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int nsteps = (int)((K + 255) / 256);
  const int n = wave < nsteps ? (nsteps - wave + NW - 1) / NW : 0;  // steps wave, wave + NW, ...
  constexpr int AR = lmfma_act_rows<MT>();  // activation rows staged per step
  constexpr int AG = AR / 8;                 // activation code loads per step (8 rows each)
  constexpr int SG = AR > 16 ? AR / 16 : 1;  // activation scale loads per step (16 rows each)
  constexpr int CT = AR > 16 ? AR / 16 : 1;  // 16-token column tiles

  // Buffer resources over this workgroup's weight rows and over the
  // activation: rows past them (or past M) lie outside num_records and load
  // as zeros, so no load is predicated.  Code chunks past K (last step only) load bytes of the
  // next row; their block scales are masked to zero below, which makes the
  // decoded values zero (E2M1 codes are always finite).
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_scales + tile0 * (K / 16)), (short)0, (int)(rows * (K / 16)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t acr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_codes), (short)0, (int)(M * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t asr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), (short)0, (int)(M * (K / 16)), kBufferWord3);
  const int code_off = lq * (int)(K / 2) + 16 * lc;  // + 8 rows for h = 1, + 16 rows per tile
  const int scale_off = sq * (int)(K / 16) + 4 * sp;

  auto load = [&](LmfmaStep<R>& st, int step) {
    const int cstep = step * 128, sstep = step * 16;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        st.w[r][h] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(
            wcr, code_off + (16 * r + 8 * h) * (int)(K / 2) + cstep, 0, 0));
#pragma unroll
    for (int g = 0; g < AG; ++g)
      st.a[g] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(acr, code_off + 8 * g * (int)(K / 2) + cstep, 0, 0));
    // four block scales (64 elements).  With K % 64 == 0 (K64) every 4-byte
    // word is aligned and wholly inside its row; otherwise rows are 2-byte
    // aligned and the last word of a row is half outside, so the word is
    // loaded as two halves (a load that crosses num_records reads as zero as
    // a whole).  Scales past K are masked when the step is staged, not here:
    // using the loaded value now would wait for the load.
    if constexpr (K64) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        st.ws[r] = __builtin_amdgcn_raw_buffer_load_b32(wsr, scale_off + 16 * r * (int)(K / 16) + sstep, 0, 0);
#pragma unroll
      for (int g = 0; g < SG; ++g)
        st.as[g] = __builtin_amdgcn_raw_buffer_load_b32(asr, scale_off + 16 * g * (int)(K / 16) + sstep, 0, 0);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int o = scale_off + 16 * r * (int)(K / 16) + sstep;
        st.ws[r] = __builtin_amdgcn_raw_buffer_load_b16(wsr, o, 0, 0);
        st.wsh[r] = __builtin_amdgcn_raw_buffer_load_b16(wsr, o + 2, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < SG; ++g) {
        const int o = scale_off + 16 * g * (int)(K / 16) + sstep;
        st.as[g] = __builtin_amdgcn_raw_buffer_load_b16(asr, o, 0, 0);
        st.ash[g] = __builtin_amdgcn_raw_buffer_load_b16(asr, o + 2, 0, 0);
      }
    }
  };
  // the staged scale word of a lane: its loaded bytes with the blocks past K
  // cleared
  auto scale_word = [&](uint32_t lo, uint32_t hi, int step) -> uint32_t {
    const int64_t es = (int64_t)step * 256 + 64 * sp;
    const uint32_t w = K64 ? lo : (lo & 0xFFFFu) | (hi << 16);
    return es + 32 < K ? w : es < K ? (w & 0xFFFFu) : 0u;
  };

  char* slot = reinterpret_cast<char*>(lds4) + wave * lmfma_slot_bytes<R, MT>();
  char* scl = slot + (16 * R + AR) * kLdsCodeRow;
  // operand-layout read addresses: token 16 ct + li of each column tile
  // (tokens >= M read row M - 1; ignored)
  int btok[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) btok[ct] = 16 * ct + li < M ? 16 * ct + li : M - 1;

  float4_t acc[R * CT];
#pragma unroll
  for (int rc = 0; rc < R * CT; ++rc) acc[rc] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // P register buffers in a ring: the loads of steps i+1 .. i+P-1 stay in
  // flight while step i is staged and computed; a buffer is refilled right
  // after its contents went to LDS.  Loads and staging are unconditional
  // (the step index is clamped to the wave's last step, so the few extra
  // loads re-read data already in flight) and only the compute is skipped
  // past the end: with no load behind a branch, the compiler's wait counts
  // stay exact and the P-deep pipeline is kept.
  if (n > 0) {
    LmfmaStep<R> buf[P];
    // buffers are filled one after the other, never interleaved, so the
    // wait before staging buffer j counts exactly the later buffers' loads
#pragma unroll
    for (int j = 0; j < P; ++j) {
      load(buf[j], wave + (j < n ? j : n - 1) * NW);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i0 = 0; i0 < n; i0 += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int i = i0 + j;
        const int si = wave + (i < n ? i : n - 1) * NW;  // the step held by buf[j]
        // stage the step (the previous step's operand reads are done: fence)
        wave_lds_fence();
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<uint4*>(slot + (16 * r + 8 * h + lq) * kLdsCodeRow + 16 * lc) = buf[j].w[r][h];
          *reinterpret_cast<uint32_t*>(scl + (16 * r + sq) * kLdsScaleRow + 4 * sp) =
              scale_word(buf[j].ws[r], buf[j].wsh[r], si);
        }
#pragma unroll
        for (int g = 0; g < AG; ++g)
          *reinterpret_cast<uint4*>(slot + (16 * R + 8 * g + lq) * kLdsCodeRow + 16 * lc) = buf[j].a[g];
#pragma unroll
        for (int g = 0; g < SG; ++g)
          if (16 * g + sq < AR)
            *reinterpret_cast<uint32_t*>(scl + (16 * R + 16 * g + sq) * kLdsScaleRow + 4 * sp) =
                scale_word(buf[j].as[g], buf[j].ash[g], si);
        wave_lds_fence();
        __builtin_amdgcn_sched_barrier(0);
        load(buf[j], wave + (i + P < n ? i + P : n - 1) * NW);
        __builtin_amdgcn_sched_barrier(0);
        if (i < n) {
          // read it back in the operand layout
          uint4 w[R][2];
          uint32_t sw[R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            w[r][0] = *reinterpret_cast<const uint4*>(slot + (16 * r + li) * kLdsCodeRow + 32 * kg);
            w[r][1] = *reinterpret_cast<const uint4*>(slot + (16 * r + li) * kLdsCodeRow + 32 * kg + 16);
            sw[r] = *reinterpret_cast<const uint32_t*>(scl + (16 * r + li) * kLdsScaleRow + 4 * kg);
          }
          uint4 a0[CT], a1[CT];
          uint32_t sa[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            a0[ct] = *reinterpret_cast<const uint4*>(slot + (16 * R + btok[ct]) * kLdsCodeRow + 32 * kg);
            a1[ct] = *reinterpret_cast<const uint4*>(slot + (16 * R + btok[ct]) * kLdsCodeRow + 32 * kg + 16);
            sa[ct] = *reinterpret_cast<const uint32_t*>(scl + (16 * R + btok[ct]) * kLdsScaleRow + 4 * kg);
          }
          mfma_step_ct<R, CT>(w, sw, a0, a1, sa, acc);
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its slot before the reduction reuses the LDS
  mfma_finish<MT, R, NW, EPI, CT>(p, acc, reinterpret_cast<float*>(lds4), tile0);
}

// ----------------------------------------------------------------------------
// Direct-to-LDS MFMA kernel (K % 256 == 0)
// ----------------------------------------------------------------------------
// The same operand layout and arithmetic as the LDS-staged kernel, but the
// weight, activation and scale bytes of a step travel from memory straight
// into LDS (gfx950 buffer_load ... lds: lane i of a 16-byte load lands at
// byte 16*i of the destination, 4-byte loads at 4*i), so no VGPRs hold
// loads in flight.  Each wave keeps a ring of D step slots and D - 1 steps
// in flight while it computes one.  The compiler does not see these loads
// (inline asm), so its own waits never drain the ring; the kernel waits
// with explicit vmcnt counts instead.  Its only other memory instructions
// come after the loop.
//
// Slot layout (bytes), for a 16R-row tile:
//   [0, 2048 R)          weight codes: block 2r + h holds rows 16r + 8h + q
//                        (q = 0..7) of tile r, 128 bytes each
//   [2048 R, +1024)      activation codes: rows q = 0..7, 128 bytes each
//   [+0, +256 R)         weight scales: tile r rows 0..15, 16 bytes each
//   [+256 R, +256)       activation scales: rows 0..15 (rows >= M unused)
// A 128-byte code row holds 16-byte chunk c at position c ^ q ^ h, so the
// operand reads (16 rows, one chunk each, per 16 lanes) spread over every
// bank.  Loads of rows past N or M fall outside their buffer resource and
// are never used: their outputs are not stored and tokens >= M read row
// M - 1.
template <int R>
constexpr int dma_slot_bytes() {
  return (2 * R + 1) * 1024 + (R + 1) * 256;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t raw_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int n = bytes < 0x7FFFFFFF ? (int)bytes : 0x7FFFFFFF;
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), n, kBufferWord3};
}

// lane i: 16 bytes from rsrc at voff + soff to LDS byte lds + 16 i
__device__ __forceinline__ void dma_b128(const i32x4_t& rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
// lane i: 4 bytes to LDS byte lds + 4 i
__device__ __forceinline__ void dma_b32(const i32x4_t& rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__host__ __device__ constexpr int64_t pad1k(int64_t b) { return (b + 1023) / 1024 * 1024; }

// Copy `bytes` (a multiple of 16) from rsrc into LDS at `lds`: 1 KB per wave
// instruction, chunks spread over the NW waves.  The whole source offset is
// in the per-lane operand, so lanes past `bytes` are out of range.
template <int NW>
__device__ __forceinline__ void stage_to_lds(const i32x4_t& rsrc, uint32_t lds, int64_t bytes, int wave, int lane) {
  const int chunks = (int)((bytes + 1023) / 1024);
  for (int ch = wave; ch < chunks; ch += NW) dma_b128(rsrc, lds + 1024 * ch, 1024 * ch + 16 * lane, 0);
}

template <int MT, int R, int NW, int D, bool SA, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_dma_kernel(GemvParams p) {
  static_assert(D >= 2 && D <= 4, "ring depth");
  // SA: the activation codes and scales and the tile's weight scales are
  // copied into LDS once, before the loop (as in gemv_fmma_kernel); a ring
  // slot then holds only the weight codes of a step, two 1 KB loads per row
  // tile instead of 3 R + 2 loads
  constexpr int SLOT = SA ? 2048 * R : dma_slot_bytes<R>();
  constexpr int L = SA ? 2 * R : 3 * R + 2;  // loads per step
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: step offsets go to SGPRs
  const int li = lane & 15, kg = lane >> 4;  // operand layout
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int nsteps = (int)(K / 256);
  const int n = wave < nsteps ? (nsteps - wave + NW - 1) / NW : 0;  // steps wave, wave + NW, ...
  (void)MT;

  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const i32x4_t wcr = raw_rsrc(p.w_codes + tile0 * (K / 2), rows * (K / 2));
  const i32x4_t wsr = raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16));
  const i32x4_t acr = raw_rsrc(p.a_codes, (int64_t)M * (K / 2));
  const i32x4_t asr = raw_rsrc(p.a_scales, (int64_t)M * (K / 16));
  // per-lane source offsets (every row-dependent term here, so a row past
  // the buffer is out of range whatever the step offset)
  const int q = lane >> 3, c = lane & 7;
  int vcode[2 * R], vscale[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) vcode[2 * r + h] = (16 * r + 8 * h + q) * (int)(K / 2) + 16 * (c ^ q ^ h);
    vscale[r] = (16 * r + (lane >> 2)) * (int)(K / 16) + 4 * (lane & 3);
  }

  // staged regions (SA): activation codes [MT][K/2], activation scales
  // [MT][K/16], the tile's weight scales [16 R][K/16], each padded to whole KB
  const int64_t acb = SA ? pad1k(MT * (K / 2)) : 0, asb = SA ? pad1k(MT * (K / 16)) : 0;
  const int64_t staged = SA ? acb + asb + pad1k(16 * R * (K / 16)) : 0;
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  if constexpr (SA) {
    stage_to_lds<NW>(acr, lds0, (int64_t)M * (K / 2), wave, lane);
    stage_to_lds<NW>(asr, lds0 + (uint32_t)acb, (int64_t)M * (K / 16), wave, lane);
    stage_to_lds<NW>(wsr, lds0 + (uint32_t)(acb + asb), rows * (K / 16), wave, lane);
  }
  const uint32_t ring = lds0 + (uint32_t)staged + (uint32_t)(wave * D * SLOT);
  auto issue = [&](int i) {  // the wave's i-th step into slot i % D
    const int step = wave + i * NW;
    const uint32_t s = ring + (uint32_t)((i % D) * SLOT);
    const int co = step * 128, so = step * 16;
#pragma unroll
    for (int b = 0; b < 2 * R; ++b) dma_b128(wcr, s + 1024 * b, vcode[b], co);
    if constexpr (!SA) {
      dma_b128(acr, s + 2048 * R, vcode[0], co);
#pragma unroll
      for (int r = 0; r < R; ++r) dma_b32(wsr, s + 2048 * R + 1024 + 256 * r, vscale[r], so);
      dma_b32(asr, s + 2048 * R + 1024 + 256 * R, vscale[0], so);
    }
  };

  const int btok = li < M ? li : M - 1;
  const char* lstage = reinterpret_cast<const char*>(lds4);
  const char* lbase = lstage + staged + wave * D * SLOT;
  // operand read offsets within a slot
  int wro[R][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int h = li >> 3, qq = li & 7;
      wro[r][u] = (2 * r + h) * 1024 + qq * 128 + 16 * ((2 * kg + u) ^ qq ^ h);
    }
  const int aro0 = 2048 * R + btok * 128 + 16 * ((2 * kg) ^ btok);
  const int aro1 = 2048 * R + btok * 128 + 16 * ((2 * kg + 1) ^ btok);
  const int sro = 2048 * R + 1024 + li * 16 + 4 * kg;
  const int asro = 2048 * R + 1024 + 256 * R + btok * 16 + 4 * kg;

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (j < n) issue(j);
  if constexpr (SA) {
    // this wave's staging copies (issued before the ring's first steps) have
    // landed, and after the barrier every other wave's
    if (n >= D - 1) wait_vmcnt<(D - 1) * L>();
    else wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
  }
  // staged operand offsets (SA), without the step term: token btok's codes
  // and scale word, and this lane's weight row's scale word in tile 0
  const char* sa_codes = lstage + btok * (K / 2) + 32 * kg;
  const char* sa_scale = lstage + acb + btok * (K / 16) + 4 * kg;
  const char* sw_scale = lstage + acb + asb + li * (K / 16) + 4 * kg;
  for (int i = 0; i < n; ++i) {
    if (i + D - 1 < n) {
      // into the slot of step i - 1: its operand reads must have returned
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(i + D - 1);
    }
    // steps issued after step i: min(D - 1, n - 1 - i)
    const int later = n - 1 - i;
    if (later >= D - 1) wait_vmcnt<(D - 1) * L>();
    else if (D > 3 && later == 2) wait_vmcnt<(D > 3 ? 2 * L : 0)>();
    else if (D > 2 && later == 1) wait_vmcnt<(D > 2 ? L : 0)>();
    else wait_vmcnt<0>();
    const char* sl = lbase + (i % D) * SLOT;
    const int step = wave + i * NW;
    uint4 w[R][2];
    uint32_t sw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w[r][0] = *reinterpret_cast<const uint4*>(sl + wro[r][0]);
      w[r][1] = *reinterpret_cast<const uint4*>(sl + wro[r][1]);
      sw[r] = SA ? *reinterpret_cast<const uint32_t*>(sw_scale + 16 * r * (K / 16) + step * 16)
                 : *reinterpret_cast<const uint32_t*>(sl + sro + 256 * r);
    }
    const uint4 a0 = SA ? *reinterpret_cast<const uint4*>(sa_codes + step * 128)
                        : *reinterpret_cast<const uint4*>(sl + aro0);
    const uint4 a1 = SA ? *reinterpret_cast<const uint4*>(sa_codes + step * 128 + 16)
                        : *reinterpret_cast<const uint4*>(sl + aro1);
    const uint32_t sa = SA ? *reinterpret_cast<const uint32_t*>(sa_scale + step * 16)
                           : *reinterpret_cast<const uint32_t*>(sl + asro);
    mfma_step<R>(w, sw, a0, a1, sa, acc);
  }
  __syncthreads();  // every wave is done with its ring before the reduction reuses the LDS
  mfma_finish<MT, R, NW, EPI>(p, acc, reinterpret_cast<float*>(lds4), tile0);
}

// ----------------------------------------------------------------------------
// LDS-staged VALU kernel (M <= 2, K % 256 == 0)
// ----------------------------------------------------------------------------
// The direct kernel's lane mapping and arithmetic (G lanes per weight row,
// 16 bytes per lane per step, R rows per lane, f16 dot2 block sums), but the
// activation codes and scales and the block scales of the workgroup's rows
// are copied into LDS once, with direct-to-LDS loads, before the main loop.
// The loop then issues one memory instruction per row and step, the
// non-temporal 16-byte weight load; everything else comes from LDS.
// Weight loads go through a buffer resource: chunks past K and rows past N
// read as zero without touching memory, so every lane runs the same steps
// and no load sits behind a branch (the compiler's wait before step i then
// counts exactly the loads of steps i+1 .. i+P-1).  Each LDS region is
// padded to a whole number of 1 KB copies.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // beyond any buffer resource's num_records

template <int MT, int G, int R, int NW, int P, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_staged_kernel(GemvParams p) {
  constexpr int RG = 64 / G;
  constexpr int ROWS = R * NW * RG;
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane % G;
  const int rg = lane / G;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * ROWS;
  const int64_t rows = N - tile0 < ROWS ? N - tile0 : ROWS;
  const int C = (int)(K / 32);       // 32-element chunks per row
  const int nmax = (C + G - 1) / G;  // steps of every lane (chunks g, g + G, ...)
  // LDS regions: activation codes [MT][K/2], activation scales [MT][K/16],
  // weight scales of this tile [ROWS][K/16]
  const int64_t acb = pad1k(MT * (K / 2)), asb = pad1k(MT * (K / 16));
  const uint32_t lbase = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  stage_to_lds<NW>(raw_rsrc(p.a_codes, (int64_t)M * (K / 2)), lbase, (int64_t)M * (K / 2), wave, lane);
  stage_to_lds<NW>(raw_rsrc(p.a_scales, (int64_t)M * (K / 16)), lbase + (uint32_t)acb, (int64_t)M * (K / 16), wave,
                   lane);
  stage_to_lds<NW>(raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16)), lbase + (uint32_t)(acb + asb),
                   rows * (K / 16), wave, lane);

  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  int rloc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rloc[r] = (r * NW + wave) * RG + rg;
  // a ring of P + 1 register slots, the loop unrolled over the ring: step i
  // lives in slot i % (P + 1) and the load of step i + P goes to the slot
  // step i - 1 used, so no slot is reloaded while its contents are live and
  // the compiler needs no copies (which would wait for the new loads)
  constexpr int S = P + 1;
  uint4 wb[S][R];
  auto load = [&](int slot, int i) {
    const int c = g + i * G;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t o = c < C ? (uint32_t)(rloc[r] * (int)(K / 2) + 16 * c) : kOutOfRange;
      wb[slot][r] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(wcr, (int)o, 0, 2 /* non-temporal */));
    }
  };
  // slots filled one after the other (scheduling barriers), so the wait
  // before a slot counts exactly the later slots' loads
#pragma unroll
  for (int j = 0; j < P; ++j) {
    load(j, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<P * R>();  // this wave's staging copies (issued first) have landed
  asm volatile("s_barrier" ::: "memory");  // ... and every other wave's

  const char* lds = reinterpret_cast<const char*>(lds4);
  const char* act_s = lds + acb;
  const char* w_s = lds + acb + asb;
  float acc[R][MT][2];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m][0] = acc[r][m][1] = 0.0f;

  for (int i0 = 0; i0 < nmax; i0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int i = i0 + j;
      load((j + P) % S, i + P);
      __builtin_amdgcn_sched_barrier(0);
      if (i < nmax) {
        // a lane past the row's end has zero weight codes; it reads the last
        // chunk's activation and scales so that every factor stays finite
        int c = g + i * G;
        c = c < C ? c : C - 1;
        half2_t ah[MT][16];
        float2_t saf[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int mm = m < M ? m : M - 1;  // tokens >= M reuse a valid row; never stored
          const uint4 a = *reinterpret_cast<const uint4*>(lds + mm * (K / 2) + 16 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = word_of(a, q);
            ah[m][4 * q + 0] = fp4x2<0>(word);
            ah[m][4 * q + 1] = fp4x2<1>(word);
            ah[m][4 * q + 2] = fp4x2<2>(word);
            ah[m][4 * q + 3] = fp4x2<3>(word);
          }
          saf[m] = __builtin_amdgcn_cvt_pk_f32_fp8(*reinterpret_cast<const uint16_t*>(act_s + mm * (K / 16) + 2 * c),
                                                   false);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float2_t sw =
              __builtin_amdgcn_cvt_pk_f32_fp8(*reinterpret_cast<const uint16_t*>(w_s + rloc[r] * (K / 16) + 2 * c), false);
          half2_t wh[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t word = word_of(wb[j][r], q);
            wh[4 * q + 0] = fp4x2<0>(word);
            wh[4 * q + 1] = fp4x2<1>(word);
            wh[4 * q + 2] = fp4x2<2>(word);
            wh[4 * q + 3] = fp4x2<3>(word);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              t0 = __builtin_amdgcn_fdot2(wh[k], ah[m][k], t0, false);
              t1 = __builtin_amdgcn_fdot2(wh[8 + k], ah[m][8 + k], t1, false);
            }
            acc[r][m][0] = __builtin_fmaf(t0, saf[m][0] * sw[0], acc[r][m][0]);
            acc[r][m][1] = __builtin_fmaf(t1, saf[m][1] * sw[1], acc[r][m][1]);
          }
        }
      }
    }
  }

  float scale[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) scale[m] = token_scale(p, m < M ? m : 0);
  float out[R * MT];
  int tok[R * MT];
  bool ok[R * MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m][0] + acc[r][m][1];
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      const int64_t row = tile0 + rloc[r];
      out[r * MT + m] = v * scale[m];
      tok[r * MT + m] = m;
      ok[r * MT + m] = g == 0 && row < N && m < M;
      if (ok[r * MT + m]) p.y[(int64_t)m * N + row] = out[r * MT + m];
    }
  if constexpr (EPI) {
    int rowt[R * MT];
    bool own[R * MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        rowt[r * MT + m] = rloc[r];
        own[r * MT + m] = g == 0 && m < M;
      }
    lmhead_partials<MT, ROWS, R * MT>(p, out, tok, rowt, own, ok, blockIdx.x);
  }
}

// ----------------------------------------------------------------------------
// FP4 MFMA kernel (M = 1..8, K % 256 == 0): raw E2M1 weights, block-diagonal
// activation
// ----------------------------------------------------------------------------
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 multiplies E2M1 operands
// exactly; its E8M0 scales (one per 32 elements) cannot carry NVFP4's E4M3
// scales (one per 16), so they are 1 here and the block scales are applied to
// the results.  For that every result must hold a single 16-element block:
// the A operand (16 rows) is the activation laid out block-diagonally, row
// MT*b' + j holding token j's codes of block b' of the MFMA's block group and
// zeros elsewhere, so D[MT*b' + j][n] is the exact block sum of token j with
// weight row n.  The B operand is the weight codes exactly as they sit in
// memory: no per-element decode at all.  A 128-element chunk has 8 blocks;
// one MFMA covers 16 / MT of them, so a chunk takes MT / 2 MFMAs (MT >= 2).
// Post-scaling costs two operations per result (scale product, FMA): about
// MT / 8 lane-operations per weight element, against about 1.5 for decoding
// the weights to f16.
//
// Operand layouts (checked on hardware): A lane l holds row l % 16, elements
// 32 * (l / 16) .. +31 (element t in bits 4t .. 4t+3 of the 16 bytes); B lane
// l holds column l % 16 over the same elements; D lane l holds column l % 16,
// rows 4 * (l / 16) .. +3.
//
// Loads are the direct-to-LDS ring of gemv_dma_kernel (same slot layout and
// swizzle).  Waves split K; each lane accumulates its four results per row
// tile over the wave's steps, and the final reduction adds, per weight row
// and token, the lanes and waves that hold that token in a fixed order.
typedef int v8i32_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float4_t mfma_fp4(const uint4& a, const uint4& b) {
  const v8i32_t A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i32_t B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // formats 4/4: E2M1 both; scales 127 = E8M0 1.0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, float4_t{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, 127, 0,
                                                           127);
}

template <int MT>
__device__ __forceinline__ uint32_t scale_selector(int kg) {
  if constexpr (MT == 2) return (uint32_t)(2 * kg) | (uint32_t)(2 * kg + 1) << 8;
  if constexpr (MT == 4) return (uint32_t)kg | (uint32_t)(4 + kg) << 8;
  const uint32_t x0 = (uint32_t)(kg >> 1);
  return x0 | (x0 + 2) << 8 | (x0 + 4) << 16 | (x0 + 6) << 24;
}

// The scale values a lane needs from a 16-byte record (blocks 0..7 of
// chunk 0 in its first half, chunk 1 in its second), decoded from E4M3:
// out[h][x] for chunk h and the lane's x-th block of the chunk.
template <int MT>
__device__ __forceinline__ void gather_scales(const uint4& rec, uint32_t sel, float (&out)[2][MT == 8 ? 4 : 2]) {
  if constexpr (MT == 8) {
    const uint32_t d0 = __builtin_amdgcn_perm(rec.y, rec.x, sel), d1 = __builtin_amdgcn_perm(rec.w, rec.z, sel);
    const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(d0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(d0, true);
    const float2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(d1, false), e = __builtin_amdgcn_cvt_pk_f32_fp8(d1, true);
    out[0][0] = a[0], out[0][1] = a[1], out[0][2] = b[0], out[0][3] = b[1];
    out[1][0] = c[0], out[1][1] = c[1], out[1][2] = e[0], out[1][3] = e[1];
  } else {
    // two selected bytes of each half, then both pairs in one word
    const uint32_t lo = __builtin_amdgcn_perm(rec.y, rec.x, sel), hi = __builtin_amdgcn_perm(rec.w, rec.z, sel);
    const uint32_t d = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(d, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(d, true);
    out[0][0] = a[0], out[0][1] = a[1];
    out[1][0] = b[0], out[1][1] = b[1];
  }
}

template <int MT, int R, int NW, int D, bool SA, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_fmma_kernel(GemvParams p) {
  static_assert(MT == 2 || MT == 4 || MT == 8, "tokens per block row group");
  static_assert(D >= 2 && D <= 4, "ring depth");
  // SA: the activation codes and scales and the tile's weight scales are
  // copied into LDS once, before the loop; a ring slot then holds only the
  // weight codes of a step
  constexpr int SLOT = SA ? 2048 * R : dma_slot_bytes<R>();
  constexpr int L = SA ? 2 * R : 3 * R + 2;  // loads per step
  constexpr int BPM = 16 / MT;   // blocks per MFMA
  constexpr int S = MT / 2;      // MFMAs per 128-element chunk and row tile
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kg = lane >> 4;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int nsteps = (int)(K / 256);
  const int n = wave < nsteps ? (nsteps - wave + NW - 1) / NW : 0;  // steps wave, wave + NW, ...

  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const i32x4_t wcr = raw_rsrc(p.w_codes + tile0 * (K / 2), rows * (K / 2));
  const i32x4_t wsr = raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16));
  const i32x4_t acr = raw_rsrc(p.a_codes, (int64_t)M * (K / 2));
  const i32x4_t asr = raw_rsrc(p.a_scales, (int64_t)M * (K / 16));
  const int q = lane >> 3, c = lane & 7;
  int vcode[2 * R], vscale[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) vcode[2 * r + h] = (16 * r + 8 * h + q) * (int)(K / 2) + 16 * (c ^ q ^ h);
    vscale[r] = (16 * r + (lane >> 2)) * (int)(K / 16) + 4 * (lane & 3);
  }
  // staged regions (SA): activation codes [MT][K/2], activation scales
  // [MT][K/16], the tile's weight scales [16 R][K/16], each padded to whole KB
  const int64_t acb = SA ? pad1k(MT * (K / 2)) : 0, asb = SA ? pad1k(MT * (K / 16)) : 0;
  const int64_t staged = SA ? acb + asb + pad1k(16 * R * (K / 16)) : 0;
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  if constexpr (SA) {
    stage_to_lds<NW>(acr, lds0, (int64_t)M * (K / 2), wave, lane);
    stage_to_lds<NW>(asr, lds0 + (uint32_t)acb, (int64_t)M * (K / 16), wave, lane);
    stage_to_lds<NW>(wsr, lds0 + (uint32_t)(acb + asb), rows * (K / 16), wave, lane);
  }
  const uint32_t ring = lds0 + (uint32_t)staged + (uint32_t)(wave * D * SLOT);
  auto issue = [&](int i) {  // the wave's i-th step into slot i % D
    const int step = wave + i * NW;
    const uint32_t s = ring + (uint32_t)((i % D) * SLOT);
    const int co = step * 128, so = step * 16;
#pragma unroll
    for (int b = 0; b < 2 * R; ++b) dma_b128(wcr, s + 1024 * b, vcode[b], co);
    if constexpr (!SA) {
      dma_b128(acr, s + 2048 * R, vcode[0], co);
#pragma unroll
      for (int r = 0; r < R; ++r) dma_b32(wsr, s + 2048 * R + 1024 + 256 * r, vscale[r], so);
      dma_b32(asr, s + 2048 * R + 1024 + 256 * R, vscale[0], so);
    }
  };

  // A side (this lane as an A row): token j, block b' of the MFMA's group
  const int ja = li % MT, ba = li / MT;
  // D side (this lane's four results): row 4*kg + v is token (4kg+v) % MT of
  // block (4kg+v) / MT of the group
  const char* lstage = reinterpret_cast<const char*>(lds4);
  const char* lbase = lstage + staged + wave * D * SLOT;
  int wro[R][2];  // this lane's B chunk (row li, chunk 4h + kg) in each tile
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int hh = li >> 3, qq = li & 7;
      wro[r][h] = (2 * r + hh) * 1024 + qq * 128 + 16 * ((4 * h + kg) ^ qq ^ hh);
    }
  const int aro[2] = {2048 * R + ja * 128 + 16 * ((kg) ^ ja), 2048 * R + ja * 128 + 16 * ((4 + kg) ^ ja)};
  const int wso = 2048 * R + 1024 + li * 16;       // + 256 r: this lane's weight row scale record
  const int aso = 2048 * R + 1024 + 256 * R;       // + 16 j: token j's scale record
  constexpr int SX = MT == 8 ? 4 : 2;              // scale values per chunk h
  const uint32_t sel = scale_selector<MT>(kg);

  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[r][v] = 0.0f;

#pragma unroll
  for (int jj = 0; jj < D - 1; ++jj)
    if (jj < n) issue(jj);
  if constexpr (SA) {
    // this wave's staging copies (issued before the ring's first steps) have
    // landed, and after the barrier every other wave's
    if (n >= D - 1) wait_vmcnt<(D - 1) * L>();
    else wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
  }
  for (int i = 0; i < n; ++i) {
    if (i + D - 1 < n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reused slot's reads have returned
      issue(i + D - 1);
    }
    const int later = n - 1 - i;
    if (later >= D - 1) wait_vmcnt<(D - 1) * L>();
    else if (D > 3 && later == 2) wait_vmcnt<(D > 3 ? 2 * L : 0)>();
    else if (D > 2 && later == 1) wait_vmcnt<(D > 2 ? L : 0)>();
    else wait_vmcnt<0>();
    const char* sl = lbase + (i % D) * SLOT;
    const int step = wave + i * NW;
    // scale records of the step: from the slot, or from the staged copies
    const char* wrec = SA ? lstage + acb + asb + li * (K / 16) + step * 16 : sl + wso;
    const int64_t wrec_r = SA ? 16 * (K / 16) : 256;  // to the same row of the next tile
    const char* arec = SA ? lstage + acb + step * 16 : sl + aso;
    const int64_t arec_j = SA ? K / 16 : 16;  // to the next token
    // the scales this lane's results need, gathered from the step's 16-byte
    // scale records with one byte permute per 4 bytes (selectors fixed per
    // lane) and decoded: sw[r][h][x] for its weight row, sa[v][h][x] for the
    // token of result v; x = v / 2 (MT = 2) or the MFMA index s (MT = 4, 8)
    float sw[R][2][SX], sa[4][2][SX];
#pragma unroll
    for (int r = 0; r < R; ++r) gather_scales<MT>(*reinterpret_cast<const uint4*>(wrec + r * wrec_r), sel, sw[r]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (MT == 2 && v >= 2) {  // tokens repeat: v and v - 2 hold the same token
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int x = 0; x < SX; ++x) sa[v][h][x] = sa[v - 2][h][x];
      } else {
        gather_scales<MT>(*reinterpret_cast<const uint4*>(arec + ((4 * kg + v) % MT) * arec_j), sel, sa[v]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 wb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) wb[r] = *reinterpret_cast<const uint4*>(sl + wro[r][h]);
      const char* aptr = SA ? lstage + ja * (K / 2) + step * 128 + 64 * h + 16 * kg : sl + aro[h];
      const uint4 av = ja < M ? *reinterpret_cast<const uint4*>(aptr) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int b = s * BPM + ba;  // block (0..7 of the chunk) of this lane's A row
        const bool keep = kg == (b >> 1);
        const bool hi = (b & 1) != 0;
        const uint4 A = make_uint4(keep && !hi ? av.x : 0u, keep && !hi ? av.y : 0u, keep && hi ? av.z : 0u,
                                   keep && hi ? av.w : 0u);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float4_t d = mfma_fp4(A, wb[r]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int x = MT == 2 ? v >> 1 : s;
            acc[r][v] = __builtin_fmaf(d[v], sw[r][h][x] * sa[v][h][x], acc[r][v]);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its ring before the reduction reuses the LDS

  // reduction: red[wave][r][v][lane], then y[j][row] = sum over waves and
  // over the lanes (kg) and results (v) that hold token j, in a fixed order
  float* red = reinterpret_cast<float*>(lds4);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * R + r) * 4 + v) * 64 + lane] = acc[r][v];
  __syncthreads();
  constexpr int OUTS = 16 * R * MT;                     // (row, token) results of the tile
  constexpr int NV = (OUTS + NW * 64 - 1) / (NW * 64);  // per thread
  float tsc[NV];  // global scales, loaded before the first store
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int j = ((int)threadIdx.x + u * NW * 64) % MT;
    tsc[u] = token_scale(p, j < M ? j : 0);
  }
  float out[NV];
  int tok[NV], rowt[NV];
  bool ok[NV], own[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int o = (int)threadIdx.x + u * NW * 64;
    out[u] = 0.0f;
    tok[u] = 0;
    rowt[u] = 0;
    ok[u] = own[u] = false;
    if (o < OUTS) {
      const int j = o % MT, rt = o / MT;  // token, row of the tile (16 r + nn)
      const int r = rt >> 4, nn = rt & 15;
      float sum = 0.0f;
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if ((4 * g + v) % MT == j) sum += red[((w * R + r) * 4 + v) * 64 + g * 16 + nn];
      const int64_t row = tile0 + rt;
      out[u] = sum * tsc[u];
      tok[u] = j;
      rowt[u] = rt;
      own[u] = j < M;
      ok[u] = j < M && rt < rows;
      if (ok[u]) p.y[(int64_t)j * N + row] = out[u];
    }
  }
  if constexpr (EPI) lmhead_partials<MT, 16 * R, NV>(p, out, tok, rowt, own, ok, blockIdx.x);
}

// ----------------------------------------------------------------------------
// Streaming MFMA kernels: weights straight from HBM into MFMA operands
// ----------------------------------------------------------------------------
// Both kernels below load the weight codes straight into the register
// operand of an MFMA, with no LDS staging, barrier or transpose in the loop.
// The 16 weight-side rows of the MFMA tile are 4 weight rows x 4 windows of
// K: weight lane (j, kg), j = lane % 16, kg = lane / 16, holds row j / 4 of
// the row group, window w = j % 4: the 16 bytes (32 codes) at byte
// 64 kg + 16 w of the row's 256-byte chunk (512 elements).  So the four
// lanes of a quad read 64 contiguous bytes of one row and a wave instruction
// reads 4 rows x 256 bytes: the address unit sees whole 64-byte quads.  (A
// row per column of the tile puts every lane of a quad on another cache line;
// that stalls the address unit four times as often and costs more than the
// arithmetic does.)  A window is the 4 pieces of 16 bytes with the same w;
// the activation side takes the same pieces, the MFMA sums over k, and only
// the results whose two sides share a window are used: lane l holds them as
// its accumulator entry l % 4.
// Before the loop every workgroup copies the activation codes and scales and
// its rows' block scales into LDS with direct-to-LDS loads of whole
// contiguous kilobytes, so the loop's only memory instructions are the
// weight-code loads (small scattered scale loads next to the code stream
// cost more HBM time than they carry).  Each wave keeps U chunks of loads in
// flight in a register ring (non-temporal loads) over R row groups of 4
// rows; waves split the chunks of K and the finish adds the waves' results
// in a fixed order.  Rows past the workgroup's rows get a per-lane offset
// outside the buffer and read as zeros; the chunk offset is a scalar operand
// (not range-checked), which only ever addresses bytes inside the rows.
constexpr int kStreamChunk = 512;          // K elements per chunk and row
constexpr int kStream8Chunk = 256;         // K elements per chunk and row of the eight-token form
constexpr uint32_t kOffOut = 0x80000000u;  // beyond any buffer resource used here
// A scalar offset that moves every lane's offset (kOffOut included, without
// wrapping) past the end of any buffer under 1 GiB: such a load reads zeros
// and makes no memory request (a larger buffer gets an in-bounds read)
constexpr int kPastEnd = 0x40000000;

// 32 codes (one 16-byte word) times two block scales (16 elements each) ->
// four f16 operands of 8 elements
__device__ __forceinline__ void decode32_scaled(const u32x4_t& v, uint32_t s2, half8_t (&out)[4]) {
  const float2_t s = __builtin_amdgcn_cvt_pk_f32_fp8(s2, false);
  const half2_t h0 = as_half2(pack_f16x2(s[0], s[0])), h1 = as_half2(pack_f16x2(s[1], s[1]));
  out[0] = wdecode8_scaled(v[0], h0);
  out[1] = wdecode8_scaled(v[1], h0);
  out[2] = wdecode8_scaled(v[2], h1);
  out[3] = wdecode8_scaled(v[3], h1);
}

// LDS the streaming kernels stage: activation codes [T][K/2] and scales
// [T][K/16] for T tokens, the tile's block scales [tile_rows][K/16]
__host__ __device__ constexpr int64_t stream_lds_bytes(int T, int64_t K, int64_t tile_rows) {
  return pad1k(T * (K / 2)) + pad1k(T * (K / 16)) + pad1k(tile_rows * (K / 16));
}

// Copies the activation (rows >= M are never read for a stored result) and
// the tile's block scales into LDS; returns the LDS offsets of the three
// regions through acb / asb (activation scales at acb, block scales at
// acb + asb).
template <int NW>
__device__ __forceinline__ void stream_stage(const GemvParams& p, int T, int64_t rows, int64_t tile0, int wave,
                                             int lane, int64_t& acb, int64_t& asb) {
  const int64_t K = p.K;
  const int M = p.M;
  acb = pad1k(T * (K / 2));
  asb = pad1k(T * (K / 16));
  extern __shared__ uint4 lds4[];
  const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  stage_to_lds<NW>(raw_rsrc(p.a_codes, (int64_t)M * (K / 2)), l0, (int64_t)M * (K / 2), wave, lane);
  stage_to_lds<NW>(raw_rsrc(p.a_scales, (int64_t)M * (K / 16)), l0 + (uint32_t)acb, (int64_t)M * (K / 16), wave, lane);
  stage_to_lds<NW>(raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16)), l0 + (uint32_t)(acb + asb),
                   rows * (K / 16), wave, lane);
}

// (a) f16 form, M <= MT (MT = 4 or 8), K % 512 == 0.  The token side of an
// MFMA is 4 tokens x the 4 windows (token lane (i, kg): token i / 4 of the
// set, window i % 4, the same 32 elements of the token's codes); MT = 8 runs
// two sets of tokens against each decoded weight operand.  Both sides are
// decoded to exact f16 values E2M1 * E4M3 (at most 6 significant bits) and
// v_mfma_f32_16x16x32_f16 adds the products: D[4 wr + w][4 t + w] is row wr
// with token t over window w.  Tokens >= M read as zeros.
// Each chunk's activation codes and scales (256 contiguous bytes per token,
// which every workgroup reads, so they stay in L2) come from global memory
// into the register ring beside the weights'; only the tile's block scales
// are copied into LDS.  Staging the whole activation in LDS instead held
// every wave at a barrier until up to 115 KB had landed, and measured slower.
template <int MT, int R, int NW, int U, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_stream_kernel(GemvParams p) {
  static_assert(MT == 4 || MT == 8, "token sets of 4");
  constexpr int S = MT / 4;  // token sets
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int jr = j >> 2, jw = j & 3;  // row (weight side) / token (token side), window
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const int nchunks = (int)(K / kStreamChunk);
  const int n = wave < nchunks ? (nchunks - wave + NW - 1) / NW : 0;  // chunks wave, wave + NW, ...

  const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  stage_to_lds<NW>(raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16)), l0, rows * (K / 16), wave, lane);
  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t acr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_codes), (short)0,
                                                                      (int)(M * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t asr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), (short)0,
                                                                      (int)(M * (K / 16)), kBufferWord3);
  const int b0 = 64 * kg + 16 * jw;  // byte of this lane within a row's chunk
  uint32_t vw[R];
  const char* lds = reinterpret_cast<const char*>(lds4);
  const char* lsw[R];  // block scales of each row group's row (+ 32 c); rows past the tile read the last row's
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = 4 * r + jr;
    vw[r] = row < rows ? (uint32_t)(row * (int)(K / 2) + b0) : kOffOut;
    lsw[r] = lds + (row < rows ? row : (int)rows - 1) * (K / 16) + b0 / 8;
  }
  uint32_t va[S], vsa[S];  // buffer offsets of the token's codes (+ 256 c) and scales (+ 32 c); past M: zeros
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = 4 * s + jr;
    va[s] = t < M ? (uint32_t)(t * (int)(K / 2) + b0) : kOffOut;
    vsa[s] = t < M ? (uint32_t)(t * (int)(K / 16) + b0 / 8) : kOffOut;
  }

  float4_t acc[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) acc[r][s] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t ring[U][R];
  u32x4_t aring[U][S];
  uint32_t sring[U][S];
  auto load = [&](int u, int i) {  // the wave's i-th chunk into slot u; past the last, zeros (never used)
    const int c = wave + i * NW;
    const int co = i < n ? c * 256 : kPastEnd, so = i < n ? c * 32 : kPastEnd;
#pragma unroll
    for (int r = 0; r < R; ++r)
      ring[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wcr, (int)vw[r], co, 2 /* non-temporal */);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      aring[u][s] = __builtin_amdgcn_raw_buffer_load_b128(acr, (int)va[s], co, 0);
      sring[u][s] = __builtin_amdgcn_raw_buffer_load_b16(asr, (int)vsa[s], so, 0);
    }
  };
  if (n > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  constexpr int kRingLoads = U * (R + 2 * S);
  // This wave's staging copies (issued before the ring loads) have landed ...
  if (n > 0) wait_vmcnt<(kRingLoads < 63 ? kRingLoads : 63)>();
  else wait_vmcnt<0>();  // a wave with no chunks issued no ring loads to count past
  asm volatile("s_barrier" ::: "memory");   // ... and every other wave's
  if (n > 0) {
    for (int i0 = 0; i0 < n; i0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u;
        const int c = wave + (i < n ? i : n - 1) * NW;
        u32x4_t w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = ring[u][r];
        u32x4_t ga[S];
        uint32_t gs[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          ga[s] = aring[u][s];
          gs[s] = sring[u][s];
        }
        load(u, i + U);
        __builtin_amdgcn_sched_barrier(0);
        if (i < n) {
          half8_t b[S][4];
#pragma unroll
          for (int s = 0; s < S; ++s) decode32_scaled(ga[s], gs[s], b[s]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            half8_t a[4];
            decode32_scaled(w[r], *reinterpret_cast<const uint16_t*>(lsw[r] + 32 * c), a);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int s = 0; s < S; ++s)
                acc[r][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[q], b[s][q], acc[r][s], 0, 0, 0);
          }
        }
      }
    }
  }

  // finish: lane l's entry l % 4 holds row 4 r + l / 16 with token (l % 16) / 4
  // of set s over window l % 4; output (t, row) = the sum over waves and the
  // four windows (lanes 16 (row % 4) + 4 (t % 4) + w, entry w)
  __syncthreads();  // every wave is done with the staged data before the reduction reuses the LDS
  float* red = reinterpret_cast<float*>(lds4);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) red[((wave * R + r) * S + s) * 64 + lane] = acc[r][s][lane & 3];
  __syncthreads();
  constexpr int OUTS = 4 * R * MT;
  constexpr int NV = (OUTS + NW * 64 - 1) / (NW * 64);
  float tsc[NV];  // global scales, all loaded before the first store
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int t = ((int)threadIdx.x + u * NW * 64) / (4 * R);
    tsc[u] = token_scale(p, t < M ? t : 0);
  }
  float out[NV];
  int tok[NV], rowt[NV];
  bool ok[NV], own[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int o = (int)threadIdx.x + u * NW * 64;
    out[u] = 0.0f;
    tok[u] = 0;
    rowt[u] = 0;
    ok[u] = own[u] = false;
    if (o < OUTS) {
      const int rt = o % (4 * R), t = o / (4 * R);  // consecutive threads: consecutive rows
      const int r = rt >> 2, wr = rt & 3, s = t >> 2, tt = t & 3;
      float sum = 0.0f;
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) sum += red[((w * R + r) * S + s) * 64 + 16 * wr + 4 * tt + ww];
      out[u] = sum * tsc[u];
      tok[u] = t;
      rowt[u] = rt;
      own[u] = t < M;
      ok[u] = t < M && rt < rows;
      if (ok[u]) p.y[(int64_t)t * N + tile0 + rt] = out[u];
    }
  }
  if constexpr (EPI) lmhead_partials<MT, 4 * R, NV>(p, out, tok, rowt, own, ok, blockIdx.x);
}

// (a2) Eight-token f16 form, M <= 8 S, K % 256 == 0.  The operand layout of
// form (a) with two windows instead of four: lane (j, kg) holds row (or
// token) j / 2 and window j % 2, the 16 bytes at byte 32 kg + 16 (j % 2) of
// the row's 128-byte chunk, so a wave instruction reads 8 rows x 128 B (a
// whole cache line per row).  The token side holds all 8 tokens, and
// D[2 wr + w][2 t + w] is row wr with token t over window w: half of each
// MFMA's results are used, against a quarter for form (a) with two sets of
// 4 tokens, which halves the MFMA work at M = 5..8.  The activation of each
// chunk comes from L2 into the register ring beside the weights; only the
// tile's block scales are staged in LDS.  Tokens >= M read as zeros.  With
// S sets of 8 tokens (MT = 8 S, S = 1 or 2) each decoded weight operand
// meets S token operands.
template <int R, int NW, int U, bool EPI, int S = 1>
__global__ __launch_bounds__(NW * 64) void gemv_stream8_kernel(GemvParams p) {
  constexpr int MT = 8 * S;
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int jr = j >> 1, jw = j & 1;  // row (weight side) / token (token side), window
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const int nchunks = (int)(K / kStream8Chunk);
  const int n = wave < nchunks ? (nchunks - wave + NW - 1) / NW : 0;  // chunks wave, wave + NW, ...

  const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  stage_to_lds<NW>(raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16)), l0, rows * (K / 16), wave, lane);
  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t acr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_codes), (short)0,
                                                                      (int)(M * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t asr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), (short)0,
                                                                      (int)(M * (K / 16)), kBufferWord3);
  const int b0 = 32 * kg + 16 * jw;  // byte of this lane within a row's chunk
  uint32_t vw[R];
  const char* lds = reinterpret_cast<const char*>(lds4);
  const char* lsw[R];  // block scales of each row group's row (+ 16 c); rows past the tile read the last row's
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = 8 * r + jr;
    vw[r] = row < rows ? (uint32_t)(row * (int)(K / 2) + b0) : kOffOut;
    lsw[r] = lds + (row < rows ? row : (int)rows - 1) * (K / 16) + b0 / 8;
  }
  // token 8 s + j / 2's codes (+ 128 c) and scales (+ 16 c); past M: zeros
  uint32_t va[S], vsa[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = 8 * s + jr;
    va[s] = t < M ? (uint32_t)(t * (int)(K / 2) + b0) : kOffOut;
    vsa[s] = t < M ? (uint32_t)(t * (int)(K / 16) + b0 / 8) : kOffOut;
  }

  float4_t acc[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) acc[r][s] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t ring[U][R];
  u32x4_t aring[U][S];
  uint32_t sring[U][S];
  auto load = [&](int u, int i) {  // the wave's i-th chunk into slot u; past the last, zeros (never used)
    const int c = wave + i * NW;
    const int co = i < n ? c * 128 : kPastEnd, so = i < n ? c * 16 : kPastEnd;
#pragma unroll
    for (int r = 0; r < R; ++r)
      ring[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wcr, (int)vw[r], co, 2 /* non-temporal */);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      aring[u][s] = __builtin_amdgcn_raw_buffer_load_b128(acr, (int)va[s], co, 0);
      sring[u][s] = __builtin_amdgcn_raw_buffer_load_b16(asr, (int)vsa[s], so, 0);
    }
  };
  if (n > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  constexpr int kRingLoads = U * (R + 2 * S);
  // This wave's staging copies (issued before the ring loads) have landed ...
  if (n > 0) wait_vmcnt<(kRingLoads < 63 ? kRingLoads : 63)>();
  else wait_vmcnt<0>();  // a wave with no chunks issued no ring loads to count past
  asm volatile("s_barrier" ::: "memory");   // ... and every other wave's
  if (n > 0) {
    for (int i0 = 0; i0 < n; i0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u;
        const int c = wave + (i < n ? i : n - 1) * NW;
        u32x4_t w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = ring[u][r];
        u32x4_t ga[S];
        uint32_t gs[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          ga[s] = aring[u][s];
          gs[s] = sring[u][s];
        }
        load(u, i + U);
        __builtin_amdgcn_sched_barrier(0);
        if (i < n) {
          half8_t b[S][4];
#pragma unroll
          for (int s = 0; s < S; ++s) decode32_scaled(ga[s], gs[s], b[s]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            half8_t a[4];
            decode32_scaled(w[r], *reinterpret_cast<const uint16_t*>(lsw[r] + 16 * c), a);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int s = 0; s < S; ++s)
                acc[r][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[q], b[s][q], acc[r][s], 0, 0, 0);
          }
        }
      }
    }
  }

  // finish: lane l = 16 g + i holds, in entry e = (i % 2) + 2 h of set s,
  // row 8 r + 2 g + h with token 8 s + i / 2 over window i % 2; output
  // (t, row) = the sum over waves and the two windows (lanes 16 g + 2 t + w)
  __syncthreads();  // every wave is done with the staged scales before the reduction reuses the LDS
  float* red = reinterpret_cast<float*>(lds4);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        red[(((wave * R + r) * S + s) * 2 + h) * 64 + lane] = acc[r][s][(lane & 1) + 2 * h];
  __syncthreads();
  constexpr int OUTS = 8 * R * MT;
  constexpr int NV = (OUTS + NW * 64 - 1) / (NW * 64);
  float tsc[NV];  // global scales, all loaded before the first store
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int t = ((int)threadIdx.x + u * NW * 64) / (8 * R);
    tsc[u] = token_scale(p, t < M ? t : 0);
  }
  float out[NV];
  int tok[NV], rowt[NV];
  bool ok[NV], own[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int o = (int)threadIdx.x + u * NW * 64;
    out[u] = 0.0f;
    tok[u] = 0;
    rowt[u] = 0;
    ok[u] = own[u] = false;
    if (o < OUTS) {
      const int rt = o % (8 * R), t = o / (8 * R);  // consecutive threads: consecutive rows
      const int r = rt >> 3, g = (rt & 7) >> 1, h = rt & 1, s = t >> 3, tt = t & 7;
      float sum = 0.0f;
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int ww = 0; ww < 2; ++ww) sum += red[(((w * R + r) * S + s) * 2 + h) * 64 + 16 * g + 2 * tt + ww];
      out[u] = sum * tsc[u];
      tok[u] = t;
      rowt[u] = rt;
      own[u] = t < M;
      ok[u] = t < M && rt < rows;
      if (ok[u]) p.y[(int64_t)t * N + tile0 + rt] = out[u];
    }
  }
  if constexpr (EPI) lmhead_partials<MT, 8 * R, NV>(p, out, tok, rowt, own, ok, blockIdx.x);
}

// (c) Wave-owned rows, for many-row projections at M = 2..8 (K % 512 == 0):
// the operand layout and ring of form (a), but each wave owns 4 R rows of
// the workgroup's NW x 4 R and streams every chunk of K for them, so a
// workgroup stages the activation (and its rows' block scales) once for
// NW x 4 R rows, and no partial sums cross waves: a row's four windows are
// added inside the lane quad that holds them (DPP), then stored.
template <int MT, int R, int NW, int U, bool AG = false>
__global__ __launch_bounds__(NW * 64) void gemv_wstream_kernel(GemvParams p) {
  static_assert(MT == 4 || MT == 8, "token sets of 4");
  constexpr int S = MT / 4;  // token sets
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int jr = j >> 2, jw = j & 3;  // row (weight side) / token (token side), window
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const int n = (int)(K / kStreamChunk);
  const int wrow0 = wave * 4 * R;  // first row of this wave within the tile

  int64_t acb, asb;
  if constexpr (AG) {
    acb = asb = 0;
    const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
    stage_to_lds<NW>(raw_rsrc(p.w_scales + tile0 * (K / 16), rows * (K / 16)), l0, rows * (K / 16), wave, lane);
  } else {
    stream_stage<NW>(p, MT, rows, tile0, wave, lane, acb, asb);
  }
  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t acr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_codes), (short)0,
                                                                      (int)(M * (K / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t asr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), (short)0,
                                                                      (int)(M * (K / 16)), kBufferWord3);
  const int b0 = 64 * kg + 16 * jw;  // byte of this lane within a row's chunk
  uint32_t vw[R];
  const char* lds = reinterpret_cast<const char*>(lds4);
  const char* lsw[R];  // block scales of each row group's row (+ 32 c); rows past the tile read the last row's
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = wrow0 + 4 * r + jr;
    vw[r] = row < rows ? (uint32_t)(row * (int)(K / 2) + b0) : kOffOut;
    lsw[r] = lds + acb + asb + (row < rows ? row : (int)rows - 1) * (K / 16) + b0 / 8;
  }
  bool tin[S];
  const char* la[S];
  const char* lsa[S];
  uint32_t va[S], vsa[S];  // AG: buffer offsets of the token's codes (+ 256 c) and scales (+ 32 c)
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = 4 * s + jr;
    tin[s] = t < M;
    la[s] = lds + (t < M ? t : 0) * (K / 2) + b0;               // + 256 c
    lsa[s] = lds + acb + (t < M ? t : 0) * (K / 16) + b0 / 8;   // + 32 c
    va[s] = t < M ? (uint32_t)(t * (int)(K / 2) + b0) : kOffOut;
    vsa[s] = t < M ? (uint32_t)(t * (int)(K / 16) + b0 / 8) : kOffOut;
  }

  float4_t acc[R][S];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) acc[r][s] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t ring[U][R];
  u32x4_t aring[U][AG ? S : 1];
  uint32_t sring[U][AG ? S : 1];
  auto load = [&](int u, int i) {  // chunk i into slot u; past the last, zeros (never used)
    const int co = i < n ? i * 256 : kPastEnd, so = i < n ? i * 32 : kPastEnd;
#pragma unroll
    for (int r = 0; r < R; ++r)
      ring[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wcr, (int)vw[r], co, 2 /* non-temporal */);
    if constexpr (AG) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        aring[u][s] = __builtin_amdgcn_raw_buffer_load_b128(acr, (int)va[s], co, 0);
        sring[u][s] = __builtin_amdgcn_raw_buffer_load_b16(asr, (int)vsa[s], so, 0);
      }
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    load(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int kRingLoads = U * (R + (AG ? 2 * S : 0));
  wait_vmcnt<(kRingLoads < 63 ? kRingLoads : 63)>();  // this wave's staging copies (issued first) have landed ...
  asm volatile("s_barrier" ::: "memory");   // ... and every other wave's
  for (int i0 = 0; i0 < n; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      const int c = i < n ? i : n - 1;
      u32x4_t w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = ring[u][r];
      u32x4_t ga[AG ? S : 1];
      uint32_t gs[AG ? S : 1];
      if constexpr (AG) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          ga[s] = aring[u][s];
          gs[s] = sring[u][s];
        }
      }
      load(u, i + U);
      __builtin_amdgcn_sched_barrier(0);
      if (i < n) {
        half8_t b[S][4];
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if constexpr (AG) {
            decode32_scaled(ga[s], gs[s], b[s]);  // tokens >= M loaded zeros
          } else {
            const uint4 a4 = *reinterpret_cast<const uint4*>(la[s] + 256 * c);
            const u32x4_t av = tin[s] ? u32x4_t{a4.x, a4.y, a4.z, a4.w} : u32x4_t{0u, 0u, 0u, 0u};
            const uint32_t as = tin[s] ? *reinterpret_cast<const uint16_t*>(lsa[s] + 32 * c) : 0u;
            decode32_scaled(av, as, b[s]);
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          half8_t a[4];
          decode32_scaled(w[r], *reinterpret_cast<const uint16_t*>(lsw[r] + 32 * c), a);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int s = 0; s < S; ++s)
              acc[r][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[q], b[s][q], acc[r][s], 0, 0, 0);
        }
      }
    }
  }

  // finish: lane l's entry l % 4 holds row 4 r + l / 16 with token (l % 16) / 4
  // of set s over window l % 4; a quad of lanes holds the four windows of one
  // (row, token): add them inside the quad, then its first lane stores
  const int qrow = lane >> 4, qtok = (lane >> 2) & 3;
  float tsc[S];
#pragma unroll
  for (int s = 0; s < S; ++s) tsc[s] = token_scale(p, 4 * s + qtok < M ? 4 * s + qtok : 0);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float v = acc[r][s][lane & 3];
      v += __uint_as_float(__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0xB1, 0xF, 0xF, false));
      v += __uint_as_float(__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x4E, 0xF, 0xF, false));
      const int t = 4 * s + qtok, row = wrow0 + 4 * r + qrow;
      if ((lane & 3) == 0 && t < M && row < rows) p.y[(int64_t)t * N + tile0 + row] = v * tsc[s];
    }
}

// (b) FP4 form, M = 1, K % 512 == 0.  The weight codes go into
// v_mfma_scale_f32_16x16x128_f8f6f4 as they are (E2M1 x E2M1 products are
// exact, its E8M0 scales stay 1), so no weight element is decoded.  NVFP4's
// E4M3 scales cover 16 elements, so every used result must hold a single
// 16-element block: the activation side is block-diagonal.  A lane's 32
// elements are two blocks (its low and high 8 bytes); activation row
// i = 4 b + w holds window w and, in the chunk's MFMA s (s = 0, 1), only
// half s of k-group b, so D[4 b + w][4 wr + w] is the exact block sum of row
// wr over the block 8 b + 2 w + s of the chunk (bytes 64 b + 16 w + 8 s).
// Lane l's used entry l % 4 is scaled by its two E4M3 block scales and added
// up in f32: about 12 vector operations per 16 bytes of codes per lane,
// against about 36 for decoding them to f16.
template <int R, int NW, int U, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_fstream_kernel(GemvParams p) {
  extern __shared__ uint4 lds4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int jr = j >> 2, jw = j & 3;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  const int64_t tile0 = (int64_t)blockIdx.x * p.tile_rows;
  const int64_t rows = N - tile0 < p.tile_rows ? N - tile0 : p.tile_rows;
  const int nchunks = (int)(K / kStreamChunk);
  const int n = wave < nchunks ? (nchunks - wave + NW - 1) / NW : 0;

  int64_t acb, asb;
  stream_stage<NW>(p, 1, rows, tile0, wave, lane, acb, asb);
  const __amdgpu_buffer_rsrc_t wcr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w_codes + tile0 * (K / 2)), (short)0, (int)(rows * (K / 2)), kBufferWord3);
  const int b0 = 64 * kg + 16 * jw;
  // this lane's used result: row jr, window jw, blocks 8 kg + 2 jw + s (the
  // same byte offset as its own weight codes, b0 / 8 + s)
  const char* lds = reinterpret_cast<const char*>(lds4);
  uint32_t vw[R];
  const char* lsw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = 4 * r + jr;
    vw[r] = row < rows ? (uint32_t)(row * (int)(K / 2) + b0) : kOffOut;
    lsw[r] = lds + acb + asb + (row < rows ? row : (int)rows - 1) * (K / 16) + b0 / 8;  // + 32 c
  }
  // activation side of this lane (A row j = 4 b + w, b = jr, w = jw): the
  // token's codes at b0 (+ 256 c), kept in MFMA s only if kg == b
  const char* la = lds + b0;
  const char* lsa = lds + acb + b0 / 8;  // + 32 c: the two block scales of the used result
  const uint32_t keep = kg == jr ? ~0u : 0u;

  float4_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t ring[U][R];
  auto load = [&](int u, int i) {
    const int c = wave + (i < n ? i : n - 1) * NW;
#pragma unroll
    for (int r = 0; r < R; ++r)
      ring[u][r] = __builtin_amdgcn_raw_buffer_load_b128(wcr, (int)vw[r], c * 256, 2 /* non-temporal */);
  };
  if (n > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<(U * R < 63 ? U * R : 63)>();  // this wave's staging copies (issued first) have landed ...
  asm volatile("s_barrier" ::: "memory");   // ... and every other wave's
  if (n > 0) {
    for (int i0 = 0; i0 < n; i0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u;
        const int c = wave + (i < n ? i : n - 1) * NW;
        u32x4_t w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) w[r] = ring[u][r];
        load(u, i + U);
        __builtin_amdgcn_sched_barrier(0);
        if (i < n) {
          const uint4 av = *reinterpret_cast<const uint4*>(la + 256 * c);
          const float2_t sa = __builtin_amdgcn_cvt_pk_f32_fp8(*reinterpret_cast<const uint16_t*>(lsa + 32 * c), false);
          const uint4 A0 = make_uint4(av.x & keep, av.y & keep, 0u, 0u);
          const uint4 A1 = make_uint4(0u, 0u, av.z & keep, av.w & keep);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float2_t sw =
                __builtin_amdgcn_cvt_pk_f32_fp8(*reinterpret_cast<const uint16_t*>(lsw[r] + 32 * c), false);
            const uint4 B = make_uint4(w[r][0], w[r][1], w[r][2], w[r][3]);
            const float4_t d0 = mfma_fp4(A0, B), d1 = mfma_fp4(A1, B);
            const float f0 = sw[0] * sa[0], f1 = sw[1] * sa[1];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[r][v] = __builtin_fmaf(d1[v], f1, __builtin_fmaf(d0[v], f0, acc[r][v]));
          }
        }
      }
    }
  }

  // finish: output row 4 r + wr = the sum over waves and the 16 lanes
  // 16 b + 4 wr + w (entry w) holding its windows and block groups
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds4);
#pragma unroll
  for (int r = 0; r < R; ++r) red[(wave * R + r) * 64 + lane] = acc[r][lane & 3];
  __syncthreads();
  constexpr int OUTS = 4 * R;
  constexpr int NV = (OUTS + NW * 64 - 1) / (NW * 64);
  const float tsc = token_scale(p, 0);
  float out[NV];
  int tok[NV], rowt[NV];
  bool ok[NV], own[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int o = (int)threadIdx.x + u * NW * 64;
    out[u] = 0.0f;
    tok[u] = 0;
    rowt[u] = 0;
    ok[u] = own[u] = false;
    if (o < OUTS) {
      const int r = o >> 2, wr = o & 3;
      float sum = 0.0f;
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) sum += red[(w * R + r) * 64 + 16 * b + 4 * wr + ww];
      out[u] = sum * tsc;
      rowt[u] = o;
      own[u] = true;
      ok[u] = o < rows;
      if (ok[u]) p.y[tile0 + o] = out[u];
    }
  }
  if constexpr (EPI) lmhead_partials<1, 4 * R, NV>(p, out, tok, rowt, own, ok, blockIdx.x);
}

__global__ void reset_state_init_kernel(char* state, int M, int window, size_t sbytes) {
  const int m = blockIdx.x;
  if (m >= M) return;
  ResetState* st = reinterpret_cast<ResetState*>(state + (size_t)m * sbytes);
  float* ring = reinterpret_cast<float*>(st + 1);
  for (int i = threadIdx.x; i < window; i += blockDim.x) ring[i] = 0.0f;
  if (threadIdx.x == 0) {
    st->sum_all = 0.0;
    st->step_sum = 0.0;
    st->count = 0;
    st->step_len = 0;
    st->window = window;
  }
}

// ----------------------------------------------------------------------------
// Tiled MFMA GEMM for 17..128 tokens
// ----------------------------------------------------------------------------
// At 17..128 tokens the projection is a small GEMM (the pages route large M
// to a dedicated GEMM, reading notes section 7.3): every decoded weight
// element now feeds up to 128 products, so the bound is the MFMA and decode
// work per byte as much as HBM.  A workgroup of 4 waves owns kGemmRows = 128
// weight rows and all MT (32, 64 or 128) token columns.  The K loop runs in
// stages of 256 elements: the stage's raw NVFP4 bytes (weight codes
// [128][128 B], weight block scales [128][16 B], activation codes [MT][128 B]
// and scales [MT][16 B]) are copied into one of two LDS buffers with
// direct-to-LDS loads while the waves compute on the other buffer.  Waves
// split each stage's K in two halves and the tile as a WR x WC grid (rows x
// token groups); each decodes its
// weight rows and tokens from LDS to exact f16 values (E2M1 x E4M3 has at
// most 6 significant bits) in registers and runs v_mfma_f32_16x16x32_f16 on
// 16-row x 16-token tiles, so the products are exact and only the f32
// accumulation rounds.
// K order inside a stage: a 128-element half-stage of a row is 64 bytes;
// lane (j, g) (j = lane % 16 the row or token of the 16-tile, g = lane / 16)
// reads the 16 bytes at 16 g with one LDS load and feeds word q of them to
// k-step q (q = 0..3).  Both operands use the same order, so each k-step
// sums 32 distinct elements and the four k-steps cover the half-stage.  The
// code rows are stored XOR-swizzled (16-byte window w of row r at slot
// 8 r + (w ^ (r & 7))) so that the 16 lanes reading one window of 16 rows
// spread over the LDS banks; the copy takes the permutation in its global
// offsets.  Rows past N and tokens past M are copied from outside the
// buffers (zeros) and never stored.
constexpr int kGemmRows = 128;        // weight rows per workgroup
constexpr int kGemmStageK = 256;      // K elements per stage
constexpr int kGemmThreads = 256;     // 4 waves

__host__ __device__ constexpr int gemm_stage_bytes(int mt) {
  // weight codes, weight scales, activation codes, activation scales (each
  // region a whole number of 1 KB copy instructions)
  return kGemmRows * 128 + 2048 + (mt * 128 < 1024 ? 1024 : mt * 128) + (mt * 16 < 1024 ? 1024 : mt * 16);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_le<N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// The copies of one stage: kGemmCopies(MT) 1 KB direct-to-LDS loads (weight
// codes, weight scales, activation codes, activation scales), dealt to the 4
// waves round robin.  A copy's per-lane source offset and LDS offset do not
// depend on the stage (the stage is the scalar offset), so each wave works
// them out once, before the K loop.
template <int MT>
struct GemmCopies {
  static constexpr int WC = kGemmRows * 128 / 1024;  // weight-code copies (16)
  static constexpr int WS = 2;                       // weight scales: 128 rows x 16 B
  static constexpr int AC = MT * 128 < 1024 ? 1 : MT * 128 / 1024;
  static constexpr int AS = MT * 16 < 1024 ? 1 : MT * 16 / 1024;
  static constexpr int TOTAL = WC + WS + AC + AS;
  static constexpr int PER_WAVE = (TOTAL + kGemmThreads / 64 - 1) / (kGemmThreads / 64);
};

template <int MT>
struct GemmCopyPlan {
  int voff[GemmCopies<MT>::PER_WAVE];  // per-lane source offset (kOffOut: outside the buffer)
  int n;                               // copies this wave issues per stage (wave-uniform)
};

template <int MT>
__device__ __forceinline__ GemmCopyPlan<MT> gemm_copy_plan(int64_t K, int rows, int M, int wave, int lane) {
  using C = GemmCopies<MT>;
  const int kh = (int)(K / 2), ks = (int)(K / 16);
  GemmCopyPlan<MT> pl;
  pl.n = 0;
#pragma unroll
  for (int i = 0; i < C::PER_WAVE; ++i) {
    const int ch = wave + 4 * i;
    int v = (int)kOffOut;
    if (ch < C::WC) {
      const int s = 64 * ch + lane, r = s >> 3, w = (s & 7) ^ (r & 7);
      if (r < rows) v = r * kh + 16 * w;
    } else if (ch < C::WC + C::WS) {
      const int r = 64 * (ch - C::WC) + lane;
      if (r < rows) v = r * ks;
    } else if (ch < C::WC + C::WS + C::AC) {
      const int s = 64 * (ch - C::WC - C::WS) + lane, t = s >> 3, w = (s & 7) ^ (t & 7);
      if (t < M && t < MT) v = t * kh + 16 * w;
    } else if (ch < C::TOTAL) {
      const int t = 64 * (ch - C::WC - C::WS - C::AC) + lane;
      if (t < M && t < MT) v = t * ks;
    }
    pl.voff[i] = v;
    if (ch < C::TOTAL) ++pl.n;
  }
  return pl;
}

// Issue this wave's copies of stage `st` into the stage buffer at LDS `dst`.
// The copy regions are contiguous in the order weight codes, weight scales,
// activation codes, activation scales, so copy ch lands at dst + 1 KB * ch.
template <int MT>
__device__ __forceinline__ void gemm_stage_copy(const GemmCopyPlan<MT>& pl, const i32x4_t& wcr, const i32x4_t& wsr,
                                                const i32x4_t& acr, const i32x4_t& asr, uint32_t dst, int st,
                                                int wave) {
  using C = GemmCopies<MT>;
#pragma unroll
  for (int i = 0; i < C::PER_WAVE; ++i) {
    const int ch = wave + 4 * i;  // wave-uniform
    if (ch < C::WC)
      dma_b128(wcr, dst + 1024 * ch, pl.voff[i], st * 128);
    else if (ch < C::WC + C::WS)
      dma_b128(wsr, dst + 1024 * ch, pl.voff[i], st * 16);
    else if (ch < C::WC + C::WS + C::AC)
      dma_b128(acr, dst + 1024 * ch, pl.voff[i], st * 128);
    else if (ch < C::TOTAL)
      dma_b128(asr, dst + 1024 * ch, pl.voff[i], st * 16);
  }
}

// 32 codes of row (or token) r, window w, of a stage's swizzled code region,
// with the two block scales of its 16-element halves, decoded to four f16
// operands (one per k-step)
__device__ __forceinline__ void gemm_load_decode(const char* codes, const char* scales, int r, int seg, int g,
                                                 half8_t (&out)[4]) {
  const int w = 4 * seg + g;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(codes + 16 * (8 * r + (w ^ (r & 7))));
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(scales + 16 * r + 8 * seg + 2 * g);
  decode32_scaled(v, s2, out);
}

template <int MT>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemvParams p) {
  // wave grid: KH halves of each stage's K x WR row groups x WC token groups.
  // The two 128-element halves of a stage go to different waves (KH = 2),
  // each over 64 rows and all MT tokens (MT = 32, 64) or all 128 rows and 64
  // tokens (MT = 128): a wave decodes (rows + tokens) x 128 elements of a
  // stage for rows x tokens x 128 products, fewer decodes per product than
  // 4 row groups over the whole stage, at the price of adding the two
  // halves' accumulators at the end
  constexpr int KH = 2;
  constexpr int WR = MT >= 128 ? 1 : 2;
  constexpr int WC = 4 / WR / KH;
  constexpr int RT = kGemmRows / WR / 16;  // 16-row tiles per wave
  constexpr int CT = MT / WC / 16;         // 16-token tiles per wave
  constexpr int STAGE = gemm_stage_bytes(MT);
  static_assert(KH * WR * WC == kGemmThreads / 64, "one wave per (K half, row group, token group)");
  extern __shared__ uint4 lds4[];
  char* lds = reinterpret_cast<char*>(lds4);
  const uint32_t l0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(lds);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int kh = wave % KH, wr = (wave / KH) % WR, wc = wave / KH / WR;
  const int64_t N = p.N, K = p.K;
  const int M = p.M;
  // workgroup b: row tile b % ntiles, K split b / ntiles (stages st0 .. st1 - 1)
  const int ntiles = (int)((N + kGemmRows - 1) / kGemmRows);
  const int tile = (int)blockIdx.x % ntiles, ks = (int)blockIdx.x / ntiles;
  const int64_t tile0 = (int64_t)tile * kGemmRows;
  const int rows = N - tile0 < kGemmRows ? (int)(N - tile0) : kGemmRows;
  const i32x4_t wcr = raw_rsrc(p.w_codes + tile0 * (K / 2), (int64_t)rows * (K / 2));
  const i32x4_t wsr = raw_rsrc(p.w_scales + tile0 * (K / 16), (int64_t)rows * (K / 16));
  const i32x4_t acr = raw_rsrc(p.a_codes, (int64_t)M * (K / 2));
  const i32x4_t asr = raw_rsrc(p.a_scales, (int64_t)M * (K / 16));
  const int nst_all = (int)(K / kGemmStageK);
  const int st0 = (int)((int64_t)nst_all * ks / p.ksplit), st1 = (int)((int64_t)nst_all * (ks + 1) / p.ksplit);

  float4_t acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const GemmCopyPlan<MT> plan = gemm_copy_plan<MT>(K, rows, M, wave, lane);
  if (st0 < st1) gemm_stage_copy<MT>(plan, wcr, wsr, acr, asr, l0, st0, wave);  // (splits never exceed the stages)
  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    int ahead = 0;
    if (st + 1 < st1) {
      gemm_stage_copy<MT>(plan, wcr, wsr, acr, asr, l0 + (uint32_t)((buf ^ 1) * STAGE), st + 1, wave);
      ahead = plan.n;
    }
    wait_vmcnt_le<GemmCopies<MT>::PER_WAVE>(ahead);  // this wave's copies of stage st have landed
    __syncthreads();          // ... and every other wave's
    const char* wcodes = lds + buf * STAGE;
    const char* wscales = wcodes + kGemmRows * 128;
    const char* acodes = wscales + 2048;
    const char* ascales = acodes + (MT * 128 < 1024 ? 1024 : MT * 128);
#pragma unroll
    for (int sg = 0; sg < 2 / KH; ++sg) {
      const int seg = KH == 2 ? kh : sg;  // the stage's 128-element half
      half8_t a[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) gemm_load_decode(acodes, ascales, wc * (MT / WC) + 16 * ct + j, seg, g, a[ct]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        half8_t w[4];
        gemm_load_decode(wcodes, wscales, wr * (kGemmRows / WR) + 16 * rt + j, seg, g, w);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[q], a[ct][q], acc[rt][ct], 0, 0, 0);
      }
    }
    __syncthreads();  // the buffer is refilled two stages on
  }
  if constexpr (KH == 2) {
    // the second half's accumulators through LDS (the stage buffers are
    // free: the loop ended on a barrier); the first half's waves add them
    // and finish
    float4_t* red = reinterpret_cast<float4_t*>(lds);
    static_assert(WR * WC * RT * CT * 64 * 16 <= 2 * STAGE, "the exchange fits the stage buffers");
    const int wg = wr * WC + wc;  // the wave's (row group, token group)
    if (kh == 1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) red[((wg * RT + rt) * CT + ct) * 64 + lane] = acc[rt][ct];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[rt][ct] += red[((wg * RT + rt) * CT + ct) * 64 + lane];
  }
  // lane (j, g) holds D[4 g + i][j]: weight rows 4 g .. 4 g + 3 of the tile
  // for token j of the token tile
  if (p.ksplit > 1) {  // unscaled partial sums; the reduction launch adds the splits in order
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int t = wc * (MT / WC) + 16 * ct + j;
      if (t >= M) continue;
      float* part = p.partials + ((int64_t)(ks * ntiles + tile) * M + t) * kGemmRows;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        *reinterpret_cast<float4_t*>(part + wr * (kGemmRows / WR) + 16 * rt + 4 * g) = acc[rt][ct];
    }
    return;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int t = wc * (MT / WC) + 16 * ct + j;
    if (t >= M) continue;
    const float ts = token_scale(p, t);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = wr * (kGemmRows / WR) + 16 * rt + 4 * g;
      float* y = p.y + (int64_t)t * N + tile0 + r;
      if (r + 3 < rows && (N & 3) == 0) {
        *reinterpret_cast<float4_t*>(y) = acc[rt][ct] * ts;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r + i < rows) y[i] = acc[rt][ct][i] * ts;
      }
    }
  }
}

// Second launch of a split-K GEMM: y[t][n] = (sum over the splits, in split
// order, of the partial sums) * the global scales; one thread per output.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemvParams p) {
  const int64_t N = p.N;
  const int M = p.M;
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= (int64_t)M * N) return;
  const int t = (int)(o / N);
  const int64_t n = o - (int64_t)t * N;
  const int ntiles = (int)((N + kGemmRows - 1) / kGemmRows);
  const int tile = (int)(n / kGemmRows), r = (int)(n - (int64_t)tile * kGemmRows);
  float sum = 0.0f;
  for (int ks = 0; ks < p.ksplit; ++ks) sum += p.partials[((int64_t)(ks * ntiles + tile) * M + t) * kGemmRows + r];
  p.y[o] = sum * token_scale(p, t);
}

// ----------------------------------------------------------------------------
// Variant table
// ----------------------------------------------------------------------------

enum Kind {
  VALU = 0, DIRECT = 1, MFMA = 2, LMFMA = 3, DMA = 4, STAGED = 5, FMMA = 6, FMMASA = 7, DMASA = 8, STREAM = 9,
  FSTREAM = 10, GEMM = 11, WSTREAM = 12, WSTREAMAG = 13, STREAM8 = 14
};

struct Variant {
  const char* name;
  Kind kind;
  int mt, g, r, nw, p;
  void (*plain)(GemvParams);
  void (*epi)(GemvParams);
  void (*plain_k64)(GemvParams);  // register-staged MFMA kernel: K % 64 == 0 instantiations
  void (*epi_k64)(GemvParams);
};

#define VALU_V(MT, G, R, NW, P)                                                              \
  Variant {                                                                                \
    "valu_m" #MT "_g" #G "_r" #R "_w" #NW "_p" #P, VALU, MT, G, R, NW, P,                 \
        gemv_valu_kernel<MT, G, R, NW, P, false>, gemv_valu_kernel<MT, G, R, NW, P, true> \
  }
#define DIRECT_V(MT, G, R, NW, P)                                                                              \
  Variant {                                                                                                  \
    "direct_m" #MT "_g" #G "_r" #R "_w" #NW "_p" #P, DIRECT, MT, G, R, NW, P,                               \
        gemv_direct_kernel<MT, G, R, NW, P, false, false>, gemv_direct_kernel<MT, G, R, NW, P, false, true> \
  }
#define DIRECT_NT_V(MT, G, R, NW, P)                                                                         \
  Variant {                                                                                                \
    "direct_m" #MT "_g" #G "_r" #R "_w" #NW "_p" #P "_nt", DIRECT, MT, G, R, NW, P,                       \
        gemv_direct_kernel<MT, G, R, NW, P, true, false>, gemv_direct_kernel<MT, G, R, NW, P, true, true> \
  }
#define MFMA_V(MT, R, NW, P)                                                            \
  Variant {                                                                           \
    "mfma_m" #MT "_r" #R "_w" #NW "_p" #P, MFMA, MT, 16, R, NW, P,                   \
        gemv_mfma_kernel<MT, R, NW, P, false>, gemv_mfma_kernel<MT, R, NW, P, true>  \
  }

#define LMFMA_V(MT, R, NW, P)                                                                        \
  Variant {                                                                                        \
    "lmfma_m" #MT "_r" #R "_w" #NW "_p" #P, LMFMA, MT, 16, R, NW, P,                               \
        gemv_lmfma_kernel<MT, R, NW, P, false, false>, gemv_lmfma_kernel<MT, R, NW, P, false, true>, \
        gemv_lmfma_kernel<MT, R, NW, P, true, false>, gemv_lmfma_kernel<MT, R, NW, P, true, true>    \
  }
#define STAGED_V(MT, G, R, NW, P)                                                                  \
  Variant {                                                                                      \
    "staged_m" #MT "_g" #G "_r" #R "_w" #NW "_p" #P, STAGED, MT, G, R, NW, P,                   \
        gemv_staged_kernel<MT, G, R, NW, P, false>, gemv_staged_kernel<MT, G, R, NW, P, true> \
  }
#define FMMA_V(MT, R, NW, D)                                                                         \
  Variant {                                                                                        \
    "fmma_m" #MT "_r" #R "_w" #NW "_d" #D, FMMA, MT, 16, R, NW, D,                                 \
        gemv_fmma_kernel<MT, R, NW, D, false, false>, gemv_fmma_kernel<MT, R, NW, D, false, true> \
  }
#define FMMA_SA_V(MT, R, NW, D)                                                                    \
  Variant {                                                                                      \
    "fmma_m" #MT "_r" #R "_w" #NW "_d" #D "_sa", FMMASA, MT, 16, R, NW, D,                       \
        gemv_fmma_kernel<MT, R, NW, D, true, false>, gemv_fmma_kernel<MT, R, NW, D, true, true> \
  }
#define DMA_V(MT, R, NW, D)                                                                        \
  Variant {                                                                                      \
    "dma_m" #MT "_r" #R "_w" #NW "_d" #D, DMA, MT, 16, R, NW, D,                                 \
        gemv_dma_kernel<MT, R, NW, D, false, false>, gemv_dma_kernel<MT, R, NW, D, false, true> \
  }
#define DMA_SA_V(MT, R, NW, D)                                                                   \
  Variant {                                                                                    \
    "dma_m" #MT "_r" #R "_w" #NW "_d" #D "_sa", DMASA, MT, 16, R, NW, D,                       \
        gemv_dma_kernel<MT, R, NW, D, true, false>, gemv_dma_kernel<MT, R, NW, D, true, true> \
  }

#define STREAM_V(MT, R, NW, U)                                                              \
  Variant {                                                                               \
    "stream_m" #MT "_r" #R "_w" #NW "_u" #U, STREAM, MT, 16, R, NW, U,                       \
        gemv_stream_kernel<MT, R, NW, U, false>, gemv_stream_kernel<MT, R, NW, U, true>     \
  }
#define STREAM8_V(R, NW, U)                                                               \
  Variant {                                                                             \
    "stream8_m8_r" #R "_w" #NW "_u" #U, STREAM8, 8, 16, R, NW, U,                            \
        gemv_stream8_kernel<R, NW, U, false>, gemv_stream8_kernel<R, NW, U, true>           \
  }
#define STREAM16_V(R, NW, U)                                                                 \
  Variant {                                                                                \
    "stream8_m16_r" #R "_w" #NW "_u" #U, STREAM8, 16, 16, R, NW, U,                             \
        gemv_stream8_kernel<R, NW, U, false, 2>, gemv_stream8_kernel<R, NW, U, true, 2>        \
  }
#define FSTREAM_V(R, NW, U)                                                                 \
  Variant {                                                                               \
    "fstream_m1_r" #R "_w" #NW "_u" #U, FSTREAM, 1, 16, R, NW, U,                            \
        gemv_fstream_kernel<R, NW, U, false>, gemv_fstream_kernel<R, NW, U, true>           \
  }

// the wave-owned streaming kernel has no LM-head form either (its epilogue
// slot repeats the plain kernel and is never chosen)
#define WSTREAM_V(MT, R, NW, U)                                                                      \
  Variant {                                                                                        \
    "wstream_m" #MT "_r" #R "_w" #NW "_u" #U, WSTREAM, MT, 16, R, NW, U,                               \
        gemv_wstream_kernel<MT, R, NW, U>, gemv_wstream_kernel<MT, R, NW, U>                        \
  }

// the tiled GEMM has no LM-head form: its epilogue slot repeats the plain
// kernel and is never chosen (fits() refuses GEMM with the epilogue)
#define WSTREAM_AG_V(MT, R, NW, U)                                                                     \
  Variant {                                                                                          \
    "wstream_m" #MT "_r" #R "_w" #NW "_u" #U "_ag", WSTREAMAG, MT, 16, R, NW, U,                      \
        gemv_wstream_kernel<MT, R, NW, U, true>, gemv_wstream_kernel<MT, R, NW, U, true>              \
  }

#define GEMM_V(MT)                                                                    \
  Variant {                                                                         \
    "gemm_m" #MT, GEMM, MT, 16, kGemmRows / 16, kGemmThreads / 64, 0, gemm_kernel<MT>, gemm_kernel<MT> \
  }

// The launch table's variants and the fallbacks it uses where a choice does
// not fit a shape (LDS size, K granularity, 32-bit buffer offsets).  Further
// instantiations for sweeps can be compiled in by defining
// NVFP4_GEMV_EXTRA_VARIANTS as a list of the *_V initialisers above.
const Variant kVariants[] = {
    // one token
    DIRECT_NT_V(1, 64, 1, 4, 1), DIRECT_NT_V(1, 32, 1, 4, 1), DIRECT_NT_V(1, 32, 2, 4, 1), STAGED_V(1, 32, 2, 4, 1),
    // two tokens
    FMMA_SA_V(2, 1, 4, 3), STAGED_V(2, 64, 1, 4, 2), STAGED_V(2, 64, 1, 4, 1), STAGED_V(2, 32, 2, 4, 1),
    // 3..8 tokens
    STREAM_V(4, 5, 4, 2), DMA_V(4, 2, 4, 3), DMA_V(8, 2, 4, 3),
    FMMA_V(4, 2, 4, 3), LMFMA_V(8, 2, 8, 1), LMFMA_V(8, 1, 4, 1),
    // 9..128 tokens
    LMFMA_V(16, 2, 8, 1), LMFMA_V(16, 2, 4, 1), LMFMA_V(32, 2, 8, 1), LMFMA_V(32, 2, 4, 1), LMFMA_V(64, 2, 8, 1),
    LMFMA_V(64, 2, 4, 1), LMFMA_V(128, 2, 4, 1), GEMM_V(32), GEMM_V(64), GEMM_V(128), WSTREAM_V(4, 3, 4, 2),
    WSTREAM_AG_V(4, 3, 4, 2), STREAM8_V(2, 4, 2), STREAM8_V(3, 4, 2), STREAM8_V(4, 4, 2), STREAM8_V(5, 4, 2),
    STREAM8_V(2, 8, 2), STREAM8_V(3, 8, 2), STREAM16_V(4, 4, 2), STREAM16_V(5, 4, 2),
    // fallbacks
    DIRECT_V(2, 64, 1, 4, 1), MFMA_V(4, 2, 8, 1), MFMA_V(8, 2, 8, 1), LMFMA_V(16, 1, 4, 1), LMFMA_V(32, 1, 4, 1),
    LMFMA_V(64, 1, 4, 1), LMFMA_V(128, 1, 4, 1),
#ifdef NVFP4_GEMV_EXTRA_VARIANTS
    NVFP4_GEMV_EXTRA_VARIANTS
#endif
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int mt_of(int M) {
  return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
}

int find_variant(const char* name) {
  for (int i = 0; i < kNumVariants; ++i)
    if (strcmp(kVariants[i].name, name) == 0) return i;
  return -1;
}

// Tuning override (nvfp4_gemv_tune): a forced variant index (-1 = none) and
// the row mapping of the MFMA tile kernels (1 = rows dealt out evenly where
// whole tiles would leave CUs idle, 0 = whole tiles).  Process-wide.
std::atomic<int> g_forced_variant{-1};
std::atomic<int> g_balance{1};

// Rows per workgroup of the MFMA tile kernels.  A workgroup streams its rows
// at a rate set by the loads it keeps in flight, so a grid of N / (16 R)
// workgroups that leaves CUs idle (N = 5120: 160 or 320 tiles on 256 CUs)
// runs at the speed of the busiest CU.  When the tiles fill the CUs at most
// twice over, the rows are instead dealt out evenly: ceil(N / (256 k))
// rows per workgroup for the smallest k that fits a 16 R-row tile, so that
// every CU streams the same number of rows.  The tuning override
// (nvfp4_gemv_tune) can keep whole tiles instead, for timing comparisons.
constexpr int64_t kComputeUnits = 256;  // MI355X

int64_t tile_rows_for(int64_t N, int64_t tile) {
  if (g_balance.load(std::memory_order_relaxed) == 0) return tile;
  const int64_t k = (N + tile * kComputeUnits - 1) / (tile * kComputeUnits);
  if (k > 2) return tile;
  const int64_t rows = (N + kComputeUnits * k - 1) / (kComputeUnits * k);
  return rows < tile ? rows : tile;
}

constexpr int64_t kLdsBytes = 163840;  // LDS per workgroup (gfx950)

// Rows of the tile a kernel's LM-head partials cover (the ROWS of its
// lmhead_partials instantiation)
int64_t epi_tile_rows(const Variant& v) {
  switch (v.kind) {
    case STREAM:
    case FSTREAM: return 4 * v.r;
    case STREAM8: return 8 * v.r;
    case WSTREAM:
    case WSTREAMAG: return 4 * v.r * v.nw;
    case VALU:
    case DIRECT:
    case STAGED: return (int64_t)v.r * v.nw * (64 / v.g);
    default: return 16 * v.r;
  }
}

// LDS a streaming kernel stages: the tile's block scales (the f16 form), and
// the activation codes and scales of its one token beside them (the FP4 form)
int64_t stream_kernel_lds(const Variant& v, int64_t K, int64_t tile_rows) {
  if (v.kind == STREAM || v.kind == STREAM8) return pad1k(tile_rows * (K / 16));
  return stream_lds_bytes(1, K, tile_rows);
}

// LDS of the direct-to-LDS kernels with staged activation (f16 and FP4
// MFMA): activation codes and scales for MT tokens, the tile's weight scales,
// then a ring of D weight-code slots per wave
int64_t sa_lds_bytes(const Variant& v, int64_t K) {
  return pad1k(v.mt * (K / 2)) + pad1k(v.mt * (K / 16)) + pad1k(16 * v.r * (K / 16)) + (int64_t)v.nw * v.p * 2048 * v.r;
}

// Index of a variant named by a string literal, looked up once per call site.
#define VARIANT(name) ([] {                   \
  static const int index_ = find_variant(name); \
  return index_;                                \
}())

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// K splits of the tiled GEMM: enough workgroups (tiles x splits, about 400)
// to fill the CUs when the row tiles alone do not, each split at least 4
// stages long, and only while the partial sums fit the caller's workspace.
int64_t gemm_split_ws_bytes(int M, int64_t N, int ksplit) {
  const int64_t tiles = (N + kGemmRows - 1) / kGemmRows;
  return align256((int64_t)ksplit * tiles * M * kGemmRows * 4);
}

int gemm_ksplit(int M, int64_t N, int64_t K, int64_t ws_cap) {
  const int64_t tiles = (N + kGemmRows - 1) / kGemmRows;
  const int64_t nst = K / kGemmStageK;
  int64_t s = (400 + tiles / 2) / tiles;
  if (s > nst / 4) s = nst / 4;
  if (s < 1) s = 1;
  while (s > 1 && gemm_split_ws_bytes(M, N, (int)s) > ws_cap) --s;
  return (int)s;
}

// Default variant per (M, N, K): the fastest variant of MI355X sweeps over
// the Qwen3-32B projection and LM-head shapes (graph-replayed back-to-back
// launches, each projection's weights rotated over >= 576 MB of copies so
// that every launch reads HBM; candidates interleaved, medians compared),
// generalised by N and K, with the MFMA kernels' rows dealt out evenly over
// the CUs where whole tiles would leave some idle (tile_rows_for).  The
// LDS-copy kernels need K % 256 == 0; other K use the register-staged
// kernels.
// The number R of 8-row groups per workgroup tile of the eight-token
// streaming kernel for N rows:
//   N >= 65536 (LM heads): R = 4.
//   16384 <= N < 65536: the smallest R in {3, 4, 5} whose workgroups take
//     the fewest rows per CU when dealt out over the CUs (rounds x R).
//   N < 16384: the fewest groups that hold the rows a workgroup gets when
//     40-row tiles are balanced over the CUs (tile_rows_for), 2 to 5.
int stream8_groups(int64_t N) {
  int r = 5;
  if (N >= 65536) {
    r = 4;
  } else if (N >= 16384) {
    int64_t best = -1;
    for (int c = 3; c <= 5; ++c) {
      const int64_t wgs = (N + 8 * c - 1) / (8 * c);
      const int64_t cost = (wgs + kComputeUnits - 1) / kComputeUnits * c;
      if (best < 0 || cost < best) {
        best = cost;
        r = c;
      }
    }
  } else {
    const int64_t groups = (tile_rows_for(N, 40) + 7) / 8;
    r = groups < 2 ? 2 : groups > 5 ? 5 : (int)groups;
  }
  return r;
}

// The eight-token streaming variant for N x K: R from stream8_groups, and 8
// waves instead of 4 on long rows (K >= 8192) of tiles of at most 24 rows.
int stream8_variant(int64_t N, int64_t K) {
  const int r = stream8_groups(N);
  if (N < 16384 && K >= 8192 && r <= 3) return r == 2 ? VARIANT("stream8_m8_r2_w8_u2") : VARIANT("stream8_m8_r3_w8_u2");
  return r == 2 ? VARIANT("stream8_m8_r2_w4_u2")
         : r == 3 ? VARIANT("stream8_m8_r3_w4_u2")
         : r == 4 ? VARIANT("stream8_m8_r4_w4_u2")
                  : VARIANT("stream8_m8_r5_w4_u2");
}

int default_variant(int M, int64_t N, int64_t K, bool epi, int64_t ws_cap) {
  const bool k256 = K % 256 == 0;
  // the FP4 MFMA kernel with the activation in LDS, when that fits
  auto fmma_sa = [&](int i, int otherwise) {
    return sa_lds_bytes(kVariants[i], K) + (epi ? 4 * kVariants[i].mt * epi_tile_rows(kVariants[i]) : 0) <= kLdsBytes
               ? i
               : otherwise;
  };
  // 17..128 tokens on many rows (gate_up, N >= 16384): the tiled GEMM, whose
  // 128-row workgroups then still fill the CUs (its LM-head form does not
  // exist; the epilogue keeps the GEMV kernels)
  if (M > 16 && !epi && N >= 16384 && K % kGemmStageK == 0)
    return M > 64 ? VARIANT("gemm_m128") : M > 32 ? VARIANT("gemm_m64") : VARIANT("gemm_m32");
  // 65..128 tokens on long rows of few output rows (down_proj, K >= 16384):
  // the tiled GEMM split along K, when the caller's workspace holds the
  // partial sums of the full split (fewer splits leave CUs idle)
  if (M > 64 && !epi && K >= 16384 && K % kGemmStageK == 0) {
    const int s = gemm_ksplit(M, N, K, kNoWsCap);
    if (s == 1 || gemm_split_ws_bytes(M, N, s) <= ws_cap) return VARIANT("gemm_m128");
  }
  // 65..128 tokens: eight 16-token column tiles; 33..64: four; 17..32: two;
  // 9..16: all 16 token columns of one tile (the register-staged MFMA kernel)
  if (M > 64) return VARIANT("lmfma_m128_r2_w4_p1");
  if (M > 32) return K >= 16384 ? VARIANT("lmfma_m64_r2_w8_p1") : VARIANT("lmfma_m64_r2_w4_p1");
  if (M > 16) return K >= 8192 ? VARIANT("lmfma_m32_r2_w8_p1") : VARIANT("lmfma_m32_r2_w4_p1");
  // 9..16 tokens: the streaming kernel with two sets of 8 tokens where its
  // row groups come out at R >= 4 (qkv-like and many-row shapes: 7-13%
  // faster there; with fewer rows per workgroup the register-staged kernel
  // is as fast or faster)
  if (M > 8 && K % kStream8Chunk == 0 && stream8_groups(N) >= 4) {
    const int i = stream8_groups(N) == 4 ? VARIANT("stream8_m16_r4_w4_u2") : VARIANT("stream8_m16_r5_w4_u2");
    const Variant& v = kVariants[i];
    if (stream_kernel_lds(v, K, tile_rows_for(N, 8 * v.r)) + (epi ? 4 * v.mt * epi_tile_rows(v) : 0) <= kLdsBytes)
      return i;
  }
  if (M > 8) return K >= 8192 ? VARIANT("lmfma_m16_r2_w8_p1") : VARIANT("lmfma_m16_r2_w4_p1");
  // The eight-token streaming kernel, when its staged block scales fit: at
  // 5..8 tokens on every shape, at 2..4 tokens except where another kernel
  // measured as fast or faster (o-like rows, 8192 <= K < 16384, on
  // N < 16384 whose workgroups leave some of the kernel's 8-row groups
  // empty: the four-window form; LM-head-sized N >= 65536 without the
  // epilogue: the wave-owned form), and at 1 token on few rows (N < 8192)
  // that fill its row groups (elsewhere the VALU kernels are faster)
  const bool gaps = N < 16384 && 8 * stream8_groups(N) > tile_rows_for(N, 40);
  const bool oLike = K >= 8192 && K < 16384 && gaps;
  if (K % kStream8Chunk == 0 &&
      (M >= 5 || (M >= 2 && !oLike && !(N >= 65536 && !epi)) || (M == 1 && N < 8192 && !gaps))) {
    const int i = stream8_variant(N, K);
    const Variant& v = kVariants[i];
    if (stream_kernel_lds(v, K, tile_rows_for(N, 8 * v.r)) + (epi ? 4 * v.mt * epi_tile_rows(v) : 0) <= kLdsBytes)
      return i;
  }
  // 2..4 tokens on long rows of few output rows (o_proj; down_proj where
  // the eight-token kernel does not fit): the four-window streaming kernel
  if (M >= 2 && M <= 4 && N < 16384 && K >= 8192 && K % kStreamChunk == 0) {
    const int i = VARIANT("stream_m4_r5_w4_u2");
    const Variant& v = kVariants[i];
    if (stream_kernel_lds(v, K, tile_rows_for(N, 4 * v.r)) + (epi ? 4 * v.mt * epi_tile_rows(v) : 0) <= kLdsBytes)
      return i;
  }
  // 2..4 tokens on qkv-like shapes (8192 <= N < 16384, K < 8192) and 2
  // tokens on many-row shapes (N >= 16384, K < 8192), where the eight-token
  // kernel is not taken: the wave-owned streaming kernel with the
  // activation read from L2; 3..4 tokens on many-row shapes: the same
  // kernel with the activation staged in LDS (the two forms measured within
  // 1% there)
  if (!epi && K % kStreamChunk == 0 && M >= 2 && M <= 4 && N >= 8192 && K < 8192 && (N < 16384 || M == 2)) {
    const int i = VARIANT("wstream_m4_r3_w4_u2_ag");
    if (pad1k(4 * kVariants[i].r * kVariants[i].nw * (K / 16)) <= kLdsBytes) return i;
  }
  if (!epi && K % kStreamChunk == 0 && M >= 3 && M <= 4 && N >= 16384) {
    const int i = VARIANT("wstream_m4_r3_w4_u2");
    if (stream_lds_bytes(4, K, 4 * kVariants[i].r * kVariants[i].nw) <= kLdsBytes) return i;
  }
  if (M <= 1) {
    // LM heads (N >= 65536, with or without the epilogue): the direct
    // kernel's 16-row tiles measured faster than the staged kernel's 8-row
    // ones (and leave a quarter of the epilogue's partials)
    if (N >= 65536) return VARIANT("direct_m1_g32_r2_w4_p1_nt");
    if (K >= 8192) return VARIANT("direct_m1_g64_r1_w4_p1_nt");
    if (N >= 16384) return k256 ? VARIANT("staged_m1_g32_r2_w4_p1") : VARIANT("direct_m1_g32_r2_w4_p1_nt");
    return VARIANT("direct_m1_g32_r1_w4_p1_nt");
  }
  // 2 tokens on small shapes (N, K < 8192: the 4096 x 4096 and Qwen3-8B
  // qkv / o): the register-staged MFMA kernel beats the staged VALU one
  if (M == 2 && N < 8192 && K < 8192) return VARIANT("lmfma_m8_r1_w4_p1");
  if (M <= 2 && k256)
    return K >= 12288 ? fmma_sa(VARIANT("fmma_m2_r1_w4_d3_sa"), VARIANT("staged_m2_g64_r1_w4_p2"))
           : K >= 8192 && N < 16384 ? VARIANT("staged_m2_g64_r1_w4_p1")
                                    : VARIANT("staged_m2_g32_r2_w4_p1");
  // N >= 16384: the direct-to-LDS ring (at M = 5..8 only where the
  // eight-token streaming kernel's block scales do not fit)
  if (k256 && N >= 16384) return M <= 4 ? VARIANT("dma_m4_r2_w4_d3") : VARIANT("dma_m8_r2_w4_d3");
  if (M <= 4 && k256 && K >= 12288) return VARIANT("fmma_m4_r2_w4_d3");
  if (K >= 8192) return VARIANT("lmfma_m8_r2_w8_p1");
  return VARIANT("lmfma_m8_r1_w4_p1");
}


// LDS of the staged kernel: activation codes and scales for MT tokens and
// the block scales of the workgroup's rows, each padded to whole KB
int64_t staged_lds_bytes(const Variant& v, int64_t K) {
  const int64_t rows = (int64_t)v.r * v.nw * (64 / v.g);
  return pad1k(v.mt * (K / 2)) + pad1k(v.mt * (K / 16)) + pad1k(rows * (K / 16));
}

}  // namespace

size_t reset_state_bytes(int window) {
  const size_t b = sizeof(ResetState) + sizeof(float) * (size_t)window;
  return (b + 15) & ~(size_t)15;
}

GemvConfig choose_gemv_config(int M, int64_t N, int64_t K, bool epi, int64_t ws_cap) {
  int vi = -1;
  // the LDS-staged kernel addresses a row tile and the activation with
  // 32-bit buffer offsets
  auto fits = [&](int i) {
    const Variant& v = kVariants[i];
    const Kind kd = v.kind;
    if ((kd == DMA || kd == DMASA || kd == STAGED || kd == FMMA || kd == FMMASA) && K % 256 != 0) return false;
    if ((kd == STREAM || kd == FSTREAM) && K % kStreamChunk != 0) return false;
    if (kd == STREAM8 && K % kStream8Chunk != 0) return false;
    if (kd == GEMM && (K % kGemmStageK != 0 || epi)) return false;
    if (kd == WSTREAM && (K % kStreamChunk != 0 || epi ||
                          stream_lds_bytes(v.mt, K, 4 * v.r * v.nw) > kLdsBytes))
      return false;
    if (kd == WSTREAMAG && (K % kStreamChunk != 0 || epi || pad1k(4 * v.r * v.nw * (K / 16)) > kLdsBytes))
      return false;
    // the LM-head instantiations also hold the static softmax slots
    // [MT][tile rows] of their partials
    const int64_t slot = epi ? (int64_t)4 * v.mt * epi_tile_rows(v) : 0;
    if ((kd == FMMASA || kd == DMASA) && sa_lds_bytes(v, K) + slot > kLdsBytes) return false;
    if ((kd == STREAM || kd == FSTREAM) && stream_kernel_lds(v, K, tile_rows_for(N, 4 * v.r)) + slot > kLdsBytes)
      return false;
    if (kd == STREAM8 && stream_kernel_lds(v, K, tile_rows_for(N, 8 * v.r)) + slot > kLdsBytes) return false;
    if (kd == STAGED && staged_lds_bytes(v, K) > 65536) return false;
    return (kd != LMFMA && kd != DMA && kd != DMASA && kd != FMMA && kd != FMMASA && kd != STREAM && kd != STREAM8 && kd != FSTREAM &&
            kd != GEMM && kd != WSTREAM && kd != WSTREAMAG) ||
           (int64_t)16 * v.r * (K / 2) < (1ll << 31);
  };
  // tuning override, used when the forced variant's compiled token count
  // covers M and it fits the shape
  const int forced = g_forced_variant.load(std::memory_order_relaxed);
  if (forced >= 0 && forced < kNumVariants && kVariants[forced].mt >= M && fits(forced)) vi = forced;
  if (vi < 0) vi = default_variant(M, N, K, epi, ws_cap);
  if (!fits(vi))
    vi = mt_of(M) <= 2   ? VARIANT("direct_m2_g64_r1_w4_p1")
         : mt_of(M) <= 4 ? VARIANT("mfma_m4_r2_w8_p1")
         : mt_of(M) <= 8  ? VARIANT("mfma_m8_r2_w8_p1")
         : mt_of(M) <= 16 ? VARIANT("lmfma_m16_r1_w4_p1")
         : mt_of(M) <= 32 ? VARIANT("lmfma_m32_r1_w4_p1")
         : mt_of(M) <= 64 ? VARIANT("lmfma_m64_r1_w4_p1")
                          : VARIANT("lmfma_m128_r1_w4_p1");
  const Variant& v = kVariants[vi];
  GemvConfig c{};
  c.variant = vi;
  c.mt = v.mt;
  c.g = v.g;
  c.r = v.r;
  c.waves = v.nw;
  // f16 activation elements a workgroup may stage in LDS: 64 KiB, or 48 KiB
  // when the epilogue's reduction buffers share the LDS
  const int64_t budget = epi ? 24576 : 32768;
  c.ksplit = 1;
  if (v.kind == GEMM) {
    c.kp = (int)K;
    c.rows_per_wg = kGemmRows;
    const int64_t tiles = (N + kGemmRows - 1) / kGemmRows;
    c.ksplit = gemm_ksplit(M, N, K, ws_cap);
    c.grid = tiles * c.ksplit;
    c.lds_bytes = 2 * (int64_t)gemm_stage_bytes(v.mt);
  } else if (v.kind == WSTREAM || v.kind == WSTREAMAG) {
    c.kp = (int)K;
    c.rows_per_wg = 4 * v.r * v.nw;
    c.grid = (N + c.rows_per_wg - 1) / c.rows_per_wg;
    c.lds_bytes = v.kind == WSTREAM ? stream_lds_bytes(v.mt, K, c.rows_per_wg) : pad1k(c.rows_per_wg * (K / 16));
  } else if (v.kind == MFMA || v.kind == LMFMA || v.kind == DMA || v.kind == DMASA || v.kind == FMMA || v.kind == FMMASA ||
      v.kind == STREAM || v.kind == STREAM8 || v.kind == FSTREAM) {
    c.kp = (int)K;
    const int64_t tile =
        (int64_t)(v.kind == STREAM || v.kind == FSTREAM ? 4 : v.kind == STREAM8 ? 8 : 16) * v.r;  // rows of the kernel's tile
    c.rows_per_wg = v.kind == MFMA ? tile : tile_rows_for(N, tile);
    c.grid = (N + c.rows_per_wg - 1) / c.rows_per_wg;
    const int ct = v.mt > 16 ? v.mt / 16 : 1;              // 16-token column tiles
    c.lds_bytes = (int64_t)v.nw * v.r * ct * 4 * 64 * 4;  // partial tiles of the final reduction
    if (v.kind == LMFMA) {
      const int64_t slots = (int64_t)v.nw * (16 * v.r + (v.mt > 8 ? v.mt : 8)) * (144 + 20);
      if (slots > c.lds_bytes) c.lds_bytes = slots;
    }
    if (v.kind == FMMASA || v.kind == DMASA) {
      const int64_t b = sa_lds_bytes(v, K);
      if (b > c.lds_bytes) c.lds_bytes = b;
    }
    if (v.kind == FSTREAM || v.kind == STREAM || v.kind == STREAM8) {
      const int64_t b = stream_kernel_lds(v, K, c.rows_per_wg);
      if (b > c.lds_bytes) c.lds_bytes = b;
    }
    if (v.kind == DMA || v.kind == FMMA) {
      const int64_t ring = (int64_t)v.nw * v.p * ((2 * v.r + 1) * 1024 + (v.r + 1) * 256);
      if (ring > c.lds_bytes) c.lds_bytes = ring;
    }
  } else if (v.kind == VALU) {
    int64_t kp = budget / v.mt / 512 * 512;
    const int64_t kr = (K + 127) / 128 * 128;
    if (kp > kr) kp = kr;
    c.kp = (int)kp;
    c.rows_per_wg = (int64_t)v.r * v.nw * (64 / v.g);
    c.grid = (N + c.rows_per_wg - 1) / c.rows_per_wg;
    c.lds_bytes = (int64_t)v.mt * kp * 2;
  } else {
    c.kp = (int)K;
    c.rows_per_wg = (int64_t)v.r * v.nw * (64 / v.g);
    c.grid = (N + c.rows_per_wg - 1) / c.rows_per_wg;
    c.lds_bytes = v.kind == STAGED ? staged_lds_bytes(v, K) : 0;
  }
  // workspace: with the epilogue, the per-token tickets, per-workgroup
  // softmax partials, then the slice partials; for a split-K GEMM its
  // partial sums
  c.ws_bytes =
      epi ? align256(kEpiTicketBytes + merge_slices_offset(c.grid, c.mt) + (int64_t)c.mt * kMergeGroups * 16) : 0;
  if (c.ksplit > 1) c.ws_bytes = gemm_split_ws_bytes(M, N, c.ksplit);
  return c;
}

int set_gemv_tuning(const char* variant, int balance) {
  int vi = -1;
  if (variant && variant[0]) {
    vi = find_variant(variant);
    if (vi < 0) return -1;
  }
  g_forced_variant.store(vi, std::memory_order_relaxed);
  g_balance.store(balance, std::memory_order_relaxed);
  return 0;
}

const char* gemv_variant_name(int vi) { return vi >= 0 && vi < kNumVariants ? kVariants[vi].name : "?"; }
const char* gemv_variant_by_index(int i) { return i >= 0 && i < kNumVariants ? kVariants[i].name : nullptr; }

size_t gemv_workspace_bytes(int M, int64_t N, int64_t K, bool epi, int64_t ws_cap) {
  return (size_t)choose_gemv_config(M, N, K, epi, ws_cap).ws_bytes;
}

hipError_t launch_gemv(const GemvConfig& cfg, int M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_gscale, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* w_gscale, float* y,
                       const EpilogueArgs* epi, void* ws, bool per_token, hipStream_t stream) {
  if (cfg.variant < 0 || cfg.variant >= kNumVariants) return hipErrorInvalidConfiguration;
  GemvParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.kp = cfg.kp;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_gscale = a_gscale;
  p.a_gs_stride = per_token ? 1 : 0;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.w_gscale = w_gscale;
  p.y = y;
  p.tile_rows = (int)cfg.rows_per_wg;
  char* wsb = reinterpret_cast<char*>(ws);
  if (epi) {
    p.epi = *epi;
    p.tickets = reinterpret_cast<uint32_t*>(wsb);
    p.partials = reinterpret_cast<float*>(wsb + kEpiTicketBytes);
    p.state_bytes = reset_state_bytes(epi->window);
  }
  const Variant& v = kVariants[cfg.variant];
  void (*fn)(GemvParams) = epi ? v.epi : v.plain;
  if (v.plain_k64 && K % 64 == 0) fn = epi ? v.epi_k64 : v.plain_k64;
  p.ksplit = cfg.ksplit;
  if (cfg.ksplit > 1) p.partials = reinterpret_cast<float*>(wsb);
  hipLaunchKernelGGL(fn, dim3((unsigned)cfg.grid), dim3(v.nw * 64), (size_t)cfg.lds_bytes, stream, p);
  if (cfg.ksplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)(((int64_t)M * N + 255) / 256)), dim3(256), 0, stream, p);
  }
  if (epi) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_slice_kernel, dim3(M * kMergeGroups), dim3(kMergeThreads), 0, stream, p, cfg.mt,
                       (int)cfg.grid);
  }
  return hipGetLastError();
}

hipError_t launch_reset_state_init(void* state, int M, int window, hipStream_t stream) {
  hipLaunchKernelGGL(reset_state_init_kernel, dim3(M), dim3(256), 0, stream, reinterpret_cast<char*>(state), M,
                     window, reset_state_bytes(window));
  return hipGetLastError();
}

}  // namespace nvfp4
