// NVFP4 quantization kernels for gfx950: the per-layer activation "Q" step
// (ReSET reading notes, section 5.3) and the offline weight pack.
//
// Format (reading notes, sections 2.1 and 6.1): E2M1 elements, one E4M3
// scale per 16-element block, one FP32 global scale per tensor.  Recipe:
//   s_g = amax / 2688                      (2688 = 6 * 448)
//   t_b = amax_b / (6 * s_g)               (0 when s_g == 0)
//   s_b = E4M3 round-to-nearest-even of t_b, saturated at 448
//   e_b = E4M3(s_b) * s_g
//   q   = E2M1 round-to-nearest-even of |x| / e_b, saturated at 6 (0 when
//         e_b == 0), sign bit copied from x
// every step one IEEE float32 operation, so the result is bit-reproducible.
// This file is compiled with FP contraction off; float division is the
// correctly rounded sequence and float32 denormals are kept (IEEE mode).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Nearest E4M3 code of a finite t >= 0, ties to the even code, saturated at
// 448 (code 0x7E).  Below 2^-6 the grid is the subnormal one, step 2^-9;
// above, a grid of 8 steps per binade.  t * 2^k is exact, rintf rounds half
// to even, and the code of a grid point has the parity of its step count, so
// "ties to even step" is "ties to even code".
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);            // 0 .. 8
  const int e = (int)((__float_as_uint(t) >> 23) & 0xFFu) - 127;      // -6 .. 8
  const float to_steps = __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // 2^(3-e)
  const uint32_t q = (uint32_t)rintf(t * to_steps);                   // 8 .. 16
  return ((uint32_t)(e + 7) << 3) + (q - 8u);                          // 16 carries into e+1
}

// Value of a non-negative E4M3 code (<= 0x7E) as float32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;                          // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));              // 2^(e-7) * (1 + m/8)
}

// E2M1 magnitude code of a >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
// the even code, saturated at 6.  Each comparison is one grid midpoint; a
// midpoint that ties toward the upper (even) code uses >=, toward the lower
// (even) code uses >.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ float block_amax(const float (&x)[16]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  return amax;
}

// Quantize one 16-element block whose max |x| is `amax`.  Returns the
// block-scale code; writes the 16 codes packed two per byte (element 2j in
// the low nibble) into c0/c1.
__device__ __forceinline__ uint32_t quant_block(const float (&x)[16], float amax, float s_g, uint32_t& c0,
                                                uint32_t& c1) {
  float t = 0.0f;
  if (s_g != 0.0f) {
    const float denom = 6.0f * s_g;
    t = amax / denom;
  }
  const uint32_t sb = e4m3_code(t);
  const float e = e4m3_value(sb) * s_g;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = (e != 0.0f) ? fabsf(x[i]) / e : 0.0f;
    const uint32_t q = e2m1_mag_code(v) | ((__float_as_uint(x[i]) >> 31) << 3);
    if (i < 8) lo |= q << (4 * i);
    else hi |= q << (4 * (i - 8));
  }
  c0 = lo;
  c1 = hi;
  return sb;
}

template <typename T>
struct Loader;

template <>
struct Loader<uint16_t> {  // bf16 bit patterns
  static __device__ __forceinline__ void block(const uint16_t* p, float (&x)[16]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
  // max |x| over 8 consecutive elements
  static __device__ __forceinline__ float amax8(const uint16_t* p) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    // |bf16| as the top half of a float: clear the sign bits
    const uint32_t w[4] = {a.x & 0x7FFF7FFFu, a.y & 0x7FFF7FFFu, a.z & 0x7FFF7FFFu, a.w & 0x7FFF7FFFu};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(bf16_to_f32(w[i] & 0xFFFFu), bf16_to_f32(w[i] >> 16)));
    return m;
  }
};

template <>
struct Loader<float> {
  static __device__ __forceinline__ void block(const float* p, float (&x)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
  static __device__ __forceinline__ float amax8(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  }
};

// Max over a workgroup of NT threads; result valid in every thread.
template <int NT = kThreads>
__device__ __forceinline__ float wg_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// amax of elements [lo, hi) of x (hi - lo a multiple of 8), by this workgroup.
template <typename T>
__device__ __forceinline__ float wg_amax_range(const T* x, int64_t lo, int64_t hi, float* red) {
  float m = 0.0f;
  for (int64_t i = lo + (int64_t)threadIdx.x * 8; i < hi; i += (int64_t)kThreads * 8)
    m = fmaxf(m, Loader<T>::amax8(x + i));
  return wg_max(m, red);
}

// Pass 1 of the two-launch path: partials[b] = max |x| over chunk b.
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_partials_kernel(const T* __restrict__ x, int64_t n,
                                                                 float* __restrict__ partials) {
  __shared__ float red[kThreads / 64];
  const int64_t per = ((n / 8 + gridDim.x - 1) / gridDim.x) * 8;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  const float m = wg_amax_range(x, lo < n ? lo : n, hi, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Quantize rows x [rows][K]; one thread per 16-element block, grid-stride.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const T* __restrict__ x, int64_t rows, int64_t K, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, int mode,
    const float* __restrict__ partials, int n_parts) {
  __shared__ float red[kThreads / 64];
  float s_g;
  if (mode == GS_STATIC) {
    s_g = *gscale;
  } else {
    float amax;
    if (mode == GS_SELF) {
      amax = wg_amax_range(x, 0, rows * K, red);
    } else {
      float m = 0.0f;
      for (int i = threadIdx.x; i < n_parts; i += kThreads) m = fmaxf(m, partials[i]);
      amax = wg_max(m, red);
    }
    s_g = amax / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = s_g;
  }
  const int64_t bpr = K / 16;
  const int64_t nblocks = rows * bpr;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t row = b / bpr, j = b - row * bpr;
    float v[16];
    Loader<T>::block(x + row * K + j * 16, v);
    uint32_t c0, c1;
    const uint32_t sb = quant_block(v, block_amax(v), s_g, c0, c1);
    *reinterpret_cast<uint2*>(codes + row * (K / 2) + j * 8) = make_uint2(c0, c1);
    scales[row * bpr + j] = (uint8_t)sb;
  }
}

// Activation quantization.  Thread t of workgroup w owns the 8 elements at
// (w * kActThreads + t) * 8, half of one 16-element block; the other half is
// in the neighbouring lane.  The E2M1 rounding uses v_cvt_scalef32_pk_fp4_f32
// with scale 1.0: on gfx950 it rounds to nearest, ties to the even code,
// saturates at 6 and copies the sign, exactly the rule above (checked on
// hardware over every midpoint and its neighbours).  The division before it
// stays the IEEE one.
//   mode GS_SELF: every workgroup loads the whole tensor (at most
//   kActSelfElems elements, 16 loads per thread in flight per round) for
//   the global amax, so one launch does the whole step.  Workgroups are
//   small (T threads, 8 elements each): the per-element work (an IEEE
//   division per element) then spreads over many CUs instead of queueing
//   on the SIMDs of one.
// Loads go through a buffer resource over x: chunks past the end read as
// zero, so no load is predicated and no loaded value is used before the
// whole batch has been issued.  The amax of bf16 values is the unsigned max
// of their sign-cleared bit patterns (non-negative floats order like their
// bits), two per packed 16-bit max; wave maxima use DPP.
constexpr int kActBatch = 16;         // 16-byte amax loads per thread in flight at once
constexpr int kActSelfElems = 131072;  // GS_SELF limit (above it: two launches)
constexpr int kBufferWord3 = 0x00020000;                  // gfx9-family raw buffer resource, word 3

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t e2m1_pair(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// max over the wave (every lane gets it)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0x128>(x));  // row_ror:8
  x = max(x, dpp_u32<0x124>(x));  // row_ror:4
  x = max(x, dpp_u32<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp_u32<0x4E>(x));   // quad_perm [2,3,0,1]
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
  return max(a, b);
}

// max over the workgroup (T threads); one barrier when T > 64
template <int T>
__device__ __forceinline__ uint32_t wg_max_u32(uint32_t x, uint32_t* red) {
  x = wave_max_u32(x);
  if constexpr (T == 64) return x;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < T / 64; ++i) m = max(m, red[i]);
  return m;
}

template <int T>
__global__ __launch_bounds__(T) void quantize_act_kernel(
    const uint16_t* __restrict__ x, int64_t nelem, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, int mode,
    const float* __restrict__ partials, int n_parts) {
  __shared__ __align__(16) uint32_t red[T / 64];
  // segment blockIdx.y of nelem elements: the whole tensor (gridDim.y == 1),
  // or one row with its own global scale (per-token scales, gridDim.y == M)
  const int64_t seg = blockIdx.y;
  x += seg * nelem;
  codes += seg * (nelem / 2);
  scales += seg * (nelem / 16);
  gscale += seg;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, (int)(nelem * 2), kBufferWord3);
  const int mine = ((int)blockIdx.x * T + (int)threadIdx.x) * 8;  // first element of this thread
  const u32x4_t raw = __builtin_amdgcn_raw_buffer_load_b128(xr, mine * 2, 0, 0);
  float s_g;
  if (mode == GS_SELF) {
    uint32_t m = 0;
    for (int base = 0; base < (int)nelem; base += T * 8 * kActBatch) {  // uniform trip count
      u32x4_t v[kActBatch];
#pragma unroll
      for (int j = 0; j < kActBatch; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, (base + (j * T + (int)threadIdx.x) * 8) * 2, 0, 0);
#pragma unroll
      for (int j = 0; j < kActBatch; ++j)
        m = pk_max_u16(pk_max_u16(m, v[j][0] & 0x7FFF7FFFu),
                       pk_max_u16(v[j][1] & 0x7FFF7FFFu, pk_max_u16(v[j][2] & 0x7FFF7FFFu, v[j][3] & 0x7FFF7FFFu)));
    }
    m = max(m & 0xFFFFu, m >> 16);
    s_g = bf16_to_f32(wg_max_u32<T>(m, red)) / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = s_g;
  } else if (mode == GS_STATIC) {
    s_g = *gscale;
  } else {
    uint32_t m = 0;  // partial maxima are non-negative floats: compare their bits
    for (int i = threadIdx.x; i < n_parts; i += T) m = max(m, __float_as_uint(partials[i]));
    s_g = __uint_as_float(wg_max_u32<T>(m, red)) / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = s_g;
  }
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
  }
  // block amax over the two halves (neighbouring lanes 2k, 2k+1)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(amax))));
  if (mine < nelem) {
    float tb = 0.0f;
    if (s_g != 0.0f) {
      const float denom = 6.0f * s_g;
      tb = amax / denom;
    }
    const uint32_t sb = e4m3_code(tb);
    const float e = e4m3_value(sb) * s_g;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = e != 0.0f ? v[i] / e : copysignf(0.0f, v[i]);
    const uint32_t c = e2m1_pair(r[0], r[1]) | (e2m1_pair(r[2], r[3]) << 8) | (e2m1_pair(r[4], r[5]) << 16) |
                       (e2m1_pair(r[6], r[7]) << 24);
    *reinterpret_cast<uint32_t*>(codes + mine / 2) = c;
    if ((threadIdx.x & 1) == 0) scales[mine / 16] = (uint8_t)sb;
  }
}

__global__ void fill_zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Rotation-fused activation quantization ("Q+R"): the comparison point of the
// reading notes, section 5.3 and Table 3, where rotation-based NVFP4
// pipelines rotate the activation before quantizing it.  Here the rotation
// is the normalized Walsh-Hadamard transform H_R / sqrt(R) of every run of R
// consecutive elements of a row (R = 16, 32, 64 or 128), then the unchanged
// quantization.  A lane holds 8 consecutive elements, so an R-element block
// spans R / 8 consecutive lanes of a wave.  The butterfly runs stages
// h = 1, 2, 4 inside the lane, then h = 8, 16, 32, 64 across lanes (partner
// lane = lane ^ (h / 8)); each pair (i, i + h) becomes (a + b, a - b) in
// float32, then every element is multiplied by the float32 nearest to
// 1 / sqrt(R).  The global amax is that of the rotated tensor.
// ---------------------------------------------------------------------------

// x of lane (lane ^ d), d = 1, 2, 4 or 8, by DPP moves inside a 16-lane row
// (quad permutations for 1 and 2; row rotations, where lane i reads lane
// (i - n) mod 16 of its row, for 4 and 8)
__device__ __forceinline__ float lane_xor(float x, int d, int lane) {
  const uint32_t u = __float_as_uint(x);
  if (d == 1) return __uint_as_float(dpp_u32<0xB1>(u));  // quad_perm [1,0,3,2]
  if (d == 2) return __uint_as_float(dpp_u32<0x4E>(u));  // quad_perm [2,3,0,1]
  if (d == 8) return __uint_as_float(dpp_u32<0x128>(u));  // row_ror:8
  // d == 4: lanes with bit 2 set read lane - 4 (row_ror:4), the others lane + 4 (row_ror:12)
  const uint32_t down = dpp_u32<0x124>(u), up = dpp_u32<0x12C>(u);
  return __uint_as_float((lane & 4) ? down : up);
}

template <int R>
__device__ __forceinline__ float rotation_scale() {
  static_assert(R == 16 || R == 32 || R == 64 || R == 128, "rotation sizes");
  // 1 / sqrt(R): 1/4, 1/(4 sqrt 2), 1/8, 1/(8 sqrt 2)
  return R == 16 ? 0.25f : R == 32 ? 0.17677669529663688f : R == 64 ? 0.125f : 0.088388347648318440f;
}

// bf16 bits of 8 consecutive elements -> their rotated float32 values
// (every lane of the wave must call this together: the cross-lane stages
// exchange values with __shfl_xor)
template <int R>
__device__ __forceinline__ void rotate8(const u32x4_t raw, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
  }
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  const int lane = (int)threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < R / 8; d <<= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = lane_xor(v[i], d, lane);
      v[i] = upper ? q - v[i] : v[i] + q;
    }
  }
  const float c = rotation_scale<R>();
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * c;
}

__device__ __forceinline__ uint32_t amax8_bits(const float (&v)[8]) {
  uint32_t m = 0;  // |x| of non-negative floats orders like their bits
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return m;
}

// Pass 1 of the two-launch Q+R path: partials[b] = max |rotated x| over
// chunk b (chunks are whole multiples of 128 elements, so no rotation block
// straddles two workgroups).
template <int R>
__global__ __launch_bounds__(kThreads) void amax_rot_partials_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                                     float* __restrict__ partials) {
  __shared__ __align__(16) uint32_t red[kThreads / 64];
  const int64_t per = ((n / 128 + gridDim.x - 1) / gridDim.x) * 128;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, (int)(n * 2), kBufferWord3);
  uint32_t m = 0;
  for (int64_t i = lo; i < lo + per; i += (int64_t)kThreads * 8) {  // uniform trip count
    const int64_t e = i + (int64_t)threadIdx.x * 8;
    const int off = e < hi ? (int)(e * 2) : (int)0x7FFFFFF0;  // past the range: zeros
    float v[8];
    rotate8<R>(__builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0), v);
    m = max(m, amax8_bits(v));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t = max(t, red[w]);
    partials[blockIdx.x] = __uint_as_float(t);
  }
}

// Q+R, one launch per tensor (GS_SELF: every workgroup rotates the whole
// tensor for the amax; GS_STATIC; GS_FROM_PARTIALS after the pass above).
template <int T, int R>
__global__ __launch_bounds__(T) void quantize_act_rot_kernel(
    const uint16_t* __restrict__ x, int64_t nelem, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ gscale, int mode,
    const float* __restrict__ partials, int n_parts) {
  __shared__ __align__(16) uint32_t red[T / 64];
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, (int)(nelem * 2), kBufferWord3);
  const int mine = ((int)blockIdx.x * T + (int)threadIdx.x) * 8;  // first element of this thread
  const u32x4_t raw = __builtin_amdgcn_raw_buffer_load_b128(xr, mine * 2, 0, 0);
  float s_g;
  if (mode == GS_SELF) {
    uint32_t m = 0;
    for (int base = 0; base < (int)nelem; base += T * 8 * kActBatch) {  // uniform trip count
      u32x4_t v[kActBatch];
#pragma unroll
      for (int j = 0; j < kActBatch; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, (base + (j * T + (int)threadIdx.x) * 8) * 2, 0, 0);
#pragma unroll
      for (int j = 0; j < kActBatch; ++j) {
        float f[8];
        rotate8<R>(v[j], f);
        m = max(m, amax8_bits(f));
      }
    }
    s_g = __uint_as_float(wg_max_u32<T>(m, red)) / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = s_g;
  } else if (mode == GS_STATIC) {
    s_g = *gscale;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n_parts; i += T) m = max(m, __float_as_uint(partials[i]));
    s_g = __uint_as_float(wg_max_u32<T>(m, red)) / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *gscale = s_g;
  }
  float v[8];
  rotate8<R>(raw, v);
  // block amax over the two halves (neighbouring lanes 2k, 2k+1)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(amax))));
  if (mine < nelem) {
    float tb = 0.0f;
    if (s_g != 0.0f) {
      const float denom = 6.0f * s_g;
      tb = amax / denom;
    }
    const uint32_t sb = e4m3_code(tb);
    const float e = e4m3_value(sb) * s_g;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = e != 0.0f ? v[i] / e : copysignf(0.0f, v[i]);
    const uint32_t c = e2m1_pair(r[0], r[1]) | (e2m1_pair(r[2], r[3]) << 8) | (e2m1_pair(r[4], r[5]) << 16) |
                       (e2m1_pair(r[6], r[7]) << 24);
    *reinterpret_cast<uint32_t*>(codes + mine / 2) = c;
    if ((threadIdx.x & 1) == 0) scales[mine / 16] = (uint8_t)sb;
  }
}

int64_t quant_grid(int64_t nblocks) {
  int64_t g = (nblocks + kThreads - 1) / kThreads;
  if (g > 4096) g = 4096;
  return g < 1 ? 1 : g;
}

}  // namespace

int amax_partial_count(int64_t elems) {
  int64_t p = (elems + 4095) / 4096;
  if (p > 2048) p = 2048;
  return (int)(p < 1 ? 1 : p);
}

hipError_t launch_quantize_bf16(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                                uint8_t* scales, float* gscale, GsMode mode, float* partials,
                                int n_parts, bool per_token, hipStream_t stream) {
  // per-token scales: one segment (and one global scale) per row
  const int64_t nelem = per_token ? K : rows * K;
  const unsigned segs = per_token ? (unsigned)rows : 1u;
  if (per_token && mode == GS_FROM_PARTIALS) return hipErrorInvalidValue;
  if (mode == GS_SELF && nelem > kActSelfElems) return hipErrorInvalidValue;
  if (mode == GS_FROM_PARTIALS) {
    hipLaunchKernelGGL(amax_partials_kernel<uint16_t>, dim3(n_parts), dim3(kThreads), 0, stream, x, nelem,
                       partials);
  }
  // workgroup size, from graph-replayed timings of every decode shape: when
  // every workgroup reads the whole tensor for the amax (GS_SELF), larger
  // tensors want fewer, larger workgroups; otherwise each workgroup reads
  // only its own chunk and 64 threads spread the divisions over the most CUs
  const int threads = mode != GS_SELF  ? 64
                      : nelem <= 8192  ? 64
                      : nelem <= 16384 ? 128
                      : nelem <= 32768 ? 256
                                       : 512;
  const int64_t grid = (nelem + (int64_t)threads * 8 - 1) / ((int64_t)threads * 8);
  auto fn = threads == 64    ? quantize_act_kernel<64>
            : threads == 128 ? quantize_act_kernel<128>
            : threads == 256 ? quantize_act_kernel<256>
                             : quantize_act_kernel<512>;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid, segs), dim3(threads), 0, stream, x, nelem, codes, scales, gscale,
                     (int)mode, partials, n_parts);
  return hipGetLastError();
}

namespace {

template <int R>
hipError_t launch_quantize_rot(const uint16_t* x, int64_t nelem, uint8_t* codes, uint8_t* scales, float* gscale,
                               GsMode mode, float* partials, int n_parts, hipStream_t stream) {
  if (mode == GS_FROM_PARTIALS)
    hipLaunchKernelGGL(amax_rot_partials_kernel<R>, dim3(n_parts), dim3(kThreads), 0, stream, x, nelem, partials);
  // the workgroup sizes of the plain quantization (the rotation adds a few
  // VALU operations per element and does not change the balance)
  const int threads = mode != GS_SELF  ? 64
                      : nelem <= 8192  ? 64
                      : nelem <= 16384 ? 128
                      : nelem <= 32768 ? 256
                                       : 512;
  const int64_t grid = (nelem + (int64_t)threads * 8 - 1) / ((int64_t)threads * 8);
  auto fn = threads == 64    ? quantize_act_rot_kernel<64, R>
            : threads == 128 ? quantize_act_rot_kernel<128, R>
            : threads == 256 ? quantize_act_rot_kernel<256, R>
                             : quantize_act_rot_kernel<512, R>;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), 0, stream, x, nelem, codes, scales, gscale, (int)mode,
                     partials, n_parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rotated(const uint16_t* x, int64_t elems, int rot, uint8_t* codes, uint8_t* scales,
                                   float* gscale, GsMode mode, float* partials, int n_parts, hipStream_t stream) {
  if (mode == GS_SELF && elems > kActSelfElems) return hipErrorInvalidValue;
  switch (rot) {
    case 16: return launch_quantize_rot<16>(x, elems, codes, scales, gscale, mode, partials, n_parts, stream);
    case 32: return launch_quantize_rot<32>(x, elems, codes, scales, gscale, mode, partials, n_parts, stream);
    case 64: return launch_quantize_rot<64>(x, elems, codes, scales, gscale, mode, partials, n_parts, stream);
    case 128: return launch_quantize_rot<128>(x, elems, codes, scales, gscale, mode, partials, n_parts, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_f32(const float* x, int64_t rows, int64_t K, uint8_t* codes,
                               uint8_t* scales, float* gscale, float* partials, int n_parts,
                               hipStream_t stream) {
  const int64_t nblocks = rows * (K / 16);
  hipLaunchKernelGGL(amax_partials_kernel<float>, dim3(n_parts), dim3(kThreads), 0, stream, x,
                     rows * K, partials);
  hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)quant_grid(nblocks)), dim3(kThreads), 0,
                     stream, x, rows, K, codes, scales, gscale, (int)GS_FROM_PARTIALS, partials,
                     n_parts);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t g = (n16 + 255) / 256;
  if (g > 1024) g = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace nvfp4
