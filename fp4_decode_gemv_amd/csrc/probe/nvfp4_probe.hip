// Measurement and test probes for gfx950, built as their own library
// (lib/libnvfp4_probe.so, C ABI in include/nvfp4_probe.h).  Nothing in the
// decode-projection library calls them.
//
// 1. HBM read-stream probe.  A decode projection is a single streaming read of
//    the packed weights (ReSET project page, "Why a CUDA-core NVFP4
//    kernel?": the speedup comes from moving fewer weight bytes), so the
//    fastest plain read of the same number of bytes is the ceiling the GEMV
//    can reach on this machine, next to the 8 TB/s of the data sheet.  The
//    probe reads a buffer once and folds every byte into an XOR (so no load
//    can be dropped), in one of two forms:
//      read_vgpr: each workgroup owns one contiguous slice of the buffer;
//                 every lane keeps U 16-byte buffer loads in flight in a
//                 register ring (optionally with the non-temporal hint);
//      read_lds:  the same slices, but each wave streams its 1 KB chunks
//                 straight into an LDS ring of D slots (direct-to-LDS
//                 buffer loads, no VGPRs in flight) and reads them back.
//    The launch grid is the caller's; the best over the variants and grids is
//    the measured ceiling.
// 2. Converter probe: runs the gfx950 conversion instructions the NVFP4
//    kernels rely on over caller-supplied inputs, so a test can compare them
//    with the exact decode of the E2M1 and E4M3 formats (ReSET reading notes,
//    section 2.1) and with round-to-nearest-even E2M1 encoding.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/nvfp4_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kBufferWord3 = 0x00020000;  // raw byte-addressed buffer resource (gfx9 family)
constexpr int kThreads = 256;
constexpr uint32_t kMagic = 0x9E3779B9u;  // the sink is written only if the XOR equals this

// Slice [lo, hi) of workgroup b when `bytes` (a multiple of 16) is cut into
// gridDim.x slices of whole 16-byte units.
__device__ __forceinline__ void slice_of(int64_t bytes, int64_t& lo, int64_t& hi) {
  const int64_t units = bytes / 16;
  const int64_t per = (units + gridDim.x - 1) / gridDim.x;
  lo = (int64_t)blockIdx.x * per * 16;
  hi = lo + per * 16;
  if (lo > bytes) lo = bytes;
  if (hi > bytes) hi = bytes;
}

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void read_vgpr_kernel(const uint8_t* __restrict__ buf, int64_t bytes,
                                                             uint32_t* __restrict__ sink) {
  int64_t lo, hi;
  slice_of(bytes, lo, hi);
  const int64_t per = ((bytes / 16 + gridDim.x - 1) / gridDim.x) * 16;  // same for every workgroup
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf + lo), (short)0, (int)(hi - lo), kBufferWord3);
  // step i of a lane reads 16 bytes at (i * kThreads + tid) * 16 of the slice;
  // offsets past the slice read as zero without a memory access
  const int steps = (int)((per / 16 + kThreads - 1) / kThreads);
  const int tid = (int)threadIdx.x;
  u32x4_t ring[U];
#pragma unroll
  for (int j = 0; j < U; ++j)
    ring[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (j * kThreads + tid) * 16, 0, NT ? 2 : 0);
  uint32_t acc = 0;
  for (int i0 = 0; i0 < steps; i0 += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      acc ^= ring[j][0] ^ ring[j][1] ^ ring[j][2] ^ ring[j][3];
      const int i = i0 + j + U;  // past the slice when i >= steps: reads zero
      ring[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * kThreads + tid) * 16, 0, NT ? 2 : 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the refill here: U loads stay in flight
    }
  }
  if (acc == kMagic) sink[blockIdx.x] = acc;
}

// lane i: 16 bytes from rsrc at voff to LDS byte lds + 16 i
__device__ __forceinline__ void dma_b128(const i32x4_t& rsrc, uint32_t lds, int voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(min(later, D - 1)) for a runtime `later` >= 0
template <int D>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (D <= 1) {
    wait_vmcnt<0>();
  } else {
    if (later >= D - 1) wait_vmcnt<D - 1>();
    else wait_later<D - 1>(later);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void read_lds_kernel(const uint8_t* __restrict__ buf, int64_t bytes,
                                                            uint32_t* __restrict__ sink) {
  extern __shared__ uint4 lds4[];  // [4 waves][D slots][1 KB]
  int64_t lo, hi;
  slice_of(bytes, lo, hi);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t a = reinterpret_cast<uint64_t>(buf + lo);
  const i32x4_t rsrc = {(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)(hi - lo), kBufferWord3};
  const int chunks = (int)((hi - lo + 1023) / 1024);
  const int n = wave < chunks ? (chunks - wave + 3) / 4 : 0;  // chunks wave, wave + 4, ...
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds4));
  const uint32_t ring = lds0 + (uint32_t)(wave * D * 1024);
  auto issue = [&](int i) { dma_b128(rsrc, ring + (uint32_t)((i % D) * 1024), (wave + 4 * i) * 1024 + 16 * lane); };
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (j < n) issue(j);
  const uint4* rd = lds4 + wave * D * 64 + lane;
  uint32_t acc = 0;
  for (int i = 0; i < n; ++i) {
    if (i + D - 1 < n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reused slot's reads have returned
      issue(i + D - 1);
    }
    wait_later<D>(n - 1 - i);
    const uint4 v = rd[(i % D) * 64];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kMagic) sink[blockIdx.x] = acc;
}

__global__ void empty_kernel() {}

struct ReadVariant {
  const char* name;
  void (*fn)(const uint8_t*, int64_t, uint32_t*);
  int lds_bytes;
};

#define VGPR_V(U, NT) ReadVariant{"vgpr_u" #U "_" #NT, read_vgpr_kernel<U, NT != 0>, 0}
#define LDS_V(D) ReadVariant{"lds_d" #D, read_lds_kernel<D>, 4 * D * 1024}

const ReadVariant kRead[] = {
    VGPR_V(1, 0), VGPR_V(2, 0), VGPR_V(4, 0), VGPR_V(8, 0), VGPR_V(16, 0),
    VGPR_V(1, 1), VGPR_V(2, 1), VGPR_V(4, 1), VGPR_V(8, 1), VGPR_V(16, 1),
    LDS_V(2),     LDS_V(4),     LDS_V(8),     LDS_V(16),
};
constexpr int kNumRead = sizeof(kRead) / sizeof(kRead[0]);

// ---------------------------------------------------------------- converters

template <int B>
__device__ __forceinline__ uint32_t f16x2_of_fp4(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}
// Vector elements are converted to bits with __float_as_uint: hipcc (clang
// 22, ROCm 7.2) compiles __builtin_bit_cast of an element of an
// ext_vector_type float pair as a bit cast of element 0.
template <int B>
__device__ __forceinline__ void f32x2_of_fp4(uint32_t w, uint32_t* o) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  o[0] = __float_as_uint(f[0]);
  o[1] = __float_as_uint(f[1]);
}

__global__ void convert_kernel(int op, const uint32_t* __restrict__ in, uint32_t* __restrict__ out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = in[i];
  switch (op) {
    case NVFP4_PROBE_FP4_TO_F16:  // four byte selectors, one half2 each
      out[4 * i + 0] = f16x2_of_fp4<0>(w);
      out[4 * i + 1] = f16x2_of_fp4<1>(w);
      out[4 * i + 2] = f16x2_of_fp4<2>(w);
      out[4 * i + 3] = f16x2_of_fp4<3>(w);
      break;
    case NVFP4_PROBE_FP4_TO_F32:  // four byte selectors, two floats each
      f32x2_of_fp4<0>(w, out + 8 * i + 0);
      f32x2_of_fp4<1>(w, out + 8 * i + 2);
      f32x2_of_fp4<2>(w, out + 8 * i + 4);
      f32x2_of_fp4<3>(w, out + 8 * i + 6);
      break;
    case NVFP4_PROBE_FP8_TO_F32: {  // low and high 16 bits, two floats each
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
      out[4 * i + 0] = __float_as_uint(lo[0]);
      out[4 * i + 1] = __float_as_uint(lo[1]);
      out[4 * i + 2] = __float_as_uint(hi[0]);
      out[4 * i + 3] = __float_as_uint(hi[1]);
      break;
    }
    case NVFP4_PROBE_F32_TO_FP4: {  // in[2i], in[2i+1] are two floats -> one byte (n counts pairs)
      const float a = __builtin_bit_cast(float, in[2 * i]), b = __builtin_bit_cast(float, in[2 * i + 1]);
      out[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
      break;
    }
    case NVFP4_PROBE_F16_SCALE_MUL: {  // packed f16 product (the MFMA kernels' block-scale multiply)
      const half2_t x = __builtin_bit_cast(half2_t, in[2 * i]), y = __builtin_bit_cast(half2_t, in[2 * i + 1]);
      out[i] = __builtin_bit_cast(uint32_t, x * y);
      break;
    }
  }
}

}  // namespace

extern "C" {

int nvfp4_probe_read_count(void) { return kNumRead; }

const char* nvfp4_probe_read_name(int variant) {
  return variant >= 0 && variant < kNumRead ? kRead[variant].name : nullptr;
}

int nvfp4_probe_read(int variant, const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream) {
  if (variant < 0 || variant >= kNumRead) return NVFP4_PROBE_ERR_ARG;
  if (!buf || !sink) return NVFP4_PROBE_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes < 16 || bytes % 16 != 0) return NVFP4_PROBE_ERR_ARG;
  if (grid < 1 || grid > 1 << 20) return NVFP4_PROBE_ERR_ARG;
  // a slice is addressed with 32-bit offsets
  if ((bytes / 16 + (size_t)grid - 1) / (size_t)grid * 16 >= ((size_t)1 << 31) - (1 << 20)) return NVFP4_PROBE_ERR_ARG;
  hipLaunchKernelGGL(kRead[variant].fn, dim3((unsigned)grid), dim3(kThreads), (size_t)kRead[variant].lds_bytes,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf), (int64_t)bytes, sink);
  return hipGetLastError() == hipSuccess ? NVFP4_PROBE_OK : NVFP4_PROBE_ERR_HIP;
}

int nvfp4_probe_empty(int grid, int threads, void* stream) {
  if (grid < 1 || grid > 1 << 20 || threads < 1 || threads > 1024) return NVFP4_PROBE_ERR_ARG;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)grid), dim3((unsigned)threads), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? NVFP4_PROBE_OK : NVFP4_PROBE_ERR_HIP;
}

int nvfp4_probe_convert(int op, const uint32_t* in, uint32_t* out, int n, void* stream) {
  if (op < NVFP4_PROBE_FP4_TO_F16 || op > NVFP4_PROBE_F16_SCALE_MUL) return NVFP4_PROBE_ERR_ARG;
  if (!in || !out || n < 1 || n > (1 << 24)) return NVFP4_PROBE_ERR_ARG;
  hipLaunchKernelGGL(convert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     op, in, out, n);
  return hipGetLastError() == hipSuccess ? NVFP4_PROBE_OK : NVFP4_PROBE_ERR_HIP;
}

}  // extern "C"
