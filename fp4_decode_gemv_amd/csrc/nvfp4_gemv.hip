// Small-M NVFP4 GEMV for gfx950 (CDNA4), y[M][N] = A[M][K] . W[N][K]^T.
//
// What the method asks for (ReSET project page, "Core contribution -- the
// nvfp4r CUDA-core kernel", C1-C3; reading notes section 5.2): every weight
// tile streamed from HBM once for all M tokens (C1), several independent
// accumulator chains per thread (C2), FP4 unpacked in registers and fed
// straight to the multiply-adds (C3).  The pages' Blackwell design is prior
// art; this is the CDNA4 form of the same idea:
//
//   * A workgroup owns a tile of weight rows.  G consecutive lanes of a
//     wave64 share one row; each lane loads 16 bytes (32 codes = 2 blocks)
//     per step with one dwordx4 load, so a row-group streams G*16 contiguous
//     bytes per instruction, and R rows per lane give R*M independent chains.
//   * The quantized activation of a K phase is decoded ONCE per workgroup
//     into LDS as f16 values a = E2M1(q) * E4M3(s_b) (exact in f16: at most
//     6 significant bits, magnitudes in [2^-10, 2688]), laid out so that the
//     G lanes of a row-group read 16 consecutive bytes each (no bank
//     conflicts) and the row-groups of a wave read the same addresses
//     (broadcast).
//   * Weight codes are decoded in registers with v_cvt_scalef32_pk_f16_fp4
//     (scale 1.0: that instruction applies only the exponent of its scale
//     operand, so the E4M3 block scale is applied separately).
//   * Per 16-element block and token, 8 v_dot2c_f32_f16 give the exact block
//     sum (products have <= 8 significant bits, a block sum <= 16 bits), and
//     one FMA applies the weight block scale, decoded with v_cvt_pk_f32_fp8
//     (OCP E4M3).  Two accumulators per (row, token) alternate blocks.
//   * Lanes of a row-group are reduced with cross-lane shuffles; the two
//     global scales multiply the result once.
//
// Error: products and block sums are exact; every accumulation chain is at
// most K/(32G) + 1 + log2(G) + 2 roundings long, far inside the 1e-5
// relative bound for the shapes served.
//
// Optional LM-head epilogue (ReSET project page, "Step-aware temperature
// scaling"; reading notes sections 3.1, 4.1-4.3): each workgroup also
// writes per-token softmax partials (max, sum e^(z-max), sum e^(z-max)(z-max))
// of its logits to the workspace; the last workgroup to finish (atomic
// counter, reset by that workgroup) merges them in a fixed order, computes
// the entropy and runs the ReSET update on the device-resident state.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

struct GemvParams {
  int M;
  int64_t N, K;
  int kp;  // K elements per LDS phase (multiple of 32)
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_gscale;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_gscale;
  float* y;
  // LM-head epilogue (used only by the EPI instantiations)
  EpilogueArgs epi;
  unsigned* counter;
  float* partials;      // [gridDim.x][MT][3]
  size_t state_bytes;   // bytes per ReSET state
};

// ReSET per-sequence state (device).  Followed by float ring[window].
struct ResetState {
  double sum_all;    // sum of all entropies so far
  double step_sum;   // sum over the current step
  int64_t count;     // positions seen
  int32_t step_len;  // positions in the current step
  int32_t window;
};

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

template <int B>
__device__ __forceinline__ half2_t fp4x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, B);
}

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
    out[b] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0] * sa, f[1] * sa));
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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

template <int MT, int G, int R, int NW, bool EPI>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(GemvParams p) {
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
    const int C = (int)((K - kb < p.kp ? K - kb : p.kp) / 32);  // chunks in this phase
    const uint8_t* wcp[R];
    const uint8_t* wsp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wcp[r] = wc[r] + kb / 2;
      wsp[r] = ws[r] + kb / 16;
    }
    // first weight chunk of the phase, in flight while the activation is staged
    uint4 wn[R];
    uint32_t sn[R];
    if (g < C) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wn[r] = *reinterpret_cast<const uint4*>(wcp[r] + g * 16);
        sn[r] = *reinterpret_cast<const uint16_t*>(wsp[r] + g * 2);
      }
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
        const uint32_t sb = p.a_scales[(int64_t)m * (K / 16) + k / 16];
        const float sa = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false)[0];
        v = act_decode8(word, sa);
      }
      lds[(m * 4 + q) * C + c] = v;
    }
    __syncthreads();

    for (int c = g; c < C; c += G) {
      uint4 w[R];
      uint32_t s[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        w[r] = wn[r];
        s[r] = sn[r];
      }
      if (c + G < C) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          wn[r] = *reinterpret_cast<const uint4*>(wcp[r] + (c + G) * 16);
          sn[r] = *reinterpret_cast<const uint16_t*>(wsp[r] + (c + G) * 2);
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

  // reduce the G lanes of each row-group
  const float scale = (*p.a_gscale) * (*p.w_gscale);
  float out[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m][0] + acc[r][m][1];
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      out[r][m] = v * scale;
    }
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (row[r] < N)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < M) p.y[(int64_t)m * N + row[r]] = out[r][m];
  }

  if constexpr (EPI) {
    // ---- per-workgroup softmax partials of this tile's logits ----
    __shared__ float red[NW * RG][MT][3];
    __shared__ float fin[MT][3];
    __shared__ unsigned last;
    float mx[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (row[r] < N) v = fmaxf(v, out[r][m]);
      mx[m] = v;
    }
    const int slot = wave * RG + rg;
    if (g == 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) red[slot][m][0] = mx[m];
    __syncthreads();
    if (threadIdx.x < MT) {
      float v = -INFINITY;
      for (int s = 0; s < NW * RG; ++s) v = fmaxf(v, red[s][threadIdx.x][0]);
      fin[threadIdx.x][0] = v;
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float gm = fin[m][0];
        float S = 0.0f, T = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (row[r] < N) {
            const float d = out[r][m] - gm;
            const float e = expf(d);
            S += e;
            T = __builtin_fmaf(e, d, T);
          }
        red[slot][m][1] = S;
        red[slot][m][2] = T;
      }
    }
    __syncthreads();
    if (threadIdx.x < MT) {
      float S = 0.0f, T = 0.0f;
      for (int s = 0; s < NW * RG; ++s) {
        S += red[s][threadIdx.x][1];
        T += red[s][threadIdx.x][2];
      }
      float* dst = p.partials + ((int64_t)blockIdx.x * MT + threadIdx.x) * 3;
      dst[0] = fin[threadIdx.x][0];
      dst[1] = S;
      dst[2] = T;
    }
    // ---- the last workgroup merges ----
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = (atomicAdd(p.counter, 1u) == gridDim.x - 1) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    __threadfence();
    const int nwg = gridDim.x;
    constexpr int NT = NW * 64;
    __shared__ float mred[NT];
    __shared__ float sred[NT];
    __shared__ float tred[NT];
    for (int m = 0; m < M; ++m) {
      // global max
      float gm = -INFINITY;
      for (int b = threadIdx.x; b < nwg; b += NT)
        gm = fmaxf(gm, __builtin_nontemporal_load(p.partials + ((int64_t)b * MT + m) * 3));
      mred[threadIdx.x] = gm;
      __syncthreads();
      for (int s = NT / 2; s >= 1; s >>= 1) {
        if (threadIdx.x < s) mred[threadIdx.x] = fmaxf(mred[threadIdx.x], mred[threadIdx.x + s]);
        __syncthreads();
      }
      gm = mred[0];
      // rescaled sums: S = sum_b S_b e^(m_b - gm); T = sum_b e^(m_b - gm) (T_b + (m_b - gm) S_b)
      float S = 0.0f, T = 0.0f;
      for (int b = threadIdx.x; b < nwg; b += NT) {
        const float* src = p.partials + ((int64_t)b * MT + m) * 3;
        const float mb = __builtin_nontemporal_load(src);
        const float Sb = __builtin_nontemporal_load(src + 1);
        const float Tb = __builtin_nontemporal_load(src + 2);
        if (mb == -INFINITY) continue;
        const float d = mb - gm;
        const float f = expf(d);
        S = __builtin_fmaf(Sb, f, S);
        T = __builtin_fmaf(f, __builtin_fmaf(d, Sb, Tb), T);
      }
      __syncthreads();
      sred[threadIdx.x] = S;
      tred[threadIdx.x] = T;
      __syncthreads();
      for (int s = NT / 2; s >= 1; s >>= 1) {
        if (threadIdx.x < s) {
          sred[threadIdx.x] += sred[threadIdx.x + s];
          tred[threadIdx.x] += tred[threadIdx.x + s];
        }
        __syncthreads();
      }
      if (threadIdx.x == 0) {
        const double Sd = sred[0], Td = tred[0];
        const double H = log(Sd) - Td / Sd;
        p.epi.entropy[m] = (float)H;
        // ---- ReSET update: update with H first, then decide ----
        ResetState* st = reinterpret_cast<ResetState*>(reinterpret_cast<char*>(p.epi.state) + (size_t)m * p.state_bytes);
        float* ring = reinterpret_cast<float*>(st + 1);
        // the ring holds the window the state was initialised with; never
        // index past the smaller of that and the caller's window
        int w = st->window < p.epi.window ? st->window : p.epi.window;
        if (w < 1) w = 1;
        const double h = (double)(float)H;
        if (st->count == 0 || p.epi.step_start[m]) {
          st->step_sum = 0.0;
          st->step_len = 0;
        }
        ring[st->count % w] = (float)H;
        st->count += 1;
        st->sum_all += h;
        st->step_sum += h;
        st->step_len += 1;
        const int64_t nwin = st->count < w ? st->count : w;
        double wsum = 0.0;
        for (int64_t i = st->count - nwin; i < st->count; ++i) wsum += (double)ring[i % w];
        const double hbar = st->sum_all / (double)st->count;
        const double hstep = st->step_len <= w ? wsum / (double)nwin : st->step_sum / (double)st->step_len;
        const double tau = hstep > hbar ? hstep : (double)p.epi.tau0;
        float T_t;
        if (p.epi.mode == 1) T_t = p.epi.t_base;
        else T_t = h < tau ? p.epi.t_low : p.epi.t_high;
        p.epi.temperature[m] = T_t;
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) *p.counter = 0u;  // ready for the next call / graph replay
  }
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

template <int MT, int G, int R, int NW>
hipError_t launch_one(const GemvConfig& cfg, const GemvParams& p, hipStream_t stream, bool epi) {
  const size_t lds_bytes = (size_t)MT * 4 * (cfg.kp / 32) * 16;
  if (epi)
    hipLaunchKernelGGL((gemv_kernel<MT, G, R, NW, true>), dim3((unsigned)cfg.grid), dim3(NW * 64), lds_bytes,
                       stream, p);
  else
    hipLaunchKernelGGL((gemv_kernel<MT, G, R, NW, false>), dim3((unsigned)cfg.grid), dim3(NW * 64), lds_bytes,
                       stream, p);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const GemvConfig& cfg, const GemvParams& p, hipStream_t stream, bool epi) {
  if (cfg.g == 16 && cfg.r == 1 && cfg.waves == 4) return launch_one<MT, 16, 1, 4>(cfg, p, stream, epi);
  if (cfg.g == 16 && cfg.r == 2 && cfg.waves == 4) return launch_one<MT, 16, 2, 4>(cfg, p, stream, epi);
  return hipErrorInvalidConfiguration;
}

}  // namespace

size_t reset_state_bytes(int window) {
  const size_t b = sizeof(ResetState) + sizeof(float) * (size_t)window;
  return (b + 15) & ~(size_t)15;
}

GemvConfig choose_gemv_config(int M, int64_t N, int64_t K, bool epi) {
  GemvConfig c{};
  c.mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  c.g = 16;
  c.waves = 4;
  c.r = N >= 16384 ? 2 : 1;
  // LDS phase: at most 64 KiB of f16 activation per workgroup (48 KiB when
  // the epilogue's reduction buffers share the LDS), in whole rounds of G
  // chunks when K allows it
  int64_t kp = (epi ? (int64_t)24576 : (int64_t)32768) / c.mt;
  const int64_t unit = (int64_t)32 * c.g;
  if (kp >= unit) kp = kp / unit * unit;
  if (kp > K) kp = K;
  c.kp = (int)kp;
  c.rows_per_wg = (int64_t)c.r * c.waves * (64 / c.g);
  c.grid = (N + c.rows_per_wg - 1) / c.rows_per_wg;
  return c;
}

size_t lmhead_workspace_bytes(int M, int64_t N, int64_t K) {
  const GemvConfig c = choose_gemv_config(M, N, K, true);
  return 256 + (size_t)c.grid * c.mt * 3 * sizeof(float);
}

hipError_t launch_gemv(const GemvConfig& cfg, int M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_gscale, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* w_gscale, float* y,
                       const EpilogueArgs* epi, void* ws, hipStream_t stream) {
  GemvParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.kp = cfg.kp;
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_gscale = a_gscale;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.w_gscale = w_gscale;
  p.y = y;
  if (epi) {
    p.epi = *epi;
    p.counter = reinterpret_cast<unsigned*>(ws);
    p.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 256);
    p.state_bytes = reset_state_bytes(epi->window);
  }
  const bool e = epi != nullptr;
  switch (cfg.mt) {
    case 1: return launch_mt<1>(cfg, p, stream, e);
    case 2: return launch_mt<2>(cfg, p, stream, e);
    case 4: return launch_mt<4>(cfg, p, stream, e);
    case 8: return launch_mt<8>(cfg, p, stream, e);
  }
  return hipErrorInvalidConfiguration;
}

hipError_t launch_reset_state_init(void* state, int M, int window, hipStream_t stream) {
  hipLaunchKernelGGL(reset_state_init_kernel, dim3(M), dim3(256), 0, stream, reinterpret_cast<char*>(state), M,
                     window, reset_state_bytes(window));
  return hipGetLastError();
}

}  // namespace nvfp4
