// Top-p (nucleus) sampling of one token per sequence from the LM-head logits,
// at the temperature the ReSET rule chose for it, on gfx950.
//
// What is drawn (ReSET reading notes, section 6.1: the decode loop samples
// with top-p = 0.95; section 4.3: the per-token temperature; nucleus sampling
// as published by Holtzman et al., ICLR 2020):
//   p_i    = softmax(z / T)_i over all N logits of the row
//   order  = decreasing z, equal z by increasing index
//   n      = length of the shortest prefix of the order whose mass >= top_p
//   token  = the first token of the order whose cumulative mass exceeds
//            u * (mass of the first n tokens), u in [0, 1) given per row.
//
// Four launches (for a peaked row, in effect two), no sort of the row.
// Masses are 2^-40 fixed point relative to the row maximum:
// e_i = exp2((z_i - z_max) * log2(e) / T) in float32, m_i = floor(e_i 2^40).
// Integer sums are associative, so the result does not depend on the order
// of the atomic adds, and the one floating-point sum (the row mass of the
// listed path) runs in a fixed order: repeated calls give the same token.
//   1. (G workgroups of 1024 threads per row) chunk maxima; the row's
//      histogram is cleared.
//      Also each chunk's mass relative to its own maximum and a short list
//      of its elements near that maximum.
//   2. (first) every workgroup puts the row mass together from those
//      records; when the listed elements (a prefix of the order) hold the
//      nucleus, the cuts are found among them, workgroup 0 writes the token,
//      the row is marked resolved and launches 2 to 4 end for it.
//   2. (G workgroups per row) every element's bucket b_i of
//      a_i = (z_max - z_i) log2(e) / T, 1/64 wide over 2048 buckets (the
//      last holds a_i >= 31.98, masses below 2^-31.98), is stored as 16 bits
//      and its mass and count added to the row's histograms.  The bucket index never
//      decreases as z decreases, so a bucket is a contiguous run of the
//      order.
//   3. (G workgroups per row) both cut points (the nucleus end, then the
//      draw) are "the first element of the order whose inclusive cumulative
//      mass reaches t", and t lies in the bucket whose inclusive prefix first
//      reaches it.  The first bucket follows from the histogram; the second
//      depends on the mass through the first cut, which lies within the
//      first bucket, so it lies in a bucket range the histogram also gives.
//      The elements of these buckets (key = order-preserving bits of z, then
//      index; mass; bucket) are gathered per workgroup in LDS and appended to
//      a per-row list of 4096 with one atomic per workgroup.
//   4. (one workgroup of 1024 threads per row) the list is copied into LDS;
//      each cut takes the elements of its bucket from it (the number of
//      elements before the bucket comes from the count prefix).  With at most
//      256 of them each one sums the masses of those before it and the one
//      whose interval holds t is the cut; with more, they are histogrammed
//      in LDS by the next 10 bits of the unique key (order key, index) and
//      the search narrows to one sub-bucket until at most 256 remain.  If
//      the list overflowed, passes over the bucket ids (a packed compare
//      skips each group of eight without the bucket) collect the bucket's
//      elements, reading only their logits, narrowing the same way by the
//      order key (at most four times; then all candidates share one logit
//      and, having equal masses, the cut is found by counting them in index
//      order).
//
// Logits must be finite; T must be positive and finite (otherwise the row's
// token is -1 and its nucleus size 0).  u outside [0, 1) is clamped into it.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nvfp4_internal.h"

#pragma clang fp contract(off)

namespace nvfp4 {
namespace {

constexpr int kThreads = 1024;          // selection: one workgroup per row
constexpr int kWaves = kThreads / 64;
constexpr int kWide = 256;              // launches 1 to 3: threads per workgroup
constexpr int kBuckets = 2048;          // level-0 buckets, 1/64 of a unit of a_i each
constexpr int kSubBits = 10;            // key bits per refinement level
constexpr int kSub = 1 << kSubBits;     // == kThreads: one sub-bucket per thread
constexpr int kCap = 256;               // candidates ranked directly
constexpr int kList = 4096;             // per row: elements of the buckets the cuts can fall in
constexpr int kListPer = kList / kThreads;  // list entries per selection thread
constexpr int kWGList = 1024;           // launch 3: elements a workgroup gathers before publishing
constexpr int kBatch = 4;               // 16-byte loads per thread in flight
constexpr int kSpec = 32;               // launch 1: elements a chunk lists for the listed path
constexpr float kSpecSpan = 20.0f;      // ... those within 2^-20 of the chunk maximum's mass
constexpr int kSpecMaxChunks = 256;     // longer rows (N > 1M) always take the histogram path
constexpr int kSpecPre = 8;             // listed slots per thread loaded with the chunk records
constexpr uint32_t kSpecOverflow = 0xFFFFFFFFu;
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
static_assert(kSub == kThreads, "one refinement bucket per thread");
static_assert(kSampleChunk == kWide * 16, "a chunk is four 16-byte loads per thread");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

struct SampleArgs {
  int64_t N;
  int64_t bstride;  // bucket ids per row: N rounded up to 8
  int G;            // chunks of kSampleChunk elements per row
  const float* logits;
  const float* temperature;
  const float* uniforms;
  int32_t* tokens;
  int32_t* nucleus;
  float top_p;
  float* maxp;                // [M][G] chunk maxima
  unsigned long long* hist;   // [M][kBuckets] mass per bucket
  uint32_t* hcnt;             // [M][kBuckets] elements per bucket
  uint16_t* bid;              // [M][bstride] bucket of every element
  uint32_t* lcount;           // [M] elements collected by launch 3 (may pass kList)
  uint64_t* lkey;             // [M][kList] key << 32 | index
  uint64_t* lmass;            // [M][kList]
  uint32_t* lbkt;             // [M][kList] bucket
  u32x4_t* crec;              // [M][G] chunk record: maximum (float bits), elements listed
                              // (kSpecOverflow past kSpec), mass relative to the maximum (u64)
  uint64_t* cand;             // [M][G][kSpec] listed elements: logit bits << 32 | index
  uint32_t* resolved;         // [M] 1: launch 2 drew the row's token from the lists
};

// Ascending in sampling order: larger z first; -0 and +0 are one value.
__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // increasing with z
  return ~asc;
}

__device__ __forceinline__ int bucket_of(float a) { return (int)fminf(a * 64.0f, (float)(kBuckets - 1)); }

// floor(exp2(-a) * 2^40) for a >= 0: exp2(-a) has 24 significant bits, so the
// product is split into its integer part (< 2^8 + 1) and 32 fraction bits,
// each converted exactly.
__device__ __forceinline__ uint64_t fixed_mass(float a) {
  const float e = exp2f(-a);
  if (!(e > 0.0f)) return 0;
  const float e8 = e * 256.0f;
  const uint32_t hi = (uint32_t)e8;
  const uint32_t lo = (uint32_t)((e8 - (float)hi) * 4294967296.0f);
  return ((uint64_t)hi << 32) | lo;
}

// log2(e) / T, or false when T is not positive and finite.  A denormal T
// overflows the quotient; it is clamped (the greedy limit).
__device__ __forceinline__ bool scale_of(float T, float& c) {
  if (!(T > 0.0f) || !(T <= 3.4028234663852886e38f)) return false;
  c = 1.44269504088896340736f / T;
  c = c <= 3.4028234663852886e38f ? c : 3.4028234663852886e38f;
  return true;
}
__device__ __forceinline__ bool row_scale(const SampleArgs& a, int m, float& c) { return scale_of(a.temperature[m], c); }

__device__ __forceinline__ float clamp_uniform(float u) {
  u = u >= 0.0f ? u : 0.0f;                         // NaN -> 0
  return u < 1.0f ? u : __uint_as_float(0x3F7FFFFFu);  // largest float below 1
}

// The first buckets whose inclusive prefix h[] (in LDS) reaches tA and tB
// (both <= h[last]), found by the whole workgroup at once: each thread
// tests its buckets, the one bucket whose interval holds t reports it.
template <int NT>
__device__ __forceinline__ void wg_first_ge(const uint64_t* h, uint64_t tA, uint64_t tB, int* slot, int& bA,
                                            int& bB) {
  __syncthreads();
  for (int b = threadIdx.x; b < kBuckets; b += NT) {
    const uint64_t inc = h[b], exc = b ? h[b - 1] : 0;
    if (inc >= tA && exc < tA) slot[0] = b;
    if (inc >= tB && exc < tB) slot[1] = b;
  }
  __syncthreads();
  bA = slot[0];
  bB = slot[1];
}

// The cut thresholds.  The first, t1, follows from the row mass S; the
// second depends on the mass through the first cut, which lies in bucket
// b1, so its bucket lies in [b2lo, b2hi] (at or before b1).
struct Plan {
  uint64_t t1;
  int b1, b2lo, b2hi;
};

__device__ __forceinline__ uint64_t nucleus_threshold(float top_p, uint64_t S) {
  const double tp = (double)top_p * (double)S;
  const uint64_t t = tp >= (double)S ? S : (uint64_t)ceil(tp);
  return t < 1 ? 1 : t;
}

__device__ __forceinline__ uint64_t draw_threshold(float u, uint64_t nucleus_mass) {
  uint64_t r = (uint64_t)((double)u * (double)nucleus_mass);
  r = r < nucleus_mass ? r : nucleus_mass - 1;
  return r + 1;
}

template <int NT>
__device__ __forceinline__ Plan plan_cuts(const uint64_t* h, float top_p, float u, int* slot) {
  Plan p;
  p.t1 = nucleus_threshold(top_p, h[kBuckets - 1]);
  wg_first_ge<NT>(h, p.t1, p.t1, slot, p.b1, p.b1);
  const uint64_t lo = (p.b1 ? h[p.b1 - 1] : 0) + 1, hi = h[p.b1];
  wg_first_ge<NT>(h, draw_threshold(u, lo), draw_threshold(u, hi), slot, p.b2lo, p.b2hi);
  return p;
}

__device__ __forceinline__ bool planned(const Plan& p, int b) { return b == p.b1 || (b >= p.b2lo && b <= p.b2hi); }

template <int NT>
__device__ __forceinline__ float wg_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix over the workgroup (thread order) and the total.
template <int NT>
__device__ __forceinline__ uint64_t wg_excl_scan(uint64_t x, uint64_t& total, uint64_t* red) {
  const uint64_t inc = wave_incl_scan(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 63) red[w] = inc;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint64_t r = red[i];
    before += i < w ? r : 0;
    tot += r;
  }
  total = tot;
  return before + inc - x;
}

// The maximum of the row's chunk maxima (order-independent, so every
// launch that needs it gets the same value).
template <int NT>
__device__ __forceinline__ float row_max(const SampleArgs& a, int m, float* red) {
  float v = -INFINITY;
  for (int g = threadIdx.x; g < a.G; g += NT) v = fmaxf(v, a.maxp[(int64_t)m * a.G + g]);
  return wg_max<NT>(v, red);
}

// The 16 elements of chunk g a thread of launches 1 to 3 holds: four
// 16-byte groups, 4 * (g * 1024 + j * 256 + t) .. +3 for j = 0..3.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const __amdgpu_buffer_rsrc_t& rs, int64_t N, int g, u32x4_t (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i0 = (int64_t)g * kSampleChunk + (int64_t)(j * kWide + threadIdx.x) * 4;
    if constexpr (VEC) {
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(i0 < N ? (uint32_t)(i0 * 4) : kOutOfRange), 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[j][q] = __builtin_amdgcn_raw_buffer_load_b32(
            rs, (int)(i0 + q < N ? (uint32_t)((i0 + q) * 4) : kOutOfRange), 0, 0);
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const SampleArgs& a, int m) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.logits + (int64_t)m * a.N), (short)0,
                                           (int)(a.N * 4), kBufferWord3);
}

// ---- launch 1: chunk maxima, masses and short lists ----
//
// Each workgroup also sums its chunk's masses relative to the chunk maximum
// z_g (2^-40 fixed point, exact) and lists the elements with
// z >= z_g - kSpecSpan T / log2(e) (mass >= 2^-kSpecSpan of z_g's), up to
// kSpec of them (more: the chunk overflows).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void sample_first_kernel(SampleArgs a) {
  static_assert(kSampleChunk == kThreads * 4, "one 16-byte group of the chunk per thread");
  __shared__ float red[kWaves];
  __shared__ uint64_t red64[kWaves];
  __shared__ uint64_t list[kSpec];
  __shared__ uint32_t nlist;
  const int g = blockIdx.x, m = blockIdx.y;
  const int tid = threadIdx.x;
  for (int e = g * kThreads + tid; e < kBuckets; e += a.G * kThreads) {
    a.hist[(int64_t)m * kBuckets + e] = 0;
    a.hcnt[(int64_t)m * kBuckets + e] = 0;
  }
  const float T = a.temperature[m];  // issued with the chunk's loads
  if (g == 0 && tid == 0) a.lcount[m] = 0;
  if (tid == 0) nlist = 0;
  // elements i0 .. i0 + 3 of the row
  const int64_t i0 = (int64_t)g * kSampleChunk + (int64_t)tid * 4;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(a, m);
  u32x4_t v;
  if constexpr (VEC) {
    v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(i0 < a.N ? (uint32_t)(i0 * 4) : kOutOfRange), 0, 0);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(i0 + q < a.N ? (uint32_t)((i0 + q) * 4) : kOutOfRange),
                                                  0, 0);
  }
  float zm = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) zm = i0 + q < a.N ? fmaxf(zm, __uint_as_float(v[q])) : zm;
  zm = wg_max<kThreads>(zm, red);  // barrier: nlist is set
  const int64_t cg = (int64_t)m * a.G + g;
  if (tid == 0) a.maxp[cg] = zm;
  float c;
  if (!scale_of(T, c) || a.G > kSpecMaxChunks) return;
  const float thr = zm - kSpecSpan / c;
  uint64_t s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = i0 + q;
    const bool valid = i < a.N;
    const float z = __uint_as_float(v[q]);
    s += valid ? fixed_mass((zm - z) * c) : 0;
    const bool want = valid && z >= thr;
    const uint64_t mask = __ballot(want);
    if (mask == 0) continue;
    const int lane = tid & 63;
    const int lead = __ffsll((unsigned long long)mask) - 1;
    uint32_t slot0 = 0;
    if (lane == lead) slot0 = atomicAdd(&nlist, (uint32_t)__popcll(mask));
    slot0 = __shfl(slot0, lead, 64);
    const uint32_t slot = slot0 + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (want && slot < (uint32_t)kSpec) list[slot] = ((uint64_t)v[q] << 32) | (uint64_t)(uint32_t)i;
  }
  uint64_t tot;
  (void)wg_excl_scan<kThreads>(s, tot, red64);  // barrier: every append has landed
  const uint32_t n = nlist;
  if (tid < kSpec && (uint32_t)tid < n) a.cand[cg * kSpec + tid] = list[tid];
  if (tid == 0)
    a.crec[cg] = u32x4_t{__float_as_uint(zm), n > (uint32_t)kSpec ? kSpecOverflow : n, (uint32_t)tot,
                         (uint32_t)(tot >> 32)};
}

// ---- the listed path, at the start of launch 2 ----
//
// Every element at or above z_g - kSpecSpan T / log2(e) of a chunk that did
// not overflow is listed, so with theta the largest of
// (overflowed ? z_g : z_g - kSpecSpan T / log2(e)) over the chunks, the
// lists hold every element of the row above theta: a prefix of the order.
// With the row mass S = sum_g S_g 2^((z_g - z_max) log2(e) / T) (a fixed
// summation order), when that prefix's mass reaches the nucleus threshold
// both cuts lie in it and are found by ranking it.  Every workgroup of the
// row computes the same result from launch 1's records; workgroup 0 writes
// the token.  Returns whether the row was drawn, and the row maximum.
__device__ __forceinline__ bool resolve_listed(const SampleArgs& a, int m, bool valid, float c, float u, bool writer,
                                               float& zmax) {
  __shared__ float szg[kSpecMaxChunks], sth[kSpecMaxChunks];
  __shared__ uint32_t sn[kSpecMaxChunks];
  __shared__ double sterm[kSpecMaxChunks];
  __shared__ uint64_t ck[kCap], cm[kCap];
  __shared__ uint32_t ncand;
  __shared__ uint64_t cut_cum;
  __shared__ int64_t cut_rank, cut_index;
  static_assert(kCap == kWide && kSpecMaxChunks == kWide, "one chunk record and one listed element per thread");
  const int tid = threadIdx.x;
  const int G = a.G;
  const int64_t row0 = (int64_t)m * G;
  // one round trip: the chunk records (thread g holds chunk g) and the
  // first listed slots
  const bool has = tid < G;
  const u32x4_t rec = has ? a.crec[row0 + tid] : u32x4_t{0xFF800000u, 0u, 0u, 0u};
  const float zg = __uint_as_float(rec[0]);
  const uint32_t ng = rec[1];
  const uint64_t sg = ((uint64_t)rec[3] << 32) | rec[2];
  const int64_t nslots = (int64_t)G * kSpec;
  uint64_t pre[kSpecPre];
#pragma unroll
  for (int k = 0; k < kSpecPre; ++k) {
    const int64_t sl = tid + (int64_t)k * kWide;
    pre[k] = sl < nslots ? a.cand[row0 * kSpec + sl] : 0;
  }
  if (has) {
    szg[tid] = zg;
    sn[tid] = ng;
  }
  if (tid == 0) ncand = 0;
  __syncthreads();
  // every thread reads the G records in chunk order: the row maximum, then
  // each chunk's mass rescaled to it and its listing level; the sum and the
  // level theta are taken in chunk order, so every thread (and every
  // workgroup of the row) gets the same values
  float zmx = -INFINITY;
#pragma unroll 8
  for (int g = 0; g < G; ++g) zmx = fmaxf(zmx, szg[g]);
  zmax = zmx;
  if (!valid) return false;  // no usable temperature: launch 1 listed nothing
  const float span = kSpecSpan / c;
  if (has) {
    sterm[tid] = (double)sg * (double)exp2f(-((zmx - zg) * c));
    sth[tid] = ng == kSpecOverflow ? zg : zg - span;
  }
  __syncthreads();
  double S = 0.0;
  float th = -INFINITY;
#pragma unroll 8
  for (int g = 0; g < G; ++g) {
    S += sterm[g];
    th = fmaxf(th, sth[g]);
  }
  // the listed elements above theta, with their masses relative to z_max
  auto take = [&](int64_t sl, uint64_t e) {
    const int g = (int)(sl / kSpec), j = (int)(sl % kSpec);
    const uint32_t n = sl < nslots ? sn[g] : 0u;
    const float z = __uint_as_float((uint32_t)(e >> 32));
    const bool want = (uint32_t)j < (n < (uint32_t)kSpec ? n : (uint32_t)kSpec) && z > th;
    const uint64_t mask = __ballot(want);
    if (mask == 0) return;
    const int lane = tid & 63;
    const int lead = __ffsll((unsigned long long)mask) - 1;
    uint32_t slot0 = 0;
    if (lane == lead) slot0 = atomicAdd(&ncand, (uint32_t)__popcll(mask));
    slot0 = __shfl(slot0, lead, 64);
    const uint32_t slot = slot0 + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (want && slot < (uint32_t)kCap) {
      ck[slot] = ((uint64_t)order_key(z) << 32) | (e & 0xFFFFFFFFull);
      cm[slot] = fixed_mass((zmx - z) * c);
    }
  };
#pragma unroll
  for (int k = 0; k < kSpecPre; ++k) take(tid + (int64_t)k * kWide, pre[k]);
  for (int64_t base = (int64_t)kSpecPre * kWide; base < nslots; base += kWide) {  // G > 64 only
    const int64_t sl = base + tid;
    take(sl, sl < nslots ? a.cand[row0 * kSpec + sl] : 0);
  }
  __syncthreads();
  const uint32_t cnt = ncand;
  if (cnt > (uint32_t)kCap || !(S >= 1.0)) return false;
  // each thread ranks its element against all of them (and sums them all)
  const bool mine = tid < (int)cnt;
  const uint64_t key = mine ? ck[tid] : ~0ull, mm = mine ? cm[tid] : 0;
  uint64_t pre_m = 0, nbf = 0, total = 0;
#pragma unroll 8
  for (uint32_t j = 0; j < cnt; ++j) {
    const uint64_t kj = ck[j], mj = cm[j];
    const bool earlier = kj < key;
    pre_m += earlier ? mj : 0;
    nbf += earlier;
    total += mj;
  }
  const uint64_t S64 = S < 1.8446744073709552e19 ? (uint64_t)S : ~0ull;
  const uint64_t t1 = nucleus_threshold(a.top_p, S64);
  if (total < t1) return false;
  if (mine && pre_m < t1 && pre_m + mm >= t1) {
    cut_cum = pre_m + mm;
    cut_rank = (int64_t)nbf;
  }
  __syncthreads();
  const uint64_t t2 = draw_threshold(u, cut_cum);
  if (mine && pre_m < t2 && pre_m + mm >= t2) cut_index = (int64_t)(uint32_t)key;
  __syncthreads();
  if (writer && tid == 0) {
    a.tokens[m] = (int32_t)cut_index;
    if (a.nucleus) a.nucleus[m] = (int32_t)(cut_rank + 1);
    a.resolved[m] = 1u;
  }
  return true;
}

// ---- launch 2: bucket of every element, mass histogram ----
template <bool VEC>
__global__ __launch_bounds__(kWide) void sample_hist_kernel(SampleArgs a) {
  __shared__ unsigned long long lh[kBuckets];
  __shared__ uint32_t lc[kBuckets];
  __shared__ float redf[kWide / 64];
  __shared__ uint64_t red64[kWide / 64];
  const int g = blockIdx.x, m = blockIdx.y;
  // every load the row needs is issued before the first branch on them
  const float T = a.temperature[m];
  const float u = clamp_uniform(a.uniforms[m]);
  u32x4_t v[4];
  load_chunk<VEC>(row_rsrc(a, m), a.N, g, v);
  float c;
  const bool valid = scale_of(T, c);
  float zm;
  if (a.G <= kSpecMaxChunks) {
    if (resolve_listed(a, m, valid, c, u, g == 0, zm)) return;
  } else {
    zm = row_max<kWide>(a, m, redf);
  }
  if (g == 0 && threadIdx.x == 0) a.resolved[m] = 0u;
  if (!valid) return;
  for (int e = threadIdx.x; e < kBuckets; e += kWide) {
    lh[e] = 0;
    lc[e] = 0;
  }
  __syncthreads();
  uint64_t tail = 0;  // the last bucket (negligible masses, often most of the row) in registers
  uint32_t ntail = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i0 = (int64_t)g * kSampleChunk + (int64_t)(j * kWide + threadIdx.x) * 4;
    u16x4_t ids;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool valid = i0 + q < a.N;
      const float x = (zm - __uint_as_float(v[j][q])) * c;
      const int b = bucket_of(x);
      const uint64_t mm = valid ? fixed_mass(x) : 0;
      if (b == kBuckets - 1) {
        tail += mm;
        ntail += valid;
      } else if (valid) {
        atomicAdd(&lh[b], (unsigned long long)mm);
        atomicAdd(&lc[b], 1u);
      }
      ids[q] = (uint16_t)b;
    }
    // i0 < N and i0 % 4 == 0, so the four ids lie inside the row's bstride
    if (i0 < a.N) *reinterpret_cast<u16x4_t*>(a.bid + (int64_t)m * a.bstride + i0) = ids;
  }
  uint64_t tsum, tcnt;
  (void)wg_excl_scan<kWide>(tail, tsum, red64);  // barrier: every LDS add has landed
  (void)wg_excl_scan<kWide>(ntail, tcnt, red64);
  if (threadIdx.x == 0) {
    lh[kBuckets - 1] += tsum;
    lc[kBuckets - 1] += (uint32_t)tcnt;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kBuckets; e += kWide) {
    if (lc[e]) {
      atomicAdd(&a.hist[(int64_t)m * kBuckets + e], lh[e]);
      atomicAdd(&a.hcnt[(int64_t)m * kBuckets + e], lc[e]);
    }
  }
}

// ---- launch 3: collect the elements of the buckets the cuts can fall in ----
template <bool VEC>
__global__ __launch_bounds__(kWide) void sample_collect_kernel(SampleArgs a) {
  __shared__ uint64_t h[kBuckets];
  // this workgroup's elements of the planned buckets, gathered in LDS and
  // published with one device-scope atomic (one per wave step contended on
  // the row's counter across the XCDs)
  __shared__ uint64_t gkey[kWGList], gmass[kWGList];
  __shared__ uint32_t gbkt[kWGList];
  __shared__ uint32_t gn, gbase;
  __shared__ float redf[kWide / 64];
  __shared__ uint64_t red64[kWide / 64];
  __shared__ int slot[2];
  const int g = blockIdx.x, m = blockIdx.y;
  float c;
  if (a.resolved[m] || !row_scale(a, m, c)) return;
  if (threadIdx.x == 0) gn = 0;  // ordered before its first use by the scans' barriers
  u32x4_t v[4];
  load_chunk<VEC>(row_rsrc(a, m), a.N, g, v);
  u16x4_t ids[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i0 = (int64_t)g * kSampleChunk + (int64_t)(j * kWide + threadIdx.x) * 4;
    if (i0 < a.N) ids[j] = *reinterpret_cast<const u16x4_t*>(a.bid + (int64_t)m * a.bstride + i0);
  }
  constexpr int kPer = kBuckets / kWide;  // buckets per thread
  uint64_t x[kPer], s = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) x[k] = a.hist[(int64_t)m * kBuckets + kPer * threadIdx.x + k];
  const float zm = row_max<kWide>(a, m, redf);
  {  // inclusive prefix of the row histogram
#pragma unroll
    for (int k = 0; k < kPer; ++k) s += x[k];
    uint64_t tot;
    uint64_t run = wg_excl_scan<kWide>(s, tot, red64);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      run += x[k];
      h[kPer * threadIdx.x + k] = run;
    }
  }
  __syncthreads();
  if (h[kBuckets - 1] == 0) return;
  const Plan pl = plan_cuts<kWide>(h, a.top_p, clamp_uniform(a.uniforms[m]), slot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i0 = (int64_t)g * kSampleChunk + (int64_t)(j * kWide + threadIdx.x) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q;
      const int b = i0 < a.N ? (int)ids[j][q] : 0;
      const bool want = i < a.N && planned(pl, b);
      const uint64_t mask = __ballot(want);
      if (mask == 0) continue;
      const int lane = threadIdx.x & 63;
      const int lead = __ffsll((unsigned long long)mask) - 1;
      uint32_t slot0 = 0;
      if (lane == lead) slot0 = atomicAdd(&gn, (uint32_t)__popcll(mask));
      slot0 = __shfl(slot0, lead, 64);
      const uint32_t slot = slot0 + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
      if (want && slot < (uint32_t)kWGList) {
        const float z = __uint_as_float(v[j][q]);
        gkey[slot] = ((uint64_t)order_key(z) << 32) | (uint64_t)(uint32_t)i;
        gmass[slot] = fixed_mass((zm - z) * c);
        gbkt[slot] = (uint32_t)b;
      }
    }
  }
  __syncthreads();
  const uint32_t n = gn;
  if (n == 0) return;
  // more than this workgroup could gather: push the row's count past the
  // list so that the selection takes the passes over the row
  if (threadIdx.x == 0) gbase = atomicAdd(&a.lcount[m], n <= (uint32_t)kWGList ? n : (uint32_t)kList + 1u);
  __syncthreads();
  if (n > (uint32_t)kWGList) return;
  for (uint32_t e = threadIdx.x; e < n; e += kWide) {
    const uint32_t slot = gbase + e;
    if (slot < (uint32_t)kList) {
      const int64_t o = (int64_t)m * kList + slot;
      a.lkey[o] = gkey[e];
      a.lmass[o] = gmass[e];
      a.lbkt[o] = gbkt[e];
    }
  }
}

// ---- launch 4: the two cut points, one workgroup per row ----
struct Smem {
  uint64_t h0[kBuckets];  // inclusive prefix of the row's histogram
  uint32_t c0[kBuckets];  // inclusive prefix of the row's bucket counts
  uint64_t hs[kSub];      // refinement: mass per sub-bucket
  uint32_t cs[kSub];      // refinement: count per sub-bucket
  uint64_t ckey[kCap];    // candidates: key << 32 | index
  uint64_t cmass[kCap];
  uint64_t lk[kList];     // launch 3's list (keys, masses), copied once
  uint64_t lm[kList];
  uint32_t sel[kList];    // a cut's bucket: positions of its elements in the list
  uint64_t red64[kWaves];
  float redf[kWaves];
  uint32_t ncand;
  int slot[2];
  int pick;
  uint64_t pick_before;
  uint32_t pick_nb, pick_cnt;
  uint64_t kmin, kmax;
  int64_t sel_index, sel_rank;
  uint64_t sel_cum;
};

struct Cut {
  int64_t index, rank;  // the element and how many come before it in the order
  uint64_t cum;         // inclusive cumulative mass through it
};

// Whether one of the eight 16-bit ids in v equals b (ids < 2^15): a half of
// v ^ (b, b) is zero exactly when (half - 1) borrows into its top bit while
// the half itself has that bit clear.
__device__ __forceinline__ bool has_id(const u32x4_t& v, uint32_t b) {
  const uint32_t pat = b | (b << 16);
  uint32_t hit = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = v[k] ^ pat;
    hit |= (x - 0x00010001u) & ~x & 0x80008000u;
  }
  return hit != 0;
}

__device__ __forceinline__ int id_of(const u32x4_t& v, int q) { return (int)((v[q >> 1] >> (16 * (q & 1))) & 0xFFFFu); }

// The cut among cnt <= kCap candidates in sm.ckey / sm.cmass, the whole set
// of elements ordered after `nb` elements of mass `before`: each candidate
// sums the masses ordered before it, and the one whose interval holds t is
// the cut.
// Four neighbouring lanes share a candidate, each summing every fourth one.
__device__ __forceinline__ Cut rank_candidates(uint64_t t, uint64_t before, uint64_t nb, uint32_t cnt, Smem& sm) {
  static_assert(kCap * 4 == kThreads, "four lanes per candidate");
  const int tid = threadIdx.x;
  const int ci = tid >> 2, part = tid & 3;
  const bool mine = ci < (int)cnt;
  const uint64_t k = mine ? sm.ckey[ci] : 0, mm = mine ? sm.cmass[ci] : 0;
  uint64_t pre = 0;
  uint32_t nbf = 0;
  if (mine) {
#pragma unroll 4
    for (int j = part; j < (int)cnt; j += 4) {
      const bool earlier = sm.ckey[j] < k;
      pre += earlier ? sm.cmass[j] : 0;
      nbf += earlier;
    }
  }
  pre += __shfl_xor(pre, 1, 64);
  pre += __shfl_xor(pre, 2, 64);
  nbf += __shfl_xor(nbf, 1, 64);
  nbf += __shfl_xor(nbf, 2, 64);
  if (mine && part == 0 && before + pre < t && before + pre + mm >= t) {
    sm.sel_index = (int64_t)(uint32_t)k;
    sm.sel_rank = (int64_t)(nb + nbf);
    sm.sel_cum = before + pre + mm;
  }
  __syncthreads();
  return Cut{sm.sel_index, sm.sel_rank, sm.sel_cum};
}

// The cut among the cnt elements of one bucket, list entries sm.sel[0..cnt)
// of sm.lk / sm.lm (all of the bucket's elements, ordered after nb elements
// of mass `before`).
// The composite keys (order key << 32 | index) are unique, so narrowing by
// up to 10 key bits at a time, just below the active keys' highest
// differing bit (mass and count per sub-bucket, the sub-bucket whose
// interval holds t), reaches at most kCap elements, which rank_candidates
// ranks directly.  Everything stays in LDS.
__device__ __forceinline__ Cut rank_listed(uint64_t t, uint64_t before, uint64_t nb, uint32_t cnt, Smem& sm) {
  const int tid = threadIdx.x;
  static_assert(kSub == kThreads, "one sub-bucket per thread");
  // the active elements: (key >> sh) == prefix (all of them while sh == 64)
  uint64_t prefix = 0;
  int sh = 64;
  uint32_t act = cnt;
  auto active = [&](uint64_t k) { return sh == 64 || (k >> sh) == prefix; };
  while (act > (uint32_t)kCap) {
    // the active keys' range: the window starts below their highest
    // differing bit, so every level splits the set (keys of one bucket share
    // many leading bits)
    uint64_t lo = ~0ull, hi = 0;
    for (uint32_t i = tid; i < cnt; i += kThreads) {
      const uint64_t k = sm.lk[sm.sel[i]];
      if (active(k)) {
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t lo2 = __shfl_xor(lo, o, 64), hi2 = __shfl_xor(hi, o, 64);
      lo = lo2 < lo ? lo2 : lo;
      hi = hi2 > hi ? hi2 : hi;
    }
    __syncthreads();
    if (tid == 0) {
      sm.kmin = ~0ull;
      sm.kmax = 0;
    }
    __syncthreads();
    if ((tid & 63) == 0) {
      atomicMin((unsigned long long*)&sm.kmin, (unsigned long long)lo);
      atomicMax((unsigned long long*)&sm.kmax, (unsigned long long)hi);
    }
    __syncthreads();
    const uint64_t d = sm.kmin ^ sm.kmax;  // != 0: more than one (unique) key is active
    const int top = 63 - __clzll((long long)d);  // highest differing bit
    const int shn = top + 1 > kSubBits ? top + 1 - kSubBits : 0;
    const int w = top + 1 - shn;
    const uint64_t base = top + 1 >= 64 ? 0 : sm.kmin >> (top + 1);  // bits every active key shares
    sm.hs[tid] = 0;
    sm.cs[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < cnt; i += kThreads) {
      const uint32_t e = sm.sel[i];
      const uint64_t k = sm.lk[e];
      if (active(k)) {
        const int sub = (int)((k >> shn) & (uint64_t)((1u << w) - 1u));
        atomicAdd((unsigned long long*)&sm.hs[sub], (unsigned long long)sm.lm[e]);
        atomicAdd(&sm.cs[sub], 1u);
      }
    }
    __syncthreads();
    uint64_t tot, totn;
    const uint64_t hm = sm.hs[tid], hc = sm.cs[tid];
    const uint64_t ex = wg_excl_scan<kThreads>(hm, tot, sm.red64);
    const uint64_t exn = wg_excl_scan<kThreads>(hc, totn, sm.red64);
    if (before + ex < t && before + ex + hm >= t) {
      sm.pick = tid;
      sm.pick_before = before + ex;
      sm.pick_nb = (uint32_t)exn;
      sm.pick_cnt = (uint32_t)hc;
    }
    __syncthreads();
    prefix = (base << w) | (uint64_t)sm.pick;
    sh = shn;
    before = sm.pick_before;
    nb += sm.pick_nb;
    act = sm.pick_cnt;
  }
  // the active elements (at most kCap) into the directly ranked set
  __syncthreads();
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  for (uint32_t i = tid; i < cnt; i += kThreads) {
    const uint32_t e = sm.sel[i];
    const uint64_t k = sm.lk[e];
    if (active(k)) {
      const uint32_t slot = atomicAdd(&sm.ncand, 1u);
      sm.ckey[slot] = k;  // slot < act <= kCap
      sm.cmass[slot] = sm.lm[e];
    }
  }
  __syncthreads();
  return rank_candidates(t, before, nb, act, sm);
}

// Visit the row's bucket ids eight at a time: f(base, v) for the 16-byte
// group of ids base .. base + 7 (ids past N read as zero and must be masked
// by the caller); the waves stay converged.
template <typename F>
__device__ __forceinline__ void id_pass(const __amdgpu_buffer_rsrc_t& rb, int64_t N, F&& f) {
  const int64_t per = (int64_t)kThreads * 8;
  const int64_t iters = (N + per - 1) / per;
  for (int64_t k0 = 0; k0 < iters; k0 += kBatch) {
    u32x4_t v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t base = ((k0 + j) * kThreads + threadIdx.x) * 8;
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(base < N ? (uint32_t)(base * 2) : kOutOfRange), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) f(((k0 + j) * kThreads + threadIdx.x) * 8, v[j]);
  }
}

__device__ __forceinline__ Cut select_cut(uint64_t t, const __amdgpu_buffer_rsrc_t& rs,
                                                    const __amdgpu_buffer_rsrc_t& rb, int64_t N, float zmax,
                                                    float c, Smem& sm) {
  const int tid = threadIdx.x;
  // level 0: the bucket whose inclusive prefix first reaches t (one exists:
  // 1 <= t <= the row's mass)
  __syncthreads();
  if (tid == 0) sm.pick = 0;
  __syncthreads();
  for (int b = tid; b < kBuckets; b += kThreads) {
    const uint64_t inc = sm.h0[b], exc = b ? sm.h0[b - 1] : 0;
    if (inc >= t && exc < t) sm.pick = b;
  }
  __syncthreads();
  const int b0 = sm.pick;
  uint64_t before = b0 ? sm.h0[b0 - 1] : 0;  // mass ordered before the candidate set
  const uint64_t nb0 = b0 ? sm.c0[b0 - 1] : 0;  // elements in the buckets before b0
  uint64_t prefix = 0;                        // the candidates' key >> sh
  int sh = 32;
  for (;;) {
    const int w = sh < kSubBits ? sh : kSubBits;  // bits histogrammed in this pass
    __syncthreads();
    if (tid == 0) sm.ncand = 0;
    sm.hs[tid] = 0;
    sm.cs[tid] = 0;
    __syncthreads();
    uint32_t nbefore = 0;  // elements of bucket b0 ordered before the candidate set
    id_pass(rb, N, [&](int64_t base, const u32x4_t& v) {
      if (__ballot(base < N && has_id(v, (uint32_t)b0)) == 0) return;  // wave-uniform: nothing of b0 here
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t i = base + q;
        const bool inb = i < N && id_of(v, q) == b0;
        if (__ballot(inb) == 0) continue;
        const float z =
            inb ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(uint32_t)(i * 4), 0, 0)) : 0.0f;
        const uint64_t key = order_key(z);
        const uint64_t kp = sh >= 32 ? 0 : key >> sh;
        nbefore += inb && kp < prefix;
        const bool cand = inb && kp == prefix;
        // wave-aggregated append (the wave is converged here)
        const uint64_t mask = __ballot(cand);
        if (mask == 0) continue;
        const int lead = __ffsll((unsigned long long)mask) - 1;
        uint32_t slot0 = 0;
        if ((tid & 63) == lead) slot0 = atomicAdd(&sm.ncand, (uint32_t)__popcll(mask));
        slot0 = __shfl(slot0, lead, 64);
        if (cand) {
          const uint32_t slot = slot0 + (uint32_t)__popcll(mask & ((1ull << (tid & 63)) - 1ull));
          const uint64_t mm = fixed_mass((zmax - z) * c);
          if (slot < (uint32_t)kCap) {
            sm.ckey[slot] = (key << 32) | (uint64_t)(uint32_t)i;
            sm.cmass[slot] = mm;
          }
          if (w > 0) {
            const int sub = (int)((key >> (sh - w)) & (uint64_t)((1u << w) - 1u));
            atomicAdd((unsigned long long*)&sm.hs[sub], (unsigned long long)mm);
            atomicAdd(&sm.cs[sub], 1u);
          }
        }
      }
    });
    uint64_t nb;
    (void)wg_excl_scan<kThreads>(nbefore, nb, sm.red64);  // barrier: every append has landed
    nb += nb0;
    const uint32_t cnt = sm.ncand;
    if (cnt <= (uint32_t)kCap) return rank_candidates(t, before, nb, cnt, sm);
    if (w == 0) {
      // every candidate has the same logit, hence the same mass: the cut is
      // the j-th of them in index order
      const uint64_t mt = sm.cmass[0];  // > 0: the set holds mass t - before > 0
      const uint64_t j = mt ? (t - before + mt - 1) / mt - 1 : 0;
      uint64_t seen = 0;
      const int64_t per = (int64_t)kThreads * 8;
      for (int64_t k0 = 0; k0 * per < N; ++k0) {
        const int64_t base = k0 * per + (int64_t)tid * 8;
        const u32x4_t v =
            __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(base < N ? (uint32_t)(base * 2) : kOutOfRange), 0, 0);
        uint32_t match = 0, nm = 0;
        const bool any = base < N && has_id(v, (uint32_t)b0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          bool hit = false;
          if (any && base + q < N && id_of(v, q) == b0) {
            const float z =
                __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)(uint32_t)((base + q) * 4), 0, 0));
            hit = (uint64_t)order_key(z) == prefix;
          }
          match |= (uint32_t)hit << q;
          nm += hit;
        }
        uint64_t chunk;
        const uint64_t ex = wg_excl_scan<kThreads>(nm, chunk, sm.red64);
        if (seen + ex <= j && j < seen + ex + nm) {
          uint64_t r = j - seen - ex;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if ((match >> q) & 1u) {
              if (r == 0) sm.sel_index = base + q;
              r -= 1;
            }
          }
        }
        seen += chunk;
        if (seen > j) break;
      }
      __syncthreads();
      return Cut{sm.sel_index, (int64_t)(nb + j), before + (j + 1) * mt};
    }
    // narrow to the sub-bucket whose inclusive prefix first reaches t
    uint64_t tot;
    const uint64_t ex = wg_excl_scan<kThreads>(sm.hs[tid], tot, sm.red64);
    if (before + ex < t && before + ex + sm.hs[tid] >= t) {
      sm.pick = tid;
      sm.pick_before = before + ex;
    }
    __syncthreads();
    prefix = (prefix << w) | (uint64_t)sm.pick;
    before = sm.pick_before;
    sh -= w;
  }
}

__global__ __launch_bounds__(kThreads) void sample_select_kernel(SampleArgs a) {
  __shared__ Smem sm;
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  if (a.resolved[m]) return;
  // every input of the row is loaded up front (one round trip): the
  // histograms, this thread's list entry and the chunk maxima
  const uint64_t x0 = a.hist[(int64_t)m * kBuckets + 2 * tid], x1 = a.hist[(int64_t)m * kBuckets + 2 * tid + 1];
  const uint32_t n0 = a.hcnt[(int64_t)m * kBuckets + 2 * tid], n1 = a.hcnt[(int64_t)m * kBuckets + 2 * tid + 1];
  const uint32_t listed = a.lcount[m];
  static_assert(kList % kThreads == 0, "whole list entries per thread");
  // the list: buckets stay in registers, keys and masses go to LDS (written
  // below, once the loads have landed).  The first kThreads entries come
  // with the other loads; the rest only when the list is that long
  uint32_t my_bkt[kListPer];
  uint64_t my_key[kListPer], my_mass[kListPer];
  {
    const int64_t o = (int64_t)m * kList + tid;
    my_bkt[0] = a.lbkt[o];
    my_key[0] = a.lkey[o];
    my_mass[0] = a.lmass[o];
  }
  float c;
  const float u = clamp_uniform(a.uniforms[m]);
  const float zm = row_max<kThreads>(a, m, sm.redf);
  if (!row_scale(a, m, c)) {
    if (tid == 0) {
      a.tokens[m] = -1;
      if (a.nucleus) a.nucleus[m] = 0;
    }
    return;
  }
  {
    uint64_t total;
    const uint64_t ex = wg_excl_scan<kThreads>(x0 + x1, total, sm.red64);
    const uint64_t exn = wg_excl_scan<kThreads>(n0 + n1, total, sm.red64);
    sm.h0[2 * tid] = ex + x0;
    sm.h0[2 * tid + 1] = ex + x0 + x1;
    sm.c0[2 * tid] = (uint32_t)(exn + n0);
    sm.c0[2 * tid + 1] = (uint32_t)(exn + n0 + n1);
  }
  sm.lk[tid] = my_key[0];
  sm.lm[tid] = my_mass[0];
  const int nlist = listed < (uint32_t)kList ? (int)listed : kList;
#pragma unroll
  for (int e = 1; e < kListPer; ++e) {
    my_bkt[e] = 0xFFFFFFFFu;  // no bucket
    if (e * kThreads < nlist) {  // uniform
      const int64_t o = (int64_t)m * kList + tid + e * kThreads;
      my_bkt[e] = a.lbkt[o];
      sm.lk[tid + e * kThreads] = a.lkey[o];
      sm.lm[tid + e * kThreads] = a.lmass[o];
    }
  }
  __syncthreads();
  const uint64_t S = sm.h0[kBuckets - 1];
  if (S == 0) {  // no finite maximum
    if (tid == 0) {
      a.tokens[m] = -1;
      if (a.nucleus) a.nucleus[m] = 0;
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(a, m);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      a.bid + (int64_t)m * a.bstride, (short)0, (int)(a.bstride * 2), kBufferWord3);
  // cut 0, the nucleus: the first element whose cumulative mass reaches
  // top_p * S; cut 1, the draw: the first element whose cumulative mass
  // exceeds u * (nucleus mass).  A cut in a bucket that launch 3 collected
  // whole is found among that list in LDS; any other (the list overflowed)
  // takes the passes over the row.  One loop, so each path is inlined once.
  const Plan pl = plan_cuts<kThreads>(sm.h0, a.top_p, u, sm.slot);
  uint64_t t = pl.t1;
  int64_t nucleus_size = 0;
  for (int k = 0; k < 2; ++k) {
    int b = pl.b1;
    if (k == 1) wg_first_ge<kThreads>(sm.h0, t, t, sm.slot, b, b);
    bool ranked = false;
    Cut cut{0, 0, 0};
    if (listed <= (uint32_t)kList && planned(pl, b)) {
      __syncthreads();
      if (tid == 0) sm.ncand = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kListPer; ++e) {
        if ((uint32_t)(tid + e * kThreads) < listed && my_bkt[e] == (uint32_t)b) {
          const uint32_t slot = atomicAdd(&sm.ncand, 1u);  // < listed <= kList
          sm.sel[slot] = (uint32_t)(tid + e * kThreads);
        }
      }
      __syncthreads();
      const uint32_t cnt = sm.ncand;
      const uint32_t in_b = sm.c0[b] - (b ? sm.c0[b - 1] : 0u);
      if (cnt == in_b) {  // the whole bucket is in the list
        cut = rank_listed(t, b ? sm.h0[b - 1] : 0, b ? sm.c0[b - 1] : 0, cnt, sm);
        ranked = true;
      }
    }
    if (!ranked) cut = select_cut(t, rs, rb, a.N, zm, c, sm);
    if (k == 0) {
      nucleus_size = cut.rank + 1;
      t = draw_threshold(u, cut.cum);
    } else if (tid == 0) {
      a.tokens[m] = (int32_t)cut.index;
      if (a.nucleus) a.nucleus[m] = (int32_t)nucleus_size;
    }
  }
}

struct SampleLayout {
  int64_t G, bstride, maxp_off, hist_off, hcnt_off, bid_off, lcount_off, lkey_off, lmass_off, lbkt_off, crec_off,
      cand_off, resolved_off, bytes;
};

SampleLayout sample_layout(int M, int64_t N) {
  auto al = [](int64_t b) { return (b + 255) / 256 * 256; };
  SampleLayout L;
  L.G = (N + kSampleChunk - 1) / kSampleChunk;
  L.bstride = (N + 7) / 8 * 8;
  L.maxp_off = 0;
  L.hist_off = al((int64_t)M * L.G * 4);
  L.hcnt_off = L.hist_off + al((int64_t)M * kBuckets * 8);
  L.bid_off = L.hcnt_off + al((int64_t)M * kBuckets * 4);
  L.lcount_off = L.bid_off + al((int64_t)M * L.bstride * 2);
  L.lkey_off = L.lcount_off + al((int64_t)M * 4);
  L.lmass_off = L.lkey_off + al((int64_t)M * kList * 8);
  L.lbkt_off = L.lmass_off + al((int64_t)M * kList * 8);
  L.crec_off = L.lbkt_off + al((int64_t)M * kList * 4);
  L.cand_off = L.crec_off + al((int64_t)M * L.G * 16);
  L.resolved_off = L.cand_off + al((int64_t)M * L.G * kSpec * 8);
  L.bytes = L.resolved_off + al((int64_t)M * 4);
  return L;
}

}  // namespace

size_t sample_workspace_bytes(int M, int64_t N) { return (size_t)sample_layout(M, N).bytes; }

hipError_t launch_sample_top_p(int M, int64_t N, const float* logits, const float* temperature, float top_p,
                               const float* uniforms, int32_t* tokens, int32_t* nucleus, void* ws,
                               hipStream_t stream) {
  const SampleLayout L = sample_layout(M, N);
  char* w = static_cast<char*>(ws);
  const SampleArgs a{N, L.bstride, (int)L.G, logits, temperature, uniforms, tokens, nucleus, top_p,
                     reinterpret_cast<float*>(w + L.maxp_off), reinterpret_cast<unsigned long long*>(w + L.hist_off),
                     reinterpret_cast<uint32_t*>(w + L.hcnt_off), reinterpret_cast<uint16_t*>(w + L.bid_off),
                     reinterpret_cast<uint32_t*>(w + L.lcount_off), reinterpret_cast<uint64_t*>(w + L.lkey_off),
                     reinterpret_cast<uint64_t*>(w + L.lmass_off), reinterpret_cast<uint32_t*>(w + L.lbkt_off),
                     reinterpret_cast<u32x4_t*>(w + L.crec_off),
                     reinterpret_cast<uint64_t*>(w + L.cand_off), reinterpret_cast<uint32_t*>(w + L.resolved_off)};
  const bool vec = N % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
  const dim3 wide((unsigned)L.G, (unsigned)M);
  if (vec) {
    hipLaunchKernelGGL(sample_first_kernel<true>, wide, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(sample_hist_kernel<true>, wide, dim3(kWide), 0, stream, a);
    hipLaunchKernelGGL(sample_collect_kernel<true>, wide, dim3(kWide), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sample_first_kernel<false>, wide, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(sample_hist_kernel<false>, wide, dim3(kWide), 0, stream, a);
    hipLaunchKernelGGL(sample_collect_kernel<false>, wide, dim3(kWide), 0, stream, a);
  }
  hipLaunchKernelGGL(sample_select_kernel, dim3((unsigned)M), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
