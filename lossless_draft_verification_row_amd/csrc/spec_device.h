// spec_device.h -- device helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;        // one workgroup = 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 4096;         // sampler chunk; also the streaming slice of one workgroup
constexpr int kGroup = 64;           // sampler group inside a chunk
constexpr int kPerThread = kChunk / kThreads;  // 16 logits of one row per thread per slice

constexpr int kDtF32 = 0;
constexpr int kDtBF16 = 1;

constexpr int kStNonfinite = 1;
constexpr int kStBadToken = 2;
constexpr int kStZeroQ = 4;
constexpr int kStResidualEmpty = 8;
constexpr int kStFilterOverflow = 32;
constexpr int kStBadGamma = 64;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element access

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

template <int DT>
__device__ __forceinline__ float logit_at(const void* row, int x) {
  if constexpr (DT == kDtBF16) return bf16_at((const uint16_t*)row + x);
  else return ((const float*)row)[x];
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t ld, int64_t r) {
  return (const char*)base + r * ld * (DT == kDtBF16 ? 2 : 4);
}

// Element index of register j of thread t in the slice starting at `base`: 16-byte vectors
// (8 bf16 or 4 fp32) are dealt round-robin over the 256 threads, so a wave's 64 loads are
// contiguous.  The index grows with j for a fixed thread.
template <int DT>
__device__ __forceinline__ int slice_index(int base, int t, int j) {
  if constexpr (DT == kDtBF16) return base + 8 * (t + kThreads * (j >> 3)) + (j & 7);
  else return base + 4 * (t + kThreads * (j >> 2)) + (j & 3);
}

// Load this thread's 16 logits of one slice; indices >= V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_slice(const void* row, int V, int base, float (&v)[kPerThread]) {
  const int t = threadIdx.x;
  if constexpr (DT == kDtBF16) {
    const uint16_t* r = (const uint16_t*)row;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e0 = base + 8 * (t + kThreads * k);
      if (VEC && e0 + 8 <= V) {
        const uint4 x = *(const uint4*)(r + e0);
        v[8 * k + 0] = bf16_lo(x.x); v[8 * k + 1] = bf16_hi(x.x);
        v[8 * k + 2] = bf16_lo(x.y); v[8 * k + 3] = bf16_hi(x.y);
        v[8 * k + 4] = bf16_lo(x.z); v[8 * k + 5] = bf16_hi(x.z);
        v[8 * k + 6] = bf16_lo(x.w); v[8 * k + 7] = bf16_hi(x.w);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * k + e] = (e0 + e < V) ? bf16_at(r + e0 + e) : -INFINITY;
      }
    }
  } else {
    const float* r = (const float*)row;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = base + 4 * (t + kThreads * k);
      if (VEC && e0 + 4 <= V) {
        const float4 x = *(const float4*)(r + e0);
        v[4 * k + 0] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * k + e] = (e0 + e < V) ? r[e0 + e] : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------- reductions (wave64)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

// Workgroup reductions; every thread gets the result.  `red` is 2*kWaves floats of LDS.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_min_i(int v, int* red) {
  v = wave_min_i(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = min(r, red[i]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_or(int v, int* red) {
  v = wave_or(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r |= red[i];
  __syncthreads();
  return r;
}
// Sum of per-thread fp32 partials in fp64, combined in a fixed order.
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r += red[i];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- Philox4x64-10

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds, each two 64x64 -> 128-bit
// products of counter words with fixed odd multipliers, the key bumped by two Weyl constants
// between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t k0, uint64_t k1, uint64_t c0, uint64_t c1,
                                              uint64_t c2, uint64_t c3, uint64_t (&out)[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

__device__ __forceinline__ double u53(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

// ---------------------------------------------------------------- workspace records

// Streaming partial of one 4096-logit slice of one row.
struct SlicePart {
  float m;     // max logit of the slice (-inf if none finite)
  float s;     // sum exp2((l - m) * c) over the slice
  float w;     // sum e * (l - m) * c  (entropy numerator, base 2)
  int amax;    // lowest index of the slice maximum, -1 if none, -2 if a NaN/+inf was seen
  int cnt;     // logits > -inf in the slice (kept count of an unfiltered row)
};

// Combined statistics of one row.
struct RowStat {
  double z;       // sum_kept exp2((l - m) * c)
  double log2z;
  float m;        // max logit (exact)
  float inv_z;    // (float)(1 / z)
  float h_bits;   // entropy in bits
  float maxp;     // max probability
  int amax;       // argmax, -1 if none
  int flags;      // kStNonfinite / kStFilterOverflow
  int kept;       // kept tokens with a finite logit
  float tau;      // filter threshold (kept iff l >= tau); -inf when unfiltered
};

}  // namespace specv
