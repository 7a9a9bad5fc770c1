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
constexpr int kStTimeout = 16;
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

// 16 bytes of a logit row read once: a non-temporal load (the streaming passes' policy).
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(w[0], w[1], w[2], w[3]);
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
        const uint4 x = ld_nt16(r + e0);
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
        const uint4 xw = ld_nt16(r + e0);
        const float4 x = make_float4(__uint_as_float(xw.x), __uint_as_float(xw.y), __uint_as_float(xw.z), __uint_as_float(xw.w));
        v[4 * k + 0] = x.x; v[4 * k + 1] = x.y; v[4 * k + 2] = x.z; v[4 * k + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * k + e] = (e0 + e < V) ? r[e0 + e] : -INFINITY;
      }
    }
  }
}

// Raw words of one thread's 16 logits of a slice (bf16 pairs or floats), so that the loads of
// the next slice can be in flight while the current one is processed.
template <int DT>
struct RawSlice {
  static constexpr int kWords = DT == kDtBF16 ? kPerThread / 2 : kPerThread;
  uint32_t w[kWords];
};

// Issue the loads of this thread's 16 logits; indices >= V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_raw(const void* row, int V, int base, RawSlice<DT>& r) {
  const int t = threadIdx.x;
  if constexpr (DT == kDtBF16) {
    const uint16_t* p = (const uint16_t*)row;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e0 = base + 8 * (t + kThreads * k);
      if (VEC && e0 + 8 <= V) {
        const uint4 x = ld_nt16(p + e0);
        r.w[4 * k + 0] = x.x; r.w[4 * k + 1] = x.y; r.w[4 * k + 2] = x.z; r.w[4 * k + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (e0 + 2 * e < V) ? p[e0 + 2 * e] : 0xff80u;
          const uint32_t hi = (e0 + 2 * e + 1 < V) ? p[e0 + 2 * e + 1] : 0xff80u;
          r.w[4 * k + e] = lo | (hi << 16);
        }
      }
    }
  } else {
    const float* p = (const float*)row;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = base + 4 * (t + kThreads * k);
      if (VEC && e0 + 4 <= V) {
        const uint4 x = ld_nt16(p + e0);
        r.w[4 * k + 0] = x.x; r.w[4 * k + 1] = x.y; r.w[4 * k + 2] = x.z; r.w[4 * k + 3] = x.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r.w[4 * k + e] = (e0 + e < V) ? __float_as_uint(p[e0 + e]) : 0xff800000u;
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void unpack_raw(const RawSlice<DT>& r, float (&v)[kPerThread]) {
  if constexpr (DT == kDtBF16) {
#pragma unroll
    for (int k = 0; k < kPerThread / 2; ++k) { v[2 * k] = bf16_lo(r.w[k]); v[2 * k + 1] = bf16_hi(r.w[k]); }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) v[k] = __uint_as_float(r.w[k]);
  }
}

// ---------------------------------------------------------------- reductions (wave64)

// Wave-wide reductions by DPP: two quad permutations and two row rotations reduce each row
// of 16 lanes, two row broadcasts carry the rows into lane 63, and v_readlane returns lane
// 63's value to every lane.  Lanes a DPP step does not write keep the identity `old`.  Call
// them with the whole wave active.
#define SPEC_DPP_I(old, v, ctrl, rmask) __builtin_amdgcn_update_dpp((old), (v), (ctrl), (rmask), 0xf, false)
#define SPEC_DPP_F(old, v, ctrl, rmask) \
  __builtin_bit_cast(float, SPEC_DPP_I(__builtin_bit_cast(int, (old)), __builtin_bit_cast(int, (v)), (ctrl), (rmask)))
__device__ __forceinline__ float wave_max(float v) {
  const float o = -INFINITY;
  v = fmaxf(v, SPEC_DPP_F(o, v, 0xb1, 0xf));
  v = fmaxf(v, SPEC_DPP_F(o, v, 0x4e, 0xf));
  v = fmaxf(v, SPEC_DPP_F(o, v, 0x124, 0xf));
  v = fmaxf(v, SPEC_DPP_F(o, v, 0x128, 0xf));
  v = fmaxf(v, SPEC_DPP_F(o, v, 0x142, 0xa));
  v = fmaxf(v, SPEC_DPP_F(o, v, 0x143, 0xc));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += SPEC_DPP_F(0.f, v, 0xb1, 0xf);
  v += SPEC_DPP_F(0.f, v, 0x4e, 0xf);
  v += SPEC_DPP_F(0.f, v, 0x124, 0xf);
  v += SPEC_DPP_F(0.f, v, 0x128, 0xf);
  v += SPEC_DPP_F(0.f, v, 0x142, 0xa);
  v += SPEC_DPP_F(0.f, v, 0x143, 0xc);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0xb1, 0xf));
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0x4e, 0xf));
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0x124, 0xf));
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0x128, 0xf));
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0x142, 0xa));
  v = min(v, SPEC_DPP_I(INT_MAX, v, 0x143, 0xc));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_or(int v) {
  v |= SPEC_DPP_I(0, v, 0xb1, 0xf);
  v |= SPEC_DPP_I(0, v, 0x4e, 0xf);
  v |= SPEC_DPP_I(0, v, 0x124, 0xf);
  v |= SPEC_DPP_I(0, v, 0x128, 0xf);
  v |= SPEC_DPP_I(0, v, 0x142, 0xa);
  v |= SPEC_DPP_I(0, v, 0x143, 0xc);
  return __builtin_amdgcn_readlane(v, 63);
}
// 64-bit DPP move of both halves (lanes whose source is outside the row, or rows outside
// RMASK, read 0).
template <int CTRL, int RMASK>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, RMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, RMASK, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane), hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xb1, 0xf>(v);
  v += dpp_d<0x4e, 0xf>(v);
  v += dpp_d<0x124, 0xf>(v);
  v += dpp_d<0x128, 0xf>(v);
  v += dpp_d<0x142, 0xa>(v);
  v += dpp_d<0x143, 0xc>(v);
  return readlane_d(v, 63);
}

// DPP wave reductions (gfx9 row broadcasts): the result is valid in lane 63 and is returned
// to every lane through v_readlane.
#define SPEC_DPP(old, v, ctrl, rmask) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, (old)), \
                                                        __builtin_bit_cast(int, (v)), (ctrl), (rmask), 0xf, false))
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += SPEC_DPP(0.f, v, 0xb1, 0xf);   // quad_perm [1,0,3,2]
  v += SPEC_DPP(0.f, v, 0x4e, 0xf);   // quad_perm [2,3,0,1]
  v += SPEC_DPP(0.f, v, 0x124, 0xf);  // row_ror:4
  v += SPEC_DPP(0.f, v, 0x128, 0xf);  // row_ror:8
  v += SPEC_DPP(0.f, v, 0x142, 0xa);  // row_bcast:15
  v += SPEC_DPP(0.f, v, 0x143, 0xc);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  const float ninf = -INFINITY;
  v = fmaxf(v, SPEC_DPP(ninf, v, 0xb1, 0xf));
  v = fmaxf(v, SPEC_DPP(ninf, v, 0x4e, 0xf));
  v = fmaxf(v, SPEC_DPP(ninf, v, 0x124, 0xf));
  v = fmaxf(v, SPEC_DPP(ninf, v, 0x128, 0xf));
  v = fmaxf(v, SPEC_DPP(ninf, v, 0x142, 0xa));
  v = fmaxf(v, SPEC_DPP(ninf, v, 0x143, 0xc));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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

// ---------------------------------------------------------------- light fp64 transcendentals

// 2^x as a double with ~1.5e-7 relative error: the integer part is applied exactly with
// ldexp, the fraction in [0, 1) goes through the hardware exp2.  Keeps fp64 library code
// (and its registers) out of the kernels.  NaN propagates; x below -1074 gives 0.
__device__ __forceinline__ double exp2_split(double x) {
  if (!(x > -1074.0)) return (x != x) ? x : 0.0;
  const double n = floor(x);
  const float f = (float)(x - n);
  return ldexp((double)__builtin_amdgcn_exp2f(f), (int)n);
}

// log2(z) for z > 0 with ~1e-7 absolute error: exact exponent plus the hardware log2 of the
// mantissa in [0.5, 1).
__device__ __forceinline__ double log2_split(double z) {
  int e;
  const double mant = frexp(z, &e);
  return (double)e + (double)__builtin_amdgcn_logf((float)mant);
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

// Slice partial of the fused kernel: e = exp2(l c - ref) with ref = slice max * c.
struct alignas(16) Part4 {
  float ref;   // slice reference in base-2 units (greedy: the slice max logit)
  float s;     // sum e
  float w;     // sum e * (l c - ref), clamped below at -200 (entropy numerator)
  int amax;    // greedy: lowest index of the slice maximum, -1 none, -2 NaN / +inf seen
};

// ---------------------------------------------------------------- cross-workgroup exchange
//
// Data shared between workgroups of one launch travel through relaxed agent-scope atomic
// loads and stores (coherent "sc1" accesses that bypass the per-XCD L2), ordered against
// the counters by waiting for their completion.  No acquire / release fence is used: on a
// multi-XCD device those write back and invalidate the whole L2 at every use.
__device__ __forceinline__ void st_coh(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coh(const void* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory access issued so far has completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ unsigned ctr_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ctr_load(const unsigned* p) {
  return __hip_atomic_load((unsigned*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ uint64_t pack2(float a, int b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)(uint32_t)b << 32);
}
__device__ __forceinline__ uint64_t pack2(int a, int b) {
  return (uint64_t)(uint32_t)a | ((uint64_t)(uint32_t)b << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
__device__ __forceinline__ int lo_i(uint64_t v) { return (int)(uint32_t)v; }
__device__ __forceinline__ int hi_i(uint64_t v) { return (int)(uint32_t)(v >> 32); }

constexpr int kTeamBadP = 1;
constexpr int kTeamBadQ = 2;

// Statistics of one team (a target row and, for a paired position, its draft row).
struct TeamStat {
  double z[2];    // sum over the row of exp2(l c - M)
  double beta;    // sum_x [p - q]_+ of a paired position
  float M[2];     // row reference in base-2 units (greedy: the max logit)
  float h[2];     // entropy in bits
  int amax;       // greedy: argmax of the target row
  int flags;      // kTeamBadP / kTeamBadQ: a row with NaN / +inf or without a finite logit
};

__device__ __forceinline__ void store_part(Part4* p, const Part4& v) {
  st_coh(p, pack2(v.ref, v.s));
  st_coh((char*)p + 8, pack2(v.w, v.amax));
}
__device__ __forceinline__ Part4 load_part(const Part4* p) {
  const uint64_t a = ld_coh(p), b = ld_coh((const char*)p + 8);
  Part4 v;
  v.ref = lo_f(a); v.s = hi_f(a); v.w = lo_f(b); v.amax = hi_i(b);
  return v;
}
__device__ __forceinline__ void store_double(double* p, double v) { st_coh(p, (uint64_t)__double_as_longlong(v)); }
__device__ __forceinline__ double load_double(const double* p) { return __longlong_as_double((long long)ld_coh(p)); }
__device__ __forceinline__ void store_team(TeamStat* p, const TeamStat& v) {
  st_coh(&p->z[0], (uint64_t)__double_as_longlong(v.z[0]));
  st_coh(&p->z[1], (uint64_t)__double_as_longlong(v.z[1]));
  st_coh(&p->beta, (uint64_t)__double_as_longlong(v.beta));
  st_coh(&p->M[0], pack2(v.M[0], v.M[1]));
  st_coh(&p->h[0], pack2(v.h[0], v.h[1]));
  st_coh(&p->amax, pack2(v.amax, v.flags));
}
__device__ __forceinline__ TeamStat load_team(const TeamStat* p) {
  TeamStat v;
  v.z[0] = __longlong_as_double((long long)ld_coh(&p->z[0]));
  v.z[1] = __longlong_as_double((long long)ld_coh(&p->z[1]));
  v.beta = __longlong_as_double((long long)ld_coh(&p->beta));
  uint64_t m = ld_coh(&p->M[0]), h = ld_coh(&p->h[0]), ai = ld_coh(&p->amax);
  v.M[0] = lo_f(m); v.M[1] = hi_f(m); v.h[0] = lo_f(h); v.h[1] = hi_f(h);
  v.amax = lo_i(ai); v.flags = hi_i(ai);
  return v;
}

// ---------------------------------------------------------------- scalar loads

// The wave's (uniform) pointer in scalar registers: callers pass wave-uniform addresses, and
// taking the first lane's copy lets the scalar load below take it even where the compiler cannot
// prove the uniformity itself.
__device__ __forceinline__ const int32_t* uniform_ptr(const int32_t* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const int32_t*)(((uint64_t)hi << 32) | lo);
}

// A uniform 32-bit load through the scalar data cache (read-only data of the call).
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  return v;
}

// Two consecutive uniform 32-bit values in one scalar load (p 4-byte aligned).
__device__ __forceinline__ void sload2_i32(const int32_t* p, int& a, int& b) {
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
  a = (int)(uint32_t)v;
  b = (int)(uint32_t)(v >> 32);
}

// ---------------------------------------------------------------- wave-wide fp64 helpers

// fp64 sum over the wave in a fixed order (row reductions, then row broadcasts); every lane
// gets lane 63's total.
__device__ __forceinline__ double wave_sum_dpp_d(double v) {
  v += dpp_d<0xb1, 0xf>(v);
  v += dpp_d<0x4e, 0xf>(v);
  v += dpp_d<0x124, 0xf>(v);
  v += dpp_d<0x128, 0xf>(v);
  v += dpp_d<0x142, 0xa>(v);
  v += dpp_d<0x143, 0xc>(v);
  return readlane_d(v, 63);
}
// Inclusive fp64 prefix sum over the wave's lanes (row shifts, then row broadcasts).
__device__ __forceinline__ double wave_scan_dpp_d(double v) {
  v += dpp_d<0x111, 0xf>(v);   // row_shr:1
  v += dpp_d<0x112, 0xf>(v);   // row_shr:2
  v += dpp_d<0x114, 0xf>(v);   // row_shr:4
  v += dpp_d<0x118, 0xf>(v);   // row_shr:8
  v += dpp_d<0x142, 0xa>(v);   // row_bcast:15
  v += dpp_d<0x143, 0xc>(v);   // row_bcast:31
  return v;
}
// Inverse-CDF pick over the masses held one per lane (lanes >= n hold 0): the first index
// whose prefix sum exceeds u * total; if rounding leaves none, the last index with positive
// mass; -1 when the total is not positive.  Returns the pick; `total` gets the sum.
__device__ __forceinline__ int wave_pick(double m, int n, double u, double& total) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < n;
  const double cum = wave_scan_dpp_d(in ? m : 0.0);
  total = readlane_d(cum, 63);
  if (!(total > 0.0)) return -1;
  const double target = u * total;
  const unsigned long long over = __ballot(in && cum > target);
  if (over) return __builtin_ctzll(over);
  const unsigned long long pos = __ballot(in && m > 0.0);
  return pos ? 63 - __builtin_clzll(pos) : -1;
}

// ---------------------------------------------------------------- bounds-checked row loads

// Bounds-checked row loads: a buffer resource over the row's bytes.  16-byte loads past the
// end return zeros and touch no memory (num_records 0 turns every load off).  The streaming
// loads are non-temporal (the nt cache policy): each logit is read once, and marking the lines
// for early eviction raises the read rate the HBM sustains (a plain 1 GiB read: 5.8 -> 6.6 TB/s).
constexpr int kCpolNt = 2;   // cache-policy bits of a buffer load: non-temporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, nbytes, 0x00020000);
}
template <int DT>
__device__ __forceinline__ void load_raw_buf(__amdgpu_buffer_rsrc_t rs, int base, RawSlice<DT>& r) {
  const int t = threadIdx.x;
  constexpr int kEl = DT == kDtBF16 ? 8 : 4;      // elements per 16-byte vector
  constexpr int kEsz = DT == kDtBF16 ? 2 : 4;
#pragma unroll
  for (int k = 0; k < kPerThread / kEl; ++k) {
    const int e0 = base + kEl * (t + kThreads * k);
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, e0 * kEsz, 0, kCpolNt);
    r.w[4 * k + 0] = x[0]; r.w[4 * k + 1] = x[1]; r.w[4 * k + 2] = x[2]; r.w[4 * k + 3] = x[3];
  }
}
// Logits at indices >= V (zeros from the bounds check) become -inf.
template <int DT>
__device__ __forceinline__ void mask_tail(int V, int base, float (&v)[kPerThread]) {
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (slice_index<DT>(base, threadIdx.x, j) >= V) v[j] = -INFINITY;
}

// ---------------------------------------------------------------- radix select helpers

// Order key of a logit: unsigned, larger key = larger value; -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

struct SelLds {
  uint32_t hist[256];
  int wtot[2][kWaves];
  int digit, above, total;
};

// One pass of the block-wide radix select: `cnt(d)` for the keys whose higher digits match
// `prefix` must already be in S.hist.  Wave 0 finds the digit d holding the kk-th largest
// (counting from the top) and the number of keys above it; the digit is -1 when fewer than kk
// keys were counted (S.total holds the count).
__device__ __forceinline__ void select_digit(SelLds& S, int kk) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int c[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { c[q] = (int)S.hist[255 - 4 * lane - q]; s += c[q]; }
    const int incl = wave_incl_scan_i(s);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const unsigned long long hit = __ballot(incl >= kk);
    if (lane == 0) { S.total = total; S.digit = -1; S.above = 0; }
    if (hit && total >= kk) {
      const int L = __builtin_ctzll(hit);
      if (lane == L) {
        int run = incl - s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (run + c[q] >= kk) { S.digit = 255 - 4 * lane - q; S.above = run; break; }
          run += c[q];
        }
      }
    }
  }
}

// Value of a 16-bit order key of a bf16 value (the inverse of order_key(v) >> 16).
__device__ __forceinline__ float key16_value(int k) {
  const uint32_t b = (k & 0x8000) ? ((uint32_t)k & 0x7FFFu) : (~(uint32_t)k & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// 16 consecutive logits starting at x0 (vector loads when aligned and in range).
template <int DT, bool VEC>
__device__ __forceinline__ void load_run16(const void* row, int V, int x0, float (&v)[16]) {
  if constexpr (DT == kDtBF16) {
    const uint16_t* p = (const uint16_t*)row;
    if (VEC && x0 + 16 <= V) {
      const uint4 a = *(const uint4*)(p + x0), b = *(const uint4*)(p + x0 + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = (x0 + e < V) ? bf16_at(p + x0 + e) : -INFINITY;
    }
  } else {
    const float* p = (const float*)row;
    if (VEC && x0 + 16 <= V) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *(const float4*)(p + x0 + 4 * k);
        v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = (x0 + e < V) ? p[x0 + e] : -INFINITY;
    }
  }
}

// 16 consecutive logits of a row as raw 16-byte words (two for bf16, four for fp32), loaded
// when the run is aligned and in range; raw_run_unpack turns them into floats, reading the
// elements one by one itself for a run that is not (masked: -inf past V).
template <int DT>
struct RawRun16 {
  uint4 w[DT == kDtBF16 ? 2 : 4];
};
template <int DT, bool VEC>
__device__ __forceinline__ RawRun16<DT> raw_run_load(const void* row, int V, int x0) {
  RawRun16<DT> r;
  constexpr int n = DT == kDtBF16 ? 2 : 4;
  if (VEC && x0 + 16 <= V) {
    const uint4* p = (const uint4*)((const char*)row + (size_t)x0 * (DT == kDtBF16 ? 2 : 4));
#pragma unroll
    for (int k = 0; k < n; ++k) r.w[k] = p[k];
  } else {
#pragma unroll
    for (int k = 0; k < n; ++k) r.w[k] = make_uint4(0u, 0u, 0u, 0u);
  }
  return r;
}
template <int DT, bool VEC>
__device__ __forceinline__ void raw_run_unpack(const RawRun16<DT>& r, const void* row, int V, int x0, float (&v)[16]) {
  if (VEC && x0 + 16 <= V) {
    if constexpr (DT == kDtBF16) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t w[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[8 * k + 2 * q] = bf16_lo(w[q]); v[8 * k + 2 * q + 1] = bf16_hi(w[q]); }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[4 * k] = __uint_as_float(r.w[k].x); v[4 * k + 1] = __uint_as_float(r.w[k].y);
        v[4 * k + 2] = __uint_as_float(r.w[k].z); v[4 * k + 3] = __uint_as_float(r.w[k].w);
      }
    }
  } else {
    load_run16<DT, VEC>(row, V, x0, v);
  }
}

// Pair sums of one (target, draft) row pair with the relative precision of fp64, for the rare
// positions where the streaming passes' fp32 sums would not keep it: A = sum min(p, q) when the
// two distributions barely overlap (1 - beta loses A's precision), and beta = sum [p - q]_+ when
// they nearly coincide (an error in the normalisers' ratio then moves every term the same way).
// Two passes over both rows by the whole workgroup: Z_p and Z_q as fp64 sums of the same
// e-values the second pass divides, then A and beta in fp64 (guide page "5.1 投机解码核心原理"
// §4.1 / §4.3: beta = sum [p - q]_+, A = sum min(p, q) = 1 - beta).  One workgroup reads the
// rows, so each thread keeps kPairRuns runs of 16 logits of both rows in flight before it works
// on any of them (a run at a time would leave the pass at the latency of one load per thread).
// The exponent of logit l is t = (l - ref) c when SUB, else l c - ref; logits below tau are
// masked.  `red` holds kWaves doubles of LDS.
constexpr int kPairRuns = 4;
template <int DT, bool VEC, bool SUB>
__device__ void pair_sums_fp64(const void* prow, const void* qrow, int V, float c, float refp, float refq, float taup,
                               float tauq, double* red, double& A, double& beta) {
  const int t = threadIdx.x;
  auto ex = [&](float l, float ref, float tau) -> float {
    if (l < tau) return 0.f;
    return __builtin_amdgcn_exp2f(SUB ? (l - ref) * c : fmaf(l, c, -ref));
  };
  constexpr int kStep = kThreads * 16;
  double zp = 0.0, zq = 0.0;
  for (int x0 = t * 16; x0 < V; x0 += kPairRuns * kStep) {
    RawRun16<DT> rp[kPairRuns], rq[kPairRuns];
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      rp[u] = raw_run_load<DT, VEC>(prow, V, x0 + u * kStep);
      rq[u] = raw_run_load<DT, VEC>(qrow, V, x0 + u * kStep);
    }
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      const int xu = x0 + u * kStep;
      if (xu >= V) break;
      float vp[16], vq[16];
      raw_run_unpack<DT, VEC>(rp[u], prow, V, xu, vp);
      raw_run_unpack<DT, VEC>(rq[u], qrow, V, xu, vq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        zp += (double)ex(vp[e], refp, taup);
        zq += (double)ex(vq[e], refq, tauq);
      }
    }
  }
  zp = block_sum_d(zp, red);
  zq = block_sum_d(zq, red);
  const double ip = 1.0 / zp, iq = 1.0 / zq;
  double a = 0.0, bsum = 0.0;
  for (int x0 = t * 16; x0 < V; x0 += kPairRuns * kStep) {
    RawRun16<DT> rp[kPairRuns], rq[kPairRuns];
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      rp[u] = raw_run_load<DT, VEC>(prow, V, x0 + u * kStep);
      rq[u] = raw_run_load<DT, VEC>(qrow, V, x0 + u * kStep);
    }
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      const int xu = x0 + u * kStep;
      if (xu >= V) break;
      float vp[16], vq[16];
      raw_run_unpack<DT, VEC>(rp[u], prow, V, xu, vp);
      raw_run_unpack<DT, VEC>(rq[u], qrow, V, xu, vq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const double pp = (double)ex(vp[e], refp, taup) * ip, qq = (double)ex(vq[e], refq, tauq) * iq;
        a += fmin(pp, qq);
        bsum += fmax(pp - qq, 0.0);
      }
    }
  }
  A = block_sum_d(a, red);
  beta = block_sum_d(bsum, red);
}

// 1 - TV = A = sum min(p, q) of one (target, draft) row pair in one pass over both rows, for
// positions whose two distributions barely overlap, with the rows' own normalisers: p =
// 2^(l c - refp) / zp (refp and zp as the streaming passes formed them), q alike.  Every term is
// positive, so the sum keeps the relative precision of its terms (fp32 each, about 1e-6 at
// worst from the exponent's rounding) however small A is; 16 terms are added in fp32, the runs
// in fp64 (guide page "5.1 投机解码核心原理" §4.3).  Logits below taup / tauq are masked.  `red`
// holds kWaves doubles of LDS.
template <int DT, bool VEC>
__device__ double pair_overlap(const void* prow, const void* qrow, int V, float c, float refp, float refq, double zp,
                               double zq, float taup, float tauq, double* red) {
  const int t = threadIdx.x;
  const float ip = (float)(1.0 / zp), iq = (float)(1.0 / zq);
  constexpr int kStep = kThreads * 16;
  double a = 0.0;
  for (int x0 = t * 16; x0 < V; x0 += kPairRuns * kStep) {
    RawRun16<DT> rp[kPairRuns], rq[kPairRuns];
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      rp[u] = raw_run_load<DT, VEC>(prow, V, x0 + u * kStep);
      rq[u] = raw_run_load<DT, VEC>(qrow, V, x0 + u * kStep);
    }
#pragma unroll
    for (int u = 0; u < kPairRuns; ++u) {
      const int xu = x0 + u * kStep;
      if (xu >= V) break;
      float vp[16], vq[16];
      raw_run_unpack<DT, VEC>(rp[u], prow, V, xu, vp);
      raw_run_unpack<DT, VEC>(rq[u], qrow, V, xu, vq);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = vp[e] < taup ? 0.f : __builtin_amdgcn_exp2f(fmaf(vp[e], c, -refp)) * ip;
        const float qe = vq[e] < tauq ? 0.f : __builtin_amdgcn_exp2f(fmaf(vq[e], c, -refq)) * iq;
        s += fminf(pe, qe);
      }
      a += (double)s;
    }
  }
  return block_sum_d(a, red);
}

// Below this overlap A, or this residual mass beta, a position's pair sums are recomputed with
// pair_sums_fp64: the fp32 streaming sums carry an absolute error near 1e-7, which would exceed
// 1e-5 of A (taken as 1 - beta) or of beta under about 1e-2.
constexpr double kPairRefine = 0.02;

// Expected tokens committed given the drafts, 1 + sum_{k=1..g} prod_{i<=k} a_i, from the
// per-position accept probabilities, in fp64 and position order.
__device__ __forceinline__ float expected_committed(const double* ap, int g) {
  double run = 1.0, e = 1.0;
  for (int i = 0; i < g; ++i) {
    run *= ap[i];
    e += run;
  }
  return (float)e;
}

}  // namespace specv
