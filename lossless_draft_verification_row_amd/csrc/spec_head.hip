// spec_head.hip -- the LM head fused with the row statistics.
//
// The logits of a row, l_v = sum_d h_d W_{v,d} (the projection of a hidden state onto the
// vocabulary that the DLite page's core method does once per round), are formed tile by tile
// with bf16 MFMA and reduced in the tile's epilogue to per-row partial statistics: the tile's
// maximum, its lowest arg-max, sum e and sum e t with e = 2^t, t = (l - m) log2(e) / T, the
// same partials the streaming kernels keep per slice.  The logits never reach memory.  A second
// kernel combines a row's partials in fp64 into the statistics spec_row_stats reports (the
// SpecKV page's signals) and the probability of a given token.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "spec_device.h"
#include "spec_internal.h"

namespace specv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHBK = 64;         // k per stage
constexpr int kHBV = kHeadCols;      // vocabulary columns per workgroup
constexpr int kWC = kHBV / kWaves;   // columns per wave
constexpr int kNJ = kWC / 32;        // 32-column accumulator blocks per wave
constexpr int kHLd = kHBK + 8;       // LDS row stride in bf16 (144 B: 16-B aligned, staggers the banks)
constexpr int kTLd = kWC + 1;        // epilogue transpose row stride in floats
static_assert(kNJ >= 1 && kWC % 32 == 0, "each wave takes whole 32-column blocks");

template <int RB>   // 32-row blocks per workgroup
struct HeadLds {
  union {
    struct {
      alignas(16) uint16_t a[32 * RB][kHLd];   // hidden rows x k of the current stage
      alignas(16) uint16_t b[kHBV][kHLd];      // head rows (vocabulary columns) x k
    } k;
    struct {
      float t[kWaves][32][kTLd];      // one wave's 32 x kWC logits, transposed to rows
      HeadRec part[kWaves][32 * RB];  // per wave: the partials of each row over its columns
    } e;
  };
};

// 16 bytes through a buffer resource: an offset past its end reads as zero, with no branch.
constexpr int kHeadOut = 0x7ffffff0;
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t rs, int off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Issue the global loads of one stage: the workgroup's hidden rows (32 RB x 64 k) and head
// rows (256 x 64 k), eight lanes per row and 16 bytes per lane, so every row's 128 bytes come
// in one coalesced piece.  The resources cover the tile's rows that exist; k past D gets an
// offset past the end, so rows, columns and k outside the problem all read as zero.
template <int RB>
__device__ __forceinline__ void head_load(const HeadArgs& a, __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
                                          int k0, uint4 (&ra)[RB], uint4 (&rb)[kHBV / 32]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int idx = t + kThreads * i, row = idx >> 3, k = k0 + 8 * (idx & 7);
    ra[i] = ld16(rsa, k < a.D ? (row * (int)a.h_ld + k) * 2 : kHeadOut);
  }
#pragma unroll
  for (int i = 0; i < kHBV / 32; ++i) {
    const int idx = t + kThreads * i, row = idx >> 3, k = k0 + 8 * (idx & 7);
    rb[i] = ld16(rsb, k < a.D ? (row * (int)a.w_ld + k) * 2 : kHeadOut);
  }
}
template <int RB>
__device__ __forceinline__ void head_store(HeadLds<RB>& L, const uint4 (&ra)[RB], const uint4 (&rb)[kHBV / 32]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int idx = t + kThreads * i;
    *(uint4*)&L.k.a[idx >> 3][8 * (idx & 7)] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < kHBV / 32; ++i) {
    const int idx = t + kThreads * i;
    *(uint4*)&L.k.b[idx >> 3][8 * (idx & 7)] = rb[i];
  }
}

// Two waves per SIMD for the tall tile (its accumulators, staged loads and fragments take up
// to 256 registers; two workgroups share a CU's LDS).
constexpr int head_min_waves(int rb) { return rb == 4 ? 2 : 1; }

// One workgroup per (32 RB rows) x (kHBV columns) tile.  Wave w holds columns kWC w ..
// kWC (w + 1) - 1 of every row in RB x kNJ accumulators of the 32x32x16 bf16 MFMA: A[i][k] is
// lane i + 32 (k / 8) element k % 8, B[k][j] lane j + 32 (k / 8), and C[i][j] lane j + 32 ((i / 4) % 2) element
// 4 (i / 8) + i % 4.  Workgroup i runs on XCD i mod 8; the row tiles of one column tile go to
// consecutive workgroups of one XCD, so its L2 serves the head tile they share (and the hidden
// tiles, shared by every column tile).
template <int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(head_min_waves(RB)))) void k_head(
    HeadArgs a) {
  __shared__ HeadLds<RB> L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int rt = jx % a.n_rt, ct = (jx / a.n_rt) * 8 + xcd;
  if (ct >= a.n_ct) return;
  const int r0 = rt * 32 * RB, v0 = ct * kHBV;
  f32x16 acc[RB][kNJ];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // One LDS stage: the next stage's loads are in flight in registers while this one feeds the
  // MFMAs, then replace it between two barriers.  A and B fragments are read from LDS in the
  // MFMA layout (lane l: row l % 32 of its block, k 8 (l / 32) .. + 7 of each 16).
  const __amdgpu_buffer_rsrc_t rsa = row_rsrc((const uint16_t*)a.hidden + (int64_t)r0 * a.h_ld,
                                             (int)(min(32 * RB, a.R - r0) * a.h_ld * 2));
  const __amdgpu_buffer_rsrc_t rsb = row_rsrc((const uint16_t*)a.weight + (int64_t)v0 * a.w_ld,
                                             (int)(min(kHBV, a.V - v0) * a.w_ld * 2));
  uint4 ra[RB], rb[kHBV / 32];
  const int n_k = (a.D + kHBK - 1) / kHBK;
  head_load<RB>(a, rsa, rsb, 0, ra, rb);
  head_store<RB>(L, ra, rb);
  __syncthreads();
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  for (int kt = 0; kt < n_k; ++kt) {
    const bool more = kt + 1 < n_k;
    if (more) head_load<RB>(a, rsa, rsb, (kt + 1) * kHBK, ra, rb);
    // the MFMA stretch at raised priority: a SIMD shared with the other workgroup keeps
    // issuing matrix work while that one is between its barriers
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < kHBK / 16; ++h) {
      bf16x8 fa[RB], fv[kNJ];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        fa[i] = __builtin_bit_cast(bf16x8, *(const uint4*)&L.k.a[32 * i + fr][16 * h + fk]);
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        fv[j] = __builtin_bit_cast(bf16x8, *(const uint4*)&L.k.b[kWC * wave + 32 * j + fr][16 * h + fk]);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < kNJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fv[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();   // every wave is done with this stage (and, after the last, with L.k)
    if (more) {
      head_store<RB>(L, ra, rb);
      __syncthreads();
    }
  }

  // Epilogue: per 32-row block, the wave's 32 x kWC logits go to LDS by row; lanes 2i and
  // 2i + 1 take row i, kWC / 2 columns each.
  const float c = a.c;
  const int cw0 = v0 + kWC * wave;   // this wave's first column
  const int hf = lane & 1, ri = lane >> 1;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int col = 32 * j + (lane & 31);
      const bool in = cw0 + col < a.V;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        L.e.t[wave][row][col] = in ? acc[i][j][e] : -INFINITY;
      }
    }
    __syncthreads();
    const float* x = &L.e.t[wave][ri][kWC / 2 * hf];
    const int r = r0 + 32 * i + ri;
    // the token's logit, from the one lane whose columns hold it
    if (a.tokens && r < a.R) {
      const int y = a.tokens[r] - (cw0 + kWC / 2 * hf);
      if (y >= 0 && y < kWC / 2 && cw0 + kWC / 2 * hf + y < a.V) a.ly[r] = x[y];
    }
    float m = -INFINITY;
    int am = INT_MAX, bad = 0;
#pragma unroll
    for (int q = 0; q < kWC / 2; ++q) {
      const float v = x[q];
      bad |= (v != v || v == INFINITY) ? 1 : 0;
      if (v > m) { m = v; am = q; }
    }
    am = m > -INFINITY ? cw0 + kWC / 2 * hf + am : INT_MAX;
    // the partner lane holds the row's other 32 columns
    const float m2 = __shfl_xor(m, 1);
    const int am2 = __shfl_xor(am, 1);
    bad |= __shfl_xor(bad, 1);
    const float M = fmaxf(m, m2);
    int amx = INT_MAX;
    if (m == M) amx = am;
    if (m2 == M) amx = min(amx, am2);
    // t = (l - M) c, exactly 0 at the maximum (e = 1); the sums in fp64
    double s = 0.0, w = 0.0;
    if (!a.greedy && M > -INFINITY) {
#pragma unroll
      for (int q = 0; q < kWC / 2; ++q) {
        const float tt = (x[q] - M) * c;
        const float ev = __builtin_amdgcn_exp2f(tt);
        s += (double)ev;
        if (ev > 0.f) w = fma((double)ev, (double)tt, w);
      }
      s += __shfl_xor(s, 1);
      w += __shfl_xor(w, 1);
    }
    if (hf == 0) {
      HeadRec pr;
      pr.m = M;
      pr.s = s;
      pr.w = w;
      pr.amax = bad ? -2 : (amx == INT_MAX ? -1 : amx);
      L.e.part[wave][32 * i + ri] = pr;
    }
    __syncthreads();
  }
  // the four waves' partials of each row, folded in column order into the tile's record
  if (t < 32 * RB && r0 + t < a.R) {
    float M = -INFINITY;
    int flag = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      const HeadRec p = L.e.part[q][t];
      M = fmaxf(M, p.m);
      if (p.amax == -2) flag = 1;
    }
    HeadRec out;
    out.m = M;
    out.s = 0.0;
    out.w = 0.0;
    out.amax = -1;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      const HeadRec p = L.e.part[q][t];
      if (out.amax < 0 && p.m == M && p.amax >= 0) out.amax = p.amax;
      if (!a.greedy && p.m > -INFINITY && M > -INFINITY) {
        const double d = ((double)p.m - (double)M) * (double)c;
        const double f = exp2_split(d);
        out.s += p.s * f;
        out.w += f * (p.w + p.s * d);
      }
    }
    if (flag) out.amax = -2;
    a.rec[(int64_t)(r0 + t) * a.n_ct + ct] = out;
  }
}

// One wave per row: the row's tile records in fp64 (maximum, lowest arg-max, sum e and sum e t
// relative to the row maximum), then the statistics and p(token).  A NaN or +inf logit makes
// every output of the row NaN and its arg-max -1.
__global__ __launch_bounds__(kThreads) void k_head_combine(HeadArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (r >= a.R) return;
  const HeadRec* rc = a.rec + (int64_t)r * a.n_ct;
  float M = -INFINITY;
  int bad = 0;
  for (int k = lane; k < a.n_ct; k += 64) {
    const HeadRec p = rc[k];
    M = fmaxf(M, p.m);
    bad |= p.amax == -2 ? 1 : 0;
  }
  M = wave_max_dpp(M);
  bad = wave_or(bad);
  int am = INT_MAX;
  double s = 0.0, w = 0.0;
  const double cd = (double)a.c;
  for (int k = lane; k < a.n_ct; k += 64) {
    const HeadRec p = rc[k];
    if (p.m == M && p.amax >= 0) am = min(am, p.amax);
    if (!a.greedy && p.m > -INFINITY && M > -INFINITY) {
      const double d = ((double)p.m - (double)M) * cd;
      const double f = exp2_split(d);
      s += p.s * f;
      w += f * (p.w + p.s * d);
    }
  }
  am = wave_min_i(am);
  s = wave_sum_dpp_d(s);
  w = wave_sum_dpp_d(w);
  if (lane != 0) return;
  const float nan = __int_as_float(0x7fc00000);
  const bool ok = !bad && M > -INFINITY && (a.greedy || s > 0.0);
  const int y = a.tokens ? a.tokens[r] : -1;
  const bool yv = y >= 0 && y < a.V;
  float mx = nan, lz = nan, ent = nan, mp = nan, pt = nan;
  int ax = -1;
  if (ok) {
    mx = M;
    ax = am == INT_MAX ? -1 : am;
    if (a.greedy) {
      ent = 0.f;
      mp = 1.f;
      if (yv) pt = y == ax ? 1.f : 0.f;
    } else {
      lz = (float)((double)M * a.inv_t + log2_split(s) * 0.6931471805599453);
      ent = (float)(log2_split(s) - w / s);
      mp = (float)(1.0 / s);
      if (yv) pt = (float)(exp2_split(((double)a.ly[r] - (double)M) * cd) / s);
    }
  }
  if (a.max_logit) a.max_logit[r] = mx;
  if (a.argmax) a.argmax[r] = ax;
  if (a.log_z) a.log_z[r] = lz;
  if (a.entropy_bits) a.entropy_bits[r] = ent;
  if (a.max_prob) a.max_prob[r] = mp;
  if (a.p_tok) a.p_tok[r] = pt;
}

hipError_t launch_head(const HeadArgs& a0, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  HeadArgs a = a0;
  const bool big = a.R > 64;
  a.n_rt = big ? (a.R + 127) / 128 : (a.R + 63) / 64;
  const long long grid = (long long)a.n_rt * ((a.n_ct + 7) / 8) * 8;
  if (grid < 1 || grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  if (big) launch_timed(k_head<4>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
  else launch_timed(k_head<2>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_head_combine, dim3((unsigned)((a.R + kWaves - 1) / kWaves)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace specv
