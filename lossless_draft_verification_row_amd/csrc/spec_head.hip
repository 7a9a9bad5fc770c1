// spec_head.hip -- the LM head fused with the row statistics.
//
// The logits of a row, l_v = sum_d h_d W_{v,d} (the projection of a hidden state onto the
// vocabulary that the DLite page's core method does once per round), are formed tile by tile
// with bf16 MFMA and reduced in the tile's epilogue to per-row partial statistics: the tile's
// maximum, its lowest arg-max, sum e and sum e t with e = 2^t, t = (l - m) log2(e) / T, the
// same partials the streaming kernels keep per slice.  The logits never reach memory.  A second
// kernel combines a row's partials in fp64 into the statistics spec_row_stats reports (the
// SpecKV page's signals) and the probability of a given token.
//
//   k_head_sq       more than 128 rows, D a multiple of 64: 256 x 256 tiles, one wave per
//                   SIMD with 4 x 4 accumulators, stages loaded straight into LDS
//   k_head          otherwise: 128 x 256 (or 64 x 256) tiles, two waves per SIMD, stages
//                   staged through registers
//   k_head_combine  one wave per row: the row's tile records, then the statistics
//   k_mfma_rate     benchmark instrumentation: the matrix cores' rate on the same MFMA
//                   pattern with register operands
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

// ---- Square tiles fed by direct-to-LDS loads (D a whole number of 64-deep stages) ----
//
// 256 rows x 256 columns per workgroup, four waves in a 2 x 2 arrangement of 128 x 128 (4 x 4
// accumulators of the 32x32x16 MFMA: 256 registers, which the compiler keeps in the
// accumulation registers; one wave per SIMD, one workgroup per CU).  A stage holds 64 k (eight
// 16-byte granules) of all 256 hidden rows and all 256 head rows, 64 KB in all; two stage
// buffers alternate.  The buffer load's LDS form writes each instruction's 64 granules, one per
// lane in lane order, straight into LDS, so the waves issue no LDS stores and hold no staging
// registers, and a load costs the wave one instruction plus the M0 write: each lane's offset
// within the tile is fixed, and the stage's k enters as the scalar offset.  Within a row the
// eight granules are permuted by an XOR of the row's low bits, so that the fragment reads
// (16 consecutive lanes: 16 consecutive rows, one granule each) fall in distinct 16-byte bank
// groups.  Rows past the problem read past their buffer resource, which writes zeros.
constexpr int kDR = 256;       // rows and columns per tile
constexpr int kDKS = 8;        // 16-byte granules per row per stage
constexpr int kDTLd = 129;     // epilogue transpose row stride in floats (128 columns + 1)

__device__ __forceinline__ int dma_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct HeadDmaLds {
  union {
    uint4 g[2][2][kDR * kDKS];      // [buffer][hidden rows = 0, head rows = 1][granule position]
    struct {
      float t[kWaves][32][kDTLd];   // one wave's 32 rows x 128 columns
      HeadRec part[2][kDR];         // per column half: each row's partials over its 128 columns
    } e;
  };
};
static_assert(sizeof(HeadDmaLds) <= 160 * 1024, "one workgroup per CU");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Loads i0 .. i0 + 3 of one stage: wave w fills granule positions 64 (8 w + i) + lane of both
// operands (row 64 w + 8 i + lane / 8, slot lane % 8, holding k granule slot ^ swz(row)); the
// lane's byte offsets within the tiles are va[i] and vb[i], the stage's k is the scalar offset.
__device__ __forceinline__ void dma_quarter(HeadDmaLds& L, int buf, int i0, __amdgpu_buffer_rsrc_t rsa,
                                            __amdgpu_buffer_rsrc_t rsb, const int (&va)[kDKS],
                                            const int (&vb)[kDKS], int koff, int wave_u) {
#pragma unroll
  for (int i = i0; i < i0 + 4; ++i) {
    const int p = 64 * (kDKS * wave_u + i);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)&L.g[buf][0][p], 16, va[i], koff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)&L.g[buf][1][p], 16, vb[i], koff, 0, 0);
  }
}

// s_waitcnt on the vector-memory counter alone (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// Fragments of k step h of a stage buffer (lane: row 32 i + lane % 32 of its 128-row half,
// granule 2 h + lane / 32).
__device__ __forceinline__ void sq_frags(const uint4* ga, const uint4* gb, int arow, int brow, int slot,
                                         bf16x8 (&fa)[4], bf16x8 (&fv)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = __builtin_bit_cast(bf16x8, ga[arow + 32 * kDKS * i + slot]);
#pragma unroll
  for (int j = 0; j < 4; ++j) fv[j] = __builtin_bit_cast(bf16x8, gb[brow + 32 * kDKS * j + slot]);
}

// One stage from buffer buf: step 0's fragment reads, then per k step sixteen MFMAs with the
// next step's eight reads between them.  With LOADS the next stage's sixteen loads go into the
// other buffer, half with step 0's reads and half between step 0's MFMAs.  Each step is a
// scheduling region of its own, so that no MFMA is placed right behind the read it needs.
template <bool LOADS>
__device__ __forceinline__ void sq_stage(HeadDmaLds& L, int buf, int arow, int brow, int hi, int sw,
                                         f32x16 (&acc)[4][4], __amdgpu_buffer_rsrc_t rsa,
                                         __amdgpu_buffer_rsrc_t rsb, const int (&va)[kDKS],
                                         const int (&vb)[kDKS], int koff, int wave_u) {
  const uint4* ga = L.g[buf][0];
  const uint4* gb = L.g[buf][1];
  bf16x8 fa[2][4], fv[2][4];
  sq_frags(ga, gb, arow, brow, hi ^ sw, fa[0], fv[0]);
  if (LOADS) dma_quarter(L, buf ^ 1, 0, rsa, rsb, va, vb, koff, wave_u);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < kDKS / 2; ++h) {
    const int cu = h & 1, nx = cu ^ 1;
    if (LOADS && h == 0) dma_quarter(L, buf ^ 1, 4, rsa, rsb, va, vb, koff, wave_u);
    if (h + 1 < kDKS / 2) sq_frags(ga, gb, arow, brow, (2 * (h + 1) + hi) ^ sw, fa[nx], fv[nx]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cu][i], fv[cu][j], acc[i][j], 0, 0, 0);
    if (h + 1 < kDKS / 2) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        if (LOADS && h == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_head_sq(HeadArgs a) {
  __shared__ HeadDmaLds L;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int rt = jx % a.n_rt, ct = (jx / a.n_rt) * 8 + xcd;
  if (ct >= a.n_ct) return;
  const int r0 = rt * kDR, v0 = ct * kDR;
  const __amdgpu_buffer_rsrc_t rsa = row_rsrc((const uint16_t*)a.hidden + (int64_t)r0 * a.h_ld,
                                             (int)(min(kDR, a.R - r0) * a.h_ld * 2));
  const __amdgpu_buffer_rsrc_t rsb = row_rsrc((const uint16_t*)a.weight + (int64_t)v0 * a.w_ld,
                                             (int)(min(kDR, a.V - v0) * a.w_ld * 2));
  int va[kDKS], vb[kDKS];
#pragma unroll
  for (int i = 0; i < kDKS; ++i) {
    const int r = 64 * wave + 8 * i + (lane >> 3), kg = (lane & 7) ^ dma_swz(r);
    va[i] = r * (int)a.h_ld * 2 + 16 * kg;
    vb[i] = r * (int)a.w_ld * 2 + 16 * kg;
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int n_k = a.D / (8 * kDKS);
  dma_quarter(L, 0, 0, rsa, rsb, va, vb, 0, wave);
  dma_quarter(L, 0, 4, rsa, rsb, va, vb, 0, wave);
  const int fr = lane & 31, hi = lane >> 5, sw = dma_swz(fr);
  const int arow = (128 * wr + fr) * kDKS, brow = (128 * wc + fr) * kDKS;
  for (int kt = 0; kt + 1 < n_k; ++kt) {
    // this wave's loads of stage kt have landed, and after the barrier everyone's; every wave
    // is also done with the other buffer, which the next stage's loads now fill
    wait_vm0();
    __syncthreads();
    sq_stage<true>(L, kt & 1, arow, brow, hi, sw, acc, rsa, rsb, va, vb, 2 * 8 * kDKS * (kt + 1), wave);
  }
  wait_vm0();
  __syncthreads();
  sq_stage<false>(L, (n_k - 1) & 1, arow, brow, hi, sw, acc, rsa, rsb, va, vb, 0, wave);
  __syncthreads();   // every wave is done with the stage buffers

  // Epilogue, per 32-row block: the wave's 32 x 128 logits go to its own LDS region by row;
  // lanes 2q and 2q + 1 take row q, 64 columns each.  Only this wave touches the region.
  const float c = a.c;
  const int cw0 = v0 + 128 * wc;     // the wave's first column
  const int hf = lane & 1, ri = lane >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 32 * j + fr;
      const bool in = cw0 + col < a.V;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * hi + (e & 3);
        L.e.t[wave][row][col] = in ? acc[i][j][e] : -INFINITY;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const float* x = &L.e.t[wave][ri][64 * hf];
    const int rl = 128 * wr + 32 * i + ri;     // row within the tile
    const int r = r0 + rl;
    if (a.tokens && r < a.R) {
      const int y = a.tokens[r] - (cw0 + 64 * hf);
      if (y >= 0 && y < 64 && cw0 + 64 * hf + y < a.V) a.ly[r] = x[y];
    }
    float m = -INFINITY;
    int am = INT_MAX, bad = 0;
#pragma unroll 16
    for (int q = 0; q < 64; ++q) {
      const float v = x[q];
      bad |= (v != v || v == INFINITY) ? 1 : 0;
      if (v > m) { m = v; am = q; }
    }
    am = m > -INFINITY ? cw0 + 64 * hf + am : INT_MAX;
    const float m2 = __shfl_xor(m, 1);
    const int am2 = __shfl_xor(am, 1);
    bad |= __shfl_xor(bad, 1);
    const float M = fmaxf(m, m2);
    int amx = INT_MAX;
    if (m == M) amx = am;
    if (m2 == M) amx = min(amx, am2);
    double s = 0.0, w = 0.0;
    if (!a.greedy && M > -INFINITY) {
#pragma unroll 16
      for (int q = 0; q < 64; ++q) {
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
      L.e.part[wc][rl] = pr;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // the two column halves of each row, folded in column order into the tile's record
  if (r0 + t < a.R) {
    const HeadRec p0 = L.e.part[0][t], p1 = L.e.part[1][t];
    const float M = fmaxf(p0.m, p1.m);
    HeadRec out;
    out.m = M;
    out.s = 0.0;
    out.w = 0.0;
    out.amax = -1;
    if (p0.m == M && p0.amax >= 0) out.amax = p0.amax;
    else if (p1.m == M && p1.amax >= 0) out.amax = p1.amax;
    if (!a.greedy && M > -INFINITY) {
      if (p0.m > -INFINITY) {
        const double d = ((double)p0.m - (double)M) * (double)c;
        const double f = exp2_split(d);
        out.s += p0.s * f;
        out.w += f * (p0.w + p0.s * d);
      }
      if (p1.m > -INFINITY) {
        const double d = ((double)p1.m - (double)M) * (double)c;
        const double f = exp2_split(d);
        out.s += p1.s * f;
        out.w += f * (p1.w + p1.s * d);
      }
    }
    if (p0.amax == -2 || p1.amax == -2) out.amax = -2;
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

// Benchmark instrumentation: the matrix cores' sustained rate on the head kernel's pattern
// (per wave, 4 x 4 independent 32x32x16 bf16 MFMAs per step, operands in registers, no memory
// traffic).  mode 0: every operand 1.0; mode 1: random bf16 (exponents 121-128, random sign and
// mantissa, from a per-lane linear congruential sequence), the same every step; mode 2: those
// operands with mantissa bits flipped every step, so the multipliers' inputs change from one
// MFMA to the next as a real product's do.  The accumulators' sum goes to *sink only if it is
// exactly 2^127, which keeps the work from being dropped.
__device__ __forceinline__ uint32_t lcg_next(uint32_t& x) {
  x = x * 1664525u + 1013904223u;
  return x;
}
__device__ __forceinline__ uint32_t rand_bf16_pair(uint32_t& x) {
  const uint32_t h = lcg_next(x) ^ (lcg_next(x) >> 13);
  const uint32_t lo = (h & 0x807fu) | ((121u + ((h >> 8) & 7u)) << 7);
  const uint32_t hi = ((h >> 16) & 0x807fu) | ((121u + ((h >> 24) & 7u)) << 7);
  return lo | (hi << 16);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_mfma_rate(int mode, int iters,
                                                                                                 float* sink) {
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  uint4 ra[4], rb[4];
  uint32_t x = (blockIdx.x * kThreads + threadIdx.x) * 2654435761u + 12345u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (mode == 0) {
      ra[i] = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
      rb[i] = ra[i];
    } else {
      ra[i].x = rand_bf16_pair(x); ra[i].y = rand_bf16_pair(x); ra[i].z = rand_bf16_pair(x); ra[i].w = rand_bf16_pair(x);
      rb[i].x = rand_bf16_pair(x); rb[i].y = rand_bf16_pair(x); rb[i].z = rand_bf16_pair(x); rb[i].w = rand_bf16_pair(x);
    }
  }
  const uint32_t flip = mode == 2 ? 0x002a0055u : 0u;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ra[i]),
                                                            __builtin_bit_cast(bf16x8, rb[j]), acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i].x ^= flip; ra[i].y ^= flip; ra[i].z ^= flip; ra[i].w ^= flip;
      rb[i].x ^= flip; rb[i].y ^= flip; rb[i].z ^= flip; rb[i].w ^= flip;
    }
  }
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) z += acc[i][j][e];
  if (z == 0x1.0p+127f) *sink = z;
}

hipError_t launch_mfma_rate(int mode, int iters, int workgroups, float* sink, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
  launch_timed(k_mfma_rate, dim3((unsigned)workgroups), dim3(kThreads), st, ev0, ev1, mode, iters, sink);
  return hipGetLastError();
}

hipError_t launch_head(const HeadArgs& a0, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  HeadArgs a = a0;
  if (a.R > 128 && a.D % (8 * kDKS) == 0) {
    a.n_rt = (a.R + kDR - 1) / kDR;
    const long long grid = (long long)a.n_rt * ((a.n_ct + 7) / 8) * 8;
    if (grid < 1 || grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
    launch_timed(k_head_sq, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_head_combine, dim3((unsigned)((a.R + kWaves - 1) / kWaves)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
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
