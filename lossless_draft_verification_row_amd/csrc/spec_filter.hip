// spec_filter.hip -- verification with top-k / top-p filtered distributions.
//
// With top-k on (1 <= k <= 256), every filtered distribution lives on the k largest logits of
// its row (ties at the boundary kept, reading R1 of the oracle), so after one streaming pass the
// whole method runs on small sparse sets:
//   k_filt_slices   one workgroup per candidate list: two 4096-logit chunks of a bf16 target row
//                   (one chunk of an fp32 row) and, for a paired position, the same chunks of its
//                   draft row.  The list's threshold is the k-th largest of its 256 per-thread
//                   maxima (an LDS histogram; an exact radix select over the list when they
//                   spread wider); every logit at or above it is a candidate, written as one
//                   32-bit word (bf16: raw bits, valid bit, offset in the list) or a
//                   {value, index} pair (fp32).  Each needed logit is read once; nothing waits
//                   on another workgroup.
//   k_filt_rows_w   bf16 rows, one wave per row: the row's k-th largest among its lists'
//                   candidates, the top-k set K, top-p on the renormalised K from per-key counts
//                   (or pairwise masses when K spreads wider), the kept set S with p = e / Z_S in
//                   fp64 in index order, entropy in bits, max probability, log Z (guide page
//                   "5.1 投机解码核心原理" §2.1: p and q are the distributions after temperature,
//                   top-k, top-p; SpecKV page signals).  k_filt_rows does the same for fp32
//                   rows, one workgroup per row.
//   k_filt_finalize one workgroup per request: p(y), q(y), 1 - TV = sum min(p, q) (§4.1, §4.3),
//                   the accept scan (§3.2, §5.1) and the three-level sampler over the residual
//                   [p - q]_+ or p_{g+1} (§3.2, §5.2) on the sparse kept sets, with the
//                   sampler's sequential fp64 sums taken in index order.
// A list keeps at most `cap` candidates, those strictly above its threshold first; if it had
// to drop ties that the row's own threshold would keep, or a row's top-k set exceeds kKeepMax,
// the request (or plain row) is listed for the dense threshold path, which recomputes all its
// outputs after these kernels (spec_kernels.hip, k_fb_rows and k_fb_requests / k_fb_residual).
#include "spec_device.h"
#include "spec_internal.h"

namespace specv {

constexpr int kFlagBad = 1;        // a NaN or +inf logit in the row
constexpr int kFlagOverflow = 2;   // the sparse sets could not hold the row
constexpr int kFlagEmpty = 4;      // no finite logit in the row

// The top 8 * NPASS bits of a key, right-aligned: for bf16 logits (NPASS = 2) they fix the
// value, for fp32 (NPASS = 4) they are the key.
template <int NPASS>
__device__ __forceinline__ uint32_t key_hi(uint32_t k) {
  return NPASS == 4 ? k : (k >> (32 - 8 * NPASS));
}

// Block-wide: the top 8 * NPASS bits of the k-th largest key among the valid keys (with
// multiplicity).  for_each(cb) calls cb(key, valid) for every key this thread holds.  `all`
// is set when fewer than k keys are valid (every valid key then qualifies).
template <int NPASS, typename ForEach>
__device__ uint32_t block_select(int k, SelLds& S, ForEach for_each, bool& all, int& n_valid) {
  const int t = threadIdx.x;
  uint32_t prefix = 0;
  int kk = k;
  all = false;
  n_valid = 0;
#pragma unroll 1
  for (int pass = 0; pass < NPASS; ++pass) {
    const int sh = 8 * (NPASS - 1 - pass);   // digit position within key_hi
    S.hist[t] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, bool valid) {
      const uint32_t h = key_hi<NPASS>(key);
      if (valid && (pass == 0 || (h >> (sh + 8)) == prefix)) atomicAdd(&S.hist[(h >> sh) & 255u], 1u);
    });
    __syncthreads();
    select_digit(S, kk);
    __syncthreads();
    const int d = S.digit;
    if (pass == 0) n_valid = S.total;
    __syncthreads();
    if (d < 0) { all = true; return 0u; }
    prefix = (prefix << 8) | (uint32_t)d;
    kk -= S.above;
  }
  return prefix;
}

// Exclusive block scan of two counters; returns the totals through a and b.
__device__ __forceinline__ void block_scan2(int& a, int& b, SelLds& S, int& ta, int& tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_incl_scan_i(a), ib = wave_incl_scan_i(b);
  if (lane == 63) { S.wtot[0][wave] = ia; S.wtot[1][wave] = ib; }
  __syncthreads();
  int oa = 0, ob = 0;
  ta = 0; tb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) { oa += S.wtot[0][w]; ob += S.wtot[1][w]; }
    ta += S.wtot[0][w];
    tb += S.wtot[1][w];
  }
  a = oa + ia - a;
  b = ob + ib - b;
  __syncthreads();
}

// ---------------------------------------------------------------- k_filt_slices

// A bf16 list's candidate as one 32-bit word: the raw bf16 bits of its value in the high half,
// bit 15 set, and its offset within the list's 8192 logits (lists start at multiples of 8192)
// in the low 13 bits.  The row kernel turns the bits into an order key; the streaming kernel,
// where a candidate's word takes whole issue slots for a few lanes, only ORs the parts.
__device__ __forceinline__ uint32_t list_word(float v, int x) {
  return __float_as_uint(v) | 0x8000u | ((uint32_t)x & 0x1FFFu);
}


// Candidates of one row's slice: the values at or above the slice's k-th largest, the ones
// strictly above first.  Header {stored, total, threshold digits, flags}.
// `v(j)` gives this thread's j-th logit of the list (j < N), `idx(j)` its token index.
// `bad` < 0: find whether the list holds a NaN or +inf here; else that flag, already known.
template <int DT, int N, int U, typename Get, typename Idx>
__device__ void slice_candidates_g(const FilterArgs& a, SelLds& S, Get v, Idx idx, int slot, int l, int bad = -1) {
  constexpr int NP = DT == kDtBF16 ? 2 : 4;
  const int t = threadIdx.x;
  if (bad < 0) {
    bad = 0;
#pragma unroll U
    for (int j = 0; j < N; ++j) bad |= __builtin_amdgcn_class(v(j), 0x203) ? 1 : 0;   // NaN, +inf
    bad = block_or(bad, S.wtot[0]);
  }
  auto valid = [](float x) { return x > -INFINITY && x < INFINITY; };
  bool all;
  int nv;
  const uint32_t th = block_select<NP>(a.k, S,
                                       [&](auto cb) {
#pragma unroll U
                                         for (int j = 0; j < N; ++j) {
                                           const float x = v(j);
                                           cb(order_key(x), valid(x));
                                         }
                                       }, all, nv);
  int ng = 0, ne = 0;
#pragma unroll U
  for (int j = 0; j < N; ++j) {
    const float x = v(j);
    if (!valid(x)) continue;
    const uint32_t h = key_hi<NP>(order_key(x));
    if (all || h > th) ++ng;
    else if (h == th) ++ne;
  }
  int og = ng, oe = ne, tg, te;
  block_scan2(og, oe, S, tg, te);
  const int cap = a.cap;
  const int64_t lo = ((int64_t)slot * a.n_l + l) * cap;
#pragma unroll U
  for (int j = 0; j < N; ++j) {
    const float x = v(j);
    if (!valid(x)) continue;
    const uint32_t h = key_hi<NP>(order_key(x));
    int pos = -1;
    if (all || h > th) pos = og++;
    else if (h == th) pos = tg + oe++;
    if (pos >= 0 && pos < cap) {
      if constexpr (DT == kDtBF16) {
        ((uint32_t*)a.cand)[lo + pos] = list_word(x, idx(j));
      } else {
        CandEntry c;
        c.v = x;
        c.x = idx(j);
        a.cand[lo + pos] = c;
      }
    }
  }
  if (t == 0) {
    CandHead hd;
    hd.total = tg + te;
    hd.stored = min(tg + te, cap);
    hd.th = all ? 0u : th;
    hd.flags = (bad ? kFlagBad : 0) | (all ? 8 : 0);
    a.chead[(int64_t)slot * a.n_l + l] = hd;
  }
  __syncthreads();
}

template <int DT>
__device__ void slice_candidates(const FilterArgs& a, SelLds& S, const float (&v)[kPerThread], int slot, int s,
                                 int base) {
  const int t = threadIdx.x;
  slice_candidates_g<DT, kPerThread, kPerThread>(a, S, [&](int j) { return v[j]; },
                                     [&](int j) { return slice_index<DT>(base, t, j); }, slot, s);
}

// Mask of the wave's lanes with x >= y, straight from the compare into a scalar register pair
// (one instruction; the wave is whole here, so it is the ballot).  Opaque to the compiler, so
// it is formed where it is used rather than carried across a barrier.
__device__ __forceinline__ unsigned long long wave_mask_ge(float x, float y) {
  unsigned long long m;
  asm volatile("v_cmp_ge_f32_e64 %0, %1, %2" : "=s"(m) : "v"(x), "v"(y));
  return m;
}

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0xb1, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x4e, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x124, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x128, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

constexpr int kTop2K = 128;    // above this k a list's threshold counts each thread's two largest values
constexpr int kStageW = 512;   // candidates one wave may stage per row of a list (shares LDS with raw)

struct ListLds {
  uint32_t hist[2][256];   // per row: count of per-thread maxima at order key max - b, b = 0..255
  int wmax[2][kWaves], wbad[2][kWaves];
  int wcnt[2][kWaves];
  int tau[2], fb[2];
  SelLds gen;              // the general select, for a list whose top k spread wider
  union {
    uint32_t stage[2][kWaves][kStageW];       // each wave's candidates of each row, before the copy out
    uint32_t raw[kPerThread][kThreads];       // the exact select's raw bf16 pairs, thread t's in column t
  };
};

// Order key of a bf16-exact value (16 significant bits) and back.
__device__ __forceinline__ int key16(float v) {
  uint32_t b = __float_as_uint(v) >> 16;
  if (b == 0x8000u) b = 0u;
  return (int)((b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u));
}

// Logit j (< 2 kPerThread) of a thread's bf16 list of two 4096-logit chunks held as raw words,
// and its token index.
__device__ __forceinline__ float list_elem(const RawSlice<kDtBF16> (&r)[2], int j) {
  const uint32_t w = r[j / kPerThread].w[(j % kPerThread) >> 1];
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}
// The same logit unpacked by an opaque move, so that the compiler does not keep the unpacked
// values of an earlier pass alive (the raw words take half the registers).
__device__ __forceinline__ float list_elem_fresh(const RawSlice<kDtBF16> (&r)[2], int j) {
  const uint32_t w = r[j / kPerThread].w[(j % kPerThread) >> 1];
  uint32_t x;
  if (j & 1) asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(x) : "v"(w));
  else asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(x) : "v"(w));
  return __uint_as_float(x);
}
__device__ __forceinline__ int list_index(int base, int t, int j) {
  return slice_index<kDtBF16>(base + (j / kPerThread) * kChunk, t, j % kPerThread);
}
// Raw bf16 halves at indices >= V become -inf (0xFF80): a bounds-checked vector load returns
// zeros past the row.
__device__ __forceinline__ void mask_tail_words(int V, int base, RawSlice<kDtBF16>& r) {
  const int t = threadIdx.x;
  if (base + kChunk <= V) return;
#pragma unroll
  for (int k = 0; k < kPerThread / 2; ++k) {
    const int i0 = slice_index<kDtBF16>(base, t, 2 * k);
    if (i0 >= V) r.w[k] = (r.w[k] & 0xFFFF0000u) | 0xFF80u;
    if (i0 + 1 >= V) r.w[k] = (r.w[k] & 0x0000FFFFu) | 0xFF800000u;
  }
}

// Candidates of one list of a bf16 target row and (paired) the same list of its draft row: two
// 4096-logit chunks, 32 logits per thread per row, both rows in lockstep.  The k-th largest of
// the 256 per-thread maxima (for k above kTop2K, of the 512 values that are each thread's two
// largest) is at most the list's k-th largest logit, so every finite logit at or above it is a
// valid candidate set (it holds the list's top k with all ties); for a realistic row it is
// not much larger than k.  That threshold comes from one LDS histogram of the
// maxima within 256 order keys of the list maximum (one or two atomics per thread).  Each wave then
// stages its candidates in its own LDS region in one compare pass (wave counts by popcount,
// slots by mbcnt, elements no lane keeps skipped), and the regions are copied out whole.  A row
// whose maxima spread wider, or whose candidates fill a region or the list's `cap`, takes the
// exact radix select instead, on the list read again from memory.
template <bool VEC>
__device__ void list_candidates_bf16(const FilterArgs& a, ListLds& S, const RawSlice<kDtBF16> (&rp)[2],
                                     const RawSlice<kDtBF16> (&rq)[2], bool paired, int slot_p, int slot_q, int l,
                                     int base, const void* row_p, const void* row_q) {
  constexpr int NE = 2 * kPerThread;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nrow = paired ? 2 : 1;
  // per-thread maxima with NaN propagated: a NaN or +inf anywhere makes the maximum NaN or
  // +inf, which flags the row (its candidates are then never read)
  float fm[2] = {-INFINITY, -INFINITY};
  // above kTop2K each thread also gives its second largest, so that k counts against 512
  // values: the k-th largest of the 256 maxima alone is their smallest at k = 256, far down the
  // list, and its candidates would overflow the list's slots
  float f2[2] = {-INFINITY, -INFINITY};
  const bool top2 = a.k > kTop2K;
  int bad[2];
  if (top2) {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const float v = list_elem(rp, j);
      f2[0] = fmaxf(f2[0], fminf(fm[0], v));
      fm[0] = __builtin_elementwise_maximum(fm[0], v);
      if (paired) {
        const float w = list_elem(rq, j);
        f2[1] = fmaxf(f2[1], fminf(fm[1], w));
        fm[1] = __builtin_elementwise_maximum(fm[1], w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      fm[0] = __builtin_elementwise_maximum(fm[0], list_elem(rp, j));
      if (paired) fm[1] = __builtin_elementwise_maximum(fm[1], list_elem(rq, j));
    }
  }
  int tm[2], t2[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    bad[r] = fm[r] < INFINITY ? 0 : 1;
    tm[r] = (fm[r] > -INFINITY && fm[r] < INFINITY) ? key16(fm[r]) : -1;
    t2[r] = (top2 && f2[r] > -INFINITY && f2[r] < INFINITY) ? key16(f2[r]) : -1;
  }
  S.hist[0][t] = 0u;
  S.hist[1][t] = 0u;
  int mx[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    mx[r] = wave_max_i(tm[r]);
    bad[r] = wave_or(bad[r]);
    if (lane == 0) { S.wmax[r][wave] = mx[r]; S.wbad[r][wave] = bad[r]; }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    int m = -1, bd = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { m = max(m, S.wmax[r][w]); bd |= S.wbad[r][w]; }
    mx[r] = m;
    bad[r] = bd;
    if (tm[r] >= 0 && m - tm[r] < 256) atomicAdd(&S.hist[r][m - tm[r]], 1u);
    if (t2[r] >= 0 && m - t2[r] < 256) atomicAdd(&S.hist[r][m - t2[r]], 1u);
  }
  __syncthreads();
  // wave r: the k-th largest per-thread maximum of row r (bins ascend from the maximum)
  if (wave < nrow) {
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { c[q] = (int)S.hist[wave][4 * lane + q]; sum += c[q]; }
    const int incl = wave_incl_scan_i(sum);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const unsigned long long hit = __ballot(incl >= a.k);
    if (lane == 0) { S.fb[wave] = (total < a.k) ? 1 : 0; S.tau[wave] = 0; }
    if (hit && total >= a.k) {
      const int Lh = __builtin_ctzll(hit);
      if (lane == Lh) {
        int run = incl - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (run + c[q] >= a.k) { S.tau[wave] = mx[wave] - (4 * lane + q); break; }
          run += c[q];
        }
      }
    }
  }
  __syncthreads();
  float tf[2];
  int fb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    fb[r] = r < nrow ? S.fb[r] : 1;
    tf[r] = fb[r] ? INFINITY : key16_value(S.tau[r]);
  }
  // candidates: the logits at or above the threshold value (NaN compares false; a +inf only
  // occurs in a flagged row), staged by each wave in its own region in one pass
  auto stage_row = [&](const RawSlice<kDtBF16> (&rw)[2], int r) {
    uint32_t* st = S.stage[r][wave];
    int run = 0;   // uniform over the wave
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const float v = list_elem_fresh(rw, j);
      const unsigned long long mk = wave_mask_ge(v, tf[r]);
      if (mk) {
        if (__builtin_amdgcn_inverse_ballot_w64(mk)) {
          const int o = run + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mk >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((unsigned)mk, 0u));
          if (o < kStageW) st[o] = __float_as_uint(v) | 0x8000u | (uint32_t)list_index(0, t, j);   // list_word
        }
        run += __popcll(mk);
      }
    }
    return run;
  };
  int wc0 = 0, wc1 = 0;
  if (!fb[0]) wc0 = stage_row(rp, 0);
  if (!fb[1]) wc1 = stage_row(rq, 1);
  if (lane == 0) { S.wcnt[0][wave] = wc0; S.wcnt[1][wave] = wc1; }
  __syncthreads();
  const int cap = a.cap;
  int tot[2], o1[2], o2[2], o3[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int c0 = S.wcnt[r][0], c1 = S.wcnt[r][1], c2 = S.wcnt[r][2], c3 = S.wcnt[r][3];
    o1[r] = c0;
    o2[r] = c0 + c1;
    o3[r] = c0 + c1 + c2;
    tot[r] = o3[r] + c3;
    if (tot[r] > cap || max(max(c0, c1), max(c2, c3)) > kStageW) fb[r] = 1;
  }
  // the staged rows go out whole
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r >= nrow || fb[r]) continue;
    const int slot = r == 0 ? slot_p : slot_q;
    uint32_t* out = (uint32_t*)a.cand + ((int64_t)slot * a.n_l + l) * cap;
    for (int e = t; e < tot[r]; e += kThreads) {
      const int w = (e >= o1[r]) + (e >= o2[r]) + (e >= o3[r]);
      const int wo = w == 0 ? 0 : (w == 1 ? o1[r] : (w == 2 ? o2[r] : o3[r]));
      out[e] = S.stage[r][w][e - wo];
    }
    if (t == 0) {
      CandHead hd;
      hd.total = tot[r];
      hd.stored = tot[r];
      hd.th = (uint32_t)S.tau[r];
      hd.flags = bad[r] ? kFlagBad : 0;
      a.chead[(int64_t)slot * a.n_l + l] = hd;
    }
  }
  if (!fb[0] && (nrow < 2 || !fb[1])) return;
  // the exact select for the other rows: the list's own k-th largest, ties after the larger
  // values, on the list read again (its raw words go to LDS over the staging area, once every
  // copy out has read it; each thread reads back only its own words)
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (r >= nrow || !fb[r]) continue;
    const int slot = r == 0 ? slot_p : slot_q;
    RawSlice<kDtBF16> raw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (VEC) load_raw_buf<kDtBF16>(row_rsrc(r == 0 ? row_p : row_q, a.V * 2), base + h * kChunk, raw[h]);
      else load_raw<kDtBF16, false>(r == 0 ? row_p : row_q, a.V, base + h * kChunk, raw[h]);
      mask_tail_words(a.V, base + h * kChunk, raw[h]);
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) S.raw[k][t] = raw[k / (kPerThread / 2)].w[k % (kPerThread / 2)];
    slice_candidates_g<kDtBF16, NE, 2>(
        a, S.gen,
        [&](int j) {
          const uint32_t w = *(volatile uint32_t*)&S.raw[j >> 1][t];   // read at each use
          return (j & 1) ? bf16_hi(w) : bf16_lo(w);
        },
        [&](int j) { return list_index(base, t, j); }, slot, l, bad[r]);
  }
}

template <int DT, bool VEC, bool PAIRED>
__global__ __launch_bounds__(kThreads) void k_filt_slices(FilterArgs a) {
  __shared__ ListLds S;
  // one workgroup per candidate list: two 4096-logit chunks (bf16) or one (fp32)
  constexpr int kSpan = DT == kDtBF16 ? 2 : 1;
  const int n_l = a.n_l;
  const int r = blockIdx.x / n_l, l = blockIdx.x - (blockIdx.x / n_l) * n_l;
  // the dense recomputation's list starts empty and the offsets valid (the finalize checks them)
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (a.ovf_n) *a.ovf_n = 0;
    if (a.cu_bad0) *a.cu_bad0 = 0;
  }
  if (r >= a.n_teams) return;
  constexpr int kEsz = DT == kDtBF16 ? 2 : 4;
  const int base = l * kSpan * kChunk;
  RawSlice<DT> rp[kSpan], rq[kSpan];
  {
    const void* row = row_ptr<DT>(a.tgt, a.tgt_ld, r);
#pragma unroll
    for (int h = 0; h < kSpan; ++h) {
      if (VEC) load_raw_buf<DT>(row_rsrc(row, a.V * kEsz), base + h * kChunk, rp[h]);
      else load_raw<DT, false>(row, a.V, base + h * kChunk, rp[h]);
    }
  }
  auto load_q = [&](int drow) {
    const void* row = drow >= 0 ? row_ptr<DT>(a.drf, a.drf_ld, drow) : a.tgt;
#pragma unroll
    for (int h = 0; h < kSpan; ++h) {
      if (VEC) load_raw_buf<DT>(row_rsrc(row, drow >= 0 ? a.V * kEsz : 0), base + h * kChunk, rq[h]);
      else if (drow >= 0) load_raw<DT, false>(row, a.V, base + h * kChunk, rq[h]);
    }
  };
  // the draft row of target row r, if r is not the last row of its request (scalar-cache
  // binary search over the offsets; the draft loads go out right after)
  int drow = -1;
  if (PAIRED && a.direct) {
    if (r < a.n_draft_rows) drow = r;
    load_q(drow);
  } else if (PAIRED) {
    // the request guessed as b = r / (G + 1) (exact when every request has G draft tokens):
    // its draft row is loaded at once, one scalar load checks the guess, and a wrong guess
    // falls back to a binary search over the offsets and loads again
    const int lo0 = min(r / (a.G + 1), a.B - 1);
    const bool guess_pair = r - lo0 < a.n_draft_rows && r % (a.G + 1) < a.G;
    if (VEC) load_q(guess_pair ? r - lo0 : -1);
    int lo = lo0, c0, c1;
    sload2_i32(a.cu + lo, c0, c1);
    if (!(c0 + lo <= r && (lo == a.B - 1 || c1 + lo + 1 > r))) {
      lo = 0;
      int hi = a.B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sload_i32(a.cu + mid) + mid <= r) lo = mid;
        else hi = mid;
      }
      sload2_i32(a.cu + lo, c0, c1);
    }
    const int i = r - c0 - lo;
    if (i >= 0 && i < c1 - c0 && r - lo >= 0 && r - lo < a.n_draft_rows) drow = r - lo;
    if (VEC) {
      if ((drow >= 0) != guess_pair || (drow >= 0 && lo != lo0)) load_q(drow);
    } else if (drow >= 0) {
      load_q(drow);
    }
  }
  const bool paired = PAIRED && drow >= 0;
  if constexpr (DT == kDtBF16) {
    if (VEC) {
#pragma unroll
      for (int h = 0; h < kSpan; ++h) {
        mask_tail_words(a.V, base + h * kChunk, rp[h]);
        if (paired) mask_tail_words(a.V, base + h * kChunk, rq[h]);
      }
    }
    if (!paired) {
#pragma unroll
      for (int h = 0; h < kSpan; ++h)
#pragma unroll
        for (int k = 0; k < kPerThread / 2; ++k) rq[h].w[k] = 0xFF80FF80u;
    }
    list_candidates_bf16<VEC>(a, S, rp, rq, paired, r, a.n_teams + drow, l, base, row_ptr<DT>(a.tgt, a.tgt_ld, r),
                              paired ? row_ptr<DT>(a.drf, a.drf_ld, drow) : a.tgt);
  } else {
    float vp[kPerThread], vq[kPerThread];
    unpack_raw<DT>(rp[0], vp);
    if (VEC && (a.V % kChunk) != 0 && l == n_l - 1) mask_tail<DT>(a.V, base, vp);
    slice_candidates<DT>(a, S.gen, vp, r, l, base);
    if (paired) {
      unpack_raw<DT>(rq[0], vq);
      if (VEC && (a.V % kChunk) != 0 && l == n_l - 1) mask_tail<DT>(a.V, base, vq);
      slice_candidates<DT>(a, S.gen, vq, a.n_teams + drow, l, base);
    }
  }
}

// ---------------------------------------------------------------- k_filt_rows

constexpr int kRowStage = 1280;   // candidates of a row staged in LDS (more: read in place); 16 KB of
                                  // LDS in all, so eight rows share a CU

// Partial sums per wave of the kept-set steps, in the staging area beside e and keep.
constexpr int kPartJ = (kRowStage * 8 - kKeepMax * 12) / (kWaves * 8);

struct RowLds {
  SelLds sel;
  int cnt[kMaxSlicesFused + 1];
  int off[kMaxSlicesFused + 1];
  union {
    alignas(16) CandEntry cand[kRowStage];   // the staged candidates, until the kept set is compacted
    struct {
      double ke[kKeepMax];                   // then the kept set's e-values,
      int keep[kKeepMax];                    // keep flags / ranks
      double part[kWaves][kPartJ];           // and the waves' partial sums
    } k;
  };
  float kv[kKeepMax];
  int kx[kKeepMax];
  double red[kWaves];
  int flags, nk, ns;
};
static_assert(sizeof(CandEntry) == 8 && kPartJ >= 64, "the kept-set scratch fits the staging area");

__device__ __forceinline__ double block_sum_dd(double v, double* red) {
  v = wave_sum_dpp_d(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  __syncthreads();
  return s;
}

// One row: global top-k over the slices' candidates, top-p, the kept set with probabilities.
template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_filt_rows(FilterArgs a) {
  static_assert(DT == kDtF32, "bf16 rows go to k_filt_rows_w (their lists hold 32-bit words)");
  constexpr int NP = DT == kDtBF16 ? 2 : 4;
  __shared__ RowLds L;
  const int t = threadIdx.x, lane = t & 63;
  const int slot = blockIdx.x;
  if (slot >= a.n_slots) return;
  const int n_s = a.n_l, cap = a.cap;   // candidate lists of the row
  const CandHead* hd = a.chead + (int64_t)slot * n_s;
  const CandEntry* cd = a.cand + (int64_t)slot * n_s * cap;
  // the first 64 candidates of each wave's first two lists go out with the headers (every
  // list has cap slots; entries past its count are never used)
  const int wv = t >> 6;
  CandEntry pre[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sl = wv + u * kWaves;
    if (sl < n_s && lane < cap) pre[u] = cd[(int64_t)sl * cap + lane];
  }
  // list headers, one per lane of wave 0; prefix of the stored counts
  CandHead h;
  h.stored = 0; h.total = 0; h.th = 0u; h.flags = 0;
  if (t < n_s) h = hd[t];
  if (t < 64) {
    const int inc = wave_incl_scan_i(h.stored);
    const int fl = wave_or(h.flags & kFlagBad);
    if (t < n_s) { L.cnt[t] = h.stored; L.off[t] = inc - h.stored; }
    if (t == 63) { L.off[n_s] = inc; L.flags = fl; }
  }
  __syncthreads();
  const int n = L.off[n_s];
  const bool staged = n <= kRowStage;
  // slice of candidate j: off[s] <= j < off[s + 1]
  auto slice_of = [&](int j) {
    int lo = 0, hi = n_s;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (L.off[mid] <= j) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  // bf16: the largest order key among the candidates, formed while they are copied in
  int km = -1;
  if (staged) {
    // copy the candidates in: wave w takes lists w, w + 4, ..., lane l entries l and l + 64
    // of each; four lists per wave (eight loads per thread) in flight at a time, the first
    // two already read
    for (int i0 = 0; i0 < cap; i0 += 128) {
      for (int s0 = wv; s0 < n_s; s0 += kWaves * 4) {
        CandEntry tmp[4][2];
        const bool first = i0 == 0 && s0 == wv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sl = s0 + u * kWaves;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int idx = i0 + lane + 64 * h;
            if (first && h == 0 && u < 2) tmp[u][h] = pre[u];
            else if (sl < n_s && idx < L.cnt[sl]) tmp[u][h] = cd[(int64_t)sl * cap + idx];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sl = s0 + u * kWaves;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int idx = i0 + lane + 64 * h;
            if (sl < n_s && idx < L.cnt[sl]) {
              L.cand[L.off[sl] + idx] = tmp[u][h];
              if (NP == 2) km = max(km, (int)key_hi<2>(order_key(tmp[u][h].v)));
            }
          }
        }
      }
    }
    __syncthreads();
  }
  auto at = [&](int j) -> CandEntry {
    if (staged) return L.cand[j];
    const int sl = slice_of(j);
    return cd[(int64_t)sl * cap + (j - L.off[sl])];
  };
  bool all = false;
  int nv;
  uint32_t th = 0u;
  bool done = false;
  if (NP == 2) {
    // bf16: one LDS histogram of the candidate keys within 256 of the maximum (one key per
    // bin) gives the exact k-th largest when the top k lie in that window
    if (!staged)
      for (int j = t; j < n; j += kThreads) km = max(km, (int)key_hi<2>(order_key(at(j).v)));
    L.sel.hist[t] = 0u;
    km = wave_max_i(km);
    if (lane == 0) L.sel.wtot[0][t >> 6] = km;
    __syncthreads();
    km = max(max(L.sel.wtot[0][0], L.sel.wtot[0][1]), max(L.sel.wtot[0][2], L.sel.wtot[0][3]));
    for (int j = t; j < n; j += kThreads) {
      const int d = km - (int)key_hi<2>(order_key(at(j).v));
      if (d < 256) atomicAdd(&L.sel.hist[d], 1u);
    }
    __syncthreads();
    if (t < 64) {
      int c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = (int)L.sel.hist[4 * lane + q]; sum += c[q]; }
      const int incl = wave_incl_scan_i(sum);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      const unsigned long long hit = __ballot(incl >= a.k);
      if (lane == 0) L.sel.digit = -1;
      if (hit && total >= a.k) {
        const int Lh = __builtin_ctzll(hit);
        if (lane == Lh) {
          int run = incl - sum;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (run + c[q] >= a.k) { L.sel.digit = km - (4 * lane + q); break; }
            run += c[q];
          }
        }
      }
    }
    __syncthreads();
    if (L.sel.digit >= 0) { th = (uint32_t)L.sel.digit; done = true; }
    __syncthreads();
  }
  if (!done)
    th = block_select<NP>(a.k, L.sel,
                          [&](auto cb) {
                            for (int j = t; j < n; j += kThreads) cb(order_key(at(j).v), true);
                          }, all, nv);
  // dropped ties of a slice hold its threshold digits; they belong to K if those reach th
  if (t < n_s && h.total > h.stored && (all || h.th >= th)) atomicOr(&L.flags, kFlagOverflow);
  // the top-k set K, compacted in candidate order
  int mine = 0;
  for (int j = t; j < n; j += kThreads) mine += (all || key_hi<NP>(order_key(at(j).v)) >= th) ? 1 : 0;
  int o = mine, dummy = 0, nk, tz;
  block_scan2(o, dummy, L.sel, nk, tz);
  if (nk > kKeepMax) { if (t == 0) atomicOr(&L.flags, kFlagOverflow); }
  else {
    for (int j = t; j < n; j += kThreads) {
      const CandEntry c = at(j);
      if (all || key_hi<NP>(order_key(c.v)) >= th) { L.kv[o] = c.v; L.kx[o] = c.x; ++o; }
    }
  }
  __syncthreads();
  // The kept set (at most kKeepMax entries) is in LDS.  Wave 0 takes the maximum and the
  // e-values; the quadratic top-p and rank sums are spread over the four waves (wave w takes
  // every fourth entry y), their partials meeting in LDS (the e-values, flags and partials use
  // the staging area, free again); wave 0 then forms Z_S, p, entropy and writes the kept set in
  // index order.
  const int wave = t >> 6;
  RowStat2 st;
  st.n = 0; st.flags = L.flags; st.m = -INFINITY; st.argmax = -1; st.kept_finite = 0; st.pad = 0;
  st.log_z = 0.0; st.entropy = 0.0; st.max_prob = 0.0; st.z = 0.0;
  if (nk == 0 && !(st.flags & kFlagBad)) st.flags |= kFlagEmpty;
  if (st.flags) {
    if (t == 0) a.rstat[slot] = st;
    return;
  }
  float m = -INFINITY;
  int amx = INT_MAX;
  if (wave == 0) {
    // maximum (lowest index among equal maxima)
    for (int j = lane; j < nk; j += 64) m = fmaxf(m, L.kv[j]);
    m = wave_max_dpp(m);
    for (int j = lane; j < nk; j += 64) if (L.kv[j] == m) amx = min(amx, L.kx[j]);
    amx = wave_min_i(amx);
    // e = exp((l - m) / T) in fp64; Z_K
    const double cd2 = (double)a.c;   // log2(e) / T
    double zk = 0.0;
    for (int j = lane; j < nk; j += 64) {
      const double e = exp2_split(((double)L.kv[j] - (double)m) * cd2);
      L.k.ke[j] = e;
      zk += e;
    }
    zk = wave_sum_dpp_d(zk);
    if (lane == 0) L.red[0] = zk;
  }
  __syncthreads();
  const double zk = L.red[0];
  double* part = &L.k.part[0][0];
  int* ipart = (int*)&L.k.part[0][0];
  // top-p: keep x iff the mass of values strictly above l_x is below top_p (the value group
  // that first reaches top_p is kept whole; reading R1); keep[j] = 1 for a kept entry
  for (int j0 = 0; j0 < nk; j0 += kPartJ) {
    const int j1 = min(nk, j0 + kPartJ);
    if (a.top_p < 1.f) {
      for (int j = j0 + lane; j < j1; j += 64) {
        const float lx = L.kv[j];
        double ab = 0.0;
        for (int y = wave; y < nk; y += kWaves) ab += (L.kv[y] > lx) ? L.k.ke[y] : 0.0;
        part[wave * kPartJ + (j - j0)] = ab;
      }
      __syncthreads();
      for (int j = j0 + t; j < j1; j += kThreads) {
        const int i = j - j0;
        const double above = ((part[i] + part[kPartJ + i]) + part[2 * kPartJ + i]) + part[3 * kPartJ + i];
        L.k.keep[j] = (above / zk < (double)a.top_p) ? 1 : 0;
      }
      __syncthreads();
    } else {
      for (int j = j0 + t; j < j1; j += kThreads) L.k.keep[j] = 1;
    }
  }
  __syncthreads();
  // rank of every kept entry among the kept ones by index: keep[j] becomes rank + 1
  for (int j0 = 0; j0 < nk; j0 += kPartJ) {
    const int j1 = min(nk, j0 + kPartJ);
    for (int j = j0 + lane; j < j1; j += 64) {
      int c = 0;
      if (L.k.keep[j]) {
        const int xj = L.kx[j];
        for (int y = wave; y < nk; y += kWaves) c += (L.k.keep[y] && L.kx[y] < xj) ? 1 : 0;
      }
      ipart[wave * kPartJ + (j - j0)] = c;
    }
    __syncthreads();
    for (int j = j0 + t; j < j1; j += kThreads) {
      const int i = j - j0;
      if (L.k.keep[j]) L.k.keep[j] = 1 + ipart[i] + ipart[kPartJ + i] + ipart[2 * kPartJ + i] + ipart[3 * kPartJ + i];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // Z_S, then p, entropy, the kept set in index order
  double zs = 0.0;
  int ns_all = 0, nf_all = 0;
  for (int j = lane; j < nk; j += 64)
    if (L.k.keep[j]) { zs += L.k.ke[j]; ++ns_all; nf_all += L.kv[j] > -INFINITY ? 1 : 0; }
  zs = wave_sum_dpp_d(zs);
  ns_all = wave_sum_i(ns_all);
  nf_all = wave_sum_i(nf_all);
  double ent = 0.0;
  KeptEntry* kept = a.kept + (int64_t)slot * kKeepMax;
  for (int j = lane; j < nk; j += 64) {
    if (!L.k.keep[j]) continue;
    const double p = L.k.ke[j] / zs;
    if (p > 0.0) ent -= p * log2_split(p);
    KeptEntry ke;
    ke.x = L.kx[j];
    ke.p = p;
    kept[L.k.keep[j] - 1] = ke;
  }
  ent = wave_sum_dpp_d(ent);
  if (lane == 0) {
    st.n = ns_all;
    st.kept_finite = nf_all;
    st.m = m;
    st.argmax = amx;
    st.z = zs;
    st.log_z = (double)m * (double)a.inv_t + log2_split(zs) * 0.6931471805599453;
    st.entropy = ent;
    st.max_prob = 1.0 / zs;
    a.rstat[slot] = st;
  }
}

// ---------------------------------------------------------------- k_filt_rows_w (bf16 rows)

// One wave per bf16 row, no workgroup barrier.  Entry `lane` of every candidate list (one list
// per 8192 logits, at most 32; one word per candidate: raw bf16 bits, valid bit, offset in the
// list) is read in one go into a register, its bits turned into their order key; entries past
// 64 of a longer list are read from memory at each pass.  The threshold is the same k-th largest key as in k_filt_rows.  When it lies
// within 256 keys of the row maximum (the usual case), the per-key counts that found it carry
// the rest: equal keys are equal values with equal e-values, so the mass above a key (top-p),
// Z, the entropy and every kept probability come from at most 256 keys, four per lane.  A
// top-k set spread wider, or fewer candidates than k, keeps its e-values in LDS and sums the
// masses above each entry directly.  The kept set goes out in index order: a list covers one
// index range, so an entry's place is the kept entries of the lists before its own plus those
// of its own list below it.
constexpr int kWLists = kMaxSlicesFused / 2;

// A list word with its raw bf16 bits replaced by their 16-bit order key (larger key, larger
// value; -0 and +0 share a key); offset and valid bit unchanged.
__device__ __forceinline__ uint32_t key_word(uint32_t w) {
  uint32_t b = w >> 16;
  if (b == 0x8000u) b = 0u;
  const uint32_t key = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
  return (key << 16) | (w & 0xFFFFu);
}

struct RowWLds {
  union {
    uint32_t hist[256];    // candidates per order key km - d (or per radix digit)
    double pd[256];        // window case: p of the kept key km - d
    double ke[kKeepMax];   // spread case: e-values of the top-k set
  };
  uint16_t kk[kKeepMax];   // the top-k set in list order: order keys
  int kx[kKeepMax];        // and token indices
  int kb[kWLists + 1];     // list s holds entries kb[s] .. kb[s + 1] - 1
  int kc[kWLists];         // kept entries per list, then their exclusive prefix
};

template <int NL>
__global__ __launch_bounds__(64) void k_filt_rows_w(FilterArgs a) {
  static_assert(NL <= kWLists, "a bf16 row has at most kWLists lists");
  __shared__ RowWLds L;
  const int lane = threadIdx.x;
  const int slot = blockIdx.x;
  if (slot >= a.n_slots) return;
  const int n_l = a.n_l, cap = a.cap, k = a.k;
  RowStat2 st;
  st.n = 0; st.flags = 0; st.m = -INFINITY; st.argmax = -1; st.kept_finite = 0; st.pad = 0;
  st.log_z = 0.0; st.entropy = 0.0; st.max_prob = 0.0; st.z = 0.0;
  if (n_l > NL) {   // not a bf16 row's lists: leave the row to the dense recomputation
    st.flags = kFlagOverflow;
    if (lane == 0) a.rstat[slot] = st;
    return;
  }
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (uint32_t*)a.cand + (int64_t)slot * n_l * cap, (short)0, n_l * cap * 4, 0x00020000);
  // every load at once, unconditionally (past the row's lists the bounds check returns zeros
  // and reads nothing): list headers (lane s: list s) and entry `lane` of every list
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<CandHead*>(a.chead + (int64_t)slot * n_l), (short)0, n_l * (int)sizeof(CandHead), 0x00020000);
  const auto hv = __builtin_amdgcn_raw_buffer_load_b128(rh, lane * (int)sizeof(CandHead), 0, 0);
  uint32_t w[NL];
#pragma unroll
  for (int s = 0; s < NL; ++s) w[s] = __builtin_amdgcn_raw_buffer_load_b32(rs, (s * cap + lane) * 4, 0, 0);
  CandHead h;   // zeros past the row's lists
  h.stored = (int)hv[0]; h.total = (int)hv[1]; h.th = hv[2]; h.flags = (int)hv[3];
  // opaque moves: every load is issued unconditionally before the first wait, and each word
  // stays one register rather than its key and offset apart
#pragma unroll
  for (int s = 0; s < NL; ++s) asm volatile("" : "+v"(w[s]));
#pragma unroll
  for (int s = 0; s < NL; ++s) {
    w[s] = lane < __builtin_amdgcn_readlane(h.stored, s) ? key_word(w[s]) : 0u;
    asm volatile("" : "+v"(w[s]));
  }
  const int bad = wave_or(h.flags & kFlagBad);
  const bool extra = wave_or(h.stored > 64 ? 1 : 0) != 0;
  // cb(word, valid, list) for every candidate; entries past 64 of a list in uniform rounds
  auto for_each = [&](auto cb) {
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      if (s < n_l) {
        cb(w[s], w[s] != 0u, s);
        if (extra) {
          const int cs = __builtin_amdgcn_readlane(h.stored, s);
          for (int e0 = 64; e0 < cs; e0 += 64) {
            cb(key_word(__builtin_amdgcn_raw_buffer_load_b32(rs, (s * cap + e0 + lane) * 4, 0, 0)), e0 + lane < cs, s);
          }
        }
      }
    }
  };
  // the largest key, then the candidates per key within 256 below it
  int km = -1;
  for_each([&](uint32_t wd, bool ok, int) {
    if (ok) km = max(km, (int)(wd >> 16));
  });
  km = wave_max_i(km);
#pragma unroll
  for (int q = 0; q < 4; ++q) L.hist[lane + 64 * q] = 0u;
  __builtin_amdgcn_wave_barrier();
  for_each([&](uint32_t wd, bool ok, int) {
    const int d = km - (int)(wd >> 16);
    if (ok && d < 256) atomicAdd(&L.hist[d], 1u);
  });
  __builtin_amdgcn_wave_barrier();
  int cq[4], csum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) { cq[q] = (int)L.hist[4 * lane + q]; csum += cq[q]; }
  const int cinc = wave_incl_scan_i(csum);
  const bool window = __builtin_amdgcn_readlane(cinc, 63) >= k;
  bool all = false;
  uint32_t th = 0u;
  if (window) {
    int dg = -1, run = cinc - csum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (dg < 0 && run + cq[q] >= k) dg = 4 * lane + q;
      run += cq[q];
    }
    dg = __builtin_amdgcn_readlane(dg, __builtin_ctzll(__ballot(cinc >= k)));
    th = (uint32_t)(km - dg);
  } else {
    // exact radix select, high then low byte of the key, over every candidate
    uint32_t prefix = 0u;
    int kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) L.hist[lane + 64 * q] = 0u;
      __builtin_amdgcn_wave_barrier();
      for_each([&](uint32_t wd, bool ok, int) {
        const uint32_t key = wd >> 16;
        if (ok && (pass == 0 || (key >> 8) == prefix)) atomicAdd(&L.hist[pass == 0 ? (key >> 8) : (key & 255u)], 1u);
      });
      __builtin_amdgcn_wave_barrier();
      int c[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = (int)L.hist[255 - 4 * lane - q]; s += c[q]; }
      const int inc = wave_incl_scan_i(s);
      if (__builtin_amdgcn_readlane(inc, 63) < kk) { all = true; break; }
      int dg = -1, ab = 0, run = inc - s;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (dg < 0 && run + c[q] >= kk) { dg = 255 - 4 * lane - q; ab = run; }
        run += c[q];
      }
      const int lh = __builtin_ctzll(__ballot(inc >= kk));
      dg = __builtin_amdgcn_readlane(dg, lh);
      ab = __builtin_amdgcn_readlane(ab, lh);
      prefix = (prefix << 8) | (uint32_t)dg;
      kk -= ab;
    }
    th = all ? 0u : prefix;
  }
  // dropped ties of a list hold its threshold key; they belong to the top-k set if it reaches th
  int fl = bad;
  if (lane < n_l && h.total > h.stored && (all || h.th >= th)) fl |= kFlagOverflow;
  fl = wave_or(fl);
  // the top-k set, compacted list by list
  const uint32_t thw = all ? 0u : (th << 16);
  int nk = 0, amx = INT_MAX, cur = -1;
  for_each([&](uint32_t wd, bool ok, int s) {
    if (s != cur) {   // uniform: the first entries of list s
      cur = s;
      if (lane == 0) L.kb[s] = nk;
    }
    const bool in = ok && wd >= thw;
    const unsigned long long mk = __ballot(in);
    if (in) {
      const int o = nk + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mk, 0u));
      const int x = (s << 13) | (int)(wd & 0x1FFFu);
      if (o < kKeepMax) { L.kk[o] = (uint16_t)(wd >> 16); L.kx[o] = x; }
      if ((int)(wd >> 16) == km) amx = min(amx, x);
    }
    nk += __popcll(mk);
  });
  if (lane == 0) L.kb[n_l] = nk;
  amx = wave_min_i(amx);
  if (nk > kKeepMax) fl |= kFlagOverflow;
  if (nk == 0 && !(fl & kFlagBad)) fl |= kFlagEmpty;
  if (fl) {
    st.flags = fl;
    if (lane == 0) a.rstat[slot] = st;
    return;
  }
  __builtin_amdgcn_wave_barrier();
  const float m = key16_value(km);
  const double md = (double)m, cd2 = a.c;
  const int nq8 = (nk + 63) >> 6;   // the top-k set's entries per lane
  int key_cut;
  double zs, ent = 0.0;
  int nkept = 0, nfin = 0;
  if (window) {
    // key km - d, d = 4 lane + q: its count in the top-k set, e-value and mass
    const int dth = km - (int)th;
    int nq[4];
    double eq[4], mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 4 * lane + q;
      nq[q] = d <= dth ? cq[q] : 0;
      eq[q] = nq[q] > 0 ? exp2_split(((double)key16_value(km - d) - md) * cd2) : 0.0;
      mq[q] = (double)nq[q] * eq[q];
    }
    const double inc = wave_scan_dpp_d(((mq[0] + mq[1]) + mq[2]) + mq[3]);
    const double zk = readlane_d(inc, 63);
    // mass strictly above key km - d: the lanes below, then this lane's keys before d
    const long long ib = __double_as_longlong(inc);
    const int src = (lane == 0 ? 0 : lane - 1) * 4;
    const int plo = __builtin_amdgcn_ds_bpermute(src, (int)ib), phi = __builtin_amdgcn_ds_bpermute(src, (int)(ib >> 32));
    double ab = lane == 0 ? 0.0 : __longlong_as_double(((long long)phi << 32) | (unsigned)plo);
    int dcut = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (nq[q] > 0 && (!(a.top_p < 1.f) || ab / zk < (double)a.top_p)) dcut = 4 * lane + q;
      ab += mq[q];
    }
    dcut = wave_max_i(dcut);
    key_cut = km - dcut;   // dcut < 0 keeps nothing
    double zl = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 4 * lane + q;
      if (d <= dcut) {
        zl += mq[q];
        nkept += nq[q];
        if (km - d >= 128) nfin += nq[q];   // keys below 128 are -inf
      }
    }
    zs = wave_sum_dpp_d(zl);
    double el = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 4 * lane + q;
      if (d <= dcut && nq[q] > 0) {
        const double p = eq[q] / zs;
        if (p > 0.0) el -= (double)nq[q] * (p * log2_split(p));
        L.pd[d] = p;
      }
    }
    ent = wave_sum_dpp_d(el);
  } else {
    double zl = 0.0;
    for (int q = 0; q < nq8; ++q) {
      const int j = lane + 64 * q;
      if (j < nk) {
        const double e = exp2_split(((double)key16_value(L.kk[j]) - md) * cd2);
        L.ke[j] = e;
        zl += e;
      }
    }
    const double zk = wave_sum_dpp_d(zl);
    __builtin_amdgcn_wave_barrier();
    if (a.top_p < 1.f) {
      // keep x iff the mass of the strictly larger values is below top_p (an upper set of keys)
      int kmin = INT_MAX;
      for (int q = 0; q < nq8; ++q) {
        const int j = lane + 64 * q;
        const int kj = j < nk ? (int)L.kk[j] : 0x10000;
        double ab = 0.0;
        for (int y = 0; y < nk; ++y) ab += ((int)L.kk[y] > kj) ? L.ke[y] : 0.0;
        if (j < nk && ab / zk < (double)a.top_p) kmin = min(kmin, kj);
      }
      kmin = wave_min_i(kmin);
      key_cut = kmin == INT_MAX ? 0x10000 : kmin;
    } else {
      key_cut = 0;
    }
    double zl2 = 0.0;
    for (int q = 0; q < nq8; ++q) {
      const int j = lane + 64 * q;
      if (j < nk && (int)L.kk[j] >= key_cut) {
        zl2 += L.ke[j];
        ++nkept;
        if (L.kk[j] >= 128) ++nfin;
      }
    }
    zs = wave_sum_dpp_d(zl2);
    double el = 0.0;
    for (int q = 0; q < nq8; ++q) {
      const int j = lane + 64 * q;
      if (j < nk && (int)L.kk[j] >= key_cut) {
        const double p = L.ke[j] / zs;
        if (p > 0.0) el -= p * log2_split(p);
      }
    }
    ent = wave_sum_dpp_d(el);
  }
  nkept = wave_sum_i(nkept);
  nfin = wave_sum_i(nfin);
  // the kept set in index order: kept entries of the lists before, then of its own list below it
  if (lane < n_l) L.kc[lane] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int q = 0; q < nq8; ++q) {
    const int j = lane + 64 * q;
    if (j < nk && (int)L.kk[j] >= key_cut) atomicAdd(&L.kc[L.kx[j] >> 13], 1);
  }
  __builtin_amdgcn_wave_barrier();
  {
    const int c = lane < n_l ? L.kc[lane] : 0;
    const int inc = wave_incl_scan_i(c);
    __builtin_amdgcn_wave_barrier();
    if (lane < n_l) L.kc[lane] = inc - c;
  }
  __builtin_amdgcn_wave_barrier();
  KeptEntry* kept = a.kept + (int64_t)slot * kKeepMax;
  for (int q = 0; q < nq8; ++q) {
    const int j = lane + 64 * q;
    if (j < nk) {
      const int kj = L.kk[j];
      if (kj >= key_cut) {
        const int x = L.kx[j], l = x >> 13;
        int r = L.kc[l];
        const int y1 = L.kb[l + 1];
        for (int y = L.kb[l]; y < y1; ++y) r += ((int)L.kk[y] >= key_cut && L.kx[y] < x) ? 1 : 0;
        KeptEntry e;
        e.x = x;
        e.pad = 0;
        e.p = window ? L.pd[km - kj] : L.ke[j] / zs;
        kept[r] = e;
      }
    }
  }
  if (lane == 0) {
    st.n = nkept;
    st.kept_finite = nfin;
    st.m = m;
    st.argmax = amx;
    st.z = zs;
    st.log_z = md * a.inv_t + log2_split(zs) * 0.6931471805599453;
    st.entropy = ent;
    st.max_prob = 1.0 / zs;
    a.rstat[slot] = st;
  }
}

// The wave-per-row kernel with room for the row's lists (a bf16 row has at most kWLists).
void launch_rows_w(const FilterArgs& a, hipStream_t st) {
  const dim3 g(a.n_slots), b(64);
  if (a.n_l <= 8) hipLaunchKernelGGL(k_filt_rows_w<8>, g, b, 0, st, a);
  else if (a.n_l <= 16) hipLaunchKernelGGL(k_filt_rows_w<16>, g, b, 0, st, a);
  else if (a.n_l <= 24) hipLaunchKernelGGL(k_filt_rows_w<24>, g, b, 0, st, a);
  else hipLaunchKernelGGL(k_filt_rows_w<kWLists>, g, b, 0, st, a);
}

// ---------------------------------------------------------------- k_filt_finalize

struct FinFLds {
  double py[kMaxGamma + 1], qy[kMaxGamma + 1], u0[kMaxGamma];
  double us[kMaxGamma + 1][3];                            // sampler uniforms of every position
  int ytok[kMaxGamma];
  int np[kMaxGamma + 1], nq[kMaxGamma + 1];               // kept counts of every position's rows
  float dh[kMaxGamma], dm[kMaxGamma];
  double ap[kMaxGamma];                                   // accept probability per position
  int pidx[kWaves][kKeepMax], qidx[kWaves][kKeepMax];   // a wave's kept token lists
  double ppv[kWaves][kKeepMax], qpv[kWaves][kKeepMax];  // and their probabilities
  double w[kKeepMax];                                     // sampler weights of the chosen row
  int xs[kKeepMax];
  int flags, status, n_acc, pos, wkind, y, n, x;
  double u[3];
};

// A row's kept set into LDS (indices and probabilities): the first 64 entries are read before
// the count is known (the kept array always holds kKeepMax entries), the rest after it.
__device__ __forceinline__ void stage_kept(const KeptEntry* k, int n, int* ix, double* pv, const KeptEntry& first) {
  const int lane = threadIdx.x & 63;
  if (lane < n) { ix[lane] = first.x; pv[lane] = first.p; }
  for (int j = 64 + lane; j < n; j += 64) { const KeptEntry e = k[j]; ix[j] = e.x; pv[j] = e.p; }
}

// Position of token x in a sorted index list (n entries), or -1.
__device__ __forceinline__ int find_idx(const int* ix, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ix[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return (lo < n && ix[lo] == x) ? lo : -1;
}

// First position j in xs[0..n) (increasing) with xs[j] >= key.
__device__ __forceinline__ int lower_bound_i(const int* xs, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (xs[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// One wave: the three-level inverse CDF (reading R6: chunks of 4096, groups of 64, tokens) over
// sparse weights wv[j] at increasing token indices xs[j], j < n (n_s <= 64 chunks).  Level 1:
// lane k sums chunk k's weights in index order, then a wave-wide fp64 scan picks the chunk;
// level 2: the same over the chunk's 64 groups; level 3: over the group's entries (at most 64).
// Each pick takes the first running sum above u times the level's total, or the last positive
// weight when rounding leaves none.  Every lane returns the token, or -1 with W <= 0 when the
// total weight W is not positive.
__device__ int sparse_sample_wave(const int* xs, const double* wv, int n, int n_s, const double* u, double& W) {
  const int lane = threadIdx.x & 63;
  double sk = 0.0;
  if (lane < n_s) {
    const int j1 = lower_bound_i(xs, n, (lane + 1) << 12);
    for (int j = lower_bound_i(xs, n, lane << 12); j < j1; ++j) sk += wv[j];
  }
  const int kc = wave_pick(sk, n_s, u[0], W);
  if (kc < 0) return -1;
  const int key = ((kc << 6) + lane) << 6;
  const int g0 = lower_bound_i(xs, n, key), g1 = lower_bound_i(xs, n, key + 64);
  double mg = 0.0;
  for (int j = g0; j < g1; ++j) mg += wv[j];
  double tg;
  const int gp = wave_pick(mg, 64, u[1], tg);
  if (gp < 0) return -1;
  const int a0 = __builtin_amdgcn_readlane(g0, gp), a1 = __builtin_amdgcn_readlane(g1, gp);
  double te;
  const int e = wave_pick(lane < a1 - a0 ? wv[a0 + lane] : 0.0, a1 - a0, u[2], te);
  return e >= 0 ? xs[a0 + e] : -1;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_filt_finalize(FilterArgs a) {
  __shared__ FinFLds F;
  __shared__ int cu_s[kMaxReqFused + 1];
  __shared__ int red_i[8];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = blockIdx.x;
  const float nan = __int_as_float(0x7fc00000);
  // the reads of position i; the wave's next position is read while this one is worked on
  struct PosIn {
    RowStat2 P, Q;
    KeptEntry kp0, kq0;
    int y;
  };
  auto read_pos = [&](int i, int c0, int g) {
    PosIn r;
    r.Q.n = 0; r.Q.flags = 0; r.Q.entropy = 0.0; r.Q.max_prob = 0.0;
    r.kq0.x = 0; r.kq0.p = 0.0;
    r.y = -1;
    r.P = r.Q;
    r.kp0 = r.kq0;
    if (i > g) return r;
    const int ps = c0 + b + i, qs = a.n_teams + c0 + i;
    r.P = a.rstat[ps];
    r.kp0 = a.kept[(int64_t)ps * kKeepMax + lane];
    if (MODE == kFuSample && i < g) {
      r.Q = a.rstat[qs];
      r.kq0 = a.kept[(int64_t)qs * kKeepMax + lane];
    }
    if (i < g) r.y = a.tokens[c0 + i];
    return r;
  };
  // the wave's first position goes out at once, at the guess c0 = b G (exact when every request
  // has G draft tokens); a wrong guess reads it again once the offsets are known
  const int cg = b * a.G;
  const bool guess_in = cg + a.G <= a.n_draft_rows;
  PosIn nxt = read_pos(guess_in ? wave : a.G + 1, cg, a.G);
  // the draft offsets, checked as one exclusive prefix; meanwhile thread t draws the Philox block
  // of position t (1-based t + 1): word 0 is the accept draw, words 1..3 the sampler's uniforms
  // if the emitted token is drawn there
  for (int k = t; k <= a.B; k += kThreads) cu_s[k] = a.cu[k];
  if (t <= a.G) {
    uint64_t w[4];
    philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(t + 1), 0, 0, w);
    if (t < a.G) F.u0[t] = u53(w[0]);
    F.us[t][0] = u53(w[1]);
    F.us[t][1] = u53(w[2]);
    F.us[t][2] = u53(w[3]);
  }
  __syncthreads();
  int badc = 0;
  for (int k = t; k < a.B; k += kThreads) {
    const int g = cu_s[k + 1] - cu_s[k];
    if (g < 0 || g > a.G) badc = 1;
  }
  if (t == 0 && (cu_s[0] != 0 || cu_s[a.B] != a.n_draft_rows)) badc = 1;
  badc = block_or(badc, red_i);
  if (badc) {
    if (t <= a.G) a.out_tokens[(int64_t)b * (a.G + 1) + t] = -1;
    if (t == 0) {
      a.out_num_accepted[b] = 0;
      a.out_status[b] = kStBadGamma;
      if (a.out_req_stats)
        for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = nan;
    }
    return;
  }
  const int c0 = cu_s[b], g = cu_s[b + 1] - c0;
  if (!(guess_in && c0 == cg && g == a.G)) nxt = read_pos(wave, c0, g);
  if (t == 0) F.flags = 0;
  __syncthreads();
  // A. per position (one wave each): flags, statistics, p(y), q(y), 1 - TV.  A position's row
  // statistics, token and first 64 kept entries of both rows are read at once; every later
  // lookup is in LDS.
  int* pix = F.pidx[wave];
  int* qix = F.qidx[wave];
  double* ppv = F.ppv[wave];
  double* qpv = F.qpv[wave];
  for (int i = wave; i <= g; i += kWaves) {
    const PosIn cur = nxt;
    nxt = read_pos(i + kWaves, c0, g);
    const int ps = c0 + b + i;
    const int qs = a.n_teams + c0 + i;
    const KeptEntry* kp = a.kept + (int64_t)ps * kKeepMax;
    const KeptEntry* kq = a.kept + (int64_t)qs * kKeepMax;
    const RowStat2 P = cur.P;
    const RowStat2 Q = cur.Q;
    const KeptEntry kp0 = cur.kp0, kq0 = cur.kq0;
    const int y = cur.y;
    const bool okp = P.flags == 0;
    int fl = P.flags;
    const int np = okp ? P.n : 0;
    stage_kept(kp, np, pix, ppv, kp0);
    if (lane == 0) F.np[i] = np;
    if (i < g) {
      const bool yv = y >= 0 && y < a.V;
      double pyd = 0.0, qyd = 1.0, ap = nan;
      float py = nan, qy = nan, ovl = nan, dh = nan, dm = nan, l1 = nan, klpq = nan, klqp = nan;
      const bool want_kl = a.st.kl_pq || a.st.kl_qp;
      if (MODE == kFuSample) {
        fl |= Q.flags;
        const bool okq = Q.flags == 0;
        const int nq = okq ? Q.n : 0;
        stage_kept(kq, nq, qix, qpv, kq0);
        if (lane == 0) F.nq[i] = nq;
        __builtin_amdgcn_wave_barrier();
        if (okp && yv) {
          const int m = find_idx(pix, np, y);
          pyd = m >= 0 ? ppv[m] : 0.0;
          py = (float)pyd;
        }
        if (okq && yv) {
          const int m = find_idx(qix, nq, y);
          qyd = m >= 0 ? qpv[m] : 0.0;
          qy = (float)qyd;
        }
        if (okp && okq) {
          // over p's kept set: min(p, q), [p - q]_+ (beta = TV, L1 = 2 beta) and, on request,
          // p ln(p / q); a token of S_p missing from S_q makes D(p || q) infinite
          double part = 0.0, beta = 0.0, kl1 = 0.0;
          int miss = 0;
          for (int j = lane; j < np; j += 64) {
            const int m = find_idx(qix, nq, pix[j]);
            const double pv = ppv[j], qv = m >= 0 ? qpv[m] : 0.0;
            part += fmin(pv, qv);
            beta += fmax(pv - qv, 0.0);
            if (want_kl) {
              if (m >= 0) kl1 += pv * log(pv / qv);
              else miss = 1;
            }
          }
          ovl = (float)wave_sum_dpp_d(part);
          l1 = (float)(2.0 * wave_sum_dpp_d(beta));
          ap = (yv && qyd > 0.0) ? fmin(1.0, pyd / qyd) : 0.0;
          if (want_kl) {
            kl1 = wave_sum_dpp_d(kl1);
            miss = wave_or(miss);
            klpq = miss ? INFINITY : (float)kl1;
            double kl2 = 0.0;
            miss = 0;
            for (int j = lane; j < nq; j += 64) {
              const int m = find_idx(pix, np, qix[j]);
              if (m >= 0) kl2 += qpv[j] * log(qpv[j] / ppv[m]);
              else miss = 1;
            }
            kl2 = wave_sum_dpp_d(kl2);
            miss = wave_or(miss);
            klqp = miss ? INFINITY : (float)kl2;
          }
        }
        if (okq) { dh = (float)Q.entropy; dm = (float)Q.max_prob; }
      } else {
        __builtin_amdgcn_wave_barrier();
        if (okp && yv) {
          const int m = find_idx(pix, np, y);
          pyd = m >= 0 ? ppv[m] : 0.0;
          py = (float)pyd;
        }
        qyd = 1.0;
        qy = yv ? 1.f : nan;
        ovl = okp ? (yv ? py : 0.f) : nan;
        dh = yv ? 0.f : nan;
        dm = yv ? 1.f : nan;
        ap = okp ? (yv ? fmin(1.0, pyd) : 0.0) : nan;
        if (okp && yv) {
          // q one-hot at y: D(q || p) = -ln p(y); D(p || q) is finite only for a one-hot p
          l1 = (float)(2.0 * (1.0 - pyd));
          klqp = (float)(-log(pyd));
          klpq = pyd >= 1.0 ? 0.f : INFINITY;
        }
      }
      if (lane == 0) {
        if (a.st.p_y) a.st.p_y[c0 + i] = py;
        if (a.st.q_y) a.st.q_y[c0 + i] = qy;
        if (a.st.one_minus_tv) a.st.one_minus_tv[c0 + i] = ovl;
        if (a.st.draft_entropy_bits) a.st.draft_entropy_bits[c0 + i] = dh;
        if (a.st.draft_max_prob) a.st.draft_max_prob[c0 + i] = dm;
        if (a.st.l1) a.st.l1[c0 + i] = l1;
        if (a.st.accept_prob) a.st.accept_prob[c0 + i] = (float)ap;
        if (a.st.kl_pq) a.st.kl_pq[c0 + i] = klpq;
        if (a.st.kl_qp) a.st.kl_qp[c0 + i] = klqp;
        F.ap[i] = ap;
        F.dh[i] = dh;
        F.dm[i] = dm;
        F.py[i] = pyd;
        F.qy[i] = qyd;
        F.ytok[i] = y;
      }
    }
    if (lane == 0) {
      if (a.st.target_entropy_bits) a.st.target_entropy_bits[ps] = P.flags ? nan : (float)P.entropy;
      if (a.st.target_max_prob) a.st.target_max_prob[ps] = P.flags ? nan : (float)P.max_prob;
      if (fl) atomicOr(&F.flags, fl);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // B. accept scan, the row to sample, request statistics (one thread)
  if (t == 0) {
    int status = 0, j = -1;
    if (F.flags & kFlagOverflow) {
      // the dense recomputation after this kernel replaces every output of this request
      status = kStFilterOverflow;
      if (a.ovf_list) a.ovf_list[atomicAdd(a.ovf_n, 1)] = b;
    }
    else if (F.flags) status = kStNonfinite;
    else {
      for (int i = 0; i < g; ++i) {
        const int y = F.ytok[i];
        if (y < 0 || y >= a.V) { status |= kStBadToken; j = i; break; }
        const double qy = F.qy[i];
        if (!(qy > 0.0)) { status |= kStZeroQ; j = i; break; }
        if (!(F.u0[i] < fmin(1.0, F.py[i] / qy))) { j = i; break; }
      }
    }
    F.n_acc = j < 0 ? g : j;
    F.pos = j < 0 ? g : j;
    F.y = j >= 0 ? F.ytok[j] : -1;
    F.wkind = (j < 0) ? 0 : (MODE == kFuSample ? 1 : 2);
    F.u[0] = F.us[F.pos][0];
    F.u[1] = F.us[F.pos][1];
    F.u[2] = F.us[F.pos][2];
    F.status = status;
    F.x = -1;
    if (a.st.expected_committed)
      a.st.expected_committed[b] = F.flags ? nan : expected_committed(F.ap, g);
    if (a.out_req_stats) {
      float rq[4] = {nan, nan, nan, nan};
      if (g > 0) {
        double hs = 0.0, cs = 0.0;
        float hmax = -INFINITY, cmin = INFINITY;
        bool anynan = false;
        for (int i = 0; i < g; ++i) {
          const float hh = F.dh[i], cm = F.dm[i];
          if (!(hh == hh) || !(cm == cm)) anynan = true;
          hs += hh; cs += cm;
          hmax = fmaxf(hmax, hh); cmin = fminf(cmin, cm);
        }
        if (!anynan) { rq[0] = (float)(hs / g); rq[1] = (float)(cs / g); rq[2] = hmax; rq[3] = cmin; }
      }
      for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = rq[q];
    }
  }
  __syncthreads();
  // C. the three-level sampler on the sparse weights of the chosen row (reading R6): weights in
  // LDS (all threads), then the level sums in index order (one thread)
  if (!(F.status & (kStNonfinite | kStFilterOverflow))) {
    // the chosen row's kept set (indices into xs, probabilities into w) and, for the residual,
    // its draft row's (into wave 0's lists), in one pass
    const int ps = c0 + b + F.pos;
    const KeptEntry* kp = a.kept + (int64_t)ps * kKeepMax;
    const int n = F.np[F.pos];
    const KeptEntry* kq = nullptr;
    int nq = 0;
    if (MODE == kFuSample && F.pos < g) {
      const int qs = a.n_teams + c0 + F.pos;
      kq = a.kept + (int64_t)qs * kKeepMax;
      nq = F.nq[F.pos];
    }
    __syncthreads();   // every wave is done with its lists
    for (int j = t; j < nq; j += kThreads) { const KeptEntry e = kq[j]; F.qidx[0][j] = e.x; F.qpv[0][j] = e.p; }
    for (int j = t; j < n; j += kThreads) { const KeptEntry e = kp[j]; F.xs[j] = e.x; F.ppv[0][j] = e.p; }
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      const int wkind = pass == 0 ? F.wkind : 0;
      const int yx = F.y;
      for (int j = t; j < n; j += kThreads) {
        const double p = F.ppv[0][j];
        double w = p;
        if (wkind == 1) {
          const int m = find_idx(F.qidx[0], nq, F.xs[j]);
          w = fmax(p - (m >= 0 ? F.qpv[0][m] : 0.0), 0.0);
        } else if (wkind == 2) {
          w = F.xs[j] == yx ? fmax(p - 1.0, 0.0) : p;
        }
        F.w[j] = w;
      }
      __syncthreads();
      if (t < 64) {
        double W;
        const int x = sparse_sample_wave(F.xs, F.w, n, a.n_s, F.u, W);
        if (t == 0) {
          int again = 0;
          if (!(W > 0.0)) {
            if (wkind != 0) { F.status |= kStResidualEmpty; again = 1; }
          } else {
            F.x = x;
          }
          red_i[0] = again;
        }
      }
      __syncthreads();
      if (!red_i[0]) break;
    }
  }
  __syncthreads();
  const bool ok = !(F.status & (kStNonfinite | kStFilterOverflow));
  if (t <= a.G) {
    int tok = -1;
    if (ok) {
      if (t < F.n_acc) tok = F.ytok[t];
      else if (t == F.n_acc) tok = F.x;
    }
    a.out_tokens[(int64_t)b * (a.G + 1) + t] = tok;
  }
  if (t == 0) {
    a.out_num_accepted[b] = ok ? F.n_acc : 0;
    a.out_status[b] = F.status;
  }
}

// ---------------------------------------------------------------- launch

// The candidate lists of a row: one per two 4096-logit chunks for bf16 rows, one per chunk for
// fp32 rows (the workspace holds one per chunk).
FilterArgs with_lists(const FilterArgs& a0, int dt) {
  FilterArgs a = a0;
  a.n_l = dt == kDtBF16 ? (a.n_s + 1) / 2 : a.n_s;
  return a;
}

hipError_t launch_filter(const FilterArgs& a0, int dt, int vec, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const FilterArgs a = with_lists(a0, dt);
  const long long g1 = (long long)a.n_teams * a.n_l;
  if (g1 < 1 || g1 > 0x7fffffffll || a.B < 1) return hipErrorInvalidConfiguration;
  // optional events bracket the streaming kernel alone (benchmark timing)
  const bool paired = a.mode == kFuSample;
  const dim3 g((unsigned)g1), b(kThreads);
  if (dt == kDtBF16) {
    if (paired) {
      if (vec) launch_timed(k_filt_slices<kDtBF16, true, true>, g, b, st, ev0, ev1, a);
      else launch_timed(k_filt_slices<kDtBF16, false, true>, g, b, st, ev0, ev1, a);
    } else {
      if (vec) launch_timed(k_filt_slices<kDtBF16, true, false>, g, b, st, ev0, ev1, a);
      else launch_timed(k_filt_slices<kDtBF16, false, false>, g, b, st, ev0, ev1, a);
    }
  } else {
    if (paired) {
      if (vec) launch_timed(k_filt_slices<kDtF32, true, true>, g, b, st, ev0, ev1, a);
      else launch_timed(k_filt_slices<kDtF32, false, true>, g, b, st, ev0, ev1, a);
    } else {
      if (vec) launch_timed(k_filt_slices<kDtF32, true, false>, g, b, st, ev0, ev1, a);
      else launch_timed(k_filt_slices<kDtF32, false, false>, g, b, st, ev0, ev1, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == kDtBF16) launch_rows_w(a, st);
  else hipLaunchKernelGGL((k_filt_rows<kDtF32>), dim3(a.n_slots), dim3(kThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (paired) hipLaunchKernelGGL((k_filt_finalize<kFuSample>), dim3(a.B), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((k_filt_finalize<kFuTokenOnly>), dim3(a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- plain filtered rows

// spec_row_stats: the statistics of filtered row r (SpecKV page signals on the distribution
// actually sampled from).  A row with a NaN / +inf logit or no finite logit gives argmax -1,
// NaN statistics and kept count 0; a row whose top-k set overflows the sparse sets, argmax -1,
// NaN statistics and kept count -1.
__global__ __launch_bounds__(kThreads) void k_filt_rowstats_out(FilterArgs a) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= a.n_slots) return;
  const RowStat2 st = a.rstat[r];
  const float nan = __int_as_float(0x7fc00000);
  const bool ok = st.flags == 0;
  const RowStatsOut& o = a.rso;
  if (o.max_logit) o.max_logit[r] = ok ? st.m : nan;
  if (o.argmax) o.argmax[r] = ok ? st.argmax : -1;
  if (o.log_z) o.log_z[r] = ok ? (float)st.log_z : nan;
  if (o.entropy_bits) o.entropy_bits[r] = ok ? (float)st.entropy : nan;
  if (o.max_prob) o.max_prob[r] = ok ? (float)st.max_prob : nan;
  if (o.kept_count) o.kept_count[r] = ok ? st.kept_finite : ((st.flags & kFlagOverflow) ? -1 : 0);
  // the dense recomputation after this kernel replaces this row's outputs
  if ((st.flags & kFlagOverflow) && a.ovf_list) a.ovf_list[atomicAdd(a.ovf_n, 1)] = r;
}

struct ResLds {
  int xs[kKeepMax], qx[kKeepMax];
  double w[kKeepMax];
  double red[kWaves];
  double u[3];
};

// spec_residual_sample: one draw from r(x) = [p(x) - q(x)]_+ / beta over p's kept set (guide page
// "5.1 投机解码核心原理" §3.2, beta = sum [p - q]_+ §4.1), or from p without q rows, by the sparse
// three-level sampler; uniforms injected, or Philox counter (r, 0, 1, 0) words 1..3.
template <bool WITH_Q>
__global__ __launch_bounds__(kThreads) void k_filt_residual(FilterArgs a) {
  __shared__ ResLds S;
  const int t = threadIdx.x, r = blockIdx.x;
  const double dnan = __longlong_as_double(0x7ff8000000000000ll);
  const RowStat2 P = a.rstat[r];
  int fl = P.flags;
  RowStat2 Q;
  if (WITH_Q) {
    Q = a.rstat[a.n_teams + r];
    fl |= Q.flags;
  }
  if (fl) {
    if (t == 0) {
      a.out_tokens[r] = -1;
      if (a.out_mass) a.out_mass[r] = dnan;
      a.out_status[r] = (fl & kFlagOverflow) ? kStFilterOverflow : kStNonfinite;
      // the dense recomputation after this kernel replaces this row's outputs
      if ((fl & kFlagOverflow) && a.ovf_list) a.ovf_list[atomicAdd(a.ovf_n, 1)] = r;
    }
    return;
  }
  const KeptEntry* kp = a.kept + (int64_t)r * kKeepMax;
  const int n = P.n;
  const KeptEntry* kq = WITH_Q ? a.kept + (int64_t)(a.n_teams + r) * kKeepMax : nullptr;
  const int nq = WITH_Q ? Q.n : 0;
  for (int j = t; j < n; j += kThreads) S.xs[j] = kp[j].x;
  for (int j = t; j < nq; j += kThreads) S.qx[j] = kq[j].x;
  if (t == 0) {
    if (a.uniforms) {
      for (int k = 0; k < 3; ++k) S.u[k] = a.uniforms[(int64_t)r * 3 + k];
    } else {
      uint64_t w[4];
      philox4x64_10(a.seed, a.step, (uint64_t)r, 0, 1, 0, w);
      S.u[0] = u53(w[1]);
      S.u[1] = u53(w[2]);
      S.u[2] = u53(w[3]);
    }
  }
  __syncthreads();
  double beta = 0.0;
  for (int j = t; j < n; j += kThreads) {
    double w = kp[j].p;
    if (WITH_Q) {
      const int m = find_idx(S.qx, nq, S.xs[j]);
      w = fmax(w - (m >= 0 ? kq[m].p : 0.0), 0.0);
    }
    S.w[j] = w;
    beta += w;
  }
  beta = block_sum_dd(beta, S.red);
  int status = 0;
  if (!(beta > 0.0)) {
    // an empty residual: drawn from p (reading R8)
    status = kStResidualEmpty;
    for (int j = t; j < n; j += kThreads) S.w[j] = kp[j].p;
    __syncthreads();
  }
  __syncthreads();
  if (t < 64) {
    double W;
    const int x = sparse_sample_wave(S.xs, S.w, n, a.n_s, S.u, W);
    if (t == 0) {
      a.out_tokens[r] = x;
      if (a.out_mass) a.out_mass[r] = beta;
      a.out_status[r] = status;
    }
  }
}

hipError_t launch_filter_rows(const FilterArgs& a0, int dt, int vec, int what, hipStream_t st) {
  const FilterArgs a = with_lists(a0, dt);
  const long long g1 = (long long)a.n_teams * a.n_l;
  if (g1 < 1 || g1 > 0x7fffffffll || a.n_slots < 1) return hipErrorInvalidConfiguration;
  const bool paired = what == 1 && a.drf != nullptr;
#define SPEC_SLICES(D, P)                                                                           \
  do {                                                                                              \
    if (vec) hipLaunchKernelGGL((k_filt_slices<D, true, P>), dim3((unsigned)g1), dim3(kThreads), 0, st, a);  \
    else hipLaunchKernelGGL((k_filt_slices<D, false, P>), dim3((unsigned)g1), dim3(kThreads), 0, st, a);     \
  } while (0)
  if (dt == kDtBF16) {
    if (paired) SPEC_SLICES(kDtBF16, true);
    else SPEC_SLICES(kDtBF16, false);
  } else {
    if (paired) SPEC_SLICES(kDtF32, true);
    else SPEC_SLICES(kDtF32, false);
  }
#undef SPEC_SLICES
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == kDtBF16) launch_rows_w(a, st);
  else hipLaunchKernelGGL((k_filt_rows<kDtF32>), dim3(a.n_slots), dim3(kThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (what == 0) {
    hipLaunchKernelGGL(k_filt_rowstats_out, dim3((a.n_slots + kThreads - 1) / kThreads), dim3(kThreads), 0, st, a);
  } else if (paired) {
    hipLaunchKernelGGL((k_filt_residual<true>), dim3(a.n_teams), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_filt_residual<false>), dim3(a.n_teams), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace specv
