// spec_fused.hip -- a whole verification round in two kernels: k_fused streams every needed
// logit once; k_fused_finalize (one workgroup per request) turns the records into outputs.
//
// Work unit ("ticket"): two consecutive 4096-logit slices of one target row, together with the
// same slices of its draft row when that position pairs the two (guide page "5.1 投机解码核心
// 原理", §3.2: the residual needs p and q at the same token).  The tickets of one target row
// form a team.  k_fused runs one workgroup per ticket; workgroup i lands on XCD i mod 8 (the
// dispatcher deals workgroups round-robin over the XCDs) and the tickets of the team in
// dispatch place ti are consecutive workgroups of XCD ti mod 8.  A place's rows follow from
// the place in a uniform batch and from the draft offsets (one search per workgroup) in a
// ragged one.
//
// Per ticket:
//   1. load the slices into registers (bounds-checked, non-temporal buffer loads); per wave, max and
//      e = exp2(l c - ref_w), ref_w = max * c, sums; fold the waves into one record per row
//      (ref, sum e, sum e t) and publish it, then an arrival flag;
//   2. paired positions: wait for the team's arrival flags, combine the team's records in
//      fp64 (normalisers) and form the slice's residual mass sum [p - q]_+ from the e-values
//      kept in registers, p = e_p alpha_p, q = e_q alpha_q (§3.2, §4.1: beta = sum [p - q]_+);
//      publish it.
// k_fused_finalize combines the team statistics (normaliser, entropy in bits and max
// probability as in the SpecKV page's signals, beta), runs the accept scan (§3.1 / §3.2, stop
// at the first rejection §5.1) and the three-level sampler over the residual or p_{g+1}
// (§5.2, one re-read chunk), and writes the outputs.
//
// Filtered uniform bf16 batches off the sparse path (top-p alone, top-k above 256; §2.1: p and
// q are the distributions after temperature, top-k and top-p): the MASK variant takes one
// threshold per row from the threshold kernel and turns every logit below it into -inf as the
// raw words arrive, so the records, residual masses and outputs are those of the filtered
// rows; the finalize masks the logits it reads again against the same thresholds.
//
// Synchronisation without read-modify-write atomics: records and flags carry the call's tag (a
// per-call sequence number, never 0) and travel through coherent agent-scope (sc1) loads and
// stores; a 16-byte record also carries a check word mixing the tag with its contents, so a
// stale or half-written record is never taken.  Polls are few and late: device-scope loads
// compete with the row stream.
// Progress: a workgroup waits only for the other slices of its own team, dispatched just before
// or after it on the same XCD.  Workgroups of an XCD are dispatched in order, and a team has
// far fewer members than an XCD has resident slots, so the oldest waiting team always has every
// member resident or finished.  Every wait is also bounded: one that expires reports
// SPEC_STATUS_TIMEOUT for its request instead of hanging.
#include <stdio.h>
#include <stdlib.h>

#include "spec_device.h"
#include "spec_internal.h"

namespace specv {

constexpr int kTeamTimeout = 4;

struct TeamL {      // team statistics of one position, kept in LDS by the finalizing workgroup
  double z[2];      // sum over the row of exp2(l c - M)
  double w[2];      // entropy numerator
  double beta;      // sum_x [p - q]_+
  float M[2];       // row reference (greedy: max logit)
  int amax;         // greedy: argmax
  int flags;        // kTeamBadP / kTeamBadQ / kTeamTimeout
};

struct FinScratch {
  TeamL team[kMaxGamma + 1];
  double py[kMaxGamma], qy[kMaxGamma];
  double us[kMaxGamma + 1][3];   // sampler uniforms (Philox words 1..3) of every position
  int ytok[kMaxGamma];
  double gm[kChunk / kGroup];
  int spick[kMaxGamma + 1];      // level-1 pick of each position taken early (-1: none)
  double ap[kMaxGamma];          // accept probability of every position
  alignas(16) float wall[kChunk];   // the picked chunk's sampler weights
  double u[3];
  double red[kWaves];
  unsigned long long lowm;       // positions whose 1 - TV or L1 is recomputed from the rows
  unsigned long long lowbm;      // of those, the ones whose beta needs fp64 normalisers
  int flags, status, n_acc, pos, wkind, y, kpick, xpick;
};

struct LdsFin {
  int cu[kMaxReqFused + 1];
  int i[8];
  FinScratch fin;
};

// ---------------------------------------------------------------- tagged records

__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

// Slice records: 16 bytes {ref, sum e, sum e t, check}, stored and loaded whole through a
// buffer resource over the record array with agent-scope coherence (sc1).  check = tag ^
// mix(ref, s, w): a reader accepts a record only if the check matches this call's tag, so a
// record of an earlier call, or one read while it was being written, is never taken.
// Layout: [team][row: 0 target, 1 draft][slice].
__device__ __forceinline__ uint32_t rec_mix(uint32_t a, uint32_t b, uint32_t c) {
  return a ^ ((b << 11) | (b >> 21)) ^ ((c << 22) | (c >> 10)) ^ 0x9E3779B9u;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const FusedArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)a.part, (short)0, (int)((size_t)a.n_teams * 2 * a.n_s * 16),
                                           0x00020000);
}
__device__ __forceinline__ uint32_t rec_off(int n_s, int r, int s, int row) {
  return (uint32_t)(((r * 2 + row) * n_s + s) * 16);
}
__device__ __forceinline__ void store_rec(__amdgpu_buffer_rsrc_t rs, uint32_t off, float ref, float s, float w,
                                          uint32_t tag) {
  const uint32_t x = __float_as_uint(ref), y = __float_as_uint(s), z = __float_as_uint(w);
  const __attribute__((ext_vector_type(4))) uint32_t v = {x, y, z, tag ^ rec_mix(x, y, z)};
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0x10);
}
struct Rec {
  uint32_t x, y, z, c;
};
__device__ __forceinline__ Rec load_rec_raw(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0x10);
  return Rec{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ bool rec_ok(const Rec& q, uint32_t tag) { return (q.c ^ rec_mix(q.x, q.y, q.z)) == tag; }
__device__ __forceinline__ bool load_rec(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t tag, float& ref, float& s,
                                         float& w) {
  const Rec q = load_rec_raw(rs, off);
  ref = __uint_as_float(q.x); s = __uint_as_float(q.y); w = __uint_as_float(q.z);
  return rec_ok(q, tag);
}

__device__ __forceinline__ bool wave_all(bool v) { return __ballot(!v) == 0ull; }

// ---------------------------------------------------------------- block reductions

// Sum / max of N floats over the workgroup; every thread gets the results.  Callers put a
// __syncthreads() between consecutive uses of `red`.
template <int N>
__device__ __forceinline__ void block_sum_f(float (&v)[N], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = wave_sum_dpp(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) red[k * kWaves + wave] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    float s = red[k * kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[k * kWaves + w];
    v[k] = s;
  }
}

template <int N>
__device__ __forceinline__ void block_max_f(float (&v)[N], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = wave_max_dpp(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) red[k * kWaves + wave] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    float s = red[k * kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s = fmaxf(s, red[k * kWaves + w]);
    v[k] = s;
  }
}

// Fixed-order fp64 combine of one row's slice records held one per lane (lanes >= n_s hold
// ref = -inf, s = 0): M = max ref, z = sum s 2^(ref - M), w = sum 2^(ref - M) (w_s + s_s (ref - M)).
// Several wave reductions at once, step by step in the fixed order of wave_sum_dpp_d /
// wave_max_dpp for every value, so that their DPP latencies overlap; every lane gets the
// results.
template <int N>
__device__ __forceinline__ void wave_sums_dpp_d(double (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0xb1, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0x4e, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0x124, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0x128, 0xf>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0x142, 0xa>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_d<0x143, 0xc>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = readlane_d(v[i], 63);
}
template <int N>
__device__ __forceinline__ void wave_maxs_dpp(float (&v)[N]) {
  const float ninf = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0xb1, 0xf));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0x4e, 0xf));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0x124, 0xf));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0x128, 0xf));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0x142, 0xa));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], SPEC_DPP(ninf, v[i], 0x143, 0xc));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[i]), 63));
}
// Two inverse-CDF picks (wave_pick) side by side.
__device__ __forceinline__ void wave_pick2(const double (&m)[2], int n, const double (&u)[2], int (&pick)[2]) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < n;
  double cum[2] = {in ? m[0] : 0.0, in ? m[1] : 0.0};
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x111, 0xf>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x112, 0xf>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x114, 0xf>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x118, 0xf>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x142, 0xa>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) cum[i] += dpp_d<0x143, 0xc>(cum[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double total = readlane_d(cum[i], 63);
    const unsigned long long over = __ballot(in && cum[i] > u[i] * total);
    const unsigned long long pos = __ballot(in && m[i] > 0.0);
    pick[i] = !(total > 0.0) ? -1 : (over ? __builtin_ctzll(over) : (pos ? 63 - __builtin_clzll(pos) : -1));
  }
}

// ---------------------------------------------------------------- finalize one request

// One request: combine its teams' records (normaliser, entropy in bits and max probability as
// in the SpecKV page's signals, beta = sum [p - q]_+), run the accept scan (guide page
// "5.1 投机解码核心原理" §3.1 / §3.2, stop at the first rejection §5.1) and the three-level
// sampler over the residual or p_{g+1} (§5.2), and write the outputs.  Scans over chunk,
// group and element masses are wave-wide fp64 prefix sums.
// Stage the draft offsets in LDS and check them as one exclusive prefix (every request is
// refused when any offset is out of order).
template <int N>
__device__ __forceinline__ bool stage_cu(const FusedArgs& a, const int (&pre)[N], int* cu, int* red) {
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < N; ++k)
    if (t + k * kThreads <= a.B) cu[t + k * kThreads] = pre[k];
  __syncthreads();
  int bad = 0;
  for (int k = t; k < a.B; k += kThreads) {
    const int g = cu[k + 1] - cu[k];
    if (g < 0 || g > a.G) bad = 1;
  }
  if (t == 0 && (cu[0] != 0 || cu[a.B] != a.n_draft_rows)) bad = 1;
  return block_or(bad, red) != 0;
}

// One team's raw workspace entries, loaded by one wave (one slice per lane).
struct TeamRaw {
  Rec P, Q;
  uint64_t m[kWaves];
};
template <int MODE>
__device__ __forceinline__ TeamRaw team_load(const FusedArgs& a, __amdgpu_buffer_rsrc_t rrs, int c0, int b, int g,
                                             int ti) {
  const int lane = threadIdx.x & 63;
  TeamRaw R;
  R.P = Rec{0, 0, 0, 0};
  R.Q = Rec{0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) R.m[w] = 0;
  if (ti <= g && lane < a.n_s) {
    const int r = c0 + b + ti;
    R.P = load_rec_raw(rrs, rec_off(a.n_s, r, lane, 0));
    if (MODE == kFuSample && ti < g) {
      R.Q = load_rec_raw(rrs, rec_off(a.n_s, r, lane, 1));
      const uint64_t* mw = a.smass + ((int64_t)r * a.n_s + lane) * kWaves;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) R.m[w] = ld_coh(mw + w);
    }
  }
  return R;
}

template <int DT, bool VEC, int MODE>
__device__ void finalize_request(const FusedArgs& a, LdsFin& L, int b) {
  FinScratch& F = L.fin;
  // the wave index in a scalar register, so that per-team values derived from it stay scalar
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int G1 = a.G + 1;
  const int n_s = a.n_s;
  const uint32_t tag = a.tag;
  const float nan = __int_as_float(0x7fc00000);
  const double cd = (double)a.c;
  const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
  // Every load of the request goes out before anything waits, at the guess c0 = b G, g = G
  // (exact when every request has G draft tokens): the first three teams of each wave, the draft
  // tokens and (sampling) their logits kept by the streaming kernel, the request's offsets and
  // the whole offset array.  A wrong guess loads the request's part again.
  const int cg = b * a.G;
  const bool guess_in = cg + a.G <= a.n_draft_rows;
  TeamRaw pre[3];   // teams wave, wave + 4 and (gamma >= 8) wave + 8
  int ytok = -1;
  float ly_p = 0.f, ly_q = 0.f;
  // filtered off the sparse path (uniform batches): position t's thresholds, target and draft
  float thp = -INFINITY, thq = -INFINITY;
  if (a.thr && guess_in && t <= a.G) {
    thp = a.thr[2 * (cg + b + t)];
    if (t < a.G) thq = a.thr[2 * (cg + b + t) + 1];
  }
  if (guess_in) {
    pre[0] = team_load<MODE>(a, rrs, cg, b, a.G, wave);
    pre[1] = team_load<MODE>(a, rrs, cg, b, a.G, wave + kWaves);
    pre[2] = team_load<MODE>(a, rrs, cg, b, a.G, wave + 2 * kWaves);
    if (t < a.G) {
      ytok = a.tokens[cg + t];
      if (MODE == kFuSample) { ly_p = a.ylog[2 * (cg + t)]; ly_q = a.ylog[2 * (cg + t) + 1]; }
    }
  }
  int c0 = a.cu[b], c1 = a.cu[b + 1];
  int cu_pre[(kMaxReqFused + 1 + kThreads - 1) / kThreads];
#pragma unroll
  for (int k = 0; k < (kMaxReqFused + 1 + kThreads - 1) / kThreads; ++k)
    cu_pre[k] = t + k * kThreads <= a.B ? a.cu[t + k * kThreads] : 0;
  double u_acc = 0.0;
  if (t <= a.G) {
    // the Philox block of position t (1-based i = t + 1): word 0 is the accept draw, words
    // 1..3 the sampler's uniforms if the emitted token is drawn there
    uint64_t w[4];
    philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(t + 1), 0, 0, w);
    u_acc = u53(w[0]);
    F.us[t][0] = u53(w[1]);
    F.us[t][1] = u53(w[2]);
    F.us[t][2] = u53(w[3]);
  }
  // this request's offsets are clamped into the declared arrays until the whole array is
  // checked below (an offset pair failing this test fails that check too)
  const bool gok = c0 >= 0 && c1 >= c0 && c1 - c0 <= a.G && c1 <= a.n_draft_rows && c0 + b + (c1 - c0) < a.n_teams;
  if (!gok) c0 = c1 = 0;
  const int g = c1 - c0;
  if (!(guess_in && c0 == cg && g == a.G)) {
    pre[0] = team_load<MODE>(a, rrs, c0, b, g, wave);
    pre[1] = team_load<MODE>(a, rrs, c0, b, g, wave + kWaves);
    pre[2] = team_load<MODE>(a, rrs, c0, b, g, wave + 2 * kWaves);
    ytok = t < g ? a.tokens[c0 + t] : -1;
    if (MODE == kFuSample && t < g) { ly_p = a.ylog[2 * (c0 + t)]; ly_q = a.ylog[2 * (c0 + t) + 1]; }
  }
  if (t >= g) ytok = -1;
  if (MODE == kFuTokenOnly && ytok >= 0 && ytok < a.V) ly_p = logit_at<DT>(row_ptr<DT>(a.tgt, a.tgt_ld, c0 + b + t), ytok);
  // a token below its row's threshold has probability 0 there (no threshold: -inf, nothing below)
  if (ly_p < thp) ly_p = -INFINITY;
  if (ly_q < thq) ly_q = -INFINITY;
  // the draft offsets as one exclusive prefix: every request is refused when any is out of order
  if (stage_cu(a, cu_pre, L.cu, L.i)) {
    if (t <= a.G) a.out_tokens[(int64_t)b * G1 + t] = -1;
    if (t == 0) {
      a.out_num_accepted[b] = 0;
      a.out_status[b] = kStBadGamma;
      if (a.out_req_stats)
        for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = nan;
    }
    return;
  }

  // A. combine each team's records (one wave per team, two teams per pass side by side); the
  // streaming kernel has finished.  The first two teams of each wave keep their per-slice p
  // records and residual masses in registers for the level-1 pick.  Sampling: for those teams
  // the level-1 pick of the token their position would emit (over [p - q]_+ for a paired
  // position, over p for the bonus position) is taken at once, and the picked chunk is touched
  // so that it sits in L2 when the sampler reads it (the touched words are only consumed at the
  // end, so that nothing waits for them).
  float kpr[2] = {-INFINITY, -INFINITY}, kps[2] = {0.f, 0.f};
  double ksm[2] = {0.0, 0.0};
  constexpr int kEsz = DT == kDtBF16 ? 2 : 4;
  constexpr int kTouch = kEsz / 2;   // 128-byte lines of a chunk row per lane
  uint32_t tch[2][2][kTouch];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < kTouch; ++h) tch[j][0][h] = tch[j][1][h] = 0u;
  const bool in = lane < n_s;
  for (int ti = wave, it = 0; ti <= g; ti += 2 * kWaves, it += 2) {
    const int tt[2] = {ti, ti + kWaves};
    TeamRaw R[2];
    R[0] = it == 0 ? pre[0] : (it == 2 ? pre[2] : team_load<MODE>(a, rrs, c0, b, g, tt[0]));
    R[1] = it == 0 ? pre[1] : team_load<MODE>(a, rrs, c0, b, g, tt[1]);
    // rows 2j (p) and 2j + 1 (q) of team j
    float ref[4], s[4], w[4];
    double sm[2];
    bool ok[2], pair[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pair[j] = (MODE == kFuSample) && tt[j] < g;
      ref[2 * j] = ref[2 * j + 1] = -INFINITY;
      s[2 * j] = s[2 * j + 1] = w[2 * j] = w[2 * j + 1] = 0.f;
      sm[j] = 0.0;
      ok[j] = true;
      if (in) {
        ok[j] = rec_ok(R[j].P, tag);
        ref[2 * j] = __uint_as_float(R[j].P.x); s[2 * j] = __uint_as_float(R[j].P.y); w[2 * j] = __uint_as_float(R[j].P.z);
        if (pair[j]) {
          ok[j] = ok[j] && rec_ok(R[j].Q, tag);
          ref[2 * j + 1] = __uint_as_float(R[j].Q.x); s[2 * j + 1] = __uint_as_float(R[j].Q.y);
          w[2 * j + 1] = __uint_as_float(R[j].Q.z);
#pragma unroll
          for (int q = 0; q < kWaves; ++q) {
            sm[j] += (double)lo_f(R[j].m[q]);
            ok[j] = ok[j] && tag_of(R[j].m[q]) == tag;
          }
        }
      }
    }
    if (it == 0) {
      kpr[0] = ref[0]; kps[0] = s[0]; ksm[0] = sm[0];
      kpr[1] = ref[2]; kps[1] = s[2]; ksm[1] = sm[1];
    }
    TeamL T[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      T[j].z[0] = T[j].z[1] = 1.0; T[j].w[0] = T[j].w[1] = 0.0; T[j].beta = 0.0; T[j].M[0] = T[j].M[1] = 0.f;
      T[j].amax = -1;
      T[j].flags = wave_all(ok[j]) ? 0 : kTeamTimeout;
    }
    if (MODE == kFuGreedy) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int qa = __float_as_int(s[2 * j]);
        const bool bad = in && (qa == -2 || ref[2 * j] == INFINITY);
        const float M = wave_max_dpp(in ? ref[2 * j] : -INFINITY);
        const int idx = wave_min_i((in && ref[2 * j] == M && qa >= 0) ? qa : INT_MAX);
        T[j].M[0] = M;
        T[j].amax = idx == INT_MAX ? -1 : idx;
        if (!wave_all(!bad) || !(M > -INFINITY)) { T[j].flags |= kTeamBadP; T[j].amax = -1; }
      }
    } else {
      // per row: M = max over slices, Z = sum s 2^(ref - M), W = sum 2^(ref - M) (w + s (ref - M))
      bool use[4], bad[4];
      float M[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        use[k] = in && ((k & 1) == 0 || pair[k >> 1]);
        bad[k] = use[k] && (!(s[k] == s[k]) || !(s[k] < INFINITY) || ref[k] == INFINITY);
        M[k] = use[k] ? ref[k] : -INFINITY;
      }
      wave_maxs_dpp(M);
      double sums[10];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double d = (double)ref[k] - (double)M[k];
        const double e = exp2_split(d);
        const bool on = use[k] && s[k] > 0.f;
        sums[2 * k] = on ? (double)s[k] * e : 0.0;
        // a ticket's entropy numerator rides on its slice-0 record, whose own sum is 0 when every
        // logit of that slice is masked while the other slice's are not: the numerator counts
        // whenever the record has a reference
        sums[2 * k + 1] = (use[k] && ref[k] > -INFINITY) ? e * ((double)w[k] + (double)s[k] * d) : 0.0;
      }
      sums[8] = in ? sm[0] : 0.0;
      sums[9] = in ? sm[1] : 0.0;
      wave_sums_dpp_d(sums);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        T[j].z[0] = sums[4 * j]; T[j].w[0] = sums[4 * j + 1]; T[j].M[0] = M[2 * j];
        if (!(wave_all(!bad[2 * j]) && sums[4 * j] > 0.0 && M[2 * j] > -INFINITY)) T[j].flags |= kTeamBadP;
        if (pair[j]) {
          T[j].z[1] = sums[4 * j + 2]; T[j].w[1] = sums[4 * j + 3]; T[j].M[1] = M[2 * j + 1];
          if (!(wave_all(!bad[2 * j + 1]) && sums[4 * j + 2] > 0.0 && M[2 * j + 1] > -INFINITY)) T[j].flags |= kTeamBadQ;
          // a slice whose team wait gave up marked its residual mass NaN
          if (!wave_all(!(in && !(sm[j] == sm[j])))) T[j].flags |= kTeamTimeout;
          T[j].beta = sums[8 + j];
        }
      }
    }
    int spick[2] = {-1, -1};
    if (MODE == kFuSample && it == 0) {
      // the masses the level-1 pick takes for each team's position (wkind 1 paired, 0 bonus)
      double m[2], u[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool on = in && tt[j] <= g && T[j].flags == 0;
        const double mp = s[2 * j] > 0.f ? (double)s[2 * j] * exp2_split((double)ref[2 * j] - (double)T[j].M[0]) / T[j].z[0] : 0.0;
        m[j] = on ? (pair[j] ? sm[j] : mp) : 0.0;
        u[j] = F.us[min(tt[j], g)][0];
      }
      wave_pick2(m, n_s, u, spick);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = c0 + b + min(tt[j], g);
        const __amdgpu_buffer_rsrc_t rt = row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V * kEsz);
        const __amdgpu_buffer_rsrc_t rd = row_rsrc(row_ptr<DT>(a.drf, a.drf_ld, c0 + min(tt[j], g)), a.V * kEsz);
#pragma unroll
        for (int h = 0; h < kTouch; ++h) {
          const int line = spick[j] * kChunk * kEsz + (h * 64 + lane) * 128;
          // a team without a pick (or without a draft row) reads past the resource: no access
          tch[j][0][h] = __builtin_amdgcn_raw_buffer_load_b32(rt, spick[j] >= 0 ? line : 0x40000000, 0, 0);
          tch[j][1][h] = __builtin_amdgcn_raw_buffer_load_b32(rd, spick[j] >= 0 && pair[j] ? line : 0x40000000, 0, 0);
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (tt[j] <= g) {
          F.team[tt[j]] = T[j];
          F.spick[tt[j]] = spick[j];
        }
    }
  }
  __syncthreads();

  // B. the accept test of every position: p(y), q(y) and the accept draw
  bool rej = false, low = false, lowb = false;
  int why = 0;
  if (t < g) {
    const TeamL T = F.team[t];
    const bool okp = (T.flags & (kTeamBadP | kTeamTimeout)) == 0;
    const int y = ytok;
    const bool yv = y >= 0 && y < a.V;
    double pyd = 0.0, qyd = 1.0, ap = nan;
    if (MODE == kFuGreedy) {
      ap = okp ? ((yv && y == T.amax) ? 1.0 : 0.0) : nan;
    } else {
      if (okp && yv) pyd = exp2_split((double)ly_p * cd - (double)T.M[0]) / T.z[0];
      if (MODE == kFuTokenOnly) {
        ap = okp ? (yv ? fmin(1.0, pyd) : 0.0) : nan;
      } else {
        const bool okq = (T.flags & (kTeamBadQ | kTeamTimeout)) == 0;
        if (okq && yv) qyd = exp2_split((double)ly_q * cd - (double)T.M[1]) / T.z[1];
        if (okp && okq) {
          // a requested output whose fp32 streaming sum would lose its relative precision:
          // L1 = 2 beta when the distributions nearly coincide, 1 - TV when they barely overlap
          lowb = a.st.l1 && T.beta < kPairRefine;
          low = lowb || (a.st.one_minus_tv && 1.0 - T.beta < kPairRefine);
          ap = (yv && qyd > 0.0) ? fmin(1.0, pyd / qyd) : 0.0;
        }
      }
    }
    F.ap[t] = ap;
    F.ytok[t] = y;
    F.py[t] = pyd;
    F.qy[t] = qyd;
    // the accept test of position t (evaluated for every position; the scan takes the first)
    if (!yv) { rej = true; why = kStBadToken; }
    else if (MODE == kFuGreedy) rej = y != T.amax;
    else if (!(qyd > 0.0)) { rej = true; why = kStZeroQ; }
    else rej = !(u_acc < fmin(1.0, pyd / qyd));
  }
  // C. request flags and the first rejection (wave 0 covers positions 0..63)
  if (wave == 0) {
    // flags of every team (positions 0..g; wave 0 holds 0..63, lane 0 adds position 64)
    int fl = lane <= g ? F.team[lane].flags : 0;
    if (lane == 0 && g >= 64) fl |= F.team[64].flags;
    fl = wave_or(fl);
    const unsigned long long rm = __ballot(rej);
    const unsigned long long lm = __ballot(low);
    const unsigned long long lbm = __ballot(lowb);
    const int j = rm ? __builtin_ctzll(rm) : -1;
    const int whyj = j >= 0 ? __builtin_amdgcn_readlane(why, j) : 0;
    if (lane == 0) {
      int status = 0;
      if (fl & kTeamTimeout) status = kStTimeout;
      else if (fl) status = kStNonfinite;
      else status = whyj;
      const bool stop = (status & (kStTimeout | kStNonfinite)) != 0;
      const int jj = stop ? -1 : j;
      F.n_acc = jj < 0 ? g : jj;
      F.pos = jj < 0 ? g : jj;
      F.y = jj >= 0 ? F.ytok[jj] : -1;
      // wkind: 0 = p of the row, 1 = [p - q]_+, 2 = p without token y
      F.wkind = (jj < 0) ? 0 : (MODE == kFuSample ? 1 : 2);
      F.u[0] = F.us[F.pos][0];
      F.u[1] = F.us[F.pos][1];
      F.u[2] = F.us[F.pos][2];
      F.status = status;
      F.kpick = -1;
      F.flags = fl;
      F.lowm = lm;
      F.lowbm = lbm;
    }
  }
  __syncthreads();

  int x = -1;
  const bool sampled = MODE != kFuGreedy && !(F.status & (kStTimeout | kStNonfinite));
  const int rpos = c0 + b + F.pos;
  const TeamL TP = F.team[F.pos];
  if (sampled) {
    // D. level 1 over the chunk masses (p's masses again if the residual turned out empty), by
    // the wave that combined team F.pos: taken already in A when that team was one of its
    // first two; otherwise its per-slice values are still in registers (or read again)
    const int own = F.pos & (kWaves - 1), oit = F.pos / kWaves;
    if (wave == own) {
      const bool kept = oit < 2;
      const float kr = (oit & 1) ? kpr[1] : kpr[0], ks = (oit & 1) ? kps[1] : kps[0];
      const double km = (oit & 1) ? ksm[1] : ksm[0];
      int wkind = F.wkind;
      int pick = MODE == kFuSample ? F.spick[F.pos] : -1;
      for (int pass = 0; pass < 2 && pick < 0; ++pass) {
        double m = 0.0;
        if (lane < n_s) {
          if (wkind == 1) {
            if (kept) {
              m = km;
            } else {
              const uint64_t* mw = a.smass + ((int64_t)rpos * n_s + lane) * kWaves;
#pragma unroll
              for (int w = 0; w < kWaves; ++w) m += (double)lo_f(ld_coh(mw + w));
            }
          } else {
            float ref = kr, sv = ks, wv;
            if (!kept) load_rec(rrs, rec_off(n_s, rpos, lane, 0), tag, ref, sv, wv);
            m = sv > 0.f ? (double)sv * exp2_split((double)ref - (double)TP.M[0]) / TP.z[0] : 0.0;
            if (wkind == 2) {
              const int y = F.y;
              if (y >= 0 && y < a.V && y / kChunk == lane) m = fmax(m - F.py[F.pos], 0.0);
            }
          }
        }
        double tot;
        pick = wave_pick(m, n_s, F.u[0], tot);
        if (pick >= 0 || wkind == 0) break;
        wkind = 0;
        if (lane == 0) F.status |= kStResidualEmpty;
      }
      if (lane == 0) { F.kpick = pick; F.wkind = wkind; }
    }
    __syncthreads();
  }
  // E1. the picked chunk's logits and its records go out; the statistics below are formed while
  // they travel
  const int k = sampled ? F.kpick : -1;
  const int wkind = F.wkind;
  const int grp = t >> 2, quarter = t & 3;
  const int x0 = k * kChunk + grp * kGroup + quarter * 16;
  float wv[16], vq[16];
  float refp = 0.f, refq = 0.f, rr = 0.f;
  float ctp = -INFINITY, ctq = -INFINITY;   // the picked position's thresholds (filtered, uniform)
  if (k >= 0) {
    if (a.thr) {
      ctp = a.thr[2 * rpos];
      if (wkind == 1) ctq = a.thr[2 * rpos + 1];
    }
    load_run16<DT, VEC>(row_ptr<DT>(a.tgt, a.tgt_ld, rpos), a.V, x0, wv);
    if (wkind == 1) load_run16<DT, VEC>(row_ptr<DT>(a.drf, a.drf_ld, c0 + F.pos), a.V, x0, vq);
    float sp_, wp_;
    load_rec(rrs, rec_off(n_s, rpos, k, 0), tag, refp, sp_, wp_);
    if (wkind == 1) {
      float sq_, wq_;
      load_rec(rrs, rec_off(n_s, rpos, k, 1), tag, refq, sq_, wq_);
    }
  }

  // B2. per-position statistics (the SpecKV page's signals, 1 - TV, p(y), q(y), accept
  // probability) and the request's aggregates
  if (t <= g) {
    const int r = c0 + b + t;
    const TeamL T = F.team[t];
    const bool okp = (T.flags & (kTeamBadP | kTeamTimeout)) == 0;
    const float hp = (float)(log2_split(T.z[0]) - T.w[0] / T.z[0]);
    if (a.st.target_entropy_bits) a.st.target_entropy_bits[r] = okp ? (MODE == kFuGreedy ? 0.f : hp) : nan;
    if (a.st.target_max_prob)
      a.st.target_max_prob[r] = okp ? (MODE == kFuGreedy ? 1.f : (float)(1.0 / T.z[0])) : nan;
  }
  float dh = nan, dm = nan;
  if (t < g) {
    const int drow = c0 + t;
    const TeamL T = F.team[t];
    const bool okp = (T.flags & (kTeamBadP | kTeamTimeout)) == 0;
    const int y = F.ytok[t];
    const bool yv = y >= 0 && y < a.V;
    const double pyd = F.py[t], qyd = F.qy[t];
    float py = nan, qy = nan, ovl = nan, l1 = nan;
    if (MODE == kFuGreedy) {
      py = (okp && yv) ? (y == T.amax ? 1.f : 0.f) : nan;
      qy = yv ? 1.f : nan;
      ovl = okp ? (yv ? py : 0.f) : nan;
      l1 = (okp && yv) ? (y == T.amax ? 0.f : 2.f) : nan;
    } else {
      if (okp && yv) py = (float)pyd;
      if (MODE == kFuTokenOnly) {
        qy = yv ? 1.f : nan;
        ovl = okp ? (yv ? py : 0.f) : nan;
        dh = yv ? 0.f : nan;
        dm = yv ? 1.f : nan;
        l1 = (okp && yv) ? (float)(2.0 * (1.0 - pyd)) : nan;
      } else {
        const bool okq = (T.flags & (kTeamBadQ | kTeamTimeout)) == 0;
        if (okq && yv) qy = (float)qyd;
        if (okp && okq) {
          ovl = (float)(1.0 - T.beta);
          l1 = (float)(2.0 * T.beta);
        }
        dh = okq ? (float)(log2_split(T.z[1]) - T.w[1] / T.z[1]) : nan;
        dm = okq ? (float)(1.0 / T.z[1]) : nan;
      }
    }
    const bool lw = (F.lowm >> t) & 1ull;
    if (a.st.p_y) a.st.p_y[drow] = py;
    if (a.st.q_y) a.st.q_y[drow] = qy;
    if (a.st.one_minus_tv && !lw) a.st.one_minus_tv[drow] = ovl;
    if (a.st.l1 && !lw) a.st.l1[drow] = l1;
    if (a.st.draft_entropy_bits) a.st.draft_entropy_bits[drow] = dh;
    if (a.st.draft_max_prob) a.st.draft_max_prob[drow] = dm;
    if (a.st.accept_prob) a.st.accept_prob[drow] = (float)F.ap[t];
  }
  if (wave == 0) {
    // the request's draft-signal aggregates in position order (positions 0..g-1 are lanes of
    // this wave)
    if (a.out_req_stats) {
      float rq[4] = {nan, nan, nan, nan};
      if (g > 0 && MODE != kFuGreedy) {
        double hs = 0.0, cs = 0.0;
        float hmax = -INFINITY, cmin = INFINITY;
        bool anynan = false;
        for (int i = 0; i < g; ++i) {
          const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dh), i));
          const float cm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dm), i));
          if (!(h == h) || !(cm == cm)) anynan = true;
          hs += h; cs += cm;
          hmax = fmaxf(hmax, h); cmin = fminf(cmin, cm);
        }
        if (!anynan) { rq[0] = (float)(hs / g); rq[1] = (float)(cs / g); rq[2] = hmax; rq[3] = cmin; }
      }
      if (lane == 0)
        for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = rq[q];
    }
    if (lane == 0 && a.st.expected_committed)
      a.st.expected_committed[b] = F.flags ? nan : expected_committed(F.ap, g);
  }

  if (k >= 0) {
    // E2. levels 2 and 3 inside chunk k.  Weights are relative within the chunk: e_p (p only)
    // or max(e_p r - e_q, 0) with r = alpha_p / alpha_q.  Logits below a row's threshold weigh 0.
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (wv[e] < ctp) wv[e] = -INFINITY;
      if (vq[e] < ctq) vq[e] = -INFINITY;
    }
    if (wkind == 1) {
      // a chunk where q keeps nothing (its reference is -inf: every draft logit masked) has
      // [p - q]_+ = p there, so its weights are e_p alone
      const bool hq = refq > -INFINITY;
      if (hq) {
        const double alp = exp2_split((double)refp - (double)TP.M[0]) / TP.z[0];
        const double alq = exp2_split((double)refq - (double)TP.M[1]) / TP.z[1];
        rr = (float)(alp / alq);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ep = __builtin_amdgcn_exp2f(fmaf(wv[e], a.c, -refp));
        if (hq) {
          const float eq = __builtin_amdgcn_exp2f(fmaf(vq[e], a.c, -refq));
          wv[e] = fmaxf(fmaf(ep, rr, -eq), 0.f);
        } else {
          wv[e] = ep;
        }
      }
    } else {
      const int yx = F.y;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float ep = __builtin_amdgcn_exp2f(fmaf(wv[e], a.c, -refp));
        wv[e] = (wkind == 2 && x0 + e == yx) ? 0.f : ep;
      }
    }
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) part += (double)wv[e];
    // group sum over the 4 threads of a group (quad lanes), in a fixed order
    part += dpp_d<0xb1, 0xf>(part);
    part += dpp_d<0x4e, 0xf>(part);
    if (quarter == 0) F.gm[grp] = part;
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *(float4*)&F.wall[grp * kGroup + quarter * 16 + e] = make_float4(wv[e], wv[e + 1], wv[e + 2], wv[e + 3]);
    __syncthreads();
    if (wave == 0) {
      // level 2 over the chunk's groups, level 3 inside the picked group
      const int n_in = min(kChunk, a.V - k * kChunk);
      const int n_groups = (n_in + kGroup - 1) / kGroup;
      double tot;
      const int gsel = wave_pick(lane < n_groups ? F.gm[lane] : 0.0, n_groups, F.u[1], tot);
      int pick = -1;
      if (gsel >= 0) {
        const int lo = k * kChunk + gsel * kGroup;
        const int n = min(kGroup, a.V - lo);
        pick = wave_pick(lane < n ? (double)F.wall[gsel * kGroup + lane] : 0.0, n, F.u[2], tot);
        if (pick >= 0) pick += lo;
      }
      if (lane == 0) F.xpick = pick;
    }
    __syncthreads();
    x = F.xpick;
  } else if (MODE == kFuGreedy && !(F.status & (kStTimeout | kStNonfinite))) {
    x = TP.amax;
  }
  // F. outputs
  const bool ok = !(F.status & (kStTimeout | kStNonfinite));
  if (t <= a.G) {
    int tok = -1;
    if (ok) {
      if (t < F.n_acc) tok = F.ytok[t];
      else if (t == F.n_acc) tok = x;
    }
    a.out_tokens[(int64_t)b * G1 + t] = tok;
  }
  if (t == 0) {
    a.out_num_accepted[b] = ok ? F.n_acc : 0;
    a.out_status[b] = F.status;
  }

  // positions whose requested 1 - TV or L1 the fp32 streaming sums cannot give: when beta is
  // small, A and beta again with fp64 normalisers (pair_sums_fp64, two passes); when only the
  // overlap is small, A directly as a sum of positive terms with the team's normalisers
  // (pair_overlap, one pass), beta as streamed
  if (MODE == kFuSample && (a.st.one_minus_tv || a.st.l1)) {
    unsigned long long lm = F.lowm;
    const unsigned long long lbm = F.lowbm;
    while (lm) {
      const int i = __builtin_ctzll(lm);
      lm &= lm - 1;
      const TeamL T = F.team[i];
      const void* prow = row_ptr<DT>(a.tgt, a.tgt_ld, c0 + b + i);
      const void* qrow = row_ptr<DT>(a.drf, a.drf_ld, c0 + i);
      const float tp = a.thr ? a.thr[2 * (c0 + b + i)] : -INFINITY;
      const float tq = a.thr ? a.thr[2 * (c0 + b + i) + 1] : -INFINITY;
      double A, beta;
      if ((lbm >> i) & 1ull) {
        pair_sums_fp64<DT, VEC, false>(prow, qrow, a.V, a.c, T.M[0], T.M[1], tp, tq, F.red, A, beta);
      } else {
        A = pair_overlap<DT, VEC>(prow, qrow, a.V, a.c, T.M[0], T.M[1], T.z[0], T.z[1], tp, tq, F.red);
        beta = T.beta;
      }
      if (t == 0) {
        if (a.st.one_minus_tv) a.st.one_minus_tv[c0 + i] = (float)A;
        if (a.st.l1) a.st.l1[c0 + i] = (float)(2.0 * beta);
      }
    }
  }
  // the touched words are kept alive (their loads have long completed)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < kTouch; ++h) asm volatile("" ::"v"(tch[j][0][h]), "v"(tch[j][1][h]));
}

// ---------------------------------------------------------------- streaming kernel

// DPP wave reductions, one v_*_dpp per step (row butterflies, then row broadcasts); the
// result is valid in lane 63.  Written out because the compiler's versions add a move and a
// canonicalising max per step.  Values are interleaved so that each DPP read comes at least
// two instructions after the write of its source; a block starts with s_nop 1 for the
// instructions just before it.
#define SPEC_DPP4(op, ctrl)                                \
  "v_" op "_f32_dpp %0, %0, %0 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %1, %1, %1 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %2, %2, %2 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %3, %3, %3 " ctrl "\n\t"
#define SPEC_DPP3(op, ctrl)                                \
  "v_" op "_f32_dpp %0, %0, %0 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %1, %1, %1 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %2, %2, %2 " ctrl "\n\t"
#define SPEC_DPP1(op, ctrl)                                \
  "v_" op "_f32_dpp %0, %0, %0 " ctrl "\n\t"                \
  "s_nop 1\n\t"
#define SPEC_DPP2(op, ctrl)                                \
  "v_" op "_f32_dpp %0, %0, %0 " ctrl "\n\t"                \
  "v_" op "_f32_dpp %1, %1, %1 " ctrl "\n\t"                \
  "s_nop 0\n\t"
#define SPEC_DPP_STEPS(M, op)                                             \
  M(op, "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf")                 \
  M(op, "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf")                 \
  M(op, "row_ror:4 row_mask:0xf bank_mask:0xf")                           \
  M(op, "row_ror:8 row_mask:0xf bank_mask:0xf")                           \
  M(op, "row_bcast:15 row_mask:0xa bank_mask:0xf")                        \
  M(op, "row_bcast:31 row_mask:0xc bank_mask:0xf")

__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ void dpp_sum4(float& a, float& b, float& c, float& d) {
  asm volatile("s_nop 1\n\t" SPEC_DPP_STEPS(SPEC_DPP4, "add") : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
  a = lane63(a); b = lane63(b); c = lane63(c); d = lane63(d);
}
__device__ __forceinline__ void dpp_sum3(float& a, float& b, float& c) {
  asm volatile("s_nop 1\n\t" SPEC_DPP_STEPS(SPEC_DPP3, "add") : "+v"(a), "+v"(b), "+v"(c));
  a = lane63(a); b = lane63(b); c = lane63(c);
}
__device__ __forceinline__ void dpp_sum2(float& a, float& b) {
  asm volatile("s_nop 1\n\t" SPEC_DPP_STEPS(SPEC_DPP2, "add") : "+v"(a), "+v"(b));
  a = lane63(a); b = lane63(b);
}
__device__ __forceinline__ void dpp_max1(float& a) {
  asm volatile("s_nop 1\n\t" SPEC_DPP_STEPS(SPEC_DPP1, "max") : "+v"(a));
  a = lane63(a);
}
__device__ __forceinline__ void dpp_max2(float& a, float& b) {
  asm volatile("s_nop 1\n\t" SPEC_DPP_STEPS(SPEC_DPP2, "max") : "+v"(a), "+v"(b));
  a = lane63(a); b = lane63(b);
}

// One ticket: a 4096-logit slice s of target row r, paired with the same slice of draft row
// drow when position r holds a draft token.  Every field is uniform over the workgroup.
struct Ticket {
  int r, s, drow;
  bool valid, pair;
};

// Raw-word views of one thread's slice (bf16 pairs or floats): the logits are unpacked where
// they are used, so no unpacked copy of a slice is ever held.  Element j of the slice is word
// j / 2 (bf16: low half first) or word j (fp32).
template <int DT>
__device__ __forceinline__ float raw_elem(const RawSlice<DT>& r, int j) {
  if constexpr (DT == kDtBF16) return (j & 1) ? bf16_hi(r.w[j >> 1]) : bf16_lo(r.w[j >> 1]);
  else return __uint_as_float(r.w[j]);
}
// Max of two slices given as raw words.  bf16: on the packed 16-bit patterns read as signed
// integers, non-negative values order like their patterns and negative ones (sign bit set) in
// reverse, so per half the largest non-negative pattern (the integer maximum, one packed op per
// two words), or failing any the negative pattern of least magnitude (the integer minimum,
// taken only by a wave in which some lane holds no non-negative value in a half), is the
// largest value.  No word is ever read as a float (a -inf high half would make it a signalling
// NaN).  A NaN pattern is ignored unless a half holds nothing else; a row holding one is
// reported from its sums either way.  fp32: the plain max (quiet NaN ignored).
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ float max_raw2(const RawSlice<DT>& r0, const RawSlice<DT>& r1) {
  if constexpr (DT == kDtBF16) {
    s16x2 mx = __builtin_elementwise_max(__builtin_bit_cast(s16x2, r0.w[0]), __builtin_bit_cast(s16x2, r1.w[0]));
#pragma unroll
    for (int k = 1; k < RawSlice<DT>::kWords; ++k)
      mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(__builtin_bit_cast(s16x2, r0.w[k]),
                                                                   __builtin_bit_cast(s16x2, r1.w[k])));
    uint32_t mw = __builtin_bit_cast(uint32_t, mx);
    if (__builtin_amdgcn_ballot_w64((mw & 0x80008000u) != 0u)) {
      s16x2 mn = __builtin_elementwise_min(__builtin_bit_cast(s16x2, r0.w[0]), __builtin_bit_cast(s16x2, r1.w[0]));
#pragma unroll
      for (int k = 1; k < RawSlice<DT>::kWords; ++k)
        mn = __builtin_elementwise_min(mn, __builtin_elementwise_min(__builtin_bit_cast(s16x2, r0.w[k]),
                                                                     __builtin_bit_cast(s16x2, r1.w[k])));
      const uint32_t nw = __builtin_bit_cast(uint32_t, mn);
      if (mw & 0x8000u) mw = (mw & 0xffff0000u) | (nw & 0xffffu);
      if (mw & 0x80000000u) mw = (mw & 0xffffu) | (nw & 0xffff0000u);
    }
    // both halves are quiet values or NaN patterns read from memory, never signalling
    // through arithmetic: the plain two-input maximum needs no canonicalising
    return __builtin_elementwise_maximum(__uint_as_float(mw << 16), __uint_as_float(mw & 0xffff0000u));
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < RawSlice<DT>::kWords; ++k) m = fmaxf(fmaxf(m, __uint_as_float(r0.w[k])), __uint_as_float(r1.w[k]));
    return m;
  }
}

// Logits at indices >= V (zeros from the bounds check) become -inf, on the raw words.
template <int DT>
__device__ __forceinline__ void mask_tail_raw(int V, int base, RawSlice<DT>& r) {
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (slice_index<DT>(base, threadIdx.x, j) < V) continue;
    if constexpr (DT == kDtBF16) r.w[j >> 1] = (j & 1) ? (r.w[j >> 1] & 0xffffu) | 0xff800000u : (r.w[j >> 1] & 0xffff0000u) | 0xff80u;
    else r.w[j] = 0xff800000u;
  }
}
// Filtering off the sparse path: every logit of a raw slice below the row's threshold becomes
// -inf (weight 0 from here on, as the logits past V); NaN compares false and stays, so a
// non-finite row is still reported.
template <int DT>
__device__ __forceinline__ void mask_below_raw(RawSlice<DT>& r, float tau) {
#pragma unroll
  for (int k = 0; k < RawSlice<DT>::kWords; ++k) {
    const uint32_t w = r.w[k];
    if constexpr (DT == kDtBF16) {
      const uint32_t lo = __uint_as_float(w << 16) < tau ? 0xff80u : (w & 0xffffu);
      const uint32_t hi = __uint_as_float(w & 0xffff0000u) < tau ? 0xff800000u : (w & 0xffff0000u);
      r.w[k] = hi | lo;
    } else {
      r.w[k] = __uint_as_float(w) < tau ? 0xff800000u : w;
    }
  }
}

// e = 2^(l c - ref) of a slice given as raw words, with s = sum e and (ENT) w = sum e (l c - ref).
// A masked logit (-inf) gives e = 0 and a NaN product in w; such a thread recomputes w from its
// e-values, using log2(e) for l c - ref.  Words are consumed in groups of two (four logits) so
// that the raw words die as the e-values appear.
template <int DT, bool ENT>
__device__ __forceinline__ void exp_raw(const RawSlice<DT>& r, float (&e)[kPerThread], float c, float ref, float& s,
                                        float& w) {
  w = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const float tt = fmaf(raw_elem<DT>(r, j), c, -ref);
    const float ej = __builtin_amdgcn_exp2f(tt);
    s = j == 0 ? ej : s + ej;
    if (ENT) w = j == 0 ? ej * tt : fmaf(ej, tt, w);
    e[j] = ej;
    if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
  if (ENT && !(w == w)) {
    w = 0.f;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (e[j] > 0.f) w = fmaf(e[j], __builtin_amdgcn_logf(e[j]), w);
  }
}

// e = 2^(l c - ref) in place over one slice, with s = sum e and (ENT) w = sum e (l c - ref).  A
// masked logit (-inf) gives e = 0 and a NaN product in w; such a thread recomputes w from its
// e-values, using log2(e) for l c - ref.
template <bool ENT>
__device__ __forceinline__ void exp_slice(float (&v)[kPerThread], float c, float ref, float& s, float& w) {
  const float t0 = fmaf(v[0], c, -ref);
  const float e0 = __builtin_amdgcn_exp2f(t0);
  s = e0;
  w = ENT ? e0 * t0 : 0.f;
  v[0] = e0;
#pragma unroll
  for (int j = 1; j < kPerThread; ++j) {
    const float tt = fmaf(v[j], c, -ref);
    const float e = __builtin_amdgcn_exp2f(tt);
    s += e;
    if (ENT) w = fmaf(e, tt, w);
    v[j] = e;
  }
  if (ENT && !(w == w)) {
    w = 0.f;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (v[j] > 0.f) w = fmaf(v[j], __builtin_amdgcn_logf(v[j]), w);
  }
}

__device__ __forceinline__ float max_slice(const float (&v)[kPerThread], float m) {
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) m = fmaxf(m, v[j]);
  return m;
}

// exp_raw for a slice whose e-values go straight to LDS, four at a time (stash[k][thread]).
template <int DT, bool ENT>
__device__ __forceinline__ void exp_raw_stash(const RawSlice<DT>& r, float4 (*stash)[kThreads], float c, float ref,
                                              float& s, float& w) {
  const int t = threadIdx.x;
  w = 0.f;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    float e4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float tt = fmaf(raw_elem<DT>(r, 4 * k + q), c, -ref);
      e4[q] = __builtin_amdgcn_exp2f(tt);
      s = (k == 0 && q == 0) ? e4[q] : s + e4[q];
      if (ENT) w = (k == 0 && q == 0) ? e4[q] * tt : fmaf(e4[q], tt, w);
    }
    stash[k][t] = make_float4(e4[0], e4[1], e4[2], e4[3]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (ENT && !(w == w)) {
    w = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const float4 v = stash[k][t];
      const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e4[q] > 0.f) w = fmaf(e4[q], __builtin_amdgcn_logf(e4[q]), w);
    }
  }
}

struct FusedLds {
  float4 stash[kPerThread / 4][kThreads];   // a paired ticket's target e-values of slice 1
  float qtail[3][kThreads];   // and the last three of its draft e-values of slice 1
  float wp[2][kWaves][4];   // [row][wave] {ref, sum e over slice 0, over slice 1, sum e t}
  float tn[5];              // the team's normalisers {M_p, M_q, 1 / Z_p, 1 / Z_q, Z_q / Z_p}
  int tst;                  // team status: 0 ok, 1 non-finite row, 2 wait gave up
  int bad[kWaves];
  int amax[2][kWaves];
  int req;                  // ragged batches: the request of this place's draft row
};

// The lane that publishes a workgroup's records: lane 0 of the last wave (wave 0 polls).
constexpr int kStorer = kThreads - 64;

// Fold per-wave partials {ref_w, s_w, w_w} of one row's slice (ref_w = -inf for a wave that
// holds no finite logit; s_w = pw[w][K], w_w = pw[w][3] when W, else 0) into one record relative
// to ref = max_w ref_w: s = sum_w s_w 2^(ref_w - ref), w = sum_w 2^(ref_w - ref) (w_w + s_w (ref_w - ref)).
template <int K, bool W>
__device__ __forceinline__ void fold_waves(const float (*pw)[4], float& ref, float& s, float& w) {
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) M = fmaxf(M, pw[k][0]);
  ref = -INFINITY; s = 0.f; w = 0.f;   // a slice with no finite logit: no reference either
  if (!(M > -INFINITY)) return;
  ref = M;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (!(pw[k][0] > -INFINITY)) continue;
    const float d = pw[k][0] - M;
    const float f = __builtin_amdgcn_exp2f(d);
    s = fmaf(pw[k][K], f, s);
    w = fmaf(f, fmaf(pw[k][K], d, W ? pw[k][3] : 0.f), w);
  }
}

// fold_waves with the sum field K and the entropy flag W chosen at run time (one lane per record).
__device__ __forceinline__ void fold_waves_rt(const float (*pw)[4], int K, bool W, float& ref, float& s, float& w) {
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) M = fmaxf(M, pw[k][0]);
  ref = -INFINITY; s = 0.f; w = 0.f;   // a slice with no finite logit: no reference either
  if (!(M > -INFINITY)) return;
  ref = M;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (!(pw[k][0] > -INFINITY)) continue;
    const float d = pw[k][0] - M;
    const float f = __builtin_amdgcn_exp2f(d);
    const float sk = pw[k][K];
    s = fmaf(sk, f, s);
    w = fmaf(f, fmaf(sk, d, W ? pw[k][3] : 0.f), w);
  }
}

// Team normalisers from the team's records (lane s holds slice s): M = max_s ref_s and
// Z = sum_s s_s 2^(ref_s - M) for each row.  The residual's scale factors depend on the ratio
// of the two rows' normalisers, and an error in that ratio moves sum [p - q]_+ by the same
// relative amount times the mass where p > q; the sums and the ratios are therefore formed in
// fp64 (fixed-order DPP tree) and rounded to fp32 once.  Status 0 ok, 1 a row non-finite or
// empty, 2 the wait gave up.
struct TeamNorm {
  float Mp, Mq;
  float izp, izq;   // 1 / Z_p, 1 / Z_q
  float rqp;        // Z_q / Z_p
};
// 1 / z for z > 0 in fp64: the fp32 reciprocal refined by one Newton step (relative error near
// 2^-46), lighter on registers than a full fp64 division.
__device__ __forceinline__ double recip_d(double z) {
  const double r = (double)__builtin_amdgcn_rcpf((float)z);
  return r * fma(-z, r, 2.0);
}
__device__ __forceinline__ int team_norm(float pr, float ps, float qr, float qs, int n_s, bool timed_out,
                                         TeamNorm& N) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < n_s;
  const bool bad = in && (!(ps == ps) || !(ps < INFINITY) || pr == INFINITY || !(qs == qs) || !(qs < INFINITY) ||
                          qr == INFINITY);
  float Mp = in ? pr : -INFINITY, Mq = in ? qr : -INFINITY;
  dpp_max2(Mp, Mq);
  const double zp = wave_sum_dpp_d((in && ps > 0.f) ? (double)ps * exp2_split((double)pr - (double)Mp) : 0.0);
  const double zq = wave_sum_dpp_d((in && qs > 0.f) ? (double)qs * exp2_split((double)qr - (double)Mq) : 0.0);
  const bool ok = zp > 0.0 && zq > 0.0;
  const double izp = ok ? recip_d(zp) : 0.0;
  N.Mp = Mp;
  N.Mq = Mq;
  N.izp = (float)izp;
  N.izq = ok ? (float)recip_d(zq) : 0.f;
  N.rqp = (float)(zq * izp);
  if (timed_out) return 2;
  return (wave_all(!bad) && ok && Mp > -INFINITY && Mq > -INFINITY) ? 0 : 1;
}

// Residual mass of a wave's part of one paired slice, sum [p - q]_+ (guide page "5.1 投机
// 解码核心原理", §3.2 / §4.1: beta = sum [p - q]_+), from e-values e = 2^(l c - ref_w) taken
// relative to the wave's own references.  With a_p = 2^(ref_p - M_p) / Z_p (likewise a_q) and
// r = a_p / a_q: if r <= 1 the mass is a_q sum max(e_p r - e_q, 0), else a_p sum
// max(e_p - e_q / r, 0); e <= 1, so both terms stay below 1 and the max with 0 is the fma's
// clamp modifier.
struct ResidualScale {
  float rr, ir, scale;
  int form;   // 0: e_p r - e_q, 1: e_p - e_q / r, 2: e_p alone (no draft mass in this wave)
};
__device__ __forceinline__ ResidualScale residual_scale(const TeamNorm& N, float refp, float refq) {
  ResidualScale R = {0.f, 0.f, 0.f, 2};
  const float dp = refp - N.Mp, dq = refq - N.Mq;
  const float ap = refp > -INFINITY ? __builtin_amdgcn_exp2f(dp) * N.izp : 0.f;
  if (!(refq > -INFINITY)) { R.scale = ap; return R; }
  if (ap > 0.f) {
    R.rr = __builtin_amdgcn_exp2f(dp - dq) * N.rqp;   // a_p / a_q = 2^(dp - dq) Z_q / Z_p
    R.ir = 1.f / R.rr;
  }
  if (R.rr <= 1.f) { R.form = 0; R.scale = __builtin_amdgcn_exp2f(dq) * N.izq; }
  else { R.form = 1; R.scale = ap; }
  return R;
}

// Wave 0 of a paired ticket: wait until every member of the team has raised its arrival flag
// (the team's flags share one cache line, so a poll reads one line; lanes past the last member
// read the first flag again), then read the team's records (one slice per lane) and publish
// the team's normalisers to the workgroup through LDS.  A flag goes out right behind its
// records, so a record may still be in flight when the flag is seen: its check word then fails
// and the records are read again.  Every wait is bounded.
__device__ __forceinline__ void team_gather(const FusedArgs& a, FusedLds& L, int r, int n_u) {
  const int lane = threadIdx.x & 63;
  const int n_s = a.n_s;
  const int sl = min(lane, n_s - 1);
  const uint32_t tag = a.tag;
  const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
  const long long t0 = wall_clock64();
  // the launch's last generation polls sooner: the stream is draining, so an early poll no
  // longer competes with it (measured: 1.4 us less per launch on the batch-64 workload)
  const int pd = ((int)blockIdx.x + a.tail_wgs >= (int)gridDim.x) ? a.poll_delay / 2 : a.poll_delay;
  while (wall_clock64() - t0 < pd) __builtin_amdgcn_s_sleep(4);
  const uint32_t* fl = a.arrive + (int64_t)r * kMaxMembers + (lane < n_u ? lane : 0);
  unsigned spins = 0;
  bool timed_out = false;
  while (!wave_all(__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag)) {
    if (++spins > a.spin_limit) { timed_out = true; break; }
    for (int k = 0; k < a.poll_pause; ++k) __builtin_amdgcn_s_sleep(2);
  }
  // a poll that fails costs little (one line); the records are read once the flags are up
  Rec P = load_rec_raw(rrs, rec_off(n_s, r, sl, 0)), Q = load_rec_raw(rrs, rec_off(n_s, r, sl, 1));
  while (!timed_out && !wave_all(rec_ok(P, tag) && rec_ok(Q, tag))) {
    if (++spins > a.spin_limit) { timed_out = true; break; }
    __builtin_amdgcn_s_sleep(4);
    P = load_rec_raw(rrs, rec_off(n_s, r, sl, 0));
    Q = load_rec_raw(rrs, rec_off(n_s, r, sl, 1));
  }
  TeamNorm N;
  const int st = team_norm(__uint_as_float(P.x), __uint_as_float(P.y), __uint_as_float(Q.x), __uint_as_float(Q.y),
                           n_s, timed_out, N);
  if (lane == 0) {
    L.tn[0] = N.Mp;
    L.tn[1] = N.Mq;
    L.tn[2] = N.izp;
    L.tn[3] = N.izq;
    L.tn[4] = N.rqp;
    L.tst = st;
  }
}

// The logits of a paired position's draft token y in its target and draft rows, kept for the
// finalize kernel's accept test (p(y) and q(y)): written by the one ticket whose slices hold y,
// by a wave that would otherwise idle while wave 0 waits for the team.
template <int DT>
__device__ __forceinline__ void record_token_logits(const FusedArgs& a, int r, int drow, int base) {
  const int y = sload_i32(a.tokens + drow);
  if (y < base || y >= base + 2 * kChunk || y >= a.V) return;
  if ((threadIdx.x & 63) == 0) {
    a.ylog[2 * drow] = logit_at<DT>(row_ptr<DT>(a.tgt, a.tgt_ld, r), y);
    a.ylog[2 * drow + 1] = logit_at<DT>(row_ptr<DT>(a.drf, a.drf_ld, drow), y);
  }
}

__device__ __forceinline__ float residual_slice(const ResidualScale& R, const float (&ep)[kPerThread],
                                                const float (&eq)[kPerThread]) {
  float sm;
  if (R.form == 0) {
    sm = __builtin_amdgcn_fmed3f(fmaf(ep[0], R.rr, -eq[0]), 0.f, 1.f);
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) sm += __builtin_amdgcn_fmed3f(fmaf(ep[j], R.rr, -eq[j]), 0.f, 1.f);
  } else if (R.form == 1) {
    sm = __builtin_amdgcn_fmed3f(fmaf(eq[0], -R.ir, ep[0]), 0.f, 1.f);
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) sm += __builtin_amdgcn_fmed3f(fmaf(eq[j], -R.ir, ep[j]), 0.f, 1.f);
  } else {
    sm = ep[0];
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) sm += ep[j];
  }
  return sm * R.scale;
}


// One workgroup per ticket: slices 2u and 2u + 1 of one target row (the second one absent at an
// odd end), with the same slices of its draft row when the position pairs them.  Workgroup i
// runs on XCD i mod 8 (the dispatcher deals workgroups round-robin over the XCDs), and the
// tickets of the team in dispatch place ti go to consecutive workgroups of XCD ti mod 8.
// Phase 1 publishes one record per row and slice, then (paired tickets) an arrival flag; a
// paired ticket then waits for its team's flags, reads the team's records and forms its
// residual masses from e-values kept in registers (one slice of the target's and three of the
// draft's per thread in LDS).  A member waits only for members dispatched just before or
// after it on the same XCD; every wait is bounded.
// Eight waves per SIMD for aligned bf16 rows (64 VGPRs: three of a thread's draft e-values
// wait in LDS); other layouts keep the compiler's choice.  The masked variant's compares need
// 72 VGPRs: seven waves per SIMD, nothing spilled (at eight it spills 12-15 registers and runs
// slower; at six it has one workgroup per CU fewer).
constexpr int fused_min_waves(int dt, bool vec, bool mask) { return dt == kDtBF16 && vec ? (mask ? 7 : 8) : 1; }

template <int DT, bool VEC, int MODE, bool TENT, bool RAG, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(fused_min_waves(DT, VEC, MASK)))) void k_fused(
    FusedArgs a) {
  __shared__ FusedLds L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n_s = a.n_s, n_u = (n_s + 1) >> 1;
  const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int tl = jb / n_u;
  const int u = jb - tl * n_u;
  const int ti = tl * 8 + xcd;   // the team's place in dispatch order
  if (ti >= a.n_teams) return;
  const int s0 = 2 * u;
  const bool has1 = s0 + 1 < n_s;
  const uint32_t tag = a.tag;
  const float c = a.c;
  const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
  constexpr int kEsz = DT == kDtBF16 ? 2 : 4;
  const int base = s0 * kChunk;
  const bool tail = base + 2 * kChunk > a.V;   // the row's last ticket
  RawSlice<DT> rp[2], rq[2];
  int r = ti;   // target row
  bool pair = false;
  int drow = -1;
  if (MODE == kFuSample && RAG) {
    // a ragged batch: draft row d belongs to request b = #{b' in 1..B : cu[b'] <= d} (the offsets
    // ascend), counted by ballots over bounds-checked loads of the whole offset array, all at
    // once; a bonus place reads its request's end offset.  An invalid offset array (the finalize
    // kernel reports it) can only give rows that are range-checked here.
    pair = ti < a.n_draft_rows;
    drow = pair ? ti : -1;
    if (pair) {
      // wave 0 counts (the loads the batch needs, all at once); the others take its count
      if (wave == 0) {
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.cu), (short)0,
                                                                           (a.B + 1) * 4, 0x00020000);
        int cnt = 0;
#pragma unroll 1
        for (int k0 = 0; k0 < a.B; k0 += 256) {   // 256 offsets per round (one round up to B = 256)
          int cv[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) cv[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (1 + k0 + 64 * k + lane) * 4, 0, 0);
#pragma unroll
          for (int k = 0; k < 4; ++k) cnt += __popcll(__ballot(1 + k0 + 64 * k + lane <= a.B && cv[k] <= ti));
        }
        if (lane == 0) L.req = min(cnt, a.B - 1);
      }
      __syncthreads();
      r = ti + __builtin_amdgcn_readfirstlane(L.req);
    } else {
      const int b = ti - a.n_draft_rows;
      r = sload_i32(a.cu + b + 1) + b;
    }
    if (r < 0 || r >= a.n_teams) return;
    if (VEC) {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V * kEsz);
      load_raw_buf<DT>(rs, base, rp[0]);
      load_raw_buf<DT>(rs, base + kChunk, rp[1]);
      if (pair) {
        const __amdgpu_buffer_rsrc_t rd = row_rsrc(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V * kEsz);
        load_raw_buf<DT>(rd, base, rq[0]);
        load_raw_buf<DT>(rd, base + kChunk, rq[1]);
      }
    } else {
      load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base, rp[0]);
      load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base + kChunk, rp[1]);
      if (pair) {
        load_raw<DT, false>(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V, base, rq[0]);
        load_raw<DT, false>(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V, base + kChunk, rq[1]);
      }
    }
  } else if (MODE == kFuSample) {
    // Dispatch order: every paired position first (draft row d = ti, target row d + b for its
    // request b), then each request's bonus row (ti = n_draft_rows + b, target row
    // cu[b + 1] + b).  Bonus rows have no draft row and no team wait, so the kernel's last
    // workgroups are short ones that keep the memory busy while the paired teams before them
    // finish.  The loads go out at once for the guess b = d / G (exact when every request has
    // G draft tokens); scalar loads of cu then settle the request (a binary search when the
    // guess is wrong) and a wrong target row is loaded again.  An invalid offset array (the
    // finalize kernel reports it) can only give rows that are range-checked here.
    const int G1 = max(a.G, 1);
    const bool slot_pair = ti < a.n_draft_rows;
    const int bg = slot_pair ? min(ti / G1, a.B - 1) : ti - a.n_draft_rows;
    const int rg = min(slot_pair ? ti + bg : (bg + 1) * a.G + bg, a.n_teams - 1);
    if (VEC) {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, rg), a.V * kEsz);
      load_raw_buf<DT>(rs, base, rp[0]);
      load_raw_buf<DT>(rs, base + kChunk, rp[1]);
      const __amdgpu_buffer_rsrc_t rd =
          row_rsrc(slot_pair ? row_ptr<DT>(a.drf, a.drf_ld, ti) : a.tgt, slot_pair ? a.V * kEsz : 0);
      load_raw_buf<DT>(rd, base, rq[0]);
      load_raw_buf<DT>(rd, base + kChunk, rq[1]);
    }
    bool valid;
    if (slot_pair) {
      // the request of draft row d: the largest b < B with cu[b] <= d
      int b = bg, c0, c1;
      sload2_i32(a.cu + b, c0, c1);
      if (!(c0 <= ti && (b == a.B - 1 || c1 > ti))) {
        b = 0;
        int hi = a.B;
        while (hi - b > 1) {
          const int mid = (b + hi) >> 1;
          if (sload_i32(a.cu + mid) <= ti) b = mid;
          else hi = mid;
        }
        sload2_i32(a.cu + b, c0, c1);
      }
      r = ti + b;
      drow = ti;
      pair = c0 <= ti && ti < c1;
      valid = pair && r < a.n_teams;
    } else {
      r = sload_i32(a.cu + bg + 1) + bg;
      valid = r >= 0 && r < a.n_teams;
    }
    if (!valid) return;
    if (VEC) {
      if (r != rg) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V * kEsz);
        load_raw_buf<DT>(rs, base, rp[0]);
        load_raw_buf<DT>(rs, base + kChunk, rp[1]);
      }
    } else {
      load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base, rp[0]);
      load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base + kChunk, rp[1]);
      if (pair) {
        load_raw<DT, false>(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V, base, rq[0]);
        load_raw<DT, false>(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V, base + kChunk, rq[1]);
      }
    }
  } else if (VEC) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V * kEsz);
    load_raw_buf<DT>(rs, base, rp[0]);
    load_raw_buf<DT>(rs, base + kChunk, rp[1]);
  } else {
    load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base, rp[0]);
    load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, base + kChunk, rp[1]);
  }
  // filtering off the sparse path (uniform batches only): this team's thresholds, at logical
  // rows 2 r and 2 r + 1 (a uniform batch's target row r is its slot b (G + 1) + i)
  float tau_p = -INFINITY, tau_q = -INFINITY;
  if constexpr (MASK) {
    tau_p = __int_as_float(sload_i32((const int32_t*)a.thr + 2 * r));
    if (pair) tau_q = __int_as_float(sload_i32((const int32_t*)a.thr + 2 * r + 1));
  }
  if (MODE == kFuGreedy) {
    float vp[2][kPerThread];
    unpack_raw<DT>(rp[0], vp[0]);
    unpack_raw<DT>(rp[1], vp[1]);
    if (VEC && tail) {
      // logits past V (zeros from the bounds check) become -inf
      mask_tail<DT>(a.V, base, vp[0]);
      mask_tail<DT>(a.V, base + kChunk, vp[1]);
    }
    // greedy: per slice, the max, the lowest index of it, NaN / +inf seen
    float m[2];
    int idx[2], badv = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      m[k] = max_slice(vp[k], -INFINITY);
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) badv |= __builtin_amdgcn_class(vp[k][j], 0x203) ? 1 : 0;
    }
    dpp_max2(m[0], m[1]);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      idx[k] = INT_MAX;
      if (m[k] > -INFINITY) {
#pragma unroll
        for (int j = kPerThread - 1; j >= 0; --j)
          if (vp[k][j] == m[k]) idx[k] = slice_index<DT>(base + k * kChunk, t, j);
      }
      idx[k] = wave_min_i(idx[k]);
    }
    badv = wave_or(badv);
    if (lane == 0) {
      L.wp[0][wave][0] = m[0];
      L.wp[1][wave][0] = m[1];
      L.amax[0][wave] = idx[0];
      L.amax[1][wave] = idx[1];
      L.bad[wave] = badv;
    }
    __syncthreads();
    if (t == kStorer) {
      int bb = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) bb |= L.bad[w];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k == 1 && !has1) break;
        float M = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, L.wp[k][w][0]);
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (L.wp[k][w][0] == M) bi = min(bi, L.amax[k][w]);
        store_rec(rrs, rec_off(n_s, r, s0 + k, 0), M, __int_as_float(bb ? -2 : (bi == INT_MAX ? -1 : bi)), 0.f, tag);
      }
    }
    return;
  }
  // phase 1, target row: per-wave max, e-values, sums; a paired ticket parks slice 1's
  // e-values in LDS until its residual pass
  if (VEC && tail) {
    mask_tail_raw<DT>(a.V, base, rp[0]);
    mask_tail_raw<DT>(a.V, base + kChunk, rp[1]);
  }
  if constexpr (MASK) {
    mask_below_raw<DT>(rp[0], tau_p);
    mask_below_raw<DT>(rp[1], tau_p);
  }
  float mp = max_raw2<DT>(rp[0], rp[1]);
  dpp_max1(mp);
  float refp = mp > -INFINITY ? mp * c : 0.f;
  float ep[2][kPerThread];
  float sp0, sp1, wp0, wp1;
  // the target's entropy numerator only when its entropy is asked for (TENT); slice 1's
  // e-values of a paired ticket go to LDS as they are formed
  exp_raw<DT, TENT>(rp[0], ep[0], c, refp, sp0, wp0);
  if (pair) exp_raw_stash<DT, TENT>(rp[1], L.stash, c, refp, sp1, wp1);
  else exp_raw<DT, TENT>(rp[1], ep[1], c, refp, sp1, wp1);
  if (!(mp > -INFINITY)) refp = -INFINITY;
  // the target's partials are reduced before the draft row is unpacked, so that they hold no
  // registers there
  float wpe = wp0 + wp1;
  if (TENT) dpp_sum3(sp0, sp1, wpe);
  else dpp_sum2(sp0, sp1);
  if (lane == 0) {
    L.wp[0][wave][0] = refp;
    L.wp[0][wave][1] = sp0;
    L.wp[0][wave][2] = sp1;
    L.wp[0][wave][3] = wpe;
  }
  float sq0 = 0.f, sq1 = 0.f, wq = 0.f, refq = -INFINITY;
  float eq[2][kPerThread];
  if (pair) {
    // phase 1, draft row
    if (VEC && tail) {
      mask_tail_raw<DT>(a.V, base, rq[0]);
      mask_tail_raw<DT>(a.V, base + kChunk, rq[1]);
    }
    if constexpr (MASK) {
      mask_below_raw<DT>(rq[0], tau_q);
      mask_below_raw<DT>(rq[1], tau_q);
    }
    float mq = max_raw2<DT>(rq[0], rq[1]);
    dpp_max1(mq);
    refq = mq > -INFINITY ? mq * c : 0.f;
    float wq0, wq1;
    exp_raw<DT, true>(rq[0], eq[0], c, refq, sq0, wq0);
    exp_raw<DT, true>(rq[1], eq[1], c, refq, sq1, wq1);
#pragma unroll
    for (int k = 0; k < 3; ++k) L.qtail[k][t] = eq[1][kPerThread - 3 + k];
    wq = wq0 + wq1;
    if (!(mq > -INFINITY)) refq = -INFINITY;
    dpp_sum3(sq0, sq1, wq);
    if (lane == 0) {
      L.wp[1][wave][0] = refq;
      L.wp[1][wave][1] = sq0;
      L.wp[1][wave][2] = sq1;
      L.wp[1][wave][3] = wq;
    }
  }
  __syncthreads();
  if (wave == kWaves - 1) {
    // lanes 0..3 of the last wave fold and store the records (row k >> 1, slice k & 1) side by
    // side; slice 0 carries the ticket's entropy numerator, slice 1 none (the records of a row
    // are combined with a common reference, so the split does not matter)
    const int row = lane >> 1, sl = lane & 1;
    if (lane < 4 && (row == 0 || pair) && (sl == 0 || has1)) {
      float ref, sm, wm;
      fold_waves_rt(L.wp[row], 1 + sl, sl == 0, ref, sm, wm);
      store_rec(rrs, rec_off(n_s, r, s0 + sl, row), ref, sm, wm, tag);
    }
    asm volatile("" ::: "memory");
    // the arrival flag follows the records (a poller that sees it before they land re-reads)
    if (pair && lane == 0)
      __hip_atomic_store(a.arrive + (int64_t)r * kMaxMembers + u, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!pair) return;
  if (wave == 0) team_gather(a, L, r, n_u);
  else if (MODE == kFuSample && wave == 1) record_token_logits<DT>(a, r, drow, base);
  __syncthreads();
  const int st = L.tst;
  float m0 = 0.f, m1 = 0.f;
  if (st == 0) {
    TeamNorm N;
    N.Mp = L.tn[0];
    N.Mq = L.tn[1];
    N.izp = L.tn[2];
    N.izq = L.tn[3];
    N.rqp = L.tn[4];
    const ResidualScale R = residual_scale(N, refp, refq);
    m0 = residual_slice(R, ep[0], eq[0]);
    float ep1[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread / 4; ++k) {
      const float4 v4 = L.stash[k][t];
      ep1[4 * k] = v4.x; ep1[4 * k + 1] = v4.y; ep1[4 * k + 2] = v4.z; ep1[4 * k + 3] = v4.w;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) eq[1][kPerThread - 3 + k] = L.qtail[k][t];
    m1 = residual_slice(R, ep1, eq[1]);
  }
  dpp_sum2(m0, m1);
  // NaN marks a slice whose wait gave up; 0 when a row is non-finite
  if (st == 2) m0 = m1 = __int_as_float(0x7fc00000);
  if (lane == 0) {
    st_coh(a.smass + ((int64_t)r * n_s + s0) * kWaves + wave, tagged(m0, tag));
    if (has1) st_coh(a.smass + ((int64_t)r * n_s + s0 + 1) * kWaves + wave, tagged(m1, tag));
  }
}

// One workgroup per request, after the streaming kernel: every record is in place.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_fused_finalize(FusedArgs a) {
  __shared__ LdsFin L;
  finalize_request<DT, VEC, MODE>(a, L, blockIdx.x);
}

// ---------------------------------------------------------------- launch

template <int DT, bool VEC, int MODE>
static hipError_t launch_fused_t(FusedArgs a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int teams8 = (a.n_teams + 7) / 8;
  const long long grid = 8ll * teams8 * ((a.n_s + 1) / 2);
  if (grid < 1 || grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  // optional events bracket the streaming kernel alone (benchmark timing)
  // ragged sampling batches find each place's request among the offsets (a kernel of their own,
  // so that the uniform kernel keeps its registers)
  const bool rag = MODE == kFuSample && a.ragged;
  if constexpr (DT == kDtBF16 && VEC && MODE != kFuGreedy) {
    // filtered off the sparse path: the thresholds mask the logits (uniform batches)
    if (a.thr) {
      if (rag) return hipErrorInvalidValue;
      if (a.want_t_ent) launch_timed(k_fused<DT, VEC, MODE, true, false, true>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
      else launch_timed(k_fused<DT, VEC, MODE, false, false, true>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((k_fused_finalize<DT, VEC, MODE>), dim3(a.B), dim3(kThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.thr) return hipErrorInvalidValue;
  if (MODE != kFuGreedy && a.want_t_ent) {
    if (rag) launch_timed(k_fused<DT, VEC, MODE, true, true, false>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
    else launch_timed(k_fused<DT, VEC, MODE, true, false, false>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
  } else {
    if (rag) launch_timed(k_fused<DT, VEC, MODE, false, true, false>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
    else launch_timed(k_fused<DT, VEC, MODE, false, false, false>, dim3((unsigned)grid), dim3(kThreads), st, ev0, ev1, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_fused_finalize<DT, VEC, MODE>), dim3(a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a, int dt, int vec, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (dt == kDtBF16) {
    if (a.mode == kFuSample) return vec ? launch_fused_t<kDtBF16, true, kFuSample>(a, st, ev0, ev1) : launch_fused_t<kDtBF16, false, kFuSample>(a, st, ev0, ev1);
    if (a.mode == kFuTokenOnly) return vec ? launch_fused_t<kDtBF16, true, kFuTokenOnly>(a, st, ev0, ev1) : launch_fused_t<kDtBF16, false, kFuTokenOnly>(a, st, ev0, ev1);
    return vec ? launch_fused_t<kDtBF16, true, kFuGreedy>(a, st, ev0, ev1) : launch_fused_t<kDtBF16, false, kFuGreedy>(a, st, ev0, ev1);
  }
  if (a.mode == kFuSample) return vec ? launch_fused_t<kDtF32, true, kFuSample>(a, st, ev0, ev1) : launch_fused_t<kDtF32, false, kFuSample>(a, st, ev0, ev1);
  if (a.mode == kFuTokenOnly) return vec ? launch_fused_t<kDtF32, true, kFuTokenOnly>(a, st, ev0, ev1) : launch_fused_t<kDtF32, false, kFuTokenOnly>(a, st, ev0, ev1);
  return vec ? launch_fused_t<kDtF32, true, kFuGreedy>(a, st, ev0, ev1) : launch_fused_t<kDtF32, false, kFuGreedy>(a, st, ev0, ev1);
}

size_t fused_record_bytes() { return 16; }

}  // namespace specv
