// spec_fused.hip -- a whole verification round in two kernels: k_fused streams every needed
// logit once; k_fused_finalize (one workgroup per request) turns the records into outputs.
//
// Work unit ("ticket"): one 4096-logit slice of one target row, together with the same slice
// of its draft row when that position pairs the two (guide page "5.1 投机解码核心原理", §3.2:
// the residual needs p and q at the same token).  The slices of one target row form a team.
// k_fused runs one workgroup per ticket; workgroup i lands on XCD i mod 8 (the dispatcher deals
// workgroups round-robin over the XCDs) and the slices of team r are consecutive workgroups of
// XCD r mod 8.
//
// Per ticket:
//   1. load the slice(s) into registers (bounds-checked buffer loads); per wave, max and
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
  double py[kMaxGamma], qy[kMaxGamma], u0[kMaxGamma];
  int ytok[kMaxGamma];
  double gm[kChunk / kGroup];
  float dh[kMaxGamma], dm[kMaxGamma];
  float wsel[kGroup];
  double u[3];
  int flags, status, n_acc, pos, wkind, y, kpick, gpick, xpick;
};

struct Lds {
  float red[8 * kWaves];
  float f[8];
  int i[8];
  // one buffer per reduction of a ticket, so that consecutive reductions need no protecting
  // barrier between them
  float wp[2][kWaves][3];   // per-wave {ref, sum e, sum e t} of the target and draft rows
  float rres[kWaves];
  float cmb[4];
  int cst;
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
  uint32_t h = a * 0x9E3779B1u;
  h ^= ((b << 11) | (b >> 21)) * 0x85EBCA77u;
  h ^= ((c << 22) | (c >> 10)) * 0xC2B2AE3Du;
  return h ^ (h >> 15);
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
struct RowComb {
  double z, w;
  float M;
  bool ok;
};
__device__ __forceinline__ RowComb combine_lanes(float ref, float s, float w, bool in_range) {
  RowComb rc;
  const bool bad = in_range && (!(s == s) || !(s < INFINITY) || ref == INFINITY);
  const float M = wave_max_dpp(in_range ? ref : -INFINITY);
  double z = 0.0, ww = 0.0;
  if (in_range && s > 0.f) {
    const double d = (double)ref - (double)M;
    const double f = exp2_split(d);
    z = (double)s * f;
    ww = f * ((double)w + (double)s * d);
  }
  rc.z = wave_sum_dpp_d(z);
  rc.w = wave_sum_dpp_d(ww);
  rc.M = M;
  rc.ok = wave_all(!bad) && rc.z > 0.0 && M > -INFINITY;
  return rc;
}

// ---------------------------------------------------------------- finalize one request

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

// One request: combine its teams' records (normaliser, entropy in bits and max probability as
// in the SpecKV page's signals, beta = sum [p - q]_+), run the accept scan (guide page
// "5.1 投机解码核心原理" §3.1 / §3.2, stop at the first rejection §5.1) and the three-level
// sampler over the residual or p_{g+1} (§5.2), and write the outputs.  Scans over chunk,
// group and element masses are wave-wide fp64 prefix sums.
template <int DT, bool VEC, int MODE>
__device__ void finalize_request(const FusedArgs& a, LdsFin& L, int b) {
  FinScratch& F = L.fin;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c0 = L.cu[b], g = L.cu[b + 1] - c0;
  const int G1 = a.G + 1;
  const int n_s = a.n_s;
  const uint32_t tag = a.tag;
  const float nan = __int_as_float(0x7fc00000);
  const double cd = (double)a.c;
  const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
  // the draft tokens and their logits do not depend on any record: fetch them first
  float ly_p = 0.f, ly_q = 0.f;
  int ytok = -1;
  if (t < g) {
    ytok = a.tokens[c0 + t];
    if (ytok >= 0 && ytok < a.V) {
      ly_p = logit_at<DT>(row_ptr<DT>(a.tgt, a.tgt_ld, c0 + b + t), ytok);
      if (MODE == kFuSample) ly_q = logit_at<DT>(row_ptr<DT>(a.drf, a.drf_ld, c0 + t), ytok);
    }
  }

  // A. combine each team's records (one wave per team); the streaming kernel has finished
  for (int ti = wave; ti <= g; ti += kWaves) {
    const int r = c0 + b + ti;
    const bool pair = (MODE == kFuSample) && ti < g;
    const bool in = lane < n_s;
    float pr = -INFINITY, ps = 0.f, pw = 0.f, qr = -INFINITY, qs = 0.f, qw = 0.f, sm = 0.f;
    bool ok = true;
    if (in) {
      ok = load_rec(rrs, rec_off(n_s, r, lane, 0), tag, pr, ps, pw);
      if (pair) {
        ok = load_rec(rrs, rec_off(n_s, r, lane, 1), tag, qr, qs, qw) && ok;
        const uint64_t m = ld_coh(a.smass + (int64_t)r * n_s + lane);
        sm = lo_f(m);
        ok = ok && tag_of(m) == tag;
      }
    }
    const bool missing = !wave_all(ok);
    TeamL T;
    T.z[0] = T.z[1] = 1.0; T.w[0] = T.w[1] = 0.0; T.beta = 0.0; T.M[0] = T.M[1] = 0.f;
    T.amax = -1;
    T.flags = missing ? kTeamTimeout : 0;
    if (MODE == kFuGreedy) {
      const int qa = __float_as_int(ps);
      const bool bad = in && (qa == -2 || pr == INFINITY);
      const float M = wave_max_dpp(in ? pr : -INFINITY);
      const int idx = wave_min_i((in && pr == M && qa >= 0) ? qa : INT_MAX);
      T.M[0] = M;
      T.amax = idx == INT_MAX ? -1 : idx;
      if (!wave_all(!bad) || !(M > -INFINITY)) { T.flags |= kTeamBadP; T.amax = -1; }
    } else {
      const RowComb P = combine_lanes(pr, ps, pw, in);
      T.z[0] = P.z; T.w[0] = P.w; T.M[0] = P.M;
      if (!P.ok) T.flags |= kTeamBadP;
      if (pair) {
        const RowComb Q = combine_lanes(qr, qs, qw, in);
        T.z[1] = Q.z; T.w[1] = Q.w; T.M[1] = Q.M;
        if (!Q.ok) T.flags |= kTeamBadQ;
        // a slice whose team wait gave up marked its residual mass NaN
        if (!wave_all(!(in && !(sm == sm)))) T.flags |= kTeamTimeout;
        T.beta = wave_sum_dpp_d(in ? (double)sm : 0.0);
      }
    }
    if (lane == 0) F.team[ti] = T;
  }
  __syncthreads();

  // B. per position: statistics, p(y), q(y), the accept draw
  bool rej = false;
  int why = 0;
  if (t <= g) {
    const int r = c0 + b + t;
    const TeamL T = F.team[t];
    const bool okp = (T.flags & (kTeamBadP | kTeamTimeout)) == 0;
    const float hp = (float)(log2_split(T.z[0]) - T.w[0] / T.z[0]);
    if (a.st.target_entropy_bits) a.st.target_entropy_bits[r] = okp ? (MODE == kFuGreedy ? 0.f : hp) : nan;
    if (a.st.target_max_prob)
      a.st.target_max_prob[r] = okp ? (MODE == kFuGreedy ? 1.f : (float)(1.0 / T.z[0])) : nan;
    if (t < g) {
      const int drow = c0 + t;
      const int y = ytok;
      const bool yv = y >= 0 && y < a.V;
      float py = nan, qy = nan, ovl = nan, dh = nan, dm = nan;
      double pyd = 0.0, qyd = 1.0;
      if (MODE == kFuGreedy) {
        py = (okp && yv) ? (y == T.amax ? 1.f : 0.f) : nan;
        qy = yv ? 1.f : nan;
        ovl = okp ? (yv ? py : 0.f) : nan;
      } else {
        if (okp && yv) {
          pyd = exp2_split((double)ly_p * cd - (double)T.M[0]) / T.z[0];
          py = (float)pyd;
        }
        if (MODE == kFuTokenOnly) {
          qy = yv ? 1.f : nan;
          ovl = okp ? (yv ? py : 0.f) : nan;
          dh = yv ? 0.f : nan;
          dm = yv ? 1.f : nan;
        } else {
          const bool okq = (T.flags & (kTeamBadQ | kTeamTimeout)) == 0;
          if (okq && yv) {
            qyd = exp2_split((double)ly_q * cd - (double)T.M[1]) / T.z[1];
            qy = (float)qyd;
          }
          if (okp && okq) ovl = (float)(1.0 - T.beta);
          dh = okq ? (float)(log2_split(T.z[1]) - T.w[1] / T.z[1]) : nan;
          dm = okq ? (float)(1.0 / T.z[1]) : nan;
        }
      }
      if (a.st.p_y) a.st.p_y[drow] = py;
      if (a.st.q_y) a.st.q_y[drow] = qy;
      if (a.st.one_minus_tv) a.st.one_minus_tv[drow] = ovl;
      if (a.st.draft_entropy_bits) a.st.draft_entropy_bits[drow] = dh;
      if (a.st.draft_max_prob) a.st.draft_max_prob[drow] = dm;
      F.dh[t] = dh;
      F.dm[t] = dm;
      F.ytok[t] = y;
      F.py[t] = pyd;
      F.qy[t] = qyd;
      // the accept test of position t (evaluated for every position; the scan takes the first)
      if (!yv) { rej = true; why = kStBadToken; }
      else if (MODE == kFuGreedy) rej = y != T.amax;
      else if (!(qyd > 0.0)) { rej = true; why = kStZeroQ; }
      else {
        uint64_t w[4];
        philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(t + 1), 0, 0, w);
        rej = !(u53(w[0]) < fmin(1.0, pyd / qyd));
      }
    }
  }
  // C. request flags and the first rejection (wave 0 covers positions 0..63)
  if (wave == 0) {
    // flags of every team (positions 0..g; wave 0 holds 0..63, lane 0 adds position 64)
    int fl = lane <= g ? F.team[lane].flags : 0;
    if (lane == 0 && g >= 64) fl |= F.team[64].flags;
    fl = wave_or(fl);
    const unsigned long long rm = __ballot(rej);
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
      uint64_t w[4];
      philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(F.pos + 1), 0, 0, w);
      F.u[0] = u53(w[1]);
      F.u[1] = u53(w[2]);
      F.u[2] = u53(w[3]);
      F.status = status;
      F.kpick = -1;
      if (a.out_req_stats) {
        float rq[4] = {nan, nan, nan, nan};
        if (g > 0 && MODE != kFuGreedy) {
          double hs = 0.0, cs = 0.0;
          float hmax = -INFINITY, cmin = INFINITY;
          bool anynan = false;
          for (int i = 0; i < g; ++i) {
            const float h = F.dh[i], cm = F.dm[i];
            if (!(h == h) || !(cm == cm)) anynan = true;
            hs += h; cs += cm;
            hmax = fmaxf(hmax, h); cmin = fminf(cmin, cm);
          }
          if (!anynan) { rq[0] = (float)(hs / g); rq[1] = (float)(cs / g); rq[2] = hmax; rq[3] = cmin; }
        }
        for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = rq[q];
      }
    }
  }
  __syncthreads();

  int x = -1;
  if (F.status & (kStTimeout | kStNonfinite)) {
    x = -1;
  } else if (MODE == kFuGreedy) {
    x = F.team[F.pos].amax;
  } else {
    const int r = c0 + b + F.pos;
    const TeamL T = F.team[F.pos];
    // D. level 1 over the chunk masses (p's masses again if the residual turned out empty)
    if (wave == 0) {
      int wkind = F.wkind;
      int pick = -1;
      for (int pass = 0; pass < 2; ++pass) {
        double m = 0.0;
        if (lane < n_s) {
          if (wkind == 1) {
            m = (double)lo_f(ld_coh(a.smass + (int64_t)r * n_s + lane));
          } else {
            float ref, sv, wv;
            load_rec(rrs, rec_off(n_s, r, lane, 0), tag, ref, sv, wv);
            m = sv > 0.f ? (double)sv * exp2_split((double)ref - (double)T.M[0]) / T.z[0] : 0.0;
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
    const int k = F.kpick;
    if (k >= 0) {
      // E. levels 2 and 3 inside chunk k.  Weights are relative within the chunk: e_p (p
      // only) or max(e_p r - e_q, 0) with r = alpha_p / alpha_q.
      const int wkind = F.wkind;
      float refp, sp_, wp_, refq = 0.f, rr = 0.f;
      load_rec(rrs, rec_off(n_s, r, k, 0), tag, refp, sp_, wp_);
      if (wkind == 1) {
        float sq_, wq_;
        load_rec(rrs, rec_off(n_s, r, k, 1), tag, refq, sq_, wq_);
        const double alp = exp2_split((double)refp - (double)T.M[0]) / T.z[0];
        const double alq = exp2_split((double)refq - (double)T.M[1]) / T.z[1];
        rr = (float)(alp / alq);
      }
      const int grp = t >> 2, quarter = t & 3;
      const int x0 = k * kChunk + grp * kGroup + quarter * 16;
      float wv[16];
      load_run16<DT, VEC>(row_ptr<DT>(a.tgt, a.tgt_ld, r), a.V, x0, wv);
      if (wkind == 1) {
        float vq[16];
        load_run16<DT, VEC>(row_ptr<DT>(a.drf, a.drf_ld, c0 + F.pos), a.V, x0, vq);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float ep = __builtin_amdgcn_exp2f(fmaf(wv[e], a.c, -refp));
          const float eq = __builtin_amdgcn_exp2f(fmaf(vq[e], a.c, -refq));
          wv[e] = fmaxf(fmaf(ep, rr, -eq), 0.f);
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
      __syncthreads();
      const int n_in = min(kChunk, a.V - k * kChunk);
      const int n_groups = (n_in + kGroup - 1) / kGroup;
      if (wave == 0) {
        double tot;
        const int gp = wave_pick(lane < n_groups ? F.gm[lane] : 0.0, n_groups, F.u[1], tot);
        if (lane == 0) F.gpick = gp;
      }
      __syncthreads();
      if (grp == F.gpick) {
#pragma unroll
        for (int e = 0; e < 16; ++e) F.wsel[quarter * 16 + e] = wv[e];
      }
      __syncthreads();
      if (wave == 0) {
        const int gsel = F.gpick;
        int pick = -1;
        if (gsel >= 0) {
          const int lo = k * kChunk + gsel * kGroup;
          const int n = min(kGroup, a.V - lo);
          double tot;
          pick = wave_pick(lane < n ? (double)F.wsel[lane] : 0.0, n, F.u[2], tot);
          if (pick >= 0) pick += lo;
        }
        if (lane == 0) F.xpick = pick;
      }
      __syncthreads();
      x = F.xpick;
    }
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
}

// ---------------------------------------------------------------- streaming phases

// One ticket; every field is uniform over the workgroup.
struct Ticket {
  int r, s, b, c0, g, i;
  bool pair;
};

// The lane that publishes a workgroup's records: lane 0 of the last wave.  Wave 0 polls the
// team records; keeping every store out of wave 0 means that, in wave 0, only the ticket loads
// issued after a poll stand between the poll and its use (vector memory counters retire in
// issue order).
constexpr int kStorer = kThreads - 64;
   // polls served by the XCD's L2 before device-scope polls

// Fold per-wave partials {ref_w, s_w, w_w} of one row's slice (ref_w = -inf for a wave that
// holds no finite logit) into one record relative to ref = max_w ref_w:
// s = sum_w s_w 2^(ref_w - ref), w = sum_w 2^(ref_w - ref) (w_w + s_w (ref_w - ref)).
__device__ __forceinline__ void fold_waves(const float (*pw)[3], float& ref, float& s, float& w) {
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) M = fmaxf(M, pw[k][0]);
  ref = 0.f; s = 0.f; w = 0.f;
  if (!(M > -INFINITY)) return;
  ref = M;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (!(pw[k][0] > -INFINITY)) continue;
    const float d = pw[k][0] - M;
    const float f = __builtin_amdgcn_exp2f(d);
    s = fmaf(pw[k][1], f, s);
    w = fmaf(f, fmaf(pw[k][1], d, pw[k][2]), w);
  }
}

// Phase 1 of a ticket: per-wave maxima, e = exp2(l c - ref_w) in place, sums, one record per
// row.  Returns each wave's references (0 for a wave with no finite logit).
template <int DT, int MODE>
__device__ __forceinline__ void phase1(const FusedArgs& a, Lds& L, const Ticket& T, float (&vp)[kPerThread],
                                       float (&vq)[kPerThread], float& refp, float& refq) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t tag = a.tag;
  const int base = T.s * kChunk;
  const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
  if (MODE == kFuGreedy) {
    float mv[1];
    mv[0] = vp[0];
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) mv[0] = fmaxf(mv[0], vp[j]);
    int badv = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) badv |= __builtin_amdgcn_class(vp[j], 0x203) ? 1 : 0;
    block_max_f<1>(mv, L.red);
    int idx = INT_MAX;
    if (mv[0] > -INFINITY) {
#pragma unroll
      for (int j = kPerThread - 1; j >= 0; --j)
        if (vp[j] == mv[0]) idx = slice_index<DT>(base, t, j);
    }
    __syncthreads();
    idx = block_min_i(idx, L.i);
    badv = block_or(badv, L.i);
    if (t == kStorer)
      store_rec(rrs, rec_off(a.n_s, T.r, T.s, 0), mv[0], __int_as_float(badv ? -2 : (idx == INT_MAX ? -1 : idx)),
                0.f, tag);
    return;
  }
  float mp = vp[0], mq = T.pair ? vq[0] : -INFINITY;
#pragma unroll
  for (int j = 1; j < kPerThread; ++j) mp = fmaxf(mp, vp[j]);
  if (T.pair) {
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) mq = fmaxf(mq, vq[j]);
  }
  mp = wave_max_dpp(mp);
  if (T.pair) mq = wave_max_dpp(mq);
  refp = mp > -INFINITY ? mp * a.c : 0.f;
  refq = mq > -INFINITY ? mq * a.c : 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.want_t_ent) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const float tt = fmaf(vp[j], a.c, -refp);
      const float e = __builtin_amdgcn_exp2f(tt);
      acc[0] += e;
      acc[1] = fmaf(e, fmaxf(tt, -200.f), acc[1]);
      vp[j] = e;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const float e = __builtin_amdgcn_exp2f(fmaf(vp[j], a.c, -refp));
      acc[0] += e;
      vp[j] = e;
    }
  }
  if (T.pair) {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const float tt = fmaf(vq[j], a.c, -refq);
      const float e = __builtin_amdgcn_exp2f(tt);
      acc[2] += e;
      acc[3] = fmaf(e, fmaxf(tt, -200.f), acc[3]);
      vq[j] = e;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = wave_sum_dpp(acc[k]);
  if (lane == 0) {
    L.wp[0][wave][0] = mp > -INFINITY ? refp : -INFINITY;
    L.wp[0][wave][1] = acc[0];
    L.wp[0][wave][2] = acc[1];
    L.wp[1][wave][0] = mq > -INFINITY ? refq : -INFINITY;
    L.wp[1][wave][1] = acc[2];
    L.wp[1][wave][2] = acc[3];
  }
  __syncthreads();
  if (t == kStorer) {
    float ref, sm, wm;
    fold_waves(L.wp[0], ref, sm, wm);
    store_rec(rrs, rec_off(a.n_s, T.r, T.s, 0), ref, sm, wm, tag);
    if (T.pair) {
      fold_waves(L.wp[1], ref, sm, wm);
      store_rec(rrs, rec_off(a.n_s, T.r, T.s, 1), ref, sm, wm, tag);
      // the arrival flag goes out once both records are visible
      wait_vmem();
      __hip_atomic_store(a.arrive + (int64_t)T.r * a.n_s + T.s, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!(mp > -INFINITY)) refp = -INFINITY;
  if (!(mq > -INFINITY)) refq = -INFINITY;
}

// Phase 2 of a paired ticket: wave 0 polls the team's records (one slice per lane; lanes past
// the last slice read it again) and forms the normalisers; then every wave turns its kept
// e-values into the slice's residual mass sum [p - q]_+ (guide page "5.1 投机解码核心原理",
// §3.2 / §4.1: beta = sum [p - q]_+).  Returns the tagged mass word; the caller stores it.
__device__ __forceinline__ uint64_t phase2(const FusedArgs& a, Lds& L, int r, float refp, float refq,
                                           const float (&ep)[kPerThread], const float (&eq)[kPerThread]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t tag = a.tag;
  if (wave == 0) {
    const int n_s = a.n_s;
    const bool in = lane < n_s;
    const int sl = min(lane, n_s - 1);
    const __amdgpu_buffer_rsrc_t rrs = rec_rsrc(a);
    // wait until the team has had time to publish, then poll its arrival flags (one word per
    // slice) with growing pauses, and read the records once they are all in
    const long long t0 = wall_clock64();
    while (wall_clock64() - t0 < a.poll_delay) __builtin_amdgcn_s_sleep(8);
    const uint32_t* fl = a.arrive + (int64_t)r * n_s;
    bool timed_out = false;
    unsigned spins = 0;
    for (int pause = a.poll_pause > 0 ? a.poll_pause : 4;; pause = a.poll_pause > 0 ? pause : min(2 * pause, 64)) {
      const uint32_t f = __hip_atomic_load(fl + sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (wave_all(f == tag)) break;
      if (++spins > a.spin_limit) { timed_out = true; break; }
      for (int k = 0; k < pause; ++k) __builtin_amdgcn_s_sleep(2);
    }
    Rec P = load_rec_raw(rrs, rec_off(n_s, r, sl, 0)), Q = load_rec_raw(rrs, rec_off(n_s, r, sl, 1));
    if (!timed_out && !wave_all(rec_ok(P, tag) && rec_ok(Q, tag))) {
      for (;; ++spins) {
        if (spins >= a.spin_limit) { timed_out = true; break; }
        __builtin_amdgcn_s_sleep(4);
        P = load_rec_raw(rrs, rec_off(n_s, r, sl, 0));
        Q = load_rec_raw(rrs, rec_off(n_s, r, sl, 1));
        if (wave_all(rec_ok(P, tag) && rec_ok(Q, tag))) break;
      }
    }
    const float pr = __uint_as_float(P.x), ps = __uint_as_float(P.y);
    const float qr = __uint_as_float(Q.x), qs = __uint_as_float(Q.y);
    const bool bad = in && (!(ps == ps) || !(ps < INFINITY) || pr == INFINITY || !(qs == qs) ||
                            !(qs < INFINITY) || qr == INFINITY);
    const float Mp = wave_max_dpp(in ? pr : -INFINITY), Mq = wave_max_dpp(in ? qr : -INFINITY);
    // Z = sum_s s_s 2^(ref_s - M): the difference is exact near the maximum, the product exact
    // in fp64, the sum fp64
    const double zp = wave_sum_dpp_d((in && ps > 0.f) ? (double)ps * (double)__builtin_amdgcn_exp2f(pr - Mp) : 0.0);
    const double zq = wave_sum_dpp_d((in && qs > 0.f) ? (double)qs * (double)__builtin_amdgcn_exp2f(qr - Mq) : 0.0);
    const bool all_good = wave_all(!bad);
    if (lane == 0) {
      const bool ok = !timed_out && all_good && zp > 0.0 && zq > 0.0 && Mp > -INFINITY && Mq > -INFINITY;
      L.cst = timed_out ? 2 : (ok ? 0 : 1);
      L.cmb[0] = Mp;
      L.cmb[1] = Mq;
      L.cmb[2] = (float)(1.0 / zp);
      L.cmb[3] = (float)(1.0 / zq);
    }
  }
  __syncthreads();
  const int st = L.cst;
  float wmass = 0.f;
  if (st == 0) {
    // this wave's alpha = 2^(ref_w - M) / Z of each row; p = e_p alpha_p, q = e_q alpha_q
    const float ap = refp > -INFINITY ? __builtin_amdgcn_exp2f(refp - L.cmb[0]) * L.cmb[2] : 0.f;
    const float aq = refq > -INFINITY ? __builtin_amdgcn_exp2f(refq - L.cmb[1]) * L.cmb[3] : 0.f;
    float sres = 0.f;
    if (aq > 0.f) {
      // sum_x [p - q]_+ = alpha_q sum_x max(e_p r - e_q, 0), r = alpha_p / alpha_q
      const float rr = ap / aq;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) sres += fmaxf(fmaf(ep[j], rr, -eq[j]), 0.f);
      wmass = wave_sum_dpp(sres) * aq;
    } else {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) sres += ep[j];
      wmass = wave_sum_dpp(sres) * ap;
    }
  }
  if (lane == 0) L.rres[wave] = wmass;
  __syncthreads();
  float mass = 0.f;
  if (t == kStorer) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mass += L.rres[w];
    // NaN marks a slice whose wait gave up; 0 when a row is non-finite
    mass = st == 2 ? __int_as_float(0x7fc00000) : (st == 1 ? 0.f : mass);
  }
  return tagged(mass, tag);
}

// ---------------------------------------------------------------- the kernel

// Stage the draft offsets in LDS and check them as one exclusive prefix (every request is
// refused when any offset is out of order).
__device__ __forceinline__ bool stage_cu(const FusedArgs& a, int* cu, int* red) {
  const int t = threadIdx.x;
  for (int k = t; k <= a.B; k += kThreads) cu[k] = a.cu[k];
  __syncthreads();
  int bad = 0;
  for (int k = t; k < a.B; k += kThreads) {
    const int g = cu[k + 1] - cu[k];
    if (g < 0 || g > a.G) bad = 1;
  }
  if (t == 0 && (cu[0] != 0 || cu[a.B] != a.n_draft_rows)) bad = 1;
  return block_or(bad, red) != 0;
}

// One workgroup per ticket.  Workgroup i runs on XCD i mod 8 (the dispatcher deals workgroups
// round-robin over the XCDs), and the slices of team r go to consecutive workgroups of XCD
// r mod 8, so a team's records meet in that XCD's L2.  A member waits only for members
// dispatched just before or after it on the same XCD; every wait is bounded.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_fused(FusedArgs a) {
  __shared__ Lds L;
  const int t = threadIdx.x;
  const int n_s = a.n_s;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tl = j / n_s;
  Ticket T;
  T.s = j - tl * n_s;
  T.r = tl * 8 + xcd;
  if (T.r >= a.n_teams) return;
  T.pair = false;
  T.b = 0; T.c0 = 0; T.g = 0; T.i = 0;
  int drow = -1;
  constexpr int kEsz = DT == kDtBF16 ? 2 : 4;
  RawSlice<DT> rp, rq;
  if (VEC) load_raw_buf<DT>(row_rsrc(row_ptr<DT>(a.tgt, a.tgt_ld, T.r), a.V * kEsz), T.s * kChunk, rp);
  else load_raw<DT, false>(row_ptr<DT>(a.tgt, a.tgt_ld, T.r), a.V, T.s * kChunk, rp);
  if (MODE == kFuSample) {
    // request of target row r: the largest b < B with cu[b] + b <= r (cu[b] + b grows
    // strictly with b in a valid offset array), by a binary search through the scalar cache,
    // which does not queue behind the row loads.  An invalid array (the finalize kernel
    // reports it) can only give a draft row that is range-checked here.
    int lo = 0, hi = a.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sload_i32(a.cu + mid) + mid <= T.r) lo = mid;
      else hi = mid;
    }
    const int b = lo;
    const int c0 = sload_i32(a.cu + b), c1 = sload_i32(a.cu + b + 1);
    T.b = b; T.c0 = c0; T.g = c1 - c0; T.i = T.r - c0 - b;
    drow = T.r - b;
    T.pair = T.i >= 0 && T.i < T.g && drow >= 0 && drow < a.n_draft_rows;
    if (VEC)
      load_raw_buf<DT>(row_rsrc(T.pair ? row_ptr<DT>(a.drf, a.drf_ld, drow) : a.tgt, T.pair ? a.V * kEsz : 0),
                       T.s * kChunk, rq);
    else if (T.pair)
      load_raw<DT, false>(row_ptr<DT>(a.drf, a.drf_ld, drow), a.V, T.s * kChunk, rq);
  }
  float vp[kPerThread], vq[kPerThread];
  float refp = 0.f, refq = 0.f;
  unpack_raw<DT>(rp, vp);
  if (T.pair) unpack_raw<DT>(rq, vq);
  if (VEC && (a.V % kChunk) != 0 && T.s == n_s - 1) {
    mask_tail<DT>(a.V, T.s * kChunk, vp);
    if (T.pair) mask_tail<DT>(a.V, T.s * kChunk, vq);
  }
  phase1<DT, MODE>(a, L, T, vp, vq, refp, refq);
  if (MODE == kFuSample && T.pair) {
    const uint64_t mass_word = phase2(a, L, T.r, refp, refq, vp, vq);
    if (t == kStorer) st_coh(a.smass + (int64_t)T.r * n_s + T.s, mass_word);
  }
}

// One workgroup per request, after the streaming kernel: every record is in place.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_fused_finalize(FusedArgs a) {
  __shared__ LdsFin L;
  const int t = threadIdx.x, b = blockIdx.x;
  if (stage_cu(a, L.cu, L.i)) {
    if (t <= a.G) a.out_tokens[(int64_t)b * (a.G + 1) + t] = -1;
    if (t == 0) {
      a.out_num_accepted[b] = 0;
      a.out_status[b] = kStBadGamma;
      if (a.out_req_stats)
        for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = __int_as_float(0x7fc00000);
    }
    return;
  }
  finalize_request<DT, VEC, MODE>(a, L, b);
}

// ---------------------------------------------------------------- launch

template <int DT, bool VEC, int MODE>
static hipError_t launch_fused_t(FusedArgs a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int teams8 = (a.n_teams + 7) / 8;
  const long long grid = 8ll * teams8 * a.n_s;
  if (grid < 1 || grid > 0x7fffffffll) return hipErrorInvalidConfiguration;
  a.n_fin = 0;
  if (getenv("SPEC_VERIFY_DEBUG"))
    fprintf(stderr, "[specverify] fused grid %lld tickets %d slices %d mode %d\n", grid, a.n_tickets, a.n_s, a.mode);
  // optional events bracket the streaming kernel alone (benchmark timing)
  if (ev0 && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_fused<DT, VEC, MODE>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
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
