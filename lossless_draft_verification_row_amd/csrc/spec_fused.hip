// spec_fused.hip -- a whole verification round in one persistent, cooperatively launched kernel.
//
// Work unit ("ticket"): one 4096-logit slice of one target row, together with the same slice
// of its draft row when that position pairs the two (guide page "5.1 投机解码核心原理", §3.2:
// the residual needs p and q at the same token).  The slices of one target row form a team.
// Tickets are numbered team-major and dealt round-robin to the resident workgroups.
//
// Per ticket every needed logit is read from HBM exactly once:
//   1. load the slice(s) into registers; slice max; e = exp2(l c - ref), ref = max * c;
//      publish the slice record (ref, sum e, sum e t) of each row;
//   2. paired positions: wait until every slice record of the team is present, combine them in
//      a fixed order (fp64) and form the slice's residual mass sum [p - q]_+ from the
//      registers, p = e_p alpha_p, q = e_q alpha_q (§3.2, §4.1: beta = sum [p - q]_+);
//      publish it.
// A workgroup runs phase 1 of its next ticket before phase 2 of the current one, so the team
// wait overlaps useful work, and the loads of the ticket after that are already in flight.
// A few finalizer workgroups take the requests round-robin as they complete: wait for every
// record of the request, combine the team statistics (normaliser, entropy in bits and max
// probability as in the SpecKV page's signals, beta), run the accept scan (§3.1 / §3.2, stop
// at the first rejection §5.1) and the three-level sampler over the residual or p_{g+1}
// (§5.2, one re-read chunk), and write the outputs.
//
// Synchronisation without read-modify-write atomics: every record carries the call's tag (a
// per-call sequence number, never 0) in each of its 64-bit words and travels through
// coherent agent-scope loads and stores; a reader polls until every word it needs carries the
// current tag.  (Same-address atomics serialise across the XCDs, and acquire / release fences
// write back and invalidate the whole L2, so neither is used.)
// Deadlock freedom: the launch is cooperative, so every workgroup is resident.  A workgroup
// publishes ticket k only after the team wait of ticket k - 2, whose team is lower; so the
// lowest team still waiting has every member published or about to be, and completes.  The
// finalizers wait only on streaming workgroups, never the reverse.  Every wait is bounded; one that expires
// reports SPEC_STATUS_TIMEOUT for its request.
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
  double mass[kMaxSlicesFused];
  double gm[kChunk / kGroup];
  float dh[kMaxGamma], dm[kMaxGamma];
  float wsel[kGroup];
  double u[3];
  int flags, status, n_acc, pos, wkind, y, kpick, gpick, xpick, pass;
};

struct Lds {
  uint16_t team_req[kMaxTeamsFused];
  int cu[kMaxReqFused + 1];
  float red[8 * kWaves];
  float f[8];
  int i[8];
  FinScratch fin;
};

// ---------------------------------------------------------------- tagged records

__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return (uint32_t)(w >> 32); }

// slice record of one row: 3 words {ref|tag}, {s|tag}, {w|tag}
__device__ __forceinline__ uint64_t* rec_ptr(uint64_t* part, int n_s, int r, int s, int row) {
  return part + (((int64_t)r * n_s + s) * 2 + row) * 3;
}
__device__ __forceinline__ void store_rec(uint64_t* p, float ref, float s, float w, uint32_t tag) {
  st_coh(p, tagged(ref, tag));
  st_coh(p + 1, tagged(s, tag));
  st_coh(p + 2, tagged(w, tag));
}
__device__ __forceinline__ bool load_rec(const uint64_t* p, uint32_t tag, float& ref, float& s, float& w) {
  const uint64_t a = ld_coh(p), b = ld_coh(p + 1), c = ld_coh(p + 2);
  ref = lo_f(a); s = lo_f(b); w = lo_f(c);
  return tag_of(a) == tag && tag_of(b) == tag && tag_of(c) == tag;
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

// ---------------------------------------------------------------- combining slice records

// Fixed-order fp64 combine of one row's slice records held one per lane (lanes >= n_s hold
// ref = -inf, s = 0).  Every lane gets the result.
struct RowComb {
  double z, w;
  float M;
  bool ok;
};

__device__ __forceinline__ RowComb combine_lanes(float ref, float s, float w, bool in_range) {
  RowComb rc;
  const bool bad = in_range && (!(s == s) || !(s < INFINITY) || ref == INFINITY);
  const float M = wave_max(in_range ? ref : -INFINITY);
  double z = 0.0, ww = 0.0;
  if (in_range && s > 0.f) {
    const double d = (double)ref - (double)M;
    const double f = exp2_split(d);
    z = (double)s * f;
    ww = f * ((double)w + (double)s * d);
  }
  rc.z = wave_sum_d(z);
  rc.w = wave_sum_d(ww);
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

template <int DT, bool VEC, int MODE>
__device__ void finalize_request(const FusedArgs& a, Lds& L, int b) {
  FinScratch& F = L.fin;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c0 = L.cu[b], g = L.cu[b + 1] - c0;
  const int G1 = a.G + 1;
  const int n_s = a.n_s;
  const uint32_t tag = a.tag;
  const float nan = __int_as_float(0x7fc00000);
  const double cd = (double)a.c;
  if (t == 0) { F.flags = 0; F.status = 0; }
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

  // A. wait for the request's records and combine each team (one wave per team)
  for (int ti = wave; ti <= g; ti += kWaves) {
    const int r = c0 + b + ti;
    const bool pair = (MODE == kFuSample) && ti < g;
    const bool in = lane < n_s;
    float pr = -INFINITY, ps = 0.f, pw = 0.f, qr = -INFINITY, qs = 0.f, qw = 0.f, sm = 0.f;
    bool timed_out = false;
    for (unsigned spins = 0;; ++spins) {
      bool ok = true;
      if (in) {
        ok = load_rec(rec_ptr(a.part, n_s, r, lane, 0), tag, pr, ps, pw);
        if (pair) {
          ok = load_rec(rec_ptr(a.part, n_s, r, lane, 1), tag, qr, qs, qw) && ok;
          const uint64_t m = ld_coh(a.smass + (int64_t)r * n_s + lane);
          sm = lo_f(m);
          ok = ok && tag_of(m) == tag;
        }
      }
      if (wave_all(ok)) break;
      if (spins >= a.spin_limit) { timed_out = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    TeamL T;
    T.z[0] = T.z[1] = 1.0; T.w[0] = T.w[1] = 0.0; T.beta = 0.0; T.M[0] = T.M[1] = 0.f;
    T.amax = -1;
    T.flags = timed_out ? kTeamTimeout : 0;
    if (MODE == kFuGreedy) {
      const int qa = __float_as_int(ps);
      const bool bad = in && (qa == -2 || pr == INFINITY);
      const float M = wave_max(in ? pr : -INFINITY);
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
        // a slice that gave up its own wait marked its residual mass NaN
        if (!wave_all(!(in && !(sm == sm)))) T.flags |= kTeamTimeout;
        T.beta = wave_sum_d(in ? (double)sm : 0.0);
      }
    }
    if (lane == 0) F.team[ti] = T;
  }
  __syncthreads();

  // B. per position: statistics, p(y), q(y), the accept draw
  if (t <= g) {
    const int r = c0 + b + t;
    const TeamL T = F.team[t];
    if (T.flags) atomicOr(&F.flags, T.flags);
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
      uint64_t w[4];
      philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(t + 1), 0, 0, w);
      F.u0[t] = u53(w[0]);
    }
  }
  __syncthreads();

  // C. request statistics, accept scan, choice of the sampled row (one thread)
  if (t == 0) {
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
    int status = 0, j = -1;
    if (F.flags & kTeamTimeout) status = kStTimeout;
    else if (F.flags) status = kStNonfinite;
    else {
      for (int i = 0; i < g; ++i) {
        const int y = F.ytok[i];
        if (y < 0 || y >= a.V) { status |= kStBadToken; j = i; break; }
        if (MODE == kFuGreedy) {
          if (y == F.team[i].amax) continue;
          j = i;
          break;
        }
        const double qy = F.qy[i];
        if (!(qy > 0.0)) { status |= kStZeroQ; j = i; break; }
        const double acc = fmin(1.0, F.py[i] / qy);
        if (!(F.u0[i] < acc)) { j = i; break; }
      }
    }
    F.n_acc = j < 0 ? g : j;
    F.pos = j < 0 ? g : j;
    F.y = j >= 0 ? F.ytok[j] : -1;
    // wkind: 0 = p of the row, 1 = [p - q]_+, 2 = p without token y
    F.wkind = (j < 0) ? 0 : (MODE == kFuSample ? 1 : 2);
    uint64_t w[4];
    philox4x64_10(a.seed, a.step, (uint64_t)b, (uint64_t)(F.pos + 1), 0, 0, w);
    F.u[0] = u53(w[1]);
    F.u[1] = u53(w[2]);
    F.u[2] = u53(w[3]);
    F.status = status;
    F.kpick = -1;
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
    // D. level 1 over chunk masses (a second pass only if the residual turned out empty)
    for (int pass = 0; pass < 2; ++pass) {
      const int wkind = F.wkind;
      if (t < 64) {
        for (int k = lane; k < n_s; k += 64) {
          double m;
          if (wkind == 1) {
            m = (double)lo_f(ld_coh(a.smass + (int64_t)r * n_s + k));
          } else {
            float ref, s, w;
            load_rec(rec_ptr(a.part, n_s, r, k, 0), tag, ref, s, w);
            m = s > 0.f ? (double)s * exp2_split((double)ref - (double)T.M[0]) / T.z[0] : 0.0;
            if (wkind == 2) {
              const int y = F.y;
              if (y >= 0 && y < a.V && y / kChunk == k) m = fmax(m - F.py[F.pos], 0.0);
            }
          }
          F.mass[k] = m;
        }
      }
      __syncthreads();
      if (t == 0) {
        double tot = 0.0;
        for (int k = 0; k < n_s; ++k) tot += F.mass[k];
        int pick = -1;
        if (tot > 0.0) {
          const double target = F.u[0] * tot;
          double cum = 0.0;
          int last = -1;
          for (int k = 0; k < n_s; ++k) {
            cum += F.mass[k];
            if (F.mass[k] > 0.0) last = k;
            if (cum > target) { pick = k; break; }
          }
          if (pick < 0) pick = last;
        }
        F.kpick = pick;
        F.pass = 2;
        if (pick < 0 && wkind != 0) { F.status |= kStResidualEmpty; F.wkind = 0; F.pass = 1; }
      }
      __syncthreads();
      if (F.pass == 2) break;
    }
    const int k = F.kpick;
    if (k >= 0) {
      // E. levels 2 and 3 inside chunk k.  Weights are relative within the chunk: e_p (p
      // only) or max(e_p * r - e_q, 0) with r = alpha_p / alpha_q, exactly as streamed.
      const int wkind = F.wkind;
      float refp, sp_, wp_, refq = 0.f, rr = 0.f;
      load_rec(rec_ptr(a.part, n_s, r, k, 0), tag, refp, sp_, wp_);
      if (wkind == 1) {
        float sq_, wq_;
        load_rec(rec_ptr(a.part, n_s, r, k, 1), tag, refq, sq_, wq_);
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
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      if (quarter == 0) F.gm[grp] = part;
      __syncthreads();
      if (t == 0) {
        const int n_in = min(kChunk, a.V - k * kChunk);
        const int n_groups = (n_in + kGroup - 1) / kGroup;
        double tot = 0.0;
        for (int q = 0; q < n_groups; ++q) tot += F.gm[q];
        const double target = F.u[1] * tot;
        double cum = 0.0;
        int pick = -1, last = -1;
        for (int q = 0; q < n_groups; ++q) {
          cum += F.gm[q];
          if (F.gm[q] > 0.0) last = q;
          if (cum > target) { pick = q; break; }
        }
        F.gpick = pick < 0 ? last : pick;
      }
      __syncthreads();
      if (grp == F.gpick) {
#pragma unroll
        for (int e = 0; e < 16; ++e) F.wsel[quarter * 16 + e] = wv[e];
      }
      __syncthreads();
      if (t == 0) {
        const int gsel = F.gpick;
        int pick = -1;
        if (gsel >= 0) {
          const int lo = k * kChunk + gsel * kGroup;
          const int n = min(kGroup, a.V - lo);
          const double target = F.u[2] * F.gm[gsel];
          double cum = 0.0;
          int last = -1;
          for (int e = 0; e < n; ++e) {
            cum += (double)F.wsel[e];
            if (F.wsel[e] > 0.f) last = e;
            if (cum > target) { pick = e; break; }
          }
          if (pick < 0) pick = last;
          if (pick >= 0) pick += lo;
        }
        F.xpick = pick;
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
  __syncthreads();
}

// ---------------------------------------------------------------- streaming phases

// Per-workgroup decode of a ticket.
struct Ticket {
  int r, s, b, c0, g, i;
  bool pair;
};

// Phase 1 of a ticket: slice maxima, e = exp2(l c - ref) in place, sums, records published.
template <int DT, int MODE>
__device__ __forceinline__ void phase1(const FusedArgs& a, Lds& L, const Ticket& T, float (&vp)[kPerThread],
                                       float (&vq)[kPerThread], float& refp, float& refq) {
  const int t = threadIdx.x;
  const uint32_t tag = a.tag;
  const int base = T.s * kChunk;
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
    if (t == 0)
      store_rec(rec_ptr(a.part, a.n_s, T.r, T.s, 0), mv[0],
                __int_as_float(badv ? -2 : (idx == INT_MAX ? -1 : idx)), 0.f, tag);
    return;
  }
  float mv[2];
  mv[0] = vp[0];
  mv[1] = T.pair ? vq[0] : -INFINITY;
#pragma unroll
  for (int j = 1; j < kPerThread; ++j) mv[0] = fmaxf(mv[0], vp[j]);
  if (T.pair) {
#pragma unroll
    for (int j = 1; j < kPerThread; ++j) mv[1] = fmaxf(mv[1], vq[j]);
  }
  block_max_f<2>(mv, L.red);
  refp = mv[0] > -INFINITY ? mv[0] * a.c : 0.f;
  refq = mv[1] > -INFINITY ? mv[1] * a.c : 0.f;
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
  __syncthreads();
  block_sum_f<4>(acc, L.red);
  if (t == 0) {
    store_rec(rec_ptr(a.part, a.n_s, T.r, T.s, 0), refp, acc[0], acc[1], tag);
    if (T.pair) store_rec(rec_ptr(a.part, a.n_s, T.r, T.s, 1), refq, acc[2], acc[3], tag);
  }
  __syncthreads();
}

// Phase 2 of a paired ticket: wait for the team's records, normalisers, residual mass of the
// slice from the e-values kept in registers.
__device__ __forceinline__ void phase2(const FusedArgs& a, Lds& L, int r, int s, float refp, float refq,
                                       const float (&ep)[kPerThread], const float (&eq)[kPerThread]) {
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t tag = a.tag;
  const int n_s = a.n_s;
  if (t < 64) {
    const bool in = lane < n_s;
    float pr = -INFINITY, ps = 0.f, pw = 0.f, qr = -INFINITY, qs = 0.f, qw = 0.f;
    bool timed_out = false;
    for (unsigned spins = 0;; ++spins) {
      bool ok = true;
      if (in) {
        ok = load_rec(rec_ptr(a.part, n_s, r, lane, 0), tag, pr, ps, pw);
        ok = load_rec(rec_ptr(a.part, n_s, r, lane, 1), tag, qr, qs, qw) && ok;
      }
      if (wave_all(ok)) break;
      if (spins >= a.spin_limit) { timed_out = true; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    const RowComb P = combine_lanes(pr, ps, pw, in);
    const RowComb Q = combine_lanes(qr, qs, qw, in);
    if (lane == 0) {
      const double alp = exp2_split((double)refp - (double)P.M) / P.z;
      const double alq = exp2_split((double)refq - (double)Q.M) / Q.z;
      L.i[5] = timed_out ? 2 : ((P.ok && Q.ok) ? 0 : 1);
      L.f[2] = (float)(alp / alq);
      L.f[3] = (float)alq;
    }
  }
  __syncthreads();
  const int st = L.i[5];
  const float rr = L.f[2], alq = L.f[3];
  float sres[1] = {0.f};
  if (st == 0) {
    // sum_x [p - q]_+ = alpha_q * sum_x max(e_p r - e_q, 0)
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) sres[0] += fmaxf(fmaf(ep[j], rr, -eq[j]), 0.f);
  }
  __syncthreads();
  block_sum_f<1>(sres, L.red);
  if (t == 0) {
    // NaN marks a slice whose wait gave up; 0 when a row is non-finite
    const float mass = st == 2 ? __int_as_float(0x7fc00000) : (st == 1 ? 0.f : sres[0] * alq);
    st_coh(a.smass + (int64_t)r * n_s + s, tagged(mass, tag));
  }
  __syncthreads();
}

// ---------------------------------------------------------------- the kernel

template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_fused(FusedArgs a) {
  __shared__ Lds L;
  const int t = threadIdx.x;

  // stage the draft offsets, check them as one exclusive prefix, build team -> request
  for (int k = t; k <= a.B; k += kThreads) L.cu[k] = a.cu[k];
  __syncthreads();
  int bad = 0;
  for (int k = t; k < a.B; k += kThreads) {
    const int g = L.cu[k + 1] - L.cu[k];
    if (g < 0 || g > a.G) bad = 1;
  }
  if (t == 0 && (L.cu[0] != 0 || L.cu[a.B] != a.n_draft_rows)) bad = 1;
  bad = block_or(bad, L.i);
  if (bad) {
    for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
      if (t <= a.G) a.out_tokens[(int64_t)b * (a.G + 1) + t] = -1;
      if (t == 0) {
        a.out_num_accepted[b] = 0;
        a.out_status[b] = kStBadGamma;
        if (a.out_req_stats)
          for (int q = 0; q < 4; ++q) a.out_req_stats[(int64_t)b * 4 + q] = __int_as_float(0x7fc00000);
      }
    }
    return;
  }
  for (int b = t; b < a.B; b += kThreads) {
    const int c0 = L.cu[b], g = L.cu[b + 1] - c0;
    for (int i = 0; i <= g; ++i) L.team_req[c0 + b + i] = (uint16_t)b;
  }
  __syncthreads();

  // the first n_fin workgroups finalize requests as they complete; the rest stream
  if ((int)blockIdx.x < a.n_fin) {
    for (int b = blockIdx.x; b < a.B; b += a.n_fin) finalize_request<DT, VEC, MODE>(a, L, b);
    return;
  }
  const int w0 = blockIdx.x - a.n_fin, stride = gridDim.x - a.n_fin;
  const int n_s = a.n_s;
  auto decode = [&](int xt) {
    Ticket T;
    T.r = xt / n_s;
    T.s = xt - T.r * n_s;
    T.b = L.team_req[T.r];
    T.c0 = L.cu[T.b];
    T.g = L.cu[T.b + 1] - T.c0;
    T.i = T.r - T.c0 - T.b;
    T.pair = (MODE == kFuSample) && (T.i < T.g);
    return T;
  };
  RawSlice<DT> nxp, nxq;
  auto issue = [&](const Ticket& T) {
    load_raw<DT, VEC>(row_ptr<DT>(a.tgt, a.tgt_ld, T.r), a.V, T.s * kChunk, nxp);
    if (T.pair) load_raw<DT, VEC>(row_ptr<DT>(a.drf, a.drf_ld, T.c0 + T.i), a.V, T.s * kChunk, nxq);
  };

  // two-stage pipeline: phase 1 of ticket k, then phase 2 (team wait) of ticket k - 1, while
  // the loads of ticket k + 1 are in flight
  float ep[kPerThread], eq[kPerThread];
  int pend_r = -1, pend_s = 0;
  float pend_refp = 0.f, pend_refq = 0.f;
  if (w0 < a.n_tickets) issue(decode(w0));
  for (int xt = w0;; xt += stride) {
    const bool have = xt < a.n_tickets;
    Ticket T;
    T.pair = false;
    float vp[kPerThread], vq[kPerThread];
    float refp = 0.f, refq = 0.f;
    if (have) {
      T = decode(xt);
      unpack_raw<DT>(nxp, vp);
      if (T.pair) unpack_raw<DT>(nxq, vq);
      if (xt + stride < a.n_tickets) issue(decode(xt + stride));
      phase1<DT, MODE>(a, L, T, vp, vq, refp, refq);
    }
    if (MODE == kFuSample && pend_r >= 0) phase2(a, L, pend_r, pend_s, pend_refp, pend_refq, ep, eq);
    if (!have) break;
    pend_r = -1;
    if (T.pair) {
      pend_r = T.r;
      pend_s = T.s;
      pend_refp = refp;
      pend_refq = refq;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) { ep[j] = vp[j]; eq[j] = vq[j]; }
    }
  }
}

// ---------------------------------------------------------------- launch

template <int DT, bool VEC, int MODE>
static hipError_t launch_fused_t(FusedArgs a, hipStream_t st) {
  const void* fn = (const void*)k_fused<DT, VEC, MODE>;
  static int cached_dev = -1, cached_grid = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    cached_grid = per_cu * cus;
    cached_dev = dev;
  }
  int grid = cached_grid;
  if (const char* g = getenv("SPEC_VERIFY_GRID")) {   // debug: a smaller resident grid
    const int want = atoi(g);
    if (want > 0 && want < grid) grid = want;
  }
  if (grid > a.n_tickets + 128) grid = a.n_tickets + 128;
  if (grid < 2) return hipErrorInvalidConfiguration;
  // finalizer workgroups: enough that finalizing keeps pace with the requests completing
  a.n_fin = a.B < grid / 4 ? a.B : grid / 4;
  if (a.n_fin > 128) a.n_fin = 128;
  if (grid - a.n_fin < 1) return hipErrorInvalidConfiguration;
  if (getenv("SPEC_VERIFY_DEBUG"))
    fprintf(stderr, "[specverify] fused grid %d (resident capacity %d, finalizers %d) tickets %d slices %d mode %d\n",
            grid, cached_grid, a.n_fin, a.n_tickets, a.n_s, a.mode);
  void* args[] = {&a};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, st);
}

hipError_t launch_fused(const FusedArgs& a, int dt, int vec, hipStream_t st) {
  if (dt == kDtBF16) {
    if (a.mode == kFuSample) return vec ? launch_fused_t<kDtBF16, true, kFuSample>(a, st) : launch_fused_t<kDtBF16, false, kFuSample>(a, st);
    if (a.mode == kFuTokenOnly) return vec ? launch_fused_t<kDtBF16, true, kFuTokenOnly>(a, st) : launch_fused_t<kDtBF16, false, kFuTokenOnly>(a, st);
    return vec ? launch_fused_t<kDtBF16, true, kFuGreedy>(a, st) : launch_fused_t<kDtBF16, false, kFuGreedy>(a, st);
  }
  if (a.mode == kFuSample) return vec ? launch_fused_t<kDtF32, true, kFuSample>(a, st) : launch_fused_t<kDtF32, false, kFuSample>(a, st);
  if (a.mode == kFuTokenOnly) return vec ? launch_fused_t<kDtF32, true, kFuTokenOnly>(a, st) : launch_fused_t<kDtF32, false, kFuTokenOnly>(a, st);
  return vec ? launch_fused_t<kDtF32, true, kFuGreedy>(a, st) : launch_fused_t<kDtF32, false, kFuGreedy>(a, st);
}

size_t fused_record_bytes() { return 3 * sizeof(uint64_t); }

}  // namespace specv
