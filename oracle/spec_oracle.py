"""fp64 CPU oracle for batched speculative-sampling verification -- TEST INFRASTRUCTURE ONLY.

Nothing on the product path imports this module.  It is the plain, slow, obviously correct
definition that the HIP library is checked against, written in float64 numpy with Python
loops over requests and positions.  Inputs are widened exactly (bf16/fp32 -> fp64).

Pages followed (cited by page title and section):

  [SD]  "5.1 投机解码核心原理" (speculative decoding: core principles), an inference-optimisation
        guide page:  §2.1 the draft proposes y_i from q_i and the target scores p_i for
        i = 1..gamma+1, p and q being the actual sampling distributions after temperature /
        top-k / top-p;  §3.1 greedy rule (accept iff y_i is the target argmax, else emit the
        argmax and stop);  §3.2 stochastic rule a_i = min(1, p_i(y_i)/q_i(y_i)), accept iff
        u < a_i, residual r_i = [p_i - q_i]_+ / sum [p_i - q_i]_+;  §3.3 a token-only draft is
        a one-hot q;  §4.1-4.2 q*a = min(p,q), beta = sum [p-q]_+ = 1 - A;  §4.3 A = 1 - TV;
        §5.1 stop at the first rejection;  §5.2 bonus token from p_{gamma+1};  §7 the worked
        example p = [0.6, 0.3, 0.1], q = [0.2, 0.5, 0.3].
  [DL]  "DLite: History-free Speculative Decoding for Agentic AI", section "核心方法" (core
        method): one projection onto the vocabulary per round.
  [SKV] "SpecKV: Adaptive Speculative Decoding with Compression-Aware Gamma Selection",
        section "草稿模型信号提取" (draft-model signals): per-position draft entropy in bits and
        max probability, their mean over the block, the maximum entropy and the minimum
        confidence.

Readings taken where the pages leave a step open (plainest reading the rest supports):

  R1  Filter order: temperature first, then top-k, then top-p on the renormalised top-k set.
      Top-k keeps every logit >= the k-th largest logit counted with multiplicity (ties at the
      boundary are all kept).  Top-p walks the distinct kept values from the largest down and
      keeps the shortest such prefix whose probability reaches top_p (>=), the boundary value
      group kept whole.  top_k <= 0 or >= V and top_p >= 1 switch the filter off.
  R2  Argmax ties resolve to the lowest index (float comparison, so -0 == +0).
  R3  Entropy is in bits, on the same filtered, tempered distribution used for verification.
  R4  The accept test is strict: accept iff u < min(1, p/q), u in [0, 1).
  R5  Randomness: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11), key (seed, step),
      counter (b, i, 0, 0) for request b and 1-based position i.  Word 0 is the accept draw
      at i; words 1..3 drive the three sampler levels when the emitted token is drawn at i.
      spec_residual_sample uses counter (r, 0, 1, 0), words 1..3.  u = (w >> 11) * 2^-53.
  R6  Sampling uses a three-level, fixed-order inverse CDF over the weights w (the residual or
      p_{gamma+1}): chunks of 4096 indices, groups of 64 inside a chunk, then elements; one
      independent uniform per level.  The law is exactly w/W:
      P(x) = (S_k/W) (M_kg/S_k) (w_x/M_kg).  Masses are sequential sums: M_kg over the group's
      elements, S_k over the chunk's group masses, W over the chunk masses.
  R7  T = 0 is greedy: p is one-hot at the argmax, the draft is read as token-only (one-hot q
      at y), draft-side statistics are NaN.
  R8  Errors: a request with any NaN / +inf logit, or a row with no finite logit, in any of
      its rows gets status NONFINITE, 0 accepted and no tokens.  A draft token outside
      [0, V) sets BAD_TOKEN and q(y) = 0 sets ZERO_Q; both count as a rejection at that
      position (the residual uses the full q).  An all-zero residual after a rejection sets
      RESIDUAL_EMPTY and the token is drawn from p instead.
  R9  A token-only draft at T > 0 is a one-hot q at y; a bad y there leaves q = 0 (residual
      = p).
  R10 Extra signals per position (the uncertainty features of the tree-search page's
      selector: both KL divergences and the L1 distance, with the forward KL of the DLite
      page's loss section, D_KL(p||q) = sum_v p(v) log(p(v)/q(v))): KL in nats (natural log,
      as written there), 0 log 0 = 0, +inf when one side puts mass where the other has none;
      L1 = sum_x |p - q| = 2 TV.  They use the same p_i and q_i as verification (q one-hot at
      y_i for a token-only draft; NaN there when y_i is not a token).  Under greedy (R7) both
      KL values are NaN.  The accept probability a_i = min(1, p_i(y_i) / q_i(y_i)) (0 when y_i
      is not a token or q_i(y_i) = 0; greedy: 1 iff y_i is the target argmax) and, per
      request, the expected number of tokens committed given the drafts,
      E = 1 + sum_{k=1..gamma} prod_{i<=k} a_i: the tree-search page's variance-free block
      efficiency (a sum over reachable nodes of products of branch transition probabilities)
      for a single chain under the standard rule.

  R11 Gamma selection ([SKV] "接受率预测与 gamma 选择", acceptance prediction and gamma
      selection): context x = [H_bar, c_bar, H_max, c_min, comp] (the request statistics above
      plus the caller's compression feature); a regressor f(x, gamma) predicts the acceptance
      rate; the expected tokens of a step are f(x, gamma) * gamma + 1, and gamma* is the
      argmax over {2, 4, 6, 8}.  The pages name an MLP with 16 hidden units but not its
      layout: read as input [x, gamma] (6 values), one hidden layer of 16 ReLU units and a
      linear output, weights supplied by the caller (the trained ones are not available).
      Ties go to the smallest gamma; a NaN feature gives gamma* = -1.

  R12 Fused LM head ([DL] the DLite page, section "核心方法" (core method): the draft's sequential
      head works in the hidden space and projects onto the vocabulary once).  The logits of a
      row are l_v = sum_d h_d W_{v,d} for a hidden state h [D] and a head W [V, D], taken in
      float64 from the exact bf16 values; the row statistics are those of spec_row_stats
      (R1-R3, R7, R8) with no filter, and p_tok is the row's probability of a given token
      (NaN for a token outside [0, V) or a non-finite row).  The GPU accumulates the products
      (exact in fp32) in fp32, so its logits may differ from these by up to
      D * 2^-24 * sum_d |h_d W_{v,d}|, the standard bound for a sum of D terms; the parity
      tolerances follow from it, and inputs whose partial sums are all exact in fp32 pin the
      statistics at the usual bar.

Every function states which of the above it follows.  The decision margins recorded next
to each result (distance of u from the accept ratio, of u*M from the sampler prefix sums,
of the top-p cumulative mass from top_p) let a comparison excuse a mismatch that sits
within rounding distance of a boundary.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096
GROUP = 64

STATUS_NONFINITE = 1
STATUS_BAD_TOKEN = 2
STATUS_ZERO_Q = 4
STATUS_RESIDUAL_EMPTY = 8
STATUS_TIMEOUT = 16

_MASK64 = (1 << 64) - 1


@dataclass
class SamplingParams:
    """Temperature (0 = greedy), top_k (<=0 or >=V: off), top_p (>=1: off).  [SD] §2.1."""

    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0


# ----------------------------------------------------------------------------- randomness


def philox4x64_10(key, counter):
    """Philox4x64-10 block (Salmon et al., SC'11): 10 rounds of two 64x64->128 multiplies.

    key = (k0, k1), counter = (c0, c1, c2, c3), all unsigned 64-bit.  Returns 4 words.
    Reading R5.
    """
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    c0, c1, c2, c3 = (int(c) & _MASK64 for c in counter)
    for rnd in range(10):
        if rnd > 0:  # the key is bumped by the Weyl constants before every round but the first
            k0 = (k0 + 0x9E3779B97F4A7C15) & _MASK64
            k1 = (k1 + 0xBB67AE8584CAA73B) & _MASK64
        prod0 = 0xD2E7470EE14C6C93 * c0
        prod1 = 0xCA5A826395121157 * c2
        c0, c1, c2, c3 = (
            ((prod1 >> 64) ^ c1 ^ k0) & _MASK64,
            prod1 & _MASK64,
            ((prod0 >> 64) ^ c3 ^ k1) & _MASK64,
            prod0 & _MASK64,
        )
    return (c0, c1, c2, c3)


def u53(word):
    """Map a 64-bit word to [0, 1): the top 53 bits times 2^-53 (exact in fp64).  R5."""
    return float(int(word) >> 11) * (2.0 ** -53)


def position_uniforms(seed, step, b, i):
    """The four uniforms of request b, 1-based position i.  R5."""
    return tuple(u53(w) for w in philox4x64_10((seed, step), (b, i, 0, 0)))


def residual_uniforms(seed, step, r):
    """(u1, u2, u3) of row r of the standalone residual sampler.  R5."""
    w = philox4x64_10((seed, step), (r, 0, 1, 0))
    return (u53(w[1]), u53(w[2]), u53(w[3]))


# ----------------------------------------------------------------------------- one row


@dataclass
class RowDist:
    """The sampling distribution of one logit row plus its per-row statistics."""

    probs: np.ndarray          # fp64 [V]: the filtered, tempered distribution ([SD] §2.1)
    argmax: int                # lowest index of the largest logit (R2); -1 if non-finite
    max_logit: float
    log_z: float               # ln sum_kept exp(l/T)  (NaN when greedy)
    entropy_bits: float        # [SKV]: -sum p log2 p
    max_prob: float            # [SKV]: max_x p(x)
    kept_count: int            # |{x : l_x >= final threshold, l_x > -inf}|
    finite: bool
    topp_margin: float = math.inf   # min |cum - top_p| at the boundary group and the one before


def _nonfinite_row(V):
    nan = float("nan")
    return RowDist(np.full(V, nan), -1, nan, nan, nan, nan, 0, False)


def row_distribution(logits, sp: SamplingParams) -> RowDist:
    """Filtered, tempered distribution of one row.  [SD] §2.1 with readings R1, R2, R3, R7, R8."""
    l = np.asarray(logits, dtype=np.float64)
    V = l.shape[0]
    if np.isnan(l).any() or np.isposinf(l).any() or not np.isfinite(l).any():
        return _nonfinite_row(V)
    m = float(l.max())
    amax = int(np.argmax(l))  # first occurrence of the maximum
    T = float(sp.temperature)
    if T == 0.0:  # greedy: one-hot target (R7)
        probs = np.zeros(V)
        probs[amax] = 1.0
        return RowDist(probs, amax, m, float("nan"), 0.0, 1.0, 1, True)

    keep = np.ones(V, dtype=bool)
    threshold = -math.inf
    # top-k: keep every value >= the k-th largest, counted with multiplicity (R1)
    if 0 < sp.top_k < V:
        tau_k = float(np.sort(l)[::-1][sp.top_k - 1])
        threshold = tau_k
        keep = l >= tau_k
    topp_margin = math.inf
    # top-p over the renormalised top-k set, walking distinct values downwards (R1)
    if sp.top_p < 1.0:
        e = np.where(keep, np.exp((l - m) / T), 0.0)
        pi = e / e.sum()
        values = np.unique(l[keep])[::-1]  # distinct kept values, largest first
        cum = 0.0
        chosen = values[-1]
        prev_cum = None
        for v in values:
            prev_cum = cum
            cum += float(pi[l == v].sum())
            if cum >= sp.top_p:
                chosen = v
                break
        threshold = max(threshold, float(chosen))
        topp_margin = abs(cum - sp.top_p)
        if prev_cum is not None and prev_cum > 0.0:
            topp_margin = min(topp_margin, abs(prev_cum - sp.top_p))
        keep = keep & (l >= chosen)

    e = np.where(keep, np.exp((l - m) / T), 0.0)
    z = float(e.sum())
    probs = e / z
    nz = probs > 0.0
    entropy_bits = float(-(probs[nz] * np.log2(probs[nz])).sum())
    return RowDist(
        probs=probs,
        argmax=amax,
        max_logit=m,
        log_z=m / T + math.log(z),
        entropy_bits=entropy_bits,
        max_prob=float(probs.max()),
        kept_count=int(np.count_nonzero(keep & (l > -math.inf))),
        finite=True,
        topp_margin=topp_margin,
    )


def onehot(V, y):
    """A token-only draft as a distribution: one-hot at y, all zero if y is not a token.  [SD] §3.3, R9."""
    q = np.zeros(V)
    if 0 <= y < V:
        q[y] = 1.0
    return q


# ----------------------------------------------------------------------------- sampler


def _first_exceeding(cum, target):
    """min{c : cum[c] > target}; if rounding leaves none, the last index with positive mass."""
    idx = np.nonzero(cum > target)[0]
    if idx.size:
        return int(idx[0])
    steps = np.diff(np.concatenate(([0.0], cum)))
    return int(np.nonzero(steps > 0.0)[0][-1])


def _level_margin(cum, c, target, total):
    lo = cum[c - 1] if c > 0 else 0.0
    return min(target - lo, cum[c] - target) / total


def sample_three_level(w, u1, u2, u3):
    """Three-level fixed-order inverse CDF over weights w >= 0 with sum > 0.  Reading R6.

    Returns (index, margin) where margin is the smallest relative distance of u*mass from a
    prefix-sum boundary over the three levels.
    """
    w = np.asarray(w, dtype=np.float64)
    V = w.shape[0]
    n_chunks = (V + CHUNK - 1) // CHUNK

    def group_masses(k):
        lo, hi = k * CHUNK, min((k + 1) * CHUNK, V)
        return np.array([np.cumsum(w[g:min(g + GROUP, hi)])[-1] for g in range(lo, hi, GROUP)])

    S = np.array([np.cumsum(group_masses(k))[-1] for k in range(n_chunks)])
    cumS = np.cumsum(S)
    W = cumS[-1]
    k = _first_exceeding(cumS, u1 * W)
    margin = _level_margin(cumS, k, u1 * W, W)

    M = group_masses(k)
    cumM = np.cumsum(M)
    g = _first_exceeding(cumM, u2 * cumM[-1])
    margin = min(margin, _level_margin(cumM, g, u2 * cumM[-1], cumM[-1]))

    lo = k * CHUNK + g * GROUP
    elems = w[lo:min(lo + GROUP, V)]
    cumE = np.cumsum(elems)
    x = _first_exceeding(cumE, u3 * cumE[-1])
    margin = min(margin, _level_margin(cumE, x, u3 * cumE[-1], cumE[-1]))
    return lo + x, margin


# ----------------------------------------------------------------------------- one request


@dataclass
class Decision:
    """One decision of a round and its distance from the boundary that decides it.

    kind "accept": the accept test at 1-based position i, margin |u0 - a_i|.
    kind "sample": the token drawn at position i, margin = the sampler's smallest relative
    distance over its three levels.  kind "topp": the top-p boundary of one row, margin =
    |cumulative mass - top_p| at the chosen value group and the one before it; ``row`` says
    which row ("target" or "draft") and ``position`` its 1-based position.
    """

    kind: str
    position: int
    margin: float
    row: str = ""


@dataclass
class RequestResult:
    num_accepted: int
    tokens: list                  # accepted draft tokens then the correction / bonus token
    status: int
    p_y: np.ndarray               # [gamma]
    q_y: np.ndarray               # [gamma]
    one_minus_tv: np.ndarray      # [gamma]: sum_x min(p, q)   ([SD] §4.1, §4.3)
    tv: np.ndarray                # [gamma]: 1/2 sum |p - q|
    draft_entropy_bits: np.ndarray  # [gamma]
    draft_max_prob: np.ndarray      # [gamma]
    target_entropy_bits: np.ndarray  # [gamma + 1]
    target_max_prob: np.ndarray      # [gamma + 1]
    req_stats: np.ndarray            # [4]: mean H, mean c, max H, min c   ([SKV])
    kl_pq: np.ndarray = None         # [gamma]: D_KL(p_i || q_i) in nats (R10)
    kl_qp: np.ndarray = None         # [gamma]: D_KL(q_i || p_i) in nats
    l1: np.ndarray = None            # [gamma]: sum |p_i - q_i| = 2 TV
    accept_prob: np.ndarray = None   # [gamma]: a_i = min(1, p_i(y_i) / q_i(y_i))
    expected_committed: float = float("nan")   # 1 + sum_k prod_{i<=k} a_i
    decisions: list = field(default_factory=list)
    target_rows: list = field(default_factory=list)
    draft_rows: list = field(default_factory=list)


def kl_divergence(a, b):
    """D_KL(a || b) = sum_x a(x) ln(a(x) / b(x)) in nats, terms with a(x) = 0 dropped; +inf
    when a puts mass where b has none (R10)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if np.isnan(a).any() or np.isnan(b).any():
        return float("nan")
    pos = a > 0.0
    if (b[pos] == 0.0).any():
        return math.inf
    return float((a[pos] * np.log(a[pos] / b[pos])).sum())


def verify_request(target_logits, draft_logits, draft_tokens, sp: SamplingParams,
                   seed: int, step: int, b: int, uniforms=None, resample_rule="residual"):
    """One speculative round of request b.  [SD] §3-§5 with readings R4-R9.

    target_logits: [gamma+1, V]; draft_logits: [gamma, V] or None (token-only draft);
    draft_tokens: [gamma].  ``uniforms`` (test hook) maps position i -> (u0, u1, u2, u3) and
    replaces Philox.  ``resample_rule`` = "p" is the WRONG rule of [SD] §7 (resample from p
    after a rejection) and exists only as a negative control for tests.
    """
    tl = np.asarray(target_logits, dtype=np.float64)
    gamma = tl.shape[0] - 1
    V = tl.shape[1]
    ys = [int(y) for y in draft_tokens]
    assert len(ys) == gamma
    greedy = float(sp.temperature) == 0.0
    token_only = greedy or draft_logits is None

    P = [row_distribution(tl[i], sp) for i in range(gamma + 1)]
    Q = None
    if not token_only:
        dl = np.asarray(draft_logits, dtype=np.float64)
        assert dl.shape == (gamma, V)
        Q = [row_distribution(dl[i], sp) for i in range(gamma)]

    nan = float("nan")
    res = RequestResult(
        num_accepted=0, tokens=[], status=0,
        p_y=np.full(gamma, nan), q_y=np.full(gamma, nan),
        one_minus_tv=np.full(gamma, nan), tv=np.full(gamma, nan),
        draft_entropy_bits=np.full(gamma, nan), draft_max_prob=np.full(gamma, nan),
        target_entropy_bits=np.array([r.entropy_bits for r in P]),
        target_max_prob=np.array([r.max_prob for r in P]),
        req_stats=np.full(4, nan), target_rows=P, draft_rows=Q or [],
        kl_pq=np.full(gamma, nan), kl_qp=np.full(gamma, nan), l1=np.full(gamma, nan),
        accept_prob=np.full(gamma, nan),
    )
    for kind, rows in (("target", P), ("draft", Q or [])):
        for i, r in enumerate(rows):
            if r.topp_margin < math.inf:
                res.decisions.append(Decision("topp", i + 1, r.topp_margin, kind))

    # per-position draft distributions (one-hot for token-only drafts) and pair statistics
    qdists = []
    for i in range(gamma):
        if Q is not None:
            qd = Q[i].probs
            res.draft_entropy_bits[i] = Q[i].entropy_bits
            res.draft_max_prob[i] = Q[i].max_prob
        else:
            qd = onehot(V, ys[i])
            if not greedy and 0 <= ys[i] < V:  # a one-hot draft has zero entropy, confidence 1
                res.draft_entropy_bits[i] = 0.0
                res.draft_max_prob[i] = 1.0
        qdists.append(qd)
        p = P[i].probs
        res.one_minus_tv[i] = float(np.minimum(p, qd).sum())
        res.tv[i] = 0.5 * float(np.abs(p - qd).sum())
        yv = 0 <= ys[i] < V
        if yv:
            res.p_y[i] = float(p[ys[i]])
            res.q_y[i] = float(qd[ys[i]])
        # extra signals (R10)
        if Q is not None or yv:
            res.l1[i] = float(np.abs(p - qd).sum())
            if not greedy:
                res.kl_pq[i] = kl_divergence(p, qd)
                res.kl_qp[i] = kl_divergence(qd, p)
        if not (P[i].finite and (Q is None or Q[i].finite)):
            res.accept_prob[i] = nan   # a non-finite row has no distribution (R8)
        elif greedy:
            res.accept_prob[i] = 1.0 if (yv and ys[i] == P[i].argmax) else 0.0
        elif not yv or qd[ys[i]] == 0.0:
            res.accept_prob[i] = 0.0
        else:
            res.accept_prob[i] = min(1.0, float(p[ys[i]]) / float(qd[ys[i]]))
    run = 1.0
    res.expected_committed = 1.0
    for i in range(gamma):
        run *= res.accept_prob[i]
        res.expected_committed += run
    if gamma > 0 and not greedy:
        h, c = res.draft_entropy_bits, res.draft_max_prob
        res.req_stats[:] = [h.mean(), c.mean(), h.max(), c.min()]

    if not all(r.finite for r in P + (Q or [])):
        res.status |= STATUS_NONFINITE
        res.expected_committed = float("nan")
        return res

    def draws(i):
        if uniforms is not None:
            return uniforms[i]
        return position_uniforms(seed, step, b, i)

    # accept scan: stop at the first rejection ([SD] §3.1, §3.2, §5.1)
    j = None
    for i in range(1, gamma + 1):
        y = ys[i - 1]
        p = P[i - 1]
        if not (0 <= y < V):
            res.status |= STATUS_BAD_TOKEN
            j = i
            break
        if greedy:
            if y == p.argmax:
                continue
            j = i
            break
        qy = qdists[i - 1][y]
        if qy == 0.0:
            res.status |= STATUS_ZERO_Q
            j = i
            break
        a = min(1.0, p.probs[y] / qy)
        u0 = draws(i)[0]
        res.decisions.append(Decision("accept", i, abs(u0 - a)))
        if not (u0 < a):
            j = i
            break

    if j is None:  # every draft token accepted: bonus token from p_{gamma+1} ([SD] §5.2)
        pos = gamma + 1
        w = P[gamma].probs
    else:          # correction token from the residual at the first rejection ([SD] §3.2)
        pos = j
        if resample_rule == "p":
            w = P[j - 1].probs
        else:
            w = np.maximum(P[j - 1].probs - qdists[j - 1], 0.0)
            if not (w.sum() > 0.0):
                res.status |= STATUS_RESIDUAL_EMPTY
                w = P[j - 1].probs
    _, u1, u2, u3 = draws(pos)
    x, margin = sample_three_level(w, u1, u2, u3)
    if not greedy:
        res.decisions.append(Decision("sample", pos, margin))
    n_acc = (j - 1) if j is not None else gamma
    res.num_accepted = n_acc
    res.tokens = ys[:n_acc] + [x]
    return res


# ----------------------------------------------------------------------------- batches


def _rows_of(logits, rows, V):
    return np.asarray(logits[rows], dtype=np.float64)[:, :V]


def verify_batch(target_logits, draft_logits, draft_tokens, cu_draft, sp: SamplingParams,
                 seed: int, step: int, requests=None):
    """Oracle of spec_verify_batch over ragged requests.  [SD] §2-§5.

    target_logits: [sum(gamma_b + 1), V] (fp64-convertible); request b's target rows start at
    cu_draft[b] + b.  draft_logits: [sum gamma_b, V] or None; request b's draft rows and
    tokens start at cu_draft[b].  ``requests`` restricts the work to a subset of b.
    Returns {b: RequestResult}.
    """
    cu = [int(c) for c in cu_draft]
    B = len(cu) - 1
    out = {}
    for b in (range(B) if requests is None else requests):
        g = cu[b + 1] - cu[b]
        t0 = cu[b] + b
        tl = np.asarray(target_logits[t0:t0 + g + 1], dtype=np.float64)
        dl = None if draft_logits is None else np.asarray(draft_logits[cu[b]:cu[b] + g], dtype=np.float64)
        ys = [int(y) for y in draft_tokens[cu[b]:cu[b] + g]]
        out[b] = verify_request(tl, dl, ys, sp, seed, step, b)
    return out


def row_stats(logits, sp: SamplingParams):
    """Oracle of spec_row_stats: per-row statistics of the filtered, tempered rows.

    Returns a dict of arrays: max_logit, argmax, log_z, entropy_bits, max_prob, kept_count.
    [SD] §2.1, [SKV] signal definitions, readings R1-R3, R7, R8.
    """
    rows = [row_distribution(np.asarray(r, dtype=np.float64), sp) for r in logits]
    return {
        "max_logit": np.array([r.max_logit for r in rows]),
        "argmax": np.array([r.argmax for r in rows], dtype=np.int64),
        "log_z": np.array([r.log_z for r in rows]),
        "entropy_bits": np.array([r.entropy_bits for r in rows]),
        "max_prob": np.array([r.max_prob for r in rows]),
        "kept_count": np.array([r.kept_count for r in rows], dtype=np.int64),
        "topp_margin": np.array([r.topp_margin for r in rows]),
    }


def residual_sample(p_logits, q_logits, sp: SamplingParams, uniforms=None, seed=0, step=0):
    """Oracle of spec_residual_sample: one draw per row from [p - q]_+ (or from p if q is None).

    Returns dict of arrays token, mass (beta = sum [p - q]_+, or 1 without q), status, margin.
    [SD] §3.2 residual formula and §4.1 beta identity, readings R5, R6, R8.
    """
    R = len(p_logits)
    tok = np.full(R, -1, dtype=np.int64)
    mass = np.full(R, float("nan"))
    status = np.zeros(R, dtype=np.int64)
    margin = np.full(R, math.inf)
    for r in range(R):
        P = row_distribution(np.asarray(p_logits[r], dtype=np.float64), sp)
        Q = None if q_logits is None else row_distribution(np.asarray(q_logits[r], dtype=np.float64), sp)
        if not P.finite or (Q is not None and not Q.finite):
            status[r] |= STATUS_NONFINITE
            continue
        if Q is None:
            w = P.probs
        else:
            w = np.maximum(P.probs - Q.probs, 0.0)
        beta = float(w.sum())
        mass[r] = beta
        if not beta > 0.0:
            status[r] |= STATUS_RESIDUAL_EMPTY
            w = P.probs
        u = uniforms[r] if uniforms is not None else residual_uniforms(seed, step, r)
        tok[r], margin[r] = sample_three_level(w, *u)
    return {"token": tok, "mass": mass, "status": status, "margin": margin}


# ----------------------------------------------------------------------------- gamma selection


GAMMAS = (2, 4, 6, 8)


def select_gamma(req_stats, comp, w1, b1, w2, b2, gammas=GAMMAS):
    """gamma* = argmax_gamma f(x, gamma) * gamma + 1 with f an MLP-16 over [x, gamma].  [SKV]
    acceptance prediction and gamma selection, reading R11.

    req_stats: [4] = H_bar, c_bar, H_max, c_min; comp: the compression feature; w1 [16, 6],
    b1 [16], w2 [16], b2 scalar.  Returns (gamma*, expected tokens per gamma [4], margin) where
    the margin is the gap between the best and the runner-up expectation (ties excused below
    rounding distance).
    """
    x = np.asarray(list(req_stats) + [comp], dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    if np.isnan(x).any():
        return -1, np.full(len(gammas), np.nan), math.inf
    E = np.empty(len(gammas))
    for g, gamma in enumerate(gammas):
        h = np.maximum(w1 @ np.append(x, float(gamma)) + b1, 0.0)
        E[g] = (float(w2 @ h) + float(b2)) * gamma + 1.0
    best = int(np.argmax(E))   # first maximum: the smallest gamma on ties
    rest = np.delete(E, best)
    margin = float(E[best] - rest.max()) if len(rest) else math.inf
    return gammas[best], E, margin


# ----------------------------------------------------------------------------- fused LM head


def lm_head_logits(hidden, weight):
    """l = h W^T in float64 from the exact bf16 values (as float arrays).  [DL] core method,
    reading R12."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return h @ w.T


def lm_head_row_stats(hidden, weight, sp: SamplingParams, tokens=None):
    """Oracle of spec_lm_head_row_stats: the statistics of row_stats on l = h W^T, plus p_tok.
    [DL] core method and the signals of [SKV], readings R12, R2, R3, R7, R8.

    hidden [R, D] and weight [V, D] hold the bf16 values as floats; tokens [R] or None.
    Returns row_stats's dict plus "p_tok" [R] (NaN where not defined) and "logits".
    """
    if sp.top_k > 0 and sp.top_k < np.asarray(weight).shape[0] or sp.top_p < 1.0:
        raise ValueError("the fused head takes no top-k / top-p filter")
    logits = lm_head_logits(hidden, weight)
    out = row_stats(logits, sp)
    R, V = logits.shape
    p_tok = np.full(R, float("nan"))
    if tokens is not None:
        for r in range(R):
            y = int(tokens[r])
            if 0 <= y < V:
                d = row_distribution(logits[r], sp)
                if d.finite:
                    p_tok[r] = float(d.probs[y])
    out["p_tok"] = p_tok
    out["logits"] = logits
    return out
