"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test names what it pins.  A plausible mistake in the oracle (a dropped term, a wrong sign,
a swapped p/q, an off-by-one position, a wrong counter layout) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import spec_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- Philox


@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (0, 0, 0, 0)),
    ((1, 2), (1, 0, 0, 0)),
    ((0xDEADBEEFCAFEF00D, 0x0123456789ABCDEF), (7, 3, 0, 0)),
    ((2**64 - 1, 2**64 - 1), (2**64 - 1, 2**64 - 1, 2**64 - 1, 2**64 - 2)),
    ((42, 17), (12345, 8, 1, 0)),
])
def test_philox_matches_numpy(key, ctr):
    """Pin: numpy's independent Philox4x64-10.  numpy increments the 256-bit counter before
    producing a block, so it is seeded with counter - 1."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    npctr = np.array([(c >> (64 * i)) & (2**64 - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=npctr)
    ref = [int(v) for v in bg.random_raw(4)]
    assert list(O.philox4x64_10(key, ctr)) == ref


def test_u53_exact_and_in_range():
    assert O.u53(0) == 0.0
    assert O.u53(2**64 - 1) == 1.0 - 2.0**-53
    assert O.u53(1 << 11) == 2.0**-53
    assert O.u53(1 << 63) == 0.5


def test_position_uniform_layout():
    """Counter (b, i, 0, 0), key (seed, step): words are taken in order.  Reading R5."""
    w = O.philox4x64_10((5, 9), (3, 2, 0, 0))
    assert O.position_uniforms(5, 9, 3, 2) == tuple(O.u53(x) for x in w)
    w = O.philox4x64_10((5, 9), (3, 0, 1, 0))
    assert O.residual_uniforms(5, 9, 3) == tuple(O.u53(x) for x in w[1:])


# ----------------------------------------------------------------------------- worked example


def _worked_rows():
    g = golden()
    return np.array(g["p"]), np.array(g["q"]), g


def test_worked_example_distributions():
    """[SD] §7: logits ln p, ln q at T = 1 reproduce p and q; overlap, beta, residual, TV."""
    p, q, g = _worked_rows()
    sp = O.SamplingParams(1.0)
    P = O.row_distribution(np.log(p), sp)
    Q = O.row_distribution(np.log(q), sp)
    np.testing.assert_allclose(P.probs, p, atol=1e-12)
    np.testing.assert_allclose(Q.probs, q, atol=1e-12)
    res = O.verify_request(np.log(np.stack([p, p])), np.log(q)[None], [0], sp, 1, 0, 0)
    overlap = np.minimum(P.probs, Q.probs)
    np.testing.assert_allclose(overlap, g["accept_path_mass"], atol=1e-12)
    assert res.one_minus_tv[0] == pytest.approx(sum(g["accept_path_mass"]), abs=1e-12)
    assert res.tv[0] == pytest.approx(g["rejection_mass"], abs=1e-12)
    resid = np.maximum(P.probs - Q.probs, 0)
    assert resid.sum() == pytest.approx(g["rejection_mass"], abs=1e-12)
    r = resid / resid.sum()
    assert r[g["rejection_mass_all_on_token"]] == pytest.approx(1.0, abs=1e-12)


def _exact_law(p, q_or_none, ys_weights, sp, n=2000, rule="residual"):
    """Output law of verify_request for gamma = 1 and V <= 64 (one chunk, one group, so only
    u0 and u3 act).  For each y (with its weight) the accept probability is the fraction of a
    midpoint grid of u0 that accepts, and the law after a rejection is the law of a midpoint
    grid of u3 with u0 = 1 - 2^-53 (a rejection whenever a < 1).  Deterministic; resolution
    1/n on both draws."""
    V = len(p)
    law = np.zeros(V)
    grid = (np.arange(n) + 0.5) / n
    tl = np.log(np.stack([p, p]))
    dl = None if q_or_none is None else np.log(np.asarray(q_or_none))[None]
    u_rej = 1.0 - 2.0**-53

    def run(y, u0, u3):
        us = {1: (u0, 0.3, 0.6, u3), 2: (0.5, 0.3, 0.6, u3)}
        return O.verify_request(tl, dl, [y], sp, 0, 0, 0, uniforms=us, resample_rule=rule)

    for y, wy in ys_weights:
        if wy == 0:
            continue
        acc = np.mean([run(y, u0, 0.5).num_accepted == 1 for u0 in grid])
        law[y] += wy * acc
        if acc < 1.0:
            rej = np.zeros(V)
            for u3 in grid:
                res = run(y, u_rej, u3)
                assert res.num_accepted == 0
                rej[res.tokens[0]] += 1.0 / n
            law += wy * (1.0 - acc) * rej
    return law


def test_worked_example_output_law_is_p():
    """[SD] §4.2 / §7: accept path + residual path = p exactly (to the grid resolution)."""
    p, q, g = _worked_rows()
    law = _exact_law(p, q, list(enumerate(q)), O.SamplingParams(1.0))
    np.testing.assert_allclose(law, g["standard_rule_final"], atol=2e-3)


def test_worked_example_wrong_rule_law():
    """[SD] §7: resampling from p after a rejection gives [0.44, 0.42, 0.14] (negative control)."""
    p, q, g = _worked_rows()
    law = _exact_law(p, q, list(enumerate(q)), O.SamplingParams(1.0), rule="p")
    np.testing.assert_allclose(law, g["wrong_rule_final"], atol=2e-3)
    assert np.abs(law - np.array(g["standard_rule_final"])).max() > 0.1


def test_worked_example_onehot_draft():
    """[SD] §3.3 / §7: a token-only draft proposing token 1 is accepted with p(1) = 0.3 and the
    output law is still p."""
    p, q, g = _worked_rows()
    sp = O.SamplingParams(1.0)
    law = _exact_law(p, None, [(1, 1.0)], sp)
    np.testing.assert_allclose(law, g["onehot_final"], atol=2e-3)
    res = O.verify_request(np.log(np.stack([p, p])), None, [1], sp, 0, 0, 0)
    assert res.one_minus_tv[0] == pytest.approx(g["onehot_acceptance"], abs=1e-12)
    assert res.p_y[0] == pytest.approx(g["onehot_acceptance"], abs=1e-12)
    assert res.q_y[0] == 1.0


# ----------------------------------------------------------------------------- identities


def _random_pair(rng, V, T=1.0, top_k=0, top_p=1.0, scale=2.0):
    lp = rng.normal(0, scale, V)
    lq = lp + rng.normal(0, 1.0, V)
    sp = O.SamplingParams(T, top_k, top_p)
    return O.row_distribution(lp, sp), O.row_distribution(lq, sp), sp


@pytest.mark.parametrize("V,T,k,pp", [(8, 1.0, 0, 1.0), (1000, 0.7, 0, 1.0), (5000, 1.3, 50, 0.9),
                                      (300, 0.5, 0, 0.95), (64, 1.0, 10, 1.0)])
def test_identities(V, T, k, pp):
    """[SD] §4.1-4.3: A + TV = 1, min(p,q) + [p-q]_+ = p, beta = sum [p-q]_+ = 1 - A."""
    rng = np.random.default_rng(V + k)
    for _ in range(5):
        P, Q, sp = _random_pair(rng, V, T, k, pp)
        p, q = P.probs, Q.probs
        A = np.minimum(p, q).sum()
        TV = 0.5 * np.abs(p - q).sum()
        beta = np.maximum(p - q, 0).sum()
        assert A + TV == pytest.approx(1.0, abs=1e-12)
        np.testing.assert_allclose(np.minimum(p, q) + np.maximum(p - q, 0), p, atol=1e-15)
        assert beta == pytest.approx(1.0 - A, abs=1e-12)
        res = O.verify_request(np.stack([np.log(p + 1e-300)] * 2), np.log(q + 1e-300)[None], [0],
                               O.SamplingParams(1.0), 0, 0, 0)
        assert res.one_minus_tv[0] + res.tv[0] == pytest.approx(1.0, abs=1e-9)


def test_softmax_and_entropy_match_scipy():
    """Library cross-check: scipy softmax and scipy entropy (base 2) on unfiltered rows."""
    rng = np.random.default_rng(3)
    for V, T in [(8, 1.0), (1000, 0.7), (4097, 2.0)]:
        l = rng.normal(0, 3, V)
        r = O.row_distribution(l, O.SamplingParams(T))
        ref = scipy.special.softmax(l / T)
        np.testing.assert_allclose(r.probs, ref, rtol=1e-12, atol=1e-300)
        assert r.entropy_bits == pytest.approx(scipy.stats.entropy(ref, base=2), rel=1e-12)
        assert r.max_prob == pytest.approx(ref.max(), rel=1e-12)
        assert r.log_z == pytest.approx(scipy.special.logsumexp(l / T), rel=1e-12)
        assert r.argmax == int(np.argmax(l))


def test_uniform_logits():
    """Closed form: uniform logits give H = log2 V and max-prob = 1/V."""
    for V in [3, 8, 4096, 151936]:
        r = O.row_distribution(np.full(V, 1.25), O.SamplingParams(0.7))
        assert r.entropy_bits == pytest.approx(math.log2(V), rel=1e-12)
        assert r.max_prob == pytest.approx(1.0 / V, rel=1e-12)
        assert r.argmax == 0 and r.kept_count == V


# ----------------------------------------------------------------------------- filter


def _kept_by_definition(l, k, top_p, T):
    """Independent characterisation of R1: x survives top-k iff fewer than k logits are strictly
    larger; x survives top-p iff the top-k-renormalised mass strictly above l_x is < top_p."""
    V = len(l)
    keep = np.ones(V, dtype=bool)
    if 0 < k < V:
        keep = np.array([(l > l[x]).sum() < k for x in range(V)])
    if top_p < 1.0:
        e = np.where(keep, np.exp((l - l.max()) / T), 0.0)
        pi = e / e.sum()
        keep = keep & np.array([pi[l > l[x]].sum() < top_p for x in range(V)])
    return keep


def test_filter_brute_force_small():
    """Brute force over every tie pattern of small integer-valued rows (V <= 5)."""
    T = 0.8
    for V in range(1, 6):
        for vals in itertools.product([0.0, 1.0, 2.5], repeat=V):
            l = np.array(vals)
            for k in range(0, V + 1):
                for top_p in [0.05, 0.3, 0.5, 0.7, 0.9, 1.0]:
                    r = O.row_distribution(l, O.SamplingParams(T, k, top_p))
                    keep = _kept_by_definition(l, k, top_p, T)
                    assert np.array_equal(r.probs > 0, keep), (vals, k, top_p)
                    assert r.kept_count == keep.sum()
                    e = np.where(keep, np.exp((l - l.max()) / T), 0.0)
                    np.testing.assert_allclose(r.probs, e / e.sum(), rtol=1e-12)


def test_filter_special_cases():
    """top_k = 1 without ties is one-hot; top_k >= V and top_p >= 1 are no-ops; ties kept."""
    rng = np.random.default_rng(5)
    l = rng.normal(0, 3, 1000)
    r = O.row_distribution(l, O.SamplingParams(0.7, 1, 1.0))
    assert r.kept_count == 1 and r.probs[np.argmax(l)] == 1.0 and r.entropy_bits == 0.0
    base = O.row_distribution(l, O.SamplingParams(0.7))
    for sp in [O.SamplingParams(0.7, 1000, 1.0), O.SamplingParams(0.7, 5000, 1.0),
               O.SamplingParams(0.7, 0, 1.0), O.SamplingParams(0.7, -3, 1.5)]:
        np.testing.assert_array_equal(O.row_distribution(l, sp).probs, base.probs)
    lt = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 0.0])
    r = O.row_distribution(lt, O.SamplingParams(1.0, 2, 1.0))  # k-th largest is 3.0, three copies
    assert r.kept_count == 3 and np.array_equal(r.probs > 0, lt == 3.0)


def test_masked_logits():
    """-inf logits are masked: they get probability 0 and do not count as kept."""
    l = np.array([1.0, -np.inf, 0.5, -np.inf])
    r = O.row_distribution(l, O.SamplingParams(1.0))
    assert r.probs[1] == 0 and r.probs[3] == 0 and r.kept_count == 2
    np.testing.assert_allclose(r.probs[[0, 2]], scipy.special.softmax([1.0, 0.5]))


def test_nonfinite_rows():
    """R8: NaN, +inf or all -inf make the row non-finite and the request NONFINITE."""
    for bad in [np.array([0.0, np.nan, 1.0]), np.array([0.0, np.inf, 1.0]), np.full(3, -np.inf)]:
        assert not O.row_distribution(bad, O.SamplingParams(1.0)).finite
        good = np.zeros((2, 3))
        res = O.verify_request(np.stack([good[0], bad]), good[:1], [1], O.SamplingParams(1.0), 0, 0, 0)
        assert res.status & O.STATUS_NONFINITE and res.num_accepted == 0 and res.tokens == []


# ----------------------------------------------------------------------------- sampler


def test_sampler_levels_pick_the_mass():
    """Each level of R6 decides where the mass is: one element; two elements in different
    chunks (u1 decides); same chunk, different groups (u2 decides); same group (u3 decides)."""
    V = 3 * O.CHUNK + 100
    w = np.zeros(V)
    w[9000] = 2.0
    for u in [(0.0, 0.0, 0.0), (0.999, 0.5, 0.3), (0.3, 0.999, 0.999)]:
        assert O.sample_three_level(w, *u)[0] == 9000
    w = np.zeros(V)
    w[5] = 1.0
    w[3 * O.CHUNK + 50] = 3.0
    assert O.sample_three_level(w, 0.2, 0.9, 0.9)[0] == 5
    assert O.sample_three_level(w, 0.3, 0.0, 0.0)[0] == 3 * O.CHUNK + 50
    w = np.zeros(V)
    w[O.CHUNK + 3] = 1.0
    w[O.CHUNK + 200] = 1.0
    assert O.sample_three_level(w, 0.7, 0.49, 0.9)[0] == O.CHUNK + 3
    assert O.sample_three_level(w, 0.1, 0.51, 0.0)[0] == O.CHUNK + 200
    w = np.zeros(V)
    w[130] = 1.0
    w[140] = 3.0
    assert O.sample_three_level(w, 0.5, 0.5, 0.24)[0] == 130
    assert O.sample_three_level(w, 0.5, 0.5, 0.26)[0] == 140


def test_sampler_exact_law_small_grid():
    """V <= 64 (one group): sweeping u3 over a midpoint grid reproduces w/W to 1/n."""
    rng = np.random.default_rng(11)
    for V in [1, 3, 8, 64]:
        w = rng.random(V) * (rng.random(V) > 0.3)
        if w.sum() == 0:
            w[0] = 1.0
        n = 4000
        counts = np.zeros(V)
        for u3 in (np.arange(n) + 0.5) / n:
            counts[O.sample_three_level(w, 0.37, 0.61, u3)[0]] += 1
        np.testing.assert_allclose(counts / n, w / w.sum(), atol=1.0 / n + 1e-12)


def test_sampler_exact_law_multichunk():
    """Across chunks and groups, level by level: sweeping one uniform over a midpoint grid while
    the others are held gives the conditional law of that level (S_k/W, then M_kg/S_k, then
    w_x/M_kg) to 1/n; their product is w/W.  Reading R6."""
    V = 2 * O.CHUNK + 70
    w = np.zeros(V)
    idx = [3, 70, 130, O.CHUNK + 1, O.CHUNK + 4000, 2 * O.CHUNK + 69]
    w[idx] = [1.0, 2.0, 0.5, 3.0, 1.5, 2.0]
    W = w.sum()
    n = 600
    grid = (np.arange(n) + 0.5) / n
    chunk_of = lambda x: x // O.CHUNK
    group_of = lambda x: (x % O.CHUNK) // O.GROUP
    # level 1: chunk frequencies
    c1 = np.zeros(3)
    for u1 in grid:
        c1[chunk_of(O.sample_three_level(w, u1, 0.5, 0.5)[0])] += 1.0 / n
    S = np.array([w[k * O.CHUNK:(k + 1) * O.CHUNK].sum() for k in range(3)])
    np.testing.assert_allclose(c1, S / W, atol=1.0 / n)
    # level 2 inside each chunk (u1 chosen at the middle of that chunk's interval)
    cum = np.concatenate(([0.0], np.cumsum(S))) / W
    for k in range(3):
        u1 = 0.5 * (cum[k] + cum[k + 1])
        groups = {}
        for u2 in grid:
            x = O.sample_three_level(w, u1, u2, 0.5)[0]
            assert chunk_of(x) == k
            groups[group_of(x)] = groups.get(group_of(x), 0) + 1.0 / n
        for gidx, f in groups.items():
            lo = k * O.CHUNK + gidx * O.GROUP
            assert f == pytest.approx(w[lo:lo + O.GROUP].sum() / S[k], abs=1.0 / n)
    # level 3 inside the one group that holds two elements (3 and 70 are in groups 0 and 1;
    # 70 and 130 are in groups 1 and 2): use a row with two elements in one group
    w2 = np.zeros(V)
    w2[O.CHUNK + 10] = 1.0
    w2[O.CHUNK + 20] = 3.0
    c3 = {}
    for u3 in grid:
        x = O.sample_three_level(w2, 0.9, 0.3, u3)[0]
        c3[x] = c3.get(x, 0) + 1.0 / n
    assert c3[O.CHUNK + 10] == pytest.approx(0.25, abs=1.0 / n)
    assert c3[O.CHUNK + 20] == pytest.approx(0.75, abs=1.0 / n)


def test_sampler_chi2_random_uniforms():
    """Statistical: 8k draws with PCG64 uniforms over a 2-chunk random w follow w/W."""
    rng = np.random.default_rng(12)
    V = O.CHUNK + 500
    w = np.zeros(V)
    support = rng.choice(V, 12, replace=False)
    w[support] = rng.random(12) + 0.1
    n = 8000
    counts = np.zeros(V)
    for _ in range(n):
        counts[O.sample_three_level(w, *rng.random(3))[0]] += 1
    assert counts[w == 0].sum() == 0
    exp = w[support] / w.sum() * n
    chi2 = ((counts[support] - exp) ** 2 / exp).sum()
    assert scipy.stats.chi2.sf(chi2, len(support) - 1) > 1e-3


# ----------------------------------------------------------------------------- verify rules


def test_draft_equal_target_always_accepts():
    """[SD] §4.2: if p = q the rejection path is never taken, for every seed."""
    rng = np.random.default_rng(2)
    tl = rng.normal(0, 3, (5, 300))
    for seed in range(20):
        ys = [int(rng.integers(300)) for _ in range(4)]
        res = O.verify_request(tl, tl[:4], ys, O.SamplingParams(0.9), seed, 3, 0)
        assert res.num_accepted == 4 and res.tokens[:4] == ys and res.status == 0
        np.testing.assert_allclose(res.one_minus_tv, 1.0, atol=1e-12)


def test_greedy_emits_target_argmax_sequence():
    """[SD] §3.1: greedy output equals the target's own argmax decoding of the round."""
    rng = np.random.default_rng(4)
    V = 50
    for trial in range(30):
        tl = rng.normal(0, 3, (5, V))
        amax = [int(np.argmax(r)) for r in tl]
        ys = [a if rng.random() < 0.6 else int((a + 1 + rng.integers(V - 1)) % V) for a in amax[:4]]
        res = O.verify_request(tl, None, ys, O.SamplingParams(0.0), trial, 0, 0)
        n = 0
        while n < 4 and ys[n] == amax[n]:
            n += 1
        assert res.num_accepted == n
        assert res.tokens == amax[:n + 1]


def test_stochastic_rule_with_onehot_target_is_greedy():
    """Special case: a one-hot p (all other logits -inf) and a token-only draft make the
    stochastic rule reduce to the greedy rule."""
    rng = np.random.default_rng(6)
    V = 20
    for trial in range(30):
        hot = rng.integers(V, size=5)
        tl = np.full((5, V), -np.inf)
        tl[np.arange(5), hot] = 0.0
        ys = [int(h) if rng.random() < 0.7 else int((h + 3) % V) for h in hot[:4]]
        r1 = O.verify_request(tl, None, ys, O.SamplingParams(1.0), trial, 1, 2)
        r0 = O.verify_request(tl, None, ys, O.SamplingParams(0.0), trial, 1, 2)
        assert (r1.num_accepted, r1.tokens) == (r0.num_accepted, r0.tokens)


def test_first_rejection_stops_and_uses_that_position():
    """[SD] §5.1: position j's residual is used, later drafts are discarded; the correction
    token is drawn with the uniforms of (b, j)."""
    p = np.array([0.6, 0.3, 0.1])
    q = np.array([0.2, 0.5, 0.3])
    tl = np.log(np.stack([p, p, p]))
    dl = np.log(np.stack([q, q]))
    us = {1: (0.99, 0.1, 0.1, 0.1), 2: (0.0, 0.9, 0.9, 0.9), 3: (0.0, 0.5, 0.5, 0.5)}
    res = O.verify_request(tl, dl, [1, 1], O.SamplingParams(1.0), 0, 0, 0, uniforms=us)
    assert res.num_accepted == 0 and res.tokens == [0]   # residual at position 1 is all on token 0
    us = {1: (0.1, 0.1, 0.1, 0.1), 2: (0.99, 0.9, 0.9, 0.9), 3: (0.0, 0.5, 0.5, 0.5)}
    res = O.verify_request(tl, dl, [1, 1], O.SamplingParams(1.0), 0, 0, 0, uniforms=us)
    assert res.num_accepted == 1 and res.tokens == [1, 0]
    us = {1: (0.1, 0.0, 0.0, 0.0), 2: (0.1, 0.0, 0.0, 0.0), 3: (0.0, 0.0, 0.0, 0.95)}
    res = O.verify_request(tl, dl, [0, 0], O.SamplingParams(1.0), 0, 0, 0, uniforms=us)
    assert res.num_accepted == 2 and res.tokens == [0, 0, 2]  # bonus from p_3 with u3 = 0.95


def test_accept_threshold_is_strict():
    """R4: u equal to the acceptance ratio rejects; the next double below accepts."""
    p = np.array([0.5, 0.5])
    q = np.array([0.25, 0.75])
    tl = np.log(np.stack([p, p]))
    dl = np.log(q)[None]
    probe = O.verify_request(tl, dl, [1], O.SamplingParams(1.0), 0, 0, 0)
    a = min(1.0, probe.p_y[0] / probe.q_y[0])
    assert a == pytest.approx(2.0 / 3.0, rel=1e-12)
    for u0, acc in [(a, 0), (np.nextafter(a, 0), 1)]:
        us = {1: (u0, 0.5, 0.5, 0.5), 2: (0.0, 0.5, 0.5, 0.5)}
        res = O.verify_request(tl, dl, [1], O.SamplingParams(1.0), 0, 0, 0, uniforms=us)
        assert res.num_accepted == acc


def test_error_statuses():
    """R8: bad token, q(y) = 0 and an empty residual set their bits and reject."""
    V = 6
    tl = np.zeros((2, V))
    dl = np.zeros((1, V))
    res = O.verify_request(tl, dl, [V + 3], O.SamplingParams(1.0), 0, 0, 0)
    assert res.status == O.STATUS_BAD_TOKEN | O.STATUS_RESIDUAL_EMPTY and res.num_accepted == 0
    assert np.isnan(res.p_y[0])
    dl2 = np.array([[0.0, -np.inf, 0.0, 0.0, 0.0, 0.0]])
    res = O.verify_request(tl, dl2, [1], O.SamplingParams(1.0), 0, 0, 0)
    assert res.status == O.STATUS_ZERO_Q and res.num_accepted == 0
    assert res.tokens == [1]   # all residual mass sits on token 1
    res = O.verify_request(tl, None, [-1], O.SamplingParams(0.0), 0, 0, 0)
    assert res.status == O.STATUS_BAD_TOKEN and res.tokens == [0]


def test_aggregates():
    """[SKV]: mean entropy, mean confidence, max entropy, min confidence over the block."""
    rng = np.random.default_rng(8)
    tl = rng.normal(0, 2, (5, 40))
    dl = rng.normal(0, 2, (4, 40))
    res = O.verify_request(tl, dl, [1, 2, 3, 4], O.SamplingParams(1.0), 0, 0, 0)
    H = [O.row_distribution(r, O.SamplingParams(1.0)).entropy_bits for r in dl]
    C = [scipy.special.softmax(r).max() for r in dl]
    np.testing.assert_allclose(res.draft_entropy_bits, H, rtol=1e-12)
    np.testing.assert_allclose(res.draft_max_prob, C, rtol=1e-12)
    np.testing.assert_allclose(res.req_stats, [np.mean(H), np.mean(C), np.max(H), np.min(C)], rtol=1e-12)


def test_gamma_zero_is_plain_sampling():
    rng = np.random.default_rng(9)
    tl = rng.normal(0, 1, (1, 30))
    res = O.verify_request(tl, np.zeros((0, 30)), [], O.SamplingParams(1.0), 4, 5, 6)
    u = O.position_uniforms(4, 5, 6, 1)
    x, _ = O.sample_three_level(scipy.special.softmax(tl[0]), *u[1:])
    assert res.num_accepted == 0 and res.tokens == [x] and np.isnan(res.req_stats).all()


# ----------------------------------------------------------------------------- chi-square


def _chi2_trials(rule, n, seed=77):
    """gamma = 4, V = 8 fp32 rows as in the tiny workload; y_i ~ q_i drawn with PCG64, one
    Philox counter per trial (b = trial).  Returns per-position emitted-token counts."""
    rng = np.random.default_rng(seed)
    V, g = 8, 4
    tl = rng.normal(0, 2, (g + 1, V)).astype(np.float32).astype(np.float64)
    dl = rng.normal(0, 2, (g, V)).astype(np.float32).astype(np.float64)
    sp = O.SamplingParams(1.0)
    P = [scipy.special.softmax(r) for r in tl]
    Qd = [scipy.special.softmax(r) for r in dl]
    counts = np.zeros((g + 1, V))
    for t in range(n):
        ys = [int(rng.choice(V, p=Qd[i])) for i in range(g)]
        res = O.verify_request(tl, dl, ys, sp, 2024, 1, t, resample_rule=rule)
        for k, tok in enumerate(res.tokens):
            counts[k, tok] += 1
    return counts, P


def _chi2_pvalues(counts, P):
    pv = []
    for k in range(counts.shape[0]):
        n = counts[k].sum()
        if n < 200:
            continue
        exp = P[k] * n
        mask = exp > 5
        c = counts[k][mask]
        e = exp[mask]
        e = e * c.sum() / e.sum()
        pv.append(scipy.stats.chisquare(c, e).pvalue)
    return pv


def test_chi2_standard_rule_lossless():
    """[SD] §4-§5 (and the page's Monte-Carlo check): conditioned on reaching position k, the
    emitted token follows p_k.  alpha = 1e-3 per position."""
    counts, P = _chi2_trials("residual", 6000)
    pv = _chi2_pvalues(counts, P)
    assert len(pv) >= 2
    assert min(pv) > 1e-3, pv


def test_chi2_wrong_rule_rejected():
    """Negative control: the same test rejects the wrong rule of [SD] §7."""
    counts, P = _chi2_trials("p", 6000)
    pv = _chi2_pvalues(counts, P)
    assert min(pv) < 1e-3, pv


# ----------------------------------------------------------------------------- extra signals (R10)


def test_extra_signals_worked_example():
    """Worked example p = [0.6, 0.3, 0.1], q = [0.2, 0.5, 0.3]: both KL divergences in closed
    form, L1 = 2 TV = 0.8, a(y) = min(1, p(y) / q(y)) = [1, 0.6, 1/3], and the expected committed
    length averaged over y ~ q: 1 + sum_y q(y) a(y) = 1 + sum min(p, q) = 1.6."""
    p = np.array([0.6, 0.3, 0.1])
    q = np.array([0.2, 0.5, 0.3])
    kl_pq = 0.6 * math.log(3.0) + 0.3 * math.log(0.6) + 0.1 * math.log(1.0 / 3.0)
    kl_qp = 0.2 * math.log(1.0 / 3.0) + 0.5 * math.log(5.0 / 3.0) + 0.3 * math.log(3.0)
    E = 0.0
    for y in range(3):
        r = O.verify_request(np.log(np.stack([p, p])), np.log(q)[None], [y], O.SamplingParams(1.0), 1, 1, 0)
        assert abs(r.kl_pq[0] - kl_pq) < 1e-12 and abs(r.kl_qp[0] - kl_qp) < 1e-12
        assert abs(r.l1[0] - 0.8) < 1e-12
        assert abs(r.accept_prob[0] - [1.0, 0.6, 1.0 / 3.0][y]) < 1e-12
        E += q[y] * r.expected_committed
    assert abs(E - 1.6) < 1e-12


def test_expected_committed_is_the_chain_sum():
    """Two-token rows with y = 0 give a_i = min(1, p_i(0) / q_i(0)) in closed form; E is
    1 + a1 + a1 a2 + a1 a2 a3.  A token outside [0, V) has a = 0 and ends the chain."""
    pp, qq = [0.3, 0.9, 0.5, 0.7], [0.6, 0.45, 0.8]
    tl = np.log(np.array([[x, 1.0 - x] for x in pp]))
    dl = np.log(np.array([[z, 1.0 - z] for z in qq]))
    a = [min(1.0, pp[i] / qq[i]) for i in range(3)]
    r = O.verify_request(tl, dl, [0, 0, 0], O.SamplingParams(1.0), 3, 5, 0)
    assert np.allclose(r.accept_prob, a, rtol=0, atol=1e-12)
    assert abs(r.expected_committed - (1 + a[0] + a[0] * a[1] + a[0] * a[1] * a[2])) < 1e-12
    r = O.verify_request(tl, dl, [0, 7, 0], O.SamplingParams(1.0), 3, 5, 0)
    assert r.accept_prob[1] == 0.0 and abs(r.expected_committed - (1 + a[0])) < 1e-12


def test_kl_invariants_and_support():
    """Gibbs: KL >= 0 with equality for p = q.  Pinsker: TV <= sqrt(KL / 2).  KL = +inf in each
    direction whose second distribution misses part of the first one's (filtered) support."""
    rng = np.random.default_rng(17)
    for _ in range(20):
        tl = rng.normal(0, 2, (2, 40))
        dl = tl[:1] + rng.normal(0, 1, (1, 40))
        r = O.verify_request(tl, dl, [3], O.SamplingParams(0.8), 1, 1, 0)
        assert r.kl_pq[0] >= 0 and r.kl_qp[0] >= 0
        tv = r.l1[0] / 2
        assert tv <= math.sqrt(r.kl_pq[0] / 2) + 1e-12 and tv <= math.sqrt(r.kl_qp[0] / 2) + 1e-12
        assert abs(tv - r.tv[0]) < 1e-12
    same = O.verify_request(np.stack([tl[0], tl[0]]), tl[:1], [3], O.SamplingParams(0.8), 1, 1, 0)
    assert abs(same.kl_pq[0]) < 1e-12 and abs(same.kl_qp[0]) < 1e-12 and abs(same.l1[0]) < 1e-12
    # top-k 3 on both rows, the draft's top 3 differing from the target's: p is not covered by q
    t = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.0])
    d = np.array([5.0, 4.0, 0.0, 3.0, 1.0, 0.0])
    r = O.verify_request(np.stack([t, t]), d[None], [0], O.SamplingParams(1.0, 3, 1.0), 1, 1, 0)
    assert r.kl_pq[0] == math.inf and r.kl_qp[0] == math.inf
    r = O.verify_request(np.stack([t, t]), t[None] + 0.5, [0], O.SamplingParams(1.0, 3, 1.0), 1, 1, 0)
    assert abs(r.kl_pq[0]) < 1e-12 and abs(r.kl_qp[0]) < 1e-12   # a shifted row: the same distribution


def test_extra_signals_token_only_and_greedy():
    """A token-only draft is one-hot at y: KL(q || p) = -ln p(y), KL(p || q) = +inf, L1 =
    2 (1 - p(y)), a = p(y).  Greedy: both KL values NaN, a = 1 iff y is the argmax."""
    p = np.array([0.6, 0.3, 0.1])
    r = O.verify_request(np.log(np.stack([p, p])), None, [1], O.SamplingParams(1.0), 1, 1, 0)
    assert abs(r.kl_qp[0] + math.log(0.3)) < 1e-12 and r.kl_pq[0] == math.inf
    assert abs(r.l1[0] - 1.4) < 1e-12 and abs(r.accept_prob[0] - 0.3) < 1e-12
    g = O.verify_request(np.log(np.stack([p, p])), None, [0], O.SamplingParams(0.0), 1, 1, 0)
    assert math.isnan(g.kl_pq[0]) and math.isnan(g.kl_qp[0]) and g.accept_prob[0] == 1.0 and g.l1[0] == 0.0
    g = O.verify_request(np.log(np.stack([p, p])), None, [2], O.SamplingParams(0.0), 1, 1, 0)
    assert g.accept_prob[0] == 0.0 and g.l1[0] == 2.0 and g.expected_committed == 1.0


# ----------------------------------------------------------------------------- gamma selection (R11)


def _gamma_head(alpha, beta):
    """Weights making f(x, gamma) = alpha - beta * gamma exactly (one ReLU unit passes gamma
    through, another carries a constant 1; the rest are dead), so E(gamma) = (alpha - beta
    gamma) gamma + 1 peaks at gamma = alpha / (2 beta)."""
    w1 = np.zeros((16, 6))
    b1 = np.zeros(16)
    w1[0, 5] = 1.0            # h0 = relu(gamma) = gamma
    b1[1] = 1.0               # h1 = 1
    b1[2:] = -1.0             # dead units
    w2 = np.zeros(16)
    w2[0] = -beta
    w2[1] = alpha
    return w1, b1, w2, 0.0


def test_gamma_selection_closed_form():
    """E(gamma) = (alpha - beta gamma) gamma + 1: the argmax over {2, 4, 6, 8} follows the
    parabola's vertex alpha / (2 beta); ties go to the smaller gamma; NaN features give -1."""
    stats = [3.0, 0.4, 5.0, 0.1]
    for alpha, beta, want in [(0.8, 0.1, 4), (0.9, 0.05, 8), (0.5, 0.2, 2), (1.2, 0.1, 6)]:
        g, E, margin = O.select_gamma(stats, 1.0, *_gamma_head(alpha, beta))
        assert g == want, (alpha, beta, E)
        for k, gamma in enumerate(O.GAMMAS):
            assert abs(E[k] - ((alpha - beta * gamma) * gamma + 1.0)) < 1e-12
    # vertex at 5 with binary-exact weights: E(4) = E(6) = 4 exactly -> the smaller gamma
    g, E, margin = O.select_gamma(stats, 0.0, *_gamma_head(1.25, 0.125))
    assert g == 4 and margin == 0.0
    g, E, _ = O.select_gamma([float("nan"), 0.4, 5.0, 0.1], 0.0, *_gamma_head(0.8, 0.1))
    assert g == -1 and np.isnan(E).all()


def test_gamma_selection_uses_the_features():
    """A unit reading c_min only: f = w * relu(c_min) and E = f gamma + 1 grows with gamma when
    f > 0 (gamma* = 8) and shrinks when f < 0 (gamma* = 2)."""
    w1 = np.zeros((16, 6)); w1[0, 3] = 1.0
    b1 = np.zeros(16)
    for sign, want in [(1.0, 8), (-1.0, 2)]:
        w2 = np.zeros(16); w2[0] = sign
        g, E, _ = O.select_gamma([3.0, 0.4, 5.0, 0.25], 1.0, w1, b1, w2, 0.0)
        assert g == want and abs(E[0] - (sign * 0.25 * 2 + 1.0)) < 1e-12


# ----------------------------------------------------------------------------- fused LM head (R12)


def test_lm_head_logits_brute_force():
    """A tiny case summed by hand in Python loops: l[r][v] = sum_d h[r][d] W[v][d] (not W^T h,
    not h W with V and D swapped)."""
    rng = np.random.default_rng(4)
    h = rng.integers(-3, 4, size=(2, 3)).astype(float)
    W = rng.integers(-3, 4, size=(5, 3)).astype(float)
    l = O.lm_head_logits(h, W)
    assert l.shape == (2, 5)
    for r in range(2):
        for v in range(5):
            assert l[r, v] == sum(h[r, d] * W[v, d] for d in range(3))


def test_lm_head_selector_weights_give_hidden_components():
    """A head whose row v is the unit vector of component perm[v] returns l[r, v] = h[r, perm[v]];
    its statistics are row_stats of those values (R12 composes with R2, R3)."""
    rng = np.random.default_rng(5)
    D, V = 16, 40
    perm = rng.integers(0, D, size=V)
    W = np.zeros((V, D))
    W[np.arange(V), perm] = 1.0
    h = rng.standard_normal((3, D))
    sp = O.SamplingParams(0.8)
    got = O.lm_head_row_stats(h, W, sp, tokens=np.array([0, 39, 7]))
    ref = O.row_stats(h[:, perm], sp)
    for k in ("max_logit", "argmax", "log_z", "entropy_bits", "max_prob"):
        np.testing.assert_array_equal(got[k], ref[k])


def test_lm_head_p_tok_closed_form_and_edges():
    """p_tok = exp(l_y / T - log Z); NaN for a token outside [0, V) and for a non-finite row."""
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, 8))
    W = rng.standard_normal((30, 8))
    sp = O.SamplingParams(1.3)
    tok = np.array([3, -1, 30, 29])
    got = O.lm_head_row_stats(h, W, sp, tokens=tok)
    l = h @ W.T
    for r, y in ((0, 3), (3, 29)):
        want = math.exp(l[r, y] / 1.3 - got["log_z"][r])
        assert abs(got["p_tok"][r] - want) <= 1e-12 * want
    assert np.isnan(got["p_tok"][1]) and np.isnan(got["p_tok"][2])
    h2 = h.copy()
    h2[0, 0] = np.inf
    bad = O.lm_head_row_stats(h2, W, sp, tokens=tok)
    assert np.isnan(bad["p_tok"][0]) and bad["argmax"][0] == -1
    greedy = O.lm_head_row_stats(h, W, O.SamplingParams(0.0), tokens=tok)
    assert greedy["p_tok"][0] == (1.0 if np.argmax(l[0]) == 3 else 0.0)


# ----------------------------------------------------------------------------- decision margins
#
# The margins decide which GPU/oracle mismatches are excused, so each is pinned on a row whose
# distance from its boundary is known in closed form, one case just inside 1e-6 and one just
# outside.


def test_accept_margin_is_distance_from_ratio():
    """R4 accept test: the recorded margin is |u0 - a| at that position.  p = [1/2, 1/2],
    q = [1/4, 3/4], y = 1 gives a = 2/3; u0 = 2/3 - 5e-7 accepts with margin 5e-7, u0 = 2/3 +
    3e-6 rejects with margin 3e-6."""
    p = np.array([0.5, 0.5])
    q = np.array([0.25, 0.75])
    tl = np.log(np.stack([p, p, p]))
    dl = np.log(np.stack([q, q]))
    sp = O.SamplingParams(1.0)
    for d, acc in [(-5e-7, 1), (3e-6, 0)]:
        us = {1: (2.0 / 3.0 + d, 0.5, 0.5, 0.5), 2: (0.99, 0.5, 0.5, 0.5), 3: (0.5, 0.5, 0.5, 0.5)}
        res = O.verify_request(tl, dl, [1, 1], sp, 0, 0, 0, uniforms=us)
        acc_dec = [x for x in res.decisions if x.kind == "accept"]
        assert acc_dec[0].position == 1
        assert acc_dec[0].margin == pytest.approx(abs(d), rel=1e-6)
        assert (res.num_accepted >= 1) == bool(acc)
        if acc:   # position 2 is tested too: u0 = 0.99 against a = 2/3
            assert acc_dec[1].position == 2
            assert acc_dec[1].margin == pytest.approx(0.99 - 2.0 / 3.0, rel=1e-9)
            assert res.num_accepted == 1
        else:
            assert len(acc_dec) == 1 and res.num_accepted == 0


def test_sampler_margin_level3():
    """R6, element level: w = [1, 1, 1, 1] (one chunk, one group).  u3 = 1/2 + 1e-7 puts
    u3 W = 2 + 4e-7 just past the prefix sum 2: token 2, margin 4e-7 / 4 = 1e-7; the other two
    levels sit at u = 1/2 (margin 1/2)."""
    x, m = O.sample_three_level(np.ones(4), 0.5, 0.5, 0.5 + 1e-7)
    assert x == 2 and m == pytest.approx(1e-7, rel=1e-6)
    x, m = O.sample_three_level(np.ones(4), 0.5, 0.5, 0.5 - 3e-6)
    assert x == 1 and m == pytest.approx(3e-6, rel=1e-6)


def test_sampler_margin_level1():
    """R6, chunk level: w = 1 on two full chunks (S = [4096, 4096]).  u1 = 1/2 - 2e-7 stays in
    chunk 0 at distance 2e-7 W from the boundary.  Inside it u2 = 0.3 picks group 19 (u2 S =
    1228.8 between 1216 and 1280: margin 12.8 / 4096) and u3 = 0.51 element 32 (32.64 between
    32 and 33: margin 0.36 / 64); the chunk level's 2e-7 is the smallest."""
    w = np.ones(2 * O.CHUNK)
    x, m = O.sample_three_level(w, 0.5 - 2e-7, 0.3, 0.51)
    assert x == 19 * O.GROUP + 32
    assert m == pytest.approx(2e-7, rel=1e-6)
    x, m = O.sample_three_level(w, 0.5 + 2e-6, 0.3, 0.51)
    assert x == O.CHUNK + 19 * O.GROUP + 32 and m == pytest.approx(2e-6, rel=1e-6)
    _, m = O.sample_three_level(w, 0.25, 0.3, 0.51)   # chunk margin 0.25, group 12.8 / 4096
    assert m == pytest.approx(12.8 / 4096, rel=1e-9)


def test_sampler_margin_level2():
    """R6, group level: one chunk of ones; u2 = 1/2 + 3e-6 lands 3e-6 S past the prefix sum
    2048 of the first 32 groups: group 32, margin 3e-6 (u3 = 0.76 picks element 48 at margin
    0.36 / 64)."""
    w = np.ones(O.CHUNK)
    x, m = O.sample_three_level(w, 0.5, 0.5 + 3e-6, 0.76)
    assert x == 32 * O.GROUP + 48 and m == pytest.approx(3e-6, rel=1e-6)
    x, m = O.sample_three_level(w, 0.5, 0.5 - 4e-7, 0.76)
    assert x == 31 * O.GROUP + 48 and m == pytest.approx(4e-7, rel=1e-6)


def test_topp_margin_is_distance_of_both_neighbouring_groups():
    """R1 top-p boundary: p = [1/2, 3/10, 1/5].  top_p = 0.8 - 4e-7 is reached by the second
    group (cumulative 0.8): two tokens kept, margin min(|0.8 - top_p|, |0.5 - top_p|) = 4e-7.
    top_p = 0.8 + 2e-6 needs the third group: three kept, margin |0.8 - top_p| = 2e-6.  top_p =
    0.3 is reached by the first group alone: margin |0.5 - 0.3| (no group before it)."""
    l = np.log(np.array([0.5, 0.3, 0.2]))
    for tp, kept, margin in [(0.8 - 4e-7, 2, 4e-7), (0.8 + 2e-6, 3, 2e-6), (0.3, 1, 0.2)]:
        r = O.row_distribution(l, O.SamplingParams(1.0, 0, tp))
        assert r.kept_count == kept
        assert r.topp_margin == pytest.approx(margin, rel=1e-6)
    assert O.row_distribution(l, O.SamplingParams(1.0)).topp_margin == math.inf


def test_topp_decisions_name_their_row():
    """Each filtered row's top-p decision carries the row kind and its 1-based position, so a
    comparison can tell which position a near-boundary row decides."""
    rng = np.random.default_rng(3)
    tl = rng.normal(0, 1, (3, 50))
    dl = rng.normal(0, 1, (2, 50))
    res = O.verify_request(tl, dl, [1, 2], O.SamplingParams(1.0, 0, 0.7), 1, 2, 3)
    got = sorted((d.row, d.position) for d in res.decisions if d.kind == "topp")
    assert got == [("draft", 1), ("draft", 2), ("target", 1), ("target", 2), ("target", 3)]
    for d in res.decisions:
        if d.kind == "topp":
            src = tl[d.position - 1] if d.row == "target" else dl[d.position - 1]
            assert d.margin == O.row_distribution(src, O.SamplingParams(1.0, 0, 0.7)).topp_margin


def test_accept_prob_of_a_nonfinite_row_is_nan():
    """R8 / R10: a position whose draft row holds a NaN has no distribution, so its accept
    probability is NaN while the other positions keep theirs (p = [1/2, 1/2], q = [1/4, 3/4],
    y = 1: a = 2/3); the request is NONFINITE and its expected committed length NaN."""
    p = np.array([0.5, 0.5])
    q = np.array([0.25, 0.75])
    tl = np.log(np.stack([p, p, p]))
    dl = np.log(np.stack([q, q]))
    dl[1, 0] = np.nan
    res = O.verify_request(tl, dl, [1, 1], O.SamplingParams(1.0), 0, 0, 0)
    assert res.accept_prob[0] == pytest.approx(2.0 / 3.0, rel=1e-12)
    assert np.isnan(res.accept_prob[1])
    assert res.status == O.STATUS_NONFINITE and res.num_accepted == 0 and res.tokens == []
    assert np.isnan(res.expected_committed)


def test_verify_batch_ragged_layout():
    """The batch layout of spec_verify_batch: request b's target rows start at cu[b] + b, its
    draft rows and tokens at cu[b].  Greedy rows with a known argmax (row i of request b peaks
    at token 3b + i) and drafts that match up to a chosen position give outputs fixed by
    construction."""
    V = 16
    gammas = [2, 0, 3]
    cu = [0, 2, 2, 5]
    target = np.zeros((5 + 3, V))
    ys = np.zeros(5, dtype=np.int64)
    agree = {0: 1, 1: 0, 2: 3}   # drafts of request b match the target argmax up to here
    for b, g in enumerate(gammas):
        for i in range(g + 1):
            target[cu[b] + b + i, 3 * b + i] = 5.0
        for i in range(g):
            ys[cu[b] + i] = 3 * b + i if i < agree[b] else (3 * b + i + 7) % V
    out = O.verify_batch(target, None, ys, cu, O.SamplingParams(0.0), 1, 2)
    assert sorted(out) == [0, 1, 2]
    assert (out[0].num_accepted, out[0].tokens) == (1, [0, 1])
    assert (out[1].num_accepted, out[1].tokens) == (0, [3])
    assert (out[2].num_accepted, out[2].tokens) == (3, [6, 7, 8, 9])
    assert sorted(O.verify_batch(target, None, ys, cu, O.SamplingParams(0.0), 1, 2, requests=[2])) == [2]
