"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Sizes span several 4096-logit slices and a ragged tail so every code path (vector and scalar
loads, partial chunks, ragged draft lengths) is exercised, while the oracle still finishes in
seconds.  The comparison rule is in tests/harness.py.
"""
import math
import os
import sys

import numpy as np
import pytest
import scipy.stats

torch = pytest.importorskip("torch")

import lossless_draft_verification_row_amd as L
from lossless_draft_verification_row_amd import workloads as W
from oracle import spec_oracle as O
import harness as H

pytestmark = pytest.mark.gpu

DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    L.load_library()


def custom_inputs(B, V, gammas, dtype="bf16", sigma=3.0, tau=1.0, T=1.0, seed=7, token_only=False,
                  tokens="gumbel"):
    wl = W.Workload("custom", B, V, 0, dtype, sigma, tau, T, token_only=token_only)
    rng = np.random.default_rng(seed)
    gammas = np.asarray(gammas, dtype=np.int32)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(gammas)
    Rd = int(cu[-1])
    t32 = rng.standard_normal((Rd + B, V), dtype=np.float32) * np.float32(sigma)
    d32 = np.empty((Rd, V), dtype=np.float32)
    for b in range(B):
        g = int(gammas[b])
        t0 = int(cu[b]) + b
        d32[cu[b]:cu[b] + g] = t32[t0:t0 + g] + rng.standard_normal((g, V), dtype=np.float32) * np.float32(tau)
    if dtype == "bf16":
        target, draft = W.bf16_bits_from_f32(t32), W.bf16_bits_from_f32(d32)
        dv = W.bf16_bits_to_f32(draft)
    else:
        target, draft = t32, d32
        dv = d32
    toks = W.gumbel_argmax(dv, T, rng) if (Rd and tokens == "gumbel") else np.zeros(Rd, np.int32)
    return W.Inputs(wl, gammas, cu, target, None if token_only else draft, toks.astype(np.int32), seed)


def path_options(path):
    """Call options selecting the single-kernel (fused) or the multi-kernel path."""
    return L.call_options(path="multi" if path == "multi" else "auto")


def run_gpu(inp, sp, seed, step, gamma_max=None, path="fused", kl=False):
    d = H.to_device(inp)
    G = int(inp.gammas.max()) if gamma_max is None else gamma_max
    res = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], G,
                              temperature=sp.temperature, top_k=sp.top_k, top_p=sp.top_p, seed=seed, step=step,
                              kl=kl, options=path_options(path))
    torch.cuda.synchronize()
    return H.gpu_to_numpy(res)


def check(inp, sp, seed=1234, step=5, requests=None, gamma_max=None, path="fused", kl=False):
    note(f"case B={len(inp.gammas)} V={inp.target.shape[1]} dtype={inp.wl.dtype} T={sp.temperature} "
         f"k={sp.top_k} p={sp.top_p} token_only={inp.draft is None} path={path}")
    gpu = run_gpu(inp, sp, seed, step, gamma_max, path, kl)
    reqs = range(len(inp.gammas)) if requests is None else requests
    refs = H.oracle_requests(inp, sp, seed, step, reqs)
    rep = H.compare_requests(gpu, refs, inp, H.Report())
    note(repr(rep))
    assert rep.ok(), rep
    return gpu, refs, rep


# ----------------------------------------------------------------------------- dense sampling


PATHS = ["fused", "multi"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V", [4096 * 3 + 72, 8192, 4097, 1000])
def test_dense_bf16_ragged(V, path):
    inp = custom_inputs(7, V, [0, 1, 3, 5, 2, 7, 4], T=1.0, seed=V)
    check(inp, O.SamplingParams(1.0), path=path)


def test_ragged_batch_of_many_requests():
    """A ragged batch of 600 requests (drafts 0..8 each): the streaming kernel finds each draft
    row's request among the 601 offsets in three rounds of 256; every request against the
    oracle."""
    rng = np.random.default_rng(600)
    gammas = rng.integers(0, 9, 600).tolist()
    inp = custom_inputs(600, 2 * 4096 + 40, gammas, T=1.0, seed=601)
    check(inp, O.SamplingParams(1.0))


@pytest.mark.parametrize("path", PATHS)
def test_dense_bf16_temperature(path):
    inp = custom_inputs(6, 3 * 4096 + 300, [2, 4, 6, 8, 1, 3], tau=1.5, T=0.7, seed=3)
    check(inp, O.SamplingParams(0.7), path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V", [8, 3000, 4096 * 2 + 5])
def test_dense_fp32(V, path):
    inp = custom_inputs(5, V, [4, 0, 2, 3, 1], dtype="f32", sigma=2.0, tau=1.0, T=1.3, seed=V + 1)
    check(inp, O.SamplingParams(1.3), path=path)


@pytest.mark.parametrize("path", PATHS)
def test_unaligned_rows_take_the_scalar_path(path):
    """bf16 rows with an odd stride (not a 16-byte multiple): same results as the oracle."""
    inp = custom_inputs(4, 4099, [3, 2, 0, 4], seed=11)
    check(inp, O.SamplingParams(1.0), path=path)


def test_worked_example_v3():
    """The page's example as logits ln p / ln q (V = 3, gamma = 1), many requests."""
    p = np.array([0.6, 0.3, 0.1])
    q = np.array([0.2, 0.5, 0.3])
    B = 2000
    rng = np.random.default_rng(5)
    t = np.tile(np.log(np.stack([p, p])).astype(np.float32), (B, 1))
    d = np.tile(np.log(q).astype(np.float32)[None], (B, 1))
    toks = rng.choice(3, size=B, p=q).astype(np.int32)
    wl = W.Workload("v3", B, 3, 1, "f32", 1.0, None, 1.0)
    gam = np.ones(B, dtype=np.int32)
    cu = np.arange(B + 1, dtype=np.int32)
    inp = W.Inputs(wl, gam, cu, t, d, toks, 0)
    gpu, refs, rep = check(inp, O.SamplingParams(1.0), seed=42, step=0)
    np.testing.assert_allclose(gpu["one_minus_tv"], 0.6, rtol=1e-6)
    first = gpu["tokens"][:, 0]
    acc = gpu["num_accepted"] == 1
    # rejected draws always land on token 0 (residual [1, 0, 0])
    assert np.all(first[~acc] == 0)
    # acceptance frequency: sum_y q(y) min(1, p(y) / q(y)) = sum min(p, q) = 0.6 (guide §4.3);
    # 2000 Bernoulli draws, 4 standard deviations
    freq = acc.mean()
    note(f"acceptance frequency {freq:.4f}")
    assert abs(freq - 0.6) < 4 * math.sqrt(0.6 * 0.4 / B)
    # the first emitted token (accepted draft or correction) follows p (guide §4.2, §7)
    cnt = np.bincount(first, minlength=3).astype(float)
    pval = scipy.stats.chisquare(cnt, p * B).pvalue
    note(f"first-token counts {cnt.tolist()} vs p * B {(p * B).tolist()}: chi2 p = {pval:.3g}")
    assert pval > 1e-3


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V", [3 * 4096 + 72, 151936])
def test_low_overlap_one_minus_tv(path, V):
    """Nearly disjoint p and q (overlap near 7e-4 at the small vocabulary, 7e-3 at the full
    one): the target puts its mass on tokens 0..99, the draft on tokens 100..199.
    1 - TV = sum min(p, q) must keep 1e-5 relative precision with no absolute floor (guide
    §4.3: A = sum min(p, q) = 1 - TV).  The full vocabulary takes the fp64 recomputation over
    several groups of runs per thread."""
    inp = custom_inputs(4, V, [3, 2, 1, 3], sigma=0.5, tau=0.5, seed=77)
    t32 = W.bf16_bits_to_f32(inp.target).copy()
    d32 = W.bf16_bits_to_f32(inp.draft).copy()
    t32[:, :100] += 12.0
    d32[:, 100:200] += 12.0
    inp.target[:] = W.bf16_bits_from_f32(t32)
    inp.draft[:] = W.bf16_bits_from_f32(d32)
    sp = O.SamplingParams(1.0)
    gpu, refs, rep = check(inp, sp, path=path)
    for b, ref in refs.items():
        c0, g = int(inp.cu_draft[b]), int(inp.gammas[b])
        got = gpu["one_minus_tv"][c0:c0 + g].astype(np.float64)
        assert (ref.one_minus_tv < 1e-2).all(), ref.one_minus_tv
        rel = np.abs(got - ref.one_minus_tv) / ref.one_minus_tv
        note(f"request {b}: 1 - TV {ref.one_minus_tv.tolist()} relative error {rel.max():.2e}")
        assert (rel < 1e-5).all()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V", [3 * 4096 + 72, 151936])
def test_near_identical_rows_small_tv(path, V):
    """Draft rows equal to the target rows except for a few hundred tokens: TV of a few 1e-3,
    the case where the residual mass sum [p - q]_+ is a small difference of nearly equal
    distributions (its error then comes from the normalisers' ratio)."""
    inp = custom_inputs(5, V, [4, 3, 2, 4, 1], T=0.7, seed=78)
    rng = np.random.default_rng(79)
    for b in range(5):
        g, c0 = int(inp.gammas[b]), int(inp.cu_draft[b])
        inp.draft[c0:c0 + g] = inp.target[c0 + b:c0 + b + g]
        d32 = W.bf16_bits_to_f32(inp.draft[c0:c0 + g]).copy()
        idx = rng.choice(V, size=(g, 300))
        for i in range(g):
            d32[i, idx[i]] += rng.normal(0, 1.0, 300).astype(np.float32)
        inp.draft[c0:c0 + g] = W.bf16_bits_from_f32(d32)
    gpu, refs, rep = check(inp, O.SamplingParams(0.7), path=path)
    tv = np.concatenate([r.tv for r in refs.values()])
    note(f"TV range {tv.min():.2e} .. {tv.max():.2e}; max relative error of L1 {rep.max_rel.get('l1')}")
    assert np.median(tv) < 0.01


@pytest.mark.parametrize("path", PATHS)
def test_masked_leading_slice_entropy(path):
    """Rows whose first 8192 logits are -inf (a caller's masked vocabulary block): a streaming
    ticket's first slice then holds no finite logit while its second does, and the entropy
    numerator the ticket files with its first slice must still count.  Target and draft
    entropies, max-probabilities and 1 - TV against the oracle."""
    V = 3 * 4096 + 72
    inp = custom_inputs(4, V, [3, 3, 3, 3], T=0.8, seed=83)
    for arr in (inp.target, inp.draft):
        f = W.bf16_bits_to_f32(arr).copy()
        f[1::2, :8192] = -np.inf
        arr[:] = W.bf16_bits_from_f32(f)
    rng = np.random.default_rng(84)
    dv = W.bf16_bits_to_f32(inp.draft).astype(np.float64)
    for r in range(inp.draft.shape[0]):
        q = O.row_distribution(dv[r], O.SamplingParams(0.8)).probs
        inp.tokens[r] = int(rng.choice(V, p=q / q.sum()))
    check(inp, O.SamplingParams(0.8), path=path)


def test_near_identical_rows_one_minus_tv_without_l1():
    """The benchmark's outputs (1 - TV but no L1) on near-identical rows: 1 - TV = 1 - beta is
    then close to 1 and precise from the streaming sums, so the finalize recomputes nothing;
    the value still meets the relative bar against the oracle."""
    V = 151936
    inp = custom_inputs(4, V, [4, 3, 2, 4], T=0.7, seed=81)
    rng = np.random.default_rng(82)
    for b in range(4):
        g, c0 = int(inp.gammas[b]), int(inp.cu_draft[b])
        d32 = W.bf16_bits_to_f32(inp.target[c0 + b:c0 + b + g]).copy()
        idx = rng.choice(V, size=(g, 300))
        for i in range(g):
            d32[i, idx[i]] += rng.normal(0, 1.0, 300).astype(np.float32)
        inp.draft[c0:c0 + g] = W.bf16_bits_from_f32(d32)
    d = H.to_device(inp)
    B, G, Rd = 4, int(inp.gammas.max()), int(inp.cu_draft[-1])
    out = {"tokens": torch.empty((B, G + 1), dtype=torch.int32, device=DEV),
           "num_accepted": torch.empty(B, dtype=torch.int32, device=DEV),
           "status": torch.empty(B, dtype=torch.int32, device=DEV),
           "one_minus_tv": torch.empty(Rd, dtype=torch.float32, device=DEV)}
    L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], G, temperature=0.7, seed=3, step=1, out=out)
    torch.cuda.synchronize()
    got = out["one_minus_tv"].cpu().numpy().astype(np.float64)
    refs = H.oracle_requests(inp, O.SamplingParams(0.7), 3, 1, range(B))
    tv = np.concatenate([r.tv for r in refs.values()])
    assert (tv < 0.02).sum() >= len(tv) // 2, tv
    for b, ref in refs.items():
        c0, g = int(inp.cu_draft[b]), int(inp.gammas[b])
        rel = np.abs(got[c0:c0 + g] - ref.one_minus_tv) / ref.one_minus_tv
        assert (rel < 1e-5).all(), (b, rel)


# ----------------------------------------------------------------------------- greedy / token-only


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V", [4096 * 3 + 72, 4096 + 77, 1000])
def test_greedy(V, path):
    inp = custom_inputs(9, V, [7, 7, 0, 3, 7, 1, 7, 5, 2], T=0.0, seed=V + 2, token_only=True)
    # make about half of the draft tokens the target argmax so long accepted prefixes occur
    tv = W.bf16_bits_to_f32(inp.target)
    rng = np.random.default_rng(1)
    for b in range(len(inp.gammas)):
        for i in range(int(inp.gammas[b])):
            if rng.random() < 0.7:
                inp.tokens[inp.cu_draft[b] + i] = int(np.argmax(tv[inp.cu_draft[b] + b + i]))
    gpu, refs, rep = check(inp, O.SamplingParams(0.0), path=path)
    assert gpu["num_accepted"].max() >= 3


@pytest.mark.parametrize("path", PATHS)
def test_token_only_stochastic(path):
    inp = custom_inputs(6, 2 * 4096 + 11, [1, 3, 0, 5, 2, 4], T=1.0, seed=21, token_only=True)
    rng = np.random.default_rng(2)
    tv = W.bf16_bits_to_f32(inp.target)
    for b in range(6):
        for i in range(int(inp.gammas[b])):
            inp.tokens[inp.cu_draft[b] + i] = int(np.argmax(tv[inp.cu_draft[b] + b + i] + rng.gumbel(size=tv.shape[1])))
    check(inp, O.SamplingParams(1.0), path=path)


# ----------------------------------------------------------------------------- edge cases


def test_draft_equals_target_always_accepts():
    inp = custom_inputs(5, 5000, [3, 4, 1, 2, 6], seed=9)
    for b in range(5):
        g = int(inp.gammas[b])
        c0 = int(inp.cu_draft[b])
        inp.draft[c0:c0 + g] = inp.target[c0 + b:c0 + b + g]
    gpu, _, _ = check(inp, O.SamplingParams(0.8))
    np.testing.assert_array_equal(gpu["num_accepted"], inp.gammas)
    np.testing.assert_allclose(gpu["one_minus_tv"], 1.0, atol=2e-6)


@pytest.mark.parametrize("path", PATHS)
def test_error_statuses_on_gpu(path):
    """NaN / +inf rows, -inf masked logits, out-of-range tokens, q(y) = 0, gamma 0."""
    inp = custom_inputs(8, 4096 + 100, [2, 2, 2, 2, 2, 0, 3, 2], seed=13)
    bf = lambda x: int(W.bf16_bits_from_f32(np.array([x], np.float32))[0])
    cu = inp.cu_draft
    inp.target[cu[0] + 0 + 1, 50] = bf(np.nan)               # request 0: NaN in a target row
    inp.draft[cu[1] + 0, 4000] = bf(np.inf)                  # request 1: +inf in a draft row
    inp.tokens[cu[2] + 0] = 4096 + 100                       # request 2: token out of range
    y = int(inp.tokens[cu[3] + 0])
    inp.draft[cu[3] + 0, y] = bf(-np.inf)                    # request 3: q(y) = 0
    inp.target[cu[4] + 4 + 0, :300] = bf(-np.inf)            # request 4: masked logits
    inp.draft[cu[4] + 0, 100:200] = bf(-np.inf)
    inp.tokens[cu[6] + 1] = -5                               # request 6: negative token
    gpu, refs, _ = check(inp, O.SamplingParams(1.0), path=path)
    assert gpu["status"][0] & L.STATUS["NONFINITE"] and gpu["status"][1] & L.STATUS["NONFINITE"]
    assert gpu["status"][2] & L.STATUS["BAD_TOKEN"] and gpu["status"][3] & L.STATUS["ZERO_Q"]
    assert gpu["num_accepted"][5] == 0 and gpu["tokens"][5, 0] >= 0


@pytest.mark.parametrize("path", PATHS)
def test_bad_offsets_are_reported_not_read(path):
    """Offsets that are not an exclusive prefix: every request reports BAD_GAMMA, none is read."""
    inp = custom_inputs(3, 2000, [2, 3, 1], seed=17)
    d = H.to_device(inp)
    for cu_bad in ([0, 2, 9, 6], [1, 3, 6, 7], [0, 2, 5, 5]):   # gamma > max, cu[0] != 0, cu[B] != rows
        cu = torch.tensor(cu_bad, dtype=torch.int32, device=DEV)
        res = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], cu, 3, temperature=1.0, seed=1,
                                  options=path_options(path))
        torch.cuda.synchronize()
        st = res["status"].cpu().numpy()
        assert (st == L.STATUS["BAD_GAMMA"]).all(), (cu_bad, st)
        assert (res["tokens"].cpu().numpy() == -1).all()
        assert (res["num_accepted"].cpu().numpy() == 0).all()
    # a valid call right after still verifies correctly (the counters were left clean)
    check(inp, O.SamplingParams(1.0), path=path)


def test_forced_timeout_then_clean_call():
    """A zero wait bound (a per-call option) forces the team wait to give up: the affected
    requests report TIMEOUT with no tokens, the others still match the oracle, and the next
    call, with the default bound, is exact again."""
    inp = custom_inputs(6, 6 * 4096 + 10, [5, 4, 3, 5, 2, 6], seed=29)
    sp = O.SamplingParams(1.0)
    d = H.to_device(inp)
    res = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], int(inp.gammas.max()),
                              temperature=1.0, seed=5, step=6, options=L.call_options(spin_limit=0))
    torch.cuda.synchronize()
    gpu = H.gpu_to_numpy(res)
    refs = H.oracle_requests(inp, sp, 5, 6, range(6))
    timed = (gpu["status"] & L.STATUS["TIMEOUT"]) != 0
    note(f"timed-out requests: {np.nonzero(timed)[0].tolist()}")
    assert (gpu["tokens"][timed] == -1).all() and (gpu["num_accepted"][timed] == 0).all()
    keep = {b: refs[b] for b in range(6) if not timed[b]}
    rep = H.compare_requests(gpu, keep, inp, H.Report(), stats=False)
    assert rep.ok(), rep
    check(inp, sp, seed=5, step=6)


def test_co_running_kernel_changes_nothing():
    """A team's members wait only for one another, dispatched side by side on one XCD.  With
    another kernel streaming on a second stream at the same time (its workgroups taking CU slots
    and memory bandwidth among the teams'), every wait still ends: no request reports TIMEOUT and
    every output is bit-equal to the same call run alone."""
    inp = custom_inputs(48, 16 * 4096 + 77, [7] * 48, seed=41)
    sp = O.SamplingParams(1.0)
    solo = run_gpu(inp, sp, 21, 4)
    assert (solo["status"] == 0).all()
    d = H.to_device(inp)
    buf = torch.empty(512 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    for rep in range(3):
        note(f"co-running call {rep}")
        torch.cuda.synchronize()
        L.spec_stream_read(buf, sink, stream=side)
        res = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], 7, temperature=1.0, seed=21,
                                  step=4)
        L.spec_stream_read(buf, sink, stream=side)
        torch.cuda.synchronize()
        got = H.gpu_to_numpy(res)
        assert ((got["status"] & L.STATUS["TIMEOUT"]) == 0).all()
        for k in solo:
            assert np.array_equal(got[k], solo[k], equal_nan=True), k


def test_repeated_calls_identical():
    """Back-to-back calls on one workspace give bitwise equal outputs (counters reset)."""
    inp = custom_inputs(5, 3 * 4096 + 8, [7, 7, 7, 7, 7], seed=37)
    sp = O.SamplingParams(1.0)
    outs = [run_gpu(inp, sp, 9, 9) for _ in range(3)]
    for o in outs[1:]:
        for k in o:
            assert np.array_equal(o[k], outs[0][k], equal_nan=True), k


def test_all_equal_logits():
    inp = custom_inputs(3, 4096 + 9, [2, 1, 3], seed=19)
    inp.target[:] = W.bf16_bits_from_f32(np.full(inp.target.shape, 0.5, np.float32))
    inp.draft[:] = W.bf16_bits_from_f32(np.full(inp.draft.shape, 0.5, np.float32))
    gpu, _, _ = check(inp, O.SamplingParams(1.0))
    np.testing.assert_allclose(gpu["draft_entropy_bits"], math.log2(4096 + 9), rtol=1e-6)


def test_deterministic_and_seeded():
    inp = custom_inputs(6, 3 * 4096 + 1, [5, 5, 5, 5, 5, 5], seed=23)
    sp = O.SamplingParams(1.0)
    a = run_gpu(inp, sp, 99, 3)
    b = run_gpu(inp, sp, 99, 3)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    c = run_gpu(inp, sp, 100, 3)
    assert not np.array_equal(a["tokens"], c["tokens"]) or not np.array_equal(a["num_accepted"], c["num_accepted"])


# ----------------------------------------------------------------------------- row stats / residual


@pytest.mark.parametrize("dtype,V,T", [("bf16", 3 * 4096 + 72, 1.0), ("bf16", 4096 + 77, 1.0), ("bf16", 5000, 0.7), ("f32", 1000, 1.5),
                                       ("bf16", 4096 + 3, 0.0)])
def test_row_stats(dtype, V, T):
    rng = np.random.default_rng(V)
    x = rng.standard_normal((12, V), dtype=np.float32) * 3
    x[3, :10] = -np.inf
    if dtype == "bf16":
        bits = W.bf16_bits_from_f32(x)
        t = torch.from_numpy(bits).view(torch.bfloat16).to(DEV)
        xf = W.bf16_bits_to_f32(bits).astype(np.float64)
    else:
        t = torch.from_numpy(x).to(DEV)
        xf = x.astype(np.float64)
    res = L.spec_row_stats(t, temperature=T)
    torch.cuda.synchronize()
    g = H.gpu_to_numpy(res)
    ref = O.row_stats(xf, O.SamplingParams(T))
    assert np.array_equal(g["argmax"], ref["argmax"])
    assert np.array_equal(g["kept_count"], ref["kept_count"])
    for k in ("max_logit", "log_z", "entropy_bits", "max_prob"):
        assert H.close(g[k], ref[k]), (k, H.max_rel(g[k], ref[k]))


@pytest.mark.parametrize("with_q", [True, False])
def test_residual_sample_grid(with_q):
    """Injected uniforms on a grid: every draw matches the oracle's three-level sampler."""
    V = 2 * 4096 + 500
    rng = np.random.default_rng(31)
    p = rng.standard_normal(V).astype(np.float32) * 3
    q = p + rng.standard_normal(V).astype(np.float32)
    n = 400
    grid = (np.arange(n) + 0.5) / n
    U = np.stack([grid, rng.permutation(grid), rng.permutation(grid)], axis=1)
    P = np.tile(W.bf16_bits_from_f32(p), (n, 1))
    Q = np.tile(W.bf16_bits_from_f32(q), (n, 1))
    pt = torch.from_numpy(P).view(torch.bfloat16).to(DEV)
    qt = torch.from_numpy(Q).view(torch.bfloat16).to(DEV) if with_q else None
    res = L.spec_residual_sample(pt, qt, temperature=1.0, uniforms=torch.from_numpy(U).to(DEV))
    torch.cuda.synchronize()
    g = H.gpu_to_numpy(res)
    pf = W.bf16_bits_to_f32(P[:1]).astype(np.float64)
    qf = W.bf16_bits_to_f32(Q[:1]).astype(np.float64) if with_q else None
    ref = O.residual_sample(np.repeat(pf, n, 0), None if qf is None else np.repeat(qf, n, 0),
                            O.SamplingParams(1.0), uniforms=U)
    bad = (g["token"] != ref["token"]) & (ref["margin"] >= H.DECISION_EPS)
    assert not bad.any(), np.nonzero(bad)
    assert (g["token"] != ref["token"]).sum() <= 1
    assert H.close(g["mass"], ref["mass"])


def test_residual_sample_philox():
    V = 4096 + 17
    rng = np.random.default_rng(33)
    R = 64
    p = rng.standard_normal((R, V)).astype(np.float32) * 2
    q = p + rng.standard_normal((R, V)).astype(np.float32)
    res = L.spec_residual_sample(torch.from_numpy(p).to(DEV), torch.from_numpy(q).to(DEV), temperature=0.9,
                                 seed=77, step=4)
    torch.cuda.synchronize()
    g = H.gpu_to_numpy(res)
    ref = O.residual_sample(p.astype(np.float64), q.astype(np.float64), O.SamplingParams(0.9), seed=77, step=4)
    bad = (g["token"] != ref["token"]) & (ref["margin"] >= H.DECISION_EPS)
    assert not bad.any()
    assert H.close(g["mass"], ref["mass"])


# ----------------------------------------------------------------------------- chi-square


def test_chi2_lossless_on_gpu():
    """Tiny workload (V = 8, gamma = 4, fp32): 10^5 replicated requests, one Philox counter per
    request.  Conditioned on reaching position k, the emitted token follows p_k (alpha 1e-3)."""
    n = 100_000
    rng = np.random.default_rng(1001)
    V, g = 8, 4
    tl = (rng.standard_normal((g + 1, V)) * 2).astype(np.float32)
    dl = (rng.standard_normal((g, V)) * 2).astype(np.float32)
    sp = O.SamplingParams(1.0)
    P = [O.row_distribution(r.astype(np.float64), sp).probs for r in tl]
    Qd = [O.row_distribution(r.astype(np.float64), sp).probs for r in dl]
    toks = np.stack([rng.choice(V, size=n, p=Qd[i]) for i in range(g)], axis=1).astype(np.int32)
    target = torch.from_numpy(np.tile(tl, (n, 1))).to(DEV)
    draft = torch.from_numpy(np.tile(dl, (n, 1))).to(DEV)
    cu = torch.arange(0, g * (n + 1), g, dtype=torch.int32, device=DEV)
    res = L.spec_verify_batch(target, draft, torch.from_numpy(toks.reshape(-1)).to(DEV), cu, g,
                              temperature=1.0, seed=2024, step=1, pos_stats=False, req_stats=False)
    torch.cuda.synchronize()
    out = res["tokens"].cpu().numpy()
    nacc = res["num_accepted"].cpu().numpy()
    assert (res["status"].cpu().numpy() == 0).all()
    pvals = []
    for k in range(g + 1):
        reached = nacc >= k
        emitted = out[reached, k]
        cnt = np.bincount(emitted, minlength=V).astype(float)
        exp = P[k] * reached.sum()
        mask = exp > 5
        e = exp[mask] * cnt[mask].sum() / exp[mask].sum()
        pvals.append(scipy.stats.chisquare(cnt[mask], e).pvalue)
    note(f"chi2 p-values per position: {pvals}")
    assert min(pvals) > 1e-3


# ----------------------------------------------------------------------------- full-size workloads


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_workload_sampled(cfg):
    """The full workload in the launch configuration the benchmark times; the oracle checks a
    sample of requests one by one."""
    inp = W.make_inputs(cfg)
    wl = inp.wl
    sp = O.SamplingParams(wl.temperature, wl.top_k, wl.top_p)
    B = len(inp.gammas)
    reqs = sorted(set([0, 1, B // 2, B - 1]))
    gpu, refs, rep = check(inp, sp, seed=1000 + cfg, step=0, requests=reqs,
                           gamma_max=int(inp.gammas.max()))
    assert (gpu["status"] == 0).all()


# ----------------------------------------------------------------------------- extra signals


@pytest.mark.parametrize("dtype,V,T", [("bf16", 3 * 4096 + 72, 1.0), ("f32", 2 * 4096 + 5, 0.7)])
def test_kl_and_signals(dtype, V, T):
    """Both KL divergences (nats), L1, accept probabilities and the expected committed length
    against the oracle; a KL request runs the multi-kernel path."""
    inp = custom_inputs(5, V, [3, 0, 7, 1, 4], T=T, seed=V + 1, dtype=dtype)
    gpu, refs, _ = check(inp, O.SamplingParams(T), kl=True)
    assert np.isfinite(gpu["kl_pq"]).all() and (gpu["kl_pq"] > 0).all()


def test_kl_token_only_and_greedy():
    inp = custom_inputs(4, 5000, [2, 5, 0, 3], T=1.0, seed=9, token_only=True)
    gpu, _, _ = check(inp, O.SamplingParams(1.0), kl=True)
    assert np.isinf(gpu["kl_pq"]).all()
    inp = custom_inputs(3, 5000, [2, 5, 3], T=0.0, seed=10, token_only=True)
    gpu, _, _ = check(inp, O.SamplingParams(0.0), kl=True)
    assert np.isnan(gpu["kl_pq"]).all() and np.isnan(gpu["kl_qp"]).all()


def test_kl_draft_equals_target_is_zero():
    inp = custom_inputs(2, 4096 + 100, [4, 3], T=1.0, seed=12)
    for b in range(2):
        c0, g = int(inp.cu_draft[b]), int(inp.gammas[b])
        inp.draft[c0:c0 + g] = inp.target[c0 + b:c0 + b + g]
    gpu, _, _ = check(inp, O.SamplingParams(1.0), kl=True)
    assert (gpu["kl_pq"] == 0).all() and (gpu["kl_qp"] == 0).all()
    assert np.allclose(gpu["expected_committed"], 1 + inp.gammas)


# ----------------------------------------------------------------------------- draft-length selection


def test_select_gamma_random_weights():
    """Random MLP-16 weights against the oracle's fp64 MLP on the request statistics of a
    verification call (plus made-up rows and a NaN row): gamma* exact unless the oracle's best
    and runner-up expectations lie within fp32 rounding, expectations to an fp32 dot-product
    rounding bound (relative error is no measure here: E(2) can cancel to near zero)."""
    inp = custom_inputs(6, 5000, [3, 0, 7, 1, 4, 2], T=0.8, seed=21)
    gpu = run_gpu(inp, O.SamplingParams(0.8), 5, 6)
    rng = np.random.default_rng(99)
    extra = np.array([[4.0, 0.3, 6.0, 0.05], [1.0, 0.8, 1.5, 0.6], [9.5, 0.05, 11.0, 0.01]], dtype=np.float32)
    stats = np.concatenate([gpu["req_stats"], extra]).astype(np.float32)
    B = stats.shape[0]
    comp = rng.choice([0.0, 1.0, 2.0], size=B).astype(np.float32)
    for trial in range(5):
        w1 = (rng.standard_normal((16, 6)) * 0.5).astype(np.float32)
        b1 = (rng.standard_normal(16) * 0.5).astype(np.float32)
        w2 = (rng.standard_normal(16) * 0.3).astype(np.float32)
        b2 = float(np.float32(rng.standard_normal() * 0.2))
        dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        res = L.spec_select_gamma(dv(stats), dv(w1), dv(b1), dv(w2), b2, comp=dv(comp))
        torch.cuda.synchronize()
        g = res["gamma"].cpu().numpy()
        E = res["expected"].cpu().numpy()
        for b in range(B):
            want, Eref, margin = O.select_gamma(stats[b].astype(np.float64), float(comp[b]), w1, b1, w2, b2)
            if want == -1:
                assert g[b] == -1 and np.isnan(E[b]).all(), (b, g[b])
                continue
            # fp32 evaluation: a dot product of n terms is off by at most about n * 2^-24 times
            # the sum of its terms' magnitudes; 32 * 2^-24 covers the 7-term hidden sums and the
            # 16-term output sum, scaled by the magnitudes that feed each E(gamma).
            x = np.array([*stats[b], comp[b], 0.0])
            tol = []
            for gam in O.GAMMAS:
                x[5] = gam
                hid = np.abs(w1.astype(np.float64)) @ np.abs(x) + np.abs(b1)
                tol.append(32 * 2.0 ** -24 * (gam * (np.abs(w2) @ hid + abs(b2)) + 1))
            tol = np.array(tol)
            assert np.all(np.abs(E[b] - Eref) <= tol), (b, E[b], Eref, tol)
            if margin > 2 * tol.max():
                assert g[b] == want, (trial, b, g[b], want, Eref)
    assert (gpu["req_stats"][1] != gpu["req_stats"][1]).all()   # request 1 has no draft: NaN row
