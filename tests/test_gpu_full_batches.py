"""Whole full-size batches against the oracle: every request of each workload, in the launch
configuration the benchmark times, with the oracle spread over the host's cores.

The comparison rule is in tests/harness.py: counts and tokens bit-exact unless the deciding
decision lies within 1e-6 of its boundary, such excused mismatches below 1e-4 of all draws,
statistics within 1e-5 relative.  Each test prints its draws, excused and hard mismatches.
Basis: the guide page "5.1 投机解码核心原理" §8 (a lossless verifier must reproduce the target
distribution, checked by convergence and greedy-consistency tests) and §3.2 (the accept test).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import lossless_draft_verification_row_amd as L
from lossless_draft_verification_row_amd import workloads as W
from oracle import spec_oracle as O
import harness as H
import oracle_pool as P

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


def _run(d, inp, sp, G, seed, step, out=None):
    res = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], G, temperature=sp.temperature,
                              top_k=sp.top_k, top_p=sp.top_p, seed=seed, step=step, out=out)
    torch.cuda.synchronize()
    return H.gpu_to_numpy(res)


def _whole_batch(inp, sp, keys, label):
    """GPU and oracle over every request for each (seed, step) in keys; returns the report."""
    d = H.to_device(inp)
    G = int(inp.gammas.max())
    note(f"{label}: B={len(inp.gammas)} V={inp.target.shape[1]} T={sp.temperature} k={sp.top_k} "
         f"p={sp.top_p} keys={len(keys)}; oracle over {P.n_workers()} workers")
    gpus = {k: _run(d, inp, sp, G, *k) for k in keys}
    refs = P.verify_requests(inp, sp, keys)
    rep = H.Report()
    for k in keys:
        H.compare_requests(gpus[k], refs[k], inp, rep)
        st = gpus[k]["status"]
        assert not (st & (L.STATUS["NONFINITE"] | L.STATUS["TIMEOUT"] | L.STATUS["FILTER_OVERFLOW"])).any(), st
    note(f"{label}: draws={rep.draws} excused={rep.excused} hard={len(rep.hard)} "
         f"excused_stat_positions={rep.excused_stats} max_rel={rep.max_rel}")
    return rep


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_batch_every_request(cfg):
    """Configs 2 (B=64, gamma=7, V=151,936, T=1), 3 (B=128, gamma in {2,4,6,8}, V=128,256,
    T=0.7) and 4 (greedy, B=256, token-only): every request."""
    inp = W.make_inputs(cfg)
    wl = inp.wl
    sp = O.SamplingParams(wl.temperature, wl.top_k, wl.top_p)
    rep = _whole_batch(inp, sp, [(1000 + cfg, 0)], f"config {cfg}")
    assert rep.ok(), rep


def _filtered_batch(sp, token_seed):
    inp = W.make_inputs(5, tokens="none")
    return P.filtered_draft_tokens(inp, sp, token_seed)


def test_full_batch_filtered_every_request():
    """Config 5 (B=256, gamma=7, V=151,936, T=0.7, top-k 50 then top-p 0.9): every request, the
    draft tokens drawn from each filtered draft row."""
    wl = W.WORKLOADS[5]
    sp = O.SamplingParams(wl.temperature, wl.top_k, wl.top_p)
    rep = _whole_batch(_filtered_batch(sp, 55), sp, [(99, 3)], "config 5")
    assert rep.ok(), rep


def test_full_batch_top_p_only_every_request():
    """The filtered workload's shape with top-p 0.9 alone (a uniform bf16 batch: per-row
    thresholds, then the fused streaming kernel with the logits below them masked): every
    request."""
    wl = W.WORKLOADS[5]
    sp = O.SamplingParams(wl.temperature, 0, wl.top_p)
    rep = _whole_batch(_filtered_batch(sp, 56), sp, [(98, 5)], "config 5, top-p only")
    assert rep.ok(), rep


def test_excused_rate_over_many_full_vocabulary_draws():
    """Config 2 (V = 151,936) over 60 (seed, step) keys: at least 10^4 accept and sample draws
    compared one by one; no hard mismatch and excused mismatches below 1e-4 of the draws."""
    inp = W.make_inputs(2)
    sp = O.SamplingParams(inp.wl.temperature)
    keys = [(7000 + s, s % 5) for s in range(60)]
    rep = _whole_batch(inp, sp, keys, "config 2, 60 keys")
    assert rep.draws >= 10_000, rep.draws
    assert not rep.hard, rep.hard[:3]
    assert rep.excused < 1e-4 * rep.draws, (rep.excused, rep.draws)
    assert rep.ok(), rep
