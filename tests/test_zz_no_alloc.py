"""spec_verify_batch_noalloc (the entry point for callers that cannot allocate) against
spec_verify_batch with its own workspace, through the C ABI: two calls in a row, the second with a
smaller input, give the same outputs bit for bit; a call larger than the static scratch is refused
before any launch."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import lossless_draft_verification_row_amd as L
from lossless_draft_verification_row_amd import workloads as W
import harness as H

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(B, G, Rd, dev):
    o = {"tokens": torch.full((B, G + 1), -7, dtype=torch.int32, device=dev),
         "num_accepted": torch.full((B,), -7, dtype=torch.int32, device=dev),
         "status": torch.full((B,), -7, dtype=torch.int32, device=dev),
         "req_stats": torch.full((B, 4), -7.0, dtype=torch.float32, device=dev),
         "expected_committed": torch.full((B,), -7.0, dtype=torch.float32, device=dev)}
    for k in ("p_y", "q_y", "one_minus_tv", "draft_entropy_bits", "draft_max_prob", "l1", "accept_prob"):
        o[k] = torch.full((Rd,), -7.0, dtype=torch.float32, device=dev)
    for k in ("target_entropy_bits", "target_max_prob"):
        o[k] = torch.full((Rd + B,), -7.0, dtype=torch.float32, device=dev)
    return o


def _same(a, b):
    for k in a:
        x, y = a[k].cpu().numpy(), b[k].cpu().numpy()
        assert np.array_equal(x, y, equal_nan=True), k


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    dev = "cuda"
    cases = [("batch-64 workload: B=64, gamma=7, V=151,936, T=1", W.make_inputs(2), 1.0, 0, 1.0),
             ("smaller: B=5, ragged gamma, V=12,360, T=0.7, top-k 20", W.make_inputs(3, B=5, V=3 * 4096 + 72, seed=9),
              0.7, 20, 0.9)]
    # the smaller case's draft tokens: each draft row's largest logit, inside its top-k set
    small = cases[1][1]
    small.tokens[:] = W.bf16_bits_to_f32(small.draft).argmax(axis=1).astype(np.int32)
    for label, inp, T, k, p in cases:
        note(f"case {label}")
        d = H.to_device(inp)
        B = len(inp.gammas)
        G = int(inp.gammas.max())
        Rd = int(inp.cu_draft[-1])
        ref = L.spec_verify_batch(d["target"], d["draft"], d["tokens"], d["cu"], G, temperature=T, top_k=k, top_p=p,
                                  seed=31, step=4, out=_outputs(B, G, Rd, dev))
        got = L.spec_verify_batch_noalloc(d["target"], d["draft"], d["tokens"], d["cu"], G, temperature=T, top_k=k,
                                          top_p=p, seed=31, step=4, out=_outputs(B, G, Rd, dev))
        torch.cuda.synchronize()
        _same(ref, got)
        note(f"  num_accepted {got['num_accepted'].cpu().numpy()[:8].tolist()} status sum "
             f"{int(got['status'].sum())}: identical")


def test_noalloc_refuses_a_call_beyond_the_scratch():
    lib = L.load_library()
    sp = L.SamplingParams(0.7, 50, 0.9)
    need = lib.spec_verify_workspace_bytes(256, 151936, 7, L.SPEC_BF16, sp)
    assert need > (32 << 20)
    ps = L.PosStats()
    # refused before any pointer is read or any kernel launched
    rc = lib.spec_verify_batch_noalloc(256, 151936, 7, L.SPEC_BF16, 16, 151936, 16, 151936, 16, 16, 1792, sp,
                                       0, 0, 16, 16, ps, None, 16, None)
    assert rc == -5
    assert "no-allocation" in L.spec_status_string(-5)
