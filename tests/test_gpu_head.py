"""GPU parity of the fused LM head (spec_lm_head_row_stats) against the fp64 oracle.

Two regimes.  With values from {-1, -1/2, 0, 1/2, 1} every partial sum is exact in fp32, so the
GPU's logits equal the oracle's and the statistics meet the usual bar.  With normal values the
GPU's fp32 accumulation may move a logit by up to delta_v = D 2^-24 sum_d |h_d W_{v,d}| (the
standard bound for a sum of D terms); the tolerances below follow from delta = max_v delta_v:
the maximum moves by at most delta, log Z (natural) by at most delta / T, every probability by
a factor within exp(+-2 delta / T), the entropy in bits by at most 2 delta / (T ln 2) per unit
of probability mass (so 2 delta / (T ln 2) in all), and the arg-max may differ only where the
oracle's top two logits lie within 2 delta.
"""
import math
import sys

import numpy as np
import pytest

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


def run(h_bits, w_bits, T, tokens):
    h = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    tk = None if tokens is None else torch.from_numpy(tokens.astype(np.int32)).to(DEV)
    res = L.spec_lm_head_row_stats(h, w, temperature=T, tokens=tk)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def oracle(h_bits, w_bits, T, tokens, rows=None):
    h = W.bf16_bits_to_f32(h_bits).astype(np.float64)
    if rows is not None:
        h = h[rows]
        tokens = None if tokens is None else tokens[rows]
    w = W.bf16_bits_to_f32(w_bits).astype(np.float64)
    return O.lm_head_row_stats(h, w, O.SamplingParams(T), tokens=tokens), np.abs(h) @ np.abs(w).T


def worst(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    m = np.isfinite(r) & np.isfinite(g)
    if not m.any():
        return None
    e = np.where(m, np.abs(g - r) - (H.REL_TOL * np.abs(r) + H.ABS_TOL), -np.inf)
    i = int(np.argmax(e))
    return i, float(g[i]), float(r[i])


def check_exact(gpu, ref, rows):
    for k in ("max_logit", "log_z", "entropy_bits", "max_prob", "p_tok"):
        if k in gpu:
            assert H.close(gpu[k][rows], ref[k]), (k, worst(gpu[k][rows], ref[k]))
    np.testing.assert_array_equal(gpu["argmax"][rows], ref["argmax"])


def check_bounded(gpu, ref, absprod, D, T, rows):
    delta = D * 2.0 ** -24 * absprod.max(axis=1)          # per row
    for i, r in enumerate(rows):
        d = delta[i]
        if not math.isfinite(ref["max_logit"][i]):
            assert np.isnan(gpu["max_logit"][r]) and gpu["argmax"][r] == -1
            continue
        assert abs(gpu["max_logit"][r] - ref["max_logit"][i]) <= d + 1e-6 * abs(ref["max_logit"][i]), (r, d)
        l = ref["logits"][i]
        top = np.sort(l)[::-1]
        if len(top) < 2 or top[0] - top[1] > 2 * d:
            assert gpu["argmax"][r] == ref["argmax"][i], r
        if T == 0.0:
            continue
        f = math.exp(2 * d / T) - 1 + 1e-5
        assert abs(gpu["log_z"][r] - ref["log_z"][i]) <= d / T + 1e-5 * abs(ref["log_z"][i]) + 1e-6, r
        assert abs(gpu["max_prob"][r] - ref["max_prob"][i]) <= f * ref["max_prob"][i], r
        assert abs(gpu["entropy_bits"][r] - ref["entropy_bits"][i]) <= 2 * d / (T * math.log(2)) + \
            1e-5 * abs(ref["entropy_bits"][i]) + 1e-6, r
        if "p_tok" in gpu and math.isfinite(ref["p_tok"][i]):
            assert abs(gpu["p_tok"][r] - ref["p_tok"][i]) <= f * ref["p_tok"][i] + 1e-30, r


@pytest.mark.parametrize("R,V,D", [(37, 1000, 96), (70, 4096 + 77, 40), (130, 600, 264), (300, 700, 136)])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_head_exact_values(R, V, D, T):
    """Dyadic values: the GPU's logits are exact, so every statistic meets the usual bar and the
    arg-max (many ties here) is the lowest index.  Row counts span both tile heights and a ragged
    last tile; D not a multiple of 32 exercises the zero-filled last stage."""
    note(f"case head exact R={R} V={V} D={D} T={T}")
    h, w = W.head_inputs(R, V, D, seed=R + V + D, exact=True)
    rng = np.random.default_rng(1)
    tok = rng.integers(-2, V + 2, size=R)
    gpu = run(h, w, T, tok)
    ref, _ = oracle(h, w, T, tok)
    check_exact(gpu, ref, np.arange(R))


@pytest.mark.parametrize("T", [1.0, 0.6, 0.0])
def test_head_normal_values_bounded(T):
    """Normal values: the statistics within the bounds the fp32 accumulation allows."""
    R, V, D = 66, 3000, 256
    note(f"case head normal R={R} V={V} D={D} T={T}")
    h, w = W.head_inputs(R, V, D, seed=17, scale_w=0.2)
    tok = np.random.default_rng(2).integers(0, V, size=R)
    gpu = run(h, w, T, tok)
    ref, ap = oracle(h, w, T, tok)
    check_bounded(gpu, ref, ap, D, T, np.arange(R))


def test_head_nonfinite_rows_and_no_tokens():
    """A NaN or an infinity in a hidden row makes that row's outputs NaN (arg-max -1) and
    leaves the others alone; without tokens no p_tok is produced."""
    R, V, D = 9, 700, 64
    h, w = W.head_inputs(R, V, D, seed=3, exact=True)
    h[2, 5] = 0x7FC0            # NaN
    h[6, 0] = 0x7F80            # +inf
    gpu = run(h, w, 1.0, None)
    assert "p_tok" not in gpu
    ref, _ = oracle(h, w, 1.0, None)
    check_exact(gpu, ref, np.arange(R))
    assert gpu["argmax"][2] == -1 and np.isnan(gpu["log_z"][6])


def test_head_full_vocabulary_sampled_rows():
    """The target rows of the batch-64 workload at full size (R = 512, V = 151,936, D = 4096,
    as the benchmark runs it), checked on sampled rows within the accumulation bounds."""
    R, V, D = 512, 151936, 4096
    note(f"case head full R={R} V={V} D={D}")
    h, w = W.head_inputs(R, V, D, seed=2024)
    tok = np.random.default_rng(9).integers(0, V, size=R)
    gpu = run(h, w, 1.0, tok)
    rows = np.array([0, 127, 128, 301, 511])
    ref, ap = oracle(h, w, 1.0, tok, rows=rows)
    check_bounded(gpu, ref, ap, D, 1.0, rows)


@pytest.mark.parametrize("R,V,D", [(1, 5, 8), (3, 257, 24), (65, 300, 72), (2, 1, 16)])
def test_head_small_and_ragged_shapes(R, V, D):
    """Shapes at the edges of the tiling: a single row, fewer columns than a wave holds, one
    column in the last tile, a single column, 65 rows (the tall tile with one row in its
    second half), D not a multiple of the 64-deep stage."""
    note(f"case head small R={R} V={V} D={D}")
    h, w = W.head_inputs(R, V, D, seed=5 * R + V + D, exact=True)
    tok = np.arange(R, dtype=np.int64) % max(V, 1)
    for T in (1.0, 0.0):
        gpu = run(h, w, T, tok)
        ref, _ = oracle(h, w, T, tok)
        check_exact(gpu, ref, np.arange(R))


@pytest.mark.parametrize("R", [20, 150])
def test_head_strided_rows(R):
    """Row strides larger than D (a view into wider buffers): the padding is never read."""
    V, D, pad = 900, 40, 24
    h, w = W.head_inputs(R, V, D, seed=77, exact=True)
    hb = np.full((R, D + pad), 0x7FC0, dtype=np.uint16)   # NaN padding: any read of it shows
    wb = np.full((V, D + pad), 0x7FC0, dtype=np.uint16)
    hb[:, :D] = h
    wb[:, :D] = w
    ht = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).to(DEV)[:, :D]
    wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(DEV)[:, :D]
    res = L.spec_lm_head_row_stats(ht, wt, temperature=0.9)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in res.items()}
    ref, _ = oracle(h, w, 0.9, None)
    check_exact(gpu, ref, np.arange(R))


@pytest.mark.parametrize("R,V,D", [(129, 1000, 64), (300, 4096 + 77, 192), (257, 513, 128), (512, 300, 256)])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_head_square_tiles_exact(R, V, D, T):
    """More than 128 rows and D a whole number of 64-deep stages: the 256 x 256 tiles fed by
    direct-to-LDS loads.  Ragged row and column tails (one row in a second row tile, 77 columns
    in the last column tile, fewer columns than one tile), dyadic values so the logits are exact."""
    note(f"case head square exact R={R} V={V} D={D} T={T}")
    h, w = W.head_inputs(R, V, D, seed=3 * R + V + D, exact=True)
    tok = np.random.default_rng(4).integers(-1, V + 1, size=R)
    gpu = run(h, w, T, tok)
    ref, _ = oracle(h, w, T, tok)
    check_exact(gpu, ref, np.arange(R))


def test_head_square_tiles_nonfinite_and_strided():
    """The square tiles with row strides wider than D (NaN padding that must never be read)
    and a NaN and an infinity in two hidden rows of the second row tile."""
    R, V, D, pad = 300, 700, 64, 24
    h, w = W.head_inputs(R, V, D, seed=91, exact=True)
    h[260, 3] = 0x7FC0            # NaN
    h[299, 63] = 0xFF80           # -inf
    hb = np.full((R, D + pad), 0x7FC0, dtype=np.uint16)
    wb = np.full((V, D + pad), 0x7FC0, dtype=np.uint16)
    hb[:, :D] = h
    wb[:, :D] = w
    ht = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).to(DEV)[:, :D]
    wt = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(DEV)[:, :D]
    tok = np.arange(R, dtype=np.int64) % V
    res = L.spec_lm_head_row_stats(ht, wt, temperature=0.8,
                                   tokens=torch.from_numpy(tok.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in res.items()}
    ref, _ = oracle(h, w, 0.8, tok)
    check_exact(gpu, ref, np.arange(R))
    assert gpu["argmax"][260] == -1 and np.isnan(gpu["log_z"][299])


@pytest.mark.parametrize("T", [1.0, 0.6, 0.0])
def test_head_square_tiles_normal_values_bounded(T):
    """Normal values on the 256 x 256 tiles (more than 128 rows, D a multiple of 64): the
    statistics within the bounds the fp32 accumulation allows, rows in both row tiles."""
    R, V, D = 300, 3000, 320
    note(f"case head square normal R={R} V={V} D={D} T={T}")
    h, w = W.head_inputs(R, V, D, seed=29, scale_w=0.2)
    tok = np.random.default_rng(5).integers(0, V, size=R)
    gpu = run(h, w, T, tok)
    rows = np.array([0, 77, 255, 256, 299])
    ref, ap = oracle(h, w, T, tok, rows=rows)
    check_bounded(gpu, ref, ap, D, T, rows)
