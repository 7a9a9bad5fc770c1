"""Seeded synthetic workloads for batched speculative-sampling verification.

This module only draws random inputs: logits, draft tokens and ragged draft lengths.  It holds
none of the verification arithmetic (no softmax, filter, acceptance or residual), so the HIP
path and the oracle can both be fed from it without sharing any of the method.

Shapes follow the pages' workloads: Qwen3-sized (151,936) and Llama-3-sized (128,256)
vocabularies, a draft block of 7 (the DLite page's K = 7), draft lengths from {2, 4, 6, 8}
(the SpecKV page's gamma grid), batch 64 (the DLite page's concurrency-64 run) up to 256.
Logits are i.i.d. N(0, sigma^2); a draft row is its target row plus independent N(0, tau^2)
noise, then rounded to bf16 (round to nearest even).  Data are drawn with numpy's PCG64.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QWEN3_VOCAB = 151936
LLAMA3_VOCAB = 128256


@dataclass
class Workload:
    name: str
    B: int
    V: int
    gamma: object        # int, or "mixed" for gamma_b drawn from {2, 4, 6, 8}
    dtype: str           # "bf16" or "f32"
    sigma: float         # target logit scale
    tau: float           # draft noise scale
    temperature: float
    top_k: int = 0
    top_p: float = 1.0
    token_only: bool = False   # draft supplies token ids only (greedy configuration)


WORKLOADS = {
    1: Workload("tiny-v8-f32", 1, 8, 4, "f32", 2.0, None, 1.0),
    2: Workload("qwen3-vocab-b64-g7-t1", 64, QWEN3_VOCAB, 7, "bf16", 3.0, 1.0, 1.0),
    3: Workload("llama3-vocab-b128-gmixed-t0.7", 128, LLAMA3_VOCAB, "mixed", "bf16", 3.0, 1.5, 0.7),
    4: Workload("qwen3-vocab-b256-g7-greedy", 256, QWEN3_VOCAB, 7, "bf16", 3.0, 1.0, 0.0,
                token_only=True),
    5: Workload("qwen3-vocab-b256-g7-t0.7-topk50-topp0.9", 256, QWEN3_VOCAB, 7, "bf16", 3.0, 1.0,
                0.7, top_k=50, top_p=0.9),
}


def bf16_bits_from_f32(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even (finite inputs)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draft_lengths(wl: Workload, rng, B):
    if wl.gamma == "mixed":
        return rng.choice(np.array([2, 4, 6, 8]), size=B)
    return np.full(B, int(wl.gamma))


def gumbel_argmax(rows_f32, temperature, rng):
    """Index of max(l / T + G) per row, G standard Gumbel: an exact draw from softmax(l / T).

    With T = 0 this is the plain argmax (first occurrence).  Used to make draft tokens that
    follow the unfiltered tempered draft distribution.
    """
    rows = np.asarray(rows_f32, dtype=np.float32)
    if temperature == 0.0:
        return rows.argmax(axis=1).astype(np.int32)
    out = np.empty(rows.shape[0], dtype=np.int32)
    for r in range(rows.shape[0]):
        u = rng.random(rows.shape[1])
        g = -np.log(-np.log(np.maximum(u, 1e-300)))
        out[r] = int(np.argmax(rows[r].astype(np.float64) / temperature + g))
    return out


@dataclass
class Inputs:
    wl: Workload
    gammas: np.ndarray        # [B] int32
    cu_draft: np.ndarray      # [B+1] int32, exclusive prefix of gammas
    target: np.ndarray        # [sum(gamma_b + 1), V]  uint16 bf16 bits or float32
    draft: object             # [sum gamma_b, V] same dtype, or None (token-only)
    tokens: np.ndarray        # [sum gamma_b] int32
    seed: int

    def target_f32(self, rows=slice(None)):
        t = self.target[rows]
        return bf16_bits_to_f32(t) if self.wl.dtype == "bf16" else np.asarray(t, np.float32)

    def draft_f32(self, rows=slice(None)):
        d = self.draft[rows]
        return bf16_bits_to_f32(d) if self.wl.dtype == "bf16" else np.asarray(d, np.float32)


def make_inputs(cfg, B=None, V=None, seed=None, gamma=None, tokens="gumbel") -> Inputs:
    """Draw the inputs of workload ``cfg`` (1..5), optionally at a smaller B or V.

    Request b's target rows are laid out at cu[b] + b .. cu[b] + b + gamma_b (gamma_b + 1 rows);
    its draft rows and tokens at cu[b] .. cu[b] + gamma_b - 1.  Draft row i is target row i
    plus N(0, tau^2) noise.  ``tokens``: "gumbel" draws y_i from the unfiltered tempered
    draft row (the plain argmax for greedy), "none" leaves zeros for the caller to fill.
    """
    wl = WORKLOADS[cfg]
    B = wl.B if B is None else B
    V = wl.V if V is None else V
    seed = 1000 + cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if gamma is not None:
        gammas = np.full(B, int(gamma))
    else:
        gammas = draft_lengths(wl, rng, B)
    gammas = gammas.astype(np.int32)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(gammas)
    Rd, Rt = int(cu[-1]), int(cu[-1]) + B
    bf16 = wl.dtype == "bf16"
    store = np.uint16 if bf16 else np.float32
    target = np.empty((Rt, V), dtype=store)
    draft = np.empty((Rd, V), dtype=store)
    toks = np.zeros(Rd, dtype=np.int32)
    tau = wl.tau
    for b in range(B):
        g = int(gammas[b])
        t32 = rng.standard_normal((g + 1, V), dtype=np.float32) * np.float32(wl.sigma)
        if tau is None:   # independent draft rows
            d32 = rng.standard_normal((g, V), dtype=np.float32) * np.float32(wl.sigma)
        else:
            d32 = t32[:g] + rng.standard_normal((g, V), dtype=np.float32) * np.float32(tau)
        t0 = int(cu[b]) + b
        if bf16:
            target[t0:t0 + g + 1] = bf16_bits_from_f32(t32)
            draft[cu[b]:cu[b] + g] = bf16_bits_from_f32(d32)
        else:
            target[t0:t0 + g + 1] = t32
            draft[cu[b]:cu[b] + g] = d32
    if tokens == "gumbel" and Rd:
        dv = bf16_bits_to_f32(draft) if bf16 else draft
        toks = gumbel_argmax(dv, wl.temperature, rng)
    return Inputs(wl, gammas, cu, target, None if wl.token_only else draft, toks, seed)


# ----------------------------------------------------------------------------- fused LM head inputs


def head_inputs(R, V, D, seed, scale_h=1.0, scale_w=0.02, exact=False):
    """Seeded hidden states [R, D] and a head [V, D] as bf16 bit patterns (uint16).  Normal by
    default (a unit-scale hidden state, a head scaled like a trained projection so logits have
    a standard deviation near scale_w * sqrt(D)); exact=True draws every value from
    {-1, -1/2, 0, 1/2, 1}, so every partial sum of a dot product with D <= 2^16 terms is exact
    in fp32.  W is generated in 8192-row blocks to bound host memory."""
    rng = np.random.default_rng(seed)
    if exact:
        vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32)
        h = bf16_bits_from_f32(vals[rng.integers(0, 5, size=(R, D))])
        w = np.empty((V, D), dtype=np.uint16)
        for v0 in range(0, V, 8192):
            n = min(8192, V - v0)
            w[v0:v0 + n] = bf16_bits_from_f32(vals[rng.integers(0, 5, size=(n, D))])
        return h, w
    h = bf16_bits_from_f32(rng.standard_normal((R, D), dtype=np.float32) * np.float32(scale_h))
    w = np.empty((V, D), dtype=np.uint16)
    for v0 in range(0, V, 8192):
        n = min(8192, V - v0)
        w[v0:v0 + n] = bf16_bits_from_f32(rng.standard_normal((n, D), dtype=np.float32) * np.float32(scale_w))
    return h, w
