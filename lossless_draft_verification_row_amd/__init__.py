"""Batched speculative-sampling verification for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libspecverify.so`` (the C ABI in ``include/spec_verify.h``).
Functions keep the C names; they only marshal torch tensors (device memory, strides, the
current HIP stream) into the C calls.  Every step of the computation runs in the library's
HIP kernels: there is no Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SPEC_F32", "SPEC_BF16", "STATUS", "PATHS", "load_library", "library_path", "call_options",
    "spec_verify_batch", "spec_verify_batch_noalloc", "spec_row_stats", "spec_residual_sample", "spec_status_string",
    "spec_verify_workspace_bytes", "spec_row_stats_workspace_bytes",
    "spec_residual_sample_workspace_bytes",
]

SPEC_F32 = 0
SPEC_BF16 = 1
STATUS = {
    "NONFINITE": 1, "BAD_TOKEN": 2, "ZERO_Q": 4, "RESIDUAL_EMPTY": 8, "TIMEOUT": 16,
    "FILTER_OVERFLOW": 32, "BAD_GAMMA": 64,
}
PATHS = {"auto": 0, "multi": 1}   # spec_path

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_WS_CACHE = {}   # per-device zero-initialised workspace reused by calls that pass none


class SamplingParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int), ("top_p", ctypes.c_float)]


POS_STATS_FIELDS = ("p_y", "q_y", "one_minus_tv", "draft_entropy_bits", "draft_max_prob",
                    "target_entropy_bits", "target_max_prob", "kl_pq", "kl_qp", "l1", "accept_prob",
                    "expected_committed")


class PosStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in POS_STATS_FIELDS]


class CallOptions(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("spin_limit", ctypes.c_int64), ("poll_delay", ctypes.c_int),
                ("poll_pause", ctypes.c_int), ("profile_start", ctypes.c_void_p), ("profile_stop", ctypes.c_void_p)]


def call_options(path="auto", spin_limit=None, poll_delay=None, poll_pause=None, profile_events=None):
    """A spec_call_options value, or None when every field keeps its default.  path: "auto" or
    "multi"; spin_limit, poll_delay, poll_pause: ints (None = default); profile_events: a pair
    of raw hipEvent_t handles recorded around the call's streaming kernel."""
    if path == "auto" and spin_limit is None and poll_delay is None and poll_pause is None and profile_events is None:
        return None
    ev0, ev1 = profile_events if profile_events is not None else (None, None)
    return CallOptions(PATHS[path], -1 if spin_limit is None else int(spin_limit),
                       0 if poll_delay is None else int(poll_delay), 0 if poll_pause is None else int(poll_pause),
                       ev0, ev1)


def _opt_ptr(opts):
    return None if opts is None else ctypes.byref(opts)


class GammaMLP(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("b2", ctypes.c_float)]


def library_path() -> str:
    return os.environ.get("SPEC_VERIFY_LIB", os.path.join(_HERE, "libspecverify.so"))


def load_library():
    """Load libspecverify.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m lossless_draft_verification_row_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, u64, sz, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
    op = ctypes.POINTER(CallOptions)
    lib.spec_verify_batch.restype = i32
    lib.spec_verify_batch.argtypes = [i32, i32, i32, i32, vp, i64, vp, i64, vp, vp, i32, SamplingParams,
                                      u64, u64, vp, vp, PosStats, vp, vp, vp, sz, vp]
    lib.spec_verify_batch_ex.restype = i32
    lib.spec_verify_batch_ex.argtypes = lib.spec_verify_batch.argtypes + [op]
    lib.spec_verify_batch_noalloc.restype = i32
    lib.spec_verify_batch_noalloc.argtypes = [i32, i32, i32, i32, vp, i64, vp, i64, vp, vp, i32, SamplingParams,
                                              u64, u64, vp, vp, PosStats, vp, vp, vp]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, SamplingParams]
    lib.spec_row_stats.restype = i32
    lib.spec_row_stats.argtypes = [i32, i32, i32, vp, i64, SamplingParams, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_row_stats_ex.restype = i32
    lib.spec_row_stats_ex.argtypes = lib.spec_row_stats.argtypes + [op]
    lib.spec_row_stats_workspace_bytes.restype = sz
    lib.spec_row_stats_workspace_bytes.argtypes = [i32, i32, i32, SamplingParams]
    lib.spec_residual_sample.restype = i32
    lib.spec_residual_sample.argtypes = [i32, i32, i32, vp, i64, vp, i64, SamplingParams, vp, u64, u64,
                                         vp, vp, vp, vp, sz, vp]
    lib.spec_residual_sample_ex.restype = i32
    lib.spec_residual_sample_ex.argtypes = lib.spec_residual_sample.argtypes + [op]
    lib.spec_residual_sample_workspace_bytes.restype = sz
    lib.spec_residual_sample_workspace_bytes.argtypes = [i32, i32, i32, SamplingParams]
    lib.spec_lm_head_row_stats.restype = i32
    lib.spec_lm_head_row_stats.argtypes = [i32, i32, i32, vp, i64, vp, i64, SamplingParams, vp, vp, vp, vp, vp, vp,
                                           vp, vp, sz, vp]
    lib.spec_lm_head_row_stats_ex.restype = i32
    lib.spec_lm_head_row_stats_ex.argtypes = lib.spec_lm_head_row_stats.argtypes + [op]
    lib.spec_lm_head_workspace_bytes.restype = sz
    lib.spec_lm_head_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spec_select_gamma.restype = i32
    lib.spec_select_gamma.argtypes = [i32, vp, vp, GammaMLP, vp, vp, vp]
    lib.spec_stream_read.restype = i32
    lib.spec_stream_read.argtypes = [vp, i64, vp, vp]
    lib.spec_mfma_rate.restype = i32
    lib.spec_mfma_rate.argtypes = [i32, i32, i32, vp, vp]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_status_string.argtypes = [i32]
    _LIB = lib
    return lib


def spec_status_string(code: int) -> str:
    return load_library().spec_status_string(int(code)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed: {rc} ({spec_status_string(rc)})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    return t.data_ptr(), t.stride(0)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _sp(temperature, top_k, top_p):
    return SamplingParams(float(temperature), int(top_k), float(top_p))


def new_workspace(nbytes, device="cuda"):
    """A workspace for the library: zero-filled device bytes (the counter header must start at
    zero; every completed call leaves it zero)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _workspace(nbytes, device, workspace):
    """Caller's workspace, or a cached per-device one.  The cached workspace is shared by calls
    on the same device, so calls that pass none must be ordered on one stream."""
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"{nbytes} needed")
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    cache = _WS_CACHE.get(device)
    if cache is None or cache.numel() < nbytes:
        cache = torch.zeros(nbytes, dtype=torch.uint8, device=device)   # zero once: counter header
        _WS_CACHE[device] = cache
    return cache.data_ptr(), cache.numel()


def spec_verify_workspace_bytes(B, V, gamma_max, dtype, temperature, top_k=0, top_p=1.0) -> int:
    return int(load_library().spec_verify_workspace_bytes(B, V, gamma_max, dtype, _sp(temperature, top_k, top_p)))


def spec_row_stats_workspace_bytes(R, V, dtype, temperature, top_k=0, top_p=1.0) -> int:
    return int(load_library().spec_row_stats_workspace_bytes(R, V, dtype, _sp(temperature, top_k, top_p)))


def spec_residual_sample_workspace_bytes(R, V, dtype, temperature, top_k=0, top_p=1.0) -> int:
    return int(load_library().spec_residual_sample_workspace_bytes(R, V, dtype, _sp(temperature, top_k, top_p)))


def spec_verify_batch(target_logits, draft_logits, draft_tokens, cu_draft, gamma_max, *,
                      temperature=1.0, top_k=0, top_p=1.0, seed=0, step=0, pos_stats=True,
                      req_stats=True, kl=False, workspace=None, out=None, stream=None, options=None):
    """Verify one speculative round for B ragged requests (see spec_verify_batch in the header;
    ``options`` is a call_options() value, None for the defaults).

    target_logits [sum(g_b + 1), V] and draft_logits [sum g_b, V] (or None: token-only draft)
    are bf16 or fp32 CUDA tensors; draft_tokens [sum g_b] and cu_draft [B + 1] are int32 CUDA
    tensors.  Returns a dict of CUDA tensors: tokens [B, gamma_max + 1], num_accepted [B],
    status [B], and, when requested, the per-position and per-request statistics (pos_stats:
    p_y ... target_max_prob, l1, accept_prob, expected_committed [B]; kl: kl_pq, kl_qp).
    """
    lib = load_library()
    dev = target_logits.device
    B = cu_draft.numel() - 1
    V = target_logits.shape[1]
    dt = _dtype_code(target_logits)
    tp, tld = _rows(target_logits, "target_logits")
    dp, dld = (None, 0) if draft_logits is None else _rows(draft_logits, "draft_logits")
    if draft_logits is not None and (draft_logits.dtype != target_logits.dtype or draft_logits.shape[1] != V):
        raise ValueError("draft_logits must match target_logits in dtype and vocabulary")
    for t, n in ((draft_tokens, "draft_tokens"), (cu_draft, "cu_draft")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 CUDA tensor")
    Rd = draft_tokens.numel()
    sp = _sp(temperature, top_k, top_p)
    o = out if out is not None else {}
    if "tokens" not in o:
        o["tokens"] = torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev)
        o["num_accepted"] = torch.empty(B, dtype=torch.int32, device=dev)
        o["status"] = torch.empty(B, dtype=torch.int32, device=dev)
        if pos_stats:
            for k in ("p_y", "q_y", "one_minus_tv", "draft_entropy_bits", "draft_max_prob", "l1", "accept_prob"):
                o[k] = torch.empty(Rd, dtype=torch.float32, device=dev)
            for k in ("target_entropy_bits", "target_max_prob"):
                o[k] = torch.empty(Rd + B, dtype=torch.float32, device=dev)
            o["expected_committed"] = torch.empty(B, dtype=torch.float32, device=dev)
        if kl:
            for k in ("kl_pq", "kl_qp"):
                o[k] = torch.empty(Rd, dtype=torch.float32, device=dev)
        if req_stats:
            o["req_stats"] = torch.empty((B, 4), dtype=torch.float32, device=dev)
    ps = PosStats(*[_ptr(o.get(k)) for k in POS_STATS_FIELDS])
    need = lib.spec_verify_workspace_bytes(B, V, gamma_max, dt, sp)
    wp, wn = _workspace(need, dev, workspace)
    rc = lib.spec_verify_batch_ex(B, V, gamma_max, dt, tp, tld, dp, dld, _ptr(draft_tokens), _ptr(cu_draft), Rd,
                                  sp, int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
                                  _ptr(o["tokens"]), _ptr(o["num_accepted"]), ps, _ptr(o.get("req_stats")),
                                  _ptr(o["status"]), wp, wn, _stream(stream), _opt_ptr(options))
    _check(rc, "spec_verify_batch")
    return o


def spec_verify_batch_noalloc(target_logits, draft_logits, draft_tokens, cu_draft, gamma_max, *, out,
                              temperature=1.0, top_k=0, top_p=1.0, seed=0, step=0, stream=None):
    """spec_verify_batch without a workspace, for callers that cannot allocate device memory:
    the library's static per-GPU scratch serves as the workspace (see the header).  ``out``
    holds the caller's output tensors (the keys spec_verify_batch returns; tokens, num_accepted
    and status are required, the statistics optional).  Raises when the call needs more than
    the scratch holds."""
    lib = load_library()
    B = cu_draft.numel() - 1
    V = target_logits.shape[1]
    dt = _dtype_code(target_logits)
    tp, tld = _rows(target_logits, "target_logits")
    dp, dld = (None, 0) if draft_logits is None else _rows(draft_logits, "draft_logits")
    for t, n in ((draft_tokens, "draft_tokens"), (cu_draft, "cu_draft")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 CUDA tensor")
    ps = PosStats(*[_ptr(out.get(k)) for k in POS_STATS_FIELDS])
    rc = lib.spec_verify_batch_noalloc(B, V, gamma_max, dt, tp, tld, dp, dld, _ptr(draft_tokens), _ptr(cu_draft),
                                       draft_tokens.numel(), _sp(temperature, top_k, top_p),
                                       int(seed) & (2**64 - 1), int(step) & (2**64 - 1), _ptr(out["tokens"]),
                                       _ptr(out["num_accepted"]), ps, _ptr(out.get("req_stats")),
                                       _ptr(out["status"]), _stream(stream))
    _check(rc, "spec_verify_batch_noalloc")
    return out


def spec_row_stats(logits, *, temperature=1.0, top_k=0, top_p=1.0, workspace=None, stream=None, options=None):
    """Per-row statistics of filtered, tempered logit rows.  Returns a dict of [R] tensors:
    max_logit, argmax, log_z, entropy_bits, max_prob, kept_count."""
    lib = load_library()
    dev = logits.device
    R, V = logits.shape
    dt = _dtype_code(logits)
    lp, ld = _rows(logits, "logits")
    sp = _sp(temperature, top_k, top_p)
    o = {
        "max_logit": torch.empty(R, dtype=torch.float32, device=dev),
        "argmax": torch.empty(R, dtype=torch.int32, device=dev),
        "log_z": torch.empty(R, dtype=torch.float32, device=dev),
        "entropy_bits": torch.empty(R, dtype=torch.float32, device=dev),
        "max_prob": torch.empty(R, dtype=torch.float32, device=dev),
        "kept_count": torch.empty(R, dtype=torch.int32, device=dev),
    }
    need = lib.spec_row_stats_workspace_bytes(R, V, dt, sp)
    wp, wn = _workspace(need, dev, workspace)
    rc = lib.spec_row_stats_ex(R, V, dt, lp, ld, sp, *[_ptr(o[k]) for k in (
        "max_logit", "argmax", "log_z", "entropy_bits", "max_prob", "kept_count")], wp, wn, _stream(stream),
        _opt_ptr(options))
    _check(rc, "spec_row_stats")
    return o


def spec_residual_sample(p_logits, q_logits=None, *, temperature=1.0, top_k=0, top_p=1.0, uniforms=None,
                         seed=0, step=0, workspace=None, stream=None, options=None):
    """One draw per row from [p - q]_+ (or p when q_logits is None).  Returns a dict of [R]
    tensors: token (int32), mass (fp64: beta, or 1 without q), status (int32)."""
    lib = load_library()
    dev = p_logits.device
    R, V = p_logits.shape
    dt = _dtype_code(p_logits)
    pp, pld = _rows(p_logits, "p_logits")
    qp, qld = (None, 0) if q_logits is None else _rows(q_logits, "q_logits")
    if uniforms is not None:
        if uniforms.dtype != torch.float64 or tuple(uniforms.shape) != (R, 3) or not uniforms.is_contiguous():
            raise ValueError("uniforms must be a contiguous float64 tensor of shape [R, 3]")
    sp = _sp(temperature, top_k, top_p)
    o = {
        "token": torch.empty(R, dtype=torch.int32, device=dev),
        "mass": torch.empty(R, dtype=torch.float64, device=dev),
        "status": torch.empty(R, dtype=torch.int32, device=dev),
    }
    need = lib.spec_residual_sample_workspace_bytes(R, V, dt, sp)
    wp, wn = _workspace(need, dev, workspace)
    rc = lib.spec_residual_sample_ex(R, V, dt, pp, pld, qp, qld, sp, _ptr(uniforms), int(seed) & (2**64 - 1),
                                     int(step) & (2**64 - 1), _ptr(o["token"]), _ptr(o["mass"]), _ptr(o["status"]),
                                     wp, wn, _stream(stream), _opt_ptr(options))
    _check(rc, "spec_residual_sample")
    return o


def spec_stream_read(buf, sink, stream=None):
    """A plain streaming read of a CUDA tensor's bytes (the benchmark's HBM read ceiling); `sink`
    is a one-element int32 CUDA tensor the kernel may write."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 1):
        raise ValueError("buf must be a contiguous CUDA tensor and sink a CUDA int32 tensor")
    nbytes = buf.numel() * buf.element_size()
    rc = load_library().spec_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream))
    _check(rc, "spec_stream_read")


def spec_mfma_rate(mode, iters, workgroups, sink, stream=None):
    """Benchmark instrumentation (see spec_mfma_rate in the header): `workgroups` x 4 waves of
    `iters` steps of 16 bf16 32x32x16 MFMAs on register operands; mode 0 constant, 1 random
    fixed, 2 random changing every step.  sink: a float32 CUDA tensor of at least one element."""
    if sink.dtype != torch.float32 or sink.numel() < 1 or not sink.is_cuda:
        raise ValueError("sink must be a float32 CUDA tensor")
    rc = load_library().spec_mfma_rate(int(mode), int(iters), int(workgroups), _ptr(sink), _stream(stream))
    _check(rc, "spec_mfma_rate")


def spec_select_gamma(req_stats, w1, b1, w2, b2, comp=None, stream=None):
    """Each request's next draft length, gamma* = argmax over {2, 4, 6, 8} of
    f(x, gamma) gamma + 1 (see spec_select_gamma in the header).  req_stats [B, 4] (as
    spec_verify_batch returns it), w1 [16, 6], b1 [16], w2 [16] and comp [B] (or None) are
    float32 CUDA tensors; b2 is a float.  Returns {"gamma": [B] int32, "expected": [B, 4]}."""
    lib = load_library()
    for t, n, shape in ((req_stats, "req_stats", None), (w1, "w1", (16, 6)), (b1, "b1", (16,)), (w2, "w2", (16,))):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 CUDA tensor")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{n} must have shape {shape}")
    if req_stats.dim() != 2 or req_stats.shape[1] != 4:
        raise ValueError("req_stats must be [B, 4]")
    B = req_stats.shape[0]
    if comp is not None and (comp.dtype != torch.float32 or not comp.is_cuda or comp.numel() != B):
        raise ValueError("comp must be a float32 CUDA tensor of B values")
    dev = req_stats.device
    o = {"gamma": torch.empty(B, dtype=torch.int32, device=dev),
         "expected": torch.empty((B, 4), dtype=torch.float32, device=dev)}
    rc = lib.spec_select_gamma(B, _ptr(req_stats), _ptr(comp), GammaMLP(_ptr(w1), _ptr(b1), _ptr(w2), float(b2)),
                               _ptr(o["gamma"]), _ptr(o["expected"]), _stream(stream))
    _check(rc, "spec_select_gamma")
    return o


HEAD_FIELDS = ("max_logit", "argmax", "log_z", "entropy_bits", "max_prob", "p_tok")


def spec_lm_head_row_stats(hidden, weight, *, temperature=1.0, tokens=None, workspace=None, out=None, stream=None,
                           options=None):
    """Row statistics of l = hidden @ weight^T without materialising the logits (see
    spec_lm_head_row_stats in the header).  hidden [R, D] and weight [V, D] are bf16 CUDA
    tensors with unit column stride; tokens [R] int32 or None.  Returns a dict of [R] tensors:
    max_logit, argmax, log_z, entropy_bits, max_prob and, with tokens, p_tok."""
    lib = load_library()
    for t, n in ((hidden, "hidden"), (weight, "weight")):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
    hp, hld = _rows(hidden, "hidden")
    wp_, wld = _rows(weight, "weight")
    R, D = hidden.shape
    V = weight.shape[0]
    if weight.shape[1] != D:
        raise ValueError("hidden and weight must share D")
    if tokens is not None and (tokens.dtype != torch.int32 or not tokens.is_cuda or tokens.numel() != R):
        raise ValueError("tokens must be an int32 CUDA tensor of R entries")
    dev = hidden.device
    o = out if out is not None else {}
    if "max_logit" not in o:
        for k in ("max_logit", "log_z", "entropy_bits", "max_prob"):
            o[k] = torch.empty(R, dtype=torch.float32, device=dev)
        o["argmax"] = torch.empty(R, dtype=torch.int32, device=dev)
        if tokens is not None:
            o["p_tok"] = torch.empty(R, dtype=torch.float32, device=dev)
    need = lib.spec_lm_head_workspace_bytes(R, V, D)
    wsp, wsn = _workspace(need, dev, workspace)
    rc = lib.spec_lm_head_row_stats_ex(R, V, D, hp, hld, wp_, wld, _sp(temperature, 0, 1.0), _ptr(tokens),
                                       *[_ptr(o.get(k)) for k in HEAD_FIELDS], wsp, wsn, _stream(stream),
                                       _opt_ptr(options))
    _check(rc, "spec_lm_head_row_stats")
    return o
