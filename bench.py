"""Benchmark: batched speculative-sampling verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-per-config] [--no-cpu-baseline]

A step is one spec_verify_batch call over one batch of the workload (every row read, accept
scan, correction / bonus sampling, signals).  Inputs are synthetic, seeded, resident in HBM
before the timed region; several copies of the batch are rotated so the 256 MB last-level
cache cannot serve a later step from an earlier one.  Prints one JSON line: the headline
workload (config 2 by default), then `per_config` with the other workloads (B=128 ragged
Llama-3 vocabulary, greedy B=256, filtered B=256), the streaming-read ceiling of the same GPU
and the fp64 oracle timed over the host's cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of one MI355X
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 timed calls after 20 warm-up calls (a call is 75-250 us): the first calls of a run
    # read slower, and 30 calls after 5 came out up to 7 % slower on the filtered workload
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure only --config (by default configs 3, 4 and 5 follow in per_config)")
    ap.add_argument("--filter", type=lambda v: (int(v.split(",")[0]), float(v.split(",")[1])), default=None,
                    metavar="K,P", help="the workload of --config with top-k K and top-p P instead of its own "
                                        "(the filtered paths: e.g. 0,0.9 for top-p alone); use with --no-per-config")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--lm-head", action="store_true",
                    help="time the fused LM head (spec_lm_head_row_stats) on the batch-64 workload's "
                         "target rows instead: R = 512, V = 151936, D = 4096")
    ap.add_argument("--copy-ref", action="store_true",
                    help="time plain 1 GiB copy and read kernels instead (roofline context and the "
                         "scale for HBM byte counters)")
    return ap.parse_args()


def copy_reference(steps):
    """Plain torch kernels over 1 GiB: a device-to-device copy (1 GiB read + 1 GiB written) and
    a sum (1 GiB read).  Their GB/s is the practical streaming ceiling on this machine."""
    import torch
    n = (1 << 30) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 << 30), ("sum", lambda: src.sum(), 1 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        res[name] = {"GBps": nbytes / dt / 1e9, "ms": dt * 1e3, "bytes": nbytes}
    print(json.dumps({"copy_reference": res, "peak_GBps": HBM_PEAK_GBS}), flush=True)


def stream_ceiling(torch, L, steps=20):
    """Context for the roofline: the library's plain streaming-read kernel (spec_stream_read)
    over 1 GiB on the same GPU, after the timed region, timed with events recorded on the
    kernel's stream around each launch; GB/s and the fraction of the HBM peak."""
    nbytes = 1 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        L.spec_stream_read(buf, sink)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record()
        L.spec_stream_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
    del buf
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "k_stream_read (spec_stream_read) over 1 GiB", "GBps": gbs, "frac": gbs / HBM_PEAK_GBS}


def mfma_ceiling(torch, L, reps=5):
    """Context for the matrix roofline: the library's register-operand MFMA kernel
    (spec_mfma_rate) on the head's 4 x 4 accumulator pattern, 1280 workgroups x 4 waves x 2048
    steps x 16 MFMAs, with constant operands and with random operands that change every step;
    TFLOP/s and the fraction of the dense bf16 peak, timed with events on the kernel's stream."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    wgs, iters = 1280, 2048
    flops = wgs * 4 * iters * 16 * 2.0 * 32 * 32 * 16
    out = {"kernel": "k_mfma_rate (spec_mfma_rate), 16 independent 32x32x16 bf16 MFMAs per step, "
                     "register operands, no memory traffic"}
    for mode, name in ((0, "constant_operands"), (2, "random_operands")):
        for _ in range(2):
            L.spec_mfma_rate(mode, iters, wgs, sink)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in pairs:
            a.record()
            L.spec_mfma_rate(mode, iters, wgs, sink)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in pairs]))
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"TFLOPs": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    return out


class HipEvents:
    """Raw hipEvent_t pairs, handed to the library in a call's options: the dispatch of the
    call's streaming kernel records them at its start and end.  Destroyed before the process
    exits (close())."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)

    def timed_pairs(self, n):
        self.pairs = [(self.create(), self.create()) for _ in range(n)]
        return self.pairs

    def close(self):
        for a, b in getattr(self, "pairs", []):
            self.destroy(a)
            self.destroy(b)
        self.pairs = []


def algorithmic_bytes(inp):
    """Each needed logit read once: target rows (gamma_b + 1 per request) and, when the draft
    distribution is used, draft rows (gamma_b per request)."""
    esz = 2 if inp.wl.dtype == "bf16" else 4
    V = inp.target.shape[1]
    rows = inp.target.shape[0] + (0 if (inp.draft is None or inp.wl.temperature == 0) else inp.draft.shape[0])
    return rows * V * esz


def _oracle_request(args):
    """One request through the fp64 oracle (a worker-process task of the CPU baseline)."""
    from oracle import spec_oracle as O
    tl, dl, ys, dtype, sp, b = args
    widen = ((lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
              .astype(np.float64)) if dtype == "bf16" else (lambda a: np.asarray(a, np.float64)))
    O.verify_request(widen(tl), None if dl is None else widen(dl), ys, sp, 1, 0, b)
    return len(ys)


def cpu_workers():
    """Worker count of the CPU baseline: every host core the process may use."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(inp, budget_s, pool, n_workers):
    """The fp64 oracle as it stands (never tuned for this), over a pool of worker processes, one
    request per task, on repeated passes over the workload's batch: three runs of about a third
    of the budget each, the median reported as verified positions per second."""
    from oracle import spec_oracle as O
    sp = O.SamplingParams(inp.wl.temperature, inp.wl.top_k, inp.wl.top_p)
    B = len(inp.gammas)
    tasks = []
    for b in range(B):
        g, c0 = int(inp.gammas[b]), int(inp.cu_draft[b])
        tl = np.ascontiguousarray(inp.target[c0 + b:c0 + b + g + 1])
        dl = None if (inp.draft is None or sp.temperature == 0) else np.ascontiguousarray(inp.draft[c0:c0 + g])
        tasks.append((tl, dl, [int(y) for y in inp.tokens[c0:c0 + g]], inp.wl.dtype, sp, b))
    rates, total_req, total_pos = [], 0, 0
    for _ in range(3):
        t0 = time.perf_counter()
        pos = req = 0
        while time.perf_counter() - t0 < budget_s / 3:
            pos += sum(pool.map(_oracle_request, tasks, chunksize=1))
            req += B
        el = time.perf_counter() - t0
        rates.append(pos / el)
        total_req += req
        total_pos += pos
    return {
        "value": float(np.median(rates)), "unit": "positions/s", "cores": n_workers, "kind": "oracle",
        "sample": f"{total_req} request verifications ({total_pos} verified positions; the workload's batch of "
                  f"{B} requests repeated) in three runs of about {budget_s / 3:.0f} s, median of the three rates; "
                  f"fp64 numpy oracle, one request per task over {n_workers} worker processes on {cpu_model()}",
    }


def filtered_draft_tokens(inp, seed=77):
    """Draft tokens drawn from each draft row's filtered, tempered distribution (temperature,
    top-k with its boundary ties, then top-p over the kept set by value groups), as a draft model
    that samples from its own filtered q proposes them.  Plain numpy, only to synthesise the
    inputs of a filtered workload (the unfiltered draw in the workloads module would propose
    tokens outside the filtered support)."""
    wl = inp.wl
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = inp.draft_f32().astype(np.float64)
    V = rows.shape[1]
    toks = np.empty(rows.shape[0], dtype=np.int32)
    for r in range(rows.shape[0]):
        x = rows[r]
        if 0 < wl.top_k < V:
            kth = np.partition(x, V - wl.top_k)[V - wl.top_k]
            idx = np.nonzero(x >= kth)[0]
        else:
            idx = np.arange(V)
        v = x[idx]
        e = np.exp((v - v.max()) / wl.temperature)
        if wl.top_p < 1.0:
            order = np.argsort(-v, kind="stable")
            vs, es = v[order], e[order] / e.sum()
            starts = np.r_[0, np.nonzero(vs[1:] != vs[:-1])[0] + 1]
            cum = np.add.reduceat(es, starts).cumsum()
            g = int(np.searchsorted(cum, wl.top_p))   # first value group reaching top_p
            keep = v >= vs[starts[min(g, len(starts) - 1)]]
            idx, e = idx[keep], e[keep]
        toks[r] = idx[rng.choice(len(idx), p=e / e.sum())]
    return toks


# per-position outputs every timed call writes (the target's own entropy and max-prob are
# optional outputs and not requested)
OUTPUTS_PER_POSITION = ("p_y", "q_y", "one_minus_tv", "draft_entropy_bits", "draft_max_prob")


def kernel_source_digest(kernel):
    """First 16 hex digits of the sha256 over the kernel's source file and the two headers every
    kernel includes, in that order: a profile is current only while all three are unchanged."""
    import hashlib
    csrc = os.path.join(ROOT, "lossless_draft_verification_row_amd", "csrc")
    src = {"k_fused": "spec_fused.hip", "k_filt_slices": "spec_filter.hip",
           "k_head": "spec_head.hip"}.get(kernel, "spec_kernels.hip")
    h = hashlib.sha256()
    for name in (src, "spec_device.h", "spec_internal.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """The committed rocprofv3 counter summary of the kernel (HBM bytes and VALU instructions
    per launch), if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha") != kernel_source_digest(kernel):
            return None
        return rec
    except Exception:
        return None


def lm_head_bench(args, L, W, torch):
    """The fused LM head on the target rows of the batch-64 workload (64 requests x 8 positions
    = 512 rows, the Qwen3 vocabulary, hidden size 4096): every row's statistics and p(token)
    from h W^T without writing the logits.  The streaming kernel is the MFMA one, so its
    roofline is the dense bf16 matrix-core peak (2 R V D flops per launch)."""
    R, V, D, T = 512, 151936, 4096, 1.0
    h_bits, w_bits = W.head_inputs(R, V, D, seed=2024)
    dev = torch.device("cuda", 0)
    h = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    # two copies of the head, alternated, so that no launch finds the other's head in the cache
    ws = [w0, w0.clone()]
    tok = torch.from_numpy(np.random.default_rng(9).integers(0, V, size=R).astype(np.int32)).to(dev)
    lib = L.load_library()
    out = {}
    work = L.new_workspace(lib.spec_lm_head_workspace_bytes(R, V, D), dev)

    def step(k, options=None):
        return L.spec_lm_head_row_stats(h, ws[k % 2], temperature=T, tokens=tok, workspace=work, out=out,
                                        options=options)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    ev = HipEvents()
    pairs = ev.timed_pairs(args.steps)
    for k in range(args.steps):
        step(k, L.call_options(profile_events=pairs[k]))
    torch.cuda.synchronize()
    kms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    ev.close()
    flops = 2.0 * R * V * D
    counters = load_traffic("k_head") or {}
    achieved = flops / (kms * 1e-3) / 1e12
    line = {
        "metric": "fused LM head rows/sec (row statistics and p(token) without materialised logits), 1 MI355X",
        "value": R / sec, "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": sec * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; hidden N(0, 1), head N(0, 0.02^2), bf16)",
        "config": {"workload": "qwen3-vocab-head-r512-d4096", "R": R, "V": V, "D": D, "temperature": T,
                   "flops_per_step": flops, "head_bytes": V * D * 2, "head_copies_rotated": 2},
        "roofline": {"bound": "mfma", "kernel": "k_head (bf16 MFMA tiles with the row-statistics epilogue)",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": counters.get("bytes_per_launch"),
                     "kernel_ms_avg": kms,
                     "head_read_GBps": V * D * 2 / (kms * 1e-3) / 1e9},
        "mfma_ceiling": mfma_ceiling(torch, L),
    }
    ceil = line["mfma_ceiling"]["random_operands"]["TFLOPs"]
    line["roofline"]["frac_of_random_operand_ceiling"] = achieved / ceil
    if not args.no_cpu_baseline:
        from oracle import spec_oracle as O
        rows = 0
        t0 = time.perf_counter()
        wf = W.bf16_bits_to_f32(w_bits)
        hf = W.bf16_bits_to_f32(h_bits)
        while time.perf_counter() - t0 < args.cpu_seconds:
            r = rows % R
            O.lm_head_row_stats(hf[r:r + 4], wf, O.SamplingParams(T), tokens=tok.cpu().numpy()[r:r + 4])
            rows += 4
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                "sample": f"{rows} rows in blocks of 4 in {el:.1f} s (fp64 numpy matmul and "
                                          f"row statistics, single-threaded BLAS where the host allows)"}
    print(json.dumps(line), flush=True)


def measure(cfg, args, torch, L, W, steps, warmup):
    """One workload: seeded inputs resident in HBM (rotated copies beyond the 256 MB last-level
    cache), `warmup` untimed calls, `steps` calls timed on the host clock between two
    synchronisations, then `steps` more with events recorded by the streaming kernel's own
    dispatch.  Returns the inputs and the measured figures."""
    dev = torch.device("cuda", 0)
    inp = W.make_inputs(cfg)
    if args.filter is not None:
        k, p = args.filter
        base = inp.wl.name.split("-topk")[0]
        inp.wl = dataclasses.replace(inp.wl, name=f"{base}-topk{k}-topp{p:g}", top_k=k, top_p=p)
    wl = inp.wl
    if wl.temperature > 0 and inp.draft is not None and (0 < wl.top_k < wl.V or wl.top_p < 1.0):
        inp.tokens = filtered_draft_tokens(inp)
    B = len(inp.gammas)
    G = int(inp.gammas.max())
    positions = int(inp.gammas.sum())
    alg_bytes = algorithmic_bytes(inp)

    def dev_rows(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        if wl.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    tgt0 = dev_rows(inp.target)
    drf0 = None if (wl.token_only or wl.temperature == 0) else dev_rows(inp.draft)
    copies = max(4, int(np.ceil(1.0e9 / max(alg_bytes, 1))))
    tgts = [tgt0] + [tgt0.clone() for _ in range(copies - 1)]
    drfs = [drf0] + [None if drf0 is None else drf0.clone() for _ in range(copies - 1)]
    toks = torch.from_numpy(inp.tokens.astype(np.int32)).to(dev)
    cu = torch.from_numpy(inp.cu_draft.astype(np.int32)).to(dev)
    ws_bytes = L.spec_verify_workspace_bytes(B, wl.V, G, L.SPEC_BF16 if wl.dtype == "bf16" else L.SPEC_F32,
                                             wl.temperature, wl.top_k, wl.top_p)
    ws = L.new_workspace(ws_bytes, dev)
    # the outputs of a verification round: tokens, counts, status, the per-position draft
    # entropy, draft max-prob, 1 - TV, p(y) and q(y), and the per-request signal aggregates
    Rd = int(inp.cu_draft[-1])
    out = {"tokens": torch.empty((B, G + 1), dtype=torch.int32, device=dev),
           "num_accepted": torch.empty(B, dtype=torch.int32, device=dev),
           "status": torch.empty(B, dtype=torch.int32, device=dev),
           "req_stats": torch.empty((B, 4), dtype=torch.float32, device=dev)}
    for k in OUTPUTS_PER_POSITION:
        out[k] = torch.empty(Rd, dtype=torch.float32, device=dev)

    def step(k, options=None):
        return L.spec_verify_batch(tgts[k % copies], drfs[k % copies], toks, cu, G, temperature=wl.temperature,
                                   top_k=wl.top_k, top_p=wl.top_p, seed=1234, step=k, workspace=ws, out=out,
                                   options=options)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()

    # the timed region: exactly `steps` calls, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(warmup + k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = out["status"].cpu().numpy()

    # outside the timed region: the same calls again, each with events recorded by the dispatch
    # of its streaming kernel (the roofline's kernel time)
    ev = HipEvents()
    pairs = ev.timed_pairs(steps)
    torch.cuda.synchronize()
    for k in range(steps):
        step(warmup + steps + k, L.call_options(profile_events=pairs[k]))
    torch.cuda.synchronize()
    kernel_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    ev.close()
    del tgts, drfs, ws
    torch.cuda.empty_cache()

    sec = (t1 - t0) / steps
    kern_s = float(np.mean(kernel_ms)) / 1e3
    filtered = wl.temperature > 0 and 0 < wl.top_k < wl.V
    return {
        "inp": inp, "B": B, "G": G, "positions": positions, "alg_bytes": alg_bytes, "copies": copies,
        "sec": sec, "kern_s": kern_s, "kernel_ms": kernel_ms, "status_nonzero": int((st != 0).sum()),
        "kernel_key": "k_filt_slices" if filtered else "k_fused",
    }


def summary(m):
    """The per-config figures of a measurement."""
    return {
        "workload": m["inp"].wl.name, "call_us": m["sec"] * 1e6, "positions_per_s": m["positions"] / m["sec"],
        "kernel": m["kernel_key"], "kernel_us": m["kern_s"] * 1e6,
        "kernel_frac": m["alg_bytes"] / m["kern_s"] / 1e9 / HBM_PEAK_GBS,
        "end_to_end_frac": m["alg_bytes"] / m["sec"] / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes": m["alg_bytes"], "status_nonzero_requests": m["status_nonzero"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: one GPU's share of the "
                                   "request batch is the unit measured; --gpus must be 1"}))
        sys.exit(2)
    # the CPU baseline's worker processes start before anything touches the GPU
    pool, n_workers = None, 0
    if not args.no_cpu_baseline and not args.copy_ref and not args.lm_head:
        import multiprocessing as mp
        n_workers = cpu_workers()
        pool = mp.get_context("spawn").Pool(n_workers)
    import torch
    import lossless_draft_verification_row_amd as L
    from lossless_draft_verification_row_amd import workloads as W

    if args.copy_ref:
        copy_reference(args.steps)
        return

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.lm_head:
        lm_head_bench(args, L, W, torch)
        return
    m = measure(args.config, args, torch, L, W, args.steps, args.warmup)
    inp, wl = m["inp"], m["inp"].wl
    alg_bytes, kern_avg_s, sec_per_step = m["alg_bytes"], m["kern_s"], m["sec"]
    achieved = alg_bytes / kern_avg_s / 1e9
    kernel_key = m["kernel_key"]
    kernel_name = (("k_filt_slices (streaming kernel: every needed logit read once, per-slice top-k candidates)")
                   if kernel_key == "k_filt_slices" else
                   "k_fused (streaming kernel: every needed logit read once, both phases)")
    counters = load_traffic(kernel_key) or {}
    traffic = counters.get("bytes_per_launch")
    # VALU issue fraction: the kernel's VALU instructions (SQ_INSTS_VALU per launch, from the
    # same counter summary) at 4 cycles per wave64 instruction on a 16-lane SIMD, over the
    # SIMD cycles of the measured launch (1024 SIMDs at 2.4 GHz)
    valu = counters.get("valu_insts_per_launch")
    valu_frac = valu * 4.0 / (kern_avg_s * 2.4e9 * 1024) if valu else None
    line = {
        "metric": "verified draft positions/sec (and streaming-kernel HBM GB/s vs peak), 1 MI355X",
        "value": m["positions"] / sec_per_step,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": (f"synthetic (seeded numpy PCG64; N(0, {wl.sigma:g}^2) target logits, "
                 + ("token-only draft" if inp.draft is None else
                    f"draft = target + N(0, {wl.tau:g}^2)" if wl.tau is not None else "independent draft rows")
                 + (", draft tokens drawn from the filtered tempered draft distribution)"
                    if wl.temperature > 0 and (0 < wl.top_k < wl.V or wl.top_p < 1.0) else
                    ", draft tokens drawn from the tempered draft distribution)" if wl.temperature > 0 else
                    ", draft tokens = argmax of target + noise)")),
        "config": {"workload": wl.name, "B": m["B"], "gamma": m["G"], "V": wl.V, "positions_per_step": m["positions"],
                   "temperature": wl.temperature, "top_k": wl.top_k, "top_p": wl.top_p,
                   "outputs": ["tokens", "num_accepted", "status", "req_stats", *OUTPUTS_PER_POSITION],
                   "algorithmic_bytes_per_step": alg_bytes, "input_copies_rotated": m["copies"],
                   "end_to_end_GBps": alg_bytes / sec_per_step / 1e9,
                   "status_nonzero_requests": m["status_nonzero"]},
        "roofline": {"bound": "hbm", "kernel": kernel_name,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "end_to_end_frac": alg_bytes / sec_per_step / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms_avg": kern_avg_s * 1e3,
                     "kernel_ms_p10_p50_p90": [float(x) for x in np.percentile(m["kernel_ms"], [10, 50, 90])],
                     "valu_issue_frac": valu_frac},
    }
    if not args.no_per_config:
        line["per_config"] = {}
        for c in (3, 4, 5):
            if c == args.config:
                continue
            line["per_config"][str(c)] = summary(measure(c, args, torch, L, W, args.steps,
                                                         args.warmup))
    line["stream_ceiling"] = stream_ceiling(torch, L)
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, pool, n_workers)
        pool.terminate()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
