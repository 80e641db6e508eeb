#!/usr/bin/env python3
"""Throughput of the chunk-parallel KDA forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gva_bf16] [--no-cpu-baseline]

Times K calls of kda_chunk_fwd (through the C ABI, inputs already resident in
HBM) bracketed by device synchronisation, then K more calls of
kda_chunk_fwd_profiled for per-kernel durations, and prints one JSON line:
  value         tokens per second of the whole job (Mtokens/s), tokens = B*T per call,
                from the K plain calls
  roofline      the call's algorithmic bytes (every input read once, every output
                written once) over the measured time of the whole call, against the
                8 TB/s HBM peak; traffic = the calibrated rocprofv3 counter bytes of
                one call when profiles/traffic.json matches the kernel sources
  path.stages   per kernel: HIP-event time, its algorithmic matrix FLOPs as a fraction
                of the 2.5 PFLOP/s bf16 peak, its counter bytes and rate
  timing        median single-call time warm and cold (512 MiB written before each
                cold call, which evicts the memory-side cache)
  gate_cumsum   kda_gate_chunk_cumsum on the same workload: achieved HBM GB/s
  cpu_baseline  the float64 oracle on the host cores, same workload
Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk_kda fwd Mtokens/s at HV=32,K=V=128,T=8K; % of MFMA/HBM roofline"
METRIC_RECURRENT = "fused_recurrent_kda decode Mtokens/s; % of HBM roofline"
METRIC_STATES = "chunk_kda fwd with intermediate states Mtokens/s; % of HBM roofline"
METRIC_BWD = "chunk_kda backward (forward recomputed inside) Mtokens/s; % of HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak


def algorithmic_bytes(w, inp) -> int:
    """Every input read once and every output written once: q, k, v, g, beta, o,
    plus the fp32 initial and final states when present."""
    B, T, H, K = inp["q"].shape
    HV, V = inp["v"].shape[2], inp["v"].shape[3]
    ntok = B * T
    qkv = inp["q"].element_size()
    b = ntok * (2 * H * K * qkv + HV * V * qkv + HV * K * inp["g"].element_size()
                + HV * inp["beta"].element_size() + HV * V * qkv)
    N = inp["initial_state"].shape[0] if inp["initial_state"] is not None else len(inp["seq_lens"])
    state = N * HV * K * V * 4
    if inp["initial_state"] is not None:
        b += state
    if w.output_final_state:
        b += state
    return int(b)


def algorithmic_flops(w, inp) -> int:
    """Dense 16x16 tiles with causal sub-block skipping, per (chunk, value head):
    NC(NC+1) BC^2 (3K + 2V) for Aqk, Akk0, W, U and Aqk V_new, 6 C K V for W S,
    KgT V_new and Qg S, C^3/3 for the solve (BC = 16, NC = C / BC)."""
    K, V, C = w.K, w.V, w.chunk
    HV = inp["v"].shape[2]
    NC, BC = C // 16, 16
    per_chunk = NC * (NC + 1) * BC * BC * (3 * K + 2 * V) + 6 * C * K * V + C ** 3 // 3
    chunks = sum(math.ceil(L / C) for L in inp["seq_lens"])
    return int(per_chunk * chunks * HV)


def stage_flops(w, inp) -> dict:
    """Algorithmic matrix FLOPs of each forward stage (the split of algorithmic_flops):
    intra forms Aqk, Akk0 (causal 16x16 tiles), W = A X, U = A v (lower-triangular A,
    16-row blocks) and the solve; the recurrence forms W S, KgT V_new, Qg S and the
    causal Aqk V_new."""
    K, V, C = w.K, w.V, w.chunk
    HV = inp["v"].shape[2]
    NC, BC = C // 16, 16
    chunks = sum(math.ceil(L / C) for L in inp["seq_lens"]) * HV
    tri = NC * (NC + 1) * BC * BC
    return {"intra": int(chunks * (tri * (3 * K + V) + C ** 3 // 3)),
            "recurrence": int(chunks * (6 * C * K * V + tri * V)),
            "plan": 0}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Hip:
    """The few HIP runtime calls bench.py makes itself (event timing), through the
    runtime torch already loaded."""

    def __init__(self):
        import re

        maps = open("/proc/self/maps").read()
        paths = sorted(set(re.findall(r"(\S*libamdhip64\.so\S*)", maps)))
        self.lib = ctypes.CDLL(paths[0])
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        assert self.lib.hipEventSynchronize(b) == 0
        t = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return float(t.value)


def source_digest() -> str:
    """Digest of the forward path's sources: every file under csrc/ except the backward's
    own kernels (kda_backward.*, kda_bwd_*), which the forward's kernels neither include nor
    launch."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_log2_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith(("kda_backward.", "kda_bwd_")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, per_launch_bytes_alg: float):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    entry = t.get("kernels", {}).get(kernel)
    if not entry or t.get("source_digest") != source_digest():
        return None
    return int(entry["fetch_kib"] * 1024 * t["copy_factor_fetch"] + entry["write_kib"] * 1024 * t["copy_factor_write"])


def load_call_traffic(names):
    """HBM bytes of one whole call (every stage's kernel) from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    total = 0
    for n in names:
        e = t.get("kernels", {}).get(n)
        if e is None:
            continue
        total += e["fetch_kib"] * 1024 * t["copy_factor_fetch"] + e["write_kib"] * 1024 * t["copy_factor_write"]
    return int(total) if total else None


def bench_recurrent(args, w, inp, d, desc, o, ht, stream, lib, hip):
    """Times kda_fused_recurrent_fwd (one kernel) and prints its own JSON line."""
    import torch

    def ptr(t):
        return None if t is None else t.data_ptr()

    rargs = (ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g"]), ptr(d["beta"]), ptr(d["A_log"]),
             ptr(d["dt_bias"]), ptr(d["initial_state"]), ptr(d["cu_seqlens"]), ptr(o), ptr(ht), stream)
    for _ in range(args.warmup):
        assert lib.kda_fused_recurrent_fwd(ctypes.byref(desc), *rargs) == 0
    torch.cuda.synchronize()
    start, end = hip.event(), hip.event()
    t_wall = time.perf_counter()
    hip.record(start, stream)
    for _ in range(args.steps):
        assert lib.kda_fused_recurrent_fwd(ctypes.byref(desc), *rargs) == 0
    hip.record(end, stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = hip.elapsed_ms(start, end) / args.steps
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    ntok = B * T
    alg_bytes = algorithmic_bytes(w, inp)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC_RECURRENT, "value": round(ntok / (ms * 1e-3) / 1e6, 3), "unit": "Mtokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "HV": HV, "K": K, "V": V,
                   "sequences": len(inp["seq_lens"]), "initial_state": d["initial_state"] is not None,
                   "final_state": w.output_final_state},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "fused_recurrent",
                     "kernel_ms": round(ms, 5)},
        "path": {"algorithmic_bytes": alg_bytes, "host_wall_ms_per_step": round(t_wall * 1e3 / args.steps, 4)},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_states(args, w, inp, d, desc, args_, stream, lib, hip):
    """Times kda_chunk_fwd_states (the forward plus the state each chunk starts from)
    against kda_chunk_fwd on the same inputs, and prints its own JSON line."""
    import torch

    C = w.chunk
    nchunks = sum((L + C - 1) // C for L in inp["seq_lens"])
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    hs = torch.empty((nchunks, HV, K, V), dtype=torch.float32, device=d["q"].device)
    sargs = args_[:11] + (hs.data_ptr(),) + args_[11:]

    def timed(fn, a):
        for _ in range(args.warmup):
            assert fn(ctypes.byref(desc), *a) == 0
        torch.cuda.synchronize()
        start, end = hip.event(), hip.event()
        hip.record(start, stream)
        for _ in range(args.steps):
            assert fn(ctypes.byref(desc), *a) == 0
        hip.record(end, stream)
        torch.cuda.synchronize()
        return hip.elapsed_ms(start, end) / args.steps

    ms = timed(lib.kda_chunk_fwd_states, sargs)
    ms_plain = timed(lib.kda_chunk_fwd, args_)
    ntok = B * T
    state_bytes = nchunks * HV * K * V * 4
    alg_bytes = algorithmic_bytes(w, inp) + state_bytes
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC_STATES, "value": round(ntok / (ms * 1e-3) / 1e6, 3), "unit": "Mtokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "HV": HV, "K": K, "V": V, "chunk": C,
                   "sequences": len(inp["seq_lens"]), "intermediate_states": nchunks},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "whole call",
                     "kernel_ms": round(ms, 5)},
        "path": {"algorithmic_bytes": alg_bytes, "state_bytes": state_bytes,
                 "ms_per_step_without_states": round(ms_plain, 5)},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_bwd(args, w, inp, d, desc, args_, stream, lib, hip):
    """Times kda_chunk_bwd (the forward with per-chunk states, then the backward
    kernels) and prints its own JSON line; the forward alone is timed beside it."""
    import torch

    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    N = len(inp["seq_lens"])
    dev = d["q"].device
    gen = torch.Generator(device="cpu").manual_seed(11)
    do = torch.randn((B, T, HV, V), generator=gen).to(device=dev, dtype=d["q"].dtype)
    dht = (0.5 * torch.randn((N, HV, K, V), generator=gen)).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty((B, T, H, K), **f32), torch.empty((B, T, H, K), **f32), torch.empty((B, T, HV, V), **f32),
            torch.empty((B, T, HV, K), **f32), torch.empty((B, T, HV), **f32),
            torch.empty((HV,), **f32) if d["A_log"] is not None else None,
            torch.empty((HV * K,), **f32) if d["dt_bias"] is not None else None, torch.empty((N, HV, K, V), **f32)]
    nbytes = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)

    def p(t):
        return None if t is None else t.data_ptr()

    bargs = args_[:9] + (p(do), p(dht)) + tuple(p(t) for t in outs) + (p(ws), ws.numel(), stream)

    def timed(fn, a, steps, warmup):
        for _ in range(warmup):
            assert fn(ctypes.byref(desc), *a) == 0
        torch.cuda.synchronize()
        start, end = hip.event(), hip.event()
        hip.record(start, stream)
        for _ in range(steps):
            assert fn(ctypes.byref(desc), *a) == 0
        hip.record(end, stream)
        torch.cuda.synchronize()
        return hip.elapsed_ms(start, end) / steps

    ms = timed(lib.kda_chunk_bwd, bargs, args.steps, min(args.warmup, 2))
    ms_fwd = timed(lib.kda_chunk_fwd, args_, 20, 5)
    # recomputation switched off: the saving forward, then the backward from what it kept
    # (the backward only reads the saved part, so repeated calls time the same work)
    sargs = args_[:11] + (p(ws), ws.numel(), stream)
    ms_fwd_save = timed(lib.kda_chunk_fwd_save, sargs, 20, 2)
    ms_saved = timed(lib.kda_chunk_bwd_saved, bargs, args.steps, min(args.warmup, 2))
    ntok = B * T
    eb = d["q"].element_size()
    # read: the forward's inputs, do and dht; written: the fp32 gradients
    alg_bytes = (algorithmic_bytes(w, inp) + ntok * HV * V * eb + N * HV * K * V * 4
                 + 4 * ntok * (2 * H * K + HV * V + HV * K + HV) + 4 * N * HV * K * V)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC_BWD, "value": round(ntok / (ms * 1e-3) / 1e6, 3), "unit": "Mtokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": min(args.warmup, 2), "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "HV": HV, "K": K, "V": V, "chunk": w.chunk,
                   "sequences": N},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "whole call",
                     "kernel_ms": round(ms, 4)},
        "path": {"algorithmic_bytes": alg_bytes, "forward_ms": round(ms_fwd, 5)},
        "disable_recompute": {"forward_save_ms": round(ms_fwd_save, 5), "backward_saved_ms": round(ms_saved, 4),
                              "what": "kda_chunk_fwd_save keeps the per-chunk intermediates and chunk-start "
                                      "states; kda_chunk_bwd_saved starts from them (no forward recompute)"},
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(w, inp, kw):
    from oracle import oracle_num_threads
    from tests.oracle_adapter import run_oracle

    threads = oracle_num_threads(0)
    t0 = time.perf_counter()
    run_oracle(inp, kw, nthreads=threads)
    dt = time.perf_counter() - t0
    ntok = inp["q"].shape[0] * inp["q"].shape[1]
    return {"value": ntok / dt / 1e6, "unit": "Mtokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"full workload ({ntok} tokens x {inp['v'].shape[2]} value heads), float64 "
                      f"token recurrence, {dt:.2f} s wall"}


def cold_warm(fn, args_, desc, stream, hip, reps, dev):
    """Median single-call times: warm (back-to-back, caches hold what the previous call
    left) and cold (a 512 MiB scratch buffer written right before the call, which evicts
    the 256 MB memory-side cache and every L2)."""
    import torch

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    warm, cold = [], []
    a, b = hip.event(), hip.event()
    for cold_run in (False, True):
        for _ in range(reps):
            if cold_run:
                scratch.fill_(1)
            else:
                assert fn(ctypes.byref(desc), *args_) == 0
            hip.record(a, stream)
            assert fn(ctypes.byref(desc), *args_) == 0
            hip.record(b, stream)
            (cold if cold_run else warm).append(hip.elapsed_ms(a, b))
    torch.cuda.synchronize(dev)
    med = lambda x: sorted(x)[len(x) // 2]  # noqa: E731
    return {"warm_median_ms": round(med(warm), 5), "cold_median_ms": round(med(cold), 5), "reps": reps,
            "cold_flush_bytes": 512 << 20}


def gate_stage(lib, desc, d, stream, hip, dev, steps):
    """kda_gate_chunk_cumsum on the same workload: reads g (plus A_log, dt_bias), writes
    the fp32 cumulative gate; its achieved HBM rate against the 8 TB/s peak."""
    import torch

    B, T, HV, K = d["g"].shape
    cum = torch.empty((B, T, HV, K), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    assert lib.kda_gate_chunk_cumsum_workspace_size(ctypes.byref(desc), ctypes.byref(nb)) == 0
    ws = torch.empty(max(nb.value, 256), dtype=torch.uint8, device=dev)

    def p(t):
        return None if t is None else t.data_ptr()

    ga = (p(d["g"]), p(d["A_log"]), p(d["dt_bias"]), p(d["cu_seqlens"]), None, p(cum), p(ws), ws.numel(), stream)
    for _ in range(3):
        assert lib.kda_gate_chunk_cumsum(ctypes.byref(desc), *ga) == 0
    a, b = hip.event(), hip.event()
    hip.record(a, stream)
    for _ in range(steps):
        assert lib.kda_gate_chunk_cumsum(ctypes.byref(desc), *ga) == 0
    hip.record(b, stream)
    ms = hip.elapsed_ms(a, b) / steps
    nbytes = d["g"].numel() * d["g"].element_size() + cum.numel() * 4 + HV * K * 4 + HV * 4
    return {"ms": round(ms, 5), "bytes": int(nbytes), "achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": "g read once, fp32 log2 cumulative gate written once (g_act not requested)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gva_bf16")
    ap.add_argument("--entry", choices=("chunk", "recurrent", "states", "bwd"), default="chunk",
                    help="chunk: kda_chunk_fwd (the metric); recurrent: kda_fused_recurrent_fwd, "
                         "the token-by-token decoding entry (use with --workload decode_bf16); "
                         "states: kda_chunk_fwd_states, the forward plus the per-chunk states; "
                         "bwd: kda_chunk_bwd, the backward (forward recomputed inside)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (5 times), the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this operator is benchmarked on a single MI355X "
              "(value heads shard across GPUs with no communication). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}), flush=True)
        return 0

    from gated_delta_rule_log2_amd import _abi, library
    from gated_delta_rule_log2_amd.workloads import WORKLOADS, kernel_kwargs, make_inputs

    w = WORKLOADS[args.workload]
    kw = kernel_kwargs(w)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    lib = library()
    hip = Hip()

    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    N = len(inp["seq_lens"])
    flags = (_abi.GATE_IN_KERNEL if w.gate_in_kernel else 0) | (_abi.SAFE_GATE if w.safe_gate else 0) \
        | (_abi.HAS_LOWER_BOUND if w.lower_bound is not None else 0) | (_abi.QK_L2NORM if w.qk_l2norm else 0) \
        | (_abi.BETA_SIGMOID if w.beta_sigmoid else 0) | (_abi.ALLOW_NEG_EIGVAL if w.allow_neg_eigval else 0) \
        | (_abi.OUTPUT_FINAL_STATE if w.output_final_state else 0)
    desc = _abi.KdaFwdDesc()
    desc.B, desc.T, desc.H, desc.HV, desc.K, desc.V = B, T, H, HV, K, V
    desc.chunk_size = w.chunk
    cu_host = None
    if d["cu_seqlens"] is not None:
        cu_host = inp["cu_seqlens"].contiguous()
        desc.num_seqs = N
        desc.cu_seqlens_host = ctypes.cast(cu_host.data_ptr(), ctypes.POINTER(ctypes.c_int64))
    else:
        desc.num_seqs = B
    dt = {torch.float32: _abi.DTYPE_FP32, torch.bfloat16: _abi.DTYPE_BF16}
    desc.qkv_dtype, desc.g_dtype, desc.beta_dtype = dt[d["q"].dtype], dt[d["g"].dtype], dt[d["beta"].dtype]
    desc.scale = w.scale
    desc.lower_bound = w.lower_bound if w.lower_bound is not None else 0.0
    desc.flags = flags
    nbytes = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, HV, V), dtype=d["q"].dtype, device=dev)
    ht = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    args_ = (ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g"]), ptr(d["beta"]), ptr(d["A_log"]),
             ptr(d["dt_bias"]), ptr(d["initial_state"]), ptr(d["cu_seqlens"]), ptr(o), ptr(ht),
             ptr(ws), ws.numel(), stream)
    nst = lib.kda_chunk_fwd_stage_count()
    names = [lib.kda_chunk_fwd_stage_name(i).decode() for i in range(nst)]
    if args.entry == "recurrent":
        return bench_recurrent(args, w, inp, d, desc, o, ht, stream, lib, hip)
    if args.entry == "states":
        return bench_states(args, w, inp, d, desc, args_, stream, lib, hip)
    if args.entry == "bwd":
        return bench_bwd(args, w, inp, d, desc, args_, stream, lib, hip)

    for _ in range(args.warmup):
        rc = lib.kda_chunk_fwd(ctypes.byref(desc), *args_)
        assert rc == 0, rc
    torch.cuda.synchronize(dev)

    # Timed region: K calls of kda_chunk_fwd exactly as a caller makes them (no per-stage
    # events, which cost ~5 us each on the stream), bracketed by synchronisation.
    start, end = hip.event(), hip.event()
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter()
    hip.record(start, stream)
    for s in range(args.steps):
        rc = lib.kda_chunk_fwd(ctypes.byref(desc), *args_)
        assert rc == 0, rc
    hip.record(end, stream)
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter() - t_wall
    total_ms = hip.elapsed_ms(start, end)
    ms_per_step = total_ms / args.steps
    # Kernel durations: K more calls of kda_chunk_fwd_profiled, which records a HIP event on
    # the library's stream before each stage and after the last one.
    events = [[hip.event() for _ in range(nst + 1)] for _ in range(args.steps)]
    ev_arrays = [(ctypes.c_void_p * (nst + 1))(*[e.value for e in evs]) for evs in events]
    torch.cuda.synchronize(dev)
    for s in range(args.steps):
        rc = lib.kda_chunk_fwd_profiled(ctypes.byref(desc), *args_, ev_arrays[s])
        assert rc == 0, rc
    torch.cuda.synchronize(dev)
    stage_ms = [sum(hip.elapsed_ms(events[s][i], events[s][i + 1]) for s in range(args.steps)) / args.steps
                for i in range(nst)]

    ntok = B * T
    value = ntok / (ms_per_step * 1e-3) / 1e6
    alg_bytes = algorithmic_bytes(w, inp)
    alg_flops = algorithmic_flops(w, inp)
    sflops = stage_flops(w, inp)
    # Roofline of the path: the call's algorithmic bytes over the measured time of the
    # whole call (every stage), against the HBM peak; the MFMA fraction beside it.
    achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_call_traffic(names),
                "kernel": "whole call (" + " + ".join(n for n, x in zip(names, stage_ms) if x > 0.006) + ")",
                "kernel_ms": round(ms_per_step, 5),
                "mfma_frac": round(alg_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    stages = {}
    for n, x in zip(names, stage_ms):
        tb = load_traffic(n, alg_bytes)
        stages[n] = {"ms": round(x, 4),
                     "mfma_frac": round(sflops.get(n, 0) / (x * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4) if x > 0 else 0.0,
                     "counter_bytes": tb,
                     "counter_gbs": round(tb / (x * 1e-3) / 1e9, 1) if (tb and x > 0) else None}
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "Mtokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "HV": HV, "K": K, "V": V, "chunk": w.chunk,
                   "sequences": N, "safe_gate": w.safe_gate, "lower_bound": w.lower_bound,
                   "initial_state": d["initial_state"] is not None, "final_state": w.output_final_state},
        "roofline": roofline,
        "path": {"algorithmic_bytes": alg_bytes, "algorithmic_flops": alg_flops,
                 "hbm_frac": round(alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(alg_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "stages": stages,
                 "host_wall_ms_per_step": round(t_wall * 1e3 / args.steps, 4)},
        "timing": cold_warm(lib.kda_chunk_fwd, args_, desc, stream, hip, max(5, min(args.steps, 21)), dev),
        "gate_cumsum": gate_stage(lib, desc, d, stream, hip, dev, max(5, args.steps // 2)),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, kw)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
