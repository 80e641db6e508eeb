"""kda_chunk_fwd_noalloc: the forward with its workspace in the library's fixed device
array, called through the C ABI, against kda_chunk_fwd with a caller workspace.

Two calls in a row on one stream, the second with a smaller problem (fewer tokens and
heads, a packed batch), each compared bit for bit with kda_chunk_fwd on the same inputs;
and a problem larger than the array refused with KDA_ERR_WORKSPACE before any work.
"""
from __future__ import annotations

import ctypes

import pytest
import torch

from gated_delta_rule_log2_amd import _abi, library
from gated_delta_rule_log2_amd.workloads import GVA_BF16, VARLEN_BF16, kernel_kwargs, make_inputs

DEV = "cuda"


def _desc(inp, kw):
    B, T, H, K = inp["q"].shape
    HV, V = inp["v"].shape[2], inp["v"].shape[3]
    d = _abi.KdaFwdDesc()
    d.B, d.T, d.H, d.HV, d.K, d.V = B, T, H, HV, K, V
    d.chunk_size = kw["chunk_size"]
    cu_host = None
    if inp["cu_seqlens"] is not None:
        cu_host = inp["cu_seqlens"].to(torch.int64).contiguous()
        d.num_seqs = cu_host.numel() - 1
        d.cu_seqlens_host = ctypes.cast(cu_host.data_ptr(), ctypes.POINTER(ctypes.c_int64))
    else:
        d.num_seqs = B
    dt = {torch.float32: _abi.DTYPE_FP32, torch.bfloat16: _abi.DTYPE_BF16}
    d.qkv_dtype, d.g_dtype, d.beta_dtype = dt[inp["q"].dtype], dt[inp["g"].dtype], dt[inp["beta"].dtype]
    d.scale = kw["scale"]
    d.lower_bound = kw["lower_bound"] if kw["lower_bound"] is not None else 0.0
    f = 0
    f |= _abi.GATE_IN_KERNEL if kw["use_gate_in_kernel"] else 0
    f |= _abi.SAFE_GATE if kw["safe_gate"] else 0
    f |= _abi.HAS_LOWER_BOUND if kw["lower_bound"] is not None else 0
    f |= _abi.QK_L2NORM if kw["use_qk_l2norm_in_kernel"] else 0
    f |= _abi.BETA_SIGMOID if kw["use_beta_sigmoid_in_kernel"] else 0
    f |= _abi.ALLOW_NEG_EIGVAL if kw["allow_neg_eigval"] else 0
    f |= _abi.OUTPUT_FINAL_STATE
    d.flags = f
    return d, cu_host


def _run_both(inp, kw):
    lib = library()
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    desc, cu_host = _desc(inp, kw)
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    N = desc.num_seqs

    def p(t):
        return None if t is None else t.data_ptr()

    stream = torch.cuda.current_stream().cuda_stream
    ins = (p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), p(d["A_log"]), p(d["dt_bias"]),
           p(d["initial_state"]), p(d["cu_seqlens"]))
    # the fixed-array entry
    o1 = torch.full((B, T, HV, V), float("nan"), dtype=d["q"].dtype, device=DEV)
    h1 = torch.full((N, HV, K, V), float("nan"), dtype=torch.float32, device=DEV)
    rc = lib.kda_chunk_fwd_noalloc(ctypes.byref(desc), *ins, p(o1), p(h1), stream)
    assert rc == 0, lib.kda_status_string(rc)
    # the caller-workspace entry
    nbytes = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)) == 0
    assert nbytes.value <= _abi.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o1)
    h2 = torch.empty_like(h1)
    rc = lib.kda_chunk_fwd(ctypes.byref(desc), *ins, p(o2), p(h2), p(ws), ws.numel(), stream)
    assert rc == 0, lib.kda_status_string(rc)
    torch.cuda.synchronize()
    del cu_host
    return o1, h1, o2, h2


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_two_calls():
    # first call: T = 1500 (ragged last chunk), 4 value heads in GVA pairs
    w1 = GVA_BF16.replace(name="noalloc_a", T=1500, H=2, HV=4)
    print("case noalloc_a", flush=True)
    o1, h1, o2, h2 = _run_both(make_inputs(w1), kernel_kwargs(w1))
    assert torch.isfinite(o1.float()).all() and torch.isfinite(h1).all()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # second call, smaller: three packed sequences, 2 value heads
    w2 = VARLEN_BF16.replace(name="noalloc_b", num_seqs=3, min_len=17, max_len=200, H=1, HV=2)
    print("case noalloc_b", flush=True)
    o1, h1, o2, h2 = _run_both(make_inputs(w2), kernel_kwargs(w2))
    assert torch.isfinite(o1.float()).all() and torch.isfinite(h1).all()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_noalloc_refuses_problems_over_the_array():
    """Host-side refusal: a descriptor whose workspace exceeds the array returns
    KDA_ERR_WORKSPACE before any HIP call (so this runs without a GPU)."""
    lib = library()
    d = _abi.KdaFwdDesc()
    d.B, d.T, d.H, d.HV, d.K, d.V, d.chunk_size, d.num_seqs = 1, 8192, 16, 32, 128, 128, 64, 1
    d.qkv_dtype = d.g_dtype = d.beta_dtype = _abi.DTYPE_BF16
    d.scale, d.lower_bound = 0.088, -5.0
    d.flags = _abi.GATE_IN_KERNEL | _abi.SAFE_GATE | _abi.HAS_LOWER_BOUND
    nbytes = ctypes.c_size_t(0)
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(nbytes)) == 0
    assert nbytes.value > _abi.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    rc = lib.kda_chunk_fwd_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None, None,
                                   fake, None, None)
    assert _abi.STATUS_NAMES[rc] == "KDA_ERR_WORKSPACE"
