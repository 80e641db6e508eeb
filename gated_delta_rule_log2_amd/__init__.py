"""MI355X-native chunk-parallel Kimi Delta Attention (KDA) forward.

The compute path is the HIP library ``libkda.so`` (C ABI in include/kda.h); this
module only marshals torch tensors (device memory and the current stream) into
that ABI.  There is no CPU fallback: without the built library, or without a
GPU, calls raise.

    o, final_state = chunk_kda(q, k, v, g, beta, scale=..., initial_state=...,
                               output_final_state=True, cu_seqlens=...,
                               use_qk_l2norm_in_kernel=True, use_gate_in_kernel=True,
                               safe_gate=True, lower_bound=-5.0, A_log=..., dt_bias=...,
                               use_beta_sigmoid_in_kernel=True)

The keyword set mirrors chunk_kda as described in "flash-linear-attention KDA
内核工程实践…" §2 and §2.2 and the chunk_kda_fwd signature of "Reading Notes:
Implementation Notes for KDA in FLA" (forward entry point).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _abi

__all__ = ["chunk_kda", "chunk_kda_bwd", "fused_recurrent_kda", "gate_chunk_cumsum", "KDAContractError", "KDARuntimeError",
           "workspace_bytes", "library"]


class KDAContractError(ValueError):
    """An argument breaks the operator's contract (raised before any GPU work)."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{_abi.STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = _abi.STATUS_NAMES.get(code, str(code))


class KDARuntimeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_abi.STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def library():
    return _abi.load_library()


def _raise(code: int, lib):
    msg = lib.kda_status_string(code).decode()
    if code == _abi.KDA_ERR_HIP:
        raise KDARuntimeError(code, msg)
    raise KDAContractError(code, msg)


_DT = {torch.float32: _abi.DTYPE_FP32, torch.bfloat16: _abi.DTYPE_BF16}


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype not in _DT:
        raise KDAContractError(_abi.STATUS["KDA_ERR_DTYPE"], f"{what} must be float32 or bfloat16")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(t, name, shape, device, dtype=None):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise KDAContractError(_abi.STATUS["KDA_ERR_SHAPE"], f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise KDAContractError(_abi.STATUS["KDA_ERR_SHAPE"], f"{name} must be on {device}")
    if not t.is_contiguous():
        raise KDAContractError(_abi.STATUS["KDA_ERR_SHAPE"], f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KDAContractError(_abi.STATUS["KDA_ERR_DTYPE"], f"{name} must be {dtype}")


class _Desc:
    """A kda_fwd_desc plus the host buffers it points to (kept alive)."""

    def __init__(self, q, v, g, beta, scale, chunk_size, cu_seqlens, lower_bound, flags):
        B, T, H, K = q.shape
        HV, V = v.shape[2], v.shape[3]
        self.cu_host = None
        d = _abi.KdaFwdDesc()
        d.B, d.T, d.H, d.HV, d.K, d.V = B, T, H, HV, K, V
        d.chunk_size = chunk_size
        if cu_seqlens is not None:
            cu = cu_seqlens.detach().to("cpu", torch.int64).contiguous()
            self.cu_host = cu
            d.num_seqs = cu.numel() - 1
            d.cu_seqlens_host = ctypes.cast(cu.data_ptr(), ctypes.POINTER(ctypes.c_int64))
        else:
            d.num_seqs = B
            d.cu_seqlens_host = None
        d.qkv_dtype = _dtype_code(q, "q")
        d.g_dtype = _dtype_code(g, "g")
        d.beta_dtype = _dtype_code(beta, "beta")
        d.scale = float(scale)
        d.lower_bound = float(lower_bound) if lower_bound is not None else 0.0
        d.flags = flags
        self.d = d
        self.N = d.num_seqs


_workspaces: dict = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _flags(use_gate_in_kernel, safe_gate, lower_bound, use_qk_l2norm_in_kernel,
           use_beta_sigmoid_in_kernel, allow_neg_eigval, output_final_state):
    f = 0
    if use_gate_in_kernel:
        f |= _abi.GATE_IN_KERNEL
    if safe_gate:
        f |= _abi.SAFE_GATE
    if lower_bound is not None:
        f |= _abi.HAS_LOWER_BOUND
    if use_qk_l2norm_in_kernel:
        f |= _abi.QK_L2NORM
    if use_beta_sigmoid_in_kernel:
        f |= _abi.BETA_SIGMOID
    if allow_neg_eigval:
        f |= _abi.ALLOW_NEG_EIGVAL
    if output_final_state:
        f |= _abi.OUTPUT_FINAL_STATE
    return f


def _unsupported(**kw):
    for name, val in kw.items():
        if val:
            raise KDAContractError(_abi.STATUS["KDA_ERR_UNSUPPORTED"], f"{name} is not supported")


def workspace_bytes(q, v, g, beta, *, chunk_size=64, cu_seqlens=None, scale=None, **flags) -> int:
    lib = library()
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    desc = _Desc(q, v, g, beta, scale, chunk_size, cu_seqlens, flags.get("lower_bound"), 0)
    n = ctypes.c_size_t(0)
    rc = lib.kda_chunk_fwd_workspace_size(ctypes.byref(desc.d), ctypes.byref(n))
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    return n.value


class KDASaved:
    """The forward's per-chunk intermediates and chunk-start states, kept by chunk_kda with
    disable_recompute for one chunk_kda_bwd(..., saved=...) call (the backward then skips
    recomputing them).  `workspace` is the device buffer that holds them (sized by
    kda_chunk_bwd_workspace_size); `key` identifies the call they belong to.  The backward
    only reads them, so one KDASaved serves any number of backward calls."""

    def __init__(self, workspace: torch.Tensor, key: tuple):
        self.workspace = workspace
        self.key = key


def _saved_key(desc, *tensors) -> tuple:
    d = desc.d
    cu = None if desc.cu_host is None else tuple(int(x) for x in desc.cu_host)
    fields = (d.B, d.T, d.H, d.HV, d.K, d.V, d.chunk_size, d.num_seqs, d.qkv_dtype, d.g_dtype, d.beta_dtype,
              d.scale, d.lower_bound, d.flags & ~_abi.OUTPUT_FINAL_STATE)
    return fields, cu, tuple(None if t is None else (t.data_ptr(), t.device.index) for t in tensors)


def chunk_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
              scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
              output_final_state: bool = False, cu_seqlens: Optional[torch.Tensor] = None,
              chunk_size: int = 64, use_qk_l2norm_in_kernel: bool = False,
              use_gate_in_kernel: bool = False, safe_gate: bool = False,
              lower_bound: Optional[float] = None, A_log: Optional[torch.Tensor] = None,
              dt_bias: Optional[torch.Tensor] = None, use_beta_sigmoid_in_kernel: bool = False,
              allow_neg_eigval: bool = False, *, workspace: Optional[torch.Tensor] = None,
              cp_context=None, state_v_first: bool = False, transpose_state_layout: bool = False,
              return_intermediate_states: bool = False, disable_recompute: bool = False):
    """KDA forward on the current HIP stream.  Returns (o, final_state or None), or
    (o, final_state or None, h) with return_intermediate_states, or (o, final_state or
    None, saved) with disable_recompute: saved (a KDASaved) holds the per-chunk
    intermediates and chunk-start states for chunk_kda_bwd(..., saved=saved), which then
    skips recomputing the forward (kda_chunk_fwd_save / kda_chunk_bwd_saved).

    q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T, HV, K]; beta [B, T, HV];
    initial_state / final_state [N, HV, K, V] float32 (N = B, or len(cu_seqlens) - 1),
    [N, HV, V, K] with state_v_first / transpose_state_layout (the same switch).
    h: the state each chunk starts from, float32 [B, NT, HV, K, V] (NT = ceil(T / chunk_size)),
    or [1, total chunks, HV, K, V] with cu_seqlens (chunks restart at every sequence start),
    in the same state layout.  scale defaults to K ** -0.5.  The o dtype is the q/k/v dtype.
    """
    _unsupported(cp_context=cp_context is not None)
    transpose = bool(state_v_first or transpose_state_layout)
    if disable_recompute and (return_intermediate_states or transpose):
        raise KDAContractError(_abi.STATUS["KDA_ERR_UNSUPPORTED"],
                               "disable_recompute keeps [K, V] states for the backward: it does not combine "
                               "with return_intermediate_states or a transposed state layout")
    lib = library()
    if q.dim() != 4 or v.dim() != 4:
        raise KDAContractError(_abi.STATUS["KDA_ERR_SHAPE"], "q, k, v must be 4-D [B, T, heads, dim]")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise KDARuntimeError(_abi.KDA_ERR_HIP, "chunk_kda runs on a HIP device; got a CPU tensor")
    scale = 1.0 / math.sqrt(K) if scale is None else float(scale)
    _check_tensor(k, "k", (B, T, H, K), dev, q.dtype)
    _check_tensor(v, "v", (B, T, HV, V), dev, q.dtype)
    _check_tensor(q, "q", (B, T, H, K), dev)
    _check_tensor(g, "g", (B, T, HV, K), dev)
    _check_tensor(beta, "beta", (B, T, HV), dev)
    _check_tensor(A_log, "A_log", (HV,), dev, torch.float32)
    _check_tensor(dt_bias, "dt_bias", (HV * K,), dev, torch.float32)
    flags = _flags(use_gate_in_kernel, safe_gate, lower_bound, use_qk_l2norm_in_kernel,
                   use_beta_sigmoid_in_kernel, allow_neg_eigval, output_final_state)
    if transpose:
        flags |= _abi.TRANSPOSE_STATE
    desc = _Desc(q, v, g, beta, scale, chunk_size, cu_seqlens, lower_bound, flags)
    N = desc.N
    sshape = (V, K) if transpose else (K, V)
    _check_tensor(initial_state, "initial_state", (N, HV) + sshape, dev, torch.float32)
    cu_dev = None
    if cu_seqlens is not None:
        cu_dev = cu_seqlens.to(device=dev, dtype=torch.int64).contiguous()
    nbytes = ctypes.c_size_t(0)
    size_fn = lib.kda_chunk_bwd_workspace_size if disable_recompute else lib.kda_chunk_fwd_workspace_size
    rc = size_fn(ctypes.byref(desc.d), ctypes.byref(nbytes))
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if disable_recompute:  # the caller's, or one of its own: handed back with the result
        if workspace is None:
            workspace = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
    elif workspace is None:
        workspace = _workspace(dev, stream, nbytes.value)
    o = torch.empty((B, T, HV, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, HV) + sshape, dtype=torch.float32, device=dev) if output_final_state else None
    if disable_recompute:
        rc = lib.kda_chunk_fwd_save(ctypes.byref(desc.d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_dev), _ptr(o),
                                    _ptr(ht), _ptr(workspace), workspace.numel(), stream)
        if rc != _abi.KDA_OK:
            _raise(rc, lib)
        key = _saved_key(desc, q, k, v, g, beta, A_log, dt_bias, initial_state)
        return o, ht, KDASaved(workspace, key)
    if not return_intermediate_states:
        rc = lib.kda_chunk_fwd(ctypes.byref(desc.d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_dev), _ptr(o),
                               _ptr(ht), _ptr(workspace), workspace.numel(), stream)
        if rc != _abi.KDA_OK:
            _raise(rc, lib)
        return o, ht
    if desc.cu_host is not None:
        lens = desc.cu_host[1:] - desc.cu_host[:-1]
        hshape = (1, int(((lens + chunk_size - 1) // chunk_size).sum()))
    else:
        hshape = (B, (T + chunk_size - 1) // chunk_size)
    h = torch.empty(hshape + (HV,) + sshape, dtype=torch.float32, device=dev)
    rc = lib.kda_chunk_fwd_states(ctypes.byref(desc.d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_dev), _ptr(o),
                                  _ptr(ht), _ptr(h), _ptr(workspace), workspace.numel(), stream)
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    return o, ht, h


def chunk_kda_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                  do: torch.Tensor, dht: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                  initial_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                  chunk_size: int = 64, use_qk_l2norm_in_kernel: bool = False,
                  use_gate_in_kernel: bool = False, safe_gate: bool = False,
                  lower_bound: Optional[float] = None, A_log: Optional[torch.Tensor] = None,
                  dt_bias: Optional[torch.Tensor] = None, use_beta_sigmoid_in_kernel: bool = False,
                  allow_neg_eigval: bool = False, *, workspace: Optional[torch.Tensor] = None,
                  tokenwise: bool = False, disable_recompute: bool = False,
                  saved: Optional[KDASaved] = None) -> dict:
    """Gradients of <do, o> + <dht, final_state> for chunk_kda's inputs, on the current
    HIP stream (the forward is recomputed inside).  Arguments as chunk_kda; do has o's
    shape and dtype, dht the final state's ([N, HV, K, V] float32) or None.  Returns
    float32 tensors in a dict: dq, dk, dv, dg, dbeta, and dA_log / dt_bias / dh0 for
    the inputs given (dh0 always: the gradient at the initial state, zero or given).
    tokenwise=True runs the token-level form (kda_chunk_bwd_tokenwise) instead of the
    chunked one.  The workspace is allocated per call from torch's caching allocator
    (stream-ordered, so it is reused once the call's work is done) unless one is given;
    the forward's cached workspace is never grown by a backward call.
    saved: what chunk_kda(..., disable_recompute=True) returned for these same inputs;
    the forward is then not recomputed (kda_chunk_bwd_saved, the same gradients bit for
    bit) and saved's buffer serves as the workspace (the saved part is only read).
    disable_recompute=True requires it.
    """
    if disable_recompute and saved is None:
        raise KDAContractError(_abi.STATUS["KDA_ERR_NULL_POINTER"],
                               "disable_recompute needs saved= (chunk_kda(..., disable_recompute=True))")
    if saved is not None:
        if tokenwise:
            raise KDAContractError(_abi.STATUS["KDA_ERR_UNSUPPORTED"], "saved serves the chunked backward only")
    lib = library()
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise KDARuntimeError(_abi.KDA_ERR_HIP, "chunk_kda_bwd runs on a HIP device; got a CPU tensor")
    scale = 1.0 / math.sqrt(K) if scale is None else float(scale)
    _check_tensor(k, "k", (B, T, H, K), dev, q.dtype)
    _check_tensor(v, "v", (B, T, HV, V), dev, q.dtype)
    _check_tensor(do, "do", (B, T, HV, V), dev, q.dtype)
    _check_tensor(g, "g", (B, T, HV, K), dev)
    _check_tensor(beta, "beta", (B, T, HV), dev)
    _check_tensor(A_log, "A_log", (HV,), dev, torch.float32)
    _check_tensor(dt_bias, "dt_bias", (HV * K,), dev, torch.float32)
    flags = _flags(use_gate_in_kernel, safe_gate, lower_bound, use_qk_l2norm_in_kernel,
                   use_beta_sigmoid_in_kernel, allow_neg_eigval, False)
    desc = _Desc(q, v, g, beta, scale, chunk_size, cu_seqlens, lower_bound, flags)
    N = desc.N
    _check_tensor(initial_state, "initial_state", (N, HV, K, V), dev, torch.float32)
    _check_tensor(dht, "dht", (N, HV, K, V), dev, torch.float32)
    cu_dev = None if cu_seqlens is None else cu_seqlens.to(device=dev, dtype=torch.int64).contiguous()
    if saved is not None:
        if saved.key != _saved_key(desc, q, k, v, g, beta, A_log, dt_bias, initial_state):
            raise KDAContractError(_abi.STATUS["KDA_ERR_WORKSPACE"],
                                   "saved belongs to a forward call with other inputs or settings")
    nbytes = ctypes.c_size_t(0)
    size_fn = lib.kda_chunk_bwd_tokenwise_workspace_size if tokenwise else lib.kda_chunk_bwd_workspace_size
    rc = size_fn(ctypes.byref(desc.d), ctypes.byref(nbytes))
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if saved is not None:
        workspace = saved.workspace
    elif workspace is None:
        workspace = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, K), **f32), "dk": torch.empty((B, T, H, K), **f32),
           "dv": torch.empty((B, T, HV, V), **f32), "dg": torch.empty((B, T, HV, K), **f32),
           "dbeta": torch.empty((B, T, HV), **f32), "dh0": torch.empty((N, HV, K, V), **f32)}
    if A_log is not None:
        out["dA_log"] = torch.empty((HV,), **f32)
    if dt_bias is not None:
        out["ddt_bias"] = torch.empty((HV * K,), **f32)
    run = lib.kda_chunk_bwd_tokenwise if tokenwise else (lib.kda_chunk_bwd_saved if saved is not None
                                                         else lib.kda_chunk_bwd)
    rc = run(ctypes.byref(desc.d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                           _ptr(dt_bias), _ptr(initial_state), _ptr(cu_dev), _ptr(do), _ptr(dht),
                           _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                           _ptr(out["dbeta"]), _ptr(out.get("dA_log")), _ptr(out.get("ddt_bias")),
                           _ptr(out["dh0"]), _ptr(workspace), workspace.numel(), stream)
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    return out


def fused_recurrent_kda(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, scale: Optional[float] = None,
                        initial_state: Optional[torch.Tensor] = None, output_final_state: bool = False,
                        cu_seqlens: Optional[torch.Tensor] = None, use_qk_l2norm_in_kernel: bool = False,
                        use_gate_in_kernel: bool = False, safe_gate: bool = False,
                        lower_bound: Optional[float] = None, A_log: Optional[torch.Tensor] = None,
                        dt_bias: Optional[torch.Tensor] = None, use_beta_sigmoid_in_kernel: bool = False,
                        allow_neg_eigval: bool = False, *, state_v_first: bool = False,
                        transpose_state_layout: bool = False):
    """Token-by-token KDA forward (decoding) on the current HIP stream.

    Same arguments, shapes and result as chunk_kda; the state stays on chip for each
    sequence and there is no workspace.  Returns (o, final_state or None).
    """
    transpose = bool(state_v_first or transpose_state_layout)
    lib = library()
    if q.dim() != 4 or v.dim() != 4:
        raise KDAContractError(_abi.STATUS["KDA_ERR_SHAPE"], "q, k, v must be 4-D [B, T, heads, dim]")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dev = q.device
    if dev.type != "cuda":
        raise KDARuntimeError(_abi.KDA_ERR_HIP, "fused_recurrent_kda runs on a HIP device; got a CPU tensor")
    scale = 1.0 / math.sqrt(K) if scale is None else float(scale)
    _check_tensor(k, "k", (B, T, H, K), dev, q.dtype)
    _check_tensor(v, "v", (B, T, HV, V), dev, q.dtype)
    _check_tensor(q, "q", (B, T, H, K), dev)
    _check_tensor(g, "g", (B, T, HV, K), dev)
    _check_tensor(beta, "beta", (B, T, HV), dev)
    _check_tensor(A_log, "A_log", (HV,), dev, torch.float32)
    _check_tensor(dt_bias, "dt_bias", (HV * K,), dev, torch.float32)
    flags = _flags(use_gate_in_kernel, safe_gate, lower_bound, use_qk_l2norm_in_kernel,
                   use_beta_sigmoid_in_kernel, allow_neg_eigval, output_final_state)
    if transpose:
        flags |= _abi.TRANSPOSE_STATE
    desc = _Desc(q, v, g, beta, scale, 64, cu_seqlens, lower_bound, flags)
    N = desc.N
    sshape = (V, K) if transpose else (K, V)
    _check_tensor(initial_state, "initial_state", (N, HV) + sshape, dev, torch.float32)
    cu_dev = None
    if cu_seqlens is not None:
        cu_dev = cu_seqlens.to(device=dev, dtype=torch.int64).contiguous()
    stream = torch.cuda.current_stream(dev).cuda_stream
    o = torch.empty((B, T, HV, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, HV) + sshape, dtype=torch.float32, device=dev) if output_final_state else None
    rc = lib.kda_fused_recurrent_fwd(ctypes.byref(desc.d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_dev), _ptr(o),
                                     _ptr(ht), stream)
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    return o, ht


def gate_chunk_cumsum(g: torch.Tensor, *, chunk_size: int = 64, use_gate_in_kernel: bool = False,
                      lower_bound: Optional[float] = None, safe_gate: bool = False,
                      A_log: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, H: Optional[int] = None,
                      return_activated: bool = True):
    """Fused gate activation + base-2 chunk-local cumsum.  g [B, T, HV, K].
    Returns (g_act or None, g_cum_log2), float32 [B, T, HV, K]."""
    lib = library()
    B, T, HV, K = g.shape
    dev = g.device
    if dev.type != "cuda":
        raise KDARuntimeError(_abi.KDA_ERR_HIP, "gate_chunk_cumsum runs on a HIP device")
    _check_tensor(A_log, "A_log", (HV,), dev, torch.float32)
    _check_tensor(dt_bias, "dt_bias", (HV * K,), dev, torch.float32)
    flags = _flags(use_gate_in_kernel, safe_gate, lower_bound, False, False, False, False)
    qshape = torch.empty((B, T, H or HV, K), dtype=torch.float32, device="meta")
    vshape = torch.empty((B, T, HV, 32), dtype=torch.float32, device="meta")
    bshape = torch.empty((B, T, HV), dtype=torch.float32, device="meta")
    desc = _Desc(qshape, vshape, g, bshape, 1.0, chunk_size, cu_seqlens, lower_bound, flags)
    nbytes = ctypes.c_size_t(0)
    rc = lib.kda_gate_chunk_cumsum_workspace_size(ctypes.byref(desc.d), ctypes.byref(nbytes))
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    cu_dev = None if cu_seqlens is None else cu_seqlens.to(device=dev, dtype=torch.int64).contiguous()
    ws = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=dev)
    g_cum = torch.empty((B, T, HV, K), dtype=torch.float32, device=dev)
    g_act = torch.empty_like(g_cum) if return_activated else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_gate_chunk_cumsum(ctypes.byref(desc.d), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(cu_dev),
                                   _ptr(g_act), _ptr(g_cum), _ptr(ws), ws.numel(), stream)
    if rc != _abi.KDA_OK:
        _raise(rc, lib)
    return g_act, g_cum
