"""ctypes wrapper of the float64 C oracle -- TEST INFRASTRUCTURE ONLY.

Every input is widened to float64 from exactly the values stored in the tensors
the GPU path receives (bf16 and fp32 widen exactly), so both sides see the same
numbers.  Nothing here computes any part of the method: the arithmetic is all in
``kda_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GATE_PRE, GATE_SOFTPLUS, GATE_LOWER_BOUND = 0, 1, 2
BETA_AS_GIVEN, BETA_SIGMOID, BETA_TWO_SIGMOID = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "libkda_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_ubyte)


def build_oracle(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", source, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_cache: dict[str, ctypes.CDLL] = {}


def load_oracle(path: str = LIBRARY) -> ctypes.CDLL:
    if path in _cache:
        return _cache[path]
    if not os.path.exists(path):
        if path != LIBRARY:
            raise FileNotFoundError(path)
        build_oracle()
    lib = ctypes.CDLL(path)
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [
        ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        _dp, _dp, _dp, _u8p, ctypes.c_int,
    ]
    lib.kda_oracle_fwd_states.restype = ctypes.c_int
    lib.kda_oracle_fwd_states.argtypes = [
        ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        _dp, _dp, _dp, ctypes.c_int, _i64p, _dp, ctypes.c_int,
    ]
    lib.kda_oracle_gate_cumsum.restype = ctypes.c_int
    lib.kda_oracle_gate_cumsum.argtypes = [
        ctypes.c_int, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _dp, _dp, _dp, ctypes.c_int, ctypes.c_double, _dp, _dp,
    ]
    lib.kda_oracle_num_threads.restype = ctypes.c_int
    lib.kda_oracle_num_threads.argtypes = [ctypes.c_int]
    _cache[path] = lib
    return lib


def _f64(x):
    """Widen a torch tensor / array to a contiguous float64 numpy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (imported lazily so numpy-only use works)
        import torch

        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, typ=_dp):
    return None if a is None else a.ctypes.data_as(typ)


def _seq_starts(T_total: int, B: int, T: int, cu_seqlens):
    if cu_seqlens is not None:
        cs = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
        return np.ascontiguousarray(cs)
    return np.arange(0, B * T + 1, T, dtype=np.int64) if T > 0 else np.zeros(B + 1, np.int64)


def oracle_num_threads(requested: int = 0, lib_path: str = LIBRARY) -> int:
    return load_oracle(lib_path).kda_oracle_num_threads(requested)


def oracle_fwd(q, k, v, g, beta, *, scale: float, gate_mode: int = GATE_PRE,
               lower_bound: float = 0.0, A_log=None, dt_bias=None, qk_l2norm: bool = False,
               beta_mode: int = BETA_AS_GIVEN, initial_state=None, cu_seqlens=None,
               unit_mask=None, nthreads: int = 0, chunk_states: int = 0, lib_path: str = LIBRARY):
    """Token-by-token float64 forward.

    q, k: [B, T, H, K]; v: [B, T, HV, V]; g: [B, T, HV, K]; beta: [B, T, HV].
    With cu_seqlens ([N+1], B must be 1) the token axis holds N sequences.
    Returns (o [B, T, HV, V], ht [N, HV, K, V]) as float64 numpy arrays.  With
    chunk_states = C > 0 it also returns the state each chunk of C tokens starts
    from, [total chunks, HV, K, V] (chunks restart at every sequence start;
    sequence n's chunks follow those of sequences 0..n-1); unit_mask is then not
    supported.
    """
    q, k, v, g, beta = (_f64(t) for t in (q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    starts = _seq_starts(B * T, B, T, cu_seqlens)
    N = len(starts) - 1
    A_log, dt_bias, h0 = _f64(A_log), _f64(dt_bias), _f64(initial_state)
    mask = None
    if unit_mask is not None:
        mask = np.ascontiguousarray(np.asarray(unit_mask, dtype=np.uint8).reshape(N * HV))
    o = np.zeros((B, T, HV, V), np.float64)
    ht = np.zeros((N, HV, K, V), np.float64)
    lib = load_oracle(lib_path)
    head = (N, _ptr(starts, _i64p), H, HV, K, V,
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
            int(gate_mode), float(lower_bound), int(bool(qk_l2norm)), int(beta_mode), float(scale),
            _ptr(h0), _ptr(o), _ptr(ht))
    if chunk_states:
        if mask is not None:
            raise ValueError("chunk_states and unit_mask cannot be combined")
        lens = np.diff(starts)
        nchunks = (lens + chunk_states - 1) // chunk_states
        first = np.ascontiguousarray(np.concatenate([[0], np.cumsum(nchunks)[:-1]]).astype(np.int64))
        states = np.zeros((int(nchunks.sum()), HV, K, V), np.float64)
        rc = lib.kda_oracle_fwd_states(*head, int(chunk_states), _ptr(first, _i64p), _ptr(states), int(nthreads))
        if rc < 0:
            raise ValueError("oracle rejected its arguments")
        return o, ht, states
    rc = lib.kda_oracle_fwd(*head, _ptr(mask, _u8p), int(nthreads))
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    return o, ht


def oracle_gate_cumsum(g, *, chunk_size: int, gate_mode: int, lower_bound: float = 0.0,
                       A_log=None, dt_bias=None, cu_seqlens=None, lib_path: str = LIBRARY):
    """Activated gate and its chunk-local inclusive cumsum, natural-log units.

    g: [B, T, HV, K].  Returns (g_act, g_cum), both float64 [B, T, HV, K].
    """
    g = _f64(g)
    B, T, HV, K = g.shape
    starts = _seq_starts(B * T, B, T, cu_seqlens)
    N = len(starts) - 1
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    g_act = np.zeros_like(g)
    g_cum = np.zeros_like(g)
    lib = load_oracle(lib_path)
    rc = lib.kda_oracle_gate_cumsum(
        N, _ptr(starts, _i64p), HV, K, int(chunk_size), _ptr(g), _ptr(A_log), _ptr(dt_bias),
        int(gate_mode), float(lower_bound), _ptr(g_act), _ptr(g_cum),
    )
    if rc < 0:
        raise ValueError("oracle rejected its arguments")
    return g_act, g_cum
