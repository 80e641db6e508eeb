"""Glue between chunk_kda keyword arguments and the float64 oracle (tests only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import (
    BETA_AS_GIVEN, BETA_SIGMOID, BETA_TWO_SIGMOID, GATE_LOWER_BOUND, GATE_PRE, GATE_SOFTPLUS,
    oracle_fwd, oracle_gate_cumsum,
)


def oracle_modes(kw: dict):
    if not kw.get("use_gate_in_kernel"):
        gate = GATE_PRE
    elif kw.get("lower_bound") is not None:
        gate = GATE_LOWER_BOUND
    else:
        gate = GATE_SOFTPLUS
    if not kw.get("use_beta_sigmoid_in_kernel"):
        beta = BETA_AS_GIVEN
    else:
        beta = BETA_TWO_SIGMOID if kw.get("allow_neg_eigval") else BETA_SIGMOID
    return gate, beta


def run_oracle(inp: dict, kw: dict, heads=None, nthreads: int = 0, chunk_states: int = 0):
    """Oracle o [B, T, HV', V] and ht [N, HV', K, V] for the value heads in `heads`
    (all heads when None).  Each selected head is evaluated on its own slice of the
    inputs: value head hv with its qk head hv // (HV / H).  With chunk_states = C it
    also returns the state each chunk of C tokens starts from, [chunks, HV', K, V]."""
    q, k, v, g, beta = inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"]
    H, HV = q.shape[2], v.shape[2]
    K = q.shape[3]
    gate, bmode = oracle_modes(kw)
    lb = kw.get("lower_bound") or 0.0
    common = dict(scale=kw["scale"], gate_mode=gate, lower_bound=lb, qk_l2norm=kw.get("use_qk_l2norm_in_kernel", False),
                  beta_mode=bmode, cu_seqlens=inp.get("cu_seqlens"), nthreads=nthreads, chunk_states=chunk_states)
    if heads is None:
        return oracle_fwd(q, k, v, g, beta, A_log=inp.get("A_log"), dt_bias=inp.get("dt_bias"),
                          initial_state=inp.get("initial_state"), **common)
    outs, hts, sts = [], [], []
    group = HV // H
    for hv in heads:
        h = hv // group
        A_log = None if inp.get("A_log") is None else inp["A_log"][hv:hv + 1]
        dt = None if inp.get("dt_bias") is None else inp["dt_bias"][hv * K:(hv + 1) * K]
        h0 = None if inp.get("initial_state") is None else inp["initial_state"][:, hv:hv + 1]
        r = oracle_fwd(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, hv:hv + 1], g[:, :, hv:hv + 1],
                       beta[:, :, hv:hv + 1], A_log=A_log, dt_bias=dt, initial_state=h0, **common)
        outs.append(r[0])
        hts.append(r[1])
        if chunk_states:
            sts.append(r[2])
    if chunk_states:
        return np.concatenate(outs, axis=2), np.concatenate(hts, axis=1), np.concatenate(sts, axis=1)
    return np.concatenate(outs, axis=2), np.concatenate(hts, axis=1)


def run_oracle_gate(inp: dict, kw: dict, chunk: int):
    gate, _ = oracle_modes(kw)
    return oracle_gate_cumsum(inp["g"], chunk_size=chunk, gate_mode=gate, lower_bound=kw.get("lower_bound") or 0.0,
                              A_log=inp.get("A_log"), dt_bias=inp.get("dt_bias"), cu_seqlens=inp.get("cu_seqlens"))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_frobenius(x: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))
