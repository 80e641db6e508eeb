"""Seeded synthetic inputs for the KDA forward workloads.

This module only draws random inputs: it holds none of the method's arithmetic
and is the one piece of code that both the HIP path and the float64 oracle
consume.  Every tensor is drawn on the CPU with ``torch.Generator`` seeded per
workload, in float32, then stored in the workload's dtype (bf16 uses
round-to-nearest-even).  Both sides read exactly those stored values.

Draw order: sequence lengths (packed workload only), q, k, v, beta, g, A_log,
dt_bias, initial state.  "N(0, s)" means standard deviation s.

A few inputs are *distribution definitions* rather than raw normals: the tiny
fp32 workload's q/k are uniform on the unit sphere (normal draws divided by
their norm) and its beta is logit-normal (sigmoid of a normal draw); the
long-context workload's g is minus the softplus of a normal draw.  They are
produced with torch library functions here, before either side sees them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    chunk: int
    dtype: torch.dtype                   # q, k, v (and o)
    g_dtype: torch.dtype
    beta_dtype: torch.dtype
    seed: int
    qk_l2norm: bool = False
    beta_sigmoid: bool = False
    allow_neg_eigval: bool = False
    gate_in_kernel: bool = False
    safe_gate: bool = False
    lower_bound: Optional[float] = None
    a_log: str = "none"                  # "none" | "zero" | "normal"
    dt_bias: str = "none"                # "none" | "zero" | "normal0.5"
    h0: str = "none"                     # "none" | "normal0.1"
    output_final_state: bool = True
    host_unit_qk: bool = False           # q, k drawn on the unit sphere
    host_beta_logit_normal: bool = False  # beta = sigmoid(N(0,1)) drawn as given
    pregated_softplus: bool = False      # g = -softplus(N(0,1)), fp32 log space
    num_seqs: int = 0                    # > 0: packed with cu_seqlens, B must be 1
    min_len: int = 64
    max_len: int = 8192

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.K)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY_FP32 = Workload(
    "tiny_fp32", B=1, T=256, H=2, HV=2, K=64, V=64, chunk=64, dtype=torch.float32,
    g_dtype=torch.float32, beta_dtype=torch.float32, seed=0, gate_in_kernel=True,
    a_log="zero", dt_bias="zero", host_unit_qk=True, host_beta_logit_normal=True)

TRAINING_BF16 = Workload(
    "training_bf16", B=2, T=2048, H=16, HV=16, K=128, V=128, chunk=64, dtype=torch.bfloat16,
    g_dtype=torch.bfloat16, beta_dtype=torch.bfloat16, seed=1, qk_l2norm=True, beta_sigmoid=True,
    gate_in_kernel=True, safe_gate=True, lower_bound=-5.0, a_log="normal", dt_bias="normal0.5")

GVA_BF16 = TRAINING_BF16.replace(
    name="gva_bf16", B=1, T=8192, H=16, HV=32, seed=2, h0="normal0.1")

VARLEN_BF16 = GVA_BF16.replace(name="varlen_bf16", T=0, seed=3, num_seqs=16)

LONG_BF16 = Workload(
    "long_bf16", B=1, T=131072, H=32, HV=32, K=128, V=128, chunk=64, dtype=torch.bfloat16,
    g_dtype=torch.float32, beta_dtype=torch.bfloat16, seed=4, qk_l2norm=True, beta_sigmoid=True,
    allow_neg_eigval=True, pregated_softplus=True)

# one decoding step of 64 sequences with the metric configuration's heads: the state of
# every (sequence, value head) is read and written once (the token-by-token entry)
DECODE_BF16 = GVA_BF16.replace(name="decode_bf16", B=64, T=1, seed=5)

WORKLOADS = {w.name: w for w in (TINY_FP32, TRAINING_BF16, GVA_BF16, VARLEN_BF16, LONG_BF16, DECODE_BF16)}


def _normal(gen, shape, std=1.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def make_inputs(w: Workload) -> dict:
    """Draw one workload's inputs on the CPU.  Returns a dict with q, k, v, g, beta,
    A_log, dt_bias, initial_state, cu_seqlens (int64 or None) and seq_lens."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    cu = None
    lens = None
    B, T = w.B, w.T
    if w.num_seqs > 0:
        lens = torch.randint(w.min_len, w.max_len + 1, (w.num_seqs,), generator=gen).tolist()
        B, T = 1, int(sum(lens))
        cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int64)
    N = w.num_seqs if w.num_seqs > 0 else B

    q = _normal(gen, (B, T, w.H, w.K))
    k = _normal(gen, (B, T, w.H, w.K))
    if w.host_unit_qk:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    v = _normal(gen, (B, T, w.HV, w.V))
    beta = _normal(gen, (B, T, w.HV))
    if w.host_beta_logit_normal:
        beta = torch.sigmoid(beta)
    g = _normal(gen, (B, T, w.HV, w.K))
    if w.pregated_softplus:
        g = -torch.nn.functional.softplus(g)
    A_log = None
    if w.a_log == "zero":
        A_log = torch.zeros(w.HV, dtype=torch.float32)
    elif w.a_log == "normal":
        A_log = _normal(gen, (w.HV,))
    dt_bias = None
    if w.dt_bias == "zero":
        dt_bias = torch.zeros(w.HV * w.K, dtype=torch.float32)
    elif w.dt_bias == "normal0.5":
        dt_bias = _normal(gen, (w.HV * w.K,), 0.5)
    h0 = None
    if w.h0 == "normal0.1":
        h0 = _normal(gen, (N, w.HV, w.K, w.V), 0.1)

    return dict(
        q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype), beta=beta.to(w.beta_dtype),
        g=g.to(w.g_dtype), A_log=A_log, dt_bias=dt_bias, initial_state=h0, cu_seqlens=cu,
        seq_lens=lens if lens is not None else [T] * B,
    )


def kernel_kwargs(w: Workload) -> dict:
    """Keyword arguments of ``chunk_kda`` (and of the oracle wrapper's flags) that
    the workload's recipe fixes."""
    return dict(
        scale=w.scale, chunk_size=w.chunk, use_qk_l2norm_in_kernel=w.qk_l2norm,
        use_gate_in_kernel=w.gate_in_kernel, safe_gate=w.safe_gate, lower_bound=w.lower_bound,
        use_beta_sigmoid_in_kernel=w.beta_sigmoid, allow_neg_eigval=w.allow_neg_eigval,
        output_final_state=w.output_final_state,
    )


def token_count(w: Workload, inputs: dict) -> int:
    return int(inputs["q"].shape[0] * inputs["q"].shape[1])
