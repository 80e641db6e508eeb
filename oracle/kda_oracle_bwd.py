"""Float64 gradients of the KDA forward -- TEST INFRASTRUCTURE ONLY.

Nothing in the library imports this module; only tests (and the benchmark's CPU
baseline) may.

The backward of the chunked forward ("Reading Notes: Implementation Notes for KDA in
FLA", backward steps 1-7) computes, up to rounding order, the vector-Jacobian product
of the forward map: given dL/do (and dL/d final_state), the gradients of
L = <do, o> + <dht, ht> with respect to q, k, v, g, beta, A_log, dt_bias and
initial_state.  This oracle is that definition written out: the token recurrence of
the method, in float64 with plain torch CPU tensor operations (the same contract as
kda_oracle.c: gate forms, beta forms, optional L2 norm of q and k, GVA head groups,
packed sequences), differentiated by torch.autograd.  No chunking, no WY
factorisation, no reordering.

What pins it (tests/test_oracle_bwd.py): this forward equals the C oracle's to
rounding; every gradient matches central finite differences of the C oracle's
forward on small inputs; a zero-decay, zero-beta case has closed-form gradients.
"""
from __future__ import annotations

import numpy as np
import torch

GATE_PRE, GATE_SOFTPLUS, GATE_LOWER_BOUND = 0, 1, 2
BETA_AS_GIVEN, BETA_SIGMOID, BETA_TWO_SIGMOID = 0, 1, 2

_F64 = torch.float64


def _t(x, requires_grad=False):
    """A float64 CPU copy of a tensor or array (a leaf of the graph when asked)."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        t = x.detach().to("cpu", _F64).clone()
    else:
        t = torch.tensor(np.asarray(x, dtype=np.float64))
    if requires_grad:
        t.requires_grad_(True)
    return t


def gate_activate(g, gate_mode, lower_bound, A_log, dt_bias, hv_axis_len):
    """Natural-log gate for g [Ttot, HV, K] ("flash-linear-attention KDA 内核工程实践…",
    §2: pre-gated, or -exp(A_log) softplus(g + dt_bias), or, with a lower bound,
    lower_bound * sigmoid(exp(A_log) (g + dt_bias)), exp(A_log) taken as 1 without A_log)."""
    if gate_mode == GATE_PRE:
        return g
    x = g + dt_bias.reshape(1, hv_axis_len, -1) if dt_bias is not None else g
    if gate_mode == GATE_SOFTPLUS:
        return -torch.exp(A_log).reshape(1, -1, 1) * torch.nn.functional.softplus(x)
    a = torch.exp(A_log).reshape(1, -1, 1) if A_log is not None else 1.0
    return lower_bound * torch.sigmoid(a * x)


def beta_activate(beta, beta_mode):
    if beta_mode == BETA_SIGMOID:
        return torch.sigmoid(beta)
    if beta_mode == BETA_TWO_SIGMOID:
        return 2.0 * torch.sigmoid(beta)
    return beta


def _normalise(x, on):
    """x / sqrt(sum x^2 + 1e-6) over the key axis when asked."""
    if not on:
        return x
    return x * torch.rsqrt((x * x).sum(-1, keepdim=True) + 1e-6)


def forward(q, k, v, g, beta, *, scale, gate_mode=GATE_PRE, lower_bound=0.0, A_log=None, dt_bias=None,
            qk_l2norm=False, beta_mode=BETA_AS_GIVEN, initial_state=None, seq_starts=None):
    """Token recurrence on flattened tensors (differentiable, float64).

    q, k [Ttot, H, K]; v [Ttot, HV, V]; g [Ttot, HV, K]; beta [Ttot, HV];
    seq_starts [N + 1] token offsets.  Per value head hv (qk head hv // (HV / H)):
      S <- Diag(exp g') S;  u = S^T k^;  S <- S + b k^ (v - u)^T;  o = S^T q^
    Returns o [Ttot, HV, V] and the final states [N, HV, K, V].
    """
    Ttot, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    group = HV // H
    head_of = torch.arange(HV) // group
    qn = _normalise(q, qk_l2norm) * scale
    kn = _normalise(k, qk_l2norm)
    qh, kh = qn[:, head_of, :], kn[:, head_of, :]  # [Ttot, HV, K]
    alpha = torch.exp(gate_activate(g, gate_mode, lower_bound, A_log, dt_bias, HV))
    b = beta_activate(beta, beta_mode)
    outs, finals = [], []
    N = len(seq_starts) - 1
    for n in range(N):
        S = initial_state[n] if initial_state is not None else torch.zeros(HV, K, V, dtype=_F64)
        for t in range(int(seq_starts[n]), int(seq_starts[n + 1])):
            S = S * alpha[t].unsqueeze(-1)
            u = torch.einsum("hkv,hk->hv", S, kh[t])
            S = S + (b[t].reshape(HV, 1, 1) * kh[t].unsqueeze(-1)) * (v[t] - u).unsqueeze(1)
            outs.append(torch.einsum("hkv,hk->hv", S, qh[t]))
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros(0, HV, V, dtype=_F64)
    ht = torch.stack(finals) if finals else torch.zeros(0, HV, K, V, dtype=_F64)
    return o, ht


def _starts(B, T, cu_seqlens):
    if cu_seqlens is not None:
        cs = cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens
        return np.asarray(cs, dtype=np.int64)
    return np.arange(0, B * T + 1, T, dtype=np.int64) if T > 0 else np.zeros(B + 1, np.int64)


def oracle_fwd_torch(q, k, v, g, beta, *, scale, gate_mode=GATE_PRE, lower_bound=0.0, A_log=None,
                     dt_bias=None, qk_l2norm=False, beta_mode=BETA_AS_GIVEN, initial_state=None,
                     cu_seqlens=None):
    """The differentiable forward on batch-shaped inputs ([B, T, ...], as oracle_fwd
    in kda_oracle.py takes them); returns float64 numpy (o [B, T, HV, V], ht [N, HV, K, V])."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    starts = _starts(B, T, cu_seqlens)
    with torch.no_grad():
        o, ht = forward(_t(q).reshape(B * T, H, K), _t(k).reshape(B * T, H, K), _t(v).reshape(B * T, HV, V),
                        _t(g).reshape(B * T, HV, K), _t(beta).reshape(B * T, HV), scale=scale,
                        gate_mode=gate_mode, lower_bound=lower_bound, A_log=_t(A_log), dt_bias=_t(dt_bias),
                        qk_l2norm=qk_l2norm, beta_mode=beta_mode, initial_state=_t(initial_state),
                        seq_starts=starts)
    return o.reshape(B, T, HV, V).numpy(), ht.numpy()


def oracle_bwd(q, k, v, g, beta, do, *, scale, dht=None, gate_mode=GATE_PRE, lower_bound=0.0, A_log=None,
               dt_bias=None, qk_l2norm=False, beta_mode=BETA_AS_GIVEN, initial_state=None, cu_seqlens=None):
    """Gradients of L = <do, o> + <dht, ht> (float64 numpy arrays, input shapes).

    q, k [B, T, H, K]; v [B, T, HV, V]; g [B, T, HV, K]; beta [B, T, HV];
    do [B, T, HV, V]; dht [N, HV, K, V] or None.  Returns a dict with dq, dk, dv,
    dg, dbeta, and dA_log / ddt_bias / dh0 when those inputs are given.
    """
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    starts = _starts(B, T, cu_seqlens)
    leaves = {
        "q": _t(q, True), "k": _t(k, True), "v": _t(v, True), "g": _t(g, True), "beta": _t(beta, True),
        "A_log": _t(A_log, True), "dt_bias": _t(dt_bias, True), "h0": _t(initial_state, True),
    }
    o, ht = forward(leaves["q"].reshape(B * T, H, K), leaves["k"].reshape(B * T, H, K),
                    leaves["v"].reshape(B * T, HV, V), leaves["g"].reshape(B * T, HV, K),
                    leaves["beta"].reshape(B * T, HV), scale=scale, gate_mode=gate_mode,
                    lower_bound=lower_bound, A_log=leaves["A_log"], dt_bias=leaves["dt_bias"],
                    qk_l2norm=qk_l2norm, beta_mode=beta_mode, initial_state=leaves["h0"], seq_starts=starts)
    loss = (o.reshape(B, T, HV, V) * _t(do)).sum()
    if dht is not None:
        loss = loss + (ht * _t(dht)).sum()
    want = {name: t for name, t in leaves.items() if t is not None}
    grads = torch.autograd.grad(loss, list(want.values()), allow_unused=True)
    out = {}
    for (name, t), gr in zip(want.items(), grads):
        gr = torch.zeros_like(t) if gr is None else gr
        out["d" + name] = gr.detach().numpy()
    return out
