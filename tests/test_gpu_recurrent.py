"""Parity of the token-by-token entry (kda_fused_recurrent_fwd) with the float64 oracle.

The oracle is itself the token recurrence, so this compares like with like; bars as
for the chunk path: fp32 inputs max-abs <= 1e-3, bf16 inputs relative Frobenius
<= 2e-2 on o and final_state.  Also checks that the recurrent and chunk entries agree
and that a packed batch equals its segments run one by one, bit for bit.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_log2_amd import chunk_kda, fused_recurrent_kda
from gated_delta_rule_log2_amd.workloads import (
    GVA_BF16, LONG_BF16, TINY_FP32, TRAINING_BF16, VARLEN_BF16, kernel_kwargs, make_inputs,
)
from tests.oracle_adapter import rel_frobenius, run_oracle, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_rec(inp, kw):
    kw = {k: v for k, v in kw.items() if k != "chunk_size"}
    d = to_dev(inp)
    o, ht = fused_recurrent_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=d["A_log"],
                                dt_bias=d["dt_bias"], initial_state=d["initial_state"],
                                cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, ht


def check(name, o, ht, o_ref, ht_ref, fp32):
    o_np, ht_np = to_np(o), to_np(ht)
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(ht_np)), f"{name}: non-finite output"
    if fp32:
        eo, eh = np.max(np.abs(o_np - o_ref)), np.max(np.abs(ht_np - ht_ref))
        print(f"{name}: max-abs o {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= 1e-3 and eh <= 1e-3, f"{name}: max-abs o {eo:.3e} state {eh:.3e} > 1e-3"
    else:
        eo, eh = rel_frobenius(o_np, o_ref), rel_frobenius(ht_np, ht_ref)
        print(f"{name}: rel-Frobenius o {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= 2e-2 and eh <= 2e-2, f"{name}: rel-Frobenius o {eo:.3e} state {eh:.3e} > 2e-2"


CASES = [
    TINY_FP32.replace(name="rec_tiny_fp32", T=96),
    TINY_FP32.replace(name="rec_fp32_k128_gva_h0", T=37, H=1, HV=2, K=128, V=128, h0="normal0.1"),
    TRAINING_BF16.replace(name="rec_training", T=80, H=2, HV=2),
    GVA_BF16.replace(name="rec_gva_decode", B=8, T=1, H=2, HV=4),
    GVA_BF16.replace(name="rec_gva", T=120, H=2, HV=4),
    VARLEN_BF16.replace(name="rec_varlen", num_seqs=5, min_len=1, max_len=60, H=2, HV=4),
    LONG_BF16.replace(name="rec_pregated", T=90, H=1, HV=2),
    TRAINING_BF16.replace(name="rec_k256_v64", T=40, H=1, HV=2, K=256, V=64),
    TRAINING_BF16.replace(name="rec_k32_v256", T=40, H=1, HV=1, K=32, V=256),
    TRAINING_BF16.replace(name="rec_softplus", T=70, H=2, HV=2, safe_gate=False, lower_bound=None),
    TRAINING_BF16.replace(name="rec_lb_no_alog", T=50, H=1, HV=2, a_log="none", safe_gate=False,
                          lower_bound=-2.0),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_recurrent_parity(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    o, ht = run_rec(inp, kw)
    o_ref, ht_ref = run_oracle(inp, kw)
    check(w.name, o, ht, o_ref, ht_ref, w.dtype == torch.float32)


def test_recurrent_matches_chunk():
    """Both entries compute the same operator: on one input their results agree to
    the bf16 bar against each other."""
    w = GVA_BF16.replace(name="rec_vs_chunk", T=200, H=2, HV=4)
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    o_r, ht_r = run_rec(inp, kw)
    d = to_dev(inp)
    o_c, ht_c = chunk_kda(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                          initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    assert rel_frobenius(to_np(o_r), to_np(o_c)) <= 2e-2
    assert rel_frobenius(to_np(ht_r), to_np(ht_c)) <= 2e-2


def test_recurrent_empty_and_packed_bitwise():
    """T = 0 returns the initial state; a packed batch with empty and one-token
    segments equals each segment run on its own, bit for bit."""
    w = GVA_BF16.replace(name="rec_T0", H=1, HV=2, T=0, h0="normal0.1")
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    o, ht = run_rec(inp, kernel_kwargs(w))
    assert o.shape[1] == 0
    assert torch.equal(ht.cpu(), inp["initial_state"].float())

    w = VARLEN_BF16.replace(name="rec_packed", num_seqs=4, min_len=0, max_len=40, H=1, HV=2, h0="normal0.1")
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    o, ht = run_rec(inp, kw)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        seg = {k: v for k, v in inp.items()}
        for key in ("q", "k", "v", "g", "beta"):
            seg[key] = inp[key][:, a:b].contiguous()
        seg["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        seg["cu_seqlens"] = None
        o1, ht1 = run_rec(seg, kw)
        assert torch.equal(o[:, a:b].cpu(), o1.cpu()), f"segment {n} output differs from its standalone run"
        assert torch.equal(ht[n:n + 1].cpu(), ht1.cpu()), f"segment {n} state differs from its standalone run"
