"""State-layout and intermediate-state variants of the KDA forward (GPU).

"flash-linear-attention KDA 内核工程实践…" §2.2 lists two inference-side switches of
chunk_kda: state_v_first / transpose_state_layout (states stored [V, K]) and
return_intermediate_states (the per-chunk states h, "Reading Notes: Implementation
Notes for KDA in FLA" forward step 4, returned for serving engines).

  * transposed layout: o is bit for bit that of the [K, V] layout, and every state
    tensor is the transpose of the [K, V] one, bit for bit (both entry points and
    every recurrence kernel: register-resident bf16, generic bf16 K = 256, fp32);
  * intermediate states: o and final_state are bit for bit those of the plain call;
    h matches the oracle's state at each chunk start (max-abs <= 1e-3 for fp32
    inputs, relative Frobenius <= 2e-2 for bf16); a sequence's first chunk state is
    its initial state exactly.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_log2_amd import chunk_kda, fused_recurrent_kda
from gated_delta_rule_log2_amd.workloads import GVA_BF16, TINY_FP32, TRAINING_BF16, VARLEN_BF16, kernel_kwargs, make_inputs
from tests.oracle_adapter import rel_frobenius, run_oracle, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    # register-resident recurrence (bf16, K <= 128), GVA, initial state, ragged tail
    GVA_BF16.replace(name="gva_small", T=517, H=2, HV=4),
    # packed sequences (one of length 1), chunk 32
    VARLEN_BF16.replace(name="varlen_small_c32", num_seqs=5, min_len=1, max_len=200, H=2, HV=4, chunk=32),
    # generic recurrence, bf16, K = V = 256
    TRAINING_BF16.replace(name="k256_v256", T=150, H=1, HV=2, K=256, V=256, h0="normal0.1"),
    # generic recurrence, fp32
    TINY_FP32.replace(name="tiny_fp32_h0", T=200, h0="normal0.1"),
]


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def call(fn, d, kw, **extra):
    r = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=d["A_log"], dt_bias=d["dt_bias"],
           cu_seqlens=d["cu_seqlens"], **kw, **extra)
    torch.cuda.synchronize()
    return r


def tr(x):
    return None if x is None else x.transpose(-1, -2).contiguous()


def check_close(name, x, ref, fp32):
    x = to_np(x)
    assert np.all(np.isfinite(x)), f"{name}: non-finite"
    if fp32:
        e = float(np.max(np.abs(x - ref)))
        print(f"{name}: max-abs {e:.3e}", flush=True)
        assert e <= 1e-3, f"{name}: max-abs {e:.3e} > 1e-3"
    else:
        e = rel_frobenius(x, ref)
        print(f"{name}: rel-Frobenius {e:.3e}", flush=True)
        assert e <= 2e-2, f"{name}: rel-Frobenius {e:.3e} > 2e-2"


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_transposed_state_layout_chunk(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    d = to_dev(inp)
    h0 = d["initial_state"]
    o, ht = call(chunk_kda, d, kw, initial_state=h0)
    for switch in ("transpose_state_layout", "state_v_first"):
        o2, ht2 = call(chunk_kda, d, kw, initial_state=tr(h0), **{switch: True})
        assert ht2.shape == ht.shape[:-2] + (ht.shape[-1], ht.shape[-2])
        assert torch.equal(o2, o), f"{switch}: output differs from the [K, V] layout"
        assert torch.equal(ht2, tr(ht)), f"{switch}: final state is not the transpose"


@pytest.mark.parametrize("w", CASES[:2] + CASES[3:], ids=[w.name for w in CASES[:2] + CASES[3:]])
def test_transposed_state_layout_recurrent(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    kw.pop("chunk_size")
    d = to_dev(inp)
    h0 = d["initial_state"]
    o, ht = call(fused_recurrent_kda, d, kw, initial_state=h0)
    o2, ht2 = call(fused_recurrent_kda, d, kw, initial_state=tr(h0), transpose_state_layout=True)
    assert torch.equal(o2, o), "output differs from the [K, V] layout"
    assert torch.equal(ht2, tr(ht)), "final state is not the transpose"
    # and against the oracle through the transposed layout
    o_ref, ht_ref = run_oracle(inp, kernel_kwargs(w))
    check_close(f"{w.name} recurrent transposed o", o2, o_ref, w.dtype == torch.float32)
    check_close(f"{w.name} recurrent transposed state", tr(ht2), ht_ref, w.dtype == torch.float32)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_intermediate_states(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    d = to_dev(inp)
    h0 = d["initial_state"]
    o, ht = call(chunk_kda, d, kw, initial_state=h0)
    o2, ht2, h = call(chunk_kda, d, kw, initial_state=h0, return_intermediate_states=True)
    assert torch.equal(o2, o) and torch.equal(ht2, ht), "asking for the states changed o / final_state"
    C = w.chunk
    lens = inp["seq_lens"]
    nch = [(L + C - 1) // C for L in lens]
    HV, K, V = inp["v"].shape[2], inp["q"].shape[3], inp["v"].shape[3]
    if inp["cu_seqlens"] is None:
        assert h.shape == (w.B, nch[0], HV, K, V)
    else:
        assert h.shape == (1, sum(nch), HV, K, V)
    hf = h.reshape(-1, HV, K, V)
    first = np.concatenate([[0], np.cumsum(nch)[:-1]]).astype(int)
    for n in range(len(lens)):
        if nch[n]:
            expect = h0[n] if h0 is not None else torch.zeros_like(hf[0])
            assert torch.equal(hf[first[n]], expect), f"sequence {n}: first chunk state is not the initial state"
    _, _, st_ref = run_oracle(inp, kw, chunk_states=C)
    check_close(f"{w.name} intermediate states", hf, st_ref, w.dtype == torch.float32)
    # the transposed layout gives the transposes, bit for bit
    o3, ht3, h3 = call(chunk_kda, d, kw, initial_state=tr(h0), return_intermediate_states=True,
                       transpose_state_layout=True)
    assert torch.equal(o3, o) and torch.equal(ht3, tr(ht)) and torch.equal(h3, tr(h))


def test_intermediate_states_full_size_sampled_heads():
    """The metric configuration (B=1, T=8192, H=16, HV=32, K=V=128): states of two
    value heads against the oracle, the rest through bitwise invariants."""
    w = GVA_BF16
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    d = to_dev(inp)
    o, ht = call(chunk_kda, d, kw, initial_state=d["initial_state"])
    o2, ht2, h = call(chunk_kda, d, kw, initial_state=d["initial_state"], return_intermediate_states=True)
    assert torch.equal(o2, o) and torch.equal(ht2, ht)
    heads = [3, 30]
    _, _, st_ref = run_oracle(inp, kw, heads=heads, chunk_states=w.chunk)
    check_close("gva_bf16 intermediate states, heads 3 and 30", h[0][:, heads], st_ref, False)


def test_intermediate_states_edges():
    """Empty and chunk-aligned packed segments, and T = 0: a sequence contributes
    ceil(len / chunk) states (none when empty)."""
    w = GVA_BF16.replace(name="states_edges", H=1, HV=2, h0="normal0.1")
    lens = [0, 64, 1, 65, 0, 128, 17]
    inp = make_inputs(w.replace(T=sum(lens)))
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    inp["initial_state"] = 0.1 * torch.randn(len(lens), 2, 128, 128, generator=torch.Generator().manual_seed(7))
    inp["seq_lens"] = lens
    kw = kernel_kwargs(w)
    d = to_dev(inp)
    o, ht, h = call(chunk_kda, d, kw, initial_state=d["initial_state"], return_intermediate_states=True)
    nch = [(L + 63) // 64 for L in lens]
    assert h.shape == (1, sum(nch), 2, 128, 128)
    _, ht_ref, st_ref = run_oracle(inp, kw, chunk_states=64)
    check_close("states_edges intermediate states", h[0], st_ref, False)
    check_close("states_edges final state", ht, ht_ref, False)
    first = np.concatenate([[0], np.cumsum(nch)[:-1]]).astype(int)
    for n, L in enumerate(lens):
        if L:
            assert torch.equal(h[0, first[n]], d["initial_state"][n])
        else:
            assert torch.equal(ht[n], d["initial_state"][n]), "empty segment must keep its state"
    # T = 0: no chunk, no state
    w0 = GVA_BF16.replace(name="T0", H=1, HV=2, T=0, h0="normal0.1")
    inp0 = make_inputs(w0)
    d0 = to_dev(inp0)
    o0, ht0, h0 = call(chunk_kda, d0, kernel_kwargs(w0), initial_state=d0["initial_state"],
                       return_intermediate_states=True)
    assert h0.shape == (1, 0, 2, 128, 128) and o0.shape[1] == 0
    assert torch.equal(ht0, d0["initial_state"])
