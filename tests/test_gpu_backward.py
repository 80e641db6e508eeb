"""Backward of chunk_kda on the GPU against the float64 backward oracle.

Every gradient (dq, dk, dv, dg, dbeta, dA_log, dt_bias, dh0) is compared element by
element on the same seeded inputs.  Tolerance (relative Frobenius norm of the error):
1e-3 for fp32 inputs, whose forward states carry fp32 rounding only; 2e-2 for bf16
inputs, the forward's own bar, since the states the backward starts from come from
the bf16 chunked forward.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_log2_amd import KDAContractError, chunk_kda, chunk_kda_bwd
from gated_delta_rule_log2_amd.workloads import (GVA_BF16, LONG_BF16, TINY_FP32, TRAINING_BF16, VARLEN_BF16, kernel_kwargs,
                                                make_inputs)
from oracle.kda_oracle_bwd import oracle_bwd
from tests.oracle_adapter import oracle_modes, rel_frobenius, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    TINY_FP32.replace(name="bwd_tiny_fp32_h0", T=150, h0="normal0.1"),
    TINY_FP32.replace(name="bwd_fp32_k128_c32", T=97, H=1, HV=2, K=128, V=64, chunk=32),
    GVA_BF16.replace(name="bwd_gva_bf16", T=200, H=2, HV=4),
    VARLEN_BF16.replace(name="bwd_varlen_bf16", num_seqs=4, min_len=1, max_len=120, H=1, HV=2, K=64, V=64),
    TRAINING_BF16.replace(name="bwd_softplus_bf16", T=130, H=1, HV=2, K=64, V=32, safe_gate=False, lower_bound=None),
    TRAINING_BF16.replace(name="bwd_k256_bf16", T=70, H=1, HV=1, K=256, V=64),
    LONG_BF16.replace(name="bwd_pregated_negeig", T=100, H=1, HV=2, K=64, V=64),
    VARLEN_BF16.replace(name="bwd_varlen_c32_k96_v32", num_seqs=3, min_len=20, max_len=90, H=1, HV=3, K=96, V=32,
                        chunk=32),
    TINY_FP32.replace(name="bwd_fp32_gva3_k32", T=77, H=1, HV=3, K=32, V=96, h0="normal0.1"),
    # the two-wave per-chunk kernel at chunk 32, and the one-wave form at K = 32
    VARLEN_BF16.replace(name="bwd_varlen_c32_k128", num_seqs=3, min_len=10, max_len=80, H=1, HV=2, K=128, V=64,
                        chunk=32),
    GVA_BF16.replace(name="bwd_gva_bf16_k32", T=90, H=1, HV=2, K=32, V=64),
]


def gpu_grads(inp, kw, do, dht, tokenwise=False):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = chunk_kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do.to(DEV),
                        dht=None if dht is None else dht.to(DEV), A_log=d["A_log"], dt_bias=d["dt_bias"],
                        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], tokenwise=tokenwise, **kw)
    torch.cuda.synchronize()
    return out


def oracle_grads(inp, kw, do, dht):
    gate, bmode = oracle_modes(kw)
    return oracle_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], do, dht=dht, scale=kw["scale"],
                      gate_mode=gate, lower_bound=kw.get("lower_bound") or 0.0, A_log=inp.get("A_log"),
                      dt_bias=inp.get("dt_bias"), qk_l2norm=kw.get("use_qk_l2norm_in_kernel", False),
                      beta_mode=bmode, initial_state=inp.get("initial_state"), cu_seqlens=inp.get("cu_seqlens"))


def cotangents(inp, seed=11):
    gen = torch.Generator().manual_seed(seed)
    v = inp["v"]
    N = len(inp["seq_lens"])
    HV, K, V = v.shape[2], inp["q"].shape[3], v.shape[3]
    do = torch.randn(v.shape, generator=gen).to(v.dtype)
    dht = 0.5 * torch.randn((N, HV, K, V), generator=gen)
    return do, dht


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_parity(w):
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    do, dht = cotangents(inp)
    got = gpu_grads(inp, kw, do, dht)
    ref = oracle_grads(inp, kw, do, dht)
    tol = 1e-3 if w.dtype == torch.float32 else 2e-2
    names = {"dq": "dq", "dk": "dk", "dv": "dv", "dg": "dg", "dbeta": "dbeta", "dh0": "dh0",
             "dA_log": "dA_log", "ddt_bias": "ddt_bias"}
    for key, rkey in names.items():
        if rkey not in ref and key == "dh0":
            rkey = None
        if key not in got:
            continue
        x = to_np(got[key])
        assert np.all(np.isfinite(x)), f"{w.name} {key}: non-finite"
        if rkey is None:  # no initial state given: the oracle has no leaf for it
            continue
        r = ref[rkey].reshape(x.shape)
        e = rel_frobenius(x, r)
        print(f"{w.name} {key}: rel-Frobenius {e:.3e}", flush=True)
        assert e <= tol, f"{w.name} {key}: rel-Frobenius {e:.3e} > {tol}"


CROSS = [w for w in CASES if w.name in ("bwd_tiny_fp32_h0", "bwd_gva_bf16", "bwd_varlen_c32_k96_v32",
                                        "bwd_pregated_negeig")]


@pytest.mark.parametrize("w", CROSS, ids=[w.name for w in CROSS])
def test_chunked_matches_tokenwise(w):
    """The chunked backward against the token-level form (kda_chunk_bwd_tokenwise, fp32
    token steps from the same chunk-start states) on the GPU: 1e-4 for fp32 inputs
    (both sides fp32 throughout); 2e-2 for bf16 inputs, where the chunked form's
    operands are the forward's bf16 intermediates."""
    print(f"case {w.name}", flush=True)
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    do, dht = cotangents(inp)
    got = gpu_grads(inp, kw, do, dht)
    ref = gpu_grads(inp, kw, do, dht, tokenwise=True)
    tol = 1e-4 if w.dtype == torch.float32 else 2e-2
    for key in got:
        e = rel_frobenius(to_np(got[key]), to_np(ref[key]))
        print(f"{w.name} {key}: chunked vs token-level {e:.3e}", flush=True)
        assert e <= tol, f"{w.name} {key}: chunked vs token-level {e:.3e} > {tol}"


def test_chunked_matches_tokenwise_full_size():
    """The metric configuration (B=1, T=8192, H=16, HV=32, K=V=128) in the benchmark's
    launch configuration: every gradient of every head, chunked against the token-level
    form."""
    w = GVA_BF16
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    do, dht = cotangents(inp)
    got = gpu_grads(inp, kw, do, dht)
    ref = gpu_grads(inp, kw, do, dht, tokenwise=True)
    for key in got:
        x, r = got[key].float(), ref[key].float()
        assert torch.isfinite(x).all(), f"{key}: non-finite"
        e = (torch.linalg.vector_norm(x - r) / torch.linalg.vector_norm(r)).item()
        print(f"full size {key}: chunked vs token-level {e:.3e}", flush=True)
        assert e <= 2e-2, f"full size {key}: chunked vs token-level {e:.3e}"


def test_backward_edges():
    """Empty and chunk-aligned packed segments (an empty one passes dht straight to
    dh0), and T = 0 (only dh0 = dht)."""
    w = GVA_BF16.replace(name="bwd_edges", H=1, HV=2, K=64, V=64, h0="normal0.1")
    lens = [0, 64, 1, 65, 0, 17]
    inp = make_inputs(w.replace(T=sum(lens)))
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    inp["initial_state"] = 0.1 * torch.randn(len(lens), 2, 64, 64, generator=torch.Generator().manual_seed(7))
    inp["seq_lens"] = lens
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    do, dht = cotangents(inp)
    got = gpu_grads(inp, kw, do, dht)
    ref = oracle_grads(inp, kw, do, dht)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0", "dA_log", "ddt_bias"):
        x = to_np(got[key])
        e = rel_frobenius(x, ref[key].reshape(x.shape))
        print(f"bwd_edges {key}: rel-Frobenius {e:.3e}", flush=True)
        assert e <= 2e-2, f"bwd_edges {key}: rel-Frobenius {e:.3e}"
    for n, L in enumerate(lens):
        if L == 0:
            assert torch.equal(got["dh0"][n].cpu(), dht[n]), "empty segment: dh0 must equal dht"
    w0 = GVA_BF16.replace(name="bwd_T0", H=1, HV=2, K=64, V=64, T=0, h0="normal0.1")
    inp0 = make_inputs(w0)
    kw0 = kernel_kwargs(w0)
    kw0.pop("output_final_state", None)
    do0, dht0 = cotangents(inp0)
    got0 = gpu_grads(inp0, kw0, do0, dht0)
    assert torch.equal(got0["dh0"].cpu(), dht0) and got0["dq"].shape[1] == 0


def test_backward_full_size_sampled_heads():
    """The metric configuration (B=1, T=8192, H=16, HV=32, K=V=128), in the launch
    configuration the benchmark times: every gradient of value heads 6 and 7 (one GVA
    group, so dq and dk of qk head 3 are complete) against the oracle run on those heads
    alone."""
    w = GVA_BF16
    inp = make_inputs(w)
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    do, dht = cotangents(inp)
    got = gpu_grads(inp, kw, do, dht)
    heads, h = [6, 7], 3
    K = inp["q"].shape[3]
    sub = dict(inp)
    sub["q"], sub["k"] = inp["q"][:, :, h:h + 1], inp["k"][:, :, h:h + 1]
    for name in ("v", "g", "beta"):
        sub[name] = inp[name][:, :, heads[0]:heads[-1] + 1]
    sub["A_log"] = inp["A_log"][heads[0]:heads[-1] + 1]
    sub["dt_bias"] = inp["dt_bias"][heads[0] * K:(heads[-1] + 1) * K]
    sub["initial_state"] = inp["initial_state"][:, heads[0]:heads[-1] + 1]
    ref = oracle_grads(sub, kw, do[:, :, heads[0]:heads[-1] + 1], dht[:, heads[0]:heads[-1] + 1])
    hs = slice(heads[0], heads[-1] + 1)
    pairs = {
        "dq": got["dq"][:, :, h:h + 1], "dk": got["dk"][:, :, h:h + 1], "dv": got["dv"][:, :, hs],
        "dg": got["dg"][:, :, hs], "dbeta": got["dbeta"][:, :, hs], "dh0": got["dh0"][:, hs],
        "dA_log": got["dA_log"][hs], "ddt_bias": got["ddt_bias"][heads[0] * K:(heads[-1] + 1) * K],
    }
    for key, x in pairs.items():
        xn = to_np(x)
        e = rel_frobenius(xn, ref[key].reshape(xn.shape))
        print(f"gva_bf16 full size, heads 6-7, {key}: rel-Frobenius {e:.3e}", flush=True)
        assert e <= 2e-2, f"{key}: rel-Frobenius {e:.3e} > 2e-2"


SAVED = [w for w in CASES if w.name in ("bwd_tiny_fp32_h0", "bwd_gva_bf16", "bwd_varlen_bf16", "bwd_k256_bf16",
                                        "bwd_varlen_c32_k128")]


def saved_roundtrip(w, inp=None):
    """chunk_kda with disable_recompute (kda_chunk_fwd_save) gives o and the final state of
    the plain forward bit for bit; chunk_kda_bwd with its saved intermediates
    (kda_chunk_bwd_saved) gives the recomputing backward's gradients bit for bit, also on
    a second call from the same saved buffer; saved from other inputs is refused."""
    inp = make_inputs(w) if inp is None else inp
    kw = kernel_kwargs(w)
    kw.pop("output_final_state", None)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    common = dict(A_log=d["A_log"], dt_bias=d["dt_bias"], initial_state=d["initial_state"],
                  cu_seqlens=d["cu_seqlens"], **kw)
    o, ht = chunk_kda(*args, output_final_state=True, **common)
    o2, ht2, saved = chunk_kda(*args, output_final_state=True, disable_recompute=True, **common)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(ht2, ht), f"{w.name}: the saving forward changed o / final_state"
    do, dht = cotangents(inp)
    do, dht = do.to(DEV), dht.to(DEV)
    ref = chunk_kda_bwd(*args, do, dht=dht, **common)
    if d["q"].numel() > 0:  # (empty tensors share the null address)
        with pytest.raises(KDAContractError, match="other inputs"):
            chunk_kda_bwd(d["q"].clone(), *args[1:], do, dht=dht, saved=saved, **common)
    got = chunk_kda_bwd(*args, do, dht=dht, saved=saved, **common)
    torch.cuda.synchronize()
    for key in ref:
        assert torch.equal(got[key], ref[key]), f"{w.name} {key}: saved backward differs from the recomputing one"
    again = chunk_kda_bwd(*args, do, dht=dht, saved=saved, **common)
    torch.cuda.synchronize()
    for key in ref:
        assert torch.equal(again[key], ref[key]), f"{w.name} {key}: second backward from one saved buffer differs"
    print(f"{w.name}: saved forward / backward bit-identical", flush=True)


@pytest.mark.parametrize("w", SAVED, ids=[w.name for w in SAVED])
def test_saved_forward_backward_bitwise(w):
    print(f"case {w.name}", flush=True)
    saved_roundtrip(w)


def test_saved_forward_backward_bitwise_full_size():
    """The same at the metric configuration (B=1, T=8192, H=16, HV=32, K=V=128)."""
    print("case gva_bf16 full size", flush=True)
    saved_roundtrip(GVA_BF16)


def test_saved_forward_backward_edges():
    """The same with empty and chunk-aligned packed segments, and with T = 0."""
    w = GVA_BF16.replace(name="bwd_saved_edges", H=1, HV=2, K=64, V=64, h0="normal0.1")
    lens = [0, 64, 1, 65, 0, 17]
    inp = make_inputs(w.replace(T=sum(lens)))
    inp["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    inp["initial_state"] = 0.1 * torch.randn(len(lens), 2, 64, 64, generator=torch.Generator().manual_seed(7))
    inp["seq_lens"] = lens
    saved_roundtrip(w, inp)
    w0 = GVA_BF16.replace(name="bwd_saved_T0", H=1, HV=2, K=64, V=64, T=0, h0="normal0.1")
    saved_roundtrip(w0)


def test_backward_concurrent_streams_bitwise():
    """Two host threads, each with its own stream and inputs, call the backward at the same
    time (the bf16 chunked form shares the library's side stream of the device between
    them); every gradient equals the one from a call made alone."""
    import threading

    cases = [GVA_BF16.replace(name="conc_a", T=300, H=1, HV=2, K=64, V=64, seed=21),
             GVA_BF16.replace(name="conc_b", T=500, H=2, HV=4, K=128, V=64, seed=22)]
    runs = []
    for w in cases:
        inp = make_inputs(w)
        kw = kernel_kwargs(w)
        kw.pop("output_final_state", None)
        do, dht = cotangents(inp)
        alone = gpu_grads(inp, kw, do, dht)
        runs.append((inp, kw, do, dht, alone))
    results = [[None] * 3 for _ in runs]
    errors = []

    def worker(j):
        try:
            inp, kw, do, dht, _ = runs[j]
            d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(3):
                    out = chunk_kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do.to(DEV), dht=dht.to(DEV),
                                        A_log=d["A_log"], dt_bias=d["dt_bias"], initial_state=d["initial_state"],
                                        cu_seqlens=d["cu_seqlens"], **kw)
                    results[j][it] = {k: v.clone() for k, v in out.items()}
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for j, (_, _, _, _, alone) in enumerate(runs):
        for it in range(3):
            for key in alone:
                assert torch.equal(results[j][it][key], alone[key]), f"{cases[j].name} call {it} {key} differs"
    print("concurrent backward calls bit-identical", flush=True)
