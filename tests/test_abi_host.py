"""Host-side tests of the C ABI (no GPU): exported symbols, version, and every
argument-check error path.  Checks run on the host before any HIP call, so the
failing calls below never touch a device (the fake pointers are never used)."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_delta_rule_log2_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
S = _abi.STATUS
FAKE = 0x1000  # a non-null address that must never be dereferenced


@pytest.fixture(scope="module")
def lib():
    return _abi.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, re.M)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(_abi.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(kda_\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_matches_header(lib):
    m = re.search(r"#define\s+KDA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.kda_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in S.values():
        assert lib.kda_status_string(code)
    m = dict(re.findall(r"(KDA_\w+)\s*=\s*(\d+)", open(HEADER).read()))
    for name, code in S.items():
        assert int(m[name]) == code, name


def desc(**kw):
    d = _abi.KdaFwdDesc()
    base = dict(B=1, T=256, H=2, HV=4, K=128, V=128, chunk_size=64, num_seqs=1,
                qkv_dtype=_abi.DTYPE_BF16, g_dtype=_abi.DTYPE_BF16, beta_dtype=_abi.DTYPE_BF16,
                scale=0.088, lower_bound=0.0, flags=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def ws_status(lib, d):
    n = ctypes.c_size_t(0)
    return lib.kda_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n)), n.value


def fwd_status(lib, d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=None, h0=None, cu=None,
             o=FAKE, ht=FAKE, ws=FAKE, ws_bytes=1 << 40)
    p.update(ptrs)
    return lib.kda_chunk_fwd(ctypes.byref(d), p["q"], p["k"], p["v"], p["g"], p["beta"], p["A_log"],
                             p["dt_bias"], p["h0"], p["cu"], p["o"], p["ht"], p["ws"], p["ws_bytes"], None)


CASES = [
    ("chunk size 48", dict(chunk_size=48), "KDA_ERR_CHUNK_SIZE"),
    ("chunk size 128", dict(chunk_size=128), "KDA_ERR_CHUNK_SIZE"),
    ("K = 512 (the pages' literal example)", dict(K=512, V=512), "KDA_ERR_HEAD_DIM"),
    ("K not a multiple of 32", dict(K=80), "KDA_ERR_UNSUPPORTED"),
    ("V > 256", dict(V=288), "KDA_ERR_UNSUPPORTED"),
    ("V not a multiple of 32", dict(V=48), "KDA_ERR_UNSUPPORTED"),
    ("fp32 K = V = 256 (over one CU's LDS)", dict(K=256, V=256, qkv_dtype=_abi.DTYPE_FP32), "KDA_ERR_UNSUPPORTED"),
    ("HV % H != 0", dict(H=3, HV=4), "KDA_ERR_GVA"),
    ("safe gate without lower bound", dict(flags=_abi.SAFE_GATE | _abi.GATE_IN_KERNEL), "KDA_ERR_LOWER_BOUND"),
    ("safe gate lb = -6", dict(flags=_abi.SAFE_GATE | _abi.HAS_LOWER_BOUND, lower_bound=-6.0), "KDA_ERR_LOWER_BOUND"),
    ("safe gate lb = 0", dict(flags=_abi.SAFE_GATE | _abi.HAS_LOWER_BOUND, lower_bound=0.0), "KDA_ERR_LOWER_BOUND"),
    ("lower bound > 0", dict(flags=_abi.HAS_LOWER_BOUND, lower_bound=0.5), "KDA_ERR_LOWER_BOUND"),
    ("lower bound NaN", dict(flags=_abi.HAS_LOWER_BOUND, lower_bound=float("nan")), "KDA_ERR_LOWER_BOUND"),
    ("neg eigval without sigmoid", dict(flags=_abi.ALLOW_NEG_EIGVAL), "KDA_ERR_NEG_EIGVAL"),
    ("bad qkv dtype", dict(qkv_dtype=7), "KDA_ERR_DTYPE"),
    ("bad g dtype", dict(g_dtype=-1), "KDA_ERR_DTYPE"),
    ("negative T", dict(T=-1), "KDA_ERR_SHAPE"),
    ("zero heads", dict(H=0), "KDA_ERR_SHAPE"),
    ("num_seqs != B without cu_seqlens", dict(num_seqs=3), "KDA_ERR_SHAPE"),
    ("unknown flag bit", dict(flags=1 << 12), "KDA_ERR_UNSUPPORTED"),
]


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_descriptor_errors(lib, name, kw, code):
    d = desc(**kw)
    assert ws_status(lib, d)[0] == S[code]
    assert fwd_status(lib, d) == S[code]


def test_safe_gate_bounds_accepted(lib):
    for lb in (-5.0, -1.0, -1e-3):
        d = desc(flags=_abi.SAFE_GATE | _abi.HAS_LOWER_BOUND | _abi.GATE_IN_KERNEL, lower_bound=lb)
        assert ws_status(lib, d)[0] == 0


def _cu(vals):
    arr = (ctypes.c_int64 * len(vals))(*vals)
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))


@pytest.mark.parametrize("vals,B,T,ok", [
    ([0, 100, 256], 1, 256, True),
    ([0, 0, 256], 1, 256, True),           # empty sequence is allowed
    ([1, 100, 256], 1, 256, False),        # must start at 0
    ([0, 100, 255], 1, 256, False),        # must end at T
    ([0, 200, 100, 256], 1, 256, False),   # decreasing
    ([0, 100, 256], 2, 128, False),        # B must be 1
])
def test_varlen_checks(lib, vals, B, T, ok):
    arr, ptr = _cu(vals)
    d = desc(B=B, T=T, num_seqs=len(vals) - 1)
    d.cu_seqlens_host = ptr
    rc, n = ws_status(lib, d)
    assert (rc == 0) == ok, rc
    if not ok:
        assert rc == S["KDA_ERR_VARLEN"]
        assert fwd_status(lib, d, cu=FAKE) == S["KDA_ERR_VARLEN"]


def test_varlen_device_and_host_copies_go_together(lib):
    arr, ptr = _cu([0, 100, 256])
    d = desc(num_seqs=2)
    d.cu_seqlens_host = ptr
    assert fwd_status(lib, d, cu=None) == S["KDA_ERR_VARLEN"]
    d2 = desc()
    assert fwd_status(lib, d2, cu=FAKE) == S["KDA_ERR_VARLEN"]


def test_pointer_and_workspace_errors(lib):
    d = desc(flags=_abi.OUTPUT_FINAL_STATE)
    assert fwd_status(lib, d, q=None) == S["KDA_ERR_NULL_POINTER"]
    assert fwd_status(lib, d, o=None) == S["KDA_ERR_NULL_POINTER"]
    assert fwd_status(lib, d, ht=None) == S["KDA_ERR_NULL_POINTER"]
    assert lib.kda_chunk_fwd_workspace_size(None, None) == S["KDA_ERR_NULL_POINTER"]
    d2 = desc(flags=_abi.GATE_IN_KERNEL)
    assert fwd_status(lib, d2, A_log=None) == S["KDA_ERR_MISSING_A_LOG"]
    # with a lower bound, A_log may be absent (exp(A_log) taken as 1)
    rc, need = ws_status(lib, desc())
    assert rc == 0
    assert fwd_status(lib, desc(), ws_bytes=need - 1) == S["KDA_ERR_WORKSPACE"]
    assert fwd_status(lib, desc(), ws=None) == S["KDA_ERR_WORKSPACE"]


def test_workspace_size_grows_with_chunks(lib):
    sizes = [ws_status(lib, desc(T=t))[1] for t in (64, 128, 1024)]
    assert sizes[0] < sizes[1] < sizes[2]
    # bf16 intermediates take half the bytes of fp32 ones (plan region aside)
    b = ws_status(lib, desc(T=4096))[1]
    f = ws_status(lib, desc(T=4096, qkv_dtype=_abi.DTYPE_FP32))[1]
    assert 1.9 < f / b < 2.01


def test_python_shim_rejects_unsupported_keywords():
    import torch

    from gated_delta_rule_log2_amd import KDAContractError, chunk_kda

    x = torch.zeros(1, 4, 1, 32)
    for kw in (dict(cp_context=object()), dict(disable_recompute=True, return_intermediate_states=True),
               dict(disable_recompute=True, state_v_first=True)):
        with pytest.raises(KDAContractError):
            chunk_kda(x, x, x, x, x[..., 0], **kw)
    assert issubclass(KDAContractError, ValueError)


def test_python_shim_saved_backward_contract():
    """chunk_kda_bwd: disable_recompute without saved, and saved with the token-level
    form, are refused before anything reaches the library."""
    import torch

    from gated_delta_rule_log2_amd import KDAContractError, KDASaved, chunk_kda_bwd

    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(KDAContractError, match="needs saved"):
        chunk_kda_bwd(x, x, x, x, x[..., 0], x, disable_recompute=True)
    with pytest.raises(KDAContractError, match="chunked backward only"):
        chunk_kda_bwd(x, x, x, x, x[..., 0], x, saved=KDASaved(torch.zeros(256, dtype=torch.uint8), ("x",)),
                      tokenwise=True)


def test_transposed_state_flag_and_states_entry_checks(lib):
    """KDA_TRANSPOSE_STATE passes the descriptor checks (the next bit does not), and
    kda_chunk_fwd_states refuses a NULL state output before anything is enqueued."""
    assert _abi.STATUS_NAMES[ws_status(lib, desc(flags=_abi.TRANSPOSE_STATE))[0]] == "KDA_OK"
    assert _abi.STATUS_NAMES[ws_status(lib, desc(flags=_abi.TRANSPOSE_STATE << 1))[0]] == "KDA_ERR_UNSUPPORTED"
    d = desc(flags=_abi.TRANSPOSE_STATE)
    rc = lib.kda_chunk_fwd_states(ctypes.byref(d), *([None] * 13), 0, None)
    assert _abi.STATUS_NAMES[rc] == "KDA_ERR_NULL_POINTER"



def bwd_status(lib, d, **ptrs):
    names = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "h0", "cu", "do", "dht", "dq", "dk", "dv", "dg",
             "dbeta", "dA_log", "ddt_bias", "dh0", "ws"]
    ws_bytes = ptrs.pop("ws_bytes", 1 << 40)
    p = {n: FAKE for n in names}
    p.update(dt_bias=None, h0=None, cu=None, dht=None, dA_log=None, ddt_bias=None, dh0=None)
    p.update(ptrs)
    return lib.kda_chunk_bwd(ctypes.byref(d), *[p[n] for n in names], ws_bytes, None)


def test_backward_entry_checks(lib):
    """kda_chunk_bwd: the forward's descriptor checks, the transposed state layout refused,
    missing inputs / outputs / workspace refused before anything is enqueued."""
    n = ctypes.c_size_t(0)
    assert _abi.STATUS_NAMES[lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n))] == "KDA_OK"
    fwd_need = ws_status(lib, desc())[1]
    assert n.value > fwd_need  # the forward's workspace plus the backward's own
    assert lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc()), None) == S["KDA_ERR_NULL_POINTER"]
    rc = lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc(flags=_abi.TRANSPOSE_STATE)), ctypes.byref(n))
    assert _abi.STATUS_NAMES[rc] == "KDA_ERR_UNSUPPORTED"
    assert bwd_status(lib, desc(chunk_size=48)) == S["KDA_ERR_CHUNK_SIZE"]
    assert bwd_status(lib, desc(H=3, HV=4)) == S["KDA_ERR_GVA"]
    for missing in ("do", "dq", "dk", "dv", "dg", "dbeta", "q"):
        assert bwd_status(lib, desc(), **{missing: None}) == S["KDA_ERR_NULL_POINTER"], missing
    assert bwd_status(lib, desc(flags=_abi.GATE_IN_KERNEL), A_log=None) == S["KDA_ERR_MISSING_A_LOG"]
    assert bwd_status(lib, desc(), ws=None) == S["KDA_ERR_WORKSPACE"]
    lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n))
    assert bwd_status(lib, desc(), ws_bytes=n.value - 1) == S["KDA_ERR_WORKSPACE"]


def test_saved_forward_and_backward_entry_checks(lib):
    """kda_chunk_fwd_save needs the backward's workspace size and refuses the transposed
    state layout; kda_chunk_bwd_saved makes kda_chunk_bwd's checks; all before anything is
    enqueued."""
    n = ctypes.c_size_t(0)
    lib.kda_chunk_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n))
    fwd_need = ws_status(lib, desc())[1]

    def save(d, ws_bytes, **ptrs):
        names = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "h0", "cu", "o", "ht", "ws"]
        p = {nm: FAKE for nm in names}
        p.update(dt_bias=None, h0=None, cu=None, ht=None)
        p.update(ptrs)
        return lib.kda_chunk_fwd_save(ctypes.byref(d), *[p[nm] for nm in names], ws_bytes, None)

    assert save(desc(), fwd_need) == S["KDA_ERR_WORKSPACE"]  # the forward's size is not enough
    assert save(desc(), n.value - 1) == S["KDA_ERR_WORKSPACE"]
    assert save(desc(), n.value, ws=None) == S["KDA_ERR_WORKSPACE"]
    assert save(desc(flags=_abi.TRANSPOSE_STATE), n.value) == S["KDA_ERR_UNSUPPORTED"]
    assert save(desc(chunk_size=48), n.value) == S["KDA_ERR_CHUNK_SIZE"]
    assert save(desc(), n.value, o=None) == S["KDA_ERR_NULL_POINTER"]
    assert save(desc(flags=_abi.OUTPUT_FINAL_STATE), n.value) == S["KDA_ERR_NULL_POINTER"]
    assert lib.kda_chunk_fwd_save(None, *([None] * 12), 0, None) == S["KDA_ERR_NULL_POINTER"]

    def bwd_saved(d, **ptrs):
        names = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "h0", "cu", "do", "dht", "dq", "dk", "dv", "dg",
                 "dbeta", "dA_log", "ddt_bias", "dh0", "ws"]
        ws_bytes = ptrs.pop("ws_bytes", 1 << 40)
        p = {nm: FAKE for nm in names}
        p.update(dt_bias=None, h0=None, cu=None, dht=None, dA_log=None, ddt_bias=None, dh0=None)
        p.update(ptrs)
        return lib.kda_chunk_bwd_saved(ctypes.byref(d), *[p[nm] for nm in names], ws_bytes, None)

    assert bwd_saved(desc(flags=_abi.TRANSPOSE_STATE)) == S["KDA_ERR_UNSUPPORTED"]
    assert bwd_saved(desc(H=3, HV=4)) == S["KDA_ERR_GVA"]
    for missing in ("do", "dq", "dk", "dv", "dg", "dbeta", "q"):
        assert bwd_saved(desc(), **{missing: None}) == S["KDA_ERR_NULL_POINTER"], missing
    assert bwd_saved(desc(), ws=None) == S["KDA_ERR_WORKSPACE"]
    assert bwd_saved(desc(), ws_bytes=n.value - 1) == S["KDA_ERR_WORKSPACE"]
