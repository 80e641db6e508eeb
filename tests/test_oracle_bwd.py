"""The float64 backward oracle against facts that do not come from it (CPU only).

  * its differentiable forward equals the C oracle's forward to rounding;
  * every gradient it returns matches central finite differences of the C oracle's
    forward (a different implementation, no automatic differentiation), along a
    seeded random direction per input, on small inputs that cover every gate and beta
    form, the L2 norm, GVA groups, packed sequences and the state inputs;
  * with no decay (pre-gated g = 0) and beta = 0 the state never changes, and the
    gradients have closed forms (written out here with numpy).
"""
import numpy as np
import pytest

from oracle.kda_oracle import (BETA_AS_GIVEN, BETA_SIGMOID, BETA_TWO_SIGMOID, GATE_LOWER_BOUND, GATE_PRE,
                               GATE_SOFTPLUS, oracle_fwd)
from oracle.kda_oracle_bwd import oracle_bwd, oracle_fwd_torch

CASES = {
    # name: (B, T, H, HV, K, V, gate_mode, beta_mode, l2norm, h0, dht, cu_seqlens)
    "pregated_plain": (1, 6, 1, 1, 4, 3, GATE_PRE, BETA_AS_GIVEN, False, False, False, None),
    "softplus_gva_h0": (2, 5, 1, 2, 4, 3, GATE_SOFTPLUS, BETA_SIGMOID, True, True, True, None),
    "lower_bound_varlen": (1, 9, 2, 4, 3, 2, GATE_LOWER_BOUND, BETA_TWO_SIGMOID, True, True, True, [0, 4, 4, 9]),
    "lower_bound_no_alog": (1, 7, 1, 2, 5, 4, GATE_LOWER_BOUND, BETA_SIGMOID, False, False, True, None),
}


def make_case(name, seed=0):
    B, T, H, HV, K, V, gate_mode, beta_mode, l2n, h0, dht, cu = CASES[name]
    r = np.random.default_rng(seed)
    N = len(cu) - 1 if cu is not None else B
    x = {
        "q": r.standard_normal((B, T, H, K)),
        "k": r.standard_normal((B, T, H, K)) * (1.0 if l2n else 0.4),
        "v": r.standard_normal((B, T, HV, V)),
        "g": (-r.uniform(0.05, 0.6, (B, T, HV, K)) if gate_mode == GATE_PRE else r.standard_normal((B, T, HV, K))),
        "beta": (r.uniform(0.2, 0.9, (B, T, HV)) if beta_mode == BETA_AS_GIVEN else r.standard_normal((B, T, HV))),
    }
    kw = {"scale": 0.7, "gate_mode": gate_mode, "beta_mode": beta_mode, "qk_l2norm": l2n,
          "cu_seqlens": None if cu is None else np.asarray(cu, np.int64)}
    if gate_mode != GATE_PRE:
        x["dt_bias"] = 0.3 * r.standard_normal((HV, K))
        if name != "lower_bound_no_alog":
            x["A_log"] = 0.4 * r.standard_normal(HV)
    if gate_mode == GATE_LOWER_BOUND:
        kw["lower_bound"] = -2.0
    if h0:
        x["initial_state"] = 0.5 * r.standard_normal((N, HV, K, V))
    do = r.standard_normal((B, T, HV, V))
    dht_v = r.standard_normal((N, HV, K, V)) if dht else None
    return x, kw, do, dht_v


def c_loss(x, kw, do, dht):
    """<do, o> + <dht, ht> with the C oracle's forward."""
    o, ht = oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], A_log=x.get("A_log"), dt_bias=x.get("dt_bias"),
                       initial_state=x.get("initial_state"), **kw)
    loss = float(np.sum(o * do))
    if dht is not None:
        loss += float(np.sum(ht * dht))
    return loss


def grads(x, kw, do, dht):
    return oracle_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, dht=dht, A_log=x.get("A_log"),
                      dt_bias=x.get("dt_bias"), initial_state=x.get("initial_state"), **kw)


@pytest.mark.parametrize("name", list(CASES))
def test_torch_forward_matches_c_oracle(name):
    x, kw, _, _ = make_case(name)
    args = dict(A_log=x.get("A_log"), dt_bias=x.get("dt_bias"), initial_state=x.get("initial_state"), **kw)
    o_c, ht_c = oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], **args)
    o_t, ht_t = oracle_fwd_torch(x["q"], x["k"], x["v"], x["g"], x["beta"], **args)
    np.testing.assert_allclose(o_t, o_c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht_t, ht_c, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_finite_differences(name):
    x, kw, do, dht = make_case(name)
    gr = grads(x, kw, do, dht)
    key = {"initial_state": "dh0"}
    r = np.random.default_rng(123)
    eps = 1e-5
    for inp in x:
        u = r.standard_normal(x[inp].shape)
        xp = dict(x, **{inp: x[inp] + eps * u})
        xm = dict(x, **{inp: x[inp] - eps * u})
        fd = (c_loss(xp, kw, do, dht) - c_loss(xm, kw, do, dht)) / (2 * eps)
        an = float(np.sum(gr[key.get(inp, "d" + inp)] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{name}: d{inp} {an!r} vs finite difference {fd!r}"


def test_gradient_shapes_and_empty_sequence():
    """Gradients take their inputs' shapes; an empty packed segment passes dht straight to dh0."""
    x, kw, do, dht = make_case("lower_bound_varlen")
    gr = grads(x, kw, do, dht)
    for inp in x:
        assert gr[{"initial_state": "dh0"}.get(inp, "d" + inp)].shape == x[inp].shape
    np.testing.assert_array_equal(gr["dh0"][1], dht[1])  # segment 1 is empty


def test_closed_form_without_decay_or_beta():
    """Pre-gated g = 0 and beta = 0: S_t = h0 for every t, o_t = h0^T (s q_t).  With
    R_t = sum_{s >= t} s q_s do_s^T + dht (the gradient reaching S_t):
      dq_t = s h0 do_t,  dh0 = R_0,  dv = 0,  dk = 0,
      dg_t[i] = sum_j (R_t)_ij (h0)_ij,  dbeta_t = k_t^T R_t (v_t - h0^T k_t)."""
    r = np.random.default_rng(5)
    T, K, V, s = 6, 4, 3, 0.8
    q, k, v = r.standard_normal((1, T, 1, K)), r.standard_normal((1, T, 1, K)), r.standard_normal((1, T, 1, V))
    g, beta = np.zeros((1, T, 1, K)), np.zeros((1, T, 1))
    h0, do, dht = r.standard_normal((1, 1, K, V)), r.standard_normal((1, T, 1, V)), r.standard_normal((1, 1, K, V))
    gr = oracle_bwd(q, k, v, g, beta, do, dht=dht, scale=s, initial_state=h0)
    H0 = h0[0, 0]
    R = dht[0, 0].copy()
    dq = np.zeros((T, K)); dg = np.zeros((T, K)); db = np.zeros(T)
    for t in range(T - 1, -1, -1):
        R = R + s * np.outer(q[0, t, 0], do[0, t, 0])
        dq[t] = s * H0 @ do[0, t, 0]
        dg[t] = np.sum(R * H0, axis=1)
        db[t] = k[0, t, 0] @ R @ (v[0, t, 0] - H0.T @ k[0, t, 0])
    np.testing.assert_allclose(gr["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dh0"][0, 0], R, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dbeta"][0, :, 0], db, rtol=1e-12, atol=1e-12)
    assert np.all(gr["dv"] == 0) and np.all(gr["dk"] == 0)


def _fd_mismatch(name):
    """True when some gradient of the (possibly patched) oracle misses its finite difference."""
    try:
        test_gradients_match_finite_differences(name)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("mutant", ["norm_not_differentiated", "beta_transform_not_differentiated",
                                    "decay_not_differentiated"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    """Mistakes that leave the forward values unchanged but drop a term of the gradient
    (a factor treated as a constant) must fail the finite-difference pin."""
    import oracle.kda_oracle_bwd as B
    import torch

    if mutant == "norm_not_differentiated":
        monkeypatch.setattr(B, "_normalise", lambda x, on: x * torch.rsqrt((x * x).sum(-1, keepdim=True) + 1e-6).detach()
                            if on else x)
        case = "softplus_gva_h0"
    elif mutant == "beta_transform_not_differentiated":
        orig = B.beta_activate
        monkeypatch.setattr(B, "beta_activate", lambda b, m: orig(b, m).detach())
        case = "lower_bound_no_alog"
    else:
        orig = B.gate_activate
        monkeypatch.setattr(B, "gate_activate", lambda *a: orig(*a).detach())
        case = "pregated_plain"
    assert _fd_mismatch(case), f"planted mistake '{mutant}' was not caught"
