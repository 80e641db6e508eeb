"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each ``check_*`` takes the path of an oracle shared library and raises
AssertionError when the oracle disagrees with the fact.  ``test_oracle_pins``
runs them against the real oracle; ``test_oracle_mutants`` compiles copies of
the oracle with a planted mistake and requires that some check fails for each.

Facts used (none is a re-typing of the oracle's own loop):
  * the chunk-form forward of the reading notes (tests/chunk_form.py), evaluated
    densely with a matrix inverse;
  * closed forms of special cases: beta = 0 (pure decay), beta = 0 and g = 0
    (constant state), beta = 1 with unit keys (exact write), beta = 2 (reflected
    write), T = 1 from a zero state;
  * a hand-worked recurrence and hand-worked gate values (tests/golden);
  * structural facts: sequences in a pack are independent, a run split at any
    token and continued from the carried state equals the whole run, value
    heads of one GVA group read the same q/k head, L2 normalisation removes a
    positive rescaling of q and k, the gate output lies in [lower_bound, 0).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import (
    BETA_AS_GIVEN, BETA_SIGMOID, BETA_TWO_SIGMOID, GATE_LOWER_BOUND, GATE_PRE, GATE_SOFTPLUS,
    oracle_fwd, oracle_gate_cumsum,
)
from tests.chunk_form import chunk_form, chunk_form_sequence

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= tol, f"{what}: scaled max error {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------------------------
# chunk-form agreement
# --------------------------------------------------------------------------------------------
def _chunk_case(lib, seed, lens, H, HV, K, V, chunk, beta_hi, g_lo, with_h0):
    r = _rng(seed)
    Ttot = int(sum(lens))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = _unit_rows(r.standard_normal((1, Ttot, H, K)))
    k = _unit_rows(r.standard_normal((1, Ttot, H, K)))
    v = r.standard_normal((1, Ttot, HV, V))
    g = r.uniform(g_lo, 0.0, (1, Ttot, HV, K))
    beta = r.uniform(0.0, beta_hi, (1, Ttot, HV))
    h0 = 0.3 * r.standard_normal((len(lens), HV, K, V)) if with_h0 else None
    o, ht = oracle_fwd(q, k, v, g, beta, scale=1.0, gate_mode=GATE_PRE, initial_state=h0,
                       cu_seqlens=starts, lib_path=lib)
    group = HV // H
    o2, ht2 = chunk_form(q[0], k[0], v[0], g[0], beta[0], h0, chunk, starts, lambda hv: hv // group)
    _close(o[0], o2, 1e-11, f"o vs chunk form (chunk {chunk}, lens {lens})")
    _close(ht, ht2, 1e-11, f"final state vs chunk form (chunk {chunk}, lens {lens})")


def check_chunk_form(lib):
    # single sequence, full chunks, per-channel decays
    _chunk_case(lib, 1, [64], 1, 1, 8, 5, 16, 1.0, -0.4, False)
    # partial last chunk, odd chunk size, GVA, initial state
    _chunk_case(lib, 2, [37], 2, 4, 6, 3, 8, 1.0, -0.3, True)
    # several packed sequences of ragged length, beta up to 2, chunk 32 and 64
    _chunk_case(lib, 3, [70, 5, 33], 1, 2, 4, 4, 32, 2.0, -0.1, True)
    _chunk_case(lib, 4, [130], 2, 2, 4, 3, 64, 1.0, -0.05, True)


def _chunk_states_case(lib, seed, lens, H, HV, K, V, chunk):
    r = _rng(seed)
    Ttot = int(sum(lens))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = _unit_rows(r.standard_normal((1, Ttot, H, K)))
    k = _unit_rows(r.standard_normal((1, Ttot, H, K)))
    v = r.standard_normal((1, Ttot, HV, V))
    g = r.uniform(-0.3, 0.0, (1, Ttot, HV, K))
    beta = r.uniform(0.0, 1.5, (1, Ttot, HV))
    h0 = 0.3 * r.standard_normal((len(lens), HV, K, V))
    o, ht, states = oracle_fwd(q, k, v, g, beta, scale=1.0, initial_state=h0, cu_seqlens=starts,
                               chunk_states=chunk, lib_path=lib)
    o_plain, ht_plain = oracle_fwd(q, k, v, g, beta, scale=1.0, initial_state=h0, cu_seqlens=starts, lib_path=lib)
    assert np.array_equal(o, o_plain) and np.array_equal(ht, ht_plain), "snapshots changed the forward"
    group = HV // H
    ref = []
    for n in range(len(lens)):
        a, b = starts[n], starts[n + 1]
        per_head = []
        for hv in range(HV):
            got = []
            chunk_form_sequence(q[0, a:b, hv // group], k[0, a:b, hv // group], v[0, a:b, hv], g[0, a:b, hv],
                                beta[0, a:b, hv], h0[n, hv], chunk, got)
            per_head.append(got)
        for c in range(len(per_head[0])):
            ref.append(np.stack([per_head[hv][c] for hv in range(HV)]))
    ref = np.stack(ref)
    assert states.shape == ref.shape, f"chunk states shape {states.shape} != {ref.shape}"
    _close(states, ref, 1e-11, f"chunk states vs chunk form (chunk {chunk}, lens {lens})")
    first = np.concatenate([[0], np.cumsum([(L + chunk - 1) // chunk for L in lens])[:-1]])
    for n in range(len(lens)):
        assert np.array_equal(states[first[n]], h0[n]), f"sequence {n}: first chunk state is not h0"


def check_chunk_states(lib):
    """The state each chunk starts from equals the S of the chunk form's step 4
    before its update (the initial state for a sequence's first chunk)."""
    _chunk_states_case(lib, 40, [37, 16, 50], 1, 2, 4, 3, 16)
    _chunk_states_case(lib, 41, [70, 9], 2, 2, 5, 4, 32)


# --------------------------------------------------------------------------------------------
# closed forms of special cases
# --------------------------------------------------------------------------------------------
def check_beta_zero_pure_decay(lib):
    r = _rng(10)
    T, K, V = 9, 5, 3
    q = r.standard_normal((1, T, 1, K))
    k = r.standard_normal((1, T, 1, K))
    v = r.standard_normal((1, T, 1, V))
    g = r.uniform(-1.0, 0.0, (1, T, 1, K))
    beta = np.zeros((1, T, 1))
    h0 = r.standard_normal((1, 1, K, V))
    o, ht = oracle_fwd(q, k, v, g, beta, scale=0.7, initial_state=h0, lib_path=lib)
    cum = np.cumsum(g[0, :, 0], axis=0)          # [T, K]: log of the product of decays so far
    for t in range(T):
        S_t = np.exp(cum[t])[:, None] * h0[0, 0]
        _close(o[0, t, 0], 0.7 * S_t.T @ q[0, t, 0], 1e-13, f"beta=0 output at t={t}")
    _close(ht[0, 0], np.exp(cum[-1])[:, None] * h0[0, 0], 1e-13, "beta=0 final state")


def check_constant_state(lib):
    r = _rng(11)
    T, K, V = 7, 4, 6
    q = r.standard_normal((1, T, 1, K))
    k = r.standard_normal((1, T, 1, K))
    v = r.standard_normal((1, T, 1, V))
    h0 = r.standard_normal((1, 1, K, V))
    o, ht = oracle_fwd(q, k, v, np.zeros((1, T, 1, K)), np.zeros((1, T, 1)), scale=1.0,
                       initial_state=h0, lib_path=lib)
    _close(ht, h0, 0.0, "beta=0, g=0 keeps the state")
    _close(o[0, :, 0], q[0, :, 0] @ h0[0, 0], 1e-13, "beta=0, g=0 output")


def check_exact_write(lib):
    """beta = 1, ||k|| = 1: after the step, S_t^T k_t = v_t for any decay.  With q = k
    (scale 1) the oracle's o_t is exactly S_t^T k_t."""
    r = _rng(12)
    T, K, V = 11, 6, 4
    k = _unit_rows(r.standard_normal((1, T, 1, K)))
    v = r.standard_normal((1, T, 1, V))
    g = r.uniform(-2.0, 0.0, (1, T, 1, K))
    h0 = r.standard_normal((1, 1, K, V))
    o, _ = oracle_fwd(k, k, v, g, np.ones((1, T, 1)), scale=1.0, initial_state=h0, lib_path=lib)
    _close(o, v, 1e-13, "beta=1 exact write")


def check_reflected_write(lib):
    """beta = 2, ||k|| = 1: S_t^T k_t = 2 v_t - (Diag(alpha_t) S_{t-1})^T k_t."""
    r = _rng(13)
    T, K, V = 6, 5, 3
    k = _unit_rows(r.standard_normal((1, T, 1, K)))
    v = r.standard_normal((1, T, 1, V))
    g = r.uniform(-1.0, 0.0, (1, T, 1, K))
    h0 = r.standard_normal((1, 1, K, V))
    beta = np.full((1, T, 1), 2.0)
    o, _ = oracle_fwd(k, k, v, g, beta, scale=1.0, initial_state=h0, lib_path=lib)
    _, S_prev = oracle_fwd(k[:, :T - 1], k[:, :T - 1], v[:, :T - 1], g[:, :T - 1],
                           beta[:, :T - 1], scale=1.0, initial_state=h0, lib_path=lib)
    decayed = np.exp(g[0, T - 1, 0])[:, None] * S_prev[0, 0]
    expect = 2.0 * v[0, T - 1, 0] - decayed.T @ k[0, T - 1, 0]
    _close(o[0, T - 1, 0], expect, 1e-13, "beta=2 reflected write")


def check_single_token(lib):
    """T = 1 from a zero state: S_1 = beta k v^T, o_1 = beta (k.q) v (decay irrelevant)."""
    r = _rng(14)
    K, V = 7, 5
    q = r.standard_normal((1, 1, 1, K))
    k = r.standard_normal((1, 1, 1, K))
    v = r.standard_normal((1, 1, 1, V))
    g = r.uniform(-3.0, 0.0, (1, 1, 1, K))
    b = 0.37
    o, ht = oracle_fwd(q, k, v, g, np.full((1, 1, 1), b), scale=1.0, lib_path=lib)
    kk, qq, vv = k[0, 0, 0], q[0, 0, 0], v[0, 0, 0]
    _close(ht[0, 0], b * np.outer(kk, vv), 1e-14, "T=1 state")
    _close(o[0, 0, 0], b * (kk @ qq) * vv, 1e-14, "T=1 output")


def _golden_value(x):
    if isinstance(x, list) and len(x) == 2 and isinstance(x[0], str):
        op, a = x
        return {"ln": math.log(a), "-ln": -math.log(a), "ln-1": math.log(a) - 1.0,
                "half-ln": 0.5 * math.log(a)}[op]
    return x


def check_hand_worked(lib):
    with open(os.path.join(GOLDEN, "scalar_recurrence.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        K, V, steps = case["K"], case["V"], case["steps"]
        T = len(steps)
        q = np.array([s["q"] for s in steps], float).reshape(1, T, 1, K)
        k = np.array([s["k"] for s in steps], float).reshape(1, T, 1, K)
        v = np.array([s["v"] for s in steps], float).reshape(1, T, 1, V)
        gl = [s["g"] for s in steps]
        g = np.array([[_golden_value(x) for x in row] if K > 1 else [_golden_value(row)]
                      for row in gl], float).reshape(1, T, 1, K)
        beta = np.array([s["beta"] for s in steps], float).reshape(1, T, 1)
        h0 = np.array(case["S0"], float).reshape(1, 1, K, V)
        for t in range(1, T + 1):
            o, ht = oracle_fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], scale=1.0,
                               initial_state=h0, lib_path=lib)
            _close(ht[0, 0], np.array(steps[t - 1]["S"], float), 1e-14, f"{case['name']} S_{t}")
            _close(o[0, t - 1, 0], np.array(steps[t - 1]["o"], float), 1e-14, f"{case['name']} o_{t}")


# --------------------------------------------------------------------------------------------
# gate and input transforms
# --------------------------------------------------------------------------------------------
def check_gate_closed_forms(lib):
    with open(os.path.join(GOLDEN, "gate_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    modes = {"pre": GATE_PRE, "softplus": GATE_SOFTPLUS, "lower_bound": GATE_LOWER_BOUND}
    for c in cases:
        g = np.full((1, 1, 1, 1), _golden_value(c["g"]))
        A_log = None if c["A_log"] is None else np.array([_golden_value(c["A_log"])])
        dt = np.array([float(c["dt_bias"])])
        lb = 0.0 if c["lower_bound"] is None else float(c["lower_bound"])
        act, cum = oracle_gate_cumsum(g, chunk_size=64, gate_mode=modes[c["mode"]], lower_bound=lb,
                                      A_log=A_log, dt_bias=dt, lib_path=lib)
        want = _golden_value(c["expect"])
        assert abs(act.item() - want) <= 1e-14, f"gate {c}: {act.item()} != {want}"
        assert abs(cum.item() - want) <= 1e-14, f"gate cumsum of one row {c}"


def check_gate_range_and_cumsum(lib):
    """Bounded gate lies in [lb, 0); chunk-local sums restart at chunk and sequence starts."""
    r = _rng(20)
    g = r.standard_normal((1, 10, 2, 3)) * 4.0
    A_log = r.standard_normal(2)
    dt = r.standard_normal(6)
    act, _ = oracle_gate_cumsum(g, chunk_size=4, gate_mode=GATE_LOWER_BOUND, lower_bound=-5.0,
                                A_log=A_log, dt_bias=dt, lib_path=lib)
    assert np.all(act >= -5.0) and np.all(act < 0.0), "bounded gate leaves [lb, 0)"
    act2, _ = oracle_gate_cumsum(g, chunk_size=4, gate_mode=GATE_SOFTPLUS, A_log=A_log, dt_bias=dt,
                                 lib_path=lib)
    assert np.all(act2 < 0.0), "softplus gate must be a decay"
    # constant pre-gated decay: the chunk-local sum at in-chunk row r is (r+1)*c
    c = -0.5
    gc = np.full((1, 10, 1, 1), c)
    _, cum = oracle_gate_cumsum(gc, chunk_size=4, gate_mode=GATE_PRE, cu_seqlens=[0, 3, 10], lib_path=lib)
    expect = [c * r_ for r_ in (1, 2, 3, 1, 2, 3, 4, 1, 2, 3)]
    assert np.allclose(cum[0, :, 0, 0], expect, rtol=0, atol=1e-15), f"cumsum {cum.ravel()} != {expect}"


def check_gate_parameter_layout(lib):
    """A_log is per value head, dt_bias is [HV*K] with index hv*K + d: choosing
    dt_bias = -g makes every bias-shifted input 0, so the softplus gate becomes
    -exp(A_log[hv]) ln 2 and the bounded gate lower_bound / 2, for every element."""
    r = _rng(23)
    T, HV, K = 5, 3, 4
    c = r.standard_normal((HV, K))
    g = np.broadcast_to(c, (1, T, HV, K)).copy()
    A_log = np.array([0.0, math.log(2.0), math.log(0.5)])
    dt = -c.reshape(HV * K)
    act, _ = oracle_gate_cumsum(g, chunk_size=64, gate_mode=GATE_SOFTPLUS, A_log=A_log, dt_bias=dt,
                                lib_path=lib)
    want = -np.exp(A_log)[None, None, :, None] * math.log(2.0)
    assert np.allclose(act, np.broadcast_to(want, act.shape), rtol=0, atol=1e-14), "softplus layout"
    act, _ = oracle_gate_cumsum(g, chunk_size=64, gate_mode=GATE_LOWER_BOUND, lower_bound=-3.0,
                                A_log=A_log, dt_bias=dt, lib_path=lib)
    assert np.allclose(act, -1.5, rtol=0, atol=1e-14), "bounded gate layout"


def check_beta_modes(lib):
    """sigmoid(0) = 1/2 and 2*sigmoid(0) = 1: logits of 0 equal given betas of 1/2 and 1."""
    r = _rng(21)
    T, K, V = 8, 4, 3
    q, k = r.standard_normal((1, T, 1, K)), _unit_rows(r.standard_normal((1, T, 1, K)))
    v, g = r.standard_normal((1, T, 1, V)), r.uniform(-1, 0, (1, T, 1, K))
    zeros = np.zeros((1, T, 1))
    for mode, given in ((BETA_SIGMOID, 0.5), (BETA_TWO_SIGMOID, 1.0)):
        o1, h1 = oracle_fwd(q, k, v, g, zeros, scale=1.0, beta_mode=mode, lib_path=lib)
        o2, h2 = oracle_fwd(q, k, v, g, np.full((1, T, 1), given), scale=1.0,
                            beta_mode=BETA_AS_GIVEN, lib_path=lib)
        _close(o1, o2, 1e-14, f"beta mode {mode}")
        _close(h1, h2, 1e-14, f"beta mode {mode} state")
    # sigmoid(ln 3) = 3/4
    o1, _ = oracle_fwd(q, k, v, g, np.full((1, T, 1), math.log(3.0)), scale=1.0,
                       beta_mode=BETA_TWO_SIGMOID, lib_path=lib)
    o2, _ = oracle_fwd(q, k, v, g, np.full((1, T, 1), 1.5), scale=1.0, lib_path=lib)
    _close(o1, o2, 1e-14, "2*sigmoid(ln 3) = 3/2")


def check_l2norm_and_scale(lib):
    """With L2 normalisation on, positive rescaling of q and k changes nothing (up to
    the 1e-6 epsilon); scale multiplies the output linearly."""
    r = _rng(22)
    T, K, V = 10, 8, 4
    q, k = r.standard_normal((1, T, 1, K)), r.standard_normal((1, T, 1, K))
    v, g = r.standard_normal((1, T, 1, V)), r.uniform(-1, 0, (1, T, 1, K))
    beta = r.uniform(0, 1, (1, T, 1))
    o1, h1 = oracle_fwd(q, k, v, g, beta, scale=0.5, qk_l2norm=True, lib_path=lib)
    cq = r.uniform(5, 20, (1, T, 1, 1))
    ck = r.uniform(5, 20, (1, T, 1, 1))
    o2, h2 = oracle_fwd(q * cq, k * ck, v, g, beta, scale=0.5, qk_l2norm=True, lib_path=lib)
    _close(o1, o2, 1e-7, "l2norm removes rescaling")
    _close(h1, h2, 1e-7, "l2norm removes rescaling (state)")
    o3, h3 = oracle_fwd(_unit_rows(q), _unit_rows(k), v, g, beta, scale=1.0, lib_path=lib)
    _close(2.0 * o1, o3, 1e-6, "normalised inputs without the flag, scale 1")
    _close(h1, h3, 1e-6, "state independent of scale")


# --------------------------------------------------------------------------------------------
# structure
# --------------------------------------------------------------------------------------------
def check_gva_mapping(lib):
    """Value head hv reads q/k head hv // (HV/H): equal to repeating each q/k head."""
    r = _rng(30)
    T, H, HV, K, V = 12, 2, 6, 4, 3
    q, k = r.standard_normal((1, T, H, K)), _unit_rows(r.standard_normal((1, T, H, K)))
    v, g = r.standard_normal((1, T, HV, V)), r.uniform(-1, 0, (1, T, HV, K))
    beta = r.uniform(0, 1, (1, T, HV))
    o1, h1 = oracle_fwd(q, k, v, g, beta, scale=1.0, lib_path=lib)
    qr, kr = np.repeat(q, HV // H, axis=2), np.repeat(k, HV // H, axis=2)
    o2, h2 = oracle_fwd(qr, kr, v, g, beta, scale=1.0, lib_path=lib)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2), "GVA head mapping"


def check_varlen_and_carry(lib):
    """Sequences packed with cu_seqlens equal separate runs, bit for bit; a run split
    at any token and continued from the carried state equals the whole run."""
    r = _rng(31)
    lens = [5, 0, 13, 7]
    T = sum(lens)
    H, HV, K, V = 1, 2, 4, 3
    q, k = r.standard_normal((1, T, H, K)), _unit_rows(r.standard_normal((1, T, H, K)))
    v, g = r.standard_normal((1, T, HV, V)), r.uniform(-1, 0, (1, T, HV, K))
    beta = r.uniform(0, 1.5, (1, T, HV))
    h0 = r.standard_normal((len(lens), HV, K, V))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ht = oracle_fwd(q, k, v, g, beta, scale=1.0, initial_state=h0, cu_seqlens=cu, lib_path=lib)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if a == b:
            assert np.array_equal(ht[n], h0[n]), "empty sequence keeps its state"
            continue
        o1, h1 = oracle_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], scale=1.0,
                            initial_state=h0[n:n + 1], lib_path=lib)
        assert np.array_equal(o[:, a:b], o1) and np.array_equal(ht[n], h1[0]), f"segment {n}"
    a, b = cu[2], cu[3]
    for cut in (a + 1, a + 6):
        _, hA = oracle_fwd(q[:, a:cut], k[:, a:cut], v[:, a:cut], g[:, a:cut], beta[:, a:cut],
                           scale=1.0, initial_state=h0[2:3], lib_path=lib)
        oB, hB = oracle_fwd(q[:, cut:b], k[:, cut:b], v[:, cut:b], g[:, cut:b], beta[:, cut:b],
                            scale=1.0, initial_state=hA, lib_path=lib)
        assert np.array_equal(oB, o[:, cut:b]) and np.array_equal(hB[0], ht[2]), "state carry"


def check_non_expansive(lib):
    """||k|| = 1, beta in [0, 2], decays <= 1: ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    r = _rng(32)
    T, K, V = 20, 6, 4
    k = _unit_rows(r.standard_normal((1, T, 1, K)))
    v, g = r.standard_normal((1, T, 1, V)), r.uniform(-0.5, 0, (1, T, 1, K))
    beta = r.uniform(0, 2, (1, T, 1))
    h0 = r.standard_normal((1, 1, K, V))
    prev = np.linalg.norm(h0)
    for t in range(1, T + 1):
        _, ht = oracle_fwd(k[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], scale=1.0,
                           initial_state=h0, lib_path=lib)
        now = np.linalg.norm(ht)
        assert now <= prev + beta[0, t - 1, 0] * np.linalg.norm(v[0, t - 1, 0]) + 1e-12
        prev = now


ALL_CHECKS = [
    check_chunk_form, check_chunk_states, check_beta_zero_pure_decay, check_constant_state, check_exact_write,
    check_reflected_write, check_single_token, check_hand_worked, check_gate_closed_forms,
    check_gate_range_and_cumsum, check_gate_parameter_layout, check_beta_modes, check_l2norm_and_scale, check_gva_mapping,
    check_varlen_and_carry, check_non_expansive,
]
