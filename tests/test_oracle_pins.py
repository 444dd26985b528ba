"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something other than its own code: hand
derivations, exact rational brute force in a different formulation, closed
forms, invariants of the delta rule, special cases that reduce to a library
routine, and equivariances of the slot indexing. A plausible mistake (a
dropped decay, a sign, a transposed tile, a wrong head or slot index, an
update applied after instead of before the read-out) fails at least one.
"""
import json
import math
import os
from fractions import Fraction as F

import numpy as np
import pytest
import scipy.special

import brute_rational as br
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
VARIANTS = {"lightning": oracle.LIGHTNING, "gdn": oracle.GDN, "kda": oracle.KDA}


def _frac(x):
    return F(x) if not isinstance(x, str) else F(x)


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- golden


def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_worked_k2.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    var = case["variant"]
    toks = case["tokens"]
    T = len(toks)
    S0 = np.array(case["S0"], dtype=float)
    V, K = S0.shape
    q = np.array([[[float(_frac(x)) for x in t["q"]]] for t in toks])[None]
    k = np.array([[[float(_frac(x)) for x in t["k"]]] for t in toks])[None]
    v = np.array([[[float(_frac(x)) for x in t["v"]]] for t in toks])[None]
    if var == "lightning":
        g = np.array([float(_frac(toks[0]["lam"]))])
        beta = None
    elif var == "gdn":
        g = np.array([[[math.log(float(_frac(t["alpha"])))] for t in toks]])
        beta = np.array([[[float(_frac(t["beta"]))] for t in toks]])
    else:
        g = np.array([[[[math.log(float(_frac(x))) for x in t["e"]]]
                       for t in toks]])
        beta = np.array([[[float(_frac(t["beta"]))] for t in toks]])
    pool = np.random.default_rng(0).normal(size=(case["pool_size"], 1, V, K))
    want_out = np.array([[float(_frac(x)) for x in o] for o in case["outputs"]])
    want_S = np.array([[float(_frac(x)) for x in row]
                       for row in case["final_state"]])
    if "token_slots" in case:
        table = case["token_slots"]
        seed = table[0][case["num_accepted"][0] - 1]
        pool[seed, 0] = S0
        res = oracle.decode(VARIANTS[var], q, k, v, g, beta, pool, [0],
                            inter=True, token_slots=table,
                            num_accepted=case["num_accepted"])
        S1 = np.array([[float(_frac(x)) for x in row]
                       for row in case["state_after_token0"]])
        assert _rel(res["pool"][table[0][0], 0], S1) < 1e-14
        written = set(table[0])
        w = table[0][T - 1]
    else:
        r, w = case["read_idx"][0], case["write_idx"][0]
        pool[r, 0] = S0
        res = oracle.decode(VARIANTS[var], q, k, v, g, beta, pool,
                            case["read_idx"], case["write_idx"], inter=True)
        written = {w}
    assert _rel(res["out"][0, :, 0, :], want_out) < 1e-14
    assert _rel(res["pool"][w, 0], want_S) < 1e-14
    assert _rel(res["inter"][0, T - 1, 0], want_S) < 1e-14
    for s in range(case["pool_size"]):
        if s not in written:
            assert np.array_equal(res["pool"][s], pool[s])


# ------------------------------------------------------ rational brute force


def _dyadic(rng, shape, scale=16, lo=-16, hi=17):
    """Random dyadic rationals m/scale: exact in fp64."""
    return rng.integers(lo, hi, size=shape) / scale


def _to_frac(a):
    return [_to_frac(x) for x in a] if isinstance(a, (list, np.ndarray)) \
        else F(float(a))


@pytest.mark.parametrize("variant", ["lightning", "gdn", "kda"])
@pytest.mark.parametrize("V,K", [(4, 4), (3, 5), (5, 3)])
@pytest.mark.parametrize("T", [1, 2, 3])
def test_rational_brute_force(variant, V, K, T):
    """fp64 oracle vs exact product-form evaluation, several requests in a
    larger pool with permuted read slots, separate and skipped writes."""
    rng = np.random.default_rng(1000 * V + 10 * K + T + len(variant))
    B, H, HV, pool_size = 3, 1, 2, 6
    read_idx, write_idx = [4, 0, 2], [1, -1, 5]
    pool = _dyadic(rng, (pool_size, HV, V, K))
    q = _dyadic(rng, (B, T, H, K))
    k = _dyadic(rng, (B, T, H, K), lo=-8, hi=9)
    v = _dyadic(rng, (B, T, HV, V))
    if variant == "lightning":
        lam = rng.integers(1, 17, size=HV) / 16
        g, beta = lam, None
    elif variant == "gdn":
        alpha = rng.integers(1, 17, size=(B, T, HV)) / 16
        g, beta = np.log(alpha), rng.integers(0, 9, size=(B, T, HV)) / 8
    else:
        e = rng.integers(1, 17, size=(B, T, HV, K)) / 16
        g, beta = np.log(e), rng.integers(0, 9, size=(B, T, HV)) / 8
    res = oracle.decode(VARIANTS[variant], q, k, v, g, beta, pool, read_idx,
                        write_idx, inter=True)
    for b in range(B):
        for hv in range(HV):
            toks = []
            for t in range(T):
                tok = dict(q=_to_frac(q[b, t, 0]), k=_to_frac(k[b, t, 0]),
                           v=_to_frac(v[b, t, hv]))
                if variant == "lightning":
                    tok["lam"] = F(float(lam[hv]))
                elif variant == "gdn":
                    tok["alpha"] = F(float(alpha[b, t, hv]))
                    tok["beta"] = F(float(beta[b, t, hv]))
                else:
                    tok["e"] = _to_frac(e[b, t, hv])
                    tok["beta"] = F(float(beta[b, t, hv]))
                toks.append(tok)
            outs, states = br.run(variant, _to_frac(pool[read_idx[b], hv]),
                                  toks)
            scale = max(1.0, max(abs(float(x)) for st in states
                                 for row in st for x in row))
            for t in range(T):
                o = np.array([float(x) for x in outs[t]])
                st = np.array([[float(x) for x in row] for row in states[t]])
                assert np.max(np.abs(res["out"][b, t, hv] - o)) <= 1e-14 * scale * K
                assert np.max(np.abs(res["inter"][b, t, hv] - st)) <= 1e-14 * scale
            if write_idx[b] >= 0:
                assert np.max(np.abs(res["pool"][write_idx[b], hv] - st)) \
                    <= 1e-14 * scale
    # slots 0, 3 and the read-only slots stay as they were
    for s in (0, 3, 4, 2):
        if s not in write_idx:
            assert np.array_equal(res["pool"][s], pool[s])


# ------------------------------------------------------------- invariants


def _random_case(rng, variant, B=2, T=3, H=2, HV=2, K=8, V=6, pool_size=5):
    pool = rng.normal(size=(pool_size, HV, V, K)) * 0.3
    q = rng.normal(size=(B, T, H, K))
    k = rng.normal(size=(B, T, H, K))
    v = rng.normal(size=(B, T, HV, V))
    if variant == oracle.LIGHTNING:
        g, beta = rng.uniform(0.5, 1.0, size=HV), None
    elif variant == oracle.GDN:
        g, beta = rng.uniform(-1, 0, size=(B, T, HV)), rng.normal(size=(B, T, HV))
    else:
        g = rng.uniform(-1, 0, size=(B, T, HV, K))
        beta = rng.normal(size=(B, T, HV))
    return dict(q=q, k=k, v=v, g=g, beta=beta, pool=pool)


@pytest.mark.parametrize("variant", [oracle.GDN, oracle.KDA])
def test_delta_rule_writes_value_at_unit_key(variant):
    """beta = 1 and |k| = 1: after the update S k = v, whatever the decay."""
    rng = np.random.default_rng(7)
    B, T, H, HV, K, V = 2, 1, 1, 3, 16, 12
    c = _random_case(rng, variant, B=B, T=T, H=H, HV=HV, K=K, V=V)
    k = c["k"] / np.linalg.norm(c["k"], axis=-1, keepdims=True)
    beta = np.ones((B, T, HV))
    res = oracle.decode(variant, c["q"], k, c["v"], c["g"], beta, c["pool"],
                        [1, 3], inter=True)
    for b in range(B):
        for hv in range(HV):
            S = res["inter"][b, 0, hv]
            assert _rel(S @ k[b, 0, 0], c["v"][b, 0, hv]) < 1e-12
    # exact with a coordinate key: column j of the new state equals v
    kj = np.zeros_like(k)
    kj[..., 5] = 1.0
    res = oracle.decode(variant, c["q"], kj, c["v"], c["g"], beta, c["pool"],
                        [1, 3], inter=True)
    for b in range(B):
        for hv in range(HV):
            assert _rel(res["inter"][b, 0, hv][:, 5], c["v"][b, 0, hv]) < 1e-15


@pytest.mark.parametrize("variant", [oracle.GDN, oracle.KDA])
def test_zero_beta_zero_gate_is_identity(variant):
    rng = np.random.default_rng(8)
    c = _random_case(rng, variant)
    g = np.zeros_like(c["g"])
    beta = np.zeros_like(c["beta"])
    res = oracle.decode(variant, c["q"], c["k"], c["v"], g, beta, c["pool"],
                        [3, 0], inter=True)
    for b, r in enumerate([3, 0]):
        for hv in range(2):
            S0 = c["pool"][r, hv]
            np.testing.assert_array_equal(res["pool"][r, hv], S0)
            h = hv // 1
            for t in range(3):
                np.testing.assert_allclose(res["out"][b, t, hv],
                                           S0 @ c["q"][b, t, h], rtol=1e-14)


def test_lightning_closed_form():
    """Unrolled Lightning recurrence = decay-masked linear attention:
    o_t = lam^(t+1) S0 q_t + sum_{s<=t} lam^(t-s) (k_s . q_t) v_s and
    S_T = lam^T S0 + sum_t lam^(T-1-t) v_t k_t^T."""
    rng = np.random.default_rng(9)
    B, T, H, K, V = 1, 8, 3, 16, 12
    c = _random_case(rng, oracle.LIGHTNING, B=B, T=T, H=H, HV=H, K=K, V=V,
                     pool_size=2)
    lam = c["g"]
    res = oracle.decode(oracle.LIGHTNING, c["q"], c["k"], c["v"], lam, None,
                        c["pool"], [1])
    for h in range(H):
        Q, Kt, Vt = c["q"][0, :, h], c["k"][0, :, h], c["v"][0, :, h]
        S0 = c["pool"][1, h]
        ts = np.arange(T)
        mask = np.tril(lam[h] ** (ts[:, None] - ts[None, :]).astype(float))
        A = (Q @ Kt.T) * mask                        # [T, T]
        want = A @ Vt + (lam[h] ** (ts + 1))[:, None] * (Q @ S0.T)
        assert _rel(res["out"][0, :, h], want) < 1e-13
        ST = lam[h] ** T * S0 + (Vt.T * lam[h] ** (T - 1 - ts)) @ Kt
        assert _rel(res["pool"][1, h], ST) < 1e-13


def test_lightning_builtin_decay_schedule():
    """No decay array: head h of H decays by exp(-2^(-8(h+1)/H))."""
    H, K, V = 8, 4, 4
    pool = np.ones((1, H, V, K))
    z = np.zeros((1, 1, H, K))
    res = oracle.decode(oracle.LIGHTNING, z, z, np.zeros((1, 1, H, V)), None,
                        None, pool, [0])
    # exp(-1/2) and exp(-1/256), written out
    assert abs(res["pool"][0, 0, 0, 0] - 0.6065306597126334) < 1e-15
    assert abs(res["pool"][0, 7, 0, 0] - 0.9961013694701175) < 1e-15
    vals = res["pool"][0, :, 0, 0]
    assert np.all(np.diff(vals) > 0)


def test_named_lightning_decays_follow_the_schedule():
    """The Lightning workload hands both sides an fp32 decay array: it is the
    oracle's own schedule (same head indexing) rounded once to fp32, so a
    call with it matches a call without it to fp32 rounding of the decays."""
    import workloads as W
    HV, K, V = 64, 4, 4
    lam = W.head_decays(HV)
    assert lam.dtype.is_floating_point and lam.element_size() == 4
    rng = np.random.default_rng(12)
    pool = rng.standard_normal((2, HV, V, K))
    q = rng.standard_normal((1, 1, HV, K))
    k = rng.standard_normal((1, 1, HV, K))
    v = rng.standard_normal((1, 1, HV, V))
    a = oracle.decode(oracle.LIGHTNING, q, k, v, None, None, pool, [1])
    b = oracle.decode(oracle.LIGHTNING, q, k, v, lam.double().numpy(), None,
                      pool, [1])
    assert _rel(b["pool"], a["pool"]) < 1e-7
    assert _rel(b["out"], a["out"]) < 1e-7
    # and not the schedule of another head count
    c = oracle.decode(oracle.LIGHTNING, q, k, v,
                      W.head_decays(32).repeat(2).double().numpy(), None,
                      pool, [1])
    assert _rel(c["pool"], a["pool"]) > 1e-3


def test_kda_constant_gate_equals_gdn():
    rng = np.random.default_rng(10)
    c = _random_case(rng, oracle.GDN)
    gk = np.repeat(c["g"][..., None], c["q"].shape[-1], axis=-1)
    a = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"], c["beta"],
                      c["pool"], [2, 4], flags=oracle.BETA_LOGIT)
    b = oracle.decode(oracle.KDA, c["q"], c["k"], c["v"], gk, c["beta"],
                      c["pool"], [2, 4], flags=oracle.BETA_LOGIT)
    assert _rel(b["out"], a["out"]) < 1e-14
    assert _rel(b["pool"], a["pool"]) < 1e-14


def test_gdn_zero_beta_is_pure_decay():
    rng = np.random.default_rng(11)
    c = _random_case(rng, oracle.GDN, B=1, T=4, H=1, HV=1)
    beta = np.zeros((1, 4, 1))
    res = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"], beta,
                        c["pool"], [2], inter=True)
    S0 = c["pool"][2, 0]
    cum = np.cumsum(c["g"][0, :, 0])
    for t in range(4):
        assert _rel(res["inter"][0, t, 0], math.exp(cum[t]) * S0) < 1e-14
        assert _rel(res["out"][0, t, 0], math.exp(cum[t]) * (S0 @ c["q"][0, t, 0])) < 1e-13


def test_ungated_delta_rule_orthonormal_keys():
    """g = 0, beta = 1 and orthonormal keys: every token's value is stored
    exactly at its key and directions orthogonal to all keys keep S0."""
    rng = np.random.default_rng(12)
    K, V, T = 8, 5, 4
    Qm, _ = np.linalg.qr(rng.normal(size=(K, K)))
    keys = Qm[:, :T].T                                # [T, K]
    v = rng.normal(size=(1, T, 1, V))
    pool = rng.normal(size=(1, 1, V, K))
    res = oracle.decode(oracle.GDN, rng.normal(size=(1, T, 1, K)),
                        keys[None, :, None, :], v, np.zeros((1, T, 1)),
                        np.ones((1, T, 1)), pool, [0])
    S = res["pool"][0, 0]
    for t in range(T):
        assert _rel(S @ keys[t], v[0, t, 0]) < 1e-12
    for j in range(T, K):
        assert _rel(S @ Qm[:, j], pool[0, 0] @ Qm[:, j]) < 1e-12


@pytest.mark.parametrize("variant", [oracle.LIGHTNING, oracle.GDN, oracle.KDA])
def test_token_split_equals_multi_token(variant):
    """T single-token calls chained through the pool = one T-token call."""
    rng = np.random.default_rng(13)
    c = _random_case(rng, variant, T=4)
    flags = 0 if variant == oracle.LIGHTNING else oracle.BETA_LOGIT
    whole = oracle.decode(variant, c["q"], c["k"], c["v"], c["g"], c["beta"],
                          c["pool"], [1, 4], flags=flags, inter=True)
    pool = c["pool"]
    for t in range(4):
        sl = slice(t, t + 1)
        g = c["g"] if variant == oracle.LIGHTNING else c["g"][:, sl]
        beta = None if c["beta"] is None else c["beta"][:, sl]
        step = oracle.decode(variant, c["q"][:, sl], c["k"][:, sl],
                             c["v"][:, sl], g, beta, pool, [1, 4], flags=flags)
        assert _rel(step["out"][:, 0], whole["out"][:, t]) < 1e-14
        pool = step["pool"]
    assert _rel(pool, whole["pool"]) < 1e-14


def test_grouped_value_heads_equal_repeated_qk():
    """HV = 2H with value head hv reading q/k head hv // 2 is the H = HV run
    with q and k repeated along heads."""
    rng = np.random.default_rng(14)
    c = _random_case(rng, oracle.GDN, H=2, HV=4)
    a = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"], c["beta"],
                      c["pool"], [0, 3], flags=oracle.L2NORM_QK)
    q2 = np.repeat(c["q"], 2, axis=2)
    k2 = np.repeat(c["k"], 2, axis=2)
    b = oracle.decode(oracle.GDN, q2, k2, c["v"], c["g"], c["beta"],
                      c["pool"], [0, 3], flags=oracle.L2NORM_QK)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["pool"], b["pool"])


@pytest.mark.parametrize("pattern", [
    ("identity", 4, [0, 1, 2, 3]),
    ("non_identity", 6, [2, 0, 5, 1]),
    ("reversed", 4, [3, 2, 1, 0]),
])
def test_slot_indexing_equals_direct_evaluation(pattern):
    """Index patterns of the cuLA pool tests: request b's result equals a
    one-request call on its own slot, and only written slots change."""
    _, pool_size, ridx = pattern
    rng = np.random.default_rng(15)
    c = _random_case(rng, oracle.GDN, B=4, pool_size=pool_size)
    whole = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"],
                          c["beta"], c["pool"], ridx, inter=True)
    for b in range(4):
        sl = slice(b, b + 1)
        one = oracle.decode(oracle.GDN, c["q"][sl], c["k"][sl], c["v"][sl],
                            c["g"][sl], c["beta"][sl],
                            c["pool"][ridx[b]:ridx[b] + 1], [0], inter=True)
        np.testing.assert_array_equal(whole["out"][b], one["out"][0])
        np.testing.assert_array_equal(whole["pool"][ridx[b]], one["pool"][0])
    for s in range(pool_size):
        if s not in ridx:
            np.testing.assert_array_equal(whole["pool"][s], c["pool"][s])


def test_padding_and_skipped_writes():
    rng = np.random.default_rng(16)
    c = _random_case(rng, oracle.KDA, B=3, pool_size=6)
    res = oracle.decode(oracle.KDA, c["q"], c["k"], c["v"], c["g"], c["beta"],
                        c["pool"], [2, -1, 5], [1, 3, -1], inter=True)
    # padded request: zero outputs, no cache rows, no pool write
    assert not res["out"][1].any()
    assert np.isnan(res["inter"][1]).all()  # no cache row written
    # skipped write: outputs and cache are still computed
    assert np.abs(res["out"][2]).max() > 0 and np.abs(res["inter"][2]).max() > 0
    changed = [s for s in range(6)
               if not np.array_equal(res["pool"][s], c["pool"][s])]
    assert changed == [1]
    np.testing.assert_array_equal(res["pool"][1], res["inter"][0, -1])


def test_l2norm_and_beta_logit_flags():
    rng = np.random.default_rng(17)
    c = _random_case(rng, oracle.GDN)
    qn = c["q"] / np.linalg.norm(c["q"], axis=-1, keepdims=True)
    kn = c["k"] / np.linalg.norm(c["k"], axis=-1, keepdims=True)
    ref = oracle.decode(oracle.GDN, qn, kn, c["v"], c["g"],
                        scipy.special.expit(c["beta"]), c["pool"], [0, 1])
    # large scales make the 1e-6 guard under the square root negligible
    got = oracle.decode(oracle.GDN, 1000.0 * c["q"], 300.0 * c["k"], c["v"],
                        c["g"], c["beta"], c["pool"], [0, 1],
                        flags=oracle.L2NORM_QK | oracle.BETA_LOGIT)
    assert _rel(got["out"], ref["out"]) < 1e-10
    assert _rel(got["pool"], ref["pool"]) < 1e-10


def test_l2norm_of_zero_vectors_stays_finite():
    """A zero key leaves the decayed state without a delta write and a zero
    query gives a zero output: the guard under the square root keeps both
    finite."""
    rng = np.random.default_rng(18)
    c = _random_case(rng, oracle.GDN, B=1, T=1, H=1, HV=1)
    z = np.zeros_like(c["q"])
    res = oracle.decode(oracle.GDN, z, z, c["v"], c["g"], c["beta"],
                        c["pool"], [2], flags=oracle.L2NORM_QK)
    assert not res["out"].any()
    alpha = math.exp(c["g"][0, 0, 0])
    assert _rel(res["pool"][2, 0], alpha * c["pool"][2, 0]) < 1e-15


# ---------------------------------------------- paged per-token state slots


@pytest.mark.parametrize("variant", ["lightning", "gdn", "kda"])
def test_paged_slots_rational_brute_force(variant):
    """Per-token slot table against the exact product form: the seed comes
    from the slot of the last accepted token and every token's state lands
    in its own slot (negative entries skip)."""
    rng = np.random.default_rng(77 + len(variant))
    B, T, H, HV, V, K, pool_size = 3, 3, 1, 2, 3, 4, 12
    table = [[4, 0, 7], [2, -1, 9], [5, 11, 1]]
    accepted = [2, 1, 3]
    pool = _dyadic(rng, (pool_size, HV, V, K))
    q = _dyadic(rng, (B, T, H, K))
    k = _dyadic(rng, (B, T, H, K), lo=-8, hi=9)
    v = _dyadic(rng, (B, T, HV, V))
    if variant == "lightning":
        lam = rng.integers(1, 17, size=HV) / 16
        g, beta = lam, None
    elif variant == "gdn":
        alpha = rng.integers(1, 17, size=(B, T, HV)) / 16
        g, beta = np.log(alpha), rng.integers(0, 9, size=(B, T, HV)) / 8
    else:
        e = rng.integers(1, 17, size=(B, T, HV, K)) / 16
        g, beta = np.log(e), rng.integers(0, 9, size=(B, T, HV)) / 8
    res = oracle.decode(VARIANTS[variant], q, k, v, g, beta, pool, [0] * B,
                        token_slots=table, num_accepted=accepted)
    written = set()
    for b in range(B):
        seed = table[b][accepted[b] - 1]
        for hv in range(HV):
            toks = []
            for t in range(T):
                tok = dict(q=_to_frac(q[b, t, 0]), k=_to_frac(k[b, t, 0]),
                           v=_to_frac(v[b, t, hv]))
                if variant == "lightning":
                    tok["lam"] = F(float(lam[hv]))
                elif variant == "gdn":
                    tok["alpha"] = F(float(alpha[b, t, hv]))
                    tok["beta"] = F(float(beta[b, t, hv]))
                else:
                    tok["e"] = _to_frac(e[b, t, hv])
                    tok["beta"] = F(float(beta[b, t, hv]))
                toks.append(tok)
            outs, states = br.run(variant, _to_frac(pool[seed, hv]), toks)
            for t in range(T):
                o = np.array([float(x) for x in outs[t]])
                assert np.max(np.abs(res["out"][b, t, hv] - o)) <= 1e-12
                if table[b][t] >= 0:
                    st = np.array([[float(x) for x in row] for row in states[t]])
                    assert np.max(np.abs(res["pool"][table[b][t], hv] - st)) <= 1e-12
                    written.add(table[b][t])
    for s in range(pool_size):
        if s not in written:
            np.testing.assert_array_equal(res["pool"][s], pool[s])


def test_paged_slots_equal_scattered_cache():
    """Paged mode = classic mode reading the seed slot with the per-token
    cache on, the cache rows scattered to the table's slots."""
    rng = np.random.default_rng(78)
    c = _random_case(rng, oracle.KDA, B=3, T=4, pool_size=16)
    table = np.array([[3, 8, 9, 10], [12, 0, -1, 13], [5, 6, 7, 14]])
    accepted = np.array([4, 1, 2])
    paged = oracle.decode(oracle.KDA, c["q"], c["k"], c["v"], c["g"],
                          c["beta"], c["pool"], [0, 0, 0],
                          flags=oracle.L2NORM_QK | oracle.BETA_LOGIT,
                          token_slots=table, num_accepted=accepted)
    seeds = [table[b, accepted[b] - 1] for b in range(3)]
    dense = oracle.decode(oracle.KDA, c["q"], c["k"], c["v"], c["g"],
                          c["beta"], c["pool"], seeds, [-1, -1, -1],
                          flags=oracle.L2NORM_QK | oracle.BETA_LOGIT,
                          inter=True)
    np.testing.assert_array_equal(paged["out"], dense["out"])
    want = c["pool"].copy()
    for b in range(3):
        for t in range(4):
            if table[b, t] >= 0:
                want[table[b, t]] = dense["inter"][b, t]
    np.testing.assert_array_equal(paged["pool"], want)


@pytest.mark.parametrize("bad", [0, 5, -2])
def test_paged_slots_out_of_range_accepted_count_is_padding(bad):
    """An accepted count outside [1, T] (the aiter reviewer's zero-accepted
    case) never indexes the table: the request is padding."""
    rng = np.random.default_rng(79)
    c = _random_case(rng, oracle.GDN, B=2, T=4, pool_size=10)
    table = [[1, 2, 3, 4], [5, 6, 7, 8]]
    res = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"],
                        c["beta"], c["pool"], [0, 0], token_slots=table,
                        num_accepted=[2, bad])
    assert not res["out"][1].any()
    for s in (5, 6, 7, 8):
        np.testing.assert_array_equal(res["pool"][s], c["pool"][s])
    assert np.abs(res["out"][0]).max() > 0


def test_paged_slots_negative_seed_is_padding():
    rng = np.random.default_rng(80)
    c = _random_case(rng, oracle.GDN, B=1, T=2, pool_size=4)
    res = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"],
                        c["beta"], c["pool"], [0], token_slots=[[-1, 3]],
                        num_accepted=[1])
    assert not res["out"].any()
    np.testing.assert_array_equal(res["pool"], c["pool"])


# ------------------------------------------------- factor records and replay


@pytest.mark.parametrize("variant", [oracle.LIGHTNING, oracle.GDN, oracle.KDA])
def test_factor_records_rebuild_every_token_state(variant):
    """Replaying the first n records from the seed gives the state after
    token n-1 (the per-token cache), for every n; a record's decay, key and
    coefficient are the ones the update used."""
    rng = np.random.default_rng(90 + variant)
    B, T, HV, K, V = 3, 4, 2, 6, 5
    c = _random_case(rng, variant, B=B, T=T, H=1, HV=HV, K=K, V=V,
                     pool_size=7)
    flags = 0 if variant == oracle.LIGHTNING else (
        oracle.L2NORM_QK | oracle.BETA_LOGIT)
    ridx = [5, 0, 3]
    res = oracle.decode(variant, c["q"], c["k"], c["v"], c["g"], c["beta"],
                        c["pool"], ridx, [-1, -1, -1], flags=flags,
                        inter=True, factors=True)
    fac = res["factors"]
    assert np.isfinite(fac).all()
    for n in range(0, T + 1):
        rebuilt = oracle.replay(fac, c["pool"], ridx, [1, 2, 4], [n] * B)
        for b in range(B):
            want = c["pool"][ridx[b]] if n == 0 else res["inter"][b, n - 1]
            assert _rel(rebuilt[[1, 2, 4][b]], want) < 1e-13
    # the records themselves
    a, kk, err = fac[..., :K], fac[..., K:2 * K], fac[..., 2 * K:]
    if variant == oracle.KDA:
        np.testing.assert_allclose(a, np.exp(c["g"]), rtol=1e-15)
    elif variant == oracle.GDN:
        np.testing.assert_allclose(a, np.exp(c["g"])[..., None].repeat(K, -1),
                                   rtol=1e-15)
    else:
        np.testing.assert_allclose(a[0, 0], c["g"][:, None].repeat(K, -1),
                                   rtol=1e-15)
    if variant != oracle.LIGHTNING:
        np.testing.assert_allclose(np.linalg.norm(kk, axis=-1), 1.0,
                                   rtol=1e-6)
    else:
        np.testing.assert_array_equal(err, c["v"])


def test_replay_skips_and_bounds():
    """Zero records copy the seed to the write slot; a negative read slot or
    a count outside [0, T] leaves the pool alone."""
    rng = np.random.default_rng(95)
    c = _random_case(rng, oracle.GDN, B=3, T=2, H=1, HV=1, K=4, V=3,
                     pool_size=6)
    res = oracle.decode(oracle.GDN, c["q"], c["k"], c["v"], c["g"], c["beta"],
                        c["pool"], [0, 1, 2], [-1, -1, -1], factors=True)
    out = oracle.replay(res["factors"], c["pool"], [0, -1, 2], [3, 4, 5],
                        [0, 1, 3])
    np.testing.assert_array_equal(out[3], c["pool"][0])
    for s in (0, 1, 2, 4, 5):
        np.testing.assert_array_equal(out[s], c["pool"][s])


# ---------------------------------------------------- variable-length batches


def _pack(x, lengths, T):
    """[B, T, ...] -> token-packed [sum(lengths), ...] (first lengths[b] of
    each request)."""
    return np.concatenate([x[b, :n] for b, n in enumerate(lengths)], axis=0)


def _varlen_case(rng, variant, lengths, T, H=1, HV=2, K=5, V=4, pool_size=9):
    B = len(lengths)
    c = _random_case(rng, variant, B=B, T=T, H=H, HV=HV, K=K, V=V,
                     pool_size=pool_size)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    packed = {n: _pack(c[n], lengths, T) for n in ("q", "k", "v")}
    packed["g"] = c["g"] if variant == oracle.LIGHTNING else _pack(
        c["g"], lengths, T)
    packed["beta"] = None if c["beta"] is None else _pack(c["beta"], lengths, T)
    return c, packed, cu


@pytest.mark.parametrize("variant", [oracle.LIGHTNING, oracle.GDN, oracle.KDA])
def test_varlen_equal_lengths_equals_dense(variant):
    """Offsets 0, T, 2T, ... over the packed tokens are the dense batch."""
    rng = np.random.default_rng(200 + variant)
    T = 3
    c, p, cu = _varlen_case(rng, variant, [T, T, T], T)
    flags = 0 if variant == oracle.LIGHTNING else oracle.BETA_LOGIT
    ridx, widx = [4, 0, 7], [1, 8, 2]
    dense = oracle.decode(variant, c["q"], c["k"], c["v"], c["g"], c["beta"],
                          c["pool"], ridx, widx, flags=flags, inter=True,
                          factors=True)
    var = oracle.decode(variant, p["q"], p["k"], p["v"], p["g"], p["beta"],
                        c["pool"], ridx, widx, flags=flags, inter=True,
                        factors=True, cu_seqlens=cu)
    np.testing.assert_array_equal(var["out"], dense["out"].reshape(9, 2, 4))
    np.testing.assert_array_equal(var["pool"], dense["pool"])
    np.testing.assert_array_equal(var["inter"],
                                  dense["inter"].reshape((9,) + dense["inter"].shape[2:]))
    np.testing.assert_array_equal(var["factors"],
                                  dense["factors"].reshape((9,) + dense["factors"].shape[2:]))


@pytest.mark.parametrize("variant", [oracle.LIGHTNING, oracle.GDN, oracle.KDA])
def test_varlen_equals_separate_requests(variant):
    """A variable-length batch is its requests run one by one, each with its
    own token count; a request of zero tokens copies its read state to its
    write slot and produces no output."""
    rng = np.random.default_rng(210 + variant)
    lengths, T = [2, 0, 4, 1], 4
    c, p, cu = _varlen_case(rng, variant, lengths, T, pool_size=10)
    flags = 0 if variant == oracle.LIGHTNING else (
        oracle.BETA_LOGIT | oracle.L2NORM_QK)
    ridx, widx = [3, 6, 0, 9], [5, 1, 0, 2]
    var = oracle.decode(variant, p["q"], p["k"], p["v"], p["g"], p["beta"],
                        c["pool"], ridx, widx, flags=flags, inter=True,
                        factors=True, cu_seqlens=cu, max_tokens=T)
    assert var["out"].shape[0] == sum(lengths)
    want_pool = c["pool"].copy()
    for b, n in enumerate(lengths):
        if n == 0:
            want_pool[widx[b]] = c["pool"][ridx[b]]
            continue
        sl = slice(0, n)
        g = c["g"] if variant == oracle.LIGHTNING else c["g"][b:b + 1, sl]
        beta = None if c["beta"] is None else c["beta"][b:b + 1, sl]
        one = oracle.decode(variant, c["q"][b:b + 1, sl], c["k"][b:b + 1, sl],
                            c["v"][b:b + 1, sl], g, beta, c["pool"],
                            [ridx[b]], [widx[b]], flags=flags, inter=True,
                            factors=True)
        rows = slice(cu[b], cu[b + 1])
        np.testing.assert_array_equal(var["out"][rows], one["out"][0])
        np.testing.assert_array_equal(var["inter"][rows], one["inter"][0])
        np.testing.assert_array_equal(var["factors"][rows], one["factors"][0])
        want_pool[widx[b]] = one["pool"][widx[b]]
    np.testing.assert_array_equal(var["pool"], want_pool)


def test_varlen_padding_and_paged_slots():
    """Padding (negative read slot) zeroes only the request's own packed
    outputs; with a slot table the accepted count is checked against the
    request's own token count."""
    rng = np.random.default_rng(220)
    lengths, T = [3, 1, 2], 3
    c, p, cu = _varlen_case(rng, oracle.GDN, lengths, T, pool_size=12)
    res = oracle.decode(oracle.GDN, p["q"], p["k"], p["v"], p["g"], p["beta"],
                        c["pool"], [2, -1, 5], None, cu_seqlens=cu)
    assert not res["out"][3].any()
    assert np.isfinite(res["out"]).all() and res["out"][[0, 1, 2, 4, 5]].any()
    table = np.array([[0, 1, 2, -1], [3, 7, -1, -1], [4, 6, -1, -1]],
                     dtype=np.int32)
    # request 1 has one token, so an accepted count of 2 makes it padding
    # (its table entry 1 is a valid slot, which it must not read)
    acc = np.array([2, 2, 1], dtype=np.int32)
    paged = oracle.decode(oracle.GDN, p["q"], p["k"], p["v"], p["g"],
                          p["beta"], c["pool"], None, token_slots=table,
                          num_accepted=acc, cu_seqlens=cu, inter=True)
    assert not paged["out"][3].any()
    for b, n in enumerate(lengths):
        if b == 1:
            continue
        rows = slice(cu[b], cu[b + 1])
        one = oracle.decode(oracle.GDN, c["q"][b:b + 1, :n],
                            c["k"][b:b + 1, :n], c["v"][b:b + 1, :n],
                            c["g"][b:b + 1, :n], c["beta"][b:b + 1, :n],
                            c["pool"], None, token_slots=table[b:b + 1],
                            num_accepted=acc[b:b + 1], inter=True)
        np.testing.assert_array_equal(paged["out"][rows], one["out"][0])
        np.testing.assert_array_equal(paged["inter"][rows], one["inter"][0])
        for t in range(n):
            s = table[b, t]
            np.testing.assert_array_equal(paged["pool"][s], one["pool"][s])
    np.testing.assert_array_equal(paged["pool"][3], c["pool"][3])
    np.testing.assert_array_equal(paged["pool"][7], c["pool"][7])


def test_varlen_replay_equals_per_request_cache():
    rng = np.random.default_rng(230)
    lengths, T = [3, 0, 2], 3
    c, p, cu = _varlen_case(rng, oracle.KDA, lengths, T, pool_size=8)
    ridx = [1, 4, 6]
    res = oracle.decode(oracle.KDA, p["q"], p["k"], p["v"], p["g"], p["beta"],
                        c["pool"], ridx, [-1, -1, -1], inter=True,
                        factors=True, cu_seqlens=cu)
    ntok = [2, 0, 2]
    out = oracle.replay(res["factors"], c["pool"], ridx, [0, 2, 3], ntok,
                        cu_seqlens=cu)
    np.testing.assert_allclose(out[0], res["inter"][cu[0] + 1], rtol=0,
                               atol=1e-13)
    np.testing.assert_array_equal(out[2], c["pool"][4])
    np.testing.assert_allclose(out[3], res["inter"][cu[2] + 1], rtol=0,
                               atol=1e-13)
    # a count beyond the request's own tokens skips it
    out = oracle.replay(res["factors"], c["pool"], ridx, [0, 2, 3], [1, 1, 3],
                        cu_seqlens=cu)
    np.testing.assert_array_equal(out[2], c["pool"][2])
    np.testing.assert_array_equal(out[3], c["pool"][3])


@pytest.mark.parametrize("cu", [[0, 2, 1, 3], [1, 2, 3, 5], [0, 4, 4, 5],
                                [-1, 0, 2, 3]])
def test_varlen_rejects_bad_offsets(cu):
    """Offsets must be non-decreasing, inside [0, total], and no request may
    hold more than T tokens."""
    rng = np.random.default_rng(240)
    c, p, _ = _varlen_case(rng, oracle.GDN, [1, 1, 2], 2, pool_size=6)
    with pytest.raises(ValueError):
        oracle.decode(oracle.GDN, p["q"][:4], p["k"][:4], p["v"][:4],
                      p["g"][:4], p["beta"][:4], c["pool"], [0, 1, 2],
                      cu_seqlens=np.array(cu, dtype=np.int32), max_tokens=3)


# ------------------------------------------- in-kernel gate chain (a reading)
# The pages name the chain's inputs but not its formula (parity unpinned
# against the pages). These pins fix the implementation of the reading the
# oracle states: closed forms of softplus and sigmoid at 0, the limits, and
# the per-head / per-channel indexing of A_log and dt_bias.


def _gate_case(variant, seed, HV=3, K=4):
    rng = np.random.default_rng(seed)
    c = _random_case(rng, variant, B=2, T=2, H=1, HV=HV, K=K, V=3,
                     pool_size=4)
    dt = rng.normal(size=(HV,) if variant == oracle.GDN else (HV, K))
    return c, dt


def _run_gate(variant, c, g, **kw):
    return oracle.decode(variant, c["q"], c["k"], c["v"], g, c["beta"],
                         c["pool"], [0, 2], [1, 3], inter=True,
                         factors=True, **kw)


def _decays(res, K):
    return res["factors"][..., :K]


@pytest.mark.parametrize("variant", [oracle.GDN, oracle.KDA])
def test_gate_chain_softplus_at_zero_halves(variant):
    """x + dt_bias = 0 with A_log = 0: g' = -softplus(0) = -ln 2, every decay
    is exactly 1/2, and the call equals the ungated one with g = ln(1/2)."""
    c, dt = _gate_case(variant, 300 + variant)
    HV = dt.shape[0]
    raw = -np.broadcast_to(dt[None, None] if variant == oracle.GDN
                           else dt[None, None], c["g"].shape).copy()
    gated = _run_gate(variant, c, raw, A_log=np.zeros(HV), dt_bias=dt)
    np.testing.assert_allclose(_decays(gated, 4), 0.5, rtol=1e-15)
    plain = _run_gate(variant, c, np.full(c["g"].shape, math.log(0.5)))
    assert _rel(gated["out"], plain["out"]) < 1e-13
    assert _rel(gated["pool"], plain["pool"]) < 1e-13


@pytest.mark.parametrize("variant", [oracle.GDN, oracle.KDA])
def test_gate_chain_scale_is_exp_a_log(variant):
    """A_log = ln 3 at x + dt = 0: g' = -3 ln 2, decay 1/8 in every head."""
    c, dt = _gate_case(variant, 310 + variant)
    raw = -np.broadcast_to(dt[None, None], c["g"].shape).copy()
    res = _run_gate(variant, c, raw, A_log=np.full(dt.shape[0], math.log(3)),
                    dt_bias=dt)
    np.testing.assert_allclose(_decays(res, 4), 0.125, rtol=1e-14)


@pytest.mark.parametrize("variant", [oracle.GDN, oracle.KDA])
def test_gate_chain_lower_bound_form(variant):
    """Bounded form: at x + dt = 0 the decay is exp(lb / 2) whatever A_log;
    far above 0 it tends to exp(lb), far below to 1; always inside
    (exp(lb), 1)."""
    c, dt = _gate_case(variant, 320 + variant)
    HV = dt.shape[0]
    a_log = np.random.default_rng(7).normal(size=HV)
    raw = -np.broadcast_to(dt[None, None], c["g"].shape).copy()
    lb = -5.0
    mid = _run_gate(variant, c, raw, A_log=a_log, dt_bias=dt, lower_bound=lb)
    np.testing.assert_allclose(_decays(mid, 4), math.exp(lb / 2), rtol=1e-14)
    hi = _run_gate(variant, c, raw + 60.0, A_log=np.zeros(HV), dt_bias=dt,
                   lower_bound=lb)
    np.testing.assert_allclose(_decays(hi, 4), math.exp(lb), rtol=1e-12)
    lo = _run_gate(variant, c, raw - 60.0, A_log=np.zeros(HV), dt_bias=dt,
                   lower_bound=lb)
    np.testing.assert_allclose(_decays(lo, 4), 1.0, rtol=1e-12)
    rnd = _run_gate(variant, c, np.random.default_rng(8).normal(
        size=c["g"].shape) * 3, A_log=a_log, dt_bias=dt, lower_bound=lb)
    d = _decays(rnd, 4)
    assert (d > math.exp(lb)).all() and (d < 1.0).all()


def test_gate_chain_kda_channel_indexing():
    """dt_bias is per (value head, key channel): raw gates equal to -dt_bias
    of their own head and channel give decay 1/2 everywhere; the transposed
    pattern does not."""
    HV, K = 3, 4
    c, dt = _gate_case(oracle.KDA, 330, HV=HV, K=K)
    raw = -np.broadcast_to(dt[None, None], c["g"].shape).copy()
    res = _run_gate(oracle.KDA, c, raw, A_log=np.zeros(HV), dt_bias=dt)
    np.testing.assert_allclose(_decays(res, K), 0.5, rtol=1e-15)
    wrong = -np.broadcast_to(dt.T.reshape(HV, K)[None, None], c["g"].shape)
    res = _run_gate(oracle.KDA, c, wrong.copy(), A_log=np.zeros(HV),
                    dt_bias=dt)
    assert np.abs(_decays(res, K) - 0.5).max() > 1e-3


def test_gate_chain_gdn_head_indexing_and_monotone():
    """GDN: one dt_bias per value head; a larger raw gate decays more."""
    c, dt = _gate_case(oracle.GDN, 340)
    HV = dt.shape[0]
    raw = -np.broadcast_to(dt[None, None], c["g"].shape).copy()
    base = _decays(_run_gate(oracle.GDN, c, raw, A_log=np.zeros(HV),
                             dt_bias=dt), 4)
    np.testing.assert_allclose(base, 0.5, rtol=1e-15)
    more = _decays(_run_gate(oracle.GDN, c, raw + 0.5, A_log=np.zeros(HV),
                             dt_bias=dt), 4)
    assert (more < base).all()


def test_gate_chain_refused_where_it_has_no_meaning():
    c, dt = _gate_case(oracle.GDN, 350)
    with pytest.raises(ValueError):  # lower bound without the chain
        _run_gate(oracle.GDN, c, c["g"], lower_bound=-5.0)
    with pytest.raises(ValueError):  # dt_bias of the wrong shape
        _run_gate(oracle.GDN, c, c["g"], A_log=np.zeros(3),
                  dt_bias=np.zeros((3, 4)))
