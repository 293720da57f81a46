"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Pages: "MassAlloc Attention: Let Attention Allocate Its Own Compute" --
agihunt.info summary (rule, tau -> 0, bound) and the jaehun.me review
("One tolerance governs everything", "Forward: online sparse softmax",
"Backward: offline sparse probabilities", Prop. 1 under "Theoretical upper
bound on forward omitted mass", "How it works: a concrete example").
"""
import json
import math
import os

import numpy as np
import pytest

import mala_gen as G
import pins
from oracle import oracle_bwd, oracle_decode, oracle_fwd
from oracle import ref_numpy as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def hand_value(expr: str) -> float:
    """Value of a fixture's hand-written expression: numbers, + - * / and
    parentheses, ln(...) for the natural log, inf."""
    import math
    if not set(expr) <= set("0123456789.+-*/() lninf"):
        raise ValueError(expr)
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log, "inf": math.inf}))


def assert_margin(got: float, expr: str):
    want = hand_value(expr)
    if math.isinf(want):
        assert got == want, (got, expr)
    else:
        assert abs(got - want) <= 1e-12 * max(1.0, abs(want)), (got, want, expr)


def _inputs(seed, B=1, L=300, Hq=4, Hkv=2, d=32, p=0.1, diffuse=()):
    inp = G.attn_inputs(100 + seed, B, L, Hq, Hkv, d, p, diffuse)
    return [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]


def _visited(keep):
    return keep != 255


# ---------------------------------------------------------------- worked example
def test_worked_example_forward_and_backward():
    """Page 2, 'How it works: a concrete example' (L=4, tau=1)."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    facts, tol = g["page_facts"], g["tolerances"]
    e = np.array(g["exp_scores"])
    E = np.tile(e, (4, 1))  # only row 3 (L=4) matters
    q, k = pins.scores_to_qk(E)
    v = np.random.default_rng(0).standard_normal((1, 4, 1, 4))
    f = oracle_fwd(q, k, v, facts["tau"], 1, 1)
    kept = sorted(int(j) for j in range(4) if f["keep"][0, 0, 3, j] == 1)
    assert kept == sorted(facts["retained_keys"])
    Z = np.exp(f["lse"][0, 0, 3])
    assert abs(Z - facts["final_normalizer"]) <= tol["final_normalizer_abs"]
    dense = e / e.sum()
    assert abs(dense[0] - facts["dense_mass_each_of_k0_k2"]) <= tol["dense_mass_abs"]
    assert abs(dense[2] - facts["dense_mass_each_of_k0_k2"]) <= tol["dense_mass_abs"]
    assert abs(f["omitted"][0, 0, 3] - facts["omitted_mass"]) <= tol["omitted_abs"]
    # the same facts from the key-by-key statement
    kk, ZR, om = R.per_key_row(e, facts["tau"])
    assert sorted(kk) == sorted(facts["retained_keys"]) and abs(ZR - facts["final_normalizer"]) < 0.005
    # backward with the final normaliser keeps both retained keys (7.39/27.49, 20.1/27.49 >= 1/4)
    dout = np.ones_like(v)
    b = oracle_bwd(q, k, v, f["o"], dout, f["lse"], facts["tau"], 1, 1)
    bk = sorted(int(j) for j in range(4) if b["keep"][0, 0, 3, j] == 1)
    assert bk == sorted(facts["retained_keys"])
    # decision log-margins of row 3, worked by hand from the exp-scores
    for m in g["margins"]["fwd"]:
        assert_margin(f["margin"][0, 0, 3, m["key"]], m["expr"])
    for m in g["margins"]["bwd"]:
        assert_margin(b["margin"][0, 0, 3, m["key"]], m["expr"])


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_rules.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_derived_rules(case):
    E = np.array(case["exp_scores"], dtype=np.float64)
    r0, nr = case["row0"], E.shape[0]
    L = E.shape[1]
    full = np.ones((L, L))
    full[r0:r0 + nr] = E
    q, k = pins.scores_to_qk(full)
    v = np.random.default_rng(1).standard_normal((1, L, 1, 3))
    Bq, Bk, tau = case["Bq"], case["Bk"], case["tau"]
    f = oracle_fwd(q, k, v, tau, Bq, Bk)
    km = pins.keep_to_keymask(f["keep"], L, Bq, Bk)
    for r in range(nr):
        i = r0 + r
        assert sorted(np.nonzero(km[0, 0, i])[0].tolist()) == case["fwd_kept_keys"][r], (case["name"], i)
        assert np.exp(f["lse"][0, 0, i]) == pytest.approx(case["fwd_Z"][r], rel=1e-12)
        assert f["kept_slots"][0, 0, i] == len(case["fwd_kept_keys"][r])
    b = oracle_bwd(q, k, v, f["o"], np.ones((1, L, 1, 3)), f["lse"], tau, Bq, Bk)
    kb = pins.keep_to_keymask(b["keep"], L, Bq, Bk)
    for r in range(nr):
        i = r0 + r
        assert sorted(np.nonzero(kb[0, 0, i])[0].tolist()) == case["bwd_kept_keys"][r], (case["name"], i)
    # decision log-margins of the case's block, worked by hand
    qb = r0 // Bq
    for m in case["fwd_margins"]:
        assert_margin(f["margin"][0, 0, qb, m["key_tile"]], m["expr"])
    for m in case["bwd_margins"]:
        assert_margin(b["margin"][0, 0, qb, m["key_tile"]], m["expr"])


# ---------------------------------------------------------------- tau -> 0 is full attention
@pytest.mark.parametrize("shape", [dict(L=300, Hq=4, Hkv=2, d=32), dict(L=129, Hq=3, Hkv=1, d=16),
                                   dict(L=64, Hq=2, Hkv=2, d=64)])
@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (32, 16), (16, 32)])
def test_tau0_forward_is_dense_softmax(shape, tiles):
    q, k, v, _ = _inputs(1, **shape)
    f = oracle_fwd(q, k, v, 0.0, *tiles)
    o, lse = pins.dense_attention(q, k, v)
    assert np.abs(f["o"] - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
    assert np.abs(f["lse"] - lse).max() <= 1e-12 * np.abs(lse).max()
    assert (f["keep"][_visited(f["keep"])] == 1).all()
    assert np.all(f["omitted"] == 0)
    L = shape["L"]
    assert (f["kept_slots"] == np.arange(1, L + 1)[None, None, :]).all()


@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (32, 16)])
def test_tau0_backward_is_autograd(tiles):
    q, k, v, do = _inputs(2, L=200, Hq=4, Hkv=2, d=32)
    f = oracle_fwd(q, k, v, 0.0, *tiles)
    b = oracle_bwd(q, k, v, f["o"], do, f["lse"], 0.0, *tiles)
    gq, gk, gv, _, _ = pins.autograd_masked(q, k, v, do, pins.causal_mask(1, 4, 200))
    for name, ref in (("dq", gq), ("dk", gk), ("dv", gv)):
        err = np.abs(b[name] - ref).max() / np.abs(ref).max()
        assert err <= 1e-12, (name, err)


def test_tau0_backward_finite_differences():
    """Central differences of sum(dO * o) through the oracle's own forward."""
    q, k, v, do = _inputs(3, L=70, Hq=2, Hkv=1, d=8)
    Bq, Bk = 32, 16
    f = oracle_fwd(q, k, v, 0.0, Bq, Bk)
    b = oracle_bwd(q, k, v, f["o"], do, f["lse"], 0.0, Bq, Bk)
    rng = np.random.default_rng(5)
    h = 1e-6

    def loss(qq, kk, vv):
        return float((oracle_fwd(qq, kk, vv, 0.0, Bq, Bk)["o"] * do).sum())

    for name, arr, idx in (("dq", q, 0), ("dk", k, 1), ("dv", v, 2)):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            lp = loss(*args)
            args[idx][pos] -= 2 * h
            lm = loss(*args)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - b[name][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, b[name][pos])


# ---------------------------------------------------------------- tau > 0 invariants
@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (32, 16), (1, 1)])
def test_forward_is_softmax_over_retained_tiles(tau, tiles):
    """Page 2 'Forward': the output equals softmax attention renormalised over the
    retained tiles; omitted mass = dense probability of the skipped legal keys."""
    q, k, v, _ = _inputs(4, L=260, Hq=4, Hkv=2, d=32)
    Bq, Bk = tiles
    f = oracle_fwd(q, k, v, tau, Bq, Bk)
    mask = pins.keep_to_keymask(f["keep"], 260, Bq, Bk)
    o, lse = pins.masked_attention(q, k, v, mask)
    assert np.abs(f["o"] - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(f["lse"] - lse).max() <= 1e-12 * np.abs(lse).max()
    assert (f["kept_slots"] == mask.sum(-1)).all()
    P = pins.dense_probs(q, k)
    om = np.where(mask, 0.0, P).sum(-1)
    assert np.abs(f["omitted"] - om).max() <= 1e-12


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (32, 16), (1, 1)])
def test_prop1_bounds_and_first_tile(tau, tiles):
    """Page 2 Prop. 1: omitted mass < tau/(1+tau) and |o - o_dense| <= 2tau/(1+tau) Vmax;
    page 1: the first legal tile of every row is kept."""
    q, k, v, _ = _inputs(5, L=300, Hq=4, Hkv=2, d=32, p=0.3)
    Bq, Bk = tiles
    f = oracle_fwd(q, k, v, tau, Bq, Bk)
    assert (f["omitted"] < tau / (1 + tau)).all()
    od, _ = pins.dense_attention(q, k, v)
    vmax = np.linalg.norm(v, axis=-1).max()
    err = np.linalg.norm(f["o"] - od, axis=-1)
    assert (err <= 2 * tau / (1 + tau) * vmax + 1e-12).all()
    L = 300
    for i in range(L):
        assert (f["keep"][:, :, i // Bq, i // Bk] == 1).all()


def test_prop1_bound_is_tight_in_order():
    """Adversarial row: many keys exactly below tau/L stay omitted; the bound holds
    and the omitted mass is large (the bound is not vacuous)."""
    L, tau = 64, 1.0
    e = np.full(L, 1.0)
    e[-1] = 10.0
    e[:-1] = 0.99 * tau / L * 10.0  # each just below the threshold against Z = 10
    E = np.tile(e, (L, 1))
    q, k = pins.scores_to_qk(E)
    v = np.random.default_rng(3).standard_normal((1, L, 1, 2))
    f = oracle_fwd(q, k, v, tau, 1, 1)
    w = f["omitted"][0, 0, L - 1]
    assert w < tau / (1 + tau)
    assert w > 0.45  # 63 * 0.1547 / (10 + 63 * 0.1547)


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (32, 16)])
def test_backward_support_nested_in_forward(tau, tiles):
    """Page 2 'Backward': every tile skipped by the forward is skipped by the backward."""
    q, k, v, do = _inputs(6, L=300, Hq=4, Hkv=2, d=32, p=0.2)
    f = oracle_fwd(q, k, v, tau, *tiles)
    b = oracle_bwd(q, k, v, f["o"], do, f["lse"], tau, *tiles)
    vis = _visited(f["keep"])
    assert (vis == _visited(b["keep"])).all()
    assert not np.any((b["keep"] == 1) & (f["keep"] == 0))


def test_decisions_do_not_depend_on_v():
    q, k, v, do = _inputs(7, L=256, Hq=4, Hkv=2, d=32)
    f1 = oracle_fwd(q, k, v, 1.0, 64, 32)
    f2 = oracle_fwd(q, k, 3.0 * np.random.default_rng(9).standard_normal(v.shape), 1.0, 64, 32)
    assert (f1["keep"] == f2["keep"]).all()
    assert np.array_equal(f1["lse"], f2["lse"])


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_backward_is_masked_textbook_gradient(tau):
    """The backward equals the textbook softmax-attention gradient of the forward
    (softmax over the forward-retained keys, via autograd) with the score
    gradients of backward-skipped tiles dropped."""
    Bq, Bk = 32, 16
    q, k, v, do = _inputs(8, L=160, Hq=4, Hkv=2, d=16, p=0.2)
    f = oracle_fwd(q, k, v, tau, Bq, Bk)
    b = oracle_bwd(q, k, v, f["o"], do, f["lse"], tau, Bq, Bk)
    mf = pins.keep_to_keymask(f["keep"], 160, Bq, Bk)
    mb = pins.keep_to_keymask(b["keep"], 160, Bq, Bk)
    _, _, _, dS, P = pins.autograd_masked(q, k, v, do, mf)
    dSb = np.where(mb, dS, 0.0)
    Pb = np.where(mb, P, 0.0)
    sc = 1 / np.sqrt(16)
    Gh = 2
    kk = np.repeat(k, Gh, axis=2)
    dq = sc * np.einsum("bhij,bjhc->bihc", dSb, kk)
    dk_h = sc * np.einsum("bhij,bihc->bjhc", dSb, q)
    dv_h = np.einsum("bhij,bihc->bjhc", Pb, do)
    dk = dk_h.reshape(1, 160, 2, Gh, 16).sum(3)
    dv = dv_h.reshape(1, 160, 2, Gh, 16).sum(3)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        err = np.abs(b[name] - ref).max() / np.abs(ref).max()
        assert err <= 1e-11, (name, err)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_decode_pins(tau):
    di = G.decode_inputs(40, 2, 700, 6, 2, 32)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    r = oracle_decode(q, kc, vc, tau, 64)
    nT = r["keep"].shape[-1]
    Gq = 3
    # newest tile always kept (empty state); softmax over retained tiles
    assert (r["keep"][:, :, nT - 1] == 1).all()
    S = np.einsum("bhc,bjhc->bhj", q, np.repeat(kc, Gq, axis=2)) / np.sqrt(32)
    keepj = np.repeat(r["keep"], 64, axis=-1)[:, :, :700] == 1  # [B, Hkv, N]
    mask = np.repeat(keepj, Gq, axis=1)
    Sm = np.where(mask, S, -np.inf)
    mx = Sm.max(-1, keepdims=True)
    w = np.where(mask, np.exp(Sm - mx), 0.0)
    o = np.einsum("bhj,bjhc->bhc", w / w.sum(-1, keepdims=True), np.repeat(vc, Gq, axis=2))
    assert np.abs(r["o"] - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(r["lse"] - (mx[..., 0] + np.log(w.sum(-1)))).max() <= 1e-12 * 40
    if tau == 0:
        assert (r["keep"] == 1).all()
    Pd = np.exp(S - S.max(-1, keepdims=True))
    Pd /= Pd.sum(-1, keepdims=True)
    om = np.where(mask, 0.0, Pd).sum(-1)
    assert np.abs(r["omitted"] - om).max() <= 1e-12
    assert (r["omitted"] < tau / (1 + tau) + (1 if tau == 0 else 0)).all()
    assert (r["kept_tiles"] == r["keep"].sum(-1)).all()
