"""The C oracle against the separately written numpy statement of the rule,
and against the key-by-key statement (Bq = Bk = 1), over random shapes."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import mala_gen as G
from oracle import oracle_bwd, oracle_decode, oracle_fwd
from oracle import ref_numpy as R

def _same_margins(a, b, tol=1e-9):
    """Decision log-margins agree: the same infinities and NaNs (unvisited
    tiles), finite values within tol (relative above 1)."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(np.isposinf(a), np.isposinf(b))
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    f = np.isfinite(a)
    assert np.all(np.abs(a[f] - b[f]) <= tol * np.maximum(1.0, np.abs(b[f])))


shapes = st.fixed_dictionaries({
    "L": st.integers(1, 140),
    "Hkv": st.integers(1, 2),
    "G": st.integers(1, 3),
    "d": st.sampled_from([4, 8, 16]),
    "Bq": st.sampled_from([1, 2, 8, 16, 32, 64]),
    "Bk": st.sampled_from([1, 4, 16, 32, 64]),
    "tau": st.sampled_from([0.0, 0.05, 0.25, 1.0, 4.0, 20.0]),
    "p": st.sampled_from([0.0, 0.1, 0.5]),
    "diffuse": st.booleans(),
    "seed": st.integers(0, 10_000),
})


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(shapes)
def test_c_oracle_matches_numpy(s):
    Hq = s["Hkv"] * s["G"]
    inp = G.attn_inputs(s["seed"], 1, s["L"], Hq, s["Hkv"], s["d"], s["p"],
                        diffuse_kv_heads=(0,) if s["diffuse"] else ())
    q, k, v, do = [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]
    a = oracle_fwd(q, k, v, s["tau"], s["Bq"], s["Bk"])
    b = R.fwd(q, k, v, s["tau"], s["Bq"], s["Bk"])
    assert (a["keep"] == b["keep"]).all()
    _same_margins(a["margin"], b["margin"])
    assert np.array_equal(a["margin"] >= 0, a["keep"] == 1)
    assert (a["kept_slots"] == b["kept_slots"]).all()
    assert np.abs(a["o"] - b["o"]).max() <= 1e-11
    assert np.abs(a["lse"] - b["lse"]).max() <= 1e-11
    assert np.abs(a["omitted"] - b["omitted"]).max() <= 1e-9
    c = oracle_bwd(q, k, v, a["o"], do, a["lse"], s["tau"], s["Bq"], s["Bk"])
    e = R.bwd(q, k, v, a["o"], do, a["lse"], s["tau"], s["Bq"], s["Bk"])
    assert (c["keep"] == e["keep"]).all()
    _same_margins(c["margin"], e["margin"])
    for n in ("dq", "dk", "dv"):
        assert np.abs(c[n] - e[n]).max() <= 1e-10 * max(1.0, np.abs(e[n]).max())


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 90), st.sampled_from([0.0, 0.25, 1.0, 4.0]), st.integers(0, 999))
def test_unit_tiles_match_key_by_key_statement(L, tau, seed):
    """With Bq = Bk = 1 each row is decided alone, key by key, newest first."""
    inp = G.attn_inputs(seed, 1, L, 1, 1, 8, 0.2)
    q, k, v = [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v")]
    f = oracle_fwd(q, k, v, tau, 1, 1)
    S = (q[0, :, 0, :] @ k[0, :, 0, :].T) / np.sqrt(8)
    for i in range(L):
        s = S[i, : i + 1]
        e = np.exp(s - s.max())  # ratios are scale-free
        kept, Z, om = R.per_key_row(e, tau)
        ok = f["keep"][0, 0, i, : i + 1] == 1
        assert sorted(kept) == np.nonzero(ok)[0].tolist()
        assert abs(f["lse"][0, 0, i] - (np.log(Z) + s.max())) <= 1e-12 * max(1, abs(s.max()))
        assert abs(f["omitted"][0, 0, i] - om) <= 1e-12


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 400), st.integers(1, 3), st.integers(1, 3), st.sampled_from([1, 16, 64]),
       st.sampled_from([0.0, 0.25, 1.0, 4.0]), st.integers(0, 999))
def test_c_decode_matches_numpy(N, Hkv, Gq, Bkd, tau, seed):
    di = G.decode_inputs(seed, 2, N, Hkv * Gq, Hkv, 16)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    a = oracle_decode(q, kc, vc, tau, Bkd)
    b = R.decode(q, kc, vc, tau, Bkd)
    assert (a["keep"] == b["keep"]).all()
    _same_margins(a["margin"], b["margin"])
    assert np.abs(a["o"] - b["o"]).max() <= 1e-11
    assert np.abs(a["lse"] - b["lse"]).max() <= 1e-11


def test_sampled_blocks_equal_full_run():
    """Computing a subset of query blocks / key tiles gives the same rows."""
    inp = G.attn_inputs(77, 1, 300, 4, 2, 16, 0.1)
    q, k, v, do = [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]
    full = oracle_fwd(q, k, v, 1.0, 64, 32)
    nQB, nKT = 5, 10
    ids = [3, 2 * nQB + 4, 3 * nQB + 0]
    part = oracle_fwd(q, k, v, 1.0, 64, 32, blocks=ids)
    for bid in ids:
        h, qb = divmod(bid, nQB)
        r0, r1 = qb * 64, min(300, qb * 64 + 64)
        assert np.array_equal(part["o"][0, r0:r1, h], full["o"][0, r0:r1, h])
        assert np.array_equal(part["keep"][0, h, qb], full["keep"][0, h, qb])
    bf = oracle_bwd(q, k, v, full["o"], do, full["lse"], 1.0, 64, 32)
    bp = oracle_bwd(q, k, v, full["o"], do, full["lse"], 1.0, 64, 32, qunits=[7], kunits=[3, 12])
    assert np.array_equal(bp["dq"][0, 128:192, 1], bf["dq"][0, 128:192, 1])
    assert np.array_equal(bp["dk"][0, 96:128, 0], bf["dk"][0, 96:128, 0])
    assert np.array_equal(bp["dv"][0, 64:96, 1], bf["dv"][0, 64:96, 1])
