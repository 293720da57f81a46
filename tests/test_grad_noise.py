"""The gradient checks' binary32 floor, pinned on the CPU.

The GPU gradient tests hold each (b, h) slice to |got - ref| <= 1e-2 |ref| +
u |cond|: u = 2^-24, cond the fp64 oracle's componentwise error scale of dP - D
(gamma_d |cond| being the rigorous first-order bound for binary32 evaluation).
These tests fix what that floor is, using binary32 evaluations of dP and D
(parity.fp32_gradient_noise):
  - the rigorous bound is a bound: every evaluation stays inside gamma_d cond,
    element by element;
  - the floor is needed: on heads whose rows attend to one key, even those
    evaluations (everything but dP and D exact) miss the exact dq and dk by
    far more than 1e-2 relative -- the exact values cancel below binary32
    resolution;
  - the floor is sized to that noise: the evaluations sit well inside it, and
    it is a small multiple of them, not the rigorous bound's hundreds;
  - it weakens nothing elsewhere: on diffuse heads it is far below 1e-2 |ref|;
  - the check rejects an error twice the floor, and 5% errors anywhere.
Backward rule: review page "Backward: offline sparse probabilities".
"""
import numpy as np
import pytest

import mala_gen as G
from oracle import oracle_bwd, oracle_fwd
from parity import U32, fp32_gradient_noise, gamma, grad_check

L, HQ, HKV, D, BQ, BK = 384, 4, 2, 128, 128, 64


@pytest.fixture(scope="module")
def case():
    """KV head 0 (q heads 0-1): local/sink/retrieval rows, nearly one-hot.
    KV head 1 (q heads 2-3): diffuse N(0, 1) rows.  O and LSE are the oracle
    forward's, rounded to the stored types (bf16, fp32)."""
    inp = G.attn_inputs(31, 1, L, HQ, HKV, D, 0.1, diffuse_kv_heads=(1,))
    q, k, v, do = [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]
    f = oracle_fwd(q, k, v, 1.0, BQ, BK)
    o = G.bf16_bits_to_f64(G.round_to_bf16_bits(f["o"]))
    lse = f["lse"].astype(np.float32).astype(np.float64)
    b = oracle_bwd(q, k, v, o, do, lse, 1.0, BQ, BK, cond=True)
    ddq, ddk = fp32_gradient_noise(q, k, v, o, do, lse, b["keep"], BQ, BK)
    return dict(q=q, k=k, v=v, o=o, do=do, lse=lse, b=b, ddq=ddq, ddk=ddk)


def test_noise_inside_rigorous_bound(case):
    b = case["b"]
    g = gamma(D)
    for name, dd, cond in (("dq", case["ddq"], b["dq_cond"]), ("dk", case["ddk"], b["dk_cond"])):
        for x in dd:
            slack = 1e-12 * np.abs(cond).max()
            assert np.all(np.abs(x) <= g * cond + slack), name
            # not vacuous either: somewhere the noise is a visible share of the bound
            assert (np.abs(x) / np.maximum(g * cond, 1e-300)).max() > 1e-4, name


def _slice_noise(dd, axis_h, h):
    return max(np.linalg.norm(np.take(x, h, axis=axis_h)) for x in dd)


def test_noise_exceeds_tolerance_on_one_hot_heads(case):
    b = case["b"]
    for h in (0, 1):
        rel = _slice_noise(case["ddq"], 2, h) / np.linalg.norm(b["dq"][0, :, h])
        assert rel > 1e-2, (h, rel)
    rel = _slice_noise(case["ddk"], 2, 0) / np.linalg.norm(b["dk"][0, :, 0])
    assert rel > 1e-2, rel


def test_noise_negligible_on_diffuse_heads(case):
    b = case["b"]
    for h in (2, 3):
        rel = _slice_noise(case["ddq"], 2, h) / np.linalg.norm(b["dq"][0, :, h])
        assert rel < 1e-4, (h, rel)
    rel = _slice_noise(case["ddk"], 2, 1) / np.linalg.norm(b["dk"][0, :, 1])
    assert rel < 1e-4, rel


def test_floor_is_a_small_multiple_of_the_binary32_noise(case):
    """Per slice: the evaluations' noise lies within half the floor u |cond|,
    and on the one-hot heads above a fiftieth of it."""
    b = case["b"]
    for dd, cond, slices in ((case["ddq"], b["dq_cond"], range(4)), (case["ddk"], b["dk_cond"], range(2))):
        for h in slices:
            noise = _slice_noise(dd, 2, h)
            floor = U32 * np.linalg.norm(cond[0, :, h])
            assert noise <= 0.5 * floor, (h, noise / floor)
            if (dd is case["ddq"] and h < 2) or (dd is case["ddk"] and h == 0):
                assert noise >= floor / 50, (h, noise / floor)


def test_check_accepts_binary32_results_and_rejects_planted_errors(case):
    b = case["b"]
    ref, noise, cond = b["dq"], case["ddq"], b["dq_cond"]
    # binary32 evaluations pass, and the floor decides the one-hot heads
    for x in range(2):
        rep = grad_check(ref + noise[x], ref, cond, noise)
        assert rep["ok"] and rep["floor_decided"] == 2, rep
    # 5% relative error on one diffuse head fails
    bad = ref.copy()
    bad[0, :, 3] *= 1.05
    assert not grad_check(bad, ref, cond)["ok"]
    # an error twice the floor on a one-hot head fails
    bad = ref.copy()
    e = np.random.default_rng(1).standard_normal(ref[0, :, 0].shape)
    bad[0, :, 0] += e * (2 * U32 * np.linalg.norm(cond[0, :, 0]) / np.linalg.norm(e))
    assert not grad_check(bad, ref, cond)["ok"]
    # the same for dk
    refk, nk, ck = b["dk"], case["ddk"], b["dk_cond"]
    assert grad_check(refk + nk[0], refk, ck)["ok"]
    badk = refk.copy()
    badk[0, :, 1] *= 0.95
    assert not grad_check(badk, refk, ck)["ok"]
    badk = refk.copy()
    e = np.random.default_rng(2).standard_normal(refk[0, :, 0].shape)
    badk[0, :, 0] += e * (2 * U32 * np.linalg.norm(ck[0, :, 0]) / np.linalg.norm(e))
    assert not grad_check(badk, refk, ck)["ok"]


def test_noise_of_sampled_blocks_equals_full_run(case):
    """Evaluating a subset of blocks gives those blocks' dq rows unchanged."""
    c = case
    blocks = [(0, 1, 2), (0, 3, 0)]
    ddq, _ = fp32_gradient_noise(c["q"], c["k"], c["v"], c["o"], c["do"], c["lse"], c["b"]["keep"], BQ, BK,
                                 blocks=blocks)
    for _, h, qb in blocks:
        rows = slice(qb * BQ, (qb + 1) * BQ)
        for x in range(2):
            assert np.array_equal(ddq[x][0, rows, h], c["ddq"][x][0, rows, h])
