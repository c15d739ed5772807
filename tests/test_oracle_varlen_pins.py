"""Pins for the oracle's packed variable-length attention with the prefix
mask, ALiBi and attention dropout (``attention_varlen`` and
``attention_varlen_bwd`` with those options).

* Brute force: for tiny packed batches, pure-Python loops (``math.exp``,
  ``math.fsum``) over the definition - scores, the per-sequence causal /
  prefix visibility with bottom-right alignment, the ALiBi bias, the keep
  decisions with the sequence index as the counters' batch index - agree
  with the oracle to rounding.
* Packing: a batch of equal-length sequences packed end to end gives the
  fixed-length oracle's results (forward and gradients) for every option.
* Gradients: central finite differences through the packed forward.
* Planted mistakes (a sequence index of 0 in the keep counters, positions
  counted in the packed tensor instead of the sequence) must each be caught.
"""

import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def _packed(lens, H, D, scale=0.7):
    tot = int(sum(lens))
    q = RNG.standard_normal((tot, H, D)) * scale
    k = RNG.standard_normal((tot, H, D)) * scale
    v = RNG.standard_normal((tot, H, D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, cu


def _brute(q, k, v, cu, scale, causal, prefix, slopes, dropout_p, seed, seq_index=None):
    """Pure-Python reference: sequence s, head h, row i sees key j of the same
    sequence iff (not causal) or j <= i or j < prefix (equal lengths here:
    bottom-right alignment reduces to j <= i)."""
    H, D = q.shape[1], q.shape[2]
    t = oracle.drop_threshold(dropout_p) if dropout_p else 0
    ks = oracle.keep_scale(t) if dropout_p else 1.0
    o = np.zeros_like(v)
    lse = np.zeros((H, q.shape[0]))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        sidx = s if seq_index is None else seq_index(s)
        for h in range(H):
            keep = oracle.keep_mask(seed, sidx, h, np.arange(L), L, t) if dropout_p else None
            for i in range(L):
                sc = []
                for j in range(L):
                    if causal and not (j <= i or j < prefix):
                        continue
                    x = scale * math.fsum(q[a + i, h, d] * k[a + j, h, d] for d in range(D))
                    if slopes is not None:
                        x -= slopes[h] * abs(j - i)
                    sc.append((j, x))
                if not sc:
                    lse[h, a + i] = -math.inf
                    continue
                m = max(x for _, x in sc)
                w = [(j, math.exp(x - m)) for j, x in sc]
                ell = math.fsum(e for _, e in w)
                lse[h, a + i] = m + math.log(ell)
                for d in range(v.shape[2]):
                    o[a + i, h, d] = math.fsum(
                        e * (ks if keep is None or keep[i, j] else 0.0) * v[a + j, h, d]
                        for j, e in w if keep is None or keep[i, j]) / ell
    return o, lse


CASES = [
    # lens, causal, prefix, alibi, dropout
    ([3, 5, 1], True, 0, False, 0.0),
    ([4, 6], True, 2, False, 0.0),
    ([5, 2, 6], True, 0, True, 0.0),
    ([6, 3], False, 0, True, 0.0),
    ([5, 6, 2], True, 0, False, 0.3),
    ([4, 5], False, 0, False, 0.5),
    ([6, 4, 5], True, 2, True, 0.3),   # every option at once
    ([5, 6], False, 0, True, 0.4),
]


@pytest.mark.parametrize("lens,causal,prefix,alibi,p", CASES)
def test_forward_against_brute_force(lens, causal, prefix, alibi, p):
    H, D = 2, 3
    q, k, v, cu = _packed(lens, H, D)
    slopes = np.array([0.25, 0.125]) if alibi else None
    o, lse = oracle.attention_varlen(q, k, v, cu, cu, 0.8, causal, prefix=prefix,
                                     alibi_slopes=slopes, dropout_p=p, seed=17)
    ob, lb = _brute(q, k, v, cu, 0.8, causal, prefix, slopes, p, 17)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_planted_mistakes_are_caught():
    H, D = 2, 3
    q, k, v, cu = _packed([5, 6, 4], H, D)
    o, _ = oracle.attention_varlen(q, k, v, cu, cu, 0.8, True, dropout_p=0.4, seed=3)
    # keep counters with batch index 0 for every sequence
    ob, _ = _brute(q, k, v, cu, 0.8, True, 0, None, 0.4, 3, seq_index=lambda s: 0)
    assert np.abs(o - ob).max() > 1e-3
    # prefix and ALiBi distances measured in the packed tensor instead of the sequence
    slopes = np.array([0.3, 0.2])
    o2, _ = oracle.attention_varlen(q, k, v, cu, cu, 0.8, True, prefix=2, alibi_slopes=slopes)
    ob2, _ = _brute(q, k, v, np.array([0, int(cu[-1])]), 0.8, True, 2, slopes, 0.0, 0)
    assert np.abs(o2 - ob2).max() > 1e-3


OPTIONS = [
    dict(prefix=3),
    dict(alibi_slopes=np.array([0.5, 0.0625, 0.25])),
    dict(dropout_p=0.25, seed=99),
    dict(prefix=5, alibi_slopes=np.array([0.5, 0.0625, 0.25]), dropout_p=0.25, seed=98),
]


# the prefix mask is a causal option: its cases run causal only
CASES = [pytest.param(o, c, id="%s-%s" % (name, "causal" if c else "full"))
         for o, name in zip(OPTIONS, ["prefix", "alibi", "dropout", "all"])
         for c in (True, False) if c or "prefix" not in o]


@pytest.mark.parametrize("opt,causal", CASES)
def test_equal_lengths_match_the_fixed_length_oracle(opt, causal):
    B, L, H, D = 3, 37, 3, 8
    q = RNG.standard_normal((B, L, H, D)) * 0.6
    k = RNG.standard_normal((B, L, H, D)) * 0.6
    v = RNG.standard_normal((B, L, H, D))
    do = RNG.standard_normal((B, L, H, D))
    cu = np.arange(B + 1) * L
    pq, pk, pv, pdo = (t.reshape(B * L, H, D) for t in (q, k, v, do))
    o, lse = oracle.attention_varlen(pq, pk, pv, cu, cu, 0.35, causal, **opt)
    if "dropout_p" in opt:
        masks = {n: opt[n] for n in ("prefix", "alibi_slopes") if n in opt}
        of, lf = oracle.attention_dropout(q, k, v, 0.35, causal, opt["dropout_p"], opt["seed"],
                                          **masks)
    else:
        of, lf = oracle.attention(q, k, v, 0.35, causal, **opt)
    np.testing.assert_allclose(o, of.reshape(B * L, H, D), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lf.transpose(1, 0, 2).reshape(H, B * L), rtol=0, atol=1e-13)
    g = oracle.attention_varlen_bwd(pq, pk, pv, pdo, cu, cu, 0.35, causal, **opt)
    gf = oracle.attention_bwd(q, k, v, do, 0.35, causal, **opt)
    for a, b in zip(g, gf):
        np.testing.assert_allclose(a, b.reshape(B * L, H, D), rtol=0, atol=1e-12)


@pytest.mark.parametrize("opt", OPTIONS, ids=["prefix", "alibi", "dropout", "all"])
def test_gradients_by_finite_differences(opt):
    lens, H, D = [4, 7], 3, 3
    q, k, v, cu = _packed(lens, H, D)
    do = RNG.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_varlen_bwd(q, k, v, do, cu, cu, 0.9, True, **opt)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_varlen(q_, k_, v_, cu, cu, 0.9, True, **opt)
        return float((o * do).sum())

    eps = 1e-6
    for t, g in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0, 0), (5, 1, 2), (10, 2, 1), (3, 2, 0)]:
            t0 = t[idx]
            t[idx] = t0 + eps
            lp = loss(q, k, v)
            t[idx] = t0 - eps
            lm = loss(q, k, v)
            t[idx] = t0
            assert abs((lp - lm) / (2 * eps) - g[idx]) < 1e-6, (idx, (lp - lm) / (2 * eps), g[idx])
