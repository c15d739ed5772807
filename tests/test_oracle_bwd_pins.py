"""Pins for the oracle's backward pass (gradients of the forward definition).

The gradients are checked against central finite differences of
L = sum(dO * O(q, k, v)) through the (separately pinned) forward definition,
against torch's CPU float64 autograd through plain softmax attention, and
against closed forms (over keys, dK sums to zero and dV sums to sum(dO)).
Planted mistakes in copies of the formulas must each be caught.
"""

import numpy as np
import pytest
import torch

import oracle


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def loss(q, k, v, do, scale, causal, sl):
    o, _ = oracle.attention(q, k, v, scale, causal, seqlens_k=sl)
    return float((o * do).sum())


def finite_diff(q, k, v, do, scale, causal, sl, eps=1e-6):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            a = [x.copy() for x in args]
            a[which][idx] += eps
            lp = loss(*a, do, scale, causal, sl)
            a[which][idx] -= 2 * eps
            lm = loss(*a, do, scale, causal, sl)
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


CASES = [
    dict(B=1, H=2, nq=4, nk=4, D=3, causal=True, sl=None, scale=0.7),
    dict(B=1, H=1, nq=3, nk=5, D=2, causal=False, sl=None, scale=0.5),
    dict(B=2, H=1, nq=5, nk=5, D=2, causal=True, sl=[5, 3], scale=0.9),
    dict(B=1, H=2, nq=5, nk=3, D=2, causal=True, sl=None, scale=0.6),  # rows 0, 1 see no key
]


def check_fd(bwd, c, seed):
    rng = np.random.default_rng(seed)
    q, k, v = rnd(rng, c["B"], c["nq"], c["H"], c["D"]), rnd(rng, c["B"], c["nk"], c["H"], c["D"]), \
        rnd(rng, c["B"], c["nk"], c["H"], c["D"])
    do = rnd(rng, c["B"], c["nq"], c["H"], c["D"])
    sl = None if c["sl"] is None else np.array(c["sl"])
    dq, dk, dv = bwd(q, k, v, do, c["scale"], c["causal"], seqlens_k=sl)
    fq, fk, fv = finite_diff(q, k, v, do, c["scale"], c["causal"], sl)
    np.testing.assert_allclose(dq, fq, atol=2e-7)
    np.testing.assert_allclose(dk, fk, atol=2e-7)
    np.testing.assert_allclose(dv, fv, atol=2e-7)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_bwd_matches_finite_differences(i):
    check_fd(oracle.attention_bwd, CASES[i], 100 + i)


def check_torch(bwd, causal, seed=7):
    rng = np.random.default_rng(seed)
    B, nq, nk, H, D, scale = 2, 6, 6, 2, 4, 0.45
    q, k, v, do = rnd(rng, B, nq, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nk, H, D), \
        rnd(rng, B, nq, H, D)
    dq, dk, dv = bwd(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.einsum("bihd,bjhd->bhij", tq, tk)
    if causal:
        mask = torch.ones(nq, nk, dtype=torch.bool).tril(nk - nq)
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_matches_torch_cpu_float64_autograd(causal):
    check_torch(oracle.attention_bwd, causal)


def check_sums(bwd, seed=8):
    """Softmax rows sum to one, so sum_j dS_ij = 0 (hence dK sums to zero over
    keys) and sum_j dV_j = sum_i dO_i for rows that see at least one key."""
    rng = np.random.default_rng(seed)
    q, k, v, do = rnd(rng, 1, 7, 2, 3), rnd(rng, 1, 7, 2, 3), rnd(rng, 1, 7, 2, 3), rnd(rng, 1, 7, 2, 3)
    dq, dk, dv = bwd(q, k, v, do, 0.8, True)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


def test_bwd_sums():
    check_sums(oracle.attention_bwd)


# ----------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin
# ----------------------------------------------------------------------------

def _make_bad(kind):
    def bad(q, k, v, do, scale, causal, seqlens_k=None):
        B, nq, H, D = q.shape
        nk = k.shape[1]
        dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            lk = nk if seqlens_k is None else int(seqlens_k[b])
            for h in range(H):
                qq, kk, vv, g = q[b, :, h], k[b, :lk, h], v[b, :lk, h], do[b, :, h]
                s = scale * qq @ kk.T
                j = np.arange(lk)
                i = np.arange(nq)[:, None]
                shift = 1 if kind == "causal shifted" else 0
                vis = (j[None, :] <= i + lk - nq - shift) if causal else np.ones((nq, lk), bool)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                m = np.where(np.isneginf(m), 0.0, m)
                e = np.exp(s - m[:, None])
                ell = e.sum(axis=1)
                p = np.where(ell[:, None] > 0, e / np.where(ell > 0, ell, 1.0)[:, None], 0.0)
                o = p @ vv
                if kind == "dV uses P not its transpose" and nq == lk:
                    dv[b, :lk, h] = p @ g
                else:
                    dv[b, :lk, h] = p.T @ g
                dp = g @ vv.T
                delta = 0.0 if kind == "delta dropped" else (g * o).sum(axis=1)[:, None]
                ds = p * (dp - delta)
                dq[b, :, h] = scale * ds @ kk
                dk[b, :lk, h] = (1.0 if kind == "dK scale dropped" else scale) * ds.T @ qq
        return dq, dk, dv
    return bad


@pytest.mark.parametrize("kind", ["delta dropped", "dK scale dropped", "dV uses P not its transpose",
                                  "causal shifted"])
def test_planted_bwd_mistakes_are_caught(kind):
    bad = _make_bad(kind)
    pins = [lambda: check_fd(bad, CASES[0], 100), lambda: check_fd(bad, CASES[2], 102),
            lambda: check_torch(bad, True), lambda: check_torch(bad, False), lambda: check_sums(bad)]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, "no pin caught the planted mistake: %s" % kind


# ----------------------------------------------------------------------------
# Prefix mask and ALiBi bias (the forward's mask families)
# ----------------------------------------------------------------------------

MASK_CASES = [
    # (B, nq, nk, H, D, causal, prefix, alibi)
    (1, 7, 9, 2, 4, True, 3, False),
    (2, 6, 6, 2, 3, True, 0, True),
    (1, 5, 8, 2, 4, False, 0, True),
    (1, 8, 8, 3, 4, True, 4, True),
]


def _masked_case(case, seed):
    B, nq, nk, H, D, causal, prefix, alibi = case
    rng = np.random.default_rng(seed)
    q, k, v, do = rnd(rng, B, nq, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nq, H, D)
    slopes = 2.0 ** (-8.0 * (np.arange(H) + 1) / H) * 3.0 if alibi else None
    return q, k, v, do, causal, prefix, slopes


def _masked_fd(bwd, case, seed, eps=1e-6):
    q, k, v, do, causal, prefix, slopes = _masked_case(case, seed)
    scale = 0.45
    got = bwd(q, k, v, do, scale, causal, prefix, slopes)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, scale, causal, prefix=prefix, alibi_slopes=slopes)
        return float((o * do).sum())
    rng = np.random.default_rng(seed + 1)
    for which, g in enumerate(got):
        args = [q, k, v]
        x = args[which]
        for _ in range(10):
            ix = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[ix] += eps
            xm[ix] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num = (loss(*ap) - loss(*am)) / (2 * eps)
            assert abs(num - g[ix]) < 2e-7 + 1e-6 * abs(num), (which, ix, num, g[ix])


def _oracle_masked_bwd(q, k, v, do, scale, causal, prefix, slopes):
    return oracle.attention_bwd(q, k, v, do, scale, causal, prefix=prefix, alibi_slopes=slopes)


@pytest.mark.parametrize("i", range(len(MASK_CASES)))
def test_masked_bwd_matches_finite_differences(i):
    _masked_fd(_oracle_masked_bwd, MASK_CASES[i], 300 + i)


@pytest.mark.parametrize("i", range(len(MASK_CASES)))
def test_masked_bwd_matches_torch_cpu_float64_autograd(i):
    q, k, v, do, causal, prefix, slopes = _masked_case(MASK_CASES[i], 400 + i)
    B, nq, H, D = q.shape
    nk = k.shape[1]
    scale = 0.45
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.einsum("bihd,bjhd->bhij", tq, tk)
    ii = torch.arange(nq)[:, None]
    jj = torch.arange(nk)[None, :]
    if slopes is not None:
        dist = (jj - (ii + nk - nq)).abs().to(torch.float64)
        s = s - torch.tensor(slopes)[None, :, None, None] * dist
    if causal:
        vis = (jj <= ii + nk - nq) | (jj < prefix)
        s = s.masked_fill(~vis, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    got = oracle.attention_bwd(q, k, v, do, scale, causal, prefix=prefix, alibi_slopes=slopes)
    for g, t in zip(got, (tq, tk, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("kind", ["bias dropped", "prefix ignored"])
def test_planted_masked_bwd_mistakes_are_caught(kind):
    def bad(q, k, v, do, scale, causal, prefix, slopes):
        if kind == "bias dropped":
            return oracle.attention_bwd(q, k, v, do, scale, causal, prefix=prefix)
        return oracle.attention_bwd(q, k, v, do, scale, causal, alibi_slopes=slopes)
    case = MASK_CASES[3]
    with pytest.raises(AssertionError):
        _masked_fd(bad, case, 303)


# ----------------------------------------------------------------------------
# Packed variable-length batches
# ----------------------------------------------------------------------------

def _varlen_fd(bwd, causal, seed, eps=1e-6):
    rng = np.random.default_rng(seed)
    cu_q = np.array([0, 3, 3, 8, 12])   # an empty sequence included
    cu_k = np.array([0, 4, 6, 11, 13])
    H, D, scale = 2, 3, 0.6
    q, do = rnd(rng, 12, H, D), rnd(rng, 12, H, D)
    k, v = rnd(rng, 13, H, D), rnd(rng, 13, H, D)
    got = bwd(q, k, v, do, cu_q, cu_k, scale, causal)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_varlen(qq, kk, vv, cu_q, cu_k, scale, causal)
        return float((o * do).sum())
    for which, g in enumerate(got):
        args = [q, k, v]
        x = args[which]
        for ix in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[ix] += eps
            xm[ix] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num = (loss(*ap) - loss(*am)) / (2 * eps)
            assert abs(num - g[ix]) < 2e-7 + 1e-6 * abs(num), (which, ix, num, g[ix])


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_bwd_matches_finite_differences(causal):
    """Every entry of the gradients against central differences through the
    (separately pinned) packed forward; keys of the empty query sequence get 0."""
    _varlen_fd(oracle.attention_varlen_bwd, causal, 500 + causal)


def test_planted_varlen_bwd_mistake_is_caught():
    """Treating the packed batch as one sequence must fail the pin."""
    def bad(q, k, v, do, cu_q, cu_k, scale, causal):
        gq, gk, gv = oracle.attention_bwd(q[None], k[None], v[None], do[None], scale, causal)
        return gq[0], gk[0], gv[0]
    with pytest.raises(AssertionError):
        _varlen_fd(bad, True, 501)
