"""Pins for the oracle's attention dropout (``oracle.dropout`` and the dropout
paths of ``attention_dropout`` / ``attention_bwd``).

* Philox4x32-10 against the known-answer vectors published with the
  generator (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
  1, 2, 3", SC 2011, and its Random123 distribution);
* the (query, key) -> word/byte mapping against the bytes of the first
  known-answer vector (seed 0, batch 0, head 0, query 0 has counter 0);
* keep rate and byte uniformity against the binomial law;
* closed forms: a single visible key gives O = 0 or V * 256/(256 - t); lse
  never changes; p = 0 is plain attention;
* unbiasedness: the mean over seeds approaches the undropped output;
* gradients: finite differences through the dropout forward and torch's
  float64 autograd with the same keep mask;
* planted mistakes in copies of the formulas must each be caught.
"""

import numpy as np
import pytest
import torch

import oracle

# Random123 known-answer vectors for philox4x32 with 10 rounds:
# (counter, key, output), all words hexadecimal.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = oracle.philox4x32(np.array(ctr), np.array(key))
    assert [int(x) for x in got] == list(out)


def test_philox_vectorised_broadcast():
    ctr = np.array([c for c, _, _ in KAT])
    key = np.array([k for _, k, _ in KAT])
    got = oracle.philox4x32(ctr, key)
    assert got.tolist() == [list(o) for _, _, o in KAT]


def test_mapping_against_the_first_known_answer():
    """Seed 0, batch 0, head 0, query 0, keys 0..15 use counter (0,0,0,0)
    and key (0,0): key j takes byte j%4 (least significant first) of word
    j//4 of the first known-answer output."""
    words = KAT[0][2]
    bytes_ = [(words[j // 4] >> (8 * (j % 4))) & 0xFF for j in range(16)]
    for t in (1, 64, 128, 200, 255):
        m = oracle.keep_mask(0, 0, 0, [0], 16, t)[0]
        assert m.tolist() == [b >= t for b in bytes_]
    # keys 16..31 use counter (1, 0, 0, 0): a different draw
    m = oracle.keep_mask(0, 0, 0, [0], 32, 128)[0]
    w1 = oracle.philox4x32(np.array([1, 0, 0, 0]), np.array([0, 0]))
    assert m[16:].tolist() == [((int(w1[j // 4]) >> (8 * (j % 4))) & 0xFF) >= 128 for j in range(16)]


def test_counter_fields():
    """Counter = (key group, query, head, batch), key = seed split in two."""
    seed = 0x0123456789ABCDEF
    i, h, b, j = 7, 3, 2, 37
    w = oracle.philox4x32(np.array([j // 16, i, h, b]), np.array([seed & 0xFFFFFFFF, seed >> 32]))
    byte = (int(w[(j // 4) % 4]) >> (8 * (j % 4))) & 0xFF
    for t in (byte, byte + 1):
        if t <= 255:
            assert oracle.keep_mask(seed, b, h, [i], 40, t)[0, j] == (byte >= t)


def test_threshold_and_scale():
    assert oracle.drop_threshold(0.0) == 0
    assert oracle.drop_threshold(0.1) == 26          # round(25.6)
    assert oracle.drop_threshold(0.5) == 128
    assert oracle.drop_threshold(0.999) == 255
    assert oracle.keep_scale(26) == 256.0 / 230.0
    with pytest.raises(ValueError):
        oracle.drop_threshold(1.0)
    with pytest.raises(ValueError):
        oracle.drop_threshold(-0.1)


@pytest.mark.parametrize("t", [26, 128, 230])
def test_keep_rate_binomial(t):
    n_rows, lk = 2000, 512
    m = oracle.keep_mask(99, 1, 5, np.arange(n_rows), lk, t)
    p_keep = 1.0 - t / 256.0
    sd = np.sqrt(p_keep * (1 - p_keep) / m.size)
    assert abs(m.mean() - p_keep) < 6 * sd
    # per-key-position rates (each of the 16 positions of a group) too
    for pos in range(16):
        mm = m[:, pos::16]
        sdp = np.sqrt(p_keep * (1 - p_keep) / mm.size)
        assert abs(mm.mean() - p_keep) < 6 * sdp


def test_bytes_uniform_chi_square():
    """The bytes behind the decisions are uniform: threshold sweep recovers
    the CDF, chi-square over 256 bins well inside its tail."""
    n_rows, lk = 1000, 1024
    ms = [oracle.keep_mask(7, 0, 0, np.arange(n_rows), lk, t) for t in (0, 64, 128, 192)]
    frac = [m.mean() for m in ms]
    for f, t in zip(frac, (0, 64, 128, 192)):
        sd = np.sqrt(0.25 / ms[0].size)
        assert abs(f - (1 - t / 256)) < 6 * sd
    # full histogram from the Philox words directly
    ctr = np.zeros((20000, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(20000)
    w = oracle.philox4x32(ctr, np.array([5, 6]))
    b = np.concatenate([(w >> (8 * s)) & 0xFF for s in range(4)]).ravel()
    hist = np.bincount(b.astype(np.int64), minlength=256)
    e = b.size / 256
    chi2 = ((hist - e) ** 2 / e).sum()
    assert 150 < chi2 < 380  # 255 degrees of freedom: mean 255, sd 22.6


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_p_zero_is_plain_attention():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 2, 9, 2, 8), _rand(rng, 2, 13, 2, 8), _rand(rng, 2, 13, 2, 8)
    o, l = oracle.attention_dropout(q, k, v, 0.4, True, 0.0, 77, seqlens_k=[13, 6])
    o0, l0 = oracle.attention(q, k, v, 0.4, True, seqlens_k=[13, 6])
    np.testing.assert_array_equal(o, o0)
    np.testing.assert_array_equal(l, l0)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_single_visible_key_closed_form(p):
    """Causal row 0 sees key 0 only: P = 1, so O = V0 * 256/(256 - t) if the
    key is kept, else 0; lse is the undropped one."""
    rng = np.random.default_rng(2)
    B, H, N, D = 2, 3, 5, 8
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, D)
    t = oracle.drop_threshold(p)
    o, l = oracle.attention_dropout(q, k, v, 0.3, True, p, 4242)
    _, l0 = oracle.attention(q, k, v, 0.3, True)
    np.testing.assert_array_equal(l, l0)
    for b in range(B):
        for h in range(H):
            kept = oracle.keep_mask(4242, b, h, [0], N, t)[0, 0]
            want = v[b, 0, h] * (256.0 / (256.0 - t)) if kept else np.zeros(D)
            np.testing.assert_allclose(o[b, 0, h], want, rtol=1e-14, atol=0)


def test_unbiased_over_seeds():
    """E[Z] = 1, so averaging over independent seeds approaches the
    undropped output; compared within 6 standard errors."""
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 4, 1, 8), _rand(rng, 1, 11, 1, 8), _rand(rng, 1, 11, 1, 8)
    o0, _ = oracle.attention(q, k, v, 0.5, False)
    runs = np.stack([oracle.attention_dropout(q, k, v, 0.5, False, 0.3, s)[0] for s in range(600)])
    mean = runs.mean(axis=0)
    se = runs.std(axis=0, ddof=1) / np.sqrt(runs.shape[0])
    assert np.all(np.abs(mean - o0) < 6 * se + 1e-12)


# ----------------------------------------------------------------------------
# Gradients with dropout
# ----------------------------------------------------------------------------

def _loss(q, k, v, do, scale, causal, p, seed, sl):
    o, _ = oracle.attention_dropout(q, k, v, scale, causal, p, seed, seqlens_k=sl)
    return float((o * do).sum())


def _fd(bwd, shape_q, nk, causal, sl, p, seed, rng_seed):
    rng = np.random.default_rng(rng_seed)
    B, nq, H, D = shape_q
    q, k, v = _rand(rng, B, nq, H, D), _rand(rng, B, nk, H, D), _rand(rng, B, nk, H, D)
    do = _rand(rng, B, nq, H, D)
    scale = 0.45
    got = bwd(q, k, v, do, scale, causal, sl, p, seed)
    eps = 1e-6
    for which, g in enumerate(got):
        args = [q, k, v]
        x = args[which]
        idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += eps
            xm[ix] -= eps
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num = (_loss(*ap, do, scale, causal, p, seed, sl) - _loss(*am, do, scale, causal, p, seed, sl)) / (2 * eps)
            assert abs(num - g[ix]) < 1e-6 + 1e-6 * abs(num), (which, ix, num, g[ix])


def _oracle_bwd(q, k, v, do, scale, causal, sl, p, seed):
    return oracle.attention_bwd(q, k, v, do, scale, causal, seqlens_k=sl, dropout_p=p, seed=seed)


@pytest.mark.parametrize("causal,sl", [(True, None), (False, [10, 4])])
def test_bwd_dropout_finite_differences(causal, sl):
    _fd(_oracle_bwd, (2, 7, 2, 4), 10, causal, sl, 0.3, 555, 11)


def _torch_grads(q, k, v, do, scale, causal, p, seed):
    B, nq, H, D = q.shape
    nk = k.shape[1]
    t = oracle.drop_threshold(p)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    outs = []
    for b in range(B):
        for h in range(H):
            s = scale * tq[b, :, h] @ tk[b, :, h].T
            if causal:
                vis = torch.tensor(oracle.visible(np.arange(nq), nq, nk, True))
                s = s.masked_fill(~vis, float("-inf"))
            pr = torch.softmax(s, dim=-1)
            z = torch.tensor(oracle.keep_mask(seed, b, h, np.arange(nq), nk, t) * oracle.keep_scale(t))
            outs.append(((pr * z) @ tv[b, :, h] * torch.tensor(do[b, :, h])).sum())
    torch.stack(outs).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_dropout_matches_torch_autograd(causal):
    rng = np.random.default_rng(12)
    q, k, v, do = (_rand(rng, 2, 9, 2, 8) for _ in range(4))
    ref = _torch_grads(q, k, v, do, 0.35, causal, 0.25, 31)
    got = oracle.attention_bwd(q, k, v, do, 0.35, causal, dropout_p=0.25, seed=31)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _keep_variant(kind):
    """keep_mask with one planted mistake (vectorised like the original)."""
    def keep(seed, b, h, q_pos, lk, t):
        q_pos = np.asarray(q_pos, dtype=np.int64).reshape(-1)
        groups = (lk + 15) // 16
        ctr = np.zeros((q_pos.size, groups, 4), dtype=np.uint64)
        ctr[..., 0] = np.arange(groups)[None, :]
        ctr[..., 1] = q_pos[:, None]
        ctr[..., 2], ctr[..., 3] = (b, h) if kind == "batch and head swapped" else (h, b)
        sd = int(seed)
        w = oracle.philox4x32(ctr, np.array([sd & 0xFFFFFFFF, sd >> 32])).astype(np.int64)
        j = np.arange(lk)
        byte = j & 3
        if kind == "byte order reversed":
            byte = 3 - byte
        val = (w[:, j >> 4, (j >> 2) & 3] >> (8 * byte)) & 0xFF
        return val > t if kind == "keep iff byte > t" else val >= t
    return keep


def _forward_variant(kind, keepf):
    def fwd(q, k, v, scale, causal, p, seed):
        t = oracle.drop_threshold(p)
        B, nq, H, D = q.shape
        nk = k.shape[1]
        o = np.zeros(q.shape)
        for b in range(B):
            for h in range(H):
                s = scale * q[b, :, h] @ k[b, :, h].T
                if causal:
                    s = np.where(oracle.visible(np.arange(nq), nq, nk, True), s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                keep = keepf(seed, b, h, np.arange(nq), nk, t)
                sc = 1.0 / (1.0 - p) if kind == "scale 1/(1-p)" else oracle.keep_scale(t)
                if kind == "dropped sum normalises":
                    ed = np.where(keep, e, 0.0)
                    with np.errstate(invalid="ignore"):
                        o[b, :, h] = (ed @ v[b, :, h]) / ed.sum(axis=1, keepdims=True)
                else:
                    o[b, :, h] = (np.where(keep, e, 0.0) * sc) @ v[b, :, h] / e.sum(axis=1, keepdims=True)
        return o
    return fwd


def _pin_mapping(keepf):
    words = KAT[0][2]
    bytes_ = [(words[j // 4] >> (8 * (j % 4))) & 0xFF for j in range(16)]
    for t in (1, 64, 128, 200, 255):
        assert keepf(0, 0, 0, [0], 16, t)[0].tolist() == [x >= t for x in bytes_]


def _pin_counter_fields(keepf):
    seed = 0x0123456789ABCDEF
    i, h, b, j = 7, 3, 2, 37
    w = oracle.philox4x32(np.array([j // 16, i, h, b]), np.array([seed & 0xFFFFFFFF, seed >> 32]))
    byte = (int(w[(j // 4) % 4]) >> (8 * (j % 4))) & 0xFF
    for t in (byte, byte + 1):
        if t <= 255:
            assert keepf(seed, b, h, [i], 40, t)[0, j] == (byte >= t)


def _pin_rate(keepf):
    m = keepf(99, 1, 5, np.arange(2000), 512, 128)
    sd = np.sqrt(0.25 / m.size)
    assert abs(m.mean() - 0.5) < 6 * sd


def _pin_single_key(fwd):
    rng = np.random.default_rng(2)
    B, H, N, D = 2, 3, 5, 8
    q, k, v = _rand(rng, B, N, H, D), _rand(rng, B, N, H, D), _rand(rng, B, N, H, D)
    for p in (0.1, 0.5, 0.9):
        t = oracle.drop_threshold(p)
        o = fwd(q, k, v, 0.3, True, p, 4242)
        for b in range(B):
            for h in range(H):
                kept = oracle.keep_mask(4242, b, h, [0], N, t)[0, 0]
                want = v[b, 0, h] * (256.0 / (256.0 - t)) if kept else np.zeros(D)
                np.testing.assert_allclose(o[b, 0, h], want, rtol=1e-14, atol=0)


FWD_MISTAKES = ["byte order reversed", "keep iff byte > t", "batch and head swapped", "scale 1/(1-p)",
                "dropped sum normalises"]


def test_pins_pass_on_the_oracle():
    for pin in (_pin_mapping, _pin_counter_fields, _pin_rate):
        pin(oracle.keep_mask)
    _pin_single_key(lambda q, k, v, sc, c, p, s: oracle.attention_dropout(q, k, v, sc, c, p, s)[0])


@pytest.mark.parametrize("kind", FWD_MISTAKES)
def test_planted_forward_mistakes_are_caught(kind):
    """Each planted mistake must fail at least one pin."""
    keepf = _keep_variant(kind)
    fwd = _forward_variant(kind, keepf)
    pins = [lambda: _pin_mapping(keepf), lambda: _pin_counter_fields(keepf), lambda: _pin_rate(keepf),
            lambda: _pin_single_key(fwd)]
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, "no pin caught the planted mistake: %s" % kind


BWD_MISTAKES = ["dV without the mask", "dP without the mask"]


def _bad_bwd(kind):
    def bwd(q, k, v, do, scale, causal, sl, p, seed):
        B, nq, H, D = q.shape
        nk = k.shape[1]
        t = oracle.drop_threshold(p)
        dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            lk = nk if sl is None else sl[b]
            for h in range(H):
                qq, kk, vv, g = q[b, :, h], k[b, :lk, h], v[b, :lk, h], do[b, :, h]
                s = scale * qq @ kk.T
                if causal:
                    s = np.where(oracle.visible(np.arange(nq), nq, lk, True), s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isneginf(m), 0, m)
                e = np.exp(s - m)
                pr = e / e.sum(axis=1, keepdims=True)
                z = oracle.keep_mask(seed, b, h, np.arange(nq), lk, t) * oracle.keep_scale(t)
                o = (pr * z) @ vv
                dv[b, :lk, h] = (pr if kind == "dV without the mask" else pr * z).T @ g
                dp = g @ vv.T if kind == "dP without the mask" else (g @ vv.T) * z
                ds = pr * (dp - (g * o).sum(axis=1, keepdims=True))
                dq[b, :, h] = scale * ds @ kk
                dk[b, :lk, h] = scale * ds.T @ qq
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", BWD_MISTAKES)
def test_planted_backward_mistakes_are_caught(kind):
    with pytest.raises(AssertionError):
        _fd(_bad_bwd(kind), (2, 7, 2, 4), 10, True, None, 0.3, 555, 11)
