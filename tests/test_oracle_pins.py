"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

None of these checks re-types the oracle's formula.  They use pure-Python
brute force (``math.exp`` / ``math.fsum``, no numpy), closed forms,
invariants of softmax attention, the block-merge claim of the pages, and
torch's CPU float64 attention as an independent library routine.  The last
test plants mistakes in the oracle and checks that the pins catch each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.exact as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Brute force: pure Python, independent of numpy
# ----------------------------------------------------------------------------

def brute_row(q, K, V, lk, i, lq, scale, causal):
    """O row and lse for query i, by loops over keys (standard attention)."""
    s = []
    for j in range(lk):
        if causal and j > i + lk - lq:
            continue
        s.append((math.fsum(q[d] * K[j][d] for d in range(len(q))) * scale, j))
    if not s:
        return [0.0] * len(V[0]), -math.inf
    mx = s[0][0]
    for x, _ in s:
        if x > mx:
            mx = x
    w = [(math.exp(x - mx), j) for x, j in s]
    den = math.fsum(e for e, _ in w)
    out = [math.fsum(e * V[j][d] for e, j in w) / den for d in range(len(V[0]))]
    return out, mx + math.log(den)


def brute(q, k, v, scale, causal, seqlens_k=None):
    B, nq, H, D = q.shape
    nk = k.shape[1]
    o = np.zeros((B, nq, H, v.shape[-1]))
    lse = np.zeros((B, H, nq))
    for b in range(B):
        lk = nk if seqlens_k is None else int(seqlens_k[b])
        for h in range(H):
            K = [list(map(float, k[b, j, h])) for j in range(nk)]
            V = [list(map(float, v[b, j, h])) for j in range(nk)]
            for i in range(nq):
                orow, l = brute_row(list(map(float, q[b, i, h])), K, V, lk, i, nq, scale, causal)
                o[b, i, h] = orow
                lse[b, h, i] = l
    return o, lse


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 3, 5, 2, 4), (1, 6, 6, 3, 2), (2, 5, 3, 1, 3), (1, 2, 6, 2, 4)])
def test_brute_force(shape, causal):
    """The whole oracle against loops over keys (tiny B, Nq, Nk, H, D)."""
    B, nq, nk, H, D = shape
    rng = np.random.default_rng(hash((shape, causal)) & 0xFFFF)
    q, k, v = rnd(rng, B, nq, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nk, H, D)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, scale, causal)
    ob, lb = brute(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_padded_keys(causal):
    """seqlens_k: keys at or beyond a batch entry's length are padding."""
    rng = np.random.default_rng(7)
    B, nq, nk, H, D = 3, 4, 6, 2, 3
    q, k, v = rnd(rng, B, nq, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nk, H, D)
    lens = np.array([6, 2, 4])
    o, lse = oracle.attention(q, k, v, 0.5, causal, seqlens_k=lens)
    ob, lb = brute(q, k, v, 0.5, causal, seqlens_k=lens)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    fin = np.isfinite(lb)
    np.testing.assert_array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)


def test_identical_keys_give_mean_of_visible_values():
    """All keys equal: every visible key gets the same weight, so O is the mean of V."""
    rng = np.random.default_rng(1)
    B, N, H, D = 1, 9, 2, 4
    q = rnd(rng, B, N, H, D)
    krow = rnd(rng, D)
    k = np.broadcast_to(krow, (B, N, H, D)).copy()
    v = rnd(rng, B, N, H, D)
    scale = 0.8
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, scale, causal)
        for h in range(H):
            for i in range(N):
                nvis = i + 1 if causal else N
                np.testing.assert_allclose(o[0, i, h], v[0, :nvis, h].mean(axis=0), atol=1e-13)
                s = scale * float(q[0, i, h] @ krow)
                assert abs(lse[0, h, i] - (s + math.log(nvis))) < 1e-12


def test_single_visible_key_returns_its_value_row():
    rng = np.random.default_rng(2)
    q, k, v = rnd(rng, 2, 5, 3, 4), rnd(rng, 2, 1, 3, 4), rnd(rng, 2, 1, 3, 4)
    o, lse = oracle.attention(q, k, v, 0.6, False)
    for b in range(2):
        for h in range(3):
            for i in range(5):
                np.testing.assert_array_equal(o[b, i, h], v[b, 0, h])
                assert abs(lse[b, h, i] - 0.6 * float(q[b, i, h] @ k[b, 0, h])) < 1e-13


def test_causal_row0_equals_v0():
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 2, 7, 2, 5), rnd(rng, 2, 7, 2, 5), rnd(rng, 2, 7, 2, 5)
    o, lse = oracle.attention(q, k, v, 0.3, True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), atol=1e-13)


def test_scale_zero_is_uniform_average():
    rng = np.random.default_rng(4)
    q, k, v = rnd(rng, 1, 6, 1, 3), rnd(rng, 1, 6, 1, 3), rnd(rng, 1, 6, 1, 3)
    o, lse = oracle.attention(q, k, v, 0.0, True)
    for i in range(6):
        np.testing.assert_allclose(o[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-14


def test_two_keys_closed_form():
    """Two keys: weights are the logistic function of the score difference."""
    rng = np.random.default_rng(5)
    q, k, v = rnd(rng, 1, 4, 1, 6), rnd(rng, 1, 2, 1, 6), rnd(rng, 1, 2, 1, 6)
    scale = 1.3
    o, lse = oracle.attention(q, k, v, scale, False)
    for i in range(4):
        s0 = scale * float(q[0, i, 0] @ k[0, 0, 0])
        s1 = scale * float(q[0, i, 0] @ k[0, 1, 0])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(o[0, i, 0], w0 * v[0, 0, 0] + w1 * v[0, 1, 0], atol=1e-14)
        assert abs(lse[0, 0, i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-13


def test_hand_worked_example():
    """Scores (ln 3, 0): weights 3/4 and 1/4, lse = ln 4 (worked by hand)."""
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[math.log(3.0), 5.0]], [[0.0, -2.0]]]])
    v = np.array([[[[4.0, 0.0]], [[0.0, 8.0]]]])
    o, lse = oracle.attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], [3.0, 2.0], atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(4.0)) < 1e-14


def test_large_scores_stay_finite():
    """Safe softmax: scores far past the fp16 exp overflow point give exact weights."""
    q = np.array([[[[1000.0]]]])
    k = np.array([[[[1.0]], [[0.999]]]])
    v = np.array([[[[1.0]], [[0.0]]]])
    o, lse = oracle.attention(q, k, v, 1.0, False)
    assert abs(o[0, 0, 0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-12
    assert abs(lse[0, 0, 0] - (1000.0 + math.log1p(math.exp(-1.0)))) < 1e-10


def test_shift_of_keys_leaves_output_and_shifts_lse():
    rng = np.random.default_rng(6)
    q, k, v = rnd(rng, 1, 5, 2, 4), rnd(rng, 1, 5, 2, 4), rnd(rng, 1, 5, 2, 4)
    c = rnd(rng, 4)
    scale = 0.7
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, scale, causal)
        o2, l2 = oracle.attention(q, k + c, v, scale, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-12)
        shift = scale * np.einsum("bihd,d->bhi", q, c)
        np.testing.assert_allclose(l2, l1 + shift, atol=1e-12)


def test_noncausal_invariants():
    rng = np.random.default_rng(8)
    q, k, v = rnd(rng, 2, 4, 2, 3), rnd(rng, 2, 6, 2, 3), rnd(rng, 2, 6, 2, 3)
    o, lse = oracle.attention(q, k, v, 0.9, False)
    perm = rng.permutation(6)
    o2, lse2 = oracle.attention(q, k[:, perm], v[:, perm], 0.9, False)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    o3, _ = oracle.attention(q, k, np.ones_like(v), 0.9, False)
    np.testing.assert_allclose(o3, 1.0, atol=1e-14)
    v2 = rnd(rng, 2, 6, 2, 3)
    oa_, _ = oracle.attention(q, k, v2, 0.9, False)
    ob_, _ = oracle.attention(q, k, 2.0 * v - 3.0 * v2, 0.9, False)
    np.testing.assert_allclose(ob_, 2.0 * o - 3.0 * oa_, atol=1e-12)


def test_padding_garbage_is_ignored():
    rng = np.random.default_rng(9)
    q, k, v = rnd(rng, 2, 3, 2, 4), rnd(rng, 2, 8, 2, 4), rnd(rng, 2, 8, 2, 4)
    lens = np.array([5, 8])
    o, lse = oracle.attention(q, k, v, 0.5, True, seqlens_k=lens)
    k2, v2 = k.copy(), v.copy()
    k2[0, 5:] = np.nan
    v2[0, 5:] = 1e30
    o2, lse2 = oracle.attention(q, k2, v2, 0.5, True, seqlens_k=lens)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_rows_without_visible_keys():
    """Causal, more queries than keys (bottom-right): the first Nq-Nk rows see nothing."""
    rng = np.random.default_rng(10)
    q, k, v = rnd(rng, 1, 6, 1, 2), rnd(rng, 1, 3, 1, 2), rnd(rng, 1, 3, 1, 2)
    o, lse = oracle.attention(q, k, v, 1.0, True)
    np.testing.assert_array_equal(o[0, :3], 0.0)
    assert np.all(np.isneginf(lse[0, 0, :3]))
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    np.testing.assert_array_equal(o[0, 3, 0], v[0, 0, 0])
    ob, lb = brute(q, k, v, 1.0, True)
    np.testing.assert_allclose(o, ob, atol=1e-13)
    # no keys at all
    o0, l0 = oracle.attention(q, k, v, 1.0, False, seqlens_k=[0])
    np.testing.assert_array_equal(o0, 0.0)
    assert np.all(np.isneginf(l0))


def _random_partition(rng, n):
    cuts = sorted(rng.choice(np.arange(0, n + 1), size=rng.integers(1, 5), replace=True).tolist())
    edges = [0] + cuts + [n]
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1)]


@pytest.mark.parametrize("seed", range(6))
def test_blockwise_merge_equals_full_softmax(seed):
    """The tiled-softmax claim: merging block summaries in any grouping gives the full result.

    Includes empty blocks and fully masked blocks (m = -inf).
    """
    rng = np.random.default_rng(100 + seed)
    n, c, d = 4, 17, 3
    s = rng.standard_normal((n, c)) * 3
    s[:, rng.integers(0, c, size=5)] = -np.inf      # masked keys
    s[1, 3:9] = -np.inf                              # a fully masked stretch for row 1
    v = rng.standard_normal((c, d))
    # reference: the definition with unit scale on prebuilt scores
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    o_ref = (p @ v) / p.sum(axis=1)[:, None]
    lse_ref = m + np.log(p.sum(axis=1))
    parts = [oracle.partial(s[:, a:b], v[a:b]) for a, b in _random_partition(rng, c)]
    # left fold
    acc = parts[0]
    for pp in parts[1:]:
        acc = oracle.merge(acc, pp)
    o1, l1 = oracle.finalize(acc)
    # right fold
    acc = parts[-1]
    for pp in reversed(parts[:-1]):
        acc = oracle.merge(pp, acc)
    o2, l2 = oracle.finalize(acc)
    # pairwise tree
    level = parts
    while len(level) > 1:
        nxt = [oracle.merge(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    o3, l3 = oracle.finalize(level[0])
    for o_, l_ in ((o1, l1), (o2, l2), (o3, l3)):
        np.testing.assert_allclose(o_, o_ref, atol=1e-13)
        np.testing.assert_allclose(l_, lse_ref, atol=1e-13)


def test_three_group_merge_matches_attention_rows():
    """The primer's example structure: x split into x(1), x(2), x(3), merged (1,2) then 3.

    The page's numbers are stripped; random data of the same structure is used
    and the result is compared with the oracle's materialised attention.
    """
    rng = np.random.default_rng(11)
    D, L = 5, 12
    q = rng.standard_normal((3, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    scale = 0.45
    s = scale * (q @ k.T)
    g = [(0, 4), (4, 9), (9, 12)]
    p12 = oracle.merge(oracle.partial(s[:, 0:4], v[0:4]), oracle.partial(s[:, 4:9], v[4:9]))
    o, lse = oracle.finalize(oracle.merge(p12, oracle.partial(s[:, 9:12], v[9:12])))
    o_ref, lse_ref = oracle.attention_rows(q, [0, 1, 2], k, v, 3, L, scale, False)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-13)
    assert len(g) == 3


def test_torch_cpu_float64_sdpa():
    """Library special case: torch's float64 CPU attention (non-causal; causal with Nq = Nk)."""
    rng = np.random.default_rng(12)
    B, N, H, D = 2, 37, 3, 8
    q, k, v = rnd(rng, B, N, H, D), rnd(rng, B, N, H, D), rnd(rng, B, N, H, D)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, 0.21, causal)
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.21)
        np.testing.assert_allclose(o, ot.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_varlen_equals_per_sequence_batches():
    rng = np.random.default_rng(13)
    lens = [3, 1, 6, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, D = 2, 3
    tot = cu[-1]
    q, k, v = rnd(rng, tot, H, D), rnd(rng, tot, H, D), rnd(rng, tot, H, D)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu, cu, 0.6, causal)
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            ob, lb = brute(q[None, a:b], k[None, a:b], v[None, a:b], 0.6, causal)
            np.testing.assert_allclose(o[a:b], ob[0], atol=1e-12)
            np.testing.assert_allclose(lse[:, a:b], lb[0], atol=1e-12)


def test_decode_is_one_noncausal_row():
    rng = np.random.default_rng(14)
    B, H, D, nmax = 3, 2, 4, 7
    q = rnd(rng, B, H, D)
    kc, vc = rnd(rng, B, nmax, H, D), rnd(rng, B, nmax, H, D)
    lens = np.array([7, 1, 4])
    o, lse = oracle.decode(q, kc, vc, lens, 0.4)
    ob, lb = brute(q[:, None], kc, vc, 0.4, False, seqlens_k=lens)
    np.testing.assert_allclose(o, ob[:, 0], atol=1e-13)
    np.testing.assert_allclose(lse, lb[:, :, 0], atol=1e-13)


def _scatter_pages(rng, kc, vc, lens, page_size, extra_pages=3):
    """A page pool holding each entry's cache pages at shuffled positions,
    NaN everywhere else, and the page table that finds them."""
    B, nmax, H, D = kc.shape
    per = -(-nmax // page_size)
    n_pages = B * per + extra_pages
    perm = rng.permutation(n_pages)
    kp = np.full((n_pages, page_size, H, D), np.nan)
    vp = np.full((n_pages, page_size, H, D), np.nan)
    table = np.zeros((B, per), np.int32)
    for b in range(B):
        for i in range(per):
            pg = int(perm[b * per + i])
            table[b, i] = pg
            rows = range(i * page_size, min((i + 1) * page_size, int(lens[b])))
            for t in rows:
                kp[pg, t - i * page_size] = kc[b, t]
                vp[pg, t - i * page_size] = vc[b, t]
    return kp, vp, table


def test_decode_paged_is_decode_of_the_gathered_cache():
    """Pages at shuffled pool positions, NaN in every unused page and row:
    the paged decode equals the contiguous decode exactly."""
    rng = np.random.default_rng(21)
    B, H, D, nmax, ps = 4, 2, 4, 40, 16
    q = rnd(rng, B, H, D)
    kc, vc = rnd(rng, B, nmax, H, D), rnd(rng, B, nmax, H, D)
    lens = np.array([40, 17, 1, 0])
    kp, vp, table = _scatter_pages(rng, kc, vc, lens, ps)
    o, lse = oracle.decode_paged(q, kp, vp, table, lens, 0.3)
    oc, lc = oracle.decode(q, kc, vc, lens, 0.3)
    assert np.array_equal(o, oc) and np.array_equal(lse, lc)
    assert np.isfinite(o).all()
    assert (o[3] == 0).all() and (lse[3] == -np.inf).all()  # an empty cache


def test_decode_paged_brute_force():
    """Pure-Python loop over keys reading rows through the table."""
    rng = np.random.default_rng(22)
    B, H, D, nmax, ps = 2, 2, 3, 37, 16
    q = rnd(rng, B, H, D)
    kc, vc = rnd(rng, B, nmax, H, D), rnd(rng, B, nmax, H, D)
    lens = np.array([37, 20])
    kp, vp, table = _scatter_pages(rng, kc, vc, lens, ps)
    o, lse = oracle.decode_paged(q, kp, vp, table, lens, 0.7)
    for b in range(B):
        for h in range(H):
            K = [list(map(float, kp[table[b][t // ps], t % ps, h])) for t in range(lens[b])]
            V = [list(map(float, vp[table[b][t // ps], t % ps, h])) for t in range(lens[b])]
            ob, lb = brute_row(list(map(float, q[b, h])), K, V, int(lens[b]), 0, 1, 0.7, False)
            np.testing.assert_allclose(o[b, h], ob, atol=1e-13)
            assert abs(lse[b, h] - lb) < 1e-13


def test_golden_page_facts():
    """Numbers printed by the pages (see the fixture for citations)."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        g = json.load(f)
    ex = g["cann_test_shapes"]
    rng = np.random.default_rng(15)
    shp = tuple(ex["q_shape"])
    q, k, v = rnd(rng, *shp), rnd(rng, *shp), rnd(rng, *shp)
    o, lse = oracle.attention(q[:, :16], k[:, :16], v[:, :16], 1 / math.sqrt(shp[-1]), True)
    assert list(o.shape[2:]) == ex["output_shape"][2:] and o.shape[0] == ex["output_shape"][0]
    sm = g["materialised_s_bytes"]
    B, H, N, _ = sm["shape_bhnd"]
    assert B * H * N * N * sm["bytes_per_element"] == sm["actual_bytes"]
    assert sm["actual_bytes"] * 4 == sm["printed_gb"] * 2 ** 30  # the page's figure is 4x the product
    f16 = g["fp16_overflow"]
    assert float(np.float16(f16["max"])) == 65504.0
    with np.errstate(over="ignore"):
        assert np.isfinite(np.float16(math.exp(f16["threshold_exact"] - 1e-3)))
        assert np.isinf(np.float32(np.float16(math.exp(f16["threshold_exact"] + 1e-3))))
    assert f16["printed_threshold"] <= f16["threshold_exact"] < f16["printed_threshold"] + 0.1


# ----------------------------------------------------------------------------
# Prefix mask and ALiBi bias (the integration guide's other mask families)
# ----------------------------------------------------------------------------

def brute_masked_row(q, K, V, lk, i, lq, scale, causal, prefix, slope):
    """Pure-Python row: visible keys under the causal + prefix mask, each
    score plus -slope * |j - (i + lk - lq)|."""
    pos = i + lk - lq
    s = []
    for j in range(lk):
        if causal and j > pos and j >= prefix:
            continue
        s.append((math.fsum(q[d] * K[j][d] for d in range(len(q))) * scale - slope * abs(j - pos), j))
    if not s:
        return [0.0] * len(V[0]), -math.inf
    mx = max(x for x, _ in s)
    w = [(math.exp(x - mx), j) for x, j in s]
    den = math.fsum(e for e, _ in w)
    return [math.fsum(e * V[j][d] for e, j in w) / den for d in range(len(V[0]))], mx + math.log(den)


@pytest.mark.parametrize("nq,nk,prefix,slopes,causal", [
    (5, 5, 2, None, True), (4, 7, 3, None, True), (6, 4, 1, None, True), (5, 5, 9, None, True),
    (5, 5, 0, [0.3, 1.1], True), (4, 6, 2, [0.5, 0.0], True), (5, 5, 0, [0.25, 2.0], False),
    (3, 7, 0, [0.7, 0.1], False),
])
def test_prefix_and_alibi_brute_force(nq, nk, prefix, slopes, causal):
    rng = np.random.default_rng(31 + nq * 7 + nk + prefix)
    B, H, D = 2, 2, 3
    q, k, v = rnd(rng, B, nq, H, D), rnd(rng, B, nk, H, D), rnd(rng, B, nk, H, D)
    sl = None if slopes is None else np.array(slopes)
    o, lse = oracle.attention(q, k, v, 0.6, causal, prefix=prefix, alibi_slopes=sl)
    for b in range(B):
        for h in range(H):
            K = [list(map(float, k[b, j, h])) for j in range(nk)]
            V = [list(map(float, v[b, j, h])) for j in range(nk)]
            for i in range(nq):
                ob, lb = brute_masked_row(list(map(float, q[b, i, h])), K, V, nk, i, nq, 0.6,
                                          causal, prefix, 0.0 if sl is None else sl[h])
                np.testing.assert_allclose(o[b, i, h], ob, atol=1e-13)
                assert lse[b, h, i] == lb or abs(lse[b, h, i] - lb) < 1e-13


def test_prefix_mask_special_cases():
    """prefix 0 is the causal mask; a prefix covering every key is no mask."""
    rng = np.random.default_rng(41)
    q, k, v = rnd(rng, 2, 6, 2, 4), rnd(rng, 2, 6, 2, 4), rnd(rng, 2, 6, 2, 4)
    a = oracle.attention(q, k, v, 0.5, True, prefix=0)
    b = oracle.attention(q, k, v, 0.5, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.attention(q, k, v, 0.5, True, prefix=6)
    d = oracle.attention(q, k, v, 0.5, False)
    np.testing.assert_allclose(c[0], d[0], atol=1e-14)
    np.testing.assert_allclose(c[1], d[1], atol=1e-14)


def test_alibi_special_cases():
    """Slope 0 is no bias; a huge slope leaves only the key at the query's own
    position, so the row is that key's value and the log-sum-exp its score."""
    rng = np.random.default_rng(42)
    nq, nk = 4, 6
    q, k, v = rnd(rng, 1, nq, 2, 4), rnd(rng, 1, nk, 2, 4), rnd(rng, 1, nk, 2, 4)
    a = oracle.attention(q, k, v, 0.5, True, alibi_slopes=np.zeros(2))
    b = oracle.attention(q, k, v, 0.5, True)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)
    for causal in (True, False):
        o, lse = oracle.attention(q, k, v, 0.5, causal, alibi_slopes=np.array([1e4, 1e4]))
        for i in range(nq):
            p = i + nk - nq
            np.testing.assert_allclose(o[0, i], v[0, p], atol=1e-12)
            for h in range(2):
                assert abs(lse[0, h, i] - 0.5 * float(q[0, i, h] @ k[0, p, h])) < 1e-9


def test_causal_alibi_is_attention_on_augmented_vectors():
    """For causal rows the bias slope*(j - p) is slope*j plus a per-row
    constant, which softmax ignores: it equals plain attention after appending
    1 to every query and slope*j/scale to key j (lse shifted by slope*p)."""
    rng = np.random.default_rng(43)
    nq, nk, D, scale, slope = 5, 8, 3, 0.4, 0.35
    q, k, v = rnd(rng, 1, nq, 1, D), rnd(rng, 1, nk, 1, D), rnd(rng, 1, nk, 1, D)
    o, lse = oracle.attention(q, k, v, scale, True, alibi_slopes=np.array([slope]))
    qa = np.concatenate([q, np.ones((1, nq, 1, 1))], axis=-1)
    ka = np.concatenate([k, (slope * np.arange(nk) / scale).reshape(1, nk, 1, 1)], axis=-1)
    o2, lse2 = oracle.attention(qa, ka, v, scale, True)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    p = np.arange(nq) + nk - nq
    np.testing.assert_allclose(lse[0, 0], lse2[0, 0] - slope * p, atol=1e-13)


def _alibi_sign_flip(q_pos, lq, lk, slope):
    q_pos = np.asarray(q_pos).reshape(-1)
    return float(slope) * np.abs(np.arange(lk)[None, :] - (q_pos[:, None] + lk - lq)).astype(float)


def _alibi_top_left(q_pos, lq, lk, slope):
    q_pos = np.asarray(q_pos).reshape(-1)
    return -float(slope) * np.abs(np.arange(lk)[None, :] - q_pos[:, None]).astype(float)


def _vis_prefix_inclusive(q_pos, lq, lk, causal, prefix=0):
    q_pos = np.asarray(q_pos).reshape(-1)
    j = np.arange(lk)
    if not causal:
        return np.ones((q_pos.size, lk), bool)
    return (j[None, :] <= q_pos[:, None] + lk - lq) | (j[None, :] <= prefix)


_MASK_PINS = [
    lambda: test_prefix_and_alibi_brute_force(5, 5, 2, None, True),
    lambda: test_prefix_and_alibi_brute_force(6, 4, 1, None, True),
    lambda: test_prefix_and_alibi_brute_force(4, 6, 2, [0.5, 0.0], True),
    lambda: test_prefix_and_alibi_brute_force(3, 7, 0, [0.7, 0.1], False),
    test_alibi_special_cases,
    test_causal_alibi_is_attention_on_augmented_vectors,
]


@pytest.mark.parametrize("name,attr,bad", [
    ("alibi sign flipped", "alibi_bias", _alibi_sign_flip),
    ("alibi position top-left", "alibi_bias", _alibi_top_left),
    ("prefix bound inclusive", "visible", _vis_prefix_inclusive),
])
def test_planted_mask_mistakes_are_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(oa, attr, bad)
    caught = 0
    for pin in _MASK_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"


# ----------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin above
# ----------------------------------------------------------------------------

def _no_scale(q, k, scale):
    return np.asarray(q, float) @ np.asarray(k, float).T


def _sign_flip(q, k, scale):
    return -float(scale) * (np.asarray(q, float) @ np.asarray(k, float).T)


def _vis_strict(q_pos, lq, lk, causal, prefix=0):
    q_pos = np.asarray(q_pos).reshape(-1)
    j = np.arange(lk)
    if not causal:
        return np.ones((q_pos.size, lk), bool)
    return j[None, :] < (q_pos[:, None] + lk - lq)


def _vis_top_left(q_pos, lq, lk, causal, prefix=0):
    q_pos = np.asarray(q_pos).reshape(-1)
    j = np.arange(lk)
    if not causal:
        return np.ones((q_pos.size, lk), bool)
    return j[None, :] <= q_pos[:, None]


_PINS = [
    lambda: test_brute_force((2, 3, 5, 2, 4), True),
    lambda: test_brute_force((2, 3, 5, 2, 4), False),
    test_identical_keys_give_mean_of_visible_values,
    test_causal_row0_equals_v0,
    test_two_keys_closed_form,
    test_rows_without_visible_keys,
    test_torch_cpu_float64_sdpa,
]


@pytest.mark.parametrize("name,attr,bad", [
    ("scale dropped", "scores", _no_scale),
    ("sign flipped", "scores", _sign_flip),
    ("causal off by one", "visible", _vis_strict),
    ("causal top-left aligned", "visible", _vis_top_left),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(oa, attr, bad)
    caught = 0
    for pin in _PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
