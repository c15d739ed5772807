"""GPU parity at the benchmark workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot finish whole workloads of this size in a test, so each case compares sampled
output rows (chosen at random plus tile boundaries and the first/last rows) with the oracle
computed row by row, and checks properties that hold at any size on every row: all outputs
finite (the output buffers start filled with NaN, so this also shows every element was written),
every causal row has a finite log-sum-exp, and two runs are bit-identical.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import assert_close, assert_grad_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _fa():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    return fa


def nan_like(t, shape=None, dtype=None):
    """An output buffer filled with NaN: after the call, an all-finite check over it
    shows that the kernel wrote every element."""
    return torch.full(t.shape if shape is None else shape, float("nan"),
                      dtype=t.dtype if dtype is None else dtype, device=t.device)


def nan_grads(q, k):
    return dict(dq=nan_like(q), dk=nan_like(k), dv=nan_like(k))


def _sample_rows(rng, n, extra=()):
    base = {0, 1, n - 1, n // 2}
    for t in (63, 64, 127, 128, 255, 256, 511, 512):
        if t < n:
            base.add(t)
    base.update(int(x) for x in extra if 0 <= x < n)
    base.update(int(x) for x in rng.integers(0, n, size=24))
    return sorted(base)


@pytest.mark.parametrize("cfg", [2, 3, 7, 8])
def test_prefill_full_size_sampled(cfg):
    fa = _fa()
    w = wl.CFG[cfg]
    say("generate %s" % w.name)
    q, k, v = wl.prefill_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    slopes = wl.alibi_slopes(w.H) if w.alibi else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()

    def call():
        outs = dict(out=nan_like(qd), lse=nan_like(qd, (w.B, w.H, w.Nq), torch.float32))
        if w.prefix or w.alibi:
            return fa.fwd_masked(qd, kd, vd, causal=w.causal, scale=w.scale, prefix=w.prefix,
                                 alibi_slopes=sd, **outs)
        return fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, **outs)
    say("fa_fwd %s" % w.name)
    o, lse = call()
    o2, lse2 = call()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    rng = np.random.default_rng(1000 + cfg)
    pairs = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
    for b, h in pairs:
        rows = _sample_rows(rng, w.Nq)
        kb, vb = wl.to_f64(k[b, :, h]), wl.to_f64(v[b, :, h])
        qr = wl.to_f64(q[b, rows, h])
        o_ref, lse_ref = oracle.attention_rows(qr, rows, kb, vb, w.Nq, w.Nk, w.scale, w.causal,
                                               w.prefix, None if slopes is None else float(slopes[h]))
        assert_close(w.dtype, wl.to_f64(o_c[b, rows, h]), o_ref, lse_c[b, h, rows].double().numpy(),
                     lse_ref, "%s b%d h%d" % (w.name, b, h))


def test_varlen_full_size_sampled():
    fa = _fa()
    w = wl.CFG[4]
    say("generate %s" % w.name)
    q, k, v, cu = wl.varlen_inputs(w)
    cud = torch.from_numpy(cu).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say("fa_fwd_varlen %s" % w.name)
    o, lse = fa.fwd_varlen(qd, kd, vd, cud, cud, causal=True, scale=w.scale, out=nan_like(qd),
                           lse=nan_like(qd, (w.H, qd.shape[0]), torch.float32))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    rng = np.random.default_rng(1004)
    lens = np.diff(cu)
    for s in range(len(lens)):
        h = int(rng.integers(w.H))
        a0, L = int(cu[s]), int(lens[s])
        rows = _sample_rows(rng, L)
        kb, vb = wl.to_f64(k[a0:a0 + L, h]), wl.to_f64(v[a0:a0 + L, h])
        qr = wl.to_f64(q[[a0 + r for r in rows], h])
        o_ref, lse_ref = oracle.attention_rows(qr, rows, kb, vb, L, L, w.scale, True)
        got = wl.to_f64(o_c[[a0 + r for r in rows], h])
        assert_close(w.dtype, got, o_ref, lse_c[h, [a0 + r for r in rows]].double().numpy(), lse_ref,
                     "%s seq%d h%d" % (w.name, s, h))


def test_decode_full_size_sampled():
    fa = _fa()
    w = wl.CFG[5]
    lens = w.lengths()
    say("generate %s (device caches %.1f GB each)" % (w.name, w.B * w.Nk * w.H * w.D * 2 / 1e9))
    q = wl.decode_query(w)
    kc = torch.empty((w.B, w.Nk, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for b in range(w.B):
        L = int(lens[b])
        kc[b, :L].copy_(wl.decode_cache_rows(w, 1, b, L))
        vc[b, :L].copy_(wl.decode_cache_rows(w, 2, b, L))
        # rows past the length must never be read: fill a band of them with NaN
        kc[b, L:min(w.Nk, L + 300)] = float("nan")
        vc[b, L:min(w.Nk, L + 300)] = float("nan")
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    say("fa_decode_splitkv %s" % w.name)
    qd = q.cuda()
    dout = lambda: dict(out=nan_like(qd), lse=nan_like(qd, (w.B, w.H), torch.float32))
    o, lse = fa.decode_splitkv(qd, kc, vc, sl, scale=w.scale, chunk=w.chunk, **dout())
    o2, lse2 = fa.decode_splitkv(qd, kc, vc, sl, scale=w.scale, chunk=w.chunk, **dout())
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    del kc, vc
    rng = np.random.default_rng(1005)
    bs = sorted({0, w.B - 1, int(np.argmax(lens)), int(np.argmin(lens))} | {int(x) for x in rng.integers(0, w.B, 4)})
    for b in bs:
        L = int(lens[b])
        kb = wl.to_f64(wl.decode_cache_rows(w, 1, b, L))
        vb = wl.to_f64(wl.decode_cache_rows(w, 2, b, L))
        for h in sorted({0, w.H - 1, int(rng.integers(w.H))}):
            o_ref, lse_ref = oracle.attention_rows(wl.to_f64(q[b, h])[None], [0], kb[:, h], vb[:, h], 1,
                                                   L, w.scale, False)
            assert_close(w.dtype, wl.to_f64(o_c[b, h])[None], o_ref, lse_c[b, h:h + 1].double().numpy(),
                         lse_ref, "%s b%d h%d" % (w.name, b, h))


def test_decode_paged_full_size_sampled():
    """The decode workload over 16-row pages at shuffled pool positions, in the
    launch configuration bench.py --config 6 times: bit-identical to the
    contiguous call, and sampled (batch, head) rows against the oracle."""
    fa = _fa()
    w = wl.CFG[6]
    lens = w.lengths()
    say("generate %s" % w.name)
    q = wl.decode_query(w)
    kc = torch.empty((w.B, w.Nk, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    for b in range(w.B):
        L = int(lens[b])
        kc[b, :L].copy_(wl.decode_cache_rows(w, 1, b, L))
        vc[b, :L].copy_(wl.decode_cache_rows(w, 2, b, L))
        kc[b, L:min(w.Nk, L + 300)] = float("nan")
        vc[b, L:min(w.Nk, L + 300)] = float("nan")
    table, num_pages = wl.page_layout(w, w.page_size)
    bt = torch.from_numpy(table).cuda()
    pool = (num_pages, w.page_size, w.H, w.D)
    kp = torch.full(pool, float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    kp[bt.flatten().long()] = kc.view(-1, *pool[1:])
    vp[bt.flatten().long()] = vc.view(-1, *pool[1:])
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    say("fa_decode_splitkv_paged %s" % w.name)
    qd = q.cuda()
    dout = lambda: dict(out=nan_like(qd), lse=nan_like(qd, (w.B, w.H), torch.float32))
    o, lse = fa.decode_splitkv_paged(qd, kp, vp, sl, bt, scale=w.scale, chunk=w.chunk, **dout())
    say("fa_decode_splitkv (contiguous) %s" % w.name)
    oc, lc = fa.decode_splitkv(qd, kc, vc, sl, scale=w.scale, chunk=w.chunk, **dout())
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), oc.view(torch.int16)), "paged differs from contiguous"
    assert torch.equal(lse.view(torch.int32), lc.view(torch.int32))
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    del kc, vc, kp, vp
    rng = np.random.default_rng(1006)
    for b in sorted({0, w.B - 1} | {int(x) for x in rng.integers(0, w.B, 3)}):
        L = int(lens[b])
        kb = wl.to_f64(wl.decode_cache_rows(w, 1, b, L))
        vb = wl.to_f64(wl.decode_cache_rows(w, 2, b, L))
        for h in sorted({0, int(rng.integers(w.H))}):
            o_ref, lse_ref = oracle.attention_rows(wl.to_f64(q[b, h])[None], [0], kb[:, h], vb[:, h], 1,
                                                   L, w.scale, False)
            assert_close(w.dtype, wl.to_f64(o_c[b, h])[None], o_ref, lse_c[b, h:h + 1].double().numpy(),
                         lse_ref, "%s b%d h%d" % (w.name, b, h))


def test_bwd_full_size_heads():
    """Gradients of the N8192 causal prefill, in the launch configuration
    bench.py --config 9 times: two runs bit-identical, every gradient finite,
    and three whole (batch, head) slices against the oracle's backward."""
    fa = _fa()
    w = wl.CFG[9]
    say("generate %s" % w.name)
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("fa_fwd + fa_bwd %s" % w.name)
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=nan_like(qd),
                    lse=nan_like(qd, (w.B, w.H, w.Nq), torch.float32))
    g1 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, **nan_grads(qd, kd))
    g2 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, **nan_grads(qd, kd))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
        assert torch.isfinite(a).all().item()
    dq, dk, dv = (t.cpu() for t in g1)
    rng = np.random.default_rng(1009)
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        rq, rk, rv = oracle.attention_bwd(wl.to_f64(q[sl]), wl.to_f64(k[sl]), wl.to_f64(v[sl]),
                                          wl.to_f64(do[sl]), w.scale, w.causal)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert_grad_close(w.dtype, wl.to_f64(got[sl]), ref, "%s %s b%d h%d" % (w.name, name, b, h))


def test_dropout_full_size_sampled():
    """The N8192 causal prefill with dropout 0.1, in the launch configuration
    bench.py --config 10 times: bit-identical reruns, finite outputs, lse
    equal to the plain call's (dropout leaves the softmax statistics alone),
    and sampled rows against the oracle with the same keep decisions."""
    fa = _fa()
    w = wl.CFG[10]
    say("generate %s" % w.name)
    q, k, v = wl.prefill_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say("fa_fwd_dropout %s" % w.name)
    outs = lambda: dict(out=nan_like(qd), lse=nan_like(qd, (w.B, w.H, w.Nq), torch.float32))
    o, lse = fa.fwd_dropout(qd, kd, vd, dropout_p=w.dropout, seed=w.seed, causal=w.causal,
                            scale=w.scale, **outs())
    o2, lse2 = fa.fwd_dropout(qd, kd, vd, dropout_p=w.dropout, seed=w.seed, causal=w.causal,
                              scale=w.scale, **outs())
    _, lse0 = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, **outs())
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32)), "dropout changed lse"
    assert torch.isfinite(o).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    t = oracle.drop_threshold(float(np.float32(w.dropout)))
    ks = oracle.keep_scale(t)
    rng = np.random.default_rng(1010)
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]:
        rows = _sample_rows(rng, w.Nq)
        kb, vb = wl.to_f64(k[b, :, h]), wl.to_f64(v[b, :, h])
        keep = oracle.keep_mask(w.seed, b, h, rows, w.Nk, t)
        o_ref, lse_ref = oracle.attention_rows(wl.to_f64(q[b, rows, h]), rows, kb, vb, w.Nq, w.Nk,
                                               w.scale, w.causal, keep=keep, keep_scale=ks)
        assert_close(w.dtype, wl.to_f64(o_c[b, rows, h]) / ks, o_ref / ks,
                     lse_c[b, h, rows].double().numpy(), lse_ref, "%s b%d h%d" % (w.name, b, h))


def test_dropout_bwd_full_size_heads():
    """Gradients of the N8192 causal prefill with dropout 0.1 (bench.py
    --config 11): two runs bit-identical, finite, and two whole (batch, head)
    slices against the oracle's backward with the same keep decisions."""
    fa = _fa()
    w = wl.CFG[11]
    say("generate %s" % w.name)
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("fa_fwd_dropout + fa_bwd_dropout %s" % w.name)
    o, lse = fa.fwd_dropout(qd, kd, vd, dropout_p=w.dropout, seed=w.seed, causal=w.causal,
                            scale=w.scale, out=nan_like(qd),
                            lse=nan_like(qd, (w.B, w.H, w.Nq), torch.float32))
    g1 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dropout_p=w.dropout,
                seed=w.seed, **nan_grads(qd, kd))
    g2 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dropout_p=w.dropout,
                seed=w.seed, **nan_grads(qd, kd))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
        assert torch.isfinite(a).all().item()
    dq, dk, dv = (t.cpu() for t in g1)
    pf = float(np.float32(w.dropout))
    for b, h in [(0, 1), (1, 0)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        # the oracle numbers its slices from (0, 0): zero slices in front give
        # this one its true (b, h) for the keep counters
        pad = lambda x: np.concatenate([np.zeros((b,) + x.shape[1:]), x], 0) if b else x
        padh = lambda x: np.concatenate([np.zeros(x.shape[:2] + (h,) + x.shape[3:]), x], 2) if h else x
        args = [padh(pad(wl.to_f64(t[sl]))) for t in (q, k, v, do)]
        rq, rk, rv = oracle.attention_bwd(*args, w.scale, w.causal, dropout_p=pf, seed=w.seed)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert_grad_close(w.dtype, wl.to_f64(got[sl]), ref[b:b + 1, :, h:h + 1],
                              "%s %s b%d h%d" % (w.name, name, b, h))


LONG = [
    # (name, dtype, D, causal, B, H, Nq, Nk): long key loops, a ragged tail, many heads
    ("causal f16 D128 B1 H2 N65536", "f16", 128, True, 1, 2, 65536, 65536),
    ("bidirectional bf16 D64 B1 H1 Nq1000 Nk100003", "bf16", 64, False, 1, 1, 1000, 100003),
    ("causal bf16 D64 B2 H96 N515", "bf16", 64, True, 2, 96, 515, 515),
]


@pytest.mark.parametrize("case", LONG, ids=lambda c: c[0])
def test_prefill_long_and_wide_sampled(case):
    """Sizes beyond the benchmark table: sampled rows against the oracle,
    every output finite, two runs bit-identical."""
    name, dtype, D, causal, B, H, Nq, Nk = case
    fa = _fa()
    w = wl.Workload(name, "prefill", dtype, H=H, D=D, causal=causal, scale=1 / math.sqrt(D),
                    seed=77 + Nk, B=B, Nq=Nq, Nk=Nk)
    say("generate %s" % name)
    q, k, v = wl.prefill_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say("fa_fwd %s" % name)
    outs = lambda: dict(out=nan_like(qd), lse=nan_like(qd, (B, H, Nq), torch.float32))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=w.scale, **outs())
    o2, lse2 = fa.fwd(qd, kd, vd, causal=causal, scale=w.scale, **outs())
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    o_c, lse_c = o.cpu(), lse.cpu()
    rng = np.random.default_rng(2000 + Nk)
    pairs = sorted({(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))})
    for b, h in pairs:
        rows = _sample_rows(rng, Nq, extra=(Nq - 2, 4095, 4096, 32767, 32768))
        o_ref, lse_ref = oracle.attention_rows(wl.to_f64(q[b, rows, h]), rows, wl.to_f64(k[b, :, h]),
                                               wl.to_f64(v[b, :, h]), Nq, Nk, w.scale, causal)
        assert_close(dtype, wl.to_f64(o_c[b, rows, h]), o_ref, lse_c[b, h, rows].double().numpy(),
                     lse_ref, "%s b%d h%d" % (name, b, h))


@pytest.mark.parametrize("chunk", [128, 512])
def test_decode_long_cache_sampled(chunk):
    """Decode against caches of 131072 and 100001 keys (1024 / 256 chunks):
    contiguous and paged calls bit-identical, sampled heads against the oracle."""
    fa = _fa()
    B, H, D, Nk = 2, 8, 128, 131072
    lens = np.array([131072, 100001], dtype=np.int64)
    w = wl.Workload("decode long", "decode", "bf16", H=H, D=D, causal=False, scale=1 / math.sqrt(D),
                    seed=91, B=B, Nk=Nk, len_lo=1, len_hi=Nk, chunk=chunk, lens_fixed=list(lens))
    q = wl.decode_query(w)
    kc = torch.zeros((B, Nk, H, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b in range(B):
        L = int(lens[b])
        kc[b, :L].copy_(wl.decode_cache_rows(w, 1, b, L))
        vc[b, :L].copy_(wl.decode_cache_rows(w, 2, b, L))
        if L < Nk:
            kc[b, L:] = float("nan")
            vc[b, L:] = float("nan")
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    say("fa_decode_splitkv Lk %s chunk %d" % (lens.tolist(), chunk))
    qd = q.cuda()
    dout = lambda: dict(out=nan_like(qd), lse=nan_like(qd, (B, H), torch.float32))
    o, lse = fa.decode_splitkv(qd, kc, vc, sl, scale=w.scale, chunk=chunk, **dout())
    ps = 64
    table = torch.arange(B * (Nk // ps), dtype=torch.int32, device="cuda").view(B, Nk // ps)
    table = table.flip(1).contiguous()  # pages in reverse pool order
    kp = torch.empty((B * Nk // ps, ps, H, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp[table.flatten().long()] = kc.view(-1, ps, H, D)
    vp[table.flatten().long()] = vc.view(-1, ps, H, D)
    op, lp = fa.decode_splitkv_paged(qd, kp, vp, sl, table, scale=w.scale, chunk=chunk, **dout())
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    assert torch.equal(o.view(torch.int16), op.view(torch.int16)), "paged differs from contiguous"
    assert torch.equal(lse.view(torch.int32), lp.view(torch.int32))
    o_c, lse_c = o.cpu(), lse.cpu()
    del kc, vc, kp, vp
    for b in range(B):
        L = int(lens[b])
        kb = wl.to_f64(wl.decode_cache_rows(w, 1, b, L))
        vb = wl.to_f64(wl.decode_cache_rows(w, 2, b, L))
        for h in (0, H - 1):
            o_ref, lse_ref = oracle.attention_rows(wl.to_f64(q[b, h])[None], [0], kb[:, h], vb[:, h], 1,
                                                   L, w.scale, False)
            assert_close("bf16", wl.to_f64(o_c[b, h])[None], o_ref, lse_c[b, h:h + 1].double().numpy(),
                         lse_ref, "decode Lk%d chunk%d h%d" % (L, chunk, h))


@pytest.mark.parametrize("cfg", [12, 13])
def test_bwd_masked_full_size_heads(cfg):
    """Gradients of the N8192 causal prefill with the 2048-key prefix mask /
    with ALiBi (bench.py --config 12 / 13): reruns bit-identical, finite, and
    two whole (batch, head) slices against the oracle's masked backward."""
    fa = _fa()
    w = wl.CFG[cfg]
    say("generate %s" % w.name)
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    slopes = wl.alibi_slopes(w.H) if w.alibi else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("fa_fwd_masked + fa_bwd_masked %s" % w.name)
    o, lse = fa.fwd_masked(qd, kd, vd, causal=w.causal, scale=w.scale, prefix=w.prefix,
                           alibi_slopes=sd, out=nan_like(qd),
                           lse=nan_like(qd, (w.B, w.H, w.Nq), torch.float32))
    g1 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, prefix=w.prefix,
                alibi_slopes=sd, **nan_grads(qd, kd))
    g2 = fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, prefix=w.prefix,
                alibi_slopes=sd, **nan_grads(qd, kd))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
        assert torch.isfinite(a).all().item()
    dq, dk, dv = (t.cpu() for t in g1)
    for b, h in [(0, 0), (w.B - 1, w.H - 1)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        rq, rk, rv = oracle.attention_bwd(wl.to_f64(q[sl]), wl.to_f64(k[sl]), wl.to_f64(v[sl]),
                                          wl.to_f64(do[sl]), w.scale, w.causal, prefix=w.prefix,
                                          alibi_slopes=None if slopes is None else slopes[h:h + 1])
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert_grad_close(w.dtype, wl.to_f64(got[sl]), ref, "%s %s b%d h%d" % (w.name, name, b, h))


def test_bwd_varlen_full_size_sampled():
    """Gradients of the packed varlen workload (bench.py --config 14): reruns
    bit-identical, finite, and the shortest sequence (two heads) against the
    oracle's backward of that sequence alone."""
    fa = _fa()
    w = wl.CFG[14]
    say("generate %s" % w.name)
    q, k, v, cu = wl.varlen_inputs(w)
    do = wl.tensor(w, 3, tuple(q.shape))
    cud = torch.from_numpy(cu).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    lens = np.diff(cu)
    mx = int(lens.max())
    say("fa_fwd_varlen + fa_bwd_varlen %s" % w.name)
    o, lse = fa.fwd_varlen(qd, kd, vd, cud, cud, causal=True, scale=w.scale, out=nan_like(qd),
                           lse=nan_like(qd, (w.H, qd.shape[0]), torch.float32))
    g1 = fa.bwd_varlen(qd, kd, vd, o, lse, dod, cud, cud, causal=True, scale=w.scale, max_seqlen_q=mx,
                       max_seqlen_k=mx, **nan_grads(qd, kd))
    g2 = fa.bwd_varlen(qd, kd, vd, o, lse, dod, cud, cud, causal=True, scale=w.scale, max_seqlen_q=mx,
                       max_seqlen_k=mx, **nan_grads(qd, kd))
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
        assert torch.isfinite(a).all().item()
    dq, dk, dv = (t.cpu() for t in g1)
    s = int(np.argmin(lens))
    a0, a1 = int(cu[s]), int(cu[s + 1])
    for h in (0, w.H - 1):
        sl = (slice(a0, a1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_bwd(wl.to_f64(q[sl])[None], wl.to_f64(k[sl])[None],
                                          wl.to_f64(v[sl])[None], wl.to_f64(do[sl])[None], w.scale, True)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            assert_grad_close(w.dtype, wl.to_f64(got[sl]), ref[0], "%s %s seq%d h%d" % (w.name, name, s, h))
