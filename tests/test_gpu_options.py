"""GPU parity of the options together and on packed batches: the prefix
mask, ALiBi and attention dropout through fa_fwd_varlen_masked / _dropout /
_ex, fa_bwd_varlen_masked / _dropout / _ex, fa_fwd_ex and fa_bwd_ex, against
the oracle.

* Outputs and log-sum-exp against ``oracle.attention_varlen`` with the same
  options; gradients against ``oracle.attention_varlen_bwd``.  Ragged
  lengths, an empty sequence, Lq != Lk, both head dims, both dtypes.
* Packing: equal-length sequences packed end to end give the fixed-length
  entry points' results bit for bit (same tiles, the sequence index in the
  batch index's place in the dropout counters).
* Every call runs twice and must be bit-identical.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import LSE_TOL, TOL, assert_close, assert_grad_close, errors

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _fa():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    return fa


def _inputs(name, dtype, D, H, lens_q, lens_k, seed):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    w = wl.Workload(name, "varlen", dtype, H=H, D=D, causal=True, scale=1 / math.sqrt(D), seed=seed)
    q = wl.tensor(w, 0, (int(cu_q[-1]), H, D))
    k = wl.tensor(w, 1, (int(cu_k[-1]), H, D))
    v = wl.tensor(w, 2, (int(cu_k[-1]), H, D))
    do = wl.tensor(w, 3, (int(cu_q[-1]), H, D))
    return w, q, k, v, do, cu_q, cu_k


CASES = [
    # name, dtype, D, H, causal, lens_q, lens_k, options
    ("bf16 D64 causal prefix 40", "bf16", 64, 3, True, [100, 260, 33, 0], [100, 260, 33, 0],
     dict(prefix=40)),
    ("f16 D128 causal ALiBi Lq != Lk", "f16", 128, 2, True, [100, 260, 33], [300, 130, 33],
     dict(alibi=True)),
    ("bf16 D64 bidirectional ALiBi", "bf16", 64, 4, False, [64, 200, 5], [190, 7, 128],
     dict(alibi=True)),
    ("bf16 D128 causal prefix+ALiBi", "bf16", 128, 2, True, [300, 129, 1], [300, 129, 1],
     dict(prefix=100, alibi=True)),
    ("f16 D64 causal dropout 0.2", "f16", 64, 3, True, [100, 260, 0, 33], [100, 260, 0, 33],
     dict(dropout=0.2)),
    ("bf16 D128 causal dropout 0.3 Lq != Lk", "bf16", 128, 2, True, [100, 260, 33],
     [300, 130, 33], dict(dropout=0.3)),
    ("bf16 D64 bidirectional dropout 0.5", "bf16", 64, 2, False, [64, 200, 5], [190, 7, 128],
     dict(dropout=0.5)),
    ("bf16 D64 causal prefix+ALiBi+dropout", "bf16", 64, 3, True, [100, 260, 0, 33],
     [100, 260, 0, 33], dict(prefix=40, alibi=True, dropout=0.2)),
    ("f16 D128 causal ALiBi+dropout Lq != Lk", "f16", 128, 2, True, [100, 260, 33],
     [300, 130, 33], dict(alibi=True, dropout=0.3)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_forward_and_gradients(case):
    name, dtype, D, H, causal, lens_q, lens_k, opt = case
    fa = _fa()
    w, q, k, v, do, cu_q, cu_k = _inputs(name, dtype, D, H, lens_q, lens_k, 500 + len(name))
    slopes = wl.alibi_slopes(H) if opt.get("alibi") else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    prefix = opt.get("prefix", 0)
    p = float(np.float32(opt.get("dropout", 0.0)))
    seed = 7000 + len(name)
    kw = dict(prefix=prefix, alibi_slopes=sd, dropout_p=p, seed=seed)
    cqd, ckd = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    mq, mk = int(max(lens_q)), int(max(lens_k))
    outs = []
    for rep in range(2):
        say("  varlen %s rep %d" % (name, rep))
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((H, qd.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        fa.fwd_varlen(qd, kd, vd, cqd, ckd, causal=causal, scale=w.scale, out=o, lse=lse, **kw)
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        fa.bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, causal=causal, scale=w.scale,
                      max_seqlen_q=mq, max_seqlen_k=mk, dq=dq, dk=dk, dv=dv, **kw)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "run-to-run difference"
    o, lse, dq, dk, dv = outs[0]
    okw = dict(prefix=prefix, alibi_slopes=slopes, dropout_p=p, seed=seed)
    o_ref, lse_ref = oracle.attention_varlen(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), cu_q, cu_k,
                                             w.scale, causal, **okw)
    ks = oracle.keep_scale(oracle.drop_threshold(p)) if p else 1.0
    assert_close(dtype, wl.to_f64(o) / ks, o_ref / ks, lse.double().numpy(), lse_ref, name)
    rq, rk, rv = oracle.attention_varlen_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v),
                                             wl.to_f64(do), cu_q, cu_k, w.scale, causal, **okw)
    assert_grad_close(dtype, wl.to_f64(dq), rq, "%s dq" % name)
    assert_grad_close(dtype, wl.to_f64(dk), rk, "%s dk" % name)
    assert_grad_close(dtype, wl.to_f64(dv), rv, "%s dv" % name)


@pytest.mark.parametrize("opt", [dict(prefix=50), dict(alibi=True), dict(dropout=0.25),
                                 dict(prefix=50, alibi=True, dropout=0.25)],
                         ids=["prefix", "alibi", "dropout", "all"])
@pytest.mark.parametrize("D", [64, 128])
def test_equal_lengths_match_the_fixed_length_entry_points(opt, D):
    fa = _fa()
    B, L, H = 3, 300, 2
    w = wl.Workload("pack", "prefill", "bf16", H=H, D=D, causal=True, scale=1 / math.sqrt(D),
                    seed=900 + D, B=B, Nq=L, Nk=L)
    q, k, v = (t.cuda() for t in wl.prefill_inputs(w))
    do = wl.tensor(w, 3, (B, L, H, D)).cuda()
    sd = torch.from_numpy(wl.alibi_slopes(H)).cuda() if opt.get("alibi") else None
    p = float(np.float32(opt.get("dropout", 0.0)))
    prefix = opt.get("prefix", 0)
    say("  packing %s D%d" % (sorted(opt), D))
    of, lf = fa.fwd_ex(q, k, v, causal=True, scale=w.scale, prefix=prefix, alibi_slopes=sd,
                       dropout_p=p, seed=77)
    gf = fa.bwd(q, k, v, of, lf, do, causal=True, scale=w.scale, prefix=prefix, alibi_slopes=sd,
                dropout_p=p, seed=77)
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda") * L
    pk = lambda t: t.reshape(B * L, H, D)
    ov, lv = fa.fwd_varlen(pk(q), pk(k), pk(v), cu, cu, causal=True, scale=w.scale, prefix=prefix,
                           alibi_slopes=sd, dropout_p=p, seed=77)
    gv = fa.bwd_varlen(pk(q), pk(k), pk(v), ov, lv, pk(do), cu, cu, causal=True, scale=w.scale,
                       prefix=prefix, alibi_slopes=sd, dropout_p=p, seed=77)
    torch.cuda.synchronize()
    assert torch.equal(pk(of).view(torch.int16), ov.view(torch.int16))
    assert torch.equal(lf.permute(1, 0, 2).reshape(H, B * L).contiguous().view(torch.int32),
                       lv.view(torch.int32))
    for a, b in zip(gf, gv):
        assert torch.equal(pk(a).view(torch.int16), b.view(torch.int16))


FIXED = [
    # name, dtype, D, causal, B, H, Nq, Nk, seqlens, options
    ("bf16 D64 causal prefix+ALiBi+dropout", "bf16", 64, True, 2, 3, 300, 300, None,
     dict(prefix=70, alibi=True, dropout=0.2)),
    ("f16 D128 causal ALiBi+dropout Nq300 Nk100", "f16", 128, True, 1, 2, 300, 100, None,
     dict(alibi=True, dropout=0.3)),
    ("bf16 D64 bidirectional ALiBi+dropout padded keys", "bf16", 64, False, 2, 2, 200, 333,
     [333, 129], dict(alibi=True, dropout=0.4)),
    ("bf16 D128 causal prefix+dropout", "bf16", 128, True, 2, 2, 257, 257, None,
     dict(prefix=100, dropout=0.25)),
]


@pytest.mark.parametrize("case", FIXED, ids=lambda c: c[0])
def test_fixed_length_every_option(case):
    """fa_fwd_ex and fa_bwd_ex (the options together) against the oracle."""
    name, dtype, D, causal, B, H, Nq, Nk, seqlens, opt = case
    fa = _fa()
    w = wl.Workload(name, "prefill", dtype, H=H, D=D, causal=causal, scale=1 / math.sqrt(D),
                    seed=300 + len(name), B=B, Nq=Nq, Nk=Nk)
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (B, Nq, H, D))
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    slopes = wl.alibi_slopes(H) if opt.get("alibi") else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    prefix = opt.get("prefix", 0)
    p = float(np.float32(opt.get("dropout", 0.0)))
    seed = 5000 + len(name)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    outs = []
    for rep in range(2):
        say("  fa_fwd_ex + fa_bwd_ex %s rep %d" % (name, rep))
        o, lse = fa.fwd_ex(qd, kd, vd, causal=causal, scale=w.scale, seqlens_k=sl, prefix=prefix,
                           alibi_slopes=sd, dropout_p=p, seed=seed)
        g = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=w.scale, seqlens_k=sl,
                   prefix=prefix, alibi_slopes=sd, dropout_p=p, seed=seed)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (o, lse, *g)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "run-to-run difference"
    o, lse, dq, dk, dv = outs[0]
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            assert (dk[b, L:] == 0).all() and (dv[b, L:] == 0).all()
    o_ref, lse_ref = oracle.attention_dropout(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), w.scale,
                                              causal, p, seed, seqlens_k=seqlens, prefix=prefix,
                                              alibi_slopes=slopes)
    ks = oracle.keep_scale(oracle.drop_threshold(p))
    assert_close(dtype, wl.to_f64(o) / ks, o_ref / ks, lse.double().numpy(), lse_ref, name)
    rq, rk, rv = oracle.attention_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do),
                                      w.scale, causal, seqlens_k=seqlens, dropout_p=p, seed=seed,
                                      prefix=prefix, alibi_slopes=slopes)
    assert_grad_close(dtype, wl.to_f64(dq), rq, "%s dq" % name)
    assert_grad_close(dtype, wl.to_f64(dk), rk, "%s dk" % name)
    assert_grad_close(dtype, wl.to_f64(dv), rv, "%s dv" % name)


# Rows whose running maximum keeps rising or whose scores are large, so that
# the bf16 prefill raises its exponent offset many times and lets it lag
# behind the maximum by up to its bound (block sums below 2^60) or, with
# ALiBi, places it ahead of the maximum by its lead: steep slopes over 2048
# keys (the bias climbs up to 46 log2 units per 32-key block), inputs scaled
# by 2.5 (scores with a standard deviation of about 9 log2 units), and both.
SETTLE = [
    # name, slopes, input scale
    ("bf16 D64 causal N2048 steep ALiBi", [1.0, 0.25], 1.0),
    ("bf16 D64 causal N2048 large scores", None, 2.5),
    ("bf16 D64 causal N2048 steep ALiBi large scores", [0.7, 0.05], 2.5),
]


@pytest.mark.parametrize("case", SETTLE, ids=lambda c: c[0])
def test_bf16_offset_settles(case):
    """fa_fwd / fa_fwd_masked against the oracle where the lazy offset settles often."""
    name, slopes, amp = case
    fa = _fa()
    H, N = 2, 2048
    w = wl.Workload(name, "prefill", "bf16", H=H, D=64, causal=True, scale=1 / 8,
                    seed=900 + len(name), B=1, Nq=N, Nk=N, value_scale=amp)
    q, k, v = wl.prefill_inputs(w)
    sl = None if slopes is None else np.asarray(slopes, dtype=np.float32)
    sd = None if sl is None else torch.from_numpy(sl).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say("  %s" % name)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((1, H, N), float("nan"), dtype=torch.float32, device="cuda")
    if sd is None:
        fa.fwd(qd, kd, vd, causal=True, scale=w.scale, out=o, lse=lse)
    else:
        fa.fwd_masked(qd, kd, vd, causal=True, scale=w.scale, alibi_slopes=sd, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), w.scale, True,
                                      alibi_slopes=sl)
    # O scales with the inputs, and its rounding with it.  Such rows are
    # peaked (|O| up to about 4.5 after the division), where a bf16 output's
    # own spacing is 2^-6, so O is held element-wise to 2^-6 of max(|O|, 1)
    # (two ulps at the bottom of a binade; the builds before and after the
    # settle rules measured 0.0071 - 0.0084) instead of the absolute bound
    # meant for |O| < 1; the relative RMS and lse bounds are the standard ones.
    og, orf = wl.to_f64(o.cpu()) / amp, o_ref / amp
    e = errors(og, orf, lse.cpu().double().numpy(), lse_ref)
    elem = float(np.max(np.abs(og - orf) / np.maximum(np.abs(orf), 1.0)))
    msg = "%s: %s, element-wise %.5f" % (name, e, elem)
    assert e["nonfinite"] == 0, msg
    assert elem <= 2.0 ** -6, msg
    assert e["rel_rms"] <= TOL["bf16"]["rel_rms"], msg
    assert e["lse_inf_mismatch"] == 0 and e["lse_max_abs"] <= LSE_TOL, msg
