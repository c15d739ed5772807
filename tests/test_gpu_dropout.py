"""GPU parity of attention dropout (fa_fwd_dropout, fa_bwd_dropout) against the oracle.

* Keep decisions, bit-exact: with V = one-hot rows (V_j = e_j, Nk <= D) the
  output is O[i, j] = P_ij * Z_ij, so its zero pattern is exactly the
  kernel's keep mask, compared with the oracle's Philox-based mask.
* Outputs and gradients against ``oracle.attention_dropout`` and
  ``oracle.attention_bwd(..., dropout_p, seed)`` on ragged shapes, both
  causal alignments, padded keys and several probabilities.
* p = 0 equals the plain entry points bit for bit; a call repeated with the
  same seed is bit-identical, another seed changes the output.
"""

import math

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


def W(name, dtype, D, causal, B, H, Nq, Nk, seed):
    return wl.Workload(name, "prefill", dtype, H=H, D=D, causal=causal, scale=1 / math.sqrt(D),
                       seed=seed, B=B, Nq=Nq, Nk=Nk)


def _f32(p):
    """The probability as the C ABI receives it (a float)."""
    return float(np.float32(p))


@pytest.mark.parametrize("causal,Nk,D,p,seed", [
    (False, 100, 128, 0.5, 1),
    (True, 100, 128, 0.25, 2),
    (False, 64, 64, 0.9, 0xFEEDFACECAFEBEEF),
    (True, 37, 64, 0.1, 3),
])
def test_keep_mask_bit_exact(causal, Nk, D, p, seed):
    fa = _fa()
    B, H, Nq = 2, 3, 300
    w = W("mask", "bf16", D, causal, B, H, Nq, Nk, 70 + Nk)
    q, k, _ = wl.prefill_inputs(w)
    q = (q.float() * 0.25).to(torch.bfloat16)  # small scores: every probability well above 0
    v = torch.zeros((B, Nk, H, D), dtype=torch.bfloat16)
    for j in range(Nk):
        v[:, j, :, j] = 1.0
    say("  fa_fwd_dropout one-hot V causal=%s Nk=%d D=%d p=%g" % (causal, Nk, D, p))
    o, _ = fa.fwd_dropout(q.cuda(), k.cuda(), v.cuda(), dropout_p=_f32(p), seed=seed, causal=causal)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    t = oracle.drop_threshold(_f32(p))
    vis = oracle.visible(np.arange(Nq), Nq, Nk, causal)
    for b in range(B):
        for h in range(H):
            keep = oracle.keep_mask(seed, b, h, np.arange(Nq), Nk, t)
            got = o[:, :, :, :Nk][b, :, h] != 0
            want = keep & vis
            bad = np.argwhere(got != want)
            assert bad.size == 0, "b%d h%d: %d keep decisions differ, first %s" % (
                b, h, len(bad), bad[:5].tolist())


FWD = [
    (W("bf16 D64 causal B2 H3 N300", "bf16", 64, True, 2, 3, 300, 300, 81), None, 0.1),
    (W("bf16 D64 noncausal Nq129 Nk200", "bf16", 64, False, 1, 2, 129, 200, 82), None, 0.5),
    (W("f16 D128 causal N257", "f16", 128, True, 1, 2, 257, 257, 83), None, 0.25),
    (W("bf16 D128 noncausal B2 H2 N160", "bf16", 128, False, 2, 2, 160, 160, 84), None, 0.9),
    (W("bf16 D64 causal Nq300 Nk100", "bf16", 64, True, 1, 2, 300, 100, 85), None, 0.3),
    (W("f16 D64 causal B2 H2 N300 padded keys", "f16", 64, True, 2, 2, 300, 300, 86), [300, 177], 0.2),
    (W("bf16 D128 causal Nq300 Nk100", "bf16", 128, True, 1, 2, 300, 100, 87), None, 0.3),
    (W("f16 D128 causal B2 H2 N300 padded keys", "f16", 128, True, 2, 2, 300, 300, 89), [300, 40], 0.2),
]


def _inputs(w, seqlens):
    q, k, v = wl.prefill_inputs(w)
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    return q, k, v, sl


@pytest.mark.parametrize("w,seqlens,p", FWD, ids=lambda x: getattr(x, "name", str(x)))
def test_fwd_dropout_parity(w, seqlens, p):
    fa = _fa()
    q, k, v, sl = _inputs(w, seqlens)
    seed = 1000 + w.seed
    pf = _f32(p)
    say("  fa_fwd_dropout %s p=%g" % (w.name, p))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = fa.fwd_dropout(qd, kd, vd, dropout_p=pf, seed=seed, causal=w.causal, scale=w.scale,
                            seqlens_k=sl)
    o2, lse2 = fa.fwd_dropout(qd, kd, vd, dropout_p=pf, seed=seed, causal=w.causal, scale=w.scale,
                              seqlens_k=sl)
    o3, _ = fa.fwd_dropout(qd, kd, vd, dropout_p=pf, seed=seed + 1, causal=w.causal,
                           scale=w.scale, seqlens_k=sl)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert not torch.equal(o, o3), "another seed must change the output"
    o_ref, lse_ref = oracle.attention_dropout(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), w.scale,
                                              w.causal, pf, seed, seqlens_k=seqlens)
    # kept weights are scaled by 256/(256 - t): the output and its rounding grow with it
    ks = oracle.keep_scale(oracle.drop_threshold(pf))
    assert_close(w.dtype, wl.to_f64(o.cpu()) / ks, o_ref / ks, lse.cpu().double().numpy(), lse_ref,
                 "%s p=%g" % (w.name, p))


@pytest.mark.parametrize("w,seqlens,p", FWD, ids=lambda x: getattr(x, "name", str(x)))
def test_bwd_dropout_parity(w, seqlens, p):
    fa = _fa()
    q, k, v, sl = _inputs(w, seqlens)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    seed = 2000 + w.seed
    pf = _f32(p)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("  fa_fwd_dropout + fa_bwd_dropout %s p=%g" % (w.name, p))
    o, lse = fa.fwd_dropout(qd, kd, vd, dropout_p=pf, seed=seed, causal=w.causal, scale=w.scale,
                            seqlens_k=sl)
    outs = []
    for rep in range(2):
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, seqlens_k=sl, dropout_p=pf,
               seed=seed, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
    dq, dk, dv = outs[0]
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            assert (dk[b, L:] == 0).all() and (dv[b, L:] == 0).all()
    rq, rk, rv = oracle.attention_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do),
                                      w.scale, w.causal, seqlens_k=seqlens, dropout_p=pf, seed=seed)
    assert_grad_close(w.dtype, wl.to_f64(dq), rq, "%s dq p=%g" % (w.name, p))
    assert_grad_close(w.dtype, wl.to_f64(dk), rk, "%s dk p=%g" % (w.name, p))
    assert_grad_close(w.dtype, wl.to_f64(dv), rv, "%s dv p=%g" % (w.name, p))


def test_p_zero_matches_plain_entry_points():
    fa = _fa()
    w = W("bf16 D64 causal B1 H2 N200", "bf16", 64, True, 1, 2, 200, 200, 88)
    q, k, v = (t.cuda() for t in wl.prefill_inputs(w))
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D)).cuda()
    o0, l0 = fa.fwd(q, k, v, causal=True)
    o1, l1 = fa.fwd_dropout(q, k, v, dropout_p=0.0, seed=5, causal=True)
    g0 = fa.bwd(q, k, v, o0, l0, do, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq), dtype=torch.uint8, device="cuda")
    g1 = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    st = fa.fa_bwd_dropout(*(t.data_ptr() for t in (q, k, v, o0, l0, do, *g1)), w.B, w.H, w.Nq,
                           w.Nk, w.D, w.scale, 1, None, 0.0, 5, ws.data_ptr(), ws.numel(),
                           fa.FA_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
