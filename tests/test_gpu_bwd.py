"""GPU parity of the backward pass (fa_bwd through the C ABI) against the oracle.

The GPU backward consumes the GPU forward's o and lse (as a training step
would); the oracle recomputes everything from q, k, v and dO.  Outputs are
filled with NaN before each call, padding keys are NaN, and every case runs
twice and must be bit-identical.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import assert_grad_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def P(name, dtype, D, causal, B, H, Nq, Nk, seed, scale=None):
    return wl.Workload(name, "prefill", dtype, H=H, D=D, causal=causal,
                       scale=(1 / math.sqrt(D)) if scale is None else scale, seed=seed, B=B,
                       Nq=Nq, Nk=Nk)


def bwd_case(w, seqlens=None):
    import exact_tiled_attention_11_amd as fa
    fa.load()
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    say("  fa_fwd %s" % w.name)
    o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, seqlens_k=sl)
    outs = []
    for rep in range(2):
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        say("  fa_bwd %s rep %d" % (w.name, rep))
        fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, seqlens_k=sl, dq=dq,
               dk=dk, dv=dv)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
    dq, dk, dv = outs[0]
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            assert (dk[b, L:] == 0).all() and (dv[b, L:] == 0).all(), "padding keys get no gradient"
    if w.Nk == 1 and not w.causal:
        # One key: its probability is 1, so dS = dO.v - dO.o = 0 and the exact dQ
        # and dK are zero; the GPU's only error is the rounding of o to the
        # input dtype inside delta (relative 2^-8 per element) plus fp32 sums.
        k64, v64, do64 = wl.to_f64(k), wl.to_f64(v), wl.to_f64(do)
        bound = (w.scale * np.abs(k64).max() * np.abs(do64).sum(-1).max() * np.abs(v64).max()
                 * 2.0 ** -7)
        assert float(dq.abs().max()) <= bound and float(dk.abs().max()) <= bound, (
            float(dq.abs().max()), float(dk.abs().max()), bound)
        assert torch.equal(dv, do), "one key: dV = dO exactly"
        return
    rq, rk, rv = oracle.attention_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do),
                                      w.scale, w.causal, seqlens_k=seqlens)
    assert_grad_close(w.dtype, wl.to_f64(dq), rq, "%s dq" % w.name)
    assert_grad_close(w.dtype, wl.to_f64(dk), rk, "%s dk" % w.name)
    assert_grad_close(w.dtype, wl.to_f64(dv), rv, "%s dv" % w.name)


BWD = [
    (P("bf16 D64 causal B2 H3 N300", "bf16", 64, True, 2, 3, 300, 300, 51), None),
    (P("bf16 D64 noncausal B1 H2 Nq129 Nk200", "bf16", 64, False, 1, 2, 129, 200, 52), None),
    (P("f16 D128 causal B1 H2 N257", "f16", 128, True, 1, 2, 257, 257, 53), None),
    (P("bf16 D128 noncausal B2 H2 N160", "bf16", 128, False, 2, 2, 160, 160, 54), None),
    (P("bf16 D64 causal Nq100 Nk300", "bf16", 64, True, 1, 2, 100, 300, 55), None),
    (P("bf16 D64 causal Nq300 Nk100 (rows with no visible key)", "bf16", 64, True, 1, 2, 300, 100,
       56), None),
    (P("f16 D64 causal B2 H2 N300 padded keys", "f16", 64, True, 2, 2, 300, 300, 57), [300, 177]),
    (P("bf16 D128 noncausal B1 H1 Nq1 Nk1", "bf16", 128, False, 1, 1, 1, 1, 58), None),
    (P("f16 D64 causal B1 H4 N1000", "f16", 64, True, 1, 4, 1000, 1000, 59), None),
    # head_dim 128 runs the two-wave dK/dV kernel: ragged causal shapes, and padded keys that
    # leave whole 128-key workgroups past the sequence (no chunk to visit, zero rows to write)
    (P("bf16 D128 causal Nq100 Nk300", "bf16", 128, True, 1, 2, 100, 300, 151), None),
    (P("f16 D128 causal Nq300 Nk100 (rows with no visible key)", "f16", 128, True, 1, 2, 300, 100,
       152), None),
    (P("bf16 D128 causal B2 H2 N300 padded keys", "bf16", 128, True, 2, 2, 300, 300, 153), [300, 40]),
    (P("f16 D128 noncausal B2 H1 Nq70 Nk390 padded keys", "f16", 128, False, 2, 1, 70, 390, 154),
     [390, 129]),
    # B*H a multiple of 8: each XCD walks its (batch, head) pairs in groups of four (4+1, 4+2)
    (P("bf16 D64 causal B5 H8 N300 (pair groups 4+1)", "bf16", 64, True, 5, 8, 300, 300, 60), None),
    (P("f16 D128 causal B3 H16 N200 (pair groups 4+2)", "f16", 128, True, 3, 16, 200, 200, 155),
     None),
    # head_dim 64 runs the pipelined dQ kernel: its first and last steps at the edges of the key
    # range (one key; one query row against 32 key blocks; fewer keys than one block; a long query
    # range against two key blocks)
    (P("bf16 D64 noncausal B1 H1 Nq1 Nk1", "bf16", 64, False, 1, 1, 1, 1, 61), None),
    (P("bf16 D64 causal B1 H2 Nq1 Nk1000 (one query row)", "bf16", 64, True, 1, 2, 1, 1000, 62),
     None),
    (P("f16 D64 noncausal B1 H1 Nq40 Nk20 (keys short of one block)", "f16", 64, False, 1, 1, 40,
       20, 63), None),
    (P("bf16 D64 causal B1 H2 Nq2000 Nk33", "bf16", 64, True, 1, 2, 2000, 33, 64), None),
]


@pytest.mark.parametrize("w,seqlens", BWD, ids=lambda x: getattr(x, "name", str(x)))
def test_bwd(w, seqlens):
    bwd_case(w, seqlens)


def masked_bwd_case(w, prefix, alibi, seqlens=None):
    """fa_fwd_masked then fa_bwd_masked against the oracle's masked backward."""
    import exact_tiled_attention_11_amd as fa
    fa.load()
    q, k, v = wl.prefill_inputs(w)
    do = wl.tensor(w, 3, (w.B, w.Nq, w.H, w.D))
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    slopes = wl.alibi_slopes(w.H) if alibi else None
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("  fa_fwd_masked + fa_bwd_masked %s prefix %d alibi %s" % (w.name, prefix, alibi))
    o, lse = fa.fwd_masked(qd, kd, vd, causal=w.causal, scale=w.scale, seqlens_k=sl, prefix=prefix,
                           alibi_slopes=sd)
    outs = []
    for rep in range(2):
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        fa.bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, seqlens_k=sl, prefix=prefix,
               alibi_slopes=sd, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
    dq, dk, dv = outs[0]
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            assert (dk[b, L:] == 0).all() and (dv[b, L:] == 0).all(), "padding keys get no gradient"
    rq, rk, rv = oracle.attention_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do),
                                      w.scale, w.causal, seqlens_k=seqlens, prefix=prefix,
                                      alibi_slopes=slopes)
    tag = "%s prefix %d alibi %s" % (w.name, prefix, alibi)
    assert_grad_close(w.dtype, wl.to_f64(dq), rq, "%s dq" % tag)
    assert_grad_close(w.dtype, wl.to_f64(dk), rk, "%s dk" % tag)
    assert_grad_close(w.dtype, wl.to_f64(dv), rv, "%s dv" % tag)


MASKED_BWD = [
    (P("bf16 D64 causal B2 H3 N300", "bf16", 64, True, 2, 3, 300, 300, 61), 37, False, None),
    (P("bf16 D64 causal Nq100 Nk300", "bf16", 64, True, 1, 2, 100, 300, 62), 150, False, None),
    (P("bf16 D64 causal Nq300 Nk100", "bf16", 64, True, 1, 2, 300, 100, 63), 20, False, None),
    (P("bf16 D64 causal B2 H4 N300 ALiBi", "bf16", 64, True, 2, 4, 300, 300, 64), 0, True, None),
    (P("bf16 D64 bidirectional Nq129 Nk200 ALiBi", "bf16", 64, False, 1, 4, 129, 200, 65), 0, True, None),
    (P("f16 D128 causal N257 prefix+ALiBi", "f16", 128, True, 1, 2, 257, 257, 66), 64, True, None),
    (P("f16 D64 causal B2 H2 N300 padded, prefix", "f16", 64, True, 2, 2, 300, 300, 67), 200,
     False, [300, 177]),
    (P("bf16 D128 causal B2 H2 N300 padded, prefix", "bf16", 128, True, 2, 2, 300, 300, 68), 200,
     False, [300, 177]),
    (P("bf16 D128 causal Nq300 Nk100 ALiBi", "bf16", 128, True, 1, 3, 300, 100, 69), 0, True, None),
]


@pytest.mark.parametrize("w,prefix,alibi,seqlens", MASKED_BWD,
                         ids=lambda x: getattr(x, "name", str(x)))
def test_bwd_masked(w, prefix, alibi, seqlens):
    masked_bwd_case(w, prefix, alibi, seqlens)


def varlen_bwd_case(name, dtype, D, H, causal, lens_q, lens_k, seed):
    """fa_fwd_varlen then fa_bwd_varlen against the oracle's packed backward."""
    import exact_tiled_attention_11_amd as fa
    fa.load()
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    w = wl.Workload(name, "varlen", dtype, H=H, D=D, causal=causal, scale=1 / math.sqrt(D), seed=seed)
    q = wl.tensor(w, 0, (int(cu_q[-1]), H, D))
    k = wl.tensor(w, 1, (int(cu_k[-1]), H, D))
    v = wl.tensor(w, 2, (int(cu_k[-1]), H, D))
    do = wl.tensor(w, 3, (int(cu_q[-1]), H, D))
    cqd, ckd = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("  fa_fwd_varlen + fa_bwd_varlen %s" % name)
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, causal=causal, scale=w.scale)
    outs = []
    for rep in range(2):
        dq = torch.full_like(qd, float("nan"))
        dk = torch.full_like(kd, float("nan"))
        dv = torch.full_like(vd, float("nan"))
        fa.bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, causal=causal, scale=w.scale,
                      max_seqlen_q=int(max(lens_q)), max_seqlen_k=int(max(lens_k)), dq=dq, dk=dk,
                      dv=dv)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run difference"
    dq, dk, dv = outs[0]
    rq, rk, rv = oracle.attention_varlen_bwd(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), wl.to_f64(do),
                                             cu_q, cu_k, w.scale, causal)
    assert_grad_close(dtype, wl.to_f64(dq), rq, "%s dq" % name)
    assert_grad_close(dtype, wl.to_f64(dk), rk, "%s dk" % name)
    assert_grad_close(dtype, wl.to_f64(dv), rv, "%s dv" % name)


VARLEN_BWD = [
    ("f16 D128 causal H2 5 seqs (one empty)", "f16", 128, 2, True, [300, 0, 129, 1, 450],
     [300, 0, 129, 1, 450], 71),
    ("bf16 D64 causal H3 Lq != Lk", "bf16", 64, 3, True, [100, 260, 33], [300, 130, 33], 72),
    ("bf16 D64 bidirectional H2 Lq != Lk", "bf16", 64, 2, False, [64, 200, 5], [190, 7, 128], 73),
    ("f16 D64 causal H4 8 short seqs", "f16", 64, 4, True, [17, 31, 32, 33, 63, 64, 65, 2],
     [17, 31, 32, 33, 63, 64, 65, 2], 74),
    ("bf16 D128 causal H2 Lq != Lk", "bf16", 128, 2, True, [100, 260, 33], [300, 130, 33], 75),
    ("f16 D128 bidirectional H2 Lq != Lk", "f16", 128, 2, False, [64, 200, 5], [190, 7, 128], 76),
]


@pytest.mark.parametrize("case", VARLEN_BWD, ids=lambda c: c[0])
def test_bwd_varlen(case):
    varlen_bwd_case(*case)
