"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Each case prints what it runs before touching the GPU.  Outputs are filled
with NaN before every call (an unwritten element shows up as non-finite),
padding keys are filled with NaN (a masked key that leaks into the result
shows up too), and every case is run twice and required to be bit-identical.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import assert_close

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _fa():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    return fa


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def prefill_case(w, seqlens=None, q_mul=1.0):
    fa = _fa()
    q, k, v = wl.prefill_inputs(w)
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(q.dtype)
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    outs = []
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H, w.Nq), float("nan"), dtype=torch.float32, device="cuda")
        say("  fa_fwd %s rep %d" % (w.name, rep))
        fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale, seqlens_k=sl, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.uint8) if o1.dtype != torch.float32 else o1.view(torch.int32),
                       o2.view(torch.uint8) if o2.dtype != torch.float32 else o2.view(torch.int32)), \
        "run-to-run difference"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse run-to-run difference"
    o_ref, lse_ref = oracle.attention(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), w.scale, w.causal,
                                      seqlens_k=seqlens)
    return assert_close(w.dtype, wl.to_f64(o1), o_ref, l1.double().numpy(), lse_ref, w.name)


def P(name, dtype, D, causal, B, H, Nq, Nk, scale=None, seed=1):
    return wl.Workload(name, "prefill", dtype, H=H, D=D, causal=causal,
                       scale=(1 / math.sqrt(D)) if scale is None else scale, seed=seed, B=B,
                       Nq=Nq, Nk=Nk)


PREFILL = [
    wl.SMALL[1],  # the full fp32 causal workload
    wl.SMALL[2],
    wl.SMALL[3],
    P("bf16 D128 causal B2 H3 N300", "bf16", 128, True, 2, 3, 300, 300),
    P("bf16 D128 noncausal B1 H2 N129", "bf16", 128, False, 1, 2, 129, 129),
    P("f16 D64 causal B1 H3 N513", "f16", 64, True, 1, 3, 513, 513),
    P("f16 D128 noncausal B2 H2 N200", "f16", 128, False, 2, 2, 200, 200),
    P("f32 D128 causal B1 H2 N150", "f32", 128, True, 1, 2, 150, 150),
    P("f32 D64 noncausal B1 H2 Nq70 Nk33", "f32", 64, False, 1, 2, 70, 33),
    # fp32 at head_dim 64 splits each 128-key tile over the four waves of a
    # 32-row workgroup and merges their partial results: rows with no visible
    # key, waves whose key block lies past the end, several tiles per row block
    P("f32 D64 causal Nq300 Nk100 (empty rows)", "f32", 64, True, 1, 2, 300, 100),
    P("f32 D64 causal B2 Nq100 Nk300", "f32", 64, True, 2, 2, 100, 300),
    P("f32 D64 noncausal Nq33 Nk700", "f32", 64, False, 1, 3, 33, 700),
    P("bf16 D64 N1", "bf16", 64, True, 1, 1, 1, 1),
    P("bf16 D64 Nq1 Nk1000 noncausal", "bf16", 64, False, 2, 2, 1, 1000),
    P("bf16 D64 causal Nq1 Nk300 (bottom-right)", "bf16", 64, True, 1, 2, 1, 300),
    P("bf16 D64 causal Nq300 Nk100 (empty rows)", "bf16", 64, True, 1, 2, 300, 100),
    P("bf16 D64 causal Nq100 Nk300", "bf16", 64, True, 2, 2, 100, 300),
    P("bf16 D64 causal N257", "bf16", 64, True, 1, 1, 257, 257),
    P("bf16 D64 causal N255", "bf16", 64, True, 1, 1, 255, 255),
    P("bf16 D64 noncausal Nk63", "bf16", 64, False, 1, 2, 64, 63),
    P("bf16 D64 noncausal Nk65", "bf16", 64, False, 1, 2, 64, 65),
    P("bf16 D64 scale 0", "bf16", 64, True, 1, 2, 100, 100, scale=0.0),
    P("bf16 D64 Nk0", "bf16", 64, False, 1, 2, 40, 0),
    # B*H a multiple of 8: each XCD walks its (batch, head) pairs in groups of
    # four, here four then one (40 pairs) and four then two (48)
    P("bf16 D64 causal B5 H8 N300 (pair groups 4+1)", "bf16", 64, True, 5, 8, 300, 300),
    P("f16 D128 causal B3 H16 N200 (pair groups 4+2)", "f16", 128, True, 3, 16, 200, 200),
]


@pytest.mark.parametrize("w", PREFILL, ids=lambda w: w.name)
def test_prefill(w):
    prefill_case(w)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 128), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_key_padding(dtype, D, causal):
    w = P("pad %s D%d causal=%d" % (dtype, D, causal), dtype, D, causal, 3, 2, 300, 333)
    prefill_case(w, seqlens=[333, 0, 129])


def test_prefill_large_scores_fp16():
    """Scores far beyond fp16's exp range: the safe softmax keeps them exact."""
    w = P("f16 D64 q x 8", "f16", 64, True, 1, 2, 300, 300)
    prefill_case(w, q_mul=8.0)


def varlen_case(w):
    fa = _fa()
    q, k, v, cu = wl.varlen_inputs(w)
    cud = torch.from_numpy(cu).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    outs = []
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((w.H, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        say("  fa_fwd_varlen %s rep %d" % (w.name, rep))
        fa.fwd_varlen(qd, kd, vd, cud, cud, causal=w.causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    o_ref, lse_ref = oracle.attention_varlen(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), cu, cu,
                                             w.scale, w.causal)
    return assert_close(w.dtype, wl.to_f64(outs[0][0]), o_ref, outs[0][1].double().numpy(),
                        lse_ref, w.name)


VARLEN = [
    wl.SMALL[4],
    dataclasses.replace(wl.SMALL[4], name="varlen noncausal bf16 D64 7 seqs", dtype="bf16",
                        D=64, causal=False, nseq=7, seed=11),
    dataclasses.replace(wl.SMALL[4], name="varlen with empty sequences", seed=12,
                        lens_fixed=[0, 5, 0, 300, 1, 129, 0]),
    dataclasses.replace(wl.SMALL[4], name="varlen f32 D64 causal", dtype="f32", D=64, seed=13,
                        nseq=3),
    # more sequences than the schedule kernel's threads: its tile-offset scan
    # runs over three chunks of sequences, some of them empty
    dataclasses.replace(wl.SMALL[4], name="varlen 2500 short sequences", dtype="bf16", D=64, H=2,
                        nseq=2500, len_lo=0, len_hi=40, seed=14),
    # head counts divisible by 8 take the XCD-grouped order of the packed grid
    dataclasses.replace(wl.SMALL[4], name="varlen causal bf16 D64 H8 5 seqs", dtype="bf16", D=64,
                        H=8, nseq=5, len_lo=1, len_hi=400, seed=15),
    dataclasses.replace(wl.SMALL[4], name="varlen noncausal f16 D128 H16 4 seqs", dtype="f16",
                        D=128, H=16, causal=False, nseq=4, len_lo=1, len_hi=300, seed=16),
    dataclasses.replace(wl.SMALL[4], name="varlen causal f16 D128 H16 3 seqs", dtype="f16",
                        D=128, H=16, nseq=3, len_lo=100, len_hi=500, seed=17),
    dataclasses.replace(wl.SMALL[4], name="varlen noncausal bf16 D64 H8 6 seqs", dtype="bf16",
                        D=64, H=8, causal=False, nseq=6, len_lo=0, len_hi=350, seed=18),
    dataclasses.replace(wl.SMALL[4], name="varlen 1100 short sequences H8", dtype="bf16", D=64,
                        H=8, nseq=1100, len_lo=0, len_hi=40, seed=19),
]


@pytest.mark.parametrize("w", VARLEN, ids=lambda w: w.name)
def test_varlen(w):
    varlen_case(w)


def decode_case(w, chunk=256):
    fa = _fa()
    q, kc, vc, lens = wl.decode_inputs_cpu(w)        # padding rows are NaN
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    sl = torch.from_numpy(lens).cuda()
    outs = []
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        say("  fa_decode_splitkv %s chunk %d rep %d" % (w.name, chunk, rep))
        fa.decode_splitkv(qd, kd, vd, sl, scale=w.scale, chunk=chunk, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    bits = torch.int32 if w.dtype == "f32" else torch.int16
    assert torch.equal(outs[0][0].view(bits), outs[1][0].view(bits))
    o_ref, lse_ref = oracle.decode(wl.to_f64(q), wl.to_f64(kc), wl.to_f64(vc), lens, w.scale)
    return assert_close(w.dtype, wl.to_f64(outs[0][0]), o_ref, outs[0][1].double().numpy(),
                        lse_ref, "%s chunk %d" % (w.name, chunk))


@pytest.mark.parametrize("chunk", [64, 128, 256, 512])
def test_decode_small(chunk):
    decode_case(wl.SMALL[5], chunk)


DECODE = [
    dataclasses.replace(wl.SMALL[5], name="decode f16 D64 with empty caches", dtype="f16", D=64,
                        seed=21, lens_fixed=[0, 1, 255, 256, 257, 2048]),
    dataclasses.replace(wl.SMALL[5], name="decode f32 D128", dtype="f32", seed=22, B=3),
    dataclasses.replace(wl.SMALL[5], name="decode f32 D64", dtype="f32", D=64, seed=23, B=3),
    dataclasses.replace(wl.SMALL[5], name="decode bf16 D64", dtype="bf16", D=64, seed=24, B=3),
]


@pytest.mark.parametrize("w", DECODE, ids=lambda w: w.name)
def test_decode_cases(w):
    decode_case(w)


def decode_paged_case(w, page_size, chunk=256):
    """Paged cache at shuffled pool positions with NaN in every unused page
    and row: against the oracle, and bit-identical to the contiguous call."""
    fa = _fa()
    q, kc, vc, lens = wl.decode_inputs_cpu(w)
    table, num_pages = wl.page_layout(w, page_size)
    kp, vp = wl.paged_from_cache(kc, vc, lens, table, num_pages, page_size)
    qd, kpd, vpd = q.cuda(), kp.cuda(), vp.cuda()
    sl, bt = torch.from_numpy(lens).cuda(), torch.from_numpy(table).cuda()
    outs = []
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        say("  fa_decode_splitkv_paged %s page %d chunk %d rep %d" % (w.name, page_size, chunk, rep))
        fa.decode_splitkv_paged(qd, kpd, vpd, sl, bt, scale=w.scale, chunk=chunk, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    bits = torch.int32 if w.dtype == "f32" else torch.int16
    assert torch.equal(outs[0][0].view(bits), outs[1][0].view(bits))
    say("  fa_decode_splitkv (contiguous) %s chunk %d" % (w.name, chunk))
    oc, lc = fa.decode_splitkv(qd, kc.cuda(), vc.cuda(), sl, scale=w.scale, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(bits), oc.cpu().view(bits)), "paged differs from contiguous"
    assert torch.equal(outs[0][1].view(torch.int32), lc.cpu().view(torch.int32))
    o_ref, lse_ref = oracle.decode_paged(wl.to_f64(q), wl.to_f64(kp), wl.to_f64(vp), table, lens,
                                         w.scale)
    return assert_close(w.dtype, wl.to_f64(outs[0][0]), o_ref, outs[0][1].double().numpy(),
                        lse_ref, "%s page %d chunk %d" % (w.name, page_size, chunk))


PAGED = [
    (wl.SMALL[5], 16, 256),
    (dataclasses.replace(wl.SMALL[5], name="decode f16 D64 with empty caches", dtype="f16", D=64,
                         seed=31, lens_fixed=[0, 1, 255, 256, 257, 2048]), 64, 64),
    (dataclasses.replace(wl.SMALL[5], name="decode f32 D128", dtype="f32", seed=32, B=3), 32, 128),
    (dataclasses.replace(wl.SMALL[5], name="decode bf16 D64", dtype="bf16", D=64, seed=33, B=3),
     256, 512),
    (dataclasses.replace(wl.SMALL[5], name="decode bf16 D128 one page", seed=34, B=2,
                         lens_fixed=[1024, 700]), 1024, 256),
]


@pytest.mark.parametrize("w,page_size,chunk", PAGED,
                         ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_decode_paged(w, page_size, chunk):
    decode_paged_case(w, page_size, chunk)


def masked_case(w, seqlens=None, slope_mul=1.0):
    """fa_fwd_masked (prefix mask and/or ALiBi) against the oracle."""
    fa = _fa()
    q, k, v = wl.prefill_inputs(w)
    if seqlens is not None:
        for b, L in enumerate(seqlens):
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    slopes = wl.alibi_slopes(w.H) * slope_mul if w.alibi else None
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sd = None if slopes is None else torch.from_numpy(slopes).cuda()
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    outs = []
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((w.B, w.H, w.Nq), float("nan"), dtype=torch.float32, device="cuda")
        say("  fa_fwd_masked %s prefix %d alibi %s rep %d" % (w.name, w.prefix, w.alibi, rep))
        fa.fwd_masked(qd, kd, vd, causal=w.causal, scale=w.scale, seqlens_k=sl, prefix=w.prefix,
                      alibi_slopes=sd, out=o, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    o_ref, lse_ref = oracle.attention(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), w.scale, w.causal,
                                      seqlens_k=seqlens, prefix=w.prefix,
                                      alibi_slopes=None if slopes is None else slopes.astype(np.float64))
    return assert_close(w.dtype, wl.to_f64(o1), o_ref, l1.double().numpy(), lse_ref, w.name)


MASKED = [
    (dataclasses.replace(wl.SMALL[3], name="bf16 D64 causal N1000 prefix 300", prefix=300), None, 1.0),
    (dataclasses.replace(P("f16 D128 causal Nq500 Nk700 prefix 260", "f16", 128, True, 2, 2, 500, 700,
                           seed=41), prefix=260), None, 1.0),
    (dataclasses.replace(P("bf16 D64 causal N300 prefix past every key", "bf16", 64, True, 1, 2, 300,
                           300, seed=42), prefix=400), None, 1.0),
    (dataclasses.replace(P("bf16 D64 causal Nq300 Nk100 prefix 50 (rows see only the prefix)",
                           "bf16", 64, True, 1, 2, 300, 100, seed=43), prefix=50), None, 1.0),
    (dataclasses.replace(wl.SMALL[3], name="bf16 D64 causal N1000 ALiBi", alibi=True), None, 1.0),
    (dataclasses.replace(P("bf16 D128 noncausal N333 ALiBi", "bf16", 128, False, 2, 4, 333, 333,
                           seed=44), alibi=True), None, 1.0),
    (dataclasses.replace(P("f16 D64 causal N700 prefix 128 + ALiBi, padded keys", "f16", 64, True, 2,
                           4, 700, 700, seed=45), prefix=128, alibi=True), [700, 523], 1.0),
    (dataclasses.replace(P("bf16 D64 causal N400 ALiBi steep slopes", "bf16", 64, True, 1, 4, 400,
                           400, seed=46), alibi=True), None, 40.0),
]


@pytest.mark.parametrize("w,seqlens,slope_mul", MASKED, ids=lambda x: getattr(x, "name", str(x)))
def test_masked(w, seqlens, slope_mul):
    masked_case(w, seqlens, slope_mul)
