"""Buffers past 2^31 elements: parity where every offset into Q, K, V, O, dO and
the gradients needs 64 bits.

Dense: Q, K, V, O (and dO, dQ, dK, dV) of [64, 2100, 128, 128] bf16, 2.2e9
elements (4.4 GB) each.  Packed: 2,100 sequences of 64 tokens with H 128 and
D 128, the same element count.  The inputs are drawn on the device by torch's
seeded normal generator (at this size the workloads module's host generator
would take minutes); the oracle reads the same values copied back.  Outputs are
NaN-poisoned before the call and must hold no NaN afterwards (every element
written), and whole (batch, head) slices at the start, middle and end of the
buffers are compared with the oracle at the forward's and the gradients'
tolerances.  Needs about 40 GB of device memory.
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

B, N, H, D = 64, 2100, 128, 128
SLICES = [(0, 0), (31, 64), (63, 5), (63, 127)]  # (batch, head)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def randn(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def nan_like(t, shape=None, dtype=None):
    return torch.full(t.shape if shape is None else shape, float("nan"),
                      dtype=t.dtype if dtype is None else dtype, device=t.device)


def f64(t):
    return wl.to_f64(t.cpu())


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "bidirectional"])
def test_fwd_past_2g_elements(causal):
    import exact_tiled_attention_11_amd as fa
    fa.load()
    assert B * N * H * D > 2 ** 31
    scale = 1.0 / math.sqrt(D)
    q, k, v = randn((B, N, H, D), 101), randn((B, N, H, D), 102), randn((B, N, H, D), 103)
    o = nan_like(q)
    lse = nan_like(q, (B, H, N), torch.float32)
    say("  fa_fwd B%d N%d H%d D%d causal=%s" % (B, N, H, D, causal))
    fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()), "unwritten output elements"
    assert not bool(torch.isnan(lse).any()), "unwritten lse elements"
    for b, h in SLICES:
        sl = lambda t: t[b:b + 1, :, h:h + 1, :]
        o_ref, lse_ref = oracle.attention(f64(sl(q)), f64(sl(k)), f64(sl(v)), scale, causal)
        assert_close("bf16", f64(sl(o)), o_ref, lse[b:b + 1, h:h + 1].cpu().double().numpy(),
                     lse_ref, "b%d h%d" % (b, h))
    del q, k, v, o, lse
    release()


def test_bwd_past_2g_elements():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    scale = 1.0 / math.sqrt(D)
    q, k, v = randn((B, N, H, D), 111), randn((B, N, H, D), 112), randn((B, N, H, D), 113)
    do = randn((B, N, H, D), 114)
    say("  fa_fwd then fa_bwd B%d N%d H%d D%d causal" % (B, N, H, D))
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not bool(torch.isnan(g).any()), "unwritten %s elements" % name
    for b, h in SLICES:
        sl = lambda t: t[b:b + 1, :, h:h + 1, :]
        rq, rk, rv = oracle.attention_bwd(f64(sl(q)), f64(sl(k)), f64(sl(v)), f64(sl(do)), scale,
                                          True)
        assert_grad_close("bf16", f64(sl(dq)), rq, "b%d h%d dq" % (b, h))
        assert_grad_close("bf16", f64(sl(dk)), rk, "b%d h%d dk" % (b, h))
        assert_grad_close("bf16", f64(sl(dv)), rv, "b%d h%d dv" % (b, h))
    del q, k, v, do, o, lse, dq, dk, dv
    release()


def test_varlen_past_2g_elements():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    nseq, L = 2100, 64
    total = nseq * L
    assert total * H * D > 2 ** 31
    scale = 1.0 / math.sqrt(D)
    q, k, v = randn((total, H, D), 121), randn((total, H, D), 122), randn((total, H, D), 123)
    cu = torch.arange(0, total + 1, L, dtype=torch.int32, device="cuda")
    o = nan_like(q)
    lse = nan_like(q, (H, total), torch.float32)
    say("  fa_fwd_varlen %d sequences of %d tokens, H%d D%d causal" % (nseq, L, H, D))
    fa.fwd_varlen(q, k, v, cu, cu, causal=True, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(o).any()), "unwritten output elements"
    assert not bool(torch.isnan(lse).any()), "unwritten lse elements"
    # one packed sequence is a standalone causal attention over its L tokens
    for s, h in [(0, 0), (1050, 64), (nseq - 1, 5), (nseq - 1, 127)]:
        r = slice(s * L, (s + 1) * L)
        sl = lambda t: t[r, h:h + 1, :].unsqueeze(0)
        o_ref, lse_ref = oracle.attention(f64(sl(q)), f64(sl(k)), f64(sl(v)), scale, True)
        assert_close("bf16", f64(sl(o)), o_ref, lse[h:h + 1, r].unsqueeze(0).cpu().double().numpy(),
                     lse_ref, "sequence %d h%d" % (s, h))
    del q, k, v, o, lse
    release()
