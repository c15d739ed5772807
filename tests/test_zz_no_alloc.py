"""fa_fwd_varlen_noalloc (the allocation-free packed prefill) against fa_fwd_varlen.

The two share their kernels; only the home of the tile schedule differs (the
library's static per-GPU scratch instead of the caller's workspace), so their
outputs must be bit-identical.  Three calls in a row, each smaller than the one
before, check that what a previous call left in the scratch never matters:
every output buffer starts filled with NaN, the reference call uses a fresh
workspace filled with garbage, and the smallest case is also compared with the
oracle.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import assert_close

pytestmark = pytest.mark.gpu

CASES = [
    dataclasses.replace(wl.SMALL[4], name="noalloc bf16 D64 causal 9 seqs", dtype="bf16", D=64,
                        H=4, nseq=9, len_lo=0, len_hi=700, seed=31),
    dataclasses.replace(wl.SMALL[4], name="noalloc f16 D128 noncausal 4 seqs", dtype="f16", D=128,
                        H=2, causal=False, nseq=4, len_lo=1, len_hi=300, seed=32),
    dataclasses.replace(wl.SMALL[4], name="noalloc f32 D64 causal 2 seqs", dtype="f32", D=64,
                        H=2, nseq=2, len_lo=30, len_hi=150, seed=33),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_call():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    sizes = []
    for w in CASES:
        q, k, v, cu = wl.varlen_inputs(w)
        sizes.append(int(cu[-1]))
        cud = torch.from_numpy(cu).cuda()
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        tq, H = q.shape[0], w.H
        o_n = torch.full_like(qd, float("nan"))
        l_n = torch.full((H, tq), float("nan"), dtype=torch.float32, device="cuda")
        say("fa_fwd_varlen_noalloc %s (total_q %d)" % (w.name, tq))
        st = fa.fa_fwd_varlen_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_n.data_ptr(),
                                      l_n.data_ptr(), cud.data_ptr(), cud.data_ptr(), len(cu) - 1,
                                      tq, tq, H, w.D, w.scale, int(w.causal),
                                      {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}[w.dtype],
                                      torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        ws = torch.randint(0, 255, (fa.fa_fwd_varlen_workspace_bytes(len(cu) - 1, tq),),
                           dtype=torch.uint8, device="cuda")
        o_w = torch.full_like(qd, float("nan"))
        l_w = torch.full((H, tq), float("nan"), dtype=torch.float32, device="cuda")
        say("fa_fwd_varlen %s" % w.name)
        fa.fwd_varlen(qd, kd, vd, cud, cud, causal=w.causal, scale=w.scale, out=o_w, lse=l_w,
                      workspace=ws)
        torch.cuda.synchronize()
        iv = torch.int32 if w.dtype == "f32" else torch.int16
        assert torch.isfinite(o_n).all().item(), "noalloc left output elements unwritten"
        assert torch.equal(o_n.view(iv), o_w.view(iv)), w.name
        assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32)), w.name
    assert sizes[0] > sizes[1] > sizes[2]
    o_ref, lse_ref = oracle.attention_varlen(wl.to_f64(q), wl.to_f64(k), wl.to_f64(v), cu, cu,
                                             w.scale, w.causal)
    assert_close(w.dtype, wl.to_f64(o_n.cpu()), o_ref, l_n.cpu().double().numpy(), lse_ref, w.name)


def test_noalloc_torch_wrapper_and_limit():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    w = CASES[2]
    q, k, v, cu = wl.varlen_inputs(w)
    cud = torch.from_numpy(cu).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say("fwd_varlen_noalloc wrapper %s" % w.name)
    o, lse = fa.fwd_varlen_noalloc(qd, kd, vd, cud, cud, causal=w.causal, scale=w.scale)
    o2, lse2 = fa.fwd_varlen(qd, kd, vd, cud, cud, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    # a schedule larger than the static scratch is refused before any launch
    st = fa.fa_fwd_varlen_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), cud.data_ptr(), cud.data_ptr(), 70000, 70000,
                                  70000, 2, 64, 0.125, 1, fa.FA_F32, None)
    assert st == fa.FA_ERR_TOO_LARGE
