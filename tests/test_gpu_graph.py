"""libfa355 calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

The library only launches kernels on the stream it is given (no allocation,
memset or synchronisation), so a serving loop can capture prefill, varlen,
decode and backward calls once and replay them.  The graph is replayed
several times with eager work and new input values in between; every replay
must equal the eager calls on the same inputs bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _fa():
    import exact_tiled_attention_11_amd as fa
    fa.load()
    return fa


def test_graph_capture_and_replay():
    fa = _fa()
    dev = torch.device("cuda")
    wp = dataclasses.replace(wl.SMALL[3], name="graph prefill", B=2, H=3, Nq=300, Nk=300)
    wv = dataclasses.replace(wl.SMALL[4], name="graph varlen", nseq=3, H=2)
    wd = dataclasses.replace(wl.SMALL[5], name="graph decode", B=3, H=2)

    q, k, v = (t.to(dev) for t in wl.prefill_inputs(wp))
    do = wl.tensor(wp, 3, tuple(q.shape)).to(dev)
    vq, vk, vv, cu = wl.varlen_inputs(wv)
    vq, vk, vv = vq.to(dev), vk.to(dev), vv.to(dev)
    cud = torch.from_numpy(cu).to(dev)
    dq_, kc, vc, lens = wl.decode_inputs_cpu(wd, pad_value=0.0)
    dq_, kc, vc = dq_.to(dev), kc.to(dev), vc.to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)

    # static outputs and workspaces
    o, lse = torch.empty_like(q), torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.fa_bwd_workspace_bytes(wp.B, wp.H, wp.Nq), dtype=torch.uint8, device=dev)
    vo = torch.empty_like(vq)
    vlse = torch.empty((wv.H, vq.shape[0]), dtype=torch.float32, device=dev)
    vws = torch.empty(fa.fa_fwd_varlen_workspace_bytes(len(cu) - 1, vq.shape[0]), dtype=torch.uint8,
                      device=dev)
    dout = torch.empty_like(dq_)
    dlse = torch.empty((wd.B, wd.H), dtype=torch.float32, device=dev)
    dws = torch.empty(fa.fa_decode_workspace_bytes(wd.B, wd.H, wd.Nk, wd.D, wd.chunk),
                      dtype=torch.uint8, device=dev)

    def calls():
        fa.fwd(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, scale=wp.scale, dq=gq, dk=gk, dv=gv, workspace=bws)
        fa.fwd_varlen(vq, vk, vv, cud, cud, causal=True, scale=wv.scale, out=vo, lse=vlse,
                      workspace=vws)
        fa.decode_splitkv(dq_, kc, vc, sl, scale=wd.scale, chunk=wd.chunk, out=dout, lse=dlse,
                          workspace=dws)

    outs = (o, lse, gq, gk, gv, vo, vlse, dout, dlse)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in outs]

    calls()  # eager warmup (first calls check the device outside the capture)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    rng = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(3):
        if rep:
            # new input values in the same buffers, plus unrelated eager work
            for t in (q, do, vq, dq_):
                t.copy_((torch.randn(t.shape, generator=rng) * 0.7).to(t.dtype))
            junk = torch.randn(1 << 20, device=dev).sum()
            torch.cuda.synchronize()
            del junk
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for t in outs:
            t.fill_(float("nan"))
        calls()
        ref = snapshot()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                "replay %d, output %d differs from the eager call" % (rep, i)
            assert not torch.isnan(a.float()).any(), "replay %d, output %d not written" % (rep, i)


def test_graph_capture_masked_dropout_paged_varlen_bwd():
    """The other entry points captured together: the prefix/ALiBi forward and
    its gradients, the dropout forward and its gradients, the packed
    gradients and the paged decode; every replay equals the eager calls."""
    fa = _fa()
    dev = torch.device("cuda")
    wp = dataclasses.replace(wl.SMALL[3], name="graph masked", B=2, H=4, Nq=260, Nk=260)
    wv = dataclasses.replace(wl.SMALL[4], name="graph varlen bwd", nseq=3, H=2)
    wd = dataclasses.replace(wl.SMALL[5], name="graph paged decode", B=3, H=2)

    q, k, v = (t.to(dev) for t in wl.prefill_inputs(wp))
    do = wl.tensor(wp, 3, tuple(q.shape)).to(dev)
    slopes = torch.from_numpy(wl.alibi_slopes(wp.H)).to(dev)
    vq, vk, vv, cu = wl.varlen_inputs(wv)
    vq, vk, vv = vq.to(dev), vk.to(dev), vv.to(dev)
    vdo = wl.tensor(wv, 3, tuple(vq.shape)).to(dev)
    cud = torch.from_numpy(cu).to(dev)
    mx = int(np.diff(cu).max())
    pq, kc, vc, lens = wl.decode_inputs_cpu(wd, pad_value=0.0)
    page = 16
    table, num_pages = wl.page_layout(wd, page)
    pool = (num_pages, page, wd.H, wd.D)
    kp = torch.zeros(pool, dtype=kc.dtype)
    vp = torch.zeros(pool, dtype=vc.dtype)
    kp[torch.from_numpy(table).flatten().long()] = kc.view(-1, *pool[1:])
    vp[torch.from_numpy(table).flatten().long()] = vc.view(-1, *pool[1:])
    pq, kp, vp = pq.to(dev), kp.to(dev), vp.to(dev)
    bt = torch.from_numpy(table).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)

    # static outputs and workspaces
    f32 = dict(dtype=torch.float32, device=dev)
    mo, mlse = torch.empty_like(q), torch.empty((wp.B, wp.H, wp.Nq), **f32)
    do_, dlse = torch.empty_like(q), torch.empty((wp.B, wp.H, wp.Nq), **f32)
    mg = [torch.empty_like(t) for t in (q, k, v)]
    dg = [torch.empty_like(t) for t in (q, k, v)]
    bws = torch.empty(fa.fa_bwd_workspace_bytes(wp.B, wp.H, wp.Nq), dtype=torch.uint8, device=dev)
    bws2 = torch.empty_like(bws)
    vo, vlse = torch.empty_like(vq), torch.empty((wv.H, vq.shape[0]), **f32)
    vws = torch.empty(fa.fa_fwd_varlen_workspace_bytes(len(cu) - 1, vq.shape[0]), dtype=torch.uint8,
                      device=dev)
    vg = [torch.empty_like(t) for t in (vq, vk, vv)]
    vbws = torch.empty(fa.fa_bwd_workspace_bytes(1, wv.H, vq.shape[0]), dtype=torch.uint8,
                       device=dev)
    po, plse = torch.empty_like(pq), torch.empty((wd.B, wd.H), **f32)
    pws = torch.empty(fa.fa_decode_workspace_bytes(wd.B, wd.H, table.shape[1] * page, wd.D, wd.chunk),
                      dtype=torch.uint8, device=dev)

    def calls():
        fa.fwd_masked(q, k, v, causal=True, scale=wp.scale, prefix=40, alibi_slopes=slopes, out=mo,
                      lse=mlse)
        fa.bwd(q, k, v, mo, mlse, do, causal=True, scale=wp.scale, prefix=40, alibi_slopes=slopes,
               dq=mg[0], dk=mg[1], dv=mg[2], workspace=bws)
        fa.fwd_dropout(q, k, v, dropout_p=0.2, seed=9, causal=True, scale=wp.scale, out=do_,
                       lse=dlse)
        fa.bwd(q, k, v, do_, dlse, do, causal=True, scale=wp.scale, dropout_p=0.2, seed=9,
               dq=dg[0], dk=dg[1], dv=dg[2], workspace=bws2)
        fa.fwd_varlen(vq, vk, vv, cud, cud, causal=True, scale=wv.scale, out=vo, lse=vlse,
                      workspace=vws)
        fa.bwd_varlen(vq, vk, vv, vo, vlse, vdo, cud, cud, causal=True, scale=wv.scale,
                      max_seqlen_q=mx, max_seqlen_k=mx, dq=vg[0], dk=vg[1], dv=vg[2],
                      workspace=vbws)
        fa.decode_splitkv_paged(pq, kp, vp, sl, bt, scale=wd.scale, chunk=wd.chunk, out=po,
                                lse=plse, workspace=pws)

    outs = (mo, mlse, *mg, do_, dlse, *dg, vo, vlse, *vg, po, plse)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in outs]

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    rng = torch.Generator(device="cpu").manual_seed(6)
    for rep in range(3):
        if rep:
            for t in (q, do, vq, vdo, pq):
                t.copy_((torch.randn(t.shape, generator=rng) * 0.7).to(t.dtype))
            junk = torch.randn(1 << 20, device=dev).sum()
            torch.cuda.synchronize()
            del junk
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for t in outs:
            t.fill_(float("nan"))
        calls()
        ref = snapshot()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
                "replay %d, output %d differs from the eager call" % (rep, i)
            assert not torch.isnan(a.float()).any(), "replay %d, output %d not written" % (rep, i)
