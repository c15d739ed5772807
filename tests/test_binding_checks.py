"""The torch layer of the binding rejects mismatched tensors before any call
into the library (CPU only).  The kernels size every address from q (and k),
so a smaller k/v, output or gradient buffer, or an index vector of the wrong
type or length, would otherwise make them read or write out of bounds."""

import pytest
import torch

import exact_tiled_attention_11_amd as fa

bf = torch.bfloat16


def fixed(B=2, Nq=8, Nk=8, H=4, D=64, dt=bf):
    return (torch.zeros(B, Nq, H, D, dtype=dt), torch.zeros(B, Nk, H, D, dtype=dt),
            torch.zeros(B, Nk, H, D, dtype=dt))


def packed(tq=20, tk=20, H=4, D=64, nseq=3):
    cu = torch.tensor([0, 5, 12, tq], dtype=torch.int32)[: nseq + 1]
    return (torch.zeros(tq, H, D, dtype=bf), torch.zeros(tk, H, D, dtype=bf),
            torch.zeros(tk, H, D, dtype=bf), cu, cu.clone())


FWD_CALLS = [
    lambda q, k, v, **kw: fa.fwd(q, k, v, **kw),
    lambda q, k, v, **kw: fa.fwd_masked(q, k, v, **kw),
    lambda q, k, v, **kw: fa.fwd_dropout(q, k, v, dropout_p=0.1, seed=1, **kw),
    lambda q, k, v, **kw: fa.fwd_ex(q, k, v, **kw),
]


@pytest.mark.parametrize("call", FWD_CALLS)
def test_fixed_forward_shapes(call):
    q, k, v = fixed()
    with pytest.raises(ValueError, match="q, k, v"):
        call(q, k[:, :, :2], v[:, :, :2])           # fewer heads in k, v
    with pytest.raises(ValueError, match="q, k, v"):
        call(q, k.half(), v)                        # dtype mismatch
    with pytest.raises(ValueError, match="out"):
        call(q, k, v, out=torch.zeros(2, 4, 4, 64, dtype=bf))
    with pytest.raises(ValueError, match="lse"):
        call(q, k, v, lse=torch.zeros(2, 4, 4))     # too few rows
    with pytest.raises(ValueError, match="lse"):
        call(q, k, v, lse=torch.zeros(2, 4, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="seqlens_k"):
        call(q, k, v, seqlens_k=torch.tensor([8, 8], dtype=torch.int64))  # cumsum's dtype
    with pytest.raises(ValueError, match="seqlens_k"):
        call(q, k, v, seqlens_k=torch.tensor([8], dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        call(q, k, v)                               # well-formed, but not on the device


@pytest.mark.parametrize("call", [FWD_CALLS[1], FWD_CALLS[3]])
def test_alibi_slopes(call):
    q, k, v = fixed()
    with pytest.raises(ValueError, match="alibi_slopes"):
        call(q, k, v, alibi_slopes=torch.zeros(3))
    with pytest.raises(ValueError, match="alibi_slopes"):
        call(q, k, v, alibi_slopes=torch.zeros(4, dtype=torch.float64))


def test_backward_shapes():
    q, k, v = fixed(Nk=12)
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(2, 4, 8)
    with pytest.raises(ValueError, match="q, k, v"):
        fa.bwd(q, k[:, :, :2], v[:, :, :2], o, lse, do)
    with pytest.raises(ValueError, match="dout"):
        fa.bwd(q, k, v, o, lse, do[:, :4])
    with pytest.raises(ValueError, match="o must"):
        fa.bwd(q, k, v, o.half(), lse, do)
    with pytest.raises(ValueError, match="lse"):
        fa.bwd(q, k, v, o, torch.zeros(2, 4, 7), do)
    with pytest.raises(ValueError, match="dk"):
        fa.bwd(q, k, v, o, lse, do, dk=torch.zeros_like(q))   # q's shape, not k's
    with pytest.raises(ValueError, match="dq"):
        fa.bwd(q, k, v, o, lse, do, dq=torch.zeros_like(k))
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.bwd(q, k, v, o, lse, do, seqlens_k=torch.tensor([12, 12]))
    with pytest.raises(ValueError, match="alibi_slopes"):
        fa.bwd(q, k, v, o, lse, do, alibi_slopes=torch.zeros(5))


def test_packed_forward_shapes():
    q, k, v, cq, ck = packed()
    with pytest.raises(ValueError, match="q, k, v"):
        fa.fwd_varlen(q, k[:, :2], v[:, :2], cq, ck)
    with pytest.raises(ValueError, match="cu_seqlens_q"):
        fa.fwd_varlen(q, k, v, cq.long(), ck)       # torch.cumsum gives int64
    with pytest.raises(ValueError, match="cu_seqlens_k"):
        fa.fwd_varlen(q, k, v, cq, ck.long())
    with pytest.raises(ValueError, match="same length"):
        fa.fwd_varlen(q, k, v, cq, ck[:3])
    with pytest.raises(ValueError, match="lse"):
        fa.fwd_varlen(q, k, v, cq, ck, lse=torch.zeros(20, 4))   # transposed
    with pytest.raises(ValueError, match="out"):
        fa.fwd_varlen(q, k, v, cq, ck, out=torch.zeros(20, 4, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="alibi_slopes"):
        fa.fwd_varlen(q, k, v, cq, ck, alibi_slopes=torch.zeros(2))


def test_packed_backward_shapes():
    q, k, v, cq, ck = packed()
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(4, 20)
    with pytest.raises(ValueError, match="cu_seqlens_q"):
        fa.bwd_varlen(q, k, v, o, lse, do, cq.long(), ck, max_seqlen_q=8, max_seqlen_k=8)
    with pytest.raises(ValueError, match="dout"):
        fa.bwd_varlen(q, k, v, o, lse, do[:10], cq, ck, max_seqlen_q=8, max_seqlen_k=8)
    with pytest.raises(ValueError, match="lse"):
        fa.bwd_varlen(q, k, v, o, torch.zeros(20, 4), do, cq, ck, max_seqlen_q=8, max_seqlen_k=8)
    with pytest.raises(ValueError, match="dv"):
        fa.bwd_varlen(q, k, v, o, lse, do, cq, ck, max_seqlen_q=8, max_seqlen_k=8,
                      dv=torch.zeros(19, 4, 64, dtype=bf))


def test_decode_shapes():
    q = torch.zeros(3, 4, 128, dtype=bf)
    kc = torch.zeros(3, 64, 4, 128, dtype=bf)
    sl = torch.tensor([10, 20, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="k_cache"):
        fa.decode_splitkv(q, kc[:, :, :2], kc, sl)
    with pytest.raises(ValueError, match="v_cache"):
        fa.decode_splitkv(q, kc, kc[:2], sl)
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.decode_splitkv(q, kc, kc, sl.long())
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.decode_splitkv(q, kc, kc, sl[:2])
    with pytest.raises(ValueError, match="lse"):
        fa.decode_splitkv(q, kc, kc, sl, lse=torch.zeros(3, 4, 1))
    with pytest.raises(ValueError, match="GPU"):
        fa.decode_splitkv(q, kc, kc, sl)


def test_paged_decode_shapes():
    q = torch.zeros(3, 4, 128, dtype=bf)
    pool = torch.zeros(10, 16, 4, 128, dtype=bf)
    sl = torch.tensor([10, 20, 30], dtype=torch.int32)
    bt = torch.zeros(3, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table"):
        fa.decode_splitkv_paged(q, pool, pool, sl, bt.long())
    with pytest.raises(ValueError, match="block_table"):
        fa.decode_splitkv_paged(q, pool, pool, sl, bt[:2])
    with pytest.raises(ValueError, match="v_pages"):
        fa.decode_splitkv_paged(q, pool, pool[:, :8], sl, bt)
    with pytest.raises(ValueError, match="k_pages"):
        fa.decode_splitkv_paged(q, pool[..., :64], pool, sl, bt)
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.decode_splitkv_paged(q, pool, pool, sl.long(), bt)
