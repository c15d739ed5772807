"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_11_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

# a non-null, 16-byte aligned fake device address: never dereferenced, because
# every call below fails validation before reaching the device
P = 0x10000
MIS = 0x10008  # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FA355_API\s+[\w\s\*]+?\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    assert names == sorted([
        "fa_bwd", "fa_bwd_dropout", "fa_bwd_masked", "fa_bwd_varlen", "fa_bwd_varlen_dropout",
        "fa_bwd_varlen_masked", "fa_bwd_workspace_bytes", "fa_fwd_dropout",
        "fa_fwd", "fa_fwd_masked", "fa_fwd_varlen", "fa_fwd_varlen_dropout",
        "fa_fwd_varlen_masked", "fa_fwd_varlen_workspace_bytes", "fa_fwd_ex", "fa_bwd_ex",
        "fa_fwd_varlen_ex", "fa_bwd_varlen_ex", "fa_fwd_varlen_noalloc",
        "fa_decode_splitkv",
        "fa_decode_splitkv_paged", "fa_decode_workspace_bytes", "fa_status_string",
        "fa_version"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert fa.fa_version().startswith("libfa355")


def test_status_strings():
    for code in range(6):
        assert fa.fa_status_string(code) != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"


def test_workspace_sizes():
    # 64 batches x 32 heads x 128 chunks of (128 floats + 2 floats)
    n = fa.fa_decode_workspace_bytes(64, 32, 32768, 128, 256)
    recs = 64 * 32 * 128
    assert n >= recs * 130 * 4 and n % 256 == 0
    assert fa.fa_decode_workspace_bytes(64, 32, 32768, 96, 256) == 0
    assert fa.fa_decode_workspace_bytes(64, 32, 32768, 128, 100) == 0
    w = fa.fa_fwd_varlen_workspace_bytes(8, 100816)
    assert w >= 4 * (2 + 4 * 8 + 2 * (100816 // 128 + 1 + 8))
    assert fa.fa_fwd_varlen_workspace_bytes(0, 10) == 0


def fwd_args(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, Nq=16, Nk=16, D=64, scale=0.125, causal=1,
             seqlens_k=None, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "Nq", "Nk", "D", "scale",
                           "causal", "seqlens_k", "dtype", "stream")]


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(lse=MIS), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_OK),                      # no-op, no device needed
])
def test_fwd_validation(kw, code):
    assert fa.fa_fwd(*fwd_args(**kw)) == code


def test_varlen_validation():
    base = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, nseq=2, tq=10, tk=10, H=2, D=128, scale=0.1,
                causal=1, ws=P, wsb=1 << 20, dtype=fa.FA_F16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                a["nseq"], a["tq"], a["tk"], a["H"], a["D"], a["scale"],
                                a["causal"], a["ws"], a["wsb"], a["dtype"], a["stream"])
    assert call(D=80) == fa.FA_ERR_UNSUPPORTED
    assert call(nseq=0) == fa.FA_ERR_INVALID_ARG
    assert call(cq=None) == fa.FA_ERR_INVALID_ARG
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=8) == fa.FA_ERR_WORKSPACE
    assert call(ws=MIS) == fa.FA_ERR_INVALID_ARG
    assert call(tq=0) == fa.FA_OK


def test_varlen_noalloc_validation():
    """The allocation-free call checks like fa_fwd_varlen, and rejects a schedule larger than its
    static scratch with FA_ERR_TOO_LARGE, all before any HIP call."""
    base = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, nseq=2, tq=10, tk=10, H=2, D=128, scale=0.1,
                causal=1, dtype=fa.FA_F16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_varlen_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                        a["nseq"], a["tq"], a["tk"], a["H"], a["D"], a["scale"],
                                        a["causal"], a["dtype"], a["stream"])
    assert call(D=80) == fa.FA_ERR_UNSUPPORTED
    assert call(nseq=0) == fa.FA_ERR_INVALID_ARG
    assert call(cq=None) == fa.FA_ERR_INVALID_ARG
    assert call(q=MIS) == fa.FA_ERR_INVALID_ARG
    assert call(tq=0) == fa.FA_OK
    # schedule bytes 4 * (2 + 4 nseq + 2 tiles) rounded to 256, tiles <= ceil(tq / 32) + nseq
    assert call(nseq=70000, tq=70000) == fa.FA_ERR_TOO_LARGE       # 4 nseq alone is 1.1 MB
    assert call(nseq=1, tq=1 << 30, tk=1 << 30) == fa.FA_ERR_TOO_LARGE
    assert call(nseq=1, tq=1 << 30, tk=1 << 30, dtype=fa.FA_F32, D=64) == fa.FA_ERR_TOO_LARGE
    assert fa.fa_status_string(fa.FA_ERR_TOO_LARGE).startswith("problem exceeds")


def test_decode_validation():
    base = dict(q=P, kc=P, vc=P, o=P, lse=P, sl=P, B=2, H=2, N=512, D=128, scale=0.1, chunk=256,
                ws=P, wsb=1 << 20, dtype=fa.FA_BF16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_decode_splitkv(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["sl"], a["B"],
                                    a["H"], a["N"], a["D"], a["scale"], a["chunk"], a["ws"],
                                    a["wsb"], a["dtype"], a["stream"])
    assert call(chunk=100) == fa.FA_ERR_UNSUPPORTED
    assert call(D=256) == fa.FA_ERR_UNSUPPORTED
    assert call(sl=None) == fa.FA_ERR_INVALID_ARG
    assert call(B=0) == fa.FA_ERR_INVALID_ARG
    assert call(wsb=100) == fa.FA_ERR_WORKSPACE
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(o=MIS) == fa.FA_ERR_INVALID_ARG


def test_fwd_masked_validation():
    base = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=64, Nk=64, D=64, scale=0.1, causal=1,
                sl=None, prefix=8, alibi=P, dtype=fa.FA_BF16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                a["Nk"], a["D"], a["scale"], a["causal"], a["sl"], a["prefix"],
                                a["alibi"], a["dtype"], a["stream"])
    assert call(prefix=-1) == fa.FA_ERR_INVALID_ARG
    assert call(causal=0) == fa.FA_ERR_INVALID_ARG              # a prefix needs the causal mask
    assert call(alibi=P + 2) == fa.FA_ERR_INVALID_ARG           # float slopes not 4-byte aligned
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED       # mask families are 16-bit only
    assert call(dtype=fa.FA_F32, prefix=0) == fa.FA_ERR_UNSUPPORTED
    assert call(D=96) == fa.FA_ERR_UNSUPPORTED
    assert call(Nq=0) == fa.FA_OK                               # nothing to do, no device needed


def test_decode_paged_validation():
    """Every argument check runs before any HIP call, so these need no GPU."""
    base = dict(q=P, kc=P, vc=P, o=P, lse=P, sl=P, bt=P, B=2, H=2, npg=64, ps=16, mp=32, D=128,
                scale=0.1, chunk=256, ws=P, wsb=1 << 20, dtype=fa.FA_BF16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_decode_splitkv_paged(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["sl"],
                                          a["bt"], a["B"], a["H"], a["npg"], a["ps"], a["mp"],
                                          a["D"], a["scale"], a["chunk"], a["ws"], a["wsb"],
                                          a["dtype"], a["stream"])
    assert call(ps=24) == fa.FA_ERR_UNSUPPORTED          # not a power of two
    assert call(ps=8) == fa.FA_ERR_UNSUPPORTED           # below 16 rows
    assert call(ps=2048) == fa.FA_ERR_UNSUPPORTED
    assert call(chunk=100) == fa.FA_ERR_UNSUPPORTED
    assert call(D=96) == fa.FA_ERR_UNSUPPORTED
    assert call(bt=None) == fa.FA_ERR_INVALID_ARG
    assert call(bt=P + 2) == fa.FA_ERR_INVALID_ARG       # int32 table not 4-byte aligned
    assert call(npg=0) == fa.FA_ERR_INVALID_ARG
    assert call(mp=-1) == fa.FA_ERR_INVALID_ARG
    assert call(mp=1 << 27, ps=1024) == fa.FA_ERR_INVALID_ARG  # keys per entry overflow int32
    assert call(kc=None) == fa.FA_ERR_INVALID_ARG
    assert call(sl=None) == fa.FA_ERR_INVALID_ARG
    assert call(wsb=100) == fa.FA_ERR_WORKSPACE
    need = fa.fa_decode_workspace_bytes(2, 2, 32 * 16, 128, 256)
    assert call(wsb=need - 1) == fa.FA_ERR_WORKSPACE


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """With the library missing, the binding raises instead of computing anything."""
    import importlib
    monkeypatch.setenv("FA355_LIB", str(tmp_path / "missing.so"))
    mod = importlib.reload(fa)
    try:
        with pytest.raises(ImportError):
            mod.fa_version()
    finally:
        monkeypatch.delenv("FA355_LIB")
        importlib.reload(fa)


def test_bwd_validation():
    """Argument checks of fa_bwd; all run before any HIP call."""
    base = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=2, H=2, Nq=64, Nk=80, D=64,
                scale=0.125, causal=1, sl=None, ws=P, wsb=1 << 20, dtype=fa.FA_BF16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                         a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["scale"],
                         a["causal"], a["sl"], a["ws"], a["wsb"], a["dtype"], a["stream"])
    assert fa.fa_bwd_workspace_bytes(2, 3, 100) == 5120          # 2 x 600 floats, each 256-byte rounded
    assert fa.fa_bwd_workspace_bytes(0, 3, 100) == 0
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED        # 16-bit only
    assert call(D=96) == fa.FA_ERR_UNSUPPORTED
    assert call(B=0) == fa.FA_ERR_INVALID_ARG
    assert call(Nk=-1) == fa.FA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert call(causal=3) == fa.FA_ERR_INVALID_ARG
    assert call(do=None) == fa.FA_ERR_INVALID_ARG
    assert call(dk=None) == fa.FA_ERR_INVALID_ARG
    assert call(lse=MIS) == fa.FA_ERR_INVALID_ARG
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=fa.fa_bwd_workspace_bytes(2, 2, 64) - 1) == fa.FA_ERR_WORKSPACE
    assert call(Nq=0, Nk=0) == fa.FA_OK                          # nothing to do, no device needed


def test_dropout_validation():
    """Argument checks of fa_fwd_dropout and fa_bwd_dropout; all run before any HIP call."""
    base = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=64, Nk=64, D=64, scale=0.1, causal=1,
                sl=None, p=0.1, seed=7, dtype=fa.FA_BF16, stream=None)

    def fwd(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                 a["Nk"], a["D"], a["scale"], a["causal"], a["sl"], a["p"], a["seed"],
                                 a["dtype"], a["stream"])
    assert fwd(p=1.0) == fa.FA_ERR_INVALID_ARG
    assert fwd(p=-0.01) == fa.FA_ERR_INVALID_ARG
    assert fwd(p=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fwd(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED        # 16-bit kernels only
    assert fwd(dtype=fa.FA_F32, p=0.0) == fa.FA_ERR_UNSUPPORTED
    assert fwd(D=96) == fa.FA_ERR_UNSUPPORTED
    assert fwd(q=MIS) == fa.FA_ERR_INVALID_ARG
    assert fwd(Nq=0) == fa.FA_OK
    assert fwd(Nq=0, seed=(1 << 64) - 1) == fa.FA_OK            # any 64-bit seed

    def bwd(**kw):
        a = dict(base, do=P, dq=P, dk=P, dv=P, ws=P, wsb=1 << 20)
        a.update(kw)
        return fa.fa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"],
                                 a["scale"], a["causal"], a["sl"], a["p"], a["seed"], a["ws"],
                                 a["wsb"], a["dtype"], a["stream"])
    assert bwd(p=1.5) == fa.FA_ERR_INVALID_ARG
    assert bwd(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert bwd(ws=None) == fa.FA_ERR_WORKSPACE
    assert bwd(Nq=0, Nk=0) == fa.FA_OK


def test_bwd_masked_validation():
    base = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, Nq=64, Nk=64, D=64,
                scale=0.1, causal=1, sl=None, prefix=8, alibi=P, ws=P, wsb=1 << 20,
                dtype=fa.FA_BF16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_bwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["scale"],
                                a["causal"], a["sl"], a["prefix"], a["alibi"], a["ws"], a["wsb"],
                                a["dtype"], a["stream"])
    assert call(prefix=-1) == fa.FA_ERR_INVALID_ARG
    assert call(causal=0) == fa.FA_ERR_INVALID_ARG              # a prefix needs the causal mask
    assert call(alibi=P + 2) == fa.FA_ERR_INVALID_ARG           # float slopes not 4-byte aligned
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(Nq=0, Nk=0) == fa.FA_OK


def test_bwd_varlen_validation():
    base = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cq=P, ck=P, nseq=3, tq=100, tk=120,
                mq=50, mk=60, H=2, D=128, scale=0.1, causal=1, ws=P, wsb=1 << 20,
                dtype=fa.FA_F16, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                a["dv"], a["cq"], a["ck"], a["nseq"], a["tq"], a["tk"], a["mq"],
                                a["mk"], a["H"], a["D"], a["scale"], a["causal"], a["ws"],
                                a["wsb"], a["dtype"], a["stream"])
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(D=80) == fa.FA_ERR_UNSUPPORTED
    assert call(nseq=0) == fa.FA_ERR_INVALID_ARG
    assert call(mq=-1) == fa.FA_ERR_INVALID_ARG
    assert call(cq=None) == fa.FA_ERR_INVALID_ARG
    assert call(ck=P + 2) == fa.FA_ERR_INVALID_ARG             # int32 offsets not 4-byte aligned
    assert call(dq=MIS) == fa.FA_ERR_INVALID_ARG
    assert call(ws=None) == fa.FA_ERR_WORKSPACE
    assert call(wsb=fa.fa_bwd_workspace_bytes(1, 2, 100) - 1) == fa.FA_ERR_WORKSPACE
    assert call(tq=0, tk=0) == fa.FA_OK


def test_varlen_masked_and_dropout_validation():
    """The packed entry points with the mask families or dropout check their
    options before any HIP call, as the fixed-length ones do."""
    fb = dict(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, nseq=2, tq=10, tk=10, H=2, D=128, scale=0.1,
              causal=1, ws=P, wsb=1 << 20, dtype=fa.FA_F16, stream=None)

    def fmask(prefix=4, alibi=P, **kw):
        a = dict(fb)
        a.update(kw)
        return fa.fa_fwd_varlen_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                       a["nseq"], a["tq"], a["tk"], a["H"], a["D"], a["scale"],
                                       a["causal"], prefix, alibi, a["ws"], a["wsb"], a["dtype"],
                                       a["stream"])

    def fdrop(p=0.1, seed=1, **kw):
        a = dict(fb)
        a.update(kw)
        return fa.fa_fwd_varlen_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"],
                                        a["ck"], a["nseq"], a["tq"], a["tk"], a["H"], a["D"],
                                        a["scale"], a["causal"], p, seed, a["ws"], a["wsb"],
                                        a["dtype"], a["stream"])
    assert fmask(prefix=-1) == fa.FA_ERR_INVALID_ARG
    assert fmask(causal=0) == fa.FA_ERR_INVALID_ARG           # a prefix needs the causal mask
    assert fmask(alibi=P + 2) == fa.FA_ERR_INVALID_ARG        # slopes not 4-byte aligned
    assert fmask(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert fmask(ws=None) == fa.FA_ERR_WORKSPACE
    assert fmask(tq=0) == fa.FA_OK
    assert fdrop(p=1.0) == fa.FA_ERR_INVALID_ARG
    assert fdrop(p=-0.1) == fa.FA_ERR_INVALID_ARG
    assert fdrop(p=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert fdrop(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert fdrop(D=96) == fa.FA_ERR_UNSUPPORTED
    assert fdrop(tq=0) == fa.FA_OK

    bb = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, cq=P, ck=P, nseq=3, tq=100,
              tk=120, mq=50, mk=60, H=2, D=64, scale=0.1, causal=1, ws=P, wsb=1 << 20,
              dtype=fa.FA_BF16, stream=None)

    def bargs(a):
        return (a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                a["cq"], a["ck"], a["nseq"], a["tq"], a["tk"], a["mq"], a["mk"], a["H"], a["D"],
                a["scale"], a["causal"])

    def bmask(prefix=4, alibi=P, **kw):
        a = dict(bb)
        a.update(kw)
        return fa.fa_bwd_varlen_masked(*bargs(a), prefix, alibi, a["ws"], a["wsb"], a["dtype"],
                                       a["stream"])

    def bdrop(p=0.1, seed=1, **kw):
        a = dict(bb)
        a.update(kw)
        return fa.fa_bwd_varlen_dropout(*bargs(a), p, seed, a["ws"], a["wsb"], a["dtype"],
                                        a["stream"])
    assert bmask(prefix=-1) == fa.FA_ERR_INVALID_ARG
    assert bmask(causal=0) == fa.FA_ERR_INVALID_ARG
    assert bmask(alibi=P + 2) == fa.FA_ERR_INVALID_ARG
    assert bmask(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert bmask(wsb=8) == fa.FA_ERR_WORKSPACE
    assert bmask(tq=0, tk=0) == fa.FA_OK
    assert bdrop(p=1.5) == fa.FA_ERR_INVALID_ARG
    assert bdrop(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert bdrop(ws=None) == fa.FA_ERR_WORKSPACE
    assert bdrop(tq=0, tk=0) == fa.FA_OK


def test_every_option_entry_points_validation():
    """fa_fwd_ex / fa_bwd_ex / fa_fwd_varlen_ex / fa_bwd_varlen_ex: each option's own checks,
    before any HIP call."""
    def fex(prefix=4, alibi=P, p=0.1, seed=3, dtype=fa.FA_BF16, causal=1, Nq=16):
        return fa.fa_fwd_ex(P, P, P, P, P, 2, 4, Nq, 16, 64, 0.125, causal, None, prefix, alibi, p,
                            seed, dtype, None)
    assert fex(p=1.0) == fa.FA_ERR_INVALID_ARG
    assert fex(prefix=-2) == fa.FA_ERR_INVALID_ARG
    assert fex(causal=0) == fa.FA_ERR_INVALID_ARG            # prefix without causal
    assert fex(alibi=P + 1) == fa.FA_ERR_INVALID_ARG
    assert fex(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED      # options are 16-bit only
    assert fex(dtype=fa.FA_F32, prefix=0, alibi=None, p=0.0, Nq=0) == fa.FA_OK
    assert fex(Nq=0) == fa.FA_OK

    def bex(p=0.2, **kw):
        a = dict(B=1, H=2, Nq=8, Nk=8, D=128, causal=1, prefix=2, alibi=P, ws=P, wsb=1 << 20,
                 dtype=fa.FA_F16)
        a.update(kw)
        return fa.fa_bwd_ex(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["Nq"], a["Nk"], a["D"],
                            0.1, a["causal"], None, a["prefix"], a["alibi"], p, 5, a["ws"],
                            a["wsb"], a["dtype"], None)
    assert bex(p=-0.5) == fa.FA_ERR_INVALID_ARG
    assert bex(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert bex(ws=None) == fa.FA_ERR_WORKSPACE
    assert bex(Nq=0, Nk=0) == fa.FA_OK

    def fvx(p=0.1, **kw):
        a = dict(prefix=3, alibi=P, causal=1, tq=10, dtype=fa.FA_BF16, ws=P)
        a.update(kw)
        return fa.fa_fwd_varlen_ex(P, P, P, P, P, P, P, 2, a["tq"], 10, 2, 64, 0.1, a["causal"],
                                   a["prefix"], a["alibi"], p, 9, a["ws"], 1 << 20, a["dtype"],
                                   None)
    assert fvx(p=2.0) == fa.FA_ERR_INVALID_ARG
    assert fvx(causal=0) == fa.FA_ERR_INVALID_ARG
    assert fvx(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert fvx(ws=None) == fa.FA_ERR_WORKSPACE
    assert fvx(tq=0) == fa.FA_OK

    def bvx(p=0.1, **kw):
        a = dict(prefix=3, alibi=P, tq=100, tk=100, dtype=fa.FA_BF16, wsb=1 << 20)
        a.update(kw)
        return fa.fa_bwd_varlen_ex(P, P, P, P, P, P, P, P, P, P, P, 2, a["tq"], a["tk"], 60, 60, 2,
                                   64, 0.1, 1, a["prefix"], a["alibi"], p, 9, P, a["wsb"],
                                   a["dtype"], None)
    assert bvx(p=1.0) == fa.FA_ERR_INVALID_ARG
    assert bvx(prefix=-1) == fa.FA_ERR_INVALID_ARG
    assert bvx(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert bvx(wsb=16) == fa.FA_ERR_WORKSPACE
    assert bvx(tq=0, tk=0) == fa.FA_OK
