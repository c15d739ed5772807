"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, and it imports neither the oracle nor the HIP binding.
Both sides of every parity check receive the same tensors from here.

Recipe (stated once, used everywhere):

* Values: i.i.d. N(0, 1) drawn as float32 by numpy's PCG64 generator,
  multiplied by ``value_scale`` (1 unless a workload says otherwise), then
  rounded to the workload's dtype with round-to-nearest-even (torch's
  float32 -> bfloat16 / float16 conversion).  A tensor is drawn in chunks of
  ``CHUNK`` consecutive elements of its row-major flattening; chunk c uses
  ``default_rng(SeedSequence([seed, stream, c]))`` so that chunks can be
  drawn in parallel and the result does not depend on the thread count.
* Lengths: ``default_rng(seed).integers(lo, hi, size=n, endpoint=True)``.
* Streams within a workload: 0 = q, 1 = k, 2 = v.  Decode caches draw each
  batch entry's real rows as stream 1 / 2 with sub-stream b, and leave the
  padding rows beyond the entry's length to the caller (the tests poison
  them with NaN).

The five named workloads are the prefill, varlen and decode shapes of the
method's benchmark table; ``SMALL`` holds reduced shapes of the same kind for
parity runs the oracle finishes in seconds.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

CHUNK = 1 << 22
_THREADS = 16


@dataclass(frozen=True)
class Workload:
    """One synthetic attention problem.

    kind: "prefill" (fixed length, BSHD), "varlen" (packed sequences) or
    "decode" (one query row per batch entry against a padded cache).
    """

    name: str
    kind: str
    dtype: str            # "f32" | "f16" | "bf16"
    H: int
    D: int
    causal: bool
    scale: float
    seed: int
    B: int = 0            # prefill / decode batch
    Nq: int = 0           # prefill query rows
    Nk: int = 0           # prefill key rows (decode: cache capacity Nk_max)
    nseq: int = 0         # varlen sequence count
    len_lo: int = 0       # varlen / decode length range (inclusive)
    len_hi: int = 0
    value_scale: float = 1.0
    chunk: int = 256      # decode split size
    page_size: int = 0    # paged decode: rows per cache page
    prefix: int = 0       # prefill with the prefix mask: keys every query sees
    alibi: bool = False   # prefill with ALiBi: slopes of alibi_slopes(H)
    backward: bool = False  # the gradients of the prefill (dQ, dK, dV from dO)
    dropout: float = 0.0  # attention dropout probability (training), seed = the workload seed
    lens_fixed: Optional[Sequence[int]] = field(default=None, compare=False)

    def lengths(self) -> np.ndarray:
        """Per-sequence lengths (varlen) or per-batch cache lengths (decode)."""
        if self.lens_fixed is not None:
            return np.asarray(self.lens_fixed, dtype=np.int64)
        n = self.nseq if self.kind == "varlen" else self.B
        rng = np.random.default_rng(self.seed)
        return rng.integers(self.len_lo, self.len_hi, size=n, endpoint=True).astype(np.int64)

    def cu_seqlens(self) -> np.ndarray:
        lens = self.lengths()
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*D per visible (query, key) pair for the forward
        (S = Q K^T and P V); 10*D for the backward (S recomputed, dP = dO V^T,
        dV = P^T dO, dQ = dS K, dK = dS^T Q)."""
        per_pair = 10.0 if self.backward else 4.0
        return per_pair * self.D * self.H * self.visible_pairs_per_head()

    def visible_pairs_per_head(self) -> int:
        if self.kind == "prefill":
            return self.B * _pairs(self.Nq, self.Nk, self.causal, self.prefix)
        if self.kind == "varlen":
            return int(sum(_pairs(int(L), int(L), self.causal, self.prefix) for L in self.lengths()))
        return int(self.lengths().sum())

    def bytes_moved(self) -> int:
        """Algorithmic bytes: one read of Q, K, V (real rows) and one write of O and lse."""
        es = {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]
        row = self.H * self.D * es
        if self.kind == "prefill":
            nq, nk = self.B * self.Nq, self.B * self.Nk
            return 2 * nq * row + 2 * nk * row + self.B * self.H * self.Nq * 4
        if self.kind == "varlen":
            tot = int(self.lengths().sum())
            return 4 * tot * row + self.H * tot * 4
        tot_k = int(self.lengths().sum())
        return 2 * tot_k * row + 2 * self.B * row + self.B * self.H * 4


def _pairs(nq: int, nk: int, causal: bool, prefix: int = 0) -> int:
    if not causal:
        return nq * nk
    off = nk - nq
    total = 0
    # row i sees keys 0 .. max(i + off, prefix - 1), at most nk of them
    for i in range(nq):
        total += max(0, min(nk, max(i + off, prefix - 1) + 1))
    return total


# The benchmark table's five workloads.
CFG = {
    1: Workload("causal fp32 B2 N512 H8 D64", "prefill", "f32", H=8, D=64, causal=True,
                scale=1 / 8, seed=100, B=2, Nq=512, Nk=512),
    2: Workload("bidirectional bf16 B4 H16 N2048 D64", "prefill", "bf16", H=16, D=64,
                causal=False, scale=1 / 8, seed=200, B=4, Nq=2048, Nk=2048),
    3: Workload("causal bf16 B4 H16 N8192 D64", "prefill", "bf16", H=16, D=64, causal=True,
                scale=1 / 8, seed=300, B=4, Nq=8192, Nk=8192),
    4: Workload("varlen causal fp16 8 seqs U[1024,16384] H32 D128", "varlen", "f16", H=32,
                D=128, causal=True, scale=1 / math.sqrt(128), seed=4, nseq=8, len_lo=1024,
                len_hi=16384, value_scale=0.5),
    5: Workload("decode bf16 B64 H32 D128 Lk U[4096,32768] chunk 256", "decode", "bf16",
                H=32, D=128, causal=False, scale=1 / math.sqrt(128), seed=5, B=64,
                Nk=32768, len_lo=4096, len_hi=32768, chunk=256),
}

# Reduced shapes of the same kinds (several tiles plus ragged tails).
# Beyond the table: the N8192 causal prefill with the prefix mask (the first
# 2048 keys bidirectional) and with ALiBi slopes.
CFG[7] = replace(CFG[3], name="causal bf16 B4 H16 N8192 D64 prefix 2048", prefix=2048)
CFG[8] = replace(CFG[3], name="causal bf16 B4 H16 N8192 D64 ALiBi", alibi=True)

# Beyond the table: the gradients of the N8192 causal prefill.
CFG[9] = replace(CFG[3], name="backward causal bf16 B4 H16 N8192 D64", backward=True)

# Beyond the table: training-time attention dropout (p = 0.1) in the N8192
# causal prefill and in its gradients.
CFG[10] = replace(CFG[3], name="causal bf16 B4 H16 N8192 D64 dropout 0.1", dropout=0.1)
CFG[11] = replace(CFG[9], name="backward causal bf16 B4 H16 N8192 D64 dropout 0.1", dropout=0.1)

# Beyond the table: the gradients of the N8192 causal prefill with the prefix
# mask and with ALiBi.
CFG[12] = replace(CFG[7], name="backward causal bf16 B4 H16 N8192 D64 prefix 2048", backward=True)
CFG[13] = replace(CFG[8], name="backward causal bf16 B4 H16 N8192 D64 ALiBi", backward=True)

# Beyond the table: the gradients of the packed varlen prefill.
CFG[14] = replace(CFG[4], name="backward varlen causal fp16 8 seqs U[1024,16384] H32 D128",
                  backward=True)

# Beyond the table: the options together — the packed varlen prefill with
# ALiBi and dropout 0.1 and its gradients; the N8192 causal prefill with the
# 2048-key prefix, ALiBi and dropout 0.1 and its gradients.
CFG[15] = replace(CFG[4], name="varlen causal fp16 8 seqs U[1024,16384] H32 D128 ALiBi dropout 0.1",
                  alibi=True, dropout=0.1)
CFG[16] = replace(CFG[15], name="backward " + CFG[15].name, backward=True)
CFG[17] = replace(CFG[3], name="causal bf16 B4 H16 N8192 D64 prefix 2048 ALiBi dropout 0.1",
                  prefix=2048, alibi=True, dropout=0.1)
CFG[18] = replace(CFG[17], name="backward " + CFG[17].name, backward=True)

# Beyond the table: the decode workload over a paged cache (16-row pages at
# shuffled pool positions), the cache layout of serving runtimes.
CFG[6] = replace(CFG[5], name="paged decode bf16 B64 H32 D128 Lk U[4096,32768] chunk 256 page 16",
                 kind="paged", page_size=16)

SMALL = {
    1: CFG[1],
    2: replace(CFG[2], name="bidirectional bf16 B2 H4 N700 D64", B=2, H=4, Nq=700, Nk=700),
    3: replace(CFG[3], name="causal bf16 B2 H4 N1000 D64", B=2, H=4, Nq=1000, Nk=1000),
    4: replace(CFG[4], name="varlen causal fp16 5 seqs U[1,700] H4 D128", H=4, nseq=5,
               len_lo=1, len_hi=700),
    5: replace(CFG[5], name="decode bf16 B6 H4 D128 Lk U[1,2000]", B=6, H=4, Nk=2048,
               len_lo=1, len_hi=2000),
}


# ----------------------------------------------------------------------------
# Drawing
# ----------------------------------------------------------------------------

def _draw_chunk(seed: int, stream: int, sub: int, c: int, n: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, stream, sub, c]))
    return rng.standard_normal(n, dtype=np.float32)


def normal_f32(seed: int, stream: int, n: int, sub: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """n float32 N(0,1) values for (seed, stream, sub), drawn in fixed chunks."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        a, b = c * CHUNK, min(n, (c + 1) * CHUNK)
        out[a:b] = _draw_chunk(seed, stream, sub, c, b - a)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=min(_THREADS, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def tensor(w: Workload, stream: int, shape, sub: int = 0):
    """A torch CPU tensor of ``shape`` in the workload's dtype (RNE-rounded)."""
    import torch
    n = int(np.prod(shape))
    x = normal_f32(w.seed, stream, n, sub)
    if w.value_scale != 1.0:
        x *= np.float32(w.value_scale)
    t = torch.from_numpy(x).reshape(shape)
    return t.to(_torch_dtype(w.dtype))


def prefill_inputs(w: Workload):
    """q [B,Nq,H,D], k, v [B,Nk,H,D] (torch CPU, workload dtype)."""
    assert w.kind == "prefill"
    q = tensor(w, 0, (w.B, w.Nq, w.H, w.D))
    k = tensor(w, 1, (w.B, w.Nk, w.H, w.D))
    v = tensor(w, 2, (w.B, w.Nk, w.H, w.D))
    return q, k, v


def varlen_inputs(w: Workload):
    """Packed q, k, v [total, H, D] and cu_seqlens (int32 numpy, same for q and k)."""
    assert w.kind == "varlen"
    cu = w.cu_seqlens()
    tot = int(cu[-1])
    q = tensor(w, 0, (tot, w.H, w.D))
    k = tensor(w, 1, (tot, w.H, w.D))
    v = tensor(w, 2, (tot, w.H, w.D))
    return q, k, v, cu


def decode_query(w: Workload):
    """q [B, H, D] (torch CPU, workload dtype)."""
    assert w.kind in ("decode", "paged")
    return tensor(w, 0, (w.B, w.H, w.D))


def decode_cache_rows(w: Workload, stream: int, b: int, length: int):
    """Real rows [length, H, D] of batch entry b's K (stream 1) or V (stream 2) cache."""
    return tensor(w, stream, (length, w.H, w.D), sub=1 + b)


def decode_inputs_cpu(w: Workload, pad_value: float = float("nan")):
    """Full CPU caches [B, Nk_max, H, D] with padding rows set to ``pad_value``.

    Only for shapes that fit comfortably in host memory; the benchmark and the
    full-size tests fill device caches entry by entry instead.
    """
    import torch
    lens = w.lengths()
    q = decode_query(w)
    kc = torch.full((w.B, w.Nk, w.H, w.D), pad_value, dtype=_torch_dtype(w.dtype))
    vc = torch.full((w.B, w.Nk, w.H, w.D), pad_value, dtype=_torch_dtype(w.dtype))
    for b in range(w.B):
        L = int(lens[b])
        kc[b, :L] = decode_cache_rows(w, 1, b, L)
        vc[b, :L] = decode_cache_rows(w, 2, b, L)
    return q, kc, vc, lens.astype(np.int32)


def alibi_slopes(H: int) -> np.ndarray:
    """The ALiBi paper's head slopes: the geometric sequence 2^(-8 (h+1) / H),
    float32 [H] (for a power-of-two head count)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def page_layout(w: Workload, page_size: int, extra_pages: int = 5, seed: int = 0):
    """A shuffled placement of each batch entry's cache pages in one pool.

    Returns (block_table int32 [B, max_pages], num_pages): entry b's page i
    is pool page block_table[b, i]; ``extra_pages`` pool pages belong to no
    entry.  The permutation is ``default_rng(seed or w.seed).permutation``.
    """
    max_pages = -(-w.Nk // page_size)
    num_pages = w.B * max_pages + extra_pages
    perm = np.random.default_rng(seed or w.seed).permutation(num_pages)
    table = perm[: w.B * max_pages].reshape(w.B, max_pages).astype(np.int32)
    return table, num_pages


def paged_from_cache(kc, vc, lens, table, num_pages, page_size, pad_value: float = float("nan")):
    """Copy contiguous caches [B, Nk_max, H, D] into a page pool
    [num_pages, page_size, H, D] laid out by ``table``; every pool row that
    holds no real key is ``pad_value``."""
    import torch
    B, _, H, D = kc.shape
    kp = torch.full((num_pages, page_size, H, D), pad_value, dtype=kc.dtype, device=kc.device)
    vp = torch.full_like(kp, pad_value)
    for b in range(B):
        L = int(lens[b])
        for i in range(-(-L // page_size)):
            r0, r1 = i * page_size, min((i + 1) * page_size, L)
            kp[int(table[b, i]), : r1 - r0] = kc[b, r0:r1]
            vp[int(table[b, i]), : r1 - r0] = vc[b, r0:r1]
    return kp, vp


def to_f64(t) -> np.ndarray:
    """Exact float64 copy of a (dtype-rounded) torch CPU tensor."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
