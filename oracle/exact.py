"""Plain float64 attention: the definition, written out (test infrastructure).

Sources (the pages this follows; cited by page title and section):

* Ascend CANN ``ops-transformer`` FlashAttention explainer (zskr.cn),
  section 背景 (background): standard attention is three steps, S = Q Kᵀ,
  a row softmax of S, then that times V.  Section 原理 (principle) steps 2-4
  and the 代码讲解 (code walk-through) listing: scores are divided by
  sqrt(head_dim) and a causal mask sets masked scores to -inf.
* 轻松读懂FlashAttention 上 (CSDN), section 内存卡点 (memory wall): S and P
  are both N x N; the 小知识 note on safe softmax subtracts the row maximum
  before exponentiation.  Section Softmax求解重构 (rewriting the softmax):
  a row split into groups, each group summarised by its maximum m and its
  sum ℓ, and groups combined pairwise; storing O, m and ℓ.
* Hugging Face Flash-Attention-2 integration guide (aibsz.com), 参数详解表格
  (parameter table): softmax_scale defaults to 1/sqrt(head_dim); is_causal
  selects the lower-triangular mask; the library never returns P.
* Was FlashAttention bei Transformer-Inference verändert (slavadubrov.com),
  opening section: FlashAttention computes exact attention; only the order
  of floating-point operations differs.

Readings where the pages are silent (each one is listed with its reason in
the repository's design notes):

* causal alignment when the query and key counts differ is bottom-right:
  query row i of Lq sees key j of Lk iff j <= i + Lk - Lq;
* a row with no visible key has output 0 and log-sum-exp -inf;
* the log-sum-exp is natural-log, of the *scaled* scores: lse = m + ln ℓ.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against brute force in pure Python, closed forms, invariants and torch's CPU
float64 attention (see that file); the backward in
``tests/test_oracle_bwd_pins.py`` and the dropout paths in
``tests/test_oracle_dropout_pins.py``.  ``partial``/``merge``/``finalize`` are
not used by ``attention``; they exist so the tests can check the pages'
block-merge claim against the plain definition.
"""

import numpy as np

from . import dropout as _dropout

__all__ = [
    "scores",
    "visible",
    "alibi_bias",
    "attention_rows",
    "attention",
    "attention_dropout",
    "attention_bwd",
    "attention_varlen",
    "attention_varlen_bwd",
    "decode",
    "decode_paged",
    "partial",
    "merge",
    "finalize",
]

_F64 = np.float64


def scores(q, k, scale):
    """S = scale * Q Kᵀ for query rows ``q`` [n, D] and key rows ``k`` [m, D].

    CANN FlashAttention explainer, 原理 step 2 and 代码讲解: the score of a
    query and a key is their dot product over head_dim, times the scale.
    """
    q = np.asarray(q, dtype=_F64)
    k = np.asarray(k, dtype=_F64)
    return float(scale) * (q @ k.T)


def visible(q_pos, lq, lk, causal, prefix=0):
    """Boolean [n, lk]: may query row ``q_pos[r]`` (of ``lq`` rows) see key j?

    Keys j >= lk are padding and never visible (they are not even passed).
    With ``causal`` the mask is lower-triangular, bottom-right aligned:
    j <= i + lk - lq.  HF integration guide, 原因分析 item 1 and the
    parameter table's is_causal row; CANN explainer 代码讲解 causal branch.
    The same item names the prefix mask: with ``prefix`` > 0 the first
    ``prefix`` keys are seen by every query as well (bidirectional over the
    prefix, causal after it).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(-1)
    j = np.arange(lk, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.size, lk), dtype=bool)
    return (j[None, :] <= (q_pos[:, None] + (lk - lq))) | (j[None, :] < prefix)


def alibi_bias(q_pos, lq, lk, slope):
    """Additive score bias [n, lk] of ALiBi, the other mask family that item
    names: -slope * |j - p| with p = i + lk - lq the query's own key
    position (for a causal row, slope * (j - p): linear in the distance)."""
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(-1)
    j = np.arange(lk, dtype=np.int64)
    return -float(slope) * np.abs(j[None, :] - (q_pos[:, None] + (lk - lq))).astype(_F64)


def attention_rows(q_rows, q_pos, k, v, lq, lk, scale, causal, prefix=0, alibi_slope=None,
                   keep=None, keep_scale=1.0):
    """Output rows and log-sum-exp for a set of query rows of one (batch, head).

    q_rows: [n, D] query vectors; q_pos: [n] their row indices 0..lq-1;
    k, v: [>= lk, D] key / value rows of the same (batch, head), of which the
    first ``lk`` are real.  Returns (O [n, D], lse [n]), float64.

    Standard (materialised) attention for these rows: S, safe softmax P, O =
    P V.  Rows are independent, so computing a subset of rows gives exactly
    the rows of the full result.  ``prefix`` and ``alibi_slope`` select the
    prefix mask and the ALiBi bias (see ``visible`` and ``alibi_bias``).
    ``keep`` ([n, lk] bool) applies attention dropout: O = (P o keep) V *
    keep_scale, with P (and so lse) the undropped softmax.
    """
    q_rows = np.asarray(q_rows, dtype=_F64)
    n, d = q_rows.shape
    lk = int(lk)
    if lk == 0 or n == 0:
        return np.zeros((n, np.asarray(v).shape[-1]), _F64), np.full(n, -np.inf)
    kk = np.asarray(k[:lk], dtype=_F64)
    vv = np.asarray(v[:lk], dtype=_F64)
    s = scores(q_rows, kk, scale)                       # [n, lk]
    if alibi_slope is not None:
        s = s + alibi_bias(q_pos, lq, lk, alibi_slope)
    vis = visible(q_pos, lq, lk, causal, prefix) if prefix else visible(q_pos, lq, lk, causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)                                   # row maximum (safe softmax)
    empty = np.isneginf(m)                              # no visible key in the row
    m_shift = np.where(empty, 0.0, m)
    p = np.exp(s - m_shift[:, None])                    # exp(-inf) = 0 for masked keys
    ell = p.sum(axis=1)                                 # softmax denominator
    pv = p if keep is None else np.where(keep, p, 0.0) * float(keep_scale)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (pv @ vv) / ell[:, None]
        lse = m + np.log(ell)
    o[empty] = 0.0
    lse[empty] = -np.inf
    return o, lse


def attention(q, k, v, scale, causal, seqlens_k=None, row_chunk=1024, prefix=0,
              alibi_slopes=None):
    """Batched attention in the library's BSHD layout.

    q: [B, Nq, H, D]; k, v: [B, Nk, H, D]; seqlens_k: optional [B] count of
    real keys per batch entry (the rest is padding); default Nk for all.
    prefix: prefix-mask length (with causal); alibi_slopes: optional [H].
    Returns O [B, Nq, H, D] and lse [B, H, Nq] (float64).
    """
    q = np.asarray(q)
    B, nq, H, D = q.shape
    nk = k.shape[1]
    o = np.zeros((B, nq, H, v.shape[-1]), _F64)
    lse = np.zeros((B, H, nq), _F64)
    for b in range(B):
        lk = nk if seqlens_k is None else int(seqlens_k[b])
        for h in range(H):
            kb, vb = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, nq, row_chunk):
                r1 = min(nq, r0 + row_chunk)
                ob, lb = attention_rows(q[b, r0:r1, h, :], np.arange(r0, r1), kb, vb,
                                        nq, lk, scale, causal, prefix,
                                        None if alibi_slopes is None else alibi_slopes[h])
                o[b, r0:r1, h, :] = ob
                lse[b, h, r0:r1] = lb
    return o, lse


def attention_dropout(q, k, v, scale, causal, dropout_p, seed, seqlens_k=None, row_chunk=1024,
                      prefix=0, alibi_slopes=None):
    """Batched attention with attention dropout (BSHD layout), the form the
    HF integration guide's parameter table gives for training: dropout_p is
    the probability of dropping a weight.  The keep decisions and their
    scale are those of ``oracle.dropout`` (Philox4x32-10 counters per
    (batch, head, query, 16-key group)).  ``prefix`` and ``alibi_slopes``
    add the mask families as in ``attention``.  Returns O [B, Nq, H, D] and
    the undropped lse [B, H, Nq].
    """
    q = np.asarray(q)
    B, nq, H, D = q.shape
    nk = k.shape[1]
    t = _dropout.drop_threshold(dropout_p)
    o = np.zeros((B, nq, H, v.shape[-1]), _F64)
    lse = np.zeros((B, H, nq), _F64)
    for b in range(B):
        lk = nk if seqlens_k is None else int(seqlens_k[b])
        for h in range(H):
            for r0 in range(0, nq, row_chunk):
                r1 = min(nq, r0 + row_chunk)
                rows = np.arange(r0, r1)
                keep = _dropout.keep_mask(seed, b, h, rows, lk, t)
                ob, lb = attention_rows(q[b, r0:r1, h, :], rows, k[b, :, h, :], v[b, :, h, :],
                                        nq, lk, scale, causal, prefix,
                                        None if alibi_slopes is None else alibi_slopes[h],
                                        keep=keep, keep_scale=_dropout.keep_scale(t))
                o[b, r0:r1, h, :] = ob
                lse[b, h, r0:r1] = lb
    return o, lse


def attention_bwd(q, k, v, do, scale, causal, seqlens_k=None, dropout_p=0.0, seed=0, prefix=0,
                  alibi_slopes=None, b0=0):
    """Gradients of the forward definition: given dO = dL/dO, returns
    (dQ, dK, dV) in the BSHD layout, float64.

    The CSDN primer 轻松读懂FlashAttention 上, section Softmax求解重构: with
    tiling and recompute, storing O and the row statistics is enough for the
    backward pass, which recomputes P instead of storing it.  What it
    computes is the chain rule through S = scale Q Kᵀ (masked), P = softmax
    rows of S, O = P V, written out here with S and P materialised:
      dV = Pᵀ dO;  dP = dO Vᵀ;  dS = P ∘ (dP - rowsum(dO ∘ O));
      dQ = scale dS K;  dK = scale dSᵀ Q.
    Masked pairs have P = 0 and so no gradient; keys >= Lk (padding) get
    dK = dV = 0; a row with no visible key contributes nothing.
    With dropout (``oracle.dropout``), O = (P o Z) V with Z = keep * scale;
    then dV = (P o Z)ᵀ dO, dP = (dO Vᵀ) o Z, and the rest is unchanged
    (rowsum(dO o O) still equals rowsum(P o dP)).
    ``prefix`` and ``alibi_slopes`` select the forward's prefix mask and
    ALiBi bias (``visible``, ``alibi_bias``): the bias does not depend on q or
    k, so it changes P but not the form of dS.  ``b0`` is the dropout
    counters' batch index of entry 0 (a packed sequence passes its index).
    """
    q, k, v, do = (np.asarray(t) for t in (q, k, v, do))
    B, nq, H, D = q.shape
    nk = k.shape[1]
    dq = np.zeros(q.shape, _F64)
    dk = np.zeros(k.shape, _F64)
    dv = np.zeros(v.shape, _F64)
    for b in range(B):
        lk = nk if seqlens_k is None else int(seqlens_k[b])
        if lk == 0:
            continue
        for h in range(H):
            qq = np.asarray(q[b, :, h], _F64)
            kk = np.asarray(k[b, :lk, h], _F64)
            vv = np.asarray(v[b, :lk, h], _F64)
            g = np.asarray(do[b, :, h], _F64)
            s = scores(qq, kk, scale)
            if alibi_slopes is not None:
                s = s + alibi_bias(np.arange(nq), nq, lk, alibi_slopes[h])
            vis = visible(np.arange(nq), nq, lk, causal, prefix)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1)
            m_shift = np.where(np.isneginf(m), 0.0, m)
            e = np.exp(s - m_shift[:, None])
            ell = e.sum(axis=1)
            p = np.where(ell[:, None] > 0, e / np.where(ell > 0, ell, 1.0)[:, None], 0.0)
            if dropout_p:
                t = _dropout.drop_threshold(dropout_p)
                z = _dropout.keep_mask(seed, b0 + b, h, np.arange(nq), lk, t) * _dropout.keep_scale(t)
            else:
                z = np.ones_like(p)
            o = (p * z) @ vv
            dv[b, :lk, h] = (p * z).T @ g
            dp = (g @ vv.T) * z
            delta = (g * o).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[b, :, h] = float(scale) * (ds @ kk)
            dk[b, :lk, h] = float(scale) * (ds.T @ qq)
    return dq, dk, dv


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal, row_chunk=1024,
                     prefix=0, alibi_slopes=None, dropout_p=0.0, seed=0):
    """Packed variable-length attention (the guide's flash_attn_varlen, FAQ 4).

    q: [total_q, H, D]; k, v: [total_k, H, D]; sequence s owns rows
    cu_seqlens_q[s]:cu_seqlens_q[s+1] of q and cu_seqlens_k[s]:cu_seqlens_k[s+1]
    of k and v.  Each sequence attends only to its own keys, with positions
    counted within the sequence (so ``prefix``, the ALiBi distances and the
    causal alignment are per sequence).  With ``dropout_p`` the keep decisions
    are those of ``attention_dropout`` with the sequence index s in the
    place of the batch index.
    Returns O [total_q, H, D] and lse [H, total_q] (undropped).
    """
    q = np.asarray(q)
    total_q, H, D = q.shape
    o = np.zeros((total_q, H, v.shape[-1]), _F64)
    lse = np.zeros((H, total_q), _F64)
    nseq = len(cu_seqlens_q) - 1
    t = _dropout.drop_threshold(dropout_p) if dropout_p else 0
    for s in range(nseq):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        k0, k1 = int(cu_seqlens_k[s]), int(cu_seqlens_k[s + 1])
        lq, lk = q1 - q0, k1 - k0
        for h in range(H):
            kb, vb = k[k0:k1, h, :], v[k0:k1, h, :]
            for r0 in range(0, lq, row_chunk):
                r1 = min(lq, r0 + row_chunk)
                rows = np.arange(r0, r1)
                keep = _dropout.keep_mask(seed, s, h, rows, lk, t) if dropout_p else None
                ob, lb = attention_rows(q[q0 + r0:q0 + r1, h, :], rows, kb, vb, lq, lk, scale,
                                        causal, prefix,
                                        None if alibi_slopes is None else alibi_slopes[h],
                                        keep=keep,
                                        keep_scale=_dropout.keep_scale(t) if dropout_p else 1.0)
                o[q0 + r0:q0 + r1, h, :] = ob
                lse[h, q0 + r0:q0 + r1] = lb
    return o, lse


def attention_varlen_bwd(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, causal, prefix=0,
                         alibi_slopes=None, dropout_p=0.0, seed=0):
    """Gradients of ``attention_varlen``: each packed sequence is its own
    attention problem, so its rows of (dQ, dK, dV) are ``attention_bwd`` of
    that sequence alone (with its index as the dropout counters' batch
    index).  q, do: [total_q, H, D]; k, v: [total_k, H, D].
    Keys outside every sequence get zero gradients.
    """
    q, k, v, do = (np.asarray(t) for t in (q, k, v, do))
    dq = np.zeros(q.shape, _F64)
    dk = np.zeros(k.shape, _F64)
    dv = np.zeros(v.shape, _F64)
    for s in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        k0, k1 = int(cu_seqlens_k[s]), int(cu_seqlens_k[s + 1])
        gq, gk, gv = attention_bwd(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], do[None, q0:q1],
                                   scale, causal, dropout_p=dropout_p, seed=seed, prefix=prefix,
                                   alibi_slopes=alibi_slopes, b0=s)
        dq[q0:q1], dk[k0:k1], dv[k0:k1] = gq[0], gk[0], gv[0]
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens_k, scale):
    """Single-token decode: one query row per (batch, head) against a cache.

    q: [B, H, D]; k_cache, v_cache: [B, Nk_max, H, D], of which the first
    seqlens_k[b] rows are real.  The query sees every real key (no causal
    mask: it is the newest position).  Returns O [B, H, D], lse [B, H].
    This is the same definition with one query row (the slavadubrov.com
    page's prefill/decode row: decode differs only in its parallel work).
    """
    q = np.asarray(q)
    B, H, D = q.shape
    o = np.zeros((B, H, v_cache.shape[-1]), _F64)
    lse = np.zeros((B, H), _F64)
    for b in range(B):
        lk = int(seqlens_k[b])
        for h in range(H):
            ob, lb = attention_rows(q[b, h][None, :], [0], k_cache[b, :, h, :],
                                    v_cache[b, :, h, :], 1, lk, scale, False)
            o[b, h] = ob[0]
            lse[b, h] = lb[0]
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seqlens_k, scale):
    """Single-token decode over a paged cache (the slavadubrov.com page's
    checklist row on head dimension, mask and cache layout: the layout of the
    cache changes where keys are stored, not what is computed).

    k_pages, v_pages: [num_pages, page_size, H, D]; key t of batch entry b is
    row t % page_size of page block_table[b][t // page_size].  Each entry's
    keys are gathered in key order and the decode definition is applied.
    Returns O [B, H, D], lse [B, H].
    """
    q = np.asarray(q)
    B, H, D = q.shape
    page_size = k_pages.shape[1]
    o = np.zeros((B, H, v_pages.shape[-1]), _F64)
    lse = np.zeros((B, H), _F64)
    for b in range(B):
        lk = int(seqlens_k[b])
        rows = [(int(block_table[b][t // page_size]), t % page_size) for t in range(lk)]
        kb = np.array([k_pages[p, r] for p, r in rows], _F64).reshape(lk, H, k_pages.shape[-1])
        vb = np.array([v_pages[p, r] for p, r in rows], _F64).reshape(lk, H, v_pages.shape[-1])
        for h in range(H):
            ob, lb = attention_rows(q[b, h][None, :], [0], kb[:, h, :], vb[:, h, :], 1, lk,
                                    scale, False)
            o[b, h] = ob[0]
            lse[b, h] = lb[0]
    return o, lse


# ----------------------------------------------------------------------------
# The tiled-softmax summary of the pages, kept separate from the definition
# above so that tests can check one against the other.
# ----------------------------------------------------------------------------

def partial(s, v):
    """Summary of one block of scores.

    s: [n, c] scaled scores of n query rows against a block of c keys
    (masked entries -inf); v: [c, D] the block's value rows.
    Returns (m [n], ell [n], o [n, D]) with m the row maximum, ell the sum of
    exp(s - m) and o the *unnormalised* sum of exp(s - m) * v — the pair
    (m(x), ℓ(x)) and the vector f(x) of the CSDN primer's Softmax求解重构
    section, and m_block / l_block / O_block of the CANN explainer's
    代码讲解 listing.  A block with no visible key has m = -inf, ell = 0,
    o = 0.
    """
    s = np.asarray(s, dtype=_F64)
    v = np.asarray(v, dtype=_F64)
    n = s.shape[0]
    if s.shape[1] == 0:
        return np.full(n, -np.inf), np.zeros(n), np.zeros((n, v.shape[-1]))
    m = s.max(axis=1)
    m_shift = np.where(np.isneginf(m), 0.0, m)
    p = np.exp(s - m_shift[:, None])
    return m, p.sum(axis=1), p @ v


def merge(a, b):
    """Combine two block summaries (m, ell, o) into the summary of their union.

    CSDN primer, Softmax求解重构 steps 2-3 and CANN explainer 原理 step 3:
    the new maximum is the larger of the two; each side's sum and vector are
    rescaled by exp(its maximum - new maximum) and added.
    """
    m1, l1, o1 = a
    m2, l2, o2 = b
    m = np.maximum(m1, m2)
    m_shift = np.where(np.isneginf(m), 0.0, m)
    a1 = np.exp(m1 - m_shift)        # 0 when the side is empty (m1 = -inf)
    a2 = np.exp(m2 - m_shift)
    return m, a1 * l1 + a2 * l2, a1[:, None] * o1 + a2[:, None] * o2


def finalize(p):
    """Normalise a summary: O = o / ell and lse = m + ln(ell).

    CANN explainer 代码讲解, the final division by l_block; the CSDN primer's
    closing note that O plus m and ℓ are what is stored.  Empty rows give
    O = 0 and lse = -inf.
    """
    m, ell, o = p
    empty = ell == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        out = o / ell[:, None]
        lse = m + np.log(ell)
    out[empty] = 0.0
    lse[empty] = -np.inf
    return out, lse
