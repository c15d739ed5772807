"""Attention dropout for the oracle: the keep decisions and their scale.

TEST INFRASTRUCTURE (part of the oracle package; see its header).

The Hugging Face Flash-Attention-2 integration guide (aibsz.com), 参数详解表格
(parameter table), lists dropout_p: the probability of dropping an attention
weight, 0 outside training, applied inside the fused kernel.  The pages do
not define how the random numbers are drawn; the reading taken here:

* dropout acts on the normalised probabilities P: O = (P o Z) V with
  Z = keep / (1 - p_eff); the softmax statistics (and so lse) are those of
  the undropped P;
* the random numbers come from Philox4x32-10, the counter-based generator
  of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
  1, 2, 3" (SC 2011), implemented here from that paper's definition and
  checked against its published known-answer vectors;
* pair (query i, key j) of batch entry b and head h takes byte (j mod 4) of
  word ((j div 4) mod 4) of Philox(counter = (j div 16, i, h, b),
  key = (seed mod 2^32, seed div 2^32)), bytes numbered from the least
  significant; the key is kept iff that byte is >= t, t = round(256 p)
  (at most 255), so p_eff = t / 256 and the kept weights are scaled by
  256 / (256 - t).
"""

import numpy as np

__all__ = ["philox4x32", "drop_threshold", "keep_mask", "keep_scale"]

# Philox4x32 constants (Salmon et al. 2011, section on the Philox family):
# the two round multipliers and the Weyl increments of the key schedule.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(ctr, key, rounds=10):
    """Philox4x32-R on arrays: ctr [..., 4] and key [..., 2] of uint32 values
    (broadcast together) -> [..., 4] uint32.

    One round: the products M0 * x0 and M1 * x2 are split into their high and
    low 32-bit halves; the new state is (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1,
    lo0).  The key is advanced by the Weyl increments between rounds.
    """
    ctr = np.asarray(ctr, dtype=np.uint64)
    key = np.asarray(key, dtype=np.uint64)
    x0, x1, x2, x3 = (ctr[..., i] for i in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    for r in range(rounds):
        p0 = np.uint64(PHILOX_M0) * x0
        p1 = np.uint64(PHILOX_M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return np.stack(np.broadcast_arrays(x0, x1, x2, x3), axis=-1).astype(np.uint32)


def drop_threshold(p):
    """t = round(256 p): a key is dropped when its random byte is below t."""
    p = float(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(p * 256.0 + 0.5)))


def keep_scale(t):
    """Scale of a kept weight: 1 / (1 - t/256)."""
    return 256.0 / (256.0 - t)


def keep_mask(seed, b, h, q_pos, lk, t):
    """Boolean [n, lk]: is key j kept for query row q_pos[r] of (b, h)?"""
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(-1)
    n = q_pos.size
    if n == 0 or lk == 0:
        return np.ones((n, lk), dtype=bool)
    groups = (lk + 15) // 16
    ctr = np.zeros((n, groups, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(groups, dtype=np.uint64)[None, :]
    ctr[..., 1] = q_pos.astype(np.uint64)[:, None]
    ctr[..., 2] = np.uint64(h)
    ctr[..., 3] = np.uint64(b)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    words = philox4x32(ctr, key).astype(np.uint64)             # [n, groups, 4]
    j = np.arange(lk, dtype=np.int64)
    w = words[:, j >> 4, (j >> 2) & 3]                          # [n, lk]
    byte = (w >> (8 * (j & 3)).astype(np.uint64)) & np.uint64(0xFF)
    return byte >= np.uint64(t)
