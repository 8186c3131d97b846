"""CPU oracle for the block-level eviction decision (one keep mask per sequence for a block of layers).

TEST INFRASTRUCTURE ONLY.  Only the tests import this module; the product library never does.  Plain numpy; the
block score is summed in fp32 (the precision the GPU takes the decision in), the rest is integer work.

What is computed (BellowsKV page, "Three Measurements, Three Operators" and "Key Findings": layers of a block
rank token importance alike, so one eviction decision made from all the block's layers' scores is applied once
to the shared latent).  Readings:
  * A token's block score is the sum of its per-layer importance scores (for instance each layer's window
    salience), added in fp32 in layer order.
  * Sequence b of T tokens keeps n_keep = min(T, max(1, floor(keep_ratio * T))) of them (none when T = 0):
    those of largest block score, equal scores taken in increasing position.
  * The mask holds bit t % 32 of word t // 32 for every kept token t; words [ceil(max_T / 32)] per sequence,
    zero past the sequence's end.
"""
import math

import numpy as np


def block_scores(scores):
    """scores [n_layers, B, max_T] -> fp32 [B, max_T]: the layers' scores added in layer order, each sum
    rounded to fp32."""
    s = np.asarray(scores, dtype=np.float32)
    a = s[0].copy()
    for l in range(1, s.shape[0]):
        a = (a + s[l]).astype(np.float32)
    return a


def keep_count(keep_ratio, T):
    T = int(T)
    if T == 0:
        return 0
    return min(T, max(1, int(math.floor(float(keep_ratio) * T))))


def keep_mask(scores, seq_len, keep_ratio):
    """uint32 keep mask [B, ceil(max_T / 32)]."""
    a = block_scores(scores)
    B, max_T = a.shape
    words = -(-max_T // 32)
    out = np.zeros((B, words), dtype=np.uint32)
    for b in range(B):
        T = int(seq_len[b])
        n = keep_count(keep_ratio, T)
        if n == 0:
            continue
        idx = np.arange(T)
        order = np.lexsort((idx, -a[b, :T].astype(np.float64)))     # score decreasing, then position increasing
        kept = np.zeros(words * 32, dtype=bool)
        kept[order[:n]] = True
        weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
        out[b] = (kept.reshape(words, 32).astype(np.uint64) * weights).sum(axis=1).astype(np.uint32)
    return out


def mask_bits(mask, max_T):
    """Kept flags bool [B, max_T] of a mask (bit t % 32 of word t // 32)."""
    m = np.asarray(mask, dtype=np.uint32)
    t = np.arange(max_T)
    return ((m[:, t // 32] >> (t % 32).astype(np.uint32)) & 1).astype(bool)
