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
  * Compaction (below): the kept tokens leave their pages for new ones, in tiles of 32 slots that span at most
    four 32-position blocks, each slot recording its token's source position.
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


# ---------------------------------------------------------------- compaction of the evicted tokens
#
# Reading (BellowsKV page, "Three Measurements, Three Operators": the one decision is applied to the shared latent,
# so the evicted tokens leave the cache).  The kept tokens of a sequence move, in increasing position, into
# consecutive slots of new pages, each with its stored record bytes unchanged, and each slot records the position
# its token came from, which RoPE needs.  Slots come in tiles of TILE = 32 (the decode's unit of work).  A tile
# holds only tokens within SPAN = 4 blocks of 32 positions of its first token's block: a token starts a new tile
# when the current tile is full or when its block lies SPAN or more blocks past the first token's block.  The
# slots a closed tile leaves over hold no token: position -1 and zero bytes.  The compacted sequence's length is
# its slot count up to its last token, never more than the sequence's own length.

TILE = 32
SPAN = 4


def compact_slots(positions):
    """Slot -> source position (-1: no token) for kept positions given in increasing order."""
    slots = []
    count = 0
    base = 0
    for p in positions:
        blk = int(p) // 32
        if count == TILE or (count > 0 and blk - base >= SPAN):
            slots.extend([-1] * (-len(slots) % TILE))   # close the tile: its remaining slots stay empty
            count = 0
        if count == 0:
            base = blk
        slots.append(int(p))
        count += 1
    return slots


def shared_record_sections(latent, bits, group, P):
    """Block-shared page record: P slots of latent * bits / 8 code bytes, the section padded to 16 bytes, then P
    slots of 4 * latent / group pair bytes.  Returns (code bytes per slot, offset of the pairs, pair bytes per
    slot)."""
    cb = latent * bits // 8
    return cb, (P * cb + 15) // 16 * 16, 4 * (latent // group)


def compact(latent, bits, group, P, block_table, seq_len, keep, pool, page_off, out_block_table, out_page_off,
            out_pool):
    """Compaction of a block-shared cache under a keep mask.  keep: uint32 [B, words] (bit t % 32 of word
    t // 32; tokens past seq_len or past 32 words are not kept).  out_pool: the destination pool's bytes before
    the call (returned as a modified copy: every slot of the pages the compacted sequences use is written, the
    rest is left as it was).  Returns (out_pool, tok_pos int32 [B, max_blocks * P], out_len int32 [B])."""
    bt = np.asarray(block_table)
    obt = np.asarray(out_block_table)
    B, max_blocks = bt.shape
    pool = np.asarray(pool, np.uint8)
    out = np.array(out_pool, dtype=np.uint8, copy=True)
    cb, moff, mb = shared_record_sections(latent, bits, group, P)
    kept = mask_bits(keep, 32 * np.asarray(keep).shape[1])
    tok_pos = np.full((B, max_blocks * P), -1, np.int32)
    out_len = np.zeros(B, np.int32)
    for b in range(B):
        T = min(int(seq_len[b]), kept.shape[1])
        slots = compact_slots(np.nonzero(kept[b, :T])[0])
        out_len[b] = len(slots)
        tok_pos[b, :len(slots)] = slots
        for i in range(-(-len(slots) // P)):
            dst = int(out_page_off[int(obt[b, i])])
            for s in range(P):
                j = i * P + s
                p = slots[j] if j < len(slots) else -1
                code = np.zeros(cb, np.uint8)
                meta = np.zeros(mb, np.uint8)
                if p >= 0:
                    src = int(page_off[int(bt[b, p // P])])
                    code = pool[src + (p % P) * cb: src + (p % P + 1) * cb]
                    meta = pool[src + moff + (p % P) * mb: src + moff + (p % P + 1) * mb]
                out[dst + s * cb: dst + (s + 1) * cb] = code
                out[dst + moff + s * mb: dst + moff + (s + 1) * mb] = meta
    return out, tok_pos, out_len
