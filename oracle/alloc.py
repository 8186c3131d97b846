"""CPU oracle for per-token rank allocation by query salience (the prefill step that produces the per-token
ranks the variable-rank cache stores).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg import this
module; the product library never does.  Plain numpy: the salience in fp64; the allocation's decisions in
fp32 (the precision the GPU takes them in), with a numpy sort as its one library step.

What is computed ("VarRate: Training-Free Variable-Rate KV Cache Compression for Long-Context LLMs",
"Method" and "Principles"): every token gets a low rank chosen by its query salience, and no token is
dropped (every rank nonzero).  The page defines neither the salience nor the allocation rule; the readings:
  * Salience of token t of sequence b: the attention probability that the last W prefill queries of the
    sequence put on t, summed over those queries and over all query heads.  Query i of the window sits at
    position seq_len[b] - W + i (positions below 0 are absent); it attends causally to keys t <= its
    position; RoPE (rotate-half pairs (j, j + d/2), theta_j = theta^(-2j/d)) rotates the query at its
    position and the key at t; scores are q.k / sqrt(d); query head h reads KV head h / (Hq / Hkv).
    The salience of a sequence sums to (number of present queries) x Hq.
  * Allocation: ranks come from a ladder r_0 < r_1 < ... < r_{m-1}; every token starts at r_0.  Upgrading
    token t from r_j to r_{j+1} costs r_{j+1} - r_j rank units and gains s_t * w_j (an fp32 product), with
    w_j >= 0 non-increasing: the value per rank unit of the coordinates the step adds (for instance the
    mean fitted squared singular value over them), so a token's steps are taken in order.  The steps of a
    sequence are taken in decreasing order of gain, equal gains together, as long as the total rank stays
    within the budget floor(mean_rank * seq_len); the first group that does not fit ends the allocation.
"""
import math

import numpy as np


def rope_rows(x, pos, theta):
    """Rotate-half RoPE of rows x [..., d] at positions pos (broadcast over the leading axes), fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    freq = theta ** (-2.0 * j / d) if theta > 0 else np.zeros(half)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def salience(q, k, seq_len, theta):
    """q [B, W, Hq, d] pre-RoPE window queries, k [B, max_T, Hkv, d] pre-RoPE keys -> fp64 [B, max_T]
    (zero at t >= seq_len[b])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, W, Hq, d = q.shape
    _, max_T, Hkv, _ = k.shape
    g = Hq // Hkv
    out = np.zeros((B, max_T))
    for b in range(B):
        T = int(seq_len[b])
        kr = rope_rows(k[b, :T], np.arange(T)[:, None], theta)             # [T, Hkv, d]
        for i in range(W):
            p = T - W + i
            if p < 0:
                continue
            qr = rope_rows(q[b, i], np.full((Hq,), p), theta)              # [Hq, d]
            for h in range(Hq):
                s = kr[:p + 1, h // g, :] @ qr[h] / math.sqrt(d)
                e = np.exp(s - s.max())
                out[b, :p + 1] += e / e.sum()
    return out


def budget(mean_rank, T):
    """Total rank units a sequence of T tokens may hold."""
    return int(math.floor(float(mean_rank) * int(T)))


def rank_alloc(sal, seq_len, ladder, step_w, mean_rank):
    """sal fp32 [B, max_T] (values >= 0), ladder ints increasing, step_w fp32 [m - 1] non-increasing >= 0,
    mean_rank in [ladder[0], ladder[-1]] -> uint8 ranks [B, max_T] (0 at t >= seq_len[b])."""
    sal = np.asarray(sal, dtype=np.float32)
    w = np.asarray(step_w, dtype=np.float32)
    lad = [int(r) for r in ladder]
    m = len(lad)
    B, max_T = sal.shape
    out = np.zeros((B, max_T), dtype=np.uint8)
    cost = np.array([lad[j + 1] - lad[j] for j in range(m - 1)], dtype=np.int64)
    for b in range(B):
        T = int(seq_len[b])
        if T == 0:
            continue
        extra = budget(mean_rank, T) - lad[0] * T
        gains = (sal[b, :T, None] * w[None, :]).astype(np.float32)        # [T, m - 1], fp32 products
        flat = gains.ravel()
        order = np.argsort(-flat.astype(np.float64), kind="stable")      # decreasing gain
        sg = flat[order]
        cum = np.cumsum(cost[order % (m - 1)])
        # group ends: the last position of each run of equal gains.  The cumulative cost grows along the order,
        # so the groups that fit form a prefix; the steps taken are those up to the last group end that fits.
        last = np.r_[sg[1:] != sg[:-1], True]
        ends = np.nonzero(last & (cum <= extra))[0]
        n_taken = int(ends[-1]) + 1 if len(ends) else 0
        taken = np.zeros(flat.shape, dtype=bool)
        taken[order[:n_taken]] = True
        n_steps = taken.reshape(T, m - 1).sum(axis=1)
        out[b, :T] = np.array(lad, dtype=np.int64)[n_steps]
    return out
