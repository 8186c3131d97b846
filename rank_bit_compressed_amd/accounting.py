"""Algorithmic byte and flop counts of one decode step (closed forms).

These count what the method must read, not what a kernel happens to fetch:
the roofline figures divide them by measured kernel time.
"""
from __future__ import annotations

import math

import torch


def dense_bytes_per_token(n_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes of one token's keys and values in one layer of a dense cache."""
    return n_kv_heads * head_dim * 2 * elem_bytes


def compressed_stream_bytes(w, ranks: torch.Tensor | None, seq_len) -> dict:
    """Bytes of the compressed cache one decode step reads (all sequences, heads and layers).

    per (token, kv head): K codes r_k * b_k / 8 + 4 bytes per group (b_k the key latent bits), V likewise with b_v,
    and for the rotated residual
    2 x (32 code bytes + 2 scale bytes); block-shared mode: per token latent * b / 8 + 4 per group (b the
    latent bits), read once for all layers and heads, plus with the residual 2 x (32 + 2) per layer and head.
    Variable rank adds the per-token rank byte and 4-byte offset word.
    """
    seq_len = [int(x) for x in seq_len]
    n_tok = sum(seq_len)
    if w.shared:
        per_tok = w.r_k * w.latent_bits // 8 + 4 * math.ceil(w.r_k / w.group)
        if w.residual_bits:
            per_tok += w.n_layers * w.n_kv_heads * 2 * (w.head_dim * w.residual_bits // 8 + 2)
        return {"stream": n_tok * per_tok, "tables": 0, "tokens": n_tok}
    Hkv = w.n_kv_heads
    bk = w.latent_bits
    bv = getattr(w, "latent_bits_v", 0) or w.latent_bits
    if w.variable_rank:
        r = torch.cat([ranks[b, :n].to(torch.int64).cpu() for b, n in enumerate(seq_len)])
        g = (r + w.group - 1) // w.group
        per_head = int(r.sum()) * (bk + bv) // 8 + 4 * 2 * int(g.sum())  # K and V code bytes + K and V pairs
        stream = Hkv * per_head
        tables = n_tok * (1 + 4)
    else:
        per_tok_head = (w.r_k * bk // 8 + w.r_v * bv // 8
                        + 4 * (math.ceil(w.r_k / w.group) + math.ceil(w.r_v / w.group)))
        if w.latent_bits == 32:
            per_tok_head = 4 * (w.r_k + w.r_v)
        stream = n_tok * Hkv * per_tok_head
        tables = 0
    if w.residual_bits:
        stream += n_tok * Hkv * 2 * (w.head_dim * w.residual_bits // 8 + 2)
    return {"stream": stream, "tables": tables, "tokens": n_tok}


def upprojection_flops(w, ranks: torch.Tensor | None, seq_len) -> int:
    """Flops of the key up-projection (the one dense contraction per token and head)."""
    seq_len = [int(x) for x in seq_len]
    if w.shared:
        return 2 * w.head_dim * w.r_k * w.n_kv_heads * w.n_layers * sum(seq_len)
    if w.variable_rank:
        r = sum(int(ranks[b, :n].to(torch.int64).sum()) for b, n in enumerate(seq_len))
    else:
        r = w.r_k * sum(seq_len)
    return 2 * w.head_dim * r * w.n_kv_heads
