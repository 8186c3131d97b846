"""Shared test helpers: tensor conversion and oracle-side cache building."""
import numpy as np
import torch

from oracle import ref
from rank_bit_compressed_amd import synth


def np_u16(t: torch.Tensor) -> np.ndarray:
    """bf16/fp16 tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np_f32(t) -> np.ndarray:
    if t is None:
        return None
    return t.detach().cpu().float().numpy()


def np_any(t):
    if t is None:
        return None
    return t.detach().cpu().numpy()


def layout(w: synth.Workload) -> ref.Layout:
    return ref.Layout(**w.layout_kwargs())


def pool_bytes_max(w: synth.Workload) -> int:
    L = layout(w)
    return ref.page_bytes_uniform(L) * w.n_pages


def oracle_cache(w: synth.Workload, inp: dict):
    """Compress inputs with the oracle; returns (pool, page_off, tok_rank, tok_off)."""
    L = layout(w)
    return ref.compress(L, np_any(inp["block_table"]), np_any(inp["seq_len"]), w.T, np_any(inp["ranks"]),
                        np_f32(inp["lat_k"]), np_f32(inp["lat_v"]), np_f32(inp["res_k"]), np_f32(inp["res_v"]),
                        w.n_pages, pool_bytes_max(w))


def oracle_decode(w: synth.Workload, inp: dict, cache, sel_b=None, sel_h=None) -> np.ndarray:
    pool, page_off, tok_rank, tok_off = cache
    return ref.decode_attn(layout(w), np_any(inp["block_table"]), np_any(inp["seq_len"]), np_any(inp["q_pos"]),
                           pool, page_off, tok_rank, tok_off, np_f32(inp["q"]), np_u16(inp["wk"]),
                           np_u16(inp["wv"]), sel_b, sel_h)


def sdpa64(q, k, v):
    """Textbook softmax attention in fp64 via torch: q [Hq, d], k/v [T, d] per group -> [Hq, d]."""
    q = torch.as_tensor(q, dtype=torch.float64)[None, :, None, :]
    k = torch.as_tensor(k, dtype=torch.float64)[None, None]
    v = torch.as_tensor(v, dtype=torch.float64)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k.expand(1, q.shape[1], -1, -1),
                                                            v.expand(1, q.shape[1], -1, -1))[0, :, 0].numpy()
