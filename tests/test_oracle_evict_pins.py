"""Pins of the block-level eviction oracle (oracle/evict.py) and of the oracle's attention under a keep mask.

The method (BellowsKV page, "Three Measurements, Three Operators"): one eviction decision per block of layers,
made from all the block's layers' scores and applied once to the shared latent.
"""
import itertools

import numpy as np
import pytest

from oracle import evict as E
from oracle import ref
from rank_bit_compressed_amd import synth
from tests.helpers import layout, np_any, np_f32, np_u16, oracle_cache


def test_hand_worked_mask():
    # scores 5, 1, 3, 3, 0, 7 keep 3 of 6: positions 5 and 0, then the earlier of the tied 3s (2): bits 0, 2, 5
    s = np.zeros((1, 1, 40), np.float32)
    s[0, 0, :6] = [5, 1, 3, 3, 0, 7]
    m = E.keep_mask(s, [6], 0.5)
    assert m.shape == (1, 2) and m.tolist() == [[0b100101, 0]]
    # two layers: the block score is their sum (here 6, 6, 3, 3, 0, 7 + ...)
    s2 = np.zeros((2, 1, 40), np.float32)
    s2[0, 0, :6] = [5, 1, 3, 3, 0, 7]
    s2[1, 0, :6] = [1, 5, 0, 0, 0, 0]
    assert E.keep_mask(s2, [6], 0.5).tolist() == [[0b100011, 0]]


def test_brute_force_best_subset():
    # the kept set has the largest total block score of all subsets of its size, and among those the
    # lexicographically smallest positions; counts follow floor(ratio T), at least one, at most T
    rng = np.random.default_rng(0)
    for trial in range(60):
        T = int(rng.integers(1, 11))
        n_layers = int(rng.integers(1, 4))
        s = rng.integers(0, 4, (n_layers, 1, 12)).astype(np.float32)   # small integers: ties, exact sums
        ratio = float(rng.choice([0.01, 0.2, 0.5, 0.77, 1.0]))
        kept = E.mask_bits(E.keep_mask(s, [T], ratio), 12)[0]
        n = max(1, min(T, int(np.floor(ratio * T))))
        assert kept.sum() == n and not kept[T:].any()
        a = s.sum(axis=0)[0, :T]
        best = max(itertools.combinations(range(T), n), key=lambda c: (a[list(c)].sum(), [-i for i in c]))
        assert sorted(np.nonzero(kept)[0].tolist()) == list(best), (trial, a, ratio)


def test_extremes_and_layout():
    rng = np.random.default_rng(1)
    s = rng.random((3, 4, 100)).astype(np.float32)
    seq = [100, 37, 1, 0]
    m = E.keep_mask(s, seq, 1.0)
    bits = E.mask_bits(m, 100)
    assert m.shape == (4, 4)
    for b, T in enumerate(seq):
        assert bits[b, :T].all() and not bits[b, T:].any()
    m = E.keep_mask(s, seq, 1e-9)
    assert E.mask_bits(m, 100).sum(axis=1).tolist() == [1, 1, 1, 0]
    a = E.block_scores(s)
    assert E.mask_bits(m, 100)[0, int(np.argmax(a[0]))]
    # scaling every layer's scores by 2 (exact in fp32) changes nothing; the block score is the fp32 sum
    assert np.array_equal(E.keep_mask(2 * s, seq, 0.3), E.keep_mask(s, seq, 0.3))
    assert a.dtype == np.float32 and np.array_equal(a, ((s[0] + s[1]).astype(np.float32) + s[2]).astype(np.float32))


def _shared_case(B=2, T=300, seq=(300, 130)):
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=B, T=T, n_layers=2, page_size=64)
    inp = synth.make_inputs(w, seq_len=list(seq))
    return w, inp, oracle_cache(w, inp)


def _dec(w, inp, cache, keep=None, seq=None, q=None):
    pool, page_off, tok_rank, tok_off = cache
    sl = np_any(inp["seq_len"]) if seq is None else np.asarray(seq, np.int32)
    return ref.decode_attn(layout(w), np_any(inp["block_table"]), sl, np_any(inp["q_pos"]), pool, page_off,
                           tok_rank, tok_off, np_f32(inp["q"]) if q is None else q, np_u16(inp["wk"]),
                           np_u16(inp["wv"]), keep=keep)


def test_masked_attention_reduces_to_shorter_sequences():
    w, inp, cache = _shared_case()
    words = -(-w.T // 32)
    full = _dec(w, inp, cache)
    ones = np.full((w.B, words), 0xFFFFFFFF, np.uint32)
    assert np.array_equal(_dec(w, inp, cache, keep=ones), full)
    # keeping a prefix [0, k) is the sequence cut to k tokens, the query still at its own position
    k = [97, 64]
    pre = np.zeros((w.B, words * 32), bool)
    for b in range(w.B):
        pre[b, :k[b]] = True
    mask = (pre.reshape(w.B, words, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    assert np.allclose(_dec(w, inp, cache, keep=mask), _dec(w, inp, cache, seq=k), rtol=0, atol=1e-14)


def test_masked_attention_single_and_no_token():
    w, inp, cache = _shared_case()
    words = -(-w.T // 32)
    one = np.zeros((w.B, words), np.uint32)
    one[0, 3] = 1 << 7            # sequence 0 keeps token 103 only
    one[1, 0] = 1 << 5            # sequence 1 keeps token 5 only
    a = _dec(w, inp, cache, keep=one)
    q2 = np_f32(inp["q"]) * -3.0 + 0.5
    b_ = _dec(w, inp, cache, keep=one, q=q2)
    # one kept token: the output is its value, whatever the query, the same for every head of a group
    assert np.allclose(a, b_, rtol=0, atol=1e-12)
    gsz = w.n_q_heads // w.n_kv_heads
    g = a.reshape(a.shape[0], a.shape[1], w.n_kv_heads, gsz, -1)
    assert np.allclose(g, g[:, :, :, :1], rtol=0, atol=1e-12)
    none = np.zeros((w.B, words), np.uint32)
    none[1] = one[1]
    z = _dec(w, inp, cache, keep=none)
    assert np.all(z[:, 0] == 0) and np.allclose(z[:, 1], a[:, 1], rtol=0, atol=0)
