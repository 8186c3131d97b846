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


# ---------------------------------------------------------------- compaction of the evicted tokens

def _mask_of(kept):
    B, n = kept.shape
    words = -(-n // 32)
    k = np.zeros((B, words * 32), bool)
    k[:, :n] = kept
    return (k.reshape(B, words, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)


def test_compact_slots_hand_worked():
    # tile 0 opens at block 0; 130 is in block 4, four blocks on, so it opens tile 1 (slots 32..); 200 (block 6)
    # joins it; 500 (block 15) opens tile 2 at slot 64
    s = E.compact_slots([0, 1, 2, 130, 131, 200, 500])
    assert s == [0, 1, 2] + [-1] * 29 + [130, 131, 200] + [-1] * 29 + [500]
    assert E.compact_slots([0, 127]) == [0, 127]                    # block 3: within the span
    assert E.compact_slots([0, 128]) == [0] + [-1] * 31 + [128]     # block 4: a new tile
    assert E.compact_slots(range(40)) == list(range(40))             # a full tile closes with no empty slot
    assert E.compact_slots([31, 32, 159]) == [31, 32] + [-1] * 30 + [159]   # base is the first token's block
    assert E.compact_slots([]) == []


@pytest.mark.parametrize("density,cluster", [(0.3, 0), (0.02, 0), (0.9, 0), (0.3, 256), (1.0, 0)])
def test_compact_slots_invariants(density, cluster):
    # what the layout rule fixes, checked on the result: every kept token once, in increasing position; tiles of
    # 32 slots whose tokens lie within SPAN blocks of the first token's block; empty slots only after a tile's last
    # token; a tile closes early only when the next token is out of its span; length at most the sequence's
    rng = np.random.default_rng(int(density * 100) + cluster)
    for T in (1, 31, 33, 700, 5000):
        if cluster:
            runs = rng.random(-(-T // cluster)) < density
            kept = np.repeat(runs, cluster)[:T]
        else:
            kept = rng.random(T) < density
        pos = np.nonzero(kept)[0]
        s = np.array(E.compact_slots(pos), np.int64)
        assert np.array_equal(s[s >= 0], pos)
        assert len(s) <= T and (len(s) == 0 or s[-1] >= 0)
        tiles = [s[i: i + 32] for i in range(0, len(s), 32)]
        for i, t in enumerate(tiles):
            tok = t[t >= 0]
            assert t[0] >= 0 and np.array_equal(t[: len(tok)], tok)          # tokens first, then empty slots
            base = t[0] // 32
            assert np.all(tok // 32 - base < E.SPAN)
            if i + 1 < len(tiles) and len(tok) < 32:
                assert tiles[i + 1][0] // 32 - base >= E.SPAN


def _slot_latent(pool, rec, sl, P, lat_n, G, bits):
    """The dequantized latent in slot sl of the record at rec, read from the format description alone: code
    section of P slots of lat_n * bits / 8 bytes (little-endian bit strings), padded to 16, then P slots of
    (scale, zero) fp16 pairs, one per group."""
    cb = lat_n * bits // 8
    by = pool[rec + sl * cb: rec + (sl + 1) * cb]
    codes = (np.unpackbits(by, bitorder="little").reshape(lat_n, bits).astype(np.int64) << np.arange(bits)).sum(1)
    m0 = rec + (P * cb + 15) // 16 * 16 + sl * 4 * (lat_n // G)
    meta = pool[m0: m0 + 4 * (lat_n // G)].view(np.float16).reshape(-1, 2).astype(np.float64)
    return codes * np.repeat(meta[:, 0], G) + np.repeat(meta[:, 1], G), by, pool[m0: m0 + 4 * (lat_n // G)]


def _compact_case(bits=4, seed=3):
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=2, T=700, n_layers=2, page_size=64, latent_bits=bits,
                                                     shuffle_pages=True)
    seq = [700, 333]
    inp = synth.make_inputs(w, seq_len=seq)
    cache = oracle_cache(w, inp)
    rng = np.random.default_rng(seed)
    kept = rng.random((w.B, w.T)) < 0.3
    kept[0, 200:330] = False                       # a gap of four blocks: tiles close early
    keep = _mask_of(kept)
    obt = rng.permutation(w.n_pages).astype(np.int32).reshape(w.B, -1)
    rec = cache[1][1] - cache[1][0]
    out0 = np.full(w.n_pages * rec, 0xAB, np.uint8)
    res = E.compact(512, bits, w.group, w.page_size, inp["block_table"].numpy(), seq, keep, cache[0], cache[1], obt,
                    np.arange(w.n_pages, dtype=np.int64) * rec, out0)
    return w, inp, cache, seq, kept, keep, obt, rec, out0, res


@pytest.mark.parametrize("bits", [4, 3])
def test_compacted_records_hold_the_source_records(bits):
    w, inp, cache, seq, kept, keep, obt, rec, out0, (pool2, tok_pos, out_len) = _compact_case(bits)
    P, bt = w.page_size, inp["block_table"].numpy()
    lat = np_f32(inp["lat_k"])
    for b in range(w.B):
        pos = np.nonzero(kept[b, :seq[b]])[0]
        assert np.array_equal(tok_pos[b, :out_len[b]], E.compact_slots(pos))
        assert np.all(tok_pos[b, out_len[b]:] == -1)
        used_pages = -(-int(out_len[b]) // P)
        for i in range(obt.shape[1]):
            r = int(obt[b, i]) * rec
            if i >= used_pages:                     # pages past the compacted length are left as they were
                assert np.all(pool2[r: r + rec] == 0xAB)
                continue
            for s in range(P):
                p = tok_pos[b, i * P + s]
                got, by, meta = _slot_latent(pool2, r, s, P, 512, w.group, bits)
                if p < 0:
                    assert not by.any() and not meta.any()
                    continue
                src = int(cache[1][int(bt[b, p // P])])
                want, by0, meta0 = _slot_latent(cache[0], src, p % P, P, 512, w.group, bits)
                assert np.array_equal(by, by0) and np.array_equal(meta, meta0)
                # and the bytes are the quantizer's outputs for that token's latent
                for g0 in (0, 256):
                    S, Z, Q = ref.quant_intb(lat[b, p, g0: g0 + w.group][None], bits)
                    deq = Q[0] * ref.f16_to_f64(int(S[0])) + ref.f16_to_f64(int(Z[0]))
                    assert np.array_equal(got[g0: g0 + w.group], deq)


def test_compacted_cache_attention_is_the_masked_attention():
    # attention over the compacted cache, computed in numpy from the compacted records and the recorded positions
    # (keys W_k[l]^T c rotated at the slot's source position, the query at its own), equals the oracle's attention
    # over the source cache under the keep mask
    from tests.test_oracle_attention_pins import rope_complex
    from tests.helpers import sdpa64
    w, inp, cache, seq, kept, keep, obt, rec, out0, (pool2, tok_pos, out_len) = _compact_case(4, seed=9)
    pool, page_off, tok_rank, tok_off = cache
    want = ref.decode_attn(layout(w), np_any(inp["block_table"]), np.asarray(seq, np.int32), np_any(inp["q_pos"]),
                           pool, page_off, tok_rank, tok_off, np_f32(inp["q"]), np_u16(inp["wk"]), np_u16(inp["wv"]),
                           keep=keep)
    Wk = inp["wk"].double().numpy(); Wv = inp["wv"].double().numpy()
    q = np_f32(inp["q"])
    P = w.page_size
    for b in range(w.B):
        slots = [(i, int(p)) for i, p in enumerate(tok_pos[b, :out_len[b]]) if p >= 0]
        c = np.stack([_slot_latent(pool2, int(obt[b, i // P]) * rec, i % P, P, 512, w.group, 4)[0] for i, _ in slots])
        pos = np.array([p for _, p in slots])
        qp = int(inp["q_pos"][b])
        for l in range(w.n_layers):
            for h in (0, 3, 7):
                k = c @ Wk[l][:, 128 * h: 128 * h + 128]
                v = c @ Wv[l][:, 128 * h: 128 * h + 128]
                got = sdpa64(rope_complex(q[l, b, 4 * h: 4 * h + 4], qp, w.rope_theta),
                             rope_complex(k, pos, w.rope_theta), v)
                assert np.allclose(got, want[l, b, 4 * h: 4 * h + 4], rtol=0,
                                   atol=1e-11 * np.abs(got).max()), (b, l, h)
