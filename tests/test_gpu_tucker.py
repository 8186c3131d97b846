"""Partial Tucker caches on the GPU: kvc_tucker_expand against the oracle's expansion of the same factors, and
decode attention over per-sequence up-projections against the oracle's attention over the same stored bytes.

Expansion: each fp32 output is a chain of r_f fused multiply-adds, so it lies within (r_f + 1) u sum_j
|u_f[i][j] core[c][j]| of the exact value (u = 2^-24); its bf16 store is the nearest-even rounding of that fp32
value, bit for bit; rounding being monotone, it lies between the bf16 roundings of the two ends of that
interval, which is the oracle's own rounding of the exact value wherever the interval holds no rounding boundary.
Decode: max |out - ref| <= 2e-3 max |ref|, the bound used for every decode path; the oracle's up-projections
are its own bf16 roundings of the exact expansion.
"""
import numpy as np
import pytest
import torch

from oracle import ref
from oracle import tucker as TK
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_layout, rel_err
from tests.helpers import layout, np_any, np_f32, oracle_cache

pytestmark = pytest.mark.gpu
TOL = 2e-3
U = 2.0 ** -24


def _pages_order(core_s):
    """One sequence's core in the ABI order [L][Hkv][r_t][r_f] -> the pages' mode order [r_t, r_f, H, L]."""
    return np.transpose(np.asarray(core_s, dtype=np.float64), (2, 3, 1, 0))


def _bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _expand_case(S, L, Hkv, r_t, r_f, latent, row0, seed, prefill=None):
    print(f"[tucker] expand S={S} L={L} Hkv={Hkv} r_t={r_t} r_f={r_f} latent={latent} row0={row0}", flush=True)
    g = torch.Generator().manual_seed(seed)
    uf = torch.randn(S, 128, r_f, generator=g)
    core = torch.randn(S, L, Hkv, r_t, r_f, generator=g) * 3
    w0 = None
    if prefill is not None:
        w0 = torch.full((S, L, latent, Hkv * 128), prefill, dtype=torch.bfloat16, device="cuda")
    w, w32 = kvc.tucker_expand(uf.cuda(), core.cuda(), latent, row0, w=w0, want_f32=True)
    torch.cuda.synchronize()
    gb = w.view(torch.int16).cpu().numpy().view(np.uint16)
    g32 = w32.cpu().numpy()
    ufn, coren = uf.double().numpy(), core.double().numpy()
    for s in range(S):
        want = TK.expand(ufn[s], _pages_order(coren[s]))                                  # [L, r_t, Hkv d]
        absw = TK.expand(np.abs(ufn[s]), np.abs(_pages_order(coren[s])))
        bound = (r_f + 1) * U * absw + 1e-30
        got32 = g32[s, :, row0:row0 + r_t].astype(np.float64)
        assert np.all(np.abs(got32 - want) <= bound), float(np.max(np.abs(got32 - want) / bound))
        got = gb[s, :, row0:row0 + r_t]
        assert np.array_equal(got, TK.to_bf16_bits(got32))                  # nearest even of its own fp32
        # rounding is monotone: the fp32 value lies in [want - bound, want + bound], so its bf16 lies between
        # the roundings of the two ends (where they agree, it is the oracle's own rounding)
        lo = _bits_to_f64(TK.to_bf16_bits(want - bound))
        hi = _bits_to_f64(TK.to_bf16_bits(want + bound))
        gv = _bits_to_f64(got)
        assert np.all((lo <= gv) & (gv <= hi))
        assert np.mean(got != TK.to_bf16_bits(want)) < 1e-3
        # rows outside the written range keep what they held
        keep = 0 if prefill is None else int(torch.tensor([prefill], dtype=torch.bfloat16).view(torch.int16)[0]) & 0xFFFF
        assert np.all(gb[s, :, :row0] == keep) and np.all(gb[s, :, row0 + r_t:] == keep)


def test_expand_ragged_tiles_and_chunks():
    # r_t across 64-row tiles with a tail, r_f across 32-coordinate chunks with a tail, an offset row range
    _expand_case(2, 3, 2, 100, 40, 256, 50, seed=1)


def test_expand_full_feature_rank_single_rows_and_kept_rows():
    _expand_case(1, 1, 3, 64, 128, 64, 0, seed=2)
    _expand_case(3, 2, 1, 1, 1, 8, 7, seed=3, prefill=1.5)


def _oracle_w(w, inp):
    rtk, rtv, rf = w.tucker
    S, width = w.B, w.n_kv_heads * w.head_dim
    wk = np.zeros((S, w.n_layers, w.r_k, width), np.uint16)
    wv = np.zeros_like(wk)
    for s in range(S):
        wk[s, :, :rtk] = TK.to_bf16_bits(TK.expand(np_f32(inp["tk_uf"][s]), _pages_order(np_f32(inp["tk_core"][s]))))
        wv[s, :, rtk:] = TK.to_bf16_bits(TK.expand(np_f32(inp["tv_uf"][s]), _pages_order(np_f32(inp["tv_core"][s]))))
    return wk, wv


def _gpu_w(w, d):
    rtk = w.tucker[0]
    wk, _ = kvc.tucker_expand(d["tk_uf"], d["tk_core"], w.r_k, 0)
    wv, _ = kvc.tucker_expand(d["tv_uf"], d["tv_core"], w.r_k, rtk)
    return wk, wv


def _oracle_decode(w, inp, cache, wk, wv, seqs, heads=None):
    pool, page_off, tok_rank, tok_off = cache
    want = np.full(tuple(inp["q"].shape), np.nan)
    sel_h = None
    if heads is not None:
        sel_h = np.zeros(w.n_kv_heads, np.uint8)
        sel_h[heads] = 1
    for s in seqs:
        sel_b = np.zeros(w.B, np.uint8)
        sel_b[s] = 1
        o = ref.decode_attn(layout(w), np_any(inp["block_table"]), np_any(inp["seq_len"]), np_any(inp["q_pos"]), pool,
                            page_off, tok_rank, tok_off, np_f32(inp["q"]), wk[s], wv[s], sel_b, sel_h)
        want[:, s] = o[:, s]
    return want


@pytest.mark.parametrize("kw,seq", [(dict(B=2, T=600), [600, 333]), (dict(B=3, T=300, n_layers=2, page_size=64),
                                                                        [300, 1, 129])])
def test_tucker_decode_matches_oracle(kw, seq):
    w = synth.WORKLOADS["tucker_group_32k"].scaled(**kw)
    inp = synth.make_inputs(w, seq_len=seq)
    print(f"[tucker] decode {kw} seq={seq}", flush=True)
    cache = oracle_cache(w, inp)
    wk, wv = _oracle_w(w, inp)
    want = _oracle_decode(w, inp, cache, wk, wv, range(w.B))
    d = dev(inp)
    gc = gpu_cache(w, d)
    gwk, gwv = _gpu_w(w, d)
    L = gpu_layout(w)
    out = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], gwk, gwv, w.T, q_pos=d["q_pos"])
    # the split latent skips the zero halves of W_k and W_v: exact zeros, so the same bits
    split = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], gwk, gwv, w.T, q_pos=d["q_pos"],
                            kv_split=w.tucker[0])
    ones = torch.full((w.B, -(-w.T // 32)), -1, dtype=torch.int32, device="cuda")
    split_masked = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], gwk, gwv, w.T, q_pos=d["q_pos"],
                                   kv_split=w.tucker[0], keep_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(out, split) and torch.equal(out, split_masked)
    gp = gc.pool.cpu().numpy()
    assert np.array_equal(gp[:len(cache[0])], cache[0])
    err = rel_err(out, want)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= TOL


def test_per_sequence_w_equal_to_one_shared_w_gives_the_same_bits():
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=3, T=400)
    d = dev(synth.make_inputs(w, seq_len=[400, 250, 3]))
    L = gpu_layout(w)
    cache = gpu_cache(w, d)
    one = kvc.decode_attn(L, cache, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T, q_pos=d["q_pos"])
    wk3 = d["wk"].unsqueeze(0).expand(3, -1, -1, -1).contiguous()
    wv3 = d["wv"].unsqueeze(0).expand(3, -1, -1, -1).contiguous()
    per = kvc.decode_attn(L, cache, d["block_table"], d["seq_len"], d["q"], wk3, wv3, w.T, q_pos=d["q_pos"])
    torch.cuda.synchronize()
    assert torch.equal(one, per)
    # and a sequence's own W is the one it reads: swapping two sequences' W pairs swaps nothing else
    wk3[0], wk3[2] = d["wk"] * 0.5, d["wk"]
    per2 = kvc.decode_attn(L, cache, d["block_table"], d["seq_len"], d["q"], wk3, wv3, w.T, q_pos=d["q_pos"])
    torch.cuda.synchronize()
    assert torch.equal(per2[:, 1:], one[:, 1:]) and not torch.equal(per2[:, 0], one[:, 0])


def test_tucker_fullsize_sampled():
    # the full 4-sequence, 32K-token, 4-layer group; the oracle for one sequence and two KV heads
    w = synth.WORKLOADS["tucker_group_32k"]
    inp = synth.make_inputs(w)
    print("[tucker] full size: oracle compress", flush=True)
    cache = oracle_cache(w, inp)
    wk, wv = _oracle_w(w, inp)
    d = dev(inp)
    gc = gpu_cache(w, d)
    gwk, gwv = _gpu_w(w, d)
    out = kvc.decode_attn(gpu_layout(w), gc, d["block_table"], d["seq_len"], d["q"], gwk, gwv, w.T, q_pos=d["q_pos"],
                          kv_split=w.tucker[0])
    torch.cuda.synchronize()
    assert np.array_equal(gc.pool.cpu().numpy()[:len(cache[0])], cache[0])
    print("[tucker] full size: oracle decode of sequence 1, kv heads 2 and 6", flush=True)
    want = _oracle_decode(w, inp, cache, wk, wv, [1], [2, 6])
    err = rel_err(out, want)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= TOL
