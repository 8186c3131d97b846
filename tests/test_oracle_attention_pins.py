"""Pins of the oracle's decode attention and compressor against textbook
attention (torch's scaled_dot_product_attention in fp64), closed forms,
special cases and invariants.  No GPU needed."""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import ref
from rank_bit_compressed_amd import synth
from tests.helpers import layout, np_any, np_f32, np_u16, oracle_cache, oracle_decode, sdpa64

RNG = np.random.default_rng(7)


def rope_complex(x, pos, theta):
    """Independent RoPE: pairs (x_j, x_{j+d/2}) as complex numbers times exp(i pos theta^(-2j/d))."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    f = theta ** (-2.0 * np.arange(d // 2) / d)
    pos = np.asarray(pos, np.float64)[..., None]
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos * f)
    return np.concatenate([z.real, z.imag], -1)


def fp32_workload(**kw):
    base = dict(name="t", B=2, T=300, n_q_heads=8, n_kv_heads=2, head_dim=64, r_k=64, r_v=64, group=16,
                latent_bits=32, page_size=64, shuffle_pages=True, seed=5)
    base.update(kw)
    return synth.Workload(**base)


def identity_bases(inp, w):
    """Replace the bases by the identity (exact in bf16): the latents are then the keys/values."""
    eye = torch.eye(w.head_dim, dtype=torch.float32)[:, : w.r_k]
    inp["wk"] = eye.expand(w.n_kv_heads, -1, -1).to(torch.bfloat16).contiguous()
    inp["wv"] = eye[:, : w.r_v].expand(w.n_kv_heads, -1, -1).to(torch.bfloat16).contiguous()
    return inp


@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_full_rank_identity_basis_is_textbook_attention(theta):
    # rank = head_dim, no quantization, B = I: the stored latents ARE the pre-RoPE keys and values
    w = fp32_workload(rope_theta=theta)
    inp = identity_bases(synth.make_inputs(w, seq_len=[300, 137]), w)
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    q = np_f32(inp["q"])
    for b in range(w.B):
        T = int(inp["seq_len"][b])
        for h in range(w.n_kv_heads):
            k = np_f32(inp["lat_k"])[b, :T, h]
            v = np_f32(inp["lat_v"])[b, :T, h]
            qh = q[b, 4 * h: 4 * h + 4]
            if theta:
                k = rope_complex(k, np.arange(T), theta)
                qh = rope_complex(qh, T, theta)
            want = sdpa64(qh, k, v)
            assert np.allclose(out[b, 4 * h: 4 * h + 4], want, rtol=0, atol=1e-12)


def test_full_rank_orthonormal_basis_is_textbook_attention():
    w = fp32_workload(rope_theta=500000.0, seed=9)
    inp = synth.make_inputs(w)                     # random orthonormal bf16 bases, square (r = d)
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    Bk = inp["wk"].double().numpy(); Bv = inp["wv"].double().numpy()
    q = np_f32(inp["q"])
    T = w.T
    for b in range(w.B):
        for h in range(w.n_kv_heads):
            k = np_f32(inp["lat_k"])[b, :, h].astype(np.float64) @ Bk[h].T
            v = np_f32(inp["lat_v"])[b, :, h].astype(np.float64) @ Bv[h].T
            want = sdpa64(rope_complex(q[b, 4 * h: 4 * h + 4], T, w.rope_theta),
                          rope_complex(k, np.arange(T), w.rope_theta), v)
            assert np.allclose(out[b, 4 * h: 4 * h + 4], want, rtol=0, atol=1e-12)


def test_single_token_returns_its_value():
    w = fp32_workload(T=1, B=1, page_size=64, rope_theta=500000.0)
    inp = identity_bases(synth.make_inputs(w), w)
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    v = np_f32(inp["lat_v"])[0, 0]
    for hq in range(w.n_q_heads):
        assert np.array_equal(out[0, hq], v[hq // 4].astype(np.float64))


def test_identical_keys_average_the_values():
    w = fp32_workload(B=1, T=100, rope_theta=0.0)
    inp = identity_bases(synth.make_inputs(w), w)
    inp["lat_k"][:] = inp["lat_k"][:, :1]
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    v = np_f32(inp["lat_v"])[0].astype(np.float64)
    for hq in range(w.n_q_heads):
        assert np.allclose(out[0, hq], v[:, hq // 4].mean(0), atol=1e-13)


@pytest.mark.parametrize("ranks,bits", [((64,), (4, 0)), ((8, 16, 32, 64), (4, 0)), ((64,), (3, 0)), ((64,), (3, 2)),
                                        ((8, 16, 32, 64), (2, 0))])
def test_int4_latents_dequantize_as_scale_times_code_plus_zero(ranks, bits):
    # identity bases with b-bit latents: every key/value is the dequantized latent q * scale + zero of its
    # group (zero beyond the token's rank), computed here from the quantizer's outputs
    w = synth.Workload("t", B=2, T=333, n_q_heads=8, n_kv_heads=2, head_dim=64, r_k=64, r_v=64, group=32,
                       latent_bits=bits[0], latent_bits_v=bits[1], page_size=64, shuffle_pages=True,
                       rope_theta=500000.0, seed=21,
                       variable_rank=len(ranks) > 1, rank_choices=ranks, rank_probs=(0.4, 0.3, 0.2, 0.1)[-len(ranks):])
    inp = identity_bases(synth.make_inputs(w, seq_len=[333, 200]), w)
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    q = np_f32(inp["q"])
    for b in range(w.B):
        T = int(inp["seq_len"][b])
        for h in range(w.n_kv_heads):
            kv = []
            for name in ("lat_k", "lat_v"):
                x = np_f32(inp[name])[b, :T, h]
                deq = np.zeros((T, 64))
                for t in range(T):
                    r = int(inp["ranks"][b, t]) if w.variable_rank else 64
                    for g0 in range(0, r, 32):
                        n = min(32, r - g0)
                        nb = bits[0] if name == "lat_k" else (bits[1] or bits[0])
                        S, Z, Q = ref.quant_intb(x[t, g0: g0 + n][None], nb)
                        deq[t, g0: g0 + n] = (Q[0] * S.view(np.float16).astype(np.float64)[0]
                                              + Z.view(np.float16).astype(np.float64)[0])
                kv.append(deq)
            want = sdpa64(rope_complex(q[b, 4 * h: 4 * h + 4], T, w.rope_theta),
                          rope_complex(kv[0], np.arange(T), w.rope_theta), kv[1])
            assert np.allclose(out[b, 4 * h: 4 * h + 4], want, rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    w = fp32_workload(B=1, T=50, rope_theta=0.0)
    inp = identity_bases(synth.make_inputs(w), w)
    inp["q"][:] = 0
    inp["q"][0, :, 0] = 1.0
    inp["lat_k"][:] = 0
    inp["lat_k"][0, 17, :, 0] = 400.0             # score 400/8 = 50 above the rest
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    v = np_f32(inp["lat_v"])[0].astype(np.float64)
    for hq in range(w.n_q_heads):
        assert np.allclose(out[0, hq], v[17, hq // 4], atol=100 * math.exp(-50))  # mass left on the rest


def test_shuffled_table_gives_identical_output():
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=1000)
    inp = synth.make_inputs(w, seq_len=[1000, 777])
    out_s = oracle_decode(w, inp, oracle_cache(w, inp))
    inp2 = dict(inp)
    inp2["block_table"] = torch.arange(w.n_pages, dtype=torch.int32).view(w.B, -1)
    out_i = oracle_decode(w, inp2, oracle_cache(w, inp2))
    assert np.array_equal(out_s, out_i)


def test_variable_rank_equals_zero_padded_cap():
    # ranks in {32, 64} with group 32: a rank-32 token's second group is absent; stored at the cap with
    # zeros there, that group quantizes to scale 0 / zero 0 and dequantizes to exact zeros.
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=700, rank_choices=(32, 64), rank_probs=(0.6, 0.4))
    inp = synth.make_inputs(w, seq_len=[700, 513])
    out_var = oracle_decode(w, inp, oracle_cache(w, inp))
    wu = w.scaled(variable_rank=False)
    inpu = dict(inp)
    mask = (torch.arange(64)[None, None, None, :] < inp["ranks"].long()[:, :, None, None]).float()
    inpu["lat_k"] = inp["lat_k"] * mask
    inpu["lat_v"] = inp["lat_v"] * mask
    inpu["ranks"] = None
    out_uni = oracle_decode(wu, inpu, oracle_cache(wu, inpu))
    assert np.allclose(out_var, out_uni, rtol=0, atol=1e-13 * np.abs(out_uni).max())


def test_zero_residual_equals_no_residual():
    w = synth.WORKLOADS["residual_128k"].scaled(B=1, T=600)
    inp = synth.make_inputs(w)
    inp["res_k"] = torch.zeros_like(inp["res_k"]); inp["res_v"] = torch.zeros_like(inp["res_v"])
    out_r = oracle_decode(w, inp, oracle_cache(w, inp))
    wn = w.scaled(residual_bits=0)
    inpn = dict(inp, res_k=None, res_v=None)
    out_n = oracle_decode(wn, inpn, oracle_cache(wn, inpn))
    assert np.array_equal(out_r, out_n)


def test_residual_adds_hadamard_of_dequantized_codes():
    # zero latents (scale 0 / zero 0, so they dequantize to 0): each key and value is H e, e the
    # dequantized 2-bit residual; H from scipy's Sylvester matrix
    w = synth.WORKLOADS["residual_128k"].scaled(B=1, T=200, page_size=64, n_q_heads=4, n_kv_heads=1)
    inp = synth.make_inputs(w)
    inp["lat_k"].zero_(); inp["lat_v"].zero_()
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    kv = []
    for name in ("res_k", "res_v"):
        y = np_f32(inp[name])[0, :, 0]
        S, Q = ref.quant_res2(y)
        e = (Q.astype(np.float64) - 1.5) * S.view(np.float16).astype(np.float64)[:, None]
        kv.append(e @ H.T)
    T = w.T
    want = sdpa64(rope_complex(np_f32(inp["q"])[0], T, w.rope_theta),
                  rope_complex(kv[0], np.arange(T), w.rope_theta), kv[1])
    assert np.allclose(out[0], want, rtol=0, atol=1e-12)


def test_shared_latent_with_embedded_bases_equals_per_head():
    # per-head latents of rank 64 (one group of 64 each) concatenated over 8 heads form a 512-dim
    # shared latent whose groups of 64 are exactly the heads; W = block-diagonal embedding of the bases
    wp = synth.WORKLOADS["llama8b_layer_8k"].scaled(T=300, r_k=64, r_v=64, group=64, page_size=64)
    inp = synth.make_inputs(wp)
    inp["lat_v"] = inp["lat_k"].clone()            # the shared latent feeds K and V alike
    out_p = oracle_decode(wp, inp, oracle_cache(wp, inp))
    ws = synth.WORKLOADS["shared_latent_32k"].scaled(B=1, T=300, n_layers=1, page_size=64)
    Hkv, d = 8, 128
    W = {}
    for name in ("wk", "wv"):
        M = torch.zeros(1, 512, Hkv * d, dtype=torch.bfloat16)
        for h in range(Hkv):
            M[0, 64 * h: 64 * h + 64, d * h: d * h + d] = inp[name][h].T
        W[name] = M
    inps = dict(inp, lat_k=inp["lat_k"].reshape(1, 300, 512).contiguous(), lat_v=None,
                wk=W["wk"], wv=W["wv"], q=inp["q"][None])
    out_s = oracle_decode(ws, inps, oracle_cache(ws, inps))
    assert np.allclose(out_s[0], out_p, rtol=0, atol=1e-13 * np.abs(out_p).max())


def test_dense_oracle_is_textbook_attention():
    w = synth.WORKLOADS["llama8b_layer_8k"].scaled(B=2, T=500, page_size=64, shuffle_pages=True)
    d = synth.make_dense_inputs(w)
    bt = synth.make_inputs(w)["block_table"]
    sl = np.array([500, 321], np.int32)
    out = ref.dense_attn(32, 8, 128, 64, np_any(bt), sl, np_u16(d["k_pages"]), np_u16(d["v_pages"]),
                         np_f32(d["q"]))
    K = d["k_pages"].double().numpy(); V = d["v_pages"].double().numpy()
    q = d["q"].double().numpy()
    for b in range(2):
        pages = np_any(bt)[b]
        for h in range(8):
            k = np.concatenate([K[p, h] for p in pages])[: sl[b]]
            v = np.concatenate([V[p, h] for p in pages])[: sl[b]]
            assert np.allclose(out[b, 4 * h: 4 * h + 4], sdpa64(q[b, 4 * h: 4 * h + 4], k, v), atol=1e-12)


# ---------------------------------------------------------------- compressor: layout and byte accounting

def parse_pool_per_head(w, cache, b, t, h, bt):
    """Independent reader of one slot's codes and pairs, from the layout description: b-bit codes are the
    slot's little-endian bit string (numpy's unpackbits), code i at bits b*i .."""
    pool, page_off, tok_rank, tok_off = cache
    P = w.page_size
    bk = w.latent_bits
    bv = w.latent_bits_v or w.latent_bits
    p = int(bt[b, t // P]); s = t % P
    rec = int(page_off[p])
    pad = lambda x: (x + 15) // 16 * 16
    if w.variable_rank:
        tot_r, tot_g = int(tok_off[p, P]) & 0xFFFF, int(tok_off[p, P]) >> 16
        pre_r, pre_g = int(tok_off[p, s]) & 0xFFFF, int(tok_off[p, s]) >> 16
        rk = rv = int(tok_rank[p, s])
        ck = cv = tot_r * bk // 8; mk = mv = 4 * tot_g
        prk = prv = pre_r * bk // 8; pmk = pmv = 4 * pre_g
    else:
        rk, rv = w.r_k, w.r_v
        ck, cv = P * rk * bk // 8, P * rv * bv // 8
        mk, mv = P * 4 * -(-rk // w.group), P * 4 * -(-rv // w.group)
        prk, prv = s * rk * bk // 8, s * rv * bv // 8
        pmk, pmv = s * 4 * -(-rk // w.group), s * 4 * -(-rv // w.group)
    hb = pad(ck) + pad(cv) + pad(mk) + pad(mv)
    if w.residual_bits:
        hb += 2 * pad(P * 32) + 2 * pad(P * 2)
    base = rec + h * hb
    out = {}
    for name, r, nb, sec, pre, msec, mpre in (("k", rk, bk, 0, prk, pad(ck) + pad(cv), pmk),
                                              ("v", rv, bv, pad(ck), prv, pad(ck) + pad(cv) + pad(mk), pmv)):
        by = pool[base + sec + pre: base + sec + pre + r * nb // 8]
        bitstr = np.unpackbits(by, bitorder="little")[: r * nb].reshape(r, nb)
        codes = (bitstr.astype(np.int64) << np.arange(nb)).sum(1)
        ng = -(-r // w.group)
        meta = pool[base + msec + mpre: base + msec + mpre + 4 * ng].view(np.uint16).reshape(ng, 2)
        out[name] = (codes, meta)
    return out


@pytest.mark.parametrize("name,bits", [("llama8b_layer_8k", (4, 0)), ("varrank_paged_32k", (4, 0)),
                                       ("llama8b_layer_8k", (3, 0)), ("llama8b_layer_8k", (2, 0)),
                                       ("llama8b_layer_8k", (3, 2)), ("varrank_paged_32k", (3, 0))])
def test_pool_holds_the_quantizer_outputs(name, bits):
    w = synth.WORKLOADS[name].scaled(B=2, T=700, page_size=128, latent_bits=bits[0], latent_bits_v=bits[1])
    inp = synth.make_inputs(w, seq_len=[700, 450])
    cache = oracle_cache(w, inp)
    bt = np_any(inp["block_table"])
    lat = {"k": np_f32(inp["lat_k"]), "v": np_f32(inp["lat_v"])}
    for (b, t, h) in [(0, 0, 0), (0, 699, 7), (1, 449, 3), (1, 128, 5), (0, 255, 2), (1, 77, 0)]:
        got = parse_pool_per_head(w, cache, b, t, h, bt)
        for kv in ("k", "v"):
            r = int(inp["ranks"][b, t]) if w.variable_rank else (w.r_k if kv == "k" else w.r_v)
            codes, meta = got[kv]
            for g0 in range(0, r, w.group):
                n = min(w.group, r - g0)
                nb = w.latent_bits if kv == "k" else (w.latent_bits_v or w.latent_bits)
                S, Z, Q = ref.quant_intb(lat[kv][b, t, h, g0: g0 + n][None], nb)
                assert np.array_equal(codes[g0: g0 + n], Q[0])
                assert meta[g0 // w.group, 0] == S[0] and meta[g0 // w.group, 1] == Z[0]


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_shared_pool_holds_the_quantizer_outputs(bits):
    # block-shared records (BellowsKV, "Reading the Retention Table": INT4 and INT3 on the shared latent): slot s
    # of a page holds latent * b / 8 code bytes (the latent's little-endian bit string) after s such slots, then,
    # past the 16-byte-padded code section, 4 bytes per group; read here from that description alone
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=2, T=300, page_size=64, latent_bits=bits)
    inp = synth.make_inputs(w, seq_len=[300, 129])
    pool, page_off, _, _ = oracle_cache(w, inp)
    bt = np_any(inp["block_table"])
    lat = np_f32(inp["lat_k"])
    P, Lt, G = w.page_size, w.r_k, w.group
    cb = Lt * bits // 8
    pad = lambda x: (x + 15) // 16 * 16
    assert np.array_equal(page_off, np.arange(w.n_pages) * (pad(P * cb) + pad(P * 4 * (Lt // G))))
    for (b, t) in [(0, 0), (0, 299), (1, 128), (1, 63), (0, 64)]:
        p, sl = int(bt[b, t // P]), t % P
        rec = int(page_off[p])
        by = pool[rec + sl * cb: rec + (sl + 1) * cb]
        codes = (np.unpackbits(by, bitorder="little").reshape(Lt, bits).astype(np.int64) << np.arange(bits)).sum(1)
        m0 = rec + pad(P * cb) + sl * 4 * (Lt // G)
        meta = pool[m0: m0 + 4 * (Lt // G)].view(np.uint16).reshape(-1, 2)
        for g0 in range(0, Lt, G):
            S, Z, Q = ref.quant_intb(lat[b, t, g0: g0 + G][None], bits)
            assert np.array_equal(codes[g0: g0 + G], Q[0])
            assert meta[g0 // G, 0] == S[0] and meta[g0 // G, 1] == Z[0]


def test_offsets_are_prefix_sums_and_total_is_closed_form():
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=3, T=1000)
    inp = synth.make_inputs(w, seq_len=[1000, 999, 1])
    pool, page_off, tok_rank, tok_off = oracle_cache(w, inp)
    P, G, Hkv = w.page_size, w.group, w.n_kv_heads
    ranks = np_any(inp["ranks"]); bt = np_any(inp["block_table"]); sl = np_any(inp["seq_len"])
    want_rank = np.zeros((w.n_pages, P), np.uint8)
    for b in range(w.B):
        for t in range(sl[b]):
            want_rank[bt[b, t // P], t % P] = ranks[b, t]
    assert np.array_equal(tok_rank, want_rank)
    r = want_rank.astype(np.int64)
    g = -(-r // G)
    assert np.array_equal(tok_off[:, :P] & 0xFFFF, np.cumsum(r, 1) - r)
    assert np.array_equal(tok_off[:, :P] >> 16, np.cumsum(g, 1) - g)
    pad = lambda x: (x + 15) // 16 * 16
    sizes = Hkv * (2 * pad(r.sum(1) // 2) + 2 * pad(4 * g.sum(1)))
    assert np.array_equal(page_off, np.concatenate([[0], np.cumsum(sizes)[:-1]]))
    assert len(pool) == sizes.sum()
    # algorithmic bytes: codes r/2 + 4 bytes per group, for K and V, per (token, kv head), plus padding
    tok_bytes = Hkv * 2 * (r.sum() // 2 + 4 * g.sum())
    assert 0 <= len(pool) - tok_bytes <= w.n_pages * Hkv * 4 * 15


def test_compress_rejects_bad_input():
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=512)
    inp = synth.make_inputs(w)
    bad = dict(inp, block_table=inp["block_table"].clone())
    bad["block_table"][1, 0] = bad["block_table"][0, 0]          # two blocks on one page
    with pytest.raises(ValueError):
        oracle_cache(w, bad)
    bad = dict(inp, ranks=inp["ranks"].clone())
    bad["ranks"][0, 3] = 12                                         # not a multiple of 8
    with pytest.raises(ValueError):
        oracle_cache(w, bad)


# ---------------------------------------------------------------- projection (prefill side)

def test_projection_identities_on_an_exact_orthonormal_basis():
    # columns of the Sylvester matrix H_64 / 8: entries +-1/8, exact in bf16, exactly orthonormal
    w = synth.WORKLOADS["llama8b_layer_8k"].scaled(B=1, T=64, head_dim=64, n_q_heads=4, n_kv_heads=1,
                                                    r_k=16, r_v=24, group=8, page_size=64)
    H = torch.tensor(scipy.linalg.hadamard(64) / 8.0, dtype=torch.float32)
    Bk = H[:, :16].to(torch.bfloat16)[None]; Bv = H[:, 16:40].to(torch.bfloat16)[None]
    c = torch.randn(1, 64, 1, 16); cv = torch.randn(1, 64, 1, 24)
    k = (c @ H[:, :16].T).contiguous(); v = (cv @ H[:, 16:40].T).contiguous()
    lat_k, lat_v, _, _ = ref.project(layout(w), [64], 64, None, k.numpy(), v.numpy(), np_u16(Bk), np_u16(Bv))
    assert np.allclose(lat_k, c.numpy(), atol=1e-6) and np.allclose(lat_v, cv.numpy(), atol=1e-6)
    # truncation residual of a general vector is orthogonal to the basis, and H^T H e = e; the basis is
    # block-diagonal(H_64, H_64) / 8 (exact in bf16, exactly orthonormal), split between K and V columns
    w2 = synth.WORKLOADS["residual_128k"].scaled(B=1, T=8, page_size=64)
    H128 = scipy.linalg.hadamard(128) / math.sqrt(128)
    Q = torch.block_diag(H, H)
    Bk = Q[:, :48].to(torch.bfloat16).expand(8, -1, -1).contiguous()
    Bv = Q[:, 48:112].to(torch.bfloat16).expand(8, -1, -1).contiguous()
    kk = torch.randn(1, 8, 8, 128); vv = torch.randn(1, 8, 8, 128)
    lk, lv, rk, rv = ref.project(layout(w2), [8], 8, None, kk.numpy(), vv.numpy(), np_u16(Bk), np_u16(Bv))
    for lat, res, Bm, x in ((lk, rk, Bk, kk), (lv, rv, Bv, vv)):
        Bm = Bm.double().numpy()
        e = res.astype(np.float64) @ H128                         # back from the rotated domain
        assert np.allclose(np.einsum("thd,hdr->thr", e[0], Bm), 0, atol=1e-6)
        recon = np.einsum("thr,hdr->thd", lat[0].astype(np.float64), Bm) + e[0]
        assert np.allclose(recon, x[0].numpy(), atol=1e-6)


# ---------------------------------------------------------------- layer axis of the block-shared mode

def dequant_shared_latent(lat, group):
    """The stored block-shared latent as the decode must see it: each group of `group` coordinates quantized by
    the INT4 quantizer and dequantized as code * scale + zero (computed here from the quantizer's outputs)."""
    T, n = lat.shape
    S, Z, Q = ref.quant_int4(lat.reshape(T * n // group, group))
    deq = Q * S.view(np.float16).astype(np.float64)[:, None] + Z.view(np.float16).astype(np.float64)[:, None]
    return deq.reshape(T, n)


@pytest.mark.parametrize("n_layers", [2, 4])
def test_shared_layers_each_use_their_own_up_projection_and_query(n_layers):
    # BellowsKV, "Share the Input, Not the Cache": every layer of the block rebuilds its keys and values from the
    # one stored latent through its own up-projection.  Layer l's output is textbook attention with q[l], keys
    # W_k[l]^T c and values W_v[l]^T c, everything here computed in numpy from the quantizer's outputs; the
    # per-layer W and q all differ, so a wrong layer stride in the oracle reads another layer's operands.
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=2, T=300, n_layers=n_layers, page_size=64,
                                                     shuffle_pages=True)
    inp = synth.make_inputs(w, seq_len=[300, 171])
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    Wk = inp["wk"].double().numpy(); Wv = inp["wv"].double().numpy()
    q = np_f32(inp["q"])
    assert out.shape == (n_layers, w.B, 32, 128)
    for b in range(w.B):
        T = int(inp["seq_len"][b])
        c = dequant_shared_latent(np_f32(inp["lat_k"])[b, :T], w.group)
        for l in range(n_layers):
            for h in (0, 5, 7):
                k = c @ Wk[l][:, 128 * h: 128 * h + 128]
                v = c @ Wv[l][:, 128 * h: 128 * h + 128]
                want = sdpa64(rope_complex(q[l, b, 4 * h: 4 * h + 4], T, w.rope_theta),
                              rope_complex(k, np.arange(T), w.rope_theta), v)
                assert np.allclose(out[l, b, 4 * h: 4 * h + 4], want, rtol=0, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_shared_layers_with_embedded_per_layer_bases_equal_per_head_mode(bits):
    # two layers, each with its own per-head bases embedded block-diagonally in W[l]: layer l of the shared
    # decode equals the per-head decode of the same latents with layer l's bases and query, at each code width
    # (a shared group of 64 coordinates is one head's group, so both modes quantize alike)
    wp = synth.WORKLOADS["llama8b_layer_8k"].scaled(T=200, r_k=64, r_v=64, group=64, page_size=64, latent_bits=bits)
    per_layer = []
    for l in range(2):
        inp = synth.make_inputs(wp.scaled(seed=100 + l))
        per_layer.append(inp)
    base = per_layer[0]
    lat = base["lat_k"]
    ws = synth.WORKLOADS["shared_latent_32k"].scaled(B=1, T=200, n_layers=2, page_size=64, latent_bits=bits)
    Hkv, d = 8, 128
    W = {n: torch.zeros(2, 512, Hkv * d, dtype=torch.bfloat16) for n in ("wk", "wv")}
    for l in range(2):
        for name in ("wk", "wv"):
            for h in range(Hkv):
                W[name][l, 64 * h: 64 * h + 64, d * h: d * h + d] = per_layer[l][name][h].T
    q = torch.stack([per_layer[l]["q"] for l in range(2)])
    inps = dict(base, lat_k=lat.reshape(1, 200, 512).contiguous(), lat_v=None, wk=W["wk"], wv=W["wv"], q=q)
    out_s = oracle_decode(ws, inps, oracle_cache(ws, inps))
    for l in range(2):
        inpl = dict(per_layer[l], lat_k=lat, lat_v=lat.clone())
        out_p = oracle_decode(wp, inpl, oracle_cache(wp, inpl))
        assert np.allclose(out_s[l], out_p, rtol=0, atol=1e-13 * np.abs(out_p).max())


# ---------------------------------------------------------------- projection under per-token ranks

def test_variable_rank_projection_truncates_to_each_tokens_rank():
    # VarRate, "Method": a token of rank r keeps r coordinates.  On an exactly orthonormal basis (the Sylvester
    # blocks H_64 / 8, entries +-1/8, exact in bf16) the projection of token t must be B_r^T x in its first r
    # coordinates and zero past them, and the residual must be H (x - B_r B_r^T x) over r columns only: the
    # columns r..cap-1 are left in the residual.  All expected values are numpy here.
    w = synth.WORKLOADS["residual_128k"].scaled(B=2, T=40, page_size=64, r_k=64, r_v=64, variable_rank=True,
                                                rank_choices=(8, 16, 32, 64), rank_probs=(0.4, 0.3, 0.2, 0.1))
    H64 = scipy.linalg.hadamard(64) / 8.0
    Q = np.kron(np.eye(2), H64)                                  # 128 x 128, exactly orthonormal
    rng = np.random.default_rng(3)
    perms = [rng.permutation(128) for _ in range(8)]             # a different column choice per KV head
    Bk = torch.tensor(np.stack([Q[:, p[:64]] for p in perms]), dtype=torch.float32).to(torch.bfloat16)
    Bv = torch.tensor(np.stack([Q[:, p[64:]] for p in perms]), dtype=torch.float32).to(torch.bfloat16)
    ranks = synth.make_inputs(w)["ranks"]
    seq = np.array([40, 23], np.int32)
    g = torch.Generator().manual_seed(11)
    kk = torch.randn(2, 40, 8, 128, generator=g); vv = torch.randn(2, 40, 8, 128, generator=g)
    lk, lv, rk, rv = ref.project(layout(w), seq, 40, np_any(ranks), kk.numpy(), vv.numpy(), np_u16(Bk), np_u16(Bv))
    H128 = scipy.linalg.hadamard(128) / math.sqrt(128)
    seen = set()
    for lat, res, Bm, x in ((lk, rk, Bk, kk), (lv, rv, Bv, vv)):
        Bm = Bm.double().numpy()                                 # [Hkv, d, 64]
        for b in range(2):
            for t in range(int(seq[b])):
                r = int(ranks[b, t]); seen.add(r)
                xt = x[b, t].double().numpy()                    # [Hkv, d]
                c = np.einsum("hd,hdr->hr", xt, Bm[:, :, :r])
                assert np.allclose(lat[b, t, :, :r], c, rtol=0, atol=1e-5)
                assert not lat[b, t, :, r:].any()
                e = xt - np.einsum("hr,hdr->hd", c, Bm[:, :, :r])
                assert np.allclose(res[b, t], e @ H128, rtol=0, atol=1e-5)
                if r < 64:                                       # the dropped columns stay in the residual
                    assert np.abs(np.einsum("hd,hdr->hr", e, Bm[:, :, r:])).max() > 1e-2
            for t in range(int(seq[b]), 40):                     # rows past the length are left alone
                assert not lat[b, t].any() and not res[b, t].any()
    assert seen == {8, 16, 32, 64}


# ---------------------------------------------------------------- rotated residual on the block-shared latent
# (JoLT index, Abstract, and JoLT thesis, "How JoLT works": the Tucker form plus a rotated low-bit residual; each
# layer and head keeps its own residual of what its up-projection leaves)

def _shared_res_case(n_layers=2, T=200, seq=(200, 77), B=2):
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=B, T=T, n_layers=n_layers, page_size=64, residual_bits=2,
                                                     residual_std=0.3, shuffle_pages=True)
    inp = synth.make_inputs(w, seq_len=list(seq))
    return w, inp


def test_shared_zero_residual_equals_no_residual():
    w, inp = _shared_res_case()
    inp["res_k"] = torch.zeros_like(inp["res_k"]); inp["res_v"] = torch.zeros_like(inp["res_v"])
    out_r = oracle_decode(w, inp, oracle_cache(w, inp))
    wn = w.scaled(residual_bits=0)
    inpn = dict(inp, res_k=None, res_v=None)
    out_n = oracle_decode(wn, inpn, oracle_cache(wn, inpn))
    assert np.array_equal(out_r, out_n)


def test_shared_residual_record_holds_the_quantizer_outputs():
    # read from the format description alone: after the latent's two sections, Kr and Vr hold one part of P x 32
    # code bytes per (layer, kv head) in layer-major order, then Ks and Vs one part of P fp16 scales (padded to
    # 16 bytes) per (layer, kv head); residual element i is bits 2(i % 4).. of byte i / 4
    w, inp = _shared_res_case(n_layers=3)
    pool, page_off, _, _ = oracle_cache(w, inp)
    bt = np_any(inp["block_table"])
    P, Hkv, NL = w.page_size, w.n_kv_heads, w.n_layers
    pad = lambda x: (x + 15) // 16 * 16
    lat_bytes = pad(P * 256) + pad(P * 4 * (512 // w.group))
    n = NL * Hkv
    assert np.array_equal(page_off, np.arange(w.n_pages) * (lat_bytes + 2 * n * (P * 32 + pad(2 * P))))
    for (b, t, l, h) in [(0, 0, 0, 0), (0, 199, 2, 7), (1, 76, 1, 3), (1, 64, 0, 5), (0, 130, 2, 0)]:
        rec = int(page_off[int(bt[b, t // P])]) + lat_bytes
        s, idx = t % P, l * Hkv + h
        for part, name in ((0, "res_k"), (1, "res_v")):
            by = pool[rec + (part * n + idx) * P * 32 + s * 32: rec + (part * n + idx) * P * 32 + (s + 1) * 32]
            codes = (by[:, None] >> (2 * np.arange(4))) & 3
            sc = pool[rec + 2 * n * P * 32 + (part * n + idx) * pad(2 * P) + 2 * s:][:2].view(np.uint16)[0]
            S, Q = ref.quant_res2(np_f32(inp[name])[b, t, l, h][None])
            assert np.array_equal(codes.reshape(-1), Q[0]) and sc == S[0], (b, t, l, h, name)


def test_shared_residual_adds_each_layer_and_heads_hadamard_of_its_codes():
    # keys W_k[l]^T c + H e_k[l, h] and values W_v[l]^T c + H e_v[l, h], e the dequantized 2-bit codes of that
    # layer and head (from the quantizer's outputs), H from scipy's Sylvester matrix; textbook attention in numpy
    w, inp = _shared_res_case(n_layers=2)
    out = oracle_decode(w, inp, oracle_cache(w, inp))
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    Wk = inp["wk"].double().numpy(); Wv = inp["wv"].double().numpy()
    q = np_f32(inp["q"])
    for b in range(w.B):
        T = int(inp["seq_len"][b])
        c = dequant_shared_latent(np_f32(inp["lat_k"])[b, :T], w.group)
        for l in range(w.n_layers):
            for h in (0, 6):
                kv = []
                for name, W in (("res_k", Wk), ("res_v", Wv)):
                    S, Q = ref.quant_res2(np_f32(inp[name])[b, :T, l, h])
                    e = (Q.astype(np.float64) - 1.5) * S.view(np.float16).astype(np.float64)[:, None]
                    kv.append(c @ W[l][:, 128 * h: 128 * h + 128] + e @ H.T)
                want = sdpa64(rope_complex(q[l, b, 4 * h: 4 * h + 4], T, w.rope_theta),
                              rope_complex(kv[0], np.arange(T), w.rope_theta), kv[1])
                assert np.allclose(out[l, b, 4 * h: 4 * h + 4], want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_shared_residual_with_embedded_per_layer_bases_equals_per_head_residual_mode():
    # two layers, each with its own per-head bases embedded block-diagonally in W[l] and its own residuals: layer l
    # of the shared decode equals the per-head residual decode of the same latents and layer l's residuals
    wp = synth.WORKLOADS["residual_128k"].scaled(B=1, T=200, r_k=64, r_v=64, group=64, page_size=64)
    per_layer = [synth.make_inputs(wp.scaled(seed=200 + l)) for l in range(2)]
    base = per_layer[0]
    lat = base["lat_k"]
    ws = synth.WORKLOADS["shared_latent_32k"].scaled(B=1, T=200, n_layers=2, page_size=64, residual_bits=2)
    Hkv, d = 8, 128
    W = {n: torch.zeros(2, 512, Hkv * d, dtype=torch.bfloat16) for n in ("wk", "wv")}
    for l in range(2):
        for name in ("wk", "wv"):
            for h in range(Hkv):
                W[name][l, 64 * h: 64 * h + 64, d * h: d * h + d] = per_layer[l][name][h].T
    q = torch.stack([per_layer[l]["q"] for l in range(2)])
    res = {n: torch.stack([per_layer[l][n] for l in range(2)], dim=2).contiguous() for n in ("res_k", "res_v")}
    inps = dict(base, lat_k=lat.reshape(1, 200, 512).contiguous(), lat_v=None, wk=W["wk"], wv=W["wv"], q=q, **res)
    out_s = oracle_decode(ws, inps, oracle_cache(ws, inps))
    for l in range(2):
        inpl = dict(per_layer[l], lat_k=lat, lat_v=lat.clone())
        out_p = oracle_decode(wp, inpl, oracle_cache(wp, inpl))
        assert np.allclose(out_s[l], out_p, rtol=0, atol=1e-13 * np.abs(out_p).max())
