"""Block-level eviction on the GPU: kvc_evict_select against the eviction oracle (bit for bit: the block scores
are fp32 sums in the same order on both sides, and the rest is integer work), and the block-shared decode under
a keep mask against the oracle's masked attention (max |out - ref| <= 2e-3 max |ref|, the bound of every
decode path)."""
import numpy as np
import pytest
import torch

from oracle import evict as E
from oracle import ref
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_layout, rel_err
from tests.helpers import layout, np_any, np_f32, np_u16, oracle_cache

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


def _select_case(scores, seq, ratio):
    print(f"[evict] select scores={tuple(scores.shape)} seq={list(seq)[:6]} ratio={ratio}", flush=True)
    got = kvc.evict_select(scores.cuda().contiguous(), torch.tensor(seq, dtype=torch.int32).cuda(), ratio)
    again = kvc.evict_select(scores.cuda().contiguous(), torch.tensor(seq, dtype=torch.int32).cuda(), ratio)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    want = E.keep_mask(scores.numpy(), seq, ratio)
    assert np.array_equal(_u32(got), want), ratio


def test_select_ragged_ties_and_layers():
    B, T = 5, 3000
    seq = [3000, 2999, 1, 0, 1777]
    for n_layers in (1, 2, 4):
        s = torch.stack([synth.make_salience(B, T, seed=40 + l) for l in range(n_layers)])
        s[:, 0, :700] = 1.0                       # a block of ties across chunk boundaries
        s[:, 1, 100:200] = 0.0
        s[0, 1, 300] = -0.0                       # minus zero equals zero
        for ratio in (0.3, 1e-9, 1.0, 0.5):
            _select_case(s, seq, ratio)


def test_select_many_ties_integer_scores():
    g = torch.Generator().manual_seed(7)
    s = torch.randint(0, 4, (3, 4, 5000), generator=g).float()
    _select_case(s, [5000, 4097, 1024, 33], 0.37)
    _select_case(s, [5000, 4097, 1024, 33], 0.999)


def test_select_longer_than_the_lds_stage():
    # past 32768 tokens per sequence the keys are recomputed from the scores in every pass
    s = torch.stack([synth.make_salience(2, 40000, seed=60 + l) for l in range(2)])
    s[:, 1, 35000:] = 2.0
    _select_case(s, [40000, 36001], 0.2)


def test_select_full_size():
    w = synth.WORKLOADS["shared_latent_32k_evict30"]
    inp = synth.make_inputs(w)
    _select_case(inp["layer_scores"], [w.T] * w.B, w.evict_ratio)


def _masked_oracle(w, inp, cache, mask, sel_b=None, sel_h=None):
    pool, page_off, tok_rank, tok_off = cache
    return ref.decode_attn(layout(w), np_any(inp["block_table"]), np_any(inp["seq_len"]), np_any(inp["q_pos"]), pool,
                           page_off, tok_rank, tok_off, np_f32(inp["q"]), np_u16(inp["wk"]), np_u16(inp["wv"]),
                           sel_b, sel_h, keep=mask)


def _masks(w, seq, rng):
    words = -(-w.T // 32)
    kept = rng.random((w.B, words * 32)) < 0.3
    kept[:, :64] = False                          # the first two super-tiles evicted: no reference yet
    kept[0, :160] = False                         # with four splits of five super-tiles, split 0 holds none
    m = {"random": kept}
    one = np.zeros_like(kept)
    one[0, 417] = True
    one[1, 5] = True
    m["one token"] = one
    none = kept.copy()
    none[1] = False                               # sequence 1 keeps no token: zero output
    m["none in one sequence"] = none
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    return {k: (v.reshape(w.B, words, 32).astype(np.uint64) * weights).sum(-1).astype(np.uint32) for k, v in m.items()}


@pytest.mark.parametrize("num_splits", [0, 4])
def test_masked_decode_matches_oracle(num_splits):
    w = synth.WORKLOADS["shared_latent_32k_evict30"].scaled(B=2, T=600)
    seq = [600, 333]
    inp = synth.make_inputs(w, seq_len=seq)
    cache = oracle_cache(w, inp)
    d = dev(inp)
    gc = gpu_cache(w, d)
    L = gpu_layout(w)
    plain = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T, q_pos=d["q_pos"],
                            num_splits=num_splits)
    words = -(-w.T // 32)
    ones = torch.full((w.B, words), -1, dtype=torch.int32, device="cuda")
    all_kept = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                               q_pos=d["q_pos"], num_splits=num_splits, keep_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(plain, all_kept)
    masks = _masks(w, seq, np.random.default_rng(5))
    # and the masks the eviction decision gives for the workload's layer scores, i.i.d. and clustered in runs
    # of 64 tokens (whole super-tiles evicted)
    masks["evict 30%"] = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    masks["evict 30% clustered"] = E.keep_mask(synth.make_layer_scores(w.scaled(evict_cluster=64)).numpy(), seq,
                                               w.evict_ratio)
    for name, m in masks.items():
        print(f"[evict] masked decode '{name}' num_splits={num_splits}", flush=True)
        want = _masked_oracle(w, inp, cache, m)
        gm = torch.from_numpy(m.view(np.int32)).cuda()
        out = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                              q_pos=d["q_pos"], num_splits=num_splits, keep_mask=gm)
        torch.cuda.synchronize()
        if name == "random":  # the split variant under a mask, on a W with zero halves: the plain masked bits
            wk2, wv2 = d["wk"].clone(), d["wv"].clone()
            wk2[:, 256:] = 0
            wv2[:, :256] = 0
            a = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], wk2, wv2, w.T, q_pos=d["q_pos"],
                                num_splits=num_splits, keep_mask=gm)
            s = kvc.decode_attn(L, gc, d["block_table"], d["seq_len"], d["q"], wk2, wv2, w.T, q_pos=d["q_pos"],
                                num_splits=num_splits, keep_mask=gm, kv_split=256)
            torch.cuda.synchronize()
            assert torch.equal(a, s)
        o = out.cpu().double().numpy()
        assert not np.isnan(o).any()
        if name == "none in one sequence":
            assert np.all(o[:, 1] == 0)
            assert rel_err(out[:, :1], want[:, :1]) <= TOL
        else:
            assert rel_err(out, want) <= TOL, name


def test_evict_then_decode_full_size_sampled():
    w = synth.WORKLOADS["shared_latent_32k_evict30"]
    inp = synth.make_inputs(w)
    d = dev(inp)
    seq = [w.T] * w.B
    print("[evict] full size: select, compress, decode", flush=True)
    gm = kvc.evict_select(d["layer_scores"], d["seq_len"], w.evict_ratio)
    gc = gpu_cache(w, d)
    out = kvc.decode_attn(gpu_layout(w), gc, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                          q_pos=d["q_pos"], keep_mask=gm)
    torch.cuda.synchronize()
    m = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    assert np.array_equal(_u32(gm), m)
    print("[evict] full size: oracle compress and masked decode of sequence 3, kv head 4", flush=True)
    cache = oracle_cache(w, inp)
    sel_b = np.zeros(w.B, np.uint8); sel_b[3] = 1
    sel_h = np.zeros(w.n_kv_heads, np.uint8); sel_h[4] = 1
    want = _masked_oracle(w, inp, cache, m, sel_b, sel_h)
    assert rel_err(out, want) <= TOL


# ---------------------------------------------------------------- compaction and the decode over positions

def _compact_pair(w, inp, d, mask_np, seed=11):
    """GPU compaction of the cache compressed from inp under mask_np, and the oracle's from the oracle's cache
    (the two source pools are bit-identical: compression is tested bit for bit).  Returns the GPU outputs and
    the oracle's (pool, tok_pos, out_len)."""
    gc = gpu_cache(w, d)
    rec = int(gc.page_off[1].item() - gc.page_off[0].item())
    dst = kvc.DeviceCache(gc.layout, torch.full_like(gc.pool, 0xAB), torch.arange(w.n_pages, dtype=torch.int64,
                          device="cuda") * rec, None, None, torch.zeros(2, dtype=torch.int64, device="cuda"), w.n_pages)
    obt = torch.from_numpy(np.random.default_rng(seed).permutation(w.n_pages).astype(np.int32).reshape(w.B, -1))
    gm = torch.from_numpy(np.ascontiguousarray(mask_np).view(np.int32)).cuda()
    out_len, tok_pos = kvc.evict_compact(gpu_layout(w), gc, dst, d["block_table"], d["seq_len"], gm, obt.cuda())
    torch.cuda.synchronize()
    cache = oracle_cache(w, inp)
    want = E.compact(w.r_k, w.latent_bits, w.group, w.page_size, inp["block_table"].numpy(),
                     inp["seq_len"].numpy(), mask_np, cache[0], cache[1], obt.numpy(),
                     np.arange(w.n_pages, dtype=np.int64) * rec, np.full(gc.pool.numel(), 0xAB, np.uint8))
    return gc, dst, obt.cuda(), out_len, tok_pos, gm, cache, want


@pytest.mark.parametrize("bits", [4, 3])
def test_compaction_matches_oracle_bit_for_bit(bits):
    w = synth.WORKLOADS["shared_latent_32k_evict30"].scaled(B=2, T=700, page_size=64, latent_bits=bits)
    seq = [700, 333]
    inp = synth.make_inputs(w, seq_len=seq)
    d = dev(inp)
    masks = _masks(w, seq, np.random.default_rng(8))
    masks["evict 30%"] = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    masks["all"] = np.full_like(masks["random"], 0xFFFFFFFF)
    for name, m in masks.items():
        print(f"[compact] bits={bits} mask '{name}'", flush=True)
        gc, dst, obt, out_len, tok_pos, gm, cache, (pool2, pos2, len2) = _compact_pair(w, inp, d, m)
        assert np.array_equal(out_len.cpu().numpy(), len2), name
        assert np.array_equal(tok_pos.cpu().numpy(), pos2), name
        assert np.array_equal(dst.pool.cpu().numpy(), pool2), name
        if name == "all":  # keeping everything moves every token to its own slot
            assert np.array_equal(len2, seq)


@pytest.mark.parametrize("num_splits", [0, 3])
def test_compacted_decode_matches_masked_oracle(num_splits):
    w = synth.WORKLOADS["shared_latent_32k_evict30"].scaled(B=2, T=700, page_size=64)
    seq = [700, 333]
    inp = synth.make_inputs(w, seq_len=seq)
    d = dev(inp)
    L = gpu_layout(w)
    masks = _masks(w, seq, np.random.default_rng(5))
    masks["evict 30%"] = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    masks["evict 30% clustered"] = E.keep_mask(synth.make_layer_scores(w.scaled(evict_cluster=64)).numpy(), seq,
                                               w.evict_ratio)
    sparse = np.random.default_rng(3).random((w.B, 32 * masks["random"].shape[1])) < 0.03
    masks["3% (tiles closed by the span)"] = (sparse.reshape(w.B, -1, 32).astype(np.uint64)
                                              << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    for name, m in masks.items():
        print(f"[compact] decode over positions, mask '{name}' num_splits={num_splits}", flush=True)
        gc, dst, obt, out_len, tok_pos, gm, cache, _ = _compact_pair(w, inp, d, m)
        want = _masked_oracle(w, inp, cache, m)
        args = (L, dst, obt, out_len, d["q"], d["wk"], d["wv"], w.T)
        out = kvc.decode_attn(*args, q_pos=d["q_pos"], num_splits=num_splits, tok_pos=tok_pos)
        again = kvc.decode_attn(*args, q_pos=d["q_pos"], num_splits=num_splits, tok_pos=tok_pos)
        na = kvc.decode_attn_noalloc(*args, q_pos=d["q_pos"], num_splits=num_splits, tok_pos=tok_pos)
        torch.cuda.synchronize()
        assert torch.equal(out, again) and torch.equal(out, na)
        o = out.cpu().double().numpy()
        assert not np.isnan(o).any()
        if name == "none in one sequence":
            assert int(out_len[1].item()) == 0 and np.all(o[:, 1] == 0)
            assert rel_err(out[:, :1], want[:, :1]) <= TOL
        else:
            assert rel_err(out, want) <= TOL, name
        if name == "random":  # the split-latent variant over positions gives the plain variant's bits
            wk2, wv2 = d["wk"].clone(), d["wv"].clone()
            wk2[:, 256:] = 0
            wv2[:, :256] = 0
            a = kvc.decode_attn(L, dst, obt, out_len, d["q"], wk2, wv2, w.T, q_pos=d["q_pos"], num_splits=num_splits,
                                tok_pos=tok_pos)
            s = kvc.decode_attn(L, dst, obt, out_len, d["q"], wk2, wv2, w.T, q_pos=d["q_pos"], num_splits=num_splits,
                                tok_pos=tok_pos, kv_split=256)
            torch.cuda.synchronize()
            assert torch.equal(a, s)


def test_compacted_decode_int3():
    w = synth.WORKLOADS["shared_latent_32k_evict30"].scaled(B=2, T=600, page_size=128, latent_bits=3)
    seq = [600, 411]
    inp = synth.make_inputs(w, seq_len=seq)
    d = dev(inp)
    m = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    gc, dst, obt, out_len, tok_pos, gm, cache, _ = _compact_pair(w, inp, d, m)
    out = kvc.decode_attn(gpu_layout(w), dst, obt, out_len, d["q"], d["wk"], d["wv"], w.T, q_pos=d["q_pos"],
                          tok_pos=tok_pos)
    torch.cuda.synchronize()
    assert rel_err(out, _masked_oracle(w, inp, cache, m)) <= TOL


def test_compact_then_decode_full_size_sampled():
    w = synth.WORKLOADS["shared_latent_32k_evict30"]
    inp = synth.make_inputs(w)
    d = dev(inp)
    seq = [w.T] * w.B
    print("[compact] full size: select, compress, compact, decode over positions", flush=True)
    gm = kvc.evict_select(d["layer_scores"], d["seq_len"], w.evict_ratio)
    gc = gpu_cache(w, d)
    rec = int(gc.page_off[1].item() - gc.page_off[0].item())
    dst = kvc.DeviceCache(gc.layout, torch.zeros_like(gc.pool), torch.arange(w.n_pages, dtype=torch.int64,
                          device="cuda") * rec, None, None, torch.zeros(2, dtype=torch.int64, device="cuda"), w.n_pages)
    obt = d["block_table"].flip(1).contiguous()
    out_len, tok_pos = kvc.evict_compact(gpu_layout(w), gc, dst, d["block_table"], d["seq_len"], gm, obt)
    out = kvc.decode_attn(gpu_layout(w), dst, obt, out_len, d["q"], d["wk"], d["wv"], w.T, q_pos=d["q_pos"],
                          tok_pos=tok_pos)
    masked = kvc.decode_attn(gpu_layout(w), gc, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                             q_pos=d["q_pos"], keep_mask=gm)
    torch.cuda.synchronize()
    m = E.keep_mask(inp["layer_scores"].numpy(), seq, w.evict_ratio)
    assert np.array_equal(_u32(gm), m)
    # the compacted length: every kept token once, tiles of 32 within 4 blocks (layout from the oracle's rule)
    lens = out_len.cpu().numpy()
    for b in range(w.B):
        want_slots = E.compact_slots(np.nonzero(E.mask_bits(m, w.T)[b])[0])
        assert lens[b] == len(want_slots)
        assert np.array_equal(tok_pos[b, : lens[b]].cpu().numpy(), want_slots)
    print(f"[compact] full size: {lens.tolist()} slots of {w.T}", flush=True)
    assert rel_err(out, masked.cpu().double().numpy()) <= TOL
    print("[compact] full size: oracle masked decode of sequence 1, kv head 6", flush=True)
    cache = oracle_cache(w, inp)
    sel_b = np.zeros(w.B, np.uint8); sel_b[1] = 1
    sel_h = np.zeros(w.n_kv_heads, np.uint8); sel_h[6] = 1
    want = _masked_oracle(w, inp, cache, m, sel_b, sel_h)
    assert rel_err(out, want) <= TOL
