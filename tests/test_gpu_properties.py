"""GPU decode properties: determinism, split invariance, page-table invariance, edge cases,
query dtype/position handling, sharp queries, and compression from dense K/V."""
import numpy as np
import pytest
import torch

from oracle import ref
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_decode, gpu_layout, rel_err
from tests.helpers import layout, np_any, np_f32, np_u16, oracle_cache, oracle_decode

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(w, inp, num_splits=0):
    d = dev(inp)
    out = gpu_decode(w, d, gpu_cache(w, d), num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("name", ["varrank_paged_32k", "residual_128k"])
def test_deterministic_and_page_table_invariant(name):
    w = synth.WORKLOADS[name].scaled(B=3, T=3000)
    inp = synth.make_inputs(w, seq_len=[3000, 2999, 1234])
    a = _run(w, inp)
    b = _run(w, inp)
    assert torch.equal(a, b)
    ident = dict(inp, block_table=torch.arange(w.n_pages, dtype=torch.int32).view(w.B, -1))
    c = _run(w, ident)
    assert torch.equal(a, c), "summation order must depend on logical positions only"


@pytest.mark.parametrize("name", ["varrank_paged_32k", "residual_128k", "shared_latent_32k"])
def test_split_sweep(name):
    kw = dict(B=2, T=2500) if name != "shared_latent_32k" else dict(B=1, T=2500, n_layers=2)
    w = synth.WORKLOADS[name].scaled(**kw)
    inp = synth.make_inputs(w)
    ref_out = oracle_decode(w, inp, oracle_cache(w, inp))
    outs = [_run(w, inp, s) for s in (1, 2, 3, 7, 0)]
    for o in outs:
        assert rel_err(o, ref_out) <= TOL


@pytest.mark.parametrize("name", ["varrank_paged_32k", "residual_128k"])
@pytest.mark.parametrize("seq", [[1], [31, 32, 33], [255, 256, 257, 511]])
def test_ragged_lengths_and_tails(name, seq):
    w = synth.WORKLOADS[name].scaled(B=len(seq), T=max(seq), page_size=128)
    inp = synth.make_inputs(w, seq_len=seq)
    ref_out = oracle_decode(w, inp, oracle_cache(w, inp))
    assert rel_err(_run(w, inp), ref_out) <= TOL


@pytest.mark.parametrize("name", ["llama8b_layer_8k", "residual_128k"])
def test_single_token_sequence_returns_its_value(name):
    w = synth.WORKLOADS[name].scaled(B=2, T=64, page_size=64)
    inp = synth.make_inputs(w, seq_len=[1, 64])
    ref_out = oracle_decode(w, inp, oracle_cache(w, inp))
    out = _run(w, inp).double().numpy()
    assert np.abs(out[0] - ref_out[0]).max() <= TOL * np.abs(ref_out[0]).max()


@pytest.mark.parametrize("name", ["llama8b_layer_8k", "residual_128k"])
def test_query_dtype_and_explicit_positions(name):
    w = synth.WORKLOADS[name].scaled(B=2, T=900, q_bf16=False)
    inp = synth.make_inputs(w, seq_len=[900, 500])
    inp["q_pos"] = torch.tensor([123456, 7], dtype=torch.int32)
    ref_out = oracle_decode(w, inp, oracle_cache(w, inp))
    assert rel_err(_run(w, inp), ref_out) <= TOL


def test_sharp_queries():
    # queries 32x larger than the workloads' (score std ~0.5): softmax far from uniform
    w = synth.WORKLOADS["residual_128k"].scaled(B=2, T=1500)
    inp = synth.make_inputs(w)
    inp["q"] = (inp["q"].float() * 32).to(torch.bfloat16)
    ref_out = oracle_decode(w, inp, oracle_cache(w, inp))
    assert rel_err(_run(w, inp), ref_out) <= TOL


@pytest.mark.parametrize("name,kw", [("residual_128k", dict(B=2, T=600)),
                                     ("varrank_paged_32k", dict(B=2, T=600))])
def test_compress_from_dense(name, kw):
    # dense pre-RoPE K/V = B c + noise; the GPU projects, forms the rotated truncation residual and
    # quantizes.  (1) its fp32 projections agree with the oracle's fp64 ones to fp32 rounding;
    # (2) quantizing the GPU's own fp32 projections with the oracle compressor reproduces the GPU
    # pool bit for bit (the quantizer is the same function of the same fp32 inputs).
    w = synth.WORKLOADS[name].scaled(**kw)
    inp = synth.make_inputs(w, seq_len=[kw["T"], kw["T"] - 77])
    g = torch.Generator().manual_seed(5)
    Bk = inp["wk"].float(); Bv = inp["wv"].float()
    k = torch.einsum("hdr,bthr->bthd", Bk, inp["lat_k"]) + 0.05 * torch.randn(w.B, w.T, w.n_kv_heads, 128, generator=g)
    v = torch.einsum("hdr,bthr->bthd", Bv, inp["lat_v"]) + 0.05 * torch.randn(w.B, w.T, w.n_kv_heads, 128, generator=g)
    L = gpu_layout(w)
    cache = kvc.DeviceCache.allocate(L, w.n_pages)
    lk = torch.zeros_like(inp["lat_k"]).cuda(); lv = torch.zeros_like(inp["lat_v"]).cuda()
    rk = torch.zeros(w.B, w.T, w.n_kv_heads, 128).cuda() if w.residual_bits else None
    rv = torch.zeros(w.B, w.T, w.n_kv_heads, 128).cuda() if w.residual_bits else None
    d = dev(inp)
    kvc.compress(L, cache, d["block_table"], d["seq_len"], w.T, ranks=d["ranks"], lat_k=lk, lat_v=lv, res_k=rk,
                 res_v=rv, k=k.cuda().contiguous(), v=v.cuda().contiguous(), basis_k=d["wk"], basis_v=d["wv"])
    torch.cuda.synchronize()
    olk, olv, ork, orv = ref.project(layout(w), np_any(inp["seq_len"]), w.T, np_any(inp["ranks"]), k.numpy(),
                                     v.numpy(), np_u16(inp["wk"]), np_u16(inp["wv"]))
    sl = np_any(inp["seq_len"])
    for got, want in ((lk, olk), (lv, olv), (rk, ork), (rv, orv)):
        if got is None:
            continue
        g_ = got.cpu().numpy()
        for b in range(w.B):
            assert np.allclose(g_[b, :sl[b]], want[b, :sl[b]], rtol=0, atol=1e-5 * np.abs(want).max())
    pool, page_off, _, _ = ref.compress(layout(w), np_any(inp["block_table"]), sl, w.T, np_any(inp["ranks"]),
                                        lk.cpu().numpy(), lv.cpu().numpy(),
                                        None if rk is None else rk.cpu().numpy(),
                                        None if rv is None else rv.cpu().numpy(), w.n_pages,
                                        ref.page_bytes_uniform(layout(w)) * w.n_pages)
    assert np.array_equal(cache.pool[: len(pool)].cpu().numpy(), pool)
    assert np.array_equal(cache.page_off.cpu().numpy(), page_off)


@pytest.mark.parametrize("name", ["varrank_paged_32k", "residual_128k", "shared_latent_32k"])
def test_timed_entry_matches_and_brackets_the_kernel(name):
    """kvc_decode_attn_timed gives the same bits as kvc_decode_attn; its event pair (attention kernel
    only) lies inside a pair recorded around the whole call (kernel + split merge)."""
    kw = dict(B=2, T=1500) if name != "shared_latent_32k" else dict(B=1, T=1500, n_layers=2)
    w = synth.WORKLOADS[name].scaled(**kw)
    d = dev(synth.make_inputs(w))
    cache = gpu_cache(w, d)
    L = gpu_layout(w)
    plain = gpu_decode(w, d, cache)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev[2:]:
        e.record()
    torch.cuda.synchronize()
    ev[0].record()
    timed = kvc.decode_attn(L, cache, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                            q_pos=d["q_pos"], events=(ev[2], ev[3]))
    ev[1].record()
    torch.cuda.synchronize()
    assert torch.equal(plain, timed)
    call_ms, kern_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    print(f"    call {call_ms:.4f} ms, attention kernel {kern_ms:.4f} ms", flush=True)
    assert 0.0 < kern_ms <= call_ms
    assert ev[0].elapsed_time(ev[2]) >= 0.0 and ev[3].elapsed_time(ev[1]) >= 0.0
