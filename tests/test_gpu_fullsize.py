"""Parity at the full workload sizes, in the launch configuration the bench uses (automatic splits):
bit-exact compression (whole pool, or every page of the sampled sequences) and decode outputs of
sampled (sequence, kv head[, layer]) groups against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import ref
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import gpu_cache, gpu_decode
from tests.helpers import layout, np_u16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]
TOL = 2e-3


def _host(t):
    return None if t is None else t.detach().cpu()


def _np(t):
    return None if t is None else t.numpy()


def _check(w, inp_gpu, seqs, heads, compare_whole_pool):
    print(f"[fullsize] {w.name} B={w.B} T={w.T}: compress + decode on the GPU", flush=True)
    cache = gpu_cache(w, inp_gpu)
    out = gpu_decode(w, inp_gpu, cache)
    torch.cuda.synchronize()
    # oracle inputs: the sampled sequences' rows (their pages keep their physical ids)
    rows = list(range(w.B)) if compare_whole_pool else seqs
    h = {k: _host(v) for k, v in inp_gpu.items()}
    sub = {k: (v[rows] if v is not None and k in ("lat_k", "lat_v", "res_k", "res_v", "ranks", "seq_len",
                                                   "q_pos", "block_table") else v) for k, v in h.items()}
    L = layout(w)
    print(f"[fullsize] oracle compress of {len(rows)} sequences", flush=True)
    pool, page_off, tok_rank, tok_off = ref.compress(
        L, _np(sub["block_table"]), _np(sub["seq_len"]), w.T, _np(sub["ranks"]), _np(sub["lat_k"]),
        _np(sub["lat_v"]), _np(sub["res_k"]), _np(sub["res_v"]), w.n_pages, ref.page_bytes_uniform(L) * w.n_pages)
    gp = cache.pool.cpu().numpy()
    if compare_whole_pool:
        assert int(cache.used_bytes[0]) == len(pool)
        assert np.array_equal(gp[: len(pool)], pool)
    else:  # uniform layout: every page record sits at p * page_bytes in both pools
        pb = ref.page_bytes_uniform(L)
        for p in _np(sub["block_table"]).reshape(-1):
            assert np.array_equal(gp[p * pb:(p + 1) * pb], pool[p * pb:(p + 1) * pb]), f"page {p}"
    print(f"[fullsize] oracle decode of sequences {seqs}, kv heads {heads}", flush=True)
    sel_b = np.zeros(len(rows), np.uint8)
    for s in seqs:
        sel_b[rows.index(s)] = 1
    sel_h = np.zeros(w.n_kv_heads, np.uint8)
    sel_h[heads] = 1
    q = h["q"][..., rows, :, :] if w.shared else h["q"][rows]
    want = ref.decode_attn(L, _np(sub["block_table"]), _np(sub["seq_len"]), _np(sub["q_pos"]), pool, page_off,
                           tok_rank, tok_off, q.float().numpy(), np_u16(h["wk"]), np_u16(h["wv"]), sel_b, sel_h)
    got = out.cpu().double().numpy()
    got = got[..., rows, :, :] if w.shared else got[rows]
    m = ~np.isnan(want)
    err = np.abs(got[m] - want[m]).max() / np.abs(want[m]).max()
    print(f"[fullsize] {w.name}: max|err| / max|ref| = {err:.3e} over {m.sum()} outputs", flush=True)
    assert err <= TOL


def test_fullsize_llama8b_layer_8k():
    w = synth.WORKLOADS["llama8b_layer_8k"]
    inp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in synth.make_inputs(w).items()}
    _check(w, inp, [0], list(range(8)), compare_whole_pool=True)


def test_fullsize_varrank_paged_32k():
    w = synth.WORKLOADS["varrank_paged_32k"]
    inp = synth.make_inputs(w, device="cuda")
    _check(w, inp, [0, 11], [0, 3, 7], compare_whole_pool=True)


def test_fullsize_shared_latent_32k():
    w = synth.WORKLOADS["shared_latent_32k"]
    inp = synth.make_inputs(w, device="cuda")
    _check(w, inp, [2], [5], compare_whole_pool=True)


def test_fullsize_shared_latent_32k_int3():
    # the 4 x 32K block-shared latent in INT3 (BellowsKV's INT3 row)
    w = synth.WORKLOADS["shared_latent_32k_int3"]
    inp = synth.make_inputs(w, device="cuda")
    _check(w, inp, [1], [3], compare_whole_pool=True)


def test_fullsize_residual_128k():
    w = synth.WORKLOADS["residual_128k"]
    inp = synth.make_inputs(w, device="cuda")
    _check(w, inp, [6], [1, 6], compare_whole_pool=False)


def test_fullsize_varrank_paged_32k_int3():
    # the 32K variable-rank workload with INT3 latents (general per-head kernel)
    w = synth.WORKLOADS["varrank_paged_32k_int3"]
    inp = synth.make_inputs(w, device="cuda")
    _check(w, inp, [4], [2, 5], compare_whole_pool=True)


def test_fullsize_llama8b_layer_8k_k3v2():
    w = synth.WORKLOADS["llama8b_layer_8k_k3v2"]
    inp = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in synth.make_inputs(w).items()}
    _check(w, inp, [0], list(range(8)), compare_whole_pool=True)
