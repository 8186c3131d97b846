"""Block-shared decode with the rotated 2-bit residual of each layer and head (JoLT: the Tucker form plus a rotated
low-bit residual) against the oracle, within 2e-3 max|ref| (the bound of every decode path): plain shared latents
over several layers, ragged lengths and pages, automatic and explicit splits; the split-latent form (keys and
values with their own token factors) equal to the plain one; a Tucker group at full size, sampled."""
import numpy as np
import pytest
import torch

from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_layout, rel_err
from tests.helpers import oracle_cache, oracle_decode

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.mark.parametrize("n_layers,P,seq,num_splits", [(2, 64, (300, 97), 0), (3, 128, (700, 1), 3),
                                                        (1, 256, (513, 256), 0)])
def test_shared_residual_decode_matches_oracle(n_layers, P, seq, num_splits):
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=2, T=max(seq), n_layers=n_layers, page_size=P, residual_bits=2,
                                                     residual_std=0.3, shuffle_pages=True)
    inp = synth.make_inputs(w, seq_len=list(seq))
    print(f"[shared res] layers={n_layers} P={P} seq={seq} splits={num_splits}", flush=True)
    d = dev(inp)
    c = gpu_cache(w, d)
    L = gpu_layout(w)
    args = (L, c, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T)
    out = kvc.decode_attn(*args, q_pos=d["q_pos"], num_splits=num_splits)
    again = kvc.decode_attn(*args, q_pos=d["q_pos"], num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    want = oracle_decode(w, inp, oracle_cache(w, inp))
    assert rel_err(out, want) <= TOL
    # the residual matters here: the output without it differs by far more than the tolerance
    wn = w.scaled(residual_bits=0)
    inpn = dict(inp, res_k=None, res_v=None)
    assert rel_err(out, oracle_decode(wn, inpn, oracle_cache(wn, inpn))) > 10 * TOL
    if n_layers == 2:  # keys and values with their own token factors (W_k zero on the upper latent half, W_v on
        # the lower): the split form against the oracle with those W (the key residual then joins the key waves'
        # partial keys before their fp16 RoPE, so the split and plain forms round differently)
        wk2, wv2 = d["wk"].clone(), d["wv"].clone()
        wk2[:, 256:] = 0
        wv2[:, :256] = 0
        s = kvc.decode_attn(L, c, d["block_table"], d["seq_len"], d["q"], wk2, wv2, w.T, q_pos=d["q_pos"],
                            num_splits=num_splits, kv_split=256)
        torch.cuda.synchronize()
        inp2 = dict(inp, wk=wk2.cpu(), wv=wv2.cpu())
        assert rel_err(s, oracle_decode(w, inp2, oracle_cache(w, inp2))) <= TOL


def test_shared_residual_rejects_masks_and_positions():
    w = synth.WORKLOADS["shared_latent_32k"].scaled(B=1, T=64, page_size=64, residual_bits=2)
    inp = synth.make_inputs(w)
    d = dev(inp)
    c = gpu_cache(w, d)
    keep = torch.full((1, 2), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(kvc.KvcError):
        kvc.decode_attn(gpu_layout(w), c, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T,
                        q_pos=d["q_pos"], keep_mask=keep)


@pytest.mark.timeout(600)
def test_tucker_group_with_residual_full_size_sampled():
    # the full 4-sequence, 32K-token, 4-layer Tucker group with every layer's and head's residual; compression bit
    # for bit, the oracle's decode for one sequence and one KV head (all four layers)
    from tests.test_gpu_tucker import _gpu_w, _oracle_decode, _oracle_w
    w = synth.WORKLOADS["tucker_group_32k_res"]
    inp = synth.make_inputs(w)
    print("[shared res] full size: oracle compress", flush=True)
    cache = oracle_cache(w, inp)
    wk, wv = _oracle_w(w, inp)
    d = dev(inp)
    gc = gpu_cache(w, d)
    gwk, gwv = _gpu_w(w, d)
    out = kvc.decode_attn(gpu_layout(w), gc, d["block_table"], d["seq_len"], d["q"], gwk, gwv, w.T, q_pos=d["q_pos"],
                          kv_split=w.tucker[0])
    torch.cuda.synchronize()
    assert np.array_equal(gc.pool.cpu().numpy()[:len(cache[0])], cache[0])
    del d, gc
    torch.cuda.empty_cache()
    print("[shared res] full size: oracle decode of sequence 2, kv head 5", flush=True)
    want = _oracle_decode(w, inp, cache, wk, wv, [2], [5])
    err = rel_err(out, want)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= TOL
