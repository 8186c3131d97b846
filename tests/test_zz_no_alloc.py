"""kvc_decode_attn_noalloc: the decode step with its split partials in the library's file-scope device array.
Checked against kvc_decode_attn (same kernels, same splits: bit-identical output) and the oracle, on two calls in a
row, the second with a smaller input (the array keeps the first call's contents); and the size rejection."""
import ctypes as C

import numpy as np
import pytest
import torch

from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_layout, rel_err
from tests.helpers import oracle_cache, oracle_decode


def _case(name, kw, seq):
    w = synth.WORKLOADS[name].scaled(**kw)
    inp = synth.make_inputs(w, seq_len=seq)
    d = dev(inp)
    cache = gpu_cache(w, d)
    L = gpu_layout(w)
    args = (L, cache, d["block_table"], d["seq_len"], d["q"], d["wk"], d["wv"], w.T)
    return w, inp, d, args


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", [
    (("varrank_paged_32k", dict(B=4, T=3000), [3000, 2999, 1025, 33]), ("varrank_paged_32k", dict(B=2, T=700), [700, 31])),
    (("residual_128k", dict(B=3, T=2000), [2000, 1500, 257]), ("llama8b_layer_8k", dict(B=1, T=300), None)),
    (("shared_latent_32k", dict(B=2, T=1500), [1500, 900]), ("shared_latent_32k", dict(B=1, T=200, n_layers=2), None)),
])
def test_noalloc_matches_decode_attn_on_consecutive_calls(first, second):
    for name, kw, seq in (first, second):
        print(f"[noalloc] {name} {kw} seq={seq}", flush=True)
        w, inp, d, args = _case(name, kw, seq)
        want = kvc.decode_attn(*args, q_pos=d["q_pos"])
        got = kvc.decode_attn_noalloc(*args, q_pos=d["q_pos"])
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name}: max |diff| {float((got - want).abs().max()):.3e}"
        ref = oracle_decode(w, inp, oracle_cache(w, inp))
        assert rel_err(got, ref) <= 2e-3
