"""kvc_decode_attn on the GPU vs the fp64 oracle on the same stored bytes.

Tolerance: max |out - ref| <= 2e-3 * max |ref| over all outputs (the bound
the target states for the attention output)."""
import numpy as np
import pytest
import torch

from rank_bit_compressed_amd import synth
from tests.gpu_helpers import dev, gpu_cache, gpu_decode, rel_err
from tests.helpers import np_any, oracle_cache, oracle_decode

pytestmark = pytest.mark.gpu
TOL = 2e-3

CASES = [
    ("tiny", {}, None),
    ("llama8b_layer_8k", dict(T=1000), None),
    ("llama8b_layer_8k", dict(B=2, T=333, page_size=64), [333, 1]),
    ("varrank_paged_32k", dict(B=3, T=2000), [2000, 1999, 33]),
    ("varrank_paged_32k", dict(B=2, T=300, page_size=32), [300, 17]),
    ("residual_128k", dict(B=2, T=700), [700, 512]),
    ("residual_128k", dict(B=3, T=1500, page_size=64), [1500, 1025, 31]),
    # the residual kernel's other rank variants: 4 key and value steps; 2 of each (half-width value code reads),
    # groups of 16 (a pair word per chunk)
    ("residual_128k", dict(B=2, T=700, r_k=64, r_v=64, page_size=128), [700, 255]),
    ("residual_128k", dict(B=2, T=600, r_k=32, r_v=32, page_size=128), [600, 129]),
    ("residual_128k", dict(B=2, T=500, r_k=48, r_v=64, group=16, page_size=128), [500, 33]),
    ("residual_128k", dict(B=2, T=600, r_k=32, r_v=64, page_size=128), [600, 97]),
    ("residual_128k", dict(B=2, T=600, r_k=64, r_v=32, page_size=128), [600, 300]),
    # ranks that are not multiples of 16: the general per-head kernel's residual path
    ("residual_128k", dict(B=2, T=700, r_k=40, r_v=56), [700, 300]),
    ("shared_latent_32k", dict(B=2, T=600), [600, 33]),
    ("shared_latent_32k", dict(B=1, T=300, n_layers=2, page_size=64), None),
    # lower-bit codecs on the general per-head kernel: INT3, INT2, 3-bit keys with 2-bit values
    ("llama8b_layer_8k", dict(T=1000, latent_bits=3), None),
    ("llama8b_layer_8k", dict(B=2, T=333, page_size=64, latent_bits=2), [333, 1]),
    ("llama8b_layer_8k", dict(T=700, latent_bits=3, latent_bits_v=2), None),
    ("varrank_paged_32k", dict(B=2, T=1000, latent_bits=3), [1000, 517]),
    ("varrank_paged_32k", dict(B=2, T=600, latent_bits=2), [600, 33]),
    ("residual_128k", dict(B=2, T=700, latent_bits=3), [700, 300]),
    # lower-bit codecs that the fast kernel has no variant for: the general per-head kernel
    ("llama8b_layer_8k", dict(T=700, r_k=40, r_v=40, latent_bits=3), None),
    ("llama8b_layer_8k", dict(B=2, T=500, r_k=40, r_v=40, latent_bits=3, latent_bits_v=2), [500, 77]),
    ("varrank_paged_32k", dict(B=2, T=800, r_k=48, r_v=48, rank_choices=(8, 16, 32, 48), latent_bits=2), [800, 301]),
    # lower-bit codecs on the block-shared latent: INT3 (4 layers, ragged tails) and INT2 (2 layers, pages of 64)
    ("shared_latent_32k", dict(B=2, T=600, latent_bits=3), [600, 33]),
    ("shared_latent_32k", dict(B=1, T=300, n_layers=2, page_size=64, latent_bits=2), None),
    ("shared_latent_32k", dict(B=2, T=500, group=128, latent_bits=3), [500, 1]),
]


@pytest.mark.parametrize("name,kw,seq", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_decode_matches_oracle(name, kw, seq):
    w = synth.WORKLOADS[name].scaled(**kw)
    inp = synth.make_inputs(w, seq_len=seq)
    print(f"[decode] {name} {kw} seq={seq}", flush=True)
    ref = oracle_decode(w, inp, oracle_cache(w, inp))
    d = dev(inp)
    out = gpu_decode(w, d, gpu_cache(w, d))
    torch.cuda.synchronize()
    err = rel_err(out, ref)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= TOL
