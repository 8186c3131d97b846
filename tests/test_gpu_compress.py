"""kvc_compress on the GPU vs the oracle compressor: bit-exact pool, offsets and tables."""
import numpy as np
import pytest
import torch

from rank_bit_compressed_amd import synth
from tests.gpu_helpers import dev, gpu_cache
from tests.helpers import np_any, oracle_cache

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", {}, None),
    ("llama8b_layer_8k", dict(T=1000), None),
    ("varrank_paged_32k", dict(B=3, T=2000), [2000, 1999, 33]),
    ("residual_128k", dict(B=2, T=700), [700, 512]),
    ("shared_latent_32k", dict(B=2, T=600), [600, 1]),
    ("llama8b_layer_8k", dict(T=1000, latent_bits=3), None),
    ("llama8b_layer_8k", dict(T=600, latent_bits=3, latent_bits_v=2), None),
    ("varrank_paged_32k", dict(B=3, T=2000, latent_bits=2), [2000, 1999, 33]),
    ("residual_128k", dict(B=2, T=700, latent_bits=3), [700, 512]),
    # the lower-bit codecs on the block-shared latent (one width for the latent)
    ("shared_latent_32k", dict(B=2, T=600, latent_bits=3), [600, 1]),
    ("shared_latent_32k", dict(B=2, T=300, page_size=64, latent_bits=2), [300, 65]),
    # the rotated residual of each layer and head on the block-shared latent
    ("shared_latent_32k", dict(B=2, T=300, page_size=64, n_layers=3, residual_bits=2, residual_std=0.3), [300, 97]),
]


@pytest.mark.parametrize("name,kw,seq", CASES, ids=[c[0] for c in CASES])
def test_compress_bit_exact(name, kw, seq):
    w = synth.WORKLOADS[name].scaled(**kw)
    inp = synth.make_inputs(w, seq_len=seq)
    print(f"[compress] {name} {kw}", flush=True)
    pool, page_off, tok_rank, tok_off = oracle_cache(w, inp)
    c = gpu_cache(w, dev(inp))
    torch.cuda.synchronize()
    assert int(c.used_bytes[0]) == len(pool)
    assert np.array_equal(c.page_off.cpu().numpy(), page_off)
    if w.variable_rank:
        assert np.array_equal(c.tok_rank.cpu().numpy(), tok_rank)
        assert np.array_equal(c.tok_off.cpu().numpy().view(np.uint32), tok_off)
    gp = c.pool[: len(pool)].cpu().numpy()
    bad = np.nonzero(gp != pool)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"
