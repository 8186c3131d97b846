"""kvc_decode_check: the opt-in check of the tables a decode trusts.  Each case corrupts one table of a
compressed cache and expects exactly its flag; nothing here decodes through a bad table."""
import pytest
import torch

from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import dev, gpu_cache, gpu_layout

pytestmark = pytest.mark.gpu


def _setup(name, **kw):
    w = synth.WORKLOADS[name].scaled(**kw)
    d = dev(synth.make_inputs(w, seq_len=[w.T, w.T // 2 + 1]))
    cache = gpu_cache(w, d)
    torch.cuda.synchronize()
    return w, d, gpu_layout(w), cache


def test_check_flags_each_corruption():
    w, d, L, cache = _setup("varrank_paged_32k", B=2, T=700, page_size=128)
    ck = lambda bt=d["block_table"], sl=d["seq_len"], qp=d["q_pos"], max_T=w.T: kvc.decode_check(L, cache, bt, sl, max_T, qp)
    print("[check] intact tables", flush=True)
    assert ck() == 0
    bt = d["block_table"].clone()
    bt[1, -1] = 10 ** 6                      # a block sequence 1 (351 tokens, 3 blocks of 128) does not use
    assert ck(bt=bt) == 0
    bt[1, 1] = w.n_pages                     # a used block
    assert ck(bt=bt) == kvc.BAD_PAGE
    bt[1, 1] = -1
    assert ck(bt=bt) == kvc.BAD_PAGE
    sl = d["seq_len"].clone(); sl[0] = 0
    assert ck(sl=sl) == kvc.BAD_SEQ_LEN
    sl[0] = w.T + 1
    assert ck(sl=sl) == kvc.BAD_SEQ_LEN
    qp = d["q_pos"].clone(); qp[1] = -5
    assert ck(qp=qp) == kvc.BAD_Q_POS
    page = int(d["block_table"][0, 2])
    keep = cache.page_off[page].clone()
    cache.page_off[page] = cache.pool.numel()
    assert ck() == kvc.BAD_OFFSET
    cache.page_off[page] = keep
    slot = cache.tok_rank[page, 5].clone()
    cache.tok_rank[page, 5] = 7
    assert ck() == kvc.BAD_RANK
    cache.tok_rank[page, 5] = slot
    sl = d["seq_len"].clone(); sl[0] = 0
    assert ck(bt=bt, sl=sl, qp=qp) == kvc.BAD_PAGE | kvc.BAD_SEQ_LEN | kvc.BAD_Q_POS
    assert ck() == 0


def test_check_uniform_and_shared_layouts():
    for name in ("llama8b_layer_8k", "shared_latent_32k"):
        w, d, L, cache = _setup(name, B=2, T=600)
        print(f"[check] {name}", flush=True)
        assert kvc.decode_check(L, cache, d["block_table"], d["seq_len"], w.T, d["q_pos"]) == 0
        bt = d["block_table"].clone()
        bt[0, 0] = w.n_pages + 3
        assert kvc.decode_check(L, cache, bt, d["seq_len"], w.T, d["q_pos"]) == kvc.BAD_PAGE
