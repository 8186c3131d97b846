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
    assert ck() == kvc.BAD_RANK | kvc.BAD_TOK_OFF      # the offset row no longer sums this rank
    cache.tok_rank[page, 5] = slot
    assert ck() == 0
    # offset rows: one interior word, the totals word, and an unused slot's rank above the cap
    P = w.page_size
    for col, delta in ((17, 1), (P, 1 << 16), (0, 8)):
        keep_off = cache.tok_off[page, col].clone()
        cache.tok_off[page, col] += delta
        print(f"[check] tok_off[{page}, {col}] += {delta}", flush=True)
        assert ck() == kvc.BAD_TOK_OFF
        cache.tok_off[page, col] = keep_off
    # an unused slot (sequence 1 holds 351 tokens: 95 slots of its third page) with a rank above the cap and an
    # offset row rebuilt to match it: only the cap is wrong
    last = int(d["block_table"][1, 2])
    keep_r, keep_row = cache.tok_rank[last].clone(), cache.tok_off[last].clone()
    cache.tok_rank[last, 120] = 72
    r = cache.tok_rank[last].to(torch.int64)
    g = (r + w.group - 1) // w.group
    pre = torch.cat([torch.zeros(1, dtype=torch.int64, device=r.device), torch.cumsum(r, 0)])
    pre_g = torch.cat([torch.zeros(1, dtype=torch.int64, device=r.device), torch.cumsum(g, 0)])
    cache.tok_off[last] = (pre | (pre_g << 16)).to(cache.tok_off.dtype)
    f = ck()
    assert f & kvc.BAD_TOK_OFF and f & ~(kvc.BAD_TOK_OFF | kvc.BAD_RECORD) == 0
    cache.tok_rank[last], cache.tok_off[last] = keep_r, keep_row
    assert ck() == 0
    # a record that starts inside the pool but runs past its end
    keep = cache.page_off[page].clone()
    cache.page_off[page] = cache.pool.numel() - 16
    assert ck() == kvc.BAD_RECORD
    cache.page_off[page] = keep
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
        page = int(d["block_table"][0, 1])
        keep = cache.page_off[page].clone()
        cache.page_off[page] = cache.pool.numel() - 1
        assert kvc.decode_check(L, cache, d["block_table"], d["seq_len"], w.T, d["q_pos"]) == kvc.BAD_RECORD
        cache.page_off[page] = keep


def test_check_slot_positions_of_a_compacted_cache():
    import numpy as np
    w = synth.WORKLOADS["shared_latent_32k_evict30"].scaled(B=2, T=600, page_size=64)
    d = dev(synth.make_inputs(w, seq_len=[600, 333]))
    cache = gpu_cache(w, d)
    L = gpu_layout(w)
    keep = torch.from_numpy((np.random.default_rng(4).random((2, 19 * 32)) < 0.3).reshape(2, 19, 32)
                            .astype(np.uint64).__lshift__(np.arange(32, dtype=np.uint64)).sum(-1)
                            .astype(np.uint32).view(np.int32)).cuda()
    keep[1] = 0                               # sequence 1 keeps nothing: a compacted length of 0
    dst = kvc.DeviceCache(L, torch.zeros_like(cache.pool), cache.page_off.clone(), None, None,
                          torch.zeros(2, dtype=torch.int64, device="cuda"), w.n_pages)
    out_len, tok_pos = kvc.evict_compact(L, cache, dst, d["block_table"], d["seq_len"], keep, d["block_table"])
    torch.cuda.synchronize()
    ck = lambda tp=tok_pos, sl=out_len: kvc.decode_check(L, dst, d["block_table"], sl, w.T, d["q_pos"], tok_pos=tp)
    print("[check] compacted positions", flush=True)
    assert int(out_len[1]) == 0 and ck() == 0
    n = int(out_len[0])
    for name, edit in (("first slot empty", lambda tp: tp[0].__setitem__(32, -1)),
                       ("out of the span", lambda tp: tp[0].__setitem__(33, int(tp[0, 32]) + 4 * 32 + 5)),
                       ("not increasing", lambda tp: tp[0].__setitem__(40, int(tp[0, 39])))):
        tp = tok_pos.clone()
        assert n > 64 and bool((tp[0, 32:41] >= 0).all())
        edit(tp)
        print(f"[check] {name}", flush=True)
        assert ck(tp=tp) == kvc.BAD_TOK_POS, name
    # without positions, a length of 0 is still an error
    assert kvc.decode_check(L, dst, d["block_table"], out_len, w.T, d["q_pos"]) == kvc.BAD_SEQ_LEN
