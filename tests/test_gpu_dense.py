"""kvc_dense_decode_attn (bf16 paged dense cache) vs the oracle's dense attention."""
import numpy as np
import pytest
import torch

from oracle import ref
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import rel_err
from tests.helpers import np_any, np_f32, np_u16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,seq", [
    ("llama8b_layer_8k", dict(T=1000), None),
    ("varrank_paged_32k", dict(B=3, T=2000), [2000, 1999, 33]),
    ("tiny", dict(B=2, T=300, page_size=64), [300, 1]),
])
def test_dense_matches_oracle(name, kw, seq):
    w = synth.WORKLOADS[name].scaled(**kw)
    print(f"[dense] {name} {kw}", flush=True)
    d = synth.make_dense_inputs(w)
    inp = synth.make_inputs(w, seq_len=seq)
    bt, sl = inp["block_table"], inp["seq_len"]
    want = ref.dense_attn(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size, np_any(bt), np_any(sl),
                          np_u16(d["k_pages"]), np_u16(d["v_pages"]), np_f32(d["q"]))
    out = kvc.dense_decode_attn(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size, bt.cuda(), sl.cuda(),
                                d["k_pages"].cuda(), d["v_pages"].cuda(), d["q"].cuda(), w.T)
    torch.cuda.synchronize()
    err = rel_err(out, want)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= 2e-3


def test_dense_fullsize_sampled():
    # the 16 x 32768 geometry the speedup is quoted on (shuffled pages of 256), launched as the bench launches it;
    # two sampled sequences checked against the oracle (all 32 query heads each)
    w = synth.WORKLOADS["varrank_paged_32k"]
    print(f"[dense] full size B={w.B} T={w.T}", flush=True)
    d = synth.make_dense_inputs(w, device="cuda")
    inp = synth.make_inputs(w)
    bt, sl = inp["block_table"], inp["seq_len"]
    out = kvc.dense_decode_attn(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size, bt.cuda(), sl.cuda(),
                                d["k_pages"], d["v_pages"], d["q"], w.T)
    torch.cuda.synchronize()
    sel = np.zeros(w.B, np.uint8)
    sel[[0, 9]] = 1
    want = ref.dense_attn(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size, np_any(bt), np_any(sl),
                          np_u16(d["k_pages"]), np_u16(d["v_pages"]), np_f32(d["q"]), sel_b=sel)
    got = out.cpu().double().numpy()
    rows = sel.astype(bool)
    err = float(np.abs(got[rows] - want[rows]).max() / np.abs(want[rows]).max())
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= 2e-3
    assert np.isfinite(got).all()
