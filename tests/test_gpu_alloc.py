"""kvc_salience and kvc_rank_alloc on the GPU against the salience and allocation oracle.

Salience: fp32 scores on the matrix cores and fp32 exp2 against the fp64 oracle.  A score's error is a few
fp32 roundings of |q||k|/sqrt(d) plus the rotation's (v_sin / v_cos, about 2^-20 of a turn), well under 1e-5
here; a probability then carries a relative error of about that times the score range, and a salience sums
those over the window's rows, so each value must lie within 2e-4 of the oracle's relative to itself, plus
1e-6 of the sequence total.  Totals equal (queries present) x Hq within 1e-5.

Allocation: the decisions are taken in fp32 on both sides (fp32 gains, the same comparisons), so the ranks
must match bit for bit; the saliences come from the seeded generator, not from the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import alloc as A
from rank_bit_compressed_amd import kvc, synth

pytestmark = pytest.mark.gpu


def _sal_case(B, T, W, Hkv, seq, theta, seed):
    print(f"[salience] B={B} T={T} W={W} Hkv={Hkv} seq={seq} theta={theta}", flush=True)
    k = synth.make_prefill_rows(B, T, Hkv, 128, seed=seed)
    q = synth.make_window_queries(B, W, 4 * Hkv, 128, seed=seed)
    sl = torch.tensor(seq, dtype=torch.int32)
    got = kvc.salience(q.cuda(), k.cuda(), sl.cuda(), theta)
    again = kvc.salience(q.cuda(), k.cuda(), sl.cuda(), theta)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    want = A.salience(q.numpy(), k.numpy(), seq, theta)
    g = got.cpu().double().numpy()
    for b in range(B):
        n_q = sum(1 for i in range(W) if seq[b] - W + i >= 0)
        tot = n_q * 4 * Hkv
        assert abs(g[b].sum() - tot) <= 1e-5 * max(tot, 1)
        assert np.all(g[b, seq[b]:] == 0)
        err = np.abs(g[b] - want[b])
        assert np.all(err <= 2e-4 * np.abs(want[b]) + 1e-6 * tot), (b, float(err.max()))


def test_salience_small_ragged():
    # ragged lengths across 32-key tiles, a sequence shorter than the window, one token, an empty sequence
    _sal_case(4, 700, 32, 2, [700, 333, 5, 1], 500000.0, seed=1)


def test_salience_short_window_no_rope_empty():
    _sal_case(3, 260, 7, 1, [260, 0, 33], 0.0, seed=2)


def test_salience_full_size_sampled_sequence():
    # the prefill of the 32K decode workload with a 32-query window; the oracle for one sequence
    B, T, Hkv, W = 16, 32768, 8, 32
    k = synth.make_prefill_rows(B, T, Hkv, 128, seed=3, device="cuda")
    q = synth.make_window_queries(B, W, 4 * Hkv, 128, seed=3, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    print("[salience] full size 16 x 32768 x 8, W 32", flush=True)
    got = kvc.salience(q, k, sl, 500000.0)
    torch.cuda.synchronize()
    b = 5
    want = A.salience(q[b:b + 1].cpu().numpy(), k[b:b + 1].cpu().numpy(), [T], 500000.0)[0]
    g = got[b].cpu().double().numpy()
    tot = W * 4 * Hkv
    assert abs(got.double().sum(dim=1) - tot).max().item() <= 1e-5 * tot * 4
    assert np.all(np.abs(g - want) <= 2e-4 * np.abs(want) + 1e-6 * tot)


LADDERS = [([8, 16, 32, 64], [1.0, 0.45, 0.2]), ([8, 24, 40, 56, 64], [3.0, 2.0, 2.0, 0.5]), ([16, 64], [1.0])]


@pytest.mark.parametrize("li", range(len(LADDERS)))
def test_rank_alloc_bit_exact(li):
    ladder, w = LADDERS[li]
    B, T = 5, 3000
    seq = [3000, 2999, 1, 0, 1777]
    sal = synth.make_salience(B, T, seed=10 + li)
    sal[0, :500] = sal[0, 0]                        # a block of ties
    sal[1, 100:200] = 0.0                           # zero gains
    sl = torch.tensor(seq, dtype=torch.int32)
    wf = np.array(w, np.float32)
    for mean in (ladder[0], 20.8 if ladder[-1] >= 21 else ladder[0] + 0.5, (ladder[0] + ladder[-1]) / 2, ladder[-1]):
        print(f"[alloc] ladder={ladder} mean={mean}", flush=True)
        got = kvc.rank_alloc(sal.cuda(), sl.cuda(), ladder, w, mean)
        torch.cuda.synchronize()
        want = A.rank_alloc(sal.numpy(), seq, ladder, wf, mean)
        assert np.array_equal(got.cpu().numpy(), want), (ladder, mean)
        for b in range(B):
            assert int(want[b].astype(np.int64).sum()) <= A.budget(mean, seq[b])


def test_rank_alloc_full_size_and_feeds_compress():
    # 16 x 32768 tokens at the 32K workload's mean rank (20.8); the ranks are the variable-rank input of
    # kvc_compress
    B, T = 16, 32768
    sal = synth.make_salience(B, T, seed=20)
    sl = torch.full((B,), T, dtype=torch.int32)
    ladder, w = [8, 16, 32, 64], [1.0, 0.45, 0.2]
    got = kvc.rank_alloc(sal.cuda(), sl.cuda(), ladder, w, 20.8)
    torch.cuda.synchronize()
    want = A.rank_alloc(sal.numpy(), [T] * B, ladder, np.array(w, np.float32), 20.8)
    assert np.array_equal(got.cpu().numpy(), want)
    wl = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=1000)
    inp = synth.make_inputs(wl, seq_len=[1000, 999])
    L = kvc.make_layout(**wl.layout_kwargs())
    cache = kvc.DeviceCache.allocate(L, wl.n_pages)
    ranks = got[:2, :1000].contiguous()
    kvc.compress(L, cache, inp["block_table"].cuda(), inp["seq_len"].cuda(), wl.T, ranks=ranks,
                 lat_k=inp["lat_k"].cuda(), lat_v=inp["lat_v"].cuda())
    torch.cuda.synchronize()
    assert int(cache.used_bytes[0]) > 0
