"""kvc_fit_basis on the GPU against the basis-fitting oracle (fp64 SVD of each head's rows).

Singular vectors are unique (up to sign) only where singular values are apart, so the comparison has three
parts (tolerances from the arithmetic; u = 2^-24, the fp32 unit roundoff):
  * eigenvalues, every one (Weyl): |s2_gpu - s2| <= delta;
  * each column whose neighbours in the spectrum are apart (Davis-Kahan): sin(angle) <= delta / gap + 1e-5,
    tested where that bound is below 0.2, with the sign checked where the pivot entry is unambiguous;
  * the whole rank-r subspace, gap-free (Eckart-Young): the energy it captures falls short of the optimum
    sum of the r leading eigenvalues by at most 2 r delta.
delta bounds |G_gpu - G| in the 2-norm plus the eigensolver's error: the Gram matrix is n rounded fp32
additions per entry (random-walk growth, 8x headroom: 8 u sqrt(n) |G|_F), and fp32 Jacobi adds about
100 u lambda_max (measured on a CPU emulation of the kernel's rotations; 400 u is allowed here).
"""
import numpy as np
import pytest
import torch

from oracle import fit as F
from rank_bit_compressed_amd import kvc, synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _sin(b, o):
    """sin of the angle between b and the unit vector o, from b's component orthogonal to o (fp64).  The
    form 1 - cos^2 would turn the fp32 columns' norm error (a few ulps) into a spurious angle of ~1e-4."""
    return float(np.linalg.norm(b - (b @ o) * o) / np.linalg.norm(b))


def _rows(x, seq):
    return [F.head_rows(x, seq, h) for h in range(x.shape[2])]


def _check(x_cpu, seq, rank, r_cap=None, label=""):
    print(f"[fit] {label} x={tuple(x_cpu.shape)} seq={list(seq)[:6]} rank={rank} r_cap={r_cap}", flush=True)
    x = x_cpu.cuda().contiguous()
    sl = torch.tensor(seq, dtype=torch.int32).cuda()
    bb, bf, s2 = kvc.fit_basis(x, sl, rank, r_cap)
    bb2, bf2, s22 = kvc.fit_basis(x, sl, rank, r_cap)
    torch.cuda.synchronize()
    # deterministic
    assert torch.equal(bb.view(torch.int16), bb2.view(torch.int16)) and torch.equal(bf, bf2) and torch.equal(s2, s22)
    xn = x_cpu.numpy()
    ob, os2 = F.fit_basis(xn, seq, rank)
    gb = bf.cpu().double().numpy()
    gs2 = s2.cpu().double().numpy()
    Hkv, d = xn.shape[2], xn.shape[3]
    rc = rank if r_cap is None else r_cap
    # bf16 output: round-to-nearest-even of the fp32 output, zero beyond the rank
    f32 = bf.cpu().numpy()
    u32 = f32.view(np.uint32).astype(np.uint64)
    rne = ((u32 + 0x7FFF + ((u32 >> 16) & 1)) >> 16).astype(np.uint16)
    got16 = bb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16[:, :, :rank], rne)
    assert np.all(got16[:, :, rank:rc] == 0)
    rows = _rows(xn, seq)
    n_tested = 0
    for h in range(Hkv):
        X = rows[h]
        w = os2[h]
        G = X.T @ X
        n = max(X.shape[0], 1)
        delta = 8 * U * np.sqrt(n) * np.linalg.norm(G) + 400 * U * w[0]
        # orthonormal columns, each with its entry of largest magnitude positive
        B = gb[h]
        np.testing.assert_allclose(B.T @ B, np.eye(rank), atol=2e-5)
        piv = B[np.argmax(np.abs(B), axis=0), np.arange(rank)]
        assert np.all(piv > 0)
        # eigenvalues (Weyl)
        assert np.all(np.abs(gs2[h] - w) <= delta), (h, np.max(np.abs(gs2[h] - w)), delta)
        # subspace energy (Eckart-Young), gap-free
        captured = float(np.trace(B.T @ G @ B))
        assert sum(w[:rank]) - captured <= 2 * rank * delta, (h, sum(w[:rank]) - captured, delta)
        # columns with separated neighbours (Davis-Kahan)
        wext = np.r_[np.inf, w, -np.inf]
        for c in range(rank):
            gap = min(wext[c] - wext[c + 1], wext[c + 1] - wext[c + 2])
            if gap <= 0:
                continue
            bound = delta / gap + 1e-5
            if bound >= 0.2:
                continue
            cos = float(B[:, c] @ ob[h][:, c])
            sin = _sin(B[:, c], ob[h][:, c])
            assert sin <= bound, (h, c, sin, bound)
            a = np.sort(np.abs(ob[h][:, c]))[::-1]
            if a[0] - a[1] > 4 * bound:
                assert cos > 0, (h, c, "sign")
            n_tested += 1
    return n_tested


def test_fit_small_ragged():
    # sequences across several 1024-token chunks, an odd count (one unpaired token), a single token and an
    # empty sequence; rank and r_cap below the head dimension
    x = synth.make_prefill_rows(4, 2100, 2, 128, seed=1)
    x[2, 1:] = 1e30  # rows past seq_len are never read into the result
    n = _check(x, [2100, 1027, 1, 0], 48, 64, "small")
    assert n >= 20


def test_fit_full_rank_and_rank_one():
    x = synth.make_prefill_rows(2, 1500, 3, 128, seed=2)
    assert _check(x, [1500, 700], 128, None, "rank128") >= 20
    assert _check(x, [1500, 700], 1, 8, "rank1") >= 3


def test_fit_fewer_rows_than_dims():
    # 20 rows: eigenvalues beyond the 20th are zero and their vectors any orthonormal completion; the checks
    # above then hold for the separated leading ones, and the basis still spans the row space
    x = synth.make_prefill_rows(2, 16, 1, 128, seed=3)
    _check(x, [16, 4], 32, None, "rank-deficient")
    sl = torch.tensor([16, 4], dtype=torch.int32).cuda()
    _, bf, s2 = kvc.fit_basis(x.cuda().contiguous(), sl, 32)
    X = F.head_rows(x.numpy(), [16, 4], 0)
    B = bf.cpu().double().numpy()[0]
    R = X - (X @ B) @ B.T
    assert np.abs(R).max() <= 1e-4 * np.abs(X).max()


def test_fit_empty_heads_give_axes():
    x = torch.zeros(2, 64, 2, 128)
    sl = torch.tensor([0, 0], dtype=torch.int32).cuda()
    bb, bf, s2 = kvc.fit_basis(x.cuda(), sl, 16)
    torch.cuda.synchronize()
    assert torch.equal(bf.cpu(), torch.eye(128)[:, :16].expand(2, 128, 16))
    assert torch.all(s2 == 0)


def test_fit_feeds_compress_from_dense():
    # the fitted bf16 bases are the layout kvc_compress takes: the latents it projects the same rows to hold
    # (per head) the energy the optimal rank-r subspace captures, up to the bf16 rounding of the basis (each
    # entry within 2^-9 of itself moves the captured energy by well under 1%) and the fit's own tolerance
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=600)
    inp = synth.make_inputs(w, seq_len=[600, 523])
    k = synth.make_prefill_rows(w.B, w.T, w.n_kv_heads, 128, seed=4)
    v = synth.make_prefill_rows(w.B, w.T, w.n_kv_heads, 128, seed=5)
    sl = inp["seq_len"].cuda()
    bk, _, _ = kvc.fit_basis(k.cuda().contiguous(), sl, w.r_k, w.r_k, want_f32=False, want_sigma2=False)
    bv, _, _ = kvc.fit_basis(v.cuda().contiguous(), sl, w.r_v, w.r_v, want_f32=False, want_sigma2=False)
    L = kvc.make_layout(**w.layout_kwargs())
    cache = kvc.DeviceCache.allocate(L, w.n_pages)
    ranks = torch.full_like(inp["ranks"], w.r_k).cuda()          # every token at the full rank
    lk = torch.zeros_like(inp["lat_k"]).cuda(); lv = torch.zeros_like(inp["lat_v"]).cuda()
    kvc.compress(L, cache, inp["block_table"].cuda(), sl, w.T, ranks=ranks, lat_k=lk, lat_v=lv,
                 k=k.cuda().contiguous(), v=v.cuda().contiguous(), basis_k=bk, basis_v=bv)
    torch.cuda.synchronize()
    seq = [600, 523]
    for x, lat, r in ((k, lk, w.r_k), (v, lv, w.r_v)):
        _, os2 = F.fit_basis(x.numpy(), seq, r)
        lat_ = lat.cpu().double().numpy()
        for h in range(w.n_kv_heads):
            captured = sum(float((lat_[b, :seq[b], h] ** 2).sum()) for b in range(w.B))
            opt = float(os2[h][:r].sum())
            assert abs(captured - opt) <= 1e-2 * opt, (h, captured, opt)


def test_fit_full_size_sampled_heads():
    # the prefill of the 32K decode workload: 16 sequences x 32768 tokens x 8 KV heads; the oracle's SVD
    # for two heads
    B, T, Hkv = 16, 32768, 8
    x = synth.make_prefill_rows(B, T, Hkv, 128, seed=6, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32).cuda()
    print("[fit] full size 16 x 32768 x 8", flush=True)
    bb, bf, s2 = kvc.fit_basis(x, sl, 64)
    torch.cuda.synchronize()
    for h in (0, 5):
        xh = x[:, :, h:h + 1, :].cpu().numpy()           # one head: the oracle treats heads independently
        ob, os2 = F.fit_basis(xh, [T] * B, 64)
        w = os2[0]
        X = F.head_rows(xh, [T] * B, 0)
        G = X.T @ X
        delta = 8 * U * np.sqrt(X.shape[0]) * np.linalg.norm(G) + 400 * U * w[0]
        B_ = bf[h].cpu().double().numpy()
        assert np.all(np.abs(s2[h].cpu().double().numpy() - w) <= delta)
        assert sum(w[:64]) - float(np.trace(B_.T @ G @ B_)) <= 2 * 64 * delta
        tested = 0
        wext = np.r_[np.inf, w, -np.inf]
        for c in range(64):
            bound = delta / min(wext[c] - wext[c + 1], wext[c + 1] - wext[c + 2]) + 1e-5
            if bound < 0.2:
                assert _sin(B_[:, c], ob[0][:, c]) <= bound, (h, c)
                tested += 1
        assert tested >= 8


def test_fit_timed_entry_matches_and_brackets_the_gram_kernel():
    x = synth.make_prefill_rows(3, 3000, 8, 128, seed=7).cuda().contiguous()
    sl = torch.tensor([3000, 2000, 1], dtype=torch.int32).cuda()
    plain = kvc.fit_basis(x, sl, 64)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev[2:]:
        e.record()
    torch.cuda.synchronize()
    ev[0].record()
    timed = kvc.fit_basis(x, sl, 64, events=(ev[2], ev[3]))
    ev[1].record()
    torch.cuda.synchronize()
    for a, b in zip(plain, timed):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    inner, outer = ev[2].elapsed_time(ev[3]), ev[0].elapsed_time(ev[1])
    assert 0 < inner <= outer
    assert ev[0].elapsed_time(ev[2]) >= 0 and ev[3].elapsed_time(ev[1]) >= 0


def test_fitted_bases_project_elementwise_in_compress_from_dense():
    # Element parity of the fit -> compress chain at per-token ranks: bases fitted by the fit oracle (fp64 SVD,
    # rounded to bf16 by the oracle) are given to both kvc_compress (from dense, on the GPU) and the projection
    # oracle; the GPU's fp32 latents (coordinates past each token's rank zero) equal the oracle's projection.
    # The bases come from the oracle, not from the GPU fit, so no oracle input is a GPU output.
    from oracle import ref
    from oracle import tucker as TK
    from tests.helpers import layout, np_any, np_u16
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=600)
    inp = synth.make_inputs(w, seq_len=[600, 523])
    seq = [600, 523]
    k = synth.make_prefill_rows(w.B, w.T, w.n_kv_heads, 128, seed=4)
    v = synth.make_prefill_rows(w.B, w.T, w.n_kv_heads, 128, seed=5)
    bases = []
    for x, r in ((k, w.r_k), (v, w.r_v)):
        b64, _ = F.fit_basis(x.numpy(), seq, r)                     # [Hkv][d][r] fp64
        bases.append(torch.from_numpy(TK.to_bf16_bits(b64).view(np.int16)).view(torch.bfloat16).contiguous())
    bk, bv = bases
    L = kvc.make_layout(**w.layout_kwargs())
    cache = kvc.DeviceCache.allocate(L, w.n_pages)
    sl = inp["seq_len"].cuda()
    lk = torch.zeros_like(inp["lat_k"]).cuda(); lv = torch.zeros_like(inp["lat_v"]).cuda()
    kvc.compress(L, cache, inp["block_table"].cuda(), sl, w.T, ranks=inp["ranks"].cuda(), lat_k=lk, lat_v=lv,
                 k=k.cuda().contiguous(), v=v.cuda().contiguous(), basis_k=bk.cuda(), basis_v=bv.cuda())
    torch.cuda.synchronize()
    olk, olv, _, _ = ref.project(layout(w), np_any(inp["seq_len"]), w.T, np_any(inp["ranks"]), k.numpy(), v.numpy(),
                                 np_u16(bk), np_u16(bv))
    ranks = np_any(inp["ranks"])
    for got, want in ((lk, olk), (lv, olv)):
        g_ = got.cpu().numpy()
        for b in range(w.B):
            assert np.allclose(g_[b, :seq[b]], want[b, :seq[b]], rtol=0, atol=1e-5 * np.abs(want).max())
            # coordinates past each token's rank are zero on both sides
            past = np.arange(g_.shape[-1])[None, None, :] >= ranks[b, :seq[b], None, None]
            assert not g_[b, :seq[b]][np.broadcast_to(past, g_[b, :seq[b]].shape)].any()
