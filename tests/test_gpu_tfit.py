"""kvc_tucker_fit on the GPU against the oracle's randomized partial Tucker fit (oracle/tucker.fit_randomized,
fp64) on the same rows and the same Gaussian test matrix.

Tolerances (u = 2^-24, the fp32 unit roundoff):
  * token factor: the positive-diagonal QR factor is unique, and its first-order sensitivity to a relative
    perturbation e of its argument is about kappa e (kappa the argument's condition number).  The GPU forms
    the products in fp32 (e of a few u) and the Gram and Cholesky factors in fp64, so each column may move by
    about kappa u; a CPU emulation of the same arithmetic (fp32 products, fp64 Gram/Cholesky, two passes)
    moved columns by at most 0.7 kappa(A Omega) u + 1e-6 over kappa from 10 to 1e4 and q = 0..2, the power
    iterations adding nothing above that, and the GPU's own columns moved by about the same (measured: at most
    0.6 kappa u + 1.2e-6 on these cases).  Allowed per column: (4 kappa + 64) u in the 2-norm;
  * feature factor: the basis fit's bounds (Davis-Kahan per separated column, Eckart-Young for the subspace)
    with delta = 8 u sqrt(n) |G|_F + 400 u lambda_max over the n = seq_len L Hkv rows;
  * core: equal, entry by entry, to the projection of x on the GPU's own factors computed in fp64, within
    4 u sqrt(T d) times the projection of |x| on |factors| (fp32 sums of T and d terms); and within
    |x|_2 (|dU_t|_F + |dU_f|_F) + that of the oracle's core, where dU are the factor differences.
Decode on a fitted cache: the GPU's fit, expansion, compression and decode against the oracle's fit,
expansion, compression and decode of the same rows, max |out - ref| <= 2e-3 max |ref| (the decode bound).
"""
import numpy as np
import pytest
import torch

from oracle import fit as F
from oracle import ref
from oracle import tucker as TK
from rank_bit_compressed_amd import kvc, synth
from tests.gpu_helpers import gpu_cache, gpu_layout, rel_err
from tests.helpers import layout, np_any, np_f32

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _sin(b, o):
    return float(np.linalg.norm(b - (b @ o) * o) / np.linalg.norm(b))


def _fit_gpu(x, seq, omega, r_t, r_f, q, u_t=None):
    sl = torch.tensor(seq, dtype=torch.int32, device="cuda")
    out = kvc.tucker_fit(x, sl, omega, r_t, r_f, q, u_t=u_t)
    torch.cuda.synchronize()
    return out


def _check_seq(xs, ut, uf, core, omega, r_t, r_f, q, label, feature=True):
    """One sequence: xs fp64 [T, L, H, d] (its rows < seq_len); GPU factors fp64 (ut [T, r_t])."""
    T, L, H, d = xs.shape
    A = xs.reshape(T, -1)
    ou, of, oc = TK.fit_randomized(xs, r_t, r_f, omega, q)
    # token factor, column by column
    sv = np.linalg.svd(A @ omega, compute_uv=False)
    kappa = sv[0] / sv[-1]
    col = np.linalg.norm(ut - ou, axis=0)
    tol = (4 * kappa + 64) * U
    print(f"    {label}: kappa(A omega) {kappa:.3g}, token factor max column error {col.max():.3g} (tol {tol:.3g})",
          flush=True)
    assert col.max() <= tol, (label, col.max(), tol)
    np.testing.assert_allclose(ut.T @ ut, np.eye(r_t), atol=2e-5)
    # feature factor: the basis fit's bounds over the sequence's (t, l, h) rows
    X = xs.reshape(-1, d)
    G = X.T @ X
    w = np.linalg.eigvalsh(G)[::-1]
    delta = 8 * U * np.sqrt(X.shape[0]) * np.linalg.norm(G) + 400 * U * w[0]
    np.testing.assert_allclose(uf.T @ uf, np.eye(r_f), atol=2e-5)
    assert sum(w[:r_f]) - float(np.trace(uf.T @ G @ uf)) <= 2 * r_f * delta
    if feature:
        wext = np.r_[np.inf, w, -np.inf]
        n_cols = 0
        for c in range(r_f):
            gap = min(wext[c] - wext[c + 1], wext[c + 1] - wext[c + 2])
            bound = delta / gap + 1e-5 if gap > 0 else np.inf
            if bound >= 0.2:
                continue
            assert _sin(uf[:, c], of[:, c]) <= bound, (label, c)
            a = np.sort(np.abs(of[:, c]))[::-1]
            if a[0] - a[1] > 4 * bound:
                assert float(uf[:, c] @ of[:, c]) > 0, (label, c, "sign")
            n_cols += 1
        assert n_cols >= min(r_f, 4)
    # core: the projection of x on the GPU's own factors (fp64), entry by entry
    def project(u, x, f):
        p = (u.T @ x).reshape(r_t, L * H, d) @ f                            # [r_t, LH, r_f]
        return np.transpose(p, (1, 0, 2)).reshape(L, H, r_t, r_f)
    pg = ut.T @ A
    proj = np.transpose((pg.reshape(r_t, L * H, d) @ uf), (1, 0, 2)).reshape(L, H, r_t, r_f)
    mag = project(np.abs(ut), np.abs(A), np.abs(uf))
    slack = 4 * U * np.sqrt(T * d)
    assert np.all(np.abs(core - proj) <= slack * mag + 1e-30), label
    # and the oracle's core: core - oc = (P_g - P_o)[lh] u_f + P_o[lh] (u_f - o_f), P = U_t^T A
    po = ou.T @ A
    err = np.linalg.norm(core - oc)
    bound = (np.linalg.norm(pg - po) * (1 + 1e-4) + np.linalg.norm(po) * np.linalg.norm(uf - of)
             + slack * np.linalg.norm(mag))
    print(f"    core error vs oracle {err:.3g} (bound {bound:.3g})", flush=True)
    assert err <= bound, (label, err, bound)


def _case(B, seq, max_T, L, H, r_t, r_f, q, seed, rank=None, label="", ut_wide=0):
    print(f"[tfit] {label} B={B} seq={seq} max_T={max_T} L={L} H={H} r_t={r_t} r_f={r_f} q={q}", flush=True)
    x = synth.make_group_rows(B, max_T, L, H, 128, seed=seed, rank=rank or 2 * r_t)
    x[1, seq[1]:] = float("nan")                       # rows past seq_len are never read
    omega = synth.make_omega(L * H * 128, r_t, seed=seed)
    xd, od = x.cuda(), omega.cuda()
    ut_buf = None
    if ut_wide:
        ut_buf = torch.full((B, max_T, r_t + ut_wide), 7.0, device="cuda")
        ut_view = ut_buf[:, :, ut_wide:]
    else:
        ut_view = None
    ut, uf, core, info = _fit_gpu(xd, seq, od, r_t, r_f, q, u_t=ut_view)
    ut2, uf2, core2, _ = _fit_gpu(xd, seq, od, r_t, r_f, q)
    assert torch.equal(ut, ut2) and torch.equal(uf, uf2) and torch.equal(core, core2)   # deterministic
    assert torch.all(info == 0)
    if ut_buf is not None:
        assert torch.all(ut_buf[:, :, :ut_wide] == 7.0)                                 # other columns kept
    xn = x.double().numpy()
    on = omega.double().numpy()
    for b in range(B):
        T = seq[b]
        assert torch.all(ut[b, T:] == 0)
        _check_seq(xn[b, :T], ut[b, :T].cpu().double().numpy(), uf[b].cpu().double().numpy(),
                   core[b].cpu().double().numpy(), on, r_t, r_f, q, f"{label} seq {b}")


@pytest.mark.parametrize("q", [0, 1, 2])
def test_fit_small_ragged(q):
    # token tiles with a ragged tail (640 = 5 x 128, 517 ragged), one Cholesky panel, r_f below a chunk
    _case(2, [640, 517], 640, 2, 2, 48, 32, q, seed=1, label="small")


def test_fit_full_token_rank_and_partial_panels():
    # r_t = 256: four Cholesky panels and two column tiles; r_t = 100: a partial panel and a partial tile
    _case(2, [700, 300], 700, 1, 4, 256, 64, 1, seed=2, rank=400, label="r256")
    _case(2, [333, 150], 333, 3, 1, 100, 20, 2, seed=3, label="r100", ut_wide=8)


def test_fit_short_sequence_sets_info():
    x = synth.make_group_rows(2, 200, 1, 2, 128, seed=4, rank=64)
    omega = synth.make_omega(256, 32, seed=4)
    ut, uf, core, info = _fit_gpu(x.cuda(), [200, 10], omega.cuda(), 32, 16, 1)
    assert info.cpu().tolist() == [0, 1]
    assert torch.isfinite(ut).all() and torch.isfinite(core).all() and torch.isfinite(uf).all()
    # the other sequence is unaffected
    xn = x.double().numpy()
    _check_seq(xn[0], ut[0].cpu().double().numpy(), uf[0].cpu().double().numpy(), core[0].cpu().double().numpy(),
               omega.double().numpy(), 32, 16, 1, "short: seq 0")


def _fitted_cache(w, seq, q, seed):
    """Keys and values of a layer group, fitted on the GPU into a block-shared cache, and the oracle's fit."""
    rtk, rtv, rf = w.tucker
    xk = synth.make_group_rows(w.B, w.T, w.n_layers, w.n_kv_heads, 128, seed=seed, rank=2 * rtk)
    xv = synth.make_group_rows(w.B, w.T, w.n_layers, w.n_kv_heads, 128, seed=seed + 1, rank=2 * rtv)
    D = w.n_layers * w.n_kv_heads * 128
    ok, ov = synth.make_omega(D, rtk, seed=seed), synth.make_omega(D, rtv, seed=seed + 1)
    return xk, xv, ok, ov


def test_decode_on_a_fitted_cache():
    w = synth.WORKLOADS["tucker_group_32k"].scaled(B=2, T=600, n_layers=2)
    seq = [600, 333]
    rtk, rtv, rf = w.tucker
    q = 1
    print(f"[tfit] decode on a fitted cache {seq}", flush=True)
    xk, xv, ok, ov = _fitted_cache(w, seq, q, seed=6)
    inp = synth.make_inputs(w, seq_len=seq)
    # GPU: fit keys and values into the two halves of the latent, expand, compress, decode
    lat = torch.zeros(w.B, w.T, w.r_k, device="cuda")
    _, ufk, ck, ik = _fit_gpu(xk.cuda(), seq, ok.cuda(), rtk, rf, q, u_t=lat[:, :, :rtk])
    _, ufv, cv, iv = _fit_gpu(xv.cuda(), seq, ov.cuda(), rtv, rf, q, u_t=lat[:, :, rtk:])
    assert torch.all(ik == 0) and torch.all(iv == 0)
    wk, _ = kvc.tucker_expand(ufk, ck, w.r_k, 0)
    wv, _ = kvc.tucker_expand(ufv, cv, w.r_k, rtk)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    d["lat_k"] = lat
    gc = gpu_cache(w, d)
    out = kvc.decode_attn(gpu_layout(w), gc, d["block_table"], d["seq_len"], d["q"], wk, wv, w.T, q_pos=d["q_pos"],
                          kv_split=rtk)
    torch.cuda.synchronize()
    # oracle: its own fit of the same rows, expansion, compression and decode
    lat_o = np.zeros((w.B, w.T, w.r_k), np.float32)
    width = w.n_kv_heads * 128
    wko = np.zeros((w.B, w.n_layers, w.r_k, width), np.uint16)
    wvo = np.zeros_like(wko)
    xkn, xvn = xk.double().numpy(), xv.double().numpy()
    for b in range(w.B):
        T = seq[b]
        uk, fk, cko = TK.fit_randomized(xkn[b, :T], rtk, rf, ok.double().numpy(), q)
        uv, fv, cvo = TK.fit_randomized(xvn[b, :T], rtv, rf, ov.double().numpy(), q)
        lat_o[b, :T, :rtk] = uk
        lat_o[b, :T, rtk:] = uv
        wko[b, :, :rtk] = TK.to_bf16_bits(TK.expand(fk, TK.core_to_hosvd_layout(cko)))
        wvo[b, :, rtk:] = TK.to_bf16_bits(TK.expand(fv, TK.core_to_hosvd_layout(cvo)))
    L = layout(w)
    P = ref.page_bytes_uniform(L) * w.n_pages
    pool, page_off, tok_rank, tok_off = ref.compress(L, np_any(inp["block_table"]), np_any(inp["seq_len"]), w.T,
                                                     None, lat_o, None, None, None, w.n_pages, P)
    want = np.full(tuple(inp["q"].shape), np.nan)
    for b in range(w.B):
        sel = np.zeros(w.B, np.uint8)
        sel[b] = 1
        o = ref.decode_attn(L, np_any(inp["block_table"]), np_any(inp["seq_len"]), np_any(inp["q_pos"]), pool,
                            page_off, tok_rank, tok_off, np_f32(inp["q"]), wko[b], wvo[b], sel, None)
        want[:, b] = o[:, b]
    err = rel_err(out, want)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= 2e-3


@pytest.mark.timeout(400)
def test_fit_fullsize_group():
    # the 4-sequence, 32K-token, 4-layer, 8-head group at token rank 256 and feature rank 64, one power
    # iteration; the oracle for sequence 2 (the feature-factor columns are checked in the smaller cases)
    B, T, L, H, r_t, r_f, q = 4, 32768, 4, 8, 256, 64, 1
    print("[tfit] full size: generate", flush=True)
    x = synth.make_group_rows(B, T, L, H, 128, seed=7, device="cuda")
    omega = synth.make_omega(L * H * 128, r_t, seed=7)
    ut, uf, core, info = _fit_gpu(x, [T] * B, omega.cuda(), r_t, r_f, q)
    assert torch.all(info == 0)
    for b in range(B):
        g = ut[b].T @ ut[b]
        assert float((g - torch.eye(r_t, device="cuda")).abs().max()) <= 5e-5
    print("[tfit] full size: oracle fit of sequence 2", flush=True)
    xs = x[2].cpu().double().numpy()
    del x
    _check_seq(xs, ut[2].cpu().double().numpy(), uf[2].cpu().double().numpy(), core[2].cpu().double().numpy(),
               omega.double().numpy(), r_t, r_f, q, "full size seq 2", feature=False)
