"""Seeded synthetic inputs shaped like the pages' Llama-3.1-8B-class decode
workloads.  This module only draws random inputs (queries, bases, latents,
ranks, residuals, page tables); it holds none of the method's arithmetic (no
quantization, projection, rotation or attention).  Both the GPU path and the
CPU oracle read the tensors it returns.

Distributions (the pages give shapes, not data):
  * bases: per-KV-head orthonormal d x r matrices, the Q factor of a seeded
    Gaussian matrix, stored as bf16;
  * latents: coordinate i (1-based) drawn N(0, 1) * i^-decay, i.e. standard
    deviation i^-0.7 for the decaying-spectrum workloads; i.i.d. N(0, 1) for
    the block-shared latent, whose coordinates mix all layers' channels and so
    have a flat dynamic range;
  * rotated residual: drawn directly in the rotated domain, N(0, 0.05^2) per
    element.  An orthonormal rotation of an i.i.d. Gaussian vector is again
    i.i.d. Gaussian with the same variance, so this has exactly the law of
    "draw N(0, 0.05^2), then rotate";
  * queries: N(0, 1) / 8, rounded to bf16 where the workload says bf16;
  * variable ranks: i.i.d. per (sequence, token) from a discrete distribution;
  * block tables: identity (contiguous storage) or a seeded permutation of
    all physical pages;
  * prefill rows for basis fitting (pre-RoPE keys or values, fp32): per KV
    head h, x = mu_h + Q_h (z * s) with z ~ N(0, I), s_i = 4 i^-0.7 (the same
    decaying spectrum as the latents), Q_h a seeded orthogonal d x d matrix
    and mu_h a seeded direction of length 1.5, so the rows carry a mean and a
    spread of singular values without repeated ones;
  * window queries for salience (pre-RoPE, fp32): N(0, 1) per element;
  * salience for the rank-allocation tests: exp(N(0, 1.5^2)) per token, a
    heavy-tailed positive spread like attention mass, rounded to fp32; the
    per-layer token scores of an evicting block-shared workload are one such
    draw per layer (or, clustered, exp(u + 0.3 n) with u ~ N(0, 1.5^2) per run
    of tokens shared by the layers and n ~ N(0, 1) per token and layer);
  * partial Tucker factors of a layer group (keys and values separately), per
    sequence: token factor rows N(0, 1/T) per element (the scale of a factor
    with orthonormal columns over T tokens); the feature factor an orthonormal
    d x r_f matrix as for bases; the core [L][Hkv][r_t][r_f] N(0, 1) scaled by
    sqrt(T d / (r_t r_f)) * s_c, s_c = (c + 1)^-0.35 normalised to mean square
    1 over c (a decaying token-mode spectrum), so rebuilt keys and values have
    about unit variance like the other workloads.  The block-shared latent of
    such a workload is the key factor row followed by the value factor row;
  * a layer group's keys or values for the partial Tucker fit (fp32 [B, max_T, L, Hkv, d]), per sequence:
    R planted token components, x[t, l, h, :] = sum_c a[t, c] s_c F (f * z[c, l, h, :]) + noise e, with a, z
    and e i.i.d. N(0, 1), s_c = c^-decay_t, f_i = i^-decay_f, F a seeded orthogonal d x d matrix, divided
    by the expected element RMS, so the token mode has a decaying spectrum of rank R plus a noise floor and
    the feature mode a decaying spectrum without repeated values;
  * the Gaussian test matrix of the randomized fit: N(0, 1) per element, fp32.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    r_k: int                      # key rank (cap); block-shared mode: latent dimension
    r_v: int                      # value rank (cap); block-shared mode: latent dimension
    group: int = 32
    latent_bits: int = 4
    latent_bits_v: int = 0        # value latent bits; 0 = latent_bits
    residual_bits: int = 0
    page_size: int = 256
    variable_rank: bool = False
    shared: bool = False
    n_layers: int = 1
    rope_theta: float = 0.0
    q_bf16: bool = True
    shuffle_pages: bool = False
    rank_choices: tuple = ()
    rank_probs: tuple = ()
    latent_decay: float = 0.7     # 0 = i.i.d. N(0, 1)
    residual_std: float = 0.05
    w_std: float = 0.0            # block-shared mode: W entries N(0, w_std^2)
    tucker: tuple = ()            # block-shared from partial Tucker factors: (key r_t, value r_t, r_f)
    evict_ratio: float = 0.0      # block-shared: share of tokens the block's eviction decision keeps
    evict_cluster: int = 0        # > 0: token scores clustered in runs of this many tokens (see make_layer_scores)
    evict_compact: bool = False   # the evicted tokens are compacted out of the pages before the decode
    seed: int = 0

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def max_blocks(self) -> int:
        return -(-self.T // self.page_size)

    @property
    def n_pages(self) -> int:
        return self.B * self.max_blocks

    def layout_kwargs(self) -> dict:
        """Geometry common to the GPU library and the oracle."""
        return dict(n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads, head_dim=self.head_dim,
                    r_k_cap=self.r_k, r_v_cap=self.r_v, group=self.group, latent_bits=self.latent_bits,
                    residual_bits=self.residual_bits, page_size=self.page_size,
                    variable_rank=int(self.variable_rank), shared=int(self.shared), n_layers=self.n_layers,
                    rope_theta=float(self.rope_theta), latent_bits_v=self.latent_bits_v)


# The five workloads of the build's target list; sizes as stated there.
WORKLOADS = {
    # batch 1, 4 query / 1 KV head, d 64, 256 tokens, rank-16 bases, fp32 latents, no RoPE
    "tiny": Workload("tiny", B=1, T=256, n_q_heads=4, n_kv_heads=1, head_dim=64, r_k=16, r_v=16,
                     group=16, latent_bits=32, rope_theta=0.0, q_bf16=False, seed=11),
    # one Llama-3.1-8B-shaped layer, batch 1, 8K context, INT4 G32, ranks 48 (K) / 64 (V)
    "llama8b_layer_8k": Workload("llama8b_layer_8k", B=1, T=8192, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                 r_k=48, r_v=64, group=32, rope_theta=500000.0, seed=12),
    # batch 16, 32K context, per-token rank in {8,16,32,64}, paged (256) with a shuffled table
    "varrank_paged_32k": Workload("varrank_paged_32k", B=16, T=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                  r_k=64, r_v=64, group=32, rope_theta=500000.0, variable_rank=True,
                                  rank_choices=(8, 16, 32, 64), rank_probs=(0.4, 0.3, 0.2, 0.1),
                                  shuffle_pages=True, seed=13),
    # 4 layers share one 512-dim INT4 G64 latent per token; W_k, W_v 512 -> 8 x 128 per layer
    "shared_latent_32k": Workload("shared_latent_32k", B=4, T=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                  r_k=512, r_v=512, group=64, shared=True, n_layers=4, rope_theta=500000.0,
                                  latent_decay=0.0, w_std=1.0 / math.sqrt(512.0), seed=14),
    # batch 8, 128K context, ranks 48/64, 2-bit rotated residual, paged (256) shuffled
    "residual_128k": Workload("residual_128k", B=8, T=131072, n_q_heads=32, n_kv_heads=8, head_dim=128,
                              r_k=48, r_v=64, group=32, residual_bits=2, rope_theta=500000.0,
                              shuffle_pages=True, seed=15),
    # a 4-layer group of keys and values in partial Tucker form per sequence (token ranks 256 + 256 = the
    # 512-dim block-shared latent, feature rank 64), decoded through per-sequence up-projections
    "tucker_group_32k": Workload("tucker_group_32k", B=4, T=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                 r_k=512, r_v=512, group=64, shared=True, n_layers=4, rope_theta=500000.0,
                                 latent_decay=0.0, tucker=(256, 256, 64), seed=16),
    # the same group with the rotated 2-bit residual of each layer and head (JoLT: Tucker form plus residual)
    "tucker_group_32k_res": Workload("tucker_group_32k_res", B=4, T=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                     r_k=512, r_v=512, group=64, shared=True, n_layers=4, rope_theta=500000.0,
                                     latent_decay=0.0, tucker=(256, 256, 64), residual_bits=2, seed=16),
    # the block-shared latent with one eviction decision for its 4 layers, keeping 30% of every sequence
    "shared_latent_32k_evict30": Workload("shared_latent_32k_evict30", B=4, T=32768, n_q_heads=32, n_kv_heads=8,
                                          head_dim=128, r_k=512, r_v=512, group=64, shared=True, n_layers=4,
                                          rope_theta=500000.0, latent_decay=0.0, w_std=1.0 / math.sqrt(512.0),
                                          evict_ratio=0.3, seed=14),
    # the same with the evicted tokens compacted out of the pages (the decode reads the kept tokens only)
    "shared_latent_32k_evict30_compact": Workload("shared_latent_32k_evict30_compact", B=4, T=32768, n_q_heads=32,
                                                  n_kv_heads=8, head_dim=128, r_k=512, r_v=512, group=64, shared=True,
                                                  n_layers=4, rope_theta=500000.0, latent_decay=0.0,
                                                  w_std=1.0 / math.sqrt(512.0), evict_ratio=0.3, evict_compact=True,
                                                  seed=14),
    # the same with token importance clustered in runs of 256 tokens, so that whole super-tiles are evicted
    "shared_latent_32k_evict30_clustered": Workload("shared_latent_32k_evict30_clustered", B=4, T=32768,
                                                    n_q_heads=32, n_kv_heads=8, head_dim=128, r_k=512, r_v=512,
                                                    group=64, shared=True, n_layers=4, rope_theta=500000.0,
                                                    latent_decay=0.0, w_std=1.0 / math.sqrt(512.0),
                                                    evict_ratio=0.3, evict_cluster=256, seed=14),
    # the lower-bit codecs of the BellowsKV page's retention table on per-head latents: the 32K variable-rank
    # workload with INT3 latents, and the 8K layer with 3-bit keys and 2-bit values
    "varrank_paged_32k_int3": Workload("varrank_paged_32k_int3", B=16, T=32768, n_q_heads=32, n_kv_heads=8,
                                       head_dim=128, r_k=64, r_v=64, group=32, latent_bits=3,
                                       rope_theta=500000.0, variable_rank=True, rank_choices=(8, 16, 32, 64),
                                       rank_probs=(0.4, 0.3, 0.2, 0.1), shuffle_pages=True, seed=13),
    # the block-shared latent in INT3, the BellowsKV retention table's INT3 row
    "shared_latent_32k_int3": Workload("shared_latent_32k_int3", B=4, T=32768, n_q_heads=32, n_kv_heads=8,
                                       head_dim=128, r_k=512, r_v=512, group=64, latent_bits=3, shared=True,
                                       n_layers=4, rope_theta=500000.0, latent_decay=0.0,
                                       w_std=1.0 / math.sqrt(512.0), seed=14),
    "llama8b_layer_8k_k3v2": Workload("llama8b_layer_8k_k3v2", B=1, T=8192, n_q_heads=32, n_kv_heads=8,
                                      head_dim=128, r_k=48, r_v=64, group=32, latent_bits=3, latent_bits_v=2,
                                      rope_theta=500000.0, seed=12),
}


def _gen(w: Workload, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + stream)
    return g


def _decay_scale(r: int, decay: float, device) -> torch.Tensor:
    i = torch.arange(1, r + 1, dtype=torch.float64, device=device)
    return (i ** (-decay)).to(torch.float32)


def _orthonormal(w: Workload, stream: int, rows: int, cols: int, n: int) -> torch.Tensor:
    """n matrices rows x cols with orthonormal columns (QR of a seeded Gaussian), fp64 on the CPU."""
    g = _gen(w, stream, "cpu")
    a = torch.randn(n, rows, cols, generator=g, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    return (q * torch.sign(torch.diagonal(r, dim1=-2, dim2=-1)).unsqueeze(-2)).contiguous()


def make_inputs(w: Workload, device="cpu", seq_len=None) -> dict:
    """All inputs of one decode step of workload w (seeded, deterministic per device)."""
    dev = torch.device(device)
    B, T, Hkv, d, P = w.B, w.T, w.n_kv_heads, w.head_dim, w.page_size
    out = {}
    if seq_len is None:
        seq_len = [T] * B
    sl = torch.tensor(seq_len, dtype=torch.int32)
    assert int(sl.max()) <= T and int(sl.min()) >= 1
    out["seq_len"] = sl.to(dev)
    out["q_pos"] = sl.clone().to(dev)
    nb = w.max_blocks
    if w.shuffle_pages:
        perm = torch.randperm(w.n_pages, generator=_gen(w, 1, "cpu")).to(torch.int32)
    else:
        perm = torch.arange(w.n_pages, dtype=torch.int32)
    out["block_table"] = perm.view(B, nb).to(dev)
    if w.variable_rank:
        u = torch.rand(B, T, generator=_gen(w, 2, "cpu"), dtype=torch.float64)
        cdf = torch.cumsum(torch.tensor(w.rank_probs, dtype=torch.float64), 0)
        cdf[-1] = 1.0
        idx = torch.searchsorted(cdf, u.reshape(-1), right=True).clamp_(max=len(w.rank_choices) - 1)
        ranks = torch.tensor(w.rank_choices, dtype=torch.uint8)[idx].view(B, T)
        out["ranks"] = ranks.to(dev)
    else:
        out["ranks"] = None
    gl = _gen(w, 3, dev)
    if w.tucker:
        rtk, rtv, rf = w.tucker
        assert w.shared and rtk + rtv == w.r_k
        utk = torch.randn(B, T, rtk, generator=gl, device=dev, dtype=torch.float32) / math.sqrt(T)
        utv = torch.randn(B, T, rtv, generator=_gen(w, 4, dev), device=dev, dtype=torch.float32) / math.sqrt(T)
        out["lat_k"], out["lat_v"] = torch.cat([utk, utv], dim=2).contiguous(), None
        for tag, rt, s_uf, s_core in (("k", rtk, 8, 7), ("v", rtv, 9, 17)):
            out[f"t{tag}_uf"] = _orthonormal(w, s_uf, d, rf, B).to(torch.float32).to(dev)
            c = torch.arange(1, rt + 1, dtype=torch.float64) ** -0.35
            c = c / c.pow(2).mean().sqrt()
            core = torch.randn(B, w.n_layers, Hkv, rt, rf, generator=_gen(w, s_core, "cpu"), dtype=torch.float64)
            core *= math.sqrt(T * d / (rt * rf)) * c[:, None]
            out[f"t{tag}_core"] = core.to(torch.float32).to(dev)
    elif w.shared:
        lat = torch.randn(B, T, w.r_k, generator=gl, device=dev, dtype=torch.float32)
        if w.latent_decay:
            lat *= _decay_scale(w.r_k, w.latent_decay, dev)
        out["lat_k"], out["lat_v"] = lat, None
    else:
        lk = torch.randn(B, T, Hkv, w.r_k, generator=gl, device=dev, dtype=torch.float32)
        lv = torch.randn(B, T, Hkv, w.r_v, generator=_gen(w, 4, dev), device=dev, dtype=torch.float32)
        if w.latent_decay:
            lk *= _decay_scale(w.r_k, w.latent_decay, dev)
            lv *= _decay_scale(w.r_v, w.latent_decay, dev)
        out["lat_k"], out["lat_v"] = lk, lv
    if w.residual_bits:  # block-shared mode: one residual per layer and head ([B, T, L, Hkv, d])
        rshape = (B, T, w.n_layers, Hkv, d) if w.shared else (B, T, Hkv, d)
        out["res_k"] = torch.randn(rshape, generator=_gen(w, 5, dev), device=dev) * w.residual_std
        out["res_v"] = torch.randn(rshape, generator=_gen(w, 6, dev), device=dev) * w.residual_std
    else:
        out["res_k"] = out["res_v"] = None
    if w.tucker:
        out["wk"] = out["wv"] = None                     # expanded from the factors by each side
    elif w.shared:
        gw = _gen(w, 7, "cpu")
        shape = (w.n_layers, w.r_k, Hkv * d)
        out["wk"] = (torch.randn(shape, generator=gw) * w.w_std).to(torch.bfloat16).to(dev)
        out["wv"] = (torch.randn(shape, generator=gw) * w.w_std).to(torch.bfloat16).to(dev)
    else:
        out["wk"] = _orthonormal(w, 8, d, w.r_k, Hkv).to(torch.bfloat16).to(dev)
        out["wv"] = _orthonormal(w, 9, d, w.r_v, Hkv).to(torch.bfloat16).to(dev)
    if w.evict_ratio:
        out["layer_scores"] = make_layer_scores(w, dev)
    qshape = ((w.n_layers,) if w.shared else ()) + (B, w.n_q_heads, d)
    q = torch.randn(qshape, generator=_gen(w, 10, "cpu"), dtype=torch.float32) / 8.0
    out["q"] = (q.to(torch.bfloat16) if w.q_bf16 else q).to(dev)
    return out


def make_layer_scores(w: Workload, device="cpu") -> torch.Tensor:
    """fp32 [n_layers, B, T] per-layer token importance of a block: one salience draw per layer, or (evict_cluster
    c > 0) exp(u + 0.3 n) with u ~ N(0, 1.5^2) per run of c tokens, shared by the block's layers, and n ~ N(0, 1)
    per token and layer."""
    B, T = w.B, w.T
    if not w.evict_cluster:
        return torch.stack([make_salience(B, T, seed=w.seed * 10 + l, device=device)
                            for l in range(w.n_layers)]).contiguous()
    c = w.evict_cluster
    g = _gen(w, 40, "cpu")
    u = 1.5 * torch.randn(B, -(-T // c), generator=g, dtype=torch.float64)
    u = u.repeat_interleave(c, dim=1)[:, :T]
    n = torch.randn(w.n_layers, B, T, generator=g, dtype=torch.float64)
    return torch.exp(u[None] + 0.3 * n).to(torch.float32).to(device).contiguous()


def make_dense_inputs(w: Workload, device="cpu") -> dict:
    """A dense paged bf16 cache of the same geometry (keys already rotated) and a rotated bf16 query."""
    dev = torch.device(device)
    shape = (w.n_pages * (w.n_layers if w.shared else 1), w.n_kv_heads, w.page_size, w.head_dim)
    g = _gen(w, 20, dev)
    k = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = (torch.randn(w.B, w.n_q_heads, w.head_dim, generator=_gen(w, 21, "cpu")) / 8.0).to(torch.bfloat16)
    return {"k_pages": k, "v_pages": v, "q": q.to(dev)}


def make_prefill_rows(B: int, max_T: int, n_kv_heads: int, head_dim: int, seed: int = 0, device="cpu",
                      decay: float = 0.7, scale: float = 4.0, mean_norm: float = 1.5) -> torch.Tensor:
    """fp32 rows [B, max_T, Hkv, d] for basis fitting (seeded; the law is in the module docstring)."""
    dev = torch.device(device)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + 30)
    a = torch.randn(n_kv_heads, head_dim, head_dim, generator=g, dtype=torch.float64)
    q, r = torch.linalg.qr(a)
    q = (q * torch.sign(torch.diagonal(r, dim1=-2, dim2=-1)).unsqueeze(-2)).to(torch.float32)
    mu = torch.randn(n_kv_heads, head_dim, generator=g, dtype=torch.float64)
    mu = (mu / mu.norm(dim=-1, keepdim=True) * mean_norm).to(torch.float32)
    s = scale * _decay_scale(head_dim, decay, "cpu")
    gz = torch.Generator(device=dev)
    gz.manual_seed(seed * 1000 + 31)
    x = torch.empty(B, max_T, n_kv_heads, head_dim, dtype=torch.float32, device=dev)
    for h in range(n_kv_heads):
        z = torch.randn(B * max_T, head_dim, generator=gz, device=dev, dtype=torch.float32) * s.to(dev)
        x[:, :, h, :] = (z @ q[h].T.to(dev) + mu[h].to(dev)).view(B, max_T, head_dim)
    return x


def make_window_queries(B: int, W: int, n_q_heads: int, head_dim: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [B, W, Hq, d] pre-RoPE queries of the prefill's last W positions (seeded, N(0, 1))."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed * 1000 + 32)
    return torch.randn(B, W, n_q_heads, head_dim, generator=g, device=device, dtype=torch.float32)


def make_salience(B: int, max_T: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [B, max_T] positive saliences (seeded, exp(N(0, 1.5^2)))."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed * 1000 + 33)
    return torch.exp(1.5 * torch.randn(B, max_T, generator=g, device=device, dtype=torch.float64)).to(torch.float32)


def make_group_rows(B: int, max_T: int, n_layers: int, n_kv_heads: int, head_dim: int, seed: int = 0, device="cpu",
                    rank: int = 512, decay_t: float = 0.5, decay_f: float = 0.7, noise: float = 0.05) -> torch.Tensor:
    """fp32 [B, max_T, L, Hkv, d] keys or values of a layer group (seeded; the law is in the module docstring)."""
    dev = torch.device(device)
    D = n_layers * n_kv_heads * head_dim
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + 34)
    gz = torch.Generator(device=dev)
    gz.manual_seed(seed * 1000 + 35)
    f = _decay_scale(head_dim, decay_f, "cpu").double()
    s = _decay_scale(rank, decay_t, "cpu").double()
    rms = math.sqrt(float((s ** 2).sum() * (f ** 2).mean()) + noise ** 2)
    x = torch.empty(B, max_T, n_layers, n_kv_heads, head_dim, dtype=torch.float32, device=dev)
    for b in range(B):
        q, r = torch.linalg.qr(torch.randn(head_dim, head_dim, generator=g, dtype=torch.float64))
        F = (q * torch.sign(torch.diagonal(r))).to(torch.float32).to(dev)
        z = torch.randn(rank, n_layers * n_kv_heads, head_dim, generator=gz, device=dev) * f.float().to(dev)
        m = (z @ F.T).reshape(rank, D) * s.float().to(dev)[:, None]
        a = torch.randn(max_T, rank, generator=gz, device=dev)
        e = torch.randn(max_T, D, generator=gz, device=dev)
        x[b] = ((a @ m + noise * e) / rms).view(max_T, n_layers, n_kv_heads, head_dim)
    return x


def make_omega(rows: int, cols: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [rows, cols] Gaussian test matrix (seeded, N(0, 1), drawn on the CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + 36)
    return torch.randn(rows, cols, generator=g, dtype=torch.float32).to(device)
