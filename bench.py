"""Benchmark: one decode step of attention over the compressed KV cache (the whole hot path:
paging, latent stream, dequantization, key up-projection, RoPE, scores, online softmax, latent value
accumulation, split merge and value up-projection) on one MI355X, on the batch-16, 32K-context
variable-rank paged workload; the dense bf16 decode kernel on the same geometry is timed beside it,
and the CPU oracle on a bounded sample.

Prints ONE JSON line.  Timing: W untimed warmup steps, then exactly K steps bracketed by
torch.cuda.synchronize() (wall clock: ms_per_step and value); a pair of HIP events recorded by the library
around each timed launch of the attention kernel gives its average duration (the roofline figure); the
dense kernel is timed by wall clock too, after its own warmup.  Each step reads a different replica of
the compressed cache (4 replicas, more than the 256 MB last-level cache holds) so the stream comes from
HBM.  Beside the headline line, `other_workloads` gives the other decode workloads at full size and the
basis fit (kvc_fit_basis) and the salience-driven rank allocation (kvc_salience, kvc_rank_alloc) on the prefill
rows of the 32K workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

WORKLOAD = "varrank_paged_32k"
HBM_PEAK_GBS = 8000.0
REPLICAS = 4
SETTLE_S = 0.4  # seconds of untimed steps before the counted warmup (clock settling)


KERNEL = "decode_int4_kernel"  # the attention kernel this workload runs (kvc_decode_path: INT4)
COUNTERS = os.path.join(HERE, "profiles", "decode_int4_varrank_paged_32k_counters.json")


def source_digest() -> str:
    """Digest of the sources the attention kernel is built from (ties the counter summary to them)."""
    h = hashlib.sha256()
    for f in ("decode_int4.hip", "kvc_common.hpp"):
        h.update(open(os.path.join(HERE, "rank_bit_compressed_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is for this source."""
    try:
        rec = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, min_seconds=10.0):
    """The oracle as it stands, on the whole batch (every sequence and kv head, full context), repeated
    until at least min_seconds of CPU work have been timed."""
    import numpy as np
    import torch
    from oracle import ref

    def np_u16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    L = ref.Layout(**w.layout_kwargs())
    bt = inp["block_table"].numpy()
    sl = inp["seq_len"].numpy()
    pool, page_off, tok_rank, tok_off = ref.compress(
        L, bt, sl, w.T, inp["ranks"].numpy(), inp["lat_k"].float().numpy(), inp["lat_v"].float().numpy(), None,
        None, w.n_pages, ref.page_bytes_uniform(L) * w.n_pages)
    q = inp["q"].float().numpy()
    wk, wv = np_u16(inp["wk"]), np_u16(inp["wv"])
    reps, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        out = ref.decode_attn(L, bt, sl, inp["q_pos"].numpy(), pool, page_off, tok_rank, tok_off, q, wk, wv)
        dt += time.perf_counter() - t0
        reps += 1
    assert np.isfinite(out).all()
    return {"value": round(reps * w.B / dt, 4), "unit": "tokens/s", "cores": min(ref.threads(), w.B * w.n_kv_heads),
            "kind": "oracle",
            "sample": f"{reps} decode step(s) of the whole batch ({w.B} sequences x {w.n_kv_heads} kv heads x "
                      f"{w.T} tokens), fp64 C oracle with OpenMP over (sequence, kv head), {dt:.2f} s timed; "
                      f"compression excluded"}


MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3
# basis fitting on the prefill of the 32K decode workload: 16 sequences x 32768 rows x 8 KV heads x 128
FIT_SHAPE = (16, 32768, 8, 128)
FIT_RANK = 64
# salience-driven rank allocation on the same prefill: a 32-query window, the 32K workload's ladder and mean rank
SAL_WINDOW = 32
ALLOC_LADDER, ALLOC_WEIGHTS, ALLOC_MEAN = [8, 16, 32, 64], [1.0, 0.45, 0.2], 20.8

# The other workloads of the hot path, each timed on its own bound: the uniform-rank 8K layer (cache-resident,
# a latency figure), the block-shared latent (bound by the matrix cores: the key up-projection of every layer
# and head from the 512-dim latent) and the 128K rotated-residual cache (HBM); the lower-bit codecs; and a layer
# group in partial Tucker form (the block-shared kernel over per-sequence up-projections expanded from the core);
# the block-shared latent under one eviction decision for its layers (the decision timed on its own), masked in
# place or compacted out of the pages (the compaction timed on its own).
OTHER = ("llama8b_layer_8k", "shared_latent_32k", "shared_latent_32k_int3", "residual_128k", "varrank_paged_32k_int3",
         "llama8b_layer_8k_k3v2",
         "tucker_group_32k", "tucker_group_32k_res", "shared_latent_32k_evict30", "shared_latent_32k_evict30_clustered",
         "shared_latent_32k_evict30_compact")


def decode_flops(w, ranks=None) -> int:
    """Algorithmic flops of one decode step: key up-projection, scores and the latent value product (the
    residual's Hadamard rotations are a fast transform, a few adds per element, and are not counted).  Under
    variable rank each token counts its own rank (ranks: [B, T] uint8), not the cap the storage allows."""
    import torch

    n_tok = w.B * w.T * (w.n_layers if w.shared else 1)
    score = 2 * w.head_dim * w.n_q_heads * n_tok
    if w.tucker:  # keys need only the key factor's rows of the latent; the values' product runs over all of it
        return n_tok * (2 * w.head_dim * w.tucker[0] * w.n_kv_heads + 2 * w.r_v * w.n_q_heads) + score
    if w.variable_rank:
        r_sum = int(ranks[:, : w.T].to(torch.int64).sum())  # every sequence holds w.T tokens here
        return 2 * w.head_dim * w.n_kv_heads * r_sum + score + 2 * w.n_q_heads * r_sum
    return n_tok * (2 * w.head_dim * w.r_k * w.n_kv_heads + 2 * w.r_v * w.n_q_heads) + score


def other_workloads(steps: int, warmup: int, peaks: dict, names=OTHER) -> dict:
    """Each other workload at its full size: median kernel time (library events around the attention
    kernel), wall time per call, and the figure of its own bound."""
    import torch
    from rank_bit_compressed_amd import accounting, kvc, synth

    res = {}
    for name in names:
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w, device="cuda")
        L = kvc.make_layout(**w.layout_kwargs())
        cache = kvc.DeviceCache.allocate(L, w.n_pages)
        kvc.compress(L, cache, inp["block_table"], inp["seq_len"], w.T, ranks=inp["ranks"], lat_k=inp["lat_k"],
                     lat_v=inp["lat_v"], res_k=inp["res_k"], res_v=inp["res_v"])
        extra = {}
        if w.tucker:  # per-sequence up-projections from the factors (prefill side; timed on its own)
            xe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            for _ in range(5):
                xe[0].record()
                wk, _ = kvc.tucker_expand(inp["tk_uf"], inp["tk_core"], w.r_k, 0)
                wv, _ = kvc.tucker_expand(inp["tv_uf"], inp["tv_core"], w.r_k, w.tucker[0])
                xe[1].record()
                torch.cuda.synchronize()
                times.append(xe[0].elapsed_time(xe[1]))
            inp["wk"], inp["wv"] = wk, wv
            extra = {"tucker_expand_ms_median": round(sorted(times)[2], 5),
                     "per_sequence_w_bytes": 2 * wk.numel() * 2, "kv_split": w.tucker[0]}
        keep = None
        if w.evict_ratio:  # the block's eviction decision from its layers' scores (prefill side; timed on its own)
            xe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            for _ in range(5):
                xe[0].record()
                keep = kvc.evict_select(inp["layer_scores"], inp["seq_len"], w.evict_ratio)
                xe[1].record()
                torch.cuda.synchronize()
                times.append(xe[0].elapsed_time(xe[1]))
            words = keep.view(-1).tolist()
            kept = int(sum(bin(x & 0xFFFFFFFF).count("1") for x in words))
            extra = {"evict_select_ms_median": round(sorted(times)[2], 5), "kept_fraction": round(kept / (w.B * w.T), 4),
                     "empty_super_tile_fraction": round(sum(1 for x in words if x == 0) / len(words), 4)}
        dcache, bt, sl, tok_pos, max_T = cache, inp["block_table"], inp["seq_len"], None, w.T
        if w.evict_compact:  # kept tokens moved into new pages (prefill side; timed on its own)
            rec = int(cache.page_off[1].item() - cache.page_off[0].item())
            dcache = kvc.DeviceCache(L, torch.zeros_like(cache.pool), torch.arange(w.n_pages, dtype=torch.int64,
                                     device="cuda") * rec, None, None, torch.zeros(2, dtype=torch.int64, device="cuda"),
                                     w.n_pages)
            bt = inp["block_table"].flip(1).contiguous()
            xe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            times = []
            for _ in range(5):
                xe[0].record()
                sl, tok_pos = kvc.evict_compact(L, cache, dcache, inp["block_table"], inp["seq_len"], keep, bt)
                xe[1].record()
                torch.cuda.synchronize()
                times.append(xe[0].elapsed_time(xe[1]))
            extra["evict_compact_ms_median"] = round(sorted(times)[2], 5)
            extra["slots_fraction"] = round(int(sl.sum().item()) / (w.B * w.T), 4)
            max_T = max(1, int(sl.max().item()))  # the compacted lengths size the decode's grid
            keep = None
            del cache
            cache = dcache
        plan = kvc.DecodePlan(L, dcache, bt, sl, inp["q"], inp["wk"], inp["wv"], max_T, q_pos=inp["q_pos"],
                              keep_mask=keep, kv_split=w.tucker[0] if w.tucker else 0, tok_pos=tok_pos)
        for k in ("lat_k", "lat_v", "res_k", "res_v"):
            inp[k] = None
        n = max(20, steps // 10)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            b.record()
        for _ in range(max(20, warmup // 10)):
            plan()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            plan(ev[i])
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / n
        ks = sorted(a.elapsed_time(b) for a, b in ev)
        k_ms = ks[n // 2]
        acct = accounting.compressed_stream_bytes(w, inp["ranks"], [w.T] * w.B)
        nbytes = acct["stream"] + acct["tables"]
        flops = decode_flops(w, inp["ranks"])
        if w.evict_ratio:  # attention runs over the kept tokens only (every token's latent is still read)
            flops = int(round(flops * extra["kept_fraction"]))
        if w.evict_compact:  # ... and only the compacted slots are read
            nbytes = int(round(acct["stream"] * extra["slots_fraction"])) + acct["tables"]
        path = {kvc.PATH_HEAD: "general per-head kernel", kvc.PATH_INT4: "INT4 kernel",
                kvc.PATH_SHARED: "block-shared kernel", kvc.PATH_RES: "INT4 residual kernel"}[kvc.decode_path(L)]
        r = {"kernel": path, "kernel_ms_median": round(k_ms, 5), "ms_per_call": round(wall_ms, 5),
             "compressed_bytes": nbytes, "hbm_gbs": round(nbytes / (k_ms * 1e-3) / 1e9, 1),
             "flops": flops, "tflops": round(flops / (k_ms * 1e-3) / 1e12, 1), **extra}
        if name.startswith("llama8b_layer_8k"):
            r["bound"] = "latency (the 4.7 MB cache stays in the last-level cache between calls)"
        elif w.shared:
            r["bound"] = "mfma"
            r["frac_of_f16_mfma_peak"] = round(r["tflops"] / MFMA_F16_PEAK_TFLOPS, 4)
            r["frac_of_measured_mfma"] = round(r["tflops"] / peaks["mfma_f16_tflops"], 4)
        else:
            r["bound"] = "hbm"
            r["frac_of_hbm_peak"] = round(r["hbm_gbs"] / HBM_PEAK_GBS, 4)
            r["frac_of_measured_hbm"] = round(r["hbm_gbs"] / peaks["hbm_read_gbs"], 4)
        res[name] = r
        del plan, cache, dcache, inp
        torch.cuda.empty_cache()
    return res


def fit_workload(steps: int) -> dict:
    """kvc_fit_basis on the prefill rows of the 32K workload: the Gram-matrix kernel's median duration (library
    events around it), the whole call's wall time, and the Gram kernel's figure against the fp32 matrix peak.
    Algorithmic flops: 2 per multiply-add over the d (d + 1) / 2 distinct entries of each head's symmetric
    Gram matrix, per row."""
    import torch
    from rank_bit_compressed_amd import kvc, synth

    B, T, Hkv, d = FIT_SHAPE
    x = synth.make_prefill_rows(B, T, Hkv, d, seed=6, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.fit_workspace_bytes(kvc.fit_in(x, sl, FIT_RANK)), dtype=torch.uint8, device="cuda")
    n = max(10, steps // 100)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        b.record()
    for _ in range(3):
        kvc.fit_basis(x, sl, FIT_RANK, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        kvc.fit_basis(x, sl, FIT_RANK, ws=ws, events=ev[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / n
    g_ms = sorted(a.elapsed_time(b) for a, b in ev)[n // 2]
    rows = B * T * Hkv
    flops = 2 * rows * (d * (d + 1) // 2)
    tflops = flops / (g_ms * 1e-3) / 1e12
    nbytes = rows * d * 4
    del x, ws
    torch.cuda.empty_cache()
    return {"kernel": "fit_gram_kernel (Gram matrix, fp32 matrix instructions)", "rows": rows, "rank": FIT_RANK,
            "gram_kernel_ms_median": round(g_ms, 5), "ms_per_call": round(wall_ms, 5),
            "gram_flops": flops, "tflops": round(tflops, 1), "bound": "mfma",
            "frac_of_fp32_mfma_peak": round(tflops / MFMA_F32_PEAK_TFLOPS, 4), "input_bytes": nbytes,
            "hbm_gbs": round(nbytes / (g_ms * 1e-3) / 1e9, 1),
            "rest_of_call": "split reduction and the per-head Jacobi eigensolver (one workgroup per head)"}


TFIT_SHAPE = (4, 32768, 4, 8, 128)   # the Tucker group: sequences, tokens, layers, KV heads, head dim
TFIT_RANKS = (256, 256, 64, 1)       # key and value token ranks, feature rank, power iterations


def tucker_fit_workload(steps: int) -> dict:
    """kvc_tucker_fit of the keys and of the values of the 4 x 32K-token, 4-layer, 8-head group (token ranks
    256 + 256, feature rank 64, one power iteration): median time of the two calls, on two streams (reported)
    and one after the other on one stream, and the large products' figure against the fp32 matrix peak.  Algorithmic flops: the
    four products with the token-mode unfolding per sequence and fit (A Omega, A^T Q, A Z, Q^T A), 2 T D r_t
    each; the orthonormalisations, the feature fit and the core's last product are counted as overhead."""
    import torch
    from rank_bit_compressed_amd import kvc, synth

    B, T, L, H, d = TFIT_SHAPE
    rtk, rtv, rf, q = TFIT_RANKS
    D = L * H * d
    xk = synth.make_group_rows(B, T, L, H, d, seed=8, device="cuda")
    xv = synth.make_group_rows(B, T, L, H, d, seed=9, device="cuda")
    ok, ov = synth.make_omega(D, rtk, seed=8, device="cuda"), synth.make_omega(D, rtv, seed=9, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    lat = torch.empty(B, T, rtk + rtv, device="cuda")
    need = max(kvc.tucker_fit_workspace_bytes(kvc.tucker_fit_in(xk, sl, ok, rtk, rf, q, rtk + rtv)),
               kvc.tucker_fit_workspace_bytes(kvc.tucker_fit_in(xv, sl, ov, rtv, rf, q, rtk + rtv)))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    s_k, s_v = torch.cuda.Stream(), torch.cuda.Stream()  # default priority

    def run_one_stream():
        kvc.tucker_fit(xk, sl, ok, rtk, rf, q, u_t=lat[:, :, :rtk], ws=ws)
        kvc.tucker_fit(xv, sl, ov, rtv, rf, q, u_t=lat[:, :, rtk:], ws=ws)

    def run_two_streams():
        # keys and values are independent fits: on two streams, one's sequential pivots overlap the other's products
        main = torch.cuda.current_stream()
        s_k.wait_stream(main)
        s_v.wait_stream(main)
        with torch.cuda.stream(s_k):
            kvc.tucker_fit(xk, sl, ok, rtk, rf, q, u_t=lat[:, :, :rtk], ws=ws)
        with torch.cuda.stream(s_v):
            kvc.tucker_fit(xv, sl, ov, rtv, rf, q, u_t=lat[:, :, rtk:], ws=ws2)
        main.wait_stream(s_k)
        main.wait_stream(s_v)

    def timed(run):
        n = max(5, steps // 200)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            run()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[n // 2]

    ms1 = timed(run_one_stream)
    ms = timed(run_two_streams)
    flops = sum(4 * 2 * B * T * D * r for r in (rtk, rtv))
    tflops = flops / (ms * 1e-3) / 1e12
    del xk, xv, ws, ws2, lat
    torch.cuda.empty_cache()
    return {"kernel": "gemm_kernel (fp32 matrix instructions) and the CholeskyQR2 orthonormalisations",
            "shape": {"sequences": B, "tokens": T, "layers": L, "kv_heads": H, "head_dim": d, "r_t_keys": rtk,
                      "r_t_values": rtv, "r_f": rf, "power_iters": q},
            "ms_per_group_fit_median": round(ms, 4), "streams": "keys and values on two streams",
            "ms_per_group_fit_one_stream": round(ms1, 4), "product_flops": flops, "tflops": round(tflops, 1),
            "bound": "mfma", "frac_of_fp32_mfma_peak": round(tflops / MFMA_F32_PEAK_TFLOPS, 4)}


def alloc_workload(steps: int) -> dict:
    """kvc_salience (window queries over the prefill keys) and kvc_rank_alloc on the prefill of the 32K workload:
    median times from events on the library's stream (the current torch stream).  Algorithmic flops of the
    salience: one q.k per (window query, query head, key), 2 d each; the two passes recompute them."""
    import torch
    from rank_bit_compressed_amd import kvc, synth

    B, T, Hkv, d = FIT_SHAPE
    Hq = 4 * Hkv
    k = synth.make_prefill_rows(B, T, Hkv, d, seed=3, device="cuda")
    q = synth.make_window_queries(B, SAL_WINDOW, Hq, d, seed=3, device="cuda")
    sl = torch.full((B,), T, dtype=torch.int32, device="cuda")
    sal = torch.empty(B, T, device="cuda")
    ranks = torch.empty(B, T, dtype=torch.uint8, device="cuda")
    ws = torch.empty(kvc.salience_workspace_bytes(kvc.salience_in(q, k, sl, 5e5)), dtype=torch.uint8, device="cuda")
    n = max(10, steps // 100)

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[n // 2]

    s_ms = timed(lambda: kvc.salience(q, k, sl, 5e5, out=sal, ws=ws))
    a_ms = timed(lambda: kvc.rank_alloc(sal, sl, ALLOC_LADDER, ALLOC_WEIGHTS, ALLOC_MEAN, out=ranks))
    mean_rank = float(ranks.float().mean().item())
    flops = 2 * d * SAL_WINDOW * Hq * B * T
    tflops = flops / (s_ms * 1e-3) / 1e12
    del k, q, ws
    torch.cuda.empty_cache()
    return {"kernel": "sal_kernel (two passes, fp32 matrix instructions) + rank_alloc_kernel", "window": SAL_WINDOW,
            "salience_ms_median": round(s_ms, 5), "alloc_ms_median": round(a_ms, 5),
            "salience_flops": flops, "tflops": round(tflops, 1), "bound": "mfma",
            "frac_of_fp32_mfma_peak": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
            "ladder": ALLOC_LADDER, "mean_rank_target": ALLOC_MEAN, "mean_rank_allocated": round(mean_rank, 3)}


def measured_peaks(torch, dev) -> dict:
    """Measured peaks beside the published ones: the HBM read rate of a plain 16-byte-per-lane stream over 4 GiB
    (kvc_probe_stream_read) and the rate of the fp16 32x32x16 matrix instruction on register operands
    (kvc_probe_mfma_f16); median of 5 timed runs each, after 2 untimed."""
    from rank_bit_compressed_amd import kvc

    def timed(fn, n=5):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[n // 2]

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    grid = 32768
    sink = torch.empty(grid, dtype=torch.int32, device=dev)
    ms = timed(lambda: kvc.probe_stream_read(buf, grid, sink))
    del buf
    iters, mgrid = 4000, 256 * 8
    fsink = torch.empty(mgrid, dtype=torch.float32, device=dev)
    mms = timed(lambda: kvc.probe_mfma_f16(iters, mgrid, fsink))
    clk = clock_mhz(torch, dev)  # right behind the last matrix-instruction run
    flops = mgrid * 4 * iters * 8 * 2 * 32 * 32 * 16
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "hbm_read_bytes": nbytes,
            "mfma_f16_tflops": round(flops / (mms * 1e-3) / 1e12, 1), "clock_mhz_after_mfma": clk,
            "kernels": "kvc_probe_stream_read (16-byte nontemporal loads, 8 in flight, 32768 x 256 lanes over 4 GiB), "
                       "kvc_probe_mfma_f16 "
                       "(8 independent v_mfma_f32_32x32x16_f16 chains per wave, 8192 waves)"}


def clock_mhz(torch, dev) -> float:
    """Shader clock now (kvc_probe_clock: s_memtime cycles over 100 MHz s_memrealtime ticks)."""
    from rank_bit_compressed_amd import kvc
    out = torch.zeros(3, dtype=torch.int64, device=dev)
    kvc.probe_clock(out)
    c, r, _ = out.tolist()
    return round(c / max(r, 1) * 100.0, 1)


def step_percentiles(torch, plan, dev, n=100) -> dict:
    """p10 / median / p90 in ms over n steps, warm (one cache, back to back, so its 126 MB can stay in the 256 MB
    last-level cache) and cold (1 GiB written before each step, outside the events), each after 0.1 s of
    untimed steps (the clock drops while the GPU idles, e.g. during the single-wave clock probe before).  "kernel": the attention
    kernel alone, from the library's events around its launch; "step": kernel + merge from events around the
    call (cold only: back to back, such events would also time host enqueue gaps); "step_mean": warm steps
    between two events around all n."""
    def pct(xs):
        xs = sorted(xs)
        return {q: round(xs[min(len(xs) - 1, int(f * (len(xs) - 1) + 0.5))], 5)
                for q, f in (("p10", 0.1), ("median", 0.5), ("p90", 0.9))}

    def evs(m):
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(m)]
        for a, b in e:
            a.record()
            b.record()
        return e

    def settle():
        # the clock falls while the GPU idles (after a probe, between samples): untimed steps first
        t = time.perf_counter()
        while time.perf_counter() - t < 0.1:
            for _ in range(16):
                plan()
            torch.cuda.synchronize()

    kev, sev, blk = evs(n), evs(n), evs(1)[0]
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    settle()
    blk[0].record()
    for i in range(n):
        plan(kev[i])
    blk[1].record()
    clk_warm = clock_mhz(torch, dev)  # enqueued right behind the warm block
    torch.cuda.synchronize()
    res = {"n": n, "warm": {"kernel": pct([a.elapsed_time(b) for a, b in kev]),
                            "step_mean": round(blk[0].elapsed_time(blk[1]) / n, 5), "clock_mhz_after": clk_warm}}
    settle()
    for i in range(n):
        flush.fill_(float(i))
        sev[i][0].record()
        plan(kev[i])
        sev[i][1].record()
    clk_cold = clock_mhz(torch, dev)
    torch.cuda.synchronize()
    res["cold"] = {"kernel": pct([a.elapsed_time(b) for a, b in kev]), "step": pct([a.elapsed_time(b) for a, b in sev]),
                   "clock_mhz_after": clk_cold}
    del flush
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads' figures")
    ap.add_argument("--only", choices=["tucker_fit_group_32k", *OTHER],
                    help="run only this figure (the Tucker fit or one of the other decode workloads) and print it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path here "
              f"has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    from rank_bit_compressed_amd import accounting, kvc, synth

    if args.only == "tucker_fit_group_32k":
        print(json.dumps({"workload": args.only, **tucker_fit_workload(args.steps)}), flush=True)
        return
    if args.only:
        print(json.dumps({"workload": args.only, **other_workloads(args.steps, args.warmup, measured_peaks(torch, "cuda"),
                                                                    (args.only,))[args.only]}), flush=True)
        return
    w = synth.WORKLOADS[WORKLOAD]
    dev = "cuda"
    inp = synth.make_inputs(w, device=dev)
    L = kvc.make_layout(**w.layout_kwargs())
    base = kvc.DeviceCache.allocate(L, w.n_pages)
    kvc.compress(L, base, inp["block_table"], inp["seq_len"], w.T, ranks=inp["ranks"], lat_k=inp["lat_k"],
                 lat_v=inp["lat_v"])
    torch.cuda.synchronize()
    used = int(base.used_bytes[0])
    caches = [base]
    for _ in range(REPLICAS - 1):
        c = kvc.DeviceCache(L, base.pool.clone(), base.page_off.clone(), base.tok_rank.clone(), base.tok_off.clone(),
                            base.used_bytes.clone(), w.n_pages)
        caches.append(c)
    cpu_inp = {k: inp[k] for k in ("lat_k", "lat_v", "ranks", "seq_len", "q_pos", "q", "wk", "wv", "block_table")}
    bt, sl, q, wk, wv, qp = inp["block_table"], inp["seq_len"], inp["q"], inp["wk"], inp["wv"], inp["q_pos"]
    ws = torch.empty(kvc.decode_workspace_bytes(L, w.B, w.T), dtype=torch.uint8, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)

    plans = [kvc.DecodePlan(L, c, bt, sl, q, wk, wv, w.T, q_pos=qp, out=out, ws=ws) for c in caches]

    def step(i, events=None):
        plans[i % REPLICAS](events)

    if kvc.decode_path(L) != kvc.PATH_INT4:
        raise RuntimeError(f"{WORKLOAD} is expected to run the INT4 kernel")
    # Kernel events, recorded by the library on the launch stream right around the attention kernel (the split
    # merge is outside), one pair per timed step.  They are created (at their first record) before the warmup,
    # so that no host work leaves the GPU idle between the warmup and the timed steps.
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in kev:
        a.record()
        b.record()
    # The GPU clock needs some tens of milliseconds of load to settle (the first launches run about 15% slower):
    # untimed steps for a fixed wall time come first, whatever the warmup count, so that the timed steps and the
    # kernel's events see the settled clock.
    t_set = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_set < SETTLE_S:
        for _ in range(64):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        step(i, kev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    assert torch.isfinite(out).all()
    kernel_ms = [a.elapsed_time(b) for a, b in kev]
    ms_per_step = wall * 1e3 / args.steps
    kernel_avg = sum(kernel_ms) / len(kernel_ms)

    acct = accounting.compressed_stream_bytes(w, inp["ranks"], [w.T] * w.B)
    alg_bytes = acct["stream"] + acct["tables"]
    achieved = alg_bytes / (kernel_avg * 1e-3) / 1e9
    clk_timed = clock_mhz(torch, dev)  # right after the timed steps
    step_ms = step_percentiles(torch, plans[0], dev)
    peaks = measured_peaks(torch, dev)

    dense = None
    if not args.no_dense:
        del inp
        dd = synth.make_dense_inputs(w, device=dev)
        dws = torch.empty(kvc.dense_workspace_bytes(kvc.dense_in(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size,
                                                                  bt, sl, dd["k_pages"], dd["v_pages"], dd["q"],
                                                                  w.T)), dtype=torch.uint8, device=dev)
        dout = torch.empty(dd["q"].shape, dtype=torch.float32, device=dev)

        def dstep():
            kvc.dense_decode_attn(w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size, bt, sl, dd["k_pages"],
                                  dd["v_pages"], dd["q"], w.T, out=dout, ws=dws)

        for _ in range(max(3, args.warmup // 4)):
            dstep()
        torch.cuda.synchronize()
        nd = max(10, args.steps // 4)
        t0 = time.perf_counter()
        for i in range(nd):
            dstep()
        torch.cuda.synchronize()
        d_ms = (time.perf_counter() - t0) * 1e3 / nd
        d_bytes = w.B * w.T * accounting.dense_bytes_per_token(w.n_kv_heads, w.head_dim)
        dense = {"ms_per_step": round(d_ms, 5), "hbm_gbs": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
                 "frac_of_hbm_peak": round(d_bytes / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "frac_of_measured_hbm": round(d_bytes / (d_ms * 1e-3) / 1e9 / peaks["hbm_read_gbs"], 4),
                 "bytes": d_bytes, "speedup_compressed_vs_dense": round(d_ms / ms_per_step, 3)}
        del dd

    tokens_per_s = w.B / (ms_per_step * 1e-3)
    line = {
        "metric": "compressed decode-attn tokens/s & HBM GB/s (% peak), speedup vs dense bf16 @32K",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": w.B, "context": w.T, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ranks": "8/16/32/64 w.p. .4/.3/.2/.1",
                   "rank_cap": w.r_k, "latent": "INT4, group 32, fp16 scale+zero", "page_size": w.page_size,
                   "block_table": "shuffled", "rope_theta": w.rope_theta},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(KERNEL),
                     "kernel": KERNEL, "kernel_ms_avg": round(kernel_avg, 5),
                     "peak_measured": peaks["hbm_read_gbs"],
                     "frac_of_measured": round(achieved / peaks["hbm_read_gbs"], 4),
                     "clock_mhz_after_timed_steps": clk_timed},
        "measured_peaks": peaks,
        "context_tokens_per_s": round(w.B * w.T / (ms_per_step * 1e-3), 1),
        "step_ms": step_ms,
        "compressed_bytes_per_step": alg_bytes,
        "dense": dense,
    }
    if not args.no_other:
        line["other_workloads"] = other_workloads(args.steps, args.warmup, peaks)
        line["other_workloads"]["basis_fit_prefill_32k"] = fit_workload(args.steps)
        line["other_workloads"]["rank_alloc_prefill_32k"] = alloc_workload(args.steps)
        line["other_workloads"]["tucker_fit_group_32k"] = tucker_fit_workload(args.steps)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, {k: (v.cpu() if v is not None else None) for k, v in cpu_inp.items()})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
