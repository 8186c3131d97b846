"""The C ABI library loads, exports every call include/kvc.h declares, and rejects bad
arguments before launching anything (these calls need no GPU)."""
import ctypes as C
import os
import re

import pytest

from rank_bit_compressed_amd import kvc, synth


def header_functions():
    src = open(kvc.HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(kvc_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_header():
    names = header_functions()
    assert set(names) == set(kvc.EXPORTS)
    L = C.CDLL(kvc.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert kvc.lib().kvc_abi_version() == 8
    assert kvc.lib().kvc_status_string(-3) == b"workspace or pool too small"


def test_layout_checks():
    for name, w in synth.WORKLOADS.items():
        st = kvc.layout_check(kvc.make_layout(**w.layout_kwargs()))
        assert st in (0, -2), (name, st)
    ok = kvc.make_layout(**synth.WORKLOADS["varrank_paged_32k"].layout_kwargs())
    assert kvc.layout_check(ok) == 0
    for field, val, want in [("n_kv_heads", 0, -1), ("r_k_cap", 12, -1), ("latent_bits", 8, -1),
                             ("residual_bits", 3, -1), ("page_size", 512, -1), ("page_size", 48, -2),
                             ("group", 24, -2), ("n_q_heads", 48, -2), ("rope_theta", -1.0, -1)]:
        bad = kvc.make_layout(**synth.WORKLOADS["varrank_paged_32k"].layout_kwargs())
        setattr(bad, field, val)
        assert kvc.layout_check(bad) == want, (field, val)


def test_pool_bytes_closed_form():
    w = synth.WORKLOADS["llama8b_layer_8k"]
    L = kvc.make_layout(**w.layout_kwargs())
    # per head block: K codes 256*24, V codes 256*32, K pairs 256*2*4, V pairs 256*2*4 (all 16-aligned)
    assert kvc.pool_bytes_max(L, 10) == 10 * 8 * 256 * (24 + 32 + 8 + 8)


def test_calls_reject_bad_arguments_without_launching():
    w = synth.WORKLOADS["varrank_paged_32k"]
    L = kvc.make_layout(**w.layout_kwargs())
    lib = kvc.lib()
    out = C.c_size_t()
    assert lib.kvc_decode_workspace_bytes(C.byref(L), 0, 100, 0, C.byref(out)) == -1
    assert lib.kvc_decode_workspace_bytes(C.byref(L), 2, 100, 0, C.byref(out)) == 0 and out.value > 0
    cache = kvc.Cache(None, 0, None, None, None, None, 0)
    inp = kvc.DecodeIn(2, 1, 100, None, None, None, None, 0, None, None, 0, 0, None, 0, 0)
    assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), C.c_void_p(16), C.c_void_p(16), 1 << 20,
                               None) == -1
    cin = kvc.CompressIn(0, 2, 100, 1, *([None] * 11))
    assert lib.kvc_compress(C.byref(L), C.byref(cin), C.byref(cache), None) == -1
    # misaligned pointers are refused before any launch
    cache = kvc.Cache(C.c_void_p(16), 1 << 30, C.c_void_p(32), C.c_void_p(48), C.c_void_p(64), None, 4)
    inp = kvc.DecodeIn(2, 1, 100, C.c_void_p(80), C.c_void_p(96), None, C.c_void_p(113), 1, C.c_void_p(128),
                       C.c_void_p(144), 0, 0, None, 0, 0)
    assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), C.c_void_p(160), C.c_void_p(176), 1 << 30,
                               None) == -4


def test_decode_path_selection():
    """The INT4 fast kernel serves every INT4, head-dim-128, residual-free per-head layout of the workloads
    (and their scaled test copies), the INT4 residual kernel the residual workload; the others go to the
    general per-head or the block-shared kernel."""
    want = {"tiny": kvc.PATH_HEAD, "llama8b_layer_8k": kvc.PATH_INT4, "varrank_paged_32k": kvc.PATH_INT4,
            "shared_latent_32k": kvc.PATH_SHARED, "residual_128k": kvc.PATH_RES,
            "varrank_paged_32k_int3": kvc.PATH_INT4, "llama8b_layer_8k_k3v2": kvc.PATH_INT4,
            "tucker_group_32k": kvc.PATH_SHARED, "shared_latent_32k_evict30": kvc.PATH_SHARED,
            "shared_latent_32k_evict30_clustered": kvc.PATH_SHARED,
            "shared_latent_32k_evict30_compact": kvc.PATH_SHARED, "tucker_group_32k_res": kvc.PATH_SHARED, "shared_latent_32k_int3": kvc.PATH_SHARED}
    for name, w in synth.WORKLOADS.items():
        assert kvc.decode_path(kvc.make_layout(**w.layout_kwargs())) == want[name], name
        small = w.scaled(B=2, T=700, page_size=128) if not w.shared else w.scaled(B=1, T=700)
        assert kvc.decode_path(kvc.make_layout(**small.layout_kwargs())) == want[name], name


def test_fit_calls_reject_bad_arguments_without_launching():
    lib = kvc.lib()
    out = C.c_size_t()
    ok = kvc.FitIn(2, 1000, 8, 128, 64, 64, None, None)
    assert lib.kvc_fit_workspace_bytes(C.byref(ok), C.byref(out)) == 0
    # 2 x 1000 rows -> 2 work items of 1024 tokens, so 2 slices: partials 8 x 2 x 10 tiles, and G 8 x 128 x 128
    assert out.value == (8 * 2 * 10 * 1024 + 8 * 128 * 128) * 4
    for fields, want in [((0, 1000, 8, 128, 64, 64), -1), ((2, 1000, 8, 64, 32, 32), -2),
                         ((2, 1000, 8, 128, 0, 64), -1), ((2, 1000, 8, 128, 65, 64), -1),
                         ((2, 1000, 8, 128, 64, 129), -1)]:
        bad = kvc.FitIn(*fields, None, None)
        assert lib.kvc_fit_workspace_bytes(C.byref(bad), C.byref(out)) == want, fields
    # null inputs, no outputs, misaligned pointers and a short workspace are refused before any launch
    v = C.c_void_p
    assert lib.kvc_fit_basis(C.byref(ok), v(16), None, None, v(32), 1 << 30, None) == -1
    good = kvc.FitIn(2, 1000, 8, 128, 64, 64, v(48), v(64))
    assert lib.kvc_fit_basis(C.byref(good), None, None, None, v(32), 1 << 30, None) == -1
    assert lib.kvc_fit_basis(C.byref(good), v(18), None, None, v(32), 1 << 30, None) == -4
    assert lib.kvc_fit_basis(C.byref(good), v(16), None, None, v(32), 1024, None) == -3
    # the timed entry needs both events, and otherwise checks as the plain one
    assert lib.kvc_fit_basis_timed(C.byref(good), v(16), None, None, v(32), 1 << 30, None, None, v(64)) == -1
    assert lib.kvc_fit_basis_timed(C.byref(good), v(18), None, None, v(32), 1 << 30, None, v(48), v(64)) == -4


def test_salience_and_alloc_reject_bad_arguments_without_launching():
    lib = kvc.lib()
    v = C.c_void_p
    out = C.c_size_t()
    ok = kvc.SalienceIn(2, 1000, 32, 32, 8, 128, 5e5, None, None, None)
    assert lib.kvc_salience_workspace_bytes(C.byref(ok), C.byref(out)) == 0 and out.value > 0
    for f, val, want in [("W", 0, -1), ("W", 33, -2), ("n_q_heads", 20, -1), ("n_q_heads", 24, -2),
                         ("head_dim", 64, -2), ("rope_theta", -1.0, -1)]:
        bad = kvc.SalienceIn(2, 1000, 32, 32, 8, 128, 5e5, None, None, None)
        setattr(bad, f, val)
        assert lib.kvc_salience_workspace_bytes(C.byref(bad), C.byref(out)) == want, f
    good = kvc.SalienceIn(2, 1000, 32, 32, 8, 128, 5e5, v(16), v(32), v(48))
    assert lib.kvc_salience(C.byref(ok), v(64), v(80), 1 << 30, None) == -1          # null inputs
    assert lib.kvc_salience(C.byref(good), v(66), v(80), 1 << 30, None) == -4        # misaligned output
    assert lib.kvc_salience(C.byref(good), v(64), v(80), 16, None) == -3             # short workspace

    def ain(**kw):
        d = dict(B=2, max_T=100, ladder=[8, 16, 32, 64], w=[4.0, 2.0, 1.0], mean=20.0, seq=v(16), sal=v(32))
        d.update(kw)
        lad = (C.c_int32 * 8)(*(d["ladder"] + [0] * (8 - len(d["ladder"]))))
        w = (C.c_float * 7)(*(d["w"] + [0.0] * (7 - len(d["w"]))))
        return kvc.AllocIn(d["B"], d["max_T"], len(d["ladder"]), lad, w, d["mean"], d["seq"], d["sal"])
    for kw in [dict(ladder=[8]), dict(ladder=[8, 8, 16], w=[1.0, 0.5]), dict(ladder=[8, 300], w=[1.0]),
               dict(w=[1.0, 2.0, 0.5]), dict(w=[1.0, -0.5, 0.0]), dict(mean=7.0), dict(mean=65.0), dict(sal=None),
               dict(B=0)]:
        assert lib.kvc_rank_alloc(C.byref(ain(**kw)), v(48), None) == -1, kw
    assert lib.kvc_rank_alloc(C.byref(ain(sal=v(33))), v(48), None) == -4


def test_low_bit_layouts_check_and_route():
    # INT3, INT2 and 3-bit keys with 2-bit values are valid per-head layouts: the fast kernel serves the
    # combinations it is compiled for, the general kernel the others (and the residual); block-shared stays INT4
    base = synth.WORKLOADS["llama8b_layer_8k"]
    for kw, path in [(dict(latent_bits=3), kvc.PATH_INT4), (dict(latent_bits=2), kvc.PATH_INT4),
                     (dict(latent_bits=3, latent_bits_v=2), kvc.PATH_INT4),
                     (dict(latent_bits=4, latent_bits_v=2), None),  # valid, but no kernel variant: UNSUPPORTED
                     (dict(r_k=40, r_v=40, latent_bits=3), kvc.PATH_HEAD),
                     (dict(r_k=40, r_v=40, latent_bits=3, latent_bits_v=2), kvc.PATH_HEAD),
                     (dict(r_v=48), kvc.PATH_HEAD)]:  # no fast variant for 3 key and 3 value steps: the general one
        L = kvc.make_layout(**base.scaled(**kw).layout_kwargs())
        st = kvc.layout_check(L)
        assert (st == -2) if path is None else (st == 0 and kvc.decode_path(L) == path), kw
    res = kvc.make_layout(**synth.WORKLOADS["residual_128k"].scaled(latent_bits=3).layout_kwargs())
    assert kvc.decode_path(res) == kvc.PATH_HEAD
    var = kvc.make_layout(**synth.WORKLOADS["varrank_paged_32k"].scaled(latent_bits=2).layout_kwargs())
    assert kvc.layout_check(var) == 0 and kvc.decode_path(var) == kvc.PATH_INT4
    var48 = synth.WORKLOADS["varrank_paged_32k"].scaled(r_k=48, r_v=48, rank_choices=(8, 16, 32, 48), latent_bits=2)
    assert kvc.decode_path(kvc.make_layout(**var48.layout_kwargs())) == kvc.PATH_HEAD
    for kw, want in [(dict(latent_bits=5), -1), (dict(latent_bits=4, latent_bits_v=1), -1),
                     (dict(latent_bits=32, latent_bits_v=4), -1), (dict(latent_bits=4, latent_bits_v=32), -1)]:
        assert kvc.layout_check(kvc.make_layout(**base.scaled(**kw).layout_kwargs())) == want, kw
    bad_var = synth.WORKLOADS["varrank_paged_32k"].scaled(latent_bits=3, latent_bits_v=2)
    assert kvc.layout_check(kvc.make_layout(**bad_var.layout_kwargs())) == -1
    shared32 = synth.WORKLOADS["shared_latent_32k"].scaled(latent_bits=3, latent_bits_v=2)  # one latent: one width
    assert kvc.layout_check(kvc.make_layout(**shared32.layout_kwargs())) == -1
    # pool sizes follow r * b / 8 code bytes: K 48 x 3 / 8 = 18, V 64 x 2 / 8 = 16 per slot
    L = kvc.make_layout(**base.scaled(latent_bits=3, latent_bits_v=2).layout_kwargs())
    assert kvc.pool_bytes_max(L, 10) == 10 * 8 * 256 * (18 + 16 + 8 + 8)


def test_tucker_and_per_sequence_w_rejections_without_launching():
    lib = kvc.lib()
    p = C.c_void_p
    good = dict(n_seq=2, n_layers=4, n_kv_heads=8, head_dim=128, r_t=256, r_f=64, latent=512, row0=0)

    def tin(**kw):
        v = dict(good, **kw)
        return kvc.TuckerIn(*(v[n] for n in ("n_seq", "n_layers", "n_kv_heads", "head_dim", "r_t", "r_f", "latent",
                                             "row0")), p(64), p(128))

    for bad in (dict(n_seq=0), dict(r_t=0), dict(r_f=0), dict(r_f=129), dict(row0=300), dict(latent=5000),
                dict(row0=-1)):
        assert lib.kvc_tucker_expand(C.byref(tin(**bad)), p(256), None, None) == -1, bad
    assert lib.kvc_tucker_expand(C.byref(tin()), None, None, None) == -1
    assert lib.kvc_tucker_expand(C.byref(tin(head_dim=64, r_f=32)), p(256), None, None) == -2
    assert lib.kvc_tucker_expand(C.byref(tin()), p(258), None, None) == -4
    # a per-sequence stride is for block-shared layouts only, in whole 16-byte units
    cache = kvc.Cache(p(16), 1 << 30, p(32), p(48), p(64), None, 4)
    for name, stride in (("varrank_paged_32k", 8), ("shared_latent_32k", 12), ("shared_latent_32k", -8)):
        w = synth.WORKLOADS[name]
        L = kvc.make_layout(**w.layout_kwargs())
        inp = kvc.DecodeIn(2, 1, 100, p(80), p(96), None, p(112), 1, p(128), p(144), 0, stride, None, 0, 0)
        assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), p(160), p(176), 1 << 30, None) == -1


def test_evict_and_keep_mask_rejections_without_launching():
    lib = kvc.lib()
    p = C.c_void_p
    for B, T, nl, ratio in ((0, 100, 2, 0.5), (2, 0, 2, 0.5), (2, 100, 0, 0.5), (2, 100, 2, 0.0), (2, 100, 2, 1.5),
                            (2, 100, 2, float("nan"))):
        inp = kvc.EvictIn(B, T, nl, ratio, p(64), p(128))
        assert lib.kvc_evict_select(C.byref(inp), p(256), None) == -1, (B, T, nl, ratio)
    assert lib.kvc_evict_select(C.byref(kvc.EvictIn(2, 100, 2, 0.5, p(64), p(128))), None, None) == -1
    assert lib.kvc_evict_select(C.byref(kvc.EvictIn(2, 100, 2, 0.5, p(64), p(130))), p(256), None) == -4
    # a keep mask is for block-shared layouts, with at least one word per sequence, 4-byte aligned
    cache = kvc.Cache(p(16), 1 << 30, p(32), p(48), p(64), None, 4)
    for name, mask, words, want in (("varrank_paged_32k", p(192), 4, -1), ("shared_latent_32k", p(192), 0, -1),
                                    ("shared_latent_32k", p(194), 4, -4)):
        w = synth.WORKLOADS[name]
        L = kvc.make_layout(**w.layout_kwargs())
        inp = kvc.DecodeIn(2, 1, 100, p(80), p(96), None, p(112), 1, p(128), p(144), 0, 0, mask, words, 0)
        assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), p(160), p(176), 1 << 30, None) == want


def test_kv_split_only_halves_a_block_shared_latent():
    lib = kvc.lib()
    p = C.c_void_p
    cache = kvc.Cache(p(16), 1 << 30, p(32), p(48), p(64), None, 4)
    for name, split in (("varrank_paged_32k", 32), ("shared_latent_32k", 128), ("shared_latent_32k", -256)):
        w = synth.WORKLOADS[name]
        L = kvc.make_layout(**w.layout_kwargs())
        inp = kvc.DecodeIn(2, 1, 100, p(80), p(96), None, p(112), 1, p(128), p(144), 0, 0, None, 0, split)
        assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), p(160), p(176), 1 << 30, None) == -1


def test_decode_check_rejections_without_launching():
    lib = kvc.lib()
    p = C.c_void_p
    L = kvc.make_layout(**synth.WORKLOADS["varrank_paged_32k"].layout_kwargs())
    cache = kvc.Cache(p(16), 1 << 30, p(32), None, None, None, 4)       # variable rank without tok_rank
    inp = kvc.DecodeIn(2, 1, 100, p(80), p(96), None, p(112), 1, p(128), p(144), 0, 0, None, 0, 0)
    assert lib.kvc_decode_check(C.byref(L), C.byref(cache), C.byref(inp), p(256), None) == -1
    cache = kvc.Cache(p(16), 1 << 30, p(32), p(48), p(64), None, 4)
    assert lib.kvc_decode_check(C.byref(L), C.byref(cache), C.byref(inp), None, None) == -1
    inp = kvc.DecodeIn(0, 1, 100, p(80), p(96), None, p(112), 1, p(128), p(144), 0, 0, None, 0, 0)
    assert lib.kvc_decode_check(C.byref(L), C.byref(cache), C.byref(inp), p(256), None) == -1


def test_binding_checks_decode_tensors_before_the_abi():
    # the binding rejects wrong dtypes and shapes before any raw pointer reaches the C ABI (an int64 block table
    # would otherwise be read as int32 page ids); runs on CPU tensors, nothing is launched
    import torch
    w = synth.WORKLOADS["varrank_paged_32k"].scaled(B=2, T=300)
    inp = synth.make_inputs(w)
    L = kvc.make_layout(**w.layout_kwargs())
    args = dict(block_table=inp["block_table"], seq_len=inp["seq_len"], q=inp["q"], wk=inp["wk"], wv=inp["wv"],
                q_pos=inp["q_pos"], out=None)
    kvc._check_decode_args(L, **args)
    for key, bad in (("block_table", inp["block_table"].long()), ("seq_len", inp["seq_len"].long()),
                     ("q_pos", inp["q_pos"][:1]), ("q", inp["q"][None]), ("wk", inp["wk"].half()),
                     ("wv", inp["wv"][:, :, :32]), ("out", torch.empty(inp["q"].shape, dtype=torch.bfloat16))):
        with pytest.raises(ValueError):
            kvc._check_decode_args(L, **dict(args, **{key: bad}))
    ws = synth.WORKLOADS["shared_latent_32k"].scaled(B=2, T=300, n_layers=2)
    si = synth.make_inputs(ws)
    Ls = kvc.make_layout(**ws.layout_kwargs())
    sargs = dict(block_table=si["block_table"], seq_len=si["seq_len"], q=si["q"], wk=si["wk"], wv=si["wv"],
                 q_pos=si["q_pos"], out=None)
    kvc._check_decode_args(Ls, **sargs)
    kvc._check_decode_args(Ls, **dict(sargs, wk=si["wk"].expand(2, -1, -1, -1), wv=si["wv"].expand(2, -1, -1, -1)))
    with pytest.raises(ValueError):                   # one layer's query under a two-layer layout
        kvc._check_decode_args(Ls, **dict(sargs, q=si["q"][0]))
    with pytest.raises(ValueError):
        kvc._ptr(torch.zeros(4))                      # not a device tensor


def test_noalloc_rejects_sizes_beyond_its_array_before_any_device_call():
    # 64 sequences of 131072 tokens with the residual need more split partials than the no-allocation entry point's
    # array holds: the call returns KVC_ERR_SCRATCH from host code, reading no pointer (all null here)
    w = synth.WORKLOADS["residual_128k"]
    L = kvc.make_layout(**w.layout_kwargs())
    assert kvc.decode_workspace_bytes(L, 64, 131072) > kvc.NOALLOC_SCRATCH_BYTES
    assert kvc.decode_workspace_bytes(L, w.B, w.T) <= kvc.NOALLOC_SCRATCH_BYTES
    inp = kvc.DecodeIn(64, 512, 131072, None, None, None, None, kvc.KVC_BF16, None, None, 0, 0, None, 0, 0)
    cache = kvc.Cache(None, 0, None, None, None, None, 1)
    assert kvc.lib().kvc_decode_attn_noalloc(C.byref(L), C.byref(cache), C.byref(inp), None, None) == -6
    assert kvc.lib().kvc_status_string(-6).startswith(b"decode needs more scratch")
    assert kvc.lib().kvc_decode_attn_noalloc(C.byref(L), C.byref(cache), None, None, None) == -1


def test_tucker_fit_rejects_bad_sizes_before_launch():
    def fin(**kw):
        a = dict(B=2, max_T=300, n_layers=2, n_kv_heads=2, head_dim=128, r_t=48, r_f=32, power_iters=1, ut_ld=0)
        a.update(kw)
        return kvc.TuckerFitIn(*a.values(), None, None, None)
    out = C.c_size_t()
    assert kvc.lib().kvc_tucker_fit_workspace_bytes(C.byref(fin()), C.byref(out)) == 0 and out.value > 0
    small = out.value
    assert kvc.lib().kvc_tucker_fit_workspace_bytes(C.byref(fin(power_iters=0)), C.byref(out)) == 0
    assert out.value < small                                       # no separate Q buffer without power iterations
    for bad, want in ((dict(r_t=6), -2), (dict(r_t=260), -2), (dict(r_f=130), -2), (dict(r_f=2), -2),
                      (dict(head_dim=64), -2), (dict(B=0), -1), (dict(power_iters=9), -1), (dict(ut_ld=40), -1),
                      (dict(ut_ld=50), -1), (dict(max_T=0), -1)):
        assert kvc.lib().kvc_tucker_fit_workspace_bytes(C.byref(fin(**bad)), C.byref(out)) == want, bad
    # null inputs with a valid geometry: rejected before any device call
    assert kvc.lib().kvc_tucker_fit(C.byref(fin()), None, None, None, None, None, 0, None) == -1
    assert kvc.lib().kvc_tucker_fit(None, None, None, None, None, None, 0, None) == -1


def test_shared_layout_widths():
    # one latent for keys and values: one width, 4, 3 or 2 bits
    for bits, bits_v, want in ((4, 0, 0), (3, 0, 0), (2, 0, 0), (3, 3, 0), (3, 2, -1), (32, 0, -1)):
        L = kvc.make_layout(**synth.WORKLOADS["shared_latent_32k"].scaled(latent_bits=bits, latent_bits_v=bits_v)
                            .layout_kwargs())
        assert kvc.layout_check(L) == want, (bits, bits_v)
    L = kvc.make_layout(**synth.WORKLOADS["shared_latent_32k_int3"].layout_kwargs())
    w = synth.WORKLOADS["shared_latent_32k_int3"]
    # a page of 256 slots: 512 x 3 / 8 = 192 code bytes, then 512 / 64 = 8 (scale, zero) pairs of 4 bytes per slot
    assert kvc.pool_bytes_max(L, w.n_pages) == w.n_pages * (256 * 192 + 256 * 8 * 4)


def test_compaction_and_positions_rejections_without_launching():
    lib = kvc.lib()
    p = C.c_void_p
    shared = kvc.make_layout(**synth.WORKLOADS["shared_latent_32k"].layout_kwargs())
    perhead = kvc.make_layout(**synth.WORKLOADS["varrank_paged_32k"].layout_kwargs())
    src = kvc.Cache(p(16), 1 << 30, p(32), None, None, None, 4)
    dst = kvc.Cache(p(4096), 1 << 30, p(8192), None, None, None, 4)
    good = dict(B=2, max_blocks=4, block_table=p(80), seq_len=p(96), keep_mask=p(112), keep_words=32,
                out_block_table=p(128))

    def compact(L=shared, s=src, d=dst, out=p(160), pos=p(176), **kw):
        f = dict(good, **kw)
        inp = kvc.CompactIn(f["B"], f["max_blocks"], f["block_table"], f["seq_len"], f["keep_mask"], f["keep_words"],
                            f["out_block_table"])
        return lib.kvc_evict_compact(C.byref(L), C.byref(s), C.byref(d), C.byref(inp), out, pos, None)

    assert compact(L=perhead) == -1                          # per-head caches have no block-level decision
    for bad in (dict(B=0), dict(max_blocks=0), dict(keep_words=0), dict(keep_mask=None), dict(out_block_table=None),
                dict(block_table=None), dict(max_blocks=2049)):   # 2049 pages of 128 slots: past 262144
        assert compact(**bad) == -1, bad
    assert compact(out=None) == -1 and compact(pos=None) == -1
    assert compact(d=kvc.Cache(None, 0, None, None, None, None, 4)) == -1
    assert compact(block_table=p(84)) == -4 and compact(keep_mask=p(114)) == -4 and compact(pos=p(180)) == -4
    odd = kvc.make_layout(**synth.WORKLOADS["shared_latent_32k"].layout_kwargs())
    odd.r_k_cap = odd.r_v_cap = 256                          # a latent the block-shared decode does not serve
    assert compact(L=odd) == -2
    # positions: block-shared only, with q_pos and no keep mask, 4-byte aligned
    cache = kvc.Cache(p(16), 1 << 30, p(32), p(48), p(64), None, 4)
    for L, qpos, mask, words, tp, want in ((perhead, p(100), None, 0, p(192), -1), (shared, None, None, 0, p(192), -1),
                                           (shared, p(100), p(208), 4, p(192), -1),
                                           (shared, p(100), None, 0, p(194), -4)):
        inp = kvc.DecodeIn(2, 1, 100, p(80), p(96), qpos, p(112), 1, p(128), p(144), 0, 0, mask, words, 0, tp)
        assert lib.kvc_decode_attn(C.byref(L), C.byref(cache), C.byref(inp), p(160), p(176), 1 << 30, None) == want


def test_residual_layouts_route_to_a_compiled_variant():
    # the residual kernel takes a layout only when a variant is compiled for its key and value steps (value steps 2
    # or 4); a layout with none goes to the general kernel, or is refused up front when that has none either, never
    # accepted and then failed at launch
    base = synth.WORKLOADS["residual_128k"].scaled(B=2, T=600, page_size=128)
    for kw, path in [(dict(r_k=48, r_v=64), kvc.PATH_RES), (dict(r_k=64, r_v=64), kvc.PATH_RES),
                     (dict(r_k=32, r_v=32), kvc.PATH_RES), (dict(r_k=32, r_v=64), kvc.PATH_RES),
                     (dict(r_k=64, r_v=32), kvc.PATH_RES),
                     (dict(r_k=48, r_v=48), kvc.PATH_HEAD),  # three value steps: the general kernel
                     (dict(r_k=40, r_v=56), kvc.PATH_HEAD),  # ranks off the 16-coordinate steps
                     (dict(r_k=48, r_v=32), None)]:          # valid, but no kernel variant: UNSUPPORTED
        L = kvc.make_layout(**base.scaled(**kw).layout_kwargs())
        assert kvc.layout_check(L) == (-2 if path is None else 0), kw
        if path is not None:
            assert kvc.decode_path(L) == path, kw
