"""Thin Python binding of librbc_kvc.so (include/kvc.h): argument marshalling only.

Every step of compression and decode runs in the library's HIP kernels; this
module turns torch tensors (device memory) into raw pointers and the current
HIP stream into the stream argument.  If the library is not built, importing
any call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librbc_kvc.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kvc.h")

KVC_F32, KVC_BF16 = 0, 1
KVC_FROM_LATENT, KVC_FROM_DENSE = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported geometry", -3: "workspace or pool too small",
          -4: "pointer not 16-byte aligned", -5: "HIP runtime error", -6: "decode needs more scratch than the no-allocation entry point holds"}
EXPORTS = ["kvc_abi_version", "kvc_status_string", "kvc_last_hip_error", "kvc_layout_check", "kvc_pool_bytes_max",
           "kvc_compress", "kvc_decode_workspace_bytes", "kvc_decode_attn", "kvc_dense_workspace_bytes",
           "kvc_dense_decode_attn", "kvc_decode_path", "kvc_decode_attn_timed", "kvc_fit_workspace_bytes",
           "kvc_fit_basis", "kvc_fit_basis_timed", "kvc_salience_workspace_bytes", "kvc_salience",
           "kvc_rank_alloc", "kvc_plan_budget", "kvc_tucker_expand",
           "kvc_evict_select", "kvc_decode_check", "kvc_decode_attn_noalloc", "kvc_probe_stream_read",
           "kvc_probe_mfma_f16", "kvc_probe_clock", "kvc_tucker_fit_workspace_bytes", "kvc_tucker_fit",
           "kvc_evict_compact"]


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        msg = f"{where}: {STATUS.get(status, status)}"
        if hip:
            msg += f" (hipError {hip})"
        super().__init__(msg)
        self.status = status


class Layout(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("shared", C.c_int32), ("n_layers", C.c_int32), ("r_k_cap", C.c_int32), ("r_v_cap", C.c_int32),
                ("group", C.c_int32), ("latent_bits", C.c_int32), ("residual_bits", C.c_int32),
                ("page_size", C.c_int32), ("variable_rank", C.c_int32), ("rope_theta", C.c_double),
                ("latent_bits_v", C.c_int32)]


class Cache(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("pool_bytes", C.c_int64), ("page_off", C.c_void_p),
                ("tok_rank", C.c_void_p), ("tok_off", C.c_void_p), ("used_bytes", C.c_void_p),
                ("n_pages", C.c_int32)]


class CompressIn(C.Structure):
    _fields_ = [("mode", C.c_int32), ("B", C.c_int32), ("max_T", C.c_int32), ("max_blocks", C.c_int32),
                ("block_table", C.c_void_p), ("seq_len", C.c_void_p), ("ranks", C.c_void_p),
                ("lat_k", C.c_void_p), ("lat_v", C.c_void_p), ("res_k", C.c_void_p), ("res_v", C.c_void_p),
                ("k", C.c_void_p), ("v", C.c_void_p), ("basis_k", C.c_void_p), ("basis_v", C.c_void_p)]


class DecodeIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_blocks", C.c_int32), ("max_T", C.c_int32), ("block_table", C.c_void_p),
                ("seq_len", C.c_void_p), ("q_pos", C.c_void_p), ("q", C.c_void_p), ("q_dtype", C.c_int32),
                ("wk", C.c_void_p), ("wv", C.c_void_p), ("num_splits", C.c_int32), ("w_seq_stride", C.c_int64),
                ("keep_mask", C.c_void_p), ("keep_words", C.c_int32), ("kv_split", C.c_int32),
                ("tok_pos", C.c_void_p)]


class DenseIn(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("B", C.c_int32), ("max_blocks", C.c_int32), ("max_T", C.c_int32),
                ("block_table", C.c_void_p), ("seq_len", C.c_void_p), ("k_pages", C.c_void_p),
                ("v_pages", C.c_void_p), ("q", C.c_void_p), ("q_dtype", C.c_int32), ("num_splits", C.c_int32)]


class FitIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_T", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("rank", C.c_int32), ("r_cap", C.c_int32), ("seq_len", C.c_void_p), ("x", C.c_void_p)]


class SalienceIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_T", C.c_int32), ("W", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("rope_theta", C.c_double),
                ("seq_len", C.c_void_p), ("q", C.c_void_p), ("k", C.c_void_p)]


class AllocIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_T", C.c_int32), ("n_ladder", C.c_int32), ("ladder", C.c_int32 * 8),
                ("step_w", C.c_float * 7), ("mean_rank", C.c_double), ("seq_len", C.c_void_p),
                ("sal", C.c_void_p)]


class PlanIn(C.Structure):
    _fields_ = [("n_cells", C.c_int32), ("n_options", C.c_int32), ("distortion", C.c_void_p), ("bytes", C.c_void_p),
                ("budget", C.c_double)]


_lib = None


def lib():
    """The loaded librbc_kvc.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with rank_bit_compressed_amd.build.build()")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.kvc_abi_version.restype = C.c_int32
        L.kvc_status_string.argtypes = [C.c_int32]; L.kvc_status_string.restype = C.c_char_p
        L.kvc_last_hip_error.restype = C.c_int32
        L.kvc_layout_check.argtypes = [P]; L.kvc_layout_check.restype = C.c_int32
        L.kvc_pool_bytes_max.argtypes = [P, C.c_int32, P]; L.kvc_pool_bytes_max.restype = C.c_int32
        L.kvc_compress.argtypes = [P, P, P, P]; L.kvc_compress.restype = C.c_int32
        L.kvc_decode_workspace_bytes.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, P]
        L.kvc_decode_workspace_bytes.restype = C.c_int32
        L.kvc_decode_attn.argtypes = [P, P, P, P, P, C.c_size_t, P]; L.kvc_decode_attn.restype = C.c_int32
        L.kvc_decode_attn_timed.argtypes = [P, P, P, P, P, C.c_size_t, P, P, P]
        L.kvc_decode_attn_timed.restype = C.c_int32
        L.kvc_dense_workspace_bytes.argtypes = [P, P]; L.kvc_dense_workspace_bytes.restype = C.c_int32
        L.kvc_dense_decode_attn.argtypes = [P, P, P, C.c_size_t, P]; L.kvc_dense_decode_attn.restype = C.c_int32
        L.kvc_decode_path.argtypes = [P, P]; L.kvc_decode_path.restype = C.c_int32
        L.kvc_fit_workspace_bytes.argtypes = [P, P]; L.kvc_fit_workspace_bytes.restype = C.c_int32
        L.kvc_fit_basis.argtypes = [P, P, P, P, P, C.c_size_t, P]; L.kvc_fit_basis.restype = C.c_int32
        L.kvc_fit_basis_timed.argtypes = [P, P, P, P, P, C.c_size_t, P, P, P]
        L.kvc_fit_basis_timed.restype = C.c_int32
        L.kvc_salience_workspace_bytes.argtypes = [P, P]; L.kvc_salience_workspace_bytes.restype = C.c_int32
        L.kvc_salience.argtypes = [P, P, P, C.c_size_t, P]; L.kvc_salience.restype = C.c_int32
        L.kvc_rank_alloc.argtypes = [P, P, P]; L.kvc_rank_alloc.restype = C.c_int32
        L.kvc_plan_budget.argtypes = [P, P, P]; L.kvc_plan_budget.restype = C.c_int32
        L.kvc_tucker_expand.argtypes = [P, P, P, P]; L.kvc_tucker_expand.restype = C.c_int32
        L.kvc_evict_select.argtypes = [P, P, P]; L.kvc_evict_select.restype = C.c_int32
        L.kvc_evict_compact.argtypes = [P, P, P, P, P, P, P]; L.kvc_evict_compact.restype = C.c_int32
        L.kvc_decode_check.argtypes = [P, P, P, P, P]; L.kvc_decode_check.restype = C.c_int32
        L.kvc_decode_attn_noalloc.argtypes = [P, P, P, P, P]; L.kvc_decode_attn_noalloc.restype = C.c_int32
        L.kvc_probe_stream_read.argtypes = [P, C.c_size_t, P, C.c_int32, P]; L.kvc_probe_stream_read.restype = C.c_int32
        L.kvc_probe_mfma_f16.argtypes = [C.c_int32, C.c_int32, P, P]; L.kvc_probe_mfma_f16.restype = C.c_int32
        L.kvc_probe_clock.argtypes = [C.c_int32, P, P]; L.kvc_probe_clock.restype = C.c_int32
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("device tensors must be contiguous CUDA/HIP tensors")
    return C.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None):
    """Raise ValueError unless tensor t has this dtype (and shape, where given)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_decode_args(layout, block_table, seq_len, q, wk, wv, q_pos, out):
    """Dtypes and shapes of a decode call's tensors against the layout, before the C ABI sees raw pointers
    (an int64 block table or a q of the wrong rank would otherwise be read as something else)."""
    if block_table.dim() != 2:
        raise ValueError("block_table must be int32 [B, max_blocks]")
    B = block_table.shape[0]
    _need(block_table, "block_table", torch.int32)
    _need(seq_len, "seq_len", torch.int32, (B,))
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, (B,))
    Hq, Hkv, d = layout.n_q_heads, layout.n_kv_heads, layout.head_dim
    if layout.shared:
        qs = (layout.n_layers, B, Hq, d)
        ws = (layout.n_layers, layout.r_k_cap, Hkv * d)
        for name, w in (("wk", wk), ("wv", wv)):
            _need(w, name, torch.bfloat16)
            if tuple(w.shape) != ws and tuple(w.shape) != (B, *ws):
                raise ValueError(f"{name} must have shape {ws} or {(B, *ws)}, got {tuple(w.shape)}")
    else:
        qs = (B, Hq, d)
        _need(wk, "wk", torch.bfloat16, (Hkv, d, layout.r_k_cap))
        _need(wv, "wv", torch.bfloat16, (Hkv, d, layout.r_v_cap))
    if tuple(q.shape) != qs:
        raise ValueError(f"q must have shape {qs}, got {tuple(q.shape)}")
    if out is not None:
        _need(out, "out", torch.float32, qs)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise KvcError(status, where, lib().kvc_last_hip_error() if status == -5 else 0)


def make_layout(**kw) -> Layout:
    f = dict(n_q_heads=0, n_kv_heads=0, head_dim=0, shared=0, n_layers=1, r_k_cap=0, r_v_cap=0, group=32,
             latent_bits=4, residual_bits=0, page_size=256, variable_rank=0, rope_theta=0.0, latent_bits_v=0)
    f.update(kw)
    return Layout(**f)


def layout_check(layout: Layout) -> int:
    return lib().kvc_layout_check(C.byref(layout))


def pool_bytes_max(layout: Layout, n_pages: int) -> int:
    out = C.c_int64()
    _check(lib().kvc_pool_bytes_max(C.byref(layout), n_pages, C.byref(out)), "kvc_pool_bytes_max")
    return out.value


@dataclass
class DeviceCache:
    """Device buffers of one compressed cache (allocated by torch, filled by kvc_compress)."""
    layout: Layout
    pool: torch.Tensor
    page_off: torch.Tensor
    tok_rank: torch.Tensor | None
    tok_off: torch.Tensor | None
    used_bytes: torch.Tensor
    n_pages: int

    @classmethod
    def allocate(cls, layout: Layout, n_pages: int, device="cuda") -> "DeviceCache":
        nbytes = pool_bytes_max(layout, n_pages)
        P = layout.page_size
        var = bool(layout.variable_rank)
        return cls(layout, torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device),
                   torch.empty(n_pages, dtype=torch.int64, device=device),
                   torch.empty(n_pages, P, dtype=torch.uint8, device=device) if var else None,
                   torch.empty(n_pages, P + 1, dtype=torch.int32, device=device) if var else None,
                   torch.zeros(2, dtype=torch.int64, device=device), n_pages)

    def c(self) -> Cache:
        return Cache(_ptr(self.pool), self.pool.numel(), _ptr(self.page_off), _ptr(self.tok_rank),
                     _ptr(self.tok_off), _ptr(self.used_bytes), self.n_pages)


def compress(layout: Layout, cache: DeviceCache, block_table, seq_len, max_T, ranks=None, lat_k=None, lat_v=None,
             res_k=None, res_v=None, k=None, v=None, basis_k=None, basis_v=None):
    """kvc_compress.  FROM_DENSE when k/v are given (lat_*/res_* are then outputs)."""
    mode = KVC_FROM_DENSE if k is not None else KVC_FROM_LATENT
    B, max_blocks = block_table.shape
    bk = basis_k.view(torch.int16) if basis_k is not None else None
    bv = basis_v.view(torch.int16) if basis_v is not None else None
    inp = CompressIn(mode, B, max_T, max_blocks, _ptr(block_table), _ptr(seq_len), _ptr(ranks), _ptr(lat_k),
                     _ptr(lat_v), _ptr(res_k), _ptr(res_v), _ptr(k), _ptr(v), _ptr(bk), _ptr(bv))
    c = cache.c()
    _check(lib().kvc_compress(C.byref(layout), C.byref(inp), C.byref(c), _stream()), "kvc_compress")


PATH_HEAD, PATH_INT4, PATH_SHARED, PATH_RES = 0, 1, 2, 3


def decode_path(layout: Layout) -> int:
    """Which decode kernel serves the layout (PATH_INT4, PATH_RES, PATH_HEAD or PATH_SHARED)."""
    out = C.c_int32()
    _check(lib().kvc_decode_path(C.byref(layout), C.byref(out)), "kvc_decode_path")
    return out.value


def decode_workspace_bytes(layout: Layout, B: int, max_T: int, num_splits: int = 0) -> int:
    out = C.c_size_t()
    _check(lib().kvc_decode_workspace_bytes(C.byref(layout), B, max_T, num_splits, C.byref(out)),
           "kvc_decode_workspace_bytes")
    return out.value


def _q_dtype(q):
    if q.dtype == torch.bfloat16:
        return KVC_BF16
    if q.dtype == torch.float32:
        return KVC_F32
    raise TypeError("q must be fp32 or bf16")


def decode_in(block_table, seq_len, q, wk, wv, max_T, q_pos=None, num_splits=0, w_seq_stride=0,
              keep_mask=None, kv_split=0, tok_pos=None, page_size=0) -> DecodeIn:
    B, max_blocks = block_table.shape
    words = 0
    if keep_mask is not None:
        if keep_mask.dtype != torch.int32 or keep_mask.dim() != 2 or keep_mask.shape[0] != B:
            raise ValueError("keep_mask must be an int32 (uint32 bits) tensor [B, words]")
        words = keep_mask.shape[1]
    if tok_pos is not None:
        _need(tok_pos, "tok_pos", torch.int32, (B, max_blocks * page_size))
    return DecodeIn(B, max_blocks, max_T, _ptr(block_table), _ptr(seq_len), _ptr(q_pos), _ptr(q), _q_dtype(q),
                    _ptr(wk.view(torch.int16)), _ptr(wv.view(torch.int16)), num_splits, w_seq_stride,
                    _ptr(keep_mask), words, kv_split, _ptr(tok_pos))


def _w_stride(layout, wk, wv, B):
    """Elements between sequences' up-projections: 0 unless shared mode with per-sequence [B, L, latent, Hkv d]."""
    if not (layout.shared and wk.dim() == 4):
        return 0
    if wv.shape != wk.shape or wk.shape[0] != B or not (wk.is_contiguous() and wv.is_contiguous()):
        raise ValueError("per-sequence W_k / W_v must both be contiguous [B, L, latent, Hkv * d]")
    return wk[0].numel()


def decode_attn(layout: Layout, cache: DeviceCache, block_table, seq_len, q, wk, wv, max_T, q_pos=None,
                num_splits=0, out=None, ws=None, events=None, keep_mask=None, kv_split=0, tok_pos=None):
    """kvc_decode_attn -> fp32 [(L,) B, Hq, d].  events: optional (begin, end) pair of recorded-once
    torch.cuda.Event objects; the call then goes through kvc_decode_attn_timed, which records them around
    the attention kernel alone.  Shared mode: wk, wv [L, latent, Hkv * d] for all sequences, or
    [B, L, latent, Hkv * d] (contiguous), one pair per sequence; keep_mask: optional int32 [B, words] token
    keep mask (as kvc_evict_select writes it); kv_split: latent / 2 for a latent whose lower half holds only
    key coordinates and upper half only value coordinates (keys and values with their own token factors);
    tok_pos: optional int32 [B, max_blocks * page_size] source positions of a compacted cache's slots (as
    evict_compact writes them; q_pos required)."""
    _check_decode_args(layout, block_table, seq_len, q, wk, wv, q_pos, out)
    B = block_table.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(layout, B, max_T, num_splits)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    inp = decode_in(block_table, seq_len, q, wk, wv, max_T, q_pos, num_splits, _w_stride(layout, wk, wv, B),
                    keep_mask, kv_split, tok_pos, layout.page_size)
    c = cache.c()
    if events is None:
        _check(lib().kvc_decode_attn(C.byref(layout), C.byref(c), C.byref(inp), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream()), "kvc_decode_attn")
    else:
        eb, ee = (_event_handle(e) for e in events)
        _check(lib().kvc_decode_attn_timed(C.byref(layout), C.byref(c), C.byref(inp), _ptr(out), _ptr(ws),
                                           ws.numel(), _stream(), eb, ee), "kvc_decode_attn_timed")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # KVC_NOALLOC_SCRATCH_BYTES


def decode_attn_noalloc(layout: Layout, cache: DeviceCache, block_table, seq_len, q, wk, wv, max_T, q_pos=None,
                        num_splits=0, out=None, keep_mask=None, kv_split=0, tok_pos=None):
    """kvc_decode_attn_noalloc -> fp32 [(L,) B, Hq, d]: the decode step with its split partials in the library's
    device array (no workspace argument; the library allocates nothing).  Calls overlapping on one GPU race."""
    _check_decode_args(layout, block_table, seq_len, q, wk, wv, q_pos, out)
    B = block_table.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    inp = decode_in(block_table, seq_len, q, wk, wv, max_T, q_pos, num_splits, _w_stride(layout, wk, wv, B),
                    keep_mask, kv_split, tok_pos, layout.page_size)
    c = cache.c()
    _check(lib().kvc_decode_attn_noalloc(C.byref(layout), C.byref(c), C.byref(inp), _ptr(out), _stream()),
           "kvc_decode_attn_noalloc")
    return out


class DecodePlan:
    """kvc_decode_attn with its arguments marshalled once, for calling in a loop (a decode step per call).

    The tensors given here must stay alive and in place while the plan is used; each call reads whatever
    they hold at launch time.  Calls enqueue on the current stream, like decode_attn."""

    def __init__(self, layout: Layout, cache: DeviceCache, block_table, seq_len, q, wk, wv, max_T, q_pos=None,
                 num_splits=0, out=None, ws=None, keep_mask=None, kv_split=0, tok_pos=None):
        _check_decode_args(layout, block_table, seq_len, q, wk, wv, q_pos, out)
        B = block_table.shape[0]
        self.out = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=q.device)
        need = decode_workspace_bytes(layout, B, max_T, num_splits)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        self._keep = (layout, cache, block_table, seq_len, q, wk, wv, q_pos, ws, keep_mask, tok_pos)
        self._layout, self._cache = layout, cache.c()
        self._in = decode_in(block_table, seq_len, q, wk, wv, max_T, q_pos, num_splits, _w_stride(layout, wk, wv, B),
                             keep_mask, kv_split, tok_pos, layout.page_size)
        self._args = (C.byref(self._layout), C.byref(self._cache), C.byref(self._in), _ptr(self.out), _ptr(ws),
                      ws.numel())
        self._fn, self._fn_timed = lib().kvc_decode_attn, lib().kvc_decode_attn_timed

    def __call__(self, events=None):
        if events is None:
            st = self._fn(*self._args, _stream())
        else:
            st = self._fn_timed(*self._args, _stream(), *(_event_handle(e) for e in events))
        if st != 0:
            _check(st, "kvc_decode_attn")
        return self.out


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (torch creates the event at its first record)."""
    h = ev.cuda_event
    if not h:
        raise ValueError("record the torch.cuda.Event once before passing it (its HIP event is created lazily)")
    return C.c_void_p(h)


def dense_in(Hq, Hkv, d, P, block_table, seq_len, k_pages, v_pages, q, max_T, num_splits=0) -> DenseIn:
    B, max_blocks = block_table.shape
    return DenseIn(Hq, Hkv, d, P, B, max_blocks, max_T, _ptr(block_table), _ptr(seq_len),
                   _ptr(k_pages.view(torch.int16)), _ptr(v_pages.view(torch.int16)), _ptr(q), _q_dtype(q),
                   num_splits)


def dense_workspace_bytes(inp: DenseIn) -> int:
    out = C.c_size_t()
    _check(lib().kvc_dense_workspace_bytes(C.byref(inp), C.byref(out)), "kvc_dense_workspace_bytes")
    return out.value


def dense_decode_attn(Hq, Hkv, d, P, block_table, seq_len, k_pages, v_pages, q, max_T, num_splits=0, out=None,
                      ws=None):
    """kvc_dense_decode_attn -> fp32 [B, Hq, d]."""
    inp = dense_in(Hq, Hkv, d, P, block_table, seq_len, k_pages, v_pages, q, max_T, num_splits)
    need = dense_workspace_bytes(inp)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().kvc_dense_decode_attn(C.byref(inp), _ptr(out), _ptr(ws), ws.numel(), _stream()),
           "kvc_dense_decode_attn")
    return out


def fit_in(x, seq_len, rank, r_cap=None) -> FitIn:
    B, max_T, Hkv, d = x.shape
    return FitIn(B, max_T, Hkv, d, rank, rank if r_cap is None else r_cap, _ptr(seq_len), _ptr(x))


def fit_workspace_bytes(inp: FitIn) -> int:
    out = C.c_size_t()
    _check(lib().kvc_fit_workspace_bytes(C.byref(inp), C.byref(out)), "kvc_fit_workspace_bytes")
    return out.value


def fit_basis(x, seq_len, rank, r_cap=None, want_f32=True, want_sigma2=True, ws=None, events=None):
    """kvc_fit_basis: x fp32 [B, max_T, Hkv, d] pre-RoPE rows, seq_len int32 [B] ->
    (basis bf16 [Hkv, d, r_cap], basis fp32 [Hkv, d, rank] or None, sigma2 fp32 [Hkv, d] or None).
    events: optional (begin, end) torch.cuda.Event pair recorded around the Gram-matrix kernel
    (kvc_fit_basis_timed)."""
    inp = fit_in(x, seq_len, rank, r_cap)
    B, max_T, Hkv, d = x.shape
    need = fit_workspace_bytes(inp)
    dev = x.device
    bb = torch.empty((Hkv, d, inp.r_cap), dtype=torch.bfloat16, device=dev)
    bf = torch.empty((Hkv, d, rank), dtype=torch.float32, device=dev) if want_f32 else None
    s2 = torch.empty((Hkv, d), dtype=torch.float32, device=dev) if want_sigma2 else None
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    args = (C.byref(inp), _ptr(bb.view(torch.int16)), _ptr(bf), _ptr(s2), _ptr(ws), ws.numel(), _stream())
    if events is None:
        _check(lib().kvc_fit_basis(*args), "kvc_fit_basis")
    else:
        _check(lib().kvc_fit_basis_timed(*args, _event_handle(events[0]), _event_handle(events[1])),
               "kvc_fit_basis_timed")
    return bb, bf, s2


def salience_in(q, k, seq_len, theta) -> SalienceIn:
    B, W, Hq, d = q.shape
    _, max_T, Hkv, _ = k.shape
    return SalienceIn(B, max_T, W, Hq, Hkv, d, float(theta), _ptr(seq_len), _ptr(q), _ptr(k))


def salience_workspace_bytes(inp: SalienceIn) -> int:
    out = C.c_size_t()
    _check(lib().kvc_salience_workspace_bytes(C.byref(inp), C.byref(out)), "kvc_salience_workspace_bytes")
    return out.value


def salience(q, k, seq_len, theta, out=None, ws=None):
    """kvc_salience: q fp32 [B, W, Hq, d] window queries, k fp32 [B, max_T, Hkv, d] keys (both pre-RoPE),
    seq_len int32 [B] -> fp32 [B, max_T]."""
    inp = salience_in(q, k, seq_len, theta)
    need = salience_workspace_bytes(inp)
    if out is None:
        out = torch.empty((k.shape[0], k.shape[1]), dtype=torch.float32, device=k.device)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=k.device)
    _check(lib().kvc_salience(C.byref(inp), _ptr(out), _ptr(ws), ws.numel(), _stream()), "kvc_salience")
    return out


def alloc_in(sal, seq_len, ladder, step_w, mean_rank) -> AllocIn:
    B, max_T = sal.shape
    lad = (C.c_int32 * 8)(*(list(ladder) + [0] * (8 - len(ladder))))
    w = (C.c_float * 7)(*(list(step_w) + [0.0] * (7 - len(step_w))))
    return AllocIn(B, max_T, len(ladder), lad, w, float(mean_rank), _ptr(seq_len), _ptr(sal))


def rank_alloc(sal, seq_len, ladder, step_w, mean_rank, out=None):
    """kvc_rank_alloc: sal fp32 [B, max_T] -> uint8 ranks [B, max_T]."""
    inp = alloc_in(sal, seq_len, ladder, step_w, mean_rank)
    if out is None:
        out = torch.empty(sal.shape, dtype=torch.uint8, device=sal.device)
    _check(lib().kvc_rank_alloc(C.byref(inp), _ptr(out), _stream()), "kvc_rank_alloc")
    return out


def plan_budget(distortion, bytes_, budget):
    """kvc_plan_budget (host): distortion, bytes_ array-likes [n_cells, n_options] -> (choice int32 [n_cells], lam)."""
    import numpy as np
    D = np.ascontiguousarray(distortion, dtype=np.float64)
    Bb = np.ascontiguousarray(bytes_, dtype=np.float64)
    choice = np.zeros(D.shape[0], dtype=np.int32)
    lam = C.c_double()
    inp = PlanIn(D.shape[0], D.shape[1], D.ctypes.data_as(C.c_void_p), Bb.ctypes.data_as(C.c_void_p), float(budget))
    _check(lib().kvc_plan_budget(C.byref(inp), choice.ctypes.data_as(C.c_void_p), C.byref(lam)), "kvc_plan_budget")
    return choice, lam.value


class TuckerIn(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_seq", "n_layers", "n_kv_heads", "head_dim", "r_t", "r_f", "latent",
                                         "row0")] + [("u_f", C.c_void_p), ("core", C.c_void_p)]


def tucker_expand(u_f, core, latent, row0=0, w=None, want_f32=False):
    """kvc_tucker_expand: u_f fp32 [S, d, r_f], core fp32 [S, L, Hkv, r_t, r_f] (device) -> (w bf16
    [S, L, latent, Hkv * d], w32 fp32 of the same shape or None).  Rows outside row0..row0+r_t-1 of a given w
    are left as they are; a new w starts at zero."""
    S, d, r_f = u_f.shape
    _, L, Hkv, r_t, _ = core.shape
    if w is None:
        w = torch.zeros(S, L, latent, Hkv * d, dtype=torch.bfloat16, device=u_f.device)
    w32 = torch.zeros(w.shape, dtype=torch.float32, device=u_f.device) if want_f32 else None
    for t in (u_f, core, w):
        if not t.is_contiguous():
            raise ValueError("tucker_expand takes contiguous tensors")
    inp = TuckerIn(S, L, Hkv, d, r_t, r_f, latent, row0, _ptr(u_f), _ptr(core))
    _check(lib().kvc_tucker_expand(C.byref(inp), _ptr(w.view(torch.int16)), _ptr(w32), _stream()),
           "kvc_tucker_expand")
    return w, w32


class TuckerFitIn(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "max_T", "n_layers", "n_kv_heads", "head_dim", "r_t", "r_f",
                                         "power_iters", "ut_ld")] + \
               [("seq_len", C.c_void_p), ("x", C.c_void_p), ("omega", C.c_void_p)]


def tucker_fit_in(x, seq_len, omega, r_t, r_f, power_iters, ut_ld=0) -> TuckerFitIn:
    B, max_T, L, Hkv, d = x.shape
    return TuckerFitIn(B, max_T, L, Hkv, d, r_t, r_f, power_iters, ut_ld, _ptr(seq_len), _ptr(x), _ptr(omega))


def tucker_fit_workspace_bytes(inp: TuckerFitIn) -> int:
    out = C.c_size_t()
    _check(lib().kvc_tucker_fit_workspace_bytes(C.byref(inp), C.byref(out)), "kvc_tucker_fit_workspace_bytes")
    return out.value


def tucker_fit(x, seq_len, omega, r_t, r_f, power_iters, u_t=None, ws=None):
    """kvc_tucker_fit: x fp32 [B, max_T, L, Hkv, d], seq_len int32 [B], omega fp32 [L * Hkv * d, r_t] (device) ->
    (u_t fp32 [B, max_T, r_t] or the given u_t view, u_f fp32 [B, d, r_f], core fp32 [B, L, Hkv, r_t, r_f],
    info int32 [B]).  A given u_t is a [B, max_T, r_t] view with unit column stride (for instance columns of a
    wider latent buffer); its row stride is passed as ut_ld."""
    B, max_T, L, Hkv, d = x.shape
    for t in (x, omega):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("tucker_fit takes contiguous fp32 x and omega")
    if tuple(omega.shape) != (L * Hkv * d, r_t):
        raise ValueError(f"omega must be [{L * Hkv * d}, {r_t}]")
    if seq_len.dtype != torch.int32 or tuple(seq_len.shape) != (B,):
        raise ValueError("seq_len must be int32 [B]")
    dev = x.device
    if u_t is None:
        u_t = torch.empty(B, max_T, r_t, dtype=torch.float32, device=dev)
    if (u_t.dtype != torch.float32 or tuple(u_t.shape) != (B, max_T, r_t) or u_t.stride(2) != 1
            or u_t.stride(0) != max_T * u_t.stride(1)):
        raise ValueError("u_t must be an fp32 [B, max_T, r_t] view with unit column stride and rows of one stride")
    u_f = torch.empty(B, d, r_f, dtype=torch.float32, device=dev)
    core = torch.empty(B, L, Hkv, r_t, r_f, dtype=torch.float32, device=dev)
    info = torch.empty(B, dtype=torch.int32, device=dev)
    inp = tucker_fit_in(x, seq_len, omega, r_t, r_f, power_iters, u_t.stride(1))
    need = tucker_fit_workspace_bytes(inp)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not u_t.is_cuda:
        raise ValueError("u_t must be a CUDA/HIP tensor")
    _check(lib().kvc_tucker_fit(C.byref(inp), C.c_void_p(u_t.data_ptr()), _ptr(u_f), _ptr(core), _ptr(info), _ptr(ws), ws.numel(),
                                _stream()), "kvc_tucker_fit")
    return u_t, u_f, core, info


class EvictIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_T", C.c_int32), ("n_layers", C.c_int32), ("keep_ratio", C.c_double),
                ("seq_len", C.c_void_p), ("scores", C.c_void_p)]


def evict_select(scores, seq_len, keep_ratio, out=None):
    """kvc_evict_select: scores fp32 [n_layers, B, max_T], seq_len int32 [B] (device) -> keep mask int32
    (uint32 bits) [B, ceil(max_T / 32)]."""
    n_layers, B, max_T = scores.shape
    if out is None:
        out = torch.empty(B, (max_T + 31) // 32, dtype=torch.int32, device=scores.device)
    inp = EvictIn(B, max_T, n_layers, float(keep_ratio), _ptr(seq_len), _ptr(scores))
    _check(lib().kvc_evict_select(C.byref(inp), _ptr(out), _stream()), "kvc_evict_select")
    return out


class CompactIn(C.Structure):
    _fields_ = [("B", C.c_int32), ("max_blocks", C.c_int32), ("block_table", C.c_void_p), ("seq_len", C.c_void_p),
                ("keep_mask", C.c_void_p), ("keep_words", C.c_int32), ("out_block_table", C.c_void_p)]


def evict_compact(layout: Layout, src: DeviceCache, dst: DeviceCache, block_table, seq_len, keep_mask,
                  out_block_table, out_seq_len=None, tok_pos=None):
    """kvc_evict_compact: the kept tokens of a block-shared cache moved into dst's pages out_block_table
    (dst.page_off set by the caller).  Returns (out_seq_len int32 [B], tok_pos int32 [B, max_blocks * P])."""
    B, max_blocks = block_table.shape
    _need(block_table, "block_table", torch.int32)
    _need(out_block_table, "out_block_table", torch.int32, (B, max_blocks))
    _need(seq_len, "seq_len", torch.int32, (B,))
    if keep_mask.dtype != torch.int32 or keep_mask.dim() != 2 or keep_mask.shape[0] != B:
        raise ValueError("keep_mask must be an int32 (uint32 bits) tensor [B, words]")
    if out_seq_len is None:
        out_seq_len = torch.empty(B, dtype=torch.int32, device=block_table.device)
    if tok_pos is None:
        tok_pos = torch.empty(B, max_blocks * layout.page_size, dtype=torch.int32, device=block_table.device)
    _need(tok_pos, "tok_pos", torch.int32, (B, max_blocks * layout.page_size))
    inp = CompactIn(B, max_blocks, _ptr(block_table), _ptr(seq_len), _ptr(keep_mask), keep_mask.shape[1],
                    _ptr(out_block_table))
    _check(lib().kvc_evict_compact(C.byref(layout), C.byref(src.c()), C.byref(dst.c()), C.byref(inp),
                                   _ptr(out_seq_len), _ptr(tok_pos), _stream()), "kvc_evict_compact")
    return out_seq_len, tok_pos


BAD_SEQ_LEN, BAD_PAGE, BAD_OFFSET, BAD_Q_POS, BAD_RANK, BAD_TOK_OFF, BAD_RECORD, BAD_TOK_POS = (1, 2, 4, 8, 16, 32,
                                                                                    64, 128)


def decode_check(layout: Layout, cache: DeviceCache, block_table, seq_len, max_T, q_pos=None, tok_pos=None) -> int:
    """kvc_decode_check: the or of the KVC_BAD_* flags of these tables (0 = fine).  Synchronizes."""
    flags = torch.empty(4, dtype=torch.int32, device=block_table.device)
    q = torch.empty(16, dtype=torch.float32, device=block_table.device)
    inp = decode_in(block_table, seq_len, q, q, q, max_T, q_pos, tok_pos=tok_pos, page_size=layout.page_size)
    _check(lib().kvc_decode_check(C.byref(layout), C.byref(cache.c()), C.byref(inp), _ptr(flags), _stream()),
           "kvc_decode_check")
    return int(flags[0].item())


def probe_stream_read(buf, grid: int, sink):
    """kvc_probe_stream_read over the whole uint8 device tensor buf (enqueued on the current stream)."""
    _check(lib().kvc_probe_stream_read(_ptr(buf), buf.numel(), _ptr(sink), grid, _stream()), "kvc_probe_stream_read")


def probe_mfma_f16(iters: int, grid: int, sink):
    """kvc_probe_mfma_f16: grid x 4 waves x iters x 8 matrix instructions of 32768 flops each."""
    _check(lib().kvc_probe_mfma_f16(iters, grid, _ptr(sink), _stream()), "kvc_probe_mfma_f16")


def probe_clock(out, spins: int = 200000):
    """kvc_probe_clock into out (int64 [3] device tensor); shader MHz = out[0] / out[1] * 100 after a sync."""
    _check(lib().kvc_probe_clock(spins, _ptr(out), _stream()), "kvc_probe_clock")
