"""Python view of the CPU oracle (libkvc_ref.so, built from kvc_ref.c by gcc).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg import this module; the product library never does.  Arrays
are numpy, host memory; bf16/fp16 values travel as their uint16 bit patterns.
"""
import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = C.CDLL(path)
        P = C.c_void_p
        i32, i64, f64 = C.c_int32, C.c_int64, C.c_double
        L.kvc_ref_layout_check.argtypes = [P]; L.kvc_ref_layout_check.restype = C.c_int
        L.kvc_ref_page_bytes_uniform.argtypes = [P]; L.kvc_ref_page_bytes_uniform.restype = i64
        L.kvc_ref_f32_to_f16.argtypes = [C.c_float]; L.kvc_ref_f32_to_f16.restype = C.c_uint16
        L.kvc_ref_f16_to_f64.argtypes = [C.c_uint16]; L.kvc_ref_f16_to_f64.restype = f64
        L.kvc_ref_bf16_to_f64.argtypes = [C.c_uint16]; L.kvc_ref_bf16_to_f64.restype = f64
        L.kvc_ref_f32_to_f16_n.argtypes = [P, i64, P]; L.kvc_ref_f32_to_f16_n.restype = None
        L.kvc_ref_quant_int4_n.argtypes = [P, i64, C.c_int, P, P, P]; L.kvc_ref_quant_int4_n.restype = None
        L.kvc_ref_quant_intb_n.argtypes = [P, i64, C.c_int, C.c_int, P, P, P]; L.kvc_ref_quant_intb_n.restype = None
        L.kvc_ref_quant_res2_n.argtypes = [P, i64, C.c_int, P, P]; L.kvc_ref_quant_res2_n.restype = None
        L.kvc_ref_hadamard.argtypes = [C.c_int, P]; L.kvc_ref_hadamard.restype = None
        L.kvc_ref_rope.argtypes = [P, C.c_int, f64, f64]; L.kvc_ref_rope.restype = None
        L.kvc_ref_compress.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P, P, P, P, P, P, C.c_int, P, i64, P, P, P]
        L.kvc_ref_compress.restype = i64
        L.kvc_ref_project.argtypes = [P, C.c_int, C.c_int, P, P, P, P, P, P, P, P, P, P]
        L.kvc_ref_project.restype = C.c_int
        L.kvc_ref_decode_attn.argtypes = [P, C.c_int, C.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.kvc_ref_decode_attn.restype = C.c_int
        L.kvc_ref_decode_attn_masked.argtypes = [P, C.c_int, C.c_int, P, P, P, P, P, P, P, P, P, P, P, C.c_int, P, P, P]
        L.kvc_ref_decode_attn_masked.restype = C.c_int
        L.kvc_ref_dense_attn.argtypes = [C.c_int] * 6 + [P] * 7
        L.kvc_ref_dense_attn.restype = C.c_int
        L.kvc_ref_threads.argtypes = []; L.kvc_ref_threads.restype = C.c_int
        _lib = L
    return _lib


class _Layout(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("n_q_heads", "n_kv_heads", "head_dim", "shared", "n_layers", "r_k_cap",
                                       "r_v_cap", "group", "latent_bits", "residual_bits", "page_size",
                                       "variable_rank")] + [("rope_theta", C.c_double), ("latent_bits_v", C.c_int)]


@dataclass
class Layout:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    r_k_cap: int
    r_v_cap: int
    group: int = 32
    latent_bits: int = 4
    residual_bits: int = 0
    page_size: int = 256
    variable_rank: int = 0
    shared: int = 0
    n_layers: int = 1
    rope_theta: float = 0.0
    latent_bits_v: int = 0

    def c(self):
        return _Layout(self.n_q_heads, self.n_kv_heads, self.head_dim, self.shared, self.n_layers, self.r_k_cap,
                       self.r_v_cap, self.group, self.latent_bits, self.residual_bits, self.page_size,
                       self.variable_rank, self.rope_theta, self.latent_bits_v)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def layout_check(L: Layout) -> int:
    return lib().kvc_ref_layout_check(C.byref(L.c()))


def page_bytes_uniform(L: Layout) -> int:
    return lib().kvc_ref_page_bytes_uniform(C.byref(L.c()))


def f32_to_f16(x) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    out = np.empty(x.shape, np.uint16)
    lib().kvc_ref_f32_to_f16_n(_p(x), x.size, _p(out))
    return out


def f16_to_f64(h: int) -> float:
    return lib().kvc_ref_f16_to_f64(int(h))


def bf16_to_f64(b: int) -> float:
    return lib().kvc_ref_bf16_to_f64(int(b))


def quant_int4(x):
    """x [n_groups, n] fp32 -> (s16 [n_groups] u16, z16 [n_groups] u16, codes [n_groups, n] u8)."""
    x = _c(x, np.float32)
    ng, n = x.shape
    s = np.empty(ng, np.uint16); z = np.empty(ng, np.uint16); q = np.empty((ng, n), np.uint8)
    lib().kvc_ref_quant_int4_n(_p(x), ng, n, _p(s), _p(z), _p(q))
    return s, z, q


def quant_intb(x, bits):
    """x [n_groups, n] fp32 -> (s16, z16, codes) of the bits-bit quantizer (bits 2..4)."""
    x = _c(x, np.float32)
    ng, n = x.shape
    s = np.empty(ng, np.uint16); z = np.empty(ng, np.uint16); q = np.empty((ng, n), np.uint8)
    lib().kvc_ref_quant_intb_n(_p(x), ng, n, int(bits), _p(s), _p(z), _p(q))
    return s, z, q


def quant_res2(y):
    """y [n_rows, n] fp32 -> (s16 [n_rows] u16, codes [n_rows, n] u8)."""
    y = _c(y, np.float32)
    nr, n = y.shape
    s = np.empty(nr, np.uint16); q = np.empty((nr, n), np.uint8)
    lib().kvc_ref_quant_res2_n(_p(y), nr, n, _p(s), _p(q))
    return s, q


def hadamard(n: int) -> np.ndarray:
    H = np.empty((n, n), np.float64)
    lib().kvc_ref_hadamard(n, _p(H))
    return H


def rope(x, pos: float, theta: float) -> np.ndarray:
    x = np.array(x, dtype=np.float64, copy=True)
    lib().kvc_ref_rope(_p(x), x.shape[-1], float(pos), float(theta))
    return x


def compress(L: Layout, block_table, seq_len, max_T, ranks, lat_k, lat_v, res_k, res_v, n_pages, pool_bytes):
    """Returns (pool u8 [used], page_off i64 [n_pages], tok_rank u8 [n_pages,P] | None, tok_off u32 | None)."""
    bt = _c(block_table, np.int32); sl = _c(seq_len, np.int32)
    B, max_blocks = bt.shape
    P = L.page_size
    pool = np.zeros(pool_bytes, np.uint8)
    page_off = np.zeros(n_pages, np.int64)
    tok_rank = np.zeros((n_pages, P), np.uint8) if L.variable_rank else None
    tok_off = np.zeros((n_pages, P + 1), np.uint32) if L.variable_rank else None
    args = [_c(ranks, np.uint8), _c(lat_k, np.float32), _c(lat_v, np.float32), _c(res_k, np.float32),
            _c(res_v, np.float32)]
    used = lib().kvc_ref_compress(C.byref(L.c()), B, int(max_T), max_blocks, _p(bt), _p(sl), *[_p(a) for a in args],
                                  int(n_pages), _p(pool), int(pool_bytes), _p(page_off), _p(tok_rank), _p(tok_off))
    if used < 0:
        raise ValueError(f"kvc_ref_compress rejected its input ({used})")
    return pool[:used], page_off, tok_rank, tok_off


def project(L: Layout, seq_len, max_T, ranks, k, v, basis_k, basis_v):
    """Dense pre-RoPE K/V [B, max_T, Hkv, d] -> fp32 latents and rotated residuals."""
    k = _c(k, np.float32); v = _c(v, np.float32)
    B = k.shape[0]
    Hkv, d = L.n_kv_heads, L.head_dim
    lat_k = np.zeros((B, max_T, Hkv, L.r_k_cap), np.float32)
    lat_v = np.zeros((B, max_T, Hkv, L.r_v_cap), np.float32)
    res_k = np.zeros((B, max_T, Hkv, d), np.float32) if L.residual_bits else None
    res_v = np.zeros((B, max_T, Hkv, d), np.float32) if L.residual_bits else None
    rc = lib().kvc_ref_project(C.byref(L.c()), B, int(max_T), _p(_c(seq_len, np.int32)), _p(_c(ranks, np.uint8)),
                               _p(k), _p(v), _p(_c(basis_k, np.uint16)), _p(_c(basis_v, np.uint16)),
                               _p(lat_k), _p(lat_v), _p(res_k), _p(res_v))
    if rc:
        raise ValueError("kvc_ref_project rejected its input")
    return lat_k, lat_v, res_k, res_v


def decode_attn(L: Layout, block_table, seq_len, q_pos, pool, page_off, tok_rank, tok_off, q, wk, wv,
                sel_b=None, sel_h=None, keep=None):
    """fp64 attention output [(L,) B, Hq, d]; rows of unselected (b, kv head) are NaN.  keep: optional uint32
    token keep mask [B, words] (bit t % 32 of word t // 32)."""
    bt = _c(block_table, np.int32)
    B, max_blocks = bt.shape
    q = _c(q, np.float32)
    out = np.full(q.shape, np.nan, np.float64)
    keep_words = 0 if keep is None else int(np.asarray(keep).shape[1])
    rc = lib().kvc_ref_decode_attn_masked(C.byref(L.c()), B, max_blocks, _p(bt), _p(_c(seq_len, np.int32)),
                                          _p(_c(q_pos, np.int32)), _p(_c(pool, np.uint8)),
                                          _p(_c(page_off, np.int64)), _p(_c(tok_rank, np.uint8)),
                                          _p(_c(tok_off, np.uint32)), _p(q), _p(_c(wk, np.uint16)),
                                          _p(_c(wv, np.uint16)), _p(_c(keep, np.uint32)), keep_words,
                                          _p(_c(sel_b, np.uint8)), _p(_c(sel_h, np.uint8)), _p(out))
    if rc:
        raise ValueError("kvc_ref_decode_attn rejected its input")
    return out


def dense_attn(Hq, Hkv, d, P, block_table, seq_len, k_pages, v_pages, q, sel_b=None):
    bt = _c(block_table, np.int32)
    B, max_blocks = bt.shape
    q = _c(q, np.float32)
    out = np.full(q.shape, np.nan, np.float64)
    rc = lib().kvc_ref_dense_attn(Hq, Hkv, d, P, B, max_blocks, _p(bt), _p(_c(seq_len, np.int32)),
                                  _p(_c(k_pages, np.uint16)), _p(_c(v_pages, np.uint16)), _p(q),
                                  _p(_c(sel_b, np.uint8)), _p(out))
    if rc:
        raise ValueError("kvc_ref_dense_attn rejected its input")
    return out


def threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(lib().kvc_ref_threads())
