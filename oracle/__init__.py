"""CPU oracle for the quantized-KV decode path (ctypes wrapper of liboracle.so).

TEST INFRASTRUCTURE ONLY.  This package may be imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py`` -- by
nothing else.  It never imports the HIP library's package, and the HIP
library never imports it.  The arithmetic lives in ``kvq_oracle.c``; this file
only marshals numpy arrays, except for two compositions written in numpy
(fp64): the sparse decode (a row selection in front of ``decode_attn``) and
the fused decode attention over the q4_0 pools (``decode_attn_q4_0``).

Functions mirror the C entry points (see the comments there for the
definitions and the pages each follows).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        L = ctypes.CDLL(path)
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_f16_encode.argtypes = [ctypes.c_double]
        L.oracle_f16_encode.restype = ctypes.c_uint16
        L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_f16_decode.restype = ctypes.c_double
        L.oracle_bf16_encode.argtypes = [ctypes.c_double]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_double
        for name, a, o in [("oracle_e4m3_encode_array", _c_f32p, _c_u8p),
                           ("oracle_e4m3_decode_array", _c_u8p, _c_f64p),
                           ("oracle_f16_encode_array", _c_f32p, _c_u16p),
                           ("oracle_f16_encode_array_f64", _c_f64p, _c_u16p),
                           ("oracle_f16_decode_array", _c_u16p, _c_f64p),
                           ("oracle_bf16_encode_array", _c_f32p, _c_u16p),
                           ("oracle_bf16_encode_array_f64", _c_f64p, _c_u16p)]:
            f = getattr(L, name)
            f.argtypes = [a, ctypes.c_int64, o]
            f.restype = None
        L.oracle_fwht_f32.argtypes = [_c_f32p, ctypes.c_int]
        L.oracle_fwht_f32.restype = ctypes.c_int
        L.oracle_fwht_rows_f32.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int]
        L.oracle_fwht_rows_f32.restype = ctypes.c_int
        L.oracle_fwht256_orthonormal.argtypes = [_c_f32p]
        L.oracle_fwht256_orthonormal.restype = ctypes.c_int
        L.oracle_encode_fp8.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_f32p]
        L.oracle_encode_fp8.restype = ctypes.c_int
        L.oracle_decode_fp8_rows.argtypes = [_c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_f64p]
        L.oracle_decode_fp8_rows.restype = ctypes.c_int
        L.oracle_tq4_codebook.argtypes = [_c_f64p, _c_f32p, _c_f32p, ctypes.POINTER(ctypes.c_int)]
        L.oracle_tq4_codebook.restype = ctypes.c_int
        L.oracle_tq_codebook.argtypes = [ctypes.c_int, _c_f64p, _c_f32p, _c_f32p, ctypes.POINTER(ctypes.c_int)]
        L.oracle_tq_codebook.restype = ctypes.c_int
        L.oracle_quantizer_mse.argtypes = [_c_f64p, _c_f64p]
        L.oracle_quantizer_mse_n.argtypes = [ctypes.c_int, _c_f64p, _c_f64p]
        L.oracle_quantizer_mse_n.restype = ctypes.c_double
        L.oracle_tq_code_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_tq_code_bytes.restype = ctypes.c_int64
        L.oracle_encode_tq.argtypes = [ctypes.c_int, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_u8p, _c_f32p]
        L.oracle_encode_tq.restype = ctypes.c_int
        L.oracle_decode_tq_rows.argtypes = [ctypes.c_int, _c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p,
                                            _c_f64p]
        L.oracle_decode_tq_rows.restype = ctypes.c_int
        L.oracle_tq_identity_check.argtypes = [ctypes.c_int, _c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p,
                                               _c_f64p, _c_f64p, ctypes.c_int]
        L.oracle_tq_identity_check.restype = ctypes.c_double
        L.oracle_quantizer_mse.restype = ctypes.c_double
        L.oracle_encode_tq4.argtypes = [_c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_u8p, _c_f32p]
        L.oracle_encode_tq4.restype = ctypes.c_int
        L.oracle_decode_tq4_rows.argtypes = [_c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p, _c_f64p]
        L.oracle_decode_tq4_rows.restype = ctypes.c_int
        L.oracle_tq4_identity_check.argtypes = [_c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p,
                                                _c_f64p, _c_f64p]
        L.oracle_tq4_identity_check.restype = ctypes.c_double
        L.oracle_tq4_identity_check_planted.argtypes = [_c_u8p, _c_f32p, ctypes.c_int64, ctypes.c_int, _c_u8p,
                                                        _c_f64p, _c_f64p, ctypes.c_int]
        L.oracle_tq4_identity_check_planted.restype = ctypes.c_double
        L.oracle_decode_attn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _c_i64p, _c_u8p, _c_f32p, _c_u16p, _c_u8p, _c_f32p, _c_f32p,
                                         ctypes.c_double, _c_f64p, _c_f64p]
        L.oracle_decode_attn.restype = ctypes.c_int
        L.oracle_q4_0_block.argtypes = [_c_f32p, _c_u8p]
        L.oracle_q4_0_block.restype = None
        L.oracle_q4_0_block_dequant.argtypes = [_c_u8p, _c_u16p]
        L.oracle_q4_0_block_dequant.restype = None
        L.oracle_append_q4_0.argtypes = [_c_u8p, _c_u8p, ctypes.c_int64, _c_i32p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i32p, _c_i64p,
                                         _c_f32p, _c_f32p, ctypes.c_int]
        L.oracle_append_q4_0.restype = ctypes.c_int
        L.oracle_gather_q4_0.argtypes = [_c_u8p, _c_u8p, ctypes.c_int64, _c_i32p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i64p, _c_u16p, _c_u16p]
        L.oracle_gather_q4_0.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def set_threads(n=0):
    """Sets the OpenMP thread count (n > 0); returns the count in force."""
    return lib().oracle_set_threads(int(n))


# ---- formats --------------------------------------------------------------

def e4m3_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(x, _c_f32p), x.size, _p(out, _c_u8p))
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_array(_p(c, _c_u8p), c.size, _p(out, _c_f64p))
    return out


def f16_encode(x):
    if np.asarray(x).dtype == np.float64:
        x = _c(x, np.float64)
        out = np.empty(x.shape, np.uint16)
        lib().oracle_f16_encode_array_f64(_p(x, _c_f64p), x.size, _p(out, _c_u16p))
        return out
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_encode_array(_p(x, _c_f32p), x.size, _p(out, _c_u16p))
    return out


def f16_decode(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_f16_decode_array(_p(h, _c_u16p), h.size, _p(out, _c_f64p))
    return out


def bf16_encode(x):
    if np.asarray(x).dtype == np.float64:
        x = _c(x, np.float64)
        out = np.empty(x.shape, np.uint16)
        lib().oracle_bf16_encode_array_f64(_p(x, _c_f64p), x.size, _p(out, _c_u16p))
        return out
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_encode_array(_p(x, _c_f32p), x.size, _p(out, _c_u16p))
    return out


def bf16_decode(b):
    return np.array([lib().oracle_bf16_decode(int(v)) for v in np.ravel(b)],
                    np.float64).reshape(np.shape(b))


# ---- transforms -----------------------------------------------------------

def fwht(x):
    """Unnormalized FWHT of each row (last axis, a power of two), fp32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    n = x.shape[-1]
    rows = x.size // n
    _check(lib().oracle_fwht_rows_f32(_p(x, _c_f32p), rows, n), "fwht")
    return x


def fwht256_orthonormal(x):
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    assert x.shape[-1] == 256
    flat = x.reshape(-1, 256)
    for r in range(flat.shape[0]):
        row = flat[r]
        lib().oracle_fwht256_orthonormal(_p(row, _c_f32p))
    return x


# ---- codecs ---------------------------------------------------------------

def encode_fp8(x):
    x = _c(x, np.float32)
    n, dim = x.shape
    codes = np.empty((n, dim), np.uint8)
    scales = np.empty(n, np.float32)
    _check(lib().oracle_encode_fp8(_p(x, _c_f32p), n, dim, _p(codes, _c_u8p), _p(scales, _c_f32p)),
           "encode_fp8")
    return codes, scales


def decode_fp8(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    n, dim = codes.shape
    out = np.empty((n, dim), np.float64)
    lib().oracle_decode_fp8_rows(_p(codes, _c_u8p), _p(scales, _c_f32p), n, dim, _p(out, _c_f64p))
    return out


def tq4_codebook():
    """Returns (levels_exact[16] f64, levels_bf16[16] f32, thresholds[15] f32, iterations)."""
    le = np.empty(16, np.float64)
    lb = np.empty(16, np.float32)
    th = np.empty(15, np.float32)
    it = ctypes.c_int(0)
    _check(lib().oracle_tq4_codebook(_p(le, _c_f64p), _p(lb, _c_f32p), _p(th, _c_f32p), ctypes.byref(it)),
           "tq4_codebook")
    return le, lb, th, it.value


def tq_codebook(bits):
    """Codec-1 codebook of a b-bit tier (b = 3, 4, 6): (levels_exact[2^b] f64,
    levels_bf16[2^b] f32, thresholds[2^b - 1] f32, iterations)."""
    n = 1 << bits
    le = np.empty(n, np.float64)
    lb = np.empty(n, np.float32)
    th = np.empty(n - 1, np.float32)
    it = ctypes.c_int(0)
    _check(lib().oracle_tq_codebook(int(bits), _p(le, _c_f64p), _p(lb, _c_f32p), _p(th, _c_f32p),
                                    ctypes.byref(it)), "tq_codebook")
    return le, lb, th, it.value


def tq_code_bytes(bits, dim):
    """Code bytes per row of a b-bit tier, -1 where the width is refused."""
    return lib().oracle_tq_code_bytes(int(bits), int(dim))


def quantizer_mse_n(levels, thresholds):
    lv = _c(levels, np.float64)
    th = _c(thresholds, np.float64)
    assert th.size == lv.size - 1
    return lib().oracle_quantizer_mse_n(lv.size, _p(lv, _c_f64p), _p(th, _c_f64p))


def encode_tq(x, sign_mask, bits):
    """Codec-1 row encoder of a b-bit tier: (codes [n][dim*b/8] u8, radii [n] f32)."""
    x = _c(x, np.float32)
    m = _c(sign_mask, np.uint8)
    n, dim = x.shape
    cb = tq_code_bytes(bits, dim)
    codes = np.empty((n, max(cb, 1)), np.uint8)
    radii = np.empty(max(n, 1), np.float32)
    rc = lib().oracle_encode_tq(int(bits), _p(x, _c_f32p), n, dim, _p(m, _c_u8p), _p(codes, _c_u8p),
                                _p(radii, _c_f32p))
    _check(rc, "encode_tq")
    return codes[:, :cb], radii[:n]


def encode_tq_rc(x, sign_mask, bits):
    """Raw return code of the codec-1 encoder (for the refusal tests)."""
    x = _c(x, np.float32)
    m = _c(sign_mask, np.uint8)
    n, dim = x.shape
    codes = np.empty((n, max(dim, 1)), np.uint8)
    radii = np.empty(max(n, 1), np.float32)
    return lib().oracle_encode_tq(int(bits), _p(x, _c_f32p), n, dim, _p(m, _c_u8p), _p(codes, _c_u8p),
                                  _p(radii, _c_f32p))


def decode_tq(codes, radii, sign_mask, bits, dim):
    codes = _c(codes, np.uint8)
    radii = _c(radii, np.float32)
    m = _c(sign_mask, np.uint8)
    n = codes.shape[0]
    assert codes.shape[1] == tq_code_bytes(bits, dim)
    out = np.empty((n, dim), np.float64)
    _check(lib().oracle_decode_tq_rows(int(bits), _p(codes, _c_u8p), _p(radii, _c_f32p), n, dim,
                                       _p(m, _c_u8p), _p(out, _c_f64p)), "decode_tq")
    return out


def tq_identity_check(codes, radii, sign_mask, q, w, bits, plant=0):
    """tq4_identity_check for a b-bit tier."""
    codes = _c(codes, np.uint8)
    radii = _c(radii, np.float32)
    m = _c(sign_mask, np.uint8)
    q = _c(q, np.float64)
    w = _c(w, np.float64)
    n = codes.shape[0]
    dim = q.shape[0]
    assert codes.shape[1] == tq_code_bytes(bits, dim)
    return lib().oracle_tq_identity_check(int(bits), _p(codes, _c_u8p), _p(radii, _c_f32p), n, dim,
                                          _p(m, _c_u8p), _p(q, _c_f64p), _p(w, _c_f64p), int(plant))


def quantizer_mse(levels, thresholds):
    lv = _c(levels, np.float64)
    th = _c(thresholds, np.float64)
    return lib().oracle_quantizer_mse(_p(lv, _c_f64p), _p(th, _c_f64p))


def encode_tq4(x, sign_mask):
    x = _c(x, np.float32)
    m = _c(sign_mask, np.uint8)
    n, dim = x.shape
    codes = np.empty((n, dim // 2), np.uint8)
    radii = np.empty(n, np.float32)
    rc = lib().oracle_encode_tq4(_p(x, _c_f32p), n, dim, _p(m, _c_u8p), _p(codes, _c_u8p), _p(radii, _c_f32p))
    _check(rc, "encode_tq4")
    return codes, radii


def encode_tq4_rc(x, sign_mask):
    """Raw return code of the TQ4 encoder (for the refusal tests)."""
    x = _c(x, np.float32)
    m = _c(sign_mask, np.uint8)
    n, dim = x.shape
    codes = np.empty((n, max(dim // 2, 1)), np.uint8)
    radii = np.empty(max(n, 1), np.float32)
    return lib().oracle_encode_tq4(_p(x, _c_f32p), n, dim, _p(m, _c_u8p), _p(codes, _c_u8p), _p(radii, _c_f32p))


def decode_tq4(codes, radii, sign_mask):
    codes = _c(codes, np.uint8)
    radii = _c(radii, np.float32)
    m = _c(sign_mask, np.uint8)
    n = codes.shape[0]
    dim = codes.shape[1] * 2
    out = np.empty((n, dim), np.float64)
    _check(lib().oracle_decode_tq4_rows(_p(codes, _c_u8p), _p(radii, _c_f32p), n, dim, _p(m, _c_u8p),
                                        _p(out, _c_f64p)), "decode_tq4")
    return out


def tq4_identity_check(codes, radii, sign_mask, q, w, plant=0):
    """Largest relative discrepancy of the two rotation identities; plant > 0
    plants a known mistake in the check (tests of the check's sensitivity)."""
    codes = _c(codes, np.uint8)
    radii = _c(radii, np.float32)
    m = _c(sign_mask, np.uint8)
    q = _c(q, np.float64)
    w = _c(w, np.float64)
    n = codes.shape[0]
    dim = codes.shape[1] * 2
    if plant:
        return lib().oracle_tq4_identity_check_planted(_p(codes, _c_u8p), _p(radii, _c_f32p), n, dim,
                                                       _p(m, _c_u8p), _p(q, _c_f64p), _p(w, _c_f64p), int(plant))
    return lib().oracle_tq4_identity_check(_p(codes, _c_u8p), _p(radii, _c_f32p), n, dim, _p(m, _c_u8p),
                                           _p(q, _c_f64p), _p(w, _c_f64p))


def decode_attn(qmode, seq_offsets, codes, row_scale, k_rope, q_lat, q_rope, sm_scale, sign_mask=None):
    """fp64 decode attention.  q_lat [S][H][dim], q_rope [S][H][R], k_rope bf16 bits
    [rows][R].  Returns (out [S][H][dim] f64, lse [S][H] f64)."""
    offs = _c(seq_offsets, np.int64)
    codes = _c(codes, np.uint8)
    rs = _c(row_scale, np.float32)
    kr = _c(k_rope, np.uint16)
    ql = _c(q_lat, np.float32)
    qr = _c(q_rope, np.float32)
    S, H, dim = ql.shape
    R = qr.shape[2]
    m = _c(sign_mask if sign_mask is not None else np.zeros(max(dim // 8, 1), np.uint8), np.uint8)
    out = np.empty((S, H, dim), np.float64)
    lse = np.empty((S, H), np.float64)
    rc = lib().oracle_decode_attn(int(qmode), S, H, dim, R, _p(offs, _c_i64p), _p(codes, _c_u8p),
                                  _p(rs, _c_f32p), _p(kr, _c_u16p), _p(m, _c_u8p), _p(ql, _c_f32p),
                                  _p(qr, _c_f32p), float(sm_scale), _p(out, _c_f64p), _p(lse, _c_f64p))
    _check(rc, "decode_attn")
    return out, lse


def decode_attn_sparse(qmode, index_offsets, row_index, codes, row_scale, k_rope, q_lat, q_rope, sm_scale,
                       sign_mask=None):
    """Sparse (DSA-style) decode attention, fp64: query s attends over the cache
    rows row_index[index_offsets[s]:index_offsets[s+1]], a row listed twice
    counting twice ([KV8] commit list item 2, the DSA-aware gather, and the
    rebase note on the DSA gather: the selected rows are staged into a compact
    buffer for the dense kernel).  By that definition it is decode_attn over the
    listed rows in list order; the selection is numpy indexing."""
    idx = np.asarray(row_index, np.int64)
    return decode_attn(qmode, index_offsets, np.asarray(codes)[idx], np.asarray(row_scale)[idx],
                       np.asarray(k_rope)[idx], q_lat, q_rope, sm_scale, sign_mask)


# ---- q4_0 paged tier ------------------------------------------------------

def q4_0_block(x32):
    x = _c(x32, np.float32)
    assert x.shape == (32,)
    out = np.empty(18, np.uint8)
    lib().oracle_q4_0_block(_p(x, _c_f32p), _p(out, _c_u8p))
    return out


def q4_0_block_dequant(blk):
    b = _c(blk, np.uint8)
    out = np.empty(32, np.uint16)
    lib().oracle_q4_0_block_dequant(_p(b, _c_u8p), _p(out, _c_u16p))
    return out


def append_q4_0(k_pool, v_pool, table, page_size, pos0, src_off, k_src, v_src, no_rotate=False):
    """In place on k_pool/v_pool [n_cells][n_kv_heads][144] u8."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    n_cells, n_kv, rb = k_pool.shape
    tab = _c(table, np.int32)
    n_seqs, max_pages = tab.shape
    p0 = _c(pos0, np.int32)
    so = _c(src_off, np.int64)
    ks = _c(k_src, np.float32)
    vs = _c(v_src, np.float32)
    head_dim = ks.shape[-1]
    rc = lib().oracle_append_q4_0(_p(k_pool, _c_u8p), _p(v_pool, _c_u8p), n_cells, _p(tab, _c_i32p), max_pages,
                                  page_size, n_kv, head_dim, n_seqs, _p(p0, _c_i32p), _p(so, _c_i64p),
                                  _p(ks, _c_f32p), _p(vs, _c_f32p), 1 if no_rotate else 0)
    _check(rc, "append_q4_0")


def gather_q4_0(k_pool, v_pool, table, page_size, dst_off, head_dim=256, k_dst=None, v_dst=None):
    n_cells, n_kv, rb = k_pool.shape
    kp = _c(k_pool, np.uint8)
    vp = _c(v_pool, np.uint8)
    tab = _c(table, np.int32)
    n_seqs, max_pages = tab.shape
    do = _c(dst_off, np.int64)
    total = int(do[-1])
    if k_dst is None:
        k_dst = np.zeros((total, n_kv, head_dim), np.uint16)
    if v_dst is None:
        v_dst = np.zeros((total, n_kv, head_dim), np.uint16)
    rc = lib().oracle_gather_q4_0(_p(kp, _c_u8p), _p(vp, _c_u8p), n_cells, _p(tab, _c_i32p), max_pages,
                                  page_size, n_kv, head_dim, n_seqs, _p(do, _c_i64p), _p(k_dst, _c_u16p),
                                  _p(v_dst, _c_u16p))
    _check(rc, "gather_q4_0")
    return k_dst, v_dst


def q4_0_rows_f64(rows):
    """Dequantize q4_0 head-rows u8 [..., 144] to fp64 [..., 256] in the rotated
    domain, exactly as the fused decode reads them ([Q4], QSA_KV_Q4 commit:
    every block is (nibble - 8) * f32(d), no rounding to binary16): block b is
    bytes 18b .. 18b+17, a little-endian binary16 scale d then 16 bytes whose
    low nibbles are elements 0..15 and high nibbles elements 16..31."""
    r = np.ascontiguousarray(rows, np.uint8)
    lead = r.shape[:-1]
    blk = r.reshape(-1, 8, 18)
    d = blk[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    nib = blk[:, :, 2:18]
    codes = np.concatenate([nib & 15, nib >> 4], axis=2).astype(np.float64)
    return ((codes - 8.0) * d[:, :, None]).reshape(lead + (256,))


def decode_attn_q4_0(k_pool, v_pool, table, page_size, len_off, q, sm_scale):
    """Fused decode attention over the q4_0 pools, fp64 ([Q4], QSA_KV_Q4 commit:
    the query rows pass through the orthonormal 256-point FWHT, the pools are
    dequantized per block, softmax and the weighted sum of V rows run in the
    rotated domain, and the merged row o / L is rotated back with the same
    self-inverse transform; the sigmoid gate that follows in the pages' model is
    not part of it).

    k_pool, v_pool: u8 [n_cells][n_kv][144]; table: int32 [n_seqs][max_pages];
    len_off: int64 [n_seqs + 1], sequence s attends positions
    0 .. len_off[s+1] - len_off[s] - 1; q: fp32 [n_seqs][n_q][256], n_q a
    multiple of n_kv, query head h reading kv head h // (n_q / n_kv).
    Positions whose cell does not exist (page column past the table, negative
    entry, cell past the pool) take no part.  Returns (out [n_seqs][n_q][256],
    lse [n_seqs][n_q]) in fp64; a sequence with no positions gives 0 and -inf.
    The FWHT is the Sylvester-ordered Hadamard matrix over 16 (scipy's
    ``hadamard``, a library primitive), the same order as the append's."""
    from scipy.linalg import hadamard
    kp = np.asarray(k_pool, np.uint8)
    vp = np.asarray(v_pool, np.uint8)
    tab = np.asarray(table, np.int32)
    offs = np.asarray(len_off, np.int64)
    qq = np.asarray(q, np.float32).astype(np.float64)
    n_cells, n_kv, _ = kp.shape
    n_seqs, n_q, dim = qq.shape
    assert dim == 256 and n_q % n_kv == 0
    group = n_q // n_kv
    hm = hadamard(256).astype(np.float64) / 16.0
    q_rot = qq @ hm
    out = np.zeros((n_seqs, n_q, 256), np.float64)
    lse = np.full((n_seqs, n_q), -np.inf, np.float64)
    for s in range(n_seqs):
        n = int(offs[s + 1] - offs[s])
        pos = np.arange(max(n, 0), dtype=np.int64)
        col = pos // page_size
        ok = col < tab.shape[1]
        page = np.where(ok, tab[s, np.minimum(col, tab.shape[1] - 1)], -1).astype(np.int64)
        cell = page * page_size + pos % page_size
        ok &= (page >= 0) & (cell < n_cells)
        cell = cell[ok]
        if cell.size == 0:
            continue
        for g in range(n_kv):
            kd = q4_0_rows_f64(kp[cell, g])
            vd = q4_0_rows_f64(vp[cell, g])
            for h in range(g * group, (g + 1) * group):
                sc = float(sm_scale) * (kd @ q_rot[s, h])
                m = sc.max()
                w = np.exp(sc - m)
                den = w.sum()
                out[s, h] = hm @ ((w @ vd) / den)
                lse[s, h] = m + np.log(den)
    return out, lse
