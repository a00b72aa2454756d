"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, its host-only calls answer, struct layouts match the binding,
its codebook equals the oracle's (independently derived), and invalid
arguments are refused before anything touches a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from quantized_kv_cache_row_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(kvq_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    L = kvq.lib()
    names = _declared()
    assert set(names) == set(kvq.exported_symbols()), names
    for n in names:
        assert hasattr(L, n), n


def test_host_calls():
    assert kvq.kvq_abi_version() == 1
    assert kvq.kvq_status_string(0) == "ok"
    assert "workspace" in kvq.kvq_status_string(3)
    assert kvq.kvq_status_string(99) == "unknown status"
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_FP8, 512) == 516
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ4, 512) == 260
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ4, 384) == -1
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ3, 512) == 196
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ6, 512) == 388
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ3, 8) == 7
    assert kvq.kvq_row_bytes(kvq.KVQ_QMODE_TQ6, 768) == -1
    assert kvq.kvq_row_bytes(7, 512) == -1


def test_struct_layouts_match_binding():
    for which in (0, 1, 2):
        assert kvq.kvq_struct_layout(which) == kvq.binding_layout(which)


def test_codebook_equals_oracle():
    lv, th = kvq.kvq_tq4_codebook()
    _, olv, oth, _ = oracle.tq4_codebook()
    np.testing.assert_array_equal(np.array(lv, np.float32), olv)
    np.testing.assert_array_equal(np.array(th, np.float32), oth)
    # every tier: the library's table (its own generator) equals the oracle's
    for bits in (3, 4, 6):
        lv, th = kvq.kvq_tq_codebook(bits)
        _, olv, oth, _ = oracle.tq_codebook(bits)
        assert len(lv) == 1 << bits and len(th) == (1 << bits) - 1
        np.testing.assert_array_equal(np.array(lv, np.float32), olv)
        np.testing.assert_array_equal(np.array(th, np.float32), oth)
    L = kvq.lib()
    for bits in (0, 2, 5, 8):
        assert L.kvq_tq_codebook(bits, None, None) == kvq.KVQ_ERR_UNSUPPORTED


def test_refusals_without_launch():
    L = kvq.lib()
    P = ctypes.c_void_p
    # fp8: bad widths / counts
    assert L.kvq_encode_fp8(None, 4, 7, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_encode_fp8(None, -1, 512, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_encode_fp8(None, 4, 4096, None, None, None) == kvq.KVQ_ERR_UNSUPPORTED
    assert L.kvq_encode_fp8(None, 4, 512, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_encode_fp8(None, 0, 512, None, None, None) == kvq.KVQ_OK  # empty is a no-op
    assert L.kvq_encode_fp8(P(8), 4, 512, P(16), P(16), None) == kvq.KVQ_ERR_INVALID_ARG  # misaligned
    # TQ4: non-power-of-two widths are refused, as the pages require
    for dim in (384, 500, 576, 1024):
        assert L.kvq_encode_tq4(P(16), 4, dim, P(16), P(16), P(16), None) == kvq.KVQ_ERR_UNSUPPORTED
        for bits in (3, 4, 6):
            assert L.kvq_encode_tq(bits, P(16), 4, dim, P(16), P(16), P(16), None) == kvq.KVQ_ERR_UNSUPPORTED
    for bits in (2, 5, 8):  # only the 3-, 4- and 6-bit tiers exist
        assert L.kvq_encode_tq(bits, P(16), 4, 512, P(16), P(16), P(16), None) == kvq.KVQ_ERR_UNSUPPORTED
    assert L.kvq_encode_tq(6, P(16), 0, 512, None, None, None, None) == kvq.KVQ_OK  # empty is a no-op
    assert L.kvq_encode_tq(3, P(16), 4, 512, P(16), P(18), P(16), None) == kvq.KVQ_ERR_INVALID_ARG  # misaligned
    # attention
    a = kvq.KvqAttnArgs()
    assert L.kvq_decode_attn(ctypes.byref(a), None, 0, None) == kvq.KVQ_ERR_UNSUPPORTED  # qmode 0
    a.qmode, a.precision, a.n_seqs, a.n_heads, a.dim_lat, a.dim_rope = 1, 0, 1, 128, 512, 64
    assert L.kvq_decode_attn(ctypes.byref(a), None, 0, None) == kvq.KVQ_ERR_INVALID_ARG  # null pointers
    a.seq_offsets = a.q_lat = a.q_rope = a.out = a.codes = a.row_scale = a.k_rope = 256
    a.total_rows, a.sm_scale = 32768, 0.0417
    need = L.kvq_decode_attn_workspace_bytes(ctypes.byref(a))
    assert need > 0
    assert L.kvq_decode_attn(ctypes.byref(a), P(256), need - 1, None) == kvq.KVQ_ERR_WORKSPACE
    a.dim_lat = 576
    assert L.kvq_decode_attn(ctypes.byref(a), P(256), need, None) == kvq.KVQ_ERR_UNSUPPORTED
    a.dim_lat, a.split_rows = 512, 33
    assert L.kvq_decode_attn(ctypes.byref(a), P(256), need, None) == kvq.KVQ_ERR_INVALID_ARG
    for qm in (2, 3, 4):  # the rotated codec without a sign mask
        a.split_rows, a.qmode = 0, qm
        assert L.kvq_decode_attn(ctypes.byref(a), P(256), need, None) == kvq.KVQ_ERR_INVALID_ARG
    a.qmode = 5
    assert L.kvq_decode_attn(ctypes.byref(a), P(256), need, None) == kvq.KVQ_ERR_UNSUPPORTED
    assert L.kvq_gather_rows(5, P(256), P(256), P(256), 4, P(256), 1, P(256), P(256), P(256), None) == \
        kvq.KVQ_ERR_UNSUPPORTED
    a.qmode = 2
    assert L.kvq_decode_attn_noalloc(ctypes.byref(a), None) == kvq.KVQ_ERR_INVALID_ARG
    # the no-allocation entry point refuses work beyond its static scratch before any HIP call
    a.qmode, a.total_rows, a.split_rows = 1, 1 << 22, 1024
    assert L.kvq_decode_attn_workspace_bytes(ctypes.byref(a)) > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert L.kvq_decode_attn_noalloc(ctypes.byref(a), None) == kvq.KVQ_ERR_TOO_LARGE
    assert "scratch" in kvq.kvq_status_string(kvq.KVQ_ERR_TOO_LARGE)
    a.total_rows, a.split_rows = 32768, 0
    # decode attention with appended rows: counts, pointers, alignment, workspace
    need = L.kvq_decode_attn_workspace_bytes(ctypes.byref(a))
    assert L.kvq_decode_attn_append(ctypes.byref(a), P(256), -1, P(256), P(256), P(256), need, None) == \
        kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_decode_attn_append(ctypes.byref(a), None, 1, P(256), P(256), P(256), need, None) == \
        kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_decode_attn_append(ctypes.byref(a), P(264), 1, P(256), P(256), P(256), need, None) == \
        kvq.KVQ_ERR_INVALID_ARG  # x_new not 16-byte aligned
    assert L.kvq_decode_attn_append(ctypes.byref(a), P(256), 1, P(260), P(256), P(256), need, None) == \
        kvq.KVQ_ERR_INVALID_ARG  # fp8 codes not 8-byte aligned
    assert L.kvq_decode_attn_append(ctypes.byref(a), P(256), 1, P(256), P(256), P(256), need - 1, None) == \
        kvq.KVQ_ERR_WORKSPACE
    # sparse decode: the fp8 matrix-core path reads the listed rows in place (its workspace is
    # the dense call's); a cache of 2^32 rows or more is refused
    a.total_rows = 2048
    sneed = L.kvq_decode_attn_sparse_workspace_bytes(ctypes.byref(a))
    assert sneed == L.kvq_decode_attn_workspace_bytes(ctypes.byref(a))
    for cache_rows in (-1, 1 << 32):
        assert L.kvq_decode_attn_sparse(ctypes.byref(a), P(256), cache_rows, P(256), sneed, None) == \
            kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_decode_attn_sparse(ctypes.byref(a), P(260), 4096, P(256), sneed, None) == \
        kvq.KVQ_ERR_INVALID_ARG  # index list not 8-byte aligned
    a.precision = 1  # the fp32 check path gathers a compact copy first
    assert L.kvq_decode_attn_sparse_workspace_bytes(ctypes.byref(a)) > L.kvq_decode_attn_workspace_bytes(ctypes.byref(a))
    a.precision, a.total_rows = 0, 32768
    # q4_0
    c = kvq.KvqQ4Cache(256, 256, 256, 64, 1, 64, 8, 128)
    assert L.kvq_append_q4_0(ctypes.byref(c), 1, P(256), P(256), 1, P(256), P(256), 0, None) == \
        kvq.KVQ_ERR_UNSUPPORTED  # head_dim 128
    c.head_dim = 256
    assert L.kvq_append_q4_0(ctypes.byref(c), 1, P(256), P(256), 1, P(256), P(256), 4, None) == \
        kvq.KVQ_ERR_INVALID_ARG  # unknown flag
    assert L.kvq_gather_q4_0(None, 1, P(256), 1, P(256), P(256), None) == kvq.KVQ_ERR_INVALID_ARG
    assert L.kvq_convert(9, P(256), 4, P(256), None) == kvq.KVQ_ERR_UNSUPPORTED
    # fused q4_0 decode
    qa = kvq.KvqQ4AttnArgs(2, 32, 0, 0, 1000, 256, 256, 256, None, 0.0625, 0)
    need = L.kvq_decode_attn_q4_0_workspace_bytes(ctypes.byref(c), ctypes.byref(qa))
    assert need > 0
    assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(256), need - 1, None) == kvq.KVQ_ERR_WORKSPACE
    assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(264), need, None) == \
        kvq.KVQ_ERR_INVALID_ARG  # workspace not 256-byte aligned
    for n_q in (24, 4, 8 * 32):  # ratios 3, 1/2, 32
        qa.n_q_heads = n_q
        assert L.kvq_decode_attn_q4_0_workspace_bytes(ctypes.byref(c), ctypes.byref(qa)) == -1
        assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(256), need, None) == \
            kvq.KVQ_ERR_UNSUPPORTED
    qa.n_q_heads, qa.split_rows = 32, 300  # not a multiple of 256
    assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(256), need, None) == kvq.KVQ_ERR_INVALID_ARG
    qa.split_rows, qa.q = 0, 260  # misaligned query
    assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(256), need, None) == kvq.KVQ_ERR_INVALID_ARG
    qa.q, qa.sm_scale = 256, float("nan")
    assert L.kvq_decode_attn_q4_0(ctypes.byref(c), ctypes.byref(qa), P(256), need, None) == kvq.KVQ_ERR_INVALID_ARG


def test_binding_has_no_cpu_path():
    import torch
    x = torch.zeros(4, 512)
    with pytest.raises(ValueError, match="device tensor"):
        kvq.kvq_encode_fp8(x, torch.zeros(4, 512, dtype=torch.uint8), torch.zeros(4))


def test_binding_refuses_mis_shaped_tensors():
    """The wrappers check shapes before any pointer reaches the C ABI (which
    cannot see a tensor's extent); these raise before the device check."""
    import torch
    u8, f32, i32, i64 = torch.uint8, torch.float32, torch.int32, torch.int64
    kp = torch.zeros(64, 8, 144, dtype=u8)
    tab = torch.zeros(1, 1, dtype=i32)
    with pytest.raises(ValueError, match="k_pool"):
        kvq.q4_cache(torch.zeros(64, 8, 128, dtype=u8), kp, tab, 64)
    with pytest.raises(ValueError, match="v_pool"):
        kvq.q4_cache(kp, torch.zeros(64, 4, 144, dtype=u8), tab, 64)
    with pytest.raises(ValueError, match="block_table"):
        kvq.q4_cache(kp, kp, torch.zeros(4, dtype=i32), 64)
    off = torch.zeros(3, dtype=i64)
    q = torch.zeros(2, 32, 256)
    with pytest.raises(ValueError, match="q:"):
        kvq.q4_attn_args(off, 10, torch.zeros(2, 32, 128), q)
    with pytest.raises(ValueError, match="out"):
        kvq.q4_attn_args(off, 10, q, torch.zeros(2, 16, 256))
    with pytest.raises(ValueError, match="lse"):
        kvq.q4_attn_args(off, 10, q, q, torch.zeros(2, 16))
    with pytest.raises(ValueError, match="len_off"):
        kvq.q4_attn_args(torch.zeros(2, dtype=i64), 10, q, q)
    ql, qr = torch.zeros(1, 128, 512), torch.zeros(1, 128, 64)
    codes, sc, kr = torch.zeros(100, 512, dtype=u8), torch.zeros(100), torch.zeros(100, 64, dtype=torch.int16)
    off1 = torch.zeros(2, dtype=i64)
    with pytest.raises(ValueError, match="codes"):
        kvq.attn_args(1, 0, off1, 100, torch.zeros(100, 256, dtype=u8), sc, kr, ql, qr, 0.04, ql)
    with pytest.raises(ValueError, match="row_scale"):
        kvq.attn_args(1, 0, off1, 100, codes, torch.zeros(99), kr, ql, qr, 0.04, ql)
    with pytest.raises(ValueError, match="k_rope"):
        kvq.attn_args(1, 0, off1, 100, codes, sc, torch.zeros(100, 32, dtype=torch.int16), ql, qr, 0.04, ql)
    with pytest.raises(ValueError, match="out"):
        kvq.attn_args(1, 0, off1, 100, codes, sc, kr, ql, qr, 0.04, torch.zeros(1, 64, 512))
    with pytest.raises(ValueError, match="seq_offsets"):
        kvq.attn_args(1, 0, torch.zeros(3, dtype=i64), 100, codes, sc, kr, ql, qr, 0.04, ql)
    with pytest.raises(ValueError, match="sign_mask"):
        kvq.attn_args(2, 0, off1, 100, torch.zeros(100, 256, dtype=u8), sc, kr, ql, qr, 0.04, ql,
                      sign_mask=torch.zeros(32, dtype=u8))
