"""GPU parity of the sparse (DSA-style) decode, through the C ABI.

The row gather must match numpy indexing bit for bit (clamping included).
Sparse attention must match the oracle, on the same codes, within
max|err| / max|ref| <= 2e-3 (matrix cores) or <= 1e-5 (fp32 check path).
It must also equal, bit for bit, the dense kernels run over a gathered copy
of the rows (on the fp8 matrix-core path the split kernel reads the listed
rows in place, so this compares two read paths of the same kernel).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_kv_cache_row_amd import kvq, workloads

pytestmark = pytest.mark.gpu

TOL = {kvq.KVQ_PREC_MFMA: 2e-3, kvq.KVQ_PREC_FP32: 1e-5}
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def _np(t, dtype=None):
    a = t.cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _encode(w):
    x = _t(w.latent)
    cb = kvq.code_bytes(w.qmode)
    codes = torch.empty((w.cache_rows, cb), dtype=torch.uint8, device=DEV)
    scales = torch.empty(w.cache_rows, dtype=torch.float32, device=DEV)
    if w.qmode == 1:
        kvq.kvq_encode_fp8(x, codes, scales)
    elif w.qmode == 2:
        kvq.kvq_encode_tq4(x, _t(w.sign_mask), codes, scales)
    else:
        kvq.kvq_encode_tq(kvq.TQ_QMODE_BITS[w.qmode], x, _t(w.sign_mask), codes, scales)
    return codes, scales


def _args(w, precision, offsets, n, codes, scales, k_rope, split_rows=0):
    out = torch.empty((w.n_seqs, w.n_heads, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.n_seqs, w.n_heads), dtype=torch.float32, device=DEV)
    a = kvq.attn_args(w.qmode, precision, _t(offsets), n, codes, scales, k_rope, _t(w.q_lat), _t(w.q_rope),
                      w.sm_scale, out, lse, sign_mask=_t(w.sign_mask) if w.qmode != 1 else None, split_rows=split_rows)
    return a, out, lse


def _sparse(w, precision, codes, scales, offsets, row_index, split_rows=0):
    a, out, lse = _args(w, precision, offsets, len(row_index), codes, scales, _t(w.k_rope), split_rows)
    ws = kvq.alloc_workspace_sparse(a)
    kvq.kvq_decode_attn_sparse(a, _t(np.asarray(row_index, np.int64)), w.cache_rows, ws)
    torch.cuda.synchronize()
    return _np(out).astype(np.float64), _np(lse).astype(np.float64)


def _oracle(w, codes, scales, offsets, row_index):
    return oracle.decode_attn_sparse(w.qmode, np.asarray(offsets, np.int64), np.asarray(row_index, np.int64),
                                     _np(codes), _np(scales), w.k_rope, w.q_lat, w.q_rope, w.sm_scale,
                                     sign_mask=w.sign_mask if w.qmode != 1 else None)


@pytest.mark.parametrize("qmode", [1, 2, 3, 4])
def test_gather_rows_bit_exact(qmode):
    _say(f"gather rows qmode={qmode}")
    rng = np.random.default_rng(11)
    T, cb = 1000, kvq.code_bytes(qmode)
    codes = rng.integers(0, 256, (T, cb), dtype=np.uint8)
    sc = rng.standard_normal(T).astype(np.float32)
    kr = rng.integers(0, 65536, (T, 64), dtype=np.uint16)
    # duplicates, both ends, descending runs, and two indices outside the cache
    idx = np.concatenate([[0, T - 1, T - 1, 5, -7, T + 3], np.arange(T - 1, 0, -3), rng.integers(0, T, 501)])
    idx = idx.astype(np.int64)
    n = len(idx)
    co = torch.empty((n, cb), dtype=torch.uint8, device=DEV)
    so = torch.empty(n, dtype=torch.float32, device=DEV)
    ro = torch.empty((n, 64), dtype=torch.int16, device=DEV)
    kvq.kvq_gather_rows(qmode, _t(codes), _t(sc), _t(kr), _t(idx), co, so, ro)
    torch.cuda.synchronize()
    ref = np.clip(idx, 0, T - 1)  # indices outside the cache clamp to the nearest row
    assert np.array_equal(_np(co), codes[ref])
    assert np.array_equal(_np(so).view(np.uint32), sc[ref].view(np.uint32))
    assert np.array_equal(_np(ro, np.uint16), kr[ref])


@pytest.mark.parametrize("qmode", [1, 2, 3, 4])
@pytest.mark.parametrize("precision", [kvq.KVQ_PREC_MFMA, kvq.KVQ_PREC_FP32])
def test_sparse_attn_vs_oracle(qmode, precision):
    _say(f"sparse attention qmode={qmode} precision={precision}")
    w = workloads.SparseDecodeWorkload("sparse-small", 1005, 4096, [1, 37, 300, 2048], 16, qmode=qmode,
                                       sign_seed=1002 if qmode != 1 else None)
    codes, scales = _encode(w)
    got, glse = _sparse(w, precision, codes, scales, w.offsets, w.row_index)
    ref, rlse = _oracle(w, codes, scales, w.offsets, w.row_index)
    err = rel_err(got, ref)
    assert err <= TOL[precision], f"max|err|/max|ref| = {err:.3e}"
    assert np.max(np.abs(glse - rlse)) <= 1e-3


def test_sparse_edge_lists():
    _say("sparse attention: duplicates, unsorted lists, last row, split sweep")
    w = workloads.SparseDecodeWorkload("sparse-edges", 1005, 4096, [1, 1, 1], 16)
    rng = np.random.default_rng(5)
    T = w.cache_rows
    lists = [np.array([T - 1, T - 1, T - 1, 0]), np.arange(T - 1, -1, -7), rng.integers(0, T, 333)]
    idx = np.concatenate(lists).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int64)
    codes, scales = _encode(w)
    ref, _ = _oracle(w, codes, scales, offs, idx)
    for split in (0, 32, 96):
        got, _ = _sparse(w, kvq.KVQ_PREC_MFMA, codes, scales, offs, idx, split_rows=split)
        err = rel_err(got, ref)
        assert err <= TOL[kvq.KVQ_PREC_MFMA], f"split {split}: {err:.3e}"


def _dense_on_copy(w, codes, scales, offsets, row_index, split_rows=0):
    """kvq_decode_attn over a gathered copy of the listed rows (indices clamped)."""
    ix = torch.from_numpy(np.clip(np.asarray(row_index, np.int64), 0, w.cache_rows - 1)).to(DEV)
    a, out, lse = _args(w, kvq.KVQ_PREC_MFMA, offsets, len(row_index), codes[ix].contiguous(), scales[ix].contiguous(),
                        _t(w.k_rope[ix.cpu().numpy()]), split_rows)
    kvq.kvq_decode_attn(a, kvq.alloc_workspace(a))
    torch.cuda.synchronize()
    return _np(out).astype(np.float64), _np(lse).astype(np.float64)


@pytest.mark.parametrize("lengths,split", [([2048], 0), ([100, 700, 2048], 0), ([100, 700, 2048], 256)])
def test_sparse_equals_dense_on_gathered_copy(lengths, split):
    """On the fp8 matrix-core path the split kernel reads the listed rows in place;
    the result is bit-identical to the dense kernels over a gathered copy (one
    sequence and several, automatic and fixed splits)."""
    _say(f"sparse attention == dense attention over a gathered copy: lists {lengths}, split {split}")
    w = workloads.SparseDecodeWorkload("sparse-vs-dense", 1005, 4096, lengths, 32)
    codes, scales = _encode(w)
    got, glse = _sparse(w, kvq.KVQ_PREC_MFMA, codes, scales, w.offsets, w.row_index, split_rows=split)
    out, lse = _dense_on_copy(w, codes, scales, w.offsets, w.row_index, split_rows=split)
    assert np.array_equal(out, got) and np.array_equal(lse, glse)


@pytest.mark.parametrize("n_lists", [1, 3])
def test_sparse_clamped_indices(n_lists):
    """Indices below 0 or past the cache read its first or last row (the rows read
    in place, and the gather of the other paths, clamp alike)."""
    _say(f"sparse attention: out-of-range indices clamped, {n_lists} list(s)")
    T = 1000
    w = workloads.SparseDecodeWorkload("sparse-clamp", 1005, T, [300] * n_lists, 16)
    rng = np.random.default_rng(6)
    idx = rng.integers(0, T, w.total_rows).astype(np.int64)
    idx[::7] = -3
    idx[3::11] = T
    idx[5::13] = 1 << 40
    idx[6::17] = -(1 << 40)
    codes, scales = _encode(w)
    ref, _ = _oracle(w, codes, scales, w.offsets, np.clip(idx, 0, T - 1))
    got, glse = _sparse(w, kvq.KVQ_PREC_MFMA, codes, scales, w.offsets, idx)
    assert rel_err(got, ref) <= TOL[kvq.KVQ_PREC_MFMA]
    out, lse = _dense_on_copy(w, codes, scales, w.offsets, idx)
    assert np.array_equal(out, got) and np.array_equal(lse, glse)


def test_sparse_rising_scores_in_place():
    """Scores that climb along each list (a rope-key sawtooth over the list order,
    a sharp rope query): the split kernel's first-tile reference is exceeded again
    and again, so work items restart their rows, re-reading them through the list."""
    _say("sparse attention: rising scores along the lists (restarts), rows read in place")
    T = 4096
    w = workloads.SparseDecodeWorkload("sparse-rising", 4242, T, [3000, 1000], 16)
    rng = np.random.default_rng(4244)
    perm = rng.permutation(T)
    idx = np.concatenate([perm[:3000], perm[3000:4000]]).astype(np.int64)
    rank = np.empty(T, np.int64)
    rank[perm] = np.arange(T)
    rope = rng.standard_normal((T, 64)).astype(np.float32)
    rope[:, 0] = ((rank % 512) * 0.02).astype(np.float32)
    w.k_rope = workloads.to_bf16_bits(rope)
    w.q_lat = (w.q_lat * 1e-2).astype(np.float32)
    w.q_rope = w.q_rope.copy()
    w.q_rope[..., 0] = 400.0
    codes, scales = _encode(w)
    ref, _ = _oracle(w, codes, scales, w.offsets, idx)
    for split in (0, 384):
        got, glse = _sparse(w, kvq.KVQ_PREC_MFMA, codes, scales, w.offsets, idx, split_rows=split)
        err = rel_err(got, ref)
        _say(f"  split {split}: max|err|/max|ref| = {err:.3e}")
        assert err <= TOL[kvq.KVQ_PREC_MFMA]
        out, lse = _dense_on_copy(w, codes, scales, w.offsets, idx, split_rows=split)
        assert np.array_equal(out, got) and np.array_equal(lse, glse)


def test_sparse_full_size():
    _say("sparse attention, the measured workload: T=32768 cache, 16 queries x 2048 rows, 128 heads")
    w = workloads.dsa_sparse_decode()
    codes, scales = _encode(w)
    got, _ = _sparse(w, kvq.KVQ_PREC_MFMA, codes, scales, w.offsets, w.row_index)
    ref, _ = _oracle(w, codes, scales, w.offsets, w.row_index)
    err = rel_err(got, ref)
    assert err <= TOL[kvq.KVQ_PREC_MFMA], f"max|err|/max|ref| = {err:.3e}"


def test_sparse_refusals():
    _say("sparse attention: argument checks")
    w = workloads.SparseDecodeWorkload("sparse-refuse", 1005, 256, [8], 16)
    codes, scales = _encode(w)
    a, _, _ = _args(w, kvq.KVQ_PREC_MFMA, w.offsets, 8, codes, scales, _t(w.k_rope))
    ws = kvq.alloc_workspace_sparse(a)
    with pytest.raises(kvq.KvqError) as e:  # a workspace one byte short
        kvq.kvq_decode_attn_sparse(a, _t(w.row_index), w.cache_rows, ws[: kvq.kvq_decode_attn_sparse_workspace_bytes(a) - 1])
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    with pytest.raises(kvq.KvqError) as e:  # an empty cache with a non-empty list
        kvq.kvq_decode_attn_sparse(a, _t(w.row_index), 0, ws)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG
