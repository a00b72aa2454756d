"""Pins for the oracle's sparse (DSA-style) decode attention.

Definition: query s attends over the cache rows its index list names, and a
row listed twice counts twice.  Pinned against:
  - the dense oracle, for the list of every row in order;
  - invariance under a permutation of each list;
  - every index listed twice: the output is unchanged and lse rises by
    exactly ln 2;
  - a single index: the output is that row's reconstruction and lse its score;
  - a softmax written out in numpy over rows decoded from the e4m3 bit fields
    (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals below
    exponent 1).  This one shares no arithmetic with the oracle's C code.
"""
import math

import numpy as np
import pytest

import oracle
from quantized_kv_cache_row_amd import workloads


def _case(T=300, ks=(1, 37, 120), H=4, qmode=1):
    w = workloads.SparseDecodeWorkload("sparse-pin", 1005, T, list(ks), H, qmode=qmode,
                                       sign_seed=1002 if qmode == 2 else None)
    if qmode == 1:
        codes, scales = oracle.encode_fp8(w.latent)
    else:
        codes, scales = oracle.encode_tq4(w.latent, w.sign_mask)
    mask = w.sign_mask if qmode == 2 else None
    return w, codes, scales, mask


def _sparse(w, codes, scales, mask, offsets, idx):
    return oracle.decode_attn_sparse(w.qmode, np.asarray(offsets, np.int64), np.asarray(idx, np.int64), codes, scales,
                                     w.k_rope, w.q_lat, w.q_rope, w.sm_scale, sign_mask=mask)


@pytest.mark.parametrize("qmode", [1, 2])
def test_identity_list_is_the_dense_oracle(qmode):
    w, c, s, m = _case(ks=(300,), qmode=qmode)
    offs = np.array([0, 300], np.int64)
    ref = oracle.decode_attn(qmode, offs, c, s, w.k_rope, w.q_lat, w.q_rope, w.sm_scale, sign_mask=m)
    got = _sparse(w, c, s, m, offs, np.arange(300))
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


@pytest.mark.parametrize("qmode", [1, 2])
def test_permuting_a_list_leaves_the_output(qmode):
    w, c, s, m = _case(qmode=qmode)
    rng = np.random.default_rng(3)
    perm = np.concatenate([rng.permutation(w.row_index[w.offsets[i]:w.offsets[i + 1]]) for i in range(w.n_seqs)])
    a = _sparse(w, c, s, m, w.offsets, w.row_index)
    b = _sparse(w, c, s, m, w.offsets, perm)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14) and np.allclose(a[1], b[1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("qmode", [1, 2])
def test_listing_every_row_twice_adds_ln2_to_lse(qmode):
    w, c, s, m = _case(qmode=qmode)
    twice = np.concatenate([np.repeat(w.row_index[w.offsets[i]:w.offsets[i + 1]], 2) for i in range(w.n_seqs)])
    a = _sparse(w, c, s, m, w.offsets, w.row_index)
    b = _sparse(w, c, s, m, 2 * w.offsets, twice)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    assert np.allclose(b[1] - a[1], math.log(2.0), rtol=0, atol=1e-12)


def test_a_single_index_returns_that_row():
    w, c, s, m = _case(ks=(1, 1, 1))
    out, lse = _sparse(w, c, s, m, w.offsets, w.row_index)
    for q in range(w.n_seqs):
        r = w.row_index[q]
        row = oracle.decode_fp8(c[r:r + 1], s[r:r + 1])[0]
        assert np.allclose(out[q], np.broadcast_to(row, out[q].shape), rtol=1e-12, atol=1e-30)


def _e4m3_value(b):
    sign = -1.0 if b & 0x80 else 1.0
    e, mnt = (b >> 3) & 15, b & 7
    if e == 15 and mnt == 7:
        return 0.0
    return sign * (mnt / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + mnt / 8.0) * 2.0 ** (e - 7))


def test_softmax_written_out_on_a_tiny_case():
    w, c, s, m = _case(T=40, ks=(5, 13), H=2)
    table = np.array([_e4m3_value(b) for b in range(256)])
    xh = table[c] * s.astype(np.float64)[:, None]
    kr = (w.k_rope.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out, lse = _sparse(w, c, s, m, w.offsets, w.row_index)
    for q in range(w.n_seqs):
        rows = w.row_index[w.offsets[q]:w.offsets[q + 1]]
        for h in range(w.n_heads):
            sc = w.sm_scale * (xh[rows] @ w.q_lat[q, h].astype(np.float64) + kr[rows] @ w.q_rope[q, h].astype(np.float64))
            mx = sc.max()
            p = np.exp(sc - mx)
            ref = (p[:, None] * xh[rows]).sum(0) / p.sum()
            assert np.allclose(out[q, h], ref, rtol=1e-12, atol=1e-13)
            assert abs(lse[q, h] - (mx + math.log(p.sum()))) < 1e-12
