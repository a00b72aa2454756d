"""GPU parity of the fused decode attention over the q4_0 pools, through the C ABI.

Pools are written by the oracle's append on the CPU and the same bytes are
uploaded, so both sides read identical blocks.  The HIP result must match the
oracle's fp64 evaluation within max|err| / max|ref| <= 1e-5 per sequence
(fp32 arithmetic over 256-term dots, two 256-point rotations and a softmax: a
few 1e-6 relative in practice; the pages report 1.9-2.7e-7 for their fp32
attention and merge), and lse within 1e-5 * max(1, |lse|).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_kv_cache_row_amd import kvq, workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5
DEV = "cuda"
SM = workloads.Q4_SM_SCALE


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _pools(n_seqs, lmin, lmax, seed=1004):
    w = workloads.Q4Workload(seed=seed, n_seqs=n_seqs, lmin=lmin, lmax=lmax)
    kp, vp = w.empty_pools()
    oracle.append_q4_0(kp, vp, w.table, 64, w.pos0_prefill, w.prefill_off, w.k_prefill, w.v_prefill)
    return w, kp, vp


def _run(kp, vp, table, len_off, q, split_rows=0, with_lse=True):
    kpd = torch.from_numpy(kp).to(DEV)
    vpd = torch.from_numpy(vp).to(DEV)
    tab = torch.from_numpy(np.ascontiguousarray(table, np.int32)).to(DEV)
    cache = kvq.q4_cache(kpd, vpd, tab, 64)
    off = torch.from_numpy(np.ascontiguousarray(len_off, np.int64)).to(DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    a = kvq.q4_attn_args(off, int(len_off[-1]), qd, out, lse, SM, split_rows)
    ws = kvq.alloc_workspace_q4(cache, a)
    kvq.kvq_decode_attn_q4_0(cache, a, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def _check(out, lse, ref_o, ref_l, label):
    assert np.all(np.isfinite(out)), label
    for s in range(ref_o.shape[0]):
        if np.all(np.isneginf(ref_l[s])):
            assert np.all(out[s] == 0), label
            if lse is not None:
                assert np.all(np.isneginf(lse[s])), label
            continue
        e = np.max(np.abs(out[s] - ref_o[s])) / max(np.max(np.abs(ref_o[s])), 1e-30)
        assert e <= TOL, f"{label} seq {s}: rel err {e:.3e}"
        if lse is not None:
            d = np.max(np.abs(lse[s] - ref_l[s]) / np.maximum(1.0, np.abs(ref_l[s])))
            assert d <= TOL, f"{label} seq {s}: lse err {d:.3e}"


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_q4_attn_head_groups(group):
    _say(f"q4 attn group {group}")
    w, kp, vp = _pools(4, 100, 700)
    q = workloads.q4_queries(1007, w.n_seqs, n_q_heads=8 * group)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, w.table, 64, w.prefill_off, q, SM)
    out, lse = _run(kp, vp, w.table, w.prefill_off, q)
    _check(out, lse, ref_o, ref_l, f"group {group}")


@pytest.mark.parametrize("split_rows", [256, 512, 1024])
def test_q4_attn_split_sweep(split_rows):
    _say(f"q4 attn split {split_rows}")
    w, kp, vp = _pools(5, 60, 1500, seed=1010)
    q = workloads.q4_queries(1008, w.n_seqs)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, w.table, 64, w.prefill_off, q, SM)
    out, lse = _run(kp, vp, w.table, w.prefill_off, q, split_rows=split_rows)
    _check(out, lse, ref_o, ref_l, f"split {split_rows}")
    out2, none = _run(kp, vp, w.table, w.prefill_off, q, split_rows=split_rows, with_lse=False)
    np.testing.assert_array_equal(out2, out)


def test_q4_attn_missing_cells_empty_and_overlong_sequences():
    _say("q4 attn missing cells / empty / overlong")
    w, kp, vp = _pools(4, 300, 900, seed=1011)
    q = workloads.q4_queries(1009, w.n_seqs)
    table = w.table.copy()
    table[0, 2] = -1                       # one missing page inside sequence 0
    table[1, 1:] = -1                      # sequence 1 keeps its first page only
    lens = np.diff(w.prefill_off).copy()
    lens[2] = 0                            # an empty sequence
    lens[3] = table.shape[1] * 64 + 300    # longer than the table holds
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, table, 64, off, q, SM)
    for split in (0, 256):
        out, lse = _run(kp, vp, table, off, q, split_rows=split)
        _check(out, lse, ref_o, ref_l, f"edge split {split}")


def test_q4_attn_single_position_and_all_missing():
    _say("q4 attn one position / all missing")
    w, kp, vp = _pools(3, 100, 200, seed=1012)
    q = workloads.q4_queries(1010, w.n_seqs)
    table = w.table.copy()
    table[2, :] = -1
    off = np.array([0, 1, 1 + 65, 1 + 65 + 100], np.int64)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, table, 64, off, q, SM)
    out, lse = _run(kp, vp, table, off, q)
    _check(out, lse, ref_o, ref_l, "one position")


def test_q4_attn_full_size():
    """The paged-pool workload: 16 sequences of 504 .. 8184 positions (56 mod
    64), 8 KV heads x 256, page 64, permuted pages, 32 query heads."""
    _say("q4 attn full size")
    w, kp, vp = _pools(16, 512, 8192)
    q = workloads.q4_queries(1007, w.n_seqs)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, w.table, 64, w.prefill_off, q, SM)
    out, lse = _run(kp, vp, w.table, w.prefill_off, q)
    _check(out, lse, ref_o, ref_l, "full size")


def test_q4_attn_refusals():
    _say("q4 attn refusals")
    w, kp, vp = _pools(2, 100, 200, seed=1013)
    kpd = torch.from_numpy(kp).to(DEV)
    vpd = torch.from_numpy(vp).to(DEV)
    tab = torch.from_numpy(w.table).to(DEV)
    cache = kvq.q4_cache(kpd, vpd, tab, 64)
    off = torch.from_numpy(w.prefill_off).to(DEV)
    n = int(w.prefill_off[-1])
    q3 = torch.zeros((2, 24, 256), dtype=torch.float32, device=DEV)
    o3 = torch.zeros_like(q3)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn_q4_0_workspace_bytes(cache, kvq.q4_attn_args(off, n, q3, o3))
    q = torch.zeros((2, 32, 256), dtype=torch.float32, device=DEV)
    o = torch.zeros_like(q)
    a = kvq.q4_attn_args(off, n, q, o)
    need = kvq.kvq_decode_attn_q4_0_workspace_bytes(cache, a)
    short = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn_q4_0(cache, a, short)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    bad = kvq.q4_attn_args(off, n, q, o, split_rows=100)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attn_q4_0(cache, bad, torch.empty(need, dtype=torch.uint8, device=DEV))
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG


@pytest.mark.parametrize("page_size,n_kv,group", [(48, 2, 8), (16, 3, 2), (1, 1, 16)])
def test_q4_attn_other_pages_and_kv_heads(page_size, n_kv, group):
    """Page sizes that are not powers of two (48), tiny pages (1), 1-3 KV heads."""
    _say(f"q4 attn page {page_size} kv {n_kv} group {group}")
    rng = np.random.default_rng(1014 + page_size)
    lens = np.array([0, 37, 300, 1100], np.int64)
    pages = (lens + page_size - 1) // page_size
    max_pages = int(pages.max())
    perm = rng.permutation(int(pages.sum())).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, np.int32)
    k = 0
    for s, n in enumerate(pages):
        table[s, :n] = perm[k:k + n]
        k += n
    n_cells = int(pages.sum()) * page_size
    kp = np.zeros((n_cells, n_kv, 144), np.uint8)
    vp = np.zeros_like(kp)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = int(off[-1])
    ks = (rng.standard_normal((total, n_kv, 256)) * rng.choice([0.01, 1.0, 30.0], (total, n_kv, 1))).astype(np.float32)
    vs = rng.standard_normal((total, n_kv, 256)).astype(np.float32)
    oracle.append_q4_0(kp, vp, table, page_size, np.zeros(len(lens), np.int32), off, ks, vs)
    q = (rng.standard_normal((len(lens), n_kv * group, 256)) / 16).astype(np.float32)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, table, page_size, off, q, SM)
    kpd = torch.from_numpy(kp).to(DEV)
    vpd = torch.from_numpy(vp).to(DEV)
    cache = kvq.q4_cache(kpd, vpd, torch.from_numpy(table).to(DEV), page_size)
    qd = torch.from_numpy(q).to(DEV)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    a = kvq.q4_attn_args(torch.from_numpy(off).to(DEV), total, qd, out, lse, SM, 256)
    kvq.kvq_decode_attn_q4_0(cache, a, kvq.alloc_workspace_q4(cache, a))
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"page {page_size} kv {n_kv}")


@pytest.mark.parametrize("split_rows", [65536, 0])
def test_q4_attn_long_flat_sequence(split_rows):
    """One sequence of 65536 positions under a zero query (every score 0, so
    the softmax is flat and every position weighs the same), one KV head and
    four query heads, at one split of the whole sequence and at the automatic
    split.  The value sum then adds 8192 positions per lane per parity; the
    offset nibbles' -8 term must not leave an error that grows with that."""
    _say(f"q4 attn long flat sequence split {split_rows}")
    rng = np.random.default_rng(1015)
    n = 65536
    page = 64
    n_pages = n // page
    table = rng.permutation(n_pages).astype(np.int32)[None, :]
    kp = rng.integers(0, 256, (n, 1, 144), dtype=np.uint8)
    vp = rng.integers(0, 256, (n, 1, 144), dtype=np.uint8)
    for pool in (kp, vp):  # finite binary16 scales, both signs, magnitudes 0.25 .. 4
        d = (rng.uniform(0.25, 4.0, (n, 1, 8)) * rng.choice([-1.0, 1.0], (n, 1, 8))).astype(np.float16)
        b = d.view(np.uint16)
        for blk in range(8):
            pool[:, :, 18 * blk] = (b[:, :, blk] & 0xFF).astype(np.uint8)
            pool[:, :, 18 * blk + 1] = (b[:, :, blk] >> 8).astype(np.uint8)
    off = np.array([0, n], np.int64)
    q = np.zeros((1, 4, 256), np.float32)
    ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, table, page, off, q, SM)
    out, lse = _run(kp, vp, table, off, q, split_rows=split_rows)
    _check(out, lse, ref_o, ref_l, f"long flat split {split_rows}")


def test_q4_attn_peaked_scores_and_wide_value_scales():
    """A peaked softmax (the query times 8) over value rows whose binary16 block
    scales span 2^-20 .. 2^10 (subnormal ones included, both signs) and jump
    from one 32-position stretch to the next, K scales 2^-3 .. 2^3: the three
    query terms of the scores, the two exact terms of the value products and
    their per-tile power-of-two range must keep the fp32 result.  Two KV heads,
    8 query heads each (one workgroup of 8 heads), and 4 each."""
    _say("q4 attn peaked scores, wide value scales")
    rng = np.random.default_rng(1016)
    n, page, n_kv = 4096, 64, 2
    table = rng.permutation(n // page).astype(np.int32)[None, :]
    kp = rng.integers(0, 256, (n, n_kv, 144), dtype=np.uint8)
    vp = rng.integers(0, 256, (n, n_kv, 144), dtype=np.uint8)
    stretch = np.repeat(rng.uniform(-20.0, 10.0, n // 32), 32)[:, None, None]  # per 32 positions
    for pool, lo, hi, base in ((kp, -3.0, 3.0, 0.0), (vp, -4.0, 0.0, stretch)):
        e = base + rng.uniform(lo, hi, (n, n_kv, 8))
        d = (np.exp2(e) * rng.choice([-1.0, 1.0], (n, n_kv, 8))).astype(np.float16)
        b = d.view(np.uint16)
        for blk in range(8):
            pool[:, :, 18 * blk] = (b[:, :, blk] & 0xFF).astype(np.uint8)
            pool[:, :, 18 * blk + 1] = (b[:, :, blk] >> 8).astype(np.uint8)
    off = np.array([0, n], np.int64)
    for group in (8, 4):
        q = (workloads.q4_queries(1017, 1, n_q_heads=n_kv * group) * 8.0).astype(np.float32)
        ref_o, ref_l = oracle.decode_attn_q4_0(kp, vp, table, page, off, q, SM)
        out, lse = _run(kp, vp, table, off, q)
        assert np.all(np.isfinite(out))
        # fp32 evaluation of scores up to S (natural-log units) moves the weights by about S 2^-24
        S = float(np.max(np.abs(ref_l)))
        tol = max(TOL, 4.0 * S * 2.0 ** -24)
        _say(f"  group {group}: max |lse| {S:.1f}, bar {tol:.2e}")
        e = np.max(np.abs(out - ref_o)) / np.max(np.abs(ref_o))
        d = np.max(np.abs(lse - ref_l) / np.maximum(1.0, np.abs(ref_l)))
        _say(f"  group {group}: max|err|/max|ref| {e:.2e}, lse {d:.2e}")
        assert e <= tol, f"group {group}: rel err {e:.3e}"
        assert d <= tol, f"group {group}: lse err {d:.3e}"
