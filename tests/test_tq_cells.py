"""CPU check of the cell rules the rotated-codec encoders use for bucketing.

[KV8] colibri PR #399, "Why rotated-int4 for the 4-bit tier": each rotated
coordinate w gets the index of its Lloyd-Max interval, idx = #{k : w > T_k}
with T_k = fl(t_k * r) (the 3- and 6-bit tiers of the .coli_kv reply use the
8- and 64-level codebooks the same way).  The encoders find it with one
comparison instead of a search:
  - TQ4, dim 512: c = clamp(floor(a w / r + 7.5), 0, 14), idx = c + [w > T_c];
  - TQ3 / TQ6, any dim: cell = clamp(floor(A w / r + OFF), 0, N - 1) and a
    table of (c, t_c) per cell, idx = c + [w > fl(t_c r)] (3 bits: c = cell).
That is exact only if every cell holds at most one threshold, the one the table
names, and every threshold keeps room for rounding from the cell edges.  This
file reads the constants and tables from the HIP sources, checks those
conditions against the thresholds, and replays each rule in fp32 numpy against
the definition on random and threshold-adjacent values (rounding of a / r and
of the cell value perturbed both ways).
"""
import os
import re
import struct

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_cache_row_amd", "csrc")


def _inc():
    return open(os.path.join(CSRC, "kvq_codebook.inc")).read()


def _thresholds(bits):
    m = re.search(r"#define KVQ_TQ%d_THRESH_BITS \{([^}]*)\}" % bits, _inc())
    words = [int(v, 16) for v in re.findall(r"0x[0-9A-Fa-f]+", m.group(1))]
    return np.array([struct.unpack("<f", struct.pack("<I", b))[0] for b in words], dtype=np.float32)


def _scale():
    text = open(os.path.join(CSRC, "kvq_encode.hip")).read()
    m = re.search(r"constexpr float D512_CELL_SCALE = ([0-9.]+)f;", text)
    return np.float32(float(m.group(1)))


def _cells(bits):
    """(A, OFF, table of c per cell) of the 3- and 6-bit encoders."""
    text = _inc()
    a = float(re.search(r"#define KVQ_TQ%d_CELL_A ([0-9.eE+-]+)f" % bits, text).group(1))
    off = float(re.search(r"#define KVQ_TQ%d_CELL_OFF ([0-9.eE+-]+)f" % bits, text).group(1))
    n = int(re.search(r"#define KVQ_TQ%d_CELLS (\d+)" % bits, text).group(1))
    m = re.search(r"#define KVQ_TQ%d_CELL_TABLE \{([^}]*)\}" % bits, text)
    table = np.arange(n) if m is None else np.array([int(v) for v in m.group(1).split(",")])
    assert len(table) == n
    return np.float32(a), np.float32(off), table


def test_cell_edges_separate_the_thresholds():
    t = _thresholds(4).astype(np.float64)
    a = float(_scale())
    assert len(t) == 15 and np.all(np.diff(t) > 0)
    for c in range(1, 15):
        edge = (c - 7.5) / a
        assert t[c - 1] + 0.05 < edge < t[c] - 0.05, (c, edge, t[c - 1], t[c])


@pytest.mark.parametrize("bits", [3, 6])
def test_cell_tables_name_the_one_threshold_of_each_cell(bits):
    """Cell i covers [(i - OFF) / A, (i + 1 - OFF) / A) (cell 0 from -inf, the last to
    +inf); thresholds below it: exactly table[i]; inside it: none but t_table[i], which
    keeps 0.05 cell widths from both edges."""
    t = _thresholds(bits).astype(np.float64)
    a, off, table = _cells(bits)
    a, off = float(a), float(off)
    n, K1 = len(table), len(t)
    assert K1 == (1 << bits) - 1 and np.all(np.diff(t) > 0)
    for i in range(n):
        lo = -np.inf if i == 0 else (i - off) / a
        hi = np.inf if i == n - 1 else (i + 1 - off) / a
        below = int(np.sum(t < lo))
        inside = [k for k in range(K1) if lo <= t[k] < hi]
        assert table[i] == min(below, K1 - 1), (i, table[i], below)
        assert inside in ([], [table[i]]), (i, inside, table[i])
        for k in inside:
            pos = t[k] * a + off
            if i > 0:
                assert pos - i >= 0.05, (i, k, pos)
            if i < n - 1:
                assert i + 1 - pos >= 0.05, (i, k, pos)


def _rule_d512(w, r, t, a, nudge_inv=0, nudge_cell=0):
    """The dim-512 TQ4 kernel's steps in fp32; nudge_* move a / r and the cell value
    by that many ulps (the kernel's reciprocal is not correctly rounded)."""
    return _rule(w, r, t, a, np.float32(7.5), np.arange(15), nudge_inv, nudge_cell)


def _rule(w, r, t, a, off, table, nudge_inv=0, nudge_cell=0):
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(a) * (np.float32(1.0) / r)  # +inf for a zero radius
        if nudge_inv and np.isfinite(inv):
            inv = np.nextafter(inv, np.float32(np.inf) if nudge_inv > 0 else np.float32(-np.inf))
        cf = (w.astype(np.float64) * np.float64(inv) + np.float64(off)).astype(np.float32)  # the fma: one rounding
    for _ in range(abs(nudge_cell)):
        cf = np.nextafter(cf, np.float32(np.inf) if nudge_cell > 0 else np.float32(-np.inf))
    cf = np.where(np.isnan(cf), np.float32(0.0), cf)  # 0 * inf: the clamp and conversion give 0
    cell = np.clip(cf, np.float32(0.0), np.float32(len(table) - 0.5)).astype(np.int64)  # floor of a value >= 0
    c = table[cell]
    T = (t[c] * r).astype(np.float32)
    return c + (w > T)


def _definition(w, r, t):
    T = (t * r).astype(np.float32)
    return (w[:, None] > T[None, :]).sum(axis=1)


def _replay(rule, t):
    rng = np.random.default_rng(7)
    # radii from the smallest nonzero one (the root of the smallest denormal r^2) to
    # about 1e19, and zero (a row whose squares all underflow)
    for r in (np.float32(v) for v in (0.0, 3.8e-23, 1.7e-15, 3.1e-3, 0.731, 1.0, 22.6, 4.4e9, 1.2e18)):
        T = (t * r).astype(np.float32)
        # random coordinates of a rotated row (|w| <= sqrt(512) r, or far beyond it when
        # r^2 underflowed), every threshold product and its two neighbours, zeros and
        # denormals
        w = [(rng.standard_normal(20000) * r).astype(np.float32),
             (rng.uniform(-22.6, 22.6, 5000) * r).astype(np.float32),
             (rng.uniform(-1e4, 1e4, 2000) * r).astype(np.float32),
             T, np.nextafter(T, np.float32(np.inf)), np.nextafter(T, np.float32(-np.inf)),
             np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -1e-40, 3e-38, -3e-38], dtype=np.float32)]
        w = np.concatenate(w)
        want = _definition(w, r, t)
        for ni in (-2, 0, 2):
            for nc in (-3, 0, 3):
                got = rule(w, r, ni, nc)
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, (float(r), ni, nc, w[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_cell_rule_matches_the_definition():
    t = _thresholds(4)
    a = _scale()
    _replay(lambda w, r, ni, nc: _rule_d512(w, r, t, a, ni, nc), t)


@pytest.mark.parametrize("bits", [3, 6])
def test_cell_table_rule_matches_the_definition(bits):
    t = _thresholds(bits)
    a, off, table = _cells(bits)
    _replay(lambda w, r, ni, nc: _rule(w, r, t, a, off, table, ni, nc), t)


def test_a_misplaced_edge_is_caught():
    """The edge check fails for a scale outside the separating interval."""
    t = _thresholds(4).astype(np.float64)
    for a in (3.0, 3.6):
        ok = all(t[c - 1] + 0.05 < (c - 7.5) / a < t[c] - 0.05 for c in range(1, 15))
        assert not ok


def test_a_wrong_table_entry_is_caught():
    """Off-by-one table entries and a coarser grid break the 6-bit replay."""
    t = _thresholds(6)
    a, off, table = _cells(6)
    broken = table.copy()
    broken[len(table) // 2] += 1
    with pytest.raises(AssertionError):
        _replay(lambda w, r, ni, nc: _rule(w, r, t, a, off, broken, ni, nc), t)
    coarse = np.array([min(int(np.sum(t.astype(np.float64) < (i - 43.25) / 11.875)), 62) for i in range(87)])
    with pytest.raises(AssertionError):
        _replay(lambda w, r, ni, nc: _rule(w, r, t, np.float32(11.875), np.float32(43.25), coarse, ni, nc), t)
