"""CPU check of the cell rule the dim-512 TQ4 encoder uses for bucketing.

[KV8] colibri PR #399, "Why rotated-int4 for the 4-bit tier": each rotated
coordinate w gets the index of its Lloyd-Max interval, idx = #{k : w > T_k}
with T_k = fl(t_k * r).  The dim-512 kernel finds it as
idx = c + [w > T_c], c = clamp(floor(a w / r + 7.5), 0, 14): one comparison
instead of a search.  That is exact only if every cell edge (c - 7.5) / a lies
strictly between t_{c-1} and t_c with room for rounding.  This file reads a and
the thresholds from the HIP sources, checks that condition, and replays the
rule in fp32 numpy against the definition on random and threshold-adjacent
values (rounding of a / r and of the cell value perturbed both ways).
"""
import os
import re
import struct

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_cache_row_amd", "csrc")


def _thresholds():
    text = open(os.path.join(CSRC, "kvq_codebook.inc")).read()
    m = re.search(r"#define KVQ_TQ4_THRESH_BITS \{([^}]*)\}", text)
    bits = [int(v, 16) for v in re.findall(r"0x[0-9A-Fa-f]+", m.group(1))]
    return np.array([struct.unpack("<f", struct.pack("<I", b))[0] for b in bits], dtype=np.float32)


def _scale():
    text = open(os.path.join(CSRC, "kvq_encode.hip")).read()
    m = re.search(r"constexpr float D512_CELL_SCALE = ([0-9.]+)f;", text)
    return np.float32(float(m.group(1)))


def test_cell_edges_separate_the_thresholds():
    t = _thresholds().astype(np.float64)
    a = float(_scale())
    assert len(t) == 15 and np.all(np.diff(t) > 0)
    for c in range(1, 15):
        edge = (c - 7.5) / a
        assert t[c - 1] + 0.05 < edge < t[c] - 0.05, (c, edge, t[c - 1], t[c])


def _rule(w, r, t, a, nudge_inv=0, nudge_cell=0):
    """The kernel's steps in fp32; nudge_* move a / r and the cell value by that
    many ulps (the kernel's reciprocal is not correctly rounded)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.float32(a) * (np.float32(1.0) / r)  # +inf for a zero radius
        if nudge_inv and np.isfinite(inv):
            inv = np.nextafter(inv, np.float32(np.inf) if nudge_inv > 0 else np.float32(-np.inf))
        cf = (w.astype(np.float64) * np.float64(inv) + 7.5).astype(np.float32)  # the fma: one rounding
    for _ in range(abs(nudge_cell)):
        cf = np.nextafter(cf, np.float32(np.inf) if nudge_cell > 0 else np.float32(-np.inf))
    cf = np.where(np.isnan(cf), np.float32(0.0), cf)  # 0 * inf: the clamp and conversion give 0
    c = np.clip(cf, np.float32(0.0), np.float32(14.5)).astype(np.int64)  # floor of a value >= 0
    T = (t[c] * r).astype(np.float32)
    return c + (w > T)


def _definition(w, r, t):
    T = (t * r).astype(np.float32)
    return (w[:, None] > T[None, :]).sum(axis=1)


def test_cell_rule_matches_the_definition():
    t = _thresholds()
    a = _scale()
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
                got = _rule(w, r, t, a, nudge_inv=ni, nudge_cell=nc)
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, (float(r), ni, nc, w[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_a_misplaced_edge_is_caught():
    """The edge check fails for a scale outside the separating interval."""
    t = _thresholds().astype(np.float64)
    for a in (3.0, 3.6):
        ok = all(t[c - 1] + 0.05 < (c - 7.5) / a < t[c] - 0.05 for c in range(1, 15))
        assert not ok
