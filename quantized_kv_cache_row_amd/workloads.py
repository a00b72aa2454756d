"""Seeded synthetic inputs for the quantized-KV decode path.

This module draws random numbers and lays them out; it holds none of the
codecs' or attention's arithmetic.  The same arrays feed the HIP library and
the CPU oracle.  Every generator uses numpy's PCG64 with a SeedSequence; the
substreams are spawned in one fixed order:

    0 gains, 1 latent, 2 rope, 3 q_lat, 4 q_rope, 5 signs, 6 lengths,
    7 page permutation, 8 new rows

Workload recipe (the decode workloads of the MLA pages: 512-dim latent plus a
64-dim rope key, per-row gains, outlier channels, inert all-zero rows):

* latent[t, i] = g_t * z_ti, z ~ N(0, 1), g_t ~ lognormal(mu=0, sigma=0.5);
  channels 7 and 300 are multiplied by 20; local rows 0 and 100 of every
  sequence are all zero (latent and rope key);
* k_rope ~ N(0, 1), stored as bfloat16 (round to nearest even, by torch);
* q_lat, q_rope ~ N(0, 1) / sqrt(576); softmax scale 1 / sqrt(576);
* TQ4 sign mask: 64 random bytes (512 sign bits);
* q4_0 tier: head_dim 256, 8 KV heads, page 64, lengths uniform in
  [512, 8192] snapped down to 56 mod 64, a random permutation of all physical
  pages, amplitude classes 1e-3 / 1 / 40 cycled by (token + head) mod 3, every
  token index divisible by 97 all zero.
* fused q4_0 decode: 4 query heads per KV head (32 query heads), queries
  ~ N(0, 1) / 16 (unrotated), softmax scale 1 / 16, over the prefill pools.
"""
import math

import numpy as np

DIM_LAT = 512
DIM_ROPE = 64
SM_SCALE = 1.0 / math.sqrt(DIM_LAT + DIM_ROPE)

N_STREAMS = 9
(S_GAIN, S_LATENT, S_ROPE, S_QLAT, S_QROPE, S_SIGNS, S_LENGTHS, S_PERM, S_NEW) = range(N_STREAMS)


def streams(seed):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(N_STREAMS)]


def to_bf16_bits(x):
    """fp32 -> bfloat16 bit patterns, round to nearest even (torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def latent_rows(rng_gain, rng_lat, n_rows, local_index, dim=DIM_LAT):
    """Latent rows with per-row lognormal gain, outlier channels 7 and 300 (x20)
    and all-zero rows where local_index is 0 or 100."""
    g = rng_gain.lognormal(0.0, 0.5, size=n_rows).astype(np.float32)
    z = rng_lat.standard_normal((n_rows, dim), dtype=np.float32)
    x = z * g[:, None]
    if dim > 300:
        x[:, 7] *= 20.0
        x[:, 300] *= 20.0
    elif dim > 7:
        x[:, 7] *= 20.0
    zero = (local_index == 0) | (local_index == 100)
    x[zero] = 0.0
    return x, zero


class DecodeWorkload:
    """One decode batch: S sequences with contiguous rows (offsets), H heads."""

    def __init__(self, name, seed, lengths, n_heads, qmode, sign_seed=None):
        self.name = name
        self.seed = seed
        self.qmode = qmode
        st = streams(seed)
        self.lengths = np.asarray(lengths, np.int64)
        self.n_seqs = len(self.lengths)
        self.n_heads = n_heads
        self.offsets = np.zeros(self.n_seqs + 1, np.int64)
        self.offsets[1:] = np.cumsum(self.lengths)
        self.total_rows = int(self.offsets[-1])
        local = np.concatenate([np.arange(L, dtype=np.int64) for L in self.lengths]) if self.total_rows else \
            np.zeros(0, np.int64)
        self.latent, zero = latent_rows(st[S_GAIN], st[S_LATENT], self.total_rows, local)
        rope = st[S_ROPE].standard_normal((self.total_rows, DIM_ROPE), dtype=np.float32)
        rope[zero] = 0.0
        self.k_rope = to_bf16_bits(rope)
        inv = np.float32(1.0 / math.sqrt(DIM_LAT + DIM_ROPE))
        self.q_lat = st[S_QLAT].standard_normal((self.n_seqs, n_heads, DIM_LAT), dtype=np.float32) * inv
        self.q_rope = st[S_QROPE].standard_normal((self.n_seqs, n_heads, DIM_ROPE), dtype=np.float32) * inv
        ss = streams(sign_seed)[S_SIGNS] if sign_seed is not None else st[S_SIGNS]
        self.sign_mask = ss.integers(0, 256, size=DIM_LAT // 8, dtype=np.uint8)
        self.sm_scale = SM_SCALE


class SparseDecodeWorkload:
    """DSA-style sparse decode: a cache of T rows (the recipe above, local rows 0
    and 100 zero) and len(ks) query rows (sequences), query s attending over ks[s]
    cache rows drawn uniformly without replacement and listed in ascending
    order (the index lists come from the page-permutation substream)."""

    def __init__(self, name, seed, T, ks, n_heads, qmode=1, sign_seed=None):
        self.name = name
        self.seed = seed
        self.qmode = qmode
        st = streams(seed)
        self.cache_rows = int(T)
        self.latent, zero = latent_rows(st[S_GAIN], st[S_LATENT], T, np.arange(T, dtype=np.int64))
        rope = st[S_ROPE].standard_normal((T, DIM_ROPE), dtype=np.float32)
        rope[zero] = 0.0
        self.k_rope = to_bf16_bits(rope)
        self.ks = np.asarray(ks, np.int64)
        self.n_seqs = len(self.ks)
        self.n_heads = n_heads
        inv = np.float32(1.0 / math.sqrt(DIM_LAT + DIM_ROPE))
        self.q_lat = st[S_QLAT].standard_normal((self.n_seqs, n_heads, DIM_LAT), dtype=np.float32) * inv
        self.q_rope = st[S_QROPE].standard_normal((self.n_seqs, n_heads, DIM_ROPE), dtype=np.float32) * inv
        rng = st[S_PERM]
        self.row_index = np.concatenate(
            [np.sort(rng.choice(T, size=int(k), replace=False)) for k in self.ks]).astype(np.int64)
        self.offsets = np.zeros(self.n_seqs + 1, np.int64)
        self.offsets[1:] = np.cumsum(self.ks)
        self.total_rows = int(self.offsets[-1])
        ss = streams(sign_seed)[S_SIGNS] if sign_seed is not None else st[S_SIGNS]
        self.sign_mask = ss.integers(0, 256, size=DIM_LAT // 8, dtype=np.uint8)
        self.sm_scale = SM_SCALE


def dsa_sparse_decode(T=32768, n_q=16, k=2048, qmode=1):
    """Sparse decode over a T-row cache: n_q queries, each over k selected rows
    (top-k style), 128 heads (seed 1005)."""
    return SparseDecodeWorkload(f"dsa-sparse-decode-T{T}-q{n_q}-k{k}-H128", 1005, T, [k] * n_q, 128, qmode=qmode,
                                sign_seed=1002 if qmode == 2 else None)


def tiny_fp8_decode():
    """Tiny MLA decode, fp8: 1 sequence, T = 256, 16 heads (seed 1000)."""
    return DecodeWorkload("tiny-fp8-T256-H16", 1000, [256], 16, qmode=1)


def kv8_decode(T=32768):
    """KV8 absorbed-MLA decode: batch 1, 128 heads, T = 32768 (seed 1001)."""
    return DecodeWorkload(f"kv8-mla-decode-T{T}-H128", 1001, [T], 128, qmode=1)


def tq4_decode(T=32768):
    """TQ4 decode, the same latents as the KV8 decode (seed 1001), signs from seed 1002."""
    return DecodeWorkload(f"tq4-mla-decode-T{T}-H128", 1001, [T], 128, qmode=2, sign_seed=1002)


def tq_decode(bits, T=32768):
    """The rotated codec's decode at 3, 4 or 6 bits (qmode 3, 2, 4): the TQ4
    workload's latents and signs (seeds 1001 and 1002)."""
    qmode = {3: 3, 4: 2, 6: 4}[bits]
    return DecodeWorkload(f"tq{bits}-mla-decode-T{T}-H128", 1001, [T], 128, qmode=qmode, sign_seed=1002)


def tq4_encode_rows(n=8192, dim=DIM_LAT):
    """The 8192 new rows of the TQ4 encode-throughput pass (seed 1002)."""
    st = streams(1002)
    x, _ = latent_rows(st[S_GAIN], st[S_NEW], n, np.arange(1, n + 1, dtype=np.int64), dim)
    return x


def ragged_lengths(scale=1):
    st = streams(1003)
    L = st[S_LENGTHS].integers(1024, 16384 + 1, size=32).astype(np.int64)
    L = np.concatenate([L, [131072]])
    if scale != 1:
        L = np.maximum(1, L // scale)
    return L


def ragged_kv8_decode(scale=1):
    """Ragged long-context KV8 decode: 32 sequences, T ~ U[1024, 16384], plus one
    sequence of 131072 (last); 128 heads (seed 1003).  scale > 1 shrinks every
    length by that factor (parity-test sizes)."""
    return DecodeWorkload(f"ragged-kv8-33seq{'' if scale == 1 else f'-div{scale}'}", 1003,
                          ragged_lengths(scale), 128, qmode=1)


def fp8_rows_for_encode(n, seed=1001, dim=DIM_LAT):
    st = streams(seed)
    x, _ = latent_rows(st[S_GAIN], st[S_LATENT], n, np.arange(n, dtype=np.int64), dim)
    return x


# ---- q4_0 paged tier --------------------------------------------------------

Q4_HEAD_DIM = 256
Q4_KV_HEADS = 8
Q4_PAGE = 64
Q4_ROW_BYTES = 144
Q4_GROUP = 4                 # query heads per KV head in the fused q4_0 decode
Q4_SM_SCALE = 1.0 / 16.0     # 1 / sqrt(head_dim)


class Q4Workload:
    """Paged q4_0 pools: prefill lengths L_s (56 mod 64), then a 17-token append
    starting at pos0 = L_s, which crosses a page boundary, then a gather."""

    def __init__(self, seed=1004, n_seqs=16, lmin=512, lmax=8192, append=17, scale=1):
        st = streams(seed)
        L = st[S_LENGTHS].integers(lmin, lmax + 1, size=n_seqs).astype(np.int64)
        if scale != 1:
            L = np.maximum(64, L // scale)
        L = (L // 64) * 64 - 8  # snapped down to 56 mod 64
        L = np.maximum(L, 56)
        self.prefill_len = L
        self.append_len = append
        self.n_seqs = n_seqs
        final = L + append
        pages_per = (final + Q4_PAGE - 1) // Q4_PAGE
        self.max_pages = int(pages_per.max())
        n_pages = int(pages_per.sum())
        perm = st[S_PERM].permutation(n_pages).astype(np.int32)
        self.table = np.full((n_seqs, self.max_pages), -1, np.int32)
        k = 0
        for s in range(n_seqs):
            for p in range(int(pages_per[s])):
                self.table[s, p] = perm[k]
                k += 1
        self.n_cells = n_pages * Q4_PAGE
        self.prefill_off = np.zeros(n_seqs + 1, np.int64)
        self.prefill_off[1:] = np.cumsum(L)
        self.append_off = np.arange(n_seqs + 1, dtype=np.int64) * append
        self.final_off = np.zeros(n_seqs + 1, np.int64)
        self.final_off[1:] = np.cumsum(final)
        rng = st[S_NEW]
        self.k_prefill = self._rows(rng, L, 0)
        self.v_prefill = self._rows(rng, L, 0)
        self.k_append = self._rows(rng, np.full(n_seqs, append), L)
        self.v_append = self._rows(rng, np.full(n_seqs, append), L)
        self.pos0_prefill = np.zeros(n_seqs, np.int32)
        self.pos0_append = L.astype(np.int32)

    @staticmethod
    def _rows(rng, counts, start):
        total = int(np.sum(counts))
        x = rng.standard_normal((total, Q4_KV_HEADS, Q4_HEAD_DIM), dtype=np.float32)
        tok = np.concatenate([np.arange(int(c), dtype=np.int64) + (int(start[i]) if np.ndim(start) else start)
                              for i, c in enumerate(counts)]) if total else np.zeros(0, np.int64)
        amp = np.array([1e-3, 1.0, 40.0], np.float32)
        cls = (tok[:, None] + np.arange(Q4_KV_HEADS)[None, :]) % 3
        x *= amp[cls][:, :, None]
        x[tok % 97 == 0] = 0.0
        return x

    def empty_pools(self):
        return (np.zeros((self.n_cells, Q4_KV_HEADS, Q4_ROW_BYTES), np.uint8),
                np.zeros((self.n_cells, Q4_KV_HEADS, Q4_ROW_BYTES), np.uint8))


def q4_tie_fixtures():
    """Rotated-domain fixtures for the q4_0 block rule (used with the no-rotate
    flag): {v, -v, ...}; one +v among -v; all equal; all zero; amplitude classes."""
    v = np.float32(0.75)
    blocks = []
    blocks.append(np.array([v if j % 2 == 0 else -v for j in range(32)], np.float32))
    b = np.full(32, -v, np.float32)
    b[13] = v
    blocks.append(b)
    blocks.append(np.full(32, v, np.float32))
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, -v, np.float32))
    rng = np.random.Generator(np.random.PCG64(4242))
    for a in (1e-3, 1.0, 40.0):
        blocks.append((rng.standard_normal(32) * a).astype(np.float32))
    return np.stack(blocks)


def q4_queries(seed, n_seqs, n_q_heads=Q4_KV_HEADS * Q4_GROUP, dim=Q4_HEAD_DIM):
    """Unrotated decode queries for the fused q4_0 attention, ~ N(0, 1) / 16."""
    rng = streams(seed)[S_QLAT]
    return (rng.standard_normal((n_seqs, n_q_heads, dim), dtype=np.float32) / np.float32(16.0)).astype(np.float32)
