"""kvq_decode_attn_noalloc (static per-GPU scratch, no allocation) against
kvq_decode_attn (caller's workspace) through the C ABI: the same kernels on
the same inputs, so the outputs must be identical.  Two calls in a row, the
second on a smaller input, then a TQ4 call, then an input too large for the
scratch (refused before anything is enqueued)."""
import sys

import numpy as np
import pytest
import torch

from quantized_kv_cache_row_amd import kvq, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def _args(w, precision=kvq.KVQ_PREC_MFMA):
    x = _t(w.latent.astype(np.float32))
    if w.qmode == 1:
        codes = torch.empty((w.total_rows, 512), dtype=torch.uint8, device=DEV)
        scales = torch.empty(w.total_rows, dtype=torch.float32, device=DEV)
        kvq.kvq_encode_fp8(x, codes, scales)
    else:
        codes = torch.empty((w.total_rows, 256), dtype=torch.uint8, device=DEV)
        scales = torch.empty(w.total_rows, dtype=torch.float32, device=DEV)
        kvq.kvq_encode_tq4(x, _t(w.sign_mask), codes, scales)
    outs = []
    for _ in range(2):
        out = torch.full(w.q_lat.shape, float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full(w.q_lat.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        outs.append(kvq.attn_args(w.qmode, precision, _t(w.offsets), w.total_rows, codes, scales, _t(w.k_rope),
                                  _t(w.q_lat), _t(w.q_rope), w.sm_scale, out, lse,
                                  sign_mask=_t(w.sign_mask) if w.qmode == 2 else None))
    return outs


def _compare(w, label, precision=kvq.KVQ_PREC_MFMA):
    a_ref, a_na = _args(w, precision)
    need = kvq.kvq_decode_attn_workspace_bytes(a_ref)
    assert need <= kvq.KVQ_NOALLOC_SCRATCH_BYTES, (label, need)
    kvq.kvq_decode_attn(a_ref, kvq.alloc_workspace(a_ref))
    kvq.kvq_decode_attn_noalloc(a_na)
    torch.cuda.synchronize()
    o_ref, l_ref = a_ref._keep[7].cpu().numpy(), a_ref._keep[8].cpu().numpy()
    o_na, l_na = a_na._keep[7].cpu().numpy(), a_na._keep[8].cpu().numpy()
    _say(f"  {label}: workspace {need} B, max|diff| {np.max(np.abs(o_na - o_ref)):.3e}")
    assert np.all(np.isfinite(o_ref))
    np.testing.assert_array_equal(o_na, o_ref)
    np.testing.assert_array_equal(l_na, l_ref)


def test_noalloc_matches_workspace_entry_point():
    _say("noalloc: kv8_decode T=32768 H=128, then tiny_fp8_decode T=256 H=16, then TQ4 and ragged edges")
    _compare(workloads.kv8_decode(), "kv8_decode")
    _compare(workloads.tiny_fp8_decode(), "tiny_fp8_decode (second, smaller call)")
    _compare(workloads.tq4_decode(T=5000), "tq4_decode T=5000")
    w = workloads.DecodeWorkload("edges", 77, [1, 0, 33, 100, 257, 5], 20, qmode=1)
    _compare(w, "ragged edges", kvq.KVQ_PREC_MFMA)
    _compare(w, "ragged edges fp32", kvq.KVQ_PREC_FP32)


def test_noalloc_refuses_more_than_its_scratch():
    _say("noalloc: too large")
    w = workloads.tiny_fp8_decode()
    a, _ = _args(w)
    a.total_rows, a.split_rows = 1 << 22, 1024  # host copy only: the size check runs before anything is enqueued
    assert kvq.kvq_decode_attn_workspace_bytes(a) > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    a._keep = (None,) + a._keep[1:]
    with pytest.raises(kvq.KvqError) as e:
        kvq.lib()  # the status is the point, not the binding's row check
        kvq._check("kvq_decode_attn_noalloc", kvq.lib().kvq_decode_attn_noalloc(
            __import__("ctypes").byref(a), kvq._stream(None)))
    assert e.value.status == kvq.KVQ_ERR_TOO_LARGE
