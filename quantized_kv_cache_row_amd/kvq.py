"""ctypes binding of libkvq.so (include/kvq.h), same names as the C entry points.

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no CPU or PyTorch fallback -- a missing library is an error.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_ABI_VERSION = 1
KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_LAUNCH = 0, 1, 2, 3, 4
KVQ_ERR_TOO_LARGE = 5
KVQ_NOALLOC_SCRATCH_BYTES = 32 << 20
KVQ_QMODE_FP8, KVQ_QMODE_TQ4, KVQ_QMODE_TQ3, KVQ_QMODE_TQ6 = 1, 2, 3, 4
TQ_QMODE_BITS = {KVQ_QMODE_TQ3: 3, KVQ_QMODE_TQ4: 4, KVQ_QMODE_TQ6: 6}
TQ_BITS_QMODE = {b: q for q, b in TQ_QMODE_BITS.items()}
KVQ_PREC_MFMA, KVQ_PREC_FP32 = 0, 1
KVQ_Q4_NO_ROTATE = 1
KVQ_STAGE_PREP, KVQ_STAGE_SPLITS, KVQ_STAGE_MERGE = 0, 1, 2
KVQ_CVT_F32_TO_E4M3, KVQ_CVT_E4M3_TO_BF16, KVQ_CVT_F32_TO_F16, KVQ_CVT_F32_TO_BF16, KVQ_CVT_E4M3_TO_F16 = 1, 2, 3, 4, 5


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: status {status} ({kvq_status_string(status)})")
        self.status = status


class KvqAttnArgs(ctypes.Structure):
    _fields_ = [
        ("qmode", ctypes.c_int32), ("precision", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
        ("n_heads", ctypes.c_int32), ("dim_lat", ctypes.c_int32), ("dim_rope", ctypes.c_int32),
        ("split_rows", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("total_rows", ctypes.c_int64),
        ("seq_offsets", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
        ("k_rope", ctypes.c_void_p), ("sign_mask", ctypes.c_void_p), ("q_lat", ctypes.c_void_p),
        ("q_rope", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float), ("reserved1", ctypes.c_int32),
    ]


class KvqQ4Cache(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("n_cells", ctypes.c_int64), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
    ]


class KvqQ4AttnArgs(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("split_rows", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("total_rows", ctypes.c_int64), ("len_off", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float), ("reserved1", ctypes.c_int32),
    ]


_lib = None


def lib():
    """Loads libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvq.so not found at {LIB_PATH}: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        sig = {
            "kvq_abi_version": ([], i32),
            "kvq_status_string": ([i32], ctypes.c_char_p),
            "kvq_row_bytes": ([i32, i32], i64),
            "kvq_tq4_codebook": ([vp, vp], i32),
            "kvq_tq_codebook": ([i32, vp, vp], i32),
            "kvq_encode_fp8": ([vp, i64, i32, vp, vp, vp], i32),
            "kvq_encode_tq4": ([vp, i64, i32, vp, vp, vp, vp], i32),
            "kvq_encode_tq": ([i32, vp, i64, i32, vp, vp, vp, vp], i32),
            "kvq_append_q4_0": ([ctypes.POINTER(KvqQ4Cache), i32, vp, vp, i64, vp, vp, u32, vp], i32),
            "kvq_gather_q4_0": ([ctypes.POINTER(KvqQ4Cache), i32, vp, i64, vp, vp, vp], i32),
            "kvq_decode_attn_workspace_bytes": ([ctypes.POINTER(KvqAttnArgs)], i64),
            "kvq_decode_attn": ([ctypes.POINTER(KvqAttnArgs), vp, i64, vp], i32),
            "kvq_decode_attn_stage": ([ctypes.POINTER(KvqAttnArgs), i32, vp, i64, vp], i32),
            "kvq_decode_attn_noalloc": ([ctypes.POINTER(KvqAttnArgs), vp], i32),
            "kvq_decode_attn_append": ([ctypes.POINTER(KvqAttnArgs), vp, i64, vp, vp, vp, i64, vp], i32),
            "kvq_convert": ([i32, vp, i64, vp, vp], i32),
            "kvq_gather_rows": ([i32, vp, vp, vp, i64, vp, i64, vp, vp, vp, vp], i32),
            "kvq_decode_attn_sparse_workspace_bytes": ([ctypes.POINTER(KvqAttnArgs)], i64),
            "kvq_decode_attn_sparse": ([ctypes.POINTER(KvqAttnArgs), vp, i64, vp, i64, vp], i32),
            "kvq_struct_layout": ([i32, ctypes.POINTER(ctypes.c_int64), i32], i32),
            "kvq_decode_attn_q4_0_workspace_bytes": ([ctypes.POINTER(KvqQ4Cache), ctypes.POINTER(KvqQ4AttnArgs)],
                                                     i64),
            "kvq_decode_attn_q4_0": ([ctypes.POINTER(KvqQ4Cache), ctypes.POINTER(KvqQ4AttnArgs), vp, i64, vp], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return ["kvq_abi_version", "kvq_status_string", "kvq_row_bytes", "kvq_tq4_codebook", "kvq_encode_fp8",
            "kvq_encode_tq4", "kvq_append_q4_0", "kvq_gather_q4_0", "kvq_decode_attn_workspace_bytes",
            "kvq_decode_attn", "kvq_decode_attn_stage", "kvq_gather_rows", "kvq_decode_attn_sparse_workspace_bytes",
            "kvq_decode_attn_sparse", "kvq_convert", "kvq_struct_layout", "kvq_decode_attn_q4_0_workspace_bytes",
            "kvq_decode_attn_q4_0", "kvq_decode_attn_noalloc", "kvq_tq_codebook", "kvq_encode_tq",
            "kvq_decode_attn_append"]


# ---- host-only entry points -----------------------------------------------------

def kvq_abi_version():
    return lib().kvq_abi_version()


def kvq_status_string(status):
    return lib().kvq_status_string(int(status)).decode()


def kvq_row_bytes(qmode, dim):
    return lib().kvq_row_bytes(int(qmode), int(dim))


def kvq_tq4_codebook():
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check("kvq_tq4_codebook", lib().kvq_tq4_codebook(ctypes.cast(lv, ctypes.c_void_p),
                                                      ctypes.cast(th, ctypes.c_void_p)))
    return list(lv), list(th)


def kvq_tq_codebook(bits):
    """Levels [2^bits] and thresholds [2^bits - 1] of the rotated codec's tier."""
    n = 1 << int(bits) if 0 < int(bits) <= 8 else 1
    lv = (ctypes.c_float * n)()
    th = (ctypes.c_float * n)()
    _check("kvq_tq_codebook", lib().kvq_tq_codebook(int(bits), ctypes.cast(lv, ctypes.c_void_p),
                                                    ctypes.cast(th, ctypes.c_void_p)))
    return list(lv), list(th)[:n - 1]


def code_bytes(qmode, dim=512):
    """Code bytes per row of a mode (fp8: dim; rotated codec: dim * bits / 8)."""
    return dim if qmode == KVQ_QMODE_FP8 else dim * TQ_QMODE_BITS.get(qmode, 4) // 8


def kvq_struct_layout(which):
    buf = (ctypes.c_int64 * 32)()
    n = lib().kvq_struct_layout(int(which), buf, 32)
    if n < 0:
        raise ValueError(which)
    return list(buf[:n])


def binding_layout(which):
    S = (KvqAttnArgs, KvqQ4Cache, KvqQ4AttnArgs)[which]
    return [ctypes.sizeof(S)] + [getattr(S, f).offset for f, _ in S._fields_]


# ---- helpers -----------------------------------------------------------------------

def _check(fn, status):
    if status != KVQ_OK:
        raise KvqError(fn, status)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name):
    """Raises ValueError unless tensor t has this shape (None entries match any size)."""
    if t is None:
        return
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError(f"{name}: shape {got}, expected {tuple('*' if w is None else w for w in shape)}")


# ---- device entry points --------------------------------------------------------

def kvq_encode_fp8(x, codes, scales, stream=None):
    """x fp32 [n][dim] -> codes u8 [n][dim], scales fp32 [n]."""
    n, dim = x.shape
    _check("kvq_encode_fp8", lib().kvq_encode_fp8(_ptr(x, torch.float32, "x"), n, dim,
                                                  _ptr(codes, torch.uint8, "codes"),
                                                  _ptr(scales, torch.float32, "scales"), _stream(stream)))


def kvq_encode_tq4(x, sign_mask, codes, radii, stream=None):
    """x fp32 [n][dim], sign_mask u8 [dim/8] -> codes u8 [n][dim/2], radii fp32 [n]."""
    n, dim = x.shape
    _check("kvq_encode_tq4", lib().kvq_encode_tq4(_ptr(x, torch.float32, "x"), n, dim,
                                                  _ptr(sign_mask, torch.uint8, "sign_mask"),
                                                  _ptr(codes, torch.uint8, "codes"),
                                                  _ptr(radii, torch.float32, "radii"), _stream(stream)))


def kvq_encode_tq(bits, x, sign_mask, codes, radii, stream=None):
    """x fp32 [n][dim], sign_mask u8 [dim/8] -> codes u8 [n][dim*bits/8], radii fp32 [n]."""
    n, dim = x.shape
    _shape(codes, (n, dim * int(bits) // 8), "codes")
    _shape(radii, (n,), "radii")
    _check("kvq_encode_tq", lib().kvq_encode_tq(int(bits), _ptr(x, torch.float32, "x"), n, dim,
                                                _ptr(sign_mask, torch.uint8, "sign_mask"),
                                                _ptr(codes, torch.uint8, "codes"),
                                                _ptr(radii, torch.float32, "radii"), _stream(stream)))


def q4_cache(k_pool, v_pool, block_table, page_size, head_dim=256):
    """The cache descriptor; it keeps the tensors it points to alive."""
    _shape(k_pool, (None, None, 144), "k_pool")
    n_cells, n_kv, rb = k_pool.shape
    _shape(v_pool, (n_cells, n_kv, 144), "v_pool")
    _shape(block_table, (None, None), "block_table")
    c = KvqQ4Cache(_ptr(k_pool, torch.uint8, "k_pool"), _ptr(v_pool, torch.uint8, "v_pool"),
                   _ptr(block_table, torch.int32, "block_table"), n_cells, block_table.shape[1],
                   page_size, n_kv, head_dim)
    c._keep = (k_pool, v_pool, block_table)
    return c


def kvq_append_q4_0(cache, pos0, src_off, total_new, k_src, v_src, flags=0, stream=None):
    n_seqs = pos0.shape[0]
    _check("kvq_append_q4_0", lib().kvq_append_q4_0(ctypes.byref(cache), n_seqs, _ptr(pos0, torch.int32, "pos0"),
                                                    _ptr(src_off, torch.int64, "src_off"), int(total_new),
                                                    _ptr(k_src, torch.float32, "k_src"),
                                                    _ptr(v_src, torch.float32, "v_src"), int(flags),
                                                    _stream(stream)))


def kvq_gather_q4_0(cache, dst_off, total_rows, k_dst, v_dst, stream=None):
    n_seqs = dst_off.shape[0] - 1
    _check("kvq_gather_q4_0", lib().kvq_gather_q4_0(ctypes.byref(cache), n_seqs,
                                                    _ptr(dst_off, torch.int64, "dst_off"), int(total_rows),
                                                    _ptr(k_dst, (torch.uint16, torch.int16, torch.float16), "k_dst"),
                                                    _ptr(v_dst, (torch.uint16, torch.int16, torch.float16), "v_dst"),
                                                    _stream(stream)))


def attn_args(qmode, precision, seq_offsets, total_rows, codes, row_scale, k_rope, q_lat, q_rope, sm_scale, out,
              lse=None, sign_mask=None, split_rows=0):
    """The argument struct; it keeps the tensors it points to alive."""
    _shape(q_lat, (None, None, None), "q_lat")
    n_seqs, n_heads, dim_lat = q_lat.shape
    _shape(q_rope, (n_seqs, n_heads, None), "q_rope")
    _shape(out, (n_seqs, n_heads, dim_lat), "out")
    _shape(lse, (n_seqs, n_heads), "lse")
    _shape(seq_offsets, (n_seqs + 1,), "seq_offsets")
    _shape(codes, (None, code_bytes(qmode, dim_lat)), "codes")
    rows = codes.shape[0]
    _shape(row_scale, (rows,), "row_scale")
    _shape(k_rope, (rows, q_rope.shape[2]), "k_rope")
    _shape(sign_mask, (dim_lat // 8,), "sign_mask")
    a = KvqAttnArgs(
        qmode, precision, n_seqs, n_heads, dim_lat, q_rope.shape[2], split_rows, 0, int(total_rows),
        _ptr(seq_offsets, torch.int64, "seq_offsets"), _ptr(codes, torch.uint8, "codes"),
        _ptr(row_scale, torch.float32, "row_scale"), _ptr(k_rope, (torch.uint16, torch.int16, torch.bfloat16),
                                                           "k_rope"),
        _ptr(sign_mask, torch.uint8, "sign_mask"), _ptr(q_lat, torch.float32, "q_lat"),
        _ptr(q_rope, torch.float32, "q_rope"), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), float(sm_scale), 0)
    a._keep = (seq_offsets, codes, row_scale, k_rope, sign_mask, q_lat, q_rope, out, lse)
    return a


def kvq_decode_attn_workspace_bytes(args):
    n = lib().kvq_decode_attn_workspace_bytes(ctypes.byref(args))
    if n < 0:
        raise KvqError("kvq_decode_attn_workspace_bytes", KVQ_ERR_INVALID_ARG)
    return n


def kvq_decode_attn(args, workspace, stream=None):
    """args: KvqAttnArgs (see attn_args); workspace: a device uint8 tensor of at
    least kvq_decode_attn_workspace_bytes(args) bytes."""
    _cache_rows_cover(args)
    _check("kvq_decode_attn", lib().kvq_decode_attn(ctypes.byref(args), _ptr(workspace, torch.uint8, "workspace"),
                                                    workspace.numel(), _stream(stream)))


def _cache_rows_cover(args):
    """The dense decode reads rows 0 .. total_rows - 1 of the code arrays."""
    codes = args._keep[1]
    if codes is not None and codes.shape[0] < args.total_rows:
        raise ValueError(f"codes: {codes.shape[0]} rows, fewer than total_rows = {args.total_rows}")


def kvq_decode_attn_append(args, x_new, codes_new, scale_new, workspace, stream=None):
    """Encodes x_new (fp32 [n][512]) into codes_new / scale_new, then decode attention."""
    n = x_new.shape[0]
    _shape(x_new, (n, 512), "x_new")
    _shape(codes_new, (n, code_bytes(args.qmode)), "codes_new")
    _shape(scale_new, (n,), "scale_new")
    _cache_rows_cover(args)
    _check("kvq_decode_attn_append", lib().kvq_decode_attn_append(
        ctypes.byref(args), _ptr(x_new, torch.float32, "x_new"), n, _ptr(codes_new, torch.uint8, "codes_new"),
        _ptr(scale_new, torch.float32, "scale_new"), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


def kvq_decode_attn_noalloc(args, stream=None):
    """kvq_decode_attn with the library's static per-GPU scratch as its workspace
    (no allocation; calls on one GPU must be ordered)."""
    _cache_rows_cover(args)
    _check("kvq_decode_attn_noalloc", lib().kvq_decode_attn_noalloc(ctypes.byref(args), _stream(stream)))


def kvq_decode_attn_stage(args, stage, workspace, stream=None):
    _cache_rows_cover(args)
    _check("kvq_decode_attn_stage", lib().kvq_decode_attn_stage(ctypes.byref(args), int(stage),
                                                                _ptr(workspace, torch.uint8, "workspace"),
                                                                workspace.numel(), _stream(stream)))


def kvq_gather_rows(qmode, codes, row_scale, k_rope, row_index, codes_out, scale_out, rope_out, stream=None):
    """Rows row_index of the cache (codes [rows][code_bytes(qmode)], row_scale [rows],
    k_rope [rows][64] bf16 bits) copied to row i of the outputs."""
    _shape(codes, (None, code_bytes(qmode)), "codes")
    _shape(codes_out, (row_index.numel(), code_bytes(qmode)), "codes_out")
    _check("kvq_gather_rows", lib().kvq_gather_rows(
        int(qmode), _ptr(codes, torch.uint8, "codes"), _ptr(row_scale, torch.float32, "row_scale"),
        _ptr(k_rope, (torch.uint16, torch.int16, torch.bfloat16), "k_rope"), codes.shape[0],
        _ptr(row_index, torch.int64, "row_index"), row_index.numel(), _ptr(codes_out, torch.uint8, "codes_out"),
        _ptr(scale_out, torch.float32, "scale_out"),
        _ptr(rope_out, (torch.uint16, torch.int16, torch.bfloat16), "rope_out"), _stream(stream)))


def kvq_decode_attn_sparse_workspace_bytes(args):
    n = lib().kvq_decode_attn_sparse_workspace_bytes(ctypes.byref(args))
    if n < 0:
        raise KvqError("kvq_decode_attn_sparse_workspace_bytes", KVQ_ERR_INVALID_ARG)
    return n


def kvq_decode_attn_sparse(args, row_index, cache_rows, workspace, stream=None):
    """args: KvqAttnArgs whose seq_offsets partition row_index (total_rows =
    row_index.numel()) and whose codes / row_scale / k_rope are the whole cache of
    cache_rows rows; workspace: at least kvq_decode_attn_sparse_workspace_bytes(args)."""
    _check("kvq_decode_attn_sparse", lib().kvq_decode_attn_sparse(
        ctypes.byref(args), _ptr(row_index, torch.int64, "row_index"), int(cache_rows),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def alloc_workspace_sparse(args, device="cuda"):
    n = kvq_decode_attn_sparse_workspace_bytes(args)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def kvq_convert(kind, src, dst, stream=None):
    _check("kvq_convert", lib().kvq_convert(int(kind), _ptr(src, name="src"), src.numel(), _ptr(dst, name="dst"),
                                            _stream(stream)))


def alloc_workspace(args, device="cuda"):
    n = kvq_decode_attn_workspace_bytes(args)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


# ---- fused decode attention over the q4_0 pools -------------------------------------

def q4_attn_args(len_off, total_rows, q, out, lse=None, sm_scale=1.0 / 16.0, split_rows=0):
    """Arguments of kvq_decode_attn_q4_0; q / out fp32 [n_seqs][n_q_heads][256]."""
    _shape(q, (None, None, 256), "q")
    n_seqs, n_q, _ = q.shape
    _shape(out, (n_seqs, n_q, 256), "out")
    _shape(lse, (n_seqs, n_q), "lse")
    _shape(len_off, (n_seqs + 1,), "len_off")
    a = KvqQ4AttnArgs(n_seqs, n_q, int(split_rows), 0, int(total_rows), _ptr(len_off, torch.int64, "len_off"),
                      _ptr(q, torch.float32, "q"), _ptr(out, torch.float32, "out"),
                      _ptr(lse, torch.float32, "lse") if lse is not None else None, float(sm_scale), 0)
    a._keep = (len_off, q, out, lse)
    return a


def kvq_decode_attn_q4_0_workspace_bytes(cache, args):
    n = lib().kvq_decode_attn_q4_0_workspace_bytes(ctypes.byref(cache), ctypes.byref(args))
    if n < 0:
        raise KvqError("kvq_decode_attn_q4_0_workspace_bytes", KVQ_ERR_INVALID_ARG)
    return n


def alloc_workspace_q4(cache, args, device="cuda"):
    n = kvq_decode_attn_q4_0_workspace_bytes(cache, args)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def kvq_decode_attn_q4_0(cache, args, workspace, stream=None):
    _check("kvq_decode_attn_q4_0", lib().kvq_decode_attn_q4_0(
        ctypes.byref(cache), ctypes.byref(args), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))
