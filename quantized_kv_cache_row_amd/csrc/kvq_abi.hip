// kvq_abi.hip -- the C ABI of libkvq.so (declared in include/kvq.h): argument
// validation, then launches on the caller's stream.  Nothing here allocates,
// synchronizes or falls back to another path.
#include <stddef.h>
#include <string.h>

#include <mutex>

#include "kvq_internal.h"

// Layouts the bindings mirror; a same-size reorder would otherwise go unnoticed.
static_assert(sizeof(kvq_attn_args) == 120, "kvq_attn_args size");
static_assert(offsetof(kvq_attn_args, qmode) == 0, "layout");
static_assert(offsetof(kvq_attn_args, precision) == 4, "layout");
static_assert(offsetof(kvq_attn_args, n_seqs) == 8, "layout");
static_assert(offsetof(kvq_attn_args, n_heads) == 12, "layout");
static_assert(offsetof(kvq_attn_args, dim_lat) == 16, "layout");
static_assert(offsetof(kvq_attn_args, dim_rope) == 20, "layout");
static_assert(offsetof(kvq_attn_args, split_rows) == 24, "layout");
static_assert(offsetof(kvq_attn_args, reserved0) == 28, "layout");
static_assert(offsetof(kvq_attn_args, total_rows) == 32, "layout");
static_assert(offsetof(kvq_attn_args, seq_offsets) == 40, "layout");
static_assert(offsetof(kvq_attn_args, codes) == 48, "layout");
static_assert(offsetof(kvq_attn_args, row_scale) == 56, "layout");
static_assert(offsetof(kvq_attn_args, k_rope) == 64, "layout");
static_assert(offsetof(kvq_attn_args, sign_mask) == 72, "layout");
static_assert(offsetof(kvq_attn_args, q_lat) == 80, "layout");
static_assert(offsetof(kvq_attn_args, q_rope) == 88, "layout");
static_assert(offsetof(kvq_attn_args, out) == 96, "layout");
static_assert(offsetof(kvq_attn_args, lse) == 104, "layout");
static_assert(offsetof(kvq_attn_args, sm_scale) == 112, "layout");
static_assert(offsetof(kvq_attn_args, reserved1) == 116, "layout");
static_assert(sizeof(kvq_q4_cache) == 48, "kvq_q4_cache size");
static_assert(offsetof(kvq_q4_cache, k_pool) == 0, "layout");
static_assert(offsetof(kvq_q4_cache, v_pool) == 8, "layout");
static_assert(offsetof(kvq_q4_cache, block_table) == 16, "layout");
static_assert(offsetof(kvq_q4_cache, n_cells) == 24, "layout");
static_assert(offsetof(kvq_q4_cache, max_pages) == 32, "layout");
static_assert(offsetof(kvq_q4_cache, page_size) == 36, "layout");
static_assert(offsetof(kvq_q4_cache, n_kv_heads) == 40, "layout");
static_assert(offsetof(kvq_q4_cache, head_dim) == 44, "layout");

namespace {

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }
bool pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }
hipStream_t as_stream(void* s) { return (hipStream_t)s; }
int launch_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

int check_attn(const kvq_attn_args* a) {
    if (!a) return KVQ_ERR_INVALID_ARG;
    if (a->qmode != KVQ_QMODE_FP8 && !kvq::qmode_rotated(a->qmode)) return KVQ_ERR_UNSUPPORTED;
    if (a->precision != KVQ_PREC_MFMA && a->precision != KVQ_PREC_FP32) return KVQ_ERR_UNSUPPORTED;
    if (a->dim_lat != 512 || a->dim_rope != 64) return KVQ_ERR_UNSUPPORTED;
    if (a->n_seqs < 1 || a->n_heads < 1 || a->total_rows < 0 || a->split_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (a->n_heads > 256) return KVQ_ERR_UNSUPPORTED;
    if (a->reserved0 != 0 || a->reserved1 != 0) return KVQ_ERR_INVALID_ARG;
    if (a->split_rows > 0 && a->split_rows % 32 != 0) return KVQ_ERR_INVALID_ARG;
    if (!a->seq_offsets || !a->q_lat || !a->q_rope || !a->out) return KVQ_ERR_INVALID_ARG;
    if (a->total_rows > 0 && (!a->codes || !a->row_scale || !a->k_rope)) return KVQ_ERR_INVALID_ARG;
    if (kvq::qmode_rotated(a->qmode) && !a->sign_mask) return KVQ_ERR_INVALID_ARG;
    if (!aligned(a->seq_offsets, 8) || !aligned16(a->codes) || !aligned(a->row_scale, 4) || !aligned16(a->k_rope) ||
        !aligned(a->q_lat, 4) || !aligned(a->q_rope, 4) || !aligned16(a->out) || !aligned(a->lse, 4))
        return KVQ_ERR_INVALID_ARG;
    if (!(a->sm_scale == a->sm_scale) || a->sm_scale > 3.0e38f || a->sm_scale < -3.0e38f) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
}

int check_q4(const kvq_q4_cache* c) {
    if (!c || !c->k_pool || !c->v_pool || !c->block_table) return KVQ_ERR_INVALID_ARG;
    if (c->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
    if (c->page_size < 1 || c->n_kv_heads < 1 || c->max_pages < 1 || c->n_cells < 0) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(c->k_pool) || !aligned16(c->v_pool) || !aligned(c->block_table, 4)) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
}

int check_q4_attn(const kvq_q4_cache* c, const kvq_q4_attn_args* a) {
    int rc = check_q4(c);
    if (rc != KVQ_OK) return rc;
    if (!a) return KVQ_ERR_INVALID_ARG;
    if (a->n_seqs < 1 || a->n_q_heads < 1 || a->total_rows < 0 || a->split_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (a->n_q_heads % c->n_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
    const int g = a->n_q_heads / c->n_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return KVQ_ERR_UNSUPPORTED;
    if (a->reserved0 != 0 || a->reserved1 != 0) return KVQ_ERR_INVALID_ARG;
    if (a->split_rows > 0 && (a->split_rows % 256 != 0 || a->split_rows > (1 << 24))) return KVQ_ERR_INVALID_ARG;
    if (!a->len_off || !a->q || !a->out) return KVQ_ERR_INVALID_ARG;
    if (!aligned(a->len_off, 8) || !aligned16(a->q) || !aligned16(a->out) || !aligned(a->lse, 4))
        return KVQ_ERR_INVALID_ARG;
    if (!(a->sm_scale == a->sm_scale) || a->sm_scale > 3.0e38f || a->sm_scale < -3.0e38f) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
}

// ---- static scratch of kvq_decode_attn_noalloc ----------------------------------
// The workspace of the no-allocation entry point: one array per GPU the library
// runs on, held until the process ends.  Its name is only a host-side handle;
// kernels get its device address, looked up once per device with that device
// current and kept below.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of this device's scratch array (nullptr if it cannot be had).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_INVALID_ARG: return "invalid argument (null pointer, bad count or shape, misaligned buffer)";
        case KVQ_ERR_UNSUPPORTED: return "unsupported (mode, width or size not provided by this library)";
        case KVQ_ERR_WORKSPACE: return "workspace smaller than kvq_decode_attn_workspace_bytes()";
        case KVQ_ERR_LAUNCH: return "HIP launch failed";
        case KVQ_ERR_TOO_LARGE:
            return "the call needs more workspace than the static scratch of the no-allocation entry point "
                   "(KVQ_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int64_t kvq_row_bytes(int qmode, int dim) {
    if (qmode == KVQ_QMODE_FP8) return (dim >= 8 && dim <= 2048 && dim % 8 == 0) ? (int64_t)dim + 4 : -1;
    const int bits = kvq::qmode_bits(qmode);
    if (bits) return (pow2(dim) && dim >= 8 && dim <= 512) ? (int64_t)dim * bits / 8 + 4 : -1;
    return -1;
}

int kvq_tq4_codebook(float* levels, float* thresholds) {
    kvq::host_codebook(4, levels, thresholds);
    return KVQ_OK;
}

int kvq_tq_codebook(int bits, float* levels, float* thresholds) {
    return kvq::host_codebook(bits, levels, thresholds) > 0 ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

int kvq_encode_fp8(const float* x, int64_t n_rows, int dim, uint8_t* codes, float* scales, void* stream) {
    if (n_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (dim < 8 || dim % 8 != 0) return KVQ_ERR_INVALID_ARG;
    if (dim > 2048) return KVQ_ERR_UNSUPPORTED;
    if (n_rows == 0) return KVQ_OK;
    if (!x || !codes || !scales) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned(codes, 8) || !aligned(scales, 4)) return KVQ_ERR_INVALID_ARG;
    if (n_rows > ((int64_t)1 << 40) / dim) return KVQ_ERR_UNSUPPORTED;
    return launch_status(kvq::launch_encode_fp8(x, n_rows, dim, codes, scales, as_stream(stream)));
}

int kvq_encode_tq(int bits, const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask, uint8_t* codes,
                  float* radii, void* stream) {
    if (bits != 3 && bits != 4 && bits != 6) return KVQ_ERR_UNSUPPORTED;
    if (n_rows < 0 || dim <= 0) return KVQ_ERR_INVALID_ARG;
    if (!pow2(dim) || dim < 8 || dim > 512) return KVQ_ERR_UNSUPPORTED;
    if (n_rows == 0) return KVQ_OK;
    if (!x || !sign_mask || !codes || !radii) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned(codes, 4) || !aligned(radii, 4)) return KVQ_ERR_INVALID_ARG;
    if (n_rows > ((int64_t)1 << 40) / dim) return KVQ_ERR_UNSUPPORTED;
    return launch_status(kvq::launch_encode_tq(bits, x, n_rows, dim, sign_mask, codes, radii, as_stream(stream)));
}

int kvq_encode_tq4(const float* x, int64_t n_rows, int dim, const uint8_t* sign_mask, uint8_t* codes,
                   float* radii, void* stream) {
    return kvq_encode_tq(4, x, n_rows, dim, sign_mask, codes, radii, stream);
}

int kvq_append_q4_0(const kvq_q4_cache* cache, int n_seqs, const int32_t* pos0, const int64_t* src_off,
                    int64_t total_new, const float* k_src, const float* v_src, uint32_t flags, void* stream) {
    int rc = check_q4(cache);
    if (rc != KVQ_OK) return rc;
    if (n_seqs < 1 || total_new < 0 || (flags & ~KVQ_Q4_NO_ROTATE) != 0) return KVQ_ERR_INVALID_ARG;
    if (!pos0 || !src_off) return KVQ_ERR_INVALID_ARG;
    if (total_new == 0) return KVQ_OK;
    if (!k_src || !v_src || !aligned16(k_src) || !aligned16(v_src)) return KVQ_ERR_INVALID_ARG;
    if (!aligned(pos0, 4) || !aligned(src_off, 8)) return KVQ_ERR_INVALID_ARG;
    return launch_status(kvq::launch_append_q4_0(*cache, n_seqs, pos0, src_off, total_new, k_src, v_src,
                                                 (flags & KVQ_Q4_NO_ROTATE) == 0, as_stream(stream)));
}

int kvq_gather_q4_0(const kvq_q4_cache* cache, int n_seqs, const int64_t* dst_off, int64_t total_rows,
                    uint16_t* k_dst, uint16_t* v_dst, void* stream) {
    int rc = check_q4(cache);
    if (rc != KVQ_OK) return rc;
    if (n_seqs < 1 || total_rows < 0 || !dst_off) return KVQ_ERR_INVALID_ARG;
    if (total_rows == 0) return KVQ_OK;
    if (!k_dst || !v_dst || !aligned16(k_dst) || !aligned16(v_dst) || !aligned(dst_off, 8))
        return KVQ_ERR_INVALID_ARG;
    return launch_status(
        kvq::launch_gather_q4_0(*cache, n_seqs, dst_off, total_rows, k_dst, v_dst, as_stream(stream)));
}

int64_t kvq_decode_attn_q4_0_workspace_bytes(const kvq_q4_cache* cache, const kvq_q4_attn_args* a) {
    if (check_q4_attn(cache, a) != KVQ_OK) return -1;
    return kvq::q4_attn_workspace_bytes(*cache, *a);
}

int kvq_decode_attn_q4_0(const kvq_q4_cache* cache, const kvq_q4_attn_args* a, void* workspace, int64_t ws_bytes,
                         void* stream) {
    int rc = check_q4_attn(cache, a);
    if (rc != KVQ_OK) return rc;
    const int64_t need = kvq::q4_attn_workspace_bytes(*cache, *a);
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    return launch_status(kvq::launch_decode_attn_q4_0(*cache, *a, workspace, as_stream(stream)));
}

int64_t kvq_decode_attn_workspace_bytes(const kvq_attn_args* a) {
    if (check_attn(a) != KVQ_OK) return -1;
    return kvq::attn_workspace_bytes(*a);
}

int kvq_decode_attn(const kvq_attn_args* a, void* workspace, int64_t ws_bytes, void* stream) {
    int rc = check_attn(a);
    if (rc != KVQ_OK) return rc;
    const int64_t need = kvq::attn_workspace_bytes(*a);
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    return launch_status(kvq::launch_decode_attn(*a, workspace, ws_bytes, as_stream(stream)));
}

int kvq_decode_attn_append(const kvq_attn_args* a, const float* x_new, int64_t n_new, uint8_t* codes_new,
                           float* scale_new, void* workspace, int64_t ws_bytes, void* stream) {
    int rc = check_attn(a);
    if (rc != KVQ_OK) return rc;
    if (n_new < 0) return KVQ_ERR_INVALID_ARG;
    if (n_new > ((int64_t)1 << 31)) return KVQ_ERR_UNSUPPORTED;
    if (n_new > 0) {
        if (!x_new || !codes_new || !scale_new) return KVQ_ERR_INVALID_ARG;
        if (!aligned16(x_new) || !aligned(codes_new, a->qmode == KVQ_QMODE_FP8 ? 8 : 4) || !aligned(scale_new, 4))
            return KVQ_ERR_INVALID_ARG;
    }
    const int64_t need = kvq::attn_workspace_bytes(*a);
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    const kvq::NewRows nr{x_new, n_new, codes_new, scale_new};
    return launch_status(kvq::launch_decode_attn_append(*a, nr, workspace, as_stream(stream)));
}

int kvq_decode_attn_noalloc(const kvq_attn_args* a, void* stream) {
    int rc = check_attn(a);
    if (rc != KVQ_OK) return rc;
    const int64_t need = kvq::attn_workspace_bytes(*a);
    if (need > (int64_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_TOO_LARGE;
    void* ws = scratch_for_current_device();
    if (!ws) return KVQ_ERR_LAUNCH;
    return launch_status(kvq::launch_decode_attn(*a, ws, need, as_stream(stream)));
}

int kvq_decode_attn_stage(const kvq_attn_args* a, int stage, void* workspace, int64_t ws_bytes, void* stream) {
    int rc = check_attn(a);
    if (rc != KVQ_OK) return rc;
    if (stage < KVQ_STAGE_PREP || stage > KVQ_STAGE_MERGE) return KVQ_ERR_INVALID_ARG;
    const int64_t need = kvq::attn_workspace_bytes(*a);
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    return launch_status(kvq::launch_decode_attn_stage(*a, stage, workspace, as_stream(stream)));
}

int kvq_gather_rows(int qmode, const uint8_t* codes, const float* row_scale, const uint16_t* k_rope,
                    int64_t cache_rows, const int64_t* row_index, int64_t n_index, uint8_t* codes_out,
                    float* scale_out, uint16_t* rope_out, void* stream) {
    if (qmode != KVQ_QMODE_FP8 && !kvq::qmode_rotated(qmode)) return KVQ_ERR_UNSUPPORTED;
    if (n_index < 0 || cache_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (n_index == 0) return KVQ_OK;
    if (cache_rows < 1 || !codes || !row_scale || !k_rope || !row_index || !codes_out || !scale_out || !rope_out)
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(k_rope) || !aligned16(codes_out) || !aligned16(rope_out) ||
        !aligned(row_scale, 4) || !aligned(scale_out, 4) || !aligned(row_index, 8))
        return KVQ_ERR_INVALID_ARG;
    if (n_index > ((int64_t)1 << 33)) return KVQ_ERR_UNSUPPORTED;  // grid of n_index / 4 workgroups
    const int cb = kvq::code_bytes_512(qmode);
    return launch_status(kvq::launch_gather_rows(cb, codes, row_scale, k_rope, cache_rows, row_index, n_index,
                                                 codes_out, scale_out, rope_out, as_stream(stream)));
}

int64_t kvq_decode_attn_sparse_workspace_bytes(const kvq_attn_args* a) {
    if (check_attn(a) != KVQ_OK) return -1;
    if (a->total_rows > ((int64_t)1 << 33)) return -1;
    return kvq::attn_sparse_workspace_bytes(*a);
}

int kvq_decode_attn_sparse(const kvq_attn_args* a, const int64_t* row_index, int64_t cache_rows, void* workspace,
                           int64_t ws_bytes, void* stream) {
    int rc = check_attn(a);
    if (rc != KVQ_OK) return rc;
    if (a->total_rows > ((int64_t)1 << 33)) return KVQ_ERR_UNSUPPORTED;
    if (cache_rows < 0 || cache_rows > (int64_t)0xFFFFFFFF) return KVQ_ERR_INVALID_ARG;
    if (a->total_rows > 0 && (cache_rows < 1 || !row_index || !aligned(row_index, 8))) return KVQ_ERR_INVALID_ARG;
    const int64_t need = kvq::attn_sparse_workspace_bytes(*a);
    if (!workspace || ws_bytes < need) return KVQ_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return KVQ_ERR_INVALID_ARG;
    return launch_status(
        kvq::launch_decode_attn_sparse(*a, row_index, cache_rows, workspace, ws_bytes, as_stream(stream)));
}

int kvq_convert(int kind, const void* in, int64_t n, void* out, void* stream) {
    if (kind < KVQ_CVT_F32_TO_E4M3 || kind > KVQ_CVT_E4M3_TO_F16) return KVQ_ERR_UNSUPPORTED;
    if (n < 0) return KVQ_ERR_INVALID_ARG;
    if (n == 0) return KVQ_OK;
    if (!in || !out || !aligned(in, 4) || !aligned(out, 4)) return KVQ_ERR_INVALID_ARG;
    return launch_status(kvq::launch_convert(kind, in, n, out, as_stream(stream)));
}

int kvq_struct_layout(int which, int64_t* out, int n) {
    int64_t v[24];
    int k = 0;
    if (which == 0) {
        v[k++] = sizeof(kvq_attn_args);
        v[k++] = offsetof(kvq_attn_args, qmode);
        v[k++] = offsetof(kvq_attn_args, precision);
        v[k++] = offsetof(kvq_attn_args, n_seqs);
        v[k++] = offsetof(kvq_attn_args, n_heads);
        v[k++] = offsetof(kvq_attn_args, dim_lat);
        v[k++] = offsetof(kvq_attn_args, dim_rope);
        v[k++] = offsetof(kvq_attn_args, split_rows);
        v[k++] = offsetof(kvq_attn_args, reserved0);
        v[k++] = offsetof(kvq_attn_args, total_rows);
        v[k++] = offsetof(kvq_attn_args, seq_offsets);
        v[k++] = offsetof(kvq_attn_args, codes);
        v[k++] = offsetof(kvq_attn_args, row_scale);
        v[k++] = offsetof(kvq_attn_args, k_rope);
        v[k++] = offsetof(kvq_attn_args, sign_mask);
        v[k++] = offsetof(kvq_attn_args, q_lat);
        v[k++] = offsetof(kvq_attn_args, q_rope);
        v[k++] = offsetof(kvq_attn_args, out);
        v[k++] = offsetof(kvq_attn_args, lse);
        v[k++] = offsetof(kvq_attn_args, sm_scale);
        v[k++] = offsetof(kvq_attn_args, reserved1);
    } else if (which == 1) {
        v[k++] = sizeof(kvq_q4_cache);
        v[k++] = offsetof(kvq_q4_cache, k_pool);
        v[k++] = offsetof(kvq_q4_cache, v_pool);
        v[k++] = offsetof(kvq_q4_cache, block_table);
        v[k++] = offsetof(kvq_q4_cache, n_cells);
        v[k++] = offsetof(kvq_q4_cache, max_pages);
        v[k++] = offsetof(kvq_q4_cache, page_size);
        v[k++] = offsetof(kvq_q4_cache, n_kv_heads);
        v[k++] = offsetof(kvq_q4_cache, head_dim);
    } else if (which == 2) {
        v[k++] = sizeof(kvq_q4_attn_args);
        v[k++] = offsetof(kvq_q4_attn_args, n_seqs);
        v[k++] = offsetof(kvq_q4_attn_args, n_q_heads);
        v[k++] = offsetof(kvq_q4_attn_args, split_rows);
        v[k++] = offsetof(kvq_q4_attn_args, reserved0);
        v[k++] = offsetof(kvq_q4_attn_args, total_rows);
        v[k++] = offsetof(kvq_q4_attn_args, len_off);
        v[k++] = offsetof(kvq_q4_attn_args, q);
        v[k++] = offsetof(kvq_q4_attn_args, out);
        v[k++] = offsetof(kvq_q4_attn_args, lse);
        v[k++] = offsetof(kvq_q4_attn_args, sm_scale);
        v[k++] = offsetof(kvq_q4_attn_args, reserved1);
    } else {
        return -1;
    }
    const int m = k < n ? k : n;
    if (out)
        for (int i = 0; i < m; i++) out[i] = v[i];
    return m;
}

}  // extern "C"
