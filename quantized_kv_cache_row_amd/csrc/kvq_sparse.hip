// kvq_sparse.hip -- sparse (DSA-style) decode: the row gather by absolute
// index, and the sparse decode call ([KV8] commit list item 2, the DSA-aware
// gather; the rebase note on the DSA gather).  On the fp8 matrix-core path the
// split kernel reads a query's selected rows in place through the index list;
// the other paths gather them into the workspace and run the dense decode
// kernels over the copy.
#include "kvq_internal.h"

namespace kvq {

// ---- sparse decode: the row gather ------------------------------------------------
// One wave per gathered row: lanes 0 .. cb/16 - 1 copy the code bytes, the next
// 8 lanes the rope key, the one after the row scale; 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_gather_rows(const uint8_t* __restrict__ codes,
                                                     const float* __restrict__ row_scale,
                                                     const uint16_t* __restrict__ k_rope, int64_t cache_rows,
                                                     const int64_t* __restrict__ row_index, int64_t n_index, int cb,
                                                     uint8_t* __restrict__ codes_out, float* __restrict__ scale_out,
                                                     uint16_t* __restrict__ rope_out) {
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // output row (wave-uniform)
    const int lane = threadIdx.x & 63;
    if (i >= n_index) return;
    const int64_t r = min(max(row_index[i], (int64_t)0), cache_rows - 1);  // clamped: never outside the cache
    const int nc = cb / 16;
    if (lane < nc) {
        *reinterpret_cast<uint4*>(codes_out + i * cb + 16 * lane) =
            *reinterpret_cast<const uint4*>(codes + r * cb + 16 * lane);
    } else if (lane < nc + 8) {
        const int k = lane - nc;
        *reinterpret_cast<uint4*>(rope_out + i * 64 + 8 * k) = *reinterpret_cast<const uint4*>(k_rope + r * 64 + 8 * k);
    } else if (lane == nc + 8) {
        scale_out[i] = row_scale[r];
    }
}

hipError_t launch_gather_rows(int code_bytes, const uint8_t* codes, const float* row_scale, const uint16_t* k_rope,
                              int64_t cache_rows, const int64_t* row_index, int64_t n_index, uint8_t* codes_out,
                              float* scale_out, uint16_t* rope_out, hipStream_t st) {
    if (n_index == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)((n_index + 3) / 4)), dim3(256), 0, st, codes, row_scale, k_rope,
                       cache_rows, row_index, n_index, code_bytes, codes_out, scale_out, rope_out);
    return hipGetLastError();
}

namespace {
// workspace of the sparse call: the gathered codes, scales and rope keys
// (each piece 256-byte aligned), then the dense call's workspace
int64_t sparse_compact_bytes(const kvq_attn_args& a) {
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    const int64_t n = a.total_rows, cb = code_bytes_512(a.qmode);
    return align(n * cb) + align(n * 4) + align(n * 128);
}
}  // namespace

// the fp8 matrix-core path reads the selected rows in place: no compact copy
static bool sparse_in_place(const kvq_attn_args& a) { return a.qmode == KVQ_QMODE_FP8 && a.precision == KVQ_PREC_MFMA; }

int64_t attn_sparse_workspace_bytes(const kvq_attn_args& a) {
    return (sparse_in_place(a) ? 0 : sparse_compact_bytes(a)) + attn_workspace_bytes(a);
}

hipError_t launch_decode_attn_sparse(const kvq_attn_args& a, const int64_t* row_index, int64_t cache_rows, void* ws,
                                     int64_t ws_bytes, hipStream_t st) {
    if (sparse_in_place(a)) return launch_decode_attn_indexed(a, row_index, cache_rows, ws, st);
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    const int64_t n = a.total_rows;
    const int cb = code_bytes_512(a.qmode);
    char* base = (char*)ws;
    uint8_t* codes_c = (uint8_t*)base;
    float* scale_c = (float*)(base + align(n * cb));
    uint16_t* rope_c = (uint16_t*)(base + align(n * cb) + align(n * 4));
    const int64_t compact = sparse_compact_bytes(a);
    if (n > 0) {
        const hipError_t e = launch_gather_rows(cb, a.codes, a.row_scale, a.k_rope, cache_rows, row_index, n, codes_c,
                                                scale_c, rope_c, st);
        if (e != hipSuccess) return e;
    }
    kvq_attn_args b = a;
    b.codes = codes_c;
    b.row_scale = scale_c;
    b.k_rope = rope_c;
    return launch_decode_attn(b, base + compact, ws_bytes - compact, st);
}

}  // namespace kvq
