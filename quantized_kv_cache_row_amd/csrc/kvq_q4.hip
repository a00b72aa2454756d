// kvq_q4.hip -- q4_0 paged K/V tier with the 256-point Walsh-Hadamard rotation
// (Strata PR #2533 "metal: q4_0 KV cache on the Mac engine": the first commit
// -- FWHT-256 orthonormal x 1/16, 18-byte blocks, tie rule, fp16 scale by round
// to nearest even, int(fma(x, id, 8.5)) truncated; the QSA_KV_Q4 commit -- pools
// [cell][kv head][144] and the dequant (nibble - 8) * f32(d)).
//
// Mapping for gfx950 (wave64): 16 lanes per 256-wide head-row, 16 consecutive
// fp32 per lane (four 16-byte loads), four head-rows per wave.  FWHT stages
// h = 1..8 run in registers, h = 16..128 across lanes (lane ^ 1..8); a 32-wide
// block is a lane pair.  The 144-byte head-row is assembled in LDS and written
// with nine 16-byte stores (144 = 9 x 16, so head-rows stay 16-byte aligned).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int Q4_WAVES = 4;
constexpr int Q4_ROWS_PER_BLOCK = Q4_WAVES * 4;  // head-rows per workgroup
constexpr int Q4_ROW_BYTES = 144;

// Sequence owning item `r` of a segmented range: the s with off[s] <= r < off[s+1].
__device__ __forceinline__ int find_seq(const int64_t* __restrict__ off, int n_seqs, int64_t r) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int64_t cell_of(const kvq_q4_cache& c, int s, int64_t pos) {
    if (pos < 0) return -1;
    const int64_t page = pos / c.page_size;
    if (page >= c.max_pages) return -1;
    const int64_t phys = c.block_table[(int64_t)s * c.max_pages + page];
    if (phys < 0) return -1;
    const int64_t cell = phys * c.page_size + pos % c.page_size;
    return cell < c.n_cells ? cell : -1;
}

// grid.x: groups of Q4_ROWS_PER_BLOCK head-rows of one plane; grid.y: plane (0 = K, 1 = V).
__global__ __launch_bounds__(Q4_WAVES * KVQ_WAVE) void k_append_q4_0(kvq_q4_cache c, int n_seqs,
                                                                    const int32_t* __restrict__ pos0,
                                                                    const int64_t* __restrict__ src_off,
                                                                    int64_t total_new,
                                                                    const float* __restrict__ k_src,
                                                                    const float* __restrict__ v_src,
                                                                    int rotate) {
    __shared__ __align__(16) uint8_t stage[Q4_ROWS_PER_BLOCK][Q4_ROW_BYTES];
    const int plane = blockIdx.y;
    const int lane = threadIdx.x & 15;           // lane within the head-row
    const int slot = threadIdx.x >> 4;           // head-row within the workgroup
    const int64_t hr = (int64_t)blockIdx.x * Q4_ROWS_PER_BLOCK + slot;  // head-row = r * n_kv + h
    const int64_t n_hr = total_new * c.n_kv_heads;
    const bool valid = hr < n_hr;
    const int64_t r = valid ? hr / c.n_kv_heads : 0;
    const int h = valid ? (int)(hr % c.n_kv_heads) : 0;
    int64_t cell = -1;
    float v[16];
    if (valid) {
        const int s = find_seq(src_off, n_seqs, r);
        cell = cell_of(c, s, (int64_t)pos0[s] + (r - src_off[s]));
        const float* src = (plane ? v_src : k_src) + hr * 256 + lane * 16;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 a = *reinterpret_cast<const float4*>(src + 4 * q);
            v[4 * q + 0] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = 0.0f;
    }
    if (rotate) {
#pragma unroll
        for (int hh = 1; hh < 16; hh <<= 1)
#pragma unroll
            for (int i = 0; i < 16; i++)
                if (!(i & hh)) {
                    const float a = v[i], b = v[i + hh];
                    v[i] = a + b;
                    v[i + hh] = a - b;
                }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = fwht_xlane(v[i], threadIdx.x, m);
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = v[i] * 0.0625f;
    }
    // block b = lane / 2: mval = element with the largest key (|x|, x), +0 over -0
    uint32_t best = absval_key(v[0]);
    float mval = v[0];
#pragma unroll
    for (int i = 1; i < 16; i++) {
        const uint32_t k = absval_key(v[i]);
        if (k > best) { best = k; mval = v[i]; }
    }
    {
        const uint32_t ob = shfl_xor_u(best, 1);
        const float om = shfl_xor_f(mval, 1);
        if (ob > best) { best = ob; mval = om; }
    }
    const float d = mval / -8.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    uint32_t q[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float t = __builtin_fmaf(v[i], id, 8.5f);
        q[i] = !(t >= 0.0f) ? 0u : (t >= 15.0f ? 15u : (uint32_t)(int)t);
    }
    // lane 2b holds block elements 0..15, lane 2b+1 elements 16..31.
    // byte j = q_j | q_{j+16} << 4: the even lane forms bytes 0..7, the odd lane 8..15.
    uint32_t mine_lo = 0, mine_hi = 0;  // nibbles of elements 0..7 and 8..15 of this lane
#pragma unroll
    for (int i = 0; i < 8; i++) {
        mine_lo |= q[i] << (4 * i);
        mine_hi |= q[8 + i] << (4 * i);
    }
    const bool odd = lane & 1;
    // the even lane needs the odd lane's 0..7, the odd lane needs the even lane's 8..15
    const uint32_t give = odd ? mine_lo : mine_hi;
    const uint32_t got = shfl_xor_u(give, 1);
    const uint32_t low_nib = odd ? got : mine_lo;    // q_j for the 8 bytes this lane forms
    const uint32_t high_nib = odd ? mine_hi : got;   // q_{j+16}
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w0 |= (((low_nib >> (4 * i)) & 15u) | (((high_nib >> (4 * i)) & 15u) << 4)) << (8 * i);
        w1 |= (((low_nib >> (4 * (i + 4))) & 15u) | (((high_nib >> (4 * (i + 4))) & 15u) << 4)) << (8 * i);
    }
    uint8_t* row = stage[slot];
    const int blk = (lane >> 1) * 18;
    uint16_t* row16 = reinterpret_cast<uint16_t*>(row);  // every field starts at an even offset
    if (!odd) row16[blk / 2] = (uint16_t)f32_to_f16_rne(d);
    const int qo = (blk + 2 + (odd ? 8 : 0)) / 2;
    row16[qo + 0] = (uint16_t)(w0 & 0xFFFF);
    row16[qo + 1] = (uint16_t)(w0 >> 16);
    row16[qo + 2] = (uint16_t)(w1 & 0xFFFF);
    row16[qo + 3] = (uint16_t)(w1 >> 16);
    __syncthreads();
    if (valid && cell >= 0 && lane < 9) {
        uint8_t* pool = plane ? c.v_pool : c.k_pool;
        uint4* dst = reinterpret_cast<uint4*>(pool + (cell * c.n_kv_heads + h) * Q4_ROW_BYTES);
        dst[lane] = reinterpret_cast<const uint4*>(row)[lane];
    }
}

// One 16-lane group per destination head-row: nine 16-byte loads of the
// 144-byte head-row into LDS, then each lane dequantizes 16 elements (half of
// one block) and stores 32 bytes of binary16.
__global__ __launch_bounds__(Q4_WAVES * KVQ_WAVE) void k_gather_q4_0(kvq_q4_cache c, int n_seqs,
                                                                    const int64_t* __restrict__ dst_off,
                                                                    int64_t total_rows, uint16_t* __restrict__ k_dst,
                                                                    uint16_t* __restrict__ v_dst) {
    __shared__ __align__(16) uint8_t stage[Q4_ROWS_PER_BLOCK][Q4_ROW_BYTES];
    const int plane = blockIdx.y;
    const int lane = threadIdx.x & 15;
    const int slot = threadIdx.x >> 4;
    const int64_t hr = (int64_t)blockIdx.x * Q4_ROWS_PER_BLOCK + slot;  // = R * n_kv + h
    const bool valid = hr < total_rows * c.n_kv_heads;
    int64_t cell = -1;
    int h = 0;
    if (valid) {
        const int64_t R = hr / c.n_kv_heads;
        h = (int)(hr % c.n_kv_heads);
        const int s = find_seq(dst_off, n_seqs, R);
        cell = cell_of(c, s, R - dst_off[s]);
    }
    const uint8_t* pool = plane ? c.v_pool : c.k_pool;
    if (cell >= 0 && lane < 9)
        reinterpret_cast<uint4*>(stage[slot])[lane] =
            reinterpret_cast<const uint4*>(pool + (cell * c.n_kv_heads + h) * Q4_ROW_BYTES)[lane];
    __syncthreads();
    if (cell < 0) return;
    const uint8_t* row = stage[slot];
    const int blk = (lane >> 1) * 18;
    const uint16_t* row16 = reinterpret_cast<const uint16_t*>(row);
    const float d = f16_to_f32(row16[blk / 2]);
    const int shift = (lane & 1) ? 4 : 0;  // even lane: low nibbles (elements 0..15), odd: high (16..31)
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t two = row16[blk / 2 + 1 + i];  // qs bytes 2i, 2i+1
        const int q0 = (int)((two >> shift) & 15u);
        const int q1 = (int)((two >> (8 + shift)) & 15u);
        const uint32_t h0 = f32_to_f16_rne((float)(q0 - 8) * d);
        const uint32_t h1 = f32_to_f16_rne((float)(q1 - 8) * d);
        out[i] = h0 | (h1 << 16);
    }
    uint16_t* dst = (plane ? v_dst : k_dst) + hr * 256 + lane * 16;
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(out[0], out[1], out[2], out[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

}  // namespace

hipError_t launch_append_q4_0(const kvq_q4_cache& c, int n_seqs, const int32_t* pos0,
                              const int64_t* src_off, int64_t total_new, const float* k_src,
                              const float* v_src, bool rotate, hipStream_t st) {
    const int64_t n_hr = total_new * c.n_kv_heads;
    if (n_hr == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_hr + Q4_ROWS_PER_BLOCK - 1) / Q4_ROWS_PER_BLOCK), 2), block(Q4_WAVES * KVQ_WAVE);
    hipLaunchKernelGGL(k_append_q4_0, grid, block, 0, st, c, n_seqs, pos0, src_off, total_new, k_src, v_src,
                       rotate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_gather_q4_0(const kvq_q4_cache& c, int n_seqs, const int64_t* dst_off,
                              int64_t total_rows, uint16_t* k_dst, uint16_t* v_dst, hipStream_t st) {
    const int64_t n_hr = total_rows * c.n_kv_heads;
    if (n_hr == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_hr + Q4_ROWS_PER_BLOCK - 1) / Q4_ROWS_PER_BLOCK), 2), block(Q4_WAVES * KVQ_WAVE);
    hipLaunchKernelGGL(k_gather_q4_0, grid, block, 0, st, c, n_seqs, dst_off, total_rows, k_dst, v_dst);
    return hipGetLastError();
}

}  // namespace kvq
