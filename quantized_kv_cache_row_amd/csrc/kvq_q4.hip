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

// Sequence owning item `r` of a segmented range: the largest s with off[s] <= r
// (off non-decreasing, off[0] <= r), and off[s].  The 16 lanes of a head-row
// search together, 16-ary: each step loads the first offset of 16 equal
// sub-ranges of the remaining range (one load per lane, all in flight at once)
// and keeps the last sub-range whose first offset is <= r -- ceil(log16(n_seqs))
// dependent loads where a binary search takes log2(n_seqs).  The last step has
// sub-ranges of one sequence, so off[s] is the value the winning lane loaded.
// Every lane of the wave calls it (the step count is uniform); `lane16` is the
// lane within the head-row's group, `shift` the group's first lane in the wave.
struct SeqHit {
    int s;
    int64_t start;  // off[s]
};
__device__ __forceinline__ SeqHit find_seq16(const int64_t* __restrict__ off, int n_seqs, int64_t r, int lane16,
                                             int shift) {
    int steps = 0;
    for (int64_t span = 1; span < n_seqs; span *= 16) steps++;
    if (steps == 0) return SeqHit{0, off[0]};
    int lo = 0, n = n_seqs;  // invariant: the answer lies in [lo, lo + n) and off[lo] <= r
    int64_t o = 0;
    int cnt = 1;
    for (int it = 0; it < steps; it++) {
        const int step = (n + 15) / 16;
        const int first = lo + lane16 * step;
        o = off[min(first, n_seqs - 1)];              // unconditional (clamped) load
        const bool ok = lane16 * step < n && o <= r;  // true for a prefix of the sub-ranges
        cnt = max(1, __builtin_popcount((uint32_t)(__ballot(ok) >> shift) & 0xFFFFu));
        lo += (cnt - 1) * step;
        n = min(step, n - (cnt - 1) * step);
    }
    return SeqHit{lo, __shfl(o, shift + cnt - 1, 64)};
}

// log2 of the head count and of the page size when they are powers of two, else
// -1 (set by the host).  A 64-bit division is a long instruction sequence on the
// GPU; with a power of two it is a shift (the branch is uniform).
struct Q4Shifts {
    int kv, page;
};
__device__ __forceinline__ int64_t div_by(int64_t x, int64_t d, int sh) { return sh >= 0 ? (x >> sh) : x / d; }
__device__ __forceinline__ int64_t mod_by(int64_t x, int64_t d, int sh) { return sh >= 0 ? (x & (d - 1)) : x % d; }

// Pool cell of position `pos` of sequence s through the page table, -1 if it has
// none.  Branch-free: the table load is unconditional (clamped index).
__device__ __forceinline__ int64_t cell_of(const kvq_q4_cache& c, const Q4Shifts& sh, int s, int64_t pos) {
    const int64_t p = pos >= 0 ? pos : 0;
    const int64_t page = div_by(p, c.page_size, sh.page);
    const bool in_table = pos >= 0 && page < c.max_pages;
    const int64_t phys = c.block_table[(int64_t)s * c.max_pages + (in_table ? page : 0)];
    const int64_t cell = phys * c.page_size + mod_by(p, c.page_size, sh.page);
    return (in_table && phys >= 0 && cell < c.n_cells) ? cell : -1;
}

// grid.x: groups of Q4_ROWS_PER_BLOCK head-rows of one plane; grid.y: plane (0 = K, 1 = V).
__global__ __launch_bounds__(Q4_WAVES * KVQ_WAVE) void k_append_q4_0(kvq_q4_cache c, Q4Shifts sh, int n_seqs,
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
    // past the end: work on the last head-row (clamped, so no load waits on a lane
    // condition), store nothing
    const int64_t hrc = valid ? hr : n_hr - 1;
    const int64_t r = div_by(hrc, c.n_kv_heads, sh.kv);
    const int h = (int)mod_by(hrc, c.n_kv_heads, sh.kv);
    // Lane `lane` of the head-row holds column q = lane ^ 3 bit2(lane): elements
    // 16 q .. 16 q + 15.  The FWHT partners of element-index bits 4..7 (bits 0..3
    // of q) are then lanes lane ^ 1, ^ 2, ^ 7, ^ 8 -- one DPP pattern each.
    const int q = lane ^ (((lane >> 2) & 1) * 3);
    float v[16];
    {
        const float* src = (plane ? v_src : k_src) + hrc * 256 + q * 16;  // independent of the lookup
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 a = *reinterpret_cast<const float4*>(src + 4 * q);
            v[4 * q + 0] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
        }
    }
    const SeqHit hit = find_seq16(src_off, n_seqs, r, lane, threadIdx.x & 48);
    int64_t cell = cell_of(c, sh, hit.s, (int64_t)pos0[hit.s] + (r - hit.start));
    if (!valid) cell = -1;
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
        // Cross-lane stages h = 16 .. 128: y + c * y_partner, c = +1 in the lower
        // lane and -1 in the upper (one fma, rounded once like a + b or b - a), so
        // the upper lane holds the negated butterfly output; lane q ends with
        // (-1)^popcount(q) times the transform, and the x 1/16 scale (exact)
        // carries that sign back.
        const float c0 = (q & 1) ? -1.0f : 1.0f, c1 = (q & 2) ? -1.0f : 1.0f;
        const float c2 = (q & 4) ? -1.0f : 1.0f, c3 = (q & 8) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 8) KVQ_FMAC_DPP_X8("quad_perm:[1,0,3,2]", v, i, c0);
#pragma unroll
        for (int i = 0; i < 16; i += 8) KVQ_FMAC_DPP_X8("quad_perm:[2,3,0,1]", v, i, c1);
#pragma unroll
        for (int i = 0; i < 16; i += 8) KVQ_FMAC_DPP_X8("row_half_mirror", v, i, c2);
#pragma unroll
        for (int i = 0; i < 16; i += 8) KVQ_FMAC_DPP_X8("row_ror:8", v, i, c3);
        const float sc = (__builtin_popcount(q) & 1) ? -0.0625f : 0.0625f;
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = v[i] * sc;
    }
    // block b = q / 2 (lanes q, q ^ 1): mval = element with the largest key
    // (|x|, x), +0 over -0.  key = bits of x with the sign flipped, rotated left
    // by one: magnitude << 1 | (sign ^ 1).
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t b = f2u(v[i]) ^ 0x80000000u;
        best = max(best, __builtin_amdgcn_alignbit(b, b, 31));
    }
    best = max(best, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)best, DPP_XOR1, 0xF, 0xF, true));
    const float mval = u2f((best >> 1) | ((~best & 1u) << 31));
    const float d = mval / -8.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    uint32_t qn[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float t = __builtin_fmaf(v[i], id, 8.5f);
        // v_cvt_u32_f32 truncates toward zero, gives 0 for negatives and NaN and
        // saturates above; the min caps at 15
        uint32_t u;
        asm("v_cvt_u32_f32 %0, %1" : "=v"(u) : "v"(t));
        qn[i] = min(u, 15u);
    }
    // lane 2b holds block elements 0..15, lane 2b+1 elements 16..31.
    // byte j = q_j | q_{j+16} << 4: the even lane forms bytes 0..7, the odd lane 8..15.
    uint32_t mine_lo = 0, mine_hi = 0;  // nibbles of elements 0..7 and 8..15 of this lane
#pragma unroll
    for (int i = 0; i < 8; i++) {
        mine_lo |= qn[i] << (4 * i);
        mine_hi |= qn[8 + i] << (4 * i);
    }
    const bool odd = q & 1;
    // the even lane needs the odd lane's 0..7, the odd lane needs the even lane's 8..15
    const uint32_t give = odd ? mine_lo : mine_hi;
    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, DPP_XOR1, 0xF, 0xF, false);
    const uint32_t low_nib = odd ? got : mine_lo;    // q_j for the 8 bytes this lane forms
    const uint32_t high_nib = odd ? mine_hi : got;   // q_{j+16}
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w0 |= (((low_nib >> (4 * i)) & 15u) | (((high_nib >> (4 * i)) & 15u) << 4)) << (8 * i);
        w1 |= (((low_nib >> (4 * (i + 4))) & 15u) | (((high_nib >> (4 * (i + 4))) & 15u) << 4)) << (8 * i);
    }
    uint8_t* row = stage[slot];
    const int blk = (q >> 1) * 18;
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

// One 16-lane group per destination head-row, four head-row groups per workgroup
// (64 head-rows): the lookups of all four come first, so their dependent loads
// (offsets, page table, pool) overlap instead of running one chain per group.
// Nine 16-byte loads bring a 144-byte head-row to LDS; then each lane
// dequantizes 16 elements (half of one block) and stores 32 bytes of binary16.
constexpr int G_SUB = 4;  // head-row groups per gather workgroup

__global__ __launch_bounds__(Q4_WAVES * KVQ_WAVE) void k_gather_q4_0(kvq_q4_cache c, Q4Shifts sh, int n_seqs,
                                                                    const int64_t* __restrict__ dst_off,
                                                                    int64_t total_rows, uint16_t* __restrict__ k_dst,
                                                                    uint16_t* __restrict__ v_dst) {
    __shared__ __align__(16) uint8_t stage[G_SUB][Q4_ROWS_PER_BLOCK][Q4_ROW_BYTES];
    const int plane = blockIdx.y;
    const int lane = threadIdx.x & 15;
    const int slot = threadIdx.x >> 4;
    const int64_t n_hr = total_rows * c.n_kv_heads;
    const uint8_t* pool = plane ? c.v_pool : c.k_pool;
    int64_t hr[G_SUB], cell[G_SUB];
#pragma unroll
    for (int g = 0; g < G_SUB; g++) {
        hr[g] = ((int64_t)blockIdx.x * G_SUB + g) * Q4_ROWS_PER_BLOCK + slot;  // = R * n_kv + h
        const bool valid = hr[g] < n_hr;
        const int64_t hrc = valid ? hr[g] : n_hr - 1;  // clamped: the lookup runs in every lane
        const int64_t R = div_by(hrc, c.n_kv_heads, sh.kv);
        const SeqHit hit = find_seq16(dst_off, n_seqs, R, lane, threadIdx.x & 48);
        const int64_t cl = cell_of(c, sh, hit.s, R - hit.start);
        // pool row of (cell, head); -1: no cell (a position outside the table or the pool)
        cell[g] = (valid && cl >= 0) ? cl * c.n_kv_heads + mod_by(hrc, c.n_kv_heads, sh.kv) : -1;
    }
    uint4 raw[G_SUB];
#pragma unroll
    for (int g = 0; g < G_SUB; g++)  // unconditional: no cell reads row 0, lanes 9..15 re-read chunk 8
        raw[g] = reinterpret_cast<const uint4*>(pool + max(cell[g], (int64_t)0) * Q4_ROW_BYTES)[min(lane, 8)];
#pragma unroll
    for (int g = 0; g < G_SUB; g++)
        if (lane < 9) reinterpret_cast<uint4*>(stage[g][slot])[lane] = raw[g];
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G_SUB; g++) {
        if (cell[g] < 0) continue;
        const uint16_t* row16 = reinterpret_cast<const uint16_t*>(stage[g][slot]);
        uint16_t* dst = (plane ? v_dst : k_dst) + hr[g] * 256;
        // lane l writes elements 8 l .. 8 l + 7 and 128 + 8 l .. + 7: each of the
        // two stores covers 256 contiguous bytes of the row across the 16 lanes
#pragma unroll
        for (int part = 0; part < 2; part++) {
            const int e0 = 128 * part + 8 * lane;          // first element: block e0 / 32
            const int blk = (e0 >> 5) * 18, pos = e0 & 31;  // 8 positions of one nibble side
            const float d = f16_to_f32(row16[blk / 2]);
            const int shift = pos >= 16 ? 4 : 0;            // elements 16..31 of a block: high nibbles
            const uint8_t* qs = stage[g][slot] + blk + 2 + (pos & 15);
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int q0 = (int)((qs[2 * i] >> shift) & 15u), q1 = (int)((qs[2 * i + 1] >> shift) & 15u);
                // (q - 8) d is exact in fp32; the hardware conversion rounds it to nearest even
                out[i] = f32_to_f16_rne((float)(q0 - 8) * d) | (f32_to_f16_rne((float)(q1 - 8) * d) << 16);
            }
            __builtin_nontemporal_store(make_uint4(out[0], out[1], out[2], out[3]).x, reinterpret_cast<uint32_t*>(dst + e0));
            __builtin_nontemporal_store(make_uint4(out[0], out[1], out[2], out[3]).y, reinterpret_cast<uint32_t*>(dst + e0) + 1);
            __builtin_nontemporal_store(make_uint4(out[0], out[1], out[2], out[3]).z, reinterpret_cast<uint32_t*>(dst + e0) + 2);
            __builtin_nontemporal_store(make_uint4(out[0], out[1], out[2], out[3]).w, reinterpret_cast<uint32_t*>(dst + e0) + 3);
        }
    }
}

int log2_if_pow2(int64_t v) {
    if (v <= 0 || (v & (v - 1)) != 0) return -1;
    int k = 0;
    while ((int64_t(1) << k) < v) k++;
    return k;
}
Q4Shifts shifts_of(const kvq_q4_cache& c) { return Q4Shifts{log2_if_pow2(c.n_kv_heads), log2_if_pow2(c.page_size)}; }

}  // namespace

hipError_t launch_append_q4_0(const kvq_q4_cache& c, int n_seqs, const int32_t* pos0,
                              const int64_t* src_off, int64_t total_new, const float* k_src,
                              const float* v_src, bool rotate, hipStream_t st) {
    const int64_t n_hr = total_new * c.n_kv_heads;
    if (n_hr == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_hr + Q4_ROWS_PER_BLOCK - 1) / Q4_ROWS_PER_BLOCK), 2), block(Q4_WAVES * KVQ_WAVE);
    hipLaunchKernelGGL(k_append_q4_0, grid, block, 0, st, c, shifts_of(c), n_seqs, pos0, src_off, total_new, k_src, v_src,
                       rotate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_gather_q4_0(const kvq_q4_cache& c, int n_seqs, const int64_t* dst_off,
                              int64_t total_rows, uint16_t* k_dst, uint16_t* v_dst, hipStream_t st) {
    const int64_t n_hr = total_rows * c.n_kv_heads;
    if (n_hr == 0) return hipSuccess;
    if (c.n_cells == 0) return hipSuccess;  // no cell: nothing is written
    constexpr int64_t per_wg = (int64_t)G_SUB * Q4_ROWS_PER_BLOCK;
    const dim3 grid((unsigned)((n_hr + per_wg - 1) / per_wg), 2), block(Q4_WAVES * KVQ_WAVE);
    hipLaunchKernelGGL(k_gather_q4_0, grid, block, 0, st, c, shifts_of(c), n_seqs, dst_off, total_rows, k_dst, v_dst);
    return hipGetLastError();
}

}  // namespace kvq
