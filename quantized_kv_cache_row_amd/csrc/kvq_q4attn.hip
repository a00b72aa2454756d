// kvq_q4attn.hip -- fused decode attention over the paged q4_0 K/V pools
// (Strata PR #2533 "metal: q4_0 KV cache on the Mac engine", the QSA_KV_Q4
// commit: the query row passes through the orthonormal 256-point FWHT, every
// pool block is read as (nibble - 8) * f32(d), scores and the weighted value
// sum stay in fp32 in the rotated domain, and the merged row o / L is rotated
// back by the same self-inverse transform; the sigmoid gate of the pages'
// model is the caller's).
//
// Three launches on the caller's stream:
//   prep   workgroup 0 writes the T-split prefix; every other wave rotates one
//          query row (4 values per lane, stages 1-2 in registers, 4-128 across
//          lanes), folds sm_scale * log2(e) into it and writes the score
//          products' fp16 operands (three terms per head, in lane order);
//   attn   one workgroup per (T-split, KV head, group of up to 4 query heads),
//          XCD-grouped so that the KV heads of one split (adjacent 144-byte
//          head-rows of the same cells) share an L2; four waves take contiguous
//          quarters of the split in tiles of 32 positions; partial (m, l, O)
//          per query head;
//   merge  one wave per (sequence, query head): combine the splits, divide,
//          rotate back, write out and lse.
//
// attn, per 32-position tile of a wave (kernel k_q4_attn_mx, on the gfx950
// matrix cores, v_mfma_f32_16x16x32_f16; the pages' fp32 arithmetic kept to
// fp32 accuracy by exact fp16 operands and fp16 term splits):
//   * lanes 0-31 carry the tile's K head-rows, lanes 32-63 its V head-rows
//     (nine 16-byte loads, issued a tile ahead), staged into LDS regrouped so
//     that every read is aligned (nibble bytes of block b at 16b), the block
//     scales by block and position;
//   * scores: per block, a K = 32 step with the codes minus 8 (exact in fp16)
//     against three fp16 terms of the power-of-two scaled rotated query of
//     each head (one column per head and term), then d times the result in
//     fp32;
//   * online softmax in the log2 domain per query head (lane = position);
//   * values: O^T += V^T P with V^T read transposed from the staged rows
//     (ds_read_b64_tr_b8) as (code - 8) * d * vs in two exact fp16 terms (vs a
//     power of two that keeps the products in range) and two fp16 terms of p
//     per head; the accumulators hold O * vs.
// Four waves per workgroup take contiguous quarters of the split; their
// (m, l, O) are combined through LDS into one partial per (split, query head).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int QA_WAVES = 4;
constexpr int QA_TILE = 64;   // split granularity: QA_TILE * QA_WAVES positions
constexpr int QA_HD = 256;    // head_dim
constexpr int QA_RB = 144;    // bytes per head-row: 8 blocks of 18
constexpr int QA_NXCD = 8;
// Query heads per workgroup at most: 16 heads per KV head split over two
// workgroups that read the same head-rows (neighbouring items, so from the same
// L2).  With 8 heads the value products use all 16 columns of the matrix-core
// tile (two terms of p per head).
constexpr int QA_GMAX = 8;
constexpr float QA_LOG2E = 1.4426950408889634f;
constexpr float QA_LN2 = 0.6931471805599453f;

struct Q4Plan {
    int64_t* chunk_prefix;  // [n_seqs + 1]
    uint4* q_mx;            // [n_seqs][n_kv][sub][8 blocks][64 lanes]: the score products' fp16 operands
    float* q_inv;           // [n_seqs][n_q]: 1 / qs of each head's operands
    float* part_m;          // [max_chunks][n_q] (log2 domain)
    float* part_l;          // [max_chunks][n_q]
    float* part_o;          // [max_chunks][n_q][256] (rotated domain, unnormalized)
    int64_t max_chunks;
    int64_t items_per_xcd;  // attn grid: item ((chunk * n_kv + kv head) * sub + part) runs on XCD item / items_per_xcd
    int split;
    int group;              // query heads per KV head
    int sub;                // workgroups per (split, KV head): each takes group / sub query heads
};

int q4_auto_split(const kvq_q4_attn_args& a, int n_kv) {
    // about four workgroups per compute unit over all splits and KV heads
    int64_t split = (a.total_rows * n_kv + 1023) / 1024;
    if (split < 256) split = 256;
    split = (split + QA_TILE * QA_WAVES - 1) / (QA_TILE * QA_WAVES) * (QA_TILE * QA_WAVES);
    if (split > (1 << 24)) split = 1 << 24;
    return (int)split;
}

Q4Plan q4_make_plan(const kvq_q4_cache& c, const kvq_q4_attn_args& a, void* ws, int64_t* bytes_out) {
    Q4Plan p{};
    p.split = a.split_rows > 0 ? a.split_rows : q4_auto_split(a, c.n_kv_heads);
    p.group = a.n_q_heads / c.n_kv_heads;
    p.sub = p.group > QA_GMAX ? p.group / QA_GMAX : 1;
    // sum_s max(1, ceil(len_s / split)), as for the latent decode's T-split
    p.max_chunks = std::max<int64_t>(a.n_seqs, std::min<int64_t>(a.total_rows / p.split + a.n_seqs,
                                                                  (a.total_rows + p.split - 1) / p.split + a.n_seqs - 1));
    p.items_per_xcd = (p.max_chunks * c.n_kv_heads * p.sub + QA_NXCD - 1) / QA_NXCD;
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    int64_t off = 0;
    char* base = (char*)ws;
    auto take = [&](int64_t bytes) {
        char* q = base ? base + off : nullptr;
        off = align(off + bytes);
        return q;
    };
    const int64_t rows_q = (int64_t)a.n_seqs * a.n_q_heads;
    p.chunk_prefix = (int64_t*)take(sizeof(int64_t) * (a.n_seqs + 1));
    p.q_mx = (uint4*)take(sizeof(uint4) * (int64_t)a.n_seqs * c.n_kv_heads * p.sub * 2 * 8 * 64);
    p.q_inv = (float*)take(sizeof(float) * rows_q);
    p.part_m = (float*)take(sizeof(float) * p.max_chunks * a.n_q_heads);
    p.part_l = (float*)take(sizeof(float) * p.max_chunks * a.n_q_heads);
    p.part_o = (float*)take(sizeof(float) * p.max_chunks * a.n_q_heads * QA_HD);
    if (bytes_out) *bytes_out = off;
    return p;
}

// Positions of sequence s.  The offsets are clamped to [0, total] (total =
// the host copy of off[n_seqs]), as the latent decode clamps its rows, so the
// split count built from them never exceeds what the workspace was sized for.
__device__ __forceinline__ int64_t seq_len(const int64_t* __restrict__ off, int s, int64_t total) {
    const int64_t lo = max(off[s], (int64_t)0), hi = min(off[s + 1], total);
    return hi > lo ? hi - lo : 0;
}

// Orthonormal FWHT-256 of a row held 4 consecutive values per lane (lane l has
// elements 4l .. 4l+3), Sylvester order: stages of span 1 and 2 in registers,
// spans 4 .. 128 with lane partners l ^ 1 .. l ^ 32; then / 16.
__device__ __forceinline__ void fwht256_wave(float (&x)[4], int lane) {
    float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
    x[0] = a0 + a2;
    x[1] = a1 + a3;
    x[2] = a0 - a2;
    x[3] = a1 - a3;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[i] = fwht_xlane_c<1>(x[i], lane);
        x[i] = fwht_xlane_c<2>(x[i], lane);
        x[i] = fwht_xlane_c<4>(x[i], lane);
        x[i] = fwht_xlane_c<8>(x[i], lane);
        x[i] = fwht_xlane_c<16>(x[i], lane);
        x[i] = fwht_xlane_c<32>(x[i], lane);
        x[i] *= 0.0625f;
    }
}

// Power of two 2^k with max_abs * 2^k in [2^t, 2^(t+1)) for normal max_abs; 1 for 0.
__device__ __forceinline__ float q4_pow2_scale(float max_abs, int t) {
    if (!(max_abs > 0.0f)) return 1.0f;
    int e = (int)((f2u(max_abs) >> 23) & 255u) - 127;
    if (e < -126) e = -126;
    int k = t - e;
    if (k > 127) k = 127;
    if (k < -126) k = -126;
    return u2f((uint32_t)(k + 127) << 23);
}

// ---- prep -------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_q4_prep(kvq_q4_attn_args a, Q4Plan p) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        // chunk_prefix[s] = sum_{s' < s} max(1, ceil(len_s' / split))
        __shared__ int64_t part[256];
        const int per = (a.n_seqs + 255) / 256;
        const int s0 = tid * per, s1 = min(a.n_seqs, s0 + per);
        int64_t local = 0;
        for (int s = s0; s < s1; s++) {
            const int64_t n = seq_len(a.len_off, s, a.total_rows);
            local += n > 0 ? (n + p.split - 1) / p.split : 1;
        }
        part[tid] = local;
        __syncthreads();
        for (int o = 1; o < 256; o <<= 1) {
            const int64_t v = tid >= o ? part[tid - o] : 0;
            __syncthreads();
            part[tid] += v;
            __syncthreads();
        }
        int64_t run = tid > 0 ? part[tid - 1] : 0;
        for (int s = s0; s < s1; s++) {
            p.chunk_prefix[s] = run;
            const int64_t n = seq_len(a.len_off, s, a.total_rows);
            run += n > 0 ? (n + p.split - 1) / p.split : 1;
        }
        if (tid == 255) p.chunk_prefix[a.n_seqs] = part[255];
        return;
    }
    const int lane = tid & 63;
    // wave-uniform (scalar) row and its divisions
    const int64_t row = (int64_t)(blockIdx.x - 1) * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
    if (row >= (int64_t)a.n_seqs * a.n_q_heads) return;
    const float4 v = reinterpret_cast<const float4*>(a.q + row * QA_HD)[lane];
    float x[4] = {v.x, v.y, v.z, v.w};
    fwht256_wave(x, lane);
    const float sc = a.sm_scale * QA_LOG2E;
#pragma unroll
    for (int i = 0; i < 4; i++) x[i] *= sc;
    // The score products' B operands (v_mfma_f32_16x16x32_f16, one K = 32 step per block),
    // x = H q / 16 * sm_scale * log2(e): x * qs (qs a power of two, max |x| qs in
    // [2^14, 2^15)) as three fp16 terms, about 33 significant bits together.  Up to 4 heads
    // per workgroup: column h + 4 t of column tile 0 holds term t of head h; 8 heads:
    // column h + 8 t of tile 0 holds terms 0 and 1, column h of tile 1 term 2.  Lane (g, n)
    // holds k = 8 g + e, which is block element 4 g + e for e < 4 and 16 + 4 g + e - 4 for
    // e >= 4 (the low and high nibbles of bytes 4 g .. 4 g + 3).  This lane's elements
    // 4 (lane % 8) .. + 3 of block lane / 8 are k = 8 g + 4 hf + {0..3} with g = lane % 4,
    // hf = (lane / 4) % 2.
    float qmax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    qmax = wave_max(qmax);
    const float qs = q4_pow2_scale(qmax, 14);
    const int64_t sq = row / a.n_q_heads;
    const int hq = (int)(row - sq * a.n_q_heads), kv = hq / p.group, hl = hq - kv * p.group;
    const int part = hl / QA_GMAX, hh = hl % QA_GMAX;
    const bool eight = p.group >= 8;
    const int64_t nkv = a.n_q_heads / p.group;
    uint2* qm = reinterpret_cast<uint2*>(p.q_mx + (((sq * nkv + kv) * p.sub + part) * 16 + (lane >> 3)) * 64);
    const int gk = lane & 3, hf = (lane >> 2) & 1;
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = x[i] * qs;  // exact
#pragma unroll
    for (int t = 0; t < 3; t++) {
        float tv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            tv[i] = (float)(_Float16)r[i];  // round to nearest even
            r[i] -= tv[i];                  // exact
        }
        const int tile = eight && t == 2 ? 1 : 0;
        const int colm = eight ? hh + 8 * (t & 1) * (t < 2 ? 1 : 0) : hh + 4 * t;
        qm[tile * (8 * 64 * 2) + 2 * (16 * gk + colm) + hf] =
            make_uint2(f32_to_f16_rne(tv[0]) | (f32_to_f16_rne(tv[1]) << 16),
                       f32_to_f16_rne(tv[2]) | (f32_to_f16_rne(tv[3]) << 16));
    }
    if (lane == 0) p.q_inv[row] = 1.0f / qs;  // exact
}

// ---- attn -------------------------------------------------------------------------

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// Four bytes of a head-row held as 36 dwords, starting at byte OFF (even).
template <int OFF>
__device__ __forceinline__ uint32_t row_dw(const uint32_t (&r)[36]) {
    static_assert(OFF % 2 == 0 && OFF + 4 <= QA_RB, "row_dw offset");
    if constexpr (OFF % 4 == 0) {
        return r[OFF / 4];
    } else {
        const uint64_t pair = ((uint64_t)r[OFF / 4 + 1] << 32) | r[OFF / 4];
        return (uint32_t)(pair >> (8 * (OFF % 4)));
    }
}

// A V head-row into the wave's LDS slice, blocks regrouped so that every read
// is aligned: bytes 16b .. 16b+15 = the nibble bytes of block b, bytes 128 +
// 2b = its binary16 scale.
template <int B>
__device__ __forceinline__ void stage_v_block(const uint32_t (&r)[36], uint8_t* dst) {
    *reinterpret_cast<uint4*>(dst + 16 * B) = make_uint4(row_dw<18 * B + 2>(r), row_dw<18 * B + 6>(r),
                                                          row_dw<18 * B + 10>(r), row_dw<18 * B + 14>(r));
}
__device__ __forceinline__ void stage_v_row(const uint32_t (&r)[36], uint8_t* dst) {
    stage_v_block<0>(r, dst);
    stage_v_block<1>(r, dst);
    stage_v_block<2>(r, dst);
    stage_v_block<3>(r, dst);
    stage_v_block<4>(r, dst);
    stage_v_block<5>(r, dst);
    stage_v_block<6>(r, dst);
    stage_v_block<7>(r, dst);
    auto sc2 = [&](uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); };
    *reinterpret_cast<uint4*>(dst + 128) =
        make_uint4(sc2(row_dw<0>(r), row_dw<18>(r)), sc2(row_dw<36>(r), row_dw<54>(r)),
                   sc2(row_dw<72>(r), row_dw<90>(r)), sc2(row_dw<108>(r), row_dw<126>(r)));
}

// ---- attn on the matrix cores ------------------------------------------------------
// v_mfma_f32_16x16x32_f16 (lane (g, n) = (l / 16, l % 16) holds A[n][8 g + e] and
// B[8 g + e][n], e < 8, and D[4 g + i][n], i < 4).  Per 64-position tile of a wave:
//   * scores: for 16 positions and block b, A = the codes minus 8 (exact in fp16),
//     K index 8 g + e = block element 4 g + e (e < 4) or 16 + 4 g + e - 4 (the
//     low and high nibbles of bytes 4 g .. 4 g + 3), B = three fp16 terms of
//     q~ * qs per head (column h + 4 t), C = 0; then s += d_b * D in fp32, the
//     terms summed across lanes, times 1 / qs;
//   * online softmax per head, lane = position, through LDS;
//   * values: O^T (dims x columns) += A B over 32 positions: A = (code - 8) *
//     d * vs as two exact fp16 terms (the product has at most 14 significant
//     bits; vs a power of two per tile putting 8 max |d| vs in [2^14, 2^15)),
//     read transposed from the staged rows (ds_read_b64_tr_b8: the 16 lanes
//     of group g receive byte n of block b from positions 8 g .. 8 g + 7), B =
//     two fp16 terms of p per head (column h + 4 t); the accumulators hold O * vs
//     and are rescaled by alpha * vs_new / vs per tile.
typedef _Float16 q4h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 q4h8_t __attribute__((ext_vector_type(8)));
typedef float q4f4_t __attribute__((ext_vector_type(4)));
typedef int q4i2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t h2_add(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(q4h2_t, a) + __builtin_bit_cast(q4h2_t, b));
}
__device__ __forceinline__ uint32_t h2_mul(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(q4h2_t, a) * __builtin_bit_cast(q4h2_t, b));
}
// a * b + c with one rounding
__device__ __forceinline__ uint32_t h2_fma(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(q4h2_t, a),
                                                                  __builtin_bit_cast(q4h2_t, b),
                                                                  __builtin_bit_cast(q4h2_t, c)));
}
// Eight bytes b (each 0 .. 15: bytes 0..3 of w0, then of w1) -> eight fp16 b - 8, exact:
// the byte under 0x64 is the binary16 1024 + b, then 1032 is subtracted.
__device__ __forceinline__ uint4 q4_nib_f16(uint32_t w0, uint32_t w1) {
    const uint32_t c = 0x64646464u, m = 0xE408E408u;  // m = (-1032, -1032)
    return make_uint4(h2_add(__builtin_amdgcn_perm(c, w0, 0x04010400u), m),
                      h2_add(__builtin_amdgcn_perm(c, w0, 0x04030402u), m),
                      h2_add(__builtin_amdgcn_perm(c, w1, 0x04010400u), m),
                      h2_add(__builtin_amdgcn_perm(c, w1, 0x04030402u), m));
}
__device__ __forceinline__ q4f4_t q4_mfma(uint4 a, uint4 b, q4f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(q4h8_t, a), __builtin_bit_cast(q4h8_t, b), c,
                                                  0, 0, 0);
}
// The value of lane + K within the 16-lane row (0 past its end).
template <int K>
__device__ __forceinline__ float row_from_above(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xF, 0xF, true));
}

constexpr int QM_TILE = 32;  // positions per wave tile: lanes 0-31 carry their K head-rows, 32-63 their V head-rows

// Maximum over the wave, on DPP and lane swaps (every lane gets it).
__device__ __forceinline__ float q4_wave_max(float v, int lane) {
    v = fmaxf(v, xor_lane<1>(v, lane));
    v = fmaxf(v, xor_lane<2>(v, lane));
    v = fmaxf(v, xor_lane<4>(v, lane));
    v = fmaxf(v, xor_lane<8>(v, lane));
    v = fmaxf(v, xor_lane<16>(v, lane));
    return fmaxf(v, xor_lane<32>(v, lane));
}

template <int G>
struct Q4MxShared {
    static constexpr int NH = G == 8 ? 8 : 4;
    uint4 qmx[G == 8 ? 2 : 1][8][64];     // the score operands
    uint8_t k[QA_WAVES][QM_TILE][QA_RB];  // the tile's K head-rows, regrouped as stage_v_row does
    uint8_t v[QA_WAVES][QM_TILE][QA_RB];  // the V head-rows, the same
    uint16_t dk[QA_WAVES][8][QM_TILE];    // K block scales (binary16) by block, then position
    uint16_t dv[QA_WAVES][8][QM_TILE];    // V block scales times vs (binary16), the same
    float sc[QA_WAVES][QM_TILE][NH];      // scores (log2 units) by position, then head
    float pr[QA_WAVES][NH][QM_TILE];      // probabilities by head, then position
    float m[QA_WAVES][NH];
    float l[QA_WAVES][NH];
};

template <int B>
__device__ __forceinline__ void stage_scale(const uint32_t (&r)[36], bool is_v, float vs, uint16_t* dst) {
    const uint32_t bits = row_dw<18 * B>(r) & 0xFFFFu;
    dst[B * QM_TILE] = (uint16_t)(is_v ? f32_to_f16_rne(half_bits_to_f32(bits) * vs) : bits);  // exact when normal
}
template <int B>
__device__ __forceinline__ float row_dabs(const uint32_t (&r)[36]) {
    return fabsf(half_bits_to_f32(row_dw<18 * B>(r)));
}

template <int G>
__global__ __launch_bounds__(QA_WAVES * 64, G == 8 ? 2 : 3) void k_q4_attn_mx(kvq_q4_cache c, kvq_q4_attn_args a, Q4Plan p) {
    __shared__ __align__(16) Q4MxShared<G> sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t n_items = p.max_chunks * c.n_kv_heads * p.sub;
    const int64_t item = (int64_t)(blockIdx.x % QA_NXCD) * p.items_per_xcd + blockIdx.x / QA_NXCD;
    if (item >= n_items) return;
    const int64_t ch = item / ((int64_t)c.n_kv_heads * p.sub);
    const int rem = (int)(item % ((int64_t)c.n_kv_heads * p.sub));
    const int g = rem / p.sub, part = rem % p.sub;
    const int64_t nch = p.chunk_prefix[a.n_seqs];
    if (ch >= nch) return;
    int s;
    {
        int lo = 0, hi = a.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.chunk_prefix[mid] <= ch) lo = mid; else hi = mid - 1;
        }
        s = lo;
    }
    const int64_t len = seq_len(a.len_off, s, a.total_rows);
    const int64_t r0 = (ch - p.chunk_prefix[s]) * p.split;
    const int64_t r1 = min(len, r0 + p.split);
    const int hq0 = g * p.group + part * G;
    const int64_t qrow0 = (int64_t)s * a.n_q_heads + hq0;

    // MFMA lane (gq, nq).  Column nq is (head nq % HS, term nq / HS); with 8 heads the
    // third query term is a second column tile.  The score operands of this workgroup's
    // heads (columns of absent heads and terms are zero) and 1 / qs of head nq % HS.
    constexpr int HS = G == 8 ? 8 : 4;
    constexpr int KT = G == 8 ? 2 : 1;
    const int gq = lane >> 4, nq = lane & 15, hn = nq % HS;
    // (in LDS and read there per step: registers are the occupancy limit)
    {
        const uint4* qsrc = p.q_mx + (((int64_t)s * c.n_kv_heads + g) * p.sub + part) * (16 * 64);
#pragma unroll
        for (int i = 0; i < 2 * KT; i++) {
            const int e = tid + 256 * i;  // (tile, block, lane)
            const int en = e & 15;
            const bool col = G == 8 ? ((e >> 9) == 0 || en < 8) : (en < 12 && en % 4 < G);
            const uint4 v = qsrc[e];
            (&sh.qmx[0][0][0])[e] = col ? v : make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();
    }
    const float qinv = p.q_inv[qrow0 + min(hn, G - 1)];

    const int64_t quarter = ((r1 - r0 + QA_WAVES - 1) / QA_WAVES + QM_TILE - 1) / QM_TILE * QM_TILE;
    const int64_t w0 = r0 + wave * quarter;
    const int64_t w1 = min(r1, w0 + quarter);

    // lane l carries position l % 32 of the tile: its K head-row (l < 32) or V head-row
    const bool is_v = lane >= 32;
    const int pl = lane & 31;
    const int64_t cap = (int64_t)c.max_pages * c.page_size;
    const int32_t* __restrict__ tab = c.block_table + (int64_t)s * c.max_pages;
    const uint8_t* __restrict__ pool = is_v ? c.v_pool : c.k_pool;
    // (the row is masked where it is used, a tile later: a mask applied here would make the
    // compiler wait for the loads at once)
    auto load_row = [&](int64_t t0, uint4 (&rr)[9]) {
        const int64_t pos = t0 + pl;
        bool ok = pos < w1 && pos < cap;
        int64_t cell = 0;
        if (ok) {
            const int64_t col = pos / c.page_size;
            const int32_t pg = tab[col];
            cell = (int64_t)pg * c.page_size + (pos - col * c.page_size);
            ok = pg >= 0 && cell < c.n_cells;
        }
        const uint4* rp = reinterpret_cast<const uint4*>(pool + ((ok ? cell : 0) * c.n_kv_heads + g) * QA_RB);
#pragma unroll
        for (int i = 0; i < 9; i++) rr[i] = rp[i];
        return ok;
    };

    float m[G], lp[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = -INFINITY;
        lp[h] = 0.0f;
    }
    q4f4_t acc[8][2];  // O^T * vs: dims 32 b + 16 half + 4 gq + i, column nq
#pragma unroll
    for (int b = 0; b < 8; b++) acc[b][0] = acc[b][1] = q4f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float vs = 1.0f;
    const bool any_cells = c.n_cells > 0;
    uint4 rn[9];
#pragma unroll
    for (int i = 0; i < 9; i++) rn[i] = make_uint4(0, 0, 0, 0);
    bool okn = false;
    if (w0 < w1 && any_cells) okn = load_row(w0, rn);
    const q4f4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t t0 = w0; t0 < w1; t0 += QM_TILE) {
        uint32_t r[36];
        const uint32_t keep = okn ? 0xFFFFFFFFu : 0u;  // a missing position reads as zeros
#pragma unroll
        for (int i = 0; i < 9; i++) {
            r[4 * i] = rn[i].x & keep;
            r[4 * i + 1] = rn[i].y & keep;
            r[4 * i + 2] = rn[i].z & keep;
            r[4 * i + 3] = rn[i].w & keep;
        }
        const bool ok = okn;
        // the V scale: kept while 8 max |d| vs stays in [2^10, 2^15) (the products then stay
        // exact down to 2^-24 of that bound), else chosen again with 8 max |d| vs in [2^14, 2^15)
        float dm = fmaxf(fmaxf(fmaxf(row_dabs<0>(r), row_dabs<1>(r)), fmaxf(row_dabs<2>(r), row_dabs<3>(r))),
                         fmaxf(fmaxf(row_dabs<4>(r), row_dabs<5>(r)), fmaxf(row_dabs<6>(r), row_dabs<7>(r))));
        dm = q4_wave_max(is_v ? dm : 0.0f, lane);
        const float span = 8.0f * dm * vs;
        const float vs_new = (span < 32768.0f && (span >= 1024.0f || dm == 0.0f)) ? vs : q4_pow2_scale(8.0f * dm, 14);
        stage_v_row(r, is_v ? &sh.v[wave][pl][0] : &sh.k[wave][pl][0]);
        {
            uint16_t* sd = is_v ? &sh.dv[wave][0][pl] : &sh.dk[wave][0][pl];
            stage_scale<0>(r, is_v, vs_new, sd);
            stage_scale<1>(r, is_v, vs_new, sd);
            stage_scale<2>(r, is_v, vs_new, sd);
            stage_scale<3>(r, is_v, vs_new, sd);
            stage_scale<4>(r, is_v, vs_new, sd);
            stage_scale<5>(r, is_v, vs_new, sd);
            stage_scale<6>(r, is_v, vs_new, sd);
            stage_scale<7>(r, is_v, vs_new, sd);
        }
        if (t0 + QM_TILE < w1 && any_cells) okn = load_row(t0 + QM_TILE, rn);

        // ---- scores: positions 16 P + 4 gq + i, column nq
#pragma unroll
        for (int P = 0; P < 2; P++) {
            float sp[KT][4];
#pragma unroll
            for (int kt = 0; kt < KT; kt++)
#pragma unroll
                for (int i = 0; i < 4; i++) sp[kt][i] = 0.0f;
#pragma unroll
            for (int b = 0; b < 8; b++) {
                const uint32_t x = *reinterpret_cast<const uint32_t*>(&sh.k[wave][16 * P + nq][16 * b + 4 * gq]);
                const uint4 av = q4_nib_f16(x & 0x0F0F0F0Fu, (x >> 4) & 0x0F0F0F0Fu);
                const uint2 dd = *reinterpret_cast<const uint2*>(&sh.dk[wave][b][16 * P + 4 * gq]);
                const float d4[4] = {half_bits_to_f32(dd.x), half_bits_to_f32(dd.x >> 16), half_bits_to_f32(dd.y),
                                     half_bits_to_f32(dd.y >> 16)};
#pragma unroll
                for (int kt = 0; kt < KT; kt++) {
                    const q4f4_t cb = q4_mfma(av, sh.qmx[kt][b][lane], zero4);
#pragma unroll
                    for (int i = 0; i < 4; i++) sp[kt][i] = __builtin_fmaf(d4[i], cb[i], sp[kt][i]);
                }
            }
            // the three terms of each head summed: lanes nq < HS get head nq's score
            float tp[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float v = sp[0][i];
                if constexpr (G == 8) tp[i] = ((v + row_from_above<8>(v)) + sp[KT - 1][i]) * qinv;
                else tp[i] = ((v + row_from_above<4>(v)) + row_from_above<8>(v)) * qinv;
            }
            if (nq < G) {
#pragma unroll
                for (int i = 0; i < 4; i++) sh.sc[wave][16 * P + 4 * gq + i][nq] = tp[i];
            }
        }

        // ---- online softmax per head, lane = position (lanes 0-31)
        float sl[8];
        {
            const float4 s4 = *reinterpret_cast<const float4*>(&sh.sc[wave][pl][0]);
            sl[0] = s4.x; sl[1] = s4.y; sl[2] = s4.z; sl[3] = s4.w;
            if constexpr (G == 8) {
                const float4 s8 = *reinterpret_cast<const float4*>(&sh.sc[wave][pl][4]);
                sl[4] = s8.x; sl[5] = s8.y; sl[6] = s8.z; sl[7] = s8.w;
            }
        }
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float sv = (ok && !is_v) ? sl[h] : -INFINITY;
            const float mn = fmaxf(m[h], q4_wave_max(sv, lane));
            float pv = 0.0f, al = 1.0f;
            if (mn != -INFINITY) {  // wave-uniform
                al = exp2f(m[h] - mn);
                pv = exp2f(sv - mn);
            }
            m[h] = mn;
            lp[h] = __builtin_fmaf(lp[h], al, pv);
            alpha[h] = al;
            if (!is_v) sh.pr[wave][h][pl] = pv;
        }
        {  // rescale (wave-uniform test: after the first tiles the maxima and vs rarely move):
           // column nq belongs to head nq % 4
            bool same = vs_new == vs;
#pragma unroll
            for (int h = 0; h < G; h++) same = same && alpha[h] == 1.0f;
            if (!same) {
                float f = alpha[0];
#pragma unroll
                for (int h = 1; h < G; h++) f = hn == h ? alpha[h] : f;
                f *= vs_new / vs;  // powers of two: exact
#pragma unroll
                for (int b = 0; b < 8; b++) {
                    acc[b][0] *= f;
                    acc[b][1] *= f;
                }
                vs = vs_new;
            }
        }

        // ---- values over the tile's 32 positions
        uint4 pb;  // B: term nq / HS of p of head nq % HS at positions 8 gq + e
        {
            const int hs = min(hn, G - 1);
            const float4 pa = *reinterpret_cast<const float4*>(&sh.pr[wave][hs][8 * gq]);
            const float4 pc = *reinterpret_cast<const float4*>(&sh.pr[wave][hs][8 * gq + 4]);
            const float pe[8] = {pa.x, pa.y, pa.z, pa.w, pc.x, pc.y, pc.z, pc.w};
            const bool second = nq >= HS;
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = pe[2 * j], x1 = pe[2 * j + 1];
                const float a0 = (float)(_Float16)x0, a1 = (float)(_Float16)x1;
                w[j] = f32_to_f16_rne(second ? x0 - a0 : a0) | (f32_to_f16_rne(second ? x1 - a1 : a1) << 16);
            }
            const bool col = nq < 2 * HS && hn < G;
            pb = col ? make_uint4(w[0], w[1], w[2], w[3]) : make_uint4(0u, 0u, 0u, 0u);
        }
        const int prow = 8 * gq + (nq >> 1);  // the row this lane's address names
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const q4i2_t xv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) q4i2_t*)(&sh.v[wave][prow][16 * b + 8 * (nq & 1)]));
            const uint32_t x0 = (uint32_t)xv[0], x1 = (uint32_t)xv[1];
            const uint4 ds = *reinterpret_cast<const uint4*>(&sh.dv[wave][b][8 * gq]);
            const uint4 nl = q4_nib_f16(x0 & 0x0F0F0F0Fu, x1 & 0x0F0F0F0Fu);
            const uint4 nh = q4_nib_f16((x0 >> 4) & 0x0F0F0F0Fu, (x1 >> 4) & 0x0F0F0F0Fu);
            const uint4 lhi = make_uint4(h2_mul(nl.x, ds.x), h2_mul(nl.y, ds.y), h2_mul(nl.z, ds.z), h2_mul(nl.w, ds.w));
            const uint4 llo = make_uint4(h2_fma(nl.x, ds.x, lhi.x ^ 0x80008000u), h2_fma(nl.y, ds.y, lhi.y ^ 0x80008000u),
                                         h2_fma(nl.z, ds.z, lhi.z ^ 0x80008000u), h2_fma(nl.w, ds.w, lhi.w ^ 0x80008000u));
            const uint4 hhi = make_uint4(h2_mul(nh.x, ds.x), h2_mul(nh.y, ds.y), h2_mul(nh.z, ds.z), h2_mul(nh.w, ds.w));
            const uint4 hlo = make_uint4(h2_fma(nh.x, ds.x, hhi.x ^ 0x80008000u), h2_fma(nh.y, ds.y, hhi.y ^ 0x80008000u),
                                         h2_fma(nh.z, ds.z, hhi.z ^ 0x80008000u), h2_fma(nh.w, ds.w, hhi.w ^ 0x80008000u));
            acc[b][0] = q4_mfma(lhi, pb, acc[b][0]);
            acc[b][0] = q4_mfma(llo, pb, acc[b][0]);
            acc[b][1] = q4_mfma(hhi, pb, acc[b][1]);
            acc[b][1] = q4_mfma(hlo, pb, acc[b][1]);
        }
    }

    // ---- the wave's (m, l, O): O = acc / vs, the two terms of each head added
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float l = wave_sum(lp[h]);
        if (lane == 0) {
            sh.m[wave][h] = m[h];
            sh.l[wave][h] = l;
        }
    }
    const float vinv = 1.0f / vs;  // exact
    __syncthreads();  // every wave is past its last read of the staged rows
    float* ob = reinterpret_cast<float*>(&sh.k[0][0][0]);  // [QA_WAVES][G][256]
    static_assert(sizeof(sh.k) + sizeof(sh.v) >= sizeof(float) * QA_WAVES * G * QA_HD, "exchange buffer");
#pragma unroll
    for (int b = 0; b < 8; b++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            float o4[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float v = acc[b][hf][i];
                o4[i] = (v + row_from_above<HS>(v)) * vinv;
            }
            if (nq < G)
                *reinterpret_cast<float4*>(ob + ((int64_t)wave * G + nq) * QA_HD + 32 * b + 16 * hf + 4 * gq) =
                    make_float4(o4[0], o4[1], o4[2], o4[3]);
        }
    __syncthreads();
    for (int h = 0; h < G; h++) {
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < QA_WAVES; w++) mx = fmaxf(mx, sh.m[w][h]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < QA_WAVES; w++) {
            const float f = mx == -INFINITY ? 0.0f : exp2f(sh.m[w][h] - mx);
            L = __builtin_fmaf(sh.l[w][h], f, L);
            O = __builtin_fmaf(ob[((int64_t)w * G + h) * QA_HD + tid], f, O);
        }
        const int64_t prow = ch * a.n_q_heads + hq0 + h;
        p.part_o[prow * QA_HD + tid] = O;
        if (tid == 0) {
            p.part_m[prow] = mx;
            p.part_l[prow] = L;
        }
    }
}

// ---- merge ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_q4_merge(kvq_q4_attn_args a, Q4Plan p) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (tid >> 6);  // (sequence, query head)
    if (row >= (int64_t)a.n_seqs * a.n_q_heads) return;
    const int s = (int)(row / a.n_q_heads);
    const int hq = (int)(row % a.n_q_heads);
    // clamped to the workspace's splits (the prefix is built from device offsets)
    const int64_t c0 = min(p.chunk_prefix[s], p.max_chunks);
    const int64_t nc = max(min(p.chunk_prefix[s + 1], p.max_chunks) - c0, (int64_t)0);
    // the splits' maxima and sums one split per lane (64 at a time), then the
    // partial rows with the weights broadcast from their lanes; the row loads
    // do not depend on each other
    float mx = -INFINITY;
    for (int64_t b0 = 0; b0 < nc; b0 += 64) {
        const int64_t j = b0 + lane;
        mx = fmaxf(mx, wave_max(j < nc ? p.part_m[(c0 + j) * a.n_q_heads + hq] : -INFINITY));
    }
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    if (mx != -INFINITY) {
        for (int64_t b0 = 0; b0 < nc; b0 += 64) {
            const int64_t j = b0 + lane;
            float f = 0.0f, lj = 0.0f;
            if (j < nc) {
                f = exp2f(p.part_m[(c0 + j) * a.n_q_heads + hq] - mx);
                lj = p.part_l[(c0 + j) * a.n_q_heads + hq];
            }
            L += wave_sum(lj * f);
            const int n = (int)min((int64_t)64, nc - b0);
            const float4* po = reinterpret_cast<const float4*>(p.part_o + ((c0 + b0) * a.n_q_heads + hq) * QA_HD) + lane;
            const int64_t stride = (int64_t)a.n_q_heads * (QA_HD / 4);  // float4s between splits
            auto acc = [&](float fu, const float4& ov) {
                x[0] = __builtin_fmaf(ov.x, fu, x[0]);
                x[1] = __builtin_fmaf(ov.y, fu, x[1]);
                x[2] = __builtin_fmaf(ov.z, fu, x[2]);
                x[3] = __builtin_fmaf(ov.w, fu, x[3]);
            };
            int u = 0;
            for (; u + 4 <= n; u += 4) {
                const float4 o0 = po[u * stride], o1 = po[(u + 1) * stride];
                const float4 o2 = po[(u + 2) * stride], o3 = po[(u + 3) * stride];
                acc(__shfl(f, u, 64), o0);
                acc(__shfl(f, u + 1, 64), o1);
                acc(__shfl(f, u + 2, 64), o2);
                acc(__shfl(f, u + 3, 64), o3);
            }
            for (; u < n; u++) acc(__shfl(f, u, 64), po[u * stride]);
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int i = 0; i < 4; i++) x[i] *= inv;
        fwht256_wave(x, lane);
    }
    reinterpret_cast<float4*>(a.out + row * QA_HD)[lane] = make_float4(x[0], x[1], x[2], x[3]);
    if (a.lse && lane == 0) a.lse[row] = mx == -INFINITY ? -INFINITY : (mx + __log2f(L)) * QA_LN2;
}

template <int G>
hipError_t launch_attn_g(const kvq_q4_cache& c, const kvq_q4_attn_args& a, const Q4Plan& p, hipStream_t st) {
    const int64_t grid = p.items_per_xcd * QA_NXCD;
    hipLaunchKernelGGL(k_q4_attn_mx<G>, dim3((unsigned)grid), dim3(QA_WAVES * 64), 0, st, c, a, p);
    return hipGetLastError();
}

}  // namespace

int64_t q4_attn_workspace_bytes(const kvq_q4_cache& c, const kvq_q4_attn_args& a) {
    int64_t n = 0;
    q4_make_plan(c, a, nullptr, &n);
    return n;
}

hipError_t launch_decode_attn_q4_0(const kvq_q4_cache& c, const kvq_q4_attn_args& a, void* ws, hipStream_t st) {
    const Q4Plan p = q4_make_plan(c, a, ws, nullptr);
    const int64_t rows_q = (int64_t)a.n_seqs * a.n_q_heads;
    hipLaunchKernelGGL(k_q4_prep, dim3((unsigned)(1 + (rows_q + 3) / 4)), dim3(256), 0, st, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (p.group) {
        case 1: e = launch_attn_g<1>(c, a, p, st); break;
        case 2: e = launch_attn_g<2>(c, a, p, st); break;
        case 4: e = launch_attn_g<4>(c, a, p, st); break;
        case 8:
        case 16: e = launch_attn_g<QA_GMAX>(c, a, p, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_q4_merge, dim3((unsigned)((rows_q + 3) / 4)), dim3(256), 0, st, a, p);
    return hipGetLastError();
}

}  // namespace kvq
