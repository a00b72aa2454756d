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
//          lanes), folds sm_scale * log2(e) into it and writes the 8 block sums;
//   attn   one workgroup per (T-split, KV head), XCD-grouped so that the KV
//          heads of one split (adjacent 144-byte head-rows of the same cells)
//          share an L2; four waves take contiguous quarters of the split in
//          tiles of 64 positions; partial (m, l, O) per query head;
//   merge  one wave per (sequence, query head): combine the splits, divide,
//          rotate back, write out and lse.
//
// attn, per 64-position tile of a wave:
//   * lane = position: page-table lookup, the K and V head-rows (nine 16-byte
//     loads each) for the next tile are issued before this tile's arithmetic;
//   * scores, lane = position: per block, sum_j nibble_j * q~_j over the 32
//     elements with q~ broadcast from LDS, then d * (sum - 8 * sum_j q~_j), so
//     each element costs one byte-to-float conversion and G fmas;
//   * online softmax in the log2 domain per query head;
//   * values: the tile's V head-rows go to the wave's LDS slice regrouped so
//     that every read is aligned (nibble bytes of block b at 16b, scales at
//     128); a lane owns 8 output elements (4 nibble bytes of one block) over
//     the positions of one parity, O += (p d) * nibble with p from LDS, plus a
//     per-head sum of p d for the -8 term, folded into O at the end of every
//     tile (so the offset codes' large, nearly cancelling sums never span more
//     than one tile's 32 positions per lane); the two parities are added
//     across the wave halves.
// The arithmetic stays on the vector ALU: about 9 * G + 12 wave64
// instructions per position and KV head (scores 4 * G + 5.6, values
// 5 * G + 6.5), which at G = 4 query heads per KV head outweighs the 288 HBM
// bytes of the two head-rows; the matrix cores (a K = 32 step per block for
// the scores, a V operand transposed through LDS for the values) are the way
// past that bound.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int QA_WAVES = 4;
constexpr int QA_TILE = 64;   // positions per wave tile (one per lane)
constexpr int QA_HD = 256;    // head_dim
constexpr int QA_RB = 144;    // bytes per head-row: 8 blocks of 18
constexpr int QA_NXCD = 8;
// Query heads per workgroup at most: larger groups split over workgroups that
// read the same head-rows (neighbouring items, so from the same L2).  Eight
// heads per workgroup fill all 256 registers and took 1.5 x the time of two
// workgroups of four.
constexpr int QA_GMAX = 4;
constexpr float QA_LOG2E = 1.4426950408889634f;
constexpr float QA_LN2 = 0.6931471805599453f;

struct Q4Plan {
    int64_t* chunk_prefix;  // [n_seqs + 1]
    float* q_rot;           // [n_seqs][n_q][256]: H q / 16 * sm_scale * log2(e)
    float* q_bsum;          // [n_seqs][n_q][8]: block sums of q_rot
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
    p.q_rot = (float*)take(sizeof(float) * rows_q * QA_HD);
    p.q_bsum = (float*)take(sizeof(float) * rows_q * 8);
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
    const int64_t row = (int64_t)(blockIdx.x - 1) * 4 + (tid >> 6);
    if (row >= (int64_t)a.n_seqs * a.n_q_heads) return;
    const float4 v = reinterpret_cast<const float4*>(a.q + row * QA_HD)[lane];
    float x[4] = {v.x, v.y, v.z, v.w};
    fwht256_wave(x, lane);
    const float sc = a.sm_scale * QA_LOG2E;
#pragma unroll
    for (int i = 0; i < 4; i++) x[i] *= sc;
    reinterpret_cast<float4*>(p.q_rot + row * QA_HD)[lane] = make_float4(x[0], x[1], x[2], x[3]);
    // block b = elements 32b .. 32b+31 = lanes 8b .. 8b+7
    float bs = (x[0] + x[1]) + (x[2] + x[3]);
    bs += shfl_xor_f(bs, 1);
    bs += shfl_xor_f(bs, 2);
    bs += shfl_xor_f(bs, 4);
    if ((lane & 7) == 0) p.q_bsum[row * 8 + (lane >> 3)] = bs;
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

template <int G>
struct Q4AttnShared {
    float q[G][QA_HD];
    float qb[G][8];
    uint8_t v[QA_WAVES][QA_TILE][QA_RB];
    float pr[QA_WAVES][QA_TILE][G];
    float m[QA_WAVES][G];
    float l[QA_WAVES][G];
};

// Bytes 4W .. 4W+3 of block B's nibbles: elements 4W .. 4W+3 (low nibbles) and
// 16 + 4W .. 16 + 4W + 3 (high nibbles) against the broadcast rotated queries.
template <int G, int B, int W>
__device__ __forceinline__ void qk_word(const uint32_t (&k)[36], const Q4AttnShared<G>& sh, float (&acc)[G]) {
    const uint32_t x = row_dw<18 * B + 2 + 4 * W>(k);
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    float nl[4], nh[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        nl[e] = (float)((lo >> (8 * e)) & 0xFFu);
        nh[e] = (float)((hi >> (8 * e)) & 0xFFu);
    }
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float4 ql = *reinterpret_cast<const float4*>(&sh.q[h][32 * B + 4 * W]);
        const float4 qh = *reinterpret_cast<const float4*>(&sh.q[h][32 * B + 16 + 4 * W]);
        float t = acc[h];
        t = __builtin_fmaf(nl[0], ql.x, t);
        t = __builtin_fmaf(nl[1], ql.y, t);
        t = __builtin_fmaf(nl[2], ql.z, t);
        t = __builtin_fmaf(nl[3], ql.w, t);
        t = __builtin_fmaf(nh[0], qh.x, t);
        t = __builtin_fmaf(nh[1], qh.y, t);
        t = __builtin_fmaf(nh[2], qh.z, t);
        t = __builtin_fmaf(nh[3], qh.w, t);
        acc[h] = t;
    }
}

// Block B of the K head-row: sc += d * (sum_j nibble_j q~_j - 8 sum_j q~_j).
template <int G, int B>
__device__ __forceinline__ void qk_block(const uint32_t (&k)[36], const Q4AttnShared<G>& sh, float (&sc)[G]) {
    const float d = half_bits_to_f32(row_dw<18 * B>(k));
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0.0f;
    qk_word<G, B, 0>(k, sh, acc);
    qk_word<G, B, 1>(k, sh, acc);
    qk_word<G, B, 2>(k, sh, acc);
    qk_word<G, B, 3>(k, sh, acc);
#pragma unroll
    for (int h = 0; h < G; h++) sc[h] = __builtin_fmaf(d, __builtin_fmaf(-8.0f, sh.qb[h][B], acc[h]), sc[h]);
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

template <int G>
__global__ __launch_bounds__(QA_WAVES * 64) void k_q4_attn(kvq_q4_cache c, kvq_q4_attn_args a, Q4Plan p) {
    __shared__ __align__(16) Q4AttnShared<G> sh;
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

    // rotated queries of the G heads and their block sums
    for (int i = tid; i < G * QA_HD / 4; i += QA_WAVES * 64)
        reinterpret_cast<float4*>(&sh.q[0][0])[i] = reinterpret_cast<const float4*>(p.q_rot + qrow0 * QA_HD)[i];
    if (tid < G * 8) (&sh.qb[0][0])[tid] = p.q_bsum[qrow0 * 8 + tid];
    __syncthreads();

    const int64_t quarter = ((r1 - r0 + QA_WAVES - 1) / QA_WAVES + QA_TILE - 1) / QA_TILE * QA_TILE;
    const int64_t w0 = r0 + wave * quarter;
    const int64_t w1 = min(r1, w0 + quarter);

    // position -> cell; false where the page column, entry or cell is missing
    const int64_t cap = (int64_t)c.max_pages * c.page_size;
    const int32_t* __restrict__ tab = c.block_table + (int64_t)s * c.max_pages;
    auto cell_of = [&](int64_t pos, int64_t& cell) {
        if (pos >= cap) return false;
        const int64_t col = pos / c.page_size;
        const int32_t pg = tab[col];
        cell = (int64_t)pg * c.page_size + (pos - col * c.page_size);
        return pg >= 0 && cell < c.n_cells;
    };
    auto load_rows = [&](int64_t t0, uint4 (&kr)[9], uint4 (&vr)[9]) {
        const int64_t pos = t0 + lane;
        int64_t cell = 0;
        const bool ok = pos < w1 && cell_of(pos, cell);
        const int64_t off = ((ok ? cell : 0) * c.n_kv_heads + g) * QA_RB;
        const uint4* kp = reinterpret_cast<const uint4*>(c.k_pool + off);
        const uint4* vp = reinterpret_cast<const uint4*>(c.v_pool + off);
        const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;  // a missing position reads as zeros
#pragma unroll
        for (int i = 0; i < 9; i++) {
            const uint4 kv = kp[i], vv = vp[i];
            kr[i] = make_uint4(kv.x & keep, kv.y & keep, kv.z & keep, kv.w & keep);
            vr[i] = make_uint4(vv.x & keep, vv.y & keep, vv.z & keep, vv.w & keep);
        }
        return ok;
    };

    float m[G], lp[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = -INFINITY;
        lp[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) o[h][e] = 0.0f;
    }
    const bool any_cells = c.n_cells > 0;
    uint4 kn[9], vn[9];
#pragma unroll
    for (int i = 0; i < 9; i++) kn[i] = vn[i] = make_uint4(0, 0, 0, 0);  // no cells: every row reads as zeros
    bool okn = false;
    if (w0 < w1 && any_cells) okn = load_rows(w0, kn, vn);
    // value lane: positions of parity vh, block vb, nibble bytes 4 vk .. 4 vk + 3
    const int vh = lane >> 5, vb = (lane & 31) >> 2, vk = lane & 3;
    for (int64_t t0 = w0; t0 < w1; t0 += QA_TILE) {
        const int nt = (int)min((int64_t)QA_TILE, w1 - t0);
        uint32_t k[36], vw[36];
#pragma unroll
        for (int i = 0; i < 9; i++) {
            k[4 * i] = kn[i].x;
            k[4 * i + 1] = kn[i].y;
            k[4 * i + 2] = kn[i].z;
            k[4 * i + 3] = kn[i].w;
            vw[4 * i] = vn[i].x;
            vw[4 * i + 1] = vn[i].y;
            vw[4 * i + 2] = vn[i].z;
            vw[4 * i + 3] = vn[i].w;
        }
        stage_v_row(vw, &sh.v[wave][lane][0]);
        const bool ok = okn;
        if (t0 + QA_TILE < w1 && any_cells) okn = load_rows(t0 + QA_TILE, kn, vn);

        // scores (log2 domain), lane = position
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; h++) sc[h] = 0.0f;
        qk_block<G, 0>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 1>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 2>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 3>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 4>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 5>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 6>(k, sh, sc);
        __builtin_amdgcn_sched_barrier(0);
        qk_block<G, 7>(k, sh, sc);

        // online softmax per head; p to LDS
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float sv = ok ? sc[h] : -INFINITY;
            const float mn = fmaxf(m[h], wave_max(sv));
            float pv = 0.0f, alpha = 1.0f;
            if (mn != -INFINITY) {  // wave-uniform
                alpha = exp2f(m[h] - mn);
                pv = exp2f(sv - mn);
            }
            m[h] = mn;
            lp[h] = __builtin_fmaf(lp[h], alpha, pv);
#pragma unroll
            for (int e = 0; e < 8; e++) o[h][e] *= alpha;
            sh.pr[wave][lane][h] = pv;
        }

        // values: lane = elements 32 vb + 4 vk + {0..3} and 32 vb + 16 + 4 vk + {0..3} over the
        // positions of parity vh (rows past nt are zero with p = 0, so the pair loop may read one);
        // cs = this tile's sum of p d, the weight of the -8 offset, folded in below
        float cs[G];
#pragma unroll
        for (int h = 0; h < G; h++) cs[h] = 0.0f;
#pragma unroll 4
        for (int tt = 0; tt < nt; tt += 2) {
            const int t = tt + vh;
            const uint8_t* vrow = &sh.v[wave][t][0];
            const uint32_t x = *reinterpret_cast<const uint32_t*>(vrow + 16 * vb + 4 * vk);
            const float d = half_bits_to_f32(*reinterpret_cast<const uint16_t*>(vrow + 128 + 2 * vb));
            const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
            float n[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                n[e] = (float)((lo >> (8 * e)) & 0xFFu);
                n[4 + e] = (float)((hi >> (8 * e)) & 0xFFu);
            }
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float wgt = sh.pr[wave][t][h] * d;
#pragma unroll
                for (int e = 0; e < 8; e++) o[h][e] = __builtin_fmaf(wgt, n[e], o[h][e]);
                cs[h] += wgt;
            }
        }
        // sum p d (nibble - 8) = sum p d nibble - 8 sum p d, once per tile
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int e = 0; e < 8; e++) o[h][e] = __builtin_fmaf(-8.0f, cs[h], o[h][e]);
    }
    // the two position parities
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int e = 0; e < 8; e++) o[h][e] += xor_lane<32>(o[h][e], lane);

    // wave states -> LDS, then combine the four waves per query head
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float l = wave_sum(lp[h]);
        if (lane == 0) {
            sh.m[wave][h] = m[h];
            sh.l[wave][h] = l;
        }
    }
    __syncthreads();  // every wave is past its last read of sh.v and sh.pr
    float* ob = reinterpret_cast<float*>(&sh.v[0][0][0]);  // [QA_WAVES][G][256] when it fits
    constexpr int HB = (int)(sizeof(sh.v) / (sizeof(float) * QA_WAVES * QA_HD));  // heads that fit per pass
    constexpr int HPASS = G <= 8 ? G : 8;                                          // heads per exchange pass
    static_assert(HPASS <= HB && G % HPASS == 0, "exchange buffer");
    const int e0 = 32 * vb + 4 * vk;
    for (int hb = 0; hb < G; hb += HPASS) {
        if (vh == 0) {
#pragma unroll
            for (int hh = 0; hh < HPASS; hh++) {
                const int h = hb + hh;
                float* dst = ob + ((int64_t)wave * HPASS + hh) * QA_HD;
                *reinterpret_cast<float4*>(dst + e0) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
                *reinterpret_cast<float4*>(dst + e0 + 16) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
            }
        }
        __syncthreads();
        for (int hh = 0; hh < HPASS; hh++) {
            const int h = hb + hh;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < QA_WAVES; w++) mx = fmaxf(mx, sh.m[w][h]);
            float L = 0.0f, O = 0.0f;
#pragma unroll
            for (int w = 0; w < QA_WAVES; w++) {
                const float f = mx == -INFINITY ? 0.0f : exp2f(sh.m[w][h] - mx);
                L = __builtin_fmaf(sh.l[w][h], f, L);
                O = __builtin_fmaf(ob[((int64_t)w * HPASS + hh) * QA_HD + tid], f, O);
            }
            const int64_t prow = ch * a.n_q_heads + hq0 + h;
            p.part_o[prow * QA_HD + tid] = O;
            if (tid == 0) {
                p.part_m[prow] = mx;
                p.part_l[prow] = L;
            }
        }
        __syncthreads();
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
    hipLaunchKernelGGL(k_q4_attn<G>, dim3((unsigned)grid), dim3(QA_WAVES * 64), 0, st, c, a, p);
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
        case 4:
        case 8:
        case 16: e = launch_attn_g<QA_GMAX>(c, a, p, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_q4_merge, dim3((unsigned)((rows_q + 3) / 4)), dim3(256), 0, st, a, p);
    return hipGetLastError();
}

}  // namespace kvq
