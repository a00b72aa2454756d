// kvq_attn.hip -- absorbed-MLA decode attention over quantized latent rows
// (gfx950).
//
// What is computed (colibri PR #399 "KV cache quantization: fp8 (KV8) + 4-bit
// TurboQuant (KV_TQ) ...": commit 6, the fused decode with a 3-way qmode --
// score a_score8 and context a_clat8 over fp8 rows; commit 2, split-T kernels;
// "Ready for review", the native 4-bit consumer: rotate q once per head, dot the
// codes through the codebook, un-rotate the weighted sum):
//
//   s_t = sm * (rho_t <q, c_t> + <q_rope, k_rope_t>),  p = softmax(s),
//   o   = sum_t p_t rho_t c_t
//
// where c_t is the decoded code row (fp8: e4m3 values, rho_t = scale; the
// rotated codec at 3, 4 or 6 bits (TQ3/TQ4/TQ6): the codebook levels, rho_t =
// radius / sqrt(512), q replaced by R q, and o un-rotated by R^T after the
// merge).  The latent rows are never rebuilt.
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   prep  -- fp32 check path: k_plan (per-sequence T-split counts -> prefix)
//            and, rotated codec, k_qrot (R q in fp32); matrix-core path:
//            k_qprep_fp8 / k_qprep_tq4 (the query as fp16 operands, R q for
//            the rotated codec).  The matrix-core split kernels plan their
//            chunk themselves;
//   split -- k_attn_*: online softmax over every T-split, partial (m, l, O);
//   merge -- k_merge / k_merge_f8: combine the splits (un-rotation for the
//            rotated codec), write out / lse.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_codebook.inc"

namespace kvq {

namespace {

__constant__ uint32_t c_tq4_level[16] = KVQ_TQ4_LEVEL_BITS;
__constant__ uint32_t c_tq3_level[8] = KVQ_TQ3_LEVEL_BITS;
__constant__ uint32_t c_tq6_level[64] = KVQ_TQ6_LEVEL_BITS;

constexpr int DL = 512;  // latent width
constexpr int DR = 64;   // rope width
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float INV_SQRT_DL = 0.044194173824159216f;  // 1 / sqrt(512)

constexpr int F32_HEADS = 8;      // fp32 path: heads per workgroup
constexpr int MF_HEADS = 16;      // matrix-core path: heads per workgroup (one MFMA N block)
constexpr int MF_WAVES = 4;       // matrix-core path: waves per workgroup, splitting the rows
constexpr int MF_TILE = 32;       // rows per wave tile
constexpr int TQ_HEADS = 64;      // rotated codec, matrix-core path: heads per workgroup (4 waves x 16)
constexpr int QPACK_U4 = 80;      // fp8: uint4 per prepared query (fp16 latent 64, rope hi 8, rope lo 8)
constexpr int QPACK_TQ = 144;     // rotated codec: the same, then the fp16 latent remainder (64)
// rotated codec: slots (of 64 uint4, one per lane) of a 16-head block of the pack
constexpr int QS_RH = 16, QS_RL = 18, QS_LL = 20;
constexpr int F8_HEADS = 32;      // fp8 matrix-core path: heads per workgroup (one 32x32 MFMA N block)
constexpr int F8_TILE = 128;      // fp8 matrix-core path: rows per workgroup tile (32 per wave)
constexpr int N_XCD = 8;          // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr float LAZY_LOG2 = 8.0f; // running-max slack before the accumulators are rescaled

struct Plan {
    int64_t* chunk_prefix;  // [n_seqs + 2]: chunk prefix; fp8 matrix-core path: tile prefix, total, quota
    float* q_rot;           // fp32 path, rotated codec: [n_seqs][H][512]
    uint4* q_pack;          // matrix-core paths: [n_seqs][H padded][QPACK_U4 or QPACK_TQ], in the split
                            // kernel's operand order per group of 32 (fp8) or 16 (rotated codec) heads
    float* q_inv;           // matrix-core paths: [n_seqs][H padded]
    float* part_m;          // [max_chunks][H]
    float* part_l;          // [max_chunks][H]
    float* part_o;          // fp32 path: f32 [max_chunks][H][512]
    uint16_t* part_h;       // matrix-core paths: fp16 O * 2^k, same order as part_o would be
    float* part_s;          // matrix-core paths: [max_chunks][4][H], 2^-k of each 128-dim quarter
    int64_t max_chunks;
    int split_rows;
    int heads_per_group;
    int n_groups;
    int heads_padded;
    int64_t chunks_per_xcd; // matrix-core grid: chunk c runs on XCD c % 8, all its head groups together
    // fp8 matrix-core path: each head group's F8_TILE-row tiles (every sequence's, in order) are
    // dealt in runs of tile_quota to n_work work items; a work item writes one partial state per
    // sequence it touches, in slot (work item + sequence), so max_chunks = n_work + n_seqs
    int64_t n_work;
    int64_t n_tiles;        // one sequence: the tile count (several: computed by the preparation)
    int64_t tile_quota;     // 0: the preparation computes max(1, ceil(tiles / n_work))
    int64_t one_slots;      // one sequence: its partial-state slots, ceil(n_tiles / tile_quota)
    // sparse decode on the fp8 matrix-core path: logical row t of the index list is cache row
    // clamp(row_index[t], 0, cache_rows - 1), read in place (null: the rows are contiguous)
    const int64_t* row_index;
    int64_t cache_rows;
};

// ---- workspace plan ------------------------------------------------------------

int auto_split_rows(const kvq_attn_args& a) {
    if (a.precision == KVQ_PREC_FP32) return 512;
    if (qmode_rotated(a.qmode)) {
        // one workgroup per compute unit over all splits and groups of 64 heads,
        // whole tiles, at least 8 tiles per split
        const int64_t groups = (a.n_heads + TQ_HEADS - 1) / TQ_HEADS;
        int64_t split = (a.total_rows * groups + 255) / 256;
        if (split < 8 * MF_TILE) split = 8 * MF_TILE;
        split = (split + MF_TILE - 1) / MF_TILE * MF_TILE;
        if (split > (1 << 24)) split = 1 << 24;
        return (int)split;
    }
    return F8_TILE;  // fp8 matrix-core path: work items of whole tiles (see make_plan)
}

Plan make_plan(const kvq_attn_args& a, void* ws, int64_t* bytes_out) {
    Plan p{};
    p.split_rows = a.split_rows > 0 ? a.split_rows : auto_split_rows(a);
    const bool f32 = a.precision == KVQ_PREC_FP32;
    p.heads_per_group = f32 ? F32_HEADS : (qmode_rotated(a.qmode) ? TQ_HEADS : F8_HEADS);
    p.n_groups = (a.n_heads + p.heads_per_group - 1) / p.heads_per_group;
    p.heads_padded = p.n_groups * p.heads_per_group;
    // sum_s max(1, ceil(T_s / split)) over T_s summing to at most total_rows is at
    // most floor(total / split) + n_seqs, and at most ceil(total / split) + n_seqs - 1
    // unless every sequence is empty
    p.max_chunks = std::max<int64_t>(a.n_seqs, std::min<int64_t>(a.total_rows / p.split_rows + a.n_seqs,
                                                                  (a.total_rows + p.split_rows - 1) / p.split_rows +
                                                                      a.n_seqs - 1));
    if (!f32 && a.qmode == KVQ_QMODE_FP8) {
        // one work item per compute unit over the head groups (at least two tiles each), or
        // split_rows / F8_TILE tiles each when the caller fixes it
        const int64_t ub = (a.total_rows + F8_TILE - 1) / F8_TILE + a.n_seqs;  // >= sum_s ceil(T_s / F8_TILE)
        if (a.split_rows > 0) {
            p.tile_quota = (a.split_rows + F8_TILE - 1) / F8_TILE;
            p.n_work = std::max<int64_t>(1, (ub + p.tile_quota - 1) / p.tile_quota);
        } else {
            p.tile_quota = 0;
            p.n_work = std::max<int64_t>(1, std::min<int64_t>(256 / p.n_groups, (ub + 1) / 2));
        }
        if (a.n_seqs == 1) {
            p.n_tiles = (a.total_rows + F8_TILE - 1) / F8_TILE;
            if (p.tile_quota == 0) p.tile_quota = std::max<int64_t>(1, (p.n_tiles + p.n_work - 1) / p.n_work);
            p.one_slots = (p.n_tiles + p.tile_quota - 1) / p.tile_quota;
        }
        p.max_chunks = p.n_work + a.n_seqs;
        p.chunks_per_xcd = (p.n_work + N_XCD - 1) / N_XCD;
    } else {
        p.chunks_per_xcd = (p.max_chunks + N_XCD - 1) / N_XCD;
    }
    auto align = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
    int64_t off = 0;
    char* base = (char*)ws;
    auto take = [&](int64_t bytes) {
        char* q = base ? base + off : nullptr;
        off = align(off + bytes);
        return q;
    };
    p.chunk_prefix = (int64_t*)take(sizeof(int64_t) * (a.n_seqs + 2));
    if (f32 && qmode_rotated(a.qmode)) p.q_rot = (float*)take(sizeof(float) * (int64_t)a.n_seqs * a.n_heads * DL);
    if (!f32) {  // matrix-core paths: the prepared query operands
        const int64_t rows_q = (int64_t)a.n_seqs * p.heads_padded;
        p.q_pack = (uint4*)take(sizeof(uint4) * rows_q * (qmode_rotated(a.qmode) ? QPACK_TQ : QPACK_U4));
        p.q_inv = (float*)take(sizeof(float) * rows_q);
    }
    p.part_m = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    p.part_l = (float*)take(sizeof(float) * p.max_chunks * a.n_heads);
    // (fp8 matrix-core partials are stored per group of 32 heads, the last one padded)
    const int64_t ph = (!f32 && a.qmode == KVQ_QMODE_FP8) ? p.heads_padded : a.n_heads;
    if (f32) {
        p.part_o = (float*)take(sizeof(float) * p.max_chunks * ph * DL);
    } else {
        p.part_h = (uint16_t*)take(sizeof(uint16_t) * p.max_chunks * ph * DL);
        p.part_s = (float*)take(sizeof(float) * p.max_chunks * 4 * a.n_heads);
    }
    if (bytes_out) *bytes_out = off;
    return p;
}

int64_t plan_bytes(const kvq_attn_args& a) {
    int64_t n = 0;
    make_plan(a, nullptr, &n);
    return n;
}

// ---- 0. plan -----------------------------------------------------------------------
// chunk_prefix[s] = sum_{s' < s} max(1, ceil(T_s' / split)); one workgroup.
__global__ __launch_bounds__(256) void k_plan(const int64_t* __restrict__ seq_offsets, int n_seqs, int split,
                                             int64_t total_rows, int64_t* __restrict__ chunk_prefix) {
    __shared__ int64_t part[256];
    const int tid = threadIdx.x;
    const int per = (n_seqs + 255) / 256;
    const int s0 = tid * per, s1 = min(n_seqs, s0 + per);
    int64_t local = 0;
    for (int s = s0; s < s1; s++) {
        const int64_t T = min(seq_offsets[s + 1], total_rows) - max(seq_offsets[s], (int64_t)0);
        local += T > 0 ? (T + split - 1) / split : 1;
    }
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan
        const int64_t v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t run = tid > 0 ? part[tid - 1] : 0;
    for (int s = s0; s < s1; s++) {
        chunk_prefix[s] = run;
        const int64_t T = min(seq_offsets[s + 1], total_rows) - max(seq_offsets[s], (int64_t)0);
        run += T > 0 ? (T + split - 1) / split : 1;
    }
    if (tid == 255) chunk_prefix[n_seqs] = part[255];
}

__device__ __forceinline__ int find_chunk_seq(const int64_t* __restrict__ cp, int n_seqs, int64_t c) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cp[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---- 1a. query rotation of the rotated codec (fp32 path) ----------------------------------------------------------
// One wave per (sequence, head): q~ = H (D q) / sqrt(512), 8 consecutive per lane.
__global__ __launch_bounds__(256) void k_qrot(const float* __restrict__ q, const uint8_t* __restrict__ sign_mask,
                                             int64_t n_rows, float* __restrict__ q_rot) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* src = q + row * DL + lane * 8;
    float v[8];
    const uint32_t sm = sign_mask[lane];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = ((sm >> i) & 1u) ? -src[i] : src[i];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (!(i & h)) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = fwht_xlane(v[i], lane, m);
    float* dst = q_rot + row * DL + lane * 8;
#pragma unroll
    for (int i = 0; i < 8; i++) dst[i] = v[i] * INV_SQRT_DL;
}

// Decoded value of element i of a code row (fp8: e4m3 value; rotated codec:
// codebook level of index i, bits B*i .. B*i + B - 1 of the row's little-endian
// bit stream).  The second byte is read only when the index crosses into it, so
// the last index of a row reads nothing past the row.
template <int QMODE>
__device__ __forceinline__ float code_value(const uint8_t* __restrict__ row, int i) {
    if (QMODE == KVQ_QMODE_FP8) return e4m3_to_f32(row[i]);
    if (QMODE == KVQ_QMODE_TQ4) {
        const uint32_t b = row[i >> 1];
        return u2f(c_tq4_level[(i & 1) ? (b >> 4) : (b & 15u)]);
    }
    constexpr int B = QMODE == KVQ_QMODE_TQ3 ? 3 : 6;
    const int pos = B * i, sh = pos & 7;
    uint32_t w = row[pos >> 3];
    if (sh + B > 8) w |= (uint32_t)row[(pos >> 3) + 1] << 8;
    const uint32_t idx = (w >> sh) & ((1u << B) - 1u);
    return u2f(B == 3 ? c_tq3_level[idx] : c_tq6_level[idx]);
}

// ---- 2a. fp32 check path ----------------------------------------------------------------
// Workgroup = (chunk, group of 8 heads), 256 threads.  Tiles of 256 rows: one
// row per thread for the scores, then thread (head = tid/32, 16 dims) for PV.
template <int QMODE>
__global__ __launch_bounds__(256) void k_attn_f32(kvq_attn_args a, Plan p, const float* __restrict__ qsrc) {
    constexpr int TILE = 256;
    __shared__ float q_s[F32_HEADS][DL];
    __shared__ float qr_s[F32_HEADS][DR];
    __shared__ float pr_s[F32_HEADS][TILE];  // scores, then p * rho
    __shared__ float red_s[F32_HEADS][2];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;
    if (c >= p.max_chunks || c >= p.chunk_prefix[a.n_seqs]) return;
    const int s = find_chunk_seq(p.chunk_prefix, a.n_seqs, c);
    const int64_t seq_lo = max(a.seq_offsets[s], (int64_t)0), seq_hi = min(a.seq_offsets[s + 1], a.total_rows);
    const int64_t r0 = seq_lo + (c - p.chunk_prefix[s]) * p.split_rows;
    const int64_t r1 = min(seq_hi, r0 + (int64_t)p.split_rows);
    const int h0 = blockIdx.y * F32_HEADS;
    const int nh = min(F32_HEADS, a.n_heads - h0);
    for (int i = tid; i < F32_HEADS * DL; i += 256) {
        const int hh = i / DL, d = i % DL;
        q_s[hh][d] = hh < nh ? qsrc[((int64_t)s * a.n_heads + h0 + hh) * DL + d] : 0.0f;
    }
    for (int i = tid; i < F32_HEADS * DR; i += 256) {
        const int hh = i / DR, d = i % DR;
        qr_s[hh][d] = hh < nh ? a.q_rope[((int64_t)s * a.n_heads + h0 + hh) * DR + d] : 0.0f;
    }
    __syncthreads();
    constexpr int cb = QMODE == KVQ_QMODE_FP8 ? DL : DL * (QMODE == KVQ_QMODE_TQ3 ? 3 : QMODE == KVQ_QMODE_TQ6 ? 6 : 4) / 8;
    const int ph = tid >> 5, pd = (tid & 31) * 16;       // PV ownership
    float m_run[F32_HEADS], l_run[F32_HEADS];
#pragma unroll
    for (int hh = 0; hh < F32_HEADS; hh++) { m_run[hh] = -INFINITY; l_run[hh] = 0.0f; }
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; j++) acc[j] = 0.0f;
    for (int64_t t0 = r0; t0 < r1; t0 += TILE) {
        const int nt = (int)min((int64_t)TILE, r1 - t0);
        float sc[F32_HEADS];
        float rho = 0.0f;
        if (tid < nt) {
            const int64_t t = t0 + tid;
            rho = a.row_scale[t];
            if (QMODE != KVQ_QMODE_FP8) rho *= INV_SQRT_DL;
            const uint8_t* row = a.codes + t * cb;
            float dot[F32_HEADS], dr[F32_HEADS];
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) { dot[hh] = 0.0f; dr[hh] = 0.0f; }
            for (int d = 0; d < DL; d++) {
                const float x = code_value<QMODE>(row, d);
#pragma unroll
                for (int hh = 0; hh < F32_HEADS; hh++) dot[hh] = __builtin_fmaf(q_s[hh][d], x, dot[hh]);
            }
            const uint16_t* kr = a.k_rope + t * DR;
            for (int d = 0; d < DR; d++) {
                const float x = u2f((uint32_t)kr[d] << 16);
#pragma unroll
                for (int hh = 0; hh < F32_HEADS; hh++) dr[hh] = __builtin_fmaf(qr_s[hh][d], x, dr[hh]);
            }
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) sc[hh] = a.sm_scale * (rho * dot[hh] + dr[hh]);
        } else {
#pragma unroll
            for (int hh = 0; hh < F32_HEADS; hh++) sc[hh] = -INFINITY;
        }
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) pr_s[hh][tid] = sc[hh];
        __syncthreads();
        {  // tile max per head: 32 threads per head
            const int hh = tid >> 5, l32 = tid & 31;
            float mx = -INFINITY;
            for (int k = l32; k < TILE; k += 32) mx = fmaxf(mx, pr_s[hh][k]);
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
            if (l32 == 0) red_s[hh][0] = mx;
        }
        __syncthreads();
        float alpha[F32_HEADS], m_new[F32_HEADS];
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            m_new[hh] = fmaxf(m_run[hh], red_s[hh][0]);
            alpha[hh] = m_new[hh] == -INFINITY ? 1.0f : expf(m_run[hh] - m_new[hh]);
        }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            const float pv = tid < nt ? expf(sc[hh] - m_new[hh]) : 0.0f;
            pr_s[hh][tid] = pv;
        }
        __syncthreads();
        {  // tile sum of p per head
            const int hh = tid >> 5, l32 = tid & 31;
            float sm = 0.0f;
            for (int k = l32; k < TILE; k += 32) sm += pr_s[hh][k];
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) sm += __shfl_xor(sm, o, 32);
            if (l32 == 0) red_s[hh][1] = sm;
        }
        __syncthreads();
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) {
            l_run[hh] = l_run[hh] * alpha[hh] + red_s[hh][1];
            m_run[hh] = m_new[hh];
        }
        // p * rho for PV
#pragma unroll
        for (int hh = 0; hh < F32_HEADS; hh++) pr_s[hh][tid] *= rho;
        __syncthreads();
        // PV: thread owns head ph, dims pd .. pd+15
        {
            float al = alpha[0];
#pragma unroll
            for (int hh = 1; hh < F32_HEADS; hh++) if (hh == ph) al = alpha[hh];
#pragma unroll
            for (int j = 0; j < 16; j++) acc[j] *= al;
            for (int k = 0; k < nt; k++) {
                const float w = pr_s[ph][k];
                const uint8_t* row = a.codes + (t0 + k) * cb;
#pragma unroll
                for (int j = 0; j < 16; j++) acc[j] = __builtin_fmaf(w, code_value<QMODE>(row, pd + j), acc[j]);
            }
        }
        __syncthreads();
    }
    if (ph < nh) {
        float* dst = p.part_o + (c * a.n_heads + h0 + ph) * DL + pd;
#pragma unroll
        for (int j = 0; j < 16; j++) dst[j] = acc[j];
    }
    if (tid < nh) {
        float mv = m_run[0], lv = l_run[0];
#pragma unroll
        for (int hh = 1; hh < F32_HEADS; hh++) if (hh == tid) { mv = m_run[hh]; lv = l_run[hh]; }
        p.part_m[c * a.n_heads + h0 + tid] = mv;  // natural-log units
        p.part_l[c * a.n_heads + h0 + tid] = lv;
    }
}

// ---- matrix-core path ------------------------------------------------------------------------
// Operand precision (chosen by measurement: bf16 query and probabilities cost
// 2e-3 .. 1.5e-2 of the output on these workloads, whose outputs are
// near-cancelling averages):
//  - latent codes: fp16, exact (every e4m3 value and every bf16 codebook level);
//  - latent query: per head scaled by a power of two (max |q| in [256, 512)),
//    then rounded to fp16 (fp8 rows; an emulation of this arithmetic against
//    the fp64 evaluation measures 3.4e-4, and 7.0e-4 with 50x sharper scores);
//    the TQ4 kernel also applies the fp16 remainder q - hi;
//  - rope: k_rope is bf16; the rope query is split hi + lo in bf16;
//  - probabilities p * rho_t: times a per-split power of two rs (max rho * rs in
//    [0.5, 1)), then fp16;
//  - accumulation fp32; the power-of-two scales are undone exactly in fp32.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8_t as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) { return f16_bits(lo) | (f16_bits(hi) << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Power of two 2^k with max_abs * 2^k in [2^log2_target, 2^(log2_target+1)); 1 if max_abs == 0.
__device__ __forceinline__ float pow2_scale_for(float max_abs, int log2_target) {
    if (!(max_abs > 0.0f)) return 1.0f;
    int e = (int)((f2u(max_abs) >> 23) & 255u) - 127;  // floor(log2) for normal values
    if (e < -126) e = -126;
    int k = log2_target - e;
    if (k > 127) k = 127;
    if (k < -126) k = -126;
    return u2f((uint32_t)(k + 127) << 23);
}

// Scale of a partial O stored as fp16: 2^k with max_abs * 2^k in [2^14, 2^15) (below the
// fp16 maximum 65504 after rounding), k in [-126, 126] (1 if max_abs == 0); *inv = 2^-k.
__device__ __forceinline__ float f16_store_scale(float max_abs, float* inv) {
    const uint32_t eb = min(f2u(pow2_scale_for(max_abs, 14)), 253u << 23);  // (k + 127) << 23
    *inv = u2f((254u << 23) - eb);
    return u2f(eb);
}

// Non-temporal 8-byte store and load (the fp8 path's partial states: written once in
// whole 512-byte runs per wave, read once by the merge).
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_nt(uint2* p, uint2 v) {
    __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}

// Four fp16 of a stored partial O times its 2^-k (exact unless the product leaves the
// normal range, as O itself would have).
__device__ __forceinline__ float4 f16x4_scaled(uint2 v, float s) {
    const f16x2_t a = __builtin_bit_cast(f16x2_t, v.x), b = __builtin_bit_cast(f16x2_t, v.y);
    return make_float4((float)a[0] * s, (float)a[1] * s, (float)b[0] * s, (float)b[1] * s);
}

// Two e4m3 codes (byte pair HI of w) -> two fp16, exact (hardware conversion, scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
    const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 e4m3x8_to_f16x8(uint32_t w0, uint32_t w1) {
    return make_uint4(e4m3x2_to_f16x2<false>(w0), e4m3x2_to_f16x2<true>(w0), e4m3x2_to_f16x2<false>(w1),
                      e4m3x2_to_f16x2<true>(w1));
}

// Byte tables of the fp16 bits of the 8 positive codebook levels (index 8 + m).
struct Tq4Lut {
    uint32_t lo03, lo47, hi03, hi47;
};

__device__ __forceinline__ Tq4Lut make_tq4_lut() {
    Tq4Lut t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 8; m++) {
        const uint32_t h = f16_bits(u2f(c_tq4_level[8 + m]));  // exact: 8 significant bits
        const uint32_t lo = h & 0xFF, hi = h >> 8;
        if (m < 4) { t.lo03 |= lo << (8 * m); t.hi03 |= hi << (8 * m); }
        else { t.lo47 |= lo << (8 * (m - 4)); t.hi47 |= hi << (8 * (m - 4)); }
    }
    return t;
}

// The 3-bit codebook in the same form: its 4 positive levels (index 4 + m) at
// m = 0 .. 3 (entries 4 .. 7 unused).
__device__ __forceinline__ Tq4Lut make_tq3_lut() {
    Tq4Lut t{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 4; m++) {
        const uint32_t h = f16_bits(u2f(c_tq3_level[4 + m]));
        t.lo03 |= (h & 0xFF) << (8 * m);
        t.hi03 |= (h >> 8) << (8 * m);
    }
    return t;
}

// 8 nibble indices (element k = nibble k of x) -> 8 fp16 codebook levels.  The
// codebook is symmetric: index i >= 8 is +level[i], index i < 8 is
// -level[15 - i]; the magnitude comes from a byte table lookup (v_perm).
__device__ __forceinline__ uint4 tq4x8_to_f16x8(uint32_t x, const Tq4Lut& t) {
    const uint32_t neg = ((x >> 3) & 0x11111111u) ^ 0x11111111u;  // 1 where index < 8
    const uint32_t m = (x & 0x77777777u) ^ (neg * 7u);                // magnitude index
    const uint32_t me = m & 0x0F0F0F0Fu, mo = (m >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
    const uint32_t lo_e = __builtin_amdgcn_perm(t.lo47, t.lo03, me);
    const uint32_t lo_o = __builtin_amdgcn_perm(t.lo47, t.lo03, mo);
    const uint32_t hi_e = __builtin_amdgcn_perm(t.hi47, t.hi03, me) | ((neg & 0x01010101u) << 7);
    const uint32_t hi_o = __builtin_amdgcn_perm(t.hi47, t.hi03, mo) | (((neg >> 4) & 0x01010101u) << 7);
    const uint32_t ae = __builtin_amdgcn_perm(hi_e, lo_e, 0x05010400u);  // e0 | e2 << 16
    const uint32_t ao = __builtin_amdgcn_perm(hi_o, lo_o, 0x05010400u);  // o0 | o2 << 16
    const uint32_t be = __builtin_amdgcn_perm(hi_e, lo_e, 0x07030602u);  // e4 | e6 << 16
    const uint32_t bo = __builtin_amdgcn_perm(hi_o, lo_o, 0x07030602u);  // o4 | o6 << 16
    return make_uint4(__builtin_amdgcn_perm(ao, ae, 0x05040100u), __builtin_amdgcn_perm(ao, ae, 0x07060302u),
                      __builtin_amdgcn_perm(bo, be, 0x05040100u), __builtin_amdgcn_perm(bo, be, 0x07060302u));
}


// 8 three-bit indices (element k = bits 3k .. 3k + 2 of x) -> 8 fp16 levels of
// the 8-level codebook: each index i is spread to nibble k as i + 4, which
// tq4x8_to_f16x8 reads as sign (i >= 4) and magnitude index (i - 4 or 3 - i),
// the symmetric layout of the 8 levels.
__device__ __forceinline__ uint4 tq3x8_to_f16x8(uint32_t x, const Tq4Lut& t) {
    const uint32_t y = (x & 0xFFFu) | ((x & 0xFFF000u) << 4);  // elements 4..7 to the upper half
    const uint32_t n = (y & 0x00070007u) | ((y & 0x00380038u) << 1) | ((y & 0x01C001C0u) << 2) |
                       ((y & 0x0E000E00u) << 3);
    return tq4x8_to_f16x8(n + 0x44444444u, t);
}

// 8 six-bit indices (element k = bits 6k .. 6k + 5 of the 48-bit x) -> 8 fp16
// levels of the 64-level codebook: index i >= 32 is +level[i], i < 32 is
// -level[63 - i]; the magnitude comes from lane m of tab (lane l holds the
// fp16 bits of level 32 + l % 32) through ds_bpermute.  All 64 lanes must be
// active.
__device__ __forceinline__ uint4 tq6x8_to_f16x8(uint64_t x, uint32_t tab) {
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const uint32_t i = (uint32_t)(x >> (6 * k)) & 63u;
        const uint32_t neg = (i >> 5) ^ 1u;
        const uint32_t m = (i & 31u) ^ (neg * 31u);
        h[k] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(m << 2), (int)tab) | (neg << 15);
    }
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier after this wave's LDS accesses have completed.  Unlike
// __syncthreads it does not wait for outstanding global loads (loads of later
// tiles stay in flight); the assembly is a compiler memory barrier as well.
__device__ __forceinline__ void wg_barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS DMA (global_load_lds: each lane's bytes land at the wave-uniform LDS
// base in M0 + lane * size) issued from inline assembly.  The compiler does not
// see these LDS writes, so it adds no wait of its own before the LDS reads that
// follow -- with the builtin it waits for every outstanding DMA, the next
// tile's included, before the first read of the current tile.  The kernel
// waits explicitly (vmcnt) before it reads what a DMA wrote, and finishes its
// reads of a buffer (lgkmcnt) before a DMA refills it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Scalar base + per-lane 32-bit offset form.  The global address is
// sbase + voff; the LDS address is M0 + 16 (or 4) * lane.  The compiler's
// hazard recognizer does not look inside the assembly, so each block starts
// with 5 wait states: a VALU write of an SGPR (v_readlane / v_readfirstlane,
// e.g. an SGPR reloaded from a spill lane) needs 5 before a VMEM instruction
// reads that SGPR as its base, and an SALU write of M0 needs 1 before LDS DMA.
// With fewer, the load can use a stale base register and fault.
__device__ __forceinline__ void dma_lds_b128(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}
__device__ __forceinline__ void dma_lds_b32(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}
// Per-lane 64-bit address form (rows gathered by index: every lane its own row).
__device__ __forceinline__ void dma_lds_b128_at(const void* vaddr, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(vaddr), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void dma_lds_b32_at(const void* vaddr, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off" : : "v"(vaddr), "{m0}"(lds_base) : "memory");
}
// max over the wave by lane swaps (no LDS round trips)
// (sequence, head) of a query-preparation row s * hp + head, wave-uniform: no
// division for one sequence, a 32-bit one below 2^32 rows (a 64-bit division
// is a long dependent instruction chain on the GPU).
__device__ __forceinline__ void seq_head_of(int64_t row, int n_seqs, int64_t hp, int& s, int& hd) {
    if (n_seqs == 1) {
        s = 0;
        hd = (int)row;
    } else if ((uint64_t)n_seqs * (uint64_t)hp <= 0xFFFFFFFFull) {
        const uint32_t q = (uint32_t)row / (uint32_t)hp;
        s = (int)q;
        hd = (int)((uint32_t)row - q * (uint32_t)hp);
    } else {
        s = (int)(row / hp);
        hd = (int)(row % hp);
    }
}

__device__ __forceinline__ float wave_max_swap(float v, int lane) {
    v = fmaxf(v, xor_lane<32>(v, lane));
    v = fmaxf(v, xor_lane<16>(v, lane));
    v = fmaxf(v, xor_lane<8>(v, lane));
    v = fmaxf(v, xor_lane<4>(v, lane));
    v = fmaxf(v, xor_lane<2>(v, lane));
    return fmaxf(v, xor_lane<1>(v, lane));
}
// max over the four lanes n, n ^ 16, n ^ 32, n ^ 48 (gfx950 lane-swap
// instructions: each pairs a lane with the one 16 or 32 lanes away).
__device__ __forceinline__ float max_xor16_xor32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The split plan, in-kernel (matrix-core paths), run by one wave: it scans
// max(1, ceil(T_s / split)) over the sequences, 64 at a time, and finds the
// one holding chunk c: plan_s = {first row, end row, sequence}, sequence -1
// if there is no such chunk.  The workgroup with blockIdx 0 also stores the
// prefix (chunk_prefix) for the merge.
__device__ __forceinline__ void plan_chunk(const kvq_attn_args& a, const Plan& p, int64_t c, int64_t* plan_s,
                                           int lane) {
    const bool writer = blockIdx.x == 0;
    const int64_t split = p.split_rows;
    int64_t run = 0;
    if (lane == 0) plan_s[2] = -1;
    for (int base = 0; base < a.n_seqs; base += 64) {
        const int sq = base + lane;
        int64_t cnt = 0, lo = 0, hi = 0;
        if (sq < a.n_seqs) {
            lo = max(a.seq_offsets[sq], (int64_t)0);
            hi = min(a.seq_offsets[sq + 1], a.total_rows);
            cnt = hi > lo ? (hi - lo + split - 1) / split : 1;
        }
        int64_t incl = cnt;  // inclusive scan over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        const int64_t excl = run + incl - cnt;
        const bool mine = sq < a.n_seqs && c >= excl && c < excl + cnt;  // one lane over all passes
        if (sq < a.n_seqs && writer) p.chunk_prefix[sq] = excl;
        if (mine) {
            const int64_t r0c = lo + (c - excl) * split;
            plan_s[0] = r0c;
            plan_s[1] = min(hi, r0c + split);
            plan_s[2] = sq;
        }
        run += __shfl(incl, 63, 64);
        if (!writer && __any(mine)) break;
    }
    if (writer && lane == 0) p.chunk_prefix[a.n_seqs] = run;
}

// This workgroup's chunk c: rows [r0, r1) of sequence sq; false if there is
// no such chunk (workgroup-uniform).  One sequence holds rows 0 .. total_rows - 1
// (seq_offsets[0] = 0 and seq_offsets[1] = total_rows by the interface), so its
// chunks need no loads and no barrier; otherwise wave 0 scans the offsets.
__device__ __forceinline__ bool locate_chunk(const kvq_attn_args& a, const Plan& p, int64_t c, int64_t* plan_s,
                                             int wave, int lane, int64_t& r0, int64_t& r1, int& sq) {
    if (a.n_seqs == 1) {
        const int64_t split = p.split_rows;
        const int64_t nch = max((int64_t)1, (a.total_rows + split - 1) / split);
        if (c >= nch) return false;
        r0 = c * split;
        r1 = min(a.total_rows, r0 + split);
        sq = 0;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            p.chunk_prefix[0] = 0;
            p.chunk_prefix[1] = nch;
        }
        return true;
    }
    if (wave == 0) plan_chunk(a, p, c, plan_s, lane);
    __syncthreads();  // plan_s
    if (plan_s[2] < 0) return false;
    r0 = plan_s[0];
    r1 = plan_s[1];
    sq = (int)plan_s[2];
    return true;
}

// fp8 query preparation: for every (sequence, head) the latent query scaled by
// a power of two qs (max |q| qs in [256, 512)) and rounded to fp16, the rope
// query times sm_scale log2(e) as bf16 hi + lo terms, and 1 / qs.  Stored per
// (sequence, group of 32 heads) in the split kernel's operand order, so that a
// wave's load of one operand register set is 1 KB contiguous: uint4
// ((i * 2 + j) * 2 + h) * 32 + n holds head n's latent dims 32 i + 16 h + 8 j
// .. + 7 (i < 16, j < 2, h < 2); uint4 2048 + (((i * 2 + j) * 2 + t) * 2 + h) *
// 32 + n its rope dims 32 i + 16 h + 8 j .. + 7, term t (0: hi, 1: lo; i < 2).
// One wave per (sequence, head); lane l converts dims 8 l .. 8 l + 7.
// The split kernel's tile plan over several sequences (one workgroup): tiles of
// sequence s = ceil(T_s / F8_TILE) (T_s clamped as in the plan), their exclusive
// prefix, the total and the quota of tiles per work item.
__device__ __forceinline__ void plan_tiles_fp8(const kvq_attn_args& a, const Plan& p) {
    __shared__ int64_t wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int64_t run = 0;
    for (int base = 0; base < a.n_seqs; base += 256) {
        const int s = base + tid;
        int64_t cnt = 0;
        if (s < a.n_seqs) {
            const int64_t lo = max(a.seq_offsets[s], (int64_t)0), hi = min(a.seq_offsets[s + 1], a.total_rows);
            cnt = hi > lo ? (hi - lo + F8_TILE - 1) / F8_TILE : 0;
        }
        int64_t incl = cnt;  // inclusive scan over the wave, then over the waves
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        int64_t before = run;
        for (int k = 0; k < wv; k++) before += wsum[k];
        if (s < a.n_seqs) p.chunk_prefix[s] = before + incl - cnt;
        run += (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        __syncthreads();
    }
    if (tid == 0) {
        p.chunk_prefix[a.n_seqs] = run;
        p.chunk_prefix[a.n_seqs + 1] =
            p.tile_quota > 0 ? p.tile_quota : max((int64_t)1, (run + p.n_work - 1) / p.n_work);
    }
}

__global__ __launch_bounds__(256) void k_qprep_fp8(kvq_attn_args a, Plan p, NewRows nr) {
    const int lane = threadIdx.x & 63;
    const int64_t prep_rows = (int64_t)a.n_seqs * p.heads_padded;
    const int64_t prep_blocks = (prep_rows + 3) / 4, enc_blocks = (nr.n + 3) / 4;
    if ((int64_t)blockIdx.x >= prep_blocks + enc_blocks) {  // the last block, several sequences: the tile plan
        plan_tiles_fp8(a, p);
        return;
    }
    if ((int64_t)blockIdx.x >= prep_blocks) {  // the rows appended by this call: one wave per row
        const int64_t r = ((int64_t)blockIdx.x - prep_blocks) * 4 + (threadIdx.x >> 6);
        if (r < nr.n) encode_fp8_row<1>(nr.x + r * DL, DL, nr.codes + r * DL, nr.scales + r, lane);
        return;
    }
    // wave-uniform (scalar) row and its division
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // = s * heads_padded + head
    if (row >= prep_rows) return;
    int s, hd;
    seq_head_of(row, a.n_seqs, p.heads_padded, s, hd);
    const bool hv = hd < a.n_heads;
    const int64_t qrow = (int64_t)s * a.n_heads + min(hd, a.n_heads - 1);  // absent heads: a zero query
    const float4 x0 = *reinterpret_cast<const float4*>(a.q_lat + qrow * DL + 8 * lane);
    const float4 x1 = *reinterpret_cast<const float4*>(a.q_lat + qrow * DL + 8 * lane + 4);
    const float4 y0 = *reinterpret_cast<const float4*>(a.q_rope + qrow * DR + 8 * (lane & 7));
    const float4 y1 = *reinterpret_cast<const float4*>(a.q_rope + qrow * DR + 8 * (lane & 7) + 4);
    float qmax = fmaxf(fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))),
                       fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w))));
    qmax = wave_max(qmax);
    const float qs = hv ? pow2_scale_for(qmax, 8) : 0.0f;
    uint4* dst = p.q_pack + ((int64_t)s * p.heads_padded + (hd & ~(F8_HEADS - 1))) * QPACK_U4;
    const int n = hd & (F8_HEADS - 1);
    const int i = lane >> 2, h = (lane >> 1) & 1, j = lane & 1;
    dst[((i * 2 + j) * 2 + h) * F8_HEADS + n] =
        make_uint4(pack_f16x2(x0.x * qs, x0.y * qs), pack_f16x2(x0.z * qs, x0.w * qs),
                   pack_f16x2(x1.x * qs, x1.y * qs), pack_f16x2(x1.z * qs, x1.w * qs));
    if (lane < 8) {
        const float cr = hv ? a.sm_scale * LOG2E : 0.0f;
        const float f[8] = {y0.x * cr, y0.y * cr, y0.z * cr, y0.w * cr, y1.x * cr, y1.y * cr, y1.z * cr, y1.w * cr};
        float b[8];
#pragma unroll
        for (int e = 0; e < 8; e++) b[e] = u2f(f32_to_bf16_rne(f[e]) << 16);
        dst[2048 + (((i * 2 + j) * 2 + 0) * 2 + h) * F8_HEADS + n] =
            make_uint4(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]), pack_bf16x2(b[6], b[7]));
        dst[2048 + (((i * 2 + j) * 2 + 1) * 2 + h) * F8_HEADS + n] =
            make_uint4(pack_bf16x2(f[0] - b[0], f[1] - b[1]), pack_bf16x2(f[2] - b[2], f[3] - b[3]),
                       pack_bf16x2(f[4] - b[4], f[5] - b[5]), pack_bf16x2(f[6] - b[6], f[7] - b[7]));
    }
    if (lane == 0) p.q_inv[row] = hv ? 1.0f / qs : 0.0f;  // exact
}

// fp8 split kernel.  Work item = (T-chunk, group of 32 heads); the 32 heads
// are the N dimension of v_mfma_f32_32x32x16_f16, so every e4m3 code converted
// to fp16 serves 32 heads.  The chunk is walked in tiles of 128 rows; within a
// tile the four waves split the work two ways:
//   score  wave w takes rows 32 w .. 32 w + 31 of the tile and all 32 heads:
//          S (32 rows x 32 heads) = codes (rows x k) . q~ (k x heads) on the
//          f16 matrix cores (latent, fp16 codes and query) and on the bf16 ones
//          (rope, bf16 keys and a two-term bf16 query);
//   PV     wave w takes output dims 128 w .. 128 w + 127 over all 128 rows:
//          O^T (dims x heads) += V^T (dims x rows) . P^T (rows x heads), with
//          V^T read transposed from the raw tile (ds_read_b64_tr_b8) and P^T
//          from LDS, where the score waves leave it as fp16 p * rho * rsc.
// So no wave's output overlaps another's, and nothing is merged across waves
// at the end.  Each wave streams its score rows' raw codes into the tile by
// LDS DMA (double-buffered); rope keys go straight to registers one tile ahead.
//
// Lane layouts (checked on the device): for v_mfma_f32_32x32x16, lane l holds
// A[m = l % 32][k = 8 (l / 32) + e] and B[k = 8 (l / 32) + e][n = l % 32]
// (e = 0..7), and D[m][n] sits in lane n + 32 ((m / 4) % 2), register
// 4 (m / 8) + m % 4.  The contraction index is free to relabel: in k-step j of
// pair i = j / 2, lane half h holds the latent dims 32 i + 16 h + 8 (j % 2) + e,
// the 16 contiguous code bytes of one 16-byte chunk.
//
// Tile layout: wave w's 32 rows at w * 16 KB of the buffer, row r at 512 r,
// 16-byte chunk c stored at chunk c ^ (r % 16), which puts the rows any read
// below serves on distinct banks (checked on the CPU).
//
// Softmax: one reference per head for the whole workgroup, the first tile's
// maximum, agreed through LDS at a barrier (B1) on that tile only;
// probabilities are 2^(s - m) <= 2^8, times rho * rsc (rsc a power of two with
// max rho * rsc < 1 over the chunk), rounded to fp16.  Every tile's maxima go
// to LDS beside its P, and after the barrier that publishes P (B2) a tile
// whose maximum exceeds the reference by more than 2^8 raises it and the
// workgroup starts its rows again (its P is then discarded): the accumulators
// are never rescaled inside the loop.  P and the maxima are double-buffered by
// tile parity, since without a barrier between B2 of tile t and the P writes
// of tile t + 1 a wave may still be reading P of tile t.
constexpr int F8_WROWS = 32;                    // score rows per wave
constexpr int F8_WBYTES = F8_WROWS * DL;        // one wave's rows in a code buffer: 16 KB
constexpr int F8_BUF = MF_WAVES * F8_WBYTES;    // a code buffer: 64 KB
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct F8Smem {
    uint8_t code[2][F8_BUF];               // raw e4m3 rows
    uint4 p[2][8][2][F8_HEADS];            // P^T per k-step of 16 rows: [parity][step][lane half][head] x 8 fp16
    float rho[2][MF_WAVES][64];            // each wave's row scales (lanes 32..63 hold copies)
    float xch[2][MF_WAVES][F8_HEADS];      // per-wave tile maxima per head
    float lsum[MF_WAVES][F8_HEADS];        // per-wave probability sums per head (a segment's end)
    float red[MF_WAVES];
};
static_assert(sizeof(F8Smem) <= 160 * 1024, "LDS");

__device__ __forceinline__ f32x16_t mfma32_f16(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32_bf16(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ONE: one sequence (the tile plan is the host's, and every work item is one segment).
// GATHER: sparse decode, the rows of the index list read in place (p.row_index).
template <bool ONE, bool GATHER>
__global__ __launch_bounds__(MF_WAVES * 64) void k_attn_mfma_fp8(kvq_attn_args a, Plan p) {
    __shared__ __align__(16) F8Smem sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int h = lane >> 5, n = lane & 31;  // lane half, head (and score row) within the group
    const int64_t local = blockIdx.x / N_XCD;
    const int64_t w = (int64_t)(blockIdx.x % N_XCD) + N_XCD * (local / p.n_groups);  // work item of the group
    const int hg = (int)(local % p.n_groups);
    if (w >= p.n_work) return;
    // this work item's tiles [tb, te) of the group's tile list (every sequence's tiles in order);
    // with several sequences the prefix, the total and the quota come from the preparation launch
    constexpr bool one = ONE;
    const int64_t* tp = p.chunk_prefix;
    const int64_t ntot = one ? p.n_tiles : tp[a.n_seqs];
    const int64_t quota = one ? p.tile_quota : tp[a.n_seqs + 1];
    const int64_t tb = w * quota, te = min(ntot, tb + quota);
    if (tb >= te) return;  // workgroup-uniform
    // sequence s: rows [seq_lo, seq_hi) (clamped as in the plan), tiles [seq_t0, seq_t1) of the list
    auto seq_lo = [&](int s) { return one ? (int64_t)0 : max(a.seq_offsets[s], (int64_t)0); };
    auto seq_hi = [&](int s) { return one ? a.total_rows : min(a.seq_offsets[s + 1], a.total_rows); };
    auto seq_t0 = [&](int s) { return one ? (int64_t)0 : tp[s]; };
    auto seq_t1 = [&](int s) { return one ? ntot : tp[s + 1]; };
    auto seq_of = [&](int64_t t) {  // the sequence holding tile t: the last s with seq_t0(s) <= t
        if (one) return 0;
        int lo = 0, hi = a.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tp[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    auto tile_row = [&](int64_t t, int s) { return seq_lo(s) + (int64_t)F8_TILE * (t - seq_t0(s)); };
    int sq = seq_of(tb);
    const int head = hg * F8_HEADS + n;
    // GATHER: the cache row of logical row t (t < total_rows is not required: rows past the
    // list re-read its last entry); gp = that row for row tw + lane % 32 of the wave block
    // whose loads are issued next
    auto phys = [&](int64_t t) -> uint32_t {
        const int64_t r = p.row_index[min(t, a.total_rows - 1)];
        return (uint32_t)min(max(r, (int64_t)0), p.cache_rows - 1);
    };
    uint32_t gp = 0;

    // ---- loaders.  The DMA of a tile brings this wave's 32 score rows: instruction
    // k (0..15) fills LDS chunks 64 k .. 64 k + 63 of the wave's 16 KB, lane l the
    // chunk of row 2 k + l / 32 stored at l % 32, i.e. global chunk (l % 32) ^ (row % 16);
    // instruction 16 brings the 32 row scales.  Rows past the arrays re-read the last
    // row (offsets clamped); rows past the chunk are loaded and masked later.
    const uint32_t dma_c = (uint32_t)((lane & 31) ^ h);  // (l % 32) ^ (row % 16) = dma_c ^ (2 k % 16)
    const uint32_t lds_code0 = lds_offset(&sm.code[0][0]) + (uint32_t)wave * F8_WBYTES;
    const uint32_t lds_rho0 = lds_offset(&sm.rho[0][0][0]) + (uint32_t)wave * 256u;
    auto dma_one = [&](int k, int64_t tw, int buf) __attribute__((always_inline)) {
        if constexpr (GATHER) {  // rows 2 k + h of the block from their cache rows (gp)
            if (k < 16) {
                const uint32_t g0 = __builtin_amdgcn_readlane(gp, 2 * k), g1 = __builtin_amdgcn_readlane(gp, 2 * k + 1);
                const uint32_t gr = h ? g1 : g0;
                dma_lds_b128_at(a.codes + (uint64_t)gr * DL + ((dma_c ^ (uint32_t)((2 * k) & 15)) << 4),
                                __builtin_amdgcn_readfirstlane(lds_code0 + (uint32_t)buf * F8_BUF + 1024u * k));
            } else {
                dma_lds_b32_at(a.row_scale + gp,
                               __builtin_amdgcn_readfirstlane(lds_rho0 + (uint32_t)buf * (MF_WAVES * 256u)));
            }
            return;
        }
        // tw: first row of this wave's block; the base row and the offsets stay inside the arrays
        const int64_t b = min(tw, a.total_rows - 1);
        const uint32_t lim = (uint32_t)(a.total_rows - b);  // rows from b to the end, >= 1
        if (k < 16) {
            const uint32_t voff = (uint32_t)(2 * k + h) * 512u + ((dma_c ^ (uint32_t)((2 * k) & 15)) << 4);
            dma_lds_b128(a.codes + b * DL, min(voff, lim * 512u - 16u),
                         __builtin_amdgcn_readfirstlane(lds_code0 + (uint32_t)buf * F8_BUF + 1024u * k));
        } else {
            dma_lds_b32(a.row_scale + b, 4u * min((uint32_t)(lane & 31), lim - 1u),
                        __builtin_amdgcn_readfirstlane(lds_rho0 + (uint32_t)buf * (MF_WAVES * 256u)));
        }
    };
    // rope keys of this wave's score rows: lane (h, n) takes row n, dims 32 i + 16 h .. + 15 (i = 0, 1)
    uint4 kr[2][2];
    auto load_rope = [&](int64_t tw) __attribute__((always_inline)) {
        const int64_t row = GATHER ? (int64_t)gp : min(tw + n, a.total_rows - 1);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                kr[i][j] = *reinterpret_cast<const uint4*>(a.k_rope + row * DR + 32 * i + 16 * h + 8 * j);
    };
    {
        const int64_t tw = tile_row(tb, sq) + F8_WROWS * wave;
        if (GATHER) gp = phys(tw + (lane & 31));
#pragma unroll
        for (int k = 0; k < 17; k++) dma_one(k, tw, 0);
        load_rope(tw);
    }

    // ---- query operands, prepared once per (sequence, head) by k_qprep_fp8 in this
    // kernel's operand order (40 KB per group of 32 heads).  Every wave needs all of
    // them, so they are brought into the second code buffer once per workgroup by
    // LDS DMA (each wave 10 of the 40 KB-sized instructions) and read from there.
    {
        const uint4* qp = p.q_pack + ((int64_t)sq * p.heads_padded + hg * F8_HEADS) * QPACK_U4;
        const uint32_t lq = __builtin_amdgcn_readfirstlane(lds_offset(&sm.code[1][0]));
#pragma unroll
        for (int k = 0; k < 10; k++) {
            const int blk = 10 * wave + k;  // 1 KB block of the 40 KB pack
            dma_lds_b128(qp + 64 * blk, 16u * lane, lq + 1024u * blk);
        }
    }
    float qinv = p.q_inv[(int64_t)sq * p.heads_padded + head];
    // ---- rsc from the largest row scale of the work item's rows (contiguous over its
    // sequences; four loads in flight per thread)
    const int64_t r0 = tile_row(tb, sq);
    int64_t r1;
    {
        const int sl = seq_of(te - 1);
        r1 = min(tile_row(te - 1, sl) + F8_TILE, seq_hi(sl));
        r1 = max(r1, r0 + 1);
    }
    float rm = 0.0f;
    for (int64_t t = r0 + tid; t < r1; t += 4 * MF_WAVES * 64) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t tr = min(min(t + u * MF_WAVES * 64, r1 - 1), a.total_rows - 1);
            x[u] = a.row_scale[GATHER ? (int64_t)phys(tr) : tr];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) rm = fmaxf(rm, fabsf(x[u]));
    }
    rm = wave_max_swap(rm, lane);
    if (lane == 0) sm.red[wave] = rm;

    vm_wait_all();     // this wave's share of the pack (and the loads before it) has landed
    wg_barrier_lds();  // every wave's share, and the row-scale maxima, are visible
    uint4 qh[16][2], rh[2][2], rl[2][2];
    {
        const uint4* q4 = reinterpret_cast<const uint4*>(&sm.code[1][0]) + lane;
#pragma unroll
        for (int i = 0; i < 16; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) qh[i][j] = q4[(i * 2 + j) * 64];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                rh[i][j] = q4[2048 + ((i * 2 + j) * 2 + 0) * 64];
                rl[i][j] = q4[2048 + ((i * 2 + j) * 2 + 1) * 64];
            }
    }
    float k1 = a.sm_scale * LOG2E * qinv;  // latent score scale (log2 units)
    const float rsc = pow2_scale_for(fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3])), -1);

    // ---- per-lane LDS addresses
    // score: row n of this wave's block, global chunk 2 i + h stored at (2 i + h) ^ (n % 16)
    const uint32_t sc_row = (uint32_t)wave * F8_WBYTES + (uint32_t)n * 512u;
    const uint32_t sc_x = (uint32_t)(n & 15);
    // PV: lane l in 16-lane group (h, mh), q = l % 16: row R = 8 (e / 4) + 4 h + e % 4 of
    // a 16-row k-step (e = q / 2), bytes 8 (q % 2) of global chunk 8 w + 2 b + mh
    const int q16 = lane & 15, e8 = q16 >> 1, mh = (lane >> 4) & 1;
    const uint32_t pv_r = (uint32_t)(8 * (e8 >> 2) + 4 * h + (e8 & 3));
    uint32_t pv_addr[4];
#pragma unroll
    for (int b = 0; b < 4; b++)
        pv_addr[b] = pv_r * 512u + (((uint32_t)(8 * wave + 2 * b + mh) ^ pv_r) << 4) + 8u * (uint32_t)(q16 & 1);

    f32x16_t acc_o[4];
    int g0 = 0;  // buffer and P parity of the segment's first tile
    int64_t t_seg = tb;
    for (;;) {  // segments: the work item's tiles of one sequence
    const int64_t seg_t1 = min(te, seq_t1(sq));
    const int64_t s_t0 = seq_t0(sq), s_lo = seq_lo(sq), s_hi = seq_hi(sq);
    float m_ref = -INFINITY;  // per head (lane n), identical in every wave
    float l_part = 0.0f;
    for (;;) {
#pragma unroll
    for (int b = 0; b < 4; b++) acc_o[b] = f32x16_t{};
    l_part = 0.0f;
    bool again = false;
    // (a counted loop from 0: with a bottom-tested loop LLVM copies the accumulators
    // between register files every tile)
    const int ntl = (int)(seg_t1 - t_seg);
    const bool seg_more = !ONE && seg_t1 < te;  // the work item goes on with another segment
    for (int k = 0; k < ntl; k++) {
        const int64_t t = t_seg + k;
        const int buf = (g0 + k) & 1;
        const int64_t tw = s_lo + (int64_t)F8_TILE * (t - s_t0) + F8_WROWS * wave;  // this wave's first score row
        vm_wait_all();  // this wave's rows, row scales and rope keys of the tile have landed
        if constexpr (GATHER) {  // the next tile's cache rows, used from its first DMA (in the PV below)
            if (k + 1 < ntl || seg_more) {
                const int64_t gtw = (ONE || k + 1 < ntl) ? tw + F8_TILE : tile_row(t + 1, seq_of(t + 1)) + F8_WROWS * wave;
                gp = phys(gtw + (lane & 31));
            }
        }
        // ---- scores: rope first (its keys are then free for the next tile's), latent on two chains
        f32x16_t s_r = f32x16_t{}, s_a = f32x16_t{}, s_b = f32x16_t{};
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                s_r = mfma32_bf16(kr[i][j], rh[i][j], s_r);
                s_r = mfma32_bf16(kr[i][j], rl[i][j], s_r);
            }
        // workgroup-uniform: a next tile, of this segment or the next (written on the loop
        // counter: a 64-bit compare here made LLVM move the accumulators every tile)
        const bool more = k + 1 < ntl || seg_more;
        const int64_t ntw = (ONE || k + 1 < ntl) ? tw + F8_TILE : tile_row(t + 1, seq_of(t + 1)) + F8_WROWS * wave;
        if (!GATHER && more) load_rope(ntw);  // (GATHER: with the first DMAs, after gp has landed)
        const uint8_t* cw = &sm.code[buf][0] + sc_row;
        auto chunk = [&](int i) {
            return *reinterpret_cast<const uint4*>(cw + ((((uint32_t)(2 * i + h)) ^ sc_x) << 4));
        };
        uint4 nx = chunk(0), nx2 = chunk(1);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint4 cur = nx;
            nx = nx2;
            if (i < 14) nx2 = chunk(i + 2);
            __builtin_amdgcn_sched_barrier(0);  // the look-ahead read issues before this chunk's math
            const uint4 a0 = make_uint4(e4m3x2_to_f16x2<false>(cur.x), e4m3x2_to_f16x2<true>(cur.x),
                                        e4m3x2_to_f16x2<false>(cur.y), e4m3x2_to_f16x2<true>(cur.y));
            const uint4 a1 = make_uint4(e4m3x2_to_f16x2<false>(cur.z), e4m3x2_to_f16x2<true>(cur.z),
                                        e4m3x2_to_f16x2<false>(cur.w), e4m3x2_to_f16x2<true>(cur.w));
            f32x16_t& s = (i & 1) ? s_b : s_a;
            s = mfma32_f16(a0, qh[i][0], s);
            s = mfma32_f16(a1, qh[i][1], s);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- softmax: lane (h, n) holds rows 8 (r / 4) + 4 h + r % 4 of head n
        const int nvw = (int)min((int64_t)F8_WROWS, s_hi - tw);  // valid rows of this wave's block (may be <= 0)
        float sc[16], rr[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float4 rq = *reinterpret_cast<const float4*>(&sm.rho[buf][wave][8 * j + 4 * h]);
            const float rv[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int r = 4 * j + u;
                const bool ok = 8 * j + 4 * h + u < nvw;
                rr[r] = ok ? rv[u] : 0.0f;
                sc[r] = ok ? fmaf(rv[u] * k1, s_a[r] + s_b[r], s_r[r]) : -INFINITY;
                tmax = fmaxf(tmax, sc[r]);
            }
        }
        tmax = fmaxf(tmax, xor_lane<32>(tmax, lane));
        const int par = buf;
        if (h == 0) sm.xch[par][wave][n] = tmax;
        if (m_ref == -INFINITY) {  // the first tile (workgroup-uniform): agree on the reference
            wg_barrier_lds();      // B1: every wave's tile maxima
            m_ref = fmaxf(fmaxf(sm.xch[par][0][n], sm.xch[par][1][n]), fmaxf(sm.xch[par][2][n], sm.xch[par][3][n]));
        }
        float psum = 0.0f;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(sc[r] - m_ref), p1 = __builtin_amdgcn_exp2f(sc[r + 1] - m_ref);
            psum += p0 + p1;
            pk[r / 2] = pack_f16x2(p0 * (rr[r] * rsc), p1 * (rr[r + 1] * rsc));
        }
        // (buffer par: the PV of tile t - 2 read it, and every wave was past that PV at B2 of tile t - 1)
        sm.p[par][2 * wave][h][n] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        sm.p[par][2 * wave + 1][h][n] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        wg_barrier_lds();  // B2: P of every row, every wave's tile maxima and rows of the tile are in LDS
        {
            const float mt = fmaxf(fmaxf(sm.xch[par][0][n], sm.xch[par][1][n]), fmaxf(sm.xch[par][2][n], sm.xch[par][3][n]));
            if (__any(mt > m_ref + LAZY_LOG2)) {  // workgroup-uniform: every wave sees the same maxima
                m_ref = fmaxf(m_ref, mt);
                again = true;
                break;
            }
        }
        l_part += psum;
        // ---- PV over the tile's 8 k-steps, each step's reads issued during the one
        // before; the next tile's DMA goes out between the steps
        const uint8_t* vb = &sm.code[buf][0];
        auto pv_read = [&](int J, int b) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(
                vb + (J >> 1) * F8_WBYTES + (J & 1) * 16 * 512 + pv_addr[b]));
        };
        uint4 bp = sm.p[par][0][h][n];
        i32x2_t tv[4];
#pragma unroll
        for (int b = 0; b < 4; b++) tv[b] = pv_read(0, b);
#pragma unroll
        for (int J = 0; J < 8; J++) {
            const uint4 cbp = bp;
            i32x2_t cv[4];
#pragma unroll
            for (int b = 0; b < 4; b++) cv[b] = tv[b];
            if (J < 7) {
                bp = sm.p[par][J + 1][h][n];
#pragma unroll
                for (int b = 0; b < 4; b++) tv[b] = pv_read(J + 1, b);
            }
            __builtin_amdgcn_sched_barrier(0);  // the next step's reads issue before this step's math
            if (more) {
                dma_one(2 * J, ntw, buf ^ 1);
                dma_one(2 * J + 1, ntw, buf ^ 1);
                if (J == 7) dma_one(16, ntw, buf ^ 1);
                if (GATHER && J == 0) load_rope(ntw);
            }
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const uint4 av = e4m3x8_to_f16x8((uint32_t)cv[b][0], (uint32_t)cv[b][1]);
                acc_o[b] = mfma32_f16(av, cbp, acc_o[b]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (!again) {
        g0 += ntl;
        break;
    }
    vm_wait_all();    // the rope loads in flight
    __syncthreads();  // every wave has read the tile maxima before they are written again
    {  // start the segment's rows again with the raised reference (both buffers are free)
        g0 = 0;
        const int64_t tw = s_lo + (int64_t)F8_TILE * (t_seg - s_t0) + F8_WROWS * wave;
        if (GATHER) gp = phys(tw + (lane & 31));
#pragma unroll
        for (int k = 0; k < 17; k++) dma_one(k, tw, 0);
        load_rope(tw);
    }
    }

    // ---- the segment's partial state, in slot w + sq (the merge reads a sequence's slots
    // as one run): l per head over the waves, then each wave's dims of every head.  The
    // next segment's first tile is in flight meanwhile.
    const int64_t c = w + sq;
    float lt = l_part + xor_lane<32>(l_part, lane);
    if (h == 0) sm.lsum[wave][n] = lt;
    wg_barrier_lds();  // (LDS only: the next segment's first tile stays in flight)
    const float L = (sm.lsum[0][n] + sm.lsum[1][n]) + (sm.lsum[2][n] + sm.lsum[3][n]);
    {
        // partial O of this (chunk, group) in the matrix cores' lane order, as fp16 O * 2^k
        // with one k per head and wave (128 dims) putting the largest |O| * 2^k in
        // [2^14, 2^15): uint2 ((w * 4 + b) * 4 + j) * 64 + lane holds head n = lane % 32,
        // dims 128 w + 32 b + 8 j + 4 (lane / 32) .. + 3 (k_merge_f8 reads it in the same
        // order); 2^-k in part_s
        float am = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int e = 0; e < 16; e++) am = fmaxf(am, fabsf(acc_o[b][e]));
        am = fmaxf(am, xor_lane<32>(am, lane));
        const float so = 1.0f / rsc;  // exact (a power of two)
        float sk_inv;
        const float f = so * f16_store_scale(am * so, &sk_inv);  // exact: amax(acc) * f is near 2^14
        uint2* dst = reinterpret_cast<uint2*>(p.part_h) + (c * p.n_groups + hg) * (int64_t)(F8_HEADS * DL / 4) +
                     wave * 16 * 64 + lane;
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                st_nt(dst + (b * 4 + j) * 64, make_uint2(pack_f16x2(acc_o[b][4 * j] * f, acc_o[b][4 * j + 1] * f),
                                                         pack_f16x2(acc_o[b][4 * j + 2] * f, acc_o[b][4 * j + 3] * f)));
        if (h == 0 && head < a.n_heads) {
            __builtin_nontemporal_store(sk_inv, &p.part_s[(c * 4 + wave) * a.n_heads + head]);
            if (wave == 0) {
                __builtin_nontemporal_store(m_ref, &p.part_m[c * a.n_heads + head]);  // log2 units
                __builtin_nontemporal_store(L, &p.part_l[c * a.n_heads + head]);
            }
        }
    }
    t_seg = seg_t1;
    if (ONE || t_seg >= te) break;
    // ---- the next sequence: its query operands straight from the prepared pack (the
    // staging buffer holds a tile by now)
    sq = seq_of(t_seg);
    {
        const uint4* q4 = p.q_pack + ((int64_t)sq * p.heads_padded + hg * F8_HEADS) * QPACK_U4 + lane;
#pragma unroll
        for (int i = 0; i < 16; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) qh[i][j] = q4[(i * 2 + j) * 64];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                rh[i][j] = q4[2048 + ((i * 2 + j) * 2 + 0) * 64];
                rl[i][j] = q4[2048 + ((i * 2 + j) * 2 + 1) * 64];
            }
        qinv = p.q_inv[(int64_t)sq * p.heads_padded + head];
        k1 = a.sm_scale * LOG2E * qinv;
    }
    }
}

// Rotated-codec query preparation: q~ = H D q / sqrt(512) for every
// (sequence, head), scaled by a power of two qs (max |q~| * qs in [256, 512))
// and split into two fp16 terms, hi = fp16(q~ qs) and lo = fp16(q~ qs - hi)
// (about 22 significant bits together; one fp16 term alone moves sharply
// peaked softmaxes by up to 3e-3 of the output), in the split kernel's operand
// order per block of 16 heads, so that a wave loads each operand register as
// 1 KB contiguous: uint4 64 ks + 16 g + n of the block holds head n's hi of
// dims 32 ks + 8 g .. + 7, uint4 64 (QS_LL + ks) + 16 g + n their lo; the rope
// query (times sm_scale * log2(e)) as bf16 hi (slot QS_RH + k) and lo (slot
// QS_RL + k) terms of dims 32 k + 8 g .. + 7; 1 / qs in q_inv.  One wave per
// (sequence, head); lane l rotates dims 8 l .. 8 l + 7 (three butterfly stages
// in registers, six across lanes).
__global__ __launch_bounds__(256) void k_qprep_tq4(kvq_attn_args a, Plan p) {
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) row and its division
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // = s * heads_padded + h
    if (row >= (int64_t)a.n_seqs * p.heads_padded) return;
    int s, h;
    seq_head_of(row, a.n_seqs, p.heads_padded, s, h);
    const bool valid = h < a.n_heads;
    // unconditional loads (a clamped head; a guarded load would wait for every load in flight)
    const float* src = a.q_lat + ((int64_t)s * a.n_heads + min(h, a.n_heads - 1)) * DL + 8 * lane;
    const float4 x0 = *reinterpret_cast<const float4*>(src), x1 = *reinterpret_cast<const float4*>(src + 4);
    const float* r = a.q_rope + ((int64_t)s * a.n_heads + min(h, a.n_heads - 1)) * DR + 8 * (lane & 7);
    const float4 y0 = *reinterpret_cast<const float4*>(r), y1 = *reinterpret_cast<const float4*>(r + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = valid ? v[i] : 0.0f;
    const uint32_t sm = a.sign_mask[lane];
#pragma unroll
    for (int i = 0; i < 8; i++)
        if ((sm >> i) & 1u) v[i] = -v[i];
#pragma unroll
    for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (!(i & hh)) {
                const float x = v[i], y = v[i + hh];
                v[i] = x + y;
                v[i + hh] = x - y;
            }
    // across lanes: DPP and lane-swap butterflies
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float x = v[i];
        x = fwht_xlane_c<1>(x, lane);
        x = fwht_xlane_c<2>(x, lane);
        x = fwht_xlane_c<4>(x, lane);
        x = fwht_xlane_c<8>(x, lane);
        x = fwht_xlane_c<16>(x, lane);
        v[i] = fwht_xlane_c<32>(x, lane);
    }
    float qmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        v[i] *= INV_SQRT_DL;
        qmax = fmaxf(qmax, fabsf(v[i]));
    }
    qmax = wave_max(qmax);
    const float qs = pow2_scale_for(qmax, 8);
    // (heads_padded is a multiple of 16: the block of this row's 16 heads, head row % 16 in it)
    uint4* dst = p.q_pack + (row & ~(int64_t)15) * QPACK_TQ + (row & 15);
    float hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float x = v[i] * qs;  // exact (a power of two)
        hi[i] = (float)(_Float16)x;
        lo[i] = x - hi[i];          // exact in fp32
    }
    const int ks = lane >> 2, gq = lane & 3;  // dims 8 lane = 32 ks + 8 gq
    dst[64 * ks + 16 * gq] = make_uint4(pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]),
                                       pack_f16x2(hi[4], hi[5]), pack_f16x2(hi[6], hi[7]));
    dst[64 * (QS_LL + ks) + 16 * gq] = make_uint4(pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]),
                                                 pack_f16x2(lo[4], lo[5]), pack_f16x2(lo[6], lo[7]));
    if (lane < 8) {  // rope dims 8 lane .. + 7: k-step lane / 4, lane group lane % 4
        const float c2r = valid ? a.sm_scale * LOG2E : 0.0f;
        const float rv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t rh[4], rl[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float f0 = rv[2 * i] * c2r, f1 = rv[2 * i + 1] * c2r;
            const float b0 = u2f(f32_to_bf16_rne(f0) << 16), b1 = u2f(f32_to_bf16_rne(f1) << 16);
            rh[i] = pack_bf16x2(b0, b1);
            rl[i] = pack_bf16x2(f0 - b0, f1 - b1);
        }
        dst[64 * (QS_RH + ks) + 16 * gq] = make_uint4(rh[0], rh[1], rh[2], rh[3]);
        dst[64 * (QS_RL + ks) + 16 * gq] = make_uint4(rl[0], rl[1], rl[2], rl[3]);
    }
    if (lane == 0) p.q_inv[row] = 1.0f / qs;  // exact
}

// Rotated-codec split kernel (BITS = 3, 4, 6).  Work item = (T-chunk, group of
// 64 heads); the items are dealt to XCDs in contiguous runs so the head groups
// of a chunk share one L2.  A workgroup has 8 waves in two roles, two waves on
// each SIMD (one of each role), pipelined over the chunk's 32-row tiles:
//   score wave w (0..3), heads 16 w .. 16 w + 15:
//           S^T (16 rows x 16 heads) += X(rows, k) q~^T from the decoded tile
//           (lane (g, n): row 16 rb + n, dims 32 ks + 8 g .. + 7), softmax,
//           P'^T (the PV operand, 1 KB) to LDS;
//   PV wave v (4..7, v - 4 = u), dims 128 u .. 128 u + 127 of all 64 heads:
//           O^T (16 dims x 16 heads) += X^T P'^T, X^T via ds_read_b64_tr_b16
//           (lane (g, p) gets rows 4 g .. 4 g + 3 and 16 + 4 g .. + 3 of column
//           p, the k order the score waves hold P in), one read per 16 dims
//           serving the 4 head blocks; and the decode of the tile after next
//           (each PV wave 8 rows) into the third fp16 buffer.
// At step k the score waves take tile k and the PV waves tile k - 1; one
// barrier per step.  The decoded tiles are triple-buffered (score, PV and
// decode each use one), P double-buffered.  On one SIMD the matrix cores
// alternate between the two roles' products while the other role issues its
// LDS reads and vector work; with one wave per SIMD (score and PV in one
// wave, the whole tile read twice per wave) a 32-row tile took about 3 us.
// Softmax: fixed per-head reference (first tile's max) and probabilities times
// rho * rs with rs from the chunk's largest radius; a tile more than 2^8 above
// the reference raises it, and the workgroup (which shares the tiles) starts
// its rows again at the next step's vote.
//
// The decoded tile: row r at DL halfwords r, its 16-byte chunk c (dims 8 c ..
// 8 c + 7) stored at chunk c ^ tq_swz(r), tq_swz(r) = 2 (r % 4) ^ 9 bit2(r) ^
// bit3(r) (0, 2, 4, 6, 9, 11, 13, 15, 1, 3, 5, 7, 8, 10, 12, 14 for r % 16).
// With the decode share of lane l on row l % 8 of its wave's 8 rows, the
// decode writes (8 or 16 lanes on 8 rows), score reads (8 or 16 consecutive
// rows, one chunk) and transposed PV reads (4 or 8 rows x 4 half-chunks) fall
// on distinct banks whether a read or write cycle serves 64 bytes per 8 lanes
// (32 banks) or 128 bytes per 16 (64 banks) -- checked on the CPU.
constexpr int KT = DR + 8;  // halfwords per rope tile row
constexpr int TQ_BUFS = 3;  // decoded tiles in flight: scored, multiplied, being decoded
__device__ __forceinline__ int tq_swz(int r) { return (2 * (r & 3)) ^ ((r & 4) ? 9 : 0) ^ ((r >> 3) & 1); }
template <int BITS>
__global__ __launch_bounds__(2 * MF_WAVES * 64) void k_attn_mfma_tq(kvq_attn_args a, Plan p) {
    __shared__ __align__(16) uint16_t xt_mem[TQ_BUFS * MF_TILE * DL];  // decoded latent rows, fp16
    auto xt_row = [&](int buf, int r) __attribute__((always_inline)) { return xt_mem + (buf * MF_TILE + r) * DL; };
    __shared__ __align__(16) uint16_t kt[TQ_BUFS][MF_TILE][KT];  // rope keys, bf16
    __shared__ __align__(16) float rho_s[TQ_BUFS][MF_TILE];      // radius / sqrt(512)
    __shared__ __align__(16) uint4 pb_s[2][MF_WAVES][64];         // P'^T of each score wave, by tile parity
    __shared__ float red_s[2 * MF_WAVES];
    __shared__ int flag_s[2][MF_WAVES];
    __shared__ int64_t plan_s[3];
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const bool score_wave = wid < MF_WAVES;  // workgroup-uniform per wave
    const int wave = wid & (MF_WAVES - 1);   // index within the role
    const int g = lane >> 4, n = lane & 15;
    const int64_t local = blockIdx.x / N_XCD;
    const int64_t c = (int64_t)(blockIdx.x % N_XCD) + N_XCD * (local / p.n_groups);
    const int hg = (int)(local % p.n_groups);
    if (c >= p.max_chunks) return;
    const int head = hg * TQ_HEADS + MF_HEADS * wave + n;  // score waves; may exceed n_heads (its query is zero)
    constexpr int CB = DL * BITS / 8;                         // code bytes per row
    int64_t r0, r1;
    int sq;
    if (!locate_chunk(a, p, c, plan_s, wid, lane, r0, r1, sq)) return;  // workgroup-uniform
    const int ntiles = (int)((r1 - r0 + MF_TILE - 1) / MF_TILE);

    // PV waves' decode share: tile row 8 wave + lane / 8, code bytes 8 BITS (lane % 8) ..
    // + 8 BITS - 1 (dims 64 (lane % 8) .. + 63), rope bytes 16 (lane % 8).  Group i of 8
    // dims is bits 8 BITS i .. of the lane's words.
    const int drow = 8 * wave + (lane & 7), dq = lane >> 3;
    uint4 cv[3] = {};  // codes of the tile to decode next (BITS * 2 words)
    uint4 cr;     // its rope keys
    float cs;     // its row radius (scaled by 1 / sqrt(512) when it is stored)
    auto load_share = [&](int t) __attribute__((always_inline)) {
        const int64_t t0 = r0 + (int64_t)MF_TILE * t;
        const int64_t row = t0 + min(drow, (int)(r1 - t0) - 1);  // rows past the chunk re-read its last row
        const uint8_t* cp = a.codes + row * CB + 8 * BITS * dq;
        if constexpr (BITS == 3) {  // 24 bytes, 8-byte aligned
            const uint2 v0 = *reinterpret_cast<const uint2*>(cp);
            const uint2 v1 = *reinterpret_cast<const uint2*>(cp + 8);
            const uint2 v2 = *reinterpret_cast<const uint2*>(cp + 16);
            cv[0] = make_uint4(v0.x, v0.y, v1.x, v1.y);
            cv[1] = make_uint4(v2.x, v2.y, 0u, 0u);
        } else {  // 32 or 48 bytes, 16-byte aligned
            cv[0] = *reinterpret_cast<const uint4*>(cp);
            cv[1] = *reinterpret_cast<const uint4*>(cp + 16);
            if constexpr (BITS == 6) cv[2] = *reinterpret_cast<const uint4*>(cp + 32);
        }
        cr = *reinterpret_cast<const uint4*>(a.k_rope + row * DR + 8 * dq);
        cs = a.row_scale[row];
    };
    const Tq4Lut lut = BITS == 3 ? make_tq3_lut() : make_tq4_lut();
    const uint32_t tab6 = BITS == 6 ? f16_bits(u2f(c_tq6_level[32 + (lane & 31)])) : 0u;
    const int dswz = tq_swz(drow);
    const int dq_off = 64 * (dq ^ (dswz >> 3)), di = dswz & 7;  // chunk 8 dq + i sits at 8 (dq ^ f / 8) + (i ^ f % 8)
    // group i (dims 64 dq + 8 i .. + 7) of the share, decoded into chunk 8 dq + i of the row
    auto decode_group = [&](int buf, int i) __attribute__((always_inline)) {
        uint4 hv;
        const uint32_t w[12] = {cv[0].x, cv[0].y, cv[0].z, cv[0].w, cv[1].x, cv[1].y,
                                cv[1].z, cv[1].w, cv[2].x, cv[2].y, cv[2].z, cv[2].w};
        if constexpr (BITS == 4) {
            hv = tq4x8_to_f16x8(w[i], lut);
        } else if constexpr (BITS == 3) {
            // group i = bits 24 i .. 24 i + 23 of the words w0 .. w5
            const int b = 24 * i, k = b >> 5, sh = b & 31;
            const uint32_t v = sh == 0 ? w[k] : (sh <= 8 ? (w[k] >> sh) : __builtin_amdgcn_alignbit(w[k + 1], w[k], sh));
            hv = tq3x8_to_f16x8(v & 0xFFFFFFu, lut);
        } else {
            // groups 2k and 2k + 1 = bits 0 .. 47 and 48 .. 95 of words 3k .. 3k + 2
            const int k = i >> 1;
            const uint32_t a0 = w[3 * k], a1 = w[3 * k + 1], a2 = w[3 * k + 2];
            hv = (i & 1) ? tq6x8_to_f16x8((uint64_t)(a1 >> 16) | ((uint64_t)a2 << 16), tab6)
                         : tq6x8_to_f16x8((uint64_t)a0 | ((uint64_t)(a1 & 0xFFFFu) << 32), tab6);
        }
        *reinterpret_cast<uint4*>(xt_row(buf, drow) + dq_off + 8 * (i ^ di)) = hv;
    };
    auto decode_rest = [&](int buf) __attribute__((always_inline)) {  // the rope key and the radius
        *reinterpret_cast<uint4*>(&kt[buf][drow][8 * dq]) = cr;
        rho_s[buf][drow] = cs * INV_SQRT_DL;  // the 8 lanes of a row store the same value
    };
    auto decode_share = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; i++) decode_group(buf, i);
        decode_rest(buf);
    };
    // ---- the chunk's largest row scale (four loads in flight per thread)
    float rmax = 0.0f;
    for (int64_t t = r0 + tid; t < r1; t += 8 * MF_WAVES * 64) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) x[u] = a.row_scale[min(t + u * 2 * MF_WAVES * 64, r1 - 1)];
#pragma unroll
        for (int u = 0; u < 4; u++) rmax = fmaxf(rmax, fabsf(x[u]));
    }
    rmax = wave_max_swap(rmax, lane);
    if (lane == 0) red_s[wid] = rmax;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2 * MF_WAVES; k++) rmax = fmaxf(rmax, red_s[k]);
    const float rs = pow2_scale_for(rmax * INV_SQRT_DL, -1);  // max rho * rs in [0.5, 1)

    bool over = false;
    // one vote + barrier per step: every score wave reports whether its tile was out of
    // range (any such vote restarts the workgroup); the barrier also publishes the
    // decoded tile and the P operands of the step.  The two roles run separate loops
    // with the same votes (their registers then never overlap).
    auto vote = [&](int k) __attribute__((always_inline)) {
        if (score_wave) flag_s[k & 1][wave] = over ? 1 : 0;  // every lane stores the same value
        wg_barrier_lds();
        const int4 f = *reinterpret_cast<const int4*>(&flag_s[k & 1][0]);
        return (f.x | f.y | f.z | f.w) != 0;  // workgroup-uniform
    };
    if (score_wave) {
        // ---- query operands (prepared once per sequence and head; the wave's block of
        // 16 heads, lane (g, n) = lane reads uint4 64 slot + lane, 1 KB per slot)
        const uint4* qp = p.q_pack + ((int64_t)sq * p.heads_padded + hg * TQ_HEADS + MF_HEADS * wave) * QPACK_TQ + lane;
        uint4 qh[16], qo[16], rh[2], rl[2];
#pragma unroll
        for (int k = 0; k < 16; k++) {
            qh[k] = qp[64 * k];
            qo[k] = qp[64 * (QS_LL + k)];
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            rh[k] = qp[64 * (QS_RH + k)];
            rl[k] = qp[64 * (QS_RL + k)];
        }
        const float k1 = a.sm_scale * LOG2E * p.q_inv[(int64_t)sq * p.heads_padded + head];
        // score row 16 rb + n, dims 8 g + 32 ks: chunk g + 4 ks of row n sits at
        // 4 (ks ^ f / 4) + (g ^ f % 4), f = tq_swz(n)
        const int fs = tq_swz(n);
        int sro[4];
#pragma unroll
        for (int j = 0; j < 4; j++) sro[j] = 32 * (j ^ (fs >> 2)) + 8 * (g ^ (fs & 3));
        float m_run = -INFINITY, l_part = 0.0f;
        for (;;) {
            l_part = 0.0f;
            bool again = vote(0);
            for (int k = 0; !again && k <= ntiles; k++) {
                if (k < ntiles) {
                    const int buf = k % TQ_BUFS;
                    const int nt = (int)min((int64_t)MF_TILE, r1 - (r0 + (int64_t)MF_TILE * k));
                    // ---- scores S^T (two row blocks) from the tile: four independent
                    // accumulator chains (row block x even / odd k-step), reads one step ahead
                    f32x4_t sl[2], sr[2], sx[2];
                    f32x4_t sqv[2];  // the query's fp16 remainder terms
                    sl[0] = sl[1] = sr[0] = sr[1] = sx[0] = sx[1] = sqv[0] = sqv[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    {
                        // chunk g + 4 ks of rows n and 16 + n (the same swizzle) sits at halfword
                        // 32 (ks - ks % 4) + sro[ks % 4]
                        const uint16_t* xa = xt_row(buf, n);
                        const uint16_t* xb = xt_row(buf, 16 + n);
                        auto sc_read = [&](const uint16_t* x, int ks) __attribute__((always_inline)) {
                            return *reinterpret_cast<const f16x8_t*>(x + 32 * (ks & ~3) + sro[ks & 3]);
                        };
                        f16x8_t na = sc_read(xa, 0), nb = sc_read(xb, 0);
#pragma unroll
                        for (int ks = 0; ks < 16; ks++) {
                            const f16x8_t ca2 = na, cb2 = nb;
                            if (ks < 15) {
                                na = sc_read(xa, ks + 1);
                                nb = sc_read(xb, ks + 1);
                            }
                            f32x4_t& s0 = (ks & 1) ? sx[0] : sl[0];
                            f32x4_t& s1 = (ks & 1) ? sx[1] : sl[1];
                            s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca2, as_f16x8(qh[ks]), s0, 0, 0, 0);
                            s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(cb2, as_f16x8(qh[ks]), s1, 0, 0, 0);
                            sqv[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca2, as_f16x8(qo[ks]), sqv[0], 0, 0, 0);
                            sqv[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cb2, as_f16x8(qo[ks]), sqv[1], 0, 0, 0);
                        }
#pragma unroll
                        for (int rb = 0; rb < 2; rb++) {
                            const uint16_t* kr = &kt[buf][16 * rb + n][8 * g];
#pragma unroll
                            for (int kk = 0; kk < 2; kk++) {
                                const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(kr + 32 * kk);
                                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8(rh[kk]), sr[rb], 0, 0, 0);
                                sr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8(rl[kk]), sr[rb], 0, 0, 0);
                            }
                            sl[rb] += sx[rb];
                            sl[rb] += sqv[rb];
                        }
                    }
                    // ---- softmax: lane (g, n) holds rows 16 rb + 4 g + r of head n (no branches)
                    float sc[2][4], rr[2][4];
                    float tmax = -INFINITY;
#pragma unroll
                    for (int rb = 0; rb < 2; rb++) {
                        const float4 rq = *reinterpret_cast<const float4*>(&rho_s[buf][16 * rb + 4 * g]);
                        const float rv[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const bool ok = 16 * rb + 4 * g + r < nt;
                            rr[rb][r] = ok ? rv[r] : 0.0f;
                            sc[rb][r] = ok ? fmaf(rv[r] * k1, sl[rb][r], sr[rb][r]) : -INFINITY;
                            tmax = fmaxf(tmax, sc[rb][r]);
                        }
                    }
                    tmax = max_xor16_xor32(tmax);
                    m_run = m_run == -INFINITY ? tmax : m_run;  // first tile: row 0 is valid
                    // a tile more than 2^8 above the reference raises it; the workgroup
                    // restarts at the next vote
                    const bool ov = __any(tmax > m_run + LAZY_LOG2);
                    m_run = ov ? fmaxf(m_run, tmax) : m_run;
                    over = over || ov;
                    float psum = 0.0f;
                    uint32_t pbv[4];
#pragma unroll
                    for (int rb = 0; rb < 2; rb++) {
                        float pw[4];
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const float pv = __builtin_amdgcn_exp2f(sc[rb][r] - m_run);  // masked rows: 0
                            psum += pv;
                            pw[r] = pv * (rr[rb][r] * rs);
                        }
                        pbv[2 * rb] = pack_f16x2(pw[0], pw[1]);
                        pbv[2 * rb + 1] = pack_f16x2(pw[2], pw[3]);
                    }
                    l_part += psum;
                    // (buffer k % 2: the PV waves read it during step k + 1, and were past their
                    // step k - 1 reads of it at the vote ending step k - 1)
                    pb_s[k & 1][wave][lane] = make_uint4(pbv[0], pbv[1], pbv[2], pbv[3]);
                }
                again = vote(k + 1);
            }
            if (!again) break;
            __syncthreads();  // every wave has read the votes before the restart's first vote rewrites them
            over = false;
        }
        // ---- m and l of the wave's heads
        l_part += __shfl_xor(l_part, 16, 64);
        l_part += __shfl_xor(l_part, 32, 64);
        if (g == 0 && head < a.n_heads) {
            p.part_m[c * a.n_heads + head] = m_run;  // log2 units
            p.part_l[c * a.n_heads + head] = l_part;
        }
    } else {
        // PV source lane (g, n) at row 4 g + n / 4, column 4 (n % 4) (+ 16 mb, + 16 rows):
        // dims 16 mb + 4 (n % 4) .. + 3 of row trow are half n % 2 of chunk 2 mb + b (b =
        // n / 2 % 2), which sits at chunk 2 (mb ^ f / 2) + (b ^ f % 2), f = tq_swz(trow)
        // (rows 16 + trow alike): halfword 16 (mb - mb % 8) + po[mb % 8]
        const int trow = 4 * g + (n >> 2);
        const int fp = tq_swz(trow);
        int po[8];
#pragma unroll
        for (int j = 0; j < 8; j++) po[j] = 16 * (j ^ (fp >> 1)) + 8 * (((n >> 1) & 1) ^ (fp & 1)) + 4 * (n & 1);
        f32x4_t acc_o[8][4];  // dims 128 wave + 16 mb (mb < 8) x head block hb
        if (ntiles > 0) load_share(0);
        for (;;) {
#pragma unroll
            for (int mb = 0; mb < 8; mb++)
#pragma unroll
                for (int hb = 0; hb < 4; hb++) acc_o[mb][hb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (ntiles > 0) {
                decode_share(0);
                load_share(min(1, ntiles - 1));
            }
            bool again = vote(0);
            for (int k = 0; !again && k <= ntiles; k++) {
                if (k >= 1) {
                    // ---- PV of tile k - 1: dims 128 wave + 16 mb, the transposed reads one block ahead
                    const int buf = (k - 1) % TQ_BUFS;
                    f16x8_t bo[4];
#pragma unroll
                    for (int hb = 0; hb < 4; hb++) bo[hb] = as_f16x8(pb_s[(k - 1) & 1][hb][lane]);
                    auto pv_read = [&](int mb) __attribute__((always_inline)) {
                        const int gm = 8 * wave + mb;  // dim block of the row
                        const int off = 16 * (gm & ~7) + po[gm & 7];
                        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t*)(xt_row(buf, trow) + off));
                        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t*)(xt_row(buf, 16 + trow) + off));
                        const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
                        return as_f16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
                    };
                    f16x8_t nxt = pv_read(0);
#pragma unroll
                    for (int mb = 0; mb < 8; mb++) {
                        const f16x8_t aop = nxt;
                        if (mb + 1 < 8) nxt = pv_read(mb + 1);
#pragma unroll
                        for (int hb = 0; hb < 4; hb++)
                            acc_o[mb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bo[hb], acc_o[mb][hb], 0, 0, 0);
                    }
                }
                if (k + 1 < ntiles) {  // the tile after the scored one: decoded now, its successor's codes loaded
                    decode_share((k + 1) % TQ_BUFS);
                    load_share(min(k + 2, ntiles - 1));
                }
                again = vote(k + 1);
            }
            if (!again) break;
            __syncthreads();  // (the restart barrier of the score waves)
            if (ntiles > 0) load_share(0);
        }
        // ---- O of dims 128 wave .. + 127 of every head of the group, as fp16 O * 2^k with
        // one k per head and wave putting the largest |O| * 2^k in [2^14, 2^15); 2^-k in part_s
        const float so = 1.0f / rs;  // exact (a power of two)
#pragma unroll
        for (int hb = 0; hb < 4; hb++) {
            const int h = hg * TQ_HEADS + MF_HEADS * hb + n;
            float am = 0.0f;
#pragma unroll
            for (int mb = 0; mb < 8; mb++)
#pragma unroll
                for (int i = 0; i < 4; i++) am = fmaxf(am, fabsf(acc_o[mb][hb][i]));
            am = fmaxf(am, __shfl_xor(am, 16, 64));
            am = fmaxf(am, __shfl_xor(am, 32, 64));
            float sk_inv;
            const float f = so * f16_store_scale(am * so, &sk_inv);  // exact: amax(acc) * f is near 2^14
            if (h < a.n_heads) {
                uint2* dst = reinterpret_cast<uint2*>(p.part_h + (c * a.n_heads + h) * DL + 128 * wave + 4 * g);
#pragma unroll
                for (int mb = 0; mb < 8; mb++) {
                    const f32x4_t v = acc_o[mb][hb];
                    dst[4 * mb] = make_uint2(pack_f16x2(v[0] * f, v[1] * f), pack_f16x2(v[2] * f, v[3] * f));
                }
                if (g == 0) p.part_s[(c * 4 + wave) * a.n_heads + h] = sk_inv;
            }
        }
    }
}

// ---- 3. merge --------------------------------------------------------------------------------
// NDH workgroups per (sequence, head), each over DL / NDH output dims (TQ4: the
// whole row, which the un-rotation needs).  A thread owns one float4 column and
// every NGRP-th split; it merges its splits online (running max, rescaled sums),
// then the NGRP groups are combined through LDS.  LOG2: the matrix-core
// partials (log2 units, O as scaled fp16); otherwise the fp32 path's.
template <bool TQ4, bool LOG2, int NT>
__global__ __launch_bounds__(NT) void k_merge(kvq_attn_args a, Plan p) {
    constexpr bool F16 = LOG2;
    constexpr int NDH = TQ4 ? 1 : 2;
    constexpr int DW = DL / NDH;       // dims per workgroup
    constexpr int COLS = DW / 4;       // float4 columns
    constexpr int NGRP = NT / COLS;    // split groups
    constexpr int U = 8;               // splits in flight per thread
    __shared__ __align__(16) float4 o_s[NGRP][COLS];
    __shared__ float m_s[NGRP], l_s[NGRP];
    __shared__ __align__(16) float vec[DL];
    const int tid = threadIdx.x;
    const int64_t item = blockIdx.x / NDH;
    const int part = (int)(blockIdx.x % NDH);
    const int s = (int)(item / a.n_heads), h = (int)(item % a.n_heads);
    const int64_t c0 = min(p.chunk_prefix[s], p.max_chunks), c1 = min(p.chunk_prefix[s + 1], p.max_chunks);
    const int col = tid % COLS, grp = tid / COLS;
    // (the matrix-core paths: the hardware exp2; the fp32 path: the library's exp)
    auto ex = [](float x) { return LOG2 ? __builtin_amdgcn_exp2f(x) : expf(x); };
    float m = -INFINITY, l = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int64_t nh = a.n_heads;
    const int d = part * DW + 4 * col;
    // batches of U splits: all loads first (no branch between them), then the
    // online update with selects
    for (int64_t cb = c0 + grp; cb < c1; cb += U * NGRP) {
        float mc[U], lc[U], sk[U];
        float4 v[U];
        uint2 vh[U];
        // split cb's entries, and uniform offsets from them (a split past the end reads cb's)
        const float* mb = p.part_m + cb * nh + h;
        const float* lb = p.part_l + cb * nh + h;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t du = cb + u * NGRP < c1 ? u * NGRP : 0;
            mc[u] = mb[du * nh];
            lc[u] = lb[du * nh];
            if (F16) {
                vh[u] = ld_nt(reinterpret_cast<const uint2*>(p.part_h + (cb * nh + h) * DL + d + du * nh * DL));
                sk[u] = p.part_s[(cb * 4 + (d >> 7)) * nh + h + du * 4 * nh];
            } else {
                v[u] = *reinterpret_cast<const float4*>(p.part_o + (cb * nh + h) * DL + d + du * nh * DL);
            }
        }
        // (every load above is issued before any is used: a split past the end is masked here)
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (F16) v[u] = f16x4_scaled(vh[u], sk[u]);
            if (cb + u * NGRP >= c1) mc[u] = -INFINITY;
            const float mn = fmaxf(m, mc[u]);
            const float sc = m == -INFINITY ? 0.0f : ex(m - mn);
            const float w = mc[u] == -INFINITY ? 0.0f : ex(mc[u] - mn);
            o.x = o.x * sc + w * v[u].x;
            o.y = o.y * sc + w * v[u].y;
            o.z = o.z * sc + w * v[u].z;
            o.w = o.w * sc + w * v[u].w;
            l = l * sc + w * lc[u];
            m = mn;
        }
    }
    o_s[grp][col] = o;
    if (col == 0) {
        m_s[grp] = m;
        l_s[grp] = l;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NGRP; k++) M = fmaxf(M, m_s[k]);
    float L = 0.0f;
    float wg[NGRP];
#pragma unroll
    for (int k = 0; k < NGRP; k++) {
        wg[k] = m_s[k] == -INFINITY ? 0.0f : ex(m_s[k] - M);
        L += wg[k] * l_s[k];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (grp == 0) {
        float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < NGRP; k++) {
            const float4 u = o_s[k][col];
            r.x += wg[k] * u.x; r.y += wg[k] * u.y; r.z += wg[k] * u.z; r.w += wg[k] * u.w;
        }
        r = make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
        if (TQ4) *reinterpret_cast<float4*>(&vec[4 * col]) = r;
        else *reinterpret_cast<float4*>(a.out + item * DL + part * DW + 4 * col) = r;
    }
    if (TQ4) {
        __syncthreads();
        if (tid < 64) {  // o = D H o~ / sqrt(512), 8 consecutive per lane
            const int lane = tid;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = vec[8 * lane + i];
#pragma unroll
            for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (!(i & hh)) {
                        const float x = v[i], y = v[i + hh];
                        v[i] = x + y;
                        v[i + hh] = x - y;
                    }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                float x = v[i];
                x = fwht_xlane_c<1>(x, lane);
                x = fwht_xlane_c<2>(x, lane);
                x = fwht_xlane_c<4>(x, lane);
                x = fwht_xlane_c<8>(x, lane);
                x = fwht_xlane_c<16>(x, lane);
                v[i] = fwht_xlane_c<32>(x, lane);
            }
            const uint32_t sm = a.sign_mask[lane];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                v[i] *= INV_SQRT_DL;
                if ((sm >> i) & 1u) v[i] = -v[i];
            }
            float4* dst = reinterpret_cast<float4*>(a.out + item * DL + 8 * lane);
            dst[0] = make_float4(v[0], v[1], v[2], v[3]);
            dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    if (a.lse && part == 0 && tid == 0) {
        float v;
        if (!(L > 0.0f)) v = -INFINITY;
        else v = LOG2 ? (M + log2f(L)) * LN2 : M + logf(L);
        a.lse[item] = v;
    }
}

// Merge of the fp8 matrix-core partials (stored in the split kernel's lane order,
// see its epilogue).  Workgroup = (sequence, group of 32 heads, 32-dim block
// (w, b, j) of the output): 64 threads (h, n) own head n's dims 128 w + 32 b +
// 8 j + 4 h .. + 3, so the threads of a chunk group read 1 KB contiguous per
// split; NG chunk groups take every NG-th split, U loads in flight each, merged
// online (running max, rescaled sums), then combined through LDS.
template <int NG>
__global__ __launch_bounds__(64 * NG) void k_merge_f8(kvq_attn_args a, Plan p) {
    constexpr int U = 8;
    __shared__ __align__(16) float4 o_s[NG][64];
    __shared__ float m_s[NG][64], l_s[NG][64];
    const int tid = threadIdx.x, grp = tid >> 6, l = tid & 63, n = l & 31, h = l >> 5;
    const int64_t item = blockIdx.x;
    const int wbj = (int)(item & 63);  // (w * 4 + b) * 4 + j
    const int64_t sg = item >> 6;
    const int g = (int)(sg % p.n_groups), s = (int)(sg / p.n_groups);
    const int head = g * F8_HEADS + n;
    const int hc = min(head, a.n_heads - 1);  // a padded head reads a real one's m, l and is not written
    // sequence s's partial states: slots (work item + s) of the work items its tiles went to
    int64_t c0 = 0, c1 = 0;
    if (a.n_seqs == 1) {
        c1 = min(p.one_slots, p.max_chunks);
    } else {
        const int64_t t0 = p.chunk_prefix[s], t1 = p.chunk_prefix[s + 1], q = p.chunk_prefix[a.n_seqs + 1];
        if (t1 > t0) {
            c0 = t0 / q + s;
            c1 = (t1 - 1) / q + s + 1;
        }
        c0 = min(c0, p.max_chunks);
        c1 = min(c1, p.max_chunks);
    }
    const int64_t nh = a.n_heads, cstride = (int64_t)p.n_groups * (F8_HEADS * DL / 4);
    const uint2* src = reinterpret_cast<const uint2*>(p.part_h) + g * (int64_t)(F8_HEADS * DL / 4) + wbj * 64 + l;
    const float* ssrc = p.part_s + (wbj >> 4) * nh + hc;  // 2^-k of quarter w of the head
    float m = -INFINITY, lsum = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t cb = c0 + grp; cb < c1; cb += U * NG) {
        float mc[U], lc[U], sk[U];
        uint2 vh[U];
        const uint2* vb = src + cb * cstride;
        const float* mb = p.part_m + cb * nh + hc;
        const float* lb = p.part_l + cb * nh + hc;
        const float* sb = ssrc + cb * 4 * nh;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t du = cb + u * NG < c1 ? u * NG : 0;  // a slot past the end reads slot cb
            mc[u] = mb[du * nh];
            lc[u] = lb[du * nh];
            vh[u] = ld_nt(vb + du * cstride);
            sk[u] = sb[du * 4 * nh];
        }
        // (every load above is issued before any is used: a slot past the end is masked here)
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float4 vu = f16x4_scaled(vh[u], sk[u]);
            if (cb + u * NG >= c1) mc[u] = -INFINITY;
            const float mn = fmaxf(m, mc[u]);
            const float sc = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
            const float w = mc[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc[u] - mn);
            o.x = o.x * sc + w * vu.x;
            o.y = o.y * sc + w * vu.y;
            o.z = o.z * sc + w * vu.z;
            o.w = o.w * sc + w * vu.w;
            lsum = lsum * sc + w * lc[u];
            m = mn;
        }
    }
    o_s[grp][l] = o;
    m_s[grp][l] = m;
    l_s[grp][l] = lsum;
    __syncthreads();
    if (grp != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NG; k++) M = fmaxf(M, m_s[k][l]);
    float L = 0.0f;
    float4 r = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const float wk = m_s[k][l] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_s[k][l] - M);
        L += wk * l_s[k][l];
        const float4 u = o_s[k][l];
        r.x += wk * u.x; r.y += wk * u.y; r.z += wk * u.z; r.w += wk * u.w;
    }
    if (head >= a.n_heads) return;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int w = wbj >> 4, b = (wbj >> 2) & 3, j = wbj & 3;
    *reinterpret_cast<float4*>(a.out + ((int64_t)s * a.n_heads + head) * DL + 128 * w + 32 * b + 8 * j + 4 * h) =
        make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv);
    if (a.lse && wbj == 0 && h == 0) a.lse[(int64_t)s * a.n_heads + head] = L > 0.0f ? (M + log2f(L)) * LN2 : -INFINITY;
}

// Merge of the fp8 matrix-core partials when sequences have few slots each
// (several sequences): one wave per (sequence, group of 32 heads, NB
// consecutive 32-dim blocks), thread (h, n) owning head n's dims of those
// blocks; the slots are merged online in order, U at a time with every load
// in flight, and each slot's weight serves the NB blocks.  (A workgroup per
// block with the slots dealt to several waves, combined through LDS, was
// slower here: most of its waves had one slot or none.)
template <int NB, int U>
__global__ __launch_bounds__(64) void k_merge_f8_few(kvq_attn_args a, Plan p) {
    const int l = threadIdx.x, n = l & 31, h = l >> 5;
    const int64_t item = blockIdx.x;
    const int wb0 = (int)(item % (64 / NB)) * NB;  // first (w * 4 + b) * 4 + j block
    const int64_t sg = item / (64 / NB);
    const int g = (int)(sg % p.n_groups), s = (int)(sg / p.n_groups);
    const int head = g * F8_HEADS + n;
    const int hc = min(head, a.n_heads - 1);  // a padded head reads a real one's m, l and is not written
    int64_t c0 = 0, c1 = 0;
    if (a.n_seqs == 1) {
        c1 = min(p.one_slots, p.max_chunks);
    } else {
        const int64_t t0 = p.chunk_prefix[s], t1 = p.chunk_prefix[s + 1], q = p.chunk_prefix[a.n_seqs + 1];
        if (t1 > t0) {
            c0 = t0 / q + s;
            c1 = (t1 - 1) / q + s + 1;
        }
        c0 = min(c0, p.max_chunks);
        c1 = min(c1, p.max_chunks);
    }
    static_assert(16 % NB == 0, "the NB blocks lie in one 128-dim quarter");
    const int64_t nh = a.n_heads, cstride = (int64_t)p.n_groups * (F8_HEADS * DL / 4);
    const uint2* src = reinterpret_cast<const uint2*>(p.part_h) + g * (int64_t)(F8_HEADS * DL / 4) + wb0 * 64 + l;
    const float* ssrc = p.part_s + (wb0 >> 4) * nh + hc;  // 2^-k of quarter w of the head
    float m = -INFINITY, lsum = 0.0f;
    float4 o[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) o[b] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    // batches of U slots in two register sets, each batch's loads issued before the one
    // ahead of it is used (a long sequence's slots then cost about one load latency, not one
    // per batch).  The loads are unconditional, so that the waits are the same on every path:
    // a batch past the end reads slot c1 - 1 again and is masked.
    struct Batch {
        float m[U], l[U], s[U];
        uint2 v[U][NB];
    };
    Batch A, B;
    auto load_batch = [&](Batch& t, int64_t cb) __attribute__((always_inline)) {
        const int64_t base = min(cb, c1 - 1);
        const uint2* vb = src + base * cstride;
        const float* mb = p.part_m + base * nh + hc;
        const float* lb = p.part_l + base * nh + hc;
        const float* sb = ssrc + base * 4 * nh;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t du = base + u < c1 ? u : 0;  // a slot past the end reads slot base
            t.m[u] = mb[du * nh];
            t.l[u] = lb[du * nh];
            t.s[u] = sb[du * 4 * nh];
#pragma unroll
            for (int b = 0; b < NB; b++) t.v[u][b] = ld_nt(vb + du * cstride + b * 64);
        }
    };
    auto use_batch = [&](Batch& t, int64_t cb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float mu = cb + u < c1 ? t.m[u] : -INFINITY;  // a slot past the end is masked
            float4 v[NB];
#pragma unroll
            for (int b = 0; b < NB; b++) v[b] = f16x4_scaled(t.v[u][b], t.s[u]);
            const float mn = fmaxf(m, mu);
            const float sc = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
            const float w = mu == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mu - mn);
#pragma unroll
            for (int b = 0; b < NB; b++) {
                o[b].x = o[b].x * sc + w * v[b].x;
                o[b].y = o[b].y * sc + w * v[b].y;
                o[b].z = o[b].z * sc + w * v[b].z;
                o[b].w = o[b].w * sc + w * v[b].w;
            }
            lsum = lsum * sc + w * t.l[u];
            m = mn;
        }
    };
    if (c0 < c1) {
        load_batch(A, c0);
        for (int64_t cb = c0;; cb += 2 * U) {
            load_batch(B, cb + U);
            use_batch(A, cb);
            if (cb + U >= c1) break;  // (wave-uniform)
            load_batch(A, cb + 2 * U);
            use_batch(B, cb + U);
            if (cb + 2 * U >= c1) break;
        }
    }
    if (head >= a.n_heads) return;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int wbj = wb0 + b, w = wbj >> 4, bb = (wbj >> 2) & 3, j = wbj & 3;
        *reinterpret_cast<float4*>(a.out + ((int64_t)s * a.n_heads + head) * DL + 128 * w + 32 * bb + 8 * j + 4 * h) =
            make_float4(o[b].x * inv, o[b].y * inv, o[b].z * inv, o[b].w * inv);
    }
    if (a.lse && wb0 == 0 && h == 0) a.lse[(int64_t)s * a.n_heads + head] = lsum > 0.0f ? (m + log2f(lsum)) * LN2 : -INFINITY;
}

hipError_t launch_stage(const kvq_attn_args& a, const Plan& p, int stage, hipStream_t st, const NewRows* nr) {
    const NewRows none{nullptr, 0, nullptr, nullptr};
    const bool f32 = a.precision == KVQ_PREC_FP32;
    const bool tq = qmode_rotated(a.qmode);
    switch (stage) {
        case KVQ_STAGE_PREP:
            // the matrix-core split kernels plan their chunk themselves; their
            // query operands are prepared here once per head (rotated codec: R q)
            if (!f32) {
                const int64_t rows = (int64_t)a.n_seqs * p.heads_padded;
                if (tq) {
                    hipLaunchKernelGGL(k_qprep_tq4, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a, p);
                } else {  // with the fp8 encode of the appended rows, if any, in the same launch
                    const NewRows n = nr ? *nr : none;
                    const int64_t blocks = (rows + 3) / 4 + (n.n + 3) / 4 + (a.n_seqs > 1 ? 1 : 0);
                    hipLaunchKernelGGL(k_qprep_fp8, dim3((unsigned)blocks), dim3(256), 0, st, a, p, n);
                }
                break;
            }
            hipLaunchKernelGGL(k_plan, dim3(1), dim3(256), 0, st, a.seq_offsets, a.n_seqs, p.split_rows, a.total_rows,
                               p.chunk_prefix);
            if (tq) {
                const int64_t rows = (int64_t)a.n_seqs * a.n_heads;
                hipLaunchKernelGGL(k_qrot, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a.q_lat, a.sign_mask,
                                   rows, p.q_rot);
            }
            break;
        case KVQ_STAGE_SPLITS:
            if (f32) {
                const dim3 grid((unsigned)p.max_chunks, (unsigned)p.n_groups);
                const float* qsrc = tq ? p.q_rot : a.q_lat;
                switch (a.qmode) {
                    case KVQ_QMODE_TQ4: hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_TQ4>, grid, dim3(256), 0, st, a, p, qsrc); break;
                    case KVQ_QMODE_TQ3: hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_TQ3>, grid, dim3(256), 0, st, a, p, qsrc); break;
                    case KVQ_QMODE_TQ6: hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_TQ6>, grid, dim3(256), 0, st, a, p, qsrc); break;
                    default: hipLaunchKernelGGL(k_attn_f32<KVQ_QMODE_FP8>, grid, dim3(256), 0, st, a, p, qsrc); break;
                }
            } else {
                const dim3 grid((unsigned)(p.chunks_per_xcd * N_XCD * p.n_groups));
                switch (a.qmode) {
                    case KVQ_QMODE_TQ4: hipLaunchKernelGGL(k_attn_mfma_tq<4>, grid, dim3(2 * MF_WAVES * 64), 0, st, a, p); break;
                    case KVQ_QMODE_TQ3: hipLaunchKernelGGL(k_attn_mfma_tq<3>, grid, dim3(2 * MF_WAVES * 64), 0, st, a, p); break;
                    case KVQ_QMODE_TQ6: hipLaunchKernelGGL(k_attn_mfma_tq<6>, grid, dim3(2 * MF_WAVES * 64), 0, st, a, p); break;
                    default: {
                        const dim3 wg(MF_WAVES * 64);
                        if (p.row_index) {
                            if (a.n_seqs == 1) hipLaunchKernelGGL((k_attn_mfma_fp8<true, true>), grid, wg, 0, st, a, p);
                            else hipLaunchKernelGGL((k_attn_mfma_fp8<false, true>), grid, wg, 0, st, a, p);
                        } else {
                            if (a.n_seqs == 1) hipLaunchKernelGGL((k_attn_mfma_fp8<true, false>), grid, wg, 0, st, a, p);
                            else hipLaunchKernelGGL((k_attn_mfma_fp8<false, false>), grid, wg, 0, st, a, p);
                        }
                        break;
                    }
                }
            }
            break;
        default: {
            const int64_t items = (int64_t)a.n_seqs * a.n_heads;
            // more split groups per workgroup when there are many splits per sequence,
            // a single one (one thread per float4 column) when there are few
            const bool wide = p.max_chunks >= 16 * (int64_t)a.n_seqs;
            const bool narrow = p.max_chunks <= 4 * (int64_t)a.n_seqs;
            if (tq) {
                if (!f32 && wide) hipLaunchKernelGGL((k_merge<true, true, 1024>), dim3((unsigned)items), dim3(1024), 0, st, a, p);
                else if (!f32 && narrow) hipLaunchKernelGGL((k_merge<true, true, 128>), dim3((unsigned)items), dim3(128), 0, st, a, p);
                else if (!f32) hipLaunchKernelGGL((k_merge<true, true, 256>), dim3((unsigned)items), dim3(256), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<true, false, 256>), dim3((unsigned)items), dim3(256), 0, st, a, p);
            } else {
                const int64_t f8_items = (int64_t)a.n_seqs * p.n_groups * 64;  // (sequence, group, 32-dim block)
                if (!f32 && wide) hipLaunchKernelGGL((k_merge_f8<8>), dim3((unsigned)f8_items), dim3(512), 0, st, a, p);
                else if (!f32) hipLaunchKernelGGL((k_merge_f8_few<2, 8>), dim3((unsigned)(f8_items / 2)), dim3(64), 0, st, a, p);
                else hipLaunchKernelGGL((k_merge<false, false, 256>), dim3((unsigned)(2 * items)), dim3(256), 0, st, a, p);
            }
            break;
        }
    }
    return hipGetLastError();
}

}  // namespace

int64_t attn_workspace_bytes(const kvq_attn_args& a) { return plan_bytes(a); }

hipError_t launch_decode_attn_stage(const kvq_attn_args& a, int stage, void* ws, hipStream_t st, const NewRows* nr) {
    return launch_stage(a, make_plan(a, ws, nullptr), stage, st, nr);
}

hipError_t launch_decode_attn_indexed(const kvq_attn_args& a, const int64_t* row_index, int64_t cache_rows, void* ws,
                                      hipStream_t st) {
    Plan p = make_plan(a, ws, nullptr);
    p.row_index = row_index;
    p.cache_rows = cache_rows;
    for (int stage = KVQ_STAGE_PREP; stage <= KVQ_STAGE_MERGE; stage++) {
        const hipError_t e = launch_stage(a, p, stage, st, nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_decode_attn(const kvq_attn_args& a, void* ws, int64_t ws_bytes, hipStream_t st) {
    (void)ws_bytes;
    for (int stage = KVQ_STAGE_PREP; stage <= KVQ_STAGE_MERGE; stage++) {
        const hipError_t e = launch_decode_attn_stage(a, stage, ws, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_decode_attn_append(const kvq_attn_args& a, const NewRows& nr, void* ws, hipStream_t st) {
    const bool fused = a.qmode == KVQ_QMODE_FP8 && a.precision == KVQ_PREC_MFMA;
    if (!fused && nr.n > 0) {  // the encoder first, then the attention
        const hipError_t e = a.qmode == KVQ_QMODE_FP8
                                 ? launch_encode_fp8(nr.x, nr.n, DL, nr.codes, nr.scales, st)
                                 : launch_encode_tq(qmode_bits(a.qmode), nr.x, nr.n, DL, a.sign_mask, nr.codes,
                                                    nr.scales, st);
        if (e != hipSuccess) return e;
    }
    for (int stage = KVQ_STAGE_PREP; stage <= KVQ_STAGE_MERGE; stage++) {
        const hipError_t e = launch_decode_attn_stage(a, stage, ws, st, fused ? &nr : nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kvq
